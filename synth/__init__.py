"""Seeded synthetic inputs for the hybrid-block path.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic (no attention, selection, projection or quantisation).  It
serves both the CPU oracle tests and the GPU path's tests and benchmark.

Recipe (every stream is independent and reproducible):
  rng(cfg, tensor, sub) = numpy.random.default_rng(
      SeedSequence(entropy=1000 + cfg, spawn_key=(tensor, sub)))
  tensor ids: 0 K, 1 V, 2 Q of the full layer, 3.. Q of sparse layer 1.., 8
  needles, 9 clusters, 10 ragged lengths, 11 hidden states, 12 + 2l W_k of
  target l, 13 + 2l W_v of target l; block b of a multi-block stack adds 100*b;
  sub = sequence index (so one sequence can be regenerated alone).
  Gaussian draws are float32 standard normals; bf16 inputs are those values
  rounded to nearest even (a storage conversion of the input).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HEAD_DIM = 128
TOP_K = 1024
WINDOW = 128

T_K, T_V, T_QFULL, T_QSPARSE0, T_NEEDLE, T_CLUSTER, T_LENS, T_HIDDEN, T_WBASE = 0, 1, 2, 3, 8, 9, 10, 11, 12

# The five workloads.  'kv' is the storage type of the cache, 'q' the query type.
CONFIGS = {
    1: dict(name="c1_8k_fp32_needles", B=1, L=8192, H=16, n_kv=1, n_q=16, n_sparse=3,
            kv="f32", q="f32", needles=8),
    2: dict(name="c2_b32_128k_bf16", B=32, L=131072, H=32, n_kv=1, n_q=1, n_sparse=5,
            kv="bf16", q="bf16", needles=64),
    3: dict(name="c3_1m_fp8_h64_q4", B=1, L=1048576, H=64, n_kv=1, n_q=4, n_sparse=5,
            kv="e4m3", q="bf16", needles=0, cluster_frac=0.01, n_clusters=16),
    4: dict(name="c4_bridge_32k", T=32768, D=4096, n_targets=4, capacity=1048576,
            offset=262144),
    5: dict(name="c5_ragged_8x64k-512k", B=8, L_lo=65536, L_hi=524288, H=32, n_kv=1, n_q=1,
            n_sparse=5, n_blocks=4, kv="bf16", q="bf16", needles=0),
}

# Aligned-cluster strengths for config 3 (key = alpha * sqrt(d) * unit query), one per
# aligned cluster: (t=0, h=0) and (t=1, h=1).  Tuned so that, with the oracle's scores on
# the stored E4M3 keys at L = 1,048,576, the 1024-th global score of query token t falls
# inside cluster t: part of each cluster is selected and part is not.
C3_ALPHA = (0.4285, 0.4608)


def rng(cfg, tensor, sub=0):
    return np.random.default_rng(np.random.SeedSequence(entropy=1000 + int(cfg),
                                                        spawn_key=(int(tensor), int(sub))))


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def normal_f32(cfg, tensor, sub, shape, out=None):
    g = rng(cfg, tensor, sub)
    if out is None:
        return g.standard_normal(shape, dtype=np.float32)
    g.standard_normal(dtype=np.float32, out=out)
    return out


def bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (input storage)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _par(fn, items):
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, items))


def ragged_lengths(cfg=5):
    c = CONFIGS[cfg]
    return rng(cfg, T_LENS).integers(c["L_lo"], c["L_hi"], size=c["B"], endpoint=True).astype(np.int64)


def queries(cfg, B, n_q, H, tensor, qtype, block=0):
    """[B, n_q, H, d] float32 (qtype 'f32') or bf16 bits (qtype 'bf16')."""
    tid = tensor + 100 * block
    q = np.stack([normal_f32(cfg, tid, b, (n_q, H, HEAD_DIM)) for b in range(B)])
    return q if qtype == "f32" else bf16_bits(q)


def _q_as_f32(q, qtype):
    return q if qtype == "f32" else bf16_bits_to_f32(q)


def decode_case(cfg, L=None, B=None, seqs=None, block=0, lengths=None):
    """Inputs of one hybrid-block decode step.

    Returns a dict:
      spec      the config dict (with L / B overrides applied)
      lengths   int64 [B] rows per sequence; row_start int64 [B] (packed)
      q_full    [B, n_q, H, d]   (float32, or bf16 bits)
      q_sparse  list of n_sparse arrays like q_full
      k, v      [sum L, n_kv, d] float32 (cfg kv 'f32'/'e4m3') or bf16 bits ('bf16');
                for 'e4m3' configs these are the float32 rows before quantisation
      needles   list per sequence of (position, token, head) triples
    seqs: optional subset of sequence indices to generate (others are skipped;
    lengths/row_start then describe only those sequences, in order).
    """
    spec = dict(CONFIGS[cfg])
    if L is not None:
        spec["L"] = int(L)
    if B is not None:
        spec["B"] = int(B)
    B_all = spec["B"]
    if lengths is None:
        lengths = ragged_lengths(cfg) if cfg == 5 else np.full(B_all, spec["L"], np.int64)
    lengths = np.asarray(lengths, np.int64)
    sel = list(range(B_all)) if seqs is None else [int(s) for s in seqs]
    H, n_q, n_kv, d = spec["H"], spec["n_q"], spec["n_kv"], HEAD_DIM
    lens = lengths[sel]
    row_start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    total = int(lens.sum())
    qt = spec["q"]
    q_full_all = queries(cfg, B_all, n_q, H, T_QFULL, qt, block)
    q_full = q_full_all[sel]
    q_sparse = [queries(cfg, B_all, n_q, H, T_QSPARSE0 + i, qt, block)[sel]
                for i in range(spec["n_sparse"])]
    kf = np.empty((total, n_kv, d), np.float32)
    vf = np.empty((total, n_kv, d), np.float32)

    def fill(i):
        b = sel[i]
        r0, r1 = row_start[i], row_start[i] + lens[i]
        normal_f32(cfg, T_K + 100 * block, b, None, out=kf[r0:r1])
        normal_f32(cfg, T_V + 100 * block, b, None, out=vf[r0:r1])

    _par(fill, range(len(sel)))

    needles = [[] for _ in sel]
    nn = spec.get("needles", 0)
    qf32 = _q_as_f32(q_full, qt)
    for i, b in enumerate(sel):
        if nn == 0:
            continue
        Lb = int(lens[i])
        cnt = min(nn, Lb - WINDOW)                     # short sequences carry fewer needles
        if cnt <= 0:
            continue
        g = rng(cfg, T_NEEDLE + 100 * block, b)
        pos = g.choice(Lb - WINDOW, size=cnt, replace=False)
        tok = g.integers(0, n_q, size=cnt)
        head = g.integers(0, H, size=cnt)
        for p, t, h in zip(pos, tok, head):
            kv_head = h // (H // n_kv)
            kf[row_start[i] + p, kv_head, :] = 4.0 * qf32[i, t, h, :]
            needles[i].append((int(p), int(t), int(h)))

    if spec.get("cluster_frac"):
        for i, b in enumerate(sel):
            _plant_clusters(cfg, spec, b, kf[row_start[i]:row_start[i] + lens[i]], qf32[i],
                            int(lens[i]))

    if spec["kv"] == "bf16":
        k_out = np.empty(kf.shape, np.uint16)
        v_out = np.empty(vf.shape, np.uint16)

        def conv(i):
            r0, r1 = row_start[i], row_start[i] + lens[i]
            k_out[r0:r1] = bf16_bits(kf[r0:r1])
            v_out[r0:r1] = bf16_bits(vf[r0:r1])

        _par(conv, range(len(sel)))
        del kf, vf
    else:
        k_out, v_out = kf, vf
    return dict(spec=spec, lengths=lens, row_start=row_start, q_full=q_full,
                q_sparse=q_sparse, k=k_out, v=v_out, needles=needles)


def _cluster_draw(cfg, spec, b, L):
    g = rng(cfg, T_CLUSTER, b)
    n = int(round(spec["cluster_frac"] * L))
    pos = g.choice(L - WINDOW, size=n, replace=False)
    return g, np.array_split(pos, spec["n_clusters"])


def cluster_positions(cfg, b, L):
    """Row positions of each near-duplicate cluster of sequence b (cluster 0 is aligned with
    query (t=0, h=0), cluster 1 with (t=1, h=1)), as decode_case plants them."""
    return _cluster_draw(cfg, CONFIGS[cfg], b, int(L))[1]


def _plant_clusters(cfg, spec, b, k_rows, q_f32, L):
    """Config 3's near-duplicate key clusters (1% of rows, 16 clusters).

    Two clusters are centred on alpha * sqrt(d) * (unit query of (t=0, h=0)) and
    of (t=1, h=1), so that many near-identical keys compete at the top-k
    boundary; the other centres are standard normal vectors.
    """
    g, groups = _cluster_draw(cfg, spec, b, L)
    centers = g.standard_normal((spec["n_clusters"], HEAD_DIM), dtype=np.float32)
    for ci, (t, h) in enumerate([(0, 0), (1, 1)]):
        qv = q_f32[t, h].astype(np.float64)
        centers[ci] = (C3_ALPHA[ci] * np.sqrt(HEAD_DIM) * qv / np.linalg.norm(qv)).astype(np.float32)
    for ci, grp in enumerate(groups):
        noise = g.standard_normal((len(grp), HEAD_DIM), dtype=np.float32)
        k_rows[grp, 0, :] = centers[ci][None, :] + np.float32(1e-3) * noise


def bridge_case(cfg=4, T=None, D=None, n_targets=None):
    """Hidden states and projection weights of a KV Bridging chunk (bf16 bits).

    X ~ N(0, 1); W_k, W_v ~ N(0, 2 / (D + d)) (Xavier-normal), per target.
    """
    spec = dict(CONFIGS[cfg])
    T = spec["T"] if T is None else int(T)
    D = spec["D"] if D is None else int(D)
    nt = spec["n_targets"] if n_targets is None else int(n_targets)
    x = np.empty((T, D), np.uint16)
    rows = 1024                      # fixed chunk: the streams do not depend on the host

    def fill(r0):
        r1 = min(T, r0 + rows)
        x[r0:r1] = bf16_bits(normal_f32(cfg, T_HIDDEN, r0 // rows, (r1 - r0, D)))

    _par(fill, range(0, T, rows))
    sd = np.float32(np.sqrt(2.0 / (D + HEAD_DIM)))
    wk = [bf16_bits(normal_f32(cfg, T_WBASE + 2 * l, 0, (D, HEAD_DIM)) * sd) for l in range(nt)]
    wv = [bf16_bits(normal_f32(cfg, T_WBASE + 2 * l + 1, 0, (D, HEAD_DIM)) * sd) for l in range(nt)]
    return dict(spec=spec, x=x, w_k=wk, w_v=wv, T=T, D=D, n_targets=nt)
