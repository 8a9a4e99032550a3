"""Full-attention + selection and sparse layers on the GPU against the float64 oracle.

Gates (tolerances from the method's accuracy bar):
  G1 selection indices equal the oracle's, bit for bit, on the GPU's own float32
     scores (the oracle re-selects from exactly the tensor the kernel saw);
  G2 global-part recall >= 0.999 against the oracle's own float64 selection;
  G3 max |O - O_oracle| <= 2e-3 (fp32 / bf16 caches) or 3e-2 (FP8 caches), for the
     full layer and for every sparse layer (sparse layers are checked on the GPU's
     index lists, so boundary swaps cannot confound output parity).
"""

import os

import numpy as np
import pytest
import torch

import synth
from oracle import attention, block, selection
from gpu_cases import Uploaded, banner, recall

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-3, "bf16": 2e-3, "e4m3": 3e-2}


def _run_block(up, top_k=1024, window=128, scores=True):
    from long_context_split_amd import hysparse as hs
    kv = up.kv
    B, n_q, H, _ = up.q_full.shape
    S = hs.scores_stride(kv, window)
    nan = float("nan")
    sc = torch.full((B, n_q, kv.n_kv, max(S, 1)), nan, dtype=torch.float32, device="cuda") if scores else None
    # every output starts poisoned (NaN, or an index no list can hold), so a slot the kernels
    # leave unwritten fails the comparisons below
    out, lse, idx, cnt = hs.full_attn_select(
        kv, up.q_full, top_k, window, scores_out=sc,
        out=torch.full((B, n_q, H, 128), nan, dtype=torch.float32, device="cuda"),
        lse=torch.full((B, n_q, H), nan, dtype=torch.float32, device="cuda"),
        sel_idx=torch.full((B, n_q, kv.n_kv, top_k + window), -0x7F7F7F7F, dtype=torch.int32, device="cuda"),
        sel_count=torch.full((B, n_q, kv.n_kv), -0x7F7F7F7F, dtype=torch.int32, device="cuda"))
    sparse = [hs.sparse_attn(kv, q, idx, cnt, top_k, window,
                             out=torch.full((B, n_q, H, 128), nan, dtype=torch.float32, device="cuda"))
              for q in up.q_sparse]
    torch.cuda.synchronize()
    return dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(), idx=idx.cpu().numpy(), cnt=cnt.cpu().numpy(),
                scores=None if sc is None else sc.cpu().numpy(), sparse=[s.cpu().numpy() for s in sparse])


def _check_seq(up, res, i, top_k=1024, window=128, check_sparse=True, stats=None):
    """All gates for sequence i of an uploaded case."""
    tol = TOL[up.kvtype]
    L = int(up.case["lengths"][i])
    q, k, v = up.oracle_seq(i)
    ref = block.full_layer(q, k, v, top_k, window)
    err = np.abs(res["out"][i] - ref["o"]).max()
    assert err <= tol, f"seq {i}: full-layer max|dO| = {err}"
    assert np.abs(res["lse"][i] - ref["lse"]).max() <= 1e-3 * max(1.0, np.abs(ref["lse"]).max())
    n_q, n_kv = ref["cnt"].shape
    w, kk = selection.budget(L, top_k, window)
    hit = tot = tie = 0
    worst = 1.0
    for t in range(n_q):
        for g in range(n_kv):
            assert res["cnt"][i, t, g] == ref["cnt"][t, g] == kk + w
            if res["scores"] is not None:
                gs = np.ascontiguousarray(res["scores"][i, t, g, :L - w])
                # scores themselves: float32 of the float64 definition
                if L - w > 0:
                    assert np.abs(gs - ref["s"][t, g]).max() <= 1e-4 * ref["s"][t, g].max() + 1e-12
                gi, gc = selection.select(gs, L, top_k, window, f32_keys=True)          # G1
                assert np.array_equal(res["idx"][i, t, g], gi), f"seq {i} t {t} g {g}: G1"
            h, n, th = recall(res["idx"][i, t, g], res["cnt"][i, t, g], ref["idx"][t, g], ref["cnt"][t, g], L,
                              top_k, window, ref["s"][t, g])
            hit += h
            tot += n
            tie += th
            if n:
                worst = min(worst, h / n)
    if stats is not None:
        stats["hit"] = stats.get("hit", 0) + hit
        stats["tot"] = stats.get("tot", 0) + tot
        stats["tie"] = stats.get("tie", 0) + tie
        stats["worst"] = min(stats.get("worst", 1.0), worst)
        stats["err"] = max(stats.get("err", 0.0), float(err))
    if check_sparse:
        gidx = res["idx"][i]
        gcnt = res["cnt"][i]
        same = np.array_equal(gidx, ref["idx"]) and np.array_equal(gcnt, ref["cnt"])
        for layer in range(len(up.q_sparse)):
            qs, _, _ = up.oracle_seq(i, "sparse", layer)
            so, _ = attention.sparse_attention(qs, k, v, gidx, gcnt)
            e = np.abs(res["sparse"][layer][i] - so).max()
            assert e <= tol, f"seq {i} sparse layer {layer}: max|dO| = {e}"
            # second report (not a gate): against the oracle run on its own lists, where boundary
            # swaps between near-tied scores would show up
            eo = e if same else np.abs(res["sparse"][layer][i] - attention.sparse_attention(qs, k, v, ref["idx"], ref["cnt"])[0]).max()
            if stats is not None:
                stats["serr"] = max(stats.get("serr", 0.0), float(e))
                stats["serr_own"] = max(stats.get("serr_own", 0.0), float(eo))
    return hit, tot


def _same_lists_without_scores(up, res, top_k=1024, window=128):
    """The benchmark's form of the full layer (no dense scores asked for: the score filter for one
    query token) selects exactly the lists the dense scores gave, and its outputs are identical."""
    from long_context_split_amd import hysparse as hs
    B, n_q, H, _ = up.q_full.shape
    out, lse, idx, cnt = hs.full_attn_select(
        up.kv, up.q_full, top_k, window,
        sel_idx=torch.full((B, n_q, up.kv.n_kv, top_k + window), -0x7F7F7F7F, dtype=torch.int32, device="cuda"),
        sel_count=torch.full((B, n_q, up.kv.n_kv), -0x7F7F7F7F, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), res["idx"]), "lists without dense scores"
    assert np.array_equal(cnt.cpu().numpy(), res["cnt"])
    assert np.array_equal(out.cpu().numpy(), res["out"]) and np.array_equal(lse.cpu().numpy(), res["lse"])


def _recall_report(stats):
    """Plain recall, tie-aware recall and the worst single list (gate G2 uses the plain one), and the
    sparse layers' largest error against the oracle on its own lists (a report, not a gate)."""
    return (f"recall {stats['hit'] / stats['tot']:.6f} tie-aware {stats['tie'] / stats['tot']:.6f} "
            f"worst list {stats['worst']:.6f}; sparse vs the oracle's own lists {stats.get('serr_own', 0.0):.3e}")


def test_config1_fp32_full_size():
    banner("config 1: B=1 L=8192 H=16 n_q=16 fp32, 3 sparse layers")
    up = Uploaded(synth.decode_case(1))
    res = _run_block(up)
    stats = {}
    _check_seq(up, res, 0, stats=stats)
    assert stats["hit"] / stats["tot"] >= 0.999
    sel = [set(res["idx"][0, t, 0, :1152].tolist()) for t in range(16)]
    for (p, t, h) in up.case["needles"][0]:
        assert p in sel[t], ("needle", p, t, h)
    print(f"[result] config1 max|dO| {stats['err']:.3e} sparse {stats['serr']:.3e} "
          f"{_recall_report(stats)}", flush=True)


@pytest.mark.parametrize("split,schunk", [(0, 0), (512, 1152), (4096, 512), (256, 0)])
def test_ragged_bf16_edge_lengths(split, schunk, monkeypatch):
    """Lengths below, at and around the window and the 1152 capacity, plus several tiles
    and ragged tails.  The full layer's split size changes the number of partials merged
    (256: 79 chunks, merged by the separate merge kernel; otherwise at most 64, merged
    inside the score kernel); the sparse chunk 1152 is the single-workgroup direct form."""
    if split:
        monkeypatch.setenv("HS_SPLIT_TOKENS", str(split))
    if schunk:
        monkeypatch.setenv("HS_SPARSE_CHUNK", str(schunk))
    lens = [1, 100, 128, 129, 300, 1152, 1153, 4099, 20000]
    banner(f"ragged bf16 lens={lens} split={split} sparse chunk={schunk}")
    case = synth.decode_case(2, B=len(lens), lengths=lens)
    up = Uploaded(case)
    res = _run_block(up)
    stats = {}
    for i in range(len(lens)):
        _check_seq(up, res, i, stats=stats)
    assert stats["hit"] / max(1, stats["tot"]) >= 0.999
    # every row selected when L <= 1152: sparse layers then equal full attention over all rows
    for i, L in enumerate(lens):
        if L <= 1152:
            q, k, v = up.oracle_seq(i, "sparse", 0)
            full, _, _ = attention.full_attention(q, k, v)
            assert np.abs(res["sparse"][0][i] - full).max() <= 2e-3


@pytest.mark.parametrize("kvtype,H,schunk", [("bf16", 32, 0), ("bf16", 48, 512), ("e4m3", 64, 0), ("e4m3", 32, 1152)])
def test_sparse_lists_with_absent_entries(kvtype, H, schunk, monkeypatch):
    """Sparse layer on hand-made lists: ragged counts (1 row; 300 rows, ending inside a 256-row
    chunk; the full 1152), repeated rows, and entries outside [0, L_b) inside the count, which the
    layer treats as absent.  H=48 leaves the second block of 32 query heads half empty; chunk 512
    gives each wave two tiles and 1152 is the single-workgroup direct form.  Oracle: the same lists
    with the absent entries removed."""
    from long_context_split_amd import hysparse as hs
    if schunk:
        monkeypatch.setenv("HS_SPARSE_CHUNK", str(schunk))
    banner(f"sparse lists with absent entries kv={kvtype} H={H} chunk={schunk}")
    rng = np.random.default_rng(11)
    lens = [3000, 900, 1500, 500, 700]
    nb = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    tot = sum(lens)
    kf = rng.standard_normal((tot, 1, 128)).astype(np.float32)
    vf = rng.standard_normal((tot, 1, 128)).astype(np.float32)
    q = synth.bf16_bits(rng.standard_normal((nb, 1, H, 128)).astype(np.float32))
    if kvtype == "bf16":
        kf, vf = synth.bf16_bits(kf), synth.bf16_bits(vf)
    case = dict(spec=dict(kv=kvtype, q="bf16"), lengths=np.array(lens), row_start=starts,
                q_full=q, q_sparse=[q], k=kf, v=vf, needles=[[] for _ in lens])
    up = Uploaded(case)
    cap = 1152
    idx = np.full((nb, 1, 1, cap), -1, np.int32)
    cnt = np.array([cap, 1, 300, 0, 3], np.int32).reshape(nb, 1, 1)
    idx[0, 0, 0] = rng.integers(0, lens[0], cap)                     # with repeats
    idx[0, 0, 0, [5, 40, 41, 700, 1151]] = [-1, lens[0], -7, 10 ** 6, lens[0] + 1]
    idx[1, 0, 0, 0] = 899
    idx[2, 0, 0, :300] = rng.permutation(lens[2])[:300]
    idx[2, 0, 0, [0, 255, 256, 299]] = [-2, lens[2], -1, 2 ** 31 - 1]
    idx[3, 0, 0, :4] = [1, 2, 3, 4]                                   # count 0: the entries are ignored
    idx[4, 0, 0, :3] = [-1, lens[4], 10 ** 6]                         # every listed entry absent
    poison = torch.full((nb, 1, H, 128), float("nan"), dtype=torch.float32, device="cuda")
    out = hs.sparse_attn(up.kv, up.q_sparse[0], torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                         out=poison)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    worst = 0.0
    for i in range(nb):
        sel = idx[i, 0, 0, :cnt[i, 0, 0]]
        sel = sel[(sel >= 0) & (sel < lens[i])]
        if sel.size == 0:                                              # no row: the output is zero
            assert np.array_equal(out[i], np.zeros_like(out[i])), f"seq {i}: empty list output"
            continue
        qs, k, v = up.oracle_seq(i, "sparse", 0)
        ref, _ = attention.sparse_attention(qs, k, v, sel.reshape(1, 1, -1), np.array([[sel.size]]))
        e = np.abs(out[i] - ref).max()
        worst = max(worst, float(e))
        assert e <= TOL[kvtype], f"seq {i}: max|dO| = {e}"
    print(f"[result] absent-entry lists kv={kvtype} H={H} chunk={schunk} max|dO| {worst:.3e}", flush=True)


@pytest.mark.parametrize("kvtype,H", [("bf16", 32), ("e4m3", 64)])
def test_sparse_workspace_contents_do_not_matter(kvtype, H):
    """The sparse layer's workspace (chunk partials) is scratch: filled with random bytes, then
    reused by a second call and a third with other counts, every output equals the output of the
    same call on a zero-filled workspace bit for bit, and the oracle's within the layer's
    tolerance."""
    from long_context_split_amd import hysparse as hs
    banner(f"sparse layer, random-filled and reused workspace kv={kvtype} H={H}")
    rng = np.random.default_rng(5)
    lens = [20000, 1300, 5000, 129, 70000, 3000]
    nb = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    tot = sum(lens)
    kf = rng.standard_normal((tot, 1, 128)).astype(np.float32)
    vf = rng.standard_normal((tot, 1, 128)).astype(np.float32)
    q = synth.bf16_bits(rng.standard_normal((nb, 1, H, 128)).astype(np.float32))
    if kvtype == "bf16":
        kf, vf = synth.bf16_bits(kf), synth.bf16_bits(vf)
    case = dict(spec=dict(kv=kvtype, q="bf16"), lengths=np.array(lens), row_start=starts,
                q_full=q, q_sparse=[q], k=kf, v=vf, needles=[[] for _ in lens])
    up = Uploaded(case)
    p = hs.params(H, 1)
    wsz = hs.sparse_attn_workspace_size(up.kv, p)
    ws = torch.randint(0, 256, (wsz,), dtype=torch.uint8, device="cuda")
    for call in range(3):
        idx = np.full((nb, 1, 1, 1152), -1, np.int32)
        cnt = np.zeros((nb, 1, 1), np.int32)
        for i, L in enumerate(lens):
            n = min(L, 1152 - (200 if call == 2 and i % 2 else 0))
            idx[i, 0, 0, :n] = rng.choice(L, n, replace=False)
            cnt[i] = n
        di, dc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
        poison = torch.full((nb, 1, H, 128), float("nan"), dtype=torch.float32, device="cuda")
        a = hs.sparse_attn(up.kv, up.q_sparse[0], di, dc, ws=ws, out=poison)
        b = hs.sparse_attn(up.kv, up.q_sparse[0], di, dc, ws=torch.zeros(wsz, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        a, b = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(a, b), f"call {call}"
        worst = 0.0
        for i in range(nb):
            qs, k, v = up.oracle_seq(i, "sparse", 0)
            sel = idx[i, 0, 0, :cnt[i, 0, 0]]
            ref, _ = attention.sparse_attention(qs, k, v, sel.reshape(1, 1, -1), np.array([[sel.size]]))
            e = float(np.abs(a[i] - ref).max())
            worst = max(worst, e)
            assert e <= TOL[kvtype], f"call {call} seq {i}: max|dO| = {e}"
        print(f"[result] reused random workspace kv={kvtype} H={H} call {call}: max|dO| {worst:.3e}", flush=True)

def test_gqa_multi_query_tokens_bf16():
    """n_kv = 2 KV heads of 16 query heads each, 3 query tokens (no mask among them)."""
    banner("gqa n_kv=2 H=32 n_q=3 bf16")
    from long_context_split_amd import hysparse as hs
    rng = np.random.default_rng(5)
    lens = [3000, 777]
    tot = sum(lens)
    k = synth.bf16_bits(rng.standard_normal((tot, 2, 128)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((tot, 2, 128)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((2, 3, 32, 128)).astype(np.float32))
    case = dict(spec=dict(kv="bf16", q="bf16"), lengths=np.array(lens), row_start=np.array([0, lens[0]]),
                q_full=q, q_sparse=[q], k=k, v=v, needles=[[], []])
    up = Uploaded(case)
    res = _run_block(up, top_k=200, window=16)
    for i in range(2):
        _check_seq(up, res, i, top_k=200, window=16)


@pytest.mark.parametrize("kvtype,n_kv,H,n_q", [("bf16", 1, 32, 3), ("e4m3", 2, 32, 4), ("e4m3", 1, 64, 2),
                                              ("bf16", 1, 32, 8), ("bf16", 2, 32, 6), ("bf16", 1, 256, 1),
                                              ("e4m3", 1, 128, 2)])
def test_many_row_kernels(kvtype, n_kv, H, n_q):
    """The many-row kernels (more than 32 query rows per KV head) at each row-group count: R = 96
    and 128 (4 groups, 128-token super-tiles), 64 (2 groups, 64-token super-tiles), 256 and 96
    with 8 and 6 query tokens per workgroup (no fused histogram); G = 16, 32, 64, 128 and 256 (the
    largest group: one query token's heads fill a workgroup of 8 waves); bf16 and E4M3 caches;
    lengths that end inside a super-tile."""
    banner(f"many-row kv={kvtype} n_kv={n_kv} H={H} n_q={n_q}")
    rng = np.random.default_rng(40 + H + n_q + n_kv)
    lens = [5000, 777]
    tot = sum(lens)
    k = rng.standard_normal((tot, n_kv, 128)).astype(np.float32)
    v = rng.standard_normal((tot, n_kv, 128)).astype(np.float32)
    if kvtype == "bf16":
        k, v = synth.bf16_bits(k), synth.bf16_bits(v)
    q = synth.bf16_bits(rng.standard_normal((2, n_q, H, 128)).astype(np.float32))
    case = dict(spec=dict(kv=kvtype, q="bf16"), lengths=np.array(lens), row_start=np.array([0, lens[0]]),
                q_full=q, q_sparse=[q], k=k, v=v, needles=[[], []])
    up = Uploaded(case)
    res = _run_block(up, top_k=200, window=16)
    for i in range(2):
        _check_seq(up, res, i, top_k=200, window=16)


@pytest.mark.parametrize("top_k,window", [(0, 32), (50, 0)])
def test_degenerate_budgets(top_k, window):
    """The full layer and the sparse layers with no global budget (the window alone) and with no
    window (the global tokens alone), bf16 and a length shorter than the window."""
    banner(f"degenerate budgets top_k={top_k} window={window}")
    up = Uploaded(synth.decode_case(2, B=3, lengths=[300, 20, 2000]))
    res = _run_block(up, top_k=top_k, window=window)
    for i in range(3):
        _check_seq(up, res, i, top_k=top_k, window=window)


def test_fp8_cache_h64_q4():
    """Config 3's shape (H=64, 4 query tokens, FP8 E4M3 with per-token scales,
    near-duplicate key clusters) at a 64K context."""
    banner("fp8 cache L=65536 H=64 n_q=4")
    up = Uploaded(synth.decode_case(3, L=65536))
    res = _run_block(up)
    stats = {}
    _check_seq(up, res, 0, stats=stats)
    assert stats["hit"] / stats["tot"] >= 0.999
    print(f"[result] fp8 64K max|dO| {stats['err']:.3e} sparse {stats['serr']:.3e} "
          f"{_recall_report(stats)}", flush=True)


def test_determinism_bitwise():
    banner("determinism: two runs of a bf16 ragged case")
    up = Uploaded(synth.decode_case(2, B=3, lengths=[5000, 70000, 1200]))
    a = _run_block(up)
    b = _run_block(up)
    for key in ("out", "lse", "idx", "cnt", "scores"):
        # score entries past a shorter list's candidates stay as poisoned (NaN) in both runs
        assert np.array_equal(a[key], b[key], equal_nan=key == "scores"), key
    for x, y in zip(a["sparse"], b["sparse"]):
        assert np.array_equal(x, y)


@pytest.mark.slow
def test_config2_full_size():
    """Config 2 at full size in the benchmark's launch configuration: 32 sequences
    of 131072 rows, bf16, 64 needles each, 1 full + 5 sparse layers.  Oracle on
    every sequence (outputs, LSE, scores, lists, recall, sparse layers); needles."""
    banner("config 2 full size: B=32 L=131072 H=32 bf16")
    up = Uploaded(synth.decode_case(2))
    res = _run_block(up)
    _same_lists_without_scores(up, res)
    stats = {}
    for i in range(32):
        banner(f"config 2 oracle on sequence {i}")
        _check_seq(up, res, i, stats=stats)
    assert stats["hit"] / stats["tot"] >= 0.999
    for i in range(32):
        sel = set(res["idx"][i, 0, 0, :1152].tolist())
        for (p, t, h) in up.case["needles"][i]:
            assert p in sel, ("needle", i, p, h)
    print(f"[result] config2 max|dO| {stats['err']:.3e} sparse {stats['serr']:.3e} "
          f"{_recall_report(stats)}", flush=True)


@pytest.mark.slow
def test_config3_full_size():
    banner("config 3 full size: L=1048576 H=64 n_q=4 fp8")
    up = Uploaded(synth.decode_case(3))
    res = _run_block(up)
    stats = {}
    _check_seq(up, res, 0, stats=stats)
    assert stats["hit"] / stats["tot"] >= 0.999
    print(f"[result] config3 max|dO| {stats['err']:.3e} sparse {stats['serr']:.3e} "
          f"{_recall_report(stats)}", flush=True)


@pytest.mark.slow
def test_config5_full_size():
    """Config 5 at full size in the benchmark's launch configuration: 8 ragged sequences of
    64K-512K rows, bf16, H=32, 1 full + 5 sparse layers per block, each of the 4 blocks with its
    own cache and queries.  The oracle checks every sequence of every block."""
    stats = {}
    for blk in range(4):
        banner(f"config 5 full size: block {blk}")
        up = Uploaded(synth.decode_case(5, block=blk))
        res = _run_block(up)
        _same_lists_without_scores(up, res)
        lens = up.case["lengths"]
        for i in range(len(lens)):
            banner(f"config 5 block {blk}: oracle on sequence {i} (L={int(lens[i])})")
            _check_seq(up, res, i, stats=stats)
        del up, res
        torch.cuda.empty_cache()
    assert stats["hit"] / stats["tot"] >= 0.999
    print(f"[result] config5 max|dO| {stats['err']:.3e} sparse {stats['serr']:.3e} "
          f"{_recall_report(stats)}", flush=True)


def test_block_level_variant_bf16():
    """The earlier block-level selection through the full layer: lists equal the oracle's block
    selection on the GPU's own scores (float32 tree order), overlap the float64 block selection,
    and sparse layers over the block lists match the oracle."""
    from long_context_split_amd import hysparse as hs
    lens = [1, 300, 1153, 1217, 20000, 70001]
    banner(f"block-level variant bf16 lens={lens}")
    up = Uploaded(synth.decode_case(2, B=len(lens), lengths=lens))
    kv = up.kv
    B, n_q, H, _ = up.q_full.shape
    S = hs.scores_stride(kv, 128)
    sc = torch.empty((B, n_q, 1, S), dtype=torch.float32, device="cuda")
    out, lse, idx, cnt = hs.full_attn_select(kv, up.q_full, scores_out=sc, select_block=64)
    so = hs.sparse_attn(kv, up.q_sparse[0], idx, cnt)
    torch.cuda.synchronize()
    sc, idx, cnt, so = sc.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), so.cpu().numpy()
    hit = tot = 0
    for i, L in enumerate(lens):
        w = min(128, L)
        q, k, v = up.oracle_seq(i)
        ref = block.full_layer(q, k, v, 1024, 128)
        gi, gc = selection.select_blocks(np.ascontiguousarray(sc[i, 0, 0, :L - w]), L, 1024, 128, f32_tree=True)
        assert cnt[i, 0, 0] == gc and np.array_equal(idx[i, 0, 0], gi), f"seq {i}: block lists"
        oi, oc = selection.select_blocks(ref["s"][0, 0], L, 1024, 128)
        assert gc == oc
        # order-free check on the same float32 scores: with float64 block sums, no unchosen block
        # beats a chosen one by more than the float32 pairwise tree can move two sums (six levels
        # of rounding on non-negative terms: at most 6 u (1 + u)^6 relative each, u = 2^-24)
        n = L - w
        bs64 = selection.block_scores(sc[i, 0, 0, :n].astype(np.float64))
        chosen = np.zeros(bs64.shape[0], dtype=bool)
        chosen[np.unique(gi[:gc - w] // 64)] = True
        if 0 < chosen.sum() < chosen.size:
            eps = 7.0 * 2.0 ** -24
            assert bs64[chosen].min() * (1 + eps) >= bs64[~chosen].max() * (1 - eps), f"seq {i}: block dominance"
        g = set(gi[:gc - w].tolist())
        r = set(oi[:oc - w].tolist())
        hit += len(g & r)
        tot += max(1, len(r))
        qs, _, _ = up.oracle_seq(i, "sparse", 0)
        ref_o, _ = attention.sparse_attention(qs, k, v, idx[i], cnt[i])
        assert np.abs(so[i] - ref_o).max() <= 2e-3
    assert hit / tot >= 0.99

