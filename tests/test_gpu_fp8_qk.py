"""The many-row dense pass with Q K^T on FP8 MFMA (opt-in, E4M3 caches), measured against the
float64 oracle of the exact method with the bf16 form's gates:

  G2 global-part recall >= 0.999 (plus the tie-aware recall and the worst list);
  G3 max |O - O_oracle| <= 3e-2 for the full layer and every sparse layer.

The selection scores still come from the bf16 score pass; what the FP8 products change is the
full layer's O and LSE (Q rounded to E4M3 per query row), and through the LSE each head's weight
in the scores.  Measured on MI355X: G3 holds with a wide margin (max |dO| about 8e-4), but the LSE
moves by about 1e-3 relative and recall falls to 0.997 at 64K and 0.991 at 1M rows (tie-aware
recall the same: the swapped rows are not near-ties), below G2, and the sparse layers on the moved
lists differ from the exact method's (the oracle on its own lists) by up to 6e-2 to 8e-2.  The variant is therefore not
adopted: the switch (HS_MANY_ROW_FP8_QK=1) stays off by default.  These tests hold G3 and the
list shapes, require recall >= 0.98 (a broken product would drop it far lower) and print the
measured G2 figures.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import attention, block, selection
from gpu_cases import Uploaded, banner, recall

pytestmark = pytest.mark.gpu

TOL_FP8 = 3e-2


def _run(up, top_k=1024, window=128):
    from long_context_split_amd import hysparse as hs
    kv = up.kv
    B, n_q, H, _ = up.q_full.shape
    nan = float("nan")
    out, lse, idx, cnt = hs.full_attn_select(
        kv, up.q_full, top_k, window,
        out=torch.full((B, n_q, H, 128), nan, dtype=torch.float32, device="cuda"),
        lse=torch.full((B, n_q, H), nan, dtype=torch.float32, device="cuda"),
        sel_idx=torch.full((B, n_q, kv.n_kv, top_k + window), -0x7F7F7F7F, dtype=torch.int32, device="cuda"),
        sel_count=torch.full((B, n_q, kv.n_kv), -0x7F7F7F7F, dtype=torch.int32, device="cuda"))
    sparse = [hs.sparse_attn(kv, q, idx, cnt, top_k, window,
                             out=torch.full((B, n_q, H, 128), nan, dtype=torch.float32, device="cuda"))
              for q in up.q_sparse]
    torch.cuda.synchronize()
    return dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(), idx=idx.cpu().numpy(), cnt=cnt.cpu().numpy(),
                sparse=[s.cpu().numpy() for s in sparse])


def _gates(up, res, i=0, top_k=1024, window=128):
    """Measured G2 / G3 quantities of sequence i (no assertion inside: the caller prints, then gates)."""
    L = int(up.case["lengths"][i])
    q, k, v = up.oracle_seq(i)
    ref = block.full_layer(q, k, v, top_k, window)
    st = dict(err=float(np.abs(res["out"][i] - ref["o"]).max()),
              lse_rel=float(np.abs(res["lse"][i] - ref["lse"]).max() / max(1.0, np.abs(ref["lse"]).max())),
              hit=0, tot=0, tie=0, worst=1.0, serr=0.0, counts_ok=True)
    n_q, n_kv = ref["cnt"].shape
    w, kk = selection.budget(L, top_k, window)
    for t in range(n_q):
        for g in range(n_kv):
            st["counts_ok"] &= bool(res["cnt"][i, t, g] == ref["cnt"][t, g] == kk + w)
            h, n, th = recall(res["idx"][i, t, g], res["cnt"][i, t, g], ref["idx"][t, g], ref["cnt"][t, g], L,
                              top_k, window, ref["s"][t, g])
            st["hit"] += h
            st["tot"] += n
            st["tie"] += th
            if n:
                st["worst"] = min(st["worst"], h / n)
    st["serr_own"] = 0.0
    for layer in range(len(up.q_sparse)):
        qs, _, _ = up.oracle_seq(i, "sparse", layer)
        so, _ = attention.sparse_attention(qs, k, v, res["idx"][i], res["cnt"][i])
        st["serr"] = max(st["serr"], float(np.abs(res["sparse"][layer][i] - so).max()))
        # second report: the oracle on its own lists (the rows the rounded Q moved across the boundary)
        so_own, _ = attention.sparse_attention(qs, k, v, ref["idx"], ref["cnt"])
        st["serr_own"] = max(st["serr_own"], float(np.abs(res["sparse"][layer][i] - so_own).max()))
    return st


def _variant(monkeypatch, cfg_kwargs, label):
    banner(f"FP8 Q K^T many-row pass: {label}")
    up = Uploaded(synth.decode_case(3, **cfg_kwargs))
    base = _run(up)
    monkeypatch.setenv("HS_MANY_ROW_FP8_QK", "1")
    res = _run(up)
    monkeypatch.delenv("HS_MANY_ROW_FP8_QK")
    st = _gates(up, res)
    d_bf16 = float(np.abs(res["out"] - base["out"]).max())
    same_lists = float(np.mean(res["idx"] == base["idx"]))
    print(f"[result] fp8-qk {label}: G3 full max|dO| {st['err']:.3e} sparse {st['serr']:.3e} "
          f"(vs the bf16 form: max|dO| {d_bf16:.3e}, list entries equal {same_lists:.6f}); "
          f"LSE rel {st['lse_rel']:.2e}; G2 recall {st['hit'] / st['tot']:.6f} "
          f"tie-aware {st['tie'] / st['tot']:.6f} worst list {st['worst']:.6f}; sparse vs the oracle's own "
          f"lists {st['serr_own']:.3e}", flush=True)
    assert st["counts_ok"]
    assert st["err"] <= TOL_FP8 and st["serr"] <= TOL_FP8             # G3
    assert st["hit"] / st["tot"] >= 0.98                              # below G2's 0.999: not adopted
    # the switch is read per call: the bf16 form is back
    again = _run(up)
    assert np.array_equal(again["out"], base["out"]) and np.array_equal(again["idx"], base["idx"])


def test_fp8_qk_h64_q4_64k(monkeypatch):
    _variant(monkeypatch, dict(L=65536), "L=65536 H=64 n_q=4")


@pytest.mark.slow
def test_fp8_qk_config3_full_size(monkeypatch):
    _variant(monkeypatch, {}, "config 3 full size L=1048576")


@pytest.mark.parametrize("n_kv,H,n_q", [(2, 32, 4), (1, 64, 2), (1, 128, 2)])
def test_fp8_qk_row_group_counts(monkeypatch, n_kv, H, n_q):
    """The FP8 product form at each row-group count of the many-row kernel (R = 64, 128, 256 rows per
    KV head: 2, 4 and 8 waves), two KV heads, lengths ending inside a super-tile: G3 on the full
    layer and on the sparse layers (oracle on the GPU's own lists)."""
    banner(f"FP8 Q K^T many-row pass: n_kv={n_kv} H={H} n_q={n_q}")
    rng = np.random.default_rng(70 + H + n_q + n_kv)
    lens = [5000, 777]
    tot = sum(lens)
    k = rng.standard_normal((tot, n_kv, 128)).astype(np.float32)
    v = rng.standard_normal((tot, n_kv, 128)).astype(np.float32)
    q = synth.bf16_bits(rng.standard_normal((2, n_q, H, 128)).astype(np.float32))
    case = dict(spec=dict(kv="e4m3", q="bf16"), lengths=np.array(lens), row_start=np.array([0, lens[0]]),
                q_full=q, q_sparse=[q], k=k, v=v, needles=[[], []])
    up = Uploaded(case)
    monkeypatch.setenv("HS_MANY_ROW_FP8_QK", "1")
    res = _run(up, top_k=200, window=16)
    monkeypatch.delenv("HS_MANY_ROW_FP8_QK")
    for i in range(2):
        st = _gates(up, res, i, top_k=200, window=16)
        print(f"[result] fp8-qk n_kv={n_kv} H={H} n_q={n_q} seq {i}: max|dO| {st['err']:.3e} sparse "
              f"{st['serr']:.3e} LSE rel {st['lse_rel']:.2e} recall {st['hit'] / st['tot']:.4f}", flush=True)
        assert st["counts_ok"]
        assert st["err"] <= TOL_FP8 and st["serr"] <= TOL_FP8
        assert st["lse_rel"] <= 1e-2
