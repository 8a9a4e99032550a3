"""Selection stage on the GPU, bit for bit against the oracle on identical float32
score tensors (adversarial ties, plateaus, signs, zeros, subnormals, edge lengths)."""

import numpy as np
import pytest
import torch

from oracle import selection
from gpu_cases import banner

pytestmark = pytest.mark.gpu


def _pattern(kind, n, rng):
    if kind == "random":
        return rng.random(n).astype(np.float32)
    if kind == "equal":
        return np.full(n, 0.125, np.float32)
    if kind == "plateau":       # a large block of ties straddles the k-th position
        x = np.full(n, 0.5, np.float32)
        x[rng.choice(n, min(n, 600), replace=False)] = 2.0
        x[rng.choice(n, min(n, 3000), replace=False)] = 1.0
        return x
    if kind == "zeros":
        return np.zeros(n, np.float32)
    if kind == "signed":
        x = rng.standard_normal(n).astype(np.float32)
        x[::7] = -0.0
        x[::11] = 0.0
        return x
    if kind == "subnormal":
        return (rng.integers(0, 50, n) * np.float32(1e-45)).astype(np.float32)
    if kind == "coarse":        # few distinct values -> many ties everywhere
        return (rng.integers(0, 5, n) / 4).astype(np.float32)
    raise ValueError(kind)


KINDS = ["random", "equal", "plateau", "zeros", "signed", "subnormal", "coarse"]


def _check(scores, lens, q_tokens, n_kv, top_k, window):
    from long_context_split_amd import hysparse as hs
    d = torch.from_numpy(scores).cuda()
    idx, cnt = hs.select_from_scores(d, lens, q_tokens, n_kv, top_k, window)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b, L in enumerate(lens):
        n = L - min(window, L)
        for t in range(q_tokens):
            for g in range(n_kv):
                ri, rc = selection.select(scores[b, t, g, :n], L, top_k, window, f32_keys=True)
                assert cnt[b, t, g] == rc, (b, t, g, L)
                assert np.array_equal(idx[b, t, g], ri), (b, t, g, L)


@pytest.mark.parametrize("kind", KINDS)
def test_select_bit_exact_edge_lengths(kind):
    banner(f"select kind={kind}")
    lens = [1, 2, 127, 128, 129, 1151, 1152, 1153, 2000, 5000, 70001]
    S = max(lens) - 128
    rng = np.random.default_rng(100 + KINDS.index(kind))
    scores = np.zeros((len(lens), 1, 1, S), np.float32)
    for b, L in enumerate(lens):
        n = L - min(128, L)
        scores[b, 0, 0, :n] = _pattern(kind, n, rng)
    _check(scores, lens, 1, 1, 1024, 128)


def test_select_many_queries_and_kv_heads():
    banner("select q_tokens=3 n_kv=2 small budgets")
    rng = np.random.default_rng(7)
    lens = [50, 300, 4099]
    full = (rng.integers(0, 9, (3, 3, 2, max(lens))) / 8).astype(np.float32)
    _check(np.ascontiguousarray(full[..., :max(lens) - 4]), lens, 3, 2, 16, 4)
    _check(full, lens, 3, 2, 100, 0)


def test_select_zero_budgets():
    """Degenerate budgets: no global tokens (top_k 0: the window alone) and no window (the global
    tokens alone)."""
    banner("select top_k=0 / window=0")
    rng = np.random.default_rng(13)
    lens = [1, 100, 129, 3000]
    full = rng.random((4, 2, 1, max(lens))).astype(np.float32)
    _check(np.ascontiguousarray(full[..., :max(lens) - 128]), lens, 2, 1, 0, 128)
    _check(full, lens, 2, 1, 50, 0)


def test_select_one_million_candidates():
    banner("select L=1048576")
    rng = np.random.default_rng(9)
    L = 1 << 20
    n = L - 128
    x = (rng.random(n) * 1e-4).astype(np.float32)
    x[rng.choice(n, 1500, replace=False)] = np.float32(3e-4)        # ties at the boundary
    _check(x.reshape(1, 1, 1, n), [L], 1, 1, 1024, 128)


def test_select_more_than_four_million_candidates():
    """Over 4M candidates the per-chunk kernels take several batches per workgroup; the
    second list puts every score into one first-digit bin (millions of candidates)."""
    banner("select L=5000128, two lists")
    rng = np.random.default_rng(11)
    L = 5_000_128
    n = L - 128
    x = np.empty((2, 1, 1, n), np.float32)
    x[0, 0, 0] = rng.random(n, dtype=np.float32)
    x[1, 0, 0] = (1.0 + rng.random(n) * 0.01).astype(np.float32)
    _check(x, [L, L], 1, 1, 1024, 128)


def _check_blocks(scores, lens, q_tokens, n_kv, top_k, window):
    from long_context_split_amd import hysparse as hs
    d = torch.from_numpy(scores).cuda()
    idx, cnt = hs.select_from_scores(d, lens, q_tokens, n_kv, top_k, window, select_block=64)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b, L in enumerate(lens):
        n = L - min(window, L)
        for t in range(q_tokens):
            for g in range(n_kv):
                ri, rc = selection.select_blocks(scores[b, t, g, :n], L, top_k, window, f32_tree=True)
                assert cnt[b, t, g] == rc, (b, t, g, L)
                assert np.array_equal(idx[b, t, g], ri), (b, t, g, L)


@pytest.mark.parametrize("kind", KINDS)
def test_select_blocks_bit_exact(kind):
    """Block-level variant: 64-token block sums in the float32 tree order, then the same ranking and
    tie rule, bit for bit against the oracle on identical scores (partial last blocks included)."""
    banner(f"select blocks kind={kind}")
    lens = [1, 127, 128, 129, 1151, 1152, 1153, 1217, 2000, 5000, 70001]
    S = max(lens) - 128
    rng = np.random.default_rng(200 + KINDS.index(kind))
    scores = np.zeros((len(lens), 1, 1, S), np.float32)
    for b, L in enumerate(lens):
        n = L - min(128, L)
        scores[b, 0, 0, :n] = _pattern(kind, n, rng)
    _check_blocks(scores, lens, 1, 1, 1024, 128)


def test_select_blocks_budgets_and_long_list():
    banner("select blocks budgets, q_tokens=2, n_kv=2, L=1048576")
    rng = np.random.default_rng(12)
    lens = [3000, 777]
    full = (rng.integers(0, 9, (2, 2, 2, max(lens))) / 8).astype(np.float32)
    # the score tensor's last dimension is max_len - window
    _check_blocks(np.ascontiguousarray(full[..., :max(lens) - 16]), lens, 2, 2, 200, 16)   # 3 blocks, ties
    _check_blocks(np.ascontiguousarray(full[..., :max(lens) - 4]), lens, 2, 2, 40, 4)      # < one block
    L = 1 << 20
    x = (rng.random(L - 128) * 1e-4).astype(np.float32)
    x[rng.choice(L - 128, 300, replace=False)] = np.float32(5e-3)
    _check_blocks(x.reshape(1, 1, 1, -1), [L], 1, 1, 1024, 128)


@pytest.mark.parametrize("n_q,H,L,B,ragged", [(1, 32, 40000, 16, False), (1, 32, 1153, 16, False),
                                              (1, 32, 300, 16, False), (2, 16, 40000, 16, False),
                                              (1, 32, 9000, 272, False), (1, 32, 129, 16, False),
                                              (1, 32, 100, 16, False), (1, 32, 20000, 20, False),
                                              (1, 32, 20000, 40, False), (1, 32, 40000, 5, False),
                                              (1, 32, 60000, 8, True), (1, 32, 3000, 4, True),
                                              (1, 32, 20000, 33, True)])
def test_candidate_selection_paths_agree(n_q, H, L, B, ragged, monkeypatch):
    """The full layer's selection four ways: the score filter (the default for one query token
    without dense scores: bounds from the dense pass's codes, exact scores only for the tokens
    that can reach the k'-th), the candidates the score pass appends (candidate mode, for one query
    token and at least 16 lists, lowered to 4 here so the few-list cases take it too), the same with
    the dense scores requested, and the dense three-kernel radix select.  All give identical lists,
    and the one with scores equals the oracle's selection on those scores.
    L = 1153 leaves most score workgroups without work, L = 300 selects every candidate, 272 lists
    get one score workgroup each (almost every unit is taken from the list's counter), L = 129
    leaves one candidate and L = 100 none (the window takes every row), 20 and 40 lists get 12 and 6
    score workgroups each (not aligned with the 8 XCDs), 5 lists get 51 each; ragged batches (lengths
    drawn in [L/8, L], a list's workgroup count proportional to its candidates; the 3000 case has
    lists shorter than the budget); the last sequence has identical K rows, so every score ties
    and the lowest indices must win."""
    import synth
    from long_context_split_amd import hysparse as hs
    banner(f"candidate vs dense selection n_q={n_q} H={H} L={L} B={B} ragged={ragged}")
    monkeypatch.setenv("HS_CAND_MIN_LISTS", "4")
    rng = np.random.default_rng(21 + n_q + L + B)
    lens = [int(x) for x in rng.integers(max(1, L // 8), L + 1, B)] if ragged else [L] * B
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    tot = int(sum(lens))
    k = rng.standard_normal((tot, 1, 128)).astype(np.float32)
    k[starts[-1]:] = k[starts[-1]]                                # identical rows: all scores tied
    v = rng.standard_normal((tot, 1, 128)).astype(np.float32)
    q = rng.standard_normal((B, n_q, H, 128)).astype(np.float32)
    dev = lambda x: torch.from_numpy(synth.bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)
    kv = hs.KVCache(dev(k), dev(v), lens, starts)
    qd = dev(q)
    _, _, idx_a, cnt_a = hs.full_attn_select(kv, qd)
    S = hs.scores_stride(kv, 128)
    sc = torch.empty((B, n_q, 1, max(S, 1)), dtype=torch.float32, device="cuda")
    _, _, idx_b, cnt_b = hs.full_attn_select(kv, qd, scores_out=sc)
    monkeypatch.setenv("HS_SCORE_FILTER", "0")
    _, _, idx_d, cnt_d = hs.full_attn_select(kv, qd)
    monkeypatch.setenv("HS_DENSE_SELECT", "1")
    _, _, idx_c, cnt_c = hs.full_attn_select(kv, qd)
    torch.cuda.synchronize()
    ia, ib, ic, idd = idx_a.cpu().numpy(), idx_b.cpu().numpy(), idx_c.cpu().numpy(), idx_d.cpu().numpy()
    assert np.array_equal(ia, ib) and np.array_equal(ia, ic) and np.array_equal(ia, idd)
    assert np.array_equal(cnt_a.cpu().numpy(), cnt_c.cpu().numpy())
    assert np.array_equal(cnt_d.cpu().numpy(), cnt_c.cpu().numpy())
    scores = sc.cpu().numpy()
    for i in range(B):
        Li = lens[i]
        w, kk = selection.budget(Li, 1024, 128)
        for t in range(n_q):
            gi, gc = selection.select(np.ascontiguousarray(scores[i, t, 0, :Li - w]), Li, 1024, 128, f32_keys=True)
            assert np.array_equal(ia[i, t, 0], gi), f"seq {i} t {t}"
    w, kk = selection.budget(lens[-1], 1024, 128)
    last = ia[-1, :, 0, :kk]
    assert np.array_equal(last, np.broadcast_to(np.arange(kk), last.shape))
