"""A decode step captured in a HIP graph replays identically to the eager calls.

The benchmark may time the step as a graph replay, so the captured sequence of
library launches (full layer + selection + sparse layers) is replayed several
times, with unrelated eager work and synchronisations between replays, and
every replay's outputs are compared bit for bit with the eager results.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_cases import Uploaded, banner

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    from long_context_split_amd import hysparse as hs
    banner("graph replay of a bf16 decode step")
    up = Uploaded(synth.decode_case(2, B=4, lengths=[70000, 5000, 131072, 900]))
    kv, qf, qs = up.kv, up.q_full, up.q_sparse[:2]
    B, n_q, H, _ = qf.shape
    dev = qf.device
    p = hs.params(H, n_q)
    out = torch.empty((B, n_q, H, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev)
    idx = torch.empty((B, n_q, 1, 1152), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, n_q, 1), dtype=torch.int32, device=dev)
    so = [torch.empty((B, n_q, H, 128), dtype=torch.float32, device=dev) for _ in qs]
    wsf = hs.workspace(hs.full_attn_select_workspace_size(kv, p), dev)
    wss = hs.workspace(hs.sparse_attn_workspace_size(kv, p), dev)

    def step():
        hs.full_attn_select(kv, qf, out=out, lse=lse, sel_idx=idx, sel_count=cnt, ws=wsf)
        for q, o in zip(qs, so):
            hs.sparse_attn(kv, q, idx, cnt, out=o, ws=wss)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, idx, cnt, *so)]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):            # warm the capture stream, as torch recommends
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.randn(1 << 22, device=dev)
    for rep in range(4):
        for t in (out, lse, so[0], so[1]):
            t.fill_(float("nan"))
        idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for r, t in zip(ref, (out, lse, idx, cnt, *so)):
            assert torch.equal(r, t), f"replay {rep} differs from the eager step"
        scratch.mul_(1.0001).add_(0.5)           # unrelated eager work between replays
        step()                                   # and an eager step on the same buffers
        torch.cuda.synchronize()
