"""Helpers of the GPU tests: upload seeded synthetic cases, and build the oracle's
float64 view of exactly the bytes the GPU sees."""

import numpy as np
import torch

import synth
from oracle import block, bridge as obridge


def banner(msg):
    print(f"[case] {msg}", flush=True)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_q(q, qtype):
    if qtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    return dev_bf16(q)


class Uploaded:
    """A decode case on the device plus the stored host values the oracle uses."""

    def __init__(self, case):
        from long_context_split_amd import hysparse as hs
        self.case = case
        spec = case["spec"]
        self.kvtype = spec["kv"]
        self.qtype = spec["q"]
        if self.kvtype == "bf16":
            k = dev_bf16(case["k"])
            v = dev_bf16(case["v"])
            self.k_store, self.v_store = case["k"], case["v"]
            self.k_scale = self.v_scale = None
            ks = vs = None
        elif self.kvtype == "f32":
            k = torch.from_numpy(case["k"]).cuda()
            v = torch.from_numpy(case["v"]).cuda()
            self.k_store, self.v_store = case["k"], case["v"]
            self.k_scale = self.v_scale = None
            ks = vs = None
        else:  # e4m3 stored by the oracle's quantiser, so both sides read the same bytes
            n, n_kv, d = case["k"].shape
            kc, ksc = obridge.quantize_rows_e4m3(case["k"].reshape(n * n_kv, d))
            vc, vsc = obridge.quantize_rows_e4m3(case["v"].reshape(n * n_kv, d))
            self.k_store, self.v_store = kc.reshape(n, n_kv, d), vc.reshape(n, n_kv, d)
            self.k_scale, self.v_scale = ksc.reshape(n, n_kv), vsc.reshape(n, n_kv)
            k = torch.from_numpy(self.k_store).cuda()
            v = torch.from_numpy(self.v_store).cuda()
            ks = torch.from_numpy(self.k_scale).cuda()
            vs = torch.from_numpy(self.v_scale).cuda()
        self.kv = hs.KVCache(k, v, case["lengths"], case["row_start"], ks, vs)
        self.q_full = dev_q(case["q_full"], self.qtype)
        self.q_sparse = [dev_q(q, self.qtype) for q in case["q_sparse"]]

    def oracle_seq(self, i, which="full", layer=0):
        """float64 (q, k, v) of sequence i as the GPU sees them."""
        L = int(self.case["lengths"][i])
        r0 = int(self.case["row_start"][i])
        sl = slice(r0, r0 + L)
        if self.kvtype == "e4m3":
            k = block.cache_values(self.k_store[sl], "e4m3", self.k_scale[sl])
            v = block.cache_values(self.v_store[sl], "e4m3", self.v_scale[sl])
        else:
            k = block.cache_values(self.k_store[sl], self.kvtype)
            v = block.cache_values(self.v_store[sl], self.kvtype)
        qsrc = self.case["q_full"] if which == "full" else self.case["q_sparse"][layer]
        q = block.cache_values(qsrc[i], self.qtype)
        return q, k, v


def recall(gpu_idx, gpu_cnt, ref_idx, ref_cnt, L, top_k, window, ref_scores=None):
    """Global-part recall of one list (window excluded): (|G_gpu & G_ref|, |G_ref|, tie-aware hits).

    Tie-aware hits count a GPU-selected j as correct when the oracle's score of j reaches the
    oracle's k'-th score times (1 - 1e-6), so swaps among near-tied scores at the boundary are
    not counted as misses (equal to the plain hits when ref_scores is None)."""
    kk = max(0, min(top_k, L - window))
    g = set(gpu_idx[:kk].tolist())
    r = set(ref_idx[:kk].tolist())
    hit = len(g & r)
    tie = hit
    if ref_scores is not None and kk > 0:
        kth = np.min(ref_scores[ref_idx[:kk]])
        tie = sum(1 for j in g if ref_scores[j] >= kth * (1.0 - 1e-6))
    return hit, len(r), tie


def f32_scores_view(scores_dev, b, t, g, n):
    return scores_dev[b, t, g, :n].float().cpu().numpy()
