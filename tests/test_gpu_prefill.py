"""Prefill of one prompt in consecutive chunks (hs_prefill_chunk): the Self-Decoder's sliding-window
attention of each chunk over its growing cache, with bands that reach back across chunk boundaries,
and the KV Bridging of each chunk's hidden states into four Cross-Decoder targets at advancing row
offsets.  Each chunk's attention output is checked against the float64 oracle (sliding-window
attention over the rows as stored), the targets against the oracle's bridge of the whole prompt
(the storage tolerances of the bridge tests), and the rows outside the prompt's range stay
untouched."""

import numpy as np
import pytest
import torch

import synth
from oracle import swa, block
from gpu_cases import banner, dev_bf16
from test_gpu_bridge import SENT8, SENTF, _targets, _host, _check_random, _untouched

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fp8,chunks,w,out16", [(True, [700, 700, 613], 256, True),
                                                (False, [512, 1024, 300, 77], 600, False)])
def test_prefill_chunks_feed_bridge_targets(fp8, chunks, w, out16):
    """out16: the attention output in bf16, checked within the float32 bound plus half a bf16 step."""
    from oracle import bf16
    from long_context_split_amd import hysparse as hs
    banner(f"prefill chunks={chunks} w={w} fp8 targets={fp8} bf16 attention output={out16}")
    P, H, D, nt, base = sum(chunks), 32, 512, 4, 1000
    rng = np.random.default_rng(60 + len(chunks))
    k = synth.bf16_bits(rng.standard_normal((P, 1, 128)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((P, 1, 128)).astype(np.float32))
    q = synth.bf16_bits((1.5 * rng.standard_normal((P, H, 128))).astype(np.float32))
    case = synth.bridge_case(4, T=P, D=D, n_targets=nt)
    kd, vd = dev_bf16(k), dev_bf16(v)
    x = dev_bf16(case["x"])
    wk = [dev_bf16(m) for m in case["w_k"]]
    wv = [dev_bf16(m) for m in case["w_v"]]
    cap = base + P + 50
    tg = _targets(nt, cap, fp8)
    outs = []
    start = 0
    for T in chunks:
        end = start + T
        self_kv = hs.KVCache(kd, vd, [end], [0])                       # the cache grown by this chunk
        qc = dev_bf16(q[start:end]).reshape(1, T, H, 128)
        o = torch.full((1, T, H, 128), float("nan"), dtype=torch.bfloat16 if out16 else torch.float32, device="cuda")
        hs.prefill_chunk(self_kv, qc, w, x[start:end], wk, wv, tg, base + start, swa_out=o)
        outs.append(o)
        start = end
    torch.cuda.synchronize()
    kf = block.cache_values(k, "bf16")
    vf = block.cache_values(v, "bf16")
    worst = 0.0
    start = 0
    for T, o in zip(chunks, outs):
        end = start + T
        ref = swa.swa_attention(block.cache_values(q[start:end], "bf16"), kf[:end], vf[:end], w)
        if out16:
            got = bf16.decode(o[0].view(torch.int16).cpu().numpy().view(np.uint16))
            err = float(np.max(np.abs(got - ref) - np.ldexp(1.0, np.frexp(np.abs(ref) + 2e-3)[1] - 9)))
        else:
            err = float(np.abs(o[0].cpu().numpy() - ref).max())
        worst = max(worst, err)
        assert err <= 2e-3, f"chunk at {start}: max-abs {err}"
        start = end
    eq = _check_random(case, tg, base, fp8)
    assert eq >= 0.99
    for t in tg:
        kk, ks, vv, vs = _host(t, fp8)
        if fp8:
            assert _untouched(kk, base, base + P, SENT8) and _untouched(vs, base, base + P, SENTF)
        else:
            assert _untouched(kk, base, base + P, 0x1234)
    print(f"[result] prefill {len(chunks)} chunks: swa max-abs {worst:.2e}, bridge equal fraction {eq:.5f}",
          flush=True)
