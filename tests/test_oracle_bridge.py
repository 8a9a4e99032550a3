"""Pins of the oracle's KV Bridging projection and its storage quantisers."""

import numpy as np
import torch

from oracle import bridge, e4m3, bf16
import synth


def test_project_matches_python_loops():
    rng = np.random.default_rng(30)
    x = synth.bf16_bits(rng.standard_normal((3, 5)).astype(np.float32))
    w = synth.bf16_bits(rng.standard_normal((5, 4)).astype(np.float32))
    r = bridge.project(x, w)
    xd, wd = bf16.decode(x), bf16.decode(w)
    for i in range(3):
        for j in range(4):
            assert r[i, j] == sum(xd[i, t] * wd[t, j] for t in range(5))


def test_identity_weights_are_a_pure_quantiser():
    """With W = I (d_model = head_dim) the bridge only stores X's rows."""
    rng = np.random.default_rng(31)
    x = synth.bf16_bits((rng.standard_normal((64, 128)) * 3).astype(np.float32))
    eye = synth.bf16_bits(np.eye(128, dtype=np.float32))
    out = bridge.bridge(x, [eye], [eye], "bf16")[0]
    assert np.array_equal(out["k"], x) and np.array_equal(out["v"], x)
    q = bridge.bridge(x, [eye], [eye], "e4m3")[0]
    xf = bf16.decode(x).astype(np.float32)
    a = np.abs(xf).max(axis=1)
    assert np.array_equal(q["k_scale"], (a / np.float32(448)).astype(np.float32))
    # library pin: torch's e4m3fn cast of x / scale (in range, non-zero entries)
    y = (xf / q["k_scale"][:, None]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = np.where((ref & 0x7F) == 0, 0, ref)
    ok = np.abs(y) < 464
    assert np.array_equal(q["k"][ok], ref[ok])


def test_quantiser_properties():
    rng = np.random.default_rng(32)
    r = rng.standard_normal((500, 128)) * np.exp(rng.uniform(-8, 8, (500, 1)))
    r[3] = 0.0
    codes, scale = bridge.quantize_rows_e4m3(r)
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    nz = np.arange(500) != 3
    # the largest entry of each row lands on +-448 (code 0x7E / 0xFE)
    amax_idx = np.abs(r.astype(np.float32)).argmax(axis=1)
    assert np.all((codes[nz, amax_idx[nz]] & 0x7F) == 0x7E)
    # relative error of the stored value is at most half a step (2**-4) for normals
    deq = bridge.dequantize_rows_e4m3(codes, scale)
    r32 = r.astype(np.float32).astype(np.float64)
    big = np.abs(r32) >= (2.0 ** -6) * scale[:, None] * 1.0001
    rel = np.abs(deq - r32)[big] / np.abs(r32)[big]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
    small = ~big & (np.abs(r32) > 0)
    assert np.all(np.abs(deq - r32)[small] <= (2.0 ** -10) * np.broadcast_to(scale[:, None], r.shape)[small] * (1 + 1e-6))


def test_bridge_bf16_is_rne_of_exact_product():
    rng = np.random.default_rng(33)
    x = synth.bf16_bits(rng.standard_normal((16, 256)).astype(np.float32))
    w = synth.bf16_bits((rng.standard_normal((256, 128)) * 0.05).astype(np.float32))
    out = bridge.bridge(x, [w], [w], "bf16")[0]
    exact = bf16.decode(x) @ bf16.decode(w)
    ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    # fp64 -> bf16 directly can differ from fp64 -> fp32 -> bf16 only at double-rounding ties
    diff = np.abs(out["k"].astype(np.int32) - ref.view(np.uint16).astype(np.int32))
    assert diff.max() <= 1 and np.mean(diff == 0) > 0.999
    deq = bf16.decode(out["k"])
    assert np.all(np.abs(deq - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-300)


def test_e4m3_encode_is_used_by_quantiser():
    r = np.array([[448.0, 1.0, -0.5, 0.0]])
    codes, scale = bridge.quantize_rows_e4m3(r)
    assert scale[0] == 1.0
    assert list(codes[0]) == [0x7E, 0x38, 0xB0, 0x00]
    assert list(e4m3.decode(codes[0])) == [448.0, 1.0, -0.5, 0.0]
