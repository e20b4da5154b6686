"""GPU parity of the QKV projection with the RoPE epilogue (ne_qkv_rope_proj) against the oracle
(oracle/qkv.py).  Products of bf16/fp16 inputs are exact in fp32 and accumulate in fp32, so the bar
is 1e-4 of each output's scale (fp32 outputs); 16-bit outputs add half an ulp of their format.
"""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding, inputs
from tests.test_gpu_parity import DEV, check, f64

pytestmark = pytest.mark.gpu

_NAME = {torch.bfloat16: "bf16", torch.float16: "f16"}


def check_qkv(name, got, ref, out_dt):
    got = got.double().numpy()
    scale = float(np.max(np.abs(ref)))
    assert np.all(np.isfinite(got)), name
    if out_dt == torch.float32:
        err = float(np.max(np.abs(got - ref)) / scale)
        assert err <= 1e-4, f"{name}: rel err {err:.3e}"
        return
    mant = 8 if out_dt == torch.bfloat16 else 11
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - (mant - 1))
    excess = np.abs(got - ref) - (1e-4 * scale + 0.5 * ulp)
    assert np.max(excess) <= 0, f"{name}: exceeds bar by {np.max(excess):.3e}"


def make(B, T, C, Hq, Hkv, D, seed, dtype):
    x = inputs.gaussian((B, T, C), seed, 1.0, dtype)
    w = inputs.gaussian(((Hq + 2 * Hkv) * D, C), seed + 1, 1.0 / np.sqrt(C), dtype)
    return x, w


@pytest.mark.parametrize("shape", [(2, 100, 128, 4, 2, 32), (1, 300, 256, 6, 1, 64), (2, 129, 192, 4, 2, 128),
                                   (1, 1, 64, 2, 1, 128)])
@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("variant", ["rope", "rope_qknorm", "plain"])
def test_qkv_parity(shape, in_dt, variant):
    B, T, C, Hq, Hkv, D = shape
    x, w = make(B, T, C, Hq, Hkv, D, 5000 + T, _NAME[in_dt])
    base = 0.0 if variant == "plain" else 1e4
    qkn = (1.2, 1e-6) if variant == "rope_qknorm" else None
    q, k, v = binding.ne_qkv_rope_proj(x.to(DEV), w.to(DEV), Hq, Hkv, base, qk_norm=qkn)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope_proj(f64(x), f64(w), Hq, Hkv, base, qk_norm=qkn)
    for nm, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_qkv(nm, g.cpu(), r, torch.float32)


# Shapes that select the wide-tile kernel: its 256-token x 320-feature tiling (without the QK norm,
# or with it for D <= 64) or its 128 x 640 tiling, each when the tiles cover at least three
# quarters of the compute units.  Ragged token counts, partial last tiles of heads, head sizes
# 32 / 64 / 128, and C from the minimum step count to several passes of the ring.
WIDE = [(1, 8100, 64, 12, 4, 128), (2, 4100, 320, 8, 2, 128), (1, 6200, 128, 16, 8, 64), (3, 4100, 192, 24, 8, 32),
        (2, 5000, 128, 16, 8, 64)]
VARIANTS = ["rope", "rope_qknorm", "plain"]


def tiling(B, T, Hq, Hkv, D, qk_norm, cus):
    """The host's choice in ne_qkv_rope_proj, restated."""
    M, N = B * T, (Hq + 2 * Hkv) * D
    t320 = -(-M // 256) * -(-N // 320)
    t640 = -(-M // 128) * -(-N // 640)
    if (not qk_norm or 320 % D == 0) and 4 * t320 >= 3 * cus:
        return "256x320"
    return "128x640" if 4 * t640 >= 3 * cus else "narrow"


def test_wide_shapes_cover_both_wide_tilings():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    seen = {}
    for B, T, C, Hq, Hkv, D in WIDE:
        for v in VARIANTS:
            t = tiling(B, T, Hq, Hkv, D, v == "rope_qknorm", cus)
            assert t != "narrow", (B, T, C, Hq, Hkv, D, v)
            seen.setdefault(t, set()).add((D, v))
    assert {(128, "rope"), (32, "rope_qknorm"), (64, "rope_qknorm"), (32, "plain")} <= seen["256x320"]
    assert {(128, "rope_qknorm"), (64, "rope"), (128, "plain")} <= seen["128x640"]


@pytest.mark.parametrize("shape", WIDE)
@pytest.mark.parametrize("variant", VARIANTS)
def test_qkv_wide_tiles_parity(shape, variant):
    B, T, C, Hq, Hkv, D = shape
    x, w = make(B, T, C, Hq, Hkv, D, 5500 + T + C, "bf16")
    base = 0.0 if variant == "plain" else 1e4
    qkn = (0.8, 1e-5) if variant == "rope_qknorm" else None
    q, k, v = binding.ne_qkv_rope_proj(x.to(DEV), w.to(DEV), Hq, Hkv, base, qk_norm=qkn)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope_proj(f64(x), f64(w), Hq, Hkv, base, qk_norm=qkn)
    for nm, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_qkv(nm, g.cpu(), r, torch.float32)


@pytest.mark.parametrize("out_dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("qk_norm", [None, (1.1, 1e-6)])   # D 128: 256 x 320 without, 128 x 640 with
def test_qkv_wide_tiles_16bit(out_dt, qk_norm):
    B, T, C, Hq, Hkv, D = WIDE[0]
    name = _NAME[out_dt]
    x, w = make(B, T, C, Hq, Hkv, D, 5600, name)
    q, k, v = binding.ne_qkv_rope_proj(x.to(DEV), w.to(DEV), Hq, Hkv, 5e5, qk_norm=qk_norm, out_dtype=out_dt)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope_proj(f64(x), f64(w), Hq, Hkv, 5e5, qk_norm=qk_norm)
    for nm, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_qkv(nm, g.cpu(), r, out_dt)


@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float16])
def test_qkv_16bit_outputs(in_dt):
    x, w = make(2, 200, 256, 8, 2, 64, 5100, _NAME[in_dt])
    q, k, v = binding.ne_qkv_rope_proj(x.to(DEV), w.to(DEV), 8, 2, 5e5, out_dtype=in_dt)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope_proj(f64(x), f64(w), 8, 2, 5e5)
    for nm, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_qkv(nm, g.cpu(), r, in_dt)


def test_qkv_workload_projection_sampled_tokens():
    """The projection of the wide GQA layer (B4 T2048, C = Hq D = 1536, Hq 12 / Hkv 4, D 128):
    full-size GPU run, oracle on sampled tokens at their positions."""
    B, T, Hq, Hkv, D = 4, 2048, 12, 4, 128
    C = Hq * D
    x, w = make(B, T, C, Hq, Hkv, D, 5200, "bf16")
    q, k, v = binding.ne_qkv_rope_proj(x.to(DEV), w.to(DEV), Hq, Hkv, 1e4)
    torch.cuda.synchronize()
    idx = np.array([0, 1, 255, 256, 1000, 2047])
    for b in (0, 3):
        rq, rk, rv = oracle.qkv_rope_proj(f64(x[b:b + 1, idx]), f64(w), Hq, Hkv, 1e4, positions=idx)
        for nm, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
            check_qkv(nm, g[b:b + 1, idx].cpu(), r, torch.float32)


def test_qkv_then_attention_without_rope_equals_attention_with_rope():
    B, T, C, Hq, Hkv, D = 1, 200, 256, 8, 2, 64
    x, w = make(B, T, C, Hq, Hkv, D, 5300, "bf16")
    xd, wd = x.to(DEV), w.to(DEV)
    q1, k1, v1 = binding.ne_qkv_rope_proj(xd, wd, Hq, Hkv, 1e4, out_dtype=torch.bfloat16)
    o1, l1 = binding.ne_rope_attn_fwd(q1, k1, v1, 0.0)
    q0, k0, v0 = binding.ne_qkv_rope_proj(xd, wd, Hq, Hkv, 0.0, out_dtype=torch.bfloat16)
    o2, l2 = binding.ne_rope_attn_fwd(q0, k0, v0, 1e4)
    torch.cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 4e-3 * float(o2.abs().max())
    assert float((l1 - l2).abs().max()) <= 4e-3 * float(l2.abs().max())


@pytest.mark.parametrize("shape", [(2, 300, 256, 6, 1, 64), WIDE[1], WIDE[4]])
def test_qkv_is_bitwise_deterministic(shape):
    B, T, C, Hq, Hkv, D = shape
    x, w = make(B, T, C, Hq, Hkv, D, 5400, "bf16")
    a = binding.ne_qkv_rope_proj(x.to(DEV), w.to(DEV), Hq, Hkv, 1e4, qk_norm=(1.0, 1e-6))
    a = [t.clone() for t in a]
    b = binding.ne_qkv_rope_proj(x.to(DEV), w.to(DEV), Hq, Hkv, 1e4, qk_norm=(1.0, 1e-6))
    for s, t in zip(a, b):
        assert torch.equal(s, t)
