"""GPU parity of the sliding-window entry points against the double-precision oracle.

Query t sees keys t - W + 1 .. t (the short-window layers of the nanochat guide's window_pattern
feature, section 模型架构速览: a quarter of the context).  Bars as in test_gpu_parity.py.
Windows are chosen so that blocks start at a later key tile than 0, waves of one block start at
different tiles, the window edge falls inside and on the boundary of a 64-key tile, and W = 1
(every query sees only itself).
"""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding, inputs
from tests.test_gpu_parity import BWD_FLAGS, BWD_IDS, DEV, STORE_DS, bwd_workspace, check, f64, slice_group, zero_ref_scale

pytestmark = pytest.mark.gpu

_NAME = {torch.bfloat16: "bf16", torch.float32: "f32", torch.float16: "f16"}


def run_gpu_window(q, k, v, dO, base, window, out_dtype, flags=0):
    qd, kd, vd, dOd = (t.to(DEV) for t in (q, k, v, dO))
    o, lse = binding.ne_rope_attn_fwd(qd, kd, vd, base, out_dtype=out_dtype, window=window)
    ws = bwd_workspace(qd, kd, base, flags)
    dq, dk, dv = binding.ne_rope_attn_bwd(qd, kd, vd, o, lse, dOd, base, workspace=ws, flags=flags, window=window)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o, lse, dq, dk, dv)]


def ref_window(q, k, v, dO, o_gpu, base, window, out_dtype):
    ro, rlse = oracle.fwd(f64(q), f64(k), f64(v), base, window=window)
    if out_dtype == torch.float32:
        grads = oracle.bwd(f64(q), f64(k), f64(v), f64(dO), base, window=window)
    else:
        grads = oracle.bwd_given_o(f64(q), f64(k), f64(v), f64(o_gpu), f64(dO), base, window=window)
    return (ro, rlse) + tuple(grads)


def window_parity(q, k, v, dO, base, window, out_dtype, in_dtype, flags=0):
    got = run_gpu_window(q, k, v, dO, base, window, out_dtype, flags)
    ref = ref_window(q, k, v, dO, got[0], base, window, out_dtype)
    # with W = 1 the exact dq and dk are zero (P = 1, and dS = dP - Delta cancels up to the rounding
    # of two D-term dot products): the zero-reference scale of test_gpu_parity.py
    gscale = zero_ref_scale(in_dtype, ref[2:])
    for name, g, r in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
        check(name, g, r, in_dtype, out_dtype, zero_scale=gscale)


SHAPES = [  # (B, T, Hq, Hkv, D)
    (1, 300, 6, 2, 128),
    (2, 200, 8, 2, 64),
    (1, 129, 4, 4, 32),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("window", [1, 5, 64, 65, 100])
@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float32])
def test_window_parity_small(shape, window, in_dt):
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=2000 + window, dtype=_NAME[in_dt])
    window_parity(q, k, v, dO, 1.0e4, window, torch.float32, in_dt)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("window", [1, 5, 65])
@pytest.mark.parametrize("flags", BWD_FLAGS[1:], ids=BWD_IDS[1:])
def test_window_parity_small_other_backwards(shape, window, flags):
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=2000 + window, dtype="bf16")
    window_parity(q, k, v, dO, 1.0e4, window, torch.float32, torch.bfloat16, flags=flags)


@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float16])
def test_window_parity_16bit_outputs(in_dt):
    q, k, v, dO = inputs.random_case(2, 150, 6, 2, 128, seed=78, dtype=_NAME[in_dt])
    window_parity(q, k, v, dO, 1.0e4, 37, in_dt, in_dt)


def test_window_of_T_or_more_equals_the_causal_call_bitwise():
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(1, 190, 6, 2, 128, seed=13, dtype="bf16"))
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4)
    ref = (o, lse) + tuple(binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, 1e4))
    for W in (0, -3, 190, 191, 10 ** 6):
        ow, lw = binding.ne_rope_attn_fwd(q, k, v, 1e4, window=W)
        got = (ow, lw) + tuple(binding.ne_rope_attn_bwd(q, k, v, ow, lw, dO, 1e4, window=W))
        for a, b in zip(got, ref):
            assert torch.equal(a, b), W


def test_window_keys_outside_are_bitwise_invisible():
    """Perturbing key/value j changes nothing for the queries that do not see it."""
    W, T, j = 40, 260, 97
    q, k, v, dO = inputs.random_case(1, T, 6, 2, 64, seed=14, dtype="bf16")
    o1, lse1, *_ = run_gpu_window(q, k, v, dO, 1e4, W, torch.float32)
    k2, v2 = k.clone(), v.clone()
    k2[:, j] = inputs.gaussian(k2[:, j].shape, 15, 1.0, "bf16")
    v2[:, j] = inputs.gaussian(v2[:, j].shape, 16, 1.0, "bf16")
    o2, lse2, *_ = run_gpu_window(q, k2, v2, dO, 1e4, W, torch.float32)
    outside = [t for t in range(T) if not (j <= t < j + W)]
    assert torch.equal(o1[:, outside], o2[:, outside])
    assert torch.equal(lse1[:, :, outside], lse2[:, :, outside])
    assert not torch.equal(o1[:, j:j + W], o2[:, j:j + W])


@pytest.mark.parametrize("flags", BWD_FLAGS[:2], ids=BWD_IDS[:2])
def test_window_backward_is_bitwise_deterministic(flags):
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(2, 700, 12, 4, 128, seed=17, dtype="bf16"))
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4, window=175)
    ws = bwd_workspace(q, k, 1e4, flags)
    first = [t.clone() for t in binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, 1e4, window=175, workspace=ws,
                                                         flags=flags)]
    again = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, 1e4, window=175, workspace=ws, flags=flags)
    for a, b in zip(first, again):
        assert torch.equal(a, b)


def workload_window_parity(name, window, groups, out_dtype=torch.float32, flags=0):
    """Full-size GPU run with a window; compare the (batch, KV group) slices the oracle recomputes."""
    w = inputs.WORKLOADS[name]
    q, k, v, dO = inputs.make_inputs(w)
    got = run_gpu_window(q, k, v, dO, w.rope_base, window, out_dtype, flags)
    o, lse, dq, dk, dv = got
    G = w.G
    for b, g in groups:
        qs, dOs = slice_group(q, b, g, G), slice_group(dO, b, g, G)
        ks, vs = slice_group(k, b, g, 0), slice_group(v, b, g, 0)
        ref = ref_window(qs, ks, vs, dOs, slice_group(o, b, g, G), w.rope_base, window, out_dtype)
        parts = (slice_group(o, b, g, G), lse[b:b + 1, g * G:(g + 1) * G], slice_group(dq, b, g, G),
                 slice_group(dk, b, g, 0), slice_group(dv, b, g, 0))
        for nm, gpart, r in zip(("o", "lse", "dq", "dk", "dv"), parts, ref):
            check(nm, gpart, r, q.dtype, out_dtype)


@pytest.mark.parametrize("flags", BWD_FLAGS, ids=BWD_IDS)
def test_window_workload_wide_gqa_quarter_context(flags):
    workload_window_parity("wide_gqa_t2048_d128", 512, [(0, 0), (3, 2)], flags=flags)


def test_window_workload_wide_gqa_quarter_context_bf16_out():
    workload_window_parity("wide_gqa_t2048_d128", 512, [(1, 1)], out_dtype=torch.bfloat16)


def test_window_workload_nanoeuler_gpu_layer():
    workload_window_parity("nanoeuler_gpu_layer", 128, [(0, 0), (5, 3)])
