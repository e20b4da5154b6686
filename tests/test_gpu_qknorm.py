"""GPU parity of the QK-norm option (ne_rope_attn_fwd_ex / ne_rope_attn_bwd_ex, and the cache calls)
against the oracle with qk_norm.  Every (token, head) row of q and k becomes
gain * x / sqrt(mean(x^2) + eps) before RoPE (nanochat guide, 模型架构速览: normalised and scaled
up by 1.2).  Bars as in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding, inputs
from tests.test_gpu_parity import BWD_FLAGS, BWD_IDS, DEV, STORE_DS, bwd_workspace, check, f64, slice_group, zero_ref_scale

pytestmark = pytest.mark.gpu

QKN = (1.2, 1e-6)
_NAME = {torch.bfloat16: "bf16", torch.float32: "f32", torch.float16: "f16"}


def run_ex(q, k, v, dO, base, window, qkn, out_dtype, flags=0, ds_groups=None):
    qd, kd, vd, dOd = (t.to(DEV) for t in (q, k, v, dO))
    o, lse = binding.ne_rope_attn_fwd_ex(qd, kd, vd, base, window, qkn, out_dtype=out_dtype)
    ws = bwd_workspace(qd, kd, base, flags, ds_groups)
    dq, dk, dv = binding.ne_rope_attn_bwd_ex(qd, kd, vd, o, lse, dOd, base, window, qkn, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o, lse, dq, dk, dv)]


def ref_ex(q, k, v, dO, o_gpu, base, window, qkn, out_dtype):
    ro, rlse = oracle.fwd(f64(q), f64(k), f64(v), base, window=window, qk_norm=qkn)
    if out_dtype == torch.float32:
        g = oracle.bwd(f64(q), f64(k), f64(v), f64(dO), base, window=window, qk_norm=qkn)
    else:
        g = oracle.bwd_given_o(f64(q), f64(k), f64(v), f64(o_gpu), f64(dO), base, window=window, qk_norm=qkn)
    return (ro, rlse) + tuple(g)


def ex_parity(q, k, v, dO, base, window, qkn, out_dtype, in_dtype, flags=0):
    got = run_ex(q, k, v, dO, base, window, qkn, out_dtype, flags)
    ref = ref_ex(q, k, v, dO, got[0], base, window, qkn, out_dtype)
    # T = 1: the exact dq and dk are zero: the zero-reference scale of test_gpu_parity.py
    gscale = zero_ref_scale(in_dtype, ref[2:])
    for name, g, r in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
        check(name, g, r, in_dtype, out_dtype, zero_scale=gscale)


@pytest.mark.parametrize("shape", [(1, 1, 2, 1, 64), (2, 100, 6, 2, 64), (1, 129, 4, 1, 128), (2, 257, 3, 3, 128),
                                   (1, 200, 8, 2, 32)])
@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("window", [0, 37])
def test_qk_norm_parity_small(shape, in_dt, window):
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=3000 + T, dtype=_NAME[in_dt])
    ex_parity(q, k, v, dO, 1.0e4, window, QKN, torch.float32, in_dt)


@pytest.mark.parametrize("shape", [(1, 1, 2, 1, 64), (2, 100, 6, 2, 64), (2, 257, 3, 3, 128), (1, 200, 8, 2, 32)])
@pytest.mark.parametrize("window", [0, 37])
@pytest.mark.parametrize("flags", BWD_FLAGS[1:], ids=BWD_IDS[1:])
def test_qk_norm_parity_small_other_backwards(shape, window, flags):
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=3000 + T, dtype="bf16")
    ex_parity(q, k, v, dO, 1.0e4, window, QKN, torch.float32, torch.bfloat16, flags=flags)


@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float16])
def test_qk_norm_parity_16bit_outputs(in_dt):
    q, k, v, dO = inputs.random_case(2, 150, 6, 2, 128, seed=79, dtype=_NAME[in_dt])
    ex_parity(q, k, v, dO, 1.0e4, 0, QKN, in_dt, in_dt)


def test_qk_norm_other_gain_and_eps_no_rope():
    q, k, v, dO = inputs.random_case(1, 90, 4, 2, 64, seed=81, dtype="bf16")
    ex_parity(q * 0.01, k * 30.0, v, dO, 0.0, 0, (0.7, 0.25), torch.float32, torch.bfloat16)


def test_qk_norm_workload_wide_gqa_slices():
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = inputs.make_inputs(w)
    got = run_ex(q, k, v, dO, w.rope_base, 0, QKN, torch.float32)
    o, lse, dq, dk, dv = got
    G = w.G
    for b, g in [(0, 0), (3, 2)]:
        qs, dOs = slice_group(q, b, g, G), slice_group(dO, b, g, G)
        ks, vs = slice_group(k, b, g, 0), slice_group(v, b, g, 0)
        ref = ref_ex(qs, ks, vs, dOs, None, w.rope_base, 0, QKN, torch.float32)
        parts = (slice_group(o, b, g, G), lse[b:b + 1, g * G:(g + 1) * G], slice_group(dq, b, g, G),
                 slice_group(dk, b, g, 0), slice_group(dv, b, g, 0))
        for nm, gp, r in zip(("o", "lse", "dq", "dk", "dv"), parts, ref):
            check(nm, gp, r, torch.bfloat16, torch.float32)


def test_qk_norm_rescaled_inputs_give_the_same_outputs():
    """eps = 0: per-row positive rescaling of q and k is invisible (up to the operand rounding)."""
    q, k, v, dO = inputs.random_case(1, 160, 8, 2, 128, seed=83, dtype="f32")
    a = run_ex(q, k, v, dO, 1e4, 0, (1.2, 0.0), torch.float32)
    c = torch.rand(1, 160, 8, 1, generator=torch.Generator().manual_seed(1)) * 4 + 0.25
    ck = torch.rand(1, 160, 2, 1, generator=torch.Generator().manual_seed(2)) * 4 + 0.25
    b = run_ex(q * c, k * ck, v, dO, 1e4, 0, (1.2, 0.0), torch.float32)
    for x, y in zip(a[:2], b[:2]):
        assert float((x - y).abs().max()) <= 1e-5 * float(x.abs().max())
    assert float((a[2] - b[2] * c).abs().max()) <= 1e-5 * float(a[2].abs().max())
    assert float((a[3] - b[3] * ck).abs().max()) <= 1e-5 * float(a[3].abs().max())


def test_qk_norm_off_in_opts_equals_the_plain_call_bitwise():
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(1, 130, 6, 2, 64, seed=85, dtype="bf16"))
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4)
    ref = (o, lse) + tuple(binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, 1e4))
    o2, l2 = binding.ne_rope_attn_fwd_ex(q, k, v, 1e4, 0, None)
    got = (o2, l2) + tuple(binding.ne_rope_attn_bwd_ex(q, k, v, o2, l2, dO, 1e4, 0, None))
    for x, y in zip(got, ref):
        assert torch.equal(x, y)


def test_qk_norm_decode_parity():
    B, P, Tq, Hq, Hkv, D, Tcap = 2, 300, 3, 8, 2, 128, 320
    lens = [120, 297]
    q = inputs.gaussian((B, P, Hq, D), 870, 1.0, "bf16")
    k = inputs.gaussian((B, P, Hkv, D), 871, 3.0, "bf16")
    v = inputs.gaussian((B, P, Hkv, D), 872, 1.0, "bf16")
    cache = binding.new_kv_cache(B, Tcap, Hkv, D, torch.bfloat16, DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    for p0 in range(0, P, 100):
        L = torch.full((B,), p0, dtype=torch.int32, device=DEV)
        binding.ne_kv_cache_append(cache, L, kd[:, p0:p0 + 100].contiguous(), vd[:, p0:p0 + 100].contiguous(), Tcap,
                                   1e4, qk_norm=QKN)
    q_new = torch.stack([q[b, lens[b]:lens[b] + Tq] for b in range(B)])
    for window in (0, 50):
        o, lse = binding.ne_rope_attn_decode(q_new.to(DEV), cache, lens, Tcap, Hkv, 1e4, window, qk_norm=QKN)
        torch.cuda.synchronize()
        ro, rlse = oracle.decode_fwd(f64(q_new), [f64(k[b]) for b in range(B)], [f64(v[b]) for b in range(B)], lens,
                                     1e4, window, qk_norm=QKN)
        check("o", o.cpu(), ro, torch.bfloat16, torch.float32)
        check("lse", lse.cpu(), rlse, torch.bfloat16, torch.float32)


def test_window_and_qk_norm_in_group_batches_are_bitwise_the_single_batch_run():
    """The stored dS processed one (batch, KV head) group at a time, with a window and the QK norm,
    gives the bits of the single batch."""
    B, T, Hq, Hkv, D = 2, 300, 6, 2, 128
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=41, dtype="bf16")
    one = run_ex(q, k, v, dO, 1.0e4, 100, QKN, torch.float32, flags=STORE_DS)
    again = run_ex(q, k, v, dO, 1.0e4, 100, QKN, torch.float32, flags=STORE_DS, ds_groups=1)
    for a, b in zip(one, again):
        assert torch.equal(a, b)
