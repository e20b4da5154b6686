"""GPU parity of the HIP path against the double-precision oracle (needs an MI355X).

Bars (max-abs error relative to each output's scale, err = max|x - ref| / max|ref|):
  * fp16 MFMA operands from bf16/fp16 inputs, fp32 outputs: 2e-3
  * fp32 path (fp32 operands on fp32 MFMA): 1e-5
  * 16-bit outputs: |x - ref| <= 2e-3 * max|ref| + half an ulp of the output format at ref.
Where the exact result is identically zero (dq and dk when T = 1: the only score is the
diagonal one and dS cancels exactly), the scale is 1% of the largest reference gradient of the
same call, since a relative error to zero is undefined.
The oracle gets exactly the values the GPU gets (the rounded inputs widened to float64).
With 16-bit outputs the backward is handed the forward's rounded o, and Delta = rowsum(dO * o)
is computed from it (as the ABI states), so its reference is the oracle backward with Delta from
that same o (oracle.bwd_given_o); with fp32 outputs the reference is the exact gradient.
"""
import contextlib
import math
import os

import numpy as np
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BAR = {torch.float32: 1e-5, torch.bfloat16: 2e-3, torch.float16: 2e-3}


def run_gpu(q, k, v, dO, base, out_dtype):
    qd, kd, vd, dOd = (t.to(DEV) for t in (q, k, v, dO))
    o, lse = binding.ne_rope_attn_fwd(qd, kd, vd, base, out_dtype=out_dtype)
    dq, dk, dv = binding.ne_rope_attn_bwd(qd, kd, vd, o, lse, dOd, base)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o, lse, dq, dk, dv)]


def f64(t):
    return t.double().numpy()


def check(name, got, ref, in_dtype, out_dtype, zero_scale=None):
    got = got.double().numpy()
    scale = float(np.max(np.abs(ref)))
    if scale == 0.0:
        assert zero_scale, f"{name}: reference is identically zero and no fallback scale given"
        scale = zero_scale
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    bar = BAR[in_dtype]
    if out_dtype in (torch.bfloat16, torch.float16) and name != "lse":
        mant = 8 if out_dtype == torch.bfloat16 else 11
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - (mant - 1))
        excess = np.abs(got - ref) - (bar * scale + 0.5 * ulp)
        assert np.max(excess) <= 0, f"{name}: exceeds bar by {np.max(excess):.3e} (scale {scale:.3e})"
        return float(np.max(np.abs(got - ref)) / scale)
    err = float(np.max(np.abs(got - ref)) / scale)
    assert err <= bar, f"{name}: rel err {err:.3e} > {bar:.1e} (scale {scale:.3e})"
    return err


def ref_bwd(q, k, v, dO, o_gpu, base, out_dtype):
    if out_dtype == torch.float32:
        return oracle.bwd(f64(q), f64(k), f64(v), f64(dO), base)
    return oracle.bwd_given_o(f64(q), f64(k), f64(v), f64(o_gpu), f64(dO), base)


def parity(q, k, v, dO, base, out_dtype, in_dtype):
    o, lse, dq, dk, dv = run_gpu(q, k, v, dO, base, out_dtype)
    ro, rlse = oracle.fwd(f64(q), f64(k), f64(v), base)
    rdq, rdk, rdv = ref_bwd(q, k, v, dO, o, base, out_dtype)
    errs = {}
    gscale = 0.01 * max(float(np.max(np.abs(x))) for x in (rdq, rdk, rdv))
    for name, g, r in (("o", o, ro), ("lse", lse, rlse), ("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        errs[name] = check(name, g, r, in_dtype, out_dtype, zero_scale=gscale)
    return errs


SHAPES = [  # (B, T, Hq, Hkv, D): ragged T, every group size, every head_dim
    (1, 1, 2, 1, 64),
    (1, 2, 3, 1, 32),
    (1, 17, 4, 2, 64),
    (2, 100, 6, 2, 64),
    (1, 129, 4, 1, 128),
    (1, 200, 8, 2, 32),
    (2, 257, 3, 3, 128),
    (1, 384, 12, 4, 64),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtypes", [(torch.bfloat16, torch.float32), (torch.float32, torch.float32),
                                    (torch.float16, torch.float32)])
@pytest.mark.parametrize("base", [1.0e4, 0.0])
def test_parity_small(shape, dtypes, base):
    in_dt, out_dt = dtypes
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=1000 + T, dtype={torch.bfloat16: "bf16",
                                     torch.float32: "f32", torch.float16: "f16"}[in_dt])
    parity(q, k, v, dO, base, out_dt, in_dt)


@contextlib.contextmanager
def ds_cap(nbytes):
    """Cap of the 16-bit backward's stored-dS buffer (read at every call): it holds the dS of as many
    (batch, KV head) groups as fit, and the dK/dV and dQ passes run once per such batch; below one
    group the dQ pass recomputes S and dP instead."""
    old = os.environ.get("NE_ROPE_ATTN_DS_MAX_BYTES")
    os.environ["NE_ROPE_ATTN_DS_MAX_BYTES"] = str(int(nbytes))
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("NE_ROPE_ATTN_DS_MAX_BYTES", None)
        else:
            os.environ["NE_ROPE_ATTN_DS_MAX_BYTES"] = old


def recompute_dq():
    """The 16-bit backward as it runs when one group's dS exceeds the cap."""
    return ds_cap(0)


def ds_group_bytes(T, G):
    nrt, nkb = -(-T * G // 64), -(-T // 64)
    return sum(1 for kb in range(nkb) for rt in range(nrt) if rt >= kb * G) * 8192


def test_stored_ds_in_group_batches_is_bitwise_the_single_batch_run():
    """A dS buffer smaller than every group's dS: the passes run per batch of groups (one group at a
    time; 3 + 1), with the same bits as the single batch."""
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = inputs.make_inputs(w, B=1)      # 4 groups
    one = run_gpu(q, k, v, dO, w.rope_base, torch.float32)
    for groups in (1, 3):
        with ds_cap(groups * ds_group_bytes(w.T, w.G)):
            again = run_gpu(q, k, v, dO, w.rope_base, torch.float32)
        for a, b in zip(one, again):
            assert torch.equal(a, b)


@pytest.mark.parametrize("shape", SHAPES[2:])
@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float16])
def test_parity_small_recompute_dq(shape, in_dt):
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=1000 + T, dtype="bf16" if in_dt == torch.bfloat16 else "f16")
    with recompute_dq():
        parity(q, k, v, dO, 1.0e4, torch.float32, in_dt)


def test_stored_ds_and_recompute_dq_agree():
    """Storing dS leaves the dK/dV pass's arithmetic unchanged (o, lse, dk, dv bitwise equal); the two
    dQ passes use the same dS up to where its fp16 rounding happens."""
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = inputs.make_inputs(w, B=1)
    stored = run_gpu(q, k, v, dO, w.rope_base, torch.float32)
    with recompute_dq():
        again = run_gpu(q, k, v, dO, w.rope_base, torch.float32)
    for i in (0, 1, 3, 4):
        assert torch.equal(stored[i], again[i])
    assert float((stored[2] - again[2]).abs().max() / again[2].abs().max()) < 2e-3


@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.bfloat16), (torch.float16, torch.float16)])
def test_parity_16bit_outputs(in_dt, out_dt):
    q, k, v, dO = inputs.random_case(2, 150, 6, 2, 128, seed=77, dtype="bf16" if in_dt == torch.bfloat16 else "f16")
    parity(q, k, v, dO, 1.0e4, out_dt, in_dt)


def slice_group(t, b, g, G):
    return t[b:b + 1, :, g * G:(g + 1) * G].contiguous() if G else t[b:b + 1, :, g:g + 1].contiguous()


def workload_parity(name, groups, dtype=None, out_dtype=torch.float32):
    """Full-size GPU run; compare the (batch, KV group) slices the oracle recomputes."""
    w = inputs.WORKLOADS[name]
    q, k, v, dO = inputs.make_inputs(w, dtype=dtype)
    in_dt = q.dtype
    o, lse, dq, dk, dv = run_gpu(q, k, v, dO, w.rope_base, out_dtype)
    G = w.G
    for b, g in groups:
        qs, dOs = slice_group(q, b, g, G), slice_group(dO, b, g, G)
        ks, vs = slice_group(k, b, g, 0), slice_group(v, b, g, 0)
        ro, rlse = oracle.fwd(f64(qs), f64(ks), f64(vs), w.rope_base)
        rdq, rdk, rdv = ref_bwd(qs, ks, vs, dOs, slice_group(o, b, g, G), w.rope_base, out_dtype)
        check("o", slice_group(o, b, g, G), ro, in_dt, out_dtype)
        check("lse", lse[b:b + 1, g * G:(g + 1) * G], rlse, in_dt, out_dtype)
        check("dq", slice_group(dq, b, g, G), rdq, in_dt, out_dtype)
        check("dk", slice_group(dk, b, g, 0), rdk, in_dt, out_dtype)
        check("dv", slice_group(dv, b, g, 0), rdv, in_dt, out_dtype)


def test_workload_tiny_cpu_model_fp32():
    workload_parity("tiny_cpu_model", [(0, 0), (0, 1)])


def test_workload_nanoeuler_gpu_layer_bf16():
    workload_parity("nanoeuler_gpu_layer", [(0, 0), (7, 3)])


def test_workload_nanoeuler_gpu_layer_fp32_path():
    workload_parity("nanoeuler_gpu_layer", [(3, 1)], dtype="f32")


def test_workload_gpt2_small_mha_bf16():
    workload_parity("gpt2_small_mha", [(0, 0), (15, 11)])


def test_workload_wide_gqa_bf16():
    workload_parity("wide_gqa_t2048_d128", [(0, 0), (3, 3)])


def test_workload_wide_gqa_bf16_out():
    workload_parity("wide_gqa_t2048_d128", [(2, 1)], out_dtype=torch.bfloat16)


def test_workload_long_ctx_bf16():
    workload_parity("long_ctx_t8192", [(0, 5)])


def test_one_kv_group_alone_equals_its_slice_of_the_full_run_bitwise():
    """The long-context layer sharded by KV head (one group per GPU, no exchange): a group run on
    its own, as one GPU of 8 would, gives exactly the bits of that group in the full run."""
    w = inputs.WORKLOADS["long_ctx_t8192"]
    q, k, v, dO = inputs.make_inputs(w)
    full = run_gpu(q, k, v, dO, w.rope_base, torch.float32)
    G = w.G
    for g in (0, 5):
        qs, dOs = slice_group(q, 0, g, G), slice_group(dO, 0, g, G)
        ks, vs = slice_group(k, 0, g, 0), slice_group(v, 0, g, 0)
        o, lse, dq, dk, dv = run_gpu(qs, ks, vs, dOs, w.rope_base, torch.float32)
        assert torch.equal(o.cpu(), slice_group(full[0], 0, g, G).cpu())
        assert torch.equal(lse.cpu(), full[1][:, g * G:(g + 1) * G].cpu())
        assert torch.equal(dq.cpu(), slice_group(full[2], 0, g, G).cpu())
        assert torch.equal(dk.cpu(), slice_group(full[3], 0, g, 0).cpu())
        assert torch.equal(dv.cpu(), slice_group(full[4], 0, g, 0).cpu())


# ---------------------------------------------------------------------------------------
# Properties checked on the GPU outputs themselves.
# ---------------------------------------------------------------------------------------
def test_causality_future_perturbation_is_bitwise_invisible():
    q, k, v, dO = inputs.random_case(1, 300, 6, 2, 128, seed=5, dtype="bf16")
    o1, lse1, *_ = run_gpu(q, k, v, dO, 1e4, torch.float32)
    cut = 137
    k2, v2 = k.clone(), v.clone()
    k2[:, cut + 1:] = inputs.gaussian(k2[:, cut + 1:].shape, 6, 1.0, "bf16")
    v2[:, cut + 1:] = inputs.gaussian(v2[:, cut + 1:].shape, 7, 1.0, "bf16")
    o2, lse2, *_ = run_gpu(q, k2, v2, dO, 1e4, torch.float32)
    assert torch.equal(o1[:, : cut + 1], o2[:, : cut + 1])
    assert torch.equal(lse1[:, :, : cut + 1], lse2[:, :, : cut + 1])


def test_backward_is_bitwise_deterministic():
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = (t.to(DEV) for t in inputs.make_inputs(w, B=1))
    o, lse = binding.ne_rope_attn_fwd(q, k, v, w.rope_base)
    first = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base)
    first = [t.clone() for t in first]
    for _ in range(2):
        again = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_backward_is_the_same_wherever_the_workspace_lies():
    """The stored-dS tile addresses are moved into scalar registers as two 32-bit halves; a workspace
    whose address has the low half at or above 2^31 (where a sign-extended half would corrupt the
    address) gives the same bits as one with the low half below 2^31."""
    B, T, Hq, Hkv, D = 1, 300, 6, 2, 128
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(B, T, Hq, Hkv, D, seed=31, dtype="bf16"))
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4)
    n = binding.bwd_workspace_bytes(B, T, Hq, Hkv, D, q.dtype)
    buf = torch.empty((1 << 32) + n + 512, dtype=torch.uint8, device=DEV)
    base = buf.data_ptr()
    outs = []
    for start in (0, 1 << 31):   # the low 32 address bits of the workspace
        off = ((start - (base & 0xFFFFFFFF)) % (1 << 32) + 255) // 256 * 256
        low = (base + off) & 0xFFFFFFFF
        assert (low >= 1 << 31) == (start > 0) and (low + n < 1 << 32)
        outs.append([t.clone() for t in binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, 1e4, workspace=buf[off:off + n])])
    del buf
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_gqa_matches_replicated_kv_mha():
    q, k, v, dO = inputs.random_case(1, 130, 8, 2, 64, seed=9, dtype="bf16")
    G = 4
    o, lse, dq, dk, dv = run_gpu(q, k, v, dO, 1e4, torch.float32)
    kr, vr = k.repeat_interleave(G, dim=2), v.repeat_interleave(G, dim=2)
    om, lsem, dqm, dkm, dvm = run_gpu(q, kr, vr, dO, 1e4, torch.float32)
    for a, b in ((o, om), (lse, lsem), (dq, dqm)):
        assert float((a - b).abs().max() / b.abs().max()) < 1e-3
    dks = dkm.reshape(1, 130, 2, G, 64).sum(3)
    dvs = dvm.reshape(1, 130, 2, G, 64).sum(3)
    assert float((dk - dks).abs().max() / dks.abs().max()) < 1e-3
    assert float((dv - dvs).abs().max() / dvs.abs().max()) < 1e-3


def test_single_token_and_zero_query_closed_forms():
    q, k, v, dO = inputs.random_case(3, 1, 4, 2, 64, seed=11, dtype="f32")
    o, lse, dq, dk, dv = run_gpu(q, k, v, dO, 1e4, torch.float32)
    assert torch.allclose(o, v.repeat_interleave(2, dim=2), rtol=0, atol=1e-6)
    ref = (q * k.repeat_interleave(2, dim=2)).sum(-1) / math.sqrt(64)
    assert torch.allclose(lse, ref.permute(0, 2, 1), rtol=0, atol=1e-5)
    # dq = dk = 0 exactly (dS cancels); the GPU sums dP and Delta in different orders
    assert float(dq.abs().max()) <= 1e-5 * float(dv.abs().max())
    assert float(dk.abs().max()) <= 1e-5 * float(dv.abs().max())
    # q = 0: uniform weights over the visible keys
    _, k, v, dO = inputs.random_case(1, 200, 3, 1, 128, seed=12, dtype="bf16")
    q = torch.zeros(1, 200, 3, 128, dtype=torch.bfloat16)
    o, lse, *_ = run_gpu(q, k, v, dO, 1e4, torch.float32)
    n = torch.arange(1, 201, dtype=torch.float64)
    assert torch.allclose(lse[0, 0].double(), n.log(), rtol=0, atol=1e-5)
    mean = v[0, :, 0].double().cumsum(0) / n[:, None]
    assert float((o[0, :, 1].double() - mean).abs().max()) < 2e-3 * float(mean.abs().max())
