"""GPU parity of the HIP path against the double-precision oracle (needs an MI355X).

Bars (max-abs error relative to each output's scale, err = max|x - ref| / max|ref|):
  * fp16 MFMA operands from bf16/fp16 inputs, fp32 outputs: 2e-3
  * fp32 path (fp32 operands on fp32 MFMA): 1e-5
  * 16-bit outputs: |x - ref| <= 2e-3 * max|ref| + half an ulp of the output format at ref.
Where the exact result is identically zero (dq and dk when T = 1: the only score is the
diagonal one and dS cancels exactly; with a window of 1 the same holds at every row), a relative
error to zero is undefined; those outputs are held to about 1e-5 of the largest reference gradient
of the same call: the scale is 1% of that gradient at the 2e-3 bar of 16-bit inputs and the whole
gradient at the 1e-5 bar of the fp32 path (whose dS = P (dP - Delta) cancels two D-term fp32 dot
products summed in different orders, a few 1e-7 of the gradient's scale).
The backward runs in its three designs (the flags of ne_rope_attn_bwd): the default, whose dQ pass
recomputes S and dP (O(T) workspace); NE_FLAG_STORE_DS (dQ from the dS the dK/dV pass stores);
NE_FLAG_NONDETERMINISTIC (dQ added with atomics in the dK/dV pass; bits may vary, the bar is the
same).
The oracle gets exactly the values the GPU gets (the rounded inputs widened to float64).
With 16-bit outputs the backward is handed the forward's rounded o, and Delta = rowsum(dO * o)
is computed from it (as the ABI states), so its reference is the oracle backward with Delta from
that same o (oracle.bwd_given_o); with fp32 outputs the reference is the exact gradient.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BAR = {torch.float32: 1e-5, torch.bfloat16: 2e-3, torch.float16: 2e-3}


STORE_DS, ATOMIC = binding.NE_FLAG_STORE_DS, binding.NE_FLAG_NONDETERMINISTIC
BWD_FLAGS = [0, STORE_DS, ATOMIC]
BWD_IDS = ["recompute", "stored_ds", "atomic"]


def bwd_workspace(q, k, base, flags, ds_groups=None):
    """A backward workspace for `flags` with its table built; with ds_groups, one whose stored-dS buffer
    holds that many (batch, KV head) groups only."""
    B, T, Hq, Hkv, D = q.shape[0], q.shape[1], q.shape[2], k.shape[2], q.shape[3]
    n = binding.workspace_bytes(True, B, T, Hq, Hkv, D, base, q.dtype, flags)
    if ds_groups is not None:
        n = n - ds_group_bytes(T, Hq // Hkv) * B * Hkv + ds_group_bytes(T, Hq // Hkv) * ds_groups
        n = (n + 255) // 256 * 256
    return binding.ne_rope_table_init(binding.alloc_workspace(n, q.device), T, D, base)


def run_gpu(q, k, v, dO, base, out_dtype, flags=0, ds_groups=None, window=0, qk_norm=None):
    qd, kd, vd, dOd = (t.to(DEV) for t in (q, k, v, dO))
    o, lse = binding.ne_rope_attn_fwd(qd, kd, vd, base, out_dtype=out_dtype, window=window, qk_norm=qk_norm)
    ws = bwd_workspace(qd, kd, base, flags, ds_groups)
    dq, dk, dv = binding.ne_rope_attn_bwd(qd, kd, vd, o, lse, dOd, base, workspace=ws, flags=flags, window=window,
                                          qk_norm=qk_norm)
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


def zero_ref_scale(in_dtype, grads):
    """Error scale of an identically-zero reference output: about 1e-5 of the call's largest gradient."""
    return (1.0 if in_dtype == torch.float32 else 0.01) * max(float(np.max(np.abs(x))) for x in grads)


def ref_bwd(q, k, v, dO, o_gpu, base, out_dtype):
    if out_dtype == torch.float32:
        return oracle.bwd(f64(q), f64(k), f64(v), f64(dO), base)
    return oracle.bwd_given_o(f64(q), f64(k), f64(v), f64(o_gpu), f64(dO), base)


def parity(q, k, v, dO, base, out_dtype, in_dtype, flags=0):
    o, lse, dq, dk, dv = run_gpu(q, k, v, dO, base, out_dtype, flags=flags)
    ro, rlse = oracle.fwd(f64(q), f64(k), f64(v), base)
    rdq, rdk, rdv = ref_bwd(q, k, v, dO, o, base, out_dtype)
    errs = {}
    gscale = zero_ref_scale(in_dtype, (rdq, rdk, rdv))
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


# One or two (batch, KV head) groups: the launch is short of blocks, so the forward cuts its
# longest 256-row blocks into 4 key ranges, the dQ pass its longest 128-row blocks into 2 and the
# dK/dV pass its longest key blocks' rows into 4 (the third shape: forward only; its dK/dV runs
# single key blocks), each block finished by the last of its workgroups (the plans are checked on
# the CPU in test_abi_host.test_split_plans_of_the_parity_shapes).
SPLIT_SHAPES = [(1, 1000, 4, 1, 128), (1, 1200, 4, 2, 64), (1, 777, 2, 1, 32)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
@pytest.mark.parametrize("dtypes", [(torch.bfloat16, torch.float32), (torch.float16, torch.float32),
                                    (torch.bfloat16, torch.bfloat16)])
def test_parity_split_row_blocks(shape, dtypes):
    in_dt, out_dt = dtypes
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=3000 + T,
                                     dtype="bf16" if in_dt == torch.bfloat16 else "f16")
    parity(q, k, v, dO, 1.0e4, out_dt, in_dt)
    # the combined blocks do not depend on which workgroup finishes last: bitwise repeatable
    first = run_gpu(q, k, v, dO, 1.0e4, out_dt)
    again = run_gpu(q, k, v, dO, 1.0e4, out_dt)
    for a, b in zip(first, again):
        assert torch.equal(a, b)


# Group extremes: 16 to 64 query heads per KV head (one or two KV heads), where a 64-row tile of the
# flattened rows t * G + h holds four positions or fewer (one at G = 64) and every key block's first
# row tile carries its diagonal for all heads; and many (batch, KV head) groups of a few positions,
# where most tiles are partial and the launch holds more blocks than the chip has slots.
GROUP_EXTREMES = [(1, 150, 16, 1, 128), (2, 70, 32, 1, 64), (1, 45, 64, 1, 32), (1, 97, 32, 2, 128),
                  (16, 3, 8, 8, 128), (4, 33, 64, 16, 64)]
GROUP_VARIANTS = [(torch.bfloat16, torch.float32, f) for f in BWD_FLAGS] + [
    (torch.float16, torch.float16, 0), (torch.float32, torch.float32, 0)]


@pytest.mark.parametrize("shape", GROUP_EXTREMES, ids=lambda s: "B%dT%dHq%dHkv%dD%d" % s)
@pytest.mark.parametrize("variant", GROUP_VARIANTS,
                         ids=["bf16-f32-" + i for i in BWD_IDS] + ["f16-f16-recompute", "f32-f32"])
def test_parity_group_extremes(shape, variant):
    in_dt, out_dt, flags = variant
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=4000 + T + Hq,
                                     dtype={torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[in_dt])
    parity(q, k, v, dO, 1.0e4, out_dt, in_dt, flags=flags)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [0, 70])
@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float16])
def test_rising_scores_take_the_overflow_path(D, window, in_dt):
    """Scores that rise by about 30 per 64-key tile along each row (keys growing along one direction,
    RoPE off): every tile after a row's first holds probabilities beyond the fp16 range relative to
    the reference maximum kept so far, so the forward raises the maximum and redoes the tile's
    probabilities at each step.  o, lse, dk and dv against the oracle at the usual bars.  dq is not
    compared: with logits near 140 the fp16 operands shift each score by a few hundredths, the rows
    are nearly one-hot, and dq = sum dS k (|k| up to 400) cancels to a few percent of its scale --
    a limit of 16-bit operands on such inputs that the fp32 path does not have."""
    B, T, Hq, Hkv = 1, 300, 4, 2
    g = torch.Generator().manual_seed(88 + D + window)
    q = 0.05 * torch.randn(B, T, Hq, D, generator=g, dtype=torch.float64)
    k = 0.05 * torch.randn(B, T, Hkv, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, T, Hkv, D, generator=g, dtype=torch.float64)
    dO = torch.randn(B, T, Hq, D, generator=g, dtype=torch.float64)
    q[..., 0] += 4.0
    k[..., 0] += 0.47 * D ** 0.5 / 4.0 * torch.arange(T, dtype=torch.float64)[None, :, None]
    q, k, v, dO = (t.to(in_dt) for t in (q, k, v, dO))
    o, lse, dq, dk, dv = run_gpu(q, k, v, dO, 0.0, torch.float32, window=window)
    ro, rlse = oracle.fwd(f64(q), f64(k), f64(v), 0.0, window=window)
    rdq, rdk, rdv = oracle.bwd(f64(q), f64(k), f64(v), f64(dO), 0.0, window=window)
    assert float(np.max(rlse[:, :, -1])) > 100.0      # the last rows' scores reach far past the first tiles'
    gscale = zero_ref_scale(in_dt, (rdq, rdk, rdv))
    for name, gv, rv in (("o", o, ro), ("lse", lse, rlse), ("dk", dk, rdk), ("dv", dv, rdv)):
        check(name, gv, rv, in_dt, torch.float32, zero_scale=gscale)
    assert torch.isfinite(dq).all()


def ds_group_bytes(T, G):
    nrt, nkb = -(-T * G // 64), -(-T // 64)
    return sum(1 for kb in range(nkb) for rt in range(nrt) if rt >= kb * G) * 8192


def test_stored_ds_in_group_batches_is_bitwise_the_single_batch_run():
    """A workspace whose dS buffer holds fewer groups than the call has: the passes run per batch of
    groups (one group at a time; 3 + 1), with the same bits as the single batch."""
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = inputs.make_inputs(w, B=1)      # 4 groups
    one = run_gpu(q, k, v, dO, w.rope_base, torch.float32, flags=STORE_DS)
    for groups in (1, 3):
        again = run_gpu(q, k, v, dO, w.rope_base, torch.float32, flags=STORE_DS, ds_groups=groups)
        for a, b in zip(one, again):
            assert torch.equal(a, b)


@pytest.mark.parametrize("shape", SHAPES[2:])
@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("flags", BWD_FLAGS[1:], ids=BWD_IDS[1:])
def test_parity_small_other_backwards(shape, in_dt, flags):
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=1000 + T, dtype="bf16" if in_dt == torch.bfloat16 else "f16")
    parity(q, k, v, dO, 1.0e4, torch.float32, in_dt, flags=flags)


def test_the_three_backwards_agree():
    """The dK/dV pass's arithmetic is the same in all three designs (o, lse, dk, dv bitwise equal); the
    dQ passes use the same dS up to where its fp16 rounding and the order of the sums happen.  At the
    full batch of 4: with fewer groups the default backward's dK/dV pass splits its longest key
    blocks (the same sums in another order) while the other two keep the mirrored pairs."""
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = inputs.make_inputs(w)
    ref = run_gpu(q, k, v, dO, w.rope_base, torch.float32)
    for flags in BWD_FLAGS[1:]:
        again = run_gpu(q, k, v, dO, w.rope_base, torch.float32, flags=flags)
        for i in (0, 1, 3, 4):
            assert torch.equal(ref[i], again[i]), (flags, i)
        assert float((ref[2] - again[2]).abs().max() / ref[2].abs().max()) < 2e-3


@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.bfloat16), (torch.float16, torch.float16)])
def test_parity_16bit_outputs(in_dt, out_dt):
    q, k, v, dO = inputs.random_case(2, 150, 6, 2, 128, seed=77, dtype="bf16" if in_dt == torch.bfloat16 else "f16")
    parity(q, k, v, dO, 1.0e4, out_dt, in_dt)


def slice_group(t, b, g, G):
    return t[b:b + 1, :, g * G:(g + 1) * G].contiguous() if G else t[b:b + 1, :, g:g + 1].contiguous()


def workload_parity(name, groups, dtype=None, out_dtype=torch.float32, flags=0):
    """Full-size GPU run; compare the (batch, KV group) slices the oracle recomputes."""
    w = inputs.WORKLOADS[name]
    q, k, v, dO = inputs.make_inputs(w, dtype=dtype)
    in_dt = q.dtype
    o, lse, dq, dk, dv = run_gpu(q, k, v, dO, w.rope_base, out_dtype, flags=flags)
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


@pytest.mark.parametrize("flags", BWD_FLAGS, ids=BWD_IDS)
def test_workload_wide_gqa_bf16(flags):
    workload_parity("wide_gqa_t2048_d128", [(0, 0), (3, 3)], flags=flags)


def test_workload_wide_gqa_bf16_out():
    workload_parity("wide_gqa_t2048_d128", [(2, 1)], out_dtype=torch.bfloat16)


@pytest.mark.parametrize("flags", BWD_FLAGS, ids=BWD_IDS)
def test_workload_long_ctx_bf16(flags):
    workload_parity("long_ctx_t8192", [(0, 5)], flags=flags)


def test_one_kv_group_alone_equals_its_slice_of_the_full_run():
    """The long-context layer sharded by KV head (one group per GPU, no exchange): a group run on
    its own, as one GPU of 8 would, gives the values of that group in the full run.  Not bitwise:
    with one group the launch is short of row blocks, so the longest ones are split over several
    workgroups and their partial results added (in a fixed order), while the 8-group run keeps
    them whole; only the order of fp32 sums differs."""
    w = inputs.WORKLOADS["long_ctx_t8192"]
    q, k, v, dO = inputs.make_inputs(w)
    full = run_gpu(q, k, v, dO, w.rope_base, torch.float32)
    G = w.G
    for g in (0, 5):
        qs, dOs = slice_group(q, 0, g, G), slice_group(dO, 0, g, G)
        ks, vs = slice_group(k, 0, g, 0), slice_group(v, 0, g, 0)
        got = run_gpu(qs, ks, vs, dOs, w.rope_base, torch.float32)
        want = [slice_group(full[0], 0, g, G), full[1][:, g * G:(g + 1) * G], slice_group(full[2], 0, g, G),
                slice_group(full[3], 0, g, 0), slice_group(full[4], 0, g, 0)]
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, want):
            # fp32 reassociation of sums of up to 8192 terms, plus the fp16 rounding of P and dS it
            # can flip: far below the 16-bit operand error the parity tests allow
            err = (a.double() - b.double()).abs().max().item()
            assert err <= 2e-4 * b.double().abs().max().item() + 1e-6, (g, name, err)


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


@pytest.mark.parametrize("flags", BWD_FLAGS[:2], ids=BWD_IDS[:2])
def test_backward_is_bitwise_deterministic(flags):
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = (t.to(DEV) for t in inputs.make_inputs(w, B=1))
    o, lse = binding.ne_rope_attn_fwd(q, k, v, w.rope_base)
    ws = bwd_workspace(q, k, w.rope_base, flags)
    first = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base, workspace=ws, flags=flags)
    first = [t.clone() for t in first]
    for _ in range(2):
        again = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base, workspace=ws, flags=flags)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_atomic_backward_repeats_within_the_bar():
    """NE_FLAG_NONDETERMINISTIC: dk and dv are still written once (bitwise repeatable); dq is a sum of
    atomic adds whose order varies, so repeated calls agree to rounding."""
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = (t.to(DEV) for t in inputs.make_inputs(w, B=1))
    o, lse = binding.ne_rope_attn_fwd(q, k, v, w.rope_base)
    ws = bwd_workspace(q, k, w.rope_base, ATOMIC)
    first = [t.clone() for t in binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base, workspace=ws, flags=ATOMIC)]
    for _ in range(2):
        dq, dk, dv = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base, workspace=ws, flags=ATOMIC)
        assert torch.equal(first[1], dk) and torch.equal(first[2], dv)
        assert float((first[0] - dq).abs().max() / first[0].abs().max()) < 1e-5


def test_backward_is_the_same_wherever_the_workspace_lies():
    """The stored-dS tile addresses are moved into scalar registers as two 32-bit halves; a workspace
    whose address has the low half at or above 2^31 (where a sign-extended half would corrupt the
    address) gives the same bits as one with the low half below 2^31."""
    B, T, Hq, Hkv, D = 1, 300, 6, 2, 128
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(B, T, Hq, Hkv, D, seed=31, dtype="bf16"))
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4)
    n = binding.workspace_bytes(True, B, T, Hq, Hkv, D, 1e4, q.dtype, STORE_DS)
    buf = torch.empty((1 << 32) + n + 512, dtype=torch.uint8, device=DEV)
    base = buf.data_ptr()
    outs = []
    for start in (0, 1 << 31):   # the low 32 address bits of the workspace
        off = ((start - (base & 0xFFFFFFFF)) % (1 << 32) + 255) // 256 * 256
        low = (base + off) & 0xFFFFFFFF
        assert (low >= 1 << 31) == (start > 0) and (low + n < 1 << 32)
        ws = binding.ne_rope_table_init(buf[off:off + n], T, D, 1e4)
        outs.append([t.clone() for t in binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, 1e4, workspace=ws,
                                                                 flags=STORE_DS)])
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


# ---------------------------------------------------------------------------------------
# The backward on its own: fed the oracle's o and lse (fp32), so its error is not mixed with the
# forward's.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,bar_dt,qk_scale", [("bf16", torch.bfloat16, 1.0), ("f32", torch.float32, 2.0)])
@pytest.mark.parametrize("flags", BWD_FLAGS, ids=BWD_IDS)
def test_backward_fed_the_oracle_forward(dtype, bar_dt, qk_scale, flags):
    """The C4 shape (B4 T2048 Hq12 Hkv4 D128, one KV group).  fp32 path: the workload's own inputs (q, k
    drawn at twice the unit scale).  16-bit path: q, k at the unit scale of the other workloads -- with
    the doubled scale the fp16 rounding of the rotated scores is no longer compensated by the forward's
    own lse (the pipeline tests above hold that case to the bar), and the composition reads 2.1e-3."""
    w = inputs.WORKLOADS["wide_gqa_t2048_d128"]
    q, k, v, dO = inputs.make_inputs(w, B=1, dtype=dtype)
    if qk_scale != w.qk_scale:
        q = (q.float() * (qk_scale / w.qk_scale)).to(q.dtype)
        k = (k.float() * (qk_scale / w.qk_scale)).to(k.dtype)
    G = w.G
    qs, dOs = slice_group(q, 0, 1, G), slice_group(dO, 0, 1, G)
    ks, vs = slice_group(k, 0, 1, 0), slice_group(v, 0, 1, 0)
    ro, rlse = oracle.fwd(f64(qs), f64(ks), f64(vs), w.rope_base)
    rdq, rdk, rdv = oracle.bwd(f64(qs), f64(ks), f64(vs), f64(dOs), w.rope_base)
    qd, kd, vd, dOd = (t.to(DEV) for t in (qs, ks, vs, dOs))
    o = torch.from_numpy(ro).float().to(DEV)
    lse = torch.from_numpy(rlse).float().to(DEV)
    ws = bwd_workspace(qd, kd, w.rope_base, flags)
    dq, dk, dv = binding.ne_rope_attn_bwd(qd, kd, vd, o, lse, dOd, w.rope_base, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        check(name, g.cpu(), r, bar_dt, torch.float32)


# ---------------------------------------------------------------------------------------
# Input ranges: dO is scaled per group by a power of two before its fp16 conversion, so gradients
# of tiny (or large) dO keep their relative precision; k and v of large magnitude stay in range.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("scale", [1e-6, 1e-9, 3e3])
@pytest.mark.parametrize("flags", BWD_FLAGS, ids=BWD_IDS)
def test_parity_with_do_far_from_unit_scale(scale, flags):
    q, k, v, dO = inputs.random_case(2, 150, 6, 2, 128, seed=55, dtype="bf16")
    dO = (dO.float() * scale).to(torch.bfloat16)
    parity(q, k, v, dO, 1.0e4, torch.float32, torch.bfloat16, flags=flags)


def test_parity_with_large_keys_and_values():
    q, k, v, dO = inputs.random_case(1, 200, 4, 2, 64, seed=56, dtype="bf16")
    k = (k.float() * 64.0).to(torch.bfloat16)
    v = (v.float() * 300.0).to(torch.bfloat16)
    q = (q.float() / 64.0).to(torch.bfloat16)
    parity(q, k, v, dO, 1.0e4, torch.float32, torch.bfloat16)


def test_parity_with_all_zero_do():
    q, k, v, dO = inputs.random_case(1, 100, 4, 2, 64, seed=57, dtype="bf16")
    dO = torch.zeros_like(dO)
    o, lse, dq, dk, dv = run_gpu(q, k, v, dO, 1.0e4, torch.float32)
    for g in (dq, dk, dv):
        assert torch.count_nonzero(g) == 0


# ---------------------------------------------------------------------------------------
# The RoPE table: built once per workspace by ne_rope_table_init and checked on the device.
# ---------------------------------------------------------------------------------------
def test_table_check_reports_a_missing_or_mismatched_table():
    B, T, Hq, Hkv, D = 1, 100, 4, 2, 64
    n = binding.workspace_bytes(True, B, T, Hq, Hkv, D, 1e4, torch.bfloat16)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    assert binding.ne_rope_table_check(ws, T, D, 1e4) == 6          # NE_ERR_NO_ROPE_TABLE
    binding.ne_rope_table_init(ws, T, D, 1e4)
    assert binding.ne_rope_table_check(ws, T, D, 1e4) == 0
    assert binding.ne_rope_table_check(ws, T - 1, D, 1e4) == 6
    assert binding.ne_rope_table_check(ws, T, D, 5e5) == 6
    assert binding.ne_rope_table_check(ws, T, 32, 1e4) == 6
    assert binding.ne_rope_table_check(ws, T, D, 0.0) == 0          # no RoPE: no table needed


def test_calls_without_the_table_give_nan_outputs():
    B, T, Hq, Hkv, D = 1, 100, 4, 2, 64
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(B, T, Hq, Hkv, D, seed=58, dtype="bf16"))
    ws = torch.zeros(binding.workspace_bytes(True, B, T, Hq, Hkv, D, 1e4, q.dtype), dtype=torch.uint8, device=DEV)
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4, workspace=ws)
    dq, dk, dv = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, 1e4, workspace=ws)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isnan(t).all())
    # a table built for another length is not accepted either
    binding.ne_rope_table_init(ws, T + 1, D, 1e4)
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all())
    # built for these arguments: the same bits as a fresh workspace
    binding.ne_rope_table_init(ws, T, D, 1e4)
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4, workspace=ws)
    o2, lse2 = binding.ne_rope_attn_fwd(q, k, v, 1e4)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_one_workspace_serves_forward_and_backward():
    """A backward workspace holds the table where the forward reads it: one ne_rope_table_init."""
    B, T, Hq, Hkv, D = 2, 130, 6, 2, 128
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(B, T, Hq, Hkv, D, seed=59, dtype="bf16"))
    ws = bwd_workspace(q, k, 1e4, 0)
    o, lse = binding.ne_rope_attn_fwd(q, k, v, 1e4, workspace=ws)
    dq, dk, dv = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, 1e4, workspace=ws)
    o2, lse2 = binding.ne_rope_attn_fwd(q, k, v, 1e4)
    g2 = binding.ne_rope_attn_bwd(q, k, v, o2, lse2, dO, 1e4)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip((dq, dk, dv), g2):
        assert torch.equal(a, b)
