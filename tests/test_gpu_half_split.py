"""GPU parity of the half-split rotary pairing (NE_FLAG_ROPE_HALF_SPLIT: element i rotated with element
i + D/2 by t * theta_i) against the oracle's half-split path; needs an MI355X.

Bars as in test_gpu_parity (2e-3 of each output's scale with 16-bit inputs, 1e-5 on the fp32 path;
16-bit outputs add half an ulp).  The library runs its adjacent-pair kernels on rows whose slots hold
the elements in the order i -> 2i, i + D/2 -> 2i + 1, so a half-split call must give bitwise the
results of an adjacent-pair call on inputs reordered that way (gradients reordered back), which one
test checks exactly.  The options field rope_half_split carries the same pairing to the _ex calls
(bitwise the flag's results), to the KV-cache append and decode (against the decode oracle's
half-split path) and to the QKV projection (against its oracle).
"""
import ctypes

import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding, inputs
from tests.test_gpu_decode import seqs
from tests.test_gpu_parity import ATOMIC, DEV, STORE_DS, check, f64, zero_ref_scale
from tests.test_gpu_qkv import check_qkv, make

pytestmark = pytest.mark.gpu

HALF = binding.NE_FLAG_ROPE_HALF_SPLIT
_NAME = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}
QKN = (1.2, 1e-6)

CASES = [
    # B, T, Hq, Hkv, D, in, out, backward flags, window, QK norm
    (1, 1, 2, 1, 64, torch.bfloat16, torch.float32, 0, 0, None),
    (2, 100, 6, 2, 64, torch.bfloat16, torch.float32, 0, 0, None),
    (1, 129, 4, 1, 128, torch.bfloat16, torch.bfloat16, 0, 0, None),
    (1, 200, 8, 2, 32, torch.float16, torch.float32, 0, 0, None),
    (1, 77, 4, 2, 32, torch.float32, torch.float32, 0, 0, None),
    (2, 130, 3, 3, 128, torch.float32, torch.float32, 0, 0, None),
    (1, 1000, 4, 1, 128, torch.bfloat16, torch.bfloat16, 0, 0, None),   # split blocks in every pass
    (1, 300, 6, 2, 128, torch.bfloat16, torch.float32, STORE_DS, 0, None),
    (1, 300, 6, 2, 64, torch.bfloat16, torch.float32, ATOMIC, 0, None),
    (2, 300, 4, 2, 128, torch.bfloat16, torch.float32, 0, 64, None),
    (2, 200, 6, 2, 64, torch.bfloat16, torch.float32, 0, 0, QKN),
    (1, 250, 4, 2, 128, torch.bfloat16, torch.float32, STORE_DS, 0, QKN),
    (1, 250, 4, 2, 128, torch.float16, torch.float16, ATOMIC, 0, QKN),
    (1, 150, 4, 4, 64, torch.float32, torch.float32, 0, 0, QKN),
]


def _run(q, k, v, dO, base, out_dt, flags, window, qkn):
    qd, kd, vd, dOd = (t.to(DEV) for t in (q, k, v, dO))
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    ws = binding.alloc_workspace(binding.workspace_bytes(True, B, T, Hq, Hkv, D, base, q.dtype, flags), DEV)
    binding.ne_rope_table_init(ws, T, D, base)
    o, lse = binding.ne_rope_attn_fwd(qd, kd, vd, base, out_dtype=out_dt, workspace=ws, flags=flags & HALF,
                                      window=window, qk_norm=qkn)
    dq, dk, dv = binding.ne_rope_attn_bwd(qd, kd, vd, o, lse, dOd, base, workspace=ws, flags=flags, window=window,
                                          qk_norm=qkn)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o, lse, dq, dk, dv)]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}Hq{c[2]}Hkv{c[3]}D{c[4]}-{_NAME[c[5]]}-{_NAME[c[6]]}"
                                             f"-f{c[7]}-w{c[8]}-{'qkn' if c[9] else 'plain'}" for c in CASES])
def test_half_split_parity(case):
    B, T, Hq, Hkv, D, in_dt, out_dt, flags, window, qkn = case
    base = 1.0e4
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=800 + T, dtype=_NAME[in_dt])
    o, lse, dq, dk, dv = _run(q, k, v, dO, base, out_dt, HALF | flags, window, qkn)
    ro, rlse = oracle.fwd(f64(q), f64(k), f64(v), base, window=window, qk_norm=qkn, half_split=True)
    if out_dt == torch.float32:
        rdq, rdk, rdv = oracle.bwd(f64(q), f64(k), f64(v), f64(dO), base, window=window, qk_norm=qkn, half_split=True)
    else:
        rdq, rdk, rdv = oracle.bwd_given_o(f64(q), f64(k), f64(v), f64(o), f64(dO), base, window=window, qk_norm=qkn,
                                           half_split=True)
    gscale = zero_ref_scale(in_dt, (rdq, rdk, rdv))
    for name, g, r in (("o", o, ro), ("lse", lse, rlse), ("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        check(name, g, r, in_dt, out_dt, zero_scale=gscale)


def _to_slots(x):
    """[..., D]: element i to position 2i, element i + D/2 to position 2i + 1."""
    D = x.shape[-1]
    y = torch.empty_like(x)
    y[..., 0::2], y[..., 1::2] = x[..., :D // 2], x[..., D // 2:]
    return y


def _from_slots(y):
    return torch.cat([y[..., 0::2], y[..., 1::2]], dim=-1)


@pytest.mark.parametrize("flags", [0, STORE_DS, ATOMIC], ids=["recompute", "stored_ds", "atomic"])
@pytest.mark.parametrize("shape", [(2, 300, 6, 2, 128), (1, 1000, 4, 1, 64), (1, 200, 8, 2, 32)])
def test_half_split_is_bitwise_the_adjacent_pairs_on_reordered_inputs(shape, flags):
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=900, dtype="bf16")
    h = _run(q, k, v, dO, 1.0e4, torch.float32, HALF | flags, 0, None)
    a = _run(_to_slots(q), _to_slots(k), v, dO, 1.0e4, torch.float32, flags, 0, None)
    assert torch.equal(h[0], a[0]) and torch.equal(h[1], a[1]) and torch.equal(h[4], a[4])
    assert torch.equal(h[3], _from_slots(a[3]))
    if flags == ATOMIC:   # dq: atomic adds in a varying order
        assert float((h[2] - _from_slots(a[2])).abs().max() / h[2].abs().max()) < 1e-5
    else:
        assert torch.equal(h[2], _from_slots(a[2]))


def test_half_split_without_rope_is_the_plain_call():
    q, k, v, dO = inputs.random_case(1, 150, 4, 2, 64, seed=901, dtype="bf16")
    h = _run(q, k, v, dO, 0.0, torch.float32, HALF, 0, None)
    a = _run(q, k, v, dO, 0.0, torch.float32, 0, 0, None)
    for x, y in zip(h, a):
        assert torch.equal(x, y)


# ---- the same pairing through the options struct: KV cache, decode, QKV projection -----------------


def test_options_field_equals_the_flag():
    """ne_attn_opts_t.rope_half_split on the _ex calls gives the bits of NE_FLAG_ROPE_HALF_SPLIT."""
    B, T, Hq, Hkv, D = 1, 300, 6, 2, 64
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(B, T, Hq, Hkv, D, seed=902, dtype="bf16"))
    ws = binding.new_workspace(True, q, k, 1e4, HALF)
    o1, l1 = binding.ne_rope_attn_fwd(q, k, v, 1e4, workspace=ws, flags=HALF, window=T // 2)
    g1 = [t.clone() for t in binding.ne_rope_attn_bwd(q, k, v, o1, l1, dO, 1e4, workspace=ws, flags=HALF,
                                                       window=T // 2)]
    o1, l1 = o1.clone(), l1.clone()
    opts = binding.make_opts(T // 2, None, rope_half_split=True)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    L = binding.lib()
    rc = L.ne_rope_attn_fwd_ex(binding._ptr(q), binding._ptr(k), binding._ptr(v), binding._ptr(o2), binding._ptr(l2),
                               B, T, Hq, Hkv, D, 1e4, ctypes.byref(opts), binding._DT[q.dtype],
                               binding._DT[o2.dtype], 0, binding._ptr(ws), binding._nbytes(ws), binding._stream(), None)
    assert rc == 0
    g2 = [torch.empty_like(t) for t in g1]
    rc = L.ne_rope_attn_bwd_ex(binding._ptr(q), binding._ptr(k), binding._ptr(v), binding._ptr(o2), binding._ptr(l2),
                               binding._ptr(dO), *(binding._ptr(t) for t in g2), B, T, Hq, Hkv, D, 1e4,
                               ctypes.byref(opts), binding._DT[q.dtype], binding._DT[o2.dtype], 0, binding._ptr(ws),
                               binding._nbytes(ws), binding._stream(), None)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("case", [
    # B, P, Tq, Hq, Hkv, D, lens, window, in, out, QK norm
    (3, 200, 1, 8, 2, 128, [0, 57, 199], 0, torch.bfloat16, torch.float32, None),
    (2, 300, 5, 12, 4, 64, [10, 295], 0, torch.bfloat16, torch.bfloat16, None),
    (1, 640, 1, 4, 4, 32, [639], 100, torch.float16, torch.float32, None),
    (2, 256, 9, 6, 2, 128, [100, 247], 64, torch.bfloat16, torch.float32, QKN),
])
def test_half_split_decode_parity(case):
    B, P, Tq, Hq, Hkv, D, lens, window, in_dt, out_dt, qkn = case
    Tcap = (P + 63) // 64 * 64
    base = 1e4
    q, k, v = seqs(B, P, Hq, Hkv, D, 610, _NAME[in_dt])
    cache = binding.new_kv_cache(B, Tcap, Hkv, D, k.dtype, DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    for p0 in range(0, P, 64):
        n = min(64, P - p0)
        lens0 = torch.full((B,), p0, dtype=torch.int32, device=DEV)
        binding.ne_kv_cache_append(cache, lens0, kd[:, p0:p0 + n].contiguous(), vd[:, p0:p0 + n].contiguous(), Tcap,
                                   base, qk_norm=qkn, rope_half_split=True)
    q_new = torch.stack([q[b, lens[b]:lens[b] + Tq] for b in range(B)]).to(DEV)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = binding.ne_rope_attn_decode(q_new, cache, lens_d, Tcap, Hkv, base, window, out_dtype=out_dt, qk_norm=qkn,
                                         rope_half_split=True)
    o2, lse2 = binding.ne_rope_attn_decode_noalloc(q_new, cache, lens_d, Tcap, Hkv, base, window, out_dtype=out_dt,
                                                   qk_norm=qkn, rope_half_split=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    ro, rlse = oracle.decode_fwd(f64(q_new.cpu()), [f64(k[b]) for b in range(B)], [f64(v[b]) for b in range(B)], lens,
                                 base, window, qk_norm=qkn, half_split=True)
    check("o", o.cpu(), ro, in_dt, out_dt)
    check("lse", lse.cpu(), rlse, in_dt, out_dt)


@pytest.mark.parametrize("shape", [(2, 100, 128, 4, 2, 32), (1, 300, 256, 6, 1, 64), (2, 129, 192, 4, 2, 128),
                                   (1, 8100, 64, 12, 4, 128)])
@pytest.mark.parametrize("qkn", [None, QKN])
def test_half_split_qkv_parity(shape, qkn):
    B, T, C, Hq, Hkv, D = shape
    x, w = make(B, T, C, Hq, Hkv, D, 5100 + T, "bf16")
    q, k, v = binding.ne_qkv_rope_proj(x.to(DEV), w.to(DEV), Hq, Hkv, 1e4, qk_norm=qkn, rope_half_split=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope_proj(f64(x), f64(w), Hq, Hkv, 1e4, qk_norm=qkn, half_split=True)
    for nm, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_qkv(nm, g.cpu(), r, torch.float32)
