"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every symbol the
header declares, sizes workspaces, and rejects invalid arguments before launching anything."""
import heapq
import ctypes
import os
import re

import pytest

from causal_gqa_flashattention_rope_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ne_rope_attn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ne_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from causal_gqa_flashattention_rope_amd import build
        build.build()
    return binding.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(L):
    assert L.ne_abi_version() == 3
    names = [L.ne_status_str(st) for st in range(8)]
    assert len(set(names)) == 8 and all(names)
    assert b"table" in names[6] and b"HIP" in names[7]
    assert L.ne_status_str(99) == b"unknown status"
    assert set(binding.STATUS) == set(range(8))


def up(x):
    return (x + 255) // 256 * 256


def ds_tiles(T, G):
    nrt, nkb = -(-T * G // 64), -(-T // 64)
    return sum(1 for kb in range(nkb) for rt in range(nrt) if rt >= kb * G)


def amax_parts(B, T, Hkv):
    return max(1, min(-(-512 // B), -(-T // 8), 1024))


KINDS = {  # pass: rows per job, workgroups per CU, most pieces, cost per job, cost per piece
    "fwd": (256, 1, 4, 1.0, 4.0), "dq": (128, 2, 2, 1.0, 4.0), "dkdv": (64, 1, 4, 2.0, 16.0)}


def split_plan(kind, T, G, ngrp, D=128):
    """(rs, np) of the split of the longest causal blocks of one pass, or None.  Steps per block
    (growing with the index): forward / dQ row block rb, its causal 64-key tiles; dK/dV key block
    nkb - 1 - rb, its 64-row tiles from the diagonal on.  The greedy dispatch of the longest-first
    job list (each job to the slot that frees first) over 256 CUs x wg slots, cost = steps + per
    job + per piece of a split block; the unsplit dK/dV runs mirrored pairs.  The earliest end
    wins if it is below 0.8 of the unsplit one.  (rs, 1) with rs = nrb: single dK/dV key blocks,
    none split.  dK/dV at D <= 64 always has a plan (two workgroups per CU; up to 1024 blocks); the
    forward at D <= 64 has 128-row blocks, three workgroups per CU."""
    BM, wg, maxp, cjob, cpiece = KINDS[kind]
    w4 = kind == "dkdv" and D <= 64
    if w4:
        wg = 2
    if kind == "fwd" and D <= 64:      # the forward's D <= 64 variant: 128 rows, 3 workgroups per CU
        BM, wg = 128, 3
    TG = T * G
    nrb = -(-T // 64) if kind == "dkdv" else -(-TG // BM)
    slots = 256 * wg
    if nrb > 16383 or (w4 and nrb > 1024):
        return None
    if ngrp * nrb > 4 * slots:
        return (nrb, 1) if w4 else None
    if kind == "dkdv":
        tiles = [-(-(TG - (nrb - 1 - rb) * 64 * G) // 64) for rb in range(nrb)]
    else:
        tiles = [min(rb * BM + BM - 1, TG - 1) // G // 64 + 1 for rb in range(nrb)]

    def dispatch(costs):
        h = [0.0] * slots
        last = 0.0
        for c in costs:
            for _ in range(ngrp):
                t = heapq.heappop(h) + c
                heapq.heappush(h, t)
                last = max(last, t)
        return last

    def end(rs, np_):
        jobs = []
        for rb in range(nrb):
            if rb >= rs:
                n = tiles[rb]
                jobs += [(n * (p + 1) // np_ - n * p // np_) + cjob + cpiece for p in range(np_)]
            else:
                jobs.append(tiles[rb] + cjob)
        return dispatch(sorted(jobs, reverse=True))

    ref, single = None, False
    if kind == "dkdv":
        npair = (nrb + 1) // 2
        ref = dispatch([tiles[nrb - 1 - i] + (tiles[i] + cjob if i != nrb - 1 - i else 0.0) + cjob
                        for i in range(npair)])
        m = end(nrb, 1)        # single key blocks, none split
        if w4 or m < 0.97 * ref:
            ref, single = m, True
    else:
        ref = end(nrb, 1)
    best, choice = ref, None
    step = max(1, nrb // 32)
    for np_ in range(2, maxp + 1):
        for rs in range(nrb - 1, -1, -step):
            if tiles[rs] < 2 * np_ or rs + (nrb - rs) * np_ > 1024:
                break
            m = end(rs, np_)
            if m < best:
                best, choice = m, (rs, np_)
    if choice is None or best > 0.8 * ref:
        return (nrb, 1) if single else None
    return choice


def split_bytes(B, T, Hq, Hkv, D, bwd):
    """Workspace of the split blocks: per split block, a slot per piece (forward: O, m, l of 8
    waves x 64 lanes; dQ and dK/dV: 4 waves x 64 lanes of D / 2 floats) and two counters, the
    counters of a call together; the backward's are those of its dQ and dK/dV passes."""
    G, ngrp = Hq // Hkv, B * Hkv
    regions, ncnt = [], 0
    for kind in (("dq", "dkdv") if bwd else ("fwd",)):
        plan = split_plan(kind, T, G, ngrp, D)
        n, np_ = 0, 1
        if plan is not None:
            rs, np_ = plan
            BM = 128 if kind == "fwd" and D <= 64 else KINDS[kind][0]
            nrb = -(-T // 64) if kind == "dkdv" else -(-T * G // BM)
            n = ngrp * (nrb - rs)
        slot = (4 if D <= 64 else 8) * 64 * (D // 2 + 2) if kind == "fwd" else 4 * 64 * (D // 2)
        regions.append(up(n * np_ * slot * 4))
        ncnt += 2 * n
    return sum(regions) + up(ncnt * 4)


def sizes(B, T, Hq, Hkv, D, esz, base=1e4):
    """(header + table, forward, backward base without the optional regions, v' copy); the 16-bit
    forward includes its split regions"""
    nq, nk = B * T * Hq * D, B * T * Hkv * D
    head = 256 + (up(T * (D // 2) * 8) if base > 0 else 0)
    Tp = -(-T // 64) * 64
    fwd = head + up(esz * nk) + up(esz * (B * Hkv * D * Tp if esz == 2 else nk))
    if esz == 2:
        fwd += split_bytes(B, T, Hq, Hkv, D, False)
    bwd = head + 2 * up(esz * nq) + up(esz * nk) + 3 * up(4 * B * T * Hq) + up(4 * B * T * Hkv) + \
        up(4 * B * Hkv) + up(4 * B * Hkv * amax_parts(B, T, Hkv))
    return head, fwd, bwd, up(esz * nk)


def test_split_plans_of_the_parity_shapes():
    """The GPU parity shapes meant to cover the split blocks are split: forward into 4 pieces, the
    dQ pass into 2 (not the third shape's), dK/dV into 2-4 (the third: single key blocks, the D <= 64
    variant at two workgroups per CU); the benchmark's D = 128 workloads keep
    their blocks whole, one GPU's share of the 8192-token layer (one group) splits all three passes;
    at D = 64 the dK/dV pass always has a plan (single key blocks at least)."""
    shapes = [(1, 1000, 4, 1, 128), (1, 1200, 4, 2, 64), (1, 777, 2, 1, 32)]
    fwd = [split_plan("fwd", T, Hq // Hkv, B * Hkv, D) for B, T, Hq, Hkv, D in shapes]
    dq = [split_plan("dq", T, Hq // Hkv, B * Hkv, D) for B, T, Hq, Hkv, D in shapes]
    kv = [split_plan("dkdv", T, Hq // Hkv, B * Hkv, D) for B, T, Hq, Hkv, D in shapes]
    assert all(p is not None and p[1] == 4 for p in fwd)
    assert dq[0] is not None and dq[1] is not None and dq[2] is None
    assert all(p[1] == 2 for p in dq[:2])
    assert kv[0][1] >= 2 and kv[1][1] >= 2 and kv[2] == (-(-777 // 64), 1)   # the third: single blocks
    for B, T, Hq, Hkv in ((4, 2048, 12, 4), (1, 8192, 32, 8)):
        for kind in KINDS:
            assert split_plan(kind, T, Hq // Hkv, B * Hkv, 128) is None, (kind, T)
    # D = 64 layers: forward and dQ keep their blocks; dK/dV runs single key blocks
    for B, T, Hq, Hkv in ((8, 512, 12, 4), (16, 1024, 12, 12)):
        assert split_plan("fwd", T, Hq // Hkv, B * Hkv, 64) is None
        assert split_plan("dq", T, Hq // Hkv, B * Hkv, 64) is None
        assert split_plan("dkdv", T, Hq // Hkv, B * Hkv, 64) == (-(-T // 64), 1)
    for kind in KINDS:
        assert split_plan(kind, 8192, 4, 1, 128)[1] > 1


def wsb(L, is_bwd, B, T, Hq, Hkv, D, base=1e4, dt=binding.NE_BF16, flags=0):
    return L.ne_rope_attn_workspace_bytes(is_bwd, B, T, Hq, Hkv, D, base, dt, flags)


def test_workspace_sizes(L):
    B, T, Hq, Hkv, D = 4, 2048, 12, 4, 128
    head, fwd, bwd, vcopy = sizes(B, T, Hq, Hkv, D, 2)
    assert wsb(L, 0, B, T, Hq, Hkv, D) == fwd
    # this shape keeps its row blocks whole; one group alone (B = 1, Hkv = 1) splits them, in the
    # forward and in the dQ pass
    assert split_bytes(B, T, Hq, Hkv, D, False) == 0 and split_bytes(B, T, Hq, Hkv, D, True) == 0
    assert split_bytes(1, T, 3, 1, D, False) > 0 and split_bytes(1, T, 3, 1, D, True) > 0
    assert wsb(L, 0, 1, T, 3, 1, D) == sizes(1, T, 3, 1, D, 2)[1]
    h1, f1, b1, v1 = sizes(1, T, 3, 1, D, 2)
    assert wsb(L, 1, 1, T, 3, 1, D) == max(f1, b1 + v1 + split_bytes(1, T, 3, 1, D, True))
    # default backward: O(T) -- operand copies (v' included, the dQ pass recomputes from it) and
    # the dQ pass's split regions, no dS
    assert wsb(L, 1, B, T, Hq, Hkv, D) == bwd + vcopy + split_bytes(B, T, Hq, Hkv, D, True)
    # stored dS: 8 KiB per (64-row tile, 64-key block) pair that dK/dV visits, for every group; no v' copy
    G = Hq // Hkv
    assert wsb(L, 1, B, T, Hq, Hkv, D, flags=binding.NE_FLAG_STORE_DS) == \
        bwd + up(B * Hkv * ds_tiles(T, G) * 8192)
    # atomic dQ: the fp32 accumulator (plus 64 padding rows); no v' copy
    assert wsb(L, 1, B, T, Hq, Hkv, D, flags=binding.NE_FLAG_NONDETERMINISTIC) == \
        bwd + up(4 * (B * T * Hq * D + 64 * D))
    # both: the atomic path
    assert wsb(L, 1, B, T, Hq, Hkv, D, flags=binding.NE_FLAG_NONDETERMINISTIC | binding.NE_FLAG_STORE_DS) == \
        wsb(L, 1, B, T, Hq, Hkv, D, flags=binding.NE_FLAG_NONDETERMINISTIC)
    # the fp32 path always recomputes (flags have no effect on its layout)
    h4, f4, b4, v4 = sizes(B, T, Hq, Hkv, D, 4)
    assert wsb(L, 0, B, T, Hq, Hkv, D, dt=binding.NE_F32) == f4
    for fl in (0, binding.NE_FLAG_STORE_DS, binding.NE_FLAG_NONDETERMINISTIC):
        assert wsb(L, 1, B, T, Hq, Hkv, D, dt=binding.NE_F32, flags=fl) == b4 + v4
    # no RoPE: no table after the header
    assert wsb(L, 0, B, T, Hq, Hkv, D, base=0.0) == sizes(B, T, Hq, Hkv, D, 2, base=0.0)[1]
    # a backward workspace also serves the forward (the table sits at the same place)
    assert wsb(L, 1, B, T, Hq, Hkv, D) >= wsb(L, 0, B, T, Hq, Hkv, D)
    # ragged T: the forward's transposed V' copy pads every row of keys to a multiple of 64
    assert wsb(L, 0, B, 100, Hq, Hkv, D) == sizes(B, 100, Hq, Hkv, D, 2)[1]
    # half-split pairs: the backward keeps slot-ordered copies of raw q and k (read by the QK-norm
    # backward); the forward and calls without RoPE need nothing more
    HALF = binding.NE_FLAG_ROPE_HALF_SPLIT
    nq, nk = B * T * Hq * D, B * T * Hkv * D
    assert wsb(L, 0, B, T, Hq, Hkv, D, flags=HALF) == wsb(L, 0, B, T, Hq, Hkv, D)
    for fl in (0, binding.NE_FLAG_STORE_DS, binding.NE_FLAG_NONDETERMINISTIC):
        assert wsb(L, 1, B, T, Hq, Hkv, D, flags=HALF | fl) == wsb(L, 1, B, T, Hq, Hkv, D, flags=fl) + \
            up(2 * nq) + up(2 * nk)
        assert wsb(L, 1, B, T, Hq, Hkv, D, base=0.0, flags=HALF | fl) == wsb(L, 1, B, T, Hq, Hkv, D, base=0.0, flags=fl)
    assert wsb(L, 1, B, T, Hq, Hkv, D, dt=binding.NE_F32, flags=HALF) == b4 + v4 + up(4 * nq) + up(4 * nk)
    # invalid arguments: 0
    assert wsb(L, 0, B, T, 12, 5, D) == 0
    assert wsb(L, 0, B, T, Hq, Hkv, 96) == 0
    assert wsb(L, 0, B, T, Hq, Hkv, D, base=float("nan")) == 0
    assert wsb(L, 1, B, T, Hq, Hkv, D, flags=binding.NE_FLAG_BF16_OPERANDS) == 0
    assert wsb(L, 1, B, T, Hq, Hkv, D, flags=0x100) == 0


def test_group_rows_beyond_32_bit_offsets_are_rejected(L):
    """A (batch, KV head) group's T G rows of head_dim operand elements are addressed with 32-bit byte
    offsets: T G D times 2 (16-bit operands) or 4 (fp32 path) must stay below 2^31."""
    bf, f32 = binding.NE_BF16, binding.NE_F32
    # T G D = 2^29: fine with 16-bit operands, too large on the fp32 path
    assert wsb(L, 1, 1, 1 << 20, 4, 1, 128) > 0
    assert wsb(L, 1, 1, 1 << 20, 4, 1, 128, dt=f32) == 0
    assert wsb(L, 0, 1, 1 << 20, 4, 1, 128, dt=f32) == 0
    # T G D = 2^31 / 2: too large for 16-bit operands as well
    assert wsb(L, 0, 1, 1 << 21, 8, 1, 64, dt=bf) == 0
    assert wsb(L, 0, 1, 1 << 20, 8, 1, 64, dt=bf) > 0
    # the same limit through an entry point (validation fails before any launch)
    assert fwd_call(L, T=1 << 21, Hq=8, Hkv=1, D=64, wsb=1 << 40) == 2   # NE_ERR_SHAPE


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def fwd_call(L, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, T=16, Hq=4, Hkv=2, D=64, base=1e4,
             i=binding.NE_BF16, out=binding.NE_F32, flags=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = L.ne_rope_attn_workspace_bytes(0, B, T, Hq, Hkv, D, base, i, 0) if D in (32, 64, 128) else 1 << 20
    return L.ne_rope_attn_fwd(q, k, v, o, lse, B, T, Hq, Hkv, D, base, i, out, flags, ws, wsb, None)


def bwd_call(L, ptrs=None, B=1, T=16, Hq=4, Hkv=2, D=64, base=1e4, i=binding.NE_BF16,
             out=binding.NE_F32, flags=0, ws=FAKE, wsb=1 << 30):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return L.ne_rope_attn_bwd(*p, B, T, Hq, Hkv, D, base, i, out, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(lse=None), 1), (dict(ws=None), 1),
    (dict(B=0), 2), (dict(T=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2), (dict(Hq=6, Hkv=4), 2),
    (dict(D=96), 3), (dict(D=16), 3), (dict(i=binding.NE_F32, out=binding.NE_BF16), 3),
    (dict(i=binding.NE_BF16, out=binding.NE_F16), 3), (dict(i=7), 3),
    (dict(flags=binding.NE_FLAG_BF16_OPERANDS), 3),
    (dict(flags=binding.NE_FLAG_ROPE_HALF_SPLIT, wsb=16), 5),   # the pairing flag is accepted
    (dict(flags=0x10), 3),
    (dict(q=FAKE + 8), 4), (dict(ws=FAKE + 4), 4),
    (dict(wsb=16), 5),
    (dict(base=float("nan")), 2),
])
def test_fwd_rejects_before_launch(L, kw, status):
    assert fwd_call(L, **kw) == status
    assert L.ne_last_error()


@pytest.mark.parametrize("idx,status", [(0, 1), (5, 1), (8, 1)])
def test_bwd_rejects_null(L, idx, status):
    p = [FAKE] * 9
    p[idx] = None
    assert bwd_call(L, ptrs=p) == status


def test_bwd_rejects_misaligned_small_workspace_and_flags(L):
    p = [FAKE] * 9
    p[6] = FAKE + 2
    assert bwd_call(L, ptrs=p) == 4
    assert bwd_call(L, wsb=100) == 5
    assert bwd_call(L, Hq=5, Hkv=2) == 2
    assert bwd_call(L, flags=binding.NE_FLAG_BF16_OPERANDS) == 3
    assert bwd_call(L, flags=binding.NE_FLAG_ROPE_HALF_SPLIT | binding.NE_FLAG_BF16_OPERANDS) == 3
    assert bwd_call(L, flags=binding.NE_FLAG_ROPE_HALF_SPLIT | binding.NE_FLAG_STORE_DS, wsb=100) == 5
    assert bwd_call(L, flags=1 << 31) == 3
    # the atomic dQ needs its accumulator: a workspace one region short is rejected (the stored dS
    # is covered below: a smaller buffer is valid down to one group)
    nf = L.ne_rope_attn_workspace_bytes(1, 1, 16, 4, 2, 64, 1e4, binding.NE_BF16, binding.NE_FLAG_NONDETERMINISTIC)
    assert bwd_call(L, flags=binding.NE_FLAG_NONDETERMINISTIC, wsb=nf - 256) == 5


def test_stored_ds_workspace_below_one_group_is_rejected(L):
    """With NE_FLAG_STORE_DS the workspace must hold at least one group's dS; the passes then run once
    per batch of as many groups as it holds."""
    B, T, Hq, Hkv, D = 2, 300, 6, 2, 64
    full = L.ne_rope_attn_workspace_bytes(1, B, T, Hq, Hkv, D, 1e4, binding.NE_BF16, binding.NE_FLAG_STORE_DS)
    one = ds_tiles(T, Hq // Hkv) * 8192
    base = full - up(B * Hkv * one)
    assert bwd_call(L, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, flags=binding.NE_FLAG_STORE_DS, wsb=base + one - 1) == 5
    assert b"stored dS" in L.ne_last_error()


def test_table_init_and_check_reject_before_touching_memory(L):
    # rope_base <= 0: nothing to build or check
    assert L.ne_rope_table_init(None, 0, 16, 64, 0.0, None) == 0
    assert L.ne_rope_table_check(None, 0, 16, 64, -1.0, None) == 0
    assert L.ne_rope_table_init(None, 1 << 20, 16, 64, 1e4, None) == 1
    assert L.ne_rope_table_init(FAKE + 4, 1 << 20, 16, 64, 1e4, None) == 4
    assert L.ne_rope_table_init(FAKE, 1 << 20, 0, 64, 1e4, None) == 2
    assert L.ne_rope_table_init(FAKE, 1 << 20, 16, 48, 1e4, None) == 3
    assert L.ne_rope_table_init(FAKE, 1 << 20, 16, 64, float("inf"), None) == 2
    need = 256 + 16 * 32 * 8
    assert L.ne_rope_table_init(FAKE, need - 1, 16, 64, 1e4, None) == 5
    assert L.ne_rope_table_check(None, 1 << 20, 16, 64, 1e4, None) == 1
    assert L.ne_rope_table_check(FAKE, 100, 16, 64, 1e4, None) == 5


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 32)
    with pytest.raises(RuntimeError):
        binding.ne_rope_attn_fwd(q, q[:, :, :1].contiguous(), q[:, :, :1].contiguous(), 1e4)


# ---- window, cache and decode entry points ----------------------------------------------------
def test_ex_calls_reject_before_launch(L):
    opts = binding.make_opts(8)
    args = [FAKE] * 5 + [1, 16, 4, 2, 64, 1e4, ctypes.byref(opts), binding.NE_BF16, binding.NE_F32, 0, FAKE, 16, None,
                         None]
    assert L.ne_rope_attn_fwd_ex(*args) == 5          # workspace too small
    args[5] = 0
    assert L.ne_rope_attn_fwd_ex(*args) == 2          # B = 0
    bargs = [FAKE] * 9 + [1, 16, 4, 2, 64, 1e4, ctypes.byref(opts), binding.NE_BF16, binding.NE_F32, 0, None, 1 << 30,
                          None, None]
    assert L.ne_rope_attn_bwd_ex(*bargs) == 1         # null workspace


def test_cache_and_decode_sizes(L):
    B, Tcap, Hq, Hkv, D = 8, 8192, 32, 8, 128
    assert L.ne_kv_cache_bytes(B, Tcap, Hkv, D, binding.NE_BF16) == 2 * B * Hkv * Tcap * D * 2
    assert L.ne_kv_cache_bytes(B, 100, Hkv, D, binding.NE_BF16) == 0      # Tcap not a multiple of 64
    assert L.ne_kv_cache_bytes(B, Tcap, Hkv, D, binding.NE_F32) == 0      # 16-bit inputs only
    ws = L.ne_rope_attn_decode_workspace_bytes(B, 1, Tcap, Hq, Hkv, D, binding.NE_BF16)
    assert ws >= B * Hq * D * 2
    assert L.ne_rope_attn_decode_workspace_bytes(B, Tcap + 1, Tcap, Hq, Hkv, D, binding.NE_BF16) == 0
    assert L.ne_rope_attn_decode_workspace_bytes(B, 1, Tcap, 30, Hkv, D, binding.NE_BF16) == 0


def decode_call(L, q=FAKE, cache=FAKE, cb=1 << 40, lens=FAKE, o=FAKE, lse=FAKE, B=2, Tq=1, Tcap=256, Hq=4,
                Hkv=2, D=64, base=1e4, W=0, i=binding.NE_BF16, out=binding.NE_F32, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = L.ne_rope_attn_decode_workspace_bytes(B, Tq, Tcap, Hq, Hkv, D, i) if D in (32, 64, 128) else 1 << 20
    opts = binding.make_opts(W)
    return L.ne_rope_attn_decode(q, cache, cb, lens, o, lse, B, Tq, Tcap, Hq, Hkv, D, base, ctypes.byref(opts), i,
                                 out, ws, wsb, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(lens=None), 1), (dict(cache=None), 1),
    (dict(Tcap=100), 2), (dict(Tq=0), 2), (dict(Tq=300), 2), (dict(Hq=5), 2), (dict(B=0), 2),
    (dict(D=96), 3), (dict(i=binding.NE_F32, out=binding.NE_F32), 3), (dict(out=binding.NE_F16), 3),
    (dict(lens=FAKE + 2), 4), (dict(o=FAKE + 8), 4),
    (dict(cb=16), 5), (dict(wsb=16), 5), (dict(base=float("inf")), 2),
])
def test_decode_rejects_before_launch(L, kw, status):
    assert decode_call(L, **kw) == status
    assert L.ne_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(cache=None), 1), (dict(Tn=0), 2), (dict(Tcap=96), 2), (dict(i=binding.NE_F32), 3),
    (dict(k=FAKE + 4), 4), (dict(cb=100), 5),
])
def test_append_rejects_before_launch(L, kw, status):
    a = dict(cache=FAKE, cb=1 << 40, lens=FAKE, k=FAKE, v=FAKE, B=2, Tn=3, Tcap=256, Hkv=2, D=64, base=1e4,
             i=binding.NE_BF16)
    a.update(kw)
    assert L.ne_kv_cache_append(a["cache"], a["cb"], a["lens"], a["k"], a["v"], a["B"], a["Tn"], a["Tcap"],
                                a["Hkv"], a["D"], a["base"], None, a["i"], None) == status


@pytest.mark.parametrize("qkn,status", [((float("nan"), 1e-6), 2), ((1.2, -1.0), 2), ((1.2, float("inf")), 2)])
def test_ex_calls_reject_bad_qk_norm(L, qkn, status):
    opts = binding.make_opts(0, qkn)
    wsf = L.ne_rope_attn_workspace_bytes(0, 1, 16, 4, 2, 64, 1e4, binding.NE_BF16, 0)
    assert L.ne_rope_attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16, 4, 2, 64, 1e4, ctypes.byref(opts),
                                 binding.NE_BF16, binding.NE_F32, 0, FAKE, wsf, None, None) == status
    assert L.ne_rope_attn_bwd_ex(*([FAKE] * 9), 1, 16, 4, 2, 64, 1e4, ctypes.byref(opts), binding.NE_BF16,
                                 binding.NE_F32, 0, FAKE, 1 << 30, None, None) == status


def test_noalloc_decode_rejects_before_touching_the_device(L):
    """The scratch holds NE_DECODE_SCRATCH_BYTES; larger partials fail validation before any HIP call."""
    B, Tq, Tcap, Hq, Hkv, D = 64, 1, 8192, 32, 8, 128
    assert L.ne_rope_attn_decode_workspace_bytes(B, Tq, Tcap, Hq, Hkv, D, binding.NE_BF16) > 64 << 20
    opts = binding.make_opts(0)
    st = L.ne_rope_attn_decode_noalloc(FAKE, FAKE, 1 << 40, FAKE, FAKE, FAKE, B, Tq, Tcap, Hq, Hkv, D, 1e4,
                                       ctypes.byref(opts), binding.NE_BF16, binding.NE_F32, None)
    assert st == 5 and b"scratch" in L.ne_last_error()
    assert L.ne_rope_attn_decode_noalloc(None, FAKE, 1 << 40, FAKE, FAKE, FAKE, 2, 1, 256, 4, 2, 64, 1e4,
                                         ctypes.byref(opts), binding.NE_BF16, binding.NE_F32, None) == 1
    assert L.ne_rope_attn_decode_noalloc(FAKE, FAKE, 1 << 40, FAKE, FAKE, FAKE, 2, 1, 100, 4, 2, 64, 1e4,
                                         ctypes.byref(opts), binding.NE_BF16, binding.NE_F32, None) == 2

