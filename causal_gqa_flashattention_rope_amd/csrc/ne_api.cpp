// ne_api.cpp -- the C ABI (include/ne_rope_attn.h): argument validation, workspace layout and
// dispatch to the gfx950 kernels.  Nothing here allocates, frees, synchronises or prints.
#include "../../include/ne_rope_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "ne_launch.hpp"

namespace {

thread_local char g_err[512] = "";

ne_status_t fail(ne_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

constexpr size_t kAlign = 256;
static_assert(ne::kDecodeScratchBytes == NE_DECODE_SCRATCH_BYTES, "the header states the scratch size");
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t table, qh, kh, vh, dOh, delta, lse2, rq, rk, dsc, amax, dqacc, ds, total;
    size_t qs, ks;  // backward, half-split pairs with RoPE: slot-ordered raw q and k (QK norm backward)
    bool half;      // half-split pairs with RoPE on
    // split row / key blocks: partial results and counters of the forward (fwd, 16-bit) or of the
    // dQ pass (q) and the dK/dV pass (k) of the recomputing 16-bit backward; counters of one call
    // are contiguous (one clearing range), the dQ pass's first
    size_t fpart, qpart, kpart, cnt;
    size_t ncnt_q, ncnt_k;  // counters (unsigned) of the dQ / dK/dV pass (forward: ncnt_q)
    int mode;       // ne::kBwdRecompute, kBwdStoredDs or kBwdAtomic (backward)
    int ds_groups;  // stored dS: groups whose dS the workspace holds at once
    int nparts;     // partial maxima of |dO| per group (16-bit backward)
};

bool dtype_ok(ne_dtype_t in, ne_dtype_t out) {
    if (in == NE_F32) return out == NE_F32;
    if (in == NE_BF16) return out == NE_F32 || out == NE_BF16;
    if (in == NE_F16) return out == NE_F32 || out == NE_F16;
    return false;
}

constexpr unsigned kKnownFlags = NE_FLAG_NONDETERMINISTIC | NE_FLAG_BF16_OPERANDS | NE_FLAG_ROPE_HALF_SPLIT |
                                 NE_FLAG_STORE_DS;

ne_status_t check_flags(unsigned flags) {
    if (flags & ~kKnownFlags) return fail(NE_ERR_UNSUPPORTED, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (flags & NE_FLAG_BF16_OPERANDS)
        return fail(NE_ERR_UNSUPPORTED, "NE_FLAG_BF16_OPERANDS is reserved and not implemented (fp16 operands only)");
    return NE_OK;
}

// esz: bytes of a kernel operand element (4 on the fp32 path, 2 otherwise).  The direct LDS loads
// address a (batch, KV head) group's T G rows with 32-bit byte offsets, so T G D esz stays below 2^31.
ne_status_t check_shape(int B, int T, int Hq, int Hkv, int D, int esz) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1)
        return fail(NE_ERR_SHAPE, "B=%d T=%d Hq=%d Hkv=%d must all be >= 1", B, T, Hq, Hkv);
    if (Hq % Hkv != 0) return fail(NE_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (D != 32 && D != 64 && D != 128)
        return fail(NE_ERR_UNSUPPORTED, "head_dim=%d not in {32, 64, 128}", D);
    if (B > 65535 || Hkv > 65535) return fail(NE_ERR_SHAPE, "B and Hkv must be <= 65535");
    const int64_t TG = (int64_t)T * (Hq / Hkv);
    if (TG + 128 > INT32_MAX) return fail(NE_ERR_SHAPE, "T * Hq / Hkv = %lld is too large", (long long)TG);
    if ((TG + 128) * D * esz > INT32_MAX)
        return fail(NE_ERR_SHAPE, "T * Hq / Hkv * head_dim = %lld is too large for 32-bit row offsets",
                    (long long)(TG * D));
    const int64_t n = (int64_t)B * T * Hq * D;
    if (n > ((int64_t)1 << 46)) return fail(NE_ERR_SHAPE, "tensor of %lld elements is too large", (long long)n);
    return NE_OK;
}

// Bytes of stored dS of one (batch, KV head) group for the 16-bit backward: 8 KiB per tile of 64
// flattened rows x 64 keys that the dK/dV pass visits (ne::ds_tiles_per_group).
size_t ds_group_bytes(int T, int Hq, int Hkv) {
    const int G = Hq / Hkv;
    const int nrt = (int)(((int64_t)T * G + 63) / 64), nkb = (T + 63) / 64;
    return ne::ds_tiles_per_group(nrt, nkb, G) * 8192;
}
constexpr size_t kDsCap = (size_t)4 << 30;   // the stored dS buffer holds at most 4 GiB

// Partial maxima of |dO| per group: one per block of the max pass, which reads whole tokens of one
// batch element -- enough blocks for about 512 workgroups, each at least 8 tokens, at most 1024.
int amax_parts(int B, int T, int Hkv) {
    (void)Hkv;
    const int64_t want = std::max<int64_t>(1, (512 + B - 1) / B);
    return (int)std::max<int64_t>(1, std::min<int64_t>({want, (T + 7) / 8, 1024}));
}

int bwd_mode(ne_dtype_t in, unsigned flags, int T, int Hq, int Hkv) {
    if (in == NE_F32) return ne::kBwdRecompute;
    if (flags & NE_FLAG_NONDETERMINISTIC) return ne::kBwdAtomic;
    if ((flags & NE_FLAG_STORE_DS) && ds_group_bytes(T, Hq, Hkv) <= kDsCap) return ne::kBwdStoredDs;
    return ne::kBwdRecompute;
}

// The plan of one pass (ne::kSplitFwd, kSplitDq, kSplitDkdv).  The plan struct is large: one
// per thread and pass, reused.
ne::SplitPlan* split_scratch(int kind) {
    thread_local ne::SplitPlan sp[3];
    return &sp[kind];
}
ne::SplitPlan* plan_for(int kind, int T, int G, int ngrp, int D) {
    ne::SplitPlan* sp = split_scratch(kind);
    ne::split_plan(kind, T, G, ngrp, D, sp);
    return sp;
}
// split blocks of a plan (0 without one)
size_t split_blocks(const ne::SplitPlan& sp, int ngrp) {
    return sp.njobs ? (size_t)ngrp * (sp.nrb - sp.rs) : 0;
}

// The workspace regions.  ds_bytes: bytes available for the stored dS (stored-dS mode), or
// SIZE_MAX to size it for every group (up to the cap).
Layout layout(bool bwd, int B, int T, int Hq, int Hkv, int D, double base, ne_dtype_t in, unsigned flags,
              size_t ws_bytes = SIZE_MAX) {
    const size_t esz = in == NE_F32 ? 4 : 2;
    const size_t nq = (size_t)B * T * Hq * D, nk = (size_t)B * T * Hkv * D;
    Layout L{};
    L.mode = bwd ? bwd_mode(in, flags, T, Hq, Hkv) : ne::kBwdRecompute;
    L.half = (flags & NE_FLAG_ROPE_HALF_SPLIT) && base > 0.0;
    size_t off = ne::kTableHdrBytes;
    L.table = off;
    if (base > 0.0) off += up((size_t)T * (D / 2) * 8);
    if (bwd) { L.qh = off; off += up(nq * esz); }
    // the forward keeps V'^T as [B * Hkv][D][Tp], Tp = T rounded up to 64 (zeros past T)
    const size_t nv = bwd ? nk : (size_t)B * Hkv * D * (((size_t)T + 63) / 64 * 64);
    L.kh = off; off += up(nk * esz);
    L.vh = off;
    if (!bwd || L.mode == ne::kBwdRecompute) off += up(nv * esz);  // the other backwards read v directly
    if (bwd) {
        const size_t ngrp = (size_t)B * Hkv;
        L.nparts = amax_parts(B, T, Hkv);
        L.dOh = off; off += up(nq * esz);
        L.delta = off; off += up((size_t)B * T * Hq * 4);
        L.lse2 = off; off += up((size_t)B * T * Hq * 4);
        L.rq = off; off += up((size_t)B * T * Hq * 4);
        L.rk = off; off += up((size_t)B * T * Hkv * 4);
        L.dsc = off; off += up(ngrp * 4);
        L.amax = off; off += up(ngrp * L.nparts * 4);
        // the size query sees no options, so the raw copies are kept whether or not the QK norm is on
        if (L.half) {
            L.qs = off; off += up(nq * esz);
            L.ks = off; off += up(nk * esz);
        }
        // the atomic dQ accumulator, plus 64 rows past the last group that the dK/dV pass may add zeros to
        if (L.mode == ne::kBwdAtomic) { L.dqacc = off; off += up((nq + (size_t)64 * D) * 4); }
        if (L.mode == ne::kBwdStoredDs) {
            const size_t gb = ds_group_bytes(T, Hq, Hkv);
            size_t cap = kDsCap;
            if (ws_bytes != SIZE_MAX) cap = std::min(cap, ws_bytes > off ? (ws_bytes - off) / 256 * 256 : 0);
            L.ds_groups = (int)std::min<size_t>(ngrp, cap / gb);
            L.ds = off;
            off += up((size_t)std::max(L.ds_groups, 1) * gb);
        }
    }
    // the split blocks' regions, sized for the plans without a window (a window turns them off)
    if (in != NE_F32 && (!bwd || L.mode == ne::kBwdRecompute)) {
        const int ngrp = B * Hkv, G = Hq / Hkv;
        if (!bwd) {
            const ne::SplitPlan* f = plan_for(ne::kSplitFwd, T, G, ngrp, D);
            const size_t n = split_blocks(*f, ngrp);
            L.fpart = off; off += up(n * f->np * ne::split_slot_floats_fwd(D) * 4);
            L.ncnt_q = 2 * n;
        } else {
            const ne::SplitPlan* q = plan_for(ne::kSplitDq, T, G, ngrp, D);
            const size_t nq = split_blocks(*q, ngrp);
            L.qpart = off; off += up(nq * q->np * ne::split_slot_floats_dq(D) * 4);
            const ne::SplitPlan* k = plan_for(ne::kSplitDkdv, T, G, ngrp, D);
            const size_t nk = split_blocks(*k, ngrp);
            L.kpart = off; off += up(nk * k->np * ne::split_slot_floats_dkdv(D) * 4);
            L.ncnt_q = 2 * nq;
            L.ncnt_k = 2 * nk;
        }
        L.cnt = off; off += up((L.ncnt_q + L.ncnt_k) * 4);
    }
    L.total = off;
    return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Keys a query sees at most: the window, or the whole causal prefix when window <= 0 or >= T.
int visible_keys(int window, int T) { return (window <= 0 || window >= T) ? T : window; }

const ne_attn_opts_t kNoOpts = {0, 0, 1.0f, 0.0f};

ne_status_t check_opts(const ne_attn_opts_t* o, ne::QkNorm* qkn) {
    qkn->on = o->qk_norm != 0;
    qkn->gain = o->qk_gain;
    qkn->eps = o->qk_eps;
    if (qkn->on && (!std::isfinite(o->qk_gain) || !std::isfinite(o->qk_eps) || o->qk_eps < 0.f))
        return fail(NE_ERR_SHAPE, "qk_gain must be finite and qk_eps finite and >= 0");
    return NE_OK;
}

ne_status_t common_checks(int B, int T, int Hq, int Hkv, int D, ne_dtype_t in, ne_dtype_t out, unsigned flags) {
    ne_status_t s = check_shape(B, T, Hq, Hkv, D, in == NE_F32 ? 4 : 2);
    if (s != NE_OK) return s;
    if (!dtype_ok(in, out))
        return fail(NE_ERR_UNSUPPORTED, "dtype pair in=%d out=%d is not supported", (int)in, (int)out);
    return check_flags(flags);
}

}  // namespace

extern "C" {

int ne_abi_version(void) { return NE_ABI_VERSION; }

const char* ne_last_error(void) { return g_err; }

const char* ne_status_str(ne_status_t s) {
    switch (s) {
        case NE_OK: return "ok";
        case NE_ERR_NULL: return "null pointer";
        case NE_ERR_SHAPE: return "invalid shape";
        case NE_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or flag";
        case NE_ERR_ALIGN: return "pointer not 16-byte aligned";
        case NE_ERR_WORKSPACE: return "workspace too small";
        case NE_ERR_NO_ROPE_TABLE: return "no RoPE table for these arguments in the workspace";
        case NE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t ne_rope_attn_workspace_bytes(int is_bwd, int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                    ne_dtype_t in_dtype, unsigned flags) {
    if (in_dtype != NE_F32 && in_dtype != NE_BF16 && in_dtype != NE_F16) return 0;
    if (check_shape(B, T, Hq, Hkv, head_dim, in_dtype == NE_F32 ? 4 : 2) != NE_OK) return 0;
    if (check_flags(flags) != NE_OK || !std::isfinite(rope_base)) return 0;
    const size_t fwd = layout(false, B, T, Hq, Hkv, head_dim, rope_base, in_dtype, flags).total;
    // a backward workspace of this size also serves the forward of the same arguments
    return is_bwd ? std::max(fwd, layout(true, B, T, Hq, Hkv, head_dim, rope_base, in_dtype, flags).total) : fwd;
}

ne_status_t ne_rope_table_init(void* workspace, size_t workspace_bytes, int T, int head_dim, double rope_base,
                               void* stream) {
    if (!std::isfinite(rope_base)) return fail(NE_ERR_SHAPE, "rope_base must be finite");
    if (!(rope_base > 0.0)) return NE_OK;
    if (!workspace) return fail(NE_ERR_NULL, "ne_rope_table_init: workspace must be non-null");
    if (!aligned16(workspace)) return fail(NE_ERR_ALIGN, "ne_rope_table_init: workspace must be 16-byte aligned");
    if (T < 1 || T > (1 << 30)) return fail(NE_ERR_SHAPE, "T=%d must be in [1, 2^30]", T);
    if (head_dim != 32 && head_dim != 64 && head_dim != 128)
        return fail(NE_ERR_UNSUPPORTED, "head_dim=%d not in {32, 64, 128}", head_dim);
    const size_t need = ne::kTableHdrBytes + (size_t)T * (head_dim / 2) * 8;
    if (workspace_bytes < need)
        return fail(NE_ERR_WORKSPACE, "workspace of %zu bytes < %zu for the table", workspace_bytes, need);
    ne::TableArgs a{};
    a.hdr = (ne::TableHdr*)workspace;
    a.table = (float2*)((char*)workspace + ne::kTableHdrBytes);
    a.T = T; a.D = head_dim; a.base = rope_base;
    hipError_t e = ne::launch_table(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(NE_ERR_HIP, "ne_rope_table_init: launch failed: %s", hipGetErrorString(e));
    return NE_OK;
}

ne_status_t ne_rope_table_check(const void* workspace, size_t workspace_bytes, int T, int head_dim, double rope_base,
                                void* stream) {
    if (!(rope_base > 0.0)) return NE_OK;
    if (!workspace) return fail(NE_ERR_NULL, "ne_rope_table_check: workspace must be non-null");
    if (workspace_bytes < ne::kTableHdrBytes)
        return fail(NE_ERR_WORKSPACE, "workspace of %zu bytes holds no table header", workspace_bytes);
    ne::TableHdr h{};
    hipError_t e = hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(NE_ERR_HIP, "ne_rope_table_check: copy failed: %s", hipGetErrorString(e));
    if (!ne::table_matches(h, T, head_dim, rope_base))
        return fail(NE_ERR_NO_ROPE_TABLE, "the workspace table is not built for T=%d head_dim=%d rope_base=%g", T,
                    head_dim, rope_base);
    return NE_OK;
}

}  // extern "C"

namespace {

ne_status_t fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int T, int Hq, int Hkv, int head_dim, double rope_base, const ne_attn_opts_t* opts,
                     ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                     void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    if (!q || !k || !v || !o || !lse || !workspace)
        return fail(NE_ERR_NULL, "ne_rope_attn_fwd: q, k, v, o, lse and workspace must be non-null");
    ne_status_t s = common_checks(B, T, Hq, Hkv, head_dim, in_dtype, out_dtype, flags);
    if (s != NE_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        !aligned16(workspace))
        return fail(NE_ERR_ALIGN, "ne_rope_attn_fwd: every pointer must be 16-byte aligned");
    if (!std::isfinite(rope_base)) return fail(NE_ERR_SHAPE, "rope_base must be finite");
    if (!opts) opts = &kNoOpts;
    ne::QkNorm qkn{};
    if ((s = check_opts(opts, &qkn)) != NE_OK) return s;
    const Layout L = layout(false, B, T, Hq, Hkv, head_dim, rope_base, in_dtype, flags);
    if (workspace_bytes < L.total)
        return fail(NE_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, L.total);
    char* ws = (char*)workspace;
    const int G = Hq / Hkv;
    ne::PrepArgs pa{};
    pa.q = q; pa.k = k; pa.v = v;
    pa.kh = ws + L.kh; pa.vh = ws + L.vh; pa.table = (float2*)(ws + L.table);
    pa.hdr = (const ne::TableHdr*)ws;
    pa.B = B; pa.T = T; pa.Hq = Hq; pa.Hkv = Hkv; pa.D = head_dim;
    pa.rope_base = rope_base;
    pa.qscale = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    pa.qkn = qkn;
    pa.half = L.half ? 1 : 0;
    ne::FwdArgs fa{};
    fa.q = q; fa.kh = pa.kh; fa.vh = pa.vh; fa.table = pa.table; fa.o = o; fa.lse = lse;
    fa.rope_base = rope_base; fa.qscale = pa.qscale;
    fa.B = B; fa.T = T; fa.Hq = Hq; fa.Hkv = Hkv; fa.G = G;
    fa.window = visible_keys(opts->window, T);
    fa.qkn = qkn;
    fa.half = pa.half;
    fa.nrb = (int)(((int64_t)T * G + 127) / 128);
    ne::SplitPlan* sp = split_scratch(ne::kSplitFwd);
    sp->njobs = 0;
    if (in_dtype != NE_F32 && fa.window >= T) {
        plan_for(ne::kSplitFwd, T, G, B * Hkv, head_dim);
        if (sp->njobs) {
            sp->part = (float*)(ws + L.fpart);
            sp->cnt = (unsigned*)(ws + L.cnt);
            pa.split_cnt = sp->cnt;
            pa.nsplit_cnt = (int)L.ncnt_q;
        }
    }
    hipError_t e = ne::launch_fwd((int)in_dtype, (int)out_dtype, head_dim, pa, fa, *sp, (hipStream_t)stream,
                                  (hipEvent_t const*)events);
    if (e != hipSuccess) return fail(NE_ERR_HIP, "ne_rope_attn_fwd: launch failed: %s", hipGetErrorString(e));
    return NE_OK;
}

ne_status_t bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, void* dq, void* dk, void* dv,
                     int B, int T, int Hq, int Hkv, int head_dim, double rope_base, const ne_attn_opts_t* opts,
                     ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                     void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !workspace)
        return fail(NE_ERR_NULL, "ne_rope_attn_bwd: every tensor pointer and the workspace must be non-null");
    ne_status_t s = common_checks(B, T, Hq, Hkv, head_dim, in_dtype, out_dtype, flags);
    if (s != NE_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return fail(NE_ERR_ALIGN, "ne_rope_attn_bwd: every pointer must be 16-byte aligned");
    if (!std::isfinite(rope_base)) return fail(NE_ERR_SHAPE, "rope_base must be finite");
    if (!opts) opts = &kNoOpts;
    ne::QkNorm qkn{};
    if ((s = check_opts(opts, &qkn)) != NE_OK) return s;
    const Layout L = layout(true, B, T, Hq, Hkv, head_dim, rope_base, in_dtype, flags, workspace_bytes);
    if (L.mode == ne::kBwdStoredDs && L.ds_groups < 1)
        return fail(NE_ERR_WORKSPACE, "workspace of %zu bytes holds the stored dS of no group (%zu required)",
                    workspace_bytes, L.total);
    if (workspace_bytes < L.total)
        return fail(NE_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, L.total);
    char* ws = (char*)workspace;
    const int G = Hq / Hkv;
    const bool h16 = in_dtype != NE_F32;
    ne::PrepArgs pa{};
    pa.q = q; pa.k = k; pa.v = v; pa.o = o; pa.lse = lse; pa.dO = dO;
    pa.qh = ws + L.qh; pa.kh = ws + L.kh; pa.vh = ws + L.vh; pa.dOh = ws + L.dOh;
    pa.delta = (float*)(ws + L.delta); pa.lse2 = (float*)(ws + L.lse2); pa.table = (float2*)(ws + L.table);
    pa.rq = (float*)(ws + L.rq); pa.rk = (float*)(ws + L.rk);
    pa.hdr = (const ne::TableHdr*)ws;
    pa.B = B; pa.T = T; pa.Hq = Hq; pa.Hkv = Hkv; pa.D = head_dim;
    pa.rope_base = rope_base;
    pa.qscale = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    pa.qkn = qkn;
    pa.half = L.half ? 1 : 0;
    if (L.half && qkn.on) { pa.qs = ws + L.qs; pa.ks = ws + L.ks; }
    pa.skip_v = L.mode != ne::kBwdRecompute ? 1 : 0;
    pa.amax_part = (const float*)(ws + L.amax);
    pa.nparts = L.nparts;
    pa.dsc = h16 ? (float*)(ws + L.dsc) : nullptr;
    pa.dq_acc = L.mode == ne::kBwdAtomic ? (float*)(ws + L.dqacc) : nullptr;
    ne::AmaxArgs am{};
    am.dO = dO; am.part = (float*)(ws + L.amax);
    am.B = B; am.T = T; am.Hq = Hq; am.Hkv = Hkv; am.nparts = L.nparts;
    am.tpp = (T + L.nparts - 1) / L.nparts;
    ne::BwdArgs ba{};
    ba.qh = pa.qh; ba.kh = pa.kh; ba.vh = pa.vh; ba.dOh = pa.dOh;
    ba.delta = pa.delta; ba.lse2 = pa.lse2; ba.table = pa.table;
    ba.dq = dq; ba.dk = dk; ba.dv = dv;
    ba.B = B; ba.T = T; ba.Hq = Hq; ba.Hkv = Hkv; ba.G = G;
    ba.window = visible_keys(opts->window, T);
    ba.qkn = qkn;
    ba.half = pa.half;
    // the QK norm backward reads raw q and k in the slot order of the kernels
    ba.q = pa.qs ? pa.qs : q; ba.k = pa.ks ? pa.ks : k; ba.in_dt = (int)in_dtype;
    ba.rq = pa.rq; ba.rk = pa.rk;
    ba.ds = L.mode == ne::kBwdStoredDs ? ws + L.ds : nullptr;
    ba.dsc = pa.dsc;
    ba.dq_acc = pa.dq_acc;
    ba.v = v;
    ba.ds_groups = L.ds_groups;
    ba.grp0 = 0;
    ba.ngrp = B * Hkv;
    ba.nrb = (int)(((int64_t)T * G + 127) / 128);
    ba.rope_base = rope_base;
    ba.scale = (float)(1.0 / std::sqrt((double)head_dim));
    ne::SplitPlan* spq = split_scratch(ne::kSplitDq);
    ne::SplitPlan* spk = split_scratch(ne::kSplitDkdv);
    spq->njobs = spk->njobs = 0;
    if (h16 && L.mode == ne::kBwdRecompute && ba.window >= T) {
        if (!qkn.on) plan_for(ne::kSplitDq, T, G, B * Hkv, head_dim);
        plan_for(ne::kSplitDkdv, T, G, B * Hkv, head_dim);
        spq->part = (float*)(ws + L.qpart);
        spq->cnt = (unsigned*)(ws + L.cnt);
        spk->part = (float*)(ws + L.kpart);
        spk->cnt = (unsigned*)(ws + L.cnt) + L.ncnt_q;
        if (spq->njobs || spk->njobs) {
            pa.split_cnt = spq->cnt;
            pa.nsplit_cnt = (int)(L.ncnt_q + L.ncnt_k);
        }
    }
    hipError_t e = ne::launch_bwd((int)in_dtype, (int)out_dtype, head_dim, L.mode, pa, am, ba, *spq, *spk,
                                  (hipStream_t)stream, (hipEvent_t const*)events);
    if (e != hipSuccess) return fail(NE_ERR_HIP, "ne_rope_attn_bwd: launch failed: %s", hipGetErrorString(e));
    return NE_OK;
}

}  // namespace

extern "C" {

ne_status_t ne_rope_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                             ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, head_dim, rope_base, nullptr, in_dtype, out_dtype, flags,
                    workspace, workspace_bytes, stream, nullptr);
}

ne_status_t ne_rope_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dO, void* dq, void* dk, void* dv,
                             int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                             ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, T, Hq, Hkv, head_dim, rope_base, nullptr, in_dtype,
                    out_dtype, flags, workspace, workspace_bytes, stream, nullptr);
}

ne_status_t ne_rope_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                const ne_attn_opts_t* opts, ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                                void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    const unsigned fl = flags | (opts && opts->rope_half_split ? NE_FLAG_ROPE_HALF_SPLIT : 0u);
    return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, head_dim, rope_base, opts, in_dtype, out_dtype, fl,
                    workspace, workspace_bytes, stream, events);
}

ne_status_t ne_rope_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dO, void* dq, void* dk, void* dv,
                                int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                const ne_attn_opts_t* opts, ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                                void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    const unsigned fl = flags | (opts && opts->rope_half_split ? NE_FLAG_ROPE_HALF_SPLIT : 0u);
    return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, T, Hq, Hkv, head_dim, rope_base, opts, in_dtype,
                    out_dtype, fl, workspace, workspace_bytes, stream, events);
}

}  // extern "C"

// =====================================================================================
// Key/value cache and decode.
// =====================================================================================
namespace {

bool decode_dtype_ok(ne_dtype_t in, ne_dtype_t out) {
    if (in == NE_BF16) return out == NE_F32 || out == NE_BF16;
    if (in == NE_F16) return out == NE_F32 || out == NE_F16;
    return false;
}

ne_status_t check_cache_shape(int B, int Tcap, int Hkv, int D) {
    if (B < 1 || Hkv < 1 || Tcap < 64) return fail(NE_ERR_SHAPE, "B=%d Hkv=%d must be >= 1 and Tcap=%d >= 64", B, Hkv, Tcap);
    if (Tcap % 64 != 0) return fail(NE_ERR_SHAPE, "Tcap=%d must be a multiple of 64", Tcap);
    if (D != 32 && D != 64 && D != 128) return fail(NE_ERR_UNSUPPORTED, "head_dim=%d not in {32, 64, 128}", D);
    if (B > 65535 || Hkv > 65535) return fail(NE_ERR_SHAPE, "B and Hkv must be <= 65535");
    if ((int64_t)B * Hkv * Tcap * D > ((int64_t)1 << 44)) return fail(NE_ERR_SHAPE, "cache is too large");
    return NE_OK;
}

// Key slices per (group, 32-row block): at least NE_DECODE_WORKGROUPS workgroups overall (two per
// CU), and at least one slice per NE_DECODE_SPLIT_KEYS keys of the cache's capacity (each wave
// then streams about 8 tiles: measured best on the 8192-token cache at 8 and 32 sequences); at
// most one slice per 32-key tile and kMaxSplits.
#ifndef NE_DECODE_WORKGROUPS
#define NE_DECODE_WORKGROUPS 512
#endif
#ifndef NE_DECODE_SPLIT_KEYS
#define NE_DECODE_SPLIT_KEYS 1024
#endif
int decode_nsplit(int B, int Hkv, int nrb, int Tcap) {
    const int64_t blocks = (int64_t)B * Hkv * nrb;
    int64_t ns = std::max<int64_t>((NE_DECODE_WORKGROUPS + blocks - 1) / blocks,
                                   (Tcap + NE_DECODE_SPLIT_KEYS - 1) / NE_DECODE_SPLIT_KEYS);
    ns = std::min<int64_t>(ns, std::max(1, Tcap / 32));
    ns = std::min<int64_t>(ns, ne::kMaxSplits);
    return (int)std::max<int64_t>(ns, 1);
}

struct DecodeLayout {
    size_t part_o, part_ml, total;
    int nrb, nsplit;
};

DecodeLayout decode_layout(int B, int Tq, int Tcap, int Hq, int Hkv, int D) {
    DecodeLayout L{};
    const int G = Hq / Hkv;
    L.nrb = (int)(((int64_t)Tq * G + 31) / 32);
    L.nsplit = decode_nsplit(B, Hkv, L.nrb, Tcap);
    const size_t slots = (size_t)B * Hkv * L.nrb * L.nsplit;
    size_t off = 0;
    L.part_o = off; off += up(slots * 32 * D * 4);
    L.part_ml = off; off += up(slots * 64 * 4);
    L.total = off;
    return L;
}

ne_status_t check_decode(int B, int Tq, int Tcap, int Hq, int Hkv, int D) {
    ne_status_t s = check_cache_shape(B, Tcap, Hkv, D);
    if (s != NE_OK) return s;
    if (Hq < 1 || Hq % Hkv != 0) return fail(NE_ERR_SHAPE, "Hq=%d is not a positive multiple of Hkv=%d", Hq, Hkv);
    if (Tq < 1 || Tq > Tcap) return fail(NE_ERR_SHAPE, "Tq=%d must be in [1, Tcap=%d]", Tq, Tcap);
    if ((int64_t)Tq * (Hq / Hkv) > (1 << 24)) return fail(NE_ERR_SHAPE, "Tq * Hq / Hkv is too large");
    return NE_OK;
}

}  // namespace

extern "C" {

size_t ne_kv_cache_bytes(int B, int Tcap, int Hkv, int head_dim, ne_dtype_t in_dtype) {
    if (check_cache_shape(B, Tcap, Hkv, head_dim) != NE_OK) return 0;
    if (in_dtype != NE_BF16 && in_dtype != NE_F16) return 0;
    return 2 * (size_t)B * Hkv * Tcap * head_dim * 2;
}

ne_status_t ne_kv_cache_append(void* cache, size_t cache_bytes, const int* cache_lens, const void* k_new,
                               const void* v_new, int B, int Tn, int Tcap, int Hkv, int head_dim, double rope_base,
                               const ne_attn_opts_t* opts, ne_dtype_t in_dtype, void* stream) {
    if (!cache || !cache_lens || !k_new || !v_new)
        return fail(NE_ERR_NULL, "ne_kv_cache_append: cache, cache_lens, k_new and v_new must be non-null");
    ne_status_t s = check_cache_shape(B, Tcap, Hkv, head_dim);
    if (s != NE_OK) return s;
    if (in_dtype != NE_BF16 && in_dtype != NE_F16)
        return fail(NE_ERR_UNSUPPORTED, "ne_kv_cache_append: in_dtype must be BF16 or F16");
    if (Tn < 1 || Tn > Tcap) return fail(NE_ERR_SHAPE, "Tn=%d must be in [1, Tcap=%d]", Tn, Tcap);
    if (!aligned16(cache) || !aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)cache_lens & 3u))
        return fail(NE_ERR_ALIGN, "ne_kv_cache_append: cache, k_new, v_new must be 16-byte aligned, cache_lens 4");
    if (!std::isfinite(rope_base)) return fail(NE_ERR_SHAPE, "rope_base must be finite");
    if (cache_bytes < ne_kv_cache_bytes(B, Tcap, Hkv, head_dim, in_dtype))
        return fail(NE_ERR_WORKSPACE, "cache of %zu bytes < %zu required", cache_bytes,
                    ne_kv_cache_bytes(B, Tcap, Hkv, head_dim, in_dtype));
    ne::QkNorm qkn{};
    if ((s = check_opts(opts ? opts : &kNoOpts, &qkn)) != NE_OK) return s;
    ne::AppendArgs a{};
    a.qkn = qkn;
    a.k = k_new; a.v = v_new; a.cache = cache; a.lens = cache_lens;
    a.B = B; a.Tn = Tn; a.Tcap = Tcap; a.Hkv = Hkv; a.rope_base = rope_base;
    a.half = opts && opts->rope_half_split && rope_base > 0.0 ? 1 : 0;
    for (int i = 0; i < head_dim / 2; ++i)
        a.theta[i] = rope_base > 0.0 ? std::pow(rope_base, -2.0 * i / head_dim) : 0.0;
    hipError_t e = ne::launch_append((int)in_dtype, head_dim, a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(NE_ERR_HIP, "ne_kv_cache_append: launch failed: %s", hipGetErrorString(e));
    return NE_OK;
}

size_t ne_rope_attn_decode_workspace_bytes(int B, int Tq, int Tcap, int Hq, int Hkv, int head_dim,
                                           ne_dtype_t in_dtype) {
    if (check_decode(B, Tq, Tcap, Hq, Hkv, head_dim) != NE_OK) return 0;
    if (in_dtype != NE_BF16 && in_dtype != NE_F16) return 0;
    return decode_layout(B, Tq, Tcap, Hq, Hkv, head_dim).total;
}

}  // extern "C"

namespace {

// workspace == nullptr with noalloc: the library's file-scope scratch (ne::decode_scratch).
ne_status_t decode_impl(const void* q, const void* cache, size_t cache_bytes, const int* cache_lens,
                        void* o, float* lse, int B, int Tq, int Tcap, int Hq, int Hkv, int head_dim,
                        double rope_base, const ne_attn_opts_t* opts, ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                        void* workspace, size_t workspace_bytes, bool noalloc, void* stream, void* const* events) {
    if (!q || !cache || !cache_lens || !o || !lse || (!workspace && !noalloc))
        return fail(NE_ERR_NULL, "ne_rope_attn_decode: q, cache, cache_lens, o, lse and workspace must be non-null");
    ne_status_t s = check_decode(B, Tq, Tcap, Hq, Hkv, head_dim);
    if (s != NE_OK) return s;
    if (!decode_dtype_ok(in_dtype, out_dtype))
        return fail(NE_ERR_UNSUPPORTED, "ne_rope_attn_decode: dtype pair in=%d out=%d is not supported",
                    (int)in_dtype, (int)out_dtype);
    if (!aligned16(q) || !aligned16(cache) || !aligned16(o) || !aligned16(lse) || (!noalloc && !aligned16(workspace)) ||
        ((uintptr_t)cache_lens & 3u))
        return fail(NE_ERR_ALIGN, "ne_rope_attn_decode: pointers must be 16-byte aligned (cache_lens 4)");
    if (!std::isfinite(rope_base)) return fail(NE_ERR_SHAPE, "rope_base must be finite");
    if (cache_bytes < ne_kv_cache_bytes(B, Tcap, Hkv, head_dim, in_dtype))
        return fail(NE_ERR_WORKSPACE, "cache of %zu bytes < %zu required", cache_bytes,
                    ne_kv_cache_bytes(B, Tcap, Hkv, head_dim, in_dtype));
    if (!opts) opts = &kNoOpts;
    ne::QkNorm qkn{};
    if ((s = check_opts(opts, &qkn)) != NE_OK) return s;
    const DecodeLayout L = decode_layout(B, Tq, Tcap, Hq, Hkv, head_dim);
    if (noalloc) {
        if (L.total > ne::kDecodeScratchBytes)
            return fail(NE_ERR_WORKSPACE,
                        "ne_rope_attn_decode_noalloc: the split partials need %zu bytes, more than the %zu bytes of "
                        "the library's scratch (use ne_rope_attn_decode with a workspace)", L.total,
                        ne::kDecodeScratchBytes);
        hipError_t e = ne::decode_scratch(&workspace);
        if (e != hipSuccess)
            return fail(NE_ERR_HIP, "ne_rope_attn_decode_noalloc: no scratch address on this device: %s",
                        hipGetErrorString(e));
    } else if (workspace_bytes < L.total) {
        return fail(NE_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, L.total);
    }
    char* ws = (char*)workspace;
    ne::DecodeArgs a{};
    a.q = q; a.cache = cache; a.lens = cache_lens;
    a.part_o = (float*)(ws + L.part_o); a.part_ml = (float*)(ws + L.part_ml);
    a.o = o; a.lse = lse;
    a.B = B; a.Tq = Tq; a.Tcap = Tcap; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
    a.nrb = L.nrb; a.nsplit = L.nsplit;
    a.window = visible_keys(opts->window, Tcap);
    a.qkn = qkn;
    a.rope_base = rope_base;
    a.half = opts->rope_half_split && rope_base > 0.0 ? 1 : 0;
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    for (int i = 0; i < head_dim / 2; ++i)
        a.theta[i] = rope_base > 0.0 ? std::pow(rope_base, -2.0 * i / head_dim) : 0.0;
    hipError_t e = ne::launch_decode((int)in_dtype, (int)out_dtype, head_dim, a, (hipStream_t)stream,
                                     (hipEvent_t const*)events);
    if (e != hipSuccess) return fail(NE_ERR_HIP, "ne_rope_attn_decode: launch failed: %s", hipGetErrorString(e));
    return NE_OK;
}

}  // namespace

extern "C" {

ne_status_t ne_rope_attn_decode(const void* q, const void* cache, size_t cache_bytes, const int* cache_lens,
                                void* o, float* lse, int B, int Tq, int Tcap, int Hq, int Hkv, int head_dim,
                                double rope_base, const ne_attn_opts_t* opts, ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                                void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    return decode_impl(q, cache, cache_bytes, cache_lens, o, lse, B, Tq, Tcap, Hq, Hkv, head_dim, rope_base, opts,
                       in_dtype, out_dtype, workspace, workspace_bytes, false, stream, events);
}

ne_status_t ne_rope_attn_decode_noalloc(const void* q, const void* cache, size_t cache_bytes, const int* cache_lens,
                                        void* o, float* lse, int B, int Tq, int Tcap, int Hq, int Hkv, int head_dim,
                                        double rope_base, const ne_attn_opts_t* opts, ne_dtype_t in_dtype,
                                        ne_dtype_t out_dtype, void* stream) {
    return decode_impl(q, cache, cache_bytes, cache_lens, o, lse, B, Tq, Tcap, Hq, Hkv, head_dim, rope_base, opts,
                       in_dtype, out_dtype, nullptr, 0, true, stream, nullptr);
}

}  // extern "C"

// =====================================================================================
// QKV projection with the RoPE epilogue.
// =====================================================================================
extern "C" {

size_t ne_qkv_rope_workspace_bytes(int T, int head_dim) {
    if (T < 1 || (head_dim != 32 && head_dim != 64 && head_dim != 128)) return 0;
    return up((size_t)T * (head_dim / 2) * 8);
}

ne_status_t ne_qkv_rope_proj(const void* x, const void* w, void* q, void* k, void* v,
                             int B, int T, int C, int Hq, int Hkv, int head_dim, double rope_base,
                             const ne_attn_opts_t* opts, ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                             void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    if (!x || !w || !q || !k || !v || !workspace)
        return fail(NE_ERR_NULL, "ne_qkv_rope_proj: x, w, q, k, v and workspace must be non-null");
    if (B < 1 || T < 1 || C < 64 || Hq < 1 || Hkv < 1)
        return fail(NE_ERR_SHAPE, "B=%d T=%d Hq=%d Hkv=%d must be >= 1 and C=%d >= 64", B, T, Hq, Hkv, C);
    if (head_dim != 32 && head_dim != 64 && head_dim != 128)
        return fail(NE_ERR_UNSUPPORTED, "head_dim=%d not in {32, 64, 128}", head_dim);
    if (C % 64 != 0) return fail(NE_ERR_SHAPE, "C=%d must be a multiple of 64", C);
    const int64_t N = (int64_t)(Hq + 2 * Hkv) * head_dim, M = (int64_t)B * T;
    if (N % 128 != 0) return fail(NE_ERR_SHAPE, "(Hq + 2 Hkv) * head_dim = %lld must be a multiple of 128", (long long)N);
    if (std::max(M, N) * C * 2 >= ((int64_t)1 << 31))
        return fail(NE_ERR_SHAPE, "B*T*C and N*C must stay below 2^30 elements");
    if (!decode_dtype_ok(in_dtype, out_dtype))
        return fail(NE_ERR_UNSUPPORTED, "ne_qkv_rope_proj: dtype pair in=%d out=%d is not supported",
                    (int)in_dtype, (int)out_dtype);
    if (!aligned16(x) || !aligned16(w) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(workspace))
        return fail(NE_ERR_ALIGN, "ne_qkv_rope_proj: every pointer must be 16-byte aligned");
    if (!std::isfinite(rope_base)) return fail(NE_ERR_SHAPE, "rope_base must be finite");
    if (workspace_bytes < ne_qkv_rope_workspace_bytes(T, head_dim))
        return fail(NE_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes,
                    ne_qkv_rope_workspace_bytes(T, head_dim));
    ne::QkNorm qkn{};
    ne_status_t s = check_opts(opts ? opts : &kNoOpts, &qkn);
    if (s != NE_OK) return s;
    ne::QkvArgs a{};
    a.x = x; a.w = w; a.q = q; a.k = k; a.v = v; a.table = (float2*)workspace;
    a.M = (int)M; a.C = C; a.N = (int)N; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.D = head_dim;
    a.rope_base = rope_base; a.qkn = qkn;
    a.half = opts && opts->rope_half_split && rope_base > 0.0 ? 1 : 0;
    for (int i = 0; i < head_dim / 2; ++i)
        a.theta[i] = rope_base > 0.0 ? std::pow(rope_base, -2.0 * i / head_dim) : 0.0;
    hipError_t e = ne::launch_qkv((int)in_dtype, (int)out_dtype, head_dim, a, (hipStream_t)stream,
                                  (hipEvent_t const*)events);
    if (e != hipSuccess) return fail(NE_ERR_HIP, "ne_qkv_rope_proj: launch failed: %s", hipGetErrorString(e));
    return NE_OK;
}

}  // extern "C"
