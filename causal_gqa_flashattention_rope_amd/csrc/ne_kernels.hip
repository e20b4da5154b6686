// ne_kernels.hip -- gfx950 kernels for causal grouped-query attention with RoPE.
//
// Passages followed (titles of the pages the method is described on):
//  * "NanoEuler: 使用 C 和 CUDA 从零开始构建的 GPT-2 规模 LLM" -- 技术规格 (RoPE on queries and keys;
//    grouped-query attention sharing a smaller set of key/value heads), 核心架构与设计
//    (decoder-only, no biases), 内核实现 (tiled FlashAttention with an online softmax so the
//    T x T matrix is never stored), 验证与稳定性 (hand-written backward).
//  * "用 100KB C/CUDA 单文件复刻 GPT-2:NanoEuler 116M 单卡可跑的全流程拆解" -- §3.4 (tiles of
//    query/key/value staged in on-chip shared memory; each separate pass such as RoPE costs a
//    launch and memory traffic, which is why RoPE is folded into the operand preparation here).
//
// The RoPE table (cos/sin of every position, built once per workspace by rope_table_kernel) is
// read by every call.  Pipeline of one call (all stream-ordered, no host synchronisation):
//  forward : prep  -> k' = fp16(R(k)) rows, v' = fp16(v) transposed (16-bit operands).
//            fwd   -> per 256 flattened (token, head) rows of one KV group (128 at head_dim <= 64
//                     and on the fp32 path): q~ = fp16(R(q) * scale * log2 e) in registers, online
//                     softmax over 64-key tiles staged once in LDS for all query heads of the
//                     group; o, lse.
//  backward: max   -> the largest |dO| of each (batch, KV head) group (its fp16 scale).
//            prep  -> q~, k', v', dO' = fp16(s dO) and Delta = s rowsum(dO * o), lse2 = lse log2 e.
//            dkdv  -> per pair of mirrored 64-key blocks of one KV head (or, under a plan, per key
//                     block or piece of one): dK, dV accumulated over every query row of the group
//                     (all G heads), written once; inverse RoPE in the epilogue.
//            dq    -> per 128 flattened rows: recomputes S and dP and adds dS K, written once;
//                     inverse RoPE in the epilogue.  No atomics: bit-reproducible.
//          (opt-in: the dK/dV pass stores the fp16 dS tiles and dq_ds_kernel reads them; or it
//           adds dQ with atomics into an fp32 accumulator, converted by dq_acc_convert_kernel.)
// A plan made on the host (ne_split.cpp) may cut the longest causal blocks of a launch with few
// blocks per CU over several workgroups; the last of them combines the partial results in a fixed
// order.

// Flattened rows: within a (batch, KV head) group the G query heads are interleaved with the
// tokens, row R = t * G + hh (hh = head within the group).  In the [B][T][Hq][D] input these
// rows are exactly the memory order of one token's heads, and the causal mask depends only on
// t = R / G, so any G packs into fixed 128-row blocks that share one K/V tile.
#include <algorithm>

#include "ne_common.hpp"
#include "ne_launch.hpp"

namespace ne {

// =====================================================================================
// Operand preparation.
// =====================================================================================
// cos/sin of t * theta_i, theta_i = base^(-2i/D), for tokens [t0, t0 + TT) into cs[TT][D/2].
// theta_i and the phase t * theta_i are formed in double precision and the phase is reduced to
// [-pi, pi] there (two-term 2 pi), so the single-precision sincos sees a small argument and the
// table entries are within a few fp32 ulps of the exactly rounded values at any position.
__device__ __forceinline__ float2 rope_cs_at(int t, double theta) {
    constexpr double kTwoPiHi = 6.283185307179586;        // 2 pi rounded to double
    constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2 pi - kTwoPiHi
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double phi = (double)t * theta;
    const double n = rint(phi * kInvTwoPi);
    const double r = fma(-n, kTwoPiLo, fma(-n, kTwoPiHi, phi));
    float sv, cv;
    sincosf((float)r, &sv, &cv);
    return make_float2(cv, sv);
}
// The RoPE table of positions 0 .. T-1, each entry evaluated directly, and its header.
// grid ceil(T D / 2 / 256), 256 threads.
__global__ __launch_bounds__(256) void rope_table_kernel(TableArgs a) {
    const int half = a.D / 2;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx < a.T * half) {
        const int t = idx / half, i = idx % half;
        const double theta = exp2(-2.0 * (double)i / (double)a.D * log2(a.base));
        a.table[idx] = rope_cs_at(t, theta);
    }
    if (idx == 0) {
        TableHdr h{};
        h.magic = kTableMagic; h.T = a.T; h.D = a.D; h.pad = 0; h.base = a.base;
        *a.hdr = h;
    }
}

// 1 when the workspace's table was built for this call's (T, D, base) or RoPE is off, else NaN: the
// preparation kernels multiply their rotated copies by it, so a missing table shows as NaN outputs.
__device__ __forceinline__ float table_guard(const PrepArgs& a) {
    if (!(a.rope_base > 0.0)) return 1.f;
    return table_matches(*a.hdr, a.T, a.D, a.rope_base) ? 1.f : __builtin_nanf("");
}

// Eight consecutive input elements as fp32, with 16-byte loads.
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(p), b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}
template <typename T16>
__device__ __forceinline__ void load8(const T16* p, float (&x)[8]) {
    typedef T16 v8 __attribute__((ext_vector_type(8)));
    const v8 a = *reinterpret_cast<const v8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
}

// Partial maxima of |dO| for the per-group scale of dO (16-bit operands).  grid (nparts, B), 256
// threads: block (p, b) reads tokens [p tpp, (p + 1) tpp) of batch b, all Hq heads (a token's rows
// are contiguous), and writes the max of each of its KV groups to part[(b Hkv + g) nparts + p].
// Each thread owns fixed 16-byte chunks of a token's rows (so a fixed group) and walks the block's
// tokens with a running max, several loads in flight; groups are then reduced in LDS (max of
// non-negative floats = max of their bit patterns as unsigned), kAmaxGroups per pass.
constexpr int kAmaxGroups = 256;
template <typename TI, int D>
__global__ __launch_bounds__(256) void dO_amax_kernel(AmaxArgs a) {
    __shared__ unsigned smax[kAmaxGroups];
    constexpr int CPR = D / 8;
    const int p = blockIdx.x, b = blockIdx.y;
    const int G = a.Hq / a.Hkv;
    const int t0 = p * a.tpp, t1 = min(a.T, t0 + a.tpp);
    const int rowlen = a.Hq * CPR;                               // 16-byte chunks per token
    const size_t tok = (size_t)a.Hq * D;                         // elements per token
    // rowlen < 256: 256 / rowlen sets of threads take every sets-th token; else one set
    const int sets = rowlen < 256 ? 256 / rowlen : 1;
    const int set = rowlen < 256 ? (int)threadIdx.x / rowlen : 0;
    const int q0 = rowlen < 256 ? (int)threadIdx.x % rowlen : (int)threadIdx.x;
    const TI* base = (const TI*)a.dO + ((size_t)b * a.T + t0) * tok;
    for (int g0 = 0; g0 < a.Hkv; g0 += kAmaxGroups) {
        const int ng = min(kAmaxGroups, a.Hkv - g0);
        for (int i = threadIdx.x; i < ng; i += 256) smax[i] = 0u;
        __syncthreads();
        if (set < sets) {
            for (int q = q0; q < rowlen; q += 256) {
                const int g = (q / CPR) / G - g0;
                if (g < 0 || g >= ng) continue;
                const TI* src = base + (size_t)set * tok + (size_t)q * 8;
                float m = 0.f;
#pragma unroll 4
                for (int t = t0 + set; t < t1; t += sets, src += (size_t)sets * tok) {
                    float x[8];
                    load8(src, x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
                }
                // (fmaxf skips a NaN element here; it still reaches the gradients through dO itself)
                atomicMax(&smax[g], __float_as_uint(m));
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < ng; i += 256)
            a.part[((size_t)b * a.Hkv + g0 + i) * a.nparts + p] = __uint_as_float(smax[i]);
        __syncthreads();
    }
}

constexpr int kPrepScales = 256;   // groups per batch element whose dO scales a preparation block keeps

// The power of two s that brings a group's max |dO| into [4, 8) (1 for an all-zero or non-finite
// maximum): s dO is exact in fp32 and its fp16 rounding keeps the relative precision of every
// normal element; gradients are linear in dO and are multiplied by 1 / s at the end.
__device__ __forceinline__ float dO_scale(float amax) {
    if (!(amax > 0.f) || !(amax < INFINITY)) return 1.f;
    const int e = min(120, max(-120, 2 - ilogbf(amax)));
    return ldexpf(1.f, e);
}

template <typename TI, typename OP, int D, bool ROT>
__device__ __forceinline__ void convert8(const TI* src, OP* dst, const float2* cs_row, int chunk, float mul,
                                         bool half = false, TI* raw = nullptr) {
    // 8 consecutive slots chunk*8 .. chunk*8+7 (src and dst point at slot chunk*8 of their rows),
    // pairs (2i, 2i+1) rotated by cs_row[i].  half (ROT only): the half-split pairing, slot 2i takes
    // element i and slot 2i+1 element i + D/2 of the source row, and raw (or null) receives the
    // slots unrotated.
    float x[8];
    if (ROT && half) {
        const TI* row = src - chunk * 8;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            x[2 * p] = to_f32(row[chunk * 4 + p]);
            x[2 * p + 1] = to_f32(row[D / 2 + chunk * 4 + p]);
        }
        if (raw) {
#pragma unroll
            for (int e = 0; e < 8; ++e) raw[e] = from_f32<TI>(x[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = to_f32(src[e]);
    }
    if (ROT) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float2 r = cs_row[chunk * 4 + p];
            const float a = x[2 * p], b = x[2 * p + 1];
            x[2 * p] = a * r.x - b * r.y;
            x[2 * p + 1] = a * r.y + b * r.x;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = from_f32<OP>(x[e] * mul);
}

// grid (ceil(T / TT), B, Z), 256 threads.  Forward: k, v and the cos/sin table.  Backward: q, k, v,
// dO, Delta, lse2 and the table.  The rows of a token (q heads, k, v, dO heads) are cut into Z equal
// ranges, one per blockIdx.z, so that a small call still launches enough workgroups to keep many
// loads in flight.
// The hand-off counters of the split row blocks of the attention pass that follows start at zero.
__device__ __forceinline__ void clear_split_counters(const PrepArgs& a) {
    if (!a.split_cnt) return;
    const int nthr = gridDim.x * gridDim.y * gridDim.z * blockDim.x;
    const int i0 = ((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    for (int i = i0; i < a.nsplit_cnt; i += nthr) a.split_cnt[i] = 0u;
}
template <typename TI, typename TO, typename OP, int D, bool BWD>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    constexpr int TT = 8;
    constexpr int CPR = D / 8;  // 8-element chunks per row
    __shared__ float2 cs[TT * (D / 2)];
    __shared__ unsigned gmax[BWD ? kPrepScales : 1];   // backward: max |dO| of each group of batch b
    __shared__ float gsc[BWD ? kPrepScales : 1];       // and its power-of-two scale
    const int t0 = blockIdx.x * TT, b = blockIdx.y;
    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
    const bool rope = a.rope_base > 0.0;
    clear_split_counters(a);
    for (int idx = threadIdx.x; idx < TT * (D / 2); idx += blockDim.x) {
        const int t = t0 + idx / (D / 2);
        cs[idx] = rope && t < T ? a.table[(size_t)t * (D / 2) + idx % (D / 2)] : make_float2(1.f, 0.f);
    }
    if constexpr (BWD && sizeof(OP) == 2) {
        if (Hkv <= kPrepScales) {   // the groups of batch b: their partial maxima reduced once per block
            for (int g = threadIdx.x; g < Hkv; g += blockDim.x) gmax[g] = 0u;
            __syncthreads();
            const int n = Hkv * a.nparts;
            for (int i = threadIdx.x; i < n; i += blockDim.x)
                atomicMax(&gmax[i / a.nparts], __float_as_uint(a.amax_part[(size_t)b * Hkv * a.nparts + i]));
            __syncthreads();
            for (int g = threadIdx.x; g < Hkv; g += blockDim.x) gsc[g] = dO_scale(__uint_as_float(gmax[g]));
        }
    }
    const float guard = table_guard(a);
    __syncthreads();
    const int qrows = BWD ? Hq : 0;  // the forward rotates q inside the attention kernel
    const int skip_v = BWD && a.skip_v ? Hkv : 0;  // rows of v not copied
    const int rows_per_tok = qrows + 2 * Hkv - skip_v + (BWD ? Hq : 0);
    const int zr0 = rows_per_tok * blockIdx.z / gridDim.z, zr1 = rows_per_tok * (blockIdx.z + 1) / gridDim.z;
    const int zrows = zr1 - zr0;   // this block's rows of each token
    const int items = TT * zrows * CPR;
    const int items_pad = (items + 255) / 256 * 256;  // whole waves iterate together
    const size_t TG = (size_t)T * G;
    for (int idx = threadIdx.x; idx < items_pad; idx += 256) {
        const int chunk = idx % CPR;
        const int rowid = idx / CPR;
        const int tl = rowid / zrows;
        int which = zr0 + rowid % zrows + (BWD ? 0 : Hq);  // forward: skip the q rows
        if (which >= Hq + Hkv) which += skip_v;
        const int t = t0 + tl;
        const bool live = idx < items && t < T;
        const float2* csr = cs + tl * (D / 2);
        float part = 0.f;  // Delta partial (dO rows only)
        int dO_row = -1;
        // 16-bit operands: the power-of-two scale of this dO row's group
        float sdo = 1.f;
        if constexpr (BWD && sizeof(OP) == 2) {
            if (which >= Hq + 2 * Hkv) {
                const int g = (which - Hq - 2 * Hkv) / G;
                if (Hkv <= kPrepScales) {
                    sdo = gsc[g];
                } else {  // more groups than the block keeps: reduce this group's partial maxima here
                    const float* pp = a.amax_part + ((size_t)b * Hkv + g) * a.nparts;
                    float m = 0.f;
                    for (int j = 0; j < a.nparts; ++j) m = fmaxf(m, pp[j]);
                    sdo = dO_scale(m);
                }
            }
        }
        // QK norm: the factor gain / rms of this thread's q or k row (its CPR chunks sit in
        // consecutive lanes), and 1/rms kept for the backward's epilogues
        float fac = 1.f;
        if (a.qkn.on) {
            float ss = 0.f;
            if (live && which < Hq + Hkv) {
                const TI* src = which < Hq ? (const TI*)a.q + (((size_t)b * T + t) * Hq + which) * D
                                           : (const TI*)a.k + (((size_t)b * T + t) * Hkv + (which - Hq)) * D;
                float x[8];
                load8(src + chunk * 8, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
            }
            ss = sum_lanes(ss, CPR);
            const float rho = 1.f / sqrtf(ss / (float)D + a.qkn.eps);
            fac = a.qkn.gain * rho;
            if (BWD && live && chunk == 0 && which < Hq + Hkv) {
                if (which < Hq) a.rq[((size_t)b * Hkv + which / G) * TG + (size_t)t * G + which % G] = rho;
                else a.rk[((size_t)b * Hkv + (which - Hq)) * T + t] = rho;
            }
        }
        if (live) {
            if (which < Hq) {  // q -> q~ (rotated, scaled by scale*log2e), flattened rows
                const int hq = which, g = hq / G, hh = hq % G;
                const size_t in_off = (((size_t)b * T + t) * Hq + hq) * D + chunk * 8;
                const TI* src = (const TI*)a.q + in_off;
                OP* dst = (OP*)a.qh + (((size_t)b * Hkv + g) * TG + (size_t)t * G + hh) * D + chunk * 8;
                if (rope) convert8<TI, OP, D, true>(src, dst, csr, chunk, a.qscale * fac * guard, a.half,
                                                    a.qs ? (TI*)a.qs + in_off : nullptr);
                else convert8<TI, OP, D, false>(src, dst, csr, chunk, a.qscale * fac);
            } else if (which < Hq + Hkv) {  // k -> k'
                const int g = which - Hq;
                const size_t in_off = (((size_t)b * T + t) * Hkv + g) * D + chunk * 8;
                const TI* src = (const TI*)a.k + in_off;
                OP* dst = (OP*)a.kh + (((size_t)b * Hkv + g) * T + t) * D + chunk * 8;
                if (rope) convert8<TI, OP, D, true>(src, dst, csr, chunk, fac * guard, a.half,
                                                    a.ks ? (TI*)a.ks + in_off : nullptr);
                else convert8<TI, OP, D, false>(src, dst, csr, chunk, fac);
            } else if (which < Hq + 2 * Hkv) {  // v -> v'
                const int g = which - Hq - Hkv;
                const TI* src = (const TI*)a.v + (((size_t)b * T + t) * Hkv + g) * D + chunk * 8;
                OP* dst = (OP*)a.vh + (((size_t)b * Hkv + g) * T + t) * D + chunk * 8;
                convert8<TI, OP, D, false>(src, dst, csr, chunk, 1.f);
            } else if (BWD) {  // dO -> dO' (flattened) and the Delta partial sum
                const int hq = which - Hq - 2 * Hkv, g = hq / G, hh = hq % G;
                const size_t in_off = (((size_t)b * T + t) * Hq + hq) * D + chunk * 8;
                const TI* src = (const TI*)a.dO + in_off;
                const TO* osrc = (const TO*)a.o + in_off;
                const size_t frow = ((size_t)b * Hkv + g) * TG + (size_t)t * G + hh;
                OP* dst = (OP*)a.dOh + frow * D + chunk * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = to_f32(src[e]);
                    part += x * to_f32(osrc[e]);
                    dst[e] = from_f32<OP>(x * sdo);
                }
                if (a.dq_acc) {   // the atomic dQ accumulator starts at zero
                    floatx4* acc = reinterpret_cast<floatx4*>(a.dq_acc + frow * D + chunk * 8);
                    acc[0] = floatx4{};
                    acc[1] = floatx4{};
                }
                if (a.dsc && t == 0 && hh == 0 && chunk == 0) a.dsc[(size_t)b * Hkv + g] = 1.f / sdo;
                dO_row = (int)hq;
                if (chunk == 0) a.lse2[frow] = a.lse[((size_t)b * Hq + hq) * T + t] * kLog2e;
            }
        }
        if (BWD) {
            // reduce the Delta partials over the CPR consecutive lanes of one row
#pragma unroll
            for (int off = 1; off < CPR; off <<= 1) part += __shfl_xor(part, off, 64);
            if (live && dO_row >= 0 && chunk == 0) {
                const int g = dO_row / G, hh = dO_row % G;
                a.delta[((size_t)b * Hkv + g) * TG + (size_t)t * G + hh] = part * sdo;
            }
        }
    }
}

// Forward preparation for 16-bit operands.  grid (Tp / 64, B * Hkv, 2), 256 threads: 64 tokens of
// one (batch, KV head) group; z = 0: k' = fp16(R(k)) rows as [group][T][D] with the cos/sin rows
// of the workspace table; z = 1: v' = fp16(v) transposed to [group][D][Tp] with the key
// order of vt_key_of_pos and zeros past T.
template <typename TI, int D>
__global__ __launch_bounds__(256) void prep_fwd_h(PrepArgs a) {
    constexpr int TB = 64, CPR = D / 8;
    clear_split_counters(a);
    __shared__ _Float16 vts[D][TB + 8];                // v'^T of the 64 tokens (144-byte rows)
    const int t0 = blockIdx.x * TB, grp = blockIdx.y;
    const int T = a.T, Hkv = a.Hkv, b = grp / Hkv, hkv = grp % Hkv;
    const int Tp = (T + TB - 1) / TB * TB;
    if (blockIdx.z == 0) {
        const bool rope = a.rope_base > 0.0;
        const float guard = table_guard(a);
        for (int idx = threadIdx.x; idx < TB * CPR; idx += 256) {
            const int tl = idx / CPR, chunk = idx % CPR, t = t0 + tl;
            float fac = guard;  // times the QK norm factor of this key row (its chunks sit in consecutive lanes)
            if (a.qkn.on) {
                float x[8], ss = 0.f;
                if (t < T) {
                    load8((const TI*)a.k + (((size_t)b * T + t) * Hkv + hkv) * D + chunk * 8, x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
                }
                fac *= qk_factor(sum_lanes(ss, CPR), D, a.qkn.gain, a.qkn.eps);
            }
            if (t < T) {
                const size_t in_off = (((size_t)b * T + t) * Hkv + hkv) * D + chunk * 8;
                _Float16* kdst = (_Float16*)a.kh + ((size_t)grp * T + t) * D + chunk * 8;
                if (rope) convert8<TI, _Float16, D, true>((const TI*)a.k + in_off, kdst, a.table + (size_t)t * (D / 2),
                                                          chunk, fac, a.half);
                else convert8<TI, _Float16, D, false>((const TI*)a.k + in_off, kdst, nullptr, chunk, fac);
            }
        }
        return;
    }
    for (int idx = threadIdx.x; idx < TB * CPR; idx += 256) {
        const int tl = idx / CPR, chunk = idx % CPR, t = t0 + tl;
        float x[8];
        if (t < T) {
            load8((const TI*)a.v + (((size_t)b * T + t) * Hkv + hkv) * D + chunk * 8, x);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) vts[chunk * 8 + e][tl] = (_Float16)x[e];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < D * (TB / 8); idx += 256) {
        const int d = idx / (TB / 8), pc = idx % (TB / 8);
        half8 out;
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = vts[d][vt_key_of_pos(8 * pc + j)];
        *reinterpret_cast<half8*>((_Float16*)a.vh + ((size_t)grp * D + d) * Tp + t0 + 8 * pc) = out;
    }
}

// =====================================================================================
// Block -> work mapping.  Workgroups are dispatched round-robin over the 8 XCDs (each with its
// own L2), so dispatch index i runs on XCD i % 8.  When the (batch, KV head) groups divide
// evenly, XCD x takes groups x, x + 8, ... and walks their row blocks longest-first, so the K/V
// (or Q/dO) of a group are fetched into one L2 only; otherwise blocks go longest-first in order.
// =====================================================================================
struct Work {
    int blk, grp;  // row/key block index and (b * Hkv + hkv)
};
__device__ __forceinline__ Work map_block(int nblk, int ngrp, bool longest_last) {
    const int i = blockIdx.x;
    int j, g;
    if ((ngrp & 7) == 0) {
        const int x = i & 7, k = i >> 3, per = ngrp >> 3;
        j = k / per;
        g = x + 8 * (k % per);
    } else {
        j = i / ngrp;
        g = i % ngrp;
    }
    return Work{longest_last ? nblk - 1 - j : j, g};
}

// The job of this workgroup under a split plan (SPLIT): row block, piece and piece count (np = 1:
// the block's whole key range), and its group.  Without one, blocks go longest-first as above.
// The split variants are instantiations of their own, so the plain kernels keep their registers.
struct RowJob {
    int rb, piece, np, grp;
};
template <bool SPLIT>
__device__ __forceinline__ RowJob map_row_job(const SplitPlan& sp, int nrb, int ngrp) {
    if constexpr (!SPLIT) {
        const Work w = map_block(nrb, ngrp, true);
        return RowJob{w.blk, 0, 1, w.grp};
    } else {
        const Work w = map_block(sp.njobs, ngrp, false);
        const unsigned e = sp.job[w.blk];
        const int rb = (int)(e >> 2);
        return RowJob{rb, (int)(e & 3u), rb >= sp.rs ? sp.np : 1, w.grp};
    }
}
// Key tiles [lo, hi) of piece p of np of the range [j0, j1).
__device__ __forceinline__ int piece_lo(int j0, int j1, int p, int np) { return j0 + (j1 - j0) * p / np; }

// =====================================================================================
// Forward.  grid (nrb * B * Hkv), 256 threads = 4 waves x 32 flattened rows.
// S^T = K Q^T puts one query row per lane (and its 16+16 keys in the two lane halves), so the
// online-softmax row max and sum are in-lane plus one half swap.  O^T = V^T P^T reuses the
// accumulator registers of S^T as the contraction operand.  K and V tiles (64 keys) are copied
// HBM->LDS by direct loads into swizzled, double-buffered tiles; a wave skips the tiles that
// lie wholly past its rows and masks only the tiles that cross its diagonal.  The running max
// is refreshed only when a row's new maximum exceeds it by more than 2^8 (the probabilities stay
// below 256 in between), so the rescale of O is rare.
// =====================================================================================
// Query fragments (B operand of S^T = K Q^T) of one row, rotated, scaled and converted.
// half (with cs): the half-split pairing, slot 2i takes element i of the row and slot 2i + 1
// element i + D/2.
template <typename TI, typename OP, int D>
__device__ __forceinline__ void load_q_frags(typename Mma<OP>::frag (&qf)[D / Mma<OP>::K], const TI* row,
                                             const float2* cs, float mul, int h, bool valid, bool half) {
    constexpr int KS = D / Mma<OP>::K;
    if constexpr (sizeof(OP) == 2) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
            if (valid) {
                const int e0 = 16 * ks + 8 * h;
                if (cs && half) {
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        x[2 * p] = to_f32(row[e0 / 2 + p]);
                        x[2 * p + 1] = to_f32(row[D / 2 + e0 / 2 + p]);
                    }
                } else {
                    load8(row + e0, x);
                }
                if (cs) {
                    const floatx4 c01 = *reinterpret_cast<const floatx4*>(cs + e0 / 2);
                    const floatx4 c23 = *reinterpret_cast<const floatx4*>(cs + e0 / 2 + 2);
                    const float2 rr[4] = {{c01[0], c01[1]}, {c01[2], c01[3]}, {c23[0], c23[1]}, {c23[2], c23[3]}};
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float2 r = rr[p];
                        const float u = x[2 * p], v = x[2 * p + 1];
                        x[2 * p] = u * r.x - v * r.y;
                        x[2 * p + 1] = u * r.y + v * r.x;
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = (_Float16)(x[e] * mul);
        }
    } else {
        // fp32 operands: k-step ks uses element 2ks + h, i.e. one element of rotary pair ks
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float val = 0.f;
            if (valid) {
                const bool hs = cs && half;
                const float u = to_f32(row[hs ? ks : 2 * ks]), v = to_f32(row[hs ? D / 2 + ks : 2 * ks + 1]);
                val = h == 0 ? u : v;
                if (cs) {
                    const float2 r = cs[ks];
                    val = h == 0 ? u * r.x - v * r.y : u * r.y + v * r.x;
                }
            }
            qf[ks] = val * mul;
        }
    }
}

template <typename TI, typename OP, int D, typename TOUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_kernel(FwdArgs a) {
    using M = Mma<OP>;
    using TL = Tile<OP, D>;
    constexpr bool F16 = sizeof(OP) == 2;
    constexpr int BM = 128, BN = 64, NW = 4;
    constexpr int KS = D / M::K;
    constexpr int NDB = D / 32;
    constexpr int TILE = BN * D;                      // elements per K or V tile
    constexpr float TAU = 8.f;
    __shared__ __attribute__((aligned(1024))) OP lds[2 * 2 * TILE];

    const int T = a.T, G = a.G, TG = T * G;
    const Work wk = map_block(a.nrb, a.B * a.Hkv, true);
    const int rb = wk.blk;
    const int hkv = wk.grp % a.Hkv, b = wk.grp / a.Hkv;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    const int R0 = rb * BM;
    const int Rw = R0 + 32 * w;
    const int R = Rw + c;
    const bool rvalid = R < TG;
    const int t_lane = R / G;
    const int wave_tmin = Rw / G;
    const int wave_tmax = min(Rw + 31, TG - 1) / G;
    const int ntiles = min(R0 + BM - 1, TG - 1) / G / BN + 1;
    const int W = a.window;
    const int j0 = max(0, R0 / G - W + 1) / BN;  // the block's first key tile

    const size_t grp = (size_t)wk.grp;
    const OP* kg = (const OP*)a.kh + grp * (size_t)T * D;
    const OP* vg = (const OP*)a.vh + grp * (size_t)T * D;
    const bool rope = a.rope_base > 0.0;

    typename M::frag qf[KS];
    {
        const int t = min(t_lane, T - 1), hh = R - t_lane * G;
        const TI* qrow = (const TI*)a.q + (((size_t)b * T + t) * a.Hq + hkv * G + hh) * D;
        float qmul = a.qscale;
        if (a.qkn.on && rvalid) qmul *= qk_factor(row_sumsq(qrow, D), D, a.qkn.gain, a.qkn.eps);
        load_q_frags<TI, OP, D>(qf, qrow, rope ? a.table + (size_t)t * (D / 2) : nullptr, qmul, h, rvalid, a.half);
    }
    wait_all();
    lds_fill<OP, D, BN, NW>(lds, kg, j0 * BN, T);
    lds_fill<OP, D, BN, NW>(lds + TILE, vg, j0 * BN, T);

    // kMFloor instead of -inf: a row whose first tiles are all masked keeps p = 0 until a tile
    // it sees raises m (the first such tile always does)
    float m_run = kMFloor, l_run = 0.f;
    floatx16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = floatx16{};

    for (int it = j0; it < ntiles; ++it) {
        const OP* Ks = lds + ((it - j0) & 1) * 2 * TILE;
        const OP* Vs = Ks + TILE;
        lds_fill_wait();
        if (it + 1 < ntiles) {
            OP* nxt = lds + ((it + 1 - j0) & 1) * 2 * TILE;
            lds_fill<OP, D, BN, NW>(nxt, kg, (it + 1) * BN, T);
            lds_fill<OP, D, BN, NW>(nxt + TILE, vg, (it + 1) * BN, T);
        }
        const int n0 = it * BN;
        if (n0 > wave_tmax) continue;                 // every row of this wave precedes the tile
        if (wave_tmin - (n0 + BN - 1) >= W) continue;  // the tile is older than every row's window

        floatx16 s[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            s[mb] = floatx16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[mb] = M::mma(row_frag_sw<OP, D>(Ks, 32 * mb + c, ks, h), qf[ks], s[mb]);
        }
        if (n0 + BN - 1 > wave_tmin || wave_tmax - n0 >= W) {  // crosses a diagonal or a window edge
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!visible(n0 + 32 * mb + acc_row(r, h), t_lane, W)) s[mb][r] = -INFINITY;
        }
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        mx = max_halves(mx);
        if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {  // rare: refresh the reference max
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m_run = m_new;
        }
        float psum = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[mb][r] - m_run);
                s[mb][r] = p;
                psum += p;
            }
        l_run += psum;

        if constexpr (F16) {
            half8 pf[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) pf[kk] = pack_frag_f16(s[kk >> 1], kk & 1);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    oacc[db] = M::mma(tr_frag_f16_sw<D>((const _Float16*)Vs, kk, 32 * db), pf[kk], oacc[db]);
        } else {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int st = 0; st < 16; ++st)
                        oacc[db] = M::mma(tr_frag_f32_sw<D>((const float*)Vs, mb, st, 32 * db), s[mb][st], oacc[db]);
        }
    }

    const float l_tot = sum_halves(l_run);
    const float inv = 1.f / l_tot;
    if (rvalid && h == 0) {
        const int t = t_lane, hq = hkv * G + (R - t * G);
        a.lse[((size_t)b * a.Hq + hq) * T + t] = (m_run + __log2f(l_tot)) * kLn2;
    }
    // o rows through LDS (the K/V stages are free once every wave has left the loop)
    static_assert(2 * 2 * TILE * sizeof(OP) >= 4 * 32 * D * sizeof(TOUT), "LDS holds the output rows");
    __syncthreads();
    store_rows<TOUT, D>(oacc, inv, reinterpret_cast<char*>(lds) + w * 32 * D * (int)sizeof(TOUT), [&](int i) {
        const int Ri = Rw + i;
        if (Ri >= TG) return (TOUT*)nullptr;
        const int t = Ri / G;
        return (TOUT*)a.o + (((size_t)b * T + t) * a.Hq + hkv * G + (Ri - t * G)) * D;
    });
}

// =====================================================================================
// Forward, 16-bit operands.  grid (ceil(T G / 256) * B * Hkv), 512 threads = 8 waves x 32
// flattened rows (two waves per SIMD share every 64-key K and V tile), software-pipelined
// inside each wave.  Iteration j of a wave:
//   phase 1  O^T += V^T P^T for tile j - 1 on the matrix cores while the ALU exponentiates the
//            scores of tile j (independent, so the two interleave in a fixed issue order);
//   phase 2  the scores of tile j + 1;
//   then its mask (diagonal tiles only), row max and the rare refresh of the reference max m.
// A refresh rescales the row sum at once and O after the next phase 1, which adds the last
// probabilities that still use the old m.  The row sums are packed dot products of the fp16
// probabilities that the product consumes.  The score products start from -m (one fold k-step
// per 32-key accumulator), so the exponentials take the accumulators as they are; a refresh
// rebases the tile in hand.  V arrives transposed (vt_frag), so both operand streams are plain
// 16-byte LDS reads, four products ahead of their use.  K and V^T tiles go through 3-stage LDS
// rings filled two iterations ahead by direct loads; the main loop is unrolled by six, so ring
// stages and probability buffers are compile-time and their offsets fold into the LDS
// instructions.
// =====================================================================================
template <int V> struct IC { static constexpr int value = V; };

// Shifts that ride on one extra k-step of a product: three fp16 terms with 256 a + b + c = x to
// about 2^-33 |x| (|x| < 2^24) in lane half 0 of one operand (k = 0, 1, 2; lane half 1 holds
// zeros), against fold_weights (256, 1, 1) in the other, add x to every accumulator element of
// the lane's row or column with fp32 accuracy and no per-element arithmetic.
__device__ __forceinline__ half8 fold_frag(float x, int h) {
    const _Float16 a = (_Float16)(x * (1.f / 256.f));
    const float r1 = x - 256.f * (float)a;
    const _Float16 b = (_Float16)r1;
    const _Float16 c = (_Float16)(r1 - (float)b);
    const _Float16 z = (_Float16)0.f;
    return h == 0 ? half8{a, b, c, z, z, z, z, z} : half8{z, z, z, z, z, z, z, z};
}
// The matching operand (k = 0, 1, 2 weighted 256, 1, 1 for every row or column).
__device__ __forceinline__ half8 fold_weights(int h) {
    const _Float16 z = (_Float16)0.f;
    return h == 0 ? half8{(_Float16)256.f, (_Float16)1.f, (_Float16)1.f, z, z, z, z, z} : half8{z, z, z, z, z, z, z, z};
}


// head_dim <= 64: 4 waves (128 rows) per workgroup and three workgroups per CU (168 VGPRs: one
// probability buffer, operands two products ahead), since each tile then carries half the products
// of D = 128 for the same exponentials; the 12-head 1024-token MHA layer's forward 56.5 -> 45.4 us.
template <typename TI, int D, typename TOUT, bool SPLIT>
__global__ __launch_bounds__(D <= 64 ? 256 : 512) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 2)))
void fwd_kernel_h(FwdArgs a, SplitPlan sp) {
    using OP = _Float16;
    using M = Mma<OP>;
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    constexpr int NW = D <= 64 ? 4 : 8, BM = 32 * NW, BN = 64, KS = D / 16, NDB = D / 32, TILE = BN * D;
    constexpr int N1 = 4 * NDB, N2 = 2 * KS;             // products in phase 1 and phase 2
    constexpr float TAU = 8.f;
    constexpr int NST = 3;
    constexpr int RING = 2 * NST * TILE * (int)sizeof(OP), OUTB = 4 * 32 * D * (int)sizeof(TOUT);
    __shared__ __attribute__((aligned(1024))) char lds_raw[RING > OUTB ? RING : OUTB];
    OP* const lds = reinterpret_cast<OP*>(lds_raw);    // K stages 0..2, then V^T stages 0..2

    const int T = a.T, G = a.G, TG = T * G, Tp = (T + 63) / 64 * 64;
    const RowJob job = map_row_job<SPLIT>(sp, a.nrb, a.B * a.Hkv);
    const int rb = job.rb;
    const int hkv = job.grp % a.Hkv, b = job.grp / a.Hkv;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    const int R0 = rb * BM;
    const int Rw = R0 + 32 * w;
    const int R = Rw + c;
    const bool rvalid = R < TG;
    const int t_lane = R / G;
    const int wave_tmin = Rw / G;
    const int wave_tmax = min(Rw + 31, TG - 1) / G;
    const int W = a.window;
    // the block's key tiles are [jb0, jb1); this job runs piece job.piece of them, [j0, ntiles)
    const int jb0 = max(0, R0 / G - W + 1) / BN, jb1 = min(R0 + BM - 1, TG - 1) / G / BN + 1;
    const int j0 = piece_lo(jb0, jb1, job.piece, job.np);
    const int ntiles = piece_lo(jb0, jb1, job.piece + 1, job.np);
    // this wave's last key tile in the piece (-1: none, the wave only joins the loads and barriers)
    const int wlast = Rw < TG ? wave_tmax / BN : -1;
    const int last = wlast >= j0 ? min(wlast, ntiles - 1) : -1;
    const int first = max(max(0, wave_tmin - W + 1) / BN, j0);  // this wave's first

    const size_t grp = (size_t)job.grp;
    const OP* kg = (const OP*)a.kh + grp * (size_t)T * D;
    const OP* vtg = (const OP*)a.vh + grp * (size_t)D * Tp;
    const bool rope = a.rope_base > 0.0;
    // ring stage of tile j: (j - j0) % NST, a compile-time constant in the unrolled main loop, so
    // the stage offsets fold into the LDS instructions' immediate offsets
    const unsigned lds0 = lds_addr(lds);
    auto kst = [&](int s) { return lds + s * TILE; };
    auto vst = [&](int s) { return lds + (NST + s) * TILE; };
    auto fill_k = [&](int j, int s) { lds_fill_at<OP, D, BN, NW>(lds0 + (unsigned)(s * TILE * 2), kg, j * BN, T); };
    auto fill_v = [&](int j, int s) {
        lds_fill_vt_at<D, BN, NW>(lds0 + (unsigned)((NST + s) * TILE * 2), vtg, j * BN, Tp);
    };
    const int nkw = lds_fill_count<OP, D, BN, NW>(w), nvw = lds_fill_vt_count<D, BN, NW>(w);
    auto kept = [&](int it) {  // loads this wave issued in iteration it - 1 (K of it + 2, V of it)
        return (it + 2 < ntiles ? nkw : 0) + (it < ntiles ? nvw : 0);
    };

    half8 qf[KS];
    {
        const int t = min(t_lane, T - 1), hh = R - t_lane * G;
        const TI* qrow = (const TI*)a.q + (((size_t)b * T + t) * a.Hq + hkv * G + hh) * D;
        float qmul = a.qscale;
        if (a.qkn.on && rvalid) qmul *= qk_factor(row_sumsq(qrow, D), D, a.qkn.gain, a.qkn.eps);
        load_q_frags<TI, OP, D>(qf, qrow, rope ? a.table + (size_t)t * (D / 2) : nullptr, qmul, h, rvalid, a.half);
    }
    wait_all();
    fill_k(j0, 0);
    if (ntiles > j0 + 1) fill_k(j0 + 1, 1);
    lds_fill_wait_keep(ntiles > j0 + 1 ? nkw : 0);  // K of tile j0

    floatx16 s[2];        // scores of one tile (32 keys per accumulator)
    // fp16 probabilities of two consecutive tiles (index: tile parity counted from j0); zeros
    // until written, so the product of a wave's first active iteration adds nothing
    // (D <= 64: one buffer -- phase 1 reads all of tile j - 1's probabilities before it packs tile
    // j's, which wait in hp until then)
    half8 p[D <= 64 ? 1 : 2][4] = {};
    floatx16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = floatx16{};
    float m_run = kMFloor, l_run = 0.f, apend = 1.f;
    // The score products start from -mf (an extra k-step: fold weights x the split of -mf), so the
    // accumulators hold S - mf and the exponentials need no subtraction; mf = m_run once the row
    // has seen a key (0 before, when m_run is the floor), and a refresh rebases the current tile.
    float mf = 0.f;
    const half8 fw = fold_weights(h);
    half8 fmf = fold_frag(0.f, h);
    bool pend = false;

    // scores of the current tile from S - mf to S - m_run, and the fold to the new m_run
    auto rebase = [&]() {
        const float dl = m_run - mf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[mb][r] -= dl;
        mf = m_run > 0.5f * kMFloor ? m_run : 0.f;
        fmf = fold_frag(-mf, h);
    };
    // mask of tile j (if it crosses a diagonal or a window edge)
    auto mask = [&](int j) {
        const int n0 = j * BN;
        if (n0 + BN - 1 > wave_tmin || wave_tmax - n0 >= W) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!visible(n0 + 32 * mb + acc_row(r, h), t_lane, W)) s[mb][r] = -INFINITY;
        }
    };
    // row max of the scores in s (relative to mf)
    auto row_max = [&]() {
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        return max_halves(mx);
    };
    auto mask_max = [&](int j) {
        mask(j);
        return row_max();
    };
    // phase 2: scores of tile j, products alternating between the two 32-key accumulators
    auto phase2 = [&](int j, auto SK) {
        const OP* Ks = kst(decltype(SK)::value);
        constexpr int AH = D <= 64 ? 2 : (N2 < 4 ? N2 : 4);
        half8 fr[N2];
#pragma unroll
        for (int i = 0; i < AH; ++i) fr[i] = row_frag_sw<OP, D>(Ks, 32 * (i & 1) + c, i >> 1, h);
        s[0] = M::mma(fw, fmf, floatx16{});
        s[1] = s[0];
#pragma unroll
        for (int i = 0; i < N2; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            s[i & 1] = M::mma(fr[i], qf[i >> 1], s[i & 1]);
            if (i + AH < N2) fr[i + AH] = row_frag_sw<OP, D>(Ks, 32 * ((i + AH) & 1) + c, (i + AH) >> 1, h);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // phase 1 of iteration j: O^T += V^T P^T for tile j - 1 (when PV) and the probabilities of
    // tile j (parity C), whose sum is returned; the 32 exponentials are spread over the products
    auto phase1 = [&](int j, auto PAR, auto PV, auto SV) -> float {
        constexpr int C = D <= 64 ? 0 : decltype(PAR)::value, NP = D <= 64 ? 0 : C ^ 1;
        constexpr bool DO_PV = decltype(PV)::value;
        constexpr int NS = DO_PV ? N1 : 1;              // issue slots
        constexpr int AH = D <= 64 ? 2 : (N1 < 4 ? N1 : 4);
        const OP* Vs = vst(decltype(SV)::value);
        auto rd = [&](int i) { return vt_frag<BN>(Vs, 32 * (i % NDB) + c, i / NDB, h); };
        half8 fr[N1];
        half2v hp[16];
        float ps = 0.f;
        if constexpr (DO_PV) {
#pragma unroll
            for (int i = 0; i < AH; ++i) fr[i] = rd(i);
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (DO_PV) {
                oacc[i % NDB] = M::mma(fr[i], p[NP][i / NDB], oacc[i % NDB]);
                if (i + AH < N1) fr[i + AH] = rd(i + AH);
            }
#pragma unroll
            for (int e = 32 * i / NS; e < 32 * (i + 1) / NS; ++e) {
                const float x = __builtin_amdgcn_exp2f(s[e >> 4][e & 15]);
                if (e & 1) {
                    hp[e >> 1][1] = (_Float16)x;
                    ps = __builtin_amdgcn_fdot2(hp[e >> 1], half2v{1, 1}, ps, false);
                    asm volatile("" ::"v"(hp[e >> 1]), "v"(ps));  // keep this slot's share here
                } else {
                    hp[e >> 1][0] = (_Float16)x;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            p[C][kk] = half8{hp[4 * kk][0], hp[4 * kk][1], hp[4 * kk + 1][0], hp[4 * kk + 1][1],
                             hp[4 * kk + 2][0], hp[4 * kk + 2][1], hp[4 * kk + 3][0], hp[4 * kk + 3][1]};
        return ps;
    };
    // after the scores of tile j are in s: the mask and, while a row of the wave has not seen a key
    // (m at the floor), the max and the refresh of m.  Once every row has its m, the scores are not
    // scanned: a tile whose probabilities exceed the fp16 range (a score 16 or more above m, rare) is
    // caught by its row sum in phase 1 and redone there (overflow below)
    auto refresh = [&](int j) {
        mask(j);
        if (__builtin_amdgcn_ballot_w64(m_run <= 0.5f * kMFloor) == 0) return;
        const float mx = row_max();
        if (__builtin_amdgcn_ballot_w64(mf + mx > m_run + TAU) != 0) {  // raise m to this tile's max
            const float m_new = fmaxf(m_run, mf + mx);
            apend = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            rebase();
            l_run *= apend;
            pend = true;
        }
    };
    auto sync_fill = [&](int it, auto S) {
        // K of tile it + 1 and V of tile it - 1 have landed (K of it + 2 and V of it may still be
        // in flight); every wave is done with the stages the new loads overwrite (K of tile it,
        // V of tile it - 2); S = stage of tile it
        constexpr int s = decltype(S)::value;
        lds_fill_wait_keep(kept(it));
        if (it + 3 < ntiles) fill_k(it + 3, s);
        if (it + 1 < ntiles) fill_v(it + 1, (s + 1) % NST);
    };
    // A wave starts at its own first tile: the iterations before it are skipped, the one just
    // before it exponentiates scores that are all -inf (p = 0, with m_run still at the floor).
    auto step = [&](int it, auto PAR, auto S) {
        constexpr int s = decltype(S)::value;
        sync_fill(it, S);
        if (it >= first - 1 && it <= last + 1) {
            float ps = phase1(it, PAR, IC<1>{}, IC<(s + 2) % NST>{});
            if (it <= last && __builtin_amdgcn_ballot_w64(!(ps < INFINITY)) != 0) {
                // overflow: a probability of tile it exceeded fp16.  O (tiles up to it - 1, just
                // completed) and l use the old m: raise m to this tile's max, rescale both, redo the
                // probabilities of tile it
                const float m_new = fmaxf(m_run, mf + row_max());
                const float al = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                rebase();
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= al;
                l_run *= al;
                ps = phase1(it, PAR, IC<0>{}, IC<(s + 2) % NST>{});
            }
            l_run += it <= last ? ps : 0.f;  // iteration last + 1 only finishes the product
            if (it + 1 <= last) phase2(it + 1, IC<(s + 1) % NST>{});
            if (pend) {  // O now holds every tile whose probabilities used the old m
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= apend;
                pend = false;
            }
            if (it + 1 <= last) refresh(it + 1);
        }
    };

    // iteration j0 - 1: the scores of tile j0 fix the first m exactly for the rows that see it
    // (without a window, every row); the others keep the floor until their first tile
    if (ntiles > j0 + 2) fill_k(j0 + 2, 2);
    fill_v(j0, 0);
    if (last >= 0) {
        phase2(j0, IC<0>{});
        m_run = fmaxf(mask_max(j0), kMFloor);
        rebase();
    }
    // iteration j0: no product yet
    sync_fill(j0, IC<0>{});
    if (last >= 0) {
        l_run = phase1(j0, IC<0>{}, IC<0>{}, IC<0>{});
        if (last >= j0 + 1) {
            phase2(j0 + 1, IC<1>{});
            refresh(j0 + 1);
        }
    }
    // iterations j0 + 1 .. ntiles, run by every wave (the barriers are block-wide); the parity of
    // the probability buffers counts from j0
    // unrolled by six: probability parity (it - j0) % 2 and ring stage (it - j0) % 3
    for (int it = j0 + 1; it <= ntiles; it += 6) {
        step(it, IC<1>{}, IC<1>{});
        if (it + 1 > ntiles) break;
        step(it + 1, IC<0>{}, IC<2>{});
        if (it + 2 > ntiles) break;
        step(it + 2, IC<1>{}, IC<0>{});
        if (it + 3 > ntiles) break;
        step(it + 3, IC<0>{}, IC<1>{});
        if (it + 4 > ntiles) break;
        step(it + 4, IC<1>{}, IC<2>{});
        if (it + 5 > ntiles) break;
        step(it + 5, IC<0>{}, IC<0>{});
    }

    float l_tot = sum_halves(l_run);
    if (SPLIT && job.np > 1) {
        // split block: the pieces before the last leave m, l and O (unnormalised, relative to m)
        // in their slot; the last combines all pieces in piece order and writes the output
        __shared__ unsigned sh[2];
        constexpr int NF = NDB * 16;                       // O floats per lane
        const size_t sb = (size_t)job.grp * (a.nrb - sp.rs) + (rb - sp.rs);
        unsigned* cnt = sp.cnt + 2 * sb;
        float* slots = sp.part + sb * job.np * (size_t)(NW * 64 * (NF + 2));
        auto o_at = [&](int p) { return slots + (size_t)p * (NW * 64 * (NF + 2)) + (size_t)w * 64 * NF; };
        auto ml_at = [&](int p) { return slots + (size_t)p * (NW * 64 * (NF + 2)) + (size_t)NW * 64 * NF + (w * 64 + l) * 2; };
        const unsigned ord = split_arrive(cnt, sh);
        if ((int)ord + 1 < job.np) {
            float* op = o_at(job.piece);
#pragma unroll
            for (int i = 0; i < NF / 4; ++i)
                *reinterpret_cast<floatx4*>(op + (i * 64 + l) * 4) =
                    floatx4{oacc[i / 4][4 * (i % 4)], oacc[i / 4][4 * (i % 4) + 1], oacc[i / 4][4 * (i % 4) + 2],
                            oacc[i / 4][4 * (i % 4) + 3]};
            *reinterpret_cast<float2*>(ml_at(job.piece)) = make_float2(m_run, l_tot);
            split_publish(cnt);
            return;
        }
        const bool ok = split_collect(cnt, (unsigned)job.np - 1, sh);
        // (the same operations in the same order whichever piece is last: deterministic)
        float mp[4], lp[4];
        float mx = m_run;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (p >= job.np) break;
            if (p == job.piece) { mp[p] = m_run; lp[p] = l_tot; continue; }
            const float2 ml = *reinterpret_cast<const float2*>(ml_at(p));
            mp[p] = ml.x; lp[p] = ml.y;
            mx = fmaxf(mx, ml.x);
        }
        floatx16 acc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};
        float lsum = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (p >= job.np) break;
            const float f = __builtin_amdgcn_exp2f(mp[p] - mx);
            lsum = __builtin_fmaf(lp[p], f, lsum);
            if (p == job.piece) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] = __builtin_fmaf(oacc[db][r], f, acc[db][r]);
            } else {
                const float* op = o_at(p);
#pragma unroll
                for (int i = 0; i < NF / 4; ++i) {
                    const floatx4 x = *reinterpret_cast<const floatx4*>(op + (i * 64 + l) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i / 4][4 * (i % 4) + e] = __builtin_fmaf(x[e], f, acc[i / 4][4 * (i % 4) + e]);
                }
            }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = acc[db];
        m_run = mx;
        l_tot = ok ? lsum : __builtin_nanf("");
    }
    const float inv = 1.f / l_tot;
    if (rvalid && h == 0) {
        const int t = t_lane, hq = hkv * G + (R - t * G);
        a.lse[((size_t)b * a.Hq + hq) * T + t] = (m_run + __log2f(l_tot)) * kLn2;
    }
    // o rows through LDS, waves 0-3 then 4-7: the last iteration waited for every load; the
    // first barrier makes sure no wave still reads a stage
    auto out = [&]() {
        store_rows<TOUT, D>(oacc, inv, lds_raw + (w & 3) * 32 * D * (int)sizeof(TOUT), [&](int i) {
            const int Ri = Rw + i;
            if (Ri >= TG) return (TOUT*)nullptr;
            const int t = Ri / G;
            return (TOUT*)a.o + (((size_t)b * T + t) * a.Hq + hkv * G + (Ri - t * G)) * D;
        });
    };
    __syncthreads();
    if (w < 4) out();
    __syncthreads();
    if (w >= 4) out();
}

// =====================================================================================
// Backward, dK/dV.  One workgroup = 8 waves owns a pair of 64-key blocks of one KV head, the
// block kb and its mirror nkb - 1 - kb, processed one after the other, so every workgroup has
// the same causal work.  grid (ceil(nkb / 2) * B * Hkv), nkb = ceil(T / 64).
//   wave w: row half rh = w & 1 of each 64-row tile, 32-key sub-block kq = (w >> 1) & 1,
//   role = w >> 2:
//     role 0: S = Q K^T, P = exp2(S - lse2) (masked), dV^T += dO^T P;
//     role 1: dP = dO V^T, dS = P (dP - Delta), dK^T += Q^T dS,
//   P passes from the role-0 wave to the role-1 wave of the same row half through LDS (both
//   waves hold the same (key, row) in the same lane and register).  S and dP put one key per
//   lane and 16 rows per lane half, so P and dS feed the dV / dK products directly as
//   contraction operands; dO^T and Q^T come from transposed reads of the swizzled row-major
//   tiles.  Every flattened row of the group (all G query heads) passes through the same
//   accumulators, so dK and dV are summed over the query-head group in registers; the two row
//   halves are added in a fixed order through LDS at the end of a key block and written once.
// =====================================================================================
template <typename OP, int D, typename TOUT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void dkdv_kernel(BwdArgs a) {
    using M = Mma<OP>;
    constexpr bool F16 = sizeof(OP) == 2;
    constexpr int KSUB = 2, BN = 32 * KSUB, BMR = 64, NW = 8, NST = F16 ? 3 : 2;  // ring of row tiles
    constexpr int KS = D / M::K;
    constexpr int NDB = D / 32;
    constexpr int TILE = BMR * D;
    static_assert(NST * 2 * TILE * sizeof(OP) >= KSUB * 2 * NDB * 16 * 64 * sizeof(float),
                  "staging area holds the partials");
    __shared__ __attribute__((aligned(1024))) OP lds[NST * 2 * TILE];
    __shared__ __attribute__((aligned(16))) float pbuf[KSUB][2][4][64][4];  // [kq][row half][r/4][lane][r%4]
    __shared__ __attribute__((aligned(16))) float rowv[NST][2][BMR];   // [stage][lse2 | delta][row]

    const int T = a.T, G = a.G, TG = T * G;
    const int nkb = (T + BN - 1) / BN;
    const int npair = (nkb + 1) / 2;
    const Work wk = map_block(npair, a.B * a.Hkv, false);
    const int hkv = wk.grp % a.Hkv, b = wk.grp / a.Hkv;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    // waves w and w + 4 (one per role, same row half and key sub-block) share a SIMD, so the
    // exp/VALU phase of one overlaps the MFMA phase of the other
    const int rh = w & 1, kq = (w >> 1) & 1, role = w >> 2;
    const int per_fill = 2 * lds_fill_count<OP, D, BMR, NW>(w) + (w < 2 ? 1 : 0);  // loads per fill

    const size_t grp = (size_t)wk.grp;
    const OP* qg = (const OP*)a.qh + grp * (size_t)TG * D;
    const OP* og = (const OP*)a.dOh + grp * (size_t)TG * D;
    const OP* kg = (const OP*)a.kh + grp * (size_t)T * D;
    const OP* vg = (const OP*)a.vh + grp * (size_t)T * D;
    const float* lse2g = a.lse2 + grp * (size_t)TG;
    const float* delg = a.delta + grp * (size_t)TG;
    const bool rope = a.rope_base > 0.0;

    // Q and dO rows, lse2 (wave 0) and Delta (wave 1) of rows [R0, R0 + 64), all by direct loads;
    // rows past TG are copies of row TG - 1 and are masked out (P = 0) below.
    auto fill = [&](int stage, int R0) {
        OP* dst = lds + stage * 2 * TILE;
        lds_fill<OP, D, BMR, NW>(dst, qg, R0, TG);
        lds_fill<OP, D, BMR, NW>(dst + TILE, og, R0, TG);
        if (w < 2) {
            const float* src = (w == 0 ? lse2g : delg) + min(R0 + l, TG - 1);
            dma4(src, lds_addr(&rowv[stage][w][0]));
        }
    };

    for (int pass = 0; pass < 2; ++pass) {
        const int kb = pass == 0 ? wk.blk : nkb - 1 - wk.blk;
        if (pass == 1 && kb == wk.blk) break;  // odd nkb: the middle block has no mirror
        const int n0 = kb * BN + 32 * kq;                      // first key of this wave
        const int key = n0 + c;
        const bool kvalid = key < T;
        // flattened row R (position R / G) sees this key iff keyG <= R < keyWG
        const int W = a.window;
        const int keyG = key * G;
        const int keyWG = (T - key <= W ? T : key + W) * G;
        const int rstart = (kb * BN * G) / BMR * BMR;
        const int kl = kb * BN + BN - 1;                                 // the block's last key
        const int rend = (T - kl <= W ? T : kl + W) * G;                 // rows past it see none
        const int ntiles = (rend - rstart + BMR - 1) / BMR;
        const int wlim = (T - (n0 + 31) <= W ? T : n0 + 31 + W) * G;    // rows from wlim see none
        const int wedge = (T - n0 <= W ? T : n0 + W) * G;                // of this wave's keys, from
                                                                         // wedge some are hidden

        // role 0 keeps K^T fragments, role 1 keeps V^T fragments (B operands, one key per lane)
        typename M::frag kvf[KS];
        const OP* kvrow = (role == 0 ? kg : vg) + (size_t)key * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kvf[ks] = kvalid ? M::row_frag(kvrow, ks, h, D) : typename M::frag{};
        floatx16 acc[NDB];  // role 0: dV^T, role 1: dK^T (d rows, this lane's key column)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};
        wait_all();

#pragma unroll
        for (int s0 = 0; s0 < NST - 1; ++s0)
            if (s0 < ntiles) fill(s0, rstart + s0 * BMR);
        // tile it, with its ring stage st = it % NST known at compile time (LDS offsets are constants)
        auto tile = [&](int it, auto ST) {
            constexpr int st = decltype(ST)::value;
            const OP* Qs = lds + st * 2 * TILE;
            const OP* Os = Qs + TILE;
            const int R0 = rstart + it * BMR;
            // barrier 1: tile it is in LDS (the fills of the younger tiles may still be in flight)
            lds_fill_wait_keep(per_fill * min(NST - 2, ntiles - 1 - it));
            if (it + NST - 1 < ntiles) fill((st + NST - 1) % NST, R0 + (NST - 1) * BMR);
            const int Rh = R0 + 32 * rh;                       // first row of this wave's half
            const bool active = min(Rh + 31, TG - 1) >= n0 * G && Rh < wlim;
            const bool need_mask = Rh < (n0 + 31) * G || Rh + 32 > wedge;
            floatx16 x;                                        // role 0: S -> P, role 1: dP
            if constexpr (F16) {
                // every LDS fragment of this tile first (one round trip), then the products
                half8 af[KS], tf[2][NDB];
                if (active) {
                    const OP* rows = role == 0 ? Qs : Os;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) af[ks] = row_frag_sw<OP, D>(rows, 32 * rh + c, ks, h);
                    const _Float16* trt = (const _Float16*)(role == 0 ? Os : Qs);
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                        for (int db = 0; db < NDB; ++db) tf[cc][db] = tr_frag_f16_sw<D>(trt, 2 * rh + cc, 32 * db);
                    x = M::mma(af[0], kvf[0], floatx16{});
#pragma unroll
                    for (int ks = 1; ks < KS; ++ks) x = M::mma(af[ks], kvf[ks], x);
                    if (role == 0) {
                        if (need_mask) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int row = Rh + acc_row(r, h);
                                if (row < keyG || row >= keyWG) x[r] = -INFINITY;
                            }
                        }
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const int rr = 32 * rh + 8 * q4 + 4 * h;
                            const floatx4 Lv = *reinterpret_cast<const floatx4*>(&rowv[st][0][rr]);
                            floatx4 pv;
#pragma unroll
                            for (int e = 0; e < 4; ++e) pv[e] = x[4 * q4 + e] = __builtin_amdgcn_exp2f(x[4 * q4 + e] - Lv[e]);
                            *reinterpret_cast<floatx4*>(&pbuf[kq][rh][q4][l][0]) = pv;
                        }
                    }
                }
                __syncthreads();                               // barrier 2: P of this tile shared
                if (active) {
                    floatx16 src;                              // role 0: P, role 1: dS
                    if (role == 0) {
                        src = x;
                    } else {
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const int rr = 32 * rh + 8 * q4 + 4 * h;
                            const floatx4 Dv = *reinterpret_cast<const floatx4*>(&rowv[st][1][rr]);
                            const floatx4 pv = *reinterpret_cast<const floatx4*>(&pbuf[kq][rh][q4][l][0]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) src[4 * q4 + e] = pv[e] * (x[4 * q4 + e] - Dv[e]);
                        }
                    }
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const half8 f = pack_frag_f16(src, cc);
#pragma unroll
                        for (int db = 0; db < NDB; ++db) acc[db] = M::mma(tf[cc][db], f, acc[db]);
                    }
                }
            } else {
                x = floatx16{};
                if (active) {
                    const OP* rows = role == 0 ? Qs : Os;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) x = M::mma(row_frag_sw<OP, D>(rows, 32 * rh + c, ks, h), kvf[ks], x);
                    if (role == 0) {
                        if (need_mask) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int row = Rh + acc_row(r, h);
                                if (row < keyG || row >= keyWG) x[r] = -INFINITY;
                            }
                        }
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const int rr = 32 * rh + 8 * q4 + 4 * h;
                            const floatx4 Lv = *reinterpret_cast<const floatx4*>(&rowv[st][0][rr]);
                            floatx4 pv;
#pragma unroll
                            for (int e = 0; e < 4; ++e) pv[e] = x[4 * q4 + e] = __builtin_amdgcn_exp2f(x[4 * q4 + e] - Lv[e]);
                            *reinterpret_cast<floatx4*>(&pbuf[kq][rh][q4][l][0]) = pv;
                        }
                    }
                }
                __syncthreads();                               // barrier 2: P of this tile shared
                if (active) {
                    floatx16 src;
                    if (role == 0) {
                        src = x;
                    } else {
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const int rr = 32 * rh + 8 * q4 + 4 * h;
                            const floatx4 Dv = *reinterpret_cast<const floatx4*>(&rowv[st][1][rr]);
                            const floatx4 pv = *reinterpret_cast<const floatx4*>(&pbuf[kq][rh][q4][l][0]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) src[4 * q4 + e] = pv[e] * (x[4 * q4 + e] - Dv[e]);
                        }
                    }
                    const float* trt = (const float*)(role == 0 ? Os : Qs);
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int s2 = 0; s2 < 16; ++s2)
                            acc[db] = M::mma(tr_frag_f32_sw<D>(trt, rh, s2, 32 * db), src[s2], acc[db]);
                }
            }
        };
        for (int it0 = 0; it0 < ntiles; it0 += NST) {
            tile(it0, IC<0>{});
            if (it0 + 1 >= ntiles) break;
            tile(it0 + 1, IC<1>{});
            if constexpr (NST == 3) {
                if (it0 + 2 >= ntiles) break;
                tile(it0 + 2, IC<2>{});
            }
        }

        // add the two row halves in a fixed order (half 0 + half 1) through the staging area
        __syncthreads();
        float* part = reinterpret_cast<float*>(lds) + (kq * 2 + role) * (NDB * 16 * 64);
        if (rh == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<floatx4*>(&part[((db * 4 + q4) * 64 + l) * 4]) =
                        floatx4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
        }
        __syncthreads();
        if (rh == 0 && kvalid) {  // both lanes of a key pair (c, c + 32) agree
            const size_t koff = (((size_t)b * T + key) * a.Hkv + hkv) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const floatx4 o1 = *reinterpret_cast<const floatx4*>(&part[((db * 4 + q4) * 64 + l) * 4]);
                    const int d = 32 * db + 8 * q4 + 4 * h;
                    float x0 = acc[db][4 * q4] + o1[0], x1 = acc[db][4 * q4 + 1] + o1[1];
                    float x2 = acc[db][4 * q4 + 2] + o1[2], x3 = acc[db][4 * q4 + 3] + o1[3];
                    if (role == 1) {
                        // dk' = ln2 * sum dS q~ (q~ carries scale * log2 e), then dk = R^T dk'
                        x0 *= kLn2; x1 *= kLn2; x2 *= kLn2; x3 *= kLn2;
                        if (rope) {
                            const float2 r0 = a.table[(size_t)key * (D / 2) + d / 2];
                            const float2 r1 = a.table[(size_t)key * (D / 2) + d / 2 + 1];
                            const float y0 = x0 * r0.x + x1 * r0.y, y1 = -x0 * r0.y + x1 * r0.x;
                            const float y2 = x2 * r1.x + x3 * r1.y, y3 = -x2 * r1.y + x3 * r1.x;
                            x0 = y0; x1 = y1; x2 = y2; x3 = y3;
                        }
                    }
                    acc[db][4 * q4] = x0; acc[db][4 * q4 + 1] = x1; acc[db][4 * q4 + 2] = x2; acc[db][4 * q4 + 3] = x3;
                }
            if (role == 1 && a.qkn.on) qk_norm_bwd_row<NDB>(acc, a.k, koff, a.in_dt, a.rk[grp * (size_t)T + key], a.qkn.gain, h);
            TOUT* orow = (TOUT*)(role == 0 ? a.dv : a.dk) + koff;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    store4(orow + 32 * db + 8 * q4 + 4 * h, acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2],
                           acc[db][4 * q4 + 3]);
        }
        __syncthreads();  // the staging area is refilled by the next key block
    }
}


// =====================================================================================
// Backward dK/dV, 16-bit operands.  Same work split as dkdv_kernel (8 waves: row half, 32-key
// sub-block, role; mirrored 64-key block pairs), but the two roles work one row tile apart, so
// a step needs one barrier: at step s the role-0 wave adds dO^T P of tile s - 1 to dV^T (P kept
// in registers since the previous step), then computes S and P of tile s and hands P to its role-1
// partner through an LDS buffer of step parity s & 1 -- its exponentials come last, while the
// partner runs products -- and the role-1 wave computes dP of tile s - 1, dS with the P handed
// over one step earlier and adds Q^T dS to dK^T.  The shifts by lse2 and by Delta ride on one extra k-step of the S and dP
// products: the A operand carries three fp16 terms of -lse2 (or -Delta) of the lane's row
// (fold_frag) against B = (256, 1, 1), so the accumulators come out as S - lse2 and
// dP - Delta with fp32 accuracy and no per-element subtraction.  Row tiles go through a 4-stage
// ring filled two steps ahead.  SPLIT: a host plan replaces the pairs with single key blocks,
// longest first, or with pieces of a key block's row tiles whose sums the last piece combines.
// =====================================================================================
// MODE 0: dQ is a separate pass; 1: also store dS for the dQ pass (DS); 2: atomic dQ (AT) -- the
// role-1 waves leave dS^T of each tile in LDS, and one step later the role-0 waves multiply it by
// the key block's K' (kept in LDS) and add dQ of their 32 rows x D/2 columns into an fp32
// accumulator with atomic adds (not bit-reproducible: the order of the adds varies).  With AT the
// row-tile ring has three stages filled one step ahead, to leave LDS for K' and dS^T.
// W4: head_dim <= 64, the plain-causal design under a plan (single key blocks or pieces): two
// workgroups per CU (four waves per SIMD, 128 VGPRs), a 3-stage ring filled one tile ahead and
// operands read two products ahead, which fits without spills; at D = 64 a 64-row step carries
// half the products of D = 128 for the same chain of dependent steps, so the second workgroup's
// waves are what hides it (the 12-head, 1024-token MHA layer: dK/dV 134 -> 92 us).
template <int D, int MODE, bool SPLIT>
struct DkdvShape {
    static constexpr bool W4 = D <= 64 && MODE == 0 && SPLIT;
};
template <int D, typename TOUT, int MODE, bool SPLIT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(DkdvShape<D, MODE, SPLIT>::W4 ? 4 : 2)))
void dkdv_kernel_h(BwdArgs a, SplitPlan sp) {
    using OP = _Float16;
    using M = Mma<OP>;
    constexpr bool DS = MODE == 1, AT = MODE == 2, W4 = DkdvShape<D, MODE, SPLIT>::W4;
    constexpr int KSUB = 2, BN = 32 * KSUB, BMR = 64, NW = 8, NST = AT || W4 ? 3 : 4, AHEAD = AT || W4 ? 1 : 2;
    constexpr int KS = D / 16, NDB = D / 32, TILE = BMR * D;
    // AT: the D / 32 column blocks of dQ split between the two key sub-block waves of a row half
    constexpr int NDQ = NDB >= 2 ? NDB / 2 : 1, NATOM = 16 * NDQ;
    static_assert(NST * 2 * TILE * sizeof(OP) >= KSUB * 2 * NDB * 16 * 64 * sizeof(float),
                  "the ring holds the partials of the final reduction");
    __shared__ __attribute__((aligned(1024))) OP lds[NST * 2 * TILE];     // [stage][Q~ | dO'] row tiles
    __shared__ __attribute__((aligned(16))) half8 pbuf[2][KSUB][2][2][64];  // [s & 1][kq][rh][cc][lane]
    __shared__ __attribute__((aligned(16))) float rowv[NST][2][BMR];       // [stage][lse2 | delta][row]
    __shared__ __attribute__((aligned(1024))) OP ktile[AT ? BN * D : 8];   // AT: K' of the key block
    __shared__ __attribute__((aligned(1024))) OP dstile[AT ? 2 * BN * BMR : 8];  // AT: [s & 1] dS^T [key][row]

    const int T = a.T, G = a.G, TG = T * G;
    const int nkb = (T + BN - 1) / BN;
    const int npair = (nkb + 1) / 2;
    // the job: a mirrored pair of key blocks (wk.blk and nkb - 1 - wk.blk), or, under a split
    // plan, one key block (wk.blk) or piece `piece` of its row tiles
    Work wk;
    int piece = 0, np = 1, jrb = 0;
    if constexpr (SPLIT) {
        wk = map_block(sp.njobs, a.ngrp, false);
        const unsigned e = sp.job[wk.blk];
        jrb = (int)(e >> 2);
        piece = (int)(e & 3u);
        np = jrb >= sp.rs ? sp.np : 1;
        wk.blk = nkb - 1 - jrb;
    } else {
        wk = map_block(npair, a.ngrp, false);
    }
    const int gg = a.grp0 + wk.grp;                   // the (batch, KV head) group
    const int hkv = gg % a.Hkv, b = gg / a.Hkv;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    // waves w and w + 4 (same row half and key sub-block, the two roles) share a SIMD
    const int rh = w & 1, kq = (w >> 1) & 1, role = w >> 2;
    const int per_fill = 2 * lds_fill_count<OP, D, BMR, NW>(w) + (w < 2 ? 1 : 0);  // loads per fill

    const size_t grp = (size_t)gg;
    const OP* qg = (const OP*)a.qh + grp * (size_t)TG * D;
    const OP* og = (const OP*)a.dOh + grp * (size_t)TG * D;
    const OP* kg = (const OP*)a.kh + grp * (size_t)T * D;
    const OP* vg = (const OP*)a.vh + grp * (size_t)T * D;
    const float* lse2g = a.lse2 + grp * (size_t)TG;
    const float* delg = a.delta + grp * (size_t)TG;
    const bool rope = a.rope_base > 0.0;
    const half8 fw = fold_weights(h);
    // DS: the dS tiles of this group (ds_tile_index), 512 fragments of 16 bytes each, in 1 KiB
    // blocks (2 kq + rh) * 2 + cc written whole by one store; in a block, lane (h, c) takes slot
    // 32 h + (c ^ (4 h + 8 cc)), which keeps the dQ pass's transposed reads free of bank conflicts
    half8* dsg = nullptr;
    int ds0 = 0, ds1 = 0;
    if constexpr (DS) {
        dsg = (half8*)a.ds + (size_t)wk.grp * ds_tiles_per_group((TG + 63) / 64, (T + 63) / 64, G) * 512 + (kq * 2 + rh) * 128;
        ds0 = 32 * h + (c ^ (4 * h));
        ds1 = 64 + 32 * h + (c ^ (4 * h + 8));
    }

    // Q and dO rows, lse2 (wave 0) and Delta (wave 1) of rows [R0, R0 + 64), all by direct loads;
    // rows past TG are copies of row TG - 1 and are masked out (P = 0) below.
    const unsigned lds0 = lds_addr(lds);
    auto fill = [&](int stage, int R0) {   // 32-bit LDS bases: no generic-pointer round trip
        const unsigned dst = lds0 + (unsigned)(stage * 2 * TILE * 2);
        lds_fill_at<OP, D, BMR, NW>(dst, qg, R0, TG);
        lds_fill_at<OP, D, BMR, NW>(dst + TILE * 2, og, R0, TG);
        if (w < 2) {
            const float* src = (w == 0 ? lse2g : delg) + min(R0 + l, TG - 1);
            dma4(src, lds_addr(&rowv[stage][w][0]));
        }
    };

    half8 kvf[KS];  // role 0: K^T fragments, role 1: V^T fragments (B operands, one key per lane)
    // x = rows(this wave's half of `rows`) . kvf over D, the row fragments read four products ahead
    // (KT: the key fragments from the block's K' tile in LDS instead of kvf -- role 0 with AT, whose
    // registers the dQ product needs)
    auto chain = [&](const OP* rows, auto KT) {
        constexpr bool FROM_TILE = decltype(KT)::value;
        constexpr int AH = W4 || MODE == 0 ? (KS < 2 ? KS : 2) : (KS < 4 ? KS : 4);
        half8 fr[KS];
#pragma unroll
        for (int i = 0; i < AH; ++i) fr[i] = row_frag_sw<OP, D>(rows, 32 * rh + c, i, h);
        floatx16 x = floatx16{};
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (FROM_TILE) x = M::mma(fr[i], row_frag_sw<OP, D>(ktile, 32 * kq + c, i, h), x);
            else x = M::mma(fr[i], kvf[i], x);
            if (i + AH < KS) fr[i + AH] = row_frag_sw<OP, D>(rows, 32 * rh + c, i + AH, h);
        }
        __builtin_amdgcn_sched_barrier(0);
        return x;
    };
    // second product of a step: acc[db] += trt^T (this wave's rows, transposed reads) . pf; the
    // fragments of the first k-step were read before the exponentials (tf0), those of the second
    // are read while the first k-step's products run
    auto tr_frags0 = [&](const OP* trt, half8 (&tf0)[NDB]) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) tf0[db] = tr_frag_f16_sw<D>((const _Float16*)trt, 2 * rh, 32 * db);
    };
    auto product2 = [&](const OP* trt, const half8 (&tf0)[NDB], const half8 (&pf)[2], floatx16 (&acc)[NDB]) {
        half8 tf1[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            __builtin_amdgcn_sched_barrier(0);
            acc[db] = M::mma(tf0[db], pf[0], acc[db]);
            tf1[db] = tr_frag_f16_sw<D>((const _Float16*)trt, 2 * rh + 1, 32 * db);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            __builtin_amdgcn_sched_barrier(0);
            acc[db] = M::mma(tf1[db], pf[1], acc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    for (int pass = 0; pass < 2; ++pass) {
        const int kb = pass == 0 ? wk.blk : nkb - 1 - wk.blk;
        if (pass == 1 && (kb == wk.blk || SPLIT)) break;  // odd nkb: the middle block has no mirror
        const int n0 = kb * BN + 32 * kq;                      // first key of this wave
        const int key = n0 + c;
        const bool kvalid = key < T;
        // flattened row R (position R / G) sees this key iff keyG <= R < keyWG
        const int W = a.window;
        const int keyG = key * G;
        const int keyWG = (T - key <= W ? T : key + W) * G;
        const int kl = kb * BN + BN - 1;                                 // the block's last key
        const int rend = (T - kl <= W ? T : kl + W) * G;                 // rows past it see none
        const int r0 = (kb * BN * G) / BMR * BMR;
        const int nt0 = (rend - r0 + BMR - 1) / BMR;
        // this job's row tiles: all of them, or piece `piece` of np
        const int rstart = r0 + nt0 * piece / np * BMR;
        const int ntiles = nt0 * (piece + 1) / np - nt0 * piece / np;
        // DS: tile s of this key block (row tile kb G + s) is stored at index dsb + s
        const size_t dsb = DS ? ds_tile_index(kb, kb * G, (TG + 63) / 64, G) : 0;
        const int wlim = (T - (n0 + 31) <= W ? T : n0 + 31 + W) * G;    // rows from wlim see none
        const int wedge = (T - n0 <= W ? T : n0 + W) * G;                // of this wave's keys, from
                                                                         // wedge some are hidden
        // does this wave's row half of tile j see any of its keys, and does it need the mask
        auto active = [&](int j) {
            const int Rh = rstart + j * BMR + 32 * rh;
            return min(Rh + 31, TG - 1) >= n0 * G && Rh < wlim;
        };
        auto needs_mask = [&](int j) {
            const int Rh = rstart + j * BMR + 32 * rh;
            return Rh < (n0 + 31) * G || Rh + 32 > wedge;
        };

        const OP* kvrow = (role == 0 ? kg : vg) + (size_t)key * D;
        if ((DS || AT) && role == 1) {  // fp16(v) straight from the input: no v' copy on these paths
            const size_t voff = (((size_t)b * T + min(key, T - 1)) * a.Hkv + hkv) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kvf[ks] = kvalid ? load8_f16(a.v, voff + 16 * ks + 8 * h, a.in_dt) : half8{};
        } else if (!AT) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kvf[ks] = kvalid ? M::row_frag(kvrow, ks, h, D) : half8{};
        }
        floatx16 acc[NDB];  // role 0: dV^T, role 1: dK^T (d rows, this lane's key column)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};
        wait_all();

        if constexpr (AT) lds_fill_at<OP, D, BN, NW>(lds_addr(ktile), kg, kb * BN, T);
        fill(0, rstart);
        if (AHEAD == 2 && ntiles > 1) fill(1, rstart + BMR);
        // AT: rows of this wave's half of tile j see a key of sub-block kq_
        auto active_kq = [&](int j, int kq_) {
            const int m0 = kb * BN + 32 * kq_;
            const int lim = (T - (m0 + 31) <= W ? T : m0 + 31 + W) * G;
            const int Rh = rstart + j * BMR + 32 * rh;
            return min(Rh + 31, TG - 1) >= m0 * G && Rh < lim;
        };
        // The step loop is instantiated once per role (each wave runs one copy; both copies reach
        // the same barriers), so each role's registers are allocated for its own work only.
        auto steps = [&](auto ROLE) {
        constexpr int RL = decltype(ROLE)::value;
        int natom = 0;  // AT: atomic adds this wave issued after its share of the latest fill
        half8 pcar[2] = {};  // role 0: P of tile s, formed in step s, multiplied into dV^T in step s + 1
        // step s; in the default design with K = s % UN known at compile time (UN a multiple of the ring
        // stages and of the two P-buffer parities), so stage and parity offsets are constants (the
        // stored-dS and atomic designs, whose registers are fuller, keep one copy of the step)
        constexpr bool UNR = MODE == 0;
        constexpr int UN = !UNR ? 1 : NST == 4 ? 4 : 6;
        auto step = [&](int s, auto K) {
            constexpr int k = decltype(K)::value;
            const int S0 = UNR ? k % NST : s % NST, SM1 = UNR ? (k + UN - 1) % NST : (s + NST - 1) % NST;
            const int SA = UNR ? (k + AHEAD) % NST : (s + AHEAD) % NST;
            const int P0 = UNR ? k & 1 : s & 1, PM1 = UNR ? (k + 1) & 1 : (s + 1) & 1;
            // tile s has landed (tile s + 1 may still be in flight); the P of tile s - 1 is in
            // pbuf[PM1]; every wave is done with tile s - 2 and with pbuf[P0]
            // (with DS, role 1's two dS stores of the previous step are its most recent operations;
            // with AT, the fill is one step ahead and role 0's atomic adds of the previous step were
            // issued after it: vector memory operations complete in order)
            if constexpr (AT) lds_fill_wait_keep_atomics(natom);
            else lds_fill_wait_keep((AHEAD == 2 && s + 1 < ntiles ? per_fill : 0) + (DS && RL == 1 && s >= 2 ? 2 : 0));
            natom = 0;
            if (s + AHEAD < ntiles) fill(SA, rstart + (s + AHEAD) * BMR);
            if constexpr (RL == 0) {
                if constexpr (AT) {
                    // dQ of this wave's 32 rows of tile s - 2 (whose dS^T the role-1 waves left in
                    // dstile[s & 1]) over the block's 64 keys, columns 32 db .. + 31 for the NDQ
                    // column blocks db of this key sub-block wave; every wave issues the same
                    // number of atomic adds (rows past TG add 0 to row TG - 1), so the wait count
                    // above is exact
                    const int j = s - 2;
                    if (j >= 0 && j < ntiles && (NDB >= 2 || kq == 0) && (active_kq(j, 0) || active_kq(j, 1))) {
                        const OP* dt = dstile + P0 * (BN * BMR);
                        half8 af[4];
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) af[kk] = tr_frag_f16_sw<64>((const _Float16*)dt, kk, 32 * rh);
                        // rows past TG (their dS rows are zero) land in the next group's rows or in the
                        // 64 rows of padding after the last group: adding 0 changes nothing
                        const int Rh = rstart + j * BMR + 32 * rh;
                        float* dst = a.dq_acc + grp * (size_t)TG * D + (size_t)(Rh + 4 * h) * D + c;
#pragma unroll
                        for (int i = 0; i < NDQ; ++i) {   // one column block at a time (registers)
                            floatx16 qa = floatx16{};
#pragma unroll
                            for (int kk = 0; kk < 4; ++kk)
                                qa = M::mma(af[kk], tr_frag_f16_sw<D>((const _Float16*)ktile, kk, 32 * (kq * NDQ + i)), qa);
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * D + 32 * (kq * NDQ + i), qa[r]);
                        }
                        natom = NATOM;
                    }
                }
                // dV^T += dO^T P of tile s - 1 (P kept from the previous step), then S and P of tile s:
                // the exponentials come last, while role 1 runs its products
                if (s >= 1 && active(s - 1)) {
                    const OP* Os1 = lds + SM1 * 2 * TILE + TILE;
                    half8 tf0[NDB];
                    tr_frags0(Os1, tf0);
                    product2(Os1, tf0, pcar, acc);
                }
                if (s < ntiles && active(s)) {
                    const int st = S0;
                    const OP* Qs = lds + st * 2 * TILE;
                    const int Rh = rstart + s * BMR + 32 * rh;
                    const half8 fl = fold_frag(-rowv[st][0][32 * rh + c], h);  // ahead of the chain
                    floatx16 x = chain(Qs, IC<AT ? 1 : 0>{});
                    x = M::mma(fl, fw, x);  // S - lse2
                    if (needs_mask(s)) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int row = Rh + acc_row(r, h);
                            if (row < keyG || row >= keyWG) x[r] = -INFINITY;
                        }
                    }
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) pcar[cc][j] = (_Float16)__builtin_amdgcn_exp2f(x[8 * cc + j]);
                        pbuf[P0][kq][rh][cc][l] = pcar[cc];
                    }
                }
            } else {
                if (AT && s >= 1 && !active(s - 1)) {  // this quadrant of dS^T is zero
                    char* dt = reinterpret_cast<char*>(dstile + PM1 * (BN * BMR));
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                        for (int j4 = 0; j4 < 2; ++j4)
                            *reinterpret_cast<uint2*>(dt + Tile<_Float16, 64>::off(32 * kq + c, 32 * rh + 16 * cc + 8 * j4 + 4 * h)) =
                                uint2{0u, 0u};
                }
                if (DS && s >= 1 && !active(s - 1)) {  // a stored tile is complete: zeros here
                    __builtin_nontemporal_store(half8{}, &dsg[(dsb + s - 1) * 512 + ds0]);
                    __builtin_nontemporal_store(half8{}, &dsg[(dsb + s - 1) * 512 + ds1]);
                }
                if (s >= 1 && active(s - 1)) {
                    const int st = SM1;
                    const OP* Qs = lds + st * 2 * TILE;
                    const OP* Os = Qs + TILE;
                    const half8 fd = fold_frag(-rowv[st][1][32 * rh + c], h);  // ahead of the chain
                    floatx16 y = chain(Os, IC<0>{});
                    y = M::mma(fd, fw, y);  // dP - Delta
                    half8 tf0[NDB];
                    tr_frags0(Qs, tf0);  // in flight during dS
                    half8 dsf[2];
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const half8 pv = pbuf[PM1][kq][rh][cc][l];
#pragma unroll
                        for (int j = 0; j < 8; ++j) dsf[cc][j] = (_Float16)((float)pv[j] * y[8 * cc + j]);
                    }
                    if constexpr (DS) {
                        __builtin_nontemporal_store(dsf[0], &dsg[(dsb + s - 1) * 512 + ds0]);
                        __builtin_nontemporal_store(dsf[1], &dsg[(dsb + s - 1) * 512 + ds1]);
                    }
                    if constexpr (AT) {
                        // dS^T as [key][row] (swizzled 64 x 64 tile): lane (h, c) holds key 32 kq + c and,
                        // per k-step cc, the rows 32 rh + 16 cc + 8 (j / 4) + 4 h + j % 4
                        char* dt = reinterpret_cast<char*>(dstile + PM1 * (BN * BMR));
#pragma unroll
                        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                            for (int j4 = 0; j4 < 2; ++j4)
                                *reinterpret_cast<half4v*>(dt + Tile<_Float16, 64>::off(32 * kq + c, 32 * rh + 16 * cc + 8 * j4 + 4 * h)) =
                                    half4v{dsf[cc][4 * j4], dsf[cc][4 * j4 + 1], dsf[cc][4 * j4 + 2], dsf[cc][4 * j4 + 3]};
                    }
                    product2(Qs, tf0, dsf, acc);
                }
            }
        };
        const int send = ntiles + (AT ? 1 : 0);
        for (int s0 = 0; s0 <= send; s0 += UN) {
            step(s0, IC<0>{});
            if constexpr (UN == 1) continue;
            if (s0 + 1 > send) break;
            step(s0 + 1, IC<1>{});
            if (s0 + 2 > send) break;
            step(s0 + 2, IC<2>{});
            if (s0 + 3 > send) break;
            step(s0 + 3, IC<3>{});
            if constexpr (UN == 6) {
                if (s0 + 4 > send) break;
                step(s0 + 4, IC<4>{});
                if (s0 + 5 > send) break;
                step(s0 + 5, IC<5>{});
            }
        }
        };
        if (role == 0) steps(IC<0>{});
        else steps(IC<1>{});

        // add the two row halves in a fixed order (half 0 + half 1) through the staging area
        __syncthreads();
        float* part = reinterpret_cast<float*>(lds) + (kq * 2 + role) * (NDB * 16 * 64);
        if (rh == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<floatx4*>(&part[((db * 4 + q4) * 64 + l) * 4]) =
                        floatx4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
        }
        __syncthreads();
        if (rh == 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const floatx4 o1 = *reinterpret_cast<const floatx4*>(&part[((db * 4 + q4) * 64 + l) * 4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[db][4 * q4 + e] += o1[e];
                }
        }
        if (SPLIT && np > 1) {
            // split block: the pieces before the last leave their sums (the row-half-0 waves' dV^T
            // / dK^T) in their slot; the last adds all pieces in piece order (deterministic)
            __shared__ unsigned sh[2];
            constexpr int NF = NDB * 16;
            const size_t sb = (size_t)wk.grp * (nkb - sp.rs) + (jrb - sp.rs);
            unsigned* cnt = sp.cnt + 2 * sb;
            float* slots = sp.part + sb * np * (size_t)(4 * 64 * NF);
            auto at = [&](int p) { return slots + (size_t)p * (4 * 64 * NF) + (size_t)(w >> 1) * 64 * NF; };
            const unsigned ord = split_arrive(cnt, sh);
            if ((int)ord + 1 < np) {
                if (rh == 0) {
                    float* op = at(piece);
#pragma unroll
                    for (int i = 0; i < NF / 4; ++i)
                        *reinterpret_cast<floatx4*>(op + (i * 64 + l) * 4) =
                            floatx4{acc[i / 4][4 * (i % 4)], acc[i / 4][4 * (i % 4) + 1], acc[i / 4][4 * (i % 4) + 2],
                                    acc[i / 4][4 * (i % 4) + 3]};
                }
                split_publish(cnt);
                return;
            }
            const bool ok = split_collect(cnt, (unsigned)np - 1, sh);
            if (rh == 0) {
                floatx16 sum[NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db) sum[db] = floatx16{};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    if (p >= np) break;
                    if (p == piece) {
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
#pragma unroll
                            for (int r = 0; r < 16; ++r) sum[db][r] += acc[db][r];
                    } else {
                        const float* op = at(p);
#pragma unroll
                        for (int i = 0; i < NF / 4; ++i) {
                            const floatx4 x = *reinterpret_cast<const floatx4*>(op + (i * 64 + l) * 4);
#pragma unroll
                            for (int e = 0; e < 4; ++e) sum[i / 4][4 * (i % 4) + e] += x[e];
                        }
                    }
                }
                const float poison = ok ? 1.f : __builtin_nanf("");
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] = sum[db][r] * poison;
            }
        }
        if (rh == 0 && kvalid) {  // both lanes of a key pair (c, c + 32) agree
            const size_t koff = (((size_t)b * T + key) * a.Hkv + hkv) * D;
            const float us = a.dsc ? a.dsc[grp] : 1.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d = 32 * db + 8 * q4 + 4 * h;
                    float x0 = acc[db][4 * q4], x1 = acc[db][4 * q4 + 1];
                    float x2 = acc[db][4 * q4 + 2], x3 = acc[db][4 * q4 + 3];
                    if (role == 0) {
                        x0 *= us; x1 *= us; x2 *= us; x3 *= us;
                    } else {
                        // dk' = ln2 * sum dS q~ (q~ carries scale * log2 e), then dk = R^T dk'; both
                        // gradients carry the dO scale, undone by us
                        x0 *= kLn2 * us; x1 *= kLn2 * us; x2 *= kLn2 * us; x3 *= kLn2 * us;
                        if (rope) {
                            const float2 r0 = a.table[(size_t)key * (D / 2) + d / 2];
                            const float2 r1 = a.table[(size_t)key * (D / 2) + d / 2 + 1];
                            const float y0 = x0 * r0.x + x1 * r0.y, y1 = -x0 * r0.y + x1 * r0.x;
                            const float y2 = x2 * r1.x + x3 * r1.y, y3 = -x2 * r1.y + x3 * r1.x;
                            x0 = y0; x1 = y1; x2 = y2; x3 = y3;
                        }
                    }
                    acc[db][4 * q4] = x0; acc[db][4 * q4 + 1] = x1; acc[db][4 * q4 + 2] = x2; acc[db][4 * q4 + 3] = x3;
                }
            if (role == 1 && a.qkn.on) qk_norm_bwd_row<NDB>(acc, a.k, koff, a.in_dt, a.rk[grp * (size_t)T + key], a.qkn.gain, h);
            TOUT* orow = (TOUT*)(role == 0 ? a.dv : a.dk) + koff;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    store4(orow + 32 * db + 8 * q4 + 4 * h, acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2],
                           acc[db][4 * q4 + 3]);
        }
        __syncthreads();  // the staging area is refilled by the next key block
    }
}

// =====================================================================================
// Atomic dQ: the fp32 accumulator [group][T G][D] (flattened rows) that the dK/dV pass added into,
// scaled by softmax scale / (dO scale), rotated back (R^T), QK-norm backward, written as dq.
// grid ceil(rows D / 1024), 256 threads: D / 4 lanes per row, four consecutive columns per lane.
// =====================================================================================
template <int D, typename TOUT>
__global__ __launch_bounds__(256) void dq_acc_convert_kernel(BwdArgs a) {
    constexpr int LPR = D / 4, RPB = 256 / LPR;
    const int TG = a.T * a.G;
    const int64_t nrows = (int64_t)a.B * a.Hkv * TG;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int lane = threadIdx.x % LPR, d = 4 * lane;
    const bool valid = row < nrows;
    const int64_t rr = valid ? row : nrows - 1;
    const int grp = (int)(rr / TG), R = (int)(rr % TG);
    const int t = R / a.G, hq = (grp % a.Hkv) * a.G + R % a.G, b = grp / a.Hkv;
    const floatx4 v = *reinterpret_cast<const floatx4*>(a.dq_acc + rr * D + d);
    const float sc = a.scale * a.dsc[grp];
    float x0 = v[0] * sc, x1 = v[1] * sc, x2 = v[2] * sc, x3 = v[3] * sc;
    if (a.rope_base > 0.0) {
        const float2 r0 = a.table[(size_t)t * (D / 2) + d / 2];
        const float2 r1 = a.table[(size_t)t * (D / 2) + d / 2 + 1];
        const float y0 = x0 * r0.x + x1 * r0.y, y1 = -x0 * r0.y + x1 * r0.x;
        const float y2 = x2 * r1.x + x3 * r1.y, y3 = -x2 * r1.y + x3 * r1.x;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    const size_t qoff = (((size_t)b * a.T + t) * a.Hq + hq) * D;
    if (a.qkn.on) {  // dx = gain rho (y - x rho^2 (y . x) / D), x the raw q row
        const floatx4 xr = load4_dt(a.q, qoff + d, a.in_dt);
        const float rho = a.rq[(size_t)grp * TG + R];
        const float dot = sum_lanes(x0 * xr[0] + x1 * xr[1] + x2 * xr[2] + x3 * xr[3], LPR);
        const float c1 = a.qkn.gain * rho, c2 = rho * rho * dot / (float)D;
        x0 = c1 * (x0 - xr[0] * c2); x1 = c1 * (x1 - xr[1] * c2);
        x2 = c1 * (x2 - xr[2] * c2); x3 = c1 * (x3 - xr[3] * c2);
    }
    if (valid) store4((TOUT*)a.dq + qoff + d, x0, x1, x2, x3);
}

// =====================================================================================
// Backward, dQ (deterministic: a separate pass that recomputes S and dP, no atomics).
// grid (nrb * B * Hkv), 256 threads = 4 waves x 32 flattened rows, 64-key tiles.
// S^T = K Q^T and dP^T = V dO^T put one query row per lane; dQ^T += K^T dS^T reads K^T from the
// same swizzled K tile with transposed reads.  K and V tiles arrive by direct HBM->LDS loads.
// =====================================================================================
template <typename OP, int D, typename TOUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void dq_kernel(BwdArgs a) {
    using M = Mma<OP>;
    constexpr bool F16 = sizeof(OP) == 2;
    constexpr int BM = 128, BN = 64, NW = 4;
    constexpr int KS = D / M::K;
    constexpr int NDB = D / 32;
    constexpr int TILE = BN * D;
    __shared__ __attribute__((aligned(1024))) OP lds[2 * 2 * TILE];

    const int T = a.T, G = a.G, TG = T * G;
    const Work wk = map_block(a.nrb, a.B * a.Hkv, true);
    const int rb = wk.blk;
    const int hkv = wk.grp % a.Hkv, b = wk.grp / a.Hkv;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    const int R0 = rb * BM;
    const int Rw = R0 + 32 * w;
    const int R = Rw + c;
    const bool rvalid = R < TG;
    const int t_lane = R / G;
    const int wave_tmin = Rw / G;
    const int wave_tmax = min(Rw + 31, TG - 1) / G;
    const int ntiles = min(R0 + BM - 1, TG - 1) / G / BN + 1;
    const int W = a.window;
    const int j0 = max(0, R0 / G - W + 1) / BN;  // the block's first key tile

    const size_t grp = (size_t)wk.grp;
    const OP* qg = (const OP*)a.qh + grp * (size_t)TG * D;
    const OP* og = (const OP*)a.dOh + grp * (size_t)TG * D;
    const OP* kg = (const OP*)a.kh + grp * (size_t)T * D;
    const OP* vg = (const OP*)a.vh + grp * (size_t)T * D;

    typename M::frag qf[KS], of[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (rvalid) {
            qf[ks] = M::row_frag(qg + (size_t)R * D, ks, h, D);
            of[ks] = M::row_frag(og + (size_t)R * D, ks, h, D);
        } else {
            qf[ks] = typename M::frag{};
            of[ks] = typename M::frag{};
        }
    }
    const float L = rvalid ? a.lse2[grp * (size_t)TG + R] : INFINITY;
    const float Dl = rvalid ? a.delta[grp * (size_t)TG + R] : 0.f;
    wait_all();
    lds_fill<OP, D, BN, NW>(lds, kg, j0 * BN, T);
    lds_fill<OP, D, BN, NW>(lds + TILE, vg, j0 * BN, T);

    floatx16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = floatx16{};

    for (int it = j0; it < ntiles; ++it) {
        const OP* Ks = lds + ((it - j0) & 1) * 2 * TILE;
        const OP* Vs = Ks + TILE;
        lds_fill_wait();
        if (it + 1 < ntiles) {
            OP* nxt = lds + ((it + 1 - j0) & 1) * 2 * TILE;
            lds_fill<OP, D, BN, NW>(nxt, kg, (it + 1) * BN, T);
            lds_fill<OP, D, BN, NW>(nxt + TILE, vg, (it + 1) * BN, T);
        }
        const int n0 = it * BN;
        if (n0 > wave_tmax) continue;                 // every row of this wave precedes the tile
        if (wave_tmin - (n0 + BN - 1) >= W) continue;  // the tile is older than every row's window
        const bool need_mask = n0 + BN - 1 > wave_tmin || wave_tmax - n0 >= W;

        floatx16 ds[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            floatx16 sacc = floatx16{}, dpacc = floatx16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                sacc = M::mma(row_frag_sw<OP, D>(Ks, 32 * mb + c, ks, h), qf[ks], sacc);
                dpacc = M::mma(row_frag_sw<OP, D>(Vs, 32 * mb + c, ks, h), of[ks], dpacc);
            }
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!visible(n0 + 32 * mb + acc_row(r, h), t_lane, W)) sacc[r] = -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(sacc[r] - L);
                ds[mb][r] = pv * (dpacc[r] - Dl);
            }
        }
        if constexpr (F16) {
            half8 dsf[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) dsf[kk] = pack_frag_f16(ds[kk >> 1], kk & 1);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    dq[db] = M::mma(tr_frag_f16_sw<D>((const _Float16*)Ks, kk, 32 * db), dsf[kk], dq[db]);
        } else {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int s2 = 0; s2 < 16; ++s2)
                        dq[db] = M::mma(tr_frag_f32_sw<D>((const float*)Ks, mb, s2, 32 * db), ds[mb][s2], dq[db]);
        }
    }

    if (!rvalid) return;  // both lanes of a row pair (c, c + 32) agree
    const int t = t_lane, hh = R - t * G, hq = hkv * G + hh;
    const size_t qoff = (((size_t)b * T + t) * a.Hq + hq) * D;
    const float sc = a.scale * (a.dsc ? a.dsc[grp] : 1.f);   // the dO scale undone as well
    const bool rope = a.rope_base > 0.0;
    // dq = R^T (scale * dq'), in place
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * db + 8 * q4 + 4 * h;
            float x0 = dq[db][4 * q4] * sc, x1 = dq[db][4 * q4 + 1] * sc;
            float x2 = dq[db][4 * q4 + 2] * sc, x3 = dq[db][4 * q4 + 3] * sc;
            if (rope) {
                const float2 r0 = a.table[(size_t)t * (D / 2) + d / 2];
                const float2 r1 = a.table[(size_t)t * (D / 2) + d / 2 + 1];
                const float y0 = x0 * r0.x + x1 * r0.y, y1 = -x0 * r0.y + x1 * r0.x;
                const float y2 = x2 * r1.x + x3 * r1.y, y3 = -x2 * r1.y + x3 * r1.x;
                x0 = y0; x1 = y1; x2 = y2; x3 = y3;
            }
            dq[db][4 * q4] = x0; dq[db][4 * q4 + 1] = x1; dq[db][4 * q4 + 2] = x2; dq[db][4 * q4 + 3] = x3;
        }
    if (a.qkn.on) qk_norm_bwd_row<NDB>(dq, a.q, qoff, a.in_dt, a.rq[grp * (size_t)TG + R], a.qkn.gain, h);
    TOUT* dqrow = (TOUT*)a.dq + qoff;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            store4(dqrow + 32 * db + 8 * q4 + 4 * h, dq[db][4 * q4], dq[db][4 * q4 + 1], dq[db][4 * q4 + 2],
                   dq[db][4 * q4 + 3]);
}

// =====================================================================================
// Backward dQ, 16-bit operands.  Same work split as dq_kernel.  The shifts by lse2 and Delta
// ride on an extra k-step of the S^T and dP^T products (fold_frag: here the B operand carries
// the lane's row terms, constant for the whole kernel, against A = (256, 1, 1)), so P^T and
// dS^T cost one exponential and one multiply per element.  Per key tile the four accumulator
// chains (S^T and dP^T, two 32-key halves each) advance in turn, and every product's LDS operand
// is read four products ahead.
// =====================================================================================
// EXT: a window shorter than T (its edge is masked too) and/or the QK norm (its backward in the
// epilogue).  Without them the kernel keeps every register for the plain causal case, where the
// budget is exhausted.
// At head_dim <= 64 three workgroups share a CU (three waves per SIMD, 168 VGPRs; operands read two
// products ahead): the 12-head 1024-token MHA layer's dQ pass 56.3 -> 52.7 us.
template <int D, typename TOUT, bool EXT, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 2)))
void dq_kernel_h(BwdArgs a, SplitPlan sp) {
    using OP = _Float16;
    using M = Mma<OP>;
    constexpr int BM = 128, BN = 64, NW = 4, KS = D / 16, NDB = D / 32, TILE = BN * D;
    __shared__ __attribute__((aligned(1024))) OP lds[2 * 2 * TILE];  // [stage][K | V]

    const int T = a.T, G = a.G, TG = T * G;
    const RowJob job = map_row_job<SPLIT>(sp, a.nrb, a.B * a.Hkv);
    const int rb = job.rb;
    const int hkv = job.grp % a.Hkv, b = job.grp / a.Hkv;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    const int R0 = rb * BM;
    const int Rw = R0 + 32 * w;
    const int R = Rw + c;
    const bool rvalid = R < TG;
    const int t_lane = R / G;
    const int wave_tmin = Rw / G;
    const int wave_tmax = min(Rw + 31, TG - 1) / G;
    const int W = EXT ? a.window : T;
    // the block's key tiles [jb0, jb1); this job runs piece job.piece of them, [j0, ntiles)
    const int jb0 = EXT ? max(0, R0 / G - W + 1) / BN : 0, jb1 = min(R0 + BM - 1, TG - 1) / G / BN + 1;
    const int j0 = piece_lo(jb0, jb1, job.piece, job.np);
    const int ntiles = piece_lo(jb0, jb1, job.piece + 1, job.np);

    const size_t grp = (size_t)job.grp;
    const OP* qg = (const OP*)a.qh + grp * (size_t)TG * D;
    const OP* og = (const OP*)a.dOh + grp * (size_t)TG * D;
    const OP* kg = (const OP*)a.kh + grp * (size_t)T * D;
    const OP* vg = (const OP*)a.vh + grp * (size_t)T * D;

    // this lane's row: q~ and dO' fragments (B operands), and the folded -lse2 / -Delta; rows
    // past TG use zeros (their dS is 0 and they are not stored)
    half8 qf[KS], of[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = rvalid ? M::row_frag(qg + (size_t)R * D, ks, h, D) : half8{};
        of[ks] = rvalid ? M::row_frag(og + (size_t)R * D, ks, h, D) : half8{};
    }
    const half8 fl = fold_frag(rvalid ? -a.lse2[grp * (size_t)TG + R] : 0.f, h);
    const half8 fd = fold_frag(rvalid ? -a.delta[grp * (size_t)TG + R] : 0.f, h);
    const half8 fw = fold_weights(h);
    wait_all();
    const unsigned lds0 = lds_addr(lds);
    auto fill = [&](int j, int st) {   // K and V of tile j into ring stage st (32-bit LDS bases)
        lds_fill_at<OP, D, BN, NW>(lds0 + (unsigned)(st * 2 * TILE * 2), kg, j * BN, T);
        lds_fill_at<OP, D, BN, NW>(lds0 + (unsigned)((st * 2 + 1) * TILE * 2), vg, j * BN, T);
    };
    fill(j0, 0);

    floatx16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = floatx16{};

    // tile it, with its ring stage P = (it - j0) & 1 known at compile time (LDS offsets are constants)
    auto tile = [&](int it, auto PS) {
        constexpr int P = decltype(PS)::value;
        const OP* Ks = lds + P * 2 * TILE;
        const OP* Vs = Ks + TILE;
        lds_fill_wait();
        if (it + 1 < ntiles) fill(it + 1, P ^ 1);
        const int n0 = it * BN;
        if (n0 > wave_tmax) return;                 // every row of this wave precedes the tile
        if (wave_tmin - (n0 + BN - 1) >= W) return;  // the tile is older than every row's window

        // the tile crosses some row's diagonal or window edge
        const bool diag = n0 + BN - 1 > wave_tmin || wave_tmax - n0 >= W;
        // Per 32-key half mb: two chains, S^T - lse2 (even slots) and dP^T - Delta (odd slots),
        // operands read four products ahead, then the ALU work of the half (P, dS and their fp16
        // packing); that of half 1 runs between the first dQ products.  dQ^T += K^T dS^T reads
        // its K^T fragments four products ahead.
        constexpr int NC = 2 * KS, NQ = 4 * NDB;
        // operand look-ahead: four products; two in the option instantiation, whose masks need the
        // registers (no spills; within noise of three or four on the window and QK-norm steps), and
        // at head_dim <= 64, where three waves share a SIMD
        constexpr int AHD = EXT || D <= 64 ? 2 : 4;
        auto rd = [&](int mb, int i) {
            return row_frag_sw<OP, D>((i & 1) ? Vs : Ks, 32 * mb + c, i >> 1, h);
        };
        auto rk = [&](int i) { return tr_frag_f16_sw<D>((const _Float16*)Ks, i / NDB, 32 * (i % NDB)); };
        half8 dsf[4];
        // element e (0..15) of half mb: dS^T = 2^(S^T - lse2) (dP^T - Delta) into fp16
        auto elem = [&](const floatx16 (&x)[2], int mb, int e) {
            dsf[2 * mb + (e >> 3)][e & 7] = (_Float16)(__builtin_amdgcn_exp2f(x[0][e]) * x[1][e]);
            if ((e & 7) == 7) asm volatile("" ::"v"(dsf[2 * mb + (e >> 3)]));  // keep it in its slot
        };
        auto mask = [&](floatx16 (&x)[2], int mb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = n0 + 32 * mb + acc_row(r, h);
                if (EXT ? !visible(key, t_lane, W) : key > t_lane) x[0][r] = -INFINITY;
            }
        };
        // the chains of half mb into x; with WITH_PREV, half 0's ALU work (from prev) in between
        auto chains = [&](int mb, floatx16 (&x)[2], floatx16 (&prev)[2], auto WITH_PREV) {
            half8 fr[NC];
#pragma unroll
            for (int i = 0; i < AHD; ++i) fr[i] = rd(mb, i);
            x[0] = M::mma(fw, fl, floatx16{});
            x[1] = M::mma(fw, fd, floatx16{});
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                __builtin_amdgcn_sched_barrier(0);
                x[i & 1] = M::mma(fr[i], (i & 1) ? of[i >> 1] : qf[i >> 1], x[i & 1]);
                if (i + AHD < NC) fr[i + AHD] = rd(mb, i + AHD);
                if constexpr (decltype(WITH_PREV)::value) {
#pragma unroll
                    for (int e = 16 * i / NC; e < 16 * (i + 1) / NC; ++e) elem(prev, 0, e);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        floatx16 x0[2], x1[2];
        chains(0, x0, x1, IC<0>{});
        if (diag) mask(x0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) elem(x0, 0, e);
        chains(1, x1, x0, IC<0>{});
        if (diag) mask(x1, 1);
        half8 kt[NQ];
#pragma unroll
        for (int i = 0; i < AHD; ++i) kt[i] = rk(i);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            if (i < NQ / 2) {
#pragma unroll
                for (int e = 32 * i / NQ; e < 32 * (i + 1) / NQ; ++e) elem(x1, 1, e);
            }
            dq[i % NDB] = M::mma(kt[i], dsf[i / NDB], dq[i % NDB]);
            if (i + AHD < NQ) kt[i + AHD] = rk(i + AHD);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int it = j0; it < ntiles; it += 2) {
        tile(it, IC<0>{});
        if (it + 1 >= ntiles) break;
        tile(it + 1, IC<1>{});
    }

    if (SPLIT && job.np > 1) {
        // split block (two pieces): the first to finish leaves its dQ sums in its slot; the other
        // adds them to its own (one addition per element: the same result whichever is last)
        __shared__ unsigned sh[2];
        constexpr int NF = NDB * 16;
        const size_t sb = (size_t)job.grp * (a.nrb - sp.rs) + (rb - sp.rs);
        unsigned* cnt = sp.cnt + 2 * sb;
        float* slots = sp.part + sb * 2 * (size_t)(NW * 64 * NF);
        auto at = [&](int p) { return slots + (size_t)p * (NW * 64 * NF) + (size_t)w * 64 * NF; };
        if (split_arrive(cnt, sh) == 0u) {
            float* op = at(job.piece);
#pragma unroll
            for (int i = 0; i < NF / 4; ++i)
                *reinterpret_cast<floatx4*>(op + (i * 64 + l) * 4) =
                    floatx4{dq[i / 4][4 * (i % 4)], dq[i / 4][4 * (i % 4) + 1], dq[i / 4][4 * (i % 4) + 2],
                            dq[i / 4][4 * (i % 4) + 3]};
            split_publish(cnt);
            return;
        }
        const float poison = split_collect(cnt, 1u, sh) ? 0.f : __builtin_nanf("");
        const float* op = at(job.piece ^ 1);
#pragma unroll
        for (int i = 0; i < NF / 4; ++i) {
            const floatx4 x = *reinterpret_cast<const floatx4*>(op + (i * 64 + l) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) dq[i / 4][4 * (i % 4) + e] += x[e] + poison;
        }
    }

    if (!rvalid) return;  // both lanes of a row pair (c, c + 32) agree
    const int t = t_lane, hh = R - t * G, hq = hkv * G + hh;
    const size_t qoff = (((size_t)b * T + t) * a.Hq + hq) * D;
    const float sc = a.scale * (a.dsc ? a.dsc[grp] : 1.f);   // the dO scale undone as well
    const bool rope = a.rope_base > 0.0;
    // dq = R^T (scale * dq'), in place
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * db + 8 * q4 + 4 * h;
            float x0 = dq[db][4 * q4] * sc, x1 = dq[db][4 * q4 + 1] * sc;
            float x2 = dq[db][4 * q4 + 2] * sc, x3 = dq[db][4 * q4 + 3] * sc;
            if (rope) {
                const float2 r0 = a.table[(size_t)t * (D / 2) + d / 2];
                const float2 r1 = a.table[(size_t)t * (D / 2) + d / 2 + 1];
                const float y0 = x0 * r0.x + x1 * r0.y, y1 = -x0 * r0.y + x1 * r0.x;
                const float y2 = x2 * r1.x + x3 * r1.y, y3 = -x2 * r1.y + x3 * r1.x;
                x0 = y0; x1 = y1; x2 = y2; x3 = y3;
            }
            dq[db][4 * q4] = x0; dq[db][4 * q4 + 1] = x1; dq[db][4 * q4 + 2] = x2; dq[db][4 * q4 + 3] = x3;
        }
    if (EXT && a.qkn.on) qk_norm_bwd_row<NDB>(dq, a.q, qoff, a.in_dt, a.rq[grp * (size_t)TG + R], a.qkn.gain, h);
    TOUT* dqrow = (TOUT*)a.dq + qoff;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            store4(dqrow + 32 * db + 8 * q4 + 4 * h, dq[db][4 * q4], dq[db][4 * q4 + 1], dq[db][4 * q4 + 2],
                   dq[db][4 * q4 + 3]);
}

// =====================================================================================
// Backward dQ from the stored dS, 16-bit operands (deterministic, no atomics).  The dK/dV pass
// leaves dS of every tile of 64 flattened rows x 64 keys it visits in the workspace, as its lanes
// hold it: lane (h, c) of the wave for row half rh and key half kq has, for k-step cc, the 8 rows
// 32 rh + 16 cc + 8 (j / 4) + 4 h + j % 4 (j < 8) of key 32 kq + c, stored in 1 KiB block
// (2 kq + rh) * 2 + cc at slot 32 h + (c ^ (4 h + 8 cc)).  Here dQ^T += K^T dS^T: tiles are copied
// whole into LDS, and both operands are transposed reads (ds_read_tr16_b64), dS^T addressed
// through that layout as rows of keys and columns of positions p = 32 rh + 16 cc + 8 h + j, so
// the contraction order of the two operands is the same j order; the epilogue maps positions
// back to rows.  No S, P or dP is recomputed.
// grid (ceil(nrt / 4) * ngrp), the groups grp0 .. grp0 + ngrp - 1 of one batch, 512 threads: a
// block takes 4 row tiles, wave w positions
// 32 (w & 1) .. 32 (w & 1) + 31 of tile w >> 1 and all D columns of dQ; per 64-key step the K tile
// and the 4 dS tiles come global -> registers two steps ahead (non-temporal loads for dS, which is
// read once), then registers -> a 2-stage LDS ring one step ahead.
// =====================================================================================
// B operand of dQ^T += K^T dS^T for k-step kk and positions col0 .. col0 + 31 of a stored tile
// in LDS (the same lane pattern as tr_frag_f16_sw).
__device__ __forceinline__ half8 ds_tr_frag(const _Float16* tile, int kk, int col0) {
    const int l = lane_id();
    const int g = l >> 4, s = l & 15, h = l >> 5;
    const int pos = col0 + 16 * (g & 1) + 4 * (s & 3), ch = pos >> 3;
    const int key = 16 * kk + 4 * h + (s >> 2);                    // and key + 8 (same key half)
    const int cc = (ch >> 1) & 1, hh = ch & 1, c = key & 31;
    const int blk = ((key >> 5) * 2 + (ch >> 2)) * 2 + cc;
    const int lo = (blk * 64 + 32 * hh + (c ^ (4 * hh + 8 * cc))) * 16 + (pos & 7) * 2;
    const int hi = (blk * 64 + 32 * hh + ((c + 8) ^ (4 * hh + 8 * cc))) * 16 + (pos & 7) * 2;
    const char* t = reinterpret_cast<const char*>(tile);
    fp16x4_tr a = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr_ptr)(t + lo));
    fp16x4_tr b = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr_ptr)(t + hi));
    half8 f;
    half4v x = __builtin_bit_cast(half4v, a), y = __builtin_bit_cast(half4v, b);
    f[0] = x[0]; f[1] = x[1]; f[2] = x[2]; f[3] = x[3];
    f[4] = y[0]; f[5] = y[1]; f[6] = y[2]; f[7] = y[3];
    return f;
}

constexpr int kDqRowTiles = 4;  // row tiles (64 flattened rows each) per dq_ds_kernel block
// QKN: the QK norm is on (its backward in the epilogue, the raw q values fetched up front); a
// separate instantiation, so that the plain kernel keeps its registers.
template <int D, typename TOUT, int RT, bool QKN>
__global__ __launch_bounds__(128 * RT) void dq_ds_kernel(BwdArgs a) {
    using OP = _Float16;
    using M = Mma<OP>;
    static_assert(RT == 4, "512 threads: one 16-byte unit of each dS tile per thread");
    constexpr int BN = 64, NST = 2, NDB = D / 32;
    constexpr int PF = 2;                              // register slots (two: 54 us; four: 56 us)
    constexpr int KT = BN * D, DT = BN * 64;           // elements of a K tile and of a dS^T tile
    constexpr int STG = KT + RT * DT;                  // elements per LDS stage
    constexpr int CPR = D / 8, KCH = BN * CPR;         // 16-byte chunks per K row, per K tile
    constexpr int KPT = (KCH + 511) / 512;             // K chunks per thread
    __shared__ __attribute__((aligned(1024))) OP lds[NST * STG];

    const int T = a.T, G = a.G, TG = T * G;
    const int nrt = (TG + 63) / 64, nkb = (T + 63) / 64;
    const Work wk = map_block((nrt + RT - 1) / RT, a.ngrp, true);
    const int gg = a.grp0 + wk.grp;                   // the (batch, KV head) group
    const int hkv = gg % a.Hkv, b = gg / a.Hkv;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    const int rt0 = RT * wk.blk;
    const int W = a.window;
    const size_t grp = (size_t)gg;
    const OP* kg = (const OP*)a.kh + grp * (size_t)T * D;
    const OP* dsg = (const OP*)a.ds + (size_t)wk.grp * ds_tiles_per_group(nrt, nkb, G) * 4096;

    // key blocks with a stored tile for row tile rt: kb G <= rt, and the rows that see some key
    // of the block extend past 64 rt: min(T, 64 kb + 63 + W) G > 64 rt
    auto kb_hi = [&](int rt) { return min(nkb - 1, rt / G); };
    auto kb_lo = [&](int rt) {
        const int a0 = T - 63 - W;                                   // 64 kb >= a0: reaches T
        const int la = a0 <= 0 ? 0 : (a0 + 63) / 64;
        const int y = (int)((int64_t)64 * rt / G) - 63 - W;           // 64 kb > y
        const int lb = y < 0 ? 0 : y / 64 + 1;
        return min(la, lb);
    };
    const int lo = kb_lo(rt0), hi = kb_hi(min(rt0 + RT - 1, nrt - 1));
    const int rt = rt0 + (w >> 1), pb = w & 1;          // this wave's row tile and positions
    const bool wact = rt < nrt;
    const int wlo = wact ? kb_lo(rt) : 1, whi = wact ? kb_hi(rt) : 0;

    // Step kb's K tile and RT dS tiles travel global -> registers PF steps ahead (slot
    // (kb - lo) % PF), then registers -> LDS stage (kb - lo) & 1 one step ahead (with the LDS
    // stage, three steps of loads are in flight; deeper register rings measured no faster).  Every step issues
    // the same loads (past hi, or for a row tile without a stored tile, from a valid tile that is
    // not used), so the waits before each register -> LDS copy keep the later steps' loads in flight.
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) const u32x4 gu32x4;
    u32x4 kr[PF][KPT], dr[PF][RT];
    int rlo[RT], rhi[RT];                              // key blocks of each row tile (uniform)
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int rtx = rt0 + r;
        rlo[r] = __builtin_amdgcn_readfirstlane(rtx < nrt ? kb_lo(rtx) : 1);
        rhi[r] = __builtin_amdgcn_readfirstlane(rtx < nrt ? kb_hi(rtx) : 0);
    }
    // start (in elements) of the 8 KiB that the loads past hi read from the group's K' rows
    const int64_t kdummy = (int64_t)T * D >= 4096 ? min((int64_t)hi * BN * D, (int64_t)T * D - 4096) : -1;
    auto issue = [&](int kb, auto SLOT) {
        constexpr int sl = decltype(SLOT)::value;
        const int kc = min(kb, hi);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int q = (tid + 512 * i) % KCH, r = q / CPR;
            kr[sl][i] = *reinterpret_cast<const u32x4*>(kg + (size_t)min(kc * BN + r, T - 1) * D + (q % CPR) * 8);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const bool ok = kc >= rlo[r] && kc <= rhi[r];
            // past hi the loads are not used: read 8 KiB of the group's K' rows again (L2-resident)
            // instead of dS, ending at the group's last row at most (a K tile holds only 4 KiB at
            // D = 32, and a ragged last tile less); a group with fewer than 8 KiB of K' reads its
            // first dS tile instead (a whole 8 KiB tile of its own)
            gu32x4* src = sgpr_global_ptr<const u32x4>(
                kb > hi ? (kdummy >= 0 ? kg + kdummy : dsg)
                        : dsg + (ok ? ds_tile_index(kc, rt0 + r, nrt, G) : 0) * 4096);
            dr[sl][r] = __builtin_nontemporal_load(src + tid);
        }
    };
    auto commit = [&](int kb, auto SLOT) {
        constexpr int sl = decltype(SLOT)::value;
        if (kb > hi) return;
        char* st = reinterpret_cast<char*>(lds + ((kb - lo) & 1) * STG);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int q = tid + 512 * i, r = q / CPR;
            if (KCH % 512 == 0 || q < KCH)
                *reinterpret_cast<u32x4*>(st + r * (D * 2) + (((q % CPR) ^ Tile<OP, D>::swz(r)) << 4)) = kr[sl][i];
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) *reinterpret_cast<u32x4*>(st + (KT + r * DT) * 2 + tid * 16) = dr[sl][r];
    };

    // the row of this lane's position c (both lanes of the pair c, c + 32 agree)
    const int R = 64 * rt + 32 * pb + 16 * (c >> 4) + 8 * ((c & 7) >> 2) + 4 * ((c >> 3) & 1) + (c & 3);
    const bool rvalid = wact && R < TG;
    const int t = R / G, hh = R - t * G, hq = hkv * G + hh;
    const size_t qoff = (((size_t)b * T + t) * a.Hq + hq) * D;
    // QK norm: the raw (16-bit) q values and 1/rms of the row, fetched now so that the epilogue
    // does not wait for them
    uint2 xr[NDB][4];
    float rho = 0.f;
    if (QKN && rvalid) {
        rho = a.rq[grp * (size_t)TG + R];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                xr[db][q4] = *reinterpret_cast<const uint2*>((const char*)a.q + (qoff + 32 * db + 8 * q4 + 4 * h) * 2);
    }

    floatx16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = floatx16{};
    auto compute = [&](int kb) {
        const _Float16* Ks = lds + ((kb - lo) & 1) * STG;
        const _Float16* Ds = Ks + KT + (w >> 1) * DT;
        half8 df[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) df[ks] = ds_tr_frag(Ds, ks, 32 * pb);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int db = 0; db < NDB; ++db) dq[db] = M::mma(tr_frag_f16_sw<D>(Ks, ks, 32 * db), df[ks], dq[db]);
    };
    auto body = [&](int kb, auto SLOT) {
        constexpr int sl = decltype(SLOT)::value;
        commit(kb + 1, IC<(sl + 1) % PF>{});
        issue(kb + PF, SLOT);
        if (kb >= wlo && kb <= whi) compute(kb);
        __syncthreads();
    };
    // (lo <= hi always: every row tile sees its own diagonal block)
    issue(lo, IC<0>{});
    issue(lo + 1, IC<1>{});
    commit(lo, IC<0>{});
    __syncthreads();
    for (int kb = lo; kb <= hi; kb += PF) {
        body(kb, IC<0>{});
        if (kb + 1 > hi) break;
        body(kb + 1, IC<1>{});
    }

    if (!rvalid) return;
    const float sc = a.scale * (a.dsc ? a.dsc[grp] : 1.f);   // the dO scale undone as well
    const bool rope = a.rope_base > 0.0;
    // dq = R^T (scale * dq'), in place
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * db + 8 * q4 + 4 * h;
            float x0 = dq[db][4 * q4] * sc, x1 = dq[db][4 * q4 + 1] * sc;
            float x2 = dq[db][4 * q4 + 2] * sc, x3 = dq[db][4 * q4 + 3] * sc;
            if (rope) {
                const float2 r0 = a.table[(size_t)t * (D / 2) + d / 2];
                const float2 r1 = a.table[(size_t)t * (D / 2) + d / 2 + 1];
                const float y0 = x0 * r0.x + x1 * r0.y, y1 = -x0 * r0.y + x1 * r0.x;
                const float y2 = x2 * r1.x + x3 * r1.y, y3 = -x2 * r1.y + x3 * r1.x;
                x0 = y0; x1 = y1; x2 = y2; x3 = y3;
            }
            dq[db][4 * q4] = x0; dq[db][4 * q4 + 1] = x1; dq[db][4 * q4 + 2] = x2; dq[db][4 * q4 + 3] = x3;
        }
    if constexpr (QKN) qk_norm_bwd_row_raw16<NDB>(dq, xr, a.in_dt, rho, a.qkn.gain);
    TOUT* dqrow = (TOUT*)a.dq + qoff;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            store4(dqrow + 32 * db + 8 * q4 + 4 * h, dq[db][4 * q4], dq[db][4 * q4 + 1], dq[db][4 * q4 + 2],
                   dq[db][4 * q4 + 3]);
}

// =====================================================================================
// Launchers.
// =====================================================================================
// Records ev[2i] / ev[2i + 1] around launch i when events are given (null entries skipped).
struct Marks {
    hipEvent_t const* ev;
    hipStream_t s;
    hipError_t rec(int j) const { return ev && ev[j] ? hipEventRecord(ev[j], s) : hipSuccess; }
    hipError_t before(int i) const { return rec(2 * i); }
    hipError_t after(int i) const { return rec(2 * i + 1); }
};

#define NE_TRY(x)                             \
    do {                                      \
        hipError_t e_ = (x);                  \
        if (e_ != hipSuccess) return e_;      \
    } while (0)

// Grid of prep_kernel: 8 tokens of one batch element per workgroup, and, when that gives fewer than
// 1024 workgroups (a small call, bound by loads in flight rather than bandwidth), the rows of each
// token cut into up to 4 ranges.  The NanoEuler layer (B8 T512 Hq12 Hkv4 D64: 512 workgroups) runs
// its backward preparation 3.5 us faster cut in 4; at 1024 workgroups (B4 T2048) a cut in 2 was
// 2.7 us slower.
static dim3 prep_grid(const PrepArgs& pa, bool bwd) {
    const int nb = (pa.T + 7) / 8 * pa.B;
    const int rows = bwd ? 2 * pa.Hq + 2 * pa.Hkv - (pa.skip_v ? pa.Hkv : 0) : 2 * pa.Hkv;
    const int z = nb >= 1024 ? 1 : std::max(1, std::min({4, rows, (2048 + nb - 1) / nb}));
    return dim3((pa.T + 7) / 8, pa.B, z);
}

template <typename TI, typename TO, typename OP, int D>
static hipError_t launch_fwd_t(const PrepArgs& pa, const FwdArgs& fa, const SplitPlan& sp, hipStream_t s,
                               hipEvent_t const* ev) {
    const Marks m{ev, s};
    NE_TRY(m.before(0));
    if constexpr (sizeof(OP) == 2)
        hipLaunchKernelGGL((prep_fwd_h<TI, D>), dim3((pa.T + 63) / 64, pa.B * pa.Hkv, 2), dim3(256), 0, s, pa);
    else
        hipLaunchKernelGGL((prep_kernel<TI, TO, OP, D, false>), prep_grid(pa, false), dim3(256), 0, s, pa);
    NE_TRY(hipGetLastError());
    NE_TRY(m.after(0));
    NE_TRY(m.before(1));
    if constexpr (sizeof(OP) == 2) {
        FwdArgs f2 = fa;
        constexpr int BMF = D <= 64 ? 128 : 256;         // rows per workgroup (2 threads per row)
        f2.nrb = (int)(((int64_t)fa.T * fa.G + BMF - 1) / BMF);
        const int njobs = sp.njobs ? sp.njobs : f2.nrb;
        if (sp.njobs)
            hipLaunchKernelGGL((fwd_kernel_h<TI, D, TO, true>), dim3(njobs * fa.Hkv * fa.B), dim3(2 * BMF), 0, s, f2, sp);
        else
            hipLaunchKernelGGL((fwd_kernel_h<TI, D, TO, false>), dim3(njobs * fa.Hkv * fa.B), dim3(2 * BMF), 0, s, f2, sp);
    }
    else
        hipLaunchKernelGGL((fwd_kernel<TI, OP, D, TO>), dim3(fa.nrb * fa.Hkv * fa.B), dim3(256), 0, s, fa);
    NE_TRY(hipGetLastError());
    return m.after(1);
}

// =====================================================================================
// Half-split rotary pairs: rows that the backward wrote in slot order (element i in slot 2i,
// element i + D/2 in slot 2i + 1) put back in element order, in place.  grid ceil(nrows / RPB),
// 256 threads: RPB = 256 / (D / 4) whole rows per workgroup staged through LDS, so every load of
// the workgroup has landed before any store; each thread then writes four consecutive elements.
// =====================================================================================
template <typename T, int D>
__global__ __launch_bounds__(256) void slots_to_elems_kernel(T* rows, int64_t nrows) {
    constexpr int TPR = D / 4, RPB = 256 / TPR;
    __shared__ float buf[RPB][D];
    const int rl = threadIdx.x / TPR, d = 4 * (threadIdx.x % TPR);
    const int64_t row = (int64_t)blockIdx.x * RPB + rl;
    const bool ok = row < nrows;
    T* r = rows + (ok ? row : 0) * D;
    if (ok) {
#pragma unroll
        for (int e = 0; e < 4; ++e) buf[rl][d + e] = to_f32(r[d + e]);
    }
    __syncthreads();
    if (ok) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = d + e;
            x[e] = buf[rl][i < D / 2 ? 2 * i : 2 * (i - D / 2) + 1];
        }
        store4(r + d, x[0], x[1], x[2], x[3]);
    }
}

template <typename TI, typename TO, typename OP, int D>
static hipError_t launch_bwd_passes(int mode, const PrepArgs& pa, const AmaxArgs& am, const BwdArgs& ba,
                                    const SplitPlan& sp, const SplitPlan& spk, hipStream_t s, hipEvent_t const* ev) {
    const Marks m{ev, s};
    NE_TRY(m.before(0));
    if constexpr (sizeof(OP) == 2) {
        hipLaunchKernelGGL((dO_amax_kernel<TI, D>), dim3(am.nparts, ba.B), dim3(256), 0, s, am);
        NE_TRY(hipGetLastError());
    }
    hipLaunchKernelGGL((prep_kernel<TI, TO, OP, D, true>), prep_grid(pa, true), dim3(256), 0, s, pa);
    NE_TRY(hipGetLastError());
    NE_TRY(m.after(0));
    const int ngroups = ba.B * ba.Hkv, npair = ((ba.T + 63) / 64 + 1) / 2;
    if constexpr (sizeof(OP) == 2) {
        if (mode == kBwdStoredDs) {
            // stored dS: dK/dV, then dQ, for each batch of ds_groups groups (a single batch unless the
            // dS of every group would exceed the buffer); with several batches the second marked
            // interval covers all but the last dQ launch as well
            const int nrt = (int)(((int64_t)ba.T * ba.G + 63) / 64);
            NE_TRY(m.before(1));
            for (int g0 = 0; g0 < ngroups; g0 += ba.ds_groups) {
                BwdArgs bb = ba;
                bb.grp0 = g0;
                bb.ngrp = min(ba.ds_groups, ngroups - g0);
                hipLaunchKernelGGL((dkdv_kernel_h<D, TO, 1, false>), dim3(npair * bb.ngrp), dim3(512), 0, s, bb, spk);
                NE_TRY(hipGetLastError());
                if (g0 + bb.ngrp >= ngroups) {
                    NE_TRY(m.after(1));
                    NE_TRY(m.before(2));
                }
                const dim3 grid((nrt + kDqRowTiles - 1) / kDqRowTiles * bb.ngrp);
                if (ba.qkn.on) hipLaunchKernelGGL((dq_ds_kernel<D, TO, kDqRowTiles, true>), grid, dim3(128 * kDqRowTiles), 0, s, bb);
                else hipLaunchKernelGGL((dq_ds_kernel<D, TO, kDqRowTiles, false>), grid, dim3(128 * kDqRowTiles), 0, s, bb);
                NE_TRY(hipGetLastError());
            }
            return m.after(2);
        }
        if (mode == kBwdAtomic) {
            NE_TRY(m.before(1));
            hipLaunchKernelGGL((dkdv_kernel_h<D, TO, 2, false>), dim3(npair * ngroups), dim3(512), 0, s, ba, spk);
            NE_TRY(hipGetLastError());
            NE_TRY(m.after(1));
            NE_TRY(m.before(2));
            const int64_t rows = (int64_t)ngroups * ba.T * ba.G;
            hipLaunchKernelGGL((dq_acc_convert_kernel<D, TO>), dim3((unsigned)((rows * D / 4 + 255) / 256)), dim3(256), 0,
                               s, ba);
            NE_TRY(hipGetLastError());
            return m.after(2);
        }
    }
    NE_TRY(m.before(1));
    if constexpr (sizeof(OP) == 2)
        if (spk.njobs)
            hipLaunchKernelGGL((dkdv_kernel_h<D, TO, 0, true>), dim3(spk.njobs * ngroups), dim3(512), 0, s, ba, spk);
        else
            hipLaunchKernelGGL((dkdv_kernel_h<D, TO, 0, false>), dim3(npair * ngroups), dim3(512), 0, s, ba, spk);
    else
        hipLaunchKernelGGL((dkdv_kernel<OP, D, TO>), dim3(npair * ngroups), dim3(512), 0, s, ba);
    NE_TRY(hipGetLastError());
    NE_TRY(m.after(1));
    NE_TRY(m.before(2));
    if constexpr (sizeof(OP) == 2) {
        if (ba.window < ba.T || ba.qkn.on)
            hipLaunchKernelGGL((dq_kernel_h<D, TO, true, false>), dim3(ba.nrb * ngroups), dim3(256), 0, s, ba, sp);
        else if (sp.njobs)
            hipLaunchKernelGGL((dq_kernel_h<D, TO, false, true>), dim3(sp.njobs * ngroups), dim3(256), 0, s, ba, sp);
        else
            hipLaunchKernelGGL((dq_kernel_h<D, TO, false, false>), dim3(ba.nrb * ngroups), dim3(256), 0, s, ba, sp);
    }
    else
        hipLaunchKernelGGL((dq_kernel<OP, D, TO>), dim3(ba.nrb * ngroups), dim3(256), 0, s, ba);
    NE_TRY(hipGetLastError());
    return m.after(2);
}

// The backward's passes, then (half-split pairing) dq and dk back to element order; the marked
// intervals cover the passes.
template <typename TI, typename TO, typename OP, int D>
static hipError_t launch_bwd_t(int mode, const PrepArgs& pa, const AmaxArgs& am, const BwdArgs& ba,
                               const SplitPlan& sp, const SplitPlan& spk, hipStream_t s, hipEvent_t const* ev) {
    NE_TRY((launch_bwd_passes<TI, TO, OP, D>(mode, pa, am, ba, sp, spk, s, ev)));
    if (!ba.half) return hipSuccess;
    constexpr int RPB = 256 / (D / 4);
    const int64_t nq = (int64_t)ba.B * ba.T * ba.Hq, nk = (int64_t)ba.B * ba.T * ba.Hkv;
    hipLaunchKernelGGL((slots_to_elems_kernel<TO, D>), dim3((unsigned)((nq + RPB - 1) / RPB)), dim3(256), 0, s,
                       (TO*)ba.dq, nq);
    NE_TRY(hipGetLastError());
    hipLaunchKernelGGL((slots_to_elems_kernel<TO, D>), dim3((unsigned)((nk + RPB - 1) / RPB)), dim3(256), 0, s,
                       (TO*)ba.dk, nk);
    return hipGetLastError();
}

#define NE_DISPATCH_D(FN, TI, TO, OP, D, ...)                       \
    switch (D) {                                                   \
        case 32: return FN<TI, TO, OP, 32>(__VA_ARGS__);           \
        case 64: return FN<TI, TO, OP, 64>(__VA_ARGS__);           \
        case 128: return FN<TI, TO, OP, 128>(__VA_ARGS__);         \
        default: return hipErrorInvalidValue;                      \
    }

hipError_t launch_fwd(int in_dt, int out_dt, int D, const PrepArgs& pa, const FwdArgs& fa, const SplitPlan& sp,
                      hipStream_t s, hipEvent_t const* ev) {
    if (in_dt == 0 && out_dt == 0) { NE_DISPATCH_D(launch_fwd_t, float, float, float, D, pa, fa, sp, s, ev) }
    if (in_dt == 1 && out_dt == 0) { NE_DISPATCH_D(launch_fwd_t, __bf16, float, _Float16, D, pa, fa, sp, s, ev) }
    if (in_dt == 1 && out_dt == 1) { NE_DISPATCH_D(launch_fwd_t, __bf16, __bf16, _Float16, D, pa, fa, sp, s, ev) }
    if (in_dt == 2 && out_dt == 0) { NE_DISPATCH_D(launch_fwd_t, _Float16, float, _Float16, D, pa, fa, sp, s, ev) }
    if (in_dt == 2 && out_dt == 2) { NE_DISPATCH_D(launch_fwd_t, _Float16, _Float16, _Float16, D, pa, fa, sp, s, ev) }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(int in_dt, int out_dt, int D, int mode, const PrepArgs& pa, const AmaxArgs& am,
                      const BwdArgs& ba, const SplitPlan& spq, const SplitPlan& spk, hipStream_t s,
                      hipEvent_t const* ev) {
    if (in_dt == 0 && out_dt == 0) { NE_DISPATCH_D(launch_bwd_t, float, float, float, D, mode, pa, am, ba, spq, spk, s, ev) }
    if (in_dt == 1 && out_dt == 0) { NE_DISPATCH_D(launch_bwd_t, __bf16, float, _Float16, D, mode, pa, am, ba, spq, spk, s, ev) }
    if (in_dt == 1 && out_dt == 1) { NE_DISPATCH_D(launch_bwd_t, __bf16, __bf16, _Float16, D, mode, pa, am, ba, spq, spk, s, ev) }
    if (in_dt == 2 && out_dt == 0) { NE_DISPATCH_D(launch_bwd_t, _Float16, float, _Float16, D, mode, pa, am, ba, spq, spk, s, ev) }
    if (in_dt == 2 && out_dt == 2) { NE_DISPATCH_D(launch_bwd_t, _Float16, _Float16, _Float16, D, mode, pa, am, ba, spq, spk, s, ev) }
    return hipErrorInvalidValue;
}

hipError_t launch_table(const TableArgs& a, hipStream_t s) {
    const int64_t n = (int64_t)a.T * (a.D / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ne
