// ne_qkv.hip -- QKV projection y = x W^T with the rotation (and optionally the QK norm) applied in
// the epilogue, so the rotated q' and k' (and v) leave the matrix product directly, gfx950.
//
// x [M = B*T][C] and W [N = (Hq + 2 Hkv) D][C] are row-major (W as a linear layer stores it), in
// bf16 or fp16; products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation.  The
// product is computed transposed, Y^T = W X^T (features on the accumulator rows, one token per
// lane column), so each lane holds 4 consecutive features of its token per register group:
// the rotary pairs (2i, 2i + 1) are in-lane, a head's sum of squares is in-lane plus one half
// swap, and the accumulator layout is the one store_rows writes out as whole rows.
#include <hip/hip_runtime.h>

#include "ne_common.hpp"
#include "ne_launch.hpp"

namespace ne {

namespace {

// cos and sin of t * theta_i for t < T, i < D/2 into table[T][D/2]; theta from the host in double
// precision, the phase reduced to [-pi, pi] in double so that fp32 sincos sees a small argument.
__global__ __launch_bounds__(256) void qkv_rope_table_kernel(QkvArgs a) {
    constexpr double kTwoPiHi = 6.283185307179586;
    constexpr double kTwoPiLo = 2.4492935982947064e-16;
    constexpr double kInvTwoPi = 0.15915494309189535;
    const int half = a.D / 2;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.T * half) return;
    const int t = idx / half, i = idx % half;
    const double phi = (double)t * a.theta[i];
    const double n = rint(phi * kInvTwoPi);
    const double r = fma(-n, kTwoPiLo, fma(-n, kTwoPiHi, phi));
    float s, c;
    sincosf((float)r, &s, &c);
    a.table[idx] = make_float2(c, s);
}

// Rows [row0, row0 + ROWS) x columns [k0, k0 + BK) of a row-major array with leading dimension
// ld into a swizzled LDS tile (direct global->LDS loads by the NW waves); rows at or past nrows
// repeat row nrows - 1.  Byte offsets are 32-bit: nrows * ld * sizeof(OP) < 2^31.
template <typename OP, int BK, int ROWS, int NW>
__device__ __forceinline__ void fill_rows(OP* tile, const OP* src, int row0, int nrows, int ld, int k0) {
    using TL = Tile<OP, BK>;
    constexpr int WL = ROWS * TL::CPR / 64;
    static_assert(ROWS * TL::CPR % 64 == 0 && WL % NW == 0, "whole wave loads per wave");
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < WL / NW; ++i) {
        const int j = i * NW + w;
        const int q = 64 * j + l;
        const int r = q / TL::CPR, p = q % TL::CPR;
        const int gr = min(row0 + r, nrows - 1);
        const unsigned off = (unsigned)(((size_t)gr * ld + k0 + (p ^ TL::swz(r)) * TL::EPC) * sizeof(OP));
        dma16_s(off, src, lds_addr(reinterpret_cast<char*>(tile) + 1024 * j));
    }
}

// Same, with the tile given as a wave-uniform 32-bit LDS byte address.
template <typename OP, int BK, int ROWS, int NW>
__device__ __forceinline__ void fill_rows_at(unsigned tile, const OP* src, int row0, int nrows, int ld, int k0) {
    using TL = Tile<OP, BK>;
    constexpr int WL = ROWS * TL::CPR / 64;
    static_assert(ROWS * TL::CPR % 64 == 0 && WL % NW == 0, "whole wave loads per wave");
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < WL / NW; ++i) {
        const int j = i * NW + w;
        const int q = 64 * j + l;
        const int r = q / TL::CPR, p = q % TL::CPR;
        const int gr = min(row0 + r, nrows - 1);
        const unsigned off = (unsigned)(((size_t)gr * ld + k0 + (p ^ TL::swz(r)) * TL::EPC) * sizeof(OP));
        dma16_s(off, src, __builtin_amdgcn_readfirstlane(tile + 1024u * (unsigned)j));
    }
}

template <typename TI>
__device__ __forceinline__ floatx16 mma16(half8 a, half8 b, floatx16 c) {
    if constexpr (sizeof(TI) == 2 && __is_same(TI, __bf16)) {
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                      0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
}

}  // namespace

// =====================================================================================
// Narrow tiles, for projections too small to fill the chip with the wide tiles below.
// grid (ceil(M / 256) * N / 128), 256 threads = 4 waves.  A workgroup computes 256 tokens x 128
// features; wave w takes tokens [64 w, 64 w + 64) (two 32-token blocks) against all 128 features
// (four 32-feature blocks): 8 accumulators.  W and x tiles of BK columns go through a 2-stage LDS
// ring filled one step ahead by direct loads.  Epilogue per 32-token block and head: QK norm
// (q and k heads), rotation by the token's position (q and k heads), rows out through LDS.
// Workgroups of one 256-token block are dispatched to one XCD (its L2 keeps that block of x).
// =====================================================================================
// Column step and waves per SIMD: 64 / 1 measured best on the B4 T2048 C1536 N2560 projection
// (91.6 us; 32 / 2: 100.5 us, 32 / 1: 110.1 us, 64 / 2: 93.5 us).
#ifndef NE_QKV_BK
#define NE_QKV_BK 64
#endif
#ifndef NE_QKV_WPE
#define NE_QKV_WPE 1
#endif
template <typename TI, typename TOUT, int D, int BK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NE_QKV_WPE))) void qkv_rope_kernel(QkvArgs a) {
    constexpr int BM = 256, BN = 128, NW = 4, KS = BK / 16, HPT = BN / D, FPH = D / 32;
    constexpr int ATILE = BN * BK, BTILE = BM * BK;
    constexpr int RING = 2 * (ATILE + BTILE) * 2;                  // bytes
    constexpr int OUTB = NW * 32 * D * (int)sizeof(TOUT);          // store_rows scratch
    __shared__ __attribute__((aligned(1024))) char lds_raw[RING > OUTB ? RING : OUTB];
    _Float16* const lds = reinterpret_cast<_Float16*>(lds_raw);
    auto As = [&](int st) { return lds + st * (ATILE + BTILE); };
    auto Bs = [&](int st) { return lds + st * (ATILE + BTILE) + ATILE; };

    const int M = a.M, C = a.C, N = a.N;
    const int NB = N / BN, MB = (M + BM - 1) / BM;
    int mb, nb;
    {
        const int i = blockIdx.x;
        if ((MB & 7) == 0) {  // XCD i % 8 takes the 256-token blocks congruent to it
            const int x = i & 7, k = i >> 3;
            nb = k % NB;
            mb = x + 8 * (k / NB);
        } else {
            nb = i % NB;
            mb = i / NB;
        }
    }
    const int m0 = mb * BM, n0 = nb * BN;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    const _Float16* x = (const _Float16*)a.x;   // 16-bit words; the MFMA reinterprets them as TI
    const _Float16* wt = (const _Float16*)a.w;

    floatx16 acc[2][4];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) acc[tb][fb] = floatx16{};

    const int nk = C / BK;
    fill_rows<_Float16, BK, BN, NW>(As(0), wt, n0, N, C, 0);
    fill_rows<_Float16, BK, BM, NW>(Bs(0), x, m0, M, C, 0);
    for (int it = 0; it < nk; ++it) {
        // stage it has landed and every wave is done with stage it - 1, which the next fill reuses
        lds_fill_wait();
        if (it + 1 < nk) {
            fill_rows<_Float16, BK, BN, NW>(As((it + 1) & 1), wt, n0, N, C, (it + 1) * BK);
            fill_rows<_Float16, BK, BM, NW>(Bs((it + 1) & 1), x, m0, M, C, (it + 1) * BK);
        }
        const _Float16* At = As(it & 1);
        const _Float16* Bt = Bs(it & 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            half8 bf[2], af[4];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) bf[tb] = row_frag_sw<_Float16, BK>(Bt, 64 * w + 32 * tb + c, ks, h);
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) af[fb] = row_frag_sw<_Float16, BK>(At, 32 * fb + c, ks, h);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int fb = 0; fb < 4; ++fb) acc[tb][fb] = mma16<TI>(af[fb], bf[tb], acc[tb][fb]);
        }
    }
    __syncthreads();  // the ring becomes the output scratch

    const bool rope = a.rope_base > 0.0;
    char* scratch = lds_raw + w * 32 * D * (int)sizeof(TOUT);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int mw = m0 + 64 * w + 32 * tb;   // first token of this block
        const int m = mw + c, t = (m < M ? m : M - 1) % a.T;
#pragma unroll
        for (int hh = 0; hh < HPT; ++hh) {
            const int head = (n0 + hh * D) / D;  // 0..Hq-1 q, then Hkv k heads, then Hkv v heads
            floatx16 y[FPH];
#pragma unroll
            for (int f = 0; f < FPH; ++f) y[f] = acc[tb][hh * FPH + f];
            const bool qk = head < a.Hq + a.Hkv;
            if (qk && a.qkn.on) {
                float ss = 0.f;
#pragma unroll
                for (int f = 0; f < FPH; ++f)
#pragma unroll
                    for (int r = 0; r < 16; ++r) ss += y[f][r] * y[f][r];
                const float fac = qk_factor(sum_halves(ss), D, a.qkn.gain, a.qkn.eps);
#pragma unroll
                for (int f = 0; f < FPH; ++f)
#pragma unroll
                    for (int r = 0; r < 16; ++r) y[f][r] *= fac;
            }
            if (qk && rope && a.half) {
                // half-split pairs (i, i + D/2): both in this lane -- feature block f + FPH / 2 for
                // D >= 64, the same block 16 features on (q4 + 2) for D = 32
                const float2* cs = a.table + (size_t)t * (D / 2);
                constexpr int FL = FPH >= 2 ? FPH / 2 : 1, QL = FPH >= 2 ? 4 : 2;
#pragma unroll
                for (int f = 0; f < FL; ++f)
#pragma unroll
                    for (int q4 = 0; q4 < QL; ++q4)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int i = 32 * f + 8 * q4 + 4 * h + e;   // < D / 2
                            const int fh = FPH >= 2 ? f + FPH / 2 : f, rh = FPH >= 2 ? 4 * q4 + e : 4 * (q4 + 2) + e;
                            const float2 r = cs[i];
                            const float u = y[f][4 * q4 + e], v = y[fh][rh];
                            y[f][4 * q4 + e] = u * r.x - v * r.y;
                            y[fh][rh] = u * r.y + v * r.x;
                        }
            } else if (qk && rope) {
                const float2* cs = a.table + (size_t)t * (D / 2);
#pragma unroll
                for (int f = 0; f < FPH; ++f)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int d = 32 * f + 8 * q4 + 4 * h;   // features d .. d + 3 of this lane
                        const floatx4 r01 = *reinterpret_cast<const floatx4*>(cs + d / 2);
                        const float u0 = y[f][4 * q4], v0 = y[f][4 * q4 + 1];
                        const float u1 = y[f][4 * q4 + 2], v1 = y[f][4 * q4 + 3];
                        y[f][4 * q4] = u0 * r01[0] - v0 * r01[1];
                        y[f][4 * q4 + 1] = u0 * r01[1] + v0 * r01[0];
                        y[f][4 * q4 + 2] = u1 * r01[2] - v1 * r01[3];
                        y[f][4 * q4 + 3] = u1 * r01[3] + v1 * r01[2];
                    }
            }
            TOUT* base;
            int H, hd;
            if (head < a.Hq) { base = (TOUT*)a.q; H = a.Hq; hd = head; }
            else if (head < a.Hq + a.Hkv) { base = (TOUT*)a.k; H = a.Hkv; hd = head - a.Hq; }
            else { base = (TOUT*)a.v; H = a.Hkv; hd = head - a.Hq - a.Hkv; }
            store_rows<TOUT, D>(y, 1.f, scratch, [&](int i) {
                const int mi = mw + i;
                return mi < M ? base + ((size_t)mi * H + hd) * D : (TOUT*)nullptr;
            });
            __builtin_amdgcn_wave_barrier();  // this wave's scratch is reused by its next block
        }
    }
}

// =====================================================================================
// Wide tiles, for projections that fill the chip in one round.  grid (ceil(M / BM) * ceil(N / BN)),
// 512 threads = 8 waves, two per SIMD, in a WT x (8 / WT) grid over tokens x features: each wave
// computes 64 tokens (two 32-token blocks) x 160 features (five 32-feature blocks), 10
// accumulators, so every fragment read from LDS feeds two or five products.  Workgroup tile
// BM = 64 WT tokens x BN = 1280 / WT features:
//   WT = 4: 256 x 320, 64-column steps (whole 128-byte rows per direct load) in a 2-stage ring;
//           heads of 128 features straddle tiles, so it runs without the QK norm or with D <= 64;
//   WT = 2: 128 x 640 (640 / D whole heads), 32-column steps in a 3-stage ring.
// B4 T2048 C1536 N2560 projection (256 tiles either way): see the host selection below.
// Stage s + NST reuses the stage of step s, refilled right after the mid-step barrier that shows
// every wave has read it, so loads are issued NST steps ahead and each wait keeps the newer fills
// in flight; the fragments of each 16-column k-step are read while the products of the previous
// one run.  Epilogue per block: QK norm (a head's sum of squares gathered across the waves through
// LDS), rotation, and four consecutive features per lane stored directly.  Features past N (a
// partial last tile of heads) are computed from repeated rows of W and not stored.
// =====================================================================================
template <typename TI, typename TOUT, int D, int WT, int BK, int NST>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void qkv_wide_kernel(QkvArgs a) {
    constexpr int NW = 8, WF = NW / WT, BM = 64 * WT, BN = 160 * WF, TB = 2, FB = 5, KS = BK / 16;
    constexpr int ATILE = BN * BK, BTILE = BM * BK, STAGE = ATILE + BTILE;   // 16-bit elements
    constexpr int LOADS = (BN + BM) * (BK * 2 / 16) / 64 / NW;              // direct loads per wave per step
    static_assert(KS % 2 == 0 && (NST - 2) * LOADS <= 12 && (NST - 1) * LOADS <= 12, "pipeline shape");
    __shared__ __attribute__((aligned(1024))) _Float16 lds[NST * STAGE];
    auto As = [&](int st) { return lds + st * STAGE; };
    auto Bs = [&](int st) { return lds + st * STAGE + ATILE; };

    const int M = a.M, C = a.C, N = a.N;
    const int NB = (N + BN - 1) / BN, MB = (M + BM - 1) / BM;
    int mb, nb;
    {
        const int i = blockIdx.x;
        if ((MB & 7) == 0) {  // XCD i % 8 takes the token blocks congruent to it
            const int x = i & 7, k = i >> 3;
            nb = k % NB;
            mb = x + 8 * (k / NB);
        } else {
            nb = i % NB;
            mb = i / NB;
        }
    }
    const int m0 = mb * BM, n0 = nb * BN;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    const int wt_ = w % WT, wf = w / WT;        // token block of 64, feature block of 160
    const _Float16* x = (const _Float16*)a.x;   // 16-bit words; the MFMA reinterprets them as TI
    const _Float16* wt = (const _Float16*)a.w;

    floatx16 acc[TB][FB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) acc[tb][fb] = floatx16{};

    const int nk = C / BK;
    const unsigned lds0 = lds_addr(lds);
    auto fill = [&](int st, int kstep) {
        const unsigned sa = lds0 + (unsigned)(st * STAGE * 2);
        fill_rows_at<_Float16, BK, BN, NW>(sa, wt, n0, N, C, kstep * BK);
        fill_rows_at<_Float16, BK, BM, NW>(sa + ATILE * 2, x, m0, M, C, kstep * BK);
    };
    half8 af[2][FB], bf[2][TB];
    auto frags = [&](int st, int ks, half8 (&fa)[FB], half8 (&fb_)[TB]) {
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) fa[fb] = row_frag_sw<_Float16, BK>(As(st), 160 * wf + 32 * fb + c, ks, h);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) fb_[tb] = row_frag_sw<_Float16, BK>(Bs(st), 64 * wt_ + 32 * tb + c, ks, h);
    };
    auto products = [&](const half8 (&fa)[FB], const half8 (&fb_)[TB]) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) acc[tb][fb] = mma16<TI>(fa[fb], fb_[tb], acc[tb][fb]);
    };
    // the k-steps of step it but the last, each reading the next one's fragments first
    auto body = [&](int it) {
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            frags(it % NST, ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
            products(af[ks & 1], bf[ks & 1]);
        }
    };

    __builtin_assume(nk >= 64 / BK);  // C >= 64
    const int pre = nk < NST ? nk : NST;
    for (int st = 0; st < pre; ++st) fill(st, st);
    lds_fill_wait_keep((pre - 1) * LOADS);  // step 0 has landed
    frags(0, 0, af[0], bf[0]);
    for (int it = 0; it < nk - 1; ++it) {
        body(it);
        // step it + 1 has landed for every wave (later steps may still be in flight), and every
        // wave has read all of step it, whose stage the fill of step it + NST reuses
        lds_fill_wait_keep(it + 2 < nk ? (NST - 2) * LOADS : 0);
        if (it + NST < nk) fill(it % NST, it + NST);
        frags((it + 1) % NST, 0, af[0], bf[0]);
        products(af[1], bf[1]);
    }
    body(nk - 1);
    products(af[1], bf[1]);
    __syncthreads();  // the ring becomes the sum-of-squares scratch

    const bool rope = a.rope_base > 0.0;
    const int H3 = a.Hq + 2 * a.Hkv, Hqk = a.Hq + a.Hkv;
    // QK norm factor of each block's head (1 for v heads and without the norm); the accumulators
    // are only read inside the branch and scaled in the store loop
    float fac[TB][FB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) fac[tb][fb] = 1.f;
    if (BN % D == 0 && a.qkn.on) {  // the host never asks for the norm with heads straddling tiles
        // per token and 32-feature block of the tile: sum of squares, [BM][BN / 32]
        float* ssq = reinterpret_cast<float*>(lds);
        const int row = 64 * wt_ + c;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
                float ss = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) ss += acc[tb][fb][r] * acc[tb][fb][r];
                ss = sum_halves(ss);
                if (h == 0) ssq[(row + 32 * tb) * (BN / 32) + FB * wf + fb] = ss;
            }
        __syncthreads();
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
                const int f0 = n0 + 160 * wf + 32 * fb, head = f0 / D;
                const int b0 = FB * wf + fb - (f0 % D) / 32;  // the head's first block in the tile
                float ss = 0.f;
#pragma unroll
                for (int j = 0; j < D / 32; ++j) ss += ssq[(row + 32 * tb) * (BN / 32) + b0 + j];
                if (head < Hqk) fac[tb][fb] = qk_factor(ss, D, a.qkn.gain, a.qkn.eps);
            }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int m = m0 + 64 * wt_ + 32 * tb + c;
        const int t = (m < M ? m : M - 1) % a.T;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
            const int f0 = n0 + 160 * wf + 32 * fb, head = f0 / D, dh0 = f0 % D;
            const bool qk = head < Hqk, isq = head < a.Hq;
            TOUT* const base = (TOUT*)(isq ? a.q : qk ? a.k : a.v);
            const int H = isq ? a.Hq : a.Hkv, hd = isq ? head : qk ? head - a.Hq : head - Hqk;
            TOUT* row = base + ((size_t)m * H + hd) * D;
            const bool st = m < M && head < H3;
            const bool rot = qk && rope;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = dh0 + 8 * q4 + 4 * h;   // features d .. d + 3 of this lane
                const float f = fac[tb][fb];
                float y0 = acc[tb][fb][4 * q4] * f, y1 = acc[tb][fb][4 * q4 + 1] * f;
                float y2 = acc[tb][fb][4 * q4 + 2] * f, y3 = acc[tb][fb][4 * q4 + 3] * f;
                if (rot) {
                    const floatx4 r01 = *reinterpret_cast<const floatx4*>(a.table + (size_t)t * (D / 2) + d / 2);
                    const float u0 = y0, v0 = y1, u1 = y2, v1 = y3;
                    y0 = u0 * r01[0] - v0 * r01[1];
                    y1 = u0 * r01[1] + v0 * r01[0];
                    y2 = u1 * r01[2] - v1 * r01[3];
                    y3 = u1 * r01[3] + v1 * r01[2];
                }
                if (st) store4(row + d, y0, y1, y2, y3);
            }
            __builtin_amdgcn_sched_barrier(0);  // one block at a time: its registers die here
        }
    }
}

namespace {
// compute units of the current device (cached per device)
int cu_count() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <typename TI, typename TO, int D>
hipError_t launch_qkv_t(const QkvArgs& a, hipStream_t s, hipEvent_t const* ev) {
    auto rec = [&](int j) { return ev && ev[j] ? hipEventRecord(ev[j], s) : hipSuccess; };
    hipError_t e;
    if ((e = rec(0)) != hipSuccess) return e;
    if (a.rope_base > 0.0) {
        hipLaunchKernelGGL(qkv_rope_table_kernel, dim3((a.T * (D / 2) + 255) / 256), dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = rec(1)) != hipSuccess) return e;
    if ((e = rec(2)) != hipSuccess) return e;
    // Tilings by preference: 256 x 320 (least operand traffic per flop, whole-line loads), then
    // 128 x 640, each when its tiles cover at least three quarters of the compute units in one
    // round; below that the narrow kernel spreads the work wider.  B4 T2048 C1536 N2560: 256 x 320
    // 77 us, 128 x 640 85 us, narrow 95 us; 64-byte row segments (32-column steps) stream into LDS at
    // half the rate of whole 128-byte rows.
    const int cus3 = 3 * cu_count();
    const int t320 = (a.M + 255) / 256 * ((a.N + 319) / 320), t640 = (a.M + 127) / 128 * ((a.N + 639) / 640);
    // the half-split pairs of a head sit in one lane only in the narrow tiling
    if (!a.half && (!a.qkn.on || 320 % D == 0) && 4 * t320 >= cus3) {
        hipLaunchKernelGGL((qkv_wide_kernel<TI, TO, D, 4, 64, 2>), dim3(t320), dim3(512), 0, s, a);
    } else if (!a.half && 4 * t640 >= cus3) {
        hipLaunchKernelGGL((qkv_wide_kernel<TI, TO, D, 2, 32, 3>), dim3(t640), dim3(512), 0, s, a);
    } else {
        const int grid = (a.M + 255) / 256 * (a.N / 128);
        hipLaunchKernelGGL((qkv_rope_kernel<TI, TO, D, NE_QKV_BK>), dim3(grid), dim3(256), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return rec(3);
}
}  // namespace

hipError_t launch_qkv(int in_dt, int out_dt, int D, const QkvArgs& a, hipStream_t s, hipEvent_t const* ev) {
#define NE_QCASE(TI, TO)                                                   \
    switch (D) {                                                           \
        case 32: return launch_qkv_t<TI, TO, 32>(a, s, ev);                \
        case 64: return launch_qkv_t<TI, TO, 64>(a, s, ev);                \
        case 128: return launch_qkv_t<TI, TO, 128>(a, s, ev);              \
        default: return hipErrorInvalidValue;                              \
    }
    if (in_dt == 1 && out_dt == 0) { NE_QCASE(__bf16, float) }
    if (in_dt == 1 && out_dt == 1) { NE_QCASE(__bf16, __bf16) }
    if (in_dt == 2 && out_dt == 0) { NE_QCASE(_Float16, float) }
    if (in_dt == 2 && out_dt == 2) { NE_QCASE(_Float16, _Float16) }
#undef NE_QCASE
    return hipErrorInvalidValue;
}

}  // namespace ne
