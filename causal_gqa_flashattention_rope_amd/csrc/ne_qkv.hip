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
    const int l = lane_id(), w = threadIdx.x >> 6;
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
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, c = l & 31;
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
            if (qk && rope) {
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

namespace {
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
    const int grid = (a.M + 255) / 256 * (a.N / 128);
    hipLaunchKernelGGL((qkv_rope_kernel<TI, TO, D, NE_QKV_BK>), dim3(grid), dim3(256), 0, s, a);
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
