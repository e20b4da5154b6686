// ne_common.hpp -- gfx950 building blocks shared by the attention kernels.
//
// MFMA lane layouts used throughout (wave of 64 lanes, h = lane / 32, c = lane % 32):
//   32x32x16 f16  : A[i][k] with i = c, k = 8h + j (j = 0..7);  B[k][n] with n = c, k = 8h + j;
//   32x32x2  f32  : A[i][k] with i = c, k = h;                   B[k][n] with n = c, k = h;
//   both          : C[m][n] register r (0..15) holds m = 8*(r/4) + 4h + (r%4), n = c.
// So a 32x32 accumulator gives each lane one output column and 16 rows in four runs of
// four consecutive rows.  When such an accumulator (over 32 "rows") is fed back as the
// contraction operand of the next product, its k index is a permutation of the rows:
//   f16: k-step kk covers rows 16kk..16kk+15; k = 8h + j  <->  row 16kk + 8*(j/4) + 4h + (j%4)
//   f32: k-step s (0..15 per 32 rows)        ; k = h      <->  row 8*(s/4) + 4h + (s%4)
// and the other operand is read in that same row order.
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane i element j is
// element (i % 4) of the 8 bytes addressed by source lane 4j + i/4.  Giving source lane s the
// address of row (r0 + s/4), columns (c0 + 4(s%4) .. +3) of a row-major 16-bit tile hands
// output lane i the four values tile[r0 + j][c0 + i], j = 0..3: a transposed read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ne {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_tr __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_tr* lds_tr_ptr;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Starting value of a running row maximum: finite, so exp2(-inf - kMFloor) = 0 for masked scores
// and exp2(kMFloor - m) = 0 when a real maximum m replaces it.
constexpr float kMFloor = -1.0e30f;

// QK norm: the factor gain / sqrt(mean(x^2) + eps) of a row of D elements whose squares sum to ss.
__device__ __forceinline__ float qk_factor(float ss, int D, float gain, float eps) {
    return gain / sqrtf(ss / (float)D + eps);
}
// Sum of squares of a row of D elements (16-byte loads), read whole by the calling thread.
template <typename TI>
__device__ __forceinline__ float row_sumsq(const TI* row, int D) {
    float ss = 0.f;
    if constexpr (sizeof(TI) == 4) {
        for (int d = 0; d < D; d += 4) {
            const floatx4 x = *reinterpret_cast<const floatx4*>(row + d);
            ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        }
    } else {
        typedef TI v8 __attribute__((ext_vector_type(8)));
        for (int d = 0; d < D; d += 8) {
            const v8 x = *reinterpret_cast<const v8*>(row + d);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += (float)x[e] * (float)x[e];
        }
    }
    return ss;
}
// Sum over the n consecutive lanes (n a power of two dividing 64) that hold one row.
__device__ __forceinline__ float sum_lanes(float x, int n) {
    for (int off = 1; off < n; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Query t sees key j iff t - W < j <= t (W = the window, 1..T; W = T is the causal prefix).
__device__ __forceinline__ bool visible(int j, int t, int W) { return (unsigned)(t - j) < (unsigned)W; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The wave index within the workgroup, read into a scalar register: every value derived from it
// (role, row half, fill counts) is then wave-uniform to the compiler, so branches on it are
// scalar branches and its arithmetic stays out of the vector registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---- storage element conversions ------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// ---- cross-lane ---------------------------------------------------------------------------
// v_permlane32_swap(vdst, vsrc) exchanges lanes 32..63 of vdst with lanes 0..31 of vsrc.  With
// the same value in both operands, each lane ends up holding its own value in one result and
// its partner's (lane l ^ 32) in the other, so max/sum of the pair combine the two halves and
// give both halves bit-identical results.
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Four consecutive elements base[off .. off + 3] of an array of dtype dt (0 f32, 1 bf16, 2 f16).
__device__ __forceinline__ floatx4 load4_dt(const void* base, size_t off, int dt) {
    if (dt == 0) return *reinterpret_cast<const floatx4*>((const float*)base + off);
    if (dt == 1) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 v = *reinterpret_cast<const bf16x4*>((const __bf16*)base + off);
        return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
    const half4v v = *reinterpret_cast<const half4v*>((const _Float16*)base + off);
    return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// Eight consecutive elements base[off .. off + 7] of a 16-bit array (dt 1 bf16, 2 f16) as fp16.
__device__ __forceinline__ half8 load8_f16(const void* base, size_t off, int dt) {
    if (dt == 1) {
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        const bf16x8 v = *reinterpret_cast<const bf16x8*>((const __bf16*)base + off);
        half8 r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (_Float16)(float)v[e];
        return r;
    }
    return *reinterpret_cast<const half8*>((const _Float16*)base + off);
}

// QK-norm backward of one row held in the 32x32 accumulator layout: lane (h, c) holds the values at
// d = 32 db + 8 q4 + 4 h + e (the other half of the row in lane c ^ 32, which must be active too).
// On entry y is the gradient with respect to the normalised row gain * rho * x, on return with
// respect to x: gain * rho * (y - x * rho^2 * (y . x) / D).  x = base[off ..] in dtype dt.
template <int NDB>
__device__ __forceinline__ void qk_norm_bwd_row(floatx16 (&y)[NDB], const void* base, size_t off, int dt, float rho,
                                                float gain, int h) {
    constexpr int D = 32 * NDB;
    float dot = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const floatx4 x = load4_dt(base, off + 32 * db + 8 * q4 + 4 * h, dt);
#pragma unroll
            for (int e = 0; e < 4; ++e) dot += y[db][4 * q4 + e] * x[e];
        }
    dot = sum_halves(dot);
    const float c1 = gain * rho, c2 = rho * rho * dot / (float)D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const floatx4 x = load4_dt(base, off + 32 * db + 8 * q4 + 4 * h, dt);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[db][4 * q4 + e] = c1 * (y[db][4 * q4 + e] - x[e] * c2);
        }
}

// The same with the row's values already loaded: xr[db][q4] holds the 16-bit elements
// d = 32 db + 8 q4 + 4 h .. + 3 (dt 1 bf16, 2 f16) as raw bits.
template <int NDB>
__device__ __forceinline__ void qk_norm_bwd_row_raw16(floatx16 (&y)[NDB], const uint2 (&xr)[NDB][4], int dt, float rho,
                                                      float gain) {
    constexpr int D = 32 * NDB;
    auto x4 = [&](int db, int q4) {
        if (dt == 1) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const bf16x4 v = __builtin_bit_cast(bf16x4, xr[db][q4]);
            return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
        }
        const half4v v = __builtin_bit_cast(half4v, xr[db][q4]);
        return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    };
    float dot = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const floatx4 x = x4(db, q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) dot += y[db][4 * q4 + e] * x[e];
        }
    dot = sum_halves(dot);
    const float c1 = gain * rho, c2 = rho * rho * dot / (float)D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const floatx4 x = x4(db, q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[db][4 * q4 + e] = c1 * (y[db][4 * q4 + e] - x[e] * c2);
        }
}

// ---- MFMA operand traits ----------------------------------------------------------------
template <typename OP> struct Mma;

template <> struct Mma<_Float16> {
    typedef half8 frag;
    static constexpr int K = 16;  // contraction elements per instruction
    __device__ __forceinline__ static floatx16 mma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    // Fragment along a contiguous contraction run (row-major operand): k-step ks of a row.
    __device__ __forceinline__ static frag row_frag(const _Float16* row, int ks, int h, int /*len*/) {
        return *reinterpret_cast<const half8*>(row + 16 * ks + 8 * h);
    }
};

template <> struct Mma<float> {
    typedef float frag;
    static constexpr int K = 2;
    __device__ __forceinline__ static floatx16 mma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // Contraction index of k-step ks for lane half h is 2ks + h (the instruction's own order).
    __device__ __forceinline__ static frag row_frag(const float* row, int ks, int h, int /*len*/) {
        return row[2 * ks + h];
    }
};

// Row (within a 32-row block) that accumulator register r of lane half h holds.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Contraction operand built from a 32x32 accumulator (rows = contraction index).
// f16: k-step c (0/1) of the 32-row block packs registers 8c..8c+7.
__device__ __forceinline__ half8 pack_frag_f16(const floatx16& acc, int c) {
    half8 f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (_Float16)acc[8 * c + j];
    return f;
}

// A wave-uniform global pointer moved into SGPRs: readfirstlane of each 32-bit half.  The builtin
// returns int, so each half is widened as unsigned (a sign-extended low half would corrupt the
// upper half of the address).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* sgpr_global_ptr(const void* p) {
    const uint64_t v = (uint64_t)p;
    const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)v);
    const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
    return (__attribute__((address_space(1))) T*)((hi << 32) | lo);
}

// ---- swizzled LDS tiles --------------------------------------------------------------------
// A tile of rows x D elements is stored densely (row = D * sizeof(OP) bytes) with the 16-byte
// chunks of row r permuted: chunk c lives in slot c ^ swz(r).  The permutations are chosen so
// that the two read patterns hit distinct banks: 16 lanes reading one 16-byte chunk from 16
// consecutive rows (row fragments), and 32 lanes reading 8 bytes each from 4 consecutive rows
// x 4 chunks (transposed reads).  Dense rows let a wave fill 1 KiB of the tile per
// global_load_lds_dwordx4 (lane i writes bytes 16i..16i+15 of that kilobyte).
template <typename OP, int D>
struct Tile {
    static constexpr int ROWB = D * (int)sizeof(OP);  // bytes per row
    static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
    static constexpr int EPC = 16 / (int)sizeof(OP);  // elements per chunk
    __device__ __forceinline__ static constexpr int swz(int r) {
        if constexpr (CPR == 16) return 4 * (r & 3) + ((r >> 2) & 3);
        else if constexpr (CPR == 8) return ((r >> 2) & 3) | (((r >> 1) & 1) << 2);
        else if constexpr (CPR == 4) return (r >> 2) & 3;
        else return r & (CPR - 1);                     // fp32 tiles: 8, 16 or 32 chunks
    }
    // byte offset of element e of row r
    __device__ __forceinline__ static int off(int r, int e) {
        return r * ROWB + (((e / EPC) ^ swz(r)) << 4) + (e % EPC) * (int)sizeof(OP);
    }
    __device__ __forceinline__ static const OP* ptr(const OP* base, int r, int e) {
        return reinterpret_cast<const OP*>(reinterpret_cast<const char*>(base) + off(r, e));
    }
};

// Direct global->LDS loads (global_load_lds_dwordx4 / _dword): each lane of the wave fetches
// 16 (or 4) bytes from its own global address into LDS bytes [16 lane, 16 lane + 16) (or
// [4 lane, 4 lane + 4)) above the wave-uniform base in M0.  They are issued from inline assembly
// so that the compiler does not guard every later LDS read with a wait for all outstanding
// loads (it cannot tell the ring stages apart); the kernels wait explicitly with
// lds_fill_wait / lds_fill_wait_keep, which count this wave's outstanding vector-memory
// operations.  No compiler-generated code in these kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane(
        (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ void dma16(const void* g, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(g), "s"(lds_base)
                 : "memory", "m0");
}
// Same with the global address split into a wave-uniform 64-bit base (SGPRs) and a per-lane
// 32-bit byte offset (one VGPR instead of a 64-bit address per load).
__device__ __forceinline__ void dma16_s(unsigned voff, const void* sbase, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase),
                 "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(g), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Copy rows [n0, n0 + ROWS) of a dense [nrows][D] array into a swizzled LDS tile with direct
// global->LDS loads issued by the NW waves of the block.  Rows at or past nrows are filled from
// row nrows - 1 (finite data that the callers mask out).  src must be wave-uniform and
// nrows * D * sizeof(OP) below 2^31 (byte offsets are 32-bit).  Completion: s_waitcnt vmcnt(0)
// then a barrier (ne::lds_fill_wait).
template <typename OP, int D, int ROWS, int NW>
__device__ __forceinline__ void lds_fill(OP* tile, const OP* src, int n0, int nrows) {
    using TL = Tile<OP, D>;
    constexpr int CHUNKS = ROWS * TL::CPR;
    constexpr int WL = CHUNKS / 64;                    // 1 KiB wave loads per tile
    static_assert(CHUNKS % 64 == 0, "tile must be a whole number of wave loads");
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < (WL + NW - 1) / NW; ++i) {
        const int j = i * NW + w;                      // wave load index (uniform per wave)
        if (WL % NW != 0 && j >= WL) break;
        const int q = 64 * j + l;                      // LDS slot index of this lane
        const int r = q / TL::CPR, p = q % TL::CPR;
        const int gr = min(n0 + r, nrows - 1);
        const unsigned off = (unsigned)((gr * D + (p ^ TL::swz(r)) * TL::EPC) * (int)sizeof(OP));
        dma16_s(off, src, lds_addr(reinterpret_cast<char*>(tile) + 1024 * j));
    }
}

// s_waitcnt immediate (gfx9 layout): vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Everything this wave issued to memory has completed (also tells the compiler's wait
// tracking that no earlier load is pending, so it adds no waits of its own inside the loops).
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ void lds_fill_wait() {
    wait_vmcnt<0>();
    __syncthreads();
}

// Number of direct loads one wave issues in lds_fill<OP, D, ROWS, NW>.
template <typename OP, int D, int ROWS, int NW>
__device__ __forceinline__ int lds_fill_count(int w) {
    constexpr int WL = ROWS * Tile<OP, D>::CPR / 64;
    return WL / NW + (w < WL % NW ? 1 : 0);
}

// Wait until at most n of this wave's vector-memory operations are outstanding (they complete
// in order), then barrier: the fills issued before the n most recent loads have landed.
__device__ __forceinline__ void lds_fill_wait_keep(int n) {
    switch (n) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 12: wait_vmcnt<12>(); break;
        default: wait_vmcnt<0>(); break;
    }
    __syncthreads();
}

// The same for a wave that issued n = 0, 16 or 32 other vector-memory operations (atomic adds)
// after its share of the fill being waited for.
__device__ __forceinline__ void lds_fill_wait_keep_atomics(int n) {
    if (n == 32) wait_vmcnt<32>();
    else if (n == 16) wait_vmcnt<16>();
    else wait_vmcnt<0>();
    __syncthreads();
}

// Transposed f16 fragment from a swizzled tile (same meaning as tr_frag_f16).
template <int D>
__device__ __forceinline__ half8 tr_frag_f16_sw(const _Float16* tile, int kk, int col0) {
    using TL = Tile<_Float16, D>;
    const int l = lane_id();
    const int g = l >> 4, s = l & 15, h = l >> 5;
    const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
    const int r1 = 16 * kk + 4 * h + (s >> 2);
    fp16x4_tr lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr_ptr)TL::ptr(tile, r1, col));
    fp16x4_tr hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr_ptr)TL::ptr(tile, r1 + 8, col));
    half8 f;
    half4v a = __builtin_bit_cast(half4v, lo), b = __builtin_bit_cast(half4v, hi);
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
}

// f32 column fragment from a swizzled tile: lane (h, c) reads tile[32mb + acc_row(s, h)][col0 + c].
template <int D>
__device__ __forceinline__ float tr_frag_f32_sw(const float* tile, int mb, int s, int col0) {
    const int l = lane_id();
    return *Tile<float, D>::ptr(tile, 32 * mb + acc_row(s, l >> 5), col0 + (l & 31));
}

// ---- transposed value tiles (16-bit operands) ----------------------------------------------
// V'^T of one (batch, KV head) group is stored as D rows of Tp keys (Tp = T rounded up to 64),
// with the keys of every aligned group of 16 stored in the order 0-3, 8-11, 4-7, 12-15.  That is
// the order in which a 32x32 accumulator hands its rows to the next product as contraction
// index (pack_frag_f16), so the 16 bytes at key position 16 kk + 8 h of a row are exactly the A
// operand a lane of half h needs for k-step kk of O^T += V^T P^T.  An LDS tile holds BN keys of
// every row (BN = 32 or 64); chunk c of row r sits in slot c ^ ((r / (16 / CPR)) % CPR), CPR =
// BN / 8 chunks per row, so the 16 lanes of one read touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ constexpr int vt_key_of_pos(int pos) {
    return (pos & ~15) + 8 * ((pos >> 2) & 1) + 4 * ((pos >> 3) & 1) + (pos & 3);
}
template <int BN>
struct VtTile {
    static constexpr int CPR = BN / 8, RPG = 16 / CPR;  // chunks per row, rows per 256 bytes
    __device__ __forceinline__ static constexpr int slot(int r, int c) { return c ^ ((r / RPG) % CPR); }
};
template <int BN>
__device__ __forceinline__ half8 vt_frag(const _Float16* tile, int row, int kk, int h) {
    return *reinterpret_cast<const half8*>(reinterpret_cast<const char*>(tile) + row * (2 * BN) +
                                           (VtTile<BN>::slot(row, 2 * kk + h) << 4));
}
template <int D, int BN, int NW>
__device__ __forceinline__ constexpr int lds_fill_vt_count(int w) {
    return (D * BN / 512) / NW + (w < (D * BN / 512) % NW ? 1 : 0);
}
// Keys [n0, n0 + BN) of all D rows of a transposed value array (row stride Tp) into a tile.
template <int D, int BN, int NW>
__device__ __forceinline__ void lds_fill_vt(_Float16* tile, const _Float16* src, int n0, int Tp) {
    constexpr int CPR = BN / 8, WL = D * CPR / 64;     // 1 KiB wave loads per tile
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < (WL + NW - 1) / NW; ++i) {
        const int j = i * NW + w;
        if (WL % NW != 0 && j >= WL) break;
        const int q = 64 * j + l;
        const int r = q / CPR, sl = q % CPR;
        const _Float16* g = src + (size_t)r * Tp + n0 + 8 * VtTile<BN>::slot(r, sl);
        dma16(g, lds_addr(reinterpret_cast<char*>(tile) + 1024 * j));
    }
}

// lds_fill and lds_fill_vt with the tile given as a wave-uniform 32-bit LDS byte address (no
// generic-pointer round trip per load).
template <typename OP, int D, int ROWS, int NW>
__device__ __forceinline__ void lds_fill_at(unsigned tile, const OP* src, int n0, int nrows) {
    using TL = Tile<OP, D>;
    constexpr int CHUNKS = ROWS * TL::CPR;
    constexpr int WL = CHUNKS / 64;
    static_assert(CHUNKS % 64 == 0, "tile must be a whole number of wave loads");
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < (WL + NW - 1) / NW; ++i) {
        const int j = i * NW + w;
        if (WL % NW != 0 && j >= WL) break;
        const int q = 64 * j + l;
        const int r = q / TL::CPR, p = q % TL::CPR;
        const int gr = min(n0 + r, nrows - 1);
        const unsigned off = (unsigned)((gr * D + (p ^ TL::swz(r)) * TL::EPC) * (int)sizeof(OP));
        dma16_s(off, src, __builtin_amdgcn_readfirstlane(tile + 1024u * (unsigned)j));
    }
}
template <int D, int BN, int NW>
__device__ __forceinline__ void lds_fill_vt_at(unsigned tile, const _Float16* src, int n0, int Tp) {
    constexpr int CPR = BN / 8, WL = D * CPR / 64;
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < (WL + NW - 1) / NW; ++i) {
        const int j = i * NW + w;
        if (WL % NW != 0 && j >= WL) break;
        const int q = 64 * j + l;
        const int r = q / CPR, sl = q % CPR;
        // per-lane byte offset (the same for every tile; below D * Tp * 2 < 2^32) from the tile's
        // uniform base src + n0
        const unsigned off = ((unsigned)r * (unsigned)Tp + 8u * (unsigned)VtTile<BN>::slot(r, sl)) * 2u;
        dma16_s(off, src + n0, __builtin_amdgcn_readfirstlane(tile + 1024u * (unsigned)j));
    }
}

// Row fragment from a swizzled tile (k-step ks of row r), both operand types.
template <typename OP, int D>
__device__ __forceinline__ typename Mma<OP>::frag row_frag_sw(const OP* tile, int r, int ks, int h) {
    if constexpr (sizeof(OP) == 2) return *reinterpret_cast<const half8*>(Tile<OP, D>::ptr(tile, r, 16 * ks + 8 * h));
    else return *Tile<OP, D>::ptr(tile, r, 2 * ks + h);
}

// ---- coalesced row stores through LDS ------------------------------------------------------
// A wave holds 32 rows x D outputs in the 32x32 accumulator layout (lane (h, c) holds row c,
// columns 32db + acc_row(r, h)).  store_rows writes them, times `mul`, as whole rows: first
// into a per-wave LDS scratch of 32 rows (16-byte chunks of row r XOR-permuted by r, so the
// 32 lanes writing one chunk column hit distinct banks), then 64 lanes store two contiguous
// rows per instruction.  row_ptr(i) gives the destination of row i (nullptr: skip).
template <typename T> struct Pack4;
template <> struct Pack4<float> { typedef floatx4 type; };
template <> struct Pack4<_Float16> { typedef half4v type; };
template <> struct Pack4<__bf16> { typedef __bf16 type __attribute__((ext_vector_type(4))); };

template <typename TOUT, int D, typename RowPtr>
__device__ __forceinline__ void store_rows(const floatx16 (&acc)[D / 32], float mul, char* scratch,
                                           RowPtr row_ptr) {
    constexpr int RB = D * (int)sizeof(TOUT);  // bytes per row
    constexpr int CPR = RB / 16;               // 16-byte chunks per row
    const int l = lane_id(), h = l >> 5, c = l & 31;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int byte = (32 * db + 8 * q4 + 4 * h) * (int)sizeof(TOUT);
            const int off = c * RB + (((byte >> 4) ^ (c % CPR)) << 4) + (byte & 15);
            typename Pack4<TOUT>::type v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = from_f32<TOUT>(acc[db][4 * q4 + e] * mul);
            *reinterpret_cast<typename Pack4<TOUT>::type*>(scratch + off) = v;
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
        const int idx = 64 * i + l;
        const int row = idx / CPR, ch = idx % CPR;
        const uint4 v = *reinterpret_cast<const uint4*>(scratch + row * RB + ((ch ^ (row % CPR)) << 4));
        TOUT* dst = row_ptr(row);
        if (dst) *reinterpret_cast<uint4*>(reinterpret_cast<char*>(dst) + ch * 16) = v;
    }
}

// ---- hand-off between the workgroups of one split row block --------------------------------
// Every piece of a split block counts itself in cnt[0] when its products are done; the pieces
// that arrive before the last leave their partial result in the workspace, then count it in
// cnt[1] (after an agent-scope release: the partial is visible to every XCD).  The last piece
// to arrive waits until cnt[1] shows the others' partials (they arrived before it, so they are
// running and only have stores left; the wait is bounded anyway) and acquires them.  Every
// thread of the workgroup makes the calls; sh: two words of LDS.
__device__ __forceinline__ unsigned split_arrive(unsigned* cnt, unsigned* sh) {
    if (threadIdx.x == 0) *sh = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return *sh;
}
__device__ __forceinline__ void split_publish(unsigned* cnt) {
    wait_all();             // this wave's partial stores are done
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}
// true when all n partials were seen (false after 2^20 polls, well under a second: the caller poisons its output)
__device__ __forceinline__ bool split_collect(unsigned* cnt, unsigned n, unsigned* sh) {
    if (threadIdx.x == 0) {
        unsigned it = 0;
        bool ok = true;
        while (__hip_atomic_load(cnt + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
            __builtin_amdgcn_s_sleep(2);
            if (++it >= (1u << 20)) { ok = false; break; }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        sh[1] = ok ? 1u : 0u;
    }
    __syncthreads();
    return sh[1] != 0u;
}

// ---- small vector stores of four consecutive output elements -----------------------------
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<floatx4*>(p) = floatx4{a, b, c, d};
}
__device__ __forceinline__ void store4(_Float16* p, float a, float b, float c, float d) {
    *reinterpret_cast<half4v*>(p) = half4v{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}

}  // namespace ne
