// ne_decode.hip -- attention of a few new tokens against a key/value cache (decode and chunked
// prefill), 16-bit operands, gfx950.
//
// The cache (one caller-owned buffer, ne_kv_cache_bytes) holds, per (batch, KV head) group g, its
// Tcap / 32 tiles of 32 keys, each 128 D bytes in the order one wave loads them (CacheTile):
//   K' block: for load ks < D / 16 and lane l < 64, 16 bytes: fp16(R_p(k)) of key l % 32 of the
//             tile, elements d = 16 ks + 8 (l / 32) .. + 7 (each key rotated once, at its own
//             absolute position p): the A operand of S^T = K' Q~^T for k-step ks;
//   V' block: for load (kk < 2, db < D / 32) and lane l, 16 bytes: fp16(v) at d = 32 db + l % 32 of
//             the 8 keys 16 kk + vt_key_of_pos(8 (l / 32) + j), j < 8: the A operand of
//             O^T += V'^T P^T for k-step kk, in the order the S^T accumulator hands P over.
// Every 16-byte load of the decode kernel is thus one lane's part of a contiguous 1 KiB.  With the
// half-split rotary pairs (i, i + D/2) the key's elements i and i + D/2 take dimensions 2i and 2i + 1
// of this layout, and the decode gathers its queries in the same order (scores are sums over them).
//
// Decode is bound by reading the cache, which no two workgroups share, so the kernels stream it
// from HBM straight into registers (no LDS staging) and spread every group's keys over many
// workgroups (split-KV); a second kernel merges the partial results by the log-sum-exp rule.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ne_common.hpp"
#include "ne_launch.hpp"

namespace ne {

namespace {

// cos and sin of p * theta (theta_i = base^(-2i/D), computed by the host in double precision): the
// phase is formed and reduced to [-pi, pi] in double precision
// (two-term 2 pi), so the single-precision sincos sees a small argument at any position.
__device__ __forceinline__ float2 rope_cs(int p, double theta) {
    constexpr double kTwoPiHi = 6.283185307179586;
    constexpr double kTwoPiLo = 2.4492935982947064e-16;
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double phi = (double)p * theta;
    const double n = rint(phi * kInvTwoPi);
    const double r = fma(-n, kTwoPiLo, fma(-n, kTwoPiHi, phi));
    float s, c;
    sincosf((float)r, &s, &c);
    return make_float2(c, s);
}

// Offsets (in fp16 elements) inside a group's cache of the 16-byte unit a lane loads.
template <int D>
struct CacheTile {
    static constexpr int KS = D / 16, NDB = D / 32;
    static constexpr size_t ELEMS = (size_t)64 * D;    // elements per 32-key tile (K' and V' blocks)
    __device__ __forceinline__ static size_t k_unit(int tile, int ks, int lane) {
        return tile * ELEMS + (size_t)(ks * 64 + lane) * 8;
    }
    __device__ __forceinline__ static size_t v_unit(int tile, int kk, int db, int lane) {
        return tile * ELEMS + (size_t)32 * D + (size_t)((kk * NDB + db) * 64 + lane) * 8;
    }
};

template <typename TI>
__device__ __forceinline__ void load8_in(const TI* p, float (&x)[8]) {
    typedef TI v8 __attribute__((ext_vector_type(8)));
    const v8 a = *reinterpret_cast<const v8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
}

// Tokens already in the cache, clamped so that the n new ones fit: [0, Tcap - n].
__device__ __forceinline__ int cache_len(const int* lens, int b, int n, int Tcap) {
    return min(max(lens[b], 0), Tcap - n);
}

}  // namespace

// =====================================================================================
// Append: tokens i < Tn of k_new / v_new go to positions len_b + i of their group.
// grid (ceil(Tn / 16), B * Hkv), 256 threads.  Keys: one thread per (token, 8-element chunk),
// rotated in fp32 with the cos/sin of the absolute position, one 16-byte store.  Values: staged
// through LDS and written in the tile order, one fp16 element per thread.
// =====================================================================================
template <typename TI, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
    constexpr int TB = 16, CPR = D / 8;
    __shared__ float vs[TB][D + 1];
    const int grp = blockIdx.y, b = grp / a.Hkv, hkv = grp % a.Hkv;
    const int t0 = blockIdx.x * TB, Tn = a.Tn, Tcap = a.Tcap;
    const int len = cache_len(a.lens, b, Tn, Tcap);
    const bool rope = a.rope_base > 0.0;
    using CT = CacheTile<D>;
    _Float16* gc = (_Float16*)a.cache + (size_t)grp * Tcap * D * 2;   // this group's tiles
    for (int idx = threadIdx.x; idx < TB * CPR; idx += 256) {
        const int tl = idx / CPR, chunk = idx % CPR, t = t0 + tl;
        const size_t in_off = (((size_t)b * Tn + min(t, Tn - 1)) * a.Hkv + hkv) * D + chunk * 8;
        float x[8];
        if (a.half) {   // half-split pairs: slot 2i takes element i, slot 2i + 1 element i + D/2
            const TI* row = (const TI*)a.k + (in_off - chunk * 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[2 * q] = to_f32(row[chunk * 4 + q]);
                x[2 * q + 1] = to_f32(row[D / 2 + chunk * 4 + q]);
            }
        } else {
            load8_in((const TI*)a.k + in_off, x);
        }
        float fac = 1.f;  // QK norm of this key row (its chunks sit in consecutive lanes)
        if (a.qkn.on) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
            fac = qk_factor(sum_lanes(ss, CPR), D, a.qkn.gain, a.qkn.eps);
        }
        if (t >= Tn) continue;
        const int p = len + t;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= fac;
        if (rope) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float2 r = rope_cs(p, a.theta[chunk * 4 + q]);
                const float u = x[2 * q], v = x[2 * q + 1];
                x[2 * q] = u * r.x - v * r.y;
                x[2 * q + 1] = u * r.y + v * r.x;
            }
        }
        half8 out;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = (_Float16)x[e];
        // elements 8 chunk .. 8 chunk + 7 of key p: load ks = chunk / 2 of lane 32 (chunk & 1) + p % 32
        *reinterpret_cast<half8*>(gc + CT::k_unit(p >> 5, chunk >> 1, 32 * (chunk & 1) + (p & 31))) = out;
        float y[8];
        load8_in((const TI*)a.v + in_off, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) vs[tl][chunk * 8 + e] = y[e];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < TB * D; idx += 256) {
        const int tl = idx % TB, d = idx / TB, t = t0 + tl;
        if (t >= Tn) continue;
        const int p = len + t;
        // key p of its tile sits at position pos = vt_key_of_pos(p % 16) of k-step (p % 32) / 16
        // (the order is its own inverse): lane 32 (pos / 8) + d % 32, element pos % 8
        const int pos = vt_key_of_pos(p & 15);
        gc[CT::v_unit(p >> 5, (p >> 4) & 1, d >> 5, 32 * (pos >> 3) + (d & 31)) + (pos & 7)] = (_Float16)vs[tl][d];
    }
}

// =====================================================================================
// Split-KV attention.  grid (nsplit * nrb * B * Hkv), 256 threads = 4 waves; a workgroup takes
// one block of 32 flattened query rows (row R = t * G + hh of one group: the order of one token's
// heads) and one of nsplit equal slices of the key range those rows see ([first key of the window
// of its first row, rounded down to 32], last row's position]); its 4 waves take the slice's
// 32-key tiles in turn.  The workgroup first rotates its query rows at their absolute positions
// (theta_i from the host in double precision, the phase reduced in double) and stages them in
// LDS as fp16 times scale * log2 e.  Per tile a wave loads its K' and V'^T fragments from HBM
// straight into registers, one tile ahead of the one it computes: S^T = K' Q~^T (keys on lanes,
// one query row per lane column), masks (causal, window, cache end), updates its running max and
// sum (log2 units) and adds V'^T P^T.  The waves merge in LDS in a fixed order and the workgroup
// writes its partial (unnormalised O over its keys, max m, sum l) for the valid rows.
// =====================================================================================
template <typename TI, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_kernel(DecodeArgs a) {
    using M = Mma<_Float16>;
    constexpr int KS = D / 16, NDB = D / 32, NWV = 4, CPR = D / 8;
    __shared__ __attribute__((aligned(16))) _Float16 sq[32][D + 8];
    __shared__ float so[32][D + 4];
    __shared__ float sm[NWV][32];
    __shared__ float sl[NWV][32];
    const int nsplit = a.nsplit, nrb = a.nrb;
    const int s = blockIdx.x % nsplit, rb = (blockIdx.x / nsplit) % nrb, g = blockIdx.x / (nsplit * nrb);
    const int b = g / a.Hkv, hkv = g % a.Hkv;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, c = l & 31;
    const int Tq = a.Tq, G = a.G, TqG = Tq * G, Tcap = a.Tcap, W = a.window;
    const int len = cache_len(a.lens, b, Tq, Tcap), L = len + Tq;

    const int R0 = rb * 32, R = R0 + c;
    const int nvalid = min(32, TqG - R0);
    const int p_lane = len + min(R, TqG - 1) / G;                 // this lane's query position
    const int p_min = len + R0 / G, p_max = len + (R0 + nvalid - 1) / G;
    const int Kb = max(0, p_min - W + 1) & ~31, Ke = p_max + 1;    // key range of the row block
    const int CH = ((Ke - Kb + nsplit - 1) / nsplit + 31) & ~31;  // keys per split
    const int k0 = Kb + s * CH, k1 = min(Ke, k0 + CH);

    using CT = CacheTile<D>;
    const _Float16* gc = (const _Float16*)a.cache + (size_t)g * Tcap * D * 2;   // this group's tiles

    // first tile's loads, in flight while the queries are prepared
    half8 kf[KS], vf[2][NDB];
    auto load_tile = [&](int k) {
        // k is a multiple of 32 below k1 <= Tcap (a multiple of 64): keys k .. k + 31 are in the cache
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const half8*>(gc + CT::k_unit(k >> 5, ks, l));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < NDB; ++db) vf[kk][db] = *reinterpret_cast<const half8*>(gc + CT::v_unit(k >> 5, kk, db, l));
    };
    int k = k0 + 32 * w;
    if (k < k1) load_tile(k);

    // q~ rows of this block into LDS (rows past the valid ones are zeros)
    const bool rope = a.rope_base > 0.0;
    for (int idx = tid; idx < 32 * CPR; idx += 256) {
        const int r = idx / CPR, chunk = idx % CPR;
        half8 out = half8{};
        const int Rr = R0 + min(r, nvalid - 1), t = Rr / G, hq = hkv * G + (Rr - t * G);
        float x[8];
        const TI* qrow = (const TI*)a.q + (((size_t)b * Tq + t) * a.Hq + hq) * D;
        if (a.half) {   // half-split pairs, in the slot order of the cached keys
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[2 * q] = to_f32(qrow[chunk * 4 + q]);
                x[2 * q + 1] = to_f32(qrow[D / 2 + chunk * 4 + q]);
            }
        } else {
            load8_in(qrow + chunk * 8, x);
        }
        float mul = a.qscale;  // times the QK norm of this query row (its chunks in consecutive lanes)
        if (a.qkn.on) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
            mul *= qk_factor(sum_lanes(ss, CPR), D, a.qkn.gain, a.qkn.eps);
        }
        if (r < nvalid) {
            if (rope) {
                const int p = len + t;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float2 cs = rope_cs(p, a.theta[chunk * 4 + q]);
                    const float u = x[2 * q], v = x[2 * q + 1];
                    x[2 * q] = u * cs.x - v * cs.y;
                    x[2 * q + 1] = u * cs.y + v * cs.x;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = (_Float16)(x[e] * mul);
        }
        *reinterpret_cast<half8*>(&sq[r][chunk * 8]) = out;
    }
    __syncthreads();
    half8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const half8*>(&sq[c][16 * ks + 8 * h]);

    floatx16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = floatx16{};
    float m_run = kMFloor, l_run = 0.f;

    for (; k < k1; k += 32 * NWV) {
        floatx16 sc = floatx16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc = M::mma(kf[ks], qf[ks], sc);
        half8 vc[2][NDB];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < NDB; ++db) vc[kk][db] = vf[kk][db];
        if (k + 32 * NWV < k1) load_tile(k + 32 * NWV);   // next tile in flight during this one
        if (k + 31 >= L) {  // the cache ends inside this tile: stale or unwritten values there
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (k + 16 * kk + vt_key_of_pos(8 * h + j) >= L)
#pragma unroll
                        for (int db = 0; db < NDB; ++db) vc[kk][db][j] = (_Float16)0.f;
        }
        float mx = kMFloor;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (!visible(k + acc_row(r, h), p_lane, W)) sc[r] = -INFINITY;
            mx = fmaxf(mx, sc[r]);
        }
        mx = max_halves(mx);
        if (mx > m_run) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m_run = mx;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sc[r] = __builtin_amdgcn_exp2f(sc[r] - m_run);
            l_run += sc[r];
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const half8 pf = pack_frag_f16(sc, kk);
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] = M::mma(vc[kk][db], pf, oacc[db]);
        }
    }
    l_run = sum_halves(l_run);

    // merge the four waves: common max, then O and l added in wave order
    if (h == 0) {
        sm[w][c] = m_run;
        sl[w][c] = l_run;
    }
    __syncthreads();
    float mall = sm[0][c];
#pragma unroll
    for (int i = 1; i < NWV; ++i) mall = fmaxf(mall, sm[i][c]);
    const float f = __builtin_amdgcn_exp2f(m_run - mall);  // 1 when both are the floor
    for (int i = 0; i < NWV; ++i) {
        if (w == i) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float* dst = &so[c][32 * db + acc_row(r, h)];
                    *dst = (i == 0 ? 0.f : *dst) + oacc[db][r] * f;
                }
        }
        __syncthreads();
    }
    // partials of the valid rows: O [row][D], then (m, l) per row
    const size_t slot = ((size_t)g * nrb + rb) * nsplit + s;
    float* po = a.part_o + slot * 32 * D;
    for (int idx = tid; idx < nvalid * (D / 4); idx += 256) {
        const int row = idx / (D / 4), q4 = idx % (D / 4);
        *reinterpret_cast<floatx4*>(po + row * D + 4 * q4) =
            floatx4{so[row][4 * q4], so[row][4 * q4 + 1], so[row][4 * q4 + 2], so[row][4 * q4 + 3]};
    }
    if (tid < nvalid) {
        float mt = sm[0][tid];
        for (int i = 1; i < NWV; ++i) mt = fmaxf(mt, sm[i][tid]);
        float lsum = 0.f;
        for (int i = 0; i < NWV; ++i) lsum += sl[i][tid] * __builtin_amdgcn_exp2f(sm[i][tid] - mt);
        a.part_ml[slot * 64 + tid] = mt;
        a.part_ml[slot * 64 + 32 + tid] = lsum;
    }
}

// =====================================================================================
// Merge of the nsplit partials of every valid row: m = max m_s, l = sum l_s 2^(m_s - m),
// o = sum O_s 2^(m_s - m) / l, lse = ln 2 (m + log2 l).  grid (nrb * B * Hkv), 256 threads, one
// thread per (row, 4 consecutive d).  The splits are folded in index order, 16 at a time: the
// (m_s, l_s) and O_s of a chunk are loaded together (one memory round trip per chunk), then the
// running (m, l, O) is rescaled to the chunk's max and the chunk added.
// =====================================================================================
template <int D, typename TOUT>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
    constexpr int CK = 16;
    const int nsplit = a.nsplit, nrb = a.nrb;
    const int rb = blockIdx.x % nrb, g = blockIdx.x / nrb;
    const int b = g / a.Hkv, hkv = g % a.Hkv;
    const int Tq = a.Tq, G = a.G, TqG = Tq * G;
    const int R0 = rb * 32, nvalid = min(32, TqG - R0);
    const size_t slot0 = ((size_t)g * nrb + rb) * nsplit;
    for (int idx = threadIdx.x; idx < nvalid * (D / 4); idx += 256) {
        const int row = idx / (D / 4), q4 = idx % (D / 4);
        const float* ml = a.part_ml + slot0 * 64 + row;
        const float* src = a.part_o + (slot0 * 32 + row) * D + 4 * q4;
        float m = kMFloor, lsum = 0.f;
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < nsplit; s0 += CK) {
            float ms[CK], ls[CK];
            floatx4 xs[CK];
#pragma unroll
            for (int u = 0; u < CK; ++u) {
                if (s0 + u < nsplit) {
                    ms[u] = ml[(size_t)(s0 + u) * 64];
                    ls[u] = ml[(size_t)(s0 + u) * 64 + 32];
                    xs[u] = *reinterpret_cast<const floatx4*>(src + (size_t)(s0 + u) * 32 * D);
                } else {
                    ms[u] = kMFloor;
                    ls[u] = 0.f;
                    xs[u] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
            }
            float mc = m;
#pragma unroll
            for (int u = 0; u < CK; ++u) mc = fmaxf(mc, ms[u]);
            const float fa = __builtin_amdgcn_exp2f(m - mc);
            lsum *= fa;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= fa;
#pragma unroll
            for (int u = 0; u < CK; ++u) {
                const float f = __builtin_amdgcn_exp2f(ms[u] - mc);
                lsum += ls[u] * f;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += xs[u][e] * f;
            }
            m = mc;
        }
        const float inv = 1.f / lsum;
        const int R = R0 + row, t = R / G, hq = hkv * G + (R - t * G);
        store4((TOUT*)a.o + (((size_t)b * Tq + t) * a.Hq + hq) * D + 4 * q4, acc[0] * inv, acc[1] * inv,
               acc[2] * inv, acc[3] * inv);
        if (q4 == 0) a.lse[((size_t)b * a.Hq + hq) * Tq + t] = (m + __log2f(lsum)) * kLn2;
    }
}

// =====================================================================================
// Launchers.
// =====================================================================================
namespace {
struct DMarks {
    hipEvent_t const* ev;
    hipStream_t s;
    hipError_t rec(int j) const { return ev && ev[j] ? hipEventRecord(ev[j], s) : hipSuccess; }
};
#define NE_DTRY(x)                            \
    do {                                      \
        hipError_t e_ = (x);                  \
        if (e_ != hipSuccess) return e_;      \
    } while (0)

template <typename TI, typename TO, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s, hipEvent_t const* ev) {
    const DMarks m{ev, s};
    NE_DTRY(m.rec(0));
    hipLaunchKernelGGL((decode_split_kernel<TI, D>), dim3(a.nsplit * a.nrb * a.B * a.Hkv), dim3(256), 0, s, a);
    NE_DTRY(hipGetLastError());
    NE_DTRY(m.rec(1));
    NE_DTRY(m.rec(2));
    hipLaunchKernelGGL((decode_combine_kernel<D, TO>), dim3(a.nrb * a.B * a.Hkv), dim3(256), 0, s, a);
    NE_DTRY(hipGetLastError());
    return m.rec(3);
}

template <typename TI, int D>
hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((kv_append_kernel<TI, D>), dim3((a.Tn + 15) / 16, a.B * a.Hkv), dim3(256), 0, s, a);
    return hipGetLastError();
}
}  // namespace

#define NE_DDISPATCH(FN, ...)                                  \
    switch (D) {                                               \
        case 32: return FN<__VA_ARGS__, 32>(a, s);             \
        case 64: return FN<__VA_ARGS__, 64>(a, s);             \
        case 128: return FN<__VA_ARGS__, 128>(a, s);           \
        default: return hipErrorInvalidValue;                  \
    }

hipError_t launch_append(int in_dt, int D, const AppendArgs& a, hipStream_t s) {
    if (in_dt == 1) { NE_DDISPATCH(launch_append_t, __bf16) }
    if (in_dt == 2) { NE_DDISPATCH(launch_append_t, _Float16) }
    return hipErrorInvalidValue;
}

// ---- the decode without a caller workspace ---------------------------------------------------
// A file-scope device array holds the split partials for callers that cannot allocate.  Its name is
// a host-side stand-in: host code uses only the address hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev]() {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode(int in_dt, int out_dt, int D, const DecodeArgs& a, hipStream_t s, hipEvent_t const* ev) {
#define NE_DCASE(TI, TO)                                                   \
    switch (D) {                                                           \
        case 32: return launch_decode_t<TI, TO, 32>(a, s, ev);             \
        case 64: return launch_decode_t<TI, TO, 64>(a, s, ev);             \
        case 128: return launch_decode_t<TI, TO, 128>(a, s, ev);           \
        default: return hipErrorInvalidValue;                              \
    }
    if (in_dt == 1 && out_dt == 0) { NE_DCASE(__bf16, float) }
    if (in_dt == 1 && out_dt == 1) { NE_DCASE(__bf16, __bf16) }
    if (in_dt == 2 && out_dt == 0) { NE_DCASE(_Float16, float) }
    if (in_dt == 2 && out_dt == 2) { NE_DCASE(_Float16, _Float16) }
#undef NE_DCASE
    return hipErrorInvalidValue;
}

}  // namespace ne
