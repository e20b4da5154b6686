// ne_launch.hpp -- argument blocks and launchers between the C ABI (ne_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ne {

// Stored dS (16-bit backward): one tile of 64 flattened rows x 64 keys (8 KiB of fp16) for every
// row tile rt < nrt = ceil(T G / 64) and key block kb < nkb = ceil(T / 64) with rt >= kb G -- the
// row tiles the dK/dV pass visits for that key block -- stored by key block, then row tile.
__host__ __device__ inline size_t ds_tiles_per_group(int nrt, int nkb, int G) {
    return (size_t)nkb * nrt - (size_t)G * ((size_t)nkb * (nkb - 1) / 2);
}
__host__ __device__ inline size_t ds_tile_index(int kb, int rt, int nrt, int G) {
    return (size_t)kb * nrt - (size_t)G * ((size_t)kb * (kb - 1) / 2) + (size_t)(rt - kb * G);
}

// Header of the RoPE table at the start of an attention workspace (the table follows at byte 256):
// the arguments it was built for.  The preparation kernels compare it with the call's arguments on
// the device and make their operand copies NaN when it does not match.
constexpr unsigned kTableMagic = 0x52504e45u;
constexpr size_t kTableHdrBytes = 256;
struct TableHdr {
    unsigned magic;
    int T, D, pad;
    double base;
};
__host__ __device__ inline bool table_matches(const TableHdr& h, int T, int D, double base) {
    return h.magic == kTableMagic && h.T == T && h.D == D && h.base == base;
}

// QK norm: every (token, head) row x of q and k becomes gain * x / sqrt(mean(x^2) + eps).
struct QkNorm {
    int on;
    float gain, eps;
};

// Operand preparation: rotate/scale/convert into the workspace copies.
struct PrepArgs {
    const void* q; const void* k; const void* v;   // in dtype, [B][T][H][D]
    const void* o; const float* lse; const void* dO;  // backward only (o in out dtype)
    void* qh; void* kh; void* vh; void* dOh;        // operand copies (fp16 or fp32)
    float* delta; float* lse2; float2* table;       // backward only
    float* rq; float* rk;                           // backward with QK norm: 1/rms of q rows
                                                    // (flattened, [B*Hkv][T*G]) and k rows ([B*Hkv][T])
    int B, T, Hq, Hkv, D;
    double rope_base;
    float qscale;                                   // softmax scale * log2(e)
    QkNorm qkn;
    // half-split rotary pairs: the kernels rotate adjacent slots (2i, 2i + 1); with the pairing
    // (i, i + D/2) element i of a raw q or k row goes to slot 2i and element i + D/2 to slot 2i + 1
    // (scores are sums over slots), dq and dk leave the backward in slot order and a last pass puts
    // them back in element order; qs / ks (or null): slot-ordered raw copies of q and k for the QK
    // norm backward
    int half;
    void* qs; void* ks;
    int skip_v;                                     // backward: no v' copy (the dK/dV pass reads v)
    const TableHdr* hdr;                            // the table's header (RoPE on)
    // backward, 16-bit operands: dO' = s dO with s a power of two per (batch, KV head) group chosen
    // from the group's max |dO| (amax_part: nparts partial maxima per group); dsc[group] = 1 / s
    const float* amax_part; int nparts; float* dsc;
    float* dq_acc;                                  // atomic dQ accumulator to clear (or null)
    unsigned* split_cnt; int nsplit_cnt;            // counters of the split row blocks, cleared here
};

// Partial maxima of |dO| per (batch, KV head) group: part p of group g covers tokens
// [p * tpp, (p + 1) * tpp) of the group's G heads.
struct AmaxArgs {
    const void* dO;
    float* part;
    int B, T, Hq, Hkv, nparts, tpp;
};

// RoPE table of T positions into the workspace, plus its header.
struct TableArgs {
    TableHdr* hdr; float2* table;
    int T, D;
    double base;
};

// Key-range split of the longest row blocks.  Causal work per row block grows with its position,
// so when a launch has few blocks per CU the longest ones set the time.  Row blocks rb >= rs are
// cut into np contiguous ranges of their key tiles ("pieces"), each run by its own workgroup; the
// last piece of a block to finish combines the others' partial results (read back in piece
// order, so the sum does not depend on the arrival order) and writes the output.  job[] lists the
// pieces and unsplit blocks of one group longest-first (rb << 2 | piece); workgroup i takes job
// rank i / ngrp (XCD-interleaved as for unsplit launches).  njobs == 0: no split.
constexpr int kMaxSplitJobs = 1024;
struct SplitPlan {
    int njobs, rs, np, nrb;
    float* part;                                    // [split block][piece][slot floats]
    unsigned* cnt;                                  // [split block][arrived, written]
    unsigned short job[kMaxSplitJobs];
};
// The host's plan of one pass: fills njobs, rs, np, nrb and job (not part and cnt).  It depends
// only on the causal step counts of the blocks (no window), the number of groups and the
// workgroups the chip runs at once (256 CUs).  Forward: 256-row blocks (128 rows, three workgroups
// per CU at head_dim <= 64), up to 4 pieces; dQ:
// 128-row blocks (two workgroups per CU), 2 pieces; dK/dV: 64-key blocks, up to 4 pieces, job
// index rb meaning key block nkb - 1 - rb -- a dK/dV plan replaces the mirrored pairs, and may
// split nothing (rs = nrb, np = 1: single blocks longest-first fill the CUs the pairs leave idle).
// At head_dim <= 64 the dK/dV pass always has a plan (up to 1024 key blocks): its planned variant
// runs two workgroups per CU.
enum { kSplitFwd = 0, kSplitDq = 1, kSplitDkdv = 2 };
void split_plan(int kind, int T, int G, int ngrp, int D, SplitPlan* out);
// floats of the partial-result slot of one piece (forward: O, m and l of its 8 waves, 4 at
// head_dim <= 64; dQ: 4 waves;
// dK/dV: the 4 waves that hold the block's dV^T and dK^T after the row halves are added)
inline size_t split_slot_floats_fwd(int D) { return (size_t)(D <= 64 ? 4 : 8) * 64 * (D / 2 + 2); }
inline size_t split_slot_floats_dq(int D) { return (size_t)4 * 64 * (D / 2); }
inline size_t split_slot_floats_dkdv(int D) { return (size_t)4 * 64 * (D / 2); }

struct FwdArgs {
    const void* q;                                  // raw queries (in dtype), rotated in the kernel
    const void* kh; const void* vh;                 // prepared keys / values
    const float2* table;                            // cos/sin [T][D/2] (RoPE on)
    void* o; float* lse;
    int B, T, Hq, Hkv, G, nrb;
    int window;                                     // query t sees keys t - window + 1 .. t (1..T)
    double rope_base;
    float qscale;                                   // softmax scale * log2(e)
    QkNorm qkn;
    int half;                                       // half-split rotary pairs (as in PrepArgs)
};

struct BwdArgs {
    const void* qh; const void* kh; const void* vh; const void* dOh;
    const float* delta; const float* lse2; const float2* table;
    void* dq; void* dk; void* dv;
    const void* q; const void* k; const void* v;    // raw inputs (QK norm backward; v for dK/dV
                                                    // on the stored-dS path), dtype in_dt
    int in_dt;                                      // 0 f32, 1 bf16, 2 f16
    const float* rq; const float* rk;               // 1/rms of the q and k rows (QK norm)
    void* ds;                                       // stored dS tiles (16-bit operands), or null:
                                                    // dQ then recomputes S and dP
    const float* dsc;                               // 1 / (dO scale) per group (16-bit operands), or null
    float* dq_acc;                                  // atomic dQ: fp32 accumulator [group][T G][D]
    int ds_groups;                                  // groups whose dS the buffer holds at once
    int grp0, ngrp;                                 // the (batch, KV head) groups of one launch of
                                                    // the stored-dS pair (else 0 and B * Hkv)
    int B, T, Hq, Hkv, G, nrb;
    int window;                                     // query t sees keys t - window + 1 .. t (1..T)
    double rope_base;
    float scale;                                    // softmax scale 1/sqrt(D)
    QkNorm qkn;
    int half;                                       // half-split rotary pairs (as in PrepArgs)
};

// Cache append (decode path): k_new / v_new [B][Tn][Hkv][D] into the cache at positions
// lens[b] + i (clamped to fit).
struct AppendArgs {
    const void* k; const void* v;
    void* cache; const int* lens;
    int B, Tn, Tcap, Hkv;
    QkNorm qkn;
    double rope_base;
    int half;                                       // half-split pairs: keys stored in slot order
    double theta[64];                               // base^(-2i/D), i < D/2 (RoPE on)
};

// Decode / chunked prefill: Tq new queries per sequence at positions lens[b] + t against the cache.
constexpr int kMaxSplits = 64;                      // key slices per (group, row block), at most
struct DecodeArgs {
    const void* q; const void* cache; const int* lens;
    float* part_o; float* part_ml;                  // split partials
    void* o; float* lse;
    int B, Tq, Tcap, Hq, Hkv, G, nrb, nsplit;
    int window;                                     // 1..Tcap (Tcap: no window)
    double rope_base;
    float qscale;                                   // softmax scale * log2(e)
    QkNorm qkn;
    int half;                                       // half-split pairs: queries gathered into slots
    double theta[64];                               // base^(-2i/D), i < D/2 (RoPE on)
};

// QKV projection with the rotation (and QK norm) in the epilogue.
struct QkvArgs {
    const void* x; const void* w;                   // [M][C], [N][C] (in dtype)
    void* q; void* k; void* v;                      // [M][H][D] (out dtype)
    float2* table;                                  // cos/sin [T][D/2] (workspace)
    int M, C, N, T, Hq, Hkv, D;
    double rope_base;
    QkNorm qkn;
    int half;                                       // half-split pairs (i, i + D/2)
    double theta[64];                               // base^(-2i/D), i < D/2 (RoPE on)
};

// dtype codes follow ne_dtype_t: 0 = f32, 1 = bf16, 2 = f16.
// ev (nullable): hipEvent_t pairs recorded on `s` around each kernel launch, in launch order
// (forward: prep, fwd; backward: prep, dkdv, dq).
hipError_t launch_table(const TableArgs& a, hipStream_t s);
// sp / spq / spk: the split plans of the 16-bit forward, of the recomputing dQ pass and of its
// dK/dV pass (njobs == 0: none).
hipError_t launch_fwd(int in_dt, int out_dt, int D, const PrepArgs& pa, const FwdArgs& fa, const SplitPlan& sp,
                      hipStream_t s, hipEvent_t const* ev);
// mode: 0 dQ recomputes S and dP, 1 dQ reads the stored dS, 2 atomic dQ in the dK/dV pass
enum { kBwdRecompute = 0, kBwdStoredDs = 1, kBwdAtomic = 2 };
hipError_t launch_bwd(int in_dt, int out_dt, int D, int mode, const PrepArgs& pa, const AmaxArgs& am,
                      const BwdArgs& ba, const SplitPlan& spq, const SplitPlan& spk, hipStream_t s,
                      hipEvent_t const* ev);
hipError_t launch_append(int in_dt, int D, const AppendArgs& a, hipStream_t s);
// ev (nullable): pairs around the cos/sin table and the product (4 entries).
hipError_t launch_qkv(int in_dt, int out_dt, int D, const QkvArgs& a, hipStream_t s, hipEvent_t const* ev);
// ev (nullable): pairs around the split kernel and the merge (4 entries).
hipError_t launch_decode(int in_dt, int out_dt, int D, const DecodeArgs& a, hipStream_t s, hipEvent_t const* ev);
// The decode's split partials without a caller workspace: a file-scope device array of this many
// bytes, shared by every call on a device (calls that overlap on one device race).  decode_scratch
// gives its address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(void** out);

}  // namespace ne
