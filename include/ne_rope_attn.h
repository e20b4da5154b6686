/*
 * ne_rope_attn.h -- C ABI of the causal grouped-query attention library with rotary
 * position embeddings (RoPE), forward and backward, for AMD MI355X (gfx950).
 *
 * The operation (see each call below for the passages it follows):
 *   q' = R(q), k' = R(k)         RoPE on queries and keys ("NanoEuler: 使用 C 和 CUDA 从零
 *                                开始构建的 GPT-2 规模 LLM", section 技术规格)
 *   S  = q' k'^T / sqrt(D)       query head h reads key/value head h / (Hq/Hkv): grouped-query
 *                                attention (same page, 技术规格 and table 模型配置)
 *   P  = softmax(S masked to key <= query)     decoder-only, hence causal (same page, 核心架构与设计)
 *   o  = P v,  lse = log sum exp(S) per row    computed tile by tile with an online softmax so that
 *                                the T x T matrix is never stored (same page, 内核实现; "用 100KB
 *                                C/CUDA 单文件复刻 GPT-2:NanoEuler 116M 单卡可跑的全流程拆解", §3.4)
 *   backward: gradients of sum(o * dO) with respect to the un-rotated q, k and v
 *                                (hand-written backward: agentlenshq page, 验证与稳定性).
 * Readings where the pages are silent: RoPE rotates adjacent pairs (2i, 2i+1) by +t*theta_i,
 * theta_i = rope_base^(-2i/D), positions t = 0..T-1; rope_base <= 0 disables RoPE; the softmax
 * scale is 1/sqrt(head_dim); key j is visible to query i iff j <= i; lse is the natural log.
 *
 * Layouts (dense, row-major, element strides only):
 *   q, o, dO, dq : [B][T][Hq][head_dim]
 *   k, v, dk, dv : [B][T][Hkv][head_dim]
 *   lse          : [B][Hq][T], always float32
 *
 * Ownership: every tensor pointer and the workspace are DEVICE pointers allocated and owned by
 * the caller.  The library never allocates, frees, synchronises or prints on the compute calls
 * (ne_rope_table_check, a diagnostic, is the one call that waits for its stream).
 * Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs asynchronously;
 * device-side faults surface at the caller's next synchronisation.
 *
 * Errors: arguments are validated on the host before anything is enqueued; on failure the call
 * returns a non-zero ne_status_t, enqueues nothing, and ne_last_error() gives a thread-local
 * message.  NE_ERR_HIP means a launch was rejected by the HIP runtime (hipGetLastError).
 * The one condition the host cannot see is a workspace whose RoPE table was never built for the
 * call's (T, head_dim, rope_base): the kernels detect it on the device and make the outputs NaN
 * (ne_rope_table_init, ne_rope_table_check).
 *
 * Thread safety: calls are re-entrant.  Mutable library state: the thread-local error message, a
 * host cache of the split plans (one per shape, behind a mutex; a plan depends only on the shape)
 * and the device scratch of ne_rope_attn_decode_noalloc.  Two calls that share a workspace must be
 * ordered on one stream.
 */
#ifndef NE_ROPE_ATTN_H
#define NE_ROPE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NE_ABI_VERSION 3

typedef enum { NE_F32 = 0, NE_BF16 = 1, NE_F16 = 2 } ne_dtype_t;

typedef enum {
    NE_OK = 0,
    NE_ERR_NULL = 1,          /* a required pointer is NULL                                 */
    NE_ERR_SHAPE = 2,         /* B, T, Hq, Hkv < 1, Hq % Hkv != 0, or sizes overflow (for the
                                 attention calls: T * (Hq / Hkv) * head_dim * e >= 2^31, e = 4
                                 for fp32 inputs, else 2 -- a KV group's rows are addressed
                                 with 32-bit byte offsets)                                   */
    NE_ERR_UNSUPPORTED = 3,   /* head_dim not in {32, 64, 128}, dtype pair not supported, or a
                                 flag the library does not implement                        */
    NE_ERR_ALIGN = 4,         /* a pointer is not 16-byte aligned                             */
    NE_ERR_WORKSPACE = 5,     /* workspace_bytes smaller than ne_rope_attn_workspace_bytes()  */
    NE_ERR_NO_ROPE_TABLE = 6, /* the workspace holds no cos/sin table for (T, head_dim,
                                 rope_base): returned by ne_rope_table_check; see the
                                 table notes below for what fwd / bwd do instead             */
    NE_ERR_HIP = 7            /* the HIP runtime rejected a launch or a copy                  */
} ne_status_t;

/* Flags (bitwise OR; 0 = the defaults).
 *   NE_FLAG_NONDETERMINISTIC  backward: dQ is accumulated in the dK/dV pass with fp32 atomic adds
 *                             into a workspace buffer and converted by a small pass, instead of a
 *                             separate pass that recomputes S and dP.  Results meet the same error
 *                             bound but their low bits may differ from call to call.  Without the
 *                             flag every output is written once by one thread in a fixed order and
 *                             repeated calls give identical bits.  (16-bit inputs; the fp32 path
 *                             ignores the flag and stays deterministic.)
 *   NE_FLAG_STORE_DS          backward: the dK/dV pass also stores the fp16 dS of every 64 x 64
 *                             tile of the causal band in the workspace (about T * T * Hq / Hkv bytes
 *                             per (batch, KV head) group) and the dQ pass reads it instead of
 *                             recomputing S and dP: this gives up the O(T) memory of the default
 *                             backward for fewer products.  The workspace query sizes the buffer for
 *                             every group (at most 4 GiB); a smaller workspace that still holds one
 *                             group's dS makes the two passes run once per batch of as many groups
 *                             as it holds, with the same bits.  Deterministic; 16-bit inputs only.
 *                             Ignored together with NE_FLAG_NONDETERMINISTIC.
 *   NE_FLAG_BF16_OPERANDS     reserved: bf16 MFMA operands.  Not implemented: NE_ERR_UNSUPPORTED.
 *   NE_FLAG_ROPE_HALF_SPLIT   fwd, bwd, their _ex forms and the workspace query: RoPE rotates
 *                             element i with element i + head_dim/2 by t * theta_i (the other
 *                             common pairing; the frequencies and positions are unchanged) instead
 *                             of the adjacent pair (2i, 2i + 1).  Pass the same flag to the forward
 *                             and to the backward (and to the backward's workspace query: it adds
 *                             slot-ordered copies of q and k, read by the QK-norm backward).  No
 *                             effect with rope_base <= 0.  The KV-cache, decode and QKV-projection
 *                             calls take no flags: they select this pairing with the options
 *                             struct's rope_half_split (ne_attn_opts_t, below). */
#define NE_FLAG_NONDETERMINISTIC 0x1u
#define NE_FLAG_BF16_OPERANDS 0x2u
#define NE_FLAG_ROPE_HALF_SPLIT 0x4u
#define NE_FLAG_STORE_DS 0x8u

/* Supported (in_dtype -> out_dtype) pairs: F32->F32 (fp32 operands on fp32 MFMA),
 * BF16->F32, BF16->BF16, F16->F32, F16->F16 (fp16 MFMA operands, fp32 accumulation).
 * q, k, v and dO are in_dtype; o, dq, dk and dv are out_dtype.
 * Range of 16-bit inputs: k and v become fp16 MFMA operands, so |k|, |v| must stay below 65504
 * (values under 2^-14 lose relative precision as fp16 subnormals).  dO is scaled per (batch, KV
 * head) group by a power of two before its conversion to fp16 and the gradients are scaled back, so
 * any finite dO is supported.  Scores are formed from fp16 operands, so a score carries an error of
 * about 2^-11 of |q'| |k'| / sqrt(head_dim): rows whose logits reach ~100 get probabilities accurate
 * to a few percent (their o and lse still meet 2e-3 of scale; dq of such nearly one-hot rows can
 * cancel to a few percent of its scale).  The fp32 path does not have this limit. */

/* Bytes of device workspace a forward (is_bwd = 0) or backward (is_bwd != 0) call needs for these
 * arguments and flags (256-byte aligned base recommended; 16 is required).  0 for invalid
 * arguments.  Layout, all caller-owned:
 *   [0, 256)                 table header (T, head_dim, rope_base of the table below)
 *   then, when rope_base > 0, the cos/sin table [T][head_dim / 2] of float2 (ne_rope_table_init);
 *   forward:  the rotated fp16 keys and transposed fp16 values (fp32 copies on the fp32 path);
 *             16-bit path: the partial results and counters of the split row blocks (below);
 *   backward: the rotated, scaled copies of q, k, dO (and v), Delta = rowsum(dO * o), the
 *             log2-scaled lse, the per-row 1/rms of the QK norm, the dO scales; with
 *             NE_FLAG_NONDETERMINISTIC the fp32 dQ accumulator [B][Hq][T][head_dim]; with
 *             NE_FLAG_STORE_DS the stored dS; otherwise (16-bit) the split regions of the dQ and
 *             dK/dV passes;
 *             with NE_FLAG_ROPE_HALF_SPLIT and rope_base > 0 copies of q and k in in_dtype.
 * Split blocks: when a call has few causal blocks per CU, the longest row blocks of the forward and
 * of the recomputing dQ pass are cut into 2-4 ranges of keys, and the dK/dV pass of the default
 * backward runs single key blocks instead of mirrored pairs, the longest cut into 2-4 ranges of row
 * tiles; the pieces of a block run on separate workgroups and the last to finish combines the others'
 * partial results in a fixed order (the result does not depend on which finishes last).  The plan
 * depends only on the shape; a window shorter than T turns it off, and the QK norm the dQ pass's.
 * For is_bwd != 0 the size returned is at least the forward's, so a backward workspace of that size
 * is also a valid forward workspace for the same arguments: the table sits at the same place, so
 * one ne_rope_table_init serves both calls. */
size_t ne_rope_attn_workspace_bytes(int is_bwd, int B, int T, int Hq, int Hkv, int head_dim,
                                    double rope_base, ne_dtype_t in_dtype, unsigned flags);

/* Builds the RoPE cos/sin table of positions 0 .. T-1 in the workspace and records (T, head_dim,
 * rope_base) in its header: c = cos(t theta_i), s = sin(t theta_i), theta_i = rope_base^(-2i/D)
 * (RoPE on queries and keys: "NanoEuler: 使用 C 和 CUDA 从零开始构建的 GPT-2 规模 LLM", 技术规格),
 * the phase formed and reduced to [-pi, pi] in double precision, then rounded to fp32.  Once per
 * workspace and (T, head_dim, rope_base): every forward and backward call with that workspace and
 * those arguments reads it.  rope_base <= 0: nothing to build (NE_OK).  Asynchronous on `stream`.
 * Table notes: the calls cannot read device memory without synchronising, so they do not check the
 * header on the host; their first kernel checks it on the device and, when it does not match the
 * call's (T, head_dim, rope_base), makes every output NaN.  ne_rope_table_check reports the state
 * explicitly. */
ne_status_t ne_rope_table_init(void* workspace, size_t workspace_bytes, int T, int head_dim,
                               double rope_base, void* stream);

/* NE_OK when the workspace's table header matches (T, head_dim, rope_base) (or rope_base <= 0),
 * NE_ERR_NO_ROPE_TABLE otherwise.  Copies the 256-byte header to the host and waits for `stream`:
 * the one call of this library that synchronises (a diagnostic, not for the hot path). */
ne_status_t ne_rope_table_check(const void* workspace, size_t workspace_bytes, int T, int head_dim,
                                double rope_base, void* stream);

/* Forward: o = softmax(mask(R(q) R(k)^T / sqrt(D))) v, lse = log-sum-exp of each score row, computed
 * over 64-key tiles with an online softmax so no T x T matrix is stored ("NanoEuler: 使用 C 和 CUDA
 * 从零开始构建的 GPT-2 规模 LLM", 内核实现; "用 100KB C/CUDA 单文件复刻 GPT-2:NanoEuler 116M 单卡可跑的
 * 全流程拆解", §3.4).  rope_base <= 0 disables the rotation.  flags: 0 (the backward flags are
 * accepted and have no effect here). */
ne_status_t ne_rope_attn_fwd(const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                             ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Backward (the hand-written backward of the same pages, 验证与稳定性): given q, k, v, the forward's
 * o (out_dtype) and lse, and dO (in_dtype), writes the gradients of sum(o * dO): dq (w.r.t. the
 * un-rotated q), dk (un-rotated k, summed over the query heads of each group) and dv.
 * Delta = rowsum(dO * o) is computed from the o passed in.  By default dK/dV and dQ are separate
 * passes, dQ recomputing S and dP: the workspace is O(T) and every output element is written once
 * (bit-reproducible).  NE_FLAG_STORE_DS and NE_FLAG_NONDETERMINISTIC select the other two backward
 * designs (see the flags); the workspace must be sized with the same flags. */
ne_status_t ne_rope_attn_bwd(const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dO,
                             void* dq, void* dk, void* dv,
                             int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                             ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Options of the *_ex calls and of the cache calls (a NULL pointer means all defaults: no window,
 * no QK norm). */
typedef struct {
    int window;     /* > 0: query t sees keys t - window + 1 .. t, its own position included, as in
                       the short-window layers of the window_pattern feature ("nanochat 全栈 LLM 训练
                       实践指南", 模型架构速览, where a short window is a quarter of the context);
                       <= 0 or >= T: the whole causal prefix (the same bits as no window)            */
    int qk_norm;    /* nonzero: QK norm -- every (token, head) row x of q and of k is replaced by
                       qk_gain * x / sqrt(mean(x^2) + qk_eps) before RoPE ("nanochat 全栈 LLM 训练实践
                       指南", section 模型架构速览: q and k normalised and scaled up by 1.2); the
                       backward returns gradients with respect to the raw q and k                     */
    float qk_gain;  /* 1.2 in the guide; finite                                                       */
    float qk_eps;   /* added to the mean square; finite, >= 0 (0 with an all-zero row: non-finite)    */
    int rope_half_split; /* nonzero: RoPE rotates element i with element i + head_dim/2 (the pairing of
                       NE_FLAG_ROPE_HALF_SPLIT, which the fwd / bwd calls also take as a flag).  The
                       KV cache holds keys rotated with the pairing of its appends, so appends and
                       decodes must agree; the QKV projection then runs its narrower tiling (the
                       pairs of a head are in one lane only there).                                   */
} ne_attn_opts_t;

/* The forward and backward with every option (window and QK norm) and, for measurement, HIP events:
 * arguments as in ne_rope_attn_fwd / ne_rope_attn_bwd; opts may be NULL; the backward must be given
 * the options the forward used (lse depends on them).  events: NULL, or an array of hipEvent_t
 * recorded on `stream` around each kernel launch -- events[2i] before and events[2i+1] after launch
 * i; a NULL entry skips that record (a record costs stream time, so a measurement brackets only the
 * launches it needs).  Forward: i = 0 operand preparation, 1 attention (4 entries).  Backward: i = 0
 * preparation with Delta (and the dO scales), 1 dK/dV, 2 dQ (the dQ pass, or with
 * NE_FLAG_NONDETERMINISTIC the conversion of the accumulated dQ) (6 entries; with NE_FLAG_STORE_DS
 * run in several group batches, interval 1 spans every batch's dK/dV and all but the last dQ,
 * interval 2 the last dQ; with NE_FLAG_ROPE_HALF_SPLIT the two small launches that put dq and dk back
 * in element order follow the last interval).  The events are created and owned by the caller. */
ne_status_t ne_rope_attn_fwd_ex(const void* q, const void* k, const void* v,
                                void* o, float* lse,
                                int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                const ne_attn_opts_t* opts,
                                ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events);
ne_status_t ne_rope_attn_bwd_ex(const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dO,
                                void* dq, void* dk, void* dv,
                                int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                const ne_attn_opts_t* opts,
                                ne_dtype_t in_dtype, ne_dtype_t out_dtype, unsigned flags,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events);

/* ---- Key/value cache: decode and chunked prefill ----------------------------------------------
 * The second workload of the same operation: a few new tokens per sequence attend to everything
 * before them, held in a key/value cache -- nanochat's inference stage generates with a KV cache
 * ("nanochat 全栈 LLM 训练实践指南", sections 项目定位 and 测试体系; section 模型架构速览 notes, with its
 * peak-bandwidth table, that decoding is bound by memory bandwidth).  The new tokens of sequence b sit at absolute positions cache_lens[b] ..
 * cache_lens[b] + n - 1: keys are rotated at their own positions when appended, queries at theirs
 * when attending, so the results equal the last rows of ne_rope_attn_fwd over the whole sequence
 * (up to rounding).  Query t of sequence b sees the cached keys max(0, p - window + 1) .. p,
 * p = cache_lens[b] + t (window <= 0 or >= Tcap: every key up to p).
 *
 * The cache is one caller-owned device buffer of ne_kv_cache_bytes() bytes in the library's
 * layout: for each (b, kv head) group g = b * Hkv + h, its Tcap / 32 tiles of 32 positions, tile i
 * at element offset (g * Tcap / 32 + i) * 64 * head_dim, each holding
 *   keys after RoPE (fp16): for u < head_dim / 16 and lane l < 64, 8 elements: key i * 32 + l % 32,
 *     dimensions 16 u + 8 (l / 32) .. + 7, at element (u * 64 + l) * 8 of the tile (appended with
 *     opts->rope_half_split, "dimension" 2m holds element m of the rotated key and 2m + 1 element
 *     m + head_dim / 2: the slot order the decode then gives its queries too);
 *   values (fp16), from element 32 * head_dim of the tile: for kk < 2, db < head_dim / 32 and lane
 *     l, 8 elements: dimension 32 db + l % 32 of the keys i * 32 + 16 kk + s(8 (l / 32) + j),
 *     j < 8, at element ((kk * head_dim / 32 + db) * 64 + l) * 8 + j, where s swaps bits 2 and 3
 * (the order of the decode kernel's 16-byte loads).  Values are converted to fp16 (|v| must stay
 * below 65504).
 * Tcap, the capacity in tokens, is a multiple of 64.  cache_lens is a DEVICE array of B int32:
 * the tokens each sequence already holds.  It is read on the device, so it cannot be checked on
 * the host: each call uses min(max(cache_lens[b], 0), Tcap - n), n the tokens of the call, and
 * never touches memory outside the cache.  Neither call changes cache_lens; the caller advances
 * it after the tokens of a step are appended and attended to.  Only in_dtype BF16 and F16. */
size_t ne_kv_cache_bytes(int B, int Tcap, int Hkv, int head_dim, ne_dtype_t in_dtype);

/* Writes k_new, v_new ([B][Tn][Hkv][head_dim], in_dtype) into the cache at positions
 * cache_lens[b] .. cache_lens[b] + Tn - 1, keys rotated at those positions (after the QK norm when
 * opts asks for it; opts may be NULL; its window is not used here). */
ne_status_t ne_kv_cache_append(void* cache, size_t cache_bytes, const int* cache_lens,
                               const void* k_new, const void* v_new,
                               int B, int Tn, int Tcap, int Hkv, int head_dim, double rope_base,
                               const ne_attn_opts_t* opts, ne_dtype_t in_dtype, void* stream);

size_t ne_rope_attn_decode_workspace_bytes(int B, int Tq, int Tcap, int Hq, int Hkv, int head_dim,
                                           ne_dtype_t in_dtype);

/* o [B][Tq][Hq][head_dim] (out_dtype F32 or in_dtype), lse [B][Hq][Tq] for the queries q
 * ([B][Tq][Hq][head_dim], in_dtype) at positions cache_lens[b] + t against the cache, whose
 * positions up to cache_lens[b] + Tq - 1 must have been appended (with the same QK-norm options;
 * opts may be NULL; a window counts positions as in the *_ex calls).  The keys are split into slices
 * processed by separate workgroups and merged by the log-sum-exp rule in a fixed order
 * (deterministic).  events: NULL or 4 hipEvent_t entries (pairs around the attention and the
 * merge; null entries are skipped). */
ne_status_t ne_rope_attn_decode(const void* q, const void* cache, size_t cache_bytes, const int* cache_lens,
                                void* o, float* lse,
                                int B, int Tq, int Tcap, int Hq, int Hkv, int head_dim,
                                double rope_base, const ne_attn_opts_t* opts,
                                ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events);

/* The same decode for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): no workspace argument.  The split partials live in a
 * scratch array inside the library, NE_DECODE_SCRATCH_BYTES (64 MiB) per GPU, held until the process
 * ends; its address on the current device is looked up on the first call there and kept (library
 * state, like the error message and the cache of split plans).  Shapes whose partials
 * (ne_rope_attn_decode_workspace_bytes) exceed it are rejected with NE_ERR_WORKSPACE before anything
 * is enqueued.  Nothing is allocated or freed.  Every call on a device shares that device's array, so
 * calls that overlap on one device (different streams, or threads) race: order them on one stream.
 * Each call writes every partial it reads, so no state carries over between calls.  Same arguments,
 * results (bitwise) and errors as ne_rope_attn_decode otherwise. */
#define NE_DECODE_SCRATCH_BYTES ((size_t)64 << 20)
ne_status_t ne_rope_attn_decode_noalloc(const void* q, const void* cache, size_t cache_bytes,
                                        const int* cache_lens, void* o, float* lse,
                                        int B, int Tq, int Tcap, int Hq, int Hkv, int head_dim,
                                        double rope_base, const ne_attn_opts_t* opts,
                                        ne_dtype_t in_dtype, ne_dtype_t out_dtype, void* stream);

/* ---- QKV projection with the RoPE epilogue ----------------------------------------------------
 * The step before attention: y = x W^T for every token, then RoPE on the query and key heads --
 * on the pages a tensor-core matrix product followed by a RoPE kernel of its own ("NanoEuler: 使用
 * C 和 CUDA 从零开始构建的 GPT-2 规模 LLM", 内核实现; the cnblogs walkthrough §3.4 counts the cost
 * of such separate passes).  Here the rotation (and, with opts->qk_norm, the QK norm before it)
 * is applied to the product's accumulators before they are stored, so q' and k' leave rotated:
 *   x [B][T][C] (in_dtype BF16 or F16), w [(Hq + 2 Hkv) * head_dim][C] (in_dtype; rows: the Hq
 *   query heads, then the Hkv key heads, then the Hkv value heads, head_dim features each),
 *   q [B][T][Hq][head_dim] = R_t(norm(x W_q^T)), k [B][T][Hkv][head_dim] = R_t(norm(x W_k^T)),
 *   v [B][T][Hkv][head_dim] = x W_v^T, in out_dtype (F32 or in_dtype); t the token's position.
 * Feeding q, k, v to ne_rope_attn_fwd with rope_base <= 0 (and no QK norm) gives attention with
 * RoPE.  Requires C % 64 == 0 and (Hq + 2 Hkv) * head_dim % 128 == 0.  Products run on bf16/fp16
 * MFMA with fp32 accumulation.  The workspace holds the cos/sin table of the T positions.
 * events: NULL or 4 entries (pairs around the table and the product). */
size_t ne_qkv_rope_workspace_bytes(int T, int head_dim);
ne_status_t ne_qkv_rope_proj(const void* x, const void* w, void* q, void* k, void* v,
                             int B, int T, int C, int Hq, int Hkv, int head_dim, double rope_base,
                             const ne_attn_opts_t* opts, ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                             void* workspace, size_t workspace_bytes, void* stream, void* const* events);

const char* ne_status_str(ne_status_t status);
const char* ne_last_error(void);
int ne_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NE_ROPE_ATTN_H */
