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
 * the caller.  The library never allocates, frees, synchronises or prints on the compute calls.
 * Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs asynchronously;
 * device-side faults surface at the caller's next synchronisation.
 *
 * Errors: arguments are validated on the host before anything is enqueued; on failure the call
 * returns a non-zero ne_status_t, enqueues nothing, and ne_last_error() gives a thread-local
 * message.  NE_ERR_HIP means a launch was rejected by the HIP runtime (hipGetLastError).
 *
 * Thread safety: calls are re-entrant; the only mutable library state is the thread-local error
 * message.  Two calls that share a workspace must be ordered on one stream.
 */
#ifndef NE_ROPE_ATTN_H
#define NE_ROPE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NE_ABI_VERSION 1

typedef enum { NE_F32 = 0, NE_BF16 = 1, NE_F16 = 2 } ne_dtype_t;

typedef enum {
    NE_OK = 0,
    NE_ERR_NULL = 1,        /* a required pointer is NULL                                   */
    NE_ERR_SHAPE = 2,       /* B, T, Hq, Hkv < 1, Hq % Hkv != 0, or sizes overflow (for the
                               attention calls: T * (Hq / Hkv) * head_dim * e >= 2^31, e = 4
                               for fp32 inputs, else 2 -- a KV group's rows are addressed with
                               32-bit byte offsets)                                           */
    NE_ERR_UNSUPPORTED = 3, /* head_dim not in {32, 64, 128}, or dtype pair not supported     */
    NE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                               */
    NE_ERR_WORKSPACE = 5,   /* workspace_bytes smaller than the matching *_workspace_bytes()  */
    NE_ERR_HIP = 6          /* the HIP runtime rejected a launch                              */
} ne_status_t;

/* Supported (in_dtype -> out_dtype) pairs: F32->F32 (fp32 operands on fp32 MFMA),
 * BF16->F32, BF16->BF16, F16->F32, F16->F16 (fp16 MFMA operands, fp32 accumulation).
 * q, k, v and dO are in_dtype; o, dq, dk and dv are out_dtype. */

/* Bytes of device workspace the forward needs (256-byte aligned base recommended; 16 is
 * required).  Holds the rotated, scaled, converted operand copies.  Returns 0 for invalid
 * arguments. */
size_t ne_rope_attn_fwd_workspace_bytes(int B, int T, int Hq, int Hkv, int head_dim,
                                        ne_dtype_t in_dtype);

/* Bytes of device workspace the backward needs (operand copies, the per-row
 * Delta = rowsum(dO * o), the log2-scaled lse, the per-row 1/rms of q and k used by the QK norm,
 * the cos/sin table and, for 16-bit inputs, the fp16 dS of every 64-row x 64-key tile of the
 * causal band: 8 KiB per tile, about T * T * (Hq / Hkv) bytes per (batch, KV head) group).  The
 * dS buffer holds as many groups as fit 4 GiB, or the byte count in the environment variable
 * NE_ROPE_ATTN_DS_MAX_BYTES (0: none), and the dK/dV and dQ passes run once per batch of that many
 * groups; when not even one group fits, dQ recomputes S and dP and the workspace omits the
 * buffer.  The variable is read by this call and by ne_rope_attn_bwd*: keep it unchanged between
 * them.  Results agree within rounding either way, and are bitwise the same for every batch size;
 * each choice is bit-reproducible. */
size_t ne_rope_attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int head_dim,
                                        ne_dtype_t in_dtype);

/* Forward: o = softmax(mask(R(q) R(k)^T / sqrt(D))) v, lse = log-sum-exp of each score row.
 * rope_base <= 0 disables the rotation. */
ne_status_t ne_rope_attn_fwd(const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                             ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Backward: given q, k, v, the forward's o (out_dtype) and lse, and dO (in_dtype), writes the
 * gradients of sum(o * dO): dq (w.r.t. the un-rotated q), dk (un-rotated k, summed over the
 * query heads of each group) and dv.  Deterministic: every output element is written once by
 * one thread in a fixed order (no atomics), so repeated calls give identical bits.
 * Delta = rowsum(dO * o) is computed from the o passed in. */
ne_status_t ne_rope_attn_bwd(const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dO,
                             void* dq, void* dk, void* dv,
                             int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                             ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Instrumented variants for measurement: identical work, plus hipEvent_t records on `stream`
 * around each kernel launch -- events[2i] before and events[2i+1] after launch i.  Forward:
 * i = 0 operand preparation, 1 attention (an array of 4).  Backward: i = 0 preparation with
 * Delta, 1 dK/dV, 2 dQ (an array of 6; when the stored dS is processed in several group batches,
 * interval 1 spans every batch's dK/dV and all but the last dQ, interval 2 the last dQ).  The
 * array must be non-null; a null entry skips that
 * record (a record costs microseconds of stream time, so a measurement brackets only the
 * launches it needs).  The events are created and owned by the caller. */
ne_status_t ne_rope_attn_fwd_timed(const void* q, const void* k, const void* v,
                                   void* o, float* lse,
                                   int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                   ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* events);
ne_status_t ne_rope_attn_bwd_timed(const void* q, const void* k, const void* v,
                                   const void* o, const float* lse, const void* dO,
                                   void* dq, void* dk, void* dv,
                                   int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                   ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* events);

/* Options of the *_ex calls and of the cache calls (a NULL pointer means all defaults: no window,
 * no QK norm). */
typedef struct {
    int window;     /* > 0: query t sees keys t - window + 1 .. t; <= 0: the whole causal prefix   */
    int qk_norm;    /* nonzero: QK norm -- every (token, head) row x of q and of k is replaced by
                       qk_gain * x / sqrt(mean(x^2) + qk_eps) before RoPE ("nanochat 全栈 LLM 训练实践
                       指南", section 模型架构速览: q and k normalised and scaled up by 1.2); the
                       backward returns gradients with respect to the raw q and k                     */
    float qk_gain;  /* 1.2 in the guide; finite                                                       */
    float qk_eps;   /* added to the mean square; finite, >= 0 (0 with an all-zero row: non-finite)    */
} ne_attn_opts_t;

/* The forward and backward with every option (window and QK norm).  Arguments as in
 * ne_rope_attn_fwd / ne_rope_attn_bwd; opts may be NULL; events NULL or as for the *_timed calls.
 * The backward must be given the options the forward used. */
ne_status_t ne_rope_attn_fwd_ex(const void* q, const void* k, const void* v,
                                void* o, float* lse,
                                int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                const ne_attn_opts_t* opts,
                                ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events);
ne_status_t ne_rope_attn_bwd_ex(const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dO,
                                void* dq, void* dk, void* dv,
                                int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                const ne_attn_opts_t* opts,
                                ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events);

/* Sliding-window attention: the same operation with each query seeing only the `window` most
 * recent keys, its own position included -- query t sees keys t - window + 1 .. t -- as in the
 * short-window layers of the window_pattern feature ("nanochat 全栈 LLM 训练实践指南", section
 * 模型架构速览, where a short window is a quarter of the context).  window <= 0, or >= T, is the
 * full causal prefix and gives the same bits as ne_rope_attn_fwd / ne_rope_attn_bwd.  The backward
 * must be given the window the forward used (lse depends on it).  Arguments, layouts, workspace
 * sizes and errors are those of ne_rope_attn_fwd / ne_rope_attn_bwd; `events` is NULL (untimed) or
 * an array as for the *_timed calls (4 forward, 6 backward). */
ne_status_t ne_rope_attn_fwd_window(const void* q, const void* k, const void* v,
                                    void* o, float* lse,
                                    int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                    int window,
                                    ne_dtype_t in_dtype, ne_dtype_t out_dtype,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    void* const* events);
ne_status_t ne_rope_attn_bwd_window(const void* q, const void* k, const void* v,
                                    const void* o, const float* lse, const void* dO,
                                    void* dq, void* dk, void* dv,
                                    int B, int T, int Hq, int Hkv, int head_dim, double rope_base,
                                    int window,
                                    ne_dtype_t in_dtype, ne_dtype_t out_dtype,
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
 *     dimensions 16 u + 8 (l / 32) .. + 7, at element (u * 64 + l) * 8 of the tile;
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
