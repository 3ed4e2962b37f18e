/*
 * fa.h -- C ABI of the exact tiled attention library (libfa.so, gfx950).
 *
 * The operation is exact softmax attention, O = softmax(scale * Q K^T) V, as
 * defined in the "FlashAttention" concept note (llm-wiki-maxwellmou), section
 * "是什么": the definition, and the per-block online-softmax update of a
 * running row max m, row sum l and output O that lets K/V be streamed in
 * blocks past a Q block held on chip.  The same section places causal masks,
 * padding masks and multi-head / GQA handling inside the tile, and names
 * one-token decode as bound by reading the KV cache.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory.
 *  - Layouts are contiguous, row-major "BHSD":
 *        q, o : [B, Hq,  Nq, d]      k, v : [B, Hkv, Nk, d]
 *        lse  : [B, Hq,  Nq] float32 (natural log)
 *  - dtype (enum fa_dtype) applies to q, k, v and o.  lse and the split-KV
 *    partials are always float32.  FA_BF16 runs both contractions on bf16
 *    matrix cores with float32 accumulation (P is rounded to bf16 before the
 *    P.V product, O is rounded to bf16 at the end); FA_F32 computes in float32
 *    throughout.
 *  - d must be 64 or 128.  Hq must be a multiple of Hkv; query head h reads KV
 *    head h / (Hq / Hkv).
 *  - scale must be finite and > 0 (the pages use 1/sqrt(d)).
 *  - Causal masking is aligned bottom-right: key j is visible to query i iff
 *    j <= i + (Nk - Nq).  With Nq == Nk this is the usual j <= i.
 *  - kv_seqlens is NULL (all Nk keys valid) or a DEVICE int32[B]: keys
 *    j >= kv_seqlens[b] of sequence b are excluded.  Values are clamped to
 *    [0, Nk] on the device (they cannot be checked without a sync).  Key and
 *    value rows at or beyond a sequence's length are never read.
 *  - A query row with no visible key gets O = 0 and LSE = -inf.
 *  - q, k, v, o and the partials must be 16-byte aligned; lse 4-byte aligned.
 *  - stream is a hipStream_t (NULL = the null stream).  Calls enqueue work and
 *    return without synchronising.  Arguments are validated on the host before
 *    any HIP call; a device fault surfaces at the caller's next sync.  A call
 *    launches kernels only (no allocation, memset or synchronisation), so it
 *    may be captured in a HIP graph and replayed.
 *  - Every call returns an fa_status; on failure fa_last_error() gives a
 *    thread-local message.
 *  - Sizes may be zero: a call with no output elements returns FA_OK without
 *    launching anything; Nk == 0 (or every length 0) yields O = 0, LSE = -inf.
 *    Pointers of empty tensors may be NULL.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null / misaligned pointer, negative size, bad scale */
  FA_ERR_UNSUPPORTED = -2, /* d, dtype, head ratio or num_splits outside the supported set */
  FA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than fa_decode_workspace_bytes / fa_bwd_workspace_bytes */
  FA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
};

enum fa_dtype { FA_F32 = 0, FA_BF16 = 1, FA_FP8_E4M3 = 2, FA_FP8_E5M2 = 3 };

/* Split-KV decode partitions each sequence's keys [0, L) into num_splits
 * chunks of C = ceil(L / num_splits) keys, C rounded up to a multiple of
 * FA_DECODE_SPLIT_ALIGN; split s covers [s*C, min((s+1)*C, L)) and may be
 * empty (then its partial is O_s = 0, lse_s = -inf). */
#define FA_DECODE_SPLIT_ALIGN 128
#define FA_MAX_SPLITS 256

/*
 * fa_fwd -- exact attention forward (prefill).
 *
 * Implements the definition and the blocked online-softmax update of the
 * concept note, section "是什么": each work-group holds a block of query rows
 * on chip, streams the K/V blocks it may see through LDS, and writes only O
 * and LSE to memory (no score or probability matrix reaches HBM).
 *
 *   q   [B,Hq,Nq,d]  in     k, v [B,Hkv,Nk,d] in     o [B,Hq,Nq,d] out
 *   lse [B,Hq,Nq] float32 out: ln sum_j exp(scale * q_i . k_j) over visible j
 *   causal: 0 or 1.   kv_seqlens: NULL or device int32[B] (padding mask).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
           const int32_t* kv_seqlens, int dtype, void* stream);

/*
 * fa_fwd_fp8 -- fa_fwd on FP8 inputs.  The pages credit FP8 matrix units for
 * part of FlashAttention-3's throughput (2026 explainer, section "二代和三代")
 * without fixing formats or scaling; here q, k and v hold 8-bit OCP
 * floating-point codes of one format (dtype FA_FP8_E4M3 or FA_FP8_E5M2), and
 * each tensor has one float32 descale, so the real inputs are
 * q_descale * value(q code), and likewise for k and v.  The attention of those
 * real inputs is computed as by fa_fwd: S = Q K^T on the FP8 matrix cores
 * (float32 accumulators, both descales folded into the softmax scale; the
 * instruction's internal sums are less precise than float32 -- measured
 * errors up to ~2^-15 of sum_d |q_d k_d|); V converted exactly to bf16 and
 * O = P V on the bf16 matrix cores with P rounded to bf16; O multiplied by
 * v_descale at the end.
 *   q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d]: FP8 codes (one byte each), in
 *   o [B,Hq,Nq,d] bf16 out, lse [B,Hq,Nq] float32 out
 *   q_descale, k_descale, v_descale: finite and > 0.
 * d must be 128.  scale, causal, kv_seqlens, GQA, alignment (16 bytes for
 * q, k, v, o) and errors as for fa_fwd.  NaN or infinite codes propagate as
 * IEEE arithmetic does.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
               const int32_t* kv_seqlens, float q_descale, float k_descale, float v_descale,
               int dtype, void* stream);

/*
 * fa_fwd_varlen -- fa_fwd over packed variable-length sequences (varlen and
 * chunked prefill).  The pages put padding masks inside the tile and set
 * prompt processing apart from one-token decode against a KV cache (concept
 * note, section "是什么" and its list of misconceptions); they fix no packed
 * layout.  Here the B sequences of a batch are concatenated along the token
 * axis of every head:
 *   q [Hq, total_q, d] in     k, v [Hkv, total_k, d] in     o [Hq, total_q, d] out
 *   lse [Hq, total_q] float32 out
 *   cu_seqlens_q, cu_seqlens_k: DEVICE int32[B + 1], non-decreasing, from 0
 *   to total_q (total_k): sequence b owns query rows cu_seqlens_q[b] ..
 *   cu_seqlens_q[b+1] - 1 and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1,
 *   and attends only to its own keys.
 *   max_seqlen_q: at least the longest query sequence (it sizes the grid).
 * Each sequence is fa_fwd with Nq = Lq_b, Nk = Lk_b, so under causal = 1 the
 * mask is bottom-right aligned per sequence: local key j is visible to local
 * query i iff j <= i + Lk_b - Lq_b -- a chunk of Lq_b new queries sees the
 * Lk_b - Lq_b cached keys before it.  Offsets cannot be checked without a
 * sync: the kernels clamp them to [0, total] and read a decreasing pair as an
 * empty sequence, so no row outside the tensors is addressed; query rows of a
 * sequence longer than max_seqlen_q, and rows outside every sequence, are not
 * written.  dtype, d, scale, GQA and alignment as for fa_fwd.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int Hq, int Hkv,
                  int total_q, int total_k, int max_seqlen_q, int d, float scale, int causal, int dtype,
                  void* stream);

/*
 * fa_decode_workspace_bytes -- bytes of device workspace fa_decode needs:
 * float32 partial outputs [B,Hq,num_splits,d] followed (at a 256-byte aligned
 * offset) by float32 partial LSEs [B,Hq,num_splits].  Returns 0 for invalid
 * sizes.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int d, int num_splits);

/*
 * fa_decode_splitkv -- split-KV single-token decode, first stage.
 *
 * The concept note ("是什么", last remarks) notes that one-token decode is
 * bound by reading the KV cache; here the cache of each sequence is split
 * into num_splits key ranges (see FA_DECODE_SPLIT_ALIGN) processed by
 * separate work-groups, and the Hq/Hkv query heads that share a KV head are
 * processed together so each cache byte is read once.
 *
 *   q        [B,Hq,1,d]    in       k_cache, v_cache [B,Hkv,Nk,d] in
 *   o_part   [B,Hq,S,d]    float32 out: normalised partial output of split s
 *   lse_part [B,Hq,S]      float32 out: log-sum-exp of split s (-inf if empty)
 *   num_splits S in [1, FA_MAX_SPLITS].  No causal mask: the single query is
 *   the newest token and sees every valid key.
 */
int fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      float* o_part, float* lse_part,
                      int B, int Hq, int Hkv, int Nk, int d, float scale,
                      const int32_t* kv_seqlens, int num_splits, int dtype, void* stream);

/*
 * fa_lse_merge -- exact merge of split partials (decode second stage).
 *
 * The online-softmax update of the concept note ("是什么") applied with the
 * blocks taken to be the splits: per row, M = max_s lse_s,
 * LSE = M + ln sum_s exp(lse_s - M), O = sum_s exp(lse_s - LSE) O_s.
 * Rows whose splits are all empty get O = 0, LSE = -inf.
 *
 *   o_part [rows,S,d] float32 in    lse_part [rows,S] float32 in
 *   o [rows,d] (dtype) out          lse [rows] float32 out
 */
int fa_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                 int rows, int d, int num_splits, int dtype, void* stream);

/*
 * fa_decode -- fa_decode_splitkv followed by fa_lse_merge on the same stream,
 * using a caller-provided device workspace of at least
 * fa_decode_workspace_bytes(B, Hq, d, num_splits) bytes (256-byte aligned).
 *   o [B,Hq,1,d] (dtype) out, lse [B,Hq,1] float32 out.
 */
int fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
              int B, int Hq, int Hkv, int Nk, int d, float scale, const int32_t* kv_seqlens,
              int num_splits, void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * fa_decode_noalloc -- fa_decode for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It computes exactly what
 * fa_decode computes, with the same kernels, but keeps the split partials in
 * a static device array of FA_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends.  The array's address
 * on a device is looked up on the first call made with that device current;
 * the call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).
 *   Arguments as for fa_decode, without the workspace.
 *   Errors: FA_ERR_WORKSPACE (before any HIP call) when
 *   fa_decode_workspace_bytes(B, Hq, d, num_splits) exceeds
 *   FA_NOALLOC_SCRATCH_BYTES; otherwise as for fa_decode.
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's partials (every partial a call reads is first written by the same
 * call, so nothing needs clearing).  Calls that overlap on one GPU -- on
 * different streams, or from different threads without ordering -- race on the
 * array and may return wrong results: serialise them.
 */
#define FA_NOALLOC_SCRATCH_BYTES 33554432
int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nk, int d, float scale, const int32_t* kv_seqlens,
                      int num_splits, int dtype, void* stream);

/*
 * fa_decode_paged -- fa_decode over a paged KV cache.  The pages place the KV
 * cache under page management (PagedAttention) without fixing a layout
 * (Concept note, section "是什么", table of related concepts; Explainer,
 * "paged" variants).  Here the cache is a pool of pages:
 *   k_pages, v_pages [num_pages, Hkv, page_size, d] bf16 in;
 *   block_table [B, max_pages_per_seq] int32 in (DEVICE): sequence b's pages
 *   in key order, so key j of sequence b is row j % page_size of page
 *   block_table[b][j / page_size];
 *   kv_seqlens [B] int32 in (DEVICE, required): valid keys per sequence,
 *   clamped to [0, page_size * max_pages_per_seq].
 * Table entries are clamped to [0, num_pages) on the device (they cannot be
 * checked without a sync); entries past a sequence's length are never read.
 * q, o, lse, num_splits, workspace (fa_decode_workspace_bytes) and scale are
 * as for fa_decode.  Only dtype FA_BF16 is supported, and a sequence holds at
 * most 2^24 keys (page_size * max_pages_per_seq <= 2^24).
 */
int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                    void* o, float* lse, int B, int Hq, int Hkv, int num_pages, int page_size,
                    int max_pages_per_seq, int d, float scale, const int32_t* kv_seqlens, int num_splits,
                    void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * fa_bwd_workspace_bytes -- bytes of device workspace fa_bwd needs: one
 * float32 per query row, [B, Hq, Nq] (rowsum(dO * O)).  Returns 0 for
 * invalid arguments.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq, int d);

/*
 * fa_bwd -- gradients of fa_fwd's output for training: given dO = dL/dO,
 * computes dQ, dK, dV of the loss L.  The backward pass recomputes the score
 * and probability tiles from Q, K and the forward's LSE instead of storing
 * them (Exam deep-dive "Flash Attention 在改善什麼？", section 技術版,
 * "Recomputation"; Interview note, section 节省显存，不等于所有内存都变少); what
 * it computes is the derivative of the forward definition:
 *     dV = P^T dO,   dS = P * (dO V^T - rowsum(dO * O)),
 *     dQ = scale * dS K,   dK = scale * dS^T Q,
 * with P = softmax(scale * Q K^T) under the same masks as fa_fwd (disallowed
 * pairs contribute nothing) and, with GQA, dK/dV summed over the query heads
 * that share a KV head.
 *   q, o, dout [B,Hq,Nq,d] bf16 in; k, v [B,Hkv,Nk,d] bf16 in;
 *   lse [B,Hq,Nq] float32 in: exactly what fa_fwd returned for these inputs;
 *   dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d] bf16 out (fully written: key rows at
 *   or beyond a sequence's length and rows with no visible key get zeros);
 *   causal, kv_seqlens, scale as for fa_fwd;
 *   workspace: device memory of at least fa_bwd_workspace_bytes(B, Hq, Nq, d)
 *   bytes, 256-byte aligned, overwritten.
 * Only dtype FA_BF16 is supported (FA_F32 returns FA_ERR_UNSUPPORTED); dO and
 * dS are rounded to bf16 before their matrix-core products, accumulation is
 * float32.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk,
           int d, float scale, int causal, const int32_t* kv_seqlens, void* workspace,
           size_t workspace_bytes, int dtype, void* stream);

/* Static string for a status code. */
const char* fa_status_string(int status);

/* Thread-local detail for the last non-OK return on this thread ("" if none). */
const char* fa_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
