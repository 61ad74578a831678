/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * Every entry point computes exact attention, O = softmax(scale * Q K^T) V,
 * row by row, plus the natural-log log-sum-exp of each row's scaled logits.
 * The kernels follow the fused forward pass described on the page
 * "I/O-Aware Kernels" (datasystem.school, Module 5), section "FlashAttention:
 * tiling + online softmax": one on-chip Q tile streams K/V tiles, keeps a
 * running row max m and sum l, and rescales its output accumulator, so the
 * score matrix is never written to device memory. The serving variants
 * (ragged batches, grouped-query heads, K/V gathered from a paged cache) are
 * those of section "FlashInfer: I/O-aware attention for serving".
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers on the current HIP device,
 *   allocated and owned by the caller. The library never allocates, frees
 *   or synchronises (apart from the opt-in FA_DEBUG_VALIDATE check below);
 *   each call enqueues one or two kernels on `stream` (a hipStream_t passed
 *   as void*, NULL = the null stream) and returns.
 * - Tensors are dense and contiguous in the layouts stated per call, with
 *   the element type `dtype` (O has the type of Q). LSE is always float32.
 *   Q/K/V/O/pool pointers must be 16-byte aligned.
 * - `scale` multiplies Q K^T before the softmax; it must be finite and > 0
 *   (1/sqrt(d) is the usual value).
 * - Head dimension d must be 64 or 128.
 * - Grouped-query attention: Hq must be a multiple of Hkv and query head h
 *   reads key/value head h / (Hq / Hkv).
 * - Causal masking is aligned bottom-right: query row i of a sequence with
 *   Lq queries and Lk keys sees key j iff j <= i + (Lk - Lq). A row that sees
 *   no key gets O = 0 and LSE = -inf.
 * - Arguments are validated on the host before any HIP call; on an invalid
 *   argument nothing is launched and outputs are untouched. A pointer may be
 *   NULL only when its tensor holds no element (e.g. q, o and lse of a
 *   ragged call with Tq = 0, k and v with Tk = 0, k_new and v_new with
 *   T_new = 0).
 * - Index arrays that live on the device (cu_seqlens, page_table, seq_lens,
 *   prefix_pages, cu_new) are trusted: out-of-range contents are undefined
 *   behaviour. With the environment variable FA_DEBUG_VALIDATE set to a
 *   value other than "" or "0" (read at every call), each call copies them
 *   to the host after the work already queued on its stream, waits for that
 *   copy, and returns FA_ERR_INVALID_ARG without launching anything when
 *   they break the stated preconditions (cu_seqlens: cu[0] = 0,
 *   non-decreasing, cu[B] = the token count, no query run above
 *   max_seqlen_q; lengths within the page-table row; every page entry a
 *   sequence uses inside the pool), or FA_ERR_HIP when the copy fails. This
 *   is a debugging aid: it synchronises the stream.
 * - Calls keep no state between them and may be issued from several host
 *   threads; calls on different streams that write the same outputs race.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad scale, Hq % Hkv != 0, small workspace */
  FA_ERR_UNSUPPORTED = 2, /* valid request outside what is built: d, page size, dtype for a call */
  FA_ERR_HIP = 3,         /* the HIP runtime reported an error at launch */
  FA_ERR_NO_SPACE = 4     /* fa_decode_paged_noalloc: the request needs more workspace than
                             its fixed device buffer holds */
} fa_status;

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/* Human-readable text for a status code (static storage). */
const char* fa_status_string(fa_status s);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

/*
 * fa_fwd - dense batch, optional causal mask.
 * ("I/O-Aware Kernels", section "FlashAttention: tiling + online softmax".)
 *   q   [B, Nq, Hq, d]     dtype
 *   k,v [B, Nk, Hkv, d]    dtype
 *   o   [B, Nq, Hq, d]     dtype (written)
 *   lse [B, Nq, Hq]        float32 (written), natural log
 * B, Nq, Nk, Hq, Hkv >= 1. dtype FA_F32, FA_F16 or FA_BF16.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Nq, int Nk, int Hq, int Hkv, int d, fa_dtype dtype,
                 float scale, int causal, void* stream);

/*
 * fa_fwd_varlen - packed ragged batch of B sequences.
 * ("I/O-Aware Kernels", section "FlashInfer: I/O-aware attention for
 * serving": ragged, variable-length batches, multi-head and grouped-query.)
 *   q   [Tq, Hq, d], k/v [Tk, Hkv, d], o [Tq, Hq, d]   dtype
 *   lse [Tq, Hq] float32
 *   cu_seqlens_q, cu_seqlens_k: device int32 [B+1], cu[0] = 0, non-decreasing,
 *     cu_q[B] = Tq, cu_k[B] = Tk; sequence s owns rows cu[s] .. cu[s+1]-1.
 *   max_seqlen_q >= every query length (sizes the grid); max_seqlen_k is
 *     accepted for interface symmetry and only checked for sign.
 * Sequences may be empty. B >= 1, Tq, Tk >= 0.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                        int max_seqlen_q, int max_seqlen_k, int Tq, int Tk, int Hq, int Hkv,
                        int d, fa_dtype dtype, float scale, int causal, void* stream);

/*
 * fa_fwd_paged - prefill of a ragged batch of query chunks against K/V held
 * in a paged cache ("chunked prefill").
 * ("I/O-Aware Kernels", section "FlashInfer: I/O-aware attention for
 * serving": ragged batches, paged KV layouts, grouped-query attention.)
 *   q   [Tq, Hq, d] dtype, packed like fa_fwd_varlen; o [Tq, Hq, d] dtype;
 *   lse [Tq, Hq] float32
 *   cu_seqlens_q device int32 [B+1]: chunk s owns query rows
 *               cu[s] .. cu[s+1]-1 (chunks may be empty)
 *   k_pool, v_pool [num_pages, page_size, Hkv, d] dtype, page_table device
 *               int32 [B, max_pages] and seq_lens device int32 [B] exactly
 *               as for fa_decode_paged. seq_lens[s] counts every key of
 *               sequence s - the cached prefix and the chunk itself, whose
 *               K/V must already be in the pages - so the chunk's queries
 *               are the last Lq of its Lk tokens: with causal masking, query
 *               row i of the chunk sees keys j <= i + Lk - Lq (bottom-right).
 *   max_seqlen_q >= every chunk length (sizes the grid).
 * page_size must be 16, max_pages <= 8192 (sequences of at most 131072
 * tokens), dtype FA_F16 or FA_BF16. Preconditions on the device arrays:
 * Lq <= seq_lens[s] <= max_pages * 16, and the page-table entries of the
 * first ceil(seq_lens[s] / 16) pages are valid page indices.
 */
fa_status fa_fwd_paged(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                       const int32_t* cu_seqlens_q, const int32_t* page_table,
                       const int32_t* seq_lens, int B, int max_seqlen_q, int Tq, int max_pages,
                       int num_pages, int page_size, int Hq, int Hkv, int d, fa_dtype dtype,
                       float scale, int causal, void* stream);

/*
 * fa_decode_paged_workspace_size - bytes of device workspace that
 * fa_decode_paged needs for these sizes (float32 partial outputs and
 * log-sum-exps of every split). Returns 0 for invalid sizes.
 */
size_t fa_decode_paged_workspace_size(int B, int Hq, int d, int max_pages, int page_size,
                                      int num_splits);

/*
 * fa_decode_paged - one query token per sequence against K/V gathered from
 * a paged cache through a page table, split over the key axis and merged
 * with a log-sum-exp combine pass.
 * ("I/O-Aware Kernels", section "FlashInfer: I/O-aware attention for
 * serving": paged KV layouts, grouped-query attention.)
 *   q          [B, Hq, d]                      dtype
 *   k_pool,v_pool [num_pages, page_size, Hkv, d] dtype: page p, slot t holds
 *              the key/value of one token for every KV head
 *   page_table device int32 [B, max_pages]: entry i of sequence b is the
 *              physical page holding its tokens 16*i .. 16*i+15; entries at
 *              or beyond ceil(seq_lens[b]/page_size) are not read
 *   seq_lens   device int32 [B], 0 <= seq_lens[b] <= max_pages*page_size
 *   o [B, Hq, d] dtype, lse [B, Hq] float32 (written)
 *   num_splits 0 = automatic (48 pages per split), else the number of key
 *              splits of the longest sequence (1 .. max_pages); a split never
 *              holds more than 64 pages, so smaller values are raised to
 *              ceil(max_pages / 64)
 *   workspace  device buffer of at least
 *              fa_decode_paged_workspace_size(B, Hq, d, max_pages, page_size,
 *              num_splits) bytes, owned by the caller; its contents are
 *              scratch (overwritten, not read before written).
 * page_size must be 16. The query is the last token of its sequence, so it
 * sees every key; slots of a last page beyond seq_lens are never read into
 * the result (their contents, even NaN, do not matter).
 */
fa_status fa_decode_paged(const void* q, const void* k_pool, const void* v_pool, void* o,
                          float* lse, const int32_t* page_table, const int32_t* seq_lens, int B,
                          int max_pages, int num_pages, int page_size, int Hq, int Hkv, int d,
                          fa_dtype dtype, float scale, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * fa_decode_paged_noalloc - fa_decode_paged without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It computes
 * exactly what fa_decode_paged computes with the same kernels (bitwise the
 * same outputs), with its split partials in a fixed device buffer of
 * FA_DECODE_NOALLOC_MAX_WORKSPACE bytes that the library holds on every GPU
 * it runs on until the process ends. The call itself allocates nothing.
 *   Arguments, layouts and errors as for fa_decode_paged, plus
 *   FA_ERR_NO_SPACE when fa_decode_paged_workspace_size(B, Hq, d, max_pages,
 *   page_size, num_splits) exceeds FA_DECODE_NOALLOC_MAX_WORKSPACE (nothing
 *   is launched then).
 * The buffer's address on a device is looked up once, at the first call made
 * with that device current (FA_ERR_HIP if that fails). Every call on a GPU
 * shares that GPU's buffer and leaves the last call's partials in it: calls
 * that overlap on one GPU (on different streams, or from several host
 * threads without ordering) race and may corrupt each other's results.
 * Calls on one stream are ordered and safe. The buffer needs no clearing:
 * the merge pass reads only partials that the same call wrote.
 */
#define FA_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
fa_status fa_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool, void* o,
                                  float* lse, const int32_t* page_table, const int32_t* seq_lens,
                                  int B, int max_pages, int num_pages, int page_size, int Hq,
                                  int Hkv, int d, fa_dtype dtype, float scale, int num_splits,
                                  void* stream);

/*
 * fa_decode_cascade_workspace_size - bytes of device workspace that
 * fa_decode_cascade needs (float32 partials of the prefix splits and of the
 * suffix splits). Returns 0 for invalid sizes.
 */
size_t fa_decode_cascade_workspace_size(int B, int Hq, int d, int prefix_len, int max_pages,
                                        int page_size);

/*
 * fa_decode_cascade - decode of B sequences that share one cached prefix.
 * ("I/O-Aware Kernels", section "FlashInfer: I/O-aware attention for
 * serving": paged KV layouts, grouped-query attention, and the shared
 * prefixes of the RadixAttention layout seen from the kernel.)
 * The keys of sequence b are the prefix_len tokens held on prefix_pages
 * followed by its own seq_lens[b] tokens held through page_table row b; its
 * one query sees all of them. The prefix pages are read once for the whole
 * batch: one pass reduces them against the queries of every sequence (the
 * query heads of a KV head as columns of one MFMA operand), a second pass
 * reduces each sequence's own pages, and a log-sum-exp merge combines both.
 *   q [B, Hq, d], o [B, Hq, d] dtype; lse [B, Hq] float32
 *   k_pool, v_pool [num_pages, page_size, Hkv, d] dtype (prefix and
 *              suffix pages live in the same pools)
 *   prefix_pages device int32 [ceil(prefix_len / 16)]: physical pages of
 *              prefix tokens 16*i .. 16*i+15 (slots of a last, partial prefix
 *              page beyond prefix_len are not read); may be NULL when
 *              prefix_len == 0
 *   page_table device int32 [B, max_pages], seq_lens device int32 [B]: the
 *              suffix of each sequence, as for fa_decode_paged (suffix
 *              token 0 is key prefix_len); seq_lens[b] may be 0
 *   workspace  at least fa_decode_cascade_workspace_size(...) bytes of
 *              device memory owned by the caller (scratch).
 * page_size must be 16, dtype FA_F16 or FA_BF16. Prefix splits of 32 pages,
 * suffix splits of 8 pages.
 */
fa_status fa_decode_cascade(const void* q, const void* k_pool, const void* v_pool, void* o,
                            float* lse, const int32_t* prefix_pages, int prefix_len,
                            const int32_t* page_table, const int32_t* seq_lens, int B,
                            int max_pages, int num_pages, int page_size, int Hq, int Hkv, int d,
                            fa_dtype dtype, float scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * fa_kv_append - write the K/V rows of new tokens into the paged cache.
 * ("I/O-Aware Kernels", section "FlashInfer: I/O-aware attention for
 * serving": paged KV layouts; the step that fills the pages fa_fwd_paged and
 * fa_decode_paged read.)
 *   k_new, v_new  [T_new, Hkv, d] dtype; sequence s owns rows
 *                 cu_new[s] .. cu_new[s+1]-1 (device int32 [B+1], cu_new[0] = 0,
 *                 non-decreasing, cu_new[B] = T_new; sequences may get none)
 *   k_pool, v_pool [num_pages, page_size, Hkv, d] dtype (written in place)
 *   page_table    device int32 [B, max_pages], as for fa_decode_paged
 *   seq_lens_before device int32 [B]: tokens each sequence already holds
 * Token i of sequence s goes to position p = seq_lens_before[s] + i, i.e.
 * page page_table[s][p / 16], slot p % 16; nothing else in the pools changes
 * (bit-exact copy). The caller owns seq_lens and adds the new counts
 * afterwards. A token whose position is at or past max_pages * 16, or whose
 * page-table entry is outside [0, num_pages), is not written. Any dtype; d
 * must be 64 or 128, page_size 16. T_new = 0 is a no-op.
 */
fa_status fa_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                       const int32_t* cu_new, const int32_t* page_table,
                       const int32_t* seq_lens_before, int B, int T_new, int max_pages,
                       int num_pages, int page_size, int Hkv, int d, fa_dtype dtype, void* stream);

/*
 * fa_bwd_workspace_size - bytes of device workspace that fa_bwd needs
 * (two float32 per query row and head, rows rounded up to a multiple of
 * 64). Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(int B, int Nq, int Hq);

/*
 * fa_bwd - gradients of dense attention with respect to Q, K and V, given
 * the output gradient dO and the O and LSE that fa_fwd returned for the
 * same q, k, v, scale and mask. The pages define only the forward pass
 * ("I/O-Aware Kernels", section "Naive attention: materializing the k x k
 * score matrix": S = scale Q K^T, P = row softmax of S, O = P V); these are
 * its chain-rule gradients, dV = P^T dO, dS = P o (dO V^T - rowsum(dO o O)),
 * dQ = scale dS K, dK = scale dS^T Q, computed as in section "FlashAttention:
 * tiling + online softmax": P is recomputed tile by tile from the saved LSE
 * and nothing of size Nq x Nk reaches device memory. LSE is not
 * differentiated.
 *   q, o, dout [B, Nq, Hq, d] dtype; k, v [B, Nk, Hkv, d] dtype;
 *   lse [B, Nq, Hq] float32 (as written by fa_fwd)
 *   dq [B, Nq, Hq, d], dk, dv [B, Nk, Hkv, d] dtype (written): with
 *     grouped-query heads, dk and dv of a key/value head sum the gradients
 *     of every query head that reads it
 *   workspace  at least fa_bwd_workspace_size(B, Nq, Hq) bytes of device
 *     memory owned by the caller (scratch: rowsum(dO o O) and the LSE in
 *     base 2 per row and head, laid out head by head)
 * B, Nq, Nk, Hq, Hkv >= 1 and a workspace of at least the stated size, else
 * FA_ERR_INVALID_ARG; dtype FA_F16 or FA_BF16 (FA_F32: FA_ERR_UNSUPPORTED);
 * causal masks as for fa_fwd (bottom-right). Two kernels on `stream`,
 * deterministic (fixed summation order, no atomics).
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq,
                 int Hkv, int d, fa_dtype dtype, float scale, int causal, void* workspace,
                 size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
