/*
 * attn.h -- C ABI of the MI355X (gfx950) causal attention library (libattn.so).
 *
 * Three operations, each following the riftco-transformer documentation pages:
 *
 *   attn_causal_fwd    full-sequence causal scaled-dot-product attention with a
 *                      memory-linear forward that returns O and the per-row
 *                      log-sum-exp ("Architecture", "Intentional limits";
 *                      "Execution Backends and the Python ABI", "What the Metal
 *                      slice does": Flash keeps [B,H,T] row statistics instead
 *                      of the [B,H,T,T] probabilities).
 *   attn_causal_bwd    its vector-Jacobian product (dQ, dK, dV), recomputing
 *                      the probabilities from Q, K and the saved row statistics
 *                      (same sections).
 *   attn_paged_decode  single-token decode over a paged K/V cache addressed
 *                      through per-sequence block tables ("Execution Backends
 *                      and the Python ABI", "Incremental attention").
 *   attn_materialized_fwd  the materialized path: O, the row log-sum-exp and the
 *   attn_materialized_bwd  probabilities P [B,H,T,T]; its VJP uses the stored P and
 *                      accepts a cotangent of P ("Architecture", "Intentional
 *                      limits"; "What the Metal slice does": the materialized
 *                      path returns probabilities and context and keeps P for
 *                      the VJPs; the probability diagnostic always takes it).
 *   attn_paged_prefill  batched prefill: the new tokens of a ragged batch of
 *                      sequences attend causally to their sequence's paged K/V
 *                      (same sections; the pages prefill one token at a time
 *                      through the decode op, this takes all of them at once).
 *   attn_kv_append     the step before decode: lease pages from a device-resident
 *   attn_kv_release    free list and append each sequence's newest K/V rows, or
 *                      return a finished sequence's pages ("Architecture",
 *                      "Serving boundary": a request's logical page table, pages
 *                      leased from shared per-layer pools; "Incremental
 *                      attention": [physical_page, H, page_offset, d_h] pools).
 *   attn_kv_append_tokens  the same append for a ragged batch of several new
 *                      rows per sequence (the step before attn_paged_prefill).
 *
 * Conventions ("Architecture", "Tensor conventions"): contiguous row-major
 * float32; scores are [B,H,Tq,Tk] with Tq = Tk = T; the key at position t_k is
 * excluded from query t_q when t_k > t_q (the diagonal is kept).  Query head h
 * reads key/value head h / (Hq/Hkv), which requires Hq % Hkv == 0 (grouped-query
 * attention; ARCHITECTURE.md of algo-v1-codepoint, "config.py").
 *
 * ABI conventions ("Execution Backends and the Python ABI", "Stable C ABI"):
 * fixed-width integers, status returns, a thread-local error message, no C++
 * type crosses the boundary, and a version word major<<16 | minor.
 *
 * Ownership and synchrony.  Every tensor pointer is a DEVICE pointer owned by
 * the caller; the library never allocates, frees or keeps a pointer after a call
 * returns (the one buffer of its own, attn_paged_decode_noalloc's static scratch,
 * is part of its loaded device code, not a per-call allocation).  Outputs are fully overwritten.  A call validates its arguments on the
 * host, enqueues its kernels on `stream` (a hipStream_t; NULL is the null
 * stream) and returns without waiting: results are ready when the stream reaches
 * that point.  Inputs must stay unchanged and alive until then.
 *
 * Errors.  Every argument is checked before any HIP call.  A non-zero status
 * leaves the outputs untouched and attn_last_error() describes the problem.
 * No C++ exception escapes.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 0x00010004u /* 1.4: major << 16 | minor */

typedef int32_t attn_status;
enum {
    ATTN_OK = 0,
    ATTN_INVALID_ARGUMENT = 1,    /* null pointer, non-positive size, Hq % Hkv != 0,
                                     non-finite scale, misaligned or overlapping buffer */
    ATTN_UNSUPPORTED = 2,         /* a head width or page size without a kernel */
    ATTN_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the matching size query */
    ATTN_DEVICE_ERROR = 4         /* no HIP device, or a HIP call / kernel launch failed */
};

/* ABI version of the loaded library (ATTN_ABI_VERSION it was built with). */
uint32_t attn_abi_version(void);

/* Message of the last failing call on this thread ("" after a success).  The
 * pointer stays valid until the next attn_* call on the same thread. */
const char* attn_last_error(void);

/* Kernels exist for head widths D in {8, 16, 32, 64, 128} (all calls), decode
 * page sizes in {16, 32, 64} and decode group sizes 1 <= Hq/Hkv <= 16; other
 * values return ATTN_UNSUPPORTED. */

/*
 * Causal forward.
 *   q      [B, Hq,  T, D]   queries
 *   k, v   [B, Hkv, T, D]   keys, values
 *   scale  multiplies q.k (usually 1/sqrt(D)); any finite value
 *   o      [B, Hq,  T, D]   out: softmax(scale q k^T, keys t_k <= t_q) v
 *   lse    [B, Hq,  T]      out: natural-log log-sum-exp of each score row,
 *                           m + ln(sum exp(s - m)) over the unmasked keys
 * q, k, v, o 16-byte aligned, lse 4-byte aligned; o and lse may not overlap
 * any input or each other.  T * D, B * Hq and ceil(T / 64) * B * Hq must stay
 * below 2^31 and B * Hq * T * D below 2^40 (ATTN_INVALID_ARGUMENT otherwise; the
 * same limits hold for attn_causal_bwd).
 */
attn_status attn_causal_fwd(const float* q, const float* k, const float* v,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                            float scale, float* o, float* lse, void* stream);

/* Bytes of device workspace attn_causal_bwd needs for these sizes (0 when a
 * size is invalid): one float per query row, and, when B * Hkv * ceil(T / 64)
 * is small enough that the work is cut finer than per key block (at most 512
 * pieces of work), two 64 x D slices of dK and of dV per piece. */
size_t attn_causal_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D);

/*
 * Causal backward (vector-Jacobian product of attn_causal_fwd for the loss
 * sum(dout * O)).
 *   q, k, v, scale  as given to attn_causal_fwd
 *   o, lse          that call's outputs
 *   dout   [B, Hq,  T, D]   upstream gradient dL/dO
 *   dq     [B, Hq,  T, D]   out: dL/dQ
 *   dk, dv [B, Hkv, T, D]   out: dL/dK, dL/dV, each summed over the Hq/Hkv
 *                           query heads that share the key/value head
 *   workspace  device scratch of at least attn_causal_bwd_workspace_bytes(...)
 *              bytes (16-byte aligned); its contents on entry do not matter
 * q, k, v, o, dout, dq, dk, dv 16-byte aligned, lse 4-byte aligned; no output
 * (dq, dk, dv, workspace) may overlap an input or another output.
 * dQ is accumulated with float atomics, so its last bits may vary from run to
 * run; dK and dV are deterministic.
 */
attn_status attn_causal_bwd(const float* q, const float* k, const float* v,
                            const float* o, const float* lse, const float* dout,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                            float scale, float* dq, float* dk, float* dv,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_paged_decode needs for these sizes (0 when a
 * size is invalid): partial results of 1024 + S (position range, query head)
 * pieces and two int32 per sequence, whatever the page size and table width. */
size_t attn_paged_decode_workspace_bytes(int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                                         int64_t page_size, int64_t max_pages_per_seq);

/*
 * Batched single-token paged decode: S independent sequences, one new query
 * token each, sharing one K/V page pool.
 *   q             [S, Hq, D]                           queries of the newest token
 *   k_pool, v_pool [num_pages, Hkv, page_size, D]       page pools
 *   block_table   [S, max_pages_per_seq] int32         logical page -> physical page
 *   context_lens  [S] int32                            cached positions per sequence,
 *                                                      the new token's own K/V included
 *   scale         multiplies q.k
 *   o             [S, Hq, D]     out: softmax over the sequence's positions of
 *                                scale q.k, times v (no mask inside the context)
 *   lse           [S, Hq] or NULL  out: natural-log log-sum-exp of each score row
 *   workspace     device scratch of attn_paged_decode_workspace_bytes(...) bytes
 * q, k_pool, v_pool, o, workspace 16-byte aligned; the int32 tables and lse
 * 4-byte aligned; o, lse and workspace may not overlap an input or each other.
 * Position t of sequence s is read from
 *   pool[block_table[s, t / page_size], kv_head, t % page_size, :].
 * Device-side preconditions (not checked on the host): 1 <= context_lens[s] <=
 * max_pages_per_seq * page_size and 0 <= block_table[s, p] < num_pages for
 * p < ceil(context_lens[s] / page_size).  Entries past that are never read, and
 * pool slots past a sequence's length are never used, so they may hold anything.
 * A violated precondition gives wrong numbers but never an out-of-bounds access.
 * With the environment variable ATTN_DEBUG_CHECKS=1 (read once per process) the call
 * first checks them on the device and waits for the stream; a violation returns
 * ATTN_INVALID_ARGUMENT naming the first offending sequence (and page) and nothing
 * is launched.  The check is skipped while the stream is being captured into a graph.
 */
attn_status attn_paged_decode(const float* q, const float* k_pool, const float* v_pool,
                              const int32_t* block_table, const int32_t* context_lens,
                              int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                              int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages,
                              float scale, float* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_paged_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace and allocates and frees nothing: the partial results of the split path
 * go to a static scratch array of ATTN_PAGED_DECODE_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on, from its first use there until the process
 * ends (its address is looked up once per device).  Arguments, outputs, device-side
 * preconditions and results are those of attn_paged_decode (the same kernels).
 * Up to 1024 sequences the batch needs
 *   (W + S) * Hq * (D + 2) * 4 + 8 * S bytes of scratch, W = min(1024, 4 * CUs / (w * ceil(Hkv / w))),
 * w = min(Hkv, 4) (CUs: the device's compute units; 4.5 MB for 32 sequences of 16
 * query heads, d = 64, on 256 CUs); a batch that needs more returns
 * ATTN_WORKSPACE_TOO_SMALL (attn_paged_decode takes a workspace of any size).  More
 * than 1024 sequences need none.  The scratch's contents on entry do not matter.
 * ATTN_DEBUG_CHECKS=1 checks the tables first, as for attn_paged_decode.
 * Every call on one GPU uses that GPU's one scratch array, so calls that overlap in
 * time on one GPU (from several streams or threads) race and may give wrong results:
 * order them, e.g. on one stream.
 */
#define ATTN_PAGED_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
attn_status attn_paged_decode_noalloc(const float* q, const float* k_pool, const float* v_pool,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                                      int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages,
                                      float scale, float* o, float* lse, void* stream);

/*
 * Batched prefill over a paged K/V cache, for a ragged batch: sequence s brings
 * n_s = token_start[s+1] - token_start[s] new tokens (n_s may be 0), whose K/V
 * rows are already in the cache (attn_kv_append_tokens), so that it now holds
 * context_lens[s] >= n_s positions.  New token j of sequence s sits at position
 *   t = context_lens[s] - n_s + j
 * and attends to positions 0 .. t of its sequence (keys past t are excluded), each
 * read in place through the block table as in attn_paged_decode.
 *   q             [N, Hq, D]      new tokens' queries, sequence by sequence:
 *                                 row token_start[s] + j is token j of sequence s
 *   k_pool, v_pool [num_pages, Hkv, page_size, D]
 *   block_table   [S, max_pages_per_seq] int32;  context_lens [S] int32
 *   token_start   [S + 1] int32   nondecreasing, token_start[0] = 0, token_start[S] = N
 *   o             [N, Hq, D]      out;  lse [N, Hq] or NULL: out, natural log
 * N >= 1.  q, pools, o 16-byte aligned; int32 arrays and lse 4-byte aligned; o and
 * lse overlap no input or each other.  D in {8,16,32,64,128}, page_size in
 * {16,32,64}, Hq % Hkv == 0.  With n_s = 1 for every s this is attn_paged_decode;
 * with context_lens[s] = n_s it is attn_causal_fwd on the sequence's rows.
 * Device-side preconditions (not checked on the host; violated ones give wrong
 * numbers but never an out-of-bounds access): the token_start properties above,
 * n_s <= context_lens[s] <= max_pages_per_seq * page_size, and table entries
 * below ceil(context_lens[s] / page_size) in [0, num_pages).  ATTN_DEBUG_CHECKS=1
 * checks them first, as for attn_paged_decode.
 */
attn_status attn_paged_prefill(const float* q, const float* k_pool, const float* v_pool,
                               const int32_t* block_table, const int32_t* context_lens,
                               const int32_t* token_start, int64_t S, int64_t N,
                               int64_t Hq, int64_t Hkv, int64_t D,
                               int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages,
                               float scale, float* o, float* lse, void* stream);

/*
 * Materialized causal attention: the same O and LSE as attn_causal_fwd, plus
 *   p  [B, Hq, T, T] float32   p[b,h,i,j] = exp(scale q_i.k_j - lse[b,h,i]) for
 *                              j <= i and 0 for j > i (every row sums to 1).
 * o, p 16-byte aligned, lse 4-byte aligned; no output overlaps an input or
 * another output.  B*Hq*T*T must stay below 2^40 elements.  Shapes and
 * supported D as for attn_causal_fwd.
 */
attn_status attn_materialized_fwd(const float* q, const float* k, const float* v,
                                  int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                                  float scale, float* o, float* lse, float* p, void* stream);

/* Bytes of device workspace attn_materialized_bwd needs (0 when a size is invalid). */
size_t attn_materialized_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D);

/*
 * VJP of the materialized path for L = sum(dout * O) + sum(dp * P), with the
 * stored probabilities p (as written by attn_materialized_fwd; entries above the
 * diagonal are taken as 0) and o the matching output:
 *   dV = P^T dout,  dP = dout V^T + dp,  Delta_i = sum_j P_ij dP_ij,
 *   dS = P (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q,
 * with dK, dV summed over the query heads of each key/value head.  dp
 * [B,Hq,T,T] may be NULL (no loss on P).  Alignment, overlap and workspace rules
 * as for attn_causal_bwd.  dQ accumulates with float atomics (last bits may vary);
 * dK and dV are deterministic.
 */
attn_status attn_materialized_bwd(const float* q, const float* k, const float* v,
                                  const float* o, const float* p, const float* dout, const float* dp,
                                  int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                                  float scale, float* dq, float* dk, float* dv,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged K/V cache maintenance: the step before attn_paged_decode.
 *
 * State, all in device memory and owned by the caller (one set per layer):
 *   k_pool, v_pool  [num_pages, Hkv, page_size, D] float32
 *   block_table     [S, max_pages_per_seq] int32   logical page -> physical page
 *   context_lens    [S] int32                      cached positions per sequence
 *   free_pages      [num_pages] int32              stack of free physical pages;
 *   free_count      [1] int32                      entries 0 .. free_count-1 are free,
 *                                                  free_pages[free_count-1] is the top
 *   kv_status       [1] int32                      outcome of the last call (below)
 * Initial state: every page free (free_pages a permutation of 0 .. num_pages-1,
 * free_count = num_pages), every context length 0.
 *
 * The outcome is written to kv_status on the device, because the calls do not
 * wait for the stream: ATTN_KV_OK, or one of the codes below, in which case the
 * call changed nothing else.
 */
enum {
    ATTN_KV_OK = 0,
    ATTN_KV_POOL_EXHAUSTED = 1, /* append: fewer free pages than sequences starting a page */
    ATTN_KV_SEQUENCE_FULL = 2,  /* append: a sequence already holds max_pages_per_seq * page_size */
    ATTN_KV_STACK_OVERFLOW = 3  /* release: the free stack would exceed num_pages (a page
                                   released twice) */
};

/*
 * Appends one position to each of the S sequences:
 *   k_new, v_new  [S, Hkv, D] float32   the newest token's key and value rows
 * For sequence s with t = context_lens[s]: when t % page_size == 0 a page is
 * leased first -- sequences needing one are ranked in index order and rank r
 * takes free_pages[free_count - 1 - r]; free_count drops by their number -- and
 * recorded as block_table[s, t / page_size].  Then
 *   k_pool[block_table[s, t / page_size], h, t % page_size, :] = k_new[s, h, :]
 * (same for v) for every KV head h, and context_lens[s] = t + 1.
 * k_new, v_new, pools 16-byte aligned; the int32 arrays 4-byte aligned; no
 * output overlaps an input or another output.  D and page_size as for
 * attn_paged_decode.  Device-side precondition: the state is consistent (every
 * page of a live sequence is outside the free stack, and the table entries below
 * ceil(context_lens[s] / page_size) are its pages).
 */
attn_status attn_kv_append(const float* k_new, const float* v_new,
                           int64_t S, int64_t Hkv, int64_t D,
                           int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages,
                           float* k_pool, float* v_pool, int32_t* block_table, int32_t* context_lens,
                           int32_t* free_pages, int32_t* free_count, int32_t* kv_status, void* stream);

/*
 * Appends n_s = token_start[s+1] - token_start[s] positions (n_s >= 0) to each of
 * the S sequences:
 *   k_new, v_new  [N, Hkv, D] float32   new rows, sequence by sequence: row
 *                                       token_start[s] + j is sequence s's j-th
 *   token_start   [S + 1] int32         nondecreasing, 0 .. N
 * For sequence s with t = context_lens[s]: the logical pages t / page_size ..
 * (t + n_s - 1) / page_size that do not exist yet are leased -- over all sequences
 * in index order, and within a sequence in logical order, the r-th page leased is
 * free_pages[free_count - 1 - r]; free_count drops by their number -- then
 *   pool[block_table[s, (t + j) / page_size], h, (t + j) % page_size, :] = new row j
 * for every KV head h, and context_lens[s] = t + n_s.  With n_s = 1 for every s
 * this is attn_kv_append.  kv_status as there: ATTN_KV_SEQUENCE_FULL if some
 * t + n_s exceeds max_pages_per_seq * page_size, ATTN_KV_POOL_EXHAUSTED if fewer
 * pages are free than leased; then nothing changes.  N >= 0 (k_new and v_new may
 * be NULL when N == 0).  Alignment and overlap rules as for attn_kv_append;
 * token_start is an input.
 */
attn_status attn_kv_append_tokens(const float* k_new, const float* v_new, const int32_t* token_start,
                                  int64_t S, int64_t N, int64_t Hkv, int64_t D,
                                  int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages,
                                  float* k_pool, float* v_pool, int32_t* block_table, int32_t* context_lens,
                                  int32_t* free_pages, int32_t* free_count, int32_t* kv_status, void* stream);

/*
 * Returns the pages of sequences seq_ids[0 .. n-1] (distinct indices in [0, S))
 * to the free stack and sets their context lengths to 0.  The pages are pushed
 * in order: sequence seq_ids[0]'s logical pages 0, 1, ..., then seq_ids[1]'s, ...
 * (the last one pushed is the next one leased).  seq_ids 4-byte aligned device
 * memory; n >= 0 (n == 0 does nothing but write ATTN_KV_OK).
 */
attn_status attn_kv_release(const int32_t* seq_ids, int64_t n, int64_t S,
                            int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages,
                            int32_t* block_table, int32_t* context_lens,
                            int32_t* free_pages, int32_t* free_count, int32_t* kv_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
