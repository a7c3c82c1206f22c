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
 * returns.  Outputs are fully overwritten.  A call validates its arguments on the
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

#define ATTN_ABI_VERSION 0x00010000u /* 1.0: major << 16 | minor */

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
 * any input or each other.  T * D and B * Hq must stay below 2^31.
 */
attn_status attn_causal_fwd(const float* q, const float* k, const float* v,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                            float scale, float* o, float* lse, void* stream);

/* Bytes of device workspace attn_causal_bwd needs for these sizes (0 when a
 * size is invalid). */
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
 * size is invalid). */
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
 */
attn_status attn_paged_decode(const float* q, const float* k_pool, const float* v_pool,
                              const int32_t* block_table, const int32_t* context_lens,
                              int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                              int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages,
                              float scale, float* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
