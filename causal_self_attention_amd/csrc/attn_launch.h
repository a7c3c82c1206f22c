// Internal host-side launch interface between the C ABI (attn_api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/attn.h"

namespace attn {

struct FwdArgs {
    const float *q, *k, *v;
    float *o, *lse;
    int64_t B, Hq, Hkv, T, D;
    float scale;
    int cu_count;  // compute units of the device (work ordering)
};

struct BwdArgs {
    const float *q, *k, *v, *o, *lse, *dout;
    float *dq, *dk, *dv;
    float* delta;  // workspace: Delta [B, Hq, T], then the finer cut's dK, dV pieces
    int64_t B, Hq, Hkv, T, D;
    float scale;
    int cu_count;
    const float* p = nullptr;    // materialized variant: stored probabilities [B, Hq, T, T]
    const float* dpx = nullptr;  // materialized variant: cotangent of P (may be NULL)
};

struct MatFwdArgs {
    const float *q, *k, *v;
    float *o, *lse, *p;  // p: [B, Hq, T, T]
    int64_t B, Hq, Hkv, T, D;
    float scale;
    int cu_count;
};

struct DecodeArgs {
    const float *q, *k_pool, *v_pool;
    const int32_t *block_table, *context_lens;
    float *o, *lse;  // lse may be NULL
    float* partial;  // workspace (see decode_workspace_floats)
    int64_t S, Hq, Hkv, D, page_size, max_pages, num_pages;
    float scale;
    int cu_count;   // compute units of the device (choice of the fused or the split path)
    int64_t slots;  // partial slots the workspace is laid out for (at least the split grid + S)
};

struct KvAppendArgs {
    const float *k_new, *v_new;
    float *k_pool, *v_pool;
    int32_t *block_table, *context_lens, *free_pages, *free_count, *status;
    int64_t S, Hkv, D, page_size, max_pages, num_pages;
};

struct KvAppendTokensArgs {
    const float *k_new, *v_new;  // [N, Hkv, D]
    const int32_t* token_start;  // [S + 1]
    float *k_pool, *v_pool;
    int32_t *block_table, *context_lens, *free_pages, *free_count, *status;
    int64_t S, N, Hkv, D, page_size, max_pages, num_pages;
};

struct PrefillArgs {
    const float *q, *k_pool, *v_pool;  // q [N, Hq, D]
    const int32_t *block_table, *context_lens, *token_start;
    float *o, *lse;  // o [N, Hq, D]; lse [N, Hq] or NULL
    int64_t S, N, Hq, Hkv, D, page_size, max_pages, num_pages;
    float scale;
};

struct KvReleaseArgs {
    const int32_t* seq_ids;
    int64_t n, S;
    int32_t *block_table, *context_lens, *free_pages, *free_count, *status;
    int64_t page_size, max_pages, num_pages;
};

// Work ordering for triangular (causal) grids.  Work items are ranked heaviest
// first; work-group ids are dealt to the compute units in rounds of `ncu`, and
// every second round is reversed, so the work-groups that end up sharing a
// compute unit pair heavy items with light ones.  Returns the rank of `id`.
__device__ __forceinline__ int snake_rank(int id, int n, int ncu) {
    const int round = id / ncu;
    const int base = round * ncu;
    const int m = n - base < ncu ? n - base : ncu;
    return (round & 1) ? base + (m - 1 - (id - base)) : id;
}

// XCD-aware work order.  Work-group x runs on XCD x % kXcds (round-robin dispatch over
// the 8 XCDs, each with its own L2).  Work items come in groups of G consecutive
// indices that read the same K/V (the query heads of one KV head); this maps work-group x
// to an item index so that the G items of a group go to work-groups on one XCD in
// consecutive dispatch slots -- x = (grp % 8) + 8 * ((grp / 8) * G + i) for item
// grp * G + i -- and their K/V tiles are fetched into that XCD's L2 once.  The order of
// the groups is kept to within 8 groups, and x + 8 G m maps to the item 8 G m further on
// (so a pairing of work-groups x and x + ncu with ncu a multiple of 8 G is preserved).
// Returns -1 for the padding work-groups past the last group (the grid is rounded up to
// whole sets of 8 groups).  G == 1 is the identity.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_grouped_item(int x, int G, int ngroups) {
    if (G == 1) return x < ngroups ? x : -1;
    const int slot = x / kXcds;
    const int grp = (slot / G) * kXcds + x % kXcds;
    return grp < ngroups ? grp * G + slot % G : -1;
}
inline int64_t xcd_grouped_grid(int64_t G, int64_t ngroups) {
    return G == 1 ? ngroups : (ngroups + kXcds - 1) / kXcds * kXcds * G;
}

// Kernels exist for these head widths / page sizes.
bool causal_head_dim_supported(int64_t D);
bool decode_shape_supported(int64_t D, int64_t page_size, int64_t group);

// Workspace sizes in floats.
size_t bwd_workspace_floats(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D);
// Work-groups of the backward's finer cut at most (two per CU of a 256-CU chip; it
// bounds that cut's workspace)
constexpr int64_t kBwdMaxRunWgs = 512;
size_t decode_workspace_floats(int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t max_pages);
// Partial slots of the caller-workspace layout (device independent: the largest split grid).
int64_t decode_workspace_slots(int64_t S);

// The decode's own static scratch (for callers that cannot allocate): the slots the split
// path needs on a device with cu_count compute units (0 when the fused path takes the
// batch), the floats they occupy, the scratch's capacity in floats, and its address on
// the current device (looked up once per device).
int64_t decode_scratch_slots(int64_t S, int64_t Hkv, int cu_count);
size_t decode_scratch_floats(int64_t S, int64_t Hq, int64_t D, int64_t slots);
size_t decode_scratch_capacity_floats();
hipError_t decode_scratch_address(float** ptr);

// Opt-in checks of the block tables, lengths and ragged offsets (ATTN_DEBUG_CHECKS=1):
// the first violation, by sequence.  The call waits for the stream.
enum { kTableOk = 0, kTableBadLength = 1, kTableBadPage = 2, kTableBadOffsets = 3 };
struct TableCheck {
    int32_t kind, seq, page, value;
};
// min_len: the smallest valid length (1 for decode, 0 for prefill, where a sequence
// also needs at least its new tokens); ts may be NULL (decode).
hipError_t check_paged_tables(const int32_t* ctx, const int32_t* bt, const int32_t* ts, int64_t S, int64_t N,
                              int64_t max_pages, int64_t page_size, int64_t num_pages, int min_len,
                              hipStream_t stream, TableCheck* out);

hipError_t launch_causal_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_causal_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_materialized_fwd(const MatFwdArgs& a, hipStream_t stream);
hipError_t launch_materialized_bwd(const BwdArgs& a, hipStream_t stream);  // a.p set
hipError_t launch_mat_delta(const float* p, const float* dpx, float* delta, int64_t rows, int64_t T,
                            hipStream_t stream);
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream);
hipError_t launch_kv_append_tokens(const KvAppendTokensArgs& a, hipStream_t stream);
hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_kv_release(const KvReleaseArgs& a, hipStream_t stream);

}  // namespace attn
