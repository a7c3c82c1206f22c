// Paged K/V cache maintenance on gfx950: the step before single-token decode.
//
// What is computed: "Architecture", "Serving boundary" -- a request owns a
// logical page table and the pool leases physical pages from shared per-layer
// key/value pools; each new token's K/V is appended before attention reads it.
// "Execution Backends and the Python ABI", "Incremental attention" -- pools are
// [physical_page, H, page_offset, d_h] and the table maps logical to physical
// page ids.
//
// The free pages form a stack in device memory (free_pages[0 .. free_count-1],
// top at free_count-1), so leasing and releasing need no host round trip and the
// whole serving step stays on the stream:
//   1. attn_kv_lease (one work-group): finds the sequences whose next position
//      starts a page, ranks them in index order with a block-wide scan and gives
//      rank r the page free_pages[free_count - 1 - r].  If a sequence is full or
//      the stack is short, it writes the status code and changes nothing.
//   2. attn_kv_write (one work-group per sequence): if the status is OK, copies
//      the token's Hkv x D key and value rows into their page slot (16-byte
//      vectors) and advances the sequence's length.
//   attn_kv_release (one work-group) pushes the pages of the given sequences
//   back, in order, and zeroes their lengths.
//   attn_kv_append_tokens does the same for a ragged batch of several new rows per
//   sequence (the step before a batched prefill): one lease work-group, then one
//   wave per new row.
// The work is a few kilobytes per call; the kernels are latency bound by design
// (one block-wide scan, one vector copy), not HBM bound.
#include "attn_launch.h"
#include "device_common.h"

namespace attn {

constexpr int kScanThreads = 1024;

// Exclusive prefix sum of x over the work-group (kScanThreads threads, 16 waves): each
// wave scans its 64 values on DPP moves, the 16 wave totals go through LDS (`buf`, at
// least 16 ints), and each thread adds the totals of the waves before its own.  The
// group's total goes to *total.  Two barriers.
__device__ __forceinline__ int block_exclusive_scan(int x, int* buf, int* total) {
    constexpr int NW = kScanThreads / 64;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int incl = wave_incl_scan(x);
    if (lane == 63) buf[wv] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = buf[i];
        before += i < wv ? t : 0;
        all += t;
    }
    *total = all;
    __syncthreads();  // buf is reused by the next call
    return before + incl - x;
}

// Largest single-token append that the lease work-group also copies itself (float4
// copies of each of K and V, 4 per thread), saving the second launch; larger batches
// take one copy work-group per sequence.
constexpr int kKvFusedCopies = 4 * kScanThreads;

// WRITE (at most kScanThreads sequences, kKvFusedCopies float4 of each of K and V): the
// same work-group also copies the token's rows.  Everything that does not depend on the
// lease -- the new rows, the stack height, each sequence's current page -- is loaded at
// the start, so the call costs two dependent rounds of loads (lengths, then the leased
// page ids) before the stores.
template <bool WRITE>
__global__ __launch_bounds__(kScanThreads) void attn_kv_lease_kernel(
    int32_t* __restrict__ BT, int32_t* __restrict__ CTX, const int32_t* __restrict__ FREE,
    int32_t* __restrict__ FCOUNT, int32_t* __restrict__ STATUS, int S, int PS, int max_pages,
    const float* __restrict__ Kn, const float* __restrict__ Vn, float* __restrict__ Kp, float* __restrict__ Vp,
    int Hkv, int D, int num_pages) {
    constexpr int CPT = WRITE ? kKvFusedCopies / kScanThreads : 1;  // float4 copies per thread
    __shared__ int buf[kScanThreads / 64];
    __shared__ int pg[WRITE ? kScanThreads : 1], tl[WRITE ? kScanThreads : 1], fr[WRITE ? kScanThreads : 1];
    const int tid = threadIdx.x;
    const int cap = PS * max_pages;
    const int d4 = D / 4;
    const int ncopy = WRITE ? S * Hkv * d4 : 0;
    f32x4 kx[CPT], vx[CPT];
    if constexpr (WRITE) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int idx = tid + kScanThreads * k;
            if (idx < ncopy) {
                kx[k] = *(const f32x4*)(Kn + 4 * (size_t)idx);  // rows [S, Hkv, D]: float4 idx
                vx[k] = *(const f32x4*)(Vn + 4 * (size_t)idx);
            }
        }
    }
    const int top = *FCOUNT;
    int needed = 0, full = 0;
    int t_own = 1, page_own = 0;  // WRITE: this thread's sequence (s = tid)
    if constexpr (WRITE) {
        // One work-group holds the whole batch (S <= kScanThreads): one scan gives both the
        // counts and each sequence's rank, and the S entries at the top of the free stack
        // are read as soon as its height is known, beside the lengths' table reads, so
        // that no global read waits on the scan.
        const int s = tid;
        const int t = s < S ? CTX[s] : 1;
        const int fi = top - 1 - tid;  // rank tid would take free_pages[top - 1 - tid]
        if (tid < S && fi >= 0 && fi < num_pages) fr[tid] = FREE[fi];
        if (s < S) {
            t_own = t;
            if (t >= 0 && t < cap && t % PS != 0) page_own = BT[(size_t)s * max_pages + t / PS];
        }
        const int f = s < S && t >= cap ? 1 : 0;
        const int nd = s < S && t >= 0 && t < cap && t % PS == 0 ? 1 : 0;
        int tot;
        const int ex = block_exclusive_scan((f << 16) | nd, buf, &tot);  // its barriers publish fr
        full = tot >> 16;
        needed = tot & 0xFFFF;
        if (full > 0 || needed > top) {
            if (tid == 0) *STATUS = full > 0 ? ATTN_KV_SEQUENCE_FULL : ATTN_KV_POOL_EXHAUSTED;
            return;  // uniform
        }
        if (nd) {  // rank = the sequences before it that start a page (none is full here)
            const int leased = fr[ex & 0xFFFF];
            BT[(size_t)s * max_pages + t / PS] = leased;
            page_own = leased;
        }
    } else {
        // pass 1: how many sequences start a page, and is any sequence full (one scan of
        // both counts, full ones in the high half: each is at most kScanThreads per chunk)
        for (int base = 0; base < S; base += kScanThreads) {
            const int s = base + tid;
            const int t = s < S ? CTX[s] : 1;
            const int f = s < S && t >= cap ? 1 : 0;
            const int nd = s < S && t >= 0 && t < cap && t % PS == 0 ? 1 : 0;
            int tot;
            block_exclusive_scan((f << 16) | nd, buf, &tot);
            full += tot >> 16;
            needed += tot & 0xFFFF;
        }
        if (full > 0 || needed > top) {
            if (tid == 0) *STATUS = full > 0 ? ATTN_KV_SEQUENCE_FULL : ATTN_KV_POOL_EXHAUSTED;
            return;  // uniform
        }
        // pass 2: rank r (index order) takes free_pages[top - 1 - r]
        int offset = 0;
        for (int base = 0; base < S; base += kScanThreads) {
            const int s = base + tid;
            const int t = s < S ? CTX[s] : 1;
            const bool need = s < S && t >= 0 && t % PS == 0;  // t < cap: no sequence is full here
            int tot;
            const int rank = offset + block_exclusive_scan(need ? 1 : 0, buf, &tot);
            if (need) BT[(size_t)s * max_pages + t / PS] = FREE[top - 1 - rank];
            offset += tot;
        }
    }
    if constexpr (WRITE) {
        if (tid < S) {
            tl[tid] = t_own;
            pg[tid] = page_own;
        }
        __syncthreads();  // pages and positions of every sequence are in LDS
        // a table entry outside the pool (a broken state) is clamped: wrong data, never an
        // out-of-bounds write; a negative length (broken) leaves its sequence alone
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int idx = tid + kScanThreads * k;
            if (idx < ncopy) {
                const int s = idx / (Hkv * d4), h = (idx / d4) % Hkv, c = idx % d4;
                const int t = tl[s];
                if (t >= 0) {
                    const int page = min(max(pg[s], 0), num_pages - 1);
                    const size_t dst = (((size_t)page * Hkv + h) * PS + t % PS) * D + 4 * c;
                    *(f32x4*)(Kp + dst) = kx[k];
                    *(f32x4*)(Vp + dst) = vx[k];
                }
            }
        }
        if (tid < S && t_own >= 0) CTX[tid] = t_own + 1;
    }
    if (tid == 0) {
        *FCOUNT = top - needed;
        *STATUS = ATTN_KV_OK;
    }
}

__global__ __launch_bounds__(256) void attn_kv_write_kernel(
    const float* __restrict__ Kn, const float* __restrict__ Vn, float* __restrict__ Kp, float* __restrict__ Vp,
    const int32_t* __restrict__ BT, int32_t* __restrict__ CTX, const int32_t* __restrict__ STATUS, int Hkv,
    int D, int PS, int max_pages, int num_pages) {
    if (*STATUS != ATTN_KV_OK) return;  // uniform: the lease failed, change nothing
    const int s = blockIdx.x;
    const int t = CTX[s];
    if (t < 0) return;  // uniform; a broken length (the lease found no sequence full, so t < cap)
    // a table entry outside the pool (a broken state) is clamped: wrong data, never an
    // out-of-bounds write
    const int page = min(max(BT[(size_t)s * max_pages + t / PS], 0), num_pages - 1);
    const int d4 = D / 4;
    for (int idx = threadIdx.x; idx < Hkv * d4; idx += blockDim.x) {
        const int h = idx / d4, c = idx % d4;
        const size_t src = ((size_t)s * Hkv + h) * D + 4 * c;
        const size_t dst = (((size_t)page * Hkv + h) * PS + t % PS) * D + 4 * c;
        *(f32x4*)(Kp + dst) = *(const f32x4*)(Kn + src);
        *(f32x4*)(Vp + dst) = *(const f32x4*)(Vn + src);
    }
    __syncthreads();  // every thread has used t
    if (threadIdx.x == 0) CTX[s] = t + 1;
}

__global__ __launch_bounds__(kScanThreads) void attn_kv_release_kernel(
    const int32_t* __restrict__ IDS, int n, int32_t* __restrict__ BT, int32_t* __restrict__ CTX,
    int32_t* __restrict__ FREE, int32_t* __restrict__ FCOUNT, int32_t* __restrict__ STATUS, int S, int PS,
    int max_pages, int num_pages) {
    __shared__ int buf[kScanThreads / 64];
    const int tid = threadIdx.x;
    const int cap = PS * max_pages;
    auto pages_of = [&](int i) -> int {  // pages held by sequence IDS[i] (0 for an index out of range)
        if (i >= n) return 0;
        const int s = IDS[i];
        if (s < 0 || s >= S) return 0;
        const int t = min(max(CTX[s], 0), cap);
        return (t + PS - 1) / PS;
    };
    int total = 0;
    for (int base = 0; base < n; base += kScanThreads) {
        int tot;
        block_exclusive_scan(pages_of(base + tid), buf, &tot);
        total += tot;
    }
    const int top = *FCOUNT;
    if (top + total > num_pages) {
        if (tid == 0) *STATUS = ATTN_KV_STACK_OVERFLOW;
        return;  // uniform
    }
    int offset = 0;
    for (int base = 0; base < n; base += kScanThreads) {
        const int i = base + tid;
        const int np = pages_of(i);
        int tot;
        const int at = top + offset + block_exclusive_scan(np, buf, &tot);
        for (int p = 0; p < np; ++p) FREE[at + p] = BT[(size_t)IDS[i] * max_pages + p];
        offset += tot;
    }
    __syncthreads();  // every length has been read
    for (int base = 0; base < n; base += kScanThreads) {
        const int i = base + tid;
        if (i < n && IDS[i] >= 0 && IDS[i] < S) CTX[IDS[i]] = 0;
    }
    if (tid == 0) {
        *FCOUNT = top + total;
        *STATUS = ATTN_KV_OK;
    }
}

// Ragged multi-token append (the step before a batched prefill): sequence s brings
// n_s = token_start[s+1] - token_start[s] new rows.  One work-group leases, in index
// order, the pages each sequence's new positions start -- sequence s's k-th new page
// (logical order) is the (o_s + k)-th from the top of the stack, o_s the pages taken
// by the sequences before it -- records them in the table and sets the new lengths;
// if a sequence would pass its capacity or the stack is short it writes the status
// and changes nothing.  (With one token per sequence this is the single-token lease.)
__device__ __forceinline__ int tokens_of(const int32_t* __restrict__ TS, int s, int N) {
    const int a = min(max(TS[s], 0), N), b = min(max(TS[s + 1], 0), N);
    return max(b - a, 0);  // a broken (decreasing) table counts as no tokens
}

__global__ __launch_bounds__(kScanThreads) void attn_kv_lease_tokens_kernel(
    int32_t* __restrict__ BT, int32_t* __restrict__ CTX, const int32_t* __restrict__ TS,
    const int32_t* __restrict__ FREE, int32_t* __restrict__ FCOUNT, int32_t* __restrict__ STATUS, int S, int N,
    int PS, int max_pages) {
    __shared__ int buf[kScanThreads / 64];
    const int tid = threadIdx.x;
    const int cap = PS * max_pages;
    auto new_pages = [&](int t, int n) { return (t + n + PS - 1) / PS - (t + PS - 1) / PS; };
    int needed = 0, full = 0;
    for (int base = 0; base < S; base += kScanThreads) {
        const int s = base + tid;
        const int t = s < S ? max(CTX[s], 0) : 0;
        const int n = s < S ? tokens_of(TS, s, N) : 0;
        int tot;
        block_exclusive_scan(s < S && t + n > cap ? 1 : 0, buf, &tot);
        full += tot;
        block_exclusive_scan(s < S && t + n <= cap ? new_pages(t, n) : 0, buf, &tot);
        needed += tot;
    }
    const int top = *FCOUNT;
    if (full > 0 || needed > top) {
        if (tid == 0) *STATUS = full > 0 ? ATTN_KV_SEQUENCE_FULL : ATTN_KV_POOL_EXHAUSTED;
        return;  // uniform
    }
    int offset = 0;
    for (int base = 0; base < S; base += kScanThreads) {
        const int s = base + tid;
        const int t = s < S ? max(CTX[s], 0) : 0;
        const int n = s < S ? tokens_of(TS, s, N) : 0;
        const int np = s < S ? new_pages(t, n) : 0;
        int tot;
        const int rank = offset + block_exclusive_scan(np, buf, &tot);
        const int p0 = (t + PS - 1) / PS;  // first logical page to lease
        for (int k = 0; k < np; ++k) BT[(size_t)s * max_pages + p0 + k] = FREE[top - 1 - (rank + k)];
        if (s < S) CTX[s] = t + n;
        offset += tot;
    }
    if (tid == 0) {
        *FCOUNT = top - needed;
        *STATUS = ATTN_KV_OK;
    }
}

// One wave per new row r: its sequence is the last s with token_start[s] <= r (a
// ballot over the table, 64 sequences at a time), its position new_length - n_s +
// (r - token_start[s]); the Hkv x D key and value rows go to that page slot.
__global__ __launch_bounds__(256) void attn_kv_write_tokens_kernel(
    const float* __restrict__ Kn, const float* __restrict__ Vn, float* __restrict__ Kp, float* __restrict__ Vp,
    const int32_t* __restrict__ BT, const int32_t* __restrict__ CTX, const int32_t* __restrict__ TS,
    const int32_t* __restrict__ STATUS, int S, int N, int Hkv, int D, int PS, int max_pages, int num_pages) {
    if (*STATUS != ATTN_KV_OK) return;  // uniform: the lease failed, change nothing
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (r >= N) return;  // wave-uniform
    int count = 0;  // sequences s < S with token_start[s] <= r
    for (int c0 = 0; c0 < S; c0 += 64) {
        const int s = c0 + lane;
        count += __popcll(__ballot(s < S && TS[min(s, S - 1)] <= r));
    }
    const int s = count - 1;
    if (s < 0) return;  // wave-uniform: r precedes every sequence (a broken table)
    const int n = tokens_of(TS, s, N);
    const int j = r - TS[s];
    if (j < 0 || j >= n) return;  // wave-uniform: not a row of sequence s
    const int pos = CTX[s] - n + j;
    if (pos < 0 || pos >= PS * max_pages) return;  // wave-uniform; a broken state
    const int page = min(max(BT[(size_t)s * max_pages + pos / PS], 0), num_pages - 1);
    const int d4 = D / 4;
    for (int idx = lane; idx < Hkv * d4; idx += 64) {
        const int h = idx / d4, c = idx % d4;
        const size_t src = ((size_t)r * Hkv + h) * D + 4 * c;
        const size_t dst = (((size_t)page * Hkv + h) * PS + pos % PS) * D + 4 * c;
        *(f32x4*)(Kp + dst) = *(const f32x4*)(Kn + src);
        *(f32x4*)(Vp + dst) = *(const f32x4*)(Vn + src);
    }
}

hipError_t launch_kv_append_tokens(const KvAppendTokensArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(attn_kv_lease_tokens_kernel, dim3(1), dim3(kScanThreads), 0, stream, a.block_table,
                       a.context_lens, a.token_start, a.free_pages, a.free_count, a.status, (int)a.S, (int)a.N,
                       (int)a.page_size, (int)a.max_pages);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.N == 0) return e;
    hipLaunchKernelGGL(attn_kv_write_tokens_kernel, dim3((unsigned)((a.N + 3) / 4)), dim3(256), 0, stream, a.k_new,
                       a.v_new, a.k_pool, a.v_pool, a.block_table, a.context_lens, a.token_start, a.status,
                       (int)a.S, (int)a.N, (int)a.Hkv, (int)a.D, (int)a.page_size, (int)a.max_pages,
                       (int)a.num_pages);
    return hipGetLastError();
}

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
    if (a.S <= kScanThreads && a.S * a.Hkv * (a.D / 4) <= kKvFusedCopies) {  // lease and copy in one launch
        hipLaunchKernelGGL(attn_kv_lease_kernel<true>, dim3(1), dim3(kScanThreads), 0, stream, a.block_table,
                           a.context_lens, a.free_pages, a.free_count, a.status, (int)a.S, (int)a.page_size,
                           (int)a.max_pages, a.k_new, a.v_new, a.k_pool, a.v_pool, (int)a.Hkv, (int)a.D,
                           (int)a.num_pages);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(attn_kv_lease_kernel<false>, dim3(1), dim3(kScanThreads), 0, stream, a.block_table,
                       a.context_lens, a.free_pages, a.free_count, a.status, (int)a.S, (int)a.page_size,
                       (int)a.max_pages, nullptr, nullptr, nullptr, nullptr, 0, 0, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_kv_write_kernel, dim3((unsigned)a.S), dim3(256), 0, stream, a.k_new, a.v_new,
                       a.k_pool, a.v_pool, a.block_table, a.context_lens, a.status, (int)a.Hkv, (int)a.D,
                       (int)a.page_size, (int)a.max_pages, (int)a.num_pages);
    return hipGetLastError();
}

hipError_t launch_kv_release(const KvReleaseArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(attn_kv_release_kernel, dim3(1), dim3(kScanThreads), 0, stream, a.seq_ids, (int)a.n,
                       a.block_table, a.context_lens, a.free_pages, a.free_count, a.status, (int)a.S,
                       (int)a.page_size, (int)a.max_pages, (int)a.num_pages);
    return hipGetLastError();
}

}  // namespace attn
