// Opt-in device-side precondition checks (ATTN_DEBUG_CHECKS=1) for the calls that
// address the paged K/V pools through block tables: attn_paged_decode (and its
// no-allocation variant) and attn_paged_prefill.
//
// Their preconditions live in device memory, so the host cannot check them without a
// copy; the kernels themselves clamp every index they derive from the tables, so a
// broken table can give wrong numbers but never an out-of-bounds access.  With the
// checks on, a call first runs attn_check_tables_kernel, which reads the lengths, the
// block-table entries in use and the ragged offsets (each within its own array),
// writes one status record, and the call waits for it and reports the first violation
// with the sequence and page it concerns ("Execution Backends and the Python ABI",
// "What the Metal slice does": a preflight that fails with an immediate, descriptive
// error; "Architecture", "Tensor conventions": incompatible inputs fail fast).
#include <climits>
#include <mutex>

#include "attn_launch.h"

namespace attn {

// The status record: kind (TableCheck), sequence, page, offending value.  One per
// device, written by every check in full, so it needs no clearing.
static __device__ __align__(16) int32_t check_record[4];

constexpr int kCheckThreads = 1024;

// One work-group: thread t checks sequences t, t + 1024, ... in order and keeps its
// first violation; the smallest violating sequence wins (its owner writes the record),
// else thread 0 writes "no violation".  A sequence's table entries are read only when
// its length has passed, and then only the ceil(len / page_size) <= max_pages in use.
__global__ __launch_bounds__(kCheckThreads) void attn_check_tables_kernel(
    const int32_t* __restrict__ CTX, const int32_t* __restrict__ BT, const int32_t* __restrict__ TS, int S, int N,
    int max_pages, int PS, int num_pages, int min_len, int32_t* __restrict__ rec) {
    __shared__ int best;
    const int tid = threadIdx.x;
    if (tid == 0) best = INT_MAX;
    __syncthreads();
    int kind = kTableOk, seq = -1, page = -1, value = 0;
    const int64_t cap = (int64_t)max_pages * PS;
    for (int s = tid; s < S && kind == kTableOk; s += kCheckThreads) {
        if (TS) {  // ragged offsets: nondecreasing from 0 to N
            const int a = TS[s], b = TS[s + 1];
            if ((s == 0 && a != 0) || b < a || (s == S - 1 && b != N)) {
                kind = kTableBadOffsets, seq = s, value = s == 0 && a != 0 ? a : b;
                break;
            }
        }
        const int len = CTX[s];
        const int need = TS ? max(min_len, TS[s + 1] - TS[s]) : min_len;  // prefill: the new tokens fit
        if (len < need || (int64_t)len > cap) {
            kind = kTableBadLength, seq = s, value = len;
            break;
        }
        const int pages = (int)(((int64_t)len + PS - 1) / PS);
        for (int p = 0; p < pages; ++p) {
            const int v = BT[(int64_t)s * max_pages + p];
            if (v < 0 || v >= num_pages) {
                kind = kTableBadPage, seq = s, page = p, value = v;
                break;
            }
        }
    }
    if (kind != kTableOk) atomicMin(&best, seq);
    __syncthreads();
    if (kind != kTableOk && seq == best) {
        rec[0] = kind;
        rec[1] = seq;
        rec[2] = page;
        rec[3] = value;
    } else if (tid == 0 && best == INT_MAX) {
        rec[0] = kTableOk;
        rec[1] = -1;
        rec[2] = -1;
        rec[3] = 0;
    }
}

static std::mutex g_check_mutex;  // one checked call at a time shares a device's record

hipError_t check_paged_tables(const int32_t* ctx, const int32_t* bt, const int32_t* ts, int64_t S, int64_t N,
                              int64_t max_pages, int64_t page_size, int64_t num_pages, int min_len,
                              hipStream_t stream, TableCheck* out) {
    std::lock_guard<std::mutex> lock(g_check_mutex);
    void* addr = nullptr;
    hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(check_record));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_check_tables_kernel, dim3(1), dim3(kCheckThreads), 0, stream, ctx, bt, ts, (int)S,
                       (int)N, (int)max_pages, (int)page_size, (int)num_pages, min_len, (int32_t*)addr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int32_t rec[4] = {0, 0, 0, 0};
    if ((e = hipMemcpyAsync(rec, addr, sizeof(rec), hipMemcpyDeviceToHost, stream)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
    out->kind = rec[0];
    out->seq = rec[1];
    out->page = rec[2];
    out->value = rec[3];
    return hipSuccess;
}

}  // namespace attn
