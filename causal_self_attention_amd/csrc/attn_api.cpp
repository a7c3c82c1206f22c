// C ABI of the attention library: argument validation, error reporting and
// dispatch to the gfx950 kernels.
//
// Conventions ("Execution Backends and the Python ABI", "Stable C ABI"): status
// returns, thread-local error details, every exception caught at the boundary,
// no C++ type in the signatures.  Shapes are checked before anything else runs
// ("Architecture", "Tensor conventions": incompatible shapes fail immediately),
// and all checks finish before the first HIP call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace {

thread_local std::string g_last_error;

attn_status fail(attn_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

attn_status ok() {
    g_last_error.clear();
    return ATTN_OK;
}

struct Range {
    const void* p;
    size_t bytes;
    const char* name;
};

bool overlaps(const Range& a, const Range& b) {
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output range must be disjoint from every input and every other output.
attn_status check_disjoint(std::initializer_list<Range> outs, std::initializer_list<Range> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Range& i : ins)
            if (overlaps(*o, i))
                return fail(ATTN_INVALID_ARGUMENT,
                            std::string("output '") + o->name + "' overlaps input '" + i.name + "'");
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(*o, *o2))
                return fail(ATTN_INVALID_ARGUMENT,
                            std::string("outputs '") + o->name + "' and '" + o2->name + "' overlap");
    }
    return ATTN_OK;
}

attn_status check_ptr(const void* p, const char* name, size_t align) {
    if (!p) return fail(ATTN_INVALID_ARGUMENT, std::string("'") + name + "' is NULL");
    if ((uintptr_t)p % align != 0)
        return fail(ATTN_INVALID_ARGUMENT,
                    std::string("'") + name + "' is not " + std::to_string(align) + "-byte aligned");
    return ATTN_OK;
}

#define ATTN_TRY(expr)                         \
    do {                                       \
        attn_status st_ = (expr);              \
        if (st_ != ATTN_OK) return st_;        \
    } while (0)

const int64_t kMaxElems = (int64_t)1 << 31;  // per-head T*D and index arithmetic limit

// Launch grids: one forward work-group per 64-row block and head (plus fewer than 8
// groups of Hq/Hkv padding work-groups for the XCD-grouped order); the backward's
// preprocess takes D/4 threads per row.  Both stay far below 2^31 work-groups here
// (B*Hq*T*D < 2^40 floats is 4 TB, beyond any device memory).
bool causal_grid_fits(int64_t B, int64_t Hq, int64_t T, int64_t D) {
    return (T + 63) / 64 * (B * Hq) + 8 * Hq < kMaxElems && B * Hq * T * D < ((int64_t)1 << 40);
}

// Shape checks shared by the two causal calls.
attn_status check_causal_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D, float scale) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0)
        return fail(ATTN_INVALID_ARGUMENT, "B, Hq, Hkv, T and D must all be positive (got B=" + std::to_string(B) +
                                               " Hq=" + std::to_string(Hq) + " Hkv=" + std::to_string(Hkv) +
                                               " T=" + std::to_string(T) + " D=" + std::to_string(D) + ")");
    if (Hq % Hkv != 0)
        return fail(ATTN_INVALID_ARGUMENT, "Hq % Hkv != 0: query heads cannot be grouped over the key/value heads (Hq=" +
                                               std::to_string(Hq) + ", Hkv=" + std::to_string(Hkv) + ")");
    if (!std::isfinite(scale)) return fail(ATTN_INVALID_ARGUMENT, "scale is not finite");
    if (T * D >= kMaxElems || B * Hq >= kMaxElems || T >= kMaxElems / 64)
        return fail(ATTN_INVALID_ARGUMENT, "tensor too large: T*D and B*Hq must stay below 2^31");
    if (!causal_grid_fits(B, Hq, T, D))
        return fail(ATTN_INVALID_ARGUMENT, "tensor too large: ceil(T/64)*B*Hq row blocks must stay below 2^31 and "
                                           "B*Hq*T*D below 2^40");
    if (!attn::causal_head_dim_supported(D))
        return fail(ATTN_UNSUPPORTED, "head width D=" + std::to_string(D) +
                                          " has no kernel (supported: 8, 16, 32, 64, 128)");
    return ATTN_OK;
}

// Compute-unit count of each device, read once (0 = not read yet).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

attn_status device_ready(int* cu_count) {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0)
        return fail(ATTN_DEVICE_ERROR, std::string("no HIP device: ") +
                                           (e != hipSuccess ? hipGetErrorString(e) : "device count is 0"));
    int dev = -1;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_DEVICE_ERROR, std::string("no current HIP device: ") + hipGetErrorString(e));
    int cu = (dev >= 0 && dev < kMaxDevices) ? g_cu_count[dev].load(std::memory_order_relaxed) : 0;
    if (cu <= 0) {
        e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || cu <= 0)
            return fail(ATTN_DEVICE_ERROR, std::string("cannot read the compute-unit count: ") + hipGetErrorString(e));
        if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cu, std::memory_order_relaxed);
    }
    *cu_count = cu;
    return ATTN_OK;
}

attn_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ATTN_DEVICE_ERROR, std::string(what) + ": " + hipGetErrorString(e));
    return ok();
}

// ATTN_DEBUG_CHECKS=1 (read once per process) turns on the device-side checks of the
// tables that paged decode and prefill read.
bool debug_checks() {
    static const bool on = [] {
        const char* v = std::getenv("ATTN_DEBUG_CHECKS");
        return v && v[0] == '1' && v[1] == 0;
    }();
    return on;
}

// Runs the table checks when they are on and the stream is not being captured into a
// graph (a check waits for the stream, which capture forbids); a violation becomes
// ATTN_INVALID_ARGUMENT naming the sequence and page, and nothing else is launched.
attn_status debug_check_tables(const char* fn, const int32_t* ctx, const int32_t* bt, const int32_t* ts, int64_t S,
                               int64_t N, int64_t max_pages, int64_t page_size, int64_t num_pages, int min_len,
                               hipStream_t stream) {
    if (!debug_checks()) return ATTN_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return fail(ATTN_DEVICE_ERROR, std::string(fn) + ": " + hipGetErrorString(e));
    if (cap != hipStreamCaptureStatusNone) return ATTN_OK;
    attn::TableCheck r{};
    e = attn::check_paged_tables(ctx, bt, ts, S, N, max_pages, page_size, num_pages, min_len, stream, &r);
    if (e != hipSuccess)
        return fail(ATTN_DEVICE_ERROR, std::string(fn) + ": ATTN_DEBUG_CHECKS table check: " + hipGetErrorString(e));
    const std::string s = std::to_string(r.seq);
    switch (r.kind) {
        case attn::kTableOk:
            return ATTN_OK;
        case attn::kTableBadLength:
            return fail(ATTN_INVALID_ARGUMENT,
                        std::string(fn) + ": context_lens[" + s + "] = " + std::to_string(r.value) + " is outside [" +
                            (ts ? "its new tokens" : "1") + ", max_pages_per_seq * page_size = " +
                            std::to_string(max_pages * page_size) + "] (ATTN_DEBUG_CHECKS)");
        case attn::kTableBadPage:
            return fail(ATTN_INVALID_ARGUMENT,
                        std::string(fn) + ": block_table[" + s + ", " + std::to_string(r.page) + "] = " +
                            std::to_string(r.value) + " is not a page of the pool (0 <= page < num_pages = " +
                            std::to_string(num_pages) + ") (ATTN_DEBUG_CHECKS)");
        case attn::kTableBadOffsets:
            return fail(ATTN_INVALID_ARGUMENT,
                        std::string(fn) + ": token_start is not nondecreasing from 0 to N at sequence " + s +
                            " (value " + std::to_string(r.value) + ") (ATTN_DEBUG_CHECKS)");
        default:
            return fail(ATTN_DEVICE_ERROR, std::string(fn) + ": unknown table check result");
    }
}

}  // namespace

namespace attn {
bool causal_head_dim_supported(int64_t D) { return D == 8 || D == 16 || D == 32 || D == 64 || D == 128; }
}  // namespace attn

extern "C" {

uint32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_last_error.c_str(); }

attn_status attn_causal_fwd(const float* q, const float* k, const float* v, int64_t B, int64_t Hq, int64_t Hkv,
                            int64_t T, int64_t D, float scale, float* o, float* lse, void* stream) {
    try {
        ATTN_TRY(check_causal_shape(B, Hq, Hkv, T, D, scale));
        ATTN_TRY(check_ptr(q, "q", 16));
        ATTN_TRY(check_ptr(k, "k", 16));
        ATTN_TRY(check_ptr(v, "v", 16));
        ATTN_TRY(check_ptr(o, "o", 16));
        ATTN_TRY(check_ptr(lse, "lse", 4));
        const size_t qb = (size_t)(B * Hq * T * D) * 4, kb = (size_t)(B * Hkv * T * D) * 4;
        const size_t lb = (size_t)(B * Hq * T) * 4;
        ATTN_TRY(check_disjoint({{o, qb, "o"}, {lse, lb, "lse"}}, {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, T, D, scale, cus};
        return launched(attn::launch_causal_fwd(a, (hipStream_t)stream), "attn_causal_fwd launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_causal_fwd: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_causal_fwd: unknown exception");
    }
}

size_t attn_causal_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0 || Hq % Hkv != 0) return 0;
    if (T * D >= kMaxElems || B * Hq >= kMaxElems || !causal_grid_fits(B, Hq, T, D)) return 0;
    const size_t bytes = attn::bwd_workspace_floats(B, Hq, Hkv, T, D) * 4;
    return (bytes + 255) / 256 * 256;
}

attn_status attn_causal_bwd(const float* q, const float* k, const float* v, const float* o, const float* lse,
                            const float* dout, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D, float scale,
                            float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        ATTN_TRY(check_causal_shape(B, Hq, Hkv, T, D, scale));
        ATTN_TRY(check_ptr(q, "q", 16));
        ATTN_TRY(check_ptr(k, "k", 16));
        ATTN_TRY(check_ptr(v, "v", 16));
        ATTN_TRY(check_ptr(o, "o", 16));
        ATTN_TRY(check_ptr(lse, "lse", 4));
        ATTN_TRY(check_ptr(dout, "dout", 16));
        ATTN_TRY(check_ptr(dq, "dq", 16));
        ATTN_TRY(check_ptr(dk, "dk", 16));
        ATTN_TRY(check_ptr(dv, "dv", 16));
        ATTN_TRY(check_ptr(workspace, "workspace", 16));
        const size_t need = attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D);
        if (workspace_bytes < need)
            return fail(ATTN_WORKSPACE_TOO_SMALL, "workspace has " + std::to_string(workspace_bytes) +
                                                      " bytes, attn_causal_bwd needs " + std::to_string(need));
        const size_t qb = (size_t)(B * Hq * T * D) * 4, kb = (size_t)(B * Hkv * T * D) * 4;
        const size_t lb = (size_t)(B * Hq * T) * 4;
        ATTN_TRY(check_disjoint({{dq, qb, "dq"}, {dk, kb, "dk"}, {dv, kb, "dv"}, {workspace, need, "workspace"}},
                                {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {o, qb, "o"}, {lse, lb, "lse"},
                                 {dout, qb, "dout"}}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        attn::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, (float*)workspace, B, Hq, Hkv, T, D, scale, cus};
        return launched(attn::launch_causal_bwd(a, (hipStream_t)stream), "attn_causal_bwd launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_causal_bwd: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_causal_bwd: unknown exception");
    }
}

size_t attn_paged_decode_workspace_bytes(int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                                         int64_t max_pages_per_seq) {
    if (S <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || max_pages_per_seq <= 0 || Hq % Hkv != 0)
        return 0;
    if (page_size * max_pages_per_seq >= kMaxElems || S * Hq >= kMaxElems) return 0;
    const size_t bytes = attn::decode_workspace_floats(S, Hq, Hkv, D, page_size, max_pages_per_seq) * 4;
    return (bytes + 255) / 256 * 256;
}

}  // extern "C"

namespace {

// Checks shared by the two decode calls, except for the workspace: sizes, the kernels'
// shape support and the pointers.
attn_status check_decode(const float* q, const float* k_pool, const float* v_pool, const int32_t* block_table,
                         const int32_t* context_lens, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                         int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages, float scale, float* o,
                         float* lse) {
    if (S <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || max_pages_per_seq <= 0 || num_pages <= 0)
        return fail(ATTN_INVALID_ARGUMENT,
                    "S, Hq, Hkv, D, page_size, max_pages_per_seq and num_pages must all be positive");
    if (Hq % Hkv != 0)
        return fail(ATTN_INVALID_ARGUMENT, "Hq % Hkv != 0: query heads cannot be grouped over the key/value heads");
    if (!std::isfinite(scale)) return fail(ATTN_INVALID_ARGUMENT, "scale is not finite");
    if (page_size * max_pages_per_seq >= kMaxElems || S * Hq >= kMaxElems ||
        num_pages * Hkv * page_size * D >= ((int64_t)1 << 40))
        return fail(ATTN_INVALID_ARGUMENT, "sizes too large: page_size*max_pages_per_seq must stay below 2^31");
    if (!attn::decode_shape_supported(D, page_size, Hq / Hkv))
        return fail(ATTN_UNSUPPORTED, "no decode kernel for D=" + std::to_string(D) + ", page_size=" +
                                          std::to_string(page_size) + ", Hq/Hkv=" + std::to_string(Hq / Hkv) +
                                          " (supported: D in {8,16,32,64,128}, page_size in {16,32,64}, "
                                          "1 <= Hq/Hkv <= 16)");
    ATTN_TRY(check_ptr(q, "q", 16));
    ATTN_TRY(check_ptr(k_pool, "k_pool", 16));
    ATTN_TRY(check_ptr(v_pool, "v_pool", 16));
    ATTN_TRY(check_ptr(block_table, "block_table", 4));
    ATTN_TRY(check_ptr(context_lens, "context_lens", 4));
    ATTN_TRY(check_ptr(o, "o", 16));
    if (lse) ATTN_TRY(check_ptr(lse, "lse", 4));
    return ATTN_OK;
}

// The decode outputs (and the caller's workspace, `ws`, possibly empty) overlap no input
// and no other output.
attn_status check_decode_disjoint(const float* q, const float* k_pool, const float* v_pool,
                                  const int32_t* block_table, const int32_t* context_lens, int64_t S, int64_t Hq,
                                  int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages_per_seq,
                                  int64_t num_pages, float* o, float* lse, Range ws) {
    const size_t qb = (size_t)(S * Hq * D) * 4, pb = (size_t)(num_pages * Hkv * page_size * D) * 4;
    const size_t tb = (size_t)(S * max_pages_per_seq) * 4, cb = (size_t)S * 4, lb = (size_t)(S * Hq) * 4;
    const Range lr{lse, lse ? lb : 0, "lse"};
    return check_disjoint({{o, qb, "o"}, lr, ws},
                          {{q, qb, "q"}, {k_pool, pb, "k_pool"}, {v_pool, pb, "v_pool"},
                           {block_table, tb, "block_table"}, {context_lens, cb, "context_lens"}});
}

}  // namespace

extern "C" {

attn_status attn_paged_decode(const float* q, const float* k_pool, const float* v_pool, const int32_t* block_table,
                              const int32_t* context_lens, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                              int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages, float scale, float* o,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        ATTN_TRY(check_decode(q, k_pool, v_pool, block_table, context_lens, S, Hq, Hkv, D, page_size,
                              max_pages_per_seq, num_pages, scale, o, lse));
        ATTN_TRY(check_ptr(workspace, "workspace", 16));
        const size_t need = attn_paged_decode_workspace_bytes(S, Hq, Hkv, D, page_size, max_pages_per_seq);
        if (workspace_bytes < need)
            return fail(ATTN_WORKSPACE_TOO_SMALL, "workspace has " + std::to_string(workspace_bytes) +
                                                      " bytes, attn_paged_decode needs " + std::to_string(need));
        ATTN_TRY(check_decode_disjoint(q, k_pool, v_pool, block_table, context_lens, S, Hq, Hkv, D, page_size,
                                       max_pages_per_seq, num_pages, o, lse, Range{workspace, need, "workspace"}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        ATTN_TRY(debug_check_tables("attn_paged_decode", context_lens, block_table, nullptr, S, 0, max_pages_per_seq,
                                    page_size, num_pages, 1, (hipStream_t)stream));
        attn::DecodeArgs a{q, k_pool, v_pool, block_table, context_lens, o, lse, (float*)workspace,
                           S, Hq, Hkv, D, page_size, max_pages_per_seq, num_pages, scale, cus,
                           attn::decode_workspace_slots(S)};
        return launched(attn::launch_paged_decode(a, (hipStream_t)stream), "attn_paged_decode launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_paged_decode: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_paged_decode: unknown exception");
    }
}

attn_status attn_paged_decode_noalloc(const float* q, const float* k_pool, const float* v_pool,
                                      const int32_t* block_table, const int32_t* context_lens, int64_t S, int64_t Hq,
                                      int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages_per_seq,
                                      int64_t num_pages, float scale, float* o, float* lse, void* stream) {
    try {
        ATTN_TRY(check_decode(q, k_pool, v_pool, block_table, context_lens, S, Hq, Hkv, D, page_size,
                              max_pages_per_seq, num_pages, scale, o, lse));
        ATTN_TRY(check_decode_disjoint(q, k_pool, v_pool, block_table, context_lens, S, Hq, Hkv, D, page_size,
                                       max_pages_per_seq, num_pages, o, lse, Range{nullptr, 0, "scratch"}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        const int64_t slots = attn::decode_scratch_slots(S, Hkv, cus);
        const size_t need = attn::decode_scratch_floats(S, Hq, D, slots);
        if (slots > 0 && need > attn::decode_scratch_capacity_floats())
            return fail(ATTN_WORKSPACE_TOO_SMALL,
                        "attn_paged_decode_noalloc: this batch needs " + std::to_string(need * 4) +
                            " bytes of scratch, the library's static scratch holds " +
                            std::to_string(attn::decode_scratch_capacity_floats() * 4) +
                            " (fewer sequences, query heads or head dims fit; attn_paged_decode takes a "
                            "caller workspace of any size)");
        ATTN_TRY(debug_check_tables("attn_paged_decode_noalloc", context_lens, block_table, nullptr, S, 0,
                                    max_pages_per_seq, page_size, num_pages, 1, (hipStream_t)stream));
        float* scratch = nullptr;
        if (slots > 0) {
            const hipError_t e = attn::decode_scratch_address(&scratch);
            if (e != hipSuccess)
                return fail(ATTN_DEVICE_ERROR, std::string("attn_paged_decode_noalloc: scratch address: ") +
                                                   hipGetErrorString(e));
        }
        attn::DecodeArgs a{q, k_pool, v_pool, block_table, context_lens, o, lse, scratch,
                           S, Hq, Hkv, D, page_size, max_pages_per_seq, num_pages, scale, cus, slots};
        return launched(attn::launch_paged_decode(a, (hipStream_t)stream), "attn_paged_decode_noalloc launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_paged_decode_noalloc: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_paged_decode_noalloc: unknown exception");
    }
}

attn_status attn_materialized_fwd(const float* q, const float* k, const float* v, int64_t B, int64_t Hq,
                                  int64_t Hkv, int64_t T, int64_t D, float scale, float* o, float* lse, float* p,
                                  void* stream) {
    try {
        ATTN_TRY(check_causal_shape(B, Hq, Hkv, T, D, scale));
        if (B * Hq * T * T >= ((int64_t)1 << 40))
            return fail(ATTN_INVALID_ARGUMENT, "attn_materialized_fwd: B*Hq*T*T must stay below 2^40");
        ATTN_TRY(check_ptr(q, "q", 16));
        ATTN_TRY(check_ptr(k, "k", 16));
        ATTN_TRY(check_ptr(v, "v", 16));
        ATTN_TRY(check_ptr(o, "o", 16));
        ATTN_TRY(check_ptr(lse, "lse", 4));
        ATTN_TRY(check_ptr(p, "p", 16));
        const size_t qb = (size_t)(B * Hq * T * D) * 4, kb = (size_t)(B * Hkv * T * D) * 4;
        const size_t lb = (size_t)(B * Hq * T) * 4, pb = (size_t)(B * Hq * T * T) * 4;
        ATTN_TRY(check_disjoint({{o, qb, "o"}, {lse, lb, "lse"}, {p, pb, "p"}},
                                {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        attn::MatFwdArgs a{q, k, v, o, lse, p, B, Hq, Hkv, T, D, scale, cus};
        return launched(attn::launch_materialized_fwd(a, (hipStream_t)stream), "attn_materialized_fwd launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_materialized_fwd: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_materialized_fwd: unknown exception");
    }
}

size_t attn_materialized_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D) {
    return attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D);
}

attn_status attn_materialized_bwd(const float* q, const float* k, const float* v, const float* o, const float* p,
                                  const float* dout, const float* dp, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                                  int64_t D, float scale, float* dq, float* dk, float* dv, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    try {
        ATTN_TRY(check_causal_shape(B, Hq, Hkv, T, D, scale));
        if (B * Hq * T * T >= ((int64_t)1 << 40))
            return fail(ATTN_INVALID_ARGUMENT, "attn_materialized_bwd: B*Hq*T*T must stay below 2^40");
        ATTN_TRY(check_ptr(q, "q", 16));
        ATTN_TRY(check_ptr(k, "k", 16));
        ATTN_TRY(check_ptr(v, "v", 16));
        ATTN_TRY(check_ptr(o, "o", 16));
        ATTN_TRY(check_ptr(p, "p", 4));
        ATTN_TRY(check_ptr(dout, "dout", 16));
        if (dp) ATTN_TRY(check_ptr(dp, "dp", 4));
        ATTN_TRY(check_ptr(dq, "dq", 16));
        ATTN_TRY(check_ptr(dk, "dk", 16));
        ATTN_TRY(check_ptr(dv, "dv", 16));
        ATTN_TRY(check_ptr(workspace, "workspace", 16));
        const size_t need = attn_materialized_bwd_workspace_bytes(B, Hq, Hkv, T, D);
        if (workspace_bytes < need)
            return fail(ATTN_WORKSPACE_TOO_SMALL, "workspace has " + std::to_string(workspace_bytes) +
                                                      " bytes, attn_materialized_bwd needs " + std::to_string(need));
        const size_t qb = (size_t)(B * Hq * T * D) * 4, kb = (size_t)(B * Hkv * T * D) * 4;
        const size_t pb = (size_t)(B * Hq * T * T) * 4;
        const Range dpr{dp, dp ? pb : 0, "dp"};
        ATTN_TRY(check_disjoint({{dq, qb, "dq"}, {dk, kb, "dk"}, {dv, kb, "dv"}, {workspace, need, "workspace"}},
                                {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {o, qb, "o"}, {p, pb, "p"},
                                 {dout, qb, "dout"}, dpr}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        attn::BwdArgs a{q, k, v, o, nullptr, dout, dq, dk, dv, (float*)workspace, B, Hq, Hkv, T, D, scale, cus, p, dp};
        return launched(attn::launch_materialized_bwd(a, (hipStream_t)stream), "attn_materialized_bwd launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_materialized_bwd: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_materialized_bwd: unknown exception");
    }
}

// Sizes shared by the two K/V cache calls.
static attn_status check_kv_shape(const char* fn, int64_t S, int64_t page_size, int64_t max_pages_per_seq,
                                  int64_t num_pages) {
    if (S <= 0 || page_size <= 0 || max_pages_per_seq <= 0 || num_pages <= 0)
        return fail(ATTN_INVALID_ARGUMENT,
                    std::string(fn) + ": S, page_size, max_pages_per_seq and num_pages must all be positive");
    if (page_size * max_pages_per_seq >= kMaxElems || S * max_pages_per_seq >= kMaxElems ||
        num_pages >= kMaxElems)
        return fail(ATTN_INVALID_ARGUMENT, std::string(fn) + ": sizes too large for int32 page ids and lengths");
    if (page_size != 16 && page_size != 32 && page_size != 64)
        return fail(ATTN_UNSUPPORTED, std::string(fn) + ": page_size " + std::to_string(page_size) +
                                          " is not one of 16, 32, 64");
    return ATTN_OK;
}

attn_status attn_kv_append(const float* k_new, const float* v_new, int64_t S, int64_t Hkv, int64_t D,
                           int64_t page_size, int64_t max_pages_per_seq, int64_t num_pages, float* k_pool,
                           float* v_pool, int32_t* block_table, int32_t* context_lens, int32_t* free_pages,
                           int32_t* free_count, int32_t* kv_status, void* stream) {
    try {
        ATTN_TRY(check_kv_shape("attn_kv_append", S, page_size, max_pages_per_seq, num_pages));
        if (Hkv <= 0 || D <= 0) return fail(ATTN_INVALID_ARGUMENT, "attn_kv_append: Hkv and D must be positive");
        if (num_pages * Hkv * page_size * D >= ((int64_t)1 << 40) || S * Hkv * D >= kMaxElems)
            return fail(ATTN_INVALID_ARGUMENT, "attn_kv_append: pool or rows too large");
        if (!attn::causal_head_dim_supported(D))
            return fail(ATTN_UNSUPPORTED, "attn_kv_append: head width D=" + std::to_string(D) +
                                              " is not one of 8, 16, 32, 64, 128");
        ATTN_TRY(check_ptr(k_new, "k_new", 16));
        ATTN_TRY(check_ptr(v_new, "v_new", 16));
        ATTN_TRY(check_ptr(k_pool, "k_pool", 16));
        ATTN_TRY(check_ptr(v_pool, "v_pool", 16));
        ATTN_TRY(check_ptr(block_table, "block_table", 4));
        ATTN_TRY(check_ptr(context_lens, "context_lens", 4));
        ATTN_TRY(check_ptr(free_pages, "free_pages", 4));
        ATTN_TRY(check_ptr(free_count, "free_count", 4));
        ATTN_TRY(check_ptr(kv_status, "kv_status", 4));
        const size_t nb = (size_t)(S * Hkv * D) * 4, pb = (size_t)(num_pages * Hkv * page_size * D) * 4;
        ATTN_TRY(check_disjoint({{k_pool, pb, "k_pool"}, {v_pool, pb, "v_pool"},
                                 {block_table, (size_t)(S * max_pages_per_seq) * 4, "block_table"},
                                 {context_lens, (size_t)S * 4, "context_lens"},
                                 {free_pages, (size_t)num_pages * 4, "free_pages"}, {free_count, 4, "free_count"},
                                 {kv_status, 4, "kv_status"}},
                                {{k_new, nb, "k_new"}, {v_new, nb, "v_new"}}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        attn::KvAppendArgs a{k_new, v_new, k_pool, v_pool, block_table, context_lens, free_pages, free_count,
                             kv_status, S, Hkv, D, page_size, max_pages_per_seq, num_pages};
        return launched(attn::launch_kv_append(a, (hipStream_t)stream), "attn_kv_append launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_kv_append: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_kv_append: unknown exception");
    }
}

attn_status attn_kv_append_tokens(const float* k_new, const float* v_new, const int32_t* token_start, int64_t S,
                                  int64_t N, int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages_per_seq,
                                  int64_t num_pages, float* k_pool, float* v_pool, int32_t* block_table,
                                  int32_t* context_lens, int32_t* free_pages, int32_t* free_count,
                                  int32_t* kv_status, void* stream) {
    try {
        ATTN_TRY(check_kv_shape("attn_kv_append_tokens", S, page_size, max_pages_per_seq, num_pages));
        if (Hkv <= 0 || D <= 0 || N < 0)
            return fail(ATTN_INVALID_ARGUMENT, "attn_kv_append_tokens: Hkv and D must be positive and N >= 0");
        if (num_pages * Hkv * page_size * D >= ((int64_t)1 << 40) || N * Hkv * D >= kMaxElems || S + 1 >= kMaxElems)
            return fail(ATTN_INVALID_ARGUMENT, "attn_kv_append_tokens: pool or rows too large");
        if (!attn::causal_head_dim_supported(D))
            return fail(ATTN_UNSUPPORTED, "attn_kv_append_tokens: head width D=" + std::to_string(D) +
                                              " is not one of 8, 16, 32, 64, 128");
        if (N > 0) {
            ATTN_TRY(check_ptr(k_new, "k_new", 16));
            ATTN_TRY(check_ptr(v_new, "v_new", 16));
        }
        ATTN_TRY(check_ptr(token_start, "token_start", 4));
        ATTN_TRY(check_ptr(k_pool, "k_pool", 16));
        ATTN_TRY(check_ptr(v_pool, "v_pool", 16));
        ATTN_TRY(check_ptr(block_table, "block_table", 4));
        ATTN_TRY(check_ptr(context_lens, "context_lens", 4));
        ATTN_TRY(check_ptr(free_pages, "free_pages", 4));
        ATTN_TRY(check_ptr(free_count, "free_count", 4));
        ATTN_TRY(check_ptr(kv_status, "kv_status", 4));
        const size_t nb = (size_t)(N * Hkv * D) * 4, pb = (size_t)(num_pages * Hkv * page_size * D) * 4;
        const Range kn{k_new, N > 0 ? nb : 0, "k_new"}, vn{v_new, N > 0 ? nb : 0, "v_new"};
        ATTN_TRY(check_disjoint({{k_pool, pb, "k_pool"}, {v_pool, pb, "v_pool"},
                                 {block_table, (size_t)(S * max_pages_per_seq) * 4, "block_table"},
                                 {context_lens, (size_t)S * 4, "context_lens"},
                                 {free_pages, (size_t)num_pages * 4, "free_pages"}, {free_count, 4, "free_count"},
                                 {kv_status, 4, "kv_status"}},
                                {kn, vn, {token_start, (size_t)(S + 1) * 4, "token_start"}}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        attn::KvAppendTokensArgs a{k_new, v_new, token_start, k_pool, v_pool, block_table, context_lens,
                                   free_pages, free_count, kv_status, S, N, Hkv, D, page_size,
                                   max_pages_per_seq, num_pages};
        return launched(attn::launch_kv_append_tokens(a, (hipStream_t)stream), "attn_kv_append_tokens launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_kv_append_tokens: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_kv_append_tokens: unknown exception");
    }
}

attn_status attn_paged_prefill(const float* q, const float* k_pool, const float* v_pool, const int32_t* block_table,
                               const int32_t* context_lens, const int32_t* token_start, int64_t S, int64_t N,
                               int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages_per_seq,
                               int64_t num_pages, float scale, float* o, float* lse, void* stream) {
    try {
        if (S <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || max_pages_per_seq <= 0 ||
            num_pages <= 0)
            return fail(ATTN_INVALID_ARGUMENT, "attn_paged_prefill: S, N, Hq, Hkv, D, page_size, "
                                               "max_pages_per_seq and num_pages must all be positive");
        if (Hq % Hkv != 0)
            return fail(ATTN_INVALID_ARGUMENT, "Hq % Hkv != 0: query heads cannot be grouped over the key/value heads");
        if (!std::isfinite(scale)) return fail(ATTN_INVALID_ARGUMENT, "scale is not finite");
        if (page_size * max_pages_per_seq >= kMaxElems || S * max_pages_per_seq >= kMaxElems ||
            N * Hq * D >= kMaxElems || (N / 64 + S + 8) * Hq >= kMaxElems ||
            num_pages * Hkv * page_size * D >= ((int64_t)1 << 40))
            return fail(ATTN_INVALID_ARGUMENT, "attn_paged_prefill: sizes too large");
        if (!attn::causal_head_dim_supported(D) || (page_size != 16 && page_size != 32 && page_size != 64))
            return fail(ATTN_UNSUPPORTED, "attn_paged_prefill: no kernel for D=" + std::to_string(D) +
                                              ", page_size=" + std::to_string(page_size) +
                                              " (supported: D in {8,16,32,64,128}, page_size in {16,32,64})");
        ATTN_TRY(check_ptr(q, "q", 16));
        ATTN_TRY(check_ptr(k_pool, "k_pool", 16));
        ATTN_TRY(check_ptr(v_pool, "v_pool", 16));
        ATTN_TRY(check_ptr(block_table, "block_table", 4));
        ATTN_TRY(check_ptr(context_lens, "context_lens", 4));
        ATTN_TRY(check_ptr(token_start, "token_start", 4));
        ATTN_TRY(check_ptr(o, "o", 16));
        if (lse) ATTN_TRY(check_ptr(lse, "lse", 4));
        const size_t qb = (size_t)(N * Hq * D) * 4, pb = (size_t)(num_pages * Hkv * page_size * D) * 4;
        const Range lr{lse, lse ? (size_t)(N * Hq) * 4 : 0, "lse"};
        ATTN_TRY(check_disjoint({{o, qb, "o"}, lr},
                                {{q, qb, "q"}, {k_pool, pb, "k_pool"}, {v_pool, pb, "v_pool"},
                                 {block_table, (size_t)(S * max_pages_per_seq) * 4, "block_table"},
                                 {context_lens, (size_t)S * 4, "context_lens"},
                                 {token_start, (size_t)(S + 1) * 4, "token_start"}}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        ATTN_TRY(debug_check_tables("attn_paged_prefill", context_lens, block_table, token_start, S, N,
                                    max_pages_per_seq, page_size, num_pages, 0, (hipStream_t)stream));
        attn::PrefillArgs a{q, k_pool, v_pool, block_table, context_lens, token_start, o, lse,
                            S, N, Hq, Hkv, D, page_size, max_pages_per_seq, num_pages, scale};
        return launched(attn::launch_paged_prefill(a, (hipStream_t)stream), "attn_paged_prefill launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_paged_prefill: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_paged_prefill: unknown exception");
    }
}

attn_status attn_kv_release(const int32_t* seq_ids, int64_t n, int64_t S, int64_t page_size,
                            int64_t max_pages_per_seq, int64_t num_pages, int32_t* block_table,
                            int32_t* context_lens, int32_t* free_pages, int32_t* free_count, int32_t* kv_status,
                            void* stream) {
    try {
        ATTN_TRY(check_kv_shape("attn_kv_release", S, page_size, max_pages_per_seq, num_pages));
        if (n < 0 || n > S)
            return fail(ATTN_INVALID_ARGUMENT, "attn_kv_release: n must lie in [0, S] (ids are distinct)");
        if (n > 0) ATTN_TRY(check_ptr(seq_ids, "seq_ids", 4));
        ATTN_TRY(check_ptr(block_table, "block_table", 4));
        ATTN_TRY(check_ptr(context_lens, "context_lens", 4));
        ATTN_TRY(check_ptr(free_pages, "free_pages", 4));
        ATTN_TRY(check_ptr(free_count, "free_count", 4));
        ATTN_TRY(check_ptr(kv_status, "kv_status", 4));
        const Range ids{seq_ids, n > 0 ? (size_t)n * 4 : 0, "seq_ids"};
        ATTN_TRY(check_disjoint({{context_lens, (size_t)S * 4, "context_lens"},
                                 {free_pages, (size_t)num_pages * 4, "free_pages"}, {free_count, 4, "free_count"},
                                 {kv_status, 4, "kv_status"}},
                                {ids, {block_table, (size_t)(S * max_pages_per_seq) * 4, "block_table"}}));
        int cus = 0;
        ATTN_TRY(device_ready(&cus));
        attn::KvReleaseArgs a{seq_ids, n, S, block_table, context_lens, free_pages, free_count, kv_status,
                              page_size, max_pages_per_seq, num_pages};
        return launched(attn::launch_kv_release(a, (hipStream_t)stream), "attn_kv_release launch");
    } catch (const std::exception& e) {
        return fail(ATTN_DEVICE_ERROR, std::string("attn_kv_release: ") + e.what());
    } catch (...) {
        return fail(ATTN_DEVICE_ERROR, "attn_kv_release: unknown exception");
    }
}

}  // extern "C"
