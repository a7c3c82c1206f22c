// Batched single-token paged decode on gfx950.
//
// What is computed: "Execution Backends and the Python ABI", "Incremental
// attention" -- the query of the newest token, viewed as [H, d_h], attends to
// every cached position of its sequence; K/V live in pools laid out
// [physical_page, H, page_offset, d_h] and each logical page is resolved
// through the sequence's page table; nothing is gathered into a contiguous
// copy.  Grouped-query heads share a K/V head (ARCHITECTURE.md of
// algo-v1-codepoint, "config.py").
//
// The operation is bound by the HBM read of the K/V pages, so the design aims
// at streaming every byte once with plenty of loads in flight:
//   1. attn_decode_split: one wave per (sequence, KV head, chunk of 128
//      positions).  Lane l owns position 16*sub + l/4 of a 16-position slice and
//      a quarter of the head dim, so each row of K and V is read exactly once
//      and shared by all G query heads of the KV head.  Scores are reduced over
//      the 4 lanes of a row, the running max over the 16 rows of the slice; the
//      softmax sum and the output stay lane-local until the end of the chunk.
//      Positions past the context get score -inf and a zero V (a select, so a
//      NaN in an unused slot cannot leak in).  Partial (m, l, o) go to the
//      workspace.
//   2. attn_decode_combine: per (sequence, query head), merges the chunks with
//      the log-sum-exp rule M = max m_c, L = sum 2^(m_c - M) l_c,
//      O = sum 2^(m_c - M) o_c / L.
#include "attn_launch.h"
#include "device_common.h"

namespace attn {

constexpr int kDecodeChunkTokens = 128;  // positions per wave
constexpr int kDecodeWaves = 4;          // waves (chunks) per work-group

template <int D>
struct DecTraits {
    static constexpr int CW = D >= 16 ? 4 : 2;  // contiguous head-dim values per vector load
    static constexpr int NV = D / 4;            // head-dim values a lane holds per row
    static constexpr int NI = NV / CW;          // vector loads per row per lane
};

// head-dim index of value e (0 <= e < NV) held by lane quarter c
template <int D>
__device__ __forceinline__ constexpr int dec_dim(int e, int c) {
    using Tr = DecTraits<D>;
    return Tr::CW * c + 4 * Tr::CW * (e / Tr::CW) + (e % Tr::CW);
}

template <int D>
__device__ __forceinline__ void dec_load_row(const float* __restrict__ p, int c, float (&x)[DecTraits<D>::NV]) {
    using Tr = DecTraits<D>;
#pragma unroll
    for (int i = 0; i < Tr::NI; ++i) {
        const float* src = p + Tr::CW * c + 4 * Tr::CW * i;
        if constexpr (Tr::CW == 4) {
            const f32x4 v = *(const f32x4*)src;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[4 * i + j] = v[j];
        } else {
            const f32x2 v = *(const f32x2*)src;
            x[2 * i] = v[0];
            x[2 * i + 1] = v[1];
        }
    }
}

template <int D, int G>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(
    const float* __restrict__ Qd, const float* __restrict__ Kp, const float* __restrict__ Vp,
    const int32_t* __restrict__ BT, const int32_t* __restrict__ CTX, float* __restrict__ Po,
    float* __restrict__ Pm, float* __restrict__ Pl, int Hq, int Hkv, int PS, int max_pages, int num_pages,
    int max_chunks, float c2 /* scale * log2(e) */) {
    using Tr = DecTraits<D>;
    const int s = blockIdx.z;
    const int kvh = blockIdx.y;
    const int w = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int chunk = blockIdx.x * kDecodeWaves + w;
    // a length past the block table's capacity is clamped, so a broken length can
    // give wrong numbers but never an out-of-bounds read
    const int ctx = min(CTX[s], PS * max_pages);
    const int pos_begin = chunk * kDecodeChunkTokens;
    if (pos_begin >= ctx) return;  // wave-uniform: this chunk is past the sequence
    const int pos_end = min(pos_begin + kDecodeChunkTokens, ctx);
    const int tok = lane >> 2;  // row of the 16-position slice
    const int c = lane & 3;     // quarter of the head dim

    float qv[G][Tr::NV];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) dec_load_row<D>(Qd + ((size_t)s * Hq + (size_t)kvh * G + hh) * D, c, qv[hh]);

    float m[G], l[G], o[G][Tr::NV];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < Tr::NV; ++e) o[hh][e] = 0.f;
    }

    const int32_t* bt = BT + (size_t)s * max_pages;
    for (int p0 = pos_begin; p0 < pos_end; p0 += 16) {  // 16-position slices (page_size is a multiple of 16)
        const int pos = p0 + tok;
        const bool valid = pos < pos_end;
        const int phys = min(max(bt[p0 / PS], 0), num_pages - 1);  // same for a bad page id
        const size_t row = ((size_t)phys * Hkv + kvh) * PS + (size_t)(p0 % PS) + tok;
        float kv[Tr::NV], vv[Tr::NV];
        dec_load_row<D>(Kp + row * D, c, kv);
        dec_load_row<D>(Vp + row * D, c, vv);
#pragma unroll
        for (int e = 0; e < Tr::NV; ++e) vv[e] = valid ? vv[e] : 0.f;

#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < Tr::NV; ++e) acc += qv[hh][e] * kv[e];
            acc += __shfl_xor(acc, 1);
            acc += __shfl_xor(acc, 2);
            const float x = valid ? acc * c2 : -INFINITY;
            float mt = fmaxf(x, __shfl_xor(x, 4));
            mt = fmaxf(mt, __shfl_xor(mt, 8));
            mt = rows4_max(mt);
            const float m_new = fmaxf(m[hh], mt);  // finite: the slice's first position is valid
            const float alpha = exp2_hw(m[hh] - m_new);
            m[hh] = m_new;
            const float pr = exp2_hw(x - m_new);
            l[hh] = l[hh] * alpha + pr;
#pragma unroll
            for (int e = 0; e < Tr::NV; ++e) o[hh][e] = o[hh][e] * alpha + pr * vv[e];
        }
    }

    // sum l and o over the 16 rows (lanes with equal c), then write the partials
    const size_t pbase = ((size_t)s * Hkv + kvh) * max_chunks + chunk;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        float lt = l[hh];
        lt += __shfl_xor(lt, 4);
        lt += __shfl_xor(lt, 8);
        lt = rows4_sum(lt);
#pragma unroll
        for (int e = 0; e < Tr::NV; ++e) {
            float x = o[hh][e];
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            o[hh][e] = rows4_sum(x);
        }
        if (tok == 0) {
            float* dst = Po + (pbase * G + hh) * D;
#pragma unroll
            for (int e = 0; e < Tr::NV; ++e) dst[dec_dim<D>(e, c)] = o[hh][e];
            if (c == 0) {
                Pm[pbase * G + hh] = m[hh];
                Pl[pbase * G + hh] = lt;
            }
        }
    }
}

__global__ __launch_bounds__(128) void attn_decode_combine_kernel(
    const float* __restrict__ Po, const float* __restrict__ Pm, const float* __restrict__ Pl,
    const int32_t* __restrict__ CTX, float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int D,
    int max_chunks) {
    const int s = blockIdx.x / Hq;
    const int h = blockIdx.x % Hq;
    const int G = Hq / Hkv;
    const int kvh = h / G;
    const int hh = h % G;
    const int nch = (min(CTX[s], max_chunks * kDecodeChunkTokens) + kDecodeChunkTokens - 1) / kDecodeChunkTokens;
    const size_t base = ((size_t)s * Hkv + kvh) * max_chunks;
    float M = -INFINITY;
    for (int ci = 0; ci < nch; ++ci) M = fmaxf(M, Pm[(base + ci) * G + hh]);
    float L = 0.f;
    for (int ci = 0; ci < nch; ++ci) L += exp2_hw(Pm[(base + ci) * G + hh] - M) * Pl[(base + ci) * G + hh];
    const float inv = 1.f / L;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float acc = 0.f;
        for (int ci = 0; ci < nch; ++ci)
            acc += exp2_hw(Pm[(base + ci) * G + hh] - M) * Po[((base + ci) * G + hh) * D + d];
        O[((size_t)s * Hq + h) * D + d] = acc * inv;
    }
    if (LSE && threadIdx.x == 0) LSE[(size_t)s * Hq + h] = (M + log2_hw(L)) * kLn2;
}

static int64_t decode_max_chunks(int64_t page_size, int64_t max_pages) {
    return (page_size * max_pages + kDecodeChunkTokens - 1) / kDecodeChunkTokens;
}

bool decode_shape_supported(int64_t D, int64_t page_size, int64_t group) {
    const bool d_ok = D == 8 || D == 16 || D == 32 || D == 64 || D == 128;
    const bool p_ok = page_size == 16 || page_size == 32 || page_size == 64;
    const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
    return d_ok && p_ok && g_ok && group * D <= 512;
}

size_t decode_workspace_floats(int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t max_pages) {
    (void)Hkv;
    const int64_t nch = decode_max_chunks(page_size, max_pages);
    return (size_t)(S * Hq * nch * (D + 2));
}

template <int D, int G>
static hipError_t launch_decode_dg(const DecodeArgs& a, hipStream_t stream) {
    const int64_t nch = decode_max_chunks(a.page_size, a.max_pages);
    float* Po = a.partial;
    float* Pm = Po + (size_t)(a.S * a.Hq * nch * D);
    float* Pl = Pm + (size_t)(a.S * a.Hq * nch);
    const dim3 grid((unsigned)((nch + kDecodeWaves - 1) / kDecodeWaves), (unsigned)a.Hkv, (unsigned)a.S);
    hipLaunchKernelGGL((attn_decode_split_kernel<D, G>), grid, dim3(64 * kDecodeWaves), 0, stream, a.q, a.k_pool,
                       a.v_pool, a.block_table, a.context_lens, Po, Pm, Pl, (int)a.Hq, (int)a.Hkv,
                       (int)a.page_size, (int)a.max_pages, (int)a.num_pages, (int)nch, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_decode_combine_kernel, dim3((unsigned)(a.S * a.Hq)), dim3(D >= 64 ? 64 : D), 0, stream,
                       Po, Pm, Pl, a.context_lens, a.o, a.lse, (int)a.Hq, (int)a.Hkv, D, (int)nch);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_decode_dg<D, 1>(a, stream);
        case 2: return launch_decode_dg<D, 2>(a, stream);
        case 4: return launch_decode_dg<D, 4>(a, stream);
        case 8:
            if constexpr (8 * D <= 512) return launch_decode_dg<D, 8>(a, stream);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 8: return launch_decode_d<8>(a, stream);
        case 16: return launch_decode_d<16>(a, stream);
        case 32: return launch_decode_d<32>(a, stream);
        case 64: return launch_decode_d<64>(a, stream);
        case 128: return launch_decode_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
