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
// at streaming every byte once with plenty of loads in flight while keeping the
// per-position instruction count low:
//   1. attn_decode_split: one wave per (sequence, KV head, chunk of 256
//      positions), 16 positions per step.  Both small contractions (scores of the
//      G query heads that share the KV head, and the probability-weighted sum of
//      V) run on fp32 MFMA, which is otherwise idle here; this takes the
//      multiply-adds and their cross-lane reductions off the vector ALU, whose
//      issue rate would otherwise bound the kernel below the HBM rate.  Each K
//      and V row is read exactly once per KV head, as contiguous vectors.
//      Positions past the context get score -inf and a zero V (a select, so a
//      NaN in an unused slot cannot leak in).  Partial (m, l, o) go to the
//      workspace.
//   2. attn_decode_combine: per (sequence, query head), merges the chunks with
//      the log-sum-exp rule M = max m_c, L = sum 2^(m_c - M) l_c,
//      O = sum 2^(m_c - M) o_c / L.
#include "attn_launch.h"
#include "device_common.h"

namespace attn {

constexpr int kDecodeChunkTokens = 256;  // positions per wave
constexpr int kDecodeWaves = 4;          // waves (chunks) per work-group
constexpr int kDecodeGroup = 16;         // positions per MFMA step
constexpr float kLazyRescale = 8.f;      // log2 headroom before the running max is moved

template <int D>
struct DecTraits {
    static constexpr int KW = D >= 16 ? 4 : 2;         // contiguous head-dim values per K fragment load
    static constexpr int KSTEPS = D / 4;               // MFMA k-steps of S = K Q^T
    static constexpr int NDT = D >= 16 ? D / 16 : 1;   // output tiles; lane i owns dims NDT*i .. NDT*i+NDT-1
    static constexpr int VW = D >= 16 ? NDT : 1;       // contiguous V values a lane loads per row
};

// K fragment slot s of lane row g: head-dim index, KW contiguous values per load
template <int KW>
__device__ __forceinline__ constexpr int dec_kdim(int s, int g) {
    return 4 * KW * (s / KW) + KW * g + (s % KW);
}

template <int N>
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float* x) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const f32x4 v = *(const f32x4*)(p + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[4 * i + j] = v[j];
        }
    } else if constexpr (N == 2) {
        const f32x2 v = *(const f32x2*)p;
        x[0] = v[0];
        x[1] = v[1];
    } else {
        x[0] = *p;
    }
}

// One wave = one (sequence, KV head, chunk of 256 positions), 16 positions per
// step.  With lane l = 16*g + i:
//   S  = K Q^T on 16x16x4 MFMA: A = K[pos i][d] (float4 row loads), B = Q^T with
//        query head i in column i (columns >= G are zero).  C leaves lane (g, i)
//        holding S[pos 4g + r][head i] for r = 0..3, so each head's statistics
//        live in the four lanes i, i+16, i+32, i+48.
//   O += P V on 16x16x4 MFMA: P in that C layout is already the A operand
//        (k-step r <-> position 4g + r), B = V[pos 4g + r][d], and output dims are
//        permuted so lane i owns d = NDT*i .. NDT*i+NDT-1: every V row loads as one
//        contiguous vector per lane.  C holds O[head 4g + r][d].
// The VALU only scales, masks and exponentiates; the running max is moved (and
// O, l rescaled) only when a score exceeds it by more than 2^8.
template <int D>
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
    const int li = lane & 15;
    const int g = lane >> 4;
    const int G = Hq / Hkv;
    const int chunk = blockIdx.x * kDecodeWaves + w;
    // a length past the block table's capacity is clamped, so a broken length can
    // give wrong numbers but never an out-of-bounds read
    const int ctx = min(CTX[s], PS * max_pages);
    const int pos_begin = chunk * kDecodeChunkTokens;
    if (pos_begin >= ctx) return;  // wave-uniform: this chunk is past the sequence
    const int pos_end = min(pos_begin + kDecodeChunkTokens, ctx);

    // B operand of S: Q^T[d][head li]
    float qf[Tr::KSTEPS];
    {
        const float* qrow = Qd + ((size_t)s * Hq + (size_t)kvh * G + li) * D;
#pragma unroll
        for (int u = 0; u < Tr::KSTEPS / Tr::KW; ++u) {
            float x[Tr::KW];
            if (li < G) load_vec<Tr::KW>(qrow + 4 * Tr::KW * u + Tr::KW * g, x);
            else {
#pragma unroll
                for (int j = 0; j < Tr::KW; ++j) x[j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < Tr::KW; ++j) qf[Tr::KW * u + j] = x[j];
        }
    }

    float m = -INFINITY;  // running max of head li (log2 units), same in its four lanes
    float l = 0.f;        // this lane's share of head li's running sum
    f32x4 acc[Tr::NDT];   // O[head 4g + r][d = NDT*li + dt]
#pragma unroll
    for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The chunk's page ids are fetched once, one per lane, before any K/V load, so
    // no step waits on a block-table read before it can issue its loads.
    const int page0 = pos_begin / PS;
    const int npg = (pos_end - 1) / PS - page0 + 1;  // <= kDecodeChunkTokens / 16 <= 64
    int bt_lane = 0;
    if (lane < npg) bt_lane = min(max(BT[(size_t)s * max_pages + page0 + lane], 0), num_pages - 1);  // bad ids clamped
    auto page_row = [&](int p0) -> size_t {  // first row of the 16-position group at p0
        const int phys = __builtin_amdgcn_readlane(bt_lane, p0 / PS - page0);
        return ((size_t)phys * Hkv + kvh) * PS + (size_t)(p0 % PS);
    };

    // Loads run DEPTH groups ahead through a register ring, issued unconditionally
    // (a group past the end re-reads the last valid one and is masked), so each
    // wait covers only the group about to be used.
    constexpr int NG = kDecodeChunkTokens / kDecodeGroup;
    constexpr int DEPTH = 2;
    const int last_p0 = pos_begin + kDecodeGroup * ((pos_end - 1 - pos_begin) / kDecodeGroup);
    float kr[DEPTH][Tr::KSTEPS];
    float vr[DEPTH][4][Tr::VW];
    auto issue = [&](int k) {
        const size_t r0 = page_row(min(pos_begin + kDecodeGroup * k, last_p0));
        const float* kp = Kp + (r0 + li) * D;
#pragma unroll
        for (int u = 0; u < Tr::KSTEPS / Tr::KW; ++u) load_vec<Tr::KW>(kp + 4 * Tr::KW * u + Tr::KW * g, &kr[k % DEPTH][Tr::KW * u]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float* vp = Vp + (r0 + 4 * g + r) * D;
            if (D >= 16 || li < D) load_vec<Tr::VW>(vp + Tr::VW * li, vr[k % DEPTH][r]);
            else vr[k % DEPTH][r][0] = 0.f;
        }
    };
#pragma unroll
    for (int k = 0; k < DEPTH - 1; ++k) issue(k);

#pragma unroll
    for (int k = 0; k < NG; ++k) {
        if (k + DEPTH - 1 < NG) issue(k + DEPTH - 1);
        const int p0 = pos_begin + kDecodeGroup * k;
        if (p0 >= pos_end) break;  // wave-uniform
        const float* kf = kr[k % DEPTH];
        float(*vf)[Tr::VW] = vr[k % DEPTH];

        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sidx = 0; sidx < Tr::KSTEPS; ++sidx) st = mfma16x16x4(kf[sidx], qf[sidx], st);

        // Scores are read straight-line after the MFMA chain, with the tail masking
        // done by selects: no branch may separate the last MFMA from the first read
        // of its result (a taken branch there left the read without its wait states).
        float x[4];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok = p0 + 4 * g + r < pos_end;
            x[r] = ok ? st[r] * c2 : -INFINITY;
            mt = fmaxf(mt, x[r]);
#pragma unroll
            for (int j = 0; j < Tr::VW; ++j) vf[r][j] = ok ? vf[r][j] : 0.f;  // a NaN past the end stays out
        }
        if (__ballot(mt > m + kLazyRescale)) {  // wave-uniform and rare: move the max
            const float m_new = fmaxf(m, rows4_max(mt));
            const float alpha = exp2_hw(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * g + r);  // alpha of head 4g + r
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt][r] *= ar;
            }
        }
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = exp2_hw(x[r] - m);
            l += p[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int dt = 0; dt < Tr::NDT; ++dt) {
                acc[dt] = mfma16x16x4(p[r], vf[r][dt], acc[dt]);
            }
    }

    // partials: head h = 4g + r lives in lanes (g, *), register r; head li's l in lanes (*, li)
    const float lt = rows4_sum(l);
    const size_t pbase = ((size_t)s * Hkv + kvh) * max_chunks + chunk;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * g + r;
        if (h < G) {
            float* dst = Po + (pbase * G + h) * D + Tr::NDT * li;
            if constexpr (Tr::NDT % 4 == 0) {
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; dt += 4)
                    *(f32x4*)(dst + dt) = f32x4{acc[dt][r], acc[dt + 1][r], acc[dt + 2][r], acc[dt + 3][r]};
            } else {
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt)
                    if (D >= 16 || li < D) dst[dt] = acc[dt][r];
            }
        }
    }
    if (g == 0 && li < G) {
        Pm[pbase * G + li] = m;
        Pl[pbase * G + li] = lt;
    }
}

// One wave per (sequence, query head): chunk statistics are reduced across the
// lanes, the chunk weights 2^(m_c - M) / L go through LDS, and the lanes then
// sweep the head dim, several chunks per step so the loads overlap.
constexpr int kCombineMaxChunks = 64;  // chunks handled per LDS pass
constexpr int kCombineBatch = 8;       // chunks whose loads are issued together

__global__ __launch_bounds__(64) void attn_decode_combine_kernel(
    const float* __restrict__ Po, const float* __restrict__ Pm, const float* __restrict__ Pl,
    const int32_t* __restrict__ CTX, float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int D,
    int max_chunks) {
    __shared__ float wts[kCombineMaxChunks];
    const int lane = threadIdx.x;
    const int s = blockIdx.x / Hq;
    const int h = blockIdx.x % Hq;
    const int G = Hq / Hkv;
    const int kvh = h / G;
    const int hh = h % G;
    const int nch = (min(CTX[s], max_chunks * kDecodeChunkTokens) + kDecodeChunkTokens - 1) / kDecodeChunkTokens;
    const size_t base = ((size_t)s * Hkv + kvh) * max_chunks;
    float pm0 = -INFINITY, pl0 = 0.f;
    if (lane < nch) {
        pm0 = Pm[(base + lane) * G + hh];
        pl0 = Pl[(base + lane) * G + hh];
    }
    float mloc = pm0;
    for (int ci = lane + 64; ci < nch; ci += 64) mloc = fmaxf(mloc, Pm[(base + ci) * G + hh]);
    const float M = wave_max(mloc);
    float lloc = lane < nch ? exp2_hw(pm0 - M) * pl0 : 0.f;
    for (int ci = lane + 64; ci < nch; ci += 64) lloc += exp2_hw(Pm[(base + ci) * G + hh] - M) * Pl[(base + ci) * G + hh];
    const float L = wave_sum(lloc);
    const float inv = 1.f / L;
    const bool d0 = lane < D, d1 = lane + 64 < D;
    float acc0 = 0.f, acc1 = 0.f;  // head-dim values lane and lane + 64
    for (int c0 = 0; c0 < nch; c0 += kCombineMaxChunks) {
        const int cn = min(kCombineMaxChunks, nch - c0);
        __syncthreads();
        if (lane < cn) wts[lane] = exp2_hw((c0 == 0 ? pm0 : Pm[(base + c0 + lane) * G + hh]) - M) * inv;
        __syncthreads();
        for (int cb = 0; cb < cn; cb += kCombineBatch) {
            float x0[kCombineBatch], x1[kCombineBatch];
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j) {
                const bool ok = cb + j < cn;
                const float* src = Po + ((base + c0 + cb + j) * G + hh) * D;
                x0[j] = ok && d0 ? src[lane] : 0.f;
                x1[j] = ok && d1 ? src[lane + 64] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j) {
                const float wv = cb + j < cn ? wts[cb + j] : 0.f;
                acc0 += wv * x0[j];
                acc1 += wv * x1[j];
            }
        }
    }
    float* dst = O + ((size_t)s * Hq + h) * D;
    if (d0) dst[lane] = acc0;
    if (d1) dst[lane + 64] = acc1;
    if (LSE && lane == 0) LSE[(size_t)s * Hq + h] = (M + log2_hw(L)) * kLn2;
}

static int64_t decode_max_chunks(int64_t page_size, int64_t max_pages) {
    return (page_size * max_pages + kDecodeChunkTokens - 1) / kDecodeChunkTokens;
}

bool decode_shape_supported(int64_t D, int64_t page_size, int64_t group) {
    const bool d_ok = D == 8 || D == 16 || D == 32 || D == 64 || D == 128;
    const bool p_ok = page_size == 16 || page_size == 32 || page_size == 64;
    return d_ok && p_ok && group >= 1 && group <= 16;
}

size_t decode_workspace_floats(int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t max_pages) {
    (void)Hkv;
    const int64_t nch = decode_max_chunks(page_size, max_pages);
    return (size_t)(S * Hq * nch * (D + 2));
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    const int64_t nch = decode_max_chunks(a.page_size, a.max_pages);
    float* Po = a.partial;
    float* Pm = Po + (size_t)(a.S * a.Hq * nch * D);
    float* Pl = Pm + (size_t)(a.S * a.Hq * nch);
    const dim3 grid((unsigned)((nch + kDecodeWaves - 1) / kDecodeWaves), (unsigned)a.Hkv, (unsigned)a.S);
    hipLaunchKernelGGL((attn_decode_split_kernel<D>), grid, dim3(64 * kDecodeWaves), 0, stream, a.q, a.k_pool,
                       a.v_pool, a.block_table, a.context_lens, Po, Pm, Pl, (int)a.Hq, (int)a.Hkv,
                       (int)a.page_size, (int)a.max_pages, (int)a.num_pages, (int)nch, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_decode_combine_kernel, dim3((unsigned)(a.S * a.Hq)), dim3(64), 0, stream,
                       Po, Pm, Pl, a.context_lens, a.o, a.lse, (int)a.Hq, (int)a.Hkv, D, (int)nch);
    return hipGetLastError();
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
