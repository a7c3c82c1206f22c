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
//      positions), 16 positions per step; the waves of a work-group are
//      neighbouring KV heads of one chunk, so a page is read contiguously.  Both small contractions (scores of the
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
constexpr int kDecodeWaves = 4;          // waves (KV heads) per work-group
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

// One wave works through a list of 16-position groups of one (sequence, KV head):
// group j starts at position 16 * (g_first + g_stride * j), j < ng <= 64.  With
// lane l = 16*g + i:
//   S  = K Q^T on 16x16x4 MFMA: A = K[pos i][d] (float4 row loads), B = Q^T with
//        query head i in column i (columns >= G are zero).  C leaves lane (g, i)
//        holding S[pos 4g + r][head i] for r = 0..3, so each head's statistics
//        live in the four lanes i, i+16, i+32, i+48.
//   O += P V on 16x16x4 MFMA: P in that C layout is already the A operand
//        (k-step r <-> position 4g + r), B = V[pos 4g + r][d], and output dims are
//        permuted so lane i owns d = NDT*i .. NDT*i+NDT-1: every V row loads as one
//        contiguous vector per lane.  C holds O[head 4g + r][d].
// The VALU only scales, masks and exponentiates; the running max is moved (and
// O, l rescaled) only when a score exceeds it by more than 2^8.  (m, l, acc)
// carry over between calls, so a wave may take several lists in turn.
template <int D, int DEPTH, int NG_MAX>
__device__ __forceinline__ void decode_groups(const float* __restrict__ Kp, const float* __restrict__ Vp,
                                              const int32_t* __restrict__ bt_row, int Hkv, int kvh, int PS,
                                              int num_pages, int ctx, int g_first, int g_stride, int ng,
                                              const float (&qf)[DecTraits<D>::KSTEPS], float c2, float& m,
                                              float& l, f32x4 (&acc)[DecTraits<D>::NDT]) {
    using Tr = DecTraits<D>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    // The list's page ids are fetched once, one per lane, before any K/V load, so
    // no group waits on a block-table read before it can issue its loads.
    int bt_lane = 0;
    if (lane < ng) bt_lane = min(max(bt_row[(16 * (g_first + g_stride * lane)) / PS], 0), num_pages - 1);
    auto group_row = [&](int j) -> size_t {  // first pool row of group j
        const int p0 = 16 * (g_first + g_stride * j);
        const int phys = __builtin_amdgcn_readlane(bt_lane, j);
        return ((size_t)phys * Hkv + kvh) * PS + (size_t)(p0 % PS);
    };

    // Loads run DEPTH groups ahead through a register ring, issued unconditionally
    // (a group past the list re-reads the last one and is not used), so each wait
    // covers only the group about to be used.
    float kr[DEPTH][Tr::KSTEPS];
    float vr[DEPTH][4][Tr::VW];
    auto issue = [&](int j, int slot) {
        const size_t r0 = group_row(min(j, ng - 1));
        const float* kp = Kp + (r0 + li) * D;
#pragma unroll
        for (int u = 0; u < Tr::KSTEPS / Tr::KW; ++u) load_vec<Tr::KW>(kp + 4 * Tr::KW * u + Tr::KW * g, &kr[slot][Tr::KW * u]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float* vp = Vp + (r0 + 4 * g + r) * D;
            if (D >= 16 || li < D) load_vec<Tr::VW>(vp + Tr::VW * li, vr[slot][r]);
            else vr[slot][r][0] = 0.f;
        }
    };
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) issue(d, d);

    // One group: scores, online softmax, O += P V.  A group outside the list is
    // computed fully masked.
    auto group = [&](int j, int slot, bool in_list) {
        const int p0 = 16 * (g_first + g_stride * j);
        const float* kf = kr[slot];
        float(*vf)[Tr::VW] = vr[slot];
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sidx = 0; sidx < Tr::KSTEPS; ++sidx) st = mfma16x16x4(kf[sidx], qf[sidx], st);

        // Scores are read straight-line after the MFMA chain, with the tail masking
        // done by selects: no branch may separate the last MFMA from the first read
        // of its result (a taken branch there leaves the read without its wait states).
        float x[4];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok = in_list && p0 + 4 * g + r < ctx;
            x[r] = ok ? st[r] * c2 : -INFINITY;
            mt = fmaxf(mt, x[r]);
#pragma unroll
            for (int jj = 0; jj < Tr::VW; ++jj) vf[r][jj] = ok ? vf[r][jj] : 0.f;  // a NaN past the end stays out
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
            for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = mfma16x16x4(p[r], vf[r][dt], acc[dt]);
    };

    if constexpr (NG_MAX > 0) {
        // at most NG_MAX groups: the walk is unrolled completely
#pragma unroll
        for (int j = 0; j < NG_MAX; ++j) {
            if (j + DEPTH - 1 < NG_MAX) issue(j + DEPTH - 1, (j + DEPTH - 1) % DEPTH);
            if (j >= ng) break;  // wave-uniform
            group(j, j % DEPTH, true);
        }
    } else {
        // Whole rounds of DEPTH groups, the last one padded with masked groups: an
        // exit in the middle of a rolled round would put a branch between the last
        // MFMA of a group and the loop's copies of its accumulators.
        const int ng_round = (ng + DEPTH - 1) / DEPTH * DEPTH;
        for (int j0 = 0; j0 < ng_round; j0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                issue(j0 + d + DEPTH - 1, (d + DEPTH - 1) % DEPTH);
                group(j0 + d, d, j0 + d < ng);
            }
        }
    }
}

// B operand of S: Q^T[d][head li] for the G query heads of KV head kvh (zero columns past G)
template <int D>
__device__ __forceinline__ void decode_load_q(const float* __restrict__ Qd, int s, int Hq, int kvh, int G,
                                              float (&qf)[DecTraits<D>::KSTEPS]) {
    using Tr = DecTraits<D>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
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

// Split path, one wave per (sequence, KV head, chunk of 256 positions); the waves
// of a work-group are neighbouring KV heads of one chunk, so a page is read
// contiguously.  Partials (m, l, o) go to the workspace.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(
    const float* __restrict__ Qd, const float* __restrict__ Kp, const float* __restrict__ Vp,
    const int32_t* __restrict__ BT, const int32_t* __restrict__ CTX, float* __restrict__ Po,
    float* __restrict__ Pm, float* __restrict__ Pl, int Hq, int Hkv, int PS, int max_pages, int num_pages,
    int max_chunks, float c2 /* scale * log2(e) */) {
    using Tr = DecTraits<D>;
    const int s = blockIdx.z;
    const int w = wave_uniform(threadIdx.x >> 6);
    const int kvh = blockIdx.y * kDecodeWaves + w;
    if (kvh >= Hkv) return;  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    const int G = Hq / Hkv;
    const int chunk = blockIdx.x;
    // a length past the block table's capacity is clamped, so a broken length can
    // give wrong numbers but never an out-of-bounds read
    const int ctx = min(CTX[s], PS * max_pages);
    const int pos_begin = chunk * kDecodeChunkTokens;
    if (pos_begin >= ctx) return;  // wave-uniform: this chunk is past the sequence
    const int pos_end = min(pos_begin + kDecodeChunkTokens, ctx);

    float qf[Tr::KSTEPS];
    decode_load_q<D>(Qd, s, Hq, kvh, G, qf);
    float m = -INFINITY;  // running max of head li (log2 units), same in its four lanes
    float l = 0.f;        // this lane's share of head li's running sum
    f32x4 acc[Tr::NDT];   // O[head 4g + r][d = NDT*li + dt]
#pragma unroll
    for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    decode_groups<D, 2, kDecodeChunkTokens / 16>(Kp, Vp, BT + (size_t)s * max_pages, Hkv, kvh, PS, num_pages, ctx,
                                                 pos_begin / 16, 1,
                                                 (pos_end - pos_begin + 15) / 16, qf, c2, m, l, acc);

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

// Fused path, one work-group of NW waves per (sequence, KV head): wave w takes the
// 16-position groups w, w + NW, ... of the whole context (up to 64 at a time), so
// the waves of a long or a short sequence all have about the same number of groups.  The waves' (m, l, o) are merged through LDS with the same
// log-sum-exp rule as the combine kernel, and O, LSE are written directly: no
// workspace and no second kernel.
template <int D>
constexpr int fused_waves() { return D >= 128 ? 4 : 8; }  // d = 128 keeps a whole register file per wave

template <int D>
__global__ __launch_bounds__(64 * fused_waves<D>()) void attn_decode_fused_kernel(
    const float* __restrict__ Qd, const float* __restrict__ Kp, const float* __restrict__ Vp,
    const int32_t* __restrict__ BT, const int32_t* __restrict__ CTX, float* __restrict__ O,
    float* __restrict__ LSE, int Hq, int Hkv, int PS, int max_pages, int num_pages, float c2) {
    using Tr = DecTraits<D>;
    constexpr int NW = fused_waves<D>();
    constexpr int DP = 16 * Tr::NDT;  // padded head dim of the merge buffer
    __shared__ __attribute__((aligned(16))) float po[NW * kDecodeGroup * DP];
    __shared__ float pm[NW * kDecodeGroup], pl[NW * kDecodeGroup];
    const int kvh = blockIdx.x;
    const int s = blockIdx.y;
    const int w = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    const int G = Hq / Hkv;
    const int ctx = min(CTX[s], PS * max_pages);  // clamped as in the split path
    const int ngroups = (ctx + 15) / 16;

    float qf[Tr::KSTEPS];
    decode_load_q<D>(Qd, s, Hq, kvh, G, qf);
    float m = -INFINITY;
    float l = 0.f;
    f32x4 acc[Tr::NDT];
#pragma unroll
    for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int mine = w < ngroups ? (ngroups - w + NW - 1) / NW : 0;  // this wave's groups
    for (int j0 = 0; j0 < mine; j0 += 64)
        decode_groups<D, 2, 0>(Kp, Vp, BT + (size_t)s * max_pages, Hkv, kvh, PS, num_pages, ctx,
                            w + NW * j0, NW, min(64, mine - j0), qf, c2, m, l, acc);

    // this wave's partial: O[head 4g + r][d] in registers, head li's max and sum in lanes (*, li)
    const float lt = rows4_sum(l);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int dt = 0; dt < Tr::NDT; ++dt)
            po[(w * kDecodeGroup + 4 * g + r) * DP + Tr::NDT * li + dt] = acc[dt][r];
    if (g == 0) {
        pm[w * kDecodeGroup + li] = m;
        pl[w * kDecodeGroup + li] = lt;
    }
    __syncthreads();

    // merge: one output element (query head h of this KV head, dim d) per thread
    for (int t = threadIdx.x; t < G * D; t += 64 * NW) {
        const int h = t / D, d = t % D;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < NW; ++v) M = fmaxf(M, pm[v * kDecodeGroup + h]);  // finite: wave 0 has a group
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const float wv = exp2_hw(pm[v * kDecodeGroup + h] - M);  // 0 for a wave without groups
            L += wv * pl[v * kDecodeGroup + h];
            o += wv * po[(v * kDecodeGroup + h) * DP + d];
        }
        const size_t row = (size_t)s * Hq + (size_t)kvh * G + h;
        O[row * D + d] = o / L;
        if (LSE && d == 0) LSE[row] = (M + log2_hw(L)) * kLn2;
    }
}

// One wave per (sequence, query head) merges the chunks' partials, 64 chunks per
// pass with a running (M, L, o): lane c holds chunk c's statistics, the weight of
// chunk c reaches every lane by a lane read, and the lanes sweep the head dim
// (dims lane and lane + 64).  The loads of the first pass go out before the
// context length is known (the workspace holds max_chunks slots; slots past the
// sequence's chunk count are masked by selects), so the kernel waits on about one
// memory round trip instead of three.
constexpr int kCombineBatch = 16;  // chunks whose partial rows are loaded together

__global__ __launch_bounds__(64) void attn_decode_combine_kernel(
    const float* __restrict__ Po, const float* __restrict__ Pm, const float* __restrict__ Pl,
    const int32_t* __restrict__ CTX, float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int D,
    int max_chunks) {
    const int lane = threadIdx.x;
    const int s = blockIdx.x / Hq;
    const int h = blockIdx.x % Hq;
    const int G = Hq / Hkv;
    const int kvh = h / G;
    const int hh = h % G;
    const size_t base = ((size_t)s * Hkv + kvh) * max_chunks;
    const bool d0 = lane < D, d1 = lane + 64 < D;
    const int ctx = CTX[s];
    float M = -INFINITY, L = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int c0 = 0; c0 < max_chunks; c0 += 64) {
        const int c = c0 + lane;
        const bool have = c < max_chunks;
        const float pm_raw = have ? Pm[(base + c) * G + hh] : -INFINITY;
        const float pl_raw = have ? Pl[(base + c) * G + hh] : 0.f;
        const int cn = min(64, max_chunks - c0);
        float x0[kCombineBatch], x1[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {  // first batch of partial rows, issued early
            const float* src = Po + ((base + c0 + min(j, cn - 1)) * G + hh) * D;
            x0[j] = d0 ? src[lane] : 0.f;
            x1[j] = d1 ? src[lane + 64] : 0.f;
        }
        const int nch = (min(ctx, max_chunks * kDecodeChunkTokens) + kDecodeChunkTokens - 1) / kDecodeChunkTokens;
        if (c0 >= nch) break;  // wave-uniform
        const bool valid = c < nch;
        const float pm = valid ? pm_raw : -INFINITY;
        const float m_new = fmaxf(M, wave_max(pm));  // finite: chunk c0 is valid
        const float keep = exp2_hw(M - m_new);        // 0 on the first pass
        const float wl = valid ? exp2_hw(pm - m_new) : 0.f;
        L = L * keep + wave_sum(valid ? wl * pl_raw : 0.f);
        acc0 *= keep;
        acc1 *= keep;
        M = m_new;
        const int cv = min(64, nch - c0);  // valid chunks of this pass
        for (int cb = 0; cb < cv; cb += kCombineBatch) {
            if (cb > 0) {
#pragma unroll
                for (int j = 0; j < kCombineBatch; ++j) {
                    const float* src = Po + ((base + c0 + min(cb + j, cn - 1)) * G + hh) * D;
                    x0[j] = d0 ? src[lane] : 0.f;
                    x1[j] = d1 ? src[lane + 64] : 0.f;
                }
            }
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j) {
                const float wj = __builtin_amdgcn_readlane(__float_as_int(wl), min(cb + j, 63));
                const bool ok = cb + j < cv;
                acc0 += ok ? __int_as_float(wj) * x0[j] : 0.f;
                acc1 += ok ? __int_as_float(wj) * x1[j] : 0.f;
            }
        }
    }
    const float inv = 1.f / L;
    float* dst = O + ((size_t)s * Hq + h) * D;
    if (d0) dst[lane] = acc0 * inv;
    if (d1) dst[lane + 64] = acc1 * inv;
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
    if (a.S * a.Hkv >= a.cu_count) {
        // At least one (sequence, KV head) pair per CU: one fused kernel.
        hipLaunchKernelGGL((attn_decode_fused_kernel<D>), dim3((unsigned)a.Hkv, (unsigned)a.S),
                           dim3(64 * fused_waves<D>()), 0, stream, a.q, a.k_pool, a.v_pool, a.block_table,
                           a.context_lens, a.o, a.lse, (int)a.Hq, (int)a.Hkv, (int)a.page_size,
                           (int)a.max_pages, (int)a.num_pages, a.scale * kLog2e);
        return hipGetLastError();
    }
    // Few pairs: split every context into chunks over the whole chip, then combine.
    const int64_t nch = decode_max_chunks(a.page_size, a.max_pages);
    float* Po = a.partial;
    float* Pm = Po + (size_t)(a.S * a.Hq * nch * D);
    float* Pl = Pm + (size_t)(a.S * a.Hq * nch);
    const dim3 grid((unsigned)nch, (unsigned)((a.Hkv + kDecodeWaves - 1) / kDecodeWaves), (unsigned)a.S);
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
