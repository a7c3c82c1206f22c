// Materialized causal attention on gfx950: the probability tensor
// P [B,Hq,T,T] as an output, and the VJP that uses the stored P.
//
// What is computed: "Architecture", "Intentional limits" and "Execution
// Backends and the Python ABI", "What the Metal slice does" -- the materialized
// path returns the probabilities together with the context and keeps the
// [B,H,T,T] probabilities for the VJPs; the probability-returning diagnostic
// always takes this path.  "Architecture", "Tensor conventions": scores are
// [B,H,Tq,Tk] and key t_k is excluded from query t_q when t_k > t_q (its
// probability is 0).
//
// Forward = the flash forward (O and the row log-sum-exp, attn_fwd.hip) followed
// by attn_mat_probs, which recomputes each 64 x 64 score tile on MFMA and writes
// P = exp(s - LSE), one work-group per 64-row strip, zeros above the diagonal:
// every element of P is written, the cost is the T x T store.
// Backward = the flash backward's kernels in their materialized variant
// (attn_bwd.hip: P read from memory instead of recomputed, an optional cotangent
// of P added to dP), after attn_mat_delta adds sum_j P_ij dPx_ij to Delta_i.
#include "attn_launch.h"
#include "device_common.h"

namespace attn {

// One work-group per query block qb, (batch, query head) and part: the part takes
// the key tiles part, part + nparts, part + 2 nparts, ... (at most eight) of that row
// strip, so the parts of a strip have the same number of tiles at or below the
// diagonal to within one -- a contiguous split gave the work-groups holding the
// first tiles of a strip several times the multiplies of those holding the last,
// and because a CU's resident work-groups all had the same part that imbalance set
// the kernel's length.  Wave w holds the Q fragments of rows q0+16w..+15; the part's
// key tiles up to qb are staged in LDS one after the other (the next tile's loads in
// flight in registers while the current one is multiplied), each forming
// P^T = exp2(K Q^T * c2 - LSE2) on MFMA (the query in the lane i, keys in (g, r), as
// in the forward; the four 16-key sub-tiles as independent accumulation chains),
// every lane storing its four consecutive keys; key tiles past qb are stored as zeros.
// Work-groups are small (about 70 registers a lane, 17 KB of LDS), so many waves per
// CU overlap the MFMA chains with the stores; strips are dealt heaviest first.
constexpr int kMatTilesPerPart = 8;  // 64-key tiles per work-group of attn_mat_probs (measured: 1, 2, 4, 8)

template <int D>
__global__ __launch_bounds__(256) void attn_mat_probs_kernel(const float* __restrict__ Q,
                                                             const float* __restrict__ K,
                                                             const float* __restrict__ LSE, float* __restrict__ P,
                                                             int Hq, int Hkv, int T, int nqb, int nbh, int nparts,
                                                             float c2) {
    constexpr int W = D >= 16 ? 4 : 2;
    constexpr int KSTEPS = D / 4;
    constexpr int LDK = D + 4;
    constexpr int TILE4 = 64 * D / 4;                // float4s of a K tile
    constexpr int PER = (TILE4 + 255) / 256;         // of them per thread
    __shared__ __attribute__((aligned(16))) float Ks[64 * LDK];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_uniform(tid >> 6);
    const int li = lane & 15;
    const int g = lane >> 4;
    const int bh = blockIdx.x % nbh;
    const int r = blockIdx.x / nbh;
    const int qb = nqb - 1 - r / nparts;  // the longest causal prefixes first
    const int part = r % nparts;
    // tiles kt_at(i) for i < ntile; the first nmul of them have keys <= some query of the block
    auto kt_at = [&](int i) { return part + nparts * i; };
    const int ntile = (nqb - part + nparts - 1) / nparts;
    const int nmul = min(ntile, (qb - part + nparts) / nparts);  // #{i : part + nparts * i <= qb}
    const int b = bh / Hq, h = bh % Hq;
    const int hk = h / (Hq / Hkv);
    float* Ph = P + (size_t)bh * T * T;
    const int q0 = qb * 64;
    const bool vec = (T % 4) == 0;
    const float* Kh = K + ((size_t)b * Hkv + hk) * (size_t)T * D;

    auto kload = [&](int kt, f32x4 (&x)[PER]) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + 256 * i;
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const int key = kt * 64 + row;
            x[i] = (TILE4 % 256 == 0 || idx < TILE4) && key < T ? *(const f32x4*)(Kh + (size_t)key * D + 4 * c4)
                                                                 : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    f32x4 kx[PER];
    if (nmul > 0) kload(kt_at(0), kx);

    const int qrow = q0 + 16 * w + li;
    const float* Qr = Q + ((size_t)bh * T + (qrow < T ? qrow : 0)) * D;
    float qf[KSTEPS];
#pragma unroll
    for (int u = 0; u < KSTEPS / W; ++u) {
        const int d0 = 4 * W * u + W * g;
        if constexpr (W == 4) {
            const f32x4 x = qrow < T ? *(const f32x4*)(Qr + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) qf[4 * u + j] = x[j];
        } else {
            const f32x2 x = qrow < T ? *(const f32x2*)(Qr + d0) : f32x2{0.f, 0.f};
            qf[2 * u] = x[0];
            qf[2 * u + 1] = x[1];
        }
    }
    const float lse2 = qrow < T ? LSE[(size_t)bh * T + qrow] * kLog2e : 0.f;

    auto put = [&](int c0, const float (&pv)[4]) {  // keys c0 .. c0+3 of this lane's row
        if (qrow < T && c0 < T) {
            float* dst = Ph + (size_t)qrow * T + c0;
            if (vec) {
                *(f32x4*)dst = f32x4{pv[0], pv[1], pv[2], pv[3]};
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (c0 + r < T) dst[r] = pv[r];
            }
        }
    };

    for (int i = 0; i < nmul; ++i) {
        const int kt = kt_at(i);
        __syncthreads();  // the previous tile's readers are done
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + 256 * i;
            if (TILE4 % 256 == 0 || idx < TILE4) {
                const int row = idx / (D / 4), c4 = idx % (D / 4);
                *(f32x4*)&Ks[row * LDK + 4 * c4] = kx[i];
            }
        }
        __syncthreads();
        if (i + 1 < nmul) kload(kt_at(i + 1), kx);  // lands while this tile is multiplied
        const int kv0 = kt * 64;
        f32x4 st[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KSTEPS / W; ++u) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float* kp = &Ks[(16 * t + li) * LDK + 4 * W * u + W * g];
                if constexpr (W == 4) {
                    const f32x4 a = *(const f32x4*)kp;
#pragma unroll
                    for (int j = 0; j < 4; ++j) st[t] = mfma16x16x4(a[j], qf[4 * u + j], st[t]);
                } else {
                    const f32x2 a = *(const f32x2*)kp;
                    st[t] = mfma16x16x4(a[0], qf[2 * u], st[t]);
                    st[t] = mfma16x16x4(a[1], qf[2 * u + 1], st[t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // lane (g, li): P[qrow][kv0 + 16t + 4g + r], r = 0..3
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kv0 + 16 * t + 4 * g + r;
                const float p = exp2_hw(st[t][r] * c2 - lse2);
                pv[r] = (key <= qrow && key < T) ? p : 0.f;
            }
            put(kv0 + 16 * t + 4 * g, pv);
        }
    }
    const float zero[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = nmul; i < ntile; ++i) {  // every key of these tiles is after every query of the block
#pragma unroll
        for (int t = 0; t < 4; ++t) put(kt_at(i) * 64 + 16 * t + 4 * g, zero);
    }
}

// Delta_i += sum_{j <= i} P_ij dPx_ij: one wave per row.
__global__ __launch_bounds__(256) void attn_mat_delta_kernel(const float* __restrict__ P,
                                                             const float* __restrict__ dPx,
                                                             float* __restrict__ Delta, int64_t rows, int T) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // uniform per wave
    const int i = (int)(row % T);
    const float* pr = P + row * (int64_t)T;
    const float* dr = dPx + row * (int64_t)T;
    float x = 0.f;
    for (int j = lane; j <= i; j += 64) x += pr[j] * dr[j];
    x = wave_sum(x);
    if (lane == 0) Delta[row] += x;
}

template <int D>
static hipError_t launch_mat_probs_d(const MatFwdArgs& a, hipStream_t stream) {
    const int nqb = (int)((a.T + 63) / 64);
    const int nbh = (int)(a.B * a.Hq);
    const int nparts = (nqb + kMatTilesPerPart - 1) / kMatTilesPerPart;
    hipLaunchKernelGGL(attn_mat_probs_kernel<D>, dim3((unsigned)((int64_t)nparts * nqb * nbh)), dim3(256), 0, stream,
                       a.q, a.k, a.lse, a.p, (int)a.Hq, (int)a.Hkv, (int)a.T, nqb, nbh, nparts, a.scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_materialized_fwd(const MatFwdArgs& a, hipStream_t stream) {
    FwdArgs f{a.q, a.k, a.v, a.o, a.lse, a.B, a.Hq, a.Hkv, a.T, a.D, a.scale, a.cu_count};
    hipError_t e = launch_causal_fwd(f, stream);
    if (e != hipSuccess) return e;
    switch (a.D) {
        case 8: return launch_mat_probs_d<8>(a, stream);
        case 16: return launch_mat_probs_d<16>(a, stream);
        case 32: return launch_mat_probs_d<32>(a, stream);
        case 64: return launch_mat_probs_d<64>(a, stream);
        case 128: return launch_mat_probs_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mat_delta(const float* p, const float* dpx, float* delta, int64_t rows, int64_t T,
                            hipStream_t stream) {
    hipLaunchKernelGGL(attn_mat_delta_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p, dpx, delta,
                       rows, (int)T);
    return hipGetLastError();
}

}  // namespace attn
