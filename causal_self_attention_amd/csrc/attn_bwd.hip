// Causal attention backward on gfx950: the vector-Jacobian product (dQ, dK, dV)
// of the forward for the loss sum(dO * O), recomputing the probabilities from
// Q, K and the saved per-row log-sum-exp.
//
// What is computed: "Execution Backends and the Python ABI", "What the Metal
// slice does" (the Flash backward recomputes scores and probabilities from Q, K
// and the row statistics and never allocates a quadratic buffer); "Architecture",
// "Tensor conventions" (the mask).  Gradients of a key/value head that several
// query heads share are summed over those heads (learn/neural_network page,
// "Layer normalization": a broadcast input's gradient is reduced back to its own
// shape).  With P = exp(s - LSE), dP = dO V^T, Delta_i = <dO_i, O_i> and
// dS = P (dP - Delta):  dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Kernels, in stream order:
//   1. attn_bwd_pre: Delta_i = <dO_i, O_i> into the workspace, and dQ = 0;
//   2. attn_bwd_main: one work-group per 64-key block of one (batch, KV head);
//      wave w owns keys kv0+16w .. +15 and keeps their K, V fragments and dK, dV
//      accumulators in registers while it walks every query tile at or below
//      the diagonal, for each query head of the group.  Per query tile (64 rows,
//      Q and dO staged in LDS):
//        S  = Q K^T, dP = dO V^T           (C tiles: key in the lane i)
//        P, dS                             (elementwise, masked on the diagonal)
//        dV += P^T dO,  dK += dS^T Q       (P and dS are the A operands as-is; the
//                                           dO and Q rows load as vectors because
//                                           lane i owns dims NDT*i .. NDT*i+NDT-1)
//        dS -> LDS, then dQ(16 rows per wave) = dS K, added to dQ with float
//        atomics (the contraction runs over the whole 64-key block).
#include "attn_launch.h"
#include "device_common.h"

namespace attn {

// ---------------------------------------------------------------------------
// 1. Delta = rowsum(dO * O), dQ = 0
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const float* __restrict__ O,
                                                           const float* __restrict__ dO,
                                                           float* __restrict__ Delta,
                                                           float* __restrict__ dQ, int64_t rows) {
    constexpr int TPR = D / 4;  // threads per row, one float4 each
    constexpr int RPB = 256 / TPR;
    const int tid = threadIdx.x;
    const int part = tid % TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
    float x = 0.f;
    if (row < rows) {
        const f32x4 o = *(const f32x4*)(O + row * D + 4 * part);
        const f32x4 d = *(const f32x4*)(dO + row * D + 4 * part);
        x = o[0] * d[0] + o[1] * d[1] + o[2] * d[2] + o[3] * d[3];
        *(f32x4*)(dQ + row * D + 4 * part) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) x += __shfl_xor(x, m);
    if (row < rows && part == 0) Delta[row] = x;
}

// ---------------------------------------------------------------------------
// 2. main KV-parallel kernel
// ---------------------------------------------------------------------------
template <int D>
struct BwdTraits {
    static constexpr int BM = 64;                   // query rows per tile
    static constexpr int BN = 64;                   // keys per work-group (16 per wave)
    static constexpr int NT = 256;
    static constexpr int W = D >= 16 ? 4 : 2;       // contiguous head-dim values per fragment load
    static constexpr int KSTEPS = D / 4;
    static constexpr int DP = D >= 16 ? D : 16;     // head dim padded to whole 16-column tiles
    static constexpr int NDT = DP / 16;             // C tiles over the head dim
    static constexpr int LD = DP + 4;               // LDS row stride of Q, dO, K tiles
    static constexpr int LDS_ = BN + 4;             // LDS row stride of the dS tile
    static constexpr int TILE4 = BM * D / 4;
};

template <int W>
__device__ __forceinline__ constexpr int frag_dim_b(int s, int g) {
    return 4 * W * (s / W) + W * g + (s % W);
}

// NDT contiguous floats from LDS (one vector read when NDT is 2 or a multiple of 4)
template <int N>
__device__ __forceinline__ void lds_row(const float* p, float (&x)[N]) {
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
        x[0] = p[0];
    }
}

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_main_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dQ, float* __restrict__ dK, float* __restrict__ dV, int Hq, int Hkv, int T,
    int nkb, int nbkv, int ncu, float scale, float c2 /* scale * log2(e) */) {
    using Tr = BwdTraits<D>;
    __shared__ __attribute__((aligned(16))) float Qs[Tr::BM * Tr::LD];
    __shared__ __attribute__((aligned(16))) float dOs[Tr::BM * Tr::LD];
    __shared__ __attribute__((aligned(16))) float Ks[Tr::BN * Tr::LD];
    __shared__ __attribute__((aligned(16))) float dSs[Tr::BM * Tr::LDS_];
    __shared__ __attribute__((aligned(16))) float lse2s[Tr::BM];
    __shared__ __attribute__((aligned(16))) float dls[Tr::BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_uniform(tid >> 6);
    const int li = lane & 15;
    const int g = lane >> 4;

    const int rank = snake_rank(blockIdx.x, nkb * nbkv, ncu);
    const int kb = rank / nbkv;  // key block 0 has the most query tiles: rank 0
    const int bkv = rank % nbkv;
    const int b = bkv / Hkv;
    const int hk = bkv % Hkv;
    const int G = Hq / Hkv;
    const int nqb = (T + Tr::BM - 1) / Tr::BM;
    const int kv0 = kb * Tr::BN;
    const int keyw = kv0 + 16 * w + li;  // this lane's key (column of the S / dP tiles)

    const float* Kh = K + ((size_t)b * Hkv + hk) * (size_t)T * D;
    const float* Vh = V + ((size_t)b * Hkv + hk) * (size_t)T * D;

    if constexpr (Tr::DP != D) {  // padding columns of the Q, dO, K tiles stay zero
        for (int idx = tid; idx < Tr::BM * (Tr::DP - D); idx += Tr::NT) {
            const int row = idx / (Tr::DP - D), col = D + idx % (Tr::DP - D);
            Qs[row * Tr::LD + col] = 0.f;
            dOs[row * Tr::LD + col] = 0.f;
            Ks[row * Tr::LD + col] = 0.f;
        }
    }

    // K, V fragments of this lane's key: slot s holds [keyw][frag_dim_b(s, g)]
    float kf[Tr::KSTEPS], vf[Tr::KSTEPS];
#pragma unroll
    for (int u = 0; u < Tr::KSTEPS / Tr::W; ++u) {
        const int d0 = 4 * Tr::W * u + Tr::W * g;
        if constexpr (Tr::W == 4) {
            f32x4 x = keyw < T ? *(const f32x4*)(Kh + (size_t)keyw * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 y = keyw < T ? *(const f32x4*)(Vh + (size_t)keyw * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kf[4 * u + j] = x[j];
                vf[4 * u + j] = y[j];
            }
        } else {
            f32x2 x = keyw < T ? *(const f32x2*)(Kh + (size_t)keyw * D + d0) : f32x2{0.f, 0.f};
            f32x2 y = keyw < T ? *(const f32x2*)(Vh + (size_t)keyw * D + d0) : f32x2{0.f, 0.f};
            kf[2 * u] = x[0];
            kf[2 * u + 1] = x[1];
            vf[2 * u] = y[0];
            vf[2 * u + 1] = y[1];
        }
    }
    // the key block's K tile in LDS (B operand of dQ = dS K)
    for (int idx = tid; idx < Tr::TILE4; idx += Tr::NT) {
        const int row = idx / (D / 4), c4 = idx % (D / 4);
        const int key = kv0 + row;
        *(f32x4*)&Ks[row * Tr::LD + 4 * c4] =
            key < T ? *(const f32x4*)(Kh + (size_t)key * D + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // dK, dV accumulators as [key 4g + r][dim NDT*li + dt] (this wave's 16 keys)
    f32x4 dk[Tr::NDT], dv[Tr::NDT];
#pragma unroll
    for (int dt = 0; dt < Tr::NDT; ++dt) {
        dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // The (query head, query tile) pairs this block visits, in order; the next
    // pair's Q, dO rows and row statistics are loaded into registers during the
    // current pair's dQ phase and written to LDS at the top of the next step.
    const int nqt = nqb - kb;
    const int nsteps = G * nqt;
    constexpr int PER = (Tr::TILE4 + Tr::NT - 1) / Tr::NT;
    f32x4 xq[PER], xo[PER];
    float xl = INFINITY, xd = 0.f;
    auto prefetch = [&](int step) {
        const int h = hk * G + step / nqt;
        const int q0 = (kb + step % nqt) * Tr::BM;
        const size_t hoff = ((size_t)b * Hq + h) * (size_t)T;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + Tr::NT * i;
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const int q = q0 + row;
            xq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            xo[i] = xq[i];
            if ((Tr::TILE4 % Tr::NT == 0 || idx < Tr::TILE4) && q < T) {
                xq[i] = *(const f32x4*)(Q + (hoff + q) * D + 4 * c4);
                xo[i] = *(const f32x4*)(dO + (hoff + q) * D + 4 * c4);
            }
        }
        if (tid < Tr::BM) {
            const int q = q0 + tid;
            // a padding row gets LSE = +inf, so its probabilities are exactly 0
            xl = q < T ? LSE[hoff + q] * kLog2e : INFINITY;
            xd = q < T ? Delta[hoff + q] : 0.f;
        }
    };
    prefetch(0);

    for (int step = 0; step < nsteps; ++step) {
        const int h = hk * G + step / nqt;
        const int qb = kb + step % nqt;
        const size_t hoff = ((size_t)b * Hq + h) * (size_t)T;
        float* dQh = dQ + hoff * D;
        {
            const int q0 = qb * Tr::BM;
            __syncthreads();  // the previous tile's LDS readers are done
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int idx = tid + Tr::NT * i;
                if (Tr::TILE4 % Tr::NT == 0 || idx < Tr::TILE4) {
                    const int row = idx / (D / 4), c4 = idx % (D / 4);
                    *(f32x4*)&Qs[row * Tr::LD + 4 * c4] = xq[i];
                    *(f32x4*)&dOs[row * Tr::LD + 4 * c4] = xo[i];
                }
            }
            if (tid < Tr::BM) {
                lse2s[tid] = xl;
                dls[tid] = xd;
            }
            __syncthreads();

            // Every sub-tile is computed, also on the diagonal where some lie wholly above
            // this wave's keys: their probabilities are zeroed by the causal select below.
            // Skipping them would put branches around accumulating MFMAs, and the compiler
            // then copies the accumulators at every join, which costs more than it saves.
            const bool diag = (qb == kb);

            // S = Q K^T and dP = dO V^T : C[query 16qs + 4g + r][key li]
            f32x4 sa[4], pa[4];
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) {
                sa[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
                pa[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
                {
#pragma unroll
                    for (int u = 0; u < Tr::KSTEPS / Tr::W; ++u) {
                        const int off = (16 * qs + li) * Tr::LD + 4 * Tr::W * u + Tr::W * g;
                        if constexpr (Tr::W == 4) {
                            const f32x4 a = *(const f32x4*)&Qs[off];
                            const f32x4 c = *(const f32x4*)&dOs[off];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                sa[qs] = mfma16x16x4(a[j], kf[4 * u + j], sa[qs]);
                                pa[qs] = mfma16x16x4(c[j], vf[4 * u + j], pa[qs]);
                            }
                        } else {
                            const f32x2 a = *(const f32x2*)&Qs[off];
                            const f32x2 c = *(const f32x2*)&dOs[off];
#pragma unroll
                            for (int j = 0; j < 2; ++j) {
                                sa[qs] = mfma16x16x4(a[j], kf[2 * u + j], sa[qs]);
                                pa[qs] = mfma16x16x4(c[j], vf[2 * u + j], pa[qs]);
                            }
                        }
                    }
                }
            }

            // P = exp(s - LSE) (0 where masked), dS = scale * P * (dP - Delta).  Row
            // statistics come in as one vector per sub-tile; the mask is a select.
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) {
                const f32x4 l4 = *(const f32x4*)&lse2s[16 * qs + 4 * g];
                const f32x4 d4 = *(const f32x4*)&dls[16 * qs + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qr = 16 * qs + 4 * g + r;  // row within the tile
                    float p = exp2_hw(sa[qs][r] * c2 - l4[r]);
                    p = (diag && 16 * w + li > qr) ? 0.f : p;
                    const float ds = scale * p * (pa[qs][r] - d4[r]);
                    sa[qs][r] = p;
                    pa[qs][r] = ds;
                }
            }

            // dV += P^T dO and dK += dS^T Q with P, dS as the A operands straight from their
            // accumulators (k-step (qs, r) pairs lane row g with query 16qs + 4g + r) and the
            // dO / Q rows as B operands, lane li taking dims NDT*li .. NDT*li+NDT-1
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) {
                {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = (16 * qs + 4 * g + r) * Tr::LD + Tr::NDT * li;
                        float bo[Tr::NDT], bq[Tr::NDT];
                        lds_row<Tr::NDT>(&dOs[row], bo);
                        lds_row<Tr::NDT>(&Qs[row], bq);
#pragma unroll
                        for (int dt = 0; dt < Tr::NDT; ++dt) {
                            dv[dt] = mfma16x16x4(sa[qs][r], bo[dt], dv[dt]);
                            dk[dt] = mfma16x16x4(pa[qs][r], bq[dt], dk[dt]);
                        }
                    }
                }
            }

            if (step + 1 < nsteps) prefetch(step + 1);  // lands during the dQ phase

            // dS -> LDS as [query][key]
#pragma unroll
            for (int qs = 0; qs < 4; ++qs)
#pragma unroll
                for (int r = 0; r < 4; ++r) dSs[(16 * qs + 4 * g + r) * Tr::LDS_ + 16 * w + li] = pa[qs][r];
            __syncthreads();

            // dQ rows 16w .. 16w+15 of the tile: C[query 16w + 4g + r][dim 16dt + li]
            // k-step (u, j) pairs lane row g with key 16u + 4g + j
            f32x4 qa[Tr::NDT];
#pragma unroll
            for (int dt = 0; dt < Tr::NDT; ++dt) qa[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                {
                    const f32x4 a = *(const f32x4*)&dSs[(16 * w + li) * Tr::LDS_ + 16 * u + 4 * g];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float* kp = &Ks[(16 * u + 4 * g + j) * Tr::LD + li];
#pragma unroll
                        for (int dt = 0; dt < Tr::NDT; ++dt) qa[dt] = mfma16x16x4(a[j], kp[16 * dt], qa[dt]);
                    }
                }
            }
            if (q0 + Tr::BM <= T && Tr::DP == D) {  // full tile: no per-element checks
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        unsafeAtomicAdd(dQh + (size_t)(q0 + 16 * w + 4 * g + r) * D + 16 * dt + li, qa[dt][r]);
            } else {
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt) {
                    const int d = 16 * dt + li;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int q = q0 + 16 * w + 4 * g + r;
                        if (q < T && (Tr::DP == D || d < D)) unsafeAtomicAdd(dQh + (size_t)q * D + d, qa[dt][r]);
                    }
                }
            }
        }
    }

    // dK, dV: lane (g, li) holds keys kv0 + 16w + 4g + r, dims NDT*li .. NDT*li+NDT-1
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int key = kv0 + 16 * w + 4 * g + r;
        if (key < T && (Tr::DP == D || li < D)) {
            float* dKr = dK + ((size_t)b * Hkv + hk) * (size_t)T * D + (size_t)key * D + Tr::NDT * li;
            float* dVr = dV + ((size_t)b * Hkv + hk) * (size_t)T * D + (size_t)key * D + Tr::NDT * li;
            if constexpr (Tr::NDT % 4 == 0) {
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; dt += 4) {
                    *(f32x4*)(dKr + dt) = f32x4{dk[dt][r], dk[dt + 1][r], dk[dt + 2][r], dk[dt + 3][r]};
                    *(f32x4*)(dVr + dt) = f32x4{dv[dt][r], dv[dt + 1][r], dv[dt + 2][r], dv[dt + 3][r]};
                }
            } else {
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt) {
                    dKr[dt] = dk[dt][r];
                    dVr[dt] = dv[dt][r];
                }
            }
        }
    }
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
    using Tr = BwdTraits<D>;
    const int64_t rows = a.B * a.Hq * a.T;
    constexpr int RPB = 256 / (D / 4);
    hipLaunchKernelGGL(attn_bwd_pre_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       stream, a.o, a.dout, a.delta, a.dq, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nkb = (int)((a.T + Tr::BN - 1) / Tr::BN);
    const int nbkv = (int)(a.B * a.Hkv);
    const int n = nkb * nbkv;
    const int ncu = n <= 2 * a.cu_count ? a.cu_count : n;  // snake only when all groups are resident
    hipLaunchKernelGGL(attn_bwd_main_kernel<D>, dim3((unsigned)(nkb * nbkv)), dim3(Tr::NT), 0, stream, a.q,
                       a.k, a.v, a.dout, a.lse, a.delta, a.dq, a.dk, a.dv, (int)a.Hq, (int)a.Hkv, (int)a.T, nkb,
                       nbkv, ncu, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

size_t bwd_workspace_floats(int64_t B, int64_t Hq, int64_t T) { return (size_t)(B * Hq * T); }

hipError_t launch_causal_bwd(const BwdArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 8: return launch_bwd_d<8>(a, stream);
        case 16: return launch_bwd_d<16>(a, stream);
        case 32: return launch_bwd_d<32>(a, stream);
        case 64: return launch_bwd_d<64>(a, stream);
        case 128: return launch_bwd_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
