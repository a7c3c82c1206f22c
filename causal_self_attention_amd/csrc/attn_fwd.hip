// Causal flash-style forward on gfx950: O = softmax(scale Q K^T, t_k <= t_q) V
// and the per-row log-sum-exp, in memory linear in T.
//
// What is computed: "Architecture", "Tensor conventions" (row-major [B,H,T,D],
// key t_k excluded when t_k > t_q) and "Intentional limits" (an exact
// memory-linear path that keeps only per-row statistics); "Execution Backends
// and the Python ABI", "What the Metal slice does" (the Flash forward saves row
// maxima and exponential sums -- here folded into one log-sum-exp per row).
//
// Work decomposition (MI355X-first; the pages' tile-8 kernels are not reused):
//   * one work-group = 4 x KQ waves = 64 query rows of one (batch, query head);
//     wave w owns rows q0+16(w%4) .. +15 and key part w/4 (KQ = 2 halves, or 4
//     quarters at d = 128) of every 64-key tile, so the heaviest (longest-prefix)
//     blocks have a fraction of the serial work per wave; the parts keep separate
//     softmax statistics and are merged through LDS at the end;
//   * K/V tiles of 64 keys are staged through registers into two LDS buffers: while
//     a tile is multiplied the next one is stored into the other buffer and the one
//     after is loaded into registers, so one barrier per tile suffices (with one
//     buffer, two: 52.5 -> 50.9 us at B=4 H=8 T=1024 d=64, 86.0 -> 80.2 us at d=128);
//   * each wave computes S^T = K Q^T on fp32 MFMA (16x16x4) with its Q rows held
//     in registers, so a C tile has the query in the lane (i) and the keys in
//     (g, r): the online-softmax statistics of a query stay in its four lanes;
//   * P in that layout is exactly the A operand of O += P V (keys contracted in
//     the permuted order (g, r)); the output dims are permuted so each lane reads
//     its V values as one contiguous vector per key row;
//   * the running max moves only when a score exceeds it by more than 2^8, so the
//     output rescale (which needs a cross-lane shuffle in this layout) is rare;
//   * only tiles with keys <= the block's last query are visited, and in the
//     diagonal tile a wave skips the P V products of the 16-key sub-tiles wholly
//     above its rows (their scores are formed with the others and masked);
//   * blocks are ranked heaviest first (longest causal prefix) and dealt to the
//     CUs in snake order (see snake_rank), which balances the triangular work.
#include "attn_launch.h"
#include "device_common.h"

#include <float.h>

namespace attn {

template <int D, int KQ>
struct FwdTraits {
    static constexpr int BM = 64;                     // query rows per work-group
    static constexpr int BN = 64;                     // keys per K/V tile
    static constexpr int NT = 256 * KQ;               // threads per work-group: 4 row groups x KQ key parts
    static constexpr int SUBS = 4 / KQ;               // 16-key sub-tiles of every tile per wave
    static constexpr int W = D >= 16 ? 4 : 2;         // contiguous head-dim values per lane in a fragment
    static constexpr int KSTEPS = D / 4;              // MFMA k-steps over the head dim
    static constexpr int DP = D >= 16 ? D : 16;       // head dim padded to whole 16-column O tiles
    static constexpr int NDT = DP / 16;               // O tiles per wave
    static constexpr int LDK = D + 4;                 // LDS row stride of the K tile (floats)
    static constexpr int LDV = DP + 4;                // LDS row stride of the V tile (floats)
    static constexpr int TILE4 = BN * D / 4;          // float4 loads per K (or V) tile
    static constexpr int PER = (TILE4 + NT - 1) / NT; // float4 loads per thread per tile
    static constexpr int KS_FLOATS = BN * LDK;
    static constexpr int MERGE_REGS = 4 * NDT + 2;    // per lane: O accumulators, max, sum
    static constexpr int MERGE_FLOATS = (KQ - 1) * 4 * MERGE_REGS * 64;  // key parts 1.. hand over
    static constexpr int TILE_FLOATS = BN * LDK + BN * LDV;
    static constexpr int SMEM_FLOATS = 2 * TILE_FLOATS > MERGE_FLOATS ? 2 * TILE_FLOATS : MERGE_FLOATS;  // two K/V buffers
};

// Head-dim index of fragment slot s held by lane row g: groups of W contiguous
// values per lane so that fragments load as one vector.
template <int W>
__device__ __forceinline__ constexpr int frag_dim(int s, int g) {
    return 4 * W * (s / W) + W * g + (s % W);
}

constexpr float kFwdLazyRescale = 8.f;  // log2 headroom before the running max is moved
// key parts per tile (waves per row group).  Measured on one MI355X: at d = 128 four
// parts (16 waves, 4 per SIMD, 114 registers) beat two (whose ~150 registers left one
// 8-wave work-group per CU): 188.5 vs 228.2 us for B=2 H=8 T=2048; at d <= 64 two
// parts are faster (52.6 vs 55.7 us at B=4 H=8 T=1024, 1230 vs 1328 us at the
// 8192-token grouped-query forward), the shorter per-wave MFMA chains of four parts
// costing more than the occupancy gains.
template <int D>
constexpr int fwd_key_parts() { return D >= 128 ? 4 : 2; }

template <int N>
__device__ __forceinline__ void lds_vec(const float* p, float (&x)[N]) {
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

template <int D, int KQ>
__global__ __launch_bounds__(256 * KQ) void attn_fwd_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int T, int nqb, int nbh, int ncu,
    float c2 /* scale * log2(e) */) {
    using Tr = FwdTraits<D, KQ>;
    __shared__ __attribute__((aligned(16))) float smem[Tr::SMEM_FLOATS];
    float* Ks = smem;
    float* Vs = smem + Tr::KS_FLOATS;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_uniform(tid >> 6);
    const int rw = w & 3;   // row group: rows q0 + 16rw .. +15
    const int kh = w >> 2;  // key part: sub-tiles SUBS*kh .. SUBS*kh+SUBS-1 of every tile
    const int li = lane & 15;
    const int g = lane >> 4;

    // the query heads of a KV head on one XCD, then heavy and light blocks paired on a CU
    const int G = Hq / Hkv;
    const int item = xcd_grouped_item(blockIdx.x, G, nqb * nbh / G);
    if (item < 0) return;  // uniform: a padding work-group, before any barrier
    const int rank = snake_rank(item, nqb * nbh, ncu);
    const int qb = nqb - 1 - rank / nbh;  // rank 0 = the longest causal prefix
    const int bh = rank % nbh;
    const int b = bh / Hq;
    const int h = bh % Hq;
    const int hk = h / G;
    const float* Qh = Q + ((size_t)b * Hq + h) * (size_t)T * D;
    const float* Kh = K + ((size_t)b * Hkv + hk) * (size_t)T * D;
    const float* Vh = V + ((size_t)b * Hkv + hk) * (size_t)T * D;
    const int q0 = qb * Tr::BM;
    const int qrow = q0 + 16 * rw + li;  // this lane's query row (column of the S^T tiles)

    if constexpr (Tr::DP != D) {  // zero the padding columns of both V buffers once
        for (int idx = tid; idx < Tr::BN * (Tr::DP - D); idx += Tr::NT) {
            const int row = idx / (Tr::DP - D), col = D + idx % (Tr::DP - D);
            Vs[row * Tr::LDV + col] = 0.f;
            Vs[Tr::TILE_FLOATS + row * Tr::LDV + col] = 0.f;
        }
    }

    // Q fragments: slot s holds Q[qrow][frag_dim(s, g)]  (B operand of K Q^T)
    float qf[Tr::KSTEPS];
#pragma unroll
    for (int u = 0; u < Tr::KSTEPS / Tr::W; ++u) {
        const int d0 = 4 * Tr::W * u + Tr::W * g;
        if constexpr (Tr::W == 4) {
            f32x4 x = qrow < T ? *(const f32x4*)(Qh + (size_t)qrow * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) qf[4 * u + j] = x[j];
        } else {
            f32x2 x = qrow < T ? *(const f32x2*)(Qh + (size_t)qrow * D + d0) : f32x2{0.f, 0.f};
            qf[2 * u] = x[0];
            qf[2 * u + 1] = x[1];
        }
    }

    // O accumulators as [query 16rw + 4g + r][dim NDT*li + dt]
    f32x4 acc[Tr::NDT];
#pragma unroll
    for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Running max of query qrow over this key half (log2 units, same in its four
    // lanes).  It starts at the lowest finite value rather than -inf so that a
    // half that sees no key yet gives exp2(-inf - m) = 0, never NaN.
    float m_run = -FLT_MAX;
    float l_run = 0.f;  // this lane's share of the half's running sum for query qrow

    f32x4 kreg[Tr::PER], vreg[Tr::PER];
    auto gload = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < Tr::PER; ++i) {
            const int idx = tid + Tr::NT * i;
            if (Tr::TILE4 % Tr::NT == 0 || idx < Tr::TILE4) {
                const int row = idx / (D / 4), c4 = idx % (D / 4);
                const int key = kv0 + row;
                if (key < T) {
                    kreg[i] = *(const f32x4*)(Kh + (size_t)key * D + 4 * c4);
                    vreg[i] = *(const f32x4*)(Vh + (size_t)key * D + 4 * c4);
                } else {
                    kreg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                    vreg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    };
    auto lstore = [&](int buf) {
        float* Kd = smem + buf * Tr::TILE_FLOATS;
        float* Vd = Kd + Tr::KS_FLOATS;
#pragma unroll
        for (int i = 0; i < Tr::PER; ++i) {
            const int idx = tid + Tr::NT * i;
            if (Tr::TILE4 % Tr::NT == 0 || idx < Tr::TILE4) {
                const int row = idx / (D / 4), c4 = idx % (D / 4);
                *(f32x4*)&Kd[row * Tr::LDK + 4 * c4] = kreg[i];
                *(f32x4*)&Vd[row * Tr::LDV + 4 * c4] = vreg[i];
            }
        }
    };

    const int ntiles = qb + 1;  // BN == BM: tiles 0 .. qb, the last one diagonal
    gload(0);
    lstore(0);
    if (1 < ntiles) gload(Tr::BN);
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        // tile j is in buffer j & 1; buffer (j + 1) & 1 was last read in iteration j - 1,
        // which every wave finished before the barrier that ended it
        Ks = smem + (j & 1) * Tr::TILE_FLOATS;
        Vs = Ks + Tr::KS_FLOATS;

        const int kv0 = j * Tr::BN;
        const bool diag = (j == qb);
        const int nsub = diag ? rw + 1 : 4;  // 16-key sub-tiles with any key <= this wave's rows

        // S^T = K Q^T over this wave's key part: st[tt] holds
        // S^T[key = kv0 + 16(SUBS kh + tt) + 4g + r][query = qrow].  Every sub-tile is
        // formed, also one that the diagonal tile masks whole (its scores become -inf
        // below and its P V products are skipped), so that the SUBS accumulation chains
        // interleave with no branch between them (about 1 % faster at d = 64 and 128).
        f32x4 st[Tr::SUBS];
#pragma unroll
        for (int tt = 0; tt < Tr::SUBS; ++tt) st[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < Tr::KSTEPS / Tr::W; ++u) {
            float a[Tr::SUBS][Tr::W];
#pragma unroll
            for (int tt = 0; tt < Tr::SUBS; ++tt)
                lds_vec<Tr::W>(&Ks[(16 * (Tr::SUBS * kh + tt) + li) * Tr::LDK + 4 * Tr::W * u + Tr::W * g], a[tt]);
#pragma unroll
            for (int jj = 0; jj < Tr::W; ++jj)
#pragma unroll
                for (int tt = 0; tt < Tr::SUBS; ++tt) st[tt] = mfma16x16x4(a[tt][jj], qf[Tr::W * u + jj], st[tt]);
        }

        // mask and scale to log2 units; this lane's max over its 4 SUBS keys of the tile
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < Tr::SUBS; ++tt) {
            const int t = Tr::SUBS * kh + tt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kv0 + 16 * t + 4 * g + r;
                float x = st[tt][r] * c2;
                if (t >= nsub || (diag && key > qrow)) x = -INFINITY;
                st[tt][r] = x;
                mx = fmaxf(mx, x);
            }
        }
        // The running max moves only when a score exceeds it by more than 2^8 (and on
        // the first visible key); otherwise exponents stay <= 2^8 and no rescale is needed.
        if (__ballot(mx > m_run + kFwdLazyRescale)) {  // wave-uniform
            const float m_new = fmaxf(m_run, rows4_max(mx));
            const float alpha = exp2_hw(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * g + r);  // alpha of query 16rw + 4g + r
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt][r] *= ar;
            }
        }
#pragma unroll
        for (int tt = 0; tt < Tr::SUBS; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2_hw(st[tt][r] - m_run);
                st[tt][r] = p;
                l_run += p;
            }
        }

        // O += P V : P[query li][key 16t + 4g + r] is the A operand as it stands (k-step
        // (t, r)); B = V rows, lane li taking dims NDT*li .. NDT*li+NDT-1 as one vector
#pragma unroll
        for (int tt = 0; tt < Tr::SUBS; ++tt) {
            const int t = Tr::SUBS * kh + tt;
            if (t < nsub) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float bv[Tr::NDT];
                    lds_vec<Tr::NDT>(&Vs[(16 * t + 4 * g + r) * Tr::LDV + Tr::NDT * li], bv);
#pragma unroll
                    for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = mfma16x16x4(st[tt][r], bv[dt], acc[dt]);
                }
            }
        }
        if (j + 1 < ntiles) {
            lstore((j + 1) & 1);
            if (j + 2 < ntiles) gload((j + 2) * Tr::BN);
        }
        __syncthreads();
    }

    // Merge the key parts.  Parts 1 .. KQ-1 hand their accumulators, max and sum to the
    // part-0 wave of the same rows through LDS, in the lanes' own register layout.
    const float l_part = rows4_sum(l_run);  // query qrow's sum over this part, in lanes (*, li)
    __syncthreads();  // the last tile's readers are done with the K/V buffers
    if (kh > 0) {
        float* mbuf = smem + ((kh - 1) * 4 + rw) * Tr::MERGE_REGS * 64 + lane;
#pragma unroll
        for (int dt = 0; dt < Tr::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mbuf[(4 * dt + r) * 64] = acc[dt][r];
        mbuf[(4 * Tr::NDT) * 64] = m_run;
        mbuf[(4 * Tr::NDT + 1) * 64] = l_part;
    }
    __syncthreads();
    if (kh > 0) return;

    // M = max m_p, L = sum 2^(m_p - M) l_p, O = sum 2^(m_p - M) o_p / L, per query qrow
    float m_tot = m_run;
#pragma unroll
    for (int p = 1; p < KQ; ++p) m_tot = fmaxf(m_tot, smem[((p - 1) * 4 + rw) * Tr::MERGE_REGS * 64 + lane + (4 * Tr::NDT) * 64]);
    float f[KQ];  // weight of part p, then divided by L
    float l_tot = 0.f;
#pragma unroll
    for (int p = 0; p < KQ; ++p) {
        const float* mb = smem + ((p - 1) * 4 + rw) * Tr::MERGE_REGS * 64 + lane;
        const float mp = p == 0 ? m_run : mb[(4 * Tr::NDT) * 64];
        const float lp = p == 0 ? l_part : mb[(4 * Tr::NDT + 1) * 64];
        f[p] = exp2_hw(mp - m_tot);
        l_tot += f[p] * lp;
    }
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int p = 0; p < KQ; ++p) f[p] *= inv;
    if (g == 0 && qrow < T) LSE[((size_t)b * Hq + h) * (size_t)T + qrow] = (m_tot + log2_hw(l_tot)) * kLn2;
    float* Ob = O + ((size_t)b * Hq + h) * (size_t)T * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int q = q0 + 16 * rw + 4 * g + r;
        float out[Tr::NDT];
        const float f0 = __shfl(f[0], 4 * g + r);  // factors of query 16rw + 4g + r
#pragma unroll
        for (int dt = 0; dt < Tr::NDT; ++dt) out[dt] = acc[dt][r] * f0;
#pragma unroll
        for (int p = 1; p < KQ; ++p) {
            const float fp = __shfl(f[p], 4 * g + r);
            const float* mb = smem + ((p - 1) * 4 + rw) * Tr::MERGE_REGS * 64 + lane;
#pragma unroll
            for (int dt = 0; dt < Tr::NDT; ++dt) out[dt] += mb[(4 * dt + r) * 64] * fp;
        }
        if (q < T && (Tr::DP == D || li < D)) {
            float* dst = Ob + (size_t)q * D + Tr::NDT * li;
            if constexpr (Tr::NDT % 4 == 0) {
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; dt += 4)
                    *(f32x4*)(dst + dt) = f32x4{out[dt], out[dt + 1], out[dt + 2], out[dt + 3]};
            } else {
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt) dst[dt] = out[dt];
            }
        }
    }
}

template <int D>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
    constexpr int KQ = fwd_key_parts<D>();
    using Tr = FwdTraits<D, KQ>;
    const int nqb = (int)((a.T + Tr::BM - 1) / Tr::BM);
    const int nbh = (int)(a.B * a.Hq);
    const float c2 = a.scale * kLog2e;
    // snake order only pays when every work-group is resident at once (two per CU);
    // otherwise plain heaviest-first order (the dispatcher hands the next, lighter
    // work-group to whichever CU frees up first)
    const int n = nqb * nbh;
    const int ncu = KQ == 2 && n <= 2 * a.cu_count ? a.cu_count : n;
    const int64_t G = a.Hq / a.Hkv;
    hipLaunchKernelGGL((attn_fwd_kernel<D, KQ>), dim3((unsigned)xcd_grouped_grid(G, (int64_t)n / G)), dim3(Tr::NT), 0,
                       stream, a.q, a.k,
                       a.v, a.o, a.lse, (int)a.Hq, (int)a.Hkv, (int)a.T, nqb, nbh, ncu, c2);
    return hipGetLastError();
}

hipError_t launch_causal_fwd(const FwdArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 8: return launch_fwd_d<8>(a, stream);
        case 16: return launch_fwd_d<16>(a, stream);
        case 32: return launch_fwd_d<32>(a, stream);
        case 64: return launch_fwd_d<64>(a, stream);
        case 128: return launch_fwd_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
