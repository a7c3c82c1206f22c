// Batched prefill over a paged K/V cache on gfx950: the new tokens of a ragged
// batch of sequences attend causally to everything their sequence holds.
//
// What is computed: "Architecture", "Serving boundary" (a request's K/V lives in
// pages leased from shared per-layer pools, reached through its logical page
// table) and "Tensor conventions" (key t_k excluded from query t_q when
// t_k > t_q); "Execution Backends and the Python ABI", "Incremental attention"
// (pools [physical_page, H, page_offset, d_h], read in place through the table --
// the pages prefill one token at a time through the decode op; here all new
// tokens of all sequences go in one call).  Sequence s brings n_s new tokens, packed
// row after row in q [N, Hq, D] from row token_start[s]; after they were appended
// its cache holds context_lens[s] positions, so new token j sits at position
// context_lens[s] - n_s + j and sees positions 0 .. that one.
//
// Work decomposition: the same tile engine as the causal forward (attn_fwd.hip):
// one work-group = 8 waves = 64 new tokens of one (sequence, query head); wave w
// owns rows 16(w%4) .. +15 and the key half w/4 of every 64-position tile; S^T =
// K Q^T and O += P V on fp32 MFMA with the online softmax in registers; the key
// halves merge through LDS.  What differs:
//   * a tile's K/V rows are gathered through the block table: each thread loads the
//     page ids of its rows one tile ahead of the rows themselves, so no K/V load
//     waits on a table read;
//   * the query rows start at an arbitrary position, so the causal mask is applied
//     per element on every tile that reaches past a wave's first row, and the P V
//     products of 16-key sub-tiles wholly past a wave's last row are skipped;
//   * the grid enumerates (query block, head) over the ragged batch, heaviest block
//     (most key tiles) first over the whole batch: each work-group finds its block by
//     bisection on the number of blocks with at least t tiles (one wave, one lane
//     per sequence, DPP scans), so the longest blocks of every sequence start in the
//     first round (in sequence order, the last sequence's longest blocks started
//     last and set the kernel's end).
#include "attn_launch.h"
#include "device_common.h"

#include <float.h>

namespace attn {

template <int D>
struct PrefillTraits {
    static constexpr int BM = 64;                      // new tokens per work-group
    static constexpr int BN = 64;                      // positions per K/V tile
    static constexpr int NT = 512;                     // threads per work-group (8 waves)
    static constexpr int W = D >= 16 ? 4 : 2;          // contiguous head-dim values per lane in a fragment
    static constexpr int KSTEPS = D / 4;               // MFMA k-steps over the head dim
    static constexpr int DP = D >= 16 ? D : 16;        // head dim padded to whole 16-column O tiles
    static constexpr int NDT = DP / 16;                // O tiles per wave
    static constexpr int LDK = D + 4;                  // LDS row stride of the K tile (floats)
    static constexpr int LDV = DP + 4;                 // LDS row stride of the V tile (floats)
    static constexpr int TILE4 = BN * D / 4;           // float4 loads per K (or V) tile
    static constexpr int PER = (TILE4 + NT - 1) / NT;  // float4 loads per thread per tile
    static constexpr int KS_FLOATS = BN * LDK;
    static constexpr int TILE_FLOATS = BN * LDK + BN * LDV;
    static constexpr int SMEM_FLOATS = 2 * TILE_FLOATS;  // two K/V buffers
    static constexpr int MERGE_REGS = 4 * NDT + 2;     // per lane: O accumulators, max, sum
    static_assert(4 * MERGE_REGS * 64 <= SMEM_FLOATS, "merge buffer must fit in the K/V tiles");
};

// Head-dim index of fragment slot s held by lane row g (W contiguous values per lane).
template <int W>
__device__ __forceinline__ constexpr int pf_frag_dim(int s, int g) {
    return 4 * W * (s / W) + W * g + (s % W);
}

constexpr float kPrefillLazyRescale = 8.f;  // log2 headroom before the running max is moved

template <int N>
__device__ __forceinline__ void pf_lds_vec(const float* p, float (&x)[N]) {
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
__global__ __launch_bounds__(512) void attn_prefill_kernel(
    const float* __restrict__ Q, const float* __restrict__ Kp, const float* __restrict__ Vp,
    const int32_t* __restrict__ BT, const int32_t* __restrict__ CTX, const int32_t* __restrict__ TS,
    float* __restrict__ O, float* __restrict__ LSE, int S, int N, int Hq, int Hkv, int PS, int max_pages,
    int num_pages, int ngroups, float c2 /* scale * log2(e) */) {
    using Tr = PrefillTraits<D>;
    __shared__ __attribute__((aligned(16))) float smem[Tr::SMEM_FLOATS];
    __shared__ int sel[2];  // this work-group's sequence and query block (-1: none)
    float* Ks = smem;
    float* Vs = smem + Tr::KS_FLOATS;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_uniform(tid >> 6);
    const int rw = w & 3;   // row group: rows 16rw .. +15 of the block
    const int kh = w >> 2;  // key half: sub-tiles 2kh, 2kh+1 of every tile
    const int li = lane & 15;
    const int g = lane >> 4;
    // the query heads of a KV head on one XCD (their K/V pages fetched into its L2 once)
    const int wi = xcd_grouped_item(blockIdx.x, Hq / Hkv, ngroups);
    if (wi < 0) return;  // uniform: a padding work-group, before any barrier
    const int item = wi / Hq;
    const int h = wi % Hq;

    // Which (sequence, block) is item number `item`.  Items run heaviest block first
    // over the whole batch (most key tiles; ties by sequence, then block), so the
    // longest blocks start in the first round and no long block is left for the end.
    // Block qb of sequence s reaches position L = min(base + min(64qb + 64, n) - 1,
    // ctx - 1) and visits max(L, 0) / 64 + 1 key tiles, non-decreasing in qb; the
    // item-th largest count is found by bisection on the number of blocks with at
    // least t tiles, which has a closed form per sequence (one lane each, 64
    // sequences at a time).  Token offsets and lengths are clamped as below, so a
    // broken table gives wrong numbers, never a bad read.
    if (w == 0) {
        const int cap = PS * max_pages;
        struct SeqBlocks {
            int nb, n, base, ctxm1;
        };
        auto seq_at = [&](int sq) {
            SeqBlocks r{0, 0, 0, -1};
            if (sq < S) {
                const int a = min(max(TS[sq], 0), N), b = min(max(TS[sq + 1], 0), N);
                const int n = max(b - a, 0);
                const int ctx = min(max(CTX[sq], 0), cap);
                r = SeqBlocks{(n + Tr::BM - 1) / Tr::BM, n, max(ctx - n, 0), ctx - 1};
            }
            return r;
        };
        // blocks of one sequence with at least t key tiles
        auto cnt_ge = [&](const SeqBlocks& q, int t) {
            if (t <= 1) return q.nb;
            const int P = Tr::BN * (t - 1);  // L >= P  <=>  at least t tiles
            const int R = P - q.base + 1;    // ... <=>  min(64qb + 64, n) >= R and ctx - 1 >= P
            if (q.nb == 0 || q.ctxm1 < P || q.n < R) return 0;
            return q.nb - (R <= Tr::BM ? 0 : (R - 1) / Tr::BM);  // first such qb: 64qb + 64 >= R
        };
        const SeqBlocks q0 = seq_at(lane);
        auto total_ge = [&](int t) {
            int tot = 0;
            for (int c0 = 0; c0 < S; c0 += 64) {
                const SeqBlocks q = c0 == 0 ? q0 : seq_at(c0 + lane);
                tot += __builtin_amdgcn_readlane(wave_incl_scan(cnt_ge(q, t)), 63);
            }
            return tot;
        };
        int s_sel = -1, qb_sel = 0;
        if (item < total_ge(1)) {
            int tmax = 0;  // most tiles of any block: the last block of some sequence
            for (int c0 = 0; c0 < S; c0 += 64) {
                const SeqBlocks q = c0 == 0 ? q0 : seq_at(c0 + lane);
                const int last = q.nb > 0 ? max(min(q.base + q.n - 1, q.ctxm1), 0) / Tr::BN + 1 : 0;
                tmax = max(tmax, last);
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) tmax = max(tmax, __shfl_xor(tmax, m));
            int lo = 1, hi = tmax;  // total_ge(lo) > item throughout
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (total_ge(mid) > item) lo = mid;
                else hi = mid - 1;
            }
            const int k = item - (lo < tmax ? total_ge(lo + 1) : 0);  // rank among blocks of lo tiles
            int carry = 0;
            for (int c0 = 0; c0 < S && s_sel < 0; c0 += 64) {
                const SeqBlocks q = c0 == 0 ? q0 : seq_at(c0 + lane);
                const int ge = cnt_ge(q, lo);
                const int eq = ge - cnt_ge(q, lo + 1);
                const int incl = carry + wave_incl_scan(eq);
                const uint64_t hit = __ballot(k < incl);
                if (hit) {
                    const int l = __builtin_ctzll(hit);
                    s_sel = c0 + l;
                    const int first = __builtin_amdgcn_readlane(incl - eq, l);
                    qb_sel = __builtin_amdgcn_readlane(q.nb - ge, l) + (k - first);
                }
                carry = __builtin_amdgcn_readlane(incl, 63);
            }
        }
        if (lane == 0) {
            sel[0] = s_sel;
            sel[1] = qb_sel;
        }
    }
    __syncthreads();
    const int s = sel[0];
    if (s < 0) return;  // uniform: past the batch's blocks
    const int qb = sel[1];

    const int t_lo = min(max(TS[s], 0), N);
    const int n_s = max(min(max(TS[s + 1], 0), N) - t_lo, 0);
    const int cap = PS * max_pages;
    const int ctx = min(max(CTX[s], 0), cap);
    const int base = max(ctx - n_s, 0);  // position of new token 0
    const int hk = h / (Hq / Hkv);
    const int32_t* bt_row = BT + (size_t)s * max_pages;
    const int j0 = qb * Tr::BM;          // first new token of the block
    const int jr = j0 + 16 * rw + li;    // this lane's token (column of the S^T tiles)
    const int qpos = base + jr;          // its position
    const int last_pos = min(base + min(j0 + Tr::BM, n_s) - 1, ctx - 1);  // block's last position
    const int wave_last = min(base + min(j0 + 16 * rw + 15, n_s - 1), ctx - 1);  // this wave's last
    const int ntiles = last_pos / Tr::BN + 1;

    if constexpr (Tr::DP != D) {  // zero the padding columns of both V buffers once
        for (int idx = tid; idx < Tr::BN * (Tr::DP - D); idx += Tr::NT) {
            const int row = idx / (Tr::DP - D), col = D + idx % (Tr::DP - D);
            Vs[row * Tr::LDV + col] = 0.f;
            Vs[Tr::TILE_FLOATS + row * Tr::LDV + col] = 0.f;
        }
    }

    // Q fragments: slot s holds Q[token jr][pf_frag_dim(s, g)] (B operand of K Q^T)
    const bool q_ok = jr < n_s;
    const float* Qr = Q + ((size_t)(t_lo + (q_ok ? jr : 0)) * Hq + h) * D;
    float qf[Tr::KSTEPS];
#pragma unroll
    for (int u = 0; u < Tr::KSTEPS / Tr::W; ++u) {
        const int d0 = 4 * Tr::W * u + Tr::W * g;
        if constexpr (Tr::W == 4) {
            const f32x4 x = *(const f32x4*)(Qr + d0);
#pragma unroll
            for (int j = 0; j < 4; ++j) qf[4 * u + j] = q_ok ? x[j] : 0.f;
        } else {
            const f32x2 x = *(const f32x2*)(Qr + d0);
            qf[2 * u] = q_ok ? x[0] : 0.f;
            qf[2 * u + 1] = q_ok ? x[1] : 0.f;
        }
    }

    f32x4 acc[Tr::NDT];  // O as [token 16rw + 4g + r][dim NDT*li + dt]
#pragma unroll
    for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -FLT_MAX;  // lowest finite start: a half with no visible key gives exp2(-inf) = 0
    float l_run = 0.f;

    // Each thread stages the same PER rows of every tile; their page ids are loaded
    // one tile ahead (pg_next) so the K/V loads never wait on the table.
    int pg_next[Tr::PER];
    auto table = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < Tr::PER; ++i) {
            const int idx = tid + Tr::NT * i;
            const int row = idx / (D / 4);
            const int p = min(kv0 + row, cap - 1);
            pg_next[i] = bt_row[p / PS];
        }
    };
    f32x4 kreg[Tr::PER], vreg[Tr::PER];
    auto gload = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < Tr::PER; ++i) {
            const int idx = tid + Tr::NT * i;
            if (Tr::TILE4 % Tr::NT == 0 || idx < Tr::TILE4) {
                const int row = idx / (D / 4), c4 = idx % (D / 4);
                const int p = kv0 + row;
                const int phys = min(max(pg_next[i], 0), num_pages - 1);
                const size_t at = (((size_t)phys * Hkv + hk) * PS + (p % PS)) * D + 4 * c4;
                const f32x4 kx = *(const f32x4*)(Kp + at);
                const f32x4 vx = *(const f32x4*)(Vp + at);
                const bool ok = p < ctx;  // past the context: zeros (the slot may hold anything)
                kreg[i] = ok ? kx : f32x4{0.f, 0.f, 0.f, 0.f};
                vreg[i] = ok ? vx : f32x4{0.f, 0.f, 0.f, 0.f};
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

    // Two K/V buffers: while tile j is multiplied, tile j + 1 goes into the other buffer
    // and tile j + 2 into registers, so one barrier per tile suffices (as in the forward).
    table(0);
    gload(0);
    table(Tr::BN);
    lstore(0);
    if (1 < ntiles) {
        gload(Tr::BN);
        table(2 * Tr::BN);
    }
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        // tile j is in buffer j & 1; buffer (j + 1) & 1 was last read in iteration j - 1,
        // which every wave finished before the barrier that ended it
        Ks = smem + (j & 1) * Tr::TILE_FLOATS;
        Vs = Ks + Tr::KS_FLOATS;

        const int kv0 = j * Tr::BN;
        // 16-key sub-tiles with a key <= this wave's last position
        const int nsub = wave_last < kv0 ? 0 : min((wave_last - kv0) / 16 + 1, 4);
        const bool masked = kv0 + Tr::BN - 1 > base + j0 + 16 * rw;  // some key past the wave's first row

        // S^T = K Q^T over this wave's key half: st[tt] holds
        // S^T[key = kv0 + 16(2kh + tt) + 4g + r][token = jr].  Both sub-tiles are formed,
        // also one past the wave's last position (masked below, its P V skipped), so that
        // the two accumulation chains interleave with no branch between them.
        f32x4 st[2];
        st[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        st[1] = st[0];
#pragma unroll
        for (int u = 0; u < Tr::KSTEPS / Tr::W; ++u) {
            float a[2][Tr::W];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                pf_lds_vec<Tr::W>(&Ks[(16 * (2 * kh + tt) + li) * Tr::LDK + 4 * Tr::W * u + Tr::W * g], a[tt]);
#pragma unroll
            for (int jj = 0; jj < Tr::W; ++jj)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) st[tt] = mfma16x16x4(a[tt][jj], qf[Tr::W * u + jj], st[tt]);
        }

        // mask and scale to log2 units; this lane's max over its 8 keys of the tile
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * kh + tt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kv0 + 16 * t + 4 * g + r;
                float x = st[tt][r] * c2;
                if (t >= nsub || (masked && key > qpos)) x = -INFINITY;
                st[tt][r] = x;
                mx = fmaxf(mx, x);
            }
        }
        if (__ballot(mx > m_run + kPrefillLazyRescale)) {  // wave-uniform
            const float m_new = fmaxf(m_run, rows4_max(mx));
            const float alpha = exp2_hw(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * g + r);  // alpha of token 16rw + 4g + r
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt][r] *= ar;
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2_hw(st[tt][r] - m_run);
                st[tt][r] = p;
                l_run += p;
            }
        }

        // O += P V : P[token li][key 16t + 4g + r] is the A operand as it stands
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * kh + tt;
            if (t < nsub) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float bv[Tr::NDT];
                    pf_lds_vec<Tr::NDT>(&Vs[(16 * t + 4 * g + r) * Tr::LDV + Tr::NDT * li], bv);
#pragma unroll
                    for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = mfma16x16x4(st[tt][r], bv[dt], acc[dt]);
                }
            }
        }
        if (j + 1 < ntiles) {
            lstore((j + 1) & 1);
            if (j + 2 < ntiles) {
                gload((j + 2) * Tr::BN);
                table((j + 3) * Tr::BN);
            }
        }
        __syncthreads();
    }

    // Merge the two key halves through LDS (half 1 hands its state to half 0).
    const float l_half = rows4_sum(l_run);
    float* mbuf = smem + rw * Tr::MERGE_REGS * 64 + lane;
    __syncthreads();
    if (kh == 1) {
#pragma unroll
        for (int dt = 0; dt < Tr::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mbuf[(4 * dt + r) * 64] = acc[dt][r];
        mbuf[(4 * Tr::NDT) * 64] = m_run;
        mbuf[(4 * Tr::NDT + 1) * 64] = l_half;
    }
    __syncthreads();
    if (kh == 1) return;

    const float m_o = mbuf[(4 * Tr::NDT) * 64];
    const float l_o = mbuf[(4 * Tr::NDT + 1) * 64];
    const float m_tot = fmaxf(m_run, m_o);
    const float a_s = exp2_hw(m_run - m_tot);
    const float a_o = exp2_hw(m_o - m_tot);
    const float l_tot = a_s * l_half + a_o * l_o;
    const float inv = 1.f / l_tot;
    if (g == 0 && q_ok && LSE) LSE[(size_t)(t_lo + jr) * Hq + h] = (m_tot + log2_hw(l_tot)) * kLn2;
    const float f_s = a_s * inv, f_o = a_o * inv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float fs = __shfl(f_s, 4 * g + r);  // factors of token 16rw + 4g + r
        const float fo = __shfl(f_o, 4 * g + r);
        const int jt = j0 + 16 * rw + 4 * g + r;
        float out[Tr::NDT];
#pragma unroll
        for (int dt = 0; dt < Tr::NDT; ++dt) out[dt] = acc[dt][r] * fs + mbuf[(4 * dt + r) * 64] * fo;
        if (jt < n_s && (Tr::DP == D || li < D)) {
            float* dst = O + ((size_t)(t_lo + jt) * Hq + h) * D + Tr::NDT * li;
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
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream) {
    using Tr = PrefillTraits<D>;
    // at most floor(N / 64) + S query blocks over the batch, whatever the split
    const int64_t items = a.N / Tr::BM + a.S;
    const int64_t G = a.Hq / a.Hkv, ngroups = items * a.Hkv;  // (item, KV head) groups of G query heads
    hipLaunchKernelGGL(attn_prefill_kernel<D>, dim3((unsigned)xcd_grouped_grid(G, ngroups)), dim3(Tr::NT), 0, stream,
                       a.q, a.k_pool, a.v_pool, a.block_table, a.context_lens, a.token_start, a.o, a.lse, (int)a.S,
                       (int)a.N, (int)a.Hq, (int)a.Hkv, (int)a.page_size, (int)a.max_pages, (int)a.num_pages,
                       (int)ngroups, a.scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 8: return launch_prefill_d<8>(a, stream);
        case 16: return launch_prefill_d<16>(a, stream);
        case 32: return launch_prefill_d<32>(a, stream);
        case 64: return launch_prefill_d<64>(a, stream);
        case 128: return launch_prefill_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
