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
//   1. attn_bwd_pre: Delta_i = <dO_i, O_i> into the workspace, dQ = 0, and, when
//      key blocks are shared between work-groups (below), dK = dV = 0 on the
//      key blocks that may be shared;
//   2. attn_bwd_main: the work of one (batch, KV head) is the list of steps
//      (key block kb, query head, query tile >= kb) of all its key blocks.  For a
//      long enough grid a work-group takes one whole key block, heaviest first.
//      For a short grid the heaviest key block alone would set the kernel's
//      length (key block 0 has the most steps), so the key blocks are ordered
//      0, n-1, 1, n-2, ... -- every such pair has the same number of steps -- and
//      the list is cut into equal runs, one per work-group: half a pair each, or,
//      when that leaves CUs idle (few batch x KV heads, e.g. grouped-query heads
//      at small batch), as many runs as the chip holds work-groups.  With half
//      pairs a key block that is cut in two adds its dK, dV atomically onto
//      zero; two addends onto zero give the same bits in either order.  With
//      finer runs a block can be cut into more pieces: each run then stores its
//      piece in a workspace slot of its own, and
//   3. attn_bwd_post sums the pieces of each shared block in run order.  Either
//      way dK, dV are deterministic.  Within a key block,
//      wave w owns keys kv0+16w .. +15 and keeps their K, V fragments and dK, dV
//      accumulators in registers.  Per step (64 query rows, Q and dO in LDS):
//        S  = Q K^T, dP = dO V^T           (C tiles: key in the lane i)
//        P, dS                             (elementwise, masked on the diagonal)
//        dV += P^T dO,  dK += dS^T Q       (P and dS are the A operands as-is; the
//                                           dO and Q rows load as vectors because
//                                           lane i owns dims NDT*i .. NDT*i+NDT-1)
//        dS -> LDS, then dQ(16 rows per wave) = dS K, added to dQ with float
//        atomics (the contraction runs over the whole 64-key block).
#include <algorithm>

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
                                                           float* __restrict__ dQ, int64_t rows,
                                                           float* __restrict__ dK, float* __restrict__ dV,
                                                           int64_t T, int64_t nbkv, int64_t zrows) {
    constexpr int TPR = D / 4;  // threads per row, one float4 each
    constexpr int RPB = 256 / TPR;
    const int tid = threadIdx.x;
    const int part = tid % TPR;
    const int64_t qblocks = (rows + RPB - 1) / RPB;
    if ((int64_t)blockIdx.x >= qblocks) {  // trailing blocks: dK = dV = 0 on the first zrows keys of each head
        const int64_t zr = ((int64_t)blockIdx.x - qblocks) * RPB + tid / TPR;
        if (zr < nbkv * zrows) {
            const int64_t row = (zr / zrows) * T + zr % zrows;
            *(f32x4*)(dK + row * D + 4 * part) = f32x4{0.f, 0.f, 0.f, 0.f};
            *(f32x4*)(dV + row * D + 4 * part) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }
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
    static constexpr int LD = DP + 4;               // LDS row stride of the Q, dO tiles
    static constexpr int LDS_ = BN + 4;             // LDS row stride of the dS tile
    static constexpr int LDT = BN + 4;              // LDS row stride of the transposed K tile
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

// MAT (the materialized variant): the probabilities come from a stored P
// [B,Hq,T,T] instead of exp(s - LSE), so S = Q K^T is not formed; dPx (may be
// NULL) is a cotangent of P itself, added to dP.
template <int D, bool MAT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D >= 128 ? 1 : 2, D >= 128 ? 1 : 2))) void attn_bwd_main_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    const float* __restrict__ P, const float* __restrict__ dPx,
    float* __restrict__ dQ, float* __restrict__ dK, float* __restrict__ dV, int Hq, int Hkv, int T,
    int nkb, int nbkv, int runs, int desc, float scale, float c2 /* scale * log2(e) */) {
    using Tr = BwdTraits<D>;
    __shared__ __attribute__((aligned(16))) float Qs[Tr::BM * Tr::LD];
    __shared__ __attribute__((aligned(16))) float dOs[Tr::BM * Tr::LD];
    __shared__ __attribute__((aligned(16))) float Kt[Tr::DP * Tr::LDT];  // K^T: [dim][key]
    __shared__ __attribute__((aligned(16))) float dSs[Tr::BM * Tr::LDS_];
    __shared__ __attribute__((aligned(16))) float lse2s[Tr::BM];
    __shared__ __attribute__((aligned(16))) float dls[Tr::BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_uniform(tid >> 6);
    const int li = lane & 15;
    const int g = lane >> 4;

    const int G = Hq / Hkv;
    const int nqb = (T + Tr::BM - 1) / Tr::BM;  // == nkb (BM == BN)
    // Key block kb has G * (nqb - kb) steps (query head, query tile >= kb).  In the
    // paired order 0, nkb-1, 1, nkb-2, ... two neighbours hold G * (nkb + 1) steps
    // together; position pi of that order is key block kb_at(pi), whose steps
    // start at start_at(pi) in the concatenated list.
    const int64_t pair_len = (int64_t)G * (nkb + 1);
    auto kb_at = [&](int pi) { return (pi & 1) ? nkb - 1 - (pi >> 1) : (pi >> 1); };
    auto start_at = [&](int pi) -> int64_t {
        const int pr = pi >> 1;
        return pr * pair_len + ((pi & 1) ? (int64_t)G * (nkb - pr) : 0);
    };
    // Finer runs only: (bkv * runs + run) << 16 | the run's first position pi, all the
    // epilogue needs to find a shared block's workspace slot (one register through the
    // step loop; bkv * runs + run < 512 and pi < 2 nkb <= 1024 there).
    int fine_tag = 0;
    int bkv, pi = 0, kb_fixed = 0;
    int64_t s_begin, s_end;
    if (runs == 0) {  // one work-group per key block, heaviest first
        const int rank = blockIdx.x;
        kb_fixed = rank / nbkv;
        bkv = rank % nbkv;
        s_begin = 0;
        s_end = (int64_t)G * (nqb - kb_fixed);
    } else {  // run `run` of `runs` equal runs (runs == nkb: half a pair each)
        // Runs alternate between the floor and the ceiling of total / runs steps (an odd
        // run is the longer one and holds the switch to its second key block).  When the
        // grid fills the chip once, work-groups i and i + grid/2 share a CU, and the one
        // placed first gets ahead at the start (its partner's first step took 18 us vs
        // 11 us): give the pair neighbouring runs, the longer one to work-group i.
        int run;
        const int half_grid = (int)(gridDim.x / 2);
        if ((runs & 1) == 0) {
            const int hi = (int)blockIdx.x >= half_grid ? 1 : 0;
            const int j = (int)blockIdx.x - hi * half_grid;
            run = 2 * (j / nbkv) + 1 - hi;
            bkv = j % nbkv;
        } else {
            run = blockIdx.x / nbkv;
            bkv = blockIdx.x % nbkv;
        }
        const int64_t total = (int64_t)G * nkb * (nkb + 1) / 2;
        s_begin = (int64_t)run * total / runs;
        s_end = (int64_t)(run + 1) * total / runs;
        const int pr = (int)(s_begin / pair_len);
        pi = 2 * pr + (s_begin - pr * pair_len >= (int64_t)G * (nkb - pr) ? 1 : 0);
        fine_tag = ((bkv * runs + run) << 16) | pi;
    }
    const int b = bkv / Hkv;
    const int hk = bkv % Hkv;
    const float* Kh = K + ((size_t)b * Hkv + hk) * (size_t)T * D;
    const float* Vh = V + ((size_t)b * Hkv + hk) * (size_t)T * D;
    float* dKh = dK + ((size_t)b * Hkv + hk) * (size_t)T * D;
    float* dVh = dV + ((size_t)b * Hkv + hk) * (size_t)T * D;

    if constexpr (Tr::DP != D) {  // padding dims of the Q, dO, K tiles stay zero
        for (int idx = tid; idx < Tr::BM * (Tr::DP - D); idx += Tr::NT) {
            const int row = idx / (Tr::DP - D), col = D + idx % (Tr::DP - D);
            Qs[row * Tr::LD + col] = 0.f;
            dOs[row * Tr::LD + col] = 0.f;
            Kt[col * Tr::LDT + row] = 0.f;
        }
    }

    if (s_begin >= s_end) return;

    constexpr int PER = (Tr::TILE4 + Tr::NT - 1) / Tr::NT;
    f32x4 xq[PER], xo[PER];
    float xl = INFINITY, xd = 0.f;
    float kf[Tr::KSTEPS], vf[Tr::KSTEPS];  // K, V fragments of this lane's key
    f32x4 kt[PER];                         // this thread's rows of the K tile, on their way to LDS

    // The segment of the run that starts at step s0, position p0 of the pair order: its
    // key block and its steps [j0, j1) within the block (at most two segments per run
    // with half pairs; wave-uniform).
    int kb = 0, j0 = 0, j1 = 0;
    bool whole = false;
    int64_t seg_end = 0;
    auto locate = [&](int64_t s0, int p0) {
        kb = runs ? kb_at(p0) : kb_fixed;
        const int64_t kb_first = runs ? start_at(p0) : 0;
        const int64_t kb_end = kb_first + (int64_t)G * (nqb - kb);
        seg_end = s_end < kb_end ? s_end : kb_end;
        whole = (s0 == kb_first && seg_end == kb_end);  // no other run shares this key block
        j0 = (int)(s0 - kb_first);
        j1 = (int)(seg_end - kb_first);
    };

    // Step j of key block kb is query head hk*G + j / (nqb - kb) and, with s = j % (nqb - kb),
    // query tile kb + s, or nqb - 1 - s when desc is set (see the launcher).
    auto qtile = [&](int kb_, int s) { return desc ? nqb - 1 - s : kb_ + s; };
    // A step's Q, dO rows and row statistics are loaded into registers during the previous
    // step's dQ phase (or with the segment's K, V) and written to LDS at the top of the step.
    auto prefetch = [&](int step) {
        const int nqt_ = nqb - kb;
        const int h = hk * G + step / nqt_;
        const int q0 = qtile(kb, step % nqt_) * Tr::BM;
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
            xl = !MAT && q < T ? LSE[hoff + q] * kLog2e : INFINITY;
            xd = q < T ? Delta[hoff + q] : 0.f;
        }
    };

    // What a segment reads from memory before its first step, issued at once into
    // registers: this lane's K, V fragments (slot s holds [key][frag_dim_b(s, g)]), its
    // rows of the K tile and (with_q) the first step's Q, dO rows.  For a run's second
    // segment the K, V part is issued before the first segment's dK, dV leave, so that
    // those loads do not queue behind the writes (1-2 % at the 1024- and 8192-token
    // shapes); the Q, dO rows follow the writes, since holding them across the atomic
    // flush as well made the compiler spill registers.  The materialized variant, which
    // holds more state, loads everything after the writes.
    auto load_segment = [&](bool with_q) {
        const int keyw_ = kb * Tr::BN + 16 * w + li;
#pragma unroll
        for (int u = 0; u < Tr::KSTEPS / Tr::W; ++u) {
            const int d0 = 4 * Tr::W * u + Tr::W * g;
            if constexpr (Tr::W == 4) {
                f32x4 x = !MAT && keyw_ < T ? *(const f32x4*)(Kh + (size_t)keyw_ * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
                f32x4 y = keyw_ < T ? *(const f32x4*)(Vh + (size_t)keyw_ * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kf[4 * u + j] = x[j];
                    vf[4 * u + j] = y[j];
                }
            } else {
                f32x2 x = !MAT && keyw_ < T ? *(const f32x2*)(Kh + (size_t)keyw_ * D + d0) : f32x2{0.f, 0.f};
                f32x2 y = keyw_ < T ? *(const f32x2*)(Vh + (size_t)keyw_ * D + d0) : f32x2{0.f, 0.f};
                kf[2 * u] = x[0];
                kf[2 * u + 1] = x[1];
                vf[2 * u] = y[0];
                vf[2 * u + 1] = y[1];
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + Tr::NT * i;
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const int key = kb * Tr::BN + row;
            kt[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if ((Tr::TILE4 % Tr::NT == 0 || idx < Tr::TILE4) && key < T)
                kt[i] = *(const f32x4*)(Kh + (size_t)key * D + 4 * c4);
        }
        if (with_q) prefetch(j0);
    };

    locate(s_begin, pi);
    load_segment(true);
    for (;;) {
        const int kv0 = kb * Tr::BN;
        const int nqt = nqb - kb;
        const int keyw = kv0 + 16 * w + li;  // this lane's key (column of the S / dP tiles)
        const int kbs = kb, js0 = j0, js1 = j1;
        const bool wholes = whole;
        const int64_t s_next = seg_end;

        __syncthreads();  // the previous segment's readers of Kt, Qs and dOs are done

        // the key block's K tile in LDS, transposed (B operand of dQ = dS K: four
        // consecutive keys of one dim are one vector read)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + Tr::NT * i;
            if (Tr::TILE4 % Tr::NT == 0 || idx < Tr::TILE4) {
                const int row = idx / (D / 4), c4 = idx % (D / 4);
#pragma unroll
                for (int c = 0; c < 4; ++c) Kt[(4 * c4 + c) * Tr::LDT + row] = kt[i][c];
            }
        }

        // dK, dV accumulators as [key 4g + r][dim NDT*li + dt] (this wave's 16 keys)
        f32x4 dk[Tr::NDT], dv[Tr::NDT];
#pragma unroll
        for (int dt = 0; dt < Tr::NDT; ++dt) {
            dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        for (int step = js0; step < js1; ++step) {
            const int h = hk * G + step / nqt;
            const int qb = qtile(kbs, step % nqt);
            const size_t hoff = ((size_t)b * Hq + h) * (size_t)T;
            float* dQh = dQ + hoff * D;
            {
                const int q0 = qb * Tr::BM;
                // No barrier before these stores: every reader of the previous step's Q, dO
                // and row statistics (the S/dP, softmax and dV/dK phases) came before that
                // step's barrier after the dS store, and a segment starts with a barrier.
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
                const bool diag = (qb == kbs);

                // S = Q K^T and dP = dO V^T : C[query 16qs + 4g + r][key li].  MAT: S is not
                // formed; sa takes the stored P of this lane's (query, key) entries and dP
                // starts from the cotangent of P.
                f32x4 sa[4], pa[4];
#pragma unroll
                for (int qs = 0; qs < 4; ++qs) {
                    sa[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
                    pa[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (MAT) {
                        const size_t prow = ((size_t)b * Hq + h) * (size_t)T;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int q = q0 + 16 * qs + 4 * g + r;
                            const bool in = q < T && keyw < T;
                            const size_t at = (prow + (in ? q : 0)) * (size_t)T + (in ? keyw : 0);
                            sa[qs][r] = in ? P[at] : 0.f;
                            if (dPx) pa[qs][r] = in ? dPx[at] : 0.f;
                        }
                    }
                }
                if constexpr (Tr::W == 4) {
                    // Batches k = (qs, u) of 4 k-steps: one Q and one dO vector from LDS feed 8
                    // MFMAs.  The next batch's vectors are read before this batch's MFMAs, and
                    // scheduling barriers keep that order: left to itself the compiler read each
                    // batch just before its MFMAs and waited out the LDS latency every 16 MFMAs
                    // (133 -> 130 us at B=4, H=8, T=1024, d=64).
                    constexpr int NU = Tr::KSTEPS / 4;  // batches per 16-query sub-tile
                    constexpr int NB = 4 * NU;
                    auto offk = [&](int k) { return (16 * (k / NU) + li) * Tr::LD + 16 * (k % NU) + 4 * g; };
                    f32x4 an{0.f, 0.f, 0.f, 0.f}, cn;
                    if constexpr (!MAT) an = *(const f32x4*)&Qs[offk(0)];
                    cn = *(const f32x4*)&dOs[offk(0)];
#pragma unroll
                    for (int k = 0; k < NB; ++k) {
                        const f32x4 a = an, c = cn;
                        if (k + 1 < NB) {
                            if constexpr (!MAT) an = *(const f32x4*)&Qs[offk(k + 1)];
                            cn = *(const f32x4*)&dOs[offk(k + 1)];
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        const int qs = k / NU, u = k % NU;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            if constexpr (!MAT) sa[qs] = mfma16x16x4(a[j], kf[4 * u + j], sa[qs]);
                            pa[qs] = mfma16x16x4(c[j], vf[4 * u + j], pa[qs]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
#pragma unroll
                    for (int qs = 0; qs < 4; ++qs) {
#pragma unroll
                        for (int u = 0; u < Tr::KSTEPS / Tr::W; ++u) {
                            const int off = (16 * qs + li) * Tr::LD + 4 * Tr::W * u + Tr::W * g;
                            const f32x2 a = *(const f32x2*)&Qs[off];
                            const f32x2 c = *(const f32x2*)&dOs[off];
#pragma unroll
                            for (int j = 0; j < 2; ++j) {
                                if constexpr (!MAT) sa[qs] = mfma16x16x4(a[j], kf[2 * u + j], sa[qs]);
                                pa[qs] = mfma16x16x4(c[j], vf[2 * u + j], pa[qs]);
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
                        float p = MAT ? sa[qs][r] : exp2_hw(sa[qs][r] * c2 - l4[r]);
                        p = (diag && 16 * w + li > qr) ? 0.f : p;
                        const float ds = scale * p * (pa[qs][r] - d4[r]);
                        sa[qs][r] = p;
                        pa[qs][r] = ds;
                    }
                }

                // dV += P^T dO and dK += dS^T Q with P, dS as the A operands straight from their
                // accumulators (k-step (qs, r) pairs lane row g with query 16qs + 4g + r) and the
                // dO / Q rows as B operands, lane li taking dims NDT*li .. NDT*li+NDT-1
                {
                    // batches k = (qs, r), their dO and Q row slices read one batch ahead
                    auto roff = [&](int k) { return (16 * (k / 4) + 4 * g + k % 4) * Tr::LD + Tr::NDT * li; };
                    float bon[Tr::NDT], bqn[Tr::NDT];
                    lds_row<Tr::NDT>(&dOs[roff(0)], bon);
                    lds_row<Tr::NDT>(&Qs[roff(0)], bqn);
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        float bo[Tr::NDT], bq[Tr::NDT];
#pragma unroll
                        for (int dt = 0; dt < Tr::NDT; ++dt) {
                            bo[dt] = bon[dt];
                            bq[dt] = bqn[dt];
                        }
                        if (k + 1 < 16) {
                            lds_row<Tr::NDT>(&dOs[roff(k + 1)], bon);
                            lds_row<Tr::NDT>(&Qs[roff(k + 1)], bqn);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        const int qs = k / 4, r = k % 4;
#pragma unroll
                        for (int dt = 0; dt < Tr::NDT; ++dt) {
                            dv[dt] = mfma16x16x4(sa[qs][r], bo[dt], dv[dt]);
                            dk[dt] = mfma16x16x4(pa[qs][r], bq[dt], dk[dt]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }

                if (step + 1 < js1) prefetch(step + 1);  // lands during the dQ phase

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
                        f32x4 kop[Tr::NDT];
#pragma unroll
                        for (int dt = 0; dt < Tr::NDT; ++dt)
                            kop[dt] = *(const f32x4*)&Kt[(16 * dt + li) * Tr::LDT + 16 * u + 4 * g];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int dt = 0; dt < Tr::NDT; ++dt) qa[dt] = mfma16x16x4(a[j], kop[dt][j], qa[dt]);
                    }
                }
                if constexpr (Tr::NDT % 4 == 0) {
                    // Transpose each 4x4 block (lane row g) x (dim tile dt) with the row-swap
                    // permutes so that one atomic instruction covers 64 consecutive dims of
                    // one query row: afterwards register x of lane (g, li) holds
                    // dQ[query 16w + 4x + r][dim 64c + 16g + li].
#pragma unroll
                    for (int c = 0; c < Tr::NDT / 4; ++c) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float m[4] = {qa[4 * c][r], qa[4 * c + 1][r], qa[4 * c + 2][r], qa[4 * c + 3][r]};
                            swap_rows32(m[0], m[2]);
                            swap_rows32(m[1], m[3]);
                            swap_rows16(m[0], m[1]);
                            swap_rows16(m[2], m[3]);
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                const int q = q0 + 16 * w + 4 * x + r;
                                if (q < T) unsafeAtomicAdd(dQh + (size_t)q * D + 64 * c + lane, m[x]);
                            }
                        }
                    }
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

        // dK, dV: lane (g, li) holds keys kv0 + 16w + 4g + r, dims NDT*li .. NDT*li+NDT-1.
        const bool more = s_next < s_end;  // another segment follows
        if (wholes || runs > nkb) {
            if (more && !MAT) {
                locate(s_next, pi + 1);
                load_segment(true);
            }
            // plain stores: into dK, dV when no other run shares this key block, else
            // (finer runs) into this run's workspace slot after Delta: slot 0 for the
            // run's first segment, 1 for its last.
            float* dKb = dKh + (size_t)kv0 * D;
            float* dVb = dVh + (size_t)kv0 * D;
            if (!wholes) {
                const size_t slot = (size_t)(fine_tag >> 16) * 2 + (pi != (fine_tag & 0xFFFF) ? 1 : 0);
                float* part = const_cast<float*>(Delta) + ((size_t)nbkv * G * T + 63) / 64 * 64;
                dKb = part + slot * (2 * Tr::BN * D);
                dVb = dKb + Tr::BN * D;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * w + 4 * g + r;
                if (kv0 + row < T && (Tr::DP == D || li < D)) {
                    float* dKr = dKb + (size_t)row * D + Tr::NDT * li;
                    float* dVr = dVb + (size_t)row * D + Tr::NDT * li;
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
        } else {
            // Shared with another run: add onto the zeroed outputs.  The block goes
            // through LDS (the Q and dO tiles are free now) so that each atomic
            // instruction covers whole rows.
            __syncthreads();  // the last step's readers of Qs, dOs are done
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = (16 * w + 4 * g + r) * Tr::LD + Tr::NDT * li;
#pragma unroll
                for (int dt = 0; dt < Tr::NDT; ++dt) {
                    Qs[row + dt] = dk[dt][r];
                    dOs[row + dt] = dv[dt][r];
                }
            }
            __syncthreads();
            if (more && !MAT) {
                locate(s_next, pi + 1);
                load_segment(false);
            }
            for (int idx = tid; idx < Tr::BN * D; idx += Tr::NT) {
                const int kr = idx / D, d = idx % D;
                if (kv0 + kr < T) {
                    unsafeAtomicAdd(dKh + (size_t)(kv0 + kr) * D + d, Qs[kr * Tr::LD + d]);
                    unsafeAtomicAdd(dVh + (size_t)(kv0 + kr) * D + d, dOs[kr * Tr::LD + d]);
                }
            }
        }
        if (!more) break;
        if constexpr (MAT) {
            locate(s_next, pi + 1);
            load_segment(true);
        } else if (!(wholes || runs > nkb)) {
            prefetch(j0);
        }
        ++pi;
    }
}

// ---------------------------------------------------------------------------
// 3. finer runs only: dK, dV of the key blocks that several runs share
// ---------------------------------------------------------------------------
// One work-group per (256 float4 of a key block's dK, dV; key block; batch x KV
// head).  The runs that hold a piece of the block are found from the same equal cut
// of the step list as in the main kernel, and their pieces are summed in run order,
// so the bits do not depend on which run finished first.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_post_kernel(const float* __restrict__ part, float* __restrict__ dK,
                                                            float* __restrict__ dV, int G, int T, int nkb, int nbkv,
                                                            int runs) {
    constexpr int BN = BwdTraits<D>::BN;
    constexpr int ROW4 = D / 4;  // float4 per key row
    const int blk = blockIdx.x % (nbkv * nkb);
    const int idx = (blockIdx.x / (nbkv * nkb)) * 256 + threadIdx.x;  // float4 of [dK; dV] of the block
    const int bkv = blk % nbkv;
    const int kb = blk / nbkv;
    // the block's place in the paired order 0, nkb-1, 1, nkb-2, ... and its step range
    const int pi = 2 * kb < nkb ? 2 * kb : 2 * (nkb - 1 - kb) + 1;
    const int pr = pi >> 1;
    const int64_t pair_len = (int64_t)G * (nkb + 1);
    const int64_t bs = pr * pair_len + ((pi & 1) ? (int64_t)G * (nkb - pr) : 0);
    const int64_t be = bs + (int64_t)G * (nkb - kb);
    const int64_t total = (int64_t)G * nkb * (nkb + 1) / 2;
    // run r holds steps [r * total / runs, (r + 1) * total / runs)
    const int r0 = (int)(((bs + 1) * runs - 1) / total);
    const int r1 = (int)((be * runs - 1) / total);
    if (r0 == r1) return;  // a single run held the block and stored it
    if (idx >= 2 * BN * ROW4) return;
    const int half = idx / (BN * ROW4);  // 0: dK, 1: dV
    const int e = idx % (BN * ROW4);
    const int key = kb * BN + e / ROW4;
    if (key >= T) return;
    // the block is run r0's first segment if r0 starts on it, else r0's last; it is
    // the first segment of every later run that holds a piece of it
    const int w0 = (int64_t)r0 * total / runs == bs ? 0 : 1;
    constexpr size_t PIECE = 2 * (size_t)BN * D;  // dK then dV, [BN, D] each
    const float* base = part + (size_t)bkv * runs * 2 * PIECE + (size_t)half * BN * D + 4 * (size_t)e;
    f32x4 acc = *(const f32x4*)(base + ((size_t)r0 * 2 + w0) * PIECE);
    int r = r0 + 1;
    for (; r + 4 <= r1 + 1; r += 4) {  // four loads in flight, added in run order
        const f32x4 x0 = *(const f32x4*)(base + (size_t)r * 2 * PIECE);
        const f32x4 x1 = *(const f32x4*)(base + (size_t)(r + 1) * 2 * PIECE);
        const f32x4 x2 = *(const f32x4*)(base + (size_t)(r + 2) * 2 * PIECE);
        const f32x4 x3 = *(const f32x4*)(base + (size_t)(r + 3) * 2 * PIECE);
        acc += x0;
        acc += x1;
        acc += x2;
        acc += x3;
    }
    for (; r <= r1; ++r) acc += *(const f32x4*)(base + (size_t)r * 2 * PIECE);
    *(f32x4*)((half ? dV : dK) + ((size_t)bkv * T + key) * D + 4 * (e % ROW4)) = acc;
}

// Runs per (batch, KV head) of the finer cut at most: the total over the grid stays
// within kBwdMaxRunWgs and every run gets at least two steps; 0 when this is no
// finer than half pairs.
static int64_t bwd_fine_runs_max(int64_t B, int64_t Hq, int64_t Hkv, int64_t T) {
    const int64_t nkb = (T + 63) / 64, nbkv = B * Hkv;
    const int64_t total = Hq / Hkv * nkb * (nkb + 1) / 2;
    const int64_t r = std::min<int64_t>(kBwdMaxRunWgs / nbkv, total / 2);
    return r > nkb ? r : 0;
}

static size_t bwd_delta_floats(int64_t B, int64_t Hq, int64_t T) { return (size_t)(B * Hq * T + 63) / 64 * 64; }

constexpr int kBwdDescendingFromTiles = 32;  // 64-key tiles per sequence

template <int D, bool MAT>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
    using Tr = BwdTraits<D>;
    static_assert(Tr::BN == 64, "bwd_fine_runs_max counts 64-key blocks");
    const int nkb = (int)((a.T + Tr::BN - 1) / Tr::BN);
    const int nbkv = (int)(a.B * a.Hkv);
    const int n = nkb * nbkv;  // work-groups with one key block each
    // Two work-groups fit on a CU (one at D >= 128).  When all key blocks are
    // resident at once, the heaviest one alone would set the kernel's length: take
    // half pairs instead, or finer runs when half pairs leave CUs without work.
    int runs = 0;
    float* part = nullptr;
    if (n <= 2 * a.cu_count) {
        runs = nkb;
        const int64_t slots = (int64_t)(D >= 128 ? 1 : 2) * a.cu_count;
        const int64_t fine = std::min<int64_t>(slots / nbkv, bwd_fine_runs_max(a.B, a.Hq, a.Hkv, a.T));
        if (fine > nkb) {
            runs = (int)fine;
            part = a.delta + bwd_delta_floats(a.B, a.Hq, a.T);
        }
    }
    const int64_t rows = a.B * a.Hq * a.T;
    // With half pairs only the first key block of a pair can be cut in two (the cut
    // falls inside it), so only key blocks 0 .. nkb/2 - 1 are added atomically and
    // need zeroing.  Finer runs store every block.
    int64_t zrows = runs > 0 && !part ? (int64_t)(nkb / 2) * Tr::BN : 0;
    if (zrows > a.T) zrows = a.T;
    constexpr int RPB = 256 / (D / 4);
    const int64_t pre_blocks = (rows + RPB - 1) / RPB + (nbkv * zrows + RPB - 1) / RPB;
    hipLaunchKernelGGL(attn_bwd_pre_kernel<D>, dim3((unsigned)pre_blocks), dim3(256), 0, stream, a.o, a.dout,
                       a.delta, a.dq, rows, a.dk, a.dv, a.T, (int64_t)nbkv, zrows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (MAT && a.dpx) {  // Delta_i += sum_j P_ij dPx_ij
        e = launch_mat_delta(a.p, a.dpx, a.delta, rows, a.T, stream);
        if (e != hipSuccess) return e;
    }
    const unsigned grid = runs > 0 ? (unsigned)(runs * nbkv) : (unsigned)n;
    // Query tiles of a key block in descending order for long sequences: the key blocks of
    // a head, which run at the same time on one or two XCDs, then read the same Q, dO tiles
    // at about the same time and find them in that XCD's L2 (measured on one MI355X: 1.5-2 %
    // faster at B=1, Hq=16, Hkv=4, T=8192, d=64, 0.6-0.7 % at T=2048 and 4096, and no gain
    // at T=1024, so the order follows the tile count).  dK, dV stay deterministic either way.
    const int desc = nkb >= kBwdDescendingFromTiles ? 1 : 0;
    hipLaunchKernelGGL((attn_bwd_main_kernel<D, MAT>), dim3(grid), dim3(Tr::NT), 0, stream, a.q, a.k, a.v,
                       a.dout, a.lse, a.delta, a.p, a.dpx, a.dq, a.dk, a.dv, (int)a.Hq, (int)a.Hkv, (int)a.T, nkb,
                       nbkv, runs, desc, a.scale, a.scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess || !part) return e;
    constexpr int chunks = (2 * Tr::BN * D / 4 + 255) / 256;
    hipLaunchKernelGGL(attn_bwd_post_kernel<D>, dim3((unsigned)(n * chunks)), dim3(256), 0, stream, part, a.dk,
                       a.dv, (int)(a.Hq / a.Hkv), (int)a.T, nkb, nbkv, runs);
    return hipGetLastError();
}

size_t bwd_workspace_floats(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D) {
    // Delta [B, Hq, T], then, when the grid may be cut finer than half pairs, two
    // pieces of dK, dV per run
    return bwd_delta_floats(B, Hq, T) + (size_t)(B * Hkv) * bwd_fine_runs_max(B, Hq, Hkv, T) * 2 * 2 * 64 * D;
}

hipError_t launch_causal_bwd(const BwdArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 8: return launch_bwd_d<8, false>(a, stream);
        case 16: return launch_bwd_d<16, false>(a, stream);
        case 32: return launch_bwd_d<32, false>(a, stream);
        case 64: return launch_bwd_d<64, false>(a, stream);
        case 128: return launch_bwd_d<128, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_materialized_bwd(const BwdArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 8: return launch_bwd_d<8, true>(a, stream);
        case 16: return launch_bwd_d<16, true>(a, stream);
        case 32: return launch_bwd_d<32, true>(a, stream);
        case 64: return launch_bwd_d<64, true>(a, stream);
        case 128: return launch_bwd_d<128, true>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
