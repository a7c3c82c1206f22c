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
//   1. attn_decode_split: the 16-position groups of all sequences, taken as one
//      list, are dealt out in equal contiguous shares to a grid sized to the
//      chip, so every CU streams about the same number of bytes however ragged
//      the context lengths are; the waves of a work-group are neighbouring KV
//      heads of the same positions, so a page is read contiguously.  With up to 4
//      query heads per KV head (G / 2 flops per byte) the two small contractions
//      (scores of the G query heads that share the KV head, and the
//      probability-weighted sum of V) run on the vector ALU, with each lane
//      owning a slice of the head dimension; with more they run on fp32 MFMA,
//      which takes the multiply-adds and their cross-lane reductions off the
//      vector ALU, whose issue rate would otherwise bound the kernel below the
//      HBM rate.  Each K and V row is read exactly once per KV head, as
//      contiguous vectors.  Positions past the context get score -inf and a zero
//      V (a select, so a NaN in an unused slot cannot leak in).  One partial
//      (m, l, o) per (work-group, sequence) it touches goes to the workspace.
//   2. attn_decode_combine: per (sequence, query head), merges the partials with
//      the log-sum-exp rule M = max m_c, L = sum 2^(m_c - M) l_c,
//      O = sum 2^(m_c - M) o_c / L.
// For more sequences than the split's partition holds (1024) a single fused kernel
// takes a whole (sequence, KV head) pair per work-group instead.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "attn_launch.h"
#include "device_common.h"

namespace attn {

constexpr int kDecodeWaves = 4;          // waves (KV heads) per work-group of the split path
constexpr int kDecodeWavesPerCu = 4;     // resident waves per CU the split grid aims at
constexpr int kDecodeMaxWgs = 1024;      // bound on the split grid (sizes the workspace)
constexpr int kDecodeDepth = 2;          // groups in flight per wave on the split path
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

// N contiguous floats.  STREAM: a non-temporal load, for the K/V pages that each
// call reads exactly once (measured 4 % faster at the 32-sequence workload).
template <int N, bool STREAM = false>
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float* x) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const f32x4 v = STREAM ? __builtin_nontemporal_load((const f32x4*)(p + 4 * i)) : *(const f32x4*)(p + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[4 * i + j] = v[j];
        }
    } else if constexpr (N == 2) {
        const f32x2 v = STREAM ? __builtin_nontemporal_load((const f32x2*)p) : *(const f32x2*)p;
        x[0] = v[0];
        x[1] = v[1];
    } else {
        x[0] = STREAM ? __builtin_nontemporal_load(p) : *p;
    }
}

// Physical page of group j = lane of the list that starts at group g_first with
// stride g_stride (ng groups; PS a power of two).  One unconditional load per lane:
// lanes past the list re-read its last entry, and the page index is clamped to the
// row and the id to the pool, so a broken table can never send a read out of bounds.
__device__ __forceinline__ int decode_bt_lane(const int32_t* __restrict__ bt_row, int max_pages, int PS,
                                              int num_pages, int g_first, int g_stride, int ng) {
    const int lane = threadIdx.x & 63;
    const int p = (16 * (g_first + g_stride * max(min(lane, ng - 1), 0))) >> __builtin_ctz(PS);
    return min(max(bt_row[min(p, max_pages - 1)], 0), num_pages - 1);
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
//
// The list's page ids come in bt_lane (decode_bt_lane: lane j holds group j's
// physical page), fetched by the caller before anything else it loads, so no group
// waits on a block-table read before it can issue its K/V loads.
template <int D, int DEPTH, int NG_MAX>
__device__ __forceinline__ void decode_groups(const float* __restrict__ Kp, const float* __restrict__ Vp,
                                              int bt_lane, int Hkv, int kvh, int PS, int ctx, int g_first,
                                              int g_stride, int ng, const float (&qf)[DecTraits<D>::KSTEPS],
                                              float c2, float& m, float& l, f32x4 (&acc)[DecTraits<D>::NDT]) {
    using Tr = DecTraits<D>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    auto group_row = [&](int j) -> size_t {  // first pool row of group j
        const int p0 = 16 * (g_first + g_stride * j);
        const int phys = __builtin_amdgcn_readlane(bt_lane, j);
        return ((size_t)phys * Hkv + kvh) * PS + (size_t)(p0 & (PS - 1));
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
        for (int u = 0; u < Tr::KSTEPS / Tr::KW; ++u)
            load_vec<Tr::KW, true>(kp + 4 * Tr::KW * u + Tr::KW * g, &kr[slot][Tr::KW * u]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float* vp = Vp + (r0 + 4 * g + r) * D;
            if (D >= 16 || li < D) load_vec<Tr::VW, true>(vp + Tr::VW * li, vr[slot][r]);
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

// B operand of S: Q^T[d][head li] for the G query heads of KV head kvh
template <int D>
__device__ __forceinline__ void decode_load_q(const float* __restrict__ Qd, int s, int Hq, int kvh, int G,
                                              float (&qf)[DecTraits<D>::KSTEPS]) {
    using Tr = DecTraits<D>;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    // Columns past G repeat the group's first query head: their scores and outputs
    // are formed but never stored, and the loads need no branch or select, so nothing
    // waits on them before the block-table loads are issued.
    const float* qrow = Qd + ((size_t)s * Hq + (size_t)kvh * G + (li < G ? li : 0)) * D;
#pragma unroll
    for (int u = 0; u < Tr::KSTEPS / Tr::KW; ++u) load_vec<Tr::KW>(qrow + 4 * Tr::KW * u + Tr::KW * g, &qf[Tr::KW * u]);
}

// The split path's partition, computed by every wave on its own from the
// sequence lengths (no LDS, no barrier): lane l of chunk c stands for sequence
// s = 64c + l (S <= 64 * NCH) and holds P_{s+1}, the number of 16-position groups
// of sequences 0..s, and the sequence's first partial slot and slot count.  Lengths are clamped to the block table's capacity (and a
// negative one taken as 0), so a broken length can give wrong numbers but never an
// out-of-bounds read.
constexpr int kDecodeScanChunks = 16;  // largest NCH: up to 1024 sequences on the split path

// The partition charges each sequence's start this many 16-position groups of work (a
// share that covers a sequence boundary writes one more partial, the merge of its
// position lanes): the list cut into equal shares is, per sequence, kDecodeSeqCost
// charge units followed by the sequence's groups, so a share holding a boundary gets
// that many groups fewer.
constexpr int kDecodeSeqCost = 2;

template <int NCH>
struct DecodePartition {
    int incl[NCH];  // P_{s+1} at lane s % 64 of chunk s / 64
    int len[NCH];   // clamped length of sequence s, same places
    int base[NCH];  // first partial slot of sequence s (exclusive prefix sum of the counts)
    int cnt[NCH];   // partials of sequence s: the work-groups its groups fall to
    int total;      // P_S
    int vtotal;     // total + kDecodeSeqCost * S: the length of the charged list
    int nact;       // active work-groups: min(nwg, total)

    // Two steps, so that other loads can be issued between them: load() issues the
    // length loads (all chunks at once), scan() waits for them and forms the sums.
    __device__ __forceinline__ void load(const int32_t* __restrict__ CTX, int S) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int c = 0; c < NCH; ++c) len[c] = CTX[min(64 * c + lane, S - 1)];  // unconditional loads
    }
    __device__ __forceinline__ void scan(int S, int cap, int nwg) {
        const int lane = threadIdx.x & 63;
        int carry = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            len[c] = 64 * c + lane < S ? min(max(len[c], 0), cap) : 0;
            incl[c] = carry + wave_incl_scan((len[c] + 15) / 16);
            carry = __builtin_amdgcn_readlane(incl[c], 63);
        }
        total = wave_uniform(carry);
        vtotal = total + kDecodeSeqCost * S;
        nact = min(nwg, total);
        // partial slots: sequence s owns cnt_s = owner(P_{s+1} - 1) - owner(P_s) + 1 of them
        // (0 when empty), consecutive from base_s; there are at most nact + S - 1 in all
        int carry2 = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int pe = incl[c], ps = pe - (len[c] + 15) / 16;
            cnt[c] = pe > ps ? owner(pe - 1, 64 * c + lane) - owner(ps, 64 * c + lane) + 1 : 0;
            base[c] = carry2 + wave_incl_scan(cnt[c]) - cnt[c];
            carry2 = __builtin_amdgcn_readlane(base[c] + cnt[c], 63);
        }
    }
    // value of a per-sequence register at sequence s (wave-uniform s < 64 * NCH); a
    // cross-lane read, so the whole wave must be active.  Each chunk is read out first
    // and the scalar results selected, so the arrays stay in registers (a select over
    // the array elements themselves becomes an indexed per-lane array that the compiler
    // moves to LDS).
    __device__ __forceinline__ static int at(const int (&v)[NCH], int s) {
        int x = __builtin_amdgcn_readlane(v[0], s & 63);
#pragma unroll
        for (int c = 1; c < NCH; ++c) {
            const int y = __builtin_amdgcn_readlane(v[c], s & 63);
            x = (s >> 6) == c ? y : x;
        }
        return x;
    }
    __device__ __forceinline__ int start(int s) const { return s == 0 ? 0 : at(incl, s - 1); }  // P_s
    __device__ __forceinline__ int end(int s) const { return at(incl, s); }                     // P_{s+1}
    __device__ __forceinline__ int length(int s) const { return at(len, s); }
    __device__ __forceinline__ int first_slot(int s) const { return at(base, s); }
    __device__ __forceinline__ int slots(int s) const { return at(cnt, s); }
    // Group u of sequence s sits at u + kDecodeSeqCost (s + 1) in the charged list, and
    // work-group w takes places [w V / n, (w+1) V / n) of it (V = vtotal): the work-group
    // owning group u of sequence s (total > 0)
    __device__ __forceinline__ int owner(int u, int s) const {
        const int v = u + kDecodeSeqCost * (s + 1);
        if ((int64_t)vtotal * nact < ((int64_t)1 << 31))  // wave-uniform: 32-bit when it cannot overflow
            return (int)(((uint32_t)(v + 1) * (uint32_t)nact - 1u) / (uint32_t)vtotal);
        return (int)((((int64_t)v + 1) * nact - 1) / vtotal);
    }
    // the first group at place v of the charged list or later (total if none): work-group w
    // holds groups [first_group(w V / n), first_group((w+1) V / n)), possibly none
    __device__ __forceinline__ int first_group(int v, int S) const {
        const int lane = threadIdx.x & 63;
        int n = 0;  // sequences whose charged span ends at or before v
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int s = 64 * c + lane;
            n += __popcll(__ballot(s < S && incl[c] + kDecodeSeqCost * (s + 1) <= v));
        }
        if (n >= S) return total;
        return max(start(n), v - kDecodeSeqCost * (n + 1));
    }
    // Writes each sequence's (first group, length, first slot, slot count) to part[s],
    // so that a wave can drop the per-lane arrays and read one record per sequence.
    __device__ __forceinline__ void store(int4* part, int S) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            if (64 * c + lane < S) part[64 * c + lane] = make_int4(incl[c] - (len[c] + 15) / 16, len[c], base[c], cnt[c]);
    }
    // sequences that end at or before group u
    __device__ __forceinline__ int ended_by(int u, int S) const {
        const int lane = threadIdx.x & 63;
        int n = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) n += __popcll(__ballot(64 * c + lane < S && incl[c] <= u));
        return n;
    }
};

// Balanced split path (fewer (sequence, KV head) pairs than CUs).  The 16-position
// groups of all sequences form one list, sequence after sequence (N groups in all);
// work-group w of n = min(nwg, N) takes places [w V / n, (w+1) V / n) of the list with
// kDecodeSeqCost charge units before each sequence's groups (V = N + kDecodeSeqCost S),
// so every work-group streams the same number of K/V bytes to within one group, less
// one group's worth for each sequence start it holds, whatever the mix of context
// lengths.  A range may start or end inside a sequence and may cover
// several: for each sequence it touches the work-group writes one partial (m, l, o) of
// every query head of its KV heads, into slot base_s + (w - owner(first group of s)):
// a sequence's partials are consecutive and there are at most n + S - 1 in all.  The
// work-group owning a sequence's first group records its first slot and slot count
// for the merge.  The waves of a work-group are neighbouring KV heads of the same
// positions, so a page is read contiguously.
template <int D, int DEPTH, int NCH>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(
    const float* __restrict__ Qd, const float* __restrict__ Kp, const float* __restrict__ Vp,
    const int32_t* __restrict__ BT, const int32_t* __restrict__ CTX, float* __restrict__ Po,
    float* __restrict__ Pm, float* __restrict__ Pl, int32_t* __restrict__ Meta, int S, int Hq, int Hkv, int PS,
    int max_pages, int num_pages, int nwg, float c2 /* scale * log2(e) */) {
    using Tr = DecTraits<D>;
    const int w = wave_uniform(threadIdx.x >> 6);
    const int kvh = blockIdx.y * (blockDim.x >> 6) + w;
    if (kvh >= Hkv) return;  // wave-uniform; the kernel has no barrier
    DecodePartition<NCH> pt;
    pt.load(CTX, S);
    pt.scan(S, PS * max_pages, nwg);
    const int wg = blockIdx.x;
    if (wg >= pt.nact) return;
    const int u_lo = wave_uniform(pt.first_group((int)(((int64_t)wg * pt.vtotal) / pt.nact), S));
    const int u_hi = wave_uniform(pt.first_group((int)(((int64_t)(wg + 1) * pt.vtotal) / pt.nact), S));
    if (u_lo >= u_hi) return;  // a share of charge units only
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    const int G = Hq / Hkv;
    for (int s = wave_uniform(pt.ended_by(u_lo, S)); s < S; ++s) {
        const int ps = wave_uniform(pt.start(s)), pe = wave_uniform(pt.end(s));
        if (ps >= u_hi) break;
        const int a = max(ps, u_lo), e = min(pe, u_hi);
        if (a >= e) continue;  // a sequence without positions
        const int ctx = wave_uniform(pt.length(s));
        const int32_t* bt_row = BT + (size_t)s * max_pages;
        int bt = decode_bt_lane(bt_row, max_pages, PS, num_pages, a - ps, 1, min(64, e - a));
        float qf[Tr::KSTEPS];
        decode_load_q<D>(Qd, s, Hq, kvh, G, qf);
        float m = -INFINITY;  // running max of head li (log2 units), same in its four lanes
        float l = 0.f;        // this lane's share of head li's running sum
        f32x4 acc[Tr::NDT];   // O[head 4g + r][d = NDT*li + dt]
#pragma unroll
        for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int j0 = a; j0 < e; j0 += 64) {
            decode_groups<D, DEPTH, 0>(Kp, Vp, bt, Hkv, kvh, PS, ctx, j0 - ps, 1, min(64, e - j0), qf, c2, m, l, acc);
            bt = decode_bt_lane(bt_row, max_pages, PS, num_pages, j0 + 64 - ps, 1, min(64, e - j0 - 64));
        }

        // partial: head h = 4g + r lives in lanes (g, *), register r; head li's l in lanes (*, li)
        const float lt = rows4_sum(l);
        const int k = wg - pt.owner(ps, s);  // this partial's place among the sequence's
        const int first = wave_uniform(pt.first_slot(s));
        const int nslots = wave_uniform(pt.slots(s));  // read with the whole wave active
        if (k == 0 && blockIdx.y == 0 && w == 0 && lane == 0) {  // one writer per sequence
            Meta[2 * s] = first;
            Meta[2 * s + 1] = nslots;
        }
        const size_t slot = (size_t)(first + k);
        const size_t hb = slot * Hq + (size_t)kvh * G;  // row of query head kvh * G
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * g + r;
            if (h < G) {
                float* dst = Po + (hb + h) * D + Tr::NDT * li;
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
            Pm[hb + li] = m;
            Pl[hb + li] = lt;
        }
    }
}

// ---------------------------------------------------------------------------
// Split path for up to 4 query heads per KV head, on the vector ALUs.  A cached
// position costs 4 G D flops for 8 D bytes of K and V, i.e. G / 2 flops per byte:
// at G <= 4 the VALU keeps up with HBM, while a 16x16x4 MFMA tile would pad the G
// heads to 16 columns and spend most of its cycles on zeros.
// Layout (ND = D / 8 lanes per position, NP = min(64 / ND, 16) positions per step, so
// a step stays inside one 16-position group; at D <= 16 the lanes past NP positions
// only shadow the last one):
//   lane = dq + ND * pl owns head dims 4dq .. 4dq+3 and D/2 + 4dq .. D/2 + 4dq+3 of
//   position pl of the step, so each of its two float4 loads covers ND * 16
//   contiguous bytes of a position row together with the other dq lanes;
//   score of head h: 8 FMAs, then a DPP sum over the ND lanes of the position;
//   softmax: every lane keeps its own running max and sum over the positions it
//   sees (pl, pl + NP, ...), so the loop needs no other cross-lane step; the max
//   moves only when a score exceeds it by more than 2^8 (a rare wave-wide branch);
//   O += p V: 8 FMAs per head into the lane's own dims.
// A wave streams its share of the groups as one list, whatever sequences it covers:
// the page, the position in its sequence and the sequence of up to 64 groups are
// resolved at once (lane j <-> group j of the span), and the K/V register ring runs on
// across sequence boundaries.  Where a step starts a new sequence, the finished one's
// position lanes are merged with the log-sum-exp rule and written as one partial per
// query head; the new sequence's queries were loaded when the previous one started.
// So a share that ends one sequence and starts the next pays no restart latency there
// (measured: such shares ended about 2 us after the others when each sequence restarted
// the table and K/V loads).
template <int D, int GM>
struct DecValuTraits {
    static constexpr int ND = D / 8;                        // lanes per position
    static constexpr int NP = 64 / ND < 16 ? 64 / ND : 16;  // positions per step
    static constexpr int SPG = 16 / NP;                     // steps per 16-position group
    // steps in the K/V register ring: one 16-position group (at least two steps);
    // measured at the 32-, 128- and 1024-sequence batches, deeper rings and more waves
    // per CU were slower (the memory system is already saturated by one group ahead)
    static constexpr int DEPTH = SPG > 2 ? SPG : 2;
};
// running max before any position: the lowest finite float, so no inf - inf, and any
// finite score (however negative) is above it and moves it
constexpr float kDecodeNoMax = -3.402823466e38f;

// sum over the ND lanes of a position (the low lane bits)
template <int ND>
__device__ __forceinline__ float sum_dims(float x) {
    if constexpr (ND >= 2) x += dpp_mov<kDppXor1>(x);
    if constexpr (ND >= 4) x += dpp_mov<kDppXor2>(x);
    if constexpr (ND >= 8) x += dpp_mov<kDppHalfMirror>(x);  // the other quad of the half-row
    if constexpr (ND >= 16) x += dpp_mov<kDppRor8>(x);       // the other half of the row
    return x;
}
// sum / max over the position lanes of a wave (the lane bits above the ND lanes)
template <int ND>
__device__ __forceinline__ float sum_positions(float x) {
    if constexpr (ND == 1) return wave_sum(x);
    if constexpr (ND == 2) return rows4_sum(row_stride4_sum(x + dpp_mov<kDppXor2>(x)));
    if constexpr (ND == 4) return rows4_sum(row_stride4_sum(x));
    if constexpr (ND == 8) return rows4_sum(x + dpp_mov<kDppRor8>(x));
    return rows4_sum(x);
}
template <int ND>
__device__ __forceinline__ float max_positions(float x) {
    if constexpr (ND == 1) return wave_max(x);
    if constexpr (ND == 2) return rows4_max(row_stride4_max(fmaxf(x, dpp_mov<kDppXor2>(x))));
    if constexpr (ND == 4) return rows4_max(row_stride4_max(x));
    if constexpr (ND == 8) return rows4_max(fmaxf(x, dpp_mov<kDppRor8>(x)));
    return rows4_max(x);
}

// x of lane l ^ (1 << BIT), for the position bits BIT <= 3 (DPP where an exchange
// pattern exists, else the LDS crossbar); 4 and 5 go through the row-swap permutes.
template <int BIT>
__device__ __forceinline__ float lane_xor(float x) {
    if constexpr (BIT == 0) return dpp_mov<kDppXor1>(x);
    else if constexpr (BIT == 1) return dpp_mov<kDppXor2>(x);
    else if constexpr (BIT == 3) return dpp_mov<kDppRor8>(x);  // rotating a 16-lane row by 8 swaps its halves
    else return __shfl_xor(x, 1 << BIT);
}

// Reduce-scatter over the lane bits BIT .. 5 (the position lanes): on entry v[0 .. N)
// are this lane's addends; each stage pairs lane l with l ^ (1 << bit), and the lane
// whose bit is 0 keeps the sums of the lower half of the list, its partner those of
// the upper half, so the list halves per stage.  On return v[0 .. max(N >> stages, 1))
// hold the sums over all position lanes of entries base .. of the original list; once
// one entry is left the remaining stages add it up whole (lanes then hold duplicates,
// and `dup` has the bits of those stages set in the lanes that are not the first copy).
// Far fewer cross-lane moves than a whole-wave sum per entry: N / 2 + N / 4 + ... instead
// of N per stage.
template <int BIT, int N, int V>
__device__ __forceinline__ void scatter_sum_positions(float (&v)[V], int lane, int& base, int& dup) {
    if constexpr (BIT < 6) {
        if constexpr (N >= 2) {
            constexpr int H = N / 2;
            const bool hi = (lane >> BIT) & 1;
            if constexpr (BIT >= 4) {
#pragma unroll
                for (int j = 0; j < H; ++j) {
                    float a = v[j], b = v[H + j];
                    if constexpr (BIT == 4) swap_rows16(a, b);  // row pairs (0, 1), (2, 3): row 0 gets [a0, a1]
                    else swap_rows32(a, b);                     // half pairs: rows 0-1 get [a0-1, a2-3]
                    v[j] = a + b;
                }
            } else {
#pragma unroll
                for (int j = 0; j < H; ++j) {
                    const float keep = hi ? v[H + j] : v[j];
                    const float send = hi ? v[j] : v[H + j];
                    v[j] = keep + lane_xor<BIT>(send);
                }
            }
            base += hi ? H : 0;
            scatter_sum_positions<BIT + 1, H, V>(v, lane, base, dup);
        } else {
            if constexpr (BIT >= 4) {
                float a, b;
                if constexpr (BIT == 4) pair_xor16(v[0], a, b);
                else pair_xor32(v[0], a, b);
                v[0] = a + b;
            } else {
                v[0] += lane_xor<BIT>(v[0]);
            }
            dup |= lane & (1 << BIT);
            scatter_sum_positions<BIT + 1, 1, V>(v, lane, base, dup);
        }
    }
}

// The split kernel for G <= GM query heads per KV head (GM = 1, 2 or 4): the same
// partition, grid and partial slots as the MFMA split kernel above; each wave keeps
// its copy of the per-sequence records in its own LDS area.
template <int D, int GM, int NCH>
__global__ __launch_bounds__(256) void attn_decode_split_valu_kernel(
    const float* __restrict__ Qd, const float* __restrict__ Kp, const float* __restrict__ Vp,
    const int32_t* __restrict__ BT, const int32_t* __restrict__ CTX, float* __restrict__ Po,
    float* __restrict__ Pm, float* __restrict__ Pl, int32_t* __restrict__ Meta, int S, int Hq, int Hkv, int PS,
    int max_pages, int num_pages, int nwg, float c2 /* scale * log2(e) */) {
    using Tr = DecValuTraits<D, GM>;
    constexpr int ND = Tr::ND, NP = Tr::NP, SPG = Tr::SPG, DEPTH = Tr::DEPTH;
    extern __shared__ int4 dec_seq_info[];  // [waves][64 * NCH]
    const int w = wave_uniform(threadIdx.x >> 6);
    const int kvh = blockIdx.y * (blockDim.x >> 6) + w;
    if (kvh >= Hkv) return;  // wave-uniform; the kernel has no barrier
    int4* part = dec_seq_info + w * 64 * NCH;
    DecodePartition<NCH> pt;
    pt.load(CTX, S);
    pt.scan(S, PS * max_pages, nwg);
    const int wg = blockIdx.x;
    if (wg >= pt.nact) return;
    const int u_lo = wave_uniform(pt.first_group((int)(((int64_t)wg * pt.vtotal) / pt.nact), S));
    const int u_hi = wave_uniform(pt.first_group((int)(((int64_t)(wg + 1) * pt.vtotal) / pt.nact), S));
    if (u_lo >= u_hi) return;  // a share of charge units only
    int s_walk = wave_uniform(pt.ended_by(u_lo, S));  // the sequence of group u_lo
    pt.store(part, S);
    const int lane = threadIdx.x & 63;
    const int dq = lane % ND;
    const int pl = min(lane / ND, NP - 1);  // lanes past NP positions shadow the last one
    const bool lane_on = lane / ND < NP;
    const int G = Hq / Hkv;
    const int ps_log2 = __builtin_ctz(PS);

    // queries of kvh's heads for sequence s, scaled by c2 (zero for h >= G)
    auto load_q = [&](int s, float (&qq)[GM][8]) {
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            const float* qr = Qd + ((size_t)s * Hq + (size_t)kvh * G + min(h, G - 1)) * D + 4 * dq;
            const f32x4 x0 = *(const f32x4*)qr;
            const f32x4 x1 = *(const f32x4*)(qr + D / 2);
            const float f = h < G ? c2 : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qq[h][i] = x0[i] * f;
                qq[h][4 + i] = x1[i] * f;
            }
        }
    };
    float q[GM][8], qn[GM][8];  // the current sequence's queries, and the next one's
    int qseq = s_walk, nseq = -1;
    load_q(s_walk, q);  // before the table loads: the first sequence's queries
    float m[GM], l[GM], acc[GM][8];
    int cur = -1;  // the sequence whose running state m, l, acc hold

    // the finished sequence s: merge the position lanes (M = max m, L = sum 2^(m - M) l,
    // o = sum 2^(m - M) o) and write the share's partial into the sequence's slot.  The
    // maxima and sums go whole-wave (all lanes end equal); the 8 GM output values are
    // reduce-scattered, so each lane ends with a few consecutive dims of one head.
    auto flush = [&](int s) {
        constexpr int V = 8 * GM;      // values per lane: acc[h][i] at 8h + i
        constexpr int LB = __builtin_ctz(ND);  // the lowest position bit of the lane index
        constexpr int KEEP = (V >> (6 - LB)) > 0 ? (V >> (6 - LB)) : 1;  // values left per lane
        float val[V];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            const float M = max_positions<ND>(m[h]);
            const float f = exp2_hw(m[h] - M);  // 0 for a lane that saw no position
            l[h] = sum_positions<ND>(l[h] * f);
#pragma unroll
            for (int i = 0; i < 8; ++i) val[8 * h + i] = acc[h][i] * f;
            m[h] = M;
        }
        int base = 0, dup = 0;
        scatter_sum_positions<LB, V, V>(val, lane, base, dup);
        const int4 info = part[s];
        const int k = wg - pt.owner(wave_uniform(info.x), s);  // this partial's place among the sequence's
        const int first = wave_uniform(info.z);
        const int nslots = wave_uniform(info.w);
        if (k == 0 && blockIdx.y == 0 && w == 0 && lane == 0) {  // one writer per sequence
            Meta[2 * s] = first;
            Meta[2 * s + 1] = nslots;
        }
        const size_t hb = (size_t)(first + k) * Hq + (size_t)kvh * G;  // row of query head kvh * G
        // this lane holds entries base .. base + KEEP - 1: head base / 8, dims i = base % 8 ..
        // (i < 4: 4dq + i, else D/2 + 4dq + i - 4), never across the two halves (KEEP | 8,
        // base a multiple of KEEP)
        const int h = base / 8, i0 = base % 8;
        if (h < G && dup == 0) {
            float* dst = Po + (hb + h) * D + (i0 < 4 ? 4 * dq + i0 : D / 2 + 4 * dq + i0 - 4);
            if constexpr (KEEP == 8) {
                *(f32x4*)dst = f32x4{val[0], val[1], val[2], val[3]};
                *(f32x4*)(dst + D / 2) = f32x4{val[4], val[5], val[6], val[7]};
            } else if constexpr (KEEP == 4) {
                *(f32x4*)dst = f32x4{val[0], val[1], val[2], val[3]};
            } else if constexpr (KEEP == 2) {
                *(f32x2*)dst = f32x2{val[0], val[1]};
            } else {
                dst[0] = val[0];
            }
        }
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) {
            if (hh < G && lane == hh) {
                Pm[hb + hh] = m[hh];
                Pl[hb + hh] = l[hh];
            }
        }
    };

    for (int u0 = u_lo; u0 < u_hi; u0 += 64) {
        const int ng = min(64, u_hi - u0);
        // lane j: group u0 + j of the span (lanes past it repeat its last group), its
        // sequence (the last one starting at or before it; empty ones are passed over),
        // the group's first position in that sequence, the sequence's length and the
        // group's physical page -- clamped to the table row and the pool, so a broken
        // table can give wrong numbers but never an out-of-bounds read
        const int u = u0 + min(lane, ng - 1);
        int sl = s_walk;
        while (sl + 1 < S && part[sl + 1].x <= u) ++sl;
        const int4 info = part[sl];
        const int gp0 = 16 * (u - info.x);
        const int glen = info.y;
        const int page = min(max(BT[(size_t)sl * max_pages + min(gp0 >> ps_log2, max_pages - 1)], 0), num_pages - 1);
        s_walk = wave_uniform(__builtin_amdgcn_readlane(sl, 63));
        const int nsteps = ng * SPG;

        // K/V loads run DEPTH - 1 steps ahead through a register ring and are issued
        // unconditionally (a step past the span re-reads its last one, positions past a
        // sequence's length stay inside their page); such positions score -inf and their
        // V is zeroed, so pool slots past a context may hold anything
        float kr[DEPTH][8], vr[DEPTH][8];
        auto issue = [&](int k, int slot) {
            const int kk = min(k, nsteps - 1);
            const int j = kk / SPG;
            const int pg = __builtin_amdgcn_readlane(page, j);
            const int t = __builtin_amdgcn_readlane(gp0, j) + (kk % SPG) * NP + pl;
            const size_t off = (((size_t)pg * Hkv + kvh) * PS + (t & (PS - 1))) * D + 4 * dq;
            load_vec<4, true>(Kp + off, &kr[slot][0]);
            load_vec<4, true>(Kp + off + D / 2, &kr[slot][4]);
            load_vec<4, true>(Vp + off, &vr[slot][0]);
            load_vec<4, true>(Vp + off + D / 2, &vr[slot][4]);
        };
        auto step = [&](int k, int slot) {
            const bool in = k < nsteps;
            const int j = min(k, nsteps - 1) / SPG;
            const int sj = __builtin_amdgcn_readlane(sl, j);
            if (in && sj != cur) {  // wave-uniform: this step starts sequence sj
                if (cur >= 0) flush(cur);
                if (qseq != sj) {
                    if (nseq == sj) {
#pragma unroll
                        for (int h = 0; h < GM; ++h)
#pragma unroll
                            for (int i = 0; i < 8; ++i) q[h][i] = qn[h][i];
                    } else {
                        load_q(sj, q);
                    }
                    qseq = sj;
                }
                cur = sj;
#pragma unroll
                for (int h = 0; h < GM; ++h) {
                    m[h] = kDecodeNoMax;
                    l[h] = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
                }
                // the queries of the span's next sequence, ahead of its first step
                const uint64_t later = __ballot(lane < ng && sl > sj);
                if (later) {
                    nseq = __builtin_amdgcn_readlane(sl, (int)__builtin_ctzll(later));
                    load_q(nseq, qn);
                }
            }
            const int t = __builtin_amdgcn_readlane(gp0, j) + (k % SPG) * NP + pl;
            const bool valid = in && lane_on && t < __builtin_amdgcn_readlane(glen, j);
            float sc[GM];
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                float x = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) x = fmaf(kr[slot][i], q[h][i], x);
                x = sum_dims<ND>(x);
                sc[h] = valid ? x : -INFINITY;
            }
            bool need = false;
#pragma unroll
            for (int h = 0; h < GM; ++h) need |= sc[h] > m[h] + kLazyRescale;
            if (__ballot(need)) {  // wave-uniform and rare: move the max of every lane to its max seen
#pragma unroll
                for (int h = 0; h < GM; ++h) {
                    const float mn = fmaxf(m[h], sc[h]);
                    const float al = exp2_hw(m[h] - mn);
                    m[h] = mn;
                    l[h] *= al;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[h][i] *= al;
                }
            }
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = valid ? vr[slot][i] : 0.f;
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                const float p = exp2_hw(sc[h] - m[h]);  // 0 for an invalid position
                l[h] += p;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(p, v[i], acc[h][i]);
            }
        };
        // Whole rounds of DEPTH steps, so the loop body has no branch around a step (the
        // steps past the span are fully masked), and a scheduling barrier after each issue,
        // so the loads leave in slot order: the compiler's load-count waits are then per
        // ring slot, the same on loop entry as on the back edge (with the prologue's loads
        // reordered, the entry state forced a wait for every older load into the loop).
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) {
            issue(d, d);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int k0 = 0; k0 < nsteps; k0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                issue(k0 + d + DEPTH - 1, (d + DEPTH - 1) % DEPTH);
                __builtin_amdgcn_sched_barrier(0);
                step(k0 + d, d);
            }
        }
    }
    if (cur >= 0) flush(cur);
}

// One wave per (sequence, query head) merges the sequence's partials with the
// log-sum-exp rule M = max m_c, L = sum 2^(m_c - M) l_c, O = sum 2^(m_c - M) o_c / L,
// 64 partials per pass with a running (M, L, o).  The sequence's first slot and slot
// count come first (one load); then a pass issues all its loads at once: lane c holds
// partial c's (m, l), and the partial rows are read as float4 pieces, D/4 lanes to a
// row, so that 64 rows take 64 / (64 / (D/4)) loads per lane.  Each lane weights its
// rows (the weight of partial c fetched from lane c) and the lanes holding the same
// head-dim piece are summed at the end.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(
    const float* __restrict__ Po, const float* __restrict__ Pm, const float* __restrict__ Pl,
    const int32_t* __restrict__ Meta, float* __restrict__ O, float* __restrict__ LSE, int Hq, int nslots) {
    constexpr int LPR = D / 4;     // lanes per partial row
    constexpr int RPI = 64 / LPR;  // rows per load instruction
    constexpr int NLD = 64 / RPI;  // load instructions per pass of 64 rows
    const int lane = threadIdx.x;
    const int s = blockIdx.x / Hq;
    const int h = blockIdx.x % Hq;
    // clamped to the workspace: a sequence without positions (outside the documented
    // domain) has no writer, and its output is then unspecified but its reads stay in bounds
    const int first = min(max(wave_uniform(Meta[2 * s]), 0), nslots);
    const int n = min(max(wave_uniform(Meta[2 * s + 1]), 0), nslots - first);
    const int rsub = lane / LPR;       // row of this lane within a load instruction
    const int col = (lane % LPR) * 4;  // head-dim piece of this lane
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int cv = min(64, n - c0);  // partials of this pass
        const size_t stat = (size_t)(first + c0 + min(lane, cv - 1)) * Hq + h;
        const float pm_ld = Pm[stat], pl_ld = Pl[stat];  // unconditional loads, masked below
        // only the load instructions that reach a partial of the pass (a sequence usually
        // has a handful: the work-groups its positions fall to)
        f32x4 x[NLD];
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            x[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (j * RPI < cv)  // wave-uniform
                x[j] = *(const f32x4*)(Po + ((size_t)(first + c0 + min(j * RPI + rsub, cv - 1)) * Hq + h) * D + col);
        }
        const bool valid = lane < cv;
        const float pm = valid ? pm_ld : -INFINITY;
        const float m_new = fmaxf(M, wave_max(pm));  // finite: partial c0 exists
        const float keep = exp2_hw(M - m_new);        // 0 on the first pass
        const float wl = valid ? exp2_hw(pm - m_new) : 0.f;
        L = L * keep + wave_sum(valid ? wl * pl_ld : 0.f);
        acc *= keep;
        M = m_new;
#pragma unroll
        for (int j = 0; j < NLD; ++j)
            if (j * RPI < cv) acc += __shfl(wl, j * RPI + rsub) * x[j];  // weight 0 past cv
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
        acc[0] += __shfl_xor(acc[0], off);
        acc[1] += __shfl_xor(acc[1], off);
        acc[2] += __shfl_xor(acc[2], off);
        acc[3] += __shfl_xor(acc[3], off);
    }
    const float inv = 1.f / L;
    if (lane < LPR) *(f32x4*)(O + ((size_t)s * Hq + h) * D + col) = acc * inv;
    if (LSE && lane == 0) LSE[(size_t)s * Hq + h] = (M + log2_hw(L)) * kLn2;
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

    const int mine = w < ngroups ? (ngroups - w + NW - 1) / NW : 0;  // this wave's groups
    const int32_t* bt_row = BT + (size_t)s * max_pages;
    int bt = decode_bt_lane(bt_row, max_pages, PS, num_pages, w, NW, min(64, mine));
    float qf[Tr::KSTEPS];
    decode_load_q<D>(Qd, s, Hq, kvh, G, qf);
    float m = -INFINITY;
    float l = 0.f;
    f32x4 acc[Tr::NDT];
#pragma unroll
    for (int dt = 0; dt < Tr::NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < mine; j0 += 64) {
        decode_groups<D, 2, 0>(Kp, Vp, bt, Hkv, kvh, PS, ctx, w + NW * j0, NW, min(64, mine - j0), qf, c2, m, l, acc);
        bt = decode_bt_lane(bt_row, max_pages, PS, num_pages, w + NW * (j0 + 64), NW, min(64, mine - j0 - 64));
    }

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

bool decode_shape_supported(int64_t D, int64_t page_size, int64_t group) {
    const bool d_ok = D == 8 || D == 16 || D == 32 || D == 64 || D == 128;
    const bool p_ok = page_size == 16 || page_size == 32 || page_size == 64;
    return d_ok && p_ok && group >= 1 && group <= 16;
}

// Workspace (floats): partial slots -- o [slots][Hq][D], then m and l [slots][Hq] -- for
// at most the grid plus the sequences, then each sequence's first slot and slot count
// (2 x S int32).
size_t decode_scratch_floats(int64_t S, int64_t Hq, int64_t D, int64_t slots) {
    return (size_t)(slots * Hq * (D + 2) + 2 * S);
}
int64_t decode_workspace_slots(int64_t S) { return kDecodeMaxWgs + S; }
size_t decode_workspace_floats(int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t max_pages) {
    (void)Hkv;
    (void)page_size;
    (void)max_pages;
    return decode_scratch_floats(S, Hq, D, decode_workspace_slots(S));
}

bool decode_split_supported(int64_t S) { return S <= 64 * kDecodeScanChunks; }

// Work-groups of the split grid on a device with cu_count compute units: kDecodeWaves
// KV heads per work-group (gy work-groups across the KV heads), kDecodeWavesPerCu waves
// per CU in all.
static int decode_split_wgs(int64_t Hkv, int cu_count, int* wpw_out, int* gy_out) {
    const int wpw = (int)std::min<int64_t>(Hkv, kDecodeWaves);
    const int gy = (int)((Hkv + wpw - 1) / wpw);
    if (wpw_out) *wpw_out = wpw;
    if (gy_out) *gy_out = gy;
    return (int)std::max<int64_t>(1, std::min<int64_t>(kDecodeMaxWgs, (int64_t)kDecodeWavesPerCu * cu_count / (wpw * gy)));
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (attn_paged_decode_noalloc): the
// split path's partials live here instead of in a caller workspace.  Every GPU the
// library runs on holds its own copy for the life of the process; calls on one GPU
// share it, so calls that overlap in time on one GPU race.  Host code never uses the
// array's name as an address: it uses the device address that hipGetSymbolAddress
// returns, looked up once per device.
// ---------------------------------------------------------------------------
constexpr size_t kDecodeScratchFloats = ATTN_PAGED_DECODE_NOALLOC_SCRATCH_BYTES / sizeof(float);
static __device__ __align__(256) float scratch[kDecodeScratchFloats];

size_t decode_scratch_capacity_floats() { return kDecodeScratchFloats; }

int64_t decode_scratch_slots(int64_t S, int64_t Hkv, int cu_count) {
    if (!decode_split_supported(S)) return 0;  // the fused path uses no workspace
    return decode_split_wgs(Hkv, cu_count, nullptr, nullptr) + S;
}

constexpr int kScratchDevices = 64;
static std::atomic<float*> g_scratch_addr[kScratchDevices];
static std::mutex g_scratch_mutex;

hipError_t decode_scratch_address(float** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    float* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));  // with device `dev` current
            if (e != hipSuccess) return e;
            if (!addr) return hipErrorInvalidSymbol;
            p = (float*)addr;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}
// measured: the balanced split beats one work-group per (sequence, KV head) from 32 up to
// 256 sequences (e.g. 57.8 vs 71.4 us at 64, 218 vs 246 us at 256 sequences of 512..4096
// positions), so it is used whenever its partition fits

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    if (!decode_split_supported(a.S)) {
        // More sequences than the split's partition holds: one fused work-group per
        // (sequence, KV head).
        hipLaunchKernelGGL((attn_decode_fused_kernel<D>), dim3((unsigned)a.Hkv, (unsigned)a.S),
                           dim3(64 * fused_waves<D>()), 0, stream, a.q, a.k_pool, a.v_pool, a.block_table,
                           a.context_lens, a.o, a.lse, (int)a.Hq, (int)a.Hkv, (int)a.page_size,
                           (int)a.max_pages, (int)a.num_pages, a.scale * kLog2e);
        return hipGetLastError();
    }
    // The positions of all sequences in equal shares over the whole chip, then the merge.
    int wpw = 1, gy = 1;  // waves (KV heads) per work-group, work-groups across the KV heads
    const int nwg = decode_split_wgs(a.Hkv, a.cu_count, &wpw, &gy);
    const int64_t slots = a.slots;  // the split writes at most nwg + S - 1 partials
    if (slots < nwg + a.S) return hipErrorInvalidValue;
    float* Po = a.partial;
    float* Pm = Po + (size_t)(slots * a.Hq * D);
    float* Pl = Pm + (size_t)(slots * a.Hq);
    int32_t* Meta = (int32_t*)(Pl + (size_t)(slots * a.Hq));
    const int64_t G = a.Hq / a.Hkv;
    if (G <= 4) {
        // up to 4 query heads per KV head: the VALU split kernel, instantiated for the
        // smallest head capacity GM >= G and the partition's chunk count.  Measured at
        // 32 sequences it beats the MFMA kernel for G = 1..4 (57.4 vs 68.2 us at G = 4,
        // d = 128; 94.1 vs 100.1 us at G = 1, d = 64; 5 % behind at d = 32) and loses
        // for G = 6..8 (44.7 vs 33.7 us at G = 8, d = 64), where the VALU work per byte
        // has doubled and the MFMA tile is at most half padding.
        const bool one = a.S <= 64;
        const int nch = one ? 1 : kDecodeScanChunks;
        auto pick = [&](auto k1, auto k16) { return one ? k1 : k16; };
        decltype(&attn_decode_split_valu_kernel<D, 1, 1>) valu =
            G == 1   ? pick(attn_decode_split_valu_kernel<D, 1, 1>, attn_decode_split_valu_kernel<D, 1, kDecodeScanChunks>)
            : G == 2 ? pick(attn_decode_split_valu_kernel<D, 2, 1>, attn_decode_split_valu_kernel<D, 2, kDecodeScanChunks>)
                     : pick(attn_decode_split_valu_kernel<D, 4, 1>, attn_decode_split_valu_kernel<D, 4, kDecodeScanChunks>);
        const size_t lds = (size_t)wpw * 64 * nch * sizeof(int4);
        hipLaunchKernelGGL(valu, dim3((unsigned)nwg, (unsigned)gy), dim3(64 * wpw), lds, stream, a.q, a.k_pool,
                           a.v_pool, a.block_table, a.context_lens, Po, Pm, Pl, Meta, (int)a.S, (int)a.Hq,
                           (int)a.Hkv, (int)a.page_size, (int)a.max_pages, (int)a.num_pages, nwg, a.scale * kLog2e);
    } else {
        auto split = a.S <= 64    ? attn_decode_split_kernel<D, kDecodeDepth, 1>
                     : a.S <= 256 ? attn_decode_split_kernel<D, kDecodeDepth, 4>
                                  : attn_decode_split_kernel<D, kDecodeDepth, kDecodeScanChunks>;
        hipLaunchKernelGGL(split, dim3((unsigned)nwg, (unsigned)gy), dim3(64 * wpw), 0, stream, a.q, a.k_pool,
                           a.v_pool, a.block_table, a.context_lens, Po, Pm, Pl, Meta, (int)a.S, (int)a.Hq,
                           (int)a.Hkv, (int)a.page_size, (int)a.max_pages, (int)a.num_pages, nwg, a.scale * kLog2e);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_decode_combine_kernel<D>, dim3((unsigned)(a.S * a.Hq)), dim3(64), 0, stream, Po, Pm, Pl,
                       Meta, a.o, a.lse, (int)a.Hq, (int)slots);
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
