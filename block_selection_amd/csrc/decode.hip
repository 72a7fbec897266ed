// decode.hip -- one decoding step (append, refresh, walk, leaf top-K) in one launch (gfx950).
//
// ai4snews summary, second paragraph: a decoding step refreshes only the new
// token's leaf and its ancestors, then selects. Reading note "Block Sparse
// Attention with Log-Linear Complexity", section 3.2 (the walk from the root,
// keeping all candidates of a level that has at most K of them), "Scoring:
// LogSumExp" and section 4.1 (per-head LSE summed over the GQA group).
//
// P workgroups of 8 wavefronts per (batch, KV head), P = ceil(2K / 8) for a few
// sequences and 1 for a larger batch; the query position is t = N - 1, the appended
// key. Every workgroup
//   1. appends the key and refreshes its leaf and ancestor path (wavefront 0; the
//      copies in the other workgroups write identical bits);
//   2. walks from the root down to level 2: the candidates of a level sit in the
//      2K <= 64 lanes of every wavefront; when there are more than K of them, their
//      children fill up to eight 16-row tiles, one per wavefront (summaries read from
//      the fp32 pyramid and split into hi/lo bf16 planes in registers), the candidate
//      scores go through LDS (double-buffered, so one barrier per level), and every
//      wavefront sorts the 64 slots itself;
//   3. scores the candidate leaves of its slots (8 * part + wavefront, every 8P-th slot
//      after that) from the raw keys in global memory, into a per-(batch, KV head) row
//      of the workspace.
// The last workgroup to finish (a completion counter that it resets) takes the K best
// leaves and writes them ascending, -1 padded. Spreading the leaf stage over several
// CUs matters for one sequence: its random 8 KiB key blocks are fetched far faster by
// several CUs than one CU's outstanding-request capacity allows. For a batch the
// device-scope fences of that hand-over cost more than they save, so P = 1 there.
// The arithmetic is that of the prefill kernels (walk_math.h), so the step selects
// exactly what prefill selects at the same query position.
#include "pyramid_math.h"
#include "walk_math.h"

namespace pisa {

// Leaf scores of NL leaves from raw bf16 keys in global memory (keys > t masked).
template <int NL, int S>
__device__ inline void score_leaves_global(const uint16_t* __restrict__ kbase, int64_t row_stride,
                                           const int (&leaf)[NL], int64_t t, const bf16x8 q0, const bf16x8 q1,
                                           int n, int gq, int GQ, float out[NL]) {
    f32x4 acc[NL][4];
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            // rows past t read row t (their logits are masked), so every load is unconditional
            // and all 8 * NL of them are in flight together
            const int64_t key = (int64_t)leaf[j] * kC + 16 * tau + n;
            const uint16_t* row = kbase + ((key <= t) ? key : t) * row_stride;
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(row + 8 * gq);
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(row + 32 + 8 * gq);
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), q0, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), q1, c, 0, 0, 0);
            acc[j][tau] = c;
        }
    int lim[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int64_t l64 = t - (int64_t)leaf[j] * kC;
        lim[j] = (l64 < kC - 1) ? (int)l64 : kC - 1;
    }
    leaf_scores_from_acc<NL, S>(acc, lim, n, gq, GQ, out);
}

template <int S>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(const uint16_t* __restrict__ q_new,
                                                                     const uint16_t* __restrict__ k_new,
                                                                     uint16_t* __restrict__ k_cache,
                                                                     float* __restrict__ pyr, Geom G,
                                                                     unsigned long long* __restrict__ done,
                                                                     uint32_t tag,
                                                                     float* __restrict__ leaf_score,
                                                                     int32_t* __restrict__ out) {
    __shared__ float s_F[2][64], s_D[2][64], s_P[2][64], s_fix[2][4];
    __shared__ int s_fixslot[2];
    __shared__ int s_last;
    const int part = blockIdx.x, nparts = gridDim.x;   // leaf slots 8*part .. 8*part+7
    const int bh = blockIdx.y, b = bh / G.Hkv, kvh = bh % G.Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int K = G.topk;
    const int64_t t = G.N - 1;
    const int64_t row_stride = (int64_t)G.Hkv * kD;
    uint16_t* kbase = k_cache + ((int64_t)b * G.cap * G.Hkv + kvh) * kD;
    float* pyr_bh = pyr + (int64_t)bh * G.P * kD;

    // MFMA B fragments of query head n of the group (zero columns beyond the group)
    u32x4 qa = {0u, 0u, 0u, 0u}, qb = {0u, 0u, 0u, 0u};
    if (n < G.GQ) {
        const uint16_t* qrow = q_new + ((int64_t)b * G.Hq + (int64_t)kvh * G.GQ + n) * kD;
        qa = *reinterpret_cast<const u32x4*>(qrow + 8 * gq);
        qb = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * gq);
    }
    const bf16x8 q0 = __builtin_bit_cast(bf16x8, qa), q1 = __builtin_bit_cast(bf16x8, qb);

    // Every workgroup of this (batch, KV head) refreshes the path: the copies compute and
    // store identical bits and read only nodes and keys this step does not change.
    if (wave == 0) refresh_wave<uint16_t>(k_new + (int64_t)bh * kD, kbase, row_stride, G, pyr_bh, lane);
    __syncthreads();   // the refreshed path is visible to every wavefront of the workgroup

    // candidate slot = lane; slot 2i + c holds child c of survivor i. A survivor is kept as
    // the low word of its selection key (node and the slot it came from); Pa / Pb hold, in
    // the slot a candidate was scored in, the head-summed logits of its two children.
    // Levels of at most K nodes keep every eligible node unscored: the walk starts at the
    // highest level with more than K nodes (at most 2K), node m in slot m, else at the root.
    int ls = G.L;
    for (int j = G.L; j >= 2; --j) {
        if (G.M[j] > K) {
            ls = j;
            break;
        }
    }
    uint32_t surv_low = 0;
    float Pa = 0.0f, Pb = 0.0f;
    bool pk = false;                 // P of this level's candidates known (scored level above)
    int buf = 0;
    for (int l = ls; l >= 2; --l) {
        int cand;
        float P = 0.0f;
        if (l == ls) {
            cand = (lane < G.M[l] && lane <= (int)(t >> (kLog2C + l - 1))) ? lane : -1;
        } else {
            const uint32_t lowk = (uint32_t)shfl_i((int)surv_low, lane >> 1);
            const int pnode = key_node(lowk);
            const int child = 2 * pnode + (lane & 1);
            const bool ok = lane < 2 * K && pnode >= 0 && child < G.M[l] && child <= (int)(t >> (kLog2C + l - 1));
            cand = ok ? child : -1;
            const int src = key_slot(lowk);
            const float pa = shfl_f(Pa, src), pb = shfl_f(Pb, src);
            P = (lane & 1) ? pb : pa;
        }
        const uint64_t vm = ballot(cand >= 0);
        const int nc = __popcll(vm);
        if (nc <= K) {
            // every candidate survives: compact them into lanes 0 .. nc-1
            const uint32_t low = (cand >= 0) ? (((uint32_t)((1 << 26) - 1 - cand) << 6) | (uint32_t)lane) : 0u;
            const int dst = (cand >= 0) ? lanes_below(vm) : nc + lanes_below(~vm);
            const uint32_t got = (uint32_t)push_to_lane(dst, (int)low);
            surv_low = (lane < nc) ? got : 0u;
            Pa = Pb = 0.0f;
            pk = false;
            continue;
        }
        const int lc = l - 1;
        const int shc = kLog2C + lc - 1;            // first key of a level-lc node i: i << shc
        const int Mc = G.M[lc];
        if (wave < 4) {
            // tile `wave`: MFMA column n = candidate of slot 16 * wave + n
            const int c = shfl_i(cand, 16 * wave + n);
            const int rc = 2 * c + 1;
            const bool rv = c >= 0 && rc < Mc && rc <= (int)(t >> shc);
            const int cc = (c >= 0) ? c : 0;
            const float* prow = pyr_bh + (G.off[l] + cc) * kD;
            const float* crow = pyr_bh + (G.off[lc] + 2 * cc) * kD;
            float vc0[8], vc1[8], vp0[8], vp1[8];
            load8_f32(crow + 8 * gq, vc0);
            load8_f32(crow + 32 + 8 * gq, vc1);
            load8_f32(prow + 8 * gq, vp0);
            load8_f32(prow + 32 + 8 * gq, vp1);
            {
                float d0[8], d1[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    d0[e] = 2.0f * (vc0[e] - vp0[e]);   // doubled delta, as in the prefill planes
                    d1[e] = 2.0f * (vc1[e] - vp1[e]);
                }
                u32x4 h0, l0, h1, l1;
                split8(d0, h0, l0);
                split8(d1, h1, l1);
                const f32x4 acc = summary_tile_mfma(q0, q1, h0, h1, l0, l1);
                float F, D;
                delta_tile_sums<S>(acc, rv, gq, G.GQ, F, D);
                if (gq == 0) {
                    s_F[buf][16 * wave + n] = F;
                    s_D[buf][16 * wave + n] = D;
                }
            }
            if (!pk) {
                // P of the candidates: head sums of the logits of their own summaries
                u32x4 h0, l0, h1, l1;
                split8(vp0, h0, l0);
                split8(vp1, h1, l1);
                const f32x4 acc = summary_tile_mfma(q0, q1, h0, h1, l0, l1);
                const float ps = tile_head_sums(acc);
                if (gq == 0) s_P[buf][16 * wave + n] = ps;
            }
        } else if (wave == 4) {
            // the ragged node of level l (a partial right child), read directly when it is a
            // candidate with an eligible right child
            int fix_slot = -1;
            const int crag = G.M[l] - 1, brag = 2 * crag + 1;
            if (brag < Mc && covered(lc, brag, G.N) < span_of(lc)) {
                const uint64_t rm = ballot(cand == crag && brag <= (int)(t >> shc));
                if (rm) {
                    fix_slot = __builtin_ctzll(rm);
                    const float* row = pyr_bh + (G.off[lc] + ((n == 1) ? brag : brag - 1)) * kD;
                    float v0[8], v1[8];
                    load8_f32(row + 8 * gq, v0);
                    load8_f32(row + 32 + 8 * gq, v1);
                    u32x4 h0, l0, h1, l1;
                    split8(v0, h0, l0);
                    split8(v1, h1, l1);
                    const f32x4 acc = summary_tile_mfma(q0, q1, h0, h1, l0, l1);   // column 0: left, 1: right
                    float xf, xp;
                    ragged_sums<S>(acc, gq, G.GQ, xf, xp);
                    if (lane == 0) {
                        s_fix[buf][0] = xf;
                        s_fix[buf][1] = xp;
                    }
                    if (lane == 1) s_fix[buf][2] = xp;
                }
            }
            if (lane == 0) s_fixslot[buf] = fix_slot;
        }
        __syncthreads();
        if (!pk) P = s_P[buf][lane];
        float score = P + s_F[buf][lane];
        Pa = P + s_D[buf][lane];
        Pb = P - s_D[buf][lane];
        if (lane == s_fixslot[buf]) {
            score = s_fix[buf][0];
            Pa = s_fix[buf][1];
            Pb = s_fix[buf][2];
        }
        buf ^= 1;
        pk = true;
        const uint64_t key = slot_key((cand >= 0) ? score : -INFINITY, cand, lane);
        // the survivors are the K best as a set; with 2K = 64 a partial network finds them
        const uint64_t sorted = (2 * K == 64) ? bitonic_top_half<64, SegmentLanes>(key, lane)
                                              : bitonic_desc<64, SegmentLanes>(key, lane);
        surv_low = (lane < K) ? (uint32_t)sorted : 0u;
    }

    // leaf candidates: children of the level-2 survivors (the root itself if it is a leaf)
    int leaf;
    if (G.L == 1) {
        leaf = (lane == 0) ? 0 : -1;
    } else {
        const int par = key_node((uint32_t)shfl_i((int)surv_low, lane >> 1));
        const int child = 2 * par + (lane & 1);
        const bool ok = lane < 2 * K && par >= 0 && child < G.M[1] && child <= (int)(t >> kLog2C);
        leaf = ok ? child : -1;
    }
    const bool scored = __popcll(ballot(leaf >= 0)) > K;
    if (scored) {
        // this wavefront's leaf slots; each score goes to the per-(batch, KV head) row in
        // the workspace, and the last workgroup to finish reads the whole row
        for (int slot = 8 * part + wave; slot < 2 * K; slot += 8 * nparts) {
            const int f = readlane_i(leaf, slot);
            if (f >= 0) {
                const int fl[1] = {f};
                float o[1];
                score_leaves_global<1, S>(kbase, row_stride, fl, t, q0, q1, n, gq, G.GQ, o);
                if (lane == 0) leaf_score[(int64_t)bh * 64 + slot] = o[0];
            }
        }
        if (nparts > 1) {
            __threadfence();   // scores visible device-wide before this workgroup counts itself done
            __syncthreads();
            if (threadIdx.x == 0) s_last = arrive_last(&done[bh], tag, (uint32_t)nparts);
            __syncthreads();
            if (!s_last) return;
            __threadfence();   // acquire: the other workgroups' scores
        } else {
            __syncthreads();   // one workgroup: its own wavefronts' scores
        }
    } else if (part != 0) {
        return;            // at most K candidates: all kept, workgroup 0 writes them
    }
    if (wave == 0) {
        const float my = (leaf >= 0) ? (scored ? leaf_score[(int64_t)bh * 64 + lane] : 0.0f) : -INFINITY;
        const int lidx = (leaf >= 0) ? leaf : INT_MAX;
        const int nd = (2 * K == 64) ? select_top_half<64>(my, lidx, lane) : select_sort<64>(my, lidx, lane);
        const int keep = index_sort<64>((lane < K) ? nd : INT_MAX, lane);   // ascending, INT_MAX last
        if (lane < K) out[(int64_t)bh * K + lane] = (keep != INT_MAX) ? keep : -1;
        if (scored && lane == 0) done[bh] = 0ull;   // no tag: a replay of this launch starts afresh
    }
}

#define PISA_DECODE_INST(S)                                                                              \
    template __global__ void decode_step_kernel<S>(const uint16_t*, const uint16_t*, uint16_t*, float*, Geom, \
                                                   unsigned long long*, uint32_t, float*, int32_t*);
PISA_DECODE_INST(kScoreLse)
PISA_DECODE_INST(kScoreMean)
PISA_DECODE_INST(kScoreMeanHalfVar)
#undef PISA_DECODE_INST

}  // namespace pisa
