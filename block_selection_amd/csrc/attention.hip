// attention.hip -- stage two: attention over the selected key blocks (gfx950).
//
// Reading note "Block Sparse Attention with Log-Linear Complexity", the two-stage
// formulation it opens with: once stage one has picked K key blocks per query
// (shared by the query heads of a GQA group, section 4.1), the second stage runs
// ordinary attention restricted to the raw key/value rows of the picked blocks.
// Per query head: softmax of
// q.k/sqrt(d) over the keys <= t of the selected blocks, applied to their values.
//
// Layout and arithmetic:
//   * One wavefront per (batch, position, KV head): the group's query heads are the
//     16 columns of every MFMA tile, so each key and value block is read once for
//     the whole group. Logits: v_mfma_f32_16x16x32_bf16 with A = 16 key rows of the
//     block, B = the queries; lane (g, n) holds keys 16 tau + 4g + r of head n.
//   * Online softmax in base 2 per head column (running maximum, rescaled sums);
//     the block holding position t masks its keys after t.
//   * Output O^T = V^T P on the same MFMA: A = 16 dims of V^T, B = P. The 8 keys a
//     lane needs for B are exactly the 8 logits it already holds (keys 32s + 4g + r
//     and 32s + 16 + 4g + r), so P never moves between lanes; V is tiled once per
//     call into per-block [dim][64 keys] tiles whose keys are permuted into that
//     order, so each A fragment is one 16-byte load. P enters as a bf16 hi + lo pair
//     (2^-17 relative), so the products are nearly exact and sums stay in fp32.
#include "walk_math.h"

namespace pisa {

constexpr int kAttnThreads = 256;   // four walks per workgroup

// Key held in slot `slot` (0..63) of a V^T tile row: slots 32s + 8g + r and 32s + 8g + 4 + r
// (r < 4) hold keys 32s + 4g + r and 32s + 16 + 4g + r, so the 8 keys whose logits lane
// group g holds for key half s are contiguous.
__device__ inline int vt_key_of(int slot) {
    const int s = slot >> 5, w5 = slot & 31, g = w5 >> 3, hi = (w5 >> 2) & 1, r = w5 & 3;
    return 32 * s + 16 * hi + 4 * g + r;
}

// p = hi + lo, both bf16 (round to nearest even): a 17-bit mantissa in two MFMA operands.
__device__ inline void split_bf16(float p, uint32_t& hi, uint32_t& lo) {
    hi = rne_bf16_bits(p);
    lo = rne_bf16_bits(p - __uint_as_float(hi << 16));
}

// V [B, cap, Hkv, 64] -> tiles [B*Hkv][nblk][64 dims][64 key slots] (keys >= N are zero).
// Grid: (nblk, B*Hkv), 256 threads. With a pack (pk.cu non-null, B = 1): tile slots of the
// packed layout, block j of document d at slot (cu[d] >> 6) + d + j (nblk slots per KV
// head); a slot that names no block is left unwritten.
__global__ __launch_bounds__(256) void vt_tiles_kernel(const uint16_t* __restrict__ v, Geom G, Pack pk,
                                                       int64_t nblk, uint16_t* __restrict__ vt) {
    __shared__ uint16_t tile[kC][kD + 2];
    const int blk = blockIdx.x, bh = blockIdx.y;
    const int b = bh / G.Hkv, kvh = bh % G.Hkv;
    const int tid = threadIdx.x;
    int64_t row0 = (int64_t)b * G.cap, nkeys = G.N, key0 = (int64_t)blk * kC;   // rows of this tile's sequence
    if (pk.cu) {
        const int d = pack_find_slot(pk, kLog2C, blk);
        const Seg sg = pack_seg(pk, d);
        const int64_t j = blk - ((sg.lsh >> kLog2C) + d);
        if (sg.N == 0 || j < 0 || j * kC >= sg.N) return;
        row0 = sg.tk0;
        nkeys = sg.N;
        key0 = j * kC;
    }
    {
        const int kk = tid >> 2, part = tid & 3;           // key kk, dims 16 part .. +15
        const int64_t key = key0 + kk;
        u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
        if (key < nkeys) {
            const uint16_t* src = v + ((row0 + key) * G.Hkv + kvh) * kD + 16 * part;
            x0 = *reinterpret_cast<const u32x4*>(src);
            x1 = *reinterpret_cast<const u32x4*>(src + 8);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tile[kk][16 * part + 2 * i] = (uint16_t)(x0[i] & 0xffffu);
            tile[kk][16 * part + 2 * i + 1] = (uint16_t)(x0[i] >> 16);
            tile[kk][16 * part + 8 + 2 * i] = (uint16_t)(x1[i] & 0xffffu);
            tile[kk][16 * part + 8 + 2 * i + 1] = (uint16_t)(x1[i] >> 16);
        }
    }
    __syncthreads();
    {
        const int dim = tid >> 2, part = tid & 3;           // dim, slots 16 part .. +15
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s0 = 16 * part + 2 * i;
            const uint32_t lo = tile[vt_key_of(s0)][dim], hi = tile[vt_key_of(s0 + 1)][dim];
            w[i] = lo | (hi << 16);
        }
        uint16_t* dst = vt + (((int64_t)bh * nblk + blk) * kD + dim) * kC + 16 * part;
        *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(dst + 8) = u32x4{w[4], w[5], w[6], w[7]};
    }
}

__device__ inline int64_t uniform_i64(int64_t x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// K fragments of one block: A operand rows = keys 16 tau + n, k-steps dims 8g.. and 32 + 8g..
struct KFrag {
    u32x4 a[4][2];
};

__device__ inline void load_kfrag(const uint16_t* __restrict__ base, int64_t nkeys, int64_t row_stride, int n,
                                  int gq, KFrag& f) {
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
        int64_t key = 16 * tau + n;
        key = (key < nkeys) ? key : nkeys - 1;             // rows past the keys are masked later
        const uint16_t* p = base + key * row_stride;
        f.a[tau][0] = *reinterpret_cast<const u32x4*>(p + 8 * gq);
        f.a[tau][1] = *reinterpret_cast<const u32x4*>(p + 32 + 8 * gq);
    }
}

// One wavefront per walk w = (b * N + t) * Hkv + kvh, four per workgroup. idx: [walks][K]
// selected blocks (entries < 0, or past t's block, are skipped); out: fp32 [B, N, Hq, 64].
// With a pack (pk.cu non-null, B = 1, N = T): row t lies in document d, its position and
// block indices count from cu[d], and its keys, values and tiles are the document's.
__global__ __launch_bounds__(kAttnThreads, 3) void sparse_attention_kernel(const uint16_t* __restrict__ q,
                                                                        const uint16_t* __restrict__ k,
                                                                        const uint16_t* __restrict__ vt,
                                                                        const int32_t* __restrict__ idx, Geom G,
                                                                        Pack pk, int64_t nblk,
                                                                        float* __restrict__ out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gq = lane >> 4, n = lane & 15;
    const int64_t walks = (int64_t)G.B * G.N * G.Hkv;
    const int64_t w = (int64_t)blockIdx.x * (kAttnThreads / 64) + wave;
    if (w >= walks) return;                                // whole wavefronts leave together
    const int kvh = (int)(w % G.Hkv);
    const int64_t bt = w / G.Hkv;
    int64_t b = bt / G.N, t = bt % G.N;                    // sequence and position
    int64_t krow0 = b * G.cap, nkeys = G.N, tile0 = b * G.Hkv * nblk + kvh * nblk;
    if (pk.cu) {
        const int d = pack_find_token(pk, bt);
        const Seg sg = pack_seg(pk, d);
        t = bt - sg.lsh;
        krow0 = sg.tk0;
        nkeys = sg.N;
        tile0 = kvh * nblk + (sg.lsh >> kLog2C) + d;
    }
    // wavefront-uniform: keep them in scalar registers
    t = uniform_i64(t);
    krow0 = uniform_i64(krow0);
    nkeys = uniform_i64(nkeys);
    tile0 = uniform_i64(tile0);
    const int K = G.topk;
    const int64_t row_stride = (int64_t)G.Hkv * kD;
    const uint16_t* kbase = k + (krow0 * G.Hkv + kvh) * kD;   // key r at kbase + r * row_stride
    const uint16_t* vtb = vt + tile0 * (int64_t)(kD * kC);

    // queries: B operand, head n of the group (columns n >= GQ read head 0, not written)
    u32x4 qa, qb;
    {
        const uint16_t* qrow = q + ((bt * G.Hq) + (int64_t)kvh * G.GQ + (n < G.GQ ? n : 0)) * kD;
        qa = *reinterpret_cast<const u32x4*>(qrow + 8 * gq);
        qb = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * gq);
    }
    const bf16x8 q0 = __builtin_bit_cast(bf16x8, qa), q1 = __builtin_bit_cast(bf16x8, qb);

    // the valid selected blocks, in lanes 0 .. nsel-1
    const int64_t tblk = t >> kLog2C;
    int sel = (lane < K) ? idx[w * K + lane] : -1;
    const bool ok = sel >= 0 && sel <= tblk;
    const uint64_t vm = ballot(ok);
    const int nsel = __popcll(vm);
    const int slot = lanes_below(vm);
    sel = push_to_lane(ok ? slot : nsel + lanes_below(~vm), ok ? sel : -1);

    float m = -INFINITY;        // running maximum of column n (base-2 logits)
    float lsum = 0.0f;          // this lane's share of column n's exp sum
    f32x4 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    KFrag cur;   // this block's key fragments; refilled with the next block's once the logits are issued
    if (nsel > 0) {
        const int b0 = readlane_i(sel, 0);
        load_kfrag(kbase + (int64_t)b0 * kC * row_stride, nkeys - (int64_t)b0 * kC, row_stride, n, gq, cur);
    }
    for (int s = 0; s < nsel; ++s) {
        const int blk = readlane_i(sel, s);
        const int64_t k0 = (int64_t)blk * kC;
        // V^T fragments of this block: dims 16 dt + n, slots 32 s2 + 8 gq .. +7
        u32x4 vf[4][2];
        const uint16_t* vblk = vtb + (int64_t)blk * (kD * kC);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                vf[dt][s2] = *reinterpret_cast<const u32x4*>(vblk + (16 * dt + n) * kC + 32 * s2 + 8 * gq);
        // logits
        f32x4 acc[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.a[tau][0]), q0, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.a[tau][1]), q1, c, 0, 0, 0);
            acc[tau] = c;
        }
        if (s + 1 < nsel) {
            const int bn = readlane_i(sel, s + 1);
            load_kfrag(kbase + (int64_t)bn * kC * row_stride, nkeys - (int64_t)bn * kC, row_stride, n, gq, cur);
        }
        // scale to base 2, mask keys after t, block maximum per column
        const int64_t lim = t - k0;                          // keys 0 .. lim of the block are visible
        float mb = -INFINITY;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = acc[tau][r] * kScale2;
                const bool vis = 16 * tau + 4 * gq + r <= lim;
                acc[tau][r] = vis ? x : -INFINITY;
                mb = fmaxf(mb, acc[tau][r]);
            }
        mb = cols4_max(mb);
        const float mn = fmaxf(m, mb);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first block (m = -inf)
        m = mn;
        float ps = 0.0f;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(acc[tau][r] - mn);
                acc[tau][r] = p;
                ps += p;
            }
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[dt][r] *= alpha;
        // O^T += V^T P, P as bf16 hi + lo
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = acc[2 * s2 + (e >> 1)][2 * (e & 1)];
                const float p1 = acc[2 * s2 + (e >> 1)][2 * (e & 1) + 1];
                uint32_t h0, l0, h1, l1;
                split_bf16(p0, h0, l0);
                split_bf16(p1, h1, l1);
                hi[e] = h0 | (h1 << 16);
                lo[e] = l0 | (l1 << 16);
            }
            const bf16x8 bh = __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
            const bf16x8 bl = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, vf[dt][s2]);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, o[dt], 0, 0, 0);
            }
        }
    }
    const float l = cols4_sum(lsum);
    if (n < G.GQ) {
        float* orow = out + ((bt * G.Hq) + (int64_t)kvh * G.GQ + n) * kD;
        const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const f32x4 v4 = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
            *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * gq) = v4;
        }
    }
}

}  // namespace pisa

namespace pisa {

// ------------------------------------------------------------------ decoding step --
// Attention of one decoding query per (batch, KV head) over its selected blocks. A single
// CU gathering all of them is limited by its outstanding requests, so for a few sequences
// the blocks are spread over ceil(K / 4) workgroups of four wavefronts, one block per
// wavefront: the same tiles and online softmax as the prefill kernel, the value block
// staged in the wavefront's own LDS tile in the permuted [dim][key] order. Each workgroup
// merges its four partial states (running maximum, exp sum and unnormalised output per
// head) in LDS and stores one; the last workgroup of a (batch, KV head) to finish (a
// completion counter it resets) merges the stored ones into the output. A larger batch runs
// one workgroup per (batch, KV head), each wavefront taking every fourth block, and writes
// the output from the LDS merge (the device-scope fences of the hand-over cost more than
// the spread saves there).
constexpr int kDecAttnWaves = 4;
constexpr int kDecPartFloats = 2 * kMaxGroup + kMaxGroup * kD;   // m, l, o of one partial state

// Merge n partial states (m[h], l[h], o[h][64] at stride `stride` floats) for head h, dims
// e, e+1: o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i.
template <typename P>
__device__ inline void merge_states(P part, int n, int h, int e, float& o0, float& o1) {
    float M = -INFINITY;
    for (int i = 0; i < n; ++i) M = fmaxf(M, part(i)[h]);
    float den = 0.0f, n0 = 0.0f, n1 = 0.0f;
    for (int i = 0; i < n; ++i) {
        const float mi = part(i)[h];
        const float sc = (mi == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mi - M);
        den += sc * part(i)[kMaxGroup + h];
        n0 += sc * part(i)[2 * kMaxGroup + h * kD + e];
        n1 += sc * part(i)[2 * kMaxGroup + h * kD + e + 1];
    }
    const float inv = (den > 0.0f) ? 1.0f / den : 0.0f;
    o0 = n0 * inv;
    o1 = n1 * inv;
}

// Grid: (ceil(K / 4) or 1, B * Hkv). v_new (may be null): the new token's value row per (batch,
// KV head): key t's value is taken from it, and workgroup 0 writes it to row t of v.
// done: one tagged completion counter per (batch, KV head), any contents (arrive_last); parts:
// [B * Hkv][gridDim.x][kDecPartFloats].
__global__ __launch_bounds__(64 * kDecAttnWaves) void decode_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ v_new, const uint16_t* __restrict__ k,
    uint16_t* __restrict__ v, const int32_t* __restrict__ idx, Geom G, int64_t t, unsigned long long* __restrict__ done,
    uint32_t tag, float* __restrict__ parts, float* __restrict__ out) {
    __shared__ uint16_t s_vt[kDecAttnWaves][kD * kC];       // 8 KiB per wavefront
    __shared__ float s_part[kDecAttnWaves][kDecPartFloats];
    __shared__ int s_last;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gq = lane >> 4, n = lane & 15;
    const int part = blockIdx.x, nparts = gridDim.x;
    const int bh = blockIdx.y, b = bh / G.Hkv, kvh = bh % G.Hkv;
    const int K = G.topk;
    const int64_t row_stride = (int64_t)G.Hkv * kD;
    const uint16_t* kbase = k + ((int64_t)b * G.cap * G.Hkv + kvh) * kD;
    const uint16_t* vbase = v + ((int64_t)b * G.cap * G.Hkv + kvh) * kD;
    const uint16_t* vnew_row = v_new ? v_new + (int64_t)bh * kD : nullptr;
    if (v_new && part == 0 && threadIdx.x < kD)
        v[(((int64_t)b * G.cap + t) * G.Hkv + kvh) * kD + threadIdx.x] = vnew_row[threadIdx.x];
    u32x4 qa, qb;
    {
        const uint16_t* qrow = q + ((int64_t)b * G.Hq + (int64_t)kvh * G.GQ + (n < G.GQ ? n : 0)) * kD;
        qa = *reinterpret_cast<const u32x4*>(qrow + 8 * gq);
        qb = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * gq);
    }
    const bf16x8 q0 = __builtin_bit_cast(bf16x8, qa), q1 = __builtin_bit_cast(bf16x8, qb);
    const int64_t tblk = t >> kLog2C;
    int sel = (lane < K) ? idx[(int64_t)bh * K + lane] : -1;
    const bool ok = sel >= 0 && sel <= tblk;
    const uint64_t vm = ballot(ok);
    const int nsel = __popcll(vm);
    sel = push_to_lane(ok ? lanes_below(vm) : nsel + lanes_below(~vm), ok ? sel : -1);

    float m = -INFINITY, lsum = 0.0f;
    f32x4 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this wavefront's selected blocks: one when the blocks are spread over workgroups
    for (int s = kDecAttnWaves * part + wave; s < nsel; s += kDecAttnWaves * nparts) {
        uint16_t* tile = s_vt[wave];
        // the previous block's tile reads come before this block's tile writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int blk = readlane_i(sel, s);
        const int64_t k0 = (int64_t)blk * kC;
        const int64_t nkeys = G.N - k0;
        // value rows -> this wavefront's LDS tile, [dim][slot of key]; all eight loads in
        // flight together (rows past the keys read the last key and store zeros; key t is
        // read from v_new when given)
        u32x4 vx[8];
        const int dp = lane & 7;                                   // dims 8 dp .. +7
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kk = 8 * i + (lane >> 3);
            const int64_t kr = (kk < nkeys) ? kk : nkeys - 1;
            const uint16_t* row = (vnew_row && k0 + kr == t) ? vnew_row : vbase + (k0 + kr) * row_stride;
            vx[i] = *reinterpret_cast<const u32x4*>(row + 8 * dp);
        }
        KFrag kf;
        load_kfrag(kbase + k0 * row_stride, nkeys, row_stride, n, gq, kf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kk = 8 * i + (lane >> 3);
            const bool in = kk < nkeys;
            const int slot = 32 * (kk >> 5) + 8 * ((kk >> 2) & 3) + 4 * ((kk >> 4) & 1) + (kk & 3);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = in ? vx[i][e] : 0u;
                tile[(8 * dp + 2 * e) * kC + slot] = (uint16_t)(x & 0xffffu);
                tile[(8 * dp + 2 * e + 1) * kC + slot] = (uint16_t)(x >> 16);
            }
        }
        f32x4 acc[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf.a[tau][0]), q0, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf.a[tau][1]), q1, c, 0, 0, 0);
            acc[tau] = c;
        }
        const int64_t lim = t - k0;
        float mb = -INFINITY;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = acc[tau][r] * kScale2;
                acc[tau][r] = (16 * tau + 4 * gq + r <= lim) ? x : -INFINITY;
                mb = fmaxf(mb, acc[tau][r]);
            }
        // online softmax over the wavefront's blocks (the block holding t has a visible key,
        // so the running maximum is finite after the first block)
        const float mn = fmaxf(m, cols4_max(mb));
        const float alpha = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first block (m = -inf)
        m = mn;
        float ps = 0.0f;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(acc[tau][r] - mn);
                acc[tau][r] = p;
                ps += p;
            }
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[dt][r] *= alpha;
        // the tile writes above come from this wavefront only: order them before its reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t h0, l0, h1, l1;
                split_bf16(acc[2 * s2 + (e >> 1)][2 * (e & 1)], h0, l0);
                split_bf16(acc[2 * s2 + (e >> 1)][2 * (e & 1) + 1], h1, l1);
                hi[e] = h0 | (h1 << 16);
                lo[e] = l0 | (l1 << 16);
            }
            const bf16x8 bhi = __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
            const bf16x8 blo = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const u32x4 a = *reinterpret_cast<const lds_u32x4_t*>(
                    (const lds_char_t*)tile + 2 * ((16 * dt + n) * kC + 32 * s2 + 8 * gq));
                const bf16x8 av = __builtin_bit_cast(bf16x8, a);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bhi, o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, blo, o[dt], 0, 0, 0);
            }
        }
    }
    // this wavefront's state (column n = head n), then the workgroup's merged state
    const float l = cols4_sum(lsum);
    float* sp = s_part[wave];
    if (gq == 0) {
        sp[n] = m;
        sp[kMaxGroup + n] = l;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sp[2 * kMaxGroup + n * kD + 16 * dt + 4 * gq + r] = o[dt][r];
    __syncthreads();
    if (nparts == 1) {
        // the workgroup's merged state is the answer: no hand-over between workgroups
        for (int x = threadIdx.x; x < G.GQ * (kD / 2); x += 64 * kDecAttnWaves) {
            const int h = x >> 5, e = 2 * (x & 31);
            float o0, o1;
            merge_states([&](int i) { return (const float*)s_part[i]; }, kDecAttnWaves, h, e, o0, o1);
            float* orow = out + ((int64_t)b * G.Hq + (int64_t)kvh * G.GQ + h) * kD + e;
            orow[0] = o0;
            orow[1] = o1;
        }
        return;
    }
    float* gp = parts + ((int64_t)bh * nparts + part) * kDecPartFloats;
    for (int x = threadIdx.x; x < G.GQ * (kD / 2); x += 64 * kDecAttnWaves) {
        const int h = x >> 5, e = 2 * (x & 31);             // head h, dims e and e + 1
        {
            float M = -INFINITY, den = 0.0f, n0 = 0.0f, n1 = 0.0f;
#pragma unroll
            for (int w = 0; w < kDecAttnWaves; ++w) M = fmaxf(M, s_part[w][h]);
#pragma unroll
            for (int w = 0; w < kDecAttnWaves; ++w) {
                const float mw = s_part[w][h];
                const float sc = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
                den += sc * s_part[w][kMaxGroup + h];
                n0 += sc * s_part[w][2 * kMaxGroup + h * kD + e];
                n1 += sc * s_part[w][2 * kMaxGroup + h * kD + e + 1];
            }
            // stored unnormalised against the workgroup maximum M
            if (e == 0) {
                gp[h] = M;
                gp[kMaxGroup + h] = den;
            }
            gp[2 * kMaxGroup + h * kD + e] = n0;
            gp[2 * kMaxGroup + h * kD + e + 1] = n1;
        }
    }
    __threadfence();   // the state visible device-wide before this workgroup counts itself done
    __syncthreads();
    if (threadIdx.x == 0) s_last = arrive_last(&done[bh], tag, (uint32_t)nparts);
    __syncthreads();
    if (!s_last) return;
    __threadfence();   // acquire: the other workgroups' states
    for (int x = threadIdx.x; x < G.GQ * (kD / 2); x += 64 * kDecAttnWaves) {
        const int h = x >> 5, e = 2 * (x & 31);
        {
            const float* base = parts + (int64_t)bh * nparts * kDecPartFloats;
            float o0, o1;
            merge_states([&](int i) { return base + (int64_t)i * kDecPartFloats; }, nparts, h, e, o0, o1);
            float* orow = out + ((int64_t)b * G.Hq + (int64_t)kvh * G.GQ + h) * kD + e;
            orow[0] = o0;
            orow[1] = o1;
        }
    }
    if (threadIdx.x == 0) done[bh] = 0ull;   // no tag: a replay of this launch starts afresh
}

}  // namespace pisa
