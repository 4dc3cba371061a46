// Incremental decode for gfx950: one new token per (batch, q-head) routed and
// attended against an external key/value cache.
//
// The news page says a deployed decoder must update its routing structures
// as new tokens arrive and coordinate the router with key-value storage
// (section "Learned Routing Faces Dense Attention's Reliability Advantage"),
// and that autoregressive decoding brings frequent incremental updates
// (section "The 99.35 Percent Result Does Not Establish Language Quality");
// the report page keeps the cache outside the mixer contract (section
// "Limits").  Here the cache is the caller's; the index grows block by block
// (the build kernels over a block range and a list rebuild over the indexed
// prefix, which keeps the first `cap` blocks of every list exactly as the
// whole-sequence build does), and each new query takes the route and the
// attention that the whole-sequence path gives its position.
//
// k_decode_step: one workgroup of eight waves per (batch, q-head).  Wave 0
//   routes the new query (the lists of its (batch, kv-head) staged in LDS by
//   the whole workgroup; the arithmetic of the whole-sequence router, so the
//   decisions are bit-identical) while the other waves attend the local
//   blocks, which do not depend on the selection; then every wave attends
//   its share of the selected blocks, in 64-key items with an online
//   softmax, and the eight states are merged through LDS.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "common.hpp"

namespace {

// (score, id) as one unsigned 64-bit key: (score, id) is ordered before
// (score', id') -- score > score', or equal scores and id < id' -- exactly
// when its key is larger.  The score's bits are mapped to an order-preserving
// unsigned integer (-0 taken as +0, as the float comparison does).
__device__ __forceinline__ uint64_t order_key(float sc, int id) {
    const uint32_t u = __float_as_uint(sc + 0.0f);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ int key_id(uint64_t k) {
    return (int)(0xFFFFFFFFu - (uint32_t)k);
}

__device__ __forceinline__ uint64_t key_max(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_key(uint64_t k) {
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)k, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t swap_max(uint64_t k, bool half32) {
    const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
    const auto l2 = half32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                           : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h2 = half32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                           : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const uint64_t a = ((uint64_t)h2[0] << 32) | l2[0];
    const uint64_t b = ((uint64_t)h2[1] << 32) | l2[1];
    return key_max(a, b);
}

// Largest key of the wave, in every lane: lane pairs within quads, then the
// half-row and row mirrors, then the gfx950 row and half-wave swaps (no LDS).
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    k = key_max(k, dpp_key<0xB1>(k));    // quad_perm 1,0,3,2
    k = key_max(k, dpp_key<0x4E>(k));    // quad_perm 2,3,0,1
    k = key_max(k, dpp_key<0x141>(k));   // row_half_mirror
    k = key_max(k, dpp_key<0x140>(k));   // row_mirror
    k = swap_max(k, false);
    return swap_max(k, true);
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t k, int src) {
    const int lo = __shfl((int)(uint32_t)k, src), hi = __shfl((int)(uint32_t)(k >> 32), src);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// The value lane ^ J holds (J a power of two below 64), without the LDS
// crossbar: DPP quad permutes for 1 and 2, a row shift each way for 4 and 8
// (row_shl: lane + J, row_shr: lane - J), the gfx950 swaps for 16 and 32
// (of the returned pair, the even half-row / half-wave gets the partner in
// the second element, the odd one in the first).
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int lane) {
    if constexpr (J == 1) {
        return __builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    } else if constexpr (J == 2) {
        return __builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    } else if constexpr (J == 4 || J == 8) {
        const uint32_t up = __builtin_amdgcn_mov_dpp((int)x, 0x100 + J, 0xF, 0xF, false);
        const uint32_t dn = __builtin_amdgcn_mov_dpp((int)x, 0x110 + J, 0xF, 0xF, false);
        return (lane & J) ? dn : up;
    } else if constexpr (J == 16) {
        const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? a[0] : a[1];
    } else {
        static_assert(J == 32, "lane distance");
        const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? a[0] : a[1];
    }
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t k, int lane) {
    const uint32_t lo = xor_lane<J>((uint32_t)k, lane), hi = xor_lane<J>((uint32_t)(k >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// One bitonic compare-exchange (runs of SIZE, partner distance J), then the
// rest of the network.
template <int SEG, int SIZE, int J>
__device__ __forceinline__ uint64_t bitonic_from(uint64_t k, int i, int lane) {
    const uint64_t o = xor_lane_u64<J>(k, lane);
    // in a descending run the lower lane of a pair keeps the larger key
    const bool keep_max = ((i & J) == 0) == ((i & SIZE) == 0);
    k = keep_max ? key_max(k, o) : (k < o ? k : o);
    if constexpr (J > 1) return bitonic_from<SEG, SIZE, J / 2>(k, i, lane);
    else if constexpr (SIZE < SEG) return bitonic_from<SEG, 2 * SIZE, SIZE>(k, i, lane);
    else return k;
}

// Bitonic sort of one key per lane, largest first, within aligned groups of
// SEG lanes (a power of two <= 64).
template <int SEG>
__device__ __forceinline__ uint64_t sort_desc(uint64_t k, int lane) {
    return bitonic_from<SEG, 2, 1>(k, lane & (SEG - 1), lane);
}

// fp32 fused multiply-add chain over n = N elements in index order, with the
// b operand read from global memory (all loads issued up front).
template <int N>
__device__ __forceinline__ float chain_lds_global(const float *a, const float *__restrict__ bg) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < N; j += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(bg + j);
        acc = fmaf(a[j], v.x, acc);
        acc = fmaf(a[j + 1], v.y, acc);
        acc = fmaf(a[j + 2], v.z, acc);
        acc = fmaf(a[j + 3], v.w, acc);
    }
    return acc;
}

// The router's walk window: M, and per lane the pair (x, y) of code ranks
// it scores (x | y << 8; 0xFFFF for none), the pairs with (x+1)(y+1) <= M,
// x-major.  A per-configuration constant, made on the host.
struct WalkPairs {
    int M;
    unsigned short xy[64];
};

WalkPairs walk_pairs(const Shape &s) {
    WalkPairs w;
    const int A = s.A, K = s.K, np1 = std::min(A, s.npr);
    auto count = [&](int m) {
        int c = 0;
        for (int x = 0; x < std::min(m, K); ++x) c += std::min(m / (x + 1), K);
        return c;
    };
    int M = np1;
    if (s.P == 1) {
        M = std::min(A, np1 + 16);
    } else {
        while (M < std::min(A, np1 + 16) && count(M + 1) <= 64) ++M;
    }
    w.M = M;
    int l = 0;
    for (int x = 0; x < std::min(M, K) && s.P == 2; ++x)
        for (int y = 0; y < std::min(M / (x + 1), K) && l < 64; ++y) w.xy[l++] = (unsigned short)(x | y << 8);
    for (; l < 64; ++l) w.xy[l] = 0xFFFF;
    return w;
}

constexpr int DS_THREADS = 512;   // one workgroup per route
constexpr int DS_WAVES = DS_THREADS / WAVE;

// LDS of one workgroup, in 4-byte words.  Attention part: the scaled rotated
// query [d], per-wave probabilities [W][64], (m, l) [W][2], outputs [W][d],
// back-rotated queries [W][4][d], blocks [L + R].  Route part: the rotated
// query [d], code scores [P K], list offsets [A + 1], entries [NB], pool ids
// [NB], the pool's rerank scores [NB], the addresses whose list holds an
// eligible block [min(A, NB)] (as packed codes), and two counters (those
// addresses, the waves done compacting them).
size_t decode_attend_words(const Shape &s) {
    return (size_t)s.d + (size_t)DS_WAVES * (WAVE + 2 + 5 * s.d) + s.L + s.R;
}
size_t decode_route_words(const Shape &s) {
    const size_t ac = (size_t)std::min(s.A, s.NB);
    return (size_t)s.d + s.P * s.K + (s.A + 1) + 3 * (size_t)s.NB + ac + 2;
}
size_t decode_step_lds(const Shape &s) { return (decode_attend_words(s) + decode_route_words(s)) * 4; }

// DPL consecutive elements starting at i, as floats.
template <bool BF16, int DPL>
__device__ __forceinline__ void load_run(const void *base, size_t i, float (&x)[DPL]) {
    if constexpr (BF16 && DPL == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const u16 *>(base) + i);
        x[0] = __uint_as_float(w << 16);
        x[1] = __uint_as_float(w & 0xFFFF0000u);
    } else if constexpr (!BF16 && DPL == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(base) + i);
        x[0] = v.x;
        x[1] = v.y;
    } else {
#pragma unroll
        for (int j = 0; j < DPL; ++j) x[j] = load1<BF16>(base, i + j);
    }
}

// One workgroup of eight waves per (batch, q-head) route.
//  - Every thread: the rotated query (unscaled for the route, pre-scaled by
//    log2(e)/sqrt(d) for the attention), the (batch, kv-head) list offsets
//    and entries staged in LDS, and the local blocks.
//  - Wave 0 routes (below) while waves 1..7 attend the local blocks, which
//    do not depend on the selection.
//  - After a barrier every wave attends its share of the selected blocks,
//    and the eight online-softmax states are merged through LDS.
// Route (wave 0): code scores are fp32 fused multiply-add chains in dimension
// order, the rotation products rounded before the add: the arithmetic of the
// whole-sequence router, so the decisions are bit-identical.  Addresses are
// visited in (sum desc, address asc) order by repeated wave arg-max over the
// addresses that follow the last one visited; each visited list contributes
// its eligible prefix to the pool until at least n_probes addresses were
// visited and R blocks pooled.  The pool is reranked by the inner product of
// the rotated query with the block summaries and the R best (lower block
// first on ties) are kept in ascending order.
// Attention: the blocks are split in 64-key items; four lanes score one key,
// each wave keeps an online softmax and accumulates P V with the 64 value
// rows of an item loaded back to back.  Keys are rotated relative to their
// item's first position s0 (a rotation by s is the one by s0 followed by the
// one by s - s0): the query rotated back by s0 meets the key rotated by its
// offset in the item, so the keys read only the first 64 rotary rows.
template <int D, int P, bool BF16>
__global__ __launch_bounds__(DS_THREADS) void k_decode_step(
    Shape s, int pos, const void *__restrict__ q, const void *__restrict__ kc,
    const void *__restrict__ vc, const void *__restrict__ krot, const float *__restrict__ cos_t,
    const float *__restrict__ sin_t,
    const float *__restrict__ cb, const float *__restrict__ kbar,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ entries,
    int32_t *__restrict__ sel, void *__restrict__ out, WalkPairs wp) {
    constexpr int H = D / 2, DS = D / P;
    constexpr int DPL = D / WAVE;                 // output dims per lane
    extern __shared__ __align__(16) float dstep_lds[];
    const int R = s.R, K = s.K, A = s.A, NB = s.NB;
    // attention part
    float *qa = dstep_lds;                        // [D] scaled rotated query
    float *pw = qa + D;                           // [W][64] probabilities
    float *ml = pw + DS_WAVES * WAVE;             // [W][2] (m, l)
    float *ow = ml + DS_WAVES * 2;                // [W][D]
    float *qi = ow + DS_WAVES * D;                // [W][4][D] query rotated back by s0 + 16 j
    int *blk = reinterpret_cast<int *>(qi + DS_WAVES * 4 * D);   // [L + R]
    // route part
    float *qr = reinterpret_cast<float *>(blk + s.L + R);    // [D] rotated query
    float *sc = qr + D;                                  // [P K] code scores
    int *off = reinterpret_cast<int *>(sc + P * K);      // [A + 1] list offsets
    int *ent = off + A + 1;                              // [NB] list entries
    int *pool_n = ent + NB;                              // [NB] pooled blocks
    float *pool_r = reinterpret_cast<float *>(pool_n + NB);   // [NB] rerank scores
    int *cand = reinterpret_cast<int *>(pool_r + NB);    // [min(A, NB)] eligible addresses
    int *ccount = cand + min(A, NB);                     // their number
    int *hdone = ccount + 1;                             // waves done compacting them

    // route b * Hq + h.  Workgroups are dealt to the 8 XCDs round-robin
    // (workgroup i is the (i / 8)-th on XCD i % 8); the (batch, kv-head)
    // groups go to the XCDs in turn and the G heads of a group run on one
    // XCD, so the blocks they share (the local ones, and the selected ones
    // they have in common) come from memory once into that XCD's L2.  With
    // a group count that is not a multiple of 8 the routes run in order.
    const int ngq = s.B * s.Hkv;
    const int route = ngq % 8 == 0
        ? ((int)(blockIdx.x / 8) / s.G * 8 + (int)(blockIdx.x % 8)) * s.G + (int)(blockIdx.x / 8) % s.G
        : (int)blockIdx.x;
    const int b = route / s.Hq, h = route % s.Hq, g = h / s.G;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
    const uint64_t lanemask = (1ull << lane) - 1ull;
    int32_t *out_sel = sel + (size_t)route * R;
    const int qb = pos / s.beta;
    const int E = max(0, qb - s.L + 1);
    const bool search = E > R;
    const size_t u = (size_t)b * s.Hkv + g;
    const size_t qoff = (size_t)route * D;
    const int lo = max(0, qb - s.L + 1);
    const int nloc = qb - lo + 1;
    const int per_blk = s.beta / WAVE;
    const int nloc_items = nloc * per_blk;
    const int nitems = (nloc + R) * per_blk;

    // wave 0's codebook rows (codes lane and lane + 64), in flight during
    // the set-up below
    float4 crow[2][DS / 4];
    if (wave == 0 && search) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int x = lane + k * WAVE;
            const int xc = x < P * K ? x : 0;             // in bounds; unused past P K
            const float4 *cr = reinterpret_cast<const float4 *>(
                cb + (((size_t)g * P + xc / K) * K + xc % K) * DS);
            if (k == 0 || (P == 2 && P * K > WAVE)) {
#pragma unroll
                for (int j = 0; j < DS / 4; ++j) crow[k][j] = cr[j];
            }
        }
    }
    // rotated query (fp32, products rounded before the add)
    const float scale = 1.4426950408889634f / sqrtf((float)D);
    for (int i = tid; i < H; i += DS_THREADS) {
        const float a = load1<BF16>(q, qoff + i), bb = load1<BF16>(q, qoff + i + H);
        const float c = cos_t[(size_t)pos * H + i], sn = sin_t[(size_t)pos * H + i];
        const float ac = a * c, bs = bb * sn, bc = bb * c, as = a * sn;
        const float r0 = ac - bs, r1 = bc + as;
        qr[i] = r0;
        qr[i + H] = r1;
        qa[i] = r0 * scale;
        qa[i + H] = r1 * scale;
    }
    // list offsets and entries, four loads in flight per thread
    if (search) {
        const int32_t *og = offsets + u * (A + 1), *eg = entries + u * NB;
        const int n_off = A + 1, n_all = A + 1 + NB;
        for (int b0 = 0; b0 < n_all; b0 += 4 * DS_THREADS) {
            int v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = min(b0 + k * DS_THREADS + tid, n_all - 1);
                v[k] = i < n_off ? og[i] : eg[i - n_off];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = b0 + k * DS_THREADS + tid;
                if (i < n_all) off[i] = v[k];   // ent follows off in LDS
            }
        }
    }
    for (int j = tid; j < nloc; j += DS_THREADS) blk[j] = lo + j;
    if (tid == 0) {
        *ccount = 0;
        *hdone = 0;
    }
    __syncthreads();

    // ---- attention state of this wave, and one 64-key item
    float m = -INFINITY, l = 0.0f;
    float o[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] = 0.0f;
    const size_t rs = (size_t)s.Hkv * D;          // cache row stride (elements)
    const size_t base = ((size_t)b * s.T * s.Hkv + g) * D;
    float *p_s = pw + wave * WAVE;
    float *q_i = qi + wave * 4 * D;
    // QK: four lanes per key (lane quad kq = lane / 4 takes key 16 j + kq of
    // an item in sub-pass j), each lane a quarter of the rotation pairs.  The
    // key at s0 + 16 j + kq is rotated by kq here (the lane's rotary rows,
    // loaded once) and the query back by s0 + 16 j.
    constexpr int PPL = H / 4;                    // rotation pairs per lane
    constexpr int NI = PPL / 4;                   // their groups of four
    const int part = lane & 3, kq = lane >> 2;
    // back-rotation of the query: lane takes sub-pass jq = lane / 16 and
    // pairs QPL (lane % 16) .. QPL (lane % 16) + QPL - 1
    constexpr int QPL = H / 16;
    const int jq = lane >> 4, pq = (lane & 15) * QPL;
    // bf16: every sub-pass's key words are loaded before the values
    constexpr int KJ = BF16 ? 4 : 1;
    // pre-rotated keys: lane part takes dims part D/4 .. part D/4 + D/4 - 1 of
    // its key (bf16: NW 16-byte words)
    constexpr int NW = D / 32;
    auto attend_item = [&](int it, auto rotated) {
        constexpr bool ROT = decltype(rotated)::value;
        const int bk = blk[it / per_blk];
        if (bk < 0) return;
        const int s0 = bk * s.beta + (it % per_blk) * WAVE;
        if (s0 > pos) return;
        // key row of sub-pass j for this lane (keys past pos read row pos)
        auto krow = [&](int j) { return base + (size_t)min(s0 + 16 * j + kq, pos) * rs + part * PPL; };
        auto krow_r = [&](int j) { return base + (size_t)min(s0 + 16 * j + kq, pos) * rs + part * (D / 4); };
        // loads in the order they are waited for: the rotary rows (the
        // lane's keys' offsets kq, the query's s0 + 16 jq), the keys, then
        // the values
        float rc[ROT ? 1 : PPL], rsn[ROT ? 1 : PPL];
        float cq[QPL], sq[QPL];
        uint2 ku0[ROT ? 1 : KJ][NI], ku1[ROT ? 1 : KJ][NI];
        u32x4 kw[ROT && BF16 ? 4 : 1][NW];
        if constexpr (ROT) {
            if constexpr (BF16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4 *kr = reinterpret_cast<const u32x4 *>(
                        reinterpret_cast<const u16 *>(krot) + krow_r(j));
#pragma unroll
                    for (int w = 0; w < NW; ++w) kw[j][w] = kr[w];
                }
            }
        } else {
#pragma unroll
        for (int n = 0; n < NI; ++n) {
            const float4 c4 = *reinterpret_cast<const float4 *>(cos_t + (size_t)kq * H + part * PPL + 4 * n);
            const float4 s4 = *reinterpret_cast<const float4 *>(sin_t + (size_t)kq * H + part * PPL + 4 * n);
            rc[4 * n] = c4.x; rc[4 * n + 1] = c4.y; rc[4 * n + 2] = c4.z; rc[4 * n + 3] = c4.w;
            rsn[4 * n] = s4.x; rsn[4 * n + 1] = s4.y; rsn[4 * n + 2] = s4.z; rsn[4 * n + 3] = s4.w;
        }
        {
            const size_t row = (size_t)min(s0 + 16 * jq, s.T - 1) * H + pq;   // unused past pos
#pragma unroll
            for (int e = 0; e < QPL; ++e) {
                cq[e] = cos_t[row + e];
                sq[e] = sin_t[row + e];
            }
        }
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u16 *kr = reinterpret_cast<const u16 *>(kc) + krow(j);
#pragma unroll
                for (int n = 0; n < NI; ++n) {
                    ku0[j][n] = *reinterpret_cast<const uint2 *>(kr + 4 * n);
                    ku1[j][n] = *reinterpret_cast<const uint2 *>(kr + 4 * n + H);
                }
            }
        }
        }
        // the item's value rows (this lane's dims); rows past pos read row
        // pos (p = 0 there)
        const int klast = pos - s0;
        constexpr int RW = BF16 ? 1 : DPL;        // 32-bit words of raw values per key
        uint32_t vr[WAVE][RW];
#pragma unroll
        for (int kk = 0; kk < WAVE; ++kk) {
            const size_t vo = base + (size_t)(s0 + min(kk, klast)) * rs + DPL * lane;
            if constexpr (BF16 && DPL == 2) {
                vr[kk][0] = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const u16 *>(vc) + vo);
            } else if constexpr (BF16) {
                vr[kk][0] = reinterpret_cast<const u16 *>(vc)[vo];
            } else {
#pragma unroll
                for (int j = 0; j < DPL; ++j)
                    vr[kk][j] = __float_as_uint(reinterpret_cast<const float *>(vc)[vo + j]);
            }
        }
        if constexpr (!ROT) {
            // the query rotated back by s0 + 16 jq: (x c + y s, y c - x s)
#pragma unroll
            for (int e = 0; e < QPL; ++e) {
                const float x = qa[pq + e], y = qa[pq + e + H];
                q_i[jq * D + pq + e] = x * cq[e] + y * sq[e];
                q_i[jq * D + pq + e + H] = y * cq[e] - x * sq[e];
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0): q_i written
            __builtin_amdgcn_wave_barrier();
        }
        float lg[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = s0 + 16 * j + kq;
            const float *qj = q_i + j * D + part * PPL;
            float acc = 0.0f;
            if constexpr (ROT && BF16) {
                // pre-rotated bf16 keys, unpacked; fp32 fused multiply-adds
                const float *qd = qa + part * (D / 4);
#pragma unroll
                for (int w = 0; w < NW; ++w) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t kp = kw[j][w][e];
                        acc = fmaf(qd[8 * w + 2 * e], __uint_as_float(kp << 16), acc);
                        acc = fmaf(qd[8 * w + 2 * e + 1], __uint_as_float(kp & 0xFFFF0000u), acc);
                    }
                }
            } else if constexpr (ROT) {
                const float4 *kr = reinterpret_cast<const float4 *>(
                    reinterpret_cast<const float *>(krot) + krow_r(j));
                const float *qd = qa + part * (D / 4);
#pragma unroll
                for (int w = 0; w < D / 16; ++w) {
                    const float4 k4 = kr[w];
                    acc = fmaf(qd[4 * w], k4.x, acc);
                    acc = fmaf(qd[4 * w + 1], k4.y, acc);
                    acc = fmaf(qd[4 * w + 2], k4.z, acc);
                    acc = fmaf(qd[4 * w + 3], k4.w, acc);
                }
            } else {
#pragma unroll
            for (int n = 0; n < NI; ++n) {
                float x0[4], x1[4];
                if constexpr (BF16) {
                    const uint2 u0 = ku0[j][n], u1 = ku1[j][n];
                    x0[0] = __uint_as_float(u0.x << 16); x0[1] = __uint_as_float(u0.x & 0xFFFF0000u);
                    x0[2] = __uint_as_float(u0.y << 16); x0[3] = __uint_as_float(u0.y & 0xFFFF0000u);
                    x1[0] = __uint_as_float(u1.x << 16); x1[1] = __uint_as_float(u1.x & 0xFFFF0000u);
                    x1[2] = __uint_as_float(u1.y << 16); x1[3] = __uint_as_float(u1.y & 0xFFFF0000u);
                } else {
                    const float *kr = reinterpret_cast<const float *>(kc) + krow(j);
                    const float4 f0 = *reinterpret_cast<const float4 *>(kr + 4 * n);
                    const float4 f1 = *reinterpret_cast<const float4 *>(kr + 4 * n + H);
                    x0[0] = f0.x; x0[1] = f0.y; x0[2] = f0.z; x0[3] = f0.w;
                    x1[0] = f1.x; x1[1] = f1.y; x1[2] = f1.z; x1[3] = f1.w;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float cc = rc[4 * n + e], ss = rsn[4 * n + e];
                    const float k0 = x0[e] * cc - x1[e] * ss;
                    const float k1 = x1[e] * cc + x0[e] * ss;
                    acc = fmaf(qj[4 * n + e], k0, acc);
                    acc = fmaf(qj[4 * n + e + H], k1, acc);
                }
            }
            }
            // sum over the lane quad
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xF, 0xF, false));
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xF, 0xF, false));
            lg[j] = key <= pos ? acc : -INFINITY;
        }
        float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
#pragma unroll
        for (int o2 = 32; o2 > 2; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
        const float mnew = fmaxf(m, mx);          // finite: key s0 <= pos is valid
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // exp2(-inf) = 0
        float ps = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p = __builtin_amdgcn_exp2f(lg[j] - mnew);   // 0 past pos
            ps += p;
            if (part == 0) p_s[16 * j + kq] = p;
        }
#pragma unroll
        for (int o2 = 32; o2 > 2; o2 >>= 1) ps += __shfl_xor(ps, o2);
        l = l * alpha + ps;
        m = mnew;
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[j] *= alpha;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int kk = 0; kk < WAVE; ++kk) {
            const float pk = p_s[kk];
            float x[DPL];
            if constexpr (BF16 && DPL == 2) {
                x[0] = __uint_as_float(vr[kk][0] << 16);
                x[1] = __uint_as_float(vr[kk][0] & 0xFFFF0000u);
            } else if constexpr (BF16) {
                x[0] = __uint_as_float(vr[kk][0] << 16);
            } else {
#pragma unroll
                for (int j = 0; j < DPL; ++j) x[j] = __uint_as_float(vr[kk][j]);
            }
#pragma unroll
            for (int j = 0; j < DPL; ++j) o[j] = fmaf(pk, x[j], o[j]);
        }
        __builtin_amdgcn_wave_barrier();
    };

    int *blk_rem = blk + nloc;                    // [R] the selection, for the attention
    // The addresses whose list holds an eligible block (its first entry, the
    // smallest, at most last), as codes c0 | c1 << 16 in cand, in no set
    // order: the walk past its first M addresses visits only those (below).
    // They do not depend on the query, so the waves without a local block
    // collect them while wave 0 scores and sorts (addresses first + lane,
    // step stride); with no such wave, wave 0 collects them when it needs them.
    const int last = qb - s.L;
    const int nhelp = max(0, DS_WAVES - 1 - nloc_items);
    auto compact = [&](int first, int stride) {
        const int AC = min(A, NB);
        int c0 = P == 1 ? first + lane : (first + lane) / K, c1 = P == 1 ? 0 : (first + lane) % K;
        const int s0 = P == 1 ? stride : stride / K, s1 = P == 1 ? 0 : stride % K;
        constexpr int CB = 4;                     // steps whose reads are in flight together
        for (int a0 = first; a0 < A; a0 += CB * stride) {
            int e0[CB], e1[CB], f[CB], cc[CB];
#pragma unroll
            for (int v = 0; v < CB; ++v) {
                const int ac = min(a0 + v * stride + lane, A - 1);
                e0[v] = off[ac];
                e1[v] = off[ac + 1];
                cc[v] = c0 | c1 << 16;
                c0 += s0;
                c1 += s1;
                if (P == 2 && c1 >= K) { c1 -= K; ++c0; }
            }
#pragma unroll
            for (int v = 0; v < CB; ++v) f[v] = e0[v] < e1[v] ? ent[e0[v]] : INT_MAX;
#pragma unroll
            for (int v = 0; v < CB; ++v) {
                const bool ok = a0 + v * stride + lane < A && f[v] <= last;
                const uint64_t msk = __ballot(ok);
                if (msk) {
                    int at = 0;
                    if (lane == 0) at = atomicAdd(ccount, __popcll(msk));
                    at = __builtin_amdgcn_readlane(at, 0) + __popcll(msk & lanemask);
                    if (ok && at < AC) cand[at] = cc[v];   // a valid index has at most AC such lists
                }
            }
        }
    };
    if (wave == 0) {
        if (!search) {   // bypass: every eligible block, in order
            for (int r = lane; r < R; r += WAVE) {
                const int id = r < E ? r : -1;
                out_sel[r] = id;
                blk_rem[r] = id;
            }
        } else {
            // code scores: fma chains in dimension order
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int x = lane + k * WAVE;
                if ((k == 0 || (P == 2 && P * K > WAVE)) && x < P * K) {
                    const float *qp = qr + (x / K) * DS;
                    float acc = 0.0f;
#pragma unroll
                    for (int j = 0; j < DS / 4; ++j) {
                        acc = fmaf(qp[4 * j], crow[k][j].x, acc);
                        acc = fmaf(qp[4 * j + 1], crow[k][j].y, acc);
                        acc = fmaf(qp[4 * j + 2], crow[k][j].z, acc);
                        acc = fmaf(qp[4 * j + 3], crow[k][j].w, acc);
                    }
                    sc[x] = acc;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            int npool = 0;
            // the eligible prefix of list a joins the pool
            auto take = [&](int a) {
                const int e0 = off[a], e1 = off[a + 1];
                for (int e = e0; e < e1; e += WAVE) {
                    const int n = e + lane < e1 ? ent[e + lane] : INT_MAX;
                    const bool ok = n <= last;
                    const uint64_t msk = __ballot(ok);
                    const int slot = npool + __popcll(msk & lanemask);
                    if (ok && slot < NB) pool_n[slot] = n;   // a valid index holds <= NB blocks
                    npool = min(NB, npool + __popcll(msk));
                    if (msk != ~0ull) break;   // a later block ends the prefix
                }
            };
            // Lists a_0, a_1, ... (lane r holds a_r, or a < 0 for none) taken
            // in that order at once: each lane finds its list's eligible
            // prefix by binary search (entries ascend), a wave scan places
            // the prefixes, and with stop_at > 0 only the lists up to the
            // first at which stop_at blocks were collected are taken (the
            // walk's stopping rule); then the wave copies them.
            auto take_lists = [&](int a, int stop_at) {
                // lists are in lanes 0..15 (n_probes <= 16, and R <= 16 when
                // the search runs): a DPP scan within that row
                int e0 = 0, cnt = 0;
                if (a >= 0) {
                    e0 = off[a];
                    int lo2 = e0, hi2 = off[a + 1];
                    while (lo2 < hi2) {
                        const int mid = (lo2 + hi2) >> 1;
                        if (ent[mid] <= last) lo2 = mid + 1;
                        else hi2 = mid;
                    }
                    cnt = lo2 - e0;
                }
                int incl = cnt;   // row_shr:1, 2, 4, 8 with zeros from outside the row
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);
                int nl = 16;                         // lists taken
                if (stop_at > 0) {
                    const uint64_t reach = __ballot(lane < 16 && incl >= stop_at);
                    if (reach) nl = __ffsll((long long)reach);   // through the first that reaches it
                }
                const int excl = incl - cnt;
                uint64_t todo = __ballot(lane < nl && cnt > 0);
                while (todo) {
                    const int r = __ffsll((long long)todo) - 1;
                    todo &= todo - 1;
                    const int cr = __builtin_amdgcn_readlane(cnt, r);
                    const int er = __builtin_amdgcn_readlane(e0, r);
                    const int pr = npool + __builtin_amdgcn_readlane(excl, r);
                    for (int x = lane; x < cr; x += WAVE)
                        if (pr + x < NB) pool_n[pr + x] = ent[er + x];   // a valid index holds <= NB blocks
                }
                npool = min(NB, npool + __builtin_amdgcn_readlane(incl, nl - 1));
            };
            // address sum, component 0 first (mixed radix, component 0 most significant)
            auto sigma = [&](int c0, int c1) { return P == 1 ? sc[c0] : sc[c0] + sc[K + c1]; };
            // The walk over addresses in (sum desc, address asc) order stops at
            // the first address at which at least n_probes were visited and R
            // blocks pooled.  Phase 1 visits the n_probes best addresses.  An
            // address of codes ranked x and y in their components (score desc,
            // code asc) has (x+1)(y+1)-1 addresses before it in walk order, so
            // the n_probes best are among the pairs with (x+1)(y+1) <= n_probes
            // (at most 50 for 16 probes): the codes of each component are
            // sorted (one wave sort), then those pairs, and the first n_probes
            // are the walk's.
            const int np1 = min(A, s.npr);
            // The sort gives the walk's first M >= np1 addresses in order: for
            // P = 2 the largest M (at most np1 + 16) whose pairs fit the wave
            // (19 for 8 probes; every pair rule above holds for M as for
            // n_probes), for P = 1 every code (wp, made on the host).
            const int M = wp.M;
            uint64_t wk;                             // lane r: key of the r-th visited address
            if constexpr (P == 1) {
                wk = sort_desc<64>(lane < K ? order_key(sc[lane], lane) : 0ull, lane);
            } else {
                uint64_t k0, k1;                     // sorted codes of components 0 and 1
                if (K <= 32) {
                    const int c = lane & 31, p = lane >> 5;
                    const uint64_t ks = sort_desc<32>(c < K ? order_key(sc[p * K + c], c) : 0ull, lane);
                    k0 = ks;                         // lanes 0..31: component 0
                    k1 = xor_lane_u64<32>(ks, lane);  // lanes 0..31: component 1
                } else {
                    k0 = sort_desc<64>(lane < K ? order_key(sc[lane], lane) : 0ull, lane);
                    k1 = sort_desc<64>(lane < K ? order_key(sc[K + lane], lane) : 0ull, lane);
                }
                // lane -> its pair (x, y), x-major
                const int xy = wp.xy[lane];
                const int px = xy == 0xFFFF ? -1 : (xy & 0xFF), py = xy == 0xFFFF ? 0 : xy >> 8;
                const uint64_t kx = shfl_u64(k0, max(px, 0)), ky = shfl_u64(k1, py);
                const int c0 = key_id(kx), c1 = key_id(ky);
                const bool ok = px >= 0 && kx != 0ull && ky != 0ull;
                const uint64_t pk = ok ? order_key(sigma(c0, c1), c0 * K + c1) : 0ull;
                // the pairs fill lanes 0 .. npairs-1: sort only those
                const int npairs = WAVE - __popcll(__ballot(px < 0));
                wk = npairs <= 32 ? sort_desc<32>(pk, lane) : sort_desc<64>(pk, lane);
            }
            take_lists(lane < np1 ? key_id(wk) : -1, 0);
            uint64_t prev = shfl_u64(wk, np1 - 1);         // key of the last visited address
            const int npool1 = npool;
            const float *kb = kbar + u * (size_t)NB * D;
            // the summary rows of the first 64 pooled blocks (their first 64
            // dimensions at d = 128), in flight during the extension (lanes
            // without a block read row 0)
            constexpr bool PREFETCH = BF16 || D == 64;
            constexpr int KPW = PREFETCH ? 16 : 1;
            float4 kpre[KPW];
            if constexpr (PREFETCH) {
                const float4 *kr = reinterpret_cast<const float4 *>(
                    kb + (size_t)(lane < npool1 ? pool_n[lane] : 0) * D);
#pragma unroll
                for (int j = 0; j < KPW; ++j) kpre[j] = kr[j];
            }
            // Phase 2 begins with the walk's next addresses, ranks np1 .. M-1,
            // already in order: their lists are taken up to the one that
            // brings the pool to R.  Past rank M only addresses whose list
            // has an eligible block can change the pool or end the walk; they
            // are walked alone (at most R more picks, each by a wave arg-max
            // over the collected addresses the walk has not visited).
            if (npool < R && np1 < M) {
                const int nx = M - np1;
                // every lane takes part in the exchange (a lane exchange reads 0
                // from a lane that is not active in it)
                const uint64_t kn = shfl_u64(wk, min(lane + np1, WAVE - 1));
                take_lists(lane < nx ? key_id(kn) : -1, R - npool);
                prev = shfl_u64(wk, M - 1);
            }
            if (npool < R && M < A) {
                if (nhelp == 0) {
                    compact(0, WAVE);
                } else {
                    // the helper waves end their compaction without waiting
                    // on anything, so this wait ends
                    while (__hip_atomic_load(hdone, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < nhelp)
                        __builtin_amdgcn_s_sleep(1);
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);
                __builtin_amdgcn_wave_barrier();
                const int ncand = min(*ccount, min(A, NB));
                // candidate x's key, or 0 for an address the walk has visited
                auto cand_key = [&](int x) {
                    const int cc = cand[x], c0 = cc & 0xFFFF, c1 = cc >> 16;
                    const uint64_t k = order_key(sigma(c0, c1), P == 1 ? c0 : c0 * K + c1);
                    return k < prev ? k : 0ull;
                };
                // rounds: with at most NKR candidates per lane their keys stay
                // in registers (a taken key is cleared; keys are distinct)
                constexpr int NKR = 8;
                if (ncand <= NKR * WAVE) {
                    uint64_t ck[NKR];
#pragma unroll
                    for (int t = 0; t < NKR; ++t) {
                        const int x = lane + t * WAVE;
                        ck[t] = x < ncand ? cand_key(x) : 0ull;
                    }
                    // every candidate list holds an eligible block, so the
                    // walk ends within the R - npool best: pick them in
                    // order (lane r keeps the r-th), then take them at once
                    const int need = R - npool;
                    uint64_t mine = 0;
                    for (int r = 0; r < need; ++r) {
                        uint64_t best = 0;
#pragma unroll
                        for (int t = 0; t < NKR; ++t) best = key_max(best, ck[t]);
                        best = wave_max_key(best);
                        if (best == 0) break;                // every list picked
#pragma unroll
                        for (int t = 0; t < NKR; ++t) ck[t] = ck[t] == best ? 0ull : ck[t];
                        if (lane == r) mine = best;
                    }
                    take_lists(mine ? key_id(mine) : -1, need);
                } else {
                    uint64_t pv = prev;
                    while (npool < R) {
                        uint64_t best = 0;
                        for (int x = lane; x < ncand; x += WAVE) {
                            const uint64_t k = cand_key(x);
                            if (k < pv) best = key_max(best, k);
                        }
                        best = wave_max_key(best);
                        if (best == 0) break;                // every list taken
                        pv = best;
                        take(key_id(best));
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            // rerank: fma chain over every dimension of q_rot . kbar_n
            for (int x = lane; x < npool; x += WAVE) {
                float acc;
                if (PREFETCH && x == lane && lane < npool1) {
                    const float4 *kr = reinterpret_cast<const float4 *>(kb + (size_t)pool_n[x] * D);
                    constexpr int NR = D / 4 - KPW > 0 ? D / 4 - KPW : 1;
                    float4 rest[NR];
#pragma unroll
                    for (int j = KPW; j < D / 4; ++j) rest[j - KPW] = kr[j];
                    acc = 0.0f;
#pragma unroll
                    for (int j = 0; j < D / 4; ++j) {
                        const float4 kv = j < KPW ? kpre[j] : rest[j - KPW];
                        acc = fmaf(qr[4 * j], kv.x, acc);
                        acc = fmaf(qr[4 * j + 1], kv.y, acc);
                        acc = fmaf(qr[4 * j + 2], kv.z, acc);
                        acc = fmaf(qr[4 * j + 3], kv.w, acc);
                    }
                } else {
                    acc = chain_lds_global<D>(qr, kb + (size_t)pool_n[x] * D);
                }
                pool_r[x] = acc;
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            // the R best in (score desc, block asc) order; lane r keeps pick r
            // (R <= 16 whenever the search runs): one wave sort when the pool
            // fits the wave, else R rounds of arg-max
            const int nsel = min(R, npool);
            int mine = -1;
            if (npool <= WAVE) {
                const uint64_t k0 = lane < npool ? order_key(pool_r[lane], pool_n[lane]) : 0ull;
                const uint64_t k = npool <= 16 ? sort_desc<16>(k0, lane)
                                   : npool <= 32 ? sort_desc<32>(k0, lane) : sort_desc<64>(k0, lane);
                if (lane < nsel) mine = key_id(k);
            } else {
                uint64_t pprev = ~0ull;
                for (int r = 0; r < nsel; ++r) {
                    uint64_t best = 0;
                    for (int x = lane; x < npool; x += WAVE) {
                        const uint64_t k = order_key(pool_r[x], pool_n[x]);
                        if (k < pprev) best = key_max(best, k);
                    }
                    best = wave_max_key(best);
                    pprev = best;
                    if (r == lane) mine = key_id(best);
                }
            }
            // ascending: a pick's slot is the number of smaller picks
            int rank = 0;
            for (int r = 0; r < nsel; ++r) {
                const int other = __shfl(mine, r);
                rank += other < mine ? 1 : 0;
            }
            if (lane < nsel) {
                out_sel[rank] = mine;
                blk_rem[rank] = mine;   // distinct and eligible: pooled blocks are
            }
            for (int r = nsel + lane; r < R; r += WAVE) {
                out_sel[r] = -1;
                blk_rem[r] = -1;
            }
        }
    } else if (wave - 1 < nloc_items) {
        // the local blocks, while wave 0 routes
        for (int it = wave - 1; it < nloc_items; it += DS_WAVES - 1)
            attend_item(it, std::false_type{});
    } else if (search) {
        compact((wave - 1 - nloc_items) * WAVE, nhelp * WAVE);
        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): its candidates written
        if (lane == 0) __hip_atomic_fetch_add(hdone, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    // the selected blocks, on every wave
    // (covered by the index, so pre-rotated when it holds rotated keys)
    for (int it = nloc_items + wave; it < nitems; it += DS_WAVES) {
        if (krot) attend_item(it, std::true_type{});
        else attend_item(it, std::false_type{});
    }

    // merge the waves' states
    if (lane == 0) {
        ml[2 * wave] = m;
        ml[2 * wave + 1] = l;
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) ow[wave * D + DPL * lane + j] = o[j];
    __syncthreads();
    if (wave == 0) {
        float M = -INFINITY;
        for (int w = 0; w < DS_WAVES; ++w) M = fmaxf(M, ml[2 * w]);
        float lt = 0.0f, acc[DPL];
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] = 0.0f;
        for (int w = 0; w < DS_WAVES; ++w) {
            const float mw = ml[2 * w];
            if (mw == -INFINITY) continue;        // a wave with no item
            const float f = __builtin_amdgcn_exp2f(mw - M);
            lt += f * ml[2 * w + 1];
#pragma unroll
            for (int j = 0; j < DPL; ++j) acc[j] += f * ow[w * D + DPL * lane + j];
        }
        const float inv = 1.0f / lt;
#pragma unroll
        for (int j = 0; j < DPL; ++j) store1<BF16>(out, qoff + DPL * lane + j, acc[j] * inv);
    }
}

template <typename F>
hipError_t lds_at_least(F *fn, size_t bytes) {
    return mono_lds_limit(reinterpret_cast<const void *>(fn), bytes);
}

template <int D, bool BF16>
hipError_t run_decode(const Shape &s, int pos, const void *q, const void *kc, const void *vc,
                      const void *krot, const float *cos_t, const float *sin_t, const float *cb,
                      const float *kbar,
                      const int32_t *offsets, const int32_t *entries, int32_t *sel, void *out,
                      hipStream_t st) {
    const unsigned routes = (unsigned)(s.B * s.Hq);
    const size_t lds = decode_step_lds(s);
    auto *fn = s.P == 1 ? k_decode_step<D, 1, BF16> : k_decode_step<D, 2, BF16>;
    const hipError_t e = lds_at_least(fn, lds);
    if (e != hipSuccess) return e;
    fn<<<routes, DS_THREADS, lds, st>>>(s, pos, q, kc, vc, krot, cos_t, sin_t, cb, kbar, offsets,
                                        entries, sel, out, walk_pairs(s));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Shape &s, int pos, const void *q, const void *kc, const void *vc,
                         const void *krot, const float *cos_t, const float *sin_t, const float *cb,
                         const float *kbar, const int32_t *offsets, const int32_t *entries,
                         int32_t *sel, void *out, hipStream_t st) {
    const bool bf = s.dtype == 1;
    if (s.d == 64)
        return bf ? run_decode<64, true>(s, pos, q, kc, vc, krot, cos_t, sin_t, cb, kbar, offsets,
                                         entries, sel, out, st)
                  : run_decode<64, false>(s, pos, q, kc, vc, krot, cos_t, sin_t, cb, kbar, offsets,
                                          entries, sel, out, st);
    return bf ? run_decode<128, true>(s, pos, q, kc, vc, krot, cos_t, sin_t, cb, kbar, offsets,
                                      entries, sel, out, st)
              : run_decode<128, false>(s, pos, q, kc, vc, krot, cos_t, sin_t, cb, kbar, offsets,
                                       entries, sel, out, st);
}
