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
// k_decode_route: one wave per route.  The (batch, kv-head) list offsets and
//   entries are staged in LDS once.  The rotated query and its code scores go
//   to LDS (fp32, fused multiply-add chains in dimension order,
//   rotation products rounded before the add: the same arithmetic as the
//   whole-sequence router, so the decisions are bit-identical); address sums
//   are kept per lane.  Addresses are visited in (sum desc, address asc)
//   order by repeated wave arg-max over the addresses that follow the last
//   one visited; each visited list contributes its eligible prefix to the
//   pool until at least n_probes addresses were visited and R blocks pooled.
//   The pool is reranked by the inner product of the rotated query with the
//   block summaries and the R best (lower block first on ties) are emitted
//   in ascending order.
// k_decode_attend: one workgroup per (batch, q-head).  The local blocks and
//   the valid, first-occurrence selected blocks are split in 64-key items
//   over eight waves; four lanes score one key, each wave keeps an online
//   softmax and accumulates P V with the 64 value rows of an item loaded back
//   to back, and the eight states are merged through LDS.  Keys are rotated
//   relative to their item's first position s0: a rotation by s is the
//   rotation by s0 followed by the one by s - s0, so the score is the query
//   rotated back by s0 against the key rotated by its offset in the item.
//   The query's back-rotation is done once per item; the keys then read
//   only the first 64 rows of the rotary table, which stay in the caches,
//   instead of one row per key.
#include <algorithm>
#include <climits>

#include "common.hpp"

namespace {

constexpr int DR_THREADS = WAVE;   // one wave per route

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

size_t decode_route_lds(const Shape &s) {
    // q_rot, code scores, address sums, list offsets, entries, pool ids, pool
    // scores, extension addresses
    return (size_t)(s.d + s.P * s.K + s.A + (s.A + 1) + s.NB + 2 * s.NB + std::min(s.A, s.NB)) * 4;
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

// Stage n ints from global to LDS, up to SI loads in flight per lane.
constexpr int SI = 24;
__device__ __forceinline__ void stage_ints(int *dst, const int32_t *__restrict__ src, int n,
                                           int lane) {
    for (int b0 = 0; b0 < n; b0 += SI * WAVE) {
        int v[SI];
#pragma unroll
        for (int k = 0; k < SI; ++k) {
            const int i = b0 + k * WAVE + lane;
            v[k] = i < n ? src[i] : 0;
        }
#pragma unroll
        for (int k = 0; k < SI; ++k) {
            const int i = b0 + k * WAVE + lane;
            if (i < n) dst[i] = v[k];
        }
    }
}

template <int D, int P, bool BF16>
__global__ __launch_bounds__(DR_THREADS) void k_decode_route(
    Shape s, int pos, const void *__restrict__ q, const float *__restrict__ cos_t,
    const float *__restrict__ sin_t, const float *__restrict__ cb, const float *__restrict__ kbar,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ entries,
    int32_t *__restrict__ sel) {
    constexpr int H = D / 2, DS = D / P;
    extern __shared__ __align__(16) float dr_lds[];
    const int R = s.R, K = s.K, A = s.A, NB = s.NB;
    float *qr = dr_lds;                                  // [D] rotated query
    float *sc = qr + D;                                  // [P K] code scores
    float *sig = sc + P * K;                             // [A] address sums
    int *off = reinterpret_cast<int *>(sig + A);         // [A + 1] list offsets
    int *ent = off + A + 1;                              // [NB] list entries
    int *pool_n = ent + NB;                              // [NB] pooled blocks
    float *pool_r = reinterpret_cast<float *>(pool_n + NB);   // [NB] their rerank scores
    int *cand = reinterpret_cast<int *>(pool_r + NB);    // [min(A, NB)] extension addresses

    const int route = blockIdx.x;                        // b * Hq + h
    const int b = route / s.Hq, h = route % s.Hq, g = h / s.G;
    const int lane = threadIdx.x;
    const uint64_t lanemask = (1ull << lane) - 1ull;
    int32_t *out = sel + (size_t)route * R;
    const int qb = pos / s.beta;
    const int E = max(0, qb - s.L + 1);
    if (E <= R) {   // bypass: every eligible block, in order
        for (int r = lane; r < R; r += WAVE) out[r] = r < E ? r : -1;
        return;
    }
    const size_t u = (size_t)b * s.Hkv + g;
    // Every load that does not depend on another goes out first: this lane's
    // query pair(s) and rotary values, its codebook row(s) (codes lane and
    // lane + 64), then the (batch, kv-head) lists staged into LDS.
    const size_t qoff = (size_t)route * D;
    constexpr int QP = (H + WAVE - 1) / WAVE;            // query pairs per lane
    float qa[QP], qb2[QP], qc[QP], qs[QP];
#pragma unroll
    for (int k = 0; k < QP; ++k) {
        const int i = lane + k * WAVE;
        const bool ok = i < H;
        qa[k] = ok ? load1<BF16>(q, qoff + i) : 0.0f;
        qb2[k] = ok ? load1<BF16>(q, qoff + i + H) : 0.0f;
        qc[k] = ok ? cos_t[(size_t)pos * H + i] : 0.0f;
        qs[k] = ok ? sin_t[(size_t)pos * H + i] : 0.0f;
    }
    float4 crow[2][DS / 4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int x = lane + k * WAVE;
        const int xc = x < P * K ? x : 0;                 // in bounds; unused past P K
        const float4 *cr = reinterpret_cast<const float4 *>(
            cb + (((size_t)g * P + xc / K) * K + xc % K) * DS);
        if (k == 0 || (P == 2 && P * K > WAVE)) {
#pragma unroll
            for (int j = 0; j < DS / 4; ++j) crow[k][j] = cr[j];
        }
    }
    stage_ints(off, offsets + u * (A + 1), A + 1, lane);
    stage_ints(ent, entries + u * NB, NB, lane);
    // rotate (fp32, products rounded before the add)
#pragma unroll
    for (int k = 0; k < QP; ++k) {
        const int i = lane + k * WAVE;
        if (i < H) {
            const float ac = qa[k] * qc[k], bs = qb2[k] * qs[k];
            const float bc = qb2[k] * qc[k], as = qa[k] * qs[k];
            qr[i] = ac - bs;
            qr[i + H] = bc + as;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
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
    // address sums, component 0 first (mixed radix, component 0 most significant)
    for (int a = lane; a < A; a += WAVE) sig[a] = P == 1 ? sc[a] : sc[a / K] + sc[K + a % K];
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();

    const int last = qb - s.L;
    int npool = 0;
    // the eligible prefix of list a joins the pool
    auto take = [&](int a) {
        const int e0 = off[a], e1 = off[a + 1];
        for (int e = e0; e < e1; e += WAVE) {
            const int n = e + lane < e1 ? ent[e + lane] : INT_MAX;
            const bool ok = n <= last;
            const uint64_t m = __ballot(ok);
            const int slot = npool + __popcll(m & lanemask);
            if (ok && slot < NB) pool_n[slot] = n;   // a valid index holds <= NB blocks
            npool = min(NB, npool + __popcll(m));
            if (m != ~0ull) break;   // a later block ends the prefix
        }
    };
    // The walk over addresses in (sum desc, address asc) order stops at the
    // first address at which at least n_probes were visited and R blocks
    // pooled.  Phase 1 visits the n_probes best addresses; after them only
    // addresses whose list has an eligible block can change the pool or end
    // the walk, so phase 2 walks those alone (at most R more rounds).
    uint64_t prev = ~0ull;                               // key of the last visited address
    const int np1 = min(A, s.npr);
    for (int r = 0; r < np1; ++r) {
        uint64_t best = 0;
        for (int a = lane; a < A; a += WAVE) {
            const uint64_t k = order_key(sig[a], a);
            if (k < prev) best = key_max(best, k);
        }
        best = wave_max_key(best);
        prev = best;
        take(key_id(best));
    }
    if (npool < R && np1 < A) {
        // addresses after the last visited one whose list starts with an eligible block
        int ncand = 0;
        for (int a0 = 0; a0 < A; a0 += WAVE) {
            const int a = a0 + lane;
            bool ok = false;
            if (a < A) {
                const int e0 = off[a];
                ok = e0 < off[a + 1] && ent[e0] <= last && order_key(sig[a], a) < prev;
            }
            const uint64_t m = __ballot(ok);
            if (ok) cand[ncand + __popcll(m & lanemask)] = a;
            ncand += __popcll(m);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        while (npool < R) {
            uint64_t best = 0;
            for (int x = lane; x < ncand; x += WAVE) {
                const int a = cand[x];
                const uint64_t k = order_key(sig[a], a);
                if (k < prev) best = key_max(best, k);
            }
            best = wave_max_key(best);
            if (best == 0) break;                        // every list taken
            prev = best;
            take(key_id(best));
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // rerank: fma chain over every dimension of q_rot . kbar_n
    const float *kb = kbar + u * (size_t)NB * D;
    for (int x = lane; x < npool; x += WAVE)
        pool_r[x] = chain_lds_global<D>(qr, kb + (size_t)pool_n[x] * D);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // the R best in (score desc, block asc) order; lane r keeps pick r
    // (R <= 16 whenever the search runs)
    const int nsel = min(R, npool);
    uint64_t pprev = ~0ull;
    int mine = -1;
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
    // ascending: a pick's slot is the number of smaller picks
    int rank = 0;
    for (int r = 0; r < nsel; ++r) {
        const int other = __shfl(mine, r);
        rank += other < mine ? 1 : 0;
    }
    if (lane < nsel) out[rank] = mine;
    for (int r = nsel + lane; r < R; r += WAVE) out[r] = -1;
}

constexpr int DA_THREADS = 512;
constexpr int DA_WAVES = DA_THREADS / WAVE;

size_t decode_attend_lds(const Shape &s) {
    return (size_t)(s.d + DA_WAVES * (WAVE + 2 + 2 * s.d)) * 4 + (size_t)(s.R + s.L) * 4;
}

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

// One workgroup per (batch, q-head), 8 waves.  Logits in base 2: q is
// pre-scaled by log2(e)/sqrt(d).  Lane l owns output dims DPL l .. DPL l + DPL-1.
template <int D, bool BF16>
__global__ __launch_bounds__(DA_THREADS) void k_decode_attend(
    Shape s, int pos, const void *__restrict__ q, const void *__restrict__ kc,
    const void *__restrict__ vc, const float *__restrict__ cos_t, const float *__restrict__ sin_t,
    const int32_t *__restrict__ sel, void *__restrict__ out) {
    constexpr int H = D / 2;
    constexpr int DPL = D / WAVE;                 // output dims per lane
    extern __shared__ __align__(16) float da_lds[];
    float *qr = da_lds;                           // [D]
    float *pw = qr + D;                           // [DA_WAVES][WAVE] probabilities
    float *ml = pw + DA_WAVES * WAVE;             // [DA_WAVES][2] (m, l)
    float *ow = ml + DA_WAVES * 2;                // [DA_WAVES][D]
    float *qi = ow + DA_WAVES * D;                // [DA_WAVES][D] query rotated back by s0
    int *blk = reinterpret_cast<int *>(qi + DA_WAVES * D);   // [L + R]

    const int route = blockIdx.x;
    const int b = route / s.Hq, h = route % s.Hq, g = h / s.G;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
    const int qb = pos / s.beta, R = s.R;
    const int lo = max(0, qb - s.L + 1);
    const int nloc = qb - lo + 1;
    const float scale = 1.4426950408889634f / sqrtf((float)D);
    const size_t qoff = (size_t)route * D;
    for (int i = tid; i < H; i += DA_THREADS) {
        const float a = load1<BF16>(q, qoff + i), bb = load1<BF16>(q, qoff + i + H);
        const float c = cos_t[(size_t)pos * H + i], sn = sin_t[(size_t)pos * H + i];
        qr[i] = (a * c - bb * sn) * scale;
        qr[i + H] = (bb * c + a * sn) * scale;
    }
    // blocks: the local ones, then the valid first occurrences of the selection
    const int32_t *row = sel + (size_t)route * R;
    for (int j = tid; j < nloc; j += DA_THREADS) blk[j] = lo + j;
    for (int r = tid; r < R; r += DA_THREADS) {
        const int id = row[r];
        bool ok = id >= 0 && id <= qb - s.L;
        for (int r2 = 0; ok && r2 < r; ++r2) ok = row[r2] != id;
        blk[nloc + r] = ok ? id : -1;
    }
    __syncthreads();

    const int per_blk = s.beta / WAVE;
    const int nitems = (nloc + R) * per_blk;
    float m = -INFINITY, l = 0.0f;
    float o[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] = 0.0f;
    const size_t rs = (size_t)s.Hkv * D;          // cache row stride (elements)
    const size_t base = ((size_t)b * s.T * s.Hkv + g) * D;
    float *p_s = pw + wave * WAVE;
    float *q_i = qi + wave * D;
    // QK: four lanes per key (lane quad kq = lane / 4 takes key 16 j + kq in
    // sub-pass j), each lane a quarter of the rotation pairs
    constexpr int PPL = H / 4;                    // rotation pairs per lane
    const int part = lane & 3, kq = lane >> 2;
    for (int it = wave; it < nitems; it += DA_WAVES) {
        const int bk = blk[it / per_blk];
        if (bk < 0) continue;
        const int s0 = bk * s.beta + (it % per_blk) * WAVE;
        if (s0 > pos) continue;
        // the query rotated back by s0 (pair i in lane i): (x c + y s, y c - x s)
        for (int i = lane; i < H; i += WAVE) {
            const float x = qr[i], y = qr[i + H];
            const float c = cos_t[(size_t)s0 * H + i], sn = sin_t[(size_t)s0 * H + i];
            q_i[i] = x * c + y * sn;
            q_i[i + H] = y * c - x * sn;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        // the item's value rows (this lane's dims), issued with the keys so
        // that one wait covers both; rows past pos read row pos (p = 0 there)
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
        float lg[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = s0 + 16 * j + kq;
            float acc = 0.0f;
            if (key <= pos) {
                const size_t ko = base + (size_t)key * rs + part * PPL;
                // rotation by the key's offset in the item
                const float *cr = cos_t + (size_t)(16 * j + kq) * H + part * PPL;
                const float *sr = sin_t + (size_t)(16 * j + kq) * H + part * PPL;
#pragma unroll
                for (int i = 0; i < PPL; i += 4) {
                    float x0[4], x1[4];
                    if constexpr (BF16) {
                        const uint2 u0 = *reinterpret_cast<const uint2 *>(
                            reinterpret_cast<const u16 *>(kc) + ko + i);
                        const uint2 u1 = *reinterpret_cast<const uint2 *>(
                            reinterpret_cast<const u16 *>(kc) + ko + i + H);
                        x0[0] = __uint_as_float(u0.x << 16); x0[1] = __uint_as_float(u0.x & 0xFFFF0000u);
                        x0[2] = __uint_as_float(u0.y << 16); x0[3] = __uint_as_float(u0.y & 0xFFFF0000u);
                        x1[0] = __uint_as_float(u1.x << 16); x1[1] = __uint_as_float(u1.x & 0xFFFF0000u);
                        x1[2] = __uint_as_float(u1.y << 16); x1[3] = __uint_as_float(u1.y & 0xFFFF0000u);
                    } else {
                        const float4 f0 = *reinterpret_cast<const float4 *>(
                            reinterpret_cast<const float *>(kc) + ko + i);
                        const float4 f1 = *reinterpret_cast<const float4 *>(
                            reinterpret_cast<const float *>(kc) + ko + i + H);
                        x0[0] = f0.x; x0[1] = f0.y; x0[2] = f0.z; x0[3] = f0.w;
                        x1[0] = f1.x; x1[1] = f1.y; x1[2] = f1.z; x1[3] = f1.w;
                    }
                    const float4 c4 = *reinterpret_cast<const float4 *>(cr + i);
                    const float4 s4 = *reinterpret_cast<const float4 *>(sr + i);
                    const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, ss[4] = {s4.x, s4.y, s4.z, s4.w};
                    const int i0 = part * PPL + i;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float k0 = x0[e] * cc[e] - x1[e] * ss[e];
                        const float k1 = x1[e] * cc[e] + x0[e] * ss[e];
                        acc = fmaf(q_i[i0 + e], k0, acc);
                        acc = fmaf(q_i[i0 + e + H], k1, acc);
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
        for (int w = 0; w < DA_WAVES; ++w) M = fmaxf(M, ml[2 * w]);
        float lt = 0.0f, acc[DPL];
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] = 0.0f;
        for (int w = 0; w < DA_WAVES; ++w) {
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
                      const float *cos_t, const float *sin_t, const float *cb, const float *kbar,
                      const int32_t *offsets, const int32_t *entries, int32_t *sel, void *out,
                      hipStream_t st) {
    const unsigned routes = (unsigned)(s.B * s.Hq);
    const size_t lr = decode_route_lds(s);
    hipError_t e;
    if (s.P == 1) {
        e = lds_at_least(k_decode_route<D, 1, BF16>, lr);
        if (e != hipSuccess) return e;
        k_decode_route<D, 1, BF16><<<routes, DR_THREADS, lr, st>>>(s, pos, q, cos_t, sin_t, cb,
                                                                   kbar, offsets, entries, sel);
    } else {
        e = lds_at_least(k_decode_route<D, 2, BF16>, lr);
        if (e != hipSuccess) return e;
        k_decode_route<D, 2, BF16><<<routes, DR_THREADS, lr, st>>>(s, pos, q, cos_t, sin_t, cb,
                                                                   kbar, offsets, entries, sel);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t la = decode_attend_lds(s);
    e = lds_at_least(k_decode_attend<D, BF16>, la);
    if (e != hipSuccess) return e;
    k_decode_attend<D, BF16><<<routes, DA_THREADS, la, st>>>(s, pos, q, kc, vc, cos_t, sin_t, sel,
                                                             out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Shape &s, int pos, const void *q, const void *kc, const void *vc,
                         const float *cos_t, const float *sin_t, const float *cb,
                         const float *kbar, const int32_t *offsets, const int32_t *entries,
                         int32_t *sel, void *out, hipStream_t st) {
    const bool bf = s.dtype == 1;
    if (s.d == 64)
        return bf ? run_decode<64, true>(s, pos, q, kc, vc, cos_t, sin_t, cb, kbar, offsets,
                                         entries, sel, out, st)
                  : run_decode<64, false>(s, pos, q, kc, vc, cos_t, sin_t, cb, kbar, offsets,
                                          entries, sel, out, st);
    return bf ? run_decode<128, true>(s, pos, q, kc, vc, cos_t, sin_t, cb, kbar, offsets, entries,
                                      sel, out, st)
              : run_decode<128, false>(s, pos, q, kc, vc, cos_t, sin_t, cb, kbar, offsets,
                                       entries, sel, out, st);
}
