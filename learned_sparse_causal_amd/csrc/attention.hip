// Selected-set causal attention for gfx950.
//
// Method (technical report page "Monodratic: a reproducible sparse attention
// mixer", section "Mixer"; news page, section "Monodratic Turns Sparse
// Attention Into a Retrieval Decision"): every query attends, with ordinary
// causal softmax, to the tokens of its selected remote blocks and of its
// local blocks; selected values are used as they are.
//
// Every query carries its own remote blocks, so a tile of queries rarely
// shares a remote block.  The work is regrouped by source block instead:
//   plan     per 64-query tile: is every row's selection identical (always
//            true under the bypass)?  If not, every (query, slot) with a
//            valid, first-occurrence block takes a position in its
//            (batch, kv-head, block) bin with an integer atomic.
//   scan     bin starts and 256-row chunk starts (one workgroup).
//   scatter  (query, slot) ids into bin order.
//   remote   per chunk of one bin: the block's rotated K and transposed V in
//            LDS, up to 256 gathered rotated query rows, S^T = K Q^T and
//            O^T = V^T P^T on MFMA with an fp32 softmax; writes a normalized
//            partial output and its log-sum-exp per (query, slot).
//   local    per 64-query tile: local blocks (and, for identical-selection
//            tiles, the shared remote blocks) with an online softmax and the
//            causal mask, then the log-sum-exp merge of the tile's remote
//            partials, in slot order.
// The values a row gets never depend on which other rows share its tile, so
// the result does not depend on the order the atomics hand out positions.
#include <type_traits>

#include "mfma.hpp"

namespace {

template <bool BF16>
using Elem = std::conditional_t<BF16, u16, float>;

template <int D, bool BF16>
struct Tile {
    static constexpr int PAD = BF16 ? 8 : 4;
    static constexpr int QS = D + PAD;     // row stride (elements) of Q and K tiles
    static constexpr int VS = 64 + PAD;    // row stride of the transposed V tile (64 keys)
    static constexpr int Q_ELEMS = 64 * QS;
    static constexpr int K_ELEMS = 64 * QS;
    static constexpr int V_ELEMS = D * VS;
};

template <bool BF16>
__device__ __forceinline__ void load4(const void *base, size_t i, float *o) {
    if constexpr (BF16) {
        const uint2 v = *reinterpret_cast<const uint2 *>(reinterpret_cast<const u16 *>(base) + i);
        o[0] = __uint_as_float(v.x << 16);
        o[1] = __uint_as_float(v.x & 0xFFFF0000u);
        o[2] = __uint_as_float(v.y << 16);
        o[3] = __uint_as_float(v.y & 0xFFFF0000u);
    } else {
        const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + i);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
}

__device__ __forceinline__ void store4(u16 *p, const float *x) {
    uint2 w;
    w.x = (uint32_t)f32_to_bf16_bits(x[0]) | ((uint32_t)f32_to_bf16_bits(x[1]) << 16);
    w.y = (uint32_t)f32_to_bf16_bits(x[2]) | ((uint32_t)f32_to_bf16_bits(x[3]) << 16);
    *reinterpret_cast<uint2 *>(p) = w;
}

__device__ __forceinline__ void store4(float *p, const float *x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// Stage 64 rotated rows into an LDS tile.  rowfn(r, off, t) gives the element
// offset of row r and its position, or returns false for a zero row.
template <int D, bool BF16, typename RowFn>
__device__ __forceinline__ void stage_rotated(Elem<BF16> *dst, const void *src,
                                              const float *__restrict__ cos_t,
                                              const float *__restrict__ sin_t, RowFn rowfn) {
    constexpr int H = D / 2, G4 = H / 4;
    using T = Tile<D, BF16>;
    for (int task = threadIdx.x; task < 64 * G4; task += blockDim.x) {
        const int r = task / G4, i = (task % G4) * 4;
        size_t off = 0;
        int t = 0;
        float o0[4] = {0.f, 0.f, 0.f, 0.f}, o1[4] = {0.f, 0.f, 0.f, 0.f};
        if (rowfn(r, off, t)) {
            float x0[4], x1[4];
            load4<BF16>(src, off + i, x0);
            load4<BF16>(src, off + i + H, x1);
            const float4 c = *reinterpret_cast<const float4 *>(cos_t + (size_t)t * H + i);
            const float4 sn = *reinterpret_cast<const float4 *>(sin_t + (size_t)t * H + i);
            const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = x0[e] * cc[e], p1 = x1[e] * ss[e];
                const float p2 = x1[e] * cc[e], p3 = x0[e] * ss[e];
                o0[e] = p0 - p1;
                o1[e] = p2 + p3;
            }
        }
        store4(dst + r * T::QS + i, o0);
        store4(dst + r * T::QS + i + H, o1);
    }
}

// Stage V rows [row0, row0 + 64) (row stride `stride` elements) transposed:
// dst[d][key].  Rows at or past `nvalid` are zero.
template <int D, bool BF16>
__device__ __forceinline__ void stage_vt(Elem<BF16> *dst, const void *v, size_t row0, size_t stride,
                                         int nvalid) {
    using T = Tile<D, BF16>;
    constexpr int DG = D / 4;
    for (int task = threadIdx.x; task < 64 * DG; task += blockDim.x) {
        const int kk = task / DG, d0 = (task % DG) * 4;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (kk < nvalid) load4<BF16>(v, row0 + (size_t)kk * stride + d0, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (BF16) dst[(d0 + e) * T::VS + kk] = f32_to_bf16_bits(x[e]);
            else dst[(d0 + e) * T::VS + kk] = x[e];
        }
    }
}

// One wave, 16 queries (its rows of the Q tile) against 64 keys, folded into
// the running softmax state (m, l in log2 units, o unnormalized).  Keys with
// global index > qlimit are masked (causality).
template <int D, bool BF16>
__device__ __forceinline__ void attend64(const Elem<BF16> *Qw, const Elem<BF16> *Ks,
                                         const Elem<BF16> *Vt, float sl2, int key0, int qlimit,
                                         f32x4 (&o)[D / 16], float &m, float &l) {
    using T = Tile<D, BF16>;
    const int lane = lane_id(), lr = lane & 15, lg = lane >> 4;
    f32x4 st[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        const Frag8<BF16> qf = lds_frag8(Qw + lr * T::QS + 32 * c + 8 * lg);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const Frag8<BF16> kf = lds_frag8(Ks + (mt * 16 + lr) * T::QS + 32 * c + 8 * lg);
            mma32(st[mt], kf, qf);
        }
    }
    float mx = m;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + mt * 16 + 4 * lg + r;
            const float z = key <= qlimit ? st[mt][r] * sl2 : -INFINITY;
            st[mt][r] = z;
            mx = fmaxf(mx, z);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool none = mx == -INFINITY;
    const float alpha = none ? 1.0f : exp2f(m - mx);
    float p[4][4];
    float ps = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float z = st[mt][r];
            p[mt][r] = (z == -INFINITY) ? 0.0f : exp2f(z - mx);
            ps += p[mt][r];
        }
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * alpha + ps;
    if (!none) m = mx;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float pv[8] = {p[2 * c][0], p[2 * c][1], p[2 * c][2], p[2 * c][3],
                             p[2 * c + 1][0], p[2 * c + 1][1], p[2 * c + 1][2], p[2 * c + 1][3]};
        const Frag8<BF16> pf = reg_frag8<BF16>(pv);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const Elem<BF16> *vr = Vt + (dt * 16 + lr) * T::VS + 32 * c + 4 * lg;
            const Frag8<BF16> vf = lds_frag4x2(vr, vr + 16);
            mma32(o[dt], vf, pf);
        }
    }
}

__global__ void k_fill_i32(int32_t *p, long n, int32_t v) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// One wave per 64-query tile.
__global__ __launch_bounds__(256) void k_attn_plan(Shape s, const int32_t *__restrict__ sel,
                                                   int32_t *__restrict__ count,
                                                   int32_t *__restrict__ entry_pos,
                                                   int32_t *__restrict__ tile_flag) {
    const int lane = lane_id(), wave = threadIdx.x / WAVE;
    const long ntiles = (long)s.B * s.Hq * (s.T / 64);
    const long tile = (long)blockIdx.x * 4 + wave;
    if (tile >= ntiles) return;
    const int tt = (int)(tile % (s.T / 64));
    const long bh = tile / (s.T / 64);
    const int h = (int)(bh % s.Hq), b = (int)(bh / s.Hq), g = h / s.G;
    const int t0 = tt * 64, qb = t0 / s.beta, last = qb - s.L, R = s.R;
    const long route0 = bh * s.T + t0;
    const long route = route0 + lane;
    const int32_t *row = sel + route * R;
    const int32_t *row0 = sel + route0 * R;
    bool same = true;
    for (int r = 0; r < R; ++r) same = same && row[r] == row0[r];
    const bool uni = __ballot(!same) == 0ull;
    if (lane == 0) tile_flag[tile] = uni ? 1 : 0;
    int32_t *ep = entry_pos + route * R;
    for (int r = 0; r < R; ++r) {
        const int id = row[r];
        bool valid = !uni && id >= 0 && id <= last;
        for (int r2 = 0; valid && r2 < r; ++r2) valid = row[r2] != id;
        int pos = -1;
        if (valid) pos = atomicAdd(&count[((size_t)b * s.Hkv + g) * s.NB + id], 1);
        ep[r] = pos;
    }
}

constexpr int SCAN_THREADS = 1024;
constexpr int CHUNK_ROWS = 256;

__global__ __launch_bounds__(SCAN_THREADS) void k_attn_scan(int nbins, const int32_t *__restrict__ count,
                                                            int32_t *__restrict__ bin_start,
                                                            int32_t *__restrict__ chunk_start,
                                                            int32_t *__restrict__ total_chunks) {
    __shared__ int32_t ps[SCAN_THREADS], pc[SCAN_THREADS];
    const int tid = threadIdx.x;
    const int per = (nbins + SCAN_THREADS - 1) / SCAN_THREADS;
    const int lo = min(nbins, tid * per), hi = min(nbins, lo + per);
    int s0 = 0, c0 = 0;
    for (int i = lo; i < hi; ++i) {
        const int c = count[i];
        s0 += c;
        c0 += (c + CHUNK_ROWS - 1) / CHUNK_ROWS;
    }
    ps[tid] = s0;
    pc[tid] = c0;
    __syncthreads();
    for (int off = 1; off < SCAN_THREADS; off <<= 1) {  // inclusive Hillis-Steele scan
        const int a = tid >= off ? ps[tid - off] : 0;
        const int c = tid >= off ? pc[tid - off] : 0;
        __syncthreads();
        ps[tid] += a;
        pc[tid] += c;
        __syncthreads();
    }
    int rs = tid ? ps[tid - 1] : 0, rc = tid ? pc[tid - 1] : 0;
    for (int i = lo; i < hi; ++i) {
        bin_start[i] = rs;
        chunk_start[i] = rc;
        const int c = count[i];
        rs += c;
        rc += (c + CHUNK_ROWS - 1) / CHUNK_ROWS;
    }
    if (tid == SCAN_THREADS - 1) {
        bin_start[nbins] = ps[tid];
        chunk_start[nbins] = pc[tid];
        total_chunks[0] = pc[tid];
    }
}

__global__ __launch_bounds__(256) void k_attn_scatter(Shape s, const int32_t *__restrict__ sel,
                                                      const int32_t *__restrict__ entry_pos,
                                                      const int32_t *__restrict__ bin_start,
                                                      int32_t *__restrict__ list) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long n = (long)s.B * s.Hq * s.T * s.R;
    if (i >= n) return;
    const int pos = entry_pos[i];
    if (pos < 0) return;
    const long route = i / s.R;
    const int h = (int)((route / s.T) % s.Hq), b = (int)(route / ((long)s.T * s.Hq));
    const int g = h / s.G;
    const int id = sel[i];
    list[bin_start[((size_t)b * s.Hkv + g) * s.NB + id] + pos] = (int32_t)i;
}

template <int D, int BETA, bool BF16>
__global__ __launch_bounds__(256) void k_attn_remote(Shape s, const void *__restrict__ q,
                                                     const void *__restrict__ k,
                                                     const void *__restrict__ v,
                                                     const float *__restrict__ cos_t,
                                                     const float *__restrict__ sin_t,
                                                     const int32_t *__restrict__ list,
                                                     const int32_t *__restrict__ bin_start,
                                                     const int32_t *__restrict__ chunk_start,
                                                     const int32_t *__restrict__ total_chunks,
                                                     float *__restrict__ part_lse,
                                                     Elem<BF16> *__restrict__ part_o) {
    using T = Tile<D, BF16>;
    using E = Elem<BF16>;
    constexpr int NSUB = BETA / 64;
    extern __shared__ __align__(16) unsigned char smem[];
    E *Ks = reinterpret_cast<E *>(smem);               // NSUB x [64][QS]
    E *Vts = Ks + NSUB * T::K_ELEMS;                    // NSUB x [D][VS]
    E *Qs = Vts + NSUB * T::V_ELEMS;                    // [64][QS]

    const int chunk = blockIdx.x;
    if (chunk >= total_chunks[0]) return;
    const int nbins = s.B * s.Hkv * s.NB;
    int lo = 0, hi = nbins;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (chunk_start[mid] <= chunk) lo = mid;
        else hi = mid;
    }
    const int bin = lo;
    const int r0 = bin_start[bin] + (chunk - chunk_start[bin]) * CHUNK_ROWS;
    const int r1 = min(r0 + CHUNK_ROWS, bin_start[bin + 1]);
    const int n = bin % s.NB, g = (bin / s.NB) % s.Hkv, b = bin / (s.NB * s.Hkv);
    const int T_ = s.T, Hkv = s.Hkv, Hq = s.Hq, R = s.R;

#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
        const int tb = n * BETA + sub * 64;
        stage_rotated<D, BF16>(Ks + sub * T::K_ELEMS, k, cos_t, sin_t,
                               [&](int r, size_t &off, int &t) {
                                   t = tb + r;
                                   off = (((size_t)b * T_ + t) * Hkv + g) * D;
                                   return true;
                               });
        stage_vt<D, BF16>(Vts + sub * T::V_ELEMS, v, (((size_t)b * T_ + tb) * Hkv + g) * D,
                          (size_t)Hkv * D, 64);
    }
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);
    const int lane = lane_id(), wave = threadIdx.x / WAVE, lr = lane & 15, lg = lane >> 4;
    for (int rb = r0; rb < r1; rb += 64) {
        __syncthreads();
        stage_rotated<D, BF16>(Qs, q, cos_t, sin_t, [&](int r, size_t &off, int &t) {
            const int row = rb + r;
            if (row >= r1) return false;
            const long route = list[row] / R;
            t = (int)(route % T_);
            const int hq = (int)((route / T_) % Hq);
            off = (((size_t)b * T_ + t) * Hq + hq) * D;
            return true;
        });
        __syncthreads();
        f32x4 o[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, l = 0.0f;
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub)
            attend64<D, BF16>(Qs + wave * 16 * T::QS, Ks + sub * T::K_ELEMS, Vts + sub * T::V_ELEMS,
                              sl2, 0, 0x7fffffff, o, m, l);
        const int row = rb + wave * 16 + lr;
        if (row < r1) {
            const int e = list[row];
            if (lg == 0) part_lse[e] = m + log2f(l);
            const float inv = 1.0f / l;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const float x[4] = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
                store4(part_o + (size_t)e * D + dt * 16 + 4 * lg, x);
            }
        }
    }
}

template <int D, int BETA, bool BF16>
__global__ __launch_bounds__(256) void k_attn_local(Shape s, const void *__restrict__ q,
                                                    const void *__restrict__ k,
                                                    const void *__restrict__ v,
                                                    const float *__restrict__ cos_t,
                                                    const float *__restrict__ sin_t,
                                                    const int32_t *__restrict__ sel,
                                                    const int32_t *__restrict__ tile_flag,
                                                    const int32_t *__restrict__ entry_pos,
                                                    const float *__restrict__ part_lse,
                                                    const Elem<BF16> *__restrict__ part_o,
                                                    void *__restrict__ out) {
    using T = Tile<D, BF16>;
    using E = Elem<BF16>;
    extern __shared__ __align__(16) unsigned char smem[];
    E *Qs = reinterpret_cast<E *>(smem);
    E *Ks = Qs + T::Q_ELEMS;
    E *Vt = Ks + T::K_ELEMS;
    int *blk_s = reinterpret_cast<int *>(Vt + T::V_ELEMS);  // [R] shared remote blocks

    const int ntt = s.T / 64, nbh = s.B * s.Hq;
    // latest tiles first: they have the most blocks
    const int tt = ntt - 1 - (int)(blockIdx.x / nbh);
    const int bh = (int)(blockIdx.x % nbh);
    const int h = bh % s.Hq, b = bh / s.Hq, g = h / s.G;
    const int t0 = tt * 64, qb = t0 / BETA, R = s.R, L = s.L;
    const int T_ = s.T, Hkv = s.Hkv, Hq = s.Hq;
    const long tile = (long)bh * ntt + tt;
    const bool uni = tile_flag[tile] != 0;
    const long route0 = (long)bh * T_ + t0;

    stage_rotated<D, BF16>(Qs, q, cos_t, sin_t, [&](int r, size_t &off, int &t) {
        t = t0 + r;
        off = (((size_t)b * T_ + t) * Hq + h) * D;
        return true;
    });
    if (uni) {  // shared remote blocks of the tile: valid first occurrences of row 0
        const int32_t *row0 = sel + route0 * R;
        for (int r = threadIdx.x; r < R; r += blockDim.x) {
            const int id = row0[r];
            bool ok = id >= 0 && id <= qb - L;
            for (int r2 = 0; ok && r2 < r; ++r2) ok = row0[r2] != id;
            blk_s[r] = ok ? id : -1;
        }
    }
    __syncthreads();

    const int lane = lane_id(), wave = threadIdx.x / WAVE, lr = lane & 15, lg = lane >> 4;
    const int tq = t0 + wave * 16 + lr;  // this lane's query position
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);
    f32x4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.0f;

    const int nrem = uni ? R : 0;
    const int lo_blk = max(0, qb - L + 1);
    const int nblk = nrem + (qb - lo_blk + 1);
    for (int j = 0; j < nblk; ++j) {
        const int blk = j < nrem ? blk_s[j] : lo_blk + (j - nrem);
        if (blk < 0) continue;
        for (int sub = 0; sub < BETA / 64; ++sub) {
            const int kb0 = blk * BETA + sub * 64;
            if (kb0 > t0 + 63) break;  // entirely after every query of the tile
            __syncthreads();
            stage_rotated<D, BF16>(Ks, k, cos_t, sin_t, [&](int r, size_t &off, int &t) {
                t = kb0 + r;
                off = (((size_t)b * T_ + t) * Hkv + g) * D;
                return true;
            });
            stage_vt<D, BF16>(Vt, v, (((size_t)b * T_ + kb0) * Hkv + g) * D, (size_t)Hkv * D, 64);
            __syncthreads();
            attend64<D, BF16>(Qs + wave * 16 * T::QS, Ks, Vt, sl2, kb0, tq, o, m, l);
        }
    }

    // merge: local (and shared) part, then the remote partials in slot order
    const long route = route0 + wave * 16 + lr;
    float lse = m + log2f(l);
    float inv = 1.0f / l;
    float acc[D / 16][4];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][r] = o[dt][r] * inv;
    if (!uni) {
        const int32_t *ep = entry_pos + route * R;
        float M = lse;
        for (int r = 0; r < R; ++r)
            if (ep[r] >= 0) M = fmaxf(M, part_lse[route * R + r]);
        float wsum = exp2f(lse - M);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[dt][r] *= wsum;
        for (int r = 0; r < R; ++r) {
            if (ep[r] < 0) continue;
            const long e = route * R + r;
            const float w = exp2f(part_lse[e] - M);
            wsum += w;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                float x[4];
                load4<BF16>(part_o, (size_t)e * D + dt * 16 + 4 * lg, x);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[dt][rr] += w * x[rr];
            }
        }
        const float iw = 1.0f / wsum;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[dt][r] *= iw;
    }
    E *op = reinterpret_cast<E *>(out) + (((size_t)b * T_ + tq) * Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) store4(op + dt * 16 + 4 * lg, acc[dt]);
}

template <typename F>
hipError_t ensure_lds(F *fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

struct AttnWs {
    int32_t *count, *bin_start, *chunk_start, *total, *tile_flag, *entry_pos, *list;
    float *part_lse;
    void *part_o;
};

template <int D, int BETA, bool BF16>
hipError_t run_attention(const Shape &s, const void *q, const void *k, const void *v,
                         const float *cos_t, const float *sin_t, const int32_t *sel, void *out,
                         const AttnWs &w, hipStream_t st) {
    using T = Tile<D, BF16>;
    using E = Elem<BF16>;
    const int nbins = s.B * s.Hkv * s.NB;
    const long ntiles = (long)s.B * s.Hq * (s.T / 64);
    const long nent = (long)s.B * s.Hq * s.T * s.R;
    k_fill_i32<<<dim3((unsigned)((nbins + 255) / 256)), 256, 0, st>>>(w.count, nbins, 0);
    k_attn_plan<<<dim3((unsigned)((ntiles + 3) / 4)), 256, 0, st>>>(s, sel, w.count, w.entry_pos,
                                                                     w.tile_flag);
    k_attn_scan<<<1, SCAN_THREADS, 0, st>>>(nbins, w.count, w.bin_start, w.chunk_start, w.total);
    k_attn_scatter<<<dim3((unsigned)((nent + 255) / 256)), 256, 0, st>>>(s, sel, w.entry_pos,
                                                                         w.bin_start, w.list);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const long max_chunks = nbins + (nent + CHUNK_ROWS - 1) / CHUNK_ROWS;
    const size_t lds_r = (size_t)((BETA / 64) * (T::K_ELEMS + T::V_ELEMS) + T::Q_ELEMS) * sizeof(E);
    err = ensure_lds(k_attn_remote<D, BETA, BF16>, lds_r);
    if (err != hipSuccess) return err;
    k_attn_remote<D, BETA, BF16><<<dim3((unsigned)max_chunks), 256, lds_r, st>>>(
        s, q, k, v, cos_t, sin_t, w.list, w.bin_start, w.chunk_start, w.total, w.part_lse,
        reinterpret_cast<E *>(w.part_o));
    const size_t lds_l = (size_t)(T::Q_ELEMS + T::K_ELEMS + T::V_ELEMS) * sizeof(E) +
                         (size_t)s.R * sizeof(int);
    err = ensure_lds(k_attn_local<D, BETA, BF16>, lds_l);
    if (err != hipSuccess) return err;
    k_attn_local<D, BETA, BF16><<<dim3((unsigned)ntiles), 256, lds_l, st>>>(
        s, q, k, v, cos_t, sin_t, sel, w.tile_flag, w.entry_pos, w.part_lse,
        reinterpret_cast<const E *>(w.part_o), out);
    return hipGetLastError();
}

}  // namespace

// Workspace layout of the attention call (byte offsets, 256-aligned).
size_t attention_ws_layout(const Shape &s, size_t *off) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t nbins = (size_t)s.B * s.Hkv * s.NB;
    const size_t ntiles = (size_t)s.B * s.Hq * (s.T / 64);
    const size_t nent = (size_t)s.B * s.Hq * s.T * s.R;
    const size_t esz = s.dtype == 1 ? 2 : 4;
    size_t p = 0;
    off[0] = p; p = al(p + nbins * 4);              // count
    off[1] = p; p = al(p + (nbins + 1) * 4);        // bin_start
    off[2] = p; p = al(p + (nbins + 1) * 4);        // chunk_start
    off[3] = p; p = al(p + 4);                      // total chunks
    off[4] = p; p = al(p + ntiles * 4);             // tile flags
    off[5] = p; p = al(p + nent * 4);               // entry positions
    off[6] = p; p = al(p + nent * 4);               // list
    off[7] = p; p = al(p + nent * 4);               // partial lse
    off[8] = p; p = al(p + nent * (size_t)s.d * esz);  // partial outputs
    return p;
}

hipError_t launch_attention(const Shape &s, const void *q, const void *k, const void *v,
                            const float *cos_t, const float *sin_t, const int32_t *sel, void *out,
                            void *ws, hipStream_t st) {
    size_t off[9];
    attention_ws_layout(s, off);
    unsigned char *base = reinterpret_cast<unsigned char *>(ws);
    AttnWs w;
    w.count = reinterpret_cast<int32_t *>(base + off[0]);
    w.bin_start = reinterpret_cast<int32_t *>(base + off[1]);
    w.chunk_start = reinterpret_cast<int32_t *>(base + off[2]);
    w.total = reinterpret_cast<int32_t *>(base + off[3]);
    w.tile_flag = reinterpret_cast<int32_t *>(base + off[4]);
    w.entry_pos = reinterpret_cast<int32_t *>(base + off[5]);
    w.list = reinterpret_cast<int32_t *>(base + off[6]);
    w.part_lse = reinterpret_cast<float *>(base + off[7]);
    w.part_o = base + off[8];
    const bool bf = s.dtype == 1;
#define MONO_ATTN_ARGS s, q, k, v, cos_t, sin_t, sel, out, w, st
    if (s.d == 64) {
        if (s.beta == 64) return bf ? run_attention<64, 64, true>(MONO_ATTN_ARGS)
                                    : run_attention<64, 64, false>(MONO_ATTN_ARGS);
        return bf ? run_attention<64, 128, true>(MONO_ATTN_ARGS)
                  : run_attention<64, 128, false>(MONO_ATTN_ARGS);
    }
    if (s.beta == 64) return bf ? run_attention<128, 64, true>(MONO_ATTN_ARGS)
                                : run_attention<128, 64, false>(MONO_ATTN_ARGS);
    return bf ? run_attention<128, 128, true>(MONO_ATTN_ARGS)
              : run_attention<128, 128, false>(MONO_ATTN_ARGS);
#undef MONO_ATTN_ARGS
}
