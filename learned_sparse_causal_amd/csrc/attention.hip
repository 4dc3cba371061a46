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
//   prep     per (batch, kv-head, 1024-token segment): for every 64-query tile
//            of the group's q-heads, is every row's selection identical
//            (always true under the bypass)?  If not, every (query, slot)
//            with a valid, first-occurrence block takes a rank in its
//            source-block bin from an LDS counter; the segment's per-bin
//            counts go to global memory.  The same workgroup rotates the
//            segment's q rows (all heads of the group) and k rows once and
//            stores them in the activation dtype, so no later kernel reads
//            the rotary table.
//   binsum   per bin: exclusive prefix of the segments' counts.
//   scan     bin starts and 256-row chunk starts (one workgroup).
//   scatter  (query, slot) ids into bin order (bin, then segment, then rank).
//   remote   per chunk of one bin: the block's rotated K and transposed V in
//            LDS, up to 256 gathered rotated query rows, S^T = K Q^T and
//            O^T = V^T P^T on MFMA with an fp32 softmax; writes a normalized
//            partial output and its log-sum-exp per (query, slot).
//   local    per 64-query tile: local blocks (and, for identical-selection
//            tiles, the shared remote blocks) with an online softmax and the
//            causal mask, then the log-sum-exp merge of the tile's remote
//            partials, in slot order.
// No global atomics are used.  The values a row gets never depend on which
// other rows share its chunk, so results are deterministic.  Workgroup ids
// are remapped so that consecutive work items (chunks of one bin, adjacent
// query tiles of one head) land on the same XCD and share its L2.
#include <algorithm>
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

// Partial outputs are stored lane-chunked: the values a lane holds for one
// row in the MFMA output layout (dims 16 dt + 4 lg + r, in (dt, r) order) go
// out as NCH 16-byte chunks, chunk j at 16-byte slot 4 j + lg of the row, so
// one store instruction writes 64 contiguous bytes of each of its 16 rows.
template <int D, bool BF16>
struct PartChunks {
    static constexpr int NCH = D * (BF16 ? 2 : 4) / 64;
    u32x4 c[NCH];
    __device__ __forceinline__ void pack(const float (&v)[D / 16][4]) {
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < NCH; ++j)
                c[j] = u32x4{pack_bf16x2(v[2 * j][0], v[2 * j][1]), pack_bf16x2(v[2 * j][2], v[2 * j][3]),
                             pack_bf16x2(v[2 * j + 1][0], v[2 * j + 1][1]),
                             pack_bf16x2(v[2 * j + 1][2], v[2 * j + 1][3])};
        } else {
#pragma unroll
            for (int j = 0; j < NCH; ++j)
                c[j] = u32x4{__float_as_uint(v[j][0]), __float_as_uint(v[j][1]),
                             __float_as_uint(v[j][2]), __float_as_uint(v[j][3])};
        }
    }
    __device__ __forceinline__ void unpack(float (&v)[D / 16][4]) const {
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    v[2 * j + h][0] = __uint_as_float(c[j][2 * h] << 16);
                    v[2 * j + h][1] = __uint_as_float(c[j][2 * h] & 0xFFFF0000u);
                    v[2 * j + h][2] = __uint_as_float(c[j][2 * h + 1] << 16);
                    v[2 * j + h][3] = __uint_as_float(c[j][2 * h + 1] & 0xFFFF0000u);
                }
        } else {
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[j][r] = __uint_as_float(c[j][r]);
        }
    }
    __device__ __forceinline__ void store(Elem<BF16> *row, int lg) const {
#pragma unroll
        for (int j = 0; j < NCH; ++j) reinterpret_cast<u32x4 *>(row)[4 * j + lg] = c[j];
    }
    __device__ __forceinline__ void load(const Elem<BF16> *row, int lg) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) c[j] = reinterpret_cast<const u32x4 *>(row)[4 * j + lg];
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int j = 0; j < NCH; ++j) c[j] = u32x4{0u, 0u, 0u, 0u};
    }
    // The row's log-sum-exp rides in the row itself, so the merge reads one
    // line per partial: byte lg of its 32 bits goes in the lowest mantissa
    // bits of chunk 0 of lane group lg (bf16: the last bit of each of its 8
    // elements, at most one unit in the last place each; fp32: the last two
    // bits of each of its 4).
    __device__ __forceinline__ void embed(float lse, int lg) {
        const uint32_t b = (__float_as_uint(lse) >> (8 * lg)) & 0xFFu;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (BF16)
                c[0][k] = (c[0][k] & 0xFFFEFFFEu) | ((b >> (2 * k)) & 1u) | (((b >> (2 * k + 1)) & 1u) << 16);
            else
                c[0][k] = (c[0][k] & ~3u) | ((b >> (2 * k)) & 3u);
        }
    }
    // The log-sum-exp of the row a lane group holds; every lane of the
    // wave must take part (the bytes are exchanged between the row's lanes
    // lane, lane ^ 16, lane ^ 32 and lane ^ 48).
    __device__ __forceinline__ float lse(int lg) const {
        uint32_t b = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (BF16)
                b |= ((c[0][k] & 1u) << (2 * k)) | (((c[0][k] >> 16) & 1u) << (2 * k + 1));
            else
                b |= (c[0][k] & 3u) << (2 * k);
        }
        uint32_t w = b << (8 * lg);
        w |= (uint32_t)__shfl_xor((int)w, 16);
        w |= (uint32_t)__shfl_xor((int)w, 32);
        return __uint_as_float(w);
    }
};

__device__ __forceinline__ void store4(u16 *p, const float *x) {
    uint2 w;
    w.x = pack_bf16x2(x[0], x[1]);
    w.y = pack_bf16x2(x[2], x[3]);
    *reinterpret_cast<uint2 *>(p) = w;
}

__device__ __forceinline__ void store4(float *p, const float *x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}



// Workgroup id -> work item, so that consecutive items run on one XCD
// (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int x = bid & 7, j = bid >> 3;
    const int per = n >> 3, rem = n & 7;
    return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

// Register-staged copies for software pipelining (256 threads): issue()
// starts the global loads of a 64-row tile into registers, commit() writes
// them to LDS later, so the loads of the next tile overlap the current
// tile's compute.
template <int D, bool BF16>
struct RowStager {
    using E = Elem<BF16>;
    static constexpr int VE = 16 / sizeof(E);
    static constexpr int PR = D / VE;             // 16-byte pieces per row
    static constexpr int PER = 64 * PR / 256;     // pieces per thread
    uint4 v[PER];
    template <typename RowFn>
    __device__ __forceinline__ void issue(const E *src, RowFn rowfn) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int task = threadIdx.x + p * 256;
            const int r = task / PR, c = (task % PR) * VE;
            size_t off = 0;
            v[p] = rowfn(r, off) ? *reinterpret_cast<const uint4 *>(src + off + c)
                                 : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __device__ __forceinline__ void commit(E *dst) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int task = threadIdx.x + p * 256;
            const int r = task / PR, c = (task % PR) * VE;
            *reinterpret_cast<uint4 *>(dst + r * Tile<D, BF16>::QS + c) = v[p];
        }
    }
};

template <int D, bool BF16>
struct VtStager {
    using E = Elem<BF16>;
    static constexpr int VE = 16 / sizeof(E);
    static constexpr int PER = 64 * (D / VE) / 256;
    uint4 v[PER];
    // rows row0 + kk * stride, kk < 64; consecutive threads take consecutive keys
    __device__ __forceinline__ void issue(const E *src, size_t row0, size_t stride) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int task = threadIdx.x + p * 256;
            const int kk = task & 63, d0 = (task >> 6) * VE;
            v[p] = *reinterpret_cast<const uint4 *>(src + row0 + (size_t)kk * stride + d0);
        }
    }
    __device__ __forceinline__ void commit(E *dst) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int task = threadIdx.x + p * 256;
            const int kk = task & 63, d0 = (task >> 6) * VE;
            const E *x = reinterpret_cast<const E *>(&v[p]);
#pragma unroll
            for (int e = 0; e < VE; ++e) dst[(d0 + e) * Tile<D, BF16>::VS + kk] = x[e];
        }
    }
};

// V^T tile stager for bf16 (256 threads): each task takes 4 consecutive
// keys x 4 dims (four 8-byte loads) and writes, per dim, the 4 keys as one
// 8-byte LDS store.  The 4-key granules of dim row r are stored XOR-swizzled
// by 2 (r / 16), i.e. key column x of row r sits at x ^ (8 (r / 16)): the
// stores of a half-wave (16 dim chunks x 2 quads, or 32 chunks x 1 quad)
// then fall on distinct banks, while a fragment read (16 rows of one 16-row
// block) sees one XOR for all its lanes.
template <int D>
struct VtStagerPacked {
    static constexpr int NC = D / 4;                // 4-dim chunks per key row
    static constexpr int PER = 16 * NC / 256;       // tasks per thread
    uint2 v[PER][4];
    __device__ __forceinline__ void issue(const u16 *src, size_t row0, size_t stride) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int task = threadIdx.x + p * 256;
            const int c = task % NC, j = task / NC;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[p][i] = *reinterpret_cast<const uint2 *>(src + row0 + (size_t)(4 * j + i) * stride +
                                                           4 * c);
        }
    }
    __device__ __forceinline__ void commit(u16 *dst) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int task = threadIdx.x + p * 256;
            const int c = task % NC, j = task / NC;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t x = e < 2 ? v[p][i].x : v[p][i].y;
                    w[i] = (e & 1) ? x >> 16 : x & 0xFFFFu;
                }
                const int row = 4 * c + e;
                *reinterpret_cast<uint2 *>(dst + row * Tile<D, true>::VS +
                                           ((4 * j) ^ (8 * (row >> 4)))) =
                    make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
            }
        }
    }
};

// The V^T stager of a dtype: packed and swizzled for bf16, plain for fp32.
template <int D, bool BF16>
struct VtStagerOf {
    using type = VtStager<D, BF16>;
};
template <int D>
struct VtStagerOf<D, true> {
    using type = VtStagerPacked<D>;
};

// The wave's Q^T fragments for one query row per lane (row offset `off`
// elements, all-zero if !ok): dims 32c + 8(l/16) .. +7 for c < D/32.
template <int D, bool BF16>
struct QFrags {
    using E = Elem<BF16>;
    static constexpr int VE = 16 / sizeof(E);
    static constexpr int NV = 8 / VE;   // 16-byte loads per 8 elements
    uint4 raw[D / 32][NV];
    __device__ __forceinline__ void issue(const E *src, size_t off, bool ok) {
        const int lg = lane_id() >> 4;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int u = 0; u < NV; ++u)
                raw[c][u] = ok ? *reinterpret_cast<const uint4 *>(src + off + 32 * c + 8 * lg + u * VE)
                               : make_uint4(0u, 0u, 0u, 0u);
    }
    __device__ __forceinline__ void get(Frag8<BF16> (&f)[D / 32]) const {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            if constexpr (BF16) {
                f[c].v = __builtin_bit_cast(bf16x8, raw[c][0]);
            } else {
                const float *x0 = reinterpret_cast<const float *>(&raw[c][0]);
                const float *x1 = reinterpret_cast<const float *>(&raw[c][NV - 1]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[c].v[e] = x0[e];
                    f[c].v[4 + e] = x1[e];
                }
            }
        }
    }
};

// One wave, 16 queries (B fragments of Q^T in registers: lane l holds row
// l%16, dims 32c + 8(l/16) .. +7) against 64 keys, folded into the running
// softmax state (m, l in log2 units, o unnormalized).  The query rows are
// pre-scaled by log2(e)/sqrt(d), so scores are base-2 logits.  MASK: keys
// with global index > qlimit are masked (causality).  FIRST: the state is
// empty on entry (m = -inf, l = 0, o = 0), so nothing is rescaled.
template <int D, bool BF16, bool MASK, bool FIRST>
__device__ __forceinline__ void attend64(const Frag8<BF16> (&qf)[D / 32], const Elem<BF16> *Ks,
                                         const Elem<BF16> *Vt, int key0, int qlimit,
                                         f32x4 (&o)[D / 16], float &m, float &l) {
    using T = Tile<D, BF16>;
    const int lane = lane_id(), lr = lane & 15, lg = lane >> 4;
    f32x4 st[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const Frag8<BF16> kf = lds_frag8(Ks + (mt * 16 + lr) * T::QS + 32 * c + 8 * lg);
            mma32(st[mt], kf, qf[c]);
        }
    }
    float mx = FIRST ? -INFINITY : m;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (MASK) {
                const int key = key0 + mt * 16 + 4 * lg + r;
                st[mt][r] = key <= qlimit ? st[mt][r] : -INFINITY;
            }
            mx = fmaxf(mx, st[mt][r]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // a row with every key masked so far keeps mx = -inf: no key contributes
    const bool none = MASK && mx == -INFINITY;
    const float msub = none ? 0.0f : mx;
    float p[4][4];
    float ps = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[mt][r] = __builtin_amdgcn_exp2f(st[mt][r] - msub);   // exp2(-inf) = 0
            ps += p[mt][r];
        }
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    if constexpr (FIRST) {
        l = ps;
        m = mx;
    } else {
        const float alpha = none ? 1.0f : __builtin_amdgcn_exp2f(m - mx);
        l = l * alpha + ps;
        if (!none) m = mx;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float pv[8] = {p[2 * c][0], p[2 * c][1], p[2 * c][2], p[2 * c][3],
                             p[2 * c + 1][0], p[2 * c + 1][1], p[2 * c + 1][2], p[2 * c + 1][3]};
        const Frag8<BF16> pf = reg_frag8<BF16>(pv);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            // bf16 V^T tiles are stored swizzled (VtStagerPacked)
            const int sw = BF16 ? 8 * dt : 0;
            const Elem<BF16> *vr = Vt + (dt * 16 + lr) * T::VS;
            const Frag8<BF16> vf = lds_frag4x2(vr + ((32 * c + 4 * lg) ^ sw),
                                               vr + ((32 * c + 16 + 4 * lg) ^ sw));
            mma32(o[dt], vf, pf);
        }
    }
}


constexpr int SEG = 1024;          // tokens per prep segment
constexpr int SCAN_THREADS = 1024;
constexpr int CHUNK_ROWS = 256;

constexpr int PREP_THREADS = 1024;

// RMAX > 0: R <= RMAX, and a lane keeps its row of the selection in
// registers (one load per slot; the duplicate checks compare registers).
// RMAX = 0: any R, the row is re-read from memory.
template <int RMAX>
__global__ __launch_bounds__(PREP_THREADS) void k_attn_prep(Shape s, const int32_t *__restrict__ sel,
                                                   int32_t *__restrict__ cnt,
                                                   int32_t *__restrict__ entry_pos,
                                                   int32_t *__restrict__ tile_flag, int nseg) {
    extern __shared__ int hist[];   // [NB]
    const int seg = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int T_ = s.T, Hq = s.Hq, Hkv = s.Hkv, G = s.G, R = s.R, NB = s.NB;
    const int t_beg = seg * SEG, t_end = min(T_, t_beg + SEG);
    const int lane = lane_id(), wave = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
    for (int n = threadIdx.x; n < NB; n += blockDim.x) hist[n] = 0;
    __syncthreads();

    const int ntile = (t_end - t_beg) / 64;
    for (int task = wave; task < G * ntile; task += nw) {
        const int hl = task / ntile, tl = task % ntile;
        const int h = g * G + hl, t0 = t_beg + tl * 64;
        const int qb = t0 / s.beta, last = qb - s.L;
        const long route0 = ((long)b * Hq + h) * T_ + t0;
        const long route = route0 + lane;
        const int32_t *row = sel + route * R;
        const int32_t *row0 = sel + route0 * R;
        int32_t *ep = entry_pos + route * R;
        if constexpr (RMAX > 0) {
            int v[RMAX];
#pragma unroll
            for (int r = 0; r < RMAX; ++r) v[r] = r < R ? row[r] : -1;
            bool same = true;
#pragma unroll
            for (int r = 0; r < RMAX; ++r) same = same && (r >= R || v[r] == row0[r]);
            const bool uni = __ballot(!same) == 0ull;
            if (lane == 0) tile_flag[((long)b * Hq + h) * (T_ / 64) + t0 / 64] = uni ? 1 : 0;
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                if (r < R) {   // wave-uniform
                    bool valid = !uni && v[r] >= 0 && v[r] <= last;
#pragma unroll
                    for (int r2 = 0; r2 < r; ++r2) valid = valid && v[r2] != v[r];
                    ep[r] = valid ? atomicAdd(&hist[v[r]], 1) : -1;
                }
            }
        } else {
            bool same = true;
            for (int r = 0; r < R; ++r) same = same && row[r] == row0[r];
            const bool uni = __ballot(!same) == 0ull;
            if (lane == 0) tile_flag[((long)b * Hq + h) * (T_ / 64) + t0 / 64] = uni ? 1 : 0;
            for (int r = 0; r < R; ++r) {
                const int id = row[r];
                bool valid = !uni && id >= 0 && id <= last;
                for (int r2 = 0; valid && r2 < r; ++r2) valid = row[r2] != id;
                ep[r] = valid ? atomicAdd(&hist[id], 1) : -1;
            }
        }
    }
    __syncthreads();
    int32_t *cg = cnt + (((size_t)b * Hkv + g) * nseg + seg) * NB;   // [b, g][seg][n]
    for (int n = threadIdx.x; n < NB; n += blockDim.x) cg[n] = hist[n];
}

// Rotate every q and k row once into the activation dtype (grid-wide stream;
// one thread per 8 rotation pairs, so every access is 16 bytes or more; rows
// of one position are adjacent so the rotary table row is read once from
// cache for all heads).
template <bool BF16>
__device__ __forceinline__ void store8(Elem<BF16> *p, const float *x) {
    if constexpr (BF16) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                   pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
    } else {
        reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
        reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_attn_rotate(Shape s, const void *__restrict__ q,
                                                     const void *__restrict__ k,
                                                     const float *__restrict__ cos_t,
                                                     const float *__restrict__ sin_t,
                                                     Elem<BF16> *__restrict__ q_rot,
                                                     Elem<BF16> *__restrict__ k_rot) {
    constexpr int H = D / 2, PT = H / 8;
    const int heads = s.Hq + s.Hkv;
    const long total = (long)s.B * s.T * heads * PT;
    for (long task = (long)blockIdx.x * blockDim.x + threadIdx.x; task < total;
         task += (long)gridDim.x * blockDim.x) {
        const int i = (int)(task % PT) * 8;
        const long row = task / PT;               // (b, t, head) with head fastest
        const int hd = (int)(row % heads);
        const long bt = row / heads;
        const int t = (int)(bt % s.T);
        size_t off;
        const void *src;
        Elem<BF16> *dst;
        if (hd < s.Hq) {
            off = ((size_t)bt * s.Hq + hd) * D;
            src = q;
            dst = q_rot;
        } else {
            off = ((size_t)bt * s.Hkv + (hd - s.Hq)) * D;
            src = k;
            dst = k_rot;
        }
        // query rows carry the softmax scale log2(e)/sqrt(d) (base-2 logits)
        const float sc = hd < s.Hq ? 1.4426950408889634f / sqrtf((float)D) : 1.0f;
        float x0[8], x1[8], o0[8], o1[8];
        load8<BF16>(src, off + i, x0);
        load8<BF16>(src, off + i + H, x1);
        const float4 *cp = reinterpret_cast<const float4 *>(cos_t + (size_t)t * H + i);
        const float4 *sp = reinterpret_cast<const float4 *>(sin_t + (size_t)t * H + i);
        const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
        const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p0 = x0[e] * cc[e], p1 = x1[e] * ss[e];
            const float p2 = x1[e] * cc[e], p3 = x0[e] * ss[e];
            o0[e] = (p0 - p1) * sc;
            o1[e] = (p2 + p3) * sc;
        }
        store8<BF16>(dst + off + i, o0);
        store8<BF16>(dst + off + i + H, o1);
    }
}

constexpr int BIN_WG = 64;    // bins per binsum workgroup (one wave)

// Per bin: exclusive prefix over segments; per workgroup of BIN_WG bins: the
// exclusive scan of bin sizes and of 256-row chunk counts, and their totals.
__global__ __launch_bounds__(BIN_WG) void k_attn_binsum(int nbins, int nseg, int NB,
                                                        const int32_t *__restrict__ cnt,
                                                        int32_t *__restrict__ seg_rel,
                                                        int32_t *__restrict__ bin_local,
                                                        int32_t *__restrict__ chunk_local,
                                                        int32_t *__restrict__ wg_sum) {
    const int tid = threadIdx.x;
    const long bin = (long)blockIdx.x * BIN_WG + tid;
    int acc = 0;
    if (bin < nbins) {
        // counts are [b, g][seg][n]: consecutive bins of a wave are adjacent
        const long base = (bin / NB) * nseg * (long)NB + bin % NB;
        const int32_t *c = cnt + base;
        int32_t *o = seg_rel + base;
        int sg = 0;
        for (; sg + 8 <= nseg; sg += 8) {   // eight loads in flight
            int x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = c[(long)(sg + u) * NB];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                o[(long)(sg + u) * NB] = acc;
                acc += x[u];
            }
        }
        for (; sg < nseg; ++sg) {
            const int x = c[(long)sg * NB];
            o[(long)sg * NB] = acc;
            acc += x;
        }
    }
    const int nch = (acc + CHUNK_ROWS - 1) / CHUNK_ROWS;
    // inclusive wave scans of the bin sizes and chunk counts
    int ps = acc, pc = nch;
#pragma unroll
    for (int dlt = 1; dlt < WAVE; dlt <<= 1) {
        const int a = __shfl_up(ps, dlt), c = __shfl_up(pc, dlt);
        if (tid >= dlt) { ps += a; pc += c; }
    }
    if (bin < nbins) {
        bin_local[bin] = ps - acc;
        chunk_local[bin] = pc - nch;
    }
    if (tid == BIN_WG - 1) {
        wg_sum[2 * blockIdx.x] = ps;
        wg_sum[2 * blockIdx.x + 1] = pc;
    }
}

// Exclusive scan of the workgroup totals (one workgroup of 1024 threads,
// each owning a contiguous run); the grand totals go after the last one.
__global__ __launch_bounds__(1024) void k_attn_scan(int nwg, int32_t *__restrict__ wg_sum) {
    __shared__ int32_t ws[16], wc[16];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int per = (nwg + 1023) / 1024;
    const int lo = min(nwg, tid * per), hi = min(nwg, lo + per);
    int s0 = 0, c0 = 0;
    for (int i = lo; i < hi; ++i) {
        s0 += wg_sum[2 * i];
        c0 += wg_sum[2 * i + 1];
    }
    int ps = s0, pc = c0;
#pragma unroll
    for (int dlt = 1; dlt < WAVE; dlt <<= 1) {
        const int a = __shfl_up(ps, dlt), c = __shfl_up(pc, dlt);
        if (lane >= dlt) { ps += a; pc += c; }
    }
    if (lane == WAVE - 1) { ws[wv] = ps; wc[wv] = pc; }
    __syncthreads();
    int bs = 0, bc = 0, ts = 0, tc = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        bs += w < wv ? ws[w] : 0;
        bc += w < wv ? wc[w] : 0;
        ts += ws[w];
        tc += wc[w];
    }
    int rs = bs + ps - s0, rc = bc + pc - c0;
    for (int i = lo; i < hi; ++i) {
        const int a = wg_sum[2 * i], c = wg_sum[2 * i + 1];
        wg_sum[2 * i] = rs;
        wg_sum[2 * i + 1] = rc;
        rs += a;
        rc += c;
    }
    if (tid == 0) {
        wg_sum[2 * nwg] = ts;
        wg_sum[2 * nwg + 1] = tc;
    }
}

// Remote work split: chunk c costs its rows plus CHUNK_OVH (the K/V load and
// synchronization it brings); workgroup w of the persistent grid takes the
// chunks [wg_first[w], wg_first[w + 1]) (written by k_attn_scatter).
constexpr int CHUNK_OVH = 128;
constexpr int MAX_REMOTE_GRID = 8192;   // bound of the remote kernel's persistent grid

__device__ __forceinline__ int bin_start_of(const int32_t *bin_local, const int32_t *wg_base,
                                            long bin) {
    return wg_base[2 * (bin / BIN_WG)] + bin_local[bin];
}

// Workgroup totals the scatter scans itself (into LDS) instead of reading
// the separate scan's result: at most this many (16 KB of LDS).
constexpr int SCATTER_SCAN_MAX = 2048;

// (query, slot) entries per scatter thread: their first loads are issued
// before the workgroup-total scan, and the grid is a quarter as large.
constexpr int SCATTER_EPT = 4;

// Scatter (query, slot) ids into bin order and replace each entry's rank by
// its list position (where its partial state will be written); threads
// below nbins also write their bin's entries of the chunk table.  With
// SCAN, every workgroup first forms the exclusive scan of the binsum
// workgroup totals (wg_sum, nwg pairs) in LDS; else wg_sum already holds it.
// Thread t of workgroup w takes entries (w SCATTER_EPT + k) 256 + t.
template <bool SCAN>
__global__ __launch_bounds__(256) void k_attn_scatter(Shape s, int nseg, int nbins,
                                                      const int32_t *__restrict__ sel,
                                                      int32_t *__restrict__ entry_pos,
                                                      const int32_t *__restrict__ bin_local,
                                                      const int32_t *__restrict__ chunk_local,
                                                      const int32_t *__restrict__ wg_sum,
                                                      const int32_t *__restrict__ seg_rel,
                                                      int32_t *__restrict__ list_q,
                                                      int4 *__restrict__ chunk_desc,
                                                      int grid_r, int32_t *__restrict__ wg_first) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    __shared__ int32_t base_s[SCAN ? 2 * SCATTER_SCAN_MAX + 2 : 1];
    const int32_t *wg_base = wg_sum;
    // this thread's entries: ranks and selections, in flight during the scan
    const long n = (long)s.B * s.Hq * s.T * s.R;
    const long e0 = (long)blockIdx.x * SCATTER_EPT * 256 + threadIdx.x;
    int pos[SCATTER_EPT], sl[SCATTER_EPT];
#pragma unroll
    for (int k = 0; k < SCATTER_EPT; ++k) {
        const long e = e0 + k * 256;
        pos[k] = e < n ? entry_pos[e] : -1;
        sl[k] = e < n ? sel[e] : 0;
    }
    if constexpr (SCAN) {
        // thread t owns totals [t * per, t * per + per); a workgroup scan of
        // its sums places them (same arithmetic as k_attn_scan)
        __shared__ int32_t ws[4], wc[4];
        const int nwg = (nbins + BIN_WG - 1) / BIN_WG;
        const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
        const int per = (nwg + 255) / 256;
        const int lo = min(nwg, tid * per), hi = min(nwg, lo + per);
        int s0 = 0, c0 = 0;
        for (int k = lo; k < hi; ++k) {
            s0 += wg_sum[2 * k];
            c0 += wg_sum[2 * k + 1];
        }
        int ps = s0, pc = c0;
#pragma unroll
        for (int dlt = 1; dlt < WAVE; dlt <<= 1) {
            const int a = __shfl_up(ps, dlt), c = __shfl_up(pc, dlt);
            if (lane >= dlt) { ps += a; pc += c; }
        }
        if (lane == WAVE - 1) { ws[wv] = ps; wc[wv] = pc; }
        __syncthreads();
        int bs = 0, bc = 0, ts = 0, tc = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            bs += w < wv ? ws[w] : 0;
            bc += w < wv ? wc[w] : 0;
            ts += ws[w];
            tc += wc[w];
        }
        int rs = bs + ps - s0, rc = bc + pc - c0;
        for (int k = lo; k < hi; ++k) {
            base_s[2 * k] = rs;
            base_s[2 * k + 1] = rc;
            rs += wg_sum[2 * k];
            rc += wg_sum[2 * k + 1];
        }
        if (tid == 0) {
            base_s[2 * nwg] = ts;
            base_s[2 * nwg + 1] = tc;
        }
        __syncthreads();
        wg_base = base_s;
    }
    if (i < nbins) {
        // descriptors {bin, first row, end row} of the bin's chunks
        const long nb = (long)nbins;
        const int nwg = (int)((nb + BIN_WG - 1) / BIN_WG);
        const int c0 = wg_base[2 * (i / BIN_WG) + 1] + chunk_local[i];
        const int c1 = i + 1 < nb ? wg_base[2 * ((i + 1) / BIN_WG) + 1] + chunk_local[i + 1]
                                  : wg_base[2 * nwg + 1];
        const int b0 = bin_start_of(bin_local, wg_base, i);
        const int b1 = i + 1 < nb ? bin_start_of(bin_local, wg_base, i + 1) : wg_base[2 * nwg];
        // remote work split: chunk c costs its rows plus CHUNK_OVH and spans
        // the cost interval [r0 + OVH c, r1 + OVH (c + 1)); workgroup w starts
        // at the chunk whose interval holds w * total / grid_r
        const long rows = wg_base[2 * nwg], nchunks = wg_base[2 * nwg + 1];
        const long total = rows + (long)CHUNK_OVH * nchunks;
        if (i == 0 && nchunks == 0)
            for (int w = 0; w <= grid_r; ++w) wg_first[w] = 0;
        for (int c = c0; c < c1; ++c) {
            const int r0 = b0 + (c - c0) * CHUNK_ROWS, r1 = min(r0 + CHUNK_ROWS, b1);
            chunk_desc[c] = make_int4((int)i, r0, r1, 0);
            const long pst = r0 + (long)CHUNK_OVH * c, pen = r1 + (long)CHUNK_OVH * (c + 1);
            const long w_lo = (pst * grid_r + total - 1) / total, w_hi = (pen * grid_r - 1) / total;
            for (long w = w_lo; w <= w_hi; ++w) wg_first[w] = c;
            if (c == nchunks - 1) wg_first[grid_r] = (int)nchunks;
        }
    }
    // every entry's bin start and segment offset in one batch, then the writes
    int bl[SCATTER_EPT], sg[SCATTER_EPT], qrow[SCATTER_EPT];
    long bin[SCATTER_EPT];
#pragma unroll
    for (int k = 0; k < SCATTER_EPT; ++k) {
        const long e = e0 + k * 256;
        const long route = (pos[k] >= 0 ? e : 0) / s.R;
        const int t = (int)(route % s.T);
        const int h = (int)((route / s.T) % s.Hq), b = (int)(route / ((long)s.T * s.Hq));
        bin[k] = ((long)b * s.Hkv + h / s.G) * s.NB + (pos[k] >= 0 ? sl[k] : 0);
        const long sr = ((bin[k] / s.NB) * nseg + t / SEG) * (long)s.NB + bin[k] % s.NB;
        bl[k] = bin_local[bin[k]];
        sg[k] = seg_rel[sr];
        qrow[k] = (int32_t)(((long)b * s.T + t) * s.Hq + h);   // row of q_rot
    }
#pragma unroll
    for (int k = 0; k < SCATTER_EPT; ++k) {
        if (pos[k] < 0) continue;
        const int at = wg_base[2 * (bin[k] / BIN_WG)] + bl[k] + sg[k] + pos[k];
        list_q[at] = qrow[k];
        entry_pos[e0 + k * 256] = at;                            // where its partial will be
    }
}

// Persistent over a contiguous range of chunks.  Every wave walks its tasks
// (16-row groups: group `wave`, `wave` + 4, ... of each chunk, possibly an
// idle one) as one sequence across chunk boundaries: the list entry of the
// task after next and the query rows of the next task are in flight while a
// task computes.  The next chunk's K / V^T (if its bin differs) is staged in
// registers during the current chunk and written to LDS after it.
template <int D, int BETA, bool BF16>
// bf16: capped at 256 registers (two waves per SIMD; the d = 128 kernels
// would otherwise take one)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BF16 ? 2 : 1)))
void k_attn_remote(Shape s, const Elem<BF16> *__restrict__ q_rot,
                   const Elem<BF16> *__restrict__ k_rot, const Elem<BF16> *__restrict__ v,
                   const int32_t *__restrict__ list_q, const int4 *__restrict__ chunk_desc,
                   const int32_t *__restrict__ wg_first, Elem<BF16> *__restrict__ part_o) {
    using T = Tile<D, BF16>;
    using E = Elem<BF16>;
    constexpr int NSUB = BETA / 64;
    extern __shared__ __align__(16) unsigned char smem[];
    E *Ks = reinterpret_cast<E *>(smem);               // NSUB x [64][QS]
    E *Vts = Ks + NSUB * T::K_ELEMS;                    // NSUB x [D][VS]

    const int c_beg = wg_first[blockIdx.x], c_end = wg_first[blockIdx.x + 1];
    if (c_beg >= c_end) return;
    const int T_ = s.T, Hkv = s.Hkv, NB = s.NB;
    const int lane = lane_id(), wave = threadIdx.x / WAVE, lr = lane & 15, lg = lane >> 4;
    auto desc_at = [&](int c) { return c < c_end ? chunk_desc[c] : make_int4(-1, 0, 0, 0); };
    auto ngroups = [&](const int4 &d) { return d.x < 0 ? 0 : (d.z - d.y + 15) / 16; };
    // this lane's row of group grp of a chunk, or -1
    auto row_of = [&](const int4 &d, int grp) {
        const int row = d.y + grp * 16 + lr;
        return (d.x >= 0 && row < d.z) ? row : -1;
    };
    RowStager<D, BF16> ks[NSUB];
    typename VtStagerOf<D, BF16>::type vs[NSUB];
    auto kv_issue = [&](int bin) {
        const int n = bin % NB, g = (bin / NB) % Hkv, b = bin / (NB * Hkv);
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) {
            const int tb = n * BETA + sub * 64;
            ks[sub].issue(k_rot, [&](int r, size_t &off) {
                off = (((size_t)b * T_ + tb + r) * Hkv + g) * D;
                return true;
            });
            vs[sub].issue(v, (((size_t)b * T_ + tb) * Hkv + g) * D, (size_t)Hkv * D);
        }
    };
    auto kv_commit = [&]() {
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) {
            ks[sub].commit(Ks + sub * T::K_ELEMS);
            vs[sub].commit(Vts + sub * T::V_ELEMS);
        }
    };

    int4 dcur = desc_at(c_beg), dnext = desc_at(c_beg + 1), dnn = desc_at(c_beg + 2);
    // task pipeline: Q of the current task, list entry of the next one
    int row_cur = row_of(dcur, wave);
    QFrags<D, BF16> qcur;
    qcur.issue(q_rot, row_cur >= 0 ? (size_t)list_q[row_cur] * D : 0, row_cur >= 0);
    int row_nx;
    {
        const bool same = wave + 4 < ngroups(dcur);
        row_nx = same ? row_of(dcur, wave + 4) : row_of(dnext, wave);
    }
    int q_nx = row_nx >= 0 ? list_q[row_nx] : 0;
    kv_issue(dcur.x);
    kv_commit();
    __syncthreads();

    for (int c = c_beg; c < c_end; ++c) {
        const bool stage = dnext.x >= 0 && dnext.x != dcur.x;
        if (stage) kv_issue(dnext.x);   // in flight during this chunk
        const int ng = ngroups(dcur), ng1 = ngroups(dnext);
        for (int grp = wave;; grp += 4) {
            Frag8<BF16> qf[D / 32];
            qcur.get(qf);
            const int row_now = row_cur;
            // next task: grp + 4 of this chunk, else group `wave` of the next
            const bool in_chunk = grp + 4 < ng;
            const int row1 = row_nx;
            if (row1 >= 0) qcur.issue(q_rot, (size_t)q_nx * D, true);
            // the task after next
            int row2;
            if (in_chunk) row2 = grp + 8 < ng ? row_of(dcur, grp + 8) : row_of(dnext, wave);
            else row2 = wave + 4 < ng1 ? row_of(dnext, wave + 4) : row_of(dnn, wave);
            const int q2 = row2 >= 0 ? list_q[row2] : 0;
            if (grp < ng) {   // wave-uniform: the group exists
                f32x4 o[D / 16];
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
                float m = -INFINITY, l = 0.0f;
                attend64<D, BF16, false, true>(qf, Ks, Vts, 0, 0, o, m, l);
                if constexpr (NSUB > 1)
                    attend64<D, BF16, false, false>(qf, Ks + T::K_ELEMS, Vts + T::V_ELEMS, 0, 0, o,
                                                    m, l);
                if (row_now >= 0) {
                    const float inv = 1.0f / l;
                    float x[D / 16][4];
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[dt][r] = o[dt][r] * inv;
                    PartChunks<D, BF16> pc;
                    pc.pack(x);
                    pc.embed(m + __builtin_amdgcn_logf(l), lg);   // base-2 log-sum-exp
                    pc.store(part_o + (size_t)row_now * D, lg);
                }
            }
            row_cur = row1;
            row_nx = row2;
            q_nx = q2;
            if (!in_chunk) break;
        }
        __syncthreads();   // every wave is done with this chunk's K / V^T
        if (stage) {
            kv_commit();
            __syncthreads();
        }
        dcur = dnext;
        dnext = dnn;
        dnn = desc_at(c + 3);
    }
}

template <int D, int BETA, bool BF16>
// bf16: capped at 256 registers (two waves per SIMD; the d = 128 kernels
// would otherwise take one)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BF16 ? 2 : 1)))
void k_attn_local(Shape s, const Elem<BF16> *__restrict__ q_rot,
                  const Elem<BF16> *__restrict__ k_rot, const Elem<BF16> *__restrict__ v,
                  const int32_t *__restrict__ sel, const int32_t *__restrict__ tile_flag,
                  const int32_t *__restrict__ entry_pos,
                  const Elem<BF16> *__restrict__ part_o, Elem<BF16> *__restrict__ out) {
    using T = Tile<D, BF16>;
    using E = Elem<BF16>;
    extern __shared__ __align__(16) unsigned char smem[];
    E *Ks = reinterpret_cast<E *>(smem);
    E *Vt = Ks + T::K_ELEMS;
    E *Ostg = Vt + T::V_ELEMS;                               // 4 waves x [16][D + 16 B]
    int *blk_s = reinterpret_cast<int *>(Ostg + 4 * 16 * (D + 16 / sizeof(E)));  // [R]

    const int ntt = s.T / 64;
    // each workgroup walks a contiguous run of items: the tiles of one
    // (batch, head), latest first.  A tile's local blocks are attended latest
    // first, so the last key sub-tile of one tile is usually the first of the
    // next one; it stays in LDS (resident_bh / resident_kb) and is not loaded
    // again.
    const int nitems = s.B * s.Hq * ntt;
    const int per = (nitems + gridDim.x - 1) / gridDim.x;
    const int i_beg = blockIdx.x * per, i_end = min(nitems, i_beg + per);
    int resident_bh = -1, resident_kb = -1;
    const int lane = lane_id(), wave = threadIdx.x / WAVE, lr = lane & 15, lg = lane >> 4;
    const int R = s.R;

    // Merge inputs of this lane's query for the first RP slots, one tile
    // ahead: entry positions are fetched when the previous tile starts, the
    // partial rows (which carry their log-sum-exps) when its output is
    // stored, so they land during this tile's attention; the merge reads them
    // where they were loaded (o_n).  (Prep leaves every slot of a uniform
    // tile at -1, so no tile flag is needed.)
    constexpr int RP = 2;
    constexpr int RX = 6;   // further slots merged two rows at a time (R <= RP + RX)
    int ep_c[RP], ep_n[RP];
    PartChunks<D, BF16> o_n[RP];
    auto fetch_ep = [&](int it) {
        const long rt = it < i_end ? (long)(it / ntt) * s.T + (ntt - 1 - it % ntt) * 64 +
                                         wave * 16 + lr
                                   : 0;
#pragma unroll
        for (int r = 0; r < RP; ++r) ep_n[r] = (it < i_end && r < R) ? entry_pos[rt * R + r] : -1;
    };
    auto fetch_part = [&]() {
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            if (ep_n[r] >= 0) o_n[r].load(part_o + (size_t)ep_n[r] * D, lg);
            else o_n[r].zero();
        }
    };
    auto advance = [&]() {
#pragma unroll
        for (int r = 0; r < RP; ++r) ep_c[r] = ep_n[r];
    };
    // this lane's query row of tile `it`, issued one tile ahead
    auto q_at = [&](int it) {
        const int bh_ = it / ntt, tt_ = ntt - 1 - it % ntt;
        return (((size_t)(bh_ / s.Hq) * s.T + tt_ * 64 + wave * 16 + lr) * s.Hq + bh_ % s.Hq) * D;
    };
    QFrags<D, BF16> qst, qst_n;
    qst_n.issue(q_rot, i_beg < i_end ? q_at(i_beg) : 0, i_beg < i_end);
    fetch_ep(i_beg);
    fetch_part();
    advance();
    for (int item = i_beg; item < i_end; ++item) {
    __syncthreads();   // the previous item is done with LDS
    const int tt = ntt - 1 - item % ntt;
    const int bh = item / ntt;
    const int h = bh % s.Hq, b = bh / s.Hq, g = h / s.G;
    const int t0 = tt * 64, qb = t0 / BETA, L = s.L;
    const int T_ = s.T, Hkv = s.Hkv, Hq = s.Hq;
    const long tile = (long)bh * ntt + tt;
    const bool uni = tile_flag[tile] != 0;
    const long route0 = (long)bh * T_ + t0;

    const int tq = t0 + wave * 16 + lr;  // this lane's query position
    qst = qst_n;                          // landed during the previous tile
    qst_n.issue(q_rot, item + 1 < i_end ? q_at(item + 1) : 0, item + 1 < i_end);
    const long route = route0 + wave * 16 + lr;
    fetch_ep(item + 1);   // the next tile's entry positions, in flight
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

    f32x4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.0f;

    // work items: (block, 64-key sub-tile): the local blocks latest first
    // (sub-tiles latest first), then the shared remote blocks; sub-tiles after
    // the tile's last query are skipped
    const int nrem = uni ? R : 0;
    const int lo_blk = max(0, qb - L + 1);
    const int nloc = qb - lo_blk + 1;
    const int nblk = nloc + nrem;
    auto item_key0 = [&](int j, int sub) {   // first key of item, or -1 if absent
        const int blk = j < nloc ? qb - j : blk_s[j - nloc];
        if (blk < 0) return -1;
        const int kb0 = blk * BETA + (j < nloc ? BETA / 64 - 1 - sub : sub) * 64;
        return kb0 > t0 + 63 ? -1 : kb0;
    };
    auto next_item = [&](int &j, int &sub) {   // advance to the next present item
        for (;;) {
            if (++sub == BETA / 64) { sub = 0; ++j; }
            if (j >= nblk || item_key0(j, sub) >= 0) return;
        }
    };
    int j = 0, sub = 0;
    if (nblk > 0 && item_key0(0, 0) < 0) next_item(j, sub);
    RowStager<D, BF16> kst;
    typename VtStagerOf<D, BF16>::type vst;
    auto issue_kv = [&](int kb0) {
        kst.issue(k_rot, [&](int r, size_t &off) {
            off = (((size_t)b * T_ + kb0 + r) * Hkv + g) * D;
            return true;
        });
        vst.issue(v, (((size_t)b * T_ + kb0) * Hkv + g) * D, (size_t)Hkv * D);
    };
    int kb_cur = j < nblk ? item_key0(j, sub) : -1;
    const bool reuse = kb_cur >= 0 && bh == resident_bh && kb_cur == resident_kb;
    if (kb_cur >= 0 && !reuse) issue_kv(kb_cur);
    Frag8<BF16> qf[D / 32];
    qst.get(qf);
    if (kb_cur >= 0 && !reuse) {
        kst.commit(Ks);
        vst.commit(Vt);
    }
    if (kb_cur >= 0) {
        resident_bh = bh;
        resident_kb = kb_cur;
    }
    __syncthreads();
    while (kb_cur >= 0) {
        int jn = j, sn = sub;
        next_item(jn, sn);
        const int kb_next = jn < nblk ? item_key0(jn, sn) : -1;
        if (kb_next >= 0) issue_kv(kb_next);   // in flight during this compute
        attend64<D, BF16, true, false>(qf, Ks, Vt, kb_cur, tq, o, m, l);
        __syncthreads();
        if (kb_next >= 0) {
            kst.commit(Ks);
            vst.commit(Vt);
            __syncthreads();
        }
        if (kb_next >= 0) {
            resident_bh = bh;
            resident_kb = kb_next;
        }
        j = jn;
        sub = sn;
        kb_cur = kb_next;
    }

    // merge: local (and shared) part, then the remote partials in slot order
    const float lse = m + __builtin_amdgcn_logf(l);
    const float inv = 1.0f / l;
    float acc[D / 16][4];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][r] = o[dt][r] * inv;
    if (!uni) {
        // the prefetched slots' log-sum-exps, from their rows (the exchange
        // between a row's lanes runs before any per-lane branch)
        float lse_p[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) lse_p[r] = o_n[r].lse(lg);
        float M = lse;
#pragma unroll
        for (int r = 0; r < RP; ++r)
            if (r < R && ep_c[r] >= 0) M = fmaxf(M, lse_p[r]);
        float wsum = __builtin_amdgcn_exp2f(lse - M);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[dt][r] *= wsum;
#pragma unroll
        for (int r = 0; r < RP; ++r) {   // prefetched slots (static indexes)
            if (r >= R || ep_c[r] < 0) continue;
            const float w = __builtin_amdgcn_exp2f(lse_p[r] - M);
            wsum += w;
            float x[D / 16][4];
            o_n[r].unpack(x);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[dt][rr] += w * x[dt][rr];
        }
        // slots RP .. R-1, in slot order: their rows come from global memory
        // (loads clamped to entry 0) and bring their log-sum-exps, so these
        // merge online (the running maximum rises as needed; a slot that
        // does not raise it rescales by exactly 1)
        auto add_slot = [&](float lu, const PartChunks<D, BF16> &pc) {
            const float Mn = fmaxf(M, lu);
            const float sc = __builtin_amdgcn_exp2f(M - Mn), w = __builtin_amdgcn_exp2f(lu - Mn);
            wsum = wsum * sc + w;
            float x[D / 16][4];
            pc.unpack(x);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[dt][rr] = acc[dt][rr] * sc + w * x[dt][rr];
            M = Mn;
        };
        const int32_t *ep = entry_pos + route * R;
        if (R > RP && R <= RP + RX) {
            // entry positions in one batch, then the rows two at a time
            int ex[RX];
#pragma unroll
            for (int x = 0; x < RX; ++x) ex[x] = RP + x < R ? ep[RP + x] : -1;
#pragma unroll
            for (int x0 = 0; x0 < RX; x0 += 2) {
                if (__ballot(ex[x0] >= 0 || (x0 + 1 < RX && ex[x0 + 1] >= 0)) == 0ull) continue;
                PartChunks<D, BF16> pc[2];
                float lu[2];
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    if (x0 + u < RX) pc[u].load(part_o + (size_t)max(ex[x0 + u], 0) * D, lg);
#pragma unroll
                for (int u = 0; u < 2; ++u) lu[u] = x0 + u < RX ? pc[u].lse(lg) : 0.0f;
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    if (x0 + u < RX && ex[x0 + u] >= 0) add_slot(lu[u], pc[u]);
            }
        } else {
            for (int r = RP; r < R; ++r) {
                const int e = ep[r];
                PartChunks<D, BF16> pc;
                pc.load(part_o + (size_t)max(e, 0) * D, lg);
                const float lu = pc.lse(lg);
                if (e >= 0) add_slot(lu, pc);
            }
        }
        const float iw = 1.0f / wsum;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[dt][r] *= iw;
    }
    // output rows through the wave's LDS staging area, so that each lane
    // stores 16 contiguous bytes and a store instruction covers 64 bytes of
    // each of the wave's 16 rows
    {
        constexpr int VE = 16 / sizeof(E);           // elements per 16 bytes
        constexpr int OS = D + VE;                   // staging row stride (elements)
        E *stg = Ostg + wave * 16 * OS;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) store4(stg + lr * OS + dt * 16 + 4 * lg, acc[dt]);
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        const int rr = lane >> 2, qq = lane & 3;
        E *orow = out + (((size_t)b * T_ + t0 + wave * 16 + rr) * Hq + h) * D;
#pragma unroll
        for (int j = 0; j < D / (4 * VE); ++j) {
            const int d0 = j * 4 * VE + qq * VE;
            *reinterpret_cast<u32x4 *>(orow + d0) =
                *reinterpret_cast<const u32x4 *>(stg + rr * OS + d0);
        }
    }
    fetch_part();   // the next tile's partial states, in flight during its attention
    advance();
    }
}

// ---------------------------------------------------------------------------
// Dense causal attention: every query attends to every key at or before it.
// The news page calls a comparison against optimized FlashAttention-style
// dense kernels necessary (section "The 99.35 Percent Result Does Not
// Establish Language Quality") and asks for a GPU benchmark that counts the
// routing and index costs (section "What Sparse-Attention Researchers Should
// Watch Next"); this is the dense side of that comparison, on the same
// rotation pass and tile layouts as the selected-set kernels.

// Max of a lane's value and those of the lanes 16, 32 and 48 away:
// the four lanes that hold one query's scores in the MFMA output layout.
__device__ __forceinline__ float quad_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Largest growth (log2 units) of a row's maximum that is absorbed without
// rescaling: probabilities stay below 2^8 and the running sums far from
// overflow; the result does not depend on when rescaling happens beyond
// rounding.
constexpr float DENSE_SLACK = 8.0f;

// One wave, NG groups of 16 queries (qf[g]: B fragments of Q^T as in
// attend64) against 64 keys; each K and V^T fragment read from LDS serves
// every group.  The running state is kept against a reference maximum m
// that is only raised when a row's scores exceed it by more than
// DENSE_SLACK: the score accumulators start at -m, so the logits come out of
// the MFMA already shifted, and the output is rescaled only on those rare
// tiles (decided per wave).  The row sums come from the MFMA too: P times an
// all-ones 16-row block leaves the sum over the tile's keys (of the same
// rounded P that multiplies V) in every element of l[g].  FIRST: the state is
// empty and m is set to the tile's row maximum (every row sees key 0 on its
// first tile).  MASK: keys after a lane's query (qlim[g]) are masked.
template <int D, bool BF16, bool MASK, bool FIRST, int NG>
__device__ __forceinline__ void dense_tile(const Frag8<BF16> (&qf)[NG][D / 32],
                                           const Elem<BF16> *Ks, const Elem<BF16> *Vt, int key0,
                                           const int (&qlim)[NG], f32x4 (&o)[NG][D / 16],
                                           float (&m)[NG], f32x4 (&l)[NG]) {
    using T = Tile<D, BF16>;
    const int lane = lane_id(), lr = lane & 15, lg = lane >> 4;
    f32x4 st[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float init = FIRST ? 0.0f : -m[g];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) st[g][mt] = f32x4{init, init, init, init};
    }
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const Frag8<BF16> kf = lds_frag8(Ks + (mt * 16 + lr) * T::QS + 32 * c + 8 * lg);
#pragma unroll
            for (int g = 0; g < NG; ++g) mma32(st[g][mt], kf, qf[g][c]);
        }
    }
    float mx[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float x = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (MASK) {
                    const int key = key0 + mt * 16 + 4 * lg + r;
                    st[g][mt][r] = key <= qlim[g] ? st[g][mt][r] : -INFINITY;
                }
                x = fmaxf(x, st[g][mt][r]);
            }
        }
        mx[g] = quad_max(x);
    }
    if constexpr (FIRST) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            m[g] = mx[g];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) st[g][mt] -= mx[g];
        }
    } else {
        bool grow = false;
#pragma unroll
        for (int g = 0; g < NG; ++g) grow = grow || mx[g] > DENSE_SLACK;
        if (__ballot(grow) != 0ull) {   // raise the reference of every row that grew
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float up = fmaxf(mx[g], 0.0f);   // a fully masked row has mx = -inf
                const float alpha = __builtin_amdgcn_exp2f(-up);
                m[g] += up;
                l[g] *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) o[g][dt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) st[g][mt] -= up;
            }
        }
    }
    Frag8<BF16> pf[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float p[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p[mt][r] = __builtin_amdgcn_exp2f(st[g][mt][r]);   // exp2(-inf) = 0
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const float pv[8] = {p[2 * c][0], p[2 * c][1], p[2 * c][2], p[2 * c][3],
                                 p[2 * c + 1][0], p[2 * c + 1][1], p[2 * c + 1][2], p[2 * c + 1][3]};
            pf[g][c] = reg_frag8<BF16>(pv);
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            // bf16 V^T tiles are stored swizzled (VtStagerPacked)
            const int sw = BF16 ? 8 * dt : 0;
            const Elem<BF16> *vr = Vt + (dt * 16 + lr) * T::VS;
            const Frag8<BF16> vf = lds_frag4x2(vr + ((32 * c + 4 * lg) ^ sw),
                                               vr + ((32 * c + 16 + 4 * lg) ^ sw));
#pragma unroll
            for (int g = 0; g < NG; ++g) mma32(o[g][dt], vf, pf[g][c]);
        }
        const float one[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
        const Frag8<BF16> ones = reg_frag8<BF16>(one);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (FIRST && c == 0) l[g] = f32x4{0.f, 0.f, 0.f, 0.f};
            mma32(l[g], ones, pf[g][c]);
        }
    }
}

constexpr int DENSE_NG = 2;                      // 16-query groups per wave
constexpr int DENSE_ROWS = 4 * 16 * DENSE_NG;    // queries per workgroup (4 waves)

template <int D, bool BF16>
constexpr size_t dense_lds_bytes() {
    return (size_t)2 * (Tile<D, BF16>::K_ELEMS + Tile<D, BF16>::V_ELEMS) * sizeof(Elem<BF16>);
}

// One workgroup per (batch, q-head, DENSE_ROWS-query tile).  Key tiles of 64
// are visited in ascending order through two LDS buffers: the next tile's
// loads are issued into registers before the current tile's compute and
// written to the other buffer after it, one barrier per tile.  The tiles
// that reach past a wave's first query take the causal mask; tiles wholly
// after a wave's last query are skipped by that wave.  Work items are dealt
// so that each XCD runs whole heads, heaviest (latest) tiles first: the
// workgroups of one head sweep its keys from the start at about the same
// pace and share them in that XCD's L2.
template <int D, bool BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void k_dense(Shape s, const Elem<BF16> *__restrict__ q_rot,
                                               const Elem<BF16> *__restrict__ k_rot,
                                               const Elem<BF16> *__restrict__ v,
                                               Elem<BF16> *__restrict__ out) {
    using T = Tile<D, BF16>;
    using E = Elem<BF16>;
    constexpr int NG = DENSE_NG;
    extern __shared__ __align__(16) unsigned char smem[];
    E *buf = reinterpret_cast<E *>(smem);        // 2 x [K tile | V^T tile]
    constexpr int BUF = T::K_ELEMS + T::V_ELEMS;

    const int T_ = s.T, Hq = s.Hq, Hkv = s.Hkv;
    const int ntq = (T_ + DENSE_ROWS - 1) / DENSE_ROWS;
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = item / ntq, tq = ntq - 1 - item % ntq;
    const int h = bh % Hq, b = bh / Hq, g = h / s.G;
    const int q0 = tq * DENSE_ROWS;
    const int nkt = min(T_, q0 + DENSE_ROWS) / 64;   // key tiles 0 .. nkt-1 (T % 64 == 0)
    const int lane = lane_id(), wave = threadIdx.x / WAVE, lr = lane & 15, lg = lane >> 4;
    const int w0 = q0 + wave * 16 * NG;              // the wave's first query
    const bool wave_rows = w0 < T_;                  // T % 64 == 0: all or none of its rows

    int qlim[NG];
    QFrags<D, BF16> qst[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        qlim[gi] = w0 + gi * 16 + lr;
        qst[gi].issue(q_rot, (((size_t)b * T_ + qlim[gi]) * Hq + h) * D, wave_rows);
    }
    RowStager<D, BF16> kst;
    typename VtStagerOf<D, BF16>::type vst;
    auto issue_kv = [&](int kt) {
        const int kb0 = kt * 64;
        kst.issue(k_rot, [&](int r, size_t &off) {
            off = (((size_t)b * T_ + kb0 + r) * Hkv + g) * D;
            return true;
        });
        vst.issue(v, (((size_t)b * T_ + kb0) * Hkv + g) * D, (size_t)Hkv * D);
    };
    issue_kv(0);
    Frag8<BF16> qf[NG][D / 32];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) qst[gi].get(qf[gi]);
    kst.commit(buf);
    vst.commit(buf + T::K_ELEMS);
    __syncthreads();

    f32x4 o[NG][D / 16], l[NG];
    float m[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        m[gi] = 0.0f;
        l[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[gi][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // key tile 0: every wave with rows takes it first (it holds key 0)
    if (nkt > 1) issue_kv(1);
    if (wave_rows) {
        if (63 > w0) dense_tile<D, BF16, true, true, NG>(qf, buf, buf + T::K_ELEMS, 0, qlim, o, m, l);
        else dense_tile<D, BF16, false, true, NG>(qf, buf, buf + T::K_ELEMS, 0, qlim, o, m, l);
    }
    if (nkt > 1) {
        kst.commit(buf + BUF);
        vst.commit(buf + BUF + T::K_ELEMS);
    }
    __syncthreads();
    for (int kt = 1; kt < nkt; ++kt) {
        if (kt + 1 < nkt) issue_kv(kt + 1);    // in flight during this tile's compute
        const E *Ks = buf + (kt & 1) * BUF;
        const int key0 = kt * 64;
        if (wave_rows && key0 <= w0 + 16 * NG - 1) {
            if (key0 + 63 > w0)
                dense_tile<D, BF16, true, false, NG>(qf, Ks, Ks + T::K_ELEMS, key0, qlim, o, m, l);
            else
                dense_tile<D, BF16, false, false, NG>(qf, Ks, Ks + T::K_ELEMS, key0, qlim, o, m, l);
        }
        if (kt + 1 < nkt) {
            E *nb = buf + ((kt + 1) & 1) * BUF;   // last read in the previous tile
            kst.commit(nb);
            vst.commit(nb + T::K_ELEMS);
        }
        __syncthreads();
    }
    if (!wave_rows) return;
    // output rows through a staging area in the wave's share of buffer 0 (the
    // barrier after the last tile ends every read of it): each lane stores 16
    // contiguous bytes, a store instruction covers 64 bytes of 16 rows
    constexpr int VE = 16 / sizeof(E);
    constexpr int OS = D + VE;
    static_assert(4 * 16 * OS <= 2 * BUF, "staging fits in the tile buffers");
    E *stg = buf + wave * 16 * OS;
    const int rr = lane >> 2, qq = lane & 3;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const float inv = 1.0f / l[gi][0];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const float x[4] = {o[gi][dt][0] * inv, o[gi][dt][1] * inv, o[gi][dt][2] * inv,
                                o[gi][dt][3] * inv};
            store4(stg + lr * OS + dt * 16 + 4 * lg, x);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        E *orow = out + (((size_t)b * T_ + w0 + gi * 16 + rr) * Hq + h) * D;
#pragma unroll
        for (int j = 0; j < D / (4 * VE); ++j) {
            const int d0 = j * 4 * VE + qq * VE;
            *reinterpret_cast<u32x4 *>(orow + d0) =
                *reinterpret_cast<const u32x4 *>(stg + rr * OS + d0);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);          // reads done before the next group's writes
        __builtin_amdgcn_wave_barrier();
    }
}

template <typename F>
hipError_t ensure_lds(F *fn, size_t bytes) {
    return mono_lds_limit(reinterpret_cast<const void *>(fn), bytes);
}

// Workgroups for a persistent launch: as many as fit on the device at once
// (occupancy of `fn` at 256 threads and `lds` bytes), at most `items`.
template <typename F>
unsigned persistent_grid(F *fn, size_t lds, long items) {
    const long g = mono_resident_workgroups(reinterpret_cast<const void *>(fn), 256, lds);
    return (unsigned)std::max(1L, std::min(items, g));
}

struct AttnWs {
    int32_t *cnt, *seg_rel, *bin_local, *chunk_local, *wg_sum, *tile_flag, *entry_pos, *list_q,
        *wg_first;
    int4 *chunk_desc;
    void *part_o, *q_rot, *k_rot;
};

int num_segments(const Shape &s) { return (s.T + SEG - 1) / SEG; }

long max_chunks(const Shape &s) {
    const long nbins = (long)s.B * s.Hkv * s.NB;
    const long nent = (long)s.B * s.Hq * s.T * s.R;
    return nbins + (nent + CHUNK_ROWS - 1) / CHUNK_ROWS;
}

template <int D, int BETA, bool BF16>
hipError_t run_attention(const Shape &s, const void *q, const void *k, const void *v,
                         const float *cos_t, const float *sin_t, const int32_t *sel, void *out,
                         const AttnWs &w, hipStream_t st, bool prerotated) {
    using T = Tile<D, BF16>;
    using E = Elem<BF16>;
    const int nbins = s.B * s.Hkv * s.NB;
    const int nseg = num_segments(s);
    const int nwg = (nbins + BIN_WG - 1) / BIN_WG;
    const long ntiles = (long)s.B * s.Hq * (s.T / 64);
    const long nent = (long)s.B * s.Hq * s.T * s.R;
    if (!prerotated) {
        const long rot_tasks = (long)s.B * s.T * (s.Hq + s.Hkv) * (D / 16);
        k_attn_rotate<D, BF16><<<dim3((unsigned)std::min<long>((rot_tasks + 255) / 256, 65536L)),
                                 256, 0, st>>>(s, q, k, cos_t, sin_t,
                                               reinterpret_cast<E *>(w.q_rot),
                                               reinterpret_cast<E *>(w.k_rot));
    }
    auto *prep = s.R <= 2 ? k_attn_prep<2> : s.R <= 8 ? k_attn_prep<8>
                                           : s.R <= 16 ? k_attn_prep<16> : k_attn_prep<0>;
    hipError_t err = ensure_lds(prep, (size_t)s.NB * sizeof(int));
    if (err != hipSuccess) return err;
    prep<<<dim3((unsigned)nseg, (unsigned)s.Hkv, (unsigned)s.B), PREP_THREADS,
           (size_t)s.NB * sizeof(int), st>>>(s, sel, w.cnt, w.entry_pos, w.tile_flag, nseg);
    k_attn_binsum<<<dim3((unsigned)nwg), BIN_WG, 0, st>>>(nbins, nseg, s.NB, w.cnt, w.seg_rel,
                                                          w.bin_local, w.chunk_local, w.wg_sum);
    const bool scan_in_scatter = nwg <= SCATTER_SCAN_MAX;
    if (!scan_in_scatter) k_attn_scan<<<1, 1024, 0, st>>>(nwg, w.wg_sum);
    const size_t lds_r = (size_t)((BETA / 64) * (T::K_ELEMS + T::V_ELEMS)) * sizeof(E);
    err = ensure_lds(k_attn_remote<D, BETA, BF16>, lds_r);
    if (err != hipSuccess) return err;
    const unsigned grid_r = std::min<unsigned>(
        persistent_grid(k_attn_remote<D, BETA, BF16>, lds_r, max_chunks(s)), MAX_REMOTE_GRID);
    // threads: one per SCATTER_EPT entries, and at least one per bin
    const long nscat = std::max<long>((nent + SCATTER_EPT - 1) / SCATTER_EPT, nbins);
    auto *scatter = scan_in_scatter ? k_attn_scatter<true> : k_attn_scatter<false>;
    scatter<<<dim3((unsigned)((nscat + 255) / 256)), 256, 0, st>>>(
        s, nseg, nbins, sel, w.entry_pos, w.bin_local, w.chunk_local, w.wg_sum, w.seg_rel,
        w.list_q, w.chunk_desc, (int)grid_r, w.wg_first);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    k_attn_remote<D, BETA, BF16><<<dim3(grid_r), 256, lds_r, st>>>(
        s, reinterpret_cast<const E *>(w.q_rot), reinterpret_cast<const E *>(w.k_rot),
        reinterpret_cast<const E *>(v), w.list_q, w.chunk_desc, w.wg_first,
        reinterpret_cast<E *>(w.part_o));
    const size_t lds_l = (size_t)(T::K_ELEMS + T::V_ELEMS + 4 * 16 * (D + 16 / sizeof(E))) *
                             sizeof(E) + (size_t)s.R * sizeof(int);
    err = ensure_lds(k_attn_local<D, BETA, BF16>, lds_l);
    if (err != hipSuccess) return err;
    const unsigned grid_l = persistent_grid(k_attn_local<D, BETA, BF16>, lds_l, ntiles);
    k_attn_local<D, BETA, BF16><<<dim3(grid_l), 256, lds_l, st>>>(
        s, reinterpret_cast<const E *>(w.q_rot), reinterpret_cast<const E *>(w.k_rot),
        reinterpret_cast<const E *>(v), sel, w.tile_flag, w.entry_pos,
        reinterpret_cast<const E *>(w.part_o), reinterpret_cast<E *>(out));
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t run_dense(const Shape &s, const void *q, const void *k, const void *v,
                     const float *cos_t, const float *sin_t, void *out, void *q_rot, void *k_rot,
                     hipStream_t st) {
    using E = Elem<BF16>;
    const long rot_tasks = (long)s.B * s.T * (s.Hq + s.Hkv) * (D / 16);
    k_attn_rotate<D, BF16><<<dim3((unsigned)std::min<long>((rot_tasks + 255) / 256, 65536L)), 256, 0,
                             st>>>(s, q, k, cos_t, sin_t, reinterpret_cast<E *>(q_rot),
                                   reinterpret_cast<E *>(k_rot));
    const size_t lds = dense_lds_bytes<D, BF16>();
    hipError_t err = ensure_lds(k_dense<D, BF16>, lds);
    if (err != hipSuccess) return err;
    const long items = (long)s.B * s.Hq * ((s.T + DENSE_ROWS - 1) / DENSE_ROWS);
    k_dense<D, BF16><<<dim3((unsigned)items), 256, lds, st>>>(
        s, reinterpret_cast<const E *>(q_rot), reinterpret_cast<const E *>(k_rot),
        reinterpret_cast<const E *>(v), reinterpret_cast<E *>(out));
    return hipGetLastError();
}

}  // namespace

// Workspace layout of the dense call: rotated q, rotated k.
size_t dense_ws_layout(const Shape &s, size_t *off) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t esz = s.dtype == 1 ? 2 : 4;
    size_t p = 0;
    off[0] = p; p = al(p + (size_t)s.B * s.T * s.Hq * s.d * esz);
    off[1] = p; p = al(p + (size_t)s.B * s.T * s.Hkv * s.d * esz);
    return p;
}

hipError_t launch_dense(const Shape &s, const void *q, const void *k, const void *v,
                        const float *cos_t, const float *sin_t, void *out, void *ws,
                        hipStream_t st) {
    size_t off[2];
    dense_ws_layout(s, off);
    unsigned char *base = reinterpret_cast<unsigned char *>(ws);
    void *qr = base + off[0], *kr = base + off[1];
    const bool bf = s.dtype == 1;
    if (s.d == 64)
        return bf ? run_dense<64, true>(s, q, k, v, cos_t, sin_t, out, qr, kr, st)
                  : run_dense<64, false>(s, q, k, v, cos_t, sin_t, out, qr, kr, st);
    return bf ? run_dense<128, true>(s, q, k, v, cos_t, sin_t, out, qr, kr, st)
              : run_dense<128, false>(s, q, k, v, cos_t, sin_t, out, qr, kr, st);
}

// Workspace layout of the attention call (byte offsets, 256-aligned).
size_t attention_ws_layout(const Shape &s, size_t *off) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t nbins = (size_t)s.B * s.Hkv * s.NB;
    const size_t nseg = (size_t)num_segments(s);
    const size_t nwg = (nbins + BIN_WG - 1) / BIN_WG;
    const size_t ntiles = (size_t)s.B * s.Hq * (s.T / 64);
    const size_t nent = (size_t)s.B * s.Hq * s.T * s.R;
    const size_t esz = s.dtype == 1 ? 2 : 4;
    size_t p = 0;
    off[0] = p; p = al(p + nbins * nseg * 4);                 // per-segment bin counts
    off[1] = p; p = al(p + nbins * nseg * 4);                 // segment offsets in bins
    off[2] = p; p = al(p + nbins * 4);                        // bin start within workgroup
    off[3] = p; p = al(p + nbins * 4);                        // chunk start within workgroup
    off[4] = p; p = al(p + (2 * nwg + 2) * 4);                // workgroup bases and totals
    off[5] = p; p = al(p + (size_t)max_chunks(s) * 16);       // chunk descriptors
    off[6] = p; p = al(p + ntiles * 4);                       // tile flags
    off[7] = p; p = al(p + nent * 4);                         // entry ranks
    off[8] = p; p = al(p + (size_t)(MAX_REMOTE_GRID + 1) * 4);   // remote work split
    off[9] = p;                                               // (none: partial rows carry their log-sum-exps)
    off[10] = p; p = al(p + nent * (size_t)s.d * esz);        // partial outputs
    off[11] = p; p = al(p + (size_t)s.B * s.T * s.Hq * s.d * esz);   // rotated q
    off[12] = p; p = al(p + (size_t)s.B * s.T * s.Hkv * s.d * esz);  // rotated k
    off[13] = p; p = al(p + nent * 4);                        // q rows of the list
    return p;
}

// prerotated: the workspace's rotated-q and rotated-k slots (attention_rot_slots)
// already hold the rows, so the rotation pass is skipped.
// Rotated-q and rotated-k slots of the attention workspace.
void attention_rot_slots(const Shape &s, void *ws, void **q_rot, void **k_rot) {
    size_t off[14];
    attention_ws_layout(s, off);
    unsigned char *base = reinterpret_cast<unsigned char *>(ws);
    *q_rot = base + off[11];
    *k_rot = base + off[12];
}

hipError_t launch_attention(const Shape &s, const void *q, const void *k, const void *v,
                            const float *cos_t, const float *sin_t, const int32_t *sel, void *out,
                            void *ws, hipStream_t st, bool prerotated) {
    size_t off[14];
    attention_ws_layout(s, off);
    unsigned char *base = reinterpret_cast<unsigned char *>(ws);
    AttnWs w;
    w.cnt = reinterpret_cast<int32_t *>(base + off[0]);
    w.seg_rel = reinterpret_cast<int32_t *>(base + off[1]);
    w.bin_local = reinterpret_cast<int32_t *>(base + off[2]);
    w.chunk_local = reinterpret_cast<int32_t *>(base + off[3]);
    w.wg_sum = reinterpret_cast<int32_t *>(base + off[4]);
    w.chunk_desc = reinterpret_cast<int4 *>(base + off[5]);
    w.tile_flag = reinterpret_cast<int32_t *>(base + off[6]);
    w.entry_pos = reinterpret_cast<int32_t *>(base + off[7]);
    w.part_o = base + off[10];
    w.q_rot = base + off[11];
    w.k_rot = base + off[12];
    w.list_q = reinterpret_cast<int32_t *>(base + off[13]);
    w.wg_first = reinterpret_cast<int32_t *>(base + off[8]);
    const bool bf = s.dtype == 1;
#define MONO_ATTN_ARGS s, q, k, v, cos_t, sin_t, sel, out, w, st, prerotated
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
