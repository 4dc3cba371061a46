// Index build for gfx950: block summaries, product addresses, posting lists.
//
// Method (news page "Monodratic Claims Learned Routing...", section
// "Monodratic Turns Sparse Attention Into a Retrieval Decision"; technical
// report page, sections "Mixer", "Capacity", "Finite-range scaling"): after
// rotary embedding each source block gets a product address made of one
// decision per code component; the address selects a capacity-bounded causal
// posting list; overflow is counted; the build is a stable sort.
//
// k_block_address: one rotation pair (dims i, i + d/2) per lane; each lane
//   rotates and sums its two dimensions over the block's tokens in token
//   order (fp32, products rounded before the add, as the rotation is
//   defined), so the summary is bit-identical to a sequential evaluation.
//   Code scores are fp32 fused multiply-add chains in dimension order; the
//   argmax keeps the lowest code on ties.  HBM-bound: the keys are read once.
// k_posting_lists: one workgroup per (batch, kv-head), each of its waves
//   owning a contiguous range of blocks.  Counts per (range, address) give
//   the loads and, by a prefix over the ranges, where each range's blocks of
//   an address start; an exclusive scan of the clamped loads gives the list
//   starts; then every wave ranks its own blocks within their address from
//   wavefront ballots over the address bits (chunks of 64 blocks in source
//   order, running per-address counts in LDS), so the ranking runs on all
//   waves at once, and the first `cap` blocks of every list are placed.
#include "common.hpp"

namespace {

constexpr int BA_THREADS = 256;
constexpr int BA_CHUNK_BYTES = 32768;   // LDS staging of key rows per chunk

// Tokens per staged chunk: the largest power of two dividing the block size
// whose rows (all kv-heads) fit in BA_CHUNK_BYTES and whose rotary-table
// entries (d/2 per token) fit the per-thread staging registers.
int block_chunk_tokens(const Shape &s) {
    const int row = s.Hkv * s.d * (s.dtype == 1 ? 2 : 4);
    const int tab_max = BA_CHUNK_BYTES / 16;     // VPT * BA_THREADS
    int ct = s.beta;
    while (ct > 1 && (ct * row > BA_CHUNK_BYTES || ct * (s.d / 2) > tab_max)) ct /= 2;
    return ct;
}

size_t block_address_lds(const Shape &s, int ct) {
    const int es = s.dtype == 1 ? 2 : 4;
    return (size_t)ct * s.Hkv * s.d * es          // key rows
           + (size_t)2 * ct * (s.d / 2) * 4       // cos, sin rows
           + (size_t)s.Hkv * s.d * 4              // summaries
           + (size_t)s.Hkv * s.P * s.K * 4;       // code scores
}

// One workgroup per (batch, block n).  The block's key rows (every kv-head)
// pass through LDS in chunks of CT tokens, read with 16-byte loads; the next
// chunk's loads are in flight while the current chunk is summed.  Thread slot
// j of thread x owns rotation pair x + 256 j, i.e. kv-head g and dims
// (i, i + d/2), and sums it over the tokens in order (fp32, products rounded
// before the add, as the rotation is defined).  Then one thread per
// (kv-head, code) scores the summary with an fp32 fused multiply-add chain
// in dimension order and one thread per kv-head takes the argmax of every
// component (lowest code on ties) and writes the address.  MAXP bounds the
// pairs per thread (Hkv d / 2 <= 256 MAXP).
template <int D, int P, bool BF16, int MAXP>
__global__ __launch_bounds__(BA_THREADS) void k_block_address(Shape s, int CT, int n0,
                                                              const void *__restrict__ k,
                                                              const float *__restrict__ cos_t,
                                                              const float *__restrict__ sin_t,
                                                              const float *__restrict__ cb,
                                                              float *__restrict__ kbar,
                                                              int32_t *__restrict__ addr,
                                                              void *__restrict__ k_rot) {
    constexpr int H = D / 2;
    constexpr int DS = D / P;
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int VPT = BA_CHUNK_BYTES / 16 / BA_THREADS;      // 16-byte loads per thread
    extern __shared__ __align__(16) char ba_lds[];
    const int Hkv = s.Hkv, K = s.K, PK = P * K;
    const int rowE = Hkv * D;                                   // elements per token row
    char *rows = ba_lds;                                        // [CT][rowE]
    float *cs = reinterpret_cast<float *>(ba_lds + (size_t)CT * rowE * ES);   // [CT][H]
    float *sn = cs + CT * H;                                    // [CT][H]
    float *kb = sn + CT * H;                                    // [Hkv][D]
    float *sc = kb + Hkv * D;                                   // [Hkv][PK]

    const int tid = threadIdx.x;
    const int n = n0 + blockIdx.x, b = blockIdx.y;
    const int t0 = n * s.beta;
    const int npairs = Hkv * H;
    const int vecs = CT * rowE * ES / 16;                       // 16-byte vectors per chunk
    const int tabs = CT * H;                                    // table entries per chunk
    const char *kbase = reinterpret_cast<const char *>(k) + ((size_t)b * s.T + t0) * rowE * ES;

    float a0[MAXP], a1[MAXP];
#pragma unroll
    for (int j = 0; j < MAXP; ++j) { a0[j] = 0.0f; a1[j] = 0.0f; }

    // staging registers; indexes are clamped so every thread loads in bounds
    // and only the threads that own a vector store it
    u32x4 tmp[VPT];
    float tc[VPT], ts[VPT];
#define MONO_BA_FETCH(c_)                                                                  \
    {                                                                                      \
        const u32x4 *src_ = reinterpret_cast<const u32x4 *>(kbase + (size_t)(c_)*rowE * ES); \
        const float *cg_ = cos_t + (size_t)(t0 + (c_)) * H;                                \
        const float *sg_ = sin_t + (size_t)(t0 + (c_)) * H;                                \
        _Pragma("clang loop unroll(full)") for (int j = 0; j < VPT; ++j) {                  \
            const int v = tid + j * BA_THREADS;                                            \
            tmp[j] = src_[min(v, vecs - 1)];                                               \
            tc[j] = cg_[min(v, tabs - 1)];                                                 \
            ts[j] = sg_[min(v, tabs - 1)];                                                 \
        }                                                                                  \
    }
    MONO_BA_FETCH(0)
    for (int c = 0; c < s.beta; c += CT) {
#pragma clang loop unroll(full)
        for (int j = 0; j < VPT; ++j) {
            const int v = tid + j * BA_THREADS;
            if (v < vecs) reinterpret_cast<u32x4 *>(rows)[v] = tmp[j];
        }
#pragma clang loop unroll(full)
        for (int j = 0; j < VPT; ++j) {
            const int v = tid + j * BA_THREADS;
            if (v < tabs) { cs[v] = tc[j]; sn[v] = ts[j]; }
        }
        __syncthreads();
        if (c + CT < s.beta) MONO_BA_FETCH(c + CT)
#pragma unroll
        for (int j = 0; j < MAXP; ++j) {
            const int pr = tid + j * BA_THREADS;
            if (pr < npairs) {
                const int g = pr / H, i = pr - g * H;
#pragma unroll 8
                for (int u = 0; u < CT; ++u) {
                    const int e = u * rowE + g * D + i;
                    float x0, x1;
                    if constexpr (BF16) {
                        x0 = bf16_bits_to_f32(reinterpret_cast<const u16 *>(rows)[e]);
                        x1 = bf16_bits_to_f32(reinterpret_cast<const u16 *>(rows)[e + H]);
                    } else {
                        x0 = reinterpret_cast<const float *>(rows)[e];
                        x1 = reinterpret_cast<const float *>(rows)[e + H];
                    }
                    const float cc = cs[u * H + i], ss = sn[u * H + i];
                    const float p0 = x0 * cc, p1 = x1 * ss, p2 = x1 * cc, p3 = x0 * ss;
                    const float r0 = p0 - p1, r1 = p2 + p3;
                    a0[j] = a0[j] + r0;
                    a1[j] = a1[j] + r1;
                    if (k_rot) {   // the rotated pair replaces the staged one (this thread's)
                        if constexpr (BF16) {
                            reinterpret_cast<u16 *>(rows)[e] = f32_to_bf16_bits(r0);
                            reinterpret_cast<u16 *>(rows)[e + H] = f32_to_bf16_bits(r1);
                        } else {
                            reinterpret_cast<float *>(rows)[e] = r0;
                            reinterpret_cast<float *>(rows)[e + H] = r1;
                        }
                    }
                }
            }
        }
        __syncthreads();
        if (k_rot) {   // the chunk's rotated rows, rounded to the activation dtype
            u32x4 *dst = reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(k_rot) +
                                                   ((size_t)b * s.T + t0 + c) * rowE * ES);
            for (int v = tid; v < vecs; v += BA_THREADS) dst[v] = reinterpret_cast<const u32x4 *>(rows)[v];
            __syncthreads();   // read before the next chunk overwrites the rows
        }
    }
#undef MONO_BA_FETCH

    // summaries: LDS for the scores, global for the router
    const float inv_beta = 1.0f / (float)s.beta;
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
        const int pr = tid + j * BA_THREADS;
        if (pr < npairs) {
            const int g = pr / H, i = pr - g * H;
            const float kb0 = a0[j] * inv_beta, kb1 = a1[j] * inv_beta;
            kb[g * D + i] = kb0;
            kb[g * D + i + H] = kb1;
            float *dst = kbar + (((size_t)b * Hkv + g) * s.NB + n) * D;
            dst[i] = kb0;
            dst[i + H] = kb1;
        }
    }
    __syncthreads();

    // code scores: thread per (kv-head, component code); the code row is
    // loaded whole before the chain starts
    for (int x = tid; x < Hkv * PK; x += BA_THREADS) {
        const int g = x / PK, code = x - g * PK, p = code / K;
        const float4 *crow = reinterpret_cast<const float4 *>(cb + ((size_t)g * PK + code) * DS);
        float4 cv[DS / 4];
#pragma unroll
        for (int j = 0; j < DS / 4; ++j) cv[j] = crow[j];
        const float *kv = kb + g * D + p * DS;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < DS / 4; ++j) {
            acc = __builtin_fmaf(kv[4 * j], cv[j].x, acc);
            acc = __builtin_fmaf(kv[4 * j + 1], cv[j].y, acc);
            acc = __builtin_fmaf(kv[4 * j + 2], cv[j].z, acc);
            acc = __builtin_fmaf(kv[4 * j + 3], cv[j].w, acc);
        }
        sc[x] = acc;
    }
    __syncthreads();

    // argmax per component (lowest code on ties), address = mixed radix
    for (int g = tid; g < Hkv; g += BA_THREADS) {
        int a = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const float *sv = sc + g * PK + p * K;
            int best = 0;
            float bv = sv[0];
#pragma unroll 8
            for (int c = 1; c < K; ++c) {
                const float v = sv[c];
                best = v > bv ? c : best;
                bv = v > bv ? v : bv;
            }
            a = a * K + best;
        }
        addr[((size_t)b * Hkv + g) * s.NB + n] = a;
    }
}

constexpr int PL_THREADS = 256;
constexpr int PL_WAVES = PL_THREADS / WAVE;

// nbu: blocks 0 .. nbu-1 are indexed (NB for a whole sequence); arrays keep
// their NB strides.  Wave w owns the contiguous block range
// [w * span, (w + 1) * span) (span a multiple of 64); LDS:
//   hist  [A]            loads (blocks per address, before the clamp)
//   off   [A + 1]        list starts (exclusive scan of min(load, cap))
//   cnt   [PL_WAVES][A]  blocks of each address in each wave's range, then
//                        the count in the earlier ranges (exclusive prefix
//                        over waves) and, while ranking, the running count
//   adr   [nbu]          the addresses
__global__ __launch_bounds__(PL_THREADS) void k_posting_lists(Shape s, int nbu,
                                                              const int32_t *__restrict__ addr,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ entries,
                                                              int32_t *__restrict__ load,
                                                              int32_t *__restrict__ overflow) {
    extern __shared__ int32_t lds[];
    const int A = s.A, NB = s.NB, cap = s.cap;
    int32_t *hist = lds;
    int32_t *off = lds + A;
    int32_t *cnt = lds + 2 * A + 1;
    int32_t *adr = lds + (2 + PL_WAVES) * A + 1;
    __shared__ int32_t part[PL_WAVES];
    __shared__ int32_t ovf_s[PL_WAVES];

    const int u = blockIdx.x;  // b * Hkv + g
    const int32_t *ad = addr + (size_t)u * NB;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int span = ((nbu + PL_WAVES - 1) / PL_WAVES + WAVE - 1) / WAVE * WAVE;
    for (int i = tid; i < PL_WAVES * A; i += PL_THREADS) cnt[i] = 0;
    for (int n = tid; n < nbu; n += PL_THREADS) adr[n] = ad[n];
    __syncthreads();
    // pass 1: counts per (wave range, address)
    {
        int32_t *cw = cnt + wv * A;
        const int n0 = wv * span, n1 = min(nbu, n0 + span);
        for (int n = n0 + lane; n < n1; n += WAVE) atomicAdd(&cw[adr[n]], 1);
    }
    __syncthreads();
    // per address: exclusive prefix over the wave ranges, total load
    for (int a = tid; a < A; a += PL_THREADS) {
        int acc = 0;
#pragma unroll
        for (int w = 0; w < PL_WAVES; ++w) {
            const int c = cnt[w * A + a];
            cnt[w * A + a] = acc;
            acc += c;
        }
        hist[a] = acc;
    }
    __syncthreads();

    // exclusive scan of min(load, cap): each thread owns a contiguous chunk
    const int per = (A + PL_THREADS - 1) / PL_THREADS;
    const int lo = min(A, tid * per), hi = min(A, lo + per);
    int sum = 0, ov = 0;
    for (int a = lo; a < hi; ++a) {
        const int l = hist[a];
        sum += min(l, cap);
        ov += max(0, l - cap);
    }
    // block-wide exclusive scan of the per-thread sums: wave prefix by
    // shuffles, then the wave totals
    int incl = sum;
#pragma unroll
    for (int dlt = 1; dlt < WAVE; dlt <<= 1) {
        const int o = __shfl_up(incl, dlt);
        if (lane >= dlt) incl += o;
    }
    int ovw = ov;
#pragma unroll
    for (int dlt = 32; dlt > 0; dlt >>= 1) ovw += __shfl_xor(ovw, dlt);
    if (lane == WAVE - 1) part[wv] = incl;
    if (lane == 0) ovf_s[wv] = ovw;
    __syncthreads();
    int wbase = 0, total_all = 0, ovf_all = 0;
#pragma unroll
    for (int w = 0; w < PL_WAVES; ++w) {
        const int v = part[w];
        wbase += w < wv ? v : 0;
        total_all += v;
        ovf_all += ovf_s[w];
    }
    if (tid == 0) {
        off[A] = total_all;
        overflow[u] = ovf_all;
    }
    {
        int acc = wbase + incl - sum;
        for (int a = lo; a < hi; ++a) {
            off[a] = acc;
            acc += min(hist[a], cap);
        }
    }
    __syncthreads();
    int32_t *off_g = offsets + (size_t)u * (A + 1);
    int32_t *ld_g = load + (size_t)u * A;
    for (int a = tid; a <= A; a += PL_THREADS) off_g[a] = off[a];
    for (int a = tid; a < A; a += PL_THREADS) ld_g[a] = hist[a];
    int32_t *ent_g = entries + (size_t)u * NB;
    const int total = off[A];
    for (int x = total + tid; x < NB; x += PL_THREADS) ent_g[x] = -1;

    // pass 2: stable ranks.  Each wave walks its range in source order, 64
    // blocks at a time; lanes of equal address find each other with one
    // ballot per address bit, rank by their lane order after the blocks of
    // that address in earlier ranges and earlier chunks (the running count),
    // and the first `cap` of every address are placed.
    {
        int nbits = 0;
        while ((1 << nbits) < A) ++nbits;
        const uint64_t lt = (1ull << lane) - 1ull;
        int32_t *run = cnt + wv * A;
        const int n0 = wv * span, n1 = min(nbu, n0 + span);
        for (int c0 = n0; c0 < n1; c0 += WAVE) {
            const int n = c0 + lane;
            const bool in = n < n1;
            const int a = in ? adr[n] : 0;
            uint64_t m = __ballot(in);
            for (int bit = 0; bit < nbits; ++bit) {
                const uint64_t bal = __ballot(in && ((a >> bit) & 1));
                m &= ((a >> bit) & 1) ? bal : ~bal;
            }
            int rank = 0;
            if (in) rank = run[a] + __popcll(m & lt);
            __builtin_amdgcn_wave_barrier();
            // the highest lane of each group advances the running count
            if (in && (m >> lane) == 1ull) run[a] += __popcll(m);
            __builtin_amdgcn_wave_barrier();
            if (in && rank < cap) ent_g[off[a] + rank] = n;
        }
    }
}

// ---------------------------------------------------------------- launchers
template <int D, int P, bool BF16, int MAXP>
hipError_t launch_ba_t(const Shape &s, int n0, int n1, int ct, size_t lds, const void *k,
                       const float *cos_t, const float *sin_t, const float *cb, float *kbar,
                       int32_t *addr, void *k_rot, hipStream_t st) {
    auto *fn = k_block_address<D, P, BF16, MAXP>;
    const hipError_t e = mono_lds_limit(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess) return e;
    fn<<<dim3((unsigned)(n1 - n0), (unsigned)s.B), BA_THREADS, lds, st>>>(s, ct, n0, k, cos_t,
                                                                          sin_t, cb, kbar, addr,
                                                                          k_rot);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_ba(const Shape &s, int n0, int n1, const void *k, const float *cos_t,
                     const float *sin_t, const float *cb, float *kbar, int32_t *addr,
                     void *k_rot, hipStream_t st) {
    const int ct = block_chunk_tokens(s);
    const size_t lds = block_address_lds(s, ct);
    const bool small = s.Hkv * (D / 2) <= 2 * BA_THREADS;
#define MONO_BA_ARGS s, n0, n1, ct, lds, k, cos_t, sin_t, cb, kbar, addr, k_rot, st
    if (s.P == 1)
        return small ? launch_ba_t<D, 1, BF16, 2>(MONO_BA_ARGS)
                     : launch_ba_t<D, 1, BF16, 8>(MONO_BA_ARGS);
    return small ? launch_ba_t<D, 2, BF16, 2>(MONO_BA_ARGS)
                 : launch_ba_t<D, 2, BF16, 8>(MONO_BA_ARGS);
#undef MONO_BA_ARGS
}

}  // namespace

// Summaries and addresses of blocks n0 .. n1-1 of every sequence; with k_rot
// non-null also the rotated keys of those blocks ([B][T][Hkv][d], activation
// dtype).
hipError_t launch_block_address_range(const Shape &s, int n0, int n1, const void *k,
                                      const float *cos_t, const float *sin_t, const float *cb,
                                      float *kbar, int32_t *addr, hipStream_t st,
                                      void *k_rot = nullptr) {
    if (n1 <= n0) return hipSuccess;
    const bool bf = s.dtype == 1;
    if (s.d == 64)
        return bf ? launch_ba<64, true>(s, n0, n1, k, cos_t, sin_t, cb, kbar, addr, k_rot, st)
                  : launch_ba<64, false>(s, n0, n1, k, cos_t, sin_t, cb, kbar, addr, k_rot, st);
    return bf ? launch_ba<128, true>(s, n0, n1, k, cos_t, sin_t, cb, kbar, addr, k_rot, st)
              : launch_ba<128, false>(s, n0, n1, k, cos_t, sin_t, cb, kbar, addr, k_rot, st);
}

hipError_t launch_block_address(const Shape &s, const void *k, const float *cos_t,
                                const float *sin_t, const float *cb, float *kbar, int32_t *addr,
                                hipStream_t st, void *k_rot) {
    return launch_block_address_range(s, 0, s.NB, k, cos_t, sin_t, cb, kbar, addr, st, k_rot);
}

// Lists of blocks 0 .. nbu-1 (the indexed prefix of every sequence).
hipError_t launch_posting_lists_prefix(const Shape &s, int nbu, const int32_t *addr,
                                       int32_t *offsets, int32_t *entries, int32_t *load,
                                       int32_t *overflow, hipStream_t st) {
    const size_t lds = (size_t)((2 + PL_WAVES) * s.A + 1 + nbu) * sizeof(int32_t);
    const hipError_t e = mono_lds_limit(reinterpret_cast<const void *>(k_posting_lists), lds);
    if (e != hipSuccess) return e;
    k_posting_lists<<<dim3(s.B * s.Hkv), PL_THREADS, lds, st>>>(s, nbu, addr, offsets, entries,
                                                                 load, overflow);
    return hipGetLastError();
}

hipError_t launch_posting_lists(const Shape &s, const int32_t *addr, int32_t *offsets,
                                int32_t *entries, int32_t *load, int32_t *overflow,
                                hipStream_t st) {
    return launch_posting_lists_prefix(s, s.NB, addr, offsets, entries, load, overflow, st);
}

// Totals of an index: stats[0] = sum of overflow, stats[1] = maximum load.
namespace {
__global__ __launch_bounds__(256) void k_index_stats(int nov, const int32_t *__restrict__ overflow,
                                                     long nload, const int32_t *__restrict__ load,
                                                     int32_t *__restrict__ stats) {
    __shared__ int so[256], sm[256];
    int o = 0, m = 0;
    for (int i = threadIdx.x; i < nov; i += 256) o += overflow[i];
    for (long i = threadIdx.x; i < nload; i += 256) m = max(m, load[i]);
    so[threadIdx.x] = o;
    sm[threadIdx.x] = m;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            so[threadIdx.x] += so[threadIdx.x + w];
            sm[threadIdx.x] = max(sm[threadIdx.x], sm[threadIdx.x + w]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        stats[0] = so[0];
        stats[1] = sm[0];
    }
}
}  // namespace

hipError_t launch_index_stats(const Shape &s, const int32_t *overflow, const int32_t *load,
                              int32_t *stats, hipStream_t st) {
    k_index_stats<<<1, 256, 0, st>>>(s.B * s.Hkv, overflow, (long)s.B * s.Hkv * s.A, load, stats);
    return hipGetLastError();
}
