// Index build for gfx950: block summaries, product addresses, posting lists.
//
// Method (news page "Monodratic Claims Learned Routing...", section
// "Monodratic Turns Sparse Attention Into a Retrieval Decision"; technical
// report page, sections "Mixer", "Capacity", "Finite-range scaling"): after
// rotary embedding each source block gets a product address made of one
// decision per code component; the address selects a capacity-bounded causal
// posting list; overflow is counted; the build is a stable sort.
//
// k_block_address: one workgroup per (batch, block, group of kv-heads), one
//   rotation pair (dims i, i + d/2 of one kv-head) per thread; each thread
//   rotates and sums its two dimensions over the block's tokens in token
//   order (fp32, products rounded before the add, as the rotation is
//   defined), so the summary is bit-identical to a sequential evaluation.
//   Code scores are fp32 fused multiply-add chains in dimension order; the
//   argmax keeps the lowest code on ties.  HBM-bound: the keys are read once.
//   Every step is independent per kv-head, so splitting the heads over
//   workgroups shortens each workgroup's chain of chunk loads and gives the
//   chip more workgroups to overlap.
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
constexpr int BA_CHUNK_BYTES = 16384;   // LDS staging of key rows per chunk
constexpr int BA_UB = 8;                // tokens read together per summing step (divides every chunk)

// kv-heads per workgroup: the largest power of two dividing Hkv whose
// rotation pairs fit one per thread.
int block_head_group(const Shape &s) {
    int hg = 1;
    while (s.Hkv % (2 * hg) == 0 && 2 * hg * (s.d / 2) <= BA_THREADS) hg *= 2;
    return hg;
}

// Tokens per staged chunk: the largest power of two dividing the block size
// whose rows (hg kv-heads) fit in BA_CHUNK_BYTES and whose rotary-table
// entries (d/2 per token) fit the per-thread staging registers.
int block_chunk_tokens(const Shape &s, int hg) {
    const int row = hg * s.d * (s.dtype == 1 ? 2 : 4);
    const int tab_max = BA_CHUNK_BYTES / 16;     // VPT * BA_THREADS
    int ct = s.beta;
    while (ct > 1 && (ct * row > BA_CHUNK_BYTES || ct * (s.d / 2) > tab_max)) ct /= 2;
    return ct;
}

size_t block_address_lds(const Shape &s, int ct, int hg) {
    const int es = s.dtype == 1 ? 2 : 4;
    return (size_t)ct * hg * s.d * es             // key rows
           + (size_t)2 * ct * (s.d / 2) * 4       // cos, sin rows
           + (size_t)hg * s.d * 4                 // summaries
           + (size_t)hg * s.P * s.K * 4;          // code scores
}

// One workgroup per (batch, block n, kv-heads HG z .. HG z + HG - 1).  The
// block's key rows of those heads pass through LDS in chunks of CT tokens,
// read with 16-byte loads (VSH = log2 of the 16-byte vectors per token row);
// the next chunk's loads are in flight while the current chunk is summed.
// Thread x owns rotation pair x, i.e. kv-head g0 + x / (d/2) and dims
// (i, i + d/2), and sums it over the tokens in order (fp32, products rounded
// before the add, as the rotation is defined).  Then one thread per
// (kv-head, code) scores the summary with an fp32 fused multiply-add chain
// in dimension order and one thread per kv-head takes the argmax of every
// component (lowest code on ties) and writes the address.  MAXP bounds the
// pairs per thread (HG d / 2 <= 256 MAXP).
template <int D, int P, bool BF16, int MAXP, bool ROT>
__global__ __launch_bounds__(BA_THREADS) void k_block_address(Shape s, int CT, int HG, int VSH,
                                                              int n0,
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
    const int rowE = HG * D;                                    // elements per staged token row
    const size_t growB = (size_t)Hkv * D * ES;                  // bytes per global token row
    char *rows = ba_lds;                                        // [CT][rowE]
    float *cs = reinterpret_cast<float *>(ba_lds + (size_t)CT * rowE * ES);   // [CT][H]
    float *sn = cs + CT * H;                                    // [CT][H]
    float *kb = sn + CT * H;                                    // [HG][D]
    float *sc = kb + HG * D;                                    // [HG][PK]

    const int tid = threadIdx.x;
    const int n = n0 + blockIdx.x, b = blockIdx.y, g0 = blockIdx.z * HG;
    const int t0 = n * s.beta;
    const int npairs = HG * H;
    const int vecs = CT << VSH;                                 // 16-byte vectors per chunk
    const int vmask = (1 << VSH) - 1;
    const int tabs = CT * H;                                    // table entries per chunk
    const char *kbase = reinterpret_cast<const char *>(k) + ((size_t)b * s.T + t0) * growB +
                        (size_t)g0 * D * ES;
    // byte offset of staged vector v (token v >> VSH, vector v & vmask of its row)
    auto goff = [&](int v) { return (size_t)(v >> VSH) * growB + (size_t)(v & vmask) * 16; };

    float a0[MAXP], a1[MAXP];
#pragma unroll
    for (int j = 0; j < MAXP; ++j) { a0[j] = 0.0f; a1[j] = 0.0f; }

    // staging registers; indexes are clamped so every thread loads in bounds
    // and only the threads that own a vector store it
    u32x4 tmp[VPT];
    float tc[VPT], ts[VPT];
#define MONO_BA_FETCH(c_)                                                                  \
    {                                                                                      \
        const char *src_ = kbase + (size_t)(c_)*growB;                                     \
        const float *cg_ = cos_t + (size_t)(t0 + (c_)) * H;                                \
        const float *sg_ = sin_t + (size_t)(t0 + (c_)) * H;                                \
        _Pragma("clang loop unroll(full)") for (int j = 0; j < VPT; ++j) {                  \
            const int v = tid + j * BA_THREADS;                                            \
            tmp[j] = *reinterpret_cast<const u32x4 *>(src_ + goff(min(v, vecs - 1)));      \
            tc[j] = cg_[min(v, tabs - 1)];                                                 \
            ts[j] = sg_[min(v, tabs - 1)];                                                 \
        }                                                                                  \
    }
    auto stage = [&]() {
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
    };
    MONO_BA_FETCH(0)
    stage();
    __syncthreads();
    for (int c = 0; c < s.beta; c += CT) {
        const bool more = c + CT < s.beta;
        if (more) MONO_BA_FETCH(c + CT)
#pragma unroll
        for (int j = 0; j < MAXP; ++j) {
            const int pr = tid + j * BA_THREADS;
            if (pr < npairs) {
                const int g = pr / H, i = pr - g * H;
                const int e0 = g * D + i;
                // BA_UB tokens at a time: their staged values and table
                // entries are read together, then summed in token order
                for (int u0 = 0; u0 < CT; u0 += BA_UB) {
                    float x0[BA_UB], x1[BA_UB], cc[BA_UB], ss[BA_UB];
#pragma unroll
                    for (int v = 0; v < BA_UB; ++v) {
                        const int e = (u0 + v) * rowE + e0;
                        if constexpr (BF16) {
                            x0[v] = bf16_bits_to_f32(reinterpret_cast<const u16 *>(rows)[e]);
                            x1[v] = bf16_bits_to_f32(reinterpret_cast<const u16 *>(rows)[e + H]);
                        } else {
                            x0[v] = reinterpret_cast<const float *>(rows)[e];
                            x1[v] = reinterpret_cast<const float *>(rows)[e + H];
                        }
                        cc[v] = cs[(u0 + v) * H + i];
                        ss[v] = sn[(u0 + v) * H + i];
                    }
                    float r0[BA_UB], r1[BA_UB];
#pragma unroll
                    for (int v = 0; v < BA_UB; ++v) {
                        const float p0 = x0[v] * cc[v], p1 = x1[v] * ss[v];
                        const float p2 = x1[v] * cc[v], p3 = x0[v] * ss[v];
                        r0[v] = p0 - p1;
                        r1[v] = p2 + p3;
                        a0[j] = a0[j] + r0[v];
                        a1[j] = a1[j] + r1[v];
                    }
                    if constexpr (ROT) {   // the rotated pairs replace the staged ones (this thread's)
#pragma unroll
                        for (int v = 0; v < BA_UB; ++v) {
                            const int e = (u0 + v) * rowE + e0;
                            if constexpr (BF16) {
                                reinterpret_cast<u16 *>(rows)[e] = f32_to_bf16_bits(r0[v]);
                                reinterpret_cast<u16 *>(rows)[e + H] = f32_to_bf16_bits(r1[v]);
                            } else {
                                reinterpret_cast<float *>(rows)[e] = r0[v];
                                reinterpret_cast<float *>(rows)[e + H] = r1[v];
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();
        if constexpr (ROT) {
            // the chunk's rotated rows, rounded to the activation dtype: a
            // fixed number of stores per thread (indexes clamped; a clamped
            // store rewrites the last vector with its own value), so that
            // the wait for the next chunk's loads below does not also wait
            // for these stores to complete
            char *dst = reinterpret_cast<char *>(k_rot) + ((size_t)b * s.T + t0 + c) * growB +
                        (size_t)g0 * D * ES;
            u32x4 out[VPT];
#pragma clang loop unroll(full)
            for (int j = 0; j < VPT; ++j)
                out[j] = reinterpret_cast<const u32x4 *>(rows)[min(tid + j * BA_THREADS, vecs - 1)];
#pragma clang loop unroll(full)
            for (int j = 0; j < VPT; ++j)
                *reinterpret_cast<u32x4 *>(dst + goff(min(tid + j * BA_THREADS, vecs - 1))) = out[j];
            if (more) __syncthreads();   // read before the next chunk overwrites the rows
        }
        if (more) {
            stage();
            __syncthreads();
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
            float *dst = kbar + (((size_t)b * Hkv + g0 + g) * s.NB + n) * D;
            dst[i] = kb0;
            dst[i + H] = kb1;
        }
    }
    __syncthreads();

    // code scores: thread per (kv-head, component code); the code row is
    // loaded whole before the chain starts
    for (int x = tid; x < HG * PK; x += BA_THREADS) {
        const int g = x / PK, code = x - g * PK, p = code / K;
        const float4 *crow =
            reinterpret_cast<const float4 *>(cb + ((size_t)(g0 + g) * PK + code) * DS);
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
    for (int g = tid; g < HG; g += BA_THREADS) {
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
        addr[((size_t)b * Hkv + g0 + g) * s.NB + n] = a;
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
template <int D, int P, bool BF16>
hipError_t launch_ba_t(const Shape &s, int n0, int n1, int ct, int hg, size_t lds, const void *k,
                       const float *cos_t, const float *sin_t, const float *cb, float *kbar,
                       int32_t *addr, void *k_rot, hipStream_t st) {
    // hg d / 2 <= 256 pairs: one per thread
    auto *fn = k_rot ? k_block_address<D, P, BF16, 1, true> : k_block_address<D, P, BF16, 1, false>;
    const hipError_t e = mono_lds_limit(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess) return e;
    int vsh = 0;   // 16-byte vectors per staged token row: hg d es / 16, a power of two
    while ((16 << vsh) < hg * D * (BF16 ? 2 : 4)) ++vsh;
    fn<<<dim3((unsigned)(n1 - n0), (unsigned)s.B, (unsigned)(s.Hkv / hg)), BA_THREADS, lds, st>>>(
        s, ct, hg, vsh, n0, k, cos_t, sin_t, cb, kbar, addr, k_rot);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_ba(const Shape &s, int n0, int n1, const void *k, const float *cos_t,
                     const float *sin_t, const float *cb, float *kbar, int32_t *addr,
                     void *k_rot, hipStream_t st) {
    const int hg = block_head_group(s);
    const int ct = block_chunk_tokens(s, hg);
    if (ct % BA_UB) return hipErrorInvalidValue;   // not reached for d <= 128
    const size_t lds = block_address_lds(s, ct, hg);
    if (s.P == 1)
        return launch_ba_t<D, 1, BF16>(s, n0, n1, ct, hg, lds, k, cos_t, sin_t, cb, kbar, addr,
                                       k_rot, st);
    return launch_ba_t<D, 2, BF16>(s, n0, n1, ct, hg, lds, k, cos_t, sin_t, cb, kbar, addr, k_rot,
                                   st);
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
