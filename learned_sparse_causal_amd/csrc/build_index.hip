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
// k_posting_lists: one workgroup per (batch, kv-head).  LDS histogram,
//   exclusive scan of the clamped counts, then a stable rank of every block
//   within its address from wavefront ballots over the address bits (chunks
//   of 64 blocks in source order, running per-address counts in LDS), and a
//   scatter that keeps the first `cap` blocks of every list.
#include "common.hpp"

namespace {

// One wave handles 64 / (d/2) (block, kv-head) tasks: 2 for d = 64, 1 for d = 128.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_block_address(Shape s, const void *__restrict__ k,
                                                       const float *__restrict__ cos_t,
                                                       const float *__restrict__ sin_t,
                                                       const float *__restrict__ cb,
                                                       float *__restrict__ kbar,
                                                       int32_t *__restrict__ addr) {
    constexpr int H = D / 2;
    constexpr int TPW = WAVE / H;                 // tasks per wave
    __shared__ float kb_s[4][TPW][D];
    __shared__ float sc_s[4][TPW][128];
    __shared__ int code_s[4][TPW][2];

    const int lane = lane_id(), wave = threadIdx.x / WAVE;
    const int sub = lane / H, i = lane % H;
    const long ntask = (long)s.B * s.NB * s.Hkv;
    const long task = ((long)blockIdx.x * 4 + wave) * TPW + sub;
    const bool live = task < ntask;
    // task order (b, n, g): the heads of one block are neighbours and share
    // the rotary table rows in cache.
    const long tt = live ? task : 0;
    const int g = (int)(tt % s.Hkv);
    const int n = (int)((tt / s.Hkv) % s.NB);
    const int b = (int)(tt / ((long)s.Hkv * s.NB));

    float acc0 = 0.0f, acc1 = 0.0f;
    const int beta = s.beta;
    const size_t row_stride = (size_t)s.Hkv * D;
    const size_t base = (((size_t)b * s.T + (size_t)n * beta) * s.Hkv + g) * D;
    if (live) {
#pragma unroll 8
        for (int u = 0; u < beta; ++u) {
            const int t = n * beta + u;
            const size_t r = base + (size_t)u * row_stride;
            const float x0 = load1<BF16>(k, r + i);
            const float x1 = load1<BF16>(k, r + i + H);
            const float c = cos_t[(size_t)t * H + i];
            const float sn = sin_t[(size_t)t * H + i];
            const float p0 = x0 * c, p1 = x1 * sn, p2 = x1 * c, p3 = x0 * sn;
            acc0 = acc0 + (p0 - p1);
            acc1 = acc1 + (p2 + p3);
        }
    }
    const float inv_beta = 1.0f / (float)beta;
    const float kb0 = acc0 * inv_beta, kb1 = acc1 * inv_beta;
    kb_s[wave][sub][i] = kb0;
    kb_s[wave][sub][i + H] = kb1;
    if (live) {
        float *dst = kbar + (((size_t)b * s.Hkv + g) * s.NB + n) * D;
        dst[i] = kb0;
        dst[i + H] = kb1;
    }
    __builtin_amdgcn_wave_barrier();
    __syncthreads();

    // Code scores: lane -> (task, component, code).
    const int PK = s.P * s.K, ds = s.ds;
    for (int ci = lane; ci < TPW * PK; ci += WAVE) {
        const int ts = ci / PK, code = ci % PK, p = code / s.K;
        const long task2 = ((long)blockIdx.x * 4 + wave) * TPW + ts;
        if (task2 >= ntask) continue;
        const int g2 = (int)(task2 % s.Hkv);
        const float *crow = cb + ((size_t)g2 * PK + code) * ds;
        const float *kv = &kb_s[wave][ts][p * ds];
        float acc = 0.0f;
        for (int j = 0; j < ds; j += 4) {
            const float4 cv = *reinterpret_cast<const float4 *>(crow + j);
            acc = __builtin_fmaf(kv[j], cv.x, acc);
            acc = __builtin_fmaf(kv[j + 1], cv.y, acc);
            acc = __builtin_fmaf(kv[j + 2], cv.z, acc);
            acc = __builtin_fmaf(kv[j + 3], cv.w, acc);
        }
        sc_s[wave][ts][code] = acc;
    }
    __syncthreads();
    // Per-component argmax, lowest code on ties.
    if (lane < TPW * s.P) {
        const int ts = lane / s.P, p = lane % s.P;
        const float *sv = &sc_s[wave][ts][p * s.K];
        int best = 0;
        float bv = sv[0];
        for (int c = 1; c < s.K; ++c)
            if (sv[c] > bv) { bv = sv[c]; best = c; }
        code_s[wave][ts][p] = best;
    }
    __syncthreads();
    if (lane < TPW) {
        const long task3 = ((long)blockIdx.x * 4 + wave) * TPW + lane;
        if (task3 < ntask) {
            const int g3 = (int)(task3 % s.Hkv);
            const int n3 = (int)((task3 / s.Hkv) % s.NB);
            const int b3 = (int)(task3 / ((long)s.Hkv * s.NB));
            int a = 0;
            for (int p = 0; p < s.P; ++p) a = a * s.K + code_s[wave][lane][p];
            addr[((size_t)b3 * s.Hkv + g3) * s.NB + n3] = a;
        }
    }
}

constexpr int PL_THREADS = 256;

__global__ __launch_bounds__(PL_THREADS) void k_posting_lists(Shape s,
                                                              const int32_t *__restrict__ addr,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ entries,
                                                              int32_t *__restrict__ load,
                                                              int32_t *__restrict__ overflow) {
    extern __shared__ int32_t lds[];
    const int A = s.A, NB = s.NB, cap = s.cap;
    int32_t *hist = lds;            // [A] loads
    int32_t *off = lds + A;         // [A+1] list starts
    int32_t *run = lds + 2 * A + 1; // [A] blocks already placed per address
    __shared__ int32_t part[PL_THREADS];
    __shared__ int32_t ovf_s[PL_THREADS];

    const int u = blockIdx.x;  // b * Hkv + g
    const int32_t *ad = addr + (size_t)u * NB;
    const int tid = threadIdx.x;
    for (int a = tid; a < A; a += PL_THREADS) { hist[a] = 0; run[a] = 0; }
    __syncthreads();
    for (int n = tid; n < NB; n += PL_THREADS) atomicAdd(&hist[ad[n]], 1);
    __syncthreads();

    // exclusive scan of min(load, cap): each thread owns a contiguous chunk
    const int per = (A + PL_THREADS - 1) / PL_THREADS;
    const int lo = tid * per, hi = min(A, lo + per);
    int sum = 0, ov = 0;
    for (int a = lo; a < hi; ++a) {
        const int l = hist[a];
        sum += min(l, cap);
        ov += max(0, l - cap);
    }
    part[tid] = sum;
    ovf_s[tid] = ov;
    __syncthreads();
    if (tid == 0) {
        int acc = 0, o = 0;
        for (int x = 0; x < PL_THREADS; ++x) {
            const int v = part[x];
            part[x] = acc;
            acc += v;
            o += ovf_s[x];
        }
        off[A] = acc;
        overflow[u] = o;
    }
    __syncthreads();
    {
        int acc = part[tid];
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

    // stable ranks: wave 0 walks the blocks in source order, 64 at a time
    if (tid < WAVE) {
        int nbits = 0;
        while ((1 << nbits) < A) ++nbits;
        const uint64_t lt = (1ull << tid) - 1ull;
        for (int c0 = 0; c0 < NB; c0 += WAVE) {
            const int n = c0 + tid;
            const bool in = n < NB;
            const int a = in ? ad[n] : 0;
            uint64_t m = __ballot(in);
            for (int bit = 0; bit < nbits; ++bit) {
                const uint64_t bal = __ballot(in && ((a >> bit) & 1));
                m &= ((a >> bit) & 1) ? bal : ~bal;
            }
            int rank = 0;
            if (in) rank = run[a] + __popcll(m & lt);
            __builtin_amdgcn_wave_barrier();
            // the highest lane of each group advances the running count
            if (in && (m >> tid) == 1ull) run[a] += __popcll(m);
            __builtin_amdgcn_wave_barrier();
            if (in && rank < cap) ent_g[off[a] + rank] = n;
        }
    }
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_block_address(const Shape &s, const void *k, const float *cos_t,
                                const float *sin_t, const float *cb, float *kbar, int32_t *addr,
                                hipStream_t st) {
    const long ntask = (long)s.B * s.NB * s.Hkv;
    const int tpw = WAVE / (s.d / 2);
    const long nwaves = (ntask + tpw - 1) / tpw;
    const dim3 grid((unsigned)((nwaves + 3) / 4));
    const bool bf = s.dtype == 1;
    if (s.d == 64) {
        if (bf) k_block_address<64, true><<<grid, 256, 0, st>>>(s, k, cos_t, sin_t, cb, kbar, addr);
        else k_block_address<64, false><<<grid, 256, 0, st>>>(s, k, cos_t, sin_t, cb, kbar, addr);
    } else {
        if (bf) k_block_address<128, true><<<grid, 256, 0, st>>>(s, k, cos_t, sin_t, cb, kbar, addr);
        else k_block_address<128, false><<<grid, 256, 0, st>>>(s, k, cos_t, sin_t, cb, kbar, addr);
    }
    return hipGetLastError();
}

hipError_t launch_posting_lists(const Shape &s, const int32_t *addr, int32_t *offsets,
                                int32_t *entries, int32_t *load, int32_t *overflow,
                                hipStream_t st) {
    const size_t lds = (size_t)(3 * s.A + 1) * sizeof(int32_t);
    k_posting_lists<<<dim3(s.B * s.Hkv), PL_THREADS, lds, st>>>(s, addr, offsets, entries, load,
                                                                 overflow);
    return hipGetLastError();
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
