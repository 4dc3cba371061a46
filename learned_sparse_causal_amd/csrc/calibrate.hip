// Spherical codebook calibration for gfx950.
//
// The report page (section "Capacity", with Figure 3) shows that calibrating
// the codebooks spherically on a training split removes held-out list
// overflow and lowers the largest list load.  The pages name the method
// only; it is taken as spherical k-means, for every kv-head g and component
// p, over the training split's block summaries restricted to component p's
// sub-vector (the vectors whose code decisions make the addresses):
//   assignment  each point takes the code with the largest inner product
//               (fp32 fused multiply-add chain in dimension order, ties to
//               the lowest code): the decision the address itself uses;
//   update      a code with members becomes the fp32 sum of its members, in
//               point order, divided by the square root (correctly rounded)
//               of that sum's fused-multiply-add square; a code without
//               members keeps its value;
// for a fixed number of rounds.  Every step is the plain sequential fp32
// operation, so the result is bit-identical to a sequential evaluation.
//
// k_calibrate: one workgroup per (kv-head, component).  The codes (and,
// when they fit, the assignments and member lists) stay in LDS; each round, threads assign points (the point's sub-vector in
// registers), wave 0 lists the members of every code in point order with a
// ballot counting sort over the code bits, threads sum (code, dim) pairs
// over those lists, and one thread per code normalizes.
#include "common.hpp"

namespace {

constexpr int CAL_THREADS = 256;

constexpr size_t CAL_LDS_MAX = 150 * 1024;

// Codes, sums (K x ds floats each), counts, starts (K + 1), running ranks;
// plus the assignments and member lists (N ints each) when they fit.
size_t calibrate_lds_base(const Shape &s) { return (size_t)(2 * s.K * s.ds + 3 * s.K + 1) * 4; }

bool calibrate_lists_in_lds(const Shape &s) {
    return calibrate_lds_base(s) + (size_t)2 * s.B * s.NB * 4 <= CAL_LDS_MAX;
}

size_t calibrate_lds(const Shape &s) {
    return calibrate_lds_base(s) + (calibrate_lists_in_lds(s) ? (size_t)2 * s.B * s.NB * 4 : 0);
}

template <int DS>
__global__ __launch_bounds__(CAL_THREADS) void k_calibrate(Shape s, int n_iter, int lists_in_lds,
                                                          const float *__restrict__ kbar,
                                                          float *__restrict__ codebooks,
                                                          int32_t *__restrict__ ws) {
    extern __shared__ __align__(16) float cal_lds[];
    const int K = s.K, P = s.P, NB = s.NB;
    float *C = cal_lds;                                   // [K][DS] codes
    float *S = C + K * DS;                                // [K][DS] member sums
    int *cnt = reinterpret_cast<int *>(S + K * DS);       // [K]
    int *start = cnt + K;                                 // [K + 1]
    int *run = start + K + 1;                             // [K]

    const int gp = blockIdx.x;                            // g * P + p
    const int g = gp / P, p = gp % P;
    const int N = s.B * NB;                               // points: batch-major, then block
    int32_t *asg = lists_in_lds ? run + K : ws + (size_t)gp * 2 * N;   // [N] code of each point
    int32_t *member = asg + N;                                        // [N] points grouped by code
    float *cb = codebooks + (size_t)gp * K * DS;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1);
    auto point = [&](int i) {
        const int b = i / NB, n = i % NB;
        return kbar + (((size_t)b * s.Hkv + g) * NB + n) * s.d + (size_t)p * DS;
    };
    for (int e = tid; e < K * DS; e += CAL_THREADS) C[e] = cb[e];
    __syncthreads();

    for (int it = 0; it < n_iter; ++it) {
        for (int c = tid; c < K; c += CAL_THREADS) {
            cnt[c] = 0;
            run[c] = 0;
        }
        // assignment
        for (int i = tid; i < N; i += CAL_THREADS) {
            const float *x = point(i);
            float xv[DS];
#pragma unroll
            for (int j = 0; j < DS; j += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(x + j);
                xv[j] = v.x; xv[j + 1] = v.y; xv[j + 2] = v.z; xv[j + 3] = v.w;
            }
            int best = 0;
            float bs = 0.0f;
            for (int c = 0; c < K; ++c) {
                const float *cr = C + c * DS;
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < DS; ++j) acc = fmaf(xv[j], cr[j], acc);
                if (c == 0 || acc > bs) {
                    bs = acc;
                    best = c;
                }
            }
            asg[i] = best;
        }
        __syncthreads();
        for (int i = tid; i < N; i += CAL_THREADS) atomicAdd(&cnt[asg[i]], 1);
        __syncthreads();
        if (tid == 0) {
            int acc = 0;
            for (int c = 0; c < K; ++c) {
                start[c] = acc;
                acc += cnt[c];
            }
            start[K] = acc;
        }
        __syncthreads();
        // members of every code in point order: wave 0 walks the points 64 at a
        // time; a point's rank among earlier points of its code comes from
        // ballots over the code bits
        if (tid < WAVE) {
            int nbits = 0;
            while ((1 << nbits) < K) ++nbits;
            const uint64_t lt = (1ull << lane) - 1ull;
            for (int c0 = 0; c0 < N; c0 += WAVE) {
                const int i = c0 + lane;
                const bool in = i < N;
                const int c = in ? asg[i] : 0;
                uint64_t m = __ballot(in);
                for (int bit = 0; bit < nbits; ++bit) {
                    const uint64_t bal = __ballot(in && ((c >> bit) & 1));
                    m &= ((c >> bit) & 1) ? bal : ~bal;
                }
                const int rank = in ? run[c] + __popcll(m & lt) : 0;
                __builtin_amdgcn_wave_barrier();
                // the highest lane of each code's group advances its count
                if (in && (m >> lane) == 1ull) run[c] += __popcll(m);
                __builtin_amdgcn_wave_barrier();
                if (in) member[start[c] + rank] = i;
            }
        }
        __syncthreads();
        // sums over the members in point order (eight loads in flight, the
        // additions still one after another)
        for (int e = tid; e < K * DS; e += CAL_THREADS) {
            const int c = e / DS, j = e % DS;
            const int m1 = start[c + 1];
            float acc = 0.0f;
            int m = start[c];
            for (; m + 8 <= m1; m += 8) {
                int id[8];
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) id[u] = member[m + u];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = point(id[u])[j];
#pragma unroll
                for (int u = 0; u < 8; ++u) acc = acc + v[u];
            }
            for (; m < m1; ++m) acc = acc + point(member[m])[j];
            S[e] = acc;
        }
        __syncthreads();
        // normalize; a code without members keeps its value
        for (int c = tid; c < K; c += CAL_THREADS) {
            if (cnt[c] == 0) continue;
            const float *sc = S + c * DS;
            float n2 = 0.0f;
            for (int j = 0; j < DS; ++j) n2 = fmaf(sc[j], sc[j], n2);
            // sqrtf and '/' compile to the correctly rounded sequences
            // (__fsqrt_rn would be the approximate native instruction)
            const float norm = sqrtf(n2);
            for (int j = 0; j < DS; ++j) C[c * DS + j] = sc[j] / norm;
        }
        __syncthreads();
    }
    for (int e = tid; e < K * DS; e += CAL_THREADS) cb[e] = C[e];
}

template <int DS>
hipError_t run_calibrate(const Shape &s, int n_iter, const float *kbar, float *codebooks,
                         int32_t *ws, hipStream_t st) {
    const size_t lds = calibrate_lds(s);
    const hipError_t e = mono_lds_limit(reinterpret_cast<const void *>(k_calibrate<DS>), lds);
    if (e != hipSuccess) return e;
    k_calibrate<DS><<<dim3((unsigned)(s.Hkv * s.P)), CAL_THREADS, lds, st>>>(
        s, n_iter, calibrate_lists_in_lds(s) ? 1 : 0, kbar, codebooks, ws);
    return hipGetLastError();
}

}  // namespace

// Workspace of the calibration: per (kv-head, component) the code of every
// training point and the points grouped by code.
size_t calibrate_ws_bytes(const Shape &s) {
    return (size_t)s.Hkv * s.P * 2 * s.B * s.NB * sizeof(int32_t);
}

hipError_t launch_calibrate(const Shape &s, int n_iter, const float *kbar, float *codebooks,
                            void *ws, hipStream_t st) {
    int32_t *w = reinterpret_cast<int32_t *>(ws);
    switch (s.ds) {
        case 32: return run_calibrate<32>(s, n_iter, kbar, codebooks, w, st);
        case 64: return run_calibrate<64>(s, n_iter, kbar, codebooks, w, st);
        default: return run_calibrate<128>(s, n_iter, kbar, codebooks, w, st);
    }
}
