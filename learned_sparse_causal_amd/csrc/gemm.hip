// Projection GEMMs of the mixer (technical report page "Monodratic: a
// reproducible sparse attention mixer", section "Mixer" and Figure 1: the
// mixer maps the normalized stream to queries, keys and values and returns
// a delta of the stream's shape).  C[M][N] = A[M][K] * B[K][N], row-major,
// fp32 accumulation on MFMA, 128x128 workgroup tiles, four 64x64 wave tiles,
// k in steps of 32.  Epilogues: a plain store, or the q | k | v split of the
// fused input projection into three [rows][heads*d] tensors.
#include <type_traits>

#include "mfma.hpp"

namespace {

template <bool BF16>
using Elem = std::conditional_t<BF16, u16, float>;

struct Epi {
    int mode;          // 0: C[M][N]; 1: split columns into q | k | v
    void *c;           // mode 0
    void *q, *k, *v;   // mode 1
    int nq, nk;        // mode 1: columns of q and of k (v takes the rest)
};

template <bool BF16>
__device__ __forceinline__ void put(void *base, size_t i, float x) {
    if constexpr (BF16) reinterpret_cast<u16 *>(base)[i] = f32_to_bf16_bits(x);
    else reinterpret_cast<float *>(base)[i] = x;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_gemm(int M, int N, int Kd, const void *__restrict__ A,
                                              const void *__restrict__ Bm, Epi epi) {
    using E = Elem<BF16>;
    constexpr int PAD = BF16 ? 8 : 4;
    constexpr int LS = 32 + PAD;
    __shared__ __align__(16) E As[128 * LS];
    __shared__ __align__(16) E Bs[128 * LS];   // transposed: [n][k]

    const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    const int wm = wave >> 1, wn = wave & 1, lr = lane & 15, lg = lane >> 4;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < Kd; k0 += 32) {
        __syncthreads();
        for (int task = tid; task < 128 * 4; task += 256) {   // A: 128 rows x 4 groups of 8
            const int r = task / 4, kk = (task % 4) * 8;
            float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (m0 + r < M && k0 + kk < Kd) load8<BF16>(A, (size_t)(m0 + r) * Kd + k0 + kk, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (BF16) As[r * LS + kk + e] = f32_to_bf16_bits(x[e]);
                else As[r * LS + kk + e] = x[e];
            }
        }
        for (int task = tid; task < 32 * 16; task += 256) {   // B: 32 k-rows x 16 groups of 8
            const int kk = task / 16, nn = (task % 16) * 8;
            float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (k0 + kk < Kd && n0 + nn < N) load8<BF16>(Bm, (size_t)(k0 + kk) * N + n0 + nn, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (BF16) Bs[(nn + e) * LS + kk] = f32_to_bf16_bits(x[e]);
                else Bs[(nn + e) * LS + kk] = x[e];
            }
        }
        __syncthreads();
        Frag8<BF16> af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = lds_frag8(As + (wm * 64 + i * 16 + lr) * LS + 8 * lg);
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[j] = lds_frag8(Bs + (wn * 64 + j * 16 + lr) * LS + 8 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma32(acc[i][j], af[i], bfr[j]);
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + j * 16 + lr;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 64 + i * 16 + 4 * lg + r;
                if (row >= M) continue;
                const float x = acc[i][j][r];
                if (epi.mode == 0) {
                    put<BF16>(epi.c, (size_t)row * N + col, x);
                } else if (col < epi.nq) {
                    put<BF16>(epi.q, (size_t)row * epi.nq + col, x);
                } else if (col < epi.nq + epi.nk) {
                    put<BF16>(epi.k, (size_t)row * epi.nk + (col - epi.nq), x);
                } else {
                    const int nv = N - epi.nq - epi.nk;
                    put<BF16>(epi.v, (size_t)row * nv + (col - epi.nq - epi.nk), x);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(int bf16, int M, int N, int Kd, const void *A, const void *Bm, void *C,
                       hipStream_t st) {
    Epi e{0, C, nullptr, nullptr, nullptr, 0, 0};
    const dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
    if (bf16) k_gemm<true><<<grid, 256, 0, st>>>(M, N, Kd, A, Bm, e);
    else k_gemm<false><<<grid, 256, 0, st>>>(M, N, Kd, A, Bm, e);
    return hipGetLastError();
}

hipError_t launch_gemm_qkv(int bf16, int M, int N, int Kd, const void *A, const void *Bm, void *q,
                           void *k, void *v, int nq, int nk, hipStream_t st) {
    Epi e{1, nullptr, q, k, v, nq, nk};
    const dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
    if (bf16) k_gemm<true><<<grid, 256, 0, st>>>(M, N, Kd, A, Bm, e);
    else k_gemm<false><<<grid, 256, 0, st>>>(M, N, Kd, A, Bm, e);
    return hipGetLastError();
}
