// Probe / rerank / top-R route for gfx950.
//
// Method (news page "Monodratic Claims Learned Routing...", section
// "Monodratic Turns Sparse Attention Into a Retrieval Decision"; technical
// report page, sections "Mixer", "Learned sparse route", "Capacity",
// "Finite-range scaling"): a query probes addresses, receives candidate
// blocks, reranks them and keeps a fixed number R of remote blocks; a block
// is never available to an earlier query; local blocks are separate; when
// every remote block is eligible within R the search is bypassed.
//
// One lane owns one query (route); one wave owns 64 consecutive tokens of one
// (batch, q-head), which all lie in one query block, so the query block, the
// eligible range and every loop over blocks are wave-uniform.
//
//  1. If E = qb - L + 1 <= R the selection is 0..E-1 (bypass).
//  2. Rotate the query (fp32, products rounded before the add), score every
//     code with an fp32 fused multiply-add chain in dimension order (the
//     codebook of the kv-head is staged in LDS and read as broadcasts), keep
//     the n_probes best codes of each component in registers.
//  3. The n_probes best addresses: an address (x-th best of component 0,
//     y-th best of component 1) has (x+1)(y+1)-1 addresses at least as good,
//     so only pairs with (x+1)(y+1) <= n_probes can be among them.  tau is
//     the key (sigma, address) of the n_probes-th best address.
//  4. Walking an address in rank order adds the causally eligible prefix of
//     its ascending list.  The walk stops once >= n_probes addresses were
//     probed and >= R blocks collected; equivalently the pool is every
//     indexed eligible block whose address key is <= max(tau, key_R), where
//     key_R is the key of the R-th best indexed eligible block.  Lanes whose
//     first n_probes addresses hold < R blocks need key_R: the wave scans
//     the eligible blocks once (block codes are uniform, each lane reads its
//     two component scores from LDS) keeping the R best block keys.
//  5. Rerank: rho = fp32 fma chain <q_rot, kbar_n> in dimension order; the
//     R best by (rho desc, block asc) are kept and written ascending.
#include "common.hpp"

namespace {

struct Key {           // an address or block key: larger sig first, then lower a, then lower n
    float sig;
    int a;
    int n;
};

__device__ __forceinline__ bool key_better(float s1, int a1, int n1, float s2, int a2, int n2) {
    return s1 > s2 || (s1 == s2 && (a1 < a2 || (a1 == a2 && n1 < n2)));
}

template <int D, int P, int NPRM, int RM, bool BF16>
__global__ __launch_bounds__(256) void k_route(Shape s, const void *__restrict__ q,
                                               const float *__restrict__ cos_t,
                                               const float *__restrict__ sin_t,
                                               const float *__restrict__ cb,
                                               const float *__restrict__ kbar,
                                               const int32_t *__restrict__ addr,
                                               const int32_t *__restrict__ offsets,
                                               const int32_t *__restrict__ entries,
                                               const int32_t *__restrict__ load,
                                               int32_t *__restrict__ sel) {
    constexpr int H = D / 2;
    constexpr int DS = D / P;
    extern __shared__ float lds[];
    const int K = s.K, PK = P * K;
    float *cb_s = lds;                               // [P*K][DS]
    const int lane = lane_id(), wave = threadIdx.x / WAVE;
    float *sc_s = lds + PK * DS + wave * PK * WAVE;  // [P*K][64] scores of this wave

    const int h = blockIdx.y, b = blockIdx.z, g = h / s.G;
    for (int x = threadIdx.x; x < PK * DS / 4; x += blockDim.x)
        reinterpret_cast<float4 *>(cb_s)[x] =
            reinterpret_cast<const float4 *>(cb + (size_t)g * PK * DS)[x];
    __syncthreads();

    const int t0 = (blockIdx.x * (int)(blockDim.x / WAVE) + wave) * WAVE;
    if (t0 >= s.T) return;
    const int t = t0 + lane;
    const bool live = t < s.T;
    const int qb = t0 / s.beta;
    const int E = max(0, qb - s.L + 1);
    const int R = s.R;
    int32_t *out = sel + (((size_t)b * s.Hq + h) * s.T + (live ? t : t0)) * R;

    if (E <= R) {  // bypass: every eligible block is selected
        if (live)
            for (int r = 0; r < R; ++r) out[r] = r < E ? r : -1;
        return;
    }

    // ---- rotated query (fp32, same rounding as the rotation's definition)
    float qr[D];
    {
        const size_t base = (((size_t)b * s.T + t) * s.Hq + h) * D;
        float x[D];
#pragma unroll
        for (int j = 0; j < D; j += 8) load8<BF16>(q, base + j, x + j);
        const float *cr = cos_t + (size_t)t * H;
        const float *sr = sin_t + (size_t)t * H;
#pragma unroll
        for (int i = 0; i < H; i += 4) {
            const float4 c4 = *reinterpret_cast<const float4 *>(cr + i);
            const float4 s4 = *reinterpret_cast<const float4 *>(sr + i);
            const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
            const float ss[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a0 = x[i + e], a1 = x[i + e + H];
                const float p0 = a0 * cc[e], p1 = a1 * ss[e], p2 = a1 * cc[e], p3 = a0 * ss[e];
                qr[i + e] = p0 - p1;
                qr[i + e + H] = p2 + p3;
            }
        }
    }

    // ---- component scores; n_probes best codes per component
    float tv[P][NPRM];
    int tc[P][NPRM];
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
        for (int x = 0; x < NPRM; ++x) { tv[p][x] = -INFINITY; tc[p][x] = -1; }
        for (int c = 0; c < K; ++c) {
            const float *crow = cb_s + (p * K + c) * DS;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < DS; j += 4) {
                const float4 cv = *reinterpret_cast<const float4 *>(crow + j);
                acc = __builtin_fmaf(qr[p * DS + j], cv.x, acc);
                acc = __builtin_fmaf(qr[p * DS + j + 1], cv.y, acc);
                acc = __builtin_fmaf(qr[p * DS + j + 2], cv.z, acc);
                acc = __builtin_fmaf(qr[p * DS + j + 3], cv.w, acc);
            }
            sc_s[(p * K + c) * WAVE + lane] = acc;
            // codes arrive in ascending order, so a strict compare keeps the
            // lower code first on equal scores
            float v = acc;
            int cc = c;
#pragma unroll
            for (int x = 0; x < NPRM; ++x) {
                const bool sw = v > tv[p][x];
                const float tvx = tv[p][x];
                const int tcx = tc[p][x];
                tv[p][x] = sw ? v : tvx;
                tc[p][x] = sw ? cc : tcx;
                v = sw ? tvx : v;
                cc = sw ? tcx : cc;
            }
        }
    }

    // ---- the n_probes best addresses
    const int A = s.A;
    const int npr = min(s.npr, A);
    float av[NPRM];
    int aa[NPRM];
    if constexpr (P == 1) {
#pragma unroll
        for (int x = 0; x < NPRM; ++x) { av[x] = tv[0][x]; aa[x] = tc[0][x]; }
    } else {
#pragma unroll
        for (int x = 0; x < NPRM; ++x) { av[x] = -INFINITY; aa[x] = 0x7fffffff; }
#pragma unroll
        for (int x = 0; x < NPRM; ++x) {
#pragma unroll
            for (int y = 0; y < NPRM; ++y) {
                if ((x + 1) * (y + 1) > NPRM) continue;
                const bool ok = (x + 1) * (y + 1) <= npr && tc[0][x] >= 0 && tc[1][y] >= 0;
                float v = ok ? tv[0][x] + tv[1][y] : -INFINITY;
                int a = ok ? tc[0][x] * K + tc[1][y] : 0x7fffffff;
#pragma unroll
                for (int z = 0; z < NPRM; ++z) {
                    const bool sw = v > av[z] || (v == av[z] && a < aa[z]);
                    const float avz = av[z];
                    const int aaz = aa[z];
                    av[z] = sw ? v : avz;
                    aa[z] = sw ? a : aaz;
                    v = sw ? avz : v;
                    a = sw ? aaz : a;
                }
            }
        }
    }
    float tau_s = av[0];
    int tau_a = aa[0];
#pragma unroll
    for (int x = 1; x < NPRM; ++x)
        if (x == npr - 1) { tau_s = av[x]; tau_a = aa[x]; }

    // ---- rerank state: RM slots, best first; the first RM-R are sentinels
    float rv[RM];
    int rn[RM];
#pragma unroll
    for (int x = 0; x < RM; ++x) {
        const bool sent = x < RM - R;
        rv[x] = sent ? INFINITY : -INFINITY;
        rn[x] = sent ? -1 : 0x7fffffff;
    }
    const size_t ug = (size_t)b * s.Hkv + g;
    const float *kb = kbar + ug * s.NB * D;
    const int32_t *off = offsets + ug * (A + 1);
    const int32_t *ent = entries + ug * s.NB;
    const int32_t *ad = addr + ug * s.NB;
    const int32_t *ldv = load + ug * A;
    const int last = qb - s.L;

    auto rerank = [&](int n) {
        const float *kr = kb + (size_t)n * D;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < D; j += 4) {
            const float4 kv = *reinterpret_cast<const float4 *>(kr + j);
            acc = __builtin_fmaf(qr[j], kv.x, acc);
            acc = __builtin_fmaf(qr[j + 1], kv.y, acc);
            acc = __builtin_fmaf(qr[j + 2], kv.z, acc);
            acc = __builtin_fmaf(qr[j + 3], kv.w, acc);
        }
        float v = acc;
        int nn = n;
#pragma unroll
        for (int x = 0; x < RM; ++x) {
            const bool sw = v > rv[x] || (v == rv[x] && nn < rn[x]);
            const float rvx = rv[x];
            const int rnx = rn[x];
            rv[x] = sw ? v : rvx;
            rn[x] = sw ? nn : rnx;
            v = sw ? rvx : v;
            nn = sw ? rnx : nn;
        }
    };

    // ---- pool part 1: the eligible prefixes of the n_probes best lists
    int cnt = 0;
    if (live) {
#pragma unroll
        for (int x = 0; x < NPRM; ++x) {
            if (x >= npr) break;
            const int a = aa[x];
            const int e1 = off[a + 1];
            for (int e = off[a]; e < e1; ++e) {
                const int n = ent[e];
                if (n > last) break;
                rerank(n);
                ++cnt;
            }
        }
    }

    // ---- pool part 2: extension to R blocks, for lanes that need it
    const bool need = live && cnt < R;
    if (__ballot(need) != 0ull) {
        float kv_[RM];
        int ka_[RM], kn_[RM];
#pragma unroll
        for (int x = 0; x < RM; ++x) {
            const bool sent = x < RM - R;
            kv_[x] = sent ? INFINITY : -INFINITY;
            ka_[x] = sent ? -1 : 0x7fffffff;
            kn_[x] = sent ? -1 : 0x7fffffff;
        }
        const int cap = s.cap;
        for (int n = 0; n <= last; ++n) {
            const int a = uniform(ad[n]);
            if (uniform(ldv[a]) > cap) {
                // the list is full: n is kept iff it is not after its last entry
                const int o = uniform(off[a]);
                if (n > uniform(ent[o + cap - 1])) continue;
            }
            float sg;
            if constexpr (P == 1) {
                sg = sc_s[a * WAVE + lane];
            } else {
                const int c0 = a / K, c1 = a - c0 * K;
                sg = sc_s[c0 * WAVE + lane] + sc_s[(K + c1) * WAVE + lane];
            }
            if (need) {
                float v = sg;
                int va = a, vn = n;
#pragma unroll
                for (int x = 0; x < RM; ++x) {
                    const bool sw = key_better(v, va, vn, kv_[x], ka_[x], kn_[x]);
                    const float kvx = kv_[x];
                    const int kax = ka_[x], knx = kn_[x];
                    kv_[x] = sw ? v : kvx;
                    ka_[x] = sw ? va : kax;
                    kn_[x] = sw ? vn : knx;
                    v = sw ? kvx : v;
                    va = sw ? kax : va;
                    vn = sw ? knx : vn;
                }
            }
        }
        if (need) {
            // blocks ranked after tau among the R best (the rest are in part 1)
#pragma unroll
            for (int x = 0; x < RM; ++x) {
                if (x < RM - R) continue;
                if (kn_[x] == 0x7fffffff) continue;   // fewer than R indexed eligible blocks
                const bool after_tau =
                    kv_[x] < tau_s || (kv_[x] == tau_s && ka_[x] > tau_a);
                if (after_tau) rerank(kn_[x]);
            }
            // the R-th block's address ties with it: its remaining eligible blocks
            if (kn_[RM - 1] != 0x7fffffff) {
                const int aR = ka_[RM - 1], nR = kn_[RM - 1];
                const bool after_tau =
                    kv_[RM - 1] < tau_s || (kv_[RM - 1] == tau_s && aR > tau_a);
                if (after_tau) {
                    const int e1 = off[aR + 1];
                    for (int e = off[aR]; e < e1; ++e) {
                        const int n = ent[e];
                        if (n > last) break;
                        if (n > nR) rerank(n);
                    }
                }
            }
        }
    }

    // ---- emit the kept blocks ascending, -1 padded
    int o[RM];
#pragma unroll
    for (int x = 0; x < RM; ++x) o[x] = (x >= RM - R && rn[x] != 0x7fffffff) ? rn[x] : 0x7fffffff;
#pragma unroll
    for (int pass = 0; pass < RM; ++pass) {
#pragma unroll
        for (int x = pass & 1; x + 1 < RM; x += 2) {
            const int lo = min(o[x], o[x + 1]), hi = max(o[x], o[x + 1]);
            o[x] = lo;
            o[x + 1] = hi;
        }
    }
    if (live) {
#pragma unroll
        for (int x = 0; x < RM; ++x)
            if (x < R) out[x] = o[x] == 0x7fffffff ? -1 : o[x];
    }
}

// Bypass-only route (every query has E <= R): any R.
__global__ __launch_bounds__(256) void k_route_bypass(Shape s, int32_t *__restrict__ sel) {
    const long route = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (route >= (long)s.B * s.Hq * s.T) return;
    const int t = (int)(route % s.T);
    const int E = max(0, t / s.beta - s.L + 1);
    int32_t *out = sel + (size_t)route * s.R;
    for (int r = 0; r < s.R; ++r) out[r] = r < E ? r : -1;
}

template <int D, int P, int NPRM, int RM, bool BF16>
hipError_t launch_t(const Shape &s, const void *q, const float *cos_t, const float *sin_t,
                    const float *cb, const float *kbar, const int32_t *addr,
                    const int32_t *offsets, const int32_t *entries, const int32_t *load,
                    int32_t *sel, hipStream_t st) {
    const int PK = P * s.K;
    const int waves = PK <= 64 ? 4 : 2;
    const size_t lds = (size_t)(PK * (D / P) + waves * PK * WAVE) * sizeof(float);
    const dim3 grid((unsigned)((s.T + waves * WAVE - 1) / (waves * WAVE)), (unsigned)s.Hq,
                    (unsigned)s.B);
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(k_route<D, P, NPRM, RM, BF16>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    k_route<D, P, NPRM, RM, BF16><<<grid, waves * WAVE, lds, st>>>(
        s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries, load, sel);
    return hipGetLastError();
}

template <int D, int P, bool BF16>
hipError_t launch_sel(const Shape &s, const void *q, const float *cos_t, const float *sin_t,
                      const float *cb, const float *kbar, const int32_t *addr,
                      const int32_t *offsets, const int32_t *entries, const int32_t *load,
                      int32_t *sel, hipStream_t st) {
    if (s.npr <= 2 && s.R <= 2)
        return launch_t<D, P, 2, 2, BF16>(s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries,
                                          load, sel, st);
    if (s.npr <= 4 && s.R <= 2)
        return launch_t<D, P, 4, 2, BF16>(s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries,
                                          load, sel, st);
    if (s.npr <= 8 && s.R <= 8)
        return launch_t<D, P, 8, 8, BF16>(s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries,
                                          load, sel, st);
    return launch_t<D, P, 16, 16, BF16>(s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries,
                                        load, sel, st);
}

}  // namespace

hipError_t launch_route(const Shape &s, const void *q, const float *cos_t, const float *sin_t,
                        const float *cb, const float *kbar, const int32_t *addr,
                        const int32_t *offsets, const int32_t *entries, const int32_t *load,
                        int32_t *sel, hipStream_t st) {
    if (s.NB - s.L <= s.R) {  // every query bypasses the search
        const long routes = (long)s.B * s.Hq * s.T;
        k_route_bypass<<<dim3((unsigned)((routes + 255) / 256)), 256, 0, st>>>(s, sel);
        return hipGetLastError();
    }
    const bool bf = s.dtype == 1;
#define MONO_ROUTE_ARGS s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries, load, sel, st
    if (s.d == 64) {
        if (s.P == 1) return bf ? launch_sel<64, 1, true>(MONO_ROUTE_ARGS)
                                : launch_sel<64, 1, false>(MONO_ROUTE_ARGS);
        return bf ? launch_sel<64, 2, true>(MONO_ROUTE_ARGS) : launch_sel<64, 2, false>(MONO_ROUTE_ARGS);
    }
    if (s.P == 1) return bf ? launch_sel<128, 1, true>(MONO_ROUTE_ARGS)
                            : launch_sel<128, 1, false>(MONO_ROUTE_ARGS);
    return bf ? launch_sel<128, 2, true>(MONO_ROUTE_ARGS) : launch_sel<128, 2, false>(MONO_ROUTE_ARGS);
#undef MONO_ROUTE_ARGS
}
