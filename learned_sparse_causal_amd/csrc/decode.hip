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
// k_decode_route: one wave per route.  The rotated query and its code
//   scores go to LDS (fp32, fused multiply-add chains in dimension order,
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
//   over four waves; each lane scores one key (rotated in fp32 from the
//   cache), each wave keeps an online softmax, and the four states are
//   merged through LDS.
#include <climits>

#include "common.hpp"

namespace {

constexpr int DR_THREADS = WAVE;   // one wave per route

// (score, id) is ordered before (score', id') when score > score', or
// scores are equal and id < id'.
__device__ __forceinline__ bool ahead(float s, int i, float s2, int i2) {
    return s > s2 || (s == s2 && i < i2);
}

// Wave arg-max of (score, id) in the order above; every lane gets the result.
__device__ __forceinline__ void wave_best(float &s, int &i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float s2 = __shfl_xor(s, o);
        const int i2 = __shfl_xor(i, o);
        if (ahead(s2, i2, s, i)) {
            s = s2;
            i = i2;
        }
    }
}

size_t decode_route_lds(const Shape &s) {
    return (size_t)(s.d + s.P * s.K + s.A + 2 * s.NB) * 4;
}

template <int D, bool BF16>
__global__ __launch_bounds__(DR_THREADS) void k_decode_route(
    Shape s, int pos, const void *__restrict__ q, const float *__restrict__ cos_t,
    const float *__restrict__ sin_t, const float *__restrict__ cb, const float *__restrict__ kbar,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ entries,
    int32_t *__restrict__ sel) {
    constexpr int H = D / 2;
    extern __shared__ __align__(16) float dr_lds[];
    float *qr = dr_lds;                          // [D] rotated query
    float *sc = qr + D;                          // [P K] code scores
    float *sig = sc + s.P * s.K;                 // [A] address sums
    int *pool_n = reinterpret_cast<int *>(sig + s.A);     // [NB]
    float *pool_r = reinterpret_cast<float *>(pool_n + s.NB);   // [NB]

    const int route = blockIdx.x;                // b * Hq + h
    const int b = route / s.Hq, h = route % s.Hq, g = h / s.G;
    const int lane = threadIdx.x;
    const int R = s.R, P = s.P, K = s.K, A = s.A, ds = s.ds;
    int32_t *out = sel + (size_t)route * R;
    const int qb = pos / s.beta;
    const int E = max(0, qb - s.L + 1);
    if (E <= R) {   // bypass: every eligible block, in order
        for (int r = lane; r < R; r += WAVE) out[r] = r < E ? r : -1;
        return;
    }
    // rotate (fp32, products rounded before the add)
    const size_t qoff = (size_t)route * D;
    for (int i = lane; i < H; i += WAVE) {
        const float a = load1<BF16>(q, qoff + i), bb = load1<BF16>(q, qoff + i + H);
        const float c = cos_t[(size_t)pos * H + i], sn = sin_t[(size_t)pos * H + i];
        const float ac = a * c, bs = bb * sn, bc = bb * c, as = a * sn;
        qr[i] = ac - bs;
        qr[i + H] = bc + as;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // code scores: fma chains in dimension order
    for (int x = lane; x < P * K; x += WAVE) {
        const int p = x / K;
        const float *crow = cb + ((size_t)g * P + p) * K * ds + (size_t)(x % K) * ds;
        const float *qp = qr + p * ds;
        float acc = 0.0f;
        for (int j = 0; j < ds; ++j) acc = fmaf(qp[j], crow[j], acc);
        sc[x] = acc;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // address sums, component 0 first (mixed radix, component 0 most significant)
    for (int a = lane; a < A; a += WAVE) {
        float v;
        if (P == 1) {
            v = sc[a];
        } else {
            v = sc[a / K] + sc[K + a % K];
        }
        sig[a] = v;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();

    const size_t u = (size_t)b * s.Hkv + g;
    const int32_t *off = offsets + u * (A + 1);
    const int32_t *ent = entries + u * s.NB;
    const int last = qb - s.L;
    float s_last = INFINITY;
    int a_last = -1;
    int npool = 0;
    for (int probed = 0; probed < A;) {
        // next address in (sum desc, address asc) order after (s_last, a_last)
        float bs = -INFINITY;
        int ba = INT_MAX;
        for (int a = lane; a < A; a += WAVE) {
            const float v = sig[a];
            if (ahead(s_last, a_last, v, a) && ahead(v, a, bs, ba)) {
                bs = v;
                ba = a;
            }
        }
        wave_best(bs, ba);
        if (ba == INT_MAX) break;   // no address left (only with non-finite sums)
        s_last = bs;
        a_last = ba;
        ++probed;
        // eligible prefix of the list (ascending block ids)
        const int e0 = off[ba], e1 = off[ba + 1];
        for (int e = e0; e < e1; e += WAVE) {
            const int n = e + lane < e1 ? ent[e + lane] : INT_MAX;
            const bool ok = n <= last;
            const uint64_t m = __ballot(ok);
            const int slot = npool + __popcll(m & ((1ull << lane) - 1ull));
            if (ok && slot < s.NB) pool_n[slot] = n;   // a valid index holds <= NB blocks
            npool = min(s.NB, npool + __popcll(m));
            if (m != ~0ull) break;   // a later block ends the prefix
        }
        if (probed >= s.npr && npool >= R) break;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // rerank: fma chain over every dimension of q_rot . kbar_n
    const float *kb = kbar + u * (size_t)s.NB * D;
    for (int x = lane; x < npool; x += WAVE) {
        const float *row = kb + (size_t)pool_n[x] * D;
        float acc = 0.0f;
        for (int j = 0; j < D; ++j) acc = fmaf(qr[j], row[j], acc);
        pool_r[x] = acc;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // the R best in (score desc, block asc) order; lane r keeps pick r
    const int nsel = min(R, npool);
    float r_last = INFINITY;
    int n_last = -1;
    int mine = -1;
    for (int r = 0; r < nsel; ++r) {
        float bs = -INFINITY;
        int bn = INT_MAX;
        for (int x = lane; x < npool; x += WAVE) {
            const float v = pool_r[x];
            const int n = pool_n[x];
            if (ahead(r_last, n_last, v, n) && ahead(v, n, bs, bn)) {
                bs = v;
                bn = n;
            }
        }
        wave_best(bs, bn);
        r_last = bs;
        n_last = bn;
        if ((r & (WAVE - 1)) == lane) mine = bn;   // R <= 16 here: one pick per lane
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

constexpr int DA_THREADS = 256;
constexpr int DA_WAVES = DA_THREADS / WAVE;

size_t decode_attend_lds(const Shape &s) {
    return (size_t)(s.d + DA_WAVES * (WAVE + 2 + s.d)) * 4 + (size_t)(s.R + s.L) * 4;
}

// One workgroup per (batch, q-head).  Logits in base 2: q is pre-scaled by
// log2(e)/sqrt(d).
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
    int *blk = reinterpret_cast<int *>(ow + DA_WAVES * D);   // [L + R]

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
    for (int it = wave; it < nitems; it += DA_WAVES) {
        const int bk = blk[it / per_blk];
        if (bk < 0) continue;
        const int s0 = bk * s.beta + (it % per_blk) * WAVE;
        if (s0 > pos) continue;
        const int key = s0 + lane;
        const bool valid = key <= pos;
        float logit = -INFINITY;
        if (valid) {
            const size_t ko = base + (size_t)key * rs;
            const float *cr = cos_t + (size_t)key * H, *sr = sin_t + (size_t)key * H;
            float acc = 0.0f;
            for (int i = 0; i < H; i += 4) {
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
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float k0 = x0[e] * cc[e] - x1[e] * ss[e];
                    const float k1 = x1[e] * cc[e] + x0[e] * ss[e];
                    acc = fmaf(qr[i + e], k0, acc);
                    acc = fmaf(qr[i + e + H], k1, acc);
                }
            }
            logit = acc;
        }
        float mx = logit;
#pragma unroll
        for (int o2 = 32; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
        const float mnew = fmaxf(m, mx);          // finite: key s0 <= pos is valid
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // exp2(-inf) = 0
        const float p = valid ? __builtin_amdgcn_exp2f(logit - mnew) : 0.0f;
        float ps = p;
#pragma unroll
        for (int o2 = 32; o2 > 0; o2 >>= 1) ps += __shfl_xor(ps, o2);
        l = l * alpha + ps;
        m = mnew;
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[j] *= alpha;
        p_s[lane] = p;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        const int nk = min(WAVE, pos - s0 + 1);
        for (int kk = 0; kk < nk; ++kk) {
            const float pk = p_s[kk];
            const size_t vo = base + (size_t)(s0 + kk) * rs;
#pragma unroll
            for (int j = 0; j < DPL; ++j) o[j] = fmaf(pk, load1<BF16>(vc, vo + lane + j * WAVE), o[j]);
        }
        __builtin_amdgcn_wave_barrier();
    }
    // merge the waves' states
    if (lane == 0) {
        ml[2 * wave] = m;
        ml[2 * wave + 1] = l;
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) ow[wave * D + lane + j * WAVE] = o[j];
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
            for (int j = 0; j < DPL; ++j) acc[j] += f * ow[w * D + lane + j * WAVE];
        }
        const float inv = 1.0f / lt;
#pragma unroll
        for (int j = 0; j < DPL; ++j) store1<BF16>(out, qoff + lane + j * WAVE, acc[j] * inv);
    }
}

template <typename F>
hipError_t lds_at_least(F *fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int D, bool BF16>
hipError_t run_decode(const Shape &s, int pos, const void *q, const void *kc, const void *vc,
                      const float *cos_t, const float *sin_t, const float *cb, const float *kbar,
                      const int32_t *offsets, const int32_t *entries, int32_t *sel, void *out,
                      hipStream_t st) {
    const unsigned routes = (unsigned)(s.B * s.Hq);
    const size_t lr = decode_route_lds(s);
    hipError_t e = lds_at_least(k_decode_route<D, BF16>, lr);
    if (e != hipSuccess) return e;
    k_decode_route<D, BF16><<<routes, DR_THREADS, lr, st>>>(s, pos, q, cos_t, sin_t, cb, kbar,
                                                            offsets, entries, sel);
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
