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
// eligible range and every loop over blocks are wave-uniform.  A workgroup's
// four waves share one (batch, kv-head): its list offsets, list entries and,
// per indexed block, the score-table rows of its component codes are staged
// in LDS once, so list walks and block scans never wait on global memory.
// The VALU scoring path reads the codebook with wave-uniform addresses
// (scalar loads); the matrix-core path loads its B operands per lane at the
// start of the kernel.
//
//  1. If E = qb - L + 1 <= R the selection is 0..E-1 (bypass).
//  2. Rotate the query (fp32, products rounded before the add), score every
//     code with an fp32 fused multiply-add chain in dimension order, keep
//     the n_probes best codes of each component.
//  3. The n_probes best addresses: an address (x-th best of component 0,
//     y-th best of component 1) has (x+1)(y+1)-1 addresses at least as good,
//     so only pairs with (x+1)(y+1) <= n_probes can be among them.  tau is
//     the key of the n_probes-th best address.
//  4. The walk in rank order stops once >= n_probes addresses were probed
//     and >= R blocks collected; equivalently the pool is every indexed
//     eligible block whose address key is <= max(tau, key_R), key_R being
//     the key of the address that holds the R-th eligible block in walk
//     order.  Lanes whose first n_probes lists hold < R eligible blocks need
//     key_R, which lies among the R best addresses that hold an eligible
//     block.  The wave scans the workgroup's list of such addresses, kept
//     in ascending address order, so that of two equal sums the lower
//     address is met first and kept (R <= 2: one pass over values plus the
//     batches they came from; larger R: one pass over values and a second
//     that collects the addresses).  The scan is bounded by the number of
//     addresses, whatever the sequence length.
//  5. Rerank: rho = fp32 fma chain <q_rot, kbar_n> in dimension order; the
//     R best by (rho desc, block asc) are kept and written ascending.
//
// Ordered choices use 64-bit keys where a larger key is better: the high
// word is the score mapped to an order-preserving unsigned integer, the low
// word breaks ties toward the lower address / code / block.
#include <type_traits>

#include "common.hpp"

namespace {

typedef unsigned long long u64;

// Order-preserving map of a float to an unsigned integer; -0 is taken as +0,
// as the float comparison takes it.
__device__ __forceinline__ uint32_t ordered(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// address/code/block keys: larger score first, then lower index
__device__ __forceinline__ u64 key_of(float s, uint32_t low_rank) {
    return ((u64)ordered(s) << 32) | (u64)low_rank;
}

__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int off) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
    return ((u64)hi << 32) | lo;
}

template <int M>
__device__ __forceinline__ void insert(u64 (&lst)[M], u64 k) {
#pragma unroll
    for (int x = 0; x < M; ++x) {
        const u64 cur = lst[x];
        const bool sw = k > cur;
        lst[x] = sw ? k : cur;
        k = sw ? cur : k;
    }
}

// Entries the extension scan reads past the end of the address list (its
// row offsets are loaded two batches ahead).
constexpr int SCAN_U = 8, SCAN_PAD = 2 * SCAN_U;

// Addresses the extension's list can hold: those with an indexed block.
__host__ __device__ constexpr int route_list_max(int NB, int A) { return NB < A ? NB : A; }

// Workgroup LDS, in 4-byte words: the address list (int2 score-row offsets,
// list_max + SCAN_PAD entries), its length, the list offsets [A + 1] and the
// list entries [NB]; then the per-wave score areas, 16-byte aligned.
__host__ __device__ constexpr int route_sc_off(int NB, int A) {
    return (2 * (route_list_max(NB, A) + SCAN_PAD) + 1 + A + 1 + NB + 3) & ~3;
}

// Floats per score row: 64 lanes plus 4 of padding, so the 16 rows one
// matrix-core result store writes start on different banks.
constexpr int SROW = 64 + 4;

// Floats of one wave's score area: P*K score rows and a -inf row; with
// matrix-core scoring it first holds the wave's 64 rotated rows (SROW
// floats each, or DS + 4 for the one-component-at-a-time transpose).
__host__ __device__ constexpr int route_wave_floats(int PK, int DS, bool mf) {
    return mf && 64 * SROW > (PK + 1) * SROW ? 64 * SROW : (PK + 1) * SROW;
}

// List offsets and (entry, address) pairs each thread loads per staging
// round before storing any (a round covers STAGE_OFF * threads offsets and
// half as many blocks).
constexpr int STAGE_OFF = 8, STAGE_BLK = STAGE_OFF / 2;

// At most 8 probes fits 256 registers (two waves per SIMD, the most the LDS
// allows); without the cap the compiler spends AGPRs on the matrix-core
// accumulators (d = 64) or on the rerank's summary loads (d = 128) and
// drops to one.  At d = 128 the rerank loads the summaries in quarters so
// that they fit beside the 128 registers of the rotated query, at the cost
// of a few spilled registers on the path past the register batch.
template <int D, int P, int NPRM, int RM, bool BF16, bool MF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NPRM <= 8 ? 2 : 1)))
void k_route(Shape s, const void *__restrict__ q, const float *__restrict__ cos_t,
             const float *__restrict__ sin_t, const float *__restrict__ cb,
             const float *__restrict__ kbar, const int32_t *__restrict__ addr,
             const int32_t *__restrict__ offsets, const int32_t *__restrict__ entries,
             int32_t *__restrict__ sel, void *__restrict__ q_rot) {
    constexpr int H = D / 2;
    constexpr int DS = D / P;
    extern __shared__ float lds[];
    const int K = s.K, PK = P * K, A = s.A, NB = s.NB;
    const int nw = blockDim.x / WAVE;
    const int LMAX = route_list_max(NB, A);
    int2 *alist = reinterpret_cast<int2 *>(lds);                 // [LMAX + SCAN_PAD]: score-row offsets
    int *nal_s = reinterpret_cast<int *>(alist + LMAX + SCAN_PAD);   // list length
    int *off_s = nal_s + 1;                                      // [A+1]
    int *ent_s = off_s + A + 1;                                  // [NB]
    float *sc_all = reinterpret_cast<float *>(lds) + route_sc_off(NB, A);   // [nw][...][64]
    const int lane = lane_id(), wave = uniform(threadIdx.x / WAVE);
    float *sc_s = sc_all + wave * route_wave_floats(PK, DS, MF);
    const int dummy = PK * SROW * 4;                             // byte offset of a -inf row

    // Work items: (token group, batch, q-head) with the q-heads fastest and
    // the latest token groups (the longest extension scans) first.  The
    // workgroups are dealt to the 8 XCDs round-robin (workgroup i is the
    // (i / 8)-th on XCD i % 8), and the items are placed for that: the token
    // groups go to the XCDs in rank order (rank k on XCD k % 8), so every XCD
    // gets heavy and light groups alike, and each XCD runs all batches and
    // q-heads of its group together, so that they share the group's
    // rotary-table rows in that XCD's L2 (dealt item by item, every XCD would
    // fetch every group's rows).  Each XCD then reads the block summaries of
    // every (batch, kv-head) in its reranks, so this placement is used only
    // while they all fit in half an L2 (2 MiB; measured: on the batch-8
    // 64K-token workload, 8 MiB of summaries, it made the router 30 %
    // slower).  Otherwise, or with a group count that is not a multiple of
    // 8, the items run in plain order (each XCD then sees a few kv-heads).
    const int ngrp = (s.T + nw * WAVE - 1) / (nw * WAVE);
    const int per_grp = s.Hq * s.B;
    const bool by_xcd = ngrp % 8 == 0 && (size_t)s.B * s.Hkv * NB * D * sizeof(float) <= (2u << 20);
    const int item = by_xcd
        ? ((int)(blockIdx.x / 8) / per_grp * 8 + (int)(blockIdx.x % 8)) * per_grp +
              (int)(blockIdx.x / 8) % per_grp
        : (int)blockIdx.x;
    const int h = item % s.Hq, b = (item / s.Hq) % s.B, g = h / s.G;
    const size_t ug = (size_t)b * s.Hkv + g;
    const int tw0 = (ngrp - 1 - item / (s.Hq * s.B)) * nw * WAVE;   // first token of the workgroup
    const int R = s.R;
    // blocks the workgroup can need: eligible for its last wave
    const int nblk = min(NB, max(0, (min(s.T, tw0 + nw * WAVE) - 1) / s.beta - s.L + 1));
    const bool any_search = nblk > R;

    const int t0 = tw0 + wave * WAVE;
    const int t = t0 + lane;
    const bool live = t < s.T;
    const int qb = t0 / s.beta;
    const int E = max(0, qb - s.L + 1);
    const int tq = min(t, s.T - 1);        // clamped: the loads below stay in bounds
    const size_t qbase = (((size_t)b * s.T + tq) * s.Hq + h) * D;

    // List offsets and list entries of the (batch, kv-head) are staged in
    // LDS.  Every thread issues its loads of a round (indexes clamped, so
    // none is predicated) before storing any.  The first round's loads are
    // issued before the wave's own loads, so its stores wait for them only.
    const int32_t *off_g = offsets + ug * (A + 1);
    const int32_t *ent_g = entries + ug * NB;
    const int32_t *ad_g = addr + ug * NB;
    const int bd = blockDim.x, tid = threadIdx.x;
    int vo[STAGE_OFF], ve[STAGE_BLK];
    auto stage_load = [&](int r0) {
#pragma unroll
        for (int u = 0; u < STAGE_OFF; ++u) vo[u] = off_g[min(r0 + u * bd + tid, A)];
#pragma unroll
        for (int u = 0; u < STAGE_BLK; ++u) ve[u] = ent_g[min(r0 / 2 + u * bd + tid, NB - 1)];
    };
    // (stores use the same clamped indexes: threads past the end rewrite the
    // last element with its own value)
    auto stage_store = [&](int r0) {
#pragma unroll
        for (int u = 0; u < STAGE_OFF; ++u) off_s[min(r0 + u * bd + tid, A)] = vo[u];
#pragma unroll
        for (int u = 0; u < STAGE_BLK; ++u) ent_s[min(r0 / 2 + u * bd + tid, NB - 1)] = ve[u];
    };
    if (any_search) stage_load(0);
    __builtin_amdgcn_sched_barrier(0);

    // For d = 64 in bf16 the wave's own global loads come next (the raw
    // query row, the rotary rows and, for matrix-core scoring, every
    // codebook operand), so that they are in flight while the workgroup
    // stages its lists; the barriers below wait for LDS only.  They are
    // issued by every wave (a predicated load would make the wait counts
    // after it conservative), and wider rows would hold too many registers
    // across the staging.
    constexpr int NTM = MF ? 2 : 1, NSM = MF ? DS / 4 : 1;   // matrix-core: K <= 32
    // Matrix-core scoring in bf16 loads and rotates the wave's 64 rows
    // cooperatively: lane l takes rows l/8 + 8j (j < 8) and the rotation
    // pairs 4(l%8) .. 4(l%8)+3 of each, so one load instruction covers 8
    // rows instead of 64 (a row per lane touches a cache line per lane).
    constexpr bool COOP = MF && BF16;
    constexpr int CJ = COOP ? 8 : 1;
    constexpr bool EARLY_ROT = D <= 64 && BF16 && !COOP;
    constexpr int QW = BF16 ? D / 8 : D / 4;                 // 16-byte words of the row
    constexpr int RW = EARLY_ROT ? H / 4 : 1;
    u32x4 qraw[QW];
    float4 cs4[RW], sn4[RW];
    float bpre[P][NTM][NSM];
    const float4 *cr = reinterpret_cast<const float4 *>(cos_t + (size_t)tq * H);
    const float4 *sr = reinterpret_cast<const float4 *>(sin_t + (size_t)tq * H);
    const u32x4 *qsrc = BF16 ? reinterpret_cast<const u32x4 *>(
                                   reinterpret_cast<const u16 *>(q) + qbase)
                             : reinterpret_cast<const u32x4 *>(
                                   reinterpret_cast<const float *>(q) + qbase);
    uint2 qlo[CJ], qhi[CJ];
    float4 cj[CJ], sj[CJ];
    {
        if constexpr (COOP) {
            const int k4 = 4 * (lane & 7);
#pragma unroll
            for (int j = 0; j < CJ; ++j) {
                const int tr = min(t0 + (lane >> 3) + 8 * j, s.T - 1);
                const u16 *qrow = reinterpret_cast<const u16 *>(q) + (((size_t)b * s.T + tr) * s.Hq + h) * D;
                qlo[j] = *reinterpret_cast<const uint2 *>(qrow + k4);
                qhi[j] = *reinterpret_cast<const uint2 *>(qrow + H + k4);
                cj[j] = *reinterpret_cast<const float4 *>(cos_t + (size_t)tr * H + k4);
                sj[j] = *reinterpret_cast<const float4 *>(sin_t + (size_t)tr * H + k4);
            }
        }
        if constexpr (EARLY_ROT) {
#pragma unroll
            for (int j = 0; j < QW; ++j) qraw[j] = qsrc[j];
#pragma unroll
            for (int i = 0; i < RW; ++i) {
                cs4[i] = cr[i];
                sn4[i] = sr[i];
            }
        }
        if constexpr (MF) {
            // B operand of code nt*16 + (lane & 15), dimension 4 st + lane / 16
            const float *cbg = cb + (size_t)g * PK * DS;
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int nt = 0; nt < NTM; ++nt) {
                    const int code = nt * 16 + (lane & 15);
                    const float *brow = cbg + (p * K + (code < K ? code : 0)) * DS + (lane >> 4);
#pragma unroll
                    for (int st = 0; st < NSM; ++st) bpre[p][nt][st] = brow[4 * st];   // clamped row
                }
        }
    }

    __builtin_amdgcn_sched_barrier(0);
    if (any_search) {
        stage_store(0);
        for (int r0 = STAGE_OFF * bd; r0 <= A || r0 / 2 < NB; r0 += STAGE_OFF * bd) {
            stage_load(r0);
            stage_store(r0);
        }
    }
    __syncthreads();
    // Byte offsets of the score-table rows of an address's component codes
    // (relative to the lane's column), and the address back from them.
    auto row_offsets = [&](int a) {
        const int c0 = P == 1 ? a : a / K, c1 = P == 1 ? 0 : a - c0 * K;
        return make_int2(c0 * SROW * 4, P == 1 ? dummy : (K + c1) * SROW * 4);
    };
    auto addr_of = [&](int2 m) {
        const int c0 = m.x / (SROW * 4);
        return P == 1 ? c0 : c0 * K + (m.y / (SROW * 4) - K);
    };
    // the first wave's last eligible block (later waves have later ones)
    const int last0 = tw0 / s.beta - s.L;
    if (any_search) {
        // The extension's address list: every address whose first (lowest)
        // indexed block is eligible for the workgroup's first wave, in
        // ascending address order.  Thread t owns addresses
        // [t * per, (t + 1) * per); a workgroup scan of the counts places
        // them.  The scan's read-ahead past the end lands on the -inf row.
        const int per = (A + bd - 1) / bd;
        const int a_lo = min(tid * per, A), a_hi = min(a_lo + per, A);
        int c = 0;
        for (int a = a_lo; a < a_hi; ++a) {
            const int e0 = off_s[a];
            c += (e0 < off_s[a + 1] && ent_s[e0] <= last0) ? 1 : 0;
        }
        int x = c;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const int y = __shfl_up(x, o);
            x += lane >= o ? y : 0;
        }
        // the score areas are not in use yet: wave totals go there
        int *wsum = reinterpret_cast<int *>(sc_all);
        if (lane == WAVE - 1) wsum[wave] = x;
        __syncthreads();
        int pos = x - c, tot = 0;
        for (int w = 0; w < nw; ++w) {
            const int v = wsum[w];
            pos += w < wave ? v : 0;
            tot += v;
        }
        for (int a = a_lo; a < a_hi; ++a) {
            const int e0 = off_s[a];
            if (e0 < off_s[a + 1] && ent_s[e0] <= last0) alist[pos++] = row_offsets(a);
        }
        for (int i = tid; i < SCAN_PAD; i += bd) alist[tot + i] = make_int2(dummy, dummy);
        if (tid == 0) *nal_s = tot;
    }
    __syncthreads();

    if (t0 >= s.T) return;
    int32_t *out = sel + (((size_t)b * s.Hq + h) * s.T + (live ? t : t0)) * R;

    if (E <= R && !q_rot) {  // bypass: every eligible block is selected
        if (live)
            for (int r = 0; r < R; ++r) out[r] = r < E ? r : -1;
        return;
    }

    // ---- rotated query (fp32, same rounding as the rotation's definition)
    float qr[D];
    if constexpr (COOP) {
        // rotated rows go to the wave's score area, [row][SROW], with
        // dimension p*DS + 4 st + lg at float p*DS + lg*(DS/4) + st: the
        // layout the matrix-core A fragments read as float4s
        constexpr int NS = DS / 4;
        const int k = lane & 7;
        const float sc = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
        for (int j = 0; j < CJ; ++j) {
            const int r = (lane >> 3) + 8 * j;
            const uint32_t w[4] = {qlo[j].x, qlo[j].y, qhi[j].x, qhi[j].y};
            const float lo[4] = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
            const float hi[4] = {__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xFFFF0000u),
                                 __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xFFFF0000u)};
            const float cc[4] = {cj[j].x, cj[j].y, cj[j].z, cj[j].w};
            const float ss[4] = {sj[j].x, sj[j].y, sj[j].z, sj[j].w};
            float rl[4], rh[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = lo[e] * cc[e], p1 = hi[e] * ss[e], p2 = hi[e] * cc[e], p3 = lo[e] * ss[e];
                rl[e] = p0 - p1;
                rh[e] = p2 + p3;
                sc_s[r * SROW + e * NS + k] = rl[e];           // dimension 4k + e
                sc_s[r * SROW + DS + e * NS + k] = rh[e];      // dimension H + 4k + e
            }
            // the attention's copy: pre-scaled by log2(e)/sqrt(d), bf16
            if (q_rot && t0 + r < s.T) {
                u16 *dst = reinterpret_cast<u16 *>(q_rot) + (((size_t)b * s.T + t0 + r) * s.Hq + h) * D;
                *reinterpret_cast<uint2 *>(dst + 4 * k) =
                    make_uint2(pack_bf16x2(rl[0] * sc, rl[1] * sc), pack_bf16x2(rl[2] * sc, rl[3] * sc));
                *reinterpret_cast<uint2 *>(dst + H + 4 * k) =
                    make_uint2(pack_bf16x2(rh[0] * sc, rh[1] * sc), pack_bf16x2(rh[2] * sc, rh[3] * sc));
            }
        }
        __builtin_amdgcn_wave_barrier();
        // the lane's own row, back in dimension order
#pragma unroll
        for (int m = 0; m < D / 4; ++m) {
            const float4 v = *reinterpret_cast<const float4 *>(sc_s + lane * SROW + 4 * m);
            const int p = m / 8, lg = (m % 8) / 2, st0 = 4 * (m % 2);
            qr[p * DS + 4 * (st0 + 0) + lg] = v.x;
            qr[p * DS + 4 * (st0 + 1) + lg] = v.y;
            qr[p * DS + 4 * (st0 + 2) + lg] = v.z;
            qr[p * DS + 4 * (st0 + 3) + lg] = v.w;
        }
    } else {
        float x[D];
        if constexpr (!EARLY_ROT) {
#pragma unroll
            for (int j = 0; j < QW; ++j) qraw[j] = qsrc[j];
        }
#pragma unroll
        for (int j = 0; j < QW; ++j) {
            const uint32_t w[4] = {qraw[j][0], qraw[j][1], qraw[j][2], qraw[j][3]};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (BF16) {
                    x[8 * j + 2 * e] = __uint_as_float(w[e] << 16);
                    x[8 * j + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                } else {
                    x[4 * j + e] = __uint_as_float(w[e]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < H; i += 4) {
            const float4 c4 = EARLY_ROT ? cs4[EARLY_ROT ? i / 4 : 0] : cr[i / 4];
            const float4 s4 = EARLY_ROT ? sn4[EARLY_ROT ? i / 4 : 0] : sr[i / 4];
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
        // the attention's copy of the row: pre-scaled by log2(e)/sqrt(d) and
        // rounded to the activation dtype
        if (q_rot && live) {
            const float sc = 1.4426950408889634f / sqrtf((float)D);
            if constexpr (BF16) {
                u32x4 *dst = reinterpret_cast<u32x4 *>(reinterpret_cast<u16 *>(q_rot) + qbase);
#pragma unroll
                for (int j = 0; j < D; j += 8)
                    dst[j / 8] = u32x4{pack_bf16x2(qr[j] * sc, qr[j + 1] * sc),
                                       pack_bf16x2(qr[j + 2] * sc, qr[j + 3] * sc),
                                       pack_bf16x2(qr[j + 4] * sc, qr[j + 5] * sc),
                                       pack_bf16x2(qr[j + 6] * sc, qr[j + 7] * sc)};
            } else {
                float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(q_rot) + qbase);
#pragma unroll
                for (int j = 0; j < D; j += 4)
                    dst[j / 4] = make_float4(qr[j] * sc, qr[j + 1] * sc, qr[j + 2] * sc,
                                             qr[j + 3] * sc);
            }
        }
    }
    if (E <= R) {  // bypass: every eligible block is selected
        if (live)
            for (int r = 0; r < R; ++r) out[r] = r < E ? r : -1;
        return;
    }

    // ---- component scores; the n_probes best codes of each component
    float tv[P][NPRM];
    int tc[P][NPRM];
    // insert (v, c) into a list sorted best first; codes arrive ascending,
    // so a strict compare keeps the lower code first on equal scores.  Slot
    // x takes the median of (old slot x-1, old slot x, v).
    auto top_insert = [](float (&tvp)[NPRM], int (&tcp)[NPRM], float v, int c) {
        bool bt[NPRM];
#pragma unroll
        for (int x = 0; x < NPRM; ++x) bt[x] = v > tvp[x];
#pragma unroll
        for (int x = NPRM - 1; x > 0; --x) {
            const int cx = bt[x] ? c : tcp[x];
            tcp[x] = bt[x - 1] ? tcp[x - 1] : cx;
            tvp[x] = __builtin_amdgcn_fmed3f(tvp[x - 1], tvp[x], v);
        }
        tcp[0] = bt[0] ? c : tcp[0];
        tvp[0] = bt[0] ? v : tvp[0];
    };
    if constexpr (MF) {
        // Matrix cores: per component, D[route][code] = sum_k A[route][k]
        // B[k][code] as a chain of fp32 16x16x4 MFMAs over steps st, with
        // lane group lg carrying dimension 4 st + lg.  Each MFMA adds its
        // four products in k order, one rounding each, so the chain is the
        // fused multiply-add chain in dimension order.  The A operand (the
        // routes' rotated queries) passes through the wave's score area,
        // one component at a time; every A fragment is in registers before
        // the first score is written there.
        const int lr = lane & 15, lg = lane >> 4;
        constexpr int MT = WAVE / 16, NS = DS / 4;
        constexpr int QTS = DS + 4;                      // transpose row stride (floats)
        float af[P][MT][NS];
        if constexpr (COOP) {
            // the rotated rows are already in the A-fragment layout
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int st = 0; st < NS; st += 4) {
                        const float4 v4 = *reinterpret_cast<const float4 *>(
                            sc_s + (mt * 16 + lr) * SROW + p * DS + lg * NS + st);
                        af[p][mt][st] = v4.x;
                        af[p][mt][st + 1] = v4.y;
                        af[p][mt][st + 2] = v4.z;
                        af[p][mt][st + 3] = v4.w;
                    }
        } else {
#pragma unroll
        for (int p = 0; p < P; ++p) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
                for (int st = 0; st < NS; st += 4)
                    *reinterpret_cast<float4 *>(sc_s + lane * QTS + g4 * NS + st) =
                        make_float4(qr[p * DS + 4 * st + g4], qr[p * DS + 4 * (st + 1) + g4],
                                    qr[p * DS + 4 * (st + 2) + g4], qr[p * DS + 4 * (st + 3) + g4]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int st = 0; st < NS; st += 4) {
                    const float4 v4 =
                        *reinterpret_cast<const float4 *>(sc_s + (mt * 16 + lr) * QTS + lg * NS + st);
                    af[p][mt][st] = v4.x;
                    af[p][mt][st + 1] = v4.y;
                    af[p][mt][st + 2] = v4.z;
                    af[p][mt][st + 3] = v4.w;
                }
        }
        }
        // Component p: the MFMA chains of both 16-code tiles (codes past K
        // have zero columns and are not stored), then the stores into the
        // score table.  With 32 codes the ranking of component 0 is
        // straight-line code placed after component 1's chains are issued,
        // so its VALU work fills the matrix pipe's time.
        f32x4 acc[P][NTM][MT];
        auto chains = [&](int p) {
#pragma unroll
            for (int nt = 0; nt < NTM; ++nt) {
                const int code = nt * 16 + lr;
                float bf[NS];
#pragma unroll
                for (int st = 0; st < NS; ++st) bf[st] = code < K ? bpre[p][nt][st] : 0.0f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[p][nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < NS; ++st)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[p][nt][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            af[p][mt][st], bf[st], acc[p][nt][mt], 0, 0, 0);
            }
        };
        auto store = [&](int p, auto all_codes) {
#pragma unroll
            for (int nt = 0; nt < NTM; ++nt) {
                // lane holds routes mt*16 + 4 lg + r of code nt*16 + lr
                const int code = nt * 16 + lr;
                if (decltype(all_codes)::value || code < K) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        *reinterpret_cast<float4 *>(sc_s + (p * K + code) * SROW + mt * 16 + 4 * lg) =
                            make_float4(acc[p][nt][mt][0], acc[p][nt][mt][1], acc[p][nt][mt][2],
                                        acc[p][nt][mt][3]);
                }
            }
        };
        auto rank_codes = [&](int p, auto kc) {
#pragma unroll
            for (int x = 0; x < NPRM; ++x) { tv[p][x] = -INFINITY; tc[p][x] = -1; }
            if constexpr (decltype(kc)::value > 0) {
#pragma unroll
                for (int c = 0; c < decltype(kc)::value; ++c)
                    top_insert(tv[p], tc[p], sc_s[(p * K + c) * SROW + lane], c);
            } else {
#pragma unroll 4
                for (int c = 0; c < K; ++c) top_insert(tv[p], tc[p], sc_s[(p * K + c) * SROW + lane], c);
            }
        };
        using all_codes = std::integral_constant<bool, true>;
        using some_codes = std::integral_constant<bool, false>;
        chains(0);
        if (P == 2 && K == 32) {
            store(0, all_codes{});
            __builtin_amdgcn_wave_barrier();
            chains(P - 1);
            rank_codes(0, std::integral_constant<int, 32>{});
            // one MFMA, then a score read and seven ranking instructions
#pragma unroll
            for (int i = 0; i < NTM * MT * NS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
            }
            store(P - 1, all_codes{});
            __builtin_amdgcn_wave_barrier();
            rank_codes(P - 1, std::integral_constant<int, 32>{});
        } else {
            store(0, some_codes{});
#pragma unroll
            for (int p = 1; p < P; ++p) {
                chains(p);
                store(p, some_codes{});
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int p = 0; p < P; ++p) rank_codes(p, std::integral_constant<int, 0>{});
        }
    } else {
    const float *cbg = cb + (size_t)g * PK * DS;
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
        for (int x = 0; x < NPRM; ++x) { tv[p][x] = -INFINITY; tc[p][x] = -1; }
#pragma unroll 2
        for (int c = 0; c < K; ++c) {
            const float *crow = cbg + (p * K + c) * DS;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < DS; ++j) acc = __builtin_fmaf(qr[p * DS + j], crow[j], acc);
            sc_s[(p * K + c) * SROW + lane] = acc;
            top_insert(tv[p], tc[p], acc, c);
        }
    }
    }

    // ---- the n_probes best addresses (keys: sigma, then lower address)
    const int npr = min(s.npr, A);
    float bv[NPRM];
    int ba[NPRM];
    if constexpr (P == 1) {
#pragma unroll
        for (int x = 0; x < NPRM; ++x) { bv[x] = tv[0][x]; ba[x] = tc[0][x]; }
    } else {
#pragma unroll
        for (int x = 0; x < NPRM; ++x) { bv[x] = -INFINITY; ba[x] = 0x7fffffff; }
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
                    const bool sw = (v > bv[z]) | ((v == bv[z]) & (a < ba[z]));
                    const float ov = bv[z];
                    const int oa = ba[z];
                    bv[z] = sw ? v : ov;
                    ba[z] = sw ? a : oa;
                    v = sw ? ov : v;
                    a = sw ? oa : a;
                }
            }
        }
    }
    float tau_v = bv[0];
    int tau_a = ba[0];
#pragma unroll
    for (int x = 1; x < NPRM; ++x)
        if (x == npr - 1) { tau_v = bv[x]; tau_a = ba[x]; }

    // ---- rerank state: RM slots, best first; the first RM-R are sentinels
    u64 rk[RM];
#pragma unroll
    for (int x = 0; x < RM; ++x) rk[x] = x < RM - R ? ~0ull : 0ull;
    const float *kb = kbar + ug * (size_t)NB * D;
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
        insert(rk, key_of(acc, (uint32_t)(0x7FFFFFFF - n)));
    };

    // ---- candidates (pool members) in canonical order: the part-1 walk,
    // then the extension's blocks; the first MAXC are kept in registers and
    // reranked in one batch, the rest (long lists only) afterwards
    constexpr int MAXC = 8;
    int cand[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) cand[i] = -1;
    int nc = 0;
    auto add = [&](int n) {
#pragma unroll
        for (int i = 0; i < MAXC; ++i) cand[i] = i == nc ? n : cand[i];
        ++nc;
    };

    // ---- pool part 1: the eligible prefixes of the n_probes best lists
    auto walk_part1 = [&](auto &&fn) {
#pragma unroll
        for (int x = 0; x < NPRM; ++x) {
            if (x < npr) {
                const int a = ba[x];
                const int e1 = off_s[a + 1];
                for (int e = off_s[a]; e < e1; ++e) {
                    const int n = ent_s[e];
                    if (n > last) break;
                    fn(n);
                }
            }
        }
    };
    int cnt = 0;
    if (live) walk_part1([&](int n) { add(n); ++cnt; });

    sc_s[PK * SROW + lane] = -INFINITY;   // the row past-the-end list entries point at

    // ---- pool part 2: the extension, for lanes whose part 1 holds fewer
    // than R blocks.  The R best addresses holding an eligible block, by
    // (sigma desc, address asc), as 64-bit keys, best first: a scan of the
    // workgroup's address list, then the few addresses whose first block
    // became eligible after the workgroup's first wave (inserted with their
    // full keys).  RM - R sentinel value slots never move.
    const bool need = live && cnt < R;
    u64 top[RM];
#pragma unroll
    for (int x = 0; x < RM; ++x) top[x] = 0ull;
    const char *scl = reinterpret_cast<const char *>(sc_s + lane);
    auto sigma = [&](int2 m) {
        const float a0 = *reinterpret_cast<const float *>(scl + m.x);
        if constexpr (P == 1) return a0;
        const float a1 = *reinterpret_cast<const float *>(scl + m.y);
        return a0 + a1;
    };
    auto addr_key = [&](float sg, int a) { return key_of(sg, (uint32_t)(0x7FFFFFFF - a)); };
    auto key_addr = [](u64 k) { return 0x7FFFFFFF - (int)(k & 0xFFFFFFFFu); };
    if (__ballot(need) != 0ull) {
        const int nal = *nal_s;
        float bs[RM];
#pragma unroll
        for (int x = 0; x < RM; ++x) bs[x] = x < RM - R ? INFINITY : -INFINITY;
        // more slots, first pass: the values only (slot x takes the median of
        // old slots x - 1, x and the new sigma, slot 0 the larger of the two)
        auto visit = [&](float sg) {
#pragma unroll
            for (int x = RM - 1; x > 0; --x) bs[x] = __builtin_amdgcn_fmed3f(bs[x - 1], bs[x], sg);
            bs[0] = __builtin_amdgcn_fmed3f(bs[0], sg, INFINITY);
        };
        // Software pipeline over batches of U list entries: the row offsets
        // are loaded two batches ahead and the score gathers one batch
        // ahead, so the work on a batch overlaps the next batch's LDS reads.
        // The read-ahead stays inside the padded list (-inf rows).
        constexpr int U = SCAN_U;
        auto gather = [&](const int2 (&m)[U], float (&a)[U], float (&c)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                a[u] = *reinterpret_cast<const float *>(scl + m[u].x);
                if constexpr (P == 2) c[u] = *reinterpret_cast<const float *>(scl + m[u].y);
            }
        };
        // Two slots: the scan keeps the two values only (slot 1 takes the
        // median of old slot 0, old slot 1 and the new sigma; slot 0 the
        // larger), plus the batch each slot's address came from: a batch that
        // raises slot 0 gives it its first address of that sigma; slot 1 then
        // holds the batch's runner-up or the old slot 0.  The addresses are
        // recovered afterwards from those two batches.
        float v0 = bs[0], v1 = bs[RM - 1];
        int bb0 = -1, bb1 = -1;
        auto batch_vals = [&](const float (&sg)[U], int batch) {
            float n0 = v0, n1 = v1;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // slot 0 takes the larger value: the median with +inf (one
                // instruction and no compare mask; equal values are equal)
                n1 = __builtin_amdgcn_fmed3f(n0, n1, sg[u]);
                n0 = __builtin_amdgcn_fmed3f(n0, sg[u], INFINITY);
            }
            // both candidates first, then one select: a nested conditional
            // compiles to a branch on the execution mask
            const int up0 = -(int)(n0 > v0);
            const int x1 = n1 > v0 ? batch : bb0, y1 = n1 > v1 ? batch : bb1;
            bb1 = y1 + ((x1 - y1) & up0);
            bb0 = bb0 + ((batch - bb0) & up0);
            v0 = n0;
            v1 = n1;
        };
        // one pass over the list in batches of U: consume(sg, i0) gets the
        // sigmas of entries i0 .. i0 + U - 1 (-inf past the end)
        auto scan = [&](auto &&consume) {
            int n = 0;
            if (U <= nal) {
                int2 m[U];
                float a0[U], c0[U], a1[U], c1[U];
#pragma unroll
                for (int u = 0; u < U; ++u) m[u] = alist[u];
                gather(m, a0, c0);
#pragma unroll
                for (int u = 0; u < U; ++u) m[u] = alist[U + u];
                // two batches per trip, so the buffers alternate without copies
                while (true) {
                    gather(m, a1, c1);                              // batch n + U
#pragma unroll
                    for (int u = 0; u < U; ++u) m[u] = alist[n + 2 * U + u];
                    __builtin_amdgcn_sched_barrier(0);
                    {
                        float sg[U];
#pragma unroll
                        for (int u = 0; u < U; ++u) sg[u] = P == 1 ? a0[u] : a0[u] + c0[u];
                        consume(sg, n);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    n += U;
                    if (n + U > nal) break;
                    gather(m, a0, c0);                              // batch n + U
#pragma unroll
                    for (int u = 0; u < U; ++u) m[u] = alist[n + 2 * U + u];
                    __builtin_amdgcn_sched_barrier(0);
                    {
                        float sg[U];
#pragma unroll
                        for (int u = 0; u < U; ++u) sg[u] = P == 1 ? a1[u] : a1[u] + c1[u];
                        consume(sg, n);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    n += U;
                    if (n + U > nal) break;
                }
            }
            // the partial last batch (its padded read-ahead rows are -inf)
            if (n < nal) {
                float sg[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float v = sigma(alist[n + u]);
                    sg[u] = n + u < nal ? v : -INFINITY;
                }
                consume(sg, n);
            }
        };
        if constexpr (RM == 2) {
            // the list positions of the best and second best entries
            int first = -1, second = -1;
            const u64 needm = __ballot(need);
            const int nneed = __popcll(needm);
            if (PK <= WAVE && nneed <= 6 && nneed * ((nal + WAVE - 1) / WAVE * 12 + 100) < nal * 8) {
                // Few lanes need the extension (long lists late in long
                // sequences): the whole wave scans the list once per such
                // lane.  Lane c holds that query's score of code row c, each
                // lane takes every 64th entry and keeps its two best
                // (sigma, position) keys, and a butterfly of merges gives
                // the wave's two best.  Keys order by sigma, then by lower
                // position, i.e. lower address: the single-lane scan's order.
                // The rule is wave-uniform and picks the cheaper form by its
                // instruction count (about 12 per entry and lane plus 100 per
                // needing lane, against 8 per entry).
                u64 mm = needm;
                while (mm) {
                    const int j = __ffsll((long long)mm) - 1;     // wave-uniform
                    mm &= mm - 1;
                    const float sj = lane < PK ? sc_s[lane * SROW + j] : -INFINITY;
                    u64 k0 = 0ull, k1 = 0ull;
                    constexpr int CU4 = 4;   // entries per lane in flight
                    for (int e0 = 0; e0 < nal; e0 += CU4 * WAVE) {
                        int2 m[CU4];
                        float sg[CU4];
#pragma unroll
                        for (int u = 0; u < CU4; ++u) {
                            const int e = e0 + u * WAVE + lane;
                            m[u] = alist[e < nal ? e : 0];
                        }
#pragma unroll
                        for (int u = 0; u < CU4; ++u) {
                            const float a = __shfl(sj, m[u].x / (SROW * 4));
                            const float c = P == 1 ? 0.0f : __shfl(sj, m[u].y / (SROW * 4));
                            sg[u] = P == 1 ? a : a + c;
                        }
#pragma unroll
                        for (int u = 0; u < CU4; ++u) {
                            const int e = e0 + u * WAVE + lane;
                            const u64 key = e < nal ? key_of(sg[u], (uint32_t)(0x7FFFFFFF - e)) : 0ull;
                            const bool b0 = key > k0;
                            k1 = b0 ? k0 : (key > k1 ? key : k1);
                            k0 = b0 ? key : k0;
                        }
                    }
#pragma unroll
                    for (int off = WAVE / 2; off > 0; off >>= 1) {
                        const u64 p0 = shfl_xor_u64(k0, off), p1 = shfl_xor_u64(k1, off);
                        const u64 hi = k0 > p0 ? k0 : p0, lo = k0 > p0 ? p0 : k0;
                        const u64 m1 = k1 > p1 ? k1 : p1;
                        k1 = lo > m1 ? lo : m1;
                        k0 = hi;
                    }
                    if (lane == j) {
                        first = k0 ? 0x7FFFFFFF - (int)(k0 & 0xFFFFFFFFu) : -1;
                        second = (R == 2 && k1) ? 0x7FFFFFFF - (int)(k1 & 0xFFFFFFFFu) : -1;
                    }
                }
            } else {
                scan([&](const float (&sg)[U], int i0) { batch_vals(sg, i0 / U); });
                // the first entry of a batch whose sigma equals val, other than excl
                auto find = [&](int batch, float val, int excl) {
                    int res = -1;
                    if (batch >= 0) {
#pragma unroll
                        for (int u = U - 1; u >= 0; --u) {
                            const int i = batch * U + u;
                            const bool hit = i < nal && i != excl && sigma(alist[i]) == val;
                            res = hit ? i : res;
                        }
                    }
                    return res;
                };
                const int i0 = RM - R == 0 && v0 > -INFINITY ? find(bb0, v0, -1) : -1;
                const int i1 = v1 > -INFINITY ? find(bb1, v1, i0) : -1;
                // with one slot (R = 1) slot 1 holds the best
                first = RM - R == 0 ? i0 : i1;
                second = RM - R == 0 ? i1 : -1;
            }
            top[0] = first >= 0 ? addr_key(sigma(alist[first]), addr_of(alist[first])) : 0ull;
            top[1] = second >= 0 ? addr_key(sigma(alist[second]), addr_of(alist[second])) : 0ull;
        } else {
            scan([&](const float (&sg)[U], int) {
#pragma unroll
                for (int u = 0; u < U; ++u) visit(sg[u]);
            });
            // The R best are the entries above the R-th value plus the first
            // entries (list order) equal to it, as many as slots hold that
            // value; none if that value is -inf (fewer than R addresses).
            // The second pass shifts their positions into ti.
            const float vR = bs[RM - 1];
            int eq_left = 0;
#pragma unroll
            for (int x = 0; x < RM; ++x) eq_left += (x >= RM - R && bs[x] == vR) ? 1 : 0;
            if (vR == -INFINITY) eq_left = 0;
            int ti[RM];
#pragma unroll
            for (int x = 0; x < RM; ++x) ti[x] = -1;
            scan([&](const float (&sg)[U], int i0) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool eq = (sg[u] == vR) & (eq_left > 0);
                    const bool take = (sg[u] > vR) | eq;
                    eq_left -= eq ? 1 : 0;
#pragma unroll
                    for (int x = RM - 1; x > 0; --x) ti[x] = take ? ti[x - 1] : ti[x];
                    ti[0] = take ? i0 + u : ti[0];
                }
            });
#pragma unroll
            for (int x = 0; x < RM; ++x) {
                if (ti[x] >= 0) {
                    const int2 m = alist[ti[x]];
                    insert(top, addr_key(sigma(m), addr_of(m)));
                }
            }
        }
        // addresses whose first block is eligible for this wave but not for
        // the workgroup's first one (at most the blocks between their last
        // eligible blocks): their full keys go into the list
        for (int n = max(0, last0 + 1); n <= last; ++n) {
            const int a = min(max(ad_g[n], 0), A - 1);    // (clamped: reads stay in bounds)
            if (ent_s[min(off_s[a], NB - 1)] == n) {
                const int2 m = row_offsets(a);
                insert(top, addr_key(sigma(m), a));
            }
        }
    }
    // The addresses up to the one holding the R-th eligible block in walk
    // order (their eligible counts, in key order, reach R there) join the
    // pool; all of the R if their blocks do not reach R (then every address
    // holding an eligible block is among them: the walk probes everything).
    int nadd = 0;
    if (need) {
        int cum = 0;
#pragma unroll
        for (int x = 0; x < RM; ++x) {
            if (x < R && top[x] != 0ull && cum < R) {
                const int a = key_addr(top[x]);
                const int e1 = off_s[a + 1];
                for (int e = off_s[a]; e < e1 && ent_s[e] <= last; ++e) ++cum;
                nadd = x + 1;
            }
        }
    }
    // does (sigma, address) rank after the n_probes-th address?
    auto after_tau = [&](float sg, int a) {
        return (sg < tau_v) | ((sg == tau_v) & (a > tau_a));
    };
    // the extension's pool members: the eligible blocks of those addresses
    // that rank after tau (the others are in part 1)
    auto walk_ext = [&](auto &&fn) {
        if (!need) return;
#pragma unroll
        for (int x = 0; x < RM; ++x) {
            if (x < nadd) {
                const int a = key_addr(top[x]);
                if (after_tau(sigma(row_offsets(a)), a)) {
                    const int e1 = off_s[a + 1];
                    for (int e = off_s[a]; e < e1; ++e) {
                        const int nn = ent_s[e];
                        if (nn > last) break;
                        fn(nn);
                    }
                }
            }
        }
    };
    walk_ext(add);

    // ---- rerank: two candidates at a time, their summaries loaded together
    // (indexes clamped so the loads of empty slots stay in bounds).  A pool
    // of at most R blocks is kept whole whatever its scores, so its lanes
    // skip the summaries and insert their blocks with equal keys (they come
    // out ascending either way).
    const bool rr = nc > R;
#pragma unroll
    for (int i = 0; i < MAXC; i += 2) {
        if (__ballot(i < nc) == 0ull) break;
        const int n0 = cand[i] >= 0 ? cand[i] : 0, n1 = cand[i + 1] >= 0 ? cand[i + 1] : 0;
        float acc0 = 0.0f, acc1 = 0.0f;
        if (rr && i < nc) {
            const float *k0 = kb + (size_t)n0 * D, *k1 = kb + (size_t)n1 * D;
            constexpr int CH = D == 128 ? 8 : D / 4;   // float4 per candidate per round
#pragma unroll
            for (int j0 = 0; j0 < D / 4; j0 += CH) {
                float4 v0[CH], v1[CH];
#pragma unroll
                for (int j = 0; j < CH; ++j) {
                    v0[j] = reinterpret_cast<const float4 *>(k0)[j0 + j];
                    v1[j] = reinterpret_cast<const float4 *>(k1)[j0 + j];
                }
#pragma unroll
                for (int jj = 0; jj < CH; ++jj) {
                    const int j = j0 + jj;
                    acc0 = __builtin_fmaf(qr[4 * j], v0[jj].x, acc0);
                    acc0 = __builtin_fmaf(qr[4 * j + 1], v0[jj].y, acc0);
                    acc0 = __builtin_fmaf(qr[4 * j + 2], v0[jj].z, acc0);
                    acc0 = __builtin_fmaf(qr[4 * j + 3], v0[jj].w, acc0);
                    acc1 = __builtin_fmaf(qr[4 * j], v1[jj].x, acc1);
                    acc1 = __builtin_fmaf(qr[4 * j + 1], v1[jj].y, acc1);
                    acc1 = __builtin_fmaf(qr[4 * j + 2], v1[jj].z, acc1);
                    acc1 = __builtin_fmaf(qr[4 * j + 3], v1[jj].w, acc1);
                }
                // keep the next quarter's loads behind this quarter's chains
                if constexpr (CH < D / 4) __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (i < nc) insert(rk, key_of(acc0, (uint32_t)(0x7FFFFFFF - n0)));
        if (i + 1 < nc) insert(rk, key_of(acc1, (uint32_t)(0x7FFFFFFF - n1)));
    }
    if (__ballot(nc > MAXC) != 0ull) {   // candidates past the register batch
        int k = 0;
        auto late = [&](int n) {
            if (k >= MAXC) rerank(n);
            ++k;
        };
        if (live) walk_part1(late);
        walk_ext(late);
    }

    // ---- emit the kept blocks ascending, -1 padded
    int o[RM];
#pragma unroll
    for (int x = 0; x < RM; ++x)
        o[x] = (x >= RM - R && rk[x] != 0ull) ? 0x7FFFFFFF - (int)(rk[x] & 0xFFFFFFFFu)
                                              : 0x7fffffff;
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

// LDS of one workgroup: per-block score-row offsets, list offsets, list
// entries and one score area per wave.
size_t route_lds(const Shape &s, int waves, bool mf) {
    const int PK = s.P * s.K;
    return (size_t)route_sc_off(s.NB, s.A) * sizeof(int) +
           (size_t)waves * route_wave_floats(PK, s.ds, mf) * sizeof(float);
}

// Waves per workgroup: the count that puts the most waves on a compute unit
// (at most eight, two per SIMD: the register cap), larger workgroups first.
// Each wave's score area is about 17 KiB, so when the lists grow (2048
// addresses or blocks and more) four-wave workgroups no longer fit twice in
// the 160 KiB of LDS, and three-wave ones do.
int route_waves(const Shape &s, bool mf) {
    int best = 1, best_waves = 0;
    for (int w = 4; w >= 1; --w) {
        const size_t lds = route_lds(s, w, mf);
        if (lds > 160 * 1024) continue;
        const int per_cu = std::min(8, (int)((160 * 1024) / lds) * w);
        if (per_cu > best_waves) {
            best = w;
            best_waves = per_cu;
        }
    }
    return best;
}

template <int D, int P, int NPRM, int RM, bool BF16, bool MF>
hipError_t launch_t(const Shape &s, const void *q, const float *cos_t, const float *sin_t,
                    const float *cb, const float *kbar, const int32_t *addr,
                    const int32_t *offsets, const int32_t *entries, int32_t *sel,
                    void *q_rot, hipStream_t st) {
    const int waves = route_waves(s, MF);
    const size_t lds = route_lds(s, waves, MF);
    const dim3 grid((unsigned)((s.T + waves * WAVE - 1) / (waves * WAVE)) * s.Hq * s.B);
    const hipError_t e =
        mono_lds_limit(reinterpret_cast<const void *>(k_route<D, P, NPRM, RM, BF16, MF>), lds);
    if (e != hipSuccess) return e;
    k_route<D, P, NPRM, RM, BF16, MF><<<grid, waves * WAVE, lds, st>>>(
        s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries, sel, q_rot);
    return hipGetLastError();
}

// Matrix-core scoring for d = 64, two components, at most 32 codes each.
template <int D, int P, int NPRM, int RM, bool BF16>
hipError_t launch_m(const Shape &s, const void *q, const float *cos_t, const float *sin_t,
                    const float *cb, const float *kbar, const int32_t *addr,
                    const int32_t *offsets, const int32_t *entries, int32_t *sel, void *q_rot,
                    hipStream_t st) {
    if constexpr (D == 64 && P == 2) {
        if (s.K <= 32 && route_lds(s, 1, true) <= 160 * 1024)
            return launch_t<D, P, NPRM, RM, BF16, true>(s, q, cos_t, sin_t, cb, kbar, addr,
                                                        offsets, entries, sel, q_rot, st);
    }
    return launch_t<D, P, NPRM, RM, BF16, false>(s, q, cos_t, sin_t, cb, kbar, addr, offsets,
                                                 entries, sel, q_rot, st);
}

template <int D, int P, bool BF16>
hipError_t launch_sel(const Shape &s, const void *q, const float *cos_t, const float *sin_t,
                      const float *cb, const float *kbar, const int32_t *addr,
                      const int32_t *offsets, const int32_t *entries, int32_t *sel, void *q_rot,
                      hipStream_t st) {
#define MONO_SEL_ARGS s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries, sel, q_rot, st
    if (s.npr <= 2 && s.R <= 2) return launch_m<D, P, 2, 2, BF16>(MONO_SEL_ARGS);
    if (s.npr <= 4 && s.R <= 2) return launch_m<D, P, 4, 2, BF16>(MONO_SEL_ARGS);
    if (s.npr <= 8 && s.R <= 8) return launch_m<D, P, 8, 8, BF16>(MONO_SEL_ARGS);
    return launch_m<D, P, 16, 16, BF16>(MONO_SEL_ARGS);
#undef MONO_SEL_ARGS
}

}  // namespace

// With q_rot non-null the router also writes every query's rotated row for
// the attention (pre-scaled, activation dtype); a configuration in which
// every query bypasses the search then returns hipErrorInvalidValue (the
// caller rotates separately).
hipError_t launch_route(const Shape &s, const void *q, const float *cos_t, const float *sin_t,
                        const float *cb, const float *kbar, const int32_t *addr,
                        const int32_t *offsets, const int32_t *entries, const int32_t *load,
                        int32_t *sel, hipStream_t st, void *q_rot) {
    (void)load;
    if (s.NB - s.L <= s.R) {  // every query bypasses the search
        if (q_rot) return hipErrorInvalidValue;
        const long routes = (long)s.B * s.Hq * s.T;
        k_route_bypass<<<dim3((unsigned)((routes + 255) / 256)), 256, 0, st>>>(s, sel);
        return hipGetLastError();
    }
    const bool bf = s.dtype == 1;
#define MONO_ROUTE_ARGS s, q, cos_t, sin_t, cb, kbar, addr, offsets, entries, sel, q_rot, st
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
