// Host side of the C ABI declared in include/mono.h: argument validation,
// workspace layout and kernel dispatch.  Every entry point validates on the
// host before enqueueing anything; nothing here allocates, frees or
// synchronizes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "common.hpp"
#include "mono.h"

hipError_t launch_block_address(const Shape &s, const void *k, const float *cos_t,
                                const float *sin_t, const float *cb, float *kbar, int32_t *addr,
                                hipStream_t st, void *k_rot = nullptr);
hipError_t launch_posting_lists(const Shape &s, const int32_t *addr, int32_t *offsets,
                                int32_t *entries, int32_t *load, int32_t *overflow, hipStream_t st);
hipError_t launch_index_stats(const Shape &s, const int32_t *overflow, const int32_t *load,
                              int32_t *stats, hipStream_t st);
hipError_t launch_route(const Shape &s, const void *q, const float *cos_t, const float *sin_t,
                        const float *cb, const float *kbar, const int32_t *addr,
                        const int32_t *offsets, const int32_t *entries, const int32_t *load,
                        int32_t *sel, hipStream_t st, void *q_rot = nullptr);
size_t attention_ws_layout(const Shape &s, size_t *off);
hipError_t launch_attention(const Shape &s, const void *q, const void *k, const void *v,
                            const float *cos_t, const float *sin_t, const int32_t *sel, void *out,
                            void *ws, hipStream_t st, bool prerotated = false);
void attention_rot_slots(const Shape &s, void *ws, void **q_rot, void **k_rot);
hipError_t launch_block_address_range(const Shape &s, int n0, int n1, const void *k,
                                      const float *cos_t, const float *sin_t, const float *cb,
                                      float *kbar, int32_t *addr, hipStream_t st,
                                      void *k_rot = nullptr);
hipError_t launch_posting_lists_prefix(const Shape &s, int nbu, const int32_t *addr,
                                       int32_t *offsets, int32_t *entries, int32_t *load,
                                       int32_t *overflow, hipStream_t st);
hipError_t launch_decode(const Shape &s, int pos, const void *q, const void *kc, const void *vc,
                         const void *krot, const float *cos_t, const float *sin_t, const float *cb,
                         const float *kbar, const int32_t *offsets, const int32_t *entries,
                         int32_t *sel, void *out, hipStream_t st);
size_t dense_ws_layout(const Shape &s, size_t *off);
size_t calibrate_ws_bytes(const Shape &s);
hipError_t launch_calibrate(const Shape &s, int n_iter, const float *kbar, float *codebooks,
                            void *ws, hipStream_t st);
hipError_t launch_dense(const Shape &s, const void *q, const void *k, const void *v,
                        const float *cos_t, const float *sin_t, void *out, void *ws,
                        hipStream_t st);
hipError_t launch_gemm(int bf16, int M, int N, int Kd, const void *A, const void *Bm, void *C,
                       hipStream_t st);
hipError_t launch_gemm_qkv(int bf16, int M, int N, int Kd, const void *A, const void *Bm, void *q,
                           void *k, void *v, int nq, int nk, hipStream_t st);

namespace {
// Static scratch of mono_routed_attention_noalloc.  Host code never passes
// this name to a kernel (on the host it is a stand-in, not a device
// address): the device address comes from hipGetSymbolAddress, once per
// device, and is kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[MONO_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array (set up on the
// first call on that device, with that device current).
hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

std::mutex g_cache_mutex;
std::map<std::pair<const void *, int>, size_t> g_lds_set;                  // (kernel, device)
std::map<std::tuple<const void *, int, int, size_t>, long> g_resident;    // (.., threads, lds)
}  // namespace

hipError_t mono_lds_limit(const void *fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    size_t &have = g_lds_set[{fn, dev}];
    if (have >= bytes) return hipSuccess;
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) have = bytes;
    return e;
}

long mono_resident_workgroups(const void *fn, int threads, size_t lds) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    const auto key = std::make_tuple(fn, dev, threads, lds);
    const auto it = g_resident.find(key);
    if (it != g_resident.end()) return it->second;
    int cus = 256, per_cu = 1;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const long g = (long)cus * per_cu;
    g_resident[key] = g;
    return g;
}

namespace {

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

mono_status make_shape(const mono_config *c, bool mixer, Shape &s) {
    if (!c) return MONO_ERR_NULL;
    const int32_t pos[] = {c->batch, c->seq_len, c->n_q_heads, c->n_kv_heads, c->head_dim,
                           c->block_size, c->n_components, c->codes_per_component, c->capacity,
                           c->n_probes, c->n_remote, c->n_local};
    for (int32_t x : pos)
        if (x < 1) return MONO_ERR_SHAPE;
    if (mixer && c->width < 1) return MONO_ERR_SHAPE;
    if (c->seq_len % c->block_size) return MONO_ERR_SHAPE;
    if (c->head_dim % c->n_components) return MONO_ERR_SHAPE;
    if (c->n_q_heads % c->n_kv_heads) return MONO_ERR_SHAPE;
    if (mixer && c->n_q_heads * c->head_dim != c->width) return MONO_ERR_SHAPE;
    if (c->dtype != MONO_F32 && c->dtype != MONO_BF16) return MONO_ERR_UNSUPPORTED;
    if (c->head_dim != 64 && c->head_dim != 128) return MONO_ERR_UNSUPPORTED;
    if (c->block_size != 64 && c->block_size != 128) return MONO_ERR_UNSUPPORTED;
    if (c->n_components != 1 && c->n_components != 2) return MONO_ERR_UNSUPPORTED;
    if (c->codes_per_component < 2 || c->codes_per_component > 64) return MONO_ERR_UNSUPPORTED;
    if (c->n_probes > 16) return MONO_ERR_UNSUPPORTED;
    const int NB = c->seq_len / c->block_size;
    if (NB > 8192) return MONO_ERR_UNSUPPORTED;
    if ((long)c->n_kv_heads * c->head_dim > 4096) return MONO_ERR_UNSUPPORTED;
    if (c->n_remote > 16 && NB - c->n_local > c->n_remote) return MONO_ERR_UNSUPPORTED;
    const double routes = (double)c->batch * c->n_q_heads * c->seq_len;
    if (routes * c->n_remote >= 2147483647.0) return MONO_ERR_UNSUPPORTED;
    if (mixer && c->width % 8) return MONO_ERR_UNSUPPORTED;
    s.B = c->batch;
    s.T = c->seq_len;
    s.W = c->width;
    s.Hq = c->n_q_heads;
    s.Hkv = c->n_kv_heads;
    s.d = c->head_dim;
    s.beta = c->block_size;
    s.P = c->n_components;
    s.K = c->codes_per_component;
    s.cap = c->capacity;
    s.npr = c->n_probes;
    s.R = c->n_remote;
    s.L = c->n_local;
    s.dtype = c->dtype;
    s.NB = NB;
    s.A = 1;
    for (int p = 0; p < s.P; ++p) s.A *= s.K;
    s.G = s.Hq / s.Hkv;
    s.ds = s.d / s.P;
    return MONO_OK;
}

size_t esize(const Shape &s) { return s.dtype == MONO_BF16 ? 2 : 4; }

// Mixer workspace: q, k, v, kbar, addr, offsets, entries, load, overflow,
// sel, attention output, inner workspace.
size_t mixer_layout(const Shape &s, size_t *off) {
    const size_t es = esize(s);
    const size_t BT = (size_t)s.B * s.T;
    const size_t BG = (size_t)s.B * s.Hkv;
    size_t p = 0;
    off[0] = p; p = al256(p + BT * s.Hq * s.d * es);
    off[1] = p; p = al256(p + BT * s.Hkv * s.d * es);
    off[2] = p; p = al256(p + BT * s.Hkv * s.d * es);
    off[3] = p; p = al256(p + BG * s.NB * s.d * 4);
    off[4] = p; p = al256(p + BG * s.NB * 4);
    off[5] = p; p = al256(p + BG * (s.A + 1) * 4);
    off[6] = p; p = al256(p + BG * s.NB * 4);
    off[7] = p; p = al256(p + BG * s.A * 4);
    off[8] = p; p = al256(p + BG * 4);
    off[9] = p; p = al256(p + BT * s.Hq * s.R * 4);
    off[10] = p; p = al256(p + BT * s.Hq * s.d * es);
    off[11] = p;
    size_t aoff[14];
    p += attention_ws_layout(s, aoff);
    return p;
}

mono_status hip_status(hipError_t e) { return e == hipSuccess ? MONO_OK : MONO_ERR_HIP; }

bool index_ok(const mono_index *x) {
    return x && x->kbar && x->addr && x->offsets && x->entries && x->load && x->overflow;
}

}  // namespace

extern "C" {

size_t mono_workspace_bytes(const mono_config *cfg, int which) {
    Shape s;
    const bool mixer = which == MONO_WS_MIXER;
    if (make_shape(cfg, mixer, s) != MONO_OK) return 0;
    size_t off[14];
    switch (which) {
        case MONO_WS_BUILD:
        case MONO_WS_ROUTE:
            return 0;
        case MONO_WS_ATTENTION:
            return attention_ws_layout(s, off);
        case MONO_WS_MIXER:
            return mixer_layout(s, off);
        case MONO_WS_DENSE:
            return dense_ws_layout(s, off);
        case MONO_WS_CALIBRATE:
            return calibrate_ws_bytes(s);
        default:
            return 0;
    }
}

mono_status mono_rope_table(int32_t seq_len, int32_t head_dim, double base, float *cos_tab,
                            float *sin_tab) {
    if (!cos_tab || !sin_tab) return MONO_ERR_NULL;
    if (seq_len < 1 || head_dim < 2 || head_dim % 2 || !(base > 0.0)) return MONO_ERR_SHAPE;
    const int h = head_dim / 2;
    for (int i = 0; i < h; ++i) {
        const double inv_freq = std::pow(base, -(2.0 * (double)i) / (double)head_dim);
        for (int t = 0; t < seq_len; ++t) {
            const double ang = (double)t * inv_freq;
            cos_tab[(size_t)t * h + i] = (float)std::cos(ang);
            sin_tab[(size_t)t * h + i] = (float)std::sin(ang);
        }
    }
    return MONO_OK;
}

mono_status mono_build_index(const mono_config *cfg, const void *k, const float *rope_cos,
                             const float *rope_sin, const float *codebooks, const mono_index *out,
                             void *ws, size_t ws_bytes, void *stream) {
    (void)ws;
    (void)ws_bytes;
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!k || !rope_cos || !rope_sin || !codebooks || !index_ok(out)) return MONO_ERR_NULL;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = launch_block_address(s, k, rope_cos, rope_sin, codebooks, out->kbar, out->addr, hs,
                                        out->k_rot);
    if (e != hipSuccess) return MONO_ERR_HIP;
    e = launch_posting_lists(s, out->addr, out->offsets, out->entries, out->load, out->overflow, hs);
    return hip_status(e);
}

mono_status mono_route(const mono_config *cfg, const void *q, const float *rope_cos,
                       const float *rope_sin, const float *codebooks, const mono_index *idx,
                       int32_t *sel, void *ws, size_t ws_bytes, void *stream) {
    (void)ws;
    (void)ws_bytes;
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!q || !rope_cos || !rope_sin || !codebooks || !index_ok(idx) || !sel) return MONO_ERR_NULL;
    return hip_status(launch_route(s, q, rope_cos, rope_sin, codebooks, idx->kbar, idx->addr,
                                   idx->offsets, idx->entries, idx->load, sel,
                                   reinterpret_cast<hipStream_t>(stream)));
}

mono_status mono_selected_attention(const mono_config *cfg, const void *q, const void *k,
                                    const void *v, const float *rope_cos, const float *rope_sin,
                                    const int32_t *sel, void *out, void *ws, size_t ws_bytes,
                                    void *stream) {
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!q || !k || !v || !rope_cos || !rope_sin || !sel || !out || !ws) return MONO_ERR_NULL;
    size_t off[14];
    if (ws_bytes < attention_ws_layout(s, off)) return MONO_ERR_WORKSPACE;
    return hip_status(launch_attention(s, q, k, v, rope_cos, rope_sin, sel, out, ws,
                                       reinterpret_cast<hipStream_t>(stream)));
}

mono_status mono_routed_attention(const mono_config *cfg, const void *q, const void *k,
                                  const void *v, const float *rope_cos, const float *rope_sin,
                                  const float *codebooks, const mono_index *idx, int32_t *sel,
                                  void *out, void *ws, size_t ws_bytes, void *const *stage_events,
                                  void *stream) {
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!q || !k || !v || !rope_cos || !rope_sin || !codebooks || !index_ok(idx) || !sel || !out ||
        !ws)
        return MONO_ERR_NULL;
    size_t off[14];
    if (ws_bytes < attention_ws_layout(s, off)) return MONO_ERR_WORKSPACE;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
        return stage_events && stage_events[i]
                   ? hipEventRecord(reinterpret_cast<hipEvent_t>(stage_events[i]), hs)
                   : hipSuccess;
    };
    // every query bypassing the search: the router writes no rotated rows,
    // the attention rotates them itself
    const bool fused = s.NB - s.L > s.R;
    void *q_rot = nullptr, *k_rot = nullptr;
    if (fused) attention_rot_slots(s, ws, &q_rot, &k_rot);
    if (mark(0) != hipSuccess) return MONO_ERR_HIP;
    if (launch_block_address(s, k, rope_cos, rope_sin, codebooks, idx->kbar, idx->addr, hs,
                             k_rot) != hipSuccess ||
        launch_posting_lists(s, idx->addr, idx->offsets, idx->entries, idx->load, idx->overflow,
                             hs) != hipSuccess ||
        mark(1) != hipSuccess)
        return MONO_ERR_HIP;
    if (launch_route(s, q, rope_cos, rope_sin, codebooks, idx->kbar, idx->addr, idx->offsets,
                     idx->entries, idx->load, sel, hs, q_rot) != hipSuccess ||
        mark(2) != hipSuccess)
        return MONO_ERR_HIP;
    if (launch_attention(s, q, k, v, rope_cos, rope_sin, sel, out, ws, hs, fused) != hipSuccess ||
        mark(3) != hipSuccess)
        return MONO_ERR_HIP;
    return MONO_OK;
}

mono_status mono_routed_attention_noalloc(const mono_config *cfg, const void *q, const void *k,
                                          const void *v, const float *rope_cos,
                                          const float *rope_sin, const float *codebooks,
                                          const mono_index *idx, int32_t *sel, void *out,
                                          void *const *stage_events, void *stream) {
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!q || !k || !v || !rope_cos || !rope_sin || !codebooks || !index_ok(idx) || !sel || !out)
        return MONO_ERR_NULL;
    size_t off[14];
    const size_t need = attention_ws_layout(s, off);
    if (need > MONO_NOALLOC_SCRATCH_BYTES) return MONO_ERR_SCRATCH;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return MONO_ERR_HIP;
    return mono_routed_attention(cfg, q, k, v, rope_cos, rope_sin, codebooks, idx, sel, out, ws,
                                 need, stage_events, stream);
}

mono_status mono_dense_attention(const mono_config *cfg, const void *q, const void *k,
                                 const void *v, const float *rope_cos, const float *rope_sin,
                                 void *out, void *ws, size_t ws_bytes, void *stream) {
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!q || !k || !v || !rope_cos || !rope_sin || !out || !ws) return MONO_ERR_NULL;
    size_t off[2];
    if (ws_bytes < dense_ws_layout(s, off)) return MONO_ERR_WORKSPACE;
    return hip_status(launch_dense(s, q, k, v, rope_cos, rope_sin, out, ws,
                                   reinterpret_cast<hipStream_t>(stream)));
}

mono_status mono_calibrate_codebooks(const mono_config *cfg, const float *kbar, float *codebooks,
                                     int32_t n_iter, void *ws, size_t ws_bytes, void *stream) {
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!kbar || !codebooks || !ws) return MONO_ERR_NULL;
    if (n_iter < 0 || n_iter > 10000) return MONO_ERR_SHAPE;
    if (ws_bytes < calibrate_ws_bytes(s)) return MONO_ERR_WORKSPACE;
    return hip_status(launch_calibrate(s, n_iter, kbar, codebooks, ws,
                                       reinterpret_cast<hipStream_t>(stream)));
}

mono_status mono_decode_index(const mono_config *cfg, const void *k_cache, const float *rope_cos,
                              const float *rope_sin, const float *codebooks, const mono_index *idx,
                              int32_t n_indexed, int32_t n_tokens, void *stream) {
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!k_cache || !rope_cos || !rope_sin || !codebooks || !index_ok(idx)) return MONO_ERR_NULL;
    if (n_tokens < 0 || n_tokens > s.T) return MONO_ERR_SHAPE;
    const int nb = n_tokens / s.beta;
    if (n_indexed < 0 || n_indexed > nb) return MONO_ERR_SHAPE;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (launch_block_address_range(s, n_indexed, nb, k_cache, rope_cos, rope_sin, codebooks,
                                   idx->kbar, idx->addr, hs, idx->k_rot) != hipSuccess)
        return MONO_ERR_HIP;
    return hip_status(launch_posting_lists_prefix(s, nb, idx->addr, idx->offsets, idx->entries,
                                                  idx->load, idx->overflow, hs));
}

mono_status mono_decode_step(const mono_config *cfg, const void *q, const void *k_cache,
                             const void *v_cache, const float *rope_cos, const float *rope_sin,
                             const float *codebooks, const mono_index *idx, int32_t pos,
                             int32_t *sel, void *out, void *stream) {
    Shape s;
    const mono_status st = make_shape(cfg, false, s);
    if (st != MONO_OK) return st;
    if (!q || !k_cache || !v_cache || !rope_cos || !rope_sin || !codebooks || !index_ok(idx) ||
        !sel || !out)
        return MONO_ERR_NULL;
    if (pos < 0 || pos >= s.T) return MONO_ERR_SHAPE;
    return hip_status(launch_decode(s, pos, q, k_cache, v_cache, idx->k_rot, rope_cos, rope_sin,
                                    codebooks, idx->kbar, idx->offsets, idx->entries, sel, out,
                                    reinterpret_cast<hipStream_t>(stream)));
}

mono_status mono_mixer_layout(const mono_config *cfg, size_t *offsets_out) {
    if (!offsets_out) return MONO_ERR_NULL;
    Shape s;
    const mono_status st = make_shape(cfg, true, s);
    if (st != MONO_OK) return st;
    mixer_layout(s, offsets_out);
    return MONO_OK;
}

mono_status mono_mixer_forward(const mono_config *cfg, const void *x, const void *w_qkv,
                               const void *w_o, const float *codebooks, const float *rope_cos,
                               const float *rope_sin, void *delta, int32_t *stats, void *ws,
                               size_t ws_bytes, void *stream) {
    Shape s;
    const mono_status st = make_shape(cfg, true, s);
    if (st != MONO_OK) return st;
    if (!x || !w_qkv || !w_o || !codebooks || !rope_cos || !rope_sin || !delta || !ws)
        return MONO_ERR_NULL;
    size_t off[12];
    if (ws_bytes < mixer_layout(s, off)) return MONO_ERR_WORKSPACE;
    unsigned char *base = reinterpret_cast<unsigned char *>(ws);
    void *q = base + off[0], *k = base + off[1], *v = base + off[2];
    mono_index idx;
    idx.kbar = reinterpret_cast<float *>(base + off[3]);
    idx.addr = reinterpret_cast<int32_t *>(base + off[4]);
    idx.offsets = reinterpret_cast<int32_t *>(base + off[5]);
    idx.entries = reinterpret_cast<int32_t *>(base + off[6]);
    idx.load = reinterpret_cast<int32_t *>(base + off[7]);
    idx.overflow = reinterpret_cast<int32_t *>(base + off[8]);
    idx.k_rot = nullptr;
    int32_t *sel = reinterpret_cast<int32_t *>(base + off[9]);
    void *attn = base + off[10];
    void *inner = base + off[11];
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const int bf = s.dtype == MONO_BF16;
    const int M = s.B * s.T;
    const int nq = s.Hq * s.d, nk = s.Hkv * s.d;
    if (launch_gemm_qkv(bf, M, nq + 2 * nk, s.W, x, w_qkv, q, k, v, nq, nk, hs) != hipSuccess)
        return MONO_ERR_HIP;
    // the index build and the router also write the attention's rotated rows
    // (unless every query bypasses the search)
    const bool fused = s.NB - s.L > s.R;
    void *q_rot = nullptr, *k_rot = nullptr;
    if (fused) attention_rot_slots(s, inner, &q_rot, &k_rot);
    if (launch_block_address(s, k, rope_cos, rope_sin, codebooks, idx.kbar, idx.addr, hs, k_rot) !=
        hipSuccess)
        return MONO_ERR_HIP;
    if (launch_posting_lists(s, idx.addr, idx.offsets, idx.entries, idx.load, idx.overflow, hs) !=
        hipSuccess)
        return MONO_ERR_HIP;
    if (stats && launch_index_stats(s, idx.overflow, idx.load, stats, hs) != hipSuccess)
        return MONO_ERR_HIP;
    if (launch_route(s, q, rope_cos, rope_sin, codebooks, idx.kbar, idx.addr, idx.offsets,
                     idx.entries, idx.load, sel, hs, q_rot) != hipSuccess)
        return MONO_ERR_HIP;
    if (launch_attention(s, q, k, v, rope_cos, rope_sin, sel, attn, inner, hs, fused) !=
        hipSuccess)
        return MONO_ERR_HIP;
    return hip_status(launch_gemm(bf, M, s.W, nq, attn, w_o, delta, hs));
}

const char *mono_status_string(mono_status status) {
    switch (status) {
        case MONO_OK: return "ok";
        case MONO_ERR_NULL: return "a required pointer is NULL";
        case MONO_ERR_SHAPE: return "inconsistent sizes";
        case MONO_ERR_UNSUPPORTED: return "shape or dtype outside the supported set";
        case MONO_ERR_WORKSPACE: return "workspace too small";
        case MONO_ERR_HIP: return "a HIP launch failed";
        case MONO_ERR_SCRATCH:
            return "the call needs more scratch than the static area holds "
                   "(MONO_NOALLOC_SCRATCH_BYTES); use the workspace entry point";
    }
    return "unknown status";
}

}  // extern "C"
