/*
 * mono.h -- C ABI of the MI355X (gfx950) routed sparse causal attention path.
 *
 * The operation is the Monodratic mixer's hot path as the pages state it:
 * "Monodratic: a reproducible sparse attention mixer" (technical report page,
 * sections "Mixer" with Figure 1, "Learned sparse route", "Capacity",
 * "Finite-range scaling") and "Monodratic Claims Learned Routing Can Make
 * Sparse Causal Attention More Selective" (news page, section "Monodratic
 * Turns Sparse Attention Into a Retrieval Decision").  After rotary position
 * embedding, each source block of keys gets a product address; addresses
 * feed capacity-bounded causal posting lists; each query probes addresses,
 * reranks the candidate blocks and keeps a fixed number of remote blocks;
 * local blocks are added; attention over the chosen tokens is exact causal
 * softmax.  The mixer is stateless: normalized stream [B,T,W] in, attention
 * delta [B,T,W] out.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers to caller-owned memory, row-major,
 *    densely packed, with the layouts written at each argument.  The library
 *    never allocates, frees or synchronizes; it enqueues kernels on `stream`
 *    (a hipStream_t; NULL = the null stream) and returns.
 *  - Activations (q, k, v, x, weights, attention output, delta) use
 *    cfg->dtype: MONO_F32 = IEEE float, MONO_BF16 = bfloat16.  Codebooks,
 *    rotary tables and block summaries are always float.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is enqueued and no output is touched.
 *  - Workspace: `ws` must point to at least mono_workspace_bytes(cfg, which)
 *    bytes of device memory, 256-byte aligned; its contents on entry do not
 *    matter and are garbage on return.  A workspace may be reused by calls
 *    that are ordered on one stream; calls that overlap must not share one.
 *  - Calls are deterministic: the same inputs give bitwise identical outputs.
 *
 * Supported shapes (MONO_ERR_UNSUPPORTED otherwise): head_dim 64 or 128;
 * block_size 64 or 128; n_components 1 or 2; codes_per_component 2..64 (so
 * at most 4096 addresses); 1 <= n_probes <= 16; n_remote <= 16 unless every
 * query bypasses the search (n_remote >= seq_len/block_size - n_local);
 * seq_len/block_size <= 8192; n_kv_heads * head_dim <= 4096.
 */
#ifndef MONO_H
#define MONO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MONO_OK = 0,
    MONO_ERR_NULL = 1,        /* a required pointer is NULL */
    MONO_ERR_SHAPE = 2,       /* sizes inconsistent: seq_len % block_size, head_dim %
                                 n_components, n_q_heads % n_kv_heads, a non-positive
                                 size, or n_q_heads*head_dim != width (mixer) */
    MONO_ERR_UNSUPPORTED = 3, /* consistent but outside the supported shapes above */
    MONO_ERR_WORKSPACE = 4,   /* ws_bytes smaller than mono_workspace_bytes() */
    MONO_ERR_HIP = 5,         /* a HIP launch failed */
    MONO_ERR_SCRATCH = 6      /* mono_routed_attention_noalloc: the call needs more than
                                 MONO_NOALLOC_SCRATCH_BYTES of scratch */
} mono_status;

typedef enum { MONO_F32 = 0, MONO_BF16 = 1 } mono_dtype;

/* Sizes of one call.  NB = seq_len / block_size source blocks per sequence;
 * A = codes_per_component ^ n_components addresses. */
typedef struct {
    int32_t batch;                /* B */
    int32_t seq_len;              /* T, positions 0..T-1 in every sequence */
    int32_t width;                /* W (mixer only) */
    int32_t n_q_heads;            /* Hq */
    int32_t n_kv_heads;           /* Hkv; q-head h reads kv-head h / (Hq/Hkv) */
    int32_t head_dim;             /* d */
    int32_t block_size;           /* beta */
    int32_t n_components;         /* P: product code components */
    int32_t codes_per_component;  /* K */
    int32_t capacity;             /* blocks kept per posting list, >= 1 */
    int32_t n_probes;             /* addresses a query probes at least */
    int32_t n_remote;             /* R: remote blocks selected per query */
    int32_t n_local;              /* L >= 1: local blocks, the query's own included */
    int32_t dtype;                /* mono_dtype of the activations */
} mono_config;

/* The index of one call (all device pointers, caller-owned).
 *   kbar     [B][Hkv][NB][d] float  block summaries: mean of the block's rotated keys
 *   addr     [B][Hkv][NB]    int32  product address of each block, in [0, A)
 *   offsets  [B][Hkv][A+1]   int32  list a of (b, g) is entries[offsets[a] .. offsets[a+1])
 *   entries  [B][Hkv][NB]    int32  ascending source blocks per list; -1 past offsets[A]
 *   load     [B][Hkv][A]     int32  blocks assigned per address before the capacity clamp
 *   overflow [B][Hkv]        int32  blocks dropped by the clamp
 *   k_rot    [B][T][Hkv][d]  dtype  optional (NULL: absent): the rotated keys of the
 *            indexed blocks, rounded to the activation dtype.  mono_build_index and
 *            mono_decode_index write the rows of the blocks they index when it is
 *            present; mono_decode_step then reads the selected blocks' keys from it
 *            instead of rotating the cache's, so it must have been present whenever
 *            the covered blocks were indexed. */
typedef struct {
    float *kbar;
    int32_t *addr;
    int32_t *offsets;
    int32_t *entries;
    int32_t *load;
    int32_t *overflow;
    void *k_rot;
} mono_index;

/* Which call a workspace is for. */
enum {
    MONO_WS_BUILD = 0,
    MONO_WS_ROUTE = 1,
    MONO_WS_ATTENTION = 2,
    MONO_WS_MIXER = 3,
    MONO_WS_DENSE = 4,
    MONO_WS_CALIBRATE = 5
};

/* Bytes of workspace the call `which` needs for `cfg` (0 if it needs none or
 * if cfg is invalid; MONO_WS_MIXER includes q, k, v, the index, the selection
 * and the attention output of the mixer). */
size_t mono_workspace_bytes(const mono_config *cfg, int which);

/* Host function: fill host arrays cos_tab/sin_tab [T][d/2] with the rotary
 * table, angle = t * base^(-2i/d) evaluated in double, each value rounded
 * once to float.  Dimension i is rotated together with i + d/2 (rotate-half
 * pairing).  Technical report page, section "Mixer": routing and attention
 * act on rotary-embedded queries and keys.  Returns MONO_ERR_NULL /
 * MONO_ERR_SHAPE (T < 1, d odd) or MONO_OK. */
mono_status mono_rope_table(int32_t seq_len, int32_t head_dim, double base, float *cos_tab,
                            float *sin_tab);

/* Index build (news page, "Retrieval Decision": after RoPE, source blocks get
 * product addresses combining several code components; addresses point at
 * bounded posting lists.  Report page, "Mixer": keys are written into bounded
 * causal posting lists; "Capacity": overflow is counted; "Finite-range
 * scaling": the build is a stable sort).
 *   k         [B][T][Hkv][d] dtype   un-rotated keys
 *   rope_cos, rope_sin [T][d/2] float  table from mono_rope_table
 *   codebooks [Hkv][P][K][d/P] float component p scores code c by the inner
 *             product with dimensions [p*d/P, (p+1)*d/P) of the block summary
 *   out       index arrays to fill (see mono_index)
 * Per block: summary = fp32 mean of the rotated keys (summed in token order);
 * code c_p = argmax (lowest code on ties) of the fp32 inner products (fused
 * multiply-adds in dimension order); address = sum_p c_p * K^(P-1-p).  Per
 * (batch, kv-head): a stable counting sort of blocks by address; each list
 * keeps its first `capacity` blocks in source order.  Overflow is not an
 * error.  Workspace: MONO_WS_BUILD. */
mono_status mono_build_index(const mono_config *cfg, const void *k, const float *rope_cos,
                             const float *rope_sin, const float *codebooks, const mono_index *out,
                             void *ws, size_t ws_bytes, void *stream);

/* Routing (news page, "Retrieval Decision": a query probes addresses, gets
 * candidates, reranks them and keeps a fixed number of remote blocks; no
 * source block is available to an earlier query; local blocks are separate.
 * Report page, "Learned sparse route": the latest of six blocks sees five
 * eligible remote blocks with one local block).
 *   q    [B][T][Hq][d] dtype   un-rotated queries
 *   idx  the index built by mono_build_index from the same call's keys
 *   sel  [B][Hq][T][R] int32   output: selected remote blocks, ascending, -1 padded
 * Query t is in block qb = t / beta; its eligible remote blocks are
 * 0 .. qb - L (E of them).  If E <= R the search is bypassed and the
 * selection is 0 .. E-1.  Otherwise every address is ranked by the fp32 sum
 * of its component scores (descending; lower address first on ties) and
 * lists are probed in that order, collecting indexed eligible blocks, until
 * at least n_probes addresses were probed and at least R blocks collected;
 * the candidates are reranked by the fp32 inner product of the rotated query
 * with the block summary and the R best (lower block first on ties) are
 * kept.  Workspace: none (MONO_WS_ROUTE returns 0); ws may be NULL. */
mono_status mono_route(const mono_config *cfg, const void *q, const float *rope_cos,
                       const float *rope_sin, const float *codebooks, const mono_index *idx,
                       int32_t *sel, void *ws, size_t ws_bytes, void *stream);

/* Selected-set attention (report page, "Mixer": local blocks are added
 * separately; attention over the selected set is ordinary causal softmax and
 * no value summary replaces selected values.  News page, "Retrieval
 * Decision": exact attention within the selected set under a causal mask).
 *   q   [B][T][Hq][d], k, v [B][T][Hkv][d]  dtype, un-rotated q and k
 *   sel [B][Hq][T][R] int32 remote blocks per query (ascending or not, -1 =
 *       empty; every id must satisfy 0 <= id <= qb - L; checked on device:
 *       invalid ids are ignored)
 *   out [B][T][Hq][d] dtype attention output
 * Query t attends to every token s <= t in its selected blocks and in blocks
 * qb-L+1 .. qb, with logits <rot(q_t), rot(k_s)> / sqrt(d) and fp32 softmax.
 * Workspace: MONO_WS_ATTENTION. */
mono_status mono_selected_attention(const mono_config *cfg, const void *q, const void *k,
                                    const void *v, const float *rope_cos, const float *rope_sin,
                                    const int32_t *sel, void *out, void *ws, size_t ws_bytes,
                                    void *stream);

/* The whole routed step in one call: mono_build_index, mono_route and
 * mono_selected_attention on the same inputs, with identical results.  The
 * index build and the router also write the rotated key and query rows the
 * attention needs (they compute them anyway), so the attention's own
 * rotation pass is skipped.
 *   q, k, v, rope_cos, rope_sin, codebooks  as for the three calls
 *   idx      index arrays, filled as by mono_build_index
 *   sel      [B][Hq][T][R] int32  output, as from mono_route
 *   out      [B][T][Hq][d] dtype  output, as from mono_selected_attention
 *   stage_events  NULL, or 4 hipEvent_t slots (created by the caller; a NULL
 *            slot is skipped) recorded on `stream` before the index build,
 *            after it, after the route and after the attention (stage timing
 *            without extra launches; every timed event costs the queue a few
 *            microseconds)
 * Workspace: MONO_WS_ATTENTION. */
mono_status mono_routed_attention(const mono_config *cfg, const void *q, const void *k,
                                  const void *v, const float *rope_cos, const float *rope_sin,
                                  const float *codebooks, const mono_index *idx, int32_t *sel,
                                  void *out, void *ws, size_t ws_bytes, void *const *stage_events,
                                  void *stream);

/* Bytes of the library's static scratch area (per GPU) that
 * mono_routed_attention_noalloc uses in place of a workspace: 128 MiB. */
#define MONO_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* mono_routed_attention without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments (minus ws and
 * ws_bytes), same results, same kernels.  The scratch it needs lives in a
 * static device array of MONO_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends; the call allocates and
 * frees nothing.  Configurations whose MONO_WS_ATTENTION workspace exceeds
 * that size return MONO_ERR_SCRATCH with nothing enqueued.  `stream` must
 * belong to the current device.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other host threads)
 * race and must be ordered by the caller.  The array keeps the last call's
 * contents; nothing in the step depends on its contents on entry. */
mono_status mono_routed_attention_noalloc(const mono_config *cfg, const void *q, const void *k,
                                          const void *v, const float *rope_cos,
                                          const float *rope_sin, const float *codebooks,
                                          const mono_index *idx, int32_t *sel, void *out,
                                          void *const *stage_events, void *stream);

/* Dense causal attention, the baseline the routed path is measured against
 * (news page, section "The 99.35 Percent Result Does Not Establish Language
 * Quality": a comparison with optimized FlashAttention-style dense kernels is
 * necessary; section "What Sparse-Attention Researchers Should Watch Next":
 * the GPU benchmark must count routing and index costs).
 *   q   [B][T][Hq][d], k, v [B][T][Hkv][d]  dtype, un-rotated q and k
 *   out [B][T][Hq][d] dtype
 * Query t attends to every token s <= t with logits <rot(q_t), rot(k_s)> /
 * sqrt(d) and fp32 softmax: the result of mono_selected_attention when every
 * query selects all of its eligible blocks.  Only batch, seq_len, head
 * counts, head_dim and dtype are used; the other fields of cfg are validated
 * as for every call, so the routed path's config can be passed unchanged.
 * Workspace: MONO_WS_DENSE (the rotated q and k). */
mono_status mono_dense_attention(const mono_config *cfg, const void *q, const void *k,
                                 const void *v, const float *rope_cos, const float *rope_sin,
                                 void *out, void *ws, size_t ws_bytes, void *stream);

/* Spherical codebook calibration (report page, section "Capacity" and
 * Figure 3: calibrating the codebooks spherically on a training split
 * removes held-out list overflow and lowers the largest load).
 *   kbar       [B][Hkv][NB][d] float  block summaries of the training split
 *              (mono_build_index of the training sequences; B sequences of
 *              T = cfg->seq_len tokens)
 *   codebooks  [Hkv][P][K][d/P] float  in: initial codes; out: calibrated
 *   n_iter     rounds, 0 .. 10000 (0 leaves the codes unchanged)
 * For every kv-head and component: spherical k-means over the summaries'
 * component sub-vectors.  Each round assigns every point to the code of
 * largest inner product (fp32 fused multiply-add chain in dimension order,
 * lowest code on ties: the address decision) and replaces every code that
 * has members by the fp32 sum of its members in point order (batch-major,
 * then block) divided by the correctly rounded square root of that sum's
 * fused-multiply-add square; a code without members is kept.  Deterministic
 * and bit-identical to that sequential evaluation.  MONO_ERR_SHAPE if n_iter
 * is out of range.  Workspace: MONO_WS_CALIBRATE. */
mono_status mono_calibrate_codebooks(const mono_config *cfg, const float *kbar, float *codebooks,
                                     int32_t n_iter, void *ws, size_t ws_bytes, void *stream);

/* Incremental index for decoding (news page, section "Learned Routing Faces
 * Dense Attention's Reliability Advantage": a deployed decoder updates its
 * routing structures as new tokens arrive; section "The 99.35 Percent Result
 * Does Not Establish Language Quality": decoding brings frequent incremental
 * updates.  Report page, section "Limits": the key/value cache is outside
 * the mixer contract, so it is the caller's).
 *   k_cache  [B][T][Hkv][d] dtype  un-rotated keys; T = cfg->seq_len is the
 *            cache capacity, tokens 0 .. n_tokens-1 of every sequence are valid
 *   idx      index arrays laid out for cfg (NB = T / block_size blocks)
 *   n_indexed  blocks whose summary and address idx already holds (0 for an
 *            empty index)
 *   n_tokens   valid tokens per sequence, 0 <= n_tokens <= T
 * Computes the summary and address of blocks n_indexed .. n_tokens/beta - 1
 * (as mono_build_index does) and rebuilds offsets, entries, load and
 * overflow over blocks 0 .. n_tokens/beta - 1; entries past the lists are
 * -1.  Each list keeps its first `capacity` blocks, so the lists equal those
 * mono_build_index gives for the first n_tokens/beta blocks.  A partial last
 * block is not indexed.  MONO_ERR_SHAPE if n_tokens > T or n_indexed is
 * outside 0 .. n_tokens/beta.  No workspace. */
mono_status mono_decode_index(const mono_config *cfg, const void *k_cache, const float *rope_cos,
                              const float *rope_sin, const float *codebooks, const mono_index *idx,
                              int32_t n_indexed, int32_t n_tokens, void *stream);

/* One decode step: route and attend the token at position `pos` of every
 * sequence (the same reading of the pages as mono_route and
 * mono_selected_attention, for one query position).
 *   q        [B][Hq][d] dtype  un-rotated queries of the new token
 *   k_cache, v_cache [B][T][Hkv][d] dtype  tokens 0 .. pos valid (the new
 *            token's key and value already written at pos)
 *   idx      an index covering at least blocks 0 .. pos/beta - n_local (from
 *            mono_decode_index or mono_build_index over the same layout)
 *   sel      [B][Hq][R] int32  output: selected remote blocks, ascending, -1 padded
 *   out      [B][Hq][d] dtype  output: attention of the new token
 * The selection and the output equal what mono_route and
 * mono_selected_attention give row pos of the sequence.  MONO_ERR_SHAPE if
 * pos is outside 0 .. T-1.  No workspace. */
mono_status mono_decode_step(const mono_config *cfg, const void *q, const void *k_cache,
                             const void *v_cache, const float *rope_cos, const float *rope_sin,
                             const float *codebooks, const mono_index *idx, int32_t pos,
                             int32_t *sel, void *out, void *stream);

/* The whole mixer (report page, "Mixer" and Figure 1): stateless, normalized
 * stream in, attention delta of the same shape out.
 *   x      [B][T][W] dtype
 *   w_qkv  [W][(Hq + 2 Hkv) d] dtype   columns: q heads, then k heads, then v heads
 *   w_o    [Hq d][W] dtype
 *   delta  [B][T][W] dtype             output: concat_h(attention_h) * w_o
 *   stats  int32[2] device or NULL     output: total overflow, maximum load
 * Runs projections, mono_build_index, mono_route, mono_selected_attention and
 * the output projection.  Workspace: MONO_WS_MIXER; the mixer's q, k, v,
 * index, selection and attention output live in the workspace at the offsets
 * given by mono_mixer_layout. */
mono_status mono_mixer_forward(const mono_config *cfg, const void *x, const void *w_qkv,
                               const void *w_o, const float *codebooks, const float *rope_cos,
                               const float *rope_sin, void *delta, int32_t *stats, void *ws,
                               size_t ws_bytes, void *stream);

/* Byte offsets inside the mixer workspace (for inspection by callers and
 * tests): q, k, v, kbar, addr, offsets, entries, load, overflow, sel, attn_out,
 * then the start of the inner calls' workspace.  offsets_out must hold 12
 * values.  Returns MONO_ERR_NULL / MONO_ERR_SHAPE / MONO_ERR_UNSUPPORTED or
 * MONO_OK. */
mono_status mono_mixer_layout(const mono_config *cfg, size_t *offsets_out);

/* Static description of a status code. */
const char *mono_status_string(mono_status status);

#ifdef __cplusplus
}
#endif

#endif /* MONO_H */
