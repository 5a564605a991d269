/*
 * attn.h - f32 grouped-query scaled dot-product attention on MI355X (gfx950).
 *
 * The C ABI of libattn.so. It implements three ops of the graph protocol's op
 * catalogue (page "https://vtmu.mpakt.dev/api/ops"):
 *
 *   attention    scaled dot-product attention in which several query heads
 *                may share one key/value head; q, k and v are flat
 *                row-major f32, the score matrix is never
 *                written to memory (op `attention`: summary, inputs, params,
 *                features attention.alibi/.bias/.scale/.softcap/.window).
 *   cache_write  writes rows into a preallocated cache in place (op
 *                `cache_write`: inputs cache [maxRows, width] and values
 *                [rows, width], param offset, mutatesInput 0).
 *   rope         rotary position embedding (op `rope`), standalone, fused
 *                into cache_write (rotate k, then write it) and fused into
 *                attention's q loads (attn_params.q_rope).
 *
 * Conventions for every entry point:
 *   - Tensors are dense row-major f32 (catalogue convention: tensors are
 *     row-major f32), passed as DEVICE pointers that the caller owns. The
 *     library keeps no pointer after a call returns, allocates nothing,
 *     copies nothing between host and device and never synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and runs asynchronously: a device fault shows at the caller's next
 *     synchronisation, not in the return code.
 *   - Every argument is checked before anything is launched, so a call that
 *     returns an error has written nothing. Errors name the parameter or the
 *     feature, following the catalogue's rule that a graph which needs an
 *     unsupported feature is rejected and the error names that feature;
 *     attn_last_error() returns
 *     that text for the calling thread.
 *   - Calls that write overlapping memory on one stream are ordered by the
 *     stream; on different streams they race.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ATTN_OK 0
#define ATTN_ERR_INVALID 1     /* a shape, size, pointer or parameter value is wrong */
#define ATTN_ERR_UNSUPPORTED 2 /* a valid request this library has no kernel for */
#define ATTN_ERR_DEVICE 3      /* the HIP runtime refused a launch */

/* attn_params.alibi: which ALiBi slope table (op `attention`, params alibi,
 * alibiMax, alibiSlopes; feature attention.alibi). */
#define ATTN_ALIBI_NONE 0
#define ATTN_ALIBI_BLOOM 1    /* `alibi: true`: BLOOM / ALiBi-paper slopes */
#define ATTN_ALIBI_MPT 2      /* `alibiMax`: MPT slopes with alibi_bias_max = alibi_max */
#define ATTN_ALIBI_EXPLICIT 3 /* `alibiSlopes`: alibi_slopes[heads], host memory */
#define ATTN_ALIBI_MAX_HEADS 256

/* attn_params position bias limits (thresholds and the largest threshold). */
#define ATTN_PB_MAX_BUCKETS 128
#define ATTN_PB_MAX_DIST 512

/* attn_params.bias_kind: the optional fourth input (feature attention.bias). */
#define ATTN_BIAS_NONE 0
#define ATTN_BIAS_TS 1  /* bias [T, S], shared by all heads */
#define ATTN_BIAS_HTS 2 /* bias [heads, T, S] */

/*
 * One field per parameter of the catalogue's `attention` op. Call
 * attn_params_init() first: it sets every optional field to "absent".
 *
 *   T, S         query rows and key/value rows (>= 0).
 *   heads        num_attention_heads (> 0).
 *   kv_heads     num_key_value_heads; 0 = absent = heads. heads must be a
 *                multiple of it; query head h reads key/value head
 *                floor(h * kv_heads / heads) (contiguous groups).
 *   head_dim     query/key width per head (> 0).
 *   v_head_dim   value width per head; 0 = absent = head_dim.
 *   causal       default 1. Causal: key s is visible to query row t when
 *                s <= pos with pos = pos_offset + t.
 *   pos_offset   the position query row 0 sits at (>= 0, default 0);
 *                key row s sits at position s. With a KV cache, k and v are
 *                the whole caches (S = maxRows) and causal masking hides the
 *                rows past the current position, which are never read.
 *   has_scale, scale
 *                the score scale; absent = 1/sqrt(head_dim). It multiplies
 *                q.k only, never the ALiBi or bias terms.
 *   softcap      0 = off, > 0: x = softcap * tanh(x / softcap), applied to the
 *                scaled score before ALiBi, bias and the mask (feature
 *                attention.softcap places the cap ahead of masking).
 *   window       0 = off, > 0: sliding window. Causal: pos - window < s <= pos.
 *                Non-causal: |pos - s| <= window.
 *   alibi, alibi_max, alibi_slopes
 *                ALiBi; adds -slope[h] * |pos - s| to the score. alibi_slopes
 *                is a HOST pointer to `heads` floats, read during the call and
 *                not kept. At most ATTN_ALIBI_MAX_HEADS heads.
 *   bias_kind    ATTN_BIAS_*; the bias is added after softcap and ALiBi (a
 *                -1e9 entry masks its key, as the catalogue suggests).
 *   q_rope       NULL, or a rotary embedding applied to q as the kernels load
 *                it: the call computes attention(rope(q), k, v, bias) with
 *                rope as attn_rope() defines it (its own offset gives row 0's
 *                position; its head_dim must be 0 or head_dim). HOST pointer,
 *                read during the call and not kept. It fuses the rope that
 *                precedes attention in a decode graph into the attention call.
 *   pb_weight, pb_buckets, pb_n, pb_bidirectional
 *                bucketed relative position bias (not a catalogue param: the
 *                IR schema page lists position_bias {weight, buckets} on its
 *                attention op; read as T5's relative attention bias).
 *                pb_buckets: HOST pointer to pb_n ascending distance
 *                thresholds, the first 0 and the last at most
 *                ATTN_PB_MAX_DIST (read during the call, not kept); the
 *                bucket of a key is the last threshold <= |pos - s|, plus
 *                pb_n for a key after the query when pb_bidirectional.
 *                pb_weight: DEVICE pointer to [pb_n (2 pb_n when
 *                bidirectional), heads] f32; weight[bucket, h] is added to
 *                the score where ALiBi is. pb_weight NULL = off. At most
 *                ATTN_PB_MAX_BUCKETS thresholds.
 *   rel_k, rel_v, rel_max
 *                relative key/value embeddings (IR schema relative_kv {key,
 *                value, max_distance}; read as Shaw et al.'s relative position
 *                representations, shared by all heads). With
 *                r = clip(s - pos, -rel_max, rel_max) + rel_max, rel_k[r]
 *                (DEVICE, [2 rel_max + 1, head_dim]) is added to the key before
 *                the product with q, rel_v[r] (DEVICE, [2 rel_max + 1,
 *                v_head_dim], or NULL) to the value. rel_k NULL = off.
 *   sinks        attention sinks (0 = none; not a catalogue param: the graph
 *                IR schema carries `sinks` beside `window` on op_attention and
 *                slot_kv). With a window on, keys s < sinks stay visible beside
 *                it, as StreamingLLM keeps its initial tokens; causal rows still
 *                see only s <= pos. Without a window it changes nothing.
 *
 * A query row with no visible key outputs zeros.
 */
typedef struct attn_params {
    int64_t T, S;
    int64_t heads, kv_heads;
    int64_t head_dim, v_head_dim;
    int64_t pos_offset;
    int64_t window;
    int32_t causal;
    int32_t has_scale;
    float scale;
    float softcap;
    int32_t alibi;
    float alibi_max;
    const float* alibi_slopes;
    int32_t bias_kind;
    int32_t reserved;
    const struct attn_rope_params* q_rope;
    int64_t sinks;
    const float* pb_weight;
    const int64_t* pb_buckets;
    int64_t pb_n;
    int32_t pb_bidirectional;
    int32_t reserved2;
    const float* rel_k;
    const float* rel_v;
    int64_t rel_max;
} attn_params;

/* Fill *p with the catalogue's defaults: causal = 1, everything optional
 * absent, sizes 0. */
void attn_params_init(attn_params* p);

/* Check *p without touching any device: ATTN_OK, ATTN_ERR_INVALID or
 * ATTN_ERR_UNSUPPORTED, with attn_last_error() naming the field. */
int attn_validate(const attn_params* p);

/* Bytes of device workspace attn_forward or attn_forward_append needs for
 * *p (0 if none; also 0 for an invalid *p). The workspace holds per-split
 * partial softmax state. */
size_t attn_workspace_size(const attn_params* p);

/*
 * out[T, heads*v_head_dim] = attention(q, k, v, bias) (op `attention`).
 *   q    [T, heads*head_dim]        device, read-only
 *   k    [S, kv_heads*head_dim]     device, read-only
 *   v    [S, kv_heads*v_head_dim]   device, read-only
 *   bias [T, S] or [heads, T, S]    device, read-only; NULL iff bias_kind = 0
 *   out  [T, heads*v_head_dim]      device, written; must not overlap inputs
 *   workspace, workspace_bytes
 *        device scratch of at least attn_workspace_size(p) bytes (NULL when
 *        that is 0), 256-byte aligned; it holds the partial softmax states
 *        of key-range splits. Its contents need no initialisation and mean
 *        nothing after the call. Two calls in flight at once must not share
 *        a workspace.
 * q, k, v, bias and out must be 16-byte aligned. T = 0 is a no-op; S = 0
 * writes zeros.
 */
int attn_forward(const attn_params* p, const float* q, const float* k, const float* v,
                 const float* bias, float* out, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Size of the device array attn_forward_noalloc keeps its split state in. */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * attn_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same plan, kernels and result as attn_forward, with the key-range
 * splits' partial softmax states in a library-owned array of
 * ATTN_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU instead of a caller's workspace.
 *   q, k, v, bias, out, stream  as for attn_forward; the caller still
 *                               provides every input and the output.
 * The array is a file-scope device variable: each GPU the library runs on
 * holds its own copy from its first use until the process ends. The call
 * allocates nothing and calls no allocating routine; its first call on a
 * device looks the array's address up (hipGetSymbolAddress) with that
 * device current, and later calls reuse it. `stream` must belong to the
 * current device (else ATTN_ERR_INVALID).
 * A call whose plan needs more split state than the array holds (the
 * figure attn_workspace_size reports for attn_forward's own plan) is
 * refused with ATTN_ERR_UNSUPPORTED before anything runs; decode calls
 * need at most a few MiB (heads x splits x (v_head_dim + 2) floats).
 * Every call on one GPU shares that GPU's array, and nothing in it needs
 * clearing (each split writes its whole state before the merge reads it):
 * two calls that overlap in time on one GPU, on different streams or from
 * different threads, race on it.
 */
int attn_forward_noalloc(const attn_params* p, const float* q, const float* k, const float* v,
                         const float* bias, float* out, void* stream);

/*
 * Op `cache_write`: cache[offset + r, :] = values[r, :] for r < rows, in
 * place; the rest of the cache is untouched. An exact bit copy.
 *   cache   [max_rows, width]  device, written
 *   values  [rows, width]      device, read-only; must not overlap the rows
 *                              being written
 * Requires 0 <= offset and offset + rows <= max_rows. rows = 0 is a no-op.
 */
int attn_cache_write(float* cache, int64_t max_rows, int64_t width, const float* values,
                     int64_t rows, int64_t offset, void* stream);

/*
 * Two `cache_write` ops at the same rows in one launch, as a decode step
 * appends its new K and V rows: cache_a[offset + r, :] = values_a[r, :] and
 * cache_b[offset + r, :] = values_b[r, :] for r < rows. Each cache takes
 * attn_cache_write's checks (messages prefixed "a: " / "b: "); in addition
 * neither copy may write rows the other one reads or writes. Same result,
 * bit for bit, as the two attn_cache_write calls. rows = 0 is a no-op.
 */
int attn_cache_write2(float* cache_a, int64_t max_rows_a, int64_t width_a, const float* values_a,
                      float* cache_b, int64_t max_rows_b, int64_t width_b, const float* values_b,
                      int64_t rows, int64_t offset, void* stream);

/*
 * A decode step in one call: the two `cache_write` ops that append the
 * step's new K and V rows to the caches, then op `attention` over the
 * caches (the op catalogue's cache_write feeding attention through a
 * preallocated KV cache at posOffset). Same result as
 *   attn_cache_write2(k, S, kv_heads*head_dim, k_new,
 *                     v, S, kv_heads*v_head_dim, v_new, rows, offset, stream);
 *   attn_forward(p, q, k, v, bias, out, workspace, workspace_bytes, stream);
 * with the caches bit for bit that copy's and out within rounding of that
 * attn_forward (its splits of the key range may differ).
 *   k      [S, kv_heads*head_dim]     device, the K cache; rows
 *                                     [offset, offset + rows) are written
 *   v      [S, kv_heads*v_head_dim]   device, the V cache; likewise
 *   k_new  [rows, kv_heads*head_dim]    device, read-only
 *   v_new  [rows, kv_heads*v_head_dim]  device, read-only
 *   q, bias, out, workspace, stream as for attn_forward (p->S is the
 *   caches' row count); workspace_bytes >= attn_workspace_size(p).
 * Requires 0 <= offset and offset + rows <= S; rows = 0 is attn_forward.
 * Each cache takes attn_cache_write's checks (messages prefixed "k: " and
 * "v: "). The K rows written and the V rows written must not overlap, nor
 * either of them a new-row buffer, q or bias; out and the workspace must
 * not overlap k_new or v_new. Where the new rows are the last keys the
 * call sees (offset + rows is the end of its key range, as in a causal decode
 * step appending at posOffset), there are at most 64 of them, k_new and v_new
 * are 16-byte aligned and the call takes the decode path without
 * relative-position terms, one kernel reads them from k_new and v_new while
 * it writes them to the caches; otherwise the copy runs first, in a launch
 * of its own. T = 0 only writes the rows.
 */
int attn_forward_append(const attn_params* p, const float* q, float* k, float* v, const float* k_new,
                        const float* v_new, int64_t rows, int64_t offset, const float* bias, float* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Op `rope` (graph protocol op catalogue: rotary position embedding of a
 * [tokens, heads*headDim] tensor; params headDim, base, offset, rotaryDim,
 * interleaved, scaling, invFreq, attentionFactor; features rope.interleaved,
 * rope.rotaryDim, rope.scaling).
 *
 * Row t of x sits at position offset + t. In each head the first rotary_dim
 * channels form rotary_dim/2 pairs, (i, i + rotary_dim/2) by default or
 * (2i, 2i+1) when interleaved, and pair i turns by the angle
 * position * inv_freq[i]: (a, b) -> (a cos - b sin, a sin + b cos), with cos
 * and sin both multiplied by the attention factor. Channels from rotary_dim
 * on pass through unchanged.
 *
 * The inverse-frequency table is f32. It is an explicit inv_freq if given,
 * else base^(-2i/rotary_dim), changed by `scaling` as a model config's
 * rope_scaling asks:
 *   LINEAR    every frequency divided by factor (position interpolation)
 *   LLAMA3    Llama 3.1's rule: wavelengths below original/high_freq_factor
 *             kept, above original/low_freq_factor divided by factor, blended
 *             linearly in original/wavelength in between
 *   YARN      YaRN's NTK-by-parts: pairs turning more than beta_fast times over
 *             the original context kept, fewer than beta_slow times divided by
 *             factor, a linear ramp over the pair index in between (its ends
 *             rounded outwards unless truncate = 0); attention factor
 *             0.1 ln(factor) + 1, or the ratio of that with mscale and with
 *             mscale_all_dim when both are given
 *   LONGROPE  frequencies divided by long_factor[i] once offset + T exceeds
 *             original_max_positions, else by short_factor[i]; attention
 *             factor sqrt(1 + ln(f) / ln(original)) with f = factor, or
 *             max_positions / original when factor is 0
 *   DYNAMIC   once offset + T exceeds original_max_positions (or
 *             max_positions), base grows to base * (factor * (offset + T) /
 *             original - (factor - 1))^(rotary_dim / (rotary_dim - 2))
 * Each table entry and the attention factor are computed in double precision
 * and rounded to f32 once. The attention factor is attention_factor when
 * has_attention_factor, else scaling_attention_factor when non-zero (the
 * scaling object's own attention_factor), else the scaling's derived one,
 * else 1. The angle itself is evaluated to better than 1e-7 rad for every
 * position below 2^31.
 */
#define ATTN_ROPE_DEFAULT 0
#define ATTN_ROPE_LINEAR 1
#define ATTN_ROPE_LLAMA3 2
#define ATTN_ROPE_YARN 3
#define ATTN_ROPE_LONGROPE 4
#define ATTN_ROPE_DYNAMIC 5
#define ATTN_ROPE_MAX_ROTARY_DIM 256

/*
 * One field per parameter of the catalogue's `rope` op; call
 * attn_rope_params_init() first (0 means "absent" where noted).
 *   head_dim      per-head width (> 0)
 *   rotary_dim    rotated channels per head; 0 = head_dim. Even, <= head_dim,
 *                 at most ATTN_ROPE_MAX_ROTARY_DIM.
 *   offset        position of the first row (>= 0); positions stay below 2^31
 *   interleaved   0: half-split pairs (Llama, NeoX); 1: interleaved (GPT-J)
 *   base          rope_theta; 0 = 10000
 *   inv_freq      HOST pointer to rotary_dim/2 floats, or NULL; replaces base
 *                 and scaling
 *   has_attention_factor, attention_factor
 *                 the op's attentionFactor
 *   scaling       ATTN_ROPE_*; the fields below hold the rope_scaling object's
 *                 values: factor, low_freq_factor (0 = 1), high_freq_factor
 *                 (0 = 4), original_max_positions, max_positions,
 *                 beta_fast (0 = 32), beta_slow (0 = 1), mscale,
 *                 mscale_all_dim, truncate (init: 1), short_factor and
 *                 long_factor (HOST pointers to rotary_dim/2 doubles),
 *                 scaling_attention_factor (0 = absent)
 */
typedef struct attn_rope_params {
    int64_t head_dim;
    int64_t rotary_dim;
    int64_t offset;
    int32_t interleaved;
    int32_t scaling;
    double base;
    const float* inv_freq;
    int32_t has_attention_factor;
    float attention_factor;
    double factor;
    double low_freq_factor, high_freq_factor;
    int64_t original_max_positions, max_positions;
    double beta_fast, beta_slow;
    double mscale, mscale_all_dim;
    int32_t truncate;
    int32_t reserved;
    const double* short_factor;
    const double* long_factor;
    double scaling_attention_factor;
} attn_rope_params;

/* Fill *r with the defaults: everything absent, truncate = 1. */
void attn_rope_params_init(attn_rope_params* r);

/* The resolved table for `rows` rows starting at position r->offset (host
 * only; dynamic and longrope depend on offset + rows): rotary_dim/2 floats
 * into inv_freq (host memory) and the attention factor. */
int attn_rope_table(const attn_rope_params* r, int64_t rows, float* inv_freq, float* attention_factor);

/*
 * out[T, width] = rope(x[T, width]), width = heads * head_dim (a multiple of
 * head_dim). x and out are device pointers; out may equal x (in place) but
 * must not otherwise overlap it. T = 0 is a no-op.
 */
int attn_rope(const attn_rope_params* r, int64_t T, int64_t width, const float* x, float* out,
              void* stream);

/*
 * Rotate, then write (ops `rope` then `cache_write` fused): cache[offset + t, :]
 * = rope(values)[t, :] for t < rows, the row positions taken from r->offset.
 * width = kvHeads * head_dim. Same checks as attn_cache_write.
 */
int attn_rope_cache_write(float* cache, int64_t max_rows, int64_t width, const float* values,
                          int64_t rows, int64_t offset, const attn_rope_params* r, void* stream);

/* Text of the calling thread's last error ("" if the last call succeeded). */
const char* attn_last_error(void);

/*
 * Which kernels attn_forward would launch for *p (host only). Lets tests
 * and measurement tools name the path; not needed to run the op.
 *   path    ATTN_PATH_*
 *   splits  key-range splits (decode path, or prefill on a small grid; the
 *           partial states are merged by a combine kernel); 1 elsewhere
 *   tile_q  query rows per workgroup on the prefill path
 */
#define ATTN_PATH_EMPTY 0   /* T = 0 or no work */
#define ATTN_PATH_ZERO 1    /* S = 0: zero fill */
#define ATTN_PATH_GENERIC 2 /* any shape; correctness path */
#define ATTN_PATH_DECODE 3  /* few query rows: split-S + combine */
#define ATTN_PATH_PREFILL 4 /* fp32 MFMA flash kernel */
#define ATTN_PATH_MLA 5     /* latent attention: absorb, split, combine (attn_mla_plan) */
typedef struct attn_plan_info {
    int32_t path;
    int32_t splits;
    int32_t tile_q;
    int32_t variant;  /* decode: 1 = the matrix-core kernel, 0 = the vector one;
                         prefill: the MFMA tile (32 = 32x32x2, 16 = 16x16x4);
                         MLA (attn_mla_plan): the latent slices the merge uses
                         (0 = one merge per group of output channels) */
} attn_plan_info;
int attn_plan(const attn_params* p, attn_plan_info* info);

/*
 * Latent (MLA) attention: the IR schema page's op_mla_attention (properties
 * state, heads, kv_rank, qk_nope, qk_rope, v_head_dim, k_b, v_b, scale,
 * causal, window, sinks; the op catalogue names DeepSeek MLA beside
 * attention's vHeadDim). No page gives its rule; the reading implemented is
 * DeepSeek-V2's multi-head latent attention: head h attends, exactly as op
 * `attention` would, with keys [k_b[h] c_s ; k_pe_s] and values v_b[h] c_s,
 * where state row s is [c_s (kv_rank floats) | k_pe_s (qk_rope floats)].
 *
 *   T, S         query rows and latent state rows
 *   heads, kv_rank, qk_nope, qk_rope, v_head_dim
 *                as the schema names them (qk_rope may be 0)
 *   causal       default 1
 *   has_scale, scale
 *                scale multiplies q.key; default 1/sqrt(qk_nope + qk_rope)
 *   pos_offset   position of query row 0 (>= 0); state row s sits at s
 *   window, sinks
 *                as attn_params (0 = off / none)
 */
typedef struct attn_mla_params {
    int64_t T, S;
    int64_t heads, kv_rank, qk_nope, qk_rope, v_head_dim;
    int32_t causal;
    int32_t has_scale;
    float scale;
    int32_t reserved;
    int64_t pos_offset;
    int64_t window;
    int64_t sinks;
} attn_mla_params;

/* Defaults: causal = 1, everything else 0 / absent. */
void attn_mla_params_init(attn_mla_params* p);

/* Check *p without touching any device (ATTN_ERR_INVALID / _UNSUPPORTED name
 * the field). */
int attn_mla_validate(const attn_mla_params* p);

/* Bytes of device workspace attn_mla_forward needs (0 for an invalid *p or
 * when nothing is launched). It holds the absorbed queries, the key
 * splits' partial softmax states and, for the merge by latent slices, each
 * slice's share of the outputs and a counter per row. */
size_t attn_mla_workspace_size(const attn_mla_params* p);

/* Which kernels attn_mla_forward would launch: path ATTN_PATH_MLA (or EMPTY
 * / ZERO), splits = key-range splits, tile_q = rows per workgroup (16 on
 * the matrix-core kernel, 1 on the generic one), variant = latent slices of
 * the merge (0: per-output merge). */
int attn_mla_plan(const attn_mla_params* p, attn_plan_info* info);

/*
 * out[T, heads*v_head_dim] = latent attention, evaluated in absorbed form:
 * q's no-rope part is multiplied into k_b first, the softmax runs over the
 * latent rows themselves (each read once for every head), and v_b is
 * applied to the weighted latent sum.
 *   q      [T, heads*(qk_nope + qk_rope)]   device, read-only; per head the
 *                                           no-rope part, then the rotary part
 *   state  [S, kv_rank + qk_rope]           device, read-only (the latent KV
 *                                           cache; rows past the visible
 *                                           range are never read)
 *   k_b    [heads, qk_nope, kv_rank]        device, read-only
 *   v_b    [heads, v_head_dim, kv_rank]     device, read-only
 *   out    [T, heads*v_head_dim]            device, written; must not
 *                                           overlap any input
 *   workspace, workspace_bytes
 *          at least attn_mla_workspace_size(p) bytes, 256-byte aligned, not
 *          overlapping any tensor; contents need no initialisation. Two
 *          calls in flight at once must not share a workspace.
 * All pointers 16-byte aligned. T = 0 is a no-op; rows that see no key
 * (S = 0, or a window past the state) are 0. Rotary embeddings of q and
 * k_pe are the caller's (they precede this op, as `rope` precedes
 * `attention`).
 */
int attn_mla_forward(const attn_mla_params* p, const float* q, const float* state, const float* k_b,
                     const float* v_b, float* out, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Tuning overrides for tests and sweeps (process-wide, not thread-safe):
 *   "decode_splits"  force the decode split count (0 = automatic)
 *   "decode_depth"   batches in flight per lane in the decode kernel, 2 or 3 (0 = automatic)
 *   "decode_wgs_per_cu" workgroups per CU the decode split count aims for, 1..8
 *                    (0 = automatic: 2 for the vector kernel; 1 for the
 *                    matrix-core one where headDim + vHeadDim >= 256, else 2)
 *   "decode_mfma"    1: the matrix-core decode wherever it can serve; -1: never;
 *                    0 = automatic (groups of 5 or more query rows)
 *   "decode_rotate"  split i starts its chunk (i * value mod chunk) rows in
 *                    (rounded to a batch step); 0 = automatic (5/8 of a chunk)
 *   "decode_block"   where every query row sees every key of the range, the
 *                    splits take interleaved blocks of this many rows (a power
 *                    of two in 32..4096) instead of one chunk each; -1 = always
 *                    chunks; 0 = automatic (256-row blocks, 512-row ones on
 *                    the matrix-core decode, where a split has 1024 keys or
 *                    more and blocks keep the longest split as short, else
 *                    chunks)
 *   "prefill_splits" force the prefill key-range split count (0 = automatic, max 16)
 *   "prefill_variant" force the prefill kernel: 32 (32x32x2 MFMA, 32-row waves) or
 *                    16 (16x16x4 MFMA, 16-row waves); 0 = automatic
 *   "force_path"     force ATTN_PATH_GENERIC / _DECODE / _PREFILL (0 = automatic);
 *                    a forced path that cannot serve *p is refused
 *   "mla_splits"     force the MLA key-range split count (0 = automatic)
 *   "mla_row_groups" 16-row blocks per MLA split workgroup, 1 or 2 (0 = automatic)
 *   "mla_combine_out" output channels per MLA merge workgroup, 16 or 32 (0 = automatic)
 *   "mla_slices"     1: merge the MLA splits by 64-channel latent slices (each
 *                    slice's share of the outputs, added by the row's last
 *                    slice workgroup) where kv_rank is a multiple of 64 up to 512
 *                    and v_head_dim <= 256; -1: never; 0 = automatic
 *   "mla_generic"    1: run MLA on the generic kernel even where the
 *                    matrix-core one has an instance (0 = automatic)
 * Returns ATTN_ERR_INVALID for an unknown name.
 */
int attn_set_option(const char* name, int64_t value);

/*
 * Kernel timing for measurement harnesses. While enabled, every kernel the
 * library launches is bracketed by a pair of HIP events recorded on the
 * stream it runs on. attn_timing_collect() waits for the recorded events and
 * returns, for the kernel named `kernel`, the summed duration and the launch
 * count since the last collect (then clears them). Off by default; the hot
 * path records nothing when off. Event pairs come from a fixed pool of 4096,
 * created on the first enable; launches beyond the pool are not timed.
 * Kernel names: "cache_write", "decode_split", "decode_mfma", "prefill",
 * "prefill_band" (the band tiles' launch of a prefill with relative key/value
 * embeddings at widths past 64/64), "combine" (merges key-range splits after
 * the decode and prefill kernels), "generic", "zero_fill", "rope" (attn_rope
 * and attn_rope_cache_write), "mla_absorb", "mla_split", "mla_combine".
 */
int attn_timing_enable(int on);
int attn_timing_collect(const char* kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
