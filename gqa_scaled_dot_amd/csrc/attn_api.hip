// Host side of libattn.so: the C ABI declared in attn.h. Resolves the op's
// defaults, checks every argument before anything runs (refusing by name,
// as the op catalogue's feature convention asks), builds the ALiBi slope
// table, chooses a kernel path and launches it on the caller's stream.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "attn.h"
#include "kernels.h"

// Workspace of attn_forward_noalloc: the key-range splits' partial softmax
// states live in this array instead of a caller's buffer, for callers that
// cannot allocate. Every GPU the library runs on holds its own copy until the
// process ends. Host code never uses this name as an address (on the host it
// is only a stand-in): it takes each device's address once, through
// hipGetSymbolAddress, and passes that to the kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return ATTN_OK;
}

// Process-wide tuning overrides (attn_set_option).
int64_t g_opt_decode_splits = 0;
int64_t g_opt_decode_depth = 0;
int64_t g_opt_decode_wgs = 0;
int64_t g_opt_decode_rotate = 0;
int64_t g_opt_decode_block = 0;
int64_t g_opt_prefill_splits = 0;
int64_t g_opt_prefill_variant = 0;
int64_t g_opt_force_path = 0;
int64_t g_opt_decode_mfma = 0;  // 0: automatic; 1: the matrix-core decode wherever it can serve; -1: never
int64_t g_opt_mla_splits = 0;
int64_t g_opt_mla_generic = 0;
int64_t g_opt_mla_row_groups = 0;
int64_t g_opt_mla_combine_out = 0;  // 0: automatic; 16 or 32 output channels per combine workgroup
int64_t g_opt_mla_slices = 0;       // 0: automatic; 1: merge by latent slices where possible; -1: never

constexpr int kCUs = 256;                 // MI355X compute units
constexpr int kXcdCount = 8;              // XCDs (each with its own L2) the CUs sit in
constexpr int kDecodeWgPerCU = 2;         // decode_split occupancy target (decode_mfma: see make_plan)
constexpr int kDecodeDepth = 1;           // decode_split batches per lane at a time (no prefetch ring)
// Smallest key chunk worth a workgroup. A decode_split workgroup costs ~8 us
// however few keys it reads (launch, q, two load round trips, merges), so
// short caches want many small chunks: measured on Llama widths, 4096 keys
// take 14 us in 32-64 chunks against 19 us in 16.
constexpr int64_t kDecodeMinKeys = 64;
constexpr int64_t kDecodeChunkAlign = 64; // key chunk granularity (a multiple of 16 row groups x 2 rows)
constexpr int64_t kDecodeBlock = 256;     // rows per interleaved block, automatic choice (power of two)
constexpr int64_t kDecodeMaxSplits = 1024;
constexpr int64_t kDecodeMaxAppend = 64;
constexpr int64_t kDecodeMfmaFrom = 5;    // groups of this many query rows or more take decode_mfma  // appended rows one decode split takes (two batch steps)
constexpr int64_t kPrefillMaxSplits = 16;
constexpr int64_t kPrefillMinTilesPerSplit = 4;
constexpr int64_t kMaxDim = 1 << 16;
constexpr int64_t kRelMaxDistance = 512;  // relative_kv: per-row tables of 2 max + 1 entries in LDS
constexpr int64_t kMlaMaxSplits = 1024;
constexpr int64_t kMlaMinKeys = 64;       // smallest key chunk worth an MLA split workgroup (four tiles)
constexpr int64_t kMlaChunkAlign = 16;    // the MLA split kernel's key tile
constexpr int64_t kMlaGenericMaxFloats = 15000;  // generic MLA kernel: (R + P) + R + 260 floats of LDS

// ---------------------------------------------------------------------------
// ALiBi slope tables (op `attention`, params alibi / alibiMax / alibiSlopes).
// BLOOM, as in the ALiBi paper: with p the largest power of two <= H, head
// i = 1..p gets 2^(-8i/p); further heads take 2^(-4j/p) for odd j = 1, 3, ...
// MPT with alibi_bias_max b: with n the smallest power of two >= H, head
// i = 1..n gets 2^(-ib/n); when n != H the even-numbered ones come first,
// then the odd-numbered ones, and the first H are kept.
// Computed in double and rounded once to f32, the op's number type.
// ---------------------------------------------------------------------------
void slopes_bloom(int64_t H, float* out) {
    int64_t p = 1;
    while (p * 2 <= H) p *= 2;
    int64_t n = 0;
    for (int64_t i = 1; i <= p; ++i) out[n++] = (float)exp2(-8.0 * (double)i / (double)p);
    for (int64_t j = 1; n < H; j += 2) out[n++] = (float)exp2(-4.0 * (double)j / (double)p);
}

void slopes_mpt(int64_t H, double b, float* out) {
    int64_t n = 1;
    while (n < H) n *= 2;
    int64_t k = 0;
    if (n == H) {
        for (int64_t i = 1; i <= n; ++i) out[k++] = (float)exp2(-(double)i * b / (double)n);
        return;
    }
    for (int64_t i = 2; i <= n && k < H; i += 2) out[k++] = (float)exp2(-(double)i * b / (double)n);
    for (int64_t i = 1; i <= n && k < H; i += 2) out[k++] = (float)exp2(-(double)i * b / (double)n);
}

// ---------------------------------------------------------------------------
// Rotary embedding tables (op `rope`, params base, rotaryDim, scaling,
// invFreq, attentionFactor). Every value is computed in double and rounded to
// f32 once, with no fused multiply-adds (contraction is switched off in each
// function), so the table is a fixed function of the parameters.
// ---------------------------------------------------------------------------
// RoFormer's frequencies base^(-2i/rd).
double rope_theta(double base, int64_t i, int64_t rd) {
#pragma clang fp contract(off)
    return pow(base, -2.0 * (double)i / (double)rd);
}

// Llama 3.1: keep short wavelengths, divide long ones by factor, blend linearly
// in original/wavelength between original/high_freq_factor and
// original/low_freq_factor.
double rope_llama3(double f, const attn_rope_params* r, double lo_f, double hi_f) {
#pragma clang fp contract(off)
    const double orig = (double)r->original_max_positions;
    const double wl = 2.0 * M_PI / f;
    if (wl < orig / hi_f) return f;
    if (wl > orig / lo_f) return f / r->factor;
    const double smooth = (orig / wl - lo_f) / (hi_f - lo_f);
    return (1.0 - smooth) * f / r->factor + smooth * f;
}

double yarn_mscale(double scale, double k) {
#pragma clang fp contract(off)
    return scale > 1.0 ? 0.1 * k * log(scale) + 1.0 : 1.0;
}

int rope_compute(const attn_rope_params* r, int64_t seq_len, attn::RopeArgs* out);

// The last table each thread resolved, keyed by the parameters (arrays by
// content; the row offset only moves positions, and the sequence length
// matters to dynamic and longrope alone), so a decode loop that passes the
// same rope every step skips the table's pow and log calls.
struct RopeCache {
    bool valid = false;
    attn_rope_params key;
    int64_t seq_key = 0;
    float inv[ATTN_ROPE_MAX_ROTARY_DIM / 2];
    double sf[ATTN_ROPE_MAX_ROTARY_DIM / 2], lf[ATTN_ROPE_MAX_ROTARY_DIM / 2];
    attn::RopeArgs val;
};
thread_local RopeCache g_rope_cache;

// Checks *r and fills the device-side description for rows at positions
// offset .. seq_len - 1.
int rope_resolve(const attn_rope_params* r, int64_t seq_len, attn::RopeArgs* out) {
    if (!r || r->head_dim <= 0 || r->head_dim > kMaxDim || r->offset < 0 || seq_len > INT32_MAX)
        return rope_compute(r, seq_len, out);  // the error path names the field
    const int64_t rd = r->rotary_dim ? r->rotary_dim : r->head_dim;
    if (rd <= 0 || rd % 2 || rd > r->head_dim || rd > ATTN_ROPE_MAX_ROTARY_DIM)
        return rope_compute(r, seq_len, out);
    const int64_t half = rd / 2;
    // The key keeps whether each array is given; their contents are compared below.
    attn_rope_params key = *r;
    key.offset = 0;
    key.inv_freq = r->inv_freq ? reinterpret_cast<const float*>(1) : nullptr;
    key.short_factor = r->short_factor ? reinterpret_cast<const double*>(1) : nullptr;
    key.long_factor = r->long_factor ? reinterpret_cast<const double*>(1) : nullptr;
    const bool seq_dep = !r->inv_freq && (r->scaling == ATTN_ROPE_DYNAMIC || r->scaling == ATTN_ROPE_LONGROPE);
    const int64_t seq_key = seq_dep ? seq_len : -1;
    RopeCache& c = g_rope_cache;
    if (c.valid && c.seq_key == seq_key && !memcmp(&c.key, &key, sizeof key) &&
        (!r->inv_freq || !memcmp(c.inv, r->inv_freq, sizeof(float) * half)) &&
        (!r->short_factor || !memcmp(c.sf, r->short_factor, sizeof(double) * half)) &&
        (!r->long_factor || !memcmp(c.lf, r->long_factor, sizeof(double) * half))) {
        *out = c.val;
        out->pos0 = r->offset;
        return ok();
    }
    const int rc = rope_compute(r, seq_len, out);
    if (rc) return rc;
    c.valid = true;
    c.key = key;
    c.seq_key = seq_key;
    if (r->inv_freq) memcpy(c.inv, r->inv_freq, sizeof(float) * half);
    if (r->short_factor) memcpy(c.sf, r->short_factor, sizeof(double) * half);
    if (r->long_factor) memcpy(c.lf, r->long_factor, sizeof(double) * half);
    c.val = *out;
    return ok();
}

int rope_compute(const attn_rope_params* r, int64_t seq_len, attn::RopeArgs* out) {
#pragma clang fp contract(off)
    if (!r) return fail(ATTN_ERR_INVALID, "rope: NULL params");
    if (r->head_dim <= 0 || r->head_dim > kMaxDim)
        return fail(ATTN_ERR_INVALID, "rope.headDim: must be in 1..%lld (got %lld)", (long long)kMaxDim,
                    (long long)r->head_dim);
    const int64_t rd = r->rotary_dim ? r->rotary_dim : r->head_dim;
    if (rd < 0 || rd % 2 || rd > r->head_dim)
        return fail(ATTN_ERR_INVALID, "rope.rotaryDim: must be even and in 2..headDim (got %lld)",
                    (long long)rd);
    if (rd > ATTN_ROPE_MAX_ROTARY_DIM)
        return fail(ATTN_ERR_UNSUPPORTED, "rope.rotaryDim: at most %d rotated channels (got %lld)",
                    ATTN_ROPE_MAX_ROTARY_DIM, (long long)rd);
    if (r->interleaved != 0 && r->interleaved != 1)
        return fail(ATTN_ERR_INVALID, "rope.interleaved: must be 0 or 1");
    if (r->offset < 0) return fail(ATTN_ERR_INVALID, "rope.offset: must be >= 0 (got %lld)", (long long)r->offset);
    if (seq_len > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED, "rope.offset: positions past 2^31-1");
    const double base = r->base == 0.0 ? 10000.0 : r->base;
    if (!(isfinite(base) && base > 0.0)) return fail(ATTN_ERR_INVALID, "rope.base: must be finite and > 0");
    if (r->has_attention_factor && !isfinite(r->attention_factor))
        return fail(ATTN_ERR_INVALID, "rope.attentionFactor: must be finite");
    if (!isfinite(r->scaling_attention_factor))
        return fail(ATTN_ERR_INVALID, "rope.scaling: attention_factor must be finite");
    if (r->scaling < ATTN_ROPE_DEFAULT || r->scaling > ATTN_ROPE_DYNAMIC)
        return fail(ATTN_ERR_UNSUPPORTED, "rope.scaling: unknown type %d", r->scaling);

    attn::RopeArgs& a = *out;
    memset(&a, 0, sizeof a);
    a.on = 1;
    a.rd = (int32_t)rd;
    a.interleaved = r->interleaved;
    a.pos0 = r->offset;
    const int64_t half = rd / 2;
    double af = 1.0;
    const bool needs_factor = r->scaling == ATTN_ROPE_LINEAR || r->scaling == ATTN_ROPE_LLAMA3 ||
                              r->scaling == ATTN_ROPE_YARN || r->scaling == ATTN_ROPE_DYNAMIC;
    if (r->inv_freq) {
        for (int64_t i = 0; i < half; ++i) {
            if (!isfinite(r->inv_freq[i]))
                return fail(ATTN_ERR_INVALID, "rope.invFreq: entry %lld is not finite", (long long)i);
            a.inv_freq[i] = r->inv_freq[i];
        }
    } else {
        if (needs_factor && !(isfinite(r->factor) && r->factor > 0.0))
            return fail(ATTN_ERR_INVALID, "rope.scaling: factor must be finite and > 0");
        if ((r->scaling == ATTN_ROPE_LLAMA3 || r->scaling == ATTN_ROPE_YARN ||
             r->scaling == ATTN_ROPE_LONGROPE) && r->original_max_positions <= 0)
            return fail(ATTN_ERR_INVALID, "rope.scaling: original_max_position_embeddings must be > 0");
        double eff_base = base;
        if (r->scaling == ATTN_ROPE_DYNAMIC) {
            const int64_t orig = r->original_max_positions ? r->original_max_positions : r->max_positions;
            if (orig <= 0)
                return fail(ATTN_ERR_INVALID, "rope.scaling: dynamic needs original_max_position_embeddings");
            if (rd <= 2) return fail(ATTN_ERR_INVALID, "rope.rotaryDim: dynamic scaling needs more than 2");
            if (seq_len > orig)
                eff_base = base * pow(r->factor * (double)seq_len / (double)orig - (r->factor - 1.0),
                                      (double)rd / ((double)rd - 2.0));
        }
        double lo_f = 1.0, hi_f = 4.0;
        if (r->scaling == ATTN_ROPE_LLAMA3) {
            lo_f = r->low_freq_factor ? r->low_freq_factor : 1.0;
            hi_f = r->high_freq_factor ? r->high_freq_factor : 4.0;
            if (!(lo_f > 0.0 && hi_f > lo_f))
                return fail(ATTN_ERR_INVALID, "rope.scaling: llama3 needs 0 < low_freq_factor < high_freq_factor");
        }
        const double* ext = nullptr;
        if (r->scaling == ATTN_ROPE_LONGROPE) {
            ext = seq_len > r->original_max_positions ? r->long_factor : r->short_factor;
            if (!ext) return fail(ATTN_ERR_INVALID, "rope.scaling: longrope needs short_factor and long_factor");
            for (int64_t i = 0; i < half; ++i)
                if (!(isfinite(ext[i]) && ext[i] > 0.0))
                    return fail(ATTN_ERR_INVALID, "rope.scaling: longrope factor %lld must be > 0", (long long)i);
        }
        // YaRN's ramp ends: the pair index at which the number of turns over
        // the original context equals beta_fast (resp. beta_slow).
        double ylo = 0.0, yhi = 0.0;
        if (r->scaling == ATTN_ROPE_YARN) {
            const double bf = r->beta_fast ? r->beta_fast : 32.0, bs = r->beta_slow ? r->beta_slow : 1.0;
            if (!(bf > 0.0 && bs > 0.0)) return fail(ATTN_ERR_INVALID, "rope.scaling: yarn betas must be > 0");
            const double orig = (double)r->original_max_positions;
            ylo = (double)rd * log(orig / (bf * 2.0 * M_PI)) / (2.0 * log(base));
            yhi = (double)rd * log(orig / (bs * 2.0 * M_PI)) / (2.0 * log(base));
            if (r->truncate) {
                ylo = floor(ylo);
                yhi = ceil(yhi);
            }
            if (ylo < 0.0) ylo = 0.0;
            if (yhi > (double)(rd - 1)) yhi = (double)(rd - 1);
            if (ylo == yhi) yhi += 0.001;
        }
        for (int64_t i = 0; i < half; ++i) {
            const double th = rope_theta(eff_base, i, rd);
            double f = th;
            switch (r->scaling) {
                case ATTN_ROPE_LINEAR: f = th / r->factor; break;
                case ATTN_ROPE_LLAMA3: f = rope_llama3(th, r, lo_f, hi_f); break;
                case ATTN_ROPE_YARN: {
                    double ramp = ((double)i - ylo) / (yhi - ylo);
                    ramp = ramp < 0.0 ? 0.0 : (ramp > 1.0 ? 1.0 : ramp);
                    f = th * (1.0 - ramp) + (th / r->factor) * ramp;
                    break;
                }
                case ATTN_ROPE_LONGROPE: f = th / ext[i]; break;
                default: break;
            }
            a.inv_freq[i] = (float)f;
        }
        if (r->scaling == ATTN_ROPE_YARN) {
            af = (r->mscale != 0.0 && r->mscale_all_dim != 0.0)
                     ? yarn_mscale(r->factor, r->mscale) / yarn_mscale(r->factor, r->mscale_all_dim)
                     : yarn_mscale(r->factor, 1.0);
        }
        if (r->scaling == ATTN_ROPE_LONGROPE) {
            double f = r->factor;
            if (f == 0.0) {
                if (r->max_positions <= 0 && !r->has_attention_factor && r->scaling_attention_factor == 0.0)
                    return fail(ATTN_ERR_INVALID, "rope.scaling: longrope needs factor or max_position_embeddings");
                f = (double)r->max_positions / (double)r->original_max_positions;
            }
            af = f > 1.0 ? sqrt(1.0 + log(f) / log((double)r->original_max_positions)) : 1.0;
        }
    }
    if (r->scaling_attention_factor != 0.0) af = r->scaling_attention_factor;
    if (r->has_attention_factor) af = (double)r->attention_factor;
    a.af = (float)af;
    return ok();
}


// Resolved view of attn_params.
struct Resolved {
    int64_t T, S, H, G, D, Dv, P0, window;
    bool causal;
    int bias_kind;
    attn::Epilogue ep;
    attn::RopeArgs rope;  // q_rope, resolved (rope.on = 0 without one)
};

int resolve(const attn_params* p, Resolved* r) {
    if (!p) return fail(ATTN_ERR_INVALID, "params: NULL pointer");
    if (p->T < 0) return fail(ATTN_ERR_INVALID, "T: must be >= 0 (got %lld)", (long long)p->T);
    if (p->S < 0) return fail(ATTN_ERR_INVALID, "S: must be >= 0 (got %lld)", (long long)p->S);
    if (p->heads <= 0 || p->heads > kMaxDim)
        return fail(ATTN_ERR_INVALID, "heads: must be in 1..%lld (got %lld)", (long long)kMaxDim,
                    (long long)p->heads);
    if (p->kv_heads < 0 || p->kv_heads > p->heads)
        return fail(ATTN_ERR_INVALID, "kvHeads: must be in 1..heads or 0 for absent (got %lld)",
                    (long long)p->kv_heads);
    const int64_t G = p->kv_heads ? p->kv_heads : p->heads;
    if (p->heads % G)
        return fail(ATTN_ERR_INVALID, "kvHeads: heads (%lld) is not a multiple of kvHeads (%lld)",
                    (long long)p->heads, (long long)G);
    if (p->head_dim <= 0 || p->head_dim > kMaxDim)
        return fail(ATTN_ERR_INVALID, "headDim: must be in 1..%lld (got %lld)", (long long)kMaxDim,
                    (long long)p->head_dim);
    if (p->v_head_dim < 0 || p->v_head_dim > kMaxDim)
        return fail(ATTN_ERR_INVALID, "vHeadDim: must be in 1..%lld or 0 for absent (got %lld)",
                    (long long)kMaxDim, (long long)p->v_head_dim);
    if (p->causal != 0 && p->causal != 1)
        return fail(ATTN_ERR_INVALID, "causal: must be 0 or 1 (got %d)", p->causal);
    if (p->pos_offset < 0)
        return fail(ATTN_ERR_INVALID, "posOffset: must be >= 0 (got %lld)", (long long)p->pos_offset);
    if (p->has_scale != 0 && p->has_scale != 1)
        return fail(ATTN_ERR_INVALID, "scale: has_scale must be 0 or 1 (got %d)", p->has_scale);
    if (p->has_scale && !isfinite(p->scale))
        return fail(ATTN_ERR_INVALID, "scale: must be finite");
    if (!(p->softcap >= 0.0f) || !isfinite(p->softcap))
        return fail(ATTN_ERR_INVALID, "softcap: must be finite and >= 0 (0 = off)");
    if (p->window < 0)
        return fail(ATTN_ERR_INVALID, "window: must be >= 0 (0 = off; got %lld)", (long long)p->window);
    if (p->sinks < 0)
        return fail(ATTN_ERR_INVALID, "sinks: must be >= 0 (0 = none; got %lld)", (long long)p->sinks);
    if (p->bias_kind < ATTN_BIAS_NONE || p->bias_kind > ATTN_BIAS_HTS)
        return fail(ATTN_ERR_INVALID, "bias: bias_kind must be 0, 1 ([T,S]) or 2 ([heads,T,S])");
    if (p->alibi < ATTN_ALIBI_NONE || p->alibi > ATTN_ALIBI_EXPLICIT)
        return fail(ATTN_ERR_INVALID, "alibi: mode must be 0..3 (got %d)", p->alibi);
    if (p->alibi == ATTN_ALIBI_MPT && !(isfinite(p->alibi_max) && p->alibi_max > 0.0f))
        return fail(ATTN_ERR_INVALID, "alibiMax: must be finite and > 0");
    if (p->alibi == ATTN_ALIBI_EXPLICIT && !p->alibi_slopes)
        return fail(ATTN_ERR_INVALID, "alibiSlopes: NULL pointer");
    if (p->alibi != ATTN_ALIBI_NONE && p->heads > ATTN_ALIBI_MAX_HEADS)
        return fail(ATTN_ERR_UNSUPPORTED, "attention.alibi: at most %d heads (got %lld)",
                    ATTN_ALIBI_MAX_HEADS, (long long)p->heads);

    Resolved& o = *r;
    o.T = p->T;
    o.S = p->S;
    o.H = p->heads;
    o.G = G;
    o.D = p->head_dim;
    o.Dv = p->v_head_dim ? p->v_head_dim : p->head_dim;
    o.P0 = p->pos_offset;
    o.window = p->window;
    o.causal = p->causal != 0;
    // A window that cannot hide any key of this call is switched off: causal
    // rows see s > pos - window, which excludes nothing once window > the
    // last position; non-causal rows see |pos - s| <= window, which excludes
    // nothing once window >= the largest distance to a key. (This also keeps
    // every sum of a position and the window that the kernels form below 2^31.)
    if (o.window > 0) {
        const int64_t last = o.P0 + (o.T > 0 ? o.T - 1 : 0);
        const int64_t reach = o.causal ? last + 1 : (last > o.S - 1 - o.P0 ? last : o.S - 1 - o.P0);
        if (o.window >= reach) o.window = 0;
    }
    o.bias_kind = p->bias_kind;
    // Sizes of every tensor must stay far below 2^62 bytes.
    const double elems = (double)o.T * o.H * (double)(o.D > o.Dv ? o.D : o.Dv) +
                         (double)o.S * o.G * (double)(o.D + o.Dv) +
                         (o.bias_kind ? (double)o.H * o.T * o.S : 0.0);
    if (elems > 1e17) return fail(ATTN_ERR_INVALID, "sizes: tensors too large");
    // Positions (query rows at posOffset + t, key rows at s) are kept in 32 bits.
    if (o.S > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED, "S: more than 2^31-1 key rows");
    if (o.P0 > INT32_MAX || o.T > INT32_MAX - o.P0)
        return fail(ATTN_ERR_UNSUPPORTED, "posOffset: query positions past 2^31-1");

    attn::Epilogue& e = o.ep;
    memset(&e, 0, sizeof e);
    e.scale = p->has_scale ? p->scale : (float)(1.0 / sqrt((double)o.D));
    e.softcap = p->softcap;
    e.inv_softcap = p->softcap > 0.0f ? (float)(1.0 / (double)p->softcap) : 0.0f;
    e.causal = o.causal;
    e.bias_kind = o.bias_kind;
    e.pos_offset = (int32_t)o.P0;
    // A window that is still on is below the largest position or distance,
    // so it is below 2^31.
    e.window = (int32_t)o.window;
    // Sinks only matter beside a window; keys past S do not exist.
    e.sinks = o.window > 0 ? (int32_t)(p->sinks < o.S ? p->sinks : o.S) : 0;
    e.has_alibi = p->alibi != ATTN_ALIBI_NONE;
    if (p->alibi == ATTN_ALIBI_BLOOM) slopes_bloom(o.H, e.slopes);
    if (p->alibi == ATTN_ALIBI_MPT) slopes_mpt(o.H, (double)p->alibi_max, e.slopes);
    if (p->alibi == ATTN_ALIBI_EXPLICIT) {
        for (int64_t h = 0; h < o.H; ++h) {
            if (!isfinite(p->alibi_slopes[h]))
                return fail(ATTN_ERR_INVALID, "alibiSlopes: entry %lld is not finite", (long long)h);
            e.slopes[h] = p->alibi_slopes[h];
        }
    }
    if (p->pb_weight) {
        // Bucketed relative position bias: thresholds -> a bucket per distance.
        if (!p->pb_buckets) return fail(ATTN_ERR_INVALID, "position_bias.buckets: NULL pointer");
        if (p->pb_n < 1 || p->pb_n > ATTN_PB_MAX_BUCKETS)
            return fail(p->pb_n < 1 ? ATTN_ERR_INVALID : ATTN_ERR_UNSUPPORTED,
                        "position_bias.buckets: 1..%d thresholds supported (got %lld)", ATTN_PB_MAX_BUCKETS,
                        (long long)p->pb_n);
        if (p->pb_bidirectional != 0 && p->pb_bidirectional != 1)
            return fail(ATTN_ERR_INVALID, "position_bias.bidirectional: must be 0 or 1");
        if (p->pb_buckets[0] != 0)
            return fail(ATTN_ERR_INVALID, "position_bias.buckets: the first threshold must be 0");
        for (int64_t i = 1; i < p->pb_n; ++i)
            if (p->pb_buckets[i] <= p->pb_buckets[i - 1])
                return fail(ATTN_ERR_INVALID, "position_bias.buckets: thresholds must ascend (entry %lld)",
                            (long long)i);
        const int64_t dt = p->pb_buckets[p->pb_n - 1];
        if (dt > ATTN_PB_MAX_DIST)
            return fail(ATTN_ERR_UNSUPPORTED, "position_bias.buckets: thresholds past %d", ATTN_PB_MAX_DIST);
        e.pb_weight = p->pb_weight;
        e.pb_n = (int32_t)p->pb_n;
        e.pb_bidir = p->pb_bidirectional;
        e.pb_dt = (int32_t)dt;
        e.pb_heads = (int32_t)o.H;
        int64_t b = 0;
        for (int64_t d = 0; d < dt; ++d) {
            while (b + 1 < p->pb_n && p->pb_buckets[b + 1] <= d) ++b;
            e.pb_bucket[d] = (uint8_t)b;
        }
    } else if (p->pb_buckets || p->pb_n) {
        return fail(ATTN_ERR_INVALID, "position_bias.weight: NULL pointer with buckets given");
    }
    if (p->rel_k) {
        if (p->rel_max < 0) return fail(ATTN_ERR_INVALID, "relative_kv.max_distance: must be >= 0");
        if (p->rel_max > kRelMaxDistance)
            return fail(ATTN_ERR_UNSUPPORTED, "relative_kv.max_distance: at most %lld (got %lld)",
                        (long long)kRelMaxDistance, (long long)p->rel_max);
        e.rel_k = p->rel_k;
        e.rel_v = p->rel_v;
        e.rel_max = (int32_t)p->rel_max;
    } else if (p->rel_v) {
        return fail(ATTN_ERR_INVALID, "relative_kv.key: NULL pointer with a value table given");
    }
    memset(&o.rope, 0, sizeof o.rope);
    if (p->q_rope) {
        attn_rope_params qr = *p->q_rope;
        if (qr.head_dim != 0 && qr.head_dim != o.D)
            return fail(ATTN_ERR_INVALID, "q_rope.headDim: must be 0 or headDim (%lld), got %lld",
                        (long long)o.D, (long long)qr.head_dim);
        qr.head_dim = o.D;
        if (qr.offset < 0 || qr.offset > INT32_MAX)
            return fail(ATTN_ERR_INVALID, "rope.offset: must be in 0..2^31-1 (got %lld)", (long long)qr.offset);
        const int rc = rope_resolve(&qr, qr.offset + o.T, &o.rope);
        if (rc) return rc;
    }
    return ok();
}

// Keys any query row can see (op `attention`, params causal and window).
// Keys [lo, hi) that query rows at positions first .. last can see.
attn::KeyRange key_range_rows(const Resolved& r, int64_t first, int64_t last) {
    attn::KeyRange kr{0, r.S};
    if (r.causal) {
        kr.hi = last + 1 < r.S ? last + 1 : r.S;
        if (r.window > 0) kr.lo = first - r.window + 1 > 0 ? first - r.window + 1 : 0;
    } else if (r.window > 0) {
        kr.lo = first - r.window > 0 ? first - r.window : 0;
        kr.hi = last + r.window + 1 < r.S ? last + r.window + 1 : r.S;
    }
    if (kr.lo > kr.hi) kr.lo = kr.hi;
    return kr;
}

attn::KeyRange key_range(const Resolved& r) { return key_range_rows(r, r.P0, r.P0 + r.T - 1); }

// Whether every query row sees every key of kr (same rules as key_range).
bool range_all_visible(const Resolved& r, const attn::KeyRange& kr) {
    if (kr.hi <= kr.lo) return true;
    const int64_t first = r.P0, last = r.P0 + r.T - 1;
    if (r.causal) return kr.hi - 1 <= first && (r.window == 0 || kr.lo > last - r.window);
    if (r.window == 0) return true;
    return last - kr.lo <= r.window && kr.hi - 1 - first <= r.window;
}

int next_pow2_nq(int64_t n) {
    int q = 1;
    while (q < n) q *= 2;
    return q;
}

struct Plan {
    int path;
    attn::DecodePlan decode;
    attn::PrefillPlan prefill;
    size_t workspace;  // bytes this plan's launches need
    size_t reserve;    // bytes attn_workspace_size reports: enough for this call made
                       // through attn_forward or attn_forward_append
    bool fused;        // the decode launch also appends the call's new rows
};

// Cache rows [lo, hi) that an attn_forward_append call writes.
struct AppendRows {
    int64_t lo, hi;
};

// With `app`, the plan takes the appended rows into the decode launch where
// it can (plan->fused); otherwise they are left to a separate copy.
int make_plan(const Resolved& r, Plan* plan, const AppendRows* app = nullptr) {
    memset(plan, 0, sizeof *plan);
    plan->decode.splits = 1;
    if (r.T == 0) {
        plan->path = ATTN_PATH_EMPTY;
        return ok();
    }
    const attn::KeyRange kr = key_range(r);
    // Attention sinks below the window range: keys every row sees.
    const int64_t sink_hi = r.ep.sinks < kr.lo ? r.ep.sinks : kr.lo;
    if (r.S == 0 || (kr.hi <= kr.lo && sink_hi == 0)) {
        plan->path = ATTN_PATH_ZERO;
        return ok();
    }
    const int64_t hpg = r.H / r.G;
    const int64_t nrows = r.T * hpg;
    // Two decode kernels: decode_split (rows in registers, VALU arithmetic)
    // and decode_mfma (matrix cores, up to 16 or 32 rows, no
    // relative-position terms). The automatic choice takes decode_mfma for
    // groups wider than kDecodeMfmaFrom rows, where decode_split's work per key
    // (which grows with the rows) would set the pace.
    const bool valu_ok = nrows <= 16 && attn::decode_supported((int)r.D, (int)r.Dv, next_pow2_nq(nrows));
    const bool mfma_ok = g_opt_decode_mfma >= 0 && !r.ep.pb_weight && !r.ep.rel_k &&
                         nrows <= attn::decode_mfma_max_rows((int)r.D, (int)r.Dv);
    const bool use_mfma = mfma_ok && (g_opt_decode_mfma > 0 || !valu_ok || nrows >= kDecodeMfmaFrom);
    const bool dec_ok = valu_ok || mfma_ok;
    // Relative key/value embeddings: the 32x32x2 prefill kernel holds them up
    // to headDim + vHeadDim = 256; wider heads take the generic kernel.
    const bool pre_ok = attn::prefill_supported((int)r.D, (int)r.Dv) &&
                        (!r.ep.rel_k || attn::prefill_rel_supported((int)r.D, (int)r.Dv));
    int path;
    if (g_opt_force_path) {
        path = (int)g_opt_force_path;
        if ((path == ATTN_PATH_DECODE && !dec_ok) || (path == ATTN_PATH_PREFILL && !pre_ok))
            return fail(ATTN_ERR_UNSUPPORTED, "force_path: path %d cannot serve this shape", path);
        if (path != ATTN_PATH_DECODE && path != ATTN_PATH_PREFILL && path != ATTN_PATH_GENERIC)
            return fail(ATTN_ERR_INVALID, "force_path: unknown path %d", path);
    } else if (dec_ok) {
        path = ATTN_PATH_DECODE;
    } else if (pre_ok) {
        path = ATTN_PATH_PREFILL;
    } else {
        path = ATTN_PATH_GENERIC;
    }
    if (path == ATTN_PATH_GENERIC && (r.D + r.Dv > 16000 || r.H > 65535))
        return fail(ATTN_ERR_UNSUPPORTED,
                    "headDim/vHeadDim: no kernel for headDim %lld with vHeadDim %lld and %lld heads",
                    (long long)r.D, (long long)r.Dv, (long long)r.H);
    plan->path = path;
    if (path == ATTN_PATH_DECODE) {
        attn::DecodePlan& d = plan->decode;
        d.nq = next_pow2_nq(nrows);
        d.mfma = use_mfma ? 1 : 0;
        d.depth = g_opt_decode_depth ? (int32_t)g_opt_decode_depth : kDecodeDepth;

        d.range = kr;
        // An appending call whose new rows end the key range, without
        // relative-position terms: the near split takes those rows, reading
        // them from the new-row buffers and storing them into the caches, and
        // `range` stops below them. The rows then need no copy beforehand.
        if (app && app->hi > app->lo && app->lo >= kr.lo && app->hi == kr.hi && !r.ep.pb_weight &&
            !r.ep.rel_k && app->hi - app->lo <= kDecodeMaxAppend) {
            d.near_lo = (int32_t)app->lo;
            d.near_hi = (int32_t)app->hi;
            d.range.hi = app->lo;
            plan->fused = true;
        }
        // Relative-position terms: on a causal call, keys within the tables'
        // reach of the first row (s > posOffset - reach) are looked up per
        // key; they get a split of their own, so that this slower per-key
        // work does not stretch a full-size chunk. The other splits see every
        // key at the tables' far end: per-row constants.
        if (r.causal && (r.ep.pb_weight || r.ep.rel_k) && kr.hi > kr.lo) {
            const int64_t reach_pb = r.ep.pb_weight ? r.ep.pb_dt : 0, reach_rel = r.ep.rel_k ? r.ep.rel_max : 0;
            const int64_t reach = reach_pb > reach_rel ? reach_pb : reach_rel;
            int64_t near_lo = r.P0 - reach + 1;
            if (near_lo < kr.lo) near_lo = kr.lo;
            if (near_lo < kr.hi) {
                d.near_lo = (int32_t)near_lo;
                d.near_hi = (int32_t)kr.hi;
                d.range.hi = near_lo;
            }
        }
        const bool near = d.near_hi > d.near_lo;
        const int64_t n = d.range.hi > d.range.lo ? d.range.hi - d.range.lo : 0;
        // Chunks are sized for the range with any appended rows still in it,
        // so an appending call never has more range splits than the same
        // call without the append (the workspace attn_workspace_size reports
        // holds one split more, for the append split).
        const int64_t np = plan->fused ? kr.hi - d.range.lo : n;
        int64_t splits = g_opt_decode_splits;
        if (splits <= 0) {
            // As many workgroups as the chip holds at once, near and sink
            // splits included, and no more: a few workgroups past that
            // would run as a second wave and nearly double the time.
            // (The split of appended rows is short, and at one batch per
            // lane every instance it runs in holds at least 3 workgroups per
            // CU, one more than planned: it goes beside the full set.)
            // (decode_mfma holds only 2 workgroups per CU in most instances:
            // there the append split counts like any other.)
            const bool light = plan->fused && !d.mfma && d.depth == 1;
            const int64_t extra = (near && !light ? 1 : 0) + (sink_hi > 0 ? 1 : 0);
            // decode_mfma with rows of 256 or more K and V floats (16 or more
            // float4 loads per lane per tile) plans one workgroup per CU:
            // the kernel is as fast with half the loads in flight, and the
            // combine merges half the splits (64 heads over 8 KV heads and
            // 32768 keys: call 50.4 against 51.1 us; 28 over 4: 30.0 against
            // 31.9; 32 over 1: 27.2 against 42.2). With 64-wide heads two per
            // CU stay faster (55.2 against 59.2 us).
            const int64_t per_cu = g_opt_decode_wgs ? g_opt_decode_wgs
                                   : d.mfma && r.D + r.Dv >= 256 ? 1
                                                                 : kDecodeWgPerCU;
            const int64_t target = (int64_t)kCUs * per_cu / r.G - extra;
            const int64_t most = (np + kDecodeMinKeys - 1) / kDecodeMinKeys;
            splits = target < most ? target : most;
        }
        if (splits < 1) splits = 1;
        if (splits > kDecodeMaxSplits - 2) splits = kDecodeMaxSplits - 2;
        // Chunks of a whole number of 64-key steps where that keeps 15/16 of
        // the splits, else of finer steps (down to a 2-row batch): over a
        // short range, rounding up to 64 keys could halve the split count.
        int64_t chunk = kDecodeChunkAlign;
        if (np > 0) {
            const int64_t per = (np + splits - 1) / splits;
            for (const int64_t a : {kDecodeChunkAlign, (int64_t)32, (int64_t)16, (int64_t)2}) {
                chunk = (per + a - 1) / a * a;
                if ((np + chunk - 1) / chunk * 16 >= splits * 15) break;
            }
        }
        // The kernel addresses a chunk with 32-bit offsets from its first row.
        const int64_t row_floats = r.G * (r.D > r.Dv ? r.D : r.Dv);
        const int64_t max_chunk = (INT32_MAX - row_floats) / row_floats / kDecodeChunkAlign * kDecodeChunkAlign;
        if (max_chunk < kDecodeChunkAlign || (n + max_chunk - 1) / max_chunk > kDecodeMaxSplits - 2 ||
            sink_hi > max_chunk || (near && d.near_hi - d.near_lo > max_chunk))
            return fail(ATTN_ERR_UNSUPPORTED, "S: key range too long for the decode path at this width");
        if (chunk > max_chunk) chunk = max_chunk;
        d.chunk = chunk;
        // Splits start their chunk at one of 8 phases (split i at (5 i mod 8)
        // eighths): chunks start at aligned addresses, and walking them in
        // lockstep from the same phase loads the same memory channels at once.
        // Measured on the latent-shaped decode: 30.5 -> 28.9 us.
        d.rotate = (int32_t)(g_opt_decode_rotate ? g_opt_decode_rotate : chunk * 5 / 8);
        d.main_splits = (int32_t)((n + chunk - 1) / chunk);
        // Where every row sees every key of the range, the splits can take
        // interleaved blocks of it instead of a chunk each (same keys per
        // split, fixed at planning, so results do not depend on timing):
        // all splits then stream through the same stretch of memory together.
        // Measured on decode shapes from 8k to 128k keys: blocks of 256 rows
        // beat chunks where a chunk is 1024 keys or more (Llama-shaped
        // 128k-key decode 175-195 -> 166-176 us), and are no better below.
        // decode_mfma takes blocks of 512 rows: against 256, 70B-shaped
        // (64 heads over 8) 32768 keys 47.2 -> 46.5 us, 64-wide heads over
        // 65536 keys 49.5 -> 47.3, Qwen2-shaped (28 over 4) 131072 keys
        // 90.3 -> 84.9; decode_split measured the same with either.
        // Automatic blocks never lengthen the longest split.
        int64_t block = g_opt_decode_block;
        if (block == 0) {
            block = -1;
            const int64_t widest = d.mfma ? 2 * kDecodeBlock : kDecodeBlock;
            for (int64_t b = widest; b >= 64 && chunk >= 4 * kDecodeBlock; b /= 2) {
                if ((n + b - 1) / b <= d.main_splits * (chunk / b)) {
                    block = b;
                    break;
                }
            }
        }
        if (block > 0 && n > 0 && range_all_visible(r, d.range) && n <= (INT32_MAX - row_floats) / row_floats) {
            const int64_t nblocks = (n + block - 1) / block;
            d.block = (int32_t)block;
            if (d.main_splits > nblocks) d.main_splits = (int32_t)nblocks;
            d.rotate = 0;
        }
        // The near keys, then the sink keys below the window, get a split of
        // their own each (after the splits of `range`).
        d.sink_hi = (int32_t)sink_hi;
        d.splits = d.main_splits + (near ? 1 : 0) + (sink_hi > 0 ? 1 : 0);
        const size_t per_split = sizeof(float) * (size_t)(r.T * r.H) * (size_t)(r.Dv + 2);
        if (d.splits > 1) plan->workspace = per_split * (size_t)d.splits;
        // The same call made through attn_forward_append may add the split of
        // appended rows (its range loses those rows, so it has no more of
        // the others).
        const int32_t most_splits = d.splits + (!near && !r.ep.pb_weight && !r.ep.rel_k ? 1 : 0);
        plan->reserve = most_splits > 1 ? per_split * (size_t)most_splits : 0;
        if (plan->workspace > plan->reserve) plan->reserve = plan->workspace;
    }
    if (path == ATTN_PATH_PREFILL) {
        // Four waves of 32 query rows; heads of a KV group side by side
        // (up to 4), the rest of the workgroup's waves on further query rows.
        attn::PrefillPlan& pp = plan->prefill;
        // Heads of one KV group side by side in a workgroup; its other waves
        // on further query blocks. Wide heads take the 16-row-wave variant.
        pp.variant = r.ep.rel_k ? 32 : g_opt_prefill_variant ? (int32_t)g_opt_prefill_variant : (r.D + r.Dv > 256 ? 16 : 32);
        const int64_t waves = pp.variant == 16 ? 8 : 4, rows_per_wave = pp.variant == 16 ? 16 : 32;
        int64_t nh = 1;
        while (nh * 2 <= waves && hpg % (nh * 2) == 0) nh *= 2;
        pp.nh = (int32_t)nh;
        pp.tile_q = (int32_t)(waves / nh * rows_per_wave);
        const int64_t qblocks = (r.T + pp.tile_q - 1) / pp.tile_q;
        const int64_t nwg = qblocks * r.G * (hpg / nh);
        if (nwg > INT32_MAX / kPrefillMaxSplits)
            return fail(ATTN_ERR_UNSUPPORTED, "T: too many query rows for the prefill grid");
        pp.qblocks = (int32_t)qblocks;
        // Too few workgroups to fill the chip: split each one's key range.
        // Relative embeddings at widths past 64/64: the tiles beyond the
        // tables' reach go to a launch of their own, on an instance without
        // the band code (as many workgroups per CU as the epilogue instance),
        // and the band tiles to a second launch (one part per workgroup).
        pp.rel_band = r.ep.rel_k && r.D + r.Dv > 128 ? 1 : 0;
        const bool rel_occupancy = r.ep.rel_k != nullptr && !pp.rel_band;
        if (pp.rel_band) {
            // The band launch runs one workgroup per CU: split its tiles
            // into parts where the grid alone would leave CUs idle, keeping
            // two or more band tiles per part (a causal row block has about
            // (max_distance + rows) / 32 of them).
            const int64_t band_slots = (int64_t)kCUs * attn::prefill_wgs_per_cu(pp.variant, (int)r.D, (int)r.Dv, true);
            int64_t kb = nwg >= band_slots ? 1 : (band_slots + nwg - 1) / nwg;
            const int64_t band_tiles = (r.ep.rel_max + pp.tile_q) / 32;
            if (kb > band_tiles / 2) kb = band_tiles / 2;
            if (kb < 1) kb = 1;
            if (kb > kPrefillMaxSplits) kb = kPrefillMaxSplits;
            pp.rel_band = (int32_t)kb;
        }
        const int64_t slots = (int64_t)kCUs * attn::prefill_wgs_per_cu(pp.variant, (int)r.D, (int)r.Dv, rel_occupancy);
        const int64_t tiles = (kr.hi > kr.lo ? (kr.hi - kr.lo + 31) / 32 : 0) + (sink_hi + 31) / 32;
        // Query blocks with unequal key ranges (causal calls, where block i
        // sees about i + 1 tiles): a grid of one wave then lasts as long as
        // its heaviest block while most slots idle, so such grids are split
        // to at least 1.5 waves, which the heaviest-first order balances.
        // Measured (Llama-shaped heads, one box): 2048 x 2048 causal 409 ->
        // 330 us per call (2 parts), 1024 x 1024 128 -> 120 us (3 parts);
        // 16 heads of 64 at 4096 x 4096 564 -> 374 us (2 parts); grids of 1.5
        // waves or more (3072, 4096 rows at 128) stay whole, as they were
        // fastest so.
        int64_t tile_max = 0, tile_sum = 0;
        for (int64_t qb = 0; qb < qblocks; ++qb) {
            const int64_t t0 = qb * pp.tile_q, t1 = t0 + pp.tile_q < r.T ? t0 + pp.tile_q : r.T;
            const attn::KeyRange q = key_range_rows(r, r.P0 + t0, r.P0 + t1 - 1);
            const int64_t n = (q.hi > q.lo ? (q.hi - q.lo + 31) / 32 : 0) + (sink_hi + 31) / 32;
            if (n > tile_max) tile_max = n;
            tile_sum += n;
        }
        const bool uneven = tile_max * qblocks * 4 > tile_sum * 5;  // heaviest block > 1.25 x the mean
        const int64_t want = uneven ? slots + slots / 2 : slots;
        int64_t ks = g_opt_prefill_splits;
        if (ks <= 0) {
            ks = nwg >= want ? 1 : (want + nwg - 1) / nwg;
            if (uneven) {
                // Causal grids with fewer query blocks per head than an XCD
                // runs workgroups at once (workgroups of 128 rows of one
                // head: MHA, or 5 or 7 heads per KV head): split them to
                // that many, one part more where each workgroup holds one of
                // several heads of a KV head (5 or 7 per KV head), up to 4
                // parts. Measured (one box,
                // per call): 32 heads of 128, 2048 x 2048 442 -> 372 us (4
                // parts), 4096 x 4096 1603 -> 1175 us (2 parts), although the
                // parts fetch more from HBM (a 4096-row call 0.24 -> 0.76 GB);
                // 8192 rows (64 blocks per head) stay whole at 81%. 40 heads
                // over 8, 4096 rows: 1861 us whole, 1630 in 2 parts, 1506 in
                // 3; 28 over 4: 1590 whole, 1157 in 2, 1124 in 4, and at 8192
                // rows 4287 whole, 4168 in 2; 64 over 8 (4 heads per
                // workgroup) stays whole (2 parts: 2048 rows 580 -> 624 us).
                const int64_t xcd_slots = slots / kXcdCount;
                int64_t kh = (xcd_slots + qblocks - 1) / qblocks + (nh == 1 && hpg > 1 ? 1 : 0);
                if (kh > 4) kh = 4;
                if (kh > ks) ks = kh;
            }
            const int64_t most = tiles / kPrefillMinTilesPerSplit;
            if (ks > most) ks = most;
        }
        if (ks < 1) ks = 1;
        if (ks > kPrefillMaxSplits) ks = kPrefillMaxSplits;
        pp.ksplit = (int32_t)ks;
        const int64_t kslots = ks + pp.rel_band;
        if (kslots > 1) plan->workspace = sizeof(float) * (size_t)(r.T * r.H) * (size_t)kslots * (size_t)(r.Dv + 2);
        plan->reserve = plan->workspace;
    }
    return ok();
}

// ---------------------------------------------------------------------------
// Kernel timing (attn_timing_enable / attn_timing_collect).
// ---------------------------------------------------------------------------
struct TimingRecord {
    const char* name;
    int slot;
};

struct Timing {
    std::mutex mu;
    bool on = false;
    bool created = false;
    std::vector<hipEvent_t> start, stop;
    std::vector<int> free_slots;
    std::vector<TimingRecord> records;
};

Timing& timing() {
    static Timing t;
    return t;
}

constexpr int kTimingSlots = 4096;

// Runs launch(L) with L carrying a pair of events from the pool when timing is
// on; the dispatch stamps them with the kernel's own start and end.
template <typename F>
hipError_t timed(const char* name, hipStream_t stream, F&& launch) {
    Timing& tm = timing();
    attn::Launch L{stream, nullptr, nullptr};
    if (!tm.on) return launch(L);
    int slot = -1;
    {
        std::lock_guard<std::mutex> lock(tm.mu);
        if (!tm.free_slots.empty()) {
            slot = tm.free_slots.back();
            tm.free_slots.pop_back();
        }
    }
    if (slot < 0) return launch(L);
    L.start = tm.start[slot];
    L.stop = tm.stop[slot];
    const hipError_t err = launch(L);
    std::lock_guard<std::mutex> lock(tm.mu);
    if (err == hipSuccess) tm.records.push_back({name, slot});
    else tm.free_slots.push_back(slot);
    return err;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || !an || !bn) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bn && y < x + an;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shared checks of attn_rope and attn_rope_cache_write: the row layout and
// the resolved table.
int rope_rows(const attn_rope_params* r, int64_t rows, int64_t width, attn::RopeArgs* a, int64_t* heads) {
    if (!r) return fail(ATTN_ERR_INVALID, "rope: NULL params");
    if (rows < 0) return fail(ATTN_ERR_INVALID, "rows: must be >= 0");
    if (width <= 0) return fail(ATTN_ERR_INVALID, "width: must be > 0");
    if (r->head_dim <= 0 || width % r->head_dim)
        return fail(ATTN_ERR_INVALID, "rope.headDim: the row width %lld is not a multiple of headDim %lld",
                    (long long)width, (long long)r->head_dim);
    if (width / r->head_dim > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED, "width: too many heads");
    if ((double)rows * (double)width > 1e17) return fail(ATTN_ERR_INVALID, "sizes: tensors too large");
    if (r->offset < 0 || r->offset > INT32_MAX)
        return fail(ATTN_ERR_INVALID, "rope.offset: must be in 0..2^31-1 (got %lld)", (long long)r->offset);
    *heads = width / r->head_dim;
    return rope_resolve(r, r->offset + rows, a);
}

// ---------------------------------------------------------------------------
// Latent (MLA) attention (the IR schema's op_mla_attention; read as
// DeepSeek-V2's multi-head latent attention, evaluated in absorbed form).
// ---------------------------------------------------------------------------
struct MlaResolved {
    int64_t T, S, H, R, N, P, Dv, P0, window, sinks;
    bool causal;
    float scale;
};

int mla_resolve(const attn_mla_params* p, MlaResolved* r) {
    if (!p) return fail(ATTN_ERR_INVALID, "params: NULL pointer");
    if (p->T < 0) return fail(ATTN_ERR_INVALID, "T: must be >= 0 (got %lld)", (long long)p->T);
    if (p->S < 0) return fail(ATTN_ERR_INVALID, "S: must be >= 0 (got %lld)", (long long)p->S);
    if (p->heads <= 0 || p->heads > kMaxDim)
        return fail(ATTN_ERR_INVALID, "heads: must be in 1..%lld (got %lld)", (long long)kMaxDim,
                    (long long)p->heads);
    if (p->kv_rank <= 0 || p->kv_rank > kMaxDim)
        return fail(ATTN_ERR_INVALID, "kv_rank: must be in 1..%lld (got %lld)", (long long)kMaxDim,
                    (long long)p->kv_rank);
    if (p->qk_nope <= 0 || p->qk_nope > kMaxDim)
        return fail(ATTN_ERR_INVALID, "qk_nope: must be in 1..%lld (got %lld)", (long long)kMaxDim,
                    (long long)p->qk_nope);
    if (p->qk_rope < 0 || p->qk_rope > kMaxDim)
        return fail(ATTN_ERR_INVALID, "qk_rope: must be in 0..%lld (got %lld)", (long long)kMaxDim,
                    (long long)p->qk_rope);
    if (p->v_head_dim <= 0 || p->v_head_dim > kMaxDim)
        return fail(ATTN_ERR_INVALID, "v_head_dim: must be in 1..%lld (got %lld)", (long long)kMaxDim,
                    (long long)p->v_head_dim);
    if (p->pos_offset < 0)
        return fail(ATTN_ERR_INVALID, "posOffset: must be >= 0 (got %lld)", (long long)p->pos_offset);
    if (p->window < 0) return fail(ATTN_ERR_INVALID, "window: must be >= 0 (0 = off; got %lld)", (long long)p->window);
    if (p->sinks < 0) return fail(ATTN_ERR_INVALID, "sinks: must be >= 0 (0 = none; got %lld)", (long long)p->sinks);
    if (p->has_scale && !isfinite(p->scale)) return fail(ATTN_ERR_INVALID, "scale: must be finite");
    MlaResolved o;
    o.T = p->T;
    o.S = p->S;
    o.H = p->heads;
    o.R = p->kv_rank;
    o.N = p->qk_nope;
    o.P = p->qk_rope;
    o.Dv = p->v_head_dim;
    o.P0 = p->pos_offset;
    o.causal = p->causal != 0;
    o.window = p->window;
    o.sinks = p->window > 0 ? (p->sinks < p->S ? p->sinks : p->S) : 0;
    o.scale = p->has_scale ? p->scale : (float)(1.0 / sqrt((double)(o.N + o.P)));
    if (o.S > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED, "S: more than 2^31-1 key rows");
    if (o.P0 > INT32_MAX || o.T > INT32_MAX - o.P0)
        return fail(ATTN_ERR_UNSUPPORTED, "posOffset: positions past 2^31-1");
    if (o.T * o.H > INT32_MAX / 2) return fail(ATTN_ERR_UNSUPPORTED, "T: too many (row, head) pairs");
    if (!attn::mla_fast_supported((int)o.R, (int)o.P) && 2 * o.R + o.P > kMlaGenericMaxFloats)
        return fail(ATTN_ERR_UNSUPPORTED, "kv_rank/qk_rope: no kernel for kv_rank %lld with qk_rope %lld",
                    (long long)o.R, (long long)o.P);
    *r = o;
    return ok();
}

struct MlaPlanFull {
    int path;  // ATTN_PATH_EMPTY, _ZERO or _MLA
    attn::MlaPlan plan;
    size_t q_abs_bytes;  // workspace: q_abs first, the split partials after it
    size_t part_bytes;   // then the split partials; then (slices > 0) the slice shares and counters
    size_t workspace;
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

int mla_make_plan(const MlaResolved& r, MlaPlanFull* out) {
    memset(out, 0, sizeof *out);
    out->plan.splits = 1;
    if (r.T == 0) {
        out->path = ATTN_PATH_EMPTY;
        return ok();
    }
    // Keys any query row can see: the attention op's rule over positions
    // P0 .. P0+T-1, and the sink keys below that range.
    Resolved kq{};
    kq.T = r.T;
    kq.S = r.S;
    kq.P0 = r.P0;
    kq.causal = r.causal;
    kq.window = r.window;
    const attn::KeyRange kr = key_range(kq);
    const int64_t sink_hi = r.sinks < kr.lo ? r.sinks : kr.lo;
    if (r.S == 0 || (kr.hi <= kr.lo && sink_hi == 0)) {
        out->path = ATTN_PATH_ZERO;
        return ok();
    }
    out->path = ATTN_PATH_MLA;
    attn::MlaPlan& pl = out->plan;
    pl.fast = attn::mla_fast_supported((int)r.R, (int)r.P) && !g_opt_mla_generic ? 1 : 0;
    pl.range = kr;
    const int64_t rows = r.T * r.H;
    pl.row_blocks = (int32_t)((rows + 15) / 16);
    // Two row blocks share each workgroup's key tiles when there are enough
    // blocks to keep the chip busy (one such workgroup fills a CU's LDS).
    pl.row_groups = g_opt_mla_row_groups ? (int32_t)g_opt_mla_row_groups : (pl.row_blocks >= 4 ? 2 : 1);
    // Combine workgroups of 16 outputs where 32-output ones would not fill the
    // chip (each still merges the row's splits; more of them pull at once):
    // V2-Lite-shaped decode 30.0 -> 29.1 us per call; on wider grids the
    // extra merges cost more (V3-shaped: 17.4 -> 25.7 us for the combine).
    pl.combine_out = g_opt_mla_combine_out ? (int32_t)g_opt_mla_combine_out
                     : rows * ((r.Dv + 31) / 32) < kCUs ? 16 : 32;
    const int64_t n = kr.hi > kr.lo ? kr.hi - kr.lo : 0;
    if (pl.fast) {
        if (pl.row_blocks > 65535) return fail(ATTN_ERR_UNSUPPORTED, "T: too many rows for the MLA grid");
        int64_t splits = g_opt_mla_splits;
        if (splits <= 0) {
            // Two workgroups per CU over all row blocks (one of two row
            // groups), chunks of >= 64 keys.
            // (Rounded down, the sink split included: workgroups past one
            // wave would run as a second.)
            const int64_t wg_rows = (pl.row_blocks + pl.row_groups - 1) / pl.row_groups;
            const int64_t target = (int64_t)kCUs * (3 - pl.row_groups) / wg_rows - (sink_hi > 0 ? 1 : 0);
            const int64_t most = (n + kMlaMinKeys - 1) / kMlaMinKeys;
            splits = target < most ? target : most;
        }
        if (splits < 1) splits = 1;
        if (splits > kMlaMaxSplits - 1) splits = kMlaMaxSplits - 1;
        int64_t chunk = n > 0 ? (n + splits - 1) / splits : kMlaChunkAlign;
        chunk = (chunk + kMlaChunkAlign - 1) / kMlaChunkAlign * kMlaChunkAlign;
        pl.chunk = chunk;
        pl.sink_hi = (int32_t)sink_hi;
        pl.splits = (int32_t)((n + chunk - 1) / chunk) + (sink_hi > 0 ? 1 : 0);
    } else {
        // One workgroup per row scans every key itself.
        pl.chunk = 0;
        pl.sink_hi = 0;
        pl.splits = 1;
    }
    // The merge by latent slices reads each split's accumulator once (the
    // per-output merge reads a row's partials once per group of outputs):
    // V3-shaped combine 16.1 against 17.4 us, V2-Lite-shaped the same 7.9.
    pl.slices = pl.fast && attn::mla_slices_supported((int)r.R, (int)r.Dv) && g_opt_mla_slices >= 0
                    ? (int32_t)(r.R / 64) : 0;
    out->q_abs_bytes = align256(sizeof(float) * (size_t)rows * (size_t)(r.R + r.P));
    out->part_bytes = align256(sizeof(float) * (size_t)rows * (size_t)pl.splits * (size_t)(r.R + 2));
    out->workspace = out->q_abs_bytes + out->part_bytes;
    if (pl.slices > 0)
        out->workspace += align256(sizeof(float) * (size_t)rows * (size_t)pl.slices * (size_t)r.Dv) +
                          sizeof(uint32_t) * (size_t)rows;
    return ok();
}

// The checks of op `cache_write` on one cache; *dst = the first row written
// (left NULL when rows == 0). `which` prefixes the messages ("" or "a: ").
int check_cache_write(const char* which, float* cache, int64_t max_rows, int64_t width, const float* values,
                      int64_t rows, int64_t offset, float** dst) {
    *dst = nullptr;
    if (max_rows < 0) return fail(ATTN_ERR_INVALID, "%smaxRows: must be >= 0", which);
    if (width <= 0) return fail(ATTN_ERR_INVALID, "%swidth: must be > 0", which);
    if (rows < 0) return fail(ATTN_ERR_INVALID, "rows: must be >= 0");
    if (offset < 0) return fail(ATTN_ERR_INVALID, "offset: must be >= 0 (got %lld)", (long long)offset);
    if (offset > max_rows || rows > max_rows - offset)
        return fail(ATTN_ERR_INVALID, "%soffset: rows %lld..%lld run past the cache's %lld rows", which,
                    (long long)offset, (long long)(offset + rows), (long long)max_rows);
    if ((double)max_rows * (double)width > 1e17) return fail(ATTN_ERR_INVALID, "%scache: too large", which);
    if (rows == 0) return ok();
    if (!cache) return fail(ATTN_ERR_INVALID, "%scache: NULL pointer", which);
    if (!values) return fail(ATTN_ERR_INVALID, "%svalues: NULL pointer", which);
    *dst = cache + offset * width;
    const size_t n = sizeof(float) * (size_t)(rows * width);
    if (overlaps(*dst, n, values, n)) return fail(ATTN_ERR_INVALID, "%svalues: overlap the rows being written", which);
    return ok();
}


// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "scratch: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ATTN_ERR_UNSUPPORTED, "scratch: device %d past the %d this library tracks", dev, kMaxDevices);
    if (stream) {
        // The stream must run on the current device: the address is that device's.
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess)
            return fail(ATTN_ERR_DEVICE, "scratch: hipStreamGetDevice: %s", hipGetErrorString(e));
        if ((int)sdev != dev)
            return fail(ATTN_ERR_INVALID, "stream: belongs to device %d, but device %d is current", (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(ATTN_ERR_DEVICE, "scratch: hipGetSymbolAddress: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ok();
}

// attn_forward's checks of the tensors and the workspace (`need` bytes) for
// a valid plan.
int check_forward_args(const attn_params* p, const Resolved& r, size_t need, const float* q, const float* k,
                       const float* v, const float* bias, const float* out, const void* workspace,
                       size_t workspace_bytes) {
    const size_t qn = sizeof(float) * (size_t)(r.T * r.H * r.D);
    const size_t kn = sizeof(float) * (size_t)(r.S * r.G * r.D);
    const size_t vn = sizeof(float) * (size_t)(r.S * r.G * r.Dv);
    const size_t on = sizeof(float) * (size_t)(r.T * r.H * r.Dv);
    const size_t bn = r.bias_kind == ATTN_BIAS_TS    ? sizeof(float) * (size_t)(r.T * r.S)
                      : r.bias_kind == ATTN_BIAS_HTS ? sizeof(float) * (size_t)(r.H * r.T * r.S)
                                                     : 0;
    if (!out) return fail(ATTN_ERR_INVALID, "out: NULL pointer");
    if (!q) return fail(ATTN_ERR_INVALID, "q: NULL pointer");
    if (r.S > 0 && (!k || !v)) return fail(ATTN_ERR_INVALID, "%s: NULL pointer", k ? "v" : "k");
    if (r.bias_kind && !bias) return fail(ATTN_ERR_INVALID, "bias: NULL pointer with bias_kind %d", r.bias_kind);
    if (!r.bias_kind && bias) return fail(ATTN_ERR_INVALID, "bias: pointer given with bias_kind 0");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(bias) || !aligned16(out))
        return fail(ATTN_ERR_INVALID, "q/k/v/bias/out: pointers must be 16-byte aligned");
    const size_t pbn = p->pb_weight ? sizeof(float) * (size_t)(p->pb_n * (p->pb_bidirectional ? 2 : 1) * r.H) : 0;
    if (overlaps(out, on, q, qn) || overlaps(out, on, k, kn) || overlaps(out, on, v, vn) ||
        overlaps(out, on, bias, bn) || overlaps(out, on, p->pb_weight, pbn) ||
        overlaps(out, on, p->rel_k, p->rel_k ? sizeof(float) * (size_t)((2 * p->rel_max + 1) * r.D) : 0) ||
        overlaps(out, on, p->rel_v, p->rel_v ? sizeof(float) * (size_t)((2 * p->rel_max + 1) * r.Dv) : 0))
        return fail(ATTN_ERR_INVALID, "out: overlaps an input");
    if (need) {
        if (!workspace || workspace_bytes < need)
            return fail(ATTN_ERR_INVALID, "workspace: %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (((uintptr_t)workspace & 255u) != 0)
            return fail(ATTN_ERR_INVALID, "workspace: must be 256-byte aligned");
        if (overlaps(workspace, need, out, on) || overlaps(workspace, need, q, qn) ||
            overlaps(workspace, need, k, kn) || overlaps(workspace, need, v, vn) ||
            overlaps(workspace, need, bias, bn))
            return fail(ATTN_ERR_INVALID, "workspace: overlaps a tensor");
    }
    return ok();
}

attn::Problem make_problem(const Resolved& r, const float* q, const float* k, const float* v, const float* bias,
                           float* out) {
    attn::Problem prob;
    prob.q = q;
    prob.k = k;
    prob.v = v;
    prob.bias = bias;
    prob.out = out;
    prob.T = r.T;
    prob.S = r.S;
    prob.H = (int32_t)r.H;
    prob.G = (int32_t)r.G;
    prob.D = (int32_t)r.D;
    prob.Dv = (int32_t)r.Dv;
    prob.ep = r.ep;
    prob.rope = r.rope;
    return prob;
}

// Launches a checked plan's kernels on stream s.
int run_plan(const Resolved& r, const Plan& plan, const attn::Problem& prob, void* workspace, hipStream_t s) {
    hipError_t err = hipSuccess;
    switch (plan.path) {
        case ATTN_PATH_EMPTY:
            return ok();
        case ATTN_PATH_ZERO:
            err = timed("zero_fill", s, [&](const attn::Launch& L) {
                return attn::launch_zero_fill(prob.out, r.T * r.H * r.Dv, L);
            });
            break;
        case ATTN_PATH_GENERIC:
            err = timed("generic", s, [&](const attn::Launch& L) { return attn::launch_generic(prob, L); });
            break;
        case ATTN_PATH_DECODE:
            if (plan.decode.mfma)
                err = timed("decode_mfma", s, [&](const attn::Launch& L) {
                    return attn::launch_decode_mfma(prob, plan.decode, (float*)workspace, L);
                });
            else
                err = timed("decode_split", s, [&](const attn::Launch& L) {
                    return attn::launch_decode_split(prob, plan.decode, (float*)workspace, L);
                });
            if (err == hipSuccess && plan.decode.splits > 1)
                err = timed("combine", s, [&](const attn::Launch& L) {
                    return attn::launch_decode_combine(prob, plan.decode, (const float*)workspace, L);
                });
            break;
        case ATTN_PATH_PREFILL:
            err = timed("prefill", s, [&](const attn::Launch& L) {
                return attn::launch_prefill(prob, plan.prefill, (float*)workspace, plan.prefill.rel_band ? 1 : 0, L);
            });
            if (err == hipSuccess && plan.prefill.rel_band)
                err = timed("prefill_band", s, [&](const attn::Launch& L) {
                    return attn::launch_prefill(prob, plan.prefill, (float*)workspace, 2, L);
                });
            if (err == hipSuccess && plan.prefill.ksplit + plan.prefill.rel_band > 1) {
                attn::DecodePlan merge{};
                merge.splits = plan.prefill.ksplit + plan.prefill.rel_band;
                err = timed("combine", s, [&](const attn::Launch& L) {
                    return attn::launch_decode_combine(prob, merge, (const float*)workspace, L);
                });
            }
            break;
        default:
            return fail(ATTN_ERR_INVALID, "internal: unknown path %d", plan.path);
    }
    if (err != hipSuccess) return fail(ATTN_ERR_DEVICE, "launch: %s", hipGetErrorString(err));
    return ok();
}

}  // namespace

extern "C" {

void attn_params_init(attn_params* p) {
    if (!p) return;
    memset(p, 0, sizeof *p);
    p->causal = 1;
}

int attn_validate(const attn_params* p) {
    Resolved r;
    int rc = resolve(p, &r);
    if (rc) return rc;
    Plan plan;
    return make_plan(r, &plan);
}

size_t attn_workspace_size(const attn_params* p) {
    Resolved r;
    if (resolve(p, &r)) return 0;
    Plan plan;
    if (make_plan(r, &plan)) return 0;
    return plan.reserve;
}

int attn_plan(const attn_params* p, attn_plan_info* info) {
    if (!info) return fail(ATTN_ERR_INVALID, "info: NULL pointer");
    Resolved r;
    int rc = resolve(p, &r);
    if (rc) return rc;
    Plan plan;
    rc = make_plan(r, &plan);
    if (rc) return rc;
    info->path = plan.path;
    info->splits = plan.path == ATTN_PATH_DECODE    ? plan.decode.splits
                   : plan.path == ATTN_PATH_PREFILL ? plan.prefill.ksplit + plan.prefill.rel_band
                                                    : 1;
    info->tile_q = plan.path == ATTN_PATH_PREFILL ? plan.prefill.tile_q : 0;
    info->variant = plan.path == ATTN_PATH_DECODE    ? plan.decode.mfma
                    : plan.path == ATTN_PATH_PREFILL ? plan.prefill.variant
                                                     : 0;
    return ok();
}

int attn_forward(const attn_params* p, const float* q, const float* k, const float* v,
                 const float* bias, float* out, void* workspace, size_t workspace_bytes,
                 void* stream) {
    Resolved r;
    int rc = resolve(p, &r);
    if (rc) return rc;
    Plan plan;
    rc = make_plan(r, &plan);
    if (rc) return rc;
    if (plan.path == ATTN_PATH_EMPTY) return ok();
    rc = check_forward_args(p, r, plan.workspace, q, k, v, bias, out, workspace, workspace_bytes);
    if (rc) return rc;
    return run_plan(r, plan, make_problem(r, q, k, v, bias, out), workspace, (hipStream_t)stream);
}

int attn_forward_noalloc(const attn_params* p, const float* q, const float* k, const float* v,
                         const float* bias, float* out, void* stream) {
    Resolved r;
    int rc = resolve(p, &r);
    if (rc) return rc;
    Plan plan;
    rc = make_plan(r, &plan);
    if (rc) return rc;
    if (plan.path == ATTN_PATH_EMPTY) return ok();
    if (plan.workspace > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_UNSUPPORTED,
                    "workspace: this call needs %zu bytes of split state, past the %zu-byte built-in scratch "
                    "(use attn_forward with a workspace)",
                    plan.workspace, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (plan.workspace) {
        rc = scratch_address((hipStream_t)stream, &ws);
        if (rc) return rc;
    }
    rc = check_forward_args(p, r, plan.workspace, q, k, v, bias, out, ws, ws ? (size_t)ATTN_NOALLOC_SCRATCH_BYTES : 0);
    if (rc) return rc;
    return run_plan(r, plan, make_problem(r, q, k, v, bias, out), ws, (hipStream_t)stream);
}

int attn_forward_append(const attn_params* p, const float* q, float* k, float* v, const float* k_new,
                        const float* v_new, int64_t rows, int64_t offset, const float* bias, float* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
    Resolved r;
    int rc = resolve(p, &r);
    if (rc) return rc;
    // The two cache_write ops: rows [offset, offset + rows) of the caches.
    float *dk = nullptr, *dv = nullptr;
    rc = check_cache_write("k: ", k, r.S, r.G * r.D, k_new, rows, offset, &dk);
    if (rc) return rc;
    rc = check_cache_write("v: ", v, r.S, r.G * r.Dv, v_new, rows, offset, &dv);
    if (rc) return rc;
    const size_t kw = sizeof(float) * (size_t)(rows * r.G * r.D), vw = sizeof(float) * (size_t)(rows * r.G * r.Dv);
    if (overlaps(dk, kw, dv, vw)) return fail(ATTN_ERR_INVALID, "v: rows written overlap the k rows written");
    if (overlaps(dk, kw, v_new, vw)) return fail(ATTN_ERR_INVALID, "v: values overlap the k rows written");
    if (overlaps(dv, vw, k_new, kw)) return fail(ATTN_ERR_INVALID, "k: values overlap the v rows written");
    Plan plan;
    // The fused decode reads the new rows as 16-byte vectors.
    const AppendRows app{offset, offset + rows};
    rc = make_plan(r, &plan, aligned16(k_new) && aligned16(v_new) ? &app : nullptr);
    if (rc) return rc;
    if (plan.fused) {
        // A fused plan never asks for more workspace than attn_workspace_size
        // reports; if one would, the call copies first instead.
        Plan plain;
        rc = make_plan(r, &plain);
        if (rc) return rc;
        if (plan.workspace > plain.reserve) plan = plain;
    }
    hipStream_t s = (hipStream_t)stream;
    if (plan.path != ATTN_PATH_EMPTY) {
        rc = check_forward_args(p, r, plan.workspace, q, k, v, bias, out, workspace, workspace_bytes);
        if (rc) return rc;
        // Nothing else the call reads or writes may lie in the rows written
        // (the attention may run while they are being written), and out and
        // the workspace may not hold the new rows.
        const size_t qn = sizeof(float) * (size_t)(r.T * r.H * r.D);
        const size_t on = sizeof(float) * (size_t)(r.T * r.H * r.Dv);
        const size_t bn = r.bias_kind == ATTN_BIAS_TS    ? sizeof(float) * (size_t)(r.T * r.S)
                          : r.bias_kind == ATTN_BIAS_HTS ? sizeof(float) * (size_t)(r.H * r.T * r.S)
                                                         : 0;
        if (overlaps(dk, kw, q, qn) || overlaps(dv, vw, q, qn))
            return fail(ATTN_ERR_INVALID, "q: overlaps the cache rows written");
        if (overlaps(dk, kw, bias, bn) || overlaps(dv, vw, bias, bn))
            return fail(ATTN_ERR_INVALID, "bias: overlaps the cache rows written");
        if (overlaps(out, on, k_new, kw) || overlaps(out, on, v_new, vw))
            return fail(ATTN_ERR_INVALID, "out: overlaps k_new or v_new");
        if (plan.workspace && (overlaps(workspace, plan.workspace, k_new, kw) ||
                               overlaps(workspace, plan.workspace, v_new, vw)))
            return fail(ATTN_ERR_INVALID, "workspace: overlaps k_new or v_new");
    }
    if (plan.fused) {
        plan.decode.k_new = k_new;
        plan.decode.v_new = v_new;
        plan.decode.k_cache = k;
        plan.decode.v_cache = v;
    } else if (rows > 0) {
        const hipError_t err = timed("cache_write", s, [&](const attn::Launch& L) {
            return attn::launch_cache_write_pair(dk, k_new, rows * r.G * r.D, dv, v_new, rows * r.G * r.Dv, L);
        });
        if (err != hipSuccess) return fail(ATTN_ERR_DEVICE, "launch: %s", hipGetErrorString(err));
    }
    if (plan.path == ATTN_PATH_EMPTY) return ok();
    return run_plan(r, plan, make_problem(r, q, k, v, bias, out), workspace, s);
}

int attn_cache_write(float* cache, int64_t max_rows, int64_t width, const float* values,
                     int64_t rows, int64_t offset, void* stream) {
    float* dst = nullptr;
    const int rc = check_cache_write("", cache, max_rows, width, values, rows, offset, &dst);
    if (rc || rows == 0) return rc;
    hipStream_t s = (hipStream_t)stream;
    const hipError_t err = timed("cache_write", s, [&](const attn::Launch& L) {
        return attn::launch_cache_write(dst, values, rows * width, L);
    });
    if (err != hipSuccess) return fail(ATTN_ERR_DEVICE, "launch: %s", hipGetErrorString(err));
    return ok();
}

int attn_cache_write2(float* cache_a, int64_t max_rows_a, int64_t width_a, const float* values_a,
                      float* cache_b, int64_t max_rows_b, int64_t width_b, const float* values_b,
                      int64_t rows, int64_t offset, void* stream) {
    float *dst_a = nullptr, *dst_b = nullptr;
    int rc = check_cache_write("a: ", cache_a, max_rows_a, width_a, values_a, rows, offset, &dst_a);
    if (rc) return rc;
    rc = check_cache_write("b: ", cache_b, max_rows_b, width_b, values_b, rows, offset, &dst_b);
    if (rc || rows == 0) return rc;
    // The two copies run side by side: neither may write what the other
    // reads or writes.
    const size_t na = sizeof(float) * (size_t)(rows * width_a), nb = sizeof(float) * (size_t)(rows * width_b);
    if (overlaps(dst_a, na, dst_b, nb)) return fail(ATTN_ERR_INVALID, "b: rows overlap the rows a writes");
    if (overlaps(dst_a, na, values_b, nb)) return fail(ATTN_ERR_INVALID, "b: values overlap the rows a writes");
    if (overlaps(dst_b, nb, values_a, na)) return fail(ATTN_ERR_INVALID, "a: values overlap the rows b writes");
    const hipError_t err = timed("cache_write", (hipStream_t)stream, [&](const attn::Launch& L) {
        return attn::launch_cache_write_pair(dst_a, values_a, rows * width_a, dst_b, values_b, rows * width_b, L);
    });
    if (err != hipSuccess) return fail(ATTN_ERR_DEVICE, "launch: %s", hipGetErrorString(err));
    return ok();
}

void attn_rope_params_init(attn_rope_params* r) {
    if (!r) return;
    memset(r, 0, sizeof *r);
    r->truncate = 1;
}

int attn_rope_table(const attn_rope_params* r, int64_t rows, float* inv_freq, float* attention_factor) {
    if (!inv_freq || !attention_factor) return fail(ATTN_ERR_INVALID, "rope: NULL output pointer");
    if (rows < 0) return fail(ATTN_ERR_INVALID, "rows: must be >= 0");
    if (r && (r->offset < 0 || r->offset > INT32_MAX))
        return fail(ATTN_ERR_INVALID, "rope.offset: must be in 0..2^31-1");
    attn::RopeArgs a;
    const int rc = rope_resolve(r, r ? r->offset + rows : 0, &a);
    if (rc) return rc;
    memcpy(inv_freq, a.inv_freq, sizeof(float) * (size_t)(a.rd / 2));
    *attention_factor = a.af;
    return ok();
}

int attn_rope(const attn_rope_params* r, int64_t T, int64_t width, const float* x, float* out, void* stream) {
    attn::RopeArgs a;
    int64_t heads = 0;
    int rc = rope_rows(r, T, width, &a, &heads);
    if (rc) return rc;
    if (T == 0) return ok();
    if (!x || !out) return fail(ATTN_ERR_INVALID, "%s: NULL pointer", x ? "out" : "x");
    const size_t n = sizeof(float) * (size_t)(T * width);
    if (x != out && overlaps(x, n, out, n)) return fail(ATTN_ERR_INVALID, "out: overlaps x (only out == x is allowed)");
    const hipError_t err = timed("rope", (hipStream_t)stream, [&](const attn::Launch& L) {
        return attn::launch_rope(a, x, out, T, (int)heads, (int)r->head_dim, L);
    });
    if (err != hipSuccess) return fail(ATTN_ERR_DEVICE, "launch: %s", hipGetErrorString(err));
    return ok();
}

int attn_rope_cache_write(float* cache, int64_t max_rows, int64_t width, const float* values, int64_t rows,
                          int64_t offset, const attn_rope_params* r, void* stream) {
    if (max_rows < 0) return fail(ATTN_ERR_INVALID, "maxRows: must be >= 0");
    if (offset < 0) return fail(ATTN_ERR_INVALID, "offset: must be >= 0 (got %lld)", (long long)offset);
    attn::RopeArgs a;
    int64_t heads = 0;
    int rc = rope_rows(r, rows, width, &a, &heads);
    if (rc) return rc;
    if (offset > max_rows || rows > max_rows - offset)
        return fail(ATTN_ERR_INVALID, "offset: rows %lld..%lld run past the cache's %lld rows",
                    (long long)offset, (long long)(offset + rows), (long long)max_rows);
    if ((double)max_rows * (double)width > 1e17) return fail(ATTN_ERR_INVALID, "cache: too large");
    if (rows == 0) return ok();
    if (!cache) return fail(ATTN_ERR_INVALID, "cache: NULL pointer");
    if (!values) return fail(ATTN_ERR_INVALID, "values: NULL pointer");
    float* dst = cache + offset * width;
    const size_t n = sizeof(float) * (size_t)(rows * width);
    if (overlaps(dst, n, values, n)) return fail(ATTN_ERR_INVALID, "values: overlap the rows being written");
    const hipError_t err = timed("rope", (hipStream_t)stream, [&](const attn::Launch& L) {
        return attn::launch_rope(a, values, dst, rows, (int)heads, (int)r->head_dim, L);
    });
    if (err != hipSuccess) return fail(ATTN_ERR_DEVICE, "launch: %s", hipGetErrorString(err));
    return ok();
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

void attn_mla_params_init(attn_mla_params* p) {
    if (!p) return;
    memset(p, 0, sizeof *p);
    p->causal = 1;
}

int attn_mla_validate(const attn_mla_params* p) {
    MlaResolved r;
    int rc = mla_resolve(p, &r);
    if (rc) return rc;
    MlaPlanFull plan;
    return mla_make_plan(r, &plan);
}

size_t attn_mla_workspace_size(const attn_mla_params* p) {
    MlaResolved r;
    if (mla_resolve(p, &r)) return 0;
    MlaPlanFull plan;
    if (mla_make_plan(r, &plan)) return 0;
    return plan.workspace;
}

int attn_mla_plan(const attn_mla_params* p, attn_plan_info* info) {
    if (!info) return fail(ATTN_ERR_INVALID, "info: NULL pointer");
    MlaResolved r;
    int rc = mla_resolve(p, &r);
    if (rc) return rc;
    MlaPlanFull plan;
    rc = mla_make_plan(r, &plan);
    if (rc) return rc;
    info->path = plan.path;
    info->splits = plan.path == ATTN_PATH_MLA ? plan.plan.splits : 1;
    info->tile_q = plan.path == ATTN_PATH_MLA ? (plan.plan.fast ? 16 : 1) : 0;
    info->variant = plan.path == ATTN_PATH_MLA ? plan.plan.slices : 0;
    return ok();
}

int attn_mla_forward(const attn_mla_params* p, const float* q, const float* state, const float* k_b,
                     const float* v_b, float* out, void* workspace, size_t workspace_bytes, void* stream) {
    MlaResolved r;
    int rc = mla_resolve(p, &r);
    if (rc) return rc;
    MlaPlanFull plan;
    rc = mla_make_plan(r, &plan);
    if (rc) return rc;
    if (plan.path == ATTN_PATH_EMPTY) return ok();

    const size_t qn = sizeof(float) * (size_t)(r.T * r.H * (r.N + r.P));
    const size_t sn = sizeof(float) * (size_t)(r.S * (r.R + r.P));
    const size_t kbn = sizeof(float) * (size_t)(r.H * r.N * r.R);
    const size_t vbn = sizeof(float) * (size_t)(r.H * r.Dv * r.R);
    const size_t on = sizeof(float) * (size_t)(r.T * r.H * r.Dv);
    if (!out) return fail(ATTN_ERR_INVALID, "out: NULL pointer");
    if (!q || !k_b || !v_b)
        return fail(ATTN_ERR_INVALID, "%s: NULL pointer", !q ? "q" : !k_b ? "k_b" : "v_b");
    if (r.S > 0 && !state) return fail(ATTN_ERR_INVALID, "state: NULL pointer");
    if (!aligned16(q) || !aligned16(state) || !aligned16(k_b) || !aligned16(v_b) || !aligned16(out))
        return fail(ATTN_ERR_INVALID, "q/state/k_b/v_b/out: pointers must be 16-byte aligned");
    if (overlaps(out, on, q, qn) || overlaps(out, on, state, sn) || overlaps(out, on, k_b, kbn) ||
        overlaps(out, on, v_b, vbn))
        return fail(ATTN_ERR_INVALID, "out: overlaps an input");
    hipStream_t s = (hipStream_t)stream;
    if (plan.path == ATTN_PATH_ZERO) {
        const hipError_t err = timed("zero_fill", s, [&](const attn::Launch& L) {
            return attn::launch_zero_fill(out, r.T * r.H * r.Dv, L);
        });
        if (err != hipSuccess) return fail(ATTN_ERR_DEVICE, "launch: %s", hipGetErrorString(err));
        return ok();
    }
    if (!workspace || workspace_bytes < plan.workspace)
        return fail(ATTN_ERR_INVALID, "workspace: %zu bytes needed, %zu given", plan.workspace,
                    workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace & 255u) != 0) return fail(ATTN_ERR_INVALID, "workspace: must be 256-byte aligned");
    if (overlaps(workspace, plan.workspace, out, on) || overlaps(workspace, plan.workspace, q, qn) ||
        overlaps(workspace, plan.workspace, state, sn) || overlaps(workspace, plan.workspace, k_b, kbn) ||
        overlaps(workspace, plan.workspace, v_b, vbn))
        return fail(ATTN_ERR_INVALID, "workspace: overlaps a tensor");

    attn::MlaProblem prob;
    prob.q = q;
    prob.state = state;
    prob.k_b = k_b;
    prob.v_b = v_b;
    prob.out = out;
    prob.q_abs = (float*)workspace;
    prob.part = (float*)((char*)workspace + plan.q_abs_bytes);
    prob.yslice = nullptr;
    prob.tickets = nullptr;
    if (plan.plan.slices > 0) {
        prob.yslice = (float*)((char*)workspace + plan.q_abs_bytes + plan.part_bytes);
        prob.tickets = (uint32_t*)((char*)prob.yslice +
                                   align256(sizeof(float) * (size_t)(r.T * r.H) * (size_t)plan.plan.slices *
                                            (size_t)r.Dv));
    }
    prob.T = r.T;
    prob.S = r.S;
    prob.H = (int32_t)r.H;
    prob.R = (int32_t)r.R;
    prob.N = (int32_t)r.N;
    prob.P = (int32_t)r.P;
    prob.Dv = (int32_t)r.Dv;
    prob.qk_scale = r.scale * 1.4426950408889634f;
    prob.vis.causal = r.causal ? 1 : 0;
    prob.vis.window = (int32_t)(r.window < INT32_MAX ? r.window : INT32_MAX);
    prob.vis.sinks = (int32_t)r.sinks;
    prob.vis.pos_offset = (int32_t)r.P0;

    hipError_t err = timed("mla_absorb", s, [&](const attn::Launch& L) { return attn::launch_mla_absorb(prob, L); });
    if (err == hipSuccess)
        err = timed("mla_split", s, [&](const attn::Launch& L) { return attn::launch_mla_split(prob, plan.plan, L); });
    if (err == hipSuccess)
        err = timed("mla_combine", s,
                    [&](const attn::Launch& L) { return attn::launch_mla_combine(prob, plan.plan, L); });
    if (err != hipSuccess) return fail(ATTN_ERR_DEVICE, "launch: %s", hipGetErrorString(err));
    return ok();
}

int attn_set_option(const char* name, int64_t value) {
    if (!name) return fail(ATTN_ERR_INVALID, "option: NULL name");
    if (!strcmp(name, "decode_splits")) {
        if (value < 0 || value > kDecodeMaxSplits)
            return fail(ATTN_ERR_INVALID, "decode_splits: must be in 0..%lld", (long long)kDecodeMaxSplits);
        g_opt_decode_splits = value;
        return ok();
    }
    if (!strcmp(name, "decode_rotate")) {
        if (value < 0 || value > (1 << 20)) return fail(ATTN_ERR_INVALID, "decode_rotate: must be in 0..2^20");
        g_opt_decode_rotate = value;
        return ok();
    }
    if (!strcmp(name, "decode_wgs_per_cu")) {
        if (value < 0 || value > 8) return fail(ATTN_ERR_INVALID, "decode_wgs_per_cu: must be in 0..8");
        g_opt_decode_wgs = value;
        return ok();
    }
    if (!strcmp(name, "decode_block")) {
        if (value != 0 && value != -1 && (value < 32 || value > 4096 || (value & (value - 1))))
            return fail(ATTN_ERR_INVALID, "decode_block: must be 0, -1 or a power of two in 32..4096");
        g_opt_decode_block = value;
        return ok();
    }
    if (!strcmp(name, "mla_slices")) {
        if (value < -1 || value > 1) return fail(ATTN_ERR_INVALID, "mla_slices: must be -1, 0 or 1");
        g_opt_mla_slices = value;
        return ok();
    }
    if (!strcmp(name, "mla_combine_out")) {
        if (value != 0 && value != 16 && value != 32) return fail(ATTN_ERR_INVALID, "mla_combine_out: must be 0, 16 or 32");
        g_opt_mla_combine_out = value;
        return ok();
    }
    if (!strcmp(name, "decode_mfma")) {
        if (value < -1 || value > 1) return fail(ATTN_ERR_INVALID, "decode_mfma: must be -1, 0 or 1");
        g_opt_decode_mfma = value;
        return ok();
    }
    if (!strcmp(name, "decode_depth")) {
        if (value < 0 || value > 3) return fail(ATTN_ERR_INVALID, "decode_depth: must be 0, 1, 2 or 3");
        g_opt_decode_depth = value;
        return ok();
    }
    if (!strcmp(name, "prefill_splits")) {
        if (value < 0 || value > kPrefillMaxSplits)
            return fail(ATTN_ERR_INVALID, "prefill_splits: must be in 0..%lld", (long long)kPrefillMaxSplits);
        g_opt_prefill_splits = value;
        return ok();
    }
    if (!strcmp(name, "prefill_variant")) {
        if (value != 0 && value != 16 && value != 32)
            return fail(ATTN_ERR_INVALID, "prefill_variant: must be 0, 16 or 32");
        g_opt_prefill_variant = value;
        return ok();
    }
    if (!strcmp(name, "force_path")) {
        if (value != 0 && value != ATTN_PATH_GENERIC && value != ATTN_PATH_DECODE && value != ATTN_PATH_PREFILL)
            return fail(ATTN_ERR_INVALID, "force_path: must be 0, %d, %d or %d", ATTN_PATH_GENERIC,
                        ATTN_PATH_DECODE, ATTN_PATH_PREFILL);
        g_opt_force_path = value;
        return ok();
    }
    if (!strcmp(name, "mla_splits")) {
        if (value < 0 || value > kMlaMaxSplits - 1)
            return fail(ATTN_ERR_INVALID, "mla_splits: must be in 0..%lld", (long long)(kMlaMaxSplits - 1));
        g_opt_mla_splits = value;
        return ok();
    }
    if (!strcmp(name, "mla_row_groups")) {
        if (value < 0 || value > 2) return fail(ATTN_ERR_INVALID, "mla_row_groups: must be 0, 1 or 2");
        g_opt_mla_row_groups = value;
        return ok();
    }
    if (!strcmp(name, "mla_generic")) {
        if (value != 0 && value != 1) return fail(ATTN_ERR_INVALID, "mla_generic: must be 0 or 1");
        g_opt_mla_generic = value;
        return ok();
    }
    return fail(ATTN_ERR_INVALID, "option: unknown name '%s'", name);
}

int attn_timing_enable(int on) {
    Timing& tm = timing();
    std::lock_guard<std::mutex> lock(tm.mu);
    if (on && !tm.created) {
        tm.start.resize(kTimingSlots);
        tm.stop.resize(kTimingSlots);
        for (int i = 0; i < kTimingSlots; ++i) {
            if (hipEventCreate(&tm.start[i]) != hipSuccess || hipEventCreate(&tm.stop[i]) != hipSuccess)
                return fail(ATTN_ERR_DEVICE, "timing: hipEventCreate failed");
            tm.free_slots.push_back(kTimingSlots - 1 - i);
        }
        tm.created = true;
    }
    tm.on = on != 0;
    return ok();
}

int attn_timing_collect(const char* kernel, double* total_ms, int64_t* launches) {
    if (!kernel || !total_ms || !launches) return fail(ATTN_ERR_INVALID, "timing: NULL argument");
    Timing& tm = timing();
    std::lock_guard<std::mutex> lock(tm.mu);
    double sum = 0.0;
    int64_t n = 0;
    std::vector<TimingRecord> keep;
    for (const TimingRecord& rec : tm.records) {
        if (strcmp(rec.name, kernel)) {
            keep.push_back(rec);
            continue;
        }
        if (hipEventSynchronize(tm.stop[rec.slot]) != hipSuccess)
            return fail(ATTN_ERR_DEVICE, "timing: hipEventSynchronize failed");
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, tm.start[rec.slot], tm.stop[rec.slot]) != hipSuccess)
            return fail(ATTN_ERR_DEVICE, "timing: hipEventElapsedTime failed");
        sum += ms;
        ++n;
        tm.free_slots.push_back(rec.slot);
    }
    tm.records.swap(keep);
    *total_ms = sum;
    *launches = n;
    return ok();
}

}  // extern "C"
