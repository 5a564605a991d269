// Internal interface between the host dispatch (attn_api.hip) and the HIP
// kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

// Everything the score epilogue needs (op `attention`: scale, softcap,
// ALiBi, bias, causal/window mask), resolved on the host.
struct Epilogue {
    float scale;        // multiplies q.k
    float softcap;      // 0: off
    float inv_softcap;  // 1/softcap when on
    int32_t causal;
    int32_t has_alibi;
    int32_t bias_kind;  // ATTN_BIAS_*
    int32_t pos_offset; // positions are below 2^31 (checked on the host)
    int32_t window;     // 0: off
    int32_t sinks;      // attention sinks: keys s < sinks stay visible beside the window (0 without one)
    float slopes[ATTN_ALIBI_MAX_HEADS];
    // Bucketed relative position bias: pb_weight[bucket * pb_heads + h].
    const float* pb_weight;  // NULL: off
    int32_t pb_n;            // thresholds (buckets per direction)
    int32_t pb_bidir;        // keys after the query take buckets pb_n .. 2 pb_n - 1
    int32_t pb_dt;           // distances >= pb_dt take bucket pb_n - 1
    int32_t pb_heads;        // row stride of pb_weight
    uint8_t pb_bucket[ATTN_PB_MAX_DIST];  // bucket of each distance below pb_dt
    // Relative key/value embeddings, row clip(s - pos, -rel_max, rel_max) + rel_max.
    const float* rel_k;      // NULL: off; else [2 rel_max + 1, D], joins k before the q product
    const float* rel_v;      // NULL or [2 rel_max + 1, Dv], joins v
    int32_t rel_max;

    // Whether any term beyond the scaled dot product is on (the kernels'
    // epilogue-free instances serve the rest).
    __host__ __device__ bool any() const {
        return softcap > 0.0f || has_alibi || bias_kind != ATTN_BIAS_NONE || pb_weight != nullptr ||
               rel_k != nullptr;
    }
};

// A resolved rotary embedding (op `rope`): the f32 inverse-frequency table
// and attention factor computed on the host, the pairing and the position of
// row 0.
struct RopeArgs {
    int32_t on;           // 0: no rotation (attention kernels' q path only)
    int32_t rd;           // rotated channels per head (even, <= ATTN_ROPE_MAX_ROTARY_DIM)
    int32_t interleaved;  // 1: pairs (2i, 2i+1); 0: pairs (i, i + rd/2)
    float af;             // attention factor: multiplies cos and sin
    int64_t pos0;         // position of row 0
    float inv_freq[ATTN_ROPE_MAX_ROTARY_DIM / 2];
};

struct Problem {
    const float* q;
    const float* k;
    const float* v;
    const float* bias;
    float* out;
    int64_t T, S;
    int32_t H, G, D, Dv;
    Epilogue ep;
    RopeArgs rope;  // applied to q as it is loaded when rope.on
};

// Key rows [lo, hi) that any query row of the call can see. Rows outside
// are never read (a KV cache past the current position may hold anything).
struct KeyRange {
    int64_t lo, hi;
};

struct DecodePlan {
    int32_t nq;       // query rows per KV group this instance holds (template value)
    int32_t mfma;     // 1: decode_mfma (matrix cores, rows in blocks of 16); 0: decode_split
    int32_t splits;   // key-range splits per KV group (the sink split included)
    int32_t depth;    // batches of key rows per lane in registers: 1 (one at a time) or a ring of 2 or 3
    int32_t sink_hi;  // > 0: the last split covers the sink keys [0, sink_hi) below `range`
    int32_t rotate;            // split sp starts (sp * rotate mod chunk) rows into its chunk (0: in order)
    int32_t near_lo, near_hi;  // near_hi > near_lo: a split (before the sink split) covers
                               // [near_lo, near_hi), the keys nearest the query rows: those the
                               // relative-position tables reach, or the rows the call appends
    int32_t block;    // > 0: the splits of `range` interleave blocks of this many rows (a power
                      // of two, multiple of the row-group step): split i takes blocks i,
                      // i + main_splits, ...; 0: split i takes the i-th chunk of `chunk` rows
    int32_t main_splits;  // splits over `range` (the near and sink splits follow them)
    int64_t chunk;    // keys per split of `range` (multiple of the row-group step)
    KeyRange range;
    // Appending calls: the near split reads its rows from k_new / v_new (row
    // i there is row near_lo + i; same row widths as the caches) and stores
    // them into k_cache / v_cache as it goes. Null otherwise. With them the
    // grid is 1-D: the other splits of every KV group in the usual order,
    // then the near split of each group.
    const float* k_new;
    const float* v_new;
    float* k_cache;
    float* v_cache;
};

struct PrefillPlan {
    int32_t variant;  // 32: 32x32x2 MFMA, 4 waves of 32 rows; 16: 16x16x4, 8 waves of 16 rows
    int32_t tile_q;   // query rows per workgroup and head
    int32_t nh;       // heads of one KV group per workgroup
    int32_t qblocks;  // workgroups along the query rows
    int32_t ksplit;   // key-range parts per workgroup (partials merged by the combine kernel)
    int32_t rel_band; // > 0: relative embeddings in two launches, the tiles beyond the tables'
                      // reach (ksplit parts) then the band tiles (rel_band parts): ksplit +
                      // rel_band partials; 0: one launch
};

// Where and how one kernel launch goes: the caller's stream, and optionally
// a pair of events that the dispatch itself stamps with the kernel's start
// and end (hipExtLaunchKernel), used only when timing is switched on.
struct Launch {
    hipStream_t stream;
    hipEvent_t start;
    hipEvent_t stop;
};

template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds,
                                const Launch& L, Args... args) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, L.stream, L.start, L.stop, 0, args...);
    return hipGetLastError();
}

// Latent (MLA) attention in absorbed form. Rows are (query row t, head h)
// pairs, row index t*H + h; the latent state row s is [c_s (R) | k_pe_s (P)].
struct MlaVis {
    int32_t causal;
    int32_t window;      // 0: off
    int32_t sinks;       // keys s < sinks stay visible beside the window (0 without one)
    int32_t pos_offset;  // position of query row 0
};

struct MlaProblem {
    const float* q;      // [T, H*(N+P)]: per head the no-rope part, then the rotary part
    const float* state;  // [S, R+P]
    const float* k_b;    // [H, N, R]
    const float* v_b;    // [H, Dv, R]
    float* out;          // [T, H*Dv]
    float* q_abs;        // workspace [T*H, R+P]: k_b[h]^T q_nope, then q_pe
    float* part;         // workspace: acc [T*H][splits][R], then (max, sum) [T*H][splits][2]
    float* yslice;       // workspace [T*H][slices][Dv]: each latent slice's share of out (slices > 0)
    uint32_t* tickets;   // workspace [T*H]: slices of the row finished (zeroed by mla_absorb)
    int64_t T, S;
    int32_t H, R, N, P, Dv;
    float qk_scale;      // scale * log2(e): scores live in the base-2 domain
    MlaVis vis;
};

struct MlaPlan {
    int32_t fast;        // 1: the MFMA split kernel has an instance for (R, P); 0: the generic one
    int32_t splits;      // key-range splits (the sink split included)
    int32_t sink_hi;     // > 0: the last split covers the sink keys [0, sink_hi) below `range`
    int32_t row_blocks;  // 16-row blocks along the T*H rows
    int32_t row_groups;  // 16-row blocks per workgroup of the split kernel (1 or 2)
    int32_t combine_out; // output channels per combine workgroup (32 or 16)
    int32_t slices;      // > 0: mla_combine_slice, R / 64 latent slices per row; 0: mla_combine4
    int64_t chunk;       // keys per split of `range` (a multiple of 16)
    KeyRange range;
};

// Launchers. Each returns hipSuccess or the launch error.
hipError_t launch_cache_write(float* dst, const float* src, int64_t count, const Launch& L);
// Two flat copies (count_a and count_b floats, both > 0) in one launch.
hipError_t launch_cache_write_pair(float* dst_a, const float* src_a, int64_t count_a, float* dst_b,
                                   const float* src_b, int64_t count_b, const Launch& L);
// out rows = rope(x rows): rows x heads heads of D floats each; out may equal x.
hipError_t launch_rope(const RopeArgs& ra, const float* x, float* out, int64_t rows, int heads, int D,
                       const Launch& L);
hipError_t launch_zero_fill(float* dst, int64_t count, const Launch& L);
hipError_t launch_generic(const Problem& p, const Launch& L);
bool decode_supported(int D, int Dv, int nq);
hipError_t launch_decode_split(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L);
hipError_t launch_decode_combine(const Problem& p, const DecodePlan& plan, const float* ws,
                                 const Launch& L);
int decode_mfma_max_rows(int D, int Dv);
hipError_t launch_decode_mfma(const Problem& p, const DecodePlan& plan, float* ws, const Launch& L);
bool prefill_supported(int D, int Dv);
int prefill_wgs_per_cu(int variant, int D, int Dv, bool rel);
bool prefill_rel_supported(int D, int Dv);
// part: 0 every key tile; with plan.rel_band, 1 the tiles beyond the relative
// tables' reach, 2 the band tiles.
hipError_t launch_prefill(const Problem& p, const PrefillPlan& plan, float* ws, int part, const Launch& L);
bool mla_fast_supported(int R, int P);
// Whether mla_combine_slice serves (R, Dv): R a multiple of 64 up to 512, Dv <= 256.
bool mla_slices_supported(int R, int Dv);
hipError_t launch_mla_absorb(const MlaProblem& p, const Launch& L);
hipError_t launch_mla_split(const MlaProblem& p, const MlaPlan& plan, const Launch& L);
hipError_t launch_mla_combine(const MlaProblem& p, const MlaPlan& plan, const Launch& L);

}  // namespace attn
