// Device-side pieces shared by the attention kernels: the visibility rule,
// the score epilogue and a few CDNA lane-exchange helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

constexpr float kLog2e = 1.4426950408889634f;

// Graph protocol op catalogue, op `attention`, params causal and window:
// causal keys are visible when pos - window < s <= pos, non-causal keys when
// |pos - s| <= window; window 0 means no window.
// Positions are non-negative and below 2^31, so none of this overflows.
// E is any struct with the fields causal, window and sinks (Epilogue here,
// the latent attention's own parameters elsewhere).
template <typename E>
__device__ __forceinline__ bool window_visible(const E& e, int pos, int s) {
    if (e.causal) return s <= pos && (e.window == 0 || s > pos - e.window);
    if (e.window == 0) return true;
    return abs(pos - s) <= e.window;
}

// An attention sink (one of the first e.sinks keys; e.sinks is 0 without a
// window) stays in view beside the window: non-causal rows always see it,
// causal rows once it is at or before their position.
template <typename E>
__device__ __forceinline__ bool sink_visible(const E& e, int pos, int s) {
    return (s < e.sinks) & (!e.causal | (s <= pos));
}

template <typename E>
__device__ __forceinline__ bool key_visible(const E& e, int pos, int s) {
    return window_visible(e, pos, s) | sink_visible(e, pos, s);
}

// Whether every query row of positions [pos_first, pos_last] sees every key
// of [k0, k1) (graph protocol op catalogue, op `attention`, window rule).
__device__ __forceinline__ bool chunk_all_visible(const Epilogue& e, int pos_first, int pos_last,
                                                  int k0, int k1) {
    if (k1 <= k0) return true;
    if (e.causal) return k1 - 1 <= pos_first && (e.window == 0 || k0 > pos_last - e.window);
    if (e.window == 0) return true;
    const int d = max(max(abs(pos_first - k0), abs(pos_first - (k1 - 1))),
                      max(abs(pos_last - k0), abs(pos_last - (k1 - 1))));
    return d <= e.window;
}

// The bucketed position bias of key s for a query at pos in head h: the
// bucket of distance |pos - s| (the last threshold not above it), in the
// second half of the table for a later key when the table is bidirectional.
__device__ __forceinline__ float position_bias(const Epilogue& e, int h, int pos, int s) {
    const int d = abs(pos - s);
    int b = d < e.pb_dt ? (int)e.pb_bucket[d] : e.pb_n - 1;
    if (e.pb_bidir && s > pos) b += e.pb_n;
    return e.pb_weight[b * e.pb_heads + h];
}

// The relative-embedding row of key s for a query at pos:
// clip(s - pos, -rel_max, rel_max) + rel_max.
__device__ __forceinline__ int rel_row(const Epilogue& e, int pos, int s) {
    return min(max(s - pos, -e.rel_max), e.rel_max) + e.rel_max;
}

// The same with the distance -> bucket table in LDS (tab, pb_dt entries).
__device__ __forceinline__ float position_bias_tab(const Epilogue& e, const uint8_t* tab, int h, int pos, int s) {
    const int d = abs(pos - s);
    int b = d < e.pb_dt ? (int)tab[d] : e.pb_n - 1;
    if (e.pb_bidir && s > pos) b += e.pb_n;
    return e.pb_weight[b * e.pb_heads + h];
}

// The score of one visible (query, key) pair, in the order the op fixes:
// scale the dot product, softcap it (feature attention.softcap puts the cap
// ahead of masking), then add the ALiBi penalty -slope*|pos - s| and the bias entry
// (the bias input plus the bucketed position bias, fetched ahead by the
// caller).
__device__ __forceinline__ float score_epilogue(float dot, const Epilogue& e, int h, int pos, int s,
                                                float bias) {
    float x = dot * e.scale;
    if (e.softcap > 0.0f) x = e.softcap * tanhf(x * e.inv_softcap);
    if (e.has_alibi) x -= e.slopes[h] * (float)abs(pos - s);
    return x + bias;
}

// 2^x with the hardware exponential (v_exp_f32; about 1 ulp). Inputs here are
// differences from a running maximum, so results below 2^-126 are weights
// too small to matter.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A 128-bit load that bypasses the caches' normal retention: K and V rows
// are read once per call, so keeping them would only evict other data.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream4(const float* p) {
    const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}

// Row-of-16 all-reduce with DPP row rotations: after the four steps every
// lane of each 16-lane DPP row holds the row's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f32<0x128>(x);  // row_ror:8
    x += dpp_f32<0x124>(x);  // row_ror:4
    x += dpp_f32<0x122>(x);  // row_ror:2
    x += dpp_f32<0x121>(x);  // row_ror:1
    return x;
}

__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f32<0x128>(x));
    x = fmaxf(x, dpp_f32<0x124>(x));
    x = fmaxf(x, dpp_f32<0x122>(x));
    x = fmaxf(x, dpp_f32<0x121>(x));
    return x;
}

__device__ __forceinline__ float dot4(const float4& a, const float4& b, float acc) {
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
    return acc;
}

}  // namespace attn
