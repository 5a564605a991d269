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

// The same for row r of a KV group with the weights in LDS as well
// (w[bucket * NQ + r]: the row's head's weight of each bucket).
template <int NQ>
__device__ __forceinline__ float pb_row_tab_n(const Epilogue& e, const uint8_t* tab, const float* w, int r, int pos,
                                              int s) {
    const int d = abs(pos - s);
    int b = d < e.pb_dt ? (int)tab[d] : e.pb_n - 1;
    if (e.pb_bidir && s > pos) b += e.pb_n;
    return w[b * NQ + r];
}

// tanh without branches or library calls. Below |x| = 1/4 its Taylor
// series through x^9 (truncation error under 1e-8 relative there); above,
// the identity tanh|x| = (1 - e^(-2|x|)) / (1 + e^(-2|x|)) with the hardware
// exp2 and reciprocal, where 1 - e^(-2|x|) > 0.39 loses no accuracy to
// cancellation; then the sign of x. A few ulp from the true value
// everywhere, saturating to +-1 for large |x|; NaN stays NaN.
__device__ __forceinline__ float fast_tanh(float x) {
    const float a = fabsf(x);
    const float z = x * x;
    const float series =
        fmaf(x * z, fmaf(z, fmaf(z, fmaf(z, 62.0f / 2835.0f, -17.0f / 315.0f), 2.0f / 15.0f), -1.0f / 3.0f), x);
    const float t = __builtin_amdgcn_exp2f(-2.0f * kLog2e * a);
    const float big = copysignf((1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t), x);
    return a < 0.25f ? series : big;
}

// The ALiBi slope of head h (0 without ALiBi). Kernels read it once per query
// row, ahead of their key loops: the slope table sits in the kernel's argument
// block, and an index that the compiler cannot prove uniform turns each read
// into a vector memory load, which inside a key loop also makes the wave wait
// for every load issued before it.
__device__ __forceinline__ float alibi_slope(const Epilogue& e, int h) { return e.has_alibi ? e.slopes[h] : 0.0f; }

// The score of one visible (query, key) pair, in the order the op fixes:
// scale the dot product, softcap it (feature attention.softcap puts the cap
// ahead of masking), then add the ALiBi penalty -slope*|pos - s| (slope:
// alibi_slope of the row's head) and the bias entry (the bias input plus the
// bucketed position bias, fetched ahead by the caller).
__device__ __forceinline__ float score_epilogue(float dot, const Epilogue& e, float slope, int pos, int s,
                                                float bias) {
    float x = dot * e.scale;
    if (e.softcap > 0.0f) x = e.softcap * fast_tanh(x * e.inv_softcap);
    if (e.has_alibi) x -= slope * (float)abs(pos - s);
    return x + bias;
}

// score_epilogue for N scores of one query row at once (key of score i:
// s[i]), times log2(e) (the base-2 domain): the same operations per score in
// the same order, with each term's test (the same for the whole wave) taken
// once for all N, so that their independent computations interleave instead
// of running one score at a time between branches.
template <int N>
__device__ __forceinline__ void score_epilogue_n(float (&x)[N], const Epilogue& e, float slope, int pos,
                                                 const int (&s)[N], const float (&bias)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] *= e.scale;
    if (e.softcap > 0.0f) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = e.softcap * fast_tanh(x[i] * e.inv_softcap);
    }
    if (e.has_alibi) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] -= slope * (float)abs(pos - s[i]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = (x[i] + bias[i]) * kLog2e;
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
