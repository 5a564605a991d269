// Correctness path of op `attention` for any head widths: one workgroup per
// (query row, head). It makes two passes over the visible keys: the first
// finds the row's largest score, the second forms the max-subtracted
// weights (catalogue op `softmax` subtracts the row maximum first, which
// keeps exp from overflowing) 256 keys at a time and accumulates weight * v
// into LDS.
// Slow but shape-agnostic; the tuned decode and prefill kernels cover the
// common widths.
#include "device_common.h"
#include "rope_device.h"

namespace attn {

namespace {

constexpr int kThreads = 256;

__device__ float block_reduce(float x, float* red, bool is_max) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) {
        const float y = __shfl_xor(x, o, 64);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    x = red[0];
    for (int w = 1; w < kThreads / 64; ++w) x = is_max ? fmaxf(x, red[w]) : x + red[w];
    return x;
}

// qrel: the row's products with the relative key embeddings (q . rel_k[j]),
// or NULL without them.
__device__ __forceinline__ float score_at(const Problem& p, const float* qrow, const float* qrel, int h,
                                          float slope, int g, int64_t t, int pos, int s) {
    const float* krow = p.k + s * (int64_t)p.G * p.D + (int64_t)g * p.D;
    float dot = 0.0f;
    for (int d = 0; d < p.D; ++d) dot = fmaf(qrow[d], krow[d], dot);
    if (qrel) dot += qrel[rel_row(p.ep, pos, s)];
    float b = 0.0f;
    if (p.ep.bias_kind == ATTN_BIAS_TS) b = p.bias[t * p.S + s];
    else if (p.ep.bias_kind == ATTN_BIAS_HTS) b = p.bias[((int64_t)h * p.T + t) * p.S + s];
    if (p.ep.pb_weight) b += position_bias(p.ep, h, pos, s);
    return score_epilogue(dot, p.ep, slope, pos, s, b);
}

__global__ __launch_bounds__(kThreads) void generic_kernel(Problem p) {
    extern __shared__ float smem[];
    float* qrow = smem;            // D
    float* acc = qrow + p.D;       // Dv
    float* w = acc + p.Dv;         // kThreads weights of the current key chunk
    float* red = w + kThreads;     // kThreads / 64 partials
    float* qrel = red + kThreads / 64;  // 2 rel_max + 1 products q . rel_k[j] (with relative keys)

    const int64_t t = blockIdx.x;
    const int h = blockIdx.y;
    const int g = (int)(((int64_t)h * p.G) / p.H);
    const int pos = p.ep.pos_offset + (int)t;
    const float slope = alibi_slope(p.ep, h);
    const int tid = threadIdx.x;

    const float* qhead = p.q + t * (int64_t)p.H * p.D + (int64_t)h * p.D;
    for (int d = tid; d < p.D; d += kThreads)
        qrow[d] = p.rope.on ? rope_channel(p.rope, qhead, d, p.rope.pos0 + t) : qhead[d];
    for (int e = tid; e < p.Dv; e += kThreads) acc[e] = 0.0f;
    __syncthreads();
    const int nrel = p.ep.rel_k ? 2 * p.ep.rel_max + 1 : 0;
    for (int j = tid; j < nrel; j += kThreads) {
        const float* rk = p.ep.rel_k + (int64_t)j * p.D;
        float d = 0.0f;
        for (int c = 0; c < p.D; ++c) d = fmaf(qrow[c], rk[c], d);
        qrel[j] = d;
    }
    if (nrel) __syncthreads();
    const float* qr = nrel ? qrel : nullptr;

    float m = -INFINITY;
    for (int s = tid; s < p.S; s += kThreads)
        if (key_visible(p.ep, pos, s)) m = fmaxf(m, score_at(p, qrow, qr, h, slope, g, t, pos, s));
    m = block_reduce(m, red, true);

    float* orow = p.out + t * (int64_t)p.H * p.Dv + (int64_t)h * p.Dv;
    if (m == -INFINITY) {  // no visible key: the empty sum
        for (int e = tid; e < p.Dv; e += kThreads) orow[e] = 0.0f;
        return;
    }

    float l = 0.0f;
    for (int s0 = 0; s0 < p.S; s0 += kThreads) {
        const int s = s0 + tid;
        float wt = 0.0f;
        if (s < p.S && key_visible(p.ep, pos, s))
            wt = exp2f((score_at(p, qrow, qr, h, slope, g, t, pos, s) - m) * kLog2e);
        l += wt;
        __syncthreads();
        w[tid] = wt;
        __syncthreads();
        const int n = p.S - s0 < kThreads ? (int)(p.S - s0) : kThreads;
        for (int e = tid; e < p.Dv; e += kThreads) {
            float a = acc[e];
            for (int j = 0; j < n; ++j)
                if (w[j] != 0.0f) {
                    float val = p.v[(int64_t)(s0 + j) * p.G * p.Dv + (int64_t)g * p.Dv + e];
                    if (p.ep.rel_v) val += p.ep.rel_v[(int64_t)rel_row(p.ep, pos, s0 + j) * p.Dv + e];
                    a = fmaf(w[j], val, a);
                }
            acc[e] = a;
        }
    }
    l = block_reduce(l, red, false);
    __syncthreads();
    for (int e = tid; e < p.Dv; e += kThreads) orow[e] = acc[e] / l;
}

}  // namespace

hipError_t launch_generic(const Problem& p, const Launch& L) {
    const size_t nrel = p.ep.rel_k ? 2 * (size_t)p.ep.rel_max + 1 : 0;
    const size_t lds = sizeof(float) * ((size_t)p.D + p.Dv + kThreads + kThreads / 64 + nrel);
    return launch_kernel(generic_kernel, dim3((unsigned)p.T, (unsigned)p.H), dim3(kThreads),
                         (uint32_t)lds, L, p);
}

}  // namespace attn
