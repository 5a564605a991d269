// Op `rope` (graph protocol op catalogue): rows of heads x head_dim floats,
// each head's channel pairs turned by position * invFreq[i]. One kernel serves
// the standalone op and the rotate-then-write cache path (out then points at
// the cache row `offset`). HBM-bound: every element is read and written once.
//
// Each thread owns whole pairs, so out may equal x (in place): both channels
// of a pair are read before either is written, by the same thread.
#include "kernels.h"
#include "rope_device.h"

namespace attn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

// Vector path (head_dim % 4 == 0, 16-byte aligned rows). Per head:
//   half-split (rd % 8 == 0): unit u < rd/8 owns channels 4u..4u+3 and
//     rd/2+4u..rd/2+4u+3, i.e. pairs 4u..4u+3;
//   interleaved (rd % 4 == 0): unit u < rd/4 owns channels 4u..4u+3, i.e.
//     pairs 2u and 2u+1;
//   then one unit per pass-through float4 (channels rd..D-1).
// grid (rows, ceil(heads * units / kThreads)): every head of a row turns by
// the same angles, so the workgroup computes the row's rd/2 (cos, sin)
// pairs once, into LDS, and its threads read them there (the same f32
// values each thread would compute itself).
__global__ __launch_bounds__(kThreads) void rope_vec_kernel(RopeArgs ra, const float* x, float* out, int heads,
                                                            int D, int units) {
    __shared__ float s_cos[ATTN_ROPE_MAX_ROTARY_DIM / 2], s_sin[ATTN_ROPE_MAX_ROTARY_DIM / 2];
    const int rot_units = ra.interleaved ? ra.rd / 4 : ra.rd / 8;
    const int64_t row = blockIdx.x;
    const int64_t pos = ra.pos0 + row;
    const int idx = (int)blockIdx.y * kThreads + (int)threadIdx.x;
    const bool active = idx < heads * units;
    const bool in_place = x == out;
    const int h = active ? idx / units : 0, u = active ? idx - h * units : 0;
    const int64_t rh = row * heads + h;
    const float* xh = x + rh * D;
    float* oh = out + rh * D;
    // The thread's channels are requested before the row's angles are
    // worked out, so the memory latency overlaps that arithmetic.
    const bool rot = active && u < rot_units;
    const int dpass = ra.rd + 4 * (u - rot_units);
    float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
    if (active) {
        if (!rot) {
            if (!in_place) va = ld4(xh + dpass);  // pass-through channels: copied unless in place
        }
        else if (ra.interleaved) va = ld4(xh + 4 * u);
        else {
            va = ld4(xh + 4 * u);
            vb = ld4(xh + ra.rd / 2 + 4 * u);
        }
    }
    for (int i = threadIdx.x; i < ra.rd / 2; i += kThreads) rope_cos_sin(pos, ra.inv_freq[i], ra.af, s_cos[i], s_sin[i]);
    __syncthreads();
    if (!active) return;
    if (!rot) {
        if (!in_place) st4(oh + dpass, va);
        return;
    }
    {
        if (ra.interleaved) {
            const float4 v = va;
            const float c0 = s_cos[2 * u], s0 = s_sin[2 * u], c1 = s_cos[2 * u + 1], s1 = s_sin[2 * u + 1];
            float4 o;
            o.x = fmaf(-v.y, s0, v.x * c0);
            o.y = fmaf(v.x, s0, v.y * c0);
            o.z = fmaf(-v.w, s1, v.z * c1);
            o.w = fmaf(v.z, s1, v.w * c1);
            st4(oh + 4 * u, o);
        } else {
            const int half = ra.rd / 2;
            const float4 a = va, b = vb;
            float c[4], s[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = s_cos[4 * u + j];
                s[j] = s_sin[4 * u + j];
            }
            float4 oa, ob;
            oa.x = fmaf(-b.x, s[0], a.x * c[0]);
            oa.y = fmaf(-b.y, s[1], a.y * c[1]);
            oa.z = fmaf(-b.z, s[2], a.z * c[2]);
            oa.w = fmaf(-b.w, s[3], a.w * c[3]);
            ob.x = fmaf(a.x, s[0], b.x * c[0]);
            ob.y = fmaf(a.y, s[1], b.y * c[1]);
            ob.z = fmaf(a.z, s[2], b.z * c[2]);
            ob.w = fmaf(a.w, s[3], b.w * c[3]);
            st4(oh + 4 * u, oa);
            st4(oh + half + 4 * u, ob);
        }
    }
}

// Any shape: one unit per pair (both channels) and per pass-through channel.
__global__ __launch_bounds__(kThreads) void rope_scalar_kernel(RopeArgs ra, const float* x, float* out,
                                                               int64_t rows, int heads, int D) {
    const int half = ra.rd / 2;
    const int units = half + (D - ra.rd);
    const int64_t total = rows * heads * units;
    for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * kThreads) {
        const int u = (int)(idx % units);
        const int64_t rh = idx / units;
        const int64_t pos = ra.pos0 + rh / heads;
        const float* xh = x + rh * D;
        float* oh = out + rh * D;
        if (u >= half) {
            const int d = ra.rd + (u - half);
            oh[d] = xh[d];
            continue;
        }
        const int ia = ra.interleaved ? 2 * u : u;
        const int ib = ra.interleaved ? 2 * u + 1 : u + half;
        const float a = xh[ia], b = xh[ib];
        float c, s;
        rope_cos_sin(pos, ra.inv_freq[u], ra.af, c, s);
        oh[ia] = fmaf(-b, s, a * c);
        oh[ib] = fmaf(a, s, b * c);
    }
}

int64_t grid_for(int64_t total) {
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    return blocks < (1 << 20) ? (blocks > 0 ? blocks : 1) : (1 << 20);
}

}  // namespace

hipError_t launch_rope(const RopeArgs& ra, const float* x, float* out, int64_t rows, int heads, int D,
                       const Launch& L) {
    const bool aligned = (((uintptr_t)x | (uintptr_t)out) & 15u) == 0;
    const bool vec = aligned && D % 4 == 0 && (ra.interleaved ? ra.rd % 4 == 0 : ra.rd % 8 == 0);
    const int units = (ra.interleaved ? ra.rd / 4 : ra.rd / 8) + (D - ra.rd) / 4;
    if (vec && rows > 0 && rows <= INT32_MAX && (int64_t)heads * units <= 65535LL * kThreads) {
        const dim3 grid((unsigned)rows, (unsigned)((heads * units + kThreads - 1) / kThreads));
        return launch_kernel(rope_vec_kernel, grid, dim3(kThreads), 0, L, ra, x, out, heads, D, units);
    }
    const int64_t total = rows * heads * (ra.rd / 2 + (D - ra.rd));
    return launch_kernel(rope_scalar_kernel, dim3((unsigned)grid_for(total)), dim3(kThreads), 0, L, ra, x,
                         out, rows, heads, D);
}

}  // namespace attn
