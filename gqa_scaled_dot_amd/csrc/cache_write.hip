// Op `cache_write` (graph protocol op catalogue): write `values` into rows
// [offset, offset + rows) of a preallocated cache, in place. Both the source
// rows and the destination rows are contiguous runs of rows*width floats,
// so the op is one flat copy, done with 128-bit loads and stores when the
// two pointers share their 16-byte phase, and with 32-bit ones otherwise.
// The copy is exact: floats move as bits, never through arithmetic.
#include "kernels.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxBlocks = 8192;

__global__ __launch_bounds__(kThreads) void copy_vec4_kernel(float* __restrict__ dst,
                                                             const float* __restrict__ src,
                                                             int64_t head, int64_t n4,
                                                             int64_t count) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    // Unaligned head (< 4 floats) and tail handled by the first threads.
    if (tid < head) dst[tid] = src[tid];
    const int64_t tail_start = head + n4 * 4;
    if (tid < count - tail_start) dst[tail_start + tid] = src[tail_start + tid];
    const float4* s4 = reinterpret_cast<const float4*>(src + head);
    float4* d4 = reinterpret_cast<float4*>(dst + head);
    for (int64_t i = tid; i < n4; i += stride) d4[i] = s4[i];
}

__global__ __launch_bounds__(kThreads) void copy_scalar_kernel(float* __restrict__ dst,
                                                               const float* __restrict__ src,
                                                               int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride)
        dst[i] = src[i];
}

// Two copies in one launch: blockIdx.y picks the copy. Each is done as
// above, 128-bit where its two pointers share their 16-byte phase (vec),
// 32-bit otherwise; a copy whose grid is smaller leaves the extra blocks idle.
struct CopyJob {
    float* dst;
    const float* src;
    int64_t head, n4, count;
    int32_t vec;
};

__global__ __launch_bounds__(kThreads) void copy_pair_kernel(CopyJob a, CopyJob b) {
    const CopyJob& j = blockIdx.y == 0 ? a : b;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    if (!j.vec) {
        for (int64_t i = tid; i < j.count; i += stride) j.dst[i] = j.src[i];
        return;
    }
    if (tid < j.head) j.dst[tid] = j.src[tid];
    const int64_t tail_start = j.head + j.n4 * 4;
    if (tid < j.count - tail_start) j.dst[tail_start + tid] = j.src[tail_start + tid];
    const float4* s4 = reinterpret_cast<const float4*>(j.src + j.head);
    float4* d4 = reinterpret_cast<float4*>(j.dst + j.head);
    for (int64_t i = tid; i < j.n4; i += stride) d4[i] = s4[i];
}

__global__ __launch_bounds__(kThreads) void zero_fill_kernel(float* __restrict__ dst,
                                                             int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride)
        dst[i] = 0.0f;
}

int64_t blocks_for(int64_t items) {
    int64_t b = (items + kThreads - 1) / kThreads;
    if (b < 1) b = 1;
    return b < kMaxBlocks ? b : kMaxBlocks;
}

}  // namespace

hipError_t launch_cache_write(float* dst, const float* src, int64_t count, const Launch& L) {
    if (count <= 0) return hipSuccess;
    const uintptr_t da = reinterpret_cast<uintptr_t>(dst), sa = reinterpret_cast<uintptr_t>(src);
    if ((da & 15u) == (sa & 15u)) {
        int64_t head = (int64_t)(((16u - (da & 15u)) & 15u) / 4u);
        if (head > count) head = count;
        const int64_t n4 = (count - head) / 4;
        return launch_kernel(copy_vec4_kernel, dim3((unsigned)blocks_for(n4 > 4 ? n4 : 4)),
                             dim3(kThreads), 0, L, dst, src, head, n4, count);
    }
    return launch_kernel(copy_scalar_kernel, dim3((unsigned)blocks_for(count)), dim3(kThreads), 0,
                         L, dst, src, count);
}

hipError_t launch_cache_write_pair(float* dst_a, const float* src_a, int64_t count_a, float* dst_b,
                                   const float* src_b, int64_t count_b, const Launch& L) {
    auto job = [](float* dst, const float* src, int64_t count, int64_t* items) {
        CopyJob j{dst, src, 0, 0, count, 0};
        const uintptr_t da = reinterpret_cast<uintptr_t>(dst), sa = reinterpret_cast<uintptr_t>(src);
        if ((da & 15u) == (sa & 15u)) {
            j.vec = 1;
            j.head = (int64_t)(((16u - (da & 15u)) & 15u) / 4u);
            if (j.head > count) j.head = count;
            j.n4 = (count - j.head) / 4;
            *items = j.n4 > 4 ? j.n4 : 4;
        } else {
            *items = count;
        }
        return j;
    };
    int64_t ia = 0, ib = 0;
    const CopyJob a = job(dst_a, src_a, count_a, &ia), b = job(dst_b, src_b, count_b, &ib);
    return launch_kernel(copy_pair_kernel, dim3((unsigned)blocks_for(ia > ib ? ia : ib), 2), dim3(kThreads), 0, L,
                         a, b);
}

hipError_t launch_zero_fill(float* dst, int64_t count, const Launch& L) {
    if (count <= 0) return hipSuccess;
    return launch_kernel(zero_fill_kernel, dim3((unsigned)blocks_for(count)), dim3(kThreads), 0, L,
                         dst, count);
}

}  // namespace attn
