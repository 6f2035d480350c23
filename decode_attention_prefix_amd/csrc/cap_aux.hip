// cap_aux.hip -- gfx950 kernels of libcap off the attention hot path: the
// per-step growth of the KV pools and of an uploaded plan (append_kernel,
// patch_kernel), and the measurement kernels of cap_bench.h (fill, cached
// read, streaming read probe, copy, streaming copy probe).
#include <hip/hip_runtime.h>

#include "cap_internal.h"

namespace cap {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Plan patch: word patch[2i] of the plan buffer takes the value patch[2i+1].
__global__ __launch_bounds__(256) void patch_kernel(uint32_t *base, const uint32_t *patch, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) base[patch[2 * i]] = patch[2 * i + 1];
}

// New tokens' K/V into their pool slots: one lane per (token, KV head,
// 8-dim chunk).  K: the chunk is one 16-byte piece of the page block; V:
// eight 2-byte values, one per dim row of the block.  The K/V loads do not
// depend on the destination, so all three loads are in flight together.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a)
{
    const int chunks = a.D / 8;
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= a.n * a.Hkv * chunks) return;
    const int c = t % chunks, h = (t / chunks) % a.Hkv, i = t / (chunks * a.Hkv);
    const int64_t src = ((int64_t)i * a.Hkv + h) * a.D + c * 8;
    const u32x4 k = *reinterpret_cast<const u32x4 *>(a.k_new + src);
    const u32x4 v = *reinterpret_cast<const u32x4 *>(a.v_new + src);
    const int32_t e = a.dest[i];
    if (e < 0 || (int64_t)(e >> 4) >= a.pool_pages) return;
    const int64_t blk = (int64_t)(e >> 4) * a.Hkv + h;
    const int slot = e & 15;
    *reinterpret_cast<u32x4 *>(a.k_pool + ((blk * chunks + c) * kPage + slot) * 8) = k;
    uint16_t *vd = a.v_pool + (blk * a.D + c * 8) * kPage + slot;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) vd[j * kPage] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
}

__global__ __launch_bounds__(256) void fill_kernel(uint32_t *buf, size_t words, uint32_t value)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride)
        buf[i] = value;
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4 *buf, size_t n, uint32_t *sink)
{
    // four independent 16-byte loads in flight per lane per iteration
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t x = 0;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 v0 = buf[i], v1 = buf[i + stride], v2 = buf[i + 2 * stride], v3 = buf[i + 3 * stride];
        x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
        x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
    for (; i < n; i += stride) {
        const u32x4 v = buf[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
        for (int k = 0; k < 256; ++k) y ^= red[k];
        sink[blockIdx.x] = y;
    }
}

// The achievable-read probe: each workgroup streams contiguous 256 KB runs
// (the decode kernel's access shape), eight non-temporal 16-byte loads in
// flight per lane -- the fastest of the read shapes measured on the device
// (grid-stride, per-workgroup runs of 64 KB to 1 MB, 4 or 8 loads in flight,
// plain or non-temporal).
constexpr size_t kStreamRun = 16384;               // 16-byte vectors per run (256 KB)

__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4 *buf, size_t n, uint32_t *sink)
{
    constexpr int K = 8;
    uint32_t x = 0;
    for (size_t base = (size_t)blockIdx.x * kStreamRun; base < n; base += (size_t)gridDim.x * kStreamRun) {
        const size_t end = base + kStreamRun < n ? base + kStreamRun : n;
        size_t i = base + threadIdx.x;
        for (; i + (K - 1) * 256 < end; i += K * 256) {
            u32x4 v[K];
#pragma unroll
            for (int k = 0; k < K; ++k) v[k] = __builtin_nontemporal_load(&buf[i + k * 256]);
#pragma unroll
            for (int k = 0; k < K; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
        }
        for (; i < end; i += 256) {
            const u32x4 v = buf[i];
            x ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
        for (int k = 0; k < 256; ++k) y ^= red[k];
        sink[blockIdx.x] = y;
    }
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4 *dst, const u32x4 *src, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

// The achievable read-plus-write probe: workgroup b copies runs b, b + grid,
// ... of `run` 16-byte vectors each, eight non-temporal 16-byte loads in
// flight per lane, written back with non-temporal stores (the access shape
// of a kernel that streams rows through registers).
__global__ __launch_bounds__(256) void copy_stream_kernel(u32x4 *dst, const u32x4 *src, size_t n, size_t run)
{
    constexpr int K = 8;
    for (size_t base = (size_t)blockIdx.x * run; base < n; base += (size_t)gridDim.x * run) {
        const size_t end = base + run < n ? base + run : n;
        size_t i = base + threadIdx.x;
        for (; i + (K - 1) * 256 < end; i += K * 256) {
            u32x4 v[K];
#pragma unroll
            for (int k = 0; k < K; ++k) v[k] = __builtin_nontemporal_load(&src[i + k * 256]);
#pragma unroll
            for (int k = 0; k < K; ++k) __builtin_nontemporal_store(v[k], &dst[i + k * 256]);
        }
        for (; i < end; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
    }
}

}  // namespace

static unsigned grid_for(size_t n)
{
    size_t g = (n + 255) / 256;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    return (unsigned)g;
}

int launch_fill(void *buf, size_t words, uint32_t value, void *stream)
{
    hipLaunchKernelGGL(fill_kernel, dim3(grid_for(words)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), (uint32_t *)buf, words, value);
    return (int)hipGetLastError();
}

int launch_patch(void *base, const uint32_t *patch, int n, void *stream)
{
    if (n <= 0) return 0;
    hipLaunchKernelGGL(patch_kernel, dim3((n + 255) / 256), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), (uint32_t *)base, patch, n);
    return (int)hipGetLastError();
}

int launch_append(const AppendArgs &a, void *stream)
{
    const int lanes = a.n * a.Hkv * (a.D / 8);
    if (lanes <= 0) return 0;
    hipLaunchKernelGGL(append_kernel, dim3((lanes + 255) / 256), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

int launch_read(const void *buf, size_t vec16, void *sink, void *stream)
{
    hipLaunchKernelGGL(read_kernel, dim3(grid_for(vec16)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), (const u32x4 *)buf, vec16,
                       (uint32_t *)sink);
    return (int)hipGetLastError();
}

int launch_read_stream(const void *buf, size_t vec16, void *sink, void *stream)
{
    size_t g = (vec16 + kStreamRun - 1) / kStreamRun;
    g = g > 512 ? 512 : (g < 1 ? 1 : g);             // sink holds >= 8192 words
    hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)g), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), (const u32x4 *)buf, vec16, (uint32_t *)sink);
    return (int)hipGetLastError();
}

int launch_copy(void *dst, const void *src, size_t vec16, void *stream)
{
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(vec16)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), (u32x4 *)dst, (const u32x4 *)src,
                       vec16);
    return (int)hipGetLastError();
}

int launch_copy_stream(void *dst, const void *src, size_t vec16, size_t run16, void *stream)
{
    // one workgroup per run, up to 8192 workgroups (32 per CU); longer inputs
    // loop over their runs
    size_t g = (vec16 + run16 - 1) / run16;
    g = g > 8192 ? 8192 : (g < 1 ? 1 : g);
    hipLaunchKernelGGL(copy_stream_kernel, dim3((unsigned)g), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), (u32x4 *)dst, (const u32x4 *)src, vec16, run16);
    return (int)hipGetLastError();
}

const char *hip_error_string(int err)
{
    return hipGetErrorString((hipError_t)err);
}
}  // namespace cap
