// bwprobe.hip -- HBM bandwidth probes for gfx950: the access pattern of the replay kernels'
// checkpoint stream without their arithmetic. Each 256-thread work-group moves one contiguous
// 32 KiB chunk (the size of one fp32 (sequence, head) tile at P = 64, N = 128) with 16-byte
// non-temporal accesses, eight per lane issued back to back. Measurement infrastructure for the
// benchmark's ceiling figures; not part of the replay path.
#include <hip/hip_runtime.h>

#include <stddef.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPer = 8;                                        // 16-byte accesses per lane
constexpr size_t kChunk = (size_t)kThreads * kPer * 16;        // 32 KiB per work-group

// Read: every lane sums its eight 16-byte values; one float per work-group is written (the sum
// keeps the loads live).
__global__ void __launch_bounds__(kThreads) read_kernel(const float *src, float *sink)
{
    const char *base = (const char *)src + blockIdx.x * kChunk;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    u32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        v[i] = __builtin_nontemporal_load((const u32x4 *)(base + ((size_t)i * kThreads + threadIdx.x) * 16));
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc += __builtin_bit_cast(f32x4, v[i]);
    float s = acc.x + acc.y + acc.z + acc.w;
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + threadIdx.x / 64] = s;
}

// Copy: each work-group's chunk to the same offset of dst.
__global__ void __launch_bounds__(kThreads) copy_kernel(const float *src, float *dst)
{
    const size_t off = blockIdx.x * kChunk;
    u32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        v[i] = __builtin_nontemporal_load((const u32x4 *)((const char *)src + off + ((size_t)i * kThreads + threadIdx.x) * 16));
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        __builtin_nontemporal_store(v[i], (u32x4 *)((char *)dst + off + ((size_t)i * kThreads + threadIdx.x) * 16));
}

// In-place read-modify-write: every value times `scale`.
__global__ void __launch_bounds__(kThreads) rmw_kernel(float *buf, float scale)
{
    char *base = (char *)buf + blockIdx.x * kChunk;
    f32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        v[i] = __builtin_bit_cast(f32x4, __builtin_nontemporal_load((const u32x4 *)(base + ((size_t)i * kThreads + threadIdx.x) * 16)));
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v[i] * scale),
                                    (u32x4 *)(base + ((size_t)i * kThreads + threadIdx.x) * 16));
}

}  // namespace

extern "C" {

// Bytes per work-group chunk; every size below must be a positive multiple of it.
size_t bwprobe_chunk_bytes(void) { return kChunk; }

// Read `bytes` of src (device, 16-byte aligned); sink holds bytes / 8192 floats. 0, or -1 for a
// bad size or pointer, or the HIP error of the launch.
int bwprobe_read(const float *src, size_t bytes, float *sink, void *stream)
{
    if (!src || !sink || bytes == 0 || bytes % kChunk || ((size_t)src & 15)) return -1;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)(bytes / kChunk)), dim3(kThreads), 0, (hipStream_t)stream, src, sink);
    return (int)hipGetLastError();
}

int bwprobe_copy(const float *src, float *dst, size_t bytes, void *stream)
{
    if (!src || !dst || bytes == 0 || bytes % kChunk || ((size_t)src & 15) || ((size_t)dst & 15)) return -1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)(bytes / kChunk)), dim3(kThreads), 0, (hipStream_t)stream, src, dst);
    return (int)hipGetLastError();
}

int bwprobe_rmw(float *buf, size_t bytes, float scale, void *stream)
{
    if (!buf || bytes == 0 || bytes % kChunk || ((size_t)buf & 15)) return -1;
    hipLaunchKernelGGL(rmw_kernel, dim3((unsigned)(bytes / kChunk)), dim3(kThreads), 0, (hipStream_t)stream, buf, scale);
    return (int)hipGetLastError();
}

}  // extern "C"
