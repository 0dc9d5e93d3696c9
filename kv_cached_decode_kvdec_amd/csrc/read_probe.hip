// Streaming-read probe for counter calibration (libkvdec_probe.so; not part
// of the decode library's ABI).  It reads a buffer of known size once with
// the same nontemporal 16-byte loads the attend kernels use for K/V rows,
// so that rocprofv3's FETCH_SIZE can be scaled to bytes for exactly that
// load form.  Each workgroup folds what it read into one word (so the loads
// cannot be dropped) and stores it to sink[blockIdx.x]: the probe reads
// `bytes` and writes 4 bytes per workgroup.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                              size_t n16,
                                                              unsigned int* __restrict__ sink)
{
    unsigned int acc = 0;
    for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16;
         i += static_cast<size_t>(gridDim.x) * kThreads) {
        const u32x4 w = __builtin_nontemporal_load(src + i);
        acc ^= w.x ^ w.y ^ w.z ^ w.w;
    }
    __shared__ unsigned int red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (static_cast<int>(threadIdx.x) < s) red[threadIdx.x] ^= red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

extern "C" __attribute__((visibility("default")))
int kvdec_probe_stream_read(const void* src, size_t bytes, unsigned int* sink, int blocks,
                            void* stream)
{
    if (!src || !sink || blocks < 1 || (reinterpret_cast<uintptr_t>(src) & 15u) || (bytes & 15u))
        return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                       sink);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}
