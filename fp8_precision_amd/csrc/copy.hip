// copy.hip -- a plain streaming copy, the achievable-bandwidth reference that the
// quantisation and statistic kernels are measured against.  It is no step of the
// FP8 method; it exists so that "fraction of what a copy reaches" is taken
// against a copy built the way those kernels are built.
//
// Shape, measured on MI355X (a copy of 256 MiB each way after a 1 GiB read, so
// that nothing is cached): the rate is set by the bytes in flight, and peaks at
// about 4 MiB of loads over the chip (6.9-7.0 TB/s counting both directions);
// 1-2 MiB cannot cover the latency, 16-64 MiB fall to 4.5-6.6 TB/s.  Two
// blocks of 512 lanes per CU with one 16-byte load each hold 4 MiB on 256 CUs.
// Loads are non-temporal (the source is not read again), stores plain.
#include "fp8_internal.hpp"

namespace fp8k {

typedef unsigned int cp_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 512;
constexpr int kCopyBlocksPerCu = 2;

__global__ void __launch_bounds__(kCopyThreads) stream_copy_kernel(const cp_u32x4* __restrict__ src,
                                                                   cp_u32x4* __restrict__ dst, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * kCopyThreads;
    for (size_t i = (size_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n16; i += stride)
        dst[i] = __builtin_nontemporal_load(src + i);
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream)
{
    const size_t n16 = (size_t)bytes / 16;
    const size_t blocks_needed = (n16 + kCopyThreads - 1) / kCopyThreads;
    const size_t grid = std::min<size_t>((size_t)kCopyBlocksPerCu * device_cu_count(), blocks_needed);
    return launch(stream_copy_kernel, dim3((unsigned)grid), dim3(kCopyThreads), stream,
                  static_cast<const cp_u32x4*>(src), static_cast<cp_u32x4*>(dst), n16);
}

}  // namespace fp8k
