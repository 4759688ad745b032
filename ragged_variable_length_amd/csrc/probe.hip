// Ceiling probes: what this device reaches on plain streaming and on dense
// matrix-core work, measured with kernels of this library rather than a
// vendor library's, so that a kernel's fraction of "achievable" has a
// denominator of known construction.  Not part of the attention path.
//
//  - copy: every thread moves 16-byte pieces, kCopyUnroll loads in flight
//    before their stores, over a grid-stride loop (bytes read + written);
//  - read: the same loads, folded into a per-thread XOR and one 4-byte store
//    per thread to a sink (bytes read; the sink's writes are negligible);
//  - mfma: independent 16x16x32 fp16 matrix-core products on register
//    operands, kMfmaChains accumulators per wave so consecutive products do
//    not wait on each other; one store per lane at the end.
#include "rva_device.h"
#include "rva_internal.h"

namespace rva {

constexpr int kProbeThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kMfmaChains = 8;

typedef _Float16 f16x8p __attribute__((ext_vector_type(8)));
typedef float f32x4p __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   long long n) {
  const long long stride = (long long)gridDim.x * kProbeThreads;
  long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * stride < n; i += kCopyUnroll * stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                                   uint32_t* __restrict__ sink,
                                                                   long long n) {
  const long long stride = (long long)gridDim.x * kProbeThreads;
  long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kCopyUnroll - 1) * stride < n; i += kCopyUnroll * stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += stride) acc ^= src[i][0] ^ src[i][1] ^ src[i][2] ^ src[i][3];
  sink[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  f16x8p a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(0.001f * (lane + j));
    b[j] = (_Float16)(0.002f * (lane - j));
  }
  f32x4p acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4p{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

hipError_t launch_probe_copy(const void* src, void* dst, long long pieces, int grid, hipStream_t s) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(grid), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), pieces);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, uint32_t* sink, long long pieces, int grid,
                             hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(src), sink, pieces);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, float* out, int grid, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(kProbeThreads), 0, s, iters, out);
  return hipGetLastError();
}

int probe_threads() { return kProbeThreads; }
long long probe_mfma_flops(int iters, int grid) {
  // each wave's product per iteration and chain: 16 x 16 x 32 multiply-adds
  return (long long)iters * kMfmaChains * (kProbeThreads / 64) * grid * 16LL * 16 * 32 * 2;
}

}  // namespace rva
