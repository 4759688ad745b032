// Ceiling probes: what this device reaches on plain streaming and on dense
// matrix-core work, measured with kernels of this library rather than a
// vendor library's, so that a kernel's fraction of "achievable" has a
// denominator of known construction.  Not part of the attention path.
//
//  - copy: every thread moves 16-byte pieces over a grid-stride loop with
//    non-temporal loads and stores (bytes read + written);
//  - read: non-temporal 16-byte loads, kReadUnroll in flight per thread,
//    folded into a per-thread XOR and one 4-byte store per thread to a sink
//    (bytes read; the sink's writes are negligible);
//  - mfma: independent 16x16x32 fp16 matrix-core products on register
//    operands, kMfmaChains accumulators per wave so consecutive products do
//    not wait on each other; one store per lane at the end.
// Measured on MI355X over 1 GiB, the best of the shapes tried: the copy at
// one piece in flight and 4 workgroups of 256 threads per CU (about 5.97
// TB/s read + written), the read at four in flight and 2 workgroups per CU
// (about 7.07 TB/s); plain loads and stores, and deeper unrolls, stayed at
// 4.3-5.5 TB/s.  The matrix cores reach about 2.19 PFLOP/s with 8 waves
// per SIMD.
#include "rva_device.h"
#include "rva_internal.h"

namespace rva {

constexpr int kProbeThreads = 256;
constexpr int kReadUnroll = 4;
constexpr int kMfmaChains = 8;

typedef _Float16 f16x8p __attribute__((ext_vector_type(8)));
typedef float f32x4p __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   long long n) {
  const long long stride = (long long)gridDim.x * kProbeThreads;
  for (long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                                   uint32_t* __restrict__ sink,
                                                                   long long n) {
  const long long stride = (long long)gridDim.x * kProbeThreads;
  long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(&src[i]);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeThreads, 8) void probe_mfma_kernel(int iters, float* __restrict__ out) {
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
