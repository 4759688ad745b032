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
//    not wait on each other; one store per lane at the end;
//  - gather: the fused attention's HBM traffic with none of its arithmetic
//    (the kept rows' head slices of q, k and v read, every row of o
//    written), non-temporal loads and stores, the fastest policy for this
//    pattern measured (about 5% faster than default-policy loads): what
//    that access pattern alone reaches.
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

// Gather/scatter probe, one workgroup per (image, head pair) of padded
// 16-bit [B, N, H, 64] tensors (a last single head when H is odd): every
// 16-byte piece of the kept rows' slices of q, k and v is read (four
// pieces of each in flight per thread) and their XOR written to the same
// piece of o; the pruned rows' slices of o are written zero.  Loads and
// stores are non-temporal.  Offsets come
// from cu_seqlens and kept_index (padded row b * N + j of each kept
// token, capacity B * N); rows and counts outside the tensors are skipped,
// so every access stays in bounds whatever they hold.
constexpr int kGatherUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void probe_gather_kernel(
    const char* __restrict__ q, const char* __restrict__ k, const char* __restrict__ v,
    char* __restrict__ o, const uint8_t* __restrict__ mask, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ kidx, int B, int N, int H) {
  const int ng = (H + 1) >> 1;
  const int b = blockIdx.x / ng, hg = blockIdx.x - b * ng;
  const int per = (H - 2 * hg >= 2 ? 2 : 1) * (kHeadDim * 2 / 16);  // pieces of a row's slice
  const long long rs = (long long)H * kHeadDim * 2;                 // bytes of a token row
  const long long rows = (long long)B * N;
  const long long hb = (long long)hg * 2 * kHeadDim * 2;
  const int beg = cu[b];
  const int n = min(max(cu[b + 1] - beg, 0), N);
  if (beg >= 0 && beg <= rows - n) {
    const int total = n * per;
    for (int e0 = threadIdx.x; e0 < total; e0 += kProbeThreads * kGatherUnroll) {
      u32x4 a[kGatherUnroll];
      long long off[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const int e = e0 + u * kProbeThreads;
        off[u] = -1;
        if (e < total) {
          const int r = e / per, pc = e - r * per;
          const long long row = kidx[beg + r];
          if (row >= 0 && row < rows) {
            off[u] = row * rs + hb + pc * 16;
            a[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + off[u])) ^
                   __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off[u])) ^
                   __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off[u]));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u)
        if (off[u] >= 0) __builtin_nontemporal_store(a[u], reinterpret_cast<u32x4*>(o + off[u]));
    }
  }
  const uint8_t* mrow = mask + (long long)b * N;
  for (int e = threadIdx.x; e < N * per; e += kProbeThreads) {
    const int j = e / per, pc = e - j * per;
    if (!mrow[j])
      __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                  reinterpret_cast<u32x4*>(o + ((long long)b * N + j) * rs + hb + pc * 16));
  }
}

hipError_t launch_probe_gather(const void* q, const void* k, const void* v, void* o,
                               const uint8_t* mask, const int32_t* cu, const int32_t* kidx, int B,
                               int N, int H, hipStream_t s) {
  hipLaunchKernelGGL(probe_gather_kernel, dim3(B * ((H + 1) / 2)), dim3(kProbeThreads), 0, s,
                     static_cast<const char*>(q), static_cast<const char*>(k),
                     static_cast<const char*>(v), static_cast<char*>(o), mask, cu, kidx, B, N, H);
  return hipGetLastError();
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
