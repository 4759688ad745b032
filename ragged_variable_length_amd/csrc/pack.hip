// Pack (count + prefix-sum, then gather) and unpack kernels.
//
// Packing follows the two-phase packer of "Dispatch-Aware Ragged Attention
// for Pruned Vision Transformers" (aissential.tech summary, "Method"): a
// small phase that turns the keep-mask into per-image counts and offsets,
// then a gather of the kept token rows into one contiguous ragged buffer.
// Unpacking returns rows to the padded layout (sota2.com page, Abstract).
// Both are pure byte movement: a token row is H * 64 elements, copied in
// 16-byte pieces so every load and store is a full 128-bit access.
#include "rva_device.h"
#include "rva_internal.h"

namespace rva {

__global__ __launch_bounds__(kScanThreads) void count_scan_kernel(const uint8_t* __restrict__ mask,
                                                                  int B, int N,
                                                                  int32_t* __restrict__ cu,
                                                                  int32_t* __restrict__ max_out) {
  __shared__ int lds[4 * kScanThreads + 64];
  count_scan_block<kScanThreads>(mask, B, N, cu, max_out, lds);
}

// Copies `count` rows of `pieces` 16-byte pieces.  src_row(r) / dst_row(r)
// give byte offsets of row r; a negative source offset writes zeros.  Four
// pieces per thread are loaded before any is stored so that several
// loads are in flight per thread.  Stores are non-temporal: every
// destination byte is written once and not read back by the launch
// (measured: the 1024-image unpack 123 -> 68 us, the pack 249 -> 233 us).
template <int NT, typename SrcRow, typename DstRow>
__device__ __forceinline__ void copy_rows(const char* __restrict__ src, char* __restrict__ dst,
                                          int pieces, int count, SrcRow src_row, DstRow dst_row) {
  const int total = count * pieces;
  for (int e0 = threadIdx.x; e0 < total; e0 += NT * 4) {
    u32x4 val[4];
    long long doff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * NT;
      doff[u] = -1;
      val[u] = u32x4{0u, 0u, 0u, 0u};
      if (e < total) {
        const int r = e / pieces, pc = e - r * pieces;
        const long long so = src_row(r);
        doff[u] = dst_row(r) + (long long)pc * 16;
        if (so >= 0) val[u] = *reinterpret_cast<const u32x4*>(src + so + (long long)pc * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (doff[u] >= 0) __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4*>(dst + doff[u]));
  }
}

// Gather: workgroup (b, s) compacts mask row b and copies its share of the
// kept rows of q/k/v (split s of gridDim.y) to rows cu[b] + r.
__global__ __launch_bounds__(kPackThreads) void pack_kernel(CopyParams p) {
  __shared__ int32_t idx[1024];
  __shared__ int32_t cnt[16];
  const int b = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  const int N = p.N;
  const int n = compact_row<kPackThreads>(p.mask + (size_t)b * N, N, idx, nullptr, nullptr, cnt);
  const int per = (n + S - 1) / S;
  const int r0 = min(n, s * per), r1 = min(n, r0 + per);
  if (r1 <= r0) return;
  const int cu_b = p.cu[b];
  if (p.kept_index)
    for (int r = r0 + (int)threadIdx.x; r < r1; r += kPackThreads) p.kept_index[cu_b + r] = b * N + idx[r];
  const long long R = p.row_bytes;
  const int pieces = p.row_bytes / 16;
  for (int t = 0; t < 3; ++t) {
    if (!p.src[t]) continue;
    copy_rows<kPackThreads>(
        static_cast<const char*>(p.src[t]), static_cast<char*>(p.dst[t]), pieces, r1 - r0,
        [&](int r) { return ((long long)b * N + idx[r0 + r]) * R; },
        [&](int r) { return (long long)(cu_b + r0 + r) * R; });
  }
}

// Scatter back: workgroup (b, s) covers padded positions of split s of image
// b; kept positions receive packed row cu[b] + rank, pruned positions zeros.
__global__ __launch_bounds__(kPackThreads) void unpack_kernel(CopyParams p) {
  __shared__ int32_t idx[1024];
  __shared__ int32_t rank[1024];
  __shared__ int32_t cnt[16];
  const int b = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  const int N = p.N;
  compact_row<kPackThreads>(p.mask + (size_t)b * N, N, idx, rank, nullptr, cnt);
  const int per = (N + S - 1) / S;
  const int j0 = min(N, s * per), j1 = min(N, j0 + per);
  if (j1 <= j0) return;
  const int cu_b = p.cu[b];
  const long long R = p.row_bytes;
  copy_rows<kPackThreads>(
      static_cast<const char*>(p.src[0]), static_cast<char*>(p.dst[0]), p.row_bytes / 16, j1 - j0,
      [&](int r) {
        const int rk = rank[j0 + r];
        return rk >= 0 ? (long long)(cu_b + rk) * R : -1ll;
      },
      [&](int r) { return ((long long)b * N + j0 + r) * R; });
}

__global__ void empty_kernel() {}

hipError_t launch_count_scan(const uint8_t* mask, int B, int N, int32_t* cu, int32_t* max_out,
                             hipStream_t s) {
  hipLaunchKernelGGL(count_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, mask, B, N, cu, max_out);
  return hipGetLastError();
}

hipError_t launch_pack(const CopyParams& p, int splits, hipStream_t s) {
  hipLaunchKernelGGL(pack_kernel, dim3(p.B, splits), dim3(kPackThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_unpack(const CopyParams& p, int splits, hipStream_t s) {
  hipLaunchKernelGGL(unpack_kernel, dim3(p.B, splits), dim3(kPackThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_empty(hipStream_t s) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
}

}  // namespace rva
