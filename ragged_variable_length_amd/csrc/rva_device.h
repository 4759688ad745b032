// Device helpers shared by the pack, unpack and attention kernels:
// wave/workgroup reductions and scans, and the per-image row compaction that
// turns a keep-mask row into the ascending list of kept token positions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rva {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Workgroup-wide inclusive scan of one int per thread.  `tmp` holds at least
// (blockDim.x / 64) ints.  Returns the inclusive prefix; *total receives the
// sum over the workgroup.  Contains two barriers; every thread must call it.
template <int NT>
__device__ int block_inclusive_scan(int v, int* tmp, int* total) {
  constexpr int W = NT / 64;
  const int lane = lane_id(), w = wave_id();
  int incl = wave_inclusive_scan(v);
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    int t = tmp[i];
    before += (i < w) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl;
}

template <int NT>
__device__ int block_max(int v, int* tmp) {
  constexpr int W = NT / 64;
  v = wave_max(v);
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  int m = tmp[0];
#pragma unroll
  for (int i = 1; i < W; ++i) m = max(m, tmp[i]);
  __syncthreads();
  return m;
}

// Kept counts of every image and their exclusive prefix (cu_seqlens), plus
// the largest count, computed by ONE workgroup of NT threads.  Images are
// taken NT at a time: each wave counts whole mask rows (lanes stride the
// row), then the workgroup scans the NT counts and carries the total into
// the next group.  `lds` holds at least NT + 64 ints.
template <int NT>
__device__ void count_scan_block(const uint8_t* __restrict__ mask, int B, int N,
                                 int32_t* __restrict__ cu, int32_t* __restrict__ max_out,
                                 int* lds) {
  constexpr int W = NT / 64;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  int* cnt = lds;
  int* tmp = lds + NT;
  if (tid == 0 && cu) cu[0] = 0;
  int carry = 0, mx = 0;
  for (int base = 0; base < B; base += NT) {
    const int nimg = min(NT, B - base);
    for (int i = w; i < nimg; i += W) {
      const uint8_t* row = mask + (size_t)(base + i) * N;
      int c = 0;
      for (int j = lane; j < N; j += 64) c += row[j] != 0;
      c = wave_sum(c);
      if (lane == 0) cnt[i] = c;
    }
    __syncthreads();
    const int v = tid < nimg ? cnt[tid] : 0;
    int total;
    const int incl = block_inclusive_scan<NT>(v, tmp, &total);
    if (cu && tid < nimg) cu[base + tid + 1] = carry + incl;
    mx = max(mx, block_max<NT>(v, tmp));
    carry += total;
  }
  if (tid == 0 && max_out) *max_out = mx;
}

// Row compaction: for one image's mask row (N <= 1024 bytes) build the
// ascending list of kept positions idx[0..n) in LDS and return n (the same
// value in every thread).  Each wave takes 64-token chunks; a ballot gives
// every kept lane its rank inside the chunk, a prefix over the (at most 16)
// chunk counts gives the chunk's base.  Optionally stores rank[j] (-1 for a
// pruned token) and the per-chunk ballots.  `cnt` holds 16 ints.  Contains
// two barriers; every thread must call it.
template <int NT>
__device__ int compact_row(const uint8_t* __restrict__ mrow, int N, int32_t* idx, int32_t* rank,
                           uint64_t* ballots, int32_t* cnt) {
  constexpr int W = NT / 64;
  constexpr int PER = (16 + W - 1) / W;  // chunks per wave (N <= 1024)
  const int lane = lane_id(), w = wave_id();
  const int nchunks = (N + 63) >> 6;
  uint64_t bal[PER];
  bool keep[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = w + i * W;
    const int j = c * 64 + lane;
    keep[i] = (c < nchunks) && (j < N) && (mrow[j] != 0);
    bal[i] = __ballot(keep[i]);
    if (c < nchunks && lane == 0) {
      cnt[c] = __popcll(bal[i]);
      if (ballots) ballots[c] = bal[i];
    }
  }
  __syncthreads();
  int n = 0;
  for (int c = 0; c < nchunks; ++c) n += cnt[c];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = w + i * W;
    if (c < nchunks) {
      int base = 0;
      for (int cc = 0; cc < c; ++cc) base += cnt[cc];
      const int j = c * 64 + lane;
      const int r = base + __popcll(bal[i] & lanemask_lt());
      if (keep[i]) idx[r] = j;
      if (rank && j < N) rank[j] = keep[i] ? r : -1;
    }
  }
  __syncthreads();
  return n;
}

}  // namespace rva
