// Host side of the C ABI declared in include/rva.h: argument validation,
// launch geometry, thread-local error text and captured launch plans.
// The call paths only enqueue work: they neither allocate device memory nor
// synchronise with the device.  Plan creation is the exception: a persistent
// plan allocates its 8-byte work counter (hipMalloc) and zeroes it with a
// blocking hipMemset, and graph instantiation allocates in the runtime.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "rva.h"
#include "rva_probe.h"
#include "rva_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(RVA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t esize(int dtype) { return dtype == RVA_F32 ? 4 : 2; }

int check_shape(int B, int N, int H, int d, int dtype) {
  if (dtype != RVA_F32 && dtype != RVA_F16 && dtype != RVA_BF16)
    return fail(RVA_ERR_INVALID, "unknown dtype %d", dtype);
  if (B < 1) return fail(RVA_ERR_INVALID, "B must be >= 1 (got %d)", B);
  if (N < 1 || N > RVA_MAX_TOKENS)
    return fail(RVA_ERR_INVALID, "N must be in [1, %d] (got %d)", RVA_MAX_TOKENS, N);
  if (H < 1 || H > RVA_MAX_HEADS)
    return fail(RVA_ERR_INVALID, "H must be in [1, %d] (got %d)", RVA_MAX_HEADS, H);
  if ((long long)B * N >= (1ll << 31)) return fail(RVA_ERR_INVALID, "B*N must be < 2^31");
  if (d != RVA_HEAD_DIM) return fail(RVA_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", d);
  return RVA_OK;
}

int check_data(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(RVA_ERR_INVALID, "%s is NULL", name) : RVA_OK;
  if (!aligned(p, 16)) return fail(RVA_ERR_INVALID, "%s is not 16-byte aligned", name);
  return RVA_OK;
}

int check_i32(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(RVA_ERR_INVALID, "%s is NULL", name) : RVA_OK;
  if (!aligned(p, 4)) return fail(RVA_ERR_INVALID, "%s is not 4-byte aligned", name);
  return RVA_OK;
}

#define RVA_TRY(x)            \
  do {                        \
    int _s = (x);             \
    if (_s != RVA_OK) return _s; \
  } while (0)

std::once_flag g_init_once;
hipError_t g_init_err = hipSuccess;

int ensure_init() {
  std::call_once(g_init_once, [] {
    g_init_err = rva::attend_init();
    if (g_init_err == hipSuccess) g_init_err = rva::threshold_init();
  });
  if (g_init_err != hipSuccess) return hip_fail(g_init_err, "kernel set-up");
  return RVA_OK;
}

float resolve_scale(float s, int d) {
  if (!(s > 0.f)) s = 1.0f / sqrtf((float)d);
  return s * 1.4426950408889634f;  // fold log2(e) so the kernel uses exp2
}

// Row splits for the copy kernels: enough workgroups that their loads in
// flight cover the device's memory latency (4096, about 16 per CU, measured
// best on the 1024-image batch), each keeping at least 16 rows.
int copy_splits(int B, int N) {
  int s = 1;
  while (s < 8 && B * s < 4096 && (N / (s * 2)) >= 16) s *= 2;
  return s;
}

// ---- validated argument bundles (validation never launches anything)

struct PackArgs {
  rva::CopyParams cp;
  int32_t* max_seqlen;
  int splits;
};

int validate_pack(const void* q_pad, const void* k_pad, const void* v_pad, const uint8_t* mask,
                  int B, int N, int H, int d, int dtype, void* q_out, void* k_out, void* v_out,
                  int32_t* cu, int32_t* max_seqlen, int32_t* kept_index, PackArgs* out) {
  RVA_TRY(check_shape(B, N, H, d, dtype));
  if (!mask) return fail(RVA_ERR_INVALID, "mask is NULL");
  const void* in[3] = {q_pad, k_pad, v_pad};
  void* outp[3] = {q_out, k_out, v_out};
  const char* nin[3] = {"q_pad", "k_pad", "v_pad"};
  const char* nout[3] = {"q_out", "k_out", "v_out"};
  for (int t = 0; t < 3; ++t) {
    if ((in[t] == nullptr) != (outp[t] == nullptr))
      return fail(RVA_ERR_INVALID, "%s and %s must both be given or both be NULL", nin[t], nout[t]);
    RVA_TRY(check_data(in[t], nin[t], false));
    RVA_TRY(check_data(outp[t], nout[t], false));
  }
  RVA_TRY(check_i32(cu, "cu_seqlens", true));
  RVA_TRY(check_i32(max_seqlen, "max_seqlen", false));
  RVA_TRY(check_i32(kept_index, "kept_index", false));
  rva::CopyParams& p = out->cp;
  for (int t = 0; t < 3; ++t) {
    p.src[t] = in[t];
    p.dst[t] = outp[t];
  }
  p.mask = mask;
  p.cu = cu;
  p.kept_index = kept_index;
  p.B = B;
  p.N = N;
  p.row_bytes = (int)(H * d * esize(dtype));
  out->max_seqlen = max_seqlen;
  // splits only help copies: an index-only pack (no rows) takes one
  // workgroup per image, each compacting its mask row once
  out->splits = (in[0] || in[1] || in[2]) ? copy_splits(B, N) : 1;
  return RVA_OK;
}

int enqueue_pack(const PackArgs& a, hipStream_t s) {
  hipError_t e = rva::launch_count_scan(a.cp.mask, a.cp.B, a.cp.N, const_cast<int32_t*>(a.cp.cu),
                                        a.max_seqlen, s);
  if (e != hipSuccess) return hip_fail(e, "count/scan launch");
  bool any = a.cp.src[0] || a.cp.src[1] || a.cp.src[2] || a.cp.kept_index;
  if (any) {
    e = rva::launch_pack(a.cp, a.splits, s);
    if (e != hipSuccess) return hip_fail(e, "pack launch");
  }
  return RVA_OK;
}

int validate_attend(const void* q, const void* k, const void* v, const int32_t* cu, int B, int H,
                    int d, int max_seqlen, float scale, int dtype, void* o, rva::AttnParams* p) {
  RVA_TRY(check_shape(B, 1, H, d, dtype));
  RVA_TRY(check_data(q, "q", true));
  RVA_TRY(check_data(k, "k", true));
  RVA_TRY(check_data(v, "v", true));
  RVA_TRY(check_data(o, "o", true));
  RVA_TRY(check_i32(cu, "cu_seqlens", true));
  if (max_seqlen > RVA_MAX_TOKENS)
    return fail(RVA_ERR_INVALID, "max_seqlen must be at most %d (got %d)", RVA_MAX_TOKENS,
                max_seqlen);
  memset(p, 0, sizeof(*p));
  p->q = q;
  p->k = k;
  p->v = v;
  p->o = o;
  p->cu = cu;
  p->B = B;
  p->N = 0;
  p->H = H;
  p->nbound = max_seqlen > 0 ? max_seqlen : RVA_MAX_TOKENS;
  p->scale_log2e = resolve_scale(scale, d);
  return RVA_OK;
}

int validate_unpack(const void* o_packed, const int32_t* cu, const uint8_t* mask, int B, int N,
                    int H, int d, int dtype, void* o_pad, PackArgs* out) {
  RVA_TRY(check_shape(B, N, H, d, dtype));
  if (!mask) return fail(RVA_ERR_INVALID, "mask is NULL");
  RVA_TRY(check_data(o_packed, "o_packed", true));
  RVA_TRY(check_data(o_pad, "o_pad", true));
  RVA_TRY(check_i32(cu, "cu_seqlens", true));
  rva::CopyParams& p = out->cp;
  memset(&p, 0, sizeof(p));
  p.src[0] = o_packed;
  p.dst[0] = o_pad;
  p.mask = mask;
  p.cu = cu;
  p.B = B;
  p.N = N;
  p.row_bytes = (int)(H * d * esize(dtype));
  out->max_seqlen = nullptr;
  out->splits = copy_splits(B, N);
  return RVA_OK;
}

int validate_fused(const void* q, const void* k, const void* v, const uint8_t* mask, int B, int N,
                   int H, int d, int hint, float scale, int dtype, void* o, int32_t* cu,
                   int32_t* max_seqlen, rva::AttnParams* p) {
  RVA_TRY(check_shape(B, N, H, d, dtype));
  if (!mask) return fail(RVA_ERR_INVALID, "mask is NULL");
  RVA_TRY(check_data(q, "q_pad", true));
  RVA_TRY(check_data(k, "k_pad", true));
  RVA_TRY(check_data(v, "v_pad", true));
  RVA_TRY(check_data(o, "o_pad", true));
  RVA_TRY(check_i32(cu, "cu_seqlens", false));
  RVA_TRY(check_i32(max_seqlen, "max_seqlen", false));
  memset(p, 0, sizeof(*p));
  p->q = q;
  p->k = k;
  p->v = v;
  p->o = o;
  p->mask = mask;
  p->cu_out = cu;
  p->max_out = max_seqlen;
  p->B = B;
  p->N = N;
  p->H = H;
  p->nbound = hint > 0 && hint < N ? hint : N;
  p->scale_log2e = resolve_scale(scale, d);
  return RVA_OK;
}

struct ThreshArgs {
  rva::ThreshParams p;
  int B;
  int dtype;
};

int validate_threshold(const void* x, int B, int N, int C, int dtype, double keep_quantile,
                       uint8_t* mask_out, ThreshArgs* out) {
  if (dtype != RVA_F32 && dtype != RVA_F16 && dtype != RVA_BF16)
    return fail(RVA_ERR_INVALID, "unknown dtype %d", dtype);
  if (B < 1) return fail(RVA_ERR_INVALID, "B must be >= 1 (got %d)", B);
  if (N < 1 || N > RVA_MAX_TOKENS)
    return fail(RVA_ERR_INVALID, "N must be in [1, %d] (got %d)", RVA_MAX_TOKENS, N);
  if ((long long)B * N >= (1ll << 31)) return fail(RVA_ERR_INVALID, "B*N must be < 2^31");
  if (C < 1 || C > RVA_MAX_CHANNELS)
    return fail(RVA_ERR_INVALID, "C must be in [1, %d] (got %d)", RVA_MAX_CHANNELS, C);
  if ((C * esize(dtype)) % 16 != 0)
    return fail(RVA_ERR_INVALID, "C * element size must be a multiple of 16 bytes (C = %d)", C);
  if (!(keep_quantile >= 0.0 && keep_quantile <= 1.0))
    return fail(RVA_ERR_INVALID, "keep_quantile must lie in [0, 1]");
  RVA_TRY(check_data(x, "x", true));
  if (!mask_out) return fail(RVA_ERR_INVALID, "mask_out is NULL");
  const int P = N - 1;
  out->p.x = x;
  out->p.mask = mask_out;
  out->p.N = N;
  out->p.C = C;
  out->p.r0 = P >= 1 ? (int)ceil(keep_quantile * (double)(P - 1)) : 0;
  out->B = B;
  out->dtype = dtype;
  return RVA_OK;
}

int enqueue_threshold(const ThreshArgs& a, hipStream_t s) {
  RVA_TRY(ensure_init());
  hipError_t e = rva::launch_threshold(a.p, a.B, a.dtype, s);
  if (e != hipSuccess) return hip_fail(e, "keep-mask launch");
  return RVA_OK;
}

// ---- projections

int check_proj_shape(int B, int N, int C, int dtype) {
  if (dtype != RVA_F16 && dtype != RVA_BF16)
    return dtype == RVA_F32 ? fail(RVA_ERR_UNSUPPORTED, "projections take fp16 or bf16")
                            : fail(RVA_ERR_INVALID, "unknown dtype %d", dtype);
  if (B < 1) return fail(RVA_ERR_INVALID, "B must be >= 1 (got %d)", B);
  if (N < 1 || N > RVA_MAX_TOKENS)
    return fail(RVA_ERR_INVALID, "N must be in [1, %d] (got %d)", RVA_MAX_TOKENS, N);
  if (C < RVA_HEAD_DIM || C > RVA_MAX_HEADS * RVA_HEAD_DIM || C % RVA_HEAD_DIM != 0)
    return fail(RVA_ERR_INVALID, "C must be a multiple of 64 in [64, %d] (got %d)",
                RVA_MAX_HEADS * RVA_HEAD_DIM, C);
  // every row byte offset of the padded or packed buffers fits 31 bits
  if ((long long)B * N * C * 2 >= (1ll << 31))
    return fail(RVA_ERR_INVALID, "B*N*C*2 must be < 2^31");
  return RVA_OK;
}

void linear_grid(rva::LinearParams* p) {
  const int tm = rva::linear_tile_rows(), tn = rva::linear_tile_cols();
  p->m_tiles = (p->M + tm - 1) / tm;
  p->n_tiles = (p->Nout + tn - 1) / tn;
}

int validate_qkv(const void* x, const int32_t* kept_index, const int32_t* cu, int B, int N, int C,
                 const void* w, const void* b, int dtype, void* q, void* k, void* v,
                 rva::LinearParams* p) {
  RVA_TRY(check_proj_shape(B, N, C, dtype));
  RVA_TRY(check_data(x, "x", true));
  RVA_TRY(check_i32(kept_index, "kept_index", false));
  RVA_TRY(check_i32(cu, "cu_seqlens", true));
  RVA_TRY(check_data(w, "w_qkv", true));
  RVA_TRY(check_data(b, "b_qkv", false));
  RVA_TRY(check_data(q, "q", true));
  RVA_TRY(check_data(k, "k", true));
  RVA_TRY(check_data(v, "v", true));
  memset(p, 0, sizeof(*p));
  p->x = x;
  p->x_index = kept_index;
  p->x_rows = B * N;
  p->w = w;
  p->bias = b;
  p->y[0] = q;
  p->y[1] = k;
  p->y[2] = v;
  p->y_split = 3;
  p->m_count = cu + B;
  p->M = B * N;
  p->K = C;
  p->Nout = 3 * C;
  linear_grid(p);
  return RVA_OK;
}

int validate_outproj(const void* o, const int32_t* kept_index, const int32_t* cu,
                     const uint8_t* mask, int B, int N, int C, const void* w, const void* b,
                     const void* residual, int dtype, void* y, rva::LinearParams* p) {
  RVA_TRY(check_proj_shape(B, N, C, dtype));
  RVA_TRY(check_data(o, "o", true));
  RVA_TRY(check_i32(kept_index, "kept_index", false));
  RVA_TRY(check_i32(cu, "cu_seqlens", true));
  if (kept_index && !mask) return fail(RVA_ERR_INVALID, "mask is NULL (needed with kept_index)");
  RVA_TRY(check_data(w, "w_o", true));
  RVA_TRY(check_data(b, "b_o", false));
  RVA_TRY(check_data(residual, "residual", false));
  RVA_TRY(check_data(y, "y", true));
  memset(p, 0, sizeof(*p));
  p->x = o;
  p->x_rows = B * N;
  p->w = w;
  p->bias = b;
  p->residual = residual;
  p->y[0] = y;
  p->y_index = kept_index;
  p->y_split = 1;
  p->m_count = cu + B;
  p->M = B * N;
  p->K = C;
  p->Nout = C;
  if (kept_index) {
    p->zero_mask = mask;
    p->zero_rows = B * N;
  }
  linear_grid(p);
  return RVA_OK;
}

int enqueue_linear(const rva::LinearParams& p, int dtype, hipStream_t s) {
  hipError_t e = rva::launch_linear(p, dtype, s);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return RVA_OK;
}

// Compute units of the current device (cached per device).
int device_cus(int* out) {
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return RVA_OK;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device attribute");
  if (dev >= 0 && dev < 64) cache[dev] = cus;
  *out = cus;
  return RVA_OK;
}

// Query tiles per (sequence, head) forced on every later launch (0: each
// launch chooses); rva_set_query_split.
std::atomic<int> g_query_split{0};

// Work decomposition of an attention launch.  It does not change how an
// output row is computed in the whole-sequence and fp32 forms (identical
// bits); in the chunked form a query block's key-chunk order follows its
// workgroup pass, so its last bits may differ.
//  - Fused 16-bit launches whose (image, head pair) items fill every
//    resident slot (3 per CU) at least twice give a workgroup two heads of
//    one image, so the mask row is read and compacted once for both; the
//    images dispatched last (about one slot-fill of single heads) stay
//    unpaired, so the launch ends on short workgroups.
//  - Launches with fewer (sequence, head) items than resident slots split
//    each item into S query tiles, one workgroup each: as many tiles as
//    leave every wave at most one 16-query block (one pass of two blocks in
//    the streamed form), but no more than one slot-fill of workgroups needs
//    (four for the streamed form).  Otherwise most compute units would sit
//    idle while a few run whole sequences.
//  - fp32 takes one workgroup per 16-query block (its waves split the keys).
// The persistent form (`persistent`) never splits.  `items` (if not NULL)
// receives the grid positions of the work items.
int plan_grid(rva::AttnParams* p, int dtype, bool fused, bool persistent, long long* items) {
  p->heads_per_wg = 1;
  p->tail_b = 0;
  p->qsplit = 1;
  p->keysplit = 0;
  int cus = 0;
  RVA_TRY(device_cus(&cus));
  const long long slots = 3LL * cus;
  const long long bh = (long long)p->B * p->H;
  const int nqb = (p->nbound + rva::kQBlock - 1) / rva::kQBlock;  // blocks of the longest sequence
  const int forced = persistent ? 0 : g_query_split.load(std::memory_order_relaxed);
  if (dtype == RVA_F32) {
    p->qsplit = forced > 0 && forced < nqb ? forced : nqb;
  } else if (forced > 0) {
    p->qsplit = forced < nqb ? forced : nqb;
  } else if (fused && p->H > 1 && (long long)p->B * ((p->H + 1) / 2) >= 2 * slots) {
    p->heads_per_wg = 2;
    const long long t = (slots + p->H - 1) / p->H;
    p->tail_b = (int)(t < p->B ? t : p->B);
  } else if (!persistent && bh < slots) {
    const int rc = rva::attend_resident_rows(dtype, fused, p->N);
    const bool whole = p->nbound <= rc;
    if (whole && bh * nqb <= slots) {
      // one query block per workgroup still fits one slot-fill: its four
      // waves split the block's key tiles instead of walking them in turn
      p->qsplit = nqb;
      p->keysplit = 1;
    } else {
    const long long per = whole ? (nqb + 3) / 4 : (nqb + 7) / 8;
    // streamed sequences: one pass over the keys per workgroup is worth up to
    // four slot-fills of workgroups (a second pass re-streams every key for
    // the few blocks left over)
    const long long fill = ((whole ? 1 : 4) * slots + bh - 1) / bh;
    const long long q = per < fill ? per : fill;
    p->qsplit = q > 1 ? (int)q : 1;
    }
  }
  if (p->qsplit < 1) p->qsplit = 1;
  const long long n = rva::attend_grid_items(*p, dtype, fused);
  if (n >= (1ll << 31) - 1)
    return fail(RVA_ERR_INVALID, "attention launch of %lld workgroups exceeds the grid limit", n);
  if (items) *items = n;
  return RVA_OK;
}

// The persistent form's item counter is an int32 that reaches items + grid
// (every workgroup draws one index past the last item before it leaves);
// items and grid are each at most B*H, so B*H < 2^30 keeps it in range.
// Pure host arithmetic: it runs before anything touches the device.
int check_persistent_items(int B, int H) {
  if ((long long)B * H >= (1ll << 30))
    return fail(RVA_ERR_INVALID,
                "persistent form: B*H = %lld work items exceed its 32-bit counter (limit 2^30)",
                (long long)B * H);
  return RVA_OK;
}

int enqueue_attend_persistent(const rva::AttnParams& p0, int dtype, hipStream_t s) {
  RVA_TRY(ensure_init());
  rva::AttnParams p = p0;
  long long items = 0;
  RVA_TRY(plan_grid(&p, dtype, true, true, &items));
  int cus = 0;
  RVA_TRY(device_cus(&cus));
  long long grid = (long long)rva::attend_persistent_per_cu(p.N) * cus;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  if (items + grid >= (1ll << 31))  // excluded by check_persistent_items
    return fail(RVA_ERR_INVALID, "persistent form: %lld work items exceed its 32-bit counter",
                items);
  hipError_t e = rva::launch_attend_persistent(p, dtype, (int)grid, s);
  if (e != hipSuccess) return hip_fail(e, "persistent launch");
  return RVA_OK;
}

int enqueue_attend(const rva::AttnParams& p0, int dtype, bool fused, hipStream_t s) {
  RVA_TRY(ensure_init());
  rva::AttnParams p = p0;
  RVA_TRY(plan_grid(&p, dtype, fused, false, nullptr));
  hipError_t e = rva::launch_attend(p, dtype, fused, s);
  if (e != hipSuccess) return hip_fail(e, fused ? "fused launch" : "attention launch");
  return RVA_OK;
}

}  // namespace

// ---- device scratch of the allocation-free persistent entry point

// The persistent form's work counter pair [next item, workgroups done] for
// callers that cannot allocate device memory.  Every GPU the library runs on
// holds its own copy of this array (256 bytes) until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: only
// the address hipGetSymbolAddress returns for the current device may reach
// a kernel, a copy or a fill.
constexpr int kScratchInts = 64;
constexpr int kScratchCounterInts = 2;  // what one call uses: one counter pair
static_assert(kScratchCounterInts <= kScratchInts, "counter pair fits the scratch array");
static __device__ __align__(256) int32_t scratch[kScratchInts];

__global__ void zero_i32_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per device
bool g_scratch_cleared[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current.  The first call on a device also enqueues, on `s`, a
// fill kernel that zeroes the counter pair (a kernel rather than a memset,
// so that a caller may capture it in a graph); every completed persistent
// launch leaves the pair zero again for the next stream-ordered call.
int scratch_counter(hipStream_t s, int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RVA_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "scratch symbol address");
    if (!p) return fail(RVA_ERR_HIP, "scratch symbol address is NULL");
    g_scratch_dev[dev] = static_cast<int32_t*>(p);
  }
  if (!g_scratch_cleared[dev]) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, s, g_scratch_dev[dev],
                       kScratchCounterInts);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
    g_scratch_cleared[dev] = true;
  }
  *out = g_scratch_dev[dev];
  return RVA_OK;
}

}  // namespace

struct rva_plan_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
  int32_t* work;  // persistent mode: the plan's own work counter (device), else NULL
  // direct mode (no graph): the validated launch, enqueued as is
  bool direct;
  rva::AttnParams attn;
  int dtype;
};

namespace {

// Captures the launches `enqueue(stream)` makes on a private stream and
// instantiates them as a plan.  Nothing runs on the device here.
template <typename F>
int capture_plan(rva_plan* out, F enqueue) {
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "capture stream");
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return hip_fail(e, "begin capture");
  }
  const int st = enqueue(cs);
  hipGraph_t graph = nullptr;
  hipError_t ee = hipStreamEndCapture(cs, &graph);
  (void)hipStreamDestroy(cs);
  if (st != RVA_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (ee != hipSuccess) return hip_fail(ee, "end capture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return hip_fail(e, "graph instantiate");
  }
  rva_plan_s* plan = new (std::nothrow) rva_plan_s{graph, exec, nullptr, false, {}, 0};
  if (!plan) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return fail(RVA_ERR_INVALID, "out of host memory");
  }
  *out = plan;
  return RVA_OK;
}

}  // namespace

extern "C" {

int rva_version(void) { return 104; }

const char* rva_status_string(int status) {
  switch (status) {
    case RVA_OK: return "ok";
    case RVA_ERR_INVALID: return "invalid argument";
    case RVA_ERR_UNSUPPORTED: return "unsupported configuration";
    case RVA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* rva_last_error(void) { return g_err; }

int rva_pack(const void* q_pad, const void* k_pad, const void* v_pad, const uint8_t* mask, int B,
             int N, int H, int d, int dtype, void* q_out, void* k_out, void* v_out,
             int32_t* cu_seqlens, int32_t* max_seqlen, int32_t* kept_index, void* stream) {
  PackArgs a;
  RVA_TRY(validate_pack(q_pad, k_pad, v_pad, mask, B, N, H, d, dtype, q_out, k_out, v_out,
                        cu_seqlens, max_seqlen, kept_index, &a));
  return enqueue_pack(a, static_cast<hipStream_t>(stream));
}

int rva_ragged_attend(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int B,
                      int H, int d, int max_seqlen, float softmax_scale, int dtype, void* o,
                      void* stream) {
  rva::AttnParams p;
  RVA_TRY(validate_attend(q, k, v, cu_seqlens, B, H, d, max_seqlen, softmax_scale, dtype, o, &p));
  return enqueue_attend(p, dtype, false, static_cast<hipStream_t>(stream));
}

int rva_unpack(const void* o_packed, const int32_t* cu_seqlens, const uint8_t* mask, int B, int N,
               int H, int d, int dtype, void* o_pad, void* stream) {
  PackArgs a;
  RVA_TRY(validate_unpack(o_packed, cu_seqlens, mask, B, N, H, d, dtype, o_pad, &a));
  hipError_t e = rva::launch_unpack(a.cp, a.splits, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "unpack launch");
  return RVA_OK;
}

int rva_fused(const void* q_pad, const void* k_pad, const void* v_pad, const uint8_t* mask, int B,
              int N, int H, int d, int max_seqlen_hint, float softmax_scale, int dtype, void* o_pad,
              int32_t* cu_seqlens, int32_t* max_seqlen, void* stream) {
  rva::AttnParams p;
  RVA_TRY(validate_fused(q_pad, k_pad, v_pad, mask, B, N, H, d, max_seqlen_hint, softmax_scale,
                         dtype, o_pad, cu_seqlens, max_seqlen, &p));
  return enqueue_attend(p, dtype, true, static_cast<hipStream_t>(stream));
}

int rva_threshold_l2_mask(const void* x, int B, int N, int C, int dtype, double keep_quantile,
                          uint8_t* mask_out, void* stream) {
  ThreshArgs a;
  RVA_TRY(validate_threshold(x, B, N, C, dtype, keep_quantile, mask_out, &a));
  return enqueue_threshold(a, static_cast<hipStream_t>(stream));
}

int rva_qkv_projection(const void* x, const int32_t* kept_index, const int32_t* cu_seqlens, int B,
                       int N, int C, const void* w_qkv, const void* b_qkv, int dtype, void* q,
                       void* k, void* v, void* stream) {
  rva::LinearParams p;
  RVA_TRY(validate_qkv(x, kept_index, cu_seqlens, B, N, C, w_qkv, b_qkv, dtype, q, k, v, &p));
  return enqueue_linear(p, dtype, static_cast<hipStream_t>(stream));
}

int rva_out_projection(const void* o, const int32_t* kept_index, const int32_t* cu_seqlens,
                       const uint8_t* mask, int B, int N, int C, const void* w_o, const void* b_o,
                       const void* residual, int dtype, void* y, void* stream) {
  rva::LinearParams p;
  RVA_TRY(validate_outproj(o, kept_index, cu_seqlens, mask, B, N, C, w_o, b_o, residual, dtype, y,
                           &p));
  return enqueue_linear(p, dtype, static_cast<hipStream_t>(stream));
}

int rva_fused_persistent(const void* q_pad, const void* k_pad, const void* v_pad,
                         const uint8_t* mask, int B, int N, int H, int d, int max_seqlen_hint,
                         float softmax_scale, int dtype, void* o_pad, int32_t* cu_seqlens,
                         int32_t* max_seqlen, int32_t* work, void* stream) {
  rva::AttnParams p;
  RVA_TRY(validate_fused(q_pad, k_pad, v_pad, mask, B, N, H, d, max_seqlen_hint, softmax_scale,
                         dtype, o_pad, cu_seqlens, max_seqlen, &p));
  RVA_TRY(check_i32(work, "work", true));
  RVA_TRY(check_persistent_items(B, H));
  if (dtype == RVA_F32)  // the persistent form is built for 16-bit inputs; fp32 keeps one launch
    return enqueue_attend(p, dtype, true, static_cast<hipStream_t>(stream));
  p.work = work;
  return enqueue_attend_persistent(p, dtype, static_cast<hipStream_t>(stream));
}

int rva_fused_persistent_noalloc(const void* q_pad, const void* k_pad, const void* v_pad,
                                 const uint8_t* mask, int B, int N, int H, int d,
                                 int max_seqlen_hint, float softmax_scale, int dtype, void* o_pad,
                                 int32_t* cu_seqlens, int32_t* max_seqlen, void* stream) {
  rva::AttnParams p;
  RVA_TRY(validate_fused(q_pad, k_pad, v_pad, mask, B, N, H, d, max_seqlen_hint, softmax_scale,
                         dtype, o_pad, cu_seqlens, max_seqlen, &p));
  RVA_TRY(check_persistent_items(B, H));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == RVA_F32)  // as rva_fused_persistent: fp32 runs the one-launch kernel, no counter
    return enqueue_attend(p, dtype, true, s);
  RVA_TRY(ensure_init());
  RVA_TRY(scratch_counter(s, &p.work));
  return enqueue_attend_persistent(p, dtype, s);
}

int rva_set_query_split(int split) {
  if (split < 0) return fail(RVA_ERR_INVALID, "split must be >= 0 (got %d)", split);
  g_query_split.store(split, std::memory_order_relaxed);
  return RVA_OK;
}

int rva_probe_copy(const void* src, void* dst, long long bytes, int grid, void* stream) {
  RVA_TRY(check_data(src, "src", true));
  RVA_TRY(check_data(dst, "dst", true));
  if (bytes <= 0 || bytes % 16) return fail(RVA_ERR_INVALID, "bytes must be a positive multiple of 16");
  if (grid < 1) return fail(RVA_ERR_INVALID, "grid must be >= 1");
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RVA_ERR_INVALID, "src and dst overlap");
  hipError_t e = rva::launch_probe_copy(src, dst, bytes / 16, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy probe launch");
  return RVA_OK;
}

int rva_probe_read(const void* src, uint32_t* sink, long long bytes, int grid, void* stream) {
  RVA_TRY(check_data(src, "src", true));
  RVA_TRY(check_i32(sink, "sink", true));
  if (bytes <= 0 || bytes % 16) return fail(RVA_ERR_INVALID, "bytes must be a positive multiple of 16");
  if (grid < 1) return fail(RVA_ERR_INVALID, "grid must be >= 1");
  hipError_t e = rva::launch_probe_read(src, sink, bytes / 16, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read probe launch");
  return RVA_OK;
}

int rva_probe_mfma(int iters, float* out, int grid, void* stream, long long* flops) {
  RVA_TRY(check_i32(out, "out", true));
  if (iters < 1 || grid < 1) return fail(RVA_ERR_INVALID, "iters and grid must be >= 1");
  if (flops) *flops = rva::probe_mfma_flops(iters, grid);
  hipError_t e = rva::launch_probe_mfma(iters, out, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "matrix-core probe launch");
  return RVA_OK;
}

int rva_probe_gather(const void* q, const void* k, const void* v, void* o, const uint8_t* mask,
                     const int32_t* cu_seqlens, const int32_t* kept_index, int B, int N, int H,
                     void* stream) {
  RVA_TRY(check_shape(B, N, H, RVA_HEAD_DIM, RVA_F16));
  RVA_TRY(check_data(q, "q", true));
  RVA_TRY(check_data(k, "k", true));
  RVA_TRY(check_data(v, "v", true));
  RVA_TRY(check_data(o, "o", true));
  if (!mask) return fail(RVA_ERR_INVALID, "mask is NULL");
  RVA_TRY(check_i32(cu_seqlens, "cu_seqlens", true));
  RVA_TRY(check_i32(kept_index, "kept_index", true));
  hipError_t e = rva::launch_probe_gather(q, k, v, o, mask, cu_seqlens, kept_index, B, N, H,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather probe launch");
  return RVA_OK;
}

int rva_empty(int count, void* stream) {
  if (count < 0) return fail(RVA_ERR_INVALID, "count must be >= 0");
  for (int i = 0; i < count; ++i) {
    hipError_t e = rva::launch_empty(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "empty launch");
  }
  return RVA_OK;
}

int rva_plan_create(const rva_plan_desc* desc, rva_plan* out) {
  if (!desc || !out) return fail(RVA_ERR_INVALID, "desc and out must be non-NULL");
  *out = nullptr;
  const rva_plan_desc& D = *desc;
  PackArgs pack, unpack;
  rva::AttnParams attn;
  ThreshArgs thr;
  switch (D.mode) {
    case RVA_PLAN_STAGED:
      RVA_TRY(validate_pack(D.q_pad, D.k_pad, D.v_pad, D.mask, D.B, D.N, D.H, D.d, D.dtype,
                            D.q_packed, D.k_packed, D.v_packed, D.cu_seqlens, D.max_seqlen,
                            D.kept_index, &pack));
      if (!D.q_pad || !D.k_pad || !D.v_pad)
        return fail(RVA_ERR_INVALID, "staged plan needs q, k and v");
      RVA_TRY(validate_attend(D.q_packed, D.k_packed, D.v_packed, D.cu_seqlens, D.B, D.H, D.d,
                              D.max_seqlen_hint > 0 ? D.max_seqlen_hint : D.N, D.softmax_scale,
                              D.dtype, D.o_packed, &attn));
      RVA_TRY(validate_unpack(D.o_packed, D.cu_seqlens, D.mask, D.B, D.N, D.H, D.d, D.dtype,
                              D.o_pad, &unpack));
      break;
    case RVA_PLAN_FUSED:
    case RVA_PLAN_FUSED_DIRECT:
      RVA_TRY(validate_fused(D.q_pad, D.k_pad, D.v_pad, D.mask, D.B, D.N, D.H, D.d,
                             D.max_seqlen_hint, D.softmax_scale, D.dtype, D.o_pad, D.cu_seqlens,
                             D.max_seqlen, &attn));
      break;
    case RVA_PLAN_PERSISTENT:
      RVA_TRY(validate_fused(D.q_pad, D.k_pad, D.v_pad, D.mask, D.B, D.N, D.H, D.d,
                             D.max_seqlen_hint, D.softmax_scale, D.dtype, D.o_pad, D.cu_seqlens,
                             D.max_seqlen, &attn));
      RVA_TRY(check_persistent_items(D.B, D.H));
      break;
    case RVA_PLAN_L2_FUSED:
      RVA_TRY(validate_threshold(D.x, D.B, D.N, D.C, D.x_dtype, D.keep_quantile, D.mask_out,
                                 &thr));
      RVA_TRY(validate_fused(D.q_pad, D.k_pad, D.v_pad, D.mask_out, D.B, D.N, D.H, D.d,
                             D.max_seqlen_hint, D.softmax_scale, D.dtype, D.o_pad, D.cu_seqlens,
                             D.max_seqlen, &attn));
      break;
    case RVA_PLAN_EMPTY:
      break;
    default:
      return fail(RVA_ERR_INVALID, "unknown plan mode %d", D.mode);
  }
  RVA_TRY(ensure_init());
  // direct mode: no graph, the validated launch is kept and enqueued as is
  if (D.mode == RVA_PLAN_FUSED_DIRECT) {
    rva_plan_s* plan = new (std::nothrow) rva_plan_s{nullptr, nullptr, nullptr, true, attn, D.dtype};
    if (!plan) return fail(RVA_ERR_INVALID, "out of host memory");
    *out = plan;
    return RVA_OK;
  }
  // persistent mode owns a zeroed two-int work counter for its whole life
  int32_t* work = nullptr;
  if (D.mode == RVA_PLAN_PERSISTENT) {
    hipError_t e = hipMalloc(&work, 2 * sizeof(int32_t));
    if (e != hipSuccess) return hip_fail(e, "work counter allocation");
    e = hipMemset(work, 0, 2 * sizeof(int32_t));
    if (e != hipSuccess) {
      (void)hipFree(work);
      return hip_fail(e, "work counter reset");
    }
  }
  const int st0 = capture_plan(out, [&](hipStream_t cs) -> int {
    hipError_t e;
    int st = RVA_OK;
    switch (D.mode) {
    case RVA_PLAN_STAGED:
      st = enqueue_pack(pack, cs);
      if (st == RVA_OK) st = enqueue_attend(attn, D.dtype, false, cs);
      if (st == RVA_OK) {
        e = rva::launch_unpack(unpack.cp, unpack.splits, cs);
        if (e != hipSuccess) st = hip_fail(e, "unpack launch");
      }
      break;
    case RVA_PLAN_FUSED:
      st = enqueue_attend(attn, D.dtype, true, cs);
      break;
    case RVA_PLAN_PERSISTENT:
      attn.work = work;
      st = D.dtype == RVA_F32 ? enqueue_attend(attn, D.dtype, true, cs)
                              : enqueue_attend_persistent(attn, D.dtype, cs);
      break;
    case RVA_PLAN_L2_FUSED:
      st = enqueue_threshold(thr, cs);
      if (st == RVA_OK) st = enqueue_attend(attn, D.dtype, true, cs);
      break;
    case RVA_PLAN_EMPTY:
      e = rva::launch_empty(cs);
      if (e != hipSuccess) st = hip_fail(e, "empty launch");
      break;
    }
    return st;
  });
  if (st0 != RVA_OK) {
    if (work) (void)hipFree(work);
    return st0;
  }
  (*out)->work = work;
  return RVA_OK;
}

int rva_layers_plan_create(const rva_layers_desc* desc, rva_plan* out) {
  if (!desc || !out) return fail(RVA_ERR_INVALID, "desc and out must be non-NULL");
  *out = nullptr;
  const rva_layers_desc& D = *desc;
  const int L = D.layers;
  if (L < 1 || L > RVA_MAX_LAYERS)
    return fail(RVA_ERR_INVALID, "layers must be in [1, %d] (got %d)", RVA_MAX_LAYERS, L);
  if (!D.w_qkv || !D.w_o) return fail(RVA_ERR_INVALID, "w_qkv and w_o arrays are required");
  RVA_TRY(check_shape(D.B, D.N, D.H, D.d, D.dtype));
  const int C = D.H * D.d;
  if (!D.kept_index) return fail(RVA_ERR_INVALID, "kept_index is NULL");
  // one pack of x into the residual stream, L x (qkv, attention, out + residual), one unpack
  PackArgs pack, unpack;
  RVA_TRY(validate_pack(D.x_pad, nullptr, nullptr, D.mask, D.B, D.N, D.H, D.d, D.dtype, D.resid,
                        nullptr, nullptr, D.cu_seqlens, D.max_seqlen, D.kept_index, &pack));
  RVA_TRY(validate_unpack(D.resid, D.cu_seqlens, D.mask, D.B, D.N, D.H, D.d, D.dtype, D.y_pad,
                          &unpack));
  std::vector<rva::LinearParams> qkv(L), outp(L);
  rva::AttnParams attn;
  RVA_TRY(validate_attend(D.q, D.k, D.v, D.cu_seqlens, D.B, D.H, D.d,
                          D.max_seqlen_hint > 0 ? D.max_seqlen_hint : D.N, D.softmax_scale,
                          D.dtype, D.o, &attn));
  for (int l = 0; l < L; ++l) {
    RVA_TRY(validate_qkv(D.resid, nullptr, D.cu_seqlens, D.B, D.N, C, D.w_qkv[l],
                         D.b_qkv ? D.b_qkv[l] : nullptr, D.dtype, D.q, D.k, D.v, &qkv[l]));
    RVA_TRY(validate_outproj(D.o, nullptr, D.cu_seqlens, D.mask, D.B, D.N, C, D.w_o[l],
                             D.b_o ? D.b_o[l] : nullptr, D.resid, D.dtype, D.resid, &outp[l]));
  }
  RVA_TRY(ensure_init());
  return capture_plan(out, [&](hipStream_t cs) -> int {
    RVA_TRY(enqueue_pack(pack, cs));
    for (int l = 0; l < L; ++l) {
      RVA_TRY(enqueue_linear(qkv[l], D.dtype, cs));
      RVA_TRY(enqueue_attend(attn, D.dtype, false, cs));
      RVA_TRY(enqueue_linear(outp[l], D.dtype, cs));
    }
    hipError_t e = rva::launch_unpack(unpack.cp, unpack.splits, cs);
    if (e != hipSuccess) return hip_fail(e, "unpack launch");
    return RVA_OK;
  });
}

int rva_plan_launch(rva_plan plan, void* stream) {
  if (!plan) return fail(RVA_ERR_INVALID, "plan is NULL");
  if (plan->direct)
    return enqueue_attend(plan->attn, plan->dtype, true, static_cast<hipStream_t>(stream));
  hipError_t e = hipGraphLaunch(plan->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "graph launch");
  return RVA_OK;
}

int rva_plan_destroy(rva_plan plan) {
  if (!plan) return RVA_OK;
  if (plan->exec) (void)hipGraphExecDestroy(plan->exec);
  if (plan->graph) (void)hipGraphDestroy(plan->graph);
  if (plan->work) (void)hipFree(plan->work);
  delete plan;
  return RVA_OK;
}

}  // extern "C"
