// Dispatch floor measured from C++ through the C ABI, without the Python
// layer the Python-side figure includes (the sota2.com page's Abstract puts
// the cost at these sequence lengths in host dispatch).  For each launch path
// it reports the median host time of (launch; synchronise) over many calls
// and the mean time per call of back-to-back launches:
//   * direct : rva_empty, one empty one-workgroup kernel;
//   * graph  : a captured plan holding that kernel (RVA_PLAN_EMPTY).
// Each argument names a workload file written by the bench: int32 B, N, H,
// dtype and length hint, then q, k and v ([B, N, H, 64] elements of the
// dtype's size) and the uint8 mask [B, N].  For each, the same two figures
// for the fused call itself: rva_fused, and a direct-launch plan
// (RVA_PLAN_FUSED_DIRECT) launched repeatedly.
// Output: one JSON object on stdout.  Build: see the package's build step.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <string>
#include <vector>

#include "rva.h"

namespace {

double median(std::vector<double> v) {
  std::sort(v.begin(), v.end());
  return v[v.size() / 2];
}

template <typename F>
int measure(F launch, hipStream_t s, int reps, double* lat_us, double* b2b_us) {
  for (int i = 0; i < 20; ++i)
    if (launch() != RVA_OK) return 1;
  if (hipStreamSynchronize(s) != hipSuccess) return 1;
  std::vector<double> t(reps);
  for (int i = 0; i < reps; ++i) {
    const auto t0 = std::chrono::steady_clock::now();
    if (launch() != RVA_OK) return 1;
    if (hipStreamSynchronize(s) != hipSuccess) return 1;
    t[i] = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  }
  *lat_us = median(t);
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < reps; ++i)
    if (launch() != RVA_OK) return 1;
  if (hipStreamSynchronize(s) != hipSuccess) return 1;
  *b2b_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count() / reps;
  return 0;
}

// One workload file's fused-call figures appended to `json`; 0 on success.
int measure_fused(const char* path, hipStream_t s, int reps, std::string* json) {
  FILE* f = fopen(path, "rb");
  if (!f) return 1;
  int32_t hdr[5];
  if (fread(hdr, sizeof(int32_t), 5, f) != 5) {
    fclose(f);
    return 1;
  }
  const int B = hdr[0], N = hdr[1], H = hdr[2], dtype = hdr[3], hint = hdr[4];
  if (B < 1 || N < 1 || N > RVA_MAX_TOKENS || H < 1 || H > RVA_MAX_HEADS || dtype < 0 || dtype > 2 ||
      (long long)B * N * H > (1ll << 26)) {
    fclose(f);
    return 1;
  }
  const size_t es = dtype == RVA_F32 ? 4 : 2;
  const size_t elems = (size_t)B * N * H * RVA_HEAD_DIM, bytes = elems * es, mbytes = (size_t)B * N;
  std::vector<char> host(3 * bytes + mbytes);
  const bool ok = fread(host.data(), 1, host.size(), f) == host.size();
  fclose(f);
  if (!ok) return 1;
  void *q = nullptr, *k = nullptr, *v = nullptr, *o = nullptr;
  uint8_t* m = nullptr;
  int rc = 1;
  if (hipMalloc(&q, bytes) == hipSuccess && hipMalloc(&k, bytes) == hipSuccess &&
      hipMalloc(&v, bytes) == hipSuccess && hipMalloc(&o, bytes) == hipSuccess &&
      hipMalloc(reinterpret_cast<void**>(&m), mbytes) == hipSuccess &&
      hipMemcpy(q, host.data(), bytes, hipMemcpyHostToDevice) == hipSuccess &&
      hipMemcpy(k, host.data() + bytes, bytes, hipMemcpyHostToDevice) == hipSuccess &&
      hipMemcpy(v, host.data() + 2 * bytes, bytes, hipMemcpyHostToDevice) == hipSuccess &&
      hipMemcpy(m, host.data() + 3 * bytes, mbytes, hipMemcpyHostToDevice) == hipSuccess) {
    double fl = 0, fb = 0, pl = 0, pb = 0;
    rva_plan_desc d = {};
    d.mode = RVA_PLAN_FUSED_DIRECT;
    d.B = B, d.N = N, d.H = H, d.d = RVA_HEAD_DIM, d.dtype = dtype, d.max_seqlen_hint = hint;
    d.q_pad = q, d.k_pad = k, d.v_pad = v, d.mask = m, d.o_pad = o;
    rva_plan plan = nullptr;
    if (!measure([&] { return rva_fused(q, k, v, m, B, N, H, RVA_HEAD_DIM, hint, 0.f, dtype, o,
                                        nullptr, nullptr, s); },
                 s, reps, &fl, &fb) &&
        rva_plan_create(&d, &plan) == RVA_OK &&
        !measure([&] { return rva_plan_launch(plan, s); }, s, reps, &pl, &pb)) {
      const char* base = strrchr(path, '/');
      char buf[512];
      snprintf(buf, sizeof buf,
               "%s{\"workload\": \"%s\", \"fused_latency_us\": %.2f, \"fused_back_to_back_us\": %.2f, "
               "\"plan_latency_us\": %.2f, \"plan_back_to_back_us\": %.2f}",
               json->empty() ? "" : ", ", base ? base + 1 : path, fl, fb, pl, pb);
      *json += buf;
      rc = 0;
    }
    if (plan) rva_plan_destroy(plan);
  }
  (void)hipFree(q);
  (void)hipFree(k);
  (void)hipFree(v);
  (void)hipFree(o);
  (void)hipFree(m);
  return rc;
}

}  // namespace

int main(int argc, char** argv) {
  hipStream_t s = nullptr;
  if (hipStreamCreate(&s) != hipSuccess) return 2;
  const int reps = 2000;
  double dl = 0, db = 0, gl = 0, gb = 0;
  if (measure([&] { return rva_empty(1, s); }, s, reps, &dl, &db)) {
    fprintf(stderr, "direct launch failed: %s\n", rva_last_error());
    return 3;
  }
  rva_plan_desc d = {};
  d.mode = RVA_PLAN_EMPTY;
  rva_plan plan = nullptr;
  if (rva_plan_create(&d, &plan) != RVA_OK) {
    fprintf(stderr, "plan creation failed: %s\n", rva_last_error());
    return 3;
  }
  if (measure([&] { return rva_plan_launch(plan, s); }, s, reps, &gl, &gb)) {
    fprintf(stderr, "graph launch failed: %s\n", rva_last_error());
    return 3;
  }
  rva_plan_destroy(plan);
  std::string fused;
  for (int i = 1; i < argc; ++i) {
    if (measure_fused(argv[i], s, reps, &fused)) {
      fprintf(stderr, "fused call on %s failed: %s\n", argv[i], rva_last_error());
      return 3;
    }
  }
  (void)hipStreamDestroy(s);
  printf("{\"direct_latency_us\": %.2f, \"direct_back_to_back_us\": %.2f, "
         "\"graph_latency_us\": %.2f, \"graph_back_to_back_us\": %.2f, \"reps\": %d, "
         "\"fused\": [%s]}\n",
         dl, db, gl, gb, reps, fused.c_str());
  return 0;
}
