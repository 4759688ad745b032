// Dispatch floor measured from C++ through the C ABI, without the Python
// layer the Python-side figure includes (the sota2.com page's Abstract puts
// the cost at these sequence lengths in host dispatch).  For each launch path
// it reports the median host time of (launch; synchronise) over many calls
// and the mean time per call of back-to-back launches:
//   * direct : rva_empty, one empty one-workgroup kernel;
//   * graph  : a captured plan holding that kernel (RVA_PLAN_EMPTY).
// Output: one JSON object on stdout.  Build: see the package's build step.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <algorithm>
#include <chrono>
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

}  // namespace

int main() {
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
  (void)hipStreamDestroy(s);
  printf("{\"direct_latency_us\": %.2f, \"direct_back_to_back_us\": %.2f, "
         "\"graph_latency_us\": %.2f, \"graph_back_to_back_us\": %.2f, \"reps\": %d}\n",
         dl, db, gl, gb, reps);
  return 0;
}
