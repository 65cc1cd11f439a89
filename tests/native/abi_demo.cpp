// abi_demo.cpp -- a native consumer of libsdc.so through include/sdc.h only
// (HIP runtime for memory, no Python, no torch): R = 3 replicas of a small
// tensor list with seeded bit patterns, one bit flipped in replica 2, then
// plan, scan, strict-majority compare and diff.  Prints the rows and results
// for the test that checks them against the oracle on the same patterns.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "sdc.h"

namespace {

#define CHECK_HIP(x)                                                                  \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      std::fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);           \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)
#define CHECK_SDC(x)                                                                  \
  do {                                                                                \
    int32_t s_ = (x);                                                                 \
    if (s_ != SDC_OK) {                                                               \
      std::fprintf(stderr, "%s at line %d\n", sdc_status_string(s_), __LINE__);       \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

// Seeded pattern of element i of tensor k (the test recomputes it).
uint32_t pattern(uint64_t i, uint32_t k) {
  uint32_t h = (uint32_t)((i + 1) * 0x9E3779B1u) + k * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return h;
}

struct Spec {
  uint64_t numel;
  uint32_t dtype;  // SDC_F32 or SDC_BF16
};

}  // namespace

int main() {
  const Spec specs[] = {{1, SDC_F32}, {1000, SDC_BF16}, {1048577, SDC_F32}, {33333, SDC_BF16}};
  const uint32_t T = 4, R = 3;
  const uint32_t flip_tensor = 2, flip_bit = 7;
  const uint64_t flip_index = 12345;
  std::vector<void*> bufs;
  std::vector<sdc_tensor> descs;
  for (uint32_t r = 0; r < R; ++r) {
    for (uint32_t k = 0; k < T; ++k) {
      const uint32_t es = specs[k].dtype == SDC_F32 ? 4 : 2;
      std::vector<unsigned char> host(specs[k].numel * es);
      for (uint64_t i = 0; i < specs[k].numel; ++i) {
        uint32_t v = pattern(i, k);
        if (r == 2 && k == flip_tensor && i == flip_index) v ^= 1u << flip_bit;
        for (uint32_t b = 0; b < es; ++b) host[i * es + b] = (unsigned char)(v >> (8 * b));
      }
      void* d = nullptr;
      CHECK_HIP(hipMalloc(&d, host.size()));
      CHECK_HIP(hipMemcpy(d, host.data(), host.size(), hipMemcpyHostToDevice));
      bufs.push_back(d);
      descs.push_back(sdc_tensor{d, specs[k].numel, specs[k].dtype, 0});
    }
  }
  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  uint64_t plan_bytes = 0;
  CHECK_SDC(sdc_plan_bytes(descs.data(), descs.size(), 0, &plan_bytes));
  void* d_plan = nullptr;
  CHECK_HIP(hipMalloc(&d_plan, plan_bytes));
  sdc_plan_info info;
  CHECK_SDC(sdc_plan_build(descs.data(), descs.size(), 0, d_plan, plan_bytes, &info, s));
  sdc_row* d_rows = nullptr;
  CHECK_HIP(hipMalloc(&d_rows, descs.size() * sizeof(sdc_row)));
  CHECK_SDC(sdc_fingerprint_plan(d_plan, &info, d_rows, s));
  std::vector<sdc_row> rows(descs.size());
  CHECK_HIP(hipMemcpyAsync(rows.data(), d_rows, rows.size() * sizeof(sdc_row),
                           hipMemcpyDeviceToHost, s));
  CHECK_HIP(hipStreamSynchronize(s));
  for (size_t j = 0; j < rows.size(); ++j)
    std::printf("ROW %zu %llu %llu %llu %llu\n", j, (unsigned long long)rows[j].sum,
                (unsigned long long)rows[j].wsum, (unsigned long long)rows[j].xorsum,
                (unsigned long long)rows[j].nonfinite);

  uint64_t ws_bytes = 0;
  CHECK_SDC(sdc_majority_ws_bytes(R, T, &ws_bytes));
  void* d_ws = nullptr;
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  sdc_majority res;
  uint8_t suspect[R];
  CHECK_SDC(sdc_majority_compare(d_rows, R, T, SDC_COL_ALL, d_ws, ws_bytes, &res, suspect, nullptr,
                                 s));
  std::printf("MAJ %d %d %llu %llu %d %d %d\n", res.diverged, res.has_majority,
              (unsigned long long)res.n_diff, (unsigned long long)res.first_diff, suspect[0],
              suspect[1], suspect[2]);

  uint64_t diff_ws = 0;
  CHECK_SDC(sdc_diff_ws_bytes(T, T, &diff_ws));
  void* d_dws = nullptr;
  CHECK_HIP(hipMalloc(&d_dws, diff_ws));
  uint64_t n_diff = 0, idx[T];
  sdc_flip_hint hints[T];
  CHECK_SDC(sdc_fingerprint_diff(d_rows, d_rows + 2 * T, T, SDC_COL_ALL, d_dws, diff_ws, &n_diff,
                                 idx, T, hints, s));
  std::printf("DIFF %llu", (unsigned long long)n_diff);
  for (uint64_t i = 0; i < n_diff && i < T; ++i)
    std::printf(" %llu %llu %d %d", (unsigned long long)idx[i], (unsigned long long)hints[i].index,
                hints[i].bit, hints[i].dir);
  std::printf("\n");

  for (void* d : bufs) CHECK_HIP(hipFree(d));
  CHECK_HIP(hipFree(d_plan));
  CHECK_HIP(hipFree(d_rows));
  CHECK_HIP(hipFree(d_ws));
  CHECK_HIP(hipFree(d_dws));
  CHECK_HIP(hipStreamDestroy(s));
  return 0;
}
