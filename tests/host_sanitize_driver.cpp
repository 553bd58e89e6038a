// Host-side driver for the address / undefined-behaviour sanitizer build of
// the C ABI (tests/test_host_sanitize.py).  It calls the entry points that
// read caller arrays on the host (qwha_csr_transpose, qwha_init_allocate)
// with buffers of exactly the documented sizes, on well-formed and malformed
// input, plus the argument checks of the device entry points (which return
// before any HIP call), and prints one line per check.  Any heap overread,
// overflow or undefined operation aborts under the sanitizers.  With
// --short-output it passes an output array one element short, which the
// address sanitizer must report (a check that the build is instrumented).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "whtq.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  std::printf("%-56s %s (%d)\n", what, got == want ? "ok" : "FAIL", got);
  if (got != want) ++failures;
}

// exact-size heap copies, so that one element too far is a sanitizer report
template <class T>
static T* heap(const std::vector<T>& v) {
  T* p = static_cast<T*>(std::malloc(v.empty() ? 1 : v.size() * sizeof(T)));
  if (!v.empty()) std::memcpy(p, v.data(), v.size() * sizeof(T));
  return p;
}

static int transpose(const std::vector<int32_t>& rp, const std::vector<int32_t>& ci, int64_t d_out, int64_t d_in) {
  int32_t* r = heap(rp);
  int32_t* c = heap(ci);
  const int64_t nnz = (int64_t)ci.size();
  int32_t* tr = static_cast<int32_t*>(std::malloc((d_in + 1) * sizeof(int32_t)));
  int32_t* tc = static_cast<int32_t*>(std::malloc((nnz ? nnz : 1) * sizeof(int32_t)));
  int32_t* tp = static_cast<int32_t*>(std::malloc((nnz ? nnz : 1) * sizeof(int32_t)));
  const int st = qwha_csr_transpose(r, nnz ? c : nullptr, d_out, d_in, nnz, tr, nnz ? tc : nullptr,
                                    nnz ? tp : nullptr);
  if (st == WHTQ_OK) {  // the transpose of a valid CSR is a valid CSR with the same entries
    bool good = tr[0] == 0 && tr[d_in] == nnz;
    for (int64_t k = 0; k < d_in && good; ++k) good = tr[k] <= tr[k + 1];
    for (int64_t j = 0; j < nnz && good; ++j) good = tp[j] >= 0 && tp[j] < nnz && ci[tp[j]] >= 0;
    if (!good) ++failures;
  }
  std::free(r);
  std::free(c);
  std::free(tr);
  std::free(tc);
  std::free(tp);
  return st;
}

static int allocate(const std::vector<float>& err, int64_t n, int64_t total, int floor, int cap) {
  float* e = heap(err);
  const int64_t rows = (int64_t)err.size();
  int32_t* rp = static_cast<int32_t*>(std::malloc((rows + 1) * sizeof(int32_t)));
  const int st = qwha_init_allocate(e, rows, n, total, floor, cap, rp);
  if (st == WHTQ_OK) {
    bool good = rp[0] == 0 && rp[rows] == total;
    for (int64_t o = 0; o < rows && good; ++o) good = rp[o + 1] - rp[o] >= floor && rp[o + 1] - rp[o] <= cap;
    if (!good) ++failures;
  }
  std::free(e);
  std::free(rp);
  return st;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "--short-output") == 0) {
    // a t_row_ptr one element short of d_in + 1: the sanitizer must stop this
    int32_t* rp = heap(std::vector<int32_t>{0, 1});
    int32_t* ci = heap(std::vector<int32_t>{2});
    int32_t* tr = static_cast<int32_t*>(std::malloc(4 * sizeof(int32_t)));
    int32_t tc[1], tp[1];
    const int st = qwha_csr_transpose(rp, ci, 1, 4, 1, tr, tc, tp);
    std::printf("returned %d\n", st);
    return 0;
  }
  // ---- qwha_csr_transpose
  expect("transpose: 3 x 5, rows of 2, 0, 3 entries", transpose({0, 2, 2, 5}, {1, 4, 0, 1, 4}, 3, 5), WHTQ_OK);
  expect("transpose: every column empty", transpose({0, 0, 0}, {}, 2, 7), WHTQ_OK);
  expect("transpose: one row holding every column", transpose({0, 4}, {3, 2, 1, 0}, 1, 4), WHTQ_OK);
  expect("transpose: row_ptr[0] != 0", transpose({1, 2, 3}, {0, 1, 2}, 2, 4), WHTQ_EINVAL);
  expect("transpose: row_ptr[d_out] != nnz", transpose({0, 1, 2}, {0, 1, 2}, 2, 4), WHTQ_EINVAL);
  expect("transpose: decreasing row_ptr", transpose({0, 3, 2, 3}, {0, 1, 2}, 3, 4), WHTQ_EINVAL);
  expect("transpose: column == d_in", transpose({0, 2}, {0, 4}, 1, 4), WHTQ_EINVAL);
  expect("transpose: negative column", transpose({0, 2}, {-1, 2}, 1, 4), WHTQ_EINVAL);
  expect("transpose: column INT32_MAX", transpose({0, 1}, {std::numeric_limits<int32_t>::max()}, 1, 4),
         WHTQ_EINVAL);
  {
    std::vector<int32_t> rp(1001), ci;
    uint32_t s = 7;
    for (int o = 0; o < 1000; ++o) {
      rp[o + 1] = rp[o] + (int)(o % 13);
      for (int j = 0; j < (int)(o % 13); ++j) {
        s = s * 1664525u + 1013904223u;
        ci.push_back((int32_t)(s >> 20));  // [0, 4096)
      }
    }
    expect("transpose: 1000 x 4096 random", transpose(rp, ci, 1000, 4096), WHTQ_OK);
  }

  // ---- qwha_init_allocate
  expect("allocate: 5 channels, total 30", allocate({1.f, 2.f, 0.f, 4.f, 0.5f}, 64, 30, 2, 16), WHTQ_OK);
  expect("allocate: all-zero errors", allocate({0.f, 0.f, 0.f}, 64, 12, 1, 8), WHTQ_OK);
  expect("allocate: total at the cap", allocate({1.f, 9.f}, 64, 16, 0, 8), WHTQ_OK);
  expect("allocate: total at the floor", allocate({1.f, 9.f}, 64, 4, 2, 8), WHTQ_OK);
  expect("allocate: huge error spread", allocate({1e-30f, 1e30f, 3.f}, 64, 20, 1, 10), WHTQ_OK);
  expect("allocate: NaN error", allocate({1.f, std::numeric_limits<float>::quiet_NaN()}, 64, 8, 1, 8),
         WHTQ_EINVAL);
  expect("allocate: negative error", allocate({1.f, -1.f}, 64, 8, 1, 8), WHTQ_EINVAL);
  expect("allocate: total above rows * cap", allocate({1.f, 1.f}, 64, 17, 1, 8), WHTQ_EINVAL);
  expect("allocate: cap above n", allocate({1.f, 1.f}, 4, 6, 1, 5), WHTQ_EINVAL);
  expect("allocate: cap above the supported maximum", allocate({1.f}, 4096, 200, 1, 200), WHTQ_EUNSUPPORTED);

  // ---- argument checks of device entry points (no HIP call is reached)
  expect("forward: NULL row_ptr",
         qwha_adapter_forward((void*)0x1000, WHTQ_BF16, 8, 4096, 4096, nullptr, (int32_t*)0x1000, (void*)0x1000,
                              WHTQ_BF16, 16, 10, (void*)0x2000, WHTQ_BF16, 16, nullptr),
         WHTQ_EINVAL);
  expect("forward: d_in 3000",
         qwha_adapter_forward((void*)0x1000, WHTQ_BF16, 8, 3000, 3000, (int32_t*)0x1000, (int32_t*)0x1000,
                              (void*)0x1000, WHTQ_BF16, 16, 10, (void*)0x2000, WHTQ_BF16, 16, nullptr),
         WHTQ_EUNSUPPORTED);
  expect("workspace bytes: d_in 16384", (int)qwha_grad_values_workspace_bytes(8, 16384, 100), -1);
  expect("quantise: NULL input",
         rht_quantize_rtn(nullptr, WHTQ_BF16, 16, 4096, 4096, nullptr, 4, 128, (uint8_t*)0x1000,
                          (uint16_t*)0x1000, nullptr),
         WHTQ_EINVAL);
  std::printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
