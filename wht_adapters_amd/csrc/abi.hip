// C ABI of libwhtq: argument validation, then dispatch to the kernels.
// Every check runs before the first HIP call, so an error status means
// nothing was enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/whtq.h"

namespace whtq {

hipError_t launch_stream_probe(const void* src, int64_t in_bytes, void* dst, int64_t out_bytes, hipStream_t s);
hipError_t launch_wht(int logn, int din, int dout, const void* x, void* y, int64_t rows, int64_t ldx,
                      int64_t ldy, const uint32_t* sbits, int sign_mode, float scale, hipStream_t s);
hipError_t launch_rht_quant(int logn, int din, int bits, int logg, const void* w, int64_t rows,
                            int64_t ldw, const uint32_t* sb, uint8_t* codes, uint16_t* scales,
                            hipStream_t s);
hipError_t launch_rht_dequant(int logn, int dout, int bits, int logg, const uint8_t* codes,
                              const uint16_t* scales, int64_t rows, const uint32_t* sb, void* out,
                              int64_t ldo, hipStream_t s);
hipError_t launch_rht_gemv(int logn, int bits, int logg, const void* x, int64_t tokens, int64_t ldx,
                           const uint8_t* codes, const uint16_t* scales, int64_t rows, const uint32_t* sb,
                           void* y, int64_t ldy, hipStream_t s);
hipError_t launch_qwha(const void* x, int64_t tokens, int64_t d_in, int64_t ldx, const int32_t* row_ptr,
                       const int32_t* col_idx, const void* vals, int val_dt, int64_t d_out, int64_t nnz,
                       void* y, int64_t ldy, const void* plan, int64_t plan_bytes, hipStream_t s);
int64_t qwha_fwd_plan_bytes(int64_t tokens, int64_t d_out, int64_t nnz);
hipError_t launch_qwha_fwd_plan(int64_t tokens, const int32_t* row_ptr, int64_t d_out, int64_t nnz, void* plan,
                                int64_t plan_bytes, hipStream_t s);
hipError_t launch_qwha_bwd_input(const void* dy, int64_t tokens, int64_t lddy, int64_t d_out,
                                 const int32_t* t_row_ptr, const int32_t* t_col_idx, const void* t_vals,
                                 int val_dt, int64_t d_in, int64_t nnz, void* dx, int64_t lddx, hipStream_t s);
int64_t qwha_dc_workspace_bytes(int64_t tokens, int64_t d_in, int64_t nnz);
hipError_t launch_qwha_dc(const void* x, int64_t ldx, const void* dy, int64_t lddy, int64_t tokens, int64_t d_in,
                          int64_t d_out, const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                          float* dc, void* workspace, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_permute(const void* vals, int val_dt, const int32_t* perm, int64_t nnz, void* out,
                          hipStream_t s);
hipError_t launch_harp_gen(const void* x, void* y, int xdt, int64_t tokens, int d, int64_t ldx, int64_t ldy,
                           const uint32_t* sbits, int precondition, const int32_t* radices, int n_stages,
                           const void* blocks, int bdt, hipStream_t s);
hipError_t launch_harp_build(const void* params, int pdt, const float* scales, int64_t d, const int32_t* radices,
                             int n_stages, const float* mixers, void* blocks, int bdt, hipStream_t s);
hipError_t launch_harp(const void* x, void* y, int dt, int64_t tokens, int64_t ldx, int64_t ldy,
                       const uint32_t* sbits, int precondition, const void* blocks, int bdt, hipStream_t s);
hipError_t launch_qi_sub(const void* w, int wdt, int64_t ldw, float* f, int64_t ldf, int64_t rows, int64_t n,
                         hipStream_t s);
hipError_t launch_qi_gram(const float* z, int64_t T, int64_t n, float* g, float beta, hipStream_t s);
hipError_t launch_qi_fg(const float* f, int64_t ldf, int64_t rows, int64_t n, const float* g, float* p,
                        hipStream_t s);
hipError_t launch_qi_qform(const float* f, int64_t ldf, const float* p, int64_t rows, int64_t n, float* err,
                           hipStream_t s);
hipError_t launch_qi_select(const float* f, int64_t ldf, int64_t rows, int n, const int32_t* row_ptr,
                            int32_t* col_idx, hipStream_t s);
hipError_t launch_qi_refine(const float* g, int64_t n, const float* p, int64_t rows, const int32_t* row_ptr,
                            const int32_t* col_idx, float* vals, hipStream_t s);

static thread_local int g_last_hip = 0;

static constexpr int kMaxDevices = 64;
static int g_cu[kMaxDevices];
static std::once_flag g_cu_once[kMaxDevices];

int device_cu_count(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev] {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 1)
      cu = 256;
    g_cu[dev] = cu;
  });
  return g_cu[dev];
}

}  // namespace whtq

using namespace whtq;

static whtq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return WHTQ_OK;
  g_last_hip = (int)e;
  return WHTQ_EHIP;
}

// A device must be present and current before anything is launched.
static whtq_status need_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_status(e);
  if (n < 1) return hip_status(hipErrorNoDevice);
  return WHTQ_OK;
}

static int ilog2_pow2(int64_t n) {
  if (n < 1 || (n & (n - 1))) return -1;
  int l = 0;
  while ((int64_t(1) << l) < n) ++l;
  return l;
}

static int dt_bytes(int dt) { return dt == WHTQ_F32 ? 4 : 2; }
static bool dt_valid(int dt) { return dt == WHTQ_F32 || dt == WHTQ_BF16 || dt == WHTQ_F16; }

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Row-matrix alignment rule: 16-byte base and row stride unless a row is
// shorter than 16 bytes, then element alignment.
static bool rows_aligned(const void* p, int64_t n, int64_t ld, int esz) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (n * esz >= 16) return (a & 15u) == 0 && ((ld * esz) & 15) == 0;
  return (a % (uintptr_t)esz) == 0;
}

extern "C" {

int whtq_abi_version(void) { return WHTQ_ABI_VERSION; }

int whtq_last_hip_error(void) { return g_last_hip; }

whtq_status whtq_stream_probe(const void* src, int64_t in_bytes, void* dst, int64_t out_bytes, void* stream) {
  if (in_bytes < 0 || out_bytes < 0 || (in_bytes & 15) || (out_bytes & 15)) return WHTQ_EINVAL;
  if ((in_bytes > 0 && !src) || (out_bytes > 0 && !dst)) return WHTQ_EINVAL;
  if ((src && !aligned16(src)) || (dst && !aligned16(dst))) return WHTQ_EALIGN;
  if (in_bytes == 0 && out_bytes == 0) return WHTQ_OK;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(whtq::launch_stream_probe(src, in_bytes, dst, out_bytes, (hipStream_t)stream));
}

const char* whtq_status_string(whtq_status s) {
  switch (s) {
    case WHTQ_OK: return "ok";
    case WHTQ_EINVAL: return "invalid argument";
    case WHTQ_EUNSUPPORTED: return "unsupported configuration";
    case WHTQ_EALIGN: return "misaligned pointer or row stride";
    case WHTQ_EHIP: return "HIP runtime error";
    case WHTQ_ESCRATCH: return "sizes exceed the fixed scratch capacity";
  }
  return "unknown status";
}

whtq_status wht_batched(const void* x, whtq_dtype x_dtype, void* y, whtq_dtype y_dtype, int64_t rows,
                        int64_t n, int64_t ldx, int64_t ldy, const uint32_t* sign_bits, int sign_mode,
                        int normalize, void* stream) {
  if (!dt_valid(x_dtype) || !dt_valid(y_dtype)) return WHTQ_EINVAL;
  if (rows < 0 || n < 1 || ldx < n || ldy < n) return WHTQ_EINVAL;
  if (sign_mode < WHTQ_SIGN_NONE || sign_mode > WHTQ_SIGN_AFTER) return WHTQ_EINVAL;
  if (sign_mode != WHTQ_SIGN_NONE && !sign_bits) return WHTQ_EINVAL;
  if (normalize != 0 && normalize != 1) return WHTQ_EINVAL;
  if (rows > 0 && (!x || !y)) return WHTQ_EINVAL;
  const int logn = ilog2_pow2(n);
  if (logn < 1 || logn > 13) return WHTQ_EUNSUPPORTED;
  const bool same = x_dtype == y_dtype;
  const bool widen = y_dtype == WHTQ_F32 && x_dtype != WHTQ_F32;
  if (!same && !widen) return WHTQ_EUNSUPPORTED;
  if (x == y && (!same || ldx != ldy)) return WHTQ_EINVAL;
  if (!rows_aligned(x, n, ldx, dt_bytes(x_dtype)) || !rows_aligned(y, n, ldy, dt_bytes(y_dtype)))
    return WHTQ_EALIGN;
  if (sign_bits && (reinterpret_cast<uintptr_t>(sign_bits) & 3u)) return WHTQ_EALIGN;
  if (rows == 0) return WHTQ_OK;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  const float scale = normalize ? (float)(1.0 / std::sqrt((double)n)) : 1.0f;
  return hip_status(launch_wht(logn, x_dtype, y_dtype, x, y, rows, ldx, ldy, sign_bits, sign_mode, scale,
                               (hipStream_t)stream));
}

static whtq_status check_quant_shape(int64_t rows, int64_t n, int bits, int group, int* logn, int* logg) {
  if (rows < 0 || n < 1) return WHTQ_EINVAL;
  if (bits < 2 || bits > 4) return WHTQ_EINVAL;
  if (group < 1 || n % group) return WHTQ_EINVAL;
  *logn = ilog2_pow2(n);
  if (*logn < 0) return WHTQ_EUNSUPPORTED;
  *logg = ilog2_pow2(group);
  if (*logg < 3) return WHTQ_EINVAL;  // group must be a power of two >= 8 (it divides n)
  if (*logn < 6 || *logn > 13 || *logg > 8) return WHTQ_EUNSUPPORTED;
  return WHTQ_OK;
}

whtq_status rht_quantize_rtn(const void* w, whtq_dtype w_dtype, int64_t rows, int64_t n, int64_t ldw,
                             const uint32_t* sign_bits, int bits, int group, uint8_t* codes,
                             uint16_t* scales, void* stream) {
  if (!dt_valid(w_dtype)) return WHTQ_EINVAL;
  int logn = 0, logg = 0;
  whtq_status st = check_quant_shape(rows, n, bits, group, &logn, &logg);
  if (st != WHTQ_OK) return st;
  if (ldw < n) return WHTQ_EINVAL;
  if (rows > 0 && (!w || !codes || !scales)) return WHTQ_EINVAL;
  if (!rows_aligned(w, n, ldw, dt_bytes(w_dtype)) || !aligned16(codes) || !aligned16(scales))
    return WHTQ_EALIGN;
  if (sign_bits && (reinterpret_cast<uintptr_t>(sign_bits) & 3u)) return WHTQ_EALIGN;
  if (rows == 0) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_rht_quant(logn, w_dtype, bits, logg, w, rows, ldw, sign_bits, codes, scales,
                                     (hipStream_t)stream));
}

whtq_status rht_dequantize_inverse(const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t n,
                                   const uint32_t* sign_bits, int bits, int group, void* out,
                                   whtq_dtype out_dtype, int64_t ldo, void* stream) {
  if (!dt_valid(out_dtype)) return WHTQ_EINVAL;
  int logn = 0, logg = 0;
  whtq_status st = check_quant_shape(rows, n, bits, group, &logn, &logg);
  if (st != WHTQ_OK) return st;
  if (ldo < n) return WHTQ_EINVAL;
  if (rows > 0 && (!codes || !scales || !out)) return WHTQ_EINVAL;
  if (!rows_aligned(out, n, ldo, dt_bytes(out_dtype)) || !aligned16(codes) || !aligned16(scales))
    return WHTQ_EALIGN;
  if (sign_bits && (reinterpret_cast<uintptr_t>(sign_bits) & 3u)) return WHTQ_EALIGN;
  if (rows == 0) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_rht_dequant(logn, out_dtype, bits, logg, codes, scales, rows, sign_bits, out, ldo,
                                       (hipStream_t)stream));
}

whtq_status rht_lowbit_gemv(const void* x, int64_t tokens, int64_t ldx, const uint8_t* codes,
                            const uint16_t* scales, int64_t rows, int64_t n, const uint32_t* sign_bits,
                            int bits, int group, void* y, int64_t ldy, void* stream) {
  int logn = 0, logg = 0;
  whtq_status st = check_quant_shape(rows, n, bits, group, &logn, &logg);
  if (st != WHTQ_OK) return st;
  if (tokens < 0 || ldx < n || ldy < rows) return WHTQ_EINVAL;
  if (tokens > 0 && rows > 0 && (!x || !codes || !scales || !y)) return WHTQ_EINVAL;
  if (bits == 3 || (logn != 12 && logn != 13) || (1 << logg) < 32 / bits) return WHTQ_EUNSUPPORTED;
  if (!rows_aligned(x, n, ldx, 2) || !aligned16(codes) || !aligned16(scales) ||
      (reinterpret_cast<uintptr_t>(y) & 1u))
    return WHTQ_EALIGN;
  if (sign_bits && (reinterpret_cast<uintptr_t>(sign_bits) & 3u)) return WHTQ_EALIGN;
  if (tokens == 0 || rows == 0) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_rht_gemv(logn, bits, logg, x, tokens, ldx, codes, scales, rows, sign_bits, y, ldy,
                                    (hipStream_t)stream));
}

// the argument rules of qwha_adapter_forward (shared with the planned form)
static whtq_status qwha_fwd_check(const void* x, whtq_dtype x_dtype, int64_t tokens, int64_t d_in, int64_t ldx,
                                  const int32_t* row_ptr, const int32_t* col_idx, const void* vals,
                                  whtq_dtype val_dtype, int64_t d_out, int64_t nnz, void* y, whtq_dtype y_dtype,
                                  int64_t ldy) {
  if (!dt_valid(x_dtype) || !dt_valid(val_dtype) || !dt_valid(y_dtype)) return WHTQ_EINVAL;
  if (tokens < 0 || d_in < 1 || d_out < 1 || nnz < 0 || ldx < d_in || ldy < d_out) return WHTQ_EINVAL;
  if (nnz > d_in * d_out) return WHTQ_EINVAL;
  if (!row_ptr || (nnz > 0 && (!col_idx || !vals))) return WHTQ_EINVAL;
  if (tokens > 0 && (!x || !y)) return WHTQ_EINVAL;
  if (ilog2_pow2(d_in) < 6 || ilog2_pow2(d_in) > 13 || d_out > 4096) return WHTQ_EUNSUPPORTED;
  if (x_dtype != WHTQ_BF16 || y_dtype != WHTQ_BF16) return WHTQ_EUNSUPPORTED;
  if (val_dtype != WHTQ_BF16 && val_dtype != WHTQ_F32) return WHTQ_EUNSUPPORTED;
  if (!rows_aligned(x, d_in, ldx, 2) || !rows_aligned(y, d_out, ldy, 2)) return WHTQ_EALIGN;
  if ((reinterpret_cast<uintptr_t>(row_ptr) & 3u) || !aligned16(col_idx) || !aligned16(vals)) return WHTQ_EALIGN;
  return WHTQ_OK;
}

whtq_status qwha_adapter_forward(const void* x, whtq_dtype x_dtype, int64_t tokens, int64_t d_in,
                                 int64_t ldx, const int32_t* row_ptr, const int32_t* col_idx,
                                 const void* vals, whtq_dtype val_dtype, int64_t d_out, int64_t nnz,
                                 void* y, whtq_dtype y_dtype, int64_t ldy, void* stream) {
  return qwha_adapter_forward_planned(x, x_dtype, tokens, d_in, ldx, row_ptr, col_idx, vals, val_dtype, d_out, nnz,
                                      nullptr, 0, y, y_dtype, ldy, stream);
}

int64_t qwha_forward_plan_bytes(int64_t tokens, int64_t d_in, int64_t d_out, int64_t nnz) {
  if (tokens < 1 || d_out < 1 || d_out > 4096 || nnz < 0 || nnz > d_in * d_out) return -1;
  if (ilog2_pow2(d_in) < 6 || ilog2_pow2(d_in) > 13) return -1;
  if (d_in > 4096) return 0;  // the d_in = 8192 kernel prepares nothing per chunk
  if (need_device() != WHTQ_OK) return -1;
  return qwha_fwd_plan_bytes(tokens, d_out, nnz);
}

whtq_status qwha_forward_plan(int64_t tokens, int64_t d_in, const int32_t* row_ptr, int64_t d_out, int64_t nnz,
                              void* plan, int64_t plan_bytes, void* stream) {
  if (tokens < 1 || d_out < 1 || nnz < 0 || nnz > d_in * d_out || plan_bytes < 0) return WHTQ_EINVAL;
  if (!row_ptr || (reinterpret_cast<uintptr_t>(row_ptr) & 3u)) return row_ptr ? WHTQ_EALIGN : WHTQ_EINVAL;
  if (ilog2_pow2(d_in) < 6 || ilog2_pow2(d_in) > 13 || d_out > 4096) return WHTQ_EUNSUPPORTED;
  if (d_in > 4096) return WHTQ_OK;  // nothing to plan
  if (!plan) return WHTQ_EINVAL;
  if (!aligned16(plan)) return WHTQ_EALIGN;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  if (plan_bytes < qwha_fwd_plan_bytes(tokens, d_out, nnz)) return WHTQ_EINVAL;
  return hip_status(launch_qwha_fwd_plan(tokens, row_ptr, d_out, nnz, plan, plan_bytes, (hipStream_t)stream));
}

whtq_status qwha_adapter_forward_planned(const void* x, whtq_dtype x_dtype, int64_t tokens, int64_t d_in,
                                         int64_t ldx, const int32_t* row_ptr, const int32_t* col_idx,
                                         const void* vals, whtq_dtype val_dtype, int64_t d_out, int64_t nnz,
                                         const void* plan, int64_t plan_bytes, void* y, whtq_dtype y_dtype,
                                         int64_t ldy, void* stream) {
  whtq_status st = qwha_fwd_check(x, x_dtype, tokens, d_in, ldx, row_ptr, col_idx, vals, val_dtype, d_out, nnz, y,
                                  y_dtype, ldy);
  if (st != WHTQ_OK) return st;
  if (plan_bytes < 0 || (plan && plan_bytes < 256)) return WHTQ_EINVAL;
  if (plan && !aligned16(plan)) return WHTQ_EALIGN;
  if (tokens == 0) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_qwha(x, tokens, d_in, ldx, row_ptr, col_idx, vals, val_dtype, d_out, nnz, y, ldy,
                                plan, plan ? plan_bytes : 0, (hipStream_t)stream));
}

whtq_status qwha_csr_transpose(const int32_t* row_ptr, const int32_t* col_idx, int64_t d_out, int64_t d_in,
                               int64_t nnz, int32_t* t_row_ptr, int32_t* t_col_idx, int32_t* t_perm) {
  if (d_out < 1 || d_in < 1 || nnz < 0 || d_out > INT32_MAX || d_in > INT32_MAX || nnz > INT32_MAX)
    return WHTQ_EINVAL;
  if (!row_ptr || !t_row_ptr || (nnz > 0 && (!col_idx || !t_col_idx || !t_perm))) return WHTQ_EINVAL;
  // the CSR is read here, so it is checked in full first
  if (row_ptr[0] != 0 || row_ptr[d_out] != nnz) return WHTQ_EINVAL;
  for (int64_t o = 0; o < d_out; ++o)
    if (row_ptr[o + 1] < row_ptr[o]) return WHTQ_EINVAL;
  for (int64_t j = 0; j < nnz; ++j)
    if (col_idx[j] < 0 || col_idx[j] >= d_in) return WHTQ_EINVAL;
  // counting sort by column, stable in entry order (rows ascending within a
  // column); t_row_ptr[k] serves as column k's cursor, then shifts back
  for (int64_t k = 0; k <= d_in; ++k) t_row_ptr[k] = 0;
  for (int64_t j = 0; j < nnz; ++j) ++t_row_ptr[col_idx[j] + 1];
  for (int64_t k = 0; k < d_in; ++k) t_row_ptr[k + 1] += t_row_ptr[k];
  for (int64_t o = 0; o < d_out; ++o)
    for (int32_t j = row_ptr[o]; j < row_ptr[o + 1]; ++j) {
      const int32_t pos = t_row_ptr[col_idx[j]]++;
      t_col_idx[pos] = (int32_t)o;
      t_perm[pos] = j;
    }
  for (int64_t k = d_in; k > 0; --k) t_row_ptr[k] = t_row_ptr[k - 1];
  t_row_ptr[0] = 0;
  return WHTQ_OK;
}

whtq_status qwha_permute_values(const void* vals, whtq_dtype val_dtype, const int32_t* perm, int64_t nnz,
                                void* out, void* stream) {
  if (!dt_valid(val_dtype) || nnz < 0) return WHTQ_EINVAL;
  if (nnz > 0 && (!vals || !perm || !out)) return WHTQ_EINVAL;
  if (nnz > 0 && vals == out) return WHTQ_EINVAL;
  if (val_dtype == WHTQ_F16) return WHTQ_EUNSUPPORTED;
  const uintptr_t esz = (uintptr_t)dt_bytes(val_dtype);
  if ((reinterpret_cast<uintptr_t>(vals) % esz) || (reinterpret_cast<uintptr_t>(out) % esz) ||
      (reinterpret_cast<uintptr_t>(perm) & 3u))
    return WHTQ_EALIGN;
  if (nnz == 0) return WHTQ_OK;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_permute(vals, val_dtype, perm, nnz, out, (hipStream_t)stream));
}

whtq_status qwha_adapter_backward_input(const void* dy, whtq_dtype dy_dtype, int64_t tokens, int64_t d_out,
                                        int64_t lddy, const int32_t* t_row_ptr, const int32_t* t_col_idx,
                                        const void* t_vals, whtq_dtype val_dtype, int64_t d_in, int64_t nnz,
                                        void* dx, whtq_dtype dx_dtype, int64_t lddx, void* stream) {
  if (!dt_valid(dy_dtype) || !dt_valid(val_dtype) || !dt_valid(dx_dtype)) return WHTQ_EINVAL;
  if (tokens < 0 || d_in < 1 || d_out < 1 || nnz < 0 || lddy < d_out || lddx < d_in) return WHTQ_EINVAL;
  if (nnz > d_in * d_out) return WHTQ_EINVAL;
  if (!t_row_ptr || (nnz > 0 && (!t_col_idx || !t_vals))) return WHTQ_EINVAL;
  if (tokens > 0 && (!dy || !dx)) return WHTQ_EINVAL;
  if (ilog2_pow2(d_in) < 6 || ilog2_pow2(d_in) > 13 || d_out > 4096) return WHTQ_EUNSUPPORTED;
  if (dy_dtype != WHTQ_BF16 || dx_dtype != WHTQ_BF16) return WHTQ_EUNSUPPORTED;
  if (val_dtype != WHTQ_BF16 && val_dtype != WHTQ_F32) return WHTQ_EUNSUPPORTED;
  // dy: element alignment suffices (16-byte loads are used where its rows allow them)
  if ((reinterpret_cast<uintptr_t>(dy) & 1u) || !rows_aligned(dx, d_in, lddx, 2)) return WHTQ_EALIGN;
  if ((reinterpret_cast<uintptr_t>(t_row_ptr) & 3u) || !aligned16(t_col_idx) || !aligned16(t_vals))
    return WHTQ_EALIGN;
  if (tokens == 0) return WHTQ_OK;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_qwha_bwd_input(dy, tokens, lddy, d_out, t_row_ptr, t_col_idx, t_vals, val_dtype, d_in,
                                          nnz, dx, lddx, (hipStream_t)stream));
}

int64_t qwha_grad_values_workspace_bytes(int64_t tokens, int64_t d_in, int64_t nnz) {
  if (tokens < 0 || nnz < 0 || ilog2_pow2(d_in) < 6 || ilog2_pow2(d_in) > 13) return -1;
  if (tokens == 0 || nnz == 0) return 0;
  return qwha_dc_workspace_bytes(tokens, d_in, nnz);
}

whtq_status qwha_adapter_grad_values(const void* x, const void* dy, whtq_dtype dtype, int64_t tokens,
                                     int64_t d_in, int64_t d_out, int64_t ldx, int64_t lddy,
                                     const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz, float* dc,
                                     void* workspace, int64_t workspace_bytes, void* stream) {
  if (!dt_valid(dtype)) return WHTQ_EINVAL;
  if (tokens < 0 || d_in < 1 || d_out < 1 || nnz < 0 || ldx < d_in || lddy < d_out) return WHTQ_EINVAL;
  if (nnz > d_in * d_out || nnz > INT32_MAX) return WHTQ_EINVAL;
  if (!row_ptr || (nnz > 0 && (!col_idx || !dc))) return WHTQ_EINVAL;
  if (tokens > 0 && nnz > 0 && (!x || !dy || !workspace)) return WHTQ_EINVAL;
  if (ilog2_pow2(d_in) < 6 || ilog2_pow2(d_in) > 13 || d_out > 4096) return WHTQ_EUNSUPPORTED;
  if (dtype != WHTQ_BF16) return WHTQ_EUNSUPPORTED;
  // dy is read with element loads: element alignment suffices
  if (!rows_aligned(x, d_in, ldx, 2) || (reinterpret_cast<uintptr_t>(dy) & 1u)) return WHTQ_EALIGN;
  if ((reinterpret_cast<uintptr_t>(row_ptr) & 3u) || (reinterpret_cast<uintptr_t>(col_idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(dc) & 3u) || !aligned16(workspace))
    return WHTQ_EALIGN;
  if (tokens > 0 && nnz > 0 && workspace_bytes < qwha_dc_workspace_bytes(tokens, d_in, nnz)) return WHTQ_EINVAL;
  if (nnz == 0) return WHTQ_OK;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  if (tokens == 0)  // an empty sum: dc = 0 (a fill kernel, not a memset node)
    return hip_status(launch_fill_zero(dc, nnz, (hipStream_t)stream));
  return hip_status(launch_qwha_dc(x, ldx, dy, lddy, tokens, d_in, d_out, row_ptr, col_idx, nnz, dc, workspace,
                                   (hipStream_t)stream));
}

}  // extern "C"

// Scratch of the allocation-free value gradient: one array per GPU, resolved
// to a device address once per device with that device current (the array's
// name in host code is only a host-side handle, never a device address).
static __device__ __align__(256) uint8_t scratch[WHTQ_QWHA_DC_SCRATCH_BYTES];
static void* g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];

static whtq_status scratch_of_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return WHTQ_EUNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_status(g_scratch_err[dev]);
  *ptr = g_scratch_ptr[dev];
  return WHTQ_OK;
}

extern "C" {

whtq_status qwha_adapter_grad_values_noalloc(const void* x, const void* dy, whtq_dtype dtype, int64_t tokens,
                                             int64_t d_in, int64_t d_out, int64_t ldx, int64_t lddy,
                                             const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                             float* dc, void* stream) {
  // the same checks as qwha_adapter_grad_values, then the capacity
  if (!dt_valid(dtype)) return WHTQ_EINVAL;
  if (tokens < 0 || d_in < 1 || d_out < 1 || nnz < 0 || ldx < d_in || lddy < d_out) return WHTQ_EINVAL;
  if (nnz > d_in * d_out || nnz > INT32_MAX) return WHTQ_EINVAL;
  if (!row_ptr || (nnz > 0 && (!col_idx || !dc))) return WHTQ_EINVAL;
  if (tokens > 0 && nnz > 0 && (!x || !dy)) return WHTQ_EINVAL;
  if (ilog2_pow2(d_in) < 6 || ilog2_pow2(d_in) > 13 || d_out > 4096) return WHTQ_EUNSUPPORTED;
  if (dtype != WHTQ_BF16) return WHTQ_EUNSUPPORTED;
  if (!rows_aligned(x, d_in, ldx, 2) || (reinterpret_cast<uintptr_t>(dy) & 1u)) return WHTQ_EALIGN;
  if ((reinterpret_cast<uintptr_t>(row_ptr) & 3u) || (reinterpret_cast<uintptr_t>(col_idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(dc) & 3u))
    return WHTQ_EALIGN;
  if (tokens > 0 && nnz > 0 && qwha_dc_workspace_bytes(tokens, d_in, nnz) > WHTQ_QWHA_DC_SCRATCH_BYTES)
    return WHTQ_ESCRATCH;
  if (nnz == 0) return WHTQ_OK;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  if (tokens == 0) return hip_status(launch_fill_zero(dc, nnz, (hipStream_t)stream));
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != WHTQ_OK) return st;
  return hip_status(launch_qwha_dc(x, ldx, dy, lddy, tokens, d_in, d_out, row_ptr, col_idx, nnz, dc, ws,
                                   (hipStream_t)stream));
}

whtq_status harp_rotate(const void* x, void* y, whtq_dtype dtype, int64_t tokens, int64_t d, int64_t ldx,
                        int64_t ldy, const uint32_t* sign_bits, int precondition, const int32_t* radices,
                        int n_stages, const void* blocks, whtq_dtype blocks_dtype, void* stream) {
  if (!dt_valid(dtype) || !dt_valid(blocks_dtype)) return WHTQ_EINVAL;
  if (tokens < 0 || d < 1 || ldx < d || ldy < d) return WHTQ_EINVAL;
  if (!radices || n_stages < 1 || n_stages > 64 || !blocks) return WHTQ_EINVAL;
  if (precondition != 0 && precondition != 1) return WHTQ_EINVAL;
  int64_t prod = 1;
  for (int t = 0; t < n_stages; ++t) {
    if (radices[t] < 2) return WHTQ_EINVAL;
    prod *= radices[t];
    if (prod > d) return WHTQ_EINVAL;
  }
  if (prod != d) return WHTQ_EINVAL;
  if (tokens > 0 && (!x || !y)) return WHTQ_EINVAL;
  if (tokens > 0 && x == y) return WHTQ_EINVAL;
  // the preconditioning is the Sylvester RHT, which exists for powers of two only
  if (precondition && ilog2_pow2(d) < 0) return WHTQ_EINVAL;
  // fp32 rows take the fp32-tile kernel for every schedule (the radix-16 one
  // multiplies in fp16)
  const bool r16 = dtype == WHTQ_BF16 && d == 4096 && n_stages == 3 && radices[0] == 16 && radices[1] == 16 &&
                   radices[2] == 16;
  if (!r16) {
    if (d > 8192 || n_stages > 16) return WHTQ_EUNSUPPORTED;
    for (int t = 0; t < n_stages; ++t)
      if (radices[t] > 16) return WHTQ_EUNSUPPORTED;
  }
  if ((dtype != WHTQ_BF16 && dtype != WHTQ_F32) || blocks_dtype == WHTQ_BF16) return WHTQ_EUNSUPPORTED;
  const int esz = dt_bytes(dtype);
  if (!rows_aligned(x, d, ldx, esz) || !rows_aligned(y, d, ldy, esz) || !aligned16(blocks)) return WHTQ_EALIGN;
  if (sign_bits && (reinterpret_cast<uintptr_t>(sign_bits) & 3u)) return WHTQ_EALIGN;
  if (tokens == 0) return WHTQ_OK;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  if (r16)
    return hip_status(launch_harp(x, y, dtype, tokens, ldx, ldy, sign_bits, precondition, blocks, blocks_dtype,
                                  (hipStream_t)stream));
  return hip_status(launch_harp_gen(x, y, dtype, tokens, (int)d, ldx, ldy, sign_bits, precondition, radices, n_stages,
                                    blocks, blocks_dtype, (hipStream_t)stream));
}

whtq_status harp_build_blocks(const void* params, whtq_dtype params_dtype, const float* scales, int64_t d,
                              const int32_t* radices, int n_stages, const float* mixers, void* blocks,
                              whtq_dtype blocks_dtype, void* stream) {
  if (params_dtype != WHTQ_F32 && params_dtype != WHTQ_I8) return WHTQ_EINVAL;
  if (blocks_dtype != WHTQ_F32 && blocks_dtype != WHTQ_F16) return WHTQ_EINVAL;
  if (!radices || n_stages < 1 || n_stages > 64 || d < 1 || !params || !blocks) return WHTQ_EINVAL;
  if (params_dtype == WHTQ_I8 && !scales) return WHTQ_EINVAL;
  int64_t prod = 1;
  bool pow2 = true;
  for (int t = 0; t < n_stages; ++t) {
    if (radices[t] < 2) return WHTQ_EINVAL;
    prod *= radices[t];
    if (prod > d) return WHTQ_EINVAL;
    pow2 = pow2 && (radices[t] & (radices[t] - 1)) == 0;
  }
  if (prod != d) return WHTQ_EINVAL;
  // the Sylvester mixer exists for power-of-two radices only
  if (!mixers && !pow2) return WHTQ_EINVAL;
  if (n_stages > 16 || d > (int64_t(1) << 24)) return WHTQ_EUNSUPPORTED;
  for (int t = 0; t < n_stages; ++t)
    if (radices[t] > 16) return WHTQ_EUNSUPPORTED;
  if ((params_dtype == WHTQ_F32 && (reinterpret_cast<uintptr_t>(params) & 3u)) ||
      (reinterpret_cast<uintptr_t>(blocks) % (uintptr_t)dt_bytes(blocks_dtype)) ||
      (reinterpret_cast<uintptr_t>(mixers) & 3u) || (reinterpret_cast<uintptr_t>(scales) & 3u))
    return WHTQ_EALIGN;
  whtq_status st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_harp_build(params, params_dtype, scales, d, radices, n_stages, mixers, blocks,
                                      blocks_dtype, (hipStream_t)stream));
}


// ---------------------------------------------------------------- QWHA initialisation

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// n of the initialisation calls after the error coefficients: a power of two in [256, 8192]
static whtq_status qi_n(int64_t n) {
  const int l = ilog2_pow2(n);
  if (l < 0) return WHTQ_EINVAL;
  if (l < 8 || l > 13) return WHTQ_EUNSUPPORTED;
  return WHTQ_OK;
}

whtq_status qwha_init_error_coeffs(const void* w, whtq_dtype w_dtype, int64_t rows, int64_t n, int64_t ldw,
                                   const uint8_t* codes, const uint16_t* scales, const uint32_t* sign_bits,
                                   int bits, int group, float* f, int64_t ldf, void* stream) {
  if (!dt_valid(w_dtype)) return WHTQ_EINVAL;
  int logn = 0, logg = 0;
  whtq_status st = check_quant_shape(rows, n, bits, group, &logn, &logg);
  if (st != WHTQ_OK) return st;
  if (ldw < n || ldf < n) return WHTQ_EINVAL;
  if (rows > 0 && (!w || !codes || !scales || !f)) return WHTQ_EINVAL;
  if (rows > 0 && static_cast<const void*>(f) == w) return WHTQ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(w) % (uintptr_t)dt_bytes(w_dtype)) || !rows_aligned(f, n, ldf, 4) ||
      !aligned16(codes) || !aligned16(scales))
    return WHTQ_EALIGN;
  if (sign_bits && !aligned4(sign_bits)) return WHTQ_EALIGN;
  if (rows == 0) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_rht_dequant(logn, WHTQ_F32, bits, logg, codes, scales, rows, sign_bits, f, ldf, s);
  if (e == hipSuccess) e = launch_qi_sub(w, w_dtype, ldw, f, ldf, rows, n, s);
  if (e == hipSuccess)
    e = launch_wht(logn, WHTQ_F32, WHTQ_F32, f, f, rows, ldf, ldf, nullptr, WHTQ_SIGN_NONE,
                   (float)(1.0 / std::sqrt((double)n)), s);
  return hip_status(e);
}

whtq_status qwha_init_gram(const void* x, whtq_dtype x_dtype, int64_t tokens, int64_t n, int64_t ldx, float* z,
                           float* g, int accumulate, void* stream) {
  if (!dt_valid(x_dtype)) return WHTQ_EINVAL;
  whtq_status st = qi_n(n);
  if (st != WHTQ_OK) return st;
  if (tokens < 0 || ldx < n || (accumulate != 0 && accumulate != 1)) return WHTQ_EINVAL;
  if (!g || (tokens > 0 && (!x || !z))) return WHTQ_EINVAL;
  if (tokens > 0 && z == g) return WHTQ_EINVAL;  // Z is read while G is written
  if (!rows_aligned(x, n, ldx, dt_bytes(x_dtype)) || !aligned16(z) || !aligned16(g)) return WHTQ_EALIGN;
  if (tokens == 0 && accumulate) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (tokens > 0)
    e = launch_wht(ilog2_pow2(n), x_dtype, WHTQ_F32, x, z, tokens, ldx, n, nullptr, WHTQ_SIGN_NONE,
                   (float)(1.0 / std::sqrt((double)n)), s);
  if (e == hipSuccess) e = launch_qi_gram(z, tokens, n, g, accumulate ? 1.f : 0.f, s);
  return hip_status(e);
}

whtq_status qwha_init_channel_errors(const float* f, int64_t rows, int64_t n, int64_t ldf, const float* g,
                                     float* p, float* err, void* stream) {
  whtq_status st = qi_n(n);
  if (st != WHTQ_OK) return st;
  if (rows < 0 || ldf < n) return WHTQ_EINVAL;
  if (rows > 0 && (!f || !g || !p || !err)) return WHTQ_EINVAL;
  if (rows > 0 && (p == f || p == g || static_cast<const void*>(err) == static_cast<const void*>(f) ||
                   static_cast<const void*>(err) == static_cast<const void*>(g) || err == p))
    return WHTQ_EINVAL;  // outputs must not overlay the inputs
  if (!rows_aligned(f, n, ldf, 4) || !aligned16(g) || !aligned16(p) || !aligned4(err)) return WHTQ_EALIGN;
  if (rows == 0) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_qi_fg(f, ldf, rows, n, g, p, s);
  if (e == hipSuccess) e = launch_qi_qform(f, ldf, p, rows, n, err, s);
  return hip_status(e);
}

whtq_status qwha_init_allocate(const float* err, int64_t rows, int64_t n, int64_t total, int floor, int cap,
                               int32_t* row_ptr) {
  if (rows < 1 || n < 1 || !err || !row_ptr) return WHTQ_EINVAL;
  if (floor < 0 || cap < floor || cap > n) return WHTQ_EINVAL;
  if (cap > WHTQ_QWHA_INIT_MAX_SUPPORT) return WHTQ_EUNSUPPORTED;
  if (total < (int64_t)floor * rows || total > (int64_t)cap * rows || total > INT32_MAX) return WHTQ_EINVAL;
  bool any = false;
  for (int64_t o = 0; o < rows; ++o) {
    if (!std::isfinite(err[o]) || err[o] < 0.f) return WHTQ_EINVAL;
    any = any || err[o] > 0.f;
  }
  const double p = (double)total;
  std::vector<double> e64(err, err + rows);
  auto budget = [&](double lam) {  // four independent partial sums (vectorisable)
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    const double lo_v = (double)floor, hi_v = (double)cap;
    int64_t o = 0;
    for (; o + 4 <= rows; o += 4)
      for (int q = 0; q < 4; ++q) acc[q] += std::min(hi_v, std::max(lo_v, lam * e64[o + q]));
    for (; o < rows; ++o) acc[0] += std::min(hi_v, std::max(lo_v, lam * e64[o]));
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };
  std::vector<double> real(rows);
  if (!any) {
    std::fill(real.begin(), real.end(), p / (double)rows);
  } else {
    // water level: the sum of clip(lam e, floor, cap) is continuous and
    // non-decreasing in lam; the largest lam found with sum <= p leaves a
    // non-negative remainder for the rounding below
    double lo = 0.0, hi = 1.0;
    int doublings = 0;
    while (budget(hi) < p) {
      hi *= 2.0;
      if (++doublings > 2100) return WHTQ_EINVAL;  // channels without error sit at the floor
    }
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (mid == lo || mid == hi) break;  // adjacent doubles: further steps change nothing
      if (budget(mid) < p) lo = mid;
      else hi = mid;
    }
    for (int64_t o = 0; o < rows; ++o)
      real[o] = std::min((double)cap, std::max((double)floor, lo * (double)err[o]));
  }
  std::vector<int64_t> base(rows);
  std::vector<int64_t> order;
  int64_t sum = 0;
  for (int64_t o = 0; o < rows; ++o) {
    base[o] = (int64_t)std::floor(real[o]);
    sum += base[o];
    if (base[o] < cap) order.push_back(o);
  }
  const int64_t rem = total - sum;
  if (rem < 0 || rem > (int64_t)order.size()) return WHTQ_EINVAL;
  // the rem channels of largest fractional part, ties to the lower channel index
  if (rem > 0 && rem < (int64_t)order.size())
    std::nth_element(order.begin(), order.begin() + rem, order.end(), [&](int64_t a, int64_t b) {
      const double fa = real[a] - (double)base[a], fb = real[b] - (double)base[b];
      return fa > fb || (fa == fb && a < b);
    });
  for (int64_t q = 0; q < rem; ++q) ++base[order[q]];
  row_ptr[0] = 0;
  for (int64_t o = 0; o < rows; ++o) row_ptr[o + 1] = row_ptr[o] + (int32_t)base[o];
  return WHTQ_OK;
}

whtq_status qwha_init_select(const float* f, int64_t rows, int64_t n, int64_t ldf, const int32_t* row_ptr,
                             int32_t* col_idx, void* stream) {
  whtq_status st = qi_n(n);
  if (st != WHTQ_OK) return st;
  if (rows < 0 || ldf < n) return WHTQ_EINVAL;
  if (rows > 0 && (!f || !row_ptr || !col_idx)) return WHTQ_EINVAL;
  if (rows > INT32_MAX) return WHTQ_EUNSUPPORTED;
  if (!rows_aligned(f, n, ldf, 4) || !aligned4(row_ptr) || !aligned4(col_idx)) return WHTQ_EALIGN;
  if (rows == 0) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_qi_select(f, ldf, rows, (int)n, row_ptr, col_idx, (hipStream_t)stream));
}

whtq_status qwha_init_refine(const float* g, int64_t n, const float* p, int64_t rows, const int32_t* row_ptr,
                             const int32_t* col_idx, float* vals, void* stream) {
  whtq_status st = qi_n(n);
  if (st != WHTQ_OK) return st;
  if (rows < 0) return WHTQ_EINVAL;
  if (rows > 0 && (!g || !p || !row_ptr || !col_idx || !vals)) return WHTQ_EINVAL;
  if (rows > INT32_MAX) return WHTQ_EUNSUPPORTED;
  if (!aligned4(g) || !aligned4(p) || !aligned4(row_ptr) || !aligned4(col_idx) || !aligned4(vals))
    return WHTQ_EALIGN;
  if (rows == 0) return WHTQ_OK;
  st = need_device();
  if (st != WHTQ_OK) return st;
  return hip_status(launch_qi_refine(g, n, p, rows, row_ptr, col_idx, vals, (hipStream_t)stream));
}

}  // extern "C"
