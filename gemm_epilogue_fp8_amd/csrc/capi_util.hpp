// Host-side helpers shared by the C-ABI translation units: error reporting,
// argument validation and workspace carving.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/coda.h"
#include "epilogues.hpp"

namespace coda {
std::string& last_error_slot();
}

namespace {
using coda::EpiArgs;
using coda::GemmArgs;

coda_status fail(coda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  coda::last_error_slot() = buf;
  return st;
}

#define TRY(expr)                          \
  do {                                     \
    coda_status _s = (expr);               \
    if (_s != CODA_OK) return _s;          \
  } while (0)

int esize(int dt) {
  return dt == CODA_BF16 ? 2
         : (dt == CODA_E4M3 || dt == CODA_E8M0 || dt == CODA_E2M1X2 || dt == CODA_E2M3 || dt == CODA_E3M2) ? 1
                                                                                                            : 4;
}
int vec_elems(int dt) { return 16 / esize(dt); }

bool present(const coda_mat* m) { return m != nullptr && m->ptr != nullptr; }

// Checks a matrix argument.  rows/cols < 0 = any.  A 1 x n vector only needs
// 16-byte alignment; a matrix needs cols and ld to be multiples of 16 bytes.
coda_status check_mat(const coda_mat* m, const char* name, int dtype, int64_t rows, int64_t cols,
                      bool optional = false) {
  if (!present(m)) {
    if (optional) return CODA_OK;
    // a matrix with no elements needs no memory: its pointer may be NULL
    // (it is then checked like any other and never dereferenced); a NULL
    // descriptor of the wrong type (e.g. all zeros) counts as missing
    if (m == nullptr || (m->rows != 0 && m->cols != 0) || m->dtype != dtype)
      return fail(CODA_ERR_NULL, "%s: required pointer is NULL", name);
  }
  if (m->dtype != dtype) return fail(CODA_ERR_DTYPE, "%s: dtype %d, expected %d", name, m->dtype, dtype);
  if (m->rows < 0 || m->cols < 0) return fail(CODA_ERR_SHAPE, "%s: negative size", name);
  if (rows >= 0 && m->rows != rows)
    return fail(CODA_ERR_SHAPE, "%s: %lld rows, expected %lld", name, (long long)m->rows, (long long)rows);
  if (cols >= 0 && m->cols != cols)
    return fail(CODA_ERR_SHAPE, "%s: %lld cols, expected %lld", name, (long long)m->cols, (long long)cols);
  if (reinterpret_cast<uintptr_t>(m->ptr) % 16 != 0) return fail(CODA_ERR_ALIGN, "%s: pointer not 16-byte aligned", name);
  if (m->rows > 1 && m->cols > 0) {   // rows of no elements have no layout
    if (m->ld < m->cols) return fail(CODA_ERR_LAYOUT, "%s: ld %lld < cols %lld", name, (long long)m->ld, (long long)m->cols);
    const int v = vec_elems(dtype);
    if (m->cols % v != 0 || m->ld % v != 0)
      return fail(CODA_ERR_LAYOUT, "%s: cols and ld must be multiples of %d elements", name, v);
    // a tile spans at most 256 rows, addressed by 32-bit byte offsets
    if (m->ld * esize(dtype) >= (int64_t(1) << 24))
      return fail(CODA_ERR_LAYOUT, "%s: row stride of %lld bytes, at most 16 MiB - 1 supported", name,
                  (long long)(m->ld * esize(dtype)));
  }
  if (m->rows > 0x7FFFFFFF || m->cols > 0x7FFFFFFF) return fail(CODA_ERR_SHAPE, "%s: too large", name);
  return CODA_OK;
}

coda_status check_vec(const coda_mat* m, const char* name, int dtype, int64_t n, bool optional = false) {
  TRY(check_mat(m, name, dtype, -1, -1, optional));
  if (!present(m)) return CODA_OK;
  if (m->rows * m->cols != n || (m->rows != 1 && m->cols != 1))
    return fail(CODA_ERR_SHAPE, "%s: expected a vector of %lld elements", name, (long long)n);
  return CODA_OK;
}

const float* fptr(const coda_mat* m) { return present(m) ? static_cast<const float*>(m->ptr) : nullptr; }

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

coda_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    if (e == hipErrorInvalidValue) return fail(CODA_ERR_UNSUPPORTED, "%s: program not compiled", what);
    return fail(CODA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  }
  return CODA_OK;
}
coda_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CODA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return CODA_OK;
}

// Workspace carver: the same sequence of take() calls sizes (base == null)
// and then carves (base != null) the caller's buffer; 256-byte alignment.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

coda_status ws_check(const Carver& c, size_t have, void* ws) {
  if (c.off > 0 && (ws == nullptr || have < c.off))
    return fail(CODA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", c.off, have);
  if (ws != nullptr && reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(CODA_ERR_ALIGN, "workspace must be 256-byte aligned");
  return CODA_OK;
}

EpiArgs epi0() {
  EpiArgs e;
  memset(&e, 0, sizeof(e));
  e.alpha = 1.0f;
  return e;
}

GemmArgs gemm_args(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N, int64_t K) {
  GemmArgs g;
  g.A = A; g.B = B; g.lda = lda; g.ldb = ldb;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.tiles_m = g.tiles_n = 0;
  g.kchunk = (int)K;
  g.sA = g.sB = nullptr;
  g.lds_a = g.lds_b = 0;
  return g;
}

}  // namespace
