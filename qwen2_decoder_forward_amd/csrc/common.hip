// Host side of the shared helpers: error messages and descriptor checks.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

namespace q2 {

static thread_local std::string g_err;

q2_status fail(q2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

void clear_error() { g_err.clear(); }

q2_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(Q2_EHIP, "launch of %s failed: %s", what, hipGetErrorString(e));
  return Q2_OK;
}

q2_status check_desc(const q2_tensor* t, const char* name) {
  Q2_CHECK(t != nullptr, Q2_EINVAL, "%s: null descriptor", name);
  Q2_CHECK(t->ndim >= 1 && t->ndim <= Q2_MAX_DIMS, Q2_ESHAPE, "%s: rank %d not in [1, %d]", name, t->ndim,
           Q2_MAX_DIMS);
  Q2_CHECK(dtype_valid(t->dtype), Q2_EDTYPE, "%s: unknown dtype %d", name, t->dtype);
  for (int i = 0; i < t->ndim; ++i) {
    Q2_CHECK(t->shape[i] >= 0, Q2_ESHAPE, "%s: negative size in dim %d", name, i);
    Q2_CHECK(t->stride[i] >= 0, Q2_ESTRIDE, "%s: negative stride in dim %d", name, i);
  }
  Q2_CHECK(t->data != nullptr || numel(*t) == 0, Q2_EINVAL, "%s: null data pointer", name);
  return Q2_OK;
}

bool same_shape(const q2_tensor& a, const q2_tensor& b) {
  if (a.ndim != b.ndim) return false;
  for (int i = 0; i < a.ndim; ++i)
    if (a.shape[i] != b.shape[i]) return false;
  return true;
}

bool is_contiguous(const q2_tensor& t) {
  int64_t s = 1;
  for (int i = t.ndim - 1; i >= 0; --i) {
    if (t.shape[i] != 1 && t.stride[i] != s) return false;
    s *= t.shape[i];
  }
  return true;
}

q2_status as_rows(const q2_tensor* t, const char* name, Rows* out) {
  Q2_TRY(check_desc(t, name));
  const int nd = t->ndim;
  out->data = static_cast<char*>(t->data);
  out->dtype = t->dtype;
  out->cols = t->shape[nd - 1];
  Q2_CHECK(t->stride[nd - 1] == 1 || t->shape[nd - 1] <= 1, Q2_ESTRIDE, "%s: last dim must be contiguous", name);
  int64_t rows = 1;
  for (int i = 0; i < nd - 1; ++i) rows *= t->shape[i];
  out->rows = rows;
  // Outer dims must collapse to a single stride: stride[i] = stride[i+1] * shape[i+1].
  int64_t ld = out->cols;
  int inner = -1;
  for (int i = nd - 2; i >= 0; --i) {
    if (t->shape[i] == 1) continue;
    if (inner < 0) {
      ld = t->stride[i];
    } else {
      Q2_CHECK(t->stride[i] == t->stride[inner] * t->shape[inner], Q2_ESTRIDE,
               "%s: outer dims do not collapse to one row stride", name);
    }
    inner = i;
  }
  Q2_CHECK(rows <= 1 || ld >= out->cols, Q2_ESTRIDE, "%s: overlapping rows", name);
  out->ld = ld;
  return Q2_OK;
}

}  // namespace q2

extern "C" const char* q2_last_error(void) { return q2::g_err.c_str(); }
extern "C" const char* q2_version(void) { return "q2 0.1 (gfx950)"; }
