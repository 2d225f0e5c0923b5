// Host-only argument validation for the libmuon entry points. Pure C++ (no
// HIP): it runs before anything is enqueued, so an invalid call touches no
// device memory. Rules are the ones stated in include/libmuon.h.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/libmuon.h"
#include "validate.hpp"

namespace muon {

namespace {

int fail(char* msg, int len, int code, const char* fmt, ...) {
  if (msg && len > 0) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, (size_t)len, fmt, ap);
    va_end(ap);
  }
  return code;
}

bool finitef(float x) { return isfinite(x) != 0; }

int elem_size(int32_t dt) { return dt == MUON_BF16 ? 2 : 4; }

// One descriptor. `need_ptr`: a non-empty matrix must have a pointer.
int check_matrix(const muon_matrix& m, const char* what, int i, char* msg, int len) {
  if (m.dtype != MUON_F32 && m.dtype != MUON_BF16)
    return fail(msg, len, MUON_ERR_UNSUPPORTED_DTYPE, "%s[%d]: dtype %d is not MUON_F32 or MUON_BF16", what, i,
                (int)m.dtype);
  if (m.rows < 0 || m.cols < 0)
    return fail(msg, len, MUON_ERR_SHAPE_MISMATCH, "%s[%d]: negative shape %lld x %lld", what, i,
                (long long)m.rows, (long long)m.cols);
  if (m.rows == 0 || m.cols == 0) return MUON_OK;
  if (!m.ptr) return fail(msg, len, MUON_ERR_INVALID_ARG, "%s[%d]: NULL pointer for a non-empty matrix", what, i);
  if (m.ld < m.cols)
    return fail(msg, len, MUON_ERR_SHAPE_MISMATCH, "%s[%d]: ld %lld < cols %lld", what, i, (long long)m.ld,
                (long long)m.cols);
  if (m.ld > kMaxLd)
    return fail(msg, len, MUON_ERR_SHAPE_MISMATCH, "%s[%d]: ld %lld exceeds 2^40", what, i, (long long)m.ld);
  if (m.rows > kMaxDim || m.cols > kMaxDim)
    return fail(msg, len, MUON_ERR_SHAPE_MISMATCH, "%s[%d]: %lld x %lld exceeds the %d per-dimension limit", what, i,
                (long long)m.rows, (long long)m.cols, kMaxDim);
  const int64_t s = m.rows < m.cols ? m.rows : m.cols;
  if (s > kMaxShort)
    return fail(msg, len, MUON_ERR_SHAPE_MISMATCH, "%s[%d]: short side %lld exceeds %d", what, i, (long long)s,
                kMaxShort);
  if (m.rows * m.cols >= kMaxElems)
    return fail(msg, len, MUON_ERR_SHAPE_MISMATCH, "%s[%d]: %lld elements exceed the 2^31 limit", what, i,
                (long long)(m.rows * m.cols));
  if (((uintptr_t)m.ptr) % (uintptr_t)elem_size(m.dtype) != 0)
    return fail(msg, len, MUON_ERR_INVALID_ARG, "%s[%d]: pointer not aligned to its element size", what, i);
  return MUON_OK;
}

// Buffers of one call that share memory. A matrix occupies the byte
// intervals [ptr + r ld e, ptr + r ld e + cols e) for r < rows (e = element
// size): disjoint and in address order, since ld >= cols. Two matrices
// overlap when one of these intervals meets one of the other's, so column
// slices of one parent buffer (same ld, disjoint columns) do not overlap.
// Offsets are 128-bit: rows x ld x e reaches 2^58 and the pointer adds to it.
typedef unsigned __int128 u128;
struct Span {
  u128 lo, hi;     // first byte; one past the last row's last byte
  u128 ldb, rowb;  // row stride and row length, in bytes
  int64_t rows;
  const char* what;
  int idx;
  bool writes;     // the call writes this buffer
};

Span make_span(const muon_matrix& m, const char* what, int idx, bool writes) {
  const u128 e = (u128)elem_size(m.dtype);
  Span s;
  s.lo = (u128)(uintptr_t)m.ptr;
  s.ldb = (u128)m.ld * e;
  s.rowb = (u128)m.cols * e;
  s.rows = m.rows;
  s.hi = s.lo + (u128)(m.rows - 1) * s.ldb + s.rowb;
  s.what = what;
  s.idx = idx;
  s.writes = writes;
  return s;
}

bool spans_meet(const Span& a, const Span& b) {
  if (a.hi <= b.lo || b.hi <= a.lo) return false;
  const Span& p = a.lo <= b.lo ? a : b;   // starts first
  const Span& q = a.lo <= b.lo ? b : a;
  if (p.ldb == q.ldb) {
    // q's row s starts at byte `rem` of p's row k + s and, when it runs past
    // that row's stride, ends in row k + s + 1 (never further: rowb <= ldb)
    const u128 d = q.lo - p.lo, k = d / p.ldb, rem = d % p.ldb, prow = (u128)p.rows;
    if (k < prow && rem < p.rowb) return true;
    return rem + q.rowb > p.ldb && k + 1 < prow;
  }
  // different strides: for each row of the matrix with fewer rows, the other
  // matrix's last row starting before that row's end is the only one that
  // can reach into it
  const Span& x = a.rows <= b.rows ? a : b;
  const Span& y = a.rows <= b.rows ? b : a;
  for (int64_t r = 0; r < x.rows; ++r) {
    const u128 x0 = x.lo + (u128)r * x.ldb, x1 = x0 + x.rowb;
    if (x1 <= y.lo) continue;
    if (x0 >= y.hi) break;
    u128 t = (x1 - 1 - y.lo) / y.ldb;
    if (t >= (u128)y.rows) t = (u128)y.rows - 1;
    if (y.lo + t * y.ldb + y.rowb > x0) return true;
  }
  return false;
}

// Sweep in address order; `outputs_may_overlap_inputs`: a pair of one
// written and one read-only buffer is allowed (the polar entry points read
// every input before they write the first output).
int check_overlaps(std::vector<Span>& v, bool outputs_may_overlap_inputs, char* msg, int len) {
  std::stable_sort(v.begin(), v.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  std::vector<int> live;   // earlier spans that may still reach the current one
  for (int i = 0; i < (int)v.size(); ++i) {
    size_t k = 0;
    for (int j : live)
      if (v[j].hi > v[i].lo) live[k++] = j;
    live.resize(k);
    for (int j : live) {
      const Span& a = v[j];
      const Span& b = v[i];
      if (!a.writes && !b.writes) continue;
      if (outputs_may_overlap_inputs && a.writes != b.writes) continue;
      if (spans_meet(a, b))
        return fail(msg, len, MUON_ERR_INVALID_ARG, "%s[%d] and %s[%d] share memory", a.what, a.idx, b.what,
                    b.idx);
    }
    live.push_back(i);
  }
  return MUON_OK;
}

bool nonempty(const muon_matrix& m) { return m.rows > 0 && m.cols > 0; }

int same_shape(const muon_matrix& a, const muon_matrix& b, const char* wa, const char* wb, int i, char* msg,
               int len) {
  if (a.rows != b.rows || a.cols != b.cols)
    return fail(msg, len, MUON_ERR_SHAPE_MISMATCH, "%s[%d] is %lld x %lld but %s[%d] is %lld x %lld", wb, i,
                (long long)b.rows, (long long)b.cols, wa, i, (long long)a.rows, (long long)a.cols);
  return MUON_OK;
}

}  // namespace

int check_config(const muon_config* c, char* msg, int len) {
  if (!c) return MUON_OK;
  if (c->ns_steps < 1 || c->ns_steps > 64)
    return fail(msg, len, MUON_ERR_INVALID_ARG, "ns_steps %d outside [1, 64]", (int)c->ns_steps);
  if (!finitef(c->ns_a) || !finitef(c->ns_b) || !finitef(c->ns_c))
    return fail(msg, len, MUON_ERR_INVALID_ARG, "ns coefficients must be finite");
  if (!finitef(c->ns_eps) || c->ns_eps < 0.f) return fail(msg, len, MUON_ERR_INVALID_ARG, "ns_eps must be >= 0");
  if (c->pp_iterations < 0 || c->pp_iterations > 8)
    return fail(msg, len, MUON_ERR_INVALID_ARG, "pp_iterations %d outside [0, 8]", (int)c->pp_iterations);
  if (!finitef(c->pp_beta)) return fail(msg, len, MUON_ERR_INVALID_ARG, "pp_beta must be finite");
  if (!finitef(c->pp_eps) || !(c->pp_eps > 0.f)) return fail(msg, len, MUON_ERR_INVALID_ARG, "pp_eps must be > 0");
  if (!finitef(c->mu) || c->mu < 0.f || c->mu > 1.f)
    return fail(msg, len, MUON_ERR_INVALID_ARG, "mu must lie in [0, 1]");
  if (c->nesterov != 0 && c->nesterov != 1) return fail(msg, len, MUON_ERR_INVALID_ARG, "nesterov must be 0 or 1");
  if (c->power_steps < 1 || c->power_steps > 64)
    return fail(msg, len, MUON_ERR_INVALID_ARG, "power_steps %d outside [1, 64]", (int)c->power_steps);
  if (!finitef(c->contra)) return fail(msg, len, MUON_ERR_INVALID_ARG, "contra must be finite");
  if (!finitef(c->target_uw) || c->target_uw < 0.f)
    return fail(msg, len, MUON_ERR_INVALID_ARG, "target_uw must be >= 0");
  if (!finitef(c->lr)) return fail(msg, len, MUON_ERR_INVALID_ARG, "lr must be finite");
  if (c->flags & ~MUON_FLAG_ALL)
    return fail(msg, len, MUON_ERR_INVALID_ARG, "flags 0x%x has unknown bits", (unsigned)c->flags);
  return MUON_OK;
}

int check_polar(int n, const muon_matrix* in, const muon_matrix* out, const muon_config* cfg, char* msg, int len) {
  if (msg && len > 0) msg[0] = 0;
  if (n < 0 || n > kMaxBatch) return fail(msg, len, MUON_ERR_INVALID_ARG, "batch size %d outside [0, %d]", n, kMaxBatch);
  if (n > 0 && (!in || !out)) return fail(msg, len, MUON_ERR_INVALID_ARG, "NULL descriptor array");
  int rc = check_config(cfg, msg, len);
  if (rc) return rc;
  for (int i = 0; i < n; ++i) {
    if ((rc = check_matrix(in[i], "in", i, msg, len))) return rc;
    if ((rc = check_matrix(out[i], "out", i, msg, len))) return rc;
    if ((rc = same_shape(in[i], out[i], "in", "out", i, msg, len))) return rc;
  }
  std::vector<Span> v;
  for (int i = 0; i < n; ++i) {
    if (nonempty(in[i])) v.push_back(make_span(in[i], "in", i, false));
    if (nonempty(out[i])) v.push_back(make_span(out[i], "out", i, true));
  }
  return check_overlaps(v, true, msg, len);
}

int check_update(int n, const muon_matrix* g, const muon_matrix* m, const muon_matrix* w, const muon_matrix* uo,
                 const muon_config* cfg, char* msg, int len) {
  if (msg && len > 0) msg[0] = 0;
  if (n < 0 || n > kMaxBatch) return fail(msg, len, MUON_ERR_INVALID_ARG, "batch size %d outside [0, %d]", n, kMaxBatch);
  if (n > 0 && (!g || !m)) return fail(msg, len, MUON_ERR_INVALID_ARG, "NULL grad or momentum array");
  int rc = check_config(cfg, msg, len);
  if (rc) return rc;
  for (int i = 0; i < n; ++i) {
    if ((rc = check_matrix(g[i], "grad", i, msg, len))) return rc;
    if ((rc = check_matrix(m[i], "momentum", i, msg, len))) return rc;
    if (m[i].dtype != MUON_F32)
      return fail(msg, len, MUON_ERR_UNSUPPORTED_DTYPE, "momentum[%d] must be MUON_F32", i);
    if ((rc = same_shape(g[i], m[i], "grad", "momentum", i, msg, len))) return rc;
    if (w && w[i].ptr) {
      if ((rc = check_matrix(w[i], "weight", i, msg, len))) return rc;
      if ((rc = same_shape(g[i], w[i], "grad", "weight", i, msg, len))) return rc;
    }
    if (uo && uo[i].ptr) {
      if ((rc = check_matrix(uo[i], "update_out", i, msg, len))) return rc;
      if ((rc = same_shape(g[i], uo[i], "grad", "update_out", i, msg, len))) return rc;
    }
  }
  std::vector<Span> v;
  for (int i = 0; i < n; ++i) {
    if (nonempty(g[i])) v.push_back(make_span(g[i], "grad", i, false));
    if (nonempty(m[i])) v.push_back(make_span(m[i], "momentum", i, true));
    if (w && w[i].ptr && nonempty(w[i])) v.push_back(make_span(w[i], "weight", i, true));
    if (uo && uo[i].ptr && nonempty(uo[i])) v.push_back(make_span(uo[i], "update_out", i, true));
  }
  return check_overlaps(v, false, msg, len);
}

}  // namespace muon

extern "C" muon_status muon_check_update_args(int n, const muon_matrix* grad, const muon_matrix* momentum,
                                              const muon_matrix* weight, const muon_matrix* update_out,
                                              const muon_config* cfg, char* msg, int msg_len) {
  return muon::check_update(n, grad, momentum, weight, update_out, cfg, msg, msg_len);
}

extern "C" muon_status muon_check_polar_args(int n, const muon_matrix* in, const muon_matrix* out,
                                             const muon_config* cfg, char* msg, int msg_len) {
  return muon::check_polar(n, in, out, cfg, msg, msg_len);
}

extern "C" void muon_config_default(muon_config* c) {
  if (!c) return;
  c->ns_steps = 12;
  c->ns_a = 2.0f;
  c->ns_b = -1.5f;
  c->ns_c = 0.5f;
  c->ns_eps = 1e-7f;
  c->pp_iterations = 2;
  c->pp_beta = 0.5f;
  c->pp_eps = 1e-7f;
  c->mu = 0.95f;
  c->nesterov = 1;
  c->power_steps = 5;
  c->contra = 0.4f;
  c->target_uw = 0.35f;
  c->lr = 0.0375f;
  c->flags = 0;
}

// Classic recipe of the Track-1 record page, §"训练管线与系统实现".
extern "C" void muon_config_classic(muon_config* c) {
  if (!c) return;
  muon_config_default(c);
  c->ns_steps = 5;
  c->ns_a = 3.4445f;
  c->ns_b = -4.7750f;
  c->ns_c = 2.0315f;
  c->pp_iterations = 0;
  c->contra = 0.0f;
  c->target_uw = 0.0f;
  c->mu = 0.95f;
  c->nesterov = 1;
  c->lr = 0.04f;
  c->flags = MUON_FLAG_SGD_MOMENTUM;
}

// Linear momentum warm-up of the same page: frac = min(step / n, 1).
extern "C" float muon_momentum_warmup(int64_t step, float mu_start, float mu_end, int64_t warmup_steps) {
  if (warmup_steps <= 0) return mu_end;
  const double s = step < 0 ? 0.0 : (double)step;
  const double frac = s >= (double)warmup_steps ? 1.0 : s / (double)warmup_steps;
  return (float)((1.0 - frac) * (double)mu_start + frac * (double)mu_end);
}

extern "C" const char* muon_status_string(muon_status s) {
  switch (s) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG";
    case MUON_ERR_UNSUPPORTED_DTYPE: return "MUON_ERR_UNSUPPORTED_DTYPE";
    case MUON_ERR_SHAPE_MISMATCH: return "MUON_ERR_SHAPE_MISMATCH";
    case MUON_ERR_ALLOC: return "MUON_ERR_ALLOC";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
    case MUON_ERR_NO_DEVICE: return "MUON_ERR_NO_DEVICE";
    case MUON_ERR_TOO_LARGE: return "MUON_ERR_TOO_LARGE";
    case MUON_ERR_NONFINITE: return "MUON_ERR_NONFINITE";
    default: return "MUON_ERR_UNKNOWN";
  }
}

extern "C" const char* muon_version(void) { return "0.1.0"; }
