// Host fuzz driver for the argument validation of libmuon, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitized_validation.py (CPU only: validation touches no device
// memory). Every call must return one of the declared status codes, write a
// NUL-terminated message within the buffer it is given, and accept or
// reject exactly as a plain re-statement of the rules below predicts.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <limits>
#include <random>
#include <vector>

#include "libmuon.h"

namespace {

std::mt19937_64 rng(20261203);

int64_t pick_dim() {
  static const int64_t edge[] = {0, 1, 2, 7, 8, 255, 256, 4096, 16383, 16384, 16385, 32768,
                                 65535, 65536, 65537, -1, -65536, std::numeric_limits<int64_t>::max(),
                                 std::numeric_limits<int64_t>::min()};
  if (rng() % 3 == 0) return edge[rng() % (sizeof(edge) / sizeof(edge[0]))];
  return (int64_t)(rng() % 70000);
}

// a + b without signed overflow (the driver's own arithmetic must be defined)
int64_t sat_add(int64_t a, int64_t b) {
  if (b > 0 && a > std::numeric_limits<int64_t>::max() - b) return std::numeric_limits<int64_t>::max();
  if (b < 0 && a < std::numeric_limits<int64_t>::min() - b) return std::numeric_limits<int64_t>::min();
  return a + b;
}

muon_matrix pick_matrix() {
  muon_matrix m;
  m.rows = pick_dim();
  m.cols = pick_dim();
  const int k = (int)(rng() % 6);
  m.ld = k == 0 ? m.cols : k == 1 ? sat_add(m.cols, (int64_t)(rng() % 64)) : k == 2 ? sat_add(m.cols, -1)
         : k == 3 ? ((int64_t)1 << 40) + (int64_t)(rng() % 3) - 1 : k == 4 ? std::numeric_limits<int64_t>::max()
         : pick_dim();
  const int p = (int)(rng() % 4);
  m.ptr = p == 0 ? nullptr : p == 1 ? (void*)(uintptr_t)0x1001 : (void*)(uintptr_t)(0x10000 + 16 * (rng() % 1000));
  const int d = (int)(rng() % 5);
  m.dtype = d < 2 ? MUON_F32 : d < 4 ? MUON_BF16 : (muon_dtype)(int)(rng() % 7 - 3);
  return m;
}

// The rules, restated from include/libmuon.h.
int expect_matrix(const muon_matrix& m) {
  if (m.dtype != MUON_F32 && m.dtype != MUON_BF16) return MUON_ERR_UNSUPPORTED_DTYPE;
  if (m.rows < 0 || m.cols < 0) return MUON_ERR_SHAPE_MISMATCH;
  if (m.rows == 0 || m.cols == 0) return MUON_OK;
  if (!m.ptr) return MUON_ERR_INVALID_ARG;
  if (m.ld < m.cols) return MUON_ERR_SHAPE_MISMATCH;
  if (m.ld > ((int64_t)1 << 40)) return MUON_ERR_SHAPE_MISMATCH;
  if (m.rows > 65536 || m.cols > 65536) return MUON_ERR_SHAPE_MISMATCH;
  if ((m.rows < m.cols ? m.rows : m.cols) > 16384) return MUON_ERR_SHAPE_MISMATCH;
  if (m.rows * m.cols >= ((int64_t)1 << 31)) return MUON_ERR_SHAPE_MISMATCH;
  if (((uintptr_t)m.ptr) % (m.dtype == MUON_BF16 ? 2 : 4) != 0) return MUON_ERR_INVALID_ARG;
  return MUON_OK;
}

bool known(int rc) {
  return rc == MUON_OK || rc == MUON_ERR_INVALID_ARG || rc == MUON_ERR_UNSUPPORTED_DTYPE ||
         rc == MUON_ERR_SHAPE_MISMATCH;
}

void pick_config(muon_config* c) {
  muon_config_default(c);
  const float odd[] = {NAN, INFINITY, -INFINITY, -1.f, 0.f, 1e30f, -0.f, 2.f};
  switch (rng() % 12) {
    case 0: c->ns_steps = (int)(rng() % 200) - 50; break;
    case 1: c->pp_iterations = (int)(rng() % 20) - 5; break;
    case 2: c->power_steps = (int)(rng() % 200) - 50; break;
    case 3: c->mu = odd[rng() % 8]; break;
    case 4: c->pp_eps = odd[rng() % 8]; break;
    case 5: c->lr = odd[rng() % 8]; break;
    case 6: c->target_uw = odd[rng() % 8]; break;
    case 7: c->flags = (uint32_t)rng(); break;
    case 8: c->nesterov = (int)(rng() % 5) - 2; break;
    default: break;
  }
}

// The overlap rule restated by brute force: two buffers share memory when a
// row of one meets a row of the other, as byte intervals.
struct Buf {
  uintptr_t p;
  int64_t rows, cols, ld;
  int esz;
  bool writes;
};
bool meet(const Buf& a, const Buf& b) {
  for (int64_t r = 0; r < a.rows; ++r)
    for (int64_t s = 0; s < b.rows; ++s) {
      const uintptr_t a0 = a.p + (uintptr_t)(r * a.ld * a.esz), a1 = a0 + (uintptr_t)(a.cols * a.esz);
      const uintptr_t b0 = b.p + (uintptr_t)(s * b.ld * b.esz), b1 = b0 + (uintptr_t)(b.cols * b.esz);
      if (a0 < b1 && b0 < a1) return true;
    }
  return false;
}

// Small matrices packed into a few hundred bytes, so that buffers often share
// memory; every other rule holds, so the status is OK or INVALID_ARG exactly
// as the restated overlap rule says.
int overlap_fuzz() {
  const uintptr_t arena = 0x100000;
  auto place = [&](int64_t rows, int64_t cols, muon_dtype dt) {
    muon_matrix x;
    x.rows = rows;
    x.cols = cols;
    x.ld = cols + (int64_t)(rng() % 6);
    x.dtype = dt;
    x.ptr = (void*)(arena + 4 * (uintptr_t)(rng() % 200));
    return x;
  };
  auto pick_dt = [&]() { return rng() % 2 ? MUON_F32 : MUON_BF16; };
  auto buf = [](const muon_matrix& x, bool writes) {
    return Buf{(uintptr_t)x.ptr, x.rows, x.cols, x.ld, x.dtype == MUON_BF16 ? 2 : 4, writes};
  };
  char msg[300];
  int rejected = 0, total = 0;
  for (int it = 0; it < 20000; ++it) {
    const int n = 1 + (int)(rng() % 4);
    std::vector<muon_matrix> g(n), m(n), w(n), o(n);
    std::vector<Buf> bufs;
    const bool update = it % 2 == 1;
    for (int i = 0; i < n; ++i) {
      const int64_t rows = 1 + (int64_t)(rng() % 12), cols = 1 + (int64_t)(rng() % 12);
      g[i] = place(rows, cols, pick_dt());
      o[i] = place(rows, cols, pick_dt());
      if (update) {
        m[i] = place(rows, cols, MUON_F32);
        w[i] = place(rows, cols, pick_dt());
        if (rng() % 3 == 0) w[i].ptr = nullptr;
        if (rng() % 3 == 0) o[i].ptr = nullptr;
      }
      bufs.push_back(buf(g[i], false));
      if (update) {
        bufs.push_back(buf(m[i], true));
        if (w[i].ptr) bufs.push_back(buf(w[i], true));
      }
      if (o[i].ptr) bufs.push_back(buf(o[i], true));
    }
    bool clash = false;
    for (size_t a = 0; a < bufs.size() && !clash; ++a)
      for (size_t b = a + 1; b < bufs.size() && !clash; ++b) {
        if (!bufs[a].writes && !bufs[b].writes) continue;
        if (!update && bufs[a].writes != bufs[b].writes) continue;   // an output over an input is allowed
        clash = meet(bufs[a], bufs[b]);
      }
    const int rc = update ? muon_check_update_args(n, g.data(), m.data(), w.data(), o.data(), nullptr, msg, sizeof(msg))
                          : muon_check_polar_args(n, g.data(), o.data(), nullptr, msg, sizeof(msg));
    const int want = clash ? MUON_ERR_INVALID_ARG : MUON_OK;
    if (rc != want) {
      printf("overlap rule: call %d (%s, n=%d) returned %d, expected %d: %s\n", it, update ? "update" : "polar", n,
             rc, want, msg);
      return 1;
    }
    rejected += clash;
    ++total;
  }
  printf("overlap %d calls, %d rejected\n", total, rejected);
  return 0;
}

}  // namespace

int main() {
  int calls = 0, accepted = 0;
  char msg[300];
  for (int it = 0; it < 20000; ++it) {
    const int n = it % 97 == 0 ? (int)(rng() % 3) * 65535 + (int)(rng() % 3) - 1 : (int)(rng() % 5);
    const int cap = n > 0 && n <= 65536 ? n : 1;
    std::vector<muon_matrix> g(cap), m(cap), w(cap), o(cap);
    for (int i = 0; i < cap; ++i) {
      g[i] = pick_matrix();
      m[i] = g[i];
      m[i].dtype = rng() % 8 ? MUON_F32 : MUON_BF16;
      w[i] = rng() % 2 ? g[i] : pick_matrix();
      o[i] = rng() % 3 ? g[i] : pick_matrix();
      if (rng() % 4 == 0) w[i].ptr = nullptr;
    }
    muon_config cfg;
    pick_config(&cfg);
    const int len = (int)(rng() % 4 == 0 ? rng() % 8 : sizeof(msg));
    memset(msg, 'x', sizeof(msg));
    const muon_config* pc = rng() % 5 ? &cfg : nullptr;
    const bool null_arr = rng() % 50 == 0;
    int rc;
    if (it % 2)
      rc = muon_check_update_args(n, null_arr ? nullptr : g.data(), m.data(), w.data(), o.data(), pc, len ? msg : nullptr, len);
    else
      rc = muon_check_polar_args(n, null_arr ? nullptr : g.data(), o.data(), pc, len ? msg : nullptr, len);
    ++calls;
    if (!known(rc)) { printf("unknown status %d\n", rc); return 1; }
    if (len > 0 && memchr(msg, 0, (size_t)len) == nullptr) { printf("message not terminated\n"); return 1; }
    if (len > 0 && len < (int)sizeof(msg) && msg[len] != 'x') { printf("message overran its buffer\n"); return 1; }
    // single-matrix calls with a valid config: the result must follow the rules
    if (n == 1 && !null_arr && (pc == nullptr || pc == &cfg) && rc != MUON_ERR_INVALID_ARG) {
      int e = expect_matrix(g[0]);
      if (it % 2 == 0 && e == MUON_OK) e = expect_matrix(o[0]);
      if (e != MUON_OK && rc == MUON_OK) { printf("accepted an invalid matrix (expected %d)\n", e); return 1; }
    }
    if (rc == MUON_OK) ++accepted;
  }
  if (overlap_fuzz()) return 1;
  printf("ok %d calls, %d accepted\n", calls, accepted);
  return 0;
}
