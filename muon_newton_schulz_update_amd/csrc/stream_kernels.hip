// Bandwidth-bound kernels of the Muon step (everything but the Newton-Schulz
// products). Step names and formulas follow the Aurora record page
// (www.xxmr.cn/news/295280): section 组合优化栈 (muon_update: momentum lerp,
// Nesterov blend, unit-operator-norm direction, Contra-Muon, Frobenius
// restore, aspect scale; u/w-floor and the parameter add) and sections
// Aurora 的迭代伪代码 / 源码实现 (the diagonal preconditioner D).
//
// Every launch covers a whole batch: a LaunchList maps block b to a matrix
// and a local block index. Streaming tiles are kStreamRows x kSegCols; each
// of a block's four waves owns kWaveRows rows of one, a lane 8 consecutive
// columns. All reductions are two-stage (per-block partials, then a
// fixed-order sum): no atomics, bitwise reproducible.
//
// Memory-level parallelism: every HBM access goes through a global
// address-space pointer (global_load/store: they count on vmcnt only, while
// generic-pointer loads would also hold up every scalar-load wait), element
// types are resolved once per block (a uniform branch at kernel entry into a
// body templated on them), and a lane issues the loads of all its rows before
// it converts or uses any of them (one batch per wave: short-lived waves keep
// more requests in flight than looping ones). Lanes whose 8 columns are
// ragged (the last chunk of a row) or whose buffers are not 16-byte aligned
// take an element-wise path.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "muon_device.hpp"

namespace muon {

namespace {

__device__ __forceinline__ unsigned short f2bf(float f) {
  unsigned int u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (unsigned short)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}
__device__ __forceinline__ float bf2f(unsigned short h) { return __uint_as_float(((unsigned int)h) << 16); }

typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

#define GLOBAL_AS __attribute__((address_space(1)))
// Loads and stores through global address-space pointers (all buffers here
// are device memory).
template <typename V>
__device__ __forceinline__ V gld(const void* p) {
  return *(const GLOBAL_AS V*)p;
}
template <typename V>
__device__ __forceinline__ void gst(void* p, V v) {
  *(GLOBAL_AS V*)p = v;
}

__device__ __forceinline__ int find_job(const LaunchList& L, int b, int* local) {
  int lo = 0, hi = L.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (L.off[mid] <= b) lo = mid; else hi = mid - 1;
  }
  *local = b - L.off[lo];
  return L.mat[lo];
}

// Element types: 8 consecutive elements of a row as one raw vector (16 bytes
// of bf16, 32 of fp32), converted to float after the loads of a batch.
template <typename T> struct Ty;
template <> struct Ty<__bf16> {
  typedef u16x8_t Raw;
  __device__ static Raw ld(const void* b, size_t i) { return gld<u16x8_t>((const unsigned short*)b + i); }
  __device__ static void cvt(const Raw& q, float v[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf2f(q[e]);
  }
  __device__ static float ld1(const void* b, size_t i) { return bf2f(gld<unsigned short>((const unsigned short*)b + i)); }
  __device__ static void st(void* b, size_t i, const float v[8]) {
    u16x8_t q;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = f2bf(v[e]);
    gst<u16x8_t>((unsigned short*)b + i, q);
  }
  __device__ static void st1(void* b, size_t i, float x) { gst<unsigned short>((unsigned short*)b + i, f2bf(x)); }
  __device__ static float round(float x) { return bf2f(f2bf(x)); }   // what a later read of a stored value sees
};
template <> struct Ty<float> {
  struct Raw {
    f32x4_t a, b;
  };
  __device__ static Raw ld(const void* b, size_t i) {
    const float* p = (const float*)b + i;
    Raw q;
    q.a = gld<f32x4_t>(p);
    q.b = gld<f32x4_t>(p + 4);
    return q;
  }
  __device__ static void cvt(const Raw& q, float v[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = q.a[e]; v[e + 4] = q.b[e]; }
  }
  __device__ static float ld1(const void* b, size_t i) { return gld<float>((const float*)b + i); }
  __device__ static void st(void* b, size_t i, const float v[8]) {
    float* p = (float*)b + i;
    gst<f32x4_t>(p, (f32x4_t){v[0], v[1], v[2], v[3]});
    gst<f32x4_t>(p + 4, (f32x4_t){v[4], v[5], v[6], v[7]});
  }
  __device__ static void st1(void* b, size_t i, float x) { gst<float>((float*)b + i, x); }
  __device__ static float round(float x) { return x; }
};

// Element-wise forms: the first n (0..8) elements at index i, zero past them.
template <typename T>
__device__ __forceinline__ void ld_part(const void* b, size_t i, int n, float v[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = e < n ? Ty<T>::ld1(b, i + e) : 0.f;
}
template <typename T>
__device__ __forceinline__ void st_part(void* b, size_t i, int n, const float v[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e < n) Ty<T>::st1(b, i + e, v[e]);
}
// Stores whose element type is only known at run time (caller outputs).
__device__ __forceinline__ void st_vec_rt(void* b, int dt, size_t i, const float v[8]) {
  if (dt == DT_BF16) Ty<__bf16>::st(b, i, v); else Ty<float>::st(b, i, v);
}
__device__ __forceinline__ void st_part_rt(void* b, int dt, size_t i, int n, const float v[8]) {
  if (dt == DT_BF16) st_part<__bf16>(b, i, n, v); else st_part<float>(b, i, n, v);
}
__device__ __forceinline__ float ld1_rt(const void* b, int dt, size_t i) {
  return dt == DT_BF16 ? Ty<__bf16>::ld1(b, i) : Ty<float>::ld1(b, i);
}

__device__ __forceinline__ bool aligned16(const void* p, int64_t ld, int dt) {
  const int esz = dt == DT_BF16 ? 2 : 4;
  return (((uintptr_t)p) & 15) == 0 && ((ld * esz) & 15) == 0;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Fixed-order block sum (256 threads); result valid in every thread.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return t;
}

// Block maximum (256 threads); result valid in every thread.
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t = fmaxf(t, red[i]);
  return t;
}

// float -> OCP e4m3 (bias 7, no infinities, largest finite 448), round to
// nearest even, magnitudes clamped to 448. Subnormals are m 2^-9 (m < 8);
// m reaching 8 carries into the smallest normal, whose code is also 8.
__device__ __forceinline__ unsigned int f2e4m3(float x) {
  const unsigned int sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  unsigned int code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal range
    code = (unsigned int)rintf(a * 512.f);   // 0 .. 8
  } else {
    unsigned int u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);        // round the mantissa to 3 bits, ties to even
    code = ((((u >> 23) & 0xFFu) - 120u) << 3) | ((u >> 20) & 7u);   // exponent - 127 + 7
  }
  return sign | code;
}

// Power-of-two scale for the fp8 copy of X0, from an upper bound on |X0|:
// the largest q = 2^e with q * bound <= 448 (1 when the bound is 0).
__device__ __forceinline__ float f8_scale(float bound) {
  if (!(bound > 0.f)) return 1.f;
  const float e = fminf(fmaxf(floorf(log2f(448.f / bound)), -100.f), 100.f);
  return exp2f(e);
}

// Sum of n floats p[0], p[stride], ..., in index order, eight loads at a time.
__device__ __forceinline__ float strided_sum(const float* p, size_t stride, int n) {
  float s = 0.f;
  int k = 0;
  for (; k + 8 <= n; k += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = gld<float>(p + (size_t)(k + j) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  for (; k < n; ++k) s += gld<float>(p + (size_t)k * stride);
  return s;
}

}  // namespace

// ---------------------------------------------------------------------------
// K1: momentum + Nesterov blend, and the sums of squares of the result.
//   moving average:  M <- M + (1 - mu)(G - M);  X = G + mu (M - G)
//   SGD (sgd != 0):  M <- mu M + G;             X = G + mu M
//   (X = M without Nesterov)
// X is stored in the NS type (rounded), and the norms are taken of the stored
// values. With `nesterov_pass` false this only gathers the norms of the
// matrix given in `g` (the polar entry points).
// A block is a kStreamRows x kSegCols tile, a wave kWaveRows rows of it,
// loaded in one batch. Outputs per tile: rowpart[r][seg] (row sums over the
// tile's columns) and, for wide matrices, colpart[tile_row][c] (column sums
// over the tile's rows, the four waves combined in LDS).
// ---------------------------------------------------------------------------
template <typename TG, typename TX, bool NP>
__device__ __forceinline__ void momentum_body(const DevMat& M, int local, float mu, int nesterov, int sgd,
                                              float* cp) {
  typedef Ty<TG> G;
  typedef Ty<float> F;
  constexpr int R = kWaveRows;
  const int tr = local / M.n_seg, sg = local % M.n_seg;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = sg * kSegCols + lane * 8;
  const int r = tr * kStreamRows + w * R;            // this wave's first row
  const int nr = max(0, min(R, M.rows - r));          // uniform per wave
  const int dg = sizeof(TG) == 2 ? DT_BF16 : DT_F32, dx = sizeof(TX) == 2 ? DT_BF16 : DT_F32;
  const int nv = max(0, min(8, M.cols - c));
  const bool fast = nr == R && nv == 8 && aligned16(M.g, M.ld_g, dg) &&
                    (!NP || (aligned16(M.m, M.ld_m, DT_F32) && aligned16(M.xn, M.cols, dx)));
  float col[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float rsl[R];   // this lane's part of each row's sum of squares
  // one row: the update (stored through vector or element-wise stores), then
  // this lane's sums of squares; a row's floats die before the next row is
  // converted. Lanes of one wave may take different paths, so the cross-lane
  // row sums wait until the paths have rejoined.
  auto row = [&](int k, float* x, float* m, bool vec) {
    if (NP) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = x[e];
        const float mn = sgd ? mu * m[e] + g : m[e] + (1.f - mu) * (g - m[e]);
        m[e] = mn;
        x[e] = Ty<TX>::round(nesterov ? (sgd ? g + mu * mn : g + mu * (mn - g)) : mn);
      }
      if (vec) {
        F::st(M.m, (size_t)(r + k) * M.ld_m + c, m);
        Ty<TX>::st(M.xn, (size_t)(r + k) * M.cols + c, x);
      } else {
        const int n = k < nr ? nv : 0;
        st_part<float>(M.m, (size_t)(r + k) * M.ld_m + c, n, m);
        st_part<TX>(M.xn, (size_t)(r + k) * M.cols + c, n, x);
      }
    }
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { rs += x[e] * x[e]; col[e] += x[e] * x[e]; }
    rsl[k] = rs;
  };
  if (fast) {
    // fp32 grads load in two batches of R/2 rows: the kernel's register
    // budget is set by its largest body
    constexpr int RB = sizeof(TG) == 2 ? R : R / 2;
#pragma unroll
    for (int k0 = 0; k0 < R; k0 += RB) {
      typename G::Raw qg[RB];
      typename F::Raw qm[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) qg[k] = G::ld(M.g, (size_t)(r + k0 + k) * M.ld_g + c);
      if (NP) {
#pragma unroll
        for (int k = 0; k < RB; ++k) qm[k] = F::ld(M.m, (size_t)(r + k0 + k) * M.ld_m + c);
      }
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        float x[8], m[8];
        G::cvt(qg[k], x);
        if (NP) F::cvt(qm[k], m);
        row(k0 + k, x, m, true);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float x[8], m[8];
      const int n = k < nr ? nv : 0;
      ld_part<TG>(M.g, (size_t)(r + k) * M.ld_g + c, n, x);
      if (NP) ld_part<float>(M.m, (size_t)(r + k) * M.ld_m + c, n, m);
      row(k, x, m, false);
    }
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const float rs = wave_sum(rsl[k]);
    if (lane == 0 && k < nr) gst<float>(M.rowpart + (size_t)(r + k) * M.n_seg + sg, rs);
  }
  if (M.rows < M.cols) {   // uniform per block
#pragma unroll
    for (int e = 0; e < 8; ++e) cp[w * kSegCols + lane * 8 + e] = col[e];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kSegCols / 256; ++h) {
      const int j = h * 256 + threadIdx.x;
      const float s = cp[j] + cp[kSegCols + j] + cp[2 * kSegCols + j] + cp[3 * kSegCols + j];
      if (sg * kSegCols + j < M.cols) gst<float>(M.colpart + (size_t)tr * M.cols + sg * kSegCols + j, s);
    }
  }
}

__global__ __launch_bounds__(256) void k_momentum_stats(const DevMat* __restrict__ mats, LaunchList L,
                                                        int nesterov_pass, float mu, int nesterov, int sgd) {
  static_assert(kStreamRows == 4 * kWaveRows, "four waves per streaming tile");
  __shared__ float cp[4 * kSegCols];
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  // the grad's type is the NS type (plans are keyed by it)
  if (M.dt_g == DT_BF16) {
    if (nesterov_pass) momentum_body<__bf16, __bf16, true>(M, local, mu, nesterov, sgd, cp);
    else momentum_body<__bf16, __bf16, false>(M, local, mu, nesterov, sgd, cp);
  } else {
    if (nesterov_pass) momentum_body<float, float, true>(M, local, mu, nesterov, sgd, cp);
    else momentum_body<float, float, false>(M, local, mu, nesterov, sgd, cp);
  }
}

// Fused tail: ||W||^2 per streaming tile of a matrix with a weight (fwp),
// read once before the tail (its single pass needs the norm first). A
// lane sums its 8 columns of its wave's 8 rows, loaded in one batch; the
// four waves' sums are added in order.
template <typename TW>
__device__ __forceinline__ void wnorm_body(const DevMat& M, int local, float* red) {
  constexpr int R = kWaveRows;
  const int tr = local / M.n_seg, sg = local % M.n_seg;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = sg * kSegCols + lane * 8;
  const int r = tr * kStreamRows + w * R;
  const int nr = max(0, min(R, M.rows - r));
  const int nv = max(0, min(8, M.cols - c));
  float sw = 0.f;
  if (nr == R && nv == 8 && aligned16(M.w, M.ld_w, sizeof(TW) == 2 ? DT_BF16 : DT_F32)) {
    typename Ty<TW>::Raw q[R];
#pragma unroll
    for (int k = 0; k < R; ++k) q[k] = Ty<TW>::ld(M.w, (size_t)(r + k) * M.ld_w + c);
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float v[8];
      Ty<TW>::cvt(q[k], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sw += v[e] * v[e];
    }
  } else {
    for (int k = 0; k < nr; ++k) {
      float v[8];
      ld_part<TW>(M.w, (size_t)(r + k) * M.ld_w + c, nv, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sw += v[e] * v[e];
    }
  }
  sw = wave_sum(sw);
  if (lane == 0) red[w] = sw;
  __syncthreads();
  if (threadIdx.x == 0) gst<float>(M.fwp + local, red[0] + red[1] + red[2] + red[3]);
}

__global__ __launch_bounds__(256) void k_wnorm(const DevMat* __restrict__ mats, LaunchList L) {
  __shared__ float red[4];
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (!M.ftw) return;   // no weight in this call (uniform over the block)
  if (M.dt_w == DT_BF16) wnorm_body<__bf16>(M, local, red);
  else wnorm_body<float>(M, local, red);
}

// ---------------------------------------------------------------------------
// Input check (MUON_FLAG_CHECK_FINITE), over the momentum pass's tiles: the
// grad (the polar input), with upd the momentum, and the weight when there
// is one. Reads only; a NaN or Inf anywhere in a matrix's inputs sets its
// descriptor's flag (one atomic per wave that saw one).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void ld8_rt(const void* b, int dt, int64_t ld, int r, int c, int n, float v[8]) {
  const size_t i = (size_t)r * ld + c;
  if (n == 8 && aligned16(b, ld, dt)) {
    if (dt == DT_BF16) Ty<__bf16>::cvt(Ty<__bf16>::ld(b, i), v);
    else Ty<float>::cvt(Ty<float>::ld(b, i), v);
  } else if (dt == DT_BF16) {
    ld_part<__bf16>(b, i, n, v);
  } else {
    ld_part<float>(b, i, n, v);
  }
}
__global__ __launch_bounds__(256) void k_check_finite(DevMat* __restrict__ mats, LaunchList L, int upd) {
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int tr = local / M.n_seg, sg = local % M.n_seg;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = sg * kSegCols + lane * 8;
  const int r0 = tr * kStreamRows + w * kWaveRows;
  const int nv = max(0, min(8, M.cols - c));
  bool ok = true;
  for (int k = 0; k < kWaveRows; ++k) {
    const int r = r0 + k;
    const int n = r < M.rows ? nv : 0;   // n = 0 loads nothing
    float v[8];
    ld8_rt(M.g, M.dt_g, M.ld_g, r, c, n, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ok = ok && isfinite(v[e]);
    if (upd) {
      ld8_rt(M.m, DT_F32, M.ld_m, r, c, n, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ok = ok && isfinite(v[e]);
    }
    if (M.w) {
      ld8_rt(M.w, M.dt_w, M.ld_w, r, c, n, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ok = ok && isfinite(v[e]);
    }
  }
  if (__any(!ok) && lane == 0) atomicOr(&M.bad, 1);
}

// ---------------------------------------------------------------------------
// Norms from the K1 partials, in two launches.
// Lines: one thread per row (rowsq[r] = sum of the row's segment partials)
// and, for wide matrices, per column (colsq[c] = sum over row tiles). A
// long-side line l also gets rho_l = ||line||, D_l = 1 / max(rho_l, eps)
// (Aurora's initial preconditioner) and (D_l rho_l)^2; the equilibrated
// lines are the long side, or a wide matrix's rows when M.eq_short is set
// (its own rows, the short side). Block b of a matrix
// writes linepart[2b] = its sum of row sums, linepart[2b+1] = its sum of
// (D rho)^2. Row blocks come first, then column blocks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_norms_lines(DevMat* __restrict__ mats, LaunchList L, float pp_eps) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int nrb = (M.rows + 255) / 256;
  const bool wide = M.rows < M.cols;
  const bool rowline = local < nrb;
  const int i = (rowline ? local : local - nrb) * 256 + threadIdx.x;
  float tpart = 0.f, ypart = 0.f;
  float lsq = -1.f;   // >= 0 on a long-side line
  if (rowline) {
    if (i < M.rows) {
      const float s = strided_sum(M.rowpart + (size_t)i * M.n_seg, 1, M.n_seg);
      gst<float>(M.rowsq + i, s);
      tpart = s;
      if (!wide || M.eq_short) lsq = s;
    }
  } else if (i < M.cols) {
    const float s = strided_sum(M.colpart + i, (size_t)M.cols, M.n_rt);
    gst<float>(M.colsq + i, s);
    if (!M.eq_short) lsq = s;
  }
  if (M.aurora && lsq >= 0.f) {
    const float rho = sqrtf(lsq);
    const float d = 1.f / fmaxf(rho, pp_eps);
    gst<float>(M.rho + i, rho);
    gst<float>(M.dvec + i, d);
    ypart = (d * rho) * (d * rho);
  }
  // the largest squared norm among the lines that bound every element of
  // X0 / scale: the equilibrated lines (D_l rho_l)^2, or the storage rows
  float mpart = M.aurora ? ypart : (rowline && i < M.rows ? tpart : 0.f);
  tpart = block_sum(tpart, red);
  ypart = block_sum(ypart, red);
  mpart = block_max(mpart, red);
  if (threadIdx.x == 0) {
    const int nlb = nrb + (wide ? (M.cols + 255) / 256 : 0);
    gst<float>(M.linepart + 2 * local, tpart);
    gst<float>(M.linepart + 2 * local + 1, ypart);
    gst<float>(M.linepart + 2 * nlb + local, mpart);
  }
}

// Per matrix: ||X||_F^2, the prologue scale 1 / (||D * T||_F + ns_eps) (D = 1
// without Aurora), and the power-iteration start v = ones / sqrt(cols).
__global__ __launch_bounds__(256) void k_norms_scalars(DevMat* __restrict__ mats, LaunchList L, float ns_eps,
                                                       int init_power) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int t = threadIdx.x;
  const int nrb = (M.rows + 255) / 256;
  const int nlb = nrb + (M.rows < M.cols ? (M.cols + 255) / 256 : 0);
  float tot = 0.f, ysq = 0.f, mx = 0.f;
  for (int b = t; b < nlb; b += 256) {
    tot += gld<float>(M.linepart + 2 * b);
    ysq += gld<float>(M.linepart + 2 * b + 1);
    mx = fmaxf(mx, gld<float>(M.linepart + 2 * nlb + b));
  }
  tot = block_sum(tot, red);
  ysq = block_sum(ysq, red);
  mx = block_max(mx, red);
  if (!M.aurora) ysq = tot;
  if (init_power) {
    const float v0 = 1.f / sqrtf((float)M.cols);
    for (int c = t; c < M.cols; c += 256) gst<float>(M.pv + c, v0);
  }
  if (t == 0) {
    const float scale = 1.f / (sqrtf(ysq) + ns_eps);
    const float q = f8_scale(scale * sqrtf(mx));   // every element of X0 is at most scale * sqrt(mx)
    M.scal[SC_XNORM2] = tot;
    M.scal[SC_SCALE] = scale;
    M.scal[SC_F8Q] = q;
    M.scal[SC_F8INV2] = 1.f / (q * q);
    M.scal[SC_SIGMA] = 0.f;
    M.scal[SC_KAPPA] = 0.f;
    M.ist[IS_PSTEPS] = 0;
    M.ist[IS_RESTART] = 0;
  }
}

// ---------------------------------------------------------------------------
// NS prologue through an LDS transpose: X0 = scale * D o T in the wide
// orientation, written to x[0] (s_pad x L_pad) and its transpose to xt[0]
// (L_pad x s_pad), zero padded (the first iteration's products read both;
// for a DevMat::x0n matrix xt[0] is not written: its first X' = Q X reads
// xn and applies scale D itself; for an x0g matrix x[0] is not written: its
// first Gram reads xn and applies scale^2).
// T is the source in storage orientation (rows x cols); for a tall source the
// wide iterate is its transpose. 64 x 64 tiles over the padded storage frame;
// a thread loads its two 8-column chunks (and their D entries) before using
// either.
// ---------------------------------------------------------------------------
template <typename T, typename TS>
__device__ __forceinline__ void prologue_body(const DevMat& M, int local, const void* src, int64_t lds,
                                              float (*tile)[65]) {
  const int dts = sizeof(TS) == 2 ? DT_BF16 : DT_F32;
  const int pc = M.tall ? M.s_pad : M.L_pad;   // padded storage frame: columns
  const int ntc = pc / 64;
  const int br = (local / ntc) * 64, bc = (local % ntc) * 64;
  const bool vs = aligned16(src, lds, dts);
  const float scale = M.scal[SC_SCALE];
  // the fp8 copy of x[0] for the first Gram (x8 is null when not wanted), in
  // panels of 64 columns of s_pad x 64 bytes: a 64 x 64 tile is 4 KB of
  // contiguous bytes
  uint8_t* x8 = (uint8_t*)M.x8;
  const float q8 = M.scal[SC_F8Q];
  auto put8 = [&](int r, int c, const float v[8]) {   // x[0](r, c .. c + 7), c % 8 == 0
    u32x2_t w;
    w[0] = f2e4m3(v[0] * q8) | (f2e4m3(v[1] * q8) << 8) | (f2e4m3(v[2] * q8) << 16) | (f2e4m3(v[3] * q8) << 24);
    w[1] = f2e4m3(v[4] * q8) | (f2e4m3(v[5] * q8) << 8) | (f2e4m3(v[6] * q8) << 16) | (f2e4m3(v[7] * q8) << 24);
    gst<u32x2_t>(x8 + ((size_t)(c >> 6) * M.s_pad + r) * 64 + (c & 63), w);
  };
  // direct frame: wide -> x[0] (ld L_pad); tall -> xt[0] (ld s_pad)
  void* dir = M.tall ? M.xt[0] : M.x[0];
  void* tra = M.tall ? M.x[0] : M.xt[0];
  const int ld_dir = M.tall ? M.s_pad : M.L_pad;
  const int ld_tra = M.tall ? M.L_pad : M.s_pad;
  // 64 x 64 tile = 512 chunks of 8 columns; two chunks per thread
  int rr[2], cc[2], nv[2];
  bool fv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = h * 256 + threadIdx.x;
    rr[h] = br + (q >> 3);
    cc[h] = bc + (q & 7) * 8;
    nv[h] = rr[h] < M.rows ? max(0, min(8, M.cols - cc[h])) : 0;
    fv[h] = vs && nv[h] == 8;
  }
  typename Ty<TS>::Raw qs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (fv[h]) qs[h] = Ty<TS>::ld(src, (size_t)rr[h] * lds + cc[h]);
  // D entries: along the columns of a wide source, one per row of a tall one
  // (and of a wide one equilibrated on its rows)
  float dv[2][8];
  if (M.aurora) {
    const bool per_row = M.tall || M.eq_short;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (per_row) {
        const float d = nv[h] > 0 ? gld<float>(M.dvec + rr[h]) : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dv[h][e] = d;
      } else if (nv[h] == 8) {
        Ty<float>::cvt(Ty<float>::ld(M.dvec, (size_t)cc[h]), dv[h]);   // dvec: 256-byte aligned, cc % 8 == 0
      } else {
        ld_part<float>(M.dvec, (size_t)cc[h], nv[h], dv[h]);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) dv[h][e] = 1.f;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float v[8];
    if (fv[h]) Ty<TS>::cvt(qs[h], v);
    else ld_part<TS>(src, (size_t)rr[h] * lds + cc[h], nv[h], v);
    const int i = rr[h] - br, j = cc[h] - bc;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] *= scale * dv[h][e];
      tile[i][j + e] = v[e];
    }
    // x0n, x0g: the pass's first X' = Q X or first Gram reads xn instead
    if (!M.x0n && !M.x0g) Ty<T>::st(dir, (size_t)rr[h] * ld_dir + cc[h], v);
    if (x8 && !M.tall) put8(rr[h], cc[h], v);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = h * 256 + threadIdx.x;
    const int jc = q >> 3, i0 = (q & 7) * 8;   // transposed row = tile column jc
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[i0 + e][jc];
    Ty<T>::st(tra, (size_t)(bc + jc) * ld_tra + br + i0, v);
    if (x8 && M.tall) put8(bc + jc, br + i0, v);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_prologue(const DevMat* __restrict__ mats, LaunchList L, int use_xn) {
  __shared__ float tile[64][65];
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const void* src = use_xn ? (const void*)M.xn : M.g;
  const int64_t lds = use_xn ? (int64_t)M.cols : M.ld_g;
  const int sdt = use_xn ? M.ns_t : M.dt_g;
  if (sdt == DT_BF16) prologue_body<T, __bf16>(M, local, src, lds, tile);
  else prologue_body<T, float>(M, local, src, lds, tile);
}

// ---------------------------------------------------------------------------
// Aurora D update between passes: row_sq_l = max(sum U_l^2, eps^2) over one
// equilibrated line l of the pass's result U, D_l *= (target / row_sq_l)^beta,
// then partial sums of (D_l rho_l)^2 per block. The lines are the long side
// (row l of U^T, s entries, target s / L) or, with M.eq_short, a wide
// matrix's own rows (row l of U, L entries, target 1). One wave per line; 4
// lines per block; a lane loads two chunks per round.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_aurora_dupdate(DevMat* __restrict__ mats, LaunchList L,
                                                        float pp_eps, float pp_beta) {
  __shared__ float red[4];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l = local * 4 + w;
  const int nl = M.eq_short ? M.s : M.L;      // equilibrated lines
  const int len = M.eq_short ? M.L : M.s;     // entries per line
  float contrib = 0.f;   // (D_l rho_l)^2 of this wave's line
  if (l < nl) {
    const void* ut = M.eq_short ? M.x[M.fin] : M.xt[M.fin];
    const size_t row = (size_t)l * (M.eq_short ? M.L_pad : M.s_pad);
    float s = 0.f;
    // entries past len are zero padding (a line holds a multiple of 256)
    int i = lane * 8;
    for (; i + 512 < len; i += 1024) {
      const typename Ty<T>::Raw q0 = Ty<T>::ld(ut, row + i), q1 = Ty<T>::ld(ut, row + i + 512);
      float u0[8], u1[8];
      Ty<T>::cvt(q0, u0);
      Ty<T>::cvt(q1, u1);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += u0[e] * u0[e];
#pragma unroll
      for (int e = 0; e < 8; ++e) s += u1[e] * u1[e];
    }
    if (i < len) {
      float u0[8];
      Ty<T>::cvt(Ty<T>::ld(ut, row + i), u0);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += u0[e] * u0[e];
    }
    s = wave_sum(s);
    if (lane == 0) {
      const float target = M.eq_short ? 1.f : (float)M.s / (float)M.L;
      const float rsq = fmaxf(s, pp_eps * pp_eps);
      const float d = M.dvec[l] * powf(target / rsq, pp_beta);
      M.dvec[l] = d;
      const float y = d * M.rho[l];
      contrib = y * y;
    }
  }
  if (lane == 0) red[w] = contrib;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nb = (nl + 3) / 4;   // blocks of this launch for the matrix
    M.tailpart[local] = red[0] + red[1] + red[2] + red[3];
    M.tailpart[nb + local] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
}

// The D update of a matrix equilibrated on its long side, from the band
// sums of squares the pass's last product wrote (lsq) instead of a read of
// the pass's result: one thread per line, bands summed in index order; the
// same damped update as k_aurora_dupdate and the same per-4-line partials of
// (D_l rho_l)^2 (sums and maxima) for k_aurora_scale.
__global__ __launch_bounds__(256) void k_aurora_dfinish(DevMat* __restrict__ mats, LaunchList L, float pp_eps,
                                                        float pp_beta) {
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int l = local * 256 + threadIdx.x;
  const int nl = M.L, nbands = M.s_pad / 64;
  float contrib = 0.f;
  if (l < nl) {
    float s = 0.f;
    for (int b = 0; b < nbands; ++b) s += gld<float>(M.lsq + (size_t)b * M.L_pad + l);
    const float target = (float)M.s / (float)M.L;
    const float rsq = fmaxf(s, pp_eps * pp_eps);
    const float d = M.dvec[l] * powf(target / rsq, pp_beta);
    M.dvec[l] = d;
    const float y = d * M.rho[l];
    contrib = y * y;
  }
  // lines 4g .. 4g+3 are lanes 4g .. 4g+3 of one wave
  float sum = contrib + __shfl_xor(contrib, 1, 64);
  sum += __shfl_xor(sum, 2, 64);
  float mx = fmaxf(contrib, __shfl_xor(contrib, 1, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  const int nb = (nl + 3) / 4, g = l >> 2;
  if ((threadIdx.x & 3) == 0 && g < nb) {
    M.tailpart[g] = sum;
    M.tailpart[nb + g] = mx;
  }
}

__global__ __launch_bounds__(256) void k_aurora_scale(DevMat* __restrict__ mats, LaunchList L, float ns_eps) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int nb = ((M.eq_short ? M.s : M.L) + 3) / 4;   // blocks of k_aurora_dupdate
  float s = 0.f, mx = 0.f;
  for (int i = threadIdx.x; i < nb; i += 256) {
    s += gld<float>(M.tailpart + i);
    mx = fmaxf(mx, gld<float>(M.tailpart + nb + i));
  }
  s = block_sum(s, red);
  mx = block_max(mx, red);
  if (threadIdx.x == 0) {
    const float scale = 1.f / (sqrtf(s) + ns_eps);
    const float q = f8_scale(scale * sqrtf(mx));
    M.scal[SC_SCALE] = scale;
    M.scal[SC_F8Q] = q;
    M.scal[SC_F8INV2] = 1.f / (q * q);
  }
}

// ---------------------------------------------------------------------------
// Power iteration on X^T X for the operator-norm estimate. X is scaled by
// 1/||X||_F on the fly (the estimate is scale-free; this keeps fp32 away from
// under/overflow). A matrix whose step counter reached `steps` is skipped, so
// launching steps + 1 rounds lets a restarted matrix finish its steps.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float inv_fro(const DevMat& M) {
  const float n2 = M.scal[SC_XNORM2];
  return n2 > 0.f ? 1.f / sqrtf(n2) : 0.f;
}

// u = (X / ||X||) v : each wave owns kMvRows rows (16 rows per block); a
// lane loads 8 consecutive entries of v once and reuses them for every row.
// Rows past the end are read as the last row and their sums dropped.
constexpr int kMvRows = 4;
template <typename T>
__device__ __forceinline__ void matvec_body(const DevMat& M, int local) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = (local * 4 + w) * kMvRows;
  if (r0 >= M.rows) return;
  const bool vx = aligned16(M.xn, M.cols, sizeof(T) == 2 ? DT_BF16 : DT_F32);
  size_t ro[kMvRows];
#pragma unroll
  for (int k = 0; k < kMvRows; ++k) ro[k] = (size_t)min(r0 + k, M.rows - 1) * M.cols;
  float s[kMvRows];
#pragma unroll
  for (int k = 0; k < kMvRows; ++k) s[k] = 0.f;
  for (int c = lane * 8; c < M.cols; c += 512) {
    const int nv = min(8, M.cols - c);
    float v[8], x[kMvRows][8];
    if (vx && nv == 8) {
      const Ty<float>::Raw qv = Ty<float>::ld(M.pv, (size_t)c);   // pv is 256-byte aligned workspace
      typename Ty<T>::Raw q[kMvRows];
#pragma unroll
      for (int k = 0; k < kMvRows; ++k) q[k] = Ty<T>::ld(M.xn, ro[k] + c);
      Ty<float>::cvt(qv, v);
#pragma unroll
      for (int k = 0; k < kMvRows; ++k) Ty<T>::cvt(q[k], x[k]);
    } else {
      ld_part<float>(M.pv, (size_t)c, nv, v);
#pragma unroll
      for (int k = 0; k < kMvRows; ++k) ld_part<T>(M.xn, ro[k] + c, nv, x[k]);
    }
#pragma unroll
    for (int k = 0; k < kMvRows; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[k] += x[k][e] * v[e];
  }
  const float inv = inv_fro(M);
#pragma unroll
  for (int k = 0; k < kMvRows; ++k) {
    const float t = wave_sum(s[k]);
    if (lane == 0 && r0 + k < M.rows) gst<float>(M.pu + r0 + k, t * inv);
  }
}

__global__ __launch_bounds__(256) void k_power_matvec(const DevMat* __restrict__ mats, LaunchList L,
                                                      int steps, int final_pass) {
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (!final_pass && M.ist[IS_PSTEPS] >= steps) return;
  if (M.ns_t == DT_BF16) matvec_body<__bf16>(M, local);
  else matvec_body<float>(M, local);
}

// partial w = (X / ||X||)^T u over kRmvRows rows x kStreamCols columns per
// block; a lane issues the loads of kRmvBatch rows before using them.
constexpr int kRmvBatch = 8;
template <typename T>
__device__ __forceinline__ void rmatvec_body(const DevMat& M, int local) {
  const int tr = local / M.n_ct, tc = local % M.n_ct;
  const int c = tc * kStreamCols + threadIdx.x * 8;
  if (c >= M.cols) return;
  const int r0 = tr * kRmvRows, r1 = min(r0 + kRmvRows, M.rows);
  const int nv = min(8, M.cols - c);
  const bool fast = nv == 8 && aligned16(M.xn, M.cols, sizeof(T) == 2 ? DT_BF16 : DT_F32);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int r = r0;
  if (fast) {
    for (; r + kRmvBatch <= r1; r += kRmvBatch) {
      typename Ty<T>::Raw q[kRmvBatch];
      float u[kRmvBatch];
#pragma unroll
      for (int k = 0; k < kRmvBatch; ++k) q[k] = Ty<T>::ld(M.xn, (size_t)(r + k) * M.cols + c);
#pragma unroll
      for (int k = 0; k < kRmvBatch; ++k) u[k] = gld<float>(M.pu + r + k);
#pragma unroll
      for (int k = 0; k < kRmvBatch; ++k) {
        float x[8];
        Ty<T>::cvt(q[k], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += u[k] * x[e];
      }
    }
  }
  for (; r < r1; ++r) {
    float x[8];
    ld_part<T>(M.xn, (size_t)r * M.cols + c, nv, x);
    const float u = gld<float>(M.pu + r);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += u * x[e];
  }
  const float s = inv_fro(M);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c + e < M.cols) gst<float>(M.pwpart + (size_t)tr * M.cols + c + e, acc[e] * s);
}

__global__ __launch_bounds__(256) void k_power_rmatvec(const DevMat* __restrict__ mats, LaunchList L, int steps) {
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (M.ist[IS_PSTEPS] >= steps) return;
  if (M.ns_t == DT_BF16) rmatvec_body<__bf16>(M, local);
  else rmatvec_body<float>(M, local);
}

// Row-fused power step, for matrices with at most kFusedCols columns: a
// block takes a band of M.wband rows (256, 128 or 64, chosen per plan so that
// a launch has enough blocks) and writes, for each kFusedPart rows of it,
// w_part = (X/||X||)^T (X/||X||) v over those rows, with X read once.
// Thread t owns the 8-column chunks c = 8 t + 2048 j (j < J). A group of R
// rows is loaded into registers; the block reduces the rows' dot products
// with v (u_i, fixed order: each wave's lanes, then the four waves), and the
// same registers then add u_i X_i into the thread's part of w. Output:
// pwpart[part][c], summed over the parts in order by k_power_wsum as it sums
// the X^T u kernel's partials.
// 8 consecutive elements at byte offset `off` of a buffer resource (16 or 32
// bytes). The whole offset goes in the per-lane offset and the scalar offset
// is zero: the range check compares only the per-lane offset with the
// resource's size, so this is what makes a read past the range return zeros
// without touching memory.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ typename Ty<T>::Raw ld_rsrc(__amdgpu_buffer_rsrc_t r, int off) {
  typename Ty<T>::Raw q;
  if constexpr (sizeof(T) == 2) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    q = __builtin_bit_cast(u16x8_t, v);
  } else {
    q.a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    q.b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
  }
  return q;
}

// Sum over the wave in a fixed order, valid in every lane: DPP exchanges
// within each row of 16 lanes (pairs, quads, halves, rows), then the four
// row sums read from lanes 0, 16, 32 and 48.
template <int ctrl>
__device__ __forceinline__ float dpp_sum_step(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_sum_step<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_sum_step<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_sum_step<0x141>(v);   // row_half_mirror
  v = dpp_sum_step<0x140>(v);   // row_mirror
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a + b) + (c + d);
}

// Marks loaded chunks as changed, so the compiler converts them again after
// the barrier instead of holding both the raw and the converted values
// (twice the registers) across it.
__device__ __forceinline__ void keep_raw(u16x8_t& q) { asm volatile("" : "+v"(q)); }
__device__ __forceinline__ void keep_raw(Ty<float>::Raw& q) {
  asm volatile("" : "+v"(q.a));
  asm volatile("" : "+v"(q.b));
}

// One group of R rows of a fused block: its chunks, loaded through the
// block's resource (rows past the matrix read as zeros without touching
// memory, so every group issues the same loads).
template <typename T, int J, int R>
struct FusedGroup {
  typename Ty<T>::Raw q[R][J];
  // Rows are 16-byte multiples (the planner sends other matrices to the X v,
  // X^T u kernels), so chunks are whole; a chunk past the row's end reads
  // other data that neither the dot products nor the stored sums use.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rx, int rowb, int row0, int rb0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
      for (int j = 0; j < J; ++j)
        q[k][j] = ld_rsrc<T>(rx, (row0 + k - rb0) * rowb + (8 * t + 2048 * j) * (int)sizeof(T));
  }
  // u_k = (X_{row0+k} . v) / ||X||, reduced over the block (each wave's
  // lanes, then the four waves in order); then acc += u_k X_{row0+k} for the
  // rows of the matrix, in row order.
  __device__ __forceinline__ void step(const DevMat& M, int row0, const float* vsh, float (*red)[4][16], int buf,
                                       float inv, float (&acc)[J][8]) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, cols = M.cols;
    float p[R];
#pragma unroll
    for (int k = 0; k < R; ++k) p[k] = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 8 * t + 2048 * j;
      if (c < cols) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = vsh[c + e];   // zero past cols
#pragma unroll
        for (int k = 0; k < R; ++k) {
          float x[8];
          Ty<T>::cvt(q[k][j], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) p[k] += x[e] * v[e];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) p[k] = wave_sum_dpp(p[k]);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < R; ++k) red[buf][w][k] = p[k];
    }
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
      for (int j = 0; j < J; ++j) keep_raw(q[k][j]);
    __syncthreads();   // red[buf] is rewritten two groups later, after the next group's barrier
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (row0 + k >= M.rows) break;   // uniform
      const float u = (red[buf][0][k] + red[buf][1][k] + red[buf][2][k] + red[buf][3][k]) * inv;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float x[8];
        Ty<T>::cvt(q[k][j], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] += u * x[e];
      }
    }
  }
};

// A block's groups in order, two register buffers: group g+1's loads are in
// flight during group g's reduction, barrier and accumulation. One partial w
// per kFusedPart rows (R divides it), whatever the block's band, so the sums
// do not depend on how the rows were grouped into blocks.
template <typename T, int J, int R>
__device__ __forceinline__ void fused_body(const DevMat& M, int band, const float* vsh, float (*red)[4][16]) {
  static_assert(kFusedPart % R == 0, "groups tile a part");
  const int t = threadIdx.x, cols = M.cols;
  const float inv = inv_fro(M);
  const int rb0 = band * M.wband, rbn = min(M.wband, M.rows - rb0);
  const int rowb = cols * (int)sizeof(T);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)M.xn + (size_t)rb0 * rowb), (short)0, rbn * rowb, 0x00020000);
  constexpr int kGpp = kFusedPart / R;     // groups per part
  const int ng = (rbn + R - 1) / R;        // groups holding rows of the matrix (uniform)
  float acc[J][8];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  auto flush = [&](int g) {   // after group g: write and reset the part's sums at its end
    if ((g + 1) % kGpp != 0 && g + 1 != ng) return;
    const int part = rb0 / kFusedPart + g / kGpp;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 8 * t + 2048 * j;
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = acc[j][e] * inv;
        acc[j][e] = 0.f;
      }
      // cols is a multiple of 4 and the array 256-byte aligned: 16-byte stores
      float* dst = M.pwpart + (size_t)part * cols + c;
      if (c < cols) gst<f32x4_t>(dst, (f32x4_t){o[0], o[1], o[2], o[3]});
      if (c + 4 < cols) gst<f32x4_t>(dst + 4, (f32x4_t){o[4], o[5], o[6], o[7]});
    }
  };
  FusedGroup<T, J, R> ga, gb;
  ga.load(rx, rowb, rb0, rb0);
  for (int g = 0; g < ng; g += 2) {
    gb.load(rx, rowb, rb0 + (g + 1) * R, rb0);
    ga.step(M, rb0 + g * R, vsh, red, 0, inv, acc);
    flush(g);
    ga.load(rx, rowb, rb0 + (g + 2) * R, rb0);
    if (g + 1 < ng) {
      gb.step(M, rb0 + (g + 1) * R, vsh, red, 1, inv, acc);
      flush(g + 1);
    }
  }
}

// R rows per group (a power of two): at most 16 raw chunks per thread and
// buffer for bf16, 4 for fp32.
constexpr int pow2_floor(int x) { return x >= 8 ? 8 : x >= 4 ? 4 : x >= 2 ? 2 : 1; }
template <typename T, int J>
__device__ __forceinline__ void fused_dispatch_r(const DevMat& M, int band, const float* vsh, float (*red)[4][16]) {
  constexpr int R = pow2_floor((sizeof(T) == 2 ? 16 : 4) / J);
  fused_body<T, J, R>(M, band, vsh, red);
}
// Dynamic LDS: v, padded with zeros to the launch's widest matrix rounded up
// to 8 columns (at most kFusedCols). One launch per NS type (the fp32 forms
// need more registers); a block takes the form for its matrix's chunk count
// J = ceil(cols / 2048), so matrices of all widths share the launch.
template <typename T>
__global__ __launch_bounds__(256) void k_power_fused(const DevMat* __restrict__ mats, LaunchList L, int steps) {
  extern __shared__ float vsh[];
  __shared__ float red[2][4][16];
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (M.ist[IS_PSTEPS] >= steps) return;
  const int cp = (M.cols + 7) & ~7;
  for (int c = threadIdx.x; c < cp; c += 256) vsh[c] = c < M.cols ? gld<float>(M.pv + c) : 0.f;
  __syncthreads();
  switch ((M.cols + 2047) / 2048) {
    case 1: fused_dispatch_r<T, 1>(M, local, vsh, red); break;
    case 2: fused_dispatch_r<T, 2>(M, local, vsh, red); break;
    case 3: fused_dispatch_r<T, 3>(M, local, vsh, red); break;
    case 4: fused_dispatch_r<T, 4>(M, local, vsh, red); break;
    case 5: fused_dispatch_r<T, 5>(M, local, vsh, red); break;
    default: fused_dispatch_r<T, 6>(M, local, vsh, red); break;
  }
}

// w = sum over the row tiles of the partials (one thread per column, stored
// in row 0 of the partials); block b of a matrix writes linepart[b] = its
// part of ||w||^2.
__global__ __launch_bounds__(256) void k_power_wsum(DevMat* __restrict__ mats, LaunchList L, int steps) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (M.ist[IS_PSTEPS] >= steps) return;
  const int c = local * 256 + threadIdx.x;
  float s = 0.f;
  if (c < M.cols) {
    s = strided_sum(M.pwpart + c, (size_t)M.cols, M.n_rmv);
    gst<float>(M.pwpart + c, s);   // only this thread reads column c
  }
  const float n2 = block_sum(s * s, red);
  if (threadIdx.x == 0) gst<float>(M.linepart + local, n2);
}

// v = w / ||w|| (one block per matrix), with the restart rule for a start
// vector that X annihilates.
__global__ __launch_bounds__(256) void k_power_normalize(DevMat* __restrict__ mats, LaunchList L, int steps) {
  __shared__ float red[8];
  __shared__ float bestv[256];
  __shared__ int besti[256];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (M.ist[IS_PSTEPS] >= steps) return;
  const int t = threadIdx.x;
  const int ncb = (M.cols + 255) / 256;
  float n2 = 0.f;
  for (int b = t; b < ncb; b += 256) n2 += gld<float>(M.linepart + b);
  n2 = block_sum(n2, red);
  __syncthreads();
  if (n2 > 0.f) {
    const float inv = 1.f / sqrtf(n2);
    for (int c = t; c < M.cols; c += 256) gst<float>(M.pv + c, gld<float>(M.pwpart + c) * inv);
    if (t == 0) { M.ist[IS_PSTEPS] += 1; M.scal[SC_PNORM] = sqrtf(n2); }
    return;
  }
  // w == 0
  const bool xzero = !(M.scal[SC_XNORM2] > 0.f);
  if (xzero || M.ist[IS_RESTART]) {
    if (t == 0) M.ist[IS_PSTEPS] = steps;   // nothing to iterate: sigma comes out 0
    return;
  }
  // restart from e_j, j = first column of largest norm
  float bv = -1.f; int bi = 0;
  const bool wide = M.rows < M.cols;
  for (int c = t; c < M.cols; c += 256) {
    float s;
    if (wide) {
      s = gld<float>(M.colsq + c);
    } else {
      s = 0.f;
      for (int r = 0; r < M.rows; ++r) {
        const float x = ld1_rt(M.xn, M.ns_t, (size_t)r * M.cols + c);
        s += x * x;
      }
    }
    if (s > bv) { bv = s; bi = c; }
  }
  bestv[t] = bv; besti[t] = bi;
  __syncthreads();
  if (t == 0) {
    float b = -1.f; int j = 0;
    for (int i = 0; i < 256; ++i)
      if (bestv[i] > b || (bestv[i] == b && besti[i] < j)) { b = bestv[i]; j = besti[i]; }
    besti[0] = j;
    M.ist[IS_RESTART] = 1;
  }
  __syncthreads();
  const int j = besti[0];
  for (int c = t; c < M.cols; c += 256) gst<float>(M.pv + c, (c == j) ? 1.f : 0.f);
}

// sigma = ||X v|| (from u = (X/||X||) v), kappa = (contra/2) / max(sigma, 1e-7).
// A fused-tail matrix takes sigma in the tail instead (k_tail_finalize).
__global__ __launch_bounds__(256) void k_power_sigma(DevMat* __restrict__ mats, LaunchList L, float contra) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (M.ftail) return;
  float s = 0.f;
  for (int r = threadIdx.x; r < M.rows; r += 256) {
    const float u = gld<float>(M.pu + r);
    s += u * u;
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) {
    const float n2 = M.scal[SC_XNORM2];
    const float sigma = (n2 > 0.f && M.ist[IS_PSTEPS] > 0) ? sqrtf(s) * sqrtf(n2) : 0.f;
    M.scal[SC_SIGMA] = sigma;
    M.scal[SC_KAPPA] = 0.5f * contra / fmaxf(sigma, 1e-7f);
  }
}

// ---------------------------------------------------------------------------
// Tail. U is the final NS iterate read in storage orientation: x[fin] for
// wide/square (ld L_pad), xt[fin] for tall (ld s_pad). U rows are padded to
// a multiple of 256 with zeros, so U chunks are always read whole.
// ---------------------------------------------------------------------------
__device__ __forceinline__ const void* u_ptr(const DevMat& M, int64_t* ld) {
  if (M.tall) { *ld = M.s_pad; return M.xt[M.fin]; }
  *ld = M.L_pad; return M.x[M.fin];
}

// The U, X and W rows r..r+R-1 at column c: vector loads of all three
// issued before any is used (X only when kappa != 0, W only when given);
// a row is converted when it is consumed.
template <typename T, typename TW, int R>
struct TailRows {
  typename Ty<T>::Raw qu[R], qx[R];
  typename Ty<TW>::Raw qw[R];
  __device__ __forceinline__ void load(const DevMat& M, const void* U, int64_t ldu, int r, int c, bool use_x,
                                       bool has_w) {
#pragma unroll
    for (int k = 0; k < R; ++k) qu[k] = Ty<T>::ld(U, (size_t)(r + k) * ldu + c);
    if (use_x) {
#pragma unroll
      for (int k = 0; k < R; ++k) qx[k] = Ty<T>::ld(M.xn, (size_t)(r + k) * M.cols + c);
    }
    if (has_w) {
#pragma unroll
      for (int k = 0; k < R; ++k) qw[k] = Ty<TW>::ld(M.w, (size_t)(r + k) * M.ld_w + c);
    }
  }
  __device__ __forceinline__ void row(int k, bool use_x, bool has_w, float u[8], float x[8], float w[8]) const {
    Ty<T>::cvt(qu[k], u);
    if (use_x) Ty<T>::cvt(qx[k], x);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    if (has_w) Ty<TW>::cvt(qw[k], w);
  }
};
// Element-wise form for one row (ragged chunk, short tile, or unaligned
// caller buffers).
template <typename T, typename TW>
__device__ __forceinline__ void tail_load_part(const DevMat& M, const void* U, int64_t ldu, int r, int c, int nv,
                                               bool use_x, bool has_w, float u[8], float x[8], float w[8]) {
  ld_part<T>(U, (size_t)r * ldu + c, nv, u);
  if (use_x) ld_part<T>(M.xn, (size_t)r * M.cols + c, nv, x);
  else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
  }
  if (has_w) ld_part<TW>(M.w, (size_t)r * M.ld_w + c, nv, w);
}

// Partial sums per streaming tile: ||U||^2, ||U - kappa X||^2, ||W||^2.
template <typename T, typename TW>
__device__ __forceinline__ void tail_reduce_body(const DevMat& M, int local, float (*red)[4]) {
  constexpr int R = kWaveRows;
  const int tr = local / M.n_seg, sg = local % M.n_seg;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = sg * kSegCols + lane * 8;
  const int r = tr * kStreamRows + w * R;
  const int nr = max(0, min(R, M.rows - r));
  int64_t ldu;
  const void* U = u_ptr(M, &ldu);
  const float kappa = M.scal[SC_KAPPA];
  const bool use_x = kappa != 0.f, has_w = M.w != nullptr;
  const int nv = max(0, min(8, M.cols - c));
  const bool fast = nr == R && nv == 8 && aligned16(M.xn, M.cols, M.ns_t) &&
                    (!has_w || aligned16(M.w, M.ld_w, M.dt_w));
  float su = 0.f, sv = 0.f, sw = 0.f;
  auto acc = [&](const float* u, const float* x, const float* wv) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      su += u[e] * u[e];
      const float v = u[e] - kappa * x[e];
      sv += v * v;
    }
    if (has_w) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sw += wv[e] * wv[e];
    }
  };
  if (fast) {
    // fp32 operands load in two batches of R/2 rows: the kernel's register
    // budget is set by its largest body
    constexpr int RB = (sizeof(T) == 2 && sizeof(TW) == 2) ? R : R / 2;
#pragma unroll
    for (int k0 = 0; k0 < R; k0 += RB) {
      TailRows<T, TW, RB> q;
      q.load(M, U, ldu, r + k0, c, use_x, has_w);
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        float u[8], x[8], wv[8];
        q.row(k, use_x, has_w, u, x, wv);
        acc(u, x, wv);
      }
    }
  } else if (nv > 0) {
    for (int k = 0; k < nr; ++k) {
      float u[8], x[8], wv[8];
      tail_load_part<T, TW>(M, U, ldu, r + k, c, nv, use_x, has_w, u, x, wv);
      acc(u, x, wv);
    }
  }
  su = wave_sum(su); sv = wave_sum(sv); sw = wave_sum(sw);
  if (lane == 0) { red[0][w] = su; red[1][w] = sv; red[2][w] = sw; }
  __syncthreads();
  if (threadIdx.x < 3) {
    const int k = threadIdx.x;
    gst<float>(M.tailpart + (size_t)local * 4 + k, red[k][0] + red[k][1] + red[k][2] + red[k][3]);
  }
}

// W's type when there is no W: any (its loads are skipped); T keeps one body.
#define TAIL_DISPATCH(BODY, ...)                                                    \
  do {                                                                              \
    const int tw_ = M.w ? M.dt_w : M.ns_t;                                          \
    if (M.ns_t == DT_BF16) {                                                        \
      if (tw_ == DT_BF16) BODY<__bf16, __bf16>(__VA_ARGS__);                       \
      else BODY<__bf16, float>(__VA_ARGS__);                                        \
    } else {                                                                        \
      if (tw_ == DT_BF16) BODY<float, __bf16>(__VA_ARGS__);                        \
      else BODY<float, float>(__VA_ARGS__);                                         \
    }                                                                               \
  } while (0)

__global__ __launch_bounds__(256) void k_tail_reduce(const DevMat* __restrict__ mats, LaunchList L) {
  __shared__ float red[3][4];
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  TAIL_DISPATCH(tail_reduce_body, M, local, red);
}

// Fused tail, sigma = ||X v||: u_i = the sum of storage row i's parts over
// its 64-column blocks (frow, from the final product's epilogue, in block
// order), then per block of 256 rows the sum of u_i^2 into linepart[local]
// (free by the tail: the norms and the power iteration are done with it).
__global__ __launch_bounds__(256) void k_tail_rows(const DevMat* __restrict__ mats, LaunchList L) {
  __shared__ float red[8];
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int i = local * 256 + threadIdx.x;
  const int nbc = (M.cols + 63) / 64;
  const float u = i < M.rows ? strided_sum(M.frow + i, (size_t)M.rows, nbc) : 0.f;
  const float s = block_sum(u * u, red);
  if (threadIdx.x == 0) gst<float>(M.linepart + local, s);
}

// alpha = ||U|| / max(||U - kappa X||, 1e-10) * sqrt(max(1, rows/cols)),
// then the u/w-floor: if max(||V||,1e-8) / max(||W||,1e-8) < target, scale up.
// A fused-tail matrix has ||U||^2 and <U, X> per 64 x 64 block (ftail),
// ||W||^2 per streaming tile (fwp) and, with the Contra term, sigma's row
// blocks (linepart, k_tail_rows): sigma and kappa are set here, and
// ||U - kappa X||^2 = ||U||^2 - 2 kappa <U, X> + kappa^2 ||X||^2 (no
// cancellation to fear: kappa X has operator norm contra / 2 < 1 = that of U).
__global__ __launch_bounds__(256) void k_tail_finalize(DevMat* __restrict__ mats, LaunchList L, float target_uw,
                                                       float contra) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int nb = M.n_rt * M.n_seg;
  float su = 0.f, sv = 0.f, sw = 0.f, sx = 0.f;
  if (M.ftail) {
    const int nft = ((M.rows + 63) / 64) * ((M.cols + 63) / 64);
    const int nrb = (M.rows + 255) / 256;
    for (int i = threadIdx.x; i < nft; i += 256) {
      su += gld<float>(M.ftail + (size_t)i * 2 + 0);
      sx += gld<float>(M.ftail + (size_t)i * 2 + 1);
    }
    if (M.ftw)
      for (int i = threadIdx.x; i < nb; i += 256) sw += gld<float>(M.fwp + i);
    if (M.ftx)
      for (int i = threadIdx.x; i < nrb; i += 256) sv += gld<float>(M.linepart + i);
  } else {
    for (int i = threadIdx.x; i < nb; i += 256) {
      su += gld<float>(M.tailpart + (size_t)i * 4 + 0);
      sv += gld<float>(M.tailpart + (size_t)i * 4 + 1);
      sw += gld<float>(M.tailpart + (size_t)i * 4 + 2);
    }
  }
  su = block_sum(su, red);
  sv = block_sum(sv, red);
  sw = block_sum(sw, red);
  sx = block_sum(sx, red);
  if (threadIdx.x == 0 && M.ftail) {
    // sv holds sum u_i^2 with u = (X / ||X||) v here
    float kappa = 0.f;
    const float n2 = M.scal[SC_XNORM2];
    if (M.ftx) {
      const float sigma = (n2 > 0.f && M.ist[IS_PSTEPS] > 0) ? sqrtf(sv) * sqrtf(n2) : 0.f;
      kappa = 0.5f * contra / fmaxf(sigma, 1e-7f);
      M.scal[SC_SIGMA] = sigma;
      M.scal[SC_KAPPA] = kappa;
    }
    sv = fmaxf(su - 2.f * kappa * sx + kappa * kappa * n2, 0.f);
  }
  if (threadIdx.x == 0) {
    const float f = sqrtf(su), nv = sqrtf(sv);
    float alpha = f / fmaxf(nv, 1e-10f);
    alpha *= sqrtf(fmaxf(1.f, (float)M.rows / (float)M.cols));
    if (M.w && target_uw > 0.f) {
      const float p = fmaxf(sqrtf(sw), 1e-8f);
      const float u = fmaxf(alpha * nv, 1e-8f);
      if (u / p < target_uw) alpha *= target_uw * p / u;
    }
    M.scal[SC_UNORM2] = su;
    M.scal[SC_VNORM2] = sv;
    M.scal[SC_WNORM2] = sw;
    M.scal[SC_ALPHA] = alpha;
  }
}

// V = alpha (U - kappa X); update_out <- V; W <- W - lr V.
// copy_only: V = U (the polar entry points' output copy).
template <typename T, typename TW>
__device__ __forceinline__ void tail_apply_body(const DevMat& M, int local, float lr, int copy_only) {
  constexpr int R = kWaveRows;
  const int tr = local / M.n_seg, sg = local % M.n_seg;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = sg * kSegCols + lane * 8;
  const int r = tr * kStreamRows + w * R;
  const int nr = max(0, min(R, M.rows - r));
  if (c >= M.cols || nr == 0) return;
  int64_t ldu;
  const void* U = u_ptr(M, &ldu);
  const float kappa = copy_only ? 0.f : M.scal[SC_KAPPA];
  const float alpha = copy_only ? 1.f : M.scal[SC_ALPHA];
  const bool use_x = kappa != 0.f, has_w = M.w != nullptr, has_o = M.uo != nullptr;
  const int nv = min(8, M.cols - c);
  const bool fast = nr == R && nv == 8 && aligned16(M.xn, M.cols, M.ns_t) &&
                    (!has_w || aligned16(M.w, M.ld_w, M.dt_w)) && (!has_o || aligned16(M.uo, M.ld_uo, M.dt_uo));
  auto out = [&](int rr, const float* u, const float* x, float* wv, bool vec) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = alpha * (u[e] - kappa * x[e]);
    if (has_o) {
      const size_t io = (size_t)rr * M.ld_uo + c;
      if (vec) st_vec_rt(M.uo, M.dt_uo, io, v); else st_part_rt(M.uo, M.dt_uo, io, nv, v);
    }
    if (has_w) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = wv[e] - lr * v[e];
      const size_t iw = (size_t)rr * M.ld_w + c;
      if (vec) Ty<TW>::st(M.w, iw, wv); else st_part<TW>(M.w, iw, nv, wv);
    }
  };
  if (fast) {
    // fp32 operands load in two batches of R/2 rows: the kernel's register
    // budget is set by its largest body
    constexpr int RB = (sizeof(T) == 2 && sizeof(TW) == 2) ? R : R / 2;
#pragma unroll
    for (int k0 = 0; k0 < R; k0 += RB) {
      TailRows<T, TW, RB> q;
      q.load(M, U, ldu, r + k0, c, use_x, has_w);
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        float u[8], x[8], wv[8];
        q.row(k, use_x, has_w, u, x, wv);
        out(r + k0 + k, u, x, wv, true);
      }
    }
  } else {
    for (int k = 0; k < nr; ++k) {
      float u[8], x[8], wv[8];
      tail_load_part<T, TW>(M, U, ldu, r + k, c, nv, use_x, has_w, u, x, wv);
      out(r + k, u, x, wv, false);
    }
  }
}

__global__ __launch_bounds__(256) void k_tail_apply(const DevMat* __restrict__ mats, LaunchList L, float lr,
                                                    int copy_only) {
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  TAIL_DISPATCH(tail_apply_body, M, local, lr, copy_only);
}

// ---------------------------------------------------------------------------
// Host-side launchers (grid sizes come from the planner's LaunchList).
// ---------------------------------------------------------------------------
#define LAUNCH(kern, nblk, ...)                                                            \
  do {                                                                                     \
    if ((nblk) > 0) hipLaunchKernelGGL(kern, dim3(nblk), dim3(256), 0, st, __VA_ARGS__);   \
  } while (0)

hipError_t launch_momentum_stats(const DevMat* m, LaunchList L, int nblk, int nesterov_pass, float mu,
                                 int nesterov, int sgd, hipStream_t st) {
  LAUNCH(k_momentum_stats, nblk, m, L, nesterov_pass, mu, nesterov, sgd);
  return hipGetLastError();
}
hipError_t launch_wnorm(const DevMat* m, LaunchList L, int nblk, hipStream_t st) {
  LAUNCH(k_wnorm, nblk, m, L);
  return hipGetLastError();
}
hipError_t launch_check_finite(DevMat* m, LaunchList L, int nblk, int upd, hipStream_t st) {
  LAUNCH(k_check_finite, nblk, m, L, upd);
  return hipGetLastError();
}
hipError_t launch_norms_lines(DevMat* m, LaunchList L, int nblk, float pp_eps, hipStream_t st) {
  LAUNCH(k_norms_lines, nblk, m, L, pp_eps);
  return hipGetLastError();
}
hipError_t launch_norms_scalars(DevMat* m, LaunchList L, int nblk, float ns_eps, int init_power, hipStream_t st) {
  LAUNCH(k_norms_scalars, nblk, m, L, ns_eps, init_power);
  return hipGetLastError();
}
hipError_t launch_prologue(int ns_t, const DevMat* m, LaunchList L, int nblk, int use_xn, hipStream_t st) {
  if (ns_t == DT_BF16) LAUNCH(k_prologue<__bf16>, nblk, m, L, use_xn);
  else LAUNCH(k_prologue<float>, nblk, m, L, use_xn);
  return hipGetLastError();
}
hipError_t launch_aurora_dupdate(int ns_t, DevMat* m, LaunchList L, int nblk, float pp_eps, float pp_beta,
                                 hipStream_t st) {
  if (ns_t == DT_BF16) LAUNCH(k_aurora_dupdate<__bf16>, nblk, m, L, pp_eps, pp_beta);
  else LAUNCH(k_aurora_dupdate<float>, nblk, m, L, pp_eps, pp_beta);
  return hipGetLastError();
}
hipError_t launch_aurora_dfinish(DevMat* m, LaunchList L, int nblk, float pp_eps, float pp_beta, hipStream_t st) {
  LAUNCH(k_aurora_dfinish, nblk, m, L, pp_eps, pp_beta);
  return hipGetLastError();
}
hipError_t launch_aurora_scale(DevMat* m, LaunchList L, int nblk, float ns_eps, hipStream_t st) {
  LAUNCH(k_aurora_scale, nblk, m, L, ns_eps);
  return hipGetLastError();
}
hipError_t launch_power_matvec(const DevMat* m, LaunchList L, int nblk, int steps, int final_pass, hipStream_t st) {
  LAUNCH(k_power_matvec, nblk, m, L, steps, final_pass);
  return hipGetLastError();
}
hipError_t launch_power_rmatvec(const DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st) {
  LAUNCH(k_power_rmatvec, nblk, m, L, steps);
  return hipGetLastError();
}
hipError_t launch_power_fused(int ns_t, const DevMat* m, LaunchList L, int nblk, int steps, int max_cols,
                              hipStream_t st) {
  if (max_cols > kFusedCols || max_cols < 1) return hipErrorInvalidValue;
  const size_t lds = (size_t)((max_cols + 7) & ~7) * sizeof(float);
  if (nblk <= 0) return hipSuccess;
  if (ns_t == DT_BF16) hipLaunchKernelGGL(k_power_fused<__bf16>, dim3(nblk), dim3(256), lds, st, m, L, steps);
  else hipLaunchKernelGGL(k_power_fused<float>, dim3(nblk), dim3(256), lds, st, m, L, steps);
  return hipGetLastError();
}
hipError_t launch_power_wsum(DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st) {
  LAUNCH(k_power_wsum, nblk, m, L, steps);
  return hipGetLastError();
}
hipError_t launch_power_normalize(DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st) {
  LAUNCH(k_power_normalize, nblk, m, L, steps);
  return hipGetLastError();
}
hipError_t launch_power_sigma(DevMat* m, LaunchList L, int nblk, float contra, hipStream_t st) {
  LAUNCH(k_power_sigma, nblk, m, L, contra);
  return hipGetLastError();
}
hipError_t launch_tail_reduce(const DevMat* m, LaunchList L, int nblk, hipStream_t st) {
  LAUNCH(k_tail_reduce, nblk, m, L);
  return hipGetLastError();
}
hipError_t launch_tail_rows(const DevMat* m, LaunchList L, int nblk, hipStream_t st) {
  LAUNCH(k_tail_rows, nblk, m, L);
  return hipGetLastError();
}
hipError_t launch_tail_finalize(DevMat* m, LaunchList L, int nblk, float target_uw, float contra, hipStream_t st) {
  LAUNCH(k_tail_finalize, nblk, m, L, target_uw, contra);
  return hipGetLastError();
}
hipError_t launch_tail_apply(const DevMat* m, LaunchList L, int nblk, float lr, int copy_only, hipStream_t st) {
  LAUNCH(k_tail_apply, nblk, m, L, lr, copy_only);
  return hipGetLastError();
}

}  // namespace muon
