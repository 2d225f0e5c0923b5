// Bandwidth-bound kernels of the Muon step (everything but the Newton-Schulz
// products). Step names and formulas follow the Aurora record page
// (www.xxmr.cn/news/295280): section 组合优化栈 (muon_update: momentum lerp,
// Nesterov blend, unit-operator-norm direction, Contra-Muon, Frobenius
// restore, aspect scale; u/w-floor and the parameter add) and sections
// Aurora 的迭代伪代码 / 源码实现 (the diagonal preconditioner D).
//
// Every launch covers a whole batch: a LaunchList maps block b to a matrix
// and a local block index. Streaming tiles are kStreamRows x kStreamCols; a
// wave owns a kSegCols-column segment, a lane 8 consecutive columns. All
// reductions are two-stage (per-block partials, then a fixed-order sum in a
// per-matrix block): no atomics, bitwise reproducible.
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

__device__ __forceinline__ int find_job(const LaunchList& L, int b, int* local) {
  int lo = 0, hi = L.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (L.off[mid] <= b) lo = mid; else hi = mid - 1;
  }
  *local = b - L.off[lo];
  return L.mat[lo];
}

// Load 8 consecutive elements of row r starting at column c (c % 8 == 0),
// zero beyond `cols`. `vec` = row starts and ld are 16-byte aligned.
__device__ __forceinline__ void load8(const void* base, int dt, int64_t ld, int r, int c, int cols,
                                      bool vec, float v[8]) {
  if (dt == DT_BF16) {
    const unsigned short* p = (const unsigned short*)base + (size_t)r * ld + c;
    if (vec && c + 8 <= cols) {
      const u16x8_t q = *(const u16x8_t*)p;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = bf2f(q[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (c + e < cols) ? bf2f(p[e]) : 0.f;
    }
  } else {
    const float* p = (const float*)base + (size_t)r * ld + c;
    if (vec && c + 8 <= cols) {
      const f32x4_t q0 = *(const f32x4_t*)p, q1 = *(const f32x4_t*)(p + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = q0[e]; v[e + 4] = q1[e]; }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (c + e < cols) ? p[e] : 0.f;
    }
  }
}

__device__ __forceinline__ void store8(void* base, int dt, int64_t ld, int r, int c, int cols,
                                       bool vec, const float v[8]) {
  if (dt == DT_BF16) {
    unsigned short* p = (unsigned short*)base + (size_t)r * ld + c;
    if (vec && c + 8 <= cols) {
      u16x8_t q;
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = f2bf(v[e]);
      *(u16x8_t*)p = q;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) if (c + e < cols) p[e] = f2bf(v[e]);
    }
  } else {
    float* p = (float*)base + (size_t)r * ld + c;
    if (vec && c + 8 <= cols) {
      *(f32x4_t*)p = (f32x4_t){v[0], v[1], v[2], v[3]};
      *(f32x4_t*)(p + 4) = (f32x4_t){v[4], v[5], v[6], v[7]};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) if (c + e < cols) p[e] = v[e];
    }
  }
}

// Round to the storage type and back (what a later read of a stored value sees).
__device__ __forceinline__ float round_to(int dt, float x) { return dt == DT_BF16 ? bf2f(f2bf(x)) : x; }

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

}  // namespace

// ---------------------------------------------------------------------------
// K1: momentum EMA + Nesterov blend, and the sums of squares of the result.
//   M <- M + (1 - mu)(G - M);  X = G + mu (M - G)  (X = M without Nesterov)
// X is stored in the NS type (rounded), and the norms are taken of the stored
// values. With `nesterov_pass` false this only gathers the norms of the
// matrix given in `g` (the polar entry points).
// Outputs per tile: rowpart[r][seg] (row sums over a wave segment) and, for
// wide matrices, colpart[tile_row][c].
// ---------------------------------------------------------------------------
constexpr int kRB = 4;   // rows whose loads are issued together (memory-level parallelism)

__global__ __launch_bounds__(256) void k_momentum_stats(const DevMat* __restrict__ mats, LaunchList L,
                                                        int nesterov_pass, float mu, int nesterov) {
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int tr = local / M.n_ct, tc = local % M.n_ct;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = tc * kStreamCols + w * kSegCols + lane * 8;
  const int seg = tc * (kStreamCols / kSegCols) + w;
  const int r0 = tr * kStreamRows;
  const int r1 = min(r0 + kStreamRows, M.rows);
  const bool wide_cols = M.rows < M.cols;
  const bool vg = aligned16(M.g, M.ld_g, M.dt_g);
  const bool vm = nesterov_pass ? aligned16(M.m, M.ld_m, DT_F32) : false;
  const bool vx = nesterov_pass ? aligned16(M.xn, M.cols, M.ns_t) : false;
  const bool live = c < M.cols;
  const bool seg_live = seg < M.n_seg;
  float col[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0; r < r1; r += kRB) {
    // all loads of kRB rows first: the compiler cannot prove that the
    // stores of one row do not alias the next row's inputs, so a per-row
    // loop would serialise the memory traffic row by row
    float x[kRB][8], m[kRB][8];
#pragma unroll
    for (int k = 0; k < kRB; ++k) {
      const bool ok = live && r + k < r1;
      if (ok) {
        load8(M.g, M.dt_g, M.ld_g, r + k, c, M.cols, vg, x[k]);
        if (nesterov_pass) load8(M.m, DT_F32, M.ld_m, r + k, c, M.cols, vm, m[k]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[k][e] = m[k][e] = 0.f;
      }
    }
    if (nesterov_pass) {
#pragma unroll
      for (int k = 0; k < kRB; ++k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = x[k][e];
          const float mn = m[k][e] + (1.f - mu) * (g - m[k][e]);
          m[k][e] = mn;
          x[k][e] = round_to(M.ns_t, nesterov ? g + mu * (mn - g) : mn);
        }
        if (live && r + k < r1) {
          store8(M.m, DT_F32, M.ld_m, r + k, c, M.cols, vm, m[k]);
          store8(M.xn, M.ns_t, M.cols, r + k, c, M.cols, vx, x[k]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kRB; ++k) {
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { rs += x[k][e] * x[k][e]; col[e] += x[k][e] * x[k][e]; }
      rs = wave_sum(rs);
      if (lane == 0 && seg_live && r + k < r1) M.rowpart[(size_t)(r + k) * M.n_seg + seg] = rs;
    }
  }
  if (wide_cols) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c + e < M.cols) M.colpart[(size_t)tr * M.cols + c + e] = col[e];
  }
}

// ---------------------------------------------------------------------------
// Per-matrix finaliser of the norms: row/column sums of squares, ||X||_F^2,
// the long-side norms rho, Aurora's initial D = 1 / max(rho, pp_eps), the
// prologue scale 1 / (||D * T||_F + ns_eps) (D = 1 without Aurora), and the
// power-iteration start v = ones / sqrt(cols).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_norms_finalize(DevMat* __restrict__ mats, LaunchList L,
                                                        float pp_eps, float ns_eps, int init_power) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int t = threadIdx.x;
  float tot = 0.f;
  for (int r = t; r < M.rows; r += 256) {
    float s = 0.f;
    for (int k = 0; k < M.n_seg; ++k) s += M.rowpart[(size_t)r * M.n_seg + k];
    M.rowsq[r] = s;
    tot += s;
  }
  const bool wide = M.rows < M.cols;
  if (wide) {
    for (int c = t; c < M.cols; c += 256) {
      float s = 0.f;
      for (int k = 0; k < M.n_rt; ++k) s += M.colpart[(size_t)k * M.cols + c];
      M.colsq[c] = s;
    }
  }
  tot = block_sum(tot, red);
  __syncthreads();
  float ysq = 0.f;
  if (M.aurora) {
    const float* lsq = wide ? M.colsq : M.rowsq;
    for (int l = t; l < M.L; l += 256) {
      const float rho = sqrtf(lsq[l]);
      const float d = 1.f / fmaxf(rho, pp_eps);
      M.rho[l] = rho;
      M.dvec[l] = d;
      ysq += (d * rho) * (d * rho);
    }
    ysq = block_sum(ysq, red);
  } else {
    ysq = tot;
  }
  if (init_power) {
    const float v0 = 1.f / sqrtf((float)M.cols);
    for (int c = t; c < M.cols; c += 256) M.pv[c] = v0;
  }
  if (t == 0) {
    M.scal[SC_XNORM2] = tot;
    M.scal[SC_SCALE] = 1.f / (sqrtf(ysq) + ns_eps);
    M.scal[SC_SIGMA] = 0.f;
    M.scal[SC_KAPPA] = 0.f;
    M.ist[IS_PSTEPS] = 0;
    M.ist[IS_RESTART] = 0;
  }
}

// ---------------------------------------------------------------------------
// NS prologue through an LDS transpose: X0 = scale * D o T in the wide
// orientation, written to x[0] (s_pad x L_pad) and its transpose to xt[0]
// (L_pad x s_pad), zero padded (the first iteration's products read both). T is the source in storage orientation (rows x cols); for a
// tall source the wide iterate is its transpose. 64 x 64 tiles over the
// padded storage frame.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_prologue(const DevMat* __restrict__ mats, LaunchList L, int use_xn) {
  __shared__ float tile[64][65];
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int pc = M.tall ? M.s_pad : M.L_pad;   // padded storage frame: columns
  const int ntc = pc / 64;
  const int br = (local / ntc) * 64, bc = (local % ntc) * 64;
  const void* src = use_xn ? (const void*)M.xn : M.g;
  const int64_t lds = use_xn ? (int64_t)M.cols : M.ld_g;
  const int sdt = use_xn ? M.ns_t : M.dt_g;
  const bool vs = aligned16(src, lds, sdt);
  const float scale = M.scal[SC_SCALE];
  // direct frame: wide -> x[0] (ld L_pad); tall -> xt[0] (ld s_pad)
  void* dir = M.tall ? M.xt[0] : M.x[0];
  void* tra = M.tall ? M.x[0] : M.xt[0];
  const int ld_dir = M.tall ? M.s_pad : M.L_pad;
  const int ld_tra = M.tall ? M.L_pad : M.s_pad;
  const int odt = sizeof(T) == 2 ? DT_BF16 : DT_F32;
  // 64 x 64 tile = 512 chunks of 8 columns; two chunks per thread
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = h * 256 + threadIdx.x;
    const int i = q >> 3, j = (q & 7) * 8;
    const int r = br + i, c = bc + j;
    float v[8];
    if (r < M.rows) {
      load8(src, sdt, lds, r, c, M.cols, vs, v);   // zero past cols
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float d = scale;
      if (M.aurora && r < M.rows && c + e < M.cols) d *= M.dvec[M.tall ? r : c + e];
      v[e] *= d;
      tile[i][j + e] = v[e];
    }
    store8(dir, odt, ld_dir, r, c, c + 8, true, v);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = h * 256 + threadIdx.x;
    const int jc = q >> 3, i0 = (q & 7) * 8;   // transposed row = tile column jc
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[i0 + e][jc];
    store8(tra, odt, ld_tra, bc + jc, br + i0, br + i0 + 8, true, v);
  }
}

// ---------------------------------------------------------------------------
// Aurora D update between passes: row_sq_l = max(sum_i U[i][l]^2, eps^2) over
// the short side (row l of U^T), D_l *= (target / row_sq_l)^beta with
// target = s / L; then partial sums of (D_l rho_l)^2 per block. One wave per
// long-side row l; 4 rows per block.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_aurora_dupdate(DevMat* __restrict__ mats, LaunchList L,
                                                        int fin, float pp_eps, float pp_beta) {
  __shared__ float red[4];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l = local * 4 + w;
  float contrib = 0.f;
  if (l < M.L) {
    const T* ut = (const T*)M.xt[fin] + (size_t)l * M.s_pad;
    float s = 0.f;
    for (int i = lane * 8; i < M.s; i += 512) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float u;
        if constexpr (sizeof(T) == 2) u = bf2f(((const unsigned short*)ut)[i + e]);
        else u = ((const float*)ut)[i + e];
        s += u * u;     // entries past s are zero padding
      }
    }
    s = wave_sum(s);
    if (lane == 0) {
      const float target = (float)M.s / (float)M.L;
      const float rsq = fmaxf(s, pp_eps * pp_eps);
      const float d = M.dvec[l] * powf(target / rsq, pp_beta);
      M.dvec[l] = d;
      const float y = d * M.rho[l];
      contrib = y * y;
    }
  }
  if (lane == 0) red[w] = contrib;
  __syncthreads();
  if (threadIdx.x == 0) M.tailpart[local] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void k_aurora_scale(DevMat* __restrict__ mats, LaunchList L, float ns_eps) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int nb = (M.L + 3) / 4;
  float s = 0.f;
  for (int i = threadIdx.x; i < nb; i += 256) s += M.tailpart[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) M.scal[SC_SCALE] = 1.f / (sqrtf(s) + ns_eps);
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
constexpr int kMvRows = 4;
__global__ __launch_bounds__(256) void k_power_matvec(const DevMat* __restrict__ mats, LaunchList L,
                                                      int steps, int final_pass) {
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (!final_pass && M.ist[IS_PSTEPS] >= steps) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = (local * 4 + w) * kMvRows;
  if (r0 >= M.rows) return;
  const bool vx = aligned16(M.xn, M.cols, M.ns_t);
  float s[kMvRows];
#pragma unroll
  for (int k = 0; k < kMvRows; ++k) s[k] = 0.f;
  for (int c = lane * 8; c < M.cols; c += 512) {
    float v[8];
    load8(M.pv, DT_F32, 0, 0, c, M.cols, true, v);   // pv is 256-byte aligned workspace
#pragma unroll
    for (int k = 0; k < kMvRows; ++k) {
      if (r0 + k < M.rows) {
        float x[8];
        load8(M.xn, M.ns_t, M.cols, r0 + k, c, M.cols, vx, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[k] += x[e] * v[e];
      }
    }
  }
  const float inv = inv_fro(M);
#pragma unroll
  for (int k = 0; k < kMvRows; ++k) {
    const float t = wave_sum(s[k]);
    if (lane == 0 && r0 + k < M.rows) M.pu[r0 + k] = t * inv;
  }
}

// partial w = (X / ||X||)^T u over kRmvRows rows x kStreamCols columns per block.
__global__ __launch_bounds__(256) void k_power_rmatvec(const DevMat* __restrict__ mats, LaunchList L, int steps) {
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  if (M.ist[IS_PSTEPS] >= steps) return;
  const int tr = local / M.n_ct, tc = local % M.n_ct;
  const int c = tc * kStreamCols + threadIdx.x * 8;
  const int r0 = tr * kRmvRows, r1 = min(r0 + kRmvRows, M.rows);
  const bool vx = aligned16(M.xn, M.cols, M.ns_t);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c < M.cols) {
    for (int r = r0; r < r1; ++r) {
      float x[8];
      load8(M.xn, M.ns_t, M.cols, r, c, M.cols, vx, x);
      const float u = M.pu[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += u * x[e];
    }
    const float s = inv_fro(M);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c + e < M.cols) M.pwpart[(size_t)tr * M.cols + c + e] = acc[e] * s;
  }
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
  const int nr = (M.rows + kRmvRows - 1) / kRmvRows;
  float n2 = 0.f;
  for (int c = t; c < M.cols; c += 256) {
    float s = 0.f;
    for (int k = 0; k < nr; ++k) s += M.pwpart[(size_t)k * M.cols + c];
    M.pwpart[c] = s;     // row 0 of the partials now holds w (read back below)
    n2 += s * s;
  }
  n2 = block_sum(n2, red);
  __syncthreads();
  if (n2 > 0.f) {
    const float inv = 1.f / sqrtf(n2);
    for (int c = t; c < M.cols; c += 256) M.pv[c] = M.pwpart[c] * inv;
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
      s = M.colsq[c];
    } else {
      s = 0.f;
      for (int r = 0; r < M.rows; ++r) {
        const size_t idx = (size_t)r * M.cols + c;
        const float x = (M.ns_t == DT_BF16) ? bf2f(((const unsigned short*)M.xn)[idx]) : ((const float*)M.xn)[idx];
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
  for (int c = t; c < M.cols; c += 256) M.pv[c] = (c == j) ? 1.f : 0.f;
}

// sigma = ||X v|| (from u = (X/||X||) v), kappa = (contra/2) / max(sigma, 1e-7).
__global__ __launch_bounds__(256) void k_power_sigma(DevMat* __restrict__ mats, LaunchList L, float contra) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  float s = 0.f;
  for (int r = threadIdx.x; r < M.rows; r += 256) s += M.pu[r] * M.pu[r];
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
// wide/square (ld L_pad), xt[fin] for tall (ld s_pad).
// ---------------------------------------------------------------------------
__device__ __forceinline__ const void* u_ptr(const DevMat& M, int fin, int64_t* ld) {
  if (M.tall) { *ld = M.s_pad; return M.xt[fin]; }
  *ld = M.L_pad; return M.x[fin];
}

// Partial sums per tile: ||U||^2, ||U - kappa X||^2, ||W||^2.
__global__ __launch_bounds__(256) void k_tail_reduce(const DevMat* __restrict__ mats, LaunchList L, int fin) {
  __shared__ float red[3][4];
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int tr = local / M.n_ct, tc = local % M.n_ct;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = tc * kStreamCols + w * kSegCols + lane * 8;
  const int r0 = tr * kStreamRows, r1 = min(r0 + kStreamRows, M.rows);
  int64_t ldu;
  const void* U = u_ptr(M, fin, &ldu);
  const float kappa = M.scal[SC_KAPPA];
  const bool vx = aligned16(M.xn, M.cols, M.ns_t);
  const bool vw = M.w ? aligned16(M.w, M.ld_w, M.dt_w) : false;
  float su = 0.f, sv = 0.f, sw = 0.f;
  if (c < M.cols) {
    for (int r = r0; r < r1; ++r) {
      float u[8], x[8];
      load8(U, M.ns_t, ldu, r, c, M.cols, true, u);
      if (kappa != 0.f) load8(M.xn, M.ns_t, M.cols, r, c, M.cols, vx, x);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        su += u[e] * u[e];
        const float v = u[e] - kappa * x[e];
        sv += v * v;
      }
      if (M.w) {
        float wv[8];
        load8(M.w, M.dt_w, M.ld_w, r, c, M.cols, vw, wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) sw += wv[e] * wv[e];
      }
    }
  }
  su = wave_sum(su); sv = wave_sum(sv); sw = wave_sum(sw);
  if (lane == 0) { red[0][w] = su; red[1][w] = sv; red[2][w] = sw; }
  __syncthreads();
  if (threadIdx.x < 3) {
    const int k = threadIdx.x;
    M.tailpart[(size_t)local * 4 + k] = red[k][0] + red[k][1] + red[k][2] + red[k][3];
  }
}

// alpha = ||U|| / max(||U - kappa X||, 1e-10) * sqrt(max(1, rows/cols)),
// then the u/w-floor: if max(||V||,1e-8) / max(||W||,1e-8) < target, scale up.
__global__ __launch_bounds__(256) void k_tail_finalize(DevMat* __restrict__ mats, LaunchList L, float target_uw) {
  __shared__ float red[8];
  int local;
  DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int nb = M.n_rt * M.n_ct;
  float su = 0.f, sv = 0.f, sw = 0.f;
  for (int i = threadIdx.x; i < nb; i += 256) {
    su += M.tailpart[(size_t)i * 4 + 0];
    sv += M.tailpart[(size_t)i * 4 + 1];
    sw += M.tailpart[(size_t)i * 4 + 2];
  }
  su = block_sum(su, red);
  sv = block_sum(sv, red);
  sw = block_sum(sw, red);
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
__global__ __launch_bounds__(256) void k_tail_apply(const DevMat* __restrict__ mats, LaunchList L, int fin,
                                                    float lr, int copy_only) {
  int local;
  const DevMat& M = mats[find_job(L, blockIdx.x, &local)];
  const int tr = local / M.n_ct, tc = local % M.n_ct;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = tc * kStreamCols + w * kSegCols + lane * 8;
  if (c >= M.cols) return;
  const int r0 = tr * kStreamRows, r1 = min(r0 + kStreamRows, M.rows);
  int64_t ldu;
  const void* U = u_ptr(M, fin, &ldu);
  const float kappa = copy_only ? 0.f : M.scal[SC_KAPPA];
  const float alpha = copy_only ? 1.f : M.scal[SC_ALPHA];
  const bool vx = aligned16(M.xn, M.cols, M.ns_t);
  const bool vw = M.w ? aligned16(M.w, M.ld_w, M.dt_w) : false;
  const bool vo = M.uo ? aligned16(M.uo, M.ld_uo, M.dt_uo) : false;
  for (int r = r0; r < r1; ++r) {
    float u[8], x[8];
    load8(U, M.ns_t, ldu, r, c, M.cols, true, u);
    if (kappa != 0.f) load8(M.xn, M.ns_t, M.cols, r, c, M.cols, vx, x);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = alpha * (u[e] - kappa * x[e]);
    if (M.uo) store8(M.uo, M.dt_uo, M.ld_uo, r, c, M.cols, vo, v);
    if (M.w) {
      float wv[8];
      load8(M.w, M.dt_w, M.ld_w, r, c, M.cols, vw, wv);
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = wv[e] - lr * v[e];
      store8(M.w, M.dt_w, M.ld_w, r, c, M.cols, vw, wv);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (grid sizes come from the planner's LaunchList).
// ---------------------------------------------------------------------------
#define LAUNCH(kern, nblk, ...)                                                            \
  do {                                                                                     \
    if ((nblk) > 0) hipLaunchKernelGGL(kern, dim3(nblk), dim3(256), 0, st, __VA_ARGS__);   \
  } while (0)

hipError_t launch_momentum_stats(const DevMat* m, LaunchList L, int nblk, int nesterov_pass, float mu,
                                 int nesterov, hipStream_t st) {
  LAUNCH(k_momentum_stats, nblk, m, L, nesterov_pass, mu, nesterov);
  return hipGetLastError();
}
hipError_t launch_norms_finalize(DevMat* m, LaunchList L, int nblk, float pp_eps, float ns_eps,
                                 int init_power, hipStream_t st) {
  LAUNCH(k_norms_finalize, nblk, m, L, pp_eps, ns_eps, init_power);
  return hipGetLastError();
}
hipError_t launch_prologue(int ns_t, const DevMat* m, LaunchList L, int nblk, int use_xn, hipStream_t st) {
  if (ns_t == DT_BF16) LAUNCH(k_prologue<__bf16>, nblk, m, L, use_xn);
  else LAUNCH(k_prologue<float>, nblk, m, L, use_xn);
  return hipGetLastError();
}
hipError_t launch_aurora_dupdate(int ns_t, DevMat* m, LaunchList L, int nblk, int fin, float pp_eps,
                                 float pp_beta, hipStream_t st) {
  if (ns_t == DT_BF16) LAUNCH(k_aurora_dupdate<__bf16>, nblk, m, L, fin, pp_eps, pp_beta);
  else LAUNCH(k_aurora_dupdate<float>, nblk, m, L, fin, pp_eps, pp_beta);
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
hipError_t launch_power_normalize(DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st) {
  LAUNCH(k_power_normalize, nblk, m, L, steps);
  return hipGetLastError();
}
hipError_t launch_power_sigma(DevMat* m, LaunchList L, int nblk, float contra, hipStream_t st) {
  LAUNCH(k_power_sigma, nblk, m, L, contra);
  return hipGetLastError();
}
hipError_t launch_tail_reduce(const DevMat* m, LaunchList L, int nblk, int fin, hipStream_t st) {
  LAUNCH(k_tail_reduce, nblk, m, L, fin);
  return hipGetLastError();
}
hipError_t launch_tail_finalize(DevMat* m, LaunchList L, int nblk, float target_uw, hipStream_t st) {
  LAUNCH(k_tail_finalize, nblk, m, L, target_uw);
  return hipGetLastError();
}
hipError_t launch_tail_apply(const DevMat* m, LaunchList L, int nblk, int fin, float lr, int copy_only,
                             hipStream_t st) {
  LAUNCH(k_tail_apply, nblk, m, L, fin, lr, copy_only);
  return hipGetLastError();
}

}  // namespace muon
