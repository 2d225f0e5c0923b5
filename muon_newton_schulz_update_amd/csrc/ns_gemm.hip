// Newton-Schulz matrix-core engine for gfx950.
//
// One iteration of the quintic Newton-Schulz map (Aurora record page,
// www.xxmr.cn/news/295280, section 源码实现: X <- a X + (b A + c A^2) X with
// A = X X^T, X normalised first) is three products, each a launch over every
// matrix of a batch:
//   GM_GRAM  A = X X^T            (s x s, K = L)  upper tiles only, mirrored
//   GM_SQ    B = b A + c A A^T     (s x s, K = s)  upper tiles only, mirrored
//   GM_BX    X' = a X + B X        (s x L, K = s)
// The Gram and A^2 read both operands with the reduction index contiguous
// (C[m][n] = sum_k P[m][k] Q[n][k]). For bf16, BX reads X itself (row-major,
// k = row): its operand fragments come from LDS through gfx950's transposing
// LDS reads, the a X term is added from the LDS stage that already holds
// those rows, and X'^T is written only on a pass's last iteration (where the
// preconditioner update and the output need it). fp32 keeps a transposed
// copy X^T every iteration and reads it like the other two products.
//
// Tiling: 256 x 256 output tile per workgroup; default 512 threads (8 waves
// in 4 x 2, each wave 64 x 128 = 2 x 4 MFMA 32x32 blocks, accumulators in
// AGPRs, two waves per SIMD); a 4-wave layout (2 x 2 waves of 128 x 128) is
// kept for tuning. K advances 64 bf16 (32 fp32) per stage; two LDS stages of
// 64 KB are filled by direct global->LDS 16-byte loads, so the next stage
// streams in while the current one feeds the matrix cores. LDS rows are
// XOR-swizzled in 16-byte chunks to spread the fragment reads over the banks.
// bf16 runs v_mfma_f32_32x32x16_bf16 (fp32 accumulation); fp32 runs
// v_mfma_f32_32x32x2f32 on the same tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "muon_device.hpp"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

namespace {

constexpr int kRowBytes = 128;                 // bytes of K per tile row per stage (K-contiguous operand)
constexpr int kStageA = kTile * kRowBytes;     // 32 KB
constexpr int kStageBytes = 2 * kStageA;       // A + B operand = 64 KB
constexpr int kNNRowBytes = kTile * 2;         // one k-row of a 256-wide bf16 X panel: 512 B
constexpr int kPitch = 132;                    // floats per staged epilogue row (128 + 4 spreads banks)
constexpr int kSlabBytes = 32 * kPitch * 4;    // one wave's 32 x 128 staging slab (NI*32 <= 128)
constexpr int kLdsBytes = 8 * kSlabBytes > 2 * kStageBytes ? 8 * kSlabBytes : 2 * kStageBytes;

// 16-byte chunk position of logical chunk c of a K-contiguous tile row r.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }
// 16-byte chunk position of logical chunk c (0..31) of X panel row k: four
// consecutive rows land on four different quarters of the banks.
__device__ __forceinline__ int swz_nn(int k, int c) { return c ^ ((k & 3) << 2); }

// Read one accumulator through an explicit AGPR->VGPR move. The "a"
// constraint keeps the accumulators allocated in AGPRs for their whole live
// range (plain uses in the epilogue would pull them into VGPRs).
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

__device__ __forceinline__ void wait_vm_all() {
  // s_waitcnt vmcnt(0): every direct-to-LDS load of this wave has landed.
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ unsigned short f2bf(float f) {
  // round to nearest even (inputs here are finite)
  unsigned int u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}
__device__ __forceinline__ float bf2f(unsigned short h) {
  return __uint_as_float(((unsigned int)h) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<__bf16> {
  static constexpr int kPerChunk = 8;          // bf16 per 16-byte chunk
  typedef bf16x8_t Frag;                       // one MFMA operand per lane
  __device__ static void ld8(const void* p, size_t i, float v[8]) {
    const u16x8_t q = *(const u16x8_t*)((const unsigned short*)p + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf2f(q[e]);
  }
  __device__ static void st8(void* p, size_t i, const float v[8]) {
    u16x8_t q;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = f2bf(v[e]);
    *(u16x8_t*)((unsigned short*)p + i) = q;
  }
};
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  typedef f32x4_t Frag;                        // four MFMA operands (4 consecutive k) per lane
  __device__ static void ld8(const void* p, size_t i, float v[8]) {
    const f32x4_t a = *(const f32x4_t*)((const float*)p + i), b = *(const f32x4_t*)((const float*)p + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
  }
  __device__ static void st8(void* p, size_t i, const float v[8]) {
    *(f32x4_t*)((float*)p + i) = (f32x4_t){v[0], v[1], v[2], v[3]};
    *(f32x4_t*)((float*)p + i + 4) = (f32x4_t){v[4], v[5], v[6], v[7]};
  }
};

// Direct-to-LDS loads of one operand stage. One wave instruction fills 1 KB;
// with NW waves, wave w's instruction i fills the 1 KB group g = NW i + w and
// lane p fetches the chunk that belongs at LDS position p of it. The swizzle
// of a lane's row does not depend on i, so a lane needs one 32-bit byte
// offset (`lane_off`); the per-instruction step (`rstep`) and the K position
// (`kb`) are uniform.
//   K-contiguous operand: 8 tile rows of 128 B per group;
//   X panel (NN): 2 k-rows of 512 B per group.
template <int NW>
__device__ __forceinline__ void issue_operand(uint8_t* sm, const uint8_t* src, int64_t rstep, int64_t kb,
                                              uint32_t lane_off, int wave) {
#pragma unroll
  for (int i = 0; i < 32 / NW; ++i) {
    const int g = i * NW + wave;
    __builtin_amdgcn_global_load_lds((const void*)(src + kb + i * rstep + lane_off), LDS_PTR(sm + g * 1024), 16,
                                     0, 0);
  }
}

// Fragment reads of a K-contiguous operand: lane l reads tile row
// (base + l%32), logical chunk 2j + l/32 (8 bf16 or 4 fp32 consecutive k).
// Bases are multiples of 32 rows, so the swizzle term depends on l only.
template <typename T, int N>
__device__ __forceinline__ void read_kc(const uint8_t* base, int j, int lane, typename Elem<T>::Frag (&f)[N]) {
  const int lr = lane & 31;
  const int ph = ((2 * j + (lane >> 5)) ^ ((lr >> 1) & 7)) * 16;
#pragma unroll
  for (int i = 0; i < N; ++i) f[i] = *(const typename Elem<T>::Frag*)(base + (i * 32 + lr) * kRowBytes + ph);
}

// Transposing LDS read of 4 bf16 from an X panel stage (k-rows of 512 B).
// Within each 16-lane group, lane i receives element e (e = 0..3) from the
// 8 bytes addressed by lane 4e + i/4 of its group, half-word i%4 (measured
// on gfx950). With the lane coordinates of tr_coords, lane l receives
// X[k0 + e][n0 + l%32].
__device__ __forceinline__ i16x4_t read_tr(const uint8_t* stage, int k, int n) {
  const uint8_t* p = stage + k * kNNRowBytes + swz_nn(k, n >> 3) * 16 + (n & 7) * 2;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p);
}

// Address of lane l's 8 bytes for read_tr so that lane l receives
// X[k0 + e][n0 + l%32]; k0 is the lane's own row base (it may differ
// between the two lane halves).
__device__ __forceinline__ void tr_coords(int lane, int k0, int n0, int& k, int& n) {
  const int i = lane & 15, grp = lane >> 4;
  k = k0 + (i >> 2);
  n = n0 + 16 * (grp & 1) + 4 * (i & 3);
}

}  // namespace

// Launch geometry: grid.x = 8 * per_xcd blocks; the hardware deals
// consecutive workgroups round-robin to the 8 XCDs, so block b runs on XCD
// b % 8. Items are dealt to XCDs in runs of `group` consecutive items (one
// super-tile of the planner's raster, whose tiles share operand panels), so a
// run executes together on one XCD and reuses its L2.
template <typename T, int mode, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, 1) void k_ns_gemm(const DevMat* __restrict__ mats,
                                                             const TileItem* __restrict__ items,
                                                             int n_items, int group, int cur, int write_t_bx,
                                                             float ca, float cb, float cc) {
  // two 64 KB operand stages; after the K loop the same memory stages the
  // epilogue (one 32 x (NI*32) float slab per wave, at most 132 KB)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  uint8_t* const sm0 = smem;
  uint8_t* const sm1 = smem + kStageBytes;
  constexpr bool NN = (mode == GM_BX) && (sizeof(T) == 2);   // BX reading X itself

  const int b = blockIdx.x;
  const int xcd = b & 7, j = b >> 3;
  const int item_idx = ((j / group) * 8 + xcd) * group + (j % group);
  if (item_idx >= n_items) return;
  const TileItem it = items[item_idx];
  const DevMat& M = mats[it.mat];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS bases stay in SGPRs
  constexpr int NW = WM * WN;                // waves per workgroup
  constexpr int MI = kTile / WM / 32;        // 32x32 blocks per wave, down
  constexpr int NI = kTile / WN / 32;        // 32x32 blocks per wave, across
  const int wm = wave / WN, wn = wave % WN;
  const int sp = M.s_pad, Lp = M.L_pad;

  const T *P, *Q;
  int ld, K;
  if constexpr (mode == GM_GRAM) {
    const T* x = (const T*)M.x[cur];
    P = x + (size_t)it.tm * kTile * Lp;
    Q = x + (size_t)it.tn * kTile * Lp;
    ld = Lp; K = Lp;
  } else if constexpr (mode == GM_SQ) {
    const T* a = (const T*)M.a;
    P = a + (size_t)it.tm * kTile * sp;
    Q = a + (size_t)it.tn * kTile * sp;
    ld = sp; K = sp;
  } else if constexpr (NN) {
    P = (const T*)M.b + (size_t)it.tm * kTile * sp;
    Q = (const T*)M.x[cur] + (size_t)it.tn * kTile;           // X rows k, this tile's columns
    ld = sp; K = sp;
  } else {
    P = (const T*)M.b + (size_t)it.tm * kTile * sp;
    Q = (const T*)M.xt[cur] + (size_t)it.tn * kTile * sp;
    ld = sp; K = sp;
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = (f32x16_t){};

  constexpr int KE = kRowBytes / sizeof(T);   // K elements per stage
  const int nk = K / KE;                      // K is a multiple of 256: nk is even
  // P (and Q unless NN): K-contiguous rows, 8 rows per 1 KB group
  const int lrow = wave * 8 + (lane >> 3);
  const uint32_t off_p = (uint32_t)(((int64_t)lrow * ld + swz(lrow, lane & 7) * Elem<T>::kPerChunk) * sizeof(T));
  const int64_t rstep_p = (int64_t)NW * 8 * ld * sizeof(T);
  // Q in NN form: 2 k-rows of 512 B per 1 KB group; a stage holds KE k-rows.
  // A lane's row within the stage is 2 g + lane/32, whose swizzle (row & 3)
  // does not depend on the instruction index (g steps by NW).
  const int qk = 2 * wave + (lane >> 5);
  const uint32_t off_q = NN ? (uint32_t)(((int64_t)qk * Lp + swz_nn(qk, lane & 31) * 8) * 2) : off_p;
  const int64_t rstep_q = NN ? (int64_t)NW * 2 * Lp * 2 : rstep_p;
  const int64_t kstep_q = NN ? (int64_t)KE * Lp * 2 : kRowBytes;
  const uint8_t* Pb = (const uint8_t*)P;
  const uint8_t* Qb = (const uint8_t*)Q;

  auto issue = [&](uint8_t* sm, int ks) {
    issue_operand<NW>(sm, Pb, rstep_p, (int64_t)ks * kRowBytes, off_p, wave);
    issue_operand<NW>(sm + kStageA, Qb, rstep_q, (int64_t)ks * kstep_q, off_q, wave);
  };

  auto compute = [&](const uint8_t* sm) {
    const uint8_t* pa = sm + wm * MI * 32 * kRowBytes;
    const uint8_t* qa = sm + kStageA + wn * NI * 32 * kRowBytes;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      typename Elem<T>::Frag fp[MI], fq[NI];
      read_kc<T, MI>(pa, jj, lane, fp);
      if constexpr (NN) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          int kr, nc;
          tr_coords(lane, 16 * jj + 8 * (lane >> 5), wn * NI * 32 + ni * 32, kr, nc);
          const i16x4_t lo = read_tr(sm + kStageA, kr, nc);       // k = 16jj + 8(l/32) + 0..3
          const i16x4_t hi = read_tr(sm + kStageA, kr + 4, nc);   // k = 16jj + 8(l/32) + 4..7
          fq[ni] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      } else {
        read_kc<T, NI>(qa, jj, lane, fq);
      }
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp[mi], fq[ni], acc[mi][ni], 0, 0, 0);
      } else {
        // the 4 floats of a chunk are 4 consecutive k; lanes 0-31 and 32-63
        // supply the two k slots of each 32x32x2 step from chunks 2j and 2j+1
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(fp[mi][e], fq[ni][e], acc[mi][ni], 0, 0, 0);
      }
    }
  };

  // a X for NN: the stages holding k-rows [tm*256 + wm*MI*32, +MI*32) hold
  // exactly this wave's output rows of X, so a X is added from LDS as one
  // more product: acc += (a I) X over those k, with the identity split as
  // a = a_hi + a_lo in two bf16 operands (a_lo = 0 for a = 2), so the
  // accumulators are only ever touched by MFMAs.
  const int ks_ax0 = NN ? (it.tm * kTile + wm * MI * 32) / KE : 0;
  const int ks_ax1 = NN ? ks_ax0 + (MI * 32 + KE - 1) / KE : 0;
  const unsigned short a_hi = f2bf(ca);
  const unsigned short a_lo = f2bf(ca - bf2f(a_hi));
  auto add_ax = [&](const uint8_t* sm, int ks) {
    if constexpr (NN) {
      const int stage_r0 = ks * KE - it.tm * kTile;   // tile-local row of the stage's first k-row
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r0 = wm * MI * 32 + mi * 32 - stage_r0;   // stage-local first row of block mi
        if (r0 < 0 || r0 >= KE) continue;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int jj = (r0 >> 4) + h2;
          typename Elem<T>::Frag fq[NI];
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            int kr, nc;
            tr_coords(lane, 16 * jj + 8 * (lane >> 5), wn * NI * 32 + ni * 32, kr, nc);
            const i16x4_t lo = read_tr(sm + kStageA, kr, nc);
            const i16x4_t hi = read_tr(sm + kStageA, kr + 4, nc);
            fq[ni] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
          // identity operand: row r0 + lane%32, k = 16 jj + 8 (lane/32) + t
          u16x8_t ih, il;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const bool diag = (r0 + (lane & 31)) == (16 * jj + 8 * (lane >> 5) + t);
            ih[t] = diag ? a_hi : (unsigned short)0;
            il[t] = diag ? a_lo : (unsigned short)0;
          }
          const bf16x8_t fih = __builtin_bit_cast(bf16x8_t, ih), fil = __builtin_bit_cast(bf16x8_t, il);
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fih, fq[ni], acc[mi][ni], 0, 0, 0);
            if (a_lo != 0) acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fil, fq[ni], acc[mi][ni], 0, 0, 0);
          }
        }
      }
    }
  };

  issue(sm0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    wait_vm_all();
    __syncthreads();
    issue(sm1, kt + 1);
    compute(sm0);
    if (NN && kt >= ks_ax0 && kt < ks_ax1) add_ax(sm0, kt);
    wait_vm_all();
    __syncthreads();
    if (kt + 2 < nk) issue(sm0, kt + 2);
    compute(sm1);
    if (NN && kt + 1 >= ks_ax0 && kt + 1 < ks_ax1) add_ax(sm1, kt + 1);
  }

  // Epilogue. Accumulator register r of 32x32 block (mi, ni) holds
  // row 8*(r/4) + 4*(lane/32) + r%4, column lane%32 of that block. Each wave
  // stages one 32-row slab of its tile at a time in the now idle LDS, then
  // writes it row-major (8 consecutive columns per lane) and, for mirrored
  // and X'^T outputs, transposed (8 consecutive rows per lane).
  const int row0 = it.tm * kTile + wm * MI * 32;
  const int col0 = it.tn * kTile + wn * NI * 32;
  void* out;
  void* outT;
  const void* add;
  float add_coef, acc_coef;
  int ldo, ldt;
  if constexpr (mode == GM_GRAM) {
    out = M.a; outT = M.a; add = nullptr; add_coef = 0.f; acc_coef = 1.f; ldo = sp; ldt = sp;
  } else if constexpr (mode == GM_SQ) {
    out = M.b; outT = M.b; add = M.a; add_coef = cb; acc_coef = cc; ldo = sp; ldt = sp;
  } else {
    out = M.x[cur ^ 1]; outT = M.xt[cur ^ 1]; add = M.x[cur]; add_coef = ca; acc_coef = 1.f;
    ldo = Lp; ldt = sp;
  }
  const bool write_t = (mode == GM_BX) ? (write_t_bx != 0) : (it.tm != it.tn);
  float* buf = (float*)(smem + wave * kSlabBytes);
  __syncthreads();   // every wave is done reading the operand stages
  constexpr int SC = NI * 32;                // staged slab: 32 rows x SC columns
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        buf[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kPitch + ni * 32 + (lane & 31)] = agpr_read(acc[mi][ni][r]);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SC / 16; ++k) {
      const int q = k * 64 + lane;
      const int rr = q / (SC / 8), c8 = (q % (SC / 8)) * 8;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = acc_coef * buf[rr * kPitch + c8 + e];
      const size_t idx = (size_t)(row0 + mi * 32 + rr) * ldo + col0 + c8;
      if constexpr (mode == GM_SQ || (mode == GM_BX && !NN)) {
        float av[8];
        Elem<T>::ld8(add, idx, av);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += add_coef * av[e];
      }
      Elem<T>::st8(out, idx, v);
      if (write_t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) buf[rr * kPitch + c8 + e] = v[e];
      }
    }
    __syncthreads();
    if (write_t) {
#pragma unroll
      for (int k = 0; k < SC / 16; ++k) {
        const int q = k * 64 + lane;
        const int c1 = q >> 2, rc = (q & 3) * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = buf[(rc + e) * kPitch + c1];
        Elem<T>::st8(outT, (size_t)(col0 + c1) * ldt + row0 + mi * 32 + rc, v);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Host-side launcher.
// ---------------------------------------------------------------------------
// variant 0: 8 waves in 4 x 2 (64 x 128 per wave, two waves per SIMD);
// variant 1: 4 waves in 2 x 2 (128 x 128 per wave, one wave per SIMD).
// write_t: for BX, also write X'^T (always done for fp32, whose BX reads it).
hipError_t launch_ns_gemm(int ns_t, const DevMat* mats, const TileItem* items, int n_items,
                          int mode, int cur, int write_t, float ca, float cb, float cc, int variant,
                          hipStream_t st) {
  if (n_items <= 0) return hipSuccess;
  const int group = 32;   // one super-tile of the planner's raster per XCD wave
  const int per_xcd_groups = (n_items + 8 * group - 1) / (8 * group);
  const dim3 grid(per_xcd_groups * group * 8);
  if (ns_t != DT_BF16) write_t = 1;
#define NS_LAUNCH(T, MODE, WM, WN) \
  hipLaunchKernelGGL((k_ns_gemm<T, MODE, WM, WN>), grid, dim3(WM * WN * 64), 0, st, mats, items, n_items, group, \
                     cur, write_t, ca, cb, cc)
#define NS_MODES(T, WM, WN)                          \
  do {                                               \
    if (mode == GM_GRAM) NS_LAUNCH(T, GM_GRAM, WM, WN); \
    else if (mode == GM_SQ) NS_LAUNCH(T, GM_SQ, WM, WN); \
    else NS_LAUNCH(T, GM_BX, WM, WN);                \
  } while (0)
  if (ns_t == DT_BF16) {
    if (variant == 1) NS_MODES(__bf16, 2, 2);
    else NS_MODES(__bf16, 4, 2);
  } else {
    if (variant == 1) NS_MODES(float, 2, 2);
    else NS_MODES(float, 4, 2);
  }
#undef NS_MODES
#undef NS_LAUNCH
  return hipGetLastError();
}

}  // namespace muon
