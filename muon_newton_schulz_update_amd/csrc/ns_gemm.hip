// Newton-Schulz matrix-core engine for gfx950.
//
// One iteration of the quintic Newton-Schulz map (Aurora record page,
// www.xxmr.cn/news/295280, section 源码实现: X <- a X + (b A + c A^2) X with
// A = X X^T, X normalised first) is three products, each a launch over every
// matrix of a batch:
//   GM_GRAM  A  = X X^T                  (s x s, K = L)  upper tiles only, mirrored
//   GM_SQ    B' = b A + c A A^T + a I     (s x s, K = s)  upper tiles only, mirrored
//   GM_BX    X' = B' X                   (s x L, K = s)  writes X' and X'^T
// (B' X equals a X + (b A + c A^2) X; adding a on the diagonal of B in the
// second product's epilogue turns the third into a plain product.) X^T is
// kept beside X, written by the third product's epilogue, so all three read
// both operands with the reduction index contiguous:
// C[m][n] = sum_k P[m][k] Q[n][k].
//
// Tiling: 256 x 256 output tile per workgroup. Default layout: 8 waves in
// 4 x 2, each wave 64 x 128 (2 x 4 MFMA 32x32 blocks, accumulators in
// AGPRs, two waves per SIMD, so one wave's matrix-core work covers the other
// wave's stalls on the in-order issue of memory instructions); a 4-wave
// layout (2 x 2 waves of 128 x 128) is kept for tuning. Launches with few
// tiles use 128 x 128 tiles (2 x 2 waves of 64 x 64, half the LDS, two
// workgroups per CU), which spread them over the CUs in finer steps.
//
// K advances 128 bytes per tile row per stage (64 bf16 or 32 fp32), so each
// direct-load request covers whole 128-byte lines. The LDS holds five
// operand slots (32 KB each for 256-tiles), filled by buffer-form direct
// global->LDS loads (they count on vmcnt only, so waits on LDS fragment reads
// do not also wait for them);
// stage k's two operands occupy slots 2k and 2k+1 (mod 5), so while one
// stage feeds the matrix cores the next stage and half of the one after
// stream in. A stage is four k-steps; each step's fragments are read between
// the previous step's MFMAs. The workgroup barrier sits before the last step,
// so matrix-core work continues across it, and the refill of the two freed
// slots and the next stage's first fragments are issued between that last
// step's MFMAs. LDS rows are XOR-swizzled in 16-byte chunks so fragment reads
// are conflict-free.
// bf16 runs v_mfma_f32_32x32x16_bf16 (fp32 accumulation); fp32 runs
// v_mfma_f32_32x32x2f32 on the same tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_device.hpp"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

namespace {

constexpr int kRowBytes = 128;                 // K bytes per tile row per stage
constexpr int kPitch = 132;                    // floats per staged epilogue row (widest slab 128, + 4 spreads banks)
constexpr int kSlabBytes = 32 * kPitch * 4;    // one wave's 32 x 128 staging slab

// Read one accumulator through an explicit AGPR->VGPR move. The "a"
// constraint keeps the accumulators allocated in AGPRs for their whole live
// range (plain uses in the epilogue would pull them into VGPRs).
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// s_waitcnt vmcnt(n), lgkmcnt and expcnt left free: all but this wave's n
// most recent vector-memory operations have completed (the counter retires
// them in issue order; in the K loop every such operation is a stage load).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt immediate");   // 6 bits: [3:0] and [15:14]
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}
// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier the compiler does not treat as one: before a known
// barrier it would wait for every in-flight direct-to-LDS load, draining the
// ring. Every wait it needs is explicit before it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Hand-off through LDS between the lanes of one wave: the LDS executes a
// wave's accesses in order, so only the compiler has to be kept from moving
// this wave's reads and writes of its slab across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
  typedef u16x8_t Raw;                         // 8 elements as loaded
  __device__ static Raw ldraw(const void* p, size_t i) { return *(const u16x8_t*)((const unsigned short*)p + i); }
  __device__ static void cvt(const Raw& q, float v[8]) {
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
  struct Raw {
    f32x4_t a, b;
  };
  __device__ static Raw ldraw(const void* p, size_t i) {
    Raw q;
    q.a = *(const f32x4_t*)((const float*)p + i);
    q.b = *(const f32x4_t*)((const float*)p + i + 4);
    return q;
  }
  __device__ static void cvt(const Raw& q, float v[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = q.a[e]; v[e + 4] = q.b[e]; }
  }
  __device__ static void st8(void* p, size_t i, const float v[8]) {
    *(f32x4_t*)((float*)p + i) = (f32x4_t){v[0], v[1], v[2], v[3]};
    *(f32x4_t*)((float*)p + i + 4) = (f32x4_t){v[4], v[5], v[6], v[7]};
  }
};

}  // namespace

// Launch geometry: grid.x = 8 * per_xcd blocks; the hardware deals
// consecutive workgroups round-robin to the 8 XCDs, so block b runs on XCD
// b % 8. Items are dealt to XCDs in runs of `group` consecutive items (one
// super-tile of the planner's raster, whose tiles share operand panels), so a
// run executes together on one XCD and reuses its L2.
template <typename T, int mode, int S, int WM, int WN, int TILE>
__global__ __launch_bounds__(WM * WN * 64, TILE == 256 ? 1 : 2) void k_ns_gemm(const DevMat* __restrict__ mats,
                                                             const TileItem* __restrict__ items, int n_items,
                                                             int group, int cur, float ca, float cb, float cc) {
  constexpr int NW = WM * WN;                // waves per workgroup
  constexpr int MI = TILE / WM / 32;         // 32x32 blocks per wave, down
  constexpr int NI = TILE / WN / 32;         // 32x32 blocks per wave, across
  constexpr int kOpBytes = TILE * kRowBytes; // one operand of one stage (one LDS slot)
  constexpr int LPO = TILE / 8 / NW;         // direct loads per wave per operand per stage
  constexpr int kMfmaStep = MI * NI * (sizeof(T) == 2 ? 1 : 4);   // MFMAs per k-step
  constexpr int kReadStep = MI + NI;                              // LDS reads per k-step
  // S operand slots; after the K loop the same memory stages the epilogue
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * kOpBytes];
  static_assert(S * kOpBytes >= NW * kSlabBytes, "epilogue staging fits in the slots");
  static_assert(S >= 4 && (S - 2) * LPO < 64, "slot count");

  const int b = blockIdx.x;
  const int xcd = b & 7, j = b >> 3;
  const int item_idx = ((j / group) * 8 + xcd) * group + (j % group);
  if (item_idx >= n_items) return;
  const TileItem it = items[item_idx];
  const DevMat& M = mats[it.mat];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS bases stay in SGPRs
  const int wm = wave / WN, wn = wave % WN;
  const int sp = M.s_pad, Lp = M.L_pad;

  const T *P, *Q;
  int ld, K;
  if constexpr (mode == GM_GRAM) {
    const T* x = (const T*)M.x[cur];
    P = x + (size_t)it.tm * TILE * Lp;
    Q = x + (size_t)it.tn * TILE * Lp;
    ld = Lp; K = Lp;
  } else if constexpr (mode == GM_SQ) {
    const T* a = (const T*)M.a;
    P = a + (size_t)it.tm * TILE * sp;
    Q = a + (size_t)it.tn * TILE * sp;
    ld = sp; K = sp;
  } else {
    P = (const T*)M.b + (size_t)it.tm * TILE * sp;
    Q = (const T*)M.xt[cur] + (size_t)it.tn * TILE * sp;
    ld = sp; K = sp;
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = (f32x16_t){};

  constexpr int KE = kRowBytes / sizeof(T);   // K elements per stage
  const int nk = K / KE;                      // K is a multiple of 256: nk >= 4
  constexpr int CPR = Elem<T>::kPerChunk;
  // Direct loads: one wave instruction fills one 1 KB group of 8 tile rows;
  // wave w's load i fills group g = NW i + w, lane p fetching row 8 g + p/8,
  // physical chunk p%8 of it. Physical chunk c' of row r holds logical chunk
  // c' ^ ((r >> 1) & 7); for these rows that term is (4 w + p/16) % 8, so a
  // lane needs one 32-bit byte offset for the whole K loop.
  const int prow = 8 * wave + (lane >> 3);
  const uint32_t lane_off = (uint32_t)(((int64_t)prow * ld + ((lane & 7) ^ ((prow >> 1) & 7)) * CPR) * sizeof(T));
  const int rstep = (int)((int64_t)8 * NW * ld * sizeof(T));
  // Buffer resources over the two operand panels. Every read stays inside
  // its panel: the K offset travels in the scalar offset and stages past the
  // end of K are clamped. On a diagonal tile of the two symmetric products
  // both operands are the same panel: the second resource gets no records,
  // and since the range check compares the per-lane offset with the record
  // count, each of its loads fails the check and fetches nothing (the issue
  // count, and with it every wait, stays the same); both operands' fragments
  // are read from the first panel's slot.
  const int ext = (int)((int64_t)TILE * ld * sizeof(T));
  const bool same = (mode != GM_BX) && (it.tm == it.tn);
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc((void*)P, (short)0, ext, 0x00020000);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)Q, (short)0, same ? 0 : ext, 0x00020000);

  // Operand stage o is P (o even) or Q (o odd) of stage o/2; it goes to
  // slot o % S. Stages past the end of K are clamped to the last one: an
  // L2-resident re-read into a slot nobody reads again, which keeps every
  // wait below the same.
  auto issue = [&](int slot, int o) {
    const int ks = min(o >> 1, nk - 1);
    uint8_t* sm = smem + slot * kOpBytes;
#pragma unroll
    for (int i = 0; i < LPO; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds((o & 1) ? rq : rp, LDS_PTR(sm + (NW * i + wave) * 1024), 16,
                                               lane_off, ks * kRowBytes + i * rstep, 0, 0);
  };

  // Fragments: lane l reads tile row (block base + l%32), logical chunk
  // 2 s + l/32 of the stage (8 bf16 or 4 fp32 consecutive k) for k-step s.
  typedef typename Elem<T>::Frag Frag;
  Frag fa[2][MI], fb[2][NI];
  const int lr = lane & 31;
  auto read_frags = [&](int pslot, int qslot, int s, int buf) {
    const uint8_t* sa = smem + pslot * kOpBytes;
    const uint8_t* sb = same ? sa : smem + qslot * kOpBytes;
    const int ph = ((2 * s + (lane >> 5)) ^ ((lr >> 1) & 7)) * 16;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      fa[buf][mi] = *(const Frag*)(sa + (wm * MI * 32 + mi * 32 + lr) * kRowBytes + ph);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      fb[buf][ni] = *(const Frag*)(sb + (wn * NI * 32 + ni * 32 + lr) * kRowBytes + ph);
  };
  auto mfmas = [&](int buf) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][mi], fb[buf][ni], acc[mi][ni], 0, 0, 0);
    } else {
      // the 4 floats of a chunk are 4 consecutive k; lanes 0-31 and 32-63
      // supply the two k slots of each 32x32x2 step
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[buf][mi][e], fb[buf][ni][e], acc[mi][ni], 0, 0, 0);
    }
  };
  // Spread nmem memory instructions evenly between one k-step's MFMAs, the
  // first nloads of them direct loads, the rest LDS reads. The compiler
  // cannot tell the refill and the reads apart, so the pattern keeps their
  // program order.
  auto spread = [&](int nmem, int nloads) {
#pragma unroll
    for (int q = 0; q < kMfmaStep; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
#pragma unroll
      for (int t = q * nmem / kMfmaStep; t < (q + 1) * nmem / kMfmaStep; ++t) {
        if (t < nloads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one direct load
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // one LDS read
      }
    }
  };

  // Prologue: fill every slot, wait for stage 0, read its first k-step.
#pragma unroll
  for (int o = 0; o < S; ++o) issue(o, o);
  wait_vm<(S - 2) * LPO>();
  ring_barrier();
  read_frags(0, 1, 0, 0);
  // slots of stage k (ps, qs) and of stage k+1 (pn, qn)
  int ps = 0, qs = 1, pn = 2 % S, qn = 3 % S;
  for (int k = 0; k < nk - 1; ++k) {
    // k-steps 0-2, each with the next k-step's fragments read between its MFMAs
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      read_frags(ps, qs, s + 1, (s + 1) & 1);
      mfmas(s & 1);
      spread(kReadStep, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // stage k+1 has landed for every wave (only the S - 4 most recent
    // operand stages may be in flight); stage k's slots are free
    wait_lgkm0();
    wait_vm<(S - 4) * LPO>();
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 3: the refill of the freed slots with operand stages 2k+S and
    // 2k+S+1 (longest latency first), then the next stage's first fragments.
    // With 256-tiles it runs at raised wave priority: a wave still in it
    // outranks the waves of its SIMD that have moved on to the next stage, so
    // the waves reach the next barrier closer together (1-1.2 % faster on the
    // 3072-row products). 128-tiles, two workgroups per CU, keep the default.
    if constexpr (TILE == 256) __builtin_amdgcn_s_setprio(2);
    __builtin_amdgcn_sched_barrier(0);
    issue(ps, 2 * k + S);
    issue(qs, 2 * k + S + 1);
    read_frags(pn, qn, 0, 0);
    mfmas(1);
    spread(2 * LPO + kReadStep, 2 * LPO);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TILE == 256) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    ps = pn; qs = qn;
    pn = (pn + 2 >= S) ? pn + 2 - S : pn + 2;
    qn = (qn + 2 >= S) ? qn + 2 - S : qn + 2;
  }
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    read_frags(ps, qs, s + 1, (s + 1) & 1);
    mfmas(s & 1);
  }
  mfmas(1);
  wait_vm<0>();
  // Keep every MFMA above this point and give the last ones time to write
  // their accumulators before the epilogue reads them through inline asm
  // (the compiler inserts no wait states for reads it cannot see).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // Epilogue. Accumulator register r of 32x32 block (mi, ni) holds
  // row 8*(r/4) + 4*(lane/32) + r%4, column lane%32 of that block. Each wave
  // stages its accumulators in its own part of the now idle LDS and writes
  // them row-major (8 consecutive columns per lane) and, for mirrored and
  // X'^T outputs, transposed (8 consecutive rows per lane): bf16 Gram and X'
  // tiles in one pass (below), the second product and fp32 tiles one 32-row
  // fp32 slab at a time.
  const int row0 = it.tm * TILE + wm * MI * 32;
  const int col0 = it.tn * TILE + wn * NI * 32;
  void* out;
  void* outT;
  int ldo, ldt;
  if constexpr (mode == GM_GRAM) {
    out = M.a; outT = M.a; ldo = sp; ldt = sp;
  } else if constexpr (mode == GM_SQ) {
    out = M.b; outT = M.b; ldo = sp; ldt = sp;
  } else {
    out = M.x[cur ^ 1]; outT = M.xt[cur ^ 1]; ldo = Lp; ldt = sp;
  }
  const bool write_t = (mode == GM_BX) || (it.tm != it.tn);
  __syncthreads();   // every wave is done with the slots
  if constexpr (sizeof(T) == 2 && mode != GM_SQ) {
    // bf16 outputs that are the accumulators rounded: each wave stages its
    // whole (MI*32) x (NI*32) tile at once, rounded, column-major (a column's
    // rows contiguous), so a lane's four consecutive-row accumulators go in
    // one 8-byte write and a column's rows leave in one 16-byte read; the
    // row-major output gathers 2-byte elements. Rows are held in 8-row
    // chunks, chunk index XOR-ed with f(col) = (col ^ col/8) % 8, which keeps
    // all three access patterns off repeated LDS banks.
    constexpr int TR = MI * 32, TC = NI * 32;   // the wave's tile
    static_assert(NW * TR * TC * 2 <= S * kOpBytes, "bf16 staging fits in the slots");
    unsigned short* st = (unsigned short*)(smem + wave * (TR * TC * 2));
    auto sidx = [](int row, int col) {           // element index of (row, col) in the staged tile
      return col * TR + ((((row >> 3) ^ col ^ (col >> 3)) & 7) | ((row >> 3) & ~7)) * 8 + (row & 7);
    };
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = ni * 32 + (lane & 31);
          const int row = mi * 32 + 8 * g + 4 * (lane >> 5);   // rows row..row+3: registers 4g..4g+3
          const unsigned int lo = (unsigned int)f2bf(agpr_read(acc[mi][ni][4 * g])) |
                                  ((unsigned int)f2bf(agpr_read(acc[mi][ni][4 * g + 1])) << 16);
          const unsigned int hi = (unsigned int)f2bf(agpr_read(acc[mi][ni][4 * g + 2])) |
                                  ((unsigned int)f2bf(agpr_read(acc[mi][ni][4 * g + 3])) << 16);
          *(u32x2_t*)(st + sidx(row, col)) = (u32x2_t){lo, hi};
        }
    wave_lds_sync();
    // row-major: 8 consecutive columns of one row per lane
#pragma unroll
    for (int kk = 0; kk < TR * TC / 8 / 64; ++kk) {
      const int q = kk * 64 + lane;
      const int r = q / (TC / 8), c8 = (q % (TC / 8)) * 8;
      u16x8_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = st[sidx(r, c8 + e)];
      *(u16x8_t*)((unsigned short*)out + (size_t)(row0 + r) * ldo + col0 + c8) = v;
    }
    if (write_t) {
      // transposed: 8 consecutive rows of one column per lane, a column's
      // TR rows (a whole number of 128-byte lines) by consecutive lanes
#pragma unroll
      for (int kk = 0; kk < TR * TC / 8 / 64; ++kk) {
        const int q = kk * 64 + lane;
        const int c = q / (TR / 8), r8 = (q % (TR / 8)) * 8;
        const u16x8_t v = *(const u16x8_t*)(st + sidx(r8, c));
        *(u16x8_t*)((unsigned short*)outT + (size_t)(col0 + c) * ldt + row0 + r8) = v;
      }
    }
    return;
  }
  // 32-row fp32 slabs; the second product's A values for a slab are loaded
  // before the slab is staged, so their latency overlaps the staging
  float* buf = (float*)(smem + wave * kSlabBytes);
  constexpr int SC = NI * 32;                // staged slab: 32 rows x SC columns
  constexpr int KK = SC / 16;                // 8-column chunks per lane per slab
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    typename Elem<T>::Raw araw[mode == GM_SQ ? KK : 1];
    if constexpr (mode == GM_SQ) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int q = kk * 64 + lane;
        const int rr = q / (SC / 8), c8 = (q % (SC / 8)) * 8;
        araw[kk] = Elem<T>::ldraw(M.a, (size_t)(row0 + mi * 32 + rr) * ldo + col0 + c8);
      }
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        buf[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kPitch + ni * 32 + (lane & 31)] = agpr_read(acc[mi][ni][r]);
    wave_lds_sync();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int q = kk * 64 + lane;
      const int rr = q / (SC / 8), c8 = (q % (SC / 8)) * 8;
      float v[8];
      const size_t idx = (size_t)(row0 + mi * 32 + rr) * ldo + col0 + c8;
      if constexpr (mode == GM_SQ) {
        // B' = b A + c A^2 + a I
        float av[8];
        Elem<T>::cvt(araw[kk], av);
        const int dg = (row0 + mi * 32 + rr) - (col0 + c8);   // the diagonal is at e = dg
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = cc * buf[rr * kPitch + c8 + e] + cb * av[e] + (e == dg ? ca : 0.f);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = buf[rr * kPitch + c8 + e];
      }
      Elem<T>::st8(out, idx, v);
      if (mode == GM_SQ && write_t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) buf[rr * kPitch + c8 + e] = v[e];
      }
    }
    if (write_t) {
      wave_lds_sync();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int q = kk * 64 + lane;
        const int c1 = q >> 2, rc = (q & 3) * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = buf[(rc + e) * kPitch + c1];
        Elem<T>::st8(outT, (size_t)(col0 + c1) * ldt + row0 + mi * 32 + rc, v);
      }
    }
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------------------
// Host-side launcher.
// ---------------------------------------------------------------------------
// tile 256, variant 0: 8 waves in 4 x 2 (64 x 128 per wave, two waves per
// SIMD); tile 256, variant 1: 4 waves in 2 x 2 (128 x 128 per wave, one wave
// per SIMD); tile 128: 4 waves in 2 x 2 (64 x 64 per wave), 80 KB of slots,
// two workgroups per CU, for launches with few tiles.
// The third product always writes X'^T beside X' (the next iteration's
// product, the preconditioner update and the output read it).
hipError_t launch_ns_gemm(int ns_t, const DevMat* mats, const TileItem* items, int n_items, int mode, int cur,
                          float ca, float cb, float cc, int variant, int tile, hipStream_t st) {
  if (n_items <= 0) return hipSuccess;
  if (tile != 256 && tile != 128) return hipErrorInvalidValue;
  const int group = 32;   // one super-tile of the planner's raster per XCD wave
  const int per_xcd_groups = (n_items + 8 * group - 1) / (8 * group);
  const dim3 grid(per_xcd_groups * group * 8);
#define NS_LAUNCH(T, MODE, WM, WN, TL)                                                                            \
  hipLaunchKernelGGL((k_ns_gemm<T, MODE, 5, WM, WN, TL>), grid, dim3(WM * WN * 64), 0, st, mats, items, n_items, \
                     group, cur, ca, cb, cc)
#define NS_MODES(T, WM, WN, TL)                             \
  do {                                                      \
    if (mode == GM_GRAM) NS_LAUNCH(T, GM_GRAM, WM, WN, TL); \
    else if (mode == GM_SQ) NS_LAUNCH(T, GM_SQ, WM, WN, TL); \
    else NS_LAUNCH(T, GM_BX, WM, WN, TL);                   \
  } while (0)
  if (ns_t == DT_BF16) {
    if (tile == 128) NS_MODES(__bf16, 2, 2, 128);
    else if (variant == 1) NS_MODES(__bf16, 2, 2, 256);
    else NS_MODES(__bf16, 4, 2, 256);
  } else {
    if (tile == 128) NS_MODES(float, 2, 2, 128);
    else if (variant == 1) NS_MODES(float, 2, 2, 256);
    else NS_MODES(float, 4, 2, 256);
  }
#undef NS_MODES
#undef NS_LAUNCH
  return hipGetLastError();
}

}  // namespace muon
