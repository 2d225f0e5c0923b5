// Newton-Schulz matrix-core engine for gfx950.
//
// The quintic Newton-Schulz map (Aurora record page, www.xxmr.cn/news/295280,
// section 源码实现: X <- a X + (b A + c A^2) X with A = X X^T, X normalised
// first) runs as products, each a launch over every matrix of a batch:
//   GM_GRAM  A  = X X^T                  (s x s, K = L)  upper tiles only, mirrored
//   GM_SQ    B' = b A + c A A^T + a I     (s x s, K = s)  upper tiles only, mirrored
//   GM_SYM   C  = P Q (symmetric P, Q)   (s x s, K = s)  upper tiles only, mirrored
//   GM_BX    X' = P X                    (s x L, K = s)  writes X' and X'^T
// One iteration is GRAM, SQ, then BX with P = B' (B' X equals a X + (b A +
// c A^2) X; adding a on the diagonal of B in the second product's epilogue
// turns the third into a plain product). A block of r iterations of a
// rectangular matrix stays on the short side until its last step: every A_j
// and B'_j is a polynomial in A_0, so they commute, A_{j+1} = B'_j A_j B'_j
// (two GM_SYM products) and X_{j+r} = Q X_j with Q = B'_{r-1} ... B'_0 (GM_SYM
// products, then one GM_BX), which needs 3 s^2 L + (4 r - 3) s^3 flops
// instead of r (3 s^2 L + s^3); the Q update and B'_j A_j, which need only
// B'_j, share one launch. X^T is kept beside X, written by the BX
// epilogue, so every product reads both operands with the reduction index
// contiguous: C[m][n] = sum_k P[m][k] Q[n][k].
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
// so matrix-core work continues across it. The two slots it frees are
// refilled over the following k-steps, a few loads per step between the
// MFMAs (the schedule is next to the K loop): issuing a whole stage's loads
// at once held waves in load issue while their step had little matrix work.
// LDS rows are XOR-swizzled in 16-byte chunks so fragment reads are
// conflict-free.
// On a symmetric product's diagonal tile each wave leaves out the 32x32
// blocks wholly below the diagonal (the stored result is the upper triangle
// and its mirror). The final X' = Q X of a muon_update matrix with the bf16
// type also takes the tail's sums (||U||^2, <U, X>, the rows' parts of X v)
// from the values it stores.
// bf16 runs v_mfma_f32_32x32x16_bf16 (fp32 accumulation); fp32 runs
// v_mfma_f32_32x32x2f32 on the same tiles; the optional fp8 first Gram runs
// v_mfma_scale_f32_32x32x64_f8f6f4 on an e4m3 copy of X0 stored in panels of
// 64 columns.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "muon_device.hpp"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// fp8 (OCP e4m3) operand element: the type tag of the Gram's fp8 form.
struct F8 {
  uint8_t v;
};

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#define GAS __attribute__((address_space(1)))

namespace {

constexpr int kRowBytes = 128;                 // K bytes per tile row per stage
constexpr int kPitch = 128;                    // floats per staged epilogue row (the widest slab)
constexpr int kSlabBytes = 32 * kPitch * 4;    // one wave's 32 x 128 staging slab
// Column swizzle of the fp32 staging slab: row r keeps its columns in 8-float
// chunks XOR-ed with g(r) = f((r / 8) % 4), f = 0, 16, 40, 56. The
// transposed read takes 8 rows of one column per lane, four lanes per column
// at rows 8 apart: the XOR sends those four to different banks (32 or 64 of
// them, per half-wave or per wave), and chunks stay whole for the row reads
// (with a padded pitch instead they shared a bank: the swizzle is -0.3 % on
// the 3.8B set, whose second products stage fp32 slabs).
__device__ __forceinline__ int slab_col(int r, int c) {
  const int g = (r >> 3) & 3;
  return c ^ (((g & 1) << 4) | ((g >> 1) * 40));
}

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

// Sums over lanes in one fixed order with DPP moves (rows of 16 lanes), the
// row totals read from lanes 0, 16, 32 and 48: valid in every lane.
template <int ctrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);   // row_half_mirror
  v += dpp_move<0x140>(v);   // row_mirror
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a + b) + (c + d);
}
// Each lane of a group of 8 (a half row, g = lane % 8) holds p[0..7]; returns
// in lane g the sum of p[g] over the group's 8 lanes. Three halving steps:
// partners across the half-row mirror (g, 7 - g), then g ^ 2, then g ^ 1;
// at each a lane keeps the half of its values whose index bit matches its
// own and adds the partner's copy of them.
__device__ __forceinline__ float group8_transpose_sum(const float (&p)[8], int g) {
  const bool h = (g >> 2) & 1, c = (g >> 1) & 1, d = g & 1;
  float q[4], r[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) q[k] = (h ? p[4 + k] : p[k]) + dpp_move<0x141>(h ? p[k] : p[4 + k]);
#pragma unroll
  for (int k = 0; k < 2; ++k) r[k] = (c ? q[2 + k] : q[k]) + dpp_move<0x4E>(c ? q[k] : q[2 + k]);
  return (d ? r[1] : r[0]) + dpp_move<0xB1>(d ? r[0] : r[1]);
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
// c + a.lo b.lo + a.hi b.hi on two packed bf16 pairs (v_dot2c_f32_bf16; the
// bf16 products are exact in fp32)
__device__ __forceinline__ float dot2(unsigned int a, unsigned int b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
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
  // elements e in [lo, hi) of the 8 only
  __device__ static void st8_part(void* p, size_t i, const float v[8], int lo, int hi) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e >= lo && e < hi) ((unsigned short*)p)[i + e] = f2bf(v[e]);
  }
};
template <> struct Elem<F8> {
  static constexpr int kPerChunk = 16;         // fp8 per 16-byte chunk
  typedef i32x8_t Frag;                        // 32 fp8 (two chunks) per lane per MFMA
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
  __device__ static void st8_part(void* p, size_t i, const float v[8], int lo, int hi) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e >= lo && e < hi) ((float*)p)[i + e] = v[e];
  }
};


}  // namespace

// Launch geometry: grid.x = 8 * per_xcd blocks; the hardware deals
// consecutive workgroups round-robin to the 8 XCDs, so block b runs on XCD
// b % 8. Items are dealt to XCDs in runs of `group` consecutive items (one
// super-tile of the planner's raster, whose tiles share operand panels), so a
// run executes together on one XCD and reuses its L2.
// roles: the roles in DevMat::sq of operand P (bits 0-3), operand Q (bits
// 4-7) and the output (bits 8-11); GM_BX only: bit 12 = the last product of a pass,
// bit 13 = that pass is the last Aurora pass (NS_LAST_BX, NS_LAST_PASS). A
// GM_SYM launch may hold two independent products: tiles whose item has
// pad = 1 take roles bits 16-27 instead.
template <typename T, int mode, int S, int WM, int WN, int TILE>
__global__ __launch_bounds__(WM * WN * 64, TILE == 256 ? 1 : 2) void k_ns_gemm(const DevMat* __restrict__ mats,
                                                             const TileItem* __restrict__ items, int n_items,
                                                             int group, int cur, int roles, float ca, float cb,
                                                             float cc) {
  constexpr int NW = WM * WN;                // waves per workgroup
  constexpr int MI = TILE / WM / 32;         // 32x32 blocks per wave, down
  constexpr int NI = TILE / WN / 32;         // 32x32 blocks per wave, across
  constexpr int kOpBytes = TILE * kRowBytes; // one operand of one stage (one LDS slot)
  constexpr int LPO = TILE / 8 / NW;         // direct loads per wave per operand per stage
  constexpr bool kF8 = sizeof(T) == 1;       // fp8 operands (GM_GRAM only), bf16 output
  // k-steps per stage: 16 bf16, 4 fp32 (four 32x32x2 MFMAs) or 64 fp8 of K per
  // lane pair, so a 128-byte stage row is 4, 4 or 2 k-steps
  constexpr int KS = kF8 ? 2 : 4;
  constexpr int kReadStep = (MI + NI) * (kF8 ? 2 : 1);            // LDS reads per k-step
  static_assert(!kF8 || mode == GM_GRAM, "fp8 operands are for the Gram");
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

  const int ro = it.pad ? roles >> 16 : roles;   // the tile's product (two in one GM_SYM launch)
  const int role_p = ro & 15, role_q = (ro >> 4) & 15, role_o = (ro >> 8) & 15, last = (roles >> 12) & 3;
  // a pass's first X' = Q X of a matrix whose X0^T is its blended update scaled row by row
  const bool x0n = mode == GM_BX && sizeof(T) == 2 && (roles & NS_FIRST) && M.x0n;
  // a pass's first Gram of a matrix whose X0 is its blended update times scale
  const bool x0g = mode == GM_GRAM && sizeof(T) == 2 && (roles & NS_FIRST) && M.x0g;
  const T *P, *Q;
  int ld, K;
  if constexpr (mode == GM_GRAM) {
    if constexpr (kF8) {
      // the fp8 copy of X0 (first Gram of a pass) is stored in panels of 64
      // columns, each s_pad x 64 bytes: a tile's rows start at row tm*TILE of
      // panel 0, row pitch 64 bytes
      const T* x = (const T*)M.x8;
      P = x + (size_t)it.tm * TILE * 64;
      Q = x + (size_t)it.tn * TILE * 64;
      ld = 64; K = Lp;
    } else {
      const T* x = (const T*)(x0g ? M.xn : M.x[cur]);   // xn: ld = cols = L_pad
      P = x + (size_t)it.tm * TILE * Lp;
      Q = x + (size_t)it.tn * TILE * Lp;
      ld = Lp; K = Lp;
    }
  } else if constexpr (mode == GM_SQ) {
    const T* a = (const T*)M.sq[role_p];
    P = a + (size_t)it.tm * TILE * sp;
    Q = a + (size_t)it.tn * TILE * sp;
    ld = sp; K = sp;
  } else if constexpr (mode == GM_SYM) {
    P = (const T*)M.sq[role_p] + (size_t)it.tm * TILE * sp;
    Q = (const T*)M.sq[role_q] + (size_t)it.tn * TILE * sp;
    ld = sp; K = sp;
  } else {
    P = (const T*)M.sq[role_p] + (size_t)it.tm * TILE * sp;
    Q = (const T*)(x0n ? M.xn : M.xt[cur]) + (size_t)it.tn * TILE * sp;   // xn: ld = cols = s_pad
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
  // fp8 panels: logical chunks 0-3 of a stage row lie in panel 2 ks, chunks
  // 4-7 in panel 2 ks + 1 (pstride bytes further), so the per-lane offset
  // still holds for the whole K loop and a stage advances two panels.
  const int prow = 8 * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ ((prow >> 1) & 7);
  const int pstride = kF8 ? sp * 64 : 0;   // bytes per fp8 panel
  const uint32_t lane_off =
      kF8 ? (uint32_t)(prow * 64 + (lchunk & 3) * 16 + (lchunk >> 2) * pstride)
          : (uint32_t)(((int64_t)prow * ld + lchunk * CPR) * sizeof(T));
  const int rstep = (int)((int64_t)8 * NW * ld * sizeof(T));
  const int kstride = kF8 ? 2 * pstride : kRowBytes;   // bytes from one K stage to the next
  // Buffer resources over the two operand panels. Every read stays inside
  // its panel: the K offset travels in the scalar offset and stages past the
  // end of K are clamped. On a diagonal tile of the two symmetric products
  // both operands are the same panel: the second resource gets no records,
  // and since the range check compares the per-lane offset with the record
  // count, each of its loads fails the check and fetches nothing (the issue
  // count, and with it every wait, stays the same); both operands' fragments
  // are read from the first panel's slot.
  const int ext = kF8 ? (Lp / 64 - 1) * pstride + TILE * 64 : (int)((int64_t)TILE * ld * sizeof(T));
  const bool same = (mode == GM_GRAM || mode == GM_SQ) && (it.tm == it.tn);
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc((void*)P, (short)0, ext, 0x00020000);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)Q, (short)0, same ? 0 : ext, 0x00020000);

  // Operand stage o is P (o even) or Q (o odd) of stage o/2; it goes to
  // slot o % S. Stages past the end of K are clamped to the last one: an
  // L2-resident re-read into a slot nobody reads again, which keeps every
  // wait below the same. issue() takes loads [i0, i1) of this wave's LPO.
  auto issue = [&](int slot, int o, int i0, int i1) {
    const int ks = min(o >> 1, nk - 1);
    uint8_t* sm = smem + slot * kOpBytes;
#pragma unroll
    for (int i = i0; i < i1; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds((o & 1) ? rq : rp, LDS_PTR(sm + (NW * i + wave) * 1024), 16,
                                               lane_off, ks * kstride + i * rstep, 0, 0);
  };

  // Fragments: lane l reads tile row (block base + l%32), logical chunk
  // 2 s + l/32 of the stage (8 bf16 or 4 fp32 consecutive k) for k-step s;
  // fp8: chunks 4 s + 2 (l/32) and the next one (32 consecutive k). The
  // matrix cores pair A and B elements by the same lane half and register
  // position, so any layout both operands share gives the same sums.
  typedef typename Elem<T>::Frag Frag;
  Frag fa[2][MI], fb[2][NI];
  const int lr = lane & 31;
  auto read_frags = [&](int pslot, int qslot, int s, int buf, auto off_c) {
    using K = Keep<decltype(off_c)::value, MI, NI>;
    const uint8_t* sa = smem + pslot * kOpBytes;
    const uint8_t* sb = same ? sa : smem + qslot * kOpBytes;
    if constexpr (kF8) {
      const int c0 = 4 * s + 2 * (lane >> 5);
      const int ph0 = (c0 ^ ((lr >> 1) & 7)) * 16, ph1 = ((c0 + 1) ^ ((lr >> 1) & 7)) * 16;
      auto frag = [&](const uint8_t* row) {
        const u32x4_t lo = *(const u32x4_t*)(row + ph0), hi = *(const u32x4_t*)(row + ph1);
        return (i32x8_t){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                         (int)hi[3]};
      };
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        if (K::row(mi)) fa[buf][mi] = frag(sa + (wm * MI * 32 + mi * 32 + lr) * kRowBytes);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        if (K::col(ni)) fb[buf][ni] = frag(sb + (wn * NI * 32 + ni * 32 + lr) * kRowBytes);
    } else {
      const int ph = ((2 * s + (lane >> 5)) ^ ((lr >> 1) & 7)) * 16;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        if (K::row(mi)) fa[buf][mi] = *(const Frag*)(sa + (wm * MI * 32 + mi * 32 + lr) * kRowBytes + ph);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        if (K::col(ni)) fb[buf][ni] = *(const Frag*)(sb + (wn * NI * 32 + ni * 32 + lr) * kRowBytes + ph);
    }
  };
  auto mfmas = [&](int buf, auto off_c) {
    using K = Keep<decltype(off_c)::value, MI, NI>;
    if constexpr (kF8) {
      // e4m3 operands (format 0), unit block scales (E8M0 127 = 1.0)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          if (K::blk(mi, ni))
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[buf][mi], fb[buf][ni], acc[mi][ni], 0,
                                                                          0, 0, 127, 0, 127);
    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          if (K::blk(mi, ni))
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
            if (K::blk(mi, ni))
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[buf][mi][e], fb[buf][ni][e], acc[mi][ni], 0, 0,
                                                                 0);
    }
  };
  // Spread nmem memory instructions evenly between one k-step's MFMAs, the
  // first nloads of them direct loads, the rest LDS reads. The compiler
  // cannot tell the refill and the reads apart, so the pattern keeps their
  // program order.
  // nmem counts a whole wave part's kReadStep LDS reads; a wave leaving
  // blocks out (Keep) has fewer MFMAs and reads.
  auto spread = [&](int nmem, int nloads, auto off_c) {
    using K = Keep<decltype(off_c)::value, MI, NI>;
    constexpr int nmf = K::blocks() * (sizeof(T) == 4 ? 4 : 1);
    nmem += K::frags() * (kF8 ? 2 : 1) - kReadStep;
#pragma unroll
    for (int q = 0; q < nmf; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
#pragma unroll
      for (int t = q * nmem / nmf; t < (q + 1) * nmem / nmf; ++t) {
        if (t < nloads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one direct load
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // one LDS read
      }
    }
  };

  // Refill schedule. After the barrier of stage k the slots of stage k are
  // free; the last k-step refills one of them with operand stage 2k + S
  // (needed at the next barrier), and the first two k-steps of stage k + 1
  // load operand stage 2k + S + 1 into the other, in halves (needed one
  // barrier later). Issuing all of a stage's refill at once, eight 1 KB
  // loads per wave from all eight waves, held waves in load issue while
  // their k-step had 256 cycles of matrix work (3-7 % per product).
  // With 256-tiles (one workgroup per CU, stages long enough to cover the
  // latency) the next-barrier stage is split too: its first half in the last
  // k-step, its second half in k-step 0 of the next stage, the deferred stage
  // in k-steps 1 and 2 - two loads per k-step throughout (a further 0.8 % on
  // the 3.8B set). 128-tiles, whose short stages leave less time for that
  // second half, keep the whole next-barrier stage in the last k-step (the
  // even split made them 6 % slower).
  // Prologue: operand stages 0 .. S-2 (stage S-1 is the first deferred
  // refill; with the even split, stage S-2's second half is iteration 0's);
  // wait for stage 0, read its first k-step. With 256-tiles the two operands
  // of stage 0 go out alone and land before the rest is issued: the CUs of a
  // round start together, and stage 0 no longer queues behind every CU's
  // later stages (-0.2 to -0.6 % on the 3.8B set, three boxes; the same
  // order on 128-tiles gained nothing).
  constexpr bool kEven = TILE == 256 && KS == 4;
  if constexpr (kEven) {
    issue(0, 0, 0, LPO);
    issue(1, 1, 0, LPO);
    wait_vm<0>();
#pragma unroll
    for (int o = 2; o < S - 2; ++o) issue(o, o, 0, LPO);
    issue(S - 2, S - 2, 0, LPO / 2);
  } else {
#pragma unroll
    for (int o = 0; o < S - 1; ++o) issue(o, o, 0, LPO);
    wait_vm<(S - 3) * LPO>();
  }
  ring_barrier();
  // On a diagonal tile of the symmetric products the 32x32 blocks wholly
  // below the diagonal need no work: the stored result is the upper triangle
  // and its mirror. Each wave runs the K loop compiled for its offset from
  // the diagonal (Keep), without those blocks' matrix-core work and without
  // the fragments no kept block reads (a wave wholly below the diagonal does
  // none); every wave still issues its share of every stage's loads and
  // meets every barrier, so the workgroup runs the same sequence of loads,
  // waits and barriers. The matrix cores do 28 of 64 blocks' work less on
  // those tiles (8 waves of 64 x 128), which the power-limited clock gets
  // back.
  auto kloop = [&](auto off_c) {
    constexpr bool kAny = Keep<decltype(off_c)::value, MI, NI>::blocks() > 0;
    auto rf = [&](int pslot, int qslot, int st, int buf) {
      if constexpr (kAny) read_frags(pslot, qslot, st, buf, off_c);
    };
    auto mf = [&](int buf) {
      if constexpr (kAny) mfmas(buf, off_c);
    };
    auto sp = [&](int nmem, int nloads) {
      if constexpr (kAny) spread(nmem, nloads, off_c);
    };
    rf(0, 1, 0, 0);
    // slots of stage k (ps, qs) and of stage k+1 (pn, qn)
    int ps = 0, qs = 1, pn = 2 % S, qn = 3 % S;
    constexpr int NDS = KS - 1 < 2 ? KS - 1 : 2;   // k-steps that carry the deferred refill
    for (int k = 0; k < nk - 1; ++k) {
      // all k-steps but the last, each with the next k-step's fragments read
      // between its MFMAs; the first NDS also issue part of operand stage
      // 2k + S - 1 into the slot freed at the previous barrier (the slot after
      // stage k + 1's two)
      const int dslot = (pn + 2 >= S) ? pn + 2 - S : pn + 2;
  #pragma unroll
      for (int s = 0; s < KS - 1; ++s) {
        if constexpr (kEven) {
          // k-step 0: second half of operand stage 2k + S - 2 (slot qn), at
          // wave priority 1 (like the raise over the last k-step: a wave
          // still issuing this stage's loads outranks its SIMD partner; 1.8 %
          // on the 3.8B set, priority 2 here 0.7 %); k-steps 1, 2: operand
          // stage 2k + S - 1 in halves (slot dslot)
          if (s == 0) {
            __builtin_amdgcn_s_setprio(1);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (s == 0) issue(qn, 2 * k + S - 2, LPO / 2, LPO);
          else issue(dslot, 2 * k + S - 1, (s - 1) * LPO / 2, s * LPO / 2);
          rf(ps, qs, s + 1, (s + 1) & 1);
          mf(s & 1);
          sp(kReadStep + LPO / 2, LPO / 2);
          if (s == 0) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
          }
        } else if (s < NDS) {
          issue(dslot, 2 * k + S - 1, s * LPO / NDS, (s + 1) * LPO / NDS);
          rf(ps, qs, s + 1, (s + 1) & 1);
          mf(s & 1);
          sp(kReadStep + LPO / NDS, LPO / NDS);
        } else {
          rf(ps, qs, s + 1, (s + 1) & 1);
          mf(s & 1);
          sp(kReadStep, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // stage k+1 has landed for every wave (only the deferred operand stage,
      // the S - 4 most recent, may be in flight); stage k's slots are free
      wait_lgkm0();
      wait_vm<(S - 4) * LPO>();
      ring_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // the last k-step: the refill of one freed slot with operand stage 2k+S,
      // then the next stage's first fragments.
      // With 256-tiles it runs at raised wave priority: a wave still in it
      // outranks the waves of its SIMD that have moved on to the next stage, so
      // the waves reach the next barrier closer together (1-1.2 % faster on the
      // 3072-row products). 128-tiles, two workgroups per CU, keep the default.
      if constexpr (TILE == 256) __builtin_amdgcn_s_setprio(2);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kEven) {
        issue(ps, 2 * k + S, 0, LPO / 2);
        rf(pn, qn, 0, 0);
        mf(1);
        sp(LPO / 2 + kReadStep, LPO / 2);
      } else {
        issue(ps, 2 * k + S, 0, LPO);
        rf(pn, qn, 0, 0);
        mf(1);
        sp(LPO + kReadStep, LPO);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (TILE == 256) __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      ps = pn; qs = qn;
      pn = (pn + 2 >= S) ? pn + 2 - S : pn + 2;
      qn = (qn + 2 >= S) ? qn + 2 - S : qn + 2;
    }
  #pragma unroll
    for (int s = 0; s < KS - 1; ++s) {
      rf(ps, qs, s + 1, (s + 1) & 1);
      mf(s & 1);
    }
    mf(1);   // KS is even: the last k-step's fragments are in buffer 1
  };
  using Off = std::integral_constant<int, kDiagFull>;
  if constexpr (mode == GM_BX || sizeof(T) == 4) {
    // (fp32 operands compute whole tiles: the reduced forms spill registers
    // in their second product)
    kloop(Off{});
  } else {
    // the form compiled for the wave's offset from the diagonal (diag_form)
    const int form = it.tm == it.tn ? diag_form(wm, wn, MI, NI) : kDiagFull;
    if (form == NI) kloop(std::integral_constant<int, NI>{});
    else if (form == 0) kloop(std::integral_constant<int, 0>{});
    else if (form == 2) kloop(std::integral_constant<int, 2>{});
    else kloop(Off{});
  }
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
  bool write_o = true, write_t;
  if constexpr (mode == GM_BX) {
    out = M.x[cur ^ 1]; outT = M.xt[cur ^ 1]; ldo = Lp; ldt = sp;
    // the last product of a pass writes only the orientation read next: the
    // D update reads rows of X' when the wide matrix is equilibrated on its
    // rows (on the long side it takes the band sums below instead), the tail
    // reads the storage orientation (X'^T for a tall matrix, X' otherwise)
    write_t = true;
    if (last & 1) {
      if ((last & 2) || !M.aurora) { write_t = M.tall != 0; write_o = !write_t; }   // this matrix's last pass
      else { write_o = M.eq_short != 0; write_t = !write_o; }
    }
  } else {
    out = M.sq[role_o]; outT = out; ldo = sp; ldt = sp;
    write_t = it.tm != it.tn;
  }
  // The last product of a non-final Aurora pass of a matrix equilibrated on
  // its long side feeds only the D update, which needs each long-side line's
  // (column of X') sum of squares: it writes those, per 64-row band, from the
  // values it would store, and stores nothing else.
  const bool band_sums = mode == GM_BX && (last & 1) && !(last & 2) && M.lsq != nullptr;
  if (band_sums) write_o = write_t = false;
  // Fused tail: the final product of a bf16 muon_update matrix stores U as
  // usual and also takes, per 64 x 64 block of the storage frame, ||U||^2 and
  // <U, X> of the stored values (ftail) and, per storage row, the block's part
  // of (X / ||X||_F) v (frow), X the blended update, v the power iteration's
  // last vector. In a block, lane l takes storage rows 8 k + l / 8 (k = 0..7)
  // at columns 8 (l % 8) .. + 7; the sums run in one fixed order, the same for
  // every tile size and layout, so they do not depend on how the product was
  // tiled. The X chunks are requested once the tile is staged, and arrive
  // while the wave stores U.
  constexpr int FTC = NI * 32 / 64;                  // 64-wide blocks across the wave's tile
  constexpr int FTB = (MI * 32 / 64) * FTC;          // 64 x 64 blocks per wave
  constexpr int FTP = FTB <= 2 ? FTB : 0;            // blocks whose X is requested before U is stored
  bool ft = false;
  if constexpr (mode == GM_BX && sizeof(T) == 2) ft = (last & 1) && ((last & 2) || !M.aurora) && M.ftail != nullptr;
  const bool ftx = ft && M.ftx != 0;
  const int fa0 = lane >> 3, fch = lane & 7;
  auto ft_origin = [&](int b, int& srow0, int& scol0) {
    const int bi = b / FTC, bj = b % FTC;
    if (M.tall) { srow0 = col0 + 64 * bj; scol0 = row0 + 64 * bi; }
    else { srow0 = row0 + 64 * bi; scol0 = col0 + 64 * bj; }
  };
  // a block's X chunks (rows srow0 + 8 k + l / 8, columns scol0 + 8 (l % 8)) and
  // v entries: plain vector loads for a block inside a matrix of whole
  // 16-byte rows (the branch is uniform over the wave), element-wise ones
  // with zeros outside the matrix otherwise
  auto ft_load = [&](int srow0, int scol0, u16x8_t (&q)[8], float (&vv)[8]) {
    const int j = scol0 + 8 * fch;
    if (srow0 + 64 <= M.rows && scol0 + 64 <= M.cols && (M.cols & 7) == 0) {
      const GAS unsigned short* xp = (const GAS unsigned short*)M.xn + (size_t)(srow0 + fa0) * M.cols + j;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) q[kk] = *(const GAS u16x8_t*)(xp + (size_t)8 * kk * M.cols);
      const f32x4_t v0 = *(const GAS f32x4_t*)(M.pv + j), v1 = *(const GAS f32x4_t*)(M.pv + j + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { vv[e] = v0[e]; vv[e + 4] = v1[e]; }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int i = srow0 + 8 * kk + fa0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          q[kk][e] = (i < M.rows && j + e < M.cols) ? ((const GAS unsigned short*)M.xn)[(size_t)i * M.cols + j + e]
                                                    : (unsigned short)0;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = j + e < M.cols ? ((const GAS float*)M.pv)[j + e] : 0.f;
    }
  };
  // A symmetric product's result (Gram, B', or a GM_SYM product, which is
  // symmetric only in exact arithmetic: C[m][n] and C[n][m] come from
  // different products) keeps the upper triangle of its diagonal tiles and
  // writes the lower one as its mirror: the stored matrix is the mirrored
  // upper triangle whatever the tile size, as for off-diagonal tiles, and the
  // waves wholly below the diagonal (idle above) store nothing.
  const bool diag_sym = mode != GM_BX && it.tm == it.tn;
  if (diag_sym) write_t = true;
  // the second product's first slab of A values, requested before the
  // barrier (the waves that finish their K loop first wait there)
  constexpr int kSC = NI * 32, kKK = kSC / 16;
  typename Elem<std::conditional_t<kF8, __bf16, T>>::Raw apre[mode == GM_SQ && sizeof(T) != 1 ? kKK : 1];
  if constexpr (mode == GM_SQ && sizeof(T) != 1) {
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      const int q = kk * 64 + lane;
      const int rr = q / (kSC / 8), c8 = (q % (kSC / 8)) * 8;
      apre[kk] = Elem<T>::ldraw(M.sq[role_p], (size_t)(row0 + rr) * ldo + col0 + c8);
    }
  }
  __syncthreads();   // every wave is done with the slots
  // the fp8 Gram's products carry the square of the operand scale q; a
  // pass's first X' = Q X read from xn takes the prologue's scale D_l per
  // output column l, and a first Gram read from xn the square of its scale
  const float oscale = kF8 ? M.scal[SC_F8INV2] : x0g ? M.scal[SC_SCALE] * M.scal[SC_SCALE] : 1.f;
  float cscale[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    cscale[ni] = oscale;
    if (x0n) cscale[ni] = M.scal[SC_SCALE] * (M.aurora ? M.dvec[col0 + ni * 32 + (lane & 31)] : 1.f);
  }
  if constexpr ((sizeof(T) == 2 || kF8) && mode != GM_SQ) {
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
          const unsigned int lo = (unsigned int)f2bf(agpr_read(acc[mi][ni][4 * g]) * cscale[ni]) |
                                  ((unsigned int)f2bf(agpr_read(acc[mi][ni][4 * g + 1]) * cscale[ni]) << 16);
          const unsigned int hi = (unsigned int)f2bf(agpr_read(acc[mi][ni][4 * g + 2]) * cscale[ni]) |
                                  ((unsigned int)f2bf(agpr_read(acc[mi][ni][4 * g + 3]) * cscale[ni]) << 16);
          *(u32x2_t*)(st + sidx(row, col)) = (u32x2_t){lo, hi};
        }
    wave_lds_sync();
    if (band_sums) {
#pragma unroll
      for (int b = 0; b < TR / 64; ++b)
#pragma unroll
        for (int cc = 0; cc < TC; cc += 64) {
          const int c = cc + lane;
          float sq = 0.f;
#pragma unroll
          for (int ch = 0; ch < 8; ++ch) {
            const u16x8_t v = *(const u16x8_t*)(st + sidx(64 * b + 8 * ch, c));   // rows 64b+8ch .. +7
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = bf2f(v[e]);
              sq += x * x;
            }
          }
          M.lsq[(size_t)((row0 + 64 * b) >> 6) * Lp + col0 + c] = sq;
        }
      return;
    }
    if constexpr (mode == GM_BX && sizeof(T) == 2) {
      if (ft) {
        const float n2 = M.scal[SC_XNORM2];
        const float xin = n2 > 0.f ? 1.f / sqrtf(n2) : 0.f;
        const int nbc = (M.cols + 63) >> 6;
        u16x8_t fxq[FTP > 0 ? FTP : 1][8];
        float fvv[FTP > 0 ? FTP : 1][8];
        if constexpr (FTP > 0) {
          if (ftx) {
#pragma unroll
            for (int b = 0; b < FTP; ++b) {
              int srow0, scol0;
              ft_origin(b, srow0, scol0);
              ft_load(srow0, scol0, fxq[b], fvv[b]);
            }
          }
        }
        float uus[FTB], uxs[FTB];
        // the stored chunk k of block (bi, bj) of this lane, read from the
        // staged tile; store != 0 also writes it to U
        auto chunk = [&](auto tall_c, int bi, int bj, int kk, bool store) -> u16x8_t {
          u16x8_t u;
          if constexpr (decltype(tall_c)::value) {
            // storage row col0 + c: 8 staged rows of column c
            const int r8 = 64 * bi + 8 * fch, c = 64 * bj + 8 * kk + fa0;
            u = *(const u16x8_t*)(st + sidx(r8, c));
            if (store) *(u16x8_t*)((unsigned short*)outT + (size_t)(col0 + c) * ldt + row0 + r8) = u;
          } else {
            const int r = 64 * bi + 8 * kk + fa0, c8 = 64 * bj + 8 * fch;
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = st[sidx(r, c8 + e)];
            if (store) *(u16x8_t*)((unsigned short*)out + (size_t)(row0 + r) * ldo + col0 + c8) = u;
          }
          return u;
        };
        auto blocks = [&](auto tall_c) {
          // U stored and ||U||^2 taken while the X chunks are on their way
#pragma unroll
          for (int b = 0; b < FTB; ++b) {
            float uu = 0.f;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
              const u32x4_t uw = __builtin_bit_cast(u32x4_t, chunk(tall_c, b / FTC, b % FTC, kk, true));
#pragma unroll
              for (int p = 0; p < 4; ++p) uu = dot2(uw[p], uw[p], uu);
            }
            uus[b] = uu;
            uxs[b] = 0.f;
          }
          if (!ftx) return;
#pragma unroll
          for (int b = 0; b < FTB; ++b) {
            int srow0, scol0;
            ft_origin(b, srow0, scol0);
            u16x8_t xq[8];
            float vv[8];
            if constexpr (FTP > 0) {
#pragma unroll
              for (int kk = 0; kk < 8; ++kk) xq[kk] = fxq[b < FTP ? b : 0][kk];
#pragma unroll
              for (int e = 0; e < 8; ++e) vv[e] = fvv[b < FTP ? b : 0][e];
            } else {
              ft_load(srow0, scol0, xq, vv);
            }
            // v as a sum of two bf16 parts, vh + vl (v to about 16 bits), so
            // that X v takes packed bf16 products too
            unsigned int vh[4], vl[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const unsigned short h0 = f2bf(vv[2 * p]), h1 = f2bf(vv[2 * p + 1]);
              vh[p] = (unsigned int)h0 | ((unsigned int)h1 << 16);
              vl[p] = (unsigned int)f2bf(vv[2 * p] - bf2f(h0)) | ((unsigned int)f2bf(vv[2 * p + 1] - bf2f(h1)) << 16);
            }
            float ux = 0.f, pr[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
              const u32x4_t uw = __builtin_bit_cast(u32x4_t, chunk(tall_c, b / FTC, b % FTC, kk, false));
              const u32x4_t xw = __builtin_bit_cast(u32x4_t, xq[kk]);
              pr[kk] = 0.f;
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                ux = dot2(uw[p], xw[p], ux);
                pr[kk] = dot2(xw[p], vh[p], pr[kk]);
                pr[kk] = dot2(xw[p], vl[p], pr[kk]);
              }
            }
            uxs[b] = ux;
            // each row's 8 parts (one per lane of an 8-lane group) to one
            // lane: lane g of the group ends with row 8 g + l / 8
            const float t = group8_transpose_sum(pr, fch);
            const int i = srow0 + 8 * fch + fa0;
            if (i < M.rows && scol0 < M.cols) *(GAS float*)(M.frow + (size_t)(scol0 >> 6) * M.rows + i) = t * xin;
          }
        };
        if (M.tall) blocks(std::true_type{});
        else blocks(std::false_type{});
#pragma unroll
        for (int b = 0; b < FTB; ++b) {
          int srow0, scol0;
          ft_origin(b, srow0, scol0);
          const float su = wave_sum_dpp(uus[b]), sx = wave_sum_dpp(uxs[b]);
          if (lane == 0 && srow0 < M.rows && scol0 < M.cols)
            *(GAS f32x2_t*)(M.ftail + ((size_t)(srow0 >> 6) * nbc + (scol0 >> 6)) * 2) = (f32x2_t){su, sx};
        }
        return;
      }
    }
    // row-major: 8 consecutive columns of one row per lane
    if (write_o) {
#pragma unroll
      for (int kk = 0; kk < TR * TC / 8 / 64; ++kk) {
        const int q = kk * 64 + lane;
        const int r = q / (TC / 8), c8 = (q % (TC / 8)) * 8;
        u16x8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = st[sidx(r, c8 + e)];
        unsigned short* dst = (unsigned short*)out + (size_t)(row0 + r) * ldo + col0 + c8;
        const int d = (col0 + c8) - (row0 + r);   // element e is upper when d + e >= 0
        if (!diag_sym || d >= 0) {
          *(u16x8_t*)dst = v;
        } else if (d > -8) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (d + e >= 0) dst[e] = v[e];
        }
      }
    }
    if (write_t) {
      // transposed: 8 consecutive rows of one column per lane, a column's
      // TR rows (a whole number of 128-byte lines) by consecutive lanes
#pragma unroll
      for (int kk = 0; kk < TR * TC / 8 / 64; ++kk) {
        const int q = kk * 64 + lane;
        const int c = q / (TR / 8), r8 = (q % (TR / 8)) * 8;
        const u16x8_t v = *(const u16x8_t*)(st + sidx(r8, c));
        unsigned short* dst = (unsigned short*)outT + (size_t)(col0 + c) * ldt + row0 + r8;
        // the mirror of source element (row0 + r8 + e, col0 + c): only from
        // the strict upper triangle on a GM_SYM diagonal tile
        const int d = (col0 + c) - (row0 + r8);   // element e qualifies when e < d
        if (!diag_sym || d >= 8) {
          *(u16x8_t*)dst = v;
        } else if (d > 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < d) dst[e] = v[e];
        }
      }
    }
    return;
  }
  if constexpr (!kF8) {
    // 32-row fp32 slabs; the second product's A values for a slab are loaded
    // before the slab is staged, so their latency overlaps the staging (the
    // first slab's before the barrier above, where the waves that finished
    // their K loop early wait anyway: 0.3 % on the 3.8B set)
    float* buf = (float*)(smem + wave * kSlabBytes);
    constexpr int SC = NI * 32;                // staged slab: 32 rows x SC columns
    float bsq[(SC + 63) / 64];                 // band sums of squares per column (band_sums)
    constexpr int KK = SC / 16;                // 8-column chunks per lane per slab
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      typename Elem<T>::Raw araw[mode == GM_SQ ? KK : 1];
      if constexpr (mode == GM_SQ) {
        static_assert(KK == kKK, "slab chunks");
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (mi == 0) { araw[kk] = apre[kk]; continue; }
          const int q = kk * 64 + lane;
          const int rr = q / (SC / 8), c8 = (q % (SC / 8)) * 8;
          araw[kk] = Elem<T>::ldraw(M.sq[role_p], (size_t)(row0 + mi * 32 + rr) * ldo + col0 + c8);
        }
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          buf[row * kPitch + slab_col(row, ni * 32 + (lane & 31))] = agpr_read(acc[mi][ni][r]);
        }
      wave_lds_sync();
      if (band_sums) {
        // two 32-row slabs make a 64-row band
#pragma unroll
        for (int cc = 0; cc < SC; cc += 64) {
          const int c = cc + lane;
          float sq = 0.f;
#pragma unroll
          for (int r = 0; r < 32; ++r) {
            const float x = buf[r * kPitch + slab_col(r, c)];
            sq += x * x;
          }
          bsq[cc / 64] = (mi & 1) ? bsq[cc / 64] + sq : sq;
          if (mi & 1) M.lsq[(size_t)((row0 + mi * 32) >> 6) * Lp + col0 + c] = bsq[cc / 64];
        }
        wave_lds_sync();
        continue;
      }
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
          for (int e = 0; e < 8; ++e)
            v[e] = cc * buf[rr * kPitch + slab_col(rr, c8) + e] + cb * av[e] + (e == dg ? ca : 0.f);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = buf[rr * kPitch + slab_col(rr, c8) + e];
        }
        if (write_o) {
          const int d = (col0 + c8) - (row0 + mi * 32 + rr);   // upper when d + e >= 0
          if (!diag_sym || d >= 0) Elem<T>::st8(out, idx, v);
          else if (d > -8) Elem<T>::st8_part(out, idx, v, -d, 8);
        }
        if (mode == GM_SQ && write_t) {
#pragma unroll
          for (int e = 0; e < 8; ++e) buf[rr * kPitch + slab_col(rr, c8) + e] = v[e];
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
          for (int e = 0; e < 8; ++e) v[e] = buf[(rc + e) * kPitch + slab_col(rc + e, c1)];
          const size_t tidx = (size_t)(col0 + c1) * ldt + row0 + mi * 32 + rc;
          const int d = (col0 + c1) - (row0 + mi * 32 + rc);   // mirror of a strict-upper source when e < d
          if (!diag_sym || d >= 8) Elem<T>::st8(outT, tidx, v);
          else if (d > 0) Elem<T>::st8_part(outT, tidx, v, 0, d);
        }
      }
      wave_lds_sync();
    }
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
                          int roles, float ca, float cb, float cc, int variant, int tile, hipStream_t st) {
  if (n_items <= 0) return hipSuccess;
  if (tile != 256 && tile != 128) return hipErrorInvalidValue;
  const int group = 32;   // one super-tile of the planner's raster per XCD wave
  const int per_xcd_groups = (n_items + 8 * group - 1) / (8 * group);
  const dim3 grid(per_xcd_groups * group * 8);
#define NS_LAUNCH(T, MODE, WM, WN, TL)                                                                            \
  hipLaunchKernelGGL((k_ns_gemm<T, MODE, 5, WM, WN, TL>), grid, dim3(WM * WN * 64), 0, st, mats, items, n_items, \
                     group, cur, roles, ca, cb, cc)
#define NS_MODES(T, WM, WN, TL)                               \
  do {                                                        \
    if (mode == GM_GRAM) NS_LAUNCH(T, GM_GRAM, WM, WN, TL);   \
    else if (mode == GM_SQ) NS_LAUNCH(T, GM_SQ, WM, WN, TL);  \
    else if (mode == GM_SYM) NS_LAUNCH(T, GM_SYM, WM, WN, TL); \
    else NS_LAUNCH(T, GM_BX, WM, WN, TL);                     \
  } while (0)
  if (ns_t == DT_F8) {
    // fp8 operands: the Gram only
    if (mode != GM_GRAM) return hipErrorInvalidValue;
    if (tile == 128) NS_LAUNCH(F8, GM_GRAM, 2, 2, 128);
    else if (variant == 1) NS_LAUNCH(F8, GM_GRAM, 2, 2, 256);
    else NS_LAUNCH(F8, GM_GRAM, 4, 2, 256);
  } else if (ns_t == DT_BF16) {
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
