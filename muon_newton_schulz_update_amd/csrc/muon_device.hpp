// Device-side descriptors shared by the libmuon kernels and the host planner.
//
// Layout of one matrix's work in HBM (all row-major, 256-byte aligned):
//   xn      rows x cols, ld = cols, NS type: the blended (Nesterov) update X
//   x[2]    s_pad x L_pad, ld = L_pad: Newton-Schulz iterate, ping-pong
//   xt[2]   L_pad x s_pad, ld = s_pad: its transpose, written by the same
//           epilogue, so every product of the iteration reads both operands
//           with the reduction index contiguous ("NT" form)
//   a, b    s_pad x s_pad: Gram A = X X^T and B = b A + c A^2
//   float vectors and partial-sum buffers (see DevMat)
// s = min(rows, cols) (the short side), L = max(rows, cols); both padded up to
// a multiple of the 256-wide tile. Padding is zero and stays exactly zero
// through every iteration (zero rows/columns map to zero), so the matrix-core
// kernels need no bounds checks.
#pragma once
#include <stdint.h>

namespace muon {

constexpr int kTile = 256;        // NS output tile edge (and padding unit)
constexpr int kStreamRows = 32;   // rows per tile of the streaming kernels (4 waves x kWaveRows)
constexpr int kWaveRows = 8;      // rows per wave of a streaming tile, loaded in one batch
constexpr int kSegCols = 512;     // columns per streaming tile (a lane covers 8 of them)
constexpr int kStreamCols = 2048; // columns per tile of the X^T u kernel
constexpr int kRmvRows = 256;     // rows per tile of the X^T u kernel (and the fused pass's widest band)
constexpr int kFusedCols = 12288; // widest matrix the fused X^T X v pass takes (its v sits in LDS)
constexpr int kFusedPart = 64;    // rows per partial w of the fused pass (fixed: results do not depend on batching)

enum Dtype : int32_t { DT_F32 = 0, DT_BF16 = 1 };

// Per-matrix scalar slots (fp32) in DevMat::scal.
enum Scalar : int {
  SC_XNORM2 = 0,   // ||X||_F^2 of the NS source
  SC_SCALE,        // 1 / (||D * T||_F + ns_eps): scale applied by the prologue
  SC_SIGMA,        // power-iteration estimate of ||X||_2
  SC_WNORM2,       // ||W||_F^2
  SC_UNORM2,       // ||U||_F^2
  SC_VNORM2,       // ||U - kappa X||_F^2
  SC_KAPPA,        // (contra / 2) / max(sigma, 1e-7)
  SC_ALPHA,        // final scale of (U - kappa X)
  SC_PNORM,        // ||w|| of the last power step
  SC_COUNT = 16
};

// Per-matrix integer state slots in DevMat::ist.
enum IState : int {
  IS_PSTEPS = 0,   // power steps done
  IS_RESTART,      // 1 once the ones start vector was replaced
  IS_COUNT = 4
};

struct DevMat {
  // caller buffers
  const void* g;  int64_t ld_g;  int32_t dt_g;   // grad or polar input
  float* m;       int64_t ld_m;                   // momentum (fp32), may be null
  void* w;        int64_t ld_w;  int32_t dt_w;   // weight, may be null
  void* uo;       int64_t ld_uo; int32_t dt_uo;  // update_out / polar output
  // shape
  int32_t rows, cols, s, L, s_pad, L_pad;
  int32_t tall;     // rows > cols: the NS iterate is the transpose of storage
  int32_t square;
  int32_t aurora;   // diagonal preconditioner on the long side
  int32_t ns_t;     // DT_F32 or DT_BF16: type of xn, x, xt, a, b
  int32_t n_rt, n_ct;   // ceil(rows / kStreamRows), ceil(cols / kStreamCols)
  int32_t n_seg;        // ceil(cols / kSegCols): streaming tiles are n_rt x n_seg
  int32_t n_rmv;        // partial w rows of the power step: ceil(rows / kRmvRows), fused: ceil(rows / kFusedPart)
  int32_t wband;        // rows per block of the fused pass (a multiple of kFusedPart)
  // workspace
  void* xn;
  void* x[2];
  void* xt[2];
  void* a;
  void* b;
  float* rowpart;   // rows x n_seg   : row sums of squares per tile segment
  float* colpart;   // n_rt x cols    : column sums of squares per row tile
  float* rowsq;     // rows
  float* colsq;     // cols
  float* rho;       // L : long-side norms of the NS source (unclamped)
  float* dvec;      // L : Aurora preconditioner D
  float* pu;        // rows : u = X v
  float* pv;        // cols : v
  float* pwpart;    // n_rmv x cols : partial w per row band
  float* tailpart;  // n_rt * n_seg * 4 : partial tail sums per streaming tile
  float* linepart;  // 2 * (ceil(rows/256) + (rows < cols ? ceil(cols/256) : 0)): per-block norm
                    // partials of the line sums; reused for the blocks of ||w||^2
  float* scal;      // SC_COUNT
  int32_t* ist;     // IS_COUNT
};

// One output tile of a Newton-Schulz product.
struct TileItem {
  uint16_t mat;   // index into the launch's DevMat array
  uint16_t tm;    // tile row
  uint16_t tn;    // tile column
  uint16_t pad;
};

// Matrices taking part in one streaming launch: blocks [off[i], off[i+1])
// work on matrix mat[i].
struct LaunchList {
  int32_t n;
  const int32_t* off;   // n + 1
  const int32_t* mat;   // n
};

enum GemmMode : int { GM_GRAM = 0, GM_SQ = 1, GM_BX = 2 };

}  // namespace muon
