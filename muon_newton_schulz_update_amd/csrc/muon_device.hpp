// Device-side descriptors shared by the libmuon kernels and the host planner.
//
// Layout of one matrix's work in HBM (all row-major, 256-byte aligned):
//   xn      rows x cols, ld = cols, NS type: the blended (Nesterov) update X
//   x[2]    s_pad x L_pad, ld = L_pad: Newton-Schulz iterate, ping-pong
//   xt[2]   L_pad x s_pad, ld = s_pad: its transpose, written by the same
//           epilogue, so every product of the iteration reads both operands
//           with the reduction index contiguous ("NT" form)
//   sq[5]   s_pad x s_pad: the short-side matrices of a block of iterations
//           (roles SQ_A .. SQ_Q1 below)
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

// Element types; DT_F8 (OCP e4m3) only names the fp8 form of a Gram launch.
enum Dtype : int32_t { DT_F32 = 0, DT_BF16 = 1, DT_F8 = 2 };

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
  SC_F8Q,          // power-of-two scale q of the pass's fp8 copy of X0 (|q X0| <= 448)
  SC_F8INV2,       // 1 / q^2: undoes the scale in the fp8 Gram's epilogue
  SC_COUNT = 16
};

// Per-matrix integer state slots in DevMat::ist.
enum IState : int {
  IS_PSTEPS = 0,   // power steps done
  IS_RESTART,      // 1 once the ones start vector was replaced
  IS_COUNT = 4
};

// Matrix-core products. Every product reads two row-major operands with the
// reduction index contiguous (C[m][n] = sum_k P[m][k] Q[n][k]):
//   GM_GRAM  A = X X^T            (P = Q = x[cur])          upper tiles, mirrored
//   GM_SQ    B' = b A + c A A + a I (P = Q = sq[rp])        upper tiles, mirrored
//   GM_SYM   C = P Q              (sq[rp], sq[rq]; both symmetric and
//                                  commuting, so C is too)  upper tiles, mirrored
//   GM_BX    X' = P X             (P = sq[rp], Q = xt[cur]) writes X' and X'^T
enum GemmMode : int { GM_GRAM = 0, GM_SQ = 1, GM_SYM = 2, GM_BX = 3 };

// Roles of the short-side buffers DevMat::sq.
enum SqRole : int {
  SQ_A = 0,    // A_j, the Gram of the block's iterate, advanced in place
  SQ_B,        // B'_j = a I + b A_j + c A_j^2 (j >= 1)
  SQ_T,        // B'_j A_j
  SQ_Q0,       // Q_j = B'_{j-1} ... B'_0, ping-pong (B'_0 itself is written here)
  SQ_Q1,
  SQ_COUNT
};

// Launch flags of GM_BX (in the roles word, bits 12 and 13): the last X' = Q X
// of a pass writes only the orientation its reader uses; which one depends
// on whether this is the matrix's last pass (the last Aurora pass, or the
// only pass of a matrix without the preconditioner).
constexpr int NS_LAST_BX = 1 << 12;
constexpr int NS_LAST_PASS = 1 << 13;
// Bit 14 of a GM_GRAM or GM_BX launch: the pass's first Gram or first
// X' = Q X. For a matrix with DevMat::x0n that X' = Q X reads the stored
// blended update instead of X0^T and scales its output columns by the
// prologue's factor (scale D_l); for one with DevMat::x0g that Gram reads it
// instead of X0 and scales its output by scale^2.
constexpr int NS_FIRST = 1 << 14;
// A launch of two independent short-side products carries the second
// product's roles in bits 16-27; its tiles are the ones whose TileItem::pad
// is 1.
inline constexpr int ns_roles(int rp, int rq, int rd) { return rp | (rq << 4) | (rd << 8); }

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
  int32_t aurora;   // diagonal preconditioner (on the long side unless eq_short)
  int32_t eq_short; // aurora on a wide matrix's own rows (the short side)
  int32_t ns_t;     // DT_F32 or DT_BF16: type of xn, x, xt, sq
  int32_t n_rt, n_ct;   // ceil(rows / kStreamRows), ceil(cols / kStreamCols)
  int32_t n_seg;        // ceil(cols / kSegCols): streaming tiles are n_rt x n_seg
  int32_t n_rmv;        // partial w rows of the power step: ceil(rows / kRmvRows), fused: ceil(rows / kFusedPart)
  int32_t wband;        // rows per block of the fused pass (a multiple of kFusedPart)
  // workspace
  void* xn;
  void* x[2];
  void* xt[2];
  void* x8;         // fp8 q X0 for the first Gram, or null: L_pad/64 panels of s_pad x 64 bytes (column c of
                    // row r at ((c/64) s_pad + r) 64 + c%64), written by the pass prologue
  void* sq[SQ_COUNT];   // short-side matrices by role (a matrix with one-iteration blocks aliases SQ_Q0 to SQ_B
                        // and leaves SQ_T, SQ_Q1 unused)
  int32_t fin;          // x[fin] / xt[fin] holds the result of the last pass (blocks per pass, mod 2)
  int32_t bad;          // 0 as uploaded; k_check_finite sets it when an input element is NaN or Inf
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
  float* lsq;       // (s_pad / 64) x L_pad, or null: the last product of each non-final Aurora pass of a
                    // matrix equilibrated on its long side writes, per 64-row band and long-side line
                    // (a column of X'), the sum of squares of the line's stored entries in that band
  float* linepart;  // 3 * (ceil(rows/256) + (rows < cols ? ceil(cols/256) : 0)): per-block norm
                    // partials of the line sums and the largest line norm^2; reused for the blocks
                    // of ||w||^2
  float* scal;      // SC_COUNT
  int32_t* ist;     // IS_COUNT
  // Fused tail (muon_update, bf16 NS type; null otherwise): the epilogue of
  // the matrix's final X' = Q X takes the tail's sums from the values it
  // stores, and a read-only pass takes ||W||^2, so no kernel reads U and X
  // before the tail's single pass.
  float* ftail;     // cdiv(rows,64) x cdiv(cols,64) x 2: per 64 x 64 block of the storage frame, ||U||^2 and
                    // <U, X> (X the stored blended update)
  float* frow;      // cdiv(cols,64) x rows: per storage row and 64-column block, the block's part of
                    // (X / ||X||_F) v, v the last power-iteration vector (sigma = ||X v||)
  float* fwp;       // n_rt x n_seg: ||W||^2 per streaming tile, from k_wnorm (tailpart is taken by
                    // the D update in between)
  int32_t x0n;      // a tall bf16 matrix of muon_update with rows and cols multiples of kTile: X0^T is
                    // scale D o X row by row, so the pass prologue writes only X0 and each pass's first
                    // X' = Q X reads xn (ld = cols = s_pad) and applies scale D_l to output column l
  int32_t x0g;      // a wide or square bf16 matrix of muon_update without the preconditioner, rows and
                    // cols multiples of kTile: X0 = scale X, so the pass prologue writes only X0^T and the
                    // pass's first Gram reads xn (ld = cols = L_pad) and scales A by scale^2
  int32_t ftx;      // per call: the epilogue also takes <U, X> and the sigma parts (contra != 0)
  int32_t ftw;      // per call: k_wnorm takes ||W||^2 (a weight is given)
};

// Diagonal tiles of the symmetric products (GM_GRAM, GM_SQ, GM_SYM): the
// stored result is the upper triangle and its mirror, so the 32x32 blocks
// wholly below the diagonal need no work. Keep<OFF, MI, NI> names the blocks
// a wave of MI x NI blocks computes, OFF being its row origin less its column
// origin in 32-row blocks (kDiagFull: every block): block (mi, ni) is left
// out when ni < mi + OFF. Rows and columns with no block left need no
// fragments. Plain constexpr code, shared by the engine and a host test.
constexpr int kDiagFull = -1;
template <int OFF, int MI, int NI>
struct Keep {
  static constexpr bool blk(int mi, int ni) { return !(OFF >= 0 && ni < mi + OFF); }
  static constexpr bool row(int mi) { return !(OFF >= 0 && mi + OFF >= NI); }
  static constexpr bool col(int ni) { return !(OFF >= 0 && ni < OFF); }
  static constexpr int blocks() {
    int n = 0;
    for (int mi = 0; mi < MI; ++mi)
      for (int ni = 0; ni < NI; ++ni) n += blk(mi, ni) ? 1 : 0;
    return n;
  }
  static constexpr int frags() {
    int n = 0;
    for (int mi = 0; mi < MI; ++mi) n += row(mi) ? 1 : 0;
    for (int ni = 0; ni < NI; ++ni) n += col(ni) ? 1 : 0;
    return n;
  }
};
// The K-loop form a wave (wm, wn) of a diagonal tile runs: its offset from
// the diagonal where that form is compiled (0 and 2, or NI for a wave wholly
// below it), kDiagFull otherwise (full work is always correct). The engine's
// layouts (8 waves of 2 x 4 blocks, 4 of 4 x 4, 4 of 2 x 2) meet offsets
// below 0, 0, 2 and NI or more.
constexpr int diag_form(int wm, int wn, int MI, int NI) {
  const int off = wm * MI - wn * NI;
  return off < 0 ? kDiagFull : off >= NI ? NI : (off == 0 || off == 2) ? off : kDiagFull;
}

// One output tile of a Newton-Schulz product.
struct TileItem {
  uint16_t mat;   // index into the launch's DevMat array
  uint16_t tm;    // tile row
  uint16_t tn;    // tile column
  uint16_t pad;   // 1: a tile of the launch's second product (roles bits 16-27)
};

// Matrices taking part in one streaming launch: blocks [off[i], off[i+1])
// work on matrix mat[i].
struct LaunchList {
  int32_t n;
  const int32_t* off;   // n + 1
  const int32_t* mat;   // n
};



}  // namespace muon
