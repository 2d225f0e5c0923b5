// libmuon C-ABI: handle, planner and launch sequences.
//
// The planner turns a batch of matrices into (1) a workspace layout in one
// device allocation (see muon_device.hpp), (2) per-launch block lists for the
// streaming kernels and (3) tile lists for the Newton-Schulz products. A plan
// depends only on the batch's shapes and types, so it is cached; per call only
// the descriptor array (caller pointers) is re-uploaded, and only if it changed.
//
// Sequence of one muon_update (Aurora record page, www.xxmr.cn/news/295280,
// section 组合优化栈 and the pseudocode in Aurora 的迭代伪代码):
//   momentum + Nesterov + row partial norms [-> ||W||^2, fused tail]
//   -> norm lines (row and column norms, rho, D0) -> per-matrix scalars
//      (||X||, prologue scale)
//   -> power iteration (power_steps + 1 rounds of w = X^T X v, one read of X
//      in a fused pass, or X v then X^T u for matrices wider than
//      kFusedCols; ||w||, v = w/||w||; then X v and sigma, except for the
//      fused tail, whose final product takes X v)
//   -> for each Aurora pass: prologue (scale * D o T, one or both
//      orientations), ns_steps in blocks of iterations {A = XX^T, B' = bA +
//      cA^2 + aI, ..., X' = Q X}, D update between passes
//   -> tail reduce (or, fused tail, the final product's sums and sigma's row
//      sums) -> tail finalise (Contra, Frobenius restore, aspect, floor)
//   -> tail apply (update_out, W -= lr V).
#include <hip/hip_runtime.h>
#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "../../include/libmuon.h"
#include "muon_device.hpp"
#include "validate.hpp"

namespace muon {

hipError_t launch_ns_gemm(int ns_t, const DevMat* mats, const TileItem* items, int n_items, int mode, int cur,
                          int roles, float ca, float cb, float cc, int variant, int tile, hipStream_t st);
hipError_t launch_momentum_stats(const DevMat* m, LaunchList L, int nblk, int nesterov_pass, float mu, int nesterov,
                                 int sgd, hipStream_t st);
hipError_t launch_check_finite(DevMat* m, LaunchList L, int nblk, int upd, hipStream_t st);
hipError_t launch_wnorm(const DevMat* m, LaunchList L, int nblk, hipStream_t st);
hipError_t launch_norms_lines(DevMat* m, LaunchList L, int nblk, float pp_eps, hipStream_t st);
hipError_t launch_norms_scalars(DevMat* m, LaunchList L, int nblk, float ns_eps, int init_power, hipStream_t st);
hipError_t launch_prologue(int ns_t, const DevMat* m, LaunchList L, int nblk, int use_xn, hipStream_t st);
hipError_t launch_aurora_dupdate(int ns_t, DevMat* m, LaunchList L, int nblk, float pp_eps, float pp_beta,
                                 hipStream_t st);
hipError_t launch_aurora_scale(DevMat* m, LaunchList L, int nblk, float ns_eps, hipStream_t st);
hipError_t launch_aurora_dfinish(DevMat* m, LaunchList L, int nblk, float pp_eps, float pp_beta, hipStream_t st);
hipError_t launch_power_matvec(const DevMat* m, LaunchList L, int nblk, int steps, int final_pass, hipStream_t st);
hipError_t launch_power_rmatvec(const DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st);
hipError_t launch_power_fused(int ns_t, const DevMat* m, LaunchList L, int nblk, int steps, int max_cols,
                              hipStream_t st);
hipError_t launch_power_wsum(DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st);
hipError_t launch_power_normalize(DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st);
hipError_t launch_power_sigma(DevMat* m, LaunchList L, int nblk, float contra, hipStream_t st);
hipError_t launch_tail_reduce(const DevMat* m, LaunchList L, int nblk, hipStream_t st);
hipError_t launch_tail_rows(const DevMat* m, LaunchList L, int nblk, hipStream_t st);
hipError_t launch_tail_finalize(DevMat* m, LaunchList L, int nblk, float target_uw, float contra, hipStream_t st);
hipError_t launch_tail_apply(const DevMat* m, LaunchList L, int nblk, float lr, int copy_only, hipStream_t st);
size_t static_scratch_bytes();
hipError_t static_scratch_address(int dev, void** out);

// Pinned staging for the launch tables of muon_update_static, allocated with
// the handle: the largest table set a static call may upload.
constexpr size_t kStaticStageBytes = size_t(1) << 20;

namespace {

enum Kind { KIND_NS = 0, KIND_AURORA = 1, KIND_UPDATE = 2 };

constexpr size_t kAlign = 256;
constexpr int kSuperM = 4, kSuperN = 8;   // NS tile raster (one XCD's 32 CUs)
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
// Blocks of the norm-line kernel: one per 256 rows, plus one per 256 columns
// of a wide matrix (its column norms are lines too).
inline int line_blocks(int rows, int cols) { return cdiv(rows, 256) + (rows < cols ? cdiv(cols, 256) : 0); }
inline int esz(int dt) { return dt == DT_BF16 ? 2 : 4; }

struct MatInfo {
  int user;                  // index in the caller's batch
  int rows, cols, s, L, s_pad, L_pad;
  bool tall, square, aurora, eq_short;
  bool f8;                   // the first Gram of each pass on fp8 operands (MUON_FLAG_FP8_GRAM)
  int block;                 // Newton-Schulz iterations per block (1 for squares)
  int chain[2];              // launch chain (0 or 1) in each pass group (see build_plan)
  int ns_t;
  int n_rt, n_ct, n_seg, n_rmv, wband;
  bool band_d;               // Aurora on the long side with later passes: D from the last product's band sums
  bool ft;                   // fused tail (see fused_tail)
  bool x0n;                  // X0^T read from xn by each pass's first X' = Q X (see tall_x0_direct)
  bool x0g;                  // X0 read from xn by the pass's first Gram (see tall_x0_direct)
  size_t o_lsq, o_ftail, o_frow, o_fwp;
  size_t o_xn, o_x[2], o_xt[2], o_x8, o_sq[SQ_COUNT], o_rowpart, o_colpart, o_rowsq, o_colsq, o_rho, o_dvec, o_pu, o_pv,
      o_pwpart, o_tailpart, o_linepart, o_scal, o_ist;
};

// Newton-Schulz iterations per block of a rectangular matrix. A block stays
// on the short side until its last product, so it needs 3 s^2 L + (4 r - 3)
// s^3 flops for r iterations instead of r (3 s^2 L + s^3); a square matrix
// gains nothing and keeps one iteration per block, and so does a short side
// below kBlockMinShort (its products are few tiles, bound by launch count).
// Within a block, Q = B'_{r-1} ... B'_0 has eigenvalues prod_j f(sigma_j),
// f(sigma) = a + b sigma^2 + c sigma^4; stored in bf16, its entries carry
// rounding relative to its largest eigenvalue, so the directions with the
// smallest lose (max f / min f)^r of their precision. The block length is
// the largest r <= kDefaultBlock with that ratio at most kMaxBlockSpread over
// sigma in [0, 1] (the page's polynomial: ratio 2, r = 4; the classic one,
// 3.4445 / 0.701 = 4.9, gets r = 1). MUON_NS_BLOCK (1..8, read when a plan is
// built) forces a length for every rectangular matrix.
constexpr int kDefaultBlock = 4;
constexpr double kMaxBlockSpread = 16.0;
constexpr int kBlockMinShort = 512;

// The fused power pass takes matrices up to kFusedCols columns whose rows are
// whole 16-byte chunks of the NS type (it loads 8-element chunks only); it
// depends on the matrix alone, never on the rest of the batch.
inline bool fused_power(const MatInfo& m) {
  return m.cols <= kFusedCols && ((size_t)m.cols * (m.ns_t == DT_BF16 ? 2 : 4)) % 16 == 0;
}

// Block length for the rectangular matrices of a call (see kDefaultBlock);
// *forced is set when MUON_NS_BLOCK gives it.
int rect_block(const muon_config& cfg, bool* forced) {
  *forced = false;
  if (const char* v = getenv("MUON_NS_BLOCK")) {
    *forced = true;
    return std::min(8, std::max(1, atoi(v)));
  }
  double lo = 1e300, hi = 0;
  for (int i = 0; i <= 1000; ++i) {
    const double x = i / 1000.0, x2 = x * x;
    const double f = fabs((double)cfg.ns_a + (double)cfg.ns_b * x2 + (double)cfg.ns_c * x2 * x2);
    lo = std::min(lo, f);
    hi = std::max(hi, f);
  }
  if (!(lo > 0) || hi / lo <= 1.0) return lo > 0 ? kDefaultBlock : 1;
  const int r = (int)floor(log(kMaxBlockSpread) / log(hi / lo) + 1e-9);
  return std::min(kDefaultBlock, std::max(1, r));
}

// Fused tail: the matrices of a muon_update call with the bf16 NS type take
// the tail's sums in the epilogue of their final X' = Q X (||U||^2, <U, X>
// and the parts of sigma = ||X v||) and in a read-only pass over W
// (||W||^2), so the tail reads U, X and W once, in its single pass, and the
// power iteration ends without its last X v. fp32 matrices keep the tail's
// reduction pass and the last X v (the fp32 engine's epilogue stages fp32
// slabs). MUON_FUSED_TAIL=0 (read when a plan is built) turns it off.
inline bool fused_tail(int kind, int ns_t) {
  if (kind != KIND_UPDATE || ns_t != DT_BF16) return false;
  const char* v = getenv("MUON_FUSED_TAIL");
  return !(v && atoi(v) == 0);
}

// A tall matrix's X0^T = scale D o T has the storage orientation of T, the
// blended update xn, row by row: when its rows and columns are multiples of
// the tile (no padding, so xn is laid out as xt[0] would be), the pass
// prologue writes only X0 and the pass's first X' = Q X reads xn, applying
// scale D_l to its output column l in the epilogue (bf16 NS type, muon_update
// calls, whose prologue reads xn). MUON_TALL_X0=0 (read when a plan is built)
// turns it off. Likewise a wide or square matrix without the preconditioner
// has X0 = scale X in the storage orientation: its prologue writes only X0^T
// and its pass's first Gram reads xn and scales A by scale^2.
inline bool tall_x0_direct(int kind, int ns_t, int rows, int cols) {
  if (kind != KIND_UPDATE || ns_t != DT_BF16 || rows % kTile || cols % kTile) return false;
  const char* v = getenv("MUON_TALL_X0");
  return !(v && atoi(v) == 0);
}

// Host copy of one LaunchList: offset of its int arrays in the meta buffer.
struct HostList {
  int n = 0;
  int nblk = 0;
  size_t off_off = 0, off_mat = 0;  // byte offsets into meta
  double bytes = 0;                 // algorithmic bytes of one launch over it
  int max_cols = 0;                 // widest matrix in the list (the fused power pass sizes its LDS by it)
};

struct GemmList {
  int n = 0;
  int tile = kTile;                 // output tile edge of its items (256, or 128 for small launches)
  size_t off = 0;                   // byte offset of TileItem array in meta
  double counted_iter = 0;          // 4 s^2 L + 2 s^3 summed over its matrices: one standard iteration
  double executed = 0;              // flops the tiles of one launch issue (padding, whole diagonal tiles)
  double algorithmic = 0;           // flops one launch needs (upper half of a symmetric result)
};
// tile lists: Gram, short-side products, X' = Q X, and the short-side list
// twice (items of the second copy marked), for a launch of two independent
// short-side products
enum { LIST_GRAM = 0, LIST_SQ = 1, LIST_BX = 2, LIST_SQ2 = 3 };

// A product launch with fewer 256-tiles than this uses 128-tiles: with one
// 256-tile workgroup per CU such a launch is a few rounds of workgroups and
// its last round leaves CUs idle, while 128-tiles (two workgroups per CU)
// cover the CUs in finer steps. MUON_NS_TILE=128 or 256 forces one size.
constexpr int kSmallLaunchTiles = 768;
constexpr int kSplitTiles = 1024;   // a one-kind pass group splits into two chains below this (build_plan)
// Fused power pass: band rows go down from kRmvRows to kFusedMinBand until a
// launch has at least kFusedMinBlocks blocks (four per CU).
constexpr int kFusedMinBand = kFusedPart;
constexpr int kFusedMinBlocks = 1024;

struct Plan {
  int kind = 0;
  std::vector<MatInfo> mats;
  size_t ws_bytes = 0;
  int passes = 1;
  bool any_aurora = false;
  // lists
  HostList stream, permat, lines, colblk, matvec, ascale;
  HostList stream_r;                      // the tail's reduction pass: streaming tiles of the matrices without the fused tail
  HostList stream_f;                      // the weight-norm pass: streaming tiles of the fused-tail matrices
  HostList frows;                         // fused tail: sigma's row sums, one block per 256 rows
  HostList fused[2];                      // power rounds: fused X^T X v pass, one list per NS type
  HostList matvec_w, rmatvec_w;           // X v + X^T u for matrices wider than kFusedCols
  HostList prologue[2][2];  // [group: 0 all, 1 aurora][ns_t]
  HostList dupdate[2];      // [ns_t]: D update reading the pass's result (matrices equilibrated on the short side)
  HostList dfinish;         // D update from the last product's band sums (the others)
  GemmList gemm[2][2][2][4];   // [pass group][chain][ns_t][list]
  int block = kDefaultBlock;    // iterations per block of a rectangular matrix
  // Each Newton-Schulz pass runs as two chains of launches, independent of
  // each other (see build_plan): chain_block[g][c] iterations per block in
  // chain c of pass group g; two_chains[g] when both have matrices, side[g]
  // when the second stream pays (every product launch of the group under
  // kSmallLaunchTiles 256-tiles)
  int chain_block[2][2] = {{1, kDefaultBlock}, {1, kDefaultBlock}};
  bool two_chains[2] = {false, false}, side[2] = {false, false};
  bool fp8 = false;             // MUON_FLAG_FP8_GRAM: the blocked bf16 matrices' first Gram is fp8
  // device meta: DevMat array followed by the list arrays
  std::vector<uint8_t> meta_host;  // list part (static)
  size_t meta_devmat_bytes = 0;
  void* meta_dev = nullptr;
  std::vector<DevMat> last_devmat;
  bool devmat_valid = false;
  uint64_t last_use = 0;
  std::vector<std::pair<size_t, size_t>> regions;   // workspace (offset, bytes) handed out, for the plan check
};

std::string plan_key(int kind, int pp, bool wide_rows, bool fp8, int block, bool forced, int n,
                     const muon_matrix* in) {
  std::string k;
  k.reserve(16 + n * 12);
  char buf[80];
  snprintf(buf, sizeof(buf), "%d/%d/%d/%d/%d/%d/%d|", kind, pp, (int)wide_rows, (int)fp8, block, (int)forced, n);
  k += buf;
  for (int i = 0; i < n; ++i) {
    snprintf(buf, sizeof(buf), "%lld,%lld,%d;", (long long)in[i].rows, (long long)in[i].cols, (int)in[i].dtype);
    k += buf;
  }
  return k;
}

struct ProfRec {
  hipEvent_t a, b;
  int cls;  // 0 gemm, 1 stream, 2 aux (prologue, D update)
  double amount, amount2, amount3;
  int count;  // launches between the two events (consecutive on the stream)
};

}  // namespace
}  // namespace muon

struct muon_handle {
  int device = 0;
  int ns_variant = 0;        // Newton-Schulz tile layout (MUON_NS_VARIANT; 0 = 8 waves, 1 = 4 waves)
  hipStream_t stream = nullptr;
  // second stream (default priority, non-blocking) for chain 0 of the
  // Newton-Schulz passes when the plan runs it beside chain 1, made by the
  // first call that needs it; MUON_NS_SIDE (read at creation): 0 never, 1 in
  // every pass with both chains
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  int side_mode = -1;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  std::map<std::string, std::unique_ptr<muon::Plan>> plans;
  uint64_t tick = 0;
  void* pinned = nullptr;
  int32_t* bad_host = nullptr;   // pinned, kMaxBatch flags: the input check's per-matrix results
  // ROCTx ranges per phase (MUON_ROCTX=1 at handle creation): the SDK's
  // push/pop, looked up with dlopen so the library has no link dependency
  int (*rx_push)(const char*) = nullptr;
  int (*rx_pop)() = nullptr;
  void* rx_lib = nullptr;
  size_t pinned_bytes = 0;
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  // muon_update_static: the device's static scratch and the handle's table staging
  void* scratch = nullptr;
  void* static_stage = nullptr;
  hipEvent_t static_done = nullptr;
  bool static_pending = false;
  bool in_static = false;    // inside muon_update_static: no profiling events
  std::string err;
  // profiling
  bool prof = false;
  std::vector<hipEvent_t> ev_pool;
  std::vector<muon::ProfRec> recs;
  muon_profile acc{};
};

namespace muon {
namespace {

muon_status set_err(muon_handle* h, muon_status code, const std::string& m) {
  if (h) h->err = m;
  return code;
}

#define HIP_TRY(h, expr)                                                                       \
  do {                                                                                         \
    hipError_t e_ = (expr);                                                                    \
    if (e_ != hipSuccess)                                                                      \
      return set_err((h), MUON_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));    \
  } while (0)

// ---------------------------------------------------------------------------
// Planning
// ---------------------------------------------------------------------------
void add_list(std::vector<uint8_t>& meta, HostList& L, const std::vector<int>& mats, const std::vector<int>& blocks) {
  L.n = (int)mats.size();
  std::vector<int32_t> off(mats.size() + 1, 0);
  for (size_t i = 0; i < mats.size(); ++i) off[i + 1] = off[i] + blocks[i];
  L.nblk = off.back();
  size_t pos = align_up(meta.size());
  L.off_off = pos;
  meta.resize(pos + off.size() * 4);
  memcpy(meta.data() + pos, off.data(), off.size() * 4);
  pos = align_up(meta.size());
  L.off_mat = pos;
  meta.resize(pos + std::max<size_t>(1, mats.size()) * 4);
  if (!mats.empty()) memcpy(meta.data() + pos, mats.data(), mats.size() * 4);
}

void add_gemm(std::vector<uint8_t>& meta, GemmList& G, std::vector<TileItem>& items) {
  G.n = (int)items.size();
  size_t pos = align_up(meta.size());
  G.off = pos;
  meta.resize(pos + std::max<size_t>(1, items.size()) * sizeof(TileItem));
  if (!items.empty()) memcpy(meta.data() + pos, items.data(), items.size() * sizeof(TileItem));
}

// A plan depends only on the call kind, the pass count, the wide-rows option
// and the inputs' shapes and element types (exactly what plan_key holds):
// caller pointers, strides, weights and outputs go into the per-call
// descriptors.
std::unique_ptr<Plan> build_plan(int kind, int pp, bool wide_rows, bool fp8, int block, bool forced, int n,
                                 const muon_matrix* in, bool may_split) {
  auto P = std::make_unique<Plan>();
  P->kind = kind;
  P->block = block;
  P->fp8 = fp8;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 1));
    P->regions.emplace_back(o, bytes);
    return o;
  };
  for (int i = 0; i < n; ++i) {
    if (in[i].rows == 0 || in[i].cols == 0) continue;
    MatInfo m{};
    m.user = i;
    m.rows = (int)in[i].rows;
    m.cols = (int)in[i].cols;
    m.s = std::min(m.rows, m.cols);
    m.L = std::max(m.rows, m.cols);
    m.s_pad = cdiv(m.s, kTile) * kTile;
    m.L_pad = cdiv(m.L, kTile) * kTile;
    m.tall = m.rows > m.cols;
    m.square = m.rows == m.cols;
    m.aurora = (kind != KIND_NS) && !m.square && pp > 0;
    m.eq_short = m.aurora && wide_rows && m.rows < m.cols;
    m.ns_t = in[i].dtype == MUON_BF16 ? DT_BF16 : DT_F32;
    m.n_rt = cdiv(m.rows, kStreamRows);
    m.n_ct = cdiv(m.cols, kStreamCols);
    m.n_seg = cdiv(m.cols, kSegCols);
    m.wband = kRmvRows;
    m.n_rmv = cdiv(m.rows, kRmvRows);
    const size_t e = esz(m.ns_t);
    const size_t nsl = (size_t)m.s_pad * m.L_pad * e;
    m.o_xn = kind == KIND_UPDATE ? take((size_t)m.rows * m.cols * e) : 0;
    m.block = m.square || (!forced && m.s < kBlockMinShort) ? 1 : P->block;
    // fp8 first Gram: bf16 matrices that run blocks (their first Gram is the
    // long K = L product whose sums average the operands' rounding)
    m.f8 = fp8 && m.ns_t == DT_BF16 && m.block > 1;
    m.o_x8 = m.f8 ? take((size_t)m.s_pad * m.L_pad) : 0;
    m.o_x[0] = take(nsl);
    m.o_x[1] = take(nsl);
    m.o_xt[0] = take(nsl);
    m.o_xt[1] = take(nsl);
    const size_t ssq = (size_t)m.s_pad * m.s_pad * e;
    m.o_sq[SQ_A] = take(ssq);
    m.o_sq[SQ_B] = take(ssq);
    if (m.block > 1) {
      m.o_sq[SQ_T] = take(ssq);
      m.o_sq[SQ_Q0] = take(ssq);
      m.o_sq[SQ_Q1] = take(ssq);
    } else {   // one iteration per block: B'_0 is the only factor (Q0 = B); T and Q1 unused
      m.o_sq[SQ_T] = m.o_sq[SQ_Q0] = m.o_sq[SQ_Q1] = m.o_sq[SQ_B];
    }
    m.o_rowpart = take((size_t)m.rows * m.n_seg * 4);
    m.o_colpart = take(m.rows < m.cols ? (size_t)m.n_rt * m.cols * 4 : 4);
    m.o_rowsq = take((size_t)m.rows * 4);
    m.o_colsq = take((size_t)m.cols * 4);
    m.o_rho = take((size_t)m.L * 4);
    m.o_dvec = take((size_t)m.L * 4);
    m.o_pu = take((size_t)m.rows * 4);
    m.o_pv = take((size_t)m.cols * 4);
    // partial w rows: one per kRmvRows rows, or per kFusedPart rows for the fused pass
    m.o_pwpart = take(kind == KIND_UPDATE ? (size_t)cdiv(m.rows, fused_power(m) ? kFusedPart : kRmvRows) *
                                                m.cols * 4
                                          : 4);
    // tail partials (4 per streaming tile); the D update's per-block sums and maxima
    m.o_tailpart = take(std::max((size_t)m.n_rt * m.n_seg * 4, (size_t)2 * cdiv(m.L, 4)) * 4);
    // per line block: row-sum total, (D rho)^2 total, largest line norm^2
    m.o_linepart = take((size_t)3 * line_blocks(m.rows, m.cols) * 4);
    // the D update of a long-side Aurora matrix with passes after the first
    // takes its line sums from the pass's last product (per 64-row band)
    m.band_d = m.aurora && !m.eq_short && pp > 1;
    m.o_lsq = m.band_d ? take((size_t)(m.s_pad / 64) * m.L_pad * 4) : 0;
    m.ft = fused_tail(kind, m.ns_t);
    m.x0n = m.tall && tall_x0_direct(kind, m.ns_t, m.rows, m.cols);
    m.o_ftail = m.ft ? take((size_t)cdiv(m.rows, 64) * cdiv(m.cols, 64) * 2 * 4) : 0;
    m.o_frow = m.ft ? take((size_t)cdiv(m.cols, 64) * m.rows * 4) : 0;
    m.o_fwp = m.ft ? take((size_t)m.n_rt * m.n_seg * 4) : 0;
    m.o_scal = take(SC_COUNT * 4);
    m.o_ist = take(IS_COUNT * 4);
    m.x0g = !m.tall && !m.aurora && tall_x0_direct(kind, m.ns_t, m.rows, m.cols);
    if (m.aurora) P->any_aurora = true;
    P->mats.push_back(m);
  }
  P->ws_bytes = off;
  P->passes = P->any_aurora ? pp : 1;

  // Chains, per pass group (0: every matrix, 1: the Aurora matrices in the
  // passes after the first). The one-iteration matrices (chain 0) and those
  // with blocks (chain 1) never read each other's results inside a pass, so
  // the two chains' launches may run side by side (on the second stream,
  // when the launches are small; see two_chains and side below). A group
  // with only one of the two kinds and small launches is split into two
  // chains of about equal work (largest first, each to the lighter chain)
  // when the second stream may be used.
  for (int g = 0; g < 2; ++g) {
    P->chain_block[g][0] = 1;
    P->chain_block[g][1] = block;
    std::vector<int> members;
    bool has[2] = {false, false};
    long lists[2][2][3] = {};   // [kind][ns_t][list], in 256-tiles
    for (int i = 0; i < (int)P->mats.size(); ++i) {
      MatInfo& m = P->mats[i];
      const int kind = m.block > 1 ? 1 : 0;
      m.chain[g] = kind;
      if (g == 1 && !m.aurora) continue;
      members.push_back(i);
      has[kind] = true;
      const long ts = m.s_pad / kTile, tl = m.L_pad / kTile;
      lists[kind][m.ns_t][LIST_GRAM] += ts * (ts + 1) / 2;
      lists[kind][m.ns_t][LIST_SQ] += ts * (ts + 1) / 2;
      lists[kind][m.ns_t][LIST_BX] += ts * tl;
    }
    if (!may_split || has[0] == has[1] || members.size() < 2) continue;
    const int kind = has[1] ? 1 : 0;
    long n256 = 0;
    for (int t = 0; t < 2; ++t)
      for (int li = 0; li < 3; ++li) n256 = std::max(n256, lists[kind][t][li]);
    // split when the lists are under kSplitTiles 256-tiles: the halves then
    // run as 128-tile launches side by side. Measured: the GPT-2-124M set's
    // second pass (864 tiles in its widest list) 6.17 -> 5.99 ms per step;
    // one 3.8B layer's (1248, its X' = Q X on 256-tiles with K = 3072)
    // 15.15 -> 16.03, so larger lists stay whole.
    if (n256 >= kSplitTiles) continue;
    auto cost = [&](int i) { return (double)P->mats[i].s_pad * P->mats[i].s_pad * P->mats[i].L_pad; };
    std::stable_sort(members.begin(), members.end(), [&](int a, int b) { return cost(a) > cost(b); });
    double load[2] = {0.0, 0.0};
    long half[2][2][3] = {};   // [chain][ns_t][list], in 256-tiles
    std::vector<int> to(members.size());
    for (size_t k = 0; k < members.size(); ++k) {
      const MatInfo& m = P->mats[members[k]];
      const int c = load[0] <= load[1] ? 0 : 1;
      to[k] = c;
      load[c] += cost(members[k]);
      const long ts = m.s_pad / kTile, tl = m.L_pad / kTile;
      half[c][m.ns_t][LIST_GRAM] += ts * (ts + 1) / 2;
      half[c][m.ns_t][LIST_SQ] += ts * (ts + 1) / 2;
      half[c][m.ns_t][LIST_BX] += ts * tl;
    }
    // only if both halves' launches are small enough to run side by side
    // (one dominant matrix would leave its chain as large as the whole)
    long hmax = 0;
    for (int c = 0; c < 2; ++c)
      for (int t = 0; t < 2; ++t)
        for (int li = 0; li < 3; ++li) hmax = std::max(hmax, half[c][t][li]);
    if (hmax >= kSmallLaunchTiles) continue;
    P->chain_block[g][0] = P->chain_block[g][1] = kind == 1 ? block : 1;
    for (size_t k = 0; k < members.size(); ++k) P->mats[members[k]].chain[g] = to[k];
  }

  const int nm = (int)P->mats.size();
  std::vector<uint8_t>& meta = P->meta_host;
  P->meta_devmat_bytes = align_up(std::max(1, nm) * sizeof(DevMat));
  meta.assign(P->meta_devmat_bytes, 0);

  std::vector<int> all(nm), blocks(nm);
  for (int i = 0; i < nm; ++i) all[i] = i;
  // streaming tiles
  double bytes_stream = 0;
  for (int i = 0; i < nm; ++i) {
    const MatInfo& m = P->mats[i];
    blocks[i] = m.n_rt * m.n_seg;   // kStreamRows x kSegCols tiles
  }
  add_list(meta, P->stream, all, blocks);
  {
    std::vector<int> ms, bl, fm, fb, ft;
    for (int i = 0; i < nm; ++i) {
      const MatInfo& m = P->mats[i];
      if (!m.ft) { ms.push_back(i); bl.push_back(m.n_rt * m.n_seg); }
      else { fm.push_back(i); fb.push_back(cdiv(m.rows, 256)); ft.push_back(m.n_rt * m.n_seg); }
    }
    add_list(meta, P->stream_r, ms, bl);
    add_list(meta, P->frows, fm, fb);
    add_list(meta, P->stream_f, fm, ft);
  }
  for (int i = 0; i < nm; ++i) blocks[i] = 1;
  add_list(meta, P->permat, all, blocks);
  for (int i = 0; i < nm; ++i) blocks[i] = line_blocks(P->mats[i].rows, P->mats[i].cols);
  add_list(meta, P->lines, all, blocks);
  for (int i = 0; i < nm; ++i) blocks[i] = cdiv(P->mats[i].cols, 256);
  add_list(meta, P->colblk, all, blocks);
  {
    // the final X v of every matrix without the fused tail
    std::vector<int> ms, bl;
    for (int i = 0; i < nm; ++i)
      if (!P->mats[i].ft) { ms.push_back(i); bl.push_back(cdiv(P->mats[i].rows, 16)); }   // 4 waves x 4 rows
    add_list(meta, P->matvec, ms, bl);
  }
  {
    // Power rounds: the matrices fused_power() takes run the fused X^T X v
    // pass, one launch per NS type, widest first; the others take X v then
    // X^T u. A fused block takes a band of rows: the widest of 256, 128, 64
    // that still gives its launch kFusedMinBlocks blocks (a few matrices need
    // narrow bands to fill the CUs; many take wide ones, which spend less on
    // per-block set-up). The partial sums do not depend on the band.
    std::vector<int> wm, wb, wr;
    for (int t = 0; t < 2; ++t) {
      std::vector<int> fm;
      for (int i = 0; i < nm; ++i)
        if (fused_power(P->mats[i]) && P->mats[i].ns_t == t) fm.push_back(i);
      std::stable_sort(fm.begin(), fm.end(), [&](int a, int b) { return P->mats[a].cols > P->mats[b].cols; });
      int band = kRmvRows;
      for (; band > kFusedMinBand; band /= 2) {
        long nb = 0;
        for (int i : fm) nb += cdiv(P->mats[i].rows, band);
        if (nb >= kFusedMinBlocks) break;
      }
      std::vector<int> fb;
      for (int i : fm) {
        MatInfo& m = P->mats[i];
        m.wband = band;
        m.n_rmv = cdiv(m.rows, kFusedPart);
        fb.push_back(cdiv(m.rows, band));
        P->fused[t].max_cols = std::max(P->fused[t].max_cols, m.cols);
      }
      add_list(meta, P->fused[t], fm, fb);
    }
    for (int i = 0; i < nm; ++i) {
      const MatInfo& m = P->mats[i];
      if (!fused_power(m)) { wm.push_back(i); wb.push_back(cdiv(m.rows, 16)); wr.push_back(m.n_rmv * m.n_ct); }
    }
    add_list(meta, P->matvec_w, wm, wb);
    add_list(meta, P->rmatvec_w, wm, wr);
  }
  (void)bytes_stream;

  for (int g = 0; g < 2; ++g)
    for (int t = 0; t < 2; ++t) {
      std::vector<int> ms, bl;
      for (int i = 0; i < nm; ++i) {
        const MatInfo& m = P->mats[i];
        if (m.ns_t != t || (g == 1 && !m.aurora)) continue;
        ms.push_back(i);
        bl.push_back((m.s_pad / 64) * (m.L_pad / 64));
      }
      add_list(meta, P->prologue[g][t], ms, bl);
    }
  for (int t = 0; t < 2; ++t) {
    std::vector<int> ms, bl;
    for (int i = 0; i < nm; ++i)
      if (P->mats[i].aurora && !P->mats[i].band_d && P->mats[i].ns_t == t) {
        ms.push_back(i);   // one wave per equilibrated line, 4 per block
        bl.push_back(cdiv(P->mats[i].eq_short ? P->mats[i].s : P->mats[i].L, 4));
      }
    add_list(meta, P->dupdate[t], ms, bl);
  }
  {
    std::vector<int> ms, bl;
    for (int i = 0; i < nm; ++i)
      if (P->mats[i].band_d) { ms.push_back(i); bl.push_back(cdiv(P->mats[i].L, 256)); }   // a thread per line
    add_list(meta, P->dfinish, ms, bl);
  }
  {
    std::vector<int> ms, bl;
    for (int i = 0; i < nm; ++i)
      if (P->mats[i].aurora) { ms.push_back(i); bl.push_back(1); }
    add_list(meta, P->ascale, ms, bl);
  }
  // Newton-Schulz tile lists, one set per (pass group, chain, NS type):
  // the Gram (s x s upper tiles, K = L), the short-side products (s x s upper
  // tiles, K = s; shared by GM_SQ and GM_SYM) and X' = Q X (s x L, K = s).
  // Longest reduction first (LPT); within a matrix, tiles sharing a tile row
  // are consecutive.
  int force_tile = 0;
  if (const char* v = getenv("MUON_NS_TILE")) force_tile = atoi(v) == 128 ? 128 : atoi(v) == 256 ? 256 : 0;
  for (int g = 0; g < 2; ++g)
    for (int c = 0; c < 2; ++c)
      for (int t = 0; t < 2; ++t)
        for (int li = 0; li < 3; ++li) {
          std::vector<int> order;
          for (int i = 0; i < nm; ++i) {
            const MatInfo& m = P->mats[i];
            if (m.ns_t != t || (g == 1 && !m.aurora) || m.chain[g] != c) continue;
            order.push_back(i);
          }
          auto kdim = [&](int i) {
            const MatInfo& m = P->mats[i];
            return li == LIST_GRAM ? m.L_pad : m.s_pad;
          };
          std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return kdim(a) > kdim(b); });
          std::vector<TileItem> items;
          GemmList& G = P->gemm[g][c][t][li];
          long n256 = 0;
          for (int i : order) {
            const long ts = P->mats[i].s_pad / kTile, tl = P->mats[i].L_pad / kTile;
            n256 += li == LIST_BX ? ts * tl : ts * (ts + 1) / 2;
          }
          G.tile = n256 < kSmallLaunchTiles ? 128 : kTile;
          if (force_tile) G.tile = force_tile;
          const int tile = G.tile;
          for (int i : order) {
            const MatInfo& m = P->mats[i];
            const int ts = m.s_pad / tile, tl = m.L_pad / tile;
            const double s = m.s, L = m.L;
            const int tcols = li == LIST_BX ? tl : ts;
            // Super-tiles of kSuperM x kSuperN tiles, row-major inside and
            // across: one super-tile is one XCD's wave of workgroups, so its
            // tiles share kSuperM row panels and kSuperN column panels in L2.
            for (int a0 = 0; a0 < ts; a0 += kSuperM)
              for (int b0 = 0; b0 < tcols; b0 += kSuperN)
                for (int a = a0; a < std::min(ts, a0 + kSuperM); ++a)
                  for (int b = b0; b < std::min(tcols, b0 + kSuperN); ++b) {
                    if (li != LIST_BX && b < a) continue;   // symmetric: upper tiles only
                    items.push_back(TileItem{(uint16_t)i, (uint16_t)a, (uint16_t)b, 0});
                  }
            // one standard iteration of this matrix, in the counted convention
            G.counted_iter += 4.0 * s * s * L + 2.0 * s * s * s;
            if (li == LIST_BX) {
              G.algorithmic += 2.0 * s * s * L;
              G.executed += 2.0 * ts * tl * tile * (double)tile * m.s_pad;
            } else {
              const double K = li == LIST_GRAM ? m.L_pad : m.s_pad;
              G.algorithmic += li == LIST_GRAM ? s * s * L : s * s * s;   // the upper half of a symmetric result
              // upper tiles; on the diagonal ones bf16 and fp8 operands
              // leave out the 32 x 32 blocks wholly below the diagonal (28 of
              // 64 on a 256-tile, 6 of 16 on a 128-tile, in every layout)
              const double diag_skip = t == DT_F32 ? 0.0 : (tile == 256 ? 28.0 / 64 : 6.0 / 16);
              G.executed += 2.0 * (ts * (ts + 1) / 2.0 - ts * diag_skip) * tile * (double)tile * K;
            }
          }
          add_gemm(meta, G, items);
          if (li == LIST_SQ) {
            GemmList& G2 = P->gemm[g][c][t][LIST_SQ2];
            G2 = G;
            G2.executed = 2 * G.executed;
            G2.algorithmic = 2 * G.algorithmic;
            G2.counted_iter = 0;
            const size_t n1 = items.size();
            for (size_t k = 0; k < n1; ++k) {
              TileItem x = items[k];
              x.pad = 1;
              items.push_back(x);
            }
            add_gemm(meta, G2, items);
          }
        }
  // Small sets: their launches fill a round of the CUs or less, and chain 0
  // on a second stream fills chain 1's partial rounds and launch gaps
  // (GPT-2-124M set 6.25 -> 5.96 ms, one 3.8B layer -0.4 %). With launches
  // of many rounds there is nothing to fill and the two chains' operand
  // panels share the L2s (3.8B set +2.8 %), so those stay on one stream.
  for (int g = 0; g < 2; ++g) {
    bool has[2] = {false, false}, small = true;
    for (int c = 0; c < 2; ++c)
      for (int t = 0; t < 2; ++t)
        for (int li = 0; li < 3; ++li) {
          const GemmList& G = P->gemm[g][c][t][li];
          if (G.n == 0) continue;
          has[c] = true;
          const double per256 = (double)G.tile * G.tile / ((double)kTile * kTile);
          small = small && G.n * per256 < kSmallLaunchTiles;
        }
    P->two_chains[g] = has[0] && has[1];
    P->side[g] = P->two_chains[g] && small;
  }
  return P;
}

LaunchList dev_list(const uint8_t* meta, const HostList& L) {
  LaunchList d;
  d.n = L.n;
  d.off = (const int32_t*)(meta + L.off_off);
  d.mat = (const int32_t*)(meta + L.off_mat);
  return d;
}

// ---------------------------------------------------------------------------
// Workspace and descriptor upload
// ---------------------------------------------------------------------------
muon_status ensure_workspace(muon_handle* h, size_t bytes) {
  if (bytes <= h->ws_bytes && h->ws) return MUON_OK;
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  if (h->ws) {
    HIP_TRY(h, hipFree(h->ws));
    h->ws = nullptr;
    h->ws_bytes = 0;
  }
  hipError_t e = hipMalloc(&h->ws, bytes);
  if (e != hipSuccess) {
    h->ws = nullptr;
    (void)hipGetLastError();
    return set_err(h, MUON_ERR_ALLOC, "workspace allocation of " + std::to_string(bytes) + " bytes failed");
  }
  h->ws_bytes = bytes;
  // descriptors of every cached plan now point at freed memory
  for (auto& kv : h->plans) kv.second->devmat_valid = false;
  return MUON_OK;
}

muon_status ensure_meta(muon_handle* h, Plan& P) {
  if (P.meta_dev) return MUON_OK;
  hipError_t e = hipMalloc(&P.meta_dev, P.meta_host.size());
  if (e != hipSuccess) {
    P.meta_dev = nullptr;
    (void)hipGetLastError();
    return set_err(h, MUON_ERR_ALLOC, "descriptor allocation failed");
  }
  HIP_TRY(h, hipMemcpy(P.meta_dev, P.meta_host.data(), P.meta_host.size(), hipMemcpyHostToDevice));
  P.devmat_valid = false;
  return MUON_OK;
}

muon_status upload_devmat(muon_handle* h, Plan& P, const std::vector<DevMat>& dm) {
  const size_t bytes = dm.size() * sizeof(DevMat);
  if (P.devmat_valid && P.last_devmat.size() == dm.size() && memcmp(P.last_devmat.data(), dm.data(), bytes) == 0)
    return MUON_OK;
  if (bytes == 0) return MUON_OK;
  if (h->upload_pending) {
    HIP_TRY(h, hipEventSynchronize(h->upload_done));
    h->upload_pending = false;
  }
  if (h->pinned_bytes < bytes) {
    if (h->pinned) HIP_TRY(h, hipHostFree(h->pinned));
    h->pinned = nullptr;
    h->pinned_bytes = 0;
    if (hipHostMalloc(&h->pinned, bytes, hipHostMallocDefault) != hipSuccess) {
      h->pinned = nullptr;
      (void)hipGetLastError();
      return set_err(h, MUON_ERR_ALLOC, "pinned staging allocation failed");
    }
    h->pinned_bytes = bytes;
  }
  memcpy(h->pinned, dm.data(), bytes);
  HIP_TRY(h, hipMemcpyAsync(P.meta_dev, h->pinned, bytes, hipMemcpyHostToDevice, h->stream));
  HIP_TRY(h, hipEventRecord(h->upload_done, h->stream));
  h->upload_pending = true;
  P.last_devmat = dm;
  P.devmat_valid = true;
  return MUON_OK;
}

// ---------------------------------------------------------------------------
// Profiling hooks
// ---------------------------------------------------------------------------
hipEvent_t pool_event(muon_handle* h) {
  if (!h->ev_pool.empty()) {
    hipEvent_t e = h->ev_pool.back();
    h->ev_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// A named ROCTx range over a phase of a call (annotates rocprofv3 traces run
// with --marker-trace); nothing when the handle has no ROCTx.
struct Range {
  muon_handle* h;
  explicit Range(muon_handle* hh, const char* name) : h(hh) {
    if (h->rx_push) h->rx_push(name);
  }
  ~Range() {
    if (h->rx_push) h->rx_pop();
  }
};

struct ProfScope {
  muon_handle* h;
  ProfRec r{};
  bool on;
  hipStream_t s;   // the stream the bracketed launches go to
  ProfScope(muon_handle* hh, int cls, double amount, double amount2 = 0, double amount3 = 0, bool on_side = false)
      : h(hh), on(hh->prof && !hh->in_static), s(on_side ? hh->side : hh->stream) {
    if (!on) return;
    r.cls = cls;
    r.amount = amount;
    r.amount2 = amount2;
    r.amount3 = amount3;
    r.count = 1;
    r.a = pool_event(h);
    r.b = pool_event(h);
    if (!r.a || !r.b) { on = false; return; }
    (void)hipEventRecord(r.a, s);
  }
  ~ProfScope() {
    if (!on) return;
    (void)hipEventRecord(r.b, s);
    h->recs.push_back(r);
  }
};

// Each class's time is the wall time its records cover: the sum of their
// durations less the time they overlap (records on the second stream run
// beside those on the call's stream; on one stream nothing overlaps).
muon_status drain_profile(muon_handle* h) {
  if (h->recs.empty()) return MUON_OK;
  std::vector<std::pair<float, float>> span[3];   // per class: [start, end] from the first record's start
  for (auto& r : h->recs) {
    HIP_TRY(h, hipEventSynchronize(r.b));
    float t0 = 0.f, t1 = 0.f;
    HIP_TRY(h, hipEventElapsedTime(&t0, h->recs[0].a, r.a));
    HIP_TRY(h, hipEventElapsedTime(&t1, h->recs[0].a, r.b));
    span[std::min(std::max(r.cls, 0), 2)].emplace_back(t0, t1);
  }
  double overlap[3] = {0.0, 0.0, 0.0};
  for (int k = 0; k < 3; ++k) {
    std::sort(span[k].begin(), span[k].end());
    float reach = -1e30f;
    for (auto& iv : span[k]) {
      if (iv.first < reach) overlap[k] += std::min(reach, iv.second) - iv.first;
      reach = std::max(reach, iv.second);
    }
  }
  h->acc.gemm_ms -= overlap[0];
  h->acc.stream_ms -= overlap[1];
  h->acc.aux_ms -= overlap[2];
  for (auto& r : h->recs) {
    float ms = 0.f;
    HIP_TRY(h, hipEventElapsedTime(&ms, r.a, r.b));
    if (r.cls == 0) {
      h->acc.gemm_launches += r.count;
      h->acc.gemm_ms += ms;
      h->acc.gemm_counted_flop += r.amount;
      h->acc.gemm_executed_flop += r.amount2;
      h->acc.gemm_algorithmic_flop += r.amount3;
    } else if (r.cls == 1) {
      h->acc.stream_launches += r.count;
      h->acc.stream_ms += ms;
      h->acc.stream_bytes += r.amount;
    } else {
      h->acc.aux_launches += r.count;
      h->acc.aux_ms += ms;
      h->acc.aux_bytes += r.amount;
    }
    h->ev_pool.push_back(r.a);
    h->ev_pool.push_back(r.b);
  }
  h->recs.clear();
  return MUON_OK;
}

// ---------------------------------------------------------------------------
// Enqueue
// ---------------------------------------------------------------------------
struct Call {
  int kind;
  int n;
  const muon_matrix* in;   // grad or polar input
  const muon_matrix* mom;
  const muon_matrix* w;
  const muon_matrix* out;  // update_out or polar output
  muon_config cfg;
};

#define CHECK_LAUNCH(h, expr)                                                                         \
  do {                                                                                                \
    hipError_t e_ = (expr);                                                                           \
    if (e_ != hipSuccess) return set_err((h), MUON_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(e_)); \
  } while (0)

// use_static: the workspace and the launch tables go to the device's static
// scratch (muon_update_static): no allocation, no profiling events.
muon_status run(muon_handle* h, const Call& c, bool use_static = false) {
  const muon_config& cfg = c.cfg;
  const int pp = c.kind == KIND_NS ? 0 : cfg.pp_iterations;
  const bool wide_rows = (cfg.flags & MUON_FLAG_WIDE_ROWS) != 0;
  const bool fp8 = (cfg.flags & MUON_FLAG_FP8_GRAM) != 0;
  bool forced = false;
  const int block = rect_block(cfg, &forced);
  const std::string key = plan_key(c.kind, pp, wide_rows, fp8, block, forced, c.n, c.in);
  auto it = h->plans.find(key);
  Plan* P;
  if (it == h->plans.end()) {
    if (h->plans.size() >= 16) {
      // evict the least recently used plan (its descriptors may be in flight)
      auto victim = h->plans.begin();
      for (auto i2 = h->plans.begin(); i2 != h->plans.end(); ++i2)
        if (i2->second->last_use < victim->second->last_use) victim = i2;
      HIP_TRY(h, hipStreamSynchronize(h->stream));
      if (victim->second->meta_dev) HIP_TRY(h, hipFree(victim->second->meta_dev));
      h->plans.erase(victim);
    }
    auto p = build_plan(c.kind, pp, wide_rows, fp8, block, forced, c.n, c.in, h->side_mode != 0);
    P = p.get();
    h->plans.emplace(key, std::move(p));
  } else {
    P = it->second.get();
  }
  P->last_use = ++h->tick;
  if (P->mats.empty()) return MUON_OK;
  // the second stream and its events, made by the first call whose plan
  // forks, before anything of the call is enqueued (default priority;
  // non-blocking, so it waits on the legacy null stream only through the
  // call's events)
  if (!use_static && !h->side && h->side_mode != 0 &&
      (h->side_mode == 1 ? P->two_chains[0] || P->two_chains[1] : P->side[0] || P->side[1])) {
    HIP_TRY(h, hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking));
    HIP_TRY(h, hipEventCreateWithFlags(&h->fork_ev, hipEventDisableTiming));
    HIP_TRY(h, hipEventCreateWithFlags(&h->join_ev, hipEventDisableTiming));
  }
  muon_status rc = MUON_OK;
  uint8_t* ws;
  uint8_t* meta;
  if (use_static) {
    const size_t meta_off = align_up(P->ws_bytes);
    const size_t need = meta_off + P->meta_host.size();
    if (need > static_scratch_bytes() || P->meta_host.size() > kStaticStageBytes)
      return set_err(h, MUON_ERR_TOO_LARGE,
                     "muon_update_static: the batch needs " + std::to_string(need) + " bytes of device scratch (" +
                         std::to_string(P->meta_host.size()) + " of launch tables); the static scratch holds " +
                         std::to_string(static_scratch_bytes()) + " bytes and " + std::to_string(kStaticStageBytes) +
                         " of tables");
    ws = (uint8_t*)h->scratch;
    meta = ws + meta_off;
  } else {
    rc = ensure_workspace(h, P->ws_bytes);
    if (rc) return rc;
    rc = ensure_meta(h, *P);
    if (rc) return rc;
    ws = (uint8_t*)h->ws;
    meta = (uint8_t*)P->meta_dev;
  }

  // descriptors
  std::vector<DevMat> dm(P->mats.size());
  for (size_t i = 0; i < P->mats.size(); ++i) {
    const MatInfo& m = P->mats[i];
    DevMat& d = dm[i];
    memset(&d, 0, sizeof(d));
    const muon_matrix& g = c.in[m.user];
    d.g = g.ptr; d.ld_g = g.ld; d.dt_g = g.dtype == MUON_BF16 ? DT_BF16 : DT_F32;
    if (c.kind == KIND_UPDATE) {
      d.m = (float*)c.mom[m.user].ptr; d.ld_m = c.mom[m.user].ld;
      if (c.w && c.w[m.user].ptr) {
        d.w = c.w[m.user].ptr; d.ld_w = c.w[m.user].ld; d.dt_w = c.w[m.user].dtype == MUON_BF16 ? DT_BF16 : DT_F32;
      }
    }
    if (c.out && c.out[m.user].ptr) {
      d.uo = c.out[m.user].ptr; d.ld_uo = c.out[m.user].ld;
      d.dt_uo = c.out[m.user].dtype == MUON_BF16 ? DT_BF16 : DT_F32;
    }
    d.rows = m.rows; d.cols = m.cols; d.s = m.s; d.L = m.L; d.s_pad = m.s_pad; d.L_pad = m.L_pad;
    d.tall = m.tall; d.square = m.square; d.aurora = m.aurora; d.eq_short = m.eq_short; d.ns_t = m.ns_t;
    d.n_rt = m.n_rt; d.n_ct = m.n_ct; d.n_seg = m.n_seg; d.n_rmv = m.n_rmv; d.wband = m.wband;
    d.xn = c.kind == KIND_UPDATE ? ws + m.o_xn : nullptr;
    d.x[0] = ws + m.o_x[0]; d.x[1] = ws + m.o_x[1];
    d.xt[0] = ws + m.o_xt[0]; d.xt[1] = ws + m.o_xt[1];
    for (int r = 0; r < SQ_COUNT; ++r) d.sq[r] = ws + m.o_sq[r];
    d.x8 = m.f8 ? ws + m.o_x8 : nullptr;
    d.fin = ((cfg.ns_steps + m.block - 1) / m.block) & 1;   // blocks per pass, mod 2
    d.rowpart = (float*)(ws + m.o_rowpart); d.colpart = (float*)(ws + m.o_colpart);
    d.rowsq = (float*)(ws + m.o_rowsq); d.colsq = (float*)(ws + m.o_colsq);
    d.rho = (float*)(ws + m.o_rho); d.dvec = (float*)(ws + m.o_dvec);
    d.pu = (float*)(ws + m.o_pu); d.pv = (float*)(ws + m.o_pv);
    d.pwpart = (float*)(ws + m.o_pwpart); d.tailpart = (float*)(ws + m.o_tailpart);
    d.linepart = (float*)(ws + m.o_linepart);
    d.lsq = m.band_d ? (float*)(ws + m.o_lsq) : nullptr;
    d.x0n = m.x0n;
    d.x0g = m.x0g;
    if (m.ft) {
      d.ftail = (float*)(ws + m.o_ftail);
      d.frow = (float*)(ws + m.o_frow);
      d.fwp = (float*)(ws + m.o_fwp);
      d.ftx = cfg.contra != 0.f;
      d.ftw = d.w != nullptr;
    }
    d.scal = (float*)(ws + m.o_scal); d.ist = (int32_t*)(ws + m.o_ist);
  }
  if (use_static) {
    // the whole table set (descriptors, then the lists) through the pinned
    // stage; the previous static upload from it must have been read
    if (h->static_pending) {
      HIP_TRY(h, hipEventSynchronize(h->static_done));
      h->static_pending = false;
    }
    uint8_t* stage = (uint8_t*)h->static_stage;
    memcpy(stage, P->meta_host.data(), P->meta_host.size());
    memcpy(stage, dm.data(), dm.size() * sizeof(DevMat));
    HIP_TRY(h, hipMemcpyAsync(meta, stage, P->meta_host.size(), hipMemcpyHostToDevice, h->stream));
    HIP_TRY(h, hipEventRecord(h->static_done, h->stream));
    h->static_pending = true;
  } else {
    rc = upload_devmat(h, *P, dm);
    if (rc) return rc;
  }

  DevMat* D = (DevMat*)meta;
  hipStream_t st = h->stream;
  const bool upd = c.kind == KIND_UPDATE;
  const bool contra = upd && cfg.contra != 0.f;

  // algorithmic byte counts for the profile
  double el_mv = 0, el_all = 0, el_fused[2] = {0, 0}, el_wide = 0;
  double b_mom = 0, b_wn = 0, b_tail_r = 0, b_tail_a = 0, b_pro[2][2] = {{0, 0}, {0, 0}}, b_dup[2] = {0, 0}, b_dfin = 0;
  for (size_t i = 0; i < P->mats.size(); ++i) {
    const MatInfo& m = P->mats[i];
    const double el = (double)m.rows * m.cols;
    const DevMat& d = dm[i];
    el_all += el;
    if (!m.ft) el_mv += el * esz(m.ns_t);
    (fused_power(m) ? el_fused[m.ns_t] : el_wide) += el * esz(m.ns_t);
    b_mom += upd ? el * (esz(d.dt_g) + 8 + esz(m.ns_t)) : el * esz(d.dt_g);
    if (d.ftw) b_wn += el * esz(d.dt_w);
    if (!m.ft) b_tail_r += el * (esz(m.ns_t) * (contra ? 2 : 1) + (d.w ? esz(d.dt_w) : 0));
    else if (contra) b_tail_r += el * 4.0 / 64;   // sigma's row parts
    b_tail_a += el * (esz(m.ns_t) * (contra ? 2 : 1) + (d.w ? 2 * esz(d.dt_w) : 0) + (d.uo ? esz(d.dt_uo) : 0));
    // prologue bytes: read the source, write the iterate and its transpose
    const double pro = el * esz(m.ns_t) + (m.x0n || m.x0g ? 1.0 : 2.0) * m.s_pad * (double)m.L_pad * esz(m.ns_t);
    b_pro[0][m.ns_t] += pro;
    if (m.aurora) {
      b_pro[1][m.ns_t] += pro;
      if (m.band_d) b_dfin += (double)(m.s_pad / 64) * m.L_pad * 4;   // the band sums
      else b_dup[m.ns_t] += (double)m.s * m.L * esz(m.ns_t);          // one read of U
    }
  }
  (void)el_all;

  // 0. optional input check: read-only, before anything is written; the
  // flags come back into pinned host memory and the call waits for them
  if ((cfg.flags & MUON_FLAG_CHECK_FINITE) && !P->mats.empty()) {
    const size_t nm = P->mats.size();
    CHECK_LAUNCH(h, launch_check_finite(D, dev_list(meta, P->stream), P->stream.nblk, upd ? 1 : 0, st));
    HIP_TRY(h, hipMemcpy2DAsync(h->bad_host, sizeof(int32_t), &D[0].bad, sizeof(DevMat), sizeof(int32_t), nm,
                                hipMemcpyDeviceToHost, st));
    HIP_TRY(h, hipStreamSynchronize(st));
    int first = -1;
    for (size_t i = 0; i < nm; ++i)
      if (h->bad_host[i] && (first < 0 || P->mats[i].user < first)) first = P->mats[i].user;
    if (first >= 0)
      return set_err(h, MUON_ERR_NONFINITE,
                     "matrix " + std::to_string(first) + " of the batch has a NaN or Inf among its inputs" +
                         (upd ? " (grad, momentum or weight)" : "") + "; nothing was written");
  }

  // 1. momentum/Nesterov (or input) + norms
  Range call_range(h, c.kind == KIND_UPDATE ? "libmuon muon_update" : c.kind == KIND_NS ? "libmuon ns_polar"
                                                                                  : "libmuon aurora_orthogonalize");
  {
    Range rg(h, "momentum");
    ProfScope ps(h, 1, b_mom);
    CHECK_LAUNCH(h, launch_momentum_stats(D, dev_list(meta, P->stream), P->stream.nblk, upd ? 1 : 0, cfg.mu,
                                          cfg.nesterov, (cfg.flags & MUON_FLAG_SGD_MOMENTUM) ? 1 : 0, st));
  }
  if (upd && c.w && P->stream_f.nblk) {
    ProfScope ps(h, 1, b_wn);
    CHECK_LAUNCH(h, launch_wnorm(D, dev_list(meta, P->stream_f), P->stream_f.nblk, st));
  }
  {
    ProfScope ps(h, 1, 0);
    CHECK_LAUNCH(h, launch_norms_lines(D, dev_list(meta, P->lines), P->lines.nblk, cfg.pp_eps, st));
    CHECK_LAUNCH(h, launch_norms_scalars(D, dev_list(meta, P->permat), P->permat.nblk, cfg.ns_eps, contra ? 1 : 0,
                                         st));
  }
  // 2. power iteration (profiled as one span: its launches are back to back)
  if (contra) {
    Range rg(h, "power iteration");
    ProfScope ps(h, 1, 0);
    ps.r.count = 0;
    for (int r = 0; r <= cfg.power_steps; ++r) {
      for (int t = 0; t < 2; ++t) {
        const HostList& F = P->fused[t];
        if (!F.nblk) continue;
        ps.r.amount += el_fused[t];
        ps.r.count += 1;
        CHECK_LAUNCH(h, launch_power_fused(t, D, dev_list(meta, F), F.nblk, cfg.power_steps, F.max_cols, st));
      }
      if (P->matvec_w.nblk) {
        ps.r.amount += 2 * el_wide;
        ps.r.count += 2;
        CHECK_LAUNCH(h, launch_power_matvec(D, dev_list(meta, P->matvec_w), P->matvec_w.nblk, cfg.power_steps, 0,
                                            st));
        CHECK_LAUNCH(h, launch_power_rmatvec(D, dev_list(meta, P->rmatvec_w), P->rmatvec_w.nblk, cfg.power_steps,
                                             st));
      }
      ps.r.count += 2;
      CHECK_LAUNCH(h, launch_power_wsum(D, dev_list(meta, P->colblk), P->colblk.nblk, cfg.power_steps, st));
      CHECK_LAUNCH(h, launch_power_normalize(D, dev_list(meta, P->permat), P->permat.nblk, cfg.power_steps, st));
    }
    // the final X v and sigma (fused-tail matrices take both in the tail)
    if (P->matvec.nblk) {
      ps.r.amount += el_mv;
      ps.r.count += 2;
      CHECK_LAUNCH(h, launch_power_matvec(D, dev_list(meta, P->matvec), P->matvec.nblk, cfg.power_steps, 1, st));
      CHECK_LAUNCH(h, launch_power_sigma(D, dev_list(meta, P->permat), P->permat.nblk, cfg.contra, st));
    }
  }
  // 3. Newton-Schulz passes. Per pass group, chain and type, the
  // iterations run in blocks of r (see ns_gemm.hip): A = X X^T; for each j,
  // B'_j = a I + b A + c A^2 (into Q0 when j = 0), Q <- B'_j Q, and unless j
  // is the block's last, A <- B'_j (B'_j A); then X' = Q X.
  // When the plan runs chain 0 on the second stream (in each pass where both
  // chains have matrices), that stream waits for everything enqueued so far,
  // and the call's stream waits for it at the end of the pass (before the D
  // update, which may read chain-0 matrices; on an early error return too).
  const bool may_fork = !h->in_static && h->side && h->side_mode != 0;
  struct SideJoin {
    muon_handle* h;
    hipStream_t st;
    bool pending = false;
    hipError_t join() {
      pending = false;
      hipError_t e = hipEventRecord(h->join_ev, h->side);
      return e != hipSuccess ? e : hipStreamWaitEvent(st, h->join_ev, 0);
    }
    ~SideJoin() {
      if (pending) (void)join();
    }
  } side_join{h, st};
  for (int p = 0; p < P->passes; ++p) {
    const int g = p == 0 ? 0 : 1;
    Range rg(h, p == 0 ? "Newton-Schulz pass 1" : p == 1 ? "Newton-Schulz pass 2" : "Newton-Schulz pass 3+");
    for (int t = 0; t < 2; ++t) {
      const HostList& L = P->prologue[g][t];
      if (L.nblk == 0) continue;
      ProfScope ps(h, 2, b_pro[g][t]);
      CHECK_LAUNCH(h, launch_prologue(t, D, dev_list(meta, L), L.nblk, upd ? 1 : 0, st));
    }
    const int last_pass = p + 1 == P->passes ? NS_LAST_PASS : 0;
    const bool fork_p = may_fork && (h->side_mode == 1 ? P->two_chains[g] : P->side[g]);
    if (fork_p) {
      HIP_TRY(h, hipEventRecord(h->fork_ev, st));
      HIP_TRY(h, hipStreamWaitEvent(h->side, h->fork_ev, 0));
      side_join.pending = true;
    }
    for (int c = 0; c < 2; ++c)
      for (int t = 0; t < 2; ++t) {
        const GemmList* GL = P->gemm[g][c][t];
        if (GL[LIST_GRAM].n == 0) continue;
        const bool on_side = fork_p && c == 0;
        const hipStream_t cs = on_side ? h->side : st;
        const int r = P->chain_block[g][c];
        // the first Gram of the pass reads the prologue's fp8 copy of X0 when
        // this chain's matrices have one (all or none: bf16 with blocks)
        const bool f8 = r > 1 && t == DT_BF16 && P->fp8;
        // profiling: one event pair around this chain's launches of the pass
        // (they run back to back on the stream), with their flops and count
        // summed; a pair per launch cost about 6 us each on the small sets
        ProfScope ps(h, 0, 0.0, 0.0, 0.0, on_side);
        ps.r.count = 0;
        auto gemm = [&](int li, int mode, int cur, int roles, double counted, int et) -> muon_status {
          const GemmList& G = GL[li];
          ps.r.amount += counted;
          ps.r.amount2 += G.executed;
          ps.r.amount3 += G.algorithmic;
          ps.r.count += 1;
          CHECK_LAUNCH(h, launch_ns_gemm(et, D, (const TileItem*)(meta + G.off), G.n, mode, cur,
                                         roles, cfg.ns_a, cfg.ns_b, cfg.ns_c, h->ns_variant, G.tile, cs));
          return MUON_OK;
        };
        int cur = 0;
        for (int k = 0; k < cfg.ns_steps; cur ^= 1) {
          const int rr = std::min(r, cfg.ns_steps - k);
          k += rr;
          muon_status e = gemm(LIST_GRAM, GM_GRAM, cur, ns_roles(0, 0, SQ_A) | (k == rr ? NS_FIRST : 0), 0.0,
                               f8 && k == rr ? DT_F8 : t);
          for (int j = 0; !e && j < rr; ++j) {
            const int bj = j == 0 ? SQ_Q0 : SQ_B;   // B'_0 is Q_1 itself
            e = gemm(LIST_SQ, GM_SQ, cur, ns_roles(SQ_A, SQ_A, bj), 0.0, t);
            // Q <- B'_j Q and T = B'_j A need only B'_j: one launch of both
            // (the list twice; marked tiles take the second roles)
            const int q_roles = ns_roles(SQ_B, (j - 1) & 1 ? SQ_Q1 : SQ_Q0, j & 1 ? SQ_Q1 : SQ_Q0);
            const int t_roles = ns_roles(bj, SQ_A, SQ_T);
            if (!e && j >= 1 && j + 1 < rr) e = gemm(LIST_SQ2, GM_SYM, cur, q_roles | (t_roles << 16), 0.0, t);
            else if (!e && j >= 1) e = gemm(LIST_SQ, GM_SYM, cur, q_roles, 0.0, t);
            else if (!e && j + 1 < rr) e = gemm(LIST_SQ, GM_SYM, cur, t_roles, 0.0, t);
            if (!e && j + 1 < rr) e = gemm(LIST_SQ, GM_SYM, cur, ns_roles(bj, SQ_T, SQ_A), 0.0, t);
          }
          if (!e) {
            const int roles = ns_roles((rr - 1) & 1 ? SQ_Q1 : SQ_Q0, 0, 0) |
                              (k == cfg.ns_steps ? NS_LAST_BX | last_pass : 0) | (k == rr ? NS_FIRST : 0);
            e = gemm(LIST_BX, GM_BX, cur, roles, rr * GL[LIST_BX].counted_iter, t);
          }
          if (e) return e;
        }
      }
    if (side_join.pending) HIP_TRY(h, side_join.join());
    if (p + 1 < P->passes) {
      Range rd(h, "Aurora D update");
      for (int t = 0; t < 2; ++t) {
        const HostList& L = P->dupdate[t];
        if (L.nblk == 0) continue;
        ProfScope ps(h, 2, b_dup[t]);
        CHECK_LAUNCH(h, launch_aurora_dupdate(t, D, dev_list(meta, L), L.nblk, cfg.pp_eps, cfg.pp_beta, st));
      }
      if (P->dfinish.nblk) {
        ProfScope ps(h, 2, b_dfin);
        CHECK_LAUNCH(h, launch_aurora_dfinish(D, dev_list(meta, P->dfinish), P->dfinish.nblk, cfg.pp_eps,
                                              cfg.pp_beta, st));
      }
      ProfScope ps(h, 2, 0);
      CHECK_LAUNCH(h, launch_aurora_scale(D, dev_list(meta, P->ascale), P->ascale.nblk, cfg.ns_eps, st));
    }
  }
  // 4. tail
  Range rt(h, "tail");
  if (upd) {
    if (P->stream_r.nblk || (contra && P->frows.nblk)) {
      ProfScope ps(h, 1, b_tail_r);
      CHECK_LAUNCH(h, launch_tail_reduce(D, dev_list(meta, P->stream_r), P->stream_r.nblk, st));
      if (contra) CHECK_LAUNCH(h, launch_tail_rows(D, dev_list(meta, P->frows), P->frows.nblk, st));
    }
    {
      ProfScope ps(h, 1, 0);
      CHECK_LAUNCH(h, launch_tail_finalize(D, dev_list(meta, P->permat), P->permat.nblk, cfg.target_uw, cfg.contra,
                                           st));
    }
    ProfScope ps(h, 1, b_tail_a);
    CHECK_LAUNCH(h, launch_tail_apply(D, dev_list(meta, P->stream), P->stream.nblk, cfg.lr, 0, st));
  } else {
    ProfScope ps(h, 1, b_tail_a);
    CHECK_LAUNCH(h, launch_tail_apply(D, dev_list(meta, P->stream), P->stream.nblk, 0.f, 1, st));
  }
  if (!use_static && h->prof && h->recs.size() > 200000) return drain_profile(h);
  return MUON_OK;
}

// Host-only consistency check of a plan (muon_debug_check_plan): every
// workspace region inside the workspace and disjoint from the others; every
// product tile in bounds, in the list of its matrix's pass group, chain
// and type, and every tile a product needs present exactly once; streaming
// lists with consistent block offsets. Returns an empty string when the plan
// passes, else the first violation.
std::string check_plan(const Plan& P) {
  char buf[256];
  const int nm = (int)P.mats.size();
  // workspace regions
  std::vector<std::pair<size_t, size_t>> rg = P.regions;
  std::sort(rg.begin(), rg.end());
  for (size_t i = 0; i < rg.size(); ++i) {
    if (rg[i].first + rg[i].second > P.ws_bytes) {
      snprintf(buf, sizeof(buf), "workspace region at %zu (%zu bytes) ends past the workspace (%zu)", rg[i].first,
               rg[i].second, P.ws_bytes);
      return buf;
    }
    if (i && rg[i - 1].first + rg[i - 1].second > rg[i].first) {
      snprintf(buf, sizeof(buf), "workspace regions at %zu and %zu overlap", rg[i - 1].first, rg[i].first);
      return buf;
    }
  }
  // streaming and vector lists: offsets from 0, non-decreasing, ending at nblk
  auto list_ok = [&](const HostList& L, const char* name) -> std::string {
    if (L.n == 0) return L.nblk == 0 ? "" : std::string(name) + ": blocks without matrices";
    const int32_t* off = (const int32_t*)(P.meta_host.data() + L.off_off);
    const int32_t* mat = (const int32_t*)(P.meta_host.data() + L.off_mat);
    if (off[0] != 0 || off[L.n] != L.nblk) return std::string(name) + ": block offsets do not span the launch";
    for (int i = 0; i < L.n; ++i)
      if (off[i + 1] < off[i] || mat[i] < 0 || mat[i] >= nm) return std::string(name) + ": bad entry";
    return "";
  };
  const std::pair<const HostList*, const char*> lists[] = {
      {&P.stream, "stream"}, {&P.permat, "permat"}, {&P.lines, "lines"}, {&P.colblk, "colblk"},
      {&P.matvec, "matvec"}, {&P.ascale, "ascale"}, {&P.fused[0], "fused"}, {&P.fused[1], "fused"},
      {&P.matvec_w, "matvec_w"}, {&P.rmatvec_w, "rmatvec_w"}, {&P.prologue[0][0], "prologue"},
      {&P.prologue[0][1], "prologue"}, {&P.prologue[1][0], "prologue"}, {&P.prologue[1][1], "prologue"},
      {&P.dupdate[0], "dupdate"}, {&P.dupdate[1], "dupdate"}, {&P.dfinish, "dfinish"},
      {&P.stream_r, "stream_r"}, {&P.frows, "frows"}, {&P.stream_f, "stream_f"}};
  for (const auto& l : lists) {
    std::string e = list_ok(*l.first, l.second);
    if (!e.empty()) return e;
  }
  {
    // the streaming tiles the kernels index: n_rt x n_seg per matrix
    const int32_t* off = (const int32_t*)(P.meta_host.data() + P.stream.off_off);
    const int32_t* mat = (const int32_t*)(P.meta_host.data() + P.stream.off_mat);
    for (int i = 0; i < P.stream.n; ++i) {
      const MatInfo& m = P.mats[mat[i]];
      if (off[i + 1] - off[i] != m.n_rt * m.n_seg) return "stream: block count differs from the tile grid";
    }
  }
  // chains: every matrix of a pass group in one of the group's chains, with
  // that chain's block length (its launches run that many iterations per
  // block for all their matrices)
  for (const MatInfo& m : P.mats)
    for (int g = 0; g < 2; ++g)
      if ((g == 0 || m.aurora) &&
          ((m.chain[g] != 0 && m.chain[g] != 1) || m.block != P.chain_block[g][m.chain[g]]))
        return "matrix in a chain of another block length";
  // product tile lists
  for (int g = 0; g < 2; ++g)
    for (int c = 0; c < 2; ++c)
      for (int t = 0; t < 2; ++t)
        for (int li = 0; li < 3; ++li) {
          const GemmList& G = P.gemm[g][c][t][li];
          const int tile = G.tile;
          if (tile != 128 && tile != 256) return "product list with a bad tile edge";
          std::vector<std::vector<uint8_t>> seen(nm);
          const TileItem* it = (const TileItem*)(P.meta_host.data() + G.off);
          for (int k = 0; k < G.n; ++k) {
            const TileItem& x = it[k];
            if (x.mat >= nm) return "product tile of an unknown matrix";
            const MatInfo& m = P.mats[x.mat];
            if (m.ns_t != t || m.chain[g] != c || (g == 1 && !m.aurora))
              return "product tile in another chain's list";
            if (m.s_pad % 256 || m.L_pad % 256) return "padded extents not a multiple of 256";
            const int ts = m.s_pad / tile, tcols = li == LIST_BX ? m.L_pad / tile : ts;
            if (x.tm >= ts || x.tn >= tcols || (li != LIST_BX && x.tm > x.tn)) {
              snprintf(buf, sizeof(buf), "tile (%d, %d) of matrix %d outside its %d x %d grid (list %d)", x.tm,
                       x.tn, m.user, ts, tcols, li);
              return buf;
            }
            if (seen[x.mat].empty()) seen[x.mat].assign((size_t)ts * tcols, 0);
            if (seen[x.mat][(size_t)x.tm * tcols + x.tn]++) return "product tile listed twice";
          }
          for (int i = 0; i < nm; ++i) {
            const MatInfo& m = P.mats[i];
            const bool member = m.ns_t == t && m.chain[g] == c && (g == 0 || m.aurora);
            const int ts = m.s_pad / tile, tcols = li == LIST_BX ? m.L_pad / tile : ts;
            const size_t need = li == LIST_BX ? (size_t)ts * tcols : (size_t)ts * (ts + 1) / 2;
            size_t have = 0;
            for (uint8_t v : seen[i]) have += v;
            if (member && have != need) {
              snprintf(buf, sizeof(buf), "matrix %d: %zu of its %zu tiles in list %d", m.user, have, need, li);
              return buf;
            }
            if (!member && have) return "tiles of a matrix that does not take part";
          }
          const TileItem* its = (const TileItem*)(P.meta_host.data() + G.off);
          for (int k = 0; k < G.n; ++k)
            if (its[k].pad) return "a marked tile outside the paired list";
          // the paired list: the short-side list, then the same tiles marked
          if (li == LIST_SQ) {
            const GemmList& G2 = P.gemm[g][c][t][LIST_SQ2];
            const TileItem* it2 = (const TileItem*)(P.meta_host.data() + G2.off);
            if (G2.n != 2 * G.n || G2.tile != G.tile) return "paired list not twice the short-side list";
            for (int k = 0; k < 2 * G.n; ++k) {
              const TileItem& x = its[k % G.n];
              if (it2[k].mat != x.mat || it2[k].tm != x.tm || it2[k].tn != x.tn || it2[k].pad != (k >= G.n ? 1 : 0))
                return "paired list differs from the short-side list";
            }
          }
        }
  return "";
}

muon_config resolve_cfg(const muon_config* cfg) {
  muon_config c;
  if (cfg) c = *cfg; else muon_config_default(&c);
  return c;
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" muon_status muon_create(muon_handle** out, void* stream) {
  if (!out) return MUON_ERR_INVALID_ARG;
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { (void)hipGetLastError(); return MUON_ERR_NO_DEVICE; }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) { (void)hipGetLastError(); return MUON_ERR_NO_DEVICE; }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MUON_ERR_NO_DEVICE;
  muon_handle* h = new (std::nothrow) muon_handle();
  if (!h) return MUON_ERR_ALLOC;
  h->device = dev;
  h->stream = (hipStream_t)stream;
  if (const char* v = getenv("MUON_NS_VARIANT")) h->ns_variant = atoi(v) == 1 ? 1 : 0;
  if (const char* v = getenv("MUON_NS_SIDE")) h->side_mode = atoi(v) == 0 ? 0 : 1;
  if (hipEventCreateWithFlags(&h->upload_done, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return MUON_ERR_HIP;
  }
  // set-up of muon_update_static: the device address of this device's static
  // scratch (looked up once per device), the table staging and its event
  if (static_scratch_address(dev, &h->scratch) != hipSuccess ||
      hipEventCreateWithFlags(&h->static_done, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    muon_destroy(h);
    return MUON_ERR_HIP;
  }
  if (hipHostMalloc(&h->static_stage, kStaticStageBytes, hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    h->static_stage = nullptr;
    muon_destroy(h);
    return MUON_ERR_ALLOC;
  }
  if (const char* v = getenv("MUON_ROCTX")) {
    if (atoi(v) != 0) {
      if (void* lib = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL)) {
        h->rx_lib = lib;
        h->rx_push = (int (*)(const char*))dlsym(lib, "roctxRangePushA");
        h->rx_pop = (int (*)())dlsym(lib, "roctxRangePop");
        if (!h->rx_push || !h->rx_pop) h->rx_push = nullptr, h->rx_pop = nullptr;
      }
    }
  }
  if (hipHostMalloc((void**)&h->bad_host, kMaxBatch * sizeof(int32_t), hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    h->bad_host = nullptr;
    muon_destroy(h);
    return MUON_ERR_ALLOC;
  }
  *out = h;
  return MUON_OK;
}

extern "C" muon_status muon_destroy(muon_handle* h) {
  if (!h) return MUON_OK;
  (void)hipStreamSynchronize(h->stream);
  for (auto& kv : h->plans)
    if (kv.second->meta_dev) (void)hipFree(kv.second->meta_dev);
  if (h->ws) (void)hipFree(h->ws);
  if (h->pinned) (void)hipHostFree(h->pinned);
  if (h->upload_done) (void)hipEventDestroy(h->upload_done);
  if (h->static_done) (void)hipEventDestroy(h->static_done);
  if (h->static_stage) (void)hipHostFree(h->static_stage);
  if (h->bad_host) (void)hipHostFree(h->bad_host);
  if (h->rx_lib) dlclose(h->rx_lib);
  if (h->side) {
    (void)hipStreamSynchronize(h->side);
    (void)hipStreamDestroy(h->side);
  }
  if (h->fork_ev) (void)hipEventDestroy(h->fork_ev);
  if (h->join_ev) (void)hipEventDestroy(h->join_ev);
  for (auto& r : h->recs) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
  for (auto e : h->ev_pool) (void)hipEventDestroy(e);
  delete h;
  return MUON_OK;
}

extern "C" muon_status muon_set_stream(muon_handle* h, void* stream) {
  if (!h) return MUON_ERR_INVALID_ARG;
  if ((hipStream_t)stream == h->stream) return MUON_OK;
  // descriptor uploads and workspace reuse are ordered on the old stream
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  h->stream = (hipStream_t)stream;
  return MUON_OK;
}

extern "C" const char* muon_last_error(const muon_handle* h) { return h ? h->err.c_str() : ""; }

extern "C" muon_status muon_debug_check_plan(int kind, int n, const muon_matrix* shapes, const muon_config* cfg,
                                             char* msg, int len) {
  if (msg && len > 0) msg[0] = 0;
  if (n < 0 || n > kMaxBatch || (n > 0 && !shapes) || kind < 0 || kind > 2) return MUON_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (shapes[i].rows < 0 || shapes[i].cols < 0 || shapes[i].rows > 65536 || shapes[i].cols > 65536 ||
        std::min(shapes[i].rows, shapes[i].cols) > 16384 ||
        (shapes[i].dtype != MUON_F32 && shapes[i].dtype != MUON_BF16))
      return MUON_ERR_SHAPE_MISMATCH;
  const muon_config c = resolve_cfg(cfg);
  const int k = kind == 0 ? KIND_UPDATE : kind == 1 ? KIND_NS : KIND_AURORA;
  const int pp = k == KIND_NS ? 0 : c.pp_iterations;
  bool forced = false;
  const int block = rect_block(c, &forced);
  std::unique_ptr<Plan> P = build_plan(k, pp, (c.flags & MUON_FLAG_WIDE_ROWS) != 0,
                                       (c.flags & MUON_FLAG_FP8_GRAM) != 0, block, forced, n, shapes, true);
  const std::string e = check_plan(*P);
  if (e.empty()) return MUON_OK;
  if (msg && len > 0) snprintf(msg, (size_t)len, "%s", e.c_str());
  return MUON_ERR_INVALID_ARG;
}

extern "C" muon_status muon_reserve(muon_handle* h, int n, const muon_matrix* shapes) {
  if (!h) return MUON_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxBatch || (n > 0 && !shapes)) return set_err(h, MUON_ERR_INVALID_ARG, "bad reserve batch");
  for (int i = 0; i < n; ++i) {
    if (shapes[i].rows < 0 || shapes[i].cols < 0 || shapes[i].rows > kMaxDim || shapes[i].cols > kMaxDim)
      return set_err(h, MUON_ERR_SHAPE_MISMATCH, "bad reserve shape");
    if (shapes[i].dtype != MUON_F32 && shapes[i].dtype != MUON_BF16)
      return set_err(h, MUON_ERR_UNSUPPORTED_DTYPE, "bad reserve dtype");
  }
  size_t need = 0;
  for (int kind = 0; kind < 3; ++kind) {
    bool forced = false;
    muon_config dflt;
    muon_config_default(&dflt);
    const int block = rect_block(dflt, &forced);
    auto P = build_plan(kind, 2, false, false, block, forced, n, shapes, true);
    need = std::max(need, P->ws_bytes);
  }
  return ensure_workspace(h, need);
}

extern "C" muon_status ns_polar(muon_handle* h, int n, const muon_matrix* in, const muon_matrix* out,
                                const muon_config* cfg) {
  if (!h) return MUON_ERR_INVALID_ARG;
  char msg[256];
  const int rc = check_polar(n, in, out, cfg, msg, sizeof(msg));
  if (rc) return set_err(h, rc, msg);
  h->err.clear();
  Call c{KIND_NS, n, in, nullptr, nullptr, out, resolve_cfg(cfg)};
  return run(h, c);
}

extern "C" muon_status aurora_orthogonalize(muon_handle* h, int n, const muon_matrix* in, const muon_matrix* out,
                                            const muon_config* cfg) {
  if (!h) return MUON_ERR_INVALID_ARG;
  char msg[256];
  const int rc = check_polar(n, in, out, cfg, msg, sizeof(msg));
  if (rc) return set_err(h, rc, msg);
  h->err.clear();
  Call c{KIND_AURORA, n, in, nullptr, nullptr, out, resolve_cfg(cfg)};
  return run(h, c);
}

extern "C" muon_status muon_update(muon_handle* h, int n, const muon_matrix* grad, const muon_matrix* momentum,
                                   const muon_matrix* weight, const muon_matrix* update_out, const muon_config* cfg) {
  if (!h) return MUON_ERR_INVALID_ARG;
  char msg[256];
  const int rc = check_update(n, grad, momentum, weight, update_out, cfg, msg, sizeof(msg));
  if (rc) return set_err(h, rc, msg);
  h->err.clear();
  Call c{KIND_UPDATE, n, grad, momentum, weight, update_out, resolve_cfg(cfg)};
  return run(h, c);
}

extern "C" muon_status muon_update_static(muon_handle* h, int n, const muon_matrix* grad,
                                          const muon_matrix* momentum, const muon_matrix* weight,
                                          const muon_matrix* update_out, const muon_config* cfg) {
  if (!h) return MUON_ERR_INVALID_ARG;
  char msg[256];
  const int rc = check_update(n, grad, momentum, weight, update_out, cfg, msg, sizeof(msg));
  if (rc) return set_err(h, rc, msg);
  h->err.clear();
  if (!h->scratch || !h->static_stage) return set_err(h, MUON_ERR_HIP, "static scratch not set up");
  Call c{KIND_UPDATE, n, grad, momentum, weight, update_out, resolve_cfg(cfg)};
  h->in_static = true;
  const muon_status r = run(h, c, true);
  h->in_static = false;
  return r;
}

extern "C" muon_status muon_profile_enable(muon_handle* h, int enable) {
  if (!h) return MUON_ERR_INVALID_ARG;
  h->prof = enable != 0;
  return MUON_OK;
}

extern "C" muon_status muon_profile_reset(muon_handle* h) {
  if (!h) return MUON_ERR_INVALID_ARG;
  muon_status rc = drain_profile(h);
  h->acc = muon_profile{};
  return rc;
}

extern "C" muon_status muon_profile_read(muon_handle* h, muon_profile* out) {
  if (!h || !out) return MUON_ERR_INVALID_ARG;
  muon_status rc = drain_profile(h);
  *out = h->acc;
  return rc;
}
