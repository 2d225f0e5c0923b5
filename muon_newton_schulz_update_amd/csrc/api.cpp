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
//   momentum + Nesterov + row partial norms -> norm lines (row and column
//   norms, rho, D0) -> per-matrix scalars (||X||, prologue scale)
//   -> power iteration (power_steps + 1 rounds of w = X^T X v, one read of X
//      in a fused pass, or X v then X^T u for matrices wider than
//      kFusedCols; ||w||, v = w/||w||; then X v and sigma)
//   -> for each Aurora pass: prologue (scale * D o T, both orientations),
//      ns_steps x {A = XX^T, B' = bA + cA^2 + aI, X = B'X}, D update between
//      passes
//   -> tail reduce -> tail finalise (Contra, Frobenius restore, aspect, floor)
//   -> tail apply (update_out, W -= lr V).
#include <hip/hip_runtime.h>
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
                          float ca, float cb, float cc, int variant, int tile, hipStream_t st);
hipError_t launch_momentum_stats(const DevMat* m, LaunchList L, int nblk, int nesterov_pass, float mu, int nesterov,
                                 hipStream_t st);
hipError_t launch_norms_lines(DevMat* m, LaunchList L, int nblk, float pp_eps, hipStream_t st);
hipError_t launch_norms_scalars(DevMat* m, LaunchList L, int nblk, float ns_eps, int init_power, hipStream_t st);
hipError_t launch_prologue(int ns_t, const DevMat* m, LaunchList L, int nblk, int use_xn, hipStream_t st);
hipError_t launch_aurora_dupdate(int ns_t, DevMat* m, LaunchList L, int nblk, int fin, float pp_eps, float pp_beta,
                                 hipStream_t st);
hipError_t launch_aurora_scale(DevMat* m, LaunchList L, int nblk, float ns_eps, hipStream_t st);
hipError_t launch_power_matvec(const DevMat* m, LaunchList L, int nblk, int steps, int final_pass, hipStream_t st);
hipError_t launch_power_rmatvec(const DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st);
hipError_t launch_power_fused(int ns_t, const DevMat* m, LaunchList L, int nblk, int steps, int max_cols,
                              hipStream_t st);
hipError_t launch_power_wsum(DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st);
hipError_t launch_power_normalize(DevMat* m, LaunchList L, int nblk, int steps, hipStream_t st);
hipError_t launch_power_sigma(DevMat* m, LaunchList L, int nblk, float contra, hipStream_t st);
hipError_t launch_tail_reduce(const DevMat* m, LaunchList L, int nblk, int fin, hipStream_t st);
hipError_t launch_tail_finalize(DevMat* m, LaunchList L, int nblk, float target_uw, hipStream_t st);
hipError_t launch_tail_apply(const DevMat* m, LaunchList L, int nblk, int fin, float lr, int copy_only,
                             hipStream_t st);

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
  bool tall, square, aurora;
  int ns_t;
  int n_rt, n_ct, n_seg, n_rmv, wband;
  size_t o_xn, o_x[2], o_xt[2], o_a, o_b, o_rowpart, o_colpart, o_rowsq, o_colsq, o_rho, o_dvec, o_pu, o_pv,
      o_pwpart, o_tailpart, o_linepart, o_scal, o_ist;
};

// The fused power pass takes matrices up to kFusedCols columns whose rows are
// whole 16-byte chunks of the NS type (it loads 8-element chunks only); it
// depends on the matrix alone, never on the rest of the batch.
inline bool fused_power(const MatInfo& m) {
  return m.cols <= kFusedCols && ((size_t)m.cols * (m.ns_t == DT_BF16 ? 2 : 4)) % 16 == 0;
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
  double counted = 0, executed = 0; // flops
};

// A product launch with fewer 256-tiles than this uses 128-tiles: with one
// 256-tile workgroup per CU such a launch is a few rounds of workgroups and
// its last round leaves CUs idle, while 128-tiles (two workgroups per CU)
// cover the CUs in finer steps. MUON_NS_TILE=128 or 256 forces one size.
constexpr int kSmallLaunchTiles = 768;
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
  HostList fused[2];                      // power rounds: fused X^T X v pass, one list per NS type
  HostList matvec_w, rmatvec_w;           // X v + X^T u for matrices wider than kFusedCols
  HostList prologue[2][2];  // [group: 0 all, 1 aurora][ns_t]
  HostList dupdate[2];      // [ns_t]
  GemmList gemm[2][2][3];   // [group][ns_t][mode]
  // device meta: DevMat array followed by the list arrays
  std::vector<uint8_t> meta_host;  // list part (static)
  size_t meta_devmat_bytes = 0;
  void* meta_dev = nullptr;
  std::vector<DevMat> last_devmat;
  bool devmat_valid = false;
  uint64_t last_use = 0;
};

std::string plan_key(int kind, int pp, int n, const muon_matrix* in) {
  std::string k;
  k.reserve(16 + n * 12);
  char buf[64];
  snprintf(buf, sizeof(buf), "%d/%d/%d|", kind, pp, n);
  k += buf;
  for (int i = 0; i < n; ++i) {
    snprintf(buf, sizeof(buf), "%lld,%lld,%d;", (long long)in[i].rows, (long long)in[i].cols, (int)in[i].dtype);
    k += buf;
  }
  return k;
}

struct ProfRec {
  hipEvent_t a, b;
  int cls;  // 0 gemm, 1 stream
  double amount, amount2;
};

}  // namespace
}  // namespace muon

struct muon_handle {
  int device = 0;
  int ns_variant = 0;        // Newton-Schulz tile layout (MUON_NS_VARIANT; 0 = 8 waves, 1 = 4 waves)
  hipStream_t stream = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  std::map<std::string, std::unique_ptr<muon::Plan>> plans;
  uint64_t tick = 0;
  void* pinned = nullptr;
  size_t pinned_bytes = 0;
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
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

// A plan depends only on the call kind, the pass count and the inputs' shapes
// and element types (exactly what plan_key holds): caller pointers, strides,
// weights and outputs go into the per-call descriptors.
std::unique_ptr<Plan> build_plan(int kind, int pp, int n, const muon_matrix* in) {
  auto P = std::make_unique<Plan>();
  P->kind = kind;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 1));
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
    m.ns_t = in[i].dtype == MUON_BF16 ? DT_BF16 : DT_F32;
    m.n_rt = cdiv(m.rows, kStreamRows);
    m.n_ct = cdiv(m.cols, kStreamCols);
    m.n_seg = cdiv(m.cols, kSegCols);
    m.wband = kRmvRows;
    m.n_rmv = cdiv(m.rows, kRmvRows);
    const size_t e = esz(m.ns_t);
    const size_t nsl = (size_t)m.s_pad * m.L_pad * e;
    m.o_xn = kind == KIND_UPDATE ? take((size_t)m.rows * m.cols * e) : 0;
    m.o_x[0] = take(nsl);
    m.o_x[1] = take(nsl);
    m.o_xt[0] = take(nsl);
    m.o_xt[1] = take(nsl);
    m.o_a = take((size_t)m.s_pad * m.s_pad * e);
    m.o_b = take((size_t)m.s_pad * m.s_pad * e);
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
    m.o_tailpart = take(std::max((size_t)m.n_rt * m.n_seg * 4, (size_t)cdiv(m.L, 4)) * 4);
    m.o_linepart = take((size_t)2 * line_blocks(m.rows, m.cols) * 4);
    m.o_scal = take(SC_COUNT * 4);
    m.o_ist = take(IS_COUNT * 4);
    if (m.aurora) P->any_aurora = true;
    P->mats.push_back(m);
  }
  P->ws_bytes = off;
  P->passes = P->any_aurora ? pp : 1;

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
  for (int i = 0; i < nm; ++i) blocks[i] = 1;
  add_list(meta, P->permat, all, blocks);
  for (int i = 0; i < nm; ++i) blocks[i] = line_blocks(P->mats[i].rows, P->mats[i].cols);
  add_list(meta, P->lines, all, blocks);
  for (int i = 0; i < nm; ++i) blocks[i] = cdiv(P->mats[i].cols, 256);
  add_list(meta, P->colblk, all, blocks);
  for (int i = 0; i < nm; ++i) blocks[i] = cdiv(P->mats[i].rows, 16);   // 4 waves x 4 rows
  add_list(meta, P->matvec, all, blocks);   // the final X v of every matrix
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
      if (P->mats[i].aurora && P->mats[i].ns_t == t) { ms.push_back(i); bl.push_back(cdiv(P->mats[i].L, 4)); }
    add_list(meta, P->dupdate[t], ms, bl);
  }
  {
    std::vector<int> ms, bl;
    for (int i = 0; i < nm; ++i)
      if (P->mats[i].aurora) { ms.push_back(i); bl.push_back(1); }
    add_list(meta, P->ascale, ms, bl);
  }
  // Newton-Schulz tile lists: longest reduction first (LPT); within a matrix,
  // tiles sharing a tile row are consecutive.
  int force_tile = 0;
  if (const char* v = getenv("MUON_NS_TILE")) force_tile = atoi(v) == 128 ? 128 : atoi(v) == 256 ? 256 : 0;
  for (int g = 0; g < 2; ++g)
    for (int t = 0; t < 2; ++t)
      for (int mode = 0; mode < 3; ++mode) {
        std::vector<int> order;
        for (int i = 0; i < nm; ++i) {
          const MatInfo& m = P->mats[i];
          if (m.ns_t != t || (g == 1 && !m.aurora)) continue;
          order.push_back(i);
        }
        auto kdim = [&](int i) {
          const MatInfo& m = P->mats[i];
          return mode == GM_GRAM ? m.L_pad : m.s_pad;
        };
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return kdim(a) > kdim(b); });
        std::vector<TileItem> items;
        GemmList& G = P->gemm[g][t][mode];
        long n256 = 0;
        for (int i : order) {
          const long ts = P->mats[i].s_pad / kTile, tl = P->mats[i].L_pad / kTile;
          n256 += mode == GM_BX ? ts * tl : ts * (ts + 1) / 2;
        }
        G.tile = n256 < kSmallLaunchTiles ? 128 : kTile;
        if (force_tile) G.tile = force_tile;
        const int tile = G.tile;
        for (int i : order) {
          const MatInfo& m = P->mats[i];
          const int ts = m.s_pad / tile, tl = m.L_pad / tile;
          const double s = m.s, L = m.L;
          const int tcols = mode == GM_BX ? tl : ts;
          // Super-tiles of kSuperM x kSuperN tiles, row-major inside and
          // across: one super-tile is one XCD's wave of workgroups, so its
          // tiles share kSuperM row panels and kSuperN column panels in L2.
          for (int a0 = 0; a0 < ts; a0 += kSuperM)
            for (int b0 = 0; b0 < tcols; b0 += kSuperN)
              for (int a = a0; a < std::min(ts, a0 + kSuperM); ++a)
                for (int b = b0; b < std::min(tcols, b0 + kSuperN); ++b) {
                  if (mode != GM_BX && b < a) continue;   // symmetric: upper tiles only
                  items.push_back(TileItem{(uint16_t)i, (uint16_t)a, (uint16_t)b, 0});
                }
          if (mode == GM_BX) {
            G.counted += 2.0 * s * s * L;
            G.executed += 2.0 * ts * tl * tile * (double)tile * m.s_pad;
          } else {
            const double K = mode == GM_GRAM ? m.L_pad : m.s_pad;
            G.counted += mode == GM_GRAM ? 2.0 * s * s * L : 2.0 * s * s * s;
            G.executed += 2.0 * (ts * (ts + 1) / 2) * tile * (double)tile * K;
          }
        }
        add_gemm(meta, G, items);
      }
  return P;
}

LaunchList dev_list(const Plan& P, const HostList& L) {
  LaunchList d;
  d.n = L.n;
  d.off = (const int32_t*)((const uint8_t*)P.meta_dev + L.off_off);
  d.mat = (const int32_t*)((const uint8_t*)P.meta_dev + L.off_mat);
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

struct ProfScope {
  muon_handle* h;
  ProfRec r{};
  bool on;
  ProfScope(muon_handle* hh, int cls, double amount, double amount2 = 0) : h(hh), on(hh->prof) {
    if (!on) return;
    r.cls = cls;
    r.amount = amount;
    r.amount2 = amount2;
    r.a = pool_event(h);
    r.b = pool_event(h);
    if (!r.a || !r.b) { on = false; return; }
    (void)hipEventRecord(r.a, h->stream);
  }
  ~ProfScope() {
    if (!on) return;
    (void)hipEventRecord(r.b, h->stream);
    h->recs.push_back(r);
  }
};

muon_status drain_profile(muon_handle* h) {
  for (auto& r : h->recs) {
    HIP_TRY(h, hipEventSynchronize(r.b));
    float ms = 0.f;
    HIP_TRY(h, hipEventElapsedTime(&ms, r.a, r.b));
    if (r.cls == 0) {
      h->acc.gemm_launches += 1;
      h->acc.gemm_ms += ms;
      h->acc.gemm_counted_flop += r.amount;
      h->acc.gemm_executed_flop += r.amount2;
    } else {
      h->acc.stream_launches += 1;
      h->acc.stream_ms += ms;
      h->acc.stream_bytes += r.amount;
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

muon_status run(muon_handle* h, const Call& c) {
  const muon_config& cfg = c.cfg;
  const int pp = c.kind == KIND_NS ? 0 : cfg.pp_iterations;
  const std::string key = plan_key(c.kind, pp, c.n, c.in);
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
    auto p = build_plan(c.kind, pp, c.n, c.in);
    P = p.get();
    h->plans.emplace(key, std::move(p));
  } else {
    P = it->second.get();
  }
  P->last_use = ++h->tick;
  if (P->mats.empty()) return MUON_OK;
  muon_status rc = ensure_workspace(h, P->ws_bytes);
  if (rc) return rc;
  rc = ensure_meta(h, *P);
  if (rc) return rc;

  // descriptors
  uint8_t* ws = (uint8_t*)h->ws;
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
    d.tall = m.tall; d.square = m.square; d.aurora = m.aurora; d.ns_t = m.ns_t;
    d.n_rt = m.n_rt; d.n_ct = m.n_ct; d.n_seg = m.n_seg; d.n_rmv = m.n_rmv; d.wband = m.wband;
    d.xn = c.kind == KIND_UPDATE ? ws + m.o_xn : nullptr;
    d.x[0] = ws + m.o_x[0]; d.x[1] = ws + m.o_x[1];
    d.xt[0] = ws + m.o_xt[0]; d.xt[1] = ws + m.o_xt[1];
    d.a = ws + m.o_a; d.b = ws + m.o_b;
    d.rowpart = (float*)(ws + m.o_rowpart); d.colpart = (float*)(ws + m.o_colpart);
    d.rowsq = (float*)(ws + m.o_rowsq); d.colsq = (float*)(ws + m.o_colsq);
    d.rho = (float*)(ws + m.o_rho); d.dvec = (float*)(ws + m.o_dvec);
    d.pu = (float*)(ws + m.o_pu); d.pv = (float*)(ws + m.o_pv);
    d.pwpart = (float*)(ws + m.o_pwpart); d.tailpart = (float*)(ws + m.o_tailpart);
    d.linepart = (float*)(ws + m.o_linepart);
    d.scal = (float*)(ws + m.o_scal); d.ist = (int32_t*)(ws + m.o_ist);
  }
  rc = upload_devmat(h, *P, dm);
  if (rc) return rc;

  DevMat* D = (DevMat*)P->meta_dev;
  hipStream_t st = h->stream;
  const bool upd = c.kind == KIND_UPDATE;
  const bool contra = upd && cfg.contra != 0.f;

  // algorithmic byte counts for the profile
  double el_ns = 0, el_all = 0, el_fused[2] = {0, 0}, el_wide = 0;
  double b_mom = 0, b_tail_r = 0, b_tail_a = 0, b_pro[2][2] = {{0, 0}, {0, 0}};
  for (size_t i = 0; i < P->mats.size(); ++i) {
    const MatInfo& m = P->mats[i];
    const double el = (double)m.rows * m.cols;
    const DevMat& d = dm[i];
    el_all += el;
    el_ns += el * esz(m.ns_t);
    (fused_power(m) ? el_fused[m.ns_t] : el_wide) += el * esz(m.ns_t);
    b_mom += upd ? el * (esz(d.dt_g) + 8 + esz(m.ns_t)) : el * esz(d.dt_g);
    b_tail_r += el * (esz(m.ns_t) * (contra ? 2 : 1) + (d.w ? esz(d.dt_w) : 0));
    b_tail_a += el * (esz(m.ns_t) * (contra ? 2 : 1) + (d.w ? 2 * esz(d.dt_w) : 0) + (d.uo ? esz(d.dt_uo) : 0));
    // prologue bytes: read the source, write the iterate and its transpose
    const double pro = el * esz(m.ns_t) + 2.0 * m.s_pad * (double)m.L_pad * esz(m.ns_t);
    b_pro[0][m.ns_t] += pro;
    if (m.aurora) b_pro[1][m.ns_t] += pro;
  }
  (void)el_all;

  // 1. momentum/Nesterov (or input) + norms
  {
    ProfScope ps(h, 1, b_mom);
    CHECK_LAUNCH(h, launch_momentum_stats(D, dev_list(*P, P->stream), P->stream.nblk, upd ? 1 : 0, cfg.mu,
                                          cfg.nesterov, st));
  }
  {
    ProfScope ps(h, 1, 0);
    CHECK_LAUNCH(h, launch_norms_lines(D, dev_list(*P, P->lines), P->lines.nblk, cfg.pp_eps, st));
    CHECK_LAUNCH(h, launch_norms_scalars(D, dev_list(*P, P->permat), P->permat.nblk, cfg.ns_eps, contra ? 1 : 0,
                                         st));
  }
  // 2. power iteration
  if (contra) {
    for (int r = 0; r <= cfg.power_steps; ++r) {
      for (int t = 0; t < 2; ++t) {
        const HostList& F = P->fused[t];
        if (!F.nblk) continue;
        ProfScope ps(h, 1, el_fused[t]);
        CHECK_LAUNCH(h, launch_power_fused(t, D, dev_list(*P, F), F.nblk, cfg.power_steps, F.max_cols, st));
      }
      if (P->matvec_w.nblk) {
        {
          ProfScope ps(h, 1, el_wide);
          CHECK_LAUNCH(h, launch_power_matvec(D, dev_list(*P, P->matvec_w), P->matvec_w.nblk, cfg.power_steps, 0,
                                              st));
        }
        ProfScope ps(h, 1, el_wide);
        CHECK_LAUNCH(h, launch_power_rmatvec(D, dev_list(*P, P->rmatvec_w), P->rmatvec_w.nblk, cfg.power_steps,
                                             st));
      }
      {
        ProfScope ps(h, 1, 0);
        CHECK_LAUNCH(h, launch_power_wsum(D, dev_list(*P, P->colblk), P->colblk.nblk, cfg.power_steps, st));
        CHECK_LAUNCH(h, launch_power_normalize(D, dev_list(*P, P->permat), P->permat.nblk, cfg.power_steps, st));
      }
    }
    {
      ProfScope ps(h, 1, el_ns);
      CHECK_LAUNCH(h, launch_power_matvec(D, dev_list(*P, P->matvec), P->matvec.nblk, cfg.power_steps, 1, st));
    }
    {
      ProfScope ps(h, 1, 0);
      CHECK_LAUNCH(h, launch_power_sigma(D, dev_list(*P, P->permat), P->permat.nblk, cfg.contra, st));
    }
  }
  // 3. Newton-Schulz passes
  const int fin = cfg.ns_steps & 1;
  for (int p = 0; p < P->passes; ++p) {
    const int g = p == 0 ? 0 : 1;
    for (int t = 0; t < 2; ++t) {
      const HostList& L = P->prologue[g][t];
      if (L.nblk == 0) continue;
      ProfScope ps(h, 1, b_pro[g][t]);
      CHECK_LAUNCH(h, launch_prologue(t, D, dev_list(*P, L), L.nblk, upd ? 1 : 0, st));
    }
    for (int k = 0; k < cfg.ns_steps; ++k) {
      const int cur = k & 1;
      for (int mode = 0; mode < 3; ++mode)
        for (int t = 0; t < 2; ++t) {
          const GemmList& G = P->gemm[g][t][mode];
          if (G.n == 0) continue;
          ProfScope ps(h, 0, G.counted, G.executed);
          CHECK_LAUNCH(h, launch_ns_gemm(t, D, (const TileItem*)((uint8_t*)P->meta_dev + G.off), G.n, mode, cur,
                                         cfg.ns_a, cfg.ns_b, cfg.ns_c, h->ns_variant, G.tile, st));
        }
    }
    if (p + 1 < P->passes) {
      for (int t = 0; t < 2; ++t) {
        const HostList& L = P->dupdate[t];
        if (L.nblk == 0) continue;
        ProfScope ps(h, 1, 0);
        CHECK_LAUNCH(h, launch_aurora_dupdate(t, D, dev_list(*P, L), L.nblk, fin, cfg.pp_eps, cfg.pp_beta, st));
      }
      ProfScope ps(h, 1, 0);
      CHECK_LAUNCH(h, launch_aurora_scale(D, dev_list(*P, P->ascale), P->ascale.nblk, cfg.ns_eps, st));
    }
  }
  // 4. tail
  if (upd) {
    {
      ProfScope ps(h, 1, b_tail_r);
      CHECK_LAUNCH(h, launch_tail_reduce(D, dev_list(*P, P->stream), P->stream.nblk, fin, st));
    }
    {
      ProfScope ps(h, 1, 0);
      CHECK_LAUNCH(h, launch_tail_finalize(D, dev_list(*P, P->permat), P->permat.nblk, cfg.target_uw, st));
    }
    ProfScope ps(h, 1, b_tail_a);
    CHECK_LAUNCH(h, launch_tail_apply(D, dev_list(*P, P->stream), P->stream.nblk, fin, cfg.lr, 0, st));
  } else {
    ProfScope ps(h, 1, b_tail_a);
    CHECK_LAUNCH(h, launch_tail_apply(D, dev_list(*P, P->stream), P->stream.nblk, fin, 0.f, 1, st));
  }
  if (h->prof && h->recs.size() > 200000) return drain_profile(h);
  return MUON_OK;
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
  if (hipEventCreateWithFlags(&h->upload_done, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return MUON_ERR_HIP;
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
    auto P = build_plan(kind, 2, n, shapes);
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
