// Host-only validation helpers shared by the C-ABI entry points.
#pragma once
#include <stdint.h>

#include "../../include/libmuon.h"

namespace muon {

constexpr int kMaxDim = 65536;                 // rows, cols
constexpr int kMaxShort = 16384;               // min(rows, cols)
constexpr int64_t kMaxElems = int64_t(1) << 31;
constexpr int kMaxBatch = 65535;               // matrices per call
constexpr int64_t kMaxLd = int64_t(1) << 40;   // row stride in elements (keeps every offset far from overflow)

int check_config(const muon_config* c, char* msg, int len);
int check_polar(int n, const muon_matrix* in, const muon_matrix* out, const muon_config* cfg, char* msg, int len);
int check_update(int n, const muon_matrix* g, const muon_matrix* m, const muon_matrix* w, const muon_matrix* uo,
                 const muon_config* cfg, char* msg, int len);

}  // namespace muon
