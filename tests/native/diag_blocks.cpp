// Host check of the engine's diagonal-tile block rule (Keep, diag_form in
// muon_device.hpp): for every layout, every 32x32 block on or above the
// diagonal of a diagonal tile is computed by the wave that owns it, every
// block a wave computes has its fragments read, and the blocks left out are
// exactly the strictly lower ones (n(n-1)/2 of n^2), which the planner's
// executed-flop count assumes. Prints one line per layout; exit status 0 on
// success.
#include <cstdio>

#include "muon_device.hpp"

using namespace muon;

template <int MI, int NI>
bool kept(int form, int mi, int ni, bool* row_ok) {
  bool k = true, r = true, c = true;
  // the engine's dispatch order: NI (wholly below), 0, 2, else full
  if (form == NI) {
    k = Keep<NI, MI, NI>::blk(mi, ni); r = Keep<NI, MI, NI>::row(mi); c = Keep<NI, MI, NI>::col(ni);
  } else if (form == 0) {
    k = Keep<0, MI, NI>::blk(mi, ni); r = Keep<0, MI, NI>::row(mi); c = Keep<0, MI, NI>::col(ni);
  } else if (form == 2) {
    k = Keep<2, MI, NI>::blk(mi, ni); r = Keep<2, MI, NI>::row(mi); c = Keep<2, MI, NI>::col(ni);
  }
  *row_ok = !k || (r && c);
  return k;
}

template <int WM, int WN, int TILE>
int check() {
  constexpr int MI = TILE / WM / 32, NI = TILE / WN / 32, n = TILE / 32;
  int skipped = 0, bad = 0;
  for (int wm = 0; wm < WM; ++wm)
    for (int wn = 0; wn < WN; ++wn) {
      const int form = diag_form(wm, wn, MI, NI);
      for (int mi = 0; mi < MI; ++mi)
        for (int ni = 0; ni < NI; ++ni) {
          const int bi = wm * MI + mi, bj = wn * NI + ni;   // block row and column in the tile
          bool frags_ok = true;
          const bool k = kept<MI, NI>(form, mi, ni, &frags_ok);
          if (!frags_ok) ++bad;
          if (!k) {
            ++skipped;
            if (bj >= bi) ++bad;   // a needed block left out
          }
        }
    }
  const int lower = n * (n - 1) / 2;
  std::printf("layout %dx%d waves, tile %d: %d of %d blocks left out (strictly lower %d), %d errors\n", WM, WN,
              TILE, skipped, n * n, lower, bad);
  return bad + (skipped != lower ? 1 : 0);
}

int main() {
  const int e = check<4, 2, 256>() + check<2, 2, 256>() + check<2, 2, 128>();
  return e == 0 ? 0 : 1;
}
