// Host checks of the query-tile workgroup order (wg_coords_grouped), built
// with hipcc and run on the CPU; no GPU call is made.
//
// Workgroup w is started on XCD w % 8.  For every shape below the order must
// be a bijection of [0, heads * tiles), and when an XCD's range holds whole
// heads (heads * tiles divisible by 8, range divisible by tiles) every XCD
// must receive whole heads, so that under a causal mask (tile t costing t + 1)
// all XCDs get the same work.
#include <cstdio>
#include <vector>

#include "miattn_device.h"

using miattn::wg_coords_grouped;

static int check(int nbh, int ntile, int group, bool heavy) {
  const int total = nbh * ntile;
  std::vector<int> hit(total, 0);
  std::vector<long long> work(8, 0);
  std::vector<std::vector<int>> tiles_of(8 * nbh);
  for (int w = 0; w < total; ++w) {
    int bh = -1, t = -1;
    wg_coords_grouped(w, nbh, ntile, group, heavy, bh, t);
    if (bh < 0 || bh >= nbh || t < 0 || t >= ntile) {
      std::printf("FAIL out of range: nbh %d ntile %d group %d w %d -> (%d, %d)\n", nbh, ntile, group, w, bh, t);
      return 1;
    }
    hit[bh * ntile + t] += 1;
    work[w % 8] += t + 1;
  }
  for (int i = 0; i < total; ++i)
    if (hit[i] != 1) {
      std::printf("FAIL not a bijection: nbh %d ntile %d group %d: (%d, %d) hit %d times\n", nbh, ntile, group,
                  i / ntile, i % ntile, hit[i]);
      return 1;
    }
  const bool whole_heads = total % 8 == 0 && (total / 8) % ntile == 0;
  if (whole_heads)
    for (int x = 1; x < 8; ++x)
      if (work[x] != work[0]) {
        std::printf("FAIL unbalanced: nbh %d ntile %d group %d: XCD 0 work %lld, XCD %d work %lld\n", nbh, ntile,
                    group, work[0], x, work[x]);
        return 1;
      }
  return 0;
}

// Packed sequences (wg_coords_unit_major): a bijection, and every XCD gets the
// same heads of every sequence, so per-XCD work is equal for any lengths
// (checked with sequence s costing s + 1 per tile, tile t costing t + 1).
static int check_unit_major(int nseq, int nh, int ntile) {
  const int total = nseq * nh * ntile;
  std::vector<int> hit(total, 0);
  std::vector<long long> work(8, 0);
  for (int w = 0; w < total; ++w) {
    int bh = -1, t = -1;
    miattn::wg_coords_unit_major(w, nseq, nh, ntile, bh, t);
    if (bh < 0 || bh >= nseq * nh || t < 0 || t >= ntile) {
      std::printf("FAIL unit-major out of range: nseq %d nh %d ntile %d w %d -> (%d, %d)\n", nseq, nh, ntile, w, bh, t);
      return 1;
    }
    hit[bh * ntile + t] += 1;
    work[w % 8] += (long long)(bh / nh + 1) * (t + 1);
  }
  for (int i = 0; i < total; ++i)
    if (hit[i] != 1) {
      std::printf("FAIL unit-major not a bijection: nseq %d nh %d ntile %d\n", nseq, nh, ntile);
      return 1;
    }
  if (nh % 8 == 0)
    for (int x = 1; x < 8; ++x)
      if (work[x] != work[0]) {
        std::printf("FAIL unit-major unbalanced: nseq %d nh %d ntile %d\n", nseq, nh, ntile);
        return 1;
      }
  return 0;
}

int main() {
  int fails = 0, cases = 0;
  const int heads[] = {1, 2, 3, 5, 8, 12, 16, 24, 32, 40, 64, 96, 128, 256};
  const int tiles[] = {1, 2, 3, 7, 16, 32, 64, 128};
  for (int nbh : heads)
    for (int ntile : tiles)
      for (int group : {1, 2, 3, 4})
        for (bool heavy : {false, true}) {
          fails += check(nbh, ntile, group, heavy);
          ++cases;
        }
  for (int nseq : {1, 2, 3, 16, 33})
    for (int nh : {1, 3, 8, 12, 16, 32, 64})
      for (int ntile : {1, 2, 7, 32, 63}) {
        fails += check_unit_major(nseq, nh, ntile);
        ++cases;
      }
  if (fails) {
    std::printf("%d of %d order checks failed\n", fails, cases);
    return 1;
  }
  std::printf("order checks passed (%d cases)\n", cases);
  return 0;
}
