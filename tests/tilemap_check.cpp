// Host check of the varlen tile schedule (fa_tilemap.h, the arithmetic the
// device pre-pass runs): reads "nbatch bm tq tkv reverse" and the two
// cumulative-length arrays from stdin, forms the exclusive prefix of tiles per
// sequence as the pre-pass does, and prints one line per entry of the
// ceil(tq / bm) + nbatch the grid holds: b qt q0 k0 sq skv valid.
#include <stdio.h>

#include <vector>

#include "fa_tilemap.h"

int main() {
  int nbatch, bm, tq, tkv, reverse;
  if (scanf("%d %d %d %d %d", &nbatch, &bm, &tq, &tkv, &reverse) != 5) return 2;
  std::vector<int32_t> cq(nbatch + 1), ck(nbatch + 1), prefix(nbatch + 1);
  for (auto& x : cq)
    if (scanf("%d", &x) != 1) return 2;
  for (auto& x : ck)
    if (scanf("%d", &x) != 1) return 2;
  int acc = 0;
  for (int b = 0; b < nbatch; ++b) {
    prefix[b] = acc;
    acc += fa::seq_tiles(cq.data(), b, tq, bm);
  }
  prefix[nbatch] = acc;
  const int tph = (tq + bm - 1) / bm + nbatch;
  printf("%d %d\n", acc, tph);
  for (int r = 0; r < tph; ++r) {
    int32_t e[8];
    fa::tile_entry(prefix.data(), cq.data(), ck.data(), nbatch, tq, tkv, reverse, r, e);
    printf("%d %d %d %d %d %d %d\n", e[0], e[1], e[2], e[3], e[4], e[5], e[6]);
  }
  return 0;
}
