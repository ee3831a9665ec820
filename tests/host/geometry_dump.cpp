// Host build of the library's device-side index math (rf_internal.h) for CPU
// tests: derives the geometry through rf_derive() and prints, for every
// permuted row, the natural row it comes from, then every block's (row0, len).
// Usage: geometry_dump P T H W first_frame sparsity min_blocks
#include <stdio.h>
#include <stdlib.h>

#include "rf_internal.h"

int main(int argc, char** argv) {
  if (argc != 8) return 2;
  rf_desc d = {};
  d.layout = RF_LAYOUT_BNSD;
  d.dtype = RF_DTYPE_BF16;
  d.batch = 1;
  d.heads_q = 1;
  d.heads_kv = 1;
  d.head_dim = 64;
  d.prefix_len = atoll(argv[1]);
  d.grid_t = atoi(argv[2]);
  d.grid_h = atoi(argv[3]);
  d.grid_w = atoi(argv[4]);
  d.first_frame_rows = atoi(argv[5]) ? (int64_t)d.grid_h * d.grid_w : 0;
  d.sparsity = atof(argv[6]);
  d.min_sparse_blocks = atoi(argv[7]);
  d.seq_len = d.prefix_len + (int64_t)d.grid_t * d.grid_h * d.grid_w;
  d.block_shape[0] = d.block_shape[1] = 128;
  d.scale = 0.125f;
  RfGeom g;
  rf_plan_info info;
  rf_status s = rf_derive(&d, &g, &info);
  if (s != RF_OK) {
    printf("status %d\n", (int)s);
    return 1;
  }
  printf("%lld\n", (long long)g.S);
  for (int64_t r = 0; r < g.S; ++r) printf("%lld\n", (long long)rf_natural_row(g, r));
  printf("%d\n", g.n_blocks);
  for (int j = 0; j < g.n_blocks; ++j) {
    int64_t r0;
    int32_t len;
    rf_block_rows(g, j, &r0, &len);
    printf("%lld %d\n", (long long)r0, len);
  }
  return 0;
}
