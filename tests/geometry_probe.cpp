// Host-only dump of the frame geometry the kernels use (vdn_internal.h), for
// comparison with the oracle's definitions on the CPU.
// usage: geometry_probe T C w anchor_first anchor_last P
#include <cstdio>
#include <cstdlib>

#include "vdn_internal.h"

int main(int argc, char** argv) {
  if (argc != 7) return 2;
  vdn_layout_t l = {};
  l.batch = 1; l.heads = 1; l.head_dim_k = l.head_dim_v = 16;
  l.frames = atoi(argv[1]); l.chunk_frames = atoi(argv[2]); l.window_chunks = atoi(argv[3]);
  l.anchor_first = atoi(argv[4]); l.anchor_last = atoi(argv[5]); l.tokens_per_frame = atoi(argv[6]);
  vdn::Geo g = vdn::make_geo(l);
  printf("nc %d fwd_end %d bwd_begin %d\n", g.nc, vdn::fwd_scan_end(g), vdn::bwd_scan_begin(g));
  for (int t = 0; t < g.T; ++t) {
    int s[3], n[3];
    int k = vdn::key_segments(g, t, s, n);
    printf("seg %d", t);
    for (int i = 0; i < k; ++i) printf(" %d %d", s[i], n[i]);
    printf("\n");
  }
  for (int c = 0; c < g.nc; ++c) printf("win %d %d %d\n", c, vdn::win_lo(g, c), vdn::win_hi(g, c));
  for (int dir = 0; dir < 2; ++dir) {
    printf("fold %d", dir);
    for (int f = 0; f < g.T; ++f) printf(" %d", vdn::fold_index(g, dir, f));
    printf("\nsnap %d", dir);
    for (int c = 0; c < g.nc; ++c) printf(" %d", vdn::snap_index(g, dir, c));
    printf("\n");
  }
  int ns = vdn::count_slots(g, false);
  printf("slots");
  for (int i = 0; i < ns; ++i) printf(" %d", vdn::slot_of(g, i, false));
  printf("\n");
  return 0;
}
