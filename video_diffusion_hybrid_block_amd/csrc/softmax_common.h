// Work decomposition and key addressing shared by the softmax kernels of the
// forward and the backward pass: a work item is a tile of video rows of one
// (batch, head, frame); its partner set (the keys a query frame sees, or -
// the visibility relation being symmetric - the queries that see a key frame)
// is <= 3 contiguous video token ranges plus the text block, walked as one
// virtual sequence.
// [PaperDaily "伯克利与Impossible视频生成:14.3秒视频6.70秒去噪" §二 (chunks of five,
//  own chunk +- 1, the first and last frame seen by and seeing every frame)]
#pragma once

#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

inline constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int frame_in_order(const Geo& g, int vfr) {
  int first = g.af ? 0 : -1;
  int last = (g.al && !(g.af && g.T == 1)) ? g.T - 1 : -1;
  int na = (first >= 0) + (last >= 0);
  if (vfr < na) return (vfr == 0 && first >= 0) ? first : last;
  return vfr - na + (g.af ? 1 : 0);
}

struct WorkItem {
  int b, h, t, tile;
};

__device__ __forceinline__ WorkItem decode_work(const Geo& g, int B, int H, int tpf) {
  int i = blockIdx.x;
  int G = B * H;
  int gi, rest;
  if ((G & 7) == 0) {
    int xcd = i & 7, j = i >> 3, gper = G >> 3;
    gi = xcd * gper + j % gper;
    rest = j / gper;
  } else {
    gi = i % G;
    rest = i / G;
  }
  WorkItem w;
  w.b = gi / H;
  w.h = gi % H;
  w.t = frame_in_order(g, rest / tpf);
  w.tile = rest % tpf;
  return w;
}

// Row permutation inside a 32-key block: MFMA row m holds key pi(m), so the
// score registers of lane half h hold keys 8h..8h+7 and 16+8h..16+8h+7.
__device__ __forceinline__ int perm32(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

struct KeyMap {
  int s0, n0, s1, n1, s2, n2, nvid, nkeys;
};

__device__ __forceinline__ KeyMap key_map(const Geo& g, int t) {
  int ss[3] = {0, 0, 0}, sl[3] = {0, 0, 0};
  key_segments(g, t, ss, sl);
  KeyMap m;
  m.s0 = ss[0]; m.n0 = sl[0];
  m.s1 = ss[1]; m.n1 = sl[1];
  m.s2 = ss[2]; m.n2 = sl[2];
  m.nvid = m.n0 + m.n1 + m.n2;
  m.nkeys = m.nvid + g.L;
  return m;
}

// Element offset of virtual key kv of (b, h) in the video or text tensor;
// keys past the end are clamped to the first visible key (their scores are
// masked).  Returns true when the key is a text key.
__device__ __forceinline__ bool key_src(const KeyMap& m, int kv, int b, int h, int H, int N,
                                        int L, int D, size_t& off) {
  if (kv < m.nvid) {
    int tok = kv < m.n0 ? m.s0 + kv : (kv < m.n0 + m.n1 ? m.s1 + kv - m.n0 : m.s2 + kv - m.n0 - m.n1);
    off = ((size_t)(b * (size_t)N + tok) * H + h) * D;
    return false;
  }
  if (kv < m.nkeys) {
    off = ((size_t)(b * (size_t)L + (kv - m.nvid)) * H + h) * D;
    return true;
  }
  off = ((size_t)(b * (size_t)N + m.s0) * H + h) * D;
  return false;
}

// Branch-free form for the MFMA kernel: element offset (relative to the
// head's base pointer, in units of H*D elements per token) and text flag.
struct KeyAddr {
  int e0, e1, e2, nkeys;   // ends of the three video segments and of the text
  int d0, d1, d2;          // token = kv + d_seg inside video segment seg
  int clamp_tok;
};

__device__ __forceinline__ KeyAddr key_addr(const KeyMap& m) {
  KeyAddr a;
  a.e0 = m.n0; a.e1 = m.n0 + m.n1; a.e2 = m.nvid; a.nkeys = m.nkeys;
  a.d0 = m.s0; a.d1 = m.s1 - m.n0; a.d2 = m.s2 - m.n0 - m.n1;
  a.clamp_tok = m.s0;
  return a;
}

// Token row of virtual key kv; `text` tells which tensor it indexes.
// Returns the row, plus 0x40000000 when the key is a text key.
__device__ __forceinline__ int key_row(KeyAddr a, int kv) {
  int d = kv < a.e0 ? a.d0 : (kv < a.e1 ? a.d1 : a.d2);
  bool text = (kv >= a.e2) & (kv < a.nkeys);
  int vtok = kv < a.e2 ? kv + d : a.clamp_tok;
  return text ? ((kv - a.e2) | 0x40000000) : vtok;
}

// Work order of the MFMA kernel.  Anchor-frame tiles (every key of the head)
// come first.  When B*H is a multiple of 8, XCD x (blocks x, x+8, ...) owns
// heads x*G/8 .. and walks them head by head, so the ~64 workgroups resident
// on one XCD belong to a few neighbouring chunks of one head and stream the
// same keys through that XCD's L2 at about the same time.
__device__ __forceinline__ WorkItem decode_work_xcd(const Geo& g, int B, int H, int tpf) {
  const int G = B * H;
  if ((G & 7) != 0) return decode_work(g, B, H, tpf);
  const int i = blockIdx.x;
  const int xcd = i & 7, j = i >> 3, gper = G >> 3;
  const int first = g.af ? 0 : -1;
  const int last = (g.al && !(g.af && g.T == 1)) ? g.T - 1 : -1;
  const int na = (first >= 0) + (last >= 0);
  const int nanchor_items = na * tpf * gper;
  int gl, t, tile;
  if (j < nanchor_items) {
    gl = j % gper;
    const int r = j / gper;
    t = (r / tpf == 0 && first >= 0) ? first : last;
    tile = r % tpf;
  } else {
    const int jj = j - nanchor_items;
    const int per_head = (g.T - na) * tpf;
    gl = jj / per_head;
    const int r = jj % per_head;
    t = r / tpf + (g.af ? 1 : 0);
    tile = r % tpf;
  }
  const int gi = xcd * gper + gl;
  WorkItem w;
  w.b = gi / H;
  w.h = gi % H;
  w.t = t;
  w.tile = tile;
  return w;
}

}  // namespace vdn
