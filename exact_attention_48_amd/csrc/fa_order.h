// fa_order.h -- the order in which the kernels' workgroups take their work.
//
// Workgroup b of a launch runs on XCD b % 8, and each of the 8 XCDs has its own
// L2, so the order of the work items decides which tiles share an L2.
//
// Uniform batches: level-major. Query-tile kernels (forward, dQ) take the
// items (tile level, sequence, query head), the heaviest (last) query tile
// first so the longest items start first; the G query heads of one K/V head
// (G consecutive items) go to one XCD and stream their K/V rows from one L2.
// The dK/dV kernel takes (key tile, sequence, K/V head), key tile 0 (the
// heaviest under causal masking) first. All sequences have one length, so the
// items of one level run side by side through the same rows.
//
// Packed batches: XCD-grouped. Level-major order would interleave sequences of
// different lengths; they drift apart and the workgroups resident on one XCD
// end up reading rows of many sequences, so nearly every tile read misses that
// XCD's L2. Instead XCD x takes, of every sequence, the K/V heads
// hkv = x / nc (mod 8 / nc) and the tiles t = x % nc (mod nc), nc = 8 / gcd(Hkv, 8)
// (every XCD then holds the same share of every sequence, whatever the
// lengths), and works through that share sequence by sequence and K/V head by
// K/V head, heaviest tiles first, the G query heads of a K/V head side by side.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct TileItem {
  int s;   // sequence
  int h;   // query head (query-tile kernels) or K/V head (dK/dV)
  int t;   // tile index within the sequence
};

// ---- query-tile kernels (forward, dQ): n_qt tiles per (sequence, query head) ----

inline long q_grid_level(int B, int Hq, int G, int n_qt) {
  const long n = (long)B * Hq * n_qt, g8 = 8L * G;
  return (n + g8 - 1) / g8 * g8;
}

__device__ __forceinline__ bool q_item_level(int b, int B, int Hq, int G, int n_qt, bool lpt, TileItem& it) {
  const int xcd = b & 7, j = b >> 3;
  const int w = (8 * (j / G) + xcd) * G + (j % G);   // XCD x: item groups x, x + 8, ...
  const int per_level = B * Hq;
  if (w >= per_level * n_qt) return false;
  const int lvl = w / per_level, rr = w - lvl * per_level;
  it.s = rr / Hq;
  it.h = rr - it.s * Hq;
  it.t = lpt ? n_qt - 1 - lvl : lvl;
  return true;
}

// Packed batches count every sequence as n_qt tiles long (the caller's N bounds
// every length); items past a sequence's end are the caller's to skip.
inline long q_grid_xcd(int B, int Hkv, int G, int nc, int n_qt) {
  return 8L * B * (Hkv * nc / 8) * ((n_qt + nc - 1) / nc) * G;
}

__device__ __forceinline__ bool q_item_xcd(int b, int B, int Hkv, int G, int nc, int n_qt, bool lpt,
                                           TileItem& it) {
  const int xcd = b & 7, j = b >> 3;
  const int ci = xcd % nc;                         // tile residue of this XCD
  const int cnt = (n_qt - ci + nc - 1) / nc;       // its tiles per (sequence, query head)
  if (cnt <= 0) return false;
  const int per_hkv = cnt * G;
  const int per_seq = (Hkv * nc / 8) * per_hkv;
  const int s = j / per_seq;
  if (s >= B) return false;
  int rr = j - s * per_seq;
  const int u = rr / per_hkv;
  rr -= u * per_hkv;
  const int k = rr / G;
  it.s = s;
  it.h = (xcd / nc + (8 / nc) * u) * G + (rr - k * G);
  it.t = ci + nc * (lpt ? cnt - 1 - k : k);
  return true;
}

// ---- dK/dV: n_kt key tiles per (sequence, K/V head) ----

inline long kv_grid_level(int B, int Hkv, int n_kt) { return (long)B * Hkv * n_kt; }

__device__ __forceinline__ bool kv_item_level(int b, int B, int Hkv, int n_kt, TileItem& it) {
  const int per_level = B * Hkv;
  if (b >= per_level * n_kt) return false;
  const int kt = b / per_level, rr = b - kt * per_level;
  it.s = rr / Hkv;
  it.h = rr - it.s * Hkv;
  it.t = kt;
  return true;
}

inline long kv_grid_xcd(int B, int Hkv, int nc, int n_kt) {
  return 8L * B * (Hkv * nc / 8) * ((n_kt + nc - 1) / nc);
}

// Packed batches: `prefix` (nc rows of B + 1) gives, for residue i and
// sequence s, the key tiles kt = i (mod nc) of sequences 0 .. s-1, so the
// workgroup finds its sequence by binary search and no workgroup is spent on
// tiles past a sequence's end. n_kt bounds every sequence's key tiles.
__device__ __forceinline__ bool kv_item_xcd(int b, int B, int Hkv, int nc, int n_kt, const int* prefix,
                                            TileItem& it) {
  const int xcd = b & 7, j = b >> 3;
  const int ci = xcd % nc;
  const int m = Hkv * nc / 8;                      // K/V heads per sequence on this XCD
  const int* P = prefix + ci * (B + 1);
  if (j >= m * P[B]) return false;
  int lo = 0, hi = B - 1;                          // largest s with m * P[s] <= j
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (m * P[mid] <= j) lo = mid;
    else hi = mid - 1;
  }
  const int cnt = P[lo + 1] - P[lo];
  const int jj = j - m * P[lo];
  // a table the preparation kernel did not write cannot send a workgroup
  // outside the problem: out-of-range entries end it here (or at the caller's
  // tile-past-the-end check, which the bound on cnt keeps free of overflow)
  if (cnt <= 0 || cnt > (n_kt + nc - 1) / nc || jj < 0 || jj >= m * cnt) return false;
  const int u = jj / cnt;
  it.s = lo;
  it.h = xcd / nc + (8 / nc) * u;
  it.t = ci + nc * (jj - u * cnt);
  return true;
}

}  // namespace fa
