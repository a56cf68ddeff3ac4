// Which (query row, key) tiles the prefill and backward kernels visit.
//
// The visible set (Gemma 2 model card, "Method" pseudocode and "Paper vs
// code"; Gemma 2 Guide, section 2): query row t sits at position
// p = t + S - T and sees key j iff j <= p and, on a local layer, j > p - W.
// The kernels walk blocks of rows against tiles of keys; these functions
// decide, from the band of positions a block of rows covers, which key tiles
// can hold a visible pair (the rest are skipped) and which tiles hold only
// visible pairs (those skip the per-element mask test).  They are plain
// integer arithmetic, evaluated once per workgroup, wave or tile, and are
// compiled both into the kernels and into a host-side check that compares
// them with a brute-force enumeration of the visible pairs.
//
// G2_TILES_FN supplies the function qualifiers: the kernels' sources define it
// as `__host__ __device__ inline` before including this header; the host-side
// check defines it as `inline`.
#pragma once

#ifndef G2_TILES_FN
#error "define G2_TILES_FN before including g2_tiles.h"
#endif

namespace g2 {

G2_TILES_FN int tiles_imin(int a, int b) { return a < b ? a : b; }
G2_TILES_FN int tiles_imax(int a, int b) { return a > b ? a : b; }

// The band of keys a block of rows [t_first, t_last] (t_first <= t_last < T)
// can see.  Every term fits an int: positions are below S, and p - W + 1 is
// at least 1 - W >= 1 - INT_MAX.
struct RowBand {
  int p_first, p_last;        // positions of the first and the last row
  int j_lo_first, j_lo_last;  // lowest key the first / the last row sees
};

G2_TILES_FN RowBand row_band(int t_first, int t_last, int T, int S, int W, int is_local) {
  RowBand r;
  r.p_first = t_first + (S - T);
  r.p_last = t_last + (S - T);
  r.j_lo_first = is_local ? tiles_imax(0, r.p_first - W + 1) : 0;
  r.j_lo_last = is_local ? tiles_imax(0, r.p_last - W + 1) : 0;
  return r;
}

// Key tiles of BN keys (aligned to BN) a workgroup walks: from the tile
// holding the lowest key its first row sees to the tile holding its last
// row's position.  Always at least one tile.
struct KeyTiles {
  int n_start, n_tiles;
};

G2_TILES_FN KeyTiles key_tiles(const RowBand& r, int BN) {
  KeyTiles k;
  k.n_start = (r.j_lo_first / BN) * BN;
  k.n_tiles = (r.p_last - k.n_start) / BN + 1;
  return k;
}

// No row of the band sees any key of [n0, n0 + n): the keys are all in the
// future of the last row, or all at or before the first row's window start.
G2_TILES_FN bool keys_unseen(const RowBand& r, int n0, int n) {
  return n0 > r.p_last || n0 + n - 1 < r.j_lo_first;
}

// Some pair of a row of the band and a key of [n0, n0 + n) is not visible,
// so the tile needs the per-element mask: a key past the first row's
// position, a key at or past S, or (local) a key at or below the last row's
// window start.  When this is false every row sees every key of the tile.
G2_TILES_FN bool keys_need_mask(const RowBand& r, int n0, int n, int S, int is_local) {
  return (n0 + n - 1 > r.p_first) || (n0 + n > S) || (is_local && n0 < r.j_lo_last);
}

// Rows of the backward's key-stationary kernel: the query rows that can see
// any key of [j0, j0 + KB), grouped in QT-row tiles from row t_lo (a multiple
// of QT).  A row sees the block iff p >= j0 and, on a local layer,
// p <= j0 + KB - 1 + W - 1; that bound is formed in 64 bits (W may be as
// large as INT_MAX).  n_pos = 0 when no row sees the block: chunked local
// layers (T < S) have key blocks older than every query's window.
struct RowTiles {
  int t_lo, n_pos;
};

G2_TILES_FN RowTiles rows_seeing_keys(int j0, int KB, int T, int S, int W, int is_local, int QT) {
  const long long off = (long long)S - T;
  long long lo = (long long)j0 - off;
  if (lo < 0) lo = 0;
  long long hi = T - 1;
  if (is_local) {
    const long long h2 = (long long)j0 + KB - 1 + (long long)W - 1 - off;
    if (h2 < hi) hi = h2;
  }
  RowTiles r;
  if (hi < lo || lo > T - 1) {
    r.t_lo = 0;
    r.n_pos = 0;
    return r;
  }
  r.t_lo = (int)(lo / QT) * QT;
  r.n_pos = (int)((hi - r.t_lo) / QT) + 1;
  return r;
}

// The backward's dS blocks: dS for query rows [32 tt, 32 tt + 32) of one head
// and keys [16 kb, 16 kb + 16).  The key-stationary kernel writes exactly the
// blocks for which this is true (every other block is all zero and is never
// written); the dQ kernel reads exactly those.  Blocks past T or S are unseen.
constexpr int kDsRows = 32;
constexpr int kDsKeys = 16;

G2_TILES_FN bool ds_block_seen(int tt, int kb, int T, int S, int W, int is_local) {
  const int t_first = tt * kDsRows, j0 = kb * kDsKeys;
  if (tt < 0 || kb < 0 || t_first >= T || j0 >= S) return false;
  const RowBand r = row_band(t_first, tiles_imin(t_first + kDsRows - 1, T - 1), T, S, W, is_local);
  return !keys_unseen(r, j0, kDsKeys);
}

}  // namespace g2
