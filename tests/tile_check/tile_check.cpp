// Host-side check of the kernels' tile-range arithmetic (csrc/g2_tiles.h)
// against a brute-force enumeration of the visible (query row, key) pairs.
//
// Visible set (Gemma 2 model card, "Method" pseudocode and "Paper vs code";
// Guide section 2): row t sits at position p = t + S - T and sees key j iff
// j <= p and, on a local layer, j > p - W.
//
// For each (T, S, W, local) of a grid, and each kernel's blocking:
//   * every visible pair lies in a tile the kernel walks and does not skip;
//   * every tile walked without the mask holds only visible pairs;
//   * walked key tiles start inside [0, S); row tiles start inside [0, T);
//   * the backward's dS blocks (32 rows x 16 keys) that the key-stationary
//     kernel writes are exactly those holding a visible pair, and it visits
//     every one of them.
// Prints one line per failure and "tile check: N cases, 0 failures" at the end;
// the exit status is the number of failures (capped at 100).
#include <climits>
#include <cstdio>
#include <vector>

#define G2_TILES_FN inline
#include "g2_tiles.h"

using namespace g2;

static long long failures = 0;
static void fail(const char* what, int T, int S, int W, int local, int a, int b) {
  if (failures < 40)
    std::printf("FAIL %s: T=%d S=%d W=%d local=%d at %d %d\n", what, T, S, W, local, a, b);
  ++failures;
}

static bool visible(int t, int j, int T, int S, int W, int local) {
  const long long p = (long long)t + S - T;
  if (j < 0 || j >= S || j > p) return false;
  return !local || (long long)j > p - W;
}

// Forward and dQ kernels: blocks of BMP rows, waves of QPW rows, key tiles of BN.
static void check_query_blocked(int T, int S, int W, int local, int BMP, int QPW, int BN) {
  for (int m0 = 0; m0 < T; m0 += BMP) {
    const int m1 = (m0 + BMP < T ? m0 + BMP : T) - 1;
    const KeyTiles kt = key_tiles(row_band(m0, m1, T, S, W, local), BN);
    if (kt.n_start < 0 || kt.n_tiles < 1 || kt.n_start % BN) fail("key range", T, S, W, local, m0, kt.n_start);
    if (kt.n_start + (kt.n_tiles - 1) * BN >= S) fail("key tile past S", T, S, W, local, m0, kt.n_tiles);
    for (int t0 = m0; t0 <= m1; t0 += QPW) {
      const int t1 = (t0 + QPW - 1 < T - 1 ? t0 + QPW - 1 : T - 1);
      const RowBand wb = row_band(t0, t1, T, S, W, local);
      // every visible pair of the wave's rows is in a walked, unskipped tile
      for (int t = t0; t <= t1; ++t)
        for (int j = 0; j < S; ++j) {
          if (!visible(t, j, T, S, W, local)) continue;
          const int n0 = (j / BN) * BN;
          if (n0 < kt.n_start || n0 >= kt.n_start + kt.n_tiles * BN) fail("pair outside walked tiles", T, S, W, local, t, j);
          else if (keys_unseen(wb, n0, BN)) fail("visible pair in a skipped tile", T, S, W, local, t, j);
        }
      // tiles walked without the mask hold only visible pairs
      for (int i = 0; i < kt.n_tiles; ++i) {
        const int n0 = kt.n_start + i * BN;
        if (keys_unseen(wb, n0, BN) || keys_need_mask(wb, n0, BN, S, local)) continue;
        for (int t = t0; t <= t1; ++t)
          for (int j = n0; j < n0 + BN; ++j)
            if (!visible(t, j, T, S, W, local)) fail("unmasked tile holds a hidden pair", T, S, W, local, t, j);
      }
    }
  }
}

// dK/dV kernel: blocks of KB keys, waves of KW keys, row tiles of QT.
static void check_key_blocked(int T, int S, int W, int local, int KB, int KW, int QT) {
  for (int j0 = 0; j0 < S; j0 += KB) {
    const RowTiles rt = rows_seeing_keys(j0, KB, T, S, W, local, QT);
    if (rt.n_pos < 0 || rt.t_lo < 0 || rt.t_lo % QT) fail("row range", T, S, W, local, j0, rt.n_pos);
    if (rt.n_pos > 0 && rt.t_lo + (rt.n_pos - 1) * QT >= T) fail("row tile past T", T, S, W, local, j0, rt.n_pos);
    for (int jw = j0; jw < j0 + KB; jw += KW) {
      for (int j = jw; j < jw + KW && j < S; ++j)
        for (int t = 0; t < T; ++t) {
          if (!visible(t, j, T, S, W, local)) continue;
          if (t < rt.t_lo || t >= rt.t_lo + rt.n_pos * QT) { fail("pair outside walked rows", T, S, W, local, t, j); continue; }
          const int t0 = rt.t_lo + ((t - rt.t_lo) / QT) * QT;
          const int t1 = (t0 + QT - 1 < T - 1 ? t0 + QT - 1 : T - 1);
          if (jw >= S || keys_unseen(row_band(t0, t1, T, S, W, local), jw, KW))
            fail("visible pair in a skipped row tile", T, S, W, local, t, j);
        }
      for (int i = 0; i < rt.n_pos; ++i) {
        const int t0 = rt.t_lo + i * QT;
        const int t1 = (t0 + QT - 1 < T - 1 ? t0 + QT - 1 : T - 1);
        const RowBand rb = row_band(t0, t1, T, S, W, local);
        if (jw >= S || keys_unseen(rb, jw, KW)) continue;
        if (keys_need_mask(rb, jw, KW, S, local) || t0 + QT > T) continue;
        for (int t = t0; t < t0 + QT; ++t)
          for (int j = jw; j < jw + KW; ++j)
            if (!visible(t, j, T, S, W, local)) fail("unmasked row tile holds a hidden pair", T, S, W, local, t, j);
      }
    }
  }
}

// dS blocks: seen iff the block holds a visible pair; the dK/dV kernel
// (blocks of KB keys, waves of 16 keys, row tiles of 32) reaches every seen one.
static void check_ds_blocks(int T, int S, int W, int local, int KB) {
  const int n_tt = (T + kDsRows - 1) / kDsRows + 1, n_kb = (S + kDsKeys - 1) / kDsKeys + 1;
  for (int tt = 0; tt < n_tt; ++tt)
    for (int kb = 0; kb < n_kb; ++kb) {
      bool any = false;
      for (int t = tt * kDsRows; t < (tt + 1) * kDsRows && t < T && !any; ++t)
        for (int j = kb * kDsKeys; j < (kb + 1) * kDsKeys && j < S && !any; ++j) any = visible(t, j, T, S, W, local);
      const bool seen = ds_block_seen(tt, kb, T, S, W, local);
      if (seen != any) fail(any ? "dS block with a visible pair not seen" : "dS block seen without a visible pair", T, S, W, local, tt, kb);
      if (!seen) continue;
      const int j0 = (kb * kDsKeys / KB) * KB, jw = kb * kDsKeys;
      const RowTiles rt = rows_seeing_keys(j0, KB, T, S, W, local, kDsRows);
      if (tt * kDsRows < rt.t_lo || tt * kDsRows >= rt.t_lo + rt.n_pos * kDsRows) {
        fail("seen dS block outside the dK/dV kernel's rows", T, S, W, local, tt, kb);
        continue;
      }
      const int t0 = tt * kDsRows, t1 = (t0 + kDsRows - 1 < T - 1 ? t0 + kDsRows - 1 : T - 1);
      if (jw >= S || keys_unseen(row_band(t0, t1, T, S, W, local), jw, kDsKeys))
        fail("seen dS block skipped by the dK/dV kernel", T, S, W, local, tt, kb);
    }
}

int main() {
  std::vector<int> Ts = {1, 2, 17, 31, 32, 33, 64, 100, 129, 200, 257, 300};
  std::vector<int> extra_S = {0, 1, 31, 63, 64, 160, 230};
  std::vector<int> Ws = {1, 2, 16, 31, 32, 37, 60, 64, 65, 100, 128, 300, 4096, INT_MAX - 5, INT_MAX};
  long long cases = 0;
  for (int T : Ts)
    for (int dS : extra_S)
      for (int W : Ws)
        for (int local = 0; local < 2; ++local) {
          if (!local && W != 1) continue;  // the window only matters on local layers
          const int S = T + dS;
          check_query_blocked(T, S, W, local, 128, 32, 32);   // forward, d = 256, two heads per K/V head
          check_query_blocked(T, S, W, local, 256, 32, 32);   // forward, d = 256, one head per K/V head
          check_query_blocked(T, S, W, local, 128, 32, 64);   // forward, d <= 128
          check_query_blocked(T, S, W, local, 64, 64, 32);    // dQ, d = 256, two heads per K/V head
          check_query_blocked(T, S, W, local, 128, 64, 32);   // dQ, d = 256 one head, d <= 128 two heads
          check_query_blocked(T, S, W, local, 256, 64, 32);   // dQ, d <= 128, one head per K/V head
          check_key_blocked(T, S, W, local, 64, 16, 32);      // dK/dV
          check_ds_blocks(T, S, W, local, 64);                // dS blocks between the two
          ++cases;
        }
  // the advisor's example: a chunked local layer whose first key block no row sees
  const RowTiles r = rows_seeing_keys(0, 64, 100, 260, 60, 1, 32);
  if (r.n_pos != 0) fail("T=100 S=260 W=60 key block 0 must have no rows", 100, 260, 60, 1, r.t_lo, r.n_pos);
  std::printf("tile check: %lld cases, %lld failures\n", cases, failures);
  return failures > 100 ? 100 : (int)failures;
}
