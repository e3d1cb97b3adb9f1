// Index math of the connector's permutations, written once for the kernels
// and for a host build that checks it (index_check.cpp, IVC_DEBUG):
//
//  * pixel_shuffle v2 ([14B] pixel_shuffle section): token (a, b) of the
//    (P/r) x (P/r) output grid gathers the r x r cells grid[r*a + m][r*b + k],
//    cell (m, k) in channel block r*m + k; grid[i][j] is ViT row
//    has_cls + i*P + j of its tile.  v1 ([14B] v1/v2 section) writes token
//    (a, b) at b*(P/r) + a.  The 64-token path as two r = 2 shuffles
//    ([2B-Flash] three token levels) puts cell (2*m2 + m, 2*k2 + k) of the
//    4 x 4 block in channel block 4*(2*m2 + k2) + (2*m + k);
//  * the folded products' gathered A rows (LayerNorm folded into the first
//    product: logical row m is shuffled token m % S of tile list[m / S]);
//  * the compaction closed form ([4B-Flash] section 4; [14B] token
//    injection): with k IMG_CONTEXT tokens before position p, the slots
//    deleted before p are (S - S64) * routed_before[k / S]
//    + use64[k / S] * max(0, k % S - S64), so a kept token lands at p minus that.
//
// IVC_DEBUG (host build only) turns IVC_INDEX_CHECK into a bounds check that
// reports through ivc_index_fail.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define IVC_HD __host__ __device__ __forceinline__
#else
#define IVC_HD inline
#endif

#ifdef IVC_DEBUG
extern "C" void ivc_index_fail(const char* what, long long v, long long lo, long long hi);
#define IVC_INDEX_CHECK(what, v, lo, hi)                                        \
  do {                                                                          \
    const long long v_ = (long long)(v);                                        \
    if (v_ < (long long)(lo) || v_ >= (long long)(hi)) ivc_index_fail(what, v_, lo, hi); \
  } while (0)
#else
#define IVC_INDEX_CHECK(what, v, lo, hi) ((void)0)
#endif

namespace ivc {

// ---- pixel_shuffle ----------------------------------------------------------
// Row of grid cell (gi, gj) inside its tile (CLS skipped).
IVC_HD int ps_cell_row(int P, int has_cls, int gi, int gj) {
  IVC_INDEX_CHECK("grid row", gi, 0, P);
  IVC_INDEX_CHECK("grid column", gj, 0, P);
  return has_cls + gi * P + gj;
}

// Output token of grid block (a, b) in a Q x Q token grid (Q = P / r).
IVC_HD int ps_token(int Q, int a, int b, int v1) {
  IVC_INDEX_CHECK("token row", a, 0, Q);
  IVC_INDEX_CHECK("token column", b, 0, Q);
  return v1 ? b * Q + a : a * Q + b;
}

// 64-token path: channel block of cell q (= 2m + k) of 2 x 2 sub-block w
// (= 2*m2 + k2) of the 4 x 4 block, i.e. grid offset (2*m2 + m, 2*k2 + k).
IVC_HD int ps64_channel_block(int w, int q, int twice) {
  IVC_INDEX_CHECK("sub-block", w, 0, 4);
  IVC_INDEX_CHECK("cell", q, 0, 4);
  const int m4 = 2 * (w >> 1) + (q >> 1), k4 = 2 * (w & 1) + (q & 1);
  return twice ? 4 * w + q : 4 * m4 + k4;
}

// ---- gathered A of the folded products ---------------------------------------
// G has the fields of AGather: list (nullable), rows, has_cls, P, r, C, v1, twice.

// ViT row of cell 0 of logical row m's r x r grid block.
template <class G>
IVC_HD long long gather_row0(const G& g, int m) {
  const int Q = g.P / g.r, S = Q * Q;
  const int rank = m / S, s = m - rank * S;
  const int t = g.list != nullptr ? g.list[rank] : rank;
  const int qa = s / Q, qb = s - qa * Q;
  const int a = g.v1 ? qb : qa, b = g.v1 ? qa : qb;  // v1: token (a, b) sits at b*Q + a
  return (long long)t * g.rows + g.has_cls + (long long)(g.r * a) * g.P + g.r * b;
}

// Base row of a product tile whose first logical row is m0: the first grid
// row of m0's ViT tile.  Every row the tile gathers lies at or after it (the
// tile's later rows belong to the same tile or to later ones, and the
// per-path tile lists are increasing), so offsets from it are never
// negative, whatever the token order inside a tile (v1 visits a tile's rows
// out of order, so m0's own row is not always the smallest).
template <class G>
IVC_HD long long gather_base(const G& g, int m0) {
  const int Q = g.P / g.r, S = Q * Q;
  const int rank = m0 / S;
  const int t = g.list != nullptr ? g.list[rank] : rank;
  return (long long)t * g.rows + g.has_cls;
}

// Grid offset (dm, dk) of cell q inside the r x r block (r = 2 or 4; the
// two-r=2 order for r = 4: q = 4*(2*m2 + k2) + (2*m + k)).
template <class G>
IVC_HD void gather_cell(const G& g, int q, int* dm, int* dk) {
  IVC_INDEX_CHECK("cell of the block", q, 0, g.r * g.r);
  if (g.twice) {
    const int w = q >> 2, qq = q & 3;
    *dm = 2 * (w >> 1) + (qq >> 1);
    *dk = 2 * (w & 1) + (qq & 1);
  } else {
    const int sh = g.r == 4 ? 2 : 1;
    *dm = q >> sh;
    *dk = q & (g.r - 1);
  }
}

// Byte offset of channels [c0, c0 + 64) of cell q relative to cell 0's row.
template <class G>
IVC_HD long long gather_koff(const G& g, int q, int c0) {
  int dm, dk;
  gather_cell(g, q, &dm, &dk);
  IVC_INDEX_CHECK("channel", c0, 0, g.C);
  return ((long long)(dm * g.P + dk) * g.C + c0) * 2;
}

// ---- compaction -------------------------------------------------------------
// Slots deleted before a position preceded by k IMG_CONTEXT tokens, for a
// sequence of T tiles of S slots (S64 kept by a routed tile); k may equal
// T*S (positions after the last slot).
IVC_HD long long compact_deleted_before(int k, int T, int S, int S64,
                                        const int32_t* routed_before, const uint8_t* use64) {
  const int tile = k / S, loc = k - tile * S;
  const long long drop = S - S64;
  if (tile >= T) return drop * routed_before[T];
  IVC_INDEX_CHECK("slot tile", tile, 0, T);
  const int u = use64[tile] != 0;
  return drop * routed_before[tile] + (u ? (loc > S64 ? loc - S64 : 0) : 0);
}

// Whether the slot preceded by k IMG_CONTEXT tokens survives.
IVC_HD bool compact_keeps_slot(int k, int T, int S, int S64, const uint8_t* use64) {
  const int tile = k / S, loc = k - tile * S;
  if (tile >= T) return false;  // more slots than tiles: the status word reports it
  return use64[tile] == 0 || loc < S64;
}

}  // namespace ivc
