// Host build of the connector's index math (index_math.h) with bounds checks
// on (IVC_DEBUG): walks the loader's, the folded products' and the
// compaction's index computations for a given shape exactly as the kernels
// decompose them, and returns what they address, so a CPU test can compare
// them element by element with the oracle's permutation and compaction.
// Built with g++ (no GPU code): vlm_visual_token_amd/libivc_index_check.so,
// and as a stand-alone sanitizer self-test (IVC_INDEX_CHECK_MAIN).
#ifndef IVC_DEBUG
#define IVC_DEBUG 1
#endif
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

#include "index_math.h"

static long long g_failures = 0;

extern "C" void ivc_index_fail(const char* what, long long v, long long lo, long long hi) {
  if (g_failures < 8) fprintf(stderr, "index check: %s = %lld outside [%lld, %lld)\n", what, v, lo, hi);
  ++g_failures;
}

namespace {
// The fields index_math.h's gather functions read (AGather's).
struct Gather {
  const int* list;
  int rows, has_cls, P, r, C, v1, twice;
};
}  // namespace

extern "C" {

long long ivc_index_failures(void) { return g_failures; }
void ivc_index_reset(void) { g_failures = 0; }

// Loader rows.  src[(t * Q*Q + tok) * r*r + blk] = t * rows + ViT row of
// channel block blk of output token tok, for r = 2 (one wave per 2 x 2 block)
// or r = 4 (a workgroup per 4 x 4 block, wave w = its 2 x 2 sub-block w).
// Returns the number of entries written.
long long ivc_check_loader_rows(int T, int P, int has_cls, int r, int v1, int twice,
                                long long* src) {
  const int rows = has_cls + P * P;
  long long n = 0;
  if (r == 2) {
    const int Q2 = P / 2;
    for (int t = 0; t < T; ++t)
      for (int a2 = 0; a2 < Q2; ++a2)
        for (int b2 = 0; b2 < Q2; ++b2) {
          const int tok = ivc::ps_token(Q2, a2, b2, v1);
          for (int q = 0; q < 4; ++q) {
            const int gi = 2 * a2 + (q >> 1), gj = 2 * b2 + (q & 1);
            src[((long long)t * Q2 * Q2 + tok) * 4 + q] =
                (long long)t * rows + ivc::ps_cell_row(P, has_cls, gi, gj);
            ++n;
          }
        }
    return n;
  }
  const int Q4 = P / 4;
  for (int t = 0; t < T; ++t)
    for (int a4 = 0; a4 < Q4; ++a4)
      for (int b4 = 0; b4 < Q4; ++b4) {
        const int tok = ivc::ps_token(Q4, a4, b4, v1);
        for (int w = 0; w < 4; ++w) {
          const int a2 = 2 * a4 + (w >> 1), b2 = 2 * b4 + (w & 1);
          for (int q = 0; q < 4; ++q) {
            const int gi = 2 * a2 + (q >> 1), gj = 2 * b2 + (q & 1);
            const int blk = ivc::ps64_channel_block(w, q, twice);
            IVC_INDEX_CHECK("64-path channel block", blk, 0, 16);
            src[((long long)t * Q4 * Q4 + tok) * 16 + blk] =
                (long long)t * rows + ivc::ps_cell_row(P, has_cls, gi, gj);
            ++n;
          }
        }
      }
  return n;
}

// Folded product's gathered A for M = n_list * (P/r)^2 logical rows (list:
// the path's tiles in increasing order, or NULL for tiles 0..n_list-1):
// src[m * r*r + q] = ViT row (global) of cell q of row m, as the DMA
// addresses it (base row of the row's 256-row product tile + the row's
// offset + the cell's offset).  Returns the number of rows whose offset
// from their tile's base is negative or does not fit the kernel's unsigned
// 32-bit byte offsets (must be 0).
long long ivc_check_gather(int P, int C, int has_cls, int r, int v1, int twice,
                           const int* list, int n_list, long long* src) {
  Gather g{list, has_cls + P * P, has_cls, P, r, C, v1, twice};
  const int Q = P / r, S = Q * Q;
  const long long M = (long long)n_list * S;
  long long bad = 0;
  for (long long m0 = 0; m0 < M; m0 += 256) {
    const long long base = ivc::gather_base(g, (int)m0);
    for (long long m = m0; m < std::min(M, m0 + 256); ++m) {
      const long long row0 = ivc::gather_row0(g, (int)m);
      const long long off = (row0 - base) * C * 2;  // bytes, as the kernel forms it
      if (off < 0 || off >= (1ll << 32)) ++bad;
      for (int q = 0; q < r * r; ++q) {
        const long long koff = ivc::gather_koff(g, q, 0);  // bytes from cell 0's row
        src[m * r * r + q] = base + (off + koff) / (2ll * C);
      }
    }
  }
  return bad;
}

// Compaction by the closed form, one position at a time as k_compact_map
// takes it: keep_map[p] = new index or -1; code[j] = source of output row j
// (text: position p; slot of tile t: 1<<60 | t*S + loc, or 2<<60 | t*S64 +
// loc when routed).  Returns L', or -1 when the IMG_CONTEXT count != T*S.
long long ivc_check_compact(const int32_t* ids, long long L, int img, const uint8_t* use64, int T,
                            int S, int S64, int32_t* keep_map, long long* code) {
  std::vector<int32_t> rb(T + 1, 0);
  for (int t = 0; t < T; ++t) rb[t + 1] = rb[t] + (use64[t] != 0);
  long long n_img = 0;
  for (long long p = 0; p < L; ++p) n_img += ids[p] == img;
  const bool ok = n_img == (long long)T * S;
  const long long Lp = ok ? L - (long long)(S - S64) * rb[T] : 0;
  int k = 0;
  for (long long p = 0; p < L; ++p) {
    const bool is_img = ids[p] == img;
    const long long f = ivc::compact_deleted_before(k, T, S, S64, rb.data(), use64);
    const bool keep = !is_img || ivc::compact_keeps_slot(k, T, S, S64, use64);
    const long long j = p - f;
    keep_map[p] = keep ? (int32_t)j : -1;
    if (keep) {
      IVC_INDEX_CHECK("output row", j, 0, L);
      const int tile = k / S, loc = k - tile * S;
      code[j] = !is_img ? p
                : use64[tile] != 0 ? ((2ll << 60) | ((long long)tile * S64 + loc))
                                   : ((1ll << 60) | ((long long)tile * S + loc));
    }
    if (is_img) ++k;
  }
  return ok ? Lp : -1;
}

}  // extern "C"

#ifdef IVC_INDEX_CHECK_MAIN
// Sanitizer self-test (AddressSanitizer + UndefinedBehaviorSanitizer build):
// runs every walk above over a range of grids into exactly-sized buffers and
// checks the closed forms against brute force; exit status 0 = clean.
int main() {
  long long errors = 0;
  for (int P : {4, 8, 12, 16, 24, 32, 40, 48})
    for (int has_cls : {0, 1})
      for (int v1 : {0, 1})
        for (int r : {2, 4}) {
          if (P % r) continue;
          for (int twice : {0, 1}) {
            if (twice && r != 4) continue;
            const int T = 3, Q = P / r, S = Q * Q, rows = has_cls + P * P;
            std::vector<long long> a((size_t)T * S * r * r), b((size_t)T * S * r * r);
            ivc_check_loader_rows(T, P, has_cls, r, v1, twice, a.data());
            // the loader reads every grid row of a tile exactly once per path
            for (int t = 0; t < T; ++t) {
              std::vector<int> seen(rows, 0);
              for (long long e = (long long)t * S * r * r; e < (long long)(t + 1) * S * r * r; ++e) {
                const long long rr = a[e] - (long long)t * rows;
                if (rr < has_cls || rr >= rows || seen[rr]++) ++errors;
              }
            }
            std::vector<int> list = {0, 2, 5};  // increasing, with gaps
            const long long bad = ivc_check_gather(P, 64, has_cls, r, v1, twice, list.data(), 3,
                                                   b.data());
            errors += bad;
            // every gathered row is one of its tile's grid rows, each used once
            for (int i = 0; i < 3; ++i) {
              std::vector<int> seen(rows, 0);
              for (long long e = (long long)i * S * r * r; e < (long long)(i + 1) * S * r * r; ++e) {
                const long long rr = b[e] - (long long)list[i] * rows;
                if (rr < has_cls || rr >= rows || seen[rr]++) ++errors;
              }
            }
          }
        }
  // compaction: closed form against a brute-force walk
  for (int T : {1, 3, 7}) {
    const int S = 16, S64 = 4, img = 99;
    std::vector<int32_t> ids;
    for (int t = 0; t < T; ++t) {
      ids.push_back(t);
      for (int s = 0; s < S; ++s) ids.push_back(img);
    }
    ids.push_back(7);
    std::vector<uint8_t> use(T);
    for (int t = 0; t < T; ++t) use[t] = (uint8_t)(t % 2);
    std::vector<int32_t> km(ids.size());
    std::vector<long long> code(ids.size());
    const long long Lp =
        ivc_check_compact(ids.data(), (long long)ids.size(), img, use.data(), T, S, S64, km.data(),
                          code.data());
    long long j = 0, k = 0;
    for (size_t p = 0; p < ids.size(); ++p) {
      bool keep = true;
      if (ids[p] == img) {
        keep = !use[k / S] || k % S < S64;
        ++k;
      }
      if (km[p] != (keep ? j : -1)) ++errors;
      if (keep) ++j;
    }
    if (Lp != j) ++errors;
  }
  errors += g_failures;
  printf("index self-test: %lld errors\n", errors);
  return errors == 0 ? 0 : 1;
}
#endif
