// Internal launch interface of the connector's kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ivc {

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { ACT_NONE = 0, ACT_GELU = 1 };

// ---- fused CLS drop + pixel_shuffle + LayerNorm ----------------------------
struct ShuffleArgs {
  int dtype;
  const void* X;
  int T, P, C, has_cls;
  int flash;  // 1: one workgroup per r=4 block, writes out4 (and out2 if non-null)
  int ln;     // 0: pure permutation (no normalisation)
  const float *g2, *b2;
  void* out2;
  const float *g4, *b4;
  void* out4;
  float eps;
  // statistics mode: (mean, rstd) of each LayerNorm row go to st2 / st4
  // ([rows][2] fp32) instead of the normalised rows (LayerNorm folded into
  // the products)
  float* st2 = nullptr;
  float* st4 = nullptr;
  int ps_v1 = 0;     // 1: pixel_shuffle v1, token grid transposed (token b*(P/r) + a)
  int twice_r2 = 0;  // 1: 64-path channel order of two successive r=2 shuffles
  // route-first: tile t writes only its chosen path's rows, at position rank[t]
  const uint8_t* use64 = nullptr;
  const int* rank = nullptr;
};
hipError_t launch_shuffle_ln(const ShuffleArgs& a, hipStream_t s);
// (mean, rstd) of every shuffled LayerNorm row from the per-token moments
// tokst [T, P*P] float2 (launch_token_stats or the first token pass), written
// to st2 / st4 as the statistics mode of launch_shuffle_ln writes them.
hipError_t launch_ln_stats(const float* tokst, int T, int P, int C, float eps, int ps_v1,
                           int flash, const uint8_t* use64, const int* rank, float* st2,
                           float* st4, hipStream_t s);
int shuffle_max_width(int dtype);

// ---- route-first products -----------------------------------------------------
// Optional device-side row count and output-row scatter of a GEMM: the grid
// is sized for the host M (an upper bound); the product covers
// min(M, *m_dev * m_mult) rows, and output row m is written to row
// c_map[m / c_rpg] * c_rpg + m % c_rpg.  With d_map (needs c_map; the
// 256 x 256 DMA product only) the row is written a second time, to row
// d_map[c_map[m / c_rpg] * d_stride + m % c_rpg] of d_out (same row stride
// as C), unless that entry is negative: a projector's rows placed straight
// into the compacted sequence.
struct RowMap {
  const int* m_dev = nullptr;
  int m_mult = 1;
  const int* c_map = nullptr;
  int c_rpg = 1;
  const int32_t* d_map = nullptr;
  int d_stride = 0;
  void* d_out = nullptr;
};

// A operand gathered straight from the ViT rows: logical row m is shuffled
// token m % S of tile list[m / S] (list null: tile m / S), and K block q
// (C wide) is cell q of the token's r x r grid block (pixel_shuffle order, or
// the two-r=2 order for r = 4), so no shuffled copy of the rows is written.
struct AGather {
  const int* list = nullptr;
  int rows = 0;  // has_cls + P*P
  int has_cls = 0, P = 0, r = 2, C = 0;
  int v1 = 0, twice = 0;
};

// ---- GEMM: C[M, N] = act(A[M, K] . W[N, K]^T + bias[N]) ---------------------
// A rows may be remapped: logical row m reads physical row
//   (m / a_rpg) * a_gstride + a_goff + m % a_rpg      (a_rpg > 0)
// which lets a GEMM read the ViT tensor with the CLS rows skipped.
struct GemmArgs {
  const void* A;
  long long lda;
  int a_rpg;
  long long a_gstride;
  int a_goff;
  const void* W;
  long long ldw;
  const float* bias;
  void* Cm;
  long long ldc;
  int M, N, K;
  int act;
  int a_dtype, w_dtype, c_dtype;
  // batched products (SIMT kernel): grid.z runs over `batch` independent
  // problems whose operands start b * (a_bs, w_bs, c_bs, bias_bs) elements in
  int batch;
  long long a_bs, w_bs, c_bs, bias_bs;
  // split-K (SIMT kernel): partial sums of the `ksplit` K ranges go to `part`
  // ([batch][ksplit][M][N] fp32) and a second kernel adds them in order
  int ksplit;
  float* part;
  RowMap rm;
  // LayerNorm folded into the product (DMA kernels): A is gathered by `ag`
  // from the raw rows, W holds gamma (.) W, and the epilogue computes
  //   rstd_m * acc - rstd_m * mean_m * ln_colsum[n] + bias[n]
  // with ln_rows[m] = (mean_m, rstd_m)
  int fold = 0;
  AGather ag;
  const float* ln_rows = nullptr;
  const float* ln_colsum = nullptr;
  // leftover tiles cut along K (DMA kernels): tail_grid = workgroups of a
  // whole round (a multiple of 8); tail_part / tail_cnt: scratch of
  // gemm_tail_bytes(tail_grid) bytes (partials, then counters), not shared
  // with a product running at the same time; tail_ticket: nonzero, < 2^56,
  // different from every earlier launch's.  tail_part null: one tile per
  // workgroup throughout.
  float* tail_part = nullptr;
  unsigned long long* tail_cnt = nullptr;
  unsigned long long tail_ticket = 0;
  int tail_grid = 0;
};

// K pieces for each of r leftover tiles (those past the last whole round of
// G tiles) of a product with KT K steps: the fewest rounds of pieces times
// the piece length, at most 4 pieces of at least 32 K steps each (a shorter
// piece does not earn back its pipeline fill and its partial tile's store
// and load: measured slower at 16-21 steps), at most two rounds of pieces
// (r * s <= 2 G), and only for a gain of 5% or more.
__host__ __device__ inline int gemm_tail_split(int r, int G, int KT) {
  float best = 1.0f;
  int bs = 1;
  for (int s = 2; s <= 4; ++s) {
    if (KT < 32 * s || r * s > 2 * G) break;
    const float cost = (float)((r * s + G - 1) / G) / (float)s;
    if (cost < best * 0.95f) {
      best = cost;
      bs = s;
    }
  }
  return bs;
}
// Scratch of the leftover-tile pieces: 2 G partial tiles of 256 x 256 fp32,
// then G counters.
inline size_t gemm_tail_bytes(int G) {
  return (size_t)2 * G * 256 * 256 * 4 + (size_t)G * 8;
}
// bf16 A and W, fp32 accumulation on MFMA, bf16 out.  Needs K % 64 == 0.
hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t s);
bool gemm_mfma_supported(const GemmArgs& g);
// Same product with 256 x 256 tiles fed by LDS DMA (large products).
hipError_t launch_gemm_dma(const GemmArgs& g, hipStream_t s);
bool gemm_dma_supported(const GemmArgs& g);
// Any element types, fp32 FMA.  Used for fp32 workloads and fp32-activation
// router products.
hipError_t launch_gemm_simt(const GemmArgs& g, hipStream_t s);
// fp32 A, bf16 W on MFMA (A split into bf16 high + low parts), fp32 C; with
// out_split = 1 the result times `scale` goes out as bf16 high (Cm) and low (C2)
// parts instead.  Batched via batch / a_bs / w_bs / c_bs / bias_bs.  K % 32 == 0.
bool gemm_f32a_supported(const GemmArgs& g);
hipError_t launch_gemm_f32a(const GemmArgs& g, int out_split, void* C2, float scale,
                            hipStream_t s);
// LayerNorm fold of a Linear that follows LayerNorm(gamma, beta):
//   Wg[n][k] = bf16(gamma[k] * W[n][k]),  colsum[n] = sum_k Wg[n][k],
//   bfold[n] = b[n] + sum_k beta[k] * W[n][k]        (W, Wg bf16 [N, K])
hipError_t launch_ln_fold_weights(const void* W, int N, int K, const float* gamma,
                                  const float* beta, const float* b, void* Wg, float* colsum,
                                  float* bfold, hipStream_t s);
// dst[c][r] = src[r][c], [R, Cc] bf16; row strides lds (src) and ldd (dst)
hipError_t launch_transpose_bf16(const void* src, long long lds, void* dst, long long ldd, int R,
                                 int Cc, hipStream_t s);
// split-K factor and workspace the SIMT kernel wants for a product
int simt_ksplit(int M, int N, int K, int batch);
size_t simt_part_elems(int M, int N, int batch, int ksplit);
int simt_tiles(int M, int N);

// ---- CrossAttentionPooling ---------------------------------------------------
struct PoolAttnArgs {
  int dtype;           // element type of KV
  const void* KV;      // [T*N, kv_ld] with K_l at column kcol, V_l at vcol
  long long kv_ld;
  int kcol, vcol;
  const float* Q;      // [T, C] projected queries of this layer
  const int* valid;    // [T] or null
  int* status;         // device status word or null
  int T, N, C, H;
  int splits;          // token splits per tile
  float* part;         // [T, splits, H, 2 + d]: running max, sum, weighted V
  float* O;            // [T, C] attention output (before out-projection)
};
hipError_t launch_pool_attn(const PoolAttnArgs& a, hipStream_t s);
bool pool_attn_supported(int C, int H);

// ---- Gating helpers ----------------------------------------------------------
// x[t] += LayerNorm(y[t]) * gamma + beta   (rows of width h, fp32)
hipError_t launch_residual_ln(float* x, const float* y, const float* gamma, const float* beta,
                              int T, int h, float eps, hipStream_t s);
// the same for the last block, then z = Wc x + bc and gate = softmax(z) for 2
// classes on the updated rows (one launch; Wc element type dtype)
hipError_t launch_residual_ln_head(int dtype, float* x, const float* y, const float* gamma,
                                   const float* beta, int T, int h, float eps, const void* Wc,
                                   const float* bc, float* gate, hipStream_t s);
// broadcast a [C] vector (element type dtype) into fp32 rows [T, C]
hipError_t launch_broadcast_rows(int dtype, const void* v, float* out, int T, int C,
                                 hipStream_t s);

// ---- quantile + decision -----------------------------------------------------
// rank != nullptr: also the per-path tile lists of the decision, as
// launch_route_lists writes them (one launch less in forward)
hipError_t launch_quantile_decide(const float* gate, int T, double q, double abs_thr,
                                  double* thr, uint8_t* use64, hipStream_t s,
                                  int* rank = nullptr, int* list256 = nullptr,
                                  int* list64 = nullptr, int* counts = nullptr);

// ---- compaction ----------------------------------------------------------------
struct CompactArgs {
  int dtype;
  const int32_t* ids;
  const void* embeds;
  long long L;
  int img_id;
  const uint8_t* use64;
  const void* out256;
  const void* out64;
  int T, S, S64, D;
  int32_t* out_ids;
  int32_t* out_pos;
  int32_t* keep_map;
  void* out_embeds;
  long long* out_len;
  int32_t* status;
  // workspace
  int32_t* blk_cnt;        // [nblk]
  int32_t* blk_off;        // [nblk + 1]
  int32_t* routed_before;  // [T + 1]
  long long* src;          // [L] source row code per output row
  // optional: the compacted row of every image slot k = tile * S + loc, or
  // -1 (a deleted slot, or no valid compaction), written by the index half
  int32_t* slot_dst = nullptr;  // [T * S]
};
long long compact_blocks(long long L);

// Batched form: B sequences packed back to back (sequence b = positions
// cu[b] .. cu[b+1]-1, tiles tile_off[b] .. tile_off[b+1]-1), each compacted
// on its own, outputs packed at out_cu[b].
struct CompactBatchArgs {
  CompactArgs base;          // out_len unused; status, sequence and embedding pointers as above
  const int32_t* cu;         // [B + 1]
  const int32_t* tile_off;   // [B + 1]
  int B;
  int32_t* out_cu;           // [B + 1]
  // workspace
  int32_t* seq_img;          // [B + 1] IMG_CONTEXT count before each sequence start
  int32_t* seq_ok;           // [B] 1: the sequence's slot count matches its tiles
  long long* total;          // [1] packed length (copy bound)
  int32_t* layout_ok;        // [1]
};
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
// its two halves: the index work (reads ids and use64) and the row copy
// (reads the index half's sources and out_len, and out256 / out64)
hipError_t launch_compact_index(const CompactArgs& a, hipStream_t s);
hipError_t launch_compact_copy(const CompactArgs& a, hipStream_t s);
// the rows of some sources only (kinds: bit 0 text embeddings, bit 1 rows of
// out256, bit 2 rows of out64), one wave per output row
hipError_t launch_compact_copy_kinds(const CompactArgs& a, int kinds, hipStream_t s);
// the text embedding rows only, one wave per 64 output rows (a few percent of
// a compacted sequence's rows are text)
hipError_t launch_compact_copy_text(const CompactArgs& a, hipStream_t s);
hipError_t launch_compact_batch(const CompactBatchArgs& a, hipStream_t s);

// Per-path tile lists of a routing decision: rank[t] = index of t among the
// tiles of its path, list256 / list64 = tile ids in order, counts = {n256, n64}.
hipError_t launch_route_lists(const uint8_t* use64, int T, int* rank, int* list256, int* list64,
                              int* counts, hipStream_t s);

hipError_t launch_tile_offsets(const int32_t* tiles, int B, int32_t* offsets, int32_t* status,
                               hipStream_t s);

// ---- folded pooling -------------------------------------------------------------
struct FoldedArgs {
  int dtype;
  const void* X;      // ViT rows [T, rows, C]
  int rows, has_cls;
  const int* valid;
  int* status;
  int T, N, C, H;
  const void* qt_hi;  // [T, 16, C] bf16: folded queries (log2(e)/sqrt(d) applied), high part
  const void* qt_lo;  // low part
  int qt_shared;      // 1: qt_hi / qt_lo are one [16, C] block shared by every tile
  int G, Q, segmax;   // from folded_geometry
  float* part;        // [G * segmax, 16 * (2 + C)]
  float* xbar;        // [T, H, C] softmax-weighted token means; nullptr: no merge launch
  float* tokst;       // optional [T, N] float2: each token's LayerNorm moments (mean, M2);
                      // needs valid == nullptr
  int reverse;        // 1: each workgroup walks its chunk range from the end (alternating
                      // directions between layers reuses what the memory-side cache kept)
};
// Work split of the token pass: G workgroups of Q consecutive 16-token chunks
// each (chunk index = tile * ceil(N/16) + chunk); a workgroup leaves at most
// segmax partials.  ncu = compute units of the device.
void folded_geometry(int T, int N, int C, int ncu, int* G, int* Q, int* segmax);
bool pool_folded_supported(int dtype, int C, int H);
// Each token's LayerNorm moments over its C channels, tokst[t * N + n] =
// (mean, sum of squared deviations); bf16, C a multiple of 8 up to 4096, N a
// multiple of 16.  pool_order (C of 512 or 1024 only): the same arithmetic
// as the first token pass of the folded pooling, bit for bit (Flash
// connectors, whose forward takes the moments from that pass); otherwise
// two passes per token over its row.
bool token_stats_supported(int dtype, int C, int N);
hipError_t launch_token_stats(const void* X, int T, int rows, int has_cls, int N, int C,
                              float* tokst, hipStream_t s, bool pool_order);
hipError_t launch_pool_folded(const FoldedArgs& a, hipStream_t s);
// qt[t, h, :] = scale * sum_i Q[t, h*d + i] * Wk[h*d + i, :] as bf16 high + low parts
hipError_t launch_fold_query(int dtype, const float* Q, const void* Wk, void* qt_hi, void* qt_lo,
                             int T, int C, int H, float scale, hipStream_t s);
// C = act(x_out W^T + bias) with x_out = x_in + LN(y) * gamma + beta written
// too (a Gating block's first Linear with the previous block's residual
// LayerNorm in its prologue); fp32 rows of K (a multiple of 256, <= 1024),
// bf16 W [N, K]; x_in and x_out distinct.
// The pooling's last output projection (optional: o == nullptr skips it and
// xb[0] holds the pooled rows; else it writes them there) and the whole
// Gating network in one launch.  Every product is an f32a tile and h == he.
// Each phase writes buffers of its own: xb[1..3] (block inputs), y1[b],
// y2[b] ([T, h] fp32 each).  sync: gating_fused_sync_words(T) device words
// of workspace; tag: nonzero, below 2^48, different for every launch.
// Optionally (vf_part set, o set) a leading phase makes o itself: the
// pooling's last value fold from the token pass's partials, as
// launch_fold_value_merged computes it (vf_* are that launcher's arguments,
// with C = h).
struct GatingFusedArgs {
  const float* vf_part = nullptr;
  const int* vf_valid = nullptr;
  int vf_N = 0, vf_Q = 0, vf_segmax = 0, vf_H = 0;
  const uint16_t* vf_wv = nullptr;  // bf16
  long long vf_ldw = 0;
  const float* vf_bv = nullptr;
  const float* o = nullptr;
  const uint16_t* wo = nullptr;  // bf16
  long long ldwo = 0;
  const float* bo = nullptr;
  float* xb[4] = {};
  float* y1[4] = {};
  float* y2[4] = {};
  const uint16_t* w1[4] = {};  // bf16
  const uint16_t* w2[4] = {};
  long long ldw1 = 0, ldw2 = 0;
  const float* b1[4] = {};
  const float* b2[4] = {};
  const float* lw[4] = {};
  const float* lb[4] = {};
  const uint16_t* wc = nullptr;  // bf16 [2, h]
  const float* bc = nullptr;
  float* gate = nullptr;
  int T = 0, h = 0, he = 0;
  float eps = 0.f;
  unsigned long long* sync = nullptr;
  unsigned long long tag = 0;
  int* status = nullptr;
  int first[12] = {};  // set by the launcher
  int nph = 0;
};
bool gating_fused_supported(int T, int h, int he);
size_t gating_fused_sync_words(int T);
hipError_t launch_gating_fused(GatingFusedArgs a, hipStream_t s);

bool f32a_ln_rows_supported(int K);
// (W rows at stride ldw)
hipError_t launch_f32a_ln_rows(const float* x_in, const float* y, const float* gamma,
                               const float* beta, float eps, float* x_out, const void* W,
                               long long ldw, const float* bias, float* Cm, int M, int N, int K,
                               int act, hipStream_t s);
// qp = Wq q + bq, then q~_h = scale * Wk_h^T qp_h for every head, in one launch
// (the same values as a query projection followed by the key fold).  q: rows
// of stride ldq (0: one row shared by every tile).
bool fold_query_fused_supported(int C, int H);
// Wq_lo: if set, Wq and Wq_lo are the bf16 high and low parts of fp32 weights.
// (Wq, Wq_lo rows at stride ldwq, WkT rows at stride ldk)
hipError_t launch_fold_query_fused(const float* q, long long ldq, const void* Wq, long long ldwq,
                                   const float* bq, const void* WkT, long long ldk, void* qt_hi,
                                   void* qt_lo, int T, int C, int H, float scale, hipStream_t s,
                                   const void* Wq_lo = nullptr);
// hi = bf16(x), lo = bf16(x - hi) for a dense [rows, cols] fp32 matrix; hi and
// lo with row stride ld
hipError_t launch_split_bf16(const float* x, void* hi, void* lo, long long rows, int cols,
                             long long ld, hipStream_t s);
// qt_hi / qt_lo [T, 16, C]: heads H .. 15 set to zero
hipError_t launch_zero_heads(void* qt_hi, void* qt_lo, int T, int H, int C, hipStream_t s);
// The value fold reading the token pass's partials directly (no merge launch):
// o[t, h*d + i] = bv[h*d + i] + sum_c Wv[h*d + i, c] * xbar[t, h, c], bf16 Wv.
// Usable when a tile's chunks meet at most 4 workgroups (max_parts <= 4).
int fold_value_merged_max_parts(int T, int N, int Q);
// (Wv rows at stride ldw)
hipError_t launch_fold_value_merged(const float* part, const int* valid, int N, int Q, int segmax,
                                    const void* Wv, long long ldw, const float* bv, float* o, int T,
                                    int C, int H, hipStream_t s);
// o[t, h*d + i] = bv[h*d+i] + sum_c Wv[h*d + i, c] * xbar[t, h, c]
hipError_t launch_fold_value(int dtype, const float* xbar, const void* Wv, const float* bv,
                             float* o, int T, int C, int H, hipStream_t s);
// One layer's value fold (launch_fold_value_merged's arguments) and the next
// layer's fused query fold reading its output o (launch_fold_query_fused's,
// with q = o, ldq = C) in one launch: the query-fold workgroups of a 16-tile
// row block start once that block's value-fold workgroups have counted
// themselves in sync (fold_value_query_sync_words(T) device words of
// workspace; tag: nonzero, below 2^48, different for every launch).  Same
// values as the two launches.
struct FoldVQArgs {
  const float* part = nullptr;
  const int* valid = nullptr;
  int N = 0, Q = 0, segmax = 0;
  const uint16_t* Wv = nullptr;  // bf16
  long long ldwv = 0;
  const float* bv = nullptr;
  float* o = nullptr;
  const uint16_t* Wq = nullptr;  // bf16 high part (and Wq_lo the low part) of fp32 weights
  const uint16_t* Wq_lo = nullptr;
  long long ldwq = 0;
  const float* bq = nullptr;
  const uint16_t* WkT = nullptr;
  long long ldk = 0;
  uint16_t* qt_hi = nullptr;
  uint16_t* qt_lo = nullptr;
  float scale = 0.f;
  int T = 0, C = 0, H = 0;
  unsigned long long* sync = nullptr;
  unsigned long long tag = 0;
  int* status = nullptr;
};
bool fold_value_query_supported(int T, int N, int Q, int C, int H);
size_t fold_value_query_sync_words(int T);
hipError_t launch_fold_value_query(const FoldVQArgs& a, hipStream_t s);

// ---- per-kernel timing (ivc_profile_*) -----------------------------------------
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

}  // namespace ivc
