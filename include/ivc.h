/*
 * ivc.h - C ABI of the InternVL visual-token compression connector for
 * AMD Instinct MI355X (gfx950).
 *
 * The connector turns each 448x448 image tile's ViT output into the visual
 * tokens an LLM consumes, and (Flash models) decides per tile whether 256 or
 * 64 tokens go into the prompt:
 *
 *   ViT rows [T, has_cls + P*P, C]
 *     -> drop CLS, P x P grid                              (ivc_connector_run)
 *     -> pixel_shuffle v2, r = 2: [T, (P/2)^2, 4C]  -> mlp1 -> out256 [T, (P/2)^2, D]
 *     -> pixel_shuffle v2, r = 4: [T, (P/4)^2, 16C] -> mlp2 -> out64  [T, (P/4)^2, D]
 *     -> CrossAttentionPooling -> Gating -> quantile + threshold   (ivc_connector_route)
 *     -> delete routed tiles' surplus IMG_CONTEXT slots      (ivc_connector_compact)
 *
 * Pages describing the method (cited by title and section):
 *   [14B]      "InternVL3-14B-Instruct: pixel shuffle and MLP connector,
 *               line by line" (zwxr.cn/news/271642)
 *   [4B-Flash] "InternVL3_5-4B-Flash Gating and CrossAttentionPooling
 *               explained" (mrgr.cn/news/14598)
 *   [2B-Flash] "InternVL3_5-2B-Flash dual-path visual-token compression
 *               pipeline" (kwkr.cn/news/620108)
 *
 * Conventions for every entry point:
 *   - Pointers named vit, out*, gate, use64, ids, embeds, keep_map, ws, ...
 *     are DEVICE pointers (hipMalloc'd or torch CUDA tensors).  Only the
 *     config and weight-table structs are read on the host.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Calls enqueue work on it and return without synchronising.  run, route
 *     and compact never allocate memory.
 *   - Element type: ivc_config.dtype (IVC_F32 = float, IVC_BF16 = bfloat16
 *     stored as uint16).  ViT input, weights, out256/out64 and embeddings all
 *     use it; gate probabilities and pooled vectors are float32.
 *   - Row-major layouts; weights in torch nn.Linear layout [out, in].
 *   - Device pointers must be 16-byte aligned, and every row width in bytes
 *     (C, D, ... times the element size) a multiple of 16
 *     (IVC_ERR_MISALIGNED otherwise).
 *   - Errors found on the host return a non-OK status and enqueue nothing.
 *     Data-dependent errors found on the device are written to a caller's
 *     int32 device status word (0 = fine); outputs are then undefined.
 *     Launch failures return IVC_ERR_HIP.  ivc_last_error() gives the
 *     detail of the calling thread's last failure.  Nothing throws.
 *   - Calls that overlap on one stream are ordered; calls on different
 *     streams must use different workspaces.
 */
#ifndef IVC_H
#define IVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IVC_OK = 0,
  IVC_ERR_INVALID_ARG = 1,  /* null pointer, bad size or inconsistent config   */
  IVC_ERR_UNSUPPORTED = 2,  /* shape outside what the kernels implement       */
  IVC_ERR_MISALIGNED = 3,   /* device pointer or row not 16-byte aligned      */
  IVC_ERR_WORKSPACE = 4,    /* ws_bytes smaller than ivc_connector_workspace_bytes */
  IVC_ERR_OOM = 5,          /* create could not allocate its weight copies    */
  IVC_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed     */
} ivc_status;

typedef enum { IVC_F32 = 0, IVC_BF16 = 1 } ivc_dtype;

/* How CrossAttentionPooling is evaluated (both give the same mathematics):
 * IVC_POOL_KV projects every token to K and V for all layers with one MFMA
 * GEMM, then runs single-query attention over K and V.  IVC_POOL_FOLDED
 * folds the key projection into the query (q~_h = Wk_h^T Q_h) and the value
 * projection after the weighted sum (o_h = Wv_h (sum_n p_n x_n) + bv_h), so
 * the tile's tokens are read once per layer and no K/V tensor exists. */
typedef enum { IVC_POOL_KV = 0, IVC_POOL_FOLDED = 1 } ivc_pool_mode;

/* Channel order of the 64-token path's 16C rows.  [2B-Flash] describes the
 * scale 0.25 shuffle as equivalent to two 0.5 shuffles; both orders gather
 * the same 4 x 4 cells into a token.  DIRECT is pixel_shuffle with r = 4:
 * cell (M, K) of the block goes to channel block 4*M + K.  TWICE_R2 applies
 * the r = 2 shuffle to the 16 x 16 grid of 4C tokens: cell
 * (2*m2 + m, 2*k2 + k) goes to channel block 4*(2*m2 + k2) + (2*m + k). */
typedef enum { IVC_SHUFFLE64_DIRECT = 0, IVC_SHUFFLE64_TWICE_R2 = 1 } ivc_shuffle64_order;

/* Device status codes written by run/route/compact/ivc_tile_offsets. */
#define IVC_DEV_OK 0
#define IVC_DEV_ERR_IMG_COUNT 1    /* IMG_CONTEXT slots != T * (P/2)^2          */
#define IVC_DEV_ERR_VALID_TOKENS 2 /* a valid_tokens[t] outside [1, P*P]        */
#define IVC_DEV_ERR_TILE_COUNT 4   /* a tiles_per_image[i] < 0, or sum > INT32_MAX */
#define IVC_DEV_ERR_SEQ_LAYOUT 8   /* batch: cu_seqlens / tile_offsets not an ordered partition */
#define IVC_DEV_ERR_ROUTER_SYNC 16 /* route: a phase of the one-launch Gating waited past
                                      its bound (a few seconds); gates undefined   */

#define IVC_MAX_POOL_LAYERS 8
#define IVC_GATE_BLOCKS 4

typedef struct ivc_config {
  int32_t dtype;          /* ivc_dtype                                              */
  int32_t vit_width;      /* C: ViT hidden width (1024 InternViT-300M, 3200 InternViT-6B) */
  int32_t grid;           /* P: tile grid side, P*P tokens per tile (32 for 448/14)  */
  int32_t has_cls;        /* 1: each tile has 1 + P*P rows and row 0 (CLS) is dropped */
  int32_t llm_width;      /* D: output width of mlp1 and mlp2                        */
  int32_t mlp1_hidden;    /* width after mlp1's first Linear (= D on the pages)      */
  int32_t flash;          /* 1: also build the 64-token path and the router          */
  int32_t mlp2_hidden;    /* mlp2's two hidden widths (4096 on the pages)            */
  int32_t pool_layers;    /* cross-attention layers (4)                              */
  int32_t pool_heads;     /* heads per layer; head width C / pool_heads              */
  int32_t gate_hidden;    /* gating width; must equal C (the pooled vector's width)  */
  int32_t gate_expansion; /* inner width of a gating block = gate_hidden * this      */
  int32_t pool_mode;      /* ivc_pool_mode                                          */
  int32_t ps_version;     /* pixel_shuffle version: 2 (or 0) = v2; 1 = v1, whose
                             token grid is transposed ([14B] v1/v2 section)     */
  int32_t shuffle64_order;/* ivc_shuffle64_order: channel order of the 64-token path */
  int32_t ln_fold;        /* 1: fold the projectors' LayerNorm into their first
                             Linear (bf16 only; see ivc_connector_create)       */
  double rel_quantile;    /* relative threshold, a quantile level (0.1)             */
  double abs_threshold;   /* absolute threshold on gate[:, 0] (0.5)                 */
  float ln_eps;           /* LayerNorm epsilon (1e-5, torch's default)              */
} ivc_config;

/* Device pointers to the parameters, element type ivc_config.dtype, torch
 * layouts.  create() copies them; the caller may free its copies after
 * create() returns.  mlp2_*, pool_* and gate_* are read only when flash = 1. */
typedef struct ivc_weights {
  /* mlp1: LayerNorm(4C) -> Linear(4C, H1) -> GELU -> Linear(H1, D) */
  const void *mlp1_ln_w, *mlp1_ln_b;       /* [4C]                     */
  const void *mlp1_w1, *mlp1_b1;           /* [H1, 4C], [H1]           */
  const void *mlp1_w2, *mlp1_b2;           /* [D, H1], [D]             */
  /* mlp2: LayerNorm(16C) -> Linear(16C, H2) -> GELU -> Linear(H2, H2) -> GELU -> Linear(H2, D) */
  const void *mlp2_ln_w, *mlp2_ln_b;       /* [16C]                    */
  const void *mlp2_w1, *mlp2_b1;           /* [H2, 16C], [H2]          */
  const void *mlp2_w2, *mlp2_b2;           /* [H2, H2], [H2]           */
  const void *mlp2_w3, *mlp2_b3;           /* [D, H2], [D]             */
  /* CrossAttentionPooling: learnable query, per layer q/k/v/out projections */
  const void *pool_query;                  /* [C]                      */
  const void *pool_wq[IVC_MAX_POOL_LAYERS], *pool_bq[IVC_MAX_POOL_LAYERS]; /* [C, C], [C] */
  const void *pool_wk[IVC_MAX_POOL_LAYERS], *pool_bk[IVC_MAX_POOL_LAYERS];
  const void *pool_wv[IVC_MAX_POOL_LAYERS], *pool_bv[IVC_MAX_POOL_LAYERS];
  const void *pool_wo[IVC_MAX_POOL_LAYERS], *pool_bo[IVC_MAX_POOL_LAYERS];
  /* Gating: 4 blocks x (Linear(h, h*e) -> GELU -> Linear(h*e, h) -> LayerNorm(h)), residual */
  const void *gate_w1[IVC_GATE_BLOCKS], *gate_b1[IVC_GATE_BLOCKS]; /* [h*e, h], [h*e] */
  const void *gate_w2[IVC_GATE_BLOCKS], *gate_b2[IVC_GATE_BLOCKS]; /* [h, h*e], [h]   */
  const void *gate_ln_w[IVC_GATE_BLOCKS], *gate_ln_b[IVC_GATE_BLOCKS]; /* [h]        */
  const void *gate_cls_w, *gate_cls_b;     /* [2, h], [2]              */
} ivc_weights;

typedef struct ivc_connector ivc_connector;

/* LayerNorm fold (ln_fold = 1): mlp1 and mlp2 each start LayerNorm -> Linear,
 * and LN(x) W^T + b = rstd (x . (gamma o W)^T) - rstd mean colsum(gamma o W)
 * + (b + W beta).  create() stores gamma o W (rounded to bf16), its column
 * sums and the folded bias; run and run_routed then write only each row's
 * (mean, rstd) and the first product reads the raw ViT rows in pixel-shuffle
 * order, so the normalised rows are never written.  Same results up to
 * rounding (the bf16 rounding moves from the normalised rows to gamma o W).
 * Needs bf16, C % 64 == 0 and the hidden widths % 8 == 0 (IVC_ERR_UNSUPPORTED
 * otherwise); a call may then pass at most 2 GiB of ViT rows
 * (T * (has_cls + P*P) * C * 2 bytes; IVC_ERR_UNSUPPORTED beyond). */

/* Build a connector: validates the config, copies the weights into
 * library-owned device memory (biases and LayerNorm parameters widened to
 * float32; the K/V projections of all pooling layers packed into one
 * [2 * layers * C, C] matrix), synchronises `stream`, and returns the handle
 * in *out.  A bf16 flash connector also owns two more streams (default
 * priority) and three events: run and run_routed fork the mlp1 chain onto the
 * first after the loader and join it back into the caller's stream, so the
 * two projector chains share the chip; forward_compact runs the compaction's
 * index work on the second beside them.  The handle's weights are immutable
 * afterwards; calls may use several streams, but one handle must not be used
 * by two host threads at once (the fork/join events are shared).  Errors:
 * IVC_ERR_INVALID_ARG, IVC_ERR_UNSUPPORTED, IVC_ERR_MISALIGNED, IVC_ERR_OOM,
 * IVC_ERR_HIP. */
ivc_status ivc_connector_create(const ivc_config* cfg, const ivc_weights* w, void* stream,
                                ivc_connector** out);

/* Release the handle's device memory, stream and events (synchronises the
 * device first). NULL is a no-op. */
void ivc_connector_destroy(ivc_connector* h);

/* Bytes of device workspace that run, route and compact need for up to
 * max_tiles tiles and (compact) sequences of up to max_seq_len tokens.  One
 * workspace of this size serves all three calls in sequence on one stream. */
size_t ivc_connector_workspace_bytes(const ivc_connector* h, int32_t max_tiles,
                                     int64_t max_seq_len);

/* extract_feature ([14B] extract_feature walkthrough) and, with flash = 1,
 * both branches of extract_feature_flash ([2B-Flash] dual pipeline, step 2):
 *   vit    [T, has_cls + P*P, C]  ViT output, tile-major
 *   out256 [T, (P/2)^2, D]        mlp1(LN(pixel_shuffle(grid, 2)))
 *   out64  [T, (P/4)^2, D]        mlp2(LN(pixel_shuffle(grid, 4))); required iff flash
 * pixel_shuffle v2: out[a*(P/r)+b, (r*m+k)*C + c] = grid[r*a+m][r*b+k][c]
 * ([14B] pixel_shuffle section).  T = 0 enqueues nothing. */
ivc_status ivc_connector_run(ivc_connector* h, const void* vit, int32_t T, void* out256,
                             void* out64, void* ws, size_t ws_bytes, void* stream);

/* Route-first form of ivc_connector_run (flash = 1): with the decision use64
 * [T] (device, from ivc_connector_route) already known, computes out256 only
 * for tiles with use64[t] = 0 and out64 only for tiles with use64[t] = 1;
 * rows of the other path are left untouched.  ivc_connector_compact reads
 * exactly those rows, so the compacted sequence is the same as after
 * ivc_connector_run, for about half of the projector work.  The pages
 * compute both paths for every tile because the quantile needs the whole
 * batch ([4B-Flash] section 5); deciding first removes that need.  The
 * kernels size their grids for all T tiles and read the per-path tile counts
 * from the device, so the call does not synchronise.  Same workspace as run. */
ivc_status ivc_connector_run_routed(ivc_connector* h, const void* vit, int32_t T,
                                    const uint8_t* use64, void* out256, void* out64, void* ws,
                                    size_t ws_bytes, void* stream);

/* Visual Resolution Router ([4B-Flash] sections 2-4; [2B-Flash] routing
 * decision).  Requires flash = 1.
 *   vit          [T, has_cls + P*P, C] as for run
 *   valid_tokens [T] int32 real tokens per tile, in [1, P*P]; the rest of the
 *                tile is padding at its end and is never read.  NULL = all.
 *   gate         [T, 2] float32 softmax probabilities (out)
 *   threshold    [1] float64: quantile of gate[:, 0] at rel_quantile, linear
 *                interpolation between order statistics (out)
 *   use64        [T] uint8: 1 iff gate[t,0] > threshold and gate[t,0] >= abs_threshold (out)
 *   pooled       [T, C] float32 pooled vectors (out), or NULL
 *   dev_status   int32 device word; IVC_DEV_ERR_VALID_TOKENS is OR-ed in for
 *                an out-of-range valid_tokens entry (that tile then uses the
 *                clamped count).  NULL = no report.
 * The quantile spans all T tiles of the call.  T = 0 enqueues nothing. */
ivc_status ivc_connector_route(ivc_connector* h, const void* vit, const int32_t* valid_tokens,
                               int32_t T, float* gate, double* threshold, uint8_t* use64,
                               float* pooled, int32_t* dev_status, void* ws, size_t ws_bytes,
                               void* stream);

/* ivc_connector_route followed by ivc_connector_run_routed in one call
 * ([4B-Flash] sections 2-5; [2B-Flash] dual pipeline), with the same outputs
 * (bit for bit) and one workspace of ivc_connector_workspace_bytes.  Requires
 * flash = 1; out256 and out64 are both required.  With ln_fold, folded
 * pooling and no valid_tokens, the first pooling pass also takes the
 * LayerNorm statistics the projectors need (the same arithmetic as run's own
 * statistics pass, which is then skipped), and the decision kernel also
 * writes the per-path tile lists, so the call reads the ViT tensor one time
 * less than route + run_routed. */
ivc_status ivc_connector_forward(ivc_connector* h, const void* vit, const int32_t* valid_tokens,
                                 int32_t T, float* gate, double* threshold, uint8_t* use64,
                                 float* pooled, int32_t* dev_status, void* out256, void* out64,
                                 void* ws, size_t ws_bytes, void* stream);

/* compress_visual_tokens_in_sentence plus the IMG_CONTEXT embedding
 * injection ([4B-Flash] section 4; [2B-Flash] routing decision; [14B] token
 * injection).  The k-th IMG_CONTEXT token of `ids` is slot k % S of tile
 * k / S, S = (P/2)^2.  Text tokens keep their embedding row; a slot of a
 * tile with use64 = 0 takes out256[tile][slot]; a tile with use64 = 1 keeps
 * only its first (P/4)^2 slots, filled from out64[tile][slot], and its other
 * slots are deleted.
 *   ids [L] int32, embeds [L, D]; IMG_CONTEXT rows of embeds are never read
 *   use64 [T] uint8; out256 [T, S, D]; out64 [T, (P/4)^2, D] (may be NULL if
 *   no use64 entry is set and flash = 0)
 *   out_ids [L], out_pos [L]: compacted ids and positions 0..L'-1, -1 past L'
 *   keep_map [L]: new index of each input position, or -1 if deleted
 *   out_embeds [L, D]: rows 0..L'-1 written, the rest untouched
 *   out_len [1] int64: L' (device)
 *   dev_status: IVC_DEV_ERR_IMG_COUNT when the IMG_CONTEXT count != T * S
 *   (required, not NULL).  L = 0 writes out_len = 0. */
ivc_status ivc_connector_compact(ivc_connector* h, const int32_t* ids, const void* embeds,
                                 int64_t L, int32_t img_context_id, const uint8_t* use64,
                                 const void* out256, const void* out64, int32_t T,
                                 int32_t* out_ids, int32_t* out_pos, int32_t* keep_map,
                                 void* out_embeds, int64_t* out_len, int32_t* dev_status,
                                 void* ws, size_t ws_bytes, void* stream);

/* ivc_connector_forward followed by ivc_connector_compact of its use64,
 * out256 and out64 ([4B-Flash] sections 2-5; [2B-Flash] dual pipeline and
 * routing decision; [14B] token injection), with the same outputs bit for
 * bit.  The compaction's index work (ids, positions, keep map, L', and the
 * compacted row of every image slot) needs only the decision, so it runs
 * beside the projector products, with the copy of the text embedding rows,
 * on a stream of the connector's own that `stream` then waits for (no host
 * synchronisation).  Each projector's last product writes its rows into
 * out_embeds as well as into out256 / out64 when it runs on the 256 x 256
 * kernel (bf16, enough rows to fill the chip); rows it cannot place are
 * copied once the products are done.  Arguments as in those two calls, one
 * dev_status for both; one workspace of
 * ivc_connector_forward_compact_workspace_bytes(h, max_tiles, max_seq_len)
 * bytes holds the forward's and the compaction's scratch side by side
 * (IVC_ERR_WORKSPACE if smaller; the compaction's arguments are checked
 * before anything is enqueued).  Requires flash = 1. */
size_t ivc_connector_forward_compact_workspace_bytes(const ivc_connector* h, int32_t max_tiles,
                                                     int64_t max_seq_len);
ivc_status ivc_connector_forward_compact(ivc_connector* h, const void* vit,
                                         const int32_t* valid_tokens, int32_t T, float* gate,
                                         double* threshold, uint8_t* use64, float* pooled,
                                         int32_t* dev_status, void* out256, void* out64,
                                         const int32_t* ids, const void* embeds, int64_t L,
                                         int32_t img_context_id, int32_t* out_ids,
                                         int32_t* out_pos, int32_t* keep_map, void* out_embeds,
                                         int64_t* out_len, void* ws, size_t ws_bytes,
                                         void* stream);

/* For callers that cannot allocate device memory and cannot supply a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): ivc_connector_compact with the same arguments,
 * outputs and device status, minus ws / ws_bytes.  Its scratch (per-block
 * IMG_CONTEXT counts and offsets, routed tiles before each tile, a source
 * code per output row) lives in a fixed device array of this library,
 * IVC_COMPACT_NOALLOC_SCRATCH_BYTES per device, held until the process
 * ends; its device address is taken when a connector is created on the
 * device.  It allocates nothing.  Limits: L <= IVC_COMPACT_NOALLOC_MAX_LEN
 * and T <= IVC_COMPACT_NOALLOC_MAX_TILES (IVC_ERR_UNSUPPORTED beyond, nothing
 * enqueued); IVC_ERR_HIP if the array's address could not be taken.  Every
 * call on one device shares that device's array: calls that overlap on one
 * device (different streams, or different host threads) race and must not be
 * issued; calls ordered on one stream are fine (each call writes all the
 * scratch it reads before reading it). */
#define IVC_COMPACT_NOALLOC_MAX_LEN 262144
#define IVC_COMPACT_NOALLOC_MAX_TILES 4096
#define IVC_COMPACT_NOALLOC_SCRATCH_BYTES 2116096 /* the workspace of those maxima */
ivc_status ivc_connector_compact_noalloc(ivc_connector* h, const int32_t* ids, const void* embeds,
                                         int64_t L, int32_t img_context_id, const uint8_t* use64,
                                         const void* out256, const void* out64, int32_t T,
                                         int32_t* out_ids, int32_t* out_pos, int32_t* keep_map,
                                         void* out_embeds, int64_t* out_len, int32_t* dev_status,
                                         void* stream);

/* Variable-length batch form of ivc_connector_compact: B prompts packed
 * back to back, as varlen attention takes them.  Sequence b is positions
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 of ids/embeds, and its images own
 * tiles tile_offsets[b] .. tile_offsets[b+1]-1 of use64/out256/out64
 * (image order, as ivc_tile_offsets lays them out).  Every sequence is
 * compacted on its own exactly as ivc_connector_compact does for one prompt
 * ([4B-Flash] section 4): positions restart at 0 in each sequence, and the
 * compacted sequences are packed back to back:
 *   out_cu_seqlens [B+1] int32: out_cu_seqlens[0] = 0,
 *                  out_cu_seqlens[b+1] = out_cu_seqlens[b] + L'_b
 *   out_ids [L], out_pos [L]: packed ids and per-sequence positions 0..L'_b-1,
 *                  -1 past out_cu_seqlens[B]
 *   keep_map [L]:  packed index of each input position, or -1 if deleted
 *   out_embeds [L, D]: rows 0..out_cu_seqlens[B]-1 written, the rest untouched
 * All of cu_seqlens, tile_offsets and the outputs are device arrays.
 * dev_status (required) gets IVC_DEV_ERR_IMG_COUNT when a sequence's
 * IMG_CONTEXT count differs from (P/2)^2 times its tile count (that
 * sequence then compacts to length 0, the others are unaffected), and
 * IVC_DEV_ERR_SEQ_LAYOUT when cu_seqlens does not run from 0 to L without
 * decreasing or tile_offsets decreases or leaves [0, T] (then every
 * out_cu_seqlens entry is 0 and every keep_map, out_ids and out_pos entry
 * -1).  B = 0 requires L = 0 and enqueues nothing.  Workspace:
 * ivc_connector_compact_batch_workspace_bytes. */
ivc_status ivc_connector_compact_batch(ivc_connector* h, const int32_t* ids,
                                       const int32_t* cu_seqlens, int32_t B, const void* embeds,
                                       int64_t L, int32_t img_context_id,
                                       const int32_t* tile_offsets, const uint8_t* use64,
                                       const void* out256, const void* out64, int32_t T,
                                       int32_t* out_ids, int32_t* out_pos, int32_t* keep_map,
                                       void* out_embeds, int32_t* out_cu_seqlens,
                                       int32_t* dev_status, void* ws, size_t ws_bytes,
                                       void* stream);

/* Workspace bytes of ivc_connector_compact_batch for up to max_tiles tiles,
 * max_total_len packed tokens and max_seqs sequences. */
size_t ivc_connector_compact_batch_workspace_bytes(const ivc_connector* h, int32_t max_tiles,
                                                   int64_t max_total_len, int32_t max_seqs);

/* The router's batch-wide step alone ([4B-Flash] section 4): threshold =
 * rel_quantile-quantile of gate[:, 0] (linear interpolation between order
 * statistics, computed in fp64 without fused multiply-add), use64[t] = 1 iff
 * gate[t,0] > threshold and gate[t,0] >= abs_threshold.  ivc_connector_route
 * ends with this step; it is exported for callers that gather gates from
 * several producers before deciding.
 *   gate [T, 2] float32, threshold [1] float64 (out), use64 [T] uint8 (out). */
ivc_status ivc_route_decide(const float* gate, int32_t T, double rel_quantile,
                            double abs_threshold, double* threshold, uint8_t* use64, void* stream);

/* Ragged batches: offsets[0] = 0, offsets[i+1] = offsets[i] + tiles_per_image[i]
 * (exclusive prefix sum; the per-sample split of [4B-Flash] section 5).
 * tiles_per_image [B] int32, offsets [B+1] int32 (device).  dev_status gets
 * IVC_DEV_ERR_TILE_COUNT for a negative count or an int32 overflow. */
ivc_status ivc_tile_offsets(const int32_t* tiles_per_image, int32_t B, int32_t* offsets,
                            int32_t* dev_status, void* stream);

/* Stand-alone pixel_shuffle ([14B] pixel_shuffle section), a pure
 * permutation with no normalisation:
 *   vit [T, has_cls + P*P, C] (element type dtype) -> out [T, (P/r)^2, r*r*C],
 *   v2: out[t][a*(P/r)+b][(r*m+k)*C + c] = vit[t][has_cls + (r*a+m)*P + r*b+k][c];
 *   v1 (ps_version = 1): the same row lands at token b*(P/r) + a.
 * r = 2 or 4; for r = 4, shuffle64_order selects the channel order
 * (ivc_shuffle64_order).  ps_version 0 means 2. */
ivc_status ivc_pixel_shuffle(int32_t dtype, const void* vit, int32_t T, int32_t P, int32_t C,
                             int32_t has_cls, int32_t r, int32_t ps_version,
                             int32_t shuffle64_order, void* out, void* stream);

/* Per-kernel timing for measurement: when enabled, the library records a
 * hipEvent pair around each kernel it launches, on the stream it launches it
 * on, and accumulates the elapsed time per kernel name after the events
 * complete.  on = 1: run and run_routed keep both projector chains on the
 * call's stream (no fork), so each kernel is timed alone; on = 2: the chains
 * keep their two streams, as with timing off, so each span is that of the
 * kernel beside whatever the other chain runs meanwhile; 0: off.
 * ivc_profile_read synchronises the recorded events, then returns up to
 * `cap` entries (name, total ms, launches).  Not thread-safe; off by default. */
void ivc_profile_enable(int on);
void ivc_profile_reset(void);
int32_t ivc_profile_read(const char** names, double* total_ms, int64_t* launches, int32_t cap);

const char* ivc_status_string(ivc_status s);
const char* ivc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* IVC_H */
