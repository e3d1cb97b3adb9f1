// Sequence compaction after routing (compress_visual_tokens_in_sentence) and
// IMG_CONTEXT embedding injection.
//
// InternVL3_5-4B-Flash Gating and CrossAttentionPooling page, section 4: a
// tile routed to strong compression keeps only its first 64 visual tokens,
// the other 192 are deleted from the input sequence, and positions are
// corrected.  InternVL3-14B-Instruct page, token-injection section: the
// visual vectors replace the IMG_CONTEXT positions in order, so the k-th
// IMG_CONTEXT token is slot k % S of tile k / S.
//
// Closed form used here: with k(p) IMG_CONTEXT tokens before position p, the
// slots deleted before p are
//   f(k) = (S - S64) * routed_before[k / S] + use64[k / S] * max(0, k % S - S64),
// so a kept token moves to j = p - f(k(p)).  Only one scan over the sequence
// (the IMG_CONTEXT count) is needed, plus a scan of use64 over tiles:
//   1. k_compact_count  per-1024-token block IMG_CONTEXT counts
//   2. k_compact_plan   (one workgroup) block offsets, routed_before, L', status
//   3. k_compact_map    per-position keep flag and destination; writes
//                       out_ids, out_pos, keep_map and a source code per row
//                       (and, optionally, the compacted row of every image
//                       slot, so a projector can write its rows there itself)
//   4. k_compact_copy   one wave per output row, 16-byte copies of the row
//                       (k_compact_copy_text: the text rows only)
#include "common.h"
#include "index_math.h"
#include "kernels.h"

namespace ivc {

constexpr int CB = 1024;  // positions per block
constexpr int CT = 256;   // threads per block (4 positions each)

long long compact_blocks(long long L) { return (L + CB - 1) / CB; }

IVC_DEV int block_excl_scan(int v, int* sh /*[4]*/, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += sh[i];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return before + inc - v;
}

__global__ void __launch_bounds__(CT)
k_compact_count(const int32_t* __restrict__ ids, long long L, int img, int32_t* __restrict__ cnt) {
  const long long base = (long long)blockIdx.x * CB + threadIdx.x * 4;
  int c = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) c += (base + e < L && ids[base + e] == img) ? 1 : 0;
  __shared__ int sh[4];
  int total;
  block_excl_scan(c, sh, &total);
  if (threadIdx.x == 0) cnt[blockIdx.x] = total;
}

__global__ void __launch_bounds__(1024)
k_compact_plan(const int32_t* __restrict__ cnt, long long nblk, const uint8_t* __restrict__ use64,
               int T, int S, int S64, long long L, int32_t* __restrict__ blk_off,
               int32_t* __restrict__ routed_before, long long* __restrict__ out_len,
               int32_t* __restrict__ status, int32_t* __restrict__ slot_dst) {
  __shared__ long long carry_s;
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // exclusive scans in chunks of 1024 with a running carry
  auto scan = [&](auto get, auto put, long long n) -> long long {
    if (threadIdx.x == 0) carry_s = 0;
    __syncthreads();
    for (long long c0 = 0; c0 < n; c0 += 1024) {
      const long long i = c0 + threadIdx.x;
      const int v = i < n ? get(i) : 0;
      int inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      if (lane == 63) wsum[w] = inc;
      __syncthreads();
      int before = 0, tot = 0;
      for (int k = 0; k < 16; ++k) {
        if (k < w) before += wsum[k];
        tot += wsum[k];
      }
      const long long carry = carry_s;
      if (i < n) put(i, carry + before + inc - v);
      __syncthreads();
      if (threadIdx.x == 0) carry_s = carry + tot;
      __syncthreads();
    }
    return carry_s;
  };
  const long long n_img =
      scan([&](long long i) { return (int)cnt[i]; },
           [&](long long i, long long v) { blk_off[i] = (int32_t)v; }, nblk);
  const long long n_routed =
      scan([&](long long i) { return (int)(use64[i] != 0); },
           [&](long long i, long long v) { routed_before[i] = (int32_t)v; }, (long long)T);
  if (threadIdx.x == 0) {
    routed_before[T] = (int32_t)n_routed;
    blk_off[nblk] = (int32_t)n_img;
    if (out_len != nullptr) {  // single sequence: check the slot count, set L'
      const bool ok = n_img == (long long)T * S;
      if (!ok) atomicOr(status, 1);
      *out_len = ok ? L - (long long)(S - S64) * n_routed : 0;
    }
  }
  // slot destinations: with the right slot count the map kernel writes every
  // entry; otherwise nothing is placed (slots the sequence lacks included)
  if (out_len != nullptr && slot_dst != nullptr && n_img != (long long)T * S)
    for (long long i = threadIdx.x; i < (long long)T * S; i += blockDim.x) slot_dst[i] = -1;
}

__global__ void __launch_bounds__(CT)
k_compact_map(const int32_t* __restrict__ ids, long long L, int img, const uint8_t* __restrict__ use64,
              int T, int S, int S64, const int32_t* __restrict__ blk_off,
              const int32_t* __restrict__ routed_before, const long long* __restrict__ out_len,
              int32_t* __restrict__ out_ids, int32_t* __restrict__ out_pos,
              int32_t* __restrict__ keep_map, long long* __restrict__ src,
              int32_t* __restrict__ slot_dst) {
  const long long base = (long long)blockIdx.x * CB + threadIdx.x * 4;
  int tok[4], c = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    tok[e] = base + e < L ? ids[base + e] : 0;
    c += (base + e < L && tok[e] == img) ? 1 : 0;
  }
  __shared__ int sh[4];
  int total;
  int k = blk_off[blockIdx.x] + block_excl_scan(c, sh, &total);
  const long long Lp = *out_len;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const long long p = base + e;
    if (p >= L) break;
    const bool is_img = tok[e] == img;
    const int tile = k / S, loc = k - tile * S;
    // slots deleted before p; k == T*S exactly is text after the last slot,
    // and a slot past T*S (malformed sequence: status set) is dropped
    const long long f = compact_deleted_before(k, T, S, S64, routed_before, use64);
    const bool keep = !is_img || compact_keeps_slot(k, T, S, S64, use64);
    long long code = p;  // text: its own embedding row
    if (is_img && tile < T)
      code = use64[tile] != 0 ? ((2ll << 60) | ((long long)tile * S64 + loc))
                              : ((1ll << 60) | ((long long)tile * S + loc));
    const long long j = p - f;
    keep_map[p] = keep ? (int32_t)j : -1;
    if (keep) {
      out_ids[j] = tok[e];
      src[j] = code;
    }
    // L' = 0 (wrong slot count): nothing is placed
    if (slot_dst != nullptr && is_img && tile < T) slot_dst[k] = keep && Lp > 0 ? (int32_t)j : -1;
    out_pos[p] = p < Lp ? (int32_t)p : -1;
    if (p >= Lp) out_ids[p] = -1;
    if (is_img) ++k;
  }
}

// One wave per output row, 16-byte vectors; rows whose source kind (0 text,
// 1 out256, 2 out64) is not in `kinds` are left alone.
template <int VPL>
__global__ void __launch_bounds__(256)
k_compact_copy(const long long* __restrict__ src, const long long* __restrict__ out_len,
               const u32x4* __restrict__ embeds, const u32x4* __restrict__ o256,
               const u32x4* __restrict__ o64, u32x4* __restrict__ out, int vpr, long long L,
               int kinds) {
  const long long j = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= L || j >= *out_len) return;
  const long long code = src[j];
  const int kind = (int)(code >> 60);
  if (((kinds >> kind) & 1) == 0) return;
  const long long idx = code & ((1ll << 60) - 1);
  const u32x4* s = (kind == 0 ? embeds : kind == 1 ? o256 : o64) + idx * vpr;
  u32x4* d = out + j * vpr;
  u32x4 v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = lane + 64 * i;
    if (c < vpr) v[i] = __builtin_nontemporal_load(s + c);
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = lane + 64 * i;
    if (c < vpr) __builtin_nontemporal_store(v[i], d + c);
  }
}

// The text rows only (a few percent of a compacted sequence, in runs between
// the images): one wave per 4 consecutive output rows reads their source
// codes and copies the text rows among them together (all of their loads,
// then all of their stores).
constexpr int kTextRowsPerWave = 4;
template <int VPL>
__global__ void __launch_bounds__(256)
k_compact_copy_text(const long long* __restrict__ src, const long long* __restrict__ out_len,
                    const u32x4* __restrict__ embeds, u32x4* __restrict__ out, int vpr,
                    long long L) {
  const long long j0 = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * kTextRowsPerWave;
  const int lane = threadIdx.x & 63;
  const long long n = min(L, *out_len);
  if (j0 >= n) return;
  const bool in = lane < kTextRowsPerWave && j0 + lane < n;
  const long long code = in ? src[j0 + lane] : 0;
  unsigned long long m = __ballot(in && (code >> 60) == 0);
  while (m != 0ull) {
    int b[4];
    int k = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b[q] = 0;
      if (m != 0ull) {
        b[q] = __builtin_ctzll(m);
        m &= m - 1;
        k = q + 1;
      }
    }
    u32x4 v[4][VPL];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long long idx = __shfl(code, b[q]);
      if (q < k) {
        const u32x4* s = embeds + idx * vpr;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          const int c = lane + 64 * i;
          if (c < vpr) v[q][i] = __builtin_nontemporal_load(s + c);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < k) {
        u32x4* d = out + (j0 + b[q]) * vpr;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          const int c = lane + 64 * i;
          if (c < vpr) __builtin_nontemporal_store(v[q][i], d + c);
        }
      }
    }
  }
}

__global__ void k_set_i64(long long* p, long long v) { *p = v; }

__global__ void __launch_bounds__(256) k_fill_i32(int32_t* p, long long n, int32_t v) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    p[i] = v;
}

// ---- batched, ragged compaction ---------------------------------------------
// Per sequence the closed form above holds with the sequence's own counters:
// k = IMG_CONTEXT tokens of the sequence before p, tiles numbered from
// tile_off[b], routed_before taken relative to tile_off[b], and the result
// placed at out_cu[b] + (p - cu[b]) - f.  Kernels:
//   k_compact_count (shared)  per-block IMG_CONTEXT counts
//   k_compact_plan  (shared)  block offsets and routed_before, no L' / status
//   k_cbatch_bounds           IMG_CONTEXT count before every sequence start
//   k_cbatch_plan             layout check, per-sequence L'_b, slot check,
//                             out_cu = exclusive scan of L'_b
//   k_cbatch_map              keep flag, destination, ids, positions, source
//   k_compact_copy  (shared)  the embedding rows

// One wave per sequence boundary b <= B: IMG_CONTEXT tokens before cu[b].
__global__ void __launch_bounds__(256)
k_cbatch_bounds(const int32_t* __restrict__ ids, long long L, int img,
                const int32_t* __restrict__ cu, int B, const int32_t* __restrict__ blk_off,
                int32_t* __restrict__ seq_img) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b > B) return;
  const long long p0 = min(max((long long)cu[b], 0ll), L);  // out-of-range offsets are flagged later
  const long long blk = p0 / CB;
  int c = 0;
#pragma unroll
  for (int i = 0; i < CB / 64; ++i) {
    const long long p = blk * CB + lane + 64 * i;
    c += (p < p0 && ids[p] == img) ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if (lane == 0) seq_img[b] = blk_off[blk] + c;
}

__global__ void __launch_bounds__(1024)
k_cbatch_plan(const int32_t* __restrict__ cu, const int32_t* __restrict__ tile_off, int B,
              long long L, int T, int S, int S64, const int32_t* __restrict__ seq_img,
              const int32_t* __restrict__ routed_before, int32_t* __restrict__ out_cu,
              int32_t* __restrict__ seq_ok, long long* __restrict__ total,
              int32_t* __restrict__ layout_ok, int32_t* __restrict__ status) {
  __shared__ int bad, any_miss;
  __shared__ long long carry_s;
  __shared__ long long wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    bad = (cu[0] != 0 || (long long)cu[B] != L || tile_off[0] < 0 || tile_off[B] > T) ? 1 : 0;
    any_miss = 0;
    carry_s = 0;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x)
    if (cu[b] > cu[b + 1] || tile_off[b] > tile_off[b + 1]) atomicOr(&bad, 1);
  __syncthreads();
  if (bad) {  // not an ordered partition: empty result
    for (int b = threadIdx.x; b <= B; b += blockDim.x) out_cu[b] = 0;
    if (threadIdx.x == 0) {
      *total = 0;
      *layout_ok = 0;
      atomicOr(status, 8);
    }
    return;
  }
  const long long drop = S - S64;
  for (int c0 = 0; c0 < B; c0 += 1024) {
    const int b = c0 + threadIdx.x;
    long long v = 0;
    if (b < B) {
      const int t0 = tile_off[b], t1 = tile_off[b + 1];
      const bool ok = (long long)(seq_img[b + 1] - seq_img[b]) == (long long)S * (t1 - t0);
      if (ok)
        v = (long long)(cu[b + 1] - cu[b]) - drop * (routed_before[t1] - routed_before[t0]);
      else
        atomicOr(&any_miss, 1);
      seq_ok[b] = ok ? 1 : 0;
    }
    long long inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long t = __shfl_up(inc, o, 64);
      if (lane >= o) inc += t;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    long long before = 0, tot = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < w) before += wsum[k];
      tot += wsum[k];
    }
    const long long carry = carry_s;
    if (b < B) out_cu[b] = (int32_t)(carry + before + inc - v);
    __syncthreads();
    if (threadIdx.x == 0) carry_s = carry + tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out_cu[B] = (int32_t)carry_s;
    *total = carry_s;
    *layout_ok = 1;
    if (any_miss) atomicOr(status, 1);
  }
}

__global__ void __launch_bounds__(CT)
k_cbatch_map(const int32_t* __restrict__ ids, long long L, int img,
             const uint8_t* __restrict__ use64, int S, int S64, const int32_t* __restrict__ cu,
             const int32_t* __restrict__ tile_off, int B, const int32_t* __restrict__ blk_off,
             const int32_t* __restrict__ routed_before, const int32_t* __restrict__ seq_img,
             const int32_t* __restrict__ seq_ok, const int32_t* __restrict__ out_cu,
             const long long* __restrict__ total, const int32_t* __restrict__ layout_ok,
             int32_t* __restrict__ out_ids, int32_t* __restrict__ out_pos,
             int32_t* __restrict__ keep_map, long long* __restrict__ src) {
  const long long base = (long long)blockIdx.x * CB + threadIdx.x * 4;
  if (*layout_ok == 0) {  // uniform over the grid
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (base + e < L) keep_map[base + e] = out_ids[base + e] = out_pos[base + e] = -1;
    return;
  }
  int tok[4], c = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    tok[e] = base + e < L ? ids[base + e] : 0;
    c += (base + e < L && tok[e] == img) ? 1 : 0;
  }
  __shared__ int sh[4];
  int blk_total;
  int g = blk_off[blockIdx.x] + block_excl_scan(c, sh, &blk_total);  // IMG_CONTEXT before base
  if (base >= L) return;
  const long long Lp = *total;
  const long long drop = S - S64;
  // sequence holding position base: the last b with cu[b] <= base (cu[B] = L > base)
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)cu[mid] <= base) lo = mid;
    else hi = mid - 1;
  }
  int b = -1;
  long long c0 = 0, c1 = 0;
  int t0 = 0, nt = 0, rb0 = 0, g0 = 0, ok = 0, oc = 0;
  auto enter = [&](int nb) {
    b = nb;
    c0 = cu[b];
    c1 = cu[b + 1];
    t0 = tile_off[b];
    nt = tile_off[b + 1] - t0;
    rb0 = routed_before[t0];
    g0 = seq_img[b];
    ok = seq_ok[b];
    oc = out_cu[b];
  };
  enter(lo);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const long long p = base + e;
    if (p >= L) break;
    if (p >= c1) {
      int nb = b + 1;
      while ((long long)cu[nb + 1] <= p) ++nb;  // skips empty sequences; ends since cu[B] = L
      enter(nb);
    }
    const bool is_img = tok[e] == img;
    const int k = g - g0;  // IMG_CONTEXT of this sequence before p
    const int tl = k / S, loc = k - tl * S;
    long long f;  // slots of this sequence deleted before p
    bool keep = ok != 0;
    long long code = p;
    if (tl < nt) {
      const int tile = t0 + tl;
      const int u = use64[tile] != 0;
      f = drop * (routed_before[tile] - rb0) + (u ? max(0, loc - S64) : 0);
      if (is_img) {
        keep = keep && (!u || loc < S64);
        code = u ? ((2ll << 60) | ((long long)tile * S64 + loc))
                 : ((1ll << 60) | ((long long)tile * S + loc));
      }
    } else {
      // text after the sequence's last slot (an extra slot only occurs when ok = 0)
      f = drop * (routed_before[t0 + nt] - rb0);
      if (is_img) keep = false;
    }
    const long long jl = (p - c0) - f;
    const long long j = oc + jl;
    keep_map[p] = keep ? (int32_t)j : -1;
    if (keep) {
      out_ids[j] = tok[e];
      out_pos[j] = (int32_t)jl;
      src[j] = code;
    }
    if (p >= Lp) out_ids[p] = out_pos[p] = -1;
    if (is_img) ++g;
  }
}

static hipError_t launch_copy(const CompactArgs& a, const long long* len, hipStream_t s,
                              int kinds = 7) {
  const int esz = a.dtype == DT_BF16 ? 2 : 4;
  const int vpr = (int)((long long)a.D * esz / 16);
  const int vpl = (vpr + 63) / 64;
  dim3 grid((unsigned)((a.L + 3) / 4));
#define IVC_COPY(n)                                                                              \
  hipLaunchKernelGGL(k_compact_copy<n>, grid, dim3(256), 0, s, (const long long*)a.src, len,    \
                     (const u32x4*)a.embeds, (const u32x4*)a.out256, (const u32x4*)a.out64,     \
                     (u32x4*)a.out_embeds, vpr, a.L, kinds)
  if (vpl <= 1) IVC_COPY(1);
  else if (vpl <= 2) IVC_COPY(2);
  else if (vpl <= 4) IVC_COPY(4);
  else if (vpl <= 8) IVC_COPY(8);
  else if (vpl <= 16) IVC_COPY(16);
  else return hipErrorInvalidValue;
#undef IVC_COPY
  return hipGetLastError();
}

hipError_t launch_compact_batch(const CompactBatchArgs& ba, hipStream_t s) {
  const CompactArgs& a = ba.base;
  const long long nblk = compact_blocks(a.L);
  if (a.L > 0) {
    hipLaunchKernelGGL(k_compact_count, dim3((unsigned)nblk), dim3(CT), 0, s, a.ids, a.L, a.img_id,
                       a.blk_cnt);
  }
  hipLaunchKernelGGL(k_compact_plan, dim3(1), dim3(1024), 0, s, (const int32_t*)a.blk_cnt, nblk,
                     a.use64, a.T, a.S, a.S64, a.L, a.blk_off, a.routed_before,
                     (long long*)nullptr, a.status, (int32_t*)nullptr);
  hipLaunchKernelGGL(k_cbatch_bounds, dim3((unsigned)((ba.B + 1 + 3) / 4)), dim3(256), 0, s, a.ids,
                     a.L, a.img_id, ba.cu, ba.B, (const int32_t*)a.blk_off, ba.seq_img);
  hipLaunchKernelGGL(k_cbatch_plan, dim3(1), dim3(1024), 0, s, ba.cu, ba.tile_off, ba.B, a.L, a.T,
                     a.S, a.S64, (const int32_t*)ba.seq_img, (const int32_t*)a.routed_before,
                     ba.out_cu, ba.seq_ok, ba.total, ba.layout_ok, a.status);
  if (a.L == 0) return hipGetLastError();
  hipLaunchKernelGGL(k_cbatch_map, dim3((unsigned)nblk), dim3(CT), 0, s, a.ids, a.L, a.img_id,
                     a.use64, a.S, a.S64, ba.cu, ba.tile_off, ba.B, (const int32_t*)a.blk_off,
                     (const int32_t*)a.routed_before, (const int32_t*)ba.seq_img,
                     (const int32_t*)ba.seq_ok, (const int32_t*)ba.out_cu,
                     (const long long*)ba.total, (const int32_t*)ba.layout_ok, a.out_ids, a.out_pos,
                     a.keep_map, a.src);
  return launch_copy(a, ba.total, s);
}

// The index half: ids, positions, keep map, L' and each output row's source
// (needs use64 and ids only, not the projector outputs).
hipError_t launch_compact_index(const CompactArgs& a, hipStream_t s) {
  const long long nblk = compact_blocks(a.L);
  if (a.L == 0) {
    // nothing to scan; out_len = 0 (a kernel, not a memset, so the call can be graph-captured)
    hipLaunchKernelGGL(k_set_i64, dim3(1), dim3(1), 0, s, a.out_len, 0ll);
    if (a.slot_dst != nullptr && a.T > 0) {  // tiles but no slots: nothing is placed
      const long long n = (long long)a.T * a.S;
      hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)),
                         dim3(256), 0, s, a.slot_dst, n, -1);
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_compact_count, dim3((unsigned)nblk), dim3(CT), 0, s, a.ids, a.L, a.img_id,
                     a.blk_cnt);
  hipLaunchKernelGGL(k_compact_plan, dim3(1), dim3(1024), 0, s, (const int32_t*)a.blk_cnt, nblk,
                     a.use64, a.T, a.S, a.S64, a.L, a.blk_off, a.routed_before, a.out_len, a.status,
                     a.slot_dst);
  hipLaunchKernelGGL(k_compact_map, dim3((unsigned)nblk), dim3(CT), 0, s, a.ids, a.L, a.img_id,
                     a.use64, a.T, a.S, a.S64, (const int32_t*)a.blk_off,
                     (const int32_t*)a.routed_before, (const long long*)a.out_len, a.out_ids,
                     a.out_pos, a.keep_map, a.src, a.slot_dst);
  return hipGetLastError();
}

// The copy half: the embedding rows, from the index half's sources.
hipError_t launch_compact_copy(const CompactArgs& a, hipStream_t s) {
  if (a.L == 0) return hipSuccess;
  return launch_copy(a, (const long long*)a.out_len, s);
}

hipError_t launch_compact_copy_kinds(const CompactArgs& a, int kinds, hipStream_t s) {
  if (a.L == 0 || (kinds & 7) == 0) return hipSuccess;
  return launch_copy(a, (const long long*)a.out_len, s, kinds & 7);
}

hipError_t launch_compact_copy_text(const CompactArgs& a, hipStream_t s) {
  if (a.L == 0) return hipSuccess;
  const int esz = a.dtype == DT_BF16 ? 2 : 4;
  const int vpr = (int)((long long)a.D * esz / 16);
  const int vpl = (vpr + 63) / 64;
  const long long rows_per_wg = 4ll * kTextRowsPerWave;
  dim3 grid((unsigned)((a.L + rows_per_wg - 1) / rows_per_wg));
#define IVC_COPY_TEXT(n)                                                                      \
  hipLaunchKernelGGL(k_compact_copy_text<n>, grid, dim3(256), 0, s, (const long long*)a.src, \
                     (const long long*)a.out_len, (const u32x4*)a.embeds,                    \
                     (u32x4*)a.out_embeds, vpr, a.L)
  if (vpl <= 1) IVC_COPY_TEXT(1);
  else if (vpl <= 2) IVC_COPY_TEXT(2);
  else if (vpl <= 4) IVC_COPY_TEXT(4);
  else if (vpl <= 8) IVC_COPY_TEXT(8);
  else if (vpl <= 16) IVC_COPY_TEXT(16);
  else return hipErrorInvalidValue;
#undef IVC_COPY_TEXT
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const hipError_t e = launch_compact_index(a, s);
  if (e != hipSuccess) return e;
  return launch_compact_copy(a, s);
}

// ---- ragged tile offsets -------------------------------------------------------
__global__ void __launch_bounds__(1024)
k_tile_offsets(const int32_t* __restrict__ tiles, int B, int32_t* __restrict__ off,
               int32_t* __restrict__ status) {
  __shared__ long long wsum[16];
  __shared__ long long carry_s;
  __shared__ int bad;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    carry_s = 0;
    bad = 0;
  }
  __syncthreads();
  for (int c0 = 0; c0 < B; c0 += 1024) {
    const int i = c0 + threadIdx.x;
    long long v = 0;
    if (i < B) {
      v = tiles[i];
      if (v < 0) atomicOr(&bad, 1);
    }
    long long inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long t = __shfl_up(inc, o, 64);
      if (lane >= o) inc += t;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    long long before = 0, tot = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < w) before += wsum[k];
      tot += wsum[k];
    }
    const long long carry = carry_s;
    const long long ex = carry + before + inc - v;
    if (i < B) {
      if (ex > 0x7fffffffll) atomicOr(&bad, 1);
      off[i] = (int32_t)ex;
    }
    __syncthreads();
    if (threadIdx.x == 0) carry_s = carry + tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (carry_s > 0x7fffffffll) bad = 1;
    off[B] = (int32_t)carry_s;
    if (bad && status != nullptr) atomicOr(status, 4);
  }
}

hipError_t launch_tile_offsets(const int32_t* tiles, int B, int32_t* offsets, int32_t* status,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_tile_offsets, dim3(1), dim3(1024), 0, s, tiles, B, offsets, status);
  return hipGetLastError();
}

}  // namespace ivc
