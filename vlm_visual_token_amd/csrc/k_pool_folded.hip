// CrossAttentionPooling with the key and value projections folded out of the
// token loop (same mathematics as the K/V form; InternVL3_5-4B-Flash Gating
// and CrossAttentionPooling page, section 2).
//
// For one query, head h of layer l scores token x_n as
//   s_n = Q_h . (Wk_h x_n + bk_h) / sqrt(d) = x_n . q~_h + const,
//   q~_h = Wk_h^T Q_h / sqrt(d),
// and the constant (Q_h . bk_h / sqrt(d)) cancels in the softmax.  Since the
// weights sum to one, the head output is
//   o_h = sum_n p_n (Wv_h x_n + bv_h) = Wv_h xbar_h + bv_h,  xbar_h = sum_n p_n x_n.
// So each layer needs one pass over the tile's raw tokens that produces
// xbar_h for every head, plus small per-tile products before (q~) and after
// (Wv xbar).  No K/V tensor is formed.
//
// Token pass (k_pool_folded): the chip's workgroups share the batch's
// token chunks (16 tokens of one tile) evenly, each a contiguous range that
// may cross tile boundaries; per tile touched a workgroup leaves one partial
// (running max, running sum, weighted sums of every head) and a merge kernel
// combines the partials of each tile in a fixed order.  8 waves per
// workgroup, wave w owning channels [w*C/8, (w+1)*C/8).  Per chunk:
//   load     LDS DMA (global_load_lds_dwordx4) into a 4-stage ring, three
//            chunks ahead of the one in use;
//   scores   partial S[token][head] over the wave's channels on
//            v_mfma_f32_16x16x32_bf16, token rows (from LDS) as A, q~ as B,
//            q~ split into bf16 high + low parts so the product keeps ~fp32
//            accuracy; the 8 partials meet in LDS;
//   softmax  lane (head h = lane % 16, g = lane / 16) takes tokens 4g..4g+3
//            of head h, which is exactly the A-operand layout of the next
//            product, so P (split into bf16 hi + lo) stays in registers;
//            scores are in log2 units (q~ carries log2(e)), and the running
//            max moves only when a chunk's max exceeds it by more than 8, so
//            the rescale of the accumulators is rare;
//   sum      xbar[h][c] += P[h][tokens] . X[tokens][c] on
//            v_mfma_f32_16x16x16_bf16, the B operand (4 tokens of one
//            channel) read with ds_read_b64_tr_b16 from the row-major chunk.
// LDS rows are padded to 2*(C+16) bytes (32 mod 256) and 16-byte chunk c of
// row r sits at c ^ ((r >> 3) & 1): the score operand reads (16 rows, one
// 16-byte piece each) and the transposed reads (8 rows x 32 bytes per half
// wave) are then free of bank conflicts.
// An fp32 FMA weighted sum would make the pass VALU-bound (wave64 fp32 FMA
// takes 4 cycles per instruction); on MFMA it is bound by the HBM read of the
// tokens.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace ivc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int FH = 16;  // heads per MFMA column block (fewer heads are zero-padded)

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;
typedef __attribute__((address_space(1))) const char gchar_t;

bool pool_folded_supported(int dtype, int C, int H) {
  return dtype == DT_BF16 && (C == 512 || C == 1024) && H >= 1 && H <= FH && C % H == 0;
}

namespace {
template <int C>
struct PF {
  static constexpr int NW = 8;                 // waves per workgroup
  static constexpr int FT = 16;                // tokens per chunk
  static constexpr int ST = 4;                 // LDS ring stages
  static constexpr int CW = C / NW;            // channels per wave
  static constexpr int KS = CW / 32;           // score k-steps per wave
  static constexpr int NT = CW / 16;           // 16-channel output tiles per wave
  static constexpr int RB = 2 * (C + 16);      // LDS row bytes (32 mod 256)
  static constexpr int SB = FT * RB;           // stage bytes
  static constexpr int IPR = C / 512;          // 1 KB DMA instructions per row
  static constexpr int DPW = 2 * IPR;          // DMA instructions per wave per chunk
  static constexpr int LDP = FT + 4;           // partial-score row (floats)
  static constexpr int WG_PER_CU = C <= 512 ? 2 : 1;
};

IVC_DEV int clamp_valid(const int* valid, int t, int N) {
  const int nv = valid != nullptr ? valid[t] : N;
  return nv < 1 ? 1 : (nv > N ? N : nv);
}

// Walks the non-empty chunks of a workgroup's range [c_lo, c_end) in order,
// or (rev) from the last one down: tile t, chunk j (tokens 16j .. 16j+15),
// nv valid tokens of tile t.
struct ChunkIter {
  int t, j, nv, nce, rev, c_lo;
  IVC_DEV void enter(const int* valid, int N) {
    nv = clamp_valid(valid, t, N);
    nce = (nv + 15) / 16;
  }
  IVC_DEV void rstart(int c_beg, int NC, int c_end, const int* valid, int N) {
    rev = 1;
    c_lo = c_beg;
    if (c_end <= c_beg) {
      t = -1;
      j = 0;
      return;
    }
    t = (c_end - 1) / NC;
    j = c_end - 1 - t * NC;
    enter(valid, N);
    if (j >= nce) j = nce - 1;  // done() below if the range holds none of tile t's valid chunks
  }
  IVC_DEV void start(int c, int NC, int c_end, const int* valid, int N) {
    rev = 0;
    c_lo = c;
    t = c / NC;
    j = c - t * NC;
    if (c < c_end) {
      enter(valid, N);
      if (j >= nce) next_tile(NC, c_end, valid, N);
    }
  }
  IVC_DEV void next_tile(int NC, int c_end, const int* valid, int N) {
    ++t;
    j = 0;
    if (t * NC < c_end) enter(valid, N);  // chunk 0 of a tile is never empty
  }
  IVC_DEV void next(int NC, int c_end, const int* valid, int N) {
    if (rev) {
      if (--j < 0 && --t >= 0) {
        enter(valid, N);
        j = nce - 1;
      }
      return;
    }
    if (++j >= nce) next_tile(NC, c_end, valid, N);
  }
  IVC_DEV bool done(int NC, int c_end) const {
    return rev ? t < 0 || t * NC + j < c_lo : t * NC + j >= c_end;
  }
};

// reductions over the four lanes l, l^16, l^32, l^48 (v_permlane{16,32}_swap)
IVC_DEV float max_x4(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
IVC_DEV float sum_x4(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// s_waitcnt with vmcnt = n (n < 64), expcnt and lgkmcnt left alone
#define IVC_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its outstanding global loads (__syncthreads' release fence would drain the
// DMA ring); the signal fences keep the compiler from moving memory
// operations across it.
IVC_DEV void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

IVC_DEV float bf16_lo_f(uint32_t u) { return __uint_as_float(u << 16); }
IVC_DEV float bf16_hi_f(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats to packed bf16 (v_cvt_pk_bf16_f32, round to nearest even)
IVC_DEV uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// ---- per-token LayerNorm moments ------------------------------------------
// A token's C channels as the token pass holds them: wave w (of 8) has
// channels [w C/8, (w+1) C/8), its lane (token, g = lane / 16) the 8-channel
// pieces g, g + 4, g + 8, ... of that range (KS = C / 256 of them).  Moments
// (mean, M2) are taken per lane (two passes over its 8 KS values), combined
// over the lane's 4 partners (v_permlane32_swap, then v_permlane16_swap) and
// over the 8 waves in a fixed tree.  The token pass (first layer) and
// k_token_stats both run exactly these steps, so their results are equal bit
// for bit.
template <int KS>
IVC_DEV float2 lane_moments(const bf16x8_t (&a)[KS]) {
  float f[KS][8];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const u32x4 u = __builtin_bit_cast(u32x4, a[k]);
    unpack16(u, f[k], (bf16_t*)nullptr);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += f[k][e];
  const float m = s / (float)(8 * KS);
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = f[k][e] - m;
      q = fmaf(d, d, q);
    }
  return make_float2(m, q);
}

// lane l with l ^ 32, then with l ^ 16 (n values per lane); every one of the
// four lanes ends with the same result (the swaps return the lower and the
// upper partner's value in the same order on both sides)
IVC_DEV float2 moments_x4(float2 mo, float n) {
  auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mo.x), __float_as_uint(mo.x), false, false);
  auto rq = __builtin_amdgcn_permlane32_swap(__float_as_uint(mo.y), __float_as_uint(mo.y), false, false);
  mo = moments_pair(make_float2(__uint_as_float(rm[0]), __uint_as_float(rq[0])),
                    make_float2(__uint_as_float(rm[1]), __uint_as_float(rq[1])), 0.5f * n);
  auto sm = __builtin_amdgcn_permlane16_swap(__float_as_uint(mo.x), __float_as_uint(mo.x), false, false);
  auto sq = __builtin_amdgcn_permlane16_swap(__float_as_uint(mo.y), __float_as_uint(mo.y), false, false);
  return moments_pair(make_float2(__uint_as_float(sm[0]), __uint_as_float(sq[0])),
                      make_float2(__uint_as_float(sm[1]), __uint_as_float(sq[1])), n);
}

// the 8 waves' moments of one token (n values each): ((0,1),(2,3)),((4,5),(6,7))
IVC_DEV float2 moments_8(const float2* w8, float n) {
  const float2 a = moments_pair(w8[0], w8[1], 0.5f * n), b = moments_pair(w8[2], w8[3], 0.5f * n);
  const float2 c = moments_pair(w8[4], w8[5], 0.5f * n), d = moments_pair(w8[6], w8[7], 0.5f * n);
  return moments_pair(moments_pair(a, b, n), moments_pair(c, d, n), 2.f * n);
}
}  // namespace

void folded_geometry(int T, int N, int C, int ncu, int* G, int* Q, int* segmax) {
  const int NC = (N + 15) / 16;
  const long long total = (long long)T * NC;
  const int wpc = C <= 512 ? 2 : 1;
  long long g = (long long)(ncu > 0 ? ncu : 256) * wpc;
  if (g > total) g = total;
  if (g < 1) g = 1;
  // no chunks (T = 0): no workgroups, and a quota of 1 keeps the layout defined
  const long long q = total > 0 ? (total + g - 1) / g : 1;
  *Q = (int)q;
  *G = (int)((total + q - 1) / q);
  *segmax = (int)((q + NC - 1) / NC) + 1;
}

// part layout per slot: [FH] running max (log2 units), [FH] running sum, [FH][C] weighted sums
// STATS: also leave every token's LayerNorm moments (mean, M2 over its C
// channels) in tokst[t * N + n] (all tokens valid).
template <int C, bool STATS>
__global__ void __launch_bounds__(512, 2 * PF<C>::WG_PER_CU)
k_pool_folded(const bf16_t* __restrict__ X, int rows, int has_cls, const int* __restrict__ valid,
              int T, int N, const bf16_t* __restrict__ qt_hi, const bf16_t* __restrict__ qt_lo,
              int Q, int segmax, float* __restrict__ part, int* __restrict__ status,
              float2* __restrict__ tokst, int rev, int qt_shared) {
  using P = PF<C>;
  constexpr int NW = P::NW, KS = P::KS, NT = P::NT, RB = P::RB, SB = P::SB, DPW = P::DPW;
  constexpr int LDP = P::LDP;
  __shared__ __attribute__((aligned(1024))) char st0[SB];
  __shared__ __attribute__((aligned(1024))) char st1[SB];
  __shared__ __attribute__((aligned(1024))) char st2[SB];
  __shared__ __attribute__((aligned(1024))) char st3[SB];
  __shared__ __attribute__((aligned(16))) float sP[NW][FH][LDP];
  __shared__ float2 sTS[STATS ? NW * FH : 1];  // [token][wave] moments

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lo16 = lane & 15, hi4 = lane >> 4;
  const int NC = (N + 15) / 16;
  const int total = T * NC;
  const int c_beg = blockIdx.x * Q;
  const int c_end = min(total, c_beg + Q);
  const int t_first = c_beg / NC;
  const int cw0 = w * P::CW;
  // token counts out of range are clamped and flagged (every tile meets some workgroup)
  if (valid != nullptr && status != nullptr && c_beg < c_end) {
    for (int t = t_first + (int)threadIdx.x; t <= (c_end - 1) / NC; t += 512) {
      const int nv = valid[t];
      if (nv < 1 || nv > N) atomicOr(status, 2);
    }
  }

  // ---- DMA of one chunk: wave w loads rows 2w, 2w+1 (IPR instructions each)
  const int dma_f = (w >> 2) & 1;  // swizzle term of rows 2w, 2w+1
  uint32_t dma_off[P::IPR];
#pragma unroll
  for (int hf = 0; hf < P::IPR; ++hf) dma_off[hf] = (uint32_t)(((hf * 64 + lane) ^ dma_f) * 16);
  gchar_t* xg = (gchar_t*)X;
  auto dma = [&](const ChunkIter& it, char* stage) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int R = 2 * w + r;
      const int n = min(16 * it.j + R, it.nv - 1);  // tail rows repeat a valid row (masked later)
      gchar_t* src = xg + ((long long)it.t * rows + has_cls + n) * (long long)(C * 2);
#pragma unroll
      for (int hf = 0; hf < P::IPR; ++hf)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + dma_off[hf]),
                                         (lds_void_t*)(stage + R * RB + hf * 1024), 16, 0, 0);
    }
  };

  // ---- per-lane LDS offsets (bytes within a stage)
  // score A operand: row lo16, 16-byte piece cw0/8 + 4k + hi4 (swizzled)
  const int a_off = lo16 * RB + (cw0 / 8 + (hi4 ^ ((lo16 >> 3) & 1))) * 16;
  // transposed B operand: lane (g = hi4, e = lo16/4, q = lo16%4) points at row
  // 4g + e, channels n0c + 4q .. +3 of 16-channel tile n0c = cw0 + 16 nt
  const int tr_row = 4 * hi4 + (lo16 >> 2), tr_q = lo16 & 3;
  const int tr_off = tr_row * RB + (cw0 / 8 + ((tr_q >> 1) ^ ((tr_row >> 3) & 1))) * 16 + (tr_q & 1) * 8;

  // ---- running state of the current tile.  A new tile only resets the
  // running max and sum: its first chunk then rescales the accumulators by 0.
  // l_run holds this lane's share (its 4 tokens per chunk) of head lo16's sum.
  int cur_t = -1;
  bf16x8_t qh[KS], ql[KS];
  // q~ of the next tile, loaded just before the DMA of its first chunk, so the
  // wait for that chunk covers it and a tile change does not drain the ring
  // (one tile ahead; a short tile whose prefetch is overwritten loads its own)
  bf16x8_t qn_h[KS], qn_l[KS];
  int pf_t = -1;
  auto prefetch_q = [&](int t) {
    const size_t qrow = (qt_shared ? 0 : (size_t)t * FH * C) + (size_t)lo16 * C + cw0 + 8 * hi4;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qn_h[k] = *reinterpret_cast<const bf16x8_t*>(qt_hi + qrow + 32 * k);
      qn_l[k] = *reinterpret_cast<const bf16x8_t*>(qt_lo + qrow + 32 * k);
    }
    pf_t = t;
  };
  f32x4_t acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto flush = [&](int t) {
    float* pp = part + ((size_t)blockIdx.x * segmax + (t - t_first)) * (size_t)(FH * (2 + C));
    const float l_all = sum_x4(l_run);
    if (w == 0 && hi4 == 0) {
      pp[lo16] = m_run;
      pp[FH + lo16] = l_all;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        pp[2 * FH + (size_t)(4 * hi4 + v) * C + cw0 + 16 * nt + lo16] = acc[nt][v];
  };

  // ---- prologue: the first ST-1 chunks into stages 0..ST-2
  ChunkIter pi, ci;
  if (rev) pi.rstart(c_beg, NC, c_end, valid, N);
  else pi.start(c_beg, NC, c_end, valid, N);
  ci = pi;
  int issued = 0, consumed = 0;
  auto dma_next = [&](char* stage) {
    if (pf_t < 0 || (!qt_shared && pi.t != pf_t)) prefetch_q(pi.t);
    dma(pi, stage);
    pi.next(NC, c_end, valid, N);
    ++issued;
  };
  if (!pi.done(NC, c_end)) dma_next(st0);
  if (!pi.done(NC, c_end)) dma_next(st1);
  if (!pi.done(NC, c_end)) dma_next(st2);

  auto step = [&](const char* stage, char* next_stage) {
    // this chunk's DMA is done once at most (issued - consumed - 1) chunks remain in flight
    const int ahead = issued - consumed - 1;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (ahead >= 2) IVC_WAIT_VM(2 * DPW);
    else if (ahead == 1) IVC_WAIT_VM(DPW);
    else IVC_WAIT_VM(0);
    lds_barrier();
    bf16x8_t a[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) a[k] = *reinterpret_cast<const bf16x8_t*>(stage + a_off + 64 * k);

    if (ci.t != cur_t) {
      if (cur_t >= 0) flush(cur_t);
      cur_t = ci.t;
      if (qt_shared || pf_t == ci.t) {
        // prefetched before this chunk's DMA, which the wait above covered
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          qh[k] = qn_h[k];
          ql[k] = qn_l[k];
        }
      } else {
        // q~ rows of this tile, loaded now
        const size_t qrow = (size_t)ci.t * FH * C + (size_t)lo16 * C + cw0 + 8 * hi4;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          qh[k] = *reinterpret_cast<const bf16x8_t*>(qt_hi + qrow + 32 * k);
          ql[k] = *reinterpret_cast<const bf16x8_t*>(qt_lo + qrow + 32 * k);
        }
        IVC_WAIT_VM(0);
      }
      m_run = -INFINITY;
      l_run = 0.f;
    }

    // partial scores: sc[v] = token 4*hi4 + v, head lo16, over this wave's channels
    {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], qh[k], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], ql[k], sc, 0, 0, 0);
      }
      *reinterpret_cast<f32x4_t*>(&sP[w][lo16][4 * hi4]) = sc;
    }
    if (STATS) {
      const float2 mo = moments_x4(lane_moments<KS>(a), (float)(C / 32));
      if (hi4 == 0) sTS[lo16 * NW + w] = mo;
    }
    lds_barrier();
    if (STATS && w == 0 && lane < 16) {
      const int n = 16 * ci.j + lane;
      if (n < N) tokst[(size_t)ci.t * N + n] = moments_8(&sTS[lane * NW], (float)(C / 8));
    }

    // operands of the weighted sum first: they do not depend on the softmax
    s16x4_t b[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      b[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(lds_void_t*)(stage + tr_off + 32 * nt));

    // softmax over this chunk: lane (head lo16, tokens 4*hi4 .. +3)
    f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(&sP[0][lo16][4 * hi4]);
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) s4 += *reinterpret_cast<const f32x4_t*>(&sP[ww][lo16][4 * hi4]);
    // the next DMA goes out after this step's LDS reads: the compiler makes an
    // LDS read that follows an LDS DMA wait for it
    if (!pi.done(NC, c_end)) dma_next(next_stage);
    const int n0 = 16 * ci.j;
    float cmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (n0 + 4 * hi4 + e >= ci.nv) s4[e] = -INFINITY;
      cmax = fmaxf(cmax, s4[e]);
    }
    cmax = max_x4(cmax);  // the chunk's first token is valid, so cmax is finite
    const bool need = cmax > m_run + 8.f;
    if (__ballot(need) != 0) {
      const float m_new = need ? cmax : m_run;
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
      m_run = m_new;
      float cr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) cr[v] = __shfl(corr, 4 * hi4 + v, 64);
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][v] = cr[v] == 0.f ? 0.f : acc[i][v] * cr[v];
    }
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(s4[e] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    const uint32_t h01 = cvt_pk_bf16(p[0], p[1]), h23 = cvt_pk_bf16(p[2], p[3]);
    const uint32_t l01 = cvt_pk_bf16(p[0] - bf16_lo_f(h01), p[1] - bf16_hi_f(h01));
    const uint32_t l23 = cvt_pk_bf16(p[2] - bf16_lo_f(h23), p[3] - bf16_hi_f(h23));
    s16x4_t pah, pal;
    {
      uint2 u{h01, h23}, v{l01, l23};
      pah = __builtin_bit_cast(s16x4_t, u);
      pal = __builtin_bit_cast(s16x4_t, v);
    }

    // xbar += P . X over this wave's 16-channel tiles
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pah, b[nt], acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pal, b[nt], acc[nt], 0, 0, 0);
    }
    ++consumed;
    ci.next(NC, c_end, valid, N);
  };

  // The first step is peeled: after the prologue's DMAs the compiler would
  // otherwise make a partial-score read in the loop wait for every DMA in
  // flight.
  if (!ci.done(NC, c_end)) {
    step(st0, st3);
    while (!ci.done(NC, c_end)) {
      step(st1, st0);
      if (ci.done(NC, c_end)) break;
      step(st2, st1);
      if (ci.done(NC, c_end)) break;
      step(st3, st2);
      if (ci.done(NC, c_end)) break;
      step(st0, st3);
    }
  }
  if (cur_t >= 0) flush(cur_t);
}

// xbar[t][h][c] = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) over the
// partials of tile t, in workgroup order (fmaf accumulation, as the value fold
// that reads the partials directly).  Also flags invalid token counts.
__global__ void __launch_bounds__(256)
k_pool_folded_merge(const float* __restrict__ part, const int* __restrict__ valid, int* status,
                    int N, int C, int H, int Q, int segmax, float* __restrict__ xbar) {
  const int t = blockIdx.x, h = blockIdx.y;
  const int NC = (N + 15) / 16;
  int nv = valid != nullptr ? valid[t] : N;
  if ((nv < 1 || nv > N) && status != nullptr && h == 0 && threadIdx.x == 0) atomicOr(status, 2);
  nv = nv < 1 ? 1 : (nv > N ? N : nv);
  const int lo_c = t * NC, hi_c = t * NC + (nv + 15) / 16;
  const int g0 = lo_c / Q, g1 = (hi_c - 1) / Q;
  const size_t stride = (size_t)FH * (2 + C);
  float M = -INFINITY;
  for (int g = g0; g <= g1; ++g) {
    const float* pp = part + ((size_t)g * segmax + (t - (g * Q) / NC)) * stride;
    M = fmaxf(M, pp[h]);
  }
  float L = 0.f;
  for (int g = g0; g <= g1; ++g) {
    const float* pp = part + ((size_t)g * segmax + (t - (g * Q) / NC)) * stride;
    L = fmaf(pp[FH + h], exp2f(pp[h] - M), L);
  }
  const float invL = 1.0f / L;
  for (int c4 = threadIdx.x; c4 < C / 4; c4 += 256) {
    float4 A = {0.f, 0.f, 0.f, 0.f};
    for (int g = g0; g <= g1; ++g) {
      const float* pp = part + ((size_t)g * segmax + (t - (g * Q) / NC)) * stride;
      const float sc = exp2f(pp[h] - M);
      const float4 v = *reinterpret_cast<const float4*>(pp + 2 * FH + (size_t)h * C + 4 * c4);
      A.x = fmaf(v.x, sc, A.x);
      A.y = fmaf(v.y, sc, A.y);
      A.z = fmaf(v.z, sc, A.z);
      A.w = fmaf(v.w, sc, A.w);
    }
    A.x *= invL;
    A.y *= invL;
    A.z *= invL;
    A.w *= invL;
    *reinterpret_cast<float4*>(xbar + ((size_t)t * H + h) * C + 4 * c4) = A;
  }
}

// Every token's LayerNorm moments without the pooling: workgroup = one
// 16-token chunk (tile c / (N/16)), the 8 waves and lanes holding the same
// channels as in the token pass, read straight from global memory.
template <int C>
__global__ void __launch_bounds__(512)
k_token_stats(const bf16_t* __restrict__ X, int rows, int has_cls, int N,
              float2* __restrict__ tokst) {
  using P = PF<C>;
  constexpr int NW = P::NW, KS = P::KS;
  __shared__ float2 sTS[FH * NW];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lo16 = lane & 15, hi4 = lane >> 4;
  const int NC = N / 16;
  const int t = blockIdx.x / NC, j = blockIdx.x - t * NC;
  const int n = 16 * j + lo16;
  const bf16_t* src = X + ((size_t)t * rows + has_cls + n) * C + w * P::CW + 8 * hi4;
  bf16x8_t a[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k)
    a[k] = __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(
                                            reinterpret_cast<const u32x4*>(src + 32 * k)));
  const float2 mo = moments_x4(lane_moments<KS>(a), (float)(C / 32));
  if (hi4 == 0) sTS[lo16 * NW + w] = mo;
  __syncthreads();
  if (w == 0 && lane < 16)
    tokst[(size_t)t * N + 16 * j + lane] = moments_8(&sTS[lane * NW], (float)(C / 8));
}

// Connectors without the pooling (any width, e.g. C = 3200 or 1024), whose
// moments need not match a token pass: one wave per token, two tokens per
// wave, the lane holding 16-byte pieces lane, lane + 64, ... of the row; two
// passes from registers (mean, then the sum of squared deviations), each
// wave-reduced.
template <int KP>
__global__ void __launch_bounds__(512)
k_token_stats_any(const bf16_t* __restrict__ X, int rows, int has_cls, int N, int C,
                  long long ntok, float2* __restrict__ tokst) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int vpr = C / 8;  // 16-byte pieces per row
  const long long tok0 = ((long long)blockIdx.x * 8 + w) * 2;
  bf16x8_t a[2][KP];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const long long tok = min(tok0 + r, ntok - 1);
    const long long t = tok / N, n = tok - t * N;
    const bf16_t* src = X + ((size_t)t * rows + has_cls + n) * (size_t)C;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int v = lane + 64 * k;
      a[r][k] = v < vpr ? __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(
                                                         reinterpret_cast<const u32x4*>(src) + v))
                        : bf16x8_t{};
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    float f[KP][8];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      unpack16(__builtin_bit_cast(u32x4, a[r][k]), f[k], (bf16_t*)nullptr);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += f[k][e];  // pieces past the row are zero
    }
    const float mean = wave_sum(s) / (float)C;
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      if (lane + 64 * k < vpr) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = f[k][e] - mean;
          q = fmaf(d, d, q);
        }
      }
    }
    q = wave_sum(q);
    if (lane == 0 && tok0 + r < ntok) tokst[tok0 + r] = make_float2(mean, q);
  }
}

bool token_stats_supported(int dtype, int C, int N) {
  return dtype == DT_BF16 && N % 16 == 0 && N > 0 && C % 8 == 0 && C >= 64 && C <= 8 * 64 * 8;
}

hipError_t launch_token_stats(const void* X, int T, int rows, int has_cls, int N, int C,
                              float* tokst, hipStream_t s, bool pool_order) {
  if (T <= 0) return hipSuccess;
  if (!token_stats_supported(DT_BF16, C, N) || (uintptr_t)X % 16 || (uintptr_t)tokst % 8)
    return hipErrorInvalidValue;
  const long long nb = (long long)T * (N / 16);
  if (nb > 0x7fffffffll) return hipErrorInvalidValue;
  if (pool_order && C != 512 && C != 1024) return hipErrorInvalidValue;
  if (pool_order && C == 1024) {
    hipLaunchKernelGGL(k_token_stats<1024>, dim3((unsigned)nb), dim3(512), 0, s,
                       (const bf16_t*)X, rows, has_cls, N, (float2*)tokst);
  } else if (pool_order) {
    hipLaunchKernelGGL(k_token_stats<512>, dim3((unsigned)nb), dim3(512), 0, s, (const bf16_t*)X,
                       rows, has_cls, N, (float2*)tokst);
  } else {
    // 16 tokens per workgroup, as above (nb workgroups)
    const long long ntok = (long long)T * N;
    const int kp = (C / 8 + 63) / 64;
#define IVC_TSA(K)                                                                                 \
  hipLaunchKernelGGL(k_token_stats_any<K>, dim3((unsigned)nb), dim3(512), 0, s, (const bf16_t*)X, \
                     rows, has_cls, N, C, ntok, (float2*)tokst)
    if (kp <= 2) IVC_TSA(2);
    else if (kp <= 4) IVC_TSA(4);
    else if (kp <= 7) IVC_TSA(7);
    else IVC_TSA(8);
#undef IVC_TSA
  }
  return hipGetLastError();
}

hipError_t launch_pool_folded(const FoldedArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (!pool_folded_supported(a.dtype, a.C, a.H)) return hipErrorInvalidValue;
  if (a.G < 1 || a.Q < 1 || a.segmax < 1) return hipErrorInvalidValue;
  dim3 grid((unsigned)a.G);
  if (a.tokst != nullptr && (a.valid != nullptr || a.N % 16 != 0)) return hipErrorInvalidValue;
#define IVC_PF(CV, ST)                                                                             \
  hipLaunchKernelGGL((k_pool_folded<CV, ST>), grid, dim3(512), 0, s, (const bf16_t*)a.X, a.rows,   \
                     a.has_cls, a.valid, a.T, a.N, (const bf16_t*)a.qt_hi,                         \
                     (const bf16_t*)a.qt_lo, a.Q, a.segmax, a.part, a.status, (float2*)a.tokst, \
                     a.reverse, a.qt_shared)
  if (a.C == 1024) {
    if (a.tokst) IVC_PF(1024, true);
    else IVC_PF(1024, false);
  } else {
    if (a.tokst) IVC_PF(512, true);
    else IVC_PF(512, false);
  }
#undef IVC_PF
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.xbar == nullptr) return hipSuccess;  // the partials are read by the merged value fold
  hipLaunchKernelGGL(k_pool_folded_merge, dim3((unsigned)a.T, (unsigned)a.H), dim3(256), 0, s,
                     (const float*)a.part, a.valid, a.status, a.N, a.C, a.H, a.Q, a.segmax,
                     a.xbar);
  return hipGetLastError();
}

// q~[t][h][c] = scale * sum_i Q[t][h*d + i] * Wk[h*d + i][c], split into bf16
// high and low parts; heads h >= H (padding up to 16) are zero.
// grid (C / 256, ceil(T / 16), 16), 256 threads: one channel per thread,
// 16 tiles per block.
template <typename E>
__global__ void __launch_bounds__(256)
k_fold_query(const float* __restrict__ Q, const E* __restrict__ Wk, int T, int C, int H,
             float scale, bf16_t* __restrict__ qt_hi, bf16_t* __restrict__ qt_lo) {
  constexpr int TB = 16;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int t0 = blockIdx.y * TB;
  const int h = blockIdx.z;
  const int d = C / H;
  __shared__ float sq[TB][64];
  float acc[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) acc[i] = 0.f;
  if (h < H) {
    for (int i0 = 0; i0 < d; i0 += 64) {
      const int ni = min(64, d - i0);
      __syncthreads();
      for (int e = threadIdx.x; e < TB * 64; e += 256) {
        const int tt = e / 64, ii = e % 64;
        sq[tt][ii] = (t0 + tt < T && ii < ni) ? Q[(size_t)(t0 + tt) * C + h * d + i0 + ii] : 0.f;
      }
      __syncthreads();
      if (c < C) {
        for (int ii = 0; ii < ni; ++ii) {
          const float wv = Elem<E>::to_f(Wk[(size_t)(h * d + i0 + ii) * C + c]);
#pragma unroll
          for (int tt = 0; tt < TB; ++tt) acc[tt] = fmaf(sq[tt][ii], wv, acc[tt]);
        }
      }
    }
  }
  if (c >= C) return;
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float v = acc[tt] * scale;
    const bf16_t hi = f32_to_bf16(v);
    const bf16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
    const size_t o = ((size_t)t * FH + h) * C + c;
    qt_hi[o] = hi;
    qt_lo[o] = lo;
  }
}

hipError_t launch_fold_query(int dtype, const float* Q, const void* Wk, void* qt_hi, void* qt_lo,
                             int T, int C, int H, float scale, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((C + 255) / 256), (unsigned)((T + 15) / 16), FH);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_fold_query<bf16_t>, grid, dim3(256), 0, s, Q, (const bf16_t*)Wk, T, C, H,
                       scale, (bf16_t*)qt_hi, (bf16_t*)qt_lo);
  else
    hipLaunchKernelGGL(k_fold_query<float>, grid, dim3(256), 0, s, Q, (const float*)Wk, T, C, H,
                       scale, (bf16_t*)qt_hi, (bf16_t*)qt_lo);
  return hipGetLastError();
}

// o[t][h*d + i] = bv[h*d + i] + sum_c Wv[h*d + i][c] * xbar[t][h][c]
// grid (H, ceil(T / 8)), 256 threads: the 8 tiles' xbar rows of head h are
// staged in LDS; each wave takes outputs i = w, w+4, ... and a lane holds
// C/64 channels of the Wv row.
template <typename E>
__global__ void __launch_bounds__(256)
k_fold_value(const float* __restrict__ xbar, const E* __restrict__ Wv, const float* __restrict__ bv,
             float* __restrict__ o, int T, int C, int H) {
  constexpr int TB = 8;
  extern __shared__ float sx[];  // [TB][C]
  const int h = blockIdx.x, t0 = blockIdx.y * TB;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = C / H;
  for (int e = threadIdx.x; e < TB * C; e += 256) {
    const int tt = e / C, c = e - tt * C;
    sx[e] = t0 + tt < T ? xbar[((size_t)(t0 + tt) * H + h) * C + c] : 0.f;
  }
  __syncthreads();
  for (int i = w; i < d; i += 4) {
    const int row = h * d + i;
    float acc[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) acc[tt] = 0.f;
    for (int c = lane; c < C; c += 64) {
      const float wv = Elem<E>::to_f(Wv[(size_t)row * C + c]);
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) acc[tt] = fmaf(wv, sx[tt * C + c], acc[tt]);
    }
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      const float v = wave_sum(acc[tt]);
      if (lane == 0 && t0 + tt < T) o[(size_t)(t0 + tt) * C + row] = v + bv[row];
    }
  }
}

hipError_t launch_fold_value(int dtype, const float* xbar, const void* Wv, const float* bv,
                             float* o, int T, int C, int H, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)H, (unsigned)((T + 7) / 8));
  const size_t lds = (size_t)8 * C * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_fold_value<bf16_t>, grid, dim3(256), lds, s, xbar, (const bf16_t*)Wv, bv, o,
                       T, C, H);
  else
    hipLaunchKernelGGL(k_fold_value<float>, grid, dim3(256), lds, s, xbar, (const float*)Wv, bv, o, T,
                       C, H);
  return hipGetLastError();
}

}  // namespace ivc
