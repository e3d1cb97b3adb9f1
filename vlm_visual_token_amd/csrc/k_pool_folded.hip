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
// Token pass (k_pool_folded): a workgroup takes a token range of one tile,
// 32 tokens at a time, 8 waves each owning C/8 channels.  Both products run
// on v_mfma_f32_16x16x32_bf16: the scores with the token rows as the A
// operand and q~ as B, split into a bf16 high and low part so the product
// keeps ~fp32 accuracy; the weighted sum with the softmax weights (also split
// hi + lo) as A and the token chunk, staged in LDS and read transposed, as B.
// Partial scores of the 8 waves meet in LDS; every wave runs the same
// online-softmax update (fp32).  An fp32 FMA weighted sum would make the pass
// VALU-bound (wave64 fp32 FMA takes 4 cycles per instruction); on MFMA it is
// bound by the HBM read of the tokens.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace ivc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int FH = 16;  // heads per MFMA column block (fewer heads are zero-padded)
constexpr int FT = 16;  // tokens per chunk

bool pool_folded_supported(int dtype, int C, int H) {
  return dtype == DT_BF16 && (C == 512 || C == 1024) && H >= 1 && H <= FH && C % H == 0;
}

// part layout per (tile, split): [FH] running max, [FH] running sum, [FH][C] weighted sums
//
// 8 waves per workgroup, wave w owning channels [w*C/8, (w+1)*C/8); chunks of
// FT2 = 32 tokens.  Per chunk:
//   load     the 32 token rows, row-contiguously (1 KB per wave instruction),
//            into LDS; the next chunk's rows are loaded meanwhile;
//   scores   S[token][head] (two 16-token tiles) with the token rows (from
//            LDS) as the MFMA A operand and q~ (hi + lo) as B;
//   softmax  a lane (head h = lane % 16, token group g = lane / 16) takes
//            tokens 8g .. 8g+7 of head h: exactly the A-operand layout of the
//            next product, so P (split into bf16 hi + lo) stays in registers;
//   sum      xbar[h][c] += P[h][tokens] . X[tokens][c] on MFMA, the token
//            chunk staged in LDS and read transposed (8 tokens of a channel).
constexpr int FT2 = 32;

IVC_DEV bf16x8_t pack_bf16x8(const bf16_t* v) {
  u32x4 u;
  u.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  u.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
  u.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
  u.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

template <int C>
__global__ void __launch_bounds__(512, 2)
k_pool_folded(const bf16_t* __restrict__ X, int rows, int has_cls, const int* __restrict__ valid,
              int* status, int N, const bf16_t* __restrict__ qt_hi,
              const bf16_t* __restrict__ qt_lo, int splits, float* __restrict__ part) {
  constexpr int NW = 8;
  constexpr int CW = C / NW;     // channels per wave
  constexpr int KS = CW / 32;    // score MFMA k-steps per wave
  constexpr int NT = CW / 16;    // 16-channel output tiles per wave
  constexpr int LDX = C + 8;     // padded LDS row (bf16)

  __shared__ __attribute__((aligned(16))) bf16_t sX[FT2 * LDX];
  __shared__ float sS[NW][FT2][FH];

  const int t = blockIdx.x / splits, sp = blockIdx.x % splits;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lo16 = lane & 15, hi4 = lane >> 4;

  int nv = N;
  if (valid != nullptr) {
    nv = valid[t];
    if (nv < 1 || nv > N) {
      if (status != nullptr && sp == 0 && threadIdx.x == 0) atomicOr(status, 2);
      nv = nv < 1 ? 1 : N;
    }
  }
  const int per = (N + splits - 1) / splits;
  const int n_beg = sp * per;
  const int n_end = min(nv, n_beg + per);

  // q~ as B operand of the score product: head lo16, channels cw0 + 32k + 8*hi4 + 0..7
  const int cw0 = w * CW;
  bf16x8_t qh[KS], ql[KS];
  {
    const size_t qrow = ((size_t)t * FH + lo16) * C + cw0 + 8 * hi4;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qh[k] = *reinterpret_cast<const bf16x8_t*>(qt_hi + qrow + 32 * k);
      ql[k] = *reinterpret_cast<const bf16x8_t*>(qt_lo + qrow + 32 * k);
    }
  }

  // xbar accumulators: tile nt holds heads 4*hi4 + v, channel cw0 + 16*nt + lo16
  f32x4_t acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // head lo16 (lanes sharing lo16 agree)

  const bf16_t* xt = X + ((size_t)t * rows + has_cls) * C;
  // The chunk is loaded row-contiguously (a wave instruction covers 1 KB of
  // one token row): thread i takes 16 bytes at token i / VPR + r * RPL,
  // vector i % VPR, r = 0 .. LPT-1.  The next chunk is loaded while this one
  // is processed.
  constexpr int VPR = C / 8;               // 16-byte vectors per token row
  constexpr int RPL = 512 / VPR;           // token rows per 512-thread pass
  constexpr int LPT = FT2 / RPL;           // loads per thread per chunk
  const int lrow = threadIdx.x / VPR, lvec = threadIdx.x % VPR;
  u32x4 xg[LPT], xn[LPT];
  auto load_chunk = [&](int n0, u32x4 (&dst)[LPT]) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int n = n0 + lrow + r * RPL;
      dst[r] = n < n_end ? reinterpret_cast<const u32x4*>(xt + (size_t)n * C)[lvec]
                         : u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (n_beg < n_end) load_chunk(n_beg, xg);
  for (int n0 = n_beg; n0 < n_end; n0 += FT2) {
    if (n0 + FT2 < n_end) load_chunk(n0 + FT2, xn);
#pragma unroll
    for (int r = 0; r < LPT; ++r)
      *reinterpret_cast<u32x4*>(&sX[(lrow + r * RPL) * LDX + 8 * lvec]) = xg[r];
    __syncthreads();
    // partial scores over this wave's channels; A operand = token 16*tt + lo16,
    // channels cw0 + 32k + 8*hi4 (read from LDS); sc[v] = token 16*tt + 4*hi4 + v, head lo16
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &sX[(16 * tt + lo16) * LDX + cw0 + 32 * k + 8 * hi4]);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[k], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[k], sc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) sS[w][16 * tt + 4 * hi4 + v][lo16] = sc[v];
    }
    __syncthreads();

    // online softmax: head lo16, tokens 8*hi4 .. 8*hi4+7 (all waves alike)
    float sc8[8], cmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = 8 * hi4 + j;
      float z = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) z += sS[ww][tok][lo16];
      sc8[j] = (n0 + tok < n_end) ? z : -INFINITY;
      cmax = fmaxf(cmax, sc8[j]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const float corr = expf(m_run - m_new);
    float psum = 0.f;
    bf16_t ph[8], pl[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = expf(sc8[j] - m_new);
      psum += p;
      ph[j] = f32_to_bf16(p);
      pl[j] = f32_to_bf16(p - bf16_to_f32(ph[j]));
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * corr + psum;
    m_run = m_new;
    const bf16x8_t pah = pack_bf16x8(ph), pal = pack_bf16x8(pl);

    // rescale: accumulator row v of this lane is head 4*hi4 + v
    float cr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) cr[v] = __shfl(corr, 4 * hi4 + v, 64);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][v] *= cr[v];

    // xbar += P . X: B operand = tokens 8*hi4 .. +7 of channel cw0 + 16*nt + lo16
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bf16_t xb[8];
      const bf16_t* col = &sX[(8 * hi4) * LDX + cw0 + 16 * nt + lo16];
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[j] = col[j * LDX];
      const bf16x8_t b = pack_bf16x8(xb);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pah, b, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pal, b, acc[nt], 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < LPT; ++r) xg[r] = xn[r];
  }

  float* pp = part + ((size_t)t * splits + sp) * (size_t)(FH * (2 + C));
  if (w == 0 && hi4 == 0) {
    pp[lo16] = m_run;
    pp[FH + lo16] = l_run;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      pp[2 * FH + (size_t)(4 * hi4 + v) * C + cw0 + 16 * nt + lo16] = acc[nt][v];
}

// xbar[t][h][c] = sum_s acc_s e^{m_s - M} / sum_s l_s e^{m_s - M}
__global__ void __launch_bounds__(256)
k_pool_folded_merge(const float* __restrict__ part, int splits, int C, int H,
                    float* __restrict__ xbar) {
  const int t = blockIdx.x, h = blockIdx.y;
  const size_t stride = (size_t)FH * (2 + C);
  const float* pt = part + (size_t)t * splits * stride;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, pt[s * stride + h]);
  float L = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float ms = pt[s * stride + h];
    L += (ms == -INFINITY) ? 0.f : pt[s * stride + FH + h] * expf(ms - M);
  }
  const float invL = 1.0f / L;
  for (int c = threadIdx.x; c < C; c += 256) {
    float A = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float ms = pt[s * stride + h];
      if (ms != -INFINITY) A += pt[s * stride + 2 * FH + (size_t)h * C + c] * expf(ms - M);
    }
    xbar[((size_t)t * H + h) * C + c] = A * invL;
  }
}

hipError_t launch_pool_folded(const FoldedArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (!pool_folded_supported(a.dtype, a.C, a.H)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.T * a.splits));
  if (a.C == 1024)
    hipLaunchKernelGGL(k_pool_folded<1024>, grid, dim3(512), 0, s, (const bf16_t*)a.X, a.rows,
                       a.has_cls, a.valid, a.status, a.N, (const bf16_t*)a.qt_hi,
                       (const bf16_t*)a.qt_lo, a.splits, a.part);
  else
    hipLaunchKernelGGL(k_pool_folded<512>, grid, dim3(512), 0, s, (const bf16_t*)a.X, a.rows,
                       a.has_cls, a.valid, a.status, a.N, (const bf16_t*)a.qt_hi,
                       (const bf16_t*)a.qt_lo, a.splits, a.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_pool_folded_merge, dim3((unsigned)a.T, (unsigned)a.H), dim3(256), 0, s,
                     (const float*)a.part, a.splits, a.C, a.H, a.xbar);
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
