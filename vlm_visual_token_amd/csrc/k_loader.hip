// Fused CLS drop + pixel_shuffle v2 + LayerNorm loader.
//
// pixel_shuffle v2 is a pure space-to-depth permutation of the P x P token
// grid (InternVL3-14B-Instruct pixel-shuffle page, pixel_shuffle section;
// InternVL3_5-2B-Flash page, three token levels):
//   out[a*(P/r) + b][(r*m + k)*C + c] = grid[r*a + m][r*b + k][c],
//   grid[i][j] = vit row has_cls + i*P + j.
// An r=2 token is 4 input rows of C (a 2x2 cell block); an r=4 token is the
// 4x4 block made of four r=2 blocks.  Two index-math variants:
//  * ps_version v1 (same page, v1/v2 section) leaves the two grid axes
//    swapped, so token (a, b) is written at b*(P/r) + a;
//  * the 64-token path as two successive r=2 shuffles (InternVL3_5-2B-Flash
//    page: scale 0.25 is 0.5 squared) puts cell (2*m2 + m, 2*k2 + k) of the
//    4x4 block in channel block 4*(2*m2 + k2) + (2*m + k) instead of the
//    direct r=4 block 4*(2*m2 + m) + (2*k2 + k).
// mlp1/mlp2 start with LayerNorm over the concatenated row (4C or 16C), fused
// here so the permuted rows are written once, already normalised, in the
// layout the projector GEMM reads.  In statistics mode (LayerNorm folded into
// the first product, which then reads the raw rows itself) only each row's
// mean and 1/sqrt(var + eps) are written.
//
// Work split (one wavefront = one r=2 token): the wave loads its 4 input rows
// with 16-byte loads (a row is C contiguous elements, so every load is fully
// coalesced), keeps them in registers, takes the r=2 statistics with two
// passes over the registers, and writes the normalised 4C row.  With the
// 64-token path on, a workgroup is the 4 waves of one r=4 block: they share
// their partial sums through LDS for the 16C statistics (again two passes)
// and each writes its 4 cells into the 16C row.  The ViT tensor is read
// exactly once for both paths.
#include "common.h"
#include "index_math.h"
#include "kernels.h"

namespace ivc {

template <typename E, int CPL, bool FLASH, bool LN, bool STATS>
__global__ void __launch_bounds__(256)
k_shuffle_ln(const E* __restrict__ X, int T, int P, int C, int has_cls,
             const float* __restrict__ g2, const float* __restrict__ b2, E* __restrict__ out2,
             const float* __restrict__ g4, const float* __restrict__ b4, E* __restrict__ out4,
             float eps, int ps_v1, int twice_r2, const uint8_t* __restrict__ use64,
             const int* __restrict__ rank, float* __restrict__ st2, float* __restrict__ st4) {
  static_assert(!STATS || LN, "statistics mode computes the LayerNorm statistics");
  constexpr int V = Elem<E>::kPerVec;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rows = has_cls + P * P;
  const int Q2 = P >> 1, S2 = Q2 * Q2;
  const int vpr = C / V;  // 16-byte vectors per input row

  int t, a2, b2i, a4 = 0, b4i = 0;
  if (FLASH) {
    const int Q4 = P >> 2, S4 = Q4 * Q4;
    const int blk = blockIdx.x;
    t = blk / S4;
    const int rem = blk - t * S4;
    a4 = rem / Q4;
    b4i = rem - a4 * Q4;
    a2 = 2 * a4 + (w >> 1);
    b2i = 2 * b4i + (w & 1);
  } else {
    const int tok = blockIdx.x * 4 + w;
    if (tok >= T * S2) return;  // whole wave leaves; no barrier in this variant
    t = tok / S2;
    const int rem = tok - t * S2;
    a2 = rem / Q2;
    b2i = rem - a2 * Q2;
  }

  // ---- load the 2x2 cell block: cell q = 2m + k is grid (2*a2 + m, 2*b2 + k)
  u32x4 raw[4][CPL];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int gi = 2 * a2 + (q >> 1), gj = 2 * b2i + (q & 1);
    const u32x4* src =
        reinterpret_cast<const u32x4*>(X + ((size_t)t * rows + ps_cell_row(P, has_cls, gi, gj)) * C);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int v = lane + 64 * i;
      raw[q][i] = (v < vpr) ? __builtin_nontemporal_load(src + v) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float mean2 = 0.f, rstd2 = 1.f, mean4 = 0.f, rstd4 = 1.f;
  if (LN) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        if (lane + 64 * i < vpr) {
          float f[V];
          unpack<E>(raw[q][i], f);
#pragma unroll
          for (int e = 0; e < V; ++e) s += f[e];
        }
      }
    const float s2 = wave_sum(s);
    mean2 = s2 / (float)(4 * C);
    float d2 = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        if (lane + 64 * i < vpr) {
          float f[V];
          unpack<E>(raw[q][i], f);
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const float d = f[e] - mean2;
            d2 += d * d;
          }
        }
      }
    rstd2 = 1.0f / sqrtf(wave_sum(d2) / (float)(4 * C) + eps);

    if (FLASH) {
      __shared__ float red[2][4];
      if (lane == 0) red[0][w] = s2;
      __syncthreads();
      mean4 = (red[0][0] + red[0][1] + red[0][2] + red[0][3]) / (float)(16 * C);
      float d4 = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          if (lane + 64 * i < vpr) {
            float f[V];
            unpack<E>(raw[q][i], f);
#pragma unroll
            for (int e = 0; e < V; ++e) {
              const float d = f[e] - mean4;
              d4 += d * d;
            }
          }
        }
      d4 = wave_sum(d4);
      if (lane == 0) red[1][w] = d4;
      __syncthreads();
      rstd4 = 1.0f / sqrtf((red[1][0] + red[1][1] + red[1][2] + red[1][3]) / (float)(16 * C) + eps);
    }
  }

  // route-first: only the tile's chosen path is written, at its rank in that path
  bool want2 = (STATS ? (void*)st2 : (void*)out2) != nullptr;
  bool want4 = (STATS ? (void*)st4 : (void*)out4) != nullptr;
  int t2 = t, t4 = t;
  if (use64 != nullptr) {
    const bool to64 = use64[t] != 0;
    want2 = want2 && !to64;
    want4 = want4 && to64;
    t2 = t4 = rank[t];
  }

  if (STATS) {
    if (want2 && lane == 0) {
      const int tok2 = ps_token(Q2, a2, b2i, ps_v1);
      *reinterpret_cast<float2*>(st2 + 2 * ((size_t)t2 * S2 + tok2)) = make_float2(mean2, rstd2);
    }
    if (FLASH && want4 && threadIdx.x == 0) {
      const int Q4 = P >> 2, S4 = Q4 * Q4;
      const int tok4 = ps_token(Q4, a4, b4i, ps_v1);
      *reinterpret_cast<float2*>(st4 + 2 * ((size_t)t4 * S4 + tok4)) = make_float2(mean4, rstd4);
    }
    return;
  }

  // ---- r = 2 row: channel block q holds cell q
  if (want2) {
    const int tok2 = ps_token(Q2, a2, b2i, ps_v1);
    E* dst = out2 + ((size_t)t2 * S2 + tok2) * (size_t)(4 * C);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int v = lane + 64 * i;
        if (v < vpr) {
          const int ch = q * C + v * V;
          u32x4 o = raw[q][i];
          if (LN) {
            float f[V];
            unpack<E>(raw[q][i], f);
#pragma unroll
            for (int e = 0; e < V; ++e) f[e] = (f[e] - mean2) * rstd2 * g2[ch + e] + b2[ch + e];
            o = pack<E>(f);
          }
          *reinterpret_cast<u32x4*>(dst + ch) = o;
        }
      }
  }

  // ---- r = 4 row: this wave's cell q = (m, k) sits at (2*(w>>1) + m, 2*(w&1) + k)
  //      inside the 4x4 block: channel block 4*m4 + k4 (direct) or 4*w + q
  //      (two r=2 shuffles).
  if (FLASH && want4) {
    const int Q4 = P >> 2, S4 = Q4 * Q4;
    const int tok4 = ps_token(Q4, a4, b4i, ps_v1);
    E* dst = out4 + ((size_t)t4 * S4 + tok4) * (size_t)(16 * C);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int base = ps64_channel_block(w, q, twice_r2) * C;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int v = lane + 64 * i;
        if (v < vpr) {
          const int ch = base + v * V;
          u32x4 o = raw[q][i];
          if (LN) {
            float f[V];
            unpack<E>(raw[q][i], f);
#pragma unroll
            for (int e = 0; e < V; ++e) f[e] = (f[e] - mean4) * rstd4 * g4[ch + e] + b4[ch + e];
            o = pack<E>(f);
          }
          *reinterpret_cast<u32x4*>(dst + ch) = o;
        }
      }
    }
  }
}

template <typename E, int CPL, bool LN, bool STATS>
static hipError_t launch_cpl(const ShuffleArgs& a, hipStream_t s) {
  const int Q2 = a.P / 2, Q4 = a.P / 4;
  if (a.flash) {
    dim3 grid((unsigned)(a.T * Q4 * Q4));
    hipLaunchKernelGGL((k_shuffle_ln<E, CPL, true, LN, STATS>), grid, dim3(256), 0, s, (const E*)a.X, a.T,
                       a.P, a.C, a.has_cls, a.g2, a.b2, (E*)a.out2, a.g4, a.b4, (E*)a.out4, a.eps,
                       a.ps_v1, a.twice_r2, a.use64, a.rank, a.st2, a.st4);
  } else {
    const long long toks = (long long)a.T * Q2 * Q2;
    dim3 grid((unsigned)((toks + 3) / 4));
    hipLaunchKernelGGL((k_shuffle_ln<E, CPL, false, LN, STATS>), grid, dim3(256), 0, s, (const E*)a.X,
                       a.T, a.P, a.C, a.has_cls, a.g2, a.b2, (E*)a.out2, a.g4, a.b4, (E*)a.out4,
                       a.eps, a.ps_v1, a.twice_r2, a.use64, a.rank, a.st2, a.st4);
  }
  return hipGetLastError();
}

template <typename E, bool LN, bool STATS>
static hipError_t launch_e(const ShuffleArgs& a, hipStream_t s) {
  const int vpr = a.C / Elem<E>::kPerVec;
  const int need = (vpr + 63) / 64;
  if (need <= 1) return launch_cpl<E, 1, LN, STATS>(a, s);
  if (need <= 2) return launch_cpl<E, 2, LN, STATS>(a, s);
  if (need <= 4) return launch_cpl<E, 4, LN, STATS>(a, s);
  if (need <= 8) return launch_cpl<E, 8, LN, STATS>(a, s);
  return hipErrorInvalidValue;
}

// LayerNorm statistics of the shuffled rows from the per-token moments
// tokst[t * N + n] = (mean, M2) of each grid cell's C channels: an r = 2 row
// is a 2 x 2 cell block, an r = 4 row the 4 x 4 block of four of them
// (whatever order the channel blocks take inside the row), combined
// pairwise: the two cells of a grid row, then the two rows; the four 2 x 2
// blocks likewise.  st2 / st4 get (mean, 1 / sqrt(M2 / n + eps)), n = 4C or
// 16C, at the row the projector reads (route-first: the tile's rank in its
// path, the other path skipped).  One thread per r = 2 row, then one per
// r = 4 row.
IVC_DEV float2 block2_moments(const float2* __restrict__ ts, int P, int gi, int gj, float C) {
  const float2* c0 = ts + (size_t)gi * P + gj;
  const float2 top = moments_pair(c0[0], c0[1], 0.5f * C);
  const float2 bot = moments_pair(c0[P], c0[P + 1], 0.5f * C);
  return moments_pair(top, bot, C);
}

__global__ void __launch_bounds__(256)
k_ln_stats(const float2* __restrict__ tokst, int T, int P, int C, float eps, int ps_v1, int flash,
           const uint8_t* __restrict__ use64, const int* __restrict__ rank,
           float* __restrict__ st2, float* __restrict__ st4) {
  const int Q2 = P / 2, S2 = Q2 * Q2, Q4 = P / 4, S4 = flash ? Q4 * Q4 : 0;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n2 = (long long)T * S2;
  const int N = P * P;
  if (i < n2) {
    const int t = (int)(i / S2), s = (int)(i - (long long)t * S2);
    if (st2 == nullptr || (use64 != nullptr && use64[t] != 0)) return;
    const int a = s / Q2, b = s - a * Q2;  // token (a, b) of the direct order
    const float2 mo = block2_moments(tokst + (size_t)t * N, P, 2 * a, 2 * b, (float)C);
    const int t2 = use64 != nullptr ? rank[t] : t;
    const int tok = ps_token(Q2, a, b, ps_v1);
    *reinterpret_cast<float2*>(st2 + 2 * ((size_t)t2 * S2 + tok)) =
        make_float2(mo.x, 1.0f / sqrtf(mo.y / (float)(4 * C) + eps));
    return;
  }
  const long long i4 = i - n2;
  if (i4 >= (long long)T * S4) return;
  const int t = (int)(i4 / S4), s = (int)(i4 - (long long)t * S4);
  if (st4 == nullptr || (use64 != nullptr && use64[t] == 0)) return;
  const int a = s / Q4, b = s - a * Q4;
  const float2* ts = tokst + (size_t)t * N;
  const float fc = (float)C;
  const float2 b00 = block2_moments(ts, P, 4 * a, 4 * b, fc);
  const float2 b01 = block2_moments(ts, P, 4 * a, 4 * b + 2, fc);
  const float2 b10 = block2_moments(ts, P, 4 * a + 2, 4 * b, fc);
  const float2 b11 = block2_moments(ts, P, 4 * a + 2, 4 * b + 2, fc);
  const float2 mo = moments_pair(moments_pair(b00, b01, 2.f * fc), moments_pair(b10, b11, 2.f * fc),
                                 4.f * fc);
  const int t4 = use64 != nullptr ? rank[t] : t;
  const int tok = ps_token(Q4, a, b, ps_v1);
  *reinterpret_cast<float2*>(st4 + 2 * ((size_t)t4 * S4 + tok)) =
      make_float2(mo.x, 1.0f / sqrtf(mo.y / (float)(16 * C) + eps));
}

hipError_t launch_ln_stats(const float* tokst, int T, int P, int C, float eps, int ps_v1,
                           int flash, const uint8_t* use64, const int* rank, float* st2,
                           float* st4, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (!tokst || P % (flash ? 4 : 2) || (use64 != nullptr && rank == nullptr)) return hipErrorInvalidValue;
  const long long n = (long long)T * ((P / 2) * (P / 2) + (flash ? (P / 4) * (P / 4) : 0));
  hipLaunchKernelGGL(k_ln_stats, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const float2*)tokst, T, P, C, eps, ps_v1, flash, use64, rank, st2, st4);
  return hipGetLastError();
}

int shuffle_max_width(int dtype) { return 8 * 64 * (dtype == 1 ? 8 : 4); }

hipError_t launch_shuffle_ln(const ShuffleArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.st2 != nullptr || a.st4 != nullptr) {  // statistics only (bf16: the folded products)
    if (a.dtype != 1 || !a.ln) return hipErrorInvalidValue;
    return launch_e<bf16_t, true, true>(a, s);
  }
  if (a.dtype == 1)
    return a.ln ? launch_e<bf16_t, true, false>(a, s) : launch_e<bf16_t, false, false>(a, s);
  return a.ln ? launch_e<float, true, false>(a, s) : launch_e<float, false, false>(a, s);
}

}  // namespace ivc
