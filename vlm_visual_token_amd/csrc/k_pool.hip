// CrossAttentionPooling, K/V form: one query per tile per head attends over
// the tile's projected keys and values (InternVL3_5-4B-Flash Gating and
// CrossAttentionPooling page, section 2: a learnable query reads all of a
// tile's tokens through multi-head cross-attention, padded tokens masked).
//
// K and V of all layers come from one MFMA GEMM over the ViT rows; this
// kernel does the attention of one layer.  A single query makes it a pure
// streaming pass over K and V: each workgroup takes a contiguous token range
// of one tile (the tile is split so the grid covers the chip), each wave a
// quarter of that range.  A lane owns C/64 consecutive channels, so a head of
// d channels is d/(C/64) neighbouring lanes and a score is a partial dot
// product plus a few xor-shuffles.  Softmax is online (running max and sum,
// fp32), and padded tokens are never loaded: the loop bound is the tile's
// valid count, so garbage or NaN in padding cannot reach the result.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace ivc {

bool pool_attn_supported(int C, int H) {
  if (C % 64 != 0 || H <= 0 || C % H != 0) return false;
  const int cpl = C / 64, d = C / H;
  if (cpl > 64 || d % cpl != 0) return false;
  const int lph = d / cpl;  // lanes per head
  return lph >= 1 && lph <= 64 && (lph & (lph - 1)) == 0;
}

template <typename E, int CPL>
IVC_DEV void load_chunk(const E* p, float* f) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) f[i] = Elem<E>::to_f(p[i]);
}
template <>
IVC_DEV void load_chunk<bf16_t, 16>(const bf16_t* p, float* f) {
  const u32x4* v = reinterpret_cast<const u32x4*>(p);
  unpack<bf16_t>(v[0], f);
  unpack<bf16_t>(v[1], f + 8);
}
template <>
IVC_DEV void load_chunk<bf16_t, 8>(const bf16_t* p, float* f) {
  unpack<bf16_t>(*reinterpret_cast<const u32x4*>(p), f);
}

// part layout per (tile, split): [2*H] (max, sum) per head, then [C] weighted V sums.
template <typename E, int CPL, int UNR>
__global__ void __launch_bounds__(256)
k_pool_attn(const E* __restrict__ KV, long long kv_ld, int kcol, int vcol,
            const float* __restrict__ Q, const int* __restrict__ valid, int* status, int N, int C,
            int H, int splits, float* __restrict__ part, float* __restrict__ O) {
  const int t = blockIdx.x / splits, sp = blockIdx.x % splits;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = C / H;
  const int lph = d / CPL;
  const int c0 = lane * CPL;

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

  const float scale = 1.0f / sqrtf((float)d);
  float q[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) q[i] = Q[(long long)t * C + c0 + i] * scale;

  float m = -INFINITY, l = 0.f, acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;

  const E* base = KV + (long long)t * N * kv_ld;
  // this wave's tokens: n_beg + w, n_beg + w + 4, ...
  for (int n = n_beg + w; n < n_end; n += 4 * UNR) {
    float kf[UNR][CPL], vf[UNR][CPL];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int nn = n + 4 * u;
      if (nn < n_end) {
        const E* row = base + (long long)nn * kv_ld;
        load_chunk<E, CPL>(row + kcol + c0, kf[u]);
        load_chunk<E, CPL>(row + vcol + c0, vf[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int nn = n + 4 * u;
      if (nn >= n_end) break;  // uniform across the wave
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) s = fmaf(q[i], kf[u][i], s);
      for (int o = lph >> 1; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
      const float mn = fmaxf(m, s);
      const float corr = expf(m - mn);  // m = -inf on the first token gives 0
      const float p = expf(s - mn);
      l = l * corr + p;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] = fmaf(p, vf[u][i], acc[i] * corr);
      m = mn;
    }
  }

  // merge the 4 waves
  __shared__ float s_ml[4][2][64];
  __shared__ float s_acc[4][64 * CPL];
  const int h_lane = c0 / d;  // head of this lane
  if ((lane % lph) == 0) {
    s_ml[w][0][h_lane] = m;
    s_ml[w][1][h_lane] = l;
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) s_acc[w][c0 + i] = acc[i];
  __syncthreads();

  float* pp = part + ((long long)t * splits + sp) * (2 * H + C);
  for (int c = threadIdx.x; c < C; c += 256) {
    const int h = c / d;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_ml[ww][0][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = s_ml[ww][0][h];
      const float f = (mw == -INFINITY) ? 0.f : expf(mw - M);
      L += s_ml[ww][1][h] * f;
      A += s_acc[ww][c] * f;
    }
    if (splits == 1) {
      O[(long long)t * C + c] = A / L;
    } else {
      pp[2 * H + c] = A;
      if (c % d == 0) {
        pp[2 * h] = M;
        pp[2 * h + 1] = L;
      }
    }
  }
}

// Merge the token splits of each tile: O = sum_s A_s e^{M_s - M} / sum_s L_s e^{M_s - M}.
__global__ void __launch_bounds__(256)
k_pool_merge(const float* __restrict__ part, int splits, int C, int H, float* __restrict__ O) {
  const int t = blockIdx.x;
  const int d = C / H;
  for (int c = threadIdx.x; c < C; c += 256) {
    const int h = c / d;
    const float* pt = part + (long long)t * splits * (2 * H + C);
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, pt[(long long)s * (2 * H + C) + 2 * h]);
    float L = 0.f, A = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float* ps = pt + (long long)s * (2 * H + C);
      const float ms = ps[2 * h];
      const float f = (ms == -INFINITY) ? 0.f : expf(ms - M);
      L += ps[2 * h + 1] * f;
      A += ps[2 * H + c] * f;
    }
    O[(long long)t * C + c] = A / L;
  }
}

template <typename E, int CPL>
static hipError_t launch_attn_t(const PoolAttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.T * a.splits));
  hipLaunchKernelGGL((k_pool_attn<E, CPL, 4>), grid, dim3(256), 0, s, (const E*)a.KV, a.kv_ld,
                     a.kcol, a.vcol, a.Q, a.valid, a.status, a.N, a.C, a.H, a.splits, a.part,
                     a.O);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(k_pool_merge, dim3((unsigned)a.T), dim3(256), 0, s, (const float*)a.part,
                     a.splits, a.C, a.H, a.O);
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_attn_e(const PoolAttnArgs& a, hipStream_t s) {
  switch (a.C / 64) {
    case 1: return launch_attn_t<E, 1>(a, s);
    case 2: return launch_attn_t<E, 2>(a, s);
    case 4: return launch_attn_t<E, 4>(a, s);
    case 8: return launch_attn_t<E, 8>(a, s);
    case 16: return launch_attn_t<E, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pool_attn(const PoolAttnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (!pool_attn_supported(a.C, a.H)) return hipErrorInvalidValue;
  return a.dtype == DT_BF16 ? launch_attn_e<bf16_t>(a, s) : launch_attn_e<float>(a, s);
}

}  // namespace ivc
