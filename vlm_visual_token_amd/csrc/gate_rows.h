// Residual LayerNorm of one Gating row and, for the last block, the 2-way
// classifier head (InternVL3_5-4B-Flash Gating and CrossAttentionPooling
// page, section 3): x = x + LN(y) * gamma + beta over the h values of row t,
// then z_j = bc_j + sum_i Wc[j, i] x_i and softmax(z) in fp64 to gate[t].
// Shared by the per-block kernel and the one-launch Gating kernel, so both
// do the same arithmetic in the same order.
#pragma once

#include "common.h"

#include <math.h>

namespace ivc {

// The first 256 threads of the workgroup do the work (h <= 4096: 16 values
// each, two-pass statistics from registers); any further threads only take
// part in the barriers.
template <bool HEAD, typename E>
IVC_DEV void residual_ln_row(int t, float* __restrict__ x, const float* __restrict__ y,
                             const float* __restrict__ g, const float* __restrict__ b, int h,
                             float eps, const E* __restrict__ Wc, const float* __restrict__ bc,
                             float* __restrict__ gate) {
  constexpr int MAXE = 16;
  const bool on = threadIdx.x < 256;
  const float* yr = y + (long long)t * h;
  float* xr = x + (long long)t * h;
  float v[MAXE];
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + 256 * e;
    v[e] = on && i < h ? yr[i] : 0.f;
    s += v[e];
  }
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  s = wave_sum(s);
  if (lane == 0 && w < 4) red[w] = s;
  __syncthreads();
  const float mean = (red[0] + red[1] + red[2] + red[3]) / (float)h;
  __syncthreads();
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + 256 * e;
    if (on && i < h) {
      const float dd = v[e] - mean;
      q += dd * dd;
    }
  }
  q = wave_sum(q);
  if (lane == 0 && w < 4) red[w] = q;
  __syncthreads();
  const float rstd = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)h + eps);
  float z0 = 0.f, z1 = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + 256 * e;
    if (on && i < h) {
      const float xn = xr[i] + (v[e] - mean) * rstd * g[i] + b[i];
      xr[i] = xn;
      if (HEAD) {
        z0 = fmaf(Elem<E>::to_f(Wc[i]), xn, z0);
        z1 = fmaf(Elem<E>::to_f(Wc[h + i]), xn, z1);
      }
    }
  }
  if (HEAD) {
    __shared__ float rz[2][4];
    z0 = wave_sum(z0);
    z1 = wave_sum(z1);
    if (lane == 0 && w < 4) {
      rz[0][w] = z0;
      rz[1][w] = z1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const double a = (double)((rz[0][0] + rz[0][1]) + (rz[0][2] + rz[0][3])) + bc[0];
      const double c = (double)((rz[1][0] + rz[1][1]) + (rz[1][2] + rz[1][3])) + bc[1];
      const double mx = a > c ? a : c;
      const double e0 = exp(a - mx), e1 = exp(c - mx);
      gate[2 * t] = (float)(e0 / (e0 + e1));
      gate[2 * t + 1] = (float)(e1 / (e0 + e1));
    }
  }
}

}  // namespace ivc
