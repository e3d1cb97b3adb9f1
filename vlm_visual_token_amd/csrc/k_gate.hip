// Gating network helpers (InternVL3_5-4B-Flash Gating and CrossAttentionPooling
// page, section 3): four residual blocks whose last step is a LayerNorm that
// is added back onto the block input, then a 2-way classifier and softmax.
// The block's two Linears run on the router product kernels; these kernels
// do the residual LayerNorm and (fused into the last block's) the classifier
// head, in fp32 with the 2-way softmax in fp64.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace ivc {

// One workgroup per row.  Two-pass statistics from registers (h <= 4096).
// HEAD: the last block also applies the classifier to the updated row,
// z_j = bc_j + sum_i Wc[j, i] x_i (j = 0, 1), and writes softmax(z) (fp64)
// to gate, saving the separate head launch.
template <bool HEAD, typename E>
__global__ void __launch_bounds__(256)
k_residual_ln(float* __restrict__ x, const float* __restrict__ y, const float* __restrict__ g,
              const float* __restrict__ b, int h, float eps, const E* __restrict__ Wc,
              const float* __restrict__ bc, float* __restrict__ gate) {
  constexpr int MAXE = 16;
  const int t = blockIdx.x;
  const float* yr = y + (long long)t * h;
  float* xr = x + (long long)t * h;
  float v[MAXE];
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + 256 * e;
    v[e] = i < h ? yr[i] : 0.f;
    s += v[e];
  }
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  s = wave_sum(s);
  if (lane == 0) red[w] = s;
  __syncthreads();
  const float mean = (red[0] + red[1] + red[2] + red[3]) / (float)h;
  __syncthreads();
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + 256 * e;
    if (i < h) {
      const float dd = v[e] - mean;
      q += dd * dd;
    }
  }
  q = wave_sum(q);
  if (lane == 0) red[w] = q;
  __syncthreads();
  const float rstd = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)h + eps);
  float z0 = 0.f, z1 = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + 256 * e;
    if (i < h) {
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
    if (lane == 0) {
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

hipError_t launch_residual_ln(float* x, const float* y, const float* gamma, const float* beta,
                              int T, int h, float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (h > 4096) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_residual_ln<false, float>), dim3((unsigned)T), dim3(256), 0, s, x, y,
                     gamma, beta, h, eps, (const float*)nullptr, (const float*)nullptr,
                     (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_residual_ln_head(int dtype, float* x, const float* y, const float* gamma,
                                   const float* beta, int T, int h, float eps, const void* Wc,
                                   const float* bc, float* gate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (h > 4096) return hipErrorInvalidValue;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL((k_residual_ln<true, bf16_t>), dim3((unsigned)T), dim3(256), 0, s, x, y,
                       gamma, beta, h, eps, (const bf16_t*)Wc, bc, gate);
  else
    hipLaunchKernelGGL((k_residual_ln<true, float>), dim3((unsigned)T), dim3(256), 0, s, x, y,
                       gamma, beta, h, eps, (const float*)Wc, bc, gate);
  return hipGetLastError();
}

template <typename E>
__global__ void k_broadcast_rows(const E* __restrict__ v, float* __restrict__ out, int T, int C) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (long long)T * C) out[i] = Elem<E>::to_f(v[i % C]);
}

hipError_t launch_broadcast_rows(int dtype, const void* v, float* out, int T, int C,
                                 hipStream_t s) {
  const long long n = (long long)T * C;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_broadcast_rows<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)v, out, T, C);
  else
    hipLaunchKernelGGL(k_broadcast_rows<float>, grid, dim3(256), 0, s, (const float*)v, out, T, C);
  return hipGetLastError();
}

}  // namespace ivc
