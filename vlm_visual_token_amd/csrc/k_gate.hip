// Gating network helpers (InternVL3_5-4B-Flash Gating and CrossAttentionPooling
// page, section 3): four residual blocks whose last step is a LayerNorm that
// is added back onto the block input, then a 2-way classifier and softmax.
// The block's two Linears run on the router product kernels; these kernels
// do the residual LayerNorm and (fused into the last block's) the classifier
// head, in fp32 with the 2-way softmax in fp64.
#include "common.h"
#include "gate_rows.h"
#include "kernels.h"

#include <math.h>

namespace ivc {

// One workgroup of 256 threads per row.  HEAD: the last block also applies
// the classifier to the updated row and writes softmax(z) to gate, saving
// the separate head launch.
template <bool HEAD, typename E>
__global__ void __launch_bounds__(256)
k_residual_ln(float* __restrict__ x, const float* __restrict__ y, const float* __restrict__ g,
              const float* __restrict__ b, int h, float eps, const E* __restrict__ Wc,
              const float* __restrict__ bc, float* __restrict__ gate) {
  residual_ln_row<HEAD, E>(blockIdx.x, x, y, g, b, h, eps, Wc, bc, gate);
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
