// Routing decision of the Visual Resolution Router.
//
// InternVL3_5-4B-Flash Gating and CrossAttentionPooling page, section 4, and
// the InternVL3_5-2B-Flash page's routing-decision section: the threshold is
// the 0.1-quantile of gate[:, 0] over the whole batch (linear interpolation
// between order statistics, as torch.quantile), and a tile takes the 64-token
// path only when gate[t, 0] > that quantile AND gate[t, 0] >= 0.5.
//
// One workgroup: the two order statistics come from an exact radix select
// (four 8-bit passes over order-preserving uint32 keys of the fp32 gates),
// the interpolation is done in fp64 with every operation rounded on its own
// (contraction into fused multiply-add is switched off), so the threshold and every decision are bit-identical
// to a host evaluation of the same formula on the same gates.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace ivc {

IVC_DEV uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
IVC_DEV float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

constexpr int QT = 1024;  // threads

// k-th smallest key (0-based) among the T gates.  Per pass: histogram of
// the next 8 key bits among the keys that match the prefix so far, then the
// 256 bins are scanned in parallel (4 waves) and the bin holding the k-th
// key extends the prefix.
IVC_DEV uint32_t radix_select(const float* gate, int T, int k, uint32_t* hist, uint32_t* sh,
                              uint32_t* wtot) {
  uint32_t prefix = 0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int pass = 3; pass >= 0; --pass) {
    const int shift = 8 * pass;
    const uint32_t mask = pass == 3 ? 0u : (0xffffffffu << (shift + 8));
    for (int i = threadIdx.x; i < 256; i += QT) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < T; i += QT) {
      const uint32_t key = order_key(gate[2 * i]);
      if ((key & mask) == (prefix & mask)) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    uint32_t h = 0, inc = 0;
    if (threadIdx.x < 256) {
      h = hist[threadIdx.x];
      inc = h;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(inc, o, 64);
        if (lane >= o) inc += v;
      }
      if (lane == 63) wtot[w] = inc;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      uint32_t before = 0;
      for (int q = 0; q < w; ++q) before += wtot[q];
      const uint32_t excl = before + inc - h;  // keys in lower bins
      if ((uint32_t)k >= excl && (uint32_t)k < excl + h) {
        sh[0] = prefix | ((uint32_t)threadIdx.x << shift);
        sh[1] = (uint32_t)k - excl;
      }
    }
    __syncthreads();
    prefix = sh[0];
    k = (int)sh[1];
    __syncthreads();
  }
  return prefix;
}

// Per-path tile lists of a decision (one workgroup of QT threads, chunked
// scan over tiles): rank[t] = t's index in its own path, list256 / list64 the
// tiles of each path in order, counts = (n256, n64).  u(t) gives tile t's
// decision (0 or 1).
template <typename U>
IVC_DEV void route_lists_block(int T, U u_of, int* __restrict__ rank, int* __restrict__ list256,
                               int* __restrict__ list64, int* __restrict__ counts) {
  __shared__ int wsum[16];
  __shared__ int carry_s;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int c0 = 0; c0 < T; c0 += QT) {
    const int t = c0 + threadIdx.x;
    const int u = t < T ? u_of(t) : 0;
    int inc = u;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int before = 0, tot = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < w) before += wsum[k];
      tot += wsum[k];
    }
    const int carry = carry_s;
    if (t < T) {
      const int r64 = carry + before + inc - u;  // routed tiles before t
      if (u) {
        rank[t] = r64;
        list64[r64] = t;
      } else {
        rank[t] = t - r64;
        list256[t - r64] = t;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) carry_s = carry + tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    counts[0] = T - carry_s;
    counts[1] = carry_s;
  }
}

__global__ void __launch_bounds__(1024)
k_route_lists(const uint8_t* __restrict__ use64, int T, int* __restrict__ rank,
              int* __restrict__ list256, int* __restrict__ list64, int* __restrict__ counts) {
  route_lists_block(T, [&](int t) { return use64[t] != 0 ? 1 : 0; }, rank, list256, list64,
                    counts);
}

// lists: also the per-path tile lists of the decision (rank != nullptr)
__global__ void __launch_bounds__(QT)
k_quantile_decide(const float* __restrict__ gate, int T, double q, double abs_thr,
                  double* __restrict__ thr_out, uint8_t* __restrict__ use64, int* __restrict__ rank,
                  int* __restrict__ list256, int* __restrict__ list64, int* __restrict__ counts) {
  // Every product and sum below is rounded on its own: HIP's __dmul_rn and
  // friends are plain operators that the compiler may fuse into an FMA, which
  // moves the threshold by an ulp, so plain operators with contraction off.
#pragma clang fp contract(off)
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wtot[4];

  const double pos = q * (double)(T - 1);
  const double fl = floor(pos);
  const int lo = (int)fl;
  const int hi = (int)ceil(pos);
  const double frac = pos - fl;

  const uint32_t klo = radix_select(gate, T, lo, hist, sh, wtot);
  // the next order statistic: equal to v[lo] if enough keys tie with it,
  // otherwise the smallest key above it
  if (threadIdx.x == 0) {
    sh[2] = 0;
    sh[3] = 0xffffffffu;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T; i += QT) {
    const uint32_t key = order_key(gate[2 * i]);
    if (key <= klo) atomicAdd(&sh[2], 1u);
    else atomicMin(&sh[3], key);
  }
  __syncthreads();
  const uint32_t khi = ((uint32_t)hi < sh[2]) ? klo : sh[3];

  const double a = (double)key_value(klo), b = (double)key_value(khi);
  const double diff = b - a;
  const double thr = frac < 0.5 ? a + diff * frac : b - diff * (1.0 - frac);
  if (threadIdx.x == 0) *thr_out = thr;
  auto decide = [&](int i) {
    const double g = (double)gate[2 * i];
    return (g > thr && g >= abs_thr) ? 1 : 0;
  };
  for (int i = threadIdx.x; i < T; i += QT) use64[i] = (uint8_t)decide(i);
  if (rank != nullptr) route_lists_block(T, decide, rank, list256, list64, counts);
}

hipError_t launch_route_lists(const uint8_t* use64, int T, int* rank, int* list256, int* list64,
                              int* counts, hipStream_t s) {
  hipLaunchKernelGGL(k_route_lists, dim3(1), dim3(QT), 0, s, use64, T, rank, list256, list64,
                     counts);
  return hipGetLastError();
}

hipError_t launch_quantile_decide(const float* gate, int T, double q, double abs_thr,
                                  double* thr, uint8_t* use64, hipStream_t s, int* rank,
                                  int* list256, int* list64, int* counts) {
  if (T == 0) return hipSuccess;
  if (rank != nullptr && (!list256 || !list64 || !counts)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quantile_decide, dim3(1), dim3(QT), 0, s, gate, T, q, abs_thr, thr, use64,
                     rank, list256, list64, counts);
  return hipGetLastError();
}

}  // namespace ivc
