// Small products with fp32 activations and bf16 weights on MFMA:
//   C[M, N] = act(A[M, K] . W[N, K]^T + bias[N])      (optionally batched)
// as used by the router (query / output projections of CrossAttentionPooling,
// the value fold, the Gating blocks) and the query fold.  M is the number of
// tiles (a few hundred), N and K about 1e3: too little work for large tiles,
// and an fp32 SIMT product is bound by the 4-cycle wave64 FMA.
//
// Each activation is split into bf16 high and low parts, x = hi + lo with
// |x - hi - lo| <= 2^-17 |x|; the bf16 weights are exact, so the two products
// hi.W + lo.W on v_mfma_f32_16x16x32_bf16 (fp32 accumulation) give close to
// fp32 accuracy.
//
// Workgroup: 8 waves, output tile 16 x 64.  The waves share the tile and take
// interleaved 32-wide K steps (wave w: steps w, w+8, ...), each loading the
// operands of up to 4 steps at once straight from global memory (the
// activation rows are L2-resident), so a product of K = 1024 waits for one
// round of load latency; then the eight partial tiles are added in a fixed
// order through LDS: results do not depend on timing.
#include "common.h"
#include "kernels.h"

namespace ivc {

namespace {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));


IVC_DEV uint32_t cvt_pk(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// 8 fp32 values -> bf16 high parts and the bf16 rounding of what they leave
IVC_DEV void split8(const float4& x0, const float4& x1, bf16x8_t& hi, bf16x8_t& lo) {
  u32x4 h, l;
  h.x = cvt_pk(x0.x, x0.y);
  h.y = cvt_pk(x0.z, x0.w);
  h.z = cvt_pk(x1.x, x1.y);
  h.w = cvt_pk(x1.z, x1.w);
  l.x = cvt_pk(x0.x - __uint_as_float(h.x << 16), x0.y - __uint_as_float(h.x & 0xffff0000u));
  l.y = cvt_pk(x0.z - __uint_as_float(h.y << 16), x0.w - __uint_as_float(h.y & 0xffff0000u));
  l.z = cvt_pk(x1.x - __uint_as_float(h.z << 16), x1.y - __uint_as_float(h.z & 0xffff0000u));
  l.w = cvt_pk(x1.z - __uint_as_float(h.w << 16), x1.w - __uint_as_float(h.w & 0xffff0000u));
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}
}  // namespace

// Tile (16 MB) x (16 NB), NWV waves, PD K steps loaded per wave at once.
// OUT: 0 = fp32 C, 1 = C * scale as bf16 high part (Cm) and low part (C2)
template <int MB, int NB, int NWV, int PD, int ACT, int OUT>
__global__ void __launch_bounds__(NWV * 64)
k_gemm_f32a(const float* __restrict__ A, long long lda, long long a_bs,
            const bf16_t* __restrict__ W, long long ldw, long long w_bs,
            const float* __restrict__ bias, long long bias_bs, void* __restrict__ Cm,
            void* __restrict__ C2, long long ldc, long long c_bs, int M, int N, int K,
            float scale) {
  constexpr int BM = 16 * MB, BN = 16 * NB, LDR = BN + 4;
  constexpr int NTH = NWV * 64, RPP = NTH / BN;  // epilogue rows per pass
  static_assert(NTH % BN == 0 && BM % RPP == 0, "epilogue shape");
  __shared__ __attribute__((aligned(16))) float red[NWV][BM][LDR];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lo16 = lane & 15, hi4 = lane >> 4;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM, b = blockIdx.z;
  A += b * a_bs;
  W += b * w_bs;

  // operand rows of this lane (clamped: rows past M or N are computed, not stored)
  const float* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    arow[mb] = A + (long long)min(m0 + 16 * mb + lo16, M - 1) * lda + 8 * hi4;
  const bf16_t* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    wrow[nb] = W + (long long)min(n0 + 16 * nb + lo16, N - 1) * ldw + 8 * hi4;

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // wave w takes K steps w, w + NWV, ...; up to PD of them are loaded at once
  const int nks = K / 32;
  for (int s0 = w; s0 < nks; s0 += NWV * PD) {
    float4 xa[PD][MB][2];
    u32x4 xw[PD][NB];
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      const int k0 = 32 * min(s0 + NWV * i, nks - 1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        xa[i][mb][0] = *reinterpret_cast<const float4*>(arow[mb] + k0);
        xa[i][mb][1] = *reinterpret_cast<const float4*>(arow[mb] + k0 + 4);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) xw[i][nb] = *reinterpret_cast<const u32x4*>(wrow[nb] + k0);
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads of the group go out first
    // no branch between the loads and their use (it would let the compiler
    // sink the later loads behind the earlier products): a step past the end
    // runs on a zeroed activation
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      const float keep = s0 + NWV * i < nks ? 1.f : 0.f;
      bf16x8_t ah[MB], al[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float4 x0 = xa[i][mb][0], x1 = xa[i][mb][1];
        x0.x *= keep; x0.y *= keep; x0.z *= keep; x0.w *= keep;
        x1.x *= keep; x1.y *= keep; x1.z *= keep; x1.w *= keep;
        split8(x0, x1, ah[mb], al[mb]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, xw[i][nb]);
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[mb], bw, acc[mb][nb], 0, 0, 0);
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[mb], bw, acc[mb][nb], 0, 0, 0);
        }
    }
  }

  // partial tiles -> LDS; output layout: lane holds column 16nb + lo16, rows 16mb + 4hi4 + v
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][16 * mb + 4 * hi4 + v][16 * nb + lo16] = acc[mb][nb][v];
  __syncthreads();

  const int col = threadIdx.x % BN;
  const int n = n0 + col;
  if (n >= N) return;
  const float bj = bias != nullptr ? bias[b * bias_bs + n] : 0.f;
#pragma unroll
  for (int i = 0; i < BM / RPP; ++i) {
    const int r = (int)(threadIdx.x / BN) + RPP * i;
    const int m = m0 + r;
    if (m >= M) break;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) v += red[ww][r][col];
    v += bj;
    if (ACT == ACT_GELU) v = gelu_erf(v);
    const long long o = b * c_bs + (long long)m * ldc + n;
    if (OUT == 0) {
      reinterpret_cast<float*>(Cm)[o] = v;
    } else {
      v *= scale;
      const bf16_t h = f32_to_bf16(v);
      reinterpret_cast<bf16_t*>(Cm)[o] = h;
      reinterpret_cast<bf16_t*>(C2)[o] = f32_to_bf16(v - bf16_to_f32(h));
    }
  }
}

bool gemm_f32a_supported(const GemmArgs& g) {
  const long long bs_a = g.batch > 1 ? g.a_bs : 0, bs_w = g.batch > 1 ? g.w_bs : 0;
  return g.a_dtype == DT_F32 && g.w_dtype == DT_BF16 && g.M > 0 && g.N > 0 && g.K > 0 &&
         g.K % 32 == 0 && g.a_rpg == 0 && g.rm.m_dev == nullptr && g.rm.c_map == nullptr &&
         g.lda % 4 == 0 && bs_a % 4 == 0 && ((uintptr_t)g.A % 16) == 0 && g.ldw % 8 == 0 &&
         bs_w % 8 == 0 && ((uintptr_t)g.W % 16) == 0 && g.batch <= 65535 &&
         (g.M + 15) / 16 <= 65535;
}

hipError_t launch_gemm_f32a(const GemmArgs& g, int out_split, void* C2, float scale,
                            hipStream_t s) {
  if (!gemm_f32a_supported(g)) return hipErrorInvalidValue;
  if (out_split ? g.c_dtype != DT_BF16 || C2 == nullptr : g.c_dtype != DT_F32)
    return hipErrorInvalidValue;
  const int batch = g.batch > 1 ? g.batch : 1;
  // 16 x 64 tiles; long K: 8 waves of 4 K steps each; short K (the query
  // fold, K = head width): 2 waves of one step
  const bool longk = g.K >= 256;
  const int BM = 16, BN = 64;
  dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM), (unsigned)batch);
#define IVC_F32A(NWV, ACTV, OUTV)                                                                  \
  hipLaunchKernelGGL((k_gemm_f32a<1, 4, NWV, 4, ACTV, OUTV>), grid, dim3(NWV * 64), 0, s,          \
                     (const float*)g.A, g.lda, g.a_bs, (const bf16_t*)g.W, g.ldw, g.w_bs, g.bias,  \
                     g.bias_bs, g.Cm, C2, g.ldc, g.c_bs, g.M, g.N, g.K, scale)
#define IVC_F32A_S(ACTV, OUTV)                                                                     \
  hipLaunchKernelGGL((k_gemm_f32a<1, 4, 2, 1, ACTV, OUTV>), grid, dim3(128), 0, s,                 \
                     (const float*)g.A, g.lda, g.a_bs, (const bf16_t*)g.W, g.ldw, g.w_bs, g.bias,  \
                     g.bias_bs, g.Cm, C2, g.ldc, g.c_bs, g.M, g.N, g.K, scale)
  if (out_split) {
    if (g.act != ACT_NONE) return hipErrorInvalidValue;
    if (longk) IVC_F32A(8, ACT_NONE, 1);
    else IVC_F32A_S(ACT_NONE, 1);
  } else if (g.act == ACT_GELU) {
    if (longk) IVC_F32A(8, ACT_GELU, 0);
    else IVC_F32A_S(ACT_GELU, 0);
  } else {
    if (longk) IVC_F32A(8, ACT_NONE, 0);
    else IVC_F32A_S(ACT_NONE, 0);
  }
#undef IVC_F32A
#undef IVC_F32A_S
  return hipGetLastError();
}

// dst[c][r] = src[r][c] for a [R, Cc] bf16 matrix (weights, once at creation)
__global__ void __launch_bounds__(256)
k_transpose_bf16(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int R, int Cc) {
  __shared__ bf16_t t[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < R && c < Cc) ? src[(long long)r * Cc + c] : (bf16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (c < Cc && r < R) dst[(long long)c * R + r] = t[tx][i];
  }
}

hipError_t launch_transpose_bf16(const void* src, void* dst, int R, int Cc, hipStream_t s) {
  if (R <= 0 || Cc <= 0) return hipSuccess;
  dim3 grid((unsigned)((Cc + 31) / 32), (unsigned)((R + 31) / 32));
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, (const bf16_t*)src, (bf16_t*)dst, R,
                     Cc);
  return hipGetLastError();
}

// heads H .. 15 of the folded queries [T, 16, C] set to zero (a fill kernel,
// not a memset, so the call can sit in a captured graph)
__global__ void k_zero_heads(bf16_t* hi, bf16_t* lo, int H, int C) {
  const int t = blockIdx.y;
  const long long n = (long long)(16 - H) * C;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const long long o = ((long long)t * 16 + H) * C + i;
    hi[o] = 0;
    lo[o] = 0;
  }
}

hipError_t launch_zero_heads(void* qt_hi, void* qt_lo, int T, int H, int C, hipStream_t s) {
  if (T <= 0 || H >= 16) return hipSuccess;
  hipLaunchKernelGGL(k_zero_heads, dim3(8, (unsigned)T), dim3(256), 0, s, (bf16_t*)qt_hi,
                     (bf16_t*)qt_lo, H, C);
  return hipGetLastError();
}

}  // namespace ivc
