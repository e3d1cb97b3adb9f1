// GEMMs of the connector: C[M, N] = act(A[M, K] . W[N, K]^T + bias[N]).
//
// Both operands are K-contiguous (A row-major, W in nn.Linear [out, in]
// layout), which is exactly what a CDNA MFMA lane wants: each lane feeds 8
// consecutive K values of one row of A and one row of W to
// v_mfma_f32_32x32x16_bf16.  mlp1, mlp2 and the pooling K/V projection all
// use the MFMA kernel; the SIMT kernel covers fp32 workloads and the router's
// fp32-activation products, whose M is the tile count.
#include "common.h"
#include "kernels.h"

namespace ivc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.
//
// Workgroup tile BM x BN, K step 64, WM x WN wavefronts each owning a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA blocks.  Operand tiles are
// staged through LDS with a 16-byte row pad (row stride 144 B) so that the
// 16 lanes of each ds_read_b128 phase hit 16 distinct 4-bank groups.  Two
// LDS buffers: the next K step's global loads are issued into registers
// before the current step's MFMAs and written to the other buffer after
// them, with one barrier per step.
//
// Grid mapping: workgroups are dealt round-robin to the 8 XCDs, so the linear
// id is first regrouped so that consecutive tile ids land on one XCD, then
// tiles are walked in bands of 8 tile-rows so an XCD's L2 sees the same A
// rows and W rows many times.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int ACT>
__global__ void __launch_bounds__(WM* WN * 64, 1)
k_gemm_mfma(const bf16_t* __restrict__ A, long long lda, int a_rpg, long long a_gstride,
            int a_goff, const bf16_t* __restrict__ W, long long ldw,
            const float* __restrict__ bias, bf16_t* __restrict__ Cm, long long ldc, int M, int N,
            int K, RowMap rm) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 64;
  constexpr int LDK = BK + 8;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int AV = BM * (BK / 8) / NT;
  constexpr int BV = BN * (BK / 8) / NT;
  static_assert(AV * NT == BM * (BK / 8) && BV * NT == BN * (BK / 8), "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDK];

  // rows actually present (route-first products size the grid for all
  // tiles): the tile grid is laid out over those rows only, so the active
  // workgroups stay spread over all XCDs; the rest leave at once
  if (rm.m_dev != nullptr) M = min(M, *rm.m_dev * rm.m_mult);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int nb = tiles_m * tiles_n;
  if ((int)blockIdx.x >= nb) return;  // uniform over the workgroup, before any barrier
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int in_group = GM * tiles_n;
  const int first_m = (bid / in_group) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int pid_m = first_m + (bid % in_group) % gsize;
  const int pid_n = (bid % in_group) / gsize;
  const int m0 = pid_m * BM, n0 = pid_n * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;

  const bf16_t* a_src[AV];
  const bf16_t* b_src[BV];
  int a_dst[AV], b_dst[BV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = (c & 7) * 8;
    const int gm = min(m0 + r, M - 1);
    const long long phys =
        a_rpg > 0 ? (long long)(gm / a_rpg) * a_gstride + a_goff + gm % a_rpg : (long long)gm;
    a_src[i] = A + phys * lda + kc;
    a_dst[i] = r * LDK + kc;
  }
#pragma unroll
  for (int i = 0; i < BV; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = (c & 7) * 8;
    const int gn = min(n0 + r, N - 1);
    b_src[i] = W + (long long)gn * ldw + kc;
    b_dst[i] = r * LDK + kc;
  }

  u32x4 ra[AV], rb[BV];
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = K / BK;
#pragma unroll
  for (int i = 0; i < AV; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i]);
#pragma unroll
  for (int i = 0; i < BV; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i]);
#pragma unroll
  for (int i = 0; i < AV; ++i) *reinterpret_cast<u32x4*>(&sA[0][a_dst[i]]) = ra[i];
#pragma unroll
  for (int i = 0; i < BV; ++i) *reinterpret_cast<u32x4*>(&sB[0][b_dst[i]]) = rb[i];
  __syncthreads();

  const int frag_k = (lane >> 5) * 8;
  const int frag_r = lane & 31;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      const long long ko = (long long)(kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < AV; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + ko);
#pragma unroll
      for (int i = 0; i < BV; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + ko);
    }
    const bf16_t* tA = sA[cur];
    const bf16_t* tB = sB[cur];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(
            &tA[(wm * TM + i * 32 + frag_r) * LDK + kk * 16 + frag_k]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(
            &tB[(wn * TN + j * 32 + frag_r) * LDK + kk * 16 + frag_k]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < AV; ++i) *reinterpret_cast<u32x4*>(&sA[cur ^ 1][a_dst[i]]) = ra[i];
#pragma unroll
      for (int i = 0; i < BV; ++i) *reinterpret_cast<u32x4*>(&sB[cur ^ 1][b_dst[i]]) = rb[i];
    }
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane l holds column l % 32 and rows
  // 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn * TN + j * 32 + (lane & 31);
    const bool col_ok = col < N;
    const float bj = (bias != nullptr && col_ok) ? bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * TM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (col_ok && row < M) {
          float x = acc[i][j][v] + bj;
          if (ACT == ACT_GELU) x = gelu_erf(x);
          const long long orow =
              rm.c_map != nullptr ? (long long)rm.c_map[row / rm.c_rpg] * rm.c_rpg + row % rm.c_rpg
                                  : row;
          Cm[orow * ldc + col] = f32_to_bf16(x);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_mfma_cfg(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid((unsigned)tiles), block(WM * WN * 64);
  if (g.act == ACT_GELU)
    hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, ACT_GELU>), grid, block, 0, s,
                       (const bf16_t*)g.A, g.lda, g.a_rpg, g.a_gstride, g.a_goff,
                       (const bf16_t*)g.W, g.ldw, g.bias, (bf16_t*)g.Cm, g.ldc, g.M, g.N, g.K,
                       g.rm);
  else
    hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, ACT_NONE>), grid, block, 0, s,
                       (const bf16_t*)g.A, g.lda, g.a_rpg, g.a_gstride, g.a_goff,
                       (const bf16_t*)g.W, g.ldw, g.bias, (bf16_t*)g.Cm, g.ldc, g.M, g.N, g.K,
                       g.rm);
  return hipGetLastError();
}

bool gemm_mfma_supported(const GemmArgs& g) {
  return g.a_dtype == DT_BF16 && g.w_dtype == DT_BF16 && g.c_dtype == DT_BF16 && g.K % 64 == 0 &&
         g.K > 0 && g.M > 0 && g.N > 0 && g.lda % 8 == 0 && g.ldw % 8 == 0;
}

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t s) {
  if (!gemm_mfma_supported(g)) return hipErrorInvalidValue;
  // 128 x 128 tiles (large products go to the LDS-DMA kernel instead)
  return launch_mfma_cfg<128, 128, 2, 2>(g, s);
}

// ---------------------------------------------------------------------------
// SIMT GEMM, fp32 FMA, for fp32 workloads and the router's fp32-activation
// products (M = tile count, a few hundred rows).  32 x 64 output tile, K step
// 32, 256 threads with 2 x 4 outputs each; operand tiles go to LDS K-major.
// Skinny products split K over grid.z so the grid covers the chip: each split
// writes its partial tile and a second kernel adds the splits in order and
// applies bias and activation (deterministic, and no device-scope fence,
// which on a multi-XCD part would write back and invalidate whole L2s).
// ---------------------------------------------------------------------------
constexpr int SBM = 32, SBN = 64, SBK = 32;

int simt_tiles(int M, int N) { return ((M + SBM - 1) / SBM) * ((N + SBN - 1) / SBN); }

int simt_ksplit(int M, int N, int K, int batch) {
  const long long tiles = (long long)simt_tiles(M, N) * batch;
  int ks = 1;
  while (tiles * ks < 512 && K / (ks * 2) >= 128) ks *= 2;
  return ks;
}

size_t simt_part_elems(int M, int N, int batch, int ksplit) {
  return ksplit > 1 ? (size_t)batch * ksplit * M * N : 0;
}

template <typename T> IVC_DEV void load4(const T* p, float* f);
template <> IVC_DEV void load4<float>(const float* p, float* f) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  unpack<float>(v, f);
}
template <> IVC_DEV void load4<bf16_t>(const bf16_t* p, float* f) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
}

template <typename TA, typename TW, typename TC, int ACT>
__global__ void __launch_bounds__(256)
k_gemm_simt(const TA* __restrict__ A, long long lda, int a_rpg, long long a_gstride, int a_goff,
            const TW* __restrict__ W, long long ldw, const float* __restrict__ bias,
            TC* __restrict__ Cm, long long ldc, int M, int N, int K, long long a_bs,
            long long w_bs, long long c_bs, long long bias_bs, int ksplit, int vec,
            float* __restrict__ part, RowMap rm) {
  __shared__ float sA[SBK][SBM + 1];
  __shared__ float sW[SBK][SBN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * SBM, n0 = blockIdx.x * SBN;
  const int b = blockIdx.z / ksplit, kz = blockIdx.z % ksplit;
  const int Mfull = M;  // the split-K partial buffers are laid out for all rows
  if (rm.m_dev != nullptr) M = min(M, *rm.m_dev * rm.m_mult);
  if (m0 >= M) return;  // uniform over the workgroup, before any barrier
  A += b * a_bs;
  W += b * w_bs;

  const int kchunk = ((K + ksplit - 1) / ksplit + SBK - 1) / SBK * SBK;
  const int k_beg = kz * kchunk, k_end = min(K, k_beg + kchunk);

  // loaders: A tile 32 x 32 (4 consecutive k per thread), W tile 64 x 32 (2 x 4)
  const int ar = tid >> 3, ak = (tid & 7) * 4;
  const int wr = tid >> 2, wk = (tid & 3) * 4;
  const int gm = m0 + ar, gn = n0 + wr;
  const bool a_ok = gm < M, w_ok = gn < N;
  long long a_row = 0;
  if (a_ok) a_row = a_rpg > 0 ? (long long)(gm / a_rpg) * a_gstride + a_goff + gm % a_rpg : gm;
  const TA* a_ptr = A + a_row * lda;
  const TW* w_ptr = W + (long long)(w_ok ? gn : 0) * ldw;

  float acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = k_beg; k0 < k_end; k0 += SBK) {
    float av[4], wv[8];
    if (vec && k0 + SBK <= k_end) {
      if (a_ok) load4<TA>(a_ptr + k0 + ak, av);
      else av[0] = av[1] = av[2] = av[3] = 0.f;
      if (w_ok) {
        load4<TW>(w_ptr + k0 + wk, wv);
        load4<TW>(w_ptr + k0 + wk + 16, wv + 4);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e] = 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = k0 + ak + e;
        av[e] = (a_ok && k < k_end) ? Elem<TA>::to_f(a_ptr[k]) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + wk + (e & 3) + 16 * (e >> 2);
        wv[e] = (w_ok && k < k_end) ? Elem<TW>::to_f(w_ptr[k]) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) sA[ak + e][ar] = av[e];
#pragma unroll
    for (int e = 0; e < 8; ++e) sW[wk + (e & 3) + 16 * (e >> 2)][wr] = wv[e];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SBK; ++k) {
      const float a0 = sA[k][ty * 2], a1 = sA[k][ty * 2 + 1];
      float w4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w4[j] = sW[k][tx * 4 + j];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[0][j] = fmaf(a0, w4[j], acc[0][j]);
        acc[1][j] = fmaf(a1, w4[j], acc[1][j]);
      }
    }
  }

  if (ksplit > 1) {
    float* pb = part + ((size_t)b * ksplit + kz) * Mfull * N;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = m0 + ty * 2 + i;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col < N) pb[(size_t)row * N + col] = acc[i][j];
      }
    }
    return;
  }
  Cm += b * c_bs;
  if (bias != nullptr) bias += b * bias_bs;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = m0 + ty * 2 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      float x = acc[i][j] + (bias != nullptr ? bias[col] : 0.f);
      if (ACT == ACT_GELU) x = gelu_erf(x);
      const long long orow =
          rm.c_map != nullptr ? (long long)rm.c_map[row / rm.c_rpg] * rm.c_rpg + row % rm.c_rpg : row;
      Cm[orow * ldc + col] = Elem<TC>::from_f(x);
    }
  }
}

// out = act(sum_z part[b][z] + bias), the splits added in order
template <typename TC, int ACT>
__global__ void __launch_bounds__(256)
k_splitk_reduce(const float* __restrict__ part, int ksplit, int M, int N,
                const float* __restrict__ bias, long long bias_bs, TC* __restrict__ Cm,
                long long ldc, long long c_bs, RowMap rm) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  const int Mact = rm.m_dev != nullptr ? min(M, *rm.m_dev * rm.m_mult) : M;
  if (i >= (long long)Mact * N) return;
  const int row = (int)(i / N), col = (int)(i % N);
  const float* pb = part + (size_t)b * ksplit * M * N + i;
  float x = 0.f;
  for (int z = 0; z < ksplit; ++z) x += pb[(size_t)z * M * N];
  if (bias != nullptr) x += bias[b * bias_bs + col];
  if (ACT == ACT_GELU) x = gelu_erf(x);
  const long long orow =
      rm.c_map != nullptr ? (long long)rm.c_map[row / rm.c_rpg] * rm.c_rpg + row % rm.c_rpg : row;
  Cm[b * c_bs + orow * ldc + col] = Elem<TC>::from_f(x);
}

template <typename TA, typename TW, typename TC>
static hipError_t launch_simt_t(const GemmArgs& g, hipStream_t s) {
  const int batch = g.batch > 0 ? g.batch : 1;
  const int ks = g.ksplit > 0 ? g.ksplit : 1;
  if (ks > 1 && g.part == nullptr) return hipErrorInvalidValue;
  // 16-byte-aligned rows and operands allow vector loads of 4 elements
  auto al = [](const void* p, long long ld, long long bs, int es) {
    return ((uintptr_t)p % 16 == 0) && (ld * es) % 16 == 0 && (bs * es) % 16 == 0;
  };
  const int vec = g.a_rpg == 0 && al(g.A, g.lda, g.a_bs, sizeof(TA)) &&
                  al(g.W, g.ldw, g.w_bs, sizeof(TW)) && ((uintptr_t)g.W % 8 == 0);
  dim3 grid((unsigned)((g.N + SBN - 1) / SBN), (unsigned)((g.M + SBM - 1) / SBM),
            (unsigned)(batch * ks));
  dim3 block(256);
#define IVC_SIMT(ACTV)                                                                            \
  hipLaunchKernelGGL((k_gemm_simt<TA, TW, TC, ACTV>), grid, block, 0, s, (const TA*)g.A, g.lda,  \
                     g.a_rpg, g.a_gstride, g.a_goff, (const TW*)g.W, g.ldw, g.bias, (TC*)g.Cm,   \
                     g.ldc, g.M, g.N, g.K, g.a_bs, g.w_bs, g.c_bs, g.bias_bs, ks, vec, g.part, g.rm)
  if (g.act == ACT_GELU && ks == 1) IVC_SIMT(ACT_GELU);
  else IVC_SIMT(ACT_NONE);
#undef IVC_SIMT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  const long long n = (long long)g.M * g.N;
  dim3 rg((unsigned)((n + 255) / 256), (unsigned)batch);
  if (g.act == ACT_GELU)
    hipLaunchKernelGGL((k_splitk_reduce<TC, ACT_GELU>), rg, dim3(256), 0, s, (const float*)g.part,
                       ks, g.M, g.N, g.bias, g.bias_bs, (TC*)g.Cm, g.ldc, g.c_bs, g.rm);
  else
    hipLaunchKernelGGL((k_splitk_reduce<TC, ACT_NONE>), rg, dim3(256), 0, s, (const float*)g.part,
                       ks, g.M, g.N, g.bias, g.bias_bs, (TC*)g.Cm, g.ldc, g.c_bs, g.rm);
  return hipGetLastError();
}

template <typename TA, typename TW>
static hipError_t launch_simt_c(const GemmArgs& g, hipStream_t s) {
  return g.c_dtype == DT_BF16 ? launch_simt_t<TA, TW, bf16_t>(g, s)
                              : launch_simt_t<TA, TW, float>(g, s);
}
template <typename TA>
static hipError_t launch_simt_w(const GemmArgs& g, hipStream_t s) {
  return g.w_dtype == DT_BF16 ? launch_simt_c<TA, bf16_t>(g, s) : launch_simt_c<TA, float>(g, s);
}

hipError_t launch_gemm_simt(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  return g.a_dtype == DT_BF16 ? launch_simt_w<bf16_t>(g, s) : launch_simt_w<float>(g, s);
}

}  // namespace ivc
