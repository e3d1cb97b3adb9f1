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
#include "gate_rows.h"
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

// 8 fp32 values -> bf16 high parts and the bf16 rounding of what they leave.
// No contraction: where the caller formed x as a product, a fused
// multiply-subtract would take lo from the unrounded product, and whether the
// compiler fuses depends on what it can prove about the caller's step mask
// (known to be 1 in the first step of a load round), so the same tile would
// split differently in kernels that load different numbers of K steps at once.
IVC_DEV void split8(const float4& x0, const float4& x1, bf16x8_t& hi, bf16x8_t& lo) {
#pragma clang fp contract(off)
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

// Activation row of one lane.  NS = 1: a plain fp32 row.  NS > 1: the
// weighted sum of NS partial rows, (sum_s sc[s] * p[s][k]) * inv, accumulated
// with fmaf in order s = 0, 1, ... (unused sources carry sc = 0).
template <int NS>
struct ARow {
  const float* p[NS];
  float sc[NS];
  float inv;
  struct Raw {
    float4 v[NS][2];
  };
  IVC_DEV void load(int k0, Raw& r) const {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      r.v[i][0] = *reinterpret_cast<const float4*>(p[i] + k0);
      r.v[i][1] = *reinterpret_cast<const float4*>(p[i] + k0 + 4);
    }
  }
  IVC_DEV void get(const Raw& r, float4& x0, float4& x1) const {
    if (NS == 1) {
      x0 = r.v[0][0];
      x1 = r.v[0][1];
      return;
    }
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float* v0 = reinterpret_cast<const float*>(&r.v[i][0]);
      const float* v1 = reinterpret_cast<const float*>(&r.v[i][1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = fmaf(v0[e], sc[i], a[e]);
        a[4 + e] = fmaf(v1[e], sc[i], a[4 + e]);
      }
    }
    x0 = make_float4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
    x1 = make_float4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv);
  }
};

// Main loop of one wave: MB x NB blocks of 16 x 16, K steps w, w + NWV, ...
// (each 32 wide), up to PD of them loaded at once.  arow / wrow: this lane's
// operand rows, already offset by 8 * (lane / 16) elements.  WS: the weights
// are fp32 values held as bf16 high (wrow) + low (wlo) parts, and each step
// adds a_hi.w_hi, a_lo.w_hi, a_hi.w_lo (a_lo.w_lo is below 2^-16 of them).
template <int MB, int NB, int NWV, int PD, int NS, bool WS = false>
IVC_DEV void f32a_mainloop(const ARow<NS> (&arow)[MB], const bf16_t* const (&wrow)[NB],
                           const bf16_t* const (&wlo)[NB], int w, int nks,
                           f32x4_t (&acc)[MB][NB]) {
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = w; s0 < nks; s0 += NWV * PD) {
    typename ARow<NS>::Raw xa[PD][MB];
    u32x4 xw[PD][NB], xl[WS ? PD : 1][NB];
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      const int k0 = 32 * min(s0 + NWV * i, nks - 1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) arow[mb].load(k0, xa[i][mb]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) xw[i][nb] = *reinterpret_cast<const u32x4*>(wrow[nb] + k0);
      if (WS) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          xl[WS ? i : 0][nb] = *reinterpret_cast<const u32x4*>(wlo[nb] + k0);
      }
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
        float4 x0, x1;
        arow[mb].get(xa[i][mb], x0, x1);
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
          if (WS) {
            const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, xl[WS ? i : 0][nb]);
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[mb], bl, acc[mb][nb], 0, 0, 0);
          }
        }
    }
  }
}

// One output tile (16 MB) x (16 NB) of batch entry b with NWV waves, PD K
// steps loaded per wave at once: the main loop, then the NWV partial tiles
// summed through LDS in wave order, bias, activation and the store.
// OUT: 0 = fp32 C, 1 = C * scale as bf16 high part (Cm) and low part (C2).
// The partial-tile buffer of f32a_tile: one array per size, so the tile
// functions of every instance in one kernel share it.
template <int NF>
IVC_DEV float* f32a_red_lds() {
  __shared__ __attribute__((aligned(16))) float red[NF];
  return red;
}

// CCOH: write-through stores of C (read by workgroups of the same launch on
// other XCDs).
template <int MB, int NB, int NWV, int PD, int ACT, int OUT, int NS, bool CCOH = false>
IVC_DEV void f32a_tile(const ARow<NS> (&arow)[MB], const bf16_t* __restrict__ W, long long ldw,
                       const float* __restrict__ bias, void* __restrict__ Cm,
                       void* __restrict__ C2, long long ldc, int M, int N, int K, float scale,
                       int m0, int n0) {
  constexpr int BM = 16 * MB, BN = 16 * NB, LDR = BN + 4;
  constexpr int NTH = NWV * 64, RPP = NTH / BN;  // epilogue rows per pass
  static_assert(NTH % BN == 0 && BM % RPP == 0, "epilogue shape");
  float(*red)[BM][LDR] = reinterpret_cast<float(*)[BM][LDR]>(f32a_red_lds<NWV * BM * LDR>());
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lo16 = lane & 15, hi4 = lane >> 4;
  const bf16_t* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    wrow[nb] = W + (long long)min(n0 + 16 * nb + lo16, N - 1) * ldw + 8 * hi4;

  f32x4_t acc[MB][NB];
  f32a_mainloop<MB, NB, NWV, PD, NS>(arow, wrow, wrow, w, K / 32, acc);

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
  const float bj = bias != nullptr ? bias[n] : 0.f;
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
    const long long o = (long long)m * ldc + n;
    if (OUT == 0) {
      if (CCOH)
        st_coh(reinterpret_cast<float*>(Cm) + o, v);
      else
        reinterpret_cast<float*>(Cm)[o] = v;
    } else {
      v *= scale;
      const bf16_t h = f32_to_bf16(v);
      reinterpret_cast<bf16_t*>(Cm)[o] = h;
      reinterpret_cast<bf16_t*>(C2)[o] = f32_to_bf16(v - bf16_to_f32(h));
    }
  }
}
}  // namespace

template <int MB, int NB, int NWV, int PD, int ACT, int OUT>
__global__ void __launch_bounds__(NWV * 64)
k_gemm_f32a(const float* __restrict__ A, long long lda, long long a_bs,
            const bf16_t* __restrict__ W, long long ldw, long long w_bs,
            const float* __restrict__ bias, long long bias_bs, void* __restrict__ Cm,
            void* __restrict__ C2, long long ldc, long long c_bs, int M, int N, int K,
            float scale) {
  const int lane = threadIdx.x & 63;
  const int lo16 = lane & 15, hi4 = lane >> 4;
  const int n0 = blockIdx.x * 16 * NB, m0 = blockIdx.y * 16 * MB, b = blockIdx.z;
  A += b * a_bs;
  // operand rows of this lane (clamped: rows past M or N are computed, not stored)
  ARow<1> arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    arow[mb].p[0] = A + (long long)min(m0 + 16 * mb + lo16, M - 1) * lda + 8 * hi4;
  f32a_tile<MB, NB, NWV, PD, ACT, OUT, 1>(
      arow, W + b * w_bs, ldw, bias != nullptr ? bias + b * bias_bs : nullptr,
      OUT == 0 ? (void*)((float*)Cm + b * c_bs) : (void*)((bf16_t*)Cm + b * c_bs),
      OUT == 0 ? nullptr : (void*)((bf16_t*)C2 + b * c_bs), ldc, M, N, K, scale, m0, n0);
}

// Value fold of the folded pooling, reading the token pass's per-workgroup
// partials directly (no merged xbar in between):
//   o[t, h d + i] = bv[h d + i] + sum_c Wv[h d + i, c] xbar[t, h, c],
//   xbar[t, h, :] = (sum_s 2^(m_s - M) acc_s) / (sum_s 2^(m_s - M) l_s),
// over the partials s of tile t (workgroups g0 .. g1 of the token pass, in
// order), M their largest running max: the same arithmetic as the merge
// kernel of the token pass.  grid (ceil(d / 64), ceil(T / 16), H).
// One (16-tile, 64-column) tile of head h's value fold.  COH: write-through
// stores of o (read by workgroups of the same launch on other XCDs).
template <int MAXS, bool COH>
IVC_DEV void fold_value_tile(const float* __restrict__ part, const int* __restrict__ valid,
                             int Ntok, int Q, int segmax, const bf16_t* __restrict__ Wv,
                             long long ldw, const float* __restrict__ bv, float* __restrict__ o,
                             int T, int C, int H, int n0, int m0, int h) {
  constexpr int FH = 16;
  const int lane = threadIdx.x & 63;
  const int lo16 = lane & 15, hi4 = lane >> 4;
  const int d = C / H;
  const int NC = (Ntok + 15) / 16;
  const int t = min(m0 + lo16, T - 1);
  int nv = valid != nullptr ? valid[t] : Ntok;
  nv = nv < 1 ? 1 : (nv > Ntok ? Ntok : nv);
  const int lo_c = t * NC, hi_c = t * NC + (nv + 15) / 16;
  const int g0 = lo_c / Q, g1 = (hi_c - 1) / Q;
  const size_t stride = (size_t)FH * (2 + C);
  ARow<MAXS> arow[1];
  float ms[MAXS], ls[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const int g = min(g0 + i, g1);
    const float* pp = part + ((size_t)g * segmax + (t - (g * Q) / NC)) * stride;
    ms[i] = pp[h];
    ls[i] = pp[FH + h];
    arow[0].p[i] = pp + 2 * FH + (size_t)h * C + 8 * hi4;
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < MAXS; ++i)
    if (g0 + i <= g1) M = fmaxf(M, ms[i]);
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const float e = g0 + i <= g1 ? exp2f(ms[i] - M) : 0.f;
    arow[0].sc[i] = e;
    L = fmaf(ls[i], e, L);
  }
  arow[0].inv = 1.0f / L;
  // all K steps of a wave in one round of loads while the registers allow it
  constexpr int PD = MAXS <= 3 ? 4 : 2;
  f32a_tile<1, 4, 8, PD, ACT_NONE, 0, MAXS, COH>(arow, Wv + (long long)h * d * ldw, ldw,
                                                 bv + h * d, o + h * d, nullptr, C, T, d, C, 1.f,
                                                 m0, n0);
}

template <int MAXS>
__global__ void __launch_bounds__(512)
k_fold_value_merged(const float* __restrict__ part, const int* __restrict__ valid, int Ntok,
                    int Q, int segmax, const bf16_t* __restrict__ Wv, long long ldw,
                    const float* __restrict__ bv, float* __restrict__ o, int T, int C, int H) {
  // the 16-tile row blocks of one head in one XCD's range (they share Wv_h)
  const int nx = gridDim.x, ny = gridDim.y;
  const int wg = xcd_major(blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z), nx * ny * gridDim.z);
  fold_value_tile<MAXS, false>(part, valid, Ntok, Q, segmax, Wv, ldw, bv, o, T, C, H,
                               (wg % nx) * 64, ((wg / nx) % ny) * 16, wg / (nx * ny));
}

int fold_value_merged_max_parts(int T, int N, int Q) {
  if (T <= 0 || N <= 0 || Q <= 0) return 0;
  const int NC = (N + 15) / 16;
  // a tile's chunks [t NC, t NC + NC) meet at most this many workgroups of Q chunks
  return (NC - 1 + Q - 1) / Q + 1;
}

hipError_t launch_fold_value_merged(const float* part, const int* valid, int N, int Q, int segmax,
                                    const void* Wv, long long ldw, const float* bv, float* o, int T,
                                    int C, int H, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int maxs = fold_value_merged_max_parts(T, N, Q);
  if (maxs < 1 || maxs > 4 || H < 1 || C % H || (C / H) % 16 || C % 32 || (uintptr_t)part % 16 ||
      (uintptr_t)Wv % 16 || ldw < C || ldw % 8)
    return hipErrorInvalidValue;
  const int d = C / H;
  const dim3 grid((unsigned)((d + 63) / 64), (unsigned)((T + 15) / 16), (unsigned)H);
#define IVC_FVM(S)                                                                                 \
  hipLaunchKernelGGL(k_fold_value_merged<S>, grid, dim3(512), 0, s, part, valid, N, Q, segmax,     \
                     (const bf16_t*)Wv, ldw, bv, o, T, C, H)
  if (maxs <= 2) IVC_FVM(2);
  else if (maxs == 3) IVC_FVM(3);
  else IVC_FVM(4);
#undef IVC_FVM
  return hipGetLastError();
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

// Folded pooling query of one layer, the query projection and the key fold in
// one launch (the same arithmetic, in the same order, as the two products
// above: the query projection as a 16 x 64 tile of 8 waves x 4 K steps, the
// fold as the short-K form, two K-step parities summed in order):
//   qp = Wq q + bq                                  [T, C] (never stored)
//   q~_h = scale * (Wk_h^T qp_h)   for every head h  [T, 16, C] bf16 hi + lo
// Workgroup (16 tiles, head h): the 16 x D block of qp for head h (K = C)
// summed through LDS, then the 16 x C block of q~_h with K = D = C / H,
// wave w taking columns [w C/8, (w+1) C/8); the bf16 halves go through a
// wave-private LDS slab so each row leaves with 16-byte stores.
// WS: Wq given as bf16 high (Wq) + low (Wq_lo) parts of fp32 weights.
// The (16-tile, head h) block of the fused query fold.
template <int D, bool WS>
IVC_DEV void fold_query_tile(const float* __restrict__ q, long long ldq,
                             const bf16_t* __restrict__ Wq, const bf16_t* __restrict__ Wq_lo,
                             long long ldwq, const float* __restrict__ bq,
                             const bf16_t* __restrict__ WkT, long long ldk,
                             bf16_t* __restrict__ qt_hi, bf16_t* __restrict__ qt_lo, int T, int C,
                             float scale, int m0, int h) {
  constexpr int NB = D / 16, LDR = D + 4, KS = D / 32;
  constexpr int SR = 128 + 8;  // slab row (bf16): up to 128 columns per wave, 16 bytes of pad
  __shared__ __attribute__((aligned(16))) float red[8][16][LDR];
  __shared__ __attribute__((aligned(16))) float qp_s[16][D];
  __shared__ __attribute__((aligned(16))) bf16_t slab[8][2][16][SR];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lo16 = lane & 15, hi4 = lane >> 4;

  const int CW = C / 8, nbw = CW / 16;  // columns and 16-column blocks of this wave (<= 8)
  const int c0 = w * CW;
  // key-fold weights of a group of GB column blocks (loaded ahead of their use)
  constexpr int GB = KS <= 2 ? 8 : 4;
  u32x4 xw[GB][KS];
  auto load_group = [&](int g) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int n = c0 + 16 * min(g + j, nbw - 1) + lo16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        xw[j][ks] = *reinterpret_cast<const u32x4*>(WkT + (long long)n * ldk + h * D + 32 * ks +
                                                    8 * hi4);
    }
  };

  // ---- qp block [16, D] of head h
  {
    ARow<1> arow[1];
    arow[0].p[0] = q + (long long)min(m0 + lo16, T - 1) * ldq + 8 * hi4;
    const bf16_t* wrow[NB];
    const bf16_t* wlo[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      wrow[nb] = Wq + (long long)(h * D + 16 * nb + lo16) * ldwq + 8 * hi4;
      wlo[nb] = WS ? Wq_lo + (long long)(h * D + 16 * nb + lo16) * ldwq + 8 * hi4 : wrow[nb];
    }
    f32x4_t acc[1][NB];
    // (split weights at d = 128 load half as many K steps at once, to stay in registers)
    f32a_mainloop<1, NB, 8, (WS && D >= 128) ? 2 : 4, 1, WS>(arow, wrow, wlo, w, C / 32, acc);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][4 * hi4 + v][16 * nb + lo16] = acc[0][nb][v];
  }
  load_group(0);  // in flight across the reduction
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * D; i += 512) {
    const int r = i / D, col = i - r * D;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) v += red[ww][r][col];
    v += bq[h * D + col];
    qp_s[r][col] = v;
  }
  __syncthreads();

  // ---- q~_h block [16, C]: A = qp_s (hi + lo), B rows n of WkT at column offset h D
  bf16x8_t ah[KS], al[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float4 x0 = *reinterpret_cast<const float4*>(&qp_s[lo16][32 * ks + 8 * hi4]);
    const float4 x1 = *reinterpret_cast<const float4*>(&qp_s[lo16][32 * ks + 8 * hi4 + 4]);
    split8(x0, x1, ah[ks], al[ks]);
  }
  bf16_t(*sh)[SR] = slab[w][0];
  bf16_t(*sl)[SR] = slab[w][1];
  for (int g = 0; g < nbw; g += GB) {
    if (g > 0) load_group(g);
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      if (g + j >= nbw) break;
      f32x4_t a0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, a1 = a0;  // K steps of even / odd index
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, xw[j][ks]);
        f32x4_t& a = (ks & 1) ? a1 : a0;
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bw, a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks], bw, a, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = 0.f;
        x += a0[v];
        x += a1[v];
        x += 0.f;  // the missing bias, as the two-launch form adds it (-0 becomes +0)
        x *= scale;
        const bf16_t hv = f32_to_bf16(x);
        sh[4 * hi4 + v][16 * (g + j) + lo16] = hv;
        sl[4 * hi4 + v][16 * (g + j) + lo16] = f32_to_bf16(x - bf16_to_f32(hv));
      }
    }
  }
  __syncthreads();  // slab rows are read back by other lanes
  const int ppr = CW / 8;  // 16-byte pieces per row
  for (int i = lane; i < 16 * ppr; i += 64) {
    const int r = i / ppr, p = i - r * ppr;
    const int t = m0 + r;
    if (t >= T) break;
    const long long o = ((long long)t * 16 + h) * C + c0 + 8 * p;
    *reinterpret_cast<u32x4*>(qt_hi + o) = *reinterpret_cast<const u32x4*>(&sh[r][8 * p]);
    *reinterpret_cast<u32x4*>(qt_lo + o) = *reinterpret_cast<const u32x4*>(&sl[r][8 * p]);
  }
}

template <int D, bool WS>
__global__ void __launch_bounds__(512)
k_fold_query_fused(const float* __restrict__ q, long long ldq, const bf16_t* __restrict__ Wq,
                   const bf16_t* __restrict__ Wq_lo, long long ldwq, const float* __restrict__ bq,
                   const bf16_t* __restrict__ WkT, long long ldk,
                   bf16_t* __restrict__ qt_hi, bf16_t* __restrict__ qt_lo, int T, int C,
                   float scale) {
  // the 16-tile row blocks of one head in one XCD's range (they share the
  // head's rows of Wq and columns of Wk)
  const int wg = xcd_major(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  fold_query_tile<D, WS>(q, ldq, Wq, Wq_lo, ldwq, bq, WkT, ldk, qt_hi, qt_lo, T, C, scale,
                         (wg % gridDim.x) * 16, wg / gridDim.x);
}

// A Gating block's first Linear with the previous block's residual LayerNorm
// in its prologue:
//   x_out = x_in + LN(y) * gamma + beta        (rows of K values)
//   C = act(x_out . W^T + bias)                 (the f32a product, 16 x 64 tiles)
// Workgroup (16 rows, 64 columns): its 16 rows of x_out go to LDS (each wave
// two rows: mean, then the mean square deviation, from registers, both
// wave-reduced), the workgroups of the first column block also write them to
// x_out (x_in and x_out must differ: the others still read x_in), and the
// product reads its activation rows from LDS.
// One (16-row, 64-column) tile; store_x: this tile writes its rows of x_out.
// COH: write-through stores of x_out and C (read by workgroups of the same
// launch on other XCDs).
template <int ACT, bool COH = false>
IVC_DEV void ln_rows_tile(const float* __restrict__ x_in, const float* __restrict__ y,
                          const float* __restrict__ gamma, const float* __restrict__ beta,
                          float eps, float* __restrict__ x_out, bool store_x,
                          const bf16_t* __restrict__ W, long long ldw,
                          const float* __restrict__ bias, float* __restrict__ Cm, int M, int N,
                          int K, int m0, int n0) {
  __shared__ __attribute__((aligned(16))) float xs[16 * 1024];  // [16][K], K <= 1024
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lo16 = lane & 15, hi4 = lane >> 4;
  const int vpl = K / 256;  // float4 vectors per lane (K % 256 == 0, K <= 1024)
  // both rows' y, x, gamma and beta loaded up front (one round of latency)
  float4 v[2][4], xv[2][4], gv[4], bv[4];
  int tr[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    tr[rr] = min(m0 + 2 * w + rr, M - 1);
    const float4* yr = reinterpret_cast<const float4*>(y + (long long)tr[rr] * K);
    const float4* xr = reinterpret_cast<const float4*>(x_in + (long long)tr[rr] * K);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < vpl) {
        v[rr][i] = yr[lane + 64 * i];
        xv[rr][i] = xr[lane + 64 * i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < vpl) {
      gv[i] = reinterpret_cast<const float4*>(gamma)[lane + 64 * i];
      bv[i] = reinterpret_cast<const float4*>(beta)[lane + 64 * i];
    }
  }
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int r = 2 * w + rr;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < vpl) s += (v[rr][i].x + v[rr][i].y) + (v[rr][i].z + v[rr][i].w);
    const float mean = wave_sum(s) / (float)K;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < vpl) {
        const float a = v[rr][i].x - mean, b = v[rr][i].y - mean, c = v[rr][i].z - mean,
                    d = v[rr][i].w - mean;
        q += (a * a + b * b) + (c * c + d * d);
      }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)K + eps);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < vpl) {
        const int j = lane + 64 * i;
        const float4 x = xv[rr][i], g = gv[i], b = bv[i];
        float4 o;
        o.x = x.x + (v[rr][i].x - mean) * rstd * g.x + b.x;
        o.y = x.y + (v[rr][i].y - mean) * rstd * g.y + b.y;
        o.z = x.z + (v[rr][i].z - mean) * rstd * g.z + b.z;
        o.w = x.w + (v[rr][i].w - mean) * rstd * g.w + b.w;
        reinterpret_cast<float4*>(xs + r * K)[j] = o;
        if (store_x && m0 + r < M) {
          if (COH)
            st_coh4(x_out + (long long)tr[rr] * K + 4 * j, o);
          else
            reinterpret_cast<float4*>(x_out + (long long)tr[rr] * K)[j] = o;
        }
      }
    }
  }
  __syncthreads();
  ARow<1> arow[1];
  arow[0].p[0] = xs + lo16 * K + 8 * hi4;
  f32a_tile<1, 4, 8, 4, ACT, 0, 1, COH>(arow, W, ldw, bias, Cm, nullptr, N, M, N, K, 1.f, m0,
                                        n0);
}

template <int ACT>
__global__ void __launch_bounds__(512)
k_f32a_ln_rows(const float* __restrict__ x_in, const float* __restrict__ y,
               const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
               float* __restrict__ x_out, const bf16_t* __restrict__ W, long long ldw,
               const float* __restrict__ bias, float* __restrict__ Cm, int M, int N, int K) {
  ln_rows_tile<ACT>(x_in, y, gamma, beta, eps, x_out, blockIdx.x == 0, W, ldw, bias, Cm, M, N,
                    K, blockIdx.y * 16, blockIdx.x * 64);
}

bool f32a_ln_rows_supported(int K) { return K % 256 == 0 && K >= 256 && K <= 1024; }

hipError_t launch_f32a_ln_rows(const float* x_in, const float* y, const float* gamma,
                               const float* beta, float eps, float* x_out, const void* W,
                               long long ldw, const float* bias, float* Cm, int M, int N, int K,
                               int act, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!f32a_ln_rows_supported(K) || x_in == x_out || N <= 0 || ldw < K || ldw % 8 ||
      (uintptr_t)x_in % 16 ||
      (uintptr_t)y % 16 || (uintptr_t)x_out % 16 || (uintptr_t)gamma % 16 ||
      (uintptr_t)beta % 16 || (uintptr_t)W % 16 || (act != ACT_GELU && act != ACT_NONE))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 15) / 16));
  if (act == ACT_GELU)
    hipLaunchKernelGGL(k_f32a_ln_rows<ACT_GELU>, grid, dim3(512), 0, s, x_in, y, gamma, beta, eps,
                       x_out, (const bf16_t*)W, ldw, bias, Cm, M, N, K);
  else
    hipLaunchKernelGGL(k_f32a_ln_rows<ACT_NONE>, grid, dim3(512), 0, s, x_in, y, gamma, beta, eps,
                       x_out, (const bf16_t*)W, ldw, bias, Cm, M, N, K);
  return hipGetLastError();
}

bool fold_query_fused_supported(int C, int H) {
  if (H < 1 || H > 16 || C % H != 0) return false;
  const int d = C / H;
  return (d == 32 || d == 64 || d == 128) && C % 128 == 0 && C <= 1024;
}

hipError_t launch_fold_query_fused(const float* q, long long ldq, const void* Wq, long long ldwq,
                                   const float* bq, const void* WkT, long long ldk, void* qt_hi,
                                   void* qt_lo, int T, int C, int H, float scale, hipStream_t s,
                                   const void* Wq_lo) {
  if (T <= 0) return hipSuccess;
  if (!fold_query_fused_supported(C, H) || !q || !Wq || !bq || !WkT || !qt_hi || !qt_lo ||
      (uintptr_t)q % 16 || (uintptr_t)Wq % 16 || (uintptr_t)WkT % 16 || (uintptr_t)qt_hi % 16 ||
      (uintptr_t)qt_lo % 16 || ldq < 0 || ldq % 4 || (uintptr_t)Wq_lo % 16 || ldwq < C ||
      ldwq % 8 || ldk < C || ldk % 8)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((T + 15) / 16), (unsigned)H);
  const int d = C / H;
#define IVC_FQF(DV, WSV)                                                                           \
  hipLaunchKernelGGL((k_fold_query_fused<DV, WSV>), grid, dim3(512), 0, s, q, ldq,                 \
                     (const bf16_t*)Wq, (const bf16_t*)Wq_lo, ldwq, bq, (const bf16_t*)WkT, ldk,  \
                     (bf16_t*)qt_hi, (bf16_t*)qt_lo, T, C, scale)
  if (Wq_lo != nullptr) {
    if (d == 32) IVC_FQF(32, true);
    else if (d == 64) IVC_FQF(64, true);
    else IVC_FQF(128, true);
  } else {
    if (d == 32) IVC_FQF(32, false);
    else if (d == 64) IVC_FQF(64, false);
    else IVC_FQF(128, false);
  }
#undef IVC_FQF
  return hipGetLastError();
}

// fp32 values as bf16 high and low parts: hi = bf16(x), lo = bf16(x - hi);
// x is a dense [rows, cols] matrix, hi and lo have row stride ld
__global__ void k_split_bf16(const float* __restrict__ x, bf16_t* __restrict__ hi,
                             bf16_t* __restrict__ lo, long long rows, int cols, long long ld) {
  const long long n = rows * cols;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const long long r = i / cols, o = r * ld + (i - r * cols);
    const bf16_t h = f32_to_bf16(x[i]);
    hi[o] = h;
    lo[o] = f32_to_bf16(x[i] - bf16_to_f32(h));
  }
}

hipError_t launch_split_bf16(const float* x, void* hi, void* lo, long long rows, int cols,
                             long long ld, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (ld < cols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_split_bf16, dim3(256), dim3(256), 0, s, x, (bf16_t*)hi, (bf16_t*)lo, rows,
                     cols, ld);
  return hipGetLastError();
}

// dst[c][r] = src[r][c] for a [R, Cc] bf16 matrix (weights, once at creation);
// row strides lds (src) and ldd (dst)
__global__ void __launch_bounds__(256)
k_transpose_bf16(const bf16_t* __restrict__ src, long long lds, bf16_t* __restrict__ dst,
                 long long ldd, int R, int Cc) {
  __shared__ bf16_t t[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < R && c < Cc) ? src[(long long)r * lds + c] : (bf16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (c < Cc && r < R) dst[(long long)c * ldd + r] = t[tx][i];
  }
}

hipError_t launch_transpose_bf16(const void* src, long long lds, void* dst, long long ldd, int R,
                                 int Cc, hipStream_t s) {
  if (R <= 0 || Cc <= 0) return hipSuccess;
  if (lds < Cc || ldd < R) return hipErrorInvalidValue;
  dim3 grid((unsigned)((Cc + 31) / 32), (unsigned)((R + 31) / 32));
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, (const bf16_t*)src, lds,
                     (bf16_t*)dst, ldd, R, Cc);
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

// ---------------------------------------------------------------------------
// The Gating network (InternVL3_5-4B-Flash Gating and CrossAttentionPooling
// page, section 3) and, before it, the pooling's last output projection, in
// one launch.  Its phases are the launches of the per-block form, with the
// same tile functions and so the same arithmetic:
//   [out-projection]  x0 = o . Wo^T + bo                       (the pooled rows)
//   block 0           y1_0 = GELU(x0 . W1^T + b1);  y2_0 = y1_0 . W2^T + b2
//   block b = 1..3    x_b = x_{b-1} + LN(y2_{b-1}) (prologue);
//                     y1_b = GELU(x_b . W1^T + b1);  y2_b = y1_b . W2^T + b2
//   head              x = x_3 + LN(y2_3);  gate = softmax(Wc x + bc)
// Consecutive ranges of workgroups run consecutive phases, one (16-row,
// 64-column) tile or one head row each.  A tile needs only its own 16 rows of
// the previous phase, so each phase keeps one device-scope counter per
// 16-row block (each on a line and memory channel of its own, so the polls of
// waiting workgroups do not queue behind one another); a workgroup waits
// until its block's counter in the previous phase is full (rows of later
// blocks can run ahead).
// Coherence across the XCDs' L2 caches without cache-wide write-back or
// invalidation: every phase writes a buffer of its own with write-through
// stores and counts itself done once they are acknowledged; the readers'
// plain loads cannot hit a stale line, since no XCD reads a block before it
// is complete and the launch starts with invalidated caches.
// Progress: workgroups are dispatched in index order on each XCD and every
// wait is for lower-indexed workgroups, so the lowest unfinished workgroup
// always runs.  A wait still gives up after a few seconds and reports
// IVC_DEV_ERR_ROUTER_SYNC rather than hang.  The counters carry the launch's
// tag in their high bits: values an earlier launch (or uninitialised
// workspace) left there never count.
// ---------------------------------------------------------------------------
namespace {

// Adds one to a tagged counter: the first caller of a launch finds another
// tag there and resets the count under this launch's tag (only one such
// exchange succeeds).
IVC_DEV void tagged_count(unsigned long long* c, unsigned long long tag) {
  unsigned long long cur = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while ((cur >> 16) != tag) {
    if (__hip_atomic_compare_exchange_strong(c, &cur, tag << 16, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      break;
  }
  __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

IVC_DEV void phase_wait(const unsigned long long* c, unsigned long long want, int* status) {
  for (int spin = 0;; ++spin) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want) break;
    if (spin >= (1 << 23)) {
      if (status != nullptr) atomicOr(status, 16);  // IVC_DEV_ERR_ROUTER_SYNC
      break;
    }
    __builtin_amdgcn_s_sleep(10);  // ~640 cycles between polls
  }
}

// Counter of (phase p, row block r): one per 512 bytes, so polls and counts on
// different counters go to different cache lines and memory channels.
constexpr int kSyncStride = 64;

}  // namespace

// VF: 0, or the value fold's partials per tile (2..4) when the launch starts
// with the pooling's last value fold.
template <int VF>
__global__ void __launch_bounds__(512) k_gating_fused(GatingFusedArgs a) {
  const int bid = blockIdx.x;
  int p = 0;
  while (p + 1 < a.nph && bid >= a.first[p + 1]) ++p;
  const int lt = bid - a.first[p];
  const int T = a.T, nt = a.h / 64, mt = (T + 15) / 16;
  // -2: value fold, -1: out-projection, 0..7: blocks, 8: head
  const int ph = p - (VF > 0 ? 1 : 0) - (a.o != nullptr ? 1 : 0);
  // value fold: (64-column block, row block, head), XCD-major like its own launch
  const int vnx = VF > 0 ? (a.h / a.vf_H + 63) / 64 : 1;
  const int vwg = ph == -2 ? xcd_major(lt, vnx * mt * a.vf_H) : 0;
  // 16-row block of this workgroup's work
  const int rb = ph == -2 ? (vwg / vnx) % mt : ph == 8 ? lt / 16 : lt / nt;
  if (p > 0) {
    // the previous phase's workgroups per row block
    const int prev = (VF > 0 && p == 1) ? vnx * a.vf_H : nt;
    if (threadIdx.x == 0)
      phase_wait(a.sync + ((size_t)(p - 1) * mt + rb) * kSyncStride,
                 (a.tag << 16) | (unsigned long long)prev, a.status);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int lo16 = lane & 15, hi4 = lane >> 4;
  if (ph == -2) {
    if constexpr (VF > 0)
      fold_value_tile<VF, true>(a.vf_part, a.vf_valid, a.vf_N, a.vf_Q, a.vf_segmax,
                                (const bf16_t*)a.vf_wv, a.vf_ldw, a.vf_bv,
                                const_cast<float*>(a.o), T, a.h, a.vf_H, 64 * (vwg % vnx),
                                16 * rb, vwg / (vnx * mt));
  } else if (ph == 8) {
    residual_ln_row<true, bf16_t>(lt, a.xb[3], a.y2[3], a.lw[3], a.lb[3], a.h, a.eps,
                                  (const bf16_t*)a.wc, a.bc, a.gate);
  } else {
    const int N = ph < 0 ? a.h : ((ph & 1) ? a.h : a.he);
    const int m0 = 16 * rb, n0 = 64 * (lt % nt);
    const int blk = ph < 0 ? 0 : ph >> 1;
    if (ph >= 2 && (ph & 1) == 0) {
      // block blk's first Linear with block blk-1's residual LayerNorm in front
      ln_rows_tile<ACT_GELU, true>(a.xb[blk - 1], a.y2[blk - 1], a.lw[blk - 1], a.lb[blk - 1],
                                   a.eps, a.xb[blk], n0 == 0, (const bf16_t*)a.w1[blk], a.ldw1,
                                   a.b1[blk], a.y1[blk], T, N, a.h, m0, n0);
    } else {
      const float* A;
      const bf16_t* W;
      long long lda, ldw;
      const float* bias;
      float* Cm;
      if (ph < 0) {
        A = a.o, lda = a.h, W = (const bf16_t*)a.wo, ldw = a.ldwo, bias = a.bo, Cm = a.xb[0];
      } else if (ph == 0) {
        A = a.xb[0], lda = a.h, W = (const bf16_t*)a.w1[0], ldw = a.ldw1, bias = a.b1[0];
        Cm = a.y1[0];
      } else {
        A = a.y1[blk], lda = a.he, W = (const bf16_t*)a.w2[blk], ldw = a.ldw2, bias = a.b2[blk];
        Cm = a.y2[blk];
      }
      const int K = ph > 0 ? a.he : a.h;
      ARow<1> arow[1];
      arow[0].p[0] = A + (long long)min(m0 + lo16, T - 1) * lda + 8 * hi4;
      if (ph == 0)
        f32a_tile<1, 4, 8, 4, ACT_GELU, 0, 1, true>(arow, W, ldw, bias, Cm, nullptr, N, T, N, K,
                                                    1.f, m0, n0);
      else
        f32a_tile<1, 4, 8, 4, ACT_NONE, 0, 1, true>(arow, W, ldw, bias, Cm, nullptr, N, T, N, K,
                                                    1.f, m0, n0);
    }
  }
  if (p + 1 < a.nph) {
    // every wave's write-through stores acknowledged before the count
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) tagged_count(a.sync + ((size_t)p * mt + rb) * kSyncStride, a.tag);
  }
}

bool gating_fused_supported(int T, int h, int he) {
  return T > 0 && h == he && h % 256 == 0 && h >= 256 && h <= 1024 &&
         (long long)((T + 15) / 16) * (h / 64) * 9 + T <= 0x7fffffffll;
}

// counters of up to 11 phases (value fold, out-projection, 8 block products, head)
size_t gating_fused_sync_words(int T) { return (size_t)11 * ((T + 15) / 16) * kSyncStride; }

hipError_t launch_gating_fused(GatingFusedArgs a, hipStream_t s) {
  if (!gating_fused_supported(a.T, a.h, a.he) || a.xb[0] == nullptr || a.sync == nullptr ||
      (uintptr_t)a.sync % 8 || (a.o != nullptr && a.wo == nullptr) || a.tag == 0 ||
      a.tag >= (1ull << 48))
    return hipErrorInvalidValue;
  for (int i = 0; i < 4; ++i)
    if (a.y1[i] == nullptr || a.y2[i] == nullptr || (i > 0 && a.xb[i] == nullptr))
      return hipErrorInvalidValue;
  const int mt = (a.T + 15) / 16, tiles = mt * (a.h / 64);
  int vf = 0;
  if (a.vf_part != nullptr) {
    vf = fold_value_merged_max_parts(a.T, a.vf_N, a.vf_Q);
    if (a.o == nullptr || a.vf_wv == nullptr || a.vf_bv == nullptr || a.vf_H < 1 ||
        a.h % a.vf_H || (a.h / a.vf_H) % 16 || vf < 1 || vf > 4 || (uintptr_t)a.vf_part % 16 ||
        (uintptr_t)a.vf_wv % 16 || a.vf_ldw < a.h || a.vf_ldw % 8 ||
        (long long)mt * ((a.h / a.vf_H + 63) / 64) * a.vf_H > 0x7fffffffll - 10ll * tiles - a.T)
      return hipErrorInvalidValue;
    if (vf < 2) vf = 2;
  }
  int n = 0, g = 0;
  if (vf > 0) a.first[n++] = g, g += mt * ((a.h / a.vf_H + 63) / 64) * a.vf_H;
  if (a.o != nullptr) a.first[n++] = g, g += tiles;
  for (int i = 0; i < 8; ++i) a.first[n++] = g, g += tiles;
  a.first[n++] = g, g += a.T;
  a.first[n] = g;
  a.nph = n;
  if (vf == 0)
    hipLaunchKernelGGL(k_gating_fused<0>, dim3((unsigned)g), dim3(512), 0, s, a);
  else if (vf == 2)
    hipLaunchKernelGGL(k_gating_fused<2>, dim3((unsigned)g), dim3(512), 0, s, a);
  else if (vf == 3)
    hipLaunchKernelGGL(k_gating_fused<3>, dim3((unsigned)g), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(k_gating_fused<4>, dim3((unsigned)g), dim3(512), 0, s, a);
  return hipGetLastError();
}

// ---- one layer's value fold and the next layer's query fold ------------------
// Workgroups [0, nA): value-fold tiles (64-column block, 16-tile row block,
// head), numbered as in k_fold_value_merged; [nA, nA + nB): query-fold blocks
// (row block, head), numbered as in k_fold_query_fused.  A query-fold
// workgroup waits for the counter of its row block, which every value-fold
// workgroup of that row block increments after its write-through stores of o
// are acknowledged; all of them come earlier in the launch order.
template <int MAXS, int D>
__global__ void __launch_bounds__(512) k_fold_value_query(FoldVQArgs a) {
  const int T = a.T, C = a.C, H = a.H, d = C / H;
  const int mt = (T + 15) / 16, nx = (d + 63) / 64;
  const int nA = nx * mt * H;
  const int bid = blockIdx.x;
  if (bid < nA) {
    const int wg = xcd_major(bid, nA);
    const int rb = (wg / nx) % mt;
    fold_value_tile<MAXS, true>(a.part, a.valid, a.N, a.Q, a.segmax, (const bf16_t*)a.Wv, a.ldwv,
                                a.bv, a.o, T, C, H, 64 * (wg % nx), 16 * rb, wg / (nx * mt));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) tagged_count(a.sync + (size_t)rb * kSyncStride, a.tag);
  } else {
    const int wg = xcd_major(bid - nA, mt * H);
    const int rb = wg % mt;
    if (threadIdx.x == 0)
      phase_wait(a.sync + (size_t)rb * kSyncStride, (a.tag << 16) | (unsigned long long)(nx * H),
                 a.status);
    __syncthreads();
    fold_query_tile<D, true>(a.o, C, (const bf16_t*)a.Wq, (const bf16_t*)a.Wq_lo, a.ldwq, a.bq,
                             (const bf16_t*)a.WkT, a.ldk, (bf16_t*)a.qt_hi, (bf16_t*)a.qt_lo, T,
                             C, a.scale, 16 * rb, wg / mt);
  }
}

bool fold_value_query_supported(int T, int N, int Q, int C, int H) {
  if (T <= 0 || H < 1 || H > 16 || C % H) return false;
  const int d = C / H, m = fold_value_merged_max_parts(T, N, Q);
  const long long mt = (T + 15) / 16;
  // the query fold's LDS next to the value fold's: head widths up to 64
  return (d == 32 || d == 64) && C % 128 == 0 && C <= 1024 && m >= 1 && m <= 4 &&
         mt * ((d + 63) / 64) * H + mt * H <= 0x7fffffffll;
}

size_t fold_value_query_sync_words(int T) { return (size_t)((T + 15) / 16) * kSyncStride; }

hipError_t launch_fold_value_query(const FoldVQArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (!fold_value_query_supported(a.T, a.N, a.Q, a.C, a.H) || !a.part || !a.Wv || !a.bv ||
      !a.o || !a.Wq || !a.Wq_lo || !a.bq || !a.WkT || !a.qt_hi || !a.qt_lo || !a.sync ||
      (uintptr_t)a.sync % 8 || a.tag == 0 || a.tag >= (1ull << 48) || (uintptr_t)a.part % 16 ||
      (uintptr_t)a.Wv % 16 || a.ldwv < a.C || a.ldwv % 8 || (uintptr_t)a.o % 16 ||
      (uintptr_t)a.Wq % 16 || (uintptr_t)a.Wq_lo % 16 || (uintptr_t)a.WkT % 16 ||
      (uintptr_t)a.qt_hi % 16 || (uintptr_t)a.qt_lo % 16 || a.ldwq < a.C || a.ldwq % 8 ||
      a.ldk < a.C || a.ldk % 8)
    return hipErrorInvalidValue;
  const int d = a.C / a.H, mt = (a.T + 15) / 16;
  const unsigned g = (unsigned)(mt * ((d + 63) / 64) * a.H + mt * a.H);
  int maxs = fold_value_merged_max_parts(a.T, a.N, a.Q);
  if (maxs < 2) maxs = 2;
#define IVC_FVQ(S, DV) hipLaunchKernelGGL((k_fold_value_query<S, DV>), dim3(g), dim3(512), 0, s, a)
  if (d == 32) {
    if (maxs == 2) IVC_FVQ(2, 32);
    else if (maxs == 3) IVC_FVQ(3, 32);
    else IVC_FVQ(4, 32);
  } else {
    if (maxs == 2) IVC_FVQ(2, 64);
    else if (maxs == 3) IVC_FVQ(3, 64);
    else IVC_FVQ(4, 64);
  }
#undef IVC_FVQ
  return hipGetLastError();
}

}  // namespace ivc
