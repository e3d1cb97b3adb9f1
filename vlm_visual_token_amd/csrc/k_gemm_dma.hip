// bf16 GEMM for the projector MLPs: C[M, N] = act(A[M, K] . W[N, K]^T + bias[N]).
//
// 256 x 256 output tile per workgroup, 8 wavefronts of 128 x 64 (a 4 x 2
// grid of v_mfma_f32_32x32x16_bf16 blocks, 128 fp32 accumulators per lane),
// two wavefronts per SIMD.  Operand tiles move from HBM/L2 to LDS with gfx950's LDS
// DMA (global_load_lds_dwordx4): no staging registers, so the VGPRs hold the
// MFMA fragments.  A DMA instruction writes one contiguous 1 KB block (64
// lanes x 16 bytes); each lane picks the global 16-byte piece that belongs at
// its fixed LDS position, which lets the tiles be stored XOR-swizzled, so the
// fragment reads (ds_read_b128, one row per lane) are free of bank conflicts
// without padding.
//
// Main loop: K step 64, two stages of 64 KB (A and W, 256 rows of 128 bytes
// each): full 128-byte rows per DMA request.  The next step's DMA
// instructions go out over the first half of the step's MFMAs and the next
// sub-step's fragment reads are interleaved with them.  (A four-stage ring
// of K step 32 was measured slower on every shape here: its 64-byte row
// requests cost more than the deeper prefetch gains.)
// The compiler must not make an LDS read wait for the DMAs in flight: each
// stage is a separate __shared__ array (the compiler tracks LDS DMA targets
// per array).
//
// Epilogue: the 256 x 256 bf16 tile goes through LDS (the four 32 KB stage
// arrays hold 64 rows each) and out with 16-byte row-contiguous stores;
// 2-byte stores straight from the accumulator layout reach only a fraction
// of the write bandwidth.
//
// LayerNorm fold (FOLD): for the first Linear after a LayerNorm,
//   LN(x) W^T + b = rstd * (x . (gamma o W)^T) - rstd * mean * colsum(gamma o W) + (b + W beta),
// so A is the raw ViT rows, gathered in pixel-shuffle order by the DMA
// addresses (each K step of 64 lies inside one C-wide cell, and a cell's row
// offset within its grid block is the same for every token, so the gather
// costs one scalar offset per step), and the epilogue applies the per-row
// (mean, rstd) and per-column colsum.  The normalised rows are never written.
//
// Grid: workgroups are dealt round-robin to the 8 XCDs, so the linear id is
// regrouped so consecutive tile ids land on one XCD, then tiles are walked in
// bands of 8 tile-rows so an XCD's L2 sees the same A and W rows many times.
// Route-first products read their row count from the device (RowMap) and lay
// the tile grid over the rows present.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ivc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;
typedef __attribute__((address_space(1))) const char gchar_t;

namespace {
constexpr int DBM = 256, DBN = 256, DNT = 512;  // tile rows, columns; threads
constexpr int QB = 32768;  // bytes of one stage array (also one epilogue slab of 64 rows)

// Tile of this workgroup; false if it has none (uniform, before any barrier).
IVC_DEV bool map_tile(int& M, int N, const RowMap& rm, int& m0, int& n0) {
  if (rm.m_dev != nullptr) M = min(M, *rm.m_dev * rm.m_mult);
  const int tiles_m = (M + DBM - 1) / DBM, tiles_n = (N + DBN - 1) / DBN;
  const int nb = tiles_m * tiles_n;
  if ((int)blockIdx.x >= nb) return false;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);  // consecutive ids on one XCD
  constexpr int GM = 8;
  const int in_group = GM * tiles_n;
  const int first_m = (bid / in_group) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  m0 = (first_m + (bid % in_group) % gsize) * DBM;
  n0 = ((bid % in_group) / gsize) * DBN;
  return true;
}

IVC_DEV long long phys_row(int gm, int a_rpg, long long a_gstride, int a_goff) {
  return a_rpg > 0 ? (long long)(gm / a_rpg) * a_gstride + a_goff + gm % a_rpg : (long long)gm;
}

// Gathered A: ViT row of cell 0 of logical row m's grid block.
IVC_DEV long long gather_row0(const AGather& g, int m) {
  const int Q = g.P / g.r, S = Q * Q;
  const int rank = m / S, s = m - rank * S;
  const int t = g.list != nullptr ? g.list[rank] : rank;
  const int qa = s / Q, qb = s - qa * Q;
  const int a = g.v1 ? qb : qa, b = g.v1 ? qa : qb;  // v1: token (a, b) sits at b*Q + a
  return (long long)t * g.rows + g.has_cls + (long long)(g.r * a) * g.P + g.r * b;
}

// Gathered A: byte offset of channels [c0, c0 + BK) of cell q relative to
// cell 0's row (r is 2 or 4, so the cell's grid offset is shifts and masks;
// the main loop steps (q, c0) along K without dividing).
IVC_DEV long long gather_koff(const AGather& g, int q, int c0) {
  int dm, dk;  // grid offset of cell q inside the block
  if (g.twice) {  // r = 4 as two r = 2 shuffles: q = 4*(2*m2 + k2) + (2*m + k)
    const int w = q >> 2, qq = q & 3;
    dm = 2 * (w >> 1) + (qq >> 1);
    dk = 2 * (w & 1) + (qq & 1);
  } else {
    const int sh = g.r == 4 ? 2 : 1;
    dm = q >> sh;
    dk = q & (g.r - 1);
  }
  return ((long long)(dm * g.P + dk) * g.C + c0) * 2;
}

// Byte XOR applied to a column offset in row r of an epilogue slab: one
// 4-byte write instruction covers rows R, R+1, R+4, R+5 and 64 bytes of
// columns, which this spreads over all 64 LDS banks (a permutation of the
// 16-byte pieces within the row, so the 16-byte reads stay conflict-free).
IVC_DEV int slab_swz(int r) { return ((r & 1) | ((r >> 1) & 2)) << 6; }

// Writes the 256 x 256 tile (bias, activation, bf16) through LDS slabs
// q0..q3 (rows 64s .. 64s+63 in slab s, 512 bytes per row) to C.
// 32x32 accumulator layout: lane l holds column l % 32 and rows
// 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.  Values v, v+1 (rows R, R+1) are
// converted together (v_cvt_pk_bf16_f32) and traded with the neighbouring
// lane (column c ^ 1), so the even lane writes row R, columns c, c+1 and the
// odd lane row R+1, columns c-1, c: one 4-byte LDS write per two values.
// FOLD: value = rstd_row * acc - rstd_row * mean_row * colsum[col] + bias[col],
// with the tile's 256 (mean, rstd) pairs staged in LDS first.
// NJ: 32-column blocks per wave (4: waves of 128 x 128, 4 per tile; 2: waves
// of 128 x 64, 8 per tile); NTH: threads of the workgroup.
template <int ACT, bool FOLD, int NJ = 2, int NTH = DNT>
IVC_DEV void store_tile(const f32x16_t (&acc)[4][NJ], char* q0, char* q1, char* q2, char* q3,
                        int wm, int wn, int m0, int n0, int M, int N, const float* bias,
                        bf16_t* Cm, long long ldc, const RowMap& rm, const float* ln_rows,
                        const float* ln_colsum) {
  constexpr int WC = 32 * NJ;  // columns per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const bool odd_lane = lane & 1;
  __shared__ float2 rowst[FOLD ? DBM : 1];  // (rstd, -rstd * mean) per tile row
  float ccol[NJ];
  if (FOLD) {
    if (tid < DBM) {
      const int row = min(m0 + tid, M - 1);
      const float2 mr = *reinterpret_cast<const float2*>(ln_rows + 2 * (long long)row);
      rowst[tid] = make_float2(mr.y, -mr.y * mr.x);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + wn * WC + j * 32 + (lane & 31);
      ccol[j] = col < N ? ln_colsum[col] : 0.f;
    }
    __syncthreads();
  }
  // v_perm_b32 selectors: even lane keeps its low half and takes the
  // neighbour's low half; odd lane takes the neighbour's high half and keeps
  // its own high half
  const uint32_t sel = odd_lane ? 0x07060302u : 0x05040100u;
  {
    char* slab_lo = wm ? q2 : q0;
    char* slab_hi = wm ? q3 : q1;
    float bcol[NJ];  // all loads in flight together
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + wn * WC + j * 32 + (lane & 31);
      bcol[j] = (bias != nullptr && col < N) ? bias[col] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int cl = wn * WC + j * 32 + (lane & 31);
      const float bj = bcol[j];
      const int cw = cl & ~1;  // column of the pair this lane writes
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        char* slab = i < 2 ? slab_lo : slab_hi;
        float2 rs[16];  // this lane's 16 rows of block row i, read together
        if (FOLD) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            rs[v] = rowst[wm * 128 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)];
        }
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float x0, x1;
          if (FOLD) {
            x0 = fmaf(rs[v].x, acc[i][j][v], fmaf(rs[v].y, ccol[j], bj));
            x1 = fmaf(rs[v + 1].x, acc[i][j][v + 1], fmaf(rs[v + 1].y, ccol[j], bj));
          } else {
            x0 = acc[i][j][v] + bj;
            x1 = acc[i][j][v + 1] + bj;
          }
          if (ACT == ACT_GELU) {
            x0 = gelu_erf(x0);
            x1 = gelu_erf(x1);
          }
          const uint32_t own = __builtin_bit_cast(
              uint32_t, __builtin_convertvector((f32x2_t){x0, x1}, bf16x2_t));  // rows R, R+1
          const uint32_t nbr = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);
          const uint32_t pair = __builtin_amdgcn_perm(odd_lane ? own : nbr, odd_lane ? nbr : own, sel);
          const int rl = (i & 1) * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3) + (odd_lane ? 1 : 0);
          *reinterpret_cast<uint32_t*>(slab + rl * 512 + ((cw * 2) ^ slab_swz(rl))) = pair;
        }
      }
    }
  }
  __syncthreads();
  // output row of tile row r (route-first products scatter groups of c_rpg rows)
  const bool pow2 = rm.c_map != nullptr && (rm.c_rpg & (rm.c_rpg - 1)) == 0;
  const int sh = pow2 ? __builtin_ctz((unsigned)rm.c_rpg) : 0;
  constexpr int RPI = NTH / 32;  // rows per iteration (32 threads x 16 bytes per row)
#pragma unroll 4
  for (int it = 0; it < DBM / RPI; ++it) {
    const int r = it * RPI + (tid >> 5), c = tid & 31;
    const int sl = r >> 6;
    const char* slab = sl == 0 ? q0 : sl == 1 ? q1 : sl == 2 ? q2 : q3;
    const u32x4 val =
        *reinterpret_cast<const u32x4*>(slab + (r & 63) * 512 + ((c * 16) ^ slab_swz(r & 63)));
    const int row = m0 + r, col = n0 + 8 * c;
    if (row < M && col < N) {
      long long orow = row;
      if (pow2)
        orow = ((long long)rm.c_map[row >> sh] << sh) + (row & (rm.c_rpg - 1));
      else if (rm.c_map != nullptr)
        orow = (long long)rm.c_map[row / rm.c_rpg] * rm.c_rpg + row % rm.c_rpg;
      *reinterpret_cast<u32x4*>(Cm + orow * ldc + col) = val;
    }
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// The kernel: K step 64, two stages; sA*/sB* hold 256 rows of 128 bytes, and
// 16-byte piece c of row r sits at c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1).
// 8 waves of 128 x 64 (4 x 2 MFMA blocks, 128 accumulators each), two per
// SIMD, so while one wave of a SIMD waits to issue its share of the operand
// DMA the other issues MFMAs (4 waves of 128 x 128 with all 256 AGPRs were
// 3-8% slower: nothing could cover their DMA issue stalls).  Each wave
// issues 8 of the step's 64 DMA instructions over the first half of the
// step's MFMAs.
// ---------------------------------------------------------------------------
template <int ACT, bool FOLD>
__global__ void __launch_bounds__(DNT, 1)
k_gemm_dma8(const bf16_t* __restrict__ A, long long lda, int a_rpg, long long a_gstride,
            int a_goff, const bf16_t* __restrict__ W, long long ldw,
            const float* __restrict__ bias, bf16_t* __restrict__ Cm, long long ldc, int M, int N,
            int K, RowMap rm, AGather ag, const float* __restrict__ ln_rows,
            const float* __restrict__ ln_colsum) {
  constexpr int BK = 64;
  // A offsets relative to the tile's first row are never negative (the tile's
  // rows come in increasing ViT row order, gathered or not), so they stay
  // unsigned 32-bit and the DMA takes a scalar base plus a 32-bit offset
  using aoff_t = uint32_t;
  __shared__ __attribute__((aligned(1024))) char sA0[QB];
  __shared__ __attribute__((aligned(1024))) char sB0[QB];
  __shared__ __attribute__((aligned(1024))) char sA1[QB];
  __shared__ __attribute__((aligned(1024))) char sB1[QB];
  int m0, n0;
  if (!map_tile(M, N, rm, m0, n0)) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0..7
  const int wm = w >> 2, wn = w & 3;  // rows wm*128 .., columns wn*64 ..

  // DMA j (0..3) of wave w fills rows (4w + j)*8 .. +7 of A and of W; lane:
  // row + lane/8, LDS piece lane%8 holding global piece (lane%8) ^ f(row)
  const long long a_row0 = FOLD ? gather_row0(ag, m0) : phys_row(m0, a_rpg, a_gstride, a_goff);
  gchar_t* a_tile = (gchar_t*)(A + a_row0 * lda);
  gchar_t* b_tile = (gchar_t*)(W + (long long)n0 * ldw);
  aoff_t a_off[4];
  uint32_t b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (w * 4 + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r & 7) ^ ((r >> 3) & 1));
    const int gm = min(m0 + r, M - 1);
    const long long pr = FOLD ? gather_row0(ag, gm) : phys_row(gm, a_rpg, a_gstride, a_goff);
    a_off[j] = (aoff_t)(((pr - a_row0) * lda + c * 8) * 2);
    b_off[j] = (uint32_t)(((long long)(min(n0 + r, N - 1) - n0) * ldw + c * 8) * 2);
  }
  auto dma_one = [&](int q, long long ka, long long kb, char* sa, char* sb) {  // q = 0..7
    const int j = q >> 1;
    if ((q & 1) == 0)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(a_tile + ka + a_off[j]),
                                       (lds_void_t*)(sa + (w * 4 + j) * 1024), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(b_tile + kb + b_off[j]),
                                       (lds_void_t*)(sb + (w * 4 + j) * 1024), 16, 0, 0);
  };
  // fragment (i, kk) of A at fa[kk] + i * 4096 (rows wm*128 + i*32 + lane%32),
  // of W at fb[kk] + j * 4096 (rows wn*64 + j*32 + lane%32)
  uint32_t fa[4], fb[4];
  {
    const int rl = lane & 31, sw = (rl & 7) ^ ((rl >> 3) & 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t p = (uint32_t)(((2 * kk + (lane >> 5)) ^ sw) * 16);
      fa[kk] = (uint32_t)((wm * 128 + rl) * 128) + p;
      fb[kk] = (uint32_t)((wn * 64 + rl) * 128) + p;
    }
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = K / BK;
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_one(q, FOLD ? gather_koff(ag, 0, 0) : 0, 0, sA0, sB0);
  int cell_n = 0, c0_n = 0;  // (cell, channel) of the next K step (FOLD)
  for (int kt = 0; kt < KT; ++kt) {
    const bool odd = kt & 1;
    const char* sa = odd ? sA1 : sA0;
    const char* sb = odd ? sB1 : sB0;
    char* na = odd ? sA0 : sA1;
    char* nb = odd ? sB0 : sB1;
    const bool more = kt + 1 < KT;
    const long long kb = (long long)(kt + 1) * (BK * 2);
    if (FOLD) {
      c0_n += BK;
      if (c0_n == ag.C) {
        c0_n = 0;
        ++cell_n;
      }
    }
    const long long ka = FOLD ? gather_koff(ag, cell_n, c0_n) : kb;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    bf16x8_t fa_[2][4], fb_[2][2];  // [buffer][block]
#pragma unroll
    for (int i = 0; i < 4; ++i) fa_[0][i] = *reinterpret_cast<const bf16x8_t*>(sa + fa[0] + i * 4096);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb_[0][j] = *reinterpret_cast<const bf16x8_t*>(sb + fb[0] + j * 4096);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cb = kk & 1, nbuf = cb ^ 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // 8 DMA instructions over the first 16 MFMAs of the step
          if (more && kk < 2 && j == 0) dma_one(kk * 4 + i, ka, kb, na, nb);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_[cb][i], fb_[cb][j], acc[i][j],
                                                              0, 0, 0);
        }
        if (kk < 3) {
          fa_[nbuf][i] = *reinterpret_cast<const bf16x8_t*>(sa + fa[kk + 1] + i * 4096);
          if (i < 2) fb_[nbuf][i] = *reinterpret_cast<const bf16x8_t*>(sb + fb[kk + 1] + i * 4096);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  store_tile<ACT, FOLD, 2, DNT>(acc, sA0, sB0, sA1, sB1, wm, wn, m0, n0, M, N, bias, Cm, ldc,
                                    rm, ln_rows, ln_colsum);
}

// One workgroup per output n: the folded weights of the first Linear after a
// LayerNorm, the column sum the epilogue subtracts, and the folded bias.
__global__ void __launch_bounds__(256)
k_ln_fold_weights(const bf16_t* __restrict__ W, int K, const float* __restrict__ gamma,
                  const float* __restrict__ beta, const float* __restrict__ b,
                  bf16_t* __restrict__ Wg, float* __restrict__ colsum, float* __restrict__ bfold) {
  const int n = blockIdx.x, tid = threadIdx.x;
  const bf16_t* wr = W + (long long)n * K;
  bf16_t* gr = Wg + (long long)n * K;
  float s = 0.f, c = 0.f;
  for (int k = tid; k < K; k += 256) {
    const float wv = bf16_to_f32(wr[k]);
    const bf16_t g = f32_to_bf16(gamma[k] * wv);
    gr[k] = g;
    s += bf16_to_f32(g);
    c = fmaf(beta[k], wv, c);
  }
  __shared__ float rs[256], rc[256];
  rs[tid] = s;
  rc[tid] = c;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      rs[tid] += rs[tid + o];
      rc[tid] += rc[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    colsum[n] = rs[0];
    bfold[n] = b[n] + rc[0];
  }
}

hipError_t launch_ln_fold_weights(const void* W, int N, int K, const float* gamma,
                                  const float* beta, const float* b, void* Wg, float* colsum,
                                  float* bfold, hipStream_t s) {
  if (N <= 0 || K <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_ln_fold_weights, dim3((unsigned)N), dim3(256), 0, s, (const bf16_t*)W, K,
                     gamma, beta, b, (bf16_t*)Wg, colsum, bfold);
  return hipGetLastError();
}

bool gemm_dma_supported(const GemmArgs& g) {
  const bool base =
      g.a_dtype == DT_BF16 && g.w_dtype == DT_BF16 && g.c_dtype == DT_BF16 && g.K % 64 == 0 &&
      g.K > 0 && g.M > 0 && g.N > 0 && g.lda % 8 == 0 && g.ldw % 8 == 0 &&
      ((uintptr_t)g.A % 16) == 0 && ((uintptr_t)g.W % 16) == 0 && g.N % 8 == 0 &&
      g.ldc % 8 == 0 && ((uintptr_t)g.Cm % 16) == 0;
  if (!base || !g.fold) return base;
  // gathered A: C-wide cells hold whole K steps; K = r*r*C; lda = C; signed
  // 32-bit offsets inside the gathered tensor; row statistics and colsum given
  const AGather& a = g.ag;
  return (a.r == 2 || (a.r == 4)) && a.C > 0 && a.C % 64 == 0 && g.K == a.r * a.r * a.C &&
         g.lda == a.C && a.P % a.r == 0 && (!a.twice || a.r == 4) && g.ln_rows != nullptr &&
         g.ln_colsum != nullptr && g.a_rpg == 0 &&
         (long long)a.rows * a.C * 2 * ((long long)g.M / ((a.P / a.r) * (a.P / a.r)) + 1) <
             (1ll << 31);
}

hipError_t launch_gemm_dma(const GemmArgs& g, hipStream_t s) {
  if (!gemm_dma_supported(g)) return hipErrorInvalidValue;
  const int tiles = ((g.M + DBM - 1) / DBM) * ((g.N + DBN - 1) / DBN);
#define IVC_DMA_LAUNCH(KERN)                                                                  \
  hipLaunchKernelGGL(KERN, dim3((unsigned)tiles), dim3(DNT), 0, s, (const bf16_t*)g.A,    \
                     g.lda, g.a_rpg, g.a_gstride, g.a_goff, (const bf16_t*)g.W, g.ldw, g.bias,\
                     (bf16_t*)g.Cm, g.ldc, g.M, g.N, g.K, g.rm, g.ag, g.ln_rows, g.ln_colsum)
  if (g.fold) {  // the folded products are the GELU'd first Linears
    if (g.act != ACT_GELU) return hipErrorInvalidValue;
    IVC_DMA_LAUNCH((k_gemm_dma8<ACT_GELU, true>));
  } else if (g.act == ACT_GELU) {
    IVC_DMA_LAUNCH((k_gemm_dma8<ACT_GELU, false>));
  } else {
    IVC_DMA_LAUNCH((k_gemm_dma8<ACT_NONE, false>));
  }
#undef IVC_DMA_LAUNCH
  return hipGetLastError();
}

}  // namespace ivc
