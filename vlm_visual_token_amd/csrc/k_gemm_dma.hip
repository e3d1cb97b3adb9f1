// bf16 GEMM for the projector MLPs: C[M, N] = act(A[M, K] . W[N, K]^T + bias[N]).
//
// 256 x 256 output tile per workgroup, K step 64, 4 wavefronts of 128 x 128
// (a 4 x 4 grid of v_mfma_f32_32x32x16_bf16 blocks, 256 fp32 accumulators
// per lane, held in AGPRs).
//
// Operand tiles move from HBM/L2 to LDS with gfx950's LDS DMA
// (global_load_lds_dwordx4): no staging registers, so the VGPRs can hold a
// whole K step of MFMA fragments.  A DMA instruction writes one contiguous
// 1 KB block (64 lanes x 16 bytes), i.e. 8 tile rows of 128 bytes.  To keep
// the fragment reads (ds_read_b128, one row per lane) free of bank conflicts
// without padding, 16-byte chunk c of tile row r is stored at position
// c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1): any 8 consecutive rows (and any
// 16 consecutive rows split by parity) then land in distinct bank groups.
// Each lane of a DMA picks the global chunk that belongs at its fixed LDS
// position, so every 8 lanes still read one full 128-byte row of A or W.
//
// Two LDS stages (2 x 64 KB).  Each K step first reads all of its MFMA
// fragments from the current stage into registers, then issues the DMA of
// the next K step into the other stage, then runs its 64 MFMAs, which hide
// the DMA latency; one barrier per K step.  The finished tile goes out
// through LDS with 16-byte stores.
#include "common.h"
#include "kernels.h"

namespace ivc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;
typedef __attribute__((address_space(1))) const char gchar_t;

namespace {
constexpr int DBM = 256, DBN = 256, DBK = 64;
constexpr int DNT = 256;
constexpr int TILE_ELEMS = DBM * DBK;  // one operand tile, bf16 elements (32 KB)

IVC_DEV int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct Frags {
  bf16x8_t a[4], b[4];
};

// Per-lane LDS byte addresses of one K step's fragments: fragment (i, kk) of
// A sits at a_off[kk] + i * 4096 (rows i*32 + lane%32 of the wave's 128-row
// slice), since the swizzle term depends only on lane % 32.
struct FragAddr {
  uint32_t a_off[4], b_off[4];
};

IVC_DEV void read_frags(uint32_t sa, uint32_t sb, const FragAddr& fa, int kk, Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
        (uintptr_t)(sa + fa.a_off[kk] + i * 4096));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
        (uintptr_t)(sb + fa.b_off[kk] + j * 4096));
}

IVC_DEV void mma(const Frags& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// DMA one K step: the 8 A blocks and 8 W blocks of this wave.  a_base / b_base
// are the tile's first rows at this K step (uniform); offsets are per lane.
IVC_DEV void dma_tiles(gchar_t* a_base, gchar_t* b_base, const uint32_t* a_off,
                       const uint32_t* b_off, bf16_t* sa, bf16_t* sb, int w) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(a_base + a_off[j]),
                                     (lds_void_t*)(sa + (w * 8 + j) * 512), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(b_base + b_off[j]),
                                     (lds_void_t*)(sb + (w * 8 + j) * 512), 16, 0, 0);
  }
}
}  // namespace

template <int ACT>
__global__ void __launch_bounds__(DNT, 1)
k_gemm_dma(const bf16_t* __restrict__ A, long long lda, int a_rpg, long long a_gstride,
           int a_goff, const bf16_t* __restrict__ W, long long ldw,
           const float* __restrict__ bias, bf16_t* __restrict__ Cm, long long ldc, int M, int N,
           int K, RowMap rm) {
  __shared__ __attribute__((aligned(1024))) bf16_t sA0[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16_t sB0[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16_t sA1[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16_t sB1[TILE_ELEMS];

  // rows actually present (route-first products size the grid for all
  // tiles): the tile grid is laid out over those rows only, so the active
  // workgroups stay spread over all XCDs; the rest leave at once
  if (rm.m_dev != nullptr) M = min(M, *rm.m_dev * rm.m_mult);
  const int tiles_m = (M + DBM - 1) / DBM, tiles_n = (N + DBN - 1) / DBN;
  const int nb = tiles_m * tiles_n;
  if ((int)blockIdx.x >= nb) return;  // uniform over the workgroup, before any barrier
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);  // consecutive ids on one XCD
  constexpr int GM = 8;
  const int in_group = GM * tiles_n;
  const int first_m = (bid / in_group) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int pid_m = first_m + (bid % in_group) % gsize;
  const int pid_n = (bid % in_group) / gsize;
  const int m0 = pid_m * DBM, n0 = pid_n * DBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;

  // DMA sources: load j of wave w fills tile rows (w*8 + j)*8 .. +7; lane
  // takes row + lane/8 and the global chunk that belongs at position lane%8.
  // Byte offsets are relative to the tile's first row (A rows may be
  // remapped, so that row's physical index is computed like the others).
  auto phys_a = [&](int gm) -> long long {
    return a_rpg > 0 ? (long long)(gm / a_rpg) * a_gstride + a_goff + gm % a_rpg : (long long)gm;
  };
  const long long a_row0 = phys_a(m0);
  // global-address-space bases: the DMA then takes a uniform base plus a
  // 32-bit per-lane offset (one VGPR per load)
  gchar_t* a_tile = (gchar_t*)(A + a_row0 * lda);
  gchar_t* b_tile = (gchar_t*)(W + (long long)n0 * ldw);
  uint32_t a_off[8], b_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (w * 8 + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    const int gm = min(m0 + r, M - 1);
    a_off[j] = (uint32_t)(((phys_a(gm) - a_row0) * lda + c * 8) * 2);
    const int gn = min(n0 + r, N - 1);
    b_off[j] = (uint32_t)(((long long)(gn - n0) * ldw + c * 8) * 2);
  }
  // fragment addresses (bytes within a stage array)
  FragAddr fa;
  {
    const int rl = lane & 31, half = lane >> 5, sw = swz(rl);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t p = (uint32_t)(((2 * kk + half) ^ sw) * 16);
      fa.a_off[kk] = (uint32_t)((wm * 128 + rl) * 128) + p;
      fa.b_off[kk] = (uint32_t)((wn * 128 + rl) * 128) + p;
    }
  }
  const uint32_t la0 = (uint32_t)(uintptr_t)(lds_void_t*)sA0, lb0 = (uint32_t)(uintptr_t)(lds_void_t*)sB0;
  const uint32_t la1 = (uint32_t)(uintptr_t)(lds_void_t*)sA1, lb1 = (uint32_t)(uintptr_t)(lds_void_t*)sB1;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = K / DBK;
  const long long kstep = DBK * 2;  // bytes per K step along a row
  dma_tiles(a_tile, b_tile, a_off, b_off, sA0, sB0, w);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool odd = kt & 1;
    const uint32_t la = odd ? la1 : la0, lb = odd ? lb1 : lb0;
    // all fragments of this K step first ...
    Frags f[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) read_frags(la, lb, fa, kk, f[kk]);
    // ... then the DMA of the next step into the other stage, hidden by the MFMAs
    if (kt + 1 < KT) {
      const long long ko = (long long)(kt + 1) * kstep;
      if (odd) dma_tiles(a_tile + ko, b_tile + ko, a_off, b_off, sA0, sB0, w);
      else dma_tiles(a_tile + ko, b_tile + ko, a_off, b_off, sA1, sB1, w);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) mma(f[kk], acc);
    // keep the MFMAs above the wait: otherwise they sink below the barrier
    // and the DMA latency is no longer hidden
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Epilogue through LDS: the 256 x 256 bf16 tile (128 KB; rows 64q .. 64q+63
  // in stage array q of sA0, sB0, sA1, sB1) is written from the accumulators,
  // then stored with 16-byte row-contiguous writes (2-byte stores straight
  // from the accumulator layout reach a fraction of the write bandwidth).
  // 32x32 accumulator layout: lane l holds column l % 32 and rows
  // 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  {
    char* slab_lo = wm ? (char*)sA1 : (char*)sA0;
    char* slab_hi = wm ? (char*)sB1 : (char*)sB0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = wn * 128 + j * 32 + (lane & 31);
      const int col = n0 + cl;
      const float bj = (bias != nullptr && col < N) ? bias[col] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        char* slab = i < 2 ? slab_lo : slab_hi;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = (i & 1) * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);  // row in slab
          float x = acc[i][j][v] + bj;
          if (ACT == ACT_GELU) x = gelu_erf(x);
          *reinterpret_cast<bf16_t*>(slab + rl * 512 + cl * 2) = f32_to_bf16(x);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int r = it * 8 + (tid >> 5), c = tid & 31;
    const char* slab = it < 8 ? (const char*)sA0 : it < 16 ? (const char*)sB0
                     : it < 24 ? (const char*)sA1 : (const char*)sB1;
    const u32x4 val = *reinterpret_cast<const u32x4*>(slab + (r & 63) * 512 + c * 16);
    const int row = m0 + r, col = n0 + 8 * c;
    if (row < M && col < N) {
      const long long orow =
          rm.c_map != nullptr ? (long long)rm.c_map[row / rm.c_rpg] * rm.c_rpg + row % rm.c_rpg
                              : row;
      *reinterpret_cast<u32x4*>(Cm + orow * ldc + col) = val;
    }
  }
}

bool gemm_dma_supported(const GemmArgs& g) {
  return g.a_dtype == DT_BF16 && g.w_dtype == DT_BF16 && g.c_dtype == DT_BF16 && g.K % DBK == 0 &&
         g.K > 0 && g.M > 0 && g.N > 0 && g.lda % 8 == 0 && g.ldw % 8 == 0 &&
         ((uintptr_t)g.A % 16) == 0 && ((uintptr_t)g.W % 16) == 0 && g.N % 8 == 0 &&
         g.ldc % 8 == 0 && ((uintptr_t)g.Cm % 16) == 0;
}

hipError_t launch_gemm_dma(const GemmArgs& g, hipStream_t s) {
  if (!gemm_dma_supported(g)) return hipErrorInvalidValue;
  const int tiles = ((g.M + DBM - 1) / DBM) * ((g.N + DBN - 1) / DBN);
  if (g.act == ACT_GELU)
    hipLaunchKernelGGL(k_gemm_dma<ACT_GELU>, dim3((unsigned)tiles), dim3(DNT), 0, s,
                       (const bf16_t*)g.A, g.lda, g.a_rpg, g.a_gstride, g.a_goff,
                       (const bf16_t*)g.W, g.ldw, g.bias, (bf16_t*)g.Cm, g.ldc, g.M, g.N, g.K, g.rm);
  else
    hipLaunchKernelGGL(k_gemm_dma<ACT_NONE>, dim3((unsigned)tiles), dim3(DNT), 0, s,
                       (const bf16_t*)g.A, g.lda, g.a_rpg, g.a_gstride, g.a_goff,
                       (const bf16_t*)g.W, g.ldw, g.bias, (bf16_t*)g.Cm, g.ldc, g.M, g.N, g.K, g.rm);
  return hipGetLastError();
}

}  // namespace ivc
