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
// Main loop: K step 64, full 128-byte rows per DMA request; three LDS
// stages of A (32 KB each, DMA two steps ahead) and two of W (one step
// ahead), 160 KB.  The DMA instructions go out over the first half of the
// step's MFMAs and the next sub-step's fragment reads are interleaved with
// them.  (A four-stage ring of K step 32 was measured slower on every shape
// here: its 64-byte row requests cost more than the deeper prefetch gains.)
// The compiler must not make an LDS read wait for the DMAs in flight: each
// stage is a separate __shared__ array, and the loop is unrolled over the
// stages' cycle so each step names its arrays directly (the compiler tracks
// LDS DMA targets per array, and only when it can tell which one).
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
#include "index_math.h"
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

// Output tile t of the band order: bands of 8 tile rows, each walked column
// by column, so tiles with nearby indices share A and W panels.
IVC_DEV void band_tile(int t, int tiles_m, int tiles_n, int& m0, int& n0) {
  constexpr int GM = 8;
  const int in_group = GM * tiles_n;
  const int first_m = (t / in_group) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  m0 = (first_m + (t % in_group) % gsize) * DBM;
  n0 = ((t % in_group) / gsize) * DBN;
}

// Tile of this workgroup; false if it has none (uniform, before any barrier).
IVC_DEV bool map_tile(int& M, int N, const RowMap& rm, int& m0, int& n0) {
  if (rm.m_dev != nullptr) M = min(M, *rm.m_dev * rm.m_mult);
  const int tiles_m = (M + DBM - 1) / DBM, tiles_n = (N + DBN - 1) / DBN;
  const int nb = tiles_m * tiles_n;
  if ((int)blockIdx.x >= nb) return false;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);  // consecutive ids on one XCD
  band_tile(bid, tiles_m, tiles_n, m0, n0);
  return true;
}

IVC_DEV long long phys_row(int gm, int a_rpg, long long a_gstride, int a_goff) {
  return a_rpg > 0 ? (long long)(gm / a_rpg) * a_gstride + a_goff + gm % a_rpg : (long long)gm;
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
// With a row map each tile row's output row (and, with d_map, its second
// destination) is looked up once, into LDS at rmap, while the first phase
// runs; the store loop then reads it from there.
// NJ: 32-column blocks per wave (4: waves of 128 x 128, 4 per tile; 2: waves
// of 128 x 64, 8 per tile); NTH: threads of the workgroup.
template <int ACT, bool FOLD, int NJ = 2, int NTH = DNT>
IVC_DEV void store_tile(const f32x16_t (&acc)[4][NJ], char* q0, char* q1, char* q2, char* q3,
                        int wm, int wn, int m0, int n0, int M, int N, const float* bias,
                        bf16_t* Cm, long long ldc, const RowMap& rm, const float* ln_rows,
                        const float* ln_colsum, float2* rowst /* FOLD: [256] in LDS */,
                        char* rmap /* row map: 256 * 12 bytes of LDS */) {
  constexpr int WC = 32 * NJ;  // columns per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const bool odd_lane = lane & 1;
  long long* orow_s = reinterpret_cast<long long*>(rmap);    // [256] output row
  int* dj_s = reinterpret_cast<int*>(rmap + DBM * 8);         // [256] second destination
  if (rm.c_map != nullptr) {
    for (int r = tid; r < DBM; r += NTH) {
      const int row = min(m0 + r, M - 1);
      const int ot = rm.c_map[row / rm.c_rpg], slot = row % rm.c_rpg;
      orow_s[r] = (long long)ot * rm.c_rpg + slot;
      if (rm.d_map != nullptr) dj_s[r] = rm.d_map[(long long)ot * rm.d_stride + slot];
    }
  }
  // rowst: (rstd, -rstd * mean) per tile row
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
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float x0, x1;
          if (FOLD) {
            // the row pair's (rstd, -rstd * mean), read as needed (16 pairs read
            // ahead would hold 32 more registers at the kernel's peak)
            const float2* rp = rowst + wm * 128 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
            const float2 r0 = rp[0], r1 = rp[1];
            x0 = fmaf(r0.x, acc[i][j][v], fmaf(r0.y, ccol[j], bj));
            x1 = fmaf(r1.x, acc[i][j][v + 1], fmaf(r1.y, ccol[j], bj));
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
      // output row of tile row r (route-first products scatter groups of c_rpg rows)
      const long long orow = rm.c_map != nullptr ? orow_s[r] : (long long)row;
      *reinterpret_cast<u32x4*>(Cm + orow * ldc + col) = val;
      if (rm.d_map != nullptr) {  // the same row in its place in the compacted sequence
        const int dj = dj_s[r];
        if (dj >= 0)
          *reinterpret_cast<u32x4*>(reinterpret_cast<bf16_t*>(rm.d_out) + (long long)dj * ldc + col) =
              val;
      }
    }
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// The main loop: K step 64; sA*/sB* hold 256 rows of 128 bytes, and 16-byte
// piece c of row r sits at c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1).
// 8 waves of 128 x 64 (4 x 2 MFMA blocks, 128 accumulators each), two per
// SIMD (4 waves of 128 x 128 with all 256 AGPRs were 3-8% slower: nothing
// could cover their DMA issue stalls).  The two waves of a SIMD take turns:
// one runs a half step's 16 MFMAs while the other reads its next half
// step's fragments and issues its share of the operand DMA (tile_ksteps).
// ---------------------------------------------------------------------------
constexpr int BK = 64;

struct GemmOps {
  const bf16_t* A;
  long long lda;
  int a_rpg;
  long long a_gstride;
  int a_goff;
  const bf16_t* W;
  long long ldw;
  int M, N, K;
  AGather ag;
};

// Per-wave DMA addressing of one output tile: A rows from a scalar base plus
// unsigned 32-bit offsets.  The offsets are never negative: plain A is
// addressed from the tile's first row, gathered A from the first grid row of
// the first row's ViT tile (gather_base), which no later row of the tile
// precedes.
struct TileDma {
  __amdgpu_buffer_rsrc_t a_rs, b_rs;  // buffers based at the tile's base rows
  uint32_t a_off[4];
  uint32_t b_off[4];
};

// Raw buffer over [base, base + 4 GiB): the DMA takes the tile's base from
// scalar registers, a 32-bit offset per lane and the K step's offset as a
// scalar, so no 64-bit address is formed or kept per lane.
IVC_DEV __amdgpu_buffer_rsrc_t raw_buffer(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xffffffff,
                                           0x00020000);
}

template <bool FOLD>
IVC_DEV TileDma tile_dma(const GemmOps& o, int m0, int n0, int w, int lane) {
  TileDma d;
  // DMA j (0..3) of wave w fills rows (4w + j)*8 .. +7 of A and of W; lane:
  // row + lane/8, LDS piece lane%8 holding global piece (lane%8) ^ f(row)
  const long long a_row0 =
      FOLD ? gather_base(o.ag, m0) : phys_row(m0, o.a_rpg, o.a_gstride, o.a_goff);
  d.a_rs = raw_buffer(o.A + a_row0 * o.lda);
  d.b_rs = raw_buffer(o.W + (long long)n0 * o.ldw);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (w * 4 + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r & 7) ^ ((r >> 3) & 1));
    const int gm = min(m0 + r, o.M - 1);
    const long long pr =
        FOLD ? gather_row0(o.ag, gm) : phys_row(gm, o.a_rpg, o.a_gstride, o.a_goff);
    d.a_off[j] = (uint32_t)(((pr - a_row0) * o.lda + c * 8) * 2);
    d.b_off[j] = (uint32_t)(((long long)(min(n0 + r, o.N - 1) - n0) * o.ldw + c * 8) * 2);
  }
  return d;
}

// LDS stages of the main loop: A and W tiles of one K step each (32 KB):
// three of A (its DMAs run two steps ahead) and two of W (one step ahead),
// 160 KB, the CU's whole LDS.  A is the operand whose lines an XCD's L2 sees
// fewer times (a band of 8 tile rows by 4 tile columns runs on an XCD at
// once: each A panel is read by 4 tiles, each W panel by 8), so it takes the
// L2 misses and gets the deeper prefetch (measured: 5-11% faster than two
// stages of each on the projector shapes; three of W instead: no better).
// The epilogue's slabs are the first two stages of each; the folded
// epilogue's row statistics go to the third A stage.
struct Stages {
  char *sa0, *sa1, *sa2;
  char *sb0, *sb1;
};

// s_waitcnt immediates (vmcnt in bits 3:0, expcnt and lgkmcnt left at their
// maxima): wait until at most n vector-memory operations are outstanding.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8); }

// Sums the tile's K steps into acc (overwritten).  Each wave issues 4 DMA
// instructions of W (step s + 1) and 4 of A (step s + 2) per step, 1 KB
// each, in its load phases (below); DMAs complete in issue order, so a wait
// can let A's newest step stay in flight.
template <bool FOLD>
IVC_DEV void tile_ksteps(f32x16_t (&acc)[4][2], const GemmOps& o, const TileDma& d, const Stages& st,
                         int k0, int k1, int w, int wm, int wn, int lane) {
  const int n = k1 - k0;  // K steps k0 .. k1 - 1 (the step counter s below runs from 0)
  auto dma_a = [&](int j, uint32_t ka, char* sa) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.a_rs, (lds_void_t*)(sa + (w * 4 + j) * 1024), 16,
                                             d.a_off[j], ka, 0, 0);
  };
  auto dma_b = [&](int j, uint32_t kb, char* sb) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.b_rs, (lds_void_t*)(sb + (w * 4 + j) * 1024), 16,
                                             d.b_off[j], kb, 0, 0);
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
  // byte offset of A's next K step to issue (FOLD: each step of 64 lies
  // inside one C-wide cell; the cell's grid offset comes from gather_koff)
  int cell_n = 0, c0_n = k0 * BK;  // (cell, channel) of K step k0 (plain A: c0_n is the K element)
  if (FOLD) {
    cell_n = c0_n / o.ag.C;
    c0_n -= cell_n * o.ag.C;
  }
  const uint32_t kb0 = (uint32_t)(k0 * (BK * 2));  // W's byte offset of step k0
  auto a_koff = [&]() -> uint32_t {
    const uint32_t k = FOLD ? (uint32_t)gather_koff(o.ag, cell_n, c0_n) : (uint32_t)(c0_n * 2);
    c0_n += BK;
    if (FOLD && c0_n == o.ag.C) {
      c0_n = 0;
      ++cell_n;
    }
    return k;
  };
  constexpr int NA = 3, NB = 2;
  // prologue (every wave): A and W of step 0, A of step 1
  {
    const uint32_t ka = a_koff();
#pragma unroll
    for (int j = 0; j < 4; ++j) dma_a(j, ka, st.sa0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) dma_b(j, kb0, st.sb0);
  if (n > 1) {
    const uint32_t ka = a_koff();
#pragma unroll
    for (int j = 0; j < 4; ++j) dma_a(j, ka, st.sa1);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        acc[i][j][v] = z;
      }
  // step 0's operands in LDS from every wave (A of step 1 may still fly)
  if (n > 1)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  asm volatile("s_barrier" ::: "memory");
  // Ping-pong: the two waves of a SIMD (w and w + 4) alternate between a load
  // phase (the next half step's fragments from LDS, plus a share of the
  // operand DMA) and a compute phase (that half step's 16 MFMAs), offset by
  // one phase, with a workgroup barrier after every phase: while one wave of
  // a SIMD runs its MFMAs the other issues its loads.  Half step h of step s
  // reads K columns 32h .. 32h + 31 of step s's stages.
  // DMA: W of step s + 1 in the load phase of half 0 (into the stage step
  // s - 1 used, free: its last reader finished one barrier earlier), A of
  // step s + 2 in the load phase of half 1; at the end of half 1's load phase
  // a wave waits until only that A remains in flight, so step s + 1's
  // operands are complete before any wave reads them.
  bf16x8_t ra[2][4], rb[2][2];  // [kk within the half][block]
  auto load = [&](int s, auto ia_c, auto ib_c, auto h_c, auto full_c) {
    constexpr int IA = decltype(ia_c)::value, IB = decltype(ib_c)::value;
    constexpr int H = decltype(h_c)::value;
    constexpr bool FULL = decltype(full_c)::value;
    const char* sa = IA == 0 ? st.sa0 : IA == 1 ? st.sa1 : st.sa2;
    const char* sb = IB == 0 ? st.sb0 : st.sb1;
    __builtin_amdgcn_sched_barrier(0);
    if (H == 0) {
      constexpr int JB = (IB + 1) % NB;
      char* nb = JB == 0 ? st.sb0 : st.sb1;
      if (FULL || s + 1 < n) {
        const uint32_t kb = kb0 + (uint32_t)((s + 1) * (BK * 2));
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_b(j, kb, nb);
      }
    } else {
      constexpr int JA = (IA + 2) % NA;
      char* na = JA == 0 ? st.sa0 : JA == 1 ? st.sa1 : st.sa2;
      if (FULL || s + 2 < n) {
        const uint32_t ka = a_koff();
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_a(j, ka, na);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ra[q][i] = *reinterpret_cast<const bf16x8_t*>(sa + fa[2 * H + q] + i * 4096);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        rb[q][j] = *reinterpret_cast<const bf16x8_t*>(sb + fb[2 * H + q] + j * 4096);
    }
    if (H == 1) {
      // step s + 1's operands complete (only A of step s + 2 may fly)
      if (FULL || s + 2 < n)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(4) & ~(15 << 8));  // and this phase's LDS reads
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & ~(15 << 8));
    } else {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this phase's LDS reads (lgkmcnt 0)
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
  };
  auto compute = [&]() {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[q][i], rb[q][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using TF = std::true_type;
  using FF = std::false_type;
  auto stepx = [&](int s, auto ia_c, auto ib_c, auto full_c) {
    load(s, ia_c, ib_c, I0{}, full_c);
    compute();
    load(s, ia_c, ib_c, I1{}, full_c);
    compute();
  };
  const bool late = w >= 4;  // the second wave of each SIMD runs one phase behind
  if (late) asm volatile("s_barrier" ::: "memory");
  int s = 0;
  // steady state while every step of the cycle issues both DMAs (the last
  // issues A of step s + 7), then the guarded tail
  for (; s + 8 <= n; s += 6) {
    stepx(s, I0{}, I0{}, TF{});
    stepx(s + 1, I1{}, I1{}, TF{});
    stepx(s + 2, I2{}, I0{}, TF{});
    stepx(s + 3, I0{}, I1{}, TF{});
    stepx(s + 4, I1{}, I0{}, TF{});
    stepx(s + 5, I2{}, I1{}, TF{});
  }
  for (; s < n; s += 6) {
    stepx(s, I0{}, I0{}, FF{});
    if (s + 1 < n) stepx(s + 1, I1{}, I1{}, FF{});
    if (s + 2 < n) stepx(s + 2, I2{}, I0{}, FF{});
    if (s + 3 < n) stepx(s + 3, I0{}, I1{}, FF{});
    if (s + 4 < n) stepx(s + 4, I1{}, I0{}, FF{});
    if (s + 5 < n) stepx(s + 5, I2{}, I1{}, FF{});
  }
  if (!late) asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------------------
// Leftover tiles.  A product of NT tiles on G compute units runs
// floor(NT / G) whole rounds plus a partial one in which most CUs can sit
// idle (mlp2's first product on the 2B-Flash workload: 416 tiles on 256 CUs,
// the second round 160 tiles; that round costs as much as a full one).  With
// TailSplit scratch the whole rounds stay one tile per workgroup and each of
// the r leftover tiles is cut along K into s pieces (gemm_tail_split: the
// fewest rounds of pieces times piece length; 160 tiles: 3 pieces, two
// rounds of a third).  Every piece stores its fp32 partial tile, then counts
// itself in the tile's counter; the piece that counts last adds all s
// partials in piece order (so the result does not depend on arrival order)
// and runs the epilogue.  No workgroup waits on another.  Partials and
// counters are device-coherent (sc1) accesses, so nothing is flushed; a
// counter holds (launch ticket << 8) | pieces done, so stale values from
// earlier launches need no clearing.
// ---------------------------------------------------------------------------
struct TailSplit {
  float* part;                // [2 G][128 * 512] fp32 partial tiles (slot per piece)
  unsigned long long* cnt;    // [G] per leftover tile
  unsigned long long ticket;  // this launch's tag, nonzero, < 2^56
  int G;                      // workgroups of a whole round (a multiple of 8)
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int CPOL_SC1 = 16;  // device-coherent load / store

// A scalar zero the compiler cannot see through: the 32 piece offsets of a
// partial tile built on it are formed where used, not hoisted to the
// kernel's entry as 32 live scalar registers.
IVC_DEV int opaque_zero() {
  int z = 0;
  asm volatile("" : "+s"(z));
  return z;
}

// Partial slot i: 16-byte piece q of thread tid at (q * 512 + tid) * 16, so
// each store or load instruction covers 1 KB contiguous.
IVC_DEV __amdgpu_buffer_rsrc_t part_slot(float* part, int i) {
  return __builtin_amdgcn_make_buffer_rsrc(part + (size_t)i * (128 * DNT), (short)0,
                                           128 * DNT * 4, 0x00020000);
}

// Counts one more finished piece of a leftover tile; returns how many had
// finished before it.
IVC_DEV int piece_arrive(unsigned long long* c, unsigned long long ticket) {
  unsigned long long cur = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {  // at most s contenders: every failed exchange means another one succeeded
    const bool ours = (cur >> 8) == ticket;
    const unsigned long long nv = ours ? cur + 1 : ((ticket << 8) | 1ull);
    if (__hip_atomic_compare_exchange_strong(c, &cur, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return ours ? (int)(cur & 0xff) : 0;
  }
}

// ---------------------------------------------------------------------------
// The product: one output tile (or, for leftover tiles, one K piece of one)
// per workgroup.
// ---------------------------------------------------------------------------
template <int ACT, bool FOLD>
__global__ void __launch_bounds__(DNT, 1)
k_gemm_dma8(GemmOps o, const float* __restrict__ bias, bf16_t* __restrict__ Cm, long long ldc,
            RowMap rm, const float* __restrict__ ln_rows, const float* __restrict__ ln_colsum,
            TailSplit ts) {
  __shared__ __attribute__((aligned(1024))) char sA0[QB];
  __shared__ __attribute__((aligned(1024))) char sB0[QB];
  __shared__ __attribute__((aligned(1024))) char sA1[QB];
  __shared__ __attribute__((aligned(1024))) char sB1[QB];
  __shared__ __attribute__((aligned(1024))) char sA2[QB];  // also the folded epilogue's row statistics
  int m0, n0, k0 = 0, k1 = o.K / BK, tt = -1, s = 1, piece = 0;
  {
    int M = o.M;
    if (ts.part != nullptr && rm.m_dev != nullptr) M = min(M, *rm.m_dev * rm.m_mult);
    const int tiles_m = (M + DBM - 1) / DBM, tiles_n = (o.N + DBN - 1) / DBN;
    const int NT = tiles_m * tiles_n, KT = k1;
    const int q = ts.part != nullptr ? NT / ts.G : 0, r = NT - q * ts.G;
    if (ts.part != nullptr && r > 0) s = gemm_tail_split(r, ts.G, KT);
    if (s == 1) {  // nothing split: one tile per workgroup
      if (!map_tile(o.M, o.N, rm, m0, n0)) return;
    } else {
      o.M = M;
      const int full = q * ts.G, bid = blockIdx.x;
      int t;
      if (bid < full) {
        t = (bid & 7) * (full >> 3) + (bid >> 3);  // consecutive tiles on one XCD
      } else {
        int p = bid - full;
        const int np = r * s;
        if (p >= np) return;
        // pieces XCD-major too: an XCD runs the same K piece of neighbouring tiles
        if ((np & 7) == 0) p = (p & 7) * (np >> 3) + (p >> 3);
        tt = p % r;
        piece = p / r;
        t = full + tt;
        k0 = KT * piece / s;
        k1 = KT * (piece + 1) / s;
      }
      band_tile(t, tiles_m, tiles_n, m0, n0);
    }
  }
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0..7
  const int wm = w >> 2, wn = w & 3;  // rows wm*128 .., columns wn*64 ..
  const TileDma d = tile_dma<FOLD>(o, m0, n0, w, lane);
  const Stages st{sA0, sA1, sA2, sB0, sB1};
  f32x16_t acc[4][2];
  tile_ksteps<FOLD>(acc, o, d, st, k0, k1, w, wm, wn, lane);
  if (tt >= 0) {
    // a piece of a leftover tile: store the partial, count in
    {
      const __amdgpu_buffer_rsrc_t slot = part_slot(ts.part, tt * s + piece);
      const int zs = opaque_zero();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x4_t v = {acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2],
                               acc[i][j][4 * v4 + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(v, slot, tid * 16,
                                                   zs + ((i * 2 + j) * 4 + v4) * (DNT * 16),
                                                   CPOL_SC1);
          }
    }
    __builtin_amdgcn_s_waitcnt(0);  // every wave's stores complete before the count
    __syncthreads();
    // the decision goes through the third A stage (free now; the LDS is full)
    int* last_piece = reinterpret_cast<int*>(sA2);
    if (tid == 0) *last_piece = piece_arrive(ts.cnt + tt, ts.ticket) == s - 1;
    __syncthreads();
    if (!*last_piece) return;
    // the last piece: all s partials, in piece order
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float z;
          asm volatile("v_mov_b32 %0, 0" : "=v"(z));
          acc[i][j][v] = z;
        }
    for (int pc = 0; pc < s; ++pc) {
      const __amdgpu_buffer_rsrc_t slot = part_slot(ts.part, tt * s + pc);
      const int zs = opaque_zero();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          f32x4_t pv[4];
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4)
            pv[v4] = __builtin_amdgcn_raw_buffer_load_b128(
                slot, tid * 16, zs + ((i * 2 + j) * 4 + v4) * (DNT * 16), CPOL_SC1);
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            acc[i][j][4 * v4] += pv[v4].x;
            acc[i][j][4 * v4 + 1] += pv[v4].y;
            acc[i][j][4 * v4 + 2] += pv[v4].z;
            acc[i][j][4 * v4 + 3] += pv[v4].w;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  }
  __syncthreads();
  store_tile<ACT, FOLD, 2, DNT>(acc, sA0, sB0, sA1, sB1, wm, wn, m0, n0, o.M, o.N, bias, Cm, ldc,
                                rm, ln_rows, ln_colsum, reinterpret_cast<float2*>(sA2),
                                sA2 + 4096);
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
      g.ldc % 8 == 0 && ((uintptr_t)g.Cm % 16) == 0 &&
      (g.rm.d_map == nullptr || (g.rm.c_map != nullptr && g.rm.d_out != nullptr &&
                                 ((uintptr_t)g.rm.d_out % 16) == 0 && g.rm.d_stride >= g.rm.c_rpg));
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
  if (g.fold && g.act != ACT_GELU) return hipErrorInvalidValue;  // folded: the GELU'd first Linears
  GemmOps o{(const bf16_t*)g.A, g.lda, g.a_rpg, g.a_gstride, g.a_goff, (const bf16_t*)g.W, g.ldw,
            g.M, g.N, g.K, g.ag};
  const int tiles = ((g.M + DBM - 1) / DBM) * ((g.N + DBN - 1) / DBN);
  TailSplit ts{nullptr, nullptr, 0, 0};
  int grid = tiles;
  if (g.tail_part != nullptr) {
    if (g.tail_grid <= 0 || g.tail_grid % 8 != 0 || g.tail_cnt == nullptr || g.tail_ticket == 0 ||
        (g.tail_ticket >> 56) != 0)
      return hipErrorInvalidValue;
    ts = TailSplit{g.tail_part, g.tail_cnt, g.tail_ticket, g.tail_grid};
    if (g.rm.m_dev == nullptr) {  // the tile count is known: exactly the workgroups needed
      const int q = tiles / g.tail_grid, r = tiles - q * g.tail_grid;
      grid = q * g.tail_grid + (r > 0 ? r * gemm_tail_split(r, g.tail_grid, g.K / BK) : 0);
    } else {  // an upper bound: the pieces add at most 2 G - r workgroups
      grid = tiles + 2 * g.tail_grid;
    }
  }
#define IVC_DMA_LAUNCH(ACTV, FOLDV)                                                            \
  hipLaunchKernelGGL((k_gemm_dma8<ACTV, FOLDV>), dim3((unsigned)grid), dim3(DNT), 0, s, o, g.bias, \
                     (bf16_t*)g.Cm, g.ldc, g.rm, g.ln_rows, g.ln_colsum, ts)
  if (g.fold)
    IVC_DMA_LAUNCH(ACT_GELU, true);
  else if (g.act == ACT_GELU)
    IVC_DMA_LAUNCH(ACT_GELU, false);
  else
    IVC_DMA_LAUNCH(ACT_NONE, false);
#undef IVC_DMA_LAUNCH
  return hipGetLastError();
}

}  // namespace ivc
