// Dense projections y = x . W^T on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Every projection of the drafter multiplies activations by a weight stored [out, in]
// (dflash2.ts diff, `Bf16Projection`), so both operands are K-contiguous: each lane
// loads 16 contiguous bytes of one row for either MFMA operand and no transpose is
// needed.
//
// At the drafter's row counts (B*G = 128 block rows, B*(G-1) = 120 head rows) every
// projection streams its weight once and is bound by HBM, not by the matrix cores
// (128 flop per weight byte against a ridge near 312).  What decides the speed is the
// weight bytes in flight per CU and the DRAM pattern of the stream:
//   * one 128 x 256 tile per workgroup (8 wavefronts of 64 x 64), so a K step moves a
//     32 KB weight tile and the grid stays within one resident wave of workgroups;
//   * a register ring of PF stages: the loads of step k+PF are issued before step k is
//     computed, each step is parked in one of two LDS buffers one iteration before use,
//     one barrier per 64-wide K step; loads are branch-free (rows past M or N are clamped)
//     so the compiler waits only on the stage it needs;
//   * the drafter's own weights are stored tile-contiguous, [N/256][K/64][256][64], so a K
//     step of a tile is one contiguous 32 KB block; the target's head stays row-major.
//
//   * narrow projections (N <= 2048 at M <= 128, or N <= 256 at any M) take 64-column
//     workgroups of two wavefronts reading 64-row slices of those blocks.
//
// With more rows (a 64-request block, the context projection) the projections approach
// the matrix cores' bound and take 256 x 256 tiles whose operands are copied global -> LDS
// directly (gemm_dma_kernel); weight-major grids run the M tiles of an N tile together on
// one XCD, split K when the tiles alone do not fill a round of workgroups, and run a last,
// mostly empty round's weight rows as a separate split-K launch.
//
// Split-K: grid.z slices K; slices write fp32 partials and a separate kernel sums them
// in slice order (deterministic, no float atomics) and applies the epilogue, or the
// partials are left for the consuming kernel, which sums them in the same order.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "vmem.hpp"

namespace dfl {

namespace {

constexpr int BK = 64;  // K step of the library's GEMM plans

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* W;
  int lda, M, N, K;
  int k_per_split;
  int epi;
  void* out0;
  int ld0;
  void* out1;
  int ld1;
  int nsplit;
  float* partial;
  int splits;
  float* tile_max;  // EPI_F32, one split: [M, ceil(nsplit / 256)] row maxima of each 256-column tile of out0
  uint32_t* tile_bound;  // with tile_max, optional: [M, kTileBoundSlots] (launch_gemm's declaration)
  int a_tiled;           // A in fragment order (launch_tile_rows), 256 x 256 kernel only
  // 4-bit affine weights (used instead of W): row-major packed [N, K/8] words with scales and
  // biases [N, K/64] bf16, or tile-contiguous blocks (q4_tiled_words)
  const uint32_t* Wq;
  const uint16_t* Ws;
  const uint16_t* Wb;
};

__device__ __forceinline__ void store_out(const GemmArgs& p, int m, int n, float v) {
  if (p.epi == EPI_BF16) {
    static_cast<uint16_t*>(p.out0)[(size_t)m * p.ld0 + n] = f32_to_bf16(v);
  } else if (n < p.nsplit) {
    static_cast<float*>(p.out0)[(size_t)m * p.ld0 + n] = v;
  } else {
    static_cast<float*>(p.out1)[(size_t)m * p.ld1 + (n - p.nsplit)] = v;
  }
}

// Position of 16-byte chunk c of a tile-contiguous weight block (256 rows x 64 K): chunk c
// is lane c % 64 of fragment c / 64; fragment f covers rows 16 (f / 2) .. +15 and K half
// f % 2; lane l holds row l % 16 at K offset 8 (l / 16) of that half.
__device__ __forceinline__ void frag_chunk_pos(int c, int& row, int& k) {
  const int f = c >> 6, l = c & 63;
  row = (f >> 1) * 16 + (l & 15);
  k = (f & 1) * 32 + (l >> 4) * 8;
}

// Loads one K step of the A tile [BM x BKS] and the W tile [BN x BKS] into registers.
// TILED: W is stored tile-contiguous, [N/BN][K/BKS][BN][BKS], so one step of one tile is
// a single contiguous BN*BKS*2-byte block; otherwise W is row-major [N, K].
template <int BM, int BN, int BKS, int NT, bool TILED>
struct TileLoader {
  // tiled weights come in 256 x 64 blocks; a BN-row slice (BN dividing 256) of a block is
  // BN / 16 consecutive row groups, i.e. one contiguous run in fragment order
  static_assert(!TILED || (256 % BN == 0 && BKS == 64), "tiled weights come in 256 x 64 blocks");
  static constexpr int CPR = BKS / 8;  // 16-byte chunks per tile row
  static constexpr int A_PER = BM * CPR / NT;
  static constexpr int B_PER = BN * CPR / NT;
  static_assert(A_PER * NT == BM * CPR, "A tile must split evenly over threads");
  static_assert(B_PER * NT == BN * CPR, "B tile must split evenly over threads");
  u32x4_t a[A_PER];
  u32x4_t b[B_PER];

  // Rows past M or N are clamped to the last row instead of branching around the load:
  // their products land only in accumulator rows/columns that are never stored, and a
  // branch-free body lets the compiler wait on exactly the stage it needs.
  __device__ __forceinline__ void load(const GemmArgs& p, int m0, int n0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      const int gm = min(m0 + c / CPR, p.M - 1);
      a[i] = *reinterpret_cast<const u32x4_t*>(p.A + (size_t)gm * p.lda + k0 + (c % CPR) * 8);
    }
    if (TILED) {
      const uint16_t* tile =
          p.W + ((size_t)(n0 / 256) * (p.K / BKS) + k0 / BKS) * (256 * BKS) + (size_t)(n0 % 256) * BKS;
#pragma unroll
      for (int i = 0; i < B_PER; ++i)
        b[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(tile + (tid + i * NT) * 8));
    } else {
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        const int c = tid + i * NT;
        const int gn = min(n0 + c / CPR, p.N - 1);
        b[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(p.W + (size_t)gn * p.K + k0 + (c % CPR) * 8));
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* sA, uint16_t* sB, int tid) const {
    constexpr int LS = BKS + 8;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(&sA[(c / CPR) * LS + (c % CPR) * 8]) = a[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + i * NT;
      int row, kc;
      if (TILED) {
        frag_chunk_pos(c, row, kc);
      } else {
        row = c / CPR;
        kc = (c % CPR) * 8;
      }
      *reinterpret_cast<u32x4_t*>(&sB[row * LS + kc]) = b[i];
    }
  }
};

// Eight 4-bit fields of one packed word (field e = the weight at K offset e, lowest bits
// first) as bf16 weights scale * q + bias: one fp32 fma each, rounded once.
__device__ __forceinline__ u32x4_t dequant8(uint32_t w, uint32_t sb) {
  const float sc = __uint_as_float(sb << 16);
  const float bi = __uint_as_float(sb & 0xFFFF0000u);
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = fmaf(sc, static_cast<float>((w >> (4 * e)) & 0xFu), bi);
  return pack8(f);
}

// 4-bit affine weights ([P2] `quantizedWeight`: groups of 64 inputs, w = scale * q + bias).
// A K step is one group per row: each thread loads one 16-byte chunk of packed fields (32
// weights) with their (scale, bias) and dequantizes while parking the step in LDS, so the
// tile compute is the bf16 one.  Row-major: the chunk is half a row's step.  TILED (the
// blocks of tile_q4_kernel): the chunk is four words of one lane of a 64-row group, i.e. 8
// fields at each K half for rows r0 and r0 + 16.
template <int BM, int BN, int BKS, int NT, bool TILED>
struct TileLoaderQ4 {
  static constexpr int CPR = BKS / 8;
  static constexpr int A_PER = BM * CPR / NT;
  static_assert(A_PER * NT == BM * CPR, "A tile must split evenly over threads");
  static_assert(BKS == 64 && BN == 256 && NT == 512, "one 16-byte chunk of packed fields per thread");
  u32x4_t a[A_PER];
  u32x4_t w;
  u32x2_t sb;

  __device__ __forceinline__ void load(const GemmArgs& p, int m0, int n0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      const int gm = min(m0 + c / CPR, p.M - 1);
      a[i] = *reinterpret_cast<const u32x4_t*>(p.A + (size_t)gm * p.lda + k0 + (c % CPR) * 8);
    }
    if (TILED) {
      const uint32_t* grp = p.Wq + ((size_t)(n0 / BN) * (p.K / BKS) + k0 / BKS) * (BN * 9) + (tid >> 7) * 576;
      const int l = (tid >> 1) & 63, h = tid & 1;
      w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(grp + l * 8 + h * 4));
      sb = *reinterpret_cast<const u32x2_t*>(grp + 512 + (l & 15) * 4 + h * 2);
    } else {
      const int row = tid >> 1, half = tid & 1;
      const int gn = min(n0 + row, p.N - 1);
      w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.Wq + (size_t)gn * (p.K / 8) + k0 / 8 + half * 4));
      const size_t g = (size_t)gn * (p.K / BKS) + k0 / BKS;
      sb[0] = static_cast<uint32_t>(p.Ws[g]) | (static_cast<uint32_t>(p.Wb[g]) << 16);
    }
  }
  __device__ __forceinline__ void store(uint16_t* sA, uint16_t* sB, int tid) const {
    constexpr int LS = BKS + 8;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(&sA[(c / CPR) * LS + (c % CPR) * 8]) = a[i];
    }
    if (TILED) {
      const int l = (tid >> 1) & 63, h = tid & 1;
      const int r0 = (tid >> 7) * 64 + h * 32 + (l & 15), kc = (l >> 4) * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = r0 + (j >> 1) * 16;
        *reinterpret_cast<u32x4_t*>(&sB[row * LS + (j & 1) * 32 + kc]) = dequant8(w[j], sb[j >> 1]);
      }
    } else {
      const int row = tid >> 1, half = tid & 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4_t*>(&sB[row * LS + half * 32 + j * 8]) = dequant8(w[j], sb[0]);
    }
  }
};

// W rows for EPI_SILU_MUL are interleaved per 16: [gate 16 | up 16] ... so output
// column j pairs accumulator columns (j/16)*32 + j%16 (gate) and +16 (up).
// Multiplier of the workgroup index that staggers where each workgroup starts its K loop
// (coprime with the usual step counts: 80 for K = 5120, 64, 272, 400).
constexpr unsigned kKRotate = 13;

// Workgroup -> (N tile, M tile).  Workgroups are dispatched in id order (x fastest) and
// dealt round-robin to the 8 XCDs, each with its own L2.  When the weights are the larger
// operand (N > M) and there are several M tiles, the ids are remapped so that each XCD runs
// a contiguous stretch of an M-fastest order: the M tiles of one N tile, which read the same
// weight tile, run together on one XCD and share its L2, instead of each weight tile
// streaming from HBM once per M tile (a bijection on the first 8 * floor(total / 8) ids,
// identity on the rest).  Otherwise the launch order is kept: with the activations the
// larger operand, N tiles fastest across the XCDs measured best.
__device__ __forceinline__ void tile_of_block(int M, int N, int& nt_idx, int& mt_idx) {
  const int nt = gridDim.x, mt = gridDim.y;
  if (mt == 1 || N <= M) {
    nt_idx = blockIdx.x;
    mt_idx = blockIdx.y;
    return;
  }
  const int total = nt * mt;
  const int id = blockIdx.y * nt + blockIdx.x;
  const int t8 = total / 8;
  const int rid = id < t8 * 8 ? (id % 8) * t8 + id / 8 : id;
  mt_idx = rid % mt;
  nt_idx = rid / mt;
}

// The output stage shared by the LDS kernels: split-K partial planes, SiLU(gate) * up, or a
// plain store, plus each 256-column tile's row maxima when asked for.  Accumulator layout:
// lane holds column (lane & 15) and rows 4 * (lane >> 4) + e of each 16 x 16 block.
template <int BM, int WN, int TM, int TN, int NT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& p, const f32x4_t (&acc)[TM][TN], int m0, int n0,
                                              int wm, int wn, int lane, int tid) {
  const int mrow = m0 + wm * (TM * 16) + (lane >> 4) * 4;
  const int ncol = n0 + wn * (TN * 16) + (lane & 15);
  if (p.splits > 1) {
    float* part = p.partial + (size_t)blockIdx.z * p.M * p.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mrow + i * 16 + e;
          const int n = ncol + j * 16;
          if (m < p.M && n < p.N) part[(size_t)m * p.N + n] = acc[i][j][e];
        }
    return;
  }
  if (p.epi == EPI_SILU_MUL) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; j += 2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mrow + i * 16 + e;
          const int n = ncol + j * 16;  // gate column; up is n + 16
          if (m < p.M && n < p.N) {
            const int jo = (n >> 5) * 16 + (n & 15);
            const float v = silu(acc[i][j][e]) * acc[i][j + 1][e];
            static_cast<uint16_t*>(p.out0)[(size_t)m * p.ld0 + jo] = f32_to_bf16(v);
          }
        }
    return;
  }
  // Without a bound every value is stored, first, so the stores drain while the tile maxima
  // are reduced.
  if (!p.tile_max || n0 >= p.nsplit || !p.tile_bound) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mrow + i * 16 + e;
          const int n = ncol + j * 16;
          if (m < p.M && n < p.N) store_out(p, m, n, acc[i][j][e]);
        }
    if (!p.tile_max || n0 >= p.nsplit) return;
  }
  // Row maxima of this tile over its first output's columns (< nsplit, which is N unless a
  // second output takes the columns after it): within a lane over its TN columns, then over
  // the 16 lanes that share a row, then over the WN wavefronts through LDS.  fmaxf skips NaN,
  // so a tile's maximum is NaN only when all of its values are.
  __shared__ float rmax[WN][BM];
  __shared__ int rskip[BM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = -INFINITY;
#pragma unroll
      for (int j = 0; j < TN; ++j)
        if (ncol + j * 16 < p.nsplit) v = fmaxf(v, acc[i][j][e]);
      v = row16_max(v);
      if ((lane & 15) == 0) rmax[wn][wm * (TM * 16) + i * 16 + (lane >> 4) * 4 + e] = v;
    }
  __syncthreads();
  const int tile = n0 / kGemmTileN;
  const int ntl = (p.nsplit + kGemmTileN - 1) / kGemmTileN;
  if (!p.tile_bound) {
    for (int r = tid; r < BM; r += NT) {
      const int m = m0 + r;
      if (m < p.M) {
        float v = rmax[0][r];
#pragma unroll
        for (int w = 1; w < WN; ++w) v = fmaxf(v, rmax[w][r]);
        p.tile_max[(size_t)m * ntl + tile] = v;
      }
    }
    return;
  }
  // Four lanes per row read the row's slots (one 64-byte line) as other workgroups have
  // filled them so far, with one device-scope load that bypasses this XCD's L2 (a stale
  // slot is only smaller, so the bound stays valid); then the row's tile maximum goes into
  // its own slot.
  static_assert(BM * 4 % NT == 0 && kTileBoundSlots == 16, "four lanes of four slots per row, every lane");
  for (int r4 = tid; r4 < BM * 4; r4 += NT) {
    const int r = r4 >> 2, q = r4 & 3;
    const int m = m0 + r;
    float v = rmax[0][r];
#pragma unroll
    for (int w = 1; w < WN; ++w) v = fmaxf(v, rmax[w][r]);
    uint32_t lo = 0xFFFFFFFFu;
    if (m < p.M) {
      const uint32_t* slot = p.tile_bound + (size_t)m * kTileBoundSlots + q * 4;
      u32x4_t s4;
      asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(s4) : "v"(slot) : "memory");
      lo = min(min(s4[0], s4[1]), min(s4[2], s4[3]));
    }
    lo = row16_umin<true>(lo);
    if (q == 0) {
      if (m < p.M) {
        p.tile_max[(size_t)m * ntl + tile] = v;
        if (v == v)
          __hip_atomic_fetch_max(p.tile_bound + (size_t)m * kTileBoundSlots + tile % kTileBoundSlots,
                                 float_order(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      rskip[r] = m < p.M && lo != 0u && v < order_float(lo);  // 0: a slot still empty
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = mrow + i * 16 + e;
      if (m >= p.M || rskip[m - m0]) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = ncol + j * 16;
        if (n < p.N) store_out(p, m, n, acc[i][j][e]);
      }
    }
}

// MINB is the minimum number of wavefronts per SIMD the registers must allow (the second
// launch bound); the 128 x 64 instance takes 1, since its LDS admits two 2-wavefront
// workgroups per CU, one wavefront per SIMD.
template <int BM, int BN, int BKS, int WM, int WN, int PF, int MINB, bool TILED, bool Q4 = false>
__global__ __launch_bounds__(WM* WN * 64, MINB) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 16;
  constexpr int TN = BN / WN / 16;
  constexpr int LDS_STRIDE = BKS + 8;  // +16 bytes: 16-byte reads of 16 rows hit distinct banks
  using Loader = std::conditional_t<Q4, TileLoaderQ4<BM, BN, BKS, NT, TILED>, TileLoader<BM, BN, BKS, NT, TILED>>;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  int ntile, mtile;
  tile_of_block(p.M, p.N, ntile, mtile);
  const int n0 = ntile * BN;
  const int m0 = mtile * BM;
  const int kbeg = blockIdx.z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg) / BKS;
  // Step kt reads K block (kt + rot) mod nk: workgroups start their K loops at different
  // blocks, so at any moment they read weights spread over the HBM channels instead of all
  // at the same offset of their (equally sized, aligned) weight slabs.
  const int rot = nk > 0 ? static_cast<int>((ntile * kKRotate) % static_cast<unsigned>(nk)) : 0;
  auto kof = [&](int kt) {
    const int q = kt + rot;
    return kbeg + (q >= nk ? q - nk : q) * BKS;
  };

  Loader ring[PF];
  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (s < nk) ring[s].load(p, m0, n0, kof(s), tid);
  if (nk > 0) ring[0].store(sA[0], sB[0], tid);

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BKS / 32; ++ks) {
      const int kk = ks * 32 + (lane >> 4) * 8;
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * (TM * 16) + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][row * LDS_STRIDE + kk]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = wn * (TN * 16) + j * 16 + (lane & 15);
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&sB[buf][col * LDS_STRIDE + kk]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // Iteration kt: refill ring slot kt%PF with step kt+PF, compute step kt from LDS buffer
  // kt%2, then move step kt+1 (ring slot (kt+1)%PF) into LDS buffer (kt+1)%2.  The main
  // loop runs while every refill is in range and is unrolled PF times so every ring index
  // is a compile-time constant; the last steps run in a guarded tail without refills.
  int kt0 = 0;
  for (; kt0 + 2 * PF <= nk; kt0 += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int kt = kt0 + s;
      ring[s].load(p, m0, n0, kof(kt + PF), tid);
      __syncthreads();
      compute(kt & 1);
      ring[(s + 1) % PF].store(sA[(kt + 1) & 1], sB[(kt + 1) & 1], tid);
    }
  }
#pragma unroll
  for (int s = 0; s < 2 * PF; ++s) {
    const int kt = kt0 + s;
    if (kt < nk) {
      if (kt + PF < nk) ring[s % PF].load(p, m0, n0, kof(kt + PF), tid);
      __syncthreads();
      compute(kt & 1);
      if (kt + 1 < nk) ring[(s + 1) % PF].store(sA[(kt + 1) & 1], sB[(kt + 1) & 1], tid);
    }
  }

  gemm_epilogue<BM, WN, TM, TN, NT>(p, acc, m0, n0, wm, wn, lane, tid);
}

// ---------------------------------------------------------------------------------------
// Weight-streaming kernel for M <= 128 rows (every projection of a draft block).
//
// At these row counts a projection reads each weight once, at 128 flop per bf16 weight
// byte, so it should run at HBM speed; what costs time in the LDS kernel above is staging
// the weight tile through LDS (a write and four reads of every weight) and, for the wide
// projections, having fewer 128 x 256 tiles than CUs.  Here each wavefront owns 32 weight
// rows and all M rows of the output: its weight fragments go from HBM straight into MFMA
// operand registers (the tile-contiguous layout is the operand order, so each load is 1 KB
// contiguous per wavefront) and only the activations, shared by the NW wavefronts of a
// workgroup, pass through LDS.  A weight stage (one 64-wide K step of the wave's rows) is
// loaded PF steps ahead into a register ring and the activations AD steps ahead into LDS;
// one barrier per step.  The plan picks NW (8, 5 or 2 wavefronts) and the K split so that
// the grid fills about one round of CUs; two wavefronts share a SIMD (256 registers each).

// A wavefront's weights for one K step: 32 weight rows = 2 fragments of 16 rows x 2 K
// halves.  LOADS is the number of vector-memory instructions load() issues.
template <bool TILED, bool Q4>
struct StreamW;

// bf16: the four fragments, as loaded.
template <bool TILED>
struct StreamW<TILED, false> {
  static constexpr int LOADS = 4;
  u32x4_t v[4];  // fragment (j, half) at j * 2 + half
  __device__ __forceinline__ void load(const GemmArgs& p, int nw0, int k0, int lane) {
    if (TILED) {
      // a wave whose rows start past the last tile (the grid's last workgroup) re-reads the
      // last 32 rows instead; its outputs are not stored
      nw0 = min(nw0, (p.N + kGemmTileN - 1) / kGemmTileN * kGemmTileN - 32);
      const uint16_t* blk = p.W + ((size_t)(nw0 / kGemmTileN) * (p.K / BK) + k0 / BK) * (kGemmTileN * BK) +
                            (nw0 % kGemmTileN) / 16 * 2 * 512 + lane * 8;
#pragma unroll
      for (int f = 0; f < 4; ++f) v[f] = vm_load16_nt(blk + f * 512);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = min(nw0 + j * 16 + (lane & 15), p.N - 1);
        const uint16_t* row = p.W + (size_t)n * p.K + k0 + (lane >> 4) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) v[j * 2 + h] = vm_load16_nt(row + h * 32);
      }
    }
  }
  template <int N>
  __device__ __forceinline__ void wait() {
#pragma unroll
    for (int f = 0; f < 4; ++f) vm_wait<N>(v[f]);
  }
  __device__ __forceinline__ bf16x8_t frag(int j, int h) const { return __builtin_bit_cast(bf16x8_t, v[j * 2 + h]); }
};

// 4-bit (tile-contiguous only): the wavefront's 32 rows are half of a 64-row group, so one
// 16-byte load brings the lane's four packed words (rows 16 j + lane % 16 of that half, both
// K halves) and one more the group's scale | bias words.  Kept as the loaded vectors: a
// value is never split or copied before its wait.
template <>
struct StreamW<true, true> {
  static constexpr int LOADS = 2;
  u32x4_t q;   // word j * 2 + half for the half's rows j = 0, 1
  u32x4_t sb;  // scale | bias << 16 of the group's row sets 0..3
  int half = 0;
  __device__ __forceinline__ void load(const GemmArgs& p, int nw0, int k0, int lane) {
    nw0 = min(nw0, (p.N + kGemmTileN - 1) / kGemmTileN * kGemmTileN - 32);
    const uint32_t* grp = p.Wq + ((size_t)(nw0 / kGemmTileN) * (p.K / BK) + k0 / BK) * (kGemmTileN * 9) +
                          (nw0 % kGemmTileN) / 64 * 576;
    half = (nw0 % 64) / 32;
    q = vm_load16_nt(grp + lane * 8 + half * 4);
    sb = vm_load16(grp + 512 + (lane & 15) * 4);
  }
  template <int N>
  __device__ __forceinline__ void wait() {
    vm_wait<N>(q);
    vm_wait<N>(sb);
  }
  __device__ __forceinline__ bf16x8_t frag(int j, int h) const {
    return __builtin_bit_cast(bf16x8_t, dequant8(q[j * 2 + h], half ? sb[2 + j] : sb[j]));
  }
};

// The activation slab of one K step, [MT * 16 rows][64] bf16, copied from global memory
// straight into LDS (16 bytes per lane, 1 KB = 8 rows per instruction) without passing
// through registers.  LDS rows are 128 bytes with the 16-byte chunk of K offset 8c of row r
// stored at slot c ^ (r % 8), so the fragment reads of 16 consecutive rows spread over the
// banks.  Instructions are split over the NW wavefronts; when there are fewer instructions
// than wavefronts the extra ones repeat the last (identical bytes to the same place).
template <int MT, int NW>
struct StreamA {
  static constexpr int INSTR = MT * 2;
  static constexpr int PER = (INSTR + NW - 1) / NW;  // per wavefront (NW wavefronts share them)
  __device__ __forceinline__ static void load(const GemmArgs& p, uint16_t* buf, int k0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ins = min(wave * PER + i, INSTR - 1);
      const int row = ins * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ (row & 7);
      const uint16_t* src = p.A + (size_t)min(row, p.M - 1) * p.lda + k0 + chunk * 8;
      __builtin_amdgcn_global_load_lds(src, buf + ins * 512, 16, 0, 0);
    }
  }
  // Byte offset in a buffer of this lane's fragment (i, h): row 16 i + lane % 16, K offset
  // 32 h + 8 (lane / 16); since 16 i is a multiple of 8 the slot only depends on the lane
  // and h, and fragment i sits 2048 bytes after fragment i - 1.
  __device__ __forceinline__ static uint32_t frag_offset(int h, int lane) {
    return (lane & 15) * 128 + (((h * 4 + (lane >> 4)) ^ (lane & 7)) * 16);
  }
};

// An LDS read the compiler does not see as one: its alias tracking would otherwise make
// every LDS read wait for all copies into LDS still in flight (including the ones for later
// steps).  Completion is awaited explicitly with lds_wait, which also ties the value so no
// use can be scheduled before the wait.
__device__ __forceinline__ bf16x8_t lds_read_b128(uint32_t addr) {
  bf16x8_t v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
template <int N>
__device__ __forceinline__ void lds_wait(bf16x8_t& v) {
  asm volatile("s_waitcnt lgkmcnt(%1) ; waits for %0" : "+v"(v) : "i"(N));
}
// lds_wait with the count given by a value the unrolled loop makes a constant (0..15).
__device__ __forceinline__ void lds_wait_n(bf16x8_t& v, int n) {
  switch (n) {
    case 0: lds_wait<0>(v); break;
    case 1: lds_wait<1>(v); break;
    case 2: lds_wait<2>(v); break;
    case 3: lds_wait<3>(v); break;
    case 4: lds_wait<4>(v); break;
    case 5: lds_wait<5>(v); break;
    case 6: lds_wait<6>(v); break;
    default: lds_wait<7>(v); break;
  }
}

// 256 x 256 workgroup tiles for projections with enough rows to be bound by the matrix
// cores.  Both operands go from global memory straight into LDS (global_load_lds, 16 bytes
// a lane, no registers); eight wavefronts of 128 x 64 outputs (8 x 4 MFMA blocks) step
// through K 32 deep.
//
// Weights (B) go through a ring of three 32-deep buffers in MFMA fragment order: fragment
// f (16 rows x 32 K) is 1 KB with lane l's 16 bytes (row l % 16, K offset 8 (l / 16)) at
// 16 l, so every fragment read is one contiguous 1 KB a wavefront.  Tile-contiguous
// weights are already in that order (each copy is 1 KB contiguous); row-major weights
// are copied as 16 row segments of 64 bytes.
//
// Activations (A) are row-major, and a copy of 16 rows x 64 bytes uses half of each
// 128-byte line it touches; a 64-deep block of 8 rows is 8 whole lines.  So A goes through
// a ring of three 64-deep blocks (32 KB each): chunk q (rows 8q..8q+7) is 1 KB with row p
// at 128 p and its 16-byte K chunk c in slot sw(c) ^ p ^ (q & 1), where sw swaps the two low
// bits of c.  A fragment read (rows 16F + l % 16, K chunk 4h + l / 16 of the block) then
// meets every bank once per 512 bytes read by 32 consecutive lanes (and per 256 by 16, per
// 128 by 8): within 32 lanes the slot's bit 0 follows the row parity q & 1, bit 1 the low
// bit of l / 16, bit 2 the row's bit 2.
//
// Schedule, per 32-deep step kt (h = kt & 1 of block kt / 2): the fragments of step kt + 1
// are read from LDS while step kt's MFMAs run (registers double-buffered).  Step kt
// refills the buffers read during step kt - 1: B step kt + 3 into B's slot kt % 3 and, on
// odd steps, A block (kt - 1) / 2 + 3 into its A buffer.  A wavefront's copies complete in
// issue order (B before A within a step), and in every step the last six it issued (one
// B step and one A block at most) are all that may still be outstanding when it waits,
// which leaves B step kt + 1 and A block (kt + 1) / 2 landed; the barrier after the wait
// publishes them and tells the wavefront that all others have awaited their reads of the
// buffers it is about to refill.  LDS reads are inline assembly (the compiler's alias
// tracking would make them wait for every copy in flight), each value tied to the lgkmcnt
// wait that covers it.
constexpr int kDmaStagesB = 3;
constexpr int kDmaBlocksA = 3;

template <bool TILED>
__global__ __launch_bounds__(512, 1) void gemm_dma_kernel(GemmArgs p) {
  constexpr int BN = kGemmTileN, WN = 4, TM = 8, TN = 4, NT = 512;
  constexpr int FR = 512;          // bf16 per 1 KB fragment or chunk
  constexpr int STAGE = 16 * FR;   // B: one 32-deep K half of a 256-row tile
  constexpr int BLOCK = 32 * FR;   // A: one 64-deep K block of a 256-row tile
  __shared__ __attribute__((aligned(16))) uint16_t sA[kDmaBlocksA][BLOCK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kDmaStagesB][STAGE];
  static_assert(BN == 256, "fragment-order weight blocks are 256 rows");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  int ntile, mtile;
  tile_of_block(p.M, p.N, ntile, mtile);
  const int n0 = ntile * BN;
  const int m0 = mtile * 256;
  const int kb0 = blockIdx.z * (p.k_per_split / 64);               // first 64-deep K block of this split
  const int nkb = (min(p.K, (blockIdx.z + 1) * p.k_per_split) - blockIdx.z * p.k_per_split) / 64;
  const int nst = 2 * nkb;  // K halves
  // No staggered start here (unlike the 128-row kernels): with every workgroup of an XCD at
  // the same K block, the activation block they share stays in that XCD's L2; staggered,
  // the whole activation slab (up to 10 MB) is read from the Infinity Cache instead, and every
  // projection measured 4-5% slower.
  // wavefront w copies A chunks 4w..4w+3 of every block and B fragments 2w, 2w + 1 of
  // every step; lane i of an A copy brings row 8q + i / 8's K chunk sw((i % 8) ^ (i / 8) ^ (q & 1))
  auto sw = [](int c) { return (c & 4) | ((c & 1) << 1) | ((c >> 1) & 1); };
  const int fa = 2 * wave;
  const int fk = (lane >> 4) * 8;
  const uint16_t* arow[4];
  const uint16_t* brow[2];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = 4 * wave + u;  // q & 1 == u & 1
    const int c = sw((lane & 7) ^ (lane >> 3) ^ (u & 1));
    arow[u] = p.A + (size_t)min(m0 + 8 * q + (lane >> 3), p.M - 1) * p.lda + kb0 * 64 + c * 8;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
    brow[i] = TILED ? p.W + ((size_t)(n0 / BN) * (p.K / 64) + kb0) * (BN * 64) + (size_t)(2 * (fa + i)) * FR + lane * 8
                    : p.W + (size_t)min(n0 + 16 * (fa + i) + (lane & 15), p.N - 1) * p.K + fk;
  // copies past the last step or block re-read the last one, so every step issues and
  // awaits the same number of copies
  auto issue_b = [&](int st) {  // B step st into slot st % 3
    const int s = min(st, nst - 1);
    const int h = s & 1;
    const int kb = s >> 1;  // K block within the split
    uint16_t* dst = &sB[st % kDmaStagesB][0];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint16_t* src = TILED ? brow[i] + (size_t)kb * (BN * 64) + h * FR : brow[i] + (kb0 + kb) * 64 + h * 32;
      __builtin_amdgcn_global_load_lds(src, dst + (fa + i) * FR, 16, 0, 0);
    }
  };
  auto issue_a = [&](int j) {  // A block j into buffer j % 3
    const int jj = min(j, nkb - 1);
    uint16_t* dst = &sA[j % kDmaBlocksA][0];
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_amdgcn_global_load_lds(arow[u] + jj * 64, dst + (4 * wave + u) * FR, 16, 0, 0);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A fragment i of this wavefront (tile rows 16 (8 wm + i) ..) lies in chunks 2 (8 wm + i)
  // and + 1; lane l reads chunk 2 (8 wm + i) + (l % 16) / 8, row l % 8, slot sw(4h + l / 16) ^
  // (l % 8) ^ ((l % 16) / 8), which is 4h ^ its value at h = 0
  const int slot0 = sw(lane >> 4) ^ (lane & 7) ^ ((lane >> 3) & 1);
  const uint32_t sa_lane = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&sA[0][0])) + wm * TM * 2048 +
                           ((lane >> 3) & 1) * 1024 + (lane & 7) * 128;
  const uint32_t sa0 = sa_lane + slot0 * 16, sa1 = sa_lane + (slot0 ^ 4) * 16;
  const uint32_t sb0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&sB[0][0])) + (wn * TN * FR + lane * 8) * 2;
  // Fragments are double-buffered in registers: step kt + 1's are read from LDS while step
  // kt's MFMAs run, and awaited (every value tied to a wait) after them.
  bf16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  auto read = [&](int st, bf16x8_t (&a)[TM], bf16x8_t (&b)[TN]) {
    const uint32_t oa = ((st & 1) ? sa1 : sa0) + ((st >> 1) % kDmaBlocksA) * (BLOCK * 2);
    const uint32_t ob = sb0 + (st % kDmaStagesB) * (STAGE * 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = lds_read_b128(ob + j * (FR * 2));
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = lds_read_b128(oa + i * 2048);
  };
  auto await = [&](bf16x8_t (&a)[TM], bf16x8_t (&b)[TN]) {
#pragma unroll
    for (int j = 0; j < TN; ++j) lds_wait<0>(b[j]);
#pragma unroll
    for (int i = 0; i < TM; ++i) lds_wait<0>(a[i]);
  };
  auto mfma = [&](const bf16x8_t (&a)[TM], const bf16x8_t (&b)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  auto step = [&](int kt, bool odd, const bf16x8_t (&ca)[TM], const bf16x8_t (&cb)[TN], bf16x8_t (&na)[TM],
                  bf16x8_t (&nb)[TN]) {
    wait_vmcnt<6>();
    __builtin_amdgcn_s_barrier();
    issue_b(kt + 3);
    if (odd) issue_a((kt - 1) / 2 + 3);
    read(kt + 1, na, nb);  // past the last step: a re-read copy, unused
    mfma(ca, cb);
    await(na, nb);
  };

  // issue order A0 B0 B1 A1 B2 A2: the first wait leaves the last twelve (B1 onwards)
  // outstanding, and step 0's wait for six leaves B2 and A2
  issue_a(0);
  issue_b(0);
  issue_b(1);
  issue_a(1);
  issue_b(2);
  issue_a(2);
  wait_vmcnt<12>();
  __builtin_amdgcn_s_barrier();
  read(0, fa0, fb0);
  await(fa0, fb0);
  for (int kt = 0; kt < nst; kt += 2) {  // nst is even
    step(kt, false, fa0, fb0, fa1, fb1);
    step(kt + 1, true, fa1, fb1, fa0, fb0);
  }
  wait_vmcnt<0>();  // the re-read copies past the last step land before the workgroup ends
  gemm_epilogue<256, WN, TM, TN, NT>(p, acc, m0, n0, wm, wn, lane, tid);
}

// The same 256 x 256 tiles for activations already in fragment order (launch_tile_rows):
// both operands are then copied as contiguous 1 KB fragments, through a ring of four
// buffers, each one 32-deep K half of both tiles in fragment order, and every fragment
// read is one contiguous 1 KB a wavefront.  Step kt + 3's copies are issued while step kt
// is computed.  Waits: a wavefront's copies complete in issue order, so before step kt it
// waits until at most the eight copies of steps kt + 1 and kt + 2 are outstanding; the
// barrier then makes every wavefront's step-kt copies visible and tells it that all
// wavefronts are done reading the buffer that step kt + 3 refills.  (This ring measured
// faster than the row-major kernel's for fragment-order activations.)
constexpr int kDmaStages = 4;

template <bool TILED>
__global__ __launch_bounds__(512, 1) void gemm_dma_frag_kernel(GemmArgs p) {
  constexpr int BN = kGemmTileN, WN = 4, TM = 8, TN = 4, NT = 512;
  constexpr int FR = 512;         // bf16 per fragment
  constexpr int STAGE = 16 * FR;  // one operand's K half of a 256-row tile
  __shared__ __attribute__((aligned(16))) uint16_t sA[kDmaStages][STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kDmaStages][STAGE];
  static_assert(BN == 256, "fragment-order weight blocks are 256 rows");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  int ntile, mtile;
  tile_of_block(p.M, p.N, ntile, mtile);
  const int n0 = ntile * BN;
  const int m0 = mtile * 256;
  const int kb0 = blockIdx.z * (p.k_per_split / 64);               // first 64-deep K block of this split
  const int nkb = (min(p.K, (blockIdx.z + 1) * p.k_per_split) - blockIdx.z * p.k_per_split) / 64;
  const int nst = 2 * nkb;  // K halves
  // wavefront w copies fragments 2w and 2w + 1 of both tiles every step
  const int fa = 2 * wave;
  const int fk = (lane >> 4) * 8;
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arow[i] = p.A + ((size_t)min(m0 / 16 + fa + i, (p.M + 15) / 16 - 1) * (p.K / 32) + 2 * kb0) * FR + lane * 8;
    brow[i] = TILED ? p.W + ((size_t)(n0 / BN) * (p.K / 64) + kb0) * (BN * 64) + (size_t)(2 * (fa + i)) * FR + lane * 8
                    : p.W + (size_t)min(n0 + 16 * (fa + i) + (lane & 15), p.N - 1) * p.K + fk;
  }
  // step st's copies into buffer slot (steps past the last re-read the last one, so every
  // iteration issues and awaits the same number of copies)
  auto issue = [&](int st, int slot) {
    const int s = min(st, nst - 1);
    const int h = s & 1;
    const int kb = s >> 1;  // K block within the split
    const int k0 = (kb0 + kb) * 64 + h * 32;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(arow[i] + (2 * kb + h) * FR, &sA[slot][(fa + i) * FR], 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint16_t* src = TILED ? brow[i] + (size_t)kb * (BN * 64) + h * FR : brow[i] + k0;
      __builtin_amdgcn_global_load_lds(src, &sB[slot][(fa + i) * FR], 16, 0, 0);
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t sa0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&sA[0][0])) + (wm * TM * FR + lane * 8) * 2;
  const uint32_t sb0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&sB[0][0])) + (wn * TN * FR + lane * 8) * 2;
  // Fragments are double-buffered in registers: step kt + 1's are read from LDS while step
  // kt's MFMAs run, and awaited (every value tied to a wait) after them.
  bf16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  auto read = [&](int slot, bf16x8_t (&a)[TM], bf16x8_t (&b)[TN]) {
    const uint32_t oa = sa0 + slot * (STAGE * 2), ob = sb0 + slot * (STAGE * 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = lds_read_b128(ob + j * (FR * 2));
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = lds_read_b128(oa + i * (FR * 2));
  };
  auto await = [&](bf16x8_t (&a)[TM], bf16x8_t (&b)[TN]) {
#pragma unroll
    for (int j = 0; j < TN; ++j) lds_wait<0>(b[j]);
#pragma unroll
    for (int i = 0; i < TM; ++i) lds_wait<0>(a[i]);
  };
  auto mfma = [&](const bf16x8_t (&a)[TM], const bf16x8_t (&b)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  // iteration kt: step kt + 1's copies are in (only step kt + 2's four are outstanding),
  // the barrier publishes them and frees step kt - 1's buffer, which step kt + 3 refills
  auto step = [&](int kt, const bf16x8_t (&ca)[TM], const bf16x8_t (&cb)[TN], bf16x8_t (&na)[TM],
                  bf16x8_t (&nb)[TN]) {
    wait_vmcnt<4>();
    __builtin_amdgcn_s_barrier();
    issue(kt + 3, (kt + 3) & (kDmaStages - 1));
    read((kt + 1) & (kDmaStages - 1), na, nb);  // past the last step: a re-read copy, unused
    mfma(ca, cb);
    await(na, nb);
  };

  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  wait_vmcnt<8>();
  __builtin_amdgcn_s_barrier();
  read(0, fa0, fb0);
  await(fa0, fb0);
  for (int kt = 0; kt < nst; kt += 2) {  // nst is even
    step(kt, fa0, fb0, fa1, fb1);
    step(kt + 1, fa1, fb1, fa0, fb0);
  }
  wait_vmcnt<0>();  // the re-read copies past the last step land before the LDS is reused
  gemm_epilogue<256, WN, TM, TN, NT>(p, acc, m0, n0, wm, wn, lane, tid);
}

// NW wavefronts per workgroup, 32 weight rows each, two wavefronts per SIMD (256 registers
// each), so while one waits the other computes.  A 2-wavefront workgroup's LDS admits two
// per CU, one wavefront per SIMD, so that instance asks for one.
template <int MT, int NW, int PF, int AD, bool TILED, bool Q4>
__global__ __launch_bounds__(NW * 64, NW >= 4 ? 2 : 1) void gemm_stream_kernel(GemmArgs p) {
  constexpr int MR = MT * 16;
  // AD: activation steps in flight ahead of the one being computed (AD + 1 LDS buffers)
  __shared__ __attribute__((aligned(16))) uint16_t sA[AD + 1][MR * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw0 = blockIdx.x * (NW * 32) + wave * 32;  // first weight row of this wavefront
  const int kbeg = blockIdx.y * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg) / BK;
  using SA = StreamA<MT, NW>;
  constexpr int NB = StreamW<TILED, Q4>::LOADS;
  constexpr int NA = SA::PER;

  // Weights run PF steps ahead in registers, activations AD steps ahead in LDS.  Loads past
  // the last step re-read the last step (cache hits, never used), so every iteration has the
  // same shape and the wait counts below are exact.  The vector-memory counter retires in
  // order: waiting for step kt + 1's activations also waits for what was issued before them.
  StreamW<TILED, Q4> ring[PF];
  f32x4_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The prologue issues the same pattern as the PF iterations before step 0 would (iteration
  // i starts step i + AD's activations, then loads step i + PF's weights; it skips the
  // activations of steps before 0).  At most PF weight stages and AD activation stages are
  // ever outstanding; the counter holds 63.
  static_assert(PF * NB + AD * NA <= 63, "more vector-memory operations in flight than vmcnt counts");
  static_assert(PF >= AD, "the prologue starts step 0's activations within its PF iterations");
  // Step kt's K block is (kt + rot) mod nk, staggered across workgroups as in the LDS kernel;
  // steps past the last clamp to it.
  const int rot = nk > 0 ? static_cast<int>((blockIdx.x * kKRotate) % static_cast<unsigned>(nk)) : 0;
  auto kof = [&](int step) {
    const int q = min(step, nk - 1) + rot;
    return kbeg + (q >= nk ? q - nk : q) * BK;
  };
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    const int step = s - PF + AD;
    if (step >= 0) SA::load(p, sA[step], kof(step), wave, lane);
    ring[s].load(p, nw0, kof(s), lane);
  }
  // At the end of iteration kt, step kt + 1's activations (started AD - 1 iterations
  // earlier) are awaited: AD weight stages and AD - 1 activation stages came after them.
  // Before computing step kt its weights are awaited: PF - 1 iterations and this
  // iteration's copies came after them.
  constexpr int kWaitA = AD * NB + (AD - 1) * NA;
  constexpr int kWaitWraw = (PF - 1) * (NA + NB) + NA;
  constexpr int kWaitW = kWaitWraw > 63 ? 63 : kWaitWraw;
  wait_vmcnt<kWaitA>();
  __builtin_amdgcn_s_barrier();

  // LDS byte address of sA (the low half of its generic address)
  const uint32_t sa_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&sA[0][0]));
  const uint32_t off0 = SA::frag_offset(0, lane), off1 = SA::frag_offset(1, lane);
  // One K half at a time: its MT activation fragments are read from LDS, then its 2 * MT
  // MFMAs issue (the other wavefront on the SIMD covers the read latency).
  auto compute = [&](int buf, const StreamW<TILED, Q4>& w) {
    const uint32_t b = sa_base + buf * (MR * 64 * 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8_t af[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) af[i] = lds_read_b128(b + (h ? off1 : off0) + i * 2048);
      bf16x8_t bfr[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = w.frag(j, h);
#pragma unroll
      for (int i = 0; i < MT; ++i) lds_wait<0>(af[i]);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // Iteration kt: start step kt + AD's activations into the buffer step kt - 1 used, compute
  // step kt (weight slot kt % PF), refill weight slot kt % PF with step kt + PF, wait until
  // this wavefront's copies of step kt + 1's activations have landed, barrier.  Unrolled PF
  // times so every ring index is a compile-time constant.
  for (int kt0 = 0; kt0 < nk; kt0 += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int kt = kt0 + s;
      SA::load(p, sA[(kt + AD) % (AD + 1)], kof(kt + AD), wave, lane);
      __builtin_amdgcn_sched_barrier(0);
      ring[s].template wait<kWaitW>();
      if (kt < nk) compute(kt % (AD + 1), ring[s]);
      __builtin_amdgcn_sched_barrier(0);
      ring[s].load(p, nw0, kof(kt + PF), lane);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kWaitA>();
      __builtin_amdgcn_s_barrier();
    }
  }
  // The last PF weight stages (re-reads past the end) get their one wait here, before their
  // registers can be reused, and no copy into LDS may still be in flight when the
  // workgroup's LDS is handed on.
#pragma unroll
  for (int s = 0; s < PF; ++s) ring[s].template wait<0>();
  wait_vmcnt<0>();

  // Accumulator layout: lane holds column (lane & 15) and rows 4 * (lane >> 4) + e.
  const int mrow = (lane >> 4) * 4;
  const int ncol = nw0 + (lane & 15);
  if (p.splits > 1) {
    float* part = p.partial + (size_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mrow + i * 16 + e;
          const int n = ncol + j * 16;
          if (m < p.M && n < p.N) part[(size_t)m * p.N + n] = acc[i][j][e];
        }
    return;
  }
  if (p.epi == EPI_SILU_MUL) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; j += 2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mrow + i * 16 + e;
          const int n = ncol + j * 16;  // gate column; up is n + 16
          if (m < p.M && n < p.N) {
            const int jo = (n >> 5) * 16 + (n & 15);
            const float v = silu(acc[i][j][e]) * acc[i][j + 1][e];
            static_cast<uint16_t*>(p.out0)[(size_t)m * p.ld0 + jo] = f32_to_bf16(v);
          }
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = mrow + i * 16 + e;
        const int n = ncol + j * 16;
        if (m < p.M && n < p.N) store_out(p, m, n, acc[i][j][e]);
      }
}

// Sum of split-K partials in slice order, then the epilogue.  Each thread owns VW adjacent
// outputs (VW = 4 when N and the column split are multiples of 4, else 1); planes_sum
// issues the slices' loads in batches of eight and adds them in order 0, 1, 2, ...
template <int VW>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p) {
  const int nout = p.epi == EPI_SILU_MUL ? p.N / 2 : p.N;
  const size_t idx = ((size_t)blockIdx.x * 256 + threadIdx.x) * VW;
  if (idx >= (size_t)p.M * nout) return;
  const int m = static_cast<int>(idx / nout);
  const int n = static_cast<int>(idx % nout);
  Planes pl;
  pl.p = p.partial;
  pl.S = p.splits;
  pl.ld = p.N;
  pl.plane = (size_t)p.M * p.N;
  if (p.epi == EPI_SILU_MUL) {
    // gate columns of outputs n..n+VW-1 (within one group of 16); up columns at +16
    const int ng = (n >> 4) * 32 + (n & 15);
    float g[VW], u[VW];
    planes_sum<VW>(pl, (size_t)m * p.N + ng, g);
    planes_sum<VW>(pl, (size_t)m * p.N + ng + 16, u);
    uint16_t* o = static_cast<uint16_t*>(p.out0) + (size_t)m * p.ld0 + n;
#pragma unroll
    for (int e = 0; e < VW; ++e) o[e] = f32_to_bf16(silu(g[e]) * u[e]);
    return;
  }
  float v[VW];
  planes_sum<VW>(pl, (size_t)m * p.N + n, v);
#pragma unroll
  for (int e = 0; e < VW; ++e) store_out(p, m, n + e, v[e]);
}

constexpr int kBM = 128, kBN = kGemmTileN, kMaxSplits = 8;
constexpr int kTargetWorkgroups = 256;  // one 128 x 256 workgroup per CU (110 KB of LDS)
constexpr int kMaxSplitsSmall = 12;     // K splits when all partial planes fit kSmallPartialBytes
constexpr size_t kSmallPartialBytes = size_t(16) << 20;
// Wide-M projections with at least a round of 256 x 256 tiles take those (one workgroup per
// CU, 148 KB of LDS): each wavefront then computes a 128 x 64 block, so a K step reads 43
// flop per LDS byte instead of 32 and LDS bandwidth stops bounding the matrix units as early.
// One weight stage in flight keeps the 128 accumulators within 256 registers.
constexpr int kBigBM = 256;
constexpr int kBigSplitMinM = 512, kBigSplitMinN = 4096;  // big tiles with split K from these sizes
// 64-column workgroups (LDS or streaming) for narrow projections
constexpr int kNarrowBN = 64, kNarrowMaxN = 2048, kNarrowAnyM = 256, kNarrowStreamMinN = 512;
constexpr int kStreamMaxM = 128, kStreamMaxSplits = 16;
// Wavefronts of 32 weight rows, at most two per SIMD.  Every workgroup re-reads the activation
// slab of its K range, so fewer, wider workgroups re-read less, while more workgroups bring
// more CUs' memory pipelines to bear (one CU sustains roughly 30 GB/s of weight reads): five
// wavefronts (160 rows) balance the two for the wide and deep projections (plan_gemm).
constexpr int kStreamWavesWide = 5;
constexpr int kStreamStages = 8, kStreamStagesQ4 = 4;  // 4-bit: 10 -> 4 stages, 1.836 -> 1.752 ms a draft block
constexpr size_t kStreamMidMinWeights = size_t(16) << 20;
constexpr int kStreamMidMinN = 4096;
constexpr size_t kStreamMinWeights = size_t(64) << 20;
constexpr int kStreamMinN = 16384;
constexpr size_t kStreamMaxWaves = 2048;  // two wavefronts per SIMD on 256 CUs

__global__ __launch_bounds__(256) void tile_weights_kernel(const uint16_t* __restrict__ src, int N, int K,
                                                           const int32_t* __restrict__ rows,
                                                           uint16_t* __restrict__ dst, size_t chunks) {
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  // destination chunk c = (t * (K/64) + s) * 2048 + chunk within the block, 8 bf16 each
  constexpr int kChunks = kBN * BK / 8;
  int r, k;
  frag_chunk_pos(static_cast<int>(c % kChunks), r, k);
  const size_t ts = c / kChunks;
  const int steps = K / BK;
  const int sstep = static_cast<int>(ts % steps);
  const int t = static_cast<int>(ts / steps);
  const int n = t * kBN + r;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (n < N) {
    const size_t row = rows ? static_cast<size_t>(rows[n]) : static_cast<size_t>(n);
    v = *reinterpret_cast<const u32x4_t*>(src + row * K + sstep * BK + k);
  }
  *reinterpret_cast<u32x4_t*>(dst + c * 8) = v;
}

// Tile-contiguous 4-bit weights: per (N tile t, K step s) four 64-row groups of 576 words,
// 64 lanes x 8 packed words and then [16][4] words of scale | bias << 16 (the operand order of
// a wavefront that covers the group's 64 rows); rows past N are zero (weights 0).  rows
// (optional): destination row n takes source row rows[n].
__global__ __launch_bounds__(256) void tile_q4_kernel(const uint32_t* __restrict__ q, const uint16_t* __restrict__ sc,
                                                      const uint16_t* __restrict__ bi, int N, int K,
                                                      const int32_t* __restrict__ rows, uint32_t* __restrict__ dst,
                                                      size_t words) {
  const size_t w = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= words) return;
  constexpr int BLK = kBN * 9;
  const size_t block = w / BLK;
  const int within = static_cast<int>(w % BLK);
  const int steps = K / BK;
  const int sstep = static_cast<int>(block % steps);
  const int t = static_cast<int>(block / steps);
  uint32_t v = 0;
  const int g = within / 576, rem = within % 576;
  if (rem < 512) {
    // lane l = rem / 8, word j * 2 + half = rem % 8: row 16 j + l % 16, K word half * 4 + l / 16
    const int l = rem >> 3, jw = rem & 7;
    const int n = t * kBN + g * 64 + (jw >> 1) * 16 + (l & 15);
    if (n < N) {
      const size_t src = rows ? static_cast<size_t>(rows[n]) : static_cast<size_t>(n);
      v = q[src * (K / 8) + sstep * 8 + (jw & 1) * 4 + (l >> 4)];
    }
  } else {
    const int n = t * kBN + g * 64 + ((rem - 512) & 3) * 16 + ((rem - 512) >> 2);
    if (n < N) {
      const size_t src = rows ? static_cast<size_t>(rows[n]) : static_cast<size_t>(n);
      const size_t g = src * (K / BK) + sstep;
      v = static_cast<uint32_t>(sc[g]) | (static_cast<uint32_t>(bi[g]) << 16);
    }
  }
  dst[w] = v;
}

// One thread per 16 bytes of the fragment-order copy: thread t fills lane t % 64 of fragment
// t / 64 (row group g, K step ks) with row 16 g + lane % 16, K offsets 32 ks + 8 (lane / 16)..
__global__ __launch_bounds__(256) void tile_rows_kernel(const uint16_t* __restrict__ A, int lda, int M, int K,
                                                        uint16_t* __restrict__ dst, size_t chunks) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= chunks) return;
  const size_t f = t / 64;
  const int lane = static_cast<int>(t % 64);
  const int ksteps = K / 32;
  const int g = static_cast<int>(f / ksteps), ks = static_cast<int>(f % ksteps);
  const int row = min(16 * g + (lane & 15), M - 1);
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(A + (size_t)row * lda + 32 * ks + 8 * (lane >> 4));
  *reinterpret_cast<u32x4_t*>(dst + t * 8) = v;
}

}  // namespace

size_t tiled_rows_elems(int M, int K) { return (size_t)((M + 15) / 16) * 16 * K; }

hipError_t launch_tile_rows(const uint16_t* A, int lda, int M, int K, uint16_t* dst, hipStream_t stream) {
  if (M <= 0 || K % 32 != 0 || lda % 8 != 0 || lda < K) return hipErrorInvalidValue;
  const size_t chunks = tiled_rows_elems(M, K) / 8;
  tile_rows_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, stream>>>(A, lda, M, K, dst, chunks);
  return hipGetLastError();
}

size_t q4_tiled_words(int N, int K) { return (size_t)((N + kBN - 1) / kBN) * (K / BK) * kBN * 9; }

hipError_t launch_tile_q4(const uint32_t* q, const uint16_t* scales, const uint16_t* biases, int N, int K,
                          uint32_t* dst, hipStream_t stream, const int32_t* rows) {
  const size_t words = q4_tiled_words(N, K);
  tile_q4_kernel<<<(unsigned)((words + 255) / 256), 256, 0, stream>>>(q, scales, biases, N, K, rows, dst, words);
  return hipGetLastError();
}

size_t tiled_weight_elems(int N, int K) { return (size_t)((N + kBN - 1) / kBN) * kBN * K; }

hipError_t launch_tile_weights(const uint16_t* src, int N, int K, uint16_t* dst, hipStream_t stream,
                               const int32_t* rows) {
  const size_t chunks = tiled_weight_elems(N, K) / 8;
  tile_weights_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, stream>>>(src, N, K, rows, dst, chunks);
  return hipGetLastError();
}

// Streaming plan with nw wavefronts per workgroup: split K while the whole grid stays
// resident (two wavefronts per SIMD), every split keeps >= 4 steps and the fp32 partials
// stay within a quarter of the weight bytes (or 8 MB for small weights).
GemmPlan plan_stream(int M, int N, int K, bool tile_max, int nw) {
  GemmPlan pl;
  const int tiles = (N + nw * 32 - 1) / (nw * 32);
  const int nk = K / BK;
  const double budget = std::max(0.5 * N * K, 8.0 * 1024 * 1024);
  int s = 1;
  while (!tile_max && s < kStreamMaxSplits && (size_t)tiles * (s + 1) * nw <= kStreamMaxWaves &&
         nk / (s + 1) >= 4 && 4.0 * (s + 1) * M * N <= budget)
    ++s;
  const int per = (nk + s - 1) / s;
  pl.bm = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
  pl.bn = nw * 32;
  pl.stream_waves = nw;
  pl.k_per_split = per * BK;
  pl.splits = (nk + per - 1) / per;
  pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
  return pl;
}

// Streaming plan with nw wavefronts per workgroup and K split s ways.
GemmPlan plan_stream_split(int M, int N, int K, int nw, int s) {
  GemmPlan pl;
  const int nk = K / BK;
  const int per = (nk + s - 1) / s;
  pl.bm = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
  pl.bn = nw * 32;
  pl.stream_waves = nw;
  pl.k_per_split = per * BK;
  pl.splits = (nk + per - 1) / per;
  pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
  return pl;
}

GemmPlan plan_gemm(int M, int N, int K, bool tile_max) {
  GemmPlan pl;
  if (M <= kStreamMaxM && !tile_max && K % BK == 0) {
    // Weight-streaming plans at M <= 128, sized so that about one round of workgroups covers
    // the chip.  Wide projections (gate/up): five wavefronts (160 weight rows) per workgroup,
    // 218 workgroups for N = 34816, no split.  Deep ones (down, N = 5120, K = 17408): the same
    // workgroups with K split over 8 (256 workgroups).  Mid-size (o, N = 5120, K = 4096):
    // two-wavefront workgroups, K split to fill a round (80 x 3).  Each measured faster than
    // the 8-wavefront streaming plan and the 128 x 256 LDS kernel's split plan on these shapes.
    const size_t weights = (size_t)N * K;
    if (N >= kStreamMinN && weights >= kStreamMinWeights) {
      // more than a round of 160-row workgroups (the head's 248320 rows): 256-row ones, which
      // re-read the activations less
      const bool one_round = (N + kStreamWavesWide * 32 - 1) / (kStreamWavesWide * 32) <= kTargetWorkgroups;
      return plan_stream(M, N, K, false, one_round ? kStreamWavesWide : 8);
    }
    const int nk = K / BK;
    if (weights >= kStreamMinWeights) {
      const int tiles = (N + kStreamWavesWide * 32 - 1) / (kStreamWavesWide * 32);
      int s = std::max(1, std::min(kMaxSplits, kTargetWorkgroups / tiles));
      while (s > 1 && nk / s < 4) --s;
      return plan_stream_split(M, N, K, kStreamWavesWide, s);
    }
    if (N >= kStreamMidMinN && weights >= kStreamMidMinWeights) {
      const int tiles = (N + 63) / 64;
      const int s = kTargetWorkgroups / tiles;
      if (s >= 2 && tiles * s >= kTargetWorkgroups * 7 / 8 && nk / s >= 4) return plan_stream_split(M, N, K, 2, s);
    }
  }
  pl.bm = kBM;
  pl.bn = kBN;
  if (M > kBM && (size_t)((M + kBigBM - 1) / kBigBM) * ((N + kBN - 1) / kBN) >= (size_t)kTargetWorkgroups) {
    pl.bm = kBigBM;
    pl.k_per_split = K;
    // A last round of workgroups at most half full (gate/up at M = 1024: 544 tiles, 32 in the
    // third round) would take a whole tile's time on a few CUs: the weight rows of that round
    // run as a second launch whose tiles split K over the whole chip.  Weight-major shapes
    // only (N > M), whose full rounds are whole N tiles once the M tiles are grouped.
    const int mt = (M + kBigBM - 1) / kBigBM, nt = (N + kBN - 1) / kBN;
    const int full = (mt * nt / kTargetWorkgroups) * kTargetWorkgroups;
    const int rest = mt * nt - full;
    if (N > M && rest > 0 && 2 * rest <= kTargetWorkgroups && full % mt == 0 && K % BK == 0) {
      const int nt_tail = nt - full / mt;
      const int nkb = K / BK;
      int sp = std::max(1, std::min(kMaxSplits, kTargetWorkgroups / (mt * nt_tail)));
      while (sp > 1 && nkb / sp < 4) --sp;
      if (sp > 1) {
        const int per = (nkb + sp - 1) / sp;
        pl.tail_n = (full / mt) * kBN;
        pl.tail_k_per_split = per * BK;
        pl.tail_splits = (nkb + per - 1) / per;
        pl.partial_bytes = (size_t)pl.tail_splits * M * (N - pl.tail_n) * sizeof(float);
      }
    }
    return pl;
  }
  // Enough rows for 256 x 256 tiles but too few tiles for a round (the layer projections of a
  // 64-request block: o and down give 80 tiles, q|k|v 96): split K until they fill it.  The
  // 128-row tiles would need half as many splits but move twice the operand bytes per flop.
  if (M >= kBigSplitMinM && N >= kBigSplitMinN && K % BK == 0) {
    const int bt = ((M + kBigBM - 1) / kBigBM) * ((N + kBN - 1) / kBN);
    const int nkb = K / BK;
    int s = std::max(1, std::min(kMaxSplits, kTargetWorkgroups / bt));
    while (s > 1 && nkb / s < 4) --s;
    const int per = (nkb + s - 1) / s;
    pl.bm = kBigBM;
    pl.k_per_split = per * BK;
    pl.splits = (nkb + per - 1) / per;
    pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
    return pl;
  }
  // The kernel projection at M <= 128 (N = 1280): two-wavefront streaming workgroups of 64
  // weight rows with K split to about three quarters of a round (20 x 10 = 200 workgroups).
  // Measured in the draft block against the 128 x 64 LDS kernel with 12 splits: 1.691 ->
  // 1.680 ms a step (8 splits: 1.686, 12: 1.688); fewer planes also shorten the conv that
  // sums them.
  if (!tile_max && M <= kBM && N >= kNarrowStreamMinN && N <= kNarrowMaxN && K % BK == 0) {
    const int tiles = (N + 63) / 64;
    int s = std::max(1, std::min(kMaxSplitsSmall, (kTargetWorkgroups * 3 / 4 + tiles - 1) / tiles));
    while (s > 1 && K / BK / s < 4) --s;
    return plan_stream_split(M, N, K, 2, s);
  }
  // Narrow projections at M <= 128 below that (the selector's, N = 64): 64-column
  // workgroups of two wavefronts, two per CU, K split deep (each workgroup's short K loop is
  // the time) (at any M when N <= 256: one 256-column tile would load mostly clamped
  // duplicate rows)
  const bool narrow = !tile_max && ((M <= kBM && N <= kNarrowMaxN) || N <= kNarrowAnyM);
  if (narrow) pl.bn = kNarrowBN;
  const int tiles = ((M + kBM - 1) / kBM) * ((N + pl.bn - 1) / pl.bn);
  const int nk = K / BK;
  const int target = narrow ? 2 * kTargetWorkgroups : kTargetWorkgroups;
  // Narrow projections whose partial planes stay small (the kernel projection: 0.66 MB a
  // plane) split deeper: with few tiles each workgroup's serial K loop is the time, and the
  // consumers read the extra planes in batches.
  const size_t plane = (size_t)M * N * sizeof(float);
  const bool small = plane * kMaxSplitsSmall <= kSmallPartialBytes;
  const int max_splits = small ? kMaxSplitsSmall : kMaxSplits;
  const int min_steps = small ? 4 : 6;
  int s = 1;
  while (s < max_splits && tiles * (s + 1) <= target && nk / (s + 1) >= min_steps) ++s;
  int per = (nk + s - 1) / s;
  pl.k_per_split = per * BK;
  pl.splits = (nk + per - 1) / per;
  pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
  return pl;
}

namespace {

GemmArgs make_args(const GemmPlan& pl, const uint16_t* A, int lda, const WeightRef& W, int M, int N, int K, int epi,
                   void* out0, int ld0, void* out1, int ld1, int nsplit, float* partial, float* tile_max,
                   uint32_t* tile_bound = nullptr, bool a_tiled = false) {
  GemmArgs p;
  p.A = A;
  p.W = W.w;
  p.Wq = W.q;
  p.Ws = W.scales;
  p.Wb = W.biases;
  p.lda = lda;
  p.M = M;
  p.N = N;
  p.K = K;
  p.k_per_split = pl.k_per_split;
  p.epi = epi;
  p.out0 = out0;
  p.ld0 = ld0;
  p.out1 = out1;
  p.ld1 = ld1;
  p.nsplit = epi == EPI_F32 ? (out1 ? nsplit : N) : N;
  p.partial = partial;
  p.splits = pl.splits;
  p.tile_max = tile_max;
  p.tile_bound = tile_max ? tile_bound : nullptr;
  p.a_tiled = a_tiled ? 1 : 0;
  return p;
}

// Weight stages in flight: a bf16 stage is 4 loads (4 KB), a 4-bit stage 2 (1.1 KB); the
// depth keeps a wavefront within 256 registers next to its accumulators.  At 128 rows four
// stages run faster than six (gate/up 84 -> 79 us a launch by events, down 52 -> 49): with
// every workgroup's loads in flight at once, deeper rings only add queueing in the memory
// system, and three to five stages measured within noise of each other.
template <int MT, int NW>
hipError_t launch_stream_mt(const GemmArgs& p, const WeightRef& W, hipStream_t stream) {
  const dim3 grid((p.N + NW * 32 - 1) / (NW * 32), p.splits);
  if (W.q) {
    gemm_stream_kernel<MT, NW, kStreamStagesQ4, 3, true, true><<<grid, NW * 64, 0, stream>>>(p);
  } else {
    // at 8 row fragments (128 rows) four stages
    constexpr int PF = MT == 8 ? 4 : kStreamStages;
    if (W.tiled)
      gemm_stream_kernel<MT, NW, PF, 3, true, false><<<grid, NW * 64, 0, stream>>>(p);
    else
      gemm_stream_kernel<MT, NW, PF, 3, false, false><<<grid, NW * 64, 0, stream>>>(p);
  }
  return hipGetLastError();
}

template <int NW>
hipError_t launch_stream_nw(const GemmArgs& p, const GemmPlan& pl, const WeightRef& W, hipStream_t stream) {
  switch (pl.bm) {
    case 16: return launch_stream_mt<1, NW>(p, W, stream);
    case 32: return launch_stream_mt<2, NW>(p, W, stream);
    case 64: return launch_stream_mt<4, NW>(p, W, stream);
    default: return launch_stream_mt<8, NW>(p, W, stream);
  }
}

hipError_t launch_stream(const GemmArgs& p, const GemmPlan& pl, const WeightRef& W, hipStream_t stream) {
  switch (pl.stream_waves) {
    case 8: return launch_stream_nw<8>(p, pl, W, stream);
    case 5: return launch_stream_nw<5>(p, pl, W, stream);
    case 2: return launch_stream_nw<2>(p, pl, W, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_main(const GemmArgs& p, const GemmPlan& pl, const WeightRef& W, hipStream_t stream) {
  // Row-major 4-bit weights (a one-off projection) take the LDS kernel with the same split
  // plan: loaded by hand their sixteen scalar loads a stage leave the streaming kernel short
  // of registers, and the compiler would then move values still in flight.
  if (pl.stream_waves > 0 && (W.tiled || !W.q)) {
    if (p.M > pl.bm) return hipErrorInvalidValue;
    return launch_stream(p, pl, W, stream);
  }
  if (pl.bm == kBigBM) {
    if (pl.k_per_split % BK != 0) return hipErrorInvalidValue;
    const dim3 grid((p.N + kBN - 1) / kBN, (p.M + kBigBM - 1) / kBigBM, pl.splits);
    if (W.q) {
      if (W.tiled)
        gemm_bf16_kernel<kBigBM, kBN, BK, 2, 4, 1, 1, true, true><<<grid, 512, 0, stream>>>(p);
      else
        gemm_bf16_kernel<kBigBM, kBN, BK, 2, 4, 1, 1, false, true><<<grid, 512, 0, stream>>>(p);
    } else {
      if (p.a_tiled) {
        if (W.tiled)
          gemm_dma_frag_kernel<true><<<grid, 512, 0, stream>>>(p);
        else
          gemm_dma_frag_kernel<false><<<grid, 512, 0, stream>>>(p);
      } else if (W.tiled) {
        gemm_dma_kernel<true><<<grid, 512, 0, stream>>>(p);
      } else {
        gemm_dma_kernel<false><<<grid, 512, 0, stream>>>(p);
      }
    }
    return hipGetLastError();
  }
  if (pl.bn == kNarrowBN && !W.q) {
    const dim3 grid((p.N + kNarrowBN - 1) / kNarrowBN, (p.M + kBM - 1) / kBM, pl.splits);
    if (W.tiled)
      gemm_bf16_kernel<kBM, kNarrowBN, BK, 2, 1, 2, 1, true><<<grid, 128, 0, stream>>>(p);
    else
      gemm_bf16_kernel<kBM, kNarrowBN, BK, 2, 1, 2, 1, false><<<grid, 128, 0, stream>>>(p);
    return hipGetLastError();
  }
  // (4-bit weights keep 256-column workgroups under a narrow plan: the same K splits)
  const dim3 grid((p.N + kBN - 1) / kBN, (p.M + kBM - 1) / kBM, pl.splits);
  if (W.q) {
    if (W.tiled)
      gemm_bf16_kernel<kBM, kBN, BK, 2, 4, 2, 1, true, true><<<grid, 512, 0, stream>>>(p);
    else
      gemm_bf16_kernel<kBM, kBN, BK, 2, 4, 2, 1, false, true><<<grid, 512, 0, stream>>>(p);
  } else {
    if (W.tiled)
      gemm_bf16_kernel<kBM, kBN, BK, 2, 4, 2, 1, true><<<grid, 512, 0, stream>>>(p);
    else
      gemm_bf16_kernel<kBM, kBN, BK, 2, 4, 2, 1, false><<<grid, 512, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const GemmArgs& p, hipStream_t stream) {
  const int nout = p.epi == EPI_SILU_MUL ? p.N / 2 : p.N;
  if (nout % 4 == 0 && p.nsplit % 4 == 0) {
    const size_t quads = (size_t)p.M * nout / 4;
    splitk_reduce_kernel<4><<<(unsigned)((quads + 255) / 256), 256, 0, stream>>>(p);
  } else {
    const size_t total = (size_t)p.M * nout;
    splitk_reduce_kernel<1><<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmPlan& pl, const uint16_t* A, int lda, const WeightRef& W, int M, int N, int K,
                       int epi, void* out0, int ld0, void* out1, int ld1, int nsplit, float* partial,
                       hipStream_t stream, float* tile_max, uint32_t* tile_bound, bool a_tiled) {
  // tile maxima come from the LDS kernel's epilogue (one 256-column tile per workgroup); a
  // tile may not straddle the two outputs
  if (tile_max && (epi != EPI_F32 || pl.splits != 1 || pl.stream_waves > 0 ||
                   (out1 && nsplit % kGemmTileN != 0)))
    return hipErrorInvalidValue;
  if (a_tiled && !gemm_takes_tiled_a(pl, W.q != nullptr)) return hipErrorInvalidValue;
  if (W.q && K % BK != 0) return hipErrorInvalidValue;
  if (pl.tail_n > 0 && pl.splits == 1 && !tile_max && !W.q && !out1 && pl.tail_n < N) {
    // the full rounds: weight rows [0, tail_n) into the matching output columns
    GemmPlan pm = pl;
    pm.tail_n = 0;
    const GemmArgs pa = make_args(pm, A, lda, W, M, pl.tail_n, K, epi, out0, ld0, nullptr, 0, pl.tail_n, partial,
                                  nullptr, nullptr, a_tiled);
    hipError_t e = launch_main(pa, pm, W, stream);
    if (e != hipSuccess) return e;
    // the rest with split K: weights from row tail_n (a whole tile-contiguous tile boundary),
    // outputs from the matching column (half of it for SiLU(gate) * up)
    WeightRef wt = W;
    wt.w = W.tiled ? W.w + (size_t)(pl.tail_n / kBN) * (K / BK) * (kBN * BK) : W.w + (size_t)pl.tail_n * K;
    const int nt = N - pl.tail_n;
    void* o = epi == EPI_SILU_MUL ? static_cast<void*>(static_cast<uint16_t*>(out0) + pl.tail_n / 2)
            : epi == EPI_BF16     ? static_cast<void*>(static_cast<uint16_t*>(out0) + pl.tail_n)
                                  : static_cast<void*>(static_cast<float*>(out0) + pl.tail_n);
    GemmPlan pt = pm;
    pt.splits = pl.tail_splits;
    pt.k_per_split = pl.tail_k_per_split;
    const GemmArgs pb = make_args(pt, A, lda, wt, M, nt, K, epi, o, ld0, nullptr, 0, nt, partial, nullptr, nullptr,
                                  a_tiled);
    e = launch_main(pb, pt, wt, stream);
    if (e != hipSuccess) return e;
    return launch_reduce(pb, stream);
  }
  const GemmArgs p = make_args(pl, A, lda, W, M, N, K, epi, out0, ld0, out1, ld1, nsplit, partial, tile_max,
                               tile_bound, a_tiled);
  hipError_t e = launch_main(p, pl, W, stream);
  if (e != hipSuccess || pl.splits == 1) return e;
  return launch_reduce(p, stream);
}

hipError_t launch_gemm(const GemmPlan& pl, const uint16_t* A, int lda, const uint16_t* W, bool w_tiled,
                       int M, int N, int K, int epi, void* out0, int ld0, void* out1, int ld1, int nsplit,
                       float* partial, hipStream_t stream, float* tile_max, uint32_t* tile_bound, bool a_tiled) {
  WeightRef w;
  w.w = W;
  w.tiled = w_tiled;
  return launch_gemm(pl, A, lda, w, M, N, K, epi, out0, ld0, out1, ld1, nsplit, partial, stream, tile_max,
                     tile_bound, a_tiled);
}

hipError_t launch_gemm_partials(const GemmPlan& pl, const uint16_t* A, int lda, const WeightRef& W, int M, int N,
                                int K, float* partial, hipStream_t stream) {
  // one split: the plain fp32 result is plane 0
  const GemmArgs p = make_args(pl, A, lda, W, M, N, K, EPI_F32, partial, N, nullptr, 0, N, partial, nullptr);
  return launch_main(p, pl, W, stream);
}

namespace {
hipError_t planes_sum_as(const Planes& src, int M, int N, int epi, void* out, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (src.ld != N || src.plane != (size_t)M * N || src.S < 1) return hipErrorInvalidValue;
  GemmArgs p = {};
  p.M = M;
  p.N = N;
  p.epi = epi;
  p.out0 = out;
  p.ld0 = N;
  p.nsplit = N;
  p.partial = const_cast<float*>(src.p);
  p.splits = src.S;
  return launch_reduce(p, stream);
}
}  // namespace

hipError_t launch_planes_sum(const Planes& src, int M, int N, float* out, hipStream_t stream) {
  return planes_sum_as(src, M, N, EPI_F32, out, stream);
}

hipError_t launch_planes_sum_bf16(const Planes& src, int M, int N, uint16_t* out, hipStream_t stream) {
  return planes_sum_as(src, M, N, EPI_BF16, out, stream);
}

hipError_t launch_gemm_partials(const GemmPlan& pl, const uint16_t* A, int lda, const uint16_t* W,
                                bool w_tiled, int M, int N, int K, float* partial, hipStream_t stream) {
  WeightRef w;
  w.w = W;
  w.tiled = w_tiled;
  return launch_gemm_partials(pl, A, lda, w, M, N, K, partial, stream);
}

}  // namespace dfl
