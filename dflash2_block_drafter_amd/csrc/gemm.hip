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
// Split-K: grid.z slices K; slices write fp32 partials and a separate kernel sums them
// in slice order (deterministic, no float atomics) and applies the epilogue, or the
// partials are left for the consuming kernel, which sums them in the same order.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

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
  float* tile_max;  // EPI_F32, one split: [M, gridDim.x] row maxima of each BN-column tile
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

// Loads one K step of the A tile [BM x BKS] and the W tile [BN x BKS] into registers.
// TILED: W is stored tile-contiguous, [N/BN][K/BKS][BN][BKS], so one step of one tile is
// a single contiguous BN*BKS*2-byte block; otherwise W is row-major [N, K].
template <int BM, int BN, int BKS, int NT, bool TILED>
struct TileLoader {
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
      const uint16_t* tile = p.W + ((size_t)(n0 / BN) * (p.K / BKS) + k0 / BKS) * (BN * BKS);
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
      *reinterpret_cast<u32x4_t*>(&sB[(c / CPR) * LS + (c % CPR) * 8]) = b[i];
    }
  }
};

// 4-bit affine weights ([P2] `quantizedWeight`: groups of 64 inputs, w = scale * q + bias).
// A K step is one group per row: each thread loads one 16-byte chunk of packed fields (32
// weights of one row) and that row's (scale, bias), and dequantizes in fp32 (one fma per
// weight, rounded once to bf16) while parking the step in LDS, so the tile compute is the
// bf16 one.  TILED: per (N tile, K step) a block of BN rows x 8 words followed by BN words
// of scale | bias << 16, written once by tile_q4_kernel.
template <int BM, int BN, int BKS, int NT, bool TILED>
struct TileLoaderQ4 {
  static constexpr int CPR = BKS / 8;
  static constexpr int A_PER = BM * CPR / NT;
  static_assert(A_PER * NT == BM * CPR, "A tile must split evenly over threads");
  static_assert(BKS == 64 && BN * 2 == NT, "one 16-byte chunk of packed fields per thread");
  u32x4_t a[A_PER];
  u32x4_t w;
  uint32_t sb;

  __device__ __forceinline__ void load(const GemmArgs& p, int m0, int n0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      const int gm = min(m0 + c / CPR, p.M - 1);
      a[i] = *reinterpret_cast<const u32x4_t*>(p.A + (size_t)gm * p.lda + k0 + (c % CPR) * 8);
    }
    const int row = tid >> 1, half = tid & 1;
    if (TILED) {
      const uint32_t* blk = p.Wq + ((size_t)(n0 / BN) * (p.K / BKS) + k0 / BKS) * (BN * 9);
      w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(blk + row * 8 + half * 4));
      sb = blk[BN * 8 + row];
    } else {
      const int gn = min(n0 + row, p.N - 1);
      w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.Wq + (size_t)gn * (p.K / 8) + k0 / 8 + half * 4));
      const size_t g = (size_t)gn * (p.K / BKS) + k0 / BKS;
      sb = static_cast<uint32_t>(p.Ws[g]) | (static_cast<uint32_t>(p.Wb[g]) << 16);
    }
  }
  __device__ __forceinline__ void store(uint16_t* sA, uint16_t* sB, int tid) const {
    constexpr int LS = BKS + 8;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(&sA[(c / CPR) * LS + (c % CPR) * 8]) = a[i];
    }
    const float sc = bf16_to_f32(static_cast<uint16_t>(sb & 0xFFFFu));
    const float bi = bf16_to_f32(static_cast<uint16_t>(sb >> 16));
    const int row = tid >> 1, half = tid & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = fmaf(sc, static_cast<float>((w[j] >> (4 * e)) & 0xFu), bi);
      *reinterpret_cast<u32x4_t*>(&sB[row * LS + half * 32 + j * 8]) = pack8(f);
    }
  }
};

// W rows for EPI_SILU_MUL are interleaved per 16: [gate 16 | up 16] ... so output
// column j pairs accumulator columns (j/16)*32 + j%16 (gate) and +16 (up).
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
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int kbeg = blockIdx.z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg) / BKS;

  Loader ring[PF];
  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (s < nk) ring[s].load(p, m0, n0, kbeg + s * BKS, tid);
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
      ring[s].load(p, m0, n0, kbeg + (kt + PF) * BKS, tid);
      __syncthreads();
      compute(kt & 1);
      ring[(s + 1) % PF].store(sA[(kt + 1) & 1], sB[(kt + 1) & 1], tid);
    }
  }
#pragma unroll
  for (int s = 0; s < 2 * PF; ++s) {
    const int kt = kt0 + s;
    if (kt < nk) {
      if (kt + PF < nk) ring[s % PF].load(p, m0, n0, kbeg + (kt + PF) * BKS, tid);
      __syncthreads();
      compute(kt & 1);
      if (kt + 1 < nk) ring[(s + 1) % PF].store(sA[(kt + 1) & 1], sB[(kt + 1) & 1], tid);
    }
  }

  // Accumulator layout: lane holds column (lane & 15) and rows 4*(lane >> 4) + e.
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
  if (p.tile_max) {
    // Row maxima of this tile over its columns < N: within a lane over its TN columns, then
    // over the 16 lanes that share a row, then over the WN wavefronts through LDS.  fmaxf
    // skips NaN, so a tile's maximum is NaN only when all of its values are.
    __shared__ float rmax[WN][BM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = -INFINITY;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          if (ncol + j * 16 < p.N) v = fmaxf(v, acc[i][j][e]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
        if ((lane & 15) == 0) rmax[wn][wm * (TM * 16) + i * 16 + (lane >> 4) * 4 + e] = v;
      }
    __syncthreads();
    for (int r = tid; r < BM; r += NT) {
      const int m = m0 + r;
      if (m < p.M) {
        float v = rmax[0][r];
#pragma unroll
        for (int w = 1; w < WN; ++w) v = fmaxf(v, rmax[w][r]);
        p.tile_max[(size_t)m * gridDim.x + blockIdx.x] = v;
      }
    }
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

__global__ __launch_bounds__(256) void tile_weights_kernel(const uint16_t* __restrict__ src, int N, int K,
                                                           const int32_t* __restrict__ rows,
                                                           uint16_t* __restrict__ dst, size_t chunks) {
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  // destination chunk c = ((t * (K/64) + s) * 256 + r) * 8 + q, 8 bf16 each
  const int q = static_cast<int>(c & 7);
  const size_t rest = c >> 3;
  const int r = static_cast<int>(rest % kBN);
  const size_t ts = rest / kBN;
  const int steps = K / BK;
  const int sstep = static_cast<int>(ts % steps);
  const int t = static_cast<int>(ts / steps);
  const int n = t * kBN + r;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (n < N) {
    const size_t row = rows ? static_cast<size_t>(rows[n]) : static_cast<size_t>(n);
    v = *reinterpret_cast<const u32x4_t*>(src + row * K + sstep * BK + q * 8);
  }
  *reinterpret_cast<u32x4_t*>(dst + c * 8) = v;
}

// Tile-contiguous 4-bit weights: per (N tile t, K step s) a block of kBN rows x 8 packed words
// followed by kBN words of scale | bias << 16; rows past N are zero (weights 0).  rows
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
  if (within < kBN * 8) {
    const int n = t * kBN + within / 8;
    if (n < N) {
      const size_t src = rows ? static_cast<size_t>(rows[n]) : static_cast<size_t>(n);
      v = q[src * (K / 8) + sstep * 8 + within % 8];
    }
  } else {
    const int n = t * kBN + (within - kBN * 8);
    if (n < N) {
      const size_t src = rows ? static_cast<size_t>(rows[n]) : static_cast<size_t>(n);
      const size_t g = src * (K / BK) + sstep;
      v = static_cast<uint32_t>(sc[g]) | (static_cast<uint32_t>(bi[g]) << 16);
    }
  }
  dst[w] = v;
}

}  // namespace

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

GemmPlan plan_gemm(int M, int N, int K) {
  GemmPlan pl;
  pl.bm = kBM;
  pl.bn = kBN;
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int nk = K / BK;
  int s = 1;
  while (s < kMaxSplits && tiles * (s + 1) <= kTargetWorkgroups && nk / (s + 1) >= 6) ++s;
  int per = (nk + s - 1) / s;
  pl.k_per_split = per * BK;
  pl.splits = (nk + per - 1) / per;
  pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
  return pl;
}

namespace {

GemmArgs make_args(const GemmPlan& pl, const uint16_t* A, int lda, const WeightRef& W, int M, int N, int K, int epi,
                   void* out0, int ld0, void* out1, int ld1, int nsplit, float* partial, float* tile_max) {
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
  return p;
}

hipError_t launch_main(const GemmArgs& p, const GemmPlan& pl, const WeightRef& W, hipStream_t stream) {
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
                       hipStream_t stream, float* tile_max) {
  if (tile_max && (epi != EPI_F32 || pl.splits != 1)) return hipErrorInvalidValue;
  if (W.q && K % BK != 0) return hipErrorInvalidValue;
  const GemmArgs p = make_args(pl, A, lda, W, M, N, K, epi, out0, ld0, out1, ld1, nsplit, partial, tile_max);
  hipError_t e = launch_main(p, pl, W, stream);
  if (e != hipSuccess || pl.splits == 1) return e;
  return launch_reduce(p, stream);
}

hipError_t launch_gemm(const GemmPlan& pl, const uint16_t* A, int lda, const uint16_t* W, bool w_tiled,
                       int M, int N, int K, int epi, void* out0, int ld0, void* out1, int ld1, int nsplit,
                       float* partial, hipStream_t stream, float* tile_max) {
  WeightRef w;
  w.w = W;
  w.tiled = w_tiled;
  return launch_gemm(pl, A, lda, w, M, N, K, epi, out0, ld0, out1, ld1, nsplit, partial, stream, tile_max);
}

hipError_t launch_gemm_partials(const GemmPlan& pl, const uint16_t* A, int lda, const WeightRef& W, int M, int N,
                                int K, float* partial, hipStream_t stream) {
  // one split: the plain fp32 result is plane 0
  const GemmArgs p = make_args(pl, A, lda, W, M, N, K, EPI_F32, partial, N, nullptr, 0, N, partial, nullptr);
  return launch_main(p, pl, W, stream);
}

hipError_t launch_gemm_partials(const GemmPlan& pl, const uint16_t* A, int lda, const uint16_t* W,
                                bool w_tiled, int M, int N, int K, float* partial, hipStream_t stream) {
  WeightRef w;
  w.w = W;
  w.tiled = w_tiled;
  return launch_gemm_partials(pl, A, lda, w, M, N, K, partial, stream);
}

}  // namespace dfl
