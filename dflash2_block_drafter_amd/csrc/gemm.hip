// Dense projections y = x . W^T on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Every projection of the drafter multiplies activations by a weight stored [out, in]
// (dflash2.ts diff, `Bf16Projection`), so both operands are K-contiguous: each lane
// loads 16 contiguous bytes of one row for either MFMA operand and no transpose is
// needed.  A and W tiles are staged through LDS with double buffering (one barrier per
// 64-wide K step); global loads of step k+1 are in flight while step k computes.
//
// Split-K: grid.z slices K; slices write fp32 partials and a separate kernel sums them
// in slice order (deterministic, no float atomics) and applies the epilogue.
#include "common.hpp"
#include "kernels.hpp"

namespace dfl {

namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // 144-byte rows: 16-byte reads of 16 rows hit distinct banks

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

// W rows for EPI_SILU_MUL are interleaved per 16: [gate 16 | up 16] ... so output
// column j pairs accumulator columns (j/16)*32 + j%16 (gate) and +16 (up).
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 16;
  constexpr int TN = BN / WN / 16;
  constexpr int A_PER = BM * BK / 8 / NT;
  constexpr int B_PER = BN * BK / 8 / NT;
  static_assert(A_PER * NT * 8 == BM * BK, "A tile must split evenly over threads");
  static_assert(B_PER * NT * 8 == BN * BK, "B tile must split evenly over threads");
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
  const int nk = (kend - kbeg) / BK;

  u32x4_t ra[A_PER], rb[B_PER];
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 3;
      const int kc = (c & 7) * 8;
      const int gm = m0 + r;
      ra[i] = gm < p.M ? *reinterpret_cast<const u32x4_t*>(p.A + (size_t)gm * p.lda + k0 + kc) : zero;
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 3;
      const int kc = (c & 7) * 8;
      const int gn = n0 + r;
      rb[i] = gn < p.N ? *reinterpret_cast<const u32x4_t*>(p.W + (size_t)gn * p.K + k0 + kc) : zero;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(&sA[buf][(c >> 3) * LDS_STRIDE + (c & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(&sB[buf][(c >> 3) * LDS_STRIDE + (c & 7) * 8]) = rb[i];
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    gload(kbeg);
    sstore(0);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kbeg + (kt + 1) * BK);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
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
    if (kt + 1 < nk) sstore(buf ^ 1);
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
}

// Sum of split-K partials in slice order, then the epilogue.  One thread per output.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p) {
  const int nout = p.epi == EPI_SILU_MUL ? p.N / 2 : p.N;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)p.M * nout) return;
  const int m = static_cast<int>(idx / nout);
  const int n = static_cast<int>(idx % nout);
  const size_t plane = (size_t)p.M * p.N;
  if (p.epi == EPI_SILU_MUL) {
    const int ng = (n >> 4) * 32 + (n & 15);
    float g = 0.f, u = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      g += p.partial[s * plane + (size_t)m * p.N + ng];
      u += p.partial[s * plane + (size_t)m * p.N + ng + 16];
    }
    static_cast<uint16_t*>(p.out0)[(size_t)m * p.ld0 + n] = f32_to_bf16(silu(g) * u);
    return;
  }
  float v = 0.f;
  for (int s = 0; s < p.splits; ++s) v += p.partial[s * plane + (size_t)m * p.N + n];
  store_out(p, m, n, v);
}

struct TileCfg {
  int bm, bn;
};

TileCfg pick_tile(int M) { return M <= 128 ? TileCfg{128, 64} : TileCfg{128, 128}; }

int pick_splits(int M, int N, int K, TileCfg t) {
  const int tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  const int nk = K / BK;
  int s = 1;
  while (tiles * s < 512 && nk / (s * 2) >= 8) s *= 2;
  return s;
}

}  // namespace

GemmPlan plan_gemm(int M, int N, int K) {
  const TileCfg t = pick_tile(M);
  GemmPlan pl;
  pl.bm = t.bm;
  pl.bn = t.bn;
  int s = pick_splits(M, N, K, t);
  const int nk = K / BK;
  int per = (nk + s - 1) / s;
  pl.k_per_split = per * BK;
  pl.splits = (nk + per - 1) / per;
  pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
  return pl;
}

hipError_t launch_gemm(const GemmPlan& pl, const uint16_t* A, int lda, const uint16_t* W, int M,
                       int N, int K, int epi, void* out0, int ld0, void* out1, int ld1,
                       int nsplit, float* partial, hipStream_t stream) {
  GemmArgs p;
  p.A = A;
  p.W = W;
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
  dim3 grid((N + pl.bn - 1) / pl.bn, (M + pl.bm - 1) / pl.bm, pl.splits);
  if (pl.bm == 128 && pl.bn == 64) {
    gemm_bf16_kernel<128, 64, 2, 2><<<grid, 256, 0, stream>>>(p);
  } else {
    gemm_bf16_kernel<128, 128, 2, 2><<<grid, 256, 0, stream>>>(p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  const int nout = epi == EPI_SILU_MUL ? N / 2 : N;
  const size_t total = (size_t)M * nout;
  splitk_reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace dfl
