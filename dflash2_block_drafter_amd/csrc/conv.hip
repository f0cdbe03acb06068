// Two-tap grouped dynamic depthwise conv along each block's rows (dflash2.ts diff: header
// conv equation, `#coefficients`, `#conv`; MAX DFlash2GroupedConv: prepare/finish):
//   out[t,c] = (base[side,0,c] + D[t,0,c/grp]) * y[t,c]
//            + (base[side,1,c] + D[t,1,c/grp]) * y[t-1,c],   y[t-1] = 0 when t % G == 0
// optionally plus a residual, summed in fp32 and rounded once to bf16.
//
// One thread owns 8 channels (one 16-byte load) of one row, so a 256-thread workgroup
// covers 2048 contiguous channels and every load is coalesced.  Both rows t and t-1 are
// read by the thread; the t-1 read of a row hits in cache behind its own row's reader.
// The block boundary is structural: the t-1 load is skipped at t % G == 0.
#include "common.hpp"
#include "kernels.hpp"

namespace dfl {

namespace {

__global__ __launch_bounds__(256) void conv_kernel(const uint16_t* __restrict__ y,
                                                   const float* __restrict__ coef, int ldc,
                                                   const uint16_t* __restrict__ base, int side,
                                                   int H, int G, int grp,
                                                   const uint16_t* residual, uint16_t* out) {
  const int t = blockIdx.y;
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c0 >= H) return;
  const int ng = H / grp;
  const int g = c0 / grp;
  const float d0 = coef[(size_t)t * ldc + g];
  const float d1 = coef[(size_t)t * ldc + ng + g];
  float cur[8], prev[8], b0[8], b1[8];
  unpack8(*reinterpret_cast<const u32x4_t*>(y + (size_t)t * H + c0), cur);
  if (t % G != 0) {
    unpack8(*reinterpret_cast<const u32x4_t*>(y + (size_t)(t - 1) * H + c0), prev);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) prev[e] = 0.f;
  }
  unpack8(*reinterpret_cast<const u32x4_t*>(base + (size_t)(side * 2 + 0) * H + c0), b0);
  unpack8(*reinterpret_cast<const u32x4_t*>(base + (size_t)(side * 2 + 1) * H + c0), b1);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (b0[e] + d0) * cur[e] + (b1[e] + d1) * prev[e];
  if (residual) {
    float r[8];
    unpack8(*reinterpret_cast<const u32x4_t*>(residual + (size_t)t * H + c0), r);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = r[e] + o[e];
  }
  *reinterpret_cast<u32x4_t*>(out + (size_t)t * H + c0) = pack8(o);
}

// conv finish + residual + the next sublayer's RMSNorm, one workgroup per row: the row's
// new residual stays in registers between the conv and the norm, so x is written once and
// the norm costs no extra read (dflash2.ts diff, `#block`: x = bf16(x + Conv1(..)), then
// m = rms(x) opens the next sublayer).
template <int MAXC>
__global__ __launch_bounds__(256) void conv_residual_norm_kernel(
    const uint16_t* __restrict__ y, const float* __restrict__ coef, int ldc,
    const uint16_t* __restrict__ base, int H, int G, int grp, const uint16_t* residual,
    uint16_t* x_out, const uint16_t* __restrict__ gamma, float eps, uint16_t* __restrict__ n_out) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int ng = H / grp;
  const int chunks = H >> 3;
  const bool has_prev = (t % G) != 0;
  float xv[MAXC][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = tid + i * 256;
    if (ch < chunks) {
      const int c0 = ch * 8;
      const int g = c0 / grp;
      const float d0 = coef[(size_t)t * ldc + g];
      const float d1 = coef[(size_t)t * ldc + ng + g];
      float cur[8], prev[8], b0[8], b1[8], r[8];
      unpack8(*reinterpret_cast<const u32x4_t*>(y + (size_t)t * H + c0), cur);
      if (has_prev) {
        unpack8(*reinterpret_cast<const u32x4_t*>(y + (size_t)(t - 1) * H + c0), prev);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) prev[e] = 0.f;
      }
      unpack8(*reinterpret_cast<const u32x4_t*>(base + (size_t)2 * H + c0), b0);
      unpack8(*reinterpret_cast<const u32x4_t*>(base + (size_t)3 * H + c0), b1);
      unpack8(*reinterpret_cast<const u32x4_t*>(residual + (size_t)t * H + c0), r);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = r[e] + ((b0[e] + d0) * cur[e] + (b1[e] + d1) * prev[e]);
      const u32x4_t packed = pack8(o);
      *reinterpret_cast<u32x4_t*>(x_out + (size_t)t * H + c0) = packed;
      unpack8(packed, xv[i]);  // the norm reads the rounded residual, as a separate norm would
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xv[i][e] * xv[i][e];
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = rsqrtf(tot / static_cast<float>(H) + eps);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = tid + i * 256;
    if (ch < chunks) {
      float gm[8], o[8];
      unpack8(*reinterpret_cast<const u32x4_t*>(gamma + ch * 8), gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = xv[i][e] * inv * gm[e];
      *reinterpret_cast<u32x4_t*>(n_out + (size_t)t * H + ch * 8) = pack8(o);
    }
  }
}

}  // namespace

hipError_t launch_conv_residual_norm(const uint16_t* y, const float* coef, int ldc,
                                     const uint16_t* base, int T, int H, int G, int grp,
                                     const uint16_t* residual, uint16_t* x_out,
                                     const uint16_t* gamma, float eps, uint16_t* n_out,
                                     hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  conv_residual_norm_kernel<4><<<T, 256, 0, stream>>>(y, coef, ldc, base, H, G, grp, residual, x_out,
                                                      gamma, eps, n_out);
  return hipGetLastError();
}

hipError_t launch_conv(const uint16_t* y, const float* coef, int ldc, const uint16_t* base,
                       int side, int T, int H, int G, int grp, const uint16_t* residual,
                       uint16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  dim3 grid((H / 8 + 255) / 256, T);
  conv_kernel<<<grid, 256, 0, stream>>>(y, coef, ldc, base, side, H, G, grp, residual, out);
  return hipGetLastError();
}

}  // namespace dfl
