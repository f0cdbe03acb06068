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

}  // namespace

hipError_t launch_conv(const uint16_t* y, const float* coef, int ldc, const uint16_t* base,
                       int side, int T, int H, int G, int grp, const uint16_t* residual,
                       uint16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  dim3 grid((H / 8 + 255) / 256, T);
  conv_kernel<<<grid, 256, 0, stream>>>(y, coef, ldc, base, side, H, G, grp, residual, out);
  return hipGetLastError();
}

}  // namespace dfl
