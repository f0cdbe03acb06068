// RMSNorm (one wavefront per row), per-head RMSNorm + neox RoPE, and the context K/V
// store.  All are HBM/latency-bound; loads are 16-byte vectors where rows allow.
#include "common.hpp"
#include "kernels.hpp"

namespace dfl {

namespace {

constexpr int kMaxChunks = 16;  // 16-byte chunks per lane: H <= 64 * 16 * 8 = 8192

// RMSNorm with a direct gain (dflash2.ts diff, `#rms`): y = x * rsqrt(mean(x^2) + eps) * g,
// reduced in fp32, rounded once to bf16.
__global__ __launch_bounds__(256) void rms_norm_kernel(const uint16_t* __restrict__ x, int ldx,
                                                       int rows, int H,
                                                       const uint16_t* __restrict__ gamma,
                                                       float eps, uint16_t* __restrict__ y,
                                                       int ldy, int out_per_grp, int in_per_grp,
                                                       int skip) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int rin = (r / out_per_grp) * in_per_grp + skip + r % out_per_grp;
  const uint16_t* xr = x + (size_t)rin * ldx;
  const int chunks = H >> 3;
  u32x4_t v[kMaxChunks], gv[kMaxChunks];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + i * 64;
    if (c < chunks) {  // the gains load with the row: one round trip for both
      v[i] = *reinterpret_cast<const u32x4_t*>(xr + c * 8);
      gv[i] = *reinterpret_cast<const u32x4_t*>(gamma + c * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + i * 64;
    if (c < chunks) {
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / static_cast<float>(H) + eps);
  uint16_t* yr = y + (size_t)r * ldy;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + i * 64;
    if (c < chunks) {
      float f[8], g[8];
      unpack8(v[i], f);
      unpack8(gv[i], g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] * inv * g[e];
      *reinterpret_cast<u32x4_t*>(yr + c * 8) = pack8(f);
    }
  }
}

// cos/sin of position `pos` for rotary pair i of a D-wide head, angle in fp64:
// inv_freq_i = theta^(-2i/D) (neox RoPE, mirror-sd listing's RoPE docstring).
__device__ __forceinline__ void rope_cs(int pos, int i, int D, double log_theta, float* c,
                                        float* s) {
  const double inv_freq = exp(-(2.0 * i / D) * log_theta);
  const double ang = static_cast<double>(pos) * inv_freq;
  double sd, cd;
  sincos(ang, &sd, &cd);
  *c = static_cast<float>(cd);
  *s = static_cast<float>(sd);
}

// In-place per-head RMSNorm then RoPE of one D-wide head held by one wavefront:
// lane i < D/2 holds the neox pair (x[i], x[i + D/2]).
__device__ __forceinline__ void norm_rope_head(const uint16_t* src, uint16_t* dst, int D,
                                               const uint16_t* gamma, float eps, float c,
                                               float s, int lane) {
  const int half = D >> 1;
  float a = 0.f, b = 0.f;
  if (lane < half) {
    a = bf16_to_f32(src[lane]);
    b = bf16_to_f32(src[lane + half]);
  }
  const float ss = wave_sum(a * a + b * b);
  const float inv = rsqrtf(ss / static_cast<float>(D) + eps);
  if (lane < half) {
    a = a * inv * bf16_to_f32(gamma[lane]);
    b = b * inv * bf16_to_f32(gamma[lane + half]);
    // rotate_half(x) = cat(-x2, x1): out1 = x1 c - x2 s, out2 = x2 c + x1 s
    dst[lane] = f32_to_bf16(a * c - b * s);
    dst[lane + half] = f32_to_bf16(b * c + a * s);
  }
}

// Heads [0, split) use gamma, heads [split, heads) use gamma2 (q and k of one row in one
// launch: q heads take q_norm, k heads k_norm).
__global__ __launch_bounds__(256) void head_norm_rope_kernel(uint16_t* x, int ldx, int rows,
                                                             int heads, int split, int D,
                                                             const uint16_t* __restrict__ gamma,
                                                             const uint16_t* __restrict__ gamma2,
                                                             float eps, double log_theta,
                                                             const int32_t* __restrict__ pos0,
                                                             int rows_per_req, int pos_offset) {
  const int r = blockIdx.x;
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int pos = pos0[r / rows_per_req] + r % rows_per_req + pos_offset;
  float c = 1.f, s = 0.f;
  if (lane < (D >> 1)) rope_cs(pos, lane, D, log_theta, &c, &s);
  uint16_t* row = x + (size_t)r * ldx;
  for (int h = wave; h < heads; h += 4)
    norm_rope_head(row + h * D, row + h * D, D, h < split ? gamma : gamma2, eps, c, s, lane);
}

// q|k|v projection finish from its fp32 split-K planes, one wavefront per (row, head):
// heads [0, rope_heads) get RMSNorm + RoPE of the fp32 sum over planes (q_norm below
// `split`, k_norm above), rounded once to bf16; later heads (v) are the sum, rounded.
// Lane l holds EPL = D/64 adjacent values; for l < 32 they are first-half elements, their
// rotary partners sit in lane l ^ 32.
template <int D>
__global__ __launch_bounds__(256) void head_norm_rope_planes_kernel(
    Planes src, uint16_t* __restrict__ dst, int ldd, int rows, int heads, int rope_heads, int split,
    const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ gamma2, float eps, double log_theta,
    const int32_t* __restrict__ pos0, int rows_per_req, int pos_offset) {
  constexpr int EPL = D / 64;
  typedef float ev_t __attribute__((ext_vector_type(EPL)));
  const int r = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half_lane = lane & 31;
  const int e0 = (lane >> 5) * (D / 2) + half_lane * EPL;  // this lane's first element
  // Up to eight planes: their loads go out first (row and head clamped in range), so they are
  // in flight while the rotary pairs are computed.
  const bool live = r < rows && h < heads;
  const size_t off = (size_t)min(r, rows - 1) * src.ld + min(h, heads - 1) * D + e0;
  ev_t raw[8];
  if (src.S <= 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      raw[i] = *reinterpret_cast<const ev_t*>(src.p + (size_t)min(i, src.S - 1) * src.plane + off);
  }
  // the row's D/2 rotary (cos, sin) pairs, computed once for the workgroup's four heads
  __shared__ float rc[D / 2], rs[D / 2];
  if (r < rows && threadIdx.x < D / 2) {
    const int pos = pos0[r / rows_per_req] + r % rows_per_req + pos_offset;
    rope_cs(pos, threadIdx.x, D, log_theta, &rc[threadIdx.x], &rs[threadIdx.x]);
  }
  __syncthreads();
  if (!live) return;
  float v[EPL];
  if (src.S <= 8) {
    // the planes in order 0, 1, 2, ..., as planes_sum adds them
    ev_t acc = raw[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
      if (i < src.S) acc += raw[i];
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = acc[e];
  } else {
    planes_sum<EPL>(src, off, v);
  }
  uint16_t* out = dst + (size_t)r * ldd + h * D + e0;
  if (h >= rope_heads) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = f32_to_bf16(v[e]);
    return;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) ss += v[e] * v[e];
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / static_cast<float>(D) + eps);
  const uint16_t* g = h < split ? gamma : gamma2;
  const bool first = lane < 32;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float x = v[e] * inv * bf16_to_f32(g[e0 + e]);
    // lane ^ 32's value: the row-swap permute leaves it in the second result in the lower
    // half of the wave and in the first in the upper half
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float partner = __uint_as_float(first ? sw[1] : sw[0]);
    const float c = rc[half_lane * EPL + e], s = rs[half_lane * EPL + e];
    // rotate_half: first half x1 c - x2 s, second half x2 c + x1 s
    out[e] = f32_to_bf16(first ? x * c - partner * s : x * c + partner * s);
  }
}

// Context K/V (dflash2.ts diff, `#contextKV`): kv row (b, j) holds [k | v] for all KV heads;
// K[b, row_offset + j] = RoPE(k_norm(k)) at position row_offset + j, V = v.
__global__ __launch_bounds__(256) void context_kv_store_kernel(
    const uint16_t* __restrict__ kv, int L, int NKV, int D, const uint16_t* __restrict__ k_norm,
    float eps, double log_theta, int row_offset, int Lcap, uint16_t* __restrict__ K,
    uint16_t* __restrict__ V) {
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int pos = row_offset + j;
  const uint16_t* src = kv + ((size_t)b * L + j) * (2 * NKV * D);
  const size_t dst_row = ((size_t)b * Lcap + pos) * NKV * D;
  float c = 1.f, s = 0.f;
  if (lane < (D >> 1)) rope_cs(pos, lane, D, log_theta, &c, &s);
  for (int h = wave; h < NKV; h += 4)
    norm_rope_head(src + h * D, K + dst_row + h * D, D, k_norm, eps, c, s, lane);
  const int vchunks = NKV * D / 8;
  for (int i = threadIdx.x; i < vchunks; i += 256)
    *reinterpret_cast<u32x4_t*>(V + dst_row + i * 8) =
        *reinterpret_cast<const u32x4_t*>(src + NKV * D + i * 8);
}

// Ragged context K/V store ([P3] `materialize` with `input_row_offsets`; [P2] committed rows
// projected at their absolute positions): packed kv row r belongs to request b with
// offsets[b] <= r < offsets[b+1] and goes to K/V row starts[b] + r - offsets[b] of b.
__global__ __launch_bounds__(256) void context_kv_store_ragged_kernel(
    const uint16_t* __restrict__ kv, int NKV, int D, const uint16_t* __restrict__ k_norm, float eps,
    double log_theta, const int32_t* __restrict__ offsets, const int32_t* __restrict__ starts, int B, int Lcap,
    uint16_t* __restrict__ K, uint16_t* __restrict__ V) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int lo = 0, hi = B - 1;  // the last b with offsets[b] <= r (offsets nondecreasing, checked on the host)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int pos = starts[b] + (r - offsets[b]);
  if (pos < 0 || pos >= Lcap) return;  // the host validates; never write past the cache
  const uint16_t* src = kv + (size_t)r * (2 * NKV * D);
  const size_t dst_row = ((size_t)b * Lcap + pos) * NKV * D;
  float c = 1.f, s = 0.f;
  if (lane < (D >> 1)) rope_cs(pos, lane, D, log_theta, &c, &s);
  for (int h = wave; h < NKV; h += 4)
    norm_rope_head(src + h * D, K + dst_row + h * D, D, k_norm, eps, c, s, lane);
  const int vchunks = NKV * D / 8;
  for (int i = threadIdx.x; i < vchunks; i += 256)
    *reinterpret_cast<u32x4_t*>(V + dst_row + i * 8) = *reinterpret_cast<const u32x4_t*>(src + NKV * D + i * 8);
}

}  // namespace

hipError_t launch_context_kv_store_ragged(const uint16_t* kv, int rows, int B, int NKV, int D, const uint16_t* k_norm,
                                          float eps, float theta, const int32_t* offsets, const int32_t* starts,
                                          int Lcap, uint16_t* K, uint16_t* V, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  context_kv_store_ragged_kernel<<<rows, 256, 0, stream>>>(kv, NKV, D, k_norm, eps, log(static_cast<double>(theta)),
                                                           offsets, starts, B, Lcap, K, V);
  return hipGetLastError();
}

hipError_t launch_rms_norm(const uint16_t* x, int ldx, int rows, int H, const uint16_t* gamma,
                           float eps, uint16_t* y, int ldy, int out_per_grp, int in_per_grp,
                           int skip, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  rms_norm_kernel<<<(rows + 3) / 4, 256, 0, stream>>>(x, ldx, rows, H, gamma, eps, y, ldy,
                                                      out_per_grp, in_per_grp, skip);
  return hipGetLastError();
}

hipError_t launch_head_norm_rope(uint16_t* x, int ldx, int rows, int heads, int split, int D,
                                 const uint16_t* gamma, const uint16_t* gamma2, float eps,
                                 float theta, const int32_t* pos0, int rows_per_req,
                                 int pos_offset, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  head_norm_rope_kernel<<<rows, 256, 0, stream>>>(x, ldx, rows, heads, split, D, gamma, gamma2,
                                                  eps, log(static_cast<double>(theta)), pos0,
                                                  rows_per_req, pos_offset);
  return hipGetLastError();
}

hipError_t launch_head_norm_rope_planes(const Planes& src, uint16_t* dst, int ldd, int rows, int rope_heads,
                                        int split, int D, int tail_cols, const uint16_t* gamma,
                                        const uint16_t* gamma2, float eps, float theta, const int32_t* pos0,
                                        int rows_per_req, int pos_offset, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (tail_cols % D != 0 || src.ld % 4 != 0 || (D != 64 && D != 128)) return hipErrorInvalidValue;
  const int heads = rope_heads + tail_cols / D;
  const dim3 grid(rows, (heads + 3) / 4);
  const double lt = log(static_cast<double>(theta));
  if (D == 128)
    head_norm_rope_planes_kernel<128><<<grid, 256, 0, stream>>>(src, dst, ldd, rows, heads, rope_heads, split, gamma,
                                                                gamma2, eps, lt, pos0, rows_per_req, pos_offset);
  else
    head_norm_rope_planes_kernel<64><<<grid, 256, 0, stream>>>(src, dst, ldd, rows, heads, rope_heads, split, gamma,
                                                               gamma2, eps, lt, pos0, rows_per_req, pos_offset);
  return hipGetLastError();
}

hipError_t launch_context_kv_store(const uint16_t* kv, int B, int L, int NKV, int D,
                                   const uint16_t* k_norm, float eps, float theta,
                                   int row_offset, int Lcap, uint16_t* K, uint16_t* V,
                                   hipStream_t stream) {
  if (B <= 0 || L <= 0) return hipSuccess;
  context_kv_store_kernel<<<dim3(L, B), 256, 0, stream>>>(kv, L, NKV, D, k_norm, eps,
                                                          log(static_cast<double>(theta)),
                                                          row_offset, Lcap, K, V);
  return hipGetLastError();
}

}  // namespace dfl
