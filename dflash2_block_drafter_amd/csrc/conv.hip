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
// Inside the drafter the coefficients (the kernel projection's output) arrive as that
// projection's fp32 split-K planes; each workgroup sums its row's slice once, in plane
// order, into LDS instead of a separate reduce launch writing them out.
#include "common.hpp"
#include "kernels.hpp"

namespace dfl {

namespace {

// Coefficients of row t for groups [g0, g0 + n) into cs: cs[i] = tap 0 of group g0 + i,
// cs[n + i] = tap 1, each summed over the planes; cooperative and coalesced, then a barrier.
__device__ __forceinline__ void stage_coef(const Planes& coef, int t, int ng, int g0, int n, float* cs) {
  const size_t crow = (size_t)t * coef.ld;
  for (int i = threadIdx.x; i < 2 * n; i += blockDim.x) {
    const int col = i < n ? g0 + i : ng + g0 + (i - n);
    cs[i] = planes_sum1(coef, crow + col);
  }
  __syncthreads();
}

// The raw inputs of 8 channels c0.. of row t, loaded before the coefficients are staged so
// both sets of loads are in flight together.
struct ConvIn {
  u32x4_t cur, prev, b0, b1;
};

__device__ __forceinline__ ConvIn load_conv_in(const uint16_t* y, const uint16_t* b0p, const uint16_t* b1p,
                                               int t, int H, bool has_prev, int c0) {
  ConvIn in;
  in.cur = *reinterpret_cast<const u32x4_t*>(y + (size_t)t * H + c0);
  in.prev = has_prev ? *reinterpret_cast<const u32x4_t*>(y + (size_t)(t - 1) * H + c0) : u32x4_t{0u, 0u, 0u, 0u};
  in.b0 = *reinterpret_cast<const u32x4_t*>(b0p + c0);
  in.b1 = *reinterpret_cast<const u32x4_t*>(b1p + c0);
  return in;
}

// (b0 + d0) * y[t] + (b1 + d1) * y[t-1]; y[t-1] is zero at a block start (prev = 0).
__device__ __forceinline__ void conv8(const ConvIn& in, float d0, float d1, float* o) {
  float cur[8], prev[8], b0[8], b1[8];
  unpack8(in.cur, cur);
  unpack8(in.prev, prev);
  unpack8(in.b0, b0);
  unpack8(in.b1, b1);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (b0[e] + d0) * cur[e] + (b1[e] + d1) * prev[e];
}

// Sums of two entries of the planes, in plane order, with the loads of both issued together
// (one round trip per batch of eight planes).
__device__ __forceinline__ void planes_sum_pair(const Planes& pl, size_t off0, size_t off1, float& s0, float& s1) {
  const float* q = pl.p;
  for (int b = 0; b < pl.S; b += 8) {
    float v0[8], v1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const size_t po = (size_t)min(b + i, pl.S - 1) * pl.plane;
      v0[i] = q[po + off0];
      v1[i] = q[po + off1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (b + i >= pl.S) break;
      s0 = b + i == 0 ? v0[i] : s0 + v0[i];
      s1 = b + i == 0 ? v1[i] : s1 + v1[i];
    }
  }
}

// The same with the plane count S a compile-time constant: all 2 S loads are issued before
// the first add (one round trip), the adds in the same plane order; S = 0 takes pl.S.
template <int S>
__device__ __forceinline__ void planes_sum_pair_n(const Planes& pl, size_t off0, size_t off1, float& s0, float& s1) {
  if constexpr (S == 0) {
    planes_sum_pair(pl, off0, off1, s0, s1);
  } else {
    const float* q = pl.p;
    float v0[S], v1[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      v0[i] = q[(size_t)i * pl.plane + off0];
      v1[i] = q[(size_t)i * pl.plane + off1];
    }
    s0 = v0[0];
    s1 = v1[0];
#pragma unroll
    for (int i = 1; i < S; ++i) {
      s0 += v0[i];
      s1 += v1[i];
    }
  }
}

// R consecutive rows of one block (R divides G) for kConvCh channels per workgroup of
// kConvCh/8 threads: the R + 1 input rows are loaded once (row t-1 of the first row only
// when it is in the block) and each later row reuses its predecessor from registers.
// With coef_next set (side 0 only), the workgroup also sums the other side's coefficients
// of its rows and groups, which lie 2 * ng columns further in the same planes, and writes
// them as one fp32 plane [T, 2 * ng] (tap 0 groups, then tap 1): the finish then reads one
// plane instead of every split of the kernel projection.
constexpr int kConvCh = 1024;

template <int R, int S>
__global__ __launch_bounds__(kConvCh / 8) void conv_kernel(const uint16_t* y, Planes coef,
                                                           const uint16_t* __restrict__ base, int side,
                                                           int H, int G, int grp,
                                                           const uint16_t* residual, uint16_t* out,
                                                           float* __restrict__ coef_next) {
  __shared__ float cs[R][2 * (kConvCh / 8)];  // kConvCh channels touch at most kConvCh/8 groups
  const int t0 = blockIdx.y * R;
  const int cb = blockIdx.x * kConvCh;
  const int g0 = cb / grp;
  const int ngw = (min(H, cb + kConvCh) - 1) / grp - g0 + 1;  // groups touching [cb, cb + kConvCh)
  const int c0 = cb + threadIdx.x * 8;
  const int cc = min(c0, H - 8);  // threads past H load the last chunk and store nothing
  const uint16_t* b0p = base + (size_t)(side * 2 + 0) * H;
  const uint16_t* b1p = base + (size_t)(side * 2 + 1) * H;
  u32x4_t cur[R + 1], rv[R];
  cur[0] = t0 % G != 0 ? *reinterpret_cast<const u32x4_t*>(y + (size_t)(t0 - 1) * H + cc) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < R; ++r) {
    cur[r + 1] = *reinterpret_cast<const u32x4_t*>(y + (size_t)(t0 + r) * H + cc);
    rv[r] = residual ? *reinterpret_cast<const u32x4_t*>(residual + (size_t)(t0 + r) * H + cc) : u32x4_t{0u, 0u, 0u, 0u};
  }
  const u32x4_t b0v = *reinterpret_cast<const u32x4_t*>(b0p + cc);
  const u32x4_t b1v = *reinterpret_cast<const u32x4_t*>(b1p + cc);
  const int ng = H / grp;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t crow = (size_t)(t0 + r) * coef.ld;
    for (int i = threadIdx.x; i < 2 * ngw; i += blockDim.x) {
      const int col = i < ngw ? g0 + i : ng + g0 + (i - ngw);
      if (coef_next) {
        float here, next;
        planes_sum_pair_n<S>(coef, crow + col, crow + 2 * ng + col, here, next);
        cs[r][i] = here;
        coef_next[(size_t)(t0 + r) * 2 * ng + col] = next;
      } else {
        cs[r][i] = planes_sum1(coef, crow + col);
      }
    }
  }
  __syncthreads();
  if (c0 >= H) return;
  const int gl = c0 / grp - g0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ConvIn in;
    in.cur = cur[r + 1];
    in.prev = cur[r];  // row t0 + r - 1: zero at a block start (R divides G, so only r = 0 can be one)
    in.b0 = b0v;
    in.b1 = b1v;
    float o[8];
    conv8(in, cs[r][gl], cs[r][ngw + gl], o);
    if (residual) {
      float rr[8];
      unpack8(rv[r], rr);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rr[e] + o[e];
    }
    *reinterpret_cast<u32x4_t*>(out + (size_t)(t0 + r) * H + c0) = pack8(o);
  }
}

// The same conv when the coefficients are one fp32 plane [T, 2 * ng] (the finish's side-1
// deltas, or a standalone prepare's): each thread loads its own group's two coefficients
// per row next to its inputs, so there is no LDS staging and no barrier, and the only wait
// is the one round trip for all of a thread's loads.  R rows of a block per thread, as in
// conv_kernel; kConvPlaneCh / 8 threads (one wavefront) cover kConvPlaneCh channels.  At
// T = 1024, H = 5120 that is 1280 workgroups of 8 rows, five per CU: 5.8 us a conv against
// 6.4 us for 1024 channels (2.5 workgroups per CU), 6.7 us for 256 and 6.6 us for 512 with
// 4 rows.
constexpr int kConvPlaneCh = 512;

template <int R, bool NTS>
__global__ __launch_bounds__(kConvPlaneCh / 8) void conv_plane_kernel(const uint16_t* __restrict__ y,
                                                                 const float* __restrict__ coef, int ld,
                                                                 const uint16_t* __restrict__ base, int side,
                                                                 int H, int G, int grp,
                                                                 const uint16_t* residual,
                                                                 uint16_t* out) {  // may be residual
  const int t0 = blockIdx.y * R;
  const int c0 = blockIdx.x * kConvPlaneCh + threadIdx.x * 8;
  if (c0 >= H) return;
  const int g = c0 / grp;
  const int ng = H / grp;
  u32x4_t cur[R + 1], rv[R];
  float d0[R], d1[R];
  cur[0] = t0 % G != 0 ? *reinterpret_cast<const u32x4_t*>(y + (size_t)(t0 - 1) * H + c0) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < R; ++r) {
    cur[r + 1] = *reinterpret_cast<const u32x4_t*>(y + (size_t)(t0 + r) * H + c0);
    rv[r] = residual ? *reinterpret_cast<const u32x4_t*>(residual + (size_t)(t0 + r) * H + c0) : u32x4_t{0u, 0u, 0u, 0u};
    d0[r] = coef[(size_t)(t0 + r) * ld + g];
    d1[r] = coef[(size_t)(t0 + r) * ld + ng + g];
  }
  ConvIn in;
  in.b0 = *reinterpret_cast<const u32x4_t*>(base + (size_t)(side * 2) * H + c0);
  in.b1 = *reinterpret_cast<const u32x4_t*>(base + (size_t)(side * 2 + 1) * H + c0);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    in.cur = cur[r + 1];
    in.prev = cur[r];  // zero at a block start (R divides G, so only r = 0 can be one)
    float o[8];
    conv8(in, d0[r], d1[r], o);
    if (residual) {
      float rr[8];
      unpack8(rv[r], rr);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rr[e] + o[e];
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (size_t)(t0 + r) * H + c0);
    if (NTS)
      __builtin_nontemporal_store(pack8(o), dst);
    else
      *dst = pack8(o);
  }
}

// conv finish + residual + the next sublayer's RMSNorm, one workgroup per row: the row's
// new residual stays in registers between the conv and the norm, so x is written once and
// the norm costs no extra read (dflash2.ts diff, `#block`: x = bf16(x + Conv1(..)), then
// m = rms(x) opens the next sublayer).  MAXC chunks of 8 channels per thread.
template <int MAXC>
__global__ __launch_bounds__(256) void conv_residual_norm_kernel(
    const uint16_t* y, Planes coef, const uint16_t* __restrict__ base, int H, int G, int grp,
    const uint16_t* residual, uint16_t* x_out, const uint16_t* __restrict__ gamma, float eps,
    uint16_t* __restrict__ n_out, int skip_anchor, uint32_t* __restrict__ clear_bound) {
  __shared__ float red[4];
  __shared__ float cs[2 * MAXC * 256];  // the row's groups: H / grp <= H / 8 <= MAXC * 256
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int chunks = H >> 3;
  const int ng = H / grp;
  ConvIn in[MAXC];
  u32x4_t rv[MAXC], gv[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int cc = min(tid + i * 256, chunks - 1) * 8;  // clamped: every load unconditional
    in[i] = load_conv_in(y, base + (size_t)2 * H, base + (size_t)3 * H, t, H, t % G != 0, cc);
    rv[i] = *reinterpret_cast<const u32x4_t*>(residual + (size_t)t * H + cc);
    gv[i] = *reinterpret_cast<const u32x4_t*>(gamma + cc);
  }
  stage_coef(coef, t, ng, 0, ng, cs);
  float xv[MAXC][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = tid + i * 256;
    if (ch < chunks) {
      const int c0 = ch * 8;
      const int g = c0 / grp;
      float o[8], r[8];
      conv8(in[i], cs[g], cs[ng + g], o);
      unpack8(rv[i], r);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = r[e] + o[e];
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
  // with skip_anchor the normed rows are packed without each block's row 0
  if (skip_anchor && t % G == 0) return;
  const size_t nrow = skip_anchor ? (size_t)(t / G) * (G - 1) + t % G - 1 : (size_t)t;
  if (skip_anchor && clear_bound && tid < kTileBoundSlots) clear_bound[nrow * kTileBoundSlots + tid] = 0u;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = tid + i * 256;
    if (ch < chunks) {
      float gm[8], o[8];
      unpack8(gv[i], gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = xv[i][e] * inv * gm[e];
      *reinterpret_cast<u32x4_t*>(n_out + nrow * H + ch * 8) = pack8(o);
    }
  }
}

// Sums of 8 channels at two element offsets over the planes, in plane order (the order the
// split-K reduce adds them).  With the plane count S a compile-time constant every load is
// issued before the first add (one round trip); S = 0 takes the count from pl.S, a batch of
// eight planes at a time.
template <int S>
__device__ __forceinline__ void planes_sum8_pair(const Planes& pl, size_t off0, size_t off1, float* s0, float* s1) {
  const float* q = pl.p;
  if constexpr (S > 0) {
    f32x4_t v[S][4];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const size_t po = (size_t)i * pl.plane;
      v[i][0] = *reinterpret_cast<const f32x4_t*>(q + po + off0);
      v[i][1] = *reinterpret_cast<const f32x4_t*>(q + po + off0 + 4);
      v[i][2] = *reinterpret_cast<const f32x4_t*>(q + po + off1);
      v[i][3] = *reinterpret_cast<const f32x4_t*>(q + po + off1 + 4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s0[e] = v[0][0][e];
      s0[4 + e] = v[0][1][e];
      s1[e] = v[0][2][e];
      s1[4 + e] = v[0][3][e];
    }
#pragma unroll
    for (int i = 1; i < S; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s0[e] += v[i][0][e];
        s0[4 + e] += v[i][1][e];
        s1[e] += v[i][2][e];
        s1[4 + e] += v[i][3][e];
      }
  } else {
    for (int b = 0; b < pl.S; b += 8) {
      f32x4_t v[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const size_t po = (size_t)min(b + i, pl.S - 1) * pl.plane;
        v[i][0] = *reinterpret_cast<const f32x4_t*>(q + po + off0);
        v[i][1] = *reinterpret_cast<const f32x4_t*>(q + po + off0 + 4);
        v[i][2] = *reinterpret_cast<const f32x4_t*>(q + po + off1);
        v[i][3] = *reinterpret_cast<const f32x4_t*>(q + po + off1 + 4);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (b + i >= pl.S) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s0[e] = b + i == 0 ? v[i][0][e] : s0[e] + v[i][0][e];
          s0[4 + e] = b + i == 0 ? v[i][1][e] : s0[4 + e] + v[i][1][e];
          s1[e] = b + i == 0 ? v[i][2][e] : s1[e] + v[i][2][e];
          s1[4 + e] = b + i == 0 ? v[i][3][e] : s1[4 + e] + v[i][3][e];
        }
      }
    }
  }
}

// At most 640 threads (H <= 5120): three wavefronts per SIMD leave a thread the registers
// for eight planes' loads of both rows in flight at once.
constexpr int kCrnPlanesMaxThreads = kCrnPlanesMaxH / 8;

// conv_residual_norm_kernel with the sublayer output y given as its projection's split-K
// planes (o or down) instead of the reduced bf16 rows: each thread sums its 8 channels of
// rows t and t - 1 over the planes and rounds them to bf16, which is exactly what the
// split-K reduce would have stored, so no separate reduce launch is needed.  One thread per
// 8 channels (H / 8 threads, rounded up to whole wavefronts), so a thread's plane loads for
// both rows go out as one round per batch of eight planes.
template <int S>
__global__ __launch_bounds__(kCrnPlanesMaxThreads) void conv_residual_norm_planes_kernel(
    Planes y, Planes coef, const uint16_t* __restrict__ base, int H, int G, int grp,
    const uint16_t* residual, uint16_t* x_out, const uint16_t* __restrict__ gamma, float eps,
    uint16_t* __restrict__ n_out, int skip_anchor, uint32_t* __restrict__ clear_bound) {
  __shared__ float red[kCrnPlanesMaxThreads / 64];
  __shared__ float cs[2 * kCrnPlanesMaxThreads];  // the row's groups: H / grp <= H / 8
  // Workgroups are dealt to the 8 XCDs in turn; rows are mapped so that each XCD gets a
  // contiguous run of them, and row t's read of row t - 1's planes finds them in that XCD's
  // L2 behind row t - 1's own reader.
  const int T = gridDim.x;
  const int t = T % 8 == 0 ? (blockIdx.x % 8) * (T / 8) + blockIdx.x / 8 : blockIdx.x;
  const int tid = threadIdx.x;
  const int chunks = H >> 3;
  const int ng = H / grp;
  const bool live = tid < chunks;
  const int c0 = min(tid, chunks - 1) * 8;  // clamped: every load unconditional
  const bool has_prev = t % G != 0;
  const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(residual + (size_t)t * H + c0);
  const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(gamma + c0);
  ConvIn in;
  in.b0 = *reinterpret_cast<const u32x4_t*>(base + (size_t)2 * H + c0);
  in.b1 = *reinterpret_cast<const u32x4_t*>(base + (size_t)3 * H + c0);
  // With one coefficient plane (the side-1 deltas the prepare summed) this thread's share of
  // the row's 2 * ng coefficients (at most two: grp >= 8) is loaded here too, so one round
  // trip covers every input of the row; more planes are staged after the sums.
  const bool one_plane = coef.S == 1;
  const int nthr = static_cast<int>(blockDim.x);
  float cv0 = 0.f, cv1 = 0.f;
  if (one_plane) {
    const float* crow = coef.p + (size_t)t * coef.ld;
    if (tid < 2 * ng) cv0 = crow[tid];
    if (tid + nthr < 2 * ng) cv1 = crow[tid + nthr];
  }
  {
    float cur[8], prev[8];
    planes_sum8_pair<S>(y, (size_t)t * y.ld + c0, (size_t)(has_prev ? t - 1 : t) * y.ld + c0, cur, prev);
    in.cur = pack8(cur);
    in.prev = has_prev ? pack8(prev) : u32x4_t{0u, 0u, 0u, 0u};
  }
  if (one_plane) {
    if (tid < 2 * ng) cs[tid] = cv0;
    if (tid + nthr < 2 * ng) cs[tid + nthr] = cv1;
    __syncthreads();
  } else {
    stage_coef(coef, t, ng, 0, ng, cs);
  }
  float xv[8];
  float ss = 0.f;
  if (live) {
    const int g = c0 / grp;
    float o[8], r[8];
    conv8(in, cs[g], cs[ng + g], o);
    unpack8(rv, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = r[e] + o[e];
    const u32x4_t packed = pack8(o);
    *reinterpret_cast<u32x4_t*>(x_out + (size_t)t * H + c0) = packed;
    unpack8(packed, xv);  // the norm reads the rounded residual, as a separate norm would
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += xv[e] * xv[e];
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  const int waves = (int)(blockDim.x >> 6);
  for (int w = 0; w < waves; ++w) tot += red[w];
  const float inv = rsqrtf(tot / static_cast<float>(H) + eps);
  // (the workgroup has at least 64 threads, live or not)
  if (skip_anchor && clear_bound && t % G != 0 && tid < kTileBoundSlots)
    clear_bound[((size_t)(t / G) * (G - 1) + t % G - 1) * kTileBoundSlots + tid] = 0u;
  if (!live || (skip_anchor && t % G == 0)) return;
  const size_t nrow = skip_anchor ? (size_t)(t / G) * (G - 1) + t % G - 1 : (size_t)t;
  float gm[8], o[8];
  unpack8(gv, gm);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = xv[e] * inv * gm[e];
  *reinterpret_cast<u32x4_t*>(n_out + nrow * H + c0) = pack8(o);
}

}  // namespace

hipError_t launch_conv_residual_norm(const uint16_t* y, const Planes& coef, const uint16_t* base, int T, int H,
                                     int G, int grp, const uint16_t* residual, uint16_t* x_out,
                                     const uint16_t* gamma, float eps, uint16_t* n_out, hipStream_t stream,
                                     bool skip_anchor, uint32_t* clear_bound) {
  if (T <= 0) return hipSuccess;
  const int per = (H / 8 + 255) / 256;  // chunks of 8 channels per thread
  const int sk = skip_anchor ? 1 : 0;
  switch (per) {
    case 1:
      conv_residual_norm_kernel<1><<<T, 256, 0, stream>>>(y, coef, base, H, G, grp, residual, x_out, gamma, eps, n_out, sk,
                                                          clear_bound);
      break;
    case 2:
      conv_residual_norm_kernel<2><<<T, 256, 0, stream>>>(y, coef, base, H, G, grp, residual, x_out, gamma, eps, n_out, sk,
                                                          clear_bound);
      break;
    case 3:
      conv_residual_norm_kernel<3><<<T, 256, 0, stream>>>(y, coef, base, H, G, grp, residual, x_out, gamma, eps, n_out, sk,
                                                          clear_bound);
      break;
    case 4:
      conv_residual_norm_kernel<4><<<T, 256, 0, stream>>>(y, coef, base, H, G, grp, residual, x_out, gamma, eps, n_out, sk,
                                                          clear_bound);
      break;
    default:
      return hipErrorInvalidValue;  // H > 8192
  }
  return hipGetLastError();
}

hipError_t launch_conv_residual_norm_planes(const Planes& y, const Planes& coef, const uint16_t* base, int T, int H,
                                            int G, int grp, const uint16_t* residual, uint16_t* x_out,
                                            const uint16_t* gamma, float eps, uint16_t* n_out, hipStream_t stream,
                                            bool skip_anchor, uint32_t* clear_bound) {
  if (T <= 0) return hipSuccess;
  if (H % 8 != 0 || H > 8 * kCrnPlanesMaxThreads || y.S < 1 || y.ld != H || y.plane < (size_t)T * H)
    return hipErrorInvalidValue;
  const int threads = (H / 8 + 63) / 64 * 64;
  const int sk = skip_anchor ? 1 : 0;
#define DFL_CRN_PLANES(S_)                                                                              \
  conv_residual_norm_planes_kernel<S_><<<T, threads, 0, stream>>>(y, coef, base, H, G, grp, residual, x_out, \
                                                                  gamma, eps, n_out, sk, clear_bound)
  switch (y.S) {
    case 2: DFL_CRN_PLANES(2); break;
    case 3: DFL_CRN_PLANES(3); break;
    case 4: DFL_CRN_PLANES(4); break;
    case 5: DFL_CRN_PLANES(5); break;
    case 6: DFL_CRN_PLANES(6); break;
    case 7: DFL_CRN_PLANES(7); break;
    case 8: DFL_CRN_PLANES(8); break;
    default: DFL_CRN_PLANES(0);
  }
#undef DFL_CRN_PLANES
  return hipGetLastError();
}

hipError_t launch_conv(const uint16_t* y, const Planes& coef, const uint16_t* base, int side, int T, int H, int G,
                       int grp, const uint16_t* residual, uint16_t* out, hipStream_t stream, float* coef_next) {
  if (T <= 0) return hipSuccess;
  if (coef_next && side != 0) return hipErrorInvalidValue;
  // rows per workgroup: the largest of 8 (one coefficient plane only), 4, 2, 1 dividing G that
  // still leaves >= 512 workgroups (with 1024 channels a workgroup at T = 1024, H = 5120: 8
  // rows, 640 workgroups, 6.75 -> 6.43 us a conv against 4 rows; 16 rows: 7.9 us)
  const bool plane = coef.S == 1 && !coef_next;
  const int chunks = (H + (plane ? kConvPlaneCh : kConvCh) - 1) / (plane ? kConvPlaneCh : kConvCh);
  int R = 1;
  for (int r : {8, 4, 2}) {
    if (r == 8 && !plane) continue;
    if (G % r == 0 && T % r == 0 && (long)chunks * (T / r) >= 512) {
      R = r;
      break;
    }
  }
  const dim3 grid(chunks, T / R);
  if (plane) {
    // an output larger than an XCD's 4 MB L2 would not stay there for its reader anyway:
    // stream it out with non-temporal stores
    const bool nts = (size_t)T * H * sizeof(uint16_t) > (size_t(8) << 20);
    switch (R * 2 + (nts ? 1 : 0)) {
      case 17:
        conv_plane_kernel<8, true><<<grid, kConvPlaneCh / 8, 0, stream>>>(y, coef.p, coef.ld, base, side, H, G, grp, residual, out);
        break;
      case 16:
        conv_plane_kernel<8, false><<<grid, kConvPlaneCh / 8, 0, stream>>>(y, coef.p, coef.ld, base, side, H, G, grp, residual, out);
        break;
      case 9:
        conv_plane_kernel<4, true><<<grid, kConvPlaneCh / 8, 0, stream>>>(y, coef.p, coef.ld, base, side, H, G, grp, residual, out);
        break;
      case 8:
        conv_plane_kernel<4, false><<<grid, kConvPlaneCh / 8, 0, stream>>>(y, coef.p, coef.ld, base, side, H, G, grp, residual, out);
        break;
      case 5:
        conv_plane_kernel<2, true><<<grid, kConvPlaneCh / 8, 0, stream>>>(y, coef.p, coef.ld, base, side, H, G, grp, residual, out);
        break;
      case 4:
        conv_plane_kernel<2, false><<<grid, kConvPlaneCh / 8, 0, stream>>>(y, coef.p, coef.ld, base, side, H, G, grp, residual, out);
        break;
      case 3:
        conv_plane_kernel<1, true><<<grid, kConvPlaneCh / 8, 0, stream>>>(y, coef.p, coef.ld, base, side, H, G, grp, residual, out);
        break;
      default:
        conv_plane_kernel<1, false><<<grid, kConvPlaneCh / 8, 0, stream>>>(y, coef.p, coef.ld, base, side, H, G, grp, residual, out);
    }
    return hipGetLastError();
  }
  // the kernel projection's plane count as a compile-time constant where the plans put it
  // (one round trip for all of a thread's plane loads), else read from coef
#define DFL_CONV_S(R_)                                                                                        \
  switch (coef.S) {                                                                                          \
    case 8: conv_kernel<R_, 8><<<grid, kConvCh / 8, 0, stream>>>(y, coef, base, side, H, G, grp, residual,   \
                                                                 out, coef_next); break;                     \
    case 10: conv_kernel<R_, 10><<<grid, kConvCh / 8, 0, stream>>>(y, coef, base, side, H, G, grp, residual, \
                                                                   out, coef_next); break;                   \
    case 12: conv_kernel<R_, 12><<<grid, kConvCh / 8, 0, stream>>>(y, coef, base, side, H, G, grp, residual, \
                                                                   out, coef_next); break;                   \
    default: conv_kernel<R_, 0><<<grid, kConvCh / 8, 0, stream>>>(y, coef, base, side, H, G, grp, residual,  \
                                                                  out, coef_next);                           \
  }
  switch (R) {
    case 4: DFL_CONV_S(4); break;
    case 2: DFL_CONV_S(2); break;
    default: DFL_CONV_S(1);
  }
#undef DFL_CONV_S
  return hipGetLastError();
}

}  // namespace dfl
