// Device helpers shared by the gfx950 kernels: bf16 conversion, vector types, wave
// reductions.  gfx950 runs 64-lane wavefronts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace dfl {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even, with gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw_t));
}

// 8 bf16 held as 4 uint32 -> 8 floats.
__device__ __forceinline__ void unpack8(const u32x4_t v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ u32x4_t pack8(const float* f) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

// Butterfly steps of the wave reductions without an LDS round trip: gfx950's row-swap
// permutes for the lane distances 32 and 16 (with v as both operands, the two results hold v
// of the lower and of the upper lane of each pair), DPP moves within a row of 16 lanes.
// op(lo, hi) gives both lanes of a pair the value op(v[lane], v[lane ^ d]) has (op
// commutative), so a sum adds in exactly the order of the xor tree.
struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
template <class Op>
__device__ __forceinline__ float bfly32(float v, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <class Op>
__device__ __forceinline__ float bfly16(float v, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// CTRL: a DPP lane move within each row of 16 (row_ror:8 is xor 8; quad_perm 0x4E and 0xB1
// are xor 2 and xor 1; row_ror:4 matches xor 4 once the values repeat every 8 lanes, i.e.
// after the xor-8 step)
template <int CTRL, class Op>
__device__ __forceinline__ float bfly_dpp(float v, Op op) {
  return op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false)));
}
constexpr int kDppRor8 = 0x128, kDppRor4 = 0x124, kDppXor2 = 0x4E, kDppXor1 = 0xB1;

// Reductions over the 64 lanes in the order of the xor tree 32, 16, 8, 4, 2, 1.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = bfly32(v, op);
  v = bfly16(v, op);
  v = bfly_dpp<kDppRor8>(v, op);
  v = bfly_dpp<kDppRor4>(v, op);
  v = bfly_dpp<kDppXor2>(v, op);
  return bfly_dpp<kDppXor1>(v, op);
}
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, OpAdd{}); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, OpMax{}); }

// Maximum (fmaxf: NaN only if all are) over each row of 16 lanes, in every lane of the row;
// any order gives the same maximum.
__device__ __forceinline__ float row16_max(float v) {
  v = bfly_dpp<kDppXor1>(v, OpMax{});
  v = bfly_dpp<kDppXor2>(v, OpMax{});
  v = bfly_dpp<kDppRor4>(v, OpMax{});
  return bfly_dpp<kDppRor8>(v, OpMax{});
}
// Unsigned minimum over each row of 16 lanes (or, with QUAD, each quad), in every lane of it.
template <bool QUAD = false>
__device__ __forceinline__ uint32_t row16_umin(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xF, 0xF, false));
  if (QUAD) return v;
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRor4, 0xF, 0xF, false));
  return min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRor8, 0xF, 0xF, false));
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// Order-preserving map of a float to an unsigned integer (NaN excluded by the callers), and
// back: a < b as floats implies float_order(a) < float_order(b) (-0 maps just below +0).
__device__ __forceinline__ uint32_t float_order(float x) {
  const uint32_t b = __float_as_uint(x);
  return b & 0x80000000u ? ~b : b | 0x80000000u;
}
__device__ __forceinline__ float order_float(uint32_t u) {
  return __uint_as_float(u & 0x80000000u ? u & 0x7FFFFFFFu : ~u);
}

// Sum over the S planes of pl (fp32 split-K partials) of the VW values at element offset
// `off` (VW = 1, 2, 4 or 8; off a multiple of min(VW, 4)), added in plane order 0, 1, 2, ...
// as the split-K reduce adds them.  Planes are read eight at a time with the plane index
// clamped to S-1, so each batch is one round of independent loads and the wait comes
// once per batch; the clamped repeats are not added.
template <int VW>
__device__ __forceinline__ void planes_sum(const Planes& pl, size_t off, float* out) {
  constexpr int NV = VW > 4 ? 2 : 1;   // loads per plane
  constexpr int LW = VW > 4 ? 4 : VW;  // floats per load
  typedef float lv_t __attribute__((ext_vector_type(LW)));
  const float* q = pl.p + off;
  lv_t acc[NV];
  for (int s0 = 0; s0 < pl.S; s0 += 8) {
    lv_t v[8][NV];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const size_t po = (size_t)min(s0 + i, pl.S - 1) * pl.plane;
#pragma unroll
      for (int j = 0; j < NV; ++j) v[i][j] = *reinterpret_cast<const lv_t*>(q + po + j * LW);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s0 + i >= pl.S) break;
#pragma unroll
      for (int j = 0; j < NV; ++j) acc[j] = (s0 + i == 0) ? v[i][j] : acc[j] + v[i][j];
    }
  }
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int e = 0; e < LW; ++e) out[j * LW + e] = acc[j][e];
}

__device__ __forceinline__ void planes_sum8(const Planes& pl, size_t off, float* out) { planes_sum<8>(pl, off, out); }

__device__ __forceinline__ float planes_sum1(const Planes& pl, size_t off) {
  float v;
  planes_sum<1>(pl, off, &v);
  return v;
}

}  // namespace dfl
