// Exact top-K building blocks shared by the candidate kernels: the candidate order (value
// descending, then id ascending), a 64-lane bitonic sort in that order, and a running
// top-K list kept in lanes 0..K-1 of a wavefront with candidates staged through LDS.
#pragma once
#include "common.hpp"

namespace dfl {

constexpr int kNoId = 0x7FFFFFFF;

// a precedes b in the candidate order
__device__ __forceinline__ bool before(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Sort (v, id) across the 64 lanes into the candidate order (lane 0 first).
__device__ __forceinline__ void wave_bitonic_sort(float& v, int& id, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float ov = __shfl_xor(v, j, 64);
      const int oi = __shfl_xor(id, j, 64);
      const bool lower = (lane & j) == 0;
      const bool desc = (lane & k) == 0;  // this run ends in candidate order
      // pair (lo, hi): in a candidate-order run lo must precede hi, otherwise hi precedes lo
      const float lov = lower ? v : ov, hiv = lower ? ov : v;
      const int loi = lower ? id : oi, hii = lower ? oi : id;
      const bool swap = desc ? before(hiv, hii, lov, loi) : before(lov, loi, hiv, hii);
      if (swap) {
        v = ov;
        id = oi;
      }
    }
  }
}

// Running top-K list in lanes 0..K-1; candidates are staged in `stage` (64 - K slots) and
// merged by one sort when the stage fills.
struct TopkMerger {
  float v;
  int id;
  int pending;
  int K;
  int lane;
  float* sv;
  int* si;

  __device__ __forceinline__ void init(int K_, int lane_, float* sv_, int* si_) {
    K = K_;
    lane = lane_;
    sv = sv_;
    si = si_;
    v = -INFINITY;
    id = kNoId;
    pending = 0;
  }
  __device__ __forceinline__ void flush() {
    if (pending == 0) return;
    __builtin_amdgcn_wave_barrier();
    if (lane >= K) {
      const int s = lane - K;
      if (s < pending) {
        v = sv[s];
        id = si[s];
      } else {
        v = -INFINITY;
        id = kNoId;
      }
    }
    wave_bitonic_sort(v, id, lane);
    pending = 0;
    __builtin_amdgcn_wave_barrier();
  }
  // every lane offers (cv, cid) when take is true
  __device__ __forceinline__ void offer(bool take, float cv, int cid) {
    uint64_t mask = __ballot(take);
    const int cap = 64 - K;
    while (mask) {
      const int n = __popcll(mask);
      const int room = cap - pending;
      if (room == 0) {
        flush();
        continue;
      }
      // lanes whose rank among the remaining set bits is < room write this round
      const uint64_t below = mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
      const int rank = __popcll(below);
      const bool mine = (mask >> lane) & 1ull;
      if (mine && rank < room) {
        sv[pending + rank] = cv;
        si[pending + rank] = cid;
      }
      const int taken = n < room ? n : room;
      pending += taken;
      // clear the bits just written (the lowest `taken` set bits)
      for (int i = 0; i < taken; ++i) mask &= mask - 1;
      if (pending == cap) flush();
    }
  }
};

}  // namespace dfl
