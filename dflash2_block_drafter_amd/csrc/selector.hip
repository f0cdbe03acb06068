// Candidate selector (MAX dflash2_qwen3_5: `compute_candidates`, `DFlash2CandidateSelector.
// score_edges` and `select_path`; dflash2.ts diff: `#select`).
//
// Top-k (value descending, id ascending) runs in two stages.  Stage 1: one wavefront per
// 4096-logit chunk of a row holds 64 values per lane; the K-th largest of the 64 lane
// maxima is a value at least K chunk elements reach, so only elements >= it can be in the
// chunk's top K.  Those few candidates are merged into a running top-K list with a
// 64-lane bitonic sort (lanes 0..K-1 keep the list, lanes K..63 take new candidates).
// Stage 2 merges the per-chunk lists of a row the same way.  Ties on equal values are
// ordered by id, so the result is exact and unique for any input, including constant rows.
#include "common.hpp"
#include "kernels.hpp"

namespace dfl {

namespace {

constexpr int kChunk = 4096;       // logits per stage-1 wavefront (64 lanes x 64 values)
constexpr int kPerLane = kChunk / 64;
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

  __device__ void init(int K_, int lane_, float* sv_, int* si_) {
    K = K_;
    lane = lane_;
    sv = sv_;
    si = si_;
    v = -INFINITY;
    id = kNoId;
    pending = 0;
  }
  __device__ void flush() {
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
  __device__ void offer(bool take, float cv, int cid) {
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

// Stage 1: each wavefront reduces one chunk of one row to its top K.
__global__ __launch_bounds__(256) void topk_stage1_kernel(const float* __restrict__ logits, int V,
                                                          int K, int nchunks,
                                                          float* __restrict__ pv,
                                                          int* __restrict__ pi) {
  __shared__ float sv[4][64];
  __shared__ int si[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x * 4 + wave;
  const int row = blockIdx.y;
  if (chunk >= nchunks) return;
  const float* src = logits + (size_t)row * V;
  const int base = chunk * kChunk;
  float x[kPerLane];
  const bool full = base + kChunk <= V && (V & 3) == 0;
  if (full) {
#pragma unroll
    for (int j = 0; j < kPerLane / 4; ++j) {
      const f32x4_t q = *reinterpret_cast<const f32x4_t*>(src + base + j * 256 + lane * 4);
      x[4 * j] = q[0];
      x[4 * j + 1] = q[1];
      x[4 * j + 2] = q[2];
      x[4 * j + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerLane / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = base + j * 256 + lane * 4 + e;
        x[4 * j + e] = idx < V ? src[idx] : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) mx = fmaxf(mx, x[i]);
  // K-th largest lane maximum
  float sm = mx;
  int sid = lane;
  wave_bitonic_sort(sm, sid, lane);
  const float theta = __shfl(sm, K - 1, 64);

  TopkMerger mg;
  mg.init(K, lane, sv[wave], si[wave]);
#pragma unroll
  for (int j = 0; j < kPerLane / 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float val = x[4 * j + e];
      const int idx = base + j * 256 + lane * 4 + e;
      const bool take = val >= theta && idx < V;
      if (__ballot(take)) mg.offer(take, val, idx);
    }
  mg.flush();
  if (lane < K) {
    const size_t o = ((size_t)row * nchunks + chunk) * K + lane;
    pv[o] = mg.v;
    pi[o] = mg.id;
  }
}

// Stage 2: one wavefront merges a row's nchunks lists.
__global__ __launch_bounds__(64) void topk_stage2_kernel(const float* __restrict__ pv,
                                                         const int* __restrict__ pi, int K,
                                                         int nchunks, int32_t* __restrict__ ids,
                                                         float* __restrict__ vals) {
  __shared__ float sv[64];
  __shared__ int si[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int n = nchunks * K;
  const float* rv = pv + (size_t)row * n;
  const int* ri = pi + (size_t)row * n;
  TopkMerger mg;
  mg.init(K, lane, sv, si);
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    float cv = -INFINITY;
    int ci = kNoId;
    if (i < n) {
      cv = rv[i];
      ci = ri[i];
    }
    // the running list is sorted: its K-th entry bounds what can still enter
    const float kth = __shfl(mg.v, K - 1, 64);
    const int kthi = __shfl(mg.id, K - 1, 64);
    const bool take = i < n && ci != kNoId && before(cv, ci, kth, kthi);
    if (__ballot(take)) mg.offer(take, cv, ci);
  }
  mg.flush();
  if (lane < K) {
    ids[(size_t)row * K + lane] = mg.id;
    vals[(size_t)row * K + lane] = mg.v;
  }
}

// score_edges: one wavefront per (b, l).  pred[pid] * z and succ[cand] are gathered into
// LDS in fp32, then every lane computes K*K/64 dot products of length R in order.
__global__ __launch_bounds__(64) void score_edges_kernel(
    const int32_t* __restrict__ cand, const float* __restrict__ unary, const float* __restrict__ z,
    const int32_t* __restrict__ anchors, int S, int K, int R, const uint16_t* __restrict__ pred,
    const uint16_t* __restrict__ succ, int V, float* __restrict__ scores) {
  __shared__ float pz[32 * 128];
  __shared__ float sc[32 * 128];
  __shared__ int cid[32], pid[32];
  const int lane = threadIdx.x;
  const int l = blockIdx.x;
  const int b = blockIdx.y;
  const size_t bl = (size_t)b * S + l;
  auto clampv = [V](int t) { return t < 0 ? 0 : (t >= V ? V - 1 : t); };
  if (lane < K) {
    cid[lane] = clampv(cand[bl * K + lane]);
    pid[lane] = clampv(l == 0 ? anchors[b] : cand[(bl - 1) * K + lane]);
  }
  __syncthreads();
  for (int i = lane; i < K * R; i += 64) {
    const int p = i / R, r = i % R;
    pz[i] = bf16_to_f32(pred[(size_t)pid[p] * R + r]) * z[bl * R + r];
    sc[i] = bf16_to_f32(succ[(size_t)cid[p] * R + r]);
  }
  __syncthreads();
  for (int o = lane; o < K * K; o += 64) {
    const int p = o / K, c = o % K;
    float acc = 0.f;
    for (int r = 0; r < R; ++r) acc += pz[p * R + r] * sc[c * R + r];
    scores[bl * K * K + o] = unary[bl * K + c] + acc;
  }
}

// Greedy walk: one wavefront per request, lane c holds candidate c's score on the current
// predecessor row; argmax with the lowest c on ties.
__global__ __launch_bounds__(64) void select_path_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ cand, int S,
                                                         int K, int32_t* __restrict__ tokens) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  int j = 0;
  for (int l = 0; l < S; ++l) {
    const size_t bl = (size_t)b * S + l;
    float v = lane < K ? scores[(bl * K + j) * K + lane] : -INFINITY;
    int c = lane < K ? lane : kNoId;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oc = __shfl_xor(c, o, 64);
      if (before(ov, oc, v, c)) {
        v = ov;
        c = oc;
      }
    }
    // every lane agrees for finite scores; take lane 0's winner so a NaN can never send a
    // lane past the K candidates
    j = __shfl(c, 0, 64);
    j = (j >= 0 && j < K) ? j : 0;
    if (lane == 0) tokens[bl] = cand[bl * K + j];
  }
}

}  // namespace

TopkPlan plan_topk(int N, int V, int K) {
  TopkPlan pl;
  pl.chunk = kChunk;
  pl.nchunks = (V + kChunk - 1) / kChunk;
  const size_t entries = (size_t)N * pl.nchunks * K;
  pl.ws_bytes = entries * (sizeof(float) + sizeof(int));
  return pl;
}

hipError_t launch_topk(const TopkPlan& pl, const float* logits, int N, int V, int K,
                       int32_t* ids, float* vals, void* ws, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  float* pv = static_cast<float*>(ws);
  int* pi = reinterpret_cast<int*>(pv + (size_t)N * pl.nchunks * K);
  dim3 g1((pl.nchunks + 3) / 4, N);
  topk_stage1_kernel<<<g1, 256, 0, stream>>>(logits, V, K, pl.nchunks, pv, pi);
  topk_stage2_kernel<<<N, 64, 0, stream>>>(pv, pi, K, pl.nchunks, ids, vals);
  return hipGetLastError();
}

hipError_t launch_score_edges(const int32_t* cand, const float* unary, const float* z,
                              const int32_t* anchors, int B, int S, int K, int R,
                              const uint16_t* pred, const uint16_t* succ, int V, float* scores,
                              hipStream_t stream) {
  if (B <= 0 || S <= 0) return hipSuccess;
  score_edges_kernel<<<dim3(S, B), 64, 0, stream>>>(cand, unary, z, anchors, S, K, R, pred, succ,
                                                     V, scores);
  return hipGetLastError();
}

hipError_t launch_select_path(const float* scores, const int32_t* cand, int B, int S, int K,
                              int32_t* tokens, hipStream_t stream) {
  if (B <= 0 || S <= 0) return hipSuccess;
  select_path_kernel<<<B, 64, 0, stream>>>(scores, cand, S, K, tokens);
  return hipGetLastError();
}

}  // namespace dfl
