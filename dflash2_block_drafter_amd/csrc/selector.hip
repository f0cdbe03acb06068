// Candidate selector (MAX dflash2_qwen3_5: `compute_candidates`, `DFlash2CandidateSelector.
// score_edges` and `select_path`; dflash2.ts diff: `#select`).
//
// Top-k (value descending, id ascending) is guided by the row maxima of 256-column tiles,
// which the head projection writes with its logits (a separate pass computes them for
// logits from elsewhere).  theta, the K-th largest maximum over K disjoint groups of tiles,
// is reached by K distinct logits, so every top-K logit is >= theta and sits in a tile whose
// maximum is >= theta; only those tiles are read (usually K to 2K of a row's V/256).  Their
// values >= theta (usually K to 2K) are gathered and ranked once when there are at most
// 64; otherwise they are merged
// into a running top-K list with a 64-lane bitonic sort (lanes 0..K-1 keep the list, lanes
// K..63 take new candidates).  Ties are ordered by id, so the result is exact and unique for
// any input, including constant rows (where every tile qualifies).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace dfl {

namespace {

// The tile maxima of dfl_compute_candidates_static live here instead of in a caller
// workspace: one copy of this array per GPU the library runs on, held until the process
// ends.  On the host the name is only a stand-in for the device symbol; host code passes the
// address topk_static_scratch() looked up, never the name, to a kernel.
constexpr size_t kStaticScratchFloats = size_t(1) << 20;  // 4 MiB
__device__ __align__(256) float scratch[kStaticScratchFloats];
constexpr int kMaxDevices = 64;

// Row maxima of every kGemmTileN-column tile of fp32 logits (the values the head projection
// writes alongside its logits).  A quarter-wavefront (16 lanes, 4 x float4 each) covers one
// tile; a wavefront takes kRowmaxTiles consecutive tiles of a row, so each lane has
// kRowmaxTiles/4 x 4 float4 loads in flight before any reduction.
constexpr int kRowmaxTiles = 16;

__global__ __launch_bounds__(256) void tile_rowmax_kernel(const float* __restrict__ logits, int V, int ntiles,
                                                          float* __restrict__ tile_max) {
  constexpr int TQ = kGemmTileN / 64;  // float4 per lane per tile (16 lanes per tile)
  constexpr int PASS = kRowmaxTiles / 4;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;     // which of the wavefront's 4 tiles in a pass
  const int l16 = lane & 15;
  const int t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kRowmaxTiles;
  const int row = blockIdx.y;
  if (t0 >= ntiles) return;
  const float* src = logits + (size_t)row * V;
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  float m[PASS];
#pragma unroll
  for (int p = 0; p < PASS; ++p) {
    const int t = t0 + p * 4 + q;
    float acc = -INFINITY;
#pragma unroll
    for (int j = 0; j < TQ; ++j) {
      const int col = t * kGemmTileN + j * 64 + l16 * 4;
      if (vec && col + 4 <= V) {
        // read once: non-temporal, so the stream does not evict what later kernels reuse
        const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + col));
        acc = fmaxf(acc, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < V) acc = fmaxf(acc, src[col + e]);
      }
    }
    m[p] = acc;
  }
#pragma unroll
  for (int p = 0; p < PASS; ++p) {
    m[p] = row16_max(m[p]);
    const int t = t0 + p * 4 + q;
    if (l16 == 0 && t < ntiles) tile_max[(size_t)row * ntiles + t] = m[p];
  }
}

// Top-K of a row from its tile maxima (tiles of kGemmTileN columns).  theta is a value that
// K distinct logits reach, so every top-K logit is >= theta and lies in a tile whose maximum
// is >= theta: only those tiles (ties included) are scanned.  One workgroup of four
// wavefronts per row.  Wavefront 0 reads the tile maxima 64 * kTmPerLane at a time (one
// round of loads) into 256 group maxima and takes their K-th largest as theta by ballots
// (no sorting); then the qualifying tiles are listed in LDS and each wavefront loads
// kFastTilesInFlight of them at once.  With one round of tile maxima, their values >= theta
// are gathered into LDS and, when at most 64, ranked once by wavefront 0 (each lane counts
// the candidates that precede its own); otherwise (and for longer rows) each wavefront
// merges its tiles, kTilesInFlight at a time, into its own list and wavefront 0 merges the
// four lists.
constexpr int kTmPerLane = 16;
constexpr int kTilesInFlight = 4;
constexpr int kFastTilesInFlight = 8;  // the fast path's loads: usually every qualifying tile at once

// Merge lanes 0..K-1 of the other three wavefronts' lists (lv/li) into wavefront 0's list.
__device__ __forceinline__ void merge_wave_lists(TopkMerger& mg, const float (*lv)[64], const int (*li)[64],
                                                 int K, int lane) {
  for (int w = 1; w < 4; ++w) {
    const float cv = lv[w][lane];
    const int ci = li[w][lane];
    const float kth = __shfl(mg.v, K - 1, 64);
    const int kthi = __shfl(mg.id, K - 1, 64);
    const bool take = lane < K && ci != kNoId && before(cv, ci, kth, kthi);
    if (__ballot(take)) mg.offer(take, cv, ci);
  }
  mg.flush();
}

// The top-K of one row given its tile maxima tm (in global memory, or in LDS), for one
// 256-thread workgroup: the body of topk_tiles_kernel and of topk_scan_kernel.
__device__ __forceinline__ void topk_row(const float* tm, const float* __restrict__ src, int V, int ntiles, int K,
                                         int row, int32_t* __restrict__ ids, float* __restrict__ vals,
                                         const int32_t* __restrict__ id_map,
                                         const uint32_t* __restrict__ bound = nullptr) {
  constexpr int TW = kGemmTileN;
  constexpr int TPL = TW / 64;                 // values of a tile per lane
  constexpr int CH = 64 * kTmPerLane;          // tile maxima per round
  __shared__ float sv[4][64];
  __shared__ int si[4][64];
  __shared__ float lv[4][64];
  __shared__ int li[4][64];
  __shared__ int tl[CH];                       // qualifying tiles of the current round
  __shared__ float theta_s;
  __shared__ int tcount;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  TopkMerger mg;

  // theta: a value that K distinct logits reach, as large as cheaply found.  Wavefront 0's
  // lane L keeps four group maxima, group (L, i) holding the tiles L + 64 (i + 4k); the K-th
  // largest of the 256 group maxima is reached by K distinct logits (one in each of K
  // disjoint groups), so every top-K logit is >= it, and with <= 256 tiles it is the K-th
  // largest tile maximum itself.  It is found bit by bit in an order-preserving integer map
  // of the floats (the largest u with at least K group maxima >= u): ballots, no sorting.
  // -inf with fewer than K groups (every tile then qualifies).  With one round of tile
  // maxima wavefront 0 still holds them and lists the qualifying tiles at once.
  __shared__ __attribute__((aligned(16))) float cand_v[64];
  __shared__ __attribute__((aligned(16))) int cand_i[64];
  __shared__ int ccount;
  const bool one_round = ntiles <= CH;
  if (wave == 0) {
    // the head's bound slots, when given, load with the tile maxima
    uint32_t b = bound && lane < kTileBoundSlots ? bound[lane] : 0xFFFFFFFFu;
    float g[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) g[i] = __builtin_nanf("");  // NaN: empty (fmaxf skips NaN)
    float t[kTmPerLane];
    for (int c0 = 0; c0 < ntiles; c0 += CH) {
#pragma unroll
      for (int j = 0; j < kTmPerLane; ++j) {
        const int i = c0 + j * 64 + lane;
        t[j] = i < ntiles ? tm[i] : __builtin_nanf("");
      }
#pragma unroll
      for (int j = 0; j < kTmPerLane; ++j) g[j & 3] = fmaxf(g[j & 3], t[j]);
    }
    uint32_t u[4];
    int groups = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u[i] = g[i] == g[i] ? float_order(g[i]) : 0u;
      groups += __popcll(__ballot(g[i] == g[i]));
    }
    uint32_t cu = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t tryu = cu | (1u << b);
      int n = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) n += __popcll(__ballot(g[i] == g[i] && u[i] >= tryu));
      if (n >= K) cu = tryu;
    }
    float th = groups >= K ? order_float(cu) : -INFINITY;  // the same in every lane
    if (bound) {
      // the head's bound slots (K <= kTileBoundSlots): once all are filled their least value
      // is reached by kTileBoundSlots logits of distinct tiles, so it is a theta too, and the
      // tiles below it may never have been stored
      static_assert(kTileBoundSlots == 16, "one row of lanes");
      b = (uint32_t)__builtin_amdgcn_readfirstlane((int)row16_umin(b));
      if (b != 0u) th = fmaxf(th, order_float(b));
    }
    if (lane == 0) theta_s = th;
    if (one_round) {
      int cnt = 0;
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
      for (int j = 0; j < kTmPerLane; ++j) {
        const int i = j * 64 + lane;
        const bool q = i < ntiles && t[j] >= th;
        const uint64_t mask = __ballot(q);
        if (q) tl[cnt + __popcll(mask & below)] = i;
        cnt += __popcll(mask);
      }
      if (lane == 0) {
        tcount = cnt;
        ccount = 0;
      }
    }
  }
  __syncthreads();
  const float theta = theta_s;

  // Fast path (one round of tile maxima): every value >= theta is a candidate, usually K to
  // 2K of them, so they are gathered into LDS (ballot + one LDS atomic per wavefront step)
  // and ranked once by wavefront 0.  More than 64 of them (ties at theta across many tiles,
  // constant rows, rows mostly -inf) falls through to the merging scan below.
  if (one_round) {
    constexpr int F = kFastTilesInFlight;
    const int cnt = tcount;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int b0 = wave * F; b0 < cnt; b0 += 4 * F) {
      const int n = min(F, cnt - b0);
      int tile[F];
      float x[F][TPL];
#pragma unroll
      for (int q = 0; q < F; ++q) tile[q] = tl[b0 + min(q, n - 1)];
#pragma unroll
      for (int q = 0; q < F; ++q)
#pragma unroll
        for (int e = 0; e < TPL; ++e) {
          const int col = tile[q] * TW + e * 64 + lane;
          x[q][e] = col < V ? src[col] : -INFINITY;
        }
#pragma unroll
      for (int q = 0; q < F; ++q)
#pragma unroll
        for (int e = 0; e < TPL; ++e) {
          const int col = tile[q] * TW + e * 64 + lane;
          const bool take = q < n && col < V && x[q][e] >= theta;
          const uint64_t mask = __ballot(take);
          if (mask) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&ccount, __popcll(mask));
            base = __shfl(base, 0, 64);
            const int slot = base + __popcll(mask & below);
            if (take && slot < 64) {
              cand_v[slot] = x[q][e];
              cand_i[slot] = col;
            }
          }
        }
    }
    __syncthreads();
    const int total = ccount;
    if (total <= 64) {
      if (wave != 0) return;
      // the first K in candidate order by rank: each lane counts the candidates that precede
      // its own (read four at a time, every lane the same address); ids are distinct, so the
      // ranks are 0 .. total - 1.  With fewer than K candidates the rest are (-inf, kNoId).
      const float v = lane < total ? cand_v[lane] : -INFINITY;
      const int id = lane < total ? cand_i[lane] : kNoId;
      int rank = 0;
      for (int j = 0; j < total; j += 4) {
        const f32x4_t cv = *reinterpret_cast<const f32x4_t*>(&cand_v[j]);
        const u32x4_t ci = *reinterpret_cast<const u32x4_t*>(&cand_i[j]);
#pragma unroll
        for (int t = 0; t < 4; ++t) rank += j + t < total && before(cv[t], (int)ci[t], v, id);
      }
      const int slot = lane < total ? rank : lane;
      if (slot < K) {
        ids[(size_t)row * K + slot] = id_map && id >= 0 && id < V ? id_map[id] : id;
        vals[(size_t)row * K + slot] = v;
      }
      return;
    }
  }

  // scan the qualifying tiles: per round wavefront 0 lists them in LDS, then wavefront w
  // takes list entries [w*F, w*F + F), [w*F + 4F, ...), F = kTilesInFlight at a time
  mg.init(K, lane, sv[wave], si[wave]);
  for (int c0 = 0; c0 < ntiles; c0 += CH) {
    if (wave == 0) {
      float t[kTmPerLane];
#pragma unroll
      for (int j = 0; j < kTmPerLane; ++j) {
        const int i = c0 + j * 64 + lane;
        t[j] = i < ntiles ? tm[i] : -INFINITY;
      }
      int cnt = 0;
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
      for (int j = 0; j < kTmPerLane; ++j) {
        const int i = c0 + j * 64 + lane;
        const bool q = i < ntiles && t[j] >= theta;
        const uint64_t mask = __ballot(q);
        if (q) tl[cnt + __popcll(mask & below)] = i;
        cnt += __popcll(mask);
      }
      if (lane == 0) tcount = cnt;
    }
    __syncthreads();
    const int cnt = tcount;
    for (int b0 = wave * kTilesInFlight; b0 < cnt; b0 += 4 * kTilesInFlight) {
      const int n = min(kTilesInFlight, cnt - b0);
      int tile[kTilesInFlight];
      float x[kTilesInFlight][TPL];
#pragma unroll
      for (int q = 0; q < kTilesInFlight; ++q) tile[q] = tl[b0 + min(q, n - 1)];
#pragma unroll
      for (int q = 0; q < kTilesInFlight; ++q)
#pragma unroll
        for (int e = 0; e < TPL; ++e) {
          const int col = tile[q] * TW + e * 64 + lane;
          x[q][e] = col < V ? src[col] : -INFINITY;
        }
#pragma unroll
      for (int q = 0; q < kTilesInFlight; ++q)
#pragma unroll
        for (int e = 0; e < TPL; ++e) {
          const int col = tile[q] * TW + e * 64 + lane;
          const float kth = __shfl(mg.v, K - 1, 64);
          const int kthi = __shfl(mg.id, K - 1, 64);
          // q >= n: a repeat of the last tile (n < F), not offered twice; below theta a
          // value cannot be in the top K
          const bool take = q < n && col < V && x[q][e] >= theta && before(x[q][e], col, kth, kthi);
          if (__ballot(take)) mg.offer(take, x[q][e], col);
        }
    }
    __syncthreads();  // tl is rewritten next round
  }
  mg.flush();
  lv[wave][lane] = mg.v;
  li[wave][lane] = mg.id;
  __syncthreads();
  if (wave != 0) return;
  merge_wave_lists(mg, lv, li, K, lane);
  if (lane < K) {
    // the list is ordered by (value, column); a draft vocabulary reports its listed ids
    const int col = mg.id;
    ids[(size_t)row * K + lane] = id_map && col >= 0 && col < V ? id_map[col] : col;
    vals[(size_t)row * K + lane] = mg.v;
  }
}

__global__ __launch_bounds__(256) void topk_tiles_kernel(const float* __restrict__ logits, int V,
                                                         const float* __restrict__ tile_max, int ntiles,
                                                         int K, int32_t* __restrict__ ids,
                                                         float* __restrict__ vals,
                                                         const int32_t* __restrict__ id_map,
                                                         const uint32_t* __restrict__ tile_bound) {
  const int row = blockIdx.x;
  topk_row(tile_max + (size_t)row * ntiles, logits + (size_t)row * V, V, ntiles, K, row, ids, vals, id_map,
           tile_bound ? tile_bound + (size_t)row * kTileBoundSlots : nullptr);
}

// Maximum over each aligned group of 16 lanes, left in every lane of the group, with DPP
// lane moves inside the registers (no LDS round trip): the row's mirror, the half-row's
// mirror, then the two quad permutations that swap neighbours and pairs.
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));  // row_mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));   // quad_perm 1,0,3,2
  return v;
}

// The selector projection z = h . proj^T (fp32) of kProjRows rows per 256-thread
// workgroup, on the matrix cores: the four wavefronts take a quarter of K each (H a multiple
// of 128, so each quarter is whole 32-deep steps) over NCB 16-column blocks from cb0 (16x16x32
// bf16 MFMA blocks); the four partial products are summed through LDS in wavefront order, so
// an output's value depends neither on timing nor on how many column blocks a workgroup
// takes.  Lane l supplies row / column l % 16 at K offset 8 (l / 16) of a step, 16 bytes
// straight from global memory.  Rows past N and columns past R read the last valid one and
// are not written.
constexpr int kProjRows = 16;
constexpr int kProjMaxR = 64;

// U: K steps whose loads are issued together (the order of the MFMAs, and so the result, is
// the same for every U).
template <int U, int NCB>
__device__ __forceinline__ void selproj_block(const uint16_t* __restrict__ h, int N, int H,
                                              const uint16_t* __restrict__ proj, int R, float* __restrict__ z,
                                              int blk, int cb0) {
  __shared__ float part[4][kProjRows][kProjMaxR + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r0 = blk * kProjRows;
  const int kq = H / 4;
  const int nsteps = kq / 32;
  const int koff = wave * kq + 8 * (lane >> 4);
  const uint16_t* ap = h + (size_t)min(r0 + (lane & 15), N - 1) * H + koff;
  const uint16_t* bp[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) bp[c] = proj + (size_t)min((cb0 + c) * 16 + (lane & 15), R - 1) * H + koff;
  const int nb = min(NCB, (R + 15) / 16 - cb0);  // column blocks with columns < R
  f32x4_t acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsteps; s0 += U) {
    // every load is issued (steps past the last re-read it) before the first MFMA
    bf16x8_t a[U], b[U][NCB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(s0 + u, nsteps - 1) * 32;
      a[u] = *reinterpret_cast<const bf16x8_t*>(ap + k);
#pragma unroll
      for (int c = 0; c < NCB; ++c) b[u][c] = *reinterpret_cast<const bf16x8_t*>(bp[c] + k);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < nsteps) {
#pragma unroll
        for (int c = 0; c < NCB; ++c)
          if (c < nb) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][c], acc[c], 0, 0, 0);
      }
  }
  // lane holds column (cb0 + c) * 16 + lane % 16, rows 4 (lane / 16) + e
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) part[wave][4 * (lane >> 4) + e][c * 16 + (lane & 15)] = acc[c][e];
  __syncthreads();
  const int cols = min(NCB * 16, R - cb0 * 16);
  for (int i = threadIdx.x; i < kProjRows * cols; i += 256) {
    const int r = i / cols, c = i % cols;
    if (r0 + r < N)
      z[(size_t)(r0 + r) * R + cb0 * 16 + c] = ((part[0][r][c] + part[1][r][c]) + part[2][r][c]) + part[3][r][c];
  }
}

// One 16-column block of 16 rows a workgroup (blockIdx.x: rows, blockIdx.y: columns): four
// times the workgroups of the all-columns form, each with a quarter of the weight rows.
__global__ __launch_bounds__(256) void selproj_kernel(const uint16_t* __restrict__ h, int N, int H,
                                                      const uint16_t* __restrict__ proj, int R,
                                                      float* __restrict__ z) {
  selproj_block<8, 1>(h, N, H, proj, R, z, blockIdx.x, blockIdx.y);
}

// Top-K of each row straight from the logits: one 256-thread workgroup per row scans the
// whole row once (each round, 4 wavefronts x 16 tiles of 256 columns, 16 lanes a tile; the
// next round's loads are issued before this round's reduction), keeps the row's tile maxima
// in LDS and then runs topk_row on them.  Every row's top-K thus runs as soon as its own
// scan ends, beside the other rows' scans, instead of in a launch after all of them.
constexpr int kScanMaxTiles = kSelectScanMaxTiles;

//
// Workgroups past the N rows' (launched when h is given) compute the selector projection
// (selproj_block, kProjRows rows each) beside the scans.
template <bool VEC>
__global__ __launch_bounds__(256) void topk_scan_kernel(const float* __restrict__ logits, int V, int ntiles, int K,
                                                        int32_t* __restrict__ ids, float* __restrict__ vals,
                                                        const int32_t* __restrict__ id_map,
                                                        const uint16_t* __restrict__ h, int N, int H,
                                                        const uint16_t* __restrict__ proj, int R,
                                                        float* __restrict__ z) {
  if ((int)blockIdx.x >= N) {
    selproj_block<2, kProjMaxR / 16>(h, N, H, proj, R, z, blockIdx.x - N, 0);  // (2: within the scan's registers)
    return;
  }
  constexpr int TQ = kGemmTileN / 64;  // float4 per lane per tile
  constexpr int PASS = 4;              // tiles per 16-lane group per round
  constexpr int ROUND = 4 * 4 * PASS;  // tiles per round: 4 wavefronts x 4 groups x PASS
  __shared__ float tms[kScanMaxTiles];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const int row = blockIdx.x;
  const float* src = logits + (size_t)row * V;
  // tile of (round c, pass p) for this lane's group
  auto tile_of = [&](int c, int p) { return c * ROUND + (wave * PASS + p) * 4 + q; };
  // Every load is unconditional, at an address clamped into the row (tiles past the last and
  // columns past V re-read valid ones), so no branch separates a round's loads and the next
  // round's stay in flight while this one is reduced; the clamped values are replaced by
  // -inf after the wait.
  auto load_round = [&](int c, f32x4_t (&v)[PASS][TQ]) {
#pragma unroll
    for (int p = 0; p < PASS; ++p) {
      const int t = min(tile_of(c, p), ntiles - 1);
#pragma unroll
      for (int j = 0; j < TQ; ++j) {
        const int col = t * kGemmTileN + j * 64 + l16 * 4;
        if constexpr (VEC) {
          // read once: non-temporal, so the stream does not evict what later kernels reuse
          v[p][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + min(col, V - 4)));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[p][j][e] = src[min(col + e, V - 1)];
        }
      }
    }
  };
  auto reduce_round = [&](int c, const f32x4_t (&v)[PASS][TQ]) {
#pragma unroll
    for (int p = 0; p < PASS; ++p) {
      const int t = tile_of(c, p);
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < TQ; ++j) {
        const int col = t * kGemmTileN + j * 64 + l16 * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, t < ntiles && col + e < V ? v[p][j][e] : -INFINITY);
      }
      m = max16(m);
      if (l16 == 0 && t < ntiles) tms[t] = m;
    }
  };
  // two rounds in flight: the next round's loads go out (clamped past the end) before this
  // round is reduced
  const int rounds = (ntiles + ROUND - 1) / ROUND;
  f32x4_t va[PASS][TQ], vb[PASS][TQ];
  load_round(0, va);
  for (int c = 0; c < rounds; c += 2) {
    load_round(c + 1, vb);
    reduce_round(c, va);
    load_round(c + 2, va);
    reduce_round(c + 1, vb);
  }
  __syncthreads();
  topk_row(tms, src, V, ntiles, K, row, ids, vals, id_map);
}

// score_edges, one wavefront per (b, l) slot, NW wavefronts per workgroup.  Three memory
// round trips per slot, every load of a round issued before its first use: (1) the slot's
// candidate ids, predecessor ids (the anchor at l = 0, else the previous slot's
// candidates), unary scores and z; (2) the K predecessor and K successor codebook rows,
// 16 bytes a load when R is a multiple of 8 (VEC), else one element; (3) the scores out.
// The rows go to the wavefront's LDS as fp32 rows padded to R + 1 floats (pred * z, and
// succ), so the K * K dot products read distinct banks; lane outputs o = lane, lane + 64,
// ... (predecessor o / K, candidate o % K), each summing r = 0..R-1 in order.
constexpr int kMaxRowChunks = 8;  // 16-byte chunks per lane: K * R / 8 <= 32 * 128 / 8 = 512

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool VEC>
__global__ __launch_bounds__(256) void score_edges_kernel(const int32_t* __restrict__ cand,
                                                          const float* __restrict__ unary,
                                                          const float* __restrict__ z,
                                                          const int32_t* __restrict__ anchors, int S, int K, int R,
                                                          const uint16_t* __restrict__ pred,
                                                          const uint16_t* __restrict__ succ, int V,
                                                          float* __restrict__ scores) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int l = blockIdx.x * (blockDim.x >> 6) + wave;
  if (l >= S) return;
  const int RP = R + 1;
  float* pz = smem + (size_t)wave * (2 * K * RP + R);
  float* sc = pz + K * RP;
  float* zs = sc + K * RP;
  const size_t bl = (size_t)b * S + l;
  auto clampv = [V](int t) { return t < 0 ? 0 : (t >= V ? V - 1 : t); };
  // (1) ids, unary, z
  int cid = 0, pid = 0;
  float u = 0.f;
  if (lane < K) {
    cid = clampv(cand[bl * K + lane]);
    pid = clampv(l == 0 ? anchors[b] : cand[(bl - 1) * K + lane]);
    u = unary[bl * K + lane];
  }
  const float z0 = lane < R ? z[bl * R + lane] : 0.f;
  const float z1 = lane + 64 < R ? z[bl * R + lane + 64] : 0.f;
  if (lane < R) zs[lane] = z0;
  if (lane + 64 < R) zs[lane + 64] = z1;
  wave_lds_sync();
  // (2) codebook rows
  if (VEC) {
    const int per_row = R / 8;
    u32x4_t pv[kMaxRowChunks], sv[kMaxRowChunks];
#pragma unroll
    for (int i = 0; i < kMaxRowChunks; ++i) {
      const int idx = lane + 64 * i;
      const int p = min(idx / per_row, K - 1);
      const int pi = __shfl(pid, p, 64);
      const int ci = __shfl(cid, p, 64);
      if (idx < K * per_row) {
        const int r0 = (idx % per_row) * 8;
        pv[i] = *reinterpret_cast<const u32x4_t*>(pred + (size_t)pi * R + r0);
        sv[i] = *reinterpret_cast<const u32x4_t*>(succ + (size_t)ci * R + r0);
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxRowChunks; ++i) {
      const int idx = lane + 64 * i;
      if (idx < K * per_row) {
        const int p = idx / per_row, r0 = (idx % per_row) * 8;
        float pf[8], sf[8];
        unpack8(pv[i], pf);
        unpack8(sv[i], sf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pz[p * RP + r0 + e] = pf[e] * zs[r0 + e];
          sc[p * RP + r0 + e] = sf[e];
        }
      }
    }
  } else {
    for (int i0 = 0; i0 < K * R; i0 += 64 * kMaxRowChunks) {
      float pf[kMaxRowChunks], sf[kMaxRowChunks];
#pragma unroll
      for (int i = 0; i < kMaxRowChunks; ++i) {
        const int idx = i0 + lane + 64 * i;
        const int p = min(idx / R, K - 1);
        const int pi = __shfl(pid, p, 64);
        const int ci = __shfl(cid, p, 64);
        if (idx < K * R) {
          pf[i] = bf16_to_f32(pred[(size_t)pi * R + idx % R]);
          sf[i] = bf16_to_f32(succ[(size_t)ci * R + idx % R]);
        }
      }
#pragma unroll
      for (int i = 0; i < kMaxRowChunks; ++i) {
        const int idx = i0 + lane + 64 * i;
        if (idx < K * R) {
          const int p = idx / R, r = idx % R;
          pz[p * RP + r] = pf[i] * zs[r];
          sc[p * RP + r] = sf[i];
        }
      }
    }
  }
  wave_lds_sync();
  // (3) the K * K scores
  for (int o0 = 0; o0 < K * K; o0 += 64) {
    const int o = o0 + lane;
    const int p = min(o / K, K - 1), c = o % K;
    const float uc = __shfl(u, c, 64);
    const float* a = pz + p * RP;
    const float* w = sc + c * RP;
    float acc = 0.f;
    for (int r = 0; r < R; ++r) acc += a[r] * w[r];
    if (o < K * K) scores[bl * K * K + o] = uc + acc;
  }
}

// Greedy walk over given scores: one wavefront per request.  Chunks of slots are copied into
// LDS with coalesced loads (every load of a chunk in flight at once); the argmax of each
// (slot, predecessor) row is found for all rows at once, one row per lane, and the walk then
// follows them (the argmax takes the lowest candidate on ties and stays in [0, K) whatever
// the values).
constexpr int kWalkLdsFloats = 4096;

__global__ __launch_bounds__(64) void select_path_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ cand, int S, int K,
                                                         int32_t* __restrict__ tokens) {
  __shared__ __attribute__((aligned(16))) float sc[kWalkLdsFloats];
  __shared__ int ids[kWalkLdsFloats];   // the chunk's candidate ids (n * K <= kWalkLdsFloats / K)
  __shared__ int best[kWalkLdsFloats];  // argmax of each (slot, predecessor) row of the chunk
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const int KK = K * K;
  const int chunk = max(1, min(S, kWalkLdsFloats / KK));
  int j = 0;
  for (int l0 = 0; l0 < S; l0 += chunk) {
    const int n = min(chunk, S - l0);
    const float* src = scores + ((size_t)b * S + l0) * KK;
    const int m = n * KK;
    // the chunk's candidate ids (so that no step of the walk waits on a global load): the
    // first 1024 are loaded before the scores are stored, in the same round trip
    const int32_t* csrc = cand + ((size_t)b * S + l0) * K;
    const int nk = n * K;
    int idv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = lane + 64 * i;
      if (q < nk) idv[i] = csrc[q];
    }
    if (((reinterpret_cast<uintptr_t>(src) & 15) | (m & 3)) == 0) {
      // the chunk as float4: at most kWalkLdsFloats / 4 / 64 = 16 loads a lane, all in flight
      f32x4_t v[kWalkLdsFloats / 256];
#pragma unroll
      for (int i = 0; i < kWalkLdsFloats / 256; ++i) {
        const int q = lane + 64 * i;
        if (q < m / 4) v[i] = reinterpret_cast<const f32x4_t*>(src)[q];
      }
#pragma unroll
      for (int i = 0; i < kWalkLdsFloats / 256; ++i) {
        const int q = lane + 64 * i;
        if (q < m / 4) reinterpret_cast<f32x4_t*>(sc)[q] = v[i];
      }
    } else {
      for (int i0 = 0; i0 < m; i0 += 64 * 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = i0 + lane + 64 * i;
          if (q < m) v[i] = src[q];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = i0 + lane + 64 * i;
          if (q < m) sc[q] = v[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = lane + 64 * i;
      if (q < nk) ids[q] = idv[i];
    }
    for (int i0 = 64 * 16; i0 < nk; i0 += 64 * 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = i0 + lane + 64 * i;
        if (q < nk) v[i] = csrc[q];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = i0 + lane + 64 * i;
        if (q < nk) ids[q] = v[i];
      }
    }
    __syncthreads();
    // the argmax of every (slot, predecessor) row of the chunk does not depend on the path:
    // all of them in parallel (lowest candidate on ties), then the walk is a chain of lookups
    for (int r = lane; r < n * K; r += 64) {
      const float* row = sc + (size_t)r * K;
      float bv = row[0];
      int bc = 0;
      for (int c = 1; c < K; ++c)
        if (before(row[c], c, bv, bc)) {
          bv = row[c];
          bc = c;
        }
      best[r] = bc;
    }
    __syncthreads();
    if (lane == 0) {
      for (int w = 0; w < n; ++w) {
        j = best[w * K + j];
        tokens[(size_t)b * S + l0 + w] = ids[w * K + j];
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// Edge scores of one slot on the matrix cores: S[p][c] = unary[c] + sum_r (pred[pid_p][r] *
// z[r]) * succ[cid_c][r] for p, c < K <= 16 is a [16 x R] . [R x 16] product in fp32
// (v_mfma_f32_16x16x4_f32, R/4 steps).  Lane l supplies row / column l % 16 for the R/4
// consecutive r from (R/4) (l / 16), one per step (the order in which the products of a
// sum are added is free), so its codebook and z values are contiguous runs: 16-byte loads
// when R = 64 and the codebooks are 16-byte aligned.  pred * z is rounded to fp32 as one
// product, as in the row-by-row form.  The lane ends with S[4 (l / 16) + e][l % 16], e =
// 0..3.  Every lane of the wavefront takes part; ids are clamped into [0, V) by the caller.
constexpr int kMfmaMaxK = 16;
constexpr int kMfmaMaxR = 64;

__device__ __forceinline__ f32x4_t slot_scores_mfma(const uint16_t* __restrict__ pred,
                                                    const uint16_t* __restrict__ succ, int pid, int cid,
                                                    const float* __restrict__ zrow, int K, int R, int lane) {
  constexpr int QM = kMfmaMaxR / 4;
  const int i = lane & 15, kq = lane >> 4;
  const bool live = i < K;
  const int pi = __shfl(pid, i, 64), ci = __shfl(cid, i, 64);
  const int RQ = R / 4, r0 = kq * RQ;
  float a[QM], bv[QM];
  const uint16_t* prow = pred + (size_t)pi * R + r0;
  const uint16_t* srow = succ + (size_t)ci * R + r0;
  const float* zr = zrow + r0;
  const bool vec = R == kMfmaMaxR &&
                   ((reinterpret_cast<uintptr_t>(pred) | reinterpret_cast<uintptr_t>(succ) |
                     reinterpret_cast<uintptr_t>(zrow)) & 15) == 0;
  if (vec) {
    u32x4_t pv[2], sv[2];
    f32x4_t zv[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pv[h] = *reinterpret_cast<const u32x4_t*>(prow + 8 * h);
      sv[h] = *reinterpret_cast<const u32x4_t*>(srow + 8 * h);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) zv[h] = *reinterpret_cast<const f32x4_t*>(zr + 4 * h);
    float pf[QM], sf[QM];
    unpack8(pv[0], pf);
    unpack8(pv[1], pf + 8);
    unpack8(sv[0], sf);
    unpack8(sv[1], sf + 8);
#pragma unroll
    for (int q = 0; q < QM; ++q) {
      a[q] = live ? pf[q] * zv[q >> 2][q & 3] : 0.f;
      bv[q] = live ? sf[q] : 0.f;
    }
  } else {
#pragma unroll
    for (int q = 0; q < QM; ++q)
      if (q < RQ) {
        a[q] = live ? bf16_to_f32(prow[q]) * zr[q] : 0.f;
        bv[q] = live ? bf16_to_f32(srow[q]) : 0.f;
      }
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < QM; ++q)
    if (q < RQ) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], bv[q], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ bool mfma_scores_fit(int K, int R) {
  return K >= 1 && K <= kMfmaMaxK && R >= 4 && R <= kMfmaMaxR && R % 4 == 0;
}

// The first of each aligned group of 16 lanes in candidate order (value descending, then
// id ascending), left in every lane of the group: the same DPP lane moves as max16, moving
// the value and its id together (the order is total, so any reduction order gives the same
// winner).
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& id) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oid = __builtin_amdgcn_update_dpp(0, id, CTRL, 0xF, 0xF, false);
  if (before(ov, oid, v, id)) {
    v = ov;
    id = oid;
  }
}
__device__ __forceinline__ void argmax16(float& v, int& id) {
  argmax_step<0x140>(v, id);  // row_mirror
  argmax_step<0x141>(v, id);  // row_half_mirror
  argmax_step<0x4E>(v, id);   // quad_perm 2,3,0,1
  argmax_step<0xB1>(v, id);   // quad_perm 1,0,3,2
}

// The edge scores and the walk of B requests in one launch: one workgroup per request, one
// wavefront per slot (slots l = wave, wave + kSelWaves, ...).  Each wavefront scores its slot
// on the matrix cores and keeps, for every predecessor p, the lowest candidate c of maximum
// score; after a barrier one lane walks those argmaxima from predecessor 0.  Candidates come
// from the top-k (their ids index the codebooks), scores are also written out when asked.
constexpr int kSelWaves = 16;
constexpr int kSelMaxS = 64;

__global__ __launch_bounds__(kSelWaves * 64) void edges_walk_kernel(
    const int32_t* __restrict__ cand, const float* __restrict__ unary, const float* __restrict__ z, int R,
    const int32_t* __restrict__ anchors, int S, int K, const uint16_t* __restrict__ pred,
    const uint16_t* __restrict__ succ, int V, float* __restrict__ scores_out, int32_t* __restrict__ tokens) {
  __shared__ int best_s[kSelMaxS][kMfmaMaxK];
  __shared__ int cand_s[kSelMaxS][kMfmaMaxK];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  auto clampv = [V](int t) { return t < 0 ? 0 : (t >= V ? V - 1 : t); };
  for (int l = wave; l < S; l += kSelWaves) {
    const size_t row = (size_t)b * S + l;
    int cid = 0, pid = 0, craw = 0;
    float u = 0.f;
    if (lane < K) {
      craw = cand[row * K + lane];
      cid = clampv(craw);
      pid = clampv(l == 0 ? anchors[b] : cand[(row - 1) * K + lane]);
      u = unary[row * K + lane];
    }
    const f32x4_t acc = slot_scores_mfma(pred, succ, pid, cid, z + row * R, K, R, lane);
    const int c = lane & 15;
    const float uc = __shfl(u, c, 64);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 4 * (lane >> 4) + e;
      const float sc = uc + acc[e];
      if (scores_out && p < K && c < K) scores_out[row * K * K + p * K + c] = sc;
      // argmax over the 16 lanes of this row of the tile (lowest c on ties; c >= K never wins)
      float bv = c < K ? sc : -INFINITY;
      int bc = c;
      argmax16(bv, bc);
      if (c == 0 && p < K) best_s[l][p] = bc;
    }
    if (lane < K) cand_s[l][lane] = craw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int j = 0;
    for (int l = 0; l < S; ++l) {
      j = best_s[l][j];
      tokens[(size_t)b * S + l] = cand_s[l][j];
    }
  }
}

// score_edges on the matrix cores, one wavefront per (b, l) slot, four slots per workgroup:
// the same arithmetic as edges_walk_kernel's scores.
__global__ __launch_bounds__(256) void score_edges_mfma_kernel(
    const int32_t* __restrict__ cand, const float* __restrict__ unary, const float* __restrict__ z,
    const int32_t* __restrict__ anchors, int S, int K, int R, const uint16_t* __restrict__ pred,
    const uint16_t* __restrict__ succ, int V, float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int l = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (l >= S) return;
  auto clampv = [V](int t) { return t < 0 ? 0 : (t >= V ? V - 1 : t); };
  const size_t row = (size_t)b * S + l;
  int cid = 0, pid = 0;
  float u = 0.f;
  if (lane < K) {
    cid = clampv(cand[row * K + lane]);
    pid = clampv(l == 0 ? anchors[b] : cand[(row - 1) * K + lane]);
    u = unary[row * K + lane];
  }
  const f32x4_t acc = slot_scores_mfma(pred, succ, pid, cid, z + row * R, K, R, lane);
  const int c = lane & 15;
  const float uc = __shfl(u, c, 64);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int p = 4 * (lane >> 4) + e;
    if (p < K && c < K) scores[row * K * K + p * K + c] = uc + acc[e];
  }
}

}  // namespace

size_t topk_static_scratch_floats() { return kStaticScratchFloats; }

hipError_t topk_static_scratch(hipStream_t stream, float** out) {
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // each GPU holds its own copy of the array at its own address: look it up with that
    // device current, once
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

size_t topk_ws_bytes(int N, int V) {
  return (size_t)N * ((V + kGemmTileN - 1) / kGemmTileN) * sizeof(float);
}

hipError_t launch_topk(const float* logits, int N, int V, int K, int32_t* ids, float* vals, void* ws,
                       hipStream_t stream, const int32_t* id_map) {
  if (N <= 0) return hipSuccess;
  const int ntiles = (V + kGemmTileN - 1) / kGemmTileN;
  float* tmax = static_cast<float*>(ws);
  const int waves = (ntiles + kRowmaxTiles - 1) / kRowmaxTiles;
  tile_rowmax_kernel<<<dim3((waves + 3) / 4, N), 256, 0, stream>>>(logits, V, ntiles, tmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_tiles(logits, N, V, K, tmax, ids, vals, stream, id_map);
}

hipError_t launch_tile_maxima(const float* logits, int N, int V, float* tile_max, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const int ntiles = (V + kGemmTileN - 1) / kGemmTileN;
  const int waves = (ntiles + kRowmaxTiles - 1) / kRowmaxTiles;
  tile_rowmax_kernel<<<dim3((waves + 3) / 4, N), 256, 0, stream>>>(logits, V, ntiles, tile_max);
  return hipGetLastError();
}

hipError_t launch_topk_tiles(const float* logits, int N, int V, int K, const float* tile_max,
                             int32_t* ids, float* vals, hipStream_t stream, const int32_t* id_map,
                             const uint32_t* tile_bound) {
  if (N <= 0) return hipSuccess;
  if (tile_bound && K > kTileBoundSlots) return hipErrorInvalidValue;
  const int ntiles = (V + kGemmTileN - 1) / kGemmTileN;
  topk_tiles_kernel<<<N, 256, 0, stream>>>(logits, V, tile_max, ntiles, K, ids, vals, id_map, tile_bound);
  return hipGetLastError();
}

hipError_t launch_score_edges(const int32_t* cand, const float* unary, const float* z,
                              const int32_t* anchors, int B, int S, int K, int R,
                              const uint16_t* pred, const uint16_t* succ, int V, float* scores,
                              hipStream_t stream) {
  if (B <= 0 || S <= 0) return hipSuccess;
  if (K > 32 || R > 128) return hipErrorInvalidValue;
  if (K <= kMfmaMaxK && R >= 4 && R <= kMfmaMaxR && R % 4 == 0) {
    score_edges_mfma_kernel<<<dim3((S + 3) / 4, B), 256, 0, stream>>>(cand, unary, z, anchors, S, K, R, pred, succ, V,
                                                                      scores);
    return hipGetLastError();
  }
  // wavefronts per workgroup: up to 4 slots, within 64 KB of LDS
  const size_t per_wave = (2 * (size_t)K * (R + 1) + R) * sizeof(float);
  const int nw = (int)std::max<size_t>(1, std::min<size_t>(4, (64 << 10) / per_wave));
  const dim3 grid((S + nw - 1) / nw, B);
  const bool vec = R % 8 == 0 && ((reinterpret_cast<uintptr_t>(pred) | reinterpret_cast<uintptr_t>(succ)) & 15) == 0;
  if (vec)
    score_edges_kernel<true><<<grid, 64 * nw, per_wave * nw, stream>>>(cand, unary, z, anchors, S, K, R, pred, succ, V,
                                                                       scores);
  else
    score_edges_kernel<false><<<grid, 64 * nw, per_wave * nw, stream>>>(cand, unary, z, anchors, S, K, R, pred, succ,
                                                                        V, scores);
  return hipGetLastError();
}

bool select_tokens_fits(int S, int K, int R) {
  return S >= 1 && S <= kSelMaxS && K >= 1 && K <= kMfmaMaxK && R >= 4 && R <= kMfmaMaxR && R % 4 == 0;
}

hipError_t launch_edges_walk(const int32_t* cand, const float* unary, const float* z, int R, const int32_t* anchors,
                             int B, int S, int K, const uint16_t* pred, const uint16_t* succ, int V, float* scores,
                             int32_t* tokens, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  if (!select_tokens_fits(S, K, R)) return hipErrorInvalidValue;
  edges_walk_kernel<<<B, kSelWaves * 64, 0, stream>>>(cand, unary, z, R, anchors, S, K, pred, succ, V, scores, tokens);
  return hipGetLastError();
}

// The scanning top-k of N rows, with the selector projection's workgroups first when h is
// given (selproj_fits checked by the caller).
hipError_t launch_topk_scan(const float* logits, int N, int V, int K, int32_t* cand, float* unary,
                            const int32_t* id_map, const uint16_t* h, int H, const uint16_t* proj, int R, float* z,
                            hipStream_t stream) {
  const int ntiles = (V + kGemmTileN - 1) / kGemmTileN;
  if (ntiles > kScanMaxTiles) return hipErrorInvalidValue;
  const int nproj = h ? (N + kProjRows - 1) / kProjRows : 0;
  const dim3 grid(nproj + N);
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0)
    topk_scan_kernel<true><<<grid, 256, 0, stream>>>(logits, V, ntiles, K, cand, unary, id_map, h, N, H, proj, R,
                                                     z);
  else
    topk_scan_kernel<false><<<grid, 256, 0, stream>>>(logits, V, ntiles, K, cand, unary, id_map, h, N, H, proj,
                                                      R, z);
  return hipGetLastError();
}

hipError_t launch_select_tokens(const float* logits, const float* tile_max, int B, int S, int V, int K,
                                const int32_t* id_map, const float* z, int R, const int32_t* anchors,
                                const uint16_t* pred, const uint16_t* succ, int Vcb, int32_t* cand, float* unary,
                                float* scores, int32_t* tokens, hipStream_t stream, const uint32_t* tile_bound) {
  if (B <= 0) return hipSuccess;
  if (!select_tokens_fits(S, K, R)) return hipErrorInvalidValue;
  hipError_t e;
  if (tile_max) {
    e = launch_topk_tiles(logits, B * S, V, K, tile_max, cand, unary, stream, id_map, tile_bound);
  } else {
    // no tile maxima given: each row's workgroup scans its logits and then takes its top-K
    e = launch_topk_scan(logits, B * S, V, K, cand, unary, id_map, nullptr, 0, nullptr, 0, nullptr, stream);
  }
  if (e != hipSuccess) return e;
  return launch_edges_walk(cand, unary, z, R, anchors, B, S, K, pred, succ, Vcb, scores, tokens, stream);
}

bool selproj_fits(int H, int R, const void* h, const void* proj) {
  return H > 0 && H % 128 == 0 && R >= 1 && R <= kProjMaxR &&
         ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(proj)) & 15) == 0;
}

hipError_t launch_selector_project(const uint16_t* h, int N, int H, const uint16_t* proj, int R, float* z,
                                   hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  if (!selproj_fits(H, R, h, proj)) return hipErrorInvalidValue;
  selproj_kernel<<<dim3((N + kProjRows - 1) / kProjRows, (R + 15) / 16), 256, 0, stream>>>(h, N, H, proj, R, z);
  return hipGetLastError();
}

hipError_t launch_select_tokens_projected(const float* logits, int B, int S, int V, int K, const uint16_t* h, int H,
                                          const uint16_t* proj, int R, float* z, const int32_t* anchors,
                                          const uint16_t* pred, const uint16_t* succ, int32_t* cand, float* unary,
                                          float* scores, int32_t* tokens, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  if (!select_tokens_fits(S, K, R) || !selproj_fits(H, R, h, proj)) return hipErrorInvalidValue;
  hipError_t e = launch_topk_scan(logits, B * S, V, K, cand, unary, nullptr, h, H, proj, R, z, stream);
  if (e != hipSuccess) return e;
  return launch_edges_walk(cand, unary, z, R, anchors, B, S, K, pred, succ, V, scores, tokens, stream);
}

hipError_t launch_select_path(const float* scores, const int32_t* cand, int B, int S, int K,
                              int32_t* tokens, hipStream_t stream) {
  if (B <= 0 || S <= 0) return hipSuccess;
  select_path_kernel<<<B, 64, 0, stream>>>(scores, cand, S, K, tokens);
  return hipGetLastError();
}

}  // namespace dfl
