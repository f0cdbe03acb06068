// Bidirectional block attention over a context K/V prefix (dflash2.ts diff: the header
// comment, under which the drafter attends every context row, and `#block`, which hands the
// block's own k/v to the context's attend call with scale 1/sqrt(D)).  Every query row of a
// request attends to its ctx_len[b] context rows (in a sliding-window layer, the ones inside
// its window: see the last paragraph) and all G block rows; query head h reads KV head
// h / (NH/NKV).
//
// Work split: one workgroup per (request b, KV head g, key chunk).  The Q tile is the
// G x NH/NKV query rows that share KV head g (<= 64 rows, 16 per wavefront), so every
// K/V row read from HBM serves all of them.  The chunks split the context rows, and the
// last one also takes the block's own G keys as one more tile (its first); each writes
// (max, sum, unnormalised O) in fp32 and a combine kernel merges the chunks with their
// log-sum-exp weights.  A workgroup keeps R tiles of K/V in flight: R = 3 for long chunks,
// sized so that the whole grid is resident at once (two workgroups per CU; R = 4 and R = 2
// measured slower: more loads in flight only queue longer); R = 1 for short ones, where
// three workgroups per CU and more chunks hide more latency than a deep ring.
//
// Per 64-key tile a wavefront computes S^T = K . Q^T (keys on rows, its 16 queries on
// columns) with v_mfma_f32_16x16x32_bf16, so each lane holds one query's scores and the
// softmax row statistics need only two cross-lane steps; then O^T += V^T . P^T, where
// P^T comes straight from the S^T accumulators and V is staged transposed in LDS with
// the same key order per lane.
//
// A sliding-window layer (MAX DFlash2Qwen3_5 `layer_types`) starts each context chunk at
// block row 0's first visible row and masks, per query lane, the keys before that
// query's own window start; a query with every key of a tile masked keeps its running
// (max, sum, output) unchanged.
#include <algorithm>
#include <climits>

#include "common.hpp"
#include "kernels.hpp"
#include "vmem.hpp"

namespace dfl {

namespace {

constexpr int KT = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDeepMinTiles = 8;  // tiles per chunk below which the shallow ring is used

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kb;
  const uint16_t* vb;
  const uint16_t* K;
  const uint16_t* V;
  const int32_t* ctx_len;
  const int32_t* pos0;  // [B] position of block row 0 (sliding window only)
  float* part_o;   // [B, NKV, nchunks, QR, D]
  float* part_ml;  // [B, NKV, nchunks, QR, 2]
  int ldq, ldkv, Lcap, Lmax, G, NH, NKV, chunk, nchunks, qrows;
  int window;  // 0: every context row; W: row t sees context rows >= pos0 + t - W + 1
  float scale_log2;
};

template <int D, int R>
__global__ __launch_bounds__(256, 2) void attn_chunk_kernel(AttnArgs a) {
  // K tile row stride (bf16): 2 (D / 16 + 1) 16-byte slots, twice an odd number, so a
  // fragment read's 32 lanes (16 rows x 2 adjacent chunks, which gfx950's LDS serves
  // together over 512 bytes) land on 32 distinct slots; D + 8 left one 2-way collision
  constexpr int KS = D + 16;
  constexpr int VS = KT + 4;  // V^T tile row stride (bf16): 34 dwords, conflict-free reads
  constexpr int DT = D / 16;  // output d tiles
  constexpr int DK = D / 32;  // MFMA k steps over D
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];

  const int chunk = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hpg = a.NH / a.NKV;
  const int lg = lane >> 4;  // lane group

  // this wavefront's 16 queries as MFMA B operands (column = query, k = d), loaded first: they
  // do not depend on the request's context length, which the tile loads wait for
  const int qi = wave * 16 + (lane & 15);
  const bool qvalid = qi < a.qrows;
  bf16x8_t qf[DK];
  {
    const int t = qi / hpg;
    const int h = g * hpg + qi % hpg;
    const uint16_t* qrow = a.q + ((size_t)b * a.G + t) * a.ldq + h * D;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (qvalid) v = *reinterpret_cast<const u32x4_t*>(qrow + ks * 32 + lg * 8);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // context key range of this chunk; the last chunk also takes the block's own G keys as
  // one more tile, its first
  const bool has_block = chunk == a.nchunks - 1;
  const int ctx = min(max(a.ctx_len[b], 0), a.Lmax);  // never past the rows the plan covers
  int kbeg = chunk * a.chunk;
  const int kend = min(ctx, kbeg + a.chunk);
  if (a.window > 0) kbeg = max(kbeg, a.pos0[b] - a.window + 1);  // block row 0's first visible row
  const int ctx_tiles = kbeg < kend ? (kend - kbeg + KT - 1) / KT : 0;
  const int ntiles = ctx_tiles + (has_block ? 1 : 0);
  const uint16_t* kctx = a.K + ((size_t)b * a.Lcap * a.NKV + g) * D;
  const uint16_t* vctx = a.V + ((size_t)b * a.Lcap * a.NKV + g) * D;
  const uint16_t* kblk = a.kb + (size_t)b * a.G * a.ldkv + g * D;
  const uint16_t* vblk = a.vb + (size_t)b * a.G * a.ldkv + g * D;
  const uint32_t ctx_stride = static_cast<uint32_t>(a.NKV * D);  // host checks Lcap*NKV*D < 2^31, so byte offsets fit 32 bits

  // sliding window: this lane's query (block row qi / hpg) sees context keys >= kmin; tiles
  // starting at or past kmin_hi (the largest kmin of the workgroup) need no mask
  const bool windowed = a.window > 0;
  const int kmin = windowed ? a.pos0[b] + qi / hpg - a.window + 1 : INT_MIN;
  const int kmin_hi = windowed ? a.pos0[b] + (a.G - 1) - a.window + 1 : INT_MIN;
  float m = -INFINITY, l = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Staging map: thread t owns keys ROWS_PER*kg .. +ROWS_PER-1 of a tile at dims
  // 8*dg .. +7, with dg running fastest, so each load instruction of a wavefront reads
  // whole key rows (DG lanes per row) and each V^T store is one 8-byte pack of ROWS_PER
  // keys per dim and lane.  The next R tiles are in flight in a register ring while
  // one is computed (hand-issued loads, each awaited once by name); loads past a tile's last
  // row repeat that row and loads past the last tile read one line of it, so that every
  // load is unconditional.
  constexpr int DG = D / 8;                  // 16-byte chunks per key row
  static_assert(KT * DG % 256 == 0, "tile must split over 256 threads");
  constexpr int ROWS_PER = (KT * DG) / 256;  // key rows per thread per tile (4 for D=128)
  constexpr int LOADS = 2 * ROWS_PER;        // vector loads per thread per tile
  static_assert(R * LOADS <= 63, "ring deeper than vmcnt can count");
  const int dg = tid % DG;
  const int kg = tid / DG;
  u32x4_t kreg[R][ROWS_PER], vreg[R][ROWS_PER];
  // tile t of this workgroup (uniform); rows past a tile's end repeat its last row.  Loads
  // for tiles past the last (the ring's tail) all read the last tile's first 16 bytes, one
  // line per instruction, so the ring costs no second read of a tile.
  auto tile_load = [&](u32x4_t (&kr)[ROWS_PER], u32x4_t (&vr)[ROWS_PER], int t) {
    const bool live = t < ntiles;
    t = min(t, ntiles - 1);
    const bool blk = has_block && t == 0;
    const uint16_t* kp = blk ? kblk : kctx;
    const uint16_t* vp = blk ? vblk : vctx;
    const uint32_t stride = blk ? static_cast<uint32_t>(a.ldkv) * 2u : ctx_stride * 2u;  // bytes
    const int r0 = blk ? 0 : kbeg + (t - (has_block ? 1 : 0)) * KT;
    const int rlast = blk ? a.G - 1 : kend - 1;
#pragma unroll
    for (int i = 0; i < ROWS_PER; ++i) {
      const uint32_t off = live ? static_cast<uint32_t>(min(r0 + kg * ROWS_PER + i, rlast)) * stride + dg * 16
                                : static_cast<uint32_t>(r0) * stride;
      kr[i] = vm_load16_nt(kp, off);
      vr[i] = vm_load16_nt(vp, off);
    }
  };
  // every load but the newest n tiles' is in
  auto tile_wait = [&](u32x4_t (&kr)[ROWS_PER], u32x4_t (&vr)[ROWS_PER]) {
#pragma unroll
    for (int i = 0; i < ROWS_PER; ++i) {
      vm_wait<(R - 1) * LOADS>(kr[i]);
      vm_wait<(R - 1) * LOADS>(vr[i]);
    }
  };
  // V^T row r (dim r) holds the tile's 64 keys as 32 dwords with the key pairs rotated by
  // 2 * (r / 16) dwords: the 16 lanes of one store instruction write the same key slot of
  // dims 8 apart, which without the rotation fall on two bank pairs (rows 8 apart are 272
  // dwords apart); the fragment reads of rows 16 dt .. 16 dt + 15 share one rotation, so they
  // keep their conflict-free row stride.
  auto vt_dw = [](int r, int key_dw) { return r * (VS / 2) + ((key_dw + 2 * (r >> 4)) & 31); };
  auto tile_store = [&](const u32x4_t (&kr)[ROWS_PER], const u32x4_t (&vr)[ROWS_PER]) {
#pragma unroll
    for (int i = 0; i < ROWS_PER; ++i)
      *reinterpret_cast<u32x4_t*>(&Ks[(kg * ROWS_PER + i) * KS + dg * 8]) = kr[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h[ROWS_PER];
#pragma unroll
      for (int i = 0; i < ROWS_PER; ++i) h[i] = (vr[i][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
      uint16_t* dst = &Vt[2 * vt_dw(dg * 8 + e, kg * ROWS_PER / 2)];
      if constexpr (ROWS_PER == 4) {
        *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      } else {
#pragma unroll
        for (int i = 0; i < ROWS_PER; i += 2) *reinterpret_cast<uint32_t*>(dst + i) = h[i] | (h[i + 1] << 16);
      }
    }
  };
  auto tile_compute = [&](int j0, int nvalid, bool window_tile) {
    // S^T tiles: s[kt] holds keys kt*16 + 4*lg + e for query (lane & 15)
    f32x4_t s[KT / 16];
#pragma unroll
    for (int kt = 0; kt < KT / 16; ++kt) {
      s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(&Ks[(kt * 16 + (lane & 15)) * KS + ks * 32 + lg * 8]);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[kt], 0, 0, 0);
      }
    }
    // online softmax in the log2 domain: p = 2^(s * scale_log2 - m); keys past a ragged
    // tile's end get s = -inf (uniform branch, taken only on a chunk's last tile)
    if (nvalid < KT) {
#pragma unroll
      for (int kt = 0; kt < KT / 16; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kt * 16 + lg * 4 + e >= nvalid) s[kt][e] = -INFINITY;
    }
    if (window_tile && j0 < kmin_hi) {  // uniform: only tiles that reach below some query's window start
#pragma unroll
      for (int kt = 0; kt < KT / 16; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + kt * 16 + lg * 4 + e < kmin) s[kt][e] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT / 16; ++kt)
      tmax = fmaxf(tmax, fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3])));
    tmax = bfly16(tmax, OpMax{});
    tmax = bfly32(tmax, OpMax{});
    const float mnew = fmaxf(m, tmax * a.scale_log2);
    // a query whose keys so far are all masked (sliding window) keeps m = -inf, l = 0, o = 0:
    // msafe keeps the exponents finite so that every weight below is exactly 0
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    // v_exp_f32 directly: exponents here are <= 0, and results below fp32's normal range
    // (weights under 2^-126) flush to zero
    const float alpha = __builtin_amdgcn_exp2f(m - msafe);  // m = -inf on the first tile: 0
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT / 16; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][e], a.scale_log2, -msafe));
        s[kt][e] = p;
        psum += p;
      }
    psum = bfly16(psum, OpAdd{});
    psum = bfly32(psum, OpAdd{});
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] *= alpha;

    // O^T += V^T . P^T over two 32-key steps.  Lane slots 0..3 are keys 32*ks + 4*lg + e,
    // slots 4..7 keys 32*ks + 16 + 4*lg + e: the same order for both operands.
#pragma unroll
    for (int ks = 0; ks < KT / 32; ++ks) {
      u32x4_t pw;
      pw[0] = pack_bf16x2(s[2 * ks][0], s[2 * ks][1]);
      pw[1] = pack_bf16x2(s[2 * ks][2], s[2 * ks][3]);
      pw[2] = pack_bf16x2(s[2 * ks + 1][0], s[2 * ks + 1][1]);
      pw[3] = pack_bf16x2(s[2 * ks + 1][2], s[2 * ks + 1][3]);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int r = dt * 16 + (lane & 15);
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(&Vt[2 * vt_dw(r, ks * 16 + lg * 2)]);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(&Vt[2 * vt_dw(r, ks * 16 + 8 + lg * 2)]);
        const u32x4_t vw = {lo[0], lo[1], hi[0], hi[1]};
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vw), pf,
                                                        o[dt], 0, 0, 0);
      }
    }
  };
  if (ntiles > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) tile_load(kreg[r], vreg[r], r);
    for (int t0 = 0; t0 < ntiles; t0 += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int t = t0 + r;  // uniform over the workgroup
        tile_wait(kreg[r], vreg[r]);
        if (t < ntiles) tile_store(kreg[r], vreg[r]);
        tile_load(kreg[r], vreg[r], t + R);
        __syncthreads();
        if (t < ntiles) {
          const bool ctx_tile = !(has_block && t == 0);  // else the block's own keys, all visible
          const int j0 = kbeg + (t - (has_block ? 1 : 0)) * KT;
          tile_compute(j0, ctx_tile ? min(KT, kend - j0) : a.G, ctx_tile);
        }
        __syncthreads();
      }
    }
    // the ring's last loads (clamped re-reads) are awaited before their registers go
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < ROWS_PER; ++i) {
        vm_wait<0>(kreg[r][i]);
        vm_wait<0>(vreg[r][i]);
      }
  }

  if (!qvalid) return;
  const size_t slot = (((size_t)b * a.NKV + g) * a.nchunks + chunk) * a.qrows + qi;
  if (lg == 0) {
    a.part_ml[slot * 2 + 0] = m;
    a.part_ml[slot * 2 + 1] = l;
  }
  float* po = a.part_o + slot * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4_t*>(po + dt * 16 + lg * 4) = o[dt];
}

// Merge the chunks of one query row: weights 2^(m_c - max m) and the summed denominators.
// Lane c holds chunk c's statistics (the plan keeps nchunks <= 64); the partial outputs of
// up to kCombineBatch chunks are loaded before the statistics are reduced, so one round trip
// to memory covers a typical row.  An empty chunk has m = -inf, so its weight is exactly 0
// and its (zero) partial output adds nothing.  Chunks are summed in order.
constexpr int kCombineBatch = 8;

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, uint16_t* out, int ldo) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // over NKV * qrows of request b
  const int b = blockIdx.y;
  if (row >= a.NKV * a.qrows) return;
  const int qi = row % a.qrows;
  const int g = row / a.qrows;
  const size_t base = ((size_t)b * a.NKV + g) * a.nchunks;
  constexpr int PL = D / 64;  // values per lane
  const float* po = a.part_o + (base * a.qrows + qi) * D + lane;
  const size_t cstride = (size_t)a.qrows * D;  // floats from one chunk's row to the next
  const int n0 = min(a.nchunks, kCombineBatch);
  float v[kCombineBatch][PL];
#pragma unroll
  for (int c = 0; c < kCombineBatch; ++c)
#pragma unroll
    for (int i = 0; i < PL; ++i) v[c][i] = c < n0 ? po[c * cstride + 64 * i] : 0.f;
  float mc = -INFINITY, lc = 0.f;
  if (lane < a.nchunks) {
    const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(a.part_ml + ((base + lane) * a.qrows + qi) * 2);
    mc = ml[0];
    lc = ml[1];
  }
  const float mx = wave_max(mc);
  const float wl = mc == -INFINITY ? 0.f : exp2f(mc - mx);
  const float den = wave_sum(wl * lc);
  float acc[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) acc[i] = 0.f;
#pragma unroll
  for (int c = 0; c < kCombineBatch; ++c) {
    if (c >= n0) break;
    const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), c));
#pragma unroll
    for (int i = 0; i < PL; ++i) acc[i] += w * v[c][i];
  }
  for (int c = n0; c < a.nchunks; ++c) {
    const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), c));
#pragma unroll
    for (int i = 0; i < PL; ++i) acc[i] += w * po[c * cstride + 64 * i];
  }
  const float inv = 1.f / den;
  const int hpg = a.NH / a.NKV;
  const int t = qi / hpg;
  const int h = g * hpg + qi % hpg;
  uint16_t* orow = out + ((size_t)b * a.G + t) * ldo + h * D;
#pragma unroll
  for (int i = 0; i < PL; ++i) orow[lane + 64 * i] = f32_to_bf16(acc[i] * inv);
}

}  // namespace

AttnPlan plan_attention(int B, int G, int NH, int NKV, int D, int Lmax) {
  AttnPlan pl;
  pl.qrows = G * (NH / NKV);
  // Deep ring: one resident round of 256 CUs x 2 workgroups split over the (b, g) pairs.
  // When that leaves fewer than kDeepMinTiles tiles per chunk, the ring would be mostly
  // fill, so the shallow ring takes chunks of 256 keys (or what fills 2048 workgroups).
  // Either way nchunks <= 64, one chunk per lane in the combine.
  const int pairs = B * NKV;
  auto chunk_for = [&](int want) {
    int c = (Lmax + want - 1) / want;
    c = std::max(c, (Lmax + 63) / 64);
    c = ((c + KT - 1) / KT) * KT;
    return std::max(c, 256);
  };
  pl.chunk = chunk_for(std::max(1, 512 / pairs));
  pl.stages = 3;
  if (pl.chunk / KT < kDeepMinTiles) {
    pl.chunk = chunk_for(std::max(1, 2048 / pairs));
    pl.stages = 1;
  }
  const int ctx_chunks = Lmax > 0 ? (Lmax + pl.chunk - 1) / pl.chunk : 0;
  pl.nchunks = std::max(ctx_chunks, 1);
  const size_t slots = (size_t)B * NKV * pl.nchunks * pl.qrows;
  pl.ws_bytes = slots * D * sizeof(float) + slots * 2 * sizeof(float);
  return pl;
}

hipError_t launch_attention(const AttnPlan& pl, const uint16_t* q, int ldq, const uint16_t* kb,
                            const uint16_t* vb, int ldkv, const uint16_t* K, const uint16_t* V,
                            int Lcap, const int32_t* ctx_len, const int32_t* pos0, int window, int B,
                            int G, int NH, int NKV, int D, int Lmax, uint16_t* out, int ldo, void* ws,
                            hipStream_t stream) {
  AttnArgs a;
  a.q = q;
  a.kb = kb;
  a.vb = vb;
  a.K = K;
  a.V = V;
  a.ctx_len = ctx_len;
  a.pos0 = pos0;
  a.window = window > 0 && pos0 ? window : 0;
  const size_t slots = (size_t)B * NKV * pl.nchunks * pl.qrows;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = a.part_o + slots * D;
  a.ldq = ldq;
  a.ldkv = ldkv;
  a.Lcap = Lcap;
  a.Lmax = Lmax;
  a.G = G;
  a.NH = NH;
  a.NKV = NKV;
  a.chunk = pl.chunk;
  a.nchunks = pl.nchunks;
  a.qrows = pl.qrows;
  a.scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
  if (static_cast<size_t>(Lcap) * NKV * D >= (size_t(1) << 31)) return hipErrorInvalidValue;
  dim3 grid(pl.nchunks, NKV, B);
  const int rows = NKV * pl.qrows;  // per request
  dim3 cgrid((rows + 3) / 4, B);
  if (D == 128) {
    if (pl.stages == 3)
      attn_chunk_kernel<128, 3><<<grid, 256, 0, stream>>>(a);
    else
      attn_chunk_kernel<128, 1><<<grid, 256, 0, stream>>>(a);
    attn_combine_kernel<128><<<cgrid, 256, 0, stream>>>(a, out, ldo);
  } else {
    if (pl.stages == 3)
      attn_chunk_kernel<64, 3><<<grid, 256, 0, stream>>>(a);
    else
      attn_chunk_kernel<64, 1><<<grid, 256, 0, stream>>>(a);
    attn_combine_kernel<64><<<cgrid, 256, 0, stream>>>(a, out, ldo);
  }
  return hipGetLastError();
}

}  // namespace dfl
