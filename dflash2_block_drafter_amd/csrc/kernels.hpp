// Host-side launchers of the gfx950 kernels.  Each enqueues on `stream`, assumes its
// arguments were validated by the C ABI layer, and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfl {

enum Epilogue { EPI_BF16 = 0, EPI_F32 = 1, EPI_SILU_MUL = 2 };

// S fp32 planes of rows at row stride ld, plane stride `plane` elements: the split-K
// partials of a GEMM left for the consuming kernel to sum in plane order (the order of the
// split-K reduce), or S = 1 plane of plain fp32 values.  S = 0 marks an absent source.
struct Planes {
  const float* p = nullptr;
  int S = 0;
  int ld = 0;
  size_t plane = 0;
};

struct GemmPlan {
  int bm = 0, bn = 0;
  int splits = 1;
  int k_per_split = 0;
  size_t partial_bytes = 0;  // split-K scratch (fp32 [splits, M, N])
  int stream_waves = 0;      // > 0: the weight-streaming kernel (M <= 128), waves per workgroup
  // 256 x 256 tiles whose last round of workgroups would be less than half full: weight rows
  // from tail_n on run as a second launch with tail_splits K splits (0: no tail launch)
  int tail_n = 0, tail_splits = 1, tail_k_per_split = 0;
};

// tile_max: the caller will ask launch_gemm for tile maxima (one split, 256-column workgroups).
GemmPlan plan_gemm(int M, int N, int K, bool tile_max = false);

// A projection weight [N, K]: bf16 w (row-major, or tile-contiguous when tiled), or 4-bit
// affine q (row-major packed words [N, K/8] with scales and biases [N, K/64] bf16, or the
// tile-contiguous blocks of launch_tile_q4 when tiled).
struct WeightRef {
  const uint16_t* w = nullptr;
  const uint32_t* q = nullptr;
  const uint16_t* scales = nullptr;
  const uint16_t* biases = nullptr;
  bool tiled = false;
};
hipError_t launch_gemm(const GemmPlan& pl, const uint16_t* A, int lda, const WeightRef& W, int M, int N, int K,
                       int epi, void* out0, int ld0, void* out1, int ld1, int nsplit, float* partial,
                       hipStream_t stream, float* tile_max = nullptr, uint32_t* tile_bound = nullptr,
                       bool a_tiled = false);
hipError_t launch_gemm_partials(const GemmPlan& pl, const uint16_t* A, int lda, const WeightRef& W, int M, int N,
                                int K, float* partial, hipStream_t stream);
// Tile-contiguous 4-bit weights: per (256-row tile, 64-wide K step) four 64-row groups of
// 576 words; group g holds 64 lanes x 8 packed words (lane l: rows 16 j + l % 16 of the
// group, j = 0..3, each for K offsets 8 (l / 16) and 32 + 8 (l / 16), word j * 2 + half),
// then [16][4] words scale | bias << 16 (row 16 j + r at r * 4 + j).  q4_tiled_words gives
// the size in 32-bit words; rows as for launch_tile_weights.
size_t q4_tiled_words(int N, int K);
hipError_t launch_tile_q4(const uint32_t* q, const uint16_t* scales, const uint16_t* biases, int N, int K,
                          uint32_t* dst, hipStream_t stream, const int32_t* rows = nullptr);
// y = A . W^T.  A [M, K] (lda).  W: row-major [N, K], or tile-contiguous (w_tiled) as
// written by launch_tile_weights.  EPI_BF16: out0 bf16 (ld0).  EPI_F32: columns < nsplit
// to out0 (ld0), the rest to out1 (ld1) when out1 != nullptr.  EPI_SILU_MUL: W rows
// interleaved per 16 as [gate|up]; out0 bf16 [M, N/2] = silu(gate) * up.
// tile_max (EPI_F32 with an unsplit plan only): also write the row maxima of every
// kGemmTileN-column tile of out0's columns, [M, ceil(nsplit / kGemmTileN)] (nsplit = N
// without out1; with out1, nsplit must be a multiple of kGemmTileN).
// tile_bound (with tile_max; [M, kTileBoundSlots] uint32, zero before the launch): slot s of
// row m collects, in float_order's map, the largest maximum of row m over the tiles t with
// t % kTileBoundSlots == s.  Once every slot of a row is filled, their least value is reached
// by kTileBoundSlots logits of distinct tiles, so it is at most the row's kTileBoundSlots-th
// largest logit; a tile whose row maximum is below it (as floats) cannot hold any of the
// row's top kTileBoundSlots, and its values of that row are not stored.  A top-K with K <=
// kTileBoundSlots stays exact when it reads only tiles whose maximum reaches that bound.
// a_tiled: A is not row-major but in fragment order as written by launch_tile_rows (lda is
// then unused); only plans for which gemm_takes_tiled_a holds accept it.
constexpr int kGemmTileN = 256;
constexpr int kTileBoundSlots = 16;
hipError_t launch_gemm(const GemmPlan& pl, const uint16_t* A, int lda, const uint16_t* W, bool w_tiled,
                       int M, int N, int K, int epi, void* out0, int ld0, void* out1, int ld1,
                       int nsplit, float* partial, hipStream_t stream, float* tile_max = nullptr,
                       uint32_t* tile_bound = nullptr, bool a_tiled = false);
// The plan runs the 256 x 256 kernel, which can read A in fragment order.
inline bool gemm_takes_tiled_a(const GemmPlan& pl, bool q4) { return pl.bm == 256 && pl.stream_waves == 0 && !q4; }
// Fragment-order copy of row-major activations A [M, K] (lda; K % 32 == 0, lda % 8 == 0):
// [ceil(M/16)][K/32] fragments of 16 rows x 32 K, each 64 lanes x 8 bf16 where lane l holds
// row l % 16 and K offset 8 * (l / 16); rows past M repeat row M - 1.  tiled_rows_elems gives
// the destination size in bf16 elements.
size_t tiled_rows_elems(int M, int K);
hipError_t launch_tile_rows(const uint16_t* A, int lda, int M, int K, uint16_t* dst, hipStream_t stream);
// y = A . W^T left as fp32 planes for the consumer: pl.splits planes [M, N] at plane stride
// M*N in `partial` (one plane, the plain result, when the plan does not split K).
hipError_t launch_gemm_partials(const GemmPlan& pl, const uint16_t* A, int lda, const uint16_t* W,
                                bool w_tiled, int M, int N, int K, float* partial, hipStream_t stream);
inline Planes gemm_planes(const GemmPlan& pl, const float* partial, int M, int N) {
  Planes p;
  p.p = partial;
  p.S = pl.splits;
  p.ld = N;
  p.plane = (size_t)M * N;
  return p;
}
// Sum of S fp32 planes [M, N] (src.ld = N) into one plane `out` [M, N], added in plane order.
hipError_t launch_planes_sum(const Planes& src, int M, int N, float* out, hipStream_t stream);
// The same sum rounded to bf16 (what a split-K projection with bf16 output stores).
hipError_t launch_planes_sum_bf16(const Planes& src, int M, int N, uint16_t* out, hipStream_t stream);

// Tile-contiguous copy of a row-major [N, K] weight: one block per (256-row tile, 64-wide K
// step), [ceil(N/256)][K/64][block], rows past N zero.  Inside a block the order is the
// matrix-core operand order: 32 fragments of 16 rows x 32 K (row group outer, K half inner),
// each 64 lanes x 8 bf16 where lane l holds row l % 16 and K offset 8 * (l / 16).
// tiled_weight_elems gives the destination size in bf16 elements.  rows (device, optional):
// destination row n copies source row rows[n] (a gathered subset).
size_t tiled_weight_elems(int N, int K);
hipError_t launch_tile_weights(const uint16_t* src, int N, int K, uint16_t* dst, hipStream_t stream,
                               const int32_t* rows = nullptr);

// RMSNorm of `rows` rows.  Input row r is row in_row(r) = (r / out_per_grp) * in_per_grp +
// skip + r % out_per_grp, so the final norm can drop the anchor row of every block.
hipError_t launch_rms_norm(const uint16_t* x, int ldx, int rows, int H, const uint16_t* gamma,
                           float eps, uint16_t* y, int ldy, int out_per_grp, int in_per_grp,
                           int skip, hipStream_t stream);

// Per-head RMSNorm + neox RoPE in place on `heads` heads of each row; heads below `split`
// use gamma, the rest gamma2.  Row r sits at position pos0[r / rows_per_req] +
// r % rows_per_req + pos_offset.
hipError_t launch_head_norm_rope(uint16_t* x, int ldx, int rows, int heads, int split, int D,
                                 const uint16_t* gamma, const uint16_t* gamma2, float eps,
                                 float theta, const int32_t* pos0, int rows_per_req,
                                 int pos_offset, hipStream_t stream);

// The same from fp32 planes (the q|k|v projection's split-K partials): row r of dst (ldd)
// gets bf16(sum) of every column, then RMSNorm + RoPE on the first `rope_heads` heads;
// the remaining `tail_cols` columns (the v heads) are only rounded.
hipError_t launch_head_norm_rope_planes(const Planes& src, uint16_t* dst, int ldd, int rows, int rope_heads,
                                        int split, int D, int tail_cols, const uint16_t* gamma,
                                        const uint16_t* gamma2, float eps, float theta, const int32_t* pos0,
                                        int rows_per_req, int pos_offset, hipStream_t stream);

// Context K/V store: kv [B*L, 2*NKV*D] (k then v) -> K/V caches [B, Lcap, NKV, D] at rows
// row_offset + j with k_norm and RoPE at position row_offset + j.
hipError_t launch_context_kv_store(const uint16_t* kv, int B, int L, int NKV, int D,
                                   const uint16_t* k_norm, float eps, float theta,
                                   int row_offset, int Lcap, uint16_t* K, uint16_t* V,
                                   hipStream_t stream);

// Ragged store: kv [rows, 2*NKV*D] packs the new rows of B requests back to back; device
// offsets [B+1] (offsets[0] = 0, nondecreasing, offsets[B] = rows) and starts [B]: packed row
// r of request b goes to cache row starts[b] + r - offsets[b] at that position.
hipError_t launch_context_kv_store_ragged(const uint16_t* kv, int rows, int B, int NKV, int D, const uint16_t* k_norm,
                                          float eps, float theta, const int32_t* offsets, const int32_t* starts,
                                          int Lcap, uint16_t* K, uint16_t* V, hipStream_t stream);

// Grouped dynamic conv of bf16 rows y [T, H].  coef: the side's fp32 deltas, tap 0 of group
// g at column g and tap 1 at column ng + g of each row, summed over coef.S planes.
//
// Side-1 conv + residual, then RMSNorm of the new residual row: x_out = residual +
// conv1(y); n_out = RMSNorm(x_out; gamma).  One workgroup per row; x_out may alias
// residual; H <= 8192.
// skip_anchor: n_out holds only rows t % G != 0, packed (row (t / G) * (G - 1) + t % G - 1),
// as the head reads them after the last layer; with skip_anchor, clear_bound (optional)
// receives kTileBoundSlots zeros per packed row (the head's tile_bound slots).
hipError_t launch_conv_residual_norm(const uint16_t* y, const Planes& coef, const uint16_t* base, int T, int H,
                                     int G, int grp, const uint16_t* residual, uint16_t* x_out,
                                     const uint16_t* gamma, float eps, uint16_t* n_out, hipStream_t stream,
                                     bool skip_anchor = false, uint32_t* clear_bound = nullptr);

// The same with y given as the fp32 split-K planes of its projection ([y.S][T][H], plane
// stride y.plane >= T * H): each row's sum over the planes, in plane order, is rounded to
// bf16 as the split-K reduce would store it, so the result equals reduce + the call above.
// H <= kCrnPlanesMaxH.
constexpr int kCrnPlanesMaxH = 5120;
hipError_t launch_conv_residual_norm_planes(const Planes& y, const Planes& coef, const uint16_t* base, int T, int H,
                                            int G, int grp, const uint16_t* residual, uint16_t* x_out,
                                            const uint16_t* gamma, float eps, uint16_t* n_out, hipStream_t stream,
                                            bool skip_anchor = false, uint32_t* clear_bound = nullptr);

// Grouped dynamic conv; side selects base[side]; residual may be null.  coef_next (side 0
// only; coef then holds both sides, side 1 at column 2 * ng): also write side 1's summed
// coefficients as one fp32 plane [T, 2 * ng] for the finish.
hipError_t launch_conv(const uint16_t* y, const Planes& coef, const uint16_t* base, int side, int T, int H, int G,
                       int grp, const uint16_t* residual, uint16_t* out, hipStream_t stream,
                       float* coef_next = nullptr);

struct AttnPlan {
  int chunk = 0;     // context rows per chunk (multiple of 64)
  int nchunks = 0;   // chunks (<= 64); the last one also takes the block's own keys
  int stages = 4;    // K/V tiles in flight per workgroup (4 or 1)
  int qrows = 0;     // G * NH / NKV
  size_t ws_bytes = 0;
};
AttnPlan plan_attention(int B, int G, int NH, int NKV, int D, int Lmax);
// window > 0: block row t of request b (position pos0[b] + t) sees context rows
// j >= pos0[b] + t - window + 1 only; the block's own rows are always seen.
hipError_t launch_attention(const AttnPlan& pl, const uint16_t* q, int ldq, const uint16_t* kb,
                            const uint16_t* vb, int ldkv, const uint16_t* K, const uint16_t* V,
                            int Lcap, const int32_t* ctx_len, const int32_t* pos0, int window, int B,
                            int G, int NH, int NKV, int D, int Lmax, uint16_t* out, int ldo, void* ws,
                            hipStream_t stream);

// Top-K of each row guided by its tile maxima ([N, ceil(V / kGemmTileN)], as launch_gemm's
// tile_max writes them): only tiles whose maximum reaches the K-th largest tile maximum
// are read.
// id_map (device, optional): the reported id of column c is id_map[c] (a draft vocabulary).
// tile_bound (optional, K <= kTileBoundSlots): the slots launch_gemm filled; when all of a
// row's are filled, only tiles whose maximum also reaches their least value are read (the
// logits of the others may never have been stored).
hipError_t launch_topk_tiles(const float* logits, int N, int V, int K, const float* tile_max,
                             int32_t* ids, float* vals, hipStream_t stream, const int32_t* id_map = nullptr,
                             const uint32_t* tile_bound = nullptr);
// Row maxima of every kGemmTileN-column tile of fp32 logits [N, V] -> [N, ceil(V / kGemmTileN)].
hipError_t launch_tile_maxima(const float* logits, int N, int V, float* tile_max, hipStream_t stream);
// Exact top-K of each fp32 row (value descending, id ascending): tile maxima into ws
// (topk_ws_bytes), then launch_topk_tiles.
size_t topk_ws_bytes(int N, int V);
hipError_t launch_topk(const float* logits, int N, int V, int K, int32_t* ids, float* vals, void* ws,
                       hipStream_t stream, const int32_t* id_map = nullptr);

// The library's static tile-maxima scratch (a file-scope device array of
// topk_static_scratch_floats() floats): its device address on the GPU of `stream` (the
// current device for the null stream), looked up on first use per device.
size_t topk_static_scratch_floats();
hipError_t topk_static_scratch(hipStream_t stream, float** out);

hipError_t launch_score_edges(const int32_t* cand, const float* unary, const float* z,
                              const int32_t* anchors, int B, int S, int K, int R,
                              const uint16_t* pred, const uint16_t* succ, int V, float* scores,
                              hipStream_t stream);
// Top-K from tile maxima (topk_tiles_kernel), then score_edges and the greedy walk of B
// requests of S slots in one more launch (one workgroup per request, the scores on the matrix
// cores): logits [B*S, V] with tile maxima [B*S, ceil(V/256)], z [B*S, R]; cand/unary
// [B*S, K] and tokens [B, S] out, scores [B*S, K, K] out when not NULL.  Requires
// select_tokens_fits(S, K, R): S <= 64, K <= 16, R a multiple of 4 in [4, 64].  tile_bound:
// as for launch_topk_tiles.
bool select_tokens_fits(int S, int K, int R);
// launch_select_tokens without tile maxima (tile_max = nullptr): each row's workgroup scans
// its logits, keeping the row's tile maxima in LDS, so ceil(V / 256) <= kSelectScanMaxTiles.
constexpr int kSelectScanMaxTiles = 4096;
hipError_t launch_select_tokens(const float* logits, const float* tile_max, int B, int S, int V, int K,
                                const int32_t* id_map, const float* z, int R, const int32_t* anchors,
                                const uint16_t* pred, const uint16_t* succ, int Vcb, int32_t* cand, float* unary,
                                float* scores, int32_t* tokens, hipStream_t stream,
                                const uint32_t* tile_bound = nullptr);
hipError_t launch_select_path(const float* scores, const int32_t* cand, int B, int S, int K,
                              int32_t* tokens, hipStream_t stream);
// Selector projection z = h . proj^T, fp32 [N, R], 16 rows per workgroup on the matrix cores
// (K in quarters per wavefront, summed in a fixed order): h [N, H] and proj [R, H] bf16,
// 16-byte aligned, H a multiple of 128, R <= 64 (selproj_fits).
bool selproj_fits(int H, int R, const void* h, const void* proj);
hipError_t launch_selector_project(const uint16_t* h, int N, int H, const uint16_t* proj, int R, float* z,
                                   hipStream_t stream);
// launch_select_tokens without tile maxima, with z computed by the same kernel as
// launch_selector_project in extra workgroups of the scanning top-k's launch (z is written,
// then read by the edge scores).
hipError_t launch_select_tokens_projected(const float* logits, int B, int S, int V, int K, const uint16_t* h, int H,
                                          const uint16_t* proj, int R, float* z, const int32_t* anchors,
                                          const uint16_t* pred, const uint16_t* succ, int32_t* cand, float* unary,
                                          float* scores, int32_t* tokens, hipStream_t stream);


}  // namespace dfl
