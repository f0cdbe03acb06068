/*
 * dflash2.h - C ABI of the DFlash2 block-drafter hot path for MI355X (gfx950).
 *
 * Sources cited by page title and section:
 *   [P2] @mlx-bun/inference diff, dflash2.ts (header comment, `#rms`, `#coefficients`,
 *        `#conv`, `#rope`, `projectContext`, `#contextKV`, `#block`, `#select`, `dispose`).
 *   [P3] MAX Python API, max.pipelines.architectures.dflash2_qwen3_5
 *        (`DFlash2GroupedConv.prepare/finish`, `DFlash2CandidateSelector.score_edges/
 *        select_path`, `DFlash2Qwen3_5.compute_candidates/forward_block/materialize`,
 *        `supports_zero_draft_rows`).
 *   [P1] codehub.bot listing of mirror-sd functions (neox RoPE, per-head RMSNorm docstrings).
 *
 * Conventions for every call:
 *   - Tensor pointers are HIP device pointers into row-major, contiguous memory unless a
 *     leading dimension is passed.  bf16 tensors are raw bit patterns (uint16_t).
 *   - Inputs are borrowed until the enqueued work completes; outputs are caller-owned.
 *   - Every call only enqueues work on `stream` and never synchronises it, except
 *     dfl_drafter_load (one synchronisation after repacking) and dfl_read_kernel_time.
 *   - Arguments are validated in full before anything is enqueued.  On error nothing
 *     is written, a negative status is returned and dfl_last_error() describes it; the
 *     drafter handle stays usable.  No C++ exception crosses this boundary.
 *   - Workspaces (`ws`, `ws_bytes`) are caller-allocated device memory, 256-byte
 *     aligned, sized by the matching *_workspace_bytes call.  Concurrent calls need
 *     separate workspaces.
 *   - Floating-point inputs must be finite; results for NaN/Inf inputs are undefined.
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t dfl_bf16; /* bf16 bit pattern, round-to-nearest-even by the producer */
typedef struct dfl_drafter dfl_drafter; /* opaque; immutable after load except timing state */

enum dfl_status {
  DFL_OK = 0,
  DFL_E_INVALID = -1,     /* null pointer, non-positive size, misaligned workspace */
  DFL_E_SHAPE = -2,       /* sizes inconsistent with each other or with the config */
  DFL_E_UNSUPPORTED = -3, /* conv taps != 2, G < 2 or G > block_size, repeated tap ids,
                             top_k > 32 or > vocab, head_dim not 64/128, ... */
  DFL_E_WORKSPACE = -4,   /* workspace smaller than the *_workspace_bytes figure */
  DFL_E_NOMEM = -5,       /* device allocation failed (load only) */
  DFL_E_DEVICE = -6       /* a HIP call failed; the message carries hipGetErrorString */
};

/* Drafter dimensions ([P2] `Dflash2Config`/`readConfig`; [P3] `DFlash2Qwen3_5`). */
typedef struct {
  int32_t hidden;       /* H */
  int32_t layers;
  int32_t heads;        /* NH */
  int32_t kv_heads;     /* NKV, divides NH */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t intermediate; /* F, multiple of 16 */
  int32_t n_taps;       /* target taps concatenated into fc */
  int32_t block_size;   /* G max: anchor + mask rows */
  int32_t conv_taps;    /* must be 2 ([P2] `readConfig` accepts only two taps) */
  int32_t conv_group;   /* channels per dynamic coefficient; multiple of 8, divides H */
  int32_t top_k;        /* K, 1..32 */
  int32_t rank;         /* R, multiple of 16, <= 128 */
  int32_t vocab;        /* V */
  float rms_eps;
  float rope_theta;
  const int32_t* tap_layer_ids; /* host array of n_taps target layer ids; must be distinct
                                   ([P3] `build_module` rejects repeated tap ids); may be NULL */
  int32_t sliding_window;       /* 0: every layer attends to all of its context; W > 0: a sliding
                                   layer's block row at position p sees context rows >= p - W + 1
                                   ([P3] `DFlash2Qwen3_5` `layer_types`, `construct_kv_params`) */
  const int32_t* sliding_layers; /* host array of `layers` flags (nonzero: sliding), read at load;
                                   NULL: every layer slides when sliding_window > 0 */
} dfl_config;

/* One layer's tensors under the checkpoint layout ([P2] `Layer`: weights are [out, in]). */
typedef struct {
  const dfl_bf16* input_norm;  /* [H] */
  const dfl_bf16* post_norm;   /* [H] */
  const dfl_bf16* q_proj;      /* [NH*D, H] */
  const dfl_bf16* k_proj;      /* [NKV*D, H] */
  const dfl_bf16* v_proj;      /* [NKV*D, H] */
  const dfl_bf16* o_proj;      /* [H, NH*D] */
  const dfl_bf16* q_norm;      /* [D] */
  const dfl_bf16* k_norm;      /* [D] */
  const dfl_bf16* gate_proj;   /* [F, H] */
  const dfl_bf16* up_proj;     /* [F, H] */
  const dfl_bf16* down_proj;   /* [H, F] */
  const dfl_bf16* attn_base;   /* [2 side, 2 tap, H] */
  const dfl_bf16* attn_kproj;  /* [2*2*H/grp, H], output columns [side][tap][group] */
  const dfl_bf16* mlp_base;    /* [2, 2, H] */
  const dfl_bf16* mlp_kproj;   /* [2*2*H/grp, H] */
} dfl_layer_weights;

/* A 4-bit affine projection [N, K] ([P2] `quantizedWeight`: affine mode, groups of 64 along
 * K): packed [N, K/8] uint32 (field k at bits 4*(k % 8) of word k / 8), scales and biases
 * [N, K/64] bf16, w = scale * q + bias. */
typedef struct {
  const uint32_t* packed;
  const dfl_bf16* scales;
  const dfl_bf16* biases;
} dfl_q4_weight;

/* The projections [P2] quantizes (the drafter's constructor quantizes the linear projections
 * alone; the convs, the norms and the codebooks keep bf16). */
typedef struct {
  dfl_q4_weight q_proj, k_proj, v_proj, o_proj, gate_proj, up_proj, down_proj;
} dfl_q4_layer;

typedef struct {
  const dfl_bf16* fc;          /* [H, n_taps*H] */
  const dfl_bf16* hidden_norm; /* [H] */
  const dfl_bf16* norm;        /* [H] final norm */
  const dfl_bf16* sel_proj;    /* candidate_selector.hidden_projection [R, H] */
  const dfl_bf16* pred;        /* predecessor codebook [V, R] */
  const dfl_bf16* succ;        /* successor codebook [V, R] */
  const dfl_layer_weights* layers; /* host array of `layers` entries */
  const dfl_q4_layer* q4_layers;   /* NULL, or a host array of `layers` entries: the seven layer
                                      projections (and the context k|v) then run on these 4-bit
                                      weights, and the layer entries' q/k/v/o/gate/up/down
                                      pointers are not read */
} dfl_weights;

/* Copy and repack every drafter weight into buffers the handle owns ([P2] constructor
 * and `#releaseCheckpoint`: the drafter owns its tensors; `dispose` frees them): fused
 * q|k|v, gate/up interleaved per 16 rows, fused context k|v.  Synchronises `stream`
 * once; the caller may free the source tensors afterwards.  The target's embedding and
 * lm_head are not part of the drafter ([P2] header) and are passed per call. */
int dfl_drafter_load(const dfl_config* cfg, const dfl_weights* w, hipStream_t stream,
                     dfl_drafter** out);
void dfl_drafter_free(dfl_drafter* d);

/* Workspace of dfl_context_materialize for B requests of L new rows. */
size_t dfl_context_workspace_bytes(const dfl_drafter* d, int B, int L);

/* Context K/V of every layer from the target taps ([P2] `projectContext`: c =
 * RMSNorm(fc(concat taps), hidden_norm); `#contextKV`: K = RoPE(k_norm(k_proj c)) at the
 * row's absolute position, V = v_proj c; [P3] `materialize`: no input norm, no conv).
 *   taps:   [B, L, n_taps*H] bf16, taps concatenated on the feature axis.
 *   K, V:   host arrays of `layers` device pointers, each [B, Lcap, NKV, D] bf16.
 *   Rows row_offset .. row_offset+L-1 of every request are written, at absolute positions
 *   row_offset + j, so committed rows can be appended incrementally.
 *   Requires row_offset + L <= Lcap. */
int dfl_context_materialize(dfl_drafter* d, const dfl_bf16* taps, int B, int L, int row_offset,
                            int Lcap, dfl_bf16* const* K, dfl_bf16* const* V, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* Ragged context append ([P3] `materialize` with `input_row_offsets`; [P2] committed rows
 * projected at their absolute positions): each request appends its own number of new rows.
 *   taps:        [rows, n_taps*H] bf16, the new rows of all requests packed back to back.
 *   row_offsets: host [B+1], row_offsets[0] = 0, nondecreasing, row_offsets[B] = rows:
 *                request b's rows are taps rows [row_offsets[b], row_offsets[b+1]).
 *   starts:      host [B], the absolute position (and cache row) of each request's first new
 *                row; starts[b] + its row count <= Lcap (DFL_E_SHAPE otherwise).
 *   K, V:        as for dfl_context_materialize.  Rows outside the appended ranges are not
 *                touched.  ws: dfl_context_append_workspace_bytes(d, B, rows). */
size_t dfl_context_append_workspace_bytes(const dfl_drafter* d, int B, int rows);
int dfl_context_append(dfl_drafter* d, const dfl_bf16* taps, const int32_t* row_offsets,
                       const int32_t* starts, int B, int Lcap, dfl_bf16* const* K,
                       dfl_bf16* const* V, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace of dfl_draft_block for B requests of G rows whose context holds at most
 * Lmax rows. */
size_t dfl_draft_workspace_bytes(const dfl_drafter* d, int B, int G, int Lmax);

/* Bind the target's head once ([P2] `bindTarget`: the drafter binds to one target; binding
 * a different one afterwards is an error).  lm_head [V, H] bf16 row-major is copied, once,
 * into an owned tile-contiguous buffer that the head projection streams faster than the
 * row-major original; the values are snapshotted, so later changes to lm_head are not seen.
 * vocab_ids (host, optional): a draft vocabulary ([P2] `#block`, `#select`:
 * `DraftProjection.vocabulary`), n_vocab distinct token ids in [0, V), top_k <= n_vocab: only
 * those rows are copied, drafts that use the bound head project onto them (logits_out then
 * has n_vocab columns, in list order) and their candidates are the listed ids.  NULL: the
 * whole vocabulary.  When the copied rows fill whole 256-row tiles, the copy also holds the
 * drafter's selector projection after them, so drafts with the bound head compute z in the
 * head's launch (the same products, summed in another fp32 order than the separate
 * projection).  Synchronises `stream`.  Errors: a second call with another pointer or
 * vocabulary -> DFL_E_INVALID (the same binding again is a no-op); bad ids -> DFL_E_INVALID;
 * n_vocab out of range -> DFL_E_SHAPE; allocation -> DFL_E_NOMEM; HIP failure ->
 * DFL_E_DEVICE. */
int dfl_bind_target(dfl_drafter* d, const dfl_bf16* lm_head, const int32_t* vocab_ids, int n_vocab,
                    hipStream_t stream);

/* One draft block per request ([P2] `#block` then `#select`; [P3] `forward_block`,
 * `compute_candidates`, `score_edges`, `select_path`):
 *   embeds:   [B, G, H] bf16, the target's embedding of [anchor, MASK x (G-1)]
 *             ([P3] `mask_embeddings`: the drafter has no embedding of its own).
 *   anchors:  [B] int32 device, id of each request's last verified token.
 *   K, V:     host arrays of `layers` device pointers, [B, Lcap, NKV, D] bf16 each.
 *   ctx_len:  [B] int32 device, context rows attended per request (0..Lmax, Lmax <= Lcap);
 *             values outside [0, Lmax] are clamped into it.  Lcap*NKV*D < 2^31 (DFL_E_SHAPE).
 *   pos0:     [B] int32 device, absolute position of block row 0 of each request.
 *   lm_head:  [V, H] bf16, the target's head, borrowed; NULL, or the pointer given to
 *             dfl_bind_target, selects the bound copy.
 *   tokens:   [B, G-1] int32 device output ([P2] returns the proposals on the device).
 *   logits_out: NULL or [B, G-1, V] float32 device output of the head ([B, G-1, n_vocab]
 *             when a bound draft vocabulary is used).  NULL: the logits stay in the
 *             workspace; with more than 128 head rows (B*(G-1)) and top_k <= 16 the head
 *             then stores only the 256-column tiles of a row whose maximum reaches a value
 *             that 16 of the row's logits in distinct tiles reach (the others cannot hold a
 *             candidate).  The tokens are the same either way.
 *   G must satisfy 2 <= G <= block_size ([P3] `supports_zero_draft_rows` is false). */
int dfl_draft_block(dfl_drafter* d, const dfl_bf16* embeds, const int32_t* anchors, int B, int G,
                    const dfl_bf16* const* K, const dfl_bf16* const* V, int Lcap, int Lmax,
                    const int32_t* ctx_len, const int32_t* pos0, const dfl_bf16* lm_head,
                    int32_t* tokens, float* logits_out, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* ---- stage snapshots, for parity tests ----
 *
 * dfl_draft_block_traced runs exactly the launch sequence of dfl_draft_block (the same
 * kernels, plans and workspace) and, after the kernel that produces each stage below,
 * copies that stage's output into the caller's buffer (device memory, caller-owned; a NULL
 * pointer skips the stage).  The copies are ordinary stream-ordered device copies and
 * change no result.  The stages follow [P3] `DFlash2TransformerBlock` and
 * `DFlash2GroupedConv` and [P2] `#block` / `#select`; T = B*G, N = B*(G-1), ng = H/grp,
 * qkvw = (NH + 2*NKV)*D, ntiles = ceil(V'/256) with V' the head's columns.
 * Layer stages are taken from layer `layer` only. */
typedef struct {
  int32_t layer;        /* which layer's stages to copy (any value outside [0, layers): none) */
  dfl_bf16* x_in;       /* [T, H]    the layer's input rows */
  dfl_bf16* n;          /* [T, H]    RMSNorm(x_in; input_layernorm) */
  float* coef;          /* [T, 4*ng] attention conv's kernel projection D = n . W^T (fp32,
                                     columns [side][tap][group]) */
  dfl_bf16* a;          /* [T, H]    conv side 0 of n (prepare's output) */
  float* coef1;         /* [T, 2*ng] side-1 deltas as prepare hands them to finish */
  dfl_bf16* qkv;        /* [T, qkvw] q|k after per-head norm and RoPE, v as projected */
  dfl_bf16* attn;       /* [T, NH*D] attention output */
  dfl_bf16* u;          /* [T, H]    o projection */
  dfl_bf16* x_mid;      /* [T, H]    x_in + conv side 1 of u (the attention half's residual) */
  dfl_bf16* m;          /* [T, H]    RMSNorm(x_mid; post_attention_layernorm) */
  float* coef_mlp;      /* [T, 4*ng] MLP conv's kernel projection of m */
  dfl_bf16* i;          /* [T, H]    MLP conv side 0 of m */
  float* coef1_mlp;     /* [T, 2*ng] its side-1 deltas */
  dfl_bf16* p;          /* [T, F]    silu(gate) * up */
  dfl_bf16* f;          /* [T, H]    down projection */
  dfl_bf16* x_out;      /* [T, H]    x_mid + MLP conv side 1 of f (the layer's output) */
  dfl_bf16* n_next;     /* [T, H]    RMSNorm(x_out; next layer's input_layernorm); not written
                                     for the last layer, whose normed rows are `h` */
  dfl_bf16* h;          /* [N, H]    final-normed rows 1..G-1 of every block, packed */
  float* tile_max;      /* [N, ntiles] row maxima of every 256-column tile of the logits */
  int32_t* cand;        /* [N, K]    candidate ids */
  float* unary;         /* [N, K]    their logits */
  float* z;             /* [N, R]    selector projection */
  float* scores;        /* [N, K, K] edge scores */
} dfl_trace;

int dfl_draft_block_traced(dfl_drafter* d, const dfl_bf16* embeds, const int32_t* anchors, int B, int G,
                           const dfl_bf16* const* K, const dfl_bf16* const* V, int Lcap, int Lmax,
                           const int32_t* ctx_len, const int32_t* pos0, const dfl_bf16* lm_head,
                           int32_t* tokens, float* logits_out, void* ws, size_t ws_bytes,
                           const dfl_trace* trace, hipStream_t stream);

/* The same for dfl_context_materialize: the fc output, the context rows, and one layer's
 * k|v projection rows before the K store's norm and RoPE.  M = B*L. */
typedef struct {
  int32_t layer;        /* which layer's k|v rows to copy */
  dfl_bf16* fc_out;     /* [M, H]           taps . fc^T */
  dfl_bf16* c;          /* [M, H]           RMSNorm(fc_out; hidden_norm) */
  dfl_bf16* kv;         /* [M, 2*NKV*D]     [c . k_proj^T | c . v_proj^T] of layer `layer` */
} dfl_context_trace;

/* The same for dfl_context_append (M = the appended rows, packed as in `taps`). */
int dfl_context_append_traced(dfl_drafter* d, const dfl_bf16* taps, const int32_t* row_offsets,
                              const int32_t* starts, int B, int Lcap, dfl_bf16* const* K, dfl_bf16* const* V,
                              void* ws, size_t ws_bytes, const dfl_context_trace* trace, hipStream_t stream);

int dfl_context_materialize_traced(dfl_drafter* d, const dfl_bf16* taps, int B, int L, int row_offset,
                                   int Lcap, dfl_bf16* const* K, dfl_bf16* const* V, void* ws,
                                   size_t ws_bytes, const dfl_context_trace* trace, hipStream_t stream);

/* One drafter layer on a block ([P3] `DFlash2TransformerBlock`: r = x; h = conv.prepare(norm r);
 * h = attn(h); r += conv.finish(h), then the same for the MLP; [P2] `#block`, the body of the
 * layer loop).  x_in, x_out: [B*G, H] bf16, block rows of request b at b*G..b*G+G-1; x_out may
 * alias x_in.  K, V: this layer's context cache [B, Lcap, NKV, D]; ctx_len, pos0 as for
 * dfl_draft_block.  ws: at least dfl_draft_workspace_bytes(d, B, G, Lmax). */
int dfl_block_layer(dfl_drafter* d, int layer, const dfl_bf16* x_in, dfl_bf16* x_out, int B, int G,
                    const dfl_bf16* K, const dfl_bf16* V, int Lcap, int Lmax, const int32_t* ctx_len,
                    const int32_t* pos0, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- the steps of the path, one call each ---- */

/* RMSNorm over rows ([P2] `#rms`): y = x / sqrt(mean(x^2) + eps) * gamma, fp32 reduction.
 * x [rows, H] bf16 with leading dimension ldx; y [rows, H] bf16 (ldy); gamma [H] bf16. */
int dfl_rms_norm(const dfl_bf16* x, int rows, int H, int ldx, const dfl_bf16* gamma, float eps,
                 dfl_bf16* y, int ldy, hipStream_t stream);

/* Dense projection y = x . W^T ([P2] `Bf16Projection`), bf16 in, fp32 accumulate.
 * x [M, K] (ldx >= K), W [N, K]; out_f32 != 0: y fp32 [M, N] (ldy); else bf16.
 * K must be a multiple of 64.  ws/ws_bytes: split-K partials (dfl_linear_workspace_bytes). */
size_t dfl_linear_workspace_bytes(int M, int N, int K);
int dfl_linear(const dfl_bf16* x, int M, int K, int ldx, const dfl_bf16* W, int N, void* y,
               int ldy, int out_f32, void* ws, size_t ws_bytes, hipStream_t stream);

/* Dense projection with 4-bit affine weights ([P2] `quantizedWeight`: groups of 64 inputs
 * along K, a scale and a bias per group, w = scale * q + bias with q in 0..15).
 * packed [N, K/8] uint32, 16-byte aligned: field k of row n at bits 4*(k % 8) of word
 * k / 8; scales, biases [N, K/64] bf16.  The weights are dequantized in fp32 and rounded to
 * bf16 on the way into the bf16 matrix units; accumulation is fp32.  Other arguments,
 * outputs and errors as dfl_linear (same workspace size). */
int dfl_linear_q4(const dfl_bf16* x, int M, int K, int ldx, const uint32_t* packed,
                  const dfl_bf16* scales, const dfl_bf16* biases, int N, void* y, int ldy,
                  int out_f32, void* ws, size_t ws_bytes, hipStream_t stream);

/* Per-head RMSNorm then neox RoPE, in place ([P2] `#block`: q/k norm before RoPE;
 * [P1] per-head RMSNorm and split-half RoPE docstrings).  x holds rows of `heads`
 * heads of D values at leading dimension ldx; row r sits at position
 * pos0[r / rows_per_req] + r % rows_per_req (pos0 device int32). gamma [D] bf16. */
int dfl_head_norm_rope(dfl_bf16* x, int rows, int heads, int D, int ldx, const dfl_bf16* gamma,
                       float eps, float theta, const int32_t* pos0, int rows_per_req,
                       hipStream_t stream);

/* Bidirectional block attention over each request's context prefix plus the block's own
 * rows ([P2] header and `#block`: no mask, no window, scale 1/sqrt(D); GQA kv head =
 * h / (NH/NKV)).  q [B*G, NH*D] (ldq), kb/vb [B*G, NKV*D] (ldkv), K/V [B, Lcap, NKV, D],
 * ctx_len [B] device (clamped into [0, Lmax]); out [B*G, NH*D] bf16 (ldo); Lcap*NKV*D must be
 * below 2^31 (DFL_E_SHAPE).  window > 0: sliding attention ([P3] `layer_types`): block row t
 * of request b (position pos0[b] + t, pos0 [B] device) sees context rows j >= pos0[b] + t -
 * window + 1 only; window = 0: all context rows (pos0 may then be NULL).
 * ws: dfl_attention_workspace_bytes. */
size_t dfl_attention_workspace_bytes(int B, int G, int NH, int NKV, int D, int Lmax);
int dfl_block_attention(const dfl_bf16* q, int ldq, const dfl_bf16* kb, const dfl_bf16* vb,
                        int ldkv, const dfl_bf16* K, const dfl_bf16* V, int Lcap, int Lmax,
                        const int32_t* ctx_len, const int32_t* pos0, int window, int B, int G, int NH,
                        int NKV, int D, dfl_bf16* out, int ldo, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Grouped dynamic conv, side 0 ([P3] `DFlash2GroupedConv.prepare`; [P2] `#coefficients`
 * and `#conv`): D = x . kproj^T read as [side][tap][group]; out[t,c] = sum_tap
 * (base[0,tap,c] + D[t,0,tap,c/grp]) * x[t-tap,c] with x[-1] = 0 at every block start.
 * x, out [T, H] bf16; T a multiple of G; base [2,2,H] bf16; kproj [4*H/grp, H] bf16.
 * coef1: [T, 2, H/grp] fp32 output, the side-1 deltas finish() reuses (base excluded). */
size_t dfl_conv_prepare_workspace_bytes(int T, int H, int grp);
int dfl_conv_prepare(const dfl_bf16* x, int T, int H, int G, int grp, const dfl_bf16* kproj,
                     const dfl_bf16* base, dfl_bf16* out, float* coef1, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Grouped dynamic conv, side 1 ([P3] `DFlash2GroupedConv.finish`): out[t,c] =
 * residual[t,c] + sum_tap (base[1,tap,c] + coef1[t,tap,c/grp]) * y[t-tap,c], y[-1] = 0 per
 * block, summed in fp32 and rounded once to bf16 ([P2] `#block` adds the residual in fp32).
 * residual may be NULL (then no residual) and may alias out. */
int dfl_conv_finish(const dfl_bf16* y, const float* coef1, const dfl_bf16* base, int T, int H,
                    int G, int grp, const dfl_bf16* residual, dfl_bf16* out, hipStream_t stream);

/* Top-k of each row of fp32 logits ([P3] `compute_candidates`; [P2] `#select`), listed by
 * value descending then id ascending.  logits [N, V]; ids int32 [N, K]; unary fp32 [N, K];
 * 1 <= K <= min(32, V).  ws: dfl_candidates_workspace_bytes, one fp32 row maximum per
 * 256-column tile (the top-k reads only the tiles whose maximum can hold a candidate). */
size_t dfl_candidates_workspace_bytes(int N, int V, int K);
int dfl_compute_candidates(const float* logits, int N, int V, int K, int32_t* ids, float* unary,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* dfl_compute_candidates without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * tile maxima go to a static device array owned by the library, DFL_CANDIDATES_STATIC_MAX_TILES
 * floats (4 MiB) on each GPU it runs on, held until the process ends.  The call allocates
 * nothing.  N * ceil(V / 256) above that limit -> DFL_E_WORKSPACE (checked before anything is
 * enqueued).  Every call on one GPU shares that GPU's array (each call writes all the tile
 * maxima it reads before reading them), so calls that overlap on one GPU, on different
 * streams or threads, race.  Other arguments, outputs and errors as dfl_compute_candidates. */
#define DFL_CANDIDATES_STATIC_MAX_TILES (1 << 20)
int dfl_compute_candidates_static(const float* logits, int N, int V, int K, int32_t* ids,
                                  float* unary, hipStream_t stream);

/* Selector projection z = h . proj^T kept in fp32 ([P2] `#block`: z = hidden_projection(h)).
 * h [N, H] bf16, proj [R, H] bf16, z [N, R] fp32.  With H a multiple of 128, R <= 64 and h,
 * proj 16-byte aligned it runs the kernel dfl_select_tokens_projected runs (the same z bit
 * for bit) and uses no workspace; otherwise the split-K GEMM of dfl_linear. */
size_t dfl_selector_project_workspace_bytes(int N, int H, int R);
int dfl_selector_project(const dfl_bf16* h, int N, int H, const dfl_bf16* proj, int R, float* z,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* score_edges ([P3] `DFlash2CandidateSelector.score_edges`):
 * S[b,l,p,c] = unary[b,l,c] + sum_r pred[pid(b,l,p),r] * z[b,l,r] * succ[cand[b,l,c],r],
 * pid(b,0,p) = anchors[b], pid(b,l,p) = cand[b,l-1,p].  cand int32 [B,S,K], unary fp32
 * [B,S,K], z fp32 [B,S,R], anchors int32 [B], pred/succ bf16 [V,R]; scores fp32 [B,S,K,K].
 * Ids outside [0, V) are clamped to that range. */
int dfl_score_edges(const int32_t* cand, const float* unary, const float* z,
                    const int32_t* anchors, int B, int S, int K, int R, const dfl_bf16* pred,
                    const dfl_bf16* succ, int V, float* scores, hipStream_t stream);

/* Greedy walk ([P3] `select_path`): j_0 = argmax_c S[b,0,0,c], j_l = argmax_c
 * S[b,l,j_{l-1},c], tokens[b,l] = cand[b,l,j_l]; ties go to the lowest c. */
int dfl_select_path(const float* scores, const int32_t* cand, int B, int S, int K,
                    int32_t* tokens, hipStream_t stream);

/* The selection of B requests in one launch ([P3] `compute_candidates`, `score_edges` and
 * `select_path`; [P2] `#select`): for each request's S slots the top-K of the logits (value
 * descending, id ascending), the edge scores and the greedy walk, with the same results as
 * dfl_compute_candidates, dfl_score_edges and dfl_select_path called in turn.
 *   logits:   [B*S, V] fp32;  tile_max: [B*S, ceil(V/256)] fp32, each row's maximum over every
 *             256-column tile (dfl_tile_maxima), or NULL: then one workgroup per row scans that
 *             row's logits, keeps its tile maxima on chip and takes its top-k as soon as its
 *             scan ends (ceil(V/256) <= 4096, else DFL_E_UNSUPPORTED);
 *             z: [B*S, R] fp32 (dfl_selector_project);
 *   anchors:  [B] int32;  pred, succ: [V, R] bf16;
 *   cand, unary: [B*S, K] out;  scores: [B*S, K, K] out, or NULL;  tokens: [B, S] out.
 * Requires S <= 64, K <= 16 and R a multiple of 4 in [4, 64] (DFL_E_UNSUPPORTED otherwise:
 * the three calls above cover every size).  Ids outside [0, V) are clamped for the codebook
 * reads, as in dfl_score_edges.  Two launches: the top-k, then the edge scores (fp32 on the
 * matrix cores, as dfl_score_edges computes them for these sizes) and the walk. */
int dfl_tile_maxima(const float* logits, int N, int V, float* tile_max, hipStream_t stream);
int dfl_select_tokens(const float* logits, const float* tile_max, int B, int S, int V, int K,
                      const float* z, int R, const int32_t* anchors, const dfl_bf16* pred,
                      const dfl_bf16* succ, int32_t* cand, float* unary, float* scores,
                      int32_t* tokens, hipStream_t stream);

/* The selection with its projection ([P2] `#block`: z = hidden_projection(h), then
 * `#select`; [P3] `compute_candidates`, `score_edges`, `select_path`): z = h . proj^T is
 * computed by extra workgroups of the scanning top-k's launch (dfl_select_tokens with
 * tile_max NULL), beside the scans, and written to z; then the edge scores and the walk read
 * it.  The results equal dfl_selector_project followed by dfl_select_tokens(tile_max NULL).
 *   h: [B*S, H] bf16; proj: [R, H] bf16; z: [B*S, R] fp32 out;
 *   other arguments as dfl_select_tokens.
 * Requires H a multiple of 128, h and proj 16-byte aligned, and dfl_select_tokens's limits
 * (DFL_E_UNSUPPORTED otherwise).  Two launches. */
int dfl_select_tokens_projected(const float* logits, int B, int S, int V, int K, const dfl_bf16* h, int H,
                                const dfl_bf16* proj, int R, float* z, const int32_t* anchors,
                                const dfl_bf16* pred, const dfl_bf16* succ, int32_t* cand, float* unary,
                                float* scores, int32_t* tokens, hipStream_t stream);

/* ---- measurement ---- */

/* Kernel classes whose launches can be bracketed with HIP events. */
enum dfl_kernel_class {
  DFL_K_NONE = -1,
  DFL_K_GEMM_HEAD = 0, DFL_K_GEMM_GATEUP, DFL_K_GEMM_DOWN, DFL_K_GEMM_QKV, DFL_K_GEMM_O,
  DFL_K_GEMM_KPROJ, DFL_K_GEMM_SELPROJ, DFL_K_GEMM_CONTEXT, DFL_K_ATTENTION, DFL_K_CONV_PREPARE,
  DFL_K_CONV_FINISH, DFL_K_RMSNORM, DFL_K_ROPE, DFL_K_TOPK, DFL_K_SCORE_EDGES,
  DFL_K_SELECT_PATH, DFL_K_SELECT, DFL_K_COUNT
};

/* Bracket every later launch of class `k` made through `d` with a pair of HIP events on
 * the launch's own stream (DFL_K_NONE stops).  dfl_read_kernel_time synchronises those
 * events, returns the summed duration and launch count since the last read, and resets. */
int dfl_set_timed_kernel(dfl_drafter* d, int k);
int dfl_read_kernel_time(dfl_drafter* d, double* total_ms, int64_t* launches, double* bytes);

/* Last error message of the calling thread ("" if none). */
const char* dfl_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH2_H */
