// C ABI of the drafter (include/dflash2.h): argument validation, owned weight repacking,
// workspace carving and the launch sequence of a draft block.  Nothing here synchronises
// the caller's stream except dfl_drafter_load and dfl_read_kernel_time.
#include "dflash2.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <set>
#include <string>
#include <vector>

#include "kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define DFL_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define DFL_HIP(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(DFL_E_DEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sequential carve of a caller workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

struct LayerBuf {
  uint16_t *in_norm, *post_norm, *q_norm, *k_norm;
  uint16_t *qkv, *o, *gateup, *down;
  uint16_t *attn_base, *attn_kproj, *mlp_base, *mlp_kproj;
  uint16_t* kv_ctx;  // [k | v] rows for the context path
  // 4-bit drafters: the same five projections as tile-contiguous 4-bit blocks (the bf16
  // pointers above are then NULL)
  uint32_t *qkv_q4 = nullptr, *o_q4 = nullptr, *gateup_q4 = nullptr, *down_q4 = nullptr, *kv_ctx_q4 = nullptr;
};

// the weight of one of a layer's projections, bf16 or 4-bit, both tile-contiguous
dfl::WeightRef wref(const uint16_t* bf, const uint32_t* q4) {
  dfl::WeightRef w;
  w.w = bf;
  w.q = q4;
  w.tiled = true;
  return w;
}

struct TimedLaunch {
  hipEvent_t start, stop;
  double bytes;
};

}  // namespace

struct dfl_drafter {
  dfl_config cfg;
  void* arena = nullptr;
  uint16_t *fc, *hidden_norm, *norm, *sel_proj, *pred, *succ;
  std::vector<LayerBuf> layers;
  bool q4 = false;                   // the layer projections hold 4-bit weights
  std::vector<int> window;           // per layer: 0 = full attention, W = sliding window
  uint16_t* head = nullptr;          // the bound target head, tile-contiguous (dfl_bind_target)
  const void* head_src = nullptr;    // the caller pointer it was copied from
  int head_cols = 0;                 // its rows: the vocabulary, or the listed draft vocabulary
  int32_t* head_ids = nullptr;       // device [head_cols] token ids of a draft vocabulary, else NULL
  bool head_sel = false;             // the bound head also holds sel_proj's rows, one tile after its own
  int timed_class = DFL_K_NONE;
  std::vector<TimedLaunch> timed;
  std::vector<hipEvent_t> pool;
};

namespace {

hipEvent_t pooled_event(dfl_drafter* d) {
  if (!d->pool.empty()) {
    hipEvent_t e = d->pool.back();
    d->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `f` (which enqueues the launches of kernel class k), bracketed by events when k is
// the class being timed.
template <class F>
int timed(dfl_drafter* d, int k, double bytes, hipStream_t s, F&& f) {
  const bool on = d && d->timed_class == k;
  hipEvent_t a = nullptr, b = nullptr;
  if (on) {
    a = pooled_event(d);
    b = pooled_event(d);
    if (!a || !b) return fail(DFL_E_DEVICE, "hipEventCreate failed");
    DFL_HIP(hipEventRecord(a, s));
  }
  hipError_t e = f();
  if (e != hipSuccess) return fail(DFL_E_DEVICE, "kernel launch (class %d): %s", k, hipGetErrorString(e));
  if (on) {
    DFL_HIP(hipEventRecord(b, s));
    d->timed.push_back({a, b, bytes});
  }
  return DFL_OK;
}

#define DFL_TRY(expr)          \
  do {                         \
    int rc_ = (expr);          \
    if (rc_ != DFL_OK) return rc_; \
  } while (0)

// Stage snapshot for dfl_*_traced: a stream-ordered device copy into the caller's buffer
// (skipped when the buffer is NULL).
int snap(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (!dst || bytes == 0) return DFL_OK;
  DFL_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
  return DFL_OK;
}

// Snapshot of a projection's fp32 split-K planes as their sum (in plane order, the order
// every consumer of the planes adds them).
int snap_planes(float* dst, const dfl::Planes& pl, int M, int N, hipStream_t s) {
  if (!dst) return DFL_OK;
  DFL_HIP(dfl::launch_planes_sum(pl, M, N, dst, s));
  return DFL_OK;
}

// Algorithmic bytes of y = A . W^T: A and the output once, the weight at 2 bytes per
// element, or (q4) at half a byte plus a bf16 scale and bias per 64.
double gemm_bytes(int M, int N, int K, int epi, bool q4 = false) {
  const double out = epi == dfl::EPI_F32 ? 4.0 * M * N : (epi == dfl::EPI_SILU_MUL ? 1.0 * M * N : 2.0 * M * N);
  return 2.0 * M * K + (q4 ? 0.5625 : 2.0) * N * K + out;
}

int check_config(const dfl_config* c) {
  DFL_REQUIRE(c, DFL_E_INVALID, "config is NULL");
  DFL_REQUIRE(c->hidden > 0 && c->layers > 0 && c->heads > 0 && c->kv_heads > 0 && c->head_dim > 0 &&
                  c->intermediate > 0 && c->n_taps > 0 && c->block_size > 0 && c->conv_group > 0 &&
                  c->top_k > 0 && c->rank > 0 && c->vocab > 0,
              DFL_E_INVALID, "config sizes must be positive");
  DFL_REQUIRE(c->conv_taps == 2, DFL_E_UNSUPPORTED, "conv_taps %d not supported (two-tap only)", c->conv_taps);
  DFL_REQUIRE(c->block_size >= 2, DFL_E_UNSUPPORTED, "block_size %d < 2: zero draft rows are not supported",
              c->block_size);
  DFL_REQUIRE(c->heads % c->kv_heads == 0, DFL_E_SHAPE, "heads %d not a multiple of kv_heads %d", c->heads,
              c->kv_heads);
  DFL_REQUIRE(c->head_dim == 64 || c->head_dim == 128, DFL_E_UNSUPPORTED, "head_dim %d must be 64 or 128",
              c->head_dim);
  DFL_REQUIRE(c->hidden % 64 == 0 && c->hidden <= 8192, DFL_E_UNSUPPORTED,
              "hidden %d must be a multiple of 64 and <= 8192", c->hidden);
  DFL_REQUIRE(c->intermediate % 64 == 0, DFL_E_UNSUPPORTED, "intermediate %d must be a multiple of 64",
              c->intermediate);
  DFL_REQUIRE(c->conv_group % 8 == 0 && c->hidden % c->conv_group == 0, DFL_E_UNSUPPORTED,
              "conv_group %d must be a multiple of 8 dividing hidden", c->conv_group);
  DFL_REQUIRE(c->top_k <= 32 && c->top_k <= c->vocab, DFL_E_UNSUPPORTED, "top_k %d must be <= 32 and <= vocab",
              c->top_k);
  DFL_REQUIRE(c->rank <= 128, DFL_E_UNSUPPORTED, "rank %d must be <= 128", c->rank);
  DFL_REQUIRE(c->block_size * (c->heads / c->kv_heads) <= 64, DFL_E_UNSUPPORTED,
              "block_size x heads/kv_heads = %d query rows per KV head exceeds 64",
              c->block_size * (c->heads / c->kv_heads));
  DFL_REQUIRE(c->rms_eps >= 0.f && c->rope_theta > 0.f, DFL_E_INVALID, "rms_eps must be >= 0, rope_theta > 0");
  DFL_REQUIRE(c->sliding_window >= 0, DFL_E_INVALID, "sliding_window %d must be >= 0", c->sliding_window);
  if (c->tap_layer_ids) {
    std::set<int> seen;
    for (int i = 0; i < c->n_taps; ++i)
      DFL_REQUIRE(seen.insert(c->tap_layer_ids[i]).second, DFL_E_UNSUPPORTED,
                  "tap layer id %d repeats", c->tap_layer_ids[i]);
  }
  return DFL_OK;
}

struct DraftLayout {
  size_t x, n, a, qkv, ao, u, p, h, logits, tmax, tbound, z, cand, unary, scores, attn, kpart, coef1, partial;
  size_t atile, atile_elems;
  size_t total;
};

DraftLayout draft_layout(const dfl_config& c, int B, int G, int Lmax) {
  const int H = c.hidden, ng = c.hidden / c.conv_group, T = B * G, S = G - 1, N = B * S;
  const int qkvw = (c.heads + 2 * c.kv_heads) * c.head_dim;
  const int F = c.intermediate;
  DraftLayout L;
  Carver cv(nullptr);
  L.x = cv.off; cv.take<uint16_t>((size_t)T * H);
  L.n = cv.off; cv.take<uint16_t>((size_t)T * H);
  L.a = cv.off; cv.take<uint16_t>((size_t)T * H);
  L.qkv = cv.off; cv.take<uint16_t>((size_t)T * qkvw);
  L.ao = cv.off; cv.take<uint16_t>((size_t)T * c.heads * c.head_dim);
  L.u = cv.off; cv.take<uint16_t>((size_t)T * H);
  L.p = cv.off; cv.take<uint16_t>((size_t)T * F);
  L.h = cv.off; cv.take<uint16_t>((size_t)N * H);
  L.logits = cv.off; cv.take<float>((size_t)N * c.vocab);
  L.tmax = cv.off; cv.take<float>((size_t)N * ((c.vocab + dfl::kGemmTileN - 1) / dfl::kGemmTileN));
  L.tbound = cv.off; cv.take<uint32_t>((size_t)N * dfl::kTileBoundSlots);
  L.z = cv.off; cv.take<float>((size_t)N * c.rank);
  L.cand = cv.off; cv.take<int32_t>((size_t)N * c.top_k);
  L.unary = cv.off; cv.take<float>((size_t)N * c.top_k);
  L.scores = cv.off; cv.take<float>((size_t)N * c.top_k * c.top_k);
  L.attn = cv.off; cv.take<char>(dfl::plan_attention(B, G, c.heads, c.kv_heads, c.head_dim, Lmax).ws_bytes);
  // kernel-projection planes live from the projection to the half-layer's finish; the q|k|v
  // planes and every other projection's split-K scratch share one region
  auto planes_bytes = [](int M, int N, int K) {
    return (size_t)dfl::plan_gemm(M, N, K).splits * M * N * sizeof(float);
  };
  L.kpart = cv.off; cv.take<char>(planes_bytes(T, 4 * ng, H));
  L.coef1 = cv.off; cv.take<float>((size_t)T * 2 * ng);  // side-1 coefficients, summed by prepare
  size_t part = planes_bytes(T, qkvw, H);
  const int shapes[][4] = {{T, H, c.heads * c.head_dim, 0}, {T, 2 * F, H, 0}, {T, H, F, 0}, {N, c.vocab, H, 1},
                           {N, c.rank, H, 0}};
  for (auto& s : shapes) part = std::max(part, dfl::plan_gemm(s[0], s[1], s[2], s[3] != 0).partial_bytes);
  L.partial = cv.off; cv.take<char>(part);
  // the fragment-order copy of gate/up's or the head's activations when they run on 256-row
  // tiles (the 256 x 256 kernel then copies whole contiguous 1 KB fragments)
  const bool wide = dfl::gemm_takes_tiled_a(dfl::plan_gemm(T, 2 * F, H), false) ||
                    dfl::gemm_takes_tiled_a(dfl::plan_gemm(N, c.vocab + c.rank, H, true), false) ||
                    dfl::gemm_takes_tiled_a(dfl::plan_gemm(N, c.vocab, H, true), false);
  L.atile_elems = wide ? dfl::tiled_rows_elems(std::max(T, N), H) : 0;
  L.atile = cv.off; cv.take<uint16_t>(L.atile_elems);
  L.total = cv.off;
  return L;
}

struct CtxLayout {
  size_t craw, c, kv, partial, total;
};

CtxLayout ctx_layout(const dfl_config& c, int B, int L) {
  const size_t M = (size_t)B * L;
  const int H = c.hidden, kvw = 2 * c.kv_heads * c.head_dim;
  CtxLayout o;
  Carver cv(nullptr);
  o.craw = cv.off; cv.take<uint16_t>(M * H);
  o.c = cv.off; cv.take<uint16_t>(M * H);
  o.kv = cv.off; cv.take<uint16_t>(M * kvw);
  const size_t p1 = dfl::plan_gemm((int)M, H, c.n_taps * H).partial_bytes;
  const size_t p2 = dfl::plan_gemm((int)M, kvw, H).partial_bytes;
  o.partial = cv.off; cv.take<char>(std::max(p1, p2));
  o.total = cv.off;
  return o;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

// One layer on the block (P3 DFlash2TransformerBlock; P2 #block, the body of the layer loop):
// x_out = x_in + conv1(attn(conv0(rms x_in))), then the same for the MLP.  x_out may alias
// x_in (every element is read and written by the same thread of the residual conv).
//
// n_ready: the workspace's n already holds RMSNorm(x_in; input_norm) (written by the previous
// layer's fused finish).  next_gamma: when not NULL, the MLP finish also writes
// n = RMSNorm(x_out; next_gamma), the next layer's normed input.
int run_layer(dfl_drafter* d, int li, const uint16_t* xin, uint16_t* x, int B, int G, const uint16_t* Kl,
              const uint16_t* Vl, int Lcap, int Lmax, const int32_t* ctx_len, const int32_t* pos0, char* W,
              const DraftLayout& lay, bool n_ready, const uint16_t* next_gamma, hipStream_t stream,
              uint16_t* head_rows = nullptr, const dfl_trace* trace = nullptr, uint32_t* clear_bound = nullptr) {
  const dfl_config& c = d->cfg;
  const LayerBuf& L = d->layers[li];
  const int H = c.hidden, NH = c.heads, NKV = c.kv_heads, D = c.head_dim, F = c.intermediate;
  const int ng = H / c.conv_group, T = B * G;
  const int qkvw = (NH + 2 * NKV) * D;
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(W + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(W + off); };
  uint16_t *n = u16(lay.n), *a = u16(lay.a), *qkv = u16(lay.qkv), *ao = u16(lay.ao);
  uint16_t *u = u16(lay.u), *p = u16(lay.p);
  float *kpart = f32(lay.kpart), *part = f32(lay.partial), *c1 = f32(lay.coef1);
  const dfl::AttnPlan apl = dfl::plan_attention(B, G, NH, NKV, D, Lmax);
  const dfl::GemmPlan p_kp = dfl::plan_gemm(T, 4 * ng, H), p_qkv = dfl::plan_gemm(T, qkvw, H),
                      p_o = dfl::plan_gemm(T, H, NH * D), p_gu = dfl::plan_gemm(T, 2 * F, H),
                      p_dn = dfl::plan_gemm(T, H, F);
  // The kernel projection's columns are [side][tap][group]: side 0 feeds prepare, side 1 finish.
  // prepare sums side 1's coefficients into one plane as it sums its own
  const dfl::Planes coef0 = dfl::gemm_planes(p_kp, kpart, T, 4 * ng);
  dfl::Planes coef1;
  coef1.p = c1;
  coef1.S = 1;
  coef1.ld = 2 * ng;
  coef1.plane = (size_t)T * 2 * ng;
  const double conv_bytes = 2.0 * T * H * 2 + 4.0 * T * 2 * ng;  // y in, out, one side's deltas
  const double norm_bytes = 4.0 * T * H;
  const dfl_trace* tr = trace && trace->layer == li ? trace : nullptr;
  const size_t rowsH = (size_t)T * H * sizeof(uint16_t);
  // attention half
  if (tr) DFL_TRY(snap(tr->x_in, xin, rowsH, stream));
  if (!n_ready) {
    DFL_TRY(timed(d, DFL_K_RMSNORM, norm_bytes, stream, [&] {
      return dfl::launch_rms_norm(xin, H, T, H, L.in_norm, c.rms_eps, n, H, 1, 1, 0, stream);
    }));
  }
  if (tr) DFL_TRY(snap(tr->n, n, rowsH, stream));
  DFL_TRY(timed(d, DFL_K_GEMM_KPROJ, gemm_bytes(T, 4 * ng, H, dfl::EPI_F32), stream, [&] {
    return dfl::launch_gemm_partials(p_kp, n, H, L.attn_kproj, true, T, 4 * ng, H, kpart, stream);
  }));
  if (tr) DFL_TRY(snap_planes(tr->coef, coef0, T, 4 * ng, stream));
  DFL_TRY(timed(d, DFL_K_CONV_PREPARE, conv_bytes, stream, [&] {
    return dfl::launch_conv(n, coef0, L.attn_base, 0, T, H, G, c.conv_group, nullptr, a, stream, c1);
  }));
  if (tr) {
    DFL_TRY(snap(tr->a, a, rowsH, stream));
    DFL_TRY(snap(tr->coef1, c1, (size_t)T * 2 * ng * sizeof(float), stream));
  }
  DFL_TRY(timed(d, DFL_K_GEMM_QKV, gemm_bytes(T, qkvw, H, dfl::EPI_F32, d->q4), stream, [&] {
    return dfl::launch_gemm_partials(p_qkv, a, H, wref(L.qkv, L.qkv_q4), T, qkvw, H, part, stream);
  }));
  DFL_TRY(timed(d, DFL_K_ROPE, 4.0 * T * qkvw * p_qkv.splits + 2.0 * T * qkvw, stream, [&] {
    return dfl::launch_head_norm_rope_planes(dfl::gemm_planes(p_qkv, part, T, qkvw), qkv, qkvw, T, NH + NKV, NH, D,
                                             NKV * D, L.q_norm, L.k_norm, c.rms_eps, c.rope_theta, pos0, G, 0,
                                             stream);
  }));
  if (tr) DFL_TRY(snap(tr->qkv, qkv, (size_t)T * qkvw * sizeof(uint16_t), stream));
  const double attn_bytes = 4.0 * (double)B * Lmax * NKV * D + 2.0 * T * qkvw + 2.0 * T * NH * D;
  DFL_TRY(timed(d, DFL_K_ATTENTION, attn_bytes, stream, [&] {
    return dfl::launch_attention(apl, qkv, qkvw, qkv + NH * D, qkv + (NH + NKV) * D, qkvw, Kl, Vl, Lcap, ctx_len,
                                 pos0, d->window[li], B, G, NH, NKV, D, Lmax, ao, NH * D, W + lay.attn, stream);
  }));
  if (tr) DFL_TRY(snap(tr->attn, ao, (size_t)T * NH * D * sizeof(uint16_t), stream));
  // A split o or down projection leaves its fp32 planes to the residual conv + norm, which
  // sums each row's planes itself (and rounds the sum to bf16 as the reduce would), so the
  // split-K reduce launch goes away; the bf16 output u is then only written under tracing.
  const bool o_planes = p_o.splits > 1 && H <= dfl::kCrnPlanesMaxH;
  DFL_TRY(timed(d, DFL_K_GEMM_O, gemm_bytes(T, H, NH * D, dfl::EPI_BF16, d->q4), stream, [&] {
    return o_planes ? dfl::launch_gemm_partials(p_o, ao, NH * D, wref(L.o, L.o_q4), T, H, NH * D, part, stream)
                    : dfl::launch_gemm(p_o, ao, NH * D, wref(L.o, L.o_q4), T, H, NH * D, dfl::EPI_BF16, u, H,
                                       nullptr, 0, 0, part, stream);
  }));
  const dfl::Planes o_pl{part, p_o.splits, H, (size_t)T * H};
  if (tr) {
    if (o_planes) DFL_HIP(dfl::launch_planes_sum_bf16(o_pl, T, H, u, stream));
    DFL_TRY(snap(tr->u, u, rowsH, stream));
  }
  // x = x_in + conv1(u), fused with the MLP half's input norm
  DFL_TRY(timed(d, DFL_K_CONV_FINISH, conv_bytes + 4.0 * T * H + (o_planes ? 4.0 * T * H * p_o.splits : 0.0), stream,
                [&] {
                  return o_planes ? dfl::launch_conv_residual_norm_planes(o_pl, coef1, L.attn_base, T, H, G,
                                                                          c.conv_group, xin, x, L.post_norm,
                                                                          c.rms_eps, n, stream)
                                  : dfl::launch_conv_residual_norm(u, coef1, L.attn_base, T, H, G, c.conv_group,
                                                                   xin, x, L.post_norm, c.rms_eps, n, stream);
                }));
  if (tr) {
    DFL_TRY(snap(tr->x_mid, x, rowsH, stream));
    DFL_TRY(snap(tr->m, n, rowsH, stream));
  }
  // MLP half
  DFL_TRY(timed(d, DFL_K_GEMM_KPROJ, gemm_bytes(T, 4 * ng, H, dfl::EPI_F32), stream, [&] {
    return dfl::launch_gemm_partials(p_kp, n, H, L.mlp_kproj, true, T, 4 * ng, H, kpart, stream);
  }));
  if (tr) DFL_TRY(snap_planes(tr->coef_mlp, coef0, T, 4 * ng, stream));
  DFL_TRY(timed(d, DFL_K_CONV_PREPARE, conv_bytes, stream, [&] {
    return dfl::launch_conv(n, coef0, L.mlp_base, 0, T, H, G, c.conv_group, nullptr, a, stream, c1);
  }));
  if (tr) {
    DFL_TRY(snap(tr->i, a, rowsH, stream));
    DFL_TRY(snap(tr->coef1_mlp, c1, (size_t)T * 2 * ng * sizeof(float), stream));
  }
  // on 256-row tiles gate/up reads a fragment-order copy of a (counted with the projection)
  const bool gu_tiled = dfl::gemm_takes_tiled_a(p_gu, d->q4) && lay.atile_elems >= dfl::tiled_rows_elems(T, H);
  DFL_TRY(timed(d, DFL_K_GEMM_GATEUP, gemm_bytes(T, 2 * F, H, dfl::EPI_SILU_MUL, d->q4), stream, [&] {
    if (gu_tiled) {
      const hipError_t e = dfl::launch_tile_rows(a, H, T, H, u16(lay.atile), stream);
      if (e != hipSuccess) return e;
    }
    return dfl::launch_gemm(p_gu, gu_tiled ? u16(lay.atile) : a, H, wref(L.gateup, L.gateup_q4), T, 2 * F, H,
                            dfl::EPI_SILU_MUL, p, F, nullptr, 0, 0, part, stream, nullptr, nullptr, gu_tiled);
  }));
  if (tr) DFL_TRY(snap(tr->p, p, (size_t)T * F * sizeof(uint16_t), stream));
  const bool d_planes = p_dn.splits > 1 && next_gamma && H <= dfl::kCrnPlanesMaxH;
  DFL_TRY(timed(d, DFL_K_GEMM_DOWN, gemm_bytes(T, H, F, dfl::EPI_BF16, d->q4), stream, [&] {
    return d_planes ? dfl::launch_gemm_partials(p_dn, p, F, wref(L.down, L.down_q4), T, H, F, part, stream)
                    : dfl::launch_gemm(p_dn, p, F, wref(L.down, L.down_q4), T, H, F, dfl::EPI_BF16, u, H, nullptr,
                                       0, 0, part, stream);
  }));
  const dfl::Planes d_pl{part, p_dn.splits, H, (size_t)T * H};
  if (tr) {
    if (d_planes) DFL_HIP(dfl::launch_planes_sum_bf16(d_pl, T, H, u, stream));
    DFL_TRY(snap(tr->f, u, rowsH, stream));
  }
  if (next_gamma) {
    // the next layer's input norm, or (head_rows set) the final norm of rows 1..G-1, packed
    // for the head
    uint16_t* nrows = head_rows ? head_rows : n;
    const bool pack = head_rows != nullptr;
    DFL_TRY(timed(d, DFL_K_CONV_FINISH, conv_bytes + 4.0 * T * H + (d_planes ? 4.0 * T * H * p_dn.splits : 0.0),
                  stream, [&] {
                    // with the packed rows it also clears the head's bound slots
                    uint32_t* cb = pack ? clear_bound : nullptr;
                    return d_planes ? dfl::launch_conv_residual_norm_planes(d_pl, coef1, L.mlp_base, T, H, G,
                                                                            c.conv_group, x, x, next_gamma,
                                                                            c.rms_eps, nrows, stream, pack, cb)
                                    : dfl::launch_conv_residual_norm(u, coef1, L.mlp_base, T, H, G, c.conv_group,
                                                                     x, x, next_gamma, c.rms_eps, nrows, stream,
                                                                     pack, cb);
                  }));
  } else {
    DFL_TRY(timed(d, DFL_K_CONV_FINISH, conv_bytes + 2.0 * T * H, stream, [&] {
      return dfl::launch_conv(u, coef1, L.mlp_base, 1, T, H, G, c.conv_group, x, x, stream);
    }));
  }
  if (tr) {
    DFL_TRY(snap(tr->x_out, x, rowsH, stream));
    if (next_gamma && !head_rows) DFL_TRY(snap(tr->n_next, n, rowsH, stream));
  }
  return DFL_OK;
}

}  // namespace


extern "C" {

const char* dfl_last_error(void) { return g_err.c_str(); }

int dfl_drafter_load(const dfl_config* cfg, const dfl_weights* w, hipStream_t stream,
                     dfl_drafter** out) {
  DFL_REQUIRE(out, DFL_E_INVALID, "out is NULL");
  *out = nullptr;
  DFL_TRY(check_config(cfg));
  DFL_REQUIRE(w && w->fc && w->hidden_norm && w->norm && w->sel_proj && w->pred && w->succ && w->layers,
              DFL_E_INVALID, "a drafter weight pointer is NULL");
  const dfl_config& c = *cfg;
  const bool q4 = w->q4_layers != nullptr;
  for (int i = 0; i < c.layers; ++i) {
    const dfl_layer_weights& L = w->layers[i];
    DFL_REQUIRE(L.input_norm && L.post_norm && L.q_norm && L.k_norm && L.attn_base && L.attn_kproj && L.mlp_base &&
                    L.mlp_kproj && (q4 || (L.q_proj && L.k_proj && L.v_proj && L.o_proj && L.gate_proj &&
                                           L.up_proj && L.down_proj)),
                DFL_E_INVALID, "layer %d has a NULL weight pointer", i);
    if (q4) {
      const dfl_q4_layer& Q = w->q4_layers[i];
      for (const dfl_q4_weight* qw : {&Q.q_proj, &Q.k_proj, &Q.v_proj, &Q.o_proj, &Q.gate_proj, &Q.up_proj,
                                      &Q.down_proj})
        DFL_REQUIRE(qw->packed && qw->scales && qw->biases, DFL_E_INVALID, "layer %d has a NULL 4-bit weight", i);
    }
  }
  const size_t H = c.hidden, D = c.head_dim, NH = c.heads, NKV = c.kv_heads, F = c.intermediate;
  const size_t ng = H / c.conv_group, V = c.vocab, R = c.rank;
  const size_t qkvw = (NH + 2 * NKV) * D;
  auto tiled = [](size_t n, size_t k) { return dfl::tiled_weight_elems((int)n, (int)k); };
  // owned arena: projections in the tile-contiguous layout, everything else as given
  Carver cv(nullptr);
  auto sz_fc = cv.off; cv.take<uint16_t>(tiled(H, c.n_taps * H));
  auto sz_hn = cv.off; cv.take<uint16_t>(H);
  auto sz_nm = cv.off; cv.take<uint16_t>(H);
  auto sz_sp = cv.off; cv.take<uint16_t>(tiled(R, H));
  auto sz_pr = cv.off; cv.take<uint16_t>(V * R);
  auto sz_sc = cv.off; cv.take<uint16_t>(V * R);
  const size_t layer0 = cv.off;
  size_t off_in = 0, off_post, off_qn, off_kn, off_qkv, off_o, off_gu, off_dn, off_ab, off_ak, off_mb, off_mk, off_kv;
  {
    Carver lc(nullptr);
    off_in = lc.off; lc.take<uint16_t>(H);
    off_post = lc.off; lc.take<uint16_t>(H);
    off_qn = lc.off; lc.take<uint16_t>(D);
    off_kn = lc.off; lc.take<uint16_t>(D);
    if (q4) {  // 32-bit words of 4-bit blocks
      off_qkv = lc.off; lc.take<uint32_t>(dfl::q4_tiled_words((int)qkvw, (int)H));
      off_o = lc.off; lc.take<uint32_t>(dfl::q4_tiled_words((int)H, (int)(NH * D)));
      off_gu = lc.off; lc.take<uint32_t>(dfl::q4_tiled_words((int)(2 * F), (int)H));
      off_dn = lc.off; lc.take<uint32_t>(dfl::q4_tiled_words((int)H, (int)F));
    } else {
      off_qkv = lc.off; lc.take<uint16_t>(tiled(qkvw, H));
      off_o = lc.off; lc.take<uint16_t>(tiled(H, NH * D));
      off_gu = lc.off; lc.take<uint16_t>(tiled(2 * F, H));
      off_dn = lc.off; lc.take<uint16_t>(tiled(H, F));
    }
    off_ab = lc.off; lc.take<uint16_t>(4 * H);
    off_ak = lc.off; lc.take<uint16_t>(tiled(4 * ng, H));
    off_mb = lc.off; lc.take<uint16_t>(4 * H);
    off_mk = lc.off; lc.take<uint16_t>(tiled(4 * ng, H));
    if (q4) {
      off_kv = lc.off; lc.take<uint32_t>(dfl::q4_tiled_words((int)(2 * NKV * D), (int)H));
    } else {
      off_kv = lc.off; lc.take<uint16_t>(tiled(2 * NKV * D, H));
    }
    cv.off += lc.off * c.layers;
  }
  const size_t per_layer = (cv.off - layer0) / c.layers;
  dfl_drafter* d = new (std::nothrow) dfl_drafter();
  DFL_REQUIRE(d, DFL_E_NOMEM, "host allocation failed");
  d->cfg = c;
  d->cfg.tap_layer_ids = nullptr;
  d->cfg.sliding_layers = nullptr;
  d->q4 = q4;
  d->window.assign(c.layers, 0);
  for (int i = 0; i < c.layers; ++i)
    if (c.sliding_window > 0 && (!c.sliding_layers || c.sliding_layers[i])) d->window[i] = c.sliding_window;
  if (hipMalloc(&d->arena, cv.off) != hipSuccess) {
    delete d;
    return fail(DFL_E_NOMEM, "hipMalloc of %zu bytes for the drafter weights failed", cv.off);
  }
  // row-major staging for the fused projections (q|k|v, gate/up interleaved, k|v)
  const size_t stage_elems = std::max({qkvw * H, 2 * F * H, 2 * NKV * D * H});
  uint16_t* stage = nullptr;
  if (hipMalloc(reinterpret_cast<void**>(&stage), stage_elems * 2) != hipSuccess) {
    (void)hipFree(d->arena);
    delete d;
    return fail(DFL_E_NOMEM, "hipMalloc of %zu bytes of load staging failed", stage_elems * 2);
  }
  char* A = static_cast<char*>(d->arena);
  auto at = [&](size_t off) { return reinterpret_cast<uint16_t*>(A + off); };
  d->fc = at(sz_fc);
  d->hidden_norm = at(sz_hn);
  d->norm = at(sz_nm);
  d->sel_proj = at(sz_sp);
  d->pred = at(sz_pr);
  d->succ = at(sz_sc);
  int rc = DFL_OK;
  auto cp = [&](void* dst, const void* src, size_t n) {
    if (rc == DFL_OK) {
      hipError_t e = hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, stream);
      if (e != hipSuccess) rc = fail(DFL_E_DEVICE, "hipMemcpyAsync: %s", hipGetErrorString(e));
    }
  };
  auto cp2d = [&](void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height) {
    if (rc == DFL_OK) {
      hipError_t e = hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, hipMemcpyDeviceToDevice, stream);
      if (e != hipSuccess) rc = fail(DFL_E_DEVICE, "hipMemcpy2DAsync: %s", hipGetErrorString(e));
    }
  };
  auto tile = [&](const uint16_t* src, size_t n, size_t k, uint16_t* dst) {
    if (rc == DFL_OK) {
      hipError_t e = dfl::launch_tile_weights(src, (int)n, (int)k, dst, stream);
      if (e != hipSuccess) rc = fail(DFL_E_DEVICE, "weight tiling: %s", hipGetErrorString(e));
    }
  };
  auto tile4 = [&](const uint32_t* q, const void* sc, const void* bi, size_t n, size_t k, uint32_t* dst) {
    if (rc == DFL_OK) {
      hipError_t e = dfl::launch_tile_q4(q, static_cast<const uint16_t*>(sc), static_cast<const uint16_t*>(bi),
                                         (int)n, (int)k, dst, stream);
      if (e != hipSuccess) rc = fail(DFL_E_DEVICE, "4-bit weight tiling: %s", hipGetErrorString(e));
    }
  };
  // 4-bit staging of the fused K = H projections: packed words, then scales, then biases,
  // each row-major over the fused rows (fits the bf16 staging: 9/16 of its bytes)
  const size_t nmax = std::max({qkvw, 2 * F, 2 * NKV * D});
  uint32_t* sq = reinterpret_cast<uint32_t*>(stage);
  uint16_t* ss = reinterpret_cast<uint16_t*>(sq + nmax * H / 8);
  uint16_t* sb = ss + nmax * H / 64;
  // rows [row0, row0 + n) of the staging from one K = H weight
  auto q4_rows = [&](const dfl_q4_weight& qw, size_t row0, size_t n) {
    cp(sq + row0 * H / 8, qw.packed, n * H / 2);
    cp(ss + row0 * H / 64, qw.scales, n * H / 32);
    cp(sb + row0 * H / 64, qw.biases, n * H / 32);
  };
  // gate (row0 = 0) or up (row0 = 16) into the staging interleaved per 16 rows
  auto q4_interleave = [&](const dfl_q4_weight& qw, size_t row0) {
    cp2d(sq + row0 * H / 8, 32 * H / 2, qw.packed, 16 * H / 2, 16 * H / 2, F / 16);
    cp2d(ss + row0 * H / 64, 32 * H / 32, qw.scales, 16 * H / 32, 16 * H / 32, F / 16);
    cp2d(sb + row0 * H / 64, 32 * H / 32, qw.biases, 16 * H / 32, 16 * H / 32, F / 16);
  };
  tile(w->fc, H, c.n_taps * H, d->fc);
  cp(d->hidden_norm, w->hidden_norm, H * 2);
  cp(d->norm, w->norm, H * 2);
  tile(w->sel_proj, R, H, d->sel_proj);
  cp(d->pred, w->pred, V * R * 2);
  cp(d->succ, w->succ, V * R * 2);
  d->layers.resize(c.layers);
  for (int i = 0; i < c.layers; ++i) {
    const dfl_layer_weights& s = w->layers[i];
    const size_t lb = layer0 + per_layer * i;
    LayerBuf& L = d->layers[i];
    L.in_norm = at(lb + off_in);
    L.post_norm = at(lb + off_post);
    L.q_norm = at(lb + off_qn);
    L.k_norm = at(lb + off_kn);
    L.attn_base = at(lb + off_ab);
    L.attn_kproj = at(lb + off_ak);
    L.mlp_base = at(lb + off_mb);
    L.mlp_kproj = at(lb + off_mk);
    cp(L.in_norm, s.input_norm, H * 2);
    cp(L.post_norm, s.post_norm, H * 2);
    cp(L.q_norm, s.q_norm, D * 2);
    cp(L.k_norm, s.k_norm, D * 2);
    cp(L.attn_base, s.attn_base, 4 * H * 2);
    tile(s.attn_kproj, 4 * ng, H, L.attn_kproj);
    cp(L.mlp_base, s.mlp_base, 4 * H * 2);
    tile(s.mlp_kproj, 4 * ng, H, L.mlp_kproj);
    if (q4) {
      const dfl_q4_layer& Q = w->q4_layers[i];
      auto at4 = [&](size_t off) { return reinterpret_cast<uint32_t*>(A + off); };
      L.qkv = L.o = L.gateup = L.down = L.kv_ctx = nullptr;
      L.qkv_q4 = at4(lb + off_qkv);
      L.o_q4 = at4(lb + off_o);
      L.gateup_q4 = at4(lb + off_gu);
      L.down_q4 = at4(lb + off_dn);
      L.kv_ctx_q4 = at4(lb + off_kv);
      q4_rows(Q.q_proj, 0, NH * D);
      q4_rows(Q.k_proj, NH * D, NKV * D);
      q4_rows(Q.v_proj, (NH + NKV) * D, NKV * D);
      tile4(sq, ss, sb, qkvw, H, L.qkv_q4);
      tile4(Q.o_proj.packed, Q.o_proj.scales, Q.o_proj.biases, H, NH * D, L.o_q4);
      q4_interleave(Q.gate_proj, 0);
      q4_interleave(Q.up_proj, 16);
      tile4(sq, ss, sb, 2 * F, H, L.gateup_q4);
      tile4(Q.down_proj.packed, Q.down_proj.scales, Q.down_proj.biases, H, F, L.down_q4);
      q4_rows(Q.k_proj, 0, NKV * D);
      q4_rows(Q.v_proj, NKV * D, NKV * D);
      tile4(sq, ss, sb, 2 * NKV * D, H, L.kv_ctx_q4);
      continue;
    }
    L.qkv = at(lb + off_qkv);
    L.o = at(lb + off_o);
    L.gateup = at(lb + off_gu);
    L.down = at(lb + off_dn);
    L.kv_ctx = at(lb + off_kv);
    cp(stage, s.q_proj, NH * D * H * 2);
    cp(stage + NH * D * H, s.k_proj, NKV * D * H * 2);
    cp(stage + (NH + NKV) * D * H, s.v_proj, NKV * D * H * 2);
    tile(stage, qkvw, H, L.qkv);
    tile(s.o_proj, H, NH * D, L.o);
    // gate/up interleaved per 16 rows: [gate 16 | up 16] ...
    cp2d(stage, 32 * H * 2, s.gate_proj, 16 * H * 2, 16 * H * 2, F / 16);
    cp2d(stage + 16 * H, 32 * H * 2, s.up_proj, 16 * H * 2, 16 * H * 2, F / 16);
    tile(stage, 2 * F, H, L.gateup);
    tile(s.down_proj, H, F, L.down);
    cp(stage, s.k_proj, NKV * D * H * 2);
    cp(stage + NKV * D * H, s.v_proj, NKV * D * H * 2);
    tile(stage, 2 * NKV * D, H, L.kv_ctx);
  }
  if (rc == DFL_OK) {
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) rc = fail(DFL_E_DEVICE, "hipStreamSynchronize: %s", hipGetErrorString(e));
  }
  (void)hipFree(stage);
  if (rc != DFL_OK) {
    (void)hipFree(d->arena);
    delete d;
    return rc;
  }
  *out = d;
  return DFL_OK;
}

void dfl_drafter_free(dfl_drafter* d) {
  if (!d) return;
  for (auto& t : d->timed) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  for (auto e : d->pool) (void)hipEventDestroy(e);
  if (d->arena) (void)hipFree(d->arena);
  if (d->head) (void)hipFree(d->head);
  if (d->head_ids) (void)hipFree(d->head_ids);
  delete d;
}

int dfl_bind_target(dfl_drafter* d, const dfl_bf16* lm_head, const int32_t* vocab_ids, int n_vocab,
                    hipStream_t stream) {
  DFL_REQUIRE(d && lm_head, DFL_E_INVALID, "NULL argument");
  const int V = d->cfg.vocab, H = d->cfg.hidden;
  if (d->head_src) {
    DFL_REQUIRE(d->head_src == lm_head, DFL_E_INVALID, "a different target head is already bound");
    DFL_REQUIRE(vocab_ids ? n_vocab == d->head_cols && d->head_ids : d->head_ids == nullptr, DFL_E_INVALID,
                "the target is already bound with a different vocabulary");
    return DFL_OK;
  }
  int cols = V;
  if (vocab_ids) {
    DFL_REQUIRE(n_vocab >= d->cfg.top_k && n_vocab <= V, DFL_E_SHAPE, "draft vocabulary of %d ids outside [top_k=%d, V=%d]",
                n_vocab, d->cfg.top_k, V);
    std::set<int> seen;
    for (int i = 0; i < n_vocab; ++i) {
      DFL_REQUIRE(vocab_ids[i] >= 0 && vocab_ids[i] < V, DFL_E_INVALID, "draft vocabulary id %d outside [0, %d)",
                  vocab_ids[i], V);
      DFL_REQUIRE(seen.insert(vocab_ids[i]).second, DFL_E_INVALID, "draft vocabulary id %d repeats", vocab_ids[i]);
    }
    cols = n_vocab;
  }
  void* buf = nullptr;
  void* ids = nullptr;
  // When the head's rows fill whole 256-row tiles, the selector projection's (already tiled)
  // rows follow as one more tile, so a single launch writes the logits and z.
  const bool with_sel = cols % dfl::kGemmTileN == 0;
  const size_t head_bytes = dfl::tiled_weight_elems(cols, H) * sizeof(uint16_t);
  const size_t sel_bytes = with_sel ? dfl::tiled_weight_elems(d->cfg.rank, H) * sizeof(uint16_t) : 0;
  const size_t bytes = head_bytes + sel_bytes;
  if (hipMalloc(&buf, bytes) != hipSuccess ||
      (vocab_ids && hipMalloc(&ids, (size_t)cols * sizeof(int32_t)) != hipSuccess)) {
    (void)hipGetLastError();
    if (buf) (void)hipFree(buf);
    return fail(DFL_E_NOMEM, "could not allocate the bound head (%zu bytes)", bytes);
  }
  hipError_t e = hipSuccess;
  if (ids) e = hipMemcpyAsync(ids, vocab_ids, (size_t)cols * sizeof(int32_t), hipMemcpyHostToDevice, stream);
  if (e == hipSuccess)
    e = dfl::launch_tile_weights(lm_head, cols, H, static_cast<uint16_t*>(buf), stream, static_cast<int32_t*>(ids));
  if (e == hipSuccess && with_sel)
    e = hipMemcpyAsync(static_cast<char*>(buf) + head_bytes, d->sel_proj, sel_bytes, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    (void)hipFree(buf);
    if (ids) (void)hipFree(ids);
    return fail(DFL_E_DEVICE, "binding the head: %s", hipGetErrorString(e));
  }
  d->head = static_cast<uint16_t*>(buf);
  d->head_src = lm_head;
  d->head_cols = cols;
  d->head_sel = with_sel;
  d->head_ids = static_cast<int32_t*>(ids);
  return DFL_OK;
}

size_t dfl_context_workspace_bytes(const dfl_drafter* d, int B, int L) {
  if (!d || B <= 0 || L <= 0) return 0;
  return ctx_layout(d->cfg, B, L).total;
}

int dfl_context_materialize(dfl_drafter* d, const dfl_bf16* taps, int B, int L, int row_offset,
                            int Lcap, dfl_bf16* const* K, dfl_bf16* const* V, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  return dfl_context_materialize_traced(d, taps, B, L, row_offset, Lcap, K, V, ws, ws_bytes, nullptr, stream);
}

int dfl_context_materialize_traced(dfl_drafter* d, const dfl_bf16* taps, int B, int L, int row_offset,
                                   int Lcap, dfl_bf16* const* K, dfl_bf16* const* V, void* ws,
                                   size_t ws_bytes, const dfl_context_trace* trace, hipStream_t stream) {
  DFL_REQUIRE(d && taps && K && V && ws, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(B > 0 && L > 0 && row_offset >= 0 && Lcap > 0, DFL_E_INVALID, "B, L, Lcap must be positive");
  DFL_REQUIRE((int64_t)row_offset + L <= Lcap, DFL_E_SHAPE, "row_offset %d + L %d exceeds Lcap %d", row_offset, L,
              Lcap);
  DFL_REQUIRE((int64_t)B * L <= (1 << 30), DFL_E_SHAPE, "B*L too large");
  const dfl_config& c = d->cfg;
  for (int i = 0; i < c.layers; ++i) DFL_REQUIRE(K[i] && V[i], DFL_E_INVALID, "K/V pointer of layer %d is NULL", i);
  DFL_REQUIRE(aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  const CtxLayout lay = ctx_layout(c, B, L);
  DFL_REQUIRE(ws_bytes >= lay.total, DFL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, lay.total);
  char* W = static_cast<char*>(ws);
  uint16_t* craw = reinterpret_cast<uint16_t*>(W + lay.craw);
  uint16_t* cc = reinterpret_cast<uint16_t*>(W + lay.c);
  uint16_t* kv = reinterpret_cast<uint16_t*>(W + lay.kv);
  float* part = reinterpret_cast<float*>(W + lay.partial);
  const int M = B * L, H = c.hidden, kvw = 2 * c.kv_heads * c.head_dim;
  const dfl::GemmPlan pfc = dfl::plan_gemm(M, H, c.n_taps * H);
  DFL_TRY(timed(d, DFL_K_GEMM_CONTEXT, gemm_bytes(M, H, c.n_taps * H, dfl::EPI_BF16), stream, [&] {
    return dfl::launch_gemm(pfc, taps, c.n_taps * H, d->fc, true, M, H, c.n_taps * H, dfl::EPI_BF16, craw, H, nullptr,
                            0, 0, part, stream);
  }));
  if (trace) DFL_TRY(snap(trace->fc_out, craw, (size_t)M * H * sizeof(uint16_t), stream));
  DFL_TRY(timed(d, DFL_K_RMSNORM, 4.0 * M * H, stream, [&] {
    return dfl::launch_rms_norm(craw, H, M, H, d->hidden_norm, c.rms_eps, cc, H, 1, 1, 0, stream);
  }));
  if (trace) DFL_TRY(snap(trace->c, cc, (size_t)M * H * sizeof(uint16_t), stream));
  const dfl::GemmPlan pkv = dfl::plan_gemm(M, kvw, H);
  for (int i = 0; i < c.layers; ++i) {
    const LayerBuf& Lb = d->layers[i];
    DFL_TRY(timed(d, DFL_K_GEMM_CONTEXT, gemm_bytes(M, kvw, H, dfl::EPI_BF16, d->q4), stream, [&] {
      return dfl::launch_gemm(pkv, cc, H, wref(Lb.kv_ctx, Lb.kv_ctx_q4), M, kvw, H, dfl::EPI_BF16, kv, kvw, nullptr,
                              0, 0, part, stream);
    }));
    if (trace && trace->layer == i) DFL_TRY(snap(trace->kv, kv, (size_t)M * kvw * sizeof(uint16_t), stream));
    DFL_TRY(timed(d, DFL_K_ROPE, 4.0 * M * kvw, stream, [&] {
      return dfl::launch_context_kv_store(kv, B, L, c.kv_heads, c.head_dim, Lb.k_norm, c.rms_eps, c.rope_theta,
                                          row_offset, Lcap, K[i], V[i], stream);
    }));
  }
  return DFL_OK;
}

size_t dfl_context_append_workspace_bytes(const dfl_drafter* d, int B, int rows) {
  if (!d || B <= 0 || rows <= 0) return 0;
  return ctx_layout(d->cfg, 1, rows).total + align_up((size_t)(2 * B + 1) * sizeof(int32_t));
}

int dfl_context_append(dfl_drafter* d, const dfl_bf16* taps, const int32_t* row_offsets, const int32_t* starts,
                       int B, int Lcap, dfl_bf16* const* K, dfl_bf16* const* V, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return dfl_context_append_traced(d, taps, row_offsets, starts, B, Lcap, K, V, ws, ws_bytes, nullptr, stream);
}

int dfl_context_append_traced(dfl_drafter* d, const dfl_bf16* taps, const int32_t* row_offsets,
                              const int32_t* starts, int B, int Lcap, dfl_bf16* const* K, dfl_bf16* const* V,
                              void* ws, size_t ws_bytes, const dfl_context_trace* trace, hipStream_t stream) {
  DFL_REQUIRE(d && taps && row_offsets && starts && K && V && ws, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(B > 0 && Lcap > 0, DFL_E_INVALID, "B and Lcap must be positive");
  DFL_REQUIRE(row_offsets[0] == 0, DFL_E_SHAPE, "row_offsets[0] must be 0");
  for (int b = 0; b < B; ++b) {
    const int n = row_offsets[b + 1] - row_offsets[b];
    DFL_REQUIRE(n >= 0, DFL_E_SHAPE, "row_offsets decrease at request %d", b);
    DFL_REQUIRE(starts[b] >= 0 && (int64_t)starts[b] + n <= Lcap, DFL_E_SHAPE,
                "request %d: rows [%d, %d) outside the cache of %d rows", b, starts[b], starts[b] + n, Lcap);
  }
  const int rows = row_offsets[B];
  if (rows == 0) return DFL_OK;
  DFL_REQUIRE(rows <= (1 << 30), DFL_E_SHAPE, "too many rows");
  const dfl_config& c = d->cfg;
  for (int i = 0; i < c.layers; ++i) DFL_REQUIRE(K[i] && V[i], DFL_E_INVALID, "K/V pointer of layer %d is NULL", i);
  DFL_REQUIRE((int64_t)Lcap * c.kv_heads * c.head_dim < (int64_t(1) << 31), DFL_E_SHAPE, "Lcap too large");
  DFL_REQUIRE(aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  const size_t need = dfl_context_append_workspace_bytes(d, B, rows);
  DFL_REQUIRE(ws_bytes >= need, DFL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const CtxLayout lay = ctx_layout(c, 1, rows);
  char* W = static_cast<char*>(ws);
  uint16_t* craw = reinterpret_cast<uint16_t*>(W + lay.craw);
  uint16_t* cc = reinterpret_cast<uint16_t*>(W + lay.c);
  uint16_t* kv = reinterpret_cast<uint16_t*>(W + lay.kv);
  float* part = reinterpret_cast<float*>(W + lay.partial);
  int32_t* offs_d = reinterpret_cast<int32_t*>(W + lay.total);
  int32_t* starts_d = offs_d + (B + 1);
  DFL_HIP(hipMemcpyAsync(offs_d, row_offsets, (size_t)(B + 1) * sizeof(int32_t), hipMemcpyHostToDevice, stream));
  DFL_HIP(hipMemcpyAsync(starts_d, starts, (size_t)B * sizeof(int32_t), hipMemcpyHostToDevice, stream));
  const int M = rows, H = c.hidden, kvw = 2 * c.kv_heads * c.head_dim;
  const dfl::GemmPlan pfc = dfl::plan_gemm(M, H, c.n_taps * H);
  DFL_TRY(timed(d, DFL_K_GEMM_CONTEXT, gemm_bytes(M, H, c.n_taps * H, dfl::EPI_BF16), stream, [&] {
    return dfl::launch_gemm(pfc, taps, c.n_taps * H, d->fc, true, M, H, c.n_taps * H, dfl::EPI_BF16, craw, H, nullptr,
                            0, 0, part, stream);
  }));
  if (trace) DFL_TRY(snap(trace->fc_out, craw, (size_t)M * H * sizeof(uint16_t), stream));
  DFL_TRY(timed(d, DFL_K_RMSNORM, 4.0 * M * H, stream, [&] {
    return dfl::launch_rms_norm(craw, H, M, H, d->hidden_norm, c.rms_eps, cc, H, 1, 1, 0, stream);
  }));
  if (trace) DFL_TRY(snap(trace->c, cc, (size_t)M * H * sizeof(uint16_t), stream));
  const dfl::GemmPlan pkv = dfl::plan_gemm(M, kvw, H);
  for (int i = 0; i < c.layers; ++i) {
    const LayerBuf& Lb = d->layers[i];
    DFL_TRY(timed(d, DFL_K_GEMM_CONTEXT, gemm_bytes(M, kvw, H, dfl::EPI_BF16, d->q4), stream, [&] {
      return dfl::launch_gemm(pkv, cc, H, wref(Lb.kv_ctx, Lb.kv_ctx_q4), M, kvw, H, dfl::EPI_BF16, kv, kvw, nullptr,
                              0, 0, part, stream);
    }));
    if (trace && trace->layer == i) DFL_TRY(snap(trace->kv, kv, (size_t)M * kvw * sizeof(uint16_t), stream));
    DFL_TRY(timed(d, DFL_K_ROPE, 4.0 * M * kvw, stream, [&] {
      return dfl::launch_context_kv_store_ragged(kv, M, B, c.kv_heads, c.head_dim, Lb.k_norm, c.rms_eps, c.rope_theta,
                                                 offs_d, starts_d, Lcap, K[i], V[i], stream);
    }));
  }
  return DFL_OK;
}

size_t dfl_draft_workspace_bytes(const dfl_drafter* d, int B, int G, int Lmax) {
  if (!d || B <= 0 || G < 2 || Lmax < 0) return 0;
  return draft_layout(d->cfg, B, G, Lmax).total;
}

int dfl_draft_block(dfl_drafter* d, const dfl_bf16* embeds, const int32_t* anchors, int B, int G,
                    const dfl_bf16* const* K, const dfl_bf16* const* V, int Lcap, int Lmax,
                    const int32_t* ctx_len, const int32_t* pos0, const dfl_bf16* lm_head,
                    int32_t* tokens, float* logits_out, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return dfl_draft_block_traced(d, embeds, anchors, B, G, K, V, Lcap, Lmax, ctx_len, pos0, lm_head, tokens,
                                logits_out, ws, ws_bytes, nullptr, stream);
}

int dfl_draft_block_traced(dfl_drafter* d, const dfl_bf16* embeds, const int32_t* anchors, int B, int G,
                           const dfl_bf16* const* K, const dfl_bf16* const* V, int Lcap, int Lmax,
                           const int32_t* ctx_len, const int32_t* pos0, const dfl_bf16* lm_head,
                           int32_t* tokens, float* logits_out, void* ws, size_t ws_bytes,
                           const dfl_trace* trace, hipStream_t stream) {
  DFL_REQUIRE(d && embeds && anchors && ctx_len && pos0 && tokens && ws, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(lm_head || d->head, DFL_E_INVALID, "lm_head is NULL and no target head is bound");
  // the bound (tile-contiguous) copy serves a NULL head or the pointer it was bound from
  const bool bound_head = d->head && (!lm_head || lm_head == d->head_src);
  const dfl_config& c = d->cfg;
  DFL_REQUIRE(B > 0, DFL_E_INVALID, "B must be positive");
  DFL_REQUIRE(G >= 2 && G <= c.block_size, DFL_E_UNSUPPORTED, "G=%d outside [2, block_size=%d]", G, c.block_size);
  DFL_REQUIRE(Lmax >= 0 && Lmax <= Lcap, DFL_E_SHAPE, "Lmax %d must be in [0, Lcap=%d]", Lmax, Lcap);
  DFL_REQUIRE((int64_t)Lcap * d->cfg.kv_heads * d->cfg.head_dim < (int64_t(1) << 31), DFL_E_SHAPE,
              "one request's K/V (Lcap %d x %d x %d) must hold fewer than 2^31 elements", Lcap,
              d->cfg.kv_heads, d->cfg.head_dim);
  DFL_REQUIRE((int64_t)B * G * std::max(c.vocab, c.intermediate * 2) < (1ll << 31), DFL_E_SHAPE, "B*G too large");
  if (Lmax > 0) {
    DFL_REQUIRE(K && V, DFL_E_INVALID, "K/V arrays are NULL");
    for (int i = 0; i < c.layers; ++i) DFL_REQUIRE(K[i] && V[i], DFL_E_INVALID, "K/V of layer %d is NULL", i);
  }
  DFL_REQUIRE(aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  const DraftLayout lay = draft_layout(c, B, G, Lmax);
  DFL_REQUIRE(ws_bytes >= lay.total, DFL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, lay.total);

  const int H = c.hidden, S = G - 1, N = B * S;
  // the head's columns: the bound draft vocabulary's rows when it is used, else the vocabulary
  const int V_ = bound_head ? d->head_cols : c.vocab, R = c.rank, Kc = c.top_k;
  const int32_t* id_map = bound_head ? d->head_ids : nullptr;
  char* W = static_cast<char*>(ws);
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(W + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(W + off); };
  uint16_t *x = u16(lay.x), *h = u16(lay.h);
  float *z = f32(lay.z), *unary = f32(lay.unary), *scores = f32(lay.scores);
  float* logits = logits_out ? logits_out : f32(lay.logits);
  int32_t* cand = reinterpret_cast<int32_t*>(W + lay.cand);
  float* part = f32(lay.partial);
  // A bound head holding the selector projection's rows after its own computes z in the same
  // launch: columns [0, V_) go to the logits, the R after them to z.
  const bool head_sel = bound_head && d->head_sel;
  const int NHd = V_ + (head_sel ? R : 0);
  const dfl::GemmPlan p_head = dfl::plan_gemm(N, NHd, H, true), p_sel = dfl::plan_gemm(N, R, H);
  // An unsplit head also writes every 256-column tile's row maxima, which lets the top-K
  // read only the few tiles that can hold a candidate; a split head leaves them to a pass
  // over the logits.
  const bool tiles_fused = p_head.splits == 1;
  // When nobody else reads the logits, a head on 256-row tiles leaves out each row's tiles
  // that cannot hold one of its top kTileBoundSlots (launch_gemm's tile_bound), and the top-K
  // reads only tiles above the same bound; the last layer's finish clears the slots.  (On the
  // 128-row tiles the bound's device-scope round trip per workgroup costs more than the
  // stores it saves.)
  uint32_t* tbound = tiles_fused && p_head.bm == 256 && !logits_out && !trace && Kc <= dfl::kTileBoundSlots
                         ? reinterpret_cast<uint32_t*>(W + lay.tbound)
                         : nullptr;

  const uint16_t* xin = embeds;
  for (int li = 0; li < c.layers; ++li) {
    const uint16_t* Kl = Lmax > 0 ? K[li] : nullptr;
    const uint16_t* Vl = Lmax > 0 ? V[li] : nullptr;
    const bool last = li + 1 == c.layers;
    // the last layer's finish applies the final norm to rows 1..G-1, packed into h for the head
    const uint16_t* next_gamma = last ? d->norm : d->layers[li + 1].in_norm;
    DFL_TRY(run_layer(d, li, xin, x, B, G, Kl, Vl, Lcap, Lmax, ctx_len, pos0, W, lay, li > 0, next_gamma, stream,
                      last ? h : nullptr, trace, last ? tbound : nullptr));
    xin = x;
  }
  if (trace) DFL_TRY(snap(trace->h, h, (size_t)N * H * sizeof(uint16_t), stream));
  float* tmax = f32(lay.tmax);
  // on 256-row tiles the head reads a fragment-order copy of h (counted with the projection)
  const bool head_tiled = dfl::gemm_takes_tiled_a(p_head, false) && lay.atile_elems >= dfl::tiled_rows_elems(N, H);
  uint16_t* htile = reinterpret_cast<uint16_t*>(W + lay.atile);
  DFL_TRY(timed(d, DFL_K_GEMM_HEAD, gemm_bytes(N, NHd, H, dfl::EPI_F32), stream, [&] {
    if (head_tiled) {
      const hipError_t e = dfl::launch_tile_rows(h, H, N, H, htile, stream);
      if (e != hipSuccess) return e;
    }
    return dfl::launch_gemm(p_head, head_tiled ? htile : h, H, bound_head ? d->head : lm_head, bound_head, N, NHd,
                            H, dfl::EPI_F32, logits, V_, head_sel ? z : nullptr, R, V_, part, stream,
                            tiles_fused ? tmax : nullptr, tbound, head_tiled);
  }));
  if (!head_sel) {
    DFL_TRY(timed(d, DFL_K_GEMM_SELPROJ, gemm_bytes(N, R, H, dfl::EPI_F32), stream, [&] {
      return dfl::launch_gemm(p_sel, h, H, d->sel_proj, true, N, R, H, dfl::EPI_F32, z, R, nullptr, 0, 0, part,
                              stream);
    }));
  }
  if (trace) DFL_TRY(snap(trace->z, z, (size_t)N * R * sizeof(float), stream));
  // with the tile maxima in hand, the selection (top-k, edge scores, walk) is one launch when
  // its per-request state fits one workgroup's LDS
  const bool fused_select = tiles_fused && dfl::select_tokens_fits(S, Kc, R);
  if (fused_select) {
    DFL_TRY(timed(d, DFL_K_SELECT, 4.0 * N * (V_ / dfl::kGemmTileN + Kc * dfl::kGemmTileN) + 4.0 * N * R +
                                       2.0 * 2 * N * Kc * R + 4.0 * N * Kc * (Kc + 2),
                  stream, [&] {
      return dfl::launch_select_tokens(logits, tmax, B, S, V_, Kc, id_map, z, R, anchors, d->pred, d->succ, c.vocab,
                                       cand, unary, scores, tokens, stream, tbound);
    }));
    if (trace) {
      DFL_TRY(snap(trace->tile_max, tmax, (size_t)N * ((V_ + dfl::kGemmTileN - 1) / dfl::kGemmTileN) * sizeof(float),
                   stream));
      DFL_TRY(snap(trace->cand, cand, (size_t)N * Kc * sizeof(int32_t), stream));
      DFL_TRY(snap(trace->unary, unary, (size_t)N * Kc * sizeof(float), stream));
      DFL_TRY(snap(trace->scores, scores, (size_t)N * Kc * Kc * sizeof(float), stream));
    }
    return DFL_OK;
  }
  DFL_TRY(timed(d, DFL_K_TOPK, tiles_fused ? 4.0 * N * (V_ / dfl::kGemmTileN + Kc * dfl::kGemmTileN) : 4.0 * N * V_,
                stream, [&] {
    return tiles_fused ? dfl::launch_topk_tiles(logits, N, V_, Kc, tmax, cand, unary, stream, id_map, tbound)
                       : dfl::launch_topk(logits, N, V_, Kc, cand, unary, tmax, stream, id_map);
  }));
  if (trace) {
    DFL_TRY(snap(trace->tile_max, tmax, (size_t)N * ((V_ + dfl::kGemmTileN - 1) / dfl::kGemmTileN) * sizeof(float),
                 stream));
    DFL_TRY(snap(trace->cand, cand, (size_t)N * Kc * sizeof(int32_t), stream));
    DFL_TRY(snap(trace->unary, unary, (size_t)N * Kc * sizeof(float), stream));
  }
  DFL_TRY(timed(d, DFL_K_SCORE_EDGES, 4.0 * N * Kc * (2 * R + Kc + 2) + 4.0 * N * R, stream, [&] {
    return dfl::launch_score_edges(cand, unary, z, anchors, B, S, Kc, R, d->pred, d->succ, c.vocab, scores,
                                   stream);
  }));
  if (trace) DFL_TRY(snap(trace->scores, scores, (size_t)N * Kc * Kc * sizeof(float), stream));
  DFL_TRY(timed(d, DFL_K_SELECT_PATH, 4.0 * N * Kc * (Kc + 1), stream, [&] {
    return dfl::launch_select_path(scores, cand, B, S, Kc, tokens, stream);
  }));
  return DFL_OK;
}

int dfl_block_layer(dfl_drafter* d, int layer, const dfl_bf16* x_in, dfl_bf16* x_out, int B, int G,
                    const dfl_bf16* K, const dfl_bf16* V, int Lcap, int Lmax, const int32_t* ctx_len,
                    const int32_t* pos0, void* ws, size_t ws_bytes, hipStream_t stream) {
  DFL_REQUIRE(d && x_in && x_out && ctx_len && pos0 && ws, DFL_E_INVALID, "NULL argument");
  const dfl_config& c = d->cfg;
  DFL_REQUIRE(layer >= 0 && layer < c.layers, DFL_E_INVALID, "layer %d outside [0, %d)", layer, c.layers);
  DFL_REQUIRE(B > 0, DFL_E_INVALID, "B must be positive");
  DFL_REQUIRE(G >= 2 && G <= c.block_size, DFL_E_UNSUPPORTED, "G=%d outside [2, block_size=%d]", G, c.block_size);
  DFL_REQUIRE(Lmax >= 0 && Lmax <= Lcap, DFL_E_SHAPE, "Lmax %d must be in [0, Lcap=%d]", Lmax, Lcap);
  DFL_REQUIRE((int64_t)Lcap * d->cfg.kv_heads * d->cfg.head_dim < (int64_t(1) << 31), DFL_E_SHAPE,
              "one request's K/V (Lcap %d x %d x %d) must hold fewer than 2^31 elements", Lcap,
              d->cfg.kv_heads, d->cfg.head_dim);
  DFL_REQUIRE(Lmax == 0 || (K && V), DFL_E_INVALID, "K/V NULL with Lmax > 0");
  DFL_REQUIRE((int64_t)B * G * std::max(c.vocab, c.intermediate * 2) < (1ll << 31), DFL_E_SHAPE, "B*G too large");
  DFL_REQUIRE(aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  const DraftLayout lay = draft_layout(c, B, G, Lmax);
  DFL_REQUIRE(ws_bytes >= lay.total, DFL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, lay.total);
  return run_layer(d, layer, x_in, x_out, B, G, Lmax > 0 ? K : nullptr, Lmax > 0 ? V : nullptr, Lcap, Lmax, ctx_len,
                   pos0, static_cast<char*>(ws), lay, false, nullptr, stream);
}

// ---------------------------------------------------------------- single steps

int dfl_rms_norm(const dfl_bf16* x, int rows, int H, int ldx, const dfl_bf16* gamma, float eps, dfl_bf16* y,
                 int ldy, hipStream_t stream) {
  DFL_REQUIRE(x && gamma && y, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(rows >= 0 && H > 0 && ldx >= H && ldy >= H, DFL_E_INVALID, "bad sizes");
  DFL_REQUIRE(H % 8 == 0 && H <= 8192 && ldx % 8 == 0 && ldy % 8 == 0, DFL_E_UNSUPPORTED,
              "H and leading dimensions must be multiples of 8, H <= 8192");
  DFL_REQUIRE(eps >= 0.f, DFL_E_INVALID, "eps < 0");
  hipError_t e = dfl::launch_rms_norm(x, ldx, rows, H, gamma, eps, y, ldy, 1, 1, 0, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

size_t dfl_linear_workspace_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 64) return 0;
  return dfl::plan_gemm(M, N, K).partial_bytes;
}

int dfl_linear(const dfl_bf16* x, int M, int K, int ldx, const dfl_bf16* W, int N, void* y, int ldy, int out_f32,
               void* ws, size_t ws_bytes, hipStream_t stream) {
  DFL_REQUIRE(x && W && y, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(M > 0 && N > 0 && K > 0 && ldx >= K && ldy >= N, DFL_E_INVALID, "bad sizes");
  DFL_REQUIRE(K % 64 == 0 && ldx % 8 == 0, DFL_E_UNSUPPORTED, "K must be a multiple of 64 and ldx of 8");
  const dfl::GemmPlan pl = dfl::plan_gemm(M, N, K);
  DFL_REQUIRE(ws_bytes >= pl.partial_bytes && (pl.partial_bytes == 0 || ws), DFL_E_WORKSPACE,
              "workspace %zu < %zu bytes", ws_bytes, pl.partial_bytes);
  DFL_REQUIRE(pl.partial_bytes == 0 || aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  float* part = static_cast<float*>(ws);
  hipError_t e = dfl::launch_gemm(pl, x, ldx, W, false, M, N, K, out_f32 ? dfl::EPI_F32 : dfl::EPI_BF16, y, ldy,
                                  nullptr, 0, 0, part, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

int dfl_linear_q4(const dfl_bf16* x, int M, int K, int ldx, const uint32_t* packed, const dfl_bf16* scales,
                  const dfl_bf16* biases, int N, void* y, int ldy, int out_f32, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  DFL_REQUIRE(x && packed && scales && biases && y, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(M > 0 && N > 0 && K > 0 && ldx >= K && ldy >= N, DFL_E_INVALID, "bad sizes");
  DFL_REQUIRE(K % 64 == 0 && ldx % 8 == 0, DFL_E_UNSUPPORTED, "K must be a multiple of 64 and ldx of 8");
  DFL_REQUIRE(reinterpret_cast<uintptr_t>(packed) % 16 == 0, DFL_E_INVALID, "packed weights must be 16-byte aligned");
  const dfl::GemmPlan pl = dfl::plan_gemm(M, N, K);
  DFL_REQUIRE(ws_bytes >= pl.partial_bytes && (pl.partial_bytes == 0 || ws), DFL_E_WORKSPACE,
              "workspace %zu < %zu bytes", ws_bytes, pl.partial_bytes);
  DFL_REQUIRE(pl.partial_bytes == 0 || aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  dfl::WeightRef w;
  w.q = packed;
  w.scales = scales;
  w.biases = biases;
  hipError_t e = dfl::launch_gemm(pl, x, ldx, w, M, N, K, out_f32 ? dfl::EPI_F32 : dfl::EPI_BF16, y, ldy, nullptr, 0,
                                  0, static_cast<float*>(ws), stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

int dfl_head_norm_rope(dfl_bf16* x, int rows, int heads, int D, int ldx, const dfl_bf16* gamma, float eps,
                       float theta, const int32_t* pos0, int rows_per_req, hipStream_t stream) {
  DFL_REQUIRE(x && gamma && pos0, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(rows >= 0 && heads > 0 && rows_per_req > 0 && ldx >= heads * D, DFL_E_INVALID, "bad sizes");
  DFL_REQUIRE(D == 64 || D == 128, DFL_E_UNSUPPORTED, "head_dim %d must be 64 or 128", D);
  DFL_REQUIRE(eps >= 0.f && theta > 0.f, DFL_E_INVALID, "eps < 0 or theta <= 0");
  hipError_t e =
      dfl::launch_head_norm_rope(x, ldx, rows, heads, heads, D, gamma, gamma, eps, theta, pos0, rows_per_req, 0, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

size_t dfl_attention_workspace_bytes(int B, int G, int NH, int NKV, int D, int Lmax) {
  if (B <= 0 || G <= 0 || NH <= 0 || NKV <= 0 || NH % NKV || Lmax < 0) return 0;
  return dfl::plan_attention(B, G, NH, NKV, D, Lmax).ws_bytes;
}

int dfl_block_attention(const dfl_bf16* q, int ldq, const dfl_bf16* kb, const dfl_bf16* vb, int ldkv,
                        const dfl_bf16* K, const dfl_bf16* V, int Lcap, int Lmax, const int32_t* ctx_len,
                        const int32_t* pos0, int window, int B, int G, int NH, int NKV, int D, dfl_bf16* out, int ldo,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  DFL_REQUIRE(q && kb && vb && ctx_len && out && ws, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(window >= 0, DFL_E_INVALID, "window %d must be >= 0", window);
  DFL_REQUIRE(window == 0 || pos0, DFL_E_INVALID, "a sliding window needs pos0");
  DFL_REQUIRE(B > 0 && G > 0 && NH > 0 && NKV > 0 && NH % NKV == 0, DFL_E_INVALID, "bad head counts");
  DFL_REQUIRE(D == 64 || D == 128, DFL_E_UNSUPPORTED, "head_dim %d must be 64 or 128", D);
  DFL_REQUIRE(G * (NH / NKV) <= 64, DFL_E_UNSUPPORTED, "more than 64 query rows per KV head");
  DFL_REQUIRE(Lmax >= 0 && Lmax <= Lcap, DFL_E_SHAPE, "Lmax outside [0, Lcap]");
  DFL_REQUIRE((int64_t)Lcap * NKV * D < (int64_t(1) << 31), DFL_E_SHAPE,
              "one request's K/V (Lcap %d x %d x %d) must hold fewer than 2^31 elements", Lcap, NKV, D);
  DFL_REQUIRE(Lmax == 0 || (K && V), DFL_E_INVALID, "K/V NULL with Lmax > 0");
  DFL_REQUIRE(ldq >= NH * D && ldkv >= NKV * D && ldo >= NH * D && ldq % 8 == 0 && ldkv % 8 == 0, DFL_E_SHAPE,
              "leading dimensions too small or not multiples of 8");
  DFL_REQUIRE(aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  const dfl::AttnPlan pl = dfl::plan_attention(B, G, NH, NKV, D, Lmax);
  DFL_REQUIRE(ws_bytes >= pl.ws_bytes, DFL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, pl.ws_bytes);
  hipError_t e = dfl::launch_attention(pl, q, ldq, kb, vb, ldkv, K, V, Lcap, ctx_len, pos0, window, B, G, NH, NKV,
                                       D, Lmax, out, ldo, ws, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

size_t dfl_conv_prepare_workspace_bytes(int T, int H, int grp) {
  if (T <= 0 || H <= 0 || grp <= 0 || H % grp || H % 64) return 0;
  const int ng = H / grp;
  return align_up((size_t)T * 2 * ng * sizeof(float)) + dfl::plan_gemm(T, 4 * ng, H).partial_bytes;
}

static int check_conv(int T, int H, int G, int grp) {
  DFL_REQUIRE(T > 0 && H > 0 && G > 0 && grp > 0, DFL_E_INVALID, "sizes must be positive");
  DFL_REQUIRE(T % G == 0, DFL_E_SHAPE, "T=%d is not a whole number of %d-row blocks", T, G);
  DFL_REQUIRE(grp % 8 == 0 && H % grp == 0, DFL_E_UNSUPPORTED, "group %d must be a multiple of 8 dividing H", grp);
  return DFL_OK;
}

int dfl_conv_prepare(const dfl_bf16* x, int T, int H, int G, int grp, const dfl_bf16* kproj, const dfl_bf16* base,
                     dfl_bf16* out, float* coef1, void* ws, size_t ws_bytes, hipStream_t stream) {
  DFL_REQUIRE(x && kproj && base && out && coef1 && ws, DFL_E_INVALID, "NULL argument");
  DFL_TRY(check_conv(T, H, G, grp));
  DFL_REQUIRE(x != out, DFL_E_INVALID, "x must not alias out");
  DFL_REQUIRE(H % 64 == 0, DFL_E_UNSUPPORTED, "H must be a multiple of 64");
  DFL_REQUIRE(aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  const size_t need = dfl_conv_prepare_workspace_bytes(T, H, grp);
  DFL_REQUIRE(ws_bytes >= need, DFL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const int ng = H / grp;
  float* d0 = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)T * 2 * ng * sizeof(float)));
  const dfl::GemmPlan pl = dfl::plan_gemm(T, 4 * ng, H);
  hipError_t e = dfl::launch_gemm(pl, x, H, kproj, false, T, 4 * ng, H, dfl::EPI_F32, d0, 2 * ng, coef1, 2 * ng, 2 * ng,
                                  part, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  dfl::Planes coef0;
  coef0.p = d0;
  coef0.S = 1;
  coef0.ld = 2 * ng;
  e = dfl::launch_conv(x, coef0, base, 0, T, H, G, grp, nullptr, out, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

int dfl_conv_finish(const dfl_bf16* y, const float* coef1, const dfl_bf16* base, int T, int H, int G, int grp,
                    const dfl_bf16* residual, dfl_bf16* out, hipStream_t stream) {
  DFL_REQUIRE(y && coef1 && base && out, DFL_E_INVALID, "NULL argument");
  DFL_TRY(check_conv(T, H, G, grp));
  DFL_REQUIRE(y != out, DFL_E_INVALID, "y must not alias out");
  dfl::Planes coef;
  coef.p = coef1;
  coef.S = 1;
  coef.ld = 2 * (H / grp);
  hipError_t e = dfl::launch_conv(y, coef, base, 1, T, H, G, grp, residual, out, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

size_t dfl_candidates_workspace_bytes(int N, int V, int K) {
  if (N <= 0 || V <= 0 || K <= 0) return 0;
  return dfl::topk_ws_bytes(N, V);
}

int dfl_compute_candidates(const float* logits, int N, int V, int K, int32_t* ids, float* unary, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  DFL_REQUIRE(logits && ids && unary && ws, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(N > 0 && V > 0 && K > 0, DFL_E_INVALID, "sizes must be positive");
  DFL_REQUIRE(K <= 32 && K <= V, DFL_E_UNSUPPORTED, "K=%d must be <= 32 and <= V", K);
  const size_t need = dfl::topk_ws_bytes(N, V);
  DFL_REQUIRE(ws_bytes >= need, DFL_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  DFL_REQUIRE(aligned(ws), DFL_E_INVALID, "workspace must be %zu-byte aligned", kAlign);
  hipError_t e = dfl::launch_topk(logits, N, V, K, ids, unary, ws, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

int dfl_compute_candidates_static(const float* logits, int N, int V, int K, int32_t* ids, float* unary,
                                  hipStream_t stream) {
  DFL_REQUIRE(logits && ids && unary, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(N > 0 && V > 0 && K > 0, DFL_E_INVALID, "sizes must be positive");
  DFL_REQUIRE(K <= 32 && K <= V, DFL_E_UNSUPPORTED, "K=%d must be <= 32 and <= V", K);
  const size_t need = dfl::topk_ws_bytes(N, V) / sizeof(float);
  DFL_REQUIRE(need <= (size_t)DFL_CANDIDATES_STATIC_MAX_TILES && need <= dfl::topk_static_scratch_floats(),
              DFL_E_WORKSPACE, "N * ceil(V / 256) = %zu tile maxima exceed the static scratch of %d", need,
              DFL_CANDIDATES_STATIC_MAX_TILES);
  float* scratch = nullptr;
  DFL_HIP(dfl::topk_static_scratch(stream, &scratch));
  hipError_t e = dfl::launch_topk(logits, N, V, K, ids, unary, scratch, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

size_t dfl_selector_project_workspace_bytes(int N, int H, int R) { return dfl_linear_workspace_bytes(N, R, H); }

int dfl_selector_project(const dfl_bf16* h, int N, int H, const dfl_bf16* proj, int R, float* z, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (h && proj && z && N > 0 && dfl::selproj_fits(H, R, h, proj)) {
    // the kernel dfl_select_tokens_projected runs beside its scan: the same z bit for bit
    hipError_t e = dfl::launch_selector_project(h, N, H, proj, R, z, stream);
    DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
    return DFL_OK;
  }
  return dfl_linear(h, N, H, H, proj, R, z, R, 1, ws, ws_bytes, stream);
}

int dfl_score_edges(const int32_t* cand, const float* unary, const float* z, const int32_t* anchors, int B, int S,
                    int K, int R, const dfl_bf16* pred, const dfl_bf16* succ, int V, float* scores,
                    hipStream_t stream) {
  DFL_REQUIRE(cand && unary && z && anchors && pred && succ && scores, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(B > 0 && S > 0 && K > 0 && R > 0 && V > 0, DFL_E_INVALID, "sizes must be positive");
  DFL_REQUIRE(K <= 32 && R <= 128, DFL_E_UNSUPPORTED, "K <= 32 and R <= 128 required");
  hipError_t e = dfl::launch_score_edges(cand, unary, z, anchors, B, S, K, R, pred, succ, V, scores, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

int dfl_tile_maxima(const float* logits, int N, int V, float* tile_max, hipStream_t stream) {
  DFL_REQUIRE(logits && tile_max, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(N > 0 && V > 0, DFL_E_INVALID, "sizes must be positive");
  hipError_t e = dfl::launch_tile_maxima(logits, N, V, tile_max, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

int dfl_select_tokens(const float* logits, const float* tile_max, int B, int S, int V, int K, const float* z, int R,
                      const int32_t* anchors, const dfl_bf16* pred, const dfl_bf16* succ, int32_t* cand,
                      float* unary, float* scores, int32_t* tokens, hipStream_t stream) {
  DFL_REQUIRE(logits && z && anchors && pred && succ && cand && unary && tokens, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(B > 0 && S > 0 && V > 0 && K > 0 && R > 0, DFL_E_INVALID, "sizes must be positive");
  DFL_REQUIRE(K <= V, DFL_E_UNSUPPORTED, "K=%d exceeds V=%d", K, V);
  DFL_REQUIRE(dfl::select_tokens_fits(S, K, R), DFL_E_UNSUPPORTED,
              "S=%d, K=%d, R=%d: this call needs S <= 64, K <= 16 and R a multiple of 4 in [4, 64]", S, K, R);
  DFL_REQUIRE(tile_max || (V + dfl::kGemmTileN - 1) / dfl::kGemmTileN <= dfl::kSelectScanMaxTiles, DFL_E_UNSUPPORTED,
              "without tile maxima V=%d needs at most %d tiles of %d columns", V, dfl::kSelectScanMaxTiles,
              dfl::kGemmTileN);
  hipError_t e = dfl::launch_select_tokens(logits, tile_max, B, S, V, K, nullptr, z, R, anchors, pred, succ, V, cand,
                                           unary, scores, tokens, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

int dfl_select_tokens_projected(const float* logits, int B, int S, int V, int K, const dfl_bf16* h, int H,
                                const dfl_bf16* proj, int R, float* z, const int32_t* anchors, const dfl_bf16* pred,
                                const dfl_bf16* succ, int32_t* cand, float* unary, float* scores, int32_t* tokens,
                                hipStream_t stream) {
  DFL_REQUIRE(logits && h && proj && z && anchors && pred && succ && cand && unary && tokens, DFL_E_INVALID,
              "NULL argument");
  DFL_REQUIRE(B > 0 && S > 0 && V > 0 && K > 0 && R > 0 && H > 0, DFL_E_INVALID, "sizes must be positive");
  DFL_REQUIRE(K <= V, DFL_E_UNSUPPORTED, "K=%d exceeds V=%d", K, V);
  DFL_REQUIRE(dfl::select_tokens_fits(S, K, R), DFL_E_UNSUPPORTED,
              "S=%d, K=%d, R=%d: this call needs S <= 64, K <= 16 and R a multiple of 4 in [4, 64]", S, K, R);
  DFL_REQUIRE((V + dfl::kGemmTileN - 1) / dfl::kGemmTileN <= dfl::kSelectScanMaxTiles, DFL_E_UNSUPPORTED,
              "V=%d needs at most %d tiles of %d columns", V, dfl::kSelectScanMaxTiles, dfl::kGemmTileN);
  DFL_REQUIRE(dfl::selproj_fits(H, R, h, proj), DFL_E_UNSUPPORTED,
              "H=%d must be a multiple of 128 and h, proj 16-byte aligned", H);
  hipError_t e = dfl::launch_select_tokens_projected(logits, B, S, V, K, h, H, proj, R, z, anchors, pred, succ,
                                                     cand, unary, scores, tokens, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

int dfl_select_path(const float* scores, const int32_t* cand, int B, int S, int K, int32_t* tokens,
                    hipStream_t stream) {
  DFL_REQUIRE(scores && cand && tokens, DFL_E_INVALID, "NULL argument");
  DFL_REQUIRE(B > 0 && S > 0 && K > 0, DFL_E_INVALID, "sizes must be positive");
  DFL_REQUIRE(K <= 64, DFL_E_UNSUPPORTED, "K must be <= 64");
  hipError_t e = dfl::launch_select_path(scores, cand, B, S, K, tokens, stream);
  DFL_REQUIRE(e == hipSuccess, DFL_E_DEVICE, "launch: %s", hipGetErrorString(e));
  return DFL_OK;
}

// ---------------------------------------------------------------- timing

int dfl_set_timed_kernel(dfl_drafter* d, int k) {
  DFL_REQUIRE(d, DFL_E_INVALID, "NULL drafter");
  DFL_REQUIRE(k >= DFL_K_NONE && k < DFL_K_COUNT, DFL_E_INVALID, "unknown kernel class %d", k);
  d->timed_class = k;
  return DFL_OK;
}

int dfl_read_kernel_time(dfl_drafter* d, double* total_ms, int64_t* launches, double* bytes) {
  DFL_REQUIRE(d && total_ms && launches, DFL_E_INVALID, "NULL argument");
  double ms = 0.0, by = 0.0;
  int rc = DFL_OK;
  for (auto& t : d->timed) {
    if (rc == DFL_OK) {
      float e = 0.f;
      hipError_t s = hipEventSynchronize(t.stop);
      if (s == hipSuccess) s = hipEventElapsedTime(&e, t.start, t.stop);
      if (s != hipSuccess) rc = fail(DFL_E_DEVICE, "event timing: %s", hipGetErrorString(s));
      ms += e;
      by += t.bytes;
    }
    d->pool.push_back(t.start);
    d->pool.push_back(t.stop);
  }
  *total_ms = ms;
  *launches = static_cast<int64_t>(d->timed.size());
  if (bytes) *bytes = by;
  d->timed.clear();
  return rc;
}

}  // extern "C"
