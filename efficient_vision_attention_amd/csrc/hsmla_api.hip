// C ABI of libhsmla.so: argument validation, workspace layout and the launch
// order of the forward pass on the caller's stream.  Declarations and the
// contract of every entry point are in include/hsmla.h.
#include "../../include/hsmla.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"

// Device memory of hsmla_linear_attn_noalloc: the K/V-state chunk partials
// of callers that cannot allocate.  Each GPU holds its own copy of this
// array from the library's load until the process ends; host code must use
// the per-device address hipGetSymbolAddress returns (scratch_address), not
// the array's name.
static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

using hsmla::kv_chunks;

constexpr int kHeadDim = 32;
constexpr int kMaxBlock = 16;
constexpr int kMaxBlocks = 8192;
constexpr int kMaxChannels = 2048;
constexpr int kMaxBranchK = 7;
constexpr size_t kAlign = 256;  // section alignment inside a workspace

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Dims {
  int B, gh, gw, N, C, H, T, k, Bs, w, kmax;
  int Bk;     // images of the whole call (a range keeps it): the K/V chunking
  int sw;     // sel entries per image: k (top-k), T (threshold), H*T (per head)
  int nc;     // routed-set counts: B (threshold), B*H (per head)
  size_t P;   // B * N tokens
  size_t e;   // bytes per activation element
  bool bf;
  bool thr;   // threshold routing (block or per head)
  bool ph;    // per-head routing
  bool soft;  // every block, residual scaled by its score
  bool wblk;  // the GEMM's weight copies are tile-blocked (see weights_blocked)
  bool prepared;  // taps and weight copies already in the workspace
  float tau;
};

// Where the refinement launch finds each (image, head) list.
hsmla::SelLayout sel_layout(const Dims& D) {
  if (D.ph) return {D.H * D.T, D.T, D.H, 1};
  if (D.thr) return {D.T, 0, 1, 0};
  return {D.k, 0, 0, 0};
}

hsmla_status check_desc(const hsmla_desc* d, Dims* out) {
  if (!d) return HSMLA_ERR_NULL;
  if (d->dtype != HSMLA_F32 && d->dtype != HSMLA_BF16) return HSMLA_ERR_DTYPE;
  if (d->batch < 1 || d->grid_h < 1 || d->grid_w < 1) return HSMLA_ERR_SHAPE;
  if (d->head_dim != kHeadDim || d->heads < 1) return HSMLA_ERR_SHAPE;
  if ((int64_t)d->heads * d->head_dim != d->channels) return HSMLA_ERR_SHAPE;
  if (d->channels > kMaxChannels) return HSMLA_ERR_SHAPE;
  if (d->n_branches < 0 || d->n_branches > 3) return HSMLA_ERR_SHAPE;
  int kmax = 1;
  for (int i = 0; i < d->n_branches; ++i) {
    const int k = d->branch_k[i];
    if (k < 1 || k > kMaxBranchK || k % 2 == 0) return HSMLA_ERR_SHAPE;
    if (k > kmax) kmax = k;
  }
  if (d->block < 1 || d->block > kMaxBlock) return HSMLA_ERR_SHAPE;
  if (d->grid_h % d->block || d->grid_w % d->block) return HSMLA_ERR_SHAPE;
  if (d->window < d->block || (d->window - d->block) % 2) return HSMLA_ERR_SHAPE;
  const int64_t T = (int64_t)(d->grid_h / d->block) * (d->grid_w / d->block);
  if (T > kMaxBlocks) return HSMLA_ERR_SHAPE;
  if (d->keep_blocks < 0 || d->keep_blocks > T) return HSMLA_ERR_SHAPE;
  if (d->routing != HSMLA_ROUTE_TOPK && d->routing != HSMLA_ROUTE_THRESHOLD &&
      d->routing != HSMLA_ROUTE_HEAD_THRESHOLD && d->routing != HSMLA_ROUTE_SOFT)
    return HSMLA_ERR_ARG;
  if ((d->routing == HSMLA_ROUTE_THRESHOLD ||
       d->routing == HSMLA_ROUTE_HEAD_THRESHOLD) && isnan(d->tau))
    return HSMLA_ERR_ARG;
  const int64_t N = (int64_t)d->grid_h * d->grid_w;
  // every element index must fit a 32-bit grid dimension and size_t math
  if (N * d->batch * 4 * (int64_t)d->channels > ((int64_t)1 << 40)) return HSMLA_ERR_SHAPE;
  if (N * d->batch > INT32_MAX / 2) return HSMLA_ERR_SHAPE;
  if (out) {
    out->B = d->batch;
    out->Bk = d->batch;
    out->gh = d->grid_h;
    out->gw = d->grid_w;
    out->N = (int)N;
    out->C = d->channels;
    out->H = d->heads;
    out->T = (int)T;
    out->k = d->keep_blocks;
    out->Bs = d->block;
    out->w = d->window;
    out->kmax = kmax;
    out->P = (size_t)N * d->batch;
    out->bf = d->dtype == HSMLA_BF16;
    out->thr = d->routing == HSMLA_ROUTE_THRESHOLD ||
               d->routing == HSMLA_ROUTE_HEAD_THRESHOLD;
    out->ph = d->routing == HSMLA_ROUTE_HEAD_THRESHOLD;
    out->soft = d->routing == HSMLA_ROUTE_SOFT;
    out->tau = d->tau;
    out->prepared = d->prepared != 0;
    out->sw = out->ph   ? d->heads * (int)T
              : out->thr  ? (int)T
              : out->soft ? 0
                          : d->keep_blocks;
    out->nc = out->ph ? d->batch * d->heads : d->batch;
    out->e = out->bf ? 2 : 4;
    // Tile-blocked weight copies when every projection of every image range
    // is whole GEMM tiles: output widths (3C, C, 4C) multiples of
    // kGemmTileN, input widths of kGemmTileK, and each image's token count a
    // multiple of kGemmTileM (so any range of images is too).
    out->wblk = out->bf && (3 * out->C) % hsmla::kGemmTileN == 0 &&
                out->C % hsmla::kGemmTileN == 0 && out->C % hsmla::kGemmTileK == 0 &&
                out->N % hsmla::kGemmTileM == 0;
  }
  return HSMLA_OK;
}

// Workspace sections, in this order (each start rounded up to 256 bytes):
//   qkv [P][3C], qkv_hat [P][3C], o [P][C], kv [B][H][d][d] f32,
//   ksum [B][H][d] f32, kv partials f32, dw taps [kmax^2][3C] f32,
//   scores [B][T] f32, sel [B][k] i32 (threshold: [B][T] i32, counts [B] i32;
//   per head: [B][H][T] i32, counts [B][H] i32, head scores [B][T][H] f32),
//   gate block sums [B][T][3C] f32,
//   (block only) xn [P][C], x1 [P][C], h1 [P][4C], h2 [P][4C],
//   ffn taps [9][4C] f32,
//   the GEMM's copies of W_qkv, W_o (and, block only, W1, W2): transposed
//   to [out][in], tile-blocked when Dims::wblk, else row-major.
// hsmla_qkv_branches' workspace holds the taps and the W_qkv copy only.
struct Layout {
  size_t qkv, qkv_hat, o, kv, ksum, part, taps, scores, sel, counts, head_scores;
  size_t bsum, rankp;
  size_t xn, x1, h1, h2, ffn_taps;
  size_t wq, wo, w1, w2;  // 0 when not part of the op
  size_t total;
};

Layout layout(const Dims& D, int op) {
  Layout L{};
  size_t off = 0;
  auto take = [&off](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes);
    return at;
  };
  const size_t bh = (size_t)D.B * D.H;
  const size_t part_bytes =
      bh * kv_chunks(D.bf, D.Bk, D.H, D.N) * (kHeadDim * kHeadDim + kHeadDim) * 4;
  const size_t tap_bytes = (size_t)D.kmax * D.kmax * 3 * D.C * 4;
  const size_t c2 = (size_t)D.C * D.C * D.e;
  if (op == HSMLA_OP_QKV) {
    L.taps = take(tap_bytes);
    L.wq = take(3 * c2);
  } else if (op == HSMLA_OP_LINEAR) {
    L.part = take(part_bytes);
  } else {
    L.qkv = take(D.P * 3 * D.C * D.e);
    L.qkv_hat = take(D.P * 3 * D.C * D.e);
    L.o = take(D.P * D.C * D.e);
    L.kv = take(bh * kHeadDim * kHeadDim * 4);
    L.ksum = take(bh * kHeadDim * 4);
    L.part = take(part_bytes);
    L.taps = take(tap_bytes);
    L.scores = take((size_t)D.B * D.T * 4);
    L.sel = take((size_t)D.B * D.sw * 4 + 4);
    if (D.thr) L.counts = take((size_t)D.nc * 4);
    if (D.ph) L.head_scores = take((size_t)D.B * D.T * D.H * 4);
    L.bsum = take((size_t)D.B * D.T * 3 * D.C * 4);
    L.rankp = take((size_t)D.B * hsmla::topk_parts_bytes(D.T));
    if (op == HSMLA_OP_BLOCK) {
      L.xn = take(D.P * D.C * D.e);
      L.x1 = take(D.P * D.C * D.e);
      L.h1 = take(D.P * 4 * D.C * D.e);
      L.h2 = take(D.P * 4 * D.C * D.e);
      L.ffn_taps = take((size_t)9 * 4 * D.C * 4);
    }
    L.wq = take(3 * c2);
    L.wo = take(c2);
    if (op == HSMLA_OP_BLOCK) {
      L.w1 = take(4 * c2);
      L.w2 = take(4 * c2);
    }
  }
  L.total = off;
  return L;
}

inline char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// Optional per-launch event recording for the *_timed entry points: mark()
// records events[i] on the stream just before launch i (and once more after
// the last launch); without events it does nothing.
struct Rec {
  hipEvent_t* ev = nullptr;
  const char** names = nullptr;
  int cap = 0;
  int n = 0;
  hipStream_t s = nullptr;
  bool ok = true;
  void mark(const char* name) {
    if (ev && n < cap) {
      if (hipEventRecord(ev[n], s) != hipSuccess) ok = false;
      if (names) names[n] = name;
    }
    ++n;
  }
  void end() {
    if (ev && n < cap) {
      if (hipEventRecord(ev[n], s) != hipSuccess) ok = false;
      if (names) names[n] = "end";
    }
  }
};

hsmla_status hip_status(hipError_t e) {
  return e == hipSuccess ? HSMLA_OK : HSMLA_ERR_HIP;
}

#define HSMLA_TRY(expr)                                      \
  do {                                                       \
    const hipError_t e_ = (expr);                            \
    if (e_ != hipSuccess) return HSMLA_ERR_HIP;              \
  } while (0)

hsmla_status check_weights(const hsmla_desc* d, const hsmla_weights* w) {
  if (!w || !w->w_qkv || !w->w_o || !w->gate_w || !w->gate_b) return HSMLA_ERR_NULL;
  for (int i = 0; i < d->n_branches; ++i)
    if (!w->dw[i]) return HSMLA_ERR_NULL;
  if (!aligned(w->w_qkv, 16) || !aligned(w->w_o, 16)) return HSMLA_ERR_ALIGN;
  for (int i = 0; i < d->n_branches; ++i)
    if (!aligned(w->dw[i], 4)) return HSMLA_ERR_ALIGN;
  if (!aligned(w->gate_w, 4) || !aligned(w->gate_b, 4)) return HSMLA_ERR_ALIGN;
  if (w->gate_dw && !aligned(w->gate_dw, 16)) return HSMLA_ERR_ALIGN;
  return HSMLA_OK;
}

// Workspace pointers of images [b0, b0 + nb): every section is laid out
// image by image, so a range is an offset into each.
struct Bufs {
  void *qkv, *qkvh, *o, *xn, *x1, *h1, *h2;
  float *kv, *ksum, *part, *taps, *ftaps, *scores, *hscores, *bsum;
  int32_t *sel, *counts;
  int32_t* rankp;           // top-k partial ranks
  void *wq, *wo, *w1, *w2;  // the GEMM's weight copies (shared), or null
};

Bufs bufs_for(const Dims& D, const Layout& L, void* ws, int op, int b0) {
  const size_t n = (size_t)D.N, c = (size_t)D.C, e = D.e, T = (size_t)D.T;
  const size_t H = (size_t)D.H, bb = (size_t)b0;
  const size_t chunks = (size_t)kv_chunks(D.bf, D.Bk, D.H, D.N);
  Bufs u{};
  if (op == HSMLA_OP_QKV) {  // taps and the W_qkv copy only
    u.taps = reinterpret_cast<float*>(at(ws, L.taps));
    u.wq = at(ws, L.wq);
    return u;
  }
  u.qkv = at(ws, L.qkv + bb * n * 3 * c * e);
  u.qkvh = at(ws, L.qkv_hat + bb * n * 3 * c * e);
  u.o = at(ws, L.o + bb * n * c * e);
  u.kv = reinterpret_cast<float*>(at(ws, L.kv)) + bb * H * kHeadDim * kHeadDim;
  u.ksum = reinterpret_cast<float*>(at(ws, L.ksum)) + bb * H * kHeadDim;
  u.part = reinterpret_cast<float*>(at(ws, L.part)) +
           bb * H * chunks * (kHeadDim * kHeadDim + kHeadDim);
  u.taps = reinterpret_cast<float*>(at(ws, L.taps));  // shared by all images
  u.scores = reinterpret_cast<float*>(at(ws, L.scores)) + bb * T;
  u.sel = reinterpret_cast<int32_t*>(at(ws, L.sel)) + bb * (size_t)D.sw;
  u.counts = D.thr ? reinterpret_cast<int32_t*>(at(ws, L.counts)) +
                         bb * (size_t)(D.nc / D.B)
                   : nullptr;
  u.hscores = D.ph ? reinterpret_cast<float*>(at(ws, L.head_scores)) + bb * T * H
                   : nullptr;
  u.bsum = reinterpret_cast<float*>(at(ws, L.bsum)) + bb * T * 3 * c;
  u.rankp = hsmla::topk_parts_bytes(D.T)
                ? reinterpret_cast<int32_t*>(at(ws, L.rankp + bb * hsmla::topk_parts_bytes(D.T)))
                : nullptr;
  if (op == HSMLA_OP_BLOCK) {
    u.xn = at(ws, L.xn + bb * n * c * e);
    u.x1 = at(ws, L.x1 + bb * n * c * e);
    u.h1 = at(ws, L.h1 + bb * n * 4 * c * e);
    u.h2 = at(ws, L.h2 + bb * n * 4 * c * e);
    u.ftaps = reinterpret_cast<float*>(at(ws, L.ffn_taps));  // shared
  }
  u.wq = at(ws, L.wq);
  u.wo = at(ws, L.wo);
  if (op == HSMLA_OP_BLOCK) {
    u.w1 = at(ws, L.w1);
    u.w2 = at(ws, L.w2);
  }
  return u;
}

// A projection's weights for the GEMM: the prepared copy, tile-blocked when
// Dims::wblk (every GEMM of the call, over any image range, is then whole
// tiles).
struct WSel {
  const void* w;
  bool blocked;
};
WSel wsel(const Dims& D, const void* copy) { return {copy, D.wblk}; }

// One launch before the stages (or once, by hsmla_prepare): the folded
// branch taps (and the FFN's, for the block) and the GEMM's weight copies.
// f == nullptr: the module's operands only; qkv_only: the taps and W_qkv.
hsmla_status prep(const Dims& D, const hsmla_desc* d, const hsmla_weights* w,
                  const hsmla_ffn_weights* f, const Bufs& u, hipStream_t s,
                  Rec& r, bool qkv_only = false) {
  hsmla::TapSpec taps[2];
  int ntaps = 0;
  {
    hsmla::TapSpec& q = taps[ntaps++];
    q = hsmla::TapSpec{{nullptr, nullptr, nullptr}, {0, 0, 0}, d->n_branches,
                       D.kmax, 3 * D.C, 1, u.taps};
    for (int i = 0; i < d->n_branches; ++i) {
      q.kernels[i] = w->dw[i];
      q.ks[i] = d->branch_k[i];
    }
  }
  if (f)
    taps[ntaps++] = hsmla::TapSpec{{f->dw_ffn, nullptr, nullptr}, {3, 0, 0}, 1, 3,
                                   4 * D.C, 0, u.ftaps};
  hsmla::BlockJob jobs[4];
  int njobs = 0;
  const int tr = D.wblk ? hsmla::kGemmTileN : 0;
  jobs[njobs++] = {w->w_qkv, u.wq, 3 * D.C, D.C, tr};
  if (!qkv_only) {
    jobs[njobs++] = {w->w_o, u.wo, D.C, D.C, tr};
    if (f) {
      jobs[njobs++] = {f->w1, u.w1, 4 * D.C, D.C, tr};
      jobs[njobs++] = {f->w2, u.w2, D.C, 4 * D.C, tr};
    }
  }
  r.mark("prep");
  HSMLA_TRY(hsmla::launch_prep(D.bf, taps, ntaps, jobs, njobs, s));
  return HSMLA_OK;
}

// The same dims for a range of nb images.
Dims range_dims(const Dims& D, int nb) {
  Dims r = D;
  r.B = nb;
  r.P = (size_t)D.N * nb;
  r.nc = D.ph ? nb * D.H : nb;
  return r;
}

// Steps 1-5 into the workspace views (o holds the refined output), as
// numbered stages of one or two launches each, so that two image ranges can
// interleave their launches (module_stage(0..kModuleStages-1) in order is
// the whole module, after prep).  D may describe a range of the images
// (range_dims), u the matching pointers.
constexpr int kModuleStages = 7;

// x_blk: x is tile-blocked (written so by the block's LayerNorm).
hsmla_status module_stage(int st, const Dims& D, const hsmla_desc* d,
                          const hsmla_weights* w, const void* x, const Bufs& u,
                          hipStream_t s, Rec& r, bool x_blk = false) {
  (void)d;
  // the plain gate's block sums come out of the depthwise conv when its
  // workgroup shape allows; the gate then only forms the logits
  float* bsum = (!w->gate_dw && hsmla::dwconv_can_pool(D.kmax, D.Bs)) ? u.bsum
                                                                       : nullptr;
  // the conv reduces the sums further, into the gate's partial logits: the
  // top-k launch forms the scores itself (no gate launch), the other
  // routings form them in one small launch
  const bool gate_parts = bsum && !D.soft && !D.thr && u.rankp &&
                          hsmla::gate_topk_from_parts_ok(D.T);
  const bool gate_plog = bsum && hsmla::gate_topk_from_parts_ok(D.T) &&
                         (gate_parts || D.soft || D.thr);
  switch (st) {
    case 0: {
      r.mark("qkv_gemm");
      const WSel q = wsel(D, u.wq);
      HSMLA_TRY(hsmla::launch_gemm(D.bf, x, q.w, nullptr, u.qkv, (int)D.P, 3 * D.C,
                                   D.C, s, hsmla::GemmSite::kQkv, x_blk, q.blocked));
      return HSMLA_OK;
    }
    case 1:
      r.mark("dwconv_qkv");
      HSMLA_TRY(hsmla::launch_dwconv(D.bf, u.qkv, u.qkvh, u.taps, D.kmax, D.B, D.gh,
                                     D.gw, 3 * D.C, false, bsum, D.Bs, s, false,
                                     gate_plog ? w->gate_w : nullptr, D.H));
      return HSMLA_OK;
    case 2:
      if (gate_parts && D.bf) {
        // the top-k runs in the partial-sum launch (it only reads the
        // conv's outputs, like the K/V state)
        r.mark("kv_state_gate_topk");
        HSMLA_TRY(hsmla::launch_kv_state_topk(u.qkvh, u.kv, u.ksum, u.part, D.B, D.N, D.H, s,
                                              D.Bk, bsum, w->gate_b, u.scores, u.sel, u.rankp,
                                              D.T, D.Bs, D.k));
        return HSMLA_OK;
      }
      r.mark("kv_state");
      HSMLA_TRY(hsmla::launch_kv_state(D.bf, u.qkvh, u.kv, u.ksum, u.part, D.B,
                                       D.N, D.H, s, D.Bk));
      return HSMLA_OK;
    case 3:
      r.mark("lin_apply");
      HSMLA_TRY(hsmla::launch_lin_apply(D.bf, u.qkvh, u.kv, u.ksum, u.o, D.B,
                                        D.N, D.H, s));
      return HSMLA_OK;
    case 4:
      if (gate_parts) return HSMLA_OK;  // scores formed with the selection
      r.mark("gate_scores");
      if (gate_plog)
        HSMLA_TRY(hsmla::launch_gate_from_parts(bsum, w->gate_b, u.scores, u.hscores, D.B,
                                                D.T, D.H, D.Bs, s));
      else if (bsum)
        HSMLA_TRY(hsmla::launch_gate_from_sums(bsum, w->gate_w, w->gate_b,
                                               u.scores, u.hscores, D.B, D.T,
                                               D.H, D.Bs, s));
      else
        HSMLA_TRY(hsmla::launch_gate_scores(D.bf, u.qkvh, w->gate_w, w->gate_b,
                                            w->gate_dw, u.scores, u.hscores,
                                            D.B, D.gh, D.gw, D.H, D.Bs, s));
      return HSMLA_OK;
    case 5:
      if (D.soft) return HSMLA_OK;  // every block, weighted: no list
      if (D.ph) {
        r.mark("threshold_heads");
        HSMLA_TRY(hsmla::launch_threshold_heads(u.hscores, nullptr, u.sel,
                                                u.counts, D.B, D.T, D.H, D.tau, s));
      } else if (D.thr) {
        r.mark("threshold");
        HSMLA_TRY(hsmla::launch_threshold(u.scores, nullptr, u.sel, u.counts, D.B,
                                          D.T, D.tau, s));
      } else if (gate_parts) {
        if (D.bf) return HSMLA_OK;  // selected in the K/V-state launch
        r.mark("gate_topk");
        HSMLA_TRY(hsmla::launch_gate_topk_parts(bsum, w->gate_b, u.scores, u.sel, u.rankp,
                                                D.B, D.T, D.H, D.Bs, D.k, s));
      } else {
        r.mark("topk");
        HSMLA_TRY(hsmla::launch_topk(u.scores, nullptr, u.sel, D.B, D.T, D.k, s, u.rankp));
      }
      return HSMLA_OK;
    case 6:
      r.mark("sparse_softmax");
      if (D.soft)
        HSMLA_TRY(hsmla::launch_sparse(D.bf, u.qkv, u.qkvh, nullptr, nullptr,
                                       u.scores, u.o, D.B, D.gh, D.gw, D.H, D.Bs,
                                       D.w, D.T, sel_layout(D), s));
      else
        HSMLA_TRY(hsmla::launch_sparse(D.bf, u.qkv, u.qkvh, u.sel, u.counts,
                                       nullptr, u.o, D.B, D.gh, D.gw, D.H, D.Bs,
                                       D.w, D.thr ? D.T : D.k, sel_layout(D), s));
      return HSMLA_OK;
    default:
      return HSMLA_ERR_ARG;
  }
}

hsmla_status run_module(const Dims& D, const hsmla_desc* d,
                        const hsmla_weights* w, const void* x, const Bufs& u,
                        hipStream_t s, Rec& r) {
  for (int st = 0; st < kModuleStages; ++st) {
    const hsmla_status e = module_stage(st, D, d, w, x, u, s, r);
    if (e != HSMLA_OK) return e;
  }
  return HSMLA_OK;
}

}  // namespace

extern "C" {

const char* hsmla_status_string(int32_t status) {
  switch (status) {
    case HSMLA_OK: return "ok";
    case HSMLA_ERR_NULL: return "a required pointer is NULL";
    case HSMLA_ERR_SHAPE: return "sizes violate the library limits";
    case HSMLA_ERR_DTYPE: return "unknown dtype";
    case HSMLA_ERR_ALIGN: return "pointer not aligned as required";
    case HSMLA_ERR_WORKSPACE: return "workspace too small";
    case HSMLA_ERR_HIP: return "HIP launch failed";
    case HSMLA_ERR_ARG: return "invalid argument";
    case HSMLA_ERR_SCRATCH: return "sizes exceed the allocation-free scratch";
    default: return "unknown status";
  }
}

hsmla_status hsmla_workspace_bytes(const hsmla_desc* desc, int32_t op,
                                   size_t* bytes) {
  if (!bytes) return HSMLA_ERR_NULL;
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (op < HSMLA_OP_QKV || op > HSMLA_OP_BLOCK) return HSMLA_ERR_ARG;
  *bytes = layout(D, op).total;
  return HSMLA_OK;
}

hsmla_status hsmla_workspace_views(const hsmla_desc* desc, int32_t op,
                                   void* ws, hsmla_views* v) {
  if (!ws || !v) return HSMLA_ERR_NULL;
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (op != HSMLA_OP_FORWARD && op != HSMLA_OP_BLOCK) return HSMLA_ERR_ARG;
  const Layout L = layout(D, op);
  v->qkv = at(ws, L.qkv);
  v->qkv_hat = at(ws, L.qkv_hat);
  v->o = at(ws, L.o);
  v->kv = reinterpret_cast<float*>(at(ws, L.kv));
  v->ksum = reinterpret_cast<float*>(at(ws, L.ksum));
  v->scores = reinterpret_cast<float*>(at(ws, L.scores));
  v->sel = reinterpret_cast<int32_t*>(at(ws, L.sel));
  v->counts = D.thr ? reinterpret_cast<int32_t*>(at(ws, L.counts)) : nullptr;
  v->head_scores = D.ph ? reinterpret_cast<float*>(at(ws, L.head_scores)) : nullptr;
  v->x1 = op == HSMLA_OP_BLOCK ? at(ws, L.x1) : nullptr;
  return HSMLA_OK;
}

hsmla_status hsmla_qkv_branches(const hsmla_desc* desc, const hsmla_weights* w,
                                const void* x, void* qkv, void* qkv_hat,
                                void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (!x || !qkv || !qkv_hat || !ws) return HSMLA_ERR_NULL;
  if ((st = check_weights(desc, w)) != HSMLA_OK) return st;
  if (!aligned(x, 16) || !aligned(qkv, 16) || !aligned(qkv_hat, 16) ||
      !aligned(ws, 16))
    return HSMLA_ERR_ALIGN;
  const Layout L = layout(D, HSMLA_OP_QKV);
  if (ws_bytes < L.total) return HSMLA_ERR_WORKSPACE;
  Rec r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Bufs u = bufs_for(D, L, ws, HSMLA_OP_QKV, 0);
  if (!D.prepared && (st = prep(D, desc, w, nullptr, u, s, r, true)) != HSMLA_OK)
    return st;
  const WSel q = wsel(D, u.wq);
  HSMLA_TRY(hsmla::launch_gemm(D.bf, x, q.w, nullptr, qkv, (int)D.P, 3 * D.C, D.C, s,
                               hsmla::GemmSite::kQkv, false, q.blocked));
  HSMLA_TRY(hsmla::launch_dwconv(D.bf, qkv, qkv_hat, u.taps, D.kmax, D.B, D.gh, D.gw,
                                 3 * D.C, false, nullptr, D.Bs, s));
  return HSMLA_OK;
}

hsmla_status hsmla_prepare(const hsmla_desc* desc, int32_t op,
                           const hsmla_weights* w, const hsmla_ffn_weights* f,
                           void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (op != HSMLA_OP_QKV && op != HSMLA_OP_FORWARD && op != HSMLA_OP_BLOCK)
    return HSMLA_ERR_ARG;
  if (!ws || (op == HSMLA_OP_BLOCK && !f)) return HSMLA_ERR_NULL;
  if ((st = check_weights(desc, w)) != HSMLA_OK) return st;
  if (op == HSMLA_OP_BLOCK && (!f->w1 || !f->w2 || !f->dw_ffn)) return HSMLA_ERR_NULL;
  if (!aligned(ws, 16) ||
      (op == HSMLA_OP_BLOCK &&
       (!aligned(f->w1, 16) || !aligned(f->w2, 16) || !aligned(f->dw_ffn, 4))))
    return HSMLA_ERR_ALIGN;
  const Layout L = layout(D, op);
  if (ws_bytes < L.total) return HSMLA_ERR_WORKSPACE;
  Rec r;
  const Bufs u = bufs_for(D, L, ws, op, 0);
  return prep(D, desc, w, op == HSMLA_OP_BLOCK ? f : nullptr, u,
              static_cast<hipStream_t>(stream), r, op == HSMLA_OP_QKV);
}

}  // extern "C"

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // per device, set once

// The current device's address of `scratch`, looked up on the first call
// on that device (with it current) and kept.
hsmla_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
    return HSMLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return HSMLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HSMLA_OK;
}

}  // namespace

extern "C" {

hsmla_status hsmla_linear_attn_noalloc(const hsmla_desc* desc, const void* qkv_hat,
                                       void* o, float* kv, float* ksum,
                                       void* stream) {
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (!qkv_hat || !o || !kv || !ksum) return HSMLA_ERR_NULL;
  if (!aligned(qkv_hat, 16) || !aligned(o, 16) || !aligned(kv, 4) || !aligned(ksum, 4))
    return HSMLA_ERR_ALIGN;
  // the chunk partials are the only scratch; every entry the combine reads
  // is written first by the partial launch, so nothing needs clearing
  if (layout(D, HSMLA_OP_LINEAR).total > kScratchBytes) return HSMLA_ERR_SCRATCH;
  void* part = nullptr;
  const hsmla_status sa = scratch_address(&part);
  if (sa != HSMLA_OK) return sa;
  hipStream_t s = static_cast<hipStream_t>(stream);
  HSMLA_TRY(hsmla::launch_kv_state(D.bf, qkv_hat, kv, ksum, static_cast<float*>(part),
                                   D.B, D.N, D.H, s));
  return hip_status(
      hsmla::launch_lin_apply(D.bf, qkv_hat, kv, ksum, o, D.B, D.N, D.H, s));
}

hsmla_status hsmla_linear_attn(const hsmla_desc* desc, const void* qkv_hat,
                               void* o, float* kv, float* ksum, void* ws,
                               size_t ws_bytes, void* stream) {
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (!qkv_hat || !o || !kv || !ksum || !ws) return HSMLA_ERR_NULL;
  if (!aligned(qkv_hat, 16) || !aligned(o, 16) || !aligned(ws, 16) ||
      !aligned(kv, 4) || !aligned(ksum, 4))
    return HSMLA_ERR_ALIGN;
  const Layout L = layout(D, HSMLA_OP_LINEAR);
  if (ws_bytes < L.total) return HSMLA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  HSMLA_TRY(hsmla::launch_kv_state(D.bf, qkv_hat, kv, ksum,
                                   reinterpret_cast<float*>(at(ws, L.part)),
                                   D.B, D.N, D.H, s));
  return hip_status(
      hsmla::launch_lin_apply(D.bf, qkv_hat, kv, ksum, o, D.B, D.N, D.H, s));
}

hsmla_status hsmla_gate_select(const hsmla_desc* desc, const void* qkv_hat,
                               const float* gate_w, const float* gate_b,
                               const void* gate_dw, const float* scores_in,
                               float* scores_out, int32_t* sel, void* stream) {
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (D.thr || D.soft) return HSMLA_ERR_ARG;
  if (D.k > 0 && !sel) return HSMLA_ERR_NULL;
  if (!scores_in && (!qkv_hat || !gate_w || !gate_b || !scores_out))
    return HSMLA_ERR_NULL;
  if ((qkv_hat && !aligned(qkv_hat, 16)) || (sel && !aligned(sel, 4)) ||
      (scores_in && !aligned(scores_in, 4)) ||
      (scores_out && !aligned(scores_out, 4)) ||
      (gate_w && !aligned(gate_w, 4)) || (gate_b && !aligned(gate_b, 4)) ||
      (gate_dw && !aligned(gate_dw, 16)))
    return HSMLA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (scores_in)
    return hip_status(
        hsmla::launch_topk(scores_in, scores_out, sel, D.B, D.T, D.k, s));
  HSMLA_TRY(hsmla::launch_gate_scores(D.bf, qkv_hat, gate_w, gate_b, gate_dw,
                                      scores_out, nullptr, D.B, D.gh, D.gw, D.H,
                                      D.Bs, s));
  return hip_status(hsmla::launch_topk(scores_out, nullptr, sel, D.B, D.T, D.k, s));
}

hsmla_status hsmla_gate_threshold(const hsmla_desc* desc, const void* qkv_hat,
                                  const float* gate_w, const float* gate_b,
                                  const void* gate_dw, const float* scores_in,
                                  float* scores_out, int32_t* sel,
                                  int32_t* counts, void* stream) {
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (!D.thr || D.ph) return HSMLA_ERR_ARG;
  if (!sel || !counts) return HSMLA_ERR_NULL;
  if (!scores_in && (!qkv_hat || !gate_w || !gate_b || !scores_out))
    return HSMLA_ERR_NULL;
  if ((qkv_hat && !aligned(qkv_hat, 16)) || !aligned(sel, 4) ||
      !aligned(counts, 4) || (scores_in && !aligned(scores_in, 4)) ||
      (scores_out && !aligned(scores_out, 4)) ||
      (gate_w && !aligned(gate_w, 4)) || (gate_b && !aligned(gate_b, 4)) ||
      (gate_dw && !aligned(gate_dw, 16)))
    return HSMLA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (scores_in)
    return hip_status(hsmla::launch_threshold(scores_in, scores_out, sel, counts,
                                              D.B, D.T, D.tau, s));
  HSMLA_TRY(hsmla::launch_gate_scores(D.bf, qkv_hat, gate_w, gate_b, gate_dw,
                                      scores_out, nullptr, D.B, D.gh, D.gw, D.H,
                                      D.Bs, s));
  return hip_status(hsmla::launch_threshold(scores_out, nullptr, sel, counts,
                                            D.B, D.T, D.tau, s));
}

hsmla_status hsmla_gate_head_threshold(const hsmla_desc* desc,
                                       const void* qkv_hat,
                                       const float* gate_w, const float* gate_b,
                                       const void* gate_dw,
                                       const float* head_scores_in,
                                       float* head_scores_out, int32_t* sel,
                                       int32_t* counts, void* stream) {
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (!D.ph) return HSMLA_ERR_ARG;
  if (!sel || !counts) return HSMLA_ERR_NULL;
  if (!head_scores_in && (!qkv_hat || !gate_w || !gate_b || !head_scores_out))
    return HSMLA_ERR_NULL;
  if ((qkv_hat && !aligned(qkv_hat, 16)) || !aligned(sel, 4) ||
      !aligned(counts, 4) || (head_scores_in && !aligned(head_scores_in, 4)) ||
      (head_scores_out && !aligned(head_scores_out, 4)) ||
      (gate_w && !aligned(gate_w, 4)) || (gate_b && !aligned(gate_b, 4)) ||
      (gate_dw && !aligned(gate_dw, 16)))
    return HSMLA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_scores_in)
    return hip_status(hsmla::launch_threshold_heads(
        head_scores_in, head_scores_out, sel, counts, D.B, D.T, D.H, D.tau, s));
  // per-head routing needs only G; the block scores M are not written
  HSMLA_TRY(hsmla::launch_gate_scores(D.bf, qkv_hat, gate_w, gate_b, gate_dw,
                                      nullptr, head_scores_out, D.B, D.gh, D.gw,
                                      D.H, D.Bs, s));
  return hip_status(hsmla::launch_threshold_heads(
      head_scores_out, nullptr, sel, counts, D.B, D.T, D.H, D.tau, s));
}

hsmla_status hsmla_sparse_softmax(const hsmla_desc* desc, const void* qkv,
                                  const void* qkv_hat, const int32_t* sel,
                                  void* o, void* stream) {
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (D.thr || D.soft) return HSMLA_ERR_ARG;
  if (!qkv || !qkv_hat || !o || (D.k > 0 && !sel)) return HSMLA_ERR_NULL;
  if (!aligned(qkv, 16) || !aligned(qkv_hat, 16) || !aligned(o, 16) ||
      (sel && !aligned(sel, 4)))
    return HSMLA_ERR_ALIGN;
  return hip_status(hsmla::launch_sparse(D.bf, qkv, qkv_hat, sel, nullptr,
                                         nullptr, o, D.B, D.gh, D.gw, D.H, D.Bs,
                                         D.w, D.k, sel_layout(D),
                                         static_cast<hipStream_t>(stream)));
}

hsmla_status hsmla_sparse_softmax_weighted(const hsmla_desc* desc,
                                           const void* qkv, const void* qkv_hat,
                                           const float* weights, void* o,
                                           void* stream) {
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (!D.soft) return HSMLA_ERR_ARG;
  if (!qkv || !qkv_hat || !o || !weights) return HSMLA_ERR_NULL;
  if (!aligned(qkv, 16) || !aligned(qkv_hat, 16) || !aligned(o, 16) ||
      !aligned(weights, 4))
    return HSMLA_ERR_ALIGN;
  return hip_status(hsmla::launch_sparse(D.bf, qkv, qkv_hat, nullptr, nullptr,
                                         weights, o, D.B, D.gh, D.gw, D.H, D.Bs,
                                         D.w, D.T, sel_layout(D),
                                         static_cast<hipStream_t>(stream)));
}

hsmla_status hsmla_sparse_softmax_counted(const hsmla_desc* desc,
                                          const void* qkv, const void* qkv_hat,
                                          const int32_t* sel,
                                          const int32_t* counts, void* o,
                                          void* stream) {
  Dims D;
  const hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (!D.thr) return HSMLA_ERR_ARG;
  if (!qkv || !qkv_hat || !o || !sel || !counts) return HSMLA_ERR_NULL;
  if (!aligned(qkv, 16) || !aligned(qkv_hat, 16) || !aligned(o, 16) ||
      !aligned(sel, 4) || !aligned(counts, 4))
    return HSMLA_ERR_ALIGN;
  return hip_status(hsmla::launch_sparse(D.bf, qkv, qkv_hat, sel, counts,
                                         nullptr, o, D.B, D.gh, D.gw, D.H, D.Bs,
                                         D.w, D.T, sel_layout(D),
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

hsmla_status forward_impl(const hsmla_desc* desc, const hsmla_weights* w,
                          const void* x, void* y, void* ws, size_t ws_bytes,
                          hipStream_t s, Rec& r) {
  Dims D;
  hsmla_status st = check_desc(desc, &D);
  if (st != HSMLA_OK) return st;
  if (!x || !y || !ws) return HSMLA_ERR_NULL;
  if ((st = check_weights(desc, w)) != HSMLA_OK) return st;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 16)) return HSMLA_ERR_ALIGN;
  const Layout L = layout(D, HSMLA_OP_FORWARD);
  if (ws_bytes < L.total) return HSMLA_ERR_WORKSPACE;
  const Bufs u = bufs_for(D, L, ws, HSMLA_OP_FORWARD, 0);
  if (!D.prepared && (st = prep(D, desc, w, nullptr, u, s, r)) != HSMLA_OK) return st;
  if ((st = run_module(D, desc, w, x, u, s, r)) != HSMLA_OK) return st;
  r.mark("out_proj");
  const WSel wo = wsel(D, u.wo);
  HSMLA_TRY(hsmla::launch_gemm(D.bf, u.o, wo.w, nullptr, y, (int)D.P, D.C, D.C, s,
                               hsmla::GemmSite::kOut, false, wo.blocked));
  r.end();
  return r.ok ? HSMLA_OK : HSMLA_ERR_HIP;
}

// Checks of the block entry points; fills D and L.
hsmla_status check_block(const hsmla_desc* desc, const hsmla_weights* w,
                         const hsmla_ffn_weights* f, const void* x, void* out,
                         void* ws, size_t ws_bytes, Dims* D, Layout* L) {
  hsmla_status st = check_desc(desc, D);
  if (st != HSMLA_OK) return st;
  if (!x || !out || !ws || !f) return HSMLA_ERR_NULL;
  if ((st = check_weights(desc, w)) != HSMLA_OK) return st;
  if (!f->ln1_g || !f->ln1_b || !f->ln2_g || !f->ln2_b || !f->w1 ||
      !f->dw_ffn || !f->w2)
    return HSMLA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, 16) ||
      !aligned(f->w1, 16) || !aligned(f->w2, 16) || !aligned(f->dw_ffn, 4) ||
      !aligned(f->ln1_g, 4) || !aligned(f->ln1_b, 4) || !aligned(f->ln2_g, 4) ||
      !aligned(f->ln2_b, 4))
    return HSMLA_ERR_ALIGN;
  *L = layout(*D, HSMLA_OP_BLOCK);
  if (ws_bytes < L->total) return HSMLA_ERR_WORKSPACE;
  return HSMLA_OK;
}

// The block over the images that D (a range, see range_dims) and u cover,
// as numbered stages (prep, then block_stage(0..kBlockStages-1) in order is
// the whole block); x and out point at the range's first image.
constexpr int kBlockStages = kModuleStages + 5;

hsmla_status block_stage(int st, const Dims& D, const hsmla_desc* desc,
                         const hsmla_weights* w, const hsmla_ffn_weights* f,
                         const void* x, void* out, const Bufs& u, hipStream_t s,
                         Rec& r) {
  const int P = (int)D.P, C = D.C;
  // The LayerNorms and the FFN conv write their outputs tile-blocked when
  // the GEMM that reads them takes its whole-tile path (each K step of an A
  // tile is then one contiguous block).
  const bool ln1_blk = hsmla::layernorm_can_block(D.bf, P, C) &&
                       hsmla::gemm_whole_tiles(P, 3 * C, C);
  const bool ln2_blk = hsmla::layernorm_can_block(D.bf, P, C) &&
                       hsmla::gemm_whole_tiles(P, 4 * C, C);
  const bool h2_blk = hsmla::dwconv_can_block_out(D.bf, 3, true, D.B, D.gh, D.gw, 4 * C) &&
                      hsmla::gemm_whole_tiles(P, C, 4 * C);
  // FFN1 writes h1 channel-planar (64-channel planes: each wave's output
  // rows one contiguous run) when the FFN conv can read it so
  const bool h1_planar =
      h2_blk && ln2_blk && D.wblk &&
      hsmla::gemm_planar_ok(D.bf, P, 4 * C, C, true, true) &&
      hsmla::dwconv_planar_ok(D.bf, D.B, D.gh, D.gw, 4 * C);
  if (st >= 1 && st <= kModuleStages)
    return module_stage(st - 1, D, desc, w, u.xn, u, s, r, ln1_blk);
  switch (st) {
    case 0:
      r.mark("layernorm1");
      HSMLA_TRY(hsmla::launch_layernorm(D.bf, x, f->ln1_g, f->ln1_b, u.xn, P, C, s,
                                        ln1_blk));
      return HSMLA_OK;
    case kModuleStages + 1: {
      // x1 = x + O W_o (residual fused into the projection epilogue)
      r.mark("out_proj_residual");
      const WSel wo = wsel(D, u.wo);
      HSMLA_TRY(hsmla::launch_gemm(D.bf, u.o, wo.w, x, u.x1, P, C, C, s,
                                   hsmla::GemmSite::kOut, false, wo.blocked));
      return HSMLA_OK;
    }
    case kModuleStages + 2:
      r.mark("layernorm2");
      HSMLA_TRY(hsmla::launch_layernorm(D.bf, u.x1, f->ln2_g, f->ln2_b, u.xn, P,
                                        C, s, ln2_blk));
      return HSMLA_OK;
    case kModuleStages + 3: {
      r.mark("ffn1_gemm");
      const WSel w1 = wsel(D, u.w1);
      HSMLA_TRY(hsmla::launch_gemm(D.bf, u.xn, w1.w, nullptr, u.h1, P, 4 * C, C, s,
                                   hsmla::GemmSite::kFfn1, ln2_blk, w1.blocked, h1_planar));
      return HSMLA_OK;
    }
    case kModuleStages + 4: {
      r.mark("ffn_dwconv_gelu");
      if (h1_planar)
        HSMLA_TRY(hsmla::launch_dwconv_gelu_planar(u.h1, u.h2, u.ftaps, D.B, D.gh, D.gw,
                                                   4 * C, s));
      else
        HSMLA_TRY(hsmla::launch_dwconv(D.bf, u.h1, u.h2, u.ftaps, 3, D.B, D.gh,
                                       D.gw, 4 * C, true, nullptr, 1, s, h2_blk));
      r.mark("ffn2_gemm_residual");
      const WSel w2 = wsel(D, u.w2);
      HSMLA_TRY(hsmla::launch_gemm(D.bf, u.h2, w2.w, u.x1, out, P, C, 4 * C, s,
                                   hsmla::GemmSite::kFfn2, h2_blk, w2.blocked));
      return HSMLA_OK;
    }
    default:
      return HSMLA_ERR_ARG;
  }
}

hsmla_status block_range(const Dims& D, const hsmla_desc* desc,
                         const hsmla_weights* w, const hsmla_ffn_weights* f,
                         const void* x, void* out, const Bufs& u, hipStream_t s,
                         Rec& r) {
  for (int st = 0; st < kBlockStages; ++st) {
    const hsmla_status e = block_stage(st, D, desc, w, f, x, out, u, s, r);
    if (e != HSMLA_OK) return e;
  }
  return HSMLA_OK;
}

hsmla_status block_impl(const hsmla_desc* desc, const hsmla_weights* w,
                        const hsmla_ffn_weights* f, const void* x, void* out,
                        void* ws, size_t ws_bytes, hipStream_t s, Rec& r) {
  Dims D;
  Layout L;
  hsmla_status st = check_block(desc, w, f, x, out, ws, ws_bytes, &D, &L);
  if (st != HSMLA_OK) return st;
  const Bufs u = bufs_for(D, L, ws, HSMLA_OP_BLOCK, 0);
  if (!D.prepared && (st = prep(D, desc, w, f, u, s, r)) != HSMLA_OK) return st;
  if ((st = block_range(D, desc, w, f, x, out, u, s, r)) != HSMLA_OK) return st;
  r.end();
  return r.ok ? HSMLA_OK : HSMLA_ERR_HIP;
}

// Two image ranges on two streams.  Every kernel of the block works image
// by image with a tiling that does not depend on the batch (bf16 path), so
// each range reproduces the single-stream result bit for bit.
hsmla_status block_split_impl(const hsmla_desc* desc, const hsmla_weights* w,
                              const hsmla_ffn_weights* f, const void* x,
                              void* out, void* ws, size_t ws_bytes,
                              hipStream_t s, hipStream_t aux, hipEvent_t fork,
                              hipEvent_t join) {
  Dims D;
  Layout L;
  hsmla_status st = check_block(desc, w, f, x, out, ws, ws_bytes, &D, &L);
  if (st != HSMLA_OK) return st;
  Rec r;
  // float32 chunks the K/V reduction by batch size: one stream keeps the
  // result independent of the split
  const Bufs u0 = bufs_for(D, L, ws, HSMLA_OP_BLOCK, 0);
  if (!D.prepared && (st = prep(D, desc, w, f, u0, s, r)) != HSMLA_OK) return st;
  if (D.B < 2 || !D.bf) return block_range(D, desc, w, f, x, out, u0, s, r);
  HSMLA_TRY(hipEventRecord(fork, s));
  HSMLA_TRY(hipStreamWaitEvent(aux, fork, 0));
  const int nb0 = (D.B + 1) / 2, nb1 = D.B - nb0;
  const size_t img = (size_t)D.N * D.C * D.e;
  const Dims D0 = range_dims(D, nb0), D1 = range_dims(D, nb1);
  const Bufs u1 = bufs_for(D, L, ws, HSMLA_OP_BLOCK, nb0);
  const void* x1 = at(const_cast<void*>(x), nb0 * img);
  void* out1 = at(out, nb0 * img);
  // the two ranges' launches are enqueued alternately, stage by stage, so
  // both streams have work from the start
  for (int k = 0; k < kBlockStages; ++k) {
    if ((st = block_stage(k, D0, desc, w, f, x, out, u0, s, r)) != HSMLA_OK) return st;
    if ((st = block_stage(k, D1, desc, w, f, x1, out1, u1, aux, r)) != HSMLA_OK) return st;
  }
  HSMLA_TRY(hipEventRecord(join, aux));
  HSMLA_TRY(hipStreamWaitEvent(s, join, 0));
  return HSMLA_OK;
}

Rec make_rec(void* const* events, const char** names, int32_t n_events,
             hipStream_t s) {
  Rec r;
  r.ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  r.names = names;
  r.cap = n_events;
  r.s = s;
  return r;
}

}  // namespace

extern "C" {

hsmla_status hsmla_forward(const hsmla_desc* desc, const hsmla_weights* w,
                           const void* x, void* y, void* ws, size_t ws_bytes,
                           void* stream) {
  Rec r;
  return forward_impl(desc, w, x, y, ws, ws_bytes,
                      static_cast<hipStream_t>(stream), r);
}

hsmla_status hsmla_block_forward(const hsmla_desc* desc, const hsmla_weights* w,
                                 const hsmla_ffn_weights* f, const void* x,
                                 void* out, void* ws, size_t ws_bytes,
                                 void* stream) {
  Rec r;
  return block_impl(desc, w, f, x, out, ws, ws_bytes,
                    static_cast<hipStream_t>(stream), r);
}

hsmla_status hsmla_block_forward_split(const hsmla_desc* desc,
                                       const hsmla_weights* w,
                                       const hsmla_ffn_weights* f,
                                       const void* x, void* out, void* ws,
                                       size_t ws_bytes, void* stream,
                                       void* aux_stream, void* fork_event,
                                       void* join_event) {
  if (!fork_event || !join_event) return HSMLA_ERR_NULL;
  if (aux_stream == stream) return HSMLA_ERR_ARG;
  return block_split_impl(desc, w, f, x, out, ws, ws_bytes,
                          static_cast<hipStream_t>(stream),
                          static_cast<hipStream_t>(aux_stream),
                          static_cast<hipEvent_t>(fork_event),
                          static_cast<hipEvent_t>(join_event));
}

hsmla_status hsmla_forward_timed(const hsmla_desc* desc, const hsmla_weights* w,
                                 const void* x, void* y, void* ws,
                                 size_t ws_bytes, void* stream,
                                 void* const* events, const char** names,
                                 int32_t n_events, int32_t* n_launches) {
  if (!events || !n_launches || n_events < 1) return HSMLA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Rec r = make_rec(events, names, n_events, s);
  const hsmla_status st = forward_impl(desc, w, x, y, ws, ws_bytes, s, r);
  *n_launches = r.n;
  if (st == HSMLA_OK && r.n + 1 > n_events) return HSMLA_ERR_ARG;
  return st;
}

hsmla_status hsmla_block_forward_timed(const hsmla_desc* desc,
                                       const hsmla_weights* w,
                                       const hsmla_ffn_weights* f,
                                       const void* x, void* out, void* ws,
                                       size_t ws_bytes, void* stream,
                                       void* const* events, const char** names,
                                       int32_t n_events, int32_t* n_launches) {
  if (!events || !n_launches || n_events < 1) return HSMLA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Rec r = make_rec(events, names, n_events, s);
  const hsmla_status st = block_impl(desc, w, f, x, out, ws, ws_bytes, s, r);
  *n_launches = r.n;
  if (st == HSMLA_OK && r.n + 1 > n_events) return HSMLA_ERR_ARG;
  return st;
}

}  // extern "C"
