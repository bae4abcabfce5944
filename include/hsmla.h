/*
 * hsmla.h -- C ABI of libhsmla.so, the HSMLA attention forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources named below:
 *   FT = "HSMLA: Hierarchical Softmax Multi-scale Linear Attention for
 *        Efficient Vision Transformers", full text (paperpeel.com rendering).
 *   EX = the gist.science explainer of the same paper, section
 *        "Technische Samenvatting".
 *
 * Module computed (FT 3.1-3.3, 3.5, 3.6):
 *   QKV     = X W_qkv                                  (projection, no bias)
 *   T_hat   = T + sum_s DWConv_{k_s}(T)  for T in Q,K,V (multi-scale branches)
 *   Z, D    = sum_j relu(K_hat_j)^T V_hat_j, sum_j relu(K_hat_j)   (per head)
 *   O_lin   = relu(Q_hat) Z / (relu(Q_hat) . D)           (0 when the sum is 0)
 *   M_t     = mean_h sigmoid(w_h . meanpool_t[Q_hat;K_hat;V_hat]_h + b_h),
 *             or, with the gate kernel g, meanpool_t of DWConv3x3_g(...)
 *   sel     = the keep_blocks blocks with the largest M_t (ties -> lower t),
 *             or, with threshold routing, every block with M_t > tau
 *   O_i     = O_lin_i + softmax-attn(q_i, K_W, V_W) - lin-local_i  on sel
 *   Y       = O W_o
 *
 * Conventions shared by every entry point:
 *   - Layout: a token grid of grid_h x grid_w tokens, token n = y*grid_w + x.
 *     Activations are row-major [batch][n][channels].  The projected tensor
 *     is [batch][n][3C] with channel s*C + h*head_dim + j holding component
 *     s (0 = Q, 1 = K, 2 = V) of head h.  Blocks are block x block tiles,
 *     numbered row-major over the block grid.
 *   - Element type: desc->dtype selects float32 or bfloat16 for activations
 *     and weights (the `const void*` arguments).  Gate weights, LayerNorm
 *     parameters, Z, D and scores are always float32.  All arithmetic
 *     accumulates in float32; bfloat16 results are rounded to nearest even.
 *   - Ownership: the caller allocates every buffer (device memory).  The
 *     library allocates nothing, frees nothing and keeps no pointer after a
 *     call returns.  Buffers must stay valid until the stream reaches the
 *     work.  Inputs and outputs must not overlap unless stated.
 *   - Asynchrony: every call only enqueues work on `stream` (a hipStream_t;
 *     NULL = the default stream) and never synchronises.
 *   - Errors: argument errors are detected on the host before any HIP call
 *     and returned as a negative hsmla_status; nothing is launched then.  A
 *     failed launch returns HSMLA_ERR_HIP.  No exception crosses the ABI.
 *   - Weights of the dense projections are [in][out] row-major and are
 *     applied as y = x . W.  The library keeps its own copy of each in the
 *     workspace in the layout its matrix-core kernels read (written by a
 *     preparation launch at the start of every call, or once by
 *     hsmla_prepare when desc->prepared is set).
 *   - Alignment: activation, weight and workspace pointers must be 16-byte
 *     aligned; float32 parameter and index pointers 4-byte aligned.
 *   - Threading: no mutable global state; calls on different streams may
 *     run concurrently if their buffers do not overlap.
 *   - Limits: head_dim must be 32; block <= 16; window >= block with
 *     (window - block) even; grid_h and grid_w multiples of block;
 *     0 <= keep_blocks <= number of blocks <= 8192; channels <= 2048;
 *     up to 3 depthwise branches of odd size <= 7; routing is one of
 *     hsmla_routing (otherwise HSMLA_ERR_ARG), and tau is not NaN under the
 *     threshold routings (keep_blocks is then unused but still
 *     range-checked).
 */
#ifndef HSMLA_H_
#define HSMLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSMLA_OK = 0,
  HSMLA_ERR_NULL = -1,      /* a required pointer is NULL                  */
  HSMLA_ERR_SHAPE = -2,     /* sizes violate the limits above              */
  HSMLA_ERR_DTYPE = -3,     /* unknown dtype                               */
  HSMLA_ERR_ALIGN = -4,     /* a pointer is not aligned as required        */
  HSMLA_ERR_WORKSPACE = -5, /* workspace smaller than hsmla_workspace_bytes */
  HSMLA_ERR_HIP = -6,       /* a kernel launch failed                      */
  HSMLA_ERR_ARG = -7,       /* other invalid argument (e.g. unknown op)    */
  HSMLA_ERR_SCRATCH = -8    /* sizes exceed hsmla_linear_attn_noalloc's    */
                            /* static scratch                              */
} hsmla_status;

typedef enum { HSMLA_F32 = 0, HSMLA_BF16 = 1 } hsmla_dtype;

/* How blocks are routed to the softmax path (FT 3.2).  TOPK keeps the
 * keep_blocks highest scores per image; THRESHOLD keeps every block whose
 * score exceeds desc->tau (the routed set {b : M_b > tau}), a per-image count
 * known only on the device; HEAD_THRESHOLD routes each head separately, by
 * its own head score: head h of block b is refined when G_b^(h) > tau (FT 3.2
 * per-head output routing), one list and count per (image, head).  SOFT is
 * the training-time differentiable mixture of FT 3.3, forward only: every
 * block is refined and its residual is scaled by its score,
 * O = O_lin + M_b (O_local - O_linloc). */
typedef enum {
  HSMLA_ROUTE_TOPK = 0,
  HSMLA_ROUTE_THRESHOLD = 1,
  HSMLA_ROUTE_HEAD_THRESHOLD = 2,
  HSMLA_ROUTE_SOFT = 3
} hsmla_routing;

/* Which entry point a workspace is sized for. */
typedef enum {
  HSMLA_OP_QKV = 0,     /* hsmla_qkv_branches   */
  HSMLA_OP_LINEAR = 1,  /* hsmla_linear_attn    */
  HSMLA_OP_FORWARD = 2, /* hsmla_forward        */
  HSMLA_OP_BLOCK = 3    /* hsmla_block_forward  */
} hsmla_op;

typedef struct {
  int32_t batch, grid_h, grid_w; /* N = grid_h * grid_w tokens per image  */
  int32_t channels, heads, head_dim; /* channels == heads * head_dim     */
  int32_t n_branches;            /* depthwise branches besides identity  */
  int32_t branch_k[3];           /* their (odd) kernel sizes              */
  int32_t block;                 /* block side Bs                          */
  int32_t window;                /* softmax window side w                  */
  int32_t keep_blocks;           /* refined blocks per image, 0..T (TOPK)  */
  int32_t dtype;                 /* hsmla_dtype                            */
  int32_t routing;               /* hsmla_routing                          */
  float tau;                     /* threshold of the threshold routings    */
  int32_t prepared;              /* nonzero: the workspace already holds  */
                                 /* the operands hsmla_prepare wrote for  */
                                 /* these weights; the call skips its own */
                                 /* preparation launch                    */
} hsmla_desc;

typedef struct {
  const void* w_qkv;   /* [C][3C]: qkv = x . w_qkv                      */
  const void* w_o;     /* [C][C]:  y = o . w_o                          */
  const void* dw[3];   /* branch s: [3C][k_s][k_s] cross-correlation     */
  const float* gate_w; /* [H][3*head_dim]: weights on [q; k; v] means    */
  const float* gate_b; /* [H]                                            */
  const void* gate_dw; /* NULL, or [3C][3][3]: the gate's depthwise 3x3   */
                       /* (FT 3.2 head-level score), 16-byte aligned      */
} hsmla_weights;

typedef struct {
  const float* ln1_g; const float* ln1_b; /* [C] LayerNorm before HSMLA */
  const float* ln2_g; const float* ln2_b; /* [C] LayerNorm before FFN   */
  const void* w1;      /* [C][4C]: h1 = LN2(x1) . w1                    */
  const void* dw_ffn;  /* [4C][3][3]                                    */
  const void* w2;      /* [4C][C]: out = x1 + h2 . w2                   */
} hsmla_ffn_weights;

/* Pointers into a forward/block workspace, for inspection. */
typedef struct {
  void* qkv;      /* [B][N][3C] projected Q, K, V                      */
  void* qkv_hat;  /* [B][N][3C] after the depthwise branches            */
  void* o;        /* [B][N][C]  attention output before W_o             */
  float* kv;      /* [B][H][d][d] Z                                     */
  float* ksum;    /* [B][H][d]   D                                      */
  float* scores;  /* [B][T] gate scores M                               */
  int32_t* sel;   /* [B][keep_blocks] (TOPK), [B][T] (THRESHOLD) or     */
                  /* [B][H][T] (HEAD_THRESHOLD); unused under SOFT      */
  int32_t* counts; /* THRESHOLD: [B]; HEAD_THRESHOLD: [B][H]; else NULL  */
  float* head_scores; /* HEAD_THRESHOLD: [B][T][H] G_b^(h); else NULL     */
  void* x1;       /* block only: [B][N][C] X + HSMLA(LN1(X))            */
} hsmla_views;

/* Bytes of workspace `op` needs for `desc` (written to *bytes). */
hsmla_status hsmla_workspace_bytes(const hsmla_desc* desc, int32_t op,
                                   size_t* bytes);

/* Fills `views` with the intermediate tensors that hsmla_forward (op =
 * HSMLA_OP_FORWARD) or hsmla_block_forward (HSMLA_OP_BLOCK) leave in `ws`
 * once the stream has completed.  Host-only pointer arithmetic. */
hsmla_status hsmla_workspace_views(const hsmla_desc* desc, int32_t op,
                                   void* ws, hsmla_views* views);

/* Writes the operands that depend only on the weights into the workspace
 * `ws` sized for `op` (HSMLA_OP_QKV, HSMLA_OP_FORWARD or HSMLA_OP_BLOCK;
 * HSMLA_ERR_ARG otherwise): the identity and depthwise branch kernels folded
 * into one tap set per channel (abstract, EX section 2; and the FFN's 3x3 of
 * the FT 3.5 sandwich for the block), and the dense projection weights
 * transposed, tile-blocked where the shape allows.  These are the same
 * values every call writes for itself when desc->prepared is 0.  A later
 * call of the same op with desc->prepared != 0, the same descriptor
 * otherwise and the same weights, on a stream ordered after this one, then
 * skips that launch; the weight sections of `ws` must not be written in
 * between (the views of hsmla_workspace_views never overlap them).  f is
 * required for HSMLA_OP_BLOCK (its w1, dw_ffn, w2) and ignored otherwise.
 * Asynchronous on `stream`, like every call. */
hsmla_status hsmla_prepare(const hsmla_desc* desc, int32_t op,
                           const hsmla_weights* w, const hsmla_ffn_weights* f,
                           void* ws, size_t ws_bytes, void* stream);

/* Steps 1-2 (FT 3.1 projection; abstract and EX section 2 for the
 * multi-scale depthwise branches): qkv = x W_qkv and
 * qkv_hat = qkv + sum_s DWConv_{k_s}(qkv), zero padding (k-1)/2, no bias.
 * x [B][N][C]; qkv, qkv_hat [B][N][3C]; ws sized for HSMLA_OP_QKV. */
hsmla_status hsmla_qkv_branches(const hsmla_desc* desc,
                                const hsmla_weights* w, const void* x,
                                void* qkv, void* qkv_hat, void* ws,
                                size_t ws_bytes, void* stream);

/* Step 3, the global linear path (FT 3.1 Z/D sums; FT 3.3 lin-local ratio
 * taken over all tokens).  qkv_hat [B][N][3C] in; o [B][N][C] out
 * (O_lin); kv [B][H][d][d] = Z (row: key feature, column: value feature)
 * and ksum [B][H][d] = D out, float32.  The reduction over tokens is split
 * in fixed chunks and combined in a fixed order, so results are bitwise
 * reproducible.  ws sized for HSMLA_OP_LINEAR. */
hsmla_status hsmla_linear_attn(const hsmla_desc* desc, const void* qkv_hat,
                               void* o, float* kv, float* ksum, void* ws,
                               size_t ws_bytes, void* stream);

/* hsmla_linear_attn for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, bit for bit, with the chunk
 * partials of the K/V-state reduction in a static device array of the
 * library (16 MiB per GPU, held from the library's load until the process
 * ends) instead of a caller workspace.  The call allocates nothing.  Sizes
 * whose partials exceed the array (hsmla_workspace_bytes(desc,
 * HSMLA_OP_LINEAR) > 16 MiB; in bf16, batch * heads * chunks above 3971,
 * chunks = ceil(N / 512) -- or ceil(N / 256), ceil(N / 128) for calls of
 * fewer than 256 partial workgroups) return HSMLA_ERR_SCRATCH before any
 * launch.  Every call on one GPU
 * uses that GPU's one array: calls that can overlap on a GPU (different
 * streams, or other threads) race and must be serialised by the caller.
 * The first call on each device looks up the array's address with that
 * device current (a HIP runtime query, no allocation). */
hsmla_status hsmla_linear_attn_noalloc(const hsmla_desc* desc, const void* qkv_hat,
                                       void* o, float* kv, float* ksum,
                                       void* stream);

/* Step 4, block gate and selection (FT 3.2 head-level score and block-level
 * aggregation; gate shared by all heads per EX section 2).  With
 * scores_in == NULL the scores M [B][T] are pooled from qkv_hat and written
 * to scores_out (required); gate_dw NULL pools the hatted tokens, gate_dw
 * [3C][3][3] (activation type, 16-byte aligned) pools their depthwise 3x3
 * convolution, taken over the whole grid with zero padding at the image
 * border, as in the head-level score equation.  With scores_in != NULL those float32 scores are
 * ranked instead (qkv_hat, gate_w, gate_b may be NULL) and copied to
 * scores_out if it is not NULL.  sel [B][keep_blocks] receives, per image,
 * the indices of the keep_blocks largest scores (equal scores: lower index
 * first), in ascending order.  Scores must not be NaN.  desc->routing must be
 * HSMLA_ROUTE_TOPK (HSMLA_ERR_ARG otherwise). */
hsmla_status hsmla_gate_select(const hsmla_desc* desc, const void* qkv_hat,
                               const float* gate_w, const float* gate_b,
                               const void* gate_dw, const float* scores_in,
                               float* scores_out, int32_t* sel, void* stream);

/* Step 4 with threshold routing (FT 3.2, the routed set B_tau of the
 * activation-ratio equation; FT 3.3 routing case G > tau; EX section 2
 * "Routing").  Scores as in hsmla_gate_select; desc->routing must be
 * HSMLA_ROUTE_THRESHOLD (HSMLA_ERR_ARG otherwise).  sel[b][0 .. counts[b])
 * receives, in ascending order, every block of image b whose float32 score
 * is strictly greater than desc->tau; entries of sel beyond counts[b] are
 * left as they were.  sel [B][T] int32 (T = number of blocks), counts [B]
 * int32, both device memory written by the kernel: the count is not known
 * on the host. */
hsmla_status hsmla_gate_threshold(const hsmla_desc* desc, const void* qkv_hat,
                                  const float* gate_w, const float* gate_b,
                                  const void* gate_dw, const float* scores_in,
                                  float* scores_out, int32_t* sel,
                                  int32_t* counts, void* stream);

/* Step 4 with per-head routing (FT 3.2 head-level score and per-head output
 * routing equation); desc->routing must be HSMLA_ROUTE_HEAD_THRESHOLD
 * (HSMLA_ERR_ARG otherwise).  With head_scores_in == NULL the head scores
 * G [B][T][H] are pooled from qkv_hat (gate_dw as in hsmla_gate_select) and
 * written to head_scores_out (required); with head_scores_in those float32
 * scores are thresholded instead (qkv_hat and the gate weights may be NULL)
 * and copied to head_scores_out if it is not NULL.  sel[b][h][0 ..
 * counts[b][h]) receives, ascending, every block whose float32 G_b^(h) is
 * strictly greater than desc->tau; entries beyond the count are left as
 * they were.  sel [B][H][T], counts [B][H] int32, device memory. */
hsmla_status hsmla_gate_head_threshold(const hsmla_desc* desc,
                                       const void* qkv_hat,
                                       const float* gate_w, const float* gate_b,
                                       const void* gate_dw,
                                       const float* head_scores_in,
                                       float* head_scores_out, int32_t* sel,
                                       int32_t* counts, void* stream);

/* Step 5, local softmax refinement of the selected blocks with the two-path
 * residual (FT 3.3 local-neighbourhood, lin-local and residual equations;
 * scatter of the sparse residual, FT 3.6 stage 5).  For every block in sel
 * and every head, each query i of the block gets
 *   o_i <- o_i + softmax_j(q_i.k_j / sqrt(d)) v_j - lin-local_i
 * over the window x window keys centred on the block and clipped to the
 * grid, with raw q, k, v from qkv and lin-local from qkv_hat.  o holds O_lin
 * on entry; tokens of unselected blocks are not touched.  sel entries must
 * be distinct valid block indices.  desc->routing must be HSMLA_ROUTE_TOPK
 * (HSMLA_ERR_ARG otherwise; see hsmla_sparse_softmax_counted). */
hsmla_status hsmla_sparse_softmax(const hsmla_desc* desc, const void* qkv,
                                  const void* qkv_hat, const int32_t* sel,
                                  void* o, void* stream);

/* Step 5 over a device-counted selection (the threshold-routed set, FT 3.3
 * sparse residual over |B_tau| blocks): as hsmla_sparse_softmax, for the
 * lists hsmla_gate_threshold or hsmla_gate_head_threshold write.  With
 * HSMLA_ROUTE_THRESHOLD every head of the first counts[b] blocks of
 * sel[b][0 .. T) is refined; with HSMLA_ROUTE_HEAD_THRESHOLD head h of the
 * first counts[b][h] blocks of sel[b][h][0 .. T).  Other routings:
 * HSMLA_ERR_ARG.  The launch covers T entries per (image, head); work items
 * at or beyond the count exit before reading sel. */
hsmla_status hsmla_sparse_softmax_counted(const hsmla_desc* desc,
                                          const void* qkv, const void* qkv_hat,
                                          const int32_t* sel,
                                          const int32_t* counts, void* o,
                                          void* stream);

/* Step 5 of the training-time mixture (FT 3.3 differentiable mixture
 * equation, forward only): every block of every image is refined and its
 * residual is scaled by weights[b][t] (float32, [B][T]; the block scores M
 * in the forward pass): o_i <- o_i + w (softmax part - lin-local part), as
 * in hsmla_sparse_softmax otherwise.  desc->routing must be
 * HSMLA_ROUTE_SOFT (HSMLA_ERR_ARG otherwise). */
hsmla_status hsmla_sparse_softmax_weighted(const hsmla_desc* desc,
                                           const void* qkv, const void* qkv_hat,
                                           const float* weights, void* o,
                                           void* stream);

/* The whole module: y = HSMLA(x) = O W_o, steps 1-5 then the output
 * projection (FT 3.6 stages 1-5).  x, y [B][N][C]; ws sized for
 * HSMLA_OP_FORWARD; intermediates readable through hsmla_workspace_views.
 * desc->routing picks top-k, threshold, per-head threshold selection or
 * the soft mixture (the views then also give the counts, and for per-head
 * routing the head scores). */
hsmla_status hsmla_forward(const hsmla_desc* desc, const hsmla_weights* w,
                           const void* x, void* y, void* ws, size_t ws_bytes,
                           void* stream);

/* One block (FT 3.5 block equation, with its depthwise and FFN steps fused
 * into one FFN-DWConv sandwich):
 *   x1  = x + HSMLA(LN1(x))
 *   out = x1 + GELU(DWConv3x3(LN2(x1) W1)) W2
 * LayerNorm: biased variance, eps 1e-5; GELU: exact erf form.  x, out
 * [B][N][C] (must not overlap); ws sized for HSMLA_OP_BLOCK. */
hsmla_status hsmla_block_forward(const hsmla_desc* desc,
                                 const hsmla_weights* w,
                                 const hsmla_ffn_weights* f, const void* x,
                                 void* out, void* ws, size_t ws_bytes,
                                 void* stream);

/* hsmla_block_forward with the batch split in two image ranges, the first
 * on `stream` and the second on `aux_stream`, so that the kernels of one
 * half fill the chip while those of the other half drain.  Each image's
 * result does not depend on the batch it is computed in, so `out` and the
 * workspace views equal those of hsmla_block_forward bit for bit (the
 * split is a scheduling choice, not a change of the block of FT 3.5).
 * fork_event, join_event: hipEvent_t handles owned by the caller (created
 * with default flags or hipEventDisableTiming); the call records fork_event
 * on `stream` and makes aux_stream wait on it, records join_event on
 * aux_stream at the end and makes `stream` wait on it, so work queued on
 * `stream` afterwards sees the whole output.  aux_stream must differ from
 * `stream`; both keep the default priority.  float32 descriptors and
 * batches of one image run on `stream` alone.  Concurrent calls must not
 * share the events or the workspace.  HSMLA_ERR_ARG when aux_stream equals
 * stream; otherwise the errors of hsmla_block_forward. */
hsmla_status hsmla_block_forward_split(const hsmla_desc* desc,
                                       const hsmla_weights* w,
                                       const hsmla_ffn_weights* f,
                                       const void* x, void* out, void* ws,
                                       size_t ws_bytes, void* stream,
                                       void* aux_stream, void* fork_event,
                                       void* join_event);

/* Same work, kernels and stream order as hsmla_forward /
 * hsmla_block_forward, plus an event recorded on `stream` before each
 * launch step and one after the last, for per-step timing by the caller.
 * A step is one kernel launch or two dependent ones under one name: the
 * K/V state ("kv_state": partial sums, then their combine; in bfloat16 runs
 * with top-k routing "kv_state_gate_topk", whose two launches also rank the
 * gate's scores and write the block lists) and the top-k ("gate_topk" or
 * "topk") where it runs on its own.
 * events: n_events hipEvent_t handles created by the caller; names
 * (nullable): receives a static name per recorded event ("end" for the
 * last).  *n_launches receives the number of steps L; events 0..L are
 * recorded when n_events >= L + 1, otherwise only the first n_events and
 * HSMLA_ERR_ARG is returned after the work is enqueued. */
hsmla_status hsmla_forward_timed(const hsmla_desc* desc,
                                 const hsmla_weights* w, const void* x,
                                 void* y, void* ws, size_t ws_bytes,
                                 void* stream, void* const* events,
                                 const char** names, int32_t n_events,
                                 int32_t* n_launches);
hsmla_status hsmla_block_forward_timed(const hsmla_desc* desc,
                                       const hsmla_weights* w,
                                       const hsmla_ffn_weights* f,
                                       const void* x, void* out, void* ws,
                                       size_t ws_bytes, void* stream,
                                       void* const* events,
                                       const char** names, int32_t n_events,
                                       int32_t* n_launches);

/* Static description of a status code. */
const char* hsmla_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* HSMLA_H_ */
