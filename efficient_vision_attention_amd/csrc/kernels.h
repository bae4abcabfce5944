// Host-side launchers of the HSMLA kernels.  Each returns hipSuccess or the
// launch error.  Shapes are validated by the caller (hsmla_api.hip); the
// launchers assume them.  `bf` selects bfloat16 (true) or float32 storage.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hsmla {

// Which projection a GEMM launch is (only used to name the kernel symbol).
enum class GemmSite { kQkv, kOut, kFfn1, kFfn2 };

// Tile shape of the bf16 GEMM.  Its whole-tile path (M, N, K multiples of
// the tile) can read "tile-blocked" operands: element (r, k) of a row-major
// [R][K] matrix stored at ((r / TR) * (K / 32) + k / 32) * TR * 32 +
// (r % TR) * 32 + k % 32, so one K step of one tile is one contiguous block;
// TR = kGemmTileM for A, kGemmTileN for W.
constexpr int kGemmTileM = 256, kGemmTileN = 128, kGemmTileK = 32;
bool gemm_whole_tiles(int M, int N, int K);

// C[M][N] = A[M][K] . W[N][K]^T (+ R[M][N] when R != nullptr), row-major C
// and R.  N and K must be multiples of 32 (8-element chunks are loaded
// whole).  a_blocked / w_blocked: A / W are tile-blocked (bf16 and
// gemm_whole_tiles(M, N, K) only; otherwise hipErrorInvalidValue).
// c_planar: C written channel-planar, element (m, n) at
// (n / 64) * M * 64 + m * 64 + n % 64 (only where gemm_planar_ok: bf16,
// tile-blocked A and W, whole tiles, K = 384 or 1536).
hipError_t launch_gemm(bool bf, const void* A, const void* W, const void* R,
                       void* C, int M, int N, int K, hipStream_t s,
                       GemmSite site, bool a_blocked = false,
                       bool w_blocked = false, bool c_planar = false);
bool gemm_planar_ok(bool bf, int M, int N, int K, bool a_blocked, bool w_blocked);

// Effective depthwise taps: weff[tap][ch] (float32, kmax x kmax taps) =
// identity (centre tap += 1 when `identity`) + sum of the given kernels,
// each zero-padded to kmax.  kernels[i] is [ch][k_i][k_i].
hipError_t launch_dw_taps(bool bf, const void* const* kernels, const int* ks,
                          int nk, int kmax, int ch, int identity, float* weff,
                          hipStream_t s);

// One launch folding up to two tap sets (as launch_dw_taps) and writing the
// GEMM's copies of up to four projection weights: src is [cols][rows]
// row-major ([in][out], y = x . src), dst its transpose [rows][cols] =
// [out][in], row-major (tile_rows = 0; cols a multiple of 8) or tile-blocked
// with tile_rows = kGemmTileN (bf16 only; rows a multiple of tile_rows, cols
// of kGemmTileK).
struct TapSpec {
  const void* kernels[3];
  int ks[3];
  int nk, kmax, ch, identity;
  float* weff;
};
struct BlockJob {
  const void* src;  // [cols][rows] row-major
  void* dst;        // [rows][cols]: row-major or tile-blocked
  int rows, cols, tile_rows;
};
hipError_t launch_prep(bool bf, const TapSpec* taps, int ntaps,
                       const BlockJob* jobs, int njobs, hipStream_t s);

// out[b][y][x][c] = act(sum_tap weff[tap][c] * in[b][y+dy-r][x+dx-r][c]),
// zero padding, r = (kmax-1)/2; act = exact GELU when `gelu`.  With bsum
// (no GELU; dwconv_can_pool(kmax, block) must hold) the launch also writes
// bsum[b][t][c] = sum of the stored out values over block t (block x block
// tokens, blocks numbered row-major).
bool dwconv_can_pool(int kmax, int block);
// With gate_w ([heads][96], the gate's per-head weights; ch = 3 * 32 *
// heads) the pooled sums go straight into the gate's partial logits,
// bsum[b][t][s][h] = sum_j gate_w[h][32 s + j] * blocksum(s C + 32 h + j)
// (s: Q, K, V; C = 32 heads), instead of bsum[b][t][c].
hipError_t launch_dwconv(bool bf, const void* in, void* out, const float* weff,
                         int kmax, int batch, int gh, int gw, int ch,
                         bool gelu, float* bsum, int block, hipStream_t s,
                         bool out_blocked = false, const float* gate_w = nullptr,
                         int heads = 0);
// Whether launch_dwconv can write out tile-blocked as the GEMM's A operand
// (bf16 3x3 with GELU, token count a multiple of kGemmTileM, under 2 GiB).
bool dwconv_can_block_out(bool bf, int kmax, bool gelu, int batch, int gh, int gw,
                          int ch);

// The FFN's conv + GELU from a channel-planar input (as launch_gemm writes
// it with c_planar) to the tile-blocked output of launch_dwconv; only where
// dwconv_planar_ok (bf16, out_blocked possible, gw a multiple of 256, ch a
// multiple of 64).
bool dwconv_planar_ok(bool bf, int batch, int gh, int gw, int ch);
hipError_t launch_dwconv_gelu_planar(const void* in, void* out, const float* weff, int batch,
                                     int gh, int gw, int ch, hipStream_t s);

// Number of token chunks the KV-state reduction splits each image into, for
// a call of `batch` images.
int kv_chunks(bool bf, int batch, int heads, int tokens);

// Z/D partials per chunk, then a fixed-order combine into kv and ksum.
// chunk_batch: the batch of the whole call whose images [.., + batch) this
// launch covers (bf16 chunks by it; 0 = batch); partials hold
// kv_chunks(bf, chunk_batch, ...) chunks per (image, head).
hipError_t launch_kv_state(bool bf, const void* qkv_hat, float* kv,
                           float* ksum, float* partials, int batch, int tokens,
                           int heads, hipStream_t s, int chunk_batch = 0);

// launch_kv_state (bfloat16) with the gate's top-k from its partial logits
// in the same two launches (as launch_gate_topk_parts: scores and the
// ascending list of the keep best blocks of each image; rankp as its parts,
// 128 .. 1024 blocks per image, see gate_topk_from_parts_ok).
hipError_t launch_kv_state_topk(const void* qkv_hat, float* kv, float* ksum, float* partials,
                                int batch, int tokens, int heads, hipStream_t s,
                                int chunk_batch, const float* plog, const float* gate_b,
                                float* scores, int32_t* sel, int32_t* rankp, int nblocks,
                                int block, int keep);

// o = relu(q_hat) Z / (relu(q_hat) . D), zero when the denominator is 0.
hipError_t launch_lin_apply(bool bf, const void* qkv_hat, const float* kv,
                            const float* ksum, void* o, int batch, int tokens,
                            int heads, hipStream_t s);

// Gate scores per block, then top-k selection.
// gate_dw: nullptr, or the gate's depthwise 3x3 kernel [3C][3][3] in the
// activation type (16-byte aligned).  head_scores (optional): G^(h) per
// block and head, [batch][blocks][heads].
// The same scores from block sums (bsum [batch][blocks][3C], e.g. written
// by launch_dwconv): M_t and optionally G^(h)_t.
hipError_t launch_gate_from_sums(const float* bsum, const float* gate_w,
                                 const float* gate_b, float* scores,
                                 float* head_scores, int batch, int nblocks,
                                 int heads, int block, hipStream_t s);
hipError_t launch_gate_scores(bool bf, const void* qkv_hat,
                              const float* gate_w, const float* gate_b,
                              const void* gate_dw, float* scores,
                              float* head_scores, int batch, int gh, int gw,
                              int heads, int block, hipStream_t s);
// parts (optional, batch * topk_parts_bytes(nblocks) bytes; ignored with
// scores_copy): scratch that lets 128 .. 1024 blocks per image be ranked
// over several workgroups per image (two launches).
size_t topk_parts_bytes(int nblocks);
// Top-k from the gate's partial logits (written by launch_dwconv with
// gate_w): M_t = mean_h sigmoid((plog[t][0][h] + plog[t][1][h] +
// plog[t][2][h]) / block^2 + gate_b[h]) into scores, then the selection as
// launch_topk with parts (required; 128 .. 1024 blocks per image, see
// gate_topk_from_parts_ok).
bool gate_topk_from_parts_ok(int nblocks);
hipError_t launch_gate_topk_parts(const float* plog, const float* gate_b, float* scores,
                                  int32_t* sel, int32_t* parts, int batch, int nblocks,
                                  int heads, int block, int keep, hipStream_t s);
// The scores alone from the same partial logits (the threshold routings and
// the soft mixture): M_t into scores and, when head_scores is not null,
// G^(h)_t = sigmoid((plog[t][0][h] + plog[t][1][h] + plog[t][2][h]) /
// block^2 + gate_b[h]) into head_scores [batch][blocks][heads]; the block
// scores equal launch_gate_topk_parts' bit for bit.
hipError_t launch_gate_from_parts(const float* plog, const float* gate_b, float* scores,
                                  float* head_scores, int batch, int nblocks, int heads,
                                  int block, hipStream_t s);
hipError_t launch_topk(const float* scores, float* scores_copy, int32_t* sel,
                       int batch, int nblocks, int keep, hipStream_t s,
                       int32_t* parts = nullptr);
// Threshold routing: sel[b][0 .. counts[b]) = ascending blocks with score >
// tau; sel rows are nblocks wide.
hipError_t launch_threshold(const float* scores, float* scores_copy,
                            int32_t* sel, int32_t* counts, int batch,
                            int nblocks, float tau, hipStream_t s);
// Per-head routing: sel[b][h][0 .. counts[b][h]) = ascending blocks with
// head_scores[b][t][h] > tau.
hipError_t launch_threshold_heads(const float* head_scores, float* copy,
                                  int32_t* sel, int32_t* counts, int batch,
                                  int nblocks, int heads, float tau,
                                  hipStream_t s);

// Where the sparse launch finds the list of (image b, head h): entry x is
// sel[b * sel_b + h * sel_h + x]; with counts != nullptr only entries x <
// counts[b * cnt_b + h * cnt_h] are refined.
struct SelLayout {
  int sel_b, sel_h, cnt_b, cnt_h;
};

// Windowed softmax refinement of the selected blocks, in place on o; the
// grid covers `entries` list entries per (image, head).  sel == nullptr
// refines every block (entry x = block x); wts != nullptr ([batch][blocks])
// scales each block's residual by its weight.
hipError_t launch_sparse(bool bf, const void* qkv, const void* qkv_hat,
                         const int32_t* sel, const int32_t* counts,
                         const float* wts, void* o, int batch, int gh, int gw,
                         int heads, int block, int window, int entries,
                         SelLayout lay, hipStream_t s);

// y = LN(x) . gamma + beta over the channel dimension.
hipError_t launch_layernorm(bool bf, const void* x, const float* gamma,
                            const float* beta, void* y, int rows, int ch,
                            hipStream_t s, bool blocked = false);
// Whether launch_layernorm can write y tile-blocked as the GEMM's A operand
// (bf16, rows a multiple of kGemmTileM, rows of 128..512 channels).
bool layernorm_can_block(bool bf, int rows, int ch);

}  // namespace hsmla
