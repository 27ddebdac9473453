// Parameter blocks and launchers of the gfx950 kernels (internal to libpe).
#pragma once
#include "common.h"

namespace pe {

struct BatchParams {
  int R, K, T, target_rows, mask_token_id;
  int row_bytes;  // 3 * hidden * element size (multiple of 16)
  const int32_t *cu_window, *n_rej, *kv_len, *kv_base, *window_ids, *window_pos,
      *window_hrow, *new_token, *ctx_hrow;
  const void *target_hidden, *h_shared;
  int32_t *draft_ids, *draft_pos, *slot_mapping, *hidden_src, *req_of_row, *query_rows, *cu_draft;
  uint8_t *rejected, *masked;
  void* draft_hidden;
};
void launch_build_draft_batch(const BatchParams& p, hipStream_t s);

struct NormParams {
  const void* in;
  int64_t ld_in;         // elements between input rows
  const int32_t* rows;   // [n] source rows or nullptr (identity)
  const uint8_t* skip;   // flags indexed by source row, or nullptr
  int n, segs, d;        // rows, segments per row, segment length
  const float* gain;     // [segs * d]
  float eps;
  void* out;
  int64_t ld_out;
  int* zero;             // counters cleared by the launch (block 0), or nullptr
  int nzero;
  // Deferred scale: when set, out holds x * gain only (no 1 / rms) and
  // inv_out[i * segs + seg] receives the row segment's 1 / rms (0 for skipped
  // rows); the contraction applies it to its sum over that segment.  With
  // unit gains and bf16 input the operand is then the input itself, exact.
  float* inv_out;
  // bf16 output only: 0 = rows of ld_out elements; 1 = the matrix-core operand
  // layout of the large-M contractions (ld_out = K, a multiple of 32): the
  // 16-row x 32-column piece (G, S) is the 1 KB chunk G * (K / 32) + S, whose
  // 16-byte lane slot 16 c + r holds row 16 G + r, columns 32 S + 8 c .. + 7.
  // Rows n .. n_pad - 1 (n_pad = n rounded up to 16) are written as zeros.
  int packed;
};
// Row count limit of one segment: 8 x 256 sixteen-byte chunks per row.
constexpr int kNormMaxChunks = 8;
// Packed output: a wave per row, at most this many 16-byte chunks per lane.
constexpr int kPackedMaxChunks = 12;
void launch_rmsnorm_rows(const NormParams& p, int in_bf16, int out_bf16, hipStream_t s);
// Whether launch_rmsnorm_rows can write a row segment of d elements packed.
bool norm_packable(int d, int in_bf16);

// GEMM epilogues.  The product Y[m][n] = sum_k X[m][k] W[n][k] of output row m
// (an X row) and feature n (a W row) is finished by one of these.
enum EpiKind {
  EPI_FC = 0,      // out_f32[m][n] = y + embed[ids[m]][n]; rows with rejected[m] skipped
  EPI_QKV = 1,     // n < q_cols: q_out[m][n] = y; then k, v columns go to the
                   // caches at slots[m] (skipped when slots[m] < 0)
  EPI_RESID = 2,   // out_f32[m][n] = y + res[res_rows ? res_rows[m] : m][n]
  EPI_SWIGLU = 3,  // out_s[m][n] = silu(y_gate) * y_up (and, with out_s_lo, the
                   // storage-type remainder of that value: out_s + out_s_lo
                   // carries it to about 16 mantissa bits)
  EPI_ARGMAX = 4,  // running (max, lowest index) per row; optional logits
  EPI_LSE = 5      // running (max m, sum exp(y - m)) per row and the target's logit
};
inline bool epi_rowred(int kind) { return kind == EPI_ARGMAX || kind == EPI_LSE; }

struct Epi {
  int kind;
  float* out_f32;
  int64_t ld_out;
  void* out_s;
  const void* embed;
  const int32_t* ids;
  const uint8_t* rejected;
  const float* res;
  const int32_t* res_rows;
  int64_t ld_res;
  void* k_cache;
  void* v_cache;
  const int32_t* slots;
  int q_cols, kv_cols, kv_rows;
  int embed_rows;
  void* out_s_lo;        // swiglu: optional second output (the remainder), or nullptr
  float* logits;         // argmax: optional [M, N]
  u32x4* part_top2;      // argmax: [P, M] partial (largest, index, second, index) as
                         // (float bits, int, float bits, int), index 0x7fffffff when absent
  float* part_val;       // lse: [P, M] partial maxima m
  float* part_sum;       // lse: [P, M] partial sums of exp(y - m)
  const int32_t* targets;  // lse: [M] target feature per row (< 0: none)
  float* tgt_logit;      // lse: [M] y of the target feature (written by the one tile that holds it)
};

// RMSNorm applied to the activation rows on their way into a contraction
// (gain == nullptr: X is the operand as is).  Row m of the operand is
//   X[m][s*seg_len + c] * inv * gain[s*seg_len + c],
//   inv = 1 / sqrt(mean_c X[m][s*seg_len + c]^2 + eps)   (zero for skipped rows)
// for each of the segs segments (segs * seg_len = K).
struct NormIn {
  const float* gain;
  int segs, seg_len;
  float eps;
  const uint8_t* skip;  // flags indexed by row, or nullptr
  int x_f32;            // X holds float32 (else the storage type)
  int defer;            // scale by 1 / rms after the contraction (see GemmParams)
  float* inv_tmp;       // [M, segs] room for the deferred scales when a separate
                        // norm kernel runs first
  void* tmp;            // [M, K] storage type: normalised rows when the norm
                        // cannot be fused into the contraction's staging
};

constexpr int kMaxSplitK = 8;  // K-split shares of the large-M kernel at most

struct GemmParams {
  const void* X;
  int64_t ldx;
  const void* W;
  const void* W2;  // second weight matrix of EPI_SWIGLU (up), else nullptr
  int M, N, K;
  const void* xzero;  // M <= 16: >= K zeroed elements, 16-byte aligned (padding rows of X)
  Epi epi;
  NormIn nrm;
  int* clear;  // with a norm: ints zeroed by the launch (the padding-row buffer of later launches), or nullptr
  int nclear;
  float* split_ws;     // large M: room for K-split partial products, or nullptr (no split)
  int64_t split_cap;   // its size in bytes
  int x_packed;        // X in the operand layout of NormParams::packed (large-M argmax only)
  // Operand precision (bf16 storage; no effect for f32):
  //  * nrm.defer (with a norm of several segments, or one): the operand is
  //    x * gain and each segment's sum is scaled by its 1 / rms after the
  //    contraction (the weight-streaming kernels split K by segment, the
  //    large-M kernel splits K into whole segments); where a path cannot, the
  //    normalised operand is rounded as before.
  //  * x_lo (M <= 16, no norm): the operand is X + x_lo (two bf16 parts), two
  //    matrix-core steps per weight chunk.
  //  * x_split (M <= 16, float rows with a folded norm): the rounded operand
  //    and its remainder, two matrix-core steps per weight chunk.
  const void* x_lo;
  int x_split;
  // Deferred segment scales of a normalised operand written by a separate
  // norm kernel: xinv[m * xinv_segs + s] multiplies the sum over segment s.
  const float* xinv;
  int xinv_segs;
  // Large-M K split into explicit k-step ranges (set by launch_gemm_big):
  // share y covers k-steps [split_beg[y], split_end[y]) and lies in segment
  // split_seg[y] of a deferred-scale operand; nsplit_k = 0: equal shares.
  int nsplit_k;
  int split_beg[kMaxSplitK], split_end[kMaxSplitK], split_seg[kMaxSplitK];
};


// Packs a row-major [N, row_bytes] matrix into the matrix-core-ready layout
// streamed by the GEMM kernels (see gemm.hip).
void launch_pack(const void* src, void* dst, int N, int row_bytes, hipStream_t s);
// Chooses the weight-streaming kernel (M <= 16) or the LDS-tiled kernel.
// W (and W2) are packed weights.  A requested RMSNorm (p.nrm.gain) is fused
// into the activation staging of the streaming kernels when the rows fit in
// LDS; otherwise rmsnorm_rows_kernel writes p.nrm.tmp first.
// EPI_ARGMAX (EPI_LSE) returns the number of partial rows P to reduce with
// launch_argmax_rescore (launch_lse_reduce); every other kind returns 0.
int launch_gemm(const GemmParams& p, int bf16, hipStream_t s);
// Upper bound of P for an argmax GEMM of this shape.
int gemm_argmax_partials(int M, int N);
// Large-M bf16 contraction through LDS-staged 256-row tiles (gemm_big.hip):
// EPI_ARGMAX returns the partial count P (one per feature tile, at most
// gemm_argmax_partials(M, N)); other
// epilogues return 0 when launched with a K split (p.split_ws), -1 when the
// shape does not call for one (nothing launched).
int launch_gemm_big(const GemmParams& p, hipStream_t s);
// K-split count launch_gemm_big uses for a non-argmax contraction; 0 = it
// launches nothing for this shape.
// segs > 1: for an operand whose segs segments of K are scaled after the
// contraction (p.xinv), which needs segments of whole 32-wide k-steps.
int gemm_big_splits(const GemmParams& p, int segs = 1);
// Bytes of K-split workspace worth giving a large-M stage (T rows, widest
// contraction output nmax).
int64_t gemm_split_bytes(int T, int nmax);

// Greedy token of each row: the P partial top-2 lists merged into the row's
// two largest logits (lowest index first among equal values), whose logits
// are then computed again in fp32 from the unrounded normalised row,
//   z = (sum_k W[c][k] x[m][k] g[k]) / sqrt(mean_k x[m][k]^2 + eps),
// and the larger (lower index on a tie) is the token.  x: [M, K] float32
// rows (stride ldx), W: packed [N, K] weights of storage type (bf16 when
// w_bf16).  rescore 0: the partials hold exact logits (lm_head_exact), and
// the largest is the token as it is.
void launch_argmax_rescore(const u32x4* part, int P, int M, const float* x, int64_t ldx, const float* gain,
                           float eps, const void* W, int K, int w_bf16, int32_t* tokens, int rescore, hipStream_t s);
// Whether the LM head over M float rows with a folded norm (gain, one
// segment of K) runs on the bf16 hi + lo operand (logits exact to about
// 2^-17 relative; see gemm.hip).
bool lm_head_exact(int M, int K, int bf16, const float* gain);
// lse[m] = log sum_v exp(y[m][v]) from the P partials of EPI_LSE, and
// loss[m] = lse[m] - tgt[m] (0 where targets[m] is outside [0, N)); lse or
// loss may be null.
void launch_lse_reduce(const float* pv, const float* ps, int P, int M, int N, const int32_t* targets,
                       const float* tgt, float* lse, float* loss, hipStream_t s);
// kl[m] = sum_j p[m][j] (log p[m][j] - z[m][id[m][j]] + lse[m]) over the k
// pairs of row m with an id in [0, N) and p > 0; z from the unrounded
// normalised row in fp32 (as in launch_argmax_rescore).  ids, probs: [M, k].
// Dynamic LDS: kl_topk_lds_bytes(K, w_bf16) (the row's x * g, padded).
int kl_topk_lds_bytes(int K, int w_bf16);
// Wrows: the same weight row-major [N, K] (storage type), or nullptr (the
// rows are gathered from the packed W).
void launch_kl_topk(const float* x, int64_t ldx, const float* gain, float eps, const void* W, const void* Wrows, int K,
                    int N, int w_bf16, int k, const int32_t* ids, const float* probs, const float* lse, float* kl,
                    int M, hipStream_t s);

struct AttnParams {
  const void* q;
  int64_t q_stride;
  const int32_t* q_rows;
  int meta_by_row;  // per-query metadata indexed by q_rows[i] instead of i
  const void *k, *v;
  int num_q, num_seg, q_per_seg, num_kv_rows, Hq, Hkv;
  float scale, scale_log2;
  const int32_t *seg_kv_base, *q_start, *q_depth, *q_self_row, *kv_parent;
  int max_depth;  // chain rows walked per query at most (<= attn_max_depth(G))
  int n_splits, split_len;
  void* out;
  float* lse;
  int64_t* dbg_count;
  uint64_t* dbg_hash;
  float* part_o;       // [n_splits, num_q*Hq, Dh]
  float* part_ml;      // [n_splits, num_q*Hq, 2]
  uint64_t* part_dbg;  // [n_splits, num_q*Hkv, 2]
  int win_sink, win_len;  // StreamingLLM window over the prefix keys (win_len 0: none; never split)
  // Work plan (null plan_items: every query tile is cut into n_splits pieces
  // of split_len keys, in the fixed grid order).  With a plan, attn_plan_kernel
  // cuts each tile's prefix into plan_pieces[tile] <= plan_nmax equal pieces
  // (one when plan_nmax is 1, else as many as pieces of at most plan_tiles key
  // tiles need) and lists the (tile, piece) items by decreasing work; workgroup
  // b takes item b / Hkv.  Partials use slot = piece.
  int2* plan_items;   // [tiles * plan_nmax]
  int* plan_count;    // number of items
  int* plan_pieces;   // [tiles]
  int plan_nmax, plan_tiles;
};
void launch_attention(const AttnParams& p, int bf16, int head_dim, hipStream_t s);
// Query tiles of one planned launch at most.
constexpr int kPlanMaxTiles = 2048;

// Backward of the COD attention over the depth-major training layout (bf16
// operands, f32 gradients): dq of the queries [q_begin, q_end), their dk and
// dv contributions added to every row (attention_bwd.hip).
struct AttnBwdParams {
  const void *q, *k, *v, *out, *dout;     // bf16: q, out, dout [T, Hq, Dh]; k, v [T, Hkv, Dh]
  const float* lse;                       // [T, Hq] natural-log sum-exp of the forward
  const int32_t *start, *depth, *group_off;  // [T], [T], [D + 1]
  int T, N, D, Hq, Hkv, q_begin, q_end;
  float scale;
  float* dq;                              // [q_end - q_begin, Hq, Dh]
  float *dk, *dv;                         // [T, Hkv, Dh], accumulated
  float* delta;                           // workspace [q_end - q_begin, Hq]
  float *part_k, *part_v;                 // workspace: attn_bwd_part_floats each (shares of dK, dV)
};
void launch_attention_backward(const AttnBwdParams& p, int head_dim, hipStream_t s);
int64_t attn_bwd_part_floats(int T, int D, int Hkv, int head_dim);
// Queries one attention workgroup takes: 128 (query, head) columns of one kv
// head, i.e. 128 / (n_q_heads / n_kv_heads) queries.
int attn_queries_per_workgroup(int G, int head_dim);
// Deepest chain one query may walk: 16, or fewer when a workgroup's queries
// could gather more chain rows than its LDS list holds (8 at G = 1).
int attn_max_depth(int G);

}  // namespace pe
