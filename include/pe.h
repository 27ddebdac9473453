/*
 * pe.h - C ABI of the P-EAGLE parallel-drafting hot path for AMD MI355X (gfx950).
 *
 * One drafter forward predicts all K draft tokens of every request in a single
 * pass ("P-EAGLE: parallel speculative decoding in vLLM", section "Step 2:
 * parallel drafting").  The five entry points below are its stages:
 *
 *   pe_build_draft_batch  draft-batch construction (ids, positions, KV slots,
 *                         masks, hidden-state mapping, h_shared broadcast)
 *   pe_fuse_hidden        RMSNorm of the three captured target streams, fc
 *                         fusion, token embedding
 *   pe_draft_layer        one pre-norm decoder layer with parallel-draft
 *                         masked GQA attention over per-request KV regions
 *   pe_draft_attention    the masked attention alone (decode regions and the
 *                         training-shaped COD layout)
 *   pe_lm_head_argmax     final RMSNorm, LM head and greedy argmax
 *
 * Interface choices
 * -----------------
 * Beyond one call per stage with plain tensors: every linear weight is
 * passed pre-packed (pe_pack_weight, once per weight), because the packed
 * 1 KB chunks make each weight load one contiguous matrix-core operand;
 * pe_lm_head_argmax takes the weights struct (final_gain, w_lm) so that all
 * stages share one weights handle; h_shared is an argument of
 * pe_build_draft_batch, the only stage that reads it, not a weights member;
 * pe_attn_args carries host bounds (max_prefix, max_depth) that the work
 * split and the chain-depth check need before launch.  The two LM-head
 * losses, the attention backward and the allocation-free LM head are
 * additional entry points.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer; structs passed by
 * pointer (dims, weights, batch, attention arguments) live in HOST memory and
 * are read before the call returns.  Tensors are dense and row-major, except
 * linear weights ([out, in], bias-free), which are passed in the packed
 * layout described at pe_pack_weight.  The caller allocates and owns every
 * buffer, including workspace; the library never allocates or frees device
 * memory and keeps no state between calls.
 *
 * Types.  pe_dtype names the storage type of weights, captured hidden
 * streams, h_shared and the KV cache: PE_F32 (float) or PE_BF16 (bfloat16
 * bits).  Gains are always float32.  The residual stream (x0, layer output)
 * is always float32.  Arithmetic accumulates in float32; bf16 storage feeds
 * bf16 matrix-core operands, f32 storage feeds f32 matrix-core operands.
 * Token ids, positions, rows and slots are int32; -1 is the only sentinel.
 *
 * Streams.  Every call is asynchronous on the given hipStream_t (NULL = the
 * default stream) and never synchronises the host.  Buffers must stay alive
 * until the stream work completes.  Calls are ordered by stream order.  Two
 * calls that share a workspace must not run concurrently.
 *
 * Errors.  Host-visible arguments (sizes, pointer nullness and alignment,
 * workspace size) are validated before anything is launched; a violation
 * returns PE_ERR_INVALID_ARG (or PE_ERR_UNSUPPORTED for a valid but
 * unimplemented shape or dtype) and launches nothing.  A launch failure
 * returns PE_ERR_DEVICE.  Device-resident index arrays cannot be checked by
 * the host: kernels bounds-check every index they dereference and skip an
 * out-of-range access, so inputs that break a documented precondition give
 * unspecified values but never an out-of-bounds access.  No exception
 * crosses this interface.  All 16-byte alignment requirements below refer to
 * the start address of each tensor.
 */
#ifndef PE_H_
#define PE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

/* Rejected draft-batch rows map to this KV slot and write nothing
 * ("P-EAGLE: parallel speculative decoding in vLLM", section "KV cache and
 * CUDA graphs"). */
#define PE_PADDING_SLOT_ID (-1)

typedef enum {
    PE_OK = 0,
    PE_ERR_INVALID_ARG = 1,
    PE_ERR_UNSUPPORTED = 2,
    PE_ERR_DEVICE = 3
} pe_status;

typedef enum { PE_F32 = 0, PE_BF16 = 1 } pe_dtype;

/* Human-readable name of a status code (static storage). */
const char* pe_status_string(pe_status s);

/* Library version string (static storage). */
const char* pe_version(void);

/* Drafter shape.  hidden must be a multiple of 32 (PE_BF16) or 16 (PE_F32);
 * head_dim is 64 or 128; n_q_heads a multiple of n_kv_heads; ffn a multiple
 * of 32 (PE_BF16) or 16 (PE_F32).  mask_token_id is the id of the MASK
 * token (0 <= mask_token_id < vocab).  eps is the RMSNorm epsilon:
 * RMSNorm(x) = x * g / sqrt(mean(x^2) + eps). */
typedef struct {
    int32_t hidden;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t ffn;
    int32_t vocab;
    int32_t mask_token_id;
    float eps;
    pe_dtype dtype;
} pe_drafter_dims;

/* Packed weight layout.  Every linear weight passed in pe_drafter_weights
 * (w_fc, w_qkv, w_o, w_gate, w_up, w_down, w_lm) is in the library's packed,
 * matrix-core-ready layout, produced once from a row-major [N, K] matrix by
 * pe_pack_weight.  Rows are padded to a multiple of 16; for row block b
 * (rows 16b..16b+15) and 64-byte step s of a row (S = K*elem/64 steps), the
 * 1 KB at byte offset (b*S + s)*1024 holds 64 slices of 16 bytes: slice l
 * is bytes [16*(l/16), 16*(l/16)+16) of step s of row 16b + l%16.  Each
 * 1 KB is then one contiguous load that is directly the operand of one
 * matrix-core step.  Requires K*elem to be a multiple of 64 bytes. */

/* Size in bytes of the packed form of an [N, K] weight (N rounded up to 16). */
pe_status pe_packed_weight_bytes(pe_dtype dtype, int32_t N, int32_t K, size_t* bytes);

/* Packs the row-major [N, K] weight `src` (device) into `dst` (device, at
 * least pe_packed_weight_bytes; both 16-byte aligned).  Asynchronous on
 * `stream`; padding rows are written as zeros. */
pe_status pe_pack_weight(pe_dtype dtype, int32_t N, int32_t K, const void* src, void* dst, hipStream_t stream);

/* Drafter parameters (device pointers; storage dtype unless noted; linear
 * weights in the packed layout above, their shapes given as [out, in]).
 * "Attention Drift" (arXiv 2605.09992), section 2: the EAGLE-3 drafter feeds
 * the fused target hidden states through fc into one pre-norm decoder layer;
 * section 4.1, Observation 2: each captured target stream is RMS-normalised
 * before fc. */
typedef struct {
    const void*  embed;        /* [vocab, hidden] token embedding, row-major */
    const float* stream_gain;  /* [3, hidden] f32, RMSNorm gains of the three
                                  captured streams (low, mid, high)          */
    const void*  w_fc;         /* [hidden, 3*hidden] fc over the normalised
                                  streams concatenated low|mid|high (packed) */
    const float* attn_gain;    /* [hidden] f32, pre-attention RMSNorm gain   */
    const void*  w_qkv;        /* [(Hq + 2*Hkv)*Dh, hidden] packed: q rows,
                                  then k rows, then v rows, head-major       */
    const void*  w_o;          /* [hidden, Hq*Dh] packed                     */
    const float* mlp_gain;     /* [hidden] f32, pre-MLP RMSNorm gain         */
    const void*  w_gate;       /* [ffn, hidden] packed                       */
    const void*  w_up;         /* [ffn, hidden] packed                       */
    const void*  w_down;       /* [hidden, ffn] packed                       */
    const float* final_gain;   /* [hidden] f32, RMSNorm gain before LM head  */
    const void*  w_lm;         /* [vocab, hidden] LM head, packed            */
} pe_drafter_weights;

/* Outputs of pe_build_draft_batch, T = total_window_rows + R*K rows
 * (caller-allocated device buffers). */
typedef struct {
    int32_t* draft_ids;     /* [T] token id of each row                         */
    int32_t* draft_pos;     /* [T] position of each row inside its KV region    */
    int32_t* slot_mapping;  /* [T] KV row = kv_base[r] + pos, or PE_PADDING_SLOT_ID
                               for rejected rows                                */
    int32_t* hidden_src;    /* [T] target_hidden row copied, or -1 = h_shared   */
    int32_t* req_of_row;    /* [T] request index of each row                    */
    uint8_t* rejected;      /* [T] 1 on rejected window rows                    */
    uint8_t* masked;        /* [T] 1 on MASK rows (draft slots 2..K)            */
    int32_t* query_rows;    /* [R*K] rows of the next-token and MASK slots      */
    int32_t* cu_draft;      /* [R+1] first row of each request                  */
    void*    draft_hidden;  /* [T, 3, hidden] storage dtype, 16-byte aligned    */
} pe_batch_out;

/*
 * pe_build_draft_batch - stage 1, draft-batch construction.
 *
 * Follows "P-EAGLE: parallel speculative decoding in vLLM", sections "Step 2:
 * parallel drafting" (next-token slot = new token + h_context; slots 2..K =
 * MASK token + shared hidden placeholder), "fused Triton kernel" (one pass
 * copies previous ids and positions, inserts the new token, MASK-fills the
 * parallel slots and emits the rejected mask, masked mask and hidden mapping),
 * "hidden-state management" (h_shared broadcast into the MASK slots, target
 * hidden rows mapped to their new positions) and "KV cache" (rejected tokens
 * map to PE_PADDING_SLOT_ID).
 *
 * Request r (0 <= r < R) contributes W_r = cu_window[r+1] - cu_window[r]
 * window rows (the previous verify pass; the trailing n_rej[r] are rejected),
 * then one next-token row, then K-1 MASK rows, starting at row
 * cu_draft[r] = cu_window[r] + r*K.  Window row j copies window_ids/pos/hrow
 * [cu_window[r]+j].  The next-token row holds new_token[r] at position
 * kv_len[r] + W_r - n_rej[r] with hidden row ctx_hrow[r]; MASK row k holds
 * dims->mask_token_id at that position + k with h_shared.  Every
 * non-rejected row gets slot kv_base[r] + position.  draft_hidden rows are
 * bit copies of target_hidden rows or of h_shared.
 *
 * Inputs (device): cu_window [R+1] (cu_window[0] = 0, non-decreasing,
 * cu_window[R] = total_window_rows), n_rej/kv_len/kv_base/new_token/ctx_hrow
 * [R], window_ids/window_pos/window_hrow [total_window_rows],
 * target_hidden [target_rows, 3, hidden], h_shared [3, hidden] (storage
 * dtype, 16-byte aligned).  Preconditions: 0 <= n_rej[r] <= W_r; hidden rows
 * in [0, target_rows).  Requires R >= 1, K >= 1, total_window_rows >= 0,
 * target_rows >= 1.
 */
pe_status pe_build_draft_batch(const pe_drafter_dims* dims, int32_t R, int32_t K,
                               int32_t total_window_rows, int32_t target_rows,
                               const int32_t* cu_window, const int32_t* n_rej,
                               const int32_t* kv_len, const int32_t* kv_base,
                               const int32_t* window_ids, const int32_t* window_pos,
                               const int32_t* window_hrow, const int32_t* new_token,
                               const int32_t* ctx_hrow, const void* target_hidden,
                               const void* h_shared, const pe_batch_out* out,
                               hipStream_t stream);

/*
 * pe_fuse_hidden - stage 2, stream RMSNorm + fc fusion.
 *
 * "Attention Drift" (arXiv 2605.09992), section 4.1 / Observation 2 (RMSNorm
 * on each captured target stream before fc) and section 2 (fc fusion into the
 * drafter); "P-EAGLE: parallel speculative decoding in vLLM", section "Step
 * 2: parallel drafting" (each position combines a token embedding with a
 * hidden state).  For every row t with rejected[t] == 0 (every row when
 * rejected is NULL):
 *   u_s = RMSNorm(draft_hidden[t, s, :], stream_gain[s])   s = 0, 1, 2
 *   x0[t] = embed[ids[t]] + w_fc [u_0; u_1; u_2]
 * Rejected rows of x0 are left untouched.  x0 is [T, hidden] float32.
 * Uses weights->embed, stream_gain and w_fc only.  Workspace: see
 * pe_fuse_hidden_workspace (at least 16 bytes, 256-byte aligned).
 */
pe_status pe_fuse_hidden(const pe_drafter_dims* dims, const pe_drafter_weights* w,
                         int32_t T, const void* draft_hidden, const uint8_t* rejected,
                         const int32_t* ids, float* x0, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
pe_status pe_fuse_hidden_workspace(const pe_drafter_dims* dims, int32_t T, size_t* bytes);

/* Arguments of pe_draft_attention.
 *
 * Queries are grouped in num_seg segments of q_per_seg consecutive queries
 * (num_q = num_seg * q_per_seg).  Query i of segment s sees:
 *   - the prefix rows seg_kv_base[s] + j for 0 <= j <= q_start[i], and
 *   - its chain rows: q_self_row[i], kv_parent[q_self_row[i]], ... - q_depth[i]
 *     rows in all, following kv_parent (the walk stops early at -1).
 * Prefix and chain rows of one query must be disjoint.  In a decode step a
 * segment is a request's KV region, q_start is the query's position and
 * q_depth is 0 (the earlier draft slots lie inside the prefix).  In the
 * training-shaped COD layout ("[RFC]: Add random anchor for p-eagle first
 * position", Motivation: a query at chain start i and depth d sees original
 * positions <= i plus its own chain) there is one segment, group 0 holds the
 * original positions (seg_kv_base = 0, q_start = i), and deeper rows link to
 * their depth-1 parent (kv_parent = -1 at depth 1).
 *
 * out[i, h] = softmax_j(q[i,h] . k[j, h/G] * scale) v[j, h/G], G = Hq/Hkv,
 * over the rows j seen by query i.  A query that sees no row gets zeros.
 */
typedef struct {
    int32_t num_q, num_seg, q_per_seg;
    int32_t num_kv_rows;
    int32_t n_q_heads, n_kv_heads, head_dim;   /* head_dim 64 or 128          */
    float scale;                               /* usually 1/sqrt(head_dim)    */
    pe_dtype dtype;                            /* of q, k, v and out          */
    const void* q;          /* query i, head h at q + (q_rows ? q_rows[i] : i)
                               * q_row_stride + h*head_dim (elements)           */
    int64_t q_row_stride;   /* elements between query rows (>= Hq*Dh)          */
    const int32_t* q_rows;  /* [num_q] or NULL                                 */
    const void* k;          /* [num_kv_rows, Hkv, Dh]                          */
    const void* v;          /* [num_kv_rows, Hkv, Dh]                          */
    const int32_t* seg_kv_base;  /* [num_seg]                                  */
    const int32_t* q_start;      /* [num_q] last prefix offset (-1 = none)     */
    const int32_t* q_depth;      /* [num_q] or NULL (all 0); each value at
                                    most max_depth                             */
    const int32_t* q_self_row;   /* [num_q] or NULL when q_depth is NULL       */
    const int32_t* kv_parent;    /* [num_kv_rows] or NULL when q_depth is NULL */
    int32_t max_prefix;     /* host bound on 1 + max q_start (work split only;
                               a smaller true bound only costs balance)        */
    int32_t split_len;      /* keys per split (multiple of 64) or 0 = auto:
                               launches below 512 workgroups cut every
                               query tile's prefix into pieces; from 512 to
                               2,047 a work plan built on the device runs the
                               tiles longest first and, below 1,024, cuts
                               the longer ones into up to three equal pieces
                               (workspace needed in both cases)              */
    void* out;              /* [num_q, Hq, Dh]                                 */
    float* lse;             /* [num_q, Hq] natural-log sum-exp of scaled
                               scores, or NULL                                 */
    int64_t* dbg_count;     /* [num_q, Hkv] keys seen, or NULL                 */
    uint64_t* dbg_hash;     /* [num_q, Hkv] sum mod 2^64 of SplitMix64(row)
                               over the rows seen, or NULL                     */
    int32_t window_sink;    /* StreamingLLM variant ([RFC] "Separate Ablation:
                               StreamingLLM", sink=256, window=2048): with
                               window_len > 0, prefix row j (0 <= j <= q_start)
                               is seen only when j < window_sink or
                               q_start - j < window_len; chain rows are
                               unchanged.  0 and 0 (the default of a zeroed
                               struct): the full prefix.  Both >= 0; a window
                               is never split (split_len must be 0, else
                               PE_ERR_UNSUPPORTED).                          */
    int32_t window_len;
    int32_t max_depth;      /* host bound on every q_depth[i] (ignored when
                               q_depth is NULL): the kernel walks at most
                               max_depth chain rows per query.  Required in
                               1..16 with q_depth (1..8 when n_q_heads ==
                               n_kv_heads: a workgroup of 128 single-head
                               queries gathers at most 1,024 chain rows);
                               0 or negative with q_depth is
                               PE_ERR_INVALID_ARG, above the kernel's bound
                               PE_ERR_UNSUPPORTED.  A q_depth[i] above the
                               stated bound breaks this contract: its walk
                               stops at max_depth rows.                      */
} pe_attn_args;

/*
 * pe_draft_attention - the parallel-draft / COD masked GQA attention.
 *
 * "P-EAGLE: parallel speculative decoding in vLLM", section "Training on long
 * sequences": N*K positions make a dense mask of more than 4e9 elements at
 * N=8192, K=8; the sequence partition splits them into contiguous chunks that
 * keep every dependency across chunk boundaries.  Here the mask is evaluated
 * from indices inside the kernel and never stored; a chunk of queries is a
 * call on a subset of queries (slice q, q_start, q_depth, q_self_row, q_rows)
 * with the full key arrays.  A query's outputs are bitwise the same in a
 * chunk that starts at a multiple of 256 queries (of its segment) as in one
 * call over all queries, for the same nonzero split_len (split_len 0 picks
 * the split from the launch size, which may change the summation order).
 * dbg_count/dbg_hash are accumulated by the same loop that skips and masks
 * keys.  Alignment: q, k, v, out 16 bytes.
 * Workspace: pe_draft_attention_workspace (256-byte aligned).
 */
pe_status pe_draft_attention(const pe_attn_args* args, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
pe_status pe_draft_attention_workspace(const pe_attn_args* args, size_t* bytes);

/* Arguments of pe_draft_attention_backward: the depth-major COD training
 * layout of pe_draft_attention with every row a query (one segment,
 * seg_kv_base 0): rows 0..n_pos-1 are the original positions (start = row,
 * depth 0); group e (rows group_off[e]..group_off[e+1]-1, 1 <= e < n_groups)
 * holds the depth-e chain rows sorted by start.  Row (s, d) sees the rows
 * (j, 0) with j <= s and (s, e) with 1 <= e <= d.                           */
typedef struct {
    int32_t num_rows;       /* T                                             */
    int32_t n_pos;          /* N = group_off[1]                              */
    int32_t n_groups;       /* 1..16                                         */
    int32_t n_q_heads, n_kv_heads, head_dim;   /* head_dim 64 or 128          */
    float scale;
    pe_dtype dtype;         /* PE_BF16                                       */
    const int32_t* group_off;  /* [n_groups + 1] device                      */
    const int32_t* start;      /* [T] device                                 */
    const int32_t* depth;      /* [T] device                                 */
    const void* q;          /* [T, Hq, Dh]                                   */
    const void* k;          /* [T, Hkv, Dh]                                  */
    const void* v;          /* [T, Hkv, Dh]                                  */
    const void* out;        /* [T, Hq, Dh] forward output                    */
    const void* dout;       /* [T, Hq, Dh] gradient of the output            */
    const float* lse;       /* [T, Hq] forward natural-log sum-exp           */
    int32_t q_begin, q_end; /* the query chunk [q_begin, q_end)              */
    float* dq;              /* [q_end - q_begin, Hq, Dh] f32, written        */
    float* dk;              /* [T, Hkv, Dh] f32, the chunk's part added      */
    float* dv;              /* [T, Hkv, Dh] f32, the chunk's part added      */
} pe_attn_bwd_args;

/*
 * pe_draft_attention_backward - gradients of the COD attention for a chunk of
 * queries.
 *
 * "P-EAGLE: parallel speculative decoding in vLLM", section "Training on long
 * sequences": the sequence partition trains chunk by chunk while keeping
 * every attention dependency across chunk boundaries, so a chunk's queries
 * contribute to the key and value gradients of earlier rows.  With
 * P = exp(scale q.k - lse) over each query's visible rows:
 *   dQ = scale dS K,  dK += scale dS^T Q,  dV += P^T dO,
 *   dS = P (dO.v - rowsum(dO o O)).
 * dq is written for the chunk's rows; dk and dv are accumulated (zero them
 * before the first chunk of a pass); summed over chunks they equal one call
 * over all rows up to rounding.  Each workgroup owns its outputs: results
 * do not depend on timing.  Alignment: every tensor 16 bytes.
 * Workspace: pe_draft_attention_backward_workspace (256-byte aligned).
 */
pe_status pe_draft_attention_backward(const pe_attn_bwd_args* args, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
pe_status pe_draft_attention_backward_workspace(const pe_attn_bwd_args* args, size_t* bytes);

/*
 * pe_draft_layer - stage 3, one pre-norm decoder layer of the drafter.
 *
 * "Attention Drift" (arXiv 2605.09992), section 2 (a single pre-norm decoder
 * layer after fc); "P-EAGLE: parallel speculative decoding in vLLM", sections
 * "Step 2: parallel drafting" and "KV cache" (rejected rows write nothing).
 * For the T rows of a built batch (row metadata from `batch`):
 *   a = RMSNorm(x0, attn_gain); [q|k|v] = w_qkv a
 *   every row with slot_mapping != -1 writes k, v to k_cache/v_cache at that slot
 *   then, for the R*K query rows (batch->query_rows), in that order:
 *   o = attention of q over its region rows kv_base[r] + 0..pos (GQA)
 *   x1 = x0 + w_o o;  b = RMSNorm(x1, mlp_gain)
 *   x_out = x1 + w_down(silu(w_gate b) * (w_up b))
 * Only the query rows' outputs are produced (one layer: the other rows are
 * needed only as keys and values).  x0 [T, hidden] f32; k_cache/v_cache
 * [kv_rows, Hkv, Dh] storage dtype (16-byte aligned); kv_base [R] device;
 * max_pos = host bound on 1 + the largest query position (split balance
 * only).  x_out [R*K, hidden] f32.  Workspace: pe_draft_layer_workspace.
 */
pe_status pe_draft_layer(const pe_drafter_dims* dims, const pe_drafter_weights* w,
                         int32_t T, int32_t R, int32_t K, const float* x0,
                         const pe_batch_out* batch, const int32_t* kv_base,
                         void* k_cache, void* v_cache, int32_t kv_rows, int32_t max_pos,
                         float* x_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);
pe_status pe_draft_layer_workspace(const pe_drafter_dims* dims, int32_t T, int32_t R,
                                   int32_t K, int32_t max_pos, size_t* bytes);

/*
 * pe_lm_head_argmax - stage 4, final RMSNorm + LM head + greedy argmax.
 *
 * "P-EAGLE: parallel speculative decoding in vLLM", section "Step 2: parallel
 * drafting": the LM head predicts the draft tokens t_1..t_K of every request
 * in the same pass.  For each of the n rows of x [n, hidden] f32:
 *   z = w_lm RMSNorm(x, final_gain);  tokens[i] = lowest index of max(z)
 * bf16, n <= 8 (the decode step of one request): the contraction runs on
 * the normalised row as two bf16 parts, the rounded row and its remainder,
 * so every logit is within about 2^-17 of the unrounded row's, and the
 * largest (lower index on a tie) is the token.  Otherwise the contraction
 * runs on the normalised row rounded to the storage type, the row's two
 * leading logits are computed again in fp32 from the unrounded row, and
 * the larger of those two (lower index on a tie) is the token.
 * logits [n, vocab] f32 (the contraction's values) is written when
 * non-NULL (validation runs); the fast path never materialises logits.
 * Uses weights->final_gain (16-byte aligned) and w_lm.
 * Workspace: pe_lm_head_argmax_workspace.
 */
pe_status pe_lm_head_argmax(const pe_drafter_dims* dims, const pe_drafter_weights* w,
                            int32_t n, const float* x, int32_t* tokens, float* logits,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
pe_status pe_lm_head_argmax_workspace(const pe_drafter_dims* dims, int32_t n, size_t* bytes);

/*
 * pe_lm_head_argmax_noalloc - pe_lm_head_argmax for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and results, with
 * the workspace taken from a fixed array of PE_NOALLOC_SCRATCH_BYTES in the
 * library's device code (one per GPU, held until the process ends; its
 * address is looked up once per device on the first call there).  Returns
 * PE_ERR_UNSUPPORTED when pe_lm_head_argmax_workspace(dims, n) exceeds that
 * size (with a 201,088 x 2,880 bf16 head: more than 597 rows), checked
 * before anything touches the device; PE_ERR_DEVICE when the array's address
 * cannot be resolved.  Calls
 * no allocator.  Every call on one GPU uses the same array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller; calls in one stream are ordered.
 */
#define PE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pe_status pe_lm_head_argmax_noalloc(const pe_drafter_dims* dims, const pe_drafter_weights* w,
                                    int32_t n, const float* x, int32_t* tokens, float* logits,
                                    hipStream_t stream);

/*
 * pe_lm_head_loss - the LM head's log-sum-exp and cross-entropy without the
 * logits.
 *
 * "[RFC]: Add random anchor for p-eagle first position", section "Separate
 * Ablation: StreamingLLM & The 32K Wall": at long sequences the logits tensor
 * ([T, V], 9.4 GiB per sample at 32K x 151K in bf16), not attention, runs out
 * of memory.  Here the logits are reduced tile by tile as they are produced.
 * For each of the n rows of x [n, hidden] f32:
 *   z = w_lm RMSNorm(x, final_gain);  lse[i] = log sum_v exp(z_v);
 *   loss[i] = lse[i] - z[targets[i]]  (0 where targets[i] is outside [0, vocab))
 * targets [n] int32 device (required with loss), lse and loss [n] f32
 * device, either may be NULL but not both.  Results do not depend on timing:
 * partial sums are merged in a fixed order.  Uses weights->final_gain and
 * w_lm.  Workspace: pe_lm_head_loss_workspace (256-byte aligned).
 */
pe_status pe_lm_head_loss(const pe_drafter_dims* dims, const pe_drafter_weights* weights,
                          int32_t n, const float* x, const int32_t* targets, float* lse,
                          float* loss, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);
pe_status pe_lm_head_loss_workspace(const pe_drafter_dims* dims, int32_t n, size_t* bytes);

/*
 * pe_lm_head_kl - the LM head's KL loss against a top-k target distribution,
 * without the logits.
 *
 * "[RFC]: Add random anchor for p-eagle first position", section "Experiment
 * Setup": the drafter is trained with a KL loss against the verifier's
 * distribution.  Here the target of row i arrives as k (token id,
 * probability) pairs, row-major in target_ids [n, k] int32 and target_probs
 * [n, k] f32 (device; the verifier's top-k, zero mass elsewhere).  With
 * z = w_lm RMSNorm(x[i], final_gain) and lse[i] = log sum_v exp(z_v):
 *   kl[i] = sum_j p_ij (log p_ij - z[id_ij] + lse[i])   ( = KL(p_i || softmax(z)) )
 * A pair whose id lies outside [0, vocab) or whose probability is not
 * positive (NaN included) adds nothing; the probabilities are used as given
 * (no renormalisation).  lse is streamed tile by tile as in pe_lm_head_loss;
 * the k target logits are computed in fp32 from the unrounded normalised
 * row, reading the k target rows of the LM head.  w_lm_rows (optional,
 * device, 16-byte aligned): the same LM head in its row-major [vocab,
 * hidden] storage-type layout (the matrix pe_pack_weight packed); when given
 * the target rows are read from it as whole rows, which costs about a
 * quarter of the memory requests of gathering them from the packed weight;
 * NULL gathers them from weights->w_lm.  x [n, hidden] f32 and final_gain 16-byte aligned; k >= 1 and
 * n * k < 2^31; kl [n] f32 required, lse [n] f32 may be NULL; otherwise
 * PE_ERR_INVALID_ARG.
 * Results do not depend on timing (fixed-order sums).  Workspace:
 * pe_lm_head_kl_workspace (256-byte aligned).
 */
pe_status pe_lm_head_kl(const pe_drafter_dims* dims, const pe_drafter_weights* weights,
                        int32_t n, const float* x, int32_t k, const int32_t* target_ids,
                        const float* target_probs, const void* w_lm_rows, float* lse, float* kl,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);
pe_status pe_lm_head_kl_workspace(const pe_drafter_dims* dims, int32_t n, size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* PE_H_ */
