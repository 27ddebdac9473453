// C ABI of libpe: host-side argument validation, workspace layout and the
// launch sequence of each stage.  Nothing here computes on the host; every
// step of the drafter runs in the kernels of batch.hip, norm.hip, gemm.hip
// and attention.hip on the caller's stream.
#include <math.h>
#include <string.h>
#include <mutex>
#include "pe.h"
#include "kernels.h"

using namespace pe;

// Workspace of pe_lm_head_argmax_noalloc: a fixed array in the library's
// device code.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` only names the symbol: its device
// address comes from hipGetSymbolAddress, once per device (scratch_ptr).
static __device__ __align__(256) char scratch[PE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr const char* kVersion = "pe 0.1.0 (gfx950)";

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }
int up64(int x) { return (x + 63) & ~63; }
size_t esize(pe_dtype t) { return t == PE_BF16 ? 2 : 4; }

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += up256(bytes);
    return p;
  }
};

pe_status check_dims(const pe_drafter_dims* d) {
  if (!d) return PE_ERR_INVALID_ARG;
  if (d->dtype != PE_F32 && d->dtype != PE_BF16) return PE_ERR_INVALID_ARG;
  if (d->hidden <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 || d->ffn <= 0 ||
      d->vocab <= 0)
    return PE_ERR_INVALID_ARG;
  if (d->n_q_heads % d->n_kv_heads) return PE_ERR_INVALID_ARG;
  if (d->mask_token_id < 0 || d->mask_token_id >= d->vocab) return PE_ERR_INVALID_ARG;
  if (!(d->eps >= 0.f) || !isfinite(d->eps)) return PE_ERR_INVALID_ARG;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G > 64 || 64 % G) return PE_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PE_ERR_UNSUPPORTED;
  const int step = d->dtype == PE_BF16 ? 32 : 16;
  if (d->hidden % step || d->ffn % step) return PE_ERR_UNSUPPORTED;
  // one RMSNorm row segment is at most kNormMaxChunks * 256 sixteen-byte chunks
  if ((int64_t)d->hidden * (int64_t)esize(d->dtype) > (int64_t)kNormMaxChunks * 256 * 16 ||
      (int64_t)d->hidden * 4 > (int64_t)kNormMaxChunks * 256 * 16)
    return PE_ERR_UNSUPPORTED;
  if ((int64_t)d->vocab * d->hidden >= (int64_t)1 << 40) return PE_ERR_UNSUPPORTED;
  return PE_OK;
}

pe_status launched() { return hipGetLastError() == hipSuccess ? PE_OK : PE_ERR_DEVICE; }

// Split of the prefix range so that a decode-shaped launch still fills the chip
// (two attention workgroups share a CU: 512 run at once).  A launch of 512
// or more workgroups is not split: it already occupies every slot, and the
// unnormalised partials would only add HBM traffic and a combine pass (the
// 64-request decode step's attention: 139 -> 107 us unsplit).
#ifndef PE_ATTN_NOSPLIT_GROUPS
#define PE_ATTN_NOSPLIT_GROUPS 512
#endif
// Below that, the prefix is split so that about PE_ATTN_SPLIT_TARGET
// workgroups run (at most 64 shares of at least one 64-key tile).
#ifndef PE_ATTN_SPLIT_TARGET
#define PE_ATTN_SPLIT_TARGET 2048
#endif
void choose_split(int base_groups, int max_prefix, int split_req, int* n_splits, int* split_len) {
  const int mp = max_prefix > 1 ? max_prefix : 1;
  int sl;
  if (split_req > 0) {
    sl = up64(split_req);
  } else {
    int want = base_groups >= PE_ATTN_NOSPLIT_GROUPS ? 1 : (PE_ATTN_SPLIT_TARGET + base_groups - 1) / base_groups;
    const int maxs = (mp + 63) / 64;
    if (want > maxs) want = maxs;
    if (want > 64) want = 64;
    if (want < 1) want = 1;
    sl = up64((mp + want - 1) / want);
  }
  *split_len = sl;
  *n_splits = (mp + sl - 1) / sl;
}

pe_status check_attn(const pe_attn_args* a) {
  if (!a) return PE_ERR_INVALID_ARG;
  if (a->dtype != PE_F32 && a->dtype != PE_BF16) return PE_ERR_INVALID_ARG;
  if (a->num_q < 0 || a->num_seg < 0 || a->q_per_seg < 0 || a->num_kv_rows < 0) return PE_ERR_INVALID_ARG;
  if ((int64_t)a->num_seg * a->q_per_seg != a->num_q) return PE_ERR_INVALID_ARG;
  if (a->n_q_heads <= 0 || a->n_kv_heads <= 0 || a->n_q_heads % a->n_kv_heads) return PE_ERR_INVALID_ARG;
  const int G = a->n_q_heads / a->n_kv_heads;
  if (G > 64 || 64 % G) return PE_ERR_UNSUPPORTED;
  if (a->head_dim != 64 && a->head_dim != 128) return PE_ERR_UNSUPPORTED;
  if (!(a->scale > 0.f) || !isfinite(a->scale)) return PE_ERR_INVALID_ARG;
  if (a->split_len < 0 || a->max_prefix < 0) return PE_ERR_INVALID_ARG;
  if (a->window_sink < 0 || a->window_len < 0) return PE_ERR_INVALID_ARG;
  if (a->window_len > 0 && a->split_len > 0) return PE_ERR_UNSUPPORTED;  // a window is never split
  if (a->num_q == 0) return PE_OK;
  if (!a->q || !a->k || !a->v || !a->seg_kv_base || !a->q_start || !a->out) return PE_ERR_INVALID_ARG;
  if (a->q_depth) {
    if (!a->q_self_row || !a->kv_parent || a->max_depth < 1) return PE_ERR_INVALID_ARG;
    if (a->max_depth > attn_max_depth(G)) return PE_ERR_UNSUPPORTED;
  }
  if ((a->dbg_count == nullptr) != (a->dbg_hash == nullptr)) return PE_ERR_INVALID_ARG;
  if (a->q_row_stride < (int64_t)a->n_q_heads * a->head_dim) return PE_ERR_INVALID_ARG;
  const int ch = a->dtype == PE_BF16 ? 8 : 4;
  if (a->q_row_stride % ch) return PE_ERR_INVALID_ARG;
  if (!al16(a->q) || !al16(a->k) || !al16(a->v) || !al16(a->out)) return PE_ERR_INVALID_ARG;
  return PE_OK;
}

// Launches of one to four rounds of workgroups (PE_ATTN_NOSPLIT_GROUPS up to
// PE_ATTN_PLAN_GROUPS) run from a device-built work plan: the query tiles in
// decreasing order of work, so that the longest start first and the tail is
// short (a launch of one round otherwise ends with its longest tile).  Below
// PE_ATTN_PLAN_SPLIT_GROUPS the plan also cuts the longer tiles into up to
// three equal pieces of at most 3/8 of the longest possible prefix, merged
// by the combine pass.  Explicit split lengths and windowed launches keep the
// fixed grid.
#ifndef PE_ATTN_PLAN_GROUPS
#define PE_ATTN_PLAN_GROUPS 1024
#endif
#ifndef PE_ATTN_PLAN_SPLIT_GROUPS
#define PE_ATTN_PLAN_SPLIT_GROUPS 1024
#endif
#ifndef PE_ATTN_PLAN_NMAX
#define PE_ATTN_PLAN_NMAX 3
#endif
#ifndef PE_ATTN_PLAN_NUM  // piece length: at most NUM/DEN of the longest possible prefix
#define PE_ATTN_PLAN_NUM 3
#endif
#ifndef PE_ATTN_PLAN_DEN
#define PE_ATTN_PLAN_DEN 8
#endif
struct AttnSplit {
  int n_splits = 1, split_len = 64;  // fixed grid
  int plan = 0, plan_nmax = 1, plan_tiles = 1, ntiles = 0;
};

AttnSplit attn_split(int ntiles, int Hkv, int max_prefix, int split_req, bool window) {
  AttnSplit a;
  a.ntiles = ntiles;
  const int mp = max_prefix > 1 ? max_prefix : 1;
  const int base = ntiles * Hkv > 1 ? ntiles * Hkv : 1;
  if (window) {  // the window kernel walks two tile ranges of one unsplit prefix
    a.split_len = up64(mp);
    return a;
  }
  choose_split(base, max_prefix, split_req, &a.n_splits, &a.split_len);
  if (split_req > 0 || base < PE_ATTN_NOSPLIT_GROUPS || base >= PE_ATTN_PLAN_GROUPS || ntiles > kPlanMaxTiles)
    return a;
  a.plan = 1;
  if (base < PE_ATTN_PLAN_SPLIT_GROUPS) {
    const int max_tiles = (mp + 63) / 64;
    a.plan_nmax = PE_ATTN_PLAN_NMAX;
    a.plan_tiles = (PE_ATTN_PLAN_NUM * max_tiles + PE_ATTN_PLAN_DEN - 1) / PE_ATTN_PLAN_DEN;
    if (a.plan_tiles < 1) a.plan_tiles = 1;
  }
  return a;
}

size_t attn_ws_bytes(int num_q, int Hq, int Hkv, int Dh, const AttnSplit& sp) {
  size_t b = 0;
  const int ns = sp.plan ? sp.plan_nmax : sp.n_splits;
  if (ns > 1) {
    const size_t nqh = (size_t)num_q * Hq;
    b += up256(nqh * ns * Dh * 4) + up256(nqh * ns * 8) + up256((size_t)num_q * Hkv * ns * 16);
  }
  if (sp.plan) b += up256((size_t)sp.ntiles * sp.plan_nmax * 8) + up256((size_t)sp.ntiles * 4) + 256;
  return b > 16 ? b : 16;
}

AttnSplit attn_split_for(const pe_attn_args* a) {
  const int G = a->n_q_heads / a->n_kv_heads;
  const int QPW = attn_queries_per_workgroup(G, a->head_dim);
  const int tps = (a->q_per_seg + QPW - 1) / QPW;
  return attn_split(a->num_seg * tps, a->n_kv_heads, a->max_prefix, a->split_len, a->window_len > 0);
}

pe_status run_attention(const pe_attn_args* a, void* ws, size_t ws_bytes, int meta_by_row, hipStream_t s) {
  const AttnSplit sp = attn_split_for(a);
  const int n_splits = sp.n_splits, split_len = sp.split_len;
  const int ns = sp.plan ? sp.plan_nmax : n_splits;
  const size_t need = attn_ws_bytes(a->num_q, a->n_q_heads, a->n_kv_heads, a->head_dim, sp);
  if ((ns > 1 || sp.plan) && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255)))
    return PE_ERR_INVALID_ARG;
  AttnParams p{};
  p.q = a->q;
  p.q_stride = a->q_row_stride;
  p.q_rows = a->q_rows;
  p.meta_by_row = meta_by_row;
  p.k = a->k;
  p.v = a->v;
  p.num_q = a->num_q;
  p.num_seg = a->num_seg;
  p.q_per_seg = a->q_per_seg;
  p.num_kv_rows = a->num_kv_rows;
  p.Hq = a->n_q_heads;
  p.Hkv = a->n_kv_heads;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.seg_kv_base = a->seg_kv_base;
  p.q_start = a->q_start;
  p.q_depth = a->q_depth;
  p.q_self_row = a->q_self_row;
  p.kv_parent = a->kv_parent;
  p.max_depth = a->q_depth ? a->max_depth : 0;
  p.n_splits = n_splits;
  p.split_len = split_len;
  p.win_sink = a->window_sink;
  p.win_len = a->window_len;
  p.out = a->out;
  p.lse = a->lse;
  p.dbg_count = a->dbg_count;
  p.dbg_hash = a->dbg_hash;
  Carver c(ws);
  if (ns > 1) {
    const size_t nqh = (size_t)a->num_q * a->n_q_heads;
    p.part_o = static_cast<float*>(c.take(nqh * ns * a->head_dim * 4));
    p.part_ml = static_cast<float*>(c.take(nqh * ns * 8));
    p.part_dbg = static_cast<uint64_t*>(c.take((size_t)a->num_q * a->n_kv_heads * ns * 16));
  }
  if (sp.plan) {
    p.plan_items = static_cast<int2*>(c.take((size_t)sp.ntiles * sp.plan_nmax * 8));
    p.plan_pieces = static_cast<int*>(c.take((size_t)sp.ntiles * 4));
    p.plan_count = static_cast<int*>(c.take(256));
    p.plan_nmax = sp.plan_nmax;
    p.plan_tiles = sp.plan_tiles;
  }
  if (a->num_q == 0) return PE_OK;
  launch_attention(p, a->dtype == PE_BF16, a->head_dim, s);
  return launched();
}

// Padding rows of the 16-row activation operand of the weight-streaming
// contractions (M <= 16) read a zero buffer of K elements; it lives in the
// workspace and is cleared by the first RMSNorm launch of the stage.
int zero_ints(size_t max_k_bytes) { return (int)((max_k_bytes + 255) / 256 * 64); }

// Workspace of the drafter layer.
struct LayerWs {
  void *a, *q, *o, *b, *h, *h_lo, *attn;
  float* x1;
  float* split;  // K-split partial products of the large-M contractions
  int64_t split_bytes;
  int* zero;
  int nzero;
  size_t attn_bytes, total;
};

LayerWs layer_ws(const pe_drafter_dims* d, int T, int R, int K, int max_pos, void* base) {
  LayerWs w{};
  Carver c(base);
  const size_t e = esize(d->dtype);
  const int RK = R * K;
  const int qc = d->n_q_heads * d->head_dim;
  int kmax = d->hidden > qc ? d->hidden : qc;
  if (d->ffn > kmax) kmax = d->ffn;
  w.nzero = zero_ints((size_t)kmax * e);
  w.a = c.take((size_t)((T + 15) / 16 * 16) * d->hidden * e);  // rows padded to 16 (operand layout)
  w.q = c.take((size_t)T * qc * e);
  w.o = c.take((size_t)RK * qc * e);
  w.x1 = static_cast<float*>(c.take((size_t)RK * d->hidden * 4));
  w.b = c.take((size_t)RK * d->hidden * e);
  w.h = c.take((size_t)RK * d->ffn * e);
  // remainder of the SwiGLU output: the down projection's second operand part
  // (weight-streaming batches of bf16 rows only)
  w.h_lo = (RK <= 16 && d->dtype == PE_BF16) ? c.take((size_t)RK * d->ffn * e) : nullptr;
  w.zero = static_cast<int*>(c.take((size_t)w.nzero * 4));
  const int G = d->n_q_heads / d->n_kv_heads;
  const int QPW = attn_queries_per_workgroup(G, d->head_dim);
  const AttnSplit sp = attn_split(R * ((K + QPW - 1) / QPW), d->n_kv_heads, max_pos, 0, false);
  w.attn_bytes = attn_ws_bytes(RK, d->n_q_heads, d->n_kv_heads, d->head_dim, sp);
  w.attn = c.take(w.attn_bytes);
  int nmax = d->hidden > (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim ? d->hidden
                                                                         : (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  if (d->ffn > nmax) nmax = d->ffn;
  w.split_bytes = d->dtype == PE_BF16 ? gemm_split_bytes(T, nmax) : 0;
  w.split = static_cast<float*>(c.take((size_t)w.split_bytes));
  w.total = c.off;
  return w;
}

// Workspace of the fc fusion.
struct FuseWs {
  void* u;
  float* inv;  // deferred 1 / rms per (row, stream) when a norm kernel runs first
  float* split;  // K-split partial products of a large-M fc
  int64_t split_bytes;
  int* zero;
  int nzero;
  size_t total;
};

FuseWs fuse_ws(const pe_drafter_dims* d, int T, void* base) {
  FuseWs w{};
  Carver c(base);
  w.nzero = zero_ints((size_t)3 * d->hidden * esize(d->dtype));
  w.u = c.take((size_t)((T + 15) / 16 * 16) * 3 * d->hidden * esize(d->dtype));  // rows padded to 16
  w.inv = static_cast<float*>(c.take((size_t)T * 3 * 4));
  w.zero = static_cast<int*>(c.take((size_t)w.nzero * 4));
  w.split_bytes = d->dtype == PE_BF16 ? gemm_split_bytes(T, d->hidden) : 0;
  w.split = static_cast<float*>(c.take((size_t)w.split_bytes));
  w.total = c.off;
  return w;
}

// Workspace of the LM head (loss: the log-sum-exp partial sums and the
// target logits instead of the argmax indices).
struct LmWs {
  void* f;
  float* pv;
  u32x4* top2;
  float* ps;
  float* tgt;
  float* lse;  // KL loss: the rows' log-sum-exp when the caller keeps none
  int* zero;
  int nzero;
  size_t total;
};

LmWs lm_ws(const pe_drafter_dims* d, int n, void* base, bool loss = false, bool kl = false) {
  LmWs w{};
  Carver c(base);
  const size_t P = (size_t)gemm_argmax_partials(n, d->vocab);
  w.f = c.take((size_t)((n + 15) / 16 * 16) * d->hidden * esize(d->dtype));  // rows padded to 16 (operand layout)
  if (loss) {
    w.pv = static_cast<float*>(c.take(P * n * 4));
    w.ps = static_cast<float*>(c.take(P * n * 4));
    w.tgt = static_cast<float*>(c.take((size_t)n * 4));
    if (kl) w.lse = static_cast<float*>(c.take((size_t)n * 4));
  } else {
    w.top2 = static_cast<u32x4*>(c.take(P * n * 16));
  }
  w.nzero = zero_ints((size_t)d->hidden * esize(d->dtype));
  w.zero = static_cast<int*>(c.take((size_t)w.nzero * 4));
  w.total = c.off;
  return w;
}

bool ws_ok(void* ws, size_t have, size_t need) {
  return ws && have >= need && (reinterpret_cast<uintptr_t>(ws) & 255) == 0;
}

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current (thread-safe); nullptr on failure.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    const hipError_t st = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = st == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}

pe_status check_attn_bwd(const pe_attn_bwd_args* a) {
  if (!a) return PE_ERR_INVALID_ARG;
  if (a->dtype != PE_BF16) return a->dtype == PE_F32 ? PE_ERR_UNSUPPORTED : PE_ERR_INVALID_ARG;
  if (a->num_rows <= 0 || a->n_pos <= 0 || a->n_pos > a->num_rows) return PE_ERR_INVALID_ARG;
  if (a->n_groups < 1 || a->n_groups > 16) return PE_ERR_UNSUPPORTED;
  if (a->n_q_heads <= 0 || a->n_kv_heads <= 0 || a->n_q_heads % a->n_kv_heads) return PE_ERR_INVALID_ARG;
  const int G = a->n_q_heads / a->n_kv_heads;
  if (G > 64 || 64 % G) return PE_ERR_UNSUPPORTED;
  if (a->head_dim != 64 && a->head_dim != 128) return PE_ERR_UNSUPPORTED;
  if (!(a->scale > 0.f) || !isfinite(a->scale)) return PE_ERR_INVALID_ARG;
  if (a->q_begin < 0 || a->q_end < a->q_begin || a->q_end > a->num_rows) return PE_ERR_INVALID_ARG;
  if ((int64_t)a->num_rows * a->n_q_heads * a->head_dim >= ((int64_t)1 << 31)) return PE_ERR_INVALID_ARG;
  if (!a->group_off || !a->start || !a->depth || !a->lse) return PE_ERR_INVALID_ARG;
  if (!a->q || !a->k || !a->v || !a->out || !a->dout) return PE_ERR_INVALID_ARG;
  if (!al16(a->q) || !al16(a->k) || !al16(a->v) || !al16(a->out) || !al16(a->dout)) return PE_ERR_INVALID_ARG;
  if (a->q_end > a->q_begin && (!a->dq || !a->dk || !a->dv || !al16(a->dq) || !al16(a->dk) || !al16(a->dv)))
    return PE_ERR_INVALID_ARG;
  return PE_OK;
}

size_t attn_bwd_ws_bytes(const pe_attn_bwd_args* a) {
  const size_t part = up256((size_t)attn_bwd_part_floats(a->num_rows, a->n_groups, a->n_kv_heads, a->head_dim) * 4);
  return up256((size_t)(a->q_end - a->q_begin) * a->n_q_heads * 4) + 2 * part + 256;
}

}  // namespace

extern "C" {

const char* pe_status_string(pe_status s) {
  switch (s) {
    case PE_OK: return "PE_OK";
    case PE_ERR_INVALID_ARG: return "PE_ERR_INVALID_ARG";
    case PE_ERR_UNSUPPORTED: return "PE_ERR_UNSUPPORTED";
    case PE_ERR_DEVICE: return "PE_ERR_DEVICE";
  }
  return "PE_ERR_UNKNOWN";
}

const char* pe_version(void) { return kVersion; }

pe_status pe_build_draft_batch(const pe_drafter_dims* dims, int32_t R, int32_t K, int32_t total_window_rows,
                               int32_t target_rows, const int32_t* cu_window, const int32_t* n_rej,
                               const int32_t* kv_len, const int32_t* kv_base, const int32_t* window_ids,
                               const int32_t* window_pos, const int32_t* window_hrow, const int32_t* new_token,
                               const int32_t* ctx_hrow, const void* target_hidden, const void* h_shared,
                               const pe_batch_out* out, hipStream_t stream) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (R < 1 || K < 1 || total_window_rows < 0 || target_rows < 1) return PE_ERR_INVALID_ARG;
  const int64_t T = (int64_t)total_window_rows + (int64_t)R * K;
  if (T >= ((int64_t)1 << 31) - 1) return PE_ERR_INVALID_ARG;
  if (!out || !cu_window || !n_rej || !kv_len || !kv_base || !new_token || !ctx_hrow || !target_hidden || !h_shared)
    return PE_ERR_INVALID_ARG;
  if (total_window_rows > 0 && (!window_ids || !window_pos || !window_hrow)) return PE_ERR_INVALID_ARG;
  if (!out->draft_ids || !out->draft_pos || !out->slot_mapping || !out->hidden_src || !out->req_of_row ||
      !out->rejected || !out->masked || !out->query_rows || !out->cu_draft || !out->draft_hidden)
    return PE_ERR_INVALID_ARG;
  if (!al16(target_hidden) || !al16(h_shared) || !al16(out->draft_hidden)) return PE_ERR_INVALID_ARG;
  BatchParams p{};
  p.R = R;
  p.K = K;
  p.T = (int)T;
  p.target_rows = target_rows;
  p.mask_token_id = dims->mask_token_id;
  p.row_bytes = (int)(3 * (int64_t)dims->hidden * esize(dims->dtype));
  p.cu_window = cu_window;
  p.n_rej = n_rej;
  p.kv_len = kv_len;
  p.kv_base = kv_base;
  p.window_ids = window_ids;
  p.window_pos = window_pos;
  p.window_hrow = window_hrow;
  p.new_token = new_token;
  p.ctx_hrow = ctx_hrow;
  p.target_hidden = target_hidden;
  p.h_shared = h_shared;
  p.draft_ids = out->draft_ids;
  p.draft_pos = out->draft_pos;
  p.slot_mapping = out->slot_mapping;
  p.hidden_src = out->hidden_src;
  p.req_of_row = out->req_of_row;
  p.query_rows = out->query_rows;
  p.cu_draft = out->cu_draft;
  p.rejected = out->rejected;
  p.masked = out->masked;
  p.draft_hidden = out->draft_hidden;
  launch_build_draft_batch(p, stream);
  return launched();
}

pe_status pe_packed_weight_bytes(pe_dtype dtype, int32_t N, int32_t K, size_t* bytes) {
  if ((dtype != PE_F32 && dtype != PE_BF16) || N <= 0 || K <= 0 || !bytes) return PE_ERR_INVALID_ARG;
  const int64_t row_bytes = (int64_t)K * (int64_t)esize(dtype);
  if (row_bytes % 64) return PE_ERR_UNSUPPORTED;
  *bytes = (size_t)((int64_t)(N + 15) / 16 * 16 * row_bytes);
  return PE_OK;
}

pe_status pe_pack_weight(pe_dtype dtype, int32_t N, int32_t K, const void* src, void* dst, hipStream_t stream) {
  size_t bytes;
  pe_status st = pe_packed_weight_bytes(dtype, N, K, &bytes);
  if (st != PE_OK) return st;
  if (!src || !dst || !al16(src) || !al16(dst)) return PE_ERR_INVALID_ARG;
  if ((int64_t)K * (int64_t)esize(dtype) > ((int64_t)1 << 30)) return PE_ERR_UNSUPPORTED;
  launch_pack(src, dst, N, (int)(K * esize(dtype)), stream);
  return launched();
}

pe_status pe_fuse_hidden_workspace(const pe_drafter_dims* dims, int32_t T, size_t* bytes) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (T < 0 || !bytes) return PE_ERR_INVALID_ARG;
  *bytes = fuse_ws(dims, T, nullptr).total;
  return PE_OK;
}

pe_status pe_fuse_hidden(const pe_drafter_dims* dims, const pe_drafter_weights* w, int32_t T,
                         const void* draft_hidden, const uint8_t* rejected, const int32_t* ids, float* x0,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (!w || T < 0) return PE_ERR_INVALID_ARG;
  if (T == 0) return PE_OK;
  if (!draft_hidden || !ids || !x0 || !w->embed || !w->stream_gain || !w->w_fc) return PE_ERR_INVALID_ARG;
  if (!al16(draft_hidden) || !al16(w->w_fc) || !al16(w->embed) || !al16(x0)) return PE_ERR_INVALID_ARG;
  if (!ws_ok(workspace, workspace_bytes, fuse_ws(dims, T, nullptr).total)) return PE_ERR_INVALID_ARG;
  const FuseWs fw = fuse_ws(dims, T, workspace);
  const int d = dims->hidden;
  const int bf = dims->dtype == PE_BF16;
  // u_s = RMSNorm(stream s) feeds w_fc (fused into the contraction's staging when it fits)
  GemmParams gp{};
  gp.X = draft_hidden;
  gp.ldx = 3 * (int64_t)d;
  gp.W = w->w_fc;
  gp.M = T;
  gp.N = d;
  gp.K = 3 * d;
  gp.xzero = fw.zero;
  gp.nrm.gain = w->stream_gain;
  gp.nrm.segs = 3;
  gp.nrm.seg_len = d;
  gp.nrm.eps = dims->eps;
  gp.nrm.skip = rejected;
  gp.nrm.tmp = fw.u;
  // each stream's 1 / rms scales its share of the sum after the contraction:
  // the operand is then the captured bf16 rows times their gains (the rows
  // themselves for unit gains), with no rounding of the normalised values
  gp.nrm.defer = 1;
  gp.nrm.inv_tmp = fw.inv;
  gp.clear = fw.zero;
  gp.nclear = fw.nzero;
  gp.split_ws = fw.split;
  gp.split_cap = fw.split_bytes;
  gp.epi.kind = EPI_FC;
  gp.epi.out_f32 = x0;
  gp.epi.ld_out = d;
  gp.epi.embed = w->embed;
  gp.epi.ids = ids;
  gp.epi.rejected = rejected;
  gp.epi.embed_rows = dims->vocab;
  launch_gemm(gp, bf, stream);
  return launched();
}

pe_status pe_draft_attention_workspace(const pe_attn_args* args, size_t* bytes) {
  pe_status st = check_attn(args);
  if (st != PE_OK) return st;
  if (!bytes) return PE_ERR_INVALID_ARG;
  *bytes = attn_ws_bytes(args->num_q, args->n_q_heads, args->n_kv_heads, args->head_dim, attn_split_for(args));
  return PE_OK;
}

pe_status pe_draft_attention(const pe_attn_args* args, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pe_status st = check_attn(args);
  if (st != PE_OK) return st;
  return run_attention(args, workspace, workspace_bytes, 0, stream);
}

pe_status pe_draft_layer_workspace(const pe_drafter_dims* dims, int32_t T, int32_t R, int32_t K, int32_t max_pos,
                                   size_t* bytes) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (T < 0 || R < 0 || K < 0 || max_pos < 0 || !bytes) return PE_ERR_INVALID_ARG;
  *bytes = layer_ws(dims, T, R, K, max_pos, nullptr).total;
  return PE_OK;
}

pe_status pe_draft_layer(const pe_drafter_dims* dims, const pe_drafter_weights* w, int32_t T, int32_t R, int32_t K,
                         const float* x0, const pe_batch_out* batch, const int32_t* kv_base, void* k_cache,
                         void* v_cache, int32_t kv_rows, int32_t max_pos, float* x_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (!w || !batch || T < 0 || R < 0 || K < 0 || kv_rows < 0 || max_pos < 0) return PE_ERR_INVALID_ARG;
  if ((int64_t)R * K > T) return PE_ERR_INVALID_ARG;
  if (T == 0 || R * K == 0) return PE_OK;
  if (!x0 || !kv_base || !k_cache || !v_cache || !x_out || !batch->slot_mapping || !batch->draft_pos ||
      !batch->query_rows)
    return PE_ERR_INVALID_ARG;
  if (!w->attn_gain || !w->w_qkv || !w->w_o || !w->mlp_gain || !w->w_gate || !w->w_up || !w->w_down)
    return PE_ERR_INVALID_ARG;
  if (!al16(k_cache) || !al16(v_cache) || !al16(w->w_qkv) || !al16(w->w_o) || !al16(w->w_gate) || !al16(w->w_up) ||
      !al16(w->w_down))
    return PE_ERR_INVALID_ARG;
  if (!al16(x0) || !al16(x_out)) return PE_ERR_INVALID_ARG;
  if (!ws_ok(workspace, workspace_bytes, layer_ws(dims, T, R, K, max_pos, nullptr).total)) return PE_ERR_INVALID_ARG;
  const LayerWs lw = layer_ws(dims, T, R, K, max_pos, workspace);
  const int d = dims->hidden, Hq = dims->n_q_heads, Hkv = dims->n_kv_heads, Dh = dims->head_dim, F = dims->ffn;
  const int bf = dims->dtype == PE_BF16;
  const int RK = R * K;
  const int qcols = Hq * Dh, kvcols = Hkv * Dh;

  // [q|k|v] = W_qkv RMSNorm(x0) for every row (rejected rows normalise to zeros;
  // their K/V are not written); k, v scattered to the cache by slot
  GemmParams gp{};
  gp.X = x0;
  gp.ldx = d;
  gp.W = w->w_qkv;
  gp.M = T;
  gp.N = qcols + 2 * kvcols;
  gp.K = d;
  gp.xzero = lw.zero;
  gp.split_ws = lw.split;
  gp.split_cap = lw.split_bytes;
  gp.nrm.gain = w->attn_gain;
  gp.nrm.segs = 1;
  gp.nrm.seg_len = d;
  gp.nrm.eps = dims->eps;
  gp.nrm.skip = batch->rejected;
  gp.nrm.x_f32 = 1;
  gp.nrm.tmp = lw.a;
  gp.clear = lw.zero;
  gp.nclear = lw.nzero;
  gp.epi.kind = EPI_QKV;
  gp.epi.out_s = lw.q;
  gp.epi.q_cols = qcols;
  gp.epi.kv_cols = kvcols;
  gp.epi.kv_rows = kv_rows;
  gp.epi.k_cache = k_cache;
  gp.epi.v_cache = v_cache;
  gp.epi.slots = batch->slot_mapping;
  launch_gemm(gp, bf, stream);

  // attention of the query rows over their regions
  pe_attn_args aa{};
  aa.num_q = RK;
  aa.num_seg = R;
  aa.q_per_seg = K;
  aa.num_kv_rows = kv_rows;
  aa.n_q_heads = Hq;
  aa.n_kv_heads = Hkv;
  aa.head_dim = Dh;
  aa.scale = 1.0f / sqrtf((float)Dh);
  aa.dtype = dims->dtype;
  aa.q = lw.q;
  aa.q_row_stride = qcols;
  aa.q_rows = batch->query_rows;
  aa.k = k_cache;
  aa.v = v_cache;
  aa.seg_kv_base = kv_base;
  aa.q_start = batch->draft_pos;
  aa.max_prefix = max_pos;
  aa.out = lw.o;
  st = run_attention(&aa, lw.attn, lw.attn_bytes, 1, stream);
  if (st != PE_OK) return st;

  // x1 = x0[query rows] + W_o o
  gp = GemmParams{};
  gp.X = lw.o;
  gp.ldx = qcols;
  gp.W = w->w_o;
  gp.M = RK;
  gp.N = d;
  gp.K = qcols;
  gp.xzero = lw.zero;
  gp.split_ws = lw.split;
  gp.split_cap = lw.split_bytes;
  gp.epi.kind = EPI_RESID;
  gp.epi.out_f32 = lw.x1;
  gp.epi.ld_out = d;
  gp.epi.res = x0;
  gp.epi.res_rows = batch->query_rows;
  gp.epi.ld_res = d;
  launch_gemm(gp, bf, stream);

  // h = silu(W_gate b) * (W_up b),  b = RMSNorm(x1)
  gp = GemmParams{};
  gp.X = lw.x1;
  gp.ldx = d;
  gp.W = w->w_gate;
  gp.W2 = w->w_up;
  gp.M = RK;
  gp.N = F;
  gp.K = d;
  gp.xzero = lw.zero;
  gp.split_ws = lw.split;
  gp.split_cap = lw.split_bytes;
  gp.nrm.gain = w->mlp_gain;
  gp.nrm.segs = 1;
  gp.nrm.seg_len = d;
  gp.nrm.eps = dims->eps;
  gp.nrm.x_f32 = 1;
  gp.nrm.tmp = lw.b;
  // weight-streaming batches: the normalised rows and their remainder as two
  // bf16 operand parts, and the output's remainder for the down projection
  gp.x_split = lw.h_lo != nullptr;
  gp.epi.kind = EPI_SWIGLU;
  gp.epi.out_s = lw.h;
  gp.epi.out_s_lo = lw.h_lo;
  gp.epi.ld_out = F;
  launch_gemm(gp, bf, stream);

  // x_out = x1 + W_down h
  gp = GemmParams{};
  gp.X = lw.h;
  gp.x_lo = lw.h_lo;
  gp.ldx = F;
  gp.W = w->w_down;
  gp.M = RK;
  gp.N = d;
  gp.K = F;
  gp.xzero = lw.zero;
  gp.split_ws = lw.split;
  gp.split_cap = lw.split_bytes;
  gp.epi.kind = EPI_RESID;
  gp.epi.out_f32 = x_out;
  gp.epi.ld_out = d;
  gp.epi.res = lw.x1;
  gp.epi.ld_res = d;
  launch_gemm(gp, bf, stream);
  return launched();
}

pe_status pe_lm_head_argmax_workspace(const pe_drafter_dims* dims, int32_t n, size_t* bytes) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (n < 0 || !bytes) return PE_ERR_INVALID_ARG;
  *bytes = lm_ws(dims, n, nullptr).total;
  return PE_OK;
}

}  // extern "C"

namespace {

// Argument checks of pe_lm_head_argmax (everything but the workspace).
pe_status check_lm_argmax(const pe_drafter_dims* dims, const pe_drafter_weights* w, int32_t n, const float* x,
                          const int32_t* tokens) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (!w || n < 0) return PE_ERR_INVALID_ARG;
  if (n == 0) return PE_OK;
  if (!x || !tokens || !w->final_gain || !w->w_lm || !al16(w->w_lm) || !al16(x) || !al16(w->final_gain))
    return PE_ERR_INVALID_ARG;
  return PE_OK;
}

// The LM head's launches on a checked workspace (n > 0).
pe_status run_lm_argmax(const pe_drafter_dims* dims, const pe_drafter_weights* w, int32_t n, const float* x,
                        int32_t* tokens, float* logits, void* workspace, hipStream_t stream) {
  const LmWs lw = lm_ws(dims, n, workspace);
  const int d = dims->hidden;
  const int bf = dims->dtype == PE_BF16;
  // z = w_lm RMSNorm(x): the norm is fused into the LM kernel's staging when it fits
  GemmParams gp{};
  gp.X = x;
  gp.ldx = d;
  gp.W = w->w_lm;
  gp.M = n;
  gp.N = dims->vocab;
  gp.K = d;
  gp.xzero = lw.zero;
  gp.nrm.gain = w->final_gain;
  gp.nrm.segs = 1;
  gp.nrm.seg_len = d;
  gp.nrm.eps = dims->eps;
  gp.nrm.x_f32 = 1;
  gp.nrm.tmp = lw.f;
  gp.clear = lw.zero;
  gp.nclear = lw.nzero;
  gp.epi.kind = EPI_ARGMAX;
  gp.epi.logits = logits;
  gp.epi.part_top2 = lw.top2;
  const int used = launch_gemm(gp, bf, stream);
  // the two leading tokens of each row scored again in fp32 from x, unless
  // the logits came from the hi + lo operand (then the largest is the token)
  const int rescore = lm_head_exact(n, d, bf, w->final_gain) ? 0 : 1;
  launch_argmax_rescore(lw.top2, used, n, x, d, w->final_gain, dims->eps, w->w_lm, d, bf, tokens, rescore, stream);
  return launched();
}

}  // namespace

extern "C" {

pe_status pe_lm_head_argmax(const pe_drafter_dims* dims, const pe_drafter_weights* w, int32_t n, const float* x,
                            int32_t* tokens, float* logits, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  const pe_status st = check_lm_argmax(dims, w, n, x, tokens);
  if (st != PE_OK || n == 0) return st;
  if (!ws_ok(workspace, workspace_bytes, lm_ws(dims, n, nullptr).total)) return PE_ERR_INVALID_ARG;
  return run_lm_argmax(dims, w, n, x, tokens, logits, workspace, stream);
}

pe_status pe_lm_head_argmax_noalloc(const pe_drafter_dims* dims, const pe_drafter_weights* w, int32_t n,
                                    const float* x, int32_t* tokens, float* logits, hipStream_t stream) {
  const pe_status st = check_lm_argmax(dims, w, n, x, tokens);
  if (st != PE_OK || n == 0) return st;
  if (lm_ws(dims, n, nullptr).total > PE_NOALLOC_SCRATCH_BYTES) return PE_ERR_UNSUPPORTED;
  void* ws = scratch_ptr();  // this device's array, never the symbol itself
  if (!ws) return PE_ERR_DEVICE;
  return run_lm_argmax(dims, w, n, x, tokens, logits, ws, stream);
}

pe_status pe_lm_head_loss_workspace(const pe_drafter_dims* dims, int32_t n, size_t* bytes) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (!bytes || n < 0) return PE_ERR_INVALID_ARG;
  *bytes = lm_ws(dims, n, nullptr, true).total;
  return PE_OK;
}

pe_status pe_lm_head_loss(const pe_drafter_dims* dims, const pe_drafter_weights* w, int32_t n, const float* x,
                          const int32_t* targets, float* lse, float* loss, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (!w || n < 0) return PE_ERR_INVALID_ARG;
  if (n == 0) return PE_OK;
  if (!x || !w->final_gain || !w->w_lm || !al16(w->w_lm) || !al16(x)) return PE_ERR_INVALID_ARG;
  if (!lse && !loss) return PE_ERR_INVALID_ARG;
  if (loss && !targets) return PE_ERR_INVALID_ARG;
  if (!ws_ok(workspace, workspace_bytes, lm_ws(dims, n, nullptr, true).total)) return PE_ERR_INVALID_ARG;
  const LmWs lw = lm_ws(dims, n, workspace, true);
  const int d = dims->hidden;
  const int bf = dims->dtype == PE_BF16;
  // z = w_lm RMSNorm(x), streamed tile by tile: per tile (max, sum of exp) and the target's logit
  GemmParams gp{};
  gp.X = x;
  gp.ldx = d;
  gp.W = w->w_lm;
  gp.M = n;
  gp.N = dims->vocab;
  gp.K = d;
  gp.xzero = lw.zero;
  gp.nrm.gain = w->final_gain;
  gp.nrm.segs = 1;
  gp.nrm.seg_len = d;
  gp.nrm.eps = dims->eps;
  gp.nrm.x_f32 = 1;
  gp.nrm.tmp = lw.f;
  gp.clear = lw.zero;
  gp.nclear = lw.nzero;
  gp.epi.kind = EPI_LSE;
  gp.epi.part_val = lw.pv;
  gp.epi.part_sum = lw.ps;
  gp.epi.targets = targets;
  gp.epi.tgt_logit = lw.tgt;
  const int used = launch_gemm(gp, bf, stream);
  launch_lse_reduce(lw.pv, lw.ps, used, n, dims->vocab, targets, lw.tgt, lse, loss, stream);
  return launched();
}

pe_status pe_lm_head_kl_workspace(const pe_drafter_dims* dims, int32_t n, size_t* bytes) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (!bytes || n < 0) return PE_ERR_INVALID_ARG;
  *bytes = lm_ws(dims, n, nullptr, true, true).total;
  return PE_OK;
}

pe_status pe_lm_head_kl(const pe_drafter_dims* dims, const pe_drafter_weights* w, int32_t n, const float* x,
                        int32_t k, const int32_t* target_ids, const float* target_probs, const void* w_lm_rows,
                        float* lse, float* kl, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pe_status st = check_dims(dims);
  if (st != PE_OK) return st;
  if (!w || n < 0 || k < 1) return PE_ERR_INVALID_ARG;
  if ((int64_t)n * k > INT32_MAX) return PE_ERR_INVALID_ARG;
  if (n == 0) return PE_OK;
  if (!x || !w->final_gain || !w->w_lm || !al16(w->w_lm) || !al16(x) || !al16(w->final_gain)) return PE_ERR_INVALID_ARG;
  if (!target_ids || !target_probs || !kl) return PE_ERR_INVALID_ARG;
  if (w_lm_rows && !al16(w_lm_rows)) return PE_ERR_INVALID_ARG;
  const int bf = dims->dtype == PE_BF16;
  if (kl_topk_lds_bytes(dims->hidden, bf) > 65536) return PE_ERR_UNSUPPORTED;
  if (!ws_ok(workspace, workspace_bytes, lm_ws(dims, n, nullptr, true, true).total)) return PE_ERR_INVALID_ARG;
  const LmWs lw = lm_ws(dims, n, workspace, true, true);
  const int d = dims->hidden;
  // the log-sum-exp of z = w_lm RMSNorm(x), streamed tile by tile as in pe_lm_head_loss
  GemmParams gp{};
  gp.X = x;
  gp.ldx = d;
  gp.W = w->w_lm;
  gp.M = n;
  gp.N = dims->vocab;
  gp.K = d;
  gp.xzero = lw.zero;
  gp.nrm.gain = w->final_gain;
  gp.nrm.segs = 1;
  gp.nrm.seg_len = d;
  gp.nrm.eps = dims->eps;
  gp.nrm.x_f32 = 1;
  gp.nrm.tmp = lw.f;
  gp.clear = lw.zero;
  gp.nclear = lw.nzero;
  gp.epi.kind = EPI_LSE;
  gp.epi.part_val = lw.pv;
  gp.epi.part_sum = lw.ps;
  const int used = launch_gemm(gp, bf, stream);
  float* l = lse ? lse : lw.lse;
  launch_lse_reduce(lw.pv, lw.ps, used, n, dims->vocab, nullptr, nullptr, l, nullptr, stream);
  // the target logits in fp32 and the KL sum of each row
  launch_kl_topk(x, d, w->final_gain, dims->eps, w->w_lm, w_lm_rows, d, dims->vocab, bf, k, target_ids, target_probs, l,
                 kl, n, stream);
  return launched();
}

pe_status pe_draft_attention_backward_workspace(const pe_attn_bwd_args* args, size_t* bytes) {
  pe_status st = check_attn_bwd(args);
  if (st != PE_OK) return st;
  if (!bytes) return PE_ERR_INVALID_ARG;
  *bytes = attn_bwd_ws_bytes(args);
  return PE_OK;
}

pe_status pe_draft_attention_backward(const pe_attn_bwd_args* a, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  pe_status st = check_attn_bwd(a);
  if (st != PE_OK) return st;
  if (a->q_end == a->q_begin) return PE_OK;
  if (!ws_ok(workspace, workspace_bytes, attn_bwd_ws_bytes(a))) return PE_ERR_INVALID_ARG;
  AttnBwdParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.out = a->out;
  p.dout = a->dout;
  p.lse = a->lse;
  p.start = a->start;
  p.depth = a->depth;
  p.group_off = a->group_off;
  p.T = a->num_rows;
  p.N = a->n_pos;
  p.D = a->n_groups;
  p.Hq = a->n_q_heads;
  p.Hkv = a->n_kv_heads;
  p.q_begin = a->q_begin;
  p.q_end = a->q_end;
  p.scale = a->scale;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  Carver c(workspace);
  p.delta = static_cast<float*>(c.take((size_t)(a->q_end - a->q_begin) * a->n_q_heads * 4));
  const size_t part = (size_t)attn_bwd_part_floats(a->num_rows, a->n_groups, a->n_kv_heads, a->head_dim) * 4;
  p.part_k = static_cast<float*>(c.take(part));
  p.part_v = static_cast<float*>(c.take(part));
  launch_attention_backward(p, a->head_dim, stream);
  return launched();
}

}  // extern "C"
