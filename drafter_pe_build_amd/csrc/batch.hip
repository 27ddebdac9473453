// Stage 1: draft-batch construction in one pass.
//
// "P-EAGLE: parallel speculative decoding in vLLM", sections "fused Triton
// kernel" and "hidden-state management": one kernel copies the previous ids
// and positions, inserts the new token, MASK-fills the parallel slots, emits
// the rejected / masked flags and the hidden-state mapping, and copies the
// hidden rows (target rows to their new positions, h_shared into every MASK
// slot).  Section "KV cache": rejected rows get PADDING_SLOT_ID (-1).
//
// One workgroup per draft row: the first wave finds the row's request (row
// r's request segment starts at cu_window[r] + r*K), thread 0 writes the
// integer metadata, and the whole workgroup copies the row's 3*hidden hidden
// values with 16-byte loads and stores.
#include "kernels.h"

namespace pe {

// First request whose segment starts after row t (the starts increase
// strictly with r), by the first wave: 64 evenly spaced probes per round,
// whose ballot leaves the answer between two neighbouring probes; up to 64
// requests take one round (the c=64 batch: one dependent read instead of
// six of a binary search).
__device__ int first_segment_after(const BatchParams& p, int t) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = p.R;
  while (hi > lo) {
    const int n = hi - lo;
    if (n <= 64) {
      const bool le = lane < n && p.cu_window[lo + lane] + (lo + lane) * p.K <= t;
      return lo + __popcll(__ballot(le));
    }
    // probe i(l) = lo + n (l + 1) / 65, l = 0..63: increasing, inside [lo, hi)
    auto probe = [&](int l) { return lo + (int)((int64_t)n * (l + 1) / 65); };
    const int i = probe(lane);
    const int c = __popcll(__ballot(p.cu_window[i] + i * p.K <= t));  // a prefix of the probes
    const int nlo = c > 0 ? probe(c - 1) + 1 : lo;
    const int nhi = c < 64 ? probe(c) : hi;
    if (c < 64 && nhi == nlo) return nhi;
    lo = nlo;
    hi = nhi;
  }
  return lo;
}

__global__ __launch_bounds__(256) void build_draft_batch_kernel(BatchParams p) {
  __shared__ int s_src;   // hidden source row, -1 = h_shared, -2 = none
  const int t = blockIdx.x;
  // largest r with cu_window[r] + r*K <= t (0 when none: a malformed cu_window)
  const int r = p.R > 1 && threadIdx.x < 64 ? max(first_segment_after(p, t) - 1, 0) : 0;
  if (threadIdx.x == 0) {
    // every per-request value in one round trip, whichever the row needs
    const int w0 = p.cu_window[r], w1 = p.cu_window[r + 1];
    const int nrej_in = p.n_rej[r], base = p.kv_base[r], kvl = p.kv_len[r];
    const int new_tok = p.new_token[r], ctx = p.ctx_hrow[r];
    const int W = w1 - w0;
    const int first = w0 + r * p.K;
    const int j = t - first;
    const int nrej = min(max(nrej_in, 0), max(W, 0));
    const int n_acc = W - nrej;
    int id, pos, slot, src;
    uint8_t rej = 0, msk = 0;
    if (j < W) {
      const int w = w0 + j;
      id = p.window_ids[w];
      pos = p.window_pos[w];
      src = p.window_hrow[w];
      if (j >= n_acc) { rej = 1; slot = -1; } else { slot = base + pos; }
    } else {
      const int k = j - W;
      pos = kvl + n_acc + k;
      slot = base + pos;
      if (k == 0) { id = new_tok; src = ctx; }
      else { id = p.mask_token_id; src = -1; msk = 1; }
      if (k < p.K) p.query_rows[r * p.K + k] = t;
    }
    if (j == 0) p.cu_draft[r] = t;
    if (t == p.T - 1) p.cu_draft[p.R] = p.T;
    p.draft_ids[t] = id;
    p.draft_pos[t] = pos;
    p.slot_mapping[t] = slot;
    p.hidden_src[t] = src;
    p.req_of_row[t] = r;
    p.rejected[t] = rej;
    p.masked[t] = msk;
    s_src = (src >= p.target_rows) ? -2 : (src < -1 ? -2 : src);
  }
  __syncthreads();
  const int src = s_src;
  if (src == -2) return;
  const char* from = (src < 0) ? reinterpret_cast<const char*>(p.h_shared)
                               : reinterpret_cast<const char*>(p.target_hidden) + (int64_t)src * p.row_bytes;
  char* to = reinterpret_cast<char*>(p.draft_hidden) + (int64_t)t * p.row_bytes;
  // all of a thread's chunks in flight at once (a 3 x 2,880 bf16 row is 1,080
  // chunks: one batch of 5 per thread); addresses clamped, stores predicated
  constexpr int U = 5;
  const int nch = p.row_bytes / 16;
  for (int c0 = threadIdx.x; c0 < nch; c0 += 256 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld16(from + 16 * (int64_t)min(c0 + 256 * u, nch - 1));
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + 256 * u < nch) st16(to + 16 * (int64_t)(c0 + 256 * u), v[u]);
  }
}

void launch_build_draft_batch(const BatchParams& p, hipStream_t s) {
  hipLaunchKernelGGL(build_draft_batch_kernel, dim3(p.T), dim3(256), 0, s, p);
}

}  // namespace pe
