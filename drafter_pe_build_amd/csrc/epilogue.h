// The epilogues that finish a contraction element Y[m][n] (see EpiKind in
// kernels.h), shared by the streaming and the tiled kernels.
#pragma once
#include "kernels.h"

namespace pe {

// Per-row reduction of the LM head over the features a lane, a wave, a tile
// has seen: argmax as the two largest values (v, lowest index i; then v2,
// i2; "larger" orders equal values by the lower index), or log-sum-exp
// (maximum v and s = sum of exp(y - v)).  States merge in a fixed order, so
// the results do not depend on timing.
struct RowRed {
  float v, s;
  int i;
  float v2;
  int i2;
  __device__ static RowRed init() { return RowRed{-INFINITY, 0.f, 0x7fffffff, -INFINITY, 0x7fffffff}; }
  __device__ void add(bool lse, float y, int n) {
    if (lse) {
      if (y > v) { s = s * expf(v - y) + 1.f; v = y; }
      else s += expf(y - v);
    } else if (better(y, n, v, i)) {
      v2 = v; i2 = i; v = y; i = n;
    } else if (better(y, n, v2, i2)) {
      v2 = y; i2 = n;
    }
  }
  // argmax: the value joins the largest only (for per-lane scans whose
  // lists are merged into top-2 lists afterwards)
  __device__ void add1(float y, int n) {
    if (better(y, n, v, i)) { v = y; i = n; }
  }
  // log-sum-exp state (ov, os) of other features
  __device__ void merge(bool lse, float ov, int oi, float os) {
    if (lse) {
      if (ov > v) { s = s * expf(v - ov) + os; v = ov; }
      else if (ov != -INFINITY) s += os * expf(ov - v);
    } else {
      add(false, ov, oi);
    }
  }
  // top-2 list (ov, oi), (ov2, oi2) of other features
  __device__ void merge2(float ov, int oi, float ov2, int oi2) {
    if (better(ov, oi, v, i)) {
      if (better(v, i, ov2, oi2)) { v2 = v; i2 = i; } else { v2 = ov2; i2 = oi2; }
      v = ov; i = oi;
    } else if (better(ov, oi, v2, i2)) {
      v2 = ov; i2 = oi;
    }
  }
  __device__ u32x4 pack2() const { return u32x4{__float_as_uint(v), (uint32_t)i, __float_as_uint(v2), (uint32_t)i2}; }
  __device__ void merge_packed(const u32x4& t) {
    merge2(__uint_as_float(t[0]), (int)t[1], __uint_as_float(t[2]), (int)t[3]);
  }
  // lanes 16 and 32 apart (the four lane groups that hold one row)
  __device__ void merge_groups(bool lse) {
    for (int o = 16; o < 64; o <<= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oi = __shfl_xor(i, o, 64);
      if (lse) {
        merge(true, ov, oi, __shfl_xor(s, o, 64));
      } else {
        const float ov2 = __shfl_xor(v2, o, 64);
        const int oi2 = __shfl_xor(i2, o, 64);
        merge2(ov, oi, ov2, oi2);
      }
    }
  }
};

template <typename S>
__device__ __forceinline__ void epi_store(const Epi& e, int m, int n, float y, float y2) {
  switch (e.kind) {
    case EPI_FC: {
      if (e.rejected && e.rejected[m]) return;
      const int id = e.ids[m];
      float emb = 0.f;
      if (id >= 0 && id < e.embed_rows)
        emb = Storage<S>::to_f32(reinterpret_cast<const S*>(e.embed)[(int64_t)id * e.ld_out + n]);
      e.out_f32[(int64_t)m * e.ld_out + n] = y + emb;
      break;
    }
    case EPI_QKV: {
      if (n < e.q_cols) {
        reinterpret_cast<S*>(e.out_s)[(int64_t)m * e.q_cols + n] = Storage<S>::from_f32(y);
      } else {
        const int slot = e.slots[m];
        if (slot < 0 || slot >= e.kv_rows) return;
        int c = n - e.q_cols;
        S* dst = reinterpret_cast<S*>(c < e.kv_cols ? e.k_cache : e.v_cache);
        if (c >= e.kv_cols) c -= e.kv_cols;
        dst[(int64_t)slot * e.kv_cols + c] = Storage<S>::from_f32(y);
      }
      break;
    }
    case EPI_RESID: {
      const int rr = e.res_rows ? e.res_rows[m] : m;
      e.out_f32[(int64_t)m * e.ld_out + n] = y + e.res[(int64_t)rr * e.ld_res + n];
      break;
    }
    case EPI_SWIGLU: {
      const float si = y / (1.0f + __expf(-y));
      const float h = si * y2;
      const S hs = Storage<S>::from_f32(h);
      reinterpret_cast<S*>(e.out_s)[(int64_t)m * e.ld_out + n] = hs;
      if (e.out_s_lo) reinterpret_cast<S*>(e.out_s_lo)[(int64_t)m * e.ld_out + n] = Storage<S>::from_f32(h - Storage<S>::to_f32(hs));
      break;
    }
    default:
      break;
  }
}

}  // namespace pe
