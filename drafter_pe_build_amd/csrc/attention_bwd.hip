// Backward of the parallel-draft / COD masked GQA attention on gfx950, for the
// depth-major training layout, bf16 operands and f32 gradients.
//
// "P-EAGLE: parallel speculative decoding in vLLM", "Training on long
// sequences": the sequence partition splits the N*K positions into chunks of
// queries while every attention dependency across chunk boundaries is kept,
// so a chunk's queries also produce key and value gradients for rows of
// earlier chunks.  Here a call takes the queries [q_begin, q_end), writes
// their dQ and adds their contributions to dK and dV of every row.
//
// With the forward's log-sum-exp, P = exp(s - lse) is recomputed exactly (no
// running maximum), dP = dO . v, dS = P (dP - delta) with delta = rowsum(dO o O)
// per (query, head), and
//   dQ = scale dS K,  dK += scale dS^T Q,  dV += P^T dO.
// Layout facts used to enumerate work (no mask tensor, no atomics):
//   * group 0 holds the original positions (row = start); group e >= 1 the
//     depth-e chain rows sorted by start, so in every group the rows with
//     starts in an interval are contiguous;
//   * a query (s, d) sees the group-0 rows with start <= s and the rows
//     (s, e) for 1 <= e <= d.
// dQ kernel: one workgroup = 128 (query, head) columns of one kv head (4
// waves x 32), walking the key tiles its queries can see: group 0 up to the
// largest start, and each deeper group's rows whose starts lie in the
// queries' start range.  dK/dV kernel: one workgroup = 64 key rows of one
// group and one kv head (a wave per 16 keys, K and V in registers), walking
// the query tiles that can see them: for a group-0 tile the rows of every
// group with start >= the tile's first start, for a chain tile the rows of
// the groups at least as deep whose starts lie in the tile's start range;
// the query tiles are shared out over BSPL workgroups (the first key tiles
// are seen by every query), whose partial sums a reduce kernel adds in a
// fixed order.  Each workgroup owns its outputs, so results do not depend on
// timing.
#include <math.h>
#include <type_traits>
#include "kernels.h"

typedef short short4_t __attribute__((ext_vector_type(4)));

namespace pe {

namespace {

constexpr int BKT = 64;    // keys per tile (dQ) / per workgroup (dK, dV)
constexpr int BCOL = 128;  // (query, head) columns per tile (dQ)
constexpr int BCOLK = 64;  // (query, head) columns per tile (dK, dV)
constexpr int BMAXG = 16;  // groups a layout may have
constexpr int BSPL = 4;    // dK/dV workgroups per key tile, each a share of its query tiles

// First row in [lo, hi) whose start is >= s (GT: > s), or hi if there is
// none; rows sorted by start.  All 64 lanes of the calling wave take part
// (wave-uniform arguments): each round the lanes read the starts of 64
// evenly spaced rows and the range shrinks to the gap between the last row
// below the bound and the first one at or above it, so 4,096 rows take two
// dependent reads instead of twelve.
template <bool GT>
__device__ int find_row_wave(const int32_t* start, int lo, int hi, int s) {
  const int lane = threadIdx.x & 63;
  while (hi > lo) {
    const int n = hi - lo;
    if (n <= 64) {
      const bool below = lane < n && (GT ? start[lo + lane] <= s : start[lo + lane] < s);
      return lo + __popcll(__ballot(below));
    }
    // probe i(l) = lo + n (l + 1) / 65, l = 0..63: increasing, inside [lo, hi)
    auto probe = [&](int l) { return lo + (int)((int64_t)n * (l + 1) / 65); };
    const int i = probe(lane);
    const bool below = GT ? start[i] <= s : start[i] < s;
    const int c = __popcll(__ballot(below));  // the rows below the bound are a prefix
    const int nlo = c > 0 ? probe(c - 1) + 1 : lo;
    const int nhi = c < 64 ? probe(c) : hi;
    if (c < 64 && nhi == nlo) return nhi;  // the first probe at or above the bound is the answer
    lo = nlo;
    hi = nhi;
  }
  return lo;
}

// Rows of group e, clamped into [0, T] (a malformed layout cannot send a
// search or a load outside the arrays).
__device__ __forceinline__ void group_rows(const AttnBwdParams& p, int e, int& g0, int& g1) {
  g0 = min(max(p.group_off[e], 0), p.T);
  g1 = min(max(p.group_off[e + 1], g0), p.T);
}

__device__ __forceinline__ bool sees(int qs, int qd, int ks, int kd) {
  return kd == 0 ? ks <= qs : (kd >= 1 && ks == qs && kd <= qd);
}

__device__ __forceinline__ u32x4 tr_pair(const char* p, int pitch) {
  typedef __attribute__((address_space(3))) short4_t lds_s4;
  const auto lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
  const auto hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p + 16 * pitch));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo4), h2 = __builtin_bit_cast(u32x2, hi4);
  return u32x4{l2.x, l2.y, h2.x, h2.y};
}

}  // namespace

// delta[i][h] = sum_d dO[q_begin + i][h][d] O[q_begin + i][h][d]; DH / 8 lanes
// per (query, head) row, 16 bytes of each tensor per lane, summed across the
// row's lanes in a fixed order.
template <int DH>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(AttnBwdParams p) {
  constexpr int LPR = DH / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t w = i / LPR;
  const int c = (int)(i % LPR);
  const int64_t nqh = (int64_t)(p.q_end - p.q_begin) * p.Hq;
  float acc = 0.f;
  if (w < nqh) {
    const int64_t off = ((int64_t)p.q_begin * p.Hq + w) * DH + c * 8;  // (query, head) row of out / dout
    const u32x4 o = ld16(reinterpret_cast<const uint16_t*>(p.out) + off);
    const u32x4 d = ld16(reinterpret_cast<const uint16_t*>(p.dout) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf2f((uint16_t)(o[e] & 0xffffu)), bf2f((uint16_t)(d[e] & 0xffffu)), acc);
      acc = fmaf(bf2f((uint16_t)(o[e] >> 16)), bf2f((uint16_t)(d[e] >> 16)), acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (w < nqh && c == 0) p.delta[w] = acc;
}

// ---------------------------------------------------------------------------
// dQ: columns (query, head) of one kv head; per key tile S^T = K Q^T and
// dP^T = V dO^T (B operands in registers), dQ^T += K^T dS^T (K^T read
// transposed from the same LDS copy of K, dS^T from the score registers).
// Key tiles are double-buffered in LDS and copied there straight from global
// memory one tile ahead, with one barrier per tile.
template <int DH>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(AttnBwdParams p, int G, int n_qtiles) {
  constexpr int NST = DH / 32;                  // 32-dim contraction steps
  constexpr int NMB = DH / 16;                  // 16-dim output blocks
  constexpr int KP = DH * 2 + 16;               // V row pitch (row reads)
  constexpr int TP = DH * 2 + 32;               // K row pitch (row and transposed reads)
  constexpr int CB = 2;                         // 16-column blocks per wave
  // two tile buffers: K once, at the pitch of the transposed reads (its row
  // reads use the same copy), V at the row pitch, and the labels
  __shared__ __attribute__((aligned(16))) char Ks[2][BKT * TP];
  __shared__ __attribute__((aligned(16))) char Vs[2][BKT * KP];
  __shared__ int s_ks[2][BKT], s_kd[2][BKT];
  __shared__ int s_rng[2 * BMAXG], s_red[12], s_tp[BMAXG + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.x % p.Hkv, qt = blockIdx.x / p.Hkv;
  if (qt >= n_qtiles) return;
  const int QPW = BCOL / G;
  const int qa = p.q_begin + qt * QPW;
  const int qb = min(qa + QPW, p.q_end);
  const float sl2 = p.scale * 1.4426950408889634f;

  // this lane's columns
  int cqi[CB], ch[CB], cs[CB], cd[CB];
  float clse2[CB], cdel[CB];
  u32x4 qreg[CB][NST], dreg[CB][NST];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int col = wave * 32 + cb * 16 + r;
    const int qi = qa + col / G;
    const int h = kvh * G + col % G;
    const bool act = qi < qb;
    cqi[cb] = act ? qi : -1;
    ch[cb] = h;
    cs[cb] = act ? p.start[qi] : -1;
    cd[cb] = act ? p.depth[qi] : -1;
    clse2[cb] = act ? p.lse[(int64_t)qi * p.Hq + h] * 1.4426950408889634f : 0.f;
    cdel[cb] = act ? p.delta[(int64_t)(qi - p.q_begin) * p.Hq + h] : 0.f;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)(act ? qi : 0) * p.Hq + h) * DH;
    const uint16_t* drow = reinterpret_cast<const uint16_t*>(p.dout) + ((int64_t)(act ? qi : p.q_begin) * p.Hq + h) * DH;
#pragma unroll
    for (int t = 0; t < NST; ++t) {
      qreg[cb][t] = act ? ld16(qrow + t * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
      dreg[cb][t] = act ? ld16(drow + t * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // key ranges: group 0 rows [0, max start], then per deeper group the rows
  // whose starts lie in [min start, max start] of the tile's queries
  int mn = 0x7fffffff, mx = -1, md = 0;
  if (tid < QPW && qa + tid < qb) {
    mn = p.start[qa + tid];
    mx = mn;
    md = p.depth[qa + tid];
  }
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, __shfl_xor(mn, o, 64));
    mx = max(mx, __shfl_xor(mx, o, 64));
    md = max(md, __shfl_xor(md, o, 64));
  }
  if (lane == 0) { s_red[wave] = mn; s_red[4 + wave] = mx; s_red[8 + wave] = md; }
  __syncthreads();
  const int qs_min = min(min(s_red[0], s_red[1]), min(s_red[2], s_red[3]));
  const int qs_max = max(max(s_red[4], s_red[5]), max(s_red[6], s_red[7]));
  const int qd_max = min(max(max(s_red[8], s_red[9]), max(s_red[10], s_red[11])), p.D - 1);
  // range of group e, one wave per group (e = wave, wave + 4, ...)
  for (int e = wave; e < BMAXG; e += 4) {
    int a = 0, b = 0;
    if (qs_max >= 0) {
      if (e == 0) { a = 0; b = min(qs_max + 1, p.N); }
      else if (e <= qd_max) {
        int g0, g1;
        group_rows(p, e, g0, g1);
        a = find_row_wave<false>(p.start, g0, g1, qs_min);
        b = find_row_wave<true>(p.start, a, g1, qs_max);
      }
    }
    if (lane == 0) {
      s_rng[2 * e] = a;
      s_rng[2 * e + 1] = b;
    }
  }
  __syncthreads();

  f32x4 acc[CB][NMB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < NMB; ++i) acc[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the key tiles in one list: range e's tiles follow range e - 1's
  if (tid == 0) {
    int tot = 0;
    for (int e = 0; e < BMAXG; ++e) {
      s_tp[e] = tot;
      if (e <= qd_max) tot += max(0, s_rng[2 * e + 1] - s_rng[2 * e] + BKT - 1) / BKT;
    }
    s_tp[BMAXG] = tot;
  }
  __syncthreads();
  const int ntile = s_tp[BMAXG];
  auto tile_at = [&](int tt, int& k0, int& nk, int& e) {
    e = 0;
    while (e < qd_max && tt >= s_tp[e + 1]) ++e;
    k0 = s_rng[2 * e] + (tt - s_tp[e]) * BKT;
    nk = min(BKT, s_rng[2 * e + 1] - k0);
  };
  // The next tile is copied from global memory straight into the other LDS
  // buffer (that buffer's previous tile was released by the barrier that ends
  // every tile) while this one is multiplied: one 64-lane copy fills 64
  // consecutive 16-byte slots of the padded layout (lane l -> slot l), the
  // copies spread round-robin over the waves; slots of row padding load
  // chunk 0 of their row (never read back), and keys past a range repeat the
  // range's first row (masked out).  The labels go through registers.
  const int64_t rstride = (int64_t)p.Hkv * DH;
  constexpr int KSL = TP / 16, VSL = KP / 16;                    // slots per padded row
  constexpr int NKC = BKT * KSL / 64, NVC = BKT * VSL / 64;      // 1 KB copies per tile
  static_assert(NKC * 64 == BKT * KSL && NVC * 64 == BKT * VSL, "whole copies per tile");
  constexpr int NCP = NKC + NVC, NCW = (NCP + 3) / 4;           // copies in all, per wave
  // key and chunk of copy q of this lane
  auto cslot = [&](int q, int& key, int& ck) {
    const int j = wave + 4 * q;
    const bool isv = j >= NKC;
    const int sl = isv ? VSL : KSL;
    const int slot = (isv ? j - NKC : j) * 64 + lane;
    key = slot / sl;
    ck = slot % sl < DH / 8 ? slot % sl : 0;
  };
  uint32_t coff[NCW];  // element offset of copy q within a tile of 64 rows
#pragma unroll
  for (int q = 0; q < NCW; ++q) {
    int key, ck;
    cslot(q, key, ck);
    coff[q] = (uint32_t)key * (uint32_t)rstride + (uint32_t)(ck * 8);
  }
  int pls = -1, pld = -1, pfull = 0;
  auto prefetch = [&](int tt, int b) {
    int k0, nk, e;
    tile_at(tt, k0, nk, e);
    // every query of the workgroup sees the whole tile: 64 group-0 keys whose
    // largest start is at most the smallest query start
    pfull = __builtin_amdgcn_readfirstlane(e == 0 && nk == BKT && p.start[k0 + BKT - 1] <= qs_min);
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)k0 * rstride + kvh * DH;
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)k0 * rstride + kvh * DH;
#pragma unroll
    for (int q = 0; q < NCW; ++q) {
      const int j = wave + 4 * q;
      if (j >= NCP) break;
      const bool isv = j >= NKC;
      uint32_t off = coff[q];
      if (nk < BKT) {
        int key, ck;
        cslot(q, key, ck);
        off = (uint32_t)(key < nk ? key : 0) * (uint32_t)rstride + (uint32_t)(ck * 8);
      }
      char* dst = isv ? Vs[b] + (j - NKC) * 1024 : Ks[b] + j * 1024;
      copy16_to_lds((isv ? vb : kb) + off, dst);
    }
    if (tid < BKT) {
      pls = tid < nk ? p.start[k0 + tid] : -1;
      pld = tid < nk ? p.depth[k0 + tid] : -1;
    }
  };
  auto store_labels = [&](int b) {
    if (tid < BKT) {
      s_ks[b][tid] = pls;
      s_kd[b][tid] = pld;
    }
  };

  // per-half steps (a half is 32 keys; this lane holds keys 32 h + 16 bb + 4 g + j
  // of its two columns)
  typedef f32x4 HalfS[CB][2];
  typedef u32x4 HalfB[CB];
  // S^T = K Q^T and dP^T = V dO^T (Q, dO in registers)
  auto s_half = [&](const char* Kb, const char* Vb, int h, HalfS& sacc, HalfS& pacc) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) sacc[cb][0] = sacc[cb][1] = pacc[cb][0] = pacc[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int t = 0; t < NST; ++t) {
        const int kr = 16 * (2 * h + bb) + r;
        const u32x4 ka = *reinterpret_cast<const u32x4*>(Kb + kr * TP + (4 * t + g) * 16);
        const u32x4 va = *reinterpret_cast<const u32x4*>(Vb + kr * KP + (4 * t + g) * 16);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          mma16(sacc[cb][bb], ka, qreg[cb][t], uint16_t());
          mma16(pacc[cb][bb], va, dreg[cb][t], uint16_t());
        }
      }
  };
  // scores of keys a column does not see become -inf (tiles some column sees
  // only in part)
  auto mask_half = [&](int b, int h, HalfS& sacc) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = 16 * (2 * h + bb) + 4 * g + j;
        const int ks = s_ks[b][kk], kd = s_kd[b][kk];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          sacc[cb][bb][j] = sees(cs[cb], cd[cb], ks, kd) ? sacc[cb][bb][j] : -INFINITY;
      }
  };
  // dS^T = P^T (dP^T - delta) with P from the forward's log-sum-exp, packed as
  // the B operand (inactive columns have zero Q and dO rows: dS = 0)
  auto ds_half = [&](const HalfS& sacc, const HalfS& pacc, HalfB& bop) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int bb = i >> 2, j = i & 3;
        const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[cb][bb][j], sl2, -clse2[cb]));
        ds[i] = pe * (pacc[cb][bb][j] - cdel[cb]);
      }
      bop[cb] = u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                      pack_bf16x2(ds[6], ds[7])};
    }
  };
  // dQ^T += K^T dS^T: lane r receives dim 16 mb + r of keys 32 h + 4 g + c and + 16
  auto dq_half = [&](const char* Kb, int h, const HalfB& bop) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const u32x4 aop = tr_pair(Kb + (32 * h + 4 * g + (r >> 2)) * TP + (16 * mb + 4 * (r & 3)) * 2, TP);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) mma16(acc[cb][mb], aop, bop[cb], uint16_t());
    }
  };
  // Per tile: copy next | per half S, mask, dS, dQ | wait for the copies, barrier.
  if (ntile > 0) {
    prefetch(0, 0);
    store_labels(0);
  }
  bool full = pfull;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of the first tile
  __syncthreads();
  for (int tt = 0; tt < ntile; ++tt) {
    const int b = tt & 1;
    const bool more = tt + 1 < ntile;
    if (more) prefetch(tt + 1, b ^ 1);
    const char* Kb = Ks[b];
    const char* Vb = Vs[b];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      HalfS s0, p0;
      HalfB b0;
      s_half(Kb, Vb, h, s0, p0);
      if (!full) mask_half(b, h, s0);
      ds_half(s0, p0, b0);
      dq_half(Kb, h, b0);
    }
    if (more) store_labels(b ^ 1);
    full = pfull;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of the next tile
    __syncthreads();  // the next tile is in place; this one's buffer is free
  }
  // dQ = scale dQ^T: lane (g, r) holds dims 16 mb + 4 g + j of its column
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if (cqi[cb] < 0) continue;
    float* dq = p.dq + ((int64_t)(cqi[cb] - p.q_begin) * p.Hq + ch[cb]) * DH;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      *reinterpret_cast<f32x4*>(dq + 16 * mb + 4 * g) = acc[cb][mb] * p.scale;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: 64 key rows of one group (a wave per 16, K and V as B operands in
// registers) against the query tiles that can see them; per tile
// S' = Q K^T, dP' = dO V^T (A operands from LDS), then dV^T += dO^T P' and
// dK^T += Q^T dS' (A operands read transposed from LDS).
template <int DH>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkv_kernel(AttnBwdParams p, int G) {
  constexpr int NST = DH / 32;
  constexpr int NMB = DH / 16;
  constexpr int PP = DH * 2 + 32;  // Q / dO row pitch (row reads and transposed reads)
  constexpr int NCB = BCOLK / 16;  // 16-column blocks of a query tile
  __shared__ __attribute__((aligned(16))) char Qs[BCOLK * PP];
  __shared__ __attribute__((aligned(16))) char Ds[BCOLK * PP];
  __shared__ __attribute__((aligned(16))) float s_lse2[BCOLK], s_del[BCOLK];
  __shared__ __attribute__((aligned(16))) int s_cs[BCOLK], s_cd[BCOLK];
  __shared__ int s_rng[2 * BMAXG], s_tile[4], s_tpre[BMAXG + 1], s_piece[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.x % p.Hkv;
  const int piece = (blockIdx.x / p.Hkv) % BSPL;
  const int kt = blockIdx.x / p.Hkv / BSPL;  // flat key-tile index over the groups
  int t = kt;
  // which group and which 64 rows of it
  if (tid == 0) {
    int e = 0, r0 = -1, r1 = -1;
    for (; e < p.D; ++e) {
      int g0, g1;
      group_rows(p, e, g0, g1);
      const int nt = (g1 - g0 + BKT - 1) / BKT;
      if (t < nt) { r0 = g0 + t * BKT; r1 = min(r0 + BKT, g1); break; }
      t -= nt;
    }
    s_tile[0] = e;
    s_tile[1] = r0;
    s_tile[2] = r1;
  }
  __syncthreads();
  const int ke = s_tile[0], kr0 = s_tile[1], kr1 = s_tile[2];
  if (kr0 < 0) return;
  const int QPW = BCOLK / G;
  const float sl2 = p.scale * 1.4426950408889634f;
  const int64_t rstride = (int64_t)p.Hkv * DH;

  // this lane's key (row kr0 + 16 wave + r) and its K, V operands
  const int key = kr0 + 16 * wave + r;
  const bool kact = key < kr1;
  const int krow = kact ? key : kr0;
  const int ks = kact ? p.start[key] : -1;
  const int kd = kact ? p.depth[key] : -1;
  u32x4 kreg[NST], vreg[NST];
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    kreg[s] = ld16(reinterpret_cast<const uint16_t*>(p.k) + (int64_t)krow * rstride + kvh * DH + s * 32 + g * 8);
    vreg[s] = ld16(reinterpret_cast<const uint16_t*>(p.v) + (int64_t)krow * rstride + kvh * DH + s * 32 + g * 8);
  }

  // query ranges per group that can see these keys, within [q_begin, q_end)
  // query rows of group e that can see these keys, one wave per group (e = wave, wave + 4, ...)
  const int s_lo = p.start[kr0], s_hi = p.start[kr1 - 1];
  for (int e = wave; e < BMAXG; e += 4) {
    int a = 0, b = 0;
    if (e < p.D && e >= ke) {
      int g0, g1;
      group_rows(p, e, g0, g1);
      a = find_row_wave<false>(p.start, g0, g1, s_lo);
      b = ke == 0 ? g1 : find_row_wave<true>(p.start, a, g1, s_hi);
      a = max(a, p.q_begin);
      b = min(b, p.q_end);
    }
    if (lane == 0) {
      s_rng[2 * e] = a;
      s_rng[2 * e + 1] = max(a, b);
    }
  }
  __syncthreads();
  // this workgroup's share of the key tile's query tiles (in group order)
  if (tid == 0) {
    int tot = 0;
    for (int d = 0; d < BMAXG; ++d) {
      s_tpre[d] = tot;
      tot += (s_rng[2 * d + 1] - s_rng[2 * d] + QPW - 1) / QPW;
    }
    s_tpre[BMAXG] = tot;
    s_piece[0] = (int)((int64_t)tot * piece / BSPL);
    s_piece[1] = (int)((int64_t)tot * (piece + 1) / BSPL);
  }
  __syncthreads();
  const int tlo = s_piece[0], thi = s_piece[1];

  f32x4 dka[NMB], dva[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i) dka[i] = dva[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the share's query tiles in one list; the next tile's Q, dO and labels are
  // loaded into registers while this one is multiplied
  auto tile_at = [&](int tt, int& qa, int& qb) {
    int d = 0;
    while (d < BMAXG - 1 && tt >= s_tpre[d + 1]) ++d;
    qa = s_rng[2 * d] + (tt - s_tpre[d]) * QPW;
    qb = min(qa + QPW, s_rng[2 * d + 1]);
  };
  // largest start of the workgroup's keys (a group's rows are sorted by start)
  const int kmax_s = p.start[kr1 - 1];
  constexpr int NPF = BCOLK * (DH / 8) / 256;
  static_assert(NPF * 256 == BCOLK * (DH / 8), "whole 16-byte chunks per thread");
  u32x4 pq[NPF], pd[NPF];
  int pcs = -1, pcd = -1, pfull = 0;
  float plse = 0.f, pdel = 0.f;
  auto prefetch = [&](int tt) {
    int qa, qb;
    tile_at(tt, qa, qb);
    // every column sees every key: group-0 keys, and the tile's first (smallest)
    // query start at least the keys' largest start
    pfull = __builtin_amdgcn_readfirstlane(ke == 0 && p.start[qa] >= kmax_s);
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int c = tid + 256 * i;
      const int col = c / (DH / 8), ck = c % (DH / 8);
      const int qi = qa + col / G, h = kvh * G + col % G;
      pq[i] = pd[i] = u32x4{0u, 0u, 0u, 0u};
      if (qi < qb) {
        pq[i] = ld16(reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)qi * p.Hq + h) * DH + ck * 8);
        pd[i] = ld16(reinterpret_cast<const uint16_t*>(p.dout) + ((int64_t)qi * p.Hq + h) * DH + ck * 8);
      }
    }
    if (tid < BCOLK) {
      const int qi = qa + tid / G, h = kvh * G + tid % G;
      const bool act = qi < qb;
      pcs = act ? p.start[qi] : -1;
      pcd = act ? p.depth[qi] : -1;
      plse = act ? p.lse[(int64_t)qi * p.Hq + h] * 1.4426950408889634f : 0.f;
      pdel = act ? p.delta[(int64_t)(qi - p.q_begin) * p.Hq + h] : 0.f;
    }
  };
  if (tlo < thi) prefetch(tlo);
  for (int tt = tlo; tt < thi; ++tt) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int c = tid + 256 * i;
      const int col = c / (DH / 8), ck = c % (DH / 8);
      *reinterpret_cast<u32x4*>(Qs + col * PP + ck * 16) = pq[i];
      *reinterpret_cast<u32x4*>(Ds + col * PP + ck * 16) = pd[i];
    }
    if (tid < BCOLK) {
      s_cs[tid] = pcs;
      s_cd[tid] = pcd;
      s_lse2[tid] = plse;
      s_del[tid] = pdel;
    }
    const bool full = pfull;
    __syncthreads();
    if (tt + 1 < thi) prefetch(tt + 1);
    {
      // S' and dP' of the column blocks: element j of lane (g, r) is column 16 cb + 4 g + j, key r
      f32x4 sacc[NCB], pacc[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) sacc[cb] = pacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int s = 0; s < NST; ++s) {
          const u32x4 qa_op = *reinterpret_cast<const u32x4*>(Qs + (16 * cb + r) * PP + (4 * s + g) * 16);
          const u32x4 da_op = *reinterpret_cast<const u32x4*>(Ds + (16 * cb + r) * PP + (4 * s + g) * 16);
          mma16(sacc[cb], qa_op, kreg[s], uint16_t());
          mma16(pacc[cb], da_op, vreg[s], uint16_t());
        }
      // P' and dS' packed per 32-column step as B operands (columns 32 s + 4 g + j, then + 16)
#pragma unroll
      for (int s = 0; s < NCB / 2; ++s) {
        // FULL skips the visibility test (padding keys only feed their own,
        // unwritten, accumulator columns; inactive columns have zero Q and dO rows)
        u32x4 pb, sb;
        auto make_ps = [&](auto full_c) {
          constexpr bool FULL = decltype(full_c)::value;
          float pv[8], ds[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int cb = 2 * s + (i >> 2), j = i & 3;
            const int col = 16 * cb + 4 * g + j;
            const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[cb][j], sl2, -s_lse2[col]));
            pv[i] = (FULL || sees(s_cs[col], s_cd[col], ks, kd)) ? e2 : 0.f;
            ds[i] = pv[i] * (pacc[cb][j] - s_del[col]);
          }
          pb = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                     pack_bf16x2(pv[6], pv[7])};
          sb = u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                     pack_bf16x2(ds[6], ds[7])};
        };
        if (full) make_ps(std::true_type{});
        else make_ps(std::false_type{});
        // lane r receives dim 16 mb + r of columns 32 s + 4 g + c and + 16
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const int off = (32 * s + 4 * g + (r >> 2)) * PP + (16 * mb + 4 * (r & 3)) * 2;
          mma16(dva[mb], tr_pair(Ds + off, PP), pb, uint16_t());
          mma16(dka[mb], tr_pair(Qs + off, PP), sb, uint16_t());
        }
      }
    }
  }
  // this share's partial dK = scale dK^T and dV = dV^T (lane (g, r) holds dims
  // 16 mb + 4 g + j of its key), summed into dk, dv by attn_bwd_dkv_reduce_kernel
  if (kact) {
    const int64_t base = (((int64_t)kt * p.Hkv + kvh) * BSPL + piece) * BKT * DH + (int64_t)(16 * wave + r) * DH;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      *reinterpret_cast<f32x4*>(p.part_k + base + 16 * mb + 4 * g) = dka[mb] * p.scale;
      *reinterpret_cast<f32x4*>(p.part_v + base + 16 * mb + 4 * g) = dva[mb];
    }
  }
}

// dk[j] += sum of the BSPL shares of row j's key tile, in share order; one
// thread per 4 dims of one (row, kv head).
template <int DH>
__global__ __launch_bounds__(256) void attn_bwd_dkv_reduce_kernel(AttnBwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)p.T * p.Hkv * (DH / 4)) return;
  const int c4 = (int)(i % (DH / 4));
  const int64_t rh = i / (DH / 4);
  const int h = (int)(rh % p.Hkv);
  const int j = (int)(rh / p.Hkv);
  int kt = 0, e = 0, g0 = 0, g1 = 0;
  for (; e < p.D; ++e) {
    group_rows(p, e, g0, g1);
    if (j < g1) break;
    kt += (g1 - g0 + BKT - 1) / BKT;
  }
  if (e == p.D || j < g0) return;  // not a row of any group
  kt += (j - g0) / BKT;
  const int kl = (j - g0) % BKT;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int pc = 0; pc < BSPL; ++pc) {
    const int64_t b = (((int64_t)kt * p.Hkv + h) * BSPL + pc) * BKT * DH + (int64_t)kl * DH + 4 * c4;
    sk += *reinterpret_cast<const f32x4*>(p.part_k + b);
    sv += *reinterpret_cast<const f32x4*>(p.part_v + b);
  }
  f32x4* pk = reinterpret_cast<f32x4*>(p.dk + ((int64_t)j * p.Hkv + h) * DH + 4 * c4);
  f32x4* pv = reinterpret_cast<f32x4*>(p.dv + ((int64_t)j * p.Hkv + h) * DH + 4 * c4);
  *pk = *pk + sk;
  *pv = *pv + sv;
}

int64_t attn_bwd_part_floats(int T, int D, int Hkv, int head_dim) {
  return ((int64_t)(T + BKT - 1) / BKT + D) * Hkv * BSPL * BKT * head_dim;
}

template <int DH>
static void launch_bwd_t(const AttnBwdParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  const int QPW = BCOL / G;
  const int nq = p.q_end - p.q_begin;
  if (nq <= 0) return;
  const int64_t nqh = (int64_t)nq * p.Hq;
  hipLaunchKernelGGL(attn_bwd_delta_kernel<DH>, dim3((unsigned)((nqh * (DH / 8) + 255) / 256)), dim3(256), 0, s, p);
  const int n_qtiles = (nq + QPW - 1) / QPW;
  hipLaunchKernelGGL(attn_bwd_dq_kernel<DH>, dim3((unsigned)(n_qtiles * p.Hkv)), dim3(256), 0, s, p, G, n_qtiles);
  // key tiles: ceil(group size / 64) per group, at most ceil(T / 64) + D in all
  const int n_ktiles = (p.T + BKT - 1) / BKT + p.D;
  hipLaunchKernelGGL(attn_bwd_dkv_kernel<DH>, dim3((unsigned)(n_ktiles * p.Hkv * BSPL)), dim3(256), 0, s, p, G);
  const int64_t nr = (int64_t)p.T * p.Hkv * (DH / 4);
  hipLaunchKernelGGL(attn_bwd_dkv_reduce_kernel<DH>, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, s, p);
}

void launch_attention_backward(const AttnBwdParams& p, int head_dim, hipStream_t s) {
  if (head_dim == 64) launch_bwd_t<64>(p, s); else launch_bwd_t<128>(p, s);
}

}  // namespace pe
