// Parallel-draft / COD masked GQA attention on gfx950.
//
// Visibility ("[RFC]: Add random anchor for p-eagle first position",
// Motivation; "P-EAGLE: parallel speculative decoding in vLLM", "Training on
// long sequences"): a query sees a prefix of its segment's rows (the original
// positions <= its chain start, or in decode the region rows up to its own
// position) plus its own chain rows, found by walking parent links.  The
// mask is evaluated from these indices per score element; no mask tensor
// exists, and key tiles beyond the largest prefix of a workgroup's queries
// are never touched.
//
// Work unit: one workgroup = one kv head x up to 64 query columns, a column
// being a (query, q-head) pair of that kv head's GQA group (64/G queries of
// G heads), optionally restricted to one split of the prefix range (decode
// shapes: few queries, long regions).  4 waves x 16 columns.  Per 64-key tile:
//   * keys are staged in LDS: K row-major, V transposed (V^T[dh][key]) so
//     that both MFMA operands read contiguous 8/16-byte runs;
//   * S^T = K Q^T on the matrix cores (A = K rows, B = Q columns, Q kept in
//     registers for the whole kernel), giving lane (r, g) the scores of
//     column r for keys 4g..4g+3 of each 16-key block;
//   * masking, online softmax in fp32 (exp2 with the log2(e)-folded scale);
//     each lane's column is fixed, so the rescale of the running output is
//     a per-lane scalar;
//   * O^T += V^T P^T on the matrix cores (P rounded to the operand type).
// Chain rows are gathered into extra tiles whose mask is "owner == column's
// query"; a row shared by several chains simply appears once per owner.
// Splits write unnormalised partials (m, l, O); a combine kernel merges them.
#include <math.h>
#include "kernels.h"

namespace pe {

constexpr int KT = 64;     // keys per tile
constexpr int MAXD = 16;   // deepest chain walked per query

template <typename S, int DH, bool DBG>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p, int G, int tps) {
  constexpr int CH = Storage<S>::CH;
  constexpr int STEP = 4 * CH;
  constexpr int NST = DH / STEP;
  constexpr int NMB = DH / 16;
  constexpr int DC = DH / CH;                    // 16-byte chunks per head row
  constexpr int KPITCH = DC + 1;                 // Ks row pitch, 16-byte units
  constexpr int VPB = KT * (int)sizeof(S) + 16;  // Vt row pitch, bytes
  __shared__ u32x4 Ks[KT * KPITCH];
  __shared__ __attribute__((aligned(16))) char Vt[DH * VPB];
  __shared__ int s_keyrow[KT];
  __shared__ int s_start[64], s_depth[64], s_self[64], s_cnt[64], s_off[65];
  __shared__ int s_anc_row[64 * MAXD], s_anc_own[64 * MAXD];
  __shared__ int s_maxstart;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int Hkv = p.Hkv, Hq = p.Hq;
  const int QPW = 64 / G;

  int bid = blockIdx.x;
  const int kvh = bid % Hkv;
  bid /= Hkv;
  const int sp = bid % p.n_splits;
  bid /= p.n_splits;
  const int lin = p.num_seg * tps - 1 - bid;  // later (longer) tiles first
  const int seg = lin / tps, tile = lin % tps;
  const int qbase = seg * p.q_per_seg + tile * QPW;
  const int nq = min(QPW, p.q_per_seg - tile * QPW);

  // ---- per-query metadata and chain walk
  if (tid < 64) {
    int st = -1, dp = 0, self = -1;
    if (tid < nq) {
      const int qi = qbase + tid;
      const int mi = (p.meta_by_row && p.q_rows) ? p.q_rows[qi] : qi;
      st = p.q_start[mi];
      if (p.q_depth) {
        dp = min(max(p.q_depth[mi], 0), MAXD);
        self = p.q_self_row[mi];
      }
    }
    int cnt = 0, row = self;
    for (int e = 0; e < dp; ++e) {
      if (row < 0 || row >= p.num_kv_rows) break;
      ++cnt;
      row = p.kv_parent[row];
    }
    s_start[tid] = st;
    s_depth[tid] = cnt;
    s_self[tid] = self;
    s_cnt[tid] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, mx = -1;
    for (int i = 0; i < 64; ++i) {
      s_off[i] = o;
      o += s_cnt[i];
      mx = max(mx, s_start[i]);
    }
    s_off[64] = o;
    s_maxstart = mx;
  }
  __syncthreads();
  if (tid < nq && s_cnt[tid] > 0) {
    int row = s_self[tid];
    const int o = s_off[tid];
    for (int e = 0; e < s_cnt[tid]; ++e) {
      s_anc_row[o + e] = row;
      s_anc_own[o + e] = tid;
      row = p.kv_parent[row];
    }
  }
  __syncthreads();
  const int n_anc = (sp == 0) ? s_off[64] : 0;
  const int max_start = s_maxstart;
  const int seg_base = p.seg_kv_base[seg];

  // ---- this split's prefix range [kbeg, kend]
  const int kbeg = sp * p.split_len;
  const int kend = (sp == p.n_splits - 1) ? max_start : min(max_start, kbeg + p.split_len - 1);
  const int n_pref = (kend >= kbeg) ? (kend - kbeg + KT) / KT : 0;
  const int n_tiles = n_pref + (n_anc + KT - 1) / KT;

  // ---- this lane's column
  const int col = wave * 16 + r;
  const int cq = col / G, cg = col % G;
  const bool cact = cq < nq;
  const int cstart = cact ? s_start[cq] : -1;
  const int h = kvh * G + cg;

  const S* Q = reinterpret_cast<const S*>(p.q);
  const S* Kg = reinterpret_cast<const S*>(p.k);
  const S* Vg = reinterpret_cast<const S*>(p.v);
  u32x4 qreg[NST];
  {
    int qrow = -1;
    if (cact) qrow = p.q_rows ? p.q_rows[qbase + cq] : qbase + cq;
#pragma unroll
    for (int st = 0; st < NST; ++st)
      qreg[st] = (qrow >= 0) ? ld16(Q + (int64_t)qrow * p.q_stride + (int64_t)h * DH + st * STEP + g * CH)
                             : u32x4{0u, 0u, 0u, 0u};
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  int64_t dcnt = 0;
  uint64_t dhsh = 0;
  const float sl2 = p.scale_log2;

  for (int it = 0; it < n_tiles; ++it) {
    const bool anc = it >= n_pref;
    const int k0 = anc ? (it - n_pref) * KT : kbeg + it * KT;
    if (tid < KT) {
      int row = -1;
      if (anc) {
        const int ai = k0 + tid;
        if (ai < n_anc) row = s_anc_row[ai];
      } else {
        const int pos = k0 + tid;
        if (pos <= kend) row = seg_base + pos;
      }
      if (row < 0 || row >= p.num_kv_rows) row = -1;
      s_keyrow[tid] = row;
    }
    __syncthreads();
    // K tile, row-major
    for (int c = tid; c < KT * DC; c += 256) {
      const int key = c / DC, ch = c % DC;
      const int row = s_keyrow[key];
      Ks[key * KPITCH + ch] = (row >= 0) ? ld16(Kg + ((int64_t)row * Hkv + kvh) * DH + ch * CH) : u32x4{0u, 0u, 0u, 0u};
    }
    // V tile, transposed: each task moves 4 keys x CH head dims
    for (int t = tid; t < 16 * DC; t += 256) {
      const int kg = t & 15, dc = t >> 4;
      u32x4 v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = s_keyrow[kg * 4 + i];
        v4[i] = (row >= 0) ? ld16(Vg + ((int64_t)row * Hkv + kvh) * DH + dc * CH) : u32x4{0u, 0u, 0u, 0u};
      }
      if constexpr (sizeof(S) == 2) {
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          const int sh = 16 * (e & 1);
          const uint32_t a0 = (v4[0][e >> 1] >> sh) & 0xffffu, a1 = (v4[1][e >> 1] >> sh) & 0xffffu;
          const uint32_t a2 = (v4[2][e >> 1] >> sh) & 0xffffu, a3 = (v4[3][e >> 1] >> sh) & 0xffffu;
          u32x2 w = {a0 | (a1 << 16), a2 | (a3 << 16)};
          *reinterpret_cast<u32x2*>(Vt + (dc * CH + e) * VPB + kg * 8) = w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          u32x4 w = {v4[0][e], v4[1][e], v4[2][e], v4[3][e]};
          *reinterpret_cast<u32x4*>(Vt + (dc * CH + e) * VPB + kg * 16) = w;
        }
      }
    }
    __syncthreads();

    // S^T = K Q^T
    f32x4 sacc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NST; ++st) mma16(sacc[b], Ks[(16 * b + r) * KPITCH + st * 4 + g], qreg[st], S());
    }
    // mask + online softmax
    float sv[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = 16 * b + 4 * g + j;
        const int row = s_keyrow[kk];
        bool vis;
        if (anc) vis = cact && row >= 0 && s_anc_own[k0 + kk] == cq;
        else vis = row >= 0 && (k0 + kk) <= cstart;
        const float s = vis ? sacc[b][j] : -INFINITY;
        sv[4 * b + j] = s;
        tmax = fmaxf(tmax, s);
        if constexpr (DBG) {
          if (vis) { ++dcnt; dhsh += mix64((uint64_t)(uint32_t)row); }
        }
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    float pv[16];
    float psum = 0.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[i] = 0.f;
    } else {
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
      const float mb = m_new * sl2;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], sl2, -mb));
        psum += pv[i];
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int i = 0; i < NMB; ++i) acc[i] *= alpha;
      m_run = m_new;
    }
    // O^T += V^T P^T
    if constexpr (sizeof(S) == 2) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int b0 = 2 * pr;
        u32x4 bop = {pack_bf16x2(pv[4 * b0 + 0], pv[4 * b0 + 1]), pack_bf16x2(pv[4 * b0 + 2], pv[4 * b0 + 3]),
                     pack_bf16x2(pv[4 * b0 + 4], pv[4 * b0 + 5]), pack_bf16x2(pv[4 * b0 + 6], pv[4 * b0 + 7])};
#pragma unroll
        for (int mbk = 0; mbk < NMB; ++mbk) {
          const char* vrow = Vt + (16 * mbk + r) * VPB;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + (32 * pr + 4 * g) * 2);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (32 * pr + 16 + 4 * g) * 2);
          u32x4 aop = {lo.x, lo.y, hi.x, hi.y};
          mma16(acc[mbk], aop, bop, S());
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        u32x4 bop = {__float_as_uint(pv[4 * b]), __float_as_uint(pv[4 * b + 1]), __float_as_uint(pv[4 * b + 2]),
                     __float_as_uint(pv[4 * b + 3])};
#pragma unroll
        for (int mbk = 0; mbk < NMB; ++mbk) {
          const u32x4 aop = *reinterpret_cast<const u32x4*>(Vt + (16 * mbk + r) * VPB + (16 * b + 4 * g) * 4);
          mma16(acc[mbk], aop, bop, S());
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue
  const int qo = qbase + cq;
  if (p.n_splits == 1) {
    if (cact) {
      const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
      S* o = reinterpret_cast<S*>(p.out) + ((int64_t)qo * Hq + h) * DH;
#pragma unroll
      for (int mbk = 0; mbk < NMB; ++mbk) {
        const int dh = 16 * mbk + 4 * g;
        if constexpr (sizeof(S) == 2) {
          u32x2 w = {pack_bf16x2(acc[mbk][0] * inv, acc[mbk][1] * inv), pack_bf16x2(acc[mbk][2] * inv, acc[mbk][3] * inv)};
          *reinterpret_cast<u32x2*>(o + dh) = w;
        } else {
          f32x4 w = acc[mbk] * inv;
          *reinterpret_cast<f32x4*>(o + dh) = w;
        }
      }
      if (p.lse && g == 0) p.lse[(int64_t)qo * Hq + h] = l_run > 0.f ? m_run * p.scale + logf(l_run) : -INFINITY;
    }
  } else if (cact) {
    const int64_t qh = ((int64_t)sp * p.num_q + qo) * Hq + h;
#pragma unroll
    for (int mbk = 0; mbk < NMB; ++mbk)
      *reinterpret_cast<f32x4*>(p.part_o + qh * DH + 16 * mbk + 4 * g) = acc[mbk];
    if (g == 0) {
      p.part_ml[qh * 2 + 0] = m_run;
      p.part_ml[qh * 2 + 1] = l_run;
    }
  }
  if constexpr (DBG) {
    for (int o = 16; o < 64; o <<= 1) {
      dcnt += __shfl_xor(dcnt, o, 64);
      dhsh += __shfl_xor(dhsh, o, 64);
    }
    if (cact && cg == 0 && g == 0) {
      if (p.n_splits == 1) {
        p.dbg_count[(int64_t)qo * Hkv + kvh] = dcnt;
        p.dbg_hash[(int64_t)qo * Hkv + kvh] = dhsh;
      } else {
        const int64_t qk = ((int64_t)sp * p.num_q + qo) * Hkv + kvh;
        p.part_dbg[qk * 2 + 0] = (uint64_t)dcnt;
        p.part_dbg[qk * 2 + 1] = dhsh;
      }
    }
  }
}

// Merge of split partials, one wave per (query, head), lane s = split s:
// O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^((m_s - M) * scale * log2 e), M = max_s m_s.
template <typename S, int DH>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t qh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nqh = (int64_t)p.num_q * p.Hq;
  const int ns = p.n_splits;  // <= 64
  const float sl2 = p.scale_log2;
  if (qh < nqh) {
    float m = -INFINITY, l = 0.f;
    if (lane < ns) {
      m = p.part_ml[((int64_t)lane * nqh + qh) * 2];
      l = p.part_ml[((int64_t)lane * nqh + qh) * 2 + 1];
    }
    float M = m;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float w = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - M) * sl2);
    const float L = wave_sum(w * l);
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    for (int dh = lane; dh < DH; dh += 64) {
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
      int s = 0;
      for (; s + 4 <= ns; s += 4) {
        o0 += __shfl(w, s, 64) * p.part_o[((int64_t)s * nqh + qh) * DH + dh];
        o1 += __shfl(w, s + 1, 64) * p.part_o[((int64_t)(s + 1) * nqh + qh) * DH + dh];
        o2 += __shfl(w, s + 2, 64) * p.part_o[((int64_t)(s + 2) * nqh + qh) * DH + dh];
        o3 += __shfl(w, s + 3, 64) * p.part_o[((int64_t)(s + 3) * nqh + qh) * DH + dh];
      }
      for (; s < ns; ++s) o0 += __shfl(w, s, 64) * p.part_o[((int64_t)s * nqh + qh) * DH + dh];
      reinterpret_cast<S*>(p.out)[qh * DH + dh] = Storage<S>::from_f32(((o0 + o1) + (o2 + o3)) * inv);
    }
    if (lane == 0 && p.lse) p.lse[qh] = L > 0.f ? M * p.scale + logf(L) : -INFINITY;
  }
  if (p.dbg_count) {
    const int64_t nqk = (int64_t)p.num_q * p.Hkv;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx < nqk) {
      uint64_t c = 0, h = 0;
      for (int s = 0; s < ns; ++s) {
        c += p.part_dbg[((int64_t)s * nqk + idx) * 2];
        h += p.part_dbg[((int64_t)s * nqk + idx) * 2 + 1];
      }
      p.dbg_count[idx] = (int64_t)c;
      p.dbg_hash[idx] = h;
    }
  }
}

template <typename S, int DH>
static void launch_attn_t(const AttnParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  const int QPW = 64 / G;
  const int tps = (p.q_per_seg + QPW - 1) / QPW;
  const int grid = p.num_seg * tps * p.n_splits * p.Hkv;
  if (p.dbg_count) hipLaunchKernelGGL((attn_kernel<S, DH, true>), dim3(grid), dim3(256), 0, s, p, G, tps);
  else hipLaunchKernelGGL((attn_kernel<S, DH, false>), dim3(grid), dim3(256), 0, s, p, G, tps);
  if (p.n_splits > 1) {
    const int64_t nqh = (int64_t)p.num_q * p.Hq;
    const int64_t nqk = (int64_t)p.num_q * p.Hkv;
    int64_t blocks = (nqh + 3) / 4;
    if (p.dbg_count && (nqk + 255) / 256 > blocks) blocks = (nqk + 255) / 256;
    hipLaunchKernelGGL((attn_combine_kernel<S, DH>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  }
}

void launch_attention(const AttnParams& p, int bf16, int head_dim, hipStream_t s) {
  if (bf16) {
    if (head_dim == 64) launch_attn_t<uint16_t, 64>(p, s); else launch_attn_t<uint16_t, 128>(p, s);
  } else {
    if (head_dim == 64) launch_attn_t<float, 64>(p, s); else launch_attn_t<float, 128>(p, s);
  }
}

}  // namespace pe
