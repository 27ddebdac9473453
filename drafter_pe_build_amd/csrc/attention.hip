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
// Work unit: one workgroup = one kv head x 128 columns, a column being a
// (query, q-head) pair of that kv head's GQA group (128/G queries of G
// heads), optionally restricted to one split of the prefix range (decode
// shapes: few queries, long regions).  4 waves x 32 columns (two blocks of
// 16); two workgroups share a CU, so each SIMD interleaves two waves' matrix
// and vector work.  Per 64-key tile:
//   * the tile is staged in LDS (K row-major, V transposed as V^T[dh][key] so
//     both matrix-core operands read contiguous runs); two LDS buffers and a
//     register prefetch of the next tile leave one barrier per tile and keep
//     the next tile's HBM reads in flight while this one is multiplied;
//   * S^T = K Q^T on the matrix cores (A = K rows from LDS, B = Q columns kept
//     in registers for the whole kernel), each LDS operand feeding both
//     column blocks;
//   * masking (skipped on tiles every column of the wave sees in full) and an
//     online softmax in fp32 (exp2 with the log2(e)-folded scale); each lane's
//     column is fixed, so the rescale of the running output is per lane, and
//     the running maximum moves only when it grows by more than 2^8;
//   * O^T += V^T P^T on the matrix cores (P rounded to the operand type);
//     each lane keeps the fp32 sum of its own P, reduced over the column's
//     lanes at the end.
// A wave skips the multiplications of tiles none of its columns can see.
// Chain rows are gathered into extra tiles whose mask is "owner == column's
// query"; a row shared by several chains appears once per owner.  Splits
// write unnormalised partials (m, l, O); a combine kernel merges them.
//
// Every column's result depends only on its own key set and the fixed tile
// order (prefix tiles aligned to multiples of 64 from the split start, then
// the chain tiles), so a query gives the same bits whether it is attended in
// one launch or in a chunk of queries (for the same split length and the
// same grouping of chain tiles, i.e. chunks that start at multiples of the
// workgroup's query count).
#include <math.h>
#include <type_traits>
#include "kernels.h"

typedef short short4_t __attribute__((ext_vector_type(4)));

namespace pe {

constexpr int KT = 64;          // keys per tile
constexpr int NWAVE = 4;        // waves per workgroup
constexpr int CBLK = 2;         // 16-column blocks per wave
constexpr int QMAX = NWAVE * CBLK * 16;  // columns per workgroup
constexpr int MAXD = 16;        // deepest chain walked per query
constexpr int ANC_MAX = 1024;   // chain rows gathered per workgroup

int attn_queries_per_workgroup(int G, int) { return QMAX / G; }
int attn_max_depth(int G) { return MAXD < ANC_MAX / (QMAX / G) ? MAXD : ANC_MAX / (QMAX / G); }

// Maxima of scores, which are products or -inf and never signalling NaNs:
// the plain instructions, without the quieting copies the compiler adds to
// fmaxf operands.
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max and sum over the four lanes r, r+16, r+32, r+48 (one matrix-core
// column), with the gfx950 lane-swap instructions: after a swap of the two
// 32-lane halves (then of the 16-lane rows within them) every lane holds its
// own value and its partner's.
__device__ __forceinline__ float colgroup_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float colgroup_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two workgroups per CU, except the f32 operands at head_dim 128, whose Q
// columns and output blocks take one workgroup's worth of registers.
template <typename S, int DH, bool DBG, bool WIN>
__global__ __launch_bounds__(256, (sizeof(S) == 2 || DH == 64) ? 2 : 1) void attn_kernel(AttnParams p, int G, int tps) {
  constexpr bool BF = sizeof(S) == 2;
  constexpr int CH = Storage<S>::CH;
  constexpr int STEP = 4 * CH;
  constexpr int NST = DH / STEP;
  constexpr int NMB = DH / 16;
  constexpr int DC = DH / CH;                    // 16-byte chunks per head row
  // bf16 at head_dim 128 (SWZ): K and V rows of 256 bytes, unpadded, whose
  // 16-byte chunk c sits at position c ^ swz(row) (swz(row) = 2 (row & 7)):
  // the 16 rows of a K operand read and the 4 rows x 2 chunks of a
  // transposed V read fall on distinct chunk positions, and a tile is 32
  // whole 1 KB copies (8 per wave).  Otherwise padded rows:
  constexpr bool SWZ = BF && DH == 128;
  constexpr int KPB = SWZ ? DH * 2 : DH * (int)sizeof(S) + 16;  // K row pitch, bytes
  // bf16: V row-major (pitch DH*2 + 32), read transposed by ds_read_b64_tr_b16;
  // f32: V^T[dh][key] (pitch KT*4 + 16), written transposed
  constexpr int VPB = SWZ ? DH * 2 : BF ? DH * 2 + 32 : KT * 4 + 16;
  constexpr int VBYTES = BF ? KT * VPB : DH * VPB;
  auto swz = [](int row) { return SWZ ? (row & 7) << 1 : 0; };
  constexpr int NCH = (KT * DC + 255) / 256;     // 16-byte chunks of K (and of V) per thread per tile
  constexpr int NB = BF ? 1 : 2;                 // 16-key blocks per P^T operand of one half tile
  static_assert(2 * NCH <= 32, "valid-row bits");
  // K/V ring: bf16 at head_dim 64 (the decode shapes, whose tiles carry
  // little work per byte) keeps two tiles in flight while one is used, in
  // 57 KB of the two workgroups' 160 KB; otherwise one (head_dim 128 fills
  // its 80 KB with two 32 KB stages).
  constexpr int NBUF = (BF && DH == 64) ? 3 : 2;
  __shared__ __attribute__((aligned(16))) char Ks[NBUF][KT * KPB];
  __shared__ __attribute__((aligned(16))) char Vs[NBUF][VBYTES];
  __shared__ int s_start[QMAX], s_off[QMAX + 1];
  __shared__ int s_anc_row[ANC_MAX];                               // chain rows, then
  __shared__ __attribute__((aligned(16))) int s_anc_own[ANC_MAX];  // -1 to the end of the tile
  __shared__ int s_red[12];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int Hkv = p.Hkv, Hq = p.Hq;
  const int QPW = QMAX / G;
  const int maxd = min(p.max_depth, min(MAXD, ANC_MAX / QPW));  // the host checked the bound

  int bid = blockIdx.x;
  const int kvh = bid % Hkv;
  bid /= Hkv;
  int sp, lin, ncut;
  if (p.plan_items) {  // the planned item: (tile, piece) in decreasing order of work
    if (bid >= *p.plan_count) return;
    const int2 it = p.plan_items[bid];
    lin = it.x;
    sp = it.y;
    ncut = p.plan_pieces[lin];
  } else {
    sp = bid % p.n_splits;
    bid /= p.n_splits;
    lin = p.num_seg * tps - 1 - bid;  // later (longer) tiles first
    ncut = p.n_splits;
  }
  const int seg = lin / tps, tile = lin % tps;
  const int qbase = seg * p.q_per_seg + tile * QPW;
  const int nq = min(QPW, p.q_per_seg - tile * QPW);
  // reads that depend on nothing below go out with the query metadata: the
  // segment's first key row and each column's query row (an indexed list in
  // the decode layer)
  const int seg_base = p.seg_kv_base[seg];
  int qrow_c[CBLK];
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) {
    const int cqc = (wave * (CBLK * 16) + cb * 16 + r) / G;
    qrow_c[cb] = cqc < nq ? (p.q_rows ? p.q_rows[qbase + cqc] : qbase + cqc) : -1;
  }

  // ---- per-query metadata, chain lengths, exclusive scan of the lengths.
  // The chain walk keeps its rows in the last K buffer (free until the tile
  // loop), so the compacted list is built from LDS after the scan instead
  // of walking the parents a second time.
  static_assert(QMAX * MAXD * 4 <= KT * KPB, "chain walk rows fit one K buffer");
  int* s_walk = reinterpret_cast<int*>(Ks[NBUF - 1]);
  int st = -1, cnt = 0;
  if (tid < nq) {
    const int qi = qbase + tid;
    const int mi = (p.meta_by_row && p.q_rows) ? p.q_rows[qi] : qi;
    st = p.q_start[mi];
    if (p.q_depth) {
      const int dp = min(max(p.q_depth[mi], 0), maxd);
      int row = p.q_self_row[mi];
      for (int e = 0; e < dp; ++e) {
        if (row < 0 || row >= p.num_kv_rows) break;
        s_walk[tid * MAXD + cnt] = row;
        ++cnt;
        row = p.kv_parent[row];
      }
    }
  }
  if (tid < QMAX) s_start[tid] = st;
  int incl = cnt;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  int mx = st;
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
  if (lane == 63) s_red[wave] = incl;
  if (lane == 0) s_red[4 + wave] = mx;
  if constexpr (WIN) {  // the earliest prefix end among the queries that have one
    int mn = (tid < nq && st >= 0) ? st : 0x7fffffff;
    for (int o = 32; o > 0; o >>= 1) mn = min(mn, __shfl_xor(mn, o, 64));
    if (lane == 0) s_red[8 + wave] = mn;
  }
  __syncthreads();
  int wofs = 0;
  for (int w = 0; w < wave; ++w) wofs += s_red[w];
  const int n_anc_all = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  const int max_start = max(max(s_red[4], s_red[5]), max(s_red[6], s_red[7]));
  const int min_start = WIN ? min(min(s_red[8], s_red[9]), min(s_red[10], s_red[11])) : 0;
  if (tid < QMAX) s_off[tid] = wofs + incl - cnt;
  if (tid == 0) s_off[QMAX] = n_anc_all;
  if (cnt > 0) {
    const int o = wofs + incl - cnt;
    for (int e = 0; e < cnt; ++e) {
      s_anc_row[o + e] = s_walk[tid * MAXD + e];
      s_anc_own[o + e] = tid;
    }
  }
  if (tid < KT) {  // pad the last chain tile (ANC_MAX is a multiple of KT)
    const int e = n_anc_all + tid;
    if (e < ((n_anc_all + KT - 1) / KT) * KT) {
      s_anc_own[e] = -1;
      s_anc_row[e] = -1;
    }
  }
  __syncthreads();
  const int n_anc = (sp == 0) ? n_anc_all : 0;

  // ---- this split's prefix range [kbeg, kend]: piece sp of ncut equal
  // pieces of the tile's own range (plan), or of split_len keys
  int kbeg, kend;
  if (p.plan_items) {
    const int np_all = max_start >= 0 ? (max_start + KT) / KT : 0;
    kbeg = (int)((int64_t)sp * np_all / ncut) * KT;
    kend = (sp == ncut - 1) ? max_start : (int)((int64_t)(sp + 1) * np_all / ncut) * KT - 1;
  } else {
    kbeg = sp * p.split_len;
    kend = (sp == ncut - 1) ? max_start : min(max_start, kbeg + p.split_len - 1);
  }
  int n_pref = (kend >= kbeg) ? (kend - kbeg + KT) / KT : 0;
  // StreamingLLM window (never split): the sink tiles, then the tiles from the
  // earliest window start of this workgroup's queries to its last prefix key
  int w_na = 0, w_bt = 0;
  if constexpr (WIN) {
    if (n_pref > 0) {
      w_na = min((p.win_sink + KT - 1) / KT, n_pref);
      const int wlo = min_start == 0x7fffffff ? 0x7fffffff - KT : max(min_start - p.win_len + 1, 0);
      w_bt = max(wlo / KT, w_na);
      n_pref = w_na + max(n_pref - w_bt, 0);
    }
  }
  // first key of prefix tile it
  auto pkey = [&](int it) -> int {
    if constexpr (WIN) return (it < w_na ? it : w_bt + it - w_na) * KT;
    else return kbeg + it * KT;
  };
  const int n_tiles = n_pref + (n_anc + KT - 1) / KT;

  const S* Q = reinterpret_cast<const S*>(p.q);
  const S* Kg = reinterpret_cast<const S*>(p.k);
  const S* Vg = reinterpret_cast<const S*>(p.v);
  // ---- tile staging.  Thread chunk i covers key (tid + 256 i) / DC, 16-byte
  // chunk (tid + 256 i) % DC of both K and V.  Keys a tile does not hold for
  // anyone (past the prefix end, padding of the last chain tile) load a row
  // the tile does hold - the prefix end, the tile's first chain row - so
  // every staged value is one some column attends (finite for meaningful
  // inputs) and the mask gives it P = 0.  Prefix tiles address from a
  // uniform base; chain tiles per row.  Rows stay inside [0, num_kv_rows).
  const bool have_rows = p.num_kv_rows > 0;
  const int last_row = p.num_kv_rows - 1;
  const int64_t rstride = (int64_t)Hkv * DH;  // elements between K (V) rows
  u32x4 kreg[BF ? 1 : NCH], vreg[BF ? 1 : NCH];  // f32: register staging
  auto load_tile = [&](int it) {
    if constexpr (BF) return;
    if (it < n_pref) {
      const int p0 = pkey(it);
      const int row0 = max(min(seg_base + p0, last_row), 0);
      const int room = max(min(kend - p0, last_row - row0), 0);  // keys past it repeat the last held row
      const S* kb = Kg + (int64_t)row0 * rstride + kvh * DH;
      const S* vb = Vg + (int64_t)row0 * rstride + kvh * DH;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * 256;
        const uint32_t off = (uint32_t)min(c / DC, room) * (uint32_t)rstride + (uint32_t)((c % DC) * CH);
        kreg[i] = ld16(kb + off);
        vreg[i] = ld16(vb + off);
      }
    } else {
      const int a0 = (it - n_pref) * KT;
      const int first = s_anc_row[a0];
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * 256;
        const int rw = s_anc_row[a0 + c / DC];
        const int64_t off = (int64_t)(rw < 0 ? first : rw) * rstride + kvh * DH + (c % DC) * CH;
        kreg[i] = ld16(Kg + off);
        vreg[i] = ld16(Vg + off);
      }
    }
  };
  auto store_tile = [&](int buf) {
    if constexpr (BF) return;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * 256;
      if (c >= KT * DC) continue;
      const int key = c / DC, ch = c % DC;
      *reinterpret_cast<u32x4*>(&Ks[buf][key * KPB + ch * 16]) = kreg[i];
      if constexpr (BF) {
        *reinterpret_cast<u32x4*>(&Vs[buf][key * VPB + ch * 16]) = vreg[i];
      } else {
#pragma unroll
        for (int e = 0; e < CH; ++e)
          *reinterpret_cast<uint32_t*>(&Vs[buf][(ch * CH + e) * VPB + key * 4]) = vreg[i][e];
      }
    }
  };

  // bf16: tiles are copied from global memory straight into LDS.  One
  // 64-lane instruction fills 64 consecutive 16-byte slots of the padded
  // layout (lane l -> slot l); a tile of K takes KPB / 16 of them, one of V
  // VPB / 16, spread round-robin over the waves.  Lanes whose slot is row
  // padding load chunk 0 of their row (never read back).  Each lane's slots
  // are fixed, so a full prefix tile loads from a uniform base plus
  // precomputed offsets; partial prefix tiles clamp the key, chain tiles look
  // their rows up.
  constexpr int KPS = KPB / 16, VPS = VPB / 16;       // 16-byte slots per padded row
  constexpr int NDMA = BF ? KPS + VPS : 0;             // 1 KB copies per tile
  constexpr int NDW = (NDMA + NWAVE - 1) / NWAVE;      // per wave
  // key and 16-byte chunk (0 for padding) of copy q of this lane
  auto dslot = [&](int q, int& key, int& ch) {
    const int j = wave + NWAVE * q;
    const bool isv = j >= KPS;
    const int ps = isv ? VPS : KPS;
    const int slot = (isv ? j - KPS : j) * 64 + lane;
    key = slot / ps;
    ch = SWZ ? (slot % ps) ^ swz(key) : (slot % ps < DC) ? slot % ps : 0;
  };
  uint32_t doff[BF ? NDW : 1];  // element offset of copy q within a full prefix tile
  if constexpr (BF) {
#pragma unroll
    for (int q = 0; q < NDW; ++q) {
      int key, ch;
      dslot(q, key, ch);
      doff[q] = (uint32_t)key * (uint32_t)rstride + (uint32_t)(ch * CH);
    }
  }
  auto dma_tile = [&](int it, int buf) __attribute__((always_inline)) {
    if constexpr (BF) {
      if (it < n_pref) {
        const int p0 = pkey(it);
        const int row0 = max(min(seg_base + p0, last_row), 0);
        const int room = max(min(kend - p0, last_row - row0), 0);  // keys past it repeat the last held row
        const bool whole = room >= KT - 1;
        const S* kb = Kg + (int64_t)row0 * rstride + kvh * DH;
        const S* vb = Vg + (int64_t)row0 * rstride + kvh * DH;
#pragma unroll
        for (int q = 0; q < NDW; ++q) {
          const int j = wave + NWAVE * q;
          if (j >= NDMA) break;
          const bool isv = j >= KPS;
          uint32_t off = doff[q];
          if (!whole) {
            int key, ch;
            dslot(q, key, ch);
            off = (uint32_t)min(key, room) * (uint32_t)rstride + (uint32_t)(ch * CH);
          }
          char* dst = isv ? &Vs[buf][(j - KPS) * 1024] : &Ks[buf][j * 1024];
          copy16_to_lds((isv ? vb : kb) + off, dst);
        }
      } else {
        const int a0 = (it - n_pref) * KT;
        const int first = s_anc_row[a0];
#pragma unroll
        for (int q = 0; q < NDW; ++q) {
          const int j = wave + NWAVE * q;
          if (j >= NDMA) break;
          const bool isv = j >= KPS;
          int key, ch;
          dslot(q, key, ch);
          const int rw = s_anc_row[a0 + key];
          const int64_t off = (int64_t)(rw < 0 ? first : rw) * rstride + kvh * DH + ch * CH;
          char* dst = isv ? &Vs[buf][(j - KPS) * 1024] : &Ks[buf][j * 1024];
          copy16_to_lds((isv ? Vg : Kg) + off, dst);
        }
      }
    }
  };

  // ---- this lane's columns, one per column block
  int cq[CBLK], climit[CBLK], hh[CBLK];
  bool cact[CBLK];
  u32x4 qreg[CBLK][NST];
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) {
    const int col = wave * (CBLK * 16) + cb * 16 + r;
    cq[cb] = col / G;
    hh[cb] = kvh * G + col % G;
    cact[cb] = cq[cb] < nq;
    climit[cb] = cact[cb] ? min(s_start[cq[cb]], kend) : -1;
    if (cact[cb]) {
      lo = min(lo, climit[cb]);
      hi = max(hi, climit[cb]);
    }
    const int qrow = qrow_c[cb];
#pragma unroll
    for (int t = 0; t < NST; ++t)
      qreg[cb][t] = (qrow >= 0) ? ld16(Q + (int64_t)qrow * p.q_stride + (int64_t)hh[cb] * DH + t * STEP + g * CH)
                                : u32x4{0u, 0u, 0u, 0u};
  }
  // the first tiles' copies go out beside the Q reads (one round trip for
  // both); the Q operands are complete before the tile loop, whose global
  // loads are then only the copies of later tiles
  const int n_iter = have_rows ? n_tiles : 0;
  if constexpr (BF) {
    if (n_iter > 0) dma_tile(0, 0);
    if (NBUF > 2 && n_iter > 1) dma_tile(1, 1);
  }
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb)
#pragma unroll
    for (int t = 0; t < NST; ++t) asm volatile("" : : "v"(qreg[cb][t]));
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o, 64));
    hi = max(hi, __shfl_xor(hi, o, 64));
  }
  const int wmin = __builtin_amdgcn_readfirstlane(lo);   // every active column sees keys <= wmin
  const int wmax = __builtin_amdgcn_readfirstlane(hi);   // no column sees keys > wmax
  // chain entries owned by this wave's queries (a query's G columns may
  // straddle two waves when G exceeds a wave's 16 * CBLK columns)
  const int wq0 = min(wave * CBLK * 16 / G, nq), wq1 = min(((wave + 1) * CBLK * 16 + G - 1) / G, nq);
  const int wa0 = s_off[wq0], wa1 = s_off[wq1];

  // m_run: running maximum (raw score units); thr = m_run + thr_gap; mb =
  // m_run * scale * log2 e (0 while no score has been seen, m_run = -inf)
  // l_run: this lane's share of the row sum (its keys); the column's l is
  // the sum over the column's four lanes.  bf16 at head_dim 128 (LMMA): the
  // row sum is one more matrix product per column block, a row of ones times
  // P^T (acc_l, row 0 of a 16-row block: element 0 on the lanes with g = 0,
  // zero elsewhere), so it is rescaled with O and costs no vector adds (the
  // training shapes are bound by the softmax's vector work: 316 against 324
  // us at N=4096; the decode shapes at head_dim 64 keep the adds).
  constexpr bool LMMA = BF && DH == 128;
  float m_run[CBLK], thr[CBLK], mb[CBLK], l_run[LMMA ? 1 : CBLK];
  f32x4 acc[CBLK][NMB];
  f32x4 acc_l[LMMA ? CBLK : 1];
  int64_t dcnt[CBLK];
  uint64_t dhsh[CBLK];
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) {
    m_run[cb] = -INFINITY;
    thr[cb] = -INFINITY;
    mb[cb] = 0.f;
    if constexpr (LMMA) acc_l[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    else l_run[cb] = 0.f;
    dcnt[cb] = 0;
    dhsh[cb] = 0;
#pragma unroll
    for (int i = 0; i < NMB; ++i) acc[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = p.scale_log2;
  const float thr_gap = 8.0f / sl2;

  // ---- per-half steps.  A half is 32 keys; this lane holds keys
  // k0 + 16b + 4g + j (b = 2h, 2h+1; j < 4) of each of its columns.
  typedef f32x4 HalfS[CBLK][2];
  auto s_half = [&](const char* Kb, int h, HalfS& sacc) {  // S^T = K Q^T
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) sacc[cb][0] = sacc[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int t = 0; t < NST; ++t) {
        const int kr = 16 * (2 * h + bb) + r;
        const u32x4 a = *reinterpret_cast<const u32x4*>(Kb + kr * KPB + (((4 * t + g) ^ swz(kr)) * 16));
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) mma16(sacc[cb][bb], a, qreg[cb][t], S());
      }
  };
  // Mask in place: chain keys are visible to the column whose query owns
  // them (the owner list is padded with -1); a prefix key is visible while it
  // is <= the column's limit; tiles every column of the wave sees in full are
  // left unmasked.  Then the running maximum: m of a column moves only when
  // one of its scores exceeds thr = m + 8 / (scale log2 e), i.e. when P would
  // pass 2^8 (the final division by l removes m exactly).  Each lane tests
  // its own scores; the column maximum runs only when some lane of the wave
  // is over.  Returns whether any m moved; alpha then holds the factors
  // (1 on columns that keep m) for O and l, applied by rescale().
  float alpha[CBLK];
  auto check_half = [&](int h, auto anc_c, bool full, int k0, HalfS& sacc) -> bool {
    constexpr bool anc = decltype(anc_c)::value;
    if constexpr (anc) {
      int own[8];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const u32x4 o4 = *reinterpret_cast<const u32x4*>(&s_anc_own[k0 + 16 * (2 * h + bb) + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) own[4 * bb + j] = (int)o4[j];
      }
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sacc[cb][bb][j] = (own[4 * bb + j] == cq[cb]) ? sacc[cb][bb][j] : -INFINITY;
    } else if (!full) {
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        const int d = climit[cb] - k0 - 4 * g;
        const int dl = d - p.win_len, ds = p.win_sink - k0 - 4 * g;  // window bounds, same offsets
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int x = 16 * (2 * h + bb) + j;
            const bool vis = x <= d && (!WIN || x < ds || x > dl);
            sacc[cb][bb][j] = vis ? sacc[cb][bb][j] : -INFINITY;
          }
      }
    }
    if constexpr (DBG) {
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        const int d = climit[cb] - k0 - 4 * g;
        const int dl = d - p.win_len, ds = p.win_sink - k0 - 4 * g;
        for (int i = 0; i < 8; ++i) {
          const int bq = 2 * h + (i >> 2), j = i & 3;
          const int kk = 16 * bq + 4 * g + j;
          const int x = 16 * bq + j;
          const bool vis = anc ? (s_anc_own[k0 + kk] == cq[cb]) : (x <= d && (!WIN || x < ds || x > dl));
          if (vis) {
            const int row = anc ? s_anc_row[k0 + kk] : seg_base + k0 + kk;
            ++dcnt[cb];
            dhsh[cb] += mix64((uint64_t)(uint32_t)row);
          }
        }
      }
    }
    float lmax[CBLK];
    bool over = false;
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) {
      const f32x4* sc = sacc[cb];
      lmax[cb] = max3(max3(sc[0][0], sc[0][1], sc[0][2]), max3(sc[0][3], sc[1][0], sc[1][1]),
                      max3(sc[1][2], sc[1][3], -INFINITY));
      over = over || lmax[cb] > thr[cb];
    }
    if (!__builtin_amdgcn_ballot_w64(over)) return false;
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) {
      const float cmax = colgroup_max(lmax[cb]);
      const bool grow = cmax > thr[cb];  // the same on the column's four lanes
      alpha[cb] = grow ? __builtin_amdgcn_exp2f((m_run[cb] - cmax) * sl2) : 1.0f;
      m_run[cb] = grow ? cmax : m_run[cb];
      thr[cb] = m_run[cb] + thr_gap;
      mb[cb] = (m_run[cb] == -INFINITY) ? 0.f : m_run[cb] * sl2;
    }
    return true;
  };
  auto rescale = [&]() {
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) {
      if constexpr (LMMA) acc_l[cb] *= alpha[cb];
      else l_run[cb] *= alpha[cb];
#pragma unroll
      for (int i = 0; i < NMB; ++i) acc[cb][i] *= alpha[cb];
    }
  };
  typedef u32x4 HalfP[CBLK][NB];
  // P^T packed for the PV product, and this lane's sum of the half's P (added
  // to l together with the products, after any rescale that precedes them)
  auto exp_half = [&](const HalfS& sacc, HalfP& bop, float (&lp)[CBLK]) {
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sacc[cb][i >> 2][i & 3], sl2, -mb[cb]));
      if constexpr (!LMMA) lp[cb] = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
      if constexpr (BF) {
        bop[cb][0] = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                           pack_bf16x2(pv[6], pv[7])};
      } else {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
          bop[cb][bb] = u32x4{__float_as_uint(pv[4 * bb]), __float_as_uint(pv[4 * bb + 1]),
                              __float_as_uint(pv[4 * bb + 2]), __float_as_uint(pv[4 * bb + 3])};
      }
    }
  };
  // O^T += V^T P^T and l += sum P; each V^T operand read once, used for
  // every column block
  auto pv_half = [&](const char* Vb, int h, const HalfP& bop, const float (&lp)[CBLK]) {
    if constexpr (LMMA) {
      // l += (row of ones) P^T: the ones sit in operand row 0 (lanes 0, 16, 32, 48)
      const uint32_t one2 = (r == 0) ? 0x3F803F80u : 0u;  // two bf16 1.0
      const u32x4 ones = {one2, one2, one2, one2};
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) mma16(acc_l[cb], ones, bop[cb][0], S());
    } else {
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) l_run[cb] += lp[cb];
    }
#pragma unroll
    for (int mbk = 0; mbk < NMB; ++mbk) {
      if constexpr (BF) {
        // Lane 4c + m of a 16-lane group addresses dims 16 mbk + 4m .. +3 of
        // key 32h + 16s + 4g + c; lane r then receives dim 16 mbk + r of the
        // four keys c = 0..3 (slots 4s + c of the operand).
        typedef __attribute__((address_space(3))) short4_t lds_s4;
        // (the row 16 further down has the same swizzle)
        const int vr = 32 * h + 4 * g + (r >> 2);
        const int vb = (16 * mbk + 4 * (r & 3)) * 2;  // byte of the row
        const char* vp = Vb + vr * VPB + ((((vb >> 4) ^ swz(vr)) << 4) | (vb & 15));
        const auto lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(vp));
        const auto hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(vp + 16 * VPB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo4), h2 = __builtin_bit_cast(u32x2, hi4);
        const u32x4 aop = {l2.x, l2.y, h2.x, h2.y};
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) mma16(acc[cb][mbk], aop, bop[cb][0], S());
      } else {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const u32x4 aop =
              *reinterpret_cast<const u32x4*>(Vb + (16 * mbk + r) * VPB + (16 * (2 * h + bb) + 4 * g) * 4);
#pragma unroll
          for (int cb = 0; cb < CBLK; ++cb) mma16(acc[cb][mbk], aop, bop[cb][bb], S());
        }
      }
    }
  };

  // an empty use that makes P^T of a half complete at this point
  auto pin = [&](const HalfP& bop) {
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) asm volatile("" : : "v"(bop[cb][bb]));
  };

  // ---- tile loop.  Tile it + NBUF - 1's copies are issued after the
  // barrier, into the buffer of tile it - 1 (every wave has passed the
  // barrier that follows its last read of it); f32 tiles are staged through
  // registers and written to the other buffer after this tile's work, the
  // last iteration reloading its own tile, which keeps the loop free of
  // branches around the staging.  Within a tile the
  // steps are ordered so that the exponentials of one half run beside the
  // matrix products of the other:
  //   S0 | check0 (+rescale) | S1 + exp0 | check1 | PV0 + exp1 | (rescale) | PV1
  if constexpr (!BF) {
    if (n_iter > 0) {
      load_tile(0);
      store_tile(0);
    }
  }
  // One tile; the prefix tiles and the chain tiles run in loops of their
  // own, so that each body has one masking path besides the unmasked one
  // (with both in one body the compiler copied every score at the join).
  auto tile_step = [&](int it, auto anc_c) {
    constexpr bool anc = decltype(anc_c)::value;
    const int buf = NBUF == 2 ? it & 1 : it % NBUF;
    if constexpr (BF) {
      // this wave's copies of tile it (those of tile it + 1, issued later,
      // may stay in flight: the memory counter retires them in order)
      if (NBUF == 2 || it + 1 >= n_iter) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else if (wave < NDMA - NWAVE * (NDW - 1)) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NDW) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NDW - 1) : "memory");
    }
    __syncthreads();
    if constexpr (BF) {
      if (it + NBUF - 1 < n_iter) dma_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);
    } else {
      load_tile(min(it + 1, n_iter - 1));
    }

    const int k0 = anc ? (it - n_pref) * KT : pkey(it);
    // window: a tile no column sees is past the sink and before every window
    const bool skip = anc ? (k0 + KT <= wa0 || k0 >= wa1)
                          : (k0 > wmax || (WIN && k0 >= p.win_sink && k0 + KT - 1 <= wmin - p.win_len));
    if (!skip) {
      const bool full = !DBG && !anc && (k0 + KT - 1 <= wmin) &&
                        (!WIN || k0 + KT - 1 < p.win_sink || k0 > wmax - p.win_len);
      const char* Kb = Ks[buf];
      const char* Vb = Vs[buf];
      HalfS s0, s1;
      HalfP p0, p1;
      float l0[CBLK], l1[CBLK];
      s_half(Kb, 0, s0);
      if (check_half(0, anc_c, full, k0, s0)) rescale();
      s_half(Kb, 1, s1);
      exp_half(s0, p0, l0);
      pin(p0);  // keeps exp0 beside S1 (the compiler would sink it to PV0)
      const bool moved1 = check_half(1, anc_c, full, k0, s1);
      pv_half(Vb, 0, p0, l0);
      exp_half(s1, p1, l1);
      pin(p1);  // keeps exp1 beside PV0
      if (moved1) rescale();
      pv_half(Vb, 1, p1, l1);
    }
    if constexpr (!BF) store_tile(buf ^ 1);
  };
  const int n_pit = min(n_pref, n_iter);
  for (int it = 0; it < n_pit; ++it) tile_step(it, std::false_type{});
  for (int it = n_pit; it < n_iter; ++it) tile_step(it, std::true_type{});

  // ---- epilogue
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) {
    float l_col;
    if constexpr (LMMA) l_col = colgroup_sum(acc_l[cb][0]);  // rows 4g: l on g = 0, zeros elsewhere
    else l_col = colgroup_sum(l_run[cb]);
    if constexpr (DBG) {
      for (int o = 16; o < 64; o <<= 1) {
        dcnt[cb] += __shfl_xor(dcnt[cb], o, 64);
        dhsh[cb] += __shfl_xor(dhsh[cb], o, 64);
      }
    }
    if (!cact[cb]) continue;
    const int qo = qbase + cq[cb];
    const int h = hh[cb];
    if (ncut == 1) {
      const float inv = l_col > 0.f ? 1.0f / l_col : 0.f;
      S* o = reinterpret_cast<S*>(p.out) + ((int64_t)qo * Hq + h) * DH;
#pragma unroll
      for (int mbk = 0; mbk < NMB; ++mbk) {
        const int dh = 16 * mbk + 4 * g;
        if constexpr (BF) {
          u32x2 w = {pack_bf16x2(acc[cb][mbk][0] * inv, acc[cb][mbk][1] * inv),
                     pack_bf16x2(acc[cb][mbk][2] * inv, acc[cb][mbk][3] * inv)};
          *reinterpret_cast<u32x2*>(o + dh) = w;
        } else {
          f32x4 w = acc[cb][mbk] * inv;
          *reinterpret_cast<f32x4*>(o + dh) = w;
        }
      }
      if (p.lse && g == 0)
        p.lse[(int64_t)qo * Hq + h] = l_col > 0.f ? m_run[cb] * p.scale + logf(l_col) : -INFINITY;
    } else {
      const int64_t qh = ((int64_t)sp * p.num_q + qo) * Hq + h;
#pragma unroll
      for (int mbk = 0; mbk < NMB; ++mbk)
        *reinterpret_cast<f32x4*>(p.part_o + qh * DH + 16 * mbk + 4 * g) = acc[cb][mbk];
      if (g == 0) {
        p.part_ml[qh * 2 + 0] = m_run[cb];
        p.part_ml[qh * 2 + 1] = l_col;
      }
    }
    if constexpr (DBG) {
      if (h % G == 0 && g == 0) {
        if (ncut == 1) {
          p.dbg_count[(int64_t)qo * Hkv + kvh] = dcnt[cb];
          p.dbg_hash[(int64_t)qo * Hkv + kvh] = dhsh[cb];
        } else {
          const int64_t qk = ((int64_t)sp * p.num_q + qo) * Hkv + kvh;
          p.part_dbg[qk * 2 + 0] = (uint64_t)dcnt[cb];
          p.part_dbg[qk * 2 + 1] = dhsh[cb];
        }
      }
    }
  }
}

// Merge of split partials, one wave per (query, head), lane s = split s:
// O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^((m_s - M) * scale * log2 e), M = max_s m_s.
// With a plan, query q merges the plan_pieces of its tile (one piece: the
// attention kernel wrote q's output itself, nothing to do).
template <typename S, int DH>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p, int QPW, int tps) {
  const int lane = threadIdx.x & 63;
  const int64_t qh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nqh = (int64_t)p.num_q * p.Hq;
  const float sl2 = p.scale_log2;
  auto pieces_of = [&](int64_t q) -> int {  // <= 64
    if (!p.plan_items) return p.n_splits;
    const int seg = (int)(q / p.q_per_seg), tile = (int)(q % p.q_per_seg) / QPW;
    return p.plan_pieces[seg * tps + tile];
  };
  const int ns = qh < nqh ? pieces_of(qh / p.Hq) : 1;
  if (qh < nqh && ns > 1) {
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
      // four sums over the pieces s = c mod 4; the loads of sixteen pieces
      // are in flight together
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
      const float* po = p.part_o + qh * DH + dh;
      const int64_t spo = nqh * DH;
      int s = 0;
      for (; s + 16 <= ns; s += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = po[(int64_t)(s + u) * spo];
#pragma unroll
        for (int u = 0; u < 16; u += 4) {
          o0 += __shfl(w, s + u, 64) * v[u];
          o1 += __shfl(w, s + u + 1, 64) * v[u + 1];
          o2 += __shfl(w, s + u + 2, 64) * v[u + 2];
          o3 += __shfl(w, s + u + 3, 64) * v[u + 3];
        }
      }
      for (; s + 4 <= ns; s += 4) {
        o0 += __shfl(w, s, 64) * po[(int64_t)s * spo];
        o1 += __shfl(w, s + 1, 64) * po[(int64_t)(s + 1) * spo];
        o2 += __shfl(w, s + 2, 64) * po[(int64_t)(s + 2) * spo];
        o3 += __shfl(w, s + 3, 64) * po[(int64_t)(s + 3) * spo];
      }
      for (; s < ns; ++s) o0 += __shfl(w, s, 64) * po[(int64_t)s * spo];
      reinterpret_cast<S*>(p.out)[qh * DH + dh] = Storage<S>::from_f32(((o0 + o1) + (o2 + o3)) * inv);
    }
    if (lane == 0 && p.lse) p.lse[qh] = L > 0.f ? M * p.scale + logf(L) : -INFINITY;
  }
  if (p.dbg_count) {
    const int64_t nqk = (int64_t)p.num_q * p.Hkv;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nsd = idx < nqk ? pieces_of(idx / p.Hkv) : 1;
    if (idx < nqk && nsd > 1) {
      uint64_t c = 0, h = 0;
      for (int s = 0; s < nsd; ++s) {
        c += p.part_dbg[((int64_t)s * nqk + idx) * 2];
        h += p.part_dbg[((int64_t)s * nqk + idx) * 2 + 1];
      }
      p.dbg_count[idx] = (int64_t)c;
      p.dbg_hash[idx] = h;
    }
  }
}

// The same merge for launches of a few pieces per query (a plan's at most
// three): DH / 4 threads per (query, head), four dimensions (one 16-byte
// partial load per piece) each,
// O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^((m_s - M) * scale * log2 e), M = max_s m_s,
// summed over the pieces in order.  With a plan, query q merges the
// plan_pieces of its tile (one piece: the attention kernel wrote q's output
// itself, nothing to do).
template <typename S, int DH>
__global__ __launch_bounds__(256) void attn_combine_few_kernel(AttnParams p, int QPW, int tps) {
  constexpr int TPQ = DH / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t qh = gid / TPQ;
  const int d4 = (int)(gid % TPQ) * 4;
  const int64_t nqh = (int64_t)p.num_q * p.Hq;
  const float sl2 = p.scale_log2;
  auto pieces_of = [&](int64_t q) -> int {
    if (!p.plan_items) return p.n_splits;
    const int seg = (int)(q / p.q_per_seg), tile = (int)(q % p.q_per_seg) / QPW;
    return p.plan_pieces[seg * tps + tile];
  };
  const int ns = qh < nqh ? pieces_of(qh / p.Hq) : 1;
  if (qh < nqh && ns > 1) {
    const float* ml = p.part_ml + qh * 2;
    const float* po = p.part_o + qh * DH + d4;
    const int64_t sml = nqh * 2, spo = nqh * DH;
    float M = -INFINITY, L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    // up to eight pieces: every piece's (m, l) and partial output loaded in
    // one round trip, then the maximum and the sums over the pieces in order
    auto merge = [&](auto nc) {
      constexpr int NP = decltype(nc)::value;
      float2 t[NP];
      f32x4 v[NP];
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        t[u] = *reinterpret_cast<const float2*>(ml + (int64_t)u * sml);
        v[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)u * spo);
      }
#pragma unroll
      for (int u = 0; u < NP; ++u) M = fmaxf(M, t[u].x);
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const float w = t[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((t[u].x - M) * sl2);
        L += w * t[u].y;
        o += w * v[u];
      }
    };
    switch (ns) {
      case 2: merge(std::integral_constant<int, 2>{}); break;
      case 3: merge(std::integral_constant<int, 3>{}); break;
      case 4: merge(std::integral_constant<int, 4>{}); break;
      case 5: merge(std::integral_constant<int, 5>{}); break;
      case 6: merge(std::integral_constant<int, 6>{}); break;
      case 7: merge(std::integral_constant<int, 7>{}); break;
      case 8: merge(std::integral_constant<int, 8>{}); break;
      default: {
        // more pieces: loads in batches of U pieces (independent, in flight
        // together); the sums still run over the pieces in order
        constexpr int U = 8;
        for (int s0 = 0; s0 < ns; s0 += U) {
          float t[U];
#pragma unroll
          for (int u = 0; u < U; ++u) t[u] = s0 + u < ns ? ml[(int64_t)(s0 + u) * sml] : -INFINITY;
#pragma unroll
          for (int u = 0; u < U; ++u) M = fmaxf(M, t[u]);
        }
        for (int s0 = 0; s0 < ns; s0 += U) {
          float2 t[U];
          f32x4 v[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int sc = min(s0 + u, ns - 1);  // clamped; pieces past ns get weight 0
            t[u] = *reinterpret_cast<const float2*>(ml + (int64_t)sc * sml);
            v[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)sc * spo);
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const float w = (s0 + u >= ns || t[u].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((t[u].x - M) * sl2);
            L += w * t[u].y;
            o += w * v[u];
          }
        }
      }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    S* out = reinterpret_cast<S*>(p.out) + qh * DH + d4;
    if constexpr (sizeof(S) == 2) {
      *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    } else {
      *reinterpret_cast<f32x4*>(out) = o * inv;
    }
    if (d4 == 0 && p.lse) p.lse[qh] = L > 0.f ? M * p.scale + logf(L) : -INFINITY;
  }
  if (p.dbg_count) {
    const int64_t nqk = (int64_t)p.num_q * p.Hkv;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nsd = idx < nqk ? pieces_of(idx / p.Hkv) : 1;
    if (idx < nqk && nsd > 1) {
      uint64_t c = 0, h = 0;
      for (int s = 0; s < nsd; ++s) {
        c += p.part_dbg[((int64_t)s * nqk + idx) * 2];
        h += p.part_dbg[((int64_t)s * nqk + idx) * 2 + 1];
      }
      p.dbg_count[idx] = (int64_t)c;
      p.dbg_hash[idx] = h;
    }
  }
}

// Work plan of one launch (one workgroup of 1,024 threads; at most
// kPlanMaxTiles query tiles).  A query tile's work is estimated as its prefix
// tiles (up to its largest start) plus its chain tiles; the per-query reads
// are spread over all threads (a thread per tile would wait on each of its
// queries in turn).  The tile is cut into pieces (see AttnParams) and the
// items are bucket-sorted by decreasing work (largest first: the longest
// items start in the first round and the short ones fill the tail).  The
// order within a bucket may vary from run to run; results do not depend on
// it (every piece and every merge is computed in a fixed order).
__global__ __launch_bounds__(1024) void attn_plan_kernel(AttnParams p, int QPW, int tps) {
  constexpr int NB = 2048;  // work buckets (in key tiles; larger items share the last)
  __shared__ int hist[NB];
  __shared__ int tmax[kPlanMaxTiles], tchain[kPlanMaxTiles];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = p.num_seg * tps;
  for (int b = tid; b < NB; b += 1024) hist[b] = 0;
  for (int t = tid; t < ntiles; t += 1024) {
    tmax[t] = -1;
    tchain[t] = 0;
  }
  __syncthreads();
  constexpr int UQ = 4;  // queries whose metadata loads are in flight together
  for (int q0 = tid; q0 < p.num_q; q0 += 1024 * UQ) {
    int st[UQ], dp[UQ];
#pragma unroll
    for (int u = 0; u < UQ; ++u) {
      const int q = q0 + 1024 * u;
      const int mi = q < p.num_q ? ((p.meta_by_row && p.q_rows) ? p.q_rows[q] : q) : -1;
      st[u] = mi >= 0 ? p.q_start[mi] : -1;
      dp[u] = (mi >= 0 && p.q_depth) ? min(max(p.q_depth[mi], 0), p.max_depth) : 0;
    }
#pragma unroll
    for (int u = 0; u < UQ; ++u) {
      const int q = q0 + 1024 * u;
      if (q < p.num_q) {
        const int lin = (q / p.q_per_seg) * tps + (q % p.q_per_seg) / QPW;
        atomicMax(&tmax[lin], st[u]);
        if (dp[u]) atomicAdd(&tchain[lin], dp[u]);
      }
    }
  }
  __syncthreads();
  auto pieces = [&](int npref) {
    return p.plan_nmax > 1 ? min(p.plan_nmax, max(1, (npref + p.plan_tiles - 1) / p.plan_tiles)) : 1;
  };
  auto bucket = [&](int npref, int nanc, int c, int sp) {
    const int w = (int)((int64_t)(sp + 1) * npref / c - (int64_t)sp * npref / c) + (sp == 0 ? nanc : 0);
    return min(w, NB - 1);
  };
  for (int lin = tid; lin < ntiles; lin += 1024) {
    const int np = tmax[lin] >= 0 ? (tmax[lin] + KT) / KT : 0, na = (tchain[lin] + KT - 1) / KT;
    const int c = pieces(np);
    p.plan_pieces[lin] = c;
    for (int sp = 0; sp < c; ++sp) atomicAdd(&hist[bucket(np, na, c, sp)], 1);
  }
  __syncthreads();
  // exclusive scan over the buckets in decreasing order of work: thread t
  // takes positions 2t, 2t + 1 (buckets NB-1-2t, NB-2-2t)
  const int b0 = NB - 1 - 2 * tid, b1 = b0 - 1;
  const int h0 = hist[b0], h1 = hist[b1];
  const int v = h0 + h1;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wofs = 0;
  for (int w = 0; w < wave; ++w) wofs += wsum[w];
  hist[b0] = wofs + incl - v;
  hist[b1] = wofs + incl - v + h0;
  if (tid == 1023) *p.plan_count = wofs + incl;
  __syncthreads();
  for (int lin = tid; lin < ntiles; lin += 1024) {
    const int np = tmax[lin] >= 0 ? (tmax[lin] + KT) / KT : 0, na = (tchain[lin] + KT - 1) / KT;
    const int c = pieces(np);
    for (int sp = 0; sp < c; ++sp) p.plan_items[atomicAdd(&hist[bucket(np, na, c, sp)], 1)] = make_int2(lin, sp);
  }
}

template <typename S, int DH>
static void launch_attn_t(const AttnParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  const int QPW = attn_queries_per_workgroup(G, DH);
  const int tps = (p.q_per_seg + QPW - 1) / QPW;
  const int ncut = p.plan_items ? p.plan_nmax : p.n_splits;
  const int grid = p.num_seg * tps * ncut * p.Hkv;
  if (p.plan_items) hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, s, p, QPW, tps);
  if (p.win_len > 0) {
    if (p.dbg_count) hipLaunchKernelGGL((attn_kernel<S, DH, true, true>), dim3(grid), dim3(256), 0, s, p, G, tps);
    else hipLaunchKernelGGL((attn_kernel<S, DH, false, true>), dim3(grid), dim3(256), 0, s, p, G, tps);
  } else {
    if (p.dbg_count) hipLaunchKernelGGL((attn_kernel<S, DH, true, false>), dim3(grid), dim3(256), 0, s, p, G, tps);
    else hipLaunchKernelGGL((attn_kernel<S, DH, false, false>), dim3(grid), dim3(256), 0, s, p, G, tps);
  }
  if (ncut > 1) {
    const int64_t nqh = (int64_t)p.num_q * p.Hq;
    const int64_t nqk = (int64_t)p.num_q * p.Hkv;
    if (ncut <= 8) {
      int64_t blocks = (nqh * (DH / 4) + 255) / 256;
      if (p.dbg_count && (nqk + 255) / 256 > blocks) blocks = (nqk + 255) / 256;
      hipLaunchKernelGGL((attn_combine_few_kernel<S, DH>), dim3((unsigned)blocks), dim3(256), 0, s, p, QPW, tps);
    } else {
      int64_t blocks = (nqh + 3) / 4;
      if (p.dbg_count && (nqk + 255) / 256 > blocks) blocks = (nqk + 255) / 256;
      hipLaunchKernelGGL((attn_combine_kernel<S, DH>), dim3((unsigned)blocks), dim3(256), 0, s, p, QPW, tps);
    }
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
