// Large-M contractions on the gfx950 matrix cores, bf16 operands:
//   Y[m][n] = sum_k X[m][k] * W[n][k]   (X: [M, K] activation rows, W: packed weights)
// for the batched decode shapes (M in the hundreds), finished by the same
// epilogues as the other contractions (gemm.hip).
//
// A workgroup of 2 x WN waves owns an output tile of BM activation rows x BN
// features; each wave a (BM/2) x (BN/WN) sub-tile accumulated in registers
// (112 or 128 rows x 64 features for the 224/256 x 128 tiles with four
// waves: up to 128 accumulator registers per lane; 112 x 80 and 140 for the
// LM head's 224 x 160; two waves per SIMD).  Both
// operands go through LDS in a ring of D stages, one 32-wide k-step each,
// copied by global_load_lds_dwordx4 without passing through registers; D - 1
// k-steps are in flight while one is multiplied:
//  * weights: the packed 1 KB chunks as they are (one chunk = the operand of
//    one 16-feature x 32-k step, lane l's 16 bytes at 16 l), so a wave reads
//    its operand with one conflict-free ds_read_b128;
//  * activations: 64 bytes (32 k) per row, the four 16-byte chunks of row R
//    stored at position chunk ^ ((R >> 1) & 3), so the rows of one operand
//    read land in distinct banks.  Rows past M copy row M-1 (their results
//    are dropped).  Activations already in the operand layout (PX: 1 KB
//    chunks of 16 rows x 32 k, lane slot 16 c + r = row r, k 8c..8c+7) are
//    copied chunk by chunk: one copy touches 8 cache lines instead of 16,
//    which is what bounds the activation traffic of these tiles.
// One barrier per k-step.  Workgroup ids map the M tiles of one N tile back
// to back onto one XCD (workgroup i runs on XCD i % 8), so each weight chunk
// is fetched from HBM once.  A K split takes its shares' k-step ranges from
// p.split_k when the host gives them (shares cut at the segments of an
// operand with deferred scales, each share inside one segment), else equal
// shares.  L2->LDS traffic per flop is (BM + BN) / (BM BN)
// bytes: 3/256 for 256 x 128, against 1/64 for the 128 x 128 tiles.
#include <math.h>
#include "epilogue.h"

namespace pe {

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Two waves per SIMD: two 4-wave workgroups (or one 8-wave one) per CU.
template <int BM, int BN, int WN, int D, bool DUAL, bool ARGMAX, bool SPLIT, bool PX, bool LSE>
__global__ __launch_bounds__(128 * WN) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_big_kernel(GemmParams p, int n_ft, int n_mt) {
  constexpr int NW = 2 * WN;           // waves: 2 along the rows x WN along the features
  constexpr int WB = BN / 16;          // 16-feature weight blocks per tile
  constexpr int FW = BN / 16 / WN;     // weight blocks per wave
  constexpr int RW = BM / 32;          // 16-row activation groups per wave
  constexpr int WBYTES = WB * 1024;    // one weight matrix, one k-step
  constexpr int XOFF = WBYTES * (DUAL ? 2 : 1);
  constexpr int STAGE = XOFF + BM * 64;
  constexpr int WI = (WB + NW - 1) / NW;  // weight copies per wave per k-step (per matrix; the
                                         // last block repeats when NW does not divide WB)
  constexpr int XI = (BM / 16 + NW - 1) / NW;  // activation copies per wave per k-step (the
                                               // last group repeats when NW does not divide BM / 16)
  constexpr int PT = WI * (DUAL ? 2 : 1) + XI;  // vector-memory operations per wave per k-step
  static_assert(BM % 32 == 0 && BN % (16 * WN) == 0, "tile shape");
  static_assert(!ARGMAX || D * STAGE >= WN * BM * 16, "row-reduction lists fit in the ring");
  extern __shared__ __attribute__((aligned(16))) char lds[];  // D stages

  const int bid = blockIdx.x;
  const int xcd = bid & 7, jj = bid >> 3;
  const int mt = jj % n_mt;
  const int ft = (jj / n_mt) * 8 + xcd;
  if (ft >= n_ft) return;
  const int M = p.M, N = p.N, K = p.K;
  // K split: workgroup (x, y) takes the y-th share of the 32-wide k-steps
  const int ksteps = K / 32;
  const int y = blockIdx.y;
  const int kbeg = !SPLIT ? 0 : p.nsplit_k ? p.split_beg[y] : (int)((int64_t)ksteps * y / gridDim.y);
  const int nsteps = !SPLIT ? ksteps : (p.nsplit_k ? p.split_end[y] : (int)((int64_t)ksteps * (y + 1) / gridDim.y)) - kbeg;
  const int nfb = (N + 15) >> 4;
  const int n0 = ft * BN, m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(p.X);

  // weight chunks this wave copies: blocks wave + NW * i (clamped past N)
  const char* wsrc[WI];
  const char* w2src[DUAL ? WI : 1];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int64_t off = ((int64_t)min(n0 / 16 + min(wave + NW * i, WB - 1), nfb - 1) * ksteps + kbeg) * 1024 + lane * 16;
    wsrc[i] = reinterpret_cast<const char*>(p.W) + off;
    if constexpr (DUAL) w2src[i] = reinterpret_cast<const char*>(p.W2) + off;
  }
  // activation chunks: instruction i covers rows 16 (wave + NW i) .. +15, four
  // 16-byte chunks each; row R keeps chunk c at position c ^ ((R >> 1) & 3)
  const uint16_t* xsrc[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    if constexpr (PX) {
      // chunk of 16-row group G, k-step t at element (G * ksteps + t) * 512
      const int grp = min(mt * (BM / 16) + min(wave + NW * i, BM / 16 - 1), (M + 15) / 16 - 1);
      xsrc[i] = X + ((int64_t)grp * ksteps + kbeg) * 512 + lane * 8;
    } else {
      const int row = min(wave + NW * i, BM / 16 - 1) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 1) & 3);
      xsrc[i] = X + (int64_t)min(m0 + row, M - 1) * p.ldx + kbeg * 32 + c * 8;
    }
  }
  auto issue = [&](int t) {
    char* st = lds + (t % D) * STAGE;
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      copy16_to_lds(wsrc[i] + (int64_t)t * 1024, st + min(wave + NW * i, WB - 1) * 1024);
      if constexpr (DUAL) copy16_to_lds(w2src[i] + (int64_t)t * 1024, st + WBYTES + min(wave + NW * i, WB - 1) * 1024);
    }
#pragma unroll
    for (int i = 0; i < XI; ++i)
      copy16_to_lds(xsrc[i] + (int64_t)t * (PX ? 512 : 32), st + XOFF + min(wave + NW * i, BM / 16 - 1) * 1024);
  };

  f32x4 acc[FW][RW], acc2[DUAL ? FW : 1][DUAL ? RW : 1];
#pragma unroll
  for (int f = 0; f < FW; ++f)
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      acc[f][q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (DUAL) acc2[f][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // Pipeline: every stage of the ring holds a k-step in flight or resident.
  // Iteration t: issue step t's matrix products (their operands are already
  // in registers), then wait until step t+1 has landed (the barrier also
  // means every wave is done reading step t's stage), refill that stage with
  // step t+D and read step t+1's operands into the other register set while
  // the products run.
  u32x4 fa[2][FW], fa2[2][DUAL ? FW : 1], fb[2][RW];
#define PE_BIG_FRAGS(T, SET)                                                                             \
  {                                                                                                      \
    const char* st_ = lds + ((T) % D) * STAGE;                                                           \
    _Pragma("unroll") for (int f = 0; f < FW; ++f) {                                                     \
      fa[SET][f] = *reinterpret_cast<const u32x4*>(st_ + (wn * FW + f) * 1024 + lane * 16);              \
      if constexpr (DUAL) fa2[SET][f] = *reinterpret_cast<const u32x4*>(st_ + WBYTES + (wn * FW + f) * 1024 + lane * 16); \
    }                                                                                                    \
    _Pragma("unroll") for (int q = 0; q < RW; ++q) {                                                     \
      const int R_ = wm * (BM / 2) + q * 16 + r;                                                         \
      fb[SET][q] = *reinterpret_cast<const u32x4*>(st_ + XOFF + (PX ? (R_ >> 4) * 1024 + lane * 16        \
                                                                    : R_ * 64 + 16 * (g ^ ((R_ >> 1) & 3)))); \
    }                                                                                                    \
  }
#define PE_BIG_MMA(CUR)                                                                                  \
  _Pragma("unroll") for (int f = 0; f < FW; ++f)                                                         \
    _Pragma("unroll") for (int q = 0; q < RW; ++q) {                                                     \
      mma16(acc[f][q], fa[CUR][f], fb[CUR][q], uint16_t());                                              \
      if constexpr (DUAL) mma16(acc2[f][q], fa2[CUR][f], fb[CUR][q], uint16_t());                        \
    }
#define PE_BIG_ITER(T, CUR, NXT)                                                                         \
  {                                                                                                      \
    PE_BIG_MMA(CUR)                                                                                      \
    if ((T) + 1 < nsteps) {                                                                              \
      if ((T) + D - 1 < nsteps) wait_vm<PT * (D - 2)>(); else wait_vm<0>();                              \
      __syncthreads();                                                                                   \
      if ((T) + D < nsteps) issue((T) + D);                                                              \
      PE_BIG_FRAGS((T) + 1, NXT)                                                                         \
    }                                                                                                    \
  }
#pragma unroll
  for (int t = 0; t < D; ++t)
    if (t < nsteps) issue(t);
  if (nsteps >= D) wait_vm<PT * (D - 1)>(); else wait_vm<0>();
  __syncthreads();
  PE_BIG_FRAGS(0, 0)
  for (int t = 0; t < nsteps; t += 2) {
    PE_BIG_ITER(t, 0, 1)
    if (t + 1 < nsteps) PE_BIG_ITER(t + 1, 1, 0)
  }
#undef PE_BIG_ITER
#undef PE_BIG_MMA
#undef PE_BIG_FRAGS
  if constexpr (ARGMAX) {
    // argmax (EPI_ARGMAX) or log-sum-exp (EPI_LSE, LSE set) partials of this tile's rows
    // per wave column and row: (v, s) or the top-2 list, in the copy ring's
    // LDS once every wave is done with it (a static array would take the
    // second workgroup's room on the CU)
    __syncthreads();
    u32x4* sb = reinterpret_cast<u32x4*>(lds);
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      const int mloc = wm * (BM / 2) + q * 16 + r;
      const int m = m0 + mloc;
      int tgt = -1;
      if constexpr (LSE) tgt = (p.epi.targets && m < M) ? p.epi.targets[m] : -1;
      RowRed rr = RowRed::init();
#pragma unroll
      for (int f = 0; f < FW; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * (BN / WN) + f * 16 + 4 * g + j;
          if (n < N && m < M) {
            const float v = acc[f][q][j];
            if (p.epi.logits) p.epi.logits[(int64_t)m * N + n] = v;
            if constexpr (LSE) {
              if (n == tgt) p.epi.tgt_logit[m] = v;
              rr.add(true, v, n);
            } else {
              // the largest of the lane's 16 features per row; the merges
              // below keep the two largest of the lanes' maxima
              rr.add1(v, n);
            }
          }
        }
      rr.merge_groups(LSE);
      if (g == 0) sb[wn * BM + mloc] = LSE ? u32x4{__float_as_uint(rr.v), 0u, __float_as_uint(rr.s), 0u} : rr.pack2();
    }
    __syncthreads();
    if (tid < BM && m0 + tid < M) {
      RowRed rr = RowRed::init();
      for (int w = 0; w < WN; ++w) {
        const u32x4 o = sb[w * BM + tid];
        if constexpr (LSE) rr.merge(true, __uint_as_float(o[0]), 0, __uint_as_float(o[2]));
        else rr.merge_packed(o);
      }
      if constexpr (LSE) {
        p.epi.part_val[(int64_t)ft * M + m0 + tid] = rr.v;
        p.epi.part_sum[(int64_t)ft * M + m0 + tid] = rr.s;
      } else {
        p.epi.part_top2[(int64_t)ft * M + m0 + tid] = rr.pack2();
      }
    }
  } else if constexpr (SPLIT) {
    // partial tile of split y: [y][m][n] (the second matrix's after all splits)
    float* part = p.split_ws + (int64_t)blockIdx.y * M * N;
    float* part2 = p.split_ws + ((int64_t)gridDim.y + blockIdx.y) * M * N;
#pragma unroll
    for (int f = 0; f < FW; ++f)
#pragma unroll
      for (int q = 0; q < RW; ++q) {
        const int n = n0 + wn * (BN / WN) + f * 16 + 4 * g;  // N is a multiple of 4 here
        const int m = m0 + wm * (BM / 2) + q * 16 + r;
        if (n < N && m < M) {
          *reinterpret_cast<f32x4*>(part + (int64_t)m * N + n) = acc[f][q];
          if constexpr (DUAL) *reinterpret_cast<f32x4*>(part2 + (int64_t)m * N + n) = acc2[DUAL ? f : 0][DUAL ? q : 0];
        }
      }
  } else {
#pragma unroll
    for (int f = 0; f < FW; ++f)
#pragma unroll
      for (int q = 0; q < RW; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * (BN / WN) + f * 16 + 4 * g + j;
          const int m = m0 + wm * (BM / 2) + q * 16 + r;
          if (n < N && m < M)
            epi_store<uint16_t>(p.epi, m, n, acc[f][q][j], DUAL ? acc2[DUAL ? f : 0][DUAL ? q : 0][j] : 0.f);
        }
  }
}

// The epilogue of features n..n+3 of row m (n a multiple of 4) for the kinds
// a K split finishes (fc, QKV, residual) with 8- or 16-byte accesses, in
// three steps so that the reads go out early: the row's metadata (meta: the
// token id, the residual row or the KV slot; skip: a rejected row), the
// addend (embedding or residual elements, which depend on the metadata but
// not on the sums), then the store.  The values equal epi_store's element by
// element; other kinds and unaligned operands (vec false) take epi_store.
struct Reduce4 {
  int meta;
  bool skip;
  f32x4 add;
};
__device__ __forceinline__ void reduce_meta(const Epi& e, int m, Reduce4& t) {
  t.meta = m;
  t.skip = false;
  t.add = f32x4{0.f, 0.f, 0.f, 0.f};
  switch (e.kind) {
    case EPI_FC:
      t.skip = e.rejected && e.rejected[m];
      t.meta = e.ids[m];
      break;
    case EPI_RESID:
      t.meta = e.res_rows ? e.res_rows[m] : m;
      break;
    case EPI_QKV:
      t.meta = e.slots[m];
      break;
    default:
      break;
  }
}
__device__ __forceinline__ void reduce_addend(const Epi& e, int n, Reduce4& t) {
  if (e.kind == EPI_FC) {
    if (!t.skip && t.meta >= 0 && t.meta < e.embed_rows) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(e.embed) + (int64_t)t.meta * e.ld_out + n);
      t.add = f32x4{bf2f((uint16_t)w.x), bf2f((uint16_t)(w.x >> 16)), bf2f((uint16_t)w.y), bf2f((uint16_t)(w.y >> 16))};
    }
  } else if (e.kind == EPI_RESID) {
    t.add = *reinterpret_cast<const f32x4*>(e.res + (int64_t)t.meta * e.ld_res + n);
  }
}
__device__ __forceinline__ void reduce_store4(const Epi& e, int m, int n, const f32x4& y, const Reduce4& t) {
  switch (e.kind) {
    case EPI_FC:
      if (!t.skip) *reinterpret_cast<f32x4*>(e.out_f32 + (int64_t)m * e.ld_out + n) = y + t.add;
      return;
    case EPI_RESID:
      *reinterpret_cast<f32x4*>(e.out_f32 + (int64_t)m * e.ld_out + n) = y + t.add;
      return;
    case EPI_QKV: {
      const u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      if (n < e.q_cols) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(e.out_s) + (int64_t)m * e.q_cols + n) = w;
        return;
      }
      const int slot = t.meta;
      if (slot < 0 || slot >= e.kv_rows) return;
      int c = n - e.q_cols;
      uint16_t* dst = reinterpret_cast<uint16_t*>(c < e.kv_cols ? e.k_cache : e.v_cache);
      if (c >= e.kv_cols) c -= e.kv_cols;
      *reinterpret_cast<u32x2*>(dst + (int64_t)slot * e.kv_cols + c) = w;
      return;
    }
    default:
#pragma unroll
      for (int j = 0; j < 4; ++j) epi_store<uint16_t>(e, m, n + j, y[j], 0.f);
      return;
  }
}

// Whether reduce_store4 may take the vector path for this epilogue.
static bool reduce_vec_ok(const Epi& e) {
  auto al = [](const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; };
  switch (e.kind) {
    case EPI_FC:
      return e.ld_out % 4 == 0 && al(e.out_f32, 16) && al(e.embed, 8);
    case EPI_RESID:
      return e.ld_out % 4 == 0 && e.ld_res % 4 == 0 && al(e.out_f32, 16) && al(e.res, 16);
    case EPI_QKV:
      return e.q_cols % 4 == 0 && e.kv_cols % 4 == 0 && al(e.out_s, 8) && al(e.k_cache, 8) && al(e.v_cache, 8);
    default:
      return false;
  }
}

// Sum of the K-split partial products in split order (deterministic), then
// the contraction's epilogue; one thread per four features of one row.  The
// share count is a template argument, so the partials of every share (and
// their row scales) are loaded before the first add: one round trip for all
// shares instead of one each.
template <int NS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p, int vec) {
  const int M = p.M, N = p.N;
  const int i = blockIdx.x * 256 + threadIdx.x;  // M * N / 4 < 2^31 (checked by big_split_plan)
  if (i >= M * (N / 4)) return;
  const int m = i / (N / 4), n = (i % (N / 4)) * 4;
  Reduce4 t;
  if (vec) reduce_meta(p.epi, m, t);
  f32x4 part[NS];
  float sc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    // a share of a deferred-scale operand lies in one segment: scale it by the row's 1 / rms there
    sc[s] = p.xinv ? p.xinv[(int64_t)m * p.xinv_segs + (p.nsplit_k ? p.split_seg[s] : 0)] : 1.f;
    part[s] = *reinterpret_cast<const f32x4*>(p.split_ws + ((int64_t)s * M + m) * N + n);
  }
  if (vec) reduce_addend(p.epi, n, t);
  f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) y += part[s] * sc[s];
  if (vec) {
    reduce_store4(p.epi, m, n, y, t);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) epi_store<uint16_t>(p.epi, m, n + j, y[j], 0.f);
  }
}

template <int NS>
static void launch_reduce_ns(const GemmParams& q, int64_t n4, hipStream_t s) {
  hipLaunchKernelGGL((splitk_reduce_kernel<NS>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, q,
                     reduce_vec_ok(q.epi) ? 1 : 0);
}

static void launch_splitk_reduce(const GemmParams& q, int splits, hipStream_t s) {
  static_assert(kMaxSplitK == 8, "one instantiation per share count");
  const int64_t n4 = (int64_t)q.M * (q.N / 4);
  switch (splits) {
    case 2: launch_reduce_ns<2>(q, n4, s); break;
    case 3: launch_reduce_ns<3>(q, n4, s); break;
    case 4: launch_reduce_ns<4>(q, n4, s); break;
    case 5: launch_reduce_ns<5>(q, n4, s); break;
    case 6: launch_reduce_ns<6>(q, n4, s); break;
    case 7: launch_reduce_ns<7>(q, n4, s); break;
    default: launch_reduce_ns<8>(q, n4, s); break;  // big_split_plan gives 2..kMaxSplitK
  }
}

template <int BM, int BN, int WN, int STAGES, bool DUAL, bool ARGMAX, bool SPLIT, bool PX = false, bool LSE = false>
static int launch_big(const GemmParams& p, int splits, hipStream_t s) {
  constexpr int STAGE = (BN / 16) * 1024 * (DUAL ? 2 : 1) + BM * 64;
  // once per process (thread-safe initialisation; a failure shows up as a failed launch)
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_big_kernel<BM, BN, WN, STAGES, DUAL, ARGMAX, SPLIT, PX, LSE>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, STAGES * STAGE);
  (void)attr;
  const int n_ft = (p.N + BN - 1) / BN, n_mt = (p.M + BM - 1) / BM;
  const int grid = ((n_ft + 7) / 8) * 8 * n_mt;
  hipLaunchKernelGGL((gemm_big_kernel<BM, BN, WN, STAGES, DUAL, ARGMAX, SPLIT, PX, LSE>), dim3(grid, splits), dim3(128 * WN),
                     STAGES * STAGE, s, p, n_ft, n_mt);
  return n_ft;
}

// Tile shapes: 256 or 224 rows (whichever pads M less: 448 = 2 x 224,
// 896 = 4 x 224) x 128 features, four waves and a three-stage ring, for
// single contractions and the LM head.  The LM head on 224-row tiles takes
// 160 features: the 448-row batch is then 2 x 1,257 workgroups, 4.91 rounds
// of the 512 resident slots, where 128 features give 2 x 1,571 = 6.14
// rounds whose last one runs 86 % empty (c=64 LM stage 539 -> 481 us); the
// fused loss over 7,794 rows takes the same tile for its smaller L2->LDS
// copy traffic per product (10.2 -> 9.3 ms).  Its ten weight blocks per
// k-step take three copies per wave, waves 2 and 3 copying the last block
// again (the same bytes to the same place).  The K-split projections keep
// 128 features (160 measured slower: fewer workgroups).  The
// template also takes the gate/up
// pair (DUAL: two weight streams, two accumulator sets), which measured
// slower than the 128 x 64 register-fed tiles of gemm.hip and is not
// dispatched.  Contractions with too few tiles to give every CU two
// workgroups split K over up to 4 workgroups (at least 16 k-steps each) when
// the caller's workspace holds the partial products (gemm_big_splits); without
// a split launch_gemm_big returns -1 and launches nothing.
static bool rows224(int M) { return ((M + 223) / 224) * 224 < ((M + 255) / 256) * 256; }

// K-split policy: enough workgroups for PE_SPLIT_SLOTS resident tiles, at
// most PE_SPLIT_MAX shares of at least PE_SPLIT_MINSTEPS k-steps each, and a
// PE_SPLIT_STAGES-deep copy ring.
#ifndef PE_SPLIT_SLOTS
#define PE_SPLIT_SLOTS 512
#endif
// At most 4 shares: the partial sums are written and read once more per
// share (c=64 step: 991 us with up to 8, 961 us with up to 4, 992 / 1,006 us
// with 3 / 6).
#ifndef PE_SPLIT_MAX
#define PE_SPLIT_MAX 4
#endif
#ifndef PE_SPLIT_MINSTEPS
#define PE_SPLIT_MINSTEPS 16
#endif
#ifndef PE_SPLIT_STAGES
#define PE_SPLIT_STAGES 3
#endif

// Share ranges of a K split: `base` equal shares of the ksteps k-steps, also
// cut at the segment boundaries of a deferred-scale operand (segs > 1) so that
// every share lies in one segment (the fc fusion at 896 rows: 4 shares cut at
// the three streams give 6 shares of 67, 23, 45, 45, 22 and 68 k-steps; the
// longest is as long as with 4).  The shares are ordered longest first (the
// dispatcher starts workgroups in share order, so the short ones fill in
// behind the long ones).  Writes each share's range to bb / be and its
// segment to bseg; returns the count (0 past kMaxSplitK).
static int split_ranges(int ksteps, int base, int segs, int* bb, int* be, int* bseg) {
  int bk[kMaxSplitK + 1];
  int cut[kMaxSplitK * 2 + 2];
  int n = 0;
  for (int i = 0; i <= base; ++i) cut[n++] = (int)((int64_t)ksteps * i / base);
  for (int j = 1; j < segs; ++j) cut[n++] = ksteps / segs * j;
  for (int i = 1; i < n; ++i)  // insertion sort of at most a dozen cuts
    for (int k = i; k > 0 && cut[k - 1] > cut[k]; --k) { const int t = cut[k]; cut[k] = cut[k - 1]; cut[k - 1] = t; }
  int m = 0;
  for (int i = 0; i < n; ++i)
    if (m == 0 || cut[i] != bk[m - 1]) {
      if (m > kMaxSplitK) return 0;
      bk[m++] = cut[i];
    }
  const int n_sh = m - 1;
  int ord[kMaxSplitK];
  for (int i = 0; i < n_sh; ++i) ord[i] = i;
  for (int i = 1; i < n_sh; ++i)  // stable: longer first, then in k order
    for (int k = i; k > 0 && bk[ord[k] + 1] - bk[ord[k]] > bk[ord[k - 1] + 1] - bk[ord[k - 1]]; --k) {
      const int t = ord[k]; ord[k] = ord[k - 1]; ord[k - 1] = t;
    }
  for (int i = 0; i < n_sh; ++i) {
    bb[i] = bk[ord[i]];
    be[i] = bk[ord[i] + 1];
    bseg[i] = bk[ord[i]] / (ksteps / segs);
  }
  return n_sh;
}

// The K split of a non-argmax contraction: 0 when it should not split (and
// cannot take a deferred-scale operand), else the share count, the ranges in
// bb / be / bseg when given.
static int big_split_plan(const GemmParams& p, int segs, int* bb, int* be, int* bseg) {
  // the gate/up pair measured faster on the 128 x 64 register-fed tiles
  // (67.6 us against 76 us split at 448 rows)
  if (p.epi.kind == EPI_SWIGLU || epi_rowred(p.epi.kind)) return 0;
  if (!p.split_ws || p.N % 4 || (int64_t)p.M * p.N >= ((int64_t)1 << 31)) return 0;  // the reduce indexes in 32 bits
  const int ksteps = p.K / 32;
  if (segs > 1 && (ksteps % segs || segs > kMaxSplitK)) return 0;  // segments of whole k-steps
  const int bm = rows224(p.M) ? 224 : 256;
  const int tiles = ((p.N + 127) / 128) * ((p.M + bm - 1) / bm);
  const int64_t per = (int64_t)p.M * p.N * 4;
  int splits = (PE_SPLIT_SLOTS + tiles - 1) / tiles;
  splits = min(splits, PE_SPLIT_MAX);
  splits = min(splits, ksteps / PE_SPLIT_MINSTEPS);
  if (segs <= 1) {
    while (splits > 1 && (int64_t)splits * per > p.split_cap) --splits;
    return splits >= 2 ? splits : 0;
  }
  int tb[kMaxSplitK], te[kMaxSplitK], ts[kMaxSplitK];
  if (!bb) { bb = tb; be = te; bseg = ts; }
  for (int base = max(splits, 1); base >= 1; --base) {
    const int n = split_ranges(ksteps, base, segs, bb, be, bseg);
    if (n >= 2 && (int64_t)n * per <= p.split_cap) return n;
  }
  return 0;
}

int gemm_big_splits(const GemmParams& p, int segs) { return big_split_plan(p, segs, nullptr, nullptr, nullptr); }

int launch_gemm_big(const GemmParams& p, hipStream_t s) {
  const bool r224 = rows224(p.M);
  if (epi_rowred(p.epi.kind)) {
    if (p.epi.kind == EPI_LSE) {
      if (p.x_packed)
        return r224 ? launch_big<224, 160, 2, 3, false, true, false, true, true>(p, 1, s)
                    : launch_big<256, 128, 2, 3, false, true, false, true, true>(p, 1, s);
      return r224 ? launch_big<224, 128, 2, 3, false, true, false, false, true>(p, 1, s)
                  : launch_big<256, 128, 2, 3, false, true, false, false, true>(p, 1, s);
    }
    if (p.x_packed)
      return r224 ? launch_big<224, 160, 2, 3, false, true, false, true>(p, 1, s)
                  : launch_big<256, 128, 2, 3, false, true, false, true>(p, 1, s);
    return r224 ? launch_big<224, 128, 2, 3, false, true, false>(p, 1, s)
                : launch_big<256, 128, 2, 3, false, true, false>(p, 1, s);
  }
  GemmParams q = p;
  const int splits = big_split_plan(p, p.xinv ? p.xinv_segs : 1, q.split_beg, q.split_end, q.split_seg);
  if (!splits) return -1;  // the caller's 128-tile kernel keeps the contraction
  q.nsplit_k = (p.xinv && p.xinv_segs > 1) ? splits : 0;
  if (p.x_packed) {
    if (r224) launch_big<224, 128, 2, PE_SPLIT_STAGES, false, false, true, true>(q, splits, s);
    else launch_big<256, 128, 2, PE_SPLIT_STAGES, false, false, true, true>(q, splits, s);
  } else {
    if (r224) launch_big<224, 128, 2, PE_SPLIT_STAGES, false, false, true>(q, splits, s);
    else launch_big<256, 128, 2, PE_SPLIT_STAGES, false, false, true>(q, splits, s);
  }
  launch_splitk_reduce(q, splits, s);
  return 0;
}

int64_t gemm_split_bytes(int T, int nmax) {
  if (T < 128) return 0;
  const int64_t full = (int64_t)8 * T * nmax * 4 * 2;  // 8 splits of a gate/up pair
  return full < ((int64_t)64 << 20) ? full : ((int64_t)64 << 20);
}

}  // namespace pe
