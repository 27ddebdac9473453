// Dense contractions of the drafter on the gfx950 matrix cores:
//   Y[m][n] = sum_k X[m][k] * W[n][k]      X: activations [M, K], W: weights [N, K]
// followed by a fused epilogue (embedding add, KV-cache scatter, residual add,
// SiLU-gated product, or a running argmax for the LM head).
//
// Weights are streamed from a packed, matrix-core-ready layout (pack_kernel):
// rows are padded to a multiple of 16 and, for row block b and 64-byte step s
// of a row, one contiguous 1 KB chunk at byte ((b * S + s) * 1024) holds the
// MFMA A operand of that step in lane order: lane l's 16 bytes are bytes
// [16*(l/16), 16*(l/16)+16) of step s of row 16b + l%16.  A wave therefore
// reads each weight chunk with one perfectly contiguous 1 KB load and feeds it
// to the MFMA as is; measured on MI355X this streams at ~6.1 TB/s, against
// ~5.3-5.8 TB/s for any row-major mapping.
//
// Contraction-index assignment (A and B alike): in step s, lane group g holds
// elements [s*4*CH + g*CH, +CH) of its row; the 16x16 result lands as
// D[4g+j][r] = (feature 4g+j of the block, activation row r).
//
//  * gemm_stream_kernel (M <= 16, decode shapes): a workgroup owns a 16-row
//    weight block, its KS waves split K and reduce through LDS.  Activation
//    rows (the B operand) are read from L2; padding rows from a zero buffer.
//  * lm_argmax_stream_kernel (M <= 16): the LM head with a running argmax.
//  * gemm_tiled_kernel (larger M): BM x BN output tiles; activation k-tiles
//    staged through LDS, weight operands loaded straight from the packed
//    chunks into registers with a one-tile prefetch.  Workgroup ids map the M
//    tiles of one N tile back to back onto one XCD (workgroup i runs on XCD
//    i % 8) so the weight chunks are fetched from HBM once.
#include <math.h>
#include "kernels.h"

namespace pe {

__device__ __forceinline__ u32x4 zero4() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }

// ---------------------------------------------------------------------------
// Weight packing (one thread per 16-byte output chunk; rows >= N are zero).
__global__ __launch_bounds__(256) void pack_kernel(const char* __restrict__ src, char* __restrict__ dst, int N,
                                                   int row_bytes, int64_t total16) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total16) return;
  const int S = row_bytes / 64;
  const int l = (int)(idx & 63);
  const int64_t c = idx >> 6;
  const int s = (int)(c % S);
  const int64_t b = c / S;
  const int64_t row = 16 * b + (l & 15);
  u32x4 v = zero4();
  if (row < N) v = ld16(src + row * row_bytes + s * 64 + (l >> 4) * 16);
  st16(dst + idx * 16, v);
}

void launch_pack(const void* src, void* dst, int N, int row_bytes, hipStream_t s) {
  const int64_t total16 = (int64_t)((N + 15) / 16) * (row_bytes / 64) * 64;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((total16 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const char*>(src), reinterpret_cast<char*>(dst), N, row_bytes, total16);
}

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
      reinterpret_cast<S*>(e.out_s)[(int64_t)m * e.ld_out + n] = Storage<S>::from_f32(si * y2);
      break;
    }
    default:
      break;
  }
}

// ---------------------------------------------------------------------------
// Activation rows staged in LDS by the LM-head kernel (row pitch xp bytes,
// a zero chunk at xs + M*xp for the padding rows of the 16-row operand).
// Ends with a workgroup barrier.
template <typename S>
__device__ void stage_rows(const GemmParams& p, char* xs, int xp) {
  constexpr int CH = Storage<S>::CH;
  const int cpr = p.K * (int)sizeof(S) / 16;  // 16-byte chunks per row
  const S* X = reinterpret_cast<const S*>(p.X);
  for (int c = threadIdx.x; c < p.M * cpr; c += blockDim.x) {
    const int row = c / cpr, col = c % cpr;
    *reinterpret_cast<u32x4*>(xs + row * xp + col * 16) = ld16(X + (int64_t)row * p.ldx + col * CH);
  }
  if (threadIdx.x == 0) *reinterpret_cast<u32x4*>(xs + p.M * xp) = zero4();
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Weight-streaming contraction for M <= 16.  Workgroup fb of KS waves owns the
// 16-row weight block fb; wave ks takes the ks-th share of the K steps.  Each
// wave issues U one-kilobyte weight loads (and the matching activation loads)
// back to back before its first matrix-core step; the last batch re-reads its
// final step for the slots past the end and skips their matrix-core steps, so
// the loop has no data-dependent branch.  The KS partial tiles are summed
// through LDS in ks order.  No cross-workgroup reduction: a device-scope
// fence on MI355X writes back the XCD's L2 and stalls the stream.
template <typename S, int KS, int U, bool DUAL>
__global__ __launch_bounds__(64 * KS) void gemm_stream_kernel(GemmParams p) {
  constexpr int CH = Storage<S>::CH;
  constexpr int STEP = 4 * CH;
  const int lane = threadIdx.x & 63;
  const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int nsteps = K / STEP;
  const int fb = blockIdx.x;
  const int s0 = (int)((int64_t)nsteps * ks / KS);
  const int s1 = (int)((int64_t)nsteps * (ks + 1) / KS);
  const bool xr = r < M;
  // padding rows of the 16-row B operand read a zeroed buffer: no branch in the loop
  const S* xrow = (xr ? reinterpret_cast<const S*>(p.X) + (int64_t)r * p.ldx : reinterpret_cast<const S*>(p.xzero)) + g * CH;
  const char* wb = reinterpret_cast<const char*>(p.W) + (int64_t)fb * nsteps * 1024 + lane * 16;
  const char* wb2 = reinterpret_cast<const char*>(p.W2) + (int64_t)fb * nsteps * 1024 + lane * 16;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; s += U) {
    u32x4 wv[U], w2v[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = min(s + u, s1 - 1);
      wv[u] = ld16(wb + (int64_t)su * 1024);
      if constexpr (DUAL) w2v[u] = ld16(wb2 + (int64_t)su * 1024);
      xv[u] = ld16(xrow + su * STEP);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < s1) {
        mma16(acc, wv[u], xv[u], S());
        if constexpr (DUAL) mma16(acc2, w2v[u], xv[u], S());
      }
    }
  }
  if constexpr (KS > 1) {
    __shared__ f32x4 red[(KS - 1) * 64 * (DUAL ? 2 : 1)];
    if (ks > 0) {
      red[(ks - 1) * 64 + lane] = acc;
      if constexpr (DUAL) red[((KS - 1) + ks - 1) * 64 + lane] = acc2;
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int k = 0; k < KS - 1; ++k) {
      acc += red[k * 64 + lane];
      if constexpr (DUAL) acc2 += red[((KS - 1) + k) * 64 + lane];
    }
  }
  if (xr) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = fb * 16 + 4 * g + j;
      if (n < N) epi_store<S>(p.epi, r, n, acc[j], acc2[j]);
    }
  }
}

// LM head for M <= 16: grid-stride over groups of NFB weight blocks; KS waves
// per block split K and sum through LDS in ks order.  With XL the M
// activation rows are staged once per workgroup in LDS by stage_rows (row
// pitch K + 16 bytes, so the 16 lanes of one k-chunk hit distinct banks);
// without it (rows too wide for LDS) they are read from global memory,
// padding rows from the zeroed buffer p.xzero.  Each wave streams its
// weight steps in double-buffered batches of U: batch j+1 is in flight while
// batch j is multiplied.  Each lane of the block's
// first wave keeps the best (logit, lowest index) of its activation row; the
// workgroup's best per row goes to partial slot [blockIdx][row], reduced by
// argmax_reduce_kernel.
template <typename S, int NFB, int KS, int U, bool XL>
__global__ __launch_bounds__(64 * NFB * KS) void lm_argmax_stream_kernel(GemmParams p) {
  constexpr int CH = Storage<S>::CH;
  constexpr int STEP = 4 * CH;
  constexpr int NW = NFB * KS;
  extern __shared__ __attribute__((aligned(16))) char xs[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fbl = wave / KS, ks = wave % KS;
  const int r = lane & 15, g = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int nsteps = K / STEP;
  const int s0 = nsteps * ks / KS, s1 = nsteps * (ks + 1) / KS;
  const int nfb = (N + 15) >> 4;
  const int ntiles = (nfb + NFB - 1) / NFB;
  const bool xr = r < M;
  const char* xrow;
  int xstep;  // bytes per step (0: padding rows stay on a zero chunk)
  if constexpr (XL) {
    const int xp = K * (int)sizeof(S) + 16;  // LDS row pitch, bytes
    stage_rows<S>(p, xs, xp);
    xrow = xr ? xs + r * xp + g * 16 : xs + M * xp;
    xstep = xr ? STEP * (int)sizeof(S) : 0;
  } else {
    xrow = xr ? reinterpret_cast<const char*>(reinterpret_cast<const S*>(p.X) + (int64_t)r * p.ldx + g * CH)
              : reinterpret_cast<const char*>(p.xzero) + g * 16;
    xstep = STEP * (int)sizeof(S);  // p.xzero holds >= K zeroed elements
  }
  const char* W = reinterpret_cast<const char*>(p.W) + lane * 16;
  __shared__ f32x4 red[KS > 1 ? NFB * (KS - 1) * 64 : 1];
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  const int nb = (s1 - s0 + U - 1) / U;  // batches per wave
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int fb = tile * NFB + fbl;
    const bool active = fb < nfb;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      const char* wb = W + (int64_t)fb * nsteps * 1024;
      u32x4 wv[2][U];
      auto wload = [&](int j, int slot) {
#pragma unroll
        for (int u = 0; u < U; ++u) wv[slot][u] = ld16(wb + (int64_t)min(s0 + j * U + u, s1 - 1) * 1024);
      };
      auto batch = [&](int j, int slot) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int su = s0 + j * U + u;
          if (su < s1) mma16(acc, wv[slot][u], ld16(xrow + (int64_t)su * xstep), S());
        }
      };
      wload(0, 0);
      for (int j = 0; j < nb; j += 2) {
        if (j + 1 < nb) wload(j + 1, 1);
        batch(j, 0);
        if (j + 2 < nb) wload(j + 2, 0);
        if (j + 1 < nb) batch(j + 1, 1);
      }
    }
    if constexpr (KS > 1) {
      if (ks > 0 && active) red[(fbl * (KS - 1) + ks - 1) * 64 + lane] = acc;
      __syncthreads();
      if (ks == 0 && active) {
#pragma unroll
        for (int k = 0; k < KS - 1; ++k) acc += red[(fbl * (KS - 1) + k) * 64 + lane];
      }
      __syncthreads();
    }
    if (ks == 0 && active && xr) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = fb * 16 + 4 * g + j;
        if (n >= N) continue;
        if (p.epi.logits) p.epi.logits[(int64_t)r * N + n] = acc[j];
        if (better(acc[j], n, best, bidx)) { best = acc[j]; bidx = n; }
      }
    }
  }
  for (int o = 16; o < 64; o <<= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bidx, o, 64);
    if (better(ov, oi, best, bidx)) { best = ov; bidx = oi; }
  }
  __shared__ float sbv[NW][16];
  __shared__ int sbi[NW][16];
  if (g == 0) { sbv[wave][r] = best; sbi[wave][r] = bidx; }
  __syncthreads();
  if ((int)threadIdx.x < M) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int w = 0; w < NW; ++w)
      if (better(sbv[w][threadIdx.x], sbi[w][threadIdx.x], bv, bi)) { bv = sbv[w][threadIdx.x]; bi = sbi[w][threadIdx.x]; }
    p.epi.part_val[(int64_t)blockIdx.x * M + threadIdx.x] = bv;
    p.epi.part_idx[(int64_t)blockIdx.x * M + threadIdx.x] = bi;
  }
}

// ---------------------------------------------------------------------------
template <typename S, int BM, int BN, bool DUAL, bool ARGMAX>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmParams p, int n_ft, int n_mt) {
  constexpr int CH = Storage<S>::CH;
  constexpr int BKC = 8;             // 16-byte chunks per activation row per k-tile (two steps)
  constexpr int BK = BKC * CH;
  constexpr int PITCH = BKC + 1;     // LDS row pitch in 16-byte units
  constexpr int FBW = BN / 32, RBW = BM / 32;
  constexpr int XPT = BM * BKC / 256;
  static_assert(XPT * 256 == BM * BKC, "tile/thread mismatch");
  __shared__ u32x4 Xs[BM * PITCH];

  const int bid = blockIdx.x;
  const int xcd = bid & 7, jj = bid >> 3;
  const int mt = jj % n_mt;
  const int ft = (jj / n_mt) * 8 + xcd;
  if (ft >= n_ft) return;
  const int M = p.M, N = p.N, K = p.K;
  const int nsteps = K / (4 * CH);
  const int nfb = (N + 15) >> 4;
  const int n0 = ft * BN, m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const S* X = reinterpret_cast<const S*>(p.X);
  const char* Wl = reinterpret_cast<const char*>(p.W) + lane * 16;
  const char* W2l = reinterpret_cast<const char*>(p.W2) + lane * 16;

  // weight blocks of this wave (clamped; blocks past N feed columns the epilogue drops)
  int64_t wofs[FBW];
#pragma unroll
  for (int f = 0; f < FBW; ++f) wofs[f] = (int64_t)min(n0 / 16 + wn * FBW + f, nfb - 1) * nsteps * 1024;

  f32x4 acc[FBW][RBW], acc2[DUAL ? FBW : 1][DUAL ? RBW : 1];
#pragma unroll
  for (int a = 0; a < FBW; ++a)
#pragma unroll
    for (int b = 0; b < RBW; ++b) {
      acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (DUAL) acc2[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  u32x4 xreg[XPT];
  u32x4 wcur[2][FBW], w2cur[DUAL ? 2 : 1][DUAL ? FBW : 1];
  const int nkt = (nsteps + 1) / 2;
  auto xload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * 256;
      const int row = c / BKC, col = c % BKC;
      const int m = m0 + row;
      const int k = kt * BK + col * CH;
      xreg[i] = (m < M && k < K) ? ld16(X + (int64_t)m * p.ldx + k) : zero4();
    }
  };
  auto wload = [&](int kt) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int s = min(kt * 2 + st, nsteps - 1);   // a half tile repeats its last step; zero X makes it inert
#pragma unroll
      for (int f = 0; f < FBW; ++f) {
        wcur[st][f] = ld16(Wl + wofs[f] + (int64_t)s * 1024);
        if constexpr (DUAL) w2cur[st][f] = ld16(W2l + wofs[f] + (int64_t)s * 1024);
      }
    }
  };

  xload(0);
  wload(0);
  for (int kt = 0; kt < nkt; ++kt) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * 256;
      Xs[(c / BKC) * PITCH + c % BKC] = xreg[i];
    }
    __syncthreads();
    u32x4 wuse[2][FBW], w2use[DUAL ? 2 : 1][DUAL ? FBW : 1];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int f = 0; f < FBW; ++f) {
        wuse[st][f] = wcur[st][f];
        if constexpr (DUAL) w2use[st][f] = w2cur[st][f];
      }
    if (kt + 1 < nkt) {
      xload(kt + 1);
      wload(kt + 1);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4 b[RBW];
#pragma unroll
      for (int q = 0; q < RBW; ++q) b[q] = Xs[(wm * (BM / 2) + q * 16 + r) * PITCH + st * 4 + g];
#pragma unroll
      for (int f = 0; f < FBW; ++f)
#pragma unroll
        for (int q = 0; q < RBW; ++q) {
          mma16(acc[f][q], wuse[st][f], b[q], S());
          if constexpr (DUAL) mma16(acc2[f][q], w2use[st][f], b[q], S());
        }
    }
    __syncthreads();
  }

  if constexpr (ARGMAX) {
    __shared__ float sbv[2][BM];
    __shared__ int sbi[2][BM];
#pragma unroll
    for (int q = 0; q < RBW; ++q) {
      const int mloc = wm * (BM / 2) + q * 16 + r;
      const int m = m0 + mloc;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int f = 0; f < FBW; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * (BN / 2) + f * 16 + 4 * g + j;
          if (n < N && m < M) {
            const float v = acc[f][q][j];
            if (p.epi.logits) p.epi.logits[(int64_t)m * N + n] = v;
            if (better(v, n, bv, bi)) { bv = v; bi = n; }
          }
        }
      for (int o = 16; o < 64; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (g == 0) { sbv[wn][mloc] = bv; sbi[wn][mloc] = bi; }
    }
    __syncthreads();
    if (tid < BM && m0 + tid < M) {
      float bv = sbv[0][tid];
      int bi = sbi[0][tid];
      if (better(sbv[1][tid], sbi[1][tid], bv, bi)) { bv = sbv[1][tid]; bi = sbi[1][tid]; }
      p.epi.part_val[(int64_t)ft * M + m0 + tid] = bv;
      p.epi.part_idx[(int64_t)ft * M + m0 + tid] = bi;
    }
  } else {
#pragma unroll
    for (int f = 0; f < FBW; ++f)
#pragma unroll
      for (int q = 0; q < RBW; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * (BN / 2) + f * 16 + 4 * g + j;
          const int m = m0 + wm * (BM / 2) + q * 16 + r;
          if (n < N && m < M) epi_store<S>(p.epi, m, n, acc[f][q][j], DUAL ? acc2[DUAL ? f : 0][DUAL ? q : 0][j] : 0.f);
        }
  }
}

__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float* pv, const int32_t* pi, int P, int M,
                                                            int32_t* tokens) {
  const int m = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int q = threadIdx.x; q < P; q += 4 * 256) {
    float v[4];
    int ix[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int qq = q + 256 * u;
      v[u] = qq < P ? pv[(int64_t)qq * M + m] : -INFINITY;
      ix[u] = qq < P ? pi[(int64_t)qq * M + m] : 0x7fffffff;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (better(v[u], ix[u], bv, bi)) { bv = v[u]; bi = ix[u]; }
  }
  for (int o = 1; o < 64; o <<= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    tokens[m] = (bi == 0x7fffffff) ? -1 : bi;
  }
}

void launch_argmax_reduce(const float* pv, const int32_t* pi, int P, int M, int32_t* tokens, hipStream_t s) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(M), dim3(256), 0, s, pv, pi, P, M, tokens);
}

// ---------------------------------------------------------------------------
// Dispatch
static constexpr int kStreamU = 8;     // 1 KB steps in flight per wave
// LM-head launch shape: NFB blocks x KS waves per workgroup, grid capped at kLmGrid.
#ifndef PE_LM_NFB
#define PE_LM_NFB 4
#endif
#ifndef PE_LM_KS
#define PE_LM_KS 2
#endif
#ifndef PE_LM_GRID
#define PE_LM_GRID 1024
#endif
#ifndef PE_LM_U
#define PE_LM_U 8
#endif
static constexpr int kLmNFB = PE_LM_NFB, kLmKS = PE_LM_KS, kLmGrid = PE_LM_GRID, kLmU = PE_LM_U;
// Largest activation block the LM-head kernel stages in LDS (its own arrays
// take a few KB of the 160 KB); wider rows are read from global memory.
static constexpr int kLmXLds = 144 * 1024;

// Waves per 16-row block: the most (up to 16) that still leave every wave at
// least one full batch of kStreamU steps.
static int stream_ks(int nsteps) {
  int ks = 16;
  while (ks > 1 && nsteps / ks < kStreamU) ks >>= 1;
  return ks;
}

int gemm_argmax_partials(int M, int N) {
  if (M <= 16) {
    const int ntiles = ((N + 15) / 16 + kLmNFB - 1) / kLmNFB;
    return ntiles < kLmGrid ? ntiles : kLmGrid;
  }
  return (N + 63) / 64;  // largest count over the tiled configurations (BN >= 64)
}

template <typename S, int BM, int BN, bool DUAL, bool ARGMAX>
static int launch_tiled(const GemmParams& p, hipStream_t s) {
  const int n_ft = (p.N + BN - 1) / BN, n_mt = (p.M + BM - 1) / BM;
  const int grid = ((n_ft + 7) / 8) * 8 * n_mt;
  hipLaunchKernelGGL((gemm_tiled_kernel<S, BM, BN, DUAL, ARGMAX>), dim3(grid), dim3(256), 0, s, p, n_ft, n_mt);
  return n_ft;
}

// Raises kernel K's dynamic LDS limit once (the default may be below what
// the activation block needs); one flag per kernel.
template <auto K>
static void allow_lds(int bytes) {
  static bool done = false;
  if (!done) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(K), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    done = true;
  }
}

template <typename S, bool DUAL>
static void launch_stream(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.N + 15) / 16);
  switch (stream_ks(p.K / (4 * Storage<S>::CH))) {
    case 16: hipLaunchKernelGGL((gemm_stream_kernel<S, 16, kStreamU, DUAL>), grid, dim3(1024), 0, s, p); break;
    case 8: hipLaunchKernelGGL((gemm_stream_kernel<S, 8, kStreamU, DUAL>), grid, dim3(512), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_stream_kernel<S, 4, kStreamU, DUAL>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_stream_kernel<S, 2, kStreamU, DUAL>), grid, dim3(128), 0, s, p); break;
    default: hipLaunchKernelGGL((gemm_stream_kernel<S, 1, kStreamU, DUAL>), grid, dim3(64), 0, s, p); break;
  }
}

template <typename S>
static int launch_gemm_t(const GemmParams& p, hipStream_t s) {
  const bool dual = p.epi.kind == EPI_SWIGLU;
  const bool am = p.epi.kind == EPI_ARGMAX;
  if (p.M <= 16) {
    if (am) {
      const int grid = gemm_argmax_partials(p.M, p.N);
      const size_t lds = (size_t)p.M * (p.K * sizeof(S) + 16) + 16;  // activation rows + zero chunk
      if (lds <= (size_t)kLmXLds) {
        allow_lds<&lm_argmax_stream_kernel<S, kLmNFB, kLmKS, kLmU, true>>(kLmXLds);
        hipLaunchKernelGGL((lm_argmax_stream_kernel<S, kLmNFB, kLmKS, kLmU, true>), dim3(grid),
                           dim3(64 * kLmNFB * kLmKS), lds, s, p);
      } else {
        hipLaunchKernelGGL((lm_argmax_stream_kernel<S, kLmNFB, kLmKS, kLmU, false>), dim3(grid),
                           dim3(64 * kLmNFB * kLmKS), 0, s, p);
      }
      return grid;
    }
    if (dual) launch_stream<S, true>(p, s); else launch_stream<S, false>(p, s);
    return 0;
  }
  const bool big = p.M >= 256;
  if (am) return big ? launch_tiled<S, 128, 128, false, true>(p, s) : launch_tiled<S, 64, 64, false, true>(p, s);
  if (dual) { if (big) launch_tiled<S, 128, 64, true, false>(p, s); else launch_tiled<S, 64, 64, true, false>(p, s); }
  else { if (big) launch_tiled<S, 128, 128, false, false>(p, s); else launch_tiled<S, 64, 64, false, false>(p, s); }
  return 0;
}

int launch_gemm(const GemmParams& p, int bf16, hipStream_t s) {
  return bf16 ? launch_gemm_t<uint16_t>(p, s) : launch_gemm_t<float>(p, s);
}

}  // namespace pe
