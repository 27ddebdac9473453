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
#include <type_traits>
#include "epilogue.h"

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

// ---------------------------------------------------------------------------
// Activation staging of the weight-streaming kernels: the M rows of X are
// written to LDS in the operand type S, row pitch xp bytes.  Neither function
// ends with a barrier.

// Element e of a 16-byte chunk of XT values, as float.
template <typename XT>
__device__ __forceinline__ float chunk_elem(const u32x4& v, int e) {
  if constexpr (sizeof(XT) == 2) return bf2f((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
  else return __uint_as_float(v[e]);
}

// Staging runs in two phases so that a kernel can request its first weight
// batches in between: load() issues the global reads of the first round into
// registers, finish() writes them to LDS and runs any further rounds.  The
// memory counter retires loads in issue order, so activation reads issued
// after a weight batch would wait for that batch.

// Plain copy (X already holds S): NCP sixteen-byte chunks per thread per round.
template <typename S, int NCP>
struct CopyStage {
  u32x4 v[NCP];
  __device__ void load_round(const GemmParams& p, int base) {
    const int cpr = p.K * (int)sizeof(S) / 16;
    const int total = p.M * cpr;
    const char* X = reinterpret_cast<const char*>(p.X);
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int c = min(base + (int)threadIdx.x + i * (int)blockDim.x, total - 1);
      const int row = c / cpr, col = c - row * cpr;
      v[i] = ld16(X + (int64_t)row * p.ldx * (int64_t)sizeof(S) + (int64_t)col * 16);
    }
  }
  __device__ void store_round(const GemmParams& p, char* xs, int xp, int base) {
    const int cpr = p.K * (int)sizeof(S) / 16;
    const int total = p.M * cpr;
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int c = base + (int)threadIdx.x + i * (int)blockDim.x;
      if (c < total) {
        const int row = c / cpr, col = c - row * cpr;
        *reinterpret_cast<u32x4*>(xs + row * xp + col * 16) = v[i];
      }
    }
  }
  __device__ void load(const GemmParams& p) { load_round(p, 0); }
  __device__ void finish(const GemmParams& p, char* xs, int xp) {
    const int total = p.M * (p.K * (int)sizeof(S) / 16);
    const int round = NCP * (int)blockDim.x;
    store_round(p, xs, xp, 0);
    for (int base = round; base < total; base += round) {
      load_round(p, base);
      store_round(p, xs, xp, base);
    }
  }
};

// RMSNorm on the way in ("Attention Drift", section 4.1: RMS = ||x||_2 /
// sqrt(d), each segment on its own): y = (x * inv) * g, the expression
// rmsnorm_rows_kernel evaluates; skipped rows become zeros.  One wave per
// (row, segment) pair, pairs wave, wave + nw, ...; a segment's NC chunks per
// lane stay in registers between the sum of squares and the scaled store.
// The gains (segs * seg_len floats) are copied to LDS at xg by all threads
// in the same first round.  All global reads are unconditional 16-byte loads
// (indices clamped), so none of them waits behind a branch.  finish() has a
// barrier between the gain copy and its use.  With p.nrm.defer the rows are
// written as x * g and each (row, segment)'s 1 / rms goes to the float array
// after the gains (index row * segs + seg), for the contraction to apply.
template <typename S, typename XT, int NC, bool HL = false>
struct NormStage {
  static constexpr int CI = 16 / sizeof(XT);  // elements per chunk
  static constexpr int GN = 3;                // gain chunks per thread per round
  static_assert(sizeof(S) <= sizeof(XT), "the operand type is never wider than the input");
  static_assert(!HL || (sizeof(S) == 2 && sizeof(XT) == 4), "a remainder row: float input, bf16 operand");
  u32x4 raw[NC];
  f32x4 gt[GN];
  __device__ void load_pair(const GemmParams& p, int pr) {
    const int lane = threadIdx.x & 63;
    const int segs = p.nrm.segs, sl = p.nrm.seg_len, cps = sl / CI;
    const int row = pr / segs, seg = pr - row * segs;
    const char* x = reinterpret_cast<const char*>(p.X) + ((int64_t)row * p.ldx + (int64_t)seg * sl) * (int64_t)sizeof(XT);
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] = ld16(x + (int64_t)min(lane + 64 * c, cps - 1) * 16);
  }
  __device__ void load_gains(const GemmParams& p, int base) {
    const int gch = p.nrm.segs * p.nrm.seg_len / 4;
#pragma unroll
    for (int i = 0; i < GN; ++i)
      gt[i] = *reinterpret_cast<const f32x4*>(p.nrm.gain + 4 * min(base + (int)threadIdx.x + i * (int)blockDim.x, gch - 1));
  }
  __device__ void store_gains(const GemmParams& p, char* xg, int base) {
    const int gch = p.nrm.segs * p.nrm.seg_len / 4;
#pragma unroll
    for (int i = 0; i < GN; ++i) {
      const int c = base + (int)threadIdx.x + i * (int)blockDim.x;
      if (c < gch) *reinterpret_cast<f32x4*>(xg + 16 * c) = gt[i];
    }
  }
  __device__ void store_pair(const GemmParams& p, char* xs, int xp, const char* xg, int pr) {
    const int lane = threadIdx.x & 63;
    const int segs = p.nrm.segs, sl = p.nrm.seg_len, cps = sl / CI;
    const int row = pr / segs, seg = pr - row * segs;
    const bool skip = p.nrm.skip && p.nrm.skip[row];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bool ok = lane + 64 * c < cps && !skip;
#pragma unroll
      for (int e = 0; e < CI; ++e) {
        const float f = ok ? chunk_elem<XT>(raw[c], e) : 0.f;
        ss += f * f;
      }
    }
    ss = wave_sum(ss);
    const float inv0 = skip ? 0.f : 1.0f / sqrtf(ss / (float)sl + p.nrm.eps);
    if (p.nrm.defer && lane == 0)
      reinterpret_cast<float*>(const_cast<char*>(xg) + segs * sl * 4)[row * segs + seg] = inv0;
    const float inv = p.nrm.defer ? 1.f : inv0;
    char* dst = xs + row * xp + seg * sl * (int)sizeof(S);
    const char* gsrc = xg + seg * sl * 4;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = lane + 64 * c;
      if (ch < cps) {
        const int e0 = ch * CI;
        float y[CI];
#pragma unroll
        for (int q = 0; q < CI / 4; ++q) {
          const f32x4 gq = *reinterpret_cast<const f32x4*>(gsrc + (e0 + 4 * q) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[4 * q + e] = (skip ? 0.f : chunk_elem<XT>(raw[c], 4 * q + e)) * inv * gq[e];
        }
        if constexpr (sizeof(S) == 4) {
          f32x4 w = {y[0], y[1], y[2], y[3]};
          *reinterpret_cast<f32x4*>(dst + e0 * 4) = w;
        } else if constexpr (CI == 8) {
          u32x4 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                     pack_bf16x2(y[6], y[7])};
          *reinterpret_cast<u32x4*>(dst + e0 * 2) = w;
        } else {
          u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
          *reinterpret_cast<u32x2*>(dst + e0 * 2) = w;
          if constexpr (HL) {
            // the remainder y - bf16(y) (exact in fp32) rounded to bf16, in row + 8
            float lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) lo[e] = y[e] - bf2f((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
            *reinterpret_cast<u32x2*>(dst + 8 * xp + e0 * 2) = u32x2{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
          }
        }
      }
    }
  }
  __device__ void load(const GemmParams& p, int wave) {
    if (wave < p.M * p.nrm.segs) load_pair(p, wave);
    load_gains(p, 0);
  }
  __device__ void finish(const GemmParams& p, char* xs, int xp, char* xg, int wave, int nw) {
    const int gch = p.nrm.segs * p.nrm.seg_len / 4;
    const int round = GN * (int)blockDim.x;
    store_gains(p, xg, 0);
    for (int base = round; base < gch; base += round) {
      load_gains(p, base);
      store_gains(p, xg, base);
    }
    __syncthreads();
    const int np = p.M * p.nrm.segs;
    if (wave < np) store_pair(p, xs, xp, xg, wave);
    for (int pr = wave + nw; pr < np; pr += nw) {
      load_pair(p, pr);
      store_pair(p, xs, xp, xg, pr);
    }
  }
};

// Chunks per lane held by NormStage: a segment of up to 3,072 elements.
template <typename XT>
constexpr int norm_chunks() { return 3 * (int)sizeof(XT); }

// Steps per wave of gemm_stream_fnorm_kernel (its gains live in LDS).
constexpr int kFnormMaxSteps = 16;

__device__ __forceinline__ void clear_ints(const GemmParams& p) {
  if (p.clear && blockIdx.x == 0)
    for (int j = threadIdx.x; j < p.nclear; j += blockDim.x) p.clear[j] = 0;
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
// LOM: the operand is X + p.x_lo.  1: each weight chunk multiplied by both
// parts; 2 (M <= 8): the remainder rows take columns 8..15 of the 16-row
// operand (lane r >= 8 reads row r - 8 of x_lo), one matrix-core step per
// chunk, and the two halves of the result tile are added at the end.
// p.xinv: deferred 1 / rms per (row, segment); KS is then a multiple of the
// segment count, so every wave's steps lie in one segment and its partial
// tile is scaled before the reduction.
template <typename S, int KS, int U, bool DUAL, int LOM>
__global__ __launch_bounds__(64 * KS) void gemm_stream_kernel(GemmParams p) {
  constexpr bool LO = LOM == 1;
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
  const int rm = LOM == 2 ? (r & 7) : r;  // activation row of this lane
  const bool xr = rm < M;
  // padding rows of the 16-row B operand read a zeroed buffer: no branch in the loop
  const S* xsrc = reinterpret_cast<const S*>(LOM == 2 && r >= 8 ? p.x_lo : p.X);
  const S* xrow = (xr ? xsrc + (int64_t)rm * p.ldx : reinterpret_cast<const S*>(p.xzero)) + g * CH;
  const S* xlrow = (xr && LO ? reinterpret_cast<const S*>(p.x_lo) + (int64_t)r * p.ldx : reinterpret_cast<const S*>(p.xzero)) + g * CH;
  const char* wb = reinterpret_cast<const char*>(p.W) + (int64_t)fb * nsteps * 1024 + lane * 16;
  const char* wb2 = reinterpret_cast<const char*>(p.W2) + (int64_t)fb * nsteps * 1024 + lane * 16;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; s += U) {
    u32x4 wv[U], w2v[U], xv[U], xl[LO ? U : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = min(s + u, s1 - 1);
      wv[u] = ld16(wb + (int64_t)su * 1024);
      if constexpr (DUAL) w2v[u] = ld16(wb2 + (int64_t)su * 1024);
      xv[u] = ld16(xrow + su * STEP);
      if constexpr (LO) xl[u] = ld16(xlrow + su * STEP);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < s1) {
        mma16(acc, wv[u], xv[u], S());
        if constexpr (DUAL) mma16(acc2, w2v[u], xv[u], S());
        if constexpr (LO) {
          mma16(acc, wv[u], xl[u], S());
          if constexpr (DUAL) mma16(acc2, w2v[u], xl[u], S());
        }
      }
    }
  }
  if (p.xinv) {
    // the segment of this wave's steps (all of them lie in one)
    const int seg = min(s0 * STEP / (K / p.xinv_segs), p.xinv_segs - 1);
    const float sc = xr ? p.xinv[r * p.xinv_segs + seg] : 0.f;
    acc *= sc;
    acc2 *= sc;
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
  if constexpr (LOM == 2) {
    // column r + 8 holds the remainder part of row r
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += __shfl_down(acc[j], 8, 64);
      if constexpr (DUAL) acc2[j] += __shfl_down(acc2[j], 8, 64);
    }
  }
  if (r < M) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = fb * 16 + 4 * g + j;
      if (n < N) epi_store<S>(p.epi, r, n, acc[j], acc2[j]);
    }
  }
}

// Weight-streaming contraction over RMS-normalised float rows (M <= 16, one
// segment): Y = W RMSNorm(X) with the norm folded into the stream,
//   Y[m][n] = inv[m] * sum_k W[n][k] * S(X[m][k] * g[k]),
//   inv[m] = 1 / sqrt(mean_k X[m][k]^2 + eps)          (zero for skipped rows)
// ("Attention Drift", section 4.1).  Each wave reads its share of the float
// rows with the weight steps (one round trip for both), multiplies by the
// gains of its K share, which it keeps in its own slice of LDS, accumulates
// the sum of squares of its elements, and the workgroup sums the partial
// tiles and partial sums of squares through LDS in a fixed order before the
// epilogue scales by inv.  The gain reads go out before the first weight
// batch, so waiting for them never waits for it.  HL (bf16): the operand is
// X * g as a bf16 value plus the bf16 of its remainder, two matrix-core
// steps per weight chunk, so the rounding of the float rows drops from 2^-9
// to about 2^-17 relative.
template <typename S, int KS, int U, bool DUAL, bool HL>
__global__ __launch_bounds__(64 * KS) __attribute__((amdgpu_waves_per_eu(4)))
void gemm_stream_fnorm_kernel(GemmParams p) {
  constexpr int CH = Storage<S>::CH;  // operand elements per lane per step
  constexpr int STEP = 4 * CH;
  constexpr int XQ = CH / 4;          // 16-byte float loads per lane per step
  // per wave: the gains of its steps (at most kFnormMaxSteps), then KS*64
  // partial sums of squares for the whole workgroup
  extern __shared__ __attribute__((aligned(16))) char gs[];
  const int lane = threadIdx.x & 63;
  const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int nsteps = K / STEP;
  const int fb = blockIdx.x;
  const int s0 = (int)((int64_t)nsteps * ks / KS);
  const int s1 = (int)((int64_t)nsteps * (ks + 1) / KS);
  const bool xr = r < M;
  const bool skip = xr && p.nrm.skip && p.nrm.skip[r];
  // padding rows read row M-1 (their columns of the tile are never stored)
  const char* xrow = reinterpret_cast<const char*>(reinterpret_cast<const float*>(p.X) +
                                                   (int64_t)(xr ? r : M - 1) * p.ldx + g * CH);
  const char* wb = reinterpret_cast<const char*>(p.W) + (int64_t)fb * nsteps * 1024 + lane * 16;
  const char* wb2 = reinterpret_cast<const char*>(p.W2) + (int64_t)fb * nsteps * 1024 + lane * 16;
  char* wg = gs + ks * (kFnormMaxSteps * STEP * 4);  // this wave's gains

  // this wave's gains: (s1 - s0) * STEP floats, two 16-byte chunks per lane
  const int gch = (s1 - s0) * STEP / 4;
  const float* gsrc = p.nrm.gain + s0 * STEP;
  f32x4 gt[kFnormMaxSteps * STEP / 256];
#pragma unroll
  for (int i = 0; i < kFnormMaxSteps * STEP / 256; ++i)
    gt[i] = *reinterpret_cast<const f32x4*>(gsrc + 4 * min(lane + 64 * i, gch - 1));

  u32x4 wv[U], w2v[U];
  f32x4 xv[U][XQ];
  auto load = [&](int s) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = min(s + u, s1 - 1);
      wv[u] = ld16(wb + (int64_t)su * 1024);
      if constexpr (DUAL) w2v[u] = ld16(wb2 + (int64_t)su * 1024);
#pragma unroll
      for (int q = 0; q < XQ; ++q) xv[u][q] = *reinterpret_cast<const f32x4*>(xrow + (int64_t)su * STEP * 4 + 16 * q);
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  int s = s0;
  if (s < s1) load(s);
#pragma unroll
  for (int i = 0; i < kFnormMaxSteps * STEP / 256; ++i)
    if (lane + 64 * i < gch) *reinterpret_cast<f32x4*>(wg + 16 * (lane + 64 * i)) = gt[i];
  __builtin_amdgcn_wave_barrier();  // LDS is in order within the wave
  while (s < s1) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < s1) {
        const int k0 = (s + u - s0) * STEP + g * CH;
        float y[CH];
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
          const f32x4 gq = *reinterpret_cast<const f32x4*>(wg + (k0 + 4 * q) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = xv[u][q][e];
            ss += x * x;
            y[4 * q + e] = x * gq[e];
          }
        }
        u32x4 b;
        if constexpr (CH == 8) {
          b = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
        } else {
          b = u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
        }
        if (skip) b = u32x4{0u, 0u, 0u, 0u};  // rejected rows contribute zeros whatever they hold
        mma16(acc, wv[u], b, S());
        if constexpr (DUAL) mma16(acc2, w2v[u], b, S());
        if constexpr (HL && CH == 8) {
          // remainder y - bf16(y) of each element (exact in fp32), rounded to bf16
          float lo[CH];
#pragma unroll
          for (int e = 0; e < CH; ++e) lo[e] = y[e] - bf2f((uint16_t)(b[e >> 1] >> (16 * (e & 1))));
          u32x4 bl = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(lo[4], lo[5]),
                      pack_bf16x2(lo[6], lo[7])};
          if (skip) bl = u32x4{0u, 0u, 0u, 0u};
          mma16(acc, wv[u], bl, S());
          if constexpr (DUAL) mma16(acc2, w2v[u], bl, S());
        }
      }
    }
    s += U;
    if (s < s1) load(s);
  }
  float* ssr = reinterpret_cast<float*>(gs + KS * (kFnormMaxSteps * STEP * 4));
  ssr[ks * 64 + lane] = ss;
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
  } else {
    __syncthreads();
  }
  if (xr) {
    // the row's sum of squares: every wave, every lane group, in a fixed order
    float tot = 0.f;
    for (int w = 0; w < KS; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) tot += ssr[w * 64 + q * 16 + r];
    const float inv = skip ? 0.f : 1.0f / sqrtf(tot / (float)K + p.nrm.eps);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = fb * 16 + 4 * g + j;
      if (n < N) epi_store<S>(p.epi, r, n, acc[j] * inv, acc2[j] * inv);
    }
  }
}

// The same contraction with the activation rows staged once per workgroup in
// LDS (row pitch K*elem + 16 bytes: the 16 lanes of one k-chunk hit distinct
// banks), RMS-normalised on the way when NORM.  The activation reads are
// issued first, then the first weight batch (and the second when EARLY2 and
// the registers allow), so the staging hides under the weight stream's first
// round trip; afterwards batch j+2 is in flight while batch j is multiplied.
// At most 128 registers per lane: two 512-thread workgroups per CU, so the
// 320-640 workgroups of the wide projections are resident at once.  With a
// deferred norm (p.nrm.defer) KS is a multiple of the segment count, every
// wave's steps lie in one segment, and its partial tile is scaled by that
// segment's 1 / rms before the reduction.
template <typename S, typename XT, int KS, int U, bool DUAL, bool NORM, bool EARLY2>
__global__ __launch_bounds__(64 * KS) __attribute__((amdgpu_waves_per_eu(4)))
void gemm_stream_lds_kernel(GemmParams p) {
  constexpr int CH = Storage<S>::CH;
  constexpr int STEP = 4 * CH;
  extern __shared__ __attribute__((aligned(16))) char xs[];
  const int lane = threadIdx.x & 63;
  const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int nsteps = K / STEP;
  const int fb = blockIdx.x;
  const int s0 = (int)((int64_t)nsteps * ks / KS);
  const int s1 = (int)((int64_t)nsteps * (ks + 1) / KS);
  const int nb = (s1 - s0 + U - 1) / U;  // batches of this wave
  const char* wb = reinterpret_cast<const char*>(p.W) + (int64_t)fb * nsteps * 1024 + lane * 16;
  const char* wb2 = reinterpret_cast<const char*>(p.W2) + (int64_t)fb * nsteps * 1024 + lane * 16;
  u32x4 wv[2][U], w2v[2][U];
  auto wload = [&](int j, int slot) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (int64_t)min(s0 + j * U + u, s1 - 1) * 1024;
      wv[slot][u] = ld16(wb + off);
      if constexpr (DUAL) w2v[slot][u] = ld16(wb2 + off);
    }
  };
  // activation reads first, then the weight batches (see CopyStage)
  const int xp = K * (int)sizeof(S) + 16;
  std::conditional_t<NORM, NormStage<S, XT, norm_chunks<XT>()>, CopyStage<S, 8>> stage;
  if constexpr (NORM) stage.load(p, ks); else stage.load(p);
  if (nb > 0) wload(0, 0);
  if constexpr (EARLY2) {
    if (nb > 1) wload(1, 1);
  }
  // LDS: M rows at pitch xp, the zero chunk, then the gains of a norm
  if constexpr (NORM) stage.finish(p, xs, xp, xs + M * xp + 16, ks, KS); else stage.finish(p, xs, xp);
  if constexpr (!EARLY2) {
    if (nb > 1) wload(1, 1);
  }
  clear_ints(p);
  if (threadIdx.x == 0) *reinterpret_cast<u32x4*>(xs + M * xp) = zero4();
  __syncthreads();

  const bool xr = r < M;
  const char* xrow = xr ? xs + r * xp + g * 16 : xs + M * xp;  // padding rows: the zero chunk
  const int xstep = xr ? STEP * (int)sizeof(S) : 0;
  float sc = 1.f;  // deferred 1 / rms of this wave's segment
  if (NORM && p.nrm.defer) {
    const int segs = p.nrm.segs;
    const float* sinv = reinterpret_cast<const float*>(xs + M * xp + 16 + segs * p.nrm.seg_len * 4);
    sc = xr ? sinv[r * segs + min(s0 * STEP / p.nrm.seg_len, segs - 1)] : 0.f;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
  auto batch = [&](int j, int slot) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = s0 + j * U + u;
      if (su < s1) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xrow + su * xstep);
        mma16(acc, wv[slot][u], xv, S());
        if constexpr (DUAL) mma16(acc2, w2v[slot][u], xv, S());
      }
    }
  };
  for (int j = 0; j < nb; j += 2) {
    batch(j, 0);
    if (j + 2 < nb) wload(j + 2, 0);
    if (j + 1 < nb) {
      batch(j + 1, 1);
      if (j + 3 < nb) wload(j + 3, 1);
    }
  }
  if (NORM && p.nrm.defer) {
    acc *= sc;
    acc2 *= sc;
  }
  if constexpr (KS > 1) {
    // the K-split partial tiles reuse the staged rows' LDS once every wave is done with them
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(xs);
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

// LM head for M <= 16 whose rows do not fit in LDS (XL false; staged rows go to
// lm_head_sweep_kernel): grid-stride over groups of NFB weight blocks; KS waves
// per block split K and sum through LDS in ks order.  With XL the M
// activation rows are staged once per workgroup in LDS, RMS-normalised on the
// way when NORM (row pitch K*elem + 16 bytes, so the 16 lanes of one k-chunk
// hit distinct banks);
// without it (rows too wide for LDS) they are read from global memory,
// padding rows from the zeroed buffer p.xzero.  Each wave streams its
// weight steps in double-buffered batches of U: batch j+1 is in flight while
// batch j is multiplied.  Each lane of the block's
// first wave keeps the best (logit, lowest index) of its activation row; the
// workgroup's best per row goes to partial slot [blockIdx][row], reduced by
// argmax_reduce_kernel.
// Two workgroups per CU (four waves per SIMD, at most 128 registers per lane)
// keep enough weight loads in flight.
#ifndef PE_LM_WPE
#define PE_LM_WPE 4
#endif
template <typename S, int NFB, int KS, int U, bool XL, bool NORM, bool LSE>
__global__ __launch_bounds__(64 * NFB * KS) __attribute__((amdgpu_waves_per_eu(PE_LM_WPE)))
void lm_argmax_stream_kernel(GemmParams p) {
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
  // k-steps of this wave: a contiguous share
  const int s0 = nsteps * ks / KS;
  const int sst = 1;
  const int cnt = nsteps * (ks + 1) / KS - s0;
  const int nfb = (N + 15) >> 4;
  const int ntiles = (nfb + NFB - 1) / NFB;
  const bool xr = r < M;
  const int nb = (cnt + U - 1) / U;  // batches per wave
  // padding slots of a batch re-read the wave's last step (step 0 for a wave
  // without steps, which K smaller than KS k-steps leaves), never a chunk
  // outside the block
  const int slast = cnt > 0 ? s0 + (cnt - 1) * sst : 0;
  const char* W = reinterpret_cast<const char*>(p.W) + lane * 16;
  u32x4 wv[2][U];
  auto wload = [&](const char* wb, int j, int slot) {
#pragma unroll
    for (int u = 0; u < U; ++u) wv[slot][u] = ld16(wb + (int64_t)(j * U + u < cnt ? s0 + (j * U + u) * sst : slast) * 1024);
  };
  // the first tile's first weight batch is requested right after the
  // activation reads, so the staging hides under its round trip (not with a
  // norm: its rows and the batch would not fit the 128 registers together)
  const int fb0 = blockIdx.x * NFB + fbl;
  const bool pre = !NORM && blockIdx.x < ntiles && fb0 < nfb && nb > 0;
  const char* xrow;
  int xstep;  // bytes per step (0: padding rows stay on a zero chunk)
  if constexpr (XL) {
    const int xp = K * (int)sizeof(S) + 16;  // LDS row pitch, bytes
    std::conditional_t<NORM, NormStage<S, float, norm_chunks<float>()>, CopyStage<S, 8>> stage;
    if constexpr (NORM) stage.load(p, wave); else stage.load(p);
    if (pre) wload(W + (int64_t)fb0 * nsteps * 1024, 0, 0);
    // LDS: M rows at pitch xp, the zero chunk, then the gains of a norm
    if constexpr (NORM) stage.finish(p, xs, xp, xs + M * xp + 16, wave, NW); else stage.finish(p, xs, xp);
    clear_ints(p);
    if (threadIdx.x == 0) *reinterpret_cast<u32x4*>(xs + M * xp) = zero4();
    __syncthreads();
    xrow = xr ? xs + r * xp + g * 16 : xs + M * xp;
    xstep = xr ? STEP * (int)sizeof(S) : 0;
  } else {
    if (pre) wload(W + (int64_t)fb0 * nsteps * 1024, 0, 0);
    xrow = xr ? reinterpret_cast<const char*>(reinterpret_cast<const S*>(p.X) + (int64_t)r * p.ldx + g * CH)
              : reinterpret_cast<const char*>(p.xzero) + g * 16;
    xstep = STEP * (int)sizeof(S);  // p.xzero holds >= K zeroed elements
  }
  __shared__ f32x4 red[KS > 1 ? NFB * (KS - 1) * 64 : 1];
  RowRed rr = RowRed::init();  // argmax or (LSE) log-sum-exp state of row r over this lane's features
  const int tgt = (LSE && p.epi.targets && xr) ? p.epi.targets[r] : -1;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int fb = tile * NFB + fbl;
    const bool active = fb < nfb;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      const char* wb = W + (int64_t)fb * nsteps * 1024;
      auto batch = [&](int j, int slot) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int su = s0 + (j * U + u) * sst;
          if (j * U + u < cnt) mma16(acc, wv[slot][u], ld16(xrow + (int64_t)su * xstep), S());
        }
      };
      if (!pre || tile != (int)blockIdx.x) wload(wb, 0, 0);  // else the first tile's went out before the staging
      for (int j = 0; j < nb; j += 2) {
        if (j + 1 < nb) wload(wb, j + 1, 1);
        batch(j, 0);
        if (j + 2 < nb) wload(wb, j + 2, 0);
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
        if (LSE && n == tgt) p.epi.tgt_logit[r] = acc[j];
        rr.add(LSE, acc[j], n);
      }
    }
  }
  rr.merge_groups(LSE);
  __shared__ u32x4 sb[NW][16];  // per wave and row: (v, s) or the top-2 list
  if (g == 0) sb[wave][r] = LSE ? u32x4{__float_as_uint(rr.v), 0u, __float_as_uint(rr.s), 0u} : rr.pack2();
  __syncthreads();
  if ((int)threadIdx.x < M) {
    RowRed t = RowRed::init();
    for (int w = 0; w < NW; ++w) {
      const u32x4 o = sb[w][threadIdx.x];
      if (LSE) t.merge(true, __uint_as_float(o[0]), 0, __uint_as_float(o[2]));
      else t.merge_packed(o);
    }
    if (LSE) {
      p.epi.part_val[(int64_t)blockIdx.x * M + threadIdx.x] = t.v;
      p.epi.part_sum[(int64_t)blockIdx.x * M + threadIdx.x] = t.s;
    } else {
      p.epi.part_top2[(int64_t)blockIdx.x * M + threadIdx.x] = t.pack2();
    }
  }
}

// LM head for M <= 16 with the rows staged in LDS, block-sweep form.
// Workgroup w of G (one per CU) takes the weight blocks w, w + G, w + 2G, ...,
// so at any moment the G workgroups read G neighbouring blocks: one contiguous
// region of the packed weight, which HBM streams faster than G separate runs
// (a plain read of the 1.16 GB LM head: 6.38 TB/s this way against 6.08 TB/s
// for contiguous shares per wave).  Within a block the NWV waves take
// interleaved 1 KB steps (wave v: steps v, v + NWV, ...), UB per batch; the
// next batch (of this block or the next) is in flight while one is
// multiplied.  A block's NWV partial tiles are summed in wave order through
// LDS by one wave (a different one each block), which keeps the running
// top-2 (or log-sum-exp) of its rows; the waves' lists are merged at the end
// into partial slot [blockIdx][row], reduced by argmax_rescore_kernel.  The
// first weight batch is requested right after the rows' reads, so the
// staging hides under its round trip.  Two waves per SIMD (256 registers per
// lane), one workgroup per CU.
template <typename S, int NWV, int UB, bool NORM, bool LSE, bool HL>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(2)))
void lm_head_sweep_kernel(GemmParams p) {
  constexpr int CH = Storage<S>::CH;
  constexpr int STEP = 4 * CH;
  extern __shared__ __attribute__((aligned(16))) char xs[];
  __shared__ f32x4 red[2][NWV][64];
  __shared__ u32x4 sb[NWV][16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int nsteps = K / STEP;
  const int nfb = (N + 15) >> 4;
  const int G = gridDim.x;
  const int nbat = (nsteps + NWV * UB - 1) / (NWV * UB);  // batches per block and wave
  const int nblk = (int)blockIdx.x < nfb ? (nfb - 1 - (int)blockIdx.x) / G + 1 : 0;
  const int nitems = nblk * nbat;
  const bool xr = r < M;
  // HL (M <= 8): columns 8..15 of the activation operand hold the remainder
  // of each normalised row, so every logit is the sum of two products
  const bool xop = HL ? (r & 7) < M : xr;
  // this wave's last step (step 0 for a wave without steps): slots past the
  // end re-read it, so every load stays inside the block
  const int vlast = wave < nsteps ? wave + NWV * ((nsteps - 1 - wave) / NWV) : 0;
  const char* W = reinterpret_cast<const char*>(p.W) + lane * 16;
  auto step_of = [&](int i, int u) { return wave + NWV * ((i % nbat) * UB + u); };
  auto load = [&](u32x4 (&dst)[UB], int i) {
    const char* src = W + (int64_t)((int)blockIdx.x + G * (i / nbat)) * nsteps * 1024;
#pragma unroll
    for (int u = 0; u < UB; ++u) dst[u] = ld16(src + (int64_t)min(step_of(i, u), vlast) * 1024);
  };
  u32x4 wa[UB], wb[UB];
  const int xp = K * (int)sizeof(S) + 16;  // LDS row pitch, bytes
  const int nxr = HL ? 16 : M;             // staged rows (HL: the remainders in rows 8..)
  {
    static_assert(!HL || NORM, "the remainder rows come from the norm");
    std::conditional_t<NORM, NormStage<S, float, norm_chunks<float>(), HL>, CopyStage<S, 8>> stage;
    if constexpr (NORM) stage.load(p, wave); else stage.load(p);
    if (nitems > 0) load(wa, 0);
    // LDS: the rows at pitch xp, the zero chunk, then the gains of a norm
    if constexpr (NORM) stage.finish(p, xs, xp, xs + nxr * xp + 16, wave, NWV); else stage.finish(p, xs, xp);
  }
  clear_ints(p);
  const char* xzero = xs + nxr * xp;
  if (threadIdx.x == 0) *reinterpret_cast<u32x4*>(xs + nxr * xp) = zero4();
  __syncthreads();
  const char* xrow = xop ? xs + r * xp + g * 16 : xzero;
  const int xstep = xop ? STEP * (int)sizeof(S) : 0;

  RowRed rr = RowRed::init();  // argmax or (LSE) log-sum-exp state of row r over this lane's features
  const int tgt = (LSE && p.epi.targets && xr) ? p.epi.targets[r] : -1;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4 (&src)[UB], int i) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int st = step_of(i, u);
      // slots past the wave's steps multiply the zero chunk
      mma16(acc, src[u], ld16(st < nsteps ? xrow + (int64_t)st * xstep : xzero), S());
    }
    if (i % nbat == nbat - 1) {  // the block is complete: its partial tiles summed in wave order
      const int bi = i / nbat;
      red[bi & 1][wave][lane] = acc;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      if (wave == bi % NWV) {
        f32x4 t = red[bi & 1][0][lane];
#pragma unroll
        for (int w = 1; w < NWV; ++w) t += red[bi & 1][w][lane];
        if constexpr (HL) {
#pragma unroll
          for (int j = 0; j < 4; ++j) t[j] += __shfl_down(t[j], 8, 64);  // + the remainder column r + 8
        }
        if (xr) {
          const int b = (int)blockIdx.x + G * bi;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = b * 16 + 4 * g + j;
            if (n >= N) continue;
            if (p.epi.logits) p.epi.logits[(int64_t)r * N + n] = t[j];
            if (LSE && n == tgt) p.epi.tgt_logit[r] = t[j];
            rr.add(LSE, t[j], n);
          }
        }
      }
    }
  };
  for (int i = 0; i < nitems; i += 2) {
    if (i + 1 < nitems) load(wb, i + 1);
    compute(wa, i);
    if (i + 1 >= nitems) break;
    if (i + 2 < nitems) load(wa, i + 2);
    compute(wb, i + 1);
  }
  rr.merge_groups(LSE);
  if (g == 0) sb[wave][r] = LSE ? u32x4{__float_as_uint(rr.v), 0u, __float_as_uint(rr.s), 0u} : rr.pack2();
  __syncthreads();
  if ((int)threadIdx.x < M) {
    RowRed t = RowRed::init();
    for (int w = 0; w < NWV; ++w) {
      const u32x4 o = sb[w][threadIdx.x];
      if (LSE) t.merge(true, __uint_as_float(o[0]), 0, __uint_as_float(o[2]));
      else t.merge_packed(o);
    }
    if (LSE) {
      p.epi.part_val[(int64_t)blockIdx.x * M + threadIdx.x] = t.v;
      p.epi.part_sum[(int64_t)blockIdx.x * M + threadIdx.x] = t.s;
    } else {
      p.epi.part_top2[(int64_t)blockIdx.x * M + threadIdx.x] = t.pack2();
    }
  }
}

// ---------------------------------------------------------------------------
template <typename S, int BM, int BN, bool DUAL, bool ARGMAX, bool LSE = false>
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
    // argmax (EPI_ARGMAX) or log-sum-exp (EPI_LSE, LSE set) partials of this tile's rows
    __shared__ u32x4 sb[2][BM];  // per wave column and row: (v, s) or the top-2 list
#pragma unroll
    for (int q = 0; q < RBW; ++q) {
      const int mloc = wm * (BM / 2) + q * 16 + r;
      const int m = m0 + mloc;
      int tgt = -1;
      if constexpr (LSE) tgt = (p.epi.targets && m < M) ? p.epi.targets[m] : -1;
      RowRed rr = RowRed::init();
#pragma unroll
      for (int f = 0; f < FBW; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * (BN / 2) + f * 16 + 4 * g + j;
          if (n < N && m < M) {
            const float v = acc[f][q][j];
            if (p.epi.logits) p.epi.logits[(int64_t)m * N + n] = v;
            if constexpr (LSE) {
              if (n == tgt) p.epi.tgt_logit[m] = v;
              rr.add(true, v, n);
            } else {
              rr.add1(v, n);  // the lane's largest; the merges keep the top two of those
            }
          }
        }
      rr.merge_groups(LSE);
      if (g == 0) sb[wn][mloc] = LSE ? u32x4{__float_as_uint(rr.v), 0u, __float_as_uint(rr.s), 0u} : rr.pack2();
    }
    __syncthreads();
    if (tid < BM && m0 + tid < M) {
      RowRed rr = RowRed::init();
      for (int w = 0; w < 2; ++w) {
        const u32x4 o = sb[w][tid];
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

// Greedy token of row m (one workgroup per row).  The partial lists are
// merged into the row's two leading kernel logits; the order is total (value,
// then lower index), so the result does not depend on the merge order.  The
// weight-streaming kernel's lists are the exact two largest of its features;
// the tiled kernels keep the two largest of their lanes' maxima (16 features
// per lane and row), so the pair is the row's two largest unless both of
// those share one lane of one tile, where the first alone decides.  The
// kernel's logits use the normalised row rounded to the operand type; the two
// candidates are scored again here in fp32 from the float row,
//   z_c = inv * sum_k W[c][k] * (x[k] * g[k]),  inv = 1 / sqrt(mean_k x[k]^2 + eps),
// with every sum taken in a fixed order, and the larger (lower index on a tie)
// is the token.  The rounding of the operand moves a bf16 logit by about
// 2e-3 at hidden 2880 and unit-scale rows; the re-score removes that part of
// the error from the decision between the two leading tokens.
template <typename S>
__global__ __launch_bounds__(256) void argmax_rescore_kernel(const u32x4* part, int P, int M, const float* x,
                                                             int64_t ldx, const float* gain, float eps,
                                                             const char* W, int K, int32_t* tokens, int rescore) {
  constexpr int CH = Storage<S>::CH;  // elements per 16-byte chunk
  constexpr int STEP = 4 * CH;        // elements per packed 1 KB step of a 16-row block
  constexpr int NPRE = 2;             // chunks per thread held from before the merge (K <= 512 CH)
  const int rpx = (M + 7) / 8;  // rows per XCD (see launch_argmax_rescore)
  const int m = (int)(blockIdx.x % 8) * rpx + (int)(blockIdx.x / 8);
  if (m >= M) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = K / CH;
  const float* xr = x + (int64_t)m * ldx;
  // the row and its gains first, so that their loads overlap the partials'
  // (not when the logits were exact: the largest is then the token)
  f32x4 xv[NPRE][CH / 4], gv[NPRE][CH / 4];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NPRE; ++c) {
    const int ch = rescore ? tid + 256 * c : nch;
#pragma unroll
    for (int q = 0; q < CH / 4; ++q) {
      xv[c][q] = ch < nch ? *reinterpret_cast<const f32x4*>(xr + ch * CH + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
      gv[c][q] = ch < nch ? *reinterpret_cast<const f32x4*>(gain + ch * CH + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const u32x4 none = {__float_as_uint(-INFINITY), 0x7fffffffu, __float_as_uint(-INFINITY), 0x7fffffffu};
  RowRed rr = RowRed::init();
  for (int q = tid; q < P; q += 8 * 256) {  // up to 2,048 partials in one round of loads
    u32x4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int qq = q + 256 * u;
      t[u] = qq < P ? part[(int64_t)qq * M + m] : none;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) rr.merge_packed(t[u]);
  }
#pragma unroll
  for (int c = 0; c < NPRE; ++c)
#pragma unroll
    for (int q = 0; q < CH / 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += xv[c][q][e] * xv[c][q][e];
  for (int ch = tid + 256 * NPRE; ch < nch; ch += 256)
#pragma unroll
    for (int e = 0; e < CH; ++e) ss += xr[ch * CH + e] * xr[ch * CH + e];
  for (int o = 1; o < 64; o <<= 1) {
    const u32x4 t = {__float_as_uint(__shfl_xor(rr.v, o, 64)), (uint32_t)__shfl_xor(rr.i, o, 64),
                     __float_as_uint(__shfl_xor(rr.v2, o, 64)), (uint32_t)__shfl_xor(rr.i2, o, 64)};
    rr.merge_packed(t);
  }
  __shared__ u32x4 sw[4];
  __shared__ float sred[3][4];
  if (lane == 0) sw[wave] = rr.pack2();
  __syncthreads();
  RowRed best = RowRed::init();
  for (int w = 0; w < 4; ++w) best.merge_packed(sw[w]);
  const int c1 = best.i, c2 = best.i2;
  if (!rescore) {
    if (tid == 0) tokens[m] = c1 == 0x7fffffff ? -1 : c1;
    return;
  }
  const bool has1 = c1 != 0x7fffffff, has2 = c2 != 0x7fffffff;
  // the two candidates' products with x * g
  const int steps = K / STEP;
  const char* w1 = W + (int64_t)(has1 ? c1 >> 4 : 0) * steps * 1024 + (has1 ? c1 & 15 : 0) * 16;
  const char* w2 = W + (int64_t)(has2 ? c2 >> 4 : 0) * steps * 1024 + (has2 ? c2 & 15 : 0) * 16;
  auto woff = [&](int ch) {  // k-step, then the lane group of the chunk
    const int k0 = ch * CH;
    return (int64_t)(k0 / STEP) * 1024 + ((k0 % STEP) / CH) * 256;
  };
  float d1 = 0.f, d2 = 0.f;
#pragma unroll
  for (int c = 0; c < NPRE; ++c) {
    const int ch = tid + 256 * c;
    if (ch < nch) {
      const u32x4 a = ld16(w1 + woff(ch)), b = ld16(w2 + woff(ch));
#pragma unroll
      for (int q = 0; q < CH / 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xg = xv[c][q][e] * gv[c][q][e];
          d1 += chunk_elem<S>(a, 4 * q + e) * xg;
          d2 += chunk_elem<S>(b, 4 * q + e) * xg;
        }
    }
  }
  for (int ch = tid + 256 * NPRE; ch < nch; ch += 256) {
    const u32x4 a = ld16(w1 + woff(ch)), b = ld16(w2 + woff(ch));
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const float xg = xr[ch * CH + e] * gain[ch * CH + e];
      d1 += chunk_elem<S>(a, e) * xg;
      d2 += chunk_elem<S>(b, e) * xg;
    }
  }
  ss = wave_sum(ss);
  d1 = wave_sum(d1);
  d2 = wave_sum(d2);
  if (lane == 0) { sred[0][wave] = ss; sred[1][wave] = d1; sred[2][wave] = d2; }
  __syncthreads();
  if (tid == 0) {
    const float tss = (sred[0][0] + sred[0][1]) + (sred[0][2] + sred[0][3]);
    const float inv = 1.0f / sqrtf(tss / (float)K + eps);
    const float z1 = ((sred[1][0] + sred[1][1]) + (sred[1][2] + sred[1][3])) * inv;
    const float z2 = ((sred[2][0] + sred[2][1]) + (sred[2][2] + sred[2][3])) * inv;
    tokens[m] = !has1 ? -1 : (has2 && better(z2, c2, z1, c1)) ? c2 : c1;
  }
}

void launch_argmax_rescore(const u32x4* part, int P, int M, const float* x, int64_t ldx, const float* gain,
                           float eps, const void* W, int K, int w_bf16, int32_t* tokens, int rescore, hipStream_t s) {
  const char* w = reinterpret_cast<const char*>(W);
  // workgroup b runs on XCD b % 8 and takes row (b % 8) * rpx + b / 8, so the
  // rows of one XCD are consecutive and share the lines of the tile-major
  // lists in that XCD's L2 (eight rows' lists of one partial per 128 bytes)
  const int rpx = (M + 7) / 8;
  if (w_bf16)
    hipLaunchKernelGGL(argmax_rescore_kernel<uint16_t>, dim3(8 * rpx), dim3(256), 0, s, part, P, M, x, ldx, gain, eps,
                       w, K, tokens, rescore);
  else
    hipLaunchKernelGGL(argmax_rescore_kernel<float>, dim3(8 * rpx), dim3(256), 0, s, part, P, M, x, ldx, gain, eps,
                       w, K, tokens, rescore);
}

// Log-sum-exp of each row from its P partial (maximum, sum of exp) pairs, merged
// in a fixed order (thread strides, then lanes by xor distance, then waves),
// and the cross-entropy lse - y[target] where the row has a target in [0, N).
__global__ __launch_bounds__(256) void lse_reduce_kernel(const float* pv, const float* ps, int P, int M, int N,
                                                         const int32_t* targets, const float* tgt, float* lse,
                                                         float* loss) {
  const int m = blockIdx.x;
  RowRed rr = RowRed::init();
  for (int q = threadIdx.x; q < P; q += 256) rr.merge(true, pv[(int64_t)q * M + m], 0, ps[(int64_t)q * M + m]);
  for (int o = 1; o < 64; o <<= 1) {
    const float ov = __shfl_xor(rr.v, o, 64), os = __shfl_xor(rr.s, o, 64);
    rr.merge(true, ov, 0, os);
  }
  __shared__ float sv[4], ss[4];
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = rr.v; ss[threadIdx.x >> 6] = rr.s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) rr.merge(true, sv[w], 0, ss[w]);
    const float l = rr.v + logf(rr.s);
    if (lse) lse[m] = l;
    if (loss) loss[m] = (targets && targets[m] >= 0 && targets[m] < N) ? l - tgt[m] : 0.f;
  }
}

// Large batches: 64 rows per workgroup (lane = row, so every load reads 64
// consecutive rows of one partial), 16 waves taking partials w, w + 16, ...
// in order, then the waves merged in order through LDS.
__global__ __launch_bounds__(1024) void lse_reduce_rows_kernel(const float* pv, const float* ps, int P, int M, int N,
                                                               const int32_t* targets, const float* tgt, float* lse,
                                                               float* loss) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = blockIdx.x * 64 + lane;
  const int mc = m < M ? m : M - 1;
  RowRed rr = RowRed::init();
  // eight partials loaded before they are merged (in partial order)
  for (int q = wave; q < P; q += 16 * 8) {
    float v[8], t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int qq = q + 16 * u;
      v[u] = qq < P ? pv[(int64_t)qq * M + mc] : -INFINITY;
      t[u] = qq < P ? ps[(int64_t)qq * M + mc] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) rr.merge(true, v[u], 0, t[u]);
  }
  __shared__ float sv[16][64], ss[16][64];
  sv[wave][lane] = rr.v;
  ss[wave][lane] = rr.s;
  __syncthreads();
  if (wave == 0 && m < M) {
    for (int w = 1; w < 16; ++w) rr.merge(true, sv[w][lane], 0, ss[w][lane]);
    const float l = rr.v + logf(rr.s);
    if (lse) lse[m] = l;
    if (loss) loss[m] = (targets && targets[m] >= 0 && targets[m] < N) ? l - tgt[m] : 0.f;
  }
}

void launch_lse_reduce(const float* pv, const float* ps, int P, int M, int N, const int32_t* targets,
                       const float* tgt, float* lse, float* loss, hipStream_t s) {
  if (M >= 1024)
    hipLaunchKernelGGL(lse_reduce_rows_kernel, dim3((M + 63) / 64), dim3(1024), 0, s, pv, ps, P, M, N, targets, tgt,
                       lse, loss);
  else
    hipLaunchKernelGGL(lse_reduce_kernel, dim3(M), dim3(256), 0, s, pv, ps, P, M, N, targets, tgt, lse, loss);
}

// KL divergence of row m from its k target pairs (one workgroup per row):
//   kl[m] = sum_j p_j (log p_j - z_j + lse[m]),  z_j = inv * sum_k W[id_j][k] x[m][k] g[k],
// over the pairs with id_j in [0, N) and p_j > 0.  The row's x * g is staged
// in LDS (zero-padded to whole rounds of chunks, so that the weight loads of
// a round need no predicate: their chunk index is clamped instead and meets a
// zero); wave w takes pairs w, w + 4, ..., each as one wave-wide dot product
// with U chunk loads in flight per lane; the four waves' sums are added in a
// fixed order.  The target logits are fp32 from the unrounded row, as in the
// argmax re-score.  A row of the packed weight holds 16 of every 64 bytes of
// its 16-row block, so a wave's loads of it touch 64 cache lines each; with
// the row-major weight (Wrows) a wave reads 1 KB of one row per load.
template <typename S>
__global__ __launch_bounds__(256) void kl_topk_kernel(const float* x, int64_t ldx, const float* gain, float eps,
                                                      const char* W, const char* Wrows, int K, int N, int k,
                                                      const int32_t* ids, const float* probs, const float* lse,
                                                      float* kl, int M) {
  constexpr int CH = Storage<S>::CH;  // elements per 16-byte chunk
  constexpr int STEP = 4 * CH;        // elements per packed 1 KB step of a 16-row block
  constexpr int U = 4;                // chunk loads in flight per lane
  extern __shared__ float sf[];
  const int rpx = (M + 7) / 8;  // rows per XCD, consecutive rows on one XCD (as in the re-score)
  const int m = (int)(blockIdx.x % 8) * rpx + (int)(blockIdx.x / 8);
  if (m >= M) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = K / CH;
  const int npad = (nch + 64 * U - 1) / (64 * U) * (64 * U);
  const float* xr = x + (int64_t)m * ldx;
  float ss = 0.f;
  for (int e = 4 * tid; e < npad * CH; e += 1024) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (e < K) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(xr + e);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gain + e);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ss += xv[q] * xv[q];
        v[q] = xv[q] * gv[q];
      }
    }
    *reinterpret_cast<f32x4*>(sf + e) = v;
  }
  ss = wave_sum(ss);
  __shared__ float sred[4];
  if (lane == 0) sred[wave] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf(((sred[0] + sred[1]) + (sred[2] + sred[3])) / (float)K + eps);
  const float L = lse[m];
  const int steps = K / STEP;
  float acc = 0.f;
  for (int j = wave; j < k; j += 4) {
    const int t = ids[(int64_t)m * k + j];
    const float p = probs[(int64_t)m * k + j];
    if (t < 0 || t >= N || !(p > 0.f)) continue;  // the same pair for the whole wave
    const char* wr = Wrows ? Wrows + (int64_t)t * K * (int)sizeof(S)
                           : W + (int64_t)(t >> 4) * steps * 1024 + (t & 15) * 16;
    float d = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64 * U) {
      u32x4 a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ch = min(c0 + 64 * u + lane, nch - 1);
        const int k0 = ch * CH;
        a[u] = ld16(wr + (Wrows ? (int64_t)ch * 16 : (int64_t)(k0 / STEP) * 1024 + ((k0 % STEP) / CH) * 256));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float* f = sf + (c0 + 64 * u + lane) * CH;
#pragma unroll
        for (int e = 0; e < CH; ++e) d += chunk_elem<S>(a[u], e) * f[e];
      }
    }
    d = wave_sum(d);  // the same value in every lane
    acc += p * (logf(p) - d * inv + L);
  }
  __shared__ float sacc[4];
  if (lane == 0) sacc[wave] = acc;
  __syncthreads();
  if (tid == 0) kl[m] = (sacc[0] + sacc[1]) + (sacc[2] + sacc[3]);
}

int kl_topk_lds_bytes(int K, int w_bf16) {
  const int CH = w_bf16 ? 8 : 4, U = 4;
  const int nch = K / CH;
  return (nch + 64 * U - 1) / (64 * U) * (64 * U) * CH * 4;
}

void launch_kl_topk(const float* x, int64_t ldx, const float* gain, float eps, const void* W, const void* Wrows, int K,
                    int N, int w_bf16, int k, const int32_t* ids, const float* probs, const float* lse, float* kl,
                    int M, hipStream_t s) {
  const char* w = reinterpret_cast<const char*>(W);
  const char* wrows = reinterpret_cast<const char*>(Wrows);
  const int rpx = (M + 7) / 8;
  const size_t lds = (size_t)kl_topk_lds_bytes(K, w_bf16);
  if (w_bf16)
    hipLaunchKernelGGL(kl_topk_kernel<uint16_t>, dim3(8 * rpx), dim3(256), lds, s, x, ldx, gain, eps, w, wrows, K, N,
                       k, ids, probs, lse, kl, M);
  else
    hipLaunchKernelGGL(kl_topk_kernel<float>, dim3(8 * rpx), dim3(256), lds, s, x, ldx, gain, eps, w, wrows, K, N, k,
                       ids, probs, lse, kl, M);
}

// ---------------------------------------------------------------------------
// Dispatch
static constexpr int kStreamU = 8;     // 1 KB steps in flight per wave
// Launch shape of lm_argmax_stream_kernel (rows too wide for LDS): NFB blocks x
// KS waves per workgroup.
#ifndef PE_LM_NFB
#define PE_LM_NFB 4
#endif
#ifndef PE_LM_KS
#define PE_LM_KS 3
#endif
#ifndef PE_LM_U
#define PE_LM_U 5
#endif
static constexpr int kLmNFB = PE_LM_NFB, kLmKS = PE_LM_KS, kLmU = PE_LM_U;
// The block-sweep LM-head kernel: waves per workgroup and steps per wave and
// batch (8 x 6: two batches per block of the 90-step d = 2880 rows; 8 x 3,
// 8 x 4, 8 x 12, 4 x 12, 4 x 23 and 12 x 8 measured slower, as was a third
// batch in flight), workgroups (the CU count of MI355X),
// and the largest row block it stages beside its static LDS (the two rings
// of partial tiles and the lists).
#ifndef PE_LM_SWEEP_W
#define PE_LM_SWEEP_W 8
#endif
#ifndef PE_LM_SWEEP_U
#define PE_LM_SWEEP_U 6
#endif
static constexpr int kLmSweepW = PE_LM_SWEEP_W, kLmSweepU = PE_LM_SWEEP_U, kLmSweepGrid = 256;
static constexpr int kLmSweepXLds = 158 * 1024 - 3 * kLmSweepW * 1024;

// Waves per 16-row block: the most (up to 16) that still leave every wave at
// least one full batch of kStreamU steps.
static int stream_ks(int nsteps) {
  int ks = 16;
  while (ks > 1 && nsteps / ks < kStreamU) ks >>= 1;
  return ks;
}
// The same with a deferred norm over segs segments (1 or 3): a multiple of
// segs, so that every wave's steps lie in one segment.
static int stream_ks_segs(int nsteps, int segs) {
  if (segs == 1) return stream_ks(nsteps);
  if (nsteps / 15 >= kStreamU) return 15;
  if (nsteps / 6 >= kStreamU) return 6;
  return 3;
}

int gemm_argmax_partials(int M, int N) {
  if (M <= 16) {  // one workgroup per CU, each with at least one weight block
    const int nfb = (N + 15) / 16;
    return nfb < kLmSweepGrid ? nfb : kLmSweepGrid;
  }
  return (N + 63) / 64;  // largest count over the tiled configurations (BN >= 64)
}

template <typename S, int BM, int BN, bool DUAL, bool ARGMAX, bool LSE = false>
static int launch_tiled(const GemmParams& p, hipStream_t s) {
  const int n_ft = (p.N + BN - 1) / BN, n_mt = (p.M + BM - 1) / BM;
  const int grid = ((n_ft + 7) / 8) * 8 * n_mt;
  hipLaunchKernelGGL((gemm_tiled_kernel<S, BM, BN, DUAL, ARGMAX, LSE>), dim3(grid), dim3(256), 0, s, p, n_ft, n_mt);
  return n_ft;
}

// Raises kernel K's dynamic LDS limit once per process (the default may be
// below what the activation block needs); the static's initialisation is
// thread-safe, and a failure shows up as a failed launch.
template <auto K>
static void allow_lds(int bytes) {
  static const hipError_t st =
      hipFuncSetAttribute(reinterpret_cast<const void*>(K), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)st;
}

template <typename S, bool DUAL, int LOM>
static void launch_stream(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.N + 15) / 16);
  const int nsteps = p.K / (4 * Storage<S>::CH);
  const int ks = p.xinv ? stream_ks_segs(nsteps, p.xinv_segs) : stream_ks(nsteps);
  if constexpr (!DUAL && LOM == 0) {  // deferred three-segment norms (the fc fusion)
    if (ks == 15) { hipLaunchKernelGGL((gemm_stream_kernel<S, 15, kStreamU, false, 0>), grid, dim3(960), 0, s, p); return; }
    if (ks == 6) { hipLaunchKernelGGL((gemm_stream_kernel<S, 6, kStreamU, false, 0>), grid, dim3(384), 0, s, p); return; }
    if (ks == 3) { hipLaunchKernelGGL((gemm_stream_kernel<S, 3, kStreamU, false, 0>), grid, dim3(192), 0, s, p); return; }
  }
  switch (ks) {
    case 16: hipLaunchKernelGGL((gemm_stream_kernel<S, 16, kStreamU, DUAL, LOM>), grid, dim3(1024), 0, s, p); break;
    case 8: hipLaunchKernelGGL((gemm_stream_kernel<S, 8, kStreamU, DUAL, LOM>), grid, dim3(512), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_stream_kernel<S, 4, kStreamU, DUAL, LOM>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_stream_kernel<S, 2, kStreamU, DUAL, LOM>), grid, dim3(128), 0, s, p); break;
    default: hipLaunchKernelGGL((gemm_stream_kernel<S, 1, kStreamU, DUAL, LOM>), grid, dim3(64), 0, s, p); break;
  }
}

// Weight steps per batch of the LDS-staged streaming kernel: two batches
// cover the 16-17 steps per wave of the widest decode contractions (fc with
// its norm, 9; down, 8) and the 11-12 of the gate/up pair (6).
template <bool DUAL, bool NORM>
constexpr int stream_lds_u() { return DUAL ? 6 : NORM ? 9 : 8; }
// Second weight batch requested before the staging finishes (registers
// permitting: not beside the rows of a norm).
template <typename XT, bool NORM>
constexpr bool stream_lds_early2() { return !NORM; }
// Largest LDS block it stages: the activation rows, the zero chunk and the
// gains of a norm (the K-split reduction reuses the same bytes afterwards).
static constexpr int kStreamXLds = 156 * 1024;

template <typename S, typename XT, int KS, bool DUAL, bool NORM>
static void launch_stream_lds_ks(const GemmParams& p, size_t lds, hipStream_t s) {
  constexpr int U = stream_lds_u<DUAL, NORM>();
  constexpr bool E2 = stream_lds_early2<XT, NORM>();
  const size_t red = (size_t)(KS - 1) * 64 * 16 * (DUAL ? 2 : 1);
  if (lds < red) lds = red;
  allow_lds<&gemm_stream_lds_kernel<S, XT, KS, U, DUAL, NORM, E2>>(kStreamXLds);
  hipLaunchKernelGGL((gemm_stream_lds_kernel<S, XT, KS, U, DUAL, NORM, E2>), dim3((p.N + 15) / 16),
                     dim3(64 * KS), lds, s, p);
}

template <typename S, typename XT, bool DUAL, bool NORM>
static void launch_stream_lds(const GemmParams& p, size_t lds, hipStream_t s) {
  const int nsteps = p.K / (4 * Storage<S>::CH);
  if constexpr (NORM && !DUAL) {
    if (p.nrm.defer) {  // every wave inside one segment
      switch (stream_ks_segs(nsteps, p.nrm.segs)) {
        case 15: launch_stream_lds_ks<S, XT, 15, false, true>(p, lds, s); return;
        case 6: launch_stream_lds_ks<S, XT, 6, false, true>(p, lds, s); return;
        case 3: launch_stream_lds_ks<S, XT, 3, false, true>(p, lds, s); return;
        default: break;  // one segment: any split
      }
    }
  }
  switch (stream_ks(nsteps)) {
    case 16: launch_stream_lds_ks<S, XT, 16, DUAL, NORM>(p, lds, s); break;
    case 8: launch_stream_lds_ks<S, XT, 8, DUAL, NORM>(p, lds, s); break;
    case 4: launch_stream_lds_ks<S, XT, 4, DUAL, NORM>(p, lds, s); break;
    case 2: launch_stream_lds_ks<S, XT, 2, DUAL, NORM>(p, lds, s); break;
    default: launch_stream_lds_ks<S, XT, 1, DUAL, NORM>(p, lds, s); break;
  }
}

// Float rows normalised inside the weight stream: the gate/up pair takes 6
// steps per batch (its two weight streams and the float rows share the 128
// registers), single contractions 8.
// Steps per batch of gemm_stream_fnorm_kernel, measured on the c=1 decode
// shapes (11-12 steps per wave): 6 for single contractions (two full
// batches, no clamped re-reads), 4 for the gate/up pair (its two weight
// streams and the float rows fit the 128 registers without spilling).
#ifndef PE_FNORM_U
#define PE_FNORM_U 6
#endif
#ifndef PE_FNORM_DUAL_U
#define PE_FNORM_DUAL_U 4
#endif
// Which float-row norms fold into the stream (1: single contractions, 2: the
// gate/up pair; else a separate rmsnorm_rows_kernel runs first).
#ifndef PE_FNORM_KINDS
#define PE_FNORM_KINDS 3
#endif
template <typename S, bool DUAL, bool HL>
static void launch_stream_fnorm(const GemmParams& p, int ks, hipStream_t s) {
  constexpr int U = DUAL ? PE_FNORM_DUAL_U : PE_FNORM_U;
  const dim3 grid((p.N + 15) / 16);
  const size_t lds = (size_t)ks * (kFnormMaxSteps * 4 * Storage<S>::CH * 4) + (size_t)ks * 64 * 4;
  switch (ks) {
    case 16: hipLaunchKernelGGL((gemm_stream_fnorm_kernel<S, 16, U, DUAL, HL>), grid, dim3(1024), lds, s, p); break;
    case 8: hipLaunchKernelGGL((gemm_stream_fnorm_kernel<S, 8, U, DUAL, HL>), grid, dim3(512), lds, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_stream_fnorm_kernel<S, 4, U, DUAL, HL>), grid, dim3(256), lds, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_stream_fnorm_kernel<S, 2, U, DUAL, HL>), grid, dim3(128), lds, s, p); break;
    default: hipLaunchKernelGGL((gemm_stream_fnorm_kernel<S, 1, U, DUAL, HL>), grid, dim3(64), lds, s, p); break;
  }
}

// The requested RMSNorm as its own kernel into p.nrm.tmp (also clearing
// p.clear); returns the parameters of the contraction over the normalised rows.
// packed: p.nrm.tmp receives the operand layout (rows rounded up to 16).
template <typename S>
static GemmParams norm_first(const GemmParams& p, hipStream_t s, bool packed = false, bool defer = false) {
  NormParams np{};
  np.inv_out = defer ? p.nrm.inv_tmp : nullptr;
  np.in = p.X;
  np.ld_in = p.ldx;
  np.skip = p.nrm.skip;
  np.n = p.M;
  np.segs = p.nrm.segs;
  np.d = p.nrm.seg_len;
  np.gain = p.nrm.gain;
  np.eps = p.nrm.eps;
  np.out = p.nrm.tmp;
  np.ld_out = p.K;
  np.zero = p.clear;
  np.nzero = p.nclear;
  np.packed = packed;
  const int sbf = sizeof(S) == 2;
  launch_rmsnorm_rows(np, p.nrm.x_f32 ? 0 : sbf, sbf, s);
  GemmParams q = p;
  q.X = p.nrm.tmp;
  q.ldx = p.K;
  q.nrm = NormIn{};
  q.clear = nullptr;
  q.nclear = 0;
  q.x_packed = packed;
  if (defer) {
    q.xinv = p.nrm.inv_tmp;
    q.xinv_segs = p.nrm.segs;
  }
  return q;
}

// The LM-head weight stream for M <= 16 rows (argmax or, LSE, log-sum-exp
// partials): rows and their norm staged in LDS when they fit, else read from
// global memory after a separate norm.  Returns the partial count.
// Whether the LM head over M float rows normalised with `gain` (one segment
// of K) runs with the remainder of the normalised rows as a second bf16
// operand part (hi + lo, about 2^-17 relative): M <= 8, a row the norm
// staging holds, a 16-byte aligned gain, and the 16 staged rows in LDS.
// Those logits are exact to far below the argmax's 1e-2 gap, so the
// argmax takes the largest without a re-score.
bool lm_head_exact(int M, int K, int bf16, const float* gain) {
  const size_t lds = (size_t)16 * ((size_t)K * 2 + 16) + 16 + (size_t)K * 4 + (size_t)M * 4;
  return bf16 && M >= 1 && M <= 8 && K % 4 == 0 && K / 4 <= 64 * norm_chunks<float>() &&
         (reinterpret_cast<uintptr_t>(gain) & 15) == 0 && lds <= (size_t)kLmSweepXLds;
}

template <typename S, bool LSE>
static int launch_lm_stream(const GemmParams& p0, bool norm, bool norm_fits, bool xf32, size_t lds, hipStream_t s) {
  const int grid = gemm_argmax_partials(p0.M, p0.N);
  if constexpr (sizeof(S) == 2) {
    if (norm && xf32 && p0.nrm.segs == 1 && !p0.nrm.defer && lm_head_exact(p0.M, p0.K, 1, p0.nrm.gain)) {
      const size_t lds_hl = (size_t)16 * ((size_t)p0.K * 2 + 16) + 16 + (size_t)p0.K * 4 + (size_t)p0.M * 4;
      allow_lds<&lm_head_sweep_kernel<S, kLmSweepW, kLmSweepU, true, LSE, true>>(kLmSweepXLds);
      hipLaunchKernelGGL((lm_head_sweep_kernel<S, kLmSweepW, kLmSweepU, true, LSE, true>), dim3(grid),
                         dim3(64 * kLmSweepW), lds_hl, s, p0);
      return grid;
    }
  }
  if (lds <= (size_t)kLmSweepXLds && norm_fits && (!norm || xf32)) {
    if (norm) {
      allow_lds<&lm_head_sweep_kernel<S, kLmSweepW, kLmSweepU, true, LSE, false>>(kLmSweepXLds);
      hipLaunchKernelGGL((lm_head_sweep_kernel<S, kLmSweepW, kLmSweepU, true, LSE, false>), dim3(grid),
                         dim3(64 * kLmSweepW), lds, s, p0);
    } else {
      allow_lds<&lm_head_sweep_kernel<S, kLmSweepW, kLmSweepU, false, LSE, false>>(kLmSweepXLds);
      hipLaunchKernelGGL((lm_head_sweep_kernel<S, kLmSweepW, kLmSweepU, false, LSE, false>), dim3(grid),
                         dim3(64 * kLmSweepW), lds, s, p0);
    }
    return grid;
  }
  const GemmParams p = norm ? norm_first<S>(p0, s, false) : p0;
  if (lds <= (size_t)kLmSweepXLds) {
    allow_lds<&lm_head_sweep_kernel<S, kLmSweepW, kLmSweepU, false, LSE, false>>(kLmSweepXLds);
    hipLaunchKernelGGL((lm_head_sweep_kernel<S, kLmSweepW, kLmSweepU, false, LSE, false>), dim3(grid),
                       dim3(64 * kLmSweepW), lds, s, p);
  } else {
    const dim3 block(64 * kLmNFB * kLmKS);
    hipLaunchKernelGGL((lm_argmax_stream_kernel<S, kLmNFB, kLmKS, kLmU, false, false, LSE>), dim3(grid), block, 0, s,
                       p);
  }
  return grid;
}

template <typename S>
static int launch_gemm_t(const GemmParams& p0, hipStream_t s) {
  const bool dual = p0.epi.kind == EPI_SWIGLU;
  const bool am = epi_rowred(p0.epi.kind);
  const bool lse = p0.epi.kind == EPI_LSE;
  const bool norm = p0.nrm.gain != nullptr;
  // deferred 1 / rms: storage-type rows (the operand is then the input times
  // its gains, exact for unit gains), one or three segments, bf16
  const bool defer = sizeof(S) == 2 && norm && p0.nrm.defer && !p0.nrm.x_f32 &&
                     (p0.nrm.segs == 1 || p0.nrm.segs == 3) && !epi_rowred(p0.epi.kind);
  if (p0.M <= 16) {
    // activation rows + the zero chunk of the padding rows (+ the gains of a
    // norm and its deferred scales)
    const size_t lds = (size_t)p0.M * (p0.K * sizeof(S) + 16) + 16 +
                       (norm ? (size_t)p0.K * 4 + (size_t)p0.M * p0.nrm.segs * 4 : 0);
    const int xsz = norm && p0.nrm.x_f32 ? 4 : (int)sizeof(S);
    const int seg_bytes = p0.nrm.seg_len * xsz;
    const bool xf32 = xsz == 4;
    // NormStage holds a segment in norm_chunks<XT>() chunks per lane and reads
    // the gains as 16-byte vectors
    const bool norm_fits = !norm || (seg_bytes % 16 == 0 && seg_bytes / 16 <= 64 * (xf32 ? 12 : 6) &&
                                     (reinterpret_cast<uintptr_t>(p0.nrm.gain) & 15) == 0);
    if (am) {
      if (lse) return launch_lm_stream<S, true>(p0, norm, norm_fits, xf32, lds, s);
      return launch_lm_stream<S, false>(p0, norm, norm_fits, xf32, lds, s);
    }
    const int fks = stream_ks(p0.K / (4 * Storage<S>::CH));
    const int fsteps = (p0.K / (4 * Storage<S>::CH) + fks - 1) / fks;
    if (norm && xf32 && fsteps <= kFnormMaxSteps && (reinterpret_cast<uintptr_t>(p0.nrm.gain) & 15) == 0 &&
        p0.nrm.segs == 1 && (PE_FNORM_KINDS & (dual ? 2 : 1))) {
      // float rows (the residual stream): the norm folds into the weight stream
      const bool hl = sizeof(S) == 2 && p0.x_split;
      if (dual) { if (hl) launch_stream_fnorm<S, true, true>(p0, fks, s); else launch_stream_fnorm<S, true, false>(p0, fks, s); }
      else { if (hl) launch_stream_fnorm<S, false, true>(p0, fks, s); else launch_stream_fnorm<S, false, false>(p0, fks, s); }
      return 0;
    }
    if (norm && norm_fits && !xf32 && !dual && lds <= (size_t)kStreamXLds) {
      // storage-type rows (the captured streams, several segments): normalised
      // while they are staged in LDS
      GemmParams q = p0;
      q.nrm.defer = defer;
      launch_stream_lds<S, S, false, true>(q, lds, s);
      return 0;
    }
    const GemmParams p = norm ? norm_first<S>(p0, s, false, defer && p0.nrm.inv_tmp) : p0;
    // a remainder operand: in columns 8..15 of the operand when M <= 8, else
    // as a second matrix-core step per chunk
    const int lom = (sizeof(S) == 2 && !norm && p.x_lo) ? (p.M <= 8 ? 2 : 1) : 0;
    if (dual) launch_stream<S, true, 0>(p, s);
    else if (lom == 2) launch_stream<S, false, 2>(p, s);
    else if (lom == 1) launch_stream<S, false, 1>(p, s);
    else launch_stream<S, false, 0>(p, s);
    return 0;
  }
  // rows normalised for the LDS-tiled kernel of gemm_big.hip go to its 1 KB
  // operand chunks (half the cache lines of 64-byte row pieces)
  // a deferred norm needs the large-M kernel's K split along the segments
  const bool defer_big = defer && p0.nrm.inv_tmp && gemm_big_splits(p0, p0.nrm.segs) > 0;
  const bool to_big = sizeof(S) == 2 && p0.M >= 128 && p0.K >= 64 && norm &&
                      norm_packable(p0.nrm.seg_len, !p0.nrm.x_f32) &&
                      (am || gemm_big_splits(p0, defer_big ? p0.nrm.segs : 1) > 0);
  const GemmParams p = norm ? norm_first<S>(p0, s, to_big, defer_big && to_big) : p0;
  // 128-wide tiles only when they still give every CU two workgroups (the
  // N = 2,880 projections get 64 x 64 tiles)
  const bool big = p.M >= 256 && (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128) >= 512;
  // bf16 batches of 128+ rows: the LDS-tiled kernel of gemm_big.hip (the LM
  // head always, the other contractions when they split K)
  if (sizeof(S) == 2 && p.M >= 128 && p.K >= 64) {
    const int r = launch_gemm_big(p, s);
    if (r >= 0) return r;
  }
  if (am && p.epi.kind == EPI_LSE)
    return big ? launch_tiled<S, 128, 128, false, true, true>(p, s) : launch_tiled<S, 64, 64, false, true, true>(p, s);
  if (am) return big ? launch_tiled<S, 128, 128, false, true>(p, s) : launch_tiled<S, 64, 64, false, true>(p, s);
  // the gate/up pair keeps 128 x 64 tiles from 256 rows on (two weight streams per tile)
  if (dual) { if (p.M >= 256) launch_tiled<S, 128, 64, true, false>(p, s); else launch_tiled<S, 64, 64, true, false>(p, s); }
  else { if (big) launch_tiled<S, 128, 128, false, false>(p, s); else launch_tiled<S, 64, 64, false, false>(p, s); }
  return 0;
}

int launch_gemm(const GemmParams& p, int bf16, hipStream_t s) {
  return bf16 ? launch_gemm_t<uint16_t>(p, s) : launch_gemm_t<float>(p, s);
}

}  // namespace pe
