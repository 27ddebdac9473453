// RMSNorm of row segments, written in the matrix-core operand type:
//   out[i][s*d + c] = x[row_i][s*d + c] * g[s*d + c] / sqrt(mean_c x[row_i][s*d + c]^2 + eps)
// ("Attention Drift", section 4.1: RMS is ||x||_2 / sqrt(d); Observation 2:
// each captured target stream is normalised on its own).
//
// One workgroup per (row, segment).  Every 16-byte chunk of the row segment is
// loaded into registers up front (at most kNormMaxChunks per thread), so the
// kernel costs one memory round trip, one workgroup reduction and one store.
// Rows flagged in `skip` are written as zeros.  bf16 output can also go to
// the matrix-core operand layout of the large-M contractions (`packed`,
// rmsnorm_packed_kernel below).  Block (0, 0) also clears the
// split-K tile counters of the contraction that consumes this output.  With
// inv_out the 1 / rms of each row segment goes there and the output is
// x * g only (the consuming contraction scales its sums).
#include "kernels.h"

namespace pe {

template <typename Sin, typename Sout>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(NormParams p) {
  constexpr int CI = 16 / sizeof(Sin);  // input elements per 16-byte chunk
  const int i = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x;
  if (p.zero && i == 0 && seg == 0)
    for (int j = tid; j < p.nzero; j += 256) p.zero[j] = 0;
  const int row = p.rows ? p.rows[i] : i;
  const bool skip = p.skip && p.skip[row];
  const char* x = reinterpret_cast<const char*>(p.in) + ((int64_t)row * p.ld_in + (int64_t)seg * p.d) * sizeof(Sin);
  const float* gain = p.gain + (int64_t)seg * p.d;
  Sout* out = reinterpret_cast<Sout*>(p.out) + (int64_t)i * p.ld_out + (int64_t)seg * p.d;
  const int nch = p.d / CI;
  float v[kNormMaxChunks][CI];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {
    const int ch = tid + c * 256;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (ch < nch && !skip) raw = ld16(x + (int64_t)ch * 16);
#pragma unroll
    for (int e = 0; e < CI; ++e) {
      float f;
      if constexpr (sizeof(Sin) == 2) f = bf2f((uint16_t)(raw[e >> 1] >> (16 * (e & 1))));
      else f = __uint_as_float(raw[e]);
      v[c][e] = f;
      ss += f * f;
    }
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv0 = skip ? 0.f : 1.0f / sqrtf(tot / (float)p.d + p.eps);
  if (p.inv_out && tid == 0) p.inv_out[(int64_t)i * p.segs + seg] = inv0;
  const float inv = p.inv_out ? (skip ? 0.f : 1.f) : inv0;
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {
    const int ch = tid + c * 256;
    if (ch >= nch) continue;
    const int e0 = ch * CI;
    float y[CI];
#pragma unroll
    for (int e = 0; e < CI; ++e) y[e] = v[c][e] * inv * gain[e0 + e];
    if constexpr (sizeof(Sout) == 2) {
      if constexpr (CI == 8) {
        u32x4 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
        *reinterpret_cast<u32x4*>(out + e0) = w;
      } else {
        u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<u32x2*>(out + e0) = w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < CI; e += 4) {
        f32x4 w = {y[e], y[e + 1], y[e + 2], y[e + 3]};
        *reinterpret_cast<f32x4*>(out + e0 + e) = w;
      }
    }
  }
}

// The same normalisation written in the matrix-core operand layout
// (NormParams::packed): one workgroup of 16 waves per (16-row group,
// segment, column share), a wave per row.  Each wave loads its row segment at
// once (at most kPackedMaxChunks 16-byte chunks per lane), reduces the
// squares, and writes the scaled bf16 values of the workgroup's column share
// into LDS; then the workgroup copies that share's 1 KB chunks out in order
// (lane slot 16 c + r = row r, 8 columns), so every store is part of a
// contiguous chunk.  Column shares (gridDim.z) only exist to occupy more CUs;
// each recomputes the row sums from L2.  Rows past n, and skipped rows, are
// zeros.
template <typename Sin>
__global__ __launch_bounds__(1024) void rmsnorm_packed_kernel(NormParams p) {
  constexpr int CI = 16 / sizeof(Sin);
  extern __shared__ __attribute__((aligned(16))) char lds[];  // 16 rows of the share, stride 64 (k1 - k0) + 16 bytes
  const int grp = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x, lane = tid & 63, rl = tid >> 6;
  const int kch = p.d / 32;  // 32-column chunks of this segment; this workgroup's share:
  const int k0 = kch * (int)blockIdx.z / (int)gridDim.z, k1 = kch * ((int)blockIdx.z + 1) / (int)gridDim.z;
  if (p.zero && grp == 0 && seg == 0 && blockIdx.z == 0)
    for (int j = tid; j < p.nzero; j += 1024) p.zero[j] = 0;
  const int i = grp * 16 + rl;
  const int row = i < p.n ? (p.rows ? p.rows[i] : i) : 0;
  const bool skip = i >= p.n || (p.skip && p.skip[row]);
  const char* x = reinterpret_cast<const char*>(p.in) + ((int64_t)row * p.ld_in + (int64_t)seg * p.d) * sizeof(Sin);
  const int nch = p.d / CI;
  u32x4 raw[kPackedMaxChunks];
#pragma unroll
  for (int c = 0; c < kPackedMaxChunks; ++c) {
    const int ch = lane + 64 * c;
    raw[c] = u32x4{0u, 0u, 0u, 0u};
    if (ch < nch && !skip) raw[c] = ld16(x + (int64_t)ch * 16);
  }
  auto elem = [&](const u32x4& r, int e) -> float {
    if constexpr (sizeof(Sin) == 2) return bf2f((uint16_t)(r[e >> 1] >> (16 * (e & 1))));
    else return __uint_as_float(r[e]);
  };
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kPackedMaxChunks; ++c)
#pragma unroll
    for (int e = 0; e < CI; ++e) ss += elem(raw[c], e) * elem(raw[c], e);
  ss = wave_sum(ss);
  const float inv0 = skip ? 0.f : 1.0f / sqrtf(ss / (float)p.d + p.eps);
  if (p.inv_out && blockIdx.z == 0 && lane == 0 && i < p.n) p.inv_out[(int64_t)i * p.segs + seg] = inv0;
  const float inv = p.inv_out ? (skip ? 0.f : 1.f) : inv0;
  const float* gain = p.gain + (int64_t)seg * p.d;
  const int rs = 64 * (k1 - k0) + 16;
  char* lrow = lds + rl * rs - k0 * 64;  // column k of the share at byte 2 k
#pragma unroll
  for (int c = 0; c < kPackedMaxChunks; ++c) {
    const int ch = lane + 64 * c;
    if (ch >= nch || ch * CI < k0 * 32 || ch * CI >= k1 * 32) continue;
    float y[CI];
#pragma unroll
    for (int e = 0; e < CI; ++e) y[e] = elem(raw[c], e) * inv * gain[ch * CI + e];
    if constexpr (CI == 8) {
      *reinterpret_cast<u32x4*>(lrow + ch * 16) =
          u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
    } else {
      *reinterpret_cast<u32x2*>(lrow + ch * 8) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    }
  }
  __syncthreads();
  const int64_t c0 = (int64_t)grp * (p.ld_out / 32) + (int64_t)seg * kch + k0;
  uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
  for (int it = tid; it < (k1 - k0) * 64; it += 1024) {
    const int S = it >> 6, l = it & 63;
    const u32x4 w = *reinterpret_cast<const u32x4*>(lds + (l & 15) * rs + (S * 32 + (l >> 4) * 8) * 2);
    *reinterpret_cast<u32x4*>(out + (c0 + S) * 512 + l * 8) = w;
  }
}

bool norm_packable(int d, int in_bf16) {
  const int ci = in_bf16 ? 8 : 4;
  return d % 32 == 0 && d / ci <= 64 * kPackedMaxChunks && 16 * (2 * d + 16) <= 160 * 1024;
}

void launch_rmsnorm_rows(const NormParams& p, int in_bf16, int out_bf16, hipStream_t s) {
  if (p.packed) {
    // operand layout (bf16 output; norm_packable(d, in_bf16) holds)
    if (p.n <= 0) return;
    // column shares until about 128 workgroups run
    const int groups = (p.n + 15) / 16 * p.segs;
    int shares = (128 + groups - 1) / groups;
    shares = shares < p.d / 32 ? shares : p.d / 32;
    const dim3 grid((p.n + 15) / 16, p.segs, shares);
    const size_t lds = (size_t)16 * (64 * ((p.d / 32 + shares - 1) / shares) + 16);
    // once per process per kernel (thread-safe initialisation; a failure
    // shows up as a failed launch)
    static const hipError_t attr_bf = hipFuncSetAttribute(reinterpret_cast<const void*>(&rmsnorm_packed_kernel<uint16_t>),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    static const hipError_t attr_f = hipFuncSetAttribute(reinterpret_cast<const void*>(&rmsnorm_packed_kernel<float>),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)attr_bf;
    (void)attr_f;
    if (in_bf16) hipLaunchKernelGGL(rmsnorm_packed_kernel<uint16_t>, grid, dim3(1024), lds, s, p);
    else hipLaunchKernelGGL(rmsnorm_packed_kernel<float>, grid, dim3(1024), lds, s, p);
    return;
  }
  dim3 grid(p.n, p.segs);
  if (in_bf16 && out_bf16) hipLaunchKernelGGL((rmsnorm_rows_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, s, p);
  else if (!in_bf16 && out_bf16) hipLaunchKernelGGL((rmsnorm_rows_kernel<float, uint16_t>), grid, dim3(256), 0, s, p);
  else if (in_bf16 && !out_bf16) hipLaunchKernelGGL((rmsnorm_rows_kernel<uint16_t, float>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((rmsnorm_rows_kernel<float, float>), grid, dim3(256), 0, s, p);
}

}  // namespace pe
