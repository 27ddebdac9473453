// RMSNorm of row segments, written in the matrix-core operand type:
//   out[i][s*d + c] = x[row_i][s*d + c] * g[s*d + c] / sqrt(mean_c x[row_i][s*d + c]^2 + eps)
// ("Attention Drift", section 4.1: RMS is ||x||_2 / sqrt(d); Observation 2:
// each captured target stream is normalised on its own).
//
// One workgroup per (row, segment).  Every 16-byte chunk of the row segment is
// loaded into registers up front (at most kNormMaxChunks per thread), so the
// kernel costs one memory round trip, one workgroup reduction and one store.
// Rows flagged in `skip` are written as zeros; bf16 output can also go to
// the matrix-core operand layout of the large-M contractions (`packed`).  Block (0, 0) also clears the
// split-K tile counters of the contraction that consumes this output.
#include "kernels.h"

namespace pe {

template <typename Sin, typename Sout>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(NormParams p) {
  constexpr int CI = 16 / sizeof(Sin);  // input elements per 16-byte chunk
  const int i = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x;
  if (p.zero && i == 0 && seg == 0)
    for (int j = tid; j < p.nzero; j += 256) p.zero[j] = 0;
  const bool pad = i >= p.n;  // padding rows of the packed layout
  const int row = pad ? 0 : (p.rows ? p.rows[i] : i);
  const bool skip = pad || (p.skip && p.skip[row]);
  const char* x = reinterpret_cast<const char*>(p.in) + ((int64_t)row * p.ld_in + (int64_t)seg * p.d) * sizeof(Sin);
  const float* gain = p.gain + (int64_t)seg * p.d;
  Sout* out = reinterpret_cast<Sout*>(p.out) + (int64_t)i * p.ld_out + (int64_t)seg * p.d;
  // element k of this row segment (k a multiple of 4 here)
  auto dst = [&](int k) -> Sout* {
    if (!p.packed) return out + k;
    const int col = seg * p.d + k;
    const int64_t chunk = (int64_t)(i >> 4) * (p.ld_out >> 5) + (col >> 5);
    return reinterpret_cast<Sout*>(p.out) + chunk * 512 + (((col >> 3) & 3) * 16 + (i & 15)) * 8 + (col & 7);
  };
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
  const float inv = skip ? 0.f : 1.0f / sqrtf(tot / (float)p.d + p.eps);
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
        *reinterpret_cast<u32x4*>(dst(e0)) = w;
      } else {
        u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<u32x2*>(dst(e0)) = w;
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

void launch_rmsnorm_rows(const NormParams& p, int in_bf16, int out_bf16, hipStream_t s) {
  dim3 grid(p.packed ? (p.n + 15) / 16 * 16 : p.n, p.segs);
  if (in_bf16 && out_bf16) hipLaunchKernelGGL((rmsnorm_rows_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, s, p);
  else if (!in_bf16 && out_bf16) hipLaunchKernelGGL((rmsnorm_rows_kernel<float, uint16_t>), grid, dim3(256), 0, s, p);
  else if (in_bf16 && !out_bf16) hipLaunchKernelGGL((rmsnorm_rows_kernel<uint16_t, float>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((rmsnorm_rows_kernel<float, float>), grid, dim3(256), 0, s, p);
}

}  // namespace pe
