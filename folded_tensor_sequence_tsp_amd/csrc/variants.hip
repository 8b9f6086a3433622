// Layer variants of a real decoder (not on the TSP pages, whose layer has no
// norm and no positional encoding): RMSNorm and the rotary position embedding
// of the local queries and the rank's own keys at their global zigzag
// positions.  Both are bandwidth-bound row passes.
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int NORM_WAVES = 4;  // rows per 256-thread workgroup

// y = x / sqrt(mean(x^2) + eps) * gain, one wave per row (RMSNorm, Zhang &
// Sennrich 2019): fp32 sum of squares over 8-element pieces, butterfly
// reduction, then the scaled bf16 row.
__global__ __launch_bounds__(64 * NORM_WAVES) void rms_norm_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ gain, int64_t n,
                                                                    int32_t h, float eps, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * NORM_WAVES + (threadIdx.x >> 6);
  if (row >= n) return;
  const uint16_t* xr = x + row * h;
  float ss = 0.0f;
  for (int c = lane * 8; c < h; c += 64 * 8) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(xr + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = __uint_as_float(r[j] << 16), b = __uint_as_float(r[j] & 0xffff0000u);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.0f / sqrtf(ss / (float)h + eps);
  uint16_t* yr = y + row * h;
  for (int c = lane * 8; c < h; c += 64 * 8) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(xr + c);
    const u32x4 gw = *reinterpret_cast<const u32x4*>(gain + c);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = __uint_as_float(r[j] << 16) * inv * __uint_as_float(gw[j] << 16);
      const float b = __uint_as_float(r[j] & 0xffff0000u) * inv * __uint_as_float(gw[j] & 0xffff0000u);
      o[j] = pack_bf16x2(a, b);
    }
    *reinterpret_cast<u32x4*>(yr + c) = o;
  }
}

// Rotary embedding (RoFormer, Su et al. 2021, interleaved pairs): thread
// (row, i) rotates the pair (x_{2i}, x_{2i+1}) of every head of local row
// `row` by angle = p * theta^(-2i/hd), p the row's global position.  The
// rotated row is row `row` of x, or (at_global) row p of x: the rank's own
// rows of a full-sequence tensor.  The angle and its cosine and sine are taken
// in fp64 (p reaches 10^5 rad, where an fp32 angle would already be off by
// about 1e-2), then the rotation runs in fp32.
__global__ __launch_bounds__(256) void rope_kernel(uint16_t* __restrict__ x, int64_t n_rows, int64_t ld,
                                                   int32_t n_heads, int32_t head_dim, double log2_theta,
                                                   int64_t chunk_len, int64_t start0, int64_t start1,
                                                   int32_t at_global) {
  const int half = head_dim / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / half;
  const int i = (int)(idx - row * half);
  if (row >= n_rows) return;
  const int64_t pos = row < chunk_len ? start0 + row : start1 + (row - chunk_len);
  const double ang = (double)pos * exp2(-2.0 * (double)i / (double)head_dim * log2_theta);
  double sd, cd;
  sincos(ang, &sd, &cd);
  const float c = (float)cd, s = (float)sd;
  uint32_t* p = reinterpret_cast<uint32_t*>(x + (at_global ? pos : row) * ld) + i;
  for (int a = 0; a < n_heads; ++a) {
    const uint32_t w = p[a * half];
    const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xffff0000u);
    p[a * half] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
  }
}

}  // namespace

hipError_t launch_rms_norm(const uint16_t* x, const uint16_t* gain, int64_t n, int32_t h, float eps, uint16_t* y,
                           hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + NORM_WAVES - 1) / NORM_WAVES));
  hipLaunchKernelGGL(rms_norm_kernel, grid, dim3(64 * NORM_WAVES), 0, stream, x, gain, n, h, eps, y);
  return hipGetLastError();
}

hipError_t launch_rope(uint16_t* x, int64_t n_rows, int64_t ld, int32_t n_heads, int32_t head_dim, double theta,
                       int64_t chunk_len, int64_t start0, int64_t start1, int32_t at_global, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t threads = n_rows * (head_dim / 2);
  const dim3 grid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL(rope_kernel, grid, dim3(256), 0, stream, x, n_rows, ld, n_heads, head_dim, log2(theta),
                     chunk_len, start0, start1, at_global);
  return hipGetLastError();
}

}  // namespace tsp
