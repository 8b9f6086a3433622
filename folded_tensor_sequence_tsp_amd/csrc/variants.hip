// Layer variants of a real decoder (not on the TSP pages, whose layer has no
// norm and no positional encoding): RMSNorm and the rotary position embedding
// of the local queries and the rank's own keys at their global zigzag
// positions, and their backwards.  All are bandwidth-bound row passes.
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
// about 1e-2), then the rotation runs in fp32.  INVERSE rotates by -angle (the
// transpose of the rotation: the gradient of the forward); F32 works on fp32
// rows (gradients) instead of bf16.
template <bool F32, bool INVERSE>
__global__ __launch_bounds__(256) void rope_kernel(void* __restrict__ xv, int64_t n_rows, int64_t ld,
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
  const float c = (float)cd, s = INVERSE ? -(float)sd : (float)sd;
  const int64_t r = at_global ? pos : row;
  if constexpr (F32) {
    float2* p = reinterpret_cast<float2*>(static_cast<float*>(xv) + r * ld) + i;
    for (int a = 0; a < n_heads; ++a) {
      const float2 w = p[a * half];
      p[a * half] = make_float2(w.x * c - w.y * s, w.x * s + w.y * c);
    }
  } else {
    uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(xv) + r * ld) + i;
    for (int a = 0; a < n_heads; ++a) {
      const uint32_t w = p[a * half];
      const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xffff0000u);
      p[a * half] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
    }
  }
}

// Backward of RMSNorm for a block of RMS_BWD_ROWS rows (one wave per row in
// turn): with r = sqrt(mean x^2 + eps) and t = sum_j gain_j dy_j x_j,
//   dx_j = gain_j dy_j / r - x_j t / (h r^3)    (bf16 out),
// and the block's part of dgain_j = sum_rows dy_j x_j / r: each lane keeps its
// columns' sums in registers (columns lane*8 + 512*p .. +7), the waves add them
// in LDS once per block, and the block writes partial[block][j].
constexpr int RMS_BWD_MAXP = 16;  // 512-column passes: hidden <= 8192
__global__ __launch_bounds__(64 * NORM_WAVES) void rms_norm_bwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gain, const uint16_t* __restrict__ dy, int64_t n,
    int32_t h, float eps, uint16_t* __restrict__ dx, float* __restrict__ partial) {
  extern __shared__ float acc_lds[];  // [NORM_WAVES][h]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc[RMS_BWD_MAXP][8];
#pragma unroll
  for (int p = 0; p < RMS_BWD_MAXP; ++p)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[p][j] = 0.0f;
  const int64_t r0 = (int64_t)blockIdx.x * RMS_BWD_ROWS;
  for (int k = wave; k < RMS_BWD_ROWS; k += NORM_WAVES) {
    const int64_t row = r0 + k;
    if (row >= n) break;
    const uint16_t* xr = x + row * h;
    const uint16_t* gr = dy + row * h;
    float ss = 0.0f, t = 0.0f;
#pragma unroll
    for (int p = 0; p < RMS_BWD_MAXP; ++p) {
      const int c = lane * 8 + p * 512;
      if (c < h) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + c);
        const u32x4 gv = *reinterpret_cast<const u32x4*>(gr + c);
        const u32x4 wv = *reinterpret_cast<const u32x4*>(gain + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = __uint_as_float(xv[j] << 16), x1 = __uint_as_float(xv[j] & 0xffff0000u);
          const float g0 = __uint_as_float(gv[j] << 16), g1 = __uint_as_float(gv[j] & 0xffff0000u);
          const float w0 = __uint_as_float(wv[j] << 16), w1 = __uint_as_float(wv[j] & 0xffff0000u);
          ss = fmaf(x0, x0, fmaf(x1, x1, ss));
          t = fmaf(w0 * g0, x0, fmaf(w1 * g1, x1, t));
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      ss += __shfl_xor(ss, off);
      t += __shfl_xor(t, off);
    }
    const float inv = 1.0f / sqrtf(ss / (float)h + eps);
    const float coef = t * inv * inv * inv / (float)h;
    uint16_t* dr = dx + row * h;
#pragma unroll
    for (int p = 0; p < RMS_BWD_MAXP; ++p) {
      const int c = lane * 8 + p * 512;
      if (c < h) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + c);
        const u32x4 gv = *reinterpret_cast<const u32x4*>(gr + c);
        const u32x4 wv = *reinterpret_cast<const u32x4*>(gain + c);
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = __uint_as_float(xv[j] << 16), x1 = __uint_as_float(xv[j] & 0xffff0000u);
          const float g0 = __uint_as_float(gv[j] << 16), g1 = __uint_as_float(gv[j] & 0xffff0000u);
          const float w0 = __uint_as_float(wv[j] << 16), w1 = __uint_as_float(wv[j] & 0xffff0000u);
          o[j] = pack_bf16x2(w0 * g0 * inv - x0 * coef, w1 * g1 * inv - x1 * coef);
          acc[p][2 * j] = fmaf(g0 * x0, inv, acc[p][2 * j]);
          acc[p][2 * j + 1] = fmaf(g1 * x1, inv, acc[p][2 * j + 1]);
        }
        *reinterpret_cast<u32x4*>(dr + c) = o;
      }
    }
  }
  float* mine = acc_lds + (int64_t)wave * h;
#pragma unroll
  for (int p = 0; p < RMS_BWD_MAXP; ++p) {
    const int c = lane * 8 + p * 512;
    if (c < h) {
#pragma unroll
      for (int j = 0; j < 8; ++j) mine[c + j] = acc[p][j];
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < h; c += 64 * NORM_WAVES) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NORM_WAVES; ++w) v += acc_lds[(int64_t)w * h + c];
    partial[(int64_t)blockIdx.x * h + c] = v;
  }
}

// dgain[c] = sum over the row blocks of partial[block][c]: a workgroup owns 64
// columns; its 4 waves sum the blocks b = w, w+4, ... (one coalesced 256-byte
// row segment per load), then add their 4 sums in a fixed order.
__global__ __launch_bounds__(256) void rms_norm_bwd_reduce_kernel(const float* __restrict__ partial, int64_t blocks,
                                                                  int32_t h, float* __restrict__ dgain) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float v = 0.0f;
  if (c < h) {
    int64_t b = w;
    for (; b + 12 < blocks; b += 16)  // four independent loads in flight
      v += (partial[b * h + c] + partial[(b + 4) * h + c]) + (partial[(b + 8) * h + c] + partial[(b + 12) * h + c]);
    for (; b < blocks; b += 4) v += partial[b * h + c];
  }
  part[w][lane] = v;
  __syncthreads();
  if (w == 0 && c < h) dgain[c] = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
}

}  // namespace

hipError_t launch_rms_norm(const uint16_t* x, const uint16_t* gain, int64_t n, int32_t h, float eps, uint16_t* y,
                           hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + NORM_WAVES - 1) / NORM_WAVES));
  hipLaunchKernelGGL(rms_norm_kernel, grid, dim3(64 * NORM_WAVES), 0, stream, x, gain, n, h, eps, y);
  return hipGetLastError();
}

hipError_t launch_rope(void* x, int32_t x_f32, int32_t inverse, int64_t n_rows, int64_t ld, int32_t n_heads,
                       int32_t head_dim, double theta, int64_t chunk_len, int64_t start0, int64_t start1,
                       int32_t at_global, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t threads = n_rows * (head_dim / 2);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const double l2t = log2(theta);
  if (x_f32 && inverse)
    hipLaunchKernelGGL((rope_kernel<true, true>), grid, block, 0, stream, x, n_rows, ld, n_heads, head_dim, l2t,
                       chunk_len, start0, start1, at_global);
  else if (x_f32)
    hipLaunchKernelGGL((rope_kernel<true, false>), grid, block, 0, stream, x, n_rows, ld, n_heads, head_dim, l2t,
                       chunk_len, start0, start1, at_global);
  else if (inverse)
    hipLaunchKernelGGL((rope_kernel<false, true>), grid, block, 0, stream, x, n_rows, ld, n_heads, head_dim, l2t,
                       chunk_len, start0, start1, at_global);
  else
    hipLaunchKernelGGL((rope_kernel<false, false>), grid, block, 0, stream, x, n_rows, ld, n_heads, head_dim, l2t,
                       chunk_len, start0, start1, at_global);
  return hipGetLastError();
}

hipError_t launch_rms_norm_backward(const uint16_t* x, const uint16_t* gain, const uint16_t* dy, int64_t n,
                                    int32_t h, float eps, uint16_t* dx, float* dgain, float* partial,
                                    hipStream_t stream) {
  const int64_t blocks = rms_norm_bwd_blocks(n);
  if (blocks > 0) {
    hipLaunchKernelGGL(rms_norm_bwd_kernel, dim3((unsigned)blocks), dim3(64 * NORM_WAVES),
                       (size_t)NORM_WAVES * h * sizeof(float), stream, x, gain, dy, n, h, eps, dx, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(rms_norm_bwd_reduce_kernel, dim3((unsigned)((h + 63) / 64)), dim3(256), 0, stream, partial,
                     blocks, h, dgain);
  return hipGetLastError();
}

}  // namespace tsp
