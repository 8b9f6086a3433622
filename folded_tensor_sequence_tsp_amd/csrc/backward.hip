// Helpers of the MLP backward: the GEMM engine contracts two K-contiguous
// operands (C = A B^T), so the products of the backward whose contraction runs
// over the other index of a stored matrix (dH = dY W2, dX = dU W1, and the
// weight gradients over tokens) take one operand transposed first.  A tiled
// transpose through LDS: bandwidth-bound, small next to the GEMMs it feeds.
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int TT = 64;  // tile edge

// dst[c * ld_out + r] = f(src[r * ld_in + c]): tile (c0, r0) of 64 x 64.  Loads
// are 8 consecutive elements along c (16 or 32 bytes), stores 8 consecutive
// along r (16 bytes); the tile sits in LDS as fp32 with rows padded by one
// element, so the column reads of the store phase spread over the banks.
template <bool SRC_F32, bool GELU>
__global__ __launch_bounds__(256) void transpose_kernel(const void* __restrict__ src, int64_t R, int64_t C,
                                                        int64_t ld_in, uint16_t* __restrict__ dst, int64_t ld_out) {
  __shared__ float tile[TT][TT + 1];
  const int64_t c0 = (int64_t)blockIdx.x * TT;
  const int64_t r0 = (int64_t)blockIdx.y * TT;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = k * 256 + threadIdx.x;  // 512 pieces: row q / 8, columns 8 * (q % 8) .. +7
    const int rr = q >> 3, cc = (q & 7) * 8;
    const int64_t r = r0 + rr;
    float v[8];
    if (r < R) {
      if constexpr (SRC_F32) {
        const float* p = static_cast<const float*>(src) + r * ld_in + c0 + cc;
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = a[j];
          v[4 + j] = b[j];
        }
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + r * ld_in + c0 + cc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = __uint_as_float(w[j] << 16);
          v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if constexpr (GELU) v[j] = gelu_tanh(v[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[rr][cc + j] = v[j];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = k * 256 + threadIdx.x;  // output row c0 + q / 8, columns r0 + 8 * (q % 8) .. +7
    const int cc = q >> 3, rr = (q & 7) * 8;
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(tile[rr + 2 * j][cc], tile[rr + 2 * j + 1][cc]);
    *reinterpret_cast<u32x4*>(dst + (c0 + cc) * ld_out + r0 + rr) = w;
  }
}

// 8 consecutive elements of one row per thread: two 16-byte loads, one 16-byte store.
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ src, int64_t R, int64_t C,
                                                          int64_t ld_in, uint16_t* __restrict__ dst, int64_t ld_out) {
  const int64_t per_row = C / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * per_row) return;
  const int64_t r = i / per_row, c = (i - r * per_row) * 8;
  const float* p = src + r * ld_in + c;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  *reinterpret_cast<u32x4*>(dst + r * ld_out + c) =
      u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) p[i] = 0.0f;
}

}  // namespace

hipError_t launch_zero_f32(float* p, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, p, count);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, int64_t R, int64_t C, int64_t ld_in, uint16_t* dst, int64_t ld_out,
                              hipStream_t stream) {
  const int64_t items = R * (C / 8);
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, src, R, C,
                     ld_in, dst, ld_out);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int32_t src_f32, int32_t gelu, int64_t R, int64_t C, int64_t ld_in,
                            uint16_t* dst, int64_t ld_out, hipStream_t stream) {
  if (C <= 0 || ld_out <= 0) return hipSuccess;
  const dim3 grid((unsigned)(C / TT), (unsigned)(ld_out / TT)), block(256);
  if (src_f32 && gelu)
    hipLaunchKernelGGL((transpose_kernel<true, true>), grid, block, 0, stream, src, R, C, ld_in, dst, ld_out);
  else if (src_f32)
    hipLaunchKernelGGL((transpose_kernel<true, false>), grid, block, 0, stream, src, R, C, ld_in, dst, ld_out);
  else if (gelu)
    hipLaunchKernelGGL((transpose_kernel<false, true>), grid, block, 0, stream, src, R, C, ld_in, dst, ld_out);
  else
    hipLaunchKernelGGL((transpose_kernel<false, false>), grid, block, 0, stream, src, R, C, ld_in, dst, ld_out);
  return hipGetLastError();
}

}  // namespace tsp
