// Small bandwidth-bound passes that prepare the fp16 operands of the MLP.
// The MLP's contraction inputs (its input rows h1 and the GELU output H, 16384
// wide at the 7B shape) are where 16-bit rounding costs most: rounded to bf16
// (8 significant bits) they leave an error of about 5e-3 per output at the 7B
// shape, fp16 (11 bits) about 6e-4.  fp16 has a narrow range, so each token
// row is stored scaled by a power of two taken from the RMS of the MLP input
// row (exact, undone in the epilogues), and the weight shards that meet fp16
// operands are converted to fp16 once per call.
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int RMS_WAVES = 4;  // rows per 256-thread workgroup

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(r[j] << 16);
    v[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = a[j];
    v[4 + j] = b[j];
  }
}

// One wave per row: fp32 sum of squares over 8-element pieces, butterfly
// reduction, exponent of the rms, then (optionally) the scaled fp16 copy.
template <typename T>
__global__ __launch_bounds__(64 * RMS_WAVES) void row_prep_kernel(const T* __restrict__ x, int64_t n, int32_t h,
                                                                  int32_t* __restrict__ row_exp,
                                                                  uint16_t* __restrict__ x16) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * RMS_WAVES + (threadIdx.x >> 6);
  if (row >= n) return;
  const T* xr = x + row * h;
  float ss = 0.0f;
  for (int c = lane * 8; c < h; c += 64 * 8) {
    float v[8];
    load8(xr + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float rms = sqrtf(ss / (float)h);
  int e = 0;
  if (rms > 0.0f && rms <= 3.0e38f) {
    e = (int)((__float_as_uint(rms) >> 23) & 0xffu) - 127;  // floor(log2(rms)) for a normal rms
    e = max(e, -100);
  }
  if (lane == 0) row_exp[row] = e;
  if (x16) {
    uint16_t* orow = x16 + row * h;
    for (int c = lane * 8; c < h; c += 64 * 8) {
      float v[8];
      load8(xr + c, v);
      u32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        r[j] = pack_f16x2_sat(__builtin_amdgcn_ldexpf(v[2 * j], -e), __builtin_amdgcn_ldexpf(v[2 * j + 1], -e));
      *reinterpret_cast<u32x4*>(orow + c) = r;
    }
  }
}

struct ShardPtrs {
  const uint16_t* p[TSP_MAX_D];
};

// Grid-stride bf16 -> fp16 over one shard per blockIdx.y, 8 elements per step.
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const ShardPtrs src, uint16_t* __restrict__ dst,
                                                          int64_t count) {
  const uint16_t* s = src.p[blockIdx.y];
  uint16_t* o = dst + (int64_t)blockIdx.y * count;
  const int64_t n8 = count / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(s + i * 8);
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = pack_f16x2_sat(__uint_as_float(v[j] << 16), __uint_as_float(v[j] & 0xffff0000u));
    *reinterpret_cast<u32x4*>(o + i * 8) = r;
  }
}

// Simulated arrival of weight shards (one workgroup).  Shard i is released
// (i + 1) * delay_ticks after the kernel starts: its bytes are copied, written
// back to memory by a system-scope release fence in every wave, and after a
// barrier the counter is raised to base + i + 1 with a system-scope store.
__global__ __launch_bounds__(1024) void simulate_arrival_kernel(const ArrivalCopies c, int32_t n,
                                                                uint32_t* __restrict__ counter, uint32_t base,
                                                                uint64_t delay_ticks) {
  typedef __attribute__((address_space(1))) uint32_t gu32;
  const uint64_t t0 = wall_clock64();  // 100 MHz
  for (int i = 0; i < n; ++i) {
    const uint64_t due = (uint64_t)(i + 1) * delay_ticks;
    while (wall_clock64() - t0 < due) __builtin_amdgcn_s_sleep(8);  // ends: the clock advances
    const u32x4* src = static_cast<const u32x4*>(c.src[i]);
    u32x4* dst = static_cast<u32x4*>(c.dst[i]);
    const int64_t n16 = (int64_t)(c.bytes[i] / 16);
    constexpr int U = 8;  // loads in flight per thread
    int64_t j = threadIdx.x;
    for (; j + (U - 1) * (int64_t)blockDim.x < n16; j += U * (int64_t)blockDim.x) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = src[j + u * (int64_t)blockDim.x];
#pragma unroll
      for (int u = 0; u < U; ++u) dst[j + u * (int64_t)blockDim.x] = v[u];
    }
    for (; j < n16; j += blockDim.x) dst[j] = src[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store((gu32*)counter, base + (uint32_t)i + 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace

hipError_t launch_simulate_arrival(const ArrivalCopies& c, int32_t n, uint32_t* counter, uint32_t base,
                                   uint64_t delay_ticks, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(simulate_arrival_kernel, dim3(1), dim3(1024), 0, stream, c, n, counter, base, delay_ticks);
  return hipGetLastError();
}

hipError_t launch_row_prep(const void* x, int32_t x_f32, int64_t n, int32_t h, int32_t* row_exp, uint16_t* x16,
                           hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + RMS_WAVES - 1) / RMS_WAVES)), block(64 * RMS_WAVES);
  if (x_f32)
    hipLaunchKernelGGL(row_prep_kernel<float>, grid, block, 0, stream, static_cast<const float*>(x), n, h, row_exp,
                       x16);
  else
    hipLaunchKernelGGL(row_prep_kernel<uint16_t>, grid, block, 0, stream, static_cast<const uint16_t*>(x), n, h,
                       row_exp, x16);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f16(const uint16_t* const* src, uint16_t* dst, int32_t D, int64_t count,
                              hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  ShardPtrs sp{};
  for (int d = 0; d < D; ++d) sp.p[d] = src[d];
  const int64_t n8 = count / 8;
  const unsigned bx = (unsigned)std::min<int64_t>((n8 + 255) / 256, 1024);
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3(bx, D), dim3(256), 0, stream, sp, dst, count);
  return hipGetLastError();
}

}  // namespace tsp
