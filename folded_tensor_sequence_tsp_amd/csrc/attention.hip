// Causal flash attention of a rank's two zigzag query chunks against the whole
// gathered K/V, for gfx950 (CDNA4).
//
// TSP gathers K/V over a zigzag partition of the sequence so that every rank
// holds one early and one late chunk of queries and the same causal work
// (zubnet.ai, "Zyphra TSP folds TP+SP onto one GPU axis", para. 2).  Here the
// queries of chunk i sit at global positions chunk_start[i] + row; a query at
// position p attends to keys 0..p of the full sequence.
//
// Design (one workgroup = one head x one tile of QT = 32 * NWAVES queries of
// one chunk; each wave owns 32 queries):
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     each lane then holds ONE query (lane % 32) and 16 keys per 32-key block,
//     so the row max needs a single exchange with lane ^ 32 and the row sums
//     stay per lane until the end;
//   * O^T = V^T P^T reuses the score registers directly as the B operand (no
//     LDS round trip for P); V is staged in LDS transposed, [d][key], with the
//     keys of each 16-key group permuted so every lane's 8 keys of a k-step are
//     one 16-byte read;
//   * online softmax in fp32 in the log2 domain (scale folded into one FMA,
//     hardware exp2), masking only on the tiles that cross the diagonal, and
//     whole tiles past a wave's last query skipped;
//   * K/V tiles of 64 keys are double-buffered in LDS with a register prefetch
//     of the next tile; one barrier per tile;
//   * workgroups are ordered so each XCD works through a contiguous range of
//     heads (its concurrent tiles stream the same K/V through its L2), heaviest
//     (latest) query tiles first.
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int QT = 32 * NWAVES;  // queries per workgroup
constexpr int BKV = 64;          // keys per tile

template <int HD>
struct ACfg {
  static constexpr int KLD = HD + 8;          // K row in LDS (bf16), padded
  static constexpr int VLD = BKV + 8;         // V^T row in LDS (bf16), padded
  static constexpr int K_ELEMS = BKV * KLD;
  static constexpr int V_ELEMS = HD * VLD;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int DCH = HD / 8;                    // 16-byte chunks per key row
  static constexpr int K_CHUNKS = BKV * DCH / NTHREADS; // K loads per thread
  static constexpr int V_BLOCKS = (BKV / 4) * DCH;      // 4 keys x 8 dims blocks
  static constexpr int KK = HD / 16;                    // MFMA k-steps over head_dim
  static constexpr int DT = HD / 32;                    // 32-wide d tiles of O
};

// Physical slot of logical key w (0..15) inside a 16-key group of V^T: the
// 4-key blocks are stored in the order 0, 2, 1, 3 so that lane half h finds
// its keys {4h..4h+3, 8+4h..8+4h+3} at slots 8h..8h+7.
__device__ __forceinline__ int vt_block_slot(int block4) { return ((block4 & 1) << 1) | (block4 >> 1); }

template <int HD>
__global__ __launch_bounds__(NTHREADS) void attn_kernel(const AttnArgs a) {
  using C = ACfg<HD>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::BUF_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int ql = lane & 31;

  // ---- work item: (head, chunk, tile), heaviest tiles of a head first, heads
  // contiguous per XCD.
  const int tpc = (int)((a.chunk_len + QT - 1) / QT);
  const int per_head = 2 * tpc;
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int head = pid / per_head;
  const int w = pid - head * per_head;
  const int chunk = w < tpc ? 1 : 0;
  const int tile = w < tpc ? tpc - 1 - w : per_head - 1 - w;

  const int64_t row0 = (int64_t)chunk * a.chunk_len + (int64_t)tile * QT;  // local row of query 0
  const int64_t pos0 = (chunk ? a.chunk_start1 : a.chunk_start0) + (int64_t)tile * QT;
  const int valid = (int)min((int64_t)QT, a.chunk_len - (int64_t)tile * QT);
  const int64_t key_end = pos0 + valid;  // keys [0, key_end)
  const int n_tiles = (int)((key_end + BKV - 1) / BKV);

  // This lane's query (clamped to the last valid row for the ragged tail).
  const int qi = min(wave * 32 + ql, valid - 1);
  const int64_t qpos = pos0 + qi;
  const int wave_first = wave * 32;
  const bool wave_active = wave_first < valid;
  const int64_t wave_min_pos = pos0 + wave_first;
  const int64_t wave_max_pos = pos0 + min(wave_first + 31, valid - 1);

  const int hcol = head * HD;
  const int64_t ld = a.hidden;

  // ---- Q fragments in registers: lane holds query ql, dims kk*16 + 8*half .. +7.
  bf16x8 qf[C::KK];
  {
    const uint16_t* qp = a.q + (row0 + qi) * ld + hcol + 8 * half;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + kk * 16));
  }

  // ---- K/V tile loading.
  // K: chunk c = i*NTHREADS + tid -> key c / DCH, dims (c % DCH) * 8.
  // V: block tid -> keys 4*(tid % 16) .. +3, dims (tid / 16) * 8 .. +7 (16
  // consecutive lanes fill one 128-byte row of V^T: conflict-free LDS writes).
  u32x4 rk[C::K_CHUNKS];
  u32x4 rv[4];
  const bool v_loader = tid < C::V_BLOCKS;
  const int v_kg = tid & 15;
  const int v_dc = tid >> 4;
  auto load_tile = [&](int t) {
    const int64_t k0 = (int64_t)t * BKV;
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
      const int c = i * NTHREADS + tid;
      const int key = c / C::DCH;
      const int dc = c - key * C::DCH;
      const int64_t gk = min(k0 + key, key_end - 1);
      rk[i] = *reinterpret_cast<const u32x4*>(a.k + gk * ld + hcol + dc * 8);
    }
    if (v_loader) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t gk = min(k0 + 4 * v_kg + j, key_end - 1);
        rv[j] = *reinterpret_cast<const u32x4*>(a.v + gk * ld + hcol + v_dc * 8);
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = lds + buf * C::BUF_ELEMS;
    uint16_t* vt = ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
      const int c = i * NTHREADS + tid;
      const int key = c / C::DCH;
      const int dc = c - key * C::DCH;
      *reinterpret_cast<u32x4*>(ks + key * C::KLD + dc * 8) = rk[i];
    }
    if (v_loader) {
      // transpose the 4 keys x 8 dims block: for dim j, pack keys 0..3.
      const int slot = (v_kg >> 2) * 16 + vt_block_slot(v_kg & 3) * 4;
#pragma unroll
      for (int jw = 0; jw < 4; ++jw) {
        const uint32_t x0 = rv[0][jw], x1 = rv[1][jw], x2 = rv[2][jw], x3 = rv[3][jw];
        u32x2 lo, hi;  // dims 2*jw (low halves) and 2*jw+1 (high halves)
        lo[0] = (x0 & 0xffffu) | (x1 << 16);
        lo[1] = (x2 & 0xffffu) | (x3 << 16);
        hi[0] = (x0 >> 16) | (x1 & 0xffff0000u);
        hi[1] = (x2 >> 16) | (x3 & 0xffff0000u);
        const int d = v_dc * 8 + 2 * jw;
        *reinterpret_cast<u32x2*>(vt + d * C::VLD + slot) = lo;
        *reinterpret_cast<u32x2*>(vt + (d + 1) * C::VLD + slot) = hi;
      }
    }
  };

  // ---- running state (log2 domain): m = max of scaled scores, l = lane-partial sum.
  constexpr float inv_sqrt_hd = HD == 128 ? 0.08838834764831844055f : 0.125f;
  const float scale_log2 = 1.44269504088896340736f * inv_sqrt_hd;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const int64_t k0 = (int64_t)t * BKV;
    if (wave_active && k0 <= wave_max_pos) {
      const uint16_t* ks = lds + buf * C::BUF_ELEMS;
      const uint16_t* vt = ks + C::K_ELEMS;
      // S^T for two 32-key blocks: lane holds query ql, keys 8*(e/4)+4*half+e%4.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* kp = ks + (kb * 32 + ql) * C::KLD + 8 * half;
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk)
          s[kb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(kp + kk * 16)), qf[kk], s[kb]);
      }
      // scale into the log2 domain; mask keys past the query on diagonal tiles.
      const bool diag = k0 + BKV - 1 > wave_min_pos;
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = s[kb][e] * scale_log2;
          if (diag) {
            const int64_t key = k0 + kb * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            if (key > qpos) x = -INFINITY;
          }
          s[kb][e] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      // probabilities -> bf16 B operands; lane-partial row sum.
      bf16x8 pf[4];
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          u32x4 packed;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p0 = __builtin_amdgcn_exp2f(s[kb][8 * g + 2 * j] - m_new);
            const float p1 = __builtin_amdgcn_exp2f(s[kb][8 * g + 2 * j + 1] - m_new);
            lsum += p0 + p1;
            packed[j] = pack_bf16x2(p0, p1);
          }
          pf[2 * kb + g] = as_bf16x8(packed);
        }
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
      // O^T += V^T P^T over the tile's four 16-key steps.
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const uint16_t* vp = vt + (dt * 32 + ql) * C::VLD + 8 * half;
#pragma unroll
        for (int ks16 = 0; ks16 < 4; ++ks16)
          o[dt] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(vp + ks16 * 16)), pf[ks16], o[dt]);
      }
    }
    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds query ql, dims dt*32 + 8*(e/4) + 4*half + e%4.
  if (wave_active) {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (wave_first + ql < valid) {
      const float inv = 1.0f / l_tot;
      const int64_t off = (row0 + wave_first + ql) * ld + hcol + 4 * half;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float r[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = o[dt][4 * g + j] * inv;
          u32x2 v;
          v[0] = pack_bf16x2(r[0], r[1]);
          v[1] = pack_bf16x2(r[2], r[3]);
          *reinterpret_cast<u32x2*>(a.o + off + dt * 32 + 8 * g) = v;
          if (a.o_lo) {  // rounding residual: r - bf16(r), itself rounded to bf16
            u32x2 w;
            w[0] = pack_bf16x2(r[0] - __uint_as_float(v[0] << 16), r[1] - __uint_as_float(v[0] & 0xffff0000u));
            w[1] = pack_bf16x2(r[2] - __uint_as_float(v[1] << 16), r[3] - __uint_as_float(v[1] & 0xffff0000u));
            *reinterpret_cast<u32x2*>(a.o_lo + off + dt * 32 + 8 * g) = w;
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.chunk_len <= 0) return hipSuccess;
  const int tpc = (int)((a.chunk_len + QT - 1) / QT);
  const dim3 grid(a.n_heads * 2 * tpc), block(NTHREADS);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(attn_kernel<128>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(attn_kernel<64>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace tsp
