// Backward of the causal attention of a rank's two zigzag query chunks against
// the whole gathered K/V, for gfx950 (CDNA4).
//
// With S = q k^T / sqrt(hd) (causal), P = softmax rows, o = P v and dO the
// gradient of o: dV = P^T dO, dP = dO V^T, dS = P * (dP - delta) with
// delta = rowsum(dO * o), dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd).  P is
// rebuilt from the scores and the forward's normaliser (no probabilities are
// stored).  dK and dV are this rank's contributions for every key row; in TSP
// the owners of the key rows would sum them over ranks, the reverse of the
// K/V all-gather (zubnet.ai, "Zyphra TSP folds TP+SP onto one GPU axis",
// para. 2).
//
// Two kernels, both with v_mfma_f32_32x32x16_bf16 and the operands of every
// product read straight from registers or LDS in the lane layout the MFMA
// wants (a 32x32 result holds, per lane, one column and 16 rows; fed back as
// the B operand those rows are the contraction index, in the order
// bits-2-and-3-swapped within 16-row groups, so the other operand is stored
// in that order by the transposed-tile pre-pass, or gathered in that order by
// transposing LDS reads):
//   * dK/dV: a workgroup owns 128 keys of one K/V head (32 per wave, K and V
//     fragments in registers as B operands); it streams the 64-query tiles of
//     both chunks that see those keys, for every query head reading that K/V
//     head (grouped-query attention; one for MHA), with direct global->LDS
//     loads.  Q and dO row-major feed S = Q K^T and dP = dO V^T; Q^T and dO^T
//     feed dV^T += dO^T P and dK^T += Q^T dS.  At head_dim 128 the transposed
//     operands are read from the same row-major tiles with gfx950's
//     transposing LDS read (ds_read_b64_tr_b16), so a stage holds two tiles
//     and the ring is four stages deep; at head_dim 64 the stage also holds
//     pre-transposed Q^T and dO^T tiles and the ring has two stages.  Lane =
//     key, so P and dS leave the score registers as B operands;
//   * dQ: a workgroup owns 256 queries of one chunk (32 per wave, Q and dO
//     fragments in registers); it streams the 64-key tiles (K and V row-major
//     for S^T = K Q^T and dP^T = V dO^T, K^T for dQ^T += K^T dS^T: at
//     head_dim 128 by transposing reads of the K tile, at 64 a pre-transposed
//     tile).
//     Lane = query, so the normaliser and delta are per-lane scalars.
//
// Built with the VGPR form of the MFMAs selected (-mllvm
// -amdgpu-mfma-vgpr-form, set for this file only by the build).
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int BW = 4;   // waves per workgroup of the dK/dV kernel
constexpr int QW = 8;   // waves per workgroup of the dQ kernel
constexpr int NST_DQ = 2;  // dQ ring depth with transposing reads (deeper rings spill registers)
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float PAD_LSE2 = 65536.0f;

// x as three bf16 parts (hi + mid + lo = x to about 2^-24 |x|), packed as the
// first three k values of an MFMA fragment.
__device__ __forceinline__ u32x4 bf16_split3(float x) {
  const float hi = __uint_as_float((uint32_t)f32_to_bf16(x) << 16);
  const float r1 = x - hi;
  const float mid = __uint_as_float((uint32_t)f32_to_bf16(r1) << 16);
  const float lo = r1 - mid;
  return u32x4{pack_bf16x2(hi, mid), pack_bf16x2(lo, 0.0f), 0u, 0u};
}

template <int HD, int NWAVES>
struct BCfg {
  static constexpr int NCH = HD / 8;                    // 16-byte chunks per row-major row
  static constexpr int TILE_BYTES = 64 * HD * 2;        // a 64-row tile, row-major or transposed
  static constexpr int TLOADS = TILE_BYTES / (NWAVES * 64 * 16);  // DMA instructions per thread per tile
  static constexpr int RPL = 64 / NCH;                  // row-major rows per 1 KB block
  static constexpr int KK = HD / 16;                    // MFMA k-steps over head_dim
  static constexpr int DT = HD / 32;                    // 32-wide d tiles
  static constexpr float INV_SQRT_HD = HD == 128 ? 0.08838834764831844055f : 0.125f;
};

// ---- stats: per (64-query tile, chunk, head); four waves of 16 rows, HD / 8
// lanes per row (16-byte loads along the row, so a wave reads whole 2 HD-byte
// row slices), the row's delta summed over those lanes with shuffles.
template <int HD>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const AttnBwdArgs a) {
  constexpr int LPR = HD / 8, RPP = 64 / LPR;  // lanes per row, rows per pass
  const int t = blockIdx.x, c = blockIdx.y, head = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  float* st = a.stats + ((c * (int64_t)a.n_heads + head) * a.tpc + t) * 256;
#pragma unroll
  for (int pass = 0; pass < 16 / RPP; ++pass) {
    const int r = wave * 16 + pass * RPP + lane / LPR;  // query row of the tile
    const int64_t row_in_chunk = (int64_t)t * 64 + r;
    const bool valid = row_in_chunk < a.chunk_len;
    float dl = 0.0f;
    if (valid) {
      const int64_t off = (c * a.chunk_len + row_in_chunk) * a.hidden + head * HD + 8 * sub;
      const u32x4 g = *reinterpret_cast<const u32x4*>(a.dout + off);
      const u32x4 o = *reinterpret_cast<const u32x4*>(a.o + off);
      u32x4 lo = u32x4{0u, 0u, 0u, 0u};
      if (a.o_lo) lo = *reinterpret_cast<const u32x4*>(a.o_lo + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float o0 = __uint_as_float(o[j] << 16) + __uint_as_float(lo[j] << 16);
        const float o1 = __uint_as_float(o[j] & 0xffff0000u) + __uint_as_float(lo[j] & 0xffff0000u);
        dl = fmaf(__uint_as_float(g[j] << 16), o0, dl);
        dl = fmaf(__uint_as_float(g[j] & 0xffff0000u), o1, dl);
      }
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) dl += __shfl_xor(dl, m);
    if (sub == 0) {
      // padding rows: a normaliser so large that every probability is
      // exp2(-2^16) = 0 (finite, so that it can be split into bf16 parts)
      const float l2 = valid ? a.lse[(int64_t)head * 2 * a.chunk_len + c * a.chunk_len + row_in_chunk] * LOG2E
                             : PAD_LSE2;
      st[r] = l2;
      st[64 + r] = dl;
      st[128 + r] = 0.0f;
      st[192 + r] = 0.0f;
    }
  }
}

// Transposing reads of a row-major 64-row tile of head_dim 128 (256-byte
// rows, 16-byte chunk c of row r at c ^ ((r & 3) << 2 | (r >> 2) & 3)) into
// the A fragment of the transposed tile for d tile dt and 16-row step ks.
// ds_read_b64_tr_b16: within each 16 lanes, output lane j takes element j % 4
// of the 8-byte pieces addressed by lanes j / 4, 4 + j / 4, 8 + j / 4 and
// 12 + j / 4.  Lane 32h + 16g + 4m + p addresses row 16 ks + 8 s + 4h + m,
// dims 32 dt + 16g + 4p .. +3, so output lane 32h + 16g + j holds dim
// 32 dt + 16g + j at rows 16 ks + 8 s + 4h + 0..3: reads s = 0, 1 give
// k = 8h + 0..7 in the order a 32x32 result's registers hold their rows.
// Byte offset within the tile: 4096 ks + 2048 s + (base ^ 64 dt ^ 32 s).
__device__ __forceinline__ uint32_t tr_read_base(int lane) {
  const int half = lane >> 5, m = (lane >> 2) & 3, p = lane & 3, g = (lane >> 4) & 1;
  return (uint32_t)(4 * half + m) * 256 + (uint32_t)(p & 1) * 8 + ((uint32_t)((2 * g + (p >> 1)) ^ (4 * m + half)) << 4);
}
__device__ __forceinline__ u32x4 tr_read_frag(const uint8_t* tile, uint32_t base, int dt, int ks) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const uint8_t* sb = tile + ks * 4096;
  const uint32_t o = base ^ (uint32_t)(dt << 6);
  const v4s ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(sb + o));
  const v4s rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(sb + 2048 + (o ^ 32u)));
  const u32x2 wa = __builtin_bit_cast(u32x2, ra), wb = __builtin_bit_cast(u32x2, rb);
  return u32x4{wa[0], wa[1], wb[0], wb[1]};
}

// ---- dK, dV.
template <int HD>
__global__ __launch_bounds__(64 * BW) void dkv_kernel(const AttnBwdArgs a) {
  using C = BCfg<HD, BW>;
  constexpr bool TR = !attn_bwd_stages_qt(HD);  // Q^T, dO^T by transposing reads of the row-major tiles
  constexpr int STATS = 1024;                    // per wave: its own copy of the tile's stats
  constexpr int STAGE = (TR ? 2 : 4) * C::TILE_BYTES + BW * STATS;
  constexpr int NST = TR ? 4 : 2;                // ring depth: 144 KB of LDS either way
  constexpr int PER_ISSUE = (TR ? 2 : 4) * C::TLOADS + 1;  // DMA instructions per thread per tile
  // The ring's stages are distinct arrays and every access names its stage
  // statically (the tile loops run NST tiles per iteration): the compiler
  // then knows that a transposing read of one stage does not alias the loads
  // filling another, and does not make it wait for every load in flight.
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[NST > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t stage3[NST > 3 ? STAGE : 16];
  static_assert(NST == 2 || NST == 4, "two or four stages");
  auto stage_of = [&](auto J) __attribute__((always_inline)) -> uint8_t* {
    constexpr int j = decltype(J)::value % NST;
    if constexpr (j == 0) return stage0;
    else if constexpr (j == 1) return stage1;
    else if constexpr (j == 2) return stage2;
    else return stage3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int ql = lane & 31;

  // work item: (K/V head, 128-key block), the earliest (most-seen) key blocks
  // of a head first, heads contiguous per XCD.  The block's dK, dV sum over the
  // query heads that read this K/V head (one for MHA).
  const int64_t S = a.seq_len, CL = a.chunk_len;
  const int nkb = (int)((S + 127) / 128);
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int kvh = pid / nkb;
  const int kblk = pid - kvh * nkb;
  const int group = a.n_heads / a.kv_heads;
  const int64_t kb0 = (int64_t)kblk * 128;
  const int64_t kw0 = kb0 + 32 * wave;  // this wave's first key
  const int64_t key = kw0 + ql;         // this lane's key
  const int kcol = kvh * HD;
  const int64_t ld = a.hidden, kld = a.kv_ld;

  // K and V fragments (B operands): lane holds key ql, dims 16*kk + 8*half .. +7.
  u32x4 kf[C::KK], vf[C::KK];
  {
    const int64_t kr = min(key, S - 1);  // keys past S: any finite row (masked: past every query)
    const uint16_t* kp = a.k + kr * kld + kcol + 8 * half;
    const uint16_t* vp = a.v + kr * kld + kcol + 8 * half;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      kf[kk] = *reinterpret_cast<const u32x4*>(kp + kk * 16);
      vf[kk] = *reinterpret_cast<const u32x4*>(vp + kk * 16);
    }
  }

  // Query tiles that see the block: chunk c's tiles from the one holding the
  // first query at or after kb0 to the chunk's end.
  const int tpc = (int)a.tpc;
  auto first_tile = [&](int64_t start) -> int {
    if (kb0 >= start + CL) return tpc;
    return (int)(max(kb0 - start, (int64_t)0) / 64);
  };
  const int f0 = first_tile(a.chunk_start0), f1 = first_tile(a.chunk_start1);
  const int n0 = tpc - f0, n_head = n0 + tpc - f1;  // tiles per query head
  const int n_all = n_head * group;
  // Of those, the first d0 (d1) of chunk 0 (1) hold a query before the
  // block's last key, so they need the causal mask; the rest do not.
  auto diag_tiles = [&](int64_t start, int f, int n) -> int {
    const int64_t span = kb0 + 127 - start;  // tiles t with start + 64 t < kb0 + 127
    const int64_t t_end = span > 0 ? (span + 63) / 64 : 0;
    return (int)min(max(t_end - f, (int64_t)0), (int64_t)n);
  };
  const int d0 = diag_tiles(a.chunk_start0, f0, n0), d1 = diag_tiles(a.chunk_start1, f1, tpc - f1);
  const int nd_head = d0 + d1, nr_head = n_head - nd_head;
  const int n_diag = nd_head * group;

  // DMA sources.  Row-major tiles: instruction j of wave w fills 1 KB block
  // b = j*BW + w, row b*RPL + lane/NCH, logical chunk (lane % NCH) ^ swizzle(row).
  // Transposed tiles: row d = b*8 + lane/8 (128 bytes), chunk (lane % 8) ^ ((d/2) % 8).
  // Row-major chunk swizzle.  With transposing reads (head_dim 128, 16 chunks
  // a row) the two 2-bit fields of the row's low nibble, swapped: 16
  // consecutive rows still cover all 16 chunk positions (row reads), and the
  // 4 rows x 4 chunks of a transposing read's 32 lanes do too.
  auto rm_swz = [](int r) -> int {
    if constexpr (TR) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return r & (C::NCH - 1);
  };
  // Byte offsets of this lane's loads relative to the tile's first row at the
  // head's first column (row-major) or to the transposed tile's start.
  uint32_t rm_off[C::TLOADS], tr_off[C::TLOADS];
#pragma unroll
  for (int j = 0; j < C::TLOADS; ++j) {
    const int b = j * BW + wave;
    const int r = b * C::RPL + lane / C::NCH;
    rm_off[j] = (uint32_t)((r * ld + ((lane % C::NCH) ^ rm_swz(r)) * 8) * 2);
    const int d = b * 8 + lane / 8;
    tr_off[j] = (uint32_t)((d * 64 + ((lane % 8) ^ ((d >> 1) & 7)) * 8) * 2);
  }

  // tile i: first the masked tiles (per query head: chunk 0's, chunk 1's),
  // then the others in the same order
  auto tile_of = [&](int i, int& c, int& t, int& qh) __attribute__((always_inline)) {
    int gi, j, m0, s0, s1;
    if (i < n_diag) {
      gi = i / nd_head;
      j = i - gi * nd_head;
      m0 = d0;
      s0 = f0;
      s1 = f1;
    } else {
      const int r = i - n_diag;
      gi = r / nr_head;
      j = r - gi * nr_head;
      m0 = n0 - d0;
      s0 = f0 + d0;
      s1 = f1 + d1;
    }
    qh = kvh * group + gi;
    if (j < m0) {
      c = 0;
      t = s0 + j;
    } else {
      c = 1;
      t = s1 + (j - m0);
    }
  };

  // Loads of tile i into stage J through buffer descriptors rebased per tile
  // (scalar work).  The Q/dO descriptors end at the chunk's last row, so the
  // padding rows of a chunk's last tile read as zeros (their normaliser makes
  // every probability 0 anyway).
  auto issue = [&](int i, auto J) __attribute__((always_inline)) {
    int c, t, qh;
    tile_of(i, c, t, qh);
    const int hcol = qh * HD;
    uint8_t* stage = stage_of(J);
    const int64_t row0 = c * CL + (int64_t)t * 64;
    const int64_t last = min((int64_t)63, CL - 1 - (int64_t)t * 64);  // the tile's last valid row
    const uint32_t bytes = (uint32_t)((last * ld + HD) * 2);
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(a.q + row0 * ld + hcol, bytes);
    const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(a.dout + row0 * ld + hcol, bytes);
#pragma unroll
    for (int j = 0; j < C::TLOADS; ++j) {
      dma16_buf(rq, rm_off[j], stage + (j * BW + wave) * 1024);
      dma16_buf(rd, rm_off[j], stage + C::TILE_BYTES + (j * BW + wave) * 1024);
    }
    if constexpr (!TR) {
      const int64_t tbase = ((c * (int64_t)a.n_heads + qh) * a.tpc + t) * (int64_t)(HD * 64);
      const __amdgpu_buffer_rsrc_t rqt = buffer_rsrc(a.qt + tbase, C::TILE_BYTES);
      const __amdgpu_buffer_rsrc_t rdt = buffer_rsrc(a.dot + tbase, C::TILE_BYTES);
#pragma unroll
      for (int j = 0; j < C::TLOADS; ++j) {
        dma16_buf(rqt, tr_off[j], stage + 2 * C::TILE_BYTES + (j * BW + wave) * 1024);
        dma16_buf(rdt, tr_off[j], stage + 3 * C::TILE_BYTES + (j * BW + wave) * 1024);
      }
    }
    const float* st = a.stats + ((c * (int64_t)a.n_heads + qh) * a.tpc + t) * 256;
    dma16_buf(buffer_rsrc(st, 1024), (uint32_t)lane * 16, stage + (TR ? 2 : 4) * C::TILE_BYTES + wave * STATS);
  };

  // fragment addresses within a stage (see the DMA swizzles above)
  const uint32_t rm_a0 = (uint32_t)ql * (HD * 2) + ((uint32_t)(half ^ rm_swz(ql)) << 4);
  const uint32_t tr_a0 = (uint32_t)ql * 128 + ((uint32_t)(half ^ ((ql >> 1) & 7)) << 4);
  // transposing reads: the queries come in the order the P and dS fragments hold them
  const uint32_t tr_b = TR ? tr_read_base(lane) : 0u;
  const float scale_log2 = LOG2E * C::INV_SQRT_HD;
  const float inv_scale_log2 = 1.0f / scale_log2;
  // B fragment of the normaliser/delta k-step: ones at k = 0..2 (half 0)
  const u32x4 ones = half ? u32x4{0u, 0u, 0u, 0u} : u32x4{0x3F803F80u, 0x00003F80u, 0u, 0u};

  f32x16 dkT[C::DT], dvT[C::DT];  // [d][key]: lane holds key ql, dims dt*32 + 8*(e/4) + 4*half + e%4
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    dkT[dt] = f32x16{};
    dvT[dt] = f32x16{};
  }

  // One tile as a software pipeline (one wave per SIMD: the wave itself has to
  // hide its LDS latency and its vector work): A fragments are read one MFMA
  // step ahead; the exponentials and dS of queries 0..31 run under the S/dP
  // MFMAs of queries 32..63, those of queries 32..63 under the first half of
  // the dV/dK MFMAs (which need only queries 0..31).
  auto compute = [&](int i, auto J, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    int c, t, qh;
    tile_of(i, c, t, qh);
    const int64_t qp0 = (c ? a.chunk_start1 : a.chunk_start0) + (int64_t)t * 64;  // position of query 0
    // (tiles whose queries all precede the wave's keys are computed too, the
    // mask zeroes them: a wave-uniform skip here splits the accumulators' live
    // ranges and costs register copies on every tile)
    // queries of the tile before this lane's key are masked (MASKED tiles
    // only): offsets below qmin
    const int qmin = kw0 + 31 > qp0 ? (int)min(max(key - qp0, (int64_t)0), (int64_t)64) : 0;
    const uint8_t* stage = stage_of(J);
    const uint8_t* q_st = stage;
    const uint8_t* do_st = stage + C::TILE_BYTES;
    const uint8_t* qt_st = TR ? q_st : stage + 2 * C::TILE_BYTES;
    const uint8_t* dot_st = TR ? do_st : stage + 3 * C::TILE_BYTES;
    const float* st = reinterpret_cast<const float*>(stage + (TR ? 2 : 4) * C::TILE_BYTES + wave * STATS);
    auto rm = [&](const uint8_t* base, int mb, int kk) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4*>(base + mb * 32 * (HD * 2) + (rm_a0 ^ (uint32_t)(kk << 5)));
    };
    auto tr = [&](const uint8_t* base, int dt, int ks) __attribute__((always_inline)) {
      if constexpr (TR) {
        return tr_read_frag(base, tr_b, dt, ks);
      } else {
        return *reinterpret_cast<const u32x4*>(base + dt * 32 * 128 + (tr_a0 ^ (uint32_t)(ks << 5)));
      }
    };
    uint32_t pp[16], ps[16];  // bf16 pairs of P and dS: [4*ks + j], 16-query step ks
    // The normaliser and delta enter the products as one extra k-step: A holds,
    // for the lane's query row (32*mb + ql), -l2/scale and -delta as three bf16
    // parts in k = 0..2 (lanes of half 0; half 1 and k >= 3 are zero), B holds
    // ones there, so the MFMAs give s - l2/scale and dP - delta directly.
    auto aug_s = [&](int mb) __attribute__((always_inline)) {
      return half ? u32x4{0u, 0u, 0u, 0u} : bf16_split3(-st[32 * mb + ql] * inv_scale_log2);
    };
    auto aug_d = [&](int mb) __attribute__((always_inline)) {
      return half ? u32x4{0u, 0u, 0u, 0u} : bf16_split3(-st[64 + 32 * mb + ql]);
    };
    // P and dS of entries 4g..4g+3 of half mb: queries 32*mb + 8*g + 4*half + j
    auto group = [&](const f32x16& sv, const f32x16& dpv, int mb, int g) __attribute__((always_inline)) {
      const int q0 = 32 * mb + 8 * g + 4 * half;
      float p[4], ds[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(sv[4 * g + j] * scale_log2);
        if constexpr (MASKED) p[j] = q0 + j < qmin ? 0.0f : p[j];
        ds[j] = p[j] * dpv[4 * g + j];
      }
      const int idx = 8 * mb + 2 * g;  // ks = 2*mb + g/2, pair 2*(g%2) + 0/1
      pp[idx] = pack_bf16x2(p[0], p[1]);
      pp[idx + 1] = pack_bf16x2(p[2], p[3]);
      ps[idx] = pack_bf16x2(ds[0], ds[1]);
      ps[idx + 1] = pack_bf16x2(ds[2], ds[3]);
    };
    constexpr int G2 = C::KK / 4;  // S/dP steps per group of vector work
    constexpr int G3 = C::DT / 2;  // dV/dK steps per group
    u32x4 qa = rm(q_st, 0, 0), da = rm(do_st, 0, 0);
    f32x16 s0 = mfma32(as_bf16x8(aug_s(0)), as_bf16x8(ones), f32x16{});
    f32x16 d0 = mfma32(as_bf16x8(aug_d(0)), as_bf16x8(ones), f32x16{});
    f32x16 s1 = mfma32(as_bf16x8(aug_s(1)), as_bf16x8(ones), f32x16{});
    f32x16 d1 = mfma32(as_bf16x8(aug_d(1)), as_bf16x8(ones), f32x16{});
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {  // S, dP of queries 0..31
      const int nm = kk + 1 < C::KK ? 0 : 1, nk = (kk + 1) % C::KK;
      const u32x4 qn = rm(q_st, nm, nk), dn = rm(do_st, nm, nk);
      s0 = mfma32(as_bf16x8(qa), as_bf16x8(kf[kk]), s0);
      d0 = mfma32(as_bf16x8(da), as_bf16x8(vf[kk]), d0);
      __builtin_amdgcn_sched_barrier(0);  // keep each step's reads ahead of its MFMAs
      qa = qn;
      da = dn;
    }
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {  // S, dP of queries 32..63; P, dS of queries 0..31
      u32x4 qn = qa, dn = da;
      if (kk + 1 < C::KK) {
        qn = rm(q_st, 1, kk + 1);
        dn = rm(do_st, 1, kk + 1);
      }
      s1 = mfma32(as_bf16x8(qa), as_bf16x8(kf[kk]), s1);
      d1 = mfma32(as_bf16x8(da), as_bf16x8(vf[kk]), d1);
      if ((kk + 1) % G2 == 0) group(s0, d0, 0, (kk + 1) / G2 - 1);
      __builtin_amdgcn_sched_barrier(0);
      qa = qn;
      da = dn;
    }
    u32x4 oa = tr(dot_st, 0, 0), ta = tr(qt_st, 0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {  // dV^T += dO^T P, dK^T += Q^T dS; P, dS of queries 32..63 under ks 0, 1
      const u32x4 bp = u32x4{pp[4 * ks], pp[4 * ks + 1], pp[4 * ks + 2], pp[4 * ks + 3]};
      const u32x4 bs = u32x4{ps[4 * ks], ps[4 * ks + 1], ps[4 * ks + 2], ps[4 * ks + 3]};
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        u32x4 on = oa, tn = ta;
        if (dt + 1 < C::DT) {
          on = tr(dot_st, dt + 1, ks);
          tn = tr(qt_st, dt + 1, ks);
        } else if (ks + 1 < 4) {
          on = tr(dot_st, 0, ks + 1);
          tn = tr(qt_st, 0, ks + 1);
        }
        dvT[dt] = mfma32(as_bf16x8(oa), as_bf16x8(bp), dvT[dt]);
        dkT[dt] = mfma32(as_bf16x8(ta), as_bf16x8(bs), dkT[dt]);
        const int step = ks * C::DT + dt;
        if (ks < 2 && (step + 1) % G3 == 0) group(s1, d1, 1, (step + 1) / G3 - 1);
        __builtin_amdgcn_sched_barrier(0);
        oa = on;
        ta = tn;
      }
    }
  };

  // NST-stage ring, one barrier per tile: the barrier after tile i's wait also
  // frees the stage that tile i-1 was computed from, so tile i+NST-1's loads go
  // there right after it, and land during the compute of tiles i..i+NST-2.
  // The wait leaves the loads of the tiles issued after tile i in flight.
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;
  if (n_all > 0) issue(0, J0{});
  if (NST > 2 && n_all > 1) issue(1, J1{});
  if (NST > 3 && n_all > 2) issue(2, J2{});
  // tile i in stage J = i mod NST
  auto step = [&](int i, auto J, auto masked) __attribute__((always_inline)) {
    const int ahead = min(NST - 2, n_all - 1 - i);  // tiles issued after tile i
    if (NST >= 4 && ahead >= 2)
      wait_vmcnt<2 * PER_ISSUE>();
    else if (NST >= 3 && ahead >= 1)
      wait_vmcnt<PER_ISSUE>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (i + NST - 1 < n_all) issue(i + NST - 1, std::integral_constant<int, decltype(J)::value + NST - 1>{});
    compute(i, J, masked);
  };
  // NST tiles per iteration, with the tail's tiles conditional
  auto steps = [&](int i, int end, auto masked) __attribute__((always_inline)) {
    step(i, J0{}, masked);
    if (i + 1 < end) step(i + 1, J1{}, masked);
    if constexpr (NST > 2) {
      if (i + 2 < end) step(i + 2, J2{}, masked);
      if (i + 3 < end) step(i + 3, J3{}, masked);
    }
  };
  // two loops, so that the unmasked one carries no mask code (a branch per
  // tile would split the accumulators' live ranges); the masked one runs a
  // whole number of NST-tile iterations (the mask is right on any tile), so
  // that the unmasked one starts at stage 0
  const int n_masked = min(n_all, (n_diag + NST - 1) / NST * NST);
  int i = 0;
  for (; i < n_masked; i += NST) steps(i, n_masked, std::true_type{});
  for (; i < n_all; i += NST) steps(i, n_all, std::false_type{});

  // store this lane's key row of dK (scaled) and dV; zeros where no query sees the key
  if (key < S) {
    float* dkp = a.dk + key * kld + kcol + 4 * half;
    float* dvp = a.dv + key * kld + kcol + 4 * half;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = dt * 32 + 8 * g;
        *reinterpret_cast<f32x4*>(dkp + d) =
            f32x4{dkT[dt][4 * g], dkT[dt][4 * g + 1], dkT[dt][4 * g + 2], dkT[dt][4 * g + 3]} * C::INV_SQRT_HD;
        *reinterpret_cast<f32x4*>(dvp + d) =
            f32x4{dvT[dt][4 * g], dvT[dt][4 * g + 1], dvT[dt][4 * g + 2], dvT[dt][4 * g + 3]};
      }
  }
}

// ---- dQ.
template <int HD>
__global__ __launch_bounds__(64 * QW) void dq_kernel(const AttnBwdArgs a) {
  using C = BCfg<HD, QW>;
  constexpr int QTB = 32 * QW;  // queries per workgroup
  constexpr bool TR = !attn_bwd_stages_kt(HD);  // K^T by transposing reads of the row-major K tile
  constexpr int STAGE = (TR ? 2 : 3) * C::TILE_BYTES;
  constexpr int NST = TR ? NST_DQ : 2;
  constexpr int PER_ISSUE = (TR ? 2 : 3) * C::TLOADS;  // DMA instructions per thread per tile
  // distinct stage arrays named statically, as in dkv_kernel
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[STAGE];
  static_assert(NST == 2, "two stages");
  auto stage_of = [&](auto J) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(J)::value % 2 == 0) return stage0;
    else return stage1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int ql = lane & 31;

  // work item: (head, chunk, 128-query tile), the latest (heaviest) tiles of a
  // head first, heads contiguous per XCD.
  const int64_t CL = a.chunk_len;
  const int tpcb = (int)((CL + QTB - 1) / QTB);
  const int per_head = 2 * tpcb;
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int head = pid / per_head;
  const int w = pid - head * per_head;
  const int chunk = w < tpcb ? 1 : 0;
  const int tile = w < tpcb ? tpcb - 1 - w : per_head - 1 - w;

  const int64_t row0 = chunk * CL + (int64_t)tile * QTB;  // local row of query 0
  const int64_t pos0 = (chunk ? a.chunk_start1 : a.chunk_start0) + (int64_t)tile * QTB;
  const int valid = (int)min((int64_t)QTB, CL - (int64_t)tile * QTB);
  const int64_t key_end = pos0 + valid;
  const int n_tiles = (int)((key_end + 63) / 64);

  const int qi = min(wave * 32 + ql, valid - 1);  // this lane's query (clamped in the ragged tail)
  const int64_t qpos = pos0 + qi;
  const int wave_first = wave * 32;
  const bool wave_active = wave_first < valid;
  const int64_t wave_max_pos = pos0 + min(wave_first + 31, valid - 1);
  const int wave_tiles = wave_active ? (int)(wave_max_pos / 64) + 1 : 0;

  const int hcol = head * HD;
  const int64_t ld = a.hidden, kld = a.kv_ld;
  const int kvh = head / (a.n_heads / a.kv_heads);  // this head's K/V head
  const int kcol = kvh * HD;

  // Q and dO fragments (B operands): lane holds query qi, dims 16*kk + 8*half .. +7.
  u32x4 qf[C::KK], df[C::KK];
  {
    const int64_t off = (row0 + qi) * ld + hcol + 8 * half;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      qf[kk] = *reinterpret_cast<const u32x4*>(a.q + off + kk * 16);
      df[kk] = *reinterpret_cast<const u32x4*>(a.dout + off + kk * 16);
    }
  }
  float l2q, dlq;
  {
    const int64_t rq = (int64_t)tile * QTB + qi;  // row within the chunk
    const float* st = a.stats + ((chunk * (int64_t)a.n_heads + head) * a.tpc + rq / 64) * 256 + rq % 64;
    l2q = st[0];
    dlq = st[64];
  }

  auto rm_swz = [](int r) -> int {  // as in dkv_kernel
    if constexpr (TR) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return r & (C::NCH - 1);
  };
  // byte offsets of this lane's loads (as in dkv_kernel)
  uint32_t rm_off[C::TLOADS], tr_off[C::TLOADS];
#pragma unroll
  for (int j = 0; j < C::TLOADS; ++j) {
    const int b = j * QW + wave;
    const int r = b * C::RPL + lane / C::NCH;
    rm_off[j] = (uint32_t)((r * kld + ((lane % C::NCH) ^ rm_swz(r)) * 8) * 2);
    const int d = b * 8 + lane / 8;
    tr_off[j] = (uint32_t)((d * 64 + ((lane % 8) ^ ((d >> 1) & 7)) * 8) * 2);
  }
  const uint16_t* kt_head = TR ? nullptr : a.kt + (int64_t)kvh * a.n_kv_tiles * HD * 64;

  // Loads of key tile t into stage J; the K/V descriptors end at the item's
  // last key, so rows past it read as zeros (they are masked).
  auto issue = [&](int t, auto J) __attribute__((always_inline)) {
    uint8_t* stage = stage_of(J);
    const int64_t k0 = (int64_t)t * 64;
    const int64_t last = min((int64_t)63, key_end - 1 - k0);
    const uint32_t bytes = (uint32_t)((last * kld + HD) * 2);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(a.k + k0 * kld + kcol, bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(a.v + k0 * kld + kcol, bytes);
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rt =
        buffer_rsrc(TR ? a.k : kt_head + (int64_t)t * HD * 64, C::TILE_BYTES);
#pragma unroll
    for (int j = 0; j < C::TLOADS; ++j) {
      dma16_buf(rk, rm_off[j], stage + (j * QW + wave) * 1024);
      dma16_buf(rv, rm_off[j], stage + C::TILE_BYTES + (j * QW + wave) * 1024);
      if constexpr (!TR) dma16_buf(rt, tr_off[j], stage + 2 * C::TILE_BYTES + (j * QW + wave) * 1024);
    }
  };

  const uint32_t rm_a0 = (uint32_t)ql * (HD * 2) + ((uint32_t)(half ^ rm_swz(ql)) << 4);
  const uint32_t tr_a0 = (uint32_t)ql * 128 + ((uint32_t)(half ^ ((ql >> 1) & 7)) << 4);
  const uint32_t tr_b = TR ? tr_read_base(lane) : 0u;  // transposing reads, as in dkv_kernel
  const float scale_log2 = LOG2E * C::INV_SQRT_HD;

  f32x16 dqT[C::DT];  // [d][query]: lane holds query ql, dims dt*32 + 8*(e/4) + 4*half + e%4
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) dqT[dt] = f32x16{};

  auto compute = [&](int t, auto J, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    if (t >= wave_tiles) return;  // wave-uniform
    const uint8_t* stage = stage_of(J);
    const int64_t k0 = (int64_t)t * 64;
    uint32_t ps[16];
    // dS of entries 4g..4g+3 of key block kb: keys k0 + 32 kb + 8 g + 4 half + 0..3
    auto group = [&](const f32x16& sv, const f32x16& dpv, int kb, int g) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 4 * g; e < 4 * g + 4; e += 2) {
        float p0 = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, -l2q));
        float p1 = __builtin_amdgcn_exp2f(fmaf(sv[e + 1], scale_log2, -l2q));
        if constexpr (MASKED) {
          const int64_t kx = k0 + 32 * kb + 8 * (e >> 2) + 4 * half + (e & 3);
          p0 = kx > qpos ? 0.0f : p0;
          p1 = kx + 1 > qpos ? 0.0f : p1;
        }
        ps[8 * kb + e / 2] = pack_bf16x2(p0 * (dpv[e] - dlq), p1 * (dpv[e + 1] - dlq));
      }
    };
    auto kv = [&](int kb, int kk, u32x4& ka, u32x4& va) __attribute__((always_inline)) {
      const uint32_t ad = kb * 32 * (HD * 2) + (rm_a0 ^ (uint32_t)(kk << 5));
      ka = *reinterpret_cast<const u32x4*>(stage + ad);
      va = *reinterpret_cast<const u32x4*>(stage + C::TILE_BYTES + ad);
    };
    auto kt = [&](int dt, int ks) __attribute__((always_inline)) {
      if constexpr (TR)
        return tr_read_frag(stage, tr_b, dt, ks);
      else
        return *reinterpret_cast<const u32x4*>(stage + 2 * C::TILE_BYTES + dt * 32 * 128 +
                                               (tr_a0 ^ (uint32_t)(ks << 5)));
    };
    // Software pipeline (as in dkv_kernel): fragments one MFMA step ahead; dS
    // of key block 0 under the S/dP MFMAs of block 1, dS of block 1 under the
    // dQ MFMAs of the first two 16-key steps (which need only block 0).
    constexpr int G2 = C::KK / 4, G3 = C::DT / 2;
    f32x16 s0 = f32x16{}, d0 = f32x16{}, s1 = f32x16{}, d1 = f32x16{};
    u32x4 ka, va;
    kv(0, 0, ka, va);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      u32x4 kn, vn;
      if (kk + 1 < C::KK)
        kv(0, kk + 1, kn, vn);
      else
        kv(1, 0, kn, vn);
      s0 = mfma32(as_bf16x8(ka), as_bf16x8(qf[kk]), s0);
      d0 = mfma32(as_bf16x8(va), as_bf16x8(df[kk]), d0);
      __builtin_amdgcn_sched_barrier(0);
      ka = kn;
      va = vn;
    }
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      u32x4 kn = ka, vn = va;
      if (kk + 1 < C::KK) kv(1, kk + 1, kn, vn);
      s1 = mfma32(as_bf16x8(ka), as_bf16x8(qf[kk]), s1);
      d1 = mfma32(as_bf16x8(va), as_bf16x8(df[kk]), d1);
      if ((kk + 1) % G2 == 0) group(s0, d0, 0, (kk + 1) / G2 - 1);
      __builtin_amdgcn_sched_barrier(0);
      ka = kn;
      va = vn;
    }
    u32x4 ta = kt(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 bs = u32x4{ps[4 * ks], ps[4 * ks + 1], ps[4 * ks + 2], ps[4 * ks + 3]};
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        u32x4 tn = ta;
        if (dt + 1 < C::DT)
          tn = kt(dt + 1, ks);
        else if (ks + 1 < 4)
          tn = kt(0, ks + 1);
        dqT[dt] = mfma32(as_bf16x8(ta), as_bf16x8(bs), dqT[dt]);
        const int stp = ks * C::DT + dt;
        if (ks < 2 && (stp + 1) % G3 == 0) group(s1, d1, 1, (stp + 1) / G3 - 1);
        __builtin_amdgcn_sched_barrier(0);
        ta = tn;
      }
    }
  };

  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  if (n_tiles > 0) issue(0, J0{});
  // tile t in stage t mod 2; two-stage ring, one barrier per tile, as in dkv_kernel
  auto step = [&](int t, auto J, auto masked) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    lds_barrier();
    if (t + 1 < n_tiles) issue(t + 1, std::integral_constant<int, decltype(J)::value + 1>{});
    compute(t, J, masked);
  };
  // key tiles wholly at or before the first query need no mask: a loop of
  // their own (an even number of tiles, so that both loops start at stage 0),
  // then the masked tail (as in dkv_kernel)
  const int t_m = (int)min((int64_t)n_tiles, (pos0 + 1) / 64) & ~1;
  int t = 0;
  for (; t < t_m; t += 2) {
    step(t, J0{}, std::false_type{});
    step(t + 1, J1{}, std::false_type{});
  }
  for (; t < n_tiles; t += 2) {
    step(t, J0{}, std::true_type{});
    if (t + 1 < n_tiles) step(t + 1, J1{}, std::true_type{});
  }

  if (wave_active && wave_first + ql < valid) {
    float* dqp = a.dq + (row0 + wave_first + ql) * ld + hcol + 4 * half;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(dqp + dt * 32 + 8 * g) =
            f32x4{dqT[dt][4 * g], dqT[dt][4 * g + 1], dqT[dt][4 * g + 2], dqT[dt][4 * g + 3]} * C::INV_SQRT_HD;
  }
}

}  // namespace

hipError_t launch_attention_backward(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.chunk_len <= 0) return hipSuccess;
  const int H = a.n_heads, HD = a.head_dim;
  hipError_t e;
  {
    const dim3 grid((unsigned)a.tpc, 2, (unsigned)H);
    if (HD == 128)
      hipLaunchKernelGGL(bwd_stats_kernel<128>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_stats_kernel<64>, grid, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (attn_bwd_stages_kt(HD) &&
      (e = launch_vt_tiles(a.k, a.seq_len, a.kv_ld, a.kv_heads, HD, a.kt, a.n_kv_tiles, stream)) != hipSuccess)
    return e;
  const size_t chunk_tiles = (size_t)H * a.tpc * HD * 64;
  for (int c = 0; c < 2 && attn_bwd_stages_qt(HD); ++c) {
    const int64_t off = c * a.chunk_len * a.hidden;
    if ((e = launch_vt_tiles(a.q + off, a.chunk_len, a.hidden, H, HD, a.qt + c * chunk_tiles, a.tpc, stream)) !=
        hipSuccess)
      return e;
    if ((e = launch_vt_tiles(a.dout + off, a.chunk_len, a.hidden, H, HD, a.dot + c * chunk_tiles, a.tpc,
                             stream)) != hipSuccess)
      return e;
  }
  {
    const dim3 grid((unsigned)(a.kv_heads * ((a.seq_len + 127) / 128)));
    if (HD == 128)
      hipLaunchKernelGGL(dkv_kernel<128>, grid, dim3(64 * BW), 0, stream, a);
    else
      hipLaunchKernelGGL(dkv_kernel<64>, grid, dim3(64 * BW), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    const dim3 grid((unsigned)(H * 2 * ((a.chunk_len + 32 * QW - 1) / (32 * QW))));
    if (HD == 128)
      hipLaunchKernelGGL(dq_kernel<128>, grid, dim3(64 * QW), 0, stream, a);
    else
      hipLaunchKernelGGL(dq_kernel<64>, grid, dim3(64 * QW), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tsp
