// mx8_quantize.hip -- MXFP8 (E4M3 codes + E8M0 scale per 32 along K)
// weight quantize on gfx950.
//
// Method ("perf: Reduce MXFP8 refit weight-transfer overheads", sections
// "Summary" and "Safety", and the review's "Verified clean" list: trainer
// weights prequantized to E4M3 with an E8M0 scale per 32 elements, the
// zero-scale clamp, scales shaped [rows, K/32]; the scale rule is the OCP MX
// v1.0 one):
//   X = clamp(floor(log2 amax) - 8, -127, 127),  code = X + 127,
//   q_i = satRNE_e4m3(x_i * 2^-X).
// For a finite bf16 amax with exponent field e, floor(log2 amax) - 8 >= -127
// exactly when e >= 8, and every bf16 subnormal falls below that, so
//   code = max(e, 8) - 8
// with no logarithm at all; 2^-X = 2^(127 - code) is built from its bits.
// x * 2^-X is exact wherever the result can matter (below 2^-126 it encodes
// to zero either way); the clamp to +-448 then turns the hardware's RNE
// conversion into the saturating one for the values in (448, 512).
//
// Layout.  With K a multiple of 32 the [rows, K] tensor is a flat sequence
// of 32-element blocks and the [rows, K/32] scale array is that sequence's
// block order, so the kernel never needs rows or K.  A block is 64 bytes = a
// quad of lanes x 16 B; one wave-wide 16-byte load covers 16 blocks (1 KiB
// contiguous) and the block amax takes 2 DPP steps.  A tile is U loads (16U
// blocks); lane 4g + c writes the E8M0 byte of block (u = c, g), so one byte
// write per lane puts the tile's 16U scale bytes in order into the
// workgroup's LDS staging array, from which they leave in one contiguous
// store per workgroup.  Each wave takes T consecutive tiles, issuing the
// next tile's loads before the current tile's arithmetic; the grid has one
// wave per T tiles, placed XCD-aware, in 4-wave workgroups, or one-wave
// workgroups on large tensors (see FP8Q_MX8_WIDE_N).
#include "fp8q_device.h"
#include "launch.h"

namespace fp8q {
namespace {

#ifndef FP8Q_MX_U
#define FP8Q_MX_U 2
#endif
#ifndef FP8Q_MX_T
#define FP8Q_MX_T 2
#endif
constexpr int kMxU = FP8Q_MX_U;              // 1 KiB loads in flight per wave per tile (<= 4)
constexpr int kMxT = FP8Q_MX_T;              // consecutive tiles per wave (pipelined)
static_assert(kMxU >= 1 && kMxU <= 4, "one E8M0 byte per lane covers at most 4 loads");

struct MxScale {
  uint32_t code;   // E8M0 byte
  float mul;       // 2^-X
  bool finite;
};

__device__ __forceinline__ MxScale mx_scale(uint32_t amax_bits) {
  MxScale m;
  const uint32_t e = amax_bits >> 7;
  m.finite = amax_bits < 0x7F80u;
  const uint32_t code = e > 8u ? e - 8u : 0u;
  m.code = m.finite ? code : 0xFFu;
  m.mul = __uint_as_float((254u - code) << 23);      // 2^(127 - code)
  return m;
}

__device__ __forceinline__ float mx_q(float x, float mul) {
  return sat_clamp<0>(x * mul);
}

__device__ __forceinline__ u32x2 mx_quant8(u32x4 v, const MxScale &m) {
  u32x2 r;
  r.x = cvt4<0>(mx_q(bf16_lo(v.x), m.mul), mx_q(bf16_hi(v.x), m.mul), mx_q(bf16_lo(v.y), m.mul),
                mx_q(bf16_hi(v.y), m.mul));
  r.y = cvt4<0>(mx_q(bf16_lo(v.z), m.mul), mx_q(bf16_hi(v.z), m.mul), mx_q(bf16_lo(v.w), m.mul),
                mx_q(bf16_hi(v.w), m.mul));
  if (!m.finite) {
    r.x = 0x7F7F7F7Fu;
    r.y = 0x7F7F7F7Fu;
  }
  return r;
}

// Workgroup shape by size, as for the block quantize: from FP8Q_MX8_WIDE_N
// elements a workgroup is one wave (XCD runs of 256), it waits for its code
// stores before each round's E8M0 flush, and it asks for 5.5 KiB of dynamic
// LDS so that about 28 share a CU; below that, 4-wave workgroups in XCD runs
// of 64.  On the MoE layer's 201M-element tensors (MI355X, five alternated
// rounds) the one-wave shape took 92.1-93.1 us against 93.2-94.3 us (82.4%
// against 81.4% of 8 TB/s on average).
#ifndef FP8Q_MX8_WIDE_N
#define FP8Q_MX8_WIDE_N (1ull << 27)
#endif
#ifndef FP8Q_MX8_W1_LDS
#define FP8Q_MX8_W1_LDS 5632
#endif

// One tile: quantize, store the codes, and put the tile's 16U E8M0 bytes at
// e_dst[0 .. 16U) in the workgroup's LDS staging array.
template <int U>
__device__ __forceinline__ void mx_tile(const u32x4 (&v)[U], u32x2 *__restrict__ q,
                                       uint8_t *e_dst, uint64_t t, uint32_t lane) {
  constexpr uint64_t kChunks = U * kWave;          // 16-byte chunks per tile
  const uint32_t g = lane >> 2, c = lane & 3;
  const uint64_t c0 = t * kChunks;
  uint32_t codes[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const MxScale m = mx_scale(max_quad(amax_bits8(v[u])));
    st(q + c0 + u * kWave + lane, mx_quant8(v[u], m));
    codes[u] = m.code;
  }
  if (c < U) {
    uint32_t code = codes[0];
#pragma unroll
    for (int u = 1; u < U; ++u) code = (c == (uint32_t)u) ? codes[u] : code;
    e_dst[c * 16 + g] = (uint8_t)code;
  }
}

// A wave's T consecutive tiles [t0, t0 + T) (those below full_tiles), the
// next tile's loads issued before the current tile's arithmetic; tile
// t0 + j puts its scale bytes at e_dst + 16U * j.
template <int U, int T>
__device__ __forceinline__ void mx_wave_tiles(const u32x4 *__restrict__ w, u32x2 *__restrict__ q,
                                              uint8_t *e_dst, uint64_t t0, uint64_t full_tiles,
                                              uint32_t lane) {
  constexpr uint64_t kChunks = U * kWave;
  u32x4 cur[U];
#pragma unroll
  for (int u = 0; u < U; ++u) cur[u] = ld(w + t0 * kChunks + u * kWave + lane);
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const uint64_t t = t0 + j;
    if (t >= full_tiles) break;
    u32x4 nxt[U];
    const bool more = (j + 1 < T) && (t + 1 < full_tiles);
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) nxt[u] = ld(w + (t + 1) * kChunks + u * kWave + lane);
    }
    mx_tile<U>(cur, q, e_dst + 16 * U * j, t, lane);
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
  }
}

// Each wave takes T consecutive tiles.  The workgroup's 4T tiles stage
// their E8M0 bytes in LDS, and they leave in one contiguous store (whole
// 128-byte lines: 4-byte stores when the scale pointer allows, else bytes)
// rather than as 4T partial-line byte stores from different waves.
template <int U, int T, int W, int C>
__global__ __launch_bounds__(64 * W) void mx8_kernel(const u32x4 *__restrict__ w,
                                                     u32x2 *__restrict__ q,
                                                     uint8_t *__restrict__ e8m0, uint64_t nchunks,
                                                     uint64_t full_tiles) {
  constexpr uint64_t kChunks = U * kWave;          // 16-byte chunks per tile
  constexpr uint32_t kTileBytes = 16 * U;          // E8M0 bytes per tile
  constexpr uint32_t kWgTiles = W * T;
  const uint32_t lane = lane_id();
  const uint32_t c = lane & 3;
  const uint64_t nw = wave_count<W>();
  const uint64_t w0 = wave_index<W, C>();

  __shared__ uint32_t wg_e8m0[kWgTiles * kTileBytes / 4];
  uint8_t *stage = reinterpret_cast<uint8_t *>(wg_e8m0);
  const bool words = (reinterpret_cast<uintptr_t>(e8m0) & 3u) == 0;
  workgroup_rounds<T, W, C>(
      full_tiles,
      [&](uint64_t t0, uint32_t wid) {
        mx_wave_tiles<U, T>(w, q, stage + wid * T * kTileBytes, t0, full_tiles, lane);
      },
      [&](uint64_t base, uint32_t tiles) {
        if constexpr (W == 1) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        const uint32_t nb = tiles * kTileBytes;
        uint8_t *dst = e8m0 + base * kTileBytes;
        if (words) {
          for (uint32_t i = threadIdx.x; i < nb / 4; i += 64 * W)
            reinterpret_cast<uint32_t *>(dst)[i] = wg_e8m0[i];
        } else {
          for (uint32_t i = threadIdx.x; i < nb; i += 64 * W) dst[i] = stage[i];
        }
      });
  // Tail: whole blocks only (the element count is a multiple of 32, so every
  // quad of chunks is either entirely present or entirely absent).
  if (w0 == nw - 1) {
    for (uint64_t base = full_tiles * kChunks; base < nchunks; base += kWave) {
      const uint64_t chunk = base + lane;
      const bool valid = chunk < nchunks;
      const u32x4 v = valid ? w[chunk] : u32x4{0u, 0u, 0u, 0u};
      const MxScale m = mx_scale(max_quad(amax_bits8(v)));
      if (valid) {
        q[chunk] = mx_quant8(v, m);
        if (c == 0) e8m0[chunk / 4] = (uint8_t)m.code;
      }
    }
  }
}

// One pass with a one-tile tail, as quantize_split_kernel: workgroups at
// positions below q2 (a multiple of the XCD run C) take two tiles per wave,
// the rest one tile per wave, so the launch's last waves carry half the
// serial chain.  The E8M0 flush and the tail are as in mx8_kernel.
template <int U, int W, int C>
__global__ __launch_bounds__(64 * W) void mx8_split_kernel(const u32x4 *__restrict__ w,
                                                           u32x2 *__restrict__ q,
                                                           uint8_t *__restrict__ e8m0,
                                                           uint64_t nchunks, uint64_t full_tiles,
                                                           uint32_t q2) {
  constexpr uint64_t kChunks = U * kWave;
  constexpr uint32_t kTileBytes = 16 * U;
  const uint32_t lane = lane_id();
  const uint32_t c = lane & 3;
  const uint32_t wid = uniform(threadIdx.x / kWave);
  const uint32_t pos = block_position<C>();
  __shared__ uint32_t wg_e8m0[W * 2 * kTileBytes / 4];
  uint8_t *stage = reinterpret_cast<uint8_t *>(wg_e8m0);
  const bool words = (reinterpret_cast<uintptr_t>(e8m0) & 3u) == 0;
  uint64_t base;
  uint32_t wg_tiles;
  if (pos < q2) {
    base = (uint64_t)pos * W * 2;
    wg_tiles = W * 2;
    const uint64_t t0 = base + (uint64_t)wid * 2;
    if (t0 < full_tiles) mx_wave_tiles<U, 2>(w, q, stage + wid * 2 * kTileBytes, t0, full_tiles, lane);
  } else {
    base = (uint64_t)q2 * W * 2 + (uint64_t)(pos - q2) * W;
    wg_tiles = W;
    const uint64_t t0 = base + wid;
    if (t0 < full_tiles) mx_wave_tiles<U, 1>(w, q, stage + wid * kTileBytes, t0, full_tiles, lane);
  }
  __syncthreads();
  if constexpr (W == 1) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const uint64_t left = base < full_tiles ? full_tiles - base : 0;
  const uint32_t nb = (left < wg_tiles ? (uint32_t)left : wg_tiles) * kTileBytes;
  uint8_t *dst = e8m0 + base * kTileBytes;
  if (words) {
    for (uint32_t i = threadIdx.x; i < nb / 4; i += 64 * W)
      reinterpret_cast<uint32_t *>(dst)[i] = wg_e8m0[i];
  } else {
    for (uint32_t i = threadIdx.x; i < nb; i += 64 * W) dst[i] = stage[i];
  }
  if (wave_index<W, C>() == wave_count<W>() - 1) {
    for (uint64_t b = full_tiles * kChunks; b < nchunks; b += kWave) {
      const uint64_t chunk = b + lane;
      const bool valid = chunk < nchunks;
      const u32x4 v = valid ? w[chunk] : u32x4{0u, 0u, 0u, 0u};
      const MxScale m = mx_scale(max_quad(amax_bits8(v)));
      if (valid) {
        q[chunk] = mx_quant8(v, m);
        if (c == 0) e8m0[chunk / 4] = (uint8_t)m.code;
      }
    }
  }
}

// One-wave launches (from FP8Q_MX8_WIDE_N elements) end with their last
// FP8Q_MX8_TAIL_TILES tiles one per wave (mx8_split_kernel).  On MI355X
// (graph replay over rotating windows, alternated in one run) the MoE
// layer's 201M-element tensors went from 83.3-83.5% to 83.9-84.0% of
// 8 TB/s with 4096 tiles (2048 and 8192: 83.7-83.9%).  The 4-wave shape
// below that keeps mx8_kernel: there the same tails moved 32-128 MiB
// tensors by -1.8 to +1.7 points.
#ifndef FP8Q_MX8_TAIL_TILES
#define FP8Q_MX8_TAIL_TILES 4096
#endif

// Below FP8Q_MX8_T1_BELOW_N elements (an 8 MiB payload) each wave takes one
// tile of one load (FP8Q_MX8_SMALL_U), not two tiles of two, as the block
// quantize does: four times the waves, each with a quarter of the serial
// chain.  On MI355X (alternated in one run, % change) +15% at a 768 KiB
// payload, +10% at 2 MiB, +2.4% at 4 MiB, +1% at 7.9 MiB; the same shape up
// to 32 MiB lost 6-9% at 16-24 MiB.  Measured again with the data in HBM
// (windows totalling 768 MB per graph, three times the Infinity Cache, which
// holds the 20 windows of those runs at these sizes): +1.5 / +1.3 / +2.2 /
// +0.6 points of 8 TB/s at 2 / 4 / 6 / 7.9 MiB.
#ifndef FP8Q_MX8_T1_BELOW_N
#define FP8Q_MX8_T1_BELOW_N (1ull << 22)
#endif
#ifndef FP8Q_MX8_SMALL_U
#define FP8Q_MX8_SMALL_U 1
#endif

// The split launch when it applies (full >= 2 * tail, grid under the cap).
template <int U, int W, int C>
bool launch_mx8_split(const void *w, uint64_t nchunks, uint64_t full, void *q, void *e8m0,
                      uint32_t lds, hipStream_t stream) {
  const uint64_t tail = FP8Q_MX8_TAIL_TILES;
  if (tail == 0 || full < 2 * tail) return false;
  const uint64_t q2 = (full - tail) / (2 * W) / C * C;
  const uint64_t wgs = q2 + (full - q2 * 2 * W + W - 1) / W;
  if (wgs > kMaxWorkgroups) return false;
  hipLaunchKernelGGL((mx8_split_kernel<U, W, C>), dim3((uint32_t)wgs), dim3(64 * W), lds, stream,
                     static_cast<const u32x4 *>(w), static_cast<u32x2 *>(q),
                     static_cast<uint8_t *>(e8m0), nchunks, full, (uint32_t)q2);
  return true;
}

}  // namespace

hipError_t launch_mx8_quantize(const void *w, uint64_t n, void *q, void *e8m0,
                               hipStream_t stream) {
  constexpr int U = kMxU;
  constexpr int T = kMxT;
  const uint64_t nchunks = n / 8;
  const uint64_t full = nchunks / ((uint64_t)U * kWave);
  if (n >= FP8Q_MX8_WIDE_N) {
    if (!(T == 2 && launch_mx8_split<U, 1, 256>(w, nchunks, full, q, e8m0, FP8Q_MX8_W1_LDS, stream)))
      hipLaunchKernelGGL((mx8_kernel<U, T, 1, 256>), dim3(grid_for_tiles((full + T - 1) / T, 1)),
                         dim3(64), FP8Q_MX8_W1_LDS, stream, static_cast<const u32x4 *>(w),
                         static_cast<u32x2 *>(q), static_cast<uint8_t *>(e8m0), nchunks, full);
  } else if (n < FP8Q_MX8_T1_BELOW_N) {
    constexpr int SU = FP8Q_MX8_SMALL_U;
    const uint64_t sfull = nchunks / ((uint64_t)SU * kWave);
    hipLaunchKernelGGL((mx8_kernel<SU, 1, 4, FP8Q_XCD_CHUNK>), dim3(grid_for_tiles(sfull, 4)),
                       dim3(256), 0, stream, static_cast<const u32x4 *>(w),
                       static_cast<u32x2 *>(q), static_cast<uint8_t *>(e8m0), nchunks, sfull);
  } else {
    hipLaunchKernelGGL((mx8_kernel<U, T, 4, FP8Q_XCD_CHUNK>),
                       dim3(grid_for_tiles((full + T - 1) / T, 4)), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(w), static_cast<u32x2 *>(q),
                       static_cast<uint8_t *>(e8m0), nchunks, full);
  }
  return hipGetLastError();
}

}  // namespace fp8q
