// quantize.hip -- block-128 FP8 quantize of a flat bf16 tensor on gfx950.
//
// Method ("FP8 Transmission Optimization for VLA Training", section "FP8
// Transmission Optimization and Bottlenecks", Transmission Efficiency
// bullet: FP8 e4m3/e5m2 wire format with blockwise scaling), per block of
// 128 elements:
//   amax = max |x|,  s = max(fl32(amax / FP8_MAX), 2^-126),
//   q_i  = satRNE(fl32(x_i / s)).
//
// Mapping.  A block of 128 bf16 is 256 contiguous bytes = 16 lanes x 16 B, so
// one wave-wide 16-byte load covers 4 blocks and every load instruction reads
// 1 KiB contiguous.  A wave's tile is U such loads (U * 4 blocks), all issued
// before any arithmetic; each wave takes T consecutive tiles and issues the
// next tile's loads before the current tile's arithmetic.  The block amax is
// an integer max over sign-cleared bf16 bits (packed u16 max inside the
// lane, then 4 DPP steps across the 16 lanes), so it needs no LDS; LDS only
// stages a workgroup's scales so that they leave in one contiguous store.
// The grid has one wave per T tiles (grid-stride only past the dispatch
// limit), placed XCD-aware (block_position), so the tiles in flight stay
// inside one window of the buffer; the last wave also handles the ragged
// tail (< one tile, possibly a partial block).  Loads and stores are
// non-temporal: every byte is touched once.  The kernel is bound by HBM
// bandwidth, not by its arithmetic.
//
// The quotient without a per-element divide.  Per block: s, sp = s * f and
// rp = RN(1 / sp), with f = 2^64 for blocks whose amax is below 2^-60 (else
// 1) so that every residual below stays a normal number; s and rp come from
// divide-free sequences equal to the IEEE divides (scale_from_amax,
// recip_rn).  Per element, with x' = x * f (exact):
//   q0 = RN(x' * rp);  e = RN(q0 * sp - x') (fma, exact);  q1 = RN(q0 - e * rp) (fma)
// This is Markstein's correction (markstein_quotient); q1 equals RN(x / s)
// for every bf16 x and fp32 s that can occur here (exhaustively checked on
// the host over all significand pairs, including signed zeros, and on the
// device over all pairs of fp32 significands).  q1 goes straight to the
// hardware packed FP8 conversion (round to nearest even): |q1| is at most
// one fp32 ulp above FP8_MAX, and on that whole range the conversion equals
// the saturating encode (quotient_bound in fp8q_device.h), so no clamp is
// needed.  A chunk whose wave holds only finite blocks with amax >= 2^-60
// skips the factor f and the non-finite selects (quant_chunk).
#include "fp8q_device.h"
#include "launch.h"

namespace fp8q {
namespace {

#ifndef FP8Q_QUANT_U
#define FP8Q_QUANT_U 2
#endif
#ifndef FP8Q_QUANT_T
#define FP8Q_QUANT_T 2
#endif
constexpr int kQuantU = FP8Q_QUANT_U;            // 1 KiB loads in flight per wave per tile
constexpr int kQuantT = FP8Q_QUANT_T;            // consecutive tiles per wave

struct BlockScale {
  float s;        // the stored scale (NaN for a non-finite block)
  float sp;       // s * f
  float rp;       // RN(1 / sp)
  float f;        // 2^64 for tiny blocks, else 1
  bool finite;
};

// NOT_TINY: the caller knows amax >= 2^-60, so f is the constant 1 and the
// multiplies by it fold away; FINITE: the caller knows the block is finite,
// so the selects on finite fold away too.
template <int FMT, bool NOT_TINY = false, bool FINITE = false>
__device__ __forceinline__ BlockScale block_scale(uint32_t amax_bits) {
  BlockScale b;
  b.finite = FINITE || amax_bits < 0x7F80u;
  const float s = scale_from_amax<FMT>(__uint_as_float(amax_bits << 16));  // = IEEE amax / M
  b.f = (!NOT_TINY && amax_bits < 0x2180u) ? 0x1p64f : 1.0f;  // amax < 2^-60
  b.sp = s * b.f;
  b.rp = recip_rn(b.sp);                           // = IEEE 1 / sp
  b.s = b.finite ? s : __uint_as_float(0x7FC00000u);
  return b;
}

// RN(x / s), converted by cvt4 with no clamp: |RN(x / s)| <= quotient_bound
// for every x of a finite block (see quotient_bound in fp8q_device.h).
template <int FMT>
__device__ __forceinline__ float quotient(float x, const BlockScale &b) {
  return markstein_quotient(x * b.f, b.sp, b.rp);
}

template <int FMT>
__device__ __forceinline__ u32x2 quant8(u32x4 v, const BlockScale &b) {
  u32x2 r;
  r.x = cvt4<FMT>(quotient<FMT>(bf16_lo(v.x), b), quotient<FMT>(bf16_hi(v.x), b),
                  quotient<FMT>(bf16_lo(v.y), b), quotient<FMT>(bf16_hi(v.y), b));
  r.y = cvt4<FMT>(quotient<FMT>(bf16_lo(v.z), b), quotient<FMT>(bf16_hi(v.z), b),
                  quotient<FMT>(bf16_lo(v.w), b), quotient<FMT>(bf16_hi(v.w), b));
  if (!b.finite) {
    r.x = 0x7F7F7F7Fu;
    r.y = 0x7F7F7F7Fu;
  }
  return r;
}

// One 16-byte chunk per lane (8 elements of the block its 16-lane row
// shares): the codes, and the block's stored scale in *s.  A chunk whose
// wave holds only finite blocks with amax >= 2^-60 (the usual case; one
// unsigned compare tests both) takes the path where f is the constant 1 and
// every block is finite, which saves a multiply per element and the
// selects for non-finite blocks; on MI355X
// (together with the clamp-free encode and the unzeroed conversion word,
// alternated in one run) the 64 MiB quantize went from 71.0% to 72.3% of
// 8 TB/s and 512 MiB from 84.4% to 84.7%.
template <int FMT>
__device__ __forceinline__ u32x2 quant_chunk(u32x4 v, float *s) {
  const uint32_t ab = max_row16(amax_bits8(v));
  if (!wave_any(ab - 0x2180u >= 0x7F80u - 0x2180u)) {
    const BlockScale b = block_scale<FMT, true, true>(ab);
    *s = b.s;
    return quant8<FMT>(v, b);
  }
  const BlockScale b = block_scale<FMT>(ab);
  *s = b.s;
  return quant8<FMT>(v, b);
}

// The ragged end [start, n): whole blocks plus at most one partial block.
// One wave, 4 blocks per pass (one per 16-lane row); elements past n read as
// zero (which never raises an amax) and are never written.
template <int FMT>
__device__ void quantize_tail(const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
                              float *__restrict__ scales, uint64_t n, uint64_t start) {
  const uint32_t lane = lane_id();
  const uint32_t row = lane >> 4, col = lane & 15;
  for (uint64_t blk0 = start / kBlock; blk0 * kBlock < n; blk0 += 4) {
    const uint64_t blk = blk0 + row;
    const uint64_t e0 = blk * kBlock + col * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (e0 + 8 <= n) {
      v = *reinterpret_cast<const u32x4 *>(x + e0);
    } else if (e0 < n) {
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (e0 + j < n) ? x[e0 + j] : 0u;
      v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                h[6] | (h[7] << 16)};
    }
    const BlockScale b = block_scale<FMT>(max_row16(amax_bits8(v)));
    const u32x2 r = quant8<FMT>(v, b);
    if (e0 + 8 <= n) {
      *reinterpret_cast<u32x2 *>(q + e0) = r;
    } else if (e0 < n) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (e0 + j < n) q[e0 + j] = (uint8_t)((j < 4 ? r.x : r.y) >> (8 * (j & 3)));
    }
    if (col == 0 && blk * kBlock < n) scales[blk] = b.s;
  }
}

// Workgroup shape by size.  Below FP8Q_QUANT_WIDE_N elements a workgroup is
// 4 waves and each XCD run is FP8Q_XCD_CHUNK (64) workgroups; from there up
// it is one wave, with XCD runs of FP8Q_QUANT_WIDE_XCD (256) workgroups, so
// an XCD run still covers 1 MiB of bf16.  One-wave workgroups never wait at
// the barrier before the scale flush for a slower wave.  On MI355X (e4m3,
// variants alternated in one run) they measured 83.9-84.1% of 8 TB/s on the
// 3.5e9-element gradient against 81.3-81.8% for 4 waves, 83.3-83.5% against
// 82.4-82.6% at 512 MiB and 81.2-81.4% against 80.6-80.7% at 256 MiB, but
// 68.6-69.5% against 70.2-70.4% at 64 MiB (there the 4x larger grid seems to
// cost more than the barrier waits it saves).  With the kernels' current
// arithmetic the two shapes tie at 80-96 MiB payloads, and one-wave
// workgroups are 0.5-0.8 points faster from 112 MiB to 224 MiB and 2.1
// points slower at 64 MiB, so the switch sits at a 96 MiB payload.
#ifndef FP8Q_QUANT_WIDE_N
#define FP8Q_QUANT_WIDE_N (3ull << 24)
#endif
#ifndef FP8Q_QUANT_WIDE_XCD
#define FP8Q_QUANT_WIDE_XCD 256
#endif
// Below FP8Q_QUANT_WIDE_N: workgroups of FP8Q_QUANT_MID_W waves in XCD runs
// of FP8Q_QUANT_MID_C.  Re-measured at 16-256 MiB with the kernels' current
// store waits and occupancy caps: 2-, 8- and 16-wave workgroups (XCD runs of
// the same bytes, capped and uncapped) were 1.5-4.5% slower than 4 at 64 MiB
// and no faster elsewhere.
#ifndef FP8Q_QUANT_MID_W
#define FP8Q_QUANT_MID_W 4
#endif
// Below FP8Q_QUANT_T1_BELOW_N elements (up to 7168 tiles of 512, a 7 MiB
// payload) a wave takes one tile of FP8Q_QUANT_SMALL_U loads, not T tiles
// of U: the grid has four times the waves and each wave's serial chain
// (loads, quotients, stores) is a quarter as long, which is what a small
// launch's time is made of.  On MI355X (graph replay, alternated in one run,
// e5m2, over 20 windows that the 256 MB Infinity Cache holds at these
// sizes), one tile of U = 2 took a 1 MiB payload from 3.05-3.12 us to
// 2.5-2.6 us; one tile of U = 1 then gained 10% at 767 KiB, 6% at 2 MiB,
// 20% at 3.9 MiB, 7.5% at 4 MiB and 9.7% at 6 MiB over it, and tied at
// 64 KiB.  With the data in HBM (windows totalling 768 MB per graph), it
// gained 2.4-3.9 points of 8 TB/s at 4-7 MiB and 1.3-2.5 at 0.75-2 MiB, and
// lost 3.2-4.4 points from 7.25 MiB up: 7168 one-tile waves are 28 per CU,
// the kernel's occupancy, so a larger launch needs a second round of waves.
#ifndef FP8Q_QUANT_T1_BELOW_N
#define FP8Q_QUANT_T1_BELOW_N (7168ull * 512 + 1)
#endif
#ifndef FP8Q_QUANT_SMALL_U
#define FP8Q_QUANT_SMALL_U 1
#endif
#ifndef FP8Q_QUANT_MID_C
#define FP8Q_QUANT_MID_C FP8Q_XCD_CHUNK
#endif

// One-wave workgroups wait for their code stores to be acknowledged before
// their scales leave (s_waitcnt vmcnt(0) at the top of each round's flush),
// which keeps each wave, and its slot, until its stores have landed, so
// fewer waves stream at once.  On MI355X (alternated in one run) the
// 3.5e9-element quantize took 1583-1589 us with the wait against 1601-1605
// us without it (1 GiB: 243-244 against 246-247 us; 256 MiB: 62.8-63.0
// against 63.4-63.6 us).  Waiting only at the end of the wave, after the
// scales, recovered none of it, and the 4-wave shape is the same either way
// (64 MiB: 18.1-18.2 us), so it does not wait.
#ifndef FP8Q_QUANT_FLUSH_WAIT_W1
#define FP8Q_QUANT_FLUSH_WAIT_W1 1
#endif
#ifndef FP8Q_QUANT_FLUSH_WAIT_W4
#define FP8Q_QUANT_FLUSH_WAIT_W4 0
#endif

// LDS each 4-wave workgroup reserves beyond its scale staging, so that at
// most 7 of them share a CU (160 KiB of LDS per CU: 7 x 21 KiB fits, 8 do
// not), 28 waves instead of 32.  At a 64 MiB payload (two rounds of resident
// waves) this measured 17.99-18.09 us against 18.10-18.32 us uncapped
// (alternated in one run on MI355X); a cap of 6 was no faster than none, and
// 16 and 256 MiB payloads were unchanged.
#ifndef FP8Q_QUANT_LDS_PAD_W4
#define FP8Q_QUANT_LDS_PAD_W4 21504
#endif

// The same for the one-wave workgroups of large payloads: 5.5 KiB each, so
// that about 28 share a CU instead of 32.  On MI355X (alternated in one run)
// the 3.5e9-element quantize took 1552-1557 us capped against 1590 us
// uncapped (85.3% against 83.4% of 8 TB/s), 1 GiB 240 against 244-249 us and
// 512 MiB 122 against 124 us; caps of 24 and 26 were within 0.5% of 28, 16
// was no faster than none, and without the store wait before the scale
// flush the capped kernel was 0.5% slower.
#ifndef FP8Q_QUANT_LDS_PAD_W1
#define FP8Q_QUANT_LDS_PAD_W1 5632
#endif

// One tile: quantize the U loaded chunks, store the codes, and put the
// tile's 4U scales at sc_dst[0 .. 4U) in the workgroup's LDS staging array.
template <int FMT, int U>
__device__ __forceinline__ void quantize_tile(const u32x4 (&v)[U], u32x2 *__restrict__ q,
                                              float *sc_dst, uint64_t t, uint32_t lane) {
  constexpr uint64_t kChunks = U * kWave;
  const uint32_t row = lane >> 4, col = lane & 15;
  const uint64_t c0 = t * kChunks;
  float sc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) st(q + c0 + u * kWave + lane, quant_chunk<FMT>(v[u], &sc[u]));
  // block (u, row) of the tile is block u * 4 + row; lane (row, col = u)
  // writes it, so one instruction covers the tile's 4U scales.
  if (col < U) {
    float s = sc[0];
#pragma unroll
    for (int u = 1; u < U; ++u) s = (col == (uint32_t)u) ? sc[u] : s;
    sc_dst[col * 4 + row] = s;
  }
}

// A wave's T consecutive tiles [t0, t0 + T) (those below full_tiles), the
// next tile's loads issued before the current tile's arithmetic; tile
// t0 + j puts its scales at sc_dst + 4U * j.
template <int FMT, int U, int T>
__device__ __forceinline__ void quantize_wave_tiles(const u32x4 *__restrict__ x,
                                                    u32x2 *__restrict__ q, float *sc_dst,
                                                    uint64_t t0, uint64_t full_tiles,
                                                    uint32_t lane) {
  constexpr uint64_t kChunks = U * kWave;          // 16-byte chunks per tile
  u32x4 cur[U];
#pragma unroll
  for (int u = 0; u < U; ++u) cur[u] = ld(x + t0 * kChunks + u * kWave + lane);
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const uint64_t t = t0 + j;
    if (t >= full_tiles) break;
    u32x4 nxt[U];
    const bool more = (j + 1 < T) && (t + 1 < full_tiles);
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) nxt[u] = ld(x + (t + 1) * kChunks + u * kWave + lane);
    }
    quantize_tile<FMT, U>(cur, q, sc_dst + 4 * U * j, t, lane);
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
  }
}

// Each wave takes T consecutive tiles.  The workgroup's WT tiles stage
// their 4UWT scales in LDS, and they leave in one contiguous store by the
// whole workgroup.  Storing each tile's 16U bytes from its own wave, as
// partial lines, measured 2-8% slower at 16 MiB - 1 GiB payloads (with
// 4-wave workgroups).  W waves per workgroup, XCD runs of C workgroups.

template <int FMT, int U, int T, int W, int C>
__global__ __launch_bounds__(64 * W) void quantize_kernel(const u32x4 *__restrict__ x,
                                                          u32x2 *__restrict__ q,
                                                          float *__restrict__ scales, uint64_t n,
                                                          uint64_t full_tiles) {
  constexpr uint64_t kChunks = U * kWave;          // 16-byte chunks per tile
  constexpr uint32_t kTileBlocks = 4 * U;
  __shared__ float wg_scales[W * T * kTileBlocks + (W != 1 ? FP8Q_QUANT_LDS_PAD_W4 / 4
                                                            : FP8Q_QUANT_LDS_PAD_W1 / 4)];
  const uint32_t lane = lane_id();
  workgroup_rounds<T, W, C>(
      full_tiles,
      [&](uint64_t t0, uint32_t wid) {
        quantize_wave_tiles<FMT, U, T>(x, q, wg_scales + wid * T * kTileBlocks, t0, full_tiles,
                                       lane);
      },
      [&](uint64_t base, uint32_t tiles) {
        if constexpr (W == 1 ? FP8Q_QUANT_FLUSH_WAIT_W1 != 0 : FP8Q_QUANT_FLUSH_WAIT_W4 != 0)
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        for (uint32_t i = threadIdx.x; i < tiles * kTileBlocks; i += 64 * W)
          scales[base * kTileBlocks + i] = wg_scales[i];
      });
  if (wave_index<W, C>() == wave_count<W>() - 1)
    quantize_tail<FMT>(reinterpret_cast<const uint16_t *>(x), reinterpret_cast<uint8_t *>(q),
                       scales, n, full_tiles * kChunks * 8);
}

// The last FP8Q_QUANT_TAIL_TILES tiles of a launch (at least; the split is
// rounded to an XCD run) go one per wave instead of two, so that the
// launch's final waves carry half the serial chain and the drain at its end
// is shorter.  On MI355X (graph replay over rotating windows, alternated in
// one run) a tail of 4096 tiles took the 64 MiB quantize from 72.5% to 74.5%
// of 8 TB/s, 48 MiB from 69.2% to 71.3% and 80-94 MiB up 1.4-1.5 points;
// with one-wave workgroups 96 and 192 MiB gained 0.8-0.9 points and 256 MiB
// to the 3.5e9-element gradient moved within 0.1%.  Tails of 1024-3072
// tiles gained nothing and 6144 less; with one-wave workgroups 8192 tied
// and 16384 lost up to 1.2 points.  Launches with fewer than twice the tail
// in tiles (below 16 MiB) keep a uniform shape: at 8 MiB an all-one-tile
// grid was 0.5 points slower.
#ifndef FP8Q_QUANT_TAIL_TILES
#define FP8Q_QUANT_TAIL_TILES 4096
#endif

// A launch with a one-tile tail: workgroups at positions below q2 take two
// tiles per wave (tiles [2W p, 2W p + 2W) for position p), the rest one tile
// per wave (from 2W q2 on).  q2 is a multiple of the XCD run C, and the XCD
// map (block_position) keeps positions within their dispatch round, so the
// one-tile workgroups come last in dispatch order up to one round.  The
// grid covers every tile in one pass (its launcher checks the dispatch
// cap); the scale flush and the ragged tail are as in quantize_kernel.
template <int FMT, int U, int W, int C>
__global__ __launch_bounds__(64 * W) void quantize_split_kernel(const u32x4 *__restrict__ x,
                                                                u32x2 *__restrict__ q,
                                                                float *__restrict__ scales,
                                                                uint64_t n, uint64_t full_tiles,
                                                                uint32_t q2) {
  constexpr uint64_t kChunks = U * kWave;
  constexpr uint32_t kTileBlocks = 4 * U;
  __shared__ float wg_scales[W * 2 * kTileBlocks + (W != 1 ? FP8Q_QUANT_LDS_PAD_W4 / 4
                                                            : FP8Q_QUANT_LDS_PAD_W1 / 4)];
  const uint32_t lane = lane_id();
  const uint32_t wid = uniform(threadIdx.x / kWave);
  const uint32_t pos = block_position<C>();
  uint64_t base;
  uint32_t wg_tiles;
  if (pos < q2) {
    base = (uint64_t)pos * W * 2;
    wg_tiles = W * 2;
    const uint64_t t0 = base + (uint64_t)wid * 2;
    if (t0 < full_tiles)
      quantize_wave_tiles<FMT, U, 2>(x, q, wg_scales + wid * 2 * kTileBlocks, t0, full_tiles,
                                     lane);
  } else {
    base = (uint64_t)q2 * W * 2 + (uint64_t)(pos - q2) * W;
    wg_tiles = W;
    const uint64_t t0 = base + wid;
    if (t0 < full_tiles)
      quantize_wave_tiles<FMT, U, 1>(x, q, wg_scales + wid * kTileBlocks, t0, full_tiles, lane);
  }
  __syncthreads();
  if constexpr (W == 1 && FP8Q_QUANT_FLUSH_WAIT_W1 != 0) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const uint64_t left = base < full_tiles ? full_tiles - base : 0;
  const uint32_t tiles = left < wg_tiles ? (uint32_t)left : wg_tiles;
  for (uint32_t i = threadIdx.x; i < tiles * kTileBlocks; i += 64 * W)
    scales[base * kTileBlocks + i] = wg_scales[i];
  if (wave_index<W, C>() == wave_count<W>() - 1)
    quantize_tail<FMT>(reinterpret_cast<const uint16_t *>(x), reinterpret_cast<uint8_t *>(q),
                       scales, n, full_tiles * kChunks * 8);
}

template <int FMT, int W, int C, int T = kQuantT>
void launch_shape(const void *x, uint64_t n, void *q, float *scales, uint64_t full,
                  hipStream_t stream) {
  constexpr int U = kQuantU;
  hipLaunchKernelGGL((quantize_kernel<FMT, U, T, W, C>),
                     dim3(grid_for_tiles((full + T - 1) / T, W)), dim3(64 * W), 0, stream,
                     static_cast<const u32x4 *>(x), static_cast<u32x2 *>(q), scales, n, full);
}

// A launch of the split kernel: the first q2 workgroups (a multiple of the
// XCD run C) take two tiles per wave, the rest one.  Returns false, launching
// nothing, when its grid would pass the dispatch cap (the caller then takes
// the grid-stride kernel).  Needs full >= FP8Q_QUANT_TAIL_TILES.
template <int FMT, int W, int C>
bool launch_split(const void *x, uint64_t n, void *q, float *scales, uint64_t full,
                  hipStream_t stream) {
  const uint64_t tail = FP8Q_QUANT_TAIL_TILES;
  const uint64_t q2 = (full - tail) / (2 * W) / C * C;
  const uint64_t wgs = q2 + (full - q2 * 2 * W + W - 1) / W;
  if (wgs > kMaxWorkgroups) return false;
  hipLaunchKernelGGL((quantize_split_kernel<FMT, kQuantU, W, C>), dim3((uint32_t)wgs),
                     dim3(64 * W), 0, stream, static_cast<const u32x4 *>(x),
                     static_cast<u32x2 *>(q), scales, n, full, (uint32_t)q2);
  return true;
}

template <int FMT>
hipError_t launch_t(const void *x, uint64_t n, void *q, float *scales, hipStream_t stream) {
  const uint64_t tile_elems = (uint64_t)kQuantU * kWave * 8;
  const uint64_t full = n / tile_elems;
  const bool split = FP8Q_QUANT_TAIL_TILES > 0 && full >= 2 * (uint64_t)FP8Q_QUANT_TAIL_TILES;
  if (n >= FP8Q_QUANT_WIDE_N) {
    if (!(split && launch_split<FMT, 1, FP8Q_QUANT_WIDE_XCD>(x, n, q, scales, full, stream)))
      launch_shape<FMT, 1, FP8Q_QUANT_WIDE_XCD>(x, n, q, scales, full, stream);
  } else if (n >= FP8Q_QUANT_T1_BELOW_N) {
    if (!(split &&
          launch_split<FMT, FP8Q_QUANT_MID_W, FP8Q_QUANT_MID_C>(x, n, q, scales, full, stream)))
      launch_shape<FMT, FP8Q_QUANT_MID_W, FP8Q_QUANT_MID_C>(x, n, q, scales, full, stream);
  } else {
    constexpr int SU = FP8Q_QUANT_SMALL_U, W = FP8Q_QUANT_MID_W;
    const uint64_t sfull = n / ((uint64_t)SU * kWave * 8);
    hipLaunchKernelGGL((quantize_kernel<FMT, SU, 1, W, FP8Q_QUANT_MID_C>),
                       dim3(grid_for_tiles(sfull, W)), dim3(64 * W), 0, stream,
                       static_cast<const u32x4 *>(x), static_cast<u32x2 *>(q), scales, n, sfull);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tensorwise quantize: one fp32 scale for the whole tensor (the tensorwise
// recipe of TorchAO's Float8Linear on "How to Speed Up VLA Training Step by
// Step: A 3x Acceleration Case Study on Pi0.5", FP8 section: amax, scale
// and cast per tensor), with the block rule above applied to one block that
// spans the tensor.  The global amax needs its own pass, so the bf16 input
// is read twice (5 B per element).  Four launches on the caller's stream:
//   1. tw_zero:     the caller's scale slot <- 0 (it holds amax bits first);
//   2. tw_amax:     grid-stride read-only pass, one atomic max per workgroup;
//   3. tw_quantize: the quantize mapping above with the scale from the slot;
//   4. tw_finalize: the slot <- the fp32 scale.
// Step 3 only reads the slot and step 4 writes it after every wave of step 3
// has finished (stream order), so no wave ever sees a half-written value.

__global__ __launch_bounds__(64) void tw_zero_kernel(uint32_t *slot) {
  if (threadIdx.x == 0) *slot = 0u;
}

#ifndef FP8Q_AMAX_U
#define FP8Q_AMAX_U 4
#endif
#ifndef FP8Q_AMAX_WGS
#define FP8Q_AMAX_WGS 512
#endif
constexpr int kAmaxU = FP8Q_AMAX_U;  // 16-byte loads in flight per thread

// Launched with 256-thread workgroups (kAmaxThreads); the size is a constant
// here rather than blockDim (see wave_index in fp8q_device.h).
constexpr uint32_t kAmaxThreads = 256;

__global__ __launch_bounds__(kAmaxThreads) void tw_amax_kernel(const u32x4 *__restrict__ x,
                                                               uint64_t n,
                                                               uint32_t *__restrict__ slot) {
  __shared__ uint32_t part[kAmaxThreads / kWave];
  const uint64_t nch = n / 8;
  const uint64_t stride = (uint64_t)gridDim.x * kAmaxThreads * kAmaxU;
  uint32_t m = 0;
  for (uint64_t c0 = (uint64_t)blockIdx.x * kAmaxThreads * kAmaxU + threadIdx.x; c0 < nch;
       c0 += stride) {
    u32x4 v[kAmaxU];
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) {
      const uint64_t c = c0 + (uint64_t)u * kAmaxThreads;
      v[u] = c < nch ? ld(x + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) {
      const uint32_t a = amax_bits8(v[u]);
      m = m > a ? m : a;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 8 * nch) {
    const uint32_t a = reinterpret_cast<const uint16_t *>(x)[8 * nch + threadIdx.x] & 0x7FFFu;
    m = m > a ? m : a;
  }
  m = max_wave(m);
  if (lane_id() == 0) part[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
    for (uint32_t i = 1; i < kAmaxThreads / kWave; ++i) r = r > part[i] ? r : part[i];
    atomicMax(slot, r);
  }
}

// The tensor's quantize with its one scale b (the scale is uniform, so
// the kernel picks the f = 1 copy of this loop for every tensor whose amax
// is at least 2^-60).
template <int FMT, int U>
__device__ __forceinline__ void tw_quantize_body(const u32x4 *__restrict__ x,
                                                 u32x2 *__restrict__ q, const BlockScale &b,
                                                 uint64_t n, uint64_t full_tiles, uint64_t w0,
                                                 uint64_t nw, uint32_t lane) {
  constexpr uint64_t kChunks = U * kWave;
  for (uint64_t t = w0; t < full_tiles; t += nw) {
    const uint64_t c0 = t * kChunks;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld(x + c0 + u * kWave + lane);
#pragma unroll
    for (int u = 0; u < U; ++u) st(q + c0 + u * kWave + lane, quant8<FMT>(v[u], b));
  }
  if (w0 == nw - 1) {
    const uint16_t *x16 = reinterpret_cast<const uint16_t *>(x);
    uint8_t *q8 = reinterpret_cast<uint8_t *>(q);
    for (uint64_t i = full_tiles * kChunks * 8 + lane; i < n; i += kWave) {
      const uint32_t c = cvt4<FMT>(quotient<FMT>(bf16_lo(x16[i]), b), 0.0f, 0.0f, 0.0f);
      q8[i] = b.finite ? (uint8_t)c : (uint8_t)0x7F;
    }
  }
}

template <int FMT, int U>
__global__ __launch_bounds__(256) void tw_quantize_kernel(const u32x4 *__restrict__ x,
                                                          u32x2 *__restrict__ q,
                                                          const uint32_t *__restrict__ slot,
                                                          uint64_t n, uint64_t full_tiles) {
  const uint32_t lane = lane_id();
  const uint64_t nw = wave_count<4>();
  const uint64_t w0 = wave_index<4>();
  const BlockScale b0 = block_scale<FMT>(*slot);
  if (b0.f != 1.0f) {
    tw_quantize_body<FMT, U>(x, q, b0, n, full_tiles, w0, nw, lane);
  } else {
    BlockScale b1 = b0;
    b1.f = 1.0f;                                     // a constant: x * f folds away
    tw_quantize_body<FMT, U>(x, q, b1, n, full_tiles, w0, nw, lane);
  }
}

template <int FMT>
__global__ __launch_bounds__(64) void tw_finalize_kernel(uint32_t *slot) {
  if (threadIdx.x == 0) *slot = __float_as_uint(block_scale<FMT>(*slot).s);
}

template <int FMT>
hipError_t launch_tw_t(const void *x, uint64_t n, void *q, float *scale, hipStream_t stream) {
  constexpr int U = kQuantU;
  uint32_t *slot = reinterpret_cast<uint32_t *>(scale);
  hipLaunchKernelGGL(tw_zero_kernel, dim3(1), dim3(64), 0, stream, slot);
  // the amax pass only reads: a bounded grid-stride grid, so the atomics
  // number FP8Q_AMAX_WGS at most.  On MI355X (7 GB of bf16) 512-1024
  // workgroups read at ~7.0 TB/s, 4.5% faster than 2048 and 15% faster
  // than 256.
  uint64_t wgs = (n / 8 + kAmaxThreads * kAmaxU - 1) / (kAmaxThreads * kAmaxU);
  if (wgs > FP8Q_AMAX_WGS) wgs = FP8Q_AMAX_WGS;
  if (wgs < 1) wgs = 1;
  hipLaunchKernelGGL(tw_amax_kernel, dim3((uint32_t)wgs), dim3(kAmaxThreads), 0, stream,
                     static_cast<const u32x4 *>(x), n, slot);
  const uint64_t full = n / ((uint64_t)U * kWave * 8);
  hipLaunchKernelGGL((tw_quantize_kernel<FMT, U>), dim3(grid_for_tiles(full)), dim3(256), 0, stream,
                     static_cast<const u32x4 *>(x), static_cast<u32x2 *>(q), slot, n, full);
  hipLaunchKernelGGL(tw_finalize_kernel<FMT>, dim3(1), dim3(64), 0, stream, slot);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_tensorwise(int fmt, const void *x, uint64_t n, void *q, float *scale,
                                      hipStream_t stream) {
  return fmt == 0 ? launch_tw_t<0>(x, n, q, scale, stream) : launch_tw_t<1>(x, n, q, scale, stream);
}

hipError_t launch_quantize(int fmt, const void *x, uint64_t n, void *q, float *scales,
                           hipStream_t stream) {
  return fmt == 0 ? launch_t<0>(x, n, q, scales, stream) : launch_t<1>(x, n, q, scales, stream);
}

}  // namespace fp8q
