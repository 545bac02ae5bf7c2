// dequant_reduce.hip -- fused FP8 dequantize-then-reduce of k peer shards on
// gfx950, and the plain fp32 summing kernel of the naive comparator.
//
// Method ("FP8 Transmission Optimization for VLA Training", section "FP8
// Transmission Optimization and Bottlenecks", Transmission Efficiency
// bullet: a fused kernel removes the HBM traffic of dequantizing every peer's
// chunk first and summing afterwards):
//   d_{p,i} = fl32(dec(q_p[i]) * s_p[i / 128]),
//   acc_i   = d_{0,i}, then acc_i = fl32(acc_i + d_{p,i}) for p = 1 .. k-1,
//   y_i     = acc_i (fp32) or RNE_bf16(acc_i).
// Every product and every sum is rounded on its own (the library is built
// with -ffp-contract=off), in the same order as the definition, so the
// result is bit-for-bit deterministic.  k == 1 is the dequantize.
//
// Mapping.  Element i of every peer sits at the same offset, so a wave reads
// each peer's codes with 4-byte loads: one instruction reads 256 contiguous
// bytes (4 codes per lane) and its output store writes 1 KiB (fp32) or 512 B
// (bf16) contiguous.  A wave's tile is U such groups (U * 256 elements =
// 2U blocks of 128); all k * U code loads are issued before any arithmetic,
// and each wave takes T consecutive tiles with the next tile's loads issued
// before the current tile's arithmetic.  Lanes 0-31 of a group share one
// block and lanes 32-63 the next, so a peer's 2U scales of a tile are
// wave-uniform and come in through the scalar cache (or, for the peer counts
// where scalar registers run short, through vector loads issued with the
// codes).  Codes are decoded by
// the hardware packed FP8->fp32 conversion.  The dequantized values live
// only in registers.  The file also holds the MXFP8 receiver, which shares
// this mapping, and the reduce -> requantize, which holds eight codes per
// lane so that a block is one 16-lane row.
#include "fp8q_device.h"
#include "launch.h"

namespace fp8q {
namespace {

#ifndef FP8Q_RED_U4
#define FP8Q_RED_U4 2        // tile depth for k <= 4
#endif
#ifndef FP8Q_RED_U8
#define FP8Q_RED_U8 2        // tile depth for 4 < k <= 8
#endif
#ifndef FP8Q_RED_U13
#define FP8Q_RED_U13 1       // tile depth for 8 < k <= 13
#endif
#ifndef FP8Q_RED_U16
#define FP8Q_RED_U16 2       // tile depth for 13 < k <= 16
#endif
#ifndef FP8Q_RED_T
#define FP8Q_RED_T 2         // consecutive tiles per wave (pipelined)
#endif
// The block-128 dequantize (k == 1) has its own knobs.  On MI355X (437.5M
// elements) U = 2, T = 2 beat U = 1, 2, 4 with T = 1, 2, 4 into fp32, while
// into bf16 U = 4, T = 2 was 11% faster than U = 2, T = 2 (and U = 4, T = 1
// 6% faster).  The MXFP8 receiver keeps U = 2, T = 2 for one shard (U = 4,
// T = 1 was 6% slower there).
#ifndef FP8Q_RED_U1
#define FP8Q_RED_U1 FP8Q_RED_U4   // dequantize into fp32: tile depth
#endif
#ifndef FP8Q_RED_T1
#define FP8Q_RED_T1 FP8Q_RED_T    // dequantize into fp32: tiles per wave
#endif
#ifndef FP8Q_RED_U1_BF16
#define FP8Q_RED_U1_BF16 4        // dequantize into bf16: tile depth
#endif
#ifndef FP8Q_RED_T1_BF16
#define FP8Q_RED_T1_BF16 2        // dequantize into bf16: tiles per wave
#endif

struct PeerPtrs {
  const uint32_t *q[kMaxPeers];
  const float *s[kMaxPeers];
};

struct PartPtrs {
  const float *p[kMaxPeers];
};

// Codes in flight per wave: k * U * 256 B.  The depth per peer count was
// chosen by measurement on MI355X (k-peer reduce of 218,750,000-element
// shards): past 8 peers the scalar registers run short (2k peer pointers,
// plus 2U scales per peer on the scalar path), and the best mix of tile
// depth and scale path changes with k; see the vector-scale switch below.
template <int K>
constexpr int peers_u() {
  return K <= 4 ? FP8Q_RED_U4
                : (K <= 8 ? FP8Q_RED_U8 : (K <= 13 ? FP8Q_RED_U13 : FP8Q_RED_U16));
}

#ifndef FP8Q_RED_U8_BF16
#define FP8Q_RED_U8_BF16 FP8Q_RED_U8   // tile depth for 4 < k <= 8 into bf16
#endif
template <int K, bool BF16 = false>
constexpr int reduce_u() {
  return K == 1 ? (BF16 ? FP8Q_RED_U1_BF16 : FP8Q_RED_U1)
                : ((BF16 && K > 4 && K <= 8) ? FP8Q_RED_U8_BF16 : peers_u<K>());
}

template <int K, bool BF16 = false>
constexpr int reduce_t() {
  return K == 1 ? (BF16 ? FP8Q_RED_T1_BF16 : FP8Q_RED_T1) : FP8Q_RED_T;
}

// XCD run length (block_position) of the block-128 dequantize: 16 measured
// 3-4% faster than 64 into fp32 (equal into bf16).  The k-peer reduce and
// the MXFP8 receiver keep the library default (16 was 6% slower for the
// MXFP8 dequantize into fp32).
#ifndef FP8Q_XCD_CHUNK_DEQ
#define FP8Q_XCD_CHUNK_DEQ 16
#endif
#ifndef FP8Q_XCD_CHUNK_RED
#define FP8Q_XCD_CHUNK_RED 16            // k-peer reduce into fp32: XCD run
#endif
#ifndef FP8Q_XCD_CHUNK_RED_BF16
#define FP8Q_XCD_CHUNK_RED_BF16 64       // k-peer reduce into bf16: XCD run
#endif
#ifndef FP8Q_RED_WAVES
#define FP8Q_RED_WAVES 4                 // k-peer reduce into fp32: waves per workgroup
#endif
#ifndef FP8Q_RED_WAVES_BF16
#define FP8Q_RED_WAVES_BF16 1            // k-peer reduce into bf16: waves per workgroup
#endif
#ifndef FP8Q_DEQ_WAVES
#define FP8Q_DEQ_WAVES 4                 // single-shard dequantize: waves per workgroup
#endif
template <int K, bool BF16 = false>
constexpr int reduce_waves() {
  return (BF16 && K > 1 && K <= 8) ? FP8Q_RED_WAVES_BF16
                                   : (K == 1 ? FP8Q_DEQ_WAVES : FP8Q_RED_WAVES);
}
template <int K, bool BF16 = false>
constexpr int reduce_xcd_chunk() {
  return K == 1 ? FP8Q_XCD_CHUNK_DEQ
                : ((BF16 && K <= 8) ? FP8Q_XCD_CHUNK_RED_BF16 : FP8Q_XCD_CHUNK_RED);
}

// Non-temporal code loads pay off when several peers stream in; the single
// shard of a dequantize measured faster with ordinary loads.
template <int K>
constexpr bool kNtCodes = (FP8Q_NT_LOAD != 0) && K > 1;

template <bool BF16>
__device__ __forceinline__ void store4(void *y, uint64_t elem, float a, float b, float c, float d) {
  if constexpr (BF16) {
    st(reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(y) + elem),
       u32x2{bf16_pack2(a, b), bf16_pack2(c, d)});
  } else {
    st(reinterpret_cast<f32x4 *>(static_cast<float *>(y) + elem), f32x4{a, b, c, d});
  }
}

template <bool BF16>
__device__ __forceinline__ void store1(void *y, uint64_t elem, float a) {
  if constexpr (BF16) {
    __bf16 h = (__bf16)a;
    static_cast<unsigned short *>(y)[elem] = __builtin_bit_cast(unsigned short, h);
  } else {
    static_cast<float *>(y)[elem] = a;
  }
}

template <int FMT>
__device__ __forceinline__ float dec1(uint32_t code) {
  return dec2<FMT, false>(code)[0];
}

// Elements [start, n): one wave, one element per lane per pass.
template <int FMT, int K, bool BF16>
__device__ void reduce_tail(const PeerPtrs &P, void *__restrict__ y, uint64_t n, uint64_t start) {
  for (uint64_t i = start + lane_id(); i < n; i += kWave) {
    const uint64_t blk = i / kBlock;
    const uint8_t *q0 = reinterpret_cast<const uint8_t *>(P.q[0]);
    float acc = dec1<FMT>(q0[i]) * P.s[0][blk];
#pragma unroll
    for (int p = 1; p < K; ++p) {
      const uint8_t *qp = reinterpret_cast<const uint8_t *>(P.q[p]);
      const float d = dec1<FMT>(qp[i]) * P.s[p][blk];
      acc = acc + d;
    }
    store1<BF16>(y, i, acc);
  }
}

// Scale path.  By default a peer's 2U scales of a tile are wave-uniform
// scalar loads.  In vector-scale mode they are vector loads issued together
// with the codes (each lane fetches its own block's scale; the 32 lanes of
// a block share one address), which frees scalar registers and starts the
// scale fetch a tile ahead.  Measured on MI355X (218,750,000-element
// shards, bf16 out): at U = 1, vector scales are 3-7% faster than the scalar
// path for 9 and 10 peers, even at 11 and slower at 12 and 13; for 14..16
// peers U = 2 on the scalar path is fastest (about 30% over U = 1, whose
// scalar registers spill).  The requantize loads its scales per lane too.
#ifndef FP8Q_RED_VSCALE_MIN
#define FP8Q_RED_VSCALE_MIN 9
#endif
#ifndef FP8Q_RED_VSCALE_MAX
#define FP8Q_RED_VSCALE_MAX 11
#endif
template <int K>
constexpr bool kRedVecScales = K >= FP8Q_RED_VSCALE_MIN && K <= FP8Q_RED_VSCALE_MAX;

// One tile's inputs in registers: codes, and (vector-scale mode VS) scales.
template <int K, int U, bool VS>
struct TileIn {
  uint32_t w[K][U];
  float s[VS ? K : 1][VS ? U : 1];
};

template <int K, int U, bool VS>
__device__ __forceinline__ void load_tile(const PeerPtrs &P, uint64_t t, uint32_t lane,
                                          TileIn<K, U, VS> &in) {
  const uint64_t dw0 = t * ((uint64_t)U * 64);     // first code dword of tile t
#pragma unroll
  for (int p = 0; p < K; ++p)
#pragma unroll
    for (int u = 0; u < U; ++u) in.w[p][u] = ld<uint32_t, kNtCodes<K>>(P.q[p] + dw0 + u * kWave + lane);
  if constexpr (VS) {
    const uint64_t b0 = t * (2u * U) + (lane >= 32 ? 1u : 0u);
#pragma unroll
    for (int p = 0; p < K; ++p)
#pragma unroll
      for (int u = 0; u < U; ++u) in.s[p][u] = ld<float, false>(P.s[p] + b0 + 2 * u);
  }
}

// The tile's k-peer sums: acc[u][j] is element 4 * lane + j of group u.
template <int FMT, int K, int U, bool VS>
__device__ __forceinline__ void sum_tile(const PeerPtrs &P, const TileIn<K, U, VS> &in, uint64_t t,
                                         uint32_t lane, float (&acc)[U][4]) {
  constexpr uint64_t kTileBlocks = 2 * U;
  const bool upper = lane >= 32;
#pragma unroll
  for (int p = 0; p < K; ++p) {
    const float *sp = P.s[p] + t * kTileBlocks;    // wave-uniform
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s;
      if constexpr (VS)
        s = in.s[p][u];
      else
        s = upper ? sp[2 * u + 1] : sp[2 * u];
      const f32x2 lo = dec2<FMT, false>(in.w[p][u]);
      const f32x2 hi = dec2<FMT, true>(in.w[p][u]);
      const float d0 = lo[0] * s, d1 = lo[1] * s, d2 = hi[0] * s, d3 = hi[1] * s;
      if (p == 0) {
        acc[u][0] = d0; acc[u][1] = d1; acc[u][2] = d2; acc[u][3] = d3;
      } else {
        acc[u][0] = acc[u][0] + d0; acc[u][1] = acc[u][1] + d1;
        acc[u][2] = acc[u][2] + d2; acc[u][3] = acc[u][3] + d3;
      }
    }
  }
}

template <int FMT, int K, int U, bool VS, bool BF16>
__device__ __forceinline__ void reduce_tile(const PeerPtrs &P, const TileIn<K, U, VS> &in,
                                            void *__restrict__ y, uint64_t t, uint32_t lane) {
  constexpr uint64_t kTile = (uint64_t)U * 256;    // elements per tile
  float acc[U][4];
  sum_tile<FMT, K, U, VS>(P, in, t, lane, acc);
#pragma unroll
  for (int u = 0; u < U; ++u)
    store4<BF16>(y, t * kTile + (uint64_t)u * 256 + 4 * lane, acc[u][0], acc[u][1], acc[u][2],
                 acc[u][3]);
}

// A wave's T consecutive tiles [t0, t0 + T) (those below full_tiles), the
// next tile's loads issued before the current tile's arithmetic.
template <int FMT, int K, int U, int T, bool BF16, bool VS>
__device__ __forceinline__ void reduce_wave_tiles(const PeerPtrs &P, void *__restrict__ y,
                                                  uint64_t t0, uint64_t full_tiles,
                                                  uint32_t lane) {
  TileIn<K, U, VS> cur;
  load_tile<K, U, VS>(P, t0, lane, cur);
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const uint64_t t = t0 + j;
    if (t >= full_tiles) break;
    TileIn<K, U, VS> nxt;
    const bool more = (j + 1 < T) && (t + 1 < full_tiles);
    if (more) load_tile<K, U, VS>(P, t + 1, lane, nxt);
    reduce_tile<FMT, K, U, VS, BF16>(P, cur, y, t, lane);
    if (more) cur = nxt;
  }
}

// Each wave takes T consecutive tiles per pass (grid-stride past the
// dispatch cap).
template <int FMT, int K, int U, int T, bool BF16, bool VS = kRedVecScales<K>>
__global__ __launch_bounds__((64 * reduce_waves<K, BF16>())) void reduce_kernel(
    PeerPtrs P, void *__restrict__ y, uint64_t n, uint64_t full_tiles) {
  constexpr int W = reduce_waves<K, BF16>();
  constexpr int C = reduce_xcd_chunk<K, BF16>();
  constexpr uint64_t kTile = (uint64_t)U * 256;
  const uint32_t lane = lane_id();
  const uint64_t nw = wave_count<W>();
  const uint64_t w0 = wave_index<W, C>();

  // (the loop of reduce_wave_tiles, written out: calling the helper here
  // changed the compiled loop, and this kernel's code is the measured one)
  for (uint64_t t0 = w0 * T; t0 < full_tiles; t0 += nw * T) {
    TileIn<K, U, VS> cur;
    load_tile<K, U, VS>(P, t0, lane, cur);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const uint64_t t = t0 + j;
      if (t >= full_tiles) break;
      TileIn<K, U, VS> nxt;
      const bool more = (j + 1 < T) && (t + 1 < full_tiles);
      if (more) load_tile<K, U, VS>(P, t + 1, lane, nxt);
      reduce_tile<FMT, K, U, VS, BF16>(P, cur, y, t, lane);
      if (more) cur = nxt;
    }
  }
  if (w0 == nw - 1) reduce_tail<FMT, K, BF16>(P, y, n, full_tiles * kTile);
}

// One pass with a one-tile tail: waves below q2w take two tiles (tiles
// [2w, 2w + 2) for wave w), the rest one (from 2 q2w on), so the launch's
// last waves carry half the serial chain.  q2w is a multiple of an XCD
// run's waves, so the one-tile waves come last in dispatch order up to one
// round.  The grid covers every tile (its launcher checks the dispatch cap).
template <int FMT, int K, int U, bool BF16, bool VS = kRedVecScales<K>>
__global__ __launch_bounds__((64 * reduce_waves<K, BF16>())) void reduce_split_kernel(
    PeerPtrs P, void *__restrict__ y, uint64_t n, uint64_t full_tiles, uint64_t q2w) {
  constexpr int W = reduce_waves<K, BF16>();
  constexpr int C = reduce_xcd_chunk<K, BF16>();
  constexpr uint64_t kTile = (uint64_t)U * 256;
  const uint32_t lane = lane_id();
  const uint64_t nw = wave_count<W>();
  const uint64_t w0 = wave_index<W, C>();
  if (w0 < q2w) {
    reduce_wave_tiles<FMT, K, U, 2, BF16, VS>(P, y, 2 * w0, full_tiles, lane);
  } else {
    const uint64_t t0 = 2 * q2w + (w0 - q2w);
    if (t0 < full_tiles) reduce_wave_tiles<FMT, K, U, 1, BF16, VS>(P, y, t0, full_tiles, lane);
  }
  if (w0 == nw - 1) reduce_tail<FMT, K, BF16>(P, y, n, full_tiles * kTile);
}

// The reduce into bf16 from FP8Q_RED8_MIN_K_BF16 peers up holds eight codes
// per lane (reduce8_kernel): U = 1 group of 512 elements per tile, T = 2
// tiles per wave, 4-wave workgroups, XCD runs of 16.  Each wave instruction
// reads 512 B of a peer's codes, so the loads per element halve, and the
// bf16 result leaves as one 16-byte store per lane (1 KiB per instruction).
// Measured on MI355X against reduce_kernel, alternated in one run (% of
// 8 TB/s at 437.5 MiB / 64 MiB per peer): k = 12 81.8 / 80.0 against
// 78.6 / 75.6; k = 16 80.0 / 80.0 against 76.7 / 71.6.  Up to 8 peers it
// was no faster (k = 8: 82.5 / 77.8 against 83.3 / 78.8), and into fp32,
// whose 32 bytes per lane leave as two stores at a 32-byte stride, it was
// 10-45% slower at every peer count, so those keep reduce_kernel.
#ifndef FP8Q_RED8_MIN_K_BF16
#define FP8Q_RED8_MIN_K_BF16 9
#endif
#ifndef FP8Q_RED8_U
#define FP8Q_RED8_U 1
#endif
#ifndef FP8Q_RED8_T
#define FP8Q_RED8_T 2
#endif
#ifndef FP8Q_RED8_W
#define FP8Q_RED8_W 4
#endif
#ifndef FP8Q_RED8_C
#define FP8Q_RED8_C 16
#endif
// Below FP8Q_RED8_T1_BELOW_N elements (a 32 MiB payload) each wave takes one
// tile, not two: on MI355X (alternated in one run, % of 8 TB/s, 9 / 12 / 16
// peers) 767 KiB 14.4 / 16.5 / 18.0 -> 17.9 / 21.1 / 27.3, 2 MiB 33.5 /
// 38.0 / 41.3 -> 35.9 / 42.1 / 50.6, 16 MiB 67.9 / 71.3 / 72.1 -> 71.4 /
// 73.7 / 76.4, 24 MiB 72.5 / 75.1 / 75.8 -> 76.3 / 77.8 / 79.8; tied at
// 32 MiB.
#ifndef FP8Q_RED8_T1_BELOW_N
#define FP8Q_RED8_T1_BELOW_N (1ull << 24)
#endif
// From FP8Q_RED8_MIN_K_LARGE peers into bf16 the eight-codes mapping also
// takes launches from FP8Q_RED8_LARGE_FROM_N (a 64 MiB payload) up to
// FP8Q_RED8_LARGE_BELOW_N (256 MiB), one tile per wave below
// FP8Q_RED8_T1_BELOW_N_LARGE, in place of the vector-scale, one-tile-tail
// and per-wave shapes.  On MI355X (alternated in one run, points of 8 TB/s
// at 64 / 96 / 128 / 200 MiB): 8 peers +2.2 / +1.8 / +0.4 / +1.2, 5-7
// peers +0.1 to +1.8, 2-4 peers +0.2 to +2.9; at 32-48 MiB within 0.3.  In
// the bench the full stress payload went from 79.7-80.0% to 81.7-81.8%; at
// 218.75M elements per peer it was 0.2-0.3 points lower, hence the upper
// bound.
#ifndef FP8Q_RED8_MIN_K_LARGE
#define FP8Q_RED8_MIN_K_LARGE 2
#endif
#ifndef FP8Q_RED8_LARGE_FROM_N
#define FP8Q_RED8_LARGE_FROM_N (1ull << 25)
#endif
#ifndef FP8Q_RED8_LARGE_BELOW_N
#define FP8Q_RED8_LARGE_BELOW_N (1ull << 27)
#endif
#ifndef FP8Q_RED8_T1_BELOW_N_LARGE
#define FP8Q_RED8_T1_BELOW_N_LARGE (1ull << 26)
#endif

// Below FP8Q_RED_T1_BELOW_N elements each wave takes one tile, not T: the
// grid has twice the waves and each wave's serial chain (loads, sums,
// stores) is half as long, which is what a small launch's time is made of.
// Measured on MI355X (k = 8, alternated in one run): into fp32 3.35 against
// 3.94 us at a 1 MiB payload and 6.2 against 6.5-6.7 us at 4 MiB; into bf16
// 3.06 against 3.58 us at 1 MiB.  From 24 MiB up one tile per wave was 1.5-
// 3.5% slower, and at 16 MiB the two were within the noise of the runs.
#ifndef FP8Q_RED_T1_BELOW_N
#define FP8Q_RED_T1_BELOW_N (1ull << 22)
#endif
// The tile depth of those one-tile waves from FP8Q_RED_SMALL_U_FROM_N
// elements (a 1 MiB payload) up.  Into fp32, and into bf16 from 5 peers, a
// tile of one group (U = 1, so twice the waves again) was faster on MI355X
// (alternated in one run, % change at 767 KiB / 1 / 2 / 4 / 7.9 MiB
// payloads): 8 peers into fp32 +1.6 / +7.0 / +2.2 / +0.3 / +8.3, one shard
// into fp32 -1.9 / +3.7 / +8.9 / +18.0 / +22.2, 2-7 peers into fp32 -5.5 to
// +15.0 (gains from 2 MiB, up to 2.2% lost at 767 KiB), 5-8 peers into bf16
// -2.8 to +12.3; 14 and 16 peers into fp32 (whose deeper tile is U = 2)
// +96 / +67 / +39 / +60% and +101 / +51 / +30 / +53% at 1 / 2 / 4 /
// 7.9 MiB.  Into bf16 with 1-4 peers it lost up to 18.6% (2 peers), so
// those, and every launch below 1 MiB, keep the deeper tile.  The one-shard
// figures come from windows that the 256 MB Infinity Cache holds; with the
// data in HBM (768 MB of windows per graph) one shard into fp32 measured
// +3.9 / +4.5 / +3.8 / +3.1 points of 8 TB/s at 2 / 4 / 6 / 7.9 MiB against
// two-tile waves of the wider tile.
#ifndef FP8Q_RED_SMALL_U
#define FP8Q_RED_SMALL_U 1
#endif
#ifndef FP8Q_RED_SMALL_U_FROM_N
#define FP8Q_RED_SMALL_U_FROM_N (1ull << 19)
#endif
// Into fp32 the same one-group, one-tile waves also won at mid sizes: from
// FP8Q_RED_F32_ONE_FROM_N elements (a 32 MiB payload; FP8Q_RED_F32_ONE_FROM_N_K9
// from 9 peers) up to FP8Q_RED_F32_ONE_BELOW_N (256 MiB), against the
// vector-scale, one-tile-tail and two-tile shapes there.  On MI355X
// (alternated in one run, points of 8 TB/s): 8 peers +0.7 / +2.0 / +2.7 /
// +1.4 at 32 / 48 / 96 / 192 MiB, 2 peers +2.8 to +3.0 from 32 MiB, 3 and
// 5-7 peers +0.1 to +2.4, 9-16 peers +0.3 to +11.8 from 8 MiB; 4 peers lost
// up to 1.9, so they keep their shapes.  At 437.5M elements per peer the
// two-tile shape won again (82.5% against 81.1% at 8 peers), hence the
// upper bound.
#ifndef FP8Q_RED_F32_ONE_FROM_N
#define FP8Q_RED_F32_ONE_FROM_N (1ull << 24)
#endif
#ifndef FP8Q_RED_F32_ONE_FROM_N_K9
#define FP8Q_RED_F32_ONE_FROM_N_K9 (1ull << 22)
#endif
#ifndef FP8Q_RED_F32_ONE_BELOW_N
#define FP8Q_RED_F32_ONE_BELOW_N (1ull << 27)
#endif
template <int K, bool BF16>
constexpr int reduce_small_u() {
  return (!BF16 || K >= 5) ? FP8Q_RED_SMALL_U : reduce_u<K, BF16>();
}

// From 2 to 8 peers, launches of FP8Q_RED_T1_BELOW_N up to (not including)
// FP8Q_RED_VS_BELOW_N elements take the vector scales (each lane loads its
// block's scale with the codes) instead of the per-wave scale loads, which
// the compiler issues as vector loads after the next tile's codes: since
// loads complete in order, a tile's sums then wait for the next tile's codes
// too.  Issued with the codes, the scales cost registers (3 waves per SIMD
// instead of 4 at 8 peers) but no longer hold a tile back; that shortens a
// launch's fixed cost, which is what a mid-size launch is made of.  Measured
// on MI355X (alternated in one run; graph replay over rotating windows), the
// intercept of time against bytes fell from 3.3 to 2.8 us at 8 peers (bf16
// out) and from 3.3 to 2.6 us (fp32 out), 2.6-2.8 to 1.7-2.1 us at 2 and 4
// peers; 16 MiB payloads ran 4.4-4.5% faster at 8 peers, 64 MiB 0.3-1.9%
// faster (k = 2..8), 128 MiB the same, and 224 MiB 0.5-1% slower, so larger
// launches keep the per-wave loads.
#ifndef FP8Q_RED_VS_BELOW_N
#define FP8Q_RED_VS_BELOW_N (1ull << 26)
#endif
// With the vector scales, from FP8Q_RED_TAIL_MIN_K peers, the last
// FP8Q_RED_TAIL_TILES tiles of a launch go one per wave instead of two
// (reduce_split_kernel), as in the block quantize: the launch's final waves
// carry half the serial chain, so its drain is shorter.  On MI355X (graph
// replay over rotating windows, alternated in one run, % of 8 TB/s), with
// 4096 tiles: 8 peers into bf16 67.0 -> 70.7 at 16 MiB, 74.1 -> 76.9 at
// 32 MiB, 79.4 -> 80.4 at 64 MiB; into fp32 68.9 -> 72.1 at 16 MiB and
// 79.8 -> 80.4 at 64 MiB; 4 and 6 peers up 2.2-4.5 points at 16 MiB and
// -0.3 to +1.3 at 64 MiB.  Tails of 8192 and 16384 tiles gained less.
// With fewer peers (2, 3) or on the per-wave scale path (from 2^26
// elements, 128 MiB: 0.5-2 points slower) it did not pay, nor for the
// single-shard dequantize.
#ifndef FP8Q_RED_TAIL_TILES
#define FP8Q_RED_TAIL_TILES 4096
#endif
#ifndef FP8Q_RED_TAIL_MIN_K
#define FP8Q_RED_TAIL_MIN_K 4
#endif

// Dynamic LDS the single-shard dequantize into bf16 (below FP8Q_DEQ8_FROM_N
// elements, where it still takes reduce_kernel) reserves per workgroup
// (the kernel uses none), so that at most 6 of its 4-wave workgroups share a
// CU: 437.5M elements took 206.5-207.8 us capped against 212.7-213.9 us
// uncapped (80.0% against 77.7% of 8 TB/s, alternated in one run on
// MI355X); into fp32 the cap moved it within noise, so that keeps none.
#ifndef FP8Q_DEQ_BF16_LDS
#define FP8Q_DEQ_BF16_LDS 24576
#endif
// The single-shard dequantize into bf16 from FP8Q_DEQ8_FROM_N elements up,
// except from FP8Q_DEQ8_GAP_FROM_N up to (not including)
// FP8Q_DEQ8_GAP_BELOW_N, takes the eight-codes mapping of reduce8_kernel
// (one 8-byte code load and one 16-byte bf16 store per lane) with one
// 512-element tile per wave (launch_deq8_t), in place of the four-codes
// kernel above.  On MI355X (graph replay, alternated in one run, % of
// 8 TB/s, with the data in HBM: windows totalling 768 MB or more per graph,
// three times the Infinity Cache): 1 / 2 / 4 / 6 / 7.9 MiB payloads +1.1 /
// +2.3 / +3.5 / +2.7 / +4.2 points; 22 / 24 / 32 / 48 MiB +3.5 / +5.3 /
// +5.3 / +3.8; 64 / 128 / 224 MiB +5.3 / +3.4 / +2.1; 218.75M elements
// (417 MiB) +0.5; at 0.75 MiB even.  From 8 MiB to 20 MiB it lost 1.8-8.0
// points (18 MiB: 60.7 against 52.7), which is the gap.  Into fp32 the same
// mapping lost 4-21 points at every size (its two 16-byte stores per lane
// leave each store instruction strided), so fp32 keeps its shape.
#ifndef FP8Q_DEQ8_FROM_N
#define FP8Q_DEQ8_FROM_N (1ull << 19)
#endif
#ifndef FP8Q_DEQ8_GAP_FROM_N
#define FP8Q_DEQ8_GAP_FROM_N (1ull << 22)
#endif
#ifndef FP8Q_DEQ8_GAP_BELOW_N
#define FP8Q_DEQ8_GAP_BELOW_N (11ull << 20)
#endif

template <int FMT, int K, bool BF16>
hipError_t launch_reduce8_t(const PeerPtrs &P, uint64_t n, void *y, hipStream_t stream);
template <int FMT, bool BF16>
hipError_t launch_deq8_t(const PeerPtrs &P, uint64_t n, void *y, hipStream_t stream);

template <int FMT, int K, bool BF16>
hipError_t launch_reduce_t(const PeerPtrs &P, uint64_t n, void *y, hipStream_t stream) {
  if constexpr (BF16 && K >= FP8Q_RED8_MIN_K_BF16) {
    return launch_reduce8_t<FMT, K, BF16>(P, n, y, stream);
  } else {
    if constexpr (K == 1 && BF16) {
      // the single-shard dequantize into bf16 from FP8Q_DEQ8_FROM_N elements
      if (n >= FP8Q_DEQ8_FROM_N && (n < FP8Q_DEQ8_GAP_FROM_N || n >= FP8Q_DEQ8_GAP_BELOW_N))
        return launch_deq8_t<FMT, BF16>(P, n, y, stream);
    }
    if constexpr (BF16 && K >= FP8Q_RED8_MIN_K_LARGE) {
      // into bf16, FP8Q_RED8_LARGE_FROM_N <= n < FP8Q_RED8_LARGE_BELOW_N
      if (n >= FP8Q_RED8_LARGE_FROM_N && n < FP8Q_RED8_LARGE_BELOW_N)
        return launch_reduce8_t<FMT, K, BF16>(P, n, y, stream);
    }
    constexpr int U = reduce_u<K, BF16>();
    constexpr int T = reduce_t<K, BF16>();
    const uint64_t tile = (uint64_t)U * 256;
    const uint64_t full = n / tile;
    constexpr int W = reduce_waves<K, BF16>();
    constexpr uint32_t lds = (K == 1 && BF16) ? FP8Q_DEQ_BF16_LDS : 0;
    const dim3 grid(grid_for_tiles((full + T - 1) / T, W));
    if constexpr (!BF16 && K >= 2 && K != 4) {
      // fp32 mid sizes: one-group tiles, one per wave (FP8Q_RED_F32_ONE_*)
      constexpr uint64_t kFrom = K >= 9 ? (uint64_t)FP8Q_RED_F32_ONE_FROM_N_K9
                                        : (uint64_t)FP8Q_RED_F32_ONE_FROM_N;
      if (n >= kFrom && n < FP8Q_RED_F32_ONE_BELOW_N) {
        const uint64_t sfull = n / 256;
        hipLaunchKernelGGL((reduce_kernel<FMT, K, 1, 1, BF16>), dim3(grid_for_tiles(sfull, W)),
                           dim3(64 * W), lds, stream, P, y, n, sfull);
        return hipGetLastError();
      }
    }
    if (n < FP8Q_RED_T1_BELOW_N) {
      constexpr int SU = reduce_small_u<K, BF16>();
      if constexpr (SU != U) {
        if (n >= FP8Q_RED_SMALL_U_FROM_N) {
          const uint64_t sfull = n / ((uint64_t)SU * 256);
          hipLaunchKernelGGL((reduce_kernel<FMT, K, SU, 1, BF16>),
                             dim3(grid_for_tiles(sfull, W)), dim3(64 * W), lds, stream, P, y, n,
                             sfull);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((reduce_kernel<FMT, K, U, 1, BF16>), dim3(grid_for_tiles(full, W)),
                         dim3(64 * W), lds, stream, P, y, n, full);
      return hipGetLastError();
    }
    if constexpr (K >= 2 && K <= 8) {
      if (n < FP8Q_RED_VS_BELOW_N) {
        if constexpr (K >= FP8Q_RED_TAIL_MIN_K && T == 2) {
          // the last FP8Q_RED_TAIL_TILES tiles one per wave (reduce_split_kernel)
          constexpr uint64_t kTail = FP8Q_RED_TAIL_TILES;
          constexpr uint64_t kRunWaves = (uint64_t)W * reduce_xcd_chunk<K, BF16>();
          if (kTail > 0 && full >= 2 * kTail) {
            const uint64_t q2w = (full - kTail) / 2 / kRunWaves * kRunWaves;
            const uint64_t wgs = (q2w + (full - 2 * q2w) + W - 1) / W;
            if (wgs <= kMaxWorkgroups) {
              hipLaunchKernelGGL((reduce_split_kernel<FMT, K, U, BF16, true>), dim3((uint32_t)wgs),
                                 dim3(64 * W), lds, stream, P, y, n, full, q2w);
              return hipGetLastError();
            }
          }
        }
        hipLaunchKernelGGL((reduce_kernel<FMT, K, U, T, BF16, true>), grid, dim3(64 * W), lds,
                           stream, P, y, n, full);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((reduce_kernel<FMT, K, U, T, BF16>), grid, dim3(64 * W), lds, stream, P,
                       y, n, full);
    return hipGetLastError();
  }
}

template <int FMT, bool BF16, int K = 1>
hipError_t dispatch_k(int k, const PeerPtrs &P, uint64_t n, void *y, hipStream_t stream) {
  if constexpr (K > kMaxPeers) {
    return hipErrorInvalidValue;
  } else {
    if (k == K) return launch_reduce_t<FMT, K, BF16>(P, n, y, stream);
    return dispatch_k<FMT, BF16, K + 1>(k, P, n, y, stream);
  }
}

// ---------------------------------------------------------------------------
// Dequant-reduce, then requantize the reduced chunk (the all-gather half of
// an FP8 all-reduce sends FP8 again: "FP8 Transmission Optimization for VLA
// Training", "Threshold Changes" bullet).  The fp32 sums acc_i are block-128
// quantized directly: amax over the block, s = max(fl32(amax / FP8_MAX),
// 2^-126), q_i = satRNE(fl32(acc_i / s)).
//
// The quotient without a per-element divide.  Per block: s, sp = s * f and
// rp = RN(1 / sp), with f = 2^64 for blocks whose amax is below 2^-60 (else
// 1), so that every residual that can decide a code is a normal number; s
// and rp come from divide-free sequences equal to the IEEE divides
// (scale_from_amax, recip_rn).  Per element, with x' = acc * f (exact;
// skipped for a load whose blocks all have f = 1), one Markstein step:
//   q0 = RN(x' * rp);  e = RN(q0 * sp - x') (fma);  q1 = RN(q0 - e * rp) (fma)
// (markstein_quotient).  q1 equals the IEEE quotient for every pair of fp32
// significands (all 2^46, checked on the device), for every pair in
// emulated 8- to 16-bit binary arithmetic, and on random and
// boundary-adjacent fp32 pairs (both checked on the host).  Where an
// intermediate could leave the normal range the quotient is below 2^-26, far
// under half the smallest FP8 subnormal, and the sequence keeps the
// dividend's sign, so the code is the same signed zero.

__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

struct F32Scale {
  float s;        // the stored scale (NaN for a non-finite block)
  float sp;       // s * f
  float rp;       // RN(1 / sp)
  float f;        // 2^64 for blocks with amax below 2^-60, else 1
  bool finite;
};

template <int FMT>
__device__ __forceinline__ F32Scale f32_block_scale(uint32_t amax_bits) {
  F32Scale r;
  r.finite = amax_bits < 0x7F800000u;
  const float s = scale_from_amax<FMT>(__uint_as_float(amax_bits));  // = IEEE amax / M
  r.f = amax_bits < 0x21800000u ? 0x1p64f : 1.0f;          // amax < 2^-60
  r.sp = s * r.f;
  r.rp = recip_rn(r.sp);                                    // = IEEE 1 / sp
  r.s = r.finite ? s : __uint_as_float(0x7FC00000u);
  return r;
}

// SCALED = false may only be used where b.f == 1 (it skips x' = v * f).
// The quotient goes to cvt4 with no clamp: |RN(v / s)| <= quotient_bound
// for every v of a finite block (fp8q_device.h).
template <int FMT, bool SCALED = true>
__device__ __forceinline__ float f32_quot(float v, const F32Scale &b) {
  const float xp = SCALED ? v * b.f : v;
  return markstein_quotient(xp, b.sp, b.rp);
}

// Elements [start, n) (start is block-aligned): one block per pass, two
// elements per lane, a whole-wave amax.
template <int FIN, int FOUT, int K>
__device__ void requant_tail(const PeerPtrs &P, uint8_t *__restrict__ qo, float *__restrict__ so,
                             uint64_t n, uint64_t start) {
  const uint32_t lane = lane_id();
  for (uint64_t b0 = start; b0 < n; b0 += kBlock) {
    float v[2];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint64_t i = b0 + 2 * lane + j;
      v[j] = 0.0f;
      if (i < n) {
        const uint64_t blk = i / kBlock;
        float acc = dec1<FIN>(reinterpret_cast<const uint8_t *>(P.q[0])[i]) * P.s[0][blk];
#pragma unroll
        for (int p = 1; p < K; ++p) {
          const float d = dec1<FIN>(reinterpret_cast<const uint8_t *>(P.q[p])[i]) * P.s[p][blk];
          acc = acc + d;
        }
        v[j] = acc;
        m = m > abs_bits(acc) ? m : abs_bits(acc);
      }
    }
    const F32Scale sc = f32_block_scale<FOUT>(max_wave(m));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint64_t i = b0 + 2 * lane + j;
      if (i < n) {
        const uint32_t c = cvt4<FOUT>(f32_quot<FOUT>(v[j], sc), 0.0f, 0.0f, 0.0f);
        qo[i] = sc.finite ? (uint8_t)c : (uint8_t)0x7F;
      }
    }
    if (lane == 0) so[b0 / kBlock] = sc.s;
  }
}

// Mapping: eight codes per lane.  A lane holds elements [8 lane, 8 lane + 8)
// of each 512-element group (8-byte code loads, 512 B per wave instruction
// and peer), so a 128-element block is one 16-lane DPP row, exactly as in
// the bf16 quantize: its amax is a max over the lane's 8 sums and 4 DPP
// steps (no cross-row exchange), and each lane's block scale and reciprocal
// serve 8 elements.  Each lane loads its block's input scale per peer (16
// lanes share the address).  The codes leave as 8-byte stores (512 B per
// instruction); the tile's 4U output scales are staged in LDS and leave in
// one contiguous store per workgroup round.  Where the block amax and scale
// arithmetic, rather than HBM, bind the kernel (few peers), this halves
// their cost per element against a mapping with four codes per lane.

template <int K, int U>
struct Tile8 {
  u32x2 w[K][U];
  float s[K][U];
};

template <int K, int U>
__device__ __forceinline__ void load_tile8(const PeerPtrs &P, uint64_t t, uint32_t lane,
                                           Tile8<K, U> &in) {
  const uint64_t e0 = t * ((uint64_t)U * 512) + 8u * lane;   // lane's first element of tile t
#pragma unroll
  for (int p = 0; p < K; ++p)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t e = e0 + (uint64_t)u * 512;
      in.w[p][u] = ld<u32x2, kNtCodes<K>>(reinterpret_cast<const u32x2 *>(P.q[p]) + e / 8);
      in.s[p][u] = ld<float, false>(P.s[p] + e / kBlock);
    }
}

template <int FMT, int K, int U>
__device__ __forceinline__ void sum_tile8(const Tile8<K, U> &in, float (&acc)[U][8]) {
#pragma unroll
  for (int p = 0; p < K; ++p)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float s = in.s[p][u];
      const f32x2 a = dec2<FMT, false>(in.w[p][u].x), b = dec2<FMT, true>(in.w[p][u].x);
      const f32x2 c = dec2<FMT, false>(in.w[p][u].y), d = dec2<FMT, true>(in.w[p][u].y);
      const float v[8] = {a[0] * s, a[1] * s, b[0] * s, b[1] * s,
                          c[0] * s, c[1] * s, d[0] * s, d[1] * s};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[u][j] = (p == 0) ? v[j] : acc[u][j] + v[j];
    }
}

template <int FOUT, bool SCALED>
__device__ __forceinline__ u32x2 quot8(const float (&a)[8], const F32Scale &sc) {
  return u32x2{cvt4<FOUT>(f32_quot<FOUT, SCALED>(a[0], sc), f32_quot<FOUT, SCALED>(a[1], sc),
                          f32_quot<FOUT, SCALED>(a[2], sc), f32_quot<FOUT, SCALED>(a[3], sc)),
               cvt4<FOUT>(f32_quot<FOUT, SCALED>(a[4], sc), f32_quot<FOUT, SCALED>(a[5], sc),
                          f32_quot<FOUT, SCALED>(a[6], sc), f32_quot<FOUT, SCALED>(a[7], sc))};
}

// One tile: sum, requantize, store the codes, and put the tile's 4U scales at
// s_dst[0 .. 4U) (block u * 4 + row of the tile).
template <int FIN, int FOUT, int K, int U>
__device__ __forceinline__ void requant8_tile(const Tile8<K, U> &in, u32x2 *__restrict__ qo,
                                              float *s_dst, uint64_t t, uint32_t lane) {
  const uint32_t row = lane >> 4, col = lane & 15;
  float acc[U][8];
  sum_tile8<FIN, K, U>(in, acc);
  float sc_s[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t m = abs_bits(acc[u][0]);
#pragma unroll
    for (int j = 1; j < 8; ++j) m = m > abs_bits(acc[u][j]) ? m : abs_bits(acc[u][j]);
    const F32Scale sc = f32_block_scale<FOUT>(max_row16(m));
    u32x2 c = wave_any(sc.f != 1.0f) ? quot8<FOUT, true>(acc[u], sc) : quot8<FOUT, false>(acc[u], sc);
    if (!sc.finite) c = u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
    st(qo + t * ((uint64_t)U * 64) + (uint64_t)u * 64 + lane, c);
    sc_s[u] = sc.s;
  }
  // lane (row, col = u) writes block u * 4 + row: one LDS write covers the tile
  if (col < U) {
    float s = sc_s[0];
#pragma unroll
    for (int u = 1; u < U; ++u) s = (col == (uint32_t)u) ? sc_s[u] : s;
    s_dst[col * 4 + row] = s;
  }
}

// A wave's T consecutive tiles, the next tile's loads issued first; tile
// t0 + j puts its scales at s_dst + 4U * j.
template <int FIN, int FOUT, int K, int U, int T>
__device__ __forceinline__ void requant8_wave_tiles(const PeerPtrs &P, u32x2 *__restrict__ qo,
                                                    float *s_dst, uint64_t t0,
                                                    uint64_t full_tiles, uint32_t lane) {
  Tile8<K, U> cur;
  load_tile8<K, U>(P, t0, lane, cur);
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const uint64_t t = t0 + j;
    if (t >= full_tiles) break;
    Tile8<K, U> nxt;
    const bool more = (j + 1 < T) && (t + 1 < full_tiles);
    if (more) load_tile8<K, U>(P, t + 1, lane, nxt);
    requant8_tile<FIN, FOUT, K, U>(cur, qo, s_dst + 4 * U * j, t, lane);
    if (more) cur = nxt;
  }
}

template <int FIN, int FOUT, int K, int U, int T, int W, int C>
__global__ __launch_bounds__(64 * W) void requant8_kernel(PeerPtrs P, u32x2 *__restrict__ qo,
                                                          float *__restrict__ so, uint64_t n,
                                                          uint64_t full_tiles) {
  constexpr uint64_t kTile = (uint64_t)U * 512;
  constexpr uint32_t kTileBlocks = 4 * U;
  const uint32_t lane = lane_id();
  __shared__ float wg_scales[W * T * kTileBlocks];
  workgroup_rounds<T, W, C>(
      full_tiles,
      [&](uint64_t t0, uint32_t wid) {
        requant8_wave_tiles<FIN, FOUT, K, U, T>(P, qo, wg_scales + wid * T * kTileBlocks, t0,
                                                full_tiles, lane);
      },
      [&](uint64_t base, uint32_t tiles) {
        for (uint32_t i = threadIdx.x; i < tiles * kTileBlocks; i += 64 * W)
          so[base * kTileBlocks + i] = wg_scales[i];
      });
  if (wave_index<W, C>() == wave_count<W>() - 1)
    requant_tail<FIN, FOUT, K>(P, reinterpret_cast<uint8_t *>(qo), so, n, full_tiles * kTile);
}

// One pass with a one-tile tail, as the block quantize's split kernel:
// workgroups at positions below q2 (a multiple of the XCD run C) take two
// tiles per wave, the rest one, so the launch's last waves carry half the
// serial chain.  The scale flush and the ragged tail are as in
// requant8_kernel.
template <int FIN, int FOUT, int K, int U, int W, int C>
__global__ __launch_bounds__(64 * W) void requant8_split_kernel(PeerPtrs P, u32x2 *__restrict__ qo,
                                                                float *__restrict__ so, uint64_t n,
                                                                uint64_t full_tiles, uint32_t q2) {
  constexpr uint64_t kTile = (uint64_t)U * 512;
  constexpr uint32_t kTileBlocks = 4 * U;
  const uint32_t lane = lane_id();
  const uint32_t wid = uniform(threadIdx.x / kWave);
  const uint32_t pos = block_position<C>();
  __shared__ float wg_scales[W * 2 * kTileBlocks];
  uint64_t base;
  uint32_t wg_tiles;
  if (pos < q2) {
    base = (uint64_t)pos * W * 2;
    wg_tiles = W * 2;
    const uint64_t t0 = base + (uint64_t)wid * 2;
    if (t0 < full_tiles)
      requant8_wave_tiles<FIN, FOUT, K, U, 2>(P, qo, wg_scales + wid * 2 * kTileBlocks, t0,
                                              full_tiles, lane);
  } else {
    base = (uint64_t)q2 * W * 2 + (uint64_t)(pos - q2) * W;
    wg_tiles = W;
    const uint64_t t0 = base + wid;
    if (t0 < full_tiles)
      requant8_wave_tiles<FIN, FOUT, K, U, 1>(P, qo, wg_scales + wid * kTileBlocks, t0,
                                              full_tiles, lane);
  }
  __syncthreads();
  const uint64_t left = base < full_tiles ? full_tiles - base : 0;
  const uint32_t tiles = left < wg_tiles ? (uint32_t)left : wg_tiles;
  for (uint32_t i = threadIdx.x; i < tiles * kTileBlocks; i += 64 * W)
    so[base * kTileBlocks + i] = wg_scales[i];
  if (wave_index<W, C>() == wave_count<W>() - 1)
    requant_tail<FIN, FOUT, K>(P, reinterpret_cast<uint8_t *>(qo), so, n, full_tiles * kTile);
}

// From FP8Q_RQ8_TAIL_MIN_K peers the last FP8Q_RQ8_TAIL_TILES tiles of a
// launch go one per wave (requant8_split_kernel).  On MI355X (graph replay
// over rotating windows, alternated in one run, e4m3 -> e4m3, % of 8 TB/s),
// with 4096 tiles: 4 peers 55.2 -> 59.7 at 16 MiB, 75.1 -> 76.3 at 64 MiB,
// 80.9 -> 81.6 at 128 MiB; 8 peers 61.5 -> 62.8, 77.3 -> 78.0 and equal at
// 128 MiB.  With one peer it lost 1.8 points at 16 MiB, so fewer peers keep
// requant8_kernel.
#ifndef FP8Q_RQ8_TAIL_TILES
#define FP8Q_RQ8_TAIL_TILES 4096
#endif
#ifndef FP8Q_RQ8_TAIL_MIN_K
#define FP8Q_RQ8_TAIL_MIN_K 4
#endif

// Tile shape: U = 2 groups of 512 elements per tile, T = 2 tiles per wave,
// 4-wave workgroups, at every peer count.  Against the previous requantize
// (four codes per lane, a block across 32 lanes, its tile shape tuned per
// peer count), measured on MI355X with the variants alternated in one run
// (graph replay over rotating windows, % of 8 TB/s at 437.5 MiB / 64 MiB per
// peer): k = 1 75 / 58 against 58 / 48; k = 8 80 / 76 against 78 / 69;
// k = 12 76 / 76 against 70 / 68.5; k = 16 75.5 / 78 against 75 / 71; k = 4
// 81.5 / 74 against 82 / 71.5.  T = 4 was slower, and so was U = 1 from 9
// peers up (7-10%), although it halves the registers (k >= 12 holds 256
// VGPRs, one wave per SIMD, with 32 KiB of codes in flight per wave).
#ifndef FP8Q_RQ8_U
#define FP8Q_RQ8_U 2             // 512-element groups per tile
#endif
template <int K>
constexpr int requant8_u() {
  return FP8Q_RQ8_U;
}
#ifndef FP8Q_RQ8_T
#define FP8Q_RQ8_T 2             // tiles per wave
#endif
// XCD runs of 16 workgroups: against 64 they measured 1.5-3% faster at
// 437.5 MiB per peer for 2-16 peers and on the 8 x 437.5M-element gradient
// shards (80.1% against 78.4%), about 1% slower at 64 MiB from 8 peers up.
#ifndef FP8Q_XCD_CHUNK_RQ
#define FP8Q_XCD_CHUNK_RQ 16     // XCD run (workgroups) of the requantize
#endif
// Small launches: below FP8Q_RQ8_T1_BELOW_N elements (FP8Q_RQ8_T1_BELOW_N_K4
// from 4 peers) each wave takes one tile of one 512-element group
// (FP8Q_RQ8_SMALL_U), not two tiles of two: four times the waves, each with
// a quarter of the serial chain.  Two-tile waves left small launches with
// a few hundred waves on 256 CUs.  On MI355X (graph replay over rotating
// windows, alternated in one run, e4m3 -> e4m3, % of 8 TB/s) at a 767 KiB
// payload: 1 peer 2.4 -> 4.5, 8 peers 6.1 -> 15.0, 16 peers 8.0 -> 22.9;
// 2 MiB: 8 peers 21.5 -> 30.3; 7.9 MiB: 8 peers 52.2 -> 59.3; from 4 peers
// also at 16 MiB (8 peers 62.5 -> 73.1) and 24 MiB (70.6 -> 74.4), tied at
// 32 MiB and lower from there.  With 1 and 2 peers it lost 6-21% at 12-16
// MiB, hence the lower bound below 4 peers.  One-wave workgroups measured
// within a few percent either way.  With 1 peer the windows of those runs
// fit in the 256 MB Infinity Cache; with the data in HBM (768 MB of windows
// per graph) it measured +1.4 / +0.8 / +1.0 points at 2 / 4 / 6 MiB and
// -0.4 at 7.9 MiB.
#ifndef FP8Q_RQ8_T1_BELOW_N
#define FP8Q_RQ8_T1_BELOW_N (1ull << 22)
#endif
#ifndef FP8Q_RQ8_T1_BELOW_N_K4
#define FP8Q_RQ8_T1_BELOW_N_K4 (1ull << 24)
#endif
#ifndef FP8Q_RQ8_SMALL_U
#define FP8Q_RQ8_SMALL_U 1
#endif

template <int FIN, int FOUT, int K>
void launch_requant8(const PeerPtrs &P, uint64_t n, void *qo, float *so, hipStream_t stream) {
  constexpr int U = requant8_u<K>();
  constexpr int T = FP8Q_RQ8_T;
  constexpr int W = 4;
  const uint64_t full = n / ((uint64_t)U * 512);
  constexpr uint64_t kTail = FP8Q_RQ8_TAIL_TILES;
  constexpr uint64_t C = FP8Q_XCD_CHUNK_RQ;
  constexpr uint64_t kT1Below = K >= 4 ? (uint64_t)FP8Q_RQ8_T1_BELOW_N_K4
                                       : (uint64_t)FP8Q_RQ8_T1_BELOW_N;
  if (n < kT1Below) {
    constexpr int SU = FP8Q_RQ8_SMALL_U;
    const uint64_t sfull = n / ((uint64_t)SU * 512);
    hipLaunchKernelGGL((requant8_kernel<FIN, FOUT, K, SU, 1, W, FP8Q_XCD_CHUNK_RQ>),
                       dim3(grid_for_tiles(sfull, W)), dim3(64 * W), 0, stream, P,
                       static_cast<u32x2 *>(qo), so, n, sfull);
    return;
  }
  if constexpr (T == 2 && kTail > 0 && K >= FP8Q_RQ8_TAIL_MIN_K) {
    if (full >= 2 * kTail) {
      const uint64_t q2 = (full - kTail) / (2 * W) / C * C;
      const uint64_t wgs = q2 + (full - q2 * 2 * W + W - 1) / W;
      if (wgs <= kMaxWorkgroups) {
        hipLaunchKernelGGL((requant8_split_kernel<FIN, FOUT, K, U, W, FP8Q_XCD_CHUNK_RQ>),
                           dim3((uint32_t)wgs), dim3(64 * W), 0, stream, P,
                           static_cast<u32x2 *>(qo), so, n, full, (uint32_t)q2);
        return;
      }
    }
  }
  hipLaunchKernelGGL((requant8_kernel<FIN, FOUT, K, U, T, W, FP8Q_XCD_CHUNK_RQ>),
                     dim3(grid_for_tiles((full + T - 1) / T, W)), dim3(64 * W), 0, stream, P,
                     static_cast<u32x2 *>(qo), so, n, full);
}

// The k-peer reduce with eight codes per lane: the requantize's mapping and
// tile loads, then the ordered sum stored as fp32 or bf16 (see launch_reduce_t
// for which peer counts and outputs take it).
template <bool BF16>
__device__ __forceinline__ void store8(void *y, uint64_t e, const float (&a)[8]) {
  if constexpr (BF16) {
    st(reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(y) + e),
       u32x4{bf16_pack2(a[0], a[1]), bf16_pack2(a[2], a[3]), bf16_pack2(a[4], a[5]),
             bf16_pack2(a[6], a[7])});
  } else {
    st(reinterpret_cast<f32x4 *>(static_cast<float *>(y) + e), f32x4{a[0], a[1], a[2], a[3]});
    st(reinterpret_cast<f32x4 *>(static_cast<float *>(y) + e + 4), f32x4{a[4], a[5], a[6], a[7]});
  }
}

template <int FMT, int K, int U, int T, bool BF16, int W, int C>
__global__ __launch_bounds__(64 * W) void reduce8_kernel(PeerPtrs P, void *__restrict__ y,
                                                         uint64_t n, uint64_t full_tiles) {
  constexpr uint64_t kTile = (uint64_t)U * 512;
  const uint32_t lane = lane_id();
  const uint64_t nw = wave_count<W>();
  const uint64_t w0 = wave_index<W, C>();
  for (uint64_t t0 = w0 * T; t0 < full_tiles; t0 += nw * T) {
    Tile8<K, U> cur;
    load_tile8<K, U>(P, t0, lane, cur);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const uint64_t t = t0 + j;
      if (t >= full_tiles) break;
      Tile8<K, U> nxt;
      const bool more = (j + 1 < T) && (t + 1 < full_tiles);
      if (more) load_tile8<K, U>(P, t + 1, lane, nxt);
      float acc[U][8];
      sum_tile8<FMT, K, U>(cur, acc);
#pragma unroll
      for (int u = 0; u < U; ++u) store8<BF16>(y, t * kTile + (uint64_t)u * 512 + 8u * lane, acc[u]);
      if (more) cur = nxt;
    }
  }
  if (w0 == nw - 1) reduce_tail<FMT, K, BF16>(P, y, n, full_tiles * kTile);
}

template <int FMT, int K, bool BF16>
hipError_t launch_reduce8_t(const PeerPtrs &P, uint64_t n, void *y, hipStream_t stream) {
  constexpr int U = FP8Q_RED8_U, T = FP8Q_RED8_T, W = FP8Q_RED8_W;
  const uint64_t full = n / ((uint64_t)U * 512);
  constexpr uint64_t kT1Below = K >= FP8Q_RED8_MIN_K_BF16 ? (uint64_t)FP8Q_RED8_T1_BELOW_N
                                                          : (uint64_t)FP8Q_RED8_T1_BELOW_N_LARGE;
  if (n < kT1Below) {
    hipLaunchKernelGGL((reduce8_kernel<FMT, K, U, 1, BF16, W, FP8Q_RED8_C>),
                       dim3(grid_for_tiles(full, W)), dim3(64 * W), 0, stream, P, y, n, full);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((reduce8_kernel<FMT, K, U, T, BF16, W, FP8Q_RED8_C>),
                     dim3(grid_for_tiles((full + T - 1) / T, W)), dim3(64 * W), 0, stream, P, y,
                     n, full);
  return hipGetLastError();
}

template <int FMT, bool BF16>
hipError_t launch_deq8_t(const PeerPtrs &P, uint64_t n, void *y, hipStream_t stream) {
  constexpr int W = FP8Q_RED8_W;
  const uint64_t full = n / 512;
  hipLaunchKernelGGL((reduce8_kernel<FMT, 1, 1, 1, BF16, W, FP8Q_RED8_C>),
                     dim3(grid_for_tiles(full, W)), dim3(64 * W), 0, stream, P, y, n, full);
  return hipGetLastError();
}

template <int FIN, int FOUT, int K>
hipError_t launch_requant_t(const PeerPtrs &P, uint64_t n, void *qo, float *so, hipStream_t stream) {
  launch_requant8<FIN, FOUT, K>(P, n, qo, so, stream);
  return hipGetLastError();
}

template <int FIN, int FOUT, int K = 1>
hipError_t dispatch_requant_k(int k, const PeerPtrs &P, uint64_t n, void *qo, float *so,
                              hipStream_t stream) {
  if constexpr (K > kMaxPeers) {
    return hipErrorInvalidValue;
  } else {
    if (k == K) return launch_requant_t<FIN, FOUT, K>(P, n, qo, so, stream);
    return dispatch_requant_k<FIN, FOUT, K + 1>(k, P, n, qo, so, stream);
  }
}

// ---------------------------------------------------------------------------
// MXFP8 receiver side: y = sum over peers of dec_e4m3(q_p) * 2^(code_p - 127)
// per 32-element block ("perf: Reduce MXFP8 refit weight-transfer
// overheads": the receiver of the prequantized weights; its E8M0 zero-scale
// clamp must agree with the trainer's).  The [rows, K] codes and the
// [rows, K/32] scale bytes are both flat in block order (K % 32 == 0), so the
// kernel runs over n = rows * K elements.  Each 4-code dword of a lane lies in
// one 32-element block; its E8M0 byte is loaded per lane (8 lanes share it).
// The decode and the scaling are one gfx950 scaled conversion per two codes
// (mx_dec2), equal to fl32(dec(q) * 2^(code - 127)) for every code and scale
// (code 0 scales by 2^-127, 0xFF gives NaN).  Each product is exact (unless
// it overflows to +-inf, which codes made by mx8_quantize never do); the sum
// is in peer order.  Against a decode, a multiply and the scale built from
// bits, on MI355X (alternated in one run): one shard into bf16 at 256 MiB
// 83.4 -> 85.3% of 8 TB/s, 8 peers into fp32 at 64 MiB 78.9 -> 79.8%, other
// sizes within 0.4%.

struct MxPeerPtrs {
  const uint32_t *q[kMaxPeers];
  const uint8_t *e[kMaxPeers];
};

template <int K, bool BF16>
__device__ void mx_reduce_tail(const MxPeerPtrs &P, void *__restrict__ y, uint64_t n, uint64_t start) {
  for (uint64_t i = start + lane_id(); i < n; i += kWave) {
    const uint64_t blk = i / kMxBlock;
    float acc = mx_dec2<false>(reinterpret_cast<const uint8_t *>(P.q[0])[i], P.e[0][blk])[0];
#pragma unroll
    for (int p = 1; p < K; ++p) {
      const float d = mx_dec2<false>(reinterpret_cast<const uint8_t *>(P.q[p])[i], P.e[p][blk])[0];
      acc = acc + d;
    }
    store1<BF16>(y, i, acc);
  }
}

template <int K, int U>
__device__ __forceinline__ void mx_load(const MxPeerPtrs &P, uint64_t t, uint32_t lane,
                                        uint32_t (&w)[K][U], uint32_t (&c)[K][U]) {
  constexpr uint64_t kTile = (uint64_t)U * 256;
  const uint64_t dw0 = t * (kTile / 4);
#pragma unroll
  for (int p = 0; p < K; ++p)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w[p][u] = ld<uint32_t, kNtCodes<K>>(P.q[p] + dw0 + u * kWave + lane);
      c[p][u] = P.e[p][(t * kTile + (uint64_t)u * 256) / kMxBlock + lane / 8];
    }
}

template <int K, int U, bool BF16>
__device__ __forceinline__ void mx_reduce_tile(const uint32_t (&w)[K][U], const uint32_t (&c)[K][U],
                                               void *__restrict__ y, uint64_t t, uint32_t lane) {
  constexpr uint64_t kTile = (uint64_t)U * 256;
  float acc[U][4];
#pragma unroll
  for (int p = 0; p < K; ++p)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const f32x2 lo = mx_dec2<false>(w[p][u], c[p][u]);
      const f32x2 hi = mx_dec2<true>(w[p][u], c[p][u]);
      const float d0 = lo[0], d1 = lo[1], d2 = hi[0], d3 = hi[1];
      if (p == 0) {
        acc[u][0] = d0; acc[u][1] = d1; acc[u][2] = d2; acc[u][3] = d3;
      } else {
        acc[u][0] = acc[u][0] + d0; acc[u][1] = acc[u][1] + d1;
        acc[u][2] = acc[u][2] + d2; acc[u][3] = acc[u][3] + d3;
      }
    }
#pragma unroll
  for (int u = 0; u < U; ++u)
    store4<BF16>(y, t * kTile + (uint64_t)u * 256 + 4 * lane, acc[u][0], acc[u][1], acc[u][2],
                 acc[u][3]);
}

// T consecutive tiles per wave, the next tile's loads issued first.
template <int K, int U, int T, bool BF16>
__global__ __launch_bounds__(256) void mx_reduce_kernel(MxPeerPtrs P, void *__restrict__ y,
                                                        uint64_t n, uint64_t full_tiles) {
  constexpr uint64_t kTile = (uint64_t)U * 256;
  const uint32_t lane = lane_id();
  const uint64_t nw = wave_count<4>();
  const uint64_t w0 = wave_index<4>();

  for (uint64_t t0 = w0 * T; t0 < full_tiles; t0 += nw * T) {
    uint32_t cw[K][U], cc[K][U];
    mx_load<K, U>(P, t0, lane, cw, cc);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const uint64_t t = t0 + j;
      if (t >= full_tiles) break;
      uint32_t nw_[K][U], nc[K][U];
      const bool more = (j + 1 < T) && (t + 1 < full_tiles);
      if (more) mx_load<K, U>(P, t + 1, lane, nw_, nc);
      mx_reduce_tile<K, U, BF16>(cw, cc, y, t, lane);
      if (more) {
#pragma unroll
        for (int p = 0; p < K; ++p)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            cw[p][u] = nw_[p][u];
            cc[p][u] = nc[p][u];
          }
      }
    }
  }
  if (w0 == nw - 1) mx_reduce_tail<K, BF16>(P, y, n, full_tiles * kTile);
}

// The MXFP8 receiver's tile depth: as the block-128 reduce up to 8 peers,
// U = 1 beyond (its scales are always vector byte loads).  A single shard
// into fp32 takes U = FP8Q_MX_U1_F32 (U = 1 measured 2.5% faster than 2 on
// MI355X; into bf16 U = 1 was 20% slower).
#ifndef FP8Q_MX_U1_F32
#define FP8Q_MX_U1_F32 1
#endif
template <int K, bool BF16>
constexpr int mx_reduce_u() {
  return (K == 1 && !BF16) ? FP8Q_MX_U1_F32 : (K <= 8 ? peers_u<K>() : 1);
}

// Small launches from FP8Q_MXR_SMALL_MIN_K peers: below FP8Q_MXR_T1_BELOW_N
// elements (a 4 MiB payload) each wave takes one tile of one 256-element
// group, not two tiles of two.  On MI355X (alternated in one run, % change
// at 256 KiB / 768 KiB / 2 MiB): 4 peers into fp32 +12 / +13 / +9, 8 peers
// +24 / +20 / +2.5, into bf16 +16 / +12 / +9 and +29 / +20 / +6.5.  At 4 MiB
// it lost 4-8%, and with one shard it changed nothing up to 4 MiB.
#ifndef FP8Q_MXR_T1_BELOW_N
#define FP8Q_MXR_T1_BELOW_N (1ull << 21)
#endif
#ifndef FP8Q_MXR_SMALL_MIN_K
#define FP8Q_MXR_SMALL_MIN_K 4
#endif
template <int K, bool BF16>
hipError_t launch_mx_reduce_t(const MxPeerPtrs &P, uint64_t n, void *y, hipStream_t stream) {
  constexpr int U = mx_reduce_u<K, BF16>();
  constexpr int T = FP8Q_RED_T;
  const uint64_t full = n / ((uint64_t)U * 256);
  if constexpr (K >= FP8Q_MXR_SMALL_MIN_K) {
    if (n < FP8Q_MXR_T1_BELOW_N) {
      const uint64_t sfull = n / 256;
      hipLaunchKernelGGL((mx_reduce_kernel<K, 1, 1, BF16>), dim3(grid_for_tiles(sfull)),
                         dim3(256), 0, stream, P, y, n, sfull);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((mx_reduce_kernel<K, U, T, BF16>), dim3(grid_for_tiles((full + T - 1) / T)),
                     dim3(256), 0, stream, P, y, n, full);
  return hipGetLastError();
}

template <bool BF16, int K = 1>
hipError_t dispatch_mx_k(int k, const MxPeerPtrs &P, uint64_t n, void *y, hipStream_t stream) {
  if constexpr (K > kMaxPeers) {
    return hipErrorInvalidValue;
  } else {
    if (k == K) return launch_mx_reduce_t<K, BF16>(P, n, y, stream);
    return dispatch_mx_k<BF16, K + 1>(k, P, n, y, stream);
  }
}

// ---------------------------------------------------------------------------
// Naive comparator: y = ((p_0 + p_1) + ...) over k fp32 arrays.

template <bool BF16>
__global__ __launch_bounds__(256) void sum_kernel(PartPtrs P, int k, void *__restrict__ y,
                                                  uint64_t n) {
  constexpr uint64_t kThreads = 256;               // the launch's workgroup size
  const uint64_t n4 = n / 4;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    float4 a = reinterpret_cast<const float4 *>(P.p[0])[i];
    for (int p = 1; p < k; ++p) {
      const float4 b = reinterpret_cast<const float4 *>(P.p[p])[i];
      a.x = a.x + b.x; a.y = a.y + b.y; a.z = a.z + b.z; a.w = a.w + b.w;
    }
    store4<BF16>(y, 4 * i, a.x, a.y, a.z, a.w);
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) {
    const uint64_t i = 4 * n4 + threadIdx.x;
    float a = P.p[0][i];
    for (int p = 1; p < k; ++p) a = a + P.p[p][i];
    store1<BF16>(y, i, a);
  }
}

}  // namespace

hipError_t launch_dequant_reduce(int fmt, int k, bool out_bf16, const void *const *q,
                                 const float *const *scales, uint64_t n, void *y,
                                 hipStream_t stream) {
  PeerPtrs P = {};
  for (int p = 0; p < k; ++p) {
    P.q[p] = static_cast<const uint32_t *>(q[p]);
    P.s[p] = scales[p];
  }
  if (fmt == 0)
    return out_bf16 ? dispatch_k<0, true>(k, P, n, y, stream)
                    : dispatch_k<0, false>(k, P, n, y, stream);
  return out_bf16 ? dispatch_k<1, true>(k, P, n, y, stream)
                  : dispatch_k<1, false>(k, P, n, y, stream);
}

hipError_t launch_reduce_requantize(int fmt_in, int fmt_out, int k, const void *const *q,
                                   const float *const *scales, uint64_t n, void *q_out,
                                   float *scales_out, hipStream_t stream) {
  PeerPtrs P = {};
  for (int p = 0; p < k; ++p) {
    P.q[p] = static_cast<const uint32_t *>(q[p]);
    P.s[p] = scales[p];
  }
  if (fmt_in == 0)
    return fmt_out == 0 ? dispatch_requant_k<0, 0>(k, P, n, q_out, scales_out, stream)
                        : dispatch_requant_k<0, 1>(k, P, n, q_out, scales_out, stream);
  return fmt_out == 0 ? dispatch_requant_k<1, 0>(k, P, n, q_out, scales_out, stream)
                      : dispatch_requant_k<1, 1>(k, P, n, q_out, scales_out, stream);
}

hipError_t launch_mx8_dequant_reduce(int k, bool out_bf16, const void *const *q,
                                     const void *const *e8m0, uint64_t n, void *y,
                                     hipStream_t stream) {
  MxPeerPtrs P = {};
  for (int p = 0; p < k; ++p) {
    P.q[p] = static_cast<const uint32_t *>(q[p]);
    P.e[p] = static_cast<const uint8_t *>(e8m0[p]);
  }
  return out_bf16 ? dispatch_mx_k<true>(k, P, n, y, stream) : dispatch_mx_k<false>(k, P, n, y, stream);
}

hipError_t launch_sum_f32(int k, bool out_bf16, const float *const *parts, uint64_t n, void *y,
                          hipStream_t stream) {
  PartPtrs P = {};
  for (int p = 0; p < k; ++p) P.p[p] = parts[p];
  // one float4 per thread: 256 threads = 4 "tiles" of 64 float4
  const uint32_t wgs = grid_for_tiles((n / 4 + 63) / 64);
  if (out_bf16)
    hipLaunchKernelGGL(sum_kernel<true>, dim3(wgs), dim3(256), 0, stream, P, k, y, n);
  else
    hipLaunchKernelGGL(sum_kernel<false>, dim3(wgs), dim3(256), 0, stream, P, k, y, n);
  return hipGetLastError();
}

}  // namespace fp8q
