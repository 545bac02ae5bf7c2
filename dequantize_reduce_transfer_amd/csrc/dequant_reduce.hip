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
// 2U blocks of 128); all k * U code loads are issued before any arithmetic.
// Lanes 0-31 of a group share one block and lanes 32-63 the next, so a
// peer's 2U scales of a tile are wave-uniform and come in through the scalar
// cache.  Codes are decoded by the hardware packed FP8->fp32 conversion.
// The dequantized values live only in registers.
#include "fp8q_device.h"
#include "launch.h"

namespace fp8q {
namespace {

#ifndef FP8Q_RED_U4
#define FP8Q_RED_U4 4        // tile depth for k <= 4
#endif
#ifndef FP8Q_RED_U8
#define FP8Q_RED_U8 2        // tile depth for 4 < k <= 8
#endif
#ifndef FP8Q_RED_U16
#define FP8Q_RED_U16 1       // tile depth for 8 < k <= 16
#endif

struct PeerPtrs {
  const uint32_t *q[kMaxPeers];
  const float *s[kMaxPeers];
};

struct PartPtrs {
  const float *p[kMaxPeers];
};

// Codes in flight per wave: k * U * 256 B.  U shrinks as k grows so that the
// 2U scales of every peer fit the scalar register file.
template <int K>
constexpr int reduce_u() {
  return K <= 4 ? FP8Q_RED_U4 : (K <= 8 ? FP8Q_RED_U8 : FP8Q_RED_U16);
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

template <int FMT, int K, int U, bool BF16>
__global__ __launch_bounds__(256) void reduce_kernel(PeerPtrs P, void *__restrict__ y, uint64_t n,
                                                     uint64_t full_tiles) {
  constexpr uint64_t kTile = (uint64_t)U * 256;    // elements per tile
  constexpr uint64_t kTileBlocks = kTile / kBlock; // = 2U
  const uint32_t lane = lane_id();
  const bool upper = lane >= 32;
  const uint64_t nw = wave_count();
  const uint64_t w0 = wave_index();

  for (uint64_t t = w0; t < full_tiles; t += nw) {
    const uint64_t dw0 = t * (kTile / 4);          // first code dword of the tile
    uint32_t w[K][U];
#pragma unroll
    for (int p = 0; p < K; ++p)
#pragma unroll
      for (int u = 0; u < U; ++u) w[p][u] = ld<uint32_t, kNtCodes<K>>(P.q[p] + dw0 + u * kWave + lane);

    float acc[U][4];
#pragma unroll
    for (int p = 0; p < K; ++p) {
      const float *sp = P.s[p] + t * kTileBlocks;  // wave-uniform
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float s = upper ? sp[2 * u + 1] : sp[2 * u];
        const f32x2 lo = dec2<FMT, false>(w[p][u]);
        const f32x2 hi = dec2<FMT, true>(w[p][u]);
        const float d0 = lo[0] * s, d1 = lo[1] * s, d2 = hi[0] * s, d3 = hi[1] * s;
        if (p == 0) {
          acc[u][0] = d0; acc[u][1] = d1; acc[u][2] = d2; acc[u][3] = d3;
        } else {
          acc[u][0] = acc[u][0] + d0; acc[u][1] = acc[u][1] + d1;
          acc[u][2] = acc[u][2] + d2; acc[u][3] = acc[u][3] + d3;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      store4<BF16>(y, t * kTile + (uint64_t)u * 256 + 4 * lane, acc[u][0], acc[u][1], acc[u][2],
                   acc[u][3]);
  }
  if (w0 == nw - 1) reduce_tail<FMT, K, BF16>(P, y, n, full_tiles * kTile);
}

template <int FMT, int K, bool BF16>
hipError_t launch_reduce_t(const PeerPtrs &P, uint64_t n, void *y, hipStream_t stream) {
  constexpr int U = reduce_u<K>();
  const uint64_t tile = (uint64_t)U * 256;
  const uint64_t full = n / tile;
  hipLaunchKernelGGL((reduce_kernel<FMT, K, U, BF16>), dim3(grid_for_tiles(full)), dim3(256), 0,
                     stream, P, y, n, full);
  return hipGetLastError();
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
// Naive comparator: y = ((p_0 + p_1) + ...) over k fp32 arrays.

template <bool BF16>
__global__ __launch_bounds__(256) void sum_kernel(PartPtrs P, int k, void *__restrict__ y,
                                                  uint64_t n) {
  const uint64_t n4 = n / 4;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
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
