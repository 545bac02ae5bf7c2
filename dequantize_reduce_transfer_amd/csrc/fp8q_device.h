// fp8q_device.h -- gfx950 device helpers shared by the codec's kernels.
//
// Wave64 only.  Cross-lane reductions use DPP (no LDS); FP8 conversions use
// the CDNA4 packed conversion instructions, which implement the OCP E4M3 /
// E5M2 formats with round-to-nearest-even (the default MODE rounding).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Streaming hints: non-temporal loads / stores (global_load/store ... nt).
// Every byte is touched once, so keeping it out of the caches measured
// 3-10% faster on the streaming kernels.
#ifndef FP8Q_NT_LOAD
#define FP8Q_NT_LOAD 1
#endif
#ifndef FP8Q_NT_STORE
#define FP8Q_NT_STORE 1
#endif


namespace fp8q {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T, bool NT = (FP8Q_NT_LOAD != 0)>
__device__ __forceinline__ T ld(const T *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <typename T>
__device__ __forceinline__ void st(T *p, T v) {
#if FP8Q_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

constexpr int kWave = 64;
constexpr int kBlock = 128;      // elements per fp32 scale
constexpr int kMxBlock = 32;     // elements per E8M0 scale

// DPP control words (CDNA DPP encodings).
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return v > o ? v : o;
}

// Max over the 4 lanes of a quad: every lane gets the result.
__device__ __forceinline__ uint32_t max_quad(uint32_t v) {
  v = dpp_max<kDppQuadXor1>(v);
  return dpp_max<kDppQuadXor2>(v);
}

// Max over a row of 16 lanes: every lane gets the result.
__device__ __forceinline__ uint32_t max_row16(uint32_t v) {
  v = max_quad(v);
  v = dpp_max<kDppRowHalfMirror>(v);
  return dpp_max<kDppRowMirror>(v);
}

// Max over a 32-lane half-wave (every lane gets its half's result): rows
// 0<->1 and 2<->3 are exchanged through the lane crossbar (ds_bpermute).
__device__ __forceinline__ uint32_t max_half32(uint32_t v) {
  v = max_row16(v);
  const uint32_t o = (uint32_t)__shfl_xor((int)v, 16);
  return v > o ? v : o;
}

// Max over the whole wave.
__device__ __forceinline__ uint32_t max_wave(uint32_t v) {
  v = max_half32(v);
  const uint32_t o = (uint32_t)__shfl_xor((int)v, 32);
  return v > o ? v : o;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Largest sign-cleared bf16 bit pattern among the 8 bf16 held in a u32x4.
// For finite values this is the bit pattern of max |x|; inf / NaN patterns
// (>= 0x7F80) order above every finite one.
__device__ __forceinline__ uint32_t amax_bits8(u32x4 v) {
  const uint32_t m = 0x7FFF7FFFu;
  u16x2 a = __builtin_bit_cast(u16x2, v.x & m);
  u16x2 b = __builtin_bit_cast(u16x2, v.y & m);
  u16x2 c = __builtin_bit_cast(u16x2, v.z & m);
  u16x2 d = __builtin_bit_cast(u16x2, v.w & m);
  u16x2 r = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                      __builtin_elementwise_max(c, d));
  uint32_t lo = r.x, hi = r.y;
  return lo > hi ? lo : hi;
}

// The two bf16 halves of a dword as fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Pack four fp32 values into four FP8 codes (byte i <- value i).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  // The first conversion writes the low half and the second the high half,
  // so the word they start from is never seen: it is a's own register,
  // which saves zeroing one.
  uint32_t r = __float_as_uint(a);
  if constexpr (FMT == 0) {
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)r, false);
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)r, true);
  } else {
    r = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)r, false);
    r = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, (int)r, true);
  }
  return r;
}

// Decode FP8 codes 0,1 (HI = false) or 2,3 (HI = true) of a dword to fp32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int FMT, bool HI>
__device__ __forceinline__ f32x2 dec2(uint32_t w) {
  if constexpr (FMT == 0)
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  else
    return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
}

// E4M3 codes 0,1 (HI = false) or 2,3 (HI = true) of a dword, each times the
// E8M0 scale 2^(e8m0 - 127), in one gfx950 scaled conversion.  The scale
// operand's exponent field carries the E8M0 code (e8m0 << 23): code 0 scales
// by 2^-127 and 0xFF gives NaN, as E8M0 defines.  Equal to
// fl32(dec(q) * 2^(e8m0 - 127)) for every code and every scale, NaN as NaN
// (checked on the device against the oracle's MXFP8 dequantize).
template <bool HI>
__device__ __forceinline__ f32x2 mx_dec2(uint32_t w, uint32_t e8m0) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w, __uint_as_float(e8m0 << 23), HI);
}

template <int FMT>
__device__ __forceinline__ float fp8_max() {
  return FMT == 0 ? 448.0f : 57344.0f;
}

// The encode step of the MXFP8 kernels before cvt4: clamp to +-FP8_MAX
// (v_med3_f32), so that the packed conversion only rounds and the codec's
// saturation comes from the clamp.  An input beyond the range, +-inf
// included, becomes the largest finite code of its sign.  Callers never pass
// NaN (blocks holding a non-finite value take the all-0x7F path instead).
template <int FMT>
__device__ __forceinline__ float sat_clamp(float v) {
  return __builtin_amdgcn_fmed3f(v, -fp8_max<FMT>(), fp8_max<FMT>());
}

// The quotient encode of the block-scale kernels (block quantize, tensorwise,
// requantize) needs no clamp.  With s = max(RN(amax / FP8_MAX), 2^-126) for a
// finite amax and |x| <= amax, the quotient RN(x / s) never exceeds
// quotient_bound = FP8_MAX * (1 + 2^-23) in magnitude (the next fp32 above
// FP8_MAX): RN(amax / M) >= (amax / M)(1 - 2^-24) where it is normal, the
// 2^-126 floor only makes s larger, and rounding is monotone.  This is
// checked on the host for every finite fp32 amax (quotient_bound_exhaust),
// and cvt4 alone equals the saturating RNE encode for every fp32 in
// [-quotient_bound, quotient_bound] (checked on the device against the
// oracle for all of them), so the clamp could never change a code there.
template <int FMT>
__host__ __device__ __forceinline__ constexpr float quotient_bound() {
  return FMT == 0 ? 0x1.c00002p+8f : 0x1.c00002p+15f;   // 448 (1 + 2^-23), 57344 (1 + 2^-23)
}

// The block scale max(RN(amax / FP8_MAX), 2^-126) without a divide.
// FP8_MAX = 7 * 2^m (m = 6 for e4m3, 13 for e5m2), so the quotient is
// RN(amax / 7) scaled by 2^-m, exactly, wherever it is at least 2^-126; below
// that the clamp gives 2^-126 either way.  RN(amax / 7) is one Markstein step
// from c = RN(1/7):
//   q0 = RN(amax * c),  r = amax - 7 q0 (fma, exact),  t = RN(q0 + r * c) (fma).
// t equals the IEEE quotient amax / 7 for every finite non-negative fp32
// amax, and the clamped result equals the IEEE-divide scale for both formats
// (each checked over all 2^31 such inputs).  A non-finite amax yields 2^-126
// here (the NaN quotient loses to the clamp); callers store NaN for it.
template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax) {
  constexpr float c = 0x1.24924ap-3f;                       // RN(1/7)
  const float q0 = amax * c;
  const float r = __builtin_fmaf(-q0, 7.0f, amax);
  const float t = __builtin_fmaf(r, c, q0);
  return fmaxf(t * (FMT == 0 ? 0x1p-6f : 0x1p-13f), 0x1p-126f);
}

// RN(1 / x) for a normal x whose reciprocal is normal: the hardware
// reciprocal (within one ulp) refined by one Newton step in fma.  On MI355X it
// equals the IEEE divide 1 / x for every such x (checked on the device over
// all of them).
__device__ __forceinline__ float recip_rn(float x) {
  const float r0 = __builtin_amdgcn_rcpf(x);
  const float e = __builtin_fmaf(-x, r0, 1.0f);
  return __builtin_fmaf(e, r0, r0);
}

// RN(x / s) of an fp32 x without a divide, given rp = RN(1 / s): one
// Markstein correction step,
//   q0 = RN(x * rp),  e = RN(q0 * s - x) (fma),  q1 = RN(q0 - e * rp) (fma).
// q1 equals the IEEE divide x / s for every pair of fp32 significands (all
// 2^46, checked on the device), hence for all x, s whose intermediates stay
// normal, since each step scales exactly with powers of two of x and s.
__device__ __forceinline__ float markstein_quotient(float x, float s, float rp) {
  const float q0 = x * rp;
  const float e = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-e, rp, q0);
}

// s_waitcnt immediate that waits for every vector memory operation of the
// wave (vmcnt 0, the other counters at their no-wait maxima), in the gfx9
// encoding: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
constexpr int kWaitVmcnt0 = 0x0F70;

// True on every lane when some lane of the wave has `pred` set.
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b) {
  __bf16 x = (__bf16)a;
  __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(unsigned short, x) |
         ((uint32_t)__builtin_bit_cast(unsigned short, y) << 16);
}

// Wave-uniform value (the compiler can keep it in an SGPR).
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// Workgroup -> position in the buffer, XCD-aware.  The dispatcher deals
// workgroups to the 8 XCDs round-robin (workgroup b runs on XCD b % 8), so
// with the identity every XCD streams every 8th workgroup-sized piece.  With
// FP8Q_XCD_CHUNK = C > 0 each XCD takes C consecutive positions per round of
// 8C workgroups instead, so each XCD's L2 sees long contiguous runs while the
// chip's tiles in flight still form one window of 8C workgroups; C = -1 gives
// each XCD one contiguous eighth of the grid; 0 is the identity.  Either
// remap is a bijection on the whole rounds and the identity on the rest, so
// the last workgroup stays last.  On MI355X, C = 64 measured about 3% faster
// than the identity for the block quantize (1 MiB of bf16 per XCD run),
// 1.5% for the MXFP8 quantize and 2.5% for the dequantize, with the k-peer
// reduce unchanged; C = 4 and C = -1 were slower than the identity.
#ifndef FP8Q_XCD_CHUNK
#define FP8Q_XCD_CHUNK 64
#endif
template <int C = FP8Q_XCD_CHUNK>
__device__ __forceinline__ uint32_t block_position() {
  const uint32_t b = blockIdx.x, g = gridDim.x;
  if constexpr (C > 0) {
    constexpr uint32_t kRound = 8u * C;
    if (b >= g / kRound * kRound) return b;
    const uint32_t m = b % kRound;
    return b - m + (m % 8u) * C + m / 8u;
  } else if constexpr (C < 0) {
    const uint32_t whole = g / 8u * 8u;
    if (b >= whole) return b;
    return (b % 8u) * (whole / 8u) + b / 8u;
  } else {
    return b;
  }
}

// Global wave index and wave count of a 1-D launch of W-wave workgroups (the
// workgroup placed by block_position<C>).  W is the workgroup size every
// launcher here passes for its kernel, a compile-time constant, and no device
// code reads blockDim: the workgroup size is a 16-bit field of the implicit
// kernel arguments, which gfx950 reads with a vector load (there is no 16-bit
// scalar load), and since vector loads and stores share one in-order
// counter, waiting for that load also waits for every store the wave still
// has in flight.  On a loaded chip that held each wave of the block quantize
// for about 3 us after its last store, and with it the wave's slot.
template <int W, int C = FP8Q_XCD_CHUNK>
__device__ __forceinline__ uint32_t wave_index() {
  return uniform(block_position<C>() * (uint32_t)W + threadIdx.x / kWave);
}
template <int W>
__device__ __forceinline__ uint32_t wave_count() { return gridDim.x * (uint32_t)W; }

// Workgroup rounds for kernels that stage a per-tile output (block scales,
// E8M0 bytes) in LDS and write a workgroup's worth of it as one contiguous
// store.  The W-wave workgroup at position p (block_position<C>) takes the
// WT tiles from base = p * WT, then base += grid * WT while tiles remain; its
// wave w takes [base + wT, base + wT + T).  Per round: wave_tiles(t0, w) for
// each wave with tiles left, a barrier, flush(base, tiles in this round) by
// the whole workgroup, and, when another round follows, a second barrier
// before the staging array is reused.  Every wave of a workgroup runs the
// same number of rounds, so each barrier is reached by all of them.
template <int T, int W = 4, int C = FP8Q_XCD_CHUNK, typename WaveTiles, typename Flush>
__device__ __forceinline__ void workgroup_rounds(uint64_t full_tiles, WaveTiles &&wave_tiles,
                                                 Flush &&flush) {
  constexpr uint32_t kWgTiles = W * T;
  const uint32_t wid = uniform(threadIdx.x / kWave);
  const uint64_t stride = (uint64_t)gridDim.x * kWgTiles;
  for (uint64_t base = (uint64_t)block_position<C>() * kWgTiles; base < full_tiles;
       base += stride) {
    const uint64_t t0 = base + (uint64_t)wid * T;
    if (t0 < full_tiles) wave_tiles(t0, wid);
    __syncthreads();
    const uint64_t left = full_tiles - base;
    flush(base, left < kWgTiles ? (uint32_t)left : kWgTiles);
    if (base + stride < full_tiles) __syncthreads();
  }
}

}  // namespace fp8q
