// Device helpers shared by the attention kernels (decode and extend):
// vector types, streaming loads, lane exchanges, workgroup scans, the
// register ring that keeps block loads in flight, and the lazy-softmax
// constant.  gfx950 (wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "pa_internal.h"

namespace pakv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// P.V on v_mfma_f32_16x16x32_bf16 with P carried to about 16 significant
// bits: the instruction's 32-long k runs over a lane's four tokens twice.
// In A (p_split) the first four entries are the high bf16 part of each
// probability (truncation), the last four the residual p - high rounded to
// nearest even; in B (v_twice) the same four V values appear twice.  A and B
// place their entries at the same k, so the sum is (high + low) . V.
__device__ __forceinline__ bf16x8 p_split(const float (&p)[4]) {
  uint32_t pb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pb[r] = __float_as_uint(p[r]);
  const bf16x2 lo01 = {static_cast<__bf16>(p[0] - bf16_hi(pb[0])),
                       static_cast<__bf16>(p[1] - bf16_hi(pb[1]))};
  const bf16x2 lo23 = {static_cast<__bf16>(p[2] - bf16_hi(pb[2])),
                       static_cast<__bf16>(p[3] - bf16_hi(pb[3]))};
  return __builtin_bit_cast(
      bf16x8, u32x4{(pb[0] >> 16) | (pb[1] & 0xffff0000u), (pb[2] >> 16) | (pb[3] & 0xffff0000u),
                    __builtin_bit_cast(uint32_t, lo01), __builtin_bit_cast(uint32_t, lo23)});
}
__device__ __forceinline__ bf16x8 v_twice(u32x2 v) {
  return __builtin_bit_cast(bf16x8, u32x4{v.x, v.y, v.x, v.y});
}

// Global-memory (address space 1) byte pointer.
typedef const uint8_t __attribute__((address_space(1)))* gptr;

template <typename V>
__device__ __forceinline__ V ldg_stream(gptr p) {
  typedef const V __attribute__((address_space(1)))* vptr;
#if PA_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<vptr>(p));
#else
  return *reinterpret_cast<vptr>(p);
#endif
}

// A load that leaves its lines to the caches' normal policy: used where the
// other half of the lines is read by the next tile (V rows of 32-token
// blocks), which a non-temporal load would make HBM fetch again.
template <typename V>
__device__ __forceinline__ V ldg_keep(gptr p) {
  typedef const V __attribute__((address_space(1)))* vptr;
  return *reinterpret_cast<vptr>(p);
}

// V loads of a tile: non-temporal unless the tile reads half of each row.
template <int B, typename V>
__device__ __forceinline__ V ldg_v(gptr p) {
  if constexpr (B > 16) return ldg_keep<V>(p);
  else return ldg_stream<V>(p);
}

// A generic pointer known to point into global memory, as a global pointer.
__device__ __forceinline__ gptr to_global(const uint8_t* p) {
  return reinterpret_cast<gptr>(reinterpret_cast<uint64_t>(p));
}

// A global pointer that is the same in every lane, moved to SGPRs so that
// loads can take the scalar-base + 32-bit-vector-offset form.
__device__ __forceinline__ gptr uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gptr>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1]; row rotate right by 4, 8.
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Reductions across the four 16-lane rows of a wave, on the VALU.
// v_permlane32_swap(x, x) returns x with rows {2,3} replaced by rows {0,1}
// and x with rows {0,1} replaced by rows {2,3}: in every lane the pair is
// x[i] and x[i ^ 32] in some order.  v_permlane16_swap(x, x) does the same
// for odd and even rows: x[i] and x[i ^ 16].  Max and sum are symmetric, so
// combining the pair reduces over the partner lane.  (An exchange through
// the LDS unit would wait behind every LDS access in flight.)
__device__ __forceinline__ float max_xor32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float lane_bcast(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  x = fmaxf(x, dpp<kRowRor4>(x));
  x = fmaxf(x, dpp<kRowRor8>(x));
  return max_xor32(max_xor16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  return sum_xor32(sum_xor16(x));
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(void* out, size_t idx, float v) {
  static_cast<float*>(out)[idx] = v;
}
template <>
__device__ __forceinline__ void store_out<__bf16>(void* out, size_t idx, float v) {
  static_cast<__bf16*>(out)[idx] = static_cast<__bf16>(v);  // v_cvt_pk_bf16_f32, RNE
}

// Inclusive scan of one value per lane over a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute((lane - d) << 2, v);
    if (lane >= d) v += y;
  }
  return v;
}

// Exclusive scan of one value per thread over the workgroup (at most 8
// waves: wsum holds one partial sum per wave).
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) off += wsum[w];
    tot += wsum[w];
  }
  *total = tot;
  __syncthreads();
  return off + inc - v;
}
static_assert(kWaves >= 1 && kWaves <= 8, "the plan scan keeps one sum per wave, 8 at most");

// Online softmax with a lazy reference: probabilities are 2^(x - m_ref) for a
// per-head reference m_ref that only moves when some head's block maximum
// exceeds it by more than kSlack (log2 units).  Until then the accumulators
// need no rescaling; probabilities stay below 2^kSlack, far from fp32 range
// limits, and the final (or split) normalisation divides the reference out
// exactly as it would a running maximum.
constexpr float kSlack = 8.f;

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Software pipeline over `cnt` blocks with a ring of NBUF register buffers:
// load(i, slot) issues block i's loads into ring slot `slot`; compute(i, slot)
// consumes it.  NBUF - 1 blocks are in flight while one is consumed.  The
// steady-state loop issues a load at every step, so the wait before each
// compute only covers the oldest buffer; the drain (at most 2*NBUF - 2
// blocks) is separate code, so its shorter waits do not leak into the loop.
// The prologue clamps its block indices so that it is unconditional (a unit
// shorter than the ring re-reads its last block into unused slots).  `pre`
// runs while the prologue's loads are in flight.
template <int NBUF, typename LoadF, typename ComputeF, typename PreF>
__device__ __forceinline__ void block_ring(int cnt, LoadF&& load, ComputeF&& compute, PreF&& pre) {
  static_for<NBUF - 1>([&](auto b) { load(min((int)b, cnt - 1), b); });
  pre();
  int i = 0;
  for (; i + 2 * NBUF - 2 < cnt; i += NBUF) {
    static_for<NBUF>([&](auto b) {
      load(i + b + NBUF - 1, std::integral_constant<int, (b + NBUF - 1) % NBUF>{});
      compute(i + b, b);
    });
  }
  static_for<2 * NBUF - 2>([&](auto b) {
    if (i + b < cnt) {
      if (i + b + NBUF - 1 < cnt)
        load(i + b + NBUF - 1, std::integral_constant<int, (b + NBUF - 1) % NBUF>{});
      compute(i + b, std::integral_constant<int, b % NBUF>{});
    }
  });
}
template <int NBUF, typename LoadF, typename ComputeF>
__device__ __forceinline__ void block_ring(int cnt, LoadF&& load, ComputeF&& compute) {
  block_ring<NBUF>(cnt, load, compute, [] {});
}

}  // namespace
}  // namespace pakv
