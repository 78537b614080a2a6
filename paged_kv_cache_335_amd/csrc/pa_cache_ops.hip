// Cache-maintenance kernels: slot write, copy-on-write block copy and the
// device-side table update.  All are bitwise data movement.
//
//  * Slot write ("Dynamic Growth" on the glossary page; "Add pages as the
//    request grows" on the attention-lab page): token i's K row for kv head g
//    goes to k_pool[b][g][r][:], its V row to v_pool[b][g][:][r], with
//    b = slot / block_size, r = slot % block_size.
//  * Block copy ("The bonus contiguous storage can't give you: sharing" on
//    the vLLM KV-cache page; "Shared blocks and copy-on-write" on the
//    attention-lab page): the whole of block src, every kv head and slot, is
//    copied to block dst in both pools.
//  * Table update: the block-table entry covering a written token's logical
//    position takes the block the token went to.  The append entry point
//    runs it inside the slot-write launch.
//  * 8-bit slot write (a quantized cache, vLLM post "Where it bites"): each
//    (token, kv head) row of K and of V is quantised on its own to OCP E4M3
//    codes with one scale, scale = bf16(max |x| / 448), code = x / scale
//    rounded to nearest even.  Not bitwise: the one kernel here with
//    arithmetic.
#include <algorithm>

#include "pa_internal.h"

namespace pakv {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Pool stores carry the non-temporal hint.  Decode streams the pool with
// non-temporal loads, and lines left dirty in a cache by ordinary stores made
// the next decode measurably slower (about 5% after a 256-token slot write
// into the blocks it reads); stored non-temporally they cost nothing.
template <typename T>
__device__ __forceinline__ void st_pool(T* dst, T v) {
  __builtin_nontemporal_store(v, dst);
}

constexpr int kThreads = 256;

// Optional table growth done by the slot-write launch (append = table
// update + slot write in one kernel).  tables == nullptr: no table update.
struct TableArgs {
  int32_t* tables;
  int32_t max_blocks;
  const int32_t* seq_ids;
  const int32_t* positions;
};

// Table entry of token i (thread 0 of token i's workgroup).
__device__ __forceinline__ void update_table(const TableArgs& ta, int i, int64_t blk,
                                             int block_size) {
  if (ta.tables != nullptr && threadIdx.x == 0)
    ta.tables[(size_t)ta.seq_ids[i] * ta.max_blocks + ta.positions[i] / block_size] =
        static_cast<int32_t>(blk);
}

// One workgroup per new token.
template <typename E>
__global__ __launch_bounds__(kThreads) void kv_write_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int64_t* __restrict__ slots, int32_t num_kv_heads, int32_t block_size,
    int32_t head_dim, TableArgs ta) {
  const int i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0) return;
  const int64_t blk = slot / block_size;
  update_table(ta, i, blk, block_size);
  const int r = static_cast<int>(slot % block_size);
  constexpr int ES = sizeof(E);
  const size_t row_bytes = (size_t)head_dim * ES;
  const size_t tok_bytes = (size_t)num_kv_heads * row_bytes;
  const size_t blk_bytes = tok_bytes * block_size;
  const uint8_t* ksrc = k_new + (size_t)i * tok_bytes;
  const uint8_t* vsrc = v_new + (size_t)i * tok_bytes;
  // K: each kv head's row is contiguous at [blk][g][r][:]
  if (row_bytes % 16 == 0) {
    const int n16 = static_cast<int>(tok_bytes / 16);
    const int per_row = static_cast<int>(row_bytes / 16);
    for (int c = threadIdx.x; c < n16; c += kThreads) {
      const int g = c / per_row, off = (c % per_row) * 16;
      uint8_t* dst = k_pool + blk * blk_bytes + ((size_t)g * block_size + r) * row_bytes + off;
      st_pool(reinterpret_cast<u32x4*>(dst), *reinterpret_cast<const u32x4*>(ksrc + (size_t)c * 16));
    }
  } else {
    const int n = num_kv_heads * head_dim;
    for (int c = threadIdx.x; c < n; c += kThreads) {
      const int g = c / head_dim, d = c % head_dim;
      E* dst = reinterpret_cast<E*>(k_pool + blk * blk_bytes +
                                    ((size_t)g * block_size + r) * row_bytes) + d;
      st_pool(dst, reinterpret_cast<const E*>(ksrc)[c]);
    }
  }
  // V: dim-major, element (g, d) at [blk][g][d][r]
  const int n = num_kv_heads * head_dim;
  for (int c = threadIdx.x; c < n; c += kThreads) {
    const int g = c / head_dim, d = c % head_dim;
    E* dst = reinterpret_cast<E*>(v_pool + blk * blk_bytes) +
             ((size_t)g * head_dim + d) * block_size + r;
    st_pool(dst, reinterpret_cast<const E*>(vsrc)[c]);
  }
}

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// E4M3 code of x (|x| within the finite range), nearest even: the gfx950
// packed fp32 -> OCP fp8 conversion, low byte.
__device__ __forceinline__ uint8_t to_e4m3(float x) {
  return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xffu);
}

// 8-bit slot write: one workgroup per new token, one wave per (kv head,
// K or V) row at a time.  K region of (block b, kv head g): [B*d codes,
// token-major r*d + e][scale groups: per 4 slots, 4 K then 4 V bf16 scales];
// V region: [B*d codes, dim-major e*B + r].  Region (b, g) starts at
// (b * H + g) * k_rstride in k_pool and at (b * H + g) * v_rstride in
// v_pool (the two strides are equal when K and V regions alternate in one
// buffer, with v_pool = k_pool + R_k).
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int64_t* __restrict__ slots, int32_t num_kv_heads, int32_t block_size,
    int32_t head_dim, size_t k_rstride, size_t v_rstride, TableArgs ta) {
  const int i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0) return;
  const int64_t blk = slot / block_size;
  update_table(ta, i, blk, block_size);
  const int r = static_cast<int>(slot % block_size);
  const int B = block_size, d = head_dim;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int row = wave; row < 2 * num_kv_heads; row += kThreads / 64) {
    const bool is_v = row >= num_kv_heads;
    const int g = is_v ? row - num_kv_heads : row;
    const uint16_t* src = (is_v ? v_new : k_new) + ((size_t)i * num_kv_heads + g) * d;
    uint8_t* kreg = k_pool + ((size_t)blk * num_kv_heads + g) * k_rstride;
    uint8_t* vreg = v_pool + ((size_t)blk * num_kv_heads + g) * v_rstride;
    float amax = 0.f;  // NaN inputs are skipped by fmaxf
    for (int e = lane; e < d; e += 64)
      amax = fmaxf(amax, fabsf(__uint_as_float((uint32_t)src[e] << 16)));
    amax = wave_max64(amax);
    // scale = amax / 448 (IEEE division), rounded to bf16 (v_cvt_pk_bf16_f32, RNE)
    const __bf16 sb = static_cast<__bf16>(amax / 448.f);
    const float scale = static_cast<float>(sb);
    for (int e = lane; e < d; e += 64) {
      const float x = __uint_as_float((uint32_t)src[e] << 16);
      const uint8_t c = scale > 0.f ? to_e4m3(x / scale) : uint8_t{0};
      if (is_v)
        st_pool(vreg + (size_t)e * B + r, c);
      else
        st_pool(kreg + (size_t)r * d + e, c);
    }
    if (lane == 0)
      st_pool(reinterpret_cast<uint16_t*>(kreg + (size_t)B * d + 16u * (r / 4) + 8u * is_v) +
                  (r % 4),
              __builtin_bit_cast(uint16_t, sb));
  }
}

// grid (num_pairs, 2): y = 0 copies the K block, y = 1 the V block.
__global__ __launch_bounds__(kThreads) void block_copy16_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const int32_t* __restrict__ pairs, size_t k_bytes, size_t v_bytes) {
  const int p = blockIdx.x;
  uint8_t* pool = blockIdx.y == 0 ? k_pool : v_pool;
  const size_t block_bytes = blockIdx.y == 0 ? k_bytes : v_bytes;
  const size_t src = (size_t)pairs[2 * p] * block_bytes;
  const size_t dst = (size_t)pairs[2 * p + 1] * block_bytes;
  const size_t n16 = block_bytes / 16;
  for (size_t c = threadIdx.x; c < n16; c += kThreads)
    st_pool(reinterpret_cast<u32x4*>(pool + dst + c * 16),
            *reinterpret_cast<const u32x4*>(pool + src + c * 16));
}

__global__ __launch_bounds__(kThreads) void block_copy_bytes_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const int32_t* __restrict__ pairs, size_t k_bytes, size_t v_bytes) {
  const int p = blockIdx.x;
  uint8_t* pool = blockIdx.y == 0 ? k_pool : v_pool;
  const size_t block_bytes = blockIdx.y == 0 ? k_bytes : v_bytes;
  const size_t src = (size_t)pairs[2 * p] * block_bytes;
  const size_t dst = (size_t)pairs[2 * p + 1] * block_bytes;
  for (size_t c = threadIdx.x; c < block_bytes; c += kThreads) st_pool(pool + dst + c, pool[src + c]);
}

// Block move between different buffers (device pool <-> host-mapped pool):
// grid (num_pairs, 2, chunks); y = 0 moves K, y = 1 V; z splits a block into
// chunks so that enough 16-byte requests are in flight over the host link.
__global__ __launch_bounds__(kThreads) void block_move16_kernel(
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v,
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v, const int32_t* __restrict__ pairs,
    size_t k_bytes, size_t v_bytes) {
  const int p = blockIdx.x;
  const bool is_v = blockIdx.y == 1;
  const size_t bytes = is_v ? v_bytes : k_bytes;
  const uint8_t* src = (is_v ? src_v : src_k) + (size_t)pairs[2 * p] * bytes;
  uint8_t* dst = (is_v ? dst_v : dst_k) + (size_t)pairs[2 * p + 1] * bytes;
  const size_t n16 = bytes / 16;
  for (size_t c = (size_t)blockIdx.z * kThreads + threadIdx.x; c < n16;
       c += (size_t)gridDim.z * kThreads)
    st_pool(reinterpret_cast<u32x4*>(dst + c * 16), *reinterpret_cast<const u32x4*>(src + c * 16));
}

__global__ __launch_bounds__(kThreads) void block_move_bytes_kernel(
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v,
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v, const int32_t* __restrict__ pairs,
    size_t k_bytes, size_t v_bytes) {
  const int p = blockIdx.x;
  const bool is_v = blockIdx.y == 1;
  const size_t bytes = is_v ? v_bytes : k_bytes;
  const uint8_t* src = (is_v ? src_v : src_k) + (size_t)pairs[2 * p] * bytes;
  uint8_t* dst = (is_v ? dst_v : dst_k) + (size_t)pairs[2 * p + 1] * bytes;
  for (size_t c = (size_t)blockIdx.z * kThreads + threadIdx.x; c < bytes;
       c += (size_t)gridDim.z * kThreads)
    st_pool(dst + c, src[c]);
}

__global__ __launch_bounds__(kThreads) void table_update_kernel(
    int32_t* __restrict__ tables, int32_t max_blocks, int32_t block_size,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions,
    const int64_t* __restrict__ slots, int32_t T) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= T) return;
  const int64_t slot = slots[i];
  if (slot < 0) return;
  tables[(size_t)seq_ids[i] * max_blocks + positions[i] / block_size] =
      static_cast<int32_t>(slot / block_size);
}

}  // namespace

hipError_t launch_kv_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int64_t* slots, int32_t T, int32_t num_kv_heads,
                           int32_t block_size, int32_t head_dim, pa_dtype dtype,
                           int32_t* block_tables, int32_t max_blocks, const int32_t* seq_ids,
                           const int32_t* positions, size_t k_rstride, size_t v_rstride,
                           hipStream_t st) {
  if (T <= 0) return hipSuccess;
  auto kp = static_cast<uint8_t*>(k_pool);
  auto vp = static_cast<uint8_t*>(v_pool);
  auto kn = static_cast<const uint8_t*>(k_new);
  auto vn = static_cast<const uint8_t*>(v_new);
  const TableArgs ta{block_tables, max_blocks, seq_ids, positions};
  if (dtype == PA_FP8_E4M3)
    kv_write_fp8_kernel<<<T, kThreads, 0, st>>>(kp, vp, static_cast<const uint16_t*>(k_new),
                                                static_cast<const uint16_t*>(v_new), slots,
                                                num_kv_heads, block_size, head_dim, k_rstride,
                                                v_rstride, ta);
  else if (dtype == PA_BF16)
    kv_write_kernel<uint16_t><<<T, kThreads, 0, st>>>(kp, vp, kn, vn, slots, num_kv_heads,
                                                      block_size, head_dim, ta);
  else
    kv_write_kernel<uint32_t><<<T, kThreads, 0, st>>>(kp, vp, kn, vn, slots, num_kv_heads,
                                                      block_size, head_dim, ta);
  return hipGetLastError();
}

hipError_t launch_block_copy(void* k_pool, void* v_pool, const int32_t* pairs,
                             int32_t num_pairs, size_t k_bytes, size_t v_bytes,
                             hipStream_t st) {
  if (num_pairs <= 0) return hipSuccess;
  const dim3 grid(num_pairs, 2);
  auto kp = static_cast<uint8_t*>(k_pool);
  auto vp = static_cast<uint8_t*>(v_pool);
  if (k_bytes % 16 == 0 && v_bytes % 16 == 0)
    block_copy16_kernel<<<grid, kThreads, 0, st>>>(kp, vp, pairs, k_bytes, v_bytes);
  else
    block_copy_bytes_kernel<<<grid, kThreads, 0, st>>>(kp, vp, pairs, k_bytes, v_bytes);
  return hipGetLastError();
}

hipError_t launch_block_move(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                             const int32_t* pairs, int32_t num_pairs, size_t k_bytes,
                             size_t v_bytes, hipStream_t st) {
  if (num_pairs <= 0) return hipSuccess;
  // chunks of 4 KiB per workgroup pass, at most 8 workgroups per block
  const size_t big = k_bytes > v_bytes ? k_bytes : v_bytes;
  const unsigned chunks = (unsigned)std::min<size_t>(8, (big + 4095) / 4096);
  const dim3 grid(num_pairs, 2, chunks);
  auto sk = static_cast<const uint8_t*>(src_k);
  auto sv = static_cast<const uint8_t*>(src_v);
  auto dk = static_cast<uint8_t*>(dst_k);
  auto dv = static_cast<uint8_t*>(dst_v);
  if (k_bytes % 16 == 0 && v_bytes % 16 == 0)
    block_move16_kernel<<<grid, kThreads, 0, st>>>(sk, sv, dk, dv, pairs, k_bytes, v_bytes);
  else
    block_move_bytes_kernel<<<grid, kThreads, 0, st>>>(sk, sv, dk, dv, pairs, k_bytes, v_bytes);
  return hipGetLastError();
}

hipError_t launch_table_update(int32_t* block_tables, int32_t max_blocks, int32_t block_size,
                               const int32_t* seq_ids, const int32_t* positions,
                               const int64_t* slots, int32_t T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  table_update_kernel<<<(T + kThreads - 1) / kThreads, kThreads, 0, st>>>(
      block_tables, max_blocks, block_size, seq_ids, positions, slots, T);
  return hipGetLastError();
}

}  // namespace pakv
