// Internal launch interface between the C-ABI layer (pa_api.hip) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pakv {

// Compile-time tuning knobs of the decode kernels; the defaults are the
// values measured fastest on MI355X.
#ifndef PA_WAVES
#define PA_WAVES 4   // waves per decode workgroup (one kv head each)
#endif
#ifndef PA_NBUF
#define PA_NBUF 2    // register buffers per wave: blocks in flight = PA_NBUF - 1
#endif
#ifndef PA_MFMA_MIN_WG
#define PA_MFMA_MIN_WG 2  // MFMA decode: workgroups per CU the register budget must allow
#endif
#ifndef PA_NBUF8
#define PA_NBUF8 4   // register buffers per wave for 8-bit pools (half the bytes per block)
#endif
#ifndef PA_NT_LOADS
#define PA_NT_LOADS 1  // 1: K/V loads carry the non-temporal hint
#endif

constexpr int kBlock = 16;       // tokens per block of the fp32 decode (MFMA paths: 8, 16, 32)
constexpr int kWaves = PA_WAVES;
constexpr int kNBuf = PA_NBUF;
constexpr int kNBuf8 = PA_NBUF8;
constexpr int kMaxMfmaGroup = 16;
constexpr int kMaxSlots = 1 << 20;  // partial slots per (sequence, head)
constexpr int kMaxPlanSeqs = 4096;  // sequences per decode launch (LDS work plan)

struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  void* out;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_m;       // [S][Hq][max_slots]    reference max, log2 units
  float* part_l;       // [S][Hq][max_slots]    sum of exp2(score - m)
  float* part_o;       // [S][Hq][max_slots][D] unnormalised output
  int32_t* seg_count;  // [S] pieces each sequence was cut into
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t min_seg_blocks;  // smallest range a workgroup streams (blocks)
  int32_t max_slots;       // partial slots per (sequence, query head)
  float scale_log2;  // scale * log2(e): scores are kept in log2 units
};

// Multi-token (extend / chunked prefill) attention over paged contexts.
struct ExtendArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;               // [total_q][Hq][D] bf16
  void* out;                   // [total_q][Hq][D] bf16
  const int32_t* q_start;      // [S + 1] first query row of each sequence
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  float scale_log2;
};

// Supported: bf16 pools, 16-token blocks, head_dim 64 / 128, group <= 16.
bool extend_supported(pa_dtype dtype, int head_dim, int group, int block_size);
hipError_t launch_extend(const ExtendArgs& a, int head_dim, int group, hipStream_t stream);

// Which decode kernel family handles a shape.
enum class DecodePath { kUnsupported, kValu, kMfma, kMfma8 };
DecodePath decode_path(pa_dtype dtype, int head_dim, int group, int block_size);

hipError_t launch_decode(const DecodeArgs& a, pa_dtype dtype, int head_dim, int group,
                         int block_size,
                         hipStream_t stream);

// block_tables == nullptr: no table update (plain slot write).  For
// PA_FP8_E4M3 pools k_new / v_new are bf16 and are quantised.
hipError_t launch_kv_write(void* k_pool, void* v_pool, const void* k_new,
                           const void* v_new, const int64_t* slots, int32_t T,
                           int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                           pa_dtype dtype, int32_t* block_tables, int32_t max_blocks,
                           const int32_t* seq_ids, const int32_t* positions,
                           hipStream_t stream);

hipError_t launch_block_copy(void* k_pool, void* v_pool, const int32_t* pairs,
                             int32_t num_pairs, size_t k_block_bytes, size_t v_block_bytes,
                             hipStream_t stream);

// Copy whole blocks between two pool pairs (device and host-mapped):
// dst_*[pairs[i][1]] <- src_*[pairs[i][0]].
hipError_t launch_block_move(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                             const int32_t* pairs, int32_t num_pairs, size_t k_block_bytes,
                             size_t v_block_bytes, hipStream_t stream);

hipError_t launch_table_update(int32_t* block_tables, int32_t max_blocks,
                               int32_t block_size, const int32_t* seq_ids,
                               const int32_t* positions, const int64_t* slots, int32_t T,
                               hipStream_t stream);

}  // namespace pakv
