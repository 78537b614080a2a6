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
constexpr int kMaxMfmaGroup = 16;   // head slots of one MFMA tile
constexpr int kMaxPlanSeqs = 4096;  // sequences per decode launch (LDS work plan; 2048 with groups)
// The decode plan's start cost of a segment, in blocks of a bf16 or fp32
// pool (twice as many for an 8-bit pool): a range cut of the batch counts
// each non-empty segment this much longer than its blocks.
#ifndef PA_SEG_START_BLOCKS
#define PA_SEG_START_BLOCKS 2
#endif
constexpr int kSegStartBlocks = PA_SEG_START_BLOCKS;

// Work is cut into "segments": the part of one sequence it streams alone, or
// the full blocks at the head of a prefix group's tables, which every member
// shares and which one wave streams once for all of them (each member's
// query heads take their own head slots of the MFMA tile).  Without groups a
// segment is a whole sequence.
struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  void* out;
  const int32_t* block_tables;
  const int32_t* context_lens;
  // Prefix groups (nullptr: none).  Group i is the consecutive sequences
  // group_start[i] .. group_start[i+1] - 1, whose first shared_blocks[i]
  // table entries name the same physical blocks, all full.
  const int32_t* group_start;   // [num_groups + 1]
  const int32_t* shared_blocks; // [num_groups]
  int32_t num_groups;
  int32_t seq_base;             // index of this launch's first sequence in the groups
  // Split-context partials.  A segment cut by range boundaries leaves one
  // row per (wave slot, end, head slot): a wave slot is (range r, kv head g)
  // = r * num_kv_heads + g; `end` is 0 for the piece that starts at the
  // range's first block and 1 for the range's last piece when that starts
  // later, so each (range, head) holds at most two cut pieces and these
  // rows are sized by the grid, not by the batch.  With prefix groups a
  // segment that is not cut still leaves a partial (a member's result
  // combines its own blocks' and the shared blocks'): row own_row0 + s * Hq
  // + h for sequence s's own segment, sh_row0 + s * Hq + h for its share of
  // the group's shared segment.
  float* part_m;       // [rows]    reference max, log2 units
  float* part_l;       // [rows]    sum of exp2(score - m)
  float* part_o;       // [rows][D] unnormalised output
  int32_t* seg_info;   // [S][4] where each sequence's pieces went (reduce input)
  int32_t* cut_list;   // [1 + S][8] count, then {s, seg_info[s]} of the sequences the reduce combines
  // A decode step (pa_decode_step; k_new == nullptr: plain decode): each
  // sequence's new token sits at position context_lens[s] (the lengths
  // before the step), its K/V rows are k_new/v_new [S][Hkv][D] (bf16) and
  // its block comes with the launch (StepBlocks).  The step stores the
  // token, writes the table entry of a given block, and writes the lengths
  // after the step to lens_out.
  const void* k_new;
  const void* v_new;
  int32_t* tables_w;
  int32_t* lens_out;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t min_seg_blocks;  // smallest range a wave streams (blocks)
  int32_t decode_wgs;      // workgroups of the decode grid (a step adds store workgroups)
  int32_t slots;           // head slots per (wave slot, end): G, or members * G with groups
  int32_t kv_div;          // fp32 path: head groups per pool kv head (0 or 1: one); with
                           // more, num_kv_heads counts the groups of at most 4 query heads
  int32_t own_row0;        // first per-sequence row of own segments (groups only)
  int32_t sh_row0;         // first per-sequence row of shared segments (groups only)
  float scale_log2;  // scale * log2(e): scores are kept in log2 units
  // 8-bit pools: bytes from one (block, kv head) region to the next in
  // k_pool and in v_pool -- R_k and R_v for two buffers, R_k + R_v for both
  // when the regions sit side by side in one buffer
  int32_t k_rstride;
  int32_t v_rstride;
};

// The block of each sequence's new token in a decode step (-1: the table's
// tail entry), passed by value with the launch: the host's array reaches
// the kernel with its arguments, with no copy of its own and no read of
// host memory from the kernel.  A step launch covers at most kStepSeqs
// sequences.
constexpr int kStepSeqs = 512;
struct StepBlocks {
  int32_t blk[kStepSeqs];
};

// Workgroups of a decode launch for this many kv heads (a persistent grid:
// one per CU, at least one wave per kv head); partial rows are bounded by
// 2 * grid * kWaves * slots.
int decode_grid(int num_kv_heads);

// Multi-token (extend / chunked prefill) attention over paged contexts.
struct ExtendArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;               // [total_q][Hq][D] bf16
  void* out;                   // [total_q][Hq][D] bf16
  const int32_t* q_start;      // [S + 1] first query row of each sequence
  const int32_t* block_tables;
  const int32_t* context_lens;
  // Context split: each sequence's context is cut into `splits` chunks
  // (whole 64-token stages); with more than one, every (query, head) row
  // leaves one (m, l, o) partial per chunk and a second kernel combines them.
  float* part_m;               // [total_q][Hq][splits] reference max, log2 units
  float* part_l;               // [total_q][Hq][splits]
  float* part_o;               // [total_q][Hq][splits][D] unnormalised output
  int32_t splits;
  int32_t total_q;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  float scale_log2;
};

// Supported: bf16 pools, 16-token blocks, head_dim 64 / 128, group <= 16.
bool extend_supported(pa_dtype dtype, int head_dim, int group, int block_size);
// How many chunks the library cuts each context into for this batch (1: no
// split), and the workspace that needs.
int extend_splits(int total_q, int num_q_heads, int num_kv_heads, int max_blocks, int head_dim);
size_t extend_workspace_bytes(int total_q, int num_q_heads, int splits, int head_dim);
hipError_t launch_extend(const ExtendArgs& a, int head_dim, int group, hipStream_t stream);

// Which decode kernel family handles a shape.
enum class DecodePath { kUnsupported, kValu, kMfma, kMfma8 };
DecodePath decode_path(pa_dtype dtype, int head_dim, int group, int block_size);

// host_new_blocks: a decode step's new blocks (host memory, [num_seqs]),
// read during the call; nullptr for plain decode.
hipError_t launch_decode(const DecodeArgs& a, pa_dtype dtype, int head_dim, int group,
                         int block_size, hipStream_t stream,
                         const int32_t* host_new_blocks = nullptr);

// block_tables == nullptr: no table update (plain slot write).  For
// PA_FP8_E4M3 pools k_new / v_new are bf16 and are quantised.
// k_rstride / v_rstride: 8-bit pools' region strides (as in DecodeArgs).
hipError_t launch_kv_write(void* k_pool, void* v_pool, const void* k_new,
                           const void* v_new, const int64_t* slots, int32_t T,
                           int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                           pa_dtype dtype, int32_t* block_tables, int32_t max_blocks,
                           const int32_t* seq_ids, const int32_t* positions,
                           size_t k_rstride, size_t v_rstride, hipStream_t stream);

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
