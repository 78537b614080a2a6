// C-ABI entry points of libpagedkv: argument validation, workspace sizing,
// partition choice and dispatch to the kernels.  Contract: include/pa.h.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "pa_internal.h"

using pakv::DecodeArgs;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool debug_checks() {
  const char* v = getenv("PA_DEBUG");
  return v && v[0] && strcmp(v, "0") != 0;
}

bool pool_ok(const pa_pool* p) {
  if (!p || p->num_blocks <= 0 || p->block_size <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0)
    return false;
  if (p->dtype == PA_FP8_E4M3) return p->block_size % 4 == 0;  // whole scale groups
  return p->dtype == PA_F32 || p->dtype == PA_BF16;
}

// Bytes of one (block, kv head) region in the K buffer and in the V buffer;
// an 8-bit K region also carries the block's scales.
size_t region_bytes(const pa_pool* p, bool v_side) {
  const size_t B = (size_t)p->block_size, d = (size_t)p->head_dim;
  size_t r = B * d * (p->dtype == PA_F32 ? 4 : p->dtype == PA_BF16 ? 2 : 1);
  if (p->dtype == PA_FP8_E4M3 && !v_side) r += 4 * B;
  return r;
}

// An 8-bit pool in one buffer: the K and V regions of each (block, kv head)
// side by side, v_pool = k_pool + R_k.
bool side_by_side(const pa_pool* p, const void* k_pool, const void* v_pool) {
  return p->dtype == PA_FP8_E4M3 && k_pool &&
         static_cast<const uint8_t*>(v_pool) ==
             static_cast<const uint8_t*>(k_pool) + region_bytes(p, false);
}

// Bytes from one (block, kv head) region to the next in each buffer.
size_t region_stride(const pa_pool* p, const void* k_pool, const void* v_pool, bool v_side) {
  if (side_by_side(p, k_pool, v_pool)) return region_bytes(p, false) + region_bytes(p, true);
  return region_bytes(p, v_side);
}

// Bytes of one block (every kv head) in the K buffer and in the V buffer, as
// block copies and swaps move them: with side-by-side 8-bit regions the K
// buffer's block holds both, and nothing is left to move on the V side.
size_t block_bytes(const pa_pool* p, const void* k_pool, const void* v_pool, bool v_side) {
  if (side_by_side(p, k_pool, v_pool))
    return v_side ? 0 : (size_t)p->num_kv_heads * region_stride(p, k_pool, v_pool, false);
  return (size_t)p->num_kv_heads * region_bytes(p, v_side);
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Copy n device elements to a host vector on `stream` (debug validation only).
template <typename T>
bool fetch(std::vector<T>& dst, const T* src, size_t n, hipStream_t st) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, st) != hipSuccess)
    return false;
  return hipStreamSynchronize(st) == hipSuccess;
}

// Smallest piece a workgroup streams when the library chooses: 256 tokens
// (16 blocks), or for a short table its capacity in 32 pieces (whole
// blocks, at least one).  Ranges are normally much longer (the batch's
// blocks divided evenly over the grid); the floor only matters for small
// batches, where it bounds the number of partials -- and, set too high,
// crowds many short sequences into few ranges that each walk them one
// after another (256 one-token sequences: 42 us a call with a 256-token
// floor).
constexpr int32_t kDefaultMinPiece = 256;
constexpr int32_t kDefaultPiecesPerTable = 32;

int32_t default_piece(int64_t max_len, int32_t block_size) {
  int64_t p = (max_len + kDefaultPiecesPerTable - 1) / kDefaultPiecesPerTable;
  p = (p + block_size - 1) / block_size * block_size;
  return static_cast<int32_t>(std::min<int64_t>(kDefaultMinPiece, std::max<int64_t>(block_size, p)));
}

// Head slots of one partial row group: the query heads of one kv head, or
// with prefix groups as many members' heads as fill the 16-slot MFMA tile.
int32_t part_slots(int32_t group, bool grouped) {
  return grouped && group <= pakv::kMaxMfmaGroup ? (pakv::kMaxMfmaGroup / group) * group : group;
}

// Workspace layout: part_m, part_l [rows], part_o [rows][d] (fp32), then
// seg_info int32 [min(S, plan size)][4] and the reduce's list of sequences
// int32 [1 + min(S, plan size)][8] (a header, then one record each).  rows = 2 * waves of the grid *
// head slots (each (range, kv head) wave leaves at most two cut pieces);
// with prefix groups 2 * Hq more per sequence of one launch (segments that
// are not cut but still combine: a member's own blocks and its share of
// the group's blocks).
struct WsLayout {
  size_t rows, range_rows, off_l, off_o, off_info, off_list, bytes;
};

WsLayout ws_layout(const pa_pool* pool, int32_t S, int32_t Hq, bool grouped) {
  const int32_t G = Hq / pool->num_kv_heads;
  WsLayout w{};
  w.range_rows = (size_t)2 * pakv::decode_grid(pool->num_kv_heads) * pakv::kWaves *
                 std::max(part_slots(G, true), part_slots(G, false));
  w.rows = w.range_rows +
           (grouped ? (size_t)2 * std::min(S, pakv::kMaxPlanSeqs / 2) * Hq : 0);
  w.off_l = align_up(w.rows * sizeof(float));
  w.off_o = w.off_l + align_up(w.rows * sizeof(float));
  w.off_info = w.off_o + align_up(w.rows * pool->head_dim * sizeof(float));
  const size_t sx = (size_t)std::min(S, pakv::kMaxPlanSeqs);
  w.off_list = w.off_info + align_up(sx * 4 * sizeof(int32_t));
  w.bytes = w.off_list + align_up((sx + 1) * 8 * sizeof(int32_t));
  return w;
}

pa_status decode_sizes(const pa_pool* pool, int32_t S, int32_t Hq, int32_t maxB,
                       int32_t req_piece, bool grouped, int32_t* P_out, size_t* ws_out) {
  if (!pool_ok(pool) || S < 0 || Hq <= 0 || maxB <= 0) return PA_EINVAL;
  if (Hq % pool->num_kv_heads != 0) return PA_EINVAL;
  if (req_piece < 0 || (req_piece > 0 && req_piece % pool->block_size != 0)) return PA_EINVAL;
  if ((int64_t)maxB * pool->block_size > INT32_MAX) return PA_EINVAL;
  if (grouped && (int64_t)std::min(S, pakv::kMaxPlanSeqs / 2) * Hq * 2 > INT32_MAX / 4)
    return PA_EINVAL;
  const int64_t max_len = (int64_t)maxB * pool->block_size;
  *P_out = req_piece > 0 ? req_piece : default_piece(max_len, pool->block_size);
  *ws_out = S == 0 ? 0 : ws_layout(pool, S, Hq, grouped).bytes;
  return PA_OK;
}

// Prefix groups, validated on the host under PA_DEBUG: they partition the
// batch into runs of consecutive sequences, and group i's first
// shared_blocks[i] table entries are the same blocks in every member and
// full in every member.
pa_status check_groups(const pa_pool* pool, int32_t S, int32_t maxB, const int32_t* group_start,
                       const int32_t* shared_blocks, int32_t num_groups,
                       const std::vector<int32_t>& lens, const std::vector<int32_t>& tab,
                       hipStream_t st) {
  std::vector<int32_t> gs, sb;
  if (!fetch(gs, group_start, (size_t)num_groups + 1, st) ||
      !fetch(sb, shared_blocks, (size_t)num_groups, st))
    return PA_EHIP;
  if (gs[0] != 0 || gs[num_groups] != S) return PA_EINVAL;
  for (int32_t i = 0; i < num_groups; ++i) {
    if (gs[i + 1] <= gs[i] || sb[i] < 0 || sb[i] > maxB) return PA_EINVAL;
    for (int32_t m = gs[i]; m < gs[i + 1]; ++m) {
      if (sb[i] > lens[m] / pool->block_size) return PA_EINVAL;
      for (int32_t j = 0; j < sb[i]; ++j)
        if (tab[(size_t)m * maxB + j] != tab[(size_t)gs[i] * maxB + j]) return PA_EINVAL;
    }
  }
  return PA_OK;
}

// The decode entry points share this: validation, then the launch over a
// workspace of ws_bytes at ws.
// A decode step's extra inputs (pa_decode_step); all null for plain decode.
struct StepArgs {
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* new_blocks = nullptr;  // host memory, read during the call
  int32_t* tables_w = nullptr;
  int32_t* lens_out = nullptr;
};

pa_status decode_impl(const pa_pool* pool, const void* k_pool, const void* v_pool,
                      const void* q, int32_t num_seqs, int32_t num_q_heads,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, float scale, void* out,
                      int32_t partition_tokens, int32_t num_groups, const int32_t* group_start,
                      const int32_t* shared_blocks, void* workspace, size_t workspace_bytes,
                      bool debug, hipStream_t hs, const StepArgs& step = StepArgs{}) {
  int32_t P;
  size_t ws;
  if (num_groups < 0) return PA_EINVAL;
  pa_status st = decode_sizes(pool, num_seqs, num_q_heads, max_blocks_per_seq,
                              partition_tokens, num_groups > 0, &P, &ws);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (!k_pool || !v_pool || !q || !block_tables || !context_lens || !out) return PA_EINVAL;
  if (num_groups > 0 && (!group_start || !shared_blocks)) return PA_EINVAL;
  if (!(scale == scale) || scale == __builtin_huge_valf() || scale == -__builtin_huge_valf())
    return PA_EINVAL;
  const int group = num_q_heads / pool->num_kv_heads;
  if (pakv::decode_path(pool->dtype, pool->head_dim, group, pool->block_size) ==
      pakv::DecodePath::kUnsupported)
    return PA_EUNSUPPORTED;
  if (!workspace || workspace_bytes < ws) return PA_EINVAL;
  if (debug) {
    std::vector<int32_t> lens, tab, nbk;
    if (!fetch(lens, context_lens, (size_t)num_seqs, hs)) return PA_EHIP;
    if (!fetch(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, hs)) return PA_EHIP;
    const int64_t max_len = (int64_t)max_blocks_per_seq * pool->block_size;
    if (step.k_new) {
      // lengths after the step, and the given blocks in the tables
      nbk.assign(step.new_blocks, step.new_blocks + num_seqs);
      for (int32_t s = 0; s < num_seqs; ++s) {
        if (lens[s] < 0 || lens[s] >= max_len) return PA_EINVAL;
        if (nbk[s] >= pool->num_blocks) return PA_EINVAL;
        if (nbk[s] < 0 && lens[s] % pool->block_size == 0) return PA_EINVAL;  // needs a block
        if (nbk[s] >= 0) tab[(size_t)s * max_blocks_per_seq + lens[s] / pool->block_size] = nbk[s];
        lens[s] += 1;
      }
    }
    for (int32_t s = 0; s < num_seqs; ++s) {
      if (lens[s] < 1 || lens[s] > max_len) return PA_EINVAL;
      const int32_t nb = (lens[s] + pool->block_size - 1) / pool->block_size;
      for (int32_t j = 0; j < nb; ++j) {
        const int32_t b = tab[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= pool->num_blocks) return PA_EINVAL;
      }
    }
    if (num_groups > 0) {
      st = check_groups(pool, num_seqs, max_blocks_per_seq, group_start, shared_blocks,
                        num_groups, lens, tab, hs);
      if (st != PA_OK) return st;
    }
  }
  // prefix groups serve the MFMA kernels; a group that cannot share (fp32
  // pools, or more query heads per kv head than leave room for a second
  // member in the tile) reads its blocks per sequence, with the same result
  const bool grouped = num_groups > 0 && pool->dtype != PA_F32 &&
                       part_slots(group, true) >= 2 * group;
  const WsLayout L = ws_layout(pool, num_seqs, num_q_heads, grouped);
  DecodeArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_rstride = (int32_t)region_stride(pool, k_pool, v_pool, false);
  a.v_rstride = (int32_t)region_stride(pool, k_pool, v_pool, true);
  a.q = q;
  a.out = out;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.group_start = grouped ? group_start : nullptr;
  a.shared_blocks = grouped ? shared_blocks : nullptr;
  a.num_groups = grouped ? num_groups : 0;
  uint8_t* w = static_cast<uint8_t*>(workspace);
  a.part_m = reinterpret_cast<float*>(w);
  a.part_l = reinterpret_cast<float*>(w + L.off_l);
  a.part_o = reinterpret_cast<float*>(w + L.off_o);
  a.seg_info = reinterpret_cast<int32_t*>(w + L.off_info);
  a.cut_list = reinterpret_cast<int32_t*>(w + L.off_list);
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.min_seg_blocks = P / pool->block_size;
  a.slots = part_slots(group, grouped);
  a.own_row0 = static_cast<int32_t>(L.range_rows);
  a.sh_row0 = static_cast<int32_t>(L.range_rows + (L.rows - L.range_rows) / 2);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.k_new = step.k_new;
  a.v_new = step.v_new;
  a.tables_w = step.tables_w;
  a.lens_out = step.lens_out;
  hipError_t e = pakv::launch_decode(a, pool->dtype, pool->head_dim, group, pool->block_size, hs,
                                     step.new_blocks);
  return e == hipSuccess ? PA_OK : PA_EHIP;
}

// Fixed device scratch of pa_decode_noalloc (for callers that cannot
// allocate): the decode workspace, one copy per GPU, held until the process
// ends.  Host code never names it: each device's address comes from
// hipGetSymbolAddress, taken once per device.
constexpr size_t kScratchBytes = (size_t)18 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Address of this device's scratch (nullptr if the runtime refuses).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = p;
    else (void)hipGetLastError();
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_ENOMEM: return "block pool exhausted";
    case PA_EHIP: return "HIP runtime error";
    case PA_EUNSUPPORTED: return "unsupported shape";
    case PA_ESCRATCH: return "sizes exceed the fixed scratch of the no-allocation entry point";
  }
  return "unknown status";
}

const char* pa_version(void) { return "pagedkv 0.1 gfx950"; }

pa_status pa_kv_write(const pa_pool* pool, void* k_pool, void* v_pool, const void* k_new,
                      const void* v_new, const int64_t* slot_mapping, int32_t T,
                      void* stream) {
  if (!pool_ok(pool) || T < 0) return PA_EINVAL;
  if (T == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_EINVAL;
  hipStream_t st = as_stream(stream);
  if (debug_checks()) {
    std::vector<int64_t> s;
    if (!fetch(s, slot_mapping, (size_t)T, st)) return PA_EHIP;
    const int64_t nslots = (int64_t)pool->num_blocks * pool->block_size;
    std::vector<uint8_t> seen((size_t)nslots, 0);
    for (int64_t x : s) {
      if (x < 0) continue;
      if (x >= nslots || seen[(size_t)x]) return PA_EINVAL;
      seen[(size_t)x] = 1;
    }
  }
  hipError_t e = pakv::launch_kv_write(k_pool, v_pool, k_new, v_new, slot_mapping, T,
                                       pool->num_kv_heads, pool->block_size, pool->head_dim,
                                       pool->dtype, nullptr, 0, nullptr, nullptr,
                                       region_stride(pool, k_pool, v_pool, false),
                                       region_stride(pool, k_pool, v_pool, true), st);
  return e == hipSuccess ? PA_OK : PA_EHIP;
}

pa_status pa_kv_append(const pa_pool* pool, void* k_pool, void* v_pool, const void* k_new,
                       const void* v_new, const int64_t* slot_mapping, int32_t T,
                       int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_ids, const int32_t* positions, void* stream) {
  if (!pool_ok(pool) || T < 0 || max_blocks_per_seq <= 0) return PA_EINVAL;
  if (T == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping || !block_tables || !seq_ids ||
      !positions)
    return PA_EINVAL;
  hipStream_t st = as_stream(stream);
  if (debug_checks()) {
    std::vector<int64_t> sl;
    std::vector<int32_t> sq, ps;
    if (!fetch(sl, slot_mapping, (size_t)T, st) || !fetch(sq, seq_ids, (size_t)T, st) ||
        !fetch(ps, positions, (size_t)T, st))
      return PA_EHIP;
    const int64_t nslots = (int64_t)pool->num_blocks * pool->block_size;
    std::vector<uint8_t> seen((size_t)nslots, 0);
    for (int32_t i = 0; i < T; ++i) {
      const int64_t x = sl[i];
      if (x < 0) continue;
      if (x >= nslots || seen[(size_t)x]) return PA_EINVAL;
      seen[(size_t)x] = 1;
      if (sq[i] < 0 || ps[i] < 0 || ps[i] / pool->block_size >= max_blocks_per_seq)
        return PA_EINVAL;
    }
  }
  hipError_t e = pakv::launch_kv_write(k_pool, v_pool, k_new, v_new, slot_mapping, T,
                                       pool->num_kv_heads, pool->block_size, pool->head_dim,
                                       pool->dtype, block_tables,
                                       max_blocks_per_seq, seq_ids, positions,
                                       region_stride(pool, k_pool, v_pool, false),
                                       region_stride(pool, k_pool, v_pool, true), st);
  return e == hipSuccess ? PA_OK : PA_EHIP;
}

size_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_blocks_per_seq, int32_t partition_tokens) {
  int32_t P;
  size_t ws;
  if (decode_sizes(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, false, &P,
                   &ws) != PA_OK)
    return 0;
  return ws;
}

size_t pa_decode_shared_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_blocks_per_seq,
                                        int32_t partition_tokens) {
  int32_t P;
  size_t ws;
  if (decode_sizes(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, true, &P,
                   &ws) != PA_OK)
    return 0;
  return ws;
}

int32_t pa_decode_piece_tokens(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_blocks_per_seq, int32_t partition_tokens,
                               int64_t total_blocks) {
  int32_t P;
  size_t ws;
  if (total_blocks < 0 || decode_sizes(pool, num_seqs, num_q_heads, max_blocks_per_seq,
                                       partition_tokens, false, &P, &ws) != PA_OK)
    return 0;
  // as the plan computes it: R ranges per kv head over the launch's waves,
  // every sequence taken as one segment with its start cost
  const int64_t R = std::max<int64_t>(
      1, (int64_t)pakv::decode_grid(pool->num_kv_heads) * pakv::kWaves / pool->num_kv_heads);
  const int64_t cs = (pool->dtype == PA_FP8_E4M3 ? 2 : 1) * pakv::kSegStartBlocks;
  const int64_t places = total_blocks + cs * num_seqs;
  const int64_t q = std::max<int64_t>(P / pool->block_size, (places + R - 1) / R);
  return q * pool->block_size > INT32_MAX ? 0 : static_cast<int32_t>(q * pool->block_size);
}

int32_t pa_decode_partition_tokens(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_blocks_per_seq, int32_t partition_tokens) {
  int32_t P;
  size_t ws;
  if (decode_sizes(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, false, &P,
                   &ws) != PA_OK)
    return 0;
  return P;
}

pa_status pa_decode(const pa_pool* pool, const void* k_pool, const void* v_pool,
                    const void* q, int32_t num_seqs, int32_t num_q_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, float scale, void* out,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_impl(pool, k_pool, v_pool, q, num_seqs, num_q_heads, block_tables,
                     max_blocks_per_seq, context_lens, scale, out, partition_tokens, 0, nullptr,
                     nullptr, workspace, workspace_bytes, debug_checks(), as_stream(stream));
}

pa_status pa_decode_shared(const pa_pool* pool, const void* k_pool, const void* v_pool,
                           const void* q, int32_t num_seqs, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, float scale, void* out,
                           int32_t partition_tokens, int32_t num_groups,
                           const int32_t* group_start, const int32_t* shared_blocks,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(pool, k_pool, v_pool, q, num_seqs, num_q_heads, block_tables,
                     max_blocks_per_seq, context_lens, scale, out, partition_tokens, num_groups,
                     group_start, shared_blocks, workspace, workspace_bytes, debug_checks(),
                     as_stream(stream));
}

pa_status pa_decode_step(const pa_pool* pool, void* k_pool, void* v_pool, const void* q,
                         const void* k_new, const void* v_new, int32_t num_seqs,
                         int32_t num_q_heads, int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* lens_in, int32_t* lens_out, const int32_t* new_blocks,
                         float scale, void* out, int32_t partition_tokens, int32_t num_groups,
                         const int32_t* group_start, const int32_t* shared_blocks,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!pool_ok(pool)) return PA_EINVAL;
  if (num_seqs > 0 && (!k_new || !v_new || !lens_in || !lens_out || !new_blocks))
    return PA_EINVAL;
  if (lens_out == lens_in && num_seqs > 0) return PA_EINVAL;
  // bf16 and 8-bit pools (an 8-bit step quantises the new token as the
  // slot write does); fp32 pools take pa_kv_append and pa_decode
  if (pool->dtype != PA_BF16 && pool->dtype != PA_FP8_E4M3) return PA_EUNSUPPORTED;
  StepArgs step;
  step.k_new = k_new;
  step.v_new = v_new;
  step.new_blocks = new_blocks;
  step.tables_w = block_tables;
  step.lens_out = lens_out;
  return decode_impl(pool, k_pool, v_pool, q, num_seqs, num_q_heads, block_tables,
                     max_blocks_per_seq, lens_in, scale, out, partition_tokens, num_groups,
                     group_start, shared_blocks, workspace, workspace_bytes, debug_checks(),
                     as_stream(stream), step);
}

size_t pa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

pa_status pa_decode_noalloc(const pa_pool* pool, const void* k_pool, const void* v_pool,
                            const void* q, int32_t num_seqs, int32_t num_q_heads,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, float scale, void* out,
                            int32_t partition_tokens, void* stream) {
  int32_t P;
  size_t ws;
  const pa_status st = decode_sizes(pool, num_seqs, num_q_heads, max_blocks_per_seq,
                                    partition_tokens, false, &P, &ws);
  if (st != PA_OK) return st;
  if (ws > kScratchBytes) return PA_ESCRATCH;
  if (num_seqs == 0) return PA_OK;
  void* ptr = scratch_ptr();
  if (!ptr) return PA_EHIP;
  // no host-side validation copy here (it would synchronize the stream)
  return decode_impl(pool, k_pool, v_pool, q, num_seqs, num_q_heads, block_tables,
                     max_blocks_per_seq, context_lens, scale, out, partition_tokens, 0, nullptr,
                     nullptr, ptr, kScratchBytes, false, as_stream(stream));
}

size_t pa_extend_workspace_bytes(const pa_pool* pool, int32_t total_q, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_blocks_per_seq) {
  if (!pool_ok(pool) || total_q <= 0 || num_seqs <= 0 || num_q_heads <= 0 ||
      max_blocks_per_seq <= 0 || num_q_heads % pool->num_kv_heads != 0)
    return 0;
  const int splits = pakv::extend_splits(total_q, num_q_heads, pool->num_kv_heads,
                                         max_blocks_per_seq, pool->head_dim);
  return pakv::extend_workspace_bytes(total_q, num_q_heads, splits, pool->head_dim);
}

pa_status pa_extend(const pa_pool* pool, const void* k_pool, const void* v_pool,
                    const void* q, int32_t total_q, const int32_t* q_start, int32_t num_seqs,
                    int32_t num_q_heads, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, float scale,
                    void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!pool_ok(pool) || num_seqs < 0 || total_q < 0 || num_q_heads <= 0 ||
      max_blocks_per_seq <= 0)
    return PA_EINVAL;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_EINVAL;
  if ((int64_t)max_blocks_per_seq * pool->block_size > INT32_MAX) return PA_EINVAL;
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!k_pool || !v_pool || !q || !q_start || !block_tables || !context_lens || !out)
    return PA_EINVAL;
  if (!(scale == scale) || scale == __builtin_huge_valf() || scale == -__builtin_huge_valf())
    return PA_EINVAL;
  const int group = num_q_heads / pool->num_kv_heads;
  if (!pakv::extend_supported(pool->dtype, pool->head_dim, group, pool->block_size))
    return PA_EUNSUPPORTED;
  hipStream_t hs = as_stream(stream);
  if (debug_checks()) {
    std::vector<int32_t> qs, lens, tab;
    if (!fetch(qs, q_start, (size_t)num_seqs + 1, hs) ||
        !fetch(lens, context_lens, (size_t)num_seqs, hs) ||
        !fetch(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, hs))
      return PA_EHIP;
    if (qs[0] != 0 || qs[num_seqs] != total_q) return PA_EINVAL;
    const int64_t max_len = (int64_t)max_blocks_per_seq * pool->block_size;
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t n = qs[s + 1] - qs[s];
      if (n < 0 || (n > 0 && (lens[s] < n || lens[s] > max_len))) return PA_EINVAL;
      const int32_t nb = n > 0 ? (lens[s] + pool->block_size - 1) / pool->block_size : 0;
      for (int32_t j = 0; j < nb; ++j) {
        const int32_t b = tab[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= pool->num_blocks) return PA_EINVAL;
      }
    }
  }
  pakv::ExtendArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.q = q;
  a.out = out;
  a.q_start = q_start;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.total_q = total_q;
  // the library's split, or none when the workspace cannot hold it
  a.splits = pakv::extend_splits(total_q, num_q_heads, pool->num_kv_heads, max_blocks_per_seq,
                                 pool->head_dim);
  const size_t need = pakv::extend_workspace_bytes(total_q, num_q_heads, a.splits, pool->head_dim);
  if (a.splits > 1 && (!workspace || workspace_bytes < need)) a.splits = 1;
  if (a.splits > 1) {
    const size_t n = (size_t)total_q * num_q_heads * a.splits;
    uint8_t* w = static_cast<uint8_t*>(workspace);
    a.part_m = reinterpret_cast<float*>(w);
    a.part_l = reinterpret_cast<float*>(w + align_up(n * sizeof(float)));
    a.part_o = reinterpret_cast<float*>(w + 2 * align_up(n * sizeof(float)));
  }
  hipError_t e = pakv::launch_extend(a, pool->head_dim, group, hs);
  return e == hipSuccess ? PA_OK : PA_EHIP;
}

pa_status pa_block_copy(const pa_pool* pool, void* k_pool, void* v_pool, const int32_t* pairs,
                        int32_t num_pairs, void* stream) {
  if (!pool_ok(pool) || num_pairs < 0) return PA_EINVAL;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !pairs) return PA_EINVAL;
  hipStream_t st = as_stream(stream);
  if (debug_checks()) {
    std::vector<int32_t> pr;
    if (!fetch(pr, pairs, (size_t)num_pairs * 2, st)) return PA_EHIP;
    std::vector<uint8_t> is_src((size_t)pool->num_blocks, 0), is_dst((size_t)pool->num_blocks, 0);
    for (int32_t p = 0; p < num_pairs; ++p) {
      const int32_t s = pr[2 * p], d = pr[2 * p + 1];
      if (s < 0 || s >= pool->num_blocks || d < 0 || d >= pool->num_blocks || s == d)
        return PA_EINVAL;
      if (is_dst[(size_t)d]) return PA_EINVAL;
      is_dst[(size_t)d] = 1;
      is_src[(size_t)s] = 1;
    }
    for (int32_t b = 0; b < pool->num_blocks; ++b)
      if (is_src[(size_t)b] && is_dst[(size_t)b]) return PA_EINVAL;
  }
  hipError_t e = pakv::launch_block_copy(k_pool, v_pool, pairs, num_pairs,
                                         block_bytes(pool, k_pool, v_pool, false),
                                         block_bytes(pool, k_pool, v_pool, true), st);
  return e == hipSuccess ? PA_OK : PA_EHIP;
}

pa_status pa_block_swap(const pa_pool* pool, void* k_pool, void* v_pool, void* host_k,
                        void* host_v, int32_t num_host_blocks, const int32_t* pairs,
                        int32_t num_pairs, pa_swap_dir dir, void* stream) {
  if (!pool_ok(pool) || num_pairs < 0 || num_host_blocks < 0) return PA_EINVAL;
  if (dir != PA_SWAP_OUT && dir != PA_SWAP_IN) return PA_EINVAL;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !host_k || !host_v || !pairs || num_host_blocks == 0)
    return PA_EINVAL;
  // the kernel reaches host memory through its device mapping; memory that is
  // not pinned host memory has none, and is refused before any launch
  void* dk = nullptr;
  void* dv = nullptr;
  if (hipHostGetDevicePointer(&dk, host_k, 0) != hipSuccess || !dk ||
      hipHostGetDevicePointer(&dv, host_v, 0) != hipSuccess || !dv) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return PA_EINVAL;
  }
  hipStream_t st = as_stream(stream);
  const int32_t n_src = dir == PA_SWAP_OUT ? pool->num_blocks : num_host_blocks;
  const int32_t n_dst = dir == PA_SWAP_OUT ? num_host_blocks : pool->num_blocks;
  if (debug_checks()) {
    std::vector<int32_t> pr;
    if (!fetch(pr, pairs, (size_t)num_pairs * 2, st)) return PA_EHIP;
    std::vector<uint8_t> seen((size_t)n_dst, 0);
    for (int32_t p = 0; p < num_pairs; ++p) {
      const int32_t s = pr[2 * p], d = pr[2 * p + 1];
      if (s < 0 || s >= n_src || d < 0 || d >= n_dst || seen[(size_t)d]) return PA_EINVAL;
      seen[(size_t)d] = 1;
    }
  }
  // host buffers take the device pools' layout: side-by-side 8-bit regions
  // in one host buffer too
  if (side_by_side(pool, k_pool, v_pool) != side_by_side(pool, host_k, host_v)) return PA_EINVAL;
  const size_t kb = block_bytes(pool, k_pool, v_pool, false);
  const size_t vb = block_bytes(pool, k_pool, v_pool, true);
  hipError_t e = dir == PA_SWAP_OUT
                     ? pakv::launch_block_move(k_pool, v_pool, dk, dv, pairs, num_pairs, kb, vb, st)
                     : pakv::launch_block_move(dk, dv, k_pool, v_pool, pairs, num_pairs, kb, vb, st);
  return e == hipSuccess ? PA_OK : PA_EHIP;
}

pa_status pa_table_update(int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t block_size, const int32_t* seq_ids, const int32_t* positions,
                          const int64_t* slot_mapping, int32_t T, void* stream) {
  if (max_blocks_per_seq <= 0 || block_size <= 0 || T < 0) return PA_EINVAL;
  if (T == 0) return PA_OK;
  if (!block_tables || !seq_ids || !positions || !slot_mapping) return PA_EINVAL;
  hipStream_t st = as_stream(stream);
  if (debug_checks()) {
    std::vector<int32_t> sq, ps;
    std::vector<int64_t> sl;
    if (!fetch(sq, seq_ids, (size_t)T, st) || !fetch(ps, positions, (size_t)T, st) ||
        !fetch(sl, slot_mapping, (size_t)T, st))
      return PA_EHIP;
    for (int32_t i = 0; i < T; ++i) {
      if (sl[i] < 0) continue;
      if (sq[i] < 0 || ps[i] < 0 || ps[i] / block_size >= max_blocks_per_seq) return PA_EINVAL;
    }
  }
  hipError_t e = pakv::launch_table_update(block_tables, max_blocks_per_seq, block_size,
                                           seq_ids, positions, slot_mapping, T, st);
  return e == hipSuccess ? PA_OK : PA_EHIP;
}

}  // extern "C"
