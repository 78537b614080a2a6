/*
 * pa.h - paged KV-cache kernels for one AMD Instinct MI355X (gfx950).
 *
 * The method (as the pages describe it):
 *  - "How PagedAttention Powers vLLM's KV Cache", section "PagedAttention:
 *    paging, borrowed from the operating system": keys and values live in
 *    fixed-size blocks of a shared physical pool; each sequence's block table
 *    maps its logical block j to the physical block holding it.
 *  - same page, section "The attention kernel has to read scattered blocks":
 *    decode attention walks the table and gathers K/V block by block.
 *  - attention-lab "PagedAttention" page, reference entry "How it works" and
 *    widget "Measure memory use across requests": the attention equation is
 *    unchanged, softmax(scale * q K^T) V over the logical sequence.
 *  - same page, reference entry "Shared blocks and copy-on-write": a request
 *    about to modify a shared block first gets a private copy.
 *  - vLLM post, section "Where it bites": a quantized cache shrinks each
 *    token's footprint and stacks with paging (PA_FP8_E4M3 below).
 *
 * Conventions for every entry point below:
 *  - Pointers named *_pool, q, out, block_tables, context_lens, slot_mapping,
 *    pairs, k_new, v_new, workspace and the table-update arrays are DEVICE
 *    pointers; `pool` points to a HOST struct.  The caller owns all memory;
 *    the library allocates no device memory.
 *  - `stream` is a hipStream_t passed as void* (NULL: the default stream).
 *    Work is enqueued asynchronously on it; no call synchronizes, except that
 *    with the environment variable PA_DEBUG=1 the device-resident indices are
 *    copied to the host on `stream` and validated first (synchronizing).
 *  - Host-visible arguments are validated before anything is launched; a bad
 *    one returns PA_EINVAL (or PA_EUNSUPPORTED for a valid but unimplemented
 *    shape) and has no effect.  Device-resident indices (tables, lengths,
 *    slots, pairs) are trusted unless PA_DEBUG=1.  A failed launch returns
 *    PA_EHIP.
 *  - Calls that touch the same buffers must be ordered by the caller (same
 *    stream or events).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_EINVAL = 1,        /* bad argument; nothing was done                  */
  PA_ENOMEM = 2,        /* block pool exhausted (block manager only)       */
  PA_EHIP = 3,          /* a HIP runtime call or kernel launch failed      */
  PA_EUNSUPPORTED = 4,  /* valid arguments, shape not implemented          */
  PA_ESCRATCH = 5       /* pa_decode_noalloc: sizes exceed its fixed scratch */
} pa_status;

typedef enum {
  PA_F32 = 0,       /* IEEE fp32 elements                                        */
  PA_BF16 = 1,      /* bf16 elements                                             */
  PA_FP8_E4M3 = 2   /* 8-bit cache: OCP E4M3 codes + one bf16 scale per token    */
} pa_dtype;

/*
 * Pool geometry.  Two separate device buffers hold the pool:
 *   k_pool: [num_blocks][num_kv_heads][block_size][head_dim]   token-major
 *   v_pool: [num_blocks][num_kv_heads][head_dim][block_size]   dim-major
 * so one (block, kv head) is one contiguous run of block_size*head_dim
 * elements in each buffer.  V is dim-major so that decode can reduce over
 * tokens inside each lane (the reduction dimension of P.V).  The pages leave
 * the physical layout open.
 *
 * PA_FP8_E4M3 pools hold E4M3 codes and one bf16 scale per (token slot,
 * kv head, side).  Per (block, kv head):
 *   k_pool region, R_k = block_size*head_dim + 4*block_size bytes: the K
 *       codes token-major [block_size][head_dim], then the scales: for each
 *       group of 4 token slots, their 4 K scales then their 4 V scales
 *       (bf16, 16 bytes per group);
 *   v_pool region, R_v = block_size*head_dim bytes: the V codes dim-major
 *       [head_dim][block_size].
 * Buffer layouts [num_blocks][num_kv_heads][R_k] and [..][R_v].  A stored
 * element's value is e4m3(code) * scale of its slot and side; the V scales
 * live with the K codes so that one 16-byte read fetches both scales of
 * four tokens.  For this dtype q, out, k_new and v_new are bf16.  The slot
 * write quantises each new (token, kv head) row x of K and of V on its own:
 * scale = max_i |x_i| / 448 in fp32, rounded to bf16 (nearest even), and
 * code_i = x_i / scale in fp32 rounded to the nearest E4M3 value, ties to
 * even (all codes 0 when the scale is 0).  E4M3 (OCP 8-bit floating point):
 * sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals, largest
 * finite 448, S.1111.111 NaN, no infinities.
 */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;    /* tokens per block; decode: 8, 16 or 32 (fp32: 16) */
  int32_t num_kv_heads;
  int32_t head_dim;      /* decode and extend: 64 or 128 */
  pa_dtype dtype;        /* element type of both pools (PA_FP8_E4M3: regions) */
} pa_pool;

/*
 * Slot write: store each new token's keys and values in the slot the block
 * manager gave it ("Dynamic Growth" on the glossary page; "Add pages as the
 * request grows" on the attention-lab page).
 *   k_new, v_new: [T][num_kv_heads][head_dim], pool dtype (bf16 for an
 *                 8-bit pool, stored quantised as described above), dense.
 *   slot_mapping: int64 [T]; slot = block * block_size + offset; a negative
 *                 slot skips that token.  Slots must be distinct (a repeated
 *                 slot is a write race) and below num_blocks * block_size.
 * Every other byte of the pools is left unchanged.  T = 0 is a no-op.
 */
pa_status pa_kv_write(const pa_pool* pool, void* k_pool, void* v_pool,
                      const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int32_t T, void* stream);

/*
 * Bytes of device workspace pa_decode (and pa_decode_shared) need for these
 * sizes: per-piece partials and per-sequence piece locations.  The partials
 * are bounded by the launch grid, not by the batch or the table width: each
 * (range, kv head) wave of the persistent grid leaves at most two cut
 * pieces, so for 256 CUs, 128-dim heads and 4 query heads per kv head about
 * 17 MB, and 4 KiB more per 256 sequences (at most 64 KiB).  Returns 0 for
 * num_seqs = 0 and for invalid arguments; pa_decode reports those.
 */
size_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 int32_t partition_tokens);

/*
 * The smallest piece (tokens) pa_decode cuts a sequence into for these
 * arguments; equal to partition_tokens when that is non-zero.  0 on invalid
 * arguments.
 */
int32_t pa_decode_partition_tokens(const pa_pool* pool, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_blocks_per_seq,
                                   int32_t partition_tokens);

/*
 * The length (tokens) of the ranges pa_decode cuts a batch of total_blocks
 * blocks into (all sequences of one launch of at most 4096, with the
 * launch grid of the current device): at least partition_tokens (or the
 * library's choice), and long enough that the ranges of one kv head cover
 * the batch with one range per wave, each sequence counted a few blocks
 * longer than it is (the plan's start cost of a piece).  A sequence of L
 * tokens is then cut into about L / this pieces.  For reports; 0 on
 * invalid arguments.
 */
int32_t pa_decode_piece_tokens(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_blocks_per_seq, int32_t partition_tokens,
                               int64_t total_blocks);

/*
 * Paged decode attention: for every sequence s and query head h, with
 * g = h / (num_q_heads / num_kv_heads) and L = context_lens[s],
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t) V_t,   t in [0, L),
 * where token t is read from physical block block_tables[s][t / block_size],
 * slot t % block_size, KV head g.  Accumulation is in fp32.
 *   q, out:        [num_seqs][num_q_heads][head_dim], pool dtype (bf16 for
 *                  an 8-bit pool); out is rounded to nearest even when bf16.
 *   block_tables:  int32 [num_seqs][max_blocks_per_seq], entries in
 *                  [0, num_blocks); entries at j >= ceil(L / block_size) are
 *                  never read.
 *   context_lens:  int32 [num_seqs], 1 <= L <= max_blocks_per_seq*block_size.
 *   partition_tokens: smallest piece of a sequence one workgroup streams
 *                  (0: the library's choice, 256 tokens, or less for a
 *                  table shorter than 8192 tokens: its capacity
 *                  max_blocks_per_seq * block_size in 32 pieces, rounded up
 *                  to whole blocks); otherwise a positive multiple of
 *                  block_size.  The work is split by
 *                  blocks, not by sequence: for each kv head the batch's
 *                  blocks, sequence after sequence, are cut into equal
 *                  contiguous ranges, each streamed by one wave of a grid
 *                  that fills the chip (a workgroup's waves take
 *                  consecutive (kv head, range) pairs), each range at least
 *                  partition_tokens long.  A sequence cut by range boundaries is processed in
 *                  pieces whose (max, sum-exp, unnormalised output) partials
 *                  go to `workspace` and are combined by a second kernel.
 *   workspace:     device buffer of at least pa_decode_workspace_bytes(...)
 *                  bytes; contents on entry are irrelevant.
 * Requires num_q_heads % num_kv_heads == 0, head_dim 64 or 128 and at most
 * 16 query heads per kv head; bf16 and 8-bit pools: block_size 8, 16 or 32;
 * fp32 pools: block_size 16 (PA_EUNSUPPORTED otherwise).  fp32 pools with
 * more than 4 query heads per kv head stream each kv head's blocks once per
 * group of up to 4 of its query heads.  The result does not depend on where blocks
 * sit in the pool, and two calls with the same inputs give identical bits.
 */
pa_status pa_decode(const pa_pool* pool, const void* k_pool, const void* v_pool,
                    const void* q, int32_t num_seqs, int32_t num_q_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, float scale, void* out,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * pa_decode over prefix groups: sequences that share the blocks of a common
 * prefix (vLLM post, "The bonus contiguous storage can't give you: sharing":
 * parallel samples of one prompt point their tables at the same physical
 * blocks; glossary entry, "Sampling Algorithms": the shared prompt's pages
 * are stored once and not recomputed).  Each shared block is streamed from
 * HBM once for all of its group's members, whose query heads fill the head
 * slots of one MFMA tile; each member's remaining blocks are read as in
 * pa_decode, and the two parts combine through the split-context partials.
 * The result is the same attention as pa_decode's (up to the order of fp32
 * sums).
 *   group_start:   int32 [num_groups + 1], device: the groups partition the
 *                  batch into runs of consecutive sequences, group i being
 *                  sequences group_start[i] .. group_start[i+1] - 1
 *                  (group_start[0] = 0, strictly increasing,
 *                  group_start[num_groups] = num_seqs).
 *   shared_blocks: int32 [num_groups], device: the first shared_blocks[i]
 *                  table entries of every member of group i name the same
 *                  physical blocks, and each of those blocks is full (below
 *                  every member's context length).  0: nothing shared.
 * pa_bm_prefix_groups produces both.  A group shares only when its members'
 * query heads fit one tile (members * heads per kv head <= 16) and the pool
 * is bf16 or 8-bit; otherwise its blocks are read per sequence.
 * num_groups = 0 is pa_decode.  The workspace must hold at least
 * pa_decode_shared_workspace_bytes(...) bytes (contents on entry are
 * irrelevant).  With
 * PA_DEBUG=1 the groups are validated too (PA_EINVAL if they break the
 * rules above).
 */
pa_status pa_decode_shared(const pa_pool* pool, const void* k_pool, const void* v_pool,
                           const void* q, int32_t num_seqs, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, float scale, void* out,
                           int32_t partition_tokens, int32_t num_groups,
                           const int32_t* group_start, const int32_t* shared_blocks,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step in one launch: each sequence's new token is stored in its
 * slot, its block table grows, and decode attention runs over every context
 * including the new token (glossary entry, "Dynamic Growth": the cache grows
 * a token at a time; vLLM post, "PagedAttention: paging, borrowed from the
 * operating system": a sequence that fills its last block takes a new one
 * and appends it to its table).  The same result as pa_kv_append of the
 * new tokens (with their table entries) followed by pa_decode_shared (or
 * pa_decode) over the grown contexts, up to the order of fp32 sums.
 *   q, out:       [num_seqs][num_q_heads][head_dim] bf16.
 *   k_new, v_new: [num_seqs][num_kv_heads][head_dim] bf16, device: the new
 *                 token of sequence s, at position lens_in[s].  An 8-bit
 *                 pool receives its codes and scales exactly as from
 *                 pa_kv_write, and the decode uses those quantised values.
 *   lens_in:      int32 [num_seqs], device: context lengths before the
 *                 step, 0 <= lens_in[s] < max_blocks_per_seq * block_size.
 *   lens_out:     int32 [num_seqs], device, not lens_in: receives
 *                 lens_in[s] + 1.
 *   new_blocks:   int32 [num_seqs], HOST memory, read during the call (it
 *                 travels with the kernel arguments, so the step needs no
 *                 copy of its own): the block holding the new token when
 *                 the block manager gave one -- a new block (lens_in[s] a
 *                 multiple of block_size) or a private copy of a shared
 *                 tail (after pa_block_copy) -- else -1 (the token goes to
 *                 the block block_tables[s][lens_in[s] / block_size]).
 *                 Batches of more than 512 sequences run as several
 *                 launches of at most 512.
 *   block_tables: as for pa_decode; the entry of every given block is
 *                 written (block_tables[s][lens_in[s] / block_size] =
 *                 new_blocks[s]).
 *   groups, workspace: as for pa_decode_shared (num_groups = 0: none; the
 *                 groups describe the contexts after the step).
 * bf16 and 8-bit pools (fp32 pools: PA_EUNSUPPORTED, use pa_kv_append and
 * pa_decode).  With PA_DEBUG=1 the lengths, blocks and tables are validated
 * first, as for pa_decode after the step.
 */
pa_status pa_decode_step(const pa_pool* pool, void* k_pool, void* v_pool, const void* q,
                         const void* k_new, const void* v_new, int32_t num_seqs,
                         int32_t num_q_heads, int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* lens_in, int32_t* lens_out, const int32_t* new_blocks,
                         float scale, void* out, int32_t partition_tokens, int32_t num_groups,
                         const int32_t* group_start, const int32_t* shared_blocks,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace pa_decode_shared needs: pa_decode's, plus two
 * partial rows (fp32 max, sum and head_dim outputs) per query head of each
 * sequence of one launch (up to 2048 sequences), since a grouped sequence's
 * own blocks and its share of the group's blocks always combine.  0 for
 * num_seqs = 0 and for invalid arguments.
 */
size_t pa_decode_shared_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_blocks_per_seq,
                                        int32_t partition_tokens);

/*
 * pa_decode without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Arguments and
 * result as for pa_decode.  The workspace is a fixed device array inside
 * the library, pa_decode_noalloc_max_bytes() bytes per GPU, taken when the
 * library's code is loaded on that GPU and held until the process ends;
 * its address is looked up on the first call on each device.  Sizes whose
 * pa_decode_workspace_bytes exceeds it return PA_ESCRATCH (nothing is
 * launched).  Every call on one GPU uses that GPU's array: calls that
 * overlap on one GPU (different streams, no ordering) race and give wrong
 * results; calls ordered on one stream are fine.  Nothing in the array
 * needs to start at zero (every word the second kernel reads is written by
 * the first in the same call).  PA_DEBUG=1 validation is not done here (it
 * would copy to the host and synchronize).
 */
pa_status pa_decode_noalloc(const pa_pool* pool, const void* k_pool, const void* v_pool,
                            const void* q, int32_t num_seqs, int32_t num_q_heads,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, float scale, void* out,
                            int32_t partition_tokens, void* stream);

/* Bytes of the fixed scratch array of pa_decode_noalloc. */
size_t pa_decode_noalloc_max_bytes(void);

/*
 * Multi-token paged attention: extend / chunked prefill over a paged prefix
 * with a causal mask (glossary entry, "Complex Attention Patterns" and
 * "Dynamic Growth": attention reads the cache through the block table
 * whatever the logical order, and new tokens are appended on demand).
 * Sequence s brings n_s = q_start[s+1] - q_start[s] new query tokens, rows
 * q_start[s] .. q_start[s+1] - 1 of q; their K/V are already in the cache
 * (pa_kv_write first), so context_lens[s] = L_s counts them and n_s <= L_s.
 * Query j of sequence s is at position p = L_s - n_s + j and attends to the
 * sequence's tokens 0..p:
 *   out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . K_t) V_t,
 * with K_t, V_t read as in pa_decode (kv head h / (num_q_heads / H_kv)).
 *   q, out:      [total_q][num_q_heads][head_dim] bf16, total_q = q_start[S].
 *   q_start:     int32 [num_seqs + 1], q_start[0] = 0, non-decreasing;
 *                sequences with no queries are allowed.
 *   block_tables, context_lens: as for pa_decode.
 *   workspace:   device buffer of pa_extend_workspace_bytes(...) bytes for a
 *                batch too small to fill the chip: each sequence's context is
 *                then cut into chunks streamed in parallel, whose partial
 *                (max, sum-exp, unnormalised output) rows a second kernel
 *                combines.  NULL, or fewer bytes: no split (the same result,
 *                on fewer workgroups).  Contents on entry are irrelevant.
 * Requires bf16 pools, block_size 16, head_dim 64 or 128 and at most 16
 * query heads per kv head (PA_EUNSUPPORTED otherwise).
 * With PA_DEBUG=1, q_start, lengths and table entries are validated first.
 */
pa_status pa_extend(const pa_pool* pool, const void* k_pool, const void* v_pool,
                    const void* q, int32_t total_q, const int32_t* q_start, int32_t num_seqs,
                    int32_t num_q_heads, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, float scale,
                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace pa_extend uses to split the contexts of a batch of
 * total_q query rows over num_seqs sequences (0: the batch fills the chip
 * without a split, or invalid arguments).  The split is chosen from these
 * sizes and the device: when the batch's workgroup units (8 waves of two
 * 16-row tiles of one sequence and kv head) number fewer than the grid's
 * workgroups (one per CU), each context is cut into up to 32 chunks of
 * equal token count (at least 1024 tokens); the partials take total_q *
 * num_q_heads * chunks * (head_dim + 2) fp32 values.
 */
size_t pa_extend_workspace_bytes(const pa_pool* pool, int32_t total_q, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_blocks_per_seq);

/*
 * Copy-on-write block copy ("The bonus contiguous storage can't give you:
 * sharing" on the vLLM KV-cache page; "Shared blocks and copy-on-write" on
 * the attention-lab page): for each (src, dst) pair, every KV head and slot
 * of block src is copied bit for bit to block dst, in both pools (for an
 * 8-bit pool: the whole K region, codes and scales, and the V region).
 *   pairs: int32 [num_pairs][2] = (src, dst), both in [0, num_blocks).
 *          Destinations must be distinct and no destination may also be a
 *          source in the same call (the copies run concurrently).
 * num_pairs = 0 is a no-op.
 */
pa_status pa_block_copy(const pa_pool* pool, void* k_pool, void* v_pool,
                        const int32_t* pairs, int32_t num_pairs, void* stream);

/*
 * Block swap between the device pools and host memory (preemption by
 * swapping, vLLM post "Where it bites"; glossary entry "Flexible
 * Management": pages can be swapped out, spilling to CPU RAM).
 *   host_k, host_v: caller-owned PINNED host buffers (hipHostMalloc, or a
 *       pinned torch tensor) of num_host_blocks blocks each, laid out like
 *       k_pool / v_pool (same bytes per block); host pointers.
 *   pairs: int32 [num_pairs][2] = (src, dst), device-accessible memory:
 *       PA_SWAP_OUT copies device block src to host block dst,
 *       PA_SWAP_IN copies host block src to device block dst, bitwise,
 *       every kv head and slot of K and of V.  Destinations must be
 *       distinct; src in [0, num_blocks) and dst in [0, num_host_blocks) for
 *       SWAP_OUT, the other way round for SWAP_IN.
 * One launch on `stream` moves every pair over the host link.  PA_EINVAL if
 * the host buffers are not pinned host memory; nothing is launched then.
 * num_pairs = 0 is a no-op.
 */
typedef enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 } pa_swap_dir;

pa_status pa_block_swap(const pa_pool* pool, void* k_pool, void* v_pool, void* host_k,
                        void* host_v, int32_t num_host_blocks, const int32_t* pairs,
                        int32_t num_pairs, pa_swap_dir dir, void* stream);

/*
 * Device-side mirror of table growth ("PagedAttention: paging, borrowed from
 * the operating system": a growing sequence appends an entry to its block
 * table).  For every i with slot_mapping[i] >= 0:
 *   block_tables[seq_ids[i] * max_blocks_per_seq + positions[i] / block_size]
 *       = slot_mapping[i] / block_size,
 * i.e. the entry covering the token's logical position now names the block
 * the token was written to (a new block, or a private copy after
 * copy-on-write).  seq_ids, positions: int32 [T]; slot_mapping: int64 [T].
 * positions[i] / block_size must be below max_blocks_per_seq.  Tokens of one
 * sequence that land in one block write the same value.  T = 0 is a no-op.
 */
pa_status pa_table_update(int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t block_size, const int32_t* seq_ids,
                          const int32_t* positions, const int64_t* slot_mapping,
                          int32_t T, void* stream);

/*
 * Append: pa_table_update and pa_kv_write in one launch (a growing sequence
 * writes its new tokens and appends table entries; vLLM post, "PagedAttention:
 * paging, borrowed from the operating system").  For every i with
 * slot_mapping[i] >= 0, token i's K/V go to its slot as in pa_kv_write and
 *   block_tables[seq_ids[i] * max_blocks_per_seq + positions[i] / block_size]
 *       = slot_mapping[i] / block_size.
 * Arguments and requirements as for those two calls (block_tables is
 * int32 [rows][max_blocks_per_seq] on the device).  T = 0 is a no-op.
 */
pa_status pa_kv_append(const pa_pool* pool, void* k_pool, void* v_pool,
                       const void* k_new, const void* v_new,
                       const int64_t* slot_mapping, int32_t T,
                       int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_ids, const int32_t* positions, void* stream);

/* Static description of a status code. */
const char* pa_status_str(pa_status status);

/* Library version, e.g. "pagedkv 0.1 gfx950". */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
