/*
 * pa_bm.h - host block manager for a paged KV cache (plain C, no GPU).
 *
 * What it follows:
 *  - "How PagedAttention Powers vLLM's KV Cache", section "PagedAttention:
 *    paging, borrowed from the operating system": a sequence that needs room
 *    takes a free physical block from a shared pool and appends an entry to
 *    its block table; a finished sequence's blocks return to the pool; only
 *    each sequence's last block can be partly empty.
 *  - same page, section "The bonus contiguous storage can't give you:
 *    sharing": block tables of several sequences may name one physical block,
 *    which carries a reference count; before writing into a shared block a
 *    sequence copies it (copy-on-write); parallel samples reuse the prompt's
 *    blocks.
 *  - attention-lab "PagedAttention" page, reference entry "Shared blocks and
 *    copy-on-write": growing past a full shared block needs only a new block.
 *  - same page, section "Where it bites" of the vLLM page: a full pool forces
 *    the engine to preempt; this library reports the condition (PA_ENOMEM)
 *    and leaves the policy to the caller.  One preemption it supports is
 *    swapping a sequence's blocks out to host memory and back (same section;
 *    glossary entry, "Flexible Management": pages can be swapped out or
 *    spilled to CPU RAM).
 *
 * Deterministic choices (the pages leave them open):
 *  - The free pool is a stack initialised to [N-1, ..., 1, 0] (so the first
 *    pop yields block 0) and, when shuffle_seed != 0, shuffled by
 *    Fisher-Yates driven by SplitMix64(shuffle_seed): for i = N-1 down to 1,
 *    j = next() % (i + 1), swap a[i], a[j].  Blocks are popped from the top.
 *  - Freeing a sequence pushes its blocks on the top, last table entry first.
 *  - Sequence ids are 0, 1, 2, ... in creation order, never reused.
 *  - A sequence appending into a partly filled tail block whose refcount is
 *    above 1 takes a new block, reports the pair (old, new) for the caller to
 *    copy (pa_block_copy) before writing, and drops one reference to the old
 *    block; the last holder writes in place.
 *  - Appends are all or nothing: on PA_ENOMEM no state changes.
 *  - Host swap space is a second pool of num_host_blocks blocks whose free
 *    stack starts as [H-1, ..., 1, 0] (first pop yields 0), unshuffled.
 *    Swapping a sequence out gives each table entry, in table order, a host
 *    block popped from that stack and reports (device block, host block);
 *    then the device references are dropped last entry first, exactly as
 *    freeing would (a block still shared by another sequence stays resident
 *    and the swapped sequence keeps its own copy).  Swapping in pops device
 *    blocks in table order, reports (host block, device block), and pushes
 *    the host blocks back last entry first.  Both are all or nothing.
 *
 * All pointers are HOST pointers owned by the caller.  A pa_bm is not
 * thread-safe; use one per thread or lock around it.
 */
#ifndef PA_BM_H_
#define PA_BM_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm;

typedef struct {
  int64_t num_blocks;
  int64_t block_size;
  int64_t free_blocks;      /* blocks on the free stack                      */
  int64_t used_blocks;      /* blocks with refcount >= 1                     */
  int64_t shared_blocks;    /* blocks with refcount >= 2                     */
  int64_t live_seqs;
  int64_t logical_tokens;   /* sum of live sequences' token counts           */
  int64_t logical_blocks;   /* sum of live sequences' table lengths          */
  int64_t stored_tokens;    /* distinct filled slots over used blocks        */
  int64_t allocated_slots;  /* used_blocks * block_size                      */
  int64_t cow_copies;       /* copy-on-write pairs emitted so far            */
  int64_t enomem_events;    /* appends refused for lack of blocks            */
  int64_t swapped_seqs;     /* live sequences whose blocks are in host memory */
  int64_t host_blocks;      /* size of the host swap space                   */
  int64_t host_free_blocks;
  int64_t swapped_out_blocks; /* blocks copied to host so far                */
  int64_t swapped_in_blocks;  /* blocks copied back so far                   */
} pa_bm_stats_t;
/* live_seqs, logical_tokens and logical_blocks count resident sequences only. */

/* New manager over blocks [0, num_blocks); NULL on bad sizes or host OOM. */
pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed);
void pa_bm_destroy(pa_bm* bm);

/* New empty sequence; its id is written to *seq_id. */
pa_status pa_bm_add_seq(pa_bm* bm, int32_t* seq_id);

/* New sequence sharing every block (and the token count) of `parent`. */
pa_status pa_bm_fork(pa_bm* bm, int32_t parent, int32_t* child);

/*
 * Append n_tokens >= 0 tokens to `seq`.  slots_out[n_tokens] receives each
 * new token's slot (block * block_size + offset) in order.  If the tail block
 * was shared and partly filled, cow_pairs_out[0..1] receives (src, dst) and
 * *n_cow = 1, else *n_cow = 0.  PA_ENOMEM: not enough free blocks; nothing
 * changed.  PA_EINVAL: unknown or freed sequence, n_tokens < 0, NULL output.
 */
pa_status pa_bm_append(pa_bm* bm, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                       int32_t* cow_pairs_out, int32_t* n_cow);

/*
 * Append to several distinct sequences at once: n_tokens[i] tokens to
 * seqs[i].  Outputs, concatenated in call order:
 *   slots_out[sum n]      slot of each new token,
 *   seq_out[sum n]        its sequence id,
 *   pos_out[sum n]        its logical position,
 *   cow_pairs_out[2*k]    (src, dst) of every copy-on-write, *n_cow = k
 *                         (at most n_seqs pairs).
 * All or nothing over the whole batch (PA_ENOMEM / PA_EINVAL change nothing;
 * a repeated sequence id is PA_EINVAL).  seq_out and pos_out may be NULL.
 */
pa_status pa_bm_append_batch(pa_bm* bm, const int32_t* seqs, const int32_t* n_tokens,
                             int32_t n_seqs, int64_t* slots_out, int32_t* seq_out,
                             int32_t* pos_out, int32_t* cow_pairs_out, int32_t* n_cow);

/* Return every block of `seq` (refcount - 1; pushed when it reaches 0); the
 * host blocks of a swapped-out sequence go back to the host free stack. */
pa_status pa_bm_free_seq(pa_bm* bm, int32_t seq);

/*
 * Give the manager a host swap space of num_host_blocks blocks (block ids
 * 0..num_host_blocks-1 of a caller-owned pinned host buffer laid out like
 * the pools).  Allowed while no block is swapped out; replaces any previous
 * size.  PA_EINVAL on a negative size or blocks in use.
 */
pa_status pa_bm_set_host_blocks(pa_bm* bm, int32_t num_host_blocks);

/*
 * Swap `seq` out: pairs_out[2 * len] receives (device block, host block) for
 * each table entry in order (*n_pairs = len, the caller copies them with
 * pa_block_swap(PA_SWAP_OUT) before reusing the freed device blocks); the
 * sequence keeps its token count and becomes swapped: append, fork and
 * export refuse it until it is swapped in.  PA_ENOMEM: fewer free host
 * blocks than table entries; nothing changed.  PA_EINVAL: unknown, freed or
 * already swapped sequence.
 */
pa_status pa_bm_swap_out(pa_bm* bm, int32_t seq, int32_t* pairs_out, int32_t* n_pairs);

/*
 * Swap `seq` back in: pairs_out[2 * len] receives (host block, device block)
 * per table entry in order (the caller copies them with
 * pa_block_swap(PA_SWAP_IN) before decoding it).  PA_ENOMEM: fewer free
 * device blocks than table entries; nothing changed.  PA_EINVAL: the
 * sequence is not swapped out.
 */
pa_status pa_bm_swap_in(pa_bm* bm, int32_t seq, int32_t* pairs_out, int32_t* n_pairs);

/* 1 if `seq` is swapped out, 0 if resident, -1 if unknown or freed. */
int32_t pa_bm_is_swapped(const pa_bm* bm, int32_t seq);

/* Copy the host free stack, bottom first, into out[cap]; returns its length. */
int32_t pa_bm_host_free_list(const pa_bm* bm, int32_t* out, int32_t cap);

/*
 * Copy seq's table into out[cap] (as many entries as fit); *n_blocks and
 * *n_tokens receive the table length and token count (either may be NULL).
 * For a swapped-out sequence the entries are host block ids.
 */
pa_status pa_bm_block_table(const pa_bm* bm, int32_t seq, int32_t* out, int32_t cap,
                            int32_t* n_blocks, int32_t* n_tokens);

/*
 * Dense export for a decode batch: row i of tables_out[n_seqs][width] gets
 * seqs[i]'s table, entries past its length set to pad_block; lens_out[i] its
 * token count.  PA_EINVAL if a table is longer than width or a sequence is
 * swapped out.
 */
pa_status pa_bm_export(const pa_bm* bm, const int32_t* seqs, int32_t n_seqs,
                       int32_t* tables_out, int32_t width, int32_t pad_block,
                       int32_t* lens_out);

/*
 * Prefix groups of a decode batch, for pa_decode_shared (vLLM post, "The
 * bonus contiguous storage can't give you: sharing": parallel samples of
 * one prompt point their block tables at the same physical blocks, which
 * are stored once; glossary entry, "Sampling Algorithms": the shared
 * prompt's pages need not be read or computed again per sample).  Walks
 * seqs[0..n_seqs) in order and cuts it into runs of consecutive sequences.
 * A run starts at sequence i with S = the number of full blocks (below the
 * token count) of i; the next sequence joins while the run has fewer than
 * max_members members and its first c >= 1 table entries equal i's, c
 * counted among the first min(S, its own full blocks) entries; then S = c.
 * The run shares S blocks (0 for a run of one).  Outputs:
 *   group_start_out[n_seqs + 1]  batch index of each group's first member,
 *                                then n_seqs (caller-allocated, host),
 *   shared_blocks_out[n_seqs]    full blocks each group shares,
 *   *n_groups_out                number of groups.
 * PA_EINVAL for an unknown, freed or swapped-out sequence.  Read only.
 */
pa_status pa_bm_prefix_groups(const pa_bm* bm, const int32_t* seqs, int32_t n_seqs,
                              int32_t max_members, int32_t* group_start_out,
                              int32_t* shared_blocks_out, int32_t* n_groups_out);

/* Refcount of one block (-1 if out of range). */
int32_t pa_bm_refcount(const pa_bm* bm, int32_t block);

/* Copy the free stack, bottom first, into out[cap]; returns its length. */
int32_t pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap);

pa_status pa_bm_stats(const pa_bm* bm, pa_bm_stats_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_BM_H_ */
