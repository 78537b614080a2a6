/*
 * Host block manager for the paged KV cache (C11, no GPU dependency).
 *
 * Allocation rules: "How PagedAttention Powers vLLM's KV Cache", sections
 * "PagedAttention: paging, borrowed from the operating system" (blocks taken
 * from a shared free pool on demand and returned when a sequence finishes)
 * and "The bonus contiguous storage can't give you: sharing" (refcounted
 * shared blocks, copy before writing into a shared block); attention-lab
 * "PagedAttention" page, reference entry "Shared blocks and copy-on-write"
 * (growing past a full shared block needs only a new block).  The
 * deterministic choices the pages leave open are stated in pa_bm.h.
 */
#include <stdlib.h>
#include <string.h>

#include "pa_bm.h"

typedef struct {
  int32_t* table;   /* device block ids, or host block ids while swapped */
  int32_t len;
  int32_t cap;
  int32_t n_tokens;
  int32_t alive;
  int32_t swapped;
} bm_seq;

struct pa_bm {
  int32_t num_blocks;
  int32_t block_size;
  int32_t* free_stack; /* capacity num_blocks */
  int32_t n_free;
  int32_t* refcount;   /* [num_blocks] */
  int32_t* scratch;    /* [num_blocks], per-call workspace */
  bm_seq* seqs;
  int32_t n_seqs;
  int32_t seq_cap;
  uint32_t* stamp;     /* [seq_cap], duplicate detection in batches */
  uint32_t epoch;
  int64_t cow_copies;
  int64_t enomem_events;
  int32_t num_host_blocks;
  int32_t* host_free; /* capacity num_host_blocks */
  int32_t n_host_free;
  int64_t swapped_out_blocks;
  int64_t swapped_in_blocks;
};

/* SplitMix64 (Steele, Lea, Flood 2014): Weyl step then a 64-bit mixer. */
static uint64_t splitmix64_next(uint64_t* state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed) {
  if (num_blocks <= 0 || block_size <= 0) return NULL;
  pa_bm* bm = (pa_bm*)calloc(1, sizeof(pa_bm));
  if (!bm) return NULL;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->free_stack = (int32_t*)malloc(sizeof(int32_t) * (size_t)num_blocks);
  bm->refcount = (int32_t*)calloc((size_t)num_blocks, sizeof(int32_t));
  bm->scratch = (int32_t*)calloc((size_t)num_blocks, sizeof(int32_t)); /* kept zero between calls */
  if (!bm->free_stack || !bm->refcount || !bm->scratch) {
    pa_bm_destroy(bm);
    return NULL;
  }
  for (int32_t i = 0; i < num_blocks; ++i) bm->free_stack[i] = num_blocks - 1 - i;
  if (shuffle_seed != 0) {
    uint64_t st = shuffle_seed;
    for (int32_t i = num_blocks - 1; i > 0; --i) {
      int32_t j = (int32_t)(splitmix64_next(&st) % (uint64_t)(i + 1));
      int32_t t = bm->free_stack[i];
      bm->free_stack[i] = bm->free_stack[j];
      bm->free_stack[j] = t;
    }
  }
  bm->n_free = num_blocks;
  return bm;
}

void pa_bm_destroy(pa_bm* bm) {
  if (!bm) return;
  for (int32_t s = 0; s < bm->n_seqs; ++s) free(bm->seqs[s].table);
  free(bm->seqs);
  free(bm->stamp);
  free(bm->free_stack);
  free(bm->refcount);
  free(bm->scratch);
  free(bm->host_free);
  free(bm);
}

static int live(const pa_bm* bm, int32_t s) {
  return s >= 0 && s < bm->n_seqs && bm->seqs[s].alive;
}

/* A live sequence whose blocks are on the device. */
static int resident(const pa_bm* bm, int32_t s) { return live(bm, s) && !bm->seqs[s].swapped; }

static pa_status new_seq(pa_bm* bm, int32_t* id) {
  if (bm->n_seqs == INT32_MAX) return PA_ENOMEM;
  if (bm->n_seqs == bm->seq_cap) {
    int32_t cap = bm->seq_cap ? bm->seq_cap * 2 : 64;
    if (cap < bm->seq_cap) cap = INT32_MAX;
    bm_seq* ns = (bm_seq*)realloc(bm->seqs, sizeof(bm_seq) * (size_t)cap);
    if (!ns) return PA_ENOMEM;
    bm->seqs = ns;
    uint32_t* st = (uint32_t*)realloc(bm->stamp, sizeof(uint32_t) * (size_t)cap);
    if (!st) return PA_ENOMEM;
    memset(st + bm->seq_cap, 0, sizeof(uint32_t) * (size_t)(cap - bm->seq_cap));
    bm->stamp = st;
    bm->seq_cap = cap;
  }
  bm_seq* q = &bm->seqs[bm->n_seqs];
  memset(q, 0, sizeof *q);
  q->alive = 1;
  *id = bm->n_seqs++;
  return PA_OK;
}

static int reserve_table(bm_seq* q, int32_t need) {
  if (need <= q->cap) return 1;
  int32_t cap = q->cap ? q->cap : 16;
  while (cap < need) cap *= 2;
  int32_t* t = (int32_t*)realloc(q->table, sizeof(int32_t) * (size_t)cap);
  if (!t) return 0;
  q->table = t;
  q->cap = cap;
  return 1;
}

pa_status pa_bm_add_seq(pa_bm* bm, int32_t* seq_id) {
  if (!bm || !seq_id) return PA_EINVAL;
  return new_seq(bm, seq_id);
}

pa_status pa_bm_fork(pa_bm* bm, int32_t parent, int32_t* child) {
  if (!bm || !child || !resident(bm, parent)) return PA_EINVAL;
  int32_t id;
  pa_status st = new_seq(bm, &id);
  if (st != PA_OK) return st;
  bm_seq* p = &bm->seqs[parent]; /* re-read: new_seq may move the array */
  bm_seq* c = &bm->seqs[id];
  if (!reserve_table(c, p->len)) {
    c->alive = 0; /* id stays consumed but unusable; no block state changed */
    return PA_ENOMEM;
  }
  if (p->len) memcpy(c->table, p->table, sizeof(int32_t) * (size_t)p->len);
  c->len = p->len;
  c->n_tokens = p->n_tokens;
  for (int32_t j = 0; j < c->len; ++j) bm->refcount[c->table[j]] += 1;
  *child = id;
  return PA_OK;
}

/* Blocks an append of n tokens to q needs: new blocks plus a possible copy. */
static int64_t blocks_needed(const pa_bm* bm, const bm_seq* q, int32_t n, int* cow) {
  const int64_t B = bm->block_size;
  int64_t end = (int64_t)q->n_tokens + n;
  int64_t need_new = (end + B - 1) / B - q->len;
  *cow = n > 0 && (q->n_tokens % B) != 0 && bm->refcount[q->table[q->len - 1]] > 1;
  return need_new + (*cow ? 1 : 0);
}

/* Apply an append already checked to fit.  Writes n slots (and seq/pos). */
static void apply_append(pa_bm* bm, int32_t s, int32_t n, int cow, int64_t* slots,
                         int32_t* seq_out, int32_t* pos_out, int32_t* pair_out) {
  bm_seq* q = &bm->seqs[s];
  const int32_t B = bm->block_size;
  if (cow) {
    int32_t src = q->table[q->len - 1];
    int32_t dst = bm->free_stack[--bm->n_free];
    bm->refcount[src] -= 1;
    bm->refcount[dst] = 1;
    q->table[q->len - 1] = dst;
    pair_out[0] = src;
    pair_out[1] = dst;
    bm->cow_copies += 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t p = q->n_tokens + i;
    if (p % B == 0) {
      int32_t b = bm->free_stack[--bm->n_free];
      bm->refcount[b] = 1;
      q->table[q->len++] = b;
    }
    slots[i] = (int64_t)q->table[p / B] * B + p % B;
    if (seq_out) seq_out[i] = s;
    if (pos_out) pos_out[i] = p;
  }
  q->n_tokens += n;
}

pa_status pa_bm_append(pa_bm* bm, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                       int32_t* cow_pairs_out, int32_t* n_cow) {
  if (!bm || !resident(bm, seq) || n_tokens < 0 || !n_cow) return PA_EINVAL;
  if (n_tokens > 0 && (!slots_out || !cow_pairs_out)) return PA_EINVAL;
  *n_cow = 0;
  if (n_tokens == 0) return PA_OK;
  bm_seq* q = &bm->seqs[seq];
  if ((int64_t)q->n_tokens + n_tokens > INT32_MAX) return PA_EINVAL;
  int cow;
  int64_t need = blocks_needed(bm, q, n_tokens, &cow);
  if (need > bm->n_free) {
    bm->enomem_events += 1;
    return PA_ENOMEM;
  }
  int64_t end = (int64_t)q->n_tokens + n_tokens;
  if (!reserve_table(q, (int32_t)((end + bm->block_size - 1) / bm->block_size)))
    return PA_ENOMEM;
  apply_append(bm, seq, n_tokens, cow, slots_out, NULL, NULL, cow_pairs_out);
  *n_cow = cow ? 1 : 0;
  return PA_OK;
}

pa_status pa_bm_append_batch(pa_bm* bm, const int32_t* seqs, const int32_t* n_tokens,
                             int32_t n_seqs, int64_t* slots_out, int32_t* seq_out,
                             int32_t* pos_out, int32_t* cow_pairs_out, int32_t* n_cow) {
  if (!bm || n_seqs < 0 || !n_cow) return PA_EINVAL;
  *n_cow = 0;
  if (n_seqs == 0) return PA_OK;
  if (!seqs || !n_tokens || !slots_out || !cow_pairs_out) return PA_EINVAL;
  bm->epoch += 1;
  if (bm->epoch == 0) { /* wrapped: clear stamps once */
    memset(bm->stamp, 0, sizeof(uint32_t) * (size_t)bm->seq_cap);
    bm->epoch = 1;
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    int32_t s = seqs[i];
    if (!resident(bm, s) || n_tokens[i] < 0 || bm->stamp[s] == bm->epoch) return PA_EINVAL;
    if ((int64_t)bm->seqs[s].n_tokens + n_tokens[i] > INT32_MAX) return PA_EINVAL;
    bm->stamp[s] = bm->epoch;
  }
  /* Blocks the batch takes, counted as the appends will run, one after
   * another: each copy-on-write drops the shared tail's refcount, so of k
   * sharers of a partly filled tail only the first k - 1 copy and the last
   * writes in place.  scratch[b] counts the drops of block b so far. */
  int64_t need_total = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const bm_seq* q = &bm->seqs[seqs[i]];
    const int32_t n = n_tokens[i];
    const int64_t end = (int64_t)q->n_tokens + n;
    need_total += (end + bm->block_size - 1) / bm->block_size - q->len;
    if (n > 0 && q->n_tokens % bm->block_size != 0) {
      const int32_t tail = q->table[q->len - 1];
      if (bm->refcount[tail] - bm->scratch[tail] > 1) {
        need_total += 1;
        bm->scratch[tail] += 1;
      }
    }
  }
  for (int32_t i = 0; i < n_seqs; ++i) { /* scratch back to zero */
    const bm_seq* q = &bm->seqs[seqs[i]];
    if (q->len > 0) bm->scratch[q->table[q->len - 1]] = 0;
  }
  if (need_total > bm->n_free) {
    bm->enomem_events += 1;
    return PA_ENOMEM;
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    bm_seq* q = &bm->seqs[seqs[i]];
    int64_t end = (int64_t)q->n_tokens + n_tokens[i];
    if (!reserve_table(q, (int32_t)((end + bm->block_size - 1) / bm->block_size)))
      return PA_ENOMEM; /* host OOM; only spare capacity was added so far */
  }
  int64_t off = 0;
  int32_t k = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    int32_t s = seqs[i], n = n_tokens[i];
    int cow;
    blocks_needed(bm, &bm->seqs[s], n, &cow);
    apply_append(bm, s, n, cow, slots_out + off, seq_out ? seq_out + off : NULL,
                 pos_out ? pos_out + off : NULL, cow_pairs_out + 2 * k);
    if (cow) ++k;
    off += n;
  }
  *n_cow = k;
  return PA_OK;
}

/* Drop seq's device references, last table entry first (freed blocks are
 * pushed on the free stack); PA_EINVAL if a refcount is already 0. */
static pa_status release_device_blocks(pa_bm* bm, bm_seq* q) {
  for (int32_t j = q->len - 1; j >= 0; --j)
    if (bm->refcount[q->table[j]] <= 0) return PA_EINVAL;
  for (int32_t j = q->len - 1; j >= 0; --j) {
    int32_t b = q->table[j];
    if (--bm->refcount[b] == 0) bm->free_stack[bm->n_free++] = b;
  }
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_bm* bm, int32_t seq) {
  if (!bm || !live(bm, seq)) return PA_EINVAL;
  bm_seq* q = &bm->seqs[seq];
  if (q->swapped) {
    for (int32_t j = q->len - 1; j >= 0; --j) bm->host_free[bm->n_host_free++] = q->table[j];
  } else {
    pa_status st = release_device_blocks(bm, q);
    if (st != PA_OK) return st;
  }
  free(q->table);
  q->table = NULL;
  q->len = q->cap = q->n_tokens = 0;
  q->alive = 0;
  q->swapped = 0;
  return PA_OK;
}

pa_status pa_bm_set_host_blocks(pa_bm* bm, int32_t num_host_blocks) {
  if (!bm || num_host_blocks < 0) return PA_EINVAL;
  if (bm->n_host_free != bm->num_host_blocks) return PA_EINVAL; /* blocks in use */
  int32_t* hf = NULL;
  if (num_host_blocks > 0) {
    hf = (int32_t*)malloc(sizeof(int32_t) * (size_t)num_host_blocks);
    if (!hf) return PA_ENOMEM;
    for (int32_t i = 0; i < num_host_blocks; ++i) hf[i] = num_host_blocks - 1 - i;
  }
  free(bm->host_free);
  bm->host_free = hf;
  bm->num_host_blocks = num_host_blocks;
  bm->n_host_free = num_host_blocks;
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_bm* bm, int32_t seq, int32_t* pairs_out, int32_t* n_pairs) {
  if (!bm || !n_pairs || !resident(bm, seq)) return PA_EINVAL;
  bm_seq* q = &bm->seqs[seq];
  if (q->len > 0 && !pairs_out) return PA_EINVAL;
  if (q->len > bm->n_host_free) return PA_ENOMEM;
  for (int32_t j = 0; j < q->len; ++j)
    if (bm->refcount[q->table[j]] <= 0) return PA_EINVAL;
  int32_t* host = bm->scratch; /* len <= num_blocks */
  for (int32_t j = 0; j < q->len; ++j) {
    host[j] = bm->host_free[--bm->n_host_free];
    pairs_out[2 * j] = q->table[j];
    pairs_out[2 * j + 1] = host[j];
  }
  release_device_blocks(bm, q); /* refcounts checked above */
  for (int32_t j = 0; j < q->len; ++j) {
    q->table[j] = host[j];
    host[j] = 0;
  }
  q->swapped = 1;
  bm->swapped_out_blocks += q->len;
  *n_pairs = q->len;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_bm* bm, int32_t seq, int32_t* pairs_out, int32_t* n_pairs) {
  if (!bm || !n_pairs || !live(bm, seq) || !bm->seqs[seq].swapped) return PA_EINVAL;
  bm_seq* q = &bm->seqs[seq];
  if (q->len > 0 && !pairs_out) return PA_EINVAL;
  if (q->len > bm->n_free) return PA_ENOMEM;
  for (int32_t j = 0; j < q->len; ++j) {
    int32_t d = bm->free_stack[--bm->n_free];
    bm->refcount[d] = 1;
    pairs_out[2 * j] = q->table[j];
    pairs_out[2 * j + 1] = d;
  }
  for (int32_t j = q->len - 1; j >= 0; --j) bm->host_free[bm->n_host_free++] = q->table[j];
  for (int32_t j = 0; j < q->len; ++j) q->table[j] = pairs_out[2 * j + 1];
  q->swapped = 0;
  bm->swapped_in_blocks += q->len;
  *n_pairs = q->len;
  return PA_OK;
}

int32_t pa_bm_is_swapped(const pa_bm* bm, int32_t seq) {
  if (!bm || !live(bm, seq)) return -1;
  return bm->seqs[seq].swapped ? 1 : 0;
}

int32_t pa_bm_host_free_list(const pa_bm* bm, int32_t* out, int32_t cap) {
  if (!bm) return -1;
  int32_t n = bm->n_host_free < cap ? bm->n_host_free : cap;
  if (n > 0 && out) memcpy(out, bm->host_free, sizeof(int32_t) * (size_t)n);
  return bm->n_host_free;
}

pa_status pa_bm_block_table(const pa_bm* bm, int32_t seq, int32_t* out, int32_t cap,
                            int32_t* n_blocks, int32_t* n_tokens) {
  if (!bm || !live(bm, seq) || cap < 0 || (cap > 0 && !out)) return PA_EINVAL;
  const bm_seq* q = &bm->seqs[seq];
  int32_t n = q->len < cap ? q->len : cap;
  if (n) memcpy(out, q->table, sizeof(int32_t) * (size_t)n);
  if (n_blocks) *n_blocks = q->len;
  if (n_tokens) *n_tokens = q->n_tokens;
  return PA_OK;
}

pa_status pa_bm_export(const pa_bm* bm, const int32_t* seqs, int32_t n_seqs,
                       int32_t* tables_out, int32_t width, int32_t pad_block,
                       int32_t* lens_out) {
  if (!bm || n_seqs < 0 || width < 0) return PA_EINVAL;
  if (n_seqs == 0) return PA_OK;
  if (!seqs || !tables_out || !lens_out) return PA_EINVAL;
  for (int32_t i = 0; i < n_seqs; ++i)
    if (!resident(bm, seqs[i]) || bm->seqs[seqs[i]].len > width) return PA_EINVAL;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const bm_seq* q = &bm->seqs[seqs[i]];
    int32_t* row = tables_out + (size_t)i * width;
    if (q->len) memcpy(row, q->table, sizeof(int32_t) * (size_t)q->len);
    for (int32_t j = q->len; j < width; ++j) row[j] = pad_block;
    lens_out[i] = q->n_tokens;
  }
  return PA_OK;
}

int32_t pa_bm_refcount(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[block];
}

int32_t pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap) {
  if (!bm) return -1;
  int32_t n = bm->n_free < cap ? bm->n_free : cap;
  if (n > 0 && out) memcpy(out, bm->free_stack, sizeof(int32_t) * (size_t)n);
  return bm->n_free;
}

pa_status pa_bm_stats(const pa_bm* bm, pa_bm_stats_t* out) {
  if (!bm || !out) return PA_EINVAL;
  memset(out, 0, sizeof *out);
  const int32_t B = bm->block_size;
  out->num_blocks = bm->num_blocks;
  out->block_size = B;
  out->free_blocks = bm->n_free;
  int32_t* fill = bm->scratch;
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    fill[b] = 0;
    if (bm->refcount[b] > 0) out->used_blocks += 1;
    if (bm->refcount[b] > 1) out->shared_blocks += 1;
  }
  for (int32_t s = 0; s < bm->n_seqs; ++s) {
    const bm_seq* q = &bm->seqs[s];
    if (!q->alive) continue;
    if (q->swapped) {
      out->swapped_seqs += 1;
      continue;
    }
    out->live_seqs += 1;
    out->logical_tokens += q->n_tokens;
    out->logical_blocks += q->len;
    for (int32_t j = 0; j < q->len; ++j) {
      int64_t in_block = (int64_t)q->n_tokens - (int64_t)j * B;
      int32_t f = in_block < B ? (int32_t)in_block : B;
      if (f > fill[q->table[j]]) fill[q->table[j]] = f;
    }
  }
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    out->stored_tokens += fill[b];
    fill[b] = 0;
  }
  out->allocated_slots = out->used_blocks * B;
  out->cow_copies = bm->cow_copies;
  out->enomem_events = bm->enomem_events;
  out->host_blocks = bm->num_host_blocks;
  out->host_free_blocks = bm->n_host_free;
  out->swapped_out_blocks = bm->swapped_out_blocks;
  out->swapped_in_blocks = bm->swapped_in_blocks;
  return PA_OK;
}

pa_status pa_bm_prefix_groups(const pa_bm* bm, const int32_t* seqs, int32_t n_seqs,
                              int32_t max_members, int32_t* group_start_out,
                              int32_t* shared_blocks_out, int32_t* n_groups_out) {
  if (!bm || n_seqs < 0 || max_members < 1 || !n_groups_out) return PA_EINVAL;
  *n_groups_out = 0;
  if (n_seqs == 0) {
    if (group_start_out) group_start_out[0] = 0;
    return PA_OK;
  }
  if (!seqs || !group_start_out || !shared_blocks_out) return PA_EINVAL;
  for (int32_t i = 0; i < n_seqs; ++i)
    if (!resident(bm, seqs[i])) return PA_EINVAL;
  const int32_t B = bm->block_size;
  int32_t k = 0, i = 0;
  while (i < n_seqs) {
    const bm_seq* first = &bm->seqs[seqs[i]];
    int32_t shared = first->n_tokens / B; /* full blocks of the first member */
    int32_t j = i + 1;
    while (j < n_seqs && j - i < max_members) {
      const bm_seq* q = &bm->seqs[seqs[j]];
      int32_t lim = q->n_tokens / B < shared ? q->n_tokens / B : shared;
      int32_t c = 0;
      while (c < lim && q->table[c] == first->table[c]) ++c;
      if (c == 0) break;
      shared = c;
      ++j;
    }
    group_start_out[k] = i;
    shared_blocks_out[k] = j - i > 1 ? shared : 0;
    ++k;
    i = j;
  }
  group_start_out[k] = n_seqs;
  *n_groups_out = k;
  return PA_OK;
}
