/*
 * Randomised stress of the host block manager through its public C API,
 * built by tests/test_bm_sanitized.py with AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only).  After every operation it
 * checks the invariants the pages' description of paging and sharing fixes:
 *  - a block's refcount equals the number of resident tables that name it
 *    (each table entry counts once), and every referenced block is in range;
 *  - free and referenced blocks partition the pool (free + used = all);
 *  - a resident sequence's table has ceil(tokens / block_size) entries;
 *  - appended slots lie in the tail blocks the sequence's table now names;
 *  - a copy-on-write pair copies the old tail to a new private block;
 *  - swapped-out sequences hold distinct host blocks, and swap-in gives
 *    back a table of the same length;
 *  - refused operations (exhaustion, bad ids, double frees) change nothing.
 * Exit status 0 on success; any violation prints a line and exits 1.
 * Arguments: seed, operations (default 20000).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pa_bm.h"

#define NB 600
#define B 16
#define NH 200
#define MAXSEQ 4096
#define MAXTAB 4096

static uint64_t rng_state;
static uint64_t next_u64(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 2685821657736338717ULL;
}
static int rnd(int n) { return (int)(next_u64() % (uint64_t)n); }

static int live[MAXSEQ], n_live;
static int op_no;

#define FAIL(...)                                       \
  do {                                                  \
    fprintf(stderr, "op %d: ", op_no);                  \
    fprintf(stderr, __VA_ARGS__);                       \
    fprintf(stderr, "\n");                              \
    exit(1);                                            \
  } while (0)

static void check(pa_bm* bm) {
  static int count[NB], table[MAXTAB], host_seen[NH];
  memset(count, 0, sizeof count);
  memset(host_seen, 0, sizeof host_seen);
  for (int i = 0; i < n_live; ++i) {
    int nb = 0, nt = 0;
    if (pa_bm_block_table(bm, live[i], table, MAXTAB, &nb, &nt) != PA_OK)
      FAIL("block_table of live sequence %d refused", live[i]);
    if (nb != (nt + B - 1) / B) FAIL("seq %d: %d entries for %d tokens", live[i], nb, nt);
    const int sw = pa_bm_is_swapped(bm, live[i]);
    if (sw < 0) FAIL("live sequence %d unknown", live[i]);
    for (int j = 0; j < nb; ++j) {
      if (sw) {
        if (table[j] < 0 || table[j] >= NH) FAIL("host block %d out of range", table[j]);
        if (host_seen[table[j]]++) FAIL("host block %d held twice", table[j]);
      } else {
        if (table[j] < 0 || table[j] >= NB) FAIL("block %d out of range", table[j]);
        count[table[j]]++;
      }
    }
  }
  int used = 0;
  for (int b = 0; b < NB; ++b) {
    const int rc = pa_bm_refcount(bm, b);
    if (rc != count[b]) FAIL("block %d: refcount %d, named by %d tables", b, rc, count[b]);
    used += rc > 0;
  }
  pa_bm_stats_t st;
  if (pa_bm_stats(bm, &st) != PA_OK) FAIL("stats refused");
  if (st.used_blocks != used) FAIL("stats used %lld, counted %d", (long long)st.used_blocks, used);
  if (st.free_blocks + st.used_blocks != NB)
    FAIL("free %lld + used %lld != %d", (long long)st.free_blocks, (long long)st.used_blocks, NB);
  int fl[NB];
  const int nf = pa_bm_free_list(bm, fl, NB);
  if (nf != st.free_blocks) FAIL("free list %d, stats %lld", nf, (long long)st.free_blocks);
  for (int i = 0; i < nf; ++i)
    if (fl[i] < 0 || fl[i] >= NB || count[fl[i]]) FAIL("free block %d is referenced", fl[i]);
}

static void remove_live(int i) { live[i] = live[--n_live]; }

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? strtoull(argv[1], NULL, 0) : 1;
  const int ops = argc > 2 ? atoi(argv[2]) : 20000;
  rng_state = seed * 0x9E3779B97F4A7C15ULL + 1;
  pa_bm* bm = pa_bm_create(NB, B, seed);
  if (!bm) FAIL("create failed");
  if (pa_bm_create(0, B, 1) != NULL || pa_bm_create(NB, 0, 1) != NULL) FAIL("bad sizes accepted");
  if (pa_bm_set_host_blocks(bm, NH) != PA_OK) FAIL("set_host_blocks refused");
  static int64_t slots[4 * MAXTAB];
  static int32_t seqs_b[64], ns_b[64], sq_out[4 * MAXTAB], pos_out[4 * MAXTAB], cow[128], pairs[2 * MAXTAB];
  static int tab_before[MAXTAB], tab_after[MAXTAB];
  for (op_no = 0; op_no < ops; ++op_no) {
    const int op = rnd(100);
    if (op < 10 || n_live == 0) {  /* add */
      int s;
      if (pa_bm_add_seq(bm, &s) != PA_OK) FAIL("add_seq refused");
      if (n_live < MAXSEQ) live[n_live++] = s;
    } else if (op < 18) {  /* fork */
      const int p = live[rnd(n_live)];
      int c;
      const pa_status r = pa_bm_fork(bm, p, &c);
      if (pa_bm_is_swapped(bm, p)) {
        if (r != PA_EINVAL) FAIL("fork of swapped seq %d not refused", p);
      } else {
        if (r != PA_OK) FAIL("fork refused");
        if (n_live < MAXSEQ) live[n_live++] = c; else pa_bm_free_seq(bm, c);
      }
    } else if (op < 58) {  /* append to one sequence */
      const int s = live[rnd(n_live)];
      const int n = rnd(4) == 0 ? rnd(60) : rnd(3);
      int nb0 = 0, nt0 = 0, n_cow = -1;
      pa_bm_block_table(bm, s, tab_before, MAXTAB, &nb0, &nt0);
      pa_bm_stats_t st0;
      pa_bm_stats(bm, &st0);
      const pa_status r = pa_bm_append(bm, s, n, slots, cow, &n_cow);
      if (pa_bm_is_swapped(bm, s)) {
        if (r != PA_EINVAL) FAIL("append to swapped seq not refused");
      } else if (r == PA_ENOMEM) {
        pa_bm_stats_t st1;
        int nb1 = 0, nt1 = 0;
        pa_bm_stats(bm, &st1);
        pa_bm_block_table(bm, s, tab_after, MAXTAB, &nb1, &nt1);
        if (st1.free_blocks != st0.free_blocks || nb1 != nb0 || nt1 != nt0)
          FAIL("refused append changed the state");
      } else if (r != PA_OK) {
        FAIL("append refused (%d)", (int)r);
      } else {
        int nb1 = 0, nt1 = 0;
        pa_bm_block_table(bm, s, tab_after, MAXTAB, &nb1, &nt1);
        if (nt1 != nt0 + n) FAIL("token count %d after %d + %d", nt1, nt0, n);
        for (int i = 0; i < n; ++i) {
          const int p = nt0 + i;
          if (slots[i] != (int64_t)tab_after[p / B] * B + p % B) FAIL("slot of position %d", p);
        }
        if (n_cow) {
          if (n_cow != 1 || nt0 % B == 0 || cow[0] != tab_before[nb0 - 1] ||
              cow[1] != tab_after[nb0 - 1] || cow[0] == cow[1])
            FAIL("bad copy-on-write pair (%d, %d)", cow[0], cow[1]);
        }
        for (int j = 0; j < nb0 - 1; ++j)
          if (tab_after[j] != tab_before[j]) FAIL("full block %d of seq %d moved", j, s);
      }
    } else if (op < 70) {  /* batch append over distinct sequences */
      int k = 0;
      for (int i = 0; i < n_live && k < 64; ++i) {
        if (rnd(4)) continue;
        if (pa_bm_is_swapped(bm, live[i])) continue;
        seqs_b[k] = live[i];
        ns_b[k++] = rnd(3);
      }
      if (k == 0) continue;
      int n_cow = -1;
      const pa_status r =
          pa_bm_append_batch(bm, seqs_b, ns_b, k, slots, sq_out, pos_out, cow, &n_cow);
      if (r != PA_OK && r != PA_ENOMEM) FAIL("batch append refused (%d)", (int)r);
      if (r == PA_OK) {
        int t = 0;
        for (int i = 0; i < k; ++i)
          for (int j = 0; j < ns_b[i]; ++j, ++t)
            if (sq_out[t] != seqs_b[i]) FAIL("batch token %d of the wrong sequence", t);
        if (n_cow < 0 || n_cow > k) FAIL("batch copy count %d", n_cow);
      }
      if (k >= 2) {  /* a repeated id is refused */
        seqs_b[1] = seqs_b[0];
        if (pa_bm_append_batch(bm, seqs_b, ns_b, 2, slots, NULL, NULL, cow, &n_cow) != PA_EINVAL)
          FAIL("repeated sequence id accepted");
      }
    } else if (op < 82) {  /* free */
      const int i = rnd(n_live);
      const int s = live[i];
      if (pa_bm_free_seq(bm, s) != PA_OK) FAIL("free refused");
      if (pa_bm_free_seq(bm, s) != PA_EINVAL) FAIL("double free accepted");
      if (pa_bm_is_swapped(bm, s) != -1) FAIL("freed sequence still known");
      remove_live(i);
    } else if (op < 91) {  /* swap out */
      const int s = live[rnd(n_live)];
      int np = -1, nb0 = 0;
      pa_bm_block_table(bm, s, tab_before, MAXTAB, &nb0, NULL);
      const int was = pa_bm_is_swapped(bm, s);
      const pa_status r = pa_bm_swap_out(bm, s, pairs, &np);
      if (was) {
        if (r != PA_EINVAL) FAIL("second swap-out accepted");
      } else if (r == PA_OK) {
        if (np != nb0) FAIL("swap-out pairs %d for %d entries", np, nb0);
        for (int j = 0; j < np; ++j)
          if (pairs[2 * j] != tab_before[j]) FAIL("swap-out pair %d source", j);
      } else if (r != PA_ENOMEM) {
        FAIL("swap-out refused (%d)", (int)r);
      }
    } else {  /* swap in */
      const int s = live[rnd(n_live)];
      int np = -1, nb0 = 0;
      pa_bm_block_table(bm, s, tab_before, MAXTAB, &nb0, NULL);
      const int was = pa_bm_is_swapped(bm, s);
      const pa_status r = pa_bm_swap_in(bm, s, pairs, &np);
      if (!was) {
        if (r != PA_EINVAL) FAIL("swap-in of a resident sequence accepted");
      } else if (r == PA_OK) {
        int nb1 = 0;
        pa_bm_block_table(bm, s, tab_after, MAXTAB, &nb1, NULL);
        if (np != nb0 || nb1 != nb0) FAIL("swap-in changed the table length");
        for (int j = 0; j < np; ++j)
          if (pairs[2 * j] != tab_before[j] || pairs[2 * j + 1] != tab_after[j])
            FAIL("swap-in pair %d", j);
      } else if (r != PA_ENOMEM) {
        FAIL("swap-in refused (%d)", (int)r);
      }
    }
    /* unknown ids are refused */
    if (op_no % 97 == 0) {
      int c;
      if (pa_bm_fork(bm, -1, &c) != PA_EINVAL || pa_bm_free_seq(bm, 1 << 30) != PA_EINVAL ||
          pa_bm_append(bm, -5, 1, slots, cow, &c) != PA_EINVAL)
        FAIL("bad sequence id accepted");
    }
    check(bm);
  }
  while (n_live) {
    if (pa_bm_free_seq(bm, live[n_live - 1]) != PA_OK) FAIL("final free refused");
    --n_live;
  }
  check(bm);
  pa_bm_stats_t st;
  pa_bm_stats(bm, &st);
  if (st.free_blocks != NB || st.host_free_blocks != NH) FAIL("blocks not all returned");
  pa_bm_destroy(bm);
  printf("ok: %d operations, seed %llu, cow %lld, refused appends %lld, swapped out %lld, in %lld\n",
         ops, (unsigned long long)seed, (long long)st.cow_copies, (long long)st.enomem_events,
         (long long)st.swapped_out_blocks, (long long)st.swapped_in_blocks);
  return 0;
}
