// Paged decode attention for gfx950 (CDNA4, wave64).
//
// What is computed ("How PagedAttention Powers vLLM's KV Cache", section
// "The attention kernel has to read scattered blocks"; attention-lab
// "PagedAttention" page, reference entry "How it works"): for each sequence
// and query head, softmax(scale * q K^T) V over the sequence's logical tokens,
// reading K/V block by block through the sequence's block table.  The
// equation is the textbook one; only the gather is new.
//
// Work decomposition.  For each group of 4 kv heads, the batch is one flat
// list of blocks: sequence 0's blocks in logical order, then sequence 1's,
// and so on.  The grid is persistent (as many workgroups as fit on the chip
// at once) and every workgroup takes one equal, contiguous range of that
// list for one head group; its 4 waves each stream the range for one kv head
// of the group (with fewer kv heads, or a count that is not a multiple of 4,
// the waves take the next (head, range) pairs in turn, so none idles).
// Every workgroup thus reads the same number of blocks
// whatever the length mix, and a range spans only a few sequences.  Inside
// the range a wave walks piece by piece (a piece is the part of one
// sequence inside the range), keeping a ring of register buffers so that
// the next block's K/V loads are in flight while the current one is
// consumed, and carries an online-softmax state (reference max m, running
// sum l, unnormalised output o) for every query head of the group.  A
// sequence that lies inside one range is finished in place; a sequence cut
// by range boundaries leaves one (m, l, o) partial per piece in the
// workspace, and decode_reduce_kernel combines them:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// Scores are kept in log2 units (scale * log2 e folded in), so v_exp_f32
// (2^x) serves as the exponential.
//
// Two kernel families:
//  * decode_mfma_kernel (bf16, 1..16 query heads per kv head): q.K runs on
//    v_mfma_f32_16x16x32_bf16 with A = the 16 tokens of a block x 32 dims and
//    B = 32 dims x 16 head slots (the group's heads, zero padded).  Its
//    output layout (lane holds tokens 4*(lane/16)+i of head lane%16) is
//    the A layout P.V needs, so probabilities never leave the lane.  P.V is
//    one v_mfma_f32_16x16x32_bf16 per 16 output dims whose 32-long k runs
//    over the lane's 4 tokens twice: A holds P's bf16 high part
//    (truncation) and then its low part (p - high, rounded to nearest even),
//    which carries P to about 16 significant bits, and B the lane's V values
//    twice.  V is stored dim-major in the pool so each lane's 4 tokens of
//    one dim are one 8-byte load.
//    With a single query head per kv head (MHA) the 16 head slots hold one
//    real head; the instruction count per block does not depend on the group
//    size, and measured against a VALU kernel on the 32/32-head workload the
//    MFMA form was 37% faster (its V loads are contiguous 512-byte runs).
//  * decode_valu_kernel (fp32 pools): 4 lanes per token share a K row for
//    q.K with FMAs and a DPP quad reduce, then each lane owns head_dim/64
//    output dims and accumulates P.V with FMAs, P broadcast through
//    v_readlane.
// Both stream each K/V byte of a (block, kv head) from HBM once.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "pa_device.h"
#include "pa_internal.h"

namespace pakv {
namespace {

// A piece of work for one wave: logical tokens [t0, t1) of one segment for
// kv head g.  The segment's member sequences s .. s + nmem - 1 read the same
// blocks; member m's query head h of the group takes head slot m * G + h.
// A piece that is the whole attention of one sequence (in_place) is
// normalised and stored; any other leaves (m, l, o) for head slot c in
// partial row prow + (c / G) * mstride + c % G.
struct Unit {
  int s, nmem, g, t0, t1, prow, mstride;
  bool in_place;
  bool last;  // the piece ends the sequence (its own segment's last token)
};

// The plan every workgroup builds in LDS from the context lengths (and the
// prefix groups): segments in order, and their block prefix sums.  Built
// from scans only, so every workgroup gets the same plan.
struct Plan {
  int* wsum;         // [8] scan scratch in LDS
  const int* pre;    // [K + 1] blocks before segment k; pre[K] = T
  const int* lens;   // [S] context lengths (clamped to the table capacity)
  const int* sdesc;  // [K] first member | member count << 16 (nullptr: segment k is sequence k)
  const int* sj0;    // [K] first logical block of the segment
  int S, K, T, q, R;  // R: ranges per kv head, q: places per range
  int cs;             // start cost of a segment (empty places before its blocks)
  // places [sb, se) of segment k: its blocks sit at [first(k), se)
  __device__ int first(int k) const { return pre[k + 1] > pre[k] ? pre[k] + cs : pre[k]; }
};

// Dynamic LDS bytes for a plan over S sequences (with prefix groups a
// sequence can add a segment: at most 2S).
__host__ __device__ constexpr size_t plan_lds_bytes(int S, bool grouped) {
  return ((size_t)S + (grouped ? 6 * (size_t)S : (size_t)S) + 1 + 8) * sizeof(int);
}

// Group i of the prefix groups, clipped to this launch's sequences: members
// [*m0, *m1) (launch-local indices) and the full blocks they share.  A group
// whose members would not fit the head slots of one tile, or whose shared
// blocks reach past a member's full blocks (arguments outside the
// contract), shares nothing, which gives the same result.
template <int B>
__device__ __forceinline__ void group_view(const DecodeArgs& a, const int* lens, int G, int i,
                                           int* m0, int* m1, int* P) {
  const int lo = max(a.group_start[i], a.seq_base) - a.seq_base;
  const int hi = min(a.group_start[i + 1], a.seq_base + a.num_seqs) - a.seq_base;
  *m0 = lo;
  *m1 = max(lo, hi);
  int p = min(max(a.shared_blocks[i], 0), a.max_blocks);
  if (hi - lo < 2 || (hi - lo) * G > a.slots) p = 0;
  for (int m = lo; m < hi && p > 0; ++m) p = min(p, lens[m] / B);
  *P = p;
}

// The plan's position space: each non-empty segment of n blocks takes
// n + cs places (cs: the plan's start cost), the first cs of them empty.  A
// piece costs a wave more than its blocks' loads (its q rows and table
// entries, then its first loads' latency with nothing else in flight), so
// ranges cut in this space give a wave that holds many short pieces fewer
// blocks.  The cost is counted in blocks of the kernel's pool: an 8-bit
// block is half the bytes of a bf16 one, so it counts twice as many.
constexpr int kSegStart16 = kSegStartBlocks;      // bf16 and fp32 pools
constexpr int kSegStart8 = 2 * kSegStartBlocks;   // 8-bit pools
__device__ __forceinline__ int seg_cost(int blocks, int cs) { return blocks > 0 ? blocks + cs : 0; }

// Collective over the workgroup; ends with a barrier.  B = tokens per block.
template <int B, int CS = kSegStart16>
__device__ Plan build_plan(const DecodeArgs& a, int G, int* lds) {
  const int S = a.num_seqs;
  const bool grouped = a.group_start != nullptr;
  const int Kmax = grouped ? 2 * S : S;
  int* lens = lds;                          // S
  int* pre = lens + S;                      // Kmax + 1
  int* sdesc = pre + Kmax + 1;              // Kmax (grouped only)
  int* sj0 = sdesc + Kmax;                  // Kmax (grouped only)
  int* wsum = grouped ? sj0 + Kmax : sdesc; // 8
  const int T_ = blockDim.x, t = threadIdx.x;
  // lengths outside [0, table capacity] violate the contract; clamping them
  // keeps every LDS and table index in range whatever the device data says
  const int cap = a.max_blocks * B;
  const int add = a.k_new != nullptr ? 1 : 0;  // a decode step appends one token
  for (int s = t; s < S; s += T_) lens[s] = min(max(a.context_lens[s] + add, 0), cap);
  __syncthreads();
  int K = 0, T = 0;
  bool use_groups = grouped;
  if (grouped) {
    // segments of group i: its shared blocks (when it shares any), then
    // each member's remaining blocks
    const int NG = a.num_groups;
    const int C = (NG + T_ - 1) / T_;
    const int i0 = min(NG, t * C), i1 = min(NG, i0 + C);
    int nseg = 0, nb = 0;
    for (int i = i0; i < i1; ++i) {
      int m0, m1, P;
      group_view<B>(a, lens, G, i, &m0, &m1, &P);
      nseg += (P > 0) + (m1 - m0);
      nb += seg_cost(P, CS);
      for (int m = m0; m < m1; ++m) nb += seg_cost((lens[m] + B - 1) / B - P, CS);
    }
    int k = block_excl_scan(nseg, wsum, &K);
    int run = block_excl_scan(nb, wsum, &T);
    // groups that overlap (outside the contract) could need more segments
    // than the plan holds: the workgroup-uniform total decides, before any
    // write, to plan without them
    use_groups = K <= Kmax;
    if (use_groups) {
      for (int i = i0; i < i1; ++i) {
        int m0, m1, P;
        group_view<B>(a, lens, G, i, &m0, &m1, &P);
        if (P > 0) {
          pre[k] = run;
          sdesc[k] = m0 | (m1 - m0) << 16;
          sj0[k] = 0;
          run += seg_cost(P, CS);
          ++k;
        }
        for (int m = m0; m < m1; ++m) {
          pre[k] = run;
          sdesc[k] = m | 1 << 16;
          sj0[k] = P;
          run += seg_cost((lens[m] + B - 1) / B - P, CS);
          ++k;
        }
      }
    }
  }
  if (!use_groups) {
    const int C = (S + T_ - 1) / T_;  // contiguous chunk of sequences per thread
    const int s0 = min(S, t * C), s1 = min(S, s0 + C);
    int nb = 0;
    for (int s = s0; s < s1; ++s) nb += seg_cost((lens[s] + B - 1) / B, CS);
    int run = block_excl_scan(nb, wsum, &T);
    for (int s = s0; s < s1; ++s) {
      pre[s] = run;
      run += seg_cost((lens[s] + B - 1) / B, CS);
    }
    K = S;
  }
  if (t == 0) pre[K] = T;
  __syncthreads();
  Plan pl;
  pl.wsum = wsum;
  pl.pre = pre;
  pl.lens = lens;
  pl.sdesc = use_groups ? sdesc : nullptr;
  pl.sj0 = sj0;
  pl.S = S;
  pl.K = K;
  pl.T = T;
  // every wave of the grid streams one (kv head, range) pair: R ranges per head
  pl.R = max(1, a.decode_wgs * kWaves / a.num_kv_heads);
  pl.q = max(a.min_seg_blocks, (T + pl.R - 1) / pl.R);
  pl.cs = CS;
  return pl;
}

// Segment k: first member, member count, first logical block.
__device__ __forceinline__ void seg_desc(const Plan& pl, int k, int* s, int* nmem, int* j0) {
  if (pl.sdesc) {
    const int d = pl.sdesc[k];
    *s = d & 0xffff;
    *nmem = d >> 16;
    *j0 = pl.sj0[k];
  } else {
    *s = k;
    *nmem = 1;
    *j0 = 0;
  }
}

// The kv head and range of one wave.  The grid's waves, numbered
// blockIdx * kWaves + wave, take the (head, range) pairs in order, heads
// fastest: with a multiple of kWaves kv heads a workgroup streams one range
// for kWaves consecutive heads (their blocks sit next to each other in the
// pool); with fewer kv heads, or a count that does not divide evenly, no
// wave idles but the last few.  False for a wave with nothing to do.
__device__ __forceinline__ bool wave_work(const DecodeArgs& a, const Plan& pl, int wave, int* g,
                                          int* r) {
  const int slot = blockIdx.x * kWaves + wave;
  *g = slot % a.num_kv_heads;
  *r = slot / a.num_kv_heads;
  return *r < pl.R;
}

// Collective over one workgroup: where each sequence's cut pieces went, for
// the reduce kernel.  seg_info[s] = {range of its first piece * 2 + end of
// that piece, pieces} of the sequence's own segment, then the same for the
// shared segment of its group (pieces | member index << 16; 0 pieces when
// it shares none).  Pieces after the first start at their range's first
// block (end 0).
__device__ void write_seg_info(const DecodeArgs& a, const Plan& pl) {
  // every sequence's entry starts empty, so one that no segment names (only
  // with groups outside the contract) is skipped by the reduce
  for (int s = threadIdx.x; s < pl.S; s += blockDim.x)
    *reinterpret_cast<int4*>(a.seg_info + (size_t)s * 4) = int4{0, 0, 0, 0};
  __syncthreads();
  for (int k = threadIdx.x; k < pl.K; k += blockDim.x) {
    int s, nmem, j0;
    seg_desc(pl, k, &s, &nmem, &j0);
    const int sb = pl.first(k), se = pl.pre[k + 1];
    int first = 0, np = 0;
    if (se > sb) {
      const int r0 = sb / pl.q;
      first = r0 * 2 + (sb != r0 * pl.q);
      np = (se - 1) / pl.q - r0 + 1;
    }
    int* info = a.seg_info + (size_t)s * 4;
    if (nmem == 1) {
      info[0] = first;
      info[1] = np;
    } else {
      for (int m = 0; m < nmem; ++m) {
        info[4 * m + 2] = first;
        info[4 * m + 3] = np | m << 16;
      }
    }
  }
  // the sequences the reduce must combine (cut, or sharing a group's
  // blocks), in order, as records {s, seg_info[s]} of 8 ints after a
  // header record whose first int is their count
  __syncthreads();
  const int C = (pl.S + blockDim.x - 1) / blockDim.x;
  const int s0 = min(pl.S, (int)threadIdx.x * C), s1 = min(pl.S, s0 + C);
  auto info_of = [&](int s) { return *reinterpret_cast<const int4*>(a.seg_info + (size_t)s * 4); };
  auto needs = [&](const int4& i) { return i.y > 1 || (i.w & 0xffff) > 0; };
  int n = 0;
  for (int s = s0; s < s1; ++s) n += needs(info_of(s));
  int total;
  int at = block_excl_scan(n, pl.wsum, &total);
  for (int s = s0; s < s1; ++s) {
    const int4 i = info_of(s);
    if (!needs(i)) continue;
    int4* rec = reinterpret_cast<int4*>(a.cut_list + 8 * (1 + at++));
    rec[0] = int4{s, i.x, i.y, i.z};
    rec[1] = int4{i.w, 0, 0, 0};
  }
  if (threadIdx.x == 0) a.cut_list[0] = total;
}

// Walk range r for kv head g, calling f(unit) per piece (the part of one
// segment inside the range).  G: query heads per kv head.
template <int B, typename F>
__device__ __forceinline__ void walk_range(const DecodeArgs& a, const Plan& pl, int G, int r, int g,
                                           F&& f) {
  int b0 = r * pl.q;
  const int b1 = min(pl.T, b0 + pl.q);
  if (b0 >= b1) return;
  // segment holding block b0: the largest k with pre[k] <= b0 (then
  // pre[k + 1] > b0 once empty segments are skipped, because b0 < T)
  int lo = 0, hi = pl.K - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pl.pre[mid] <= b0) lo = mid; else hi = mid - 1;
  }
  int k = lo;
  const int rb0 = b0;  // the range's first place
  while (b0 < b1) {
    while (pl.pre[k + 1] <= b0) ++k;  // skip empty segments
    const int sb = pl.first(k), se = pl.pre[k + 1];
    const int e = min(b1, se);
    const int bs = max(b0, sb);  // the piece's first block
    b0 = e;
    if (bs >= e) continue;  // only the segment's empty places fall in the range
    int s, nmem, j0;
    seg_desc(pl, k, &s, &nmem, &j0);
    Unit u;
    u.s = s;
    u.nmem = nmem;
    u.g = g;
    u.t0 = (j0 + bs - sb) * B;
    const int seg_end = nmem > 1 ? (j0 + se - sb) * B : pl.lens[s];
    u.t1 = min(seg_end, (j0 + e - sb) * B);
    u.last = nmem == 1 && u.t1 == seg_end;
    const bool cut = (se - 1) / pl.q != sb / pl.q;
    u.in_place = nmem == 1 && j0 == 0 && !cut;
    if (cut) {
      // partial rows: end 0 for the piece that starts at the range's first
      // place, 1 for the one that starts inside it (at most one of each)
      u.prow = ((r * a.num_kv_heads + g) * 2 + (bs != rb0)) * a.slots;
      u.mstride = G;
    } else {  // one piece: its rows are the sequences' own
      u.prow = (nmem == 1 ? a.own_row0 : a.sh_row0) + s * a.num_q_heads + g * G;
      u.mstride = a.num_q_heads;
    }
    f(u);
  }
}

// Epilogue of an MFMA unit: acc[nt][r] holds head slot 4*grp + r, dim
// nt*16 + col (unnormalised); m_ref and l_tot belong to head slot col.  A
// piece that is a sequence's whole attention is normalised and stored as
// bf16; any other writes (m, l, o) to its partial rows.
template <int D>
__device__ __forceinline__ void finish_mfma_unit(const DecodeArgs& a, int G, const Unit& u,
                                                 const f32x4* acc, float m_ref, float l_tot,
                                                 int lane) {
  constexpr int NT = D / 16;
  const int s = u.s, g = u.g;
  const int col = lane & 15, grp = lane >> 4;
  if (u.in_place) {
    float den[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) den[r] = lane_bcast(l_tot, 4 * grp + r);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      if (h >= G) continue;
      const size_t ob = ((size_t)s * a.num_q_heads + g * G + h) * D + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) store_out<__bf16>(a.out, ob + nt * 16, acc[nt][r] / den[r]);
    }
  } else {
    const int nslot = u.nmem * G;
    auto row = [&](int c) {
      const int m = c / G;
      return u.prow + m * u.mstride + (c - m * G);
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      if (h >= nslot) continue;
      float* po = a.part_o + (size_t)row(h) * D + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) po[nt * 16] = acc[nt][r];
    }
    if (grp == 0 && col < nslot) {
      a.part_m[row(col)] = m_ref;
      a.part_l[row(col)] = l_tot;
    }
  }
}

// B operand of q.K for an MFMA unit: head slot col of the tile is member
// col / G's query head g * G + col % G (zero past the unit's slots); lane
// (col, grp) holds 16 bytes of that row at dims kj * KSTEP + grp * 16 / 2
// in the caller's arrangement: the bytes at qoff(kj) of the row.
template <int KJ, typename Off>
__device__ __forceinline__ void load_q_operand(const DecodeArgs& a, int G, const Unit& u, int col,
                                               uint32_t row_bytes, Off qoff, bf16x8 (&qop)[KJ]) {
  u32x4 w[KJ];
#pragma unroll
  for (int kj = 0; kj < KJ; ++kj) w[kj] = u32x4{0u, 0u, 0u, 0u};
  if (col < u.nmem * G) {
    const int m = col / G, h = col - m * G;
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                        ((size_t)(u.s + m) * a.num_q_heads + u.g * G + h) * row_bytes;
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj) w[kj] = *reinterpret_cast<const u32x4*>(qp + qoff(kj));
  }
#pragma unroll
  for (int kj = 0; kj < KJ; ++kj) qop[kj] = __builtin_bit_cast(bf16x8, w[kj]);
}

// The MFMA tiles cover 16 tokens.  A unit walks its tokens [t0, t1) in
// 16-token tiles: with 16-token blocks a tile is a block; with B = 32 it is
// one half of a block; with B = 8 it is two consecutive blocks of the unit
// (the second one clamped to the first past the unit's last block, and
// masked).  Table entries arrive 64 per lane load ("chunks" of 64 blocks).
template <int B>
struct TileGeom {
  static_assert(B == 8 || B == 16 || B == 32, "block sizes 8, 16 and 32");
  static constexpr int kSub = B >= 16 ? B / 16 : 1;  // tiles per block
  static constexpr int kPer = B >= 16 ? 1 : 16 / B;  // blocks per tile
  // tiles of the chunk of blocks [c0, c0 + cnt) of a unit starting at t0
  __device__ static int tiles(const Unit& u, int c0, int cnt) {
    const int lo = u.t0 + c0 * B;
    const int hi = min(u.t1, u.t0 + (c0 + cnt) * B);
    return (hi - lo + 15) >> 4;
  }
};

// ---------------------------------------------------------------------------
// MFMA kernel: bf16 pools, 1..16 query heads per kv head.
// ---------------------------------------------------------------------------
template <int D, int B, int NBUF, bool STEP>
__device__ __forceinline__ void mfma_unit(const DecodeArgs& a, int G, const Unit& unit, int lane,
                                          const int32_t* step_blk) {
  using TG = TileGeom<B>;
  constexpr int KJ = D / 32;  // q.K MFMAs per tile (32 dims each)
  constexpr int NT = D / 16;  // P.V MFMAs per tile (16 output dims each)
  constexpr uint32_t ROW = D * 2;  // bytes per K row

  const int s = unit.s, g = unit.g;
  const int col = lane & 15, grp = lane >> 4;

  // B operand of q.K: lane holds q[head slot col][kj*32 + grp*8 .. +8]
  bf16x8 qop[KJ];
  load_q_operand<KJ>(a, G, unit, col, ROW, [&](int kj) { return grp * 16 + kj * 64; }, qop);

  // wave-uniform base of this kv head's slice of block 0, plus 32-bit lane
  // offsets: each load is a scalar block base + vector lane offset
  const size_t blk_bytes = (size_t)a.num_kv_heads * B * D * 2;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool) + (size_t)g * B * ROW;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool) + (size_t)g * D * B * 2;
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;

  // A decode step's new token (the sequence's last position p) belongs to
  // the piece that ends the sequence: its K and V come from k_new / v_new
  // and join the attention as one extra tile; the pool tiles stop before
  // p, so they need neither the token's slot nor a given block: a new
  // block holds only p, and a copy-on-write copy holds the same tokens
  // before p as the shared block the table still names.  Other workgroups
  // of the launch store the token and grow the table (step_store).
  Unit u = unit;
  const bool new_tok = STEP && u.last;
  int p_new = 0;
  uint32_t kpre = 0, vpre = 0;  // lane l: dword l of the new token's K row and V row
  if (new_tok) {
    p_new = u.t1 - 1;
    u.t1 = p_new;
    // issued now, so their latency hides behind the piece's pool tiles
    const size_t row_off = ((size_t)s * a.num_kv_heads + g) * ROW;
    if (lane < D / 2) {
      kpre = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.k_new) + row_off)[lane];
      vpre = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.v_new) + row_off)[lane];
    }
  }
  const int jb = u.t0 / B, je = (u.t1 + B - 1) / B;

  // lane offsets inside a tile's block: K row (token) col, V dim col, tokens
  // 4*grp..+4 (with B = 8, rows and tokens are taken modulo the block)
  const uint32_t koff = (B >= 16 ? col : col % 8) * ROW + grp * 16;
  const uint32_t voff = col * (B * 2) + (B >= 16 ? grp : grp % 2) * 8;

  float m_ref = kNegInf, l_run = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One 16-token tile: scores of the tile's tokens (K operand kb), the
  // first `valid` of them live, folded into the running softmax and P.V
  // (V operand vb, 4 tokens of one dim per lane).
  auto tile = [&](const u32x4* kb, u32x2* vb, int valid) {
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[kj]),
                                                   qop[kj], sc, 0, 0, 0);
    // sc[r] = score of token 4*grp + r for head col
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = sc[r] * a.scale_log2;
    // tokens past the valid ones (past the context, or a second block that
    // belongs to another unit) get score -inf and zero V, so stale bits in
    // an unused slot never reach the output
    if (valid < 16) {
      const int t = 4 * grp;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t + r >= valid) x[r] = kNegInf;
      const uint32_t m0 = (t + 0 < valid ? 0x0000ffffu : 0u) | (t + 1 < valid ? 0xffff0000u : 0u);
      const uint32_t m1 = (t + 2 < valid ? 0x0000ffffu : 0u) | (t + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        vb[nt].x &= m0;
        vb[nt].y &= m1;
      }
    }
    // A head's max passes m_ref + kSlack exactly when some lane's own max
    // does, so only the (rare) rescale exchanges values between lanes.
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__ballot(bm > m_ref + kSlack)) {  // rare: move the reference, rescale
      bm = max_xor32(max_xor16(bm));
      const float m_new = fmaxf(m_ref, bm);
      const float alpha = fexp2(m_ref - m_new);
      l_run *= alpha;
      m_ref = m_new;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = lane_bcast(alpha, 4 * grp + r);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] *= ar[r];
    }
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fexp2(x[r] - m_ref);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    // P.V: A = P (16 head slots x this lane's 4 tokens, which are exactly
    // its 4 scores), B = V (the lane's 8-byte V^T load: 4 tokens of one dim)
    const bf16x8 pp = p_split(pr);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, v_twice(vb[nt]), acc[nt], 0, 0, 0);
  };

  // One whole 32-token block (B = 32): two q.K tiles whose MFMA rows take
  // tokens 8 (m / 4) + 4 tau + m % 4, so that a lane's eight scores are
  // tokens 8 grp .. 8 grp + 7, the k entries of its P.V operand; V comes as
  // one 16-byte load per dim (those eight tokens of a dim-major row), and
  // P.V runs twice per 16 dims, on P's high and low bf16 parts (the same
  // precision as p_split).  Every lane reads whole 64-byte V rows and whole
  // K rows, so no line is fetched twice.
  auto tile32 = [&](const u32x4 (*kb)[KJ], u32x4* vb, int valid) {
    f32x4 sc[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      sc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj)
        sc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[tau][kj]),
                                                          qop[kj], sc[tau], 0, 0, 0);
    }
    float x[8];  // token 8 grp + e
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sc[e / 4][e % 4] * a.scale_log2;
    if (valid < 32) {
      const int t = 8 * grp;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (t + e >= valid) x[e] = kNegInf;
      uint32_t m[4];
#pragma unroll
      for (int w = 0; w < 4; ++w)
        m[w] = (t + 2 * w < valid ? 0x0000ffffu : 0u) | (t + 2 * w + 1 < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) vb[nt] = u32x4{vb[nt].x & m[0], vb[nt].y & m[1],
                                                      vb[nt].z & m[2], vb[nt].w & m[3]};
    }
    float bm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    if (__ballot(bm > m_ref + kSlack)) {  // rare: move the reference, rescale
      bm = max_xor32(max_xor16(bm));
      const float m_new = fmaxf(m_ref, bm);
      const float alpha = fexp2(m_ref - m_new);
      l_run *= alpha;
      m_ref = m_new;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = lane_bcast(alpha, 4 * grp + r);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] *= ar[r];
    }
    float pr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[e] = fexp2(x[e] - m_ref);
    l_run += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    // high part: truncation to bf16; low part: the residual, rounded
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a0 = __float_as_uint(pr[2 * w]), a1 = __float_as_uint(pr[2 * w + 1]);
      hi[w] = (a0 >> 16) | (a1 & 0xffff0000u);
      const bf16x2 l2 = {static_cast<__bf16>(pr[2 * w] - bf16_hi(a0)),
                         static_cast<__bf16>(pr[2 * w + 1] - bf16_hi(a1))};
      lo[w] = __builtin_bit_cast(uint32_t, l2);
    }
    const bf16x8 ph = __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
    const bf16x8 pl = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, vb[nt]);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, v, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, v, acc[nt], 0, 0, 0);
    }
  };

  // The new token is scored while the first pool tiles' loads are in
  // flight (block_ring's `pre`), off the end of the piece's serial chain.
  bool new_done = !new_tok;
  auto new_tile = [&]() {
    // The new token as tile token 0.  K operand: lane (col 0, grp) holds
    // dims kj*32 + grp*8 .. +8, i.e. dwords grp*4 + kj*16 + w of the row;
    // V operand: lane (col, grp 0) holds dim nt*16 + col as its token 0,
    // the low or high half of dword dim / 2.  Both come from the
    // prefetched dwords through ds_bpermute.
    u32x4 kb[KJ];
    u32x2 vb[NT];
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj) {
      uint32_t w4[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = __builtin_amdgcn_ds_bpermute((grp * 4 + kj * 16 + w) * 4, kpre);
        w4[w] = col == 0 ? x : 0u;
      }
      kb[kj] = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int dim = nt * 16 + col;
      const uint32_t x = __builtin_amdgcn_ds_bpermute((dim >> 1) * 4, vpre);
      const uint32_t h = (dim & 1) ? x >> 16 : x & 0xffffu;
      vb[nt] = u32x2{grp == 0 ? h : 0u, 0u};
    }
    tile(kb, vb, 1);
    new_done = true;
  };
  auto pre = [&]() {
    if (!new_done) new_tile();
  };

  const int nblk = je - jb;
  if constexpr (B == 32) {
    u32x4 kring[NBUF][2][KJ];
    u32x4 vring[NBUF][NT];
    // lane offsets in a block: K row of MFMA row col in tile tau, dims
    // kj*32 + grp*8 ..; V row of dim col (+ nt*16), tokens 8 grp .. + 7
    const uint32_t krow0 = (8 * (col / 4) + col % 4) * ROW + grp * 16;
    const uint32_t voff32 = col * (B * 2) + grp * 16;
    for (int c0 = 0; c0 < nblk; c0 += 64) {
      const int cnt = min(64, nblk - c0);
      const int tab = trow[jb + c0 + min(lane, cnt - 1)];
      auto load = [&](int i, auto slot) {
        const size_t off = (size_t)__builtin_amdgcn_readlane(tab, i) * blk_bytes;
        const gptr kblk = uniform_ptr(kpool + off);
        const gptr vblk = uniform_ptr(vpool + off);
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int kj = 0; kj < KJ; ++kj)
            kring[slot][tau][kj] = ldg_stream<u32x4>(kblk + krow0 + tau * 4 * ROW + kj * 64);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          vring[slot][nt] = ldg_stream<u32x4>(vblk + voff32 + nt * 16 * (B * 2));
      };
      // units start on block boundaries (pieces are ranges of whole blocks)
      auto compute = [&](int i, auto slot) {
        tile32(kring[slot], vring[slot], u.t1 - (u.t0 + (c0 + i) * B));
      };
      block_ring<NBUF>(cnt, load, compute, pre);
    }
  } else {
  u32x4 kring[NBUF][KJ];
  u32x2 vring[NBUF][NT];

  for (int c0 = 0; c0 < nblk; c0 += 64) {
    const int cnt = min(64, nblk - c0);
    // physical block ids of up to 64 blocks, one per lane (every lane loads a
    // valid entry); the new token's block as the step decided it
    const int tab = trow[jb + c0 + min(lane, cnt - 1)];
    const int ntile = TG::tiles(u, c0, cnt);

    auto load = [&](int i, auto slot) {
      if constexpr (B >= 16) {
        // tile i: part i % kSub of block i / kSub (tokens 16 * part ...)
        const int part = i % TG::kSub;
        const size_t off = (size_t)__builtin_amdgcn_readlane(tab, i / TG::kSub) * blk_bytes;
        const gptr kblk = uniform_ptr(kpool + off + part * 16 * ROW);
        const gptr vblk = uniform_ptr(vpool + off + part * 32);
#pragma unroll
        for (int kj = 0; kj < KJ; ++kj)
          kring[slot][kj] = ldg_stream<u32x4>(kblk + koff + kj * 64);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          vring[slot][nt] = ldg_v<B, u32x2>(vblk + voff + nt * 16 * (B * 2));
      } else {
        // tile i: blocks 2i and 2i + 1; K row col and V tokens 4*grp.. come
        // from the block that holds them
        const int b0 = __builtin_amdgcn_readlane(tab, 2 * i);
        const int b1 = __builtin_amdgcn_readlane(tab, min(2 * i + 1, cnt - 1));
        const gptr kblk = to_global(kpool) + (size_t)(col < 8 ? b0 : b1) * blk_bytes;
        const gptr vblk = to_global(vpool) + (size_t)(grp < 2 ? b0 : b1) * blk_bytes;
#pragma unroll
        for (int kj = 0; kj < KJ; ++kj)
          kring[slot][kj] = ldg_stream<u32x4>(kblk + koff + kj * 64);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          vring[slot][nt] = ldg_stream<u32x2>(vblk + voff + nt * 16 * (B * 2));
      }
    };
    auto compute = [&](int i, auto slot) {
      tile(kring[slot], vring[slot], u.t1 - (u.t0 + c0 * B + i * 16));
    };

    block_ring<NBUF>(ntile, load, compute, pre);
  }
  }

  if (!new_done) new_tile();  // a piece with no pool tiles

  // l over the four lane groups holding the same head; m_ref is uniform
  float l_tot = sum_xor16(l_run);
  l_tot = sum_xor32(l_tot);
  finish_mfma_unit<D>(a, G, u, acc, m_ref, l_tot, lane);
}

// ---------------------------------------------------------------------------
// MFMA kernel for 8-bit pools: per (block, kv head) a K region of E4M3 codes
// ([16][D] token-major) followed by bf16 scales (per group of 4 tokens, 4 K
// scales then 4 V scales) and a V region of codes ([D][16] dim-major).
// Codes widen to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1), so
// the bf16 MFMAs of the kernel above do the products; the per-token scales
// are applied where each token has one value per lane: the K scale on its
// score, the V scale on its probability.  Per block and lane (D = 128): two
// 16-byte K code loads, one 16-byte load holding the K and V scales of the
// lane's 4 tokens, and two 16-byte V code loads.
// Load shape matters more than bytes at this granularity: a wave-wide load
// that covers 1 KB contiguously streams 2 KB regions about 15% faster than
// eight 4-byte-per-lane loads of 256 B each (measured on random 2 KB
// chunks).  So V is read contiguously -- lane l gets the 16 tokens of one
// dim -- and a 4x4 transpose between the four 16-lane rows and four
// registers (v_permlane32_swap, then v_permlane16_swap) turns that into the
// MFMA operand layout, 4 tokens of a dim per lane.
// ---------------------------------------------------------------------------
// 4x4 transpose between the four 16-lane rows of a wave and four registers:
// on return r[t] in row g holds what r[g] held in row t.
__device__ __forceinline__ void transpose_rows4(uint32_t& r0, uint32_t& r1, uint32_t& r2,
                                                uint32_t& r3) {
  // rows {2,3} of r0 <-> rows {0,1} of r2, and of r1 <-> r3
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  // odd rows of the first <-> even rows of the second
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = e[0];
  r3 = e[1];
}

// Four E4M3 codes (one dword, lowest byte first) -> four bf16.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

template <int D, int B, int NBUF, bool STEP>
__device__ __forceinline__ void mfma8_unit(const DecodeArgs& a, int G, const Unit& unit, int lane,
                                           uint8_t* nts) {
  using TG = TileGeom<B>;
  constexpr int KC = D / 64;              // 16-byte K code loads per lane per block
  constexpr int VC = D / 64;              // 16-byte V code loads per lane per block
  constexpr int KJ = D / 32;              // q.K MFMAs per block
  constexpr int NT = D / 16;              // P.V MFMAs per block
  constexpr uint32_t QROW = D * 2;         // bytes per bf16 q row
  constexpr uint32_t SOFF = B * D;         // offset of the scales in a K region

  // A decode step's new token (the sequence's last position) joins the
  // piece that ends the sequence as one extra tile, quantised here exactly
  // as the slot write quantises it (the reduce kernel that follows stores
  // those codes and scales); the pool tiles stop before it.
  Unit u = unit;
  const bool new_tok = STEP && u.last;
  uint32_t kpre = 0, vpre = 0;  // lane l: dword l (dims 2l, 2l + 1) of the token's K and V rows
  if (new_tok) {
    u.t1 -= 1;
    // issued now, so their latency hides behind the piece's pool tiles
    const size_t row_off = ((size_t)u.s * a.num_kv_heads + u.g) * QROW;
    if (lane < D / 2) {
      kpre = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.k_new) + row_off)[lane];
      vpre = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.v_new) + row_off)[lane];
    }
  }
  const int s = u.s, g = u.g;
  const int jb = u.t0 / B, je = (u.t1 + B - 1) / B;
  const int col = lane & 15, grp = lane >> 4;

  // K codes: lane loads token col, dims c*64 + grp*16 .. +16 (c < KC).  MFMA
  // kj = 2c + h takes the h-th 8 of those 16 dims, so the q operand of step
  // kj holds q[head col][c*64 + grp*16 + h*8 .. +8].  The order in which
  // dims meet the MFMA does not change the dot product.
  bf16x8 qop[KJ];
  load_q_operand<KJ>(a, G, u, col, QROW,
                     [&](int kj) { return grp * 32 + (kj >> 1) * 128 + (kj & 1) * 16; }, qop);

  // regions (block b, kv head g) at (b * H + g) * stride: R_k / R_v for two
  // buffers, R_k + R_v when K and V regions alternate in one buffer (one
  // contiguous read of a block's K and V per kv head)
  const size_t kblk_bytes = (size_t)a.num_kv_heads * a.k_rstride;
  const size_t vblk_bytes = (size_t)a.num_kv_heads * a.v_rstride;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool) + (size_t)g * a.k_rstride;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool) + (size_t)g * a.v_rstride;
  // K row (token) col; scales of tokens 4*grp..+4 (with B = 8, rows and
  // scale groups are taken modulo the block); V: load h gives lane l the 16
  // tokens of dim h*64 + l (two 8-token halves with B = 8)
  const uint32_t koff = (B >= 16 ? col : col % 8) * D + grp * 16;
  const uint32_t soff = SOFF + (B >= 16 ? grp : grp % 2) * 16;
  const uint32_t voff = lane * B;
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;

  float m_ref = kNegInf, l_run = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 kring[NBUF][KC];
  u32x4 sring[NBUF];
  u32x4 vring[NBUF][VC];

  // one 16-token tile: scores, softmax, P.V; `valid` = its leading tokens
  // inside the unit (the rest masked)
  auto tile8 = [&](const u32x4* kr, const u32x4& sw_in, const u32x4* vr, int valid) {
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 w = kr[c];
      const u32x2 k0 = e4m3x4_to_bf16(w.x), k1 = e4m3x4_to_bf16(w.y);
      const u32x2 k2 = e4m3x4_to_bf16(w.z), k3 = e4m3x4_to_bf16(w.w);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, u32x4{k0.x, k0.y, k1.x, k1.y}), qop[2 * c], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, u32x4{k2.x, k2.y, k3.x, k3.y}), qop[2 * c + 1], sc, 0, 0,
          0);
    }
    // scales of tokens 4*grp + r: bf16 pairs, K in words x, y and V in z, w
    const u32x4 sw = sw_in;
    const f32x4 ks = {__uint_as_float(sw.x << 16), bf16_hi(sw.x), __uint_as_float(sw.y << 16),
                      bf16_hi(sw.y)};
    f32x4 vs = {__uint_as_float(sw.z << 16), bf16_hi(sw.z), __uint_as_float(sw.w << 16),
                bf16_hi(sw.w)};
    // load h, row r held dim h*64 + r*16 + col (tile 4h + r), token group j
    // in word j; after the transpose word t of row g is tile 4h + t, tokens
    // 4g .. 4g + 3 of dim col: the B operand layout of P.V
    uint32_t vb[NT];
#pragma unroll
    for (int h = 0; h < VC; ++h) {
      uint32_t w0 = vr[h].x, w1 = vr[h].y, w2 = vr[h].z, w3 = vr[h].w;
      transpose_rows4(w0, w1, w2, w3);
      vb[4 * h + 0] = w0;
      vb[4 * h + 1] = w1;
      vb[4 * h + 2] = w2;
      vb[4 * h + 3] = w3;
    }
    // sc[r] = code-level score of token 4*grp + r for head col
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = sc[r] * ks[r] * a.scale_log2;
    if (valid < 16) {
      // slots past the context: score -inf, V codes and scale zeroed
      const int t = 4 * grp;
      uint32_t m = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (t + r >= valid) {
          x[r] = kNegInf;
          vs[r] = 0.f;
        } else {
          m |= 0xffu << (8 * r);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) vb[nt] &= m;
    }
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__ballot(bm > m_ref + kSlack)) {  // rare: as in mfma_unit
      bm = max_xor32(max_xor16(bm));
      const float m_new = fmaxf(m_ref, bm);
      const float alpha = fexp2(m_ref - m_new);
      l_run *= alpha;
      m_ref = m_new;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = lane_bcast(alpha, 4 * grp + r);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] *= ar[r];
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fexp2(x[r] - m_ref);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    // the V scale rides on the probability: o += (p * s_v) * code
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] *= vs[r];
    const bf16x8 pp = p_split(p);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, v_twice(e4m3x4_to_bf16(vb[nt])),
                                                        acc[nt], 0, 0, 0);
  };

  // The new token as tile token 0: quantised (scale = bf16(max|x| / 448),
  // codes = E4M3(x / scale), nearest even), the codes passed through this
  // wave's LDS scratch into the tile's operand layout: K codes of token 0
  // for lanes (col 0, grp), V code of dim h*64 + lane for every lane, the
  // two scales in the lanes of token group 0.
  bool new_done = !new_tok;
  auto new_tile = [&]() {
    auto quant = [&](uint32_t w, uint16_t* sbits) {
      const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xffff0000u);
      // from 0, as the slot write: NaN inputs are skipped by fmaxf
      const float am = wave_max(fmaxf(0.f, fmaxf(fabsf(x0), fabsf(x1))));
      const __bf16 sb = static_cast<__bf16>(am / 448.f);
      const float sc = static_cast<float>(sb);
      *sbits = __builtin_bit_cast(uint16_t, sb);
      const uint32_t c0 = sc > 0.f ? (__builtin_amdgcn_cvt_pk_fp8_f32(x0 / sc, 0.f, 0, false) & 0xffu) : 0u;
      const uint32_t c1 = sc > 0.f ? (__builtin_amdgcn_cvt_pk_fp8_f32(x1 / sc, 0.f, 0, false) & 0xffu) : 0u;
      return static_cast<uint16_t>(c0 | (c1 << 8));
    };
    uint16_t ksb, vsb;
    const uint16_t kc = quant(kpre, &ksb), vc = quant(vpre, &vsb);
    if (lane < D / 2) {
      reinterpret_cast<uint16_t*>(nts)[lane] = kc;
      reinterpret_cast<uint16_t*>(nts + D)[lane] = vc;
    }
    u32x4 kr[KC], vr[VC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(nts + c * 64 + grp * 16);
      kr[c] = col == 0 ? x : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int h = 0; h < VC; ++h) vr[h] = u32x4{(uint32_t)nts[D + h * 64 + lane], 0u, 0u, 0u};
    const u32x4 sw = grp == 0 ? u32x4{(uint32_t)ksb, 0u, (uint32_t)vsb, 0u} : u32x4{0u, 0u, 0u, 0u};
    tile8(kr, sw, vr, 1);
    new_done = true;
  };
  auto pre = [&]() {
    if (!new_done) new_tile();
  };

  const int nblk = je - jb;
  for (int c0 = 0; c0 < nblk; c0 += 64) {
    const int cnt = min(64, nblk - c0);
    const int tab = trow[jb + c0 + min(lane, cnt - 1)];

    const int ntile = TG::tiles(u, c0, cnt);

    auto load = [&](int i, auto slot) {
      if constexpr (B >= 16) {
        // tile i: part i % kSub of block i / kSub
        const int part = i % TG::kSub;
        const size_t b = (size_t)__builtin_amdgcn_readlane(tab, i / TG::kSub);
        const gptr kblk = uniform_ptr(kpool + b * kblk_bytes + part * 16 * D);
        const gptr vblk = uniform_ptr(vpool + b * vblk_bytes + part * 16);
#pragma unroll
        for (int c = 0; c < KC; ++c) kring[slot][c] = ldg_stream<u32x4>(kblk + koff + c * 64);
        sring[slot] = ldg_stream<u32x4>(kblk - part * 16 * D + soff + part * 64);
#pragma unroll
        for (int h = 0; h < VC; ++h) vring[slot][h] = ldg_v<B, u32x4>(vblk + voff + h * 64 * B);
      } else {
        // tile i: blocks 2i and 2i + 1
        const int b0 = __builtin_amdgcn_readlane(tab, 2 * i);
        const int b1 = __builtin_amdgcn_readlane(tab, min(2 * i + 1, cnt - 1));
        const gptr kblk = to_global(kpool) + (size_t)(col < 8 ? b0 : b1) * kblk_bytes;
        const gptr sblk = to_global(kpool) + (size_t)(grp < 2 ? b0 : b1) * kblk_bytes;
        const gptr vb0 = uniform_ptr(vpool + (size_t)b0 * vblk_bytes);
        const gptr vb1 = uniform_ptr(vpool + (size_t)b1 * vblk_bytes);
#pragma unroll
        for (int c = 0; c < KC; ++c) kring[slot][c] = ldg_stream<u32x4>(kblk + koff + c * 64);
        sring[slot] = ldg_stream<u32x4>(sblk + soff);
#pragma unroll
        for (int h = 0; h < VC; ++h) {
          const u32x2 lo = ldg_stream<u32x2>(vb0 + voff + h * 64 * B);
          const u32x2 hi = ldg_stream<u32x2>(vb1 + voff + h * 64 * B);
          vring[slot][h] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    };

    auto compute = [&](int i, auto slot) {
      tile8(kring[slot], sring[slot], vring[slot], u.t1 - (u.t0 + c0 * B + i * 16));
    };

    block_ring<NBUF>(ntile, load, compute, pre);
  }

  if (!new_done) new_tile();  // a piece with no pool tiles
  float l_tot = sum_xor16(l_run);
  l_tot = sum_xor32(l_tot);
  finish_mfma_unit<D>(a, G, u, acc, m_ref, l_tot, lane);
}

// A decode step's stores, by the reduce kernel that follows the decode
// kernel (the decode took the new tokens from k_new / v_new and never
// reads their slots; the next step reads them): each new token's K and V
// rows go to its slot, every kv head, non-temporal like the slot write; a
// given block becomes the table entry of the token's position; the
// lengths after the step go to lens_out.  The stores are spread over every
// thread of the grid, at most one 16-byte K piece and one V element each,
// so no thread's reduce work waits behind a run of its own stores.
template <int D, int B>
__device__ void step_store(const DecodeArgs& a, const int32_t* step_blk) {
  constexpr int ROW = D * 2;
  constexpr int KP = ROW / 16;  // 16-byte pieces of a K row
  const int H = a.num_kv_heads;
  const size_t blk_bytes = (size_t)H * B * ROW;
  const size_t nt = (size_t)gridDim.x * blockDim.x;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  auto slot_of = [&](int s, int* r) {  // the new token's block and row of sequence s
    const int L = min(max(a.context_lens[s], 0), a.max_blocks * B - 1);
    *r = L % B;
    const int given = step_blk[s];
    return given >= 0 ? given : a.tables_w[(size_t)s * a.max_blocks + L / B];
  };
  for (size_t i = t; i < (size_t)a.num_seqs * H * KP; i += nt) {  // K: [g][r][:] per head
    const int s = (int)(i / (H * KP)), c = (int)(i % (H * KP));
    const int g = c / KP, off = (c % KP) * 16;
    int r;
    const int blk = slot_of(s, &r);
    __builtin_nontemporal_store(
        *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.k_new) + (size_t)s * H * ROW +
                                        (size_t)c * 16),
        reinterpret_cast<u32x4*>(static_cast<uint8_t*>(const_cast<void*>(a.k_pool)) +
                                 (size_t)blk * blk_bytes + ((size_t)g * B + r) * ROW + off));
  }
  for (size_t i = t; i < (size_t)a.num_seqs * H * D; i += nt) {  // V: [g][d][r] per element
    const int s = (int)(i / (H * D)), c = (int)(i % (H * D));
    int r;
    const int blk = slot_of(s, &r);
    __builtin_nontemporal_store(
        reinterpret_cast<const uint16_t*>(a.v_new)[(size_t)s * H * D + c],
        reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(const_cast<void*>(a.v_pool)) +
                                    (size_t)blk * blk_bytes) + (size_t)c * B + r);
  }
  // table entries and lengths last: the loops above read the entries that
  // no given block replaces, and these writes touch only the given ones
  for (size_t s = t; s < (size_t)a.num_seqs; s += nt) {
    const int L = min(max(a.context_lens[s], 0), a.max_blocks * B - 1);
    if (step_blk[s] >= 0) a.tables_w[s * a.max_blocks + L / B] = step_blk[s];
    a.lens_out[s] = L + 1;
  }
}

// The 8-bit pool's version: the new token's codes and scales, quantised
// as the slot write quantises, into its slot of the K and V regions; table
// entry and length as above.  One wave per (sequence, kv head, K or V) row,
// over every wave of the grid, so no wave takes rows one after another
// (each is a load, a wave max and a few stores); lane l takes dims 2l and
// 2l + 1.
template <int D, int B>
__device__ void step_store8(const DecodeArgs& a, const int32_t* step_blk) {
  const int H = a.num_kv_heads;
  const int nwv = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * nwv + (threadIdx.x >> 6), ngw = gridDim.x * nwv;
  for (int row = gw; row < a.num_seqs * 2 * H; row += ngw) {
    const int s = row / (2 * H), k = row % (2 * H);
    const bool is_v = k >= H;
    const int g = is_v ? k - H : k;
    const int L = min(max(a.context_lens[s], 0), a.max_blocks * B - 1);  // position of the new token
    const int j = L / B, r = L % B;
    const int given = step_blk[s];
    int32_t* entry = a.tables_w + (size_t)s * a.max_blocks + j;
    const int blk = given >= 0 ? given : *entry;  // read only when nothing writes it
    if (k == 0 && lane == 0) {
      if (given >= 0) *entry = given;
      a.lens_out[s] = L + 1;
    }
    const uint8_t* src = static_cast<const uint8_t*>(is_v ? a.v_new : a.k_new) +
                         ((size_t)s * H + g) * D * 2;
    const uint32_t w = lane < D / 2 ? reinterpret_cast<const uint32_t*>(src)[lane] : 0u;
    const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xffff0000u);
    // from 0, as the slot write: NaN inputs are skipped by fmaxf
    const float amax = wave_max(fmaxf(0.f, fmaxf(fabsf(x0), fabsf(x1))));
    const __bf16 sb = static_cast<__bf16>(amax / 448.f);
    const float scale = static_cast<float>(sb);
    const uint32_t c0 = scale > 0.f ? (__builtin_amdgcn_cvt_pk_fp8_f32(x0 / scale, 0.f, 0, false) & 0xffu) : 0u;
    const uint32_t c1 = scale > 0.f ? (__builtin_amdgcn_cvt_pk_fp8_f32(x1 / scale, 0.f, 0, false) & 0xffu) : 0u;
    uint8_t* kreg =
        static_cast<uint8_t*>(const_cast<void*>(a.k_pool)) + ((size_t)blk * H + g) * a.k_rstride;
    uint8_t* vreg =
        static_cast<uint8_t*>(const_cast<void*>(a.v_pool)) + ((size_t)blk * H + g) * a.v_rstride;
    if (lane < D / 2) {
      if (is_v) {
        __builtin_nontemporal_store(static_cast<uint8_t>(c0), vreg + (size_t)(2 * lane) * B + r);
        __builtin_nontemporal_store(static_cast<uint8_t>(c1), vreg + (size_t)(2 * lane + 1) * B + r);
      } else {
        __builtin_nontemporal_store(static_cast<uint16_t>(c0 | (c1 << 8)),
                                    reinterpret_cast<uint16_t*>(kreg + (size_t)r * D) + lane);
      }
    }
    if (lane == 0)
      __builtin_nontemporal_store(
          __builtin_bit_cast(uint16_t, sb),
          reinterpret_cast<uint16_t*>(kreg + (size_t)B * D + 16u * (r / 4) + 8u * is_v) + (r % 4));
  }
}

template <int D, int B, int NBUF, bool STEP>
__device__ __forceinline__ void decode_mfma_body(const DecodeArgs& a, int G,
                                                 const int32_t* step_blk) {
  extern __shared__ int plan_lds[];
  const Plan pl = build_plan<B>(a, G, plan_lds);
  // one workgroup past the decode grid lists the pieces for the reduce; the
  // grid's workgroups only stream their ranges (none of them is delayed)
  if ((int)blockIdx.x == a.decode_wgs) {
    write_seg_info(a, pl);
    return;
  }
  // the wave index is uniform: keep it (and everything derived) in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int g, r;
  if (!wave_work(a, pl, wave, &g, &r)) return;
  walk_range<B>(a, pl, G, r, g, [&](const Unit& u) {
    mfma_unit<D, B, NBUF, STEP>(a, G, u, lane, step_blk);
  });
}

template <int D, int B, int NBUF>
__global__ __launch_bounds__(kWaves * 64, B == 32 ? 1 : PA_MFMA_MIN_WG) void decode_mfma_kernel(
    DecodeArgs a, int G) {
  decode_mfma_body<D, B, NBUF, false>(a, G, nullptr);
}

// A decode step: the new tokens' blocks arrive with the kernel arguments.
template <int D, int B, int NBUF>
__global__ __launch_bounds__(kWaves * 64, B == 32 ? 1 : PA_MFMA_MIN_WG) void decode_step_kernel(
    DecodeArgs a, int G, StepBlocks nb) {
  decode_mfma_body<D, B, NBUF, true>(a, G, nb.blk);
}

template <int D, int B, int NBUF, bool STEP>
__device__ __forceinline__ void decode_mfma8_body(const DecodeArgs& a, int G, uint8_t* nts) {
  extern __shared__ int plan_lds[];
  const Plan pl = build_plan<B, kSegStart8>(a, G, plan_lds);
  // one workgroup past the decode grid lists the pieces for the reduce; the
  // grid's workgroups only stream their ranges (none of them is delayed)
  if ((int)blockIdx.x == a.decode_wgs) {
    write_seg_info(a, pl);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int g, r;
  if (!wave_work(a, pl, wave, &g, &r)) return;
  uint8_t* wnts = STEP ? nts + wave * 2 * D : nullptr;
  walk_range<B>(a, pl, G, r, g,
                [&](const Unit& u) { mfma8_unit<D, B, NBUF, STEP>(a, G, u, lane, wnts); });
}

template <int D, int B, int NBUF>
__global__ __launch_bounds__(kWaves * 64, PA_MFMA_MIN_WG) void decode_mfma8_kernel(DecodeArgs a, int G) {
  decode_mfma8_body<D, B, NBUF, false>(a, G, nullptr);
}

// A decode step over an 8-bit pool: each wave's LDS scratch takes the new
// token's codes (K, then V) on their way into the tile's operand layout.
template <int D, int B, int NBUF>
__global__ __launch_bounds__(kWaves * 64, PA_MFMA_MIN_WG) void decode_step8_kernel(DecodeArgs a, int G) {
  __shared__ __attribute__((aligned(16))) uint8_t nts[kWaves * 2 * D];
  decode_mfma8_body<D, B, NBUF, true>(a, G, nts);
}

// ---------------------------------------------------------------------------
// VALU kernel: fp32 pools, G (template) query heads per kv head.
// ---------------------------------------------------------------------------
template <int D, int G, int NBUF>
__device__ __forceinline__ void valu_unit(const DecodeArgs& a, const Unit& u, int lane) {
  constexpr int B = kBlock;
  constexpr int ES = 4;
  constexpr int NC = D / 16;          // 16-byte q.K chunks per lane (4 lanes per token)
  constexpr int QW = NC * 4;          // 32-bit words of q per head per lane
  constexpr int EPL = D / 64;         // output dims per lane
  constexpr int NV = EPL * B * ES / 16;  // 16-byte V loads per lane
  constexpr uint32_t ROW = D * ES;

  const int s = u.s, g = u.g, L = u.t1;  // tokens past the piece are masked
  const int jb = u.t0 / B, je = (u.t1 + B - 1) / B;
  const int tok = lane >> 2, qc = lane & 3;

  // q words: chunk (jj*4 + qc) of each head's row
  uint32_t qw[G][QW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                        ((size_t)s * a.num_q_heads + g * G + h) * ROW + qc * 16;
#pragma unroll
    for (int jj = 0; jj < NC; ++jj) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qp + jj * 64);
      qw[h][jj * 4 + 0] = w.x;
      qw[h][jj * 4 + 1] = w.y;
      qw[h][jj * 4 + 2] = w.z;
      qw[h][jj * 4 + 3] = w.w;
    }
  }

  // g counts head groups; kv_div of them share one kv head of the pool
  const int div = a.kv_div > 1 ? a.kv_div : 1;
  const size_t blk_bytes = (size_t)(a.num_kv_heads / div) * B * ROW;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool) + (size_t)(g / div) * B * ROW;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool) + (size_t)(g / div) * B * ROW;
  const uint32_t koff = tok * ROW + qc * 16;
  const uint32_t voff = lane * (EPL * B * ES);
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;

  float m_ref[G], l_run[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_ref[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  u32x4 kring[NBUF][NC], vring[NBUF][NV];

  const int nblk = je - jb;
  for (int c0 = 0; c0 < nblk; c0 += 64) {
    const int cnt = min(64, nblk - c0);
    const int tab = trow[jb + c0 + min(lane, cnt - 1)];

    auto load = [&](int i, auto slot) {
      const size_t off = (size_t)__builtin_amdgcn_readlane(tab, i) * blk_bytes;
      const gptr kblk = uniform_ptr(kpool + off);
      const gptr vblk = uniform_ptr(vpool + off);
#pragma unroll
      for (int jj = 0; jj < NC; ++jj) kring[slot][jj] = ldg_stream<u32x4>(kblk + koff + jj * 64);
#pragma unroll
      for (int v = 0; v < NV; ++v) vring[slot][v] = ldg_stream<u32x4>(vblk + voff + v * 16);
    };

    auto compute = [&](int i, auto slot) {
      const u32x4* kb = kring[slot];
      u32x4* vb = vring[slot];
      const int valid = L - (jb + c0 + i) * B;
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int jj = 0; jj < NC; ++jj) {
          const uint32_t kw[4] = {kb[jj].x, kb[jj].y, kb[jj].z, kb[jj].w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float t = fmaf(__uint_as_float(kw[w]), __uint_as_float(qw[h][jj * 4 + w]),
                                 (w & 1) ? d1 : d0);
            if (w & 1) d1 = t; else d0 = t;
          }
        }
        float d = d0 + d1;
        d += dpp<kQuadXor1>(d);
        d += dpp<kQuadXor2>(d);
        sc[h] = d * a.scale_log2;
      }
      if (valid < B) {
        // slots past the context: score -inf, V zeroed
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (tok >= valid) sc[h] = kNegInf;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          uint32_t* w = reinterpret_cast<uint32_t*>(&vb[v]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // word q of load v holds token (v*4 + q) % 16 of its V^T row
            if ((v * 4 + q) % B >= valid) w[q] = 0u;
          }
        }
      }
      // a head's max passes m_ref + kSlack exactly when some lane's score
      // does; the max over the wave is taken only in the rare branch
      bool move = false;
#pragma unroll
      for (int h = 0; h < G; ++h) move |= sc[h] > m_ref[h] + kSlack;
      if (__ballot(move)) {  // rare: move the references, rescale
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float bm = fmaxf(sc[h], dpp<kRowRor4>(sc[h]));
          bm = fmaxf(bm, dpp<kRowRor8>(bm));
          bm = max_xor32(max_xor16(bm));
          const float m_new = fmaxf(m_ref[h], bm);
          const float alpha = fexp2(m_ref[h] - m_new);
          m_ref[h] = m_new;
          l_run[h] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        }
      }
      float p[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        p[h] = fexp2(sc[h] - m_ref[h]);
        l_run[h] += qc == 0 ? p[h] : 0.f;
      }
      // P.V: element e of this lane is V^T row lane*EPL + e, 16 tokens
#pragma unroll
      for (int t = 0; t < B; ++t) {
        float pt[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          pt[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[h]), 4 * t));
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          // word within this lane's V bytes: row e, token t
          const float vv = __uint_as_float(reinterpret_cast<const uint32_t*>(vb)[e * B + t]);
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pt[h], vv, acc[h][e]);
        }
      }
    };

    block_ring<NBUF>(cnt, load, compute);
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lt = wave_sum(l_run[h]);
    const int hq = g * G + h;
    if (u.in_place) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        store_out<float>(a.out, ((size_t)s * a.num_q_heads + hq) * D + lane * EPL + e, acc[h][e] / lt);
    } else {
      const size_t pi = (size_t)u.prow + h;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a.part_o[pi * D + lane * EPL + e] = acc[h][e];
      if (lane == 0) {
        a.part_m[pi] = m_ref[h];
        a.part_l[pi] = lt;
      }
    }
  }
}

template <int D, int G, int NBUF>
__global__ __launch_bounds__(kWaves * 64) void decode_valu_kernel(DecodeArgs a) {
  extern __shared__ int plan_lds[];
  const Plan pl = build_plan<kBlock>(a, G, plan_lds);
  // one workgroup past the decode grid lists the pieces for the reduce; the
  // grid's workgroups only stream their ranges (none of them is delayed)
  if ((int)blockIdx.x == a.decode_wgs) {
    write_seg_info(a, pl);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int g, r;
  if (!wave_work(a, pl, wave, &g, &r)) return;
  walk_range<kBlock>(a, pl, G, r, g, [&](const Unit& u) { valu_unit<D, G, NBUF>(a, u, lane); });
}

// ---------------------------------------------------------------------------
// Split-context reduce: one wave per (query head, sequence), four query
// heads per workgroup.  A sequence's pieces are those of its own segment
// and, in a prefix group, those of the group's shared segment; seg_info
// says in which ranges they lie.  A wave reads the pieces' m values across
// lanes for the maximum, then walks the pieces 16 at a time (their (m, l)
// as uniform loads, o as 256-byte rows) so that a long sequence's pieces
// are fetched in a few rounds; lanes own output dims.  Sequences finished
// in place by the decode kernel return at once.
// ---------------------------------------------------------------------------
constexpr int kReduceHeads = 4;

// Partial row of piece p of a sequence: pieces [0, np_own) are its own
// segment's (head slot h), the rest the shared segment's (head slot
// member * G + h).  A segment of one piece left its row among the
// sequences' own rows.  Of a cut segment, the first piece may end its range
// (end 1); every later piece starts its range (end 0).
struct PieceMap {
  int first_own, np_own, first_sh, np_sh, slot_sh, slot_own, hkv, slots, g;
  int own_row, sh_row;  // rows of a segment that was not cut
  __device__ __forceinline__ int row(int p) const {
    const bool own = p < np_own;
    if ((own ? np_own : np_sh) == 1) return own ? own_row : sh_row;
    const int i = own ? p : p - np_own;
    const int first = own ? first_own : first_sh;
    const int r = (first >> 1) + i;
    const int end = i == 0 ? (first & 1) : 0;
    return ((r * hkv + g) * 2 + end) * slots + (own ? slot_own : slot_sh);
  }
};

// One (sequence, query head) of the reduce, over the pieces 16 at a time
// with a running reference: M = max of the pieces' references so far, and
// out = sum 2^(m_p - M) o_p / sum 2^(m_p - M) l_p (the sums rescaled when M
// moves).  A sequence has at most a few pieces, so one round of loads.
template <typename T, int D, int EPL, int UNR>
__device__ __forceinline__ void reduce_one(const DecodeArgs& a, int s, const int4 info, int hq,
                                           int G, int lane) {
  const int np_sh = info.w & 0xffff;
  const int np = info.y + np_sh;
  const int g = hq / G, h = hq - g * G;
  const int srow = s * a.num_q_heads + hq;
  const PieceMap pm{info.x, info.y, info.z, np_sh, (info.w >> 16) * G + h, h, a.num_kv_heads,
                    a.slots, g, a.own_row0 + srow, a.sh_row0 + srow};
  float M = kNegInf, den = 0.f, num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  for (int p0 = 0; p0 < np; p0 += UNR) {
    float m[UNR], l[UNR], o[UNR][EPL];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int row = pm.row(min(p0 + k, np - 1));  // clamped: past-the-end terms get f = 0
      m[k] = p0 + k < np ? a.part_m[row] : kNegInf;
      l[k] = a.part_l[row];
      const float* po = a.part_o + (size_t)row * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[k][e] = po[e * 64 + lane];
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < UNR; ++k) Mn = fmaxf(Mn, m[k]);
    const float alpha = M == kNegInf ? 0.f : fexp2(M - Mn);
    den *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] *= alpha;
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const float f = m[k] == kNegInf ? 0.f : fexp2(m[k] - Mn);
      den = fmaf(f, l[k], den);
#pragma unroll
      for (int e = 0; e < EPL; ++e) num[e] = fmaf(f, o[k][e], num[e]);
    }
    M = Mn;
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    store_out<T>(a.out, ((size_t)s * a.num_q_heads + hq) * D + e * 64 + lane, num[e] * inv);
}

template <typename T, int D>
__device__ __forceinline__ void decode_reduce_body(const DecodeArgs& a) {
  constexpr int EPL = D / 64, UNR = 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  // the records sit past the header; a record past the count holds stale
  // data that is loaded (in bounds) but not used
  const int cap = a.num_seqs * Hq;
  for (int i = blockIdx.x * kReduceHeads + wave; i < cap; i += gridDim.x * kReduceHeads) {
    const int4* rec = reinterpret_cast<const int4*>(a.cut_list + 8 * (1 + i / Hq));
    const int4 r0 = rec[0], r1 = rec[1];
    if (i >= a.cut_list[0] * Hq) break;
    // most sequences have one or two pieces (a grouped member: its own
    // blocks' and its group's shared blocks'): load just those
    const int np = r0.z + (r1.x & 0xffff);
    const int4 info{r0.y, r0.z, r0.w, r1.x};
    if (np <= 2)
      reduce_one<T, D, EPL, 2>(a, r0.x, info, i % Hq, G, lane);
    else if (np <= 4)
      reduce_one<T, D, EPL, 4>(a, r0.x, info, i % Hq, G, lane);
    else
      reduce_one<T, D, EPL, UNR>(a, r0.x, info, i % Hq, G, lane);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kReduceHeads * 64) void decode_reduce_kernel(DecodeArgs a) {
  decode_reduce_body<T, D>(a);
}

// A decode step's reduce: first the step's stores (independent of the
// reduce), then the reduce.
template <int D, int B>
__global__ __launch_bounds__(kReduceHeads * 64) void decode_reduce_step_kernel(DecodeArgs a,
                                                                               StepBlocks nb) {
  step_store<D, B>(a, nb.blk);
  decode_reduce_body<__bf16, D>(a);
}

template <int D, int B>
__global__ __launch_bounds__(kReduceHeads * 64) void decode_reduce_step8_kernel(DecodeArgs a,
                                                                                StepBlocks nb) {
  step_store8<D, B>(a, nb.blk);
  decode_reduce_body<__bf16, D>(a);
}

int cu_count();

// A grid over the (cut sequence, query head) pairs the decode kernel
// listed.
// One wave per possible (sequence, query head) pair, so that no wave walks
// pairs one after another: the reduce is a few dependent loads long, and
// waves past the listed pairs leave after their first load.
template <typename T, int D>
int reduce_grid(const DecodeArgs& a) {
  return std::max(1, (a.num_seqs * a.num_q_heads + kReduceHeads - 1) / kReduceHeads);
}

template <typename T, int D>
hipError_t launch_reduce(const DecodeArgs& a, hipStream_t st) {
  decode_reduce_kernel<T, D><<<dim3(reduce_grid<T, D>(a)), kReduceHeads * 64, 0, st>>>(a);
  return hipGetLastError();
}

// The step's reduce also stores the new tokens: at least one workgroup
// per sequence.
template <int D, int B>
hipError_t launch_reduce_step(const DecodeArgs& a, const StepBlocks& nb, hipStream_t st) {
  const int grid = std::max(reduce_grid<__bf16, D>(a), a.num_seqs);
  decode_reduce_step_kernel<D, B><<<dim3(grid), kReduceHeads * 64, 0, st>>>(a, nb);
  return hipGetLastError();
}

template <int D, int B>
hipError_t launch_reduce_step8(const DecodeArgs& a, const StepBlocks& nb, hipStream_t st) {
  const int grid = std::max(reduce_grid<__bf16, D>(a), a.num_seqs);
  decode_reduce_step8_kernel<D, B><<<dim3(grid), kReduceHeads * 64, 0, st>>>(a, nb);
  return hipGetLastError();
}

// Persistent grid: as many workgroups as the chip holds at once (the
// occupancy of the kernel at hand), rounded down to a multiple of the head
// groups so that every head group gets the same number of ranges.
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// One workgroup per CU: with two, the CU's memory arbitration favoured the
// older workgroup so much that the two finished up to 1.7x apart and the
// younger one streamed its last ranges alone (measured with per-wave
// timestamps); alone on its CU, each workgroup's four waves keep 32 KB in
// flight, which a read-bandwidth probe found is what this HBM rewards.
#ifndef PA_MAX_WG_PER_CU
#define PA_MAX_WG_PER_CU 1
#endif
constexpr int kMaxWgPerCu = PA_MAX_WG_PER_CU;

struct Launch {
  dim3 grid, block;
  size_t lds;
};

// Sequences per launch: the plan lives in LDS (with prefix groups it holds
// up to two segments per sequence), and stays under 64 KiB.
constexpr int kMaxPlanSeqsGrouped = kMaxPlanSeqs / 2;
static_assert(plan_lds_bytes(kMaxPlanSeqs, false) <= 65536 &&
                  plan_lds_bytes(kMaxPlanSeqsGrouped, true) <= 65536,
              "decode plan fits 64 KiB of LDS");

template <typename K>
Launch decode_launch(const DecodeArgs& a, K kernel) {
  static int per_cu = 0;  // per kernel instantiation
  const size_t lds = plan_lds_bytes(a.num_seqs, a.group_start != nullptr);
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, kernel, kWaves * 64, plan_lds_bytes(kMaxPlanSeqsGrouped, true)) != hipSuccess ||
        n < 1)
      n = 1;
    per_cu = std::min(n, kMaxWgPerCu);
  }
  // at least one wave per kv head, so that every head has a range
  const int grid = std::max(cu_count() * per_cu, (a.num_kv_heads + kWaves - 1) / kWaves);
  return {dim3((unsigned)grid), dim3(kWaves * 64), lds};
}

}  // namespace

int decode_grid(int num_kv_heads) {
  return std::max(cu_count() * kMaxWgPerCu, (num_kv_heads + kWaves - 1) / kWaves);
}

namespace {

// The head group (1..16) fills the 16 head slots of the MFMA tiles at run
// time, so one instantiation per head_dim serves every group size.
template <int D, int B>
hipError_t launch_mfma(const DecodeArgs& a, int G, hipStream_t st, const StepBlocks* nb) {
  if (nb) {
    const Launch l = decode_launch(a, decode_step_kernel<D, B, kNBuf>);
    DecodeArgs b = a;
    b.decode_wgs = (int)l.grid.x;
    decode_step_kernel<D, B, kNBuf><<<dim3(l.grid.x + 1), l.block, l.lds, st>>>(b, G, *nb);
  } else {
    const Launch l = decode_launch(a, decode_mfma_kernel<D, B, kNBuf>);
    DecodeArgs b = a;
    b.decode_wgs = (int)l.grid.x;
    decode_mfma_kernel<D, B, kNBuf><<<dim3(l.grid.x + 1), l.block, l.lds, st>>>(b, G);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return nb ? launch_reduce_step<D, B>(a, *nb, st) : launch_reduce<__bf16, D>(a, st);
}

template <int D, int B>
hipError_t launch_mfma8(const DecodeArgs& a, int G, hipStream_t st, const StepBlocks* nb) {
  if (nb) {
    const Launch l = decode_launch(a, decode_step8_kernel<D, B, kNBuf8>);
    DecodeArgs b = a;
    b.decode_wgs = (int)l.grid.x;
    decode_step8_kernel<D, B, kNBuf8><<<dim3(l.grid.x + 1), l.block, l.lds, st>>>(b, G);
  } else {
    const Launch l = decode_launch(a, decode_mfma8_kernel<D, B, kNBuf8>);
    DecodeArgs b = a;
    b.decode_wgs = (int)l.grid.x;
    decode_mfma8_kernel<D, B, kNBuf8><<<dim3(l.grid.x + 1), l.block, l.lds, st>>>(b, G);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return nb ? launch_reduce_step8<D, B>(a, *nb, st) : launch_reduce<__bf16, D>(a, st);
}

template <int D, int G>
hipError_t launch_valu_g(const DecodeArgs& a, hipStream_t st) {
  const Launch l = decode_launch(a, decode_valu_kernel<D, G, kNBuf>);
  DecodeArgs b = a;
  b.decode_wgs = (int)l.grid.x;
  decode_valu_kernel<D, G, kNBuf><<<dim3(l.grid.x + 1), l.block, l.lds, st>>>(b);
  return hipGetLastError();
}

// A kv head with more than four query heads is taken as kv_div head groups
// of Gs = 4, 3, 2 or 1 heads (the largest that divides G): each group is a
// head of the plan and streams the kv head's blocks itself.  The groups'
// query heads are consecutive, so the partial rows and the reduce see a
// pool of G / Gs times the kv heads with Gs query heads each.
template <int D>
hipError_t launch_valu(const DecodeArgs& a, int G, hipStream_t st) {
  int Gs = G;
  DecodeArgs b = a;
  if (G > 4) {
    Gs = G % 4 == 0 ? 4 : G % 3 == 0 ? 3 : G % 2 == 0 ? 2 : 1;
    b.kv_div = G / Gs;
    b.num_kv_heads = a.num_kv_heads * b.kv_div;
    b.slots = Gs;
  }
  hipError_t e;
  switch (Gs) {
    case 1: e = launch_valu_g<D, 1>(b, st); break;
    case 2: e = launch_valu_g<D, 2>(b, st); break;
    case 3: e = launch_valu_g<D, 3>(b, st); break;
    case 4: e = launch_valu_g<D, 4>(b, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_reduce<float, D>(b, st);
}

}  // namespace

DecodePath decode_path(pa_dtype dtype, int head_dim, int group, int block_size) {
  if (head_dim != 64 && head_dim != 128) return DecodePath::kUnsupported;
  if (group < 1) return DecodePath::kUnsupported;
  if (block_size != 8 && block_size != 16 && block_size != 32) return DecodePath::kUnsupported;
  if (dtype == PA_F32 && block_size != kBlock) return DecodePath::kUnsupported;
  if (dtype == PA_BF16) {
    if (group <= kMaxMfmaGroup) return DecodePath::kMfma;
    return DecodePath::kUnsupported;
  }
  if (dtype == PA_FP8_E4M3 && group <= kMaxMfmaGroup) return DecodePath::kMfma8;
  if (dtype == PA_F32 && group <= kMaxMfmaGroup) return DecodePath::kValu;
  return DecodePath::kUnsupported;
}

namespace {
// One instantiation per (head_dim, block size) of each MFMA kernel.
template <template <int, int> class K, int D>
hipError_t by_block(int block_size, const DecodeArgs& a, int group, hipStream_t st,
                    const StepBlocks* nb) {
  switch (block_size) {
    case 8: return K<D, 8>::run(a, group, st, nb);
    case 16: return K<D, 16>::run(a, group, st, nb);
    case 32: return K<D, 32>::run(a, group, st, nb);
    default: return hipErrorInvalidValue;
  }
}
template <int D, int B>
struct MfmaLaunch {
  static hipError_t run(const DecodeArgs& a, int G, hipStream_t st, const StepBlocks* nb) {
    return launch_mfma<D, B>(a, G, st, nb);
  }
};
template <int D, int B>
struct Mfma8Launch {
  static hipError_t run(const DecodeArgs& a, int G, hipStream_t st, const StepBlocks* nb) {
    return launch_mfma8<D, B>(a, G, st, nb);
  }
};

// nb: a decode step's new blocks (bf16 pools only), nullptr otherwise.
hipError_t launch_decode_slice(const DecodeArgs& a, pa_dtype dtype, int head_dim, int group,
                               int block_size, hipStream_t st, const StepBlocks* nb) {
  switch (decode_path(dtype, head_dim, group, block_size)) {
    case DecodePath::kMfma:
      return head_dim == 128 ? by_block<MfmaLaunch, 128>(block_size, a, group, st, nb)
                             : by_block<MfmaLaunch, 64>(block_size, a, group, st, nb);
    case DecodePath::kMfma8:
      return head_dim == 128 ? by_block<Mfma8Launch, 128>(block_size, a, group, st, nb)
                             : by_block<Mfma8Launch, 64>(block_size, a, group, st, nb);
    case DecodePath::kValu:
      if (nb) return hipErrorInvalidValue;
      return head_dim == 128 ? launch_valu<128>(a, group, st) : launch_valu<64>(a, group, st);
    default:
      return hipErrorInvalidValue;
  }
}
}  // namespace

// Batches larger than one plan are launched in slices (the per-workgroup
// plan lives in LDS; a decode step's new blocks ride in the kernel
// arguments, kStepSeqs at a time); every per-sequence array is offset to
// the slice, the prefix groups are clipped to it, and the slices reuse the
// partial buffers and seg_info one after another on the stream.
hipError_t launch_decode(const DecodeArgs& a, pa_dtype dtype, int head_dim, int group,
                         int block_size, hipStream_t st, const int32_t* host_new_blocks) {
  const size_t es = dtype == PA_F32 ? 4 : 2;  // q / out element (bf16 for 8-bit pools)
  int step = a.group_start ? kMaxPlanSeqsGrouped : kMaxPlanSeqs;
  if (a.k_new) step = std::min(step, kStepSeqs);
  for (int32_t s0 = 0; s0 < a.num_seqs; s0 += step) {
    DecodeArgs b = a;
    b.num_seqs = std::min(step, a.num_seqs - s0);
    b.seq_base = s0;
    const size_t qrow = (size_t)a.num_q_heads * head_dim * es;
    b.q = static_cast<const uint8_t*>(a.q) + (size_t)s0 * qrow;
    b.out = static_cast<uint8_t*>(a.out) + (size_t)s0 * qrow;
    b.block_tables = a.block_tables + (size_t)s0 * a.max_blocks;
    b.context_lens = a.context_lens + s0;
    StepBlocks nb;
    if (a.k_new) {
      const size_t krow = (size_t)a.num_kv_heads * head_dim * es;
      b.k_new = static_cast<const uint8_t*>(a.k_new) + (size_t)s0 * krow;
      b.v_new = static_cast<const uint8_t*>(a.v_new) + (size_t)s0 * krow;
      b.tables_w = a.tables_w + (size_t)s0 * a.max_blocks;
      b.lens_out = a.lens_out + s0;
      for (int i = 0; i < kStepSeqs; ++i)
        nb.blk[i] = i < b.num_seqs ? host_new_blocks[s0 + i] : -1;
    }
    const hipError_t e =
        launch_decode_slice(b, dtype, head_dim, group, block_size, st, a.k_new ? &nb : nullptr);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pakv
