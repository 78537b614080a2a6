// Multi-token paged attention: extend / chunked prefill over a paged prefix
// with a causal mask.  The glossary entry's "Complex Attention Patterns" and
// "Dynamic Growth" (the cache is read through the block table whatever the
// logical order; new tokens are appended on demand) and the vLLM post's
// "The bonus contiguous storage can't give you: sharing" (several sequences
// reading one prefix) make the same gather serve more than one query per
// sequence.
//
// What is computed: sequence s brings n_s new query tokens (rows
// q_start[s] .. q_start[s+1] of q), whose K/V are already in the cache, so
// its context length L_s counts them.  Query j of s sits at position
// p = L_s - n_s + j and attends to tokens 0..p of the sequence:
//   out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . K_t) V_t,
// K_t, V_t read from block_tables[s][t / 16], slot t % 16, kv head h / G.
//
// Decomposition.  A row tile is 16 MFMA "head slots" holding (query, head)
// pairs: 16 / G consecutive queries of one sequence times the G query heads
// of one kv head.  A workgroup's W waves (eight: two per SIMD) take R row
// tiles each (W R tiles of one (sequence, kv head)) and stream the
// sequence's context in stages of 64 tokens: the waves split each stage's
// loads evenly (eight waves: half a 16-token block each), straight from the
// pool into LDS (global_load_lds_dwordx4, no registers, no LDS writes), and
// every wave reads the whole stage.  Several stages are in flight; one
// barrier per stage.  A batch too small to fill the chip cuts each context
// into chunks whose (m, l, o) partials a second kernel combines.
//
// Tiles.  q.K runs as v_mfma_f32_16x16x32_bf16 with A = 16 tokens x 32 dims
// of K and B = 32 dims x 16 head slots of q, so a lane ends with 4 tokens'
// scores of one head slot.  A 32-token pair of blocks is scored as two such
// tiles whose token rows are chosen so that lane group grp holds tokens
// 8 grp .. 8 grp + 7 of the pair; P.V is then one v_mfma_f32_16x16x32_bf16
// per 16 dims with A = P (bf16, k = those 8 tokens) and B = a 16-byte LDS
// read of V holding the same 8 tokens of one dim.  K rows sit in LDS with
// their 16-byte chunks XOR-swizzled by row, so a tile's reads are free of
// bank conflicts with no padding; the swizzle is applied by choosing each
// lane's source address of the direct-to-LDS load.
#include <algorithm>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pakv {
namespace {

constexpr int kExtBlock = 16;
#ifndef PA_EXT_STAGE_BLOCKS
#define PA_EXT_STAGE_BLOCKS 4
#endif
constexpr int kStageBlocks = PA_EXT_STAGE_BLOCKS;     // blocks of one stage
constexpr int kStageTok = kStageBlocks * kExtBlock;   // tokens of a stage (64)
constexpr int kStagePairs = kStageTok / 32;           // 32-token pairs of a stage
static_assert(kStageBlocks % 2 == 0, "whole pairs per stage");

// Per head size: waves per workgroup (W), row tiles per wave (R), LDS stage
// buffers (stages in flight + 1) and workgroups per CU.  R row tiles share
// every K and V read from LDS, so R sets the LDS bytes per MFMA.  Eight
// waves (two per SIMD: one computes its softmax while the other keeps the
// matrix core busy) share each stage, which halves the K/V bytes staged per
// query against four.  Head size 128 keeps three stage buffers (a stage's
// loads have two stages of compute to arrive; four measured slower), head
// size 64 four.
#ifndef PA_EXT_WAVES
#define PA_EXT_WAVES 8
#endif
#ifndef PA_EXT128_ROWS
#define PA_EXT128_ROWS 2
#endif
#ifndef PA_EXT128_STAGES
#define PA_EXT128_STAGES 3
#endif
#ifndef PA_EXT128_WG
#define PA_EXT128_WG 1
#endif
#ifndef PA_EXT64_ROWS
#define PA_EXT64_ROWS 2
#endif
#ifndef PA_EXT64_STAGES
#define PA_EXT64_STAGES 4
#endif
#ifndef PA_EXT64_WG
#define PA_EXT64_WG 1
#endif
// A wave issuing its MFMAs (q.K, P.V) runs at raised priority, so that the
// other wave of the SIMD fills the gaps with its softmax rather than
// competing for the same issue slots.
#ifndef PA_EXT_SETPRIO
#define PA_EXT_SETPRIO 1
#endif
#if PA_EXT_SETPRIO
#define PA_EXT_PRIO_MFMA() __builtin_amdgcn_s_setprio(1)
#define PA_EXT_PRIO_VALU() __builtin_amdgcn_s_setprio(0)
#else
#define PA_EXT_PRIO_MFMA() ((void)0)
#define PA_EXT_PRIO_VALU() ((void)0)
#endif
#ifndef PA_EXT_SPLIT_UNITS
#define PA_EXT_SPLIT_UNITS 1
#endif
constexpr int kExtWaves = PA_EXT_WAVES;
static_assert(kExtWaves == 4 || kExtWaves == 8, "four or eight waves share a stage");
template <int D>
struct ExtCfg;
template <>
struct ExtCfg<128> {
  static constexpr int R = PA_EXT128_ROWS, NST = PA_EXT128_STAGES, WG = PA_EXT128_WG;
};
template <>
struct ExtCfg<64> {
  static constexpr int R = PA_EXT64_ROWS, NST = PA_EXT64_STAGES, WG = PA_EXT64_WG;
};
constexpr int kExtTabWindow = 1024;          // table entries staged in LDS at a time
static_assert(kExtTabWindow % kStageBlocks == 0, "whole stages per table window");

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// s_waitcnt immediate for gfx9: vector-memory count at most n, LDS/scalar
// count 0, export count untouched.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

template <int D>
struct StageGeom {
  static constexpr int ROW = D * 2;           // bytes of one K row
  static constexpr int KCH = ROW / 16;        // 16-byte chunks per K row
  static constexpr int kK = kStageTok * ROW;  // K bytes of a stage
  static constexpr int kVPair = 4 * D * 16;   // V bytes of a 32-token pair
  static constexpr int kV = kStagePairs * kVPair;  // V bytes of a stage
  static constexpr int kLoads = kK / kExtWaves / 1024;  // 1 KiB loads per wave, K and V each
  static_assert(kV == kK && kLoads >= 1 && kLoads * 1024 * kExtWaves == kK,
                "a stage is whole 1 KiB loads per wave");
};

// LDS of one workgroup: the stage buffers (separate arrays, so that the
// compiler sees which buffer a direct-to-LDS load writes and which one a
// read touches) and the block-table window.
template <int D>
struct ExtLds {
  static constexpr int kBuf = StageGeom<D>::kK + StageGeom<D>::kV;
};

// Work order.  A unit's cost is about its sequence's context length (every
// row tile of a sequence streams the same context), and lengths in a batch
// can differ by orders of magnitude.  Units are therefore handed out
// longest sequence first, in a snake over the grid (round r gives rank
// r * grid + b to workgroup b for even r and r * grid + grid - 1 - b for
// odd r), which pairs each workgroup's long units with shorter ones.  Every
// workgroup computes the same order: a bitonic sort of (length, sequence)
// keys in LDS, for batches of up to kExtSortMax sequences; larger batches
// keep sequence order (their many units even out without it).
constexpr int kExtSortMax = 1024;

__device__ void sort_desc(unsigned long long* key, int n) {  // n a power of two
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = key[i], y = key[ixj];
          if ((i & k) == 0 ? x < y : x > y) {
            key[i] = y;
            key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
}

// Plan in LDS: ord[i] = the sequence at position i of the work order, and
// pre[i] = units before position i (units of a sequence: ceil(n_s / qpu)
// row-tile groups times `splits` chunks).  Returns the total.
__device__ int build_extend_plan(const ExtendArgs& a, int qpu, int* pre, int* wsum,
                                 unsigned long long* key, int* ord) {
  const int S = a.num_seqs, T_ = blockDim.x, t = threadIdx.x;
  const int cap = a.max_blocks * kExtBlock;
  if (S > 1 && S <= kExtSortMax) {
    int n = 2;
    while (n < S) n <<= 1;
    for (int i = t; i < n; i += T_) {
      unsigned long long k = 0;
      if (i < S) {
        const int L = min(max(a.context_lens[i], 0), cap);
        k = ((unsigned long long)L << 32) | (0xffffffffu - (unsigned)i);
      }
      key[i] = k;
    }
    __syncthreads();
    sort_desc(key, n);
    for (int i = t; i < S; i += T_) ord[i] = (int)(0xffffffffu - (unsigned)(key[i] & 0xffffffffu));
  } else {
    for (int i = t; i < S; i += T_) ord[i] = i;
  }
  __syncthreads();
  const int C = (S + T_ - 1) / T_;
  const int i0 = min(S, t * C), i1 = min(S, i0 + C);
  auto units_of = [&](int i) {
    const int s = ord[i];
    const int n = max(0, a.q_start[s + 1] - a.q_start[s]);
    return (n + qpu - 1) / qpu * a.splits;
  };
  int nt = 0;
  for (int i = i0; i < i1; ++i) nt += units_of(i);
  int total;
  int run = block_excl_scan(nt, wsum, &total);
  for (int i = i0; i < i1; ++i) {
    pre[i] = run;
    run += units_of(i);
  }
  if (t == 0) pre[S] = total;
  __syncthreads();
  return total;
}

// K swizzle key of token t (0..31) of a pair.  The 16 lanes of one lane
// group read, for one K tile, tokens 8 a + 4 tau + b (a, b = 0..3) at the
// same chunk index; the key sends them to distinct 16-byte bank groups
// whether the LDS serves a 16-byte read 8 lanes at a time over 32 banks or
// 16 lanes at a time over 64.  Head size 128 (16 chunks a row, a row spans
// every bank): key b + 4 a.  Head size 64 (8 chunks, a row is 128 bytes, so
// two rows of different parity b mod 2 share a 64-bank line): key
// ((b / 2) + 2 a) ^ (4 (b mod 2)), distinct over a = 0, 1 for all b and,
// for a fixed b mod 2, over all a and b / 2.
template <int KCH>
__device__ __forceinline__ int kswz(int t) {
  static_assert(KCH == 16 || KCH == 8, "head size 128 or 64");
  const int a = (t >> 3) & 3, b = t & 3;
  return KCH == 16 ? b + 4 * a : (((b >> 1) + 2 * a) ^ (4 * (b & 1)));
}

// The reference a row's softmax starts from: finite, so that a row that sees
// no token of its chunk (its position lies before the chunk) keeps p = 0,
// l = 0, o = 0 instead of exp2(-inf + inf).
constexpr float kRefFloor = -1e30f;

// The stage buffers, picked by a compile-time index.
struct StageBufs {
  uint8_t* b0;
  uint8_t* b1;
  uint8_t* b2;
  uint8_t* b3;
  template <int I>
  __device__ __forceinline__ uint8_t* get(std::integral_constant<int, I>) const {
    static_assert(I < 4, "four stage buffers at most");
    return I == 0 ? b0 : I == 1 ? b1 : I == 2 ? b2 : b3;
  }
};

template <int D, int R, int NST, bool kPos>
__device__ __forceinline__ void extend_unit(const ExtendArgs& a, int G, int qpt, int s, int unit,
                                            int chunk, int g, int wave, int lane,
                                            const StageBufs& sbuf, int* tab) {
  using SG = StageGeom<D>;
  constexpr int B = kExtBlock;
  constexpr int KJ = D / 32;   // q.K MFMAs per 16-token tile (32 dims each)
  constexpr int NT = D / 16;   // P.V MFMAs per pair (16 dims each)
  constexpr int ROW = SG::ROW;
  constexpr int KCH = SG::KCH;
  const int col = lane & 15, grp = lane >> 4;

  const int q0 = a.q_start[s];
  const int n = a.q_start[s + 1] - q0;
  const int L = min(max(a.context_lens[s], 0), a.max_blocks * B);
  const int qpu = kExtWaves * R * qpt;            // queries of the unit
  const int ufirst = unit * qpu;                  // first query of the workgroup's row tiles
  const int ulast = min(n - 1, ufirst + qpu - 1);
  const int p_max = max(0, L - n + ulast);        // furthest position any row attends
  const int first = ufirst + wave * R * qpt;      // this wave's first query
  const int last = min(ulast, first + R * qpt - 1);
  const int p_lo = first <= last ? L - n + first : p_max;  // nearest position of the wave's rows

  // this chunk's tokens: [kv0, kv1), whole stages, within 0 .. p_max.
  // Chunks hold the same number of tokens in every sequence (the table's
  // capacity cut in `splits`), so units of long contexts cost the same
  // whatever the batch's other lengths; a short context's later chunks are
  // empty.
  int kv0 = 0, kv1 = p_max + 1;
  if (a.splits > 1) {
    const int cap = a.max_blocks * B;
    const int per = (cap + a.splits * kStageTok - 1) / (a.splits * kStageTok) * kStageTok;
    kv0 = chunk * per;
    kv1 = min(kv1, kv0 + per);
  }
  // (an empty context, which valid input never pairs with queries, reads
  // no table entry)
  const int nst = kv1 > kv0 && L > 0 ? (kv1 - kv0 + kStageTok - 1) / kStageTok : 0;

  int p_row[R];
  bool live[R];
  bf16x8 qop[R][KJ];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int f = first + rr * qpt;
    live[rr] = f <= last;
    const int qi = f + col / G;
    const bool row_ok = col < qpt * G && qi <= last;
    p_row[rr] = row_ok ? L - n + qi : p_max;      // padding slots: harmless finite rows
    u32x4 w[KJ];
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj) w[kj] = u32x4{0u, 0u, 0u, 0u};
    if (row_ok) {
      const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                          ((size_t)(q0 + qi) * a.num_q_heads + g * G + col % G) * ROW + grp * 16;
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj) w[kj] = *reinterpret_cast<const u32x4*>(qp + kj * 64);
    }
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj) qop[rr][kj] = __builtin_bit_cast(bf16x8, w[kj]);
  }

  // Direct-to-LDS loads: the W waves split each stage evenly.  Wave w
  // loads stage K rows w * RPW .. w * RPW + RPW - 1 (RPW = 64 / W; chunk c
  // of the row that is token t of its 32-token pair at chunk position
  // c ^ kswz<KCH>(t)) and the V chunks w * kLoads * 64 .. of the stage, all
  // from block w * 4 / W of the stage.  Load j of a wave fills 1 KiB: lane
  // l's 16 bytes land at 16 l, from the source offsets below (the same for
  // every stage).
  constexpr int RPW = kStageTok / kExtWaves;
  const int wblk = wave * kStageBlocks / kExtWaves;   // the wave's block of each stage
  const size_t blk_bytes = (size_t)a.num_kv_heads * B * ROW;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool) + (size_t)g * B * ROW;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool) + (size_t)g * D * B * 2;
  // K: load j, lane l -> stage row r = w * RPW + j * (1024 / ROW) + l / KCH
  // (row r mod 16 of the block, token r mod 32 of its pair), position
  // l mod KCH; V: chunk ci = (w * kLoads + j) * 64 + l of the stage ->
  // dim ci mod D, token half (ci / D) mod 2 of the block.
  auto ksrc = [&](int j) {
    const int r = wave * RPW + j * (1024 / ROW) + lane / KCH;
    return (uint32_t)((r % B) * ROW + (((lane % KCH) ^ kswz<KCH>(r % 32)) * 16));
  };
  auto vsrc = [&](int j) {
    const int ci = (wave * SG::kLoads + j) * 64 + lane;
    return (uint32_t)((ci % D) * (B * 2) + ((ci / D) % 2) * 16);
  };
  const uint32_t kdst = wave * RPW * ROW;                  // the wave's K rows
  const uint32_t vdst = SG::kK + wave * SG::kLoads * 1024;  // the wave's V chunks

  // LDS read offsets of this lane (stage-relative).  K tile tau of a pair:
  // MFMA row m reads token 8 (m / 4) + 4 tau + m % 4 of the pair, chunk
  // kj * 4 + grp (swizzled).  V: chunk (grp, dim) of the pair.
  auto kread = [&](int tau, int kj) {
    const int t = 8 * (col / 4) + 4 * tau + col % 4;
    return (uint32_t)(t * ROW + (((kj * 4 + grp) ^ kswz<KCH>(t)) * 16));
  };
  const uint32_t vread = SG::kK + (grp * D + col) * 16;

  float m_ref[R], thr[R], l_run[R];               // thr = m_ref + kSlack
  f32x4 acc[R][NT];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    m_ref[rr] = kRefFloor;
    thr[rr] = kRefFloor + kSlack;
    l_run[rr] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[rr][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;
  const int tid = threadIdx.x;

  // one stage's loads into buffer `buf`: the wave's block of stage i of the
  // window (clamped to the window's last block, so loads past it re-read it)
  auto dma = [&](int i, int cn, auto buf) {
    const int bi = min(i * kStageBlocks + wblk, cn - 1);
    const size_t off = (size_t)__builtin_amdgcn_readfirstlane(tab[bi]) * blk_bytes;
    const gptr kb = uniform_ptr(kpool + off);
    const gptr vb = uniform_ptr(vpool + off);
    uint8_t* d = sbuf.get(buf);
#pragma unroll
    for (int j = 0; j < SG::kLoads; ++j)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(kb + ksrc(j)),
                                       (lds_void*)(d + kdst + j * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < SG::kLoads; ++j)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(vb + vsrc(j)),
                                       (lds_void*)(d + vdst + j * 1024), 16, 0, 0);
  };

  // one stage from buffer `buf`: logical tokens t0 .. t0 + kStageTok - 1,
  // a 32-token pair at a time (scores, softmax, P.V).  Scores of tokens past
  // a row's position become -inf; that takes instructions only in pairs that
  // reach past the nearest row of the wave (the causal edge and the
  // context's end).  V needs no mask here: stale slots are zeroed in LDS first.
  auto compute = [&](int t0, auto buf) {
    const uint8_t* d = sbuf.get(buf);
#pragma unroll
    for (int pp = 0; pp < kStagePairs; ++pp) {
      const bool cmask = t0 + pp * 32 + 31 > p_lo;
      // scores: sc[rr][tau], lane's tokens 8 grp + 4 tau + r of the pair
      f32x4 sc[R][2];
      PA_EXT_PRIO_MFMA();
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        u32x4 kb[KJ];
#pragma unroll
        for (int kj = 0; kj < KJ; ++kj)
          kb[kj] = *reinterpret_cast<const u32x4*>(d + pp * 32 * ROW + kread(tau, kj));
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          sc[rr][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kj = 0; kj < KJ; ++kj)
            sc[rr][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, kb[kj]), qop[rr][kj], sc[rr][tau], 0, 0, 0);
        }
      }
      PA_EXT_PRIO_VALU();
      // With a positive scale (kPos) the scores stay unscaled until the
      // exponent: x = masked raw score, the lane's max is scaled once, and
      // p = exp2(fma(x, scale, -m)).  Otherwise x is the scaled score.
      float x[R][8];
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = sc[rr][e / 4][e % 4];
          x[rr][e] = kPos ? v : v * a.scale_log2;
        }
      if (cmask) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const int lim = p_row[rr] - (t0 + pp * 32 + 8 * grp);  // lane token e at offset e
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e > lim) x[rr][e] = kNegInf;
        }
      }
      float bm[R];
      bool grow = false;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        float mx = fmaxf(fmaxf(x[rr][0], x[rr][1]), fmaxf(x[rr][2], x[rr][3]));
        mx = fmaxf(mx, fmaxf(fmaxf(x[rr][4], x[rr][5]), fmaxf(x[rr][6], x[rr][7])));
        bm[rr] = kPos ? mx * a.scale_log2 : mx;
        grow = grow || bm[rr] > thr[rr];
      }
      // P.V of the pair; called on each side of the rescale branch so that
      // the accumulators stay in place on the common side (one copy after
      // the branch would have to merge rescaled and unscaled values, and
      // the compiler does that by copying every accumulator register)
      auto pv = [&]() {
        // P in bf16 (nearest even): the A operand of P.V, k = the lane's 8
        // tokens of the pair in order
        bf16x8 pk[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          float pr[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pr[e] = kPos ? fexp2(fmaf(x[rr][e], a.scale_log2, -m_ref[rr]))
                         : fexp2(x[rr][e] - m_ref[rr]);
          l_run[rr] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(pr[e]);
          pk[rr] = v;
        }
        PA_EXT_PRIO_MFMA();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const u32x4 vb = *reinterpret_cast<const u32x4*>(d + pp * SG::kVPair + vread + nt * 256);
#pragma unroll
          for (int rr = 0; rr < R; ++rr)
            acc[rr][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                pk[rr], __builtin_bit_cast(bf16x8, vb), acc[rr][nt], 0, 0, 0);
        }
      };
      if (__ballot(grow)) {   // rare: move references that grew, rescale
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          bm[rr] = max_xor32(max_xor16(bm[rr]));
          const float m_new = bm[rr] > thr[rr] ? bm[rr] : m_ref[rr];
          const float alpha = fexp2(m_ref[rr] - m_new);
          l_run[rr] *= alpha;
          m_ref[rr] = m_new;
          thr[rr] = m_new + kSlack;
          float ar[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = lane_bcast(alpha, 4 * grp + r);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rr][nt][r] *= ar[r];
        }
        pv();
        asm volatile("");  // the two sides differ: no merging them back
      } else {
        pv();
      }
      PA_EXT_PRIO_VALU();
    }
  };

  // V of the stage's tokens at or past the context's end (stale slots of
  // the last block, and the re-read copies of it that pad the last stage)
  // is zeroed in LDS before any wave reads the stage: their probabilities
  // are 0, and stale bits (NaN included) must not meet them.  V chunk
  // (c8, dim) of a stage holds tokens t0 + 8 c8 .. t0 + 8 c8 + 7.
  auto zero_tail = [&](int t0, auto buf) {
    uint8_t* d = sbuf.get(buf);
    for (int idx = tid; idx < (kStageTok / 8) * D; idx += kExtWaves * 64) {
      const int c8 = idx / D, dim = idx % D;
      const int lim = L - (t0 + 8 * c8);   // leading tokens of the chunk that are valid
      if (lim >= 8) continue;
      u32x4* v = reinterpret_cast<u32x4*>(d + SG::kK + (c8 * D + dim) * 16);
      u32x4 x = *v;
      x.x &= (0 < lim ? 0x0000ffffu : 0u) | (1 < lim ? 0xffff0000u : 0u);
      x.y &= (2 < lim ? 0x0000ffffu : 0u) | (3 < lim ? 0xffff0000u : 0u);
      x.z &= (4 < lim ? 0x0000ffffu : 0u) | (5 < lim ? 0xffff0000u : 0u);
      x.w &= (6 < lim ? 0x0000ffffu : 0u) | (7 < lim ? 0xffff0000u : 0u);
      *v = x;
    }
  };

  // the chunk's blocks, a table window at a time
  const int b_first = kv0 / B;
  const int b_end = nst > 0 ? b_first + nst * kStageBlocks : b_first;
  for (int w0 = b_first; w0 < b_end; w0 += kExtTabWindow) {
    const int cn = min(kExtTabWindow, b_end - w0);
    // every wave is past the previous window (its loads landed, its reads
    // done) before the window is overwritten; entries past the context
    // re-read the last one
    const int last_blk = max(0, (L - 1) / B);
    __syncthreads();
    for (int e = tid; e < cn; e += kExtWaves * 64) tab[e] = trow[min(w0 + e, last_blk)];
    __syncthreads();
    const int ns = cn / kStageBlocks;               // stages of the window
    // prologue: stages 0 .. NST-2 in flight
    static_for<NST - 1>([&](auto j) { dma((int)j, cn, j); });
    for (int i0 = 0; i0 < ns; i0 += NST) {
      static_for<NST>([&](auto j) {
        const int i = i0 + j;
        // this wave's loads of stage i landed (NST - 2 later stages may be
        // in flight), then every wave's have, and every wave is done with
        // the buffer the next loads overwrite
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NST - 2) * 2 * SG::kLoads));
        __builtin_amdgcn_s_barrier();
        dma(i + NST - 1, cn, std::integral_constant<int, (j + NST - 1) % NST>{});
        if (i < ns) {
          const int t0 = (w0 + i * kStageBlocks) * B;
          if (t0 + kStageTok > L) {   // the context ends in this stage (uniform)
            zero_tail(t0, j);
            // the zeros are in LDS before any wave reads the stage; the
            // loads just issued may stay in flight
            __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
            __builtin_amdgcn_s_barrier();
          }
          compute(t0, j);
        }
      });
    }
  }
  // no load may still be writing this workgroup's LDS when it moves on or ends
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));

  // acc[rr][nt][r] holds slot 4*grp + r of row tile rr (query first + rr*qpt
  // + slot / G, head slot % G), dim nt*16 + col.  The lane index goes
  // through an opaque copy, so that the output addresses are computed here
  // rather than before the stage loop (where the compiler would keep them
  // in scratch and reload each behind a wait for every store issued)
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int ecol = ln & 15, egrp = ln >> 4;
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (!live[rr]) continue;
    float l_tot = sum_xor16(l_run[rr]);
    l_tot = sum_xor32(l_tot);
    float den[4], mr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      den[r] = lane_bcast(l_tot, 4 * egrp + r);
      mr[r] = lane_bcast(m_ref[rr], 4 * egrp + r);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int slot = 4 * egrp + r;
      const int qq = first + rr * qpt + slot / G;
      if (slot >= qpt * G || qq > last) continue;
      const size_t row = (size_t)(q0 + qq) * a.num_q_heads + g * G + slot % G;
      if (a.splits == 1) {
        const size_t ob = row * D + ecol;
        const float inv = 1.f / den[r];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          static_cast<__bf16*>(a.out)[ob + nt * 16] = static_cast<__bf16>(acc[rr][nt][r] * inv);
      } else {
        const size_t pr = row * a.splits + chunk;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) a.part_o[pr * D + nt * 16 + ecol] = acc[rr][nt][r];
        if (ecol == 0) {
          a.part_m[pr] = mr[r];
          a.part_l[pr] = den[r];
        }
      }
    }
  }
}

template <int D, int R, int NST, int WG, bool kPos>
__global__ __launch_bounds__(kExtWaves * 64, WG) void extend_kernel(ExtendArgs a, int G, int qpt) {
  static_assert(NST >= 2 && NST <= 4, "two to four stage buffers");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[ExtLds<D>::kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[ExtLds<D>::kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[NST > 2 ? ExtLds<D>::kBuf : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[NST > 3 ? ExtLds<D>::kBuf : 16];
  __shared__ int tab_lds[kExtTabWindow];
  __shared__ unsigned long long sort_key[kExtSortMax];
  extern __shared__ int ext_lds[];
  const StageBufs sbuf{st0, st1, st2, st3};
  int* pre = ext_lds;                 // [S + 1]
  int* ord = ext_lds + a.num_seqs + 1;  // [S]
  int* wsum = ord + a.num_seqs;         // [8]
  // a unit is the workgroup's W R row tiles of qpt queries each, over one chunk
  const int tiles = build_extend_plan(a, kExtWaves * R * qpt, pre, wsum, sort_key, ord);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int units = tiles * a.num_kv_heads;
  const int grid = gridDim.x;
  for (int r = 0;; ++r) {
    const int u = r * grid + ((r & 1) ? grid - 1 - (int)blockIdx.x : (int)blockIdx.x);
    if (u >= units) break;  // ranks grow with r: no later round has work either
    const int g = u % a.num_kv_heads, k = u / a.num_kv_heads;
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= k) lo = mid; else hi = mid - 1;
    }
    int i = lo;
    while (pre[i + 1] <= k) ++i;  // skip sequences without queries
    i = __builtin_amdgcn_readfirstlane(i);
    const int s = __builtin_amdgcn_readfirstlane(ord[i]);
    const int local = k - pre[i];
    extend_unit<D, R, NST, kPos>(a, G, qpt, s, local / a.splits, local % a.splits, g, wave, lane,
                                 sbuf, tab_lds);
  }
}

// Combine of a split context: one wave per (query row, head), over the
// chunks' partials: M = max m_c, out = sum 2^(m_c - M) o_c / sum 2^(m_c - M) l_c.
constexpr int kCombineHeads = 4;

template <int D>
__global__ __launch_bounds__(kCombineHeads * 64) void extend_combine_kernel(ExtendArgs a) {
  constexpr int EPL = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * kCombineHeads + wave;
  if (row >= (size_t)a.total_q * a.num_q_heads) return;
  const int C = a.splits;
  const float* pm = a.part_m + row * C;
  const float* pl = a.part_l + row * C;
  float M = kNegInf;
  for (int c = lane; c < C; c += 64) M = fmaxf(M, pm[c]);
  M = wave_max(M);
  float den = 0.f, num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  for (int c = 0; c < C; ++c) {
    const float f = fexp2(pm[c] - M);
    den = fmaf(f, pl[c], den);
    const float* po = a.part_o + (row * C + c) * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] = fmaf(f, po[e * 64 + lane], num[e]);
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    static_cast<__bf16*>(a.out)[row * D + e * 64 + lane] = static_cast<__bf16>(num[e] * inv);
}

int cu_count_ext() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached = n;
  }
  return cached;
}

template <int D>
hipError_t launch_extend_d(const ExtendArgs& a, int G, hipStream_t st) {
  using C = ExtCfg<D>;
  const int qpt = std::max(1, 16 / G);
  // persistent grid: C::WG workgroups per CU take the units in turn
  const size_t lds = (2 * (size_t)a.num_seqs + 1 + 8) * sizeof(int);
  const int grid = std::max(1, std::min(cu_count_ext() * C::WG, 1 << 16));
  // a positive scale folds into the exponent's fma; any other takes the
  // plain form
  if (a.scale_log2 > 0.f)
    extend_kernel<D, C::R, C::NST, C::WG, true><<<dim3(grid), dim3(kExtWaves * 64), lds, st>>>(a, G, qpt);
  else
    extend_kernel<D, C::R, C::NST, C::WG, false><<<dim3(grid), dim3(kExtWaves * 64), lds, st>>>(a, G, qpt);
  return hipGetLastError();
}

template <int D>
hipError_t launch_combine_d(const ExtendArgs& a, hipStream_t st) {
  const size_t rows = (size_t)a.total_q * a.num_q_heads;
  extend_combine_kernel<D><<<dim3((unsigned)((rows + kCombineHeads - 1) / kCombineHeads)),
                             dim3(kCombineHeads * 64), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

bool extend_supported(pa_dtype dtype, int head_dim, int group, int block_size) {
  return dtype == PA_BF16 && block_size == kExtBlock && (head_dim == 64 || head_dim == 128) &&
         group >= 1 && group <= 16;
}

// Split each context when the batch's units (each workgroup's row tiles of
// one sequence and kv head) would not give every workgroup slot of the grid
// one: into as many chunks as make up for it, each at least 1024 tokens, at
// most 32.  One unit per workgroup measured fastest for long prefixes: each
// chunk adds a partial row (m, l and a fp32 o) per query head that the
// combine reads back, traffic that finer splits multiply.
int extend_splits(int total_q, int num_q_heads, int num_kv_heads, int max_blocks, int head_dim) {
  const int G = num_q_heads / num_kv_heads;
  const int rows = head_dim == 128 ? ExtCfg<128>::R : ExtCfg<64>::R;
  const int wg = head_dim == 128 ? ExtCfg<128>::WG : ExtCfg<64>::WG;
  const int qpu = kExtWaves * rows * std::max(1, 16 / G);
  const int64_t units = ((int64_t)total_q + qpu - 1) / qpu * num_kv_heads;
  const int64_t want = (int64_t)PA_EXT_SPLIT_UNITS * cu_count_ext() * wg;
  if (units <= 0 || units >= want) return 1;
  const int64_t by_len = std::max<int64_t>(1, (int64_t)max_blocks * kExtBlock / 1024);
  const int64_t k = std::min<int64_t>({(want + units - 1) / units, by_len, 32});
  return static_cast<int>(std::max<int64_t>(1, k));
}

size_t extend_workspace_bytes(int total_q, int num_q_heads, int splits, int head_dim) {
  if (splits <= 1) return 0;
  const size_t n = (size_t)total_q * num_q_heads * splits;
  const auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return 2 * al(n * sizeof(float)) + al(n * head_dim * sizeof(float));
}

// Batches larger than kMaxPlanSeqs sequences run in slices (the plan lives
// in LDS); q_start holds absolute row indices, so only the per-sequence
// arrays move, and a split batch's partials (indexed by row) are combined
// once, after every slice.
hipError_t launch_extend(const ExtendArgs& a, int head_dim, int group, hipStream_t st) {
  for (int32_t s0 = 0; s0 < a.num_seqs; s0 += kMaxPlanSeqs) {
    ExtendArgs b = a;
    b.num_seqs = std::min(kMaxPlanSeqs, a.num_seqs - s0);
    b.q_start = a.q_start + s0;
    b.block_tables = a.block_tables + (size_t)s0 * a.max_blocks;
    b.context_lens = a.context_lens + s0;
    const hipError_t e =
        head_dim == 128 ? launch_extend_d<128>(b, group, st) : launch_extend_d<64>(b, group, st);
    if (e != hipSuccess) return e;
  }
  if (a.splits <= 1) return hipSuccess;
  return head_dim == 128 ? launch_combine_d<128>(a, st) : launch_combine_d<64>(a, st);
}

}  // namespace pakv
