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
// Decomposition: the 16 "head slots" of the decode kernel's MFMA tiles hold
// (query, head) pairs here: a row tile is QPT = 16 / G consecutive queries
// of one sequence times the G query heads of one kv head.  A workgroup's
// four waves take 4R consecutive row tiles of one (sequence, kv head) and
// stream blocks 0 .. p_max of the sequence: each 16-token K/V tile is
// loaded once per workgroup into LDS and read by all four waves, and each
// wave masks its rows at their own positions.  No context split: every row
// tile finishes in place.
#include <algorithm>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pakv {
namespace {

constexpr int kExtBlock = 16;
// Tuning (measured on 32 sequences x 256-token chunks, GQA 32/8, d 128):
// two row tiles per wave and two workgroups per CU (two waves per SIMD, so
// one wave's MFMAs hide the other's softmax) ran at 530-537 TFLOP/s before
// the mask-free interior blocks and the fused scale (590 with both); three
// row tiles at 409, four at one workgroup per CU at about 330 (the last two
// with P carried to 16 bits: 332-337 and 458-479 for two row tiles), and
// one row tile at four workgroups per CU at 438.  One block in flight beyond
// the staged one is what fits two workgroups per CU (a deeper ring spills).
#ifndef PA_EXT_ROWS
#define PA_EXT_ROWS 2
#endif
constexpr int kExtRows = PA_EXT_ROWS;  // row tiles per wave
#ifndef PA_EXT_MIN_WG
#define PA_EXT_MIN_WG 2
#endif
constexpr int kExtWgPerCu = PA_EXT_MIN_WG;  // workgroups per CU (register budget 512 / this)
#ifndef PA_EXT_PREFETCH
#define PA_EXT_PREFETCH 1
#endif
constexpr int kExtPrefetch = PA_EXT_PREFETCH;  // blocks in flight beyond the staged one
constexpr int kExtTabWindow = 1024;             // table entries staged in LDS at a time

// Plan in LDS: units before each sequence (prefix sums of ceil(n_s / qpt),
// with qpt the queries of one unit).
__device__ int build_extend_plan(const ExtendArgs& a, int qpt, int* pre, int* wsum) {
  const int S = a.num_seqs, T_ = blockDim.x, t = threadIdx.x;
  const int C = (S + T_ - 1) / T_;
  const int s0 = min(S, t * C), s1 = min(S, s0 + C);
  int nt = 0;
  for (int s = s0; s < s1; ++s) {
    const int n = max(0, a.q_start[s + 1] - a.q_start[s]);
    nt += (n + qpt - 1) / qpt;
  }
  int total;
  int run = block_excl_scan(nt, wsum, &total);
  for (int s = s0; s < s1; ++s) {
    pre[s] = run;
    const int n = max(0, a.q_start[s + 1] - a.q_start[s]);
    run += (n + qpt - 1) / qpt;
  }
  if (t == 0) pre[S] = total;
  __syncthreads();
  return total;
}

// Workgroup-shared K/V: the four waves of a workgroup take 4R row tiles of
// the same (sequence, kv head), and each 16-token K/V tile is loaded once
// per workgroup into LDS (every thread fetches one chunk of K and one of V)
// and read by all four waves, so one load feeds 4R row tiles.  Global loads
// run NPF blocks ahead of the staged one in a small per-thread register
// ring; LDS holds two tiles, so one barrier per block separates the store
// of tile i + 1 from its readers and the readers of tile i - 1 from its
// overwrite.
template <int D>
struct WgTile {
  // K rows padded by 32 bytes: the LDS bank-conflict counter read a third of
  // what it read with 16 or 64 bytes of padding (8 times less than unpadded)
  static constexpr int kStrideK = D * 2 + 32;
  static constexpr int kBytesK = 16 * kStrideK;
  static constexpr int kBytesV = D * 32;        // V as [dim tile][token quad][dim][4 tokens]
  static constexpr int kBytes = kBytesK + kBytesV;
  // each thread fetches one chunk of K and one of V: 32 D / 256 bytes each
  static constexpr int kChunk = D * 32 / (kWaves * 64);
  static_assert(kChunk == 8 || kChunk == 16, "8- or 16-byte chunks");
};

template <int D, int R, int NPF, bool kPos>
__device__ __forceinline__ void extend_wg_unit(const ExtendArgs& a, int G, int qpt, int s, int unit,
                                               int g, int wave, int lane, uint8_t* lds, int* tab) {
  using T = WgTile<D>;
  constexpr int B = kExtBlock;
  constexpr int KJ = D / 32;
  constexpr int NT = D / 16;
  constexpr uint32_t ROW = D * 2;
  const int col = lane & 15, grp = lane >> 4;
  const int tid = threadIdx.x;

  const int q0 = a.q_start[s];
  const int n = a.q_start[s + 1] - q0;
  const int L = min(max(a.context_lens[s], 0), a.max_blocks * B);
  const int ufirst = unit * kWaves * R * qpt;      // first query of the workgroup's row tiles
  const int ulast = min(n - 1, ufirst + kWaves * R * qpt - 1);
  const int p_max = L - n + ulast;                 // furthest position any row attends
  const int first = ufirst + wave * R * qpt;       // this wave's first query
  const int last = min(ulast, first + R * qpt - 1);
  const int p_lo = first <= last ? L - n + first : p_max;  // nearest position of the wave's rows

  int p_row[R];
  bool live[R];
  bf16x8 qop[R][KJ];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int f = first + rr * qpt;
    live[rr] = f <= last;
    const int qi = f + col / G;
    const bool row_ok = col < qpt * G && qi <= last;
    p_row[rr] = row_ok ? L - n + qi : p_max;       // padding slots: harmless finite rows
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

  const size_t blk_bytes = (size_t)a.num_kv_heads * B * D * 2;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool) + (size_t)g * B * ROW;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool) + (size_t)g * D * B * 2;
  // this thread's chunks: byte offset inside the K (and V) tile of a block,
  // and LDS offsets.  A 16-byte V chunk is 8 tokens of one dim: two 4-token
  // quads, stored 128 bytes apart; an 8-byte chunk is one quad.
  constexpr int CB = T::kChunk;
  const uint32_t goff = tid * CB;
  const uint32_t lk = (goff / ROW) * T::kStrideK + goff % ROW;
  const int vdim = goff / 32, vquad = (goff % 32) / 8;
  const uint32_t lv = T::kBytesK + (vdim >> 4) * 512 + vquad * 128 + (vdim & 15) * 8;
  const int vtok = vquad * 4;                      // first token of the chunk in its block
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;
  // blocks holding tokens 0 .. p_max (at least one, so that lengths shorter
  // than the query count, which the caller must not pass, still read in bounds)
  const int nblk = max(1, p_max / B + 1);

  // Block ids come from a window of the table row staged in LDS: a table
  // read from global memory would be counted with the K/V loads, and
  // waiting for it would drain every K/V load in flight.
  using Chunk = std::conditional_t<CB == 16, u32x4, u32x2>;
  Chunk kring[NPF], vring[NPF];
  int cn = 1;                                      // blocks in the current window
  auto gload = [&](int i, auto slot) {
    // the block id is the same in every lane: its offset is scalar work
    const size_t off = (size_t)__builtin_amdgcn_readfirstlane(tab[min(i, cn - 1)]) * blk_bytes;
    kring[slot] = *reinterpret_cast<const Chunk*>(kpool + off + goff);
    vring[slot] = *reinterpret_cast<const Chunk*>(vpool + off + goff);
  };
  // Stages block `blk` (index in the sequence) from ring slot `slot`.  V of
  // tokens past p_max (past every row, or past the context) is zeroed, so
  // stale bits never meet a zero probability.
  auto lstore = [&](auto slot, int buf, int blk) {
    uint8_t* t = lds + buf * T::kBytes;
    *reinterpret_cast<Chunk*>(t + lk) = kring[slot];
    uint32_t v[CB / 4];
    if constexpr (CB == 16) {
      v[0] = vring[slot].x; v[1] = vring[slot].y; v[2] = vring[slot].z; v[3] = vring[slot].w;
    } else {
      v[0] = vring[slot].x; v[1] = vring[slot].y;
    }
    if (blk * B + B - 1 > p_max) {                 // uniform: the block reaches past p_max
      const int tok = blk * B + vtok;
#pragma unroll
      for (int e = 0; e < CB / 2; ++e)
        if (tok + e > p_max) v[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
    }
    *reinterpret_cast<u32x2*>(t + lv) = u32x2{v[0], v[1]};
    if constexpr (CB == 16) *reinterpret_cast<u32x2*>(t + lv + 128) = u32x2{v[2], v[3]};
  };

  float m_ref[R], thr[R], l_run[R];               // thr = m_ref + kSlack
  f32x4 acc[R][NT];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    m_ref[rr] = kNegInf;
    thr[rr] = kNegInf;
    l_run[rr] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[rr][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int i, int buf) {
    const uint8_t* t = lds + buf * T::kBytes;
    u32x4 kb[KJ];
    u32x2 vq[NT];
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj)
      kb[kj] = *reinterpret_cast<const u32x4*>(t + col * T::kStrideK + kj * 64 + grp * 16);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      vq[nt] = *reinterpret_cast<const u32x2*>(t + T::kBytesK + nt * 512 + grp * 128 + col * 8);
    const int t0 = i * B + 4 * grp;                // this lane's first token of the tile
    f32x4 sc[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      sc[rr] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj)
        sc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[kj]),
                                                         qop[rr][kj], sc[rr], 0, 0, 0);
    }
    // Softmax of the R row tiles, stage by stage so that one wave-wide
    // branch covers the (rare) moves of any tile's reference and the rest
    // of the step is one basic block in which the compiler can interleave
    // the tiles' VALU work with their MFMAs.
    // With a positive scale (kPos) the scores stay unscaled until the
    // exponent: x = masked raw score, the lane's max is scaled once, and
    // p = exp2(fma(x, scale, -m)).  Otherwise x is the scaled score.
    float x[R][4], bm[R];
    // A block whose tokens every row of the wave sees (all but the blocks
    // near the diagonal and steps past the last block) skips the mask.
    const bool seen = i * B + B - 1 <= p_lo;
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[rr][r] = kPos ? sc[rr][r] : sc[rr][r] * a.scale_log2;
    if (!seen) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int lim = p_row[rr] - t0;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[rr][r] = r <= lim ? x[rr][r] : kNegInf;
      }
    }
    // bm: this lane's max of each row's scores.  A row's max passes its
    // threshold exactly when some lane's does, so the common path needs no
    // exchange between lanes; the (rare) branch that moves references takes
    // the max over the row's four lanes first.
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      bm[rr] = fmaxf(fmaxf(x[rr][0], x[rr][1]), fmaxf(x[rr][2], x[rr][3]));
      if constexpr (kPos) bm[rr] *= a.scale_log2;
    }
    bool grow = false;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) grow = grow || bm[rr] > thr[rr];
    if (__ballot(grow)) {                          // rare: move references that grew, rescale
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
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p[r] = kPos ? fexp2(fmaf(x[rr][r], a.scale_log2, -m_ref[rr])) : fexp2(x[rr][r] - m_ref[rr]);
      l_run[rr] += (p[0] + p[1]) + (p[2] + p[3]);
      // P rounded to bf16 (nearest even) is the A operand of a 16x16x16
      // MFMA whose B operand is the lane's V quad as read.  The softmax VALU
      // work, not the MFMAs, bounds this kernel: carrying P to 16 bits as the
      // decode does (a high and a low part, with V duplicated into a
      // 16x16x32 operand) cost 15%.  Its error stays within the bf16 bar: a
      // weight is off by at most 2^-9 of itself.
      const bf16x2 p01 = {static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1])};
      const bf16x2 p23 = {static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3])};
      const i16x4 pq = __builtin_bit_cast(
          i16x4, u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)});
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[rr][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pq, __builtin_bit_cast(i16x4, vq[nt]),
                                                                acc[rr][nt], 0, 0, 0);
    }
  };

  for (int w0 = 0; w0 < nblk; w0 += kExtTabWindow) {
    cn = min(kExtTabWindow, nblk - w0);
    for (int e = tid; e < cn; e += kWaves * 64) tab[e] = trow[w0 + e];
    __syncthreads();
    // prologue: the window's blocks 0 .. NPF - 1 in flight, block 0 staged
    static_for<NPF>([&](auto j) { gload(j, j); });
    lstore(std::integral_constant<int, 0>{}, 0, w0);
    gload(NPF, std::integral_constant<int, 0>{});
    __syncthreads();
    // block i of the window is in LDS buffer i & 1 and block i + 1 in ring
    // slot (i + 1) % NPF.  Steps run in whole groups of NPF without a
    // branch (so the compiler counts the loads in flight exactly): loads
    // past the window's last block re-read it, and a step past it computes
    // on that block with every token beyond p_max, so its scores are masked
    // and its V is zeroed.  The barrier closing each step also guards the
    // reuse of both buffers and of the table window.
    for (int i0 = 0; i0 < cn; i0 += NPF) {
      static_for<NPF>([&](auto j) {
        const int i = i0 + j;
        constexpr int nxt = (j + 1) % NPF;
        compute(w0 + i, i & 1);
        lstore(std::integral_constant<int, nxt>{}, (i + 1) & 1, w0 + i + 1);
        gload(i + 1 + NPF, std::integral_constant<int, nxt>{});
        __syncthreads();
      });
    }
  }

  // acc[rr][nt][r] holds slot 4*grp + r of row tile rr (query first + rr*qpt
  // + slot / G, head slot % G), dim nt*16 + col
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (!live[rr]) continue;
    float l_tot = sum_xor16(l_run[rr]);
    l_tot = sum_xor32(l_tot);
    float den[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) den[r] = lane_bcast(l_tot, 4 * grp + r);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int slot = 4 * grp + r;
      const int q = first + rr * qpt + slot / G;
      if (slot >= qpt * G || q > last) continue;
      const size_t ob = ((size_t)(q0 + q) * a.num_q_heads + g * G + slot % G) * D + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        static_cast<__bf16*>(a.out)[ob + nt * 16] = static_cast<__bf16>(acc[rr][nt][r] / den[r]);
    }
  }
}

template <int D, int R, int NPF, bool kPos>
__global__ __launch_bounds__(kWaves * 64, kExtWgPerCu) void extend_wg_kernel(ExtendArgs a, int G,
                                                                             int qpt) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2 * WgTile<D>::kBytes];
  __shared__ int tab_lds[kExtTabWindow];
  extern __shared__ int ext_lds[];
  int* pre = ext_lds;                 // [S + 1]
  int* wsum = ext_lds + a.num_seqs + 1;
  // a unit is the workgroup's 4R row tiles of qpt queries each
  const int tiles = build_extend_plan(a, kWaves * R * qpt, pre, wsum);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int units = tiles * a.num_kv_heads;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int g = u % a.num_kv_heads, k = u / a.num_kv_heads;
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= k) lo = mid; else hi = mid - 1;
    }
    int s = lo;
    while (pre[s + 1] <= k) ++s;  // skip sequences without queries
    s = __builtin_amdgcn_readfirstlane(s);
    extend_wg_unit<D, R, NPF, kPos>(a, G, qpt, s, k - pre[s], g, wave, lane, kv_lds, tab_lds);
  }
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
  const int qpt = std::max(1, 16 / G);
  // persistent grid: kExtWgPerCu workgroups per CU take the units in turn
  const size_t lds = ((size_t)a.num_seqs + 1 + 8) * sizeof(int);
  const int grid = std::max(1, std::min(cu_count_ext() * kExtWgPerCu, 1 << 16));
  // a positive scale folds into the exponent's fma; any other takes the
  // plain form
  if (a.scale_log2 > 0.f)
    extend_wg_kernel<D, kExtRows, kExtPrefetch, true><<<dim3(grid), dim3(kWaves * 64), lds, st>>>(a, G, qpt);
  else
    extend_wg_kernel<D, kExtRows, kExtPrefetch, false><<<dim3(grid), dim3(kWaves * 64), lds, st>>>(a, G, qpt);
  return hipGetLastError();
}

}  // namespace

bool extend_supported(pa_dtype dtype, int head_dim, int group, int block_size) {
  return dtype == PA_BF16 && block_size == kExtBlock && (head_dim == 64 || head_dim == 128) &&
         group >= 1 && group <= 16;
}

// Batches larger than kMaxPlanSeqs sequences run in slices (the plan lives
// in LDS); q_start holds absolute row indices, so only the per-sequence
// arrays move.
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
  return hipSuccess;
}

}  // namespace pakv
