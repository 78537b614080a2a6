// Paged decode attention for gfx950 (CDNA4, wave64).
//
// What is computed ("How PagedAttention Powers vLLM's KV Cache", section
// "The attention kernel has to read scattered blocks"; attention-lab
// "PagedAttention" page, reference entry "How it works"): for each sequence
// and query head, softmax(scale * q K^T) V over the sequence's logical tokens,
// reading K/V block by block through the sequence's block table.  The
// equation is the textbook one; only the gather is new.
//
// Work decomposition: the unit of work is one (sequence, kv head,
// partition), where a partition is `partition_tokens` consecutive logical
// tokens (a multiple of the 16-token block), and ONE WAVE processes one unit
// from start to finish: it walks the unit's blocks in order, keeping a ring
// of register buffers so that several blocks' K/V loads are in flight while
// the oldest is consumed, and carries an online-softmax state (reference max
// m, running sum l, unnormalised output o) for every query head of the
// group.  A workgroup is 4 waves on 4 consecutive kv heads of the same
// (sequence, partition), so its waves have equal work.  The grid is
// persistent: each workgroup builds the list of units in LDS from the
// context lengths (full partitions first, then each sequence's partial last
// partition, longest first) and walks its share of it.  A sequence that
// fits one partition is finished in place; otherwise each unit writes
// (m, l, o) to the workspace and decode_reduce_kernel combines them:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// Scores are kept in log2 units (scale * log2 e folded in), so v_exp_f32
// (2^x) serves as the exponential.
//
// Two kernel families:
//  * decode_mfma_kernel (bf16, 3..16 query heads per kv head): q.K and P.V
//    run on v_mfma_f32_16x16x32_bf16.  For q.K, A = the 16 tokens of a block
//    x 32 dims, B = 32 dims x 16 head slots (the group's heads, zero padded).
//    Its output layout (lane holds tokens 4*(lane/16)+i of head lane%16) is
//    exactly the A layout P.V needs, so probabilities never leave the lane.
//    P is split into a bf16 high part (truncation) and a bf16 low part
//    (p - high, rounded), laid side by side along the MFMA's K dimension with
//    V repeated, so the product carries about 16 bits of P at no extra
//    instruction count.  V is stored dim-major in the pool so each lane's 4
//    tokens of one dim are one 8-byte load.
//  * decode_valu_kernel (fp32, or bf16 with 1..2 heads per kv head, where no
//    dense tile exists): 4 lanes per token share a K row for q.K
//    (v_dot2c_f32_bf16 for bf16), then each lane owns head_dim/64 output dims
//    and accumulates P.V with FMAs, P broadcast through v_readlane.
// Both stream each K/V byte of a (block, kv head) from HBM once.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "pa_internal.h"

namespace pakv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Global-memory (address space 1) byte pointer.
typedef const uint8_t __attribute__((address_space(1)))* gptr;

template <typename V>
__device__ __forceinline__ V ldg_stream(gptr p) {
  typedef const V __attribute__((address_space(1)))* vptr;
#if PA_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<vptr>(p));
#else
  return *reinterpret_cast<vptr>(p);
#endif
}

// A global pointer that is the same in every lane, moved to SGPRs so that
// loads can take the scalar-base + 32-bit-vector-offset form.
__device__ __forceinline__ gptr uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gptr>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1]; row rotate right by 4, 8.
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Lane i <-> lane i^16 (ds_swizzle bit mode: and 0x1F, xor 0x10).
__device__ __forceinline__ float swap16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
// Lane i <-> lane i^32.
__device__ __forceinline__ float swap32(float x) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(x)));
}
__device__ __forceinline__ float lane_bcast(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  x = fmaxf(x, dpp<kRowRor4>(x));
  x = fmaxf(x, dpp<kRowRor8>(x));
  x = fmaxf(x, swap16(x));
  return fmaxf(x, swap32(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  x += swap16(x);
  return x + swap32(x);
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(void* out, size_t idx, float v) {
  static_cast<float*>(out)[idx] = v;
}
template <>
__device__ __forceinline__ void store_out<__bf16>(void* out, size_t idx, float v) {
  static_cast<__bf16*>(out)[idx] = static_cast<__bf16>(v);  // v_cvt_pk_bf16_f32, RNE
}

// Work list.  A unit is (sequence s, partition p) for one group of kWaves
// kv heads; wave w of a workgroup takes kv head group * kWaves + w, so the
// four waves of a unit stream the same token range.  The grid is persistent
// (a few workgroups per CU) and every workgroup first builds the unit list
// in LDS from context_lens:
//   - full units: partition p < L_s / P of every sequence, sequence-major;
//   - then one partial unit per sequence with L_s % P > 0, sorted by length
//     in blocks, longest first (a counting sort over P/16 buckets),
// and then walks items blockIdx.x, blockIdx.x + gridDim.x, ...  Every item
// is real work (no empty workgroups for partitions past a short sequence's
// end), consecutive items sit on different XCDs (workgroups go to the 8
// XCDs round-robin), and each workgroup's last items are its smallest, so
// the launch ends on short units.  Which workgroup runs a unit does not
// change the unit's result.
struct Unit {
  int s, g, part, L, t0, t1, nparts;
};

struct Plan {
  const int* pre;    // [S + 1] full units before sequence s; pre[S] = NF
  const int* lens;   // [S] context lengths
  const int* plist;  // [S] sequences with a partial unit, longest first
  int S, NF, U, HG;
};

// Dynamic LDS bytes for a plan over S sequences with partition P.
__host__ __device__ constexpr size_t plan_lds_bytes(int S, int P) {
  return ((size_t)3 * S + 1 + 6 * (P / 16 + 2) + 8) * sizeof(int);
}

// Inclusive scan of one value per lane over a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute((lane - d) << 2, v);
    if (lane >= d) v += y;
  }
  return v;
}

// Exclusive scan of one value per thread over the 256-thread workgroup.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += wsum[w];
  if (total) *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return off + inc - v;
}

// Collective over the workgroup (256 threads); ends with a barrier.  Every
// workgroup builds the same plan from the same lengths, so nothing in it may
// depend on timing: counts use atomics (order-free), positions come from
// scans and ballots only.
__device__ Plan build_plan(const DecodeArgs& a, int* lds) {
  const int S = a.num_seqs, P = a.partition_tokens, NBK = P / 16, NB2 = NBK + 2;
  int* pre = lds;             // S + 1: full units before sequence s
  int* lens = pre + S + 1;    // S: clamped context lengths
  int* plist = lens + S;      // S: sequences with a partial unit, longest first
  int* base = plist + S;      // NB2: bucket count, then position of its first unit
  int* run = base + NB2;      // NB2: units of the bucket placed by earlier chunks
  int* cw = run + NB2;        // 4 * NB2: per-wave bucket counts of the current chunk
  int* wsum = cw + 4 * NB2;   // 8: scan scratch
  const int T = blockDim.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int b = t; b < NB2; b += T) {
    base[b] = 0;
    run[b] = 0;
  }
  const int C = (S + T - 1) / T;  // contiguous chunk of sequences per thread
  const int s0 = min(S, t * C), s1 = min(S, s0 + C);
  // lengths outside [0, table capacity] violate the contract; clamping them
  // keeps every LDS and table index in range whatever the device data says
  const int cap = a.max_blocks * kBlock;
  __syncthreads();
  int nfull = 0;
  for (int s = s0; s < s1; ++s) {
    const int L = min(max(a.context_lens[s], 0), cap);
    lens[s] = L;
    nfull += L / P;
    if (L % P) atomicAdd(&base[(L % P + 15) / 16], 1);
  }
  int NF;
  int run_full = block_excl_scan(nfull, wsum, &NF);
  for (int s = s0; s < s1; ++s) {
    pre[s] = run_full;
    run_full += lens[s] / P;
  }
  if (t == 0) pre[S] = NF;
  // bucket b holds partial units of b blocks; longest first: bucket NBK at 0
  int NPt = 0;
  for (int b0 = 0; b0 < NBK; b0 += T) {
    const int b = NBK - (b0 + t);
    const int c = (b >= 1) ? base[b] : 0;
    int tot;
    const int off = block_excl_scan(c, wsum, &tot);
    if (b >= 1) base[b] = NPt + off;
    NPt += tot;
    __syncthreads();
  }
  // stable placement, sequence order inside a bucket: chunks of T
  // consecutive sequences; a lane's rank among lower lanes of its wave with
  // the same bucket comes from ballots, earlier waves and chunks from counts
  for (int c0 = 0; c0 < S; c0 += T) {
    const int s = c0 + t;
    int b = 0;
    if (s < S) {
      const int r = lens[s] % P;
      if (r) b = (r + 15) / 16;
    }
    for (int i = lane; i < NB2; i += 64) cw[wave * NB2 + i] = 0;
    uint64_t todo = __ballot(b != 0);
    int rank = 0;
    while (todo) {
      const int leader = __builtin_ctzll(todo);
      const int bl = __builtin_amdgcn_readlane(b, leader);
      const uint64_t m = __ballot(b == bl);
      if (b == bl) rank = __builtin_popcountll(m & ((1ull << lane) - 1ull));
      if (lane == 0) cw[wave * NB2 + bl] = __builtin_popcountll(m);
      todo &= ~m;
    }
    __syncthreads();
    if (b) {
      int pos = base[b] + run[b] + rank;
      for (int w = 0; w < wave; ++w) pos += cw[w * NB2 + b];
      plist[pos] = s;
    }
    __syncthreads();
    for (int i = t; i < NB2; i += T)
      run[i] += (cw[i] + cw[NB2 + i]) + (cw[2 * NB2 + i] + cw[3 * NB2 + i]);
    __syncthreads();
  }
  Plan pl;
  pl.pre = pre;
  pl.lens = lens;
  pl.plist = plist;
  pl.S = S;
  pl.NF = NF;
  pl.U = NF + NPt;
  pl.HG = (a.num_kv_heads + kWaves - 1) / kWaves;
  return pl;
}

// The unit of `item` for this wave; false if the wave has no kv head there.
__device__ __forceinline__ bool plan_unit(const DecodeArgs& a, const Plan& pl, int item,
                                          int wave, Unit& u) {
  const int k = item / pl.HG;
  u.g = (item - k * pl.HG) * kWaves + wave;
  if (u.g >= a.num_kv_heads) return false;
  const int P = a.partition_tokens;
  if (k < pl.NF) {
    // largest s with pre[s] <= k (then pre[s + 1] > k: s has a full unit k)
    int lo = 0, hi = pl.S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pl.pre[mid] <= k) lo = mid; else hi = mid - 1;
    }
    u.s = lo;
    u.part = k - pl.pre[lo];
  } else {
    u.s = pl.plist[k - pl.NF];
    u.part = pl.pre[u.s + 1] - pl.pre[u.s];
  }
  u.L = pl.lens[u.s];
  u.t0 = u.part * P;
  u.t1 = min(u.L, u.t0 + P);
  u.nparts = (u.L + P - 1) / P;
  return true;
}

// Index of (sequence, query head, partition) in the partial buffers.
__device__ __forceinline__ size_t part_index(const DecodeArgs& a, int s, int hq, int part) {
  return ((size_t)s * a.num_q_heads + hq) * a.max_parts + part;
}

// Online softmax with a lazy reference: probabilities are 2^(x - m_ref) for a
// per-head reference m_ref that only moves when some head's block maximum
// exceeds it by more than kSlack (log2 units).  Until then the accumulators
// need no rescaling; probabilities stay below 2^kSlack, far from fp32 range
// limits, and the final (or split) normalisation divides the reference out
// exactly as it would a running maximum.
constexpr float kSlack = 8.f;

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Software pipeline over `cnt` blocks with a ring of NBUF register buffers:
// load(i, slot) issues block i's loads into ring slot `slot`; compute(i, slot)
// consumes it.  NBUF - 1 blocks are in flight while one is consumed.  The
// steady-state loop issues a load at every step, so the wait before each
// compute only covers the oldest buffer; the drain (at most 2*NBUF - 2
// blocks) is separate code, so its shorter waits do not leak into the loop.
// The prologue clamps its block indices so that it is unconditional (a unit
// shorter than the ring re-reads its last block into unused slots).
template <int NBUF, typename LoadF, typename ComputeF>
__device__ __forceinline__ void block_ring(int cnt, LoadF&& load, ComputeF&& compute) {
  static_for<NBUF - 1>([&](auto b) { load(min((int)b, cnt - 1), b); });
  int i = 0;
  for (; i + 2 * NBUF - 2 < cnt; i += NBUF) {
    static_for<NBUF>([&](auto b) {
      load(i + b + NBUF - 1, std::integral_constant<int, (b + NBUF - 1) % NBUF>{});
      compute(i + b, b);
    });
  }
  static_for<2 * NBUF - 2>([&](auto b) {
    if (i + b < cnt) {
      if (i + b + NBUF - 1 < cnt)
        load(i + b + NBUF - 1, std::integral_constant<int, (b + NBUF - 1) % NBUF>{});
      compute(i + b, std::integral_constant<int, b % NBUF>{});
    }
  });
}

// ---------------------------------------------------------------------------
// MFMA kernel: bf16 pools, G in (GM/2, GM] query heads per kv head.
// ---------------------------------------------------------------------------
template <int D, int GM, int NBUF>
__device__ __forceinline__ void mfma_unit(const DecodeArgs& a, int G, const Unit& u, int lane) {
  constexpr int B = kBlock;
  constexpr int KJ = D / 32;  // q.K MFMAs per block (32 dims each)
  constexpr int NT = D / 16;  // P.V MFMAs per block (16 output dims each)
  constexpr uint32_t ROW = D * 2;  // bytes per K row

  const int s = u.s, g = u.g, L = u.L;
  const int jb = u.t0 / B, je = (u.t1 + B - 1) / B;
  const int col = lane & 15, grp = lane >> 4;

  // B operand of q.K: lane holds q[head col][kj*32 + grp*8 .. +8]
  bf16x8 qop[KJ];
  {
    u32x4 w[KJ];
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj) w[kj] = u32x4{0u, 0u, 0u, 0u};
    if (col < G) {
      const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                          ((size_t)s * a.num_q_heads + g * G + col) * ROW + grp * 16;
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj) w[kj] = *reinterpret_cast<const u32x4*>(qp + kj * 64);
    }
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj) qop[kj] = __builtin_bit_cast(bf16x8, w[kj]);
  }

  // wave-uniform base of this kv head's slice of block 0, plus 32-bit lane
  // offsets: each load is a scalar block base + vector lane offset
  const size_t blk_bytes = (size_t)a.num_kv_heads * B * D * 2;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool) + (size_t)g * B * ROW;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool) + (size_t)g * D * B * 2;
  const uint32_t koff = col * ROW + grp * 16;
  const uint32_t voff = col * (B * 2) + grp * 8;
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;

  float m_ref = kNegInf, l_run = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 kring[NBUF][KJ];
  u32x2 vring[NBUF][NT];

  const int nblk = je - jb;
  for (int c0 = 0; c0 < nblk; c0 += 64) {
    const int cnt = min(64, nblk - c0);
    // physical block ids of up to 64 blocks, one per lane (every lane loads a
    // valid entry)
    const int tab = trow[jb + c0 + min(lane, cnt - 1)];

    auto load = [&](int i, auto slot) {
      const size_t off = (size_t)__builtin_amdgcn_readlane(tab, i) * blk_bytes;
      const gptr kblk = uniform_ptr(kpool + off);
      const gptr vblk = uniform_ptr(vpool + off);
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj) kring[slot][kj] = ldg_stream<u32x4>(kblk + koff + kj * 64);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        vring[slot][nt] = ldg_stream<u32x2>(vblk + voff + nt * 16 * (B * 2));
    };

    auto compute = [&](int i, auto slot) {
      u32x4* kb = kring[slot];
      u32x2* vb = vring[slot];
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[kj]),
                                                     qop[kj], sc, 0, 0, 0);
      // sc[r] = score of token 4*grp + r for head col
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = sc[r] * a.scale_log2;
      const int valid = L - (jb + c0 + i) * B;  // tokens of this block in the context
      if (valid < B) {
        // slots past the context: score -inf, V zeroed, so stale bits in an
        // unused tail slot never reach the output
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
      float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bm = fmaxf(bm, swap16(bm));
      bm = fmaxf(bm, swap32(bm));
      if (__ballot(bm > m_ref + kSlack)) {  // rare: move the reference, rescale
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
      // P.V on v_mfma_f32_16x16x16_bf16: A = P (16 head slots x 16 tokens;
      // this lane's 4 tokens are exactly its 4 scores), B = V (16 tokens x 16
      // dims; the lane's 8-byte V^T load).  P goes in twice: its high bf16
      // part (truncation), then the low part (p - high, rounded to nearest
      // even), which carries P to about 16 significant bits.
      uint32_t pb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[r] = __float_as_uint(p[r]);
      const bf16x2 lo01 = {static_cast<__bf16>(p[0] - bf16_hi(pb[0])),
                           static_cast<__bf16>(p[1] - bf16_hi(pb[1]))};
      const bf16x2 lo23 = {static_cast<__bf16>(p[2] - bf16_hi(pb[2])),
                           static_cast<__bf16>(p[3] - bf16_hi(pb[3]))};
      const i16x4 phi = __builtin_bit_cast(
          i16x4, u32x2{(pb[0] >> 16) | (pb[1] & 0xffff0000u), (pb[2] >> 16) | (pb[3] & 0xffff0000u)});
      const i16x4 plo = __builtin_bit_cast(
          i16x4, u32x2{__builtin_bit_cast(uint32_t, lo01), __builtin_bit_cast(uint32_t, lo23)});
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, __builtin_bit_cast(i16x4, vb[nt]),
                                                            acc[nt], 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, __builtin_bit_cast(i16x4, vb[nt]),
                                                            acc[nt], 0, 0, 0);
    };

    block_ring<NBUF>(cnt, load, compute);
  }

  // l over the four lane groups holding the same head; m_ref is uniform
  float l_tot = l_run + swap16(l_run);
  l_tot += swap32(l_tot);

  // acc[nt][r] holds head 4*grp + r, dim nt*16 + col
  if (u.nparts == 1) {
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
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      if (h >= G) continue;
      float* po = a.part_o + part_index(a, s, g * G + h, u.part) * D + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) po[nt * 16] = acc[nt][r];
    }
    if (grp == 0 && col < G) {
      const size_t pi = part_index(a, s, g * G + col, u.part);
      a.part_m[pi] = m_ref;
      a.part_l[pi] = l_tot;
    }
  }
}

template <int D, int GM, int NBUF>
__global__ __launch_bounds__(kWaves * 64, PA_MFMA_MIN_WG) void decode_mfma_kernel(DecodeArgs a, int G) {
  extern __shared__ int plan_lds[];
  const Plan pl = build_plan(a, plan_lds);
  // the wave index is uniform: keep it (and everything derived) in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int item = blockIdx.x; item < pl.U * pl.HG; item += gridDim.x) {
    Unit u;
    if (plan_unit(a, pl, item, wave, u)) mfma_unit<D, GM, NBUF>(a, G, u, lane);
  }
}

// ---------------------------------------------------------------------------
// VALU kernel: fp32 or bf16 pools, G (template) query heads per kv head.
// ---------------------------------------------------------------------------
template <typename T, int D, int G, int NBUF>
__device__ __forceinline__ void valu_unit(const DecodeArgs& a, const Unit& u, int lane) {
  constexpr int B = kBlock;
  constexpr int ES = sizeof(T);
  constexpr bool BF = ES == 2;
  constexpr int CH = 16 / ES;         // elements per 16-byte chunk
  constexpr int NC = D / CH / 4;      // q.K chunks per lane
  constexpr int QW = NC * 4;          // 32-bit words of q per head per lane
  constexpr int EPL = D / 64;         // output dims per lane
  constexpr int NV = EPL * B * ES / 16;  // 16-byte V loads per lane
  constexpr uint32_t ROW = D * ES;

  const int s = u.s, g = u.g, L = u.L;
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

  const size_t blk_bytes = (size_t)a.num_kv_heads * B * ROW;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool) + (size_t)g * B * ROW;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool) + (size_t)g * B * ROW;
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
            if constexpr (BF) {
              const float t = __builtin_amdgcn_fdot2_f32_bf16(
                  __builtin_bit_cast(bf16x2, kw[w]), __builtin_bit_cast(bf16x2, qw[h][jj * 4 + w]),
                  (w & 1) ? d1 : d0, false);
              if (w & 1) d1 = t; else d0 = t;
            } else {
              const float t = fmaf(__uint_as_float(kw[w]), __uint_as_float(qw[h][jj * 4 + w]),
                                   (w & 1) ? d1 : d0);
              if (w & 1) d1 = t; else d0 = t;
            }
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
            // word q of load v: token index within its V^T row
            const int word = (v * 4 + q) % (B * ES / 4);
            if constexpr (BF) {
              const int tk = word * 2;
              const uint32_t m = (tk < valid ? 0x0000ffffu : 0u) | (tk + 1 < valid ? 0xffff0000u : 0u);
              w[q] &= m;
            } else {
              if (word >= valid) w[q] = 0u;
            }
          }
        }
      }
      float bm[G];
      bool move = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        bm[h] = fmaxf(sc[h], dpp<kRowRor4>(sc[h]));
        bm[h] = fmaxf(bm[h], dpp<kRowRor8>(bm[h]));
        bm[h] = fmaxf(bm[h], swap16(bm[h]));
        bm[h] = fmaxf(bm[h], swap32(bm[h]));
        move |= bm[h] > m_ref[h] + kSlack;
      }
      if (__ballot(move)) {  // rare: move the references, rescale
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float m_new = fmaxf(m_ref[h], bm[h]);
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
          const int word = (e * B * ES + t * ES) / 4;  // word within this lane's V bytes
          const uint32_t w = reinterpret_cast<const uint32_t*>(vb)[word];
          float vv;
          if constexpr (BF) vv = (t & 1) ? bf16_hi(w) : bf16_lo(w);
          else vv = __uint_as_float(w);
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
    if (u.nparts == 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        store_out<T>(a.out, ((size_t)s * a.num_q_heads + hq) * D + lane * EPL + e, acc[h][e] / lt);
    } else {
      const size_t pi = part_index(a, s, hq, u.part);
#pragma unroll
      for (int e = 0; e < EPL; ++e) a.part_o[pi * D + lane * EPL + e] = acc[h][e];
      if (lane == 0) {
        a.part_m[pi] = m_ref[h];
        a.part_l[pi] = lt;
      }
    }
  }
}

template <typename T, int D, int G, int NBUF>
__global__ __launch_bounds__(kWaves * 64) void decode_valu_kernel(DecodeArgs a) {
  extern __shared__ int plan_lds[];
  const Plan pl = build_plan(a, plan_lds);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int item = blockIdx.x; item < pl.U * pl.HG; item += gridDim.x) {
    Unit u;
    if (plan_unit(a, pl, item, wave, u)) valu_unit<T, D, G, NBUF>(a, u, lane);
  }
}

// ---------------------------------------------------------------------------
// Split-context reduce: one workgroup of 4 waves per (query head, sequence).
// Wave w combines partitions w, w+4, ...; lanes own output dims; the four
// waves meet in LDS.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int NW = 4, EPL = D / 64, UNR = 4;
  const int hq = blockIdx.x, s = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L = min(a.context_lens[s], a.max_blocks * kBlock);  // as clamped by the plan
  const int P = a.partition_tokens;
  const int np = (L + P - 1) / P;
  if (np <= 1) return;  // finished by the partition kernel (or no context)
  const size_t base = part_index(a, s, hq, 0);
  const float* pm = a.part_m + base;
  const float* pl = a.part_l + base;

  __shared__ float sm_x[NW];
  __shared__ float sm_num[NW][D];
  float M = kNegInf;
  for (int p = threadIdx.x; p < np; p += NW * 64) M = fmaxf(M, pm[p]);
  M = wave_max(M);
  if (lane == 0) sm_x[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(sm_x[0], sm_x[1]), fmaxf(sm_x[2], sm_x[3]));
  __syncthreads();

  float den = 0.f, num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  for (int p0 = wave; p0 < np; p0 += NW * UNR) {
    float f[UNR], o[UNR][EPL];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int p = p0 + k * NW;
      f[k] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[k][e] = 0.f;
      if (p < np) {
        f[k] = fexp2(pm[p] - M);
        den = fmaf(f[k], pl[p], den);
        const float* po = a.part_o + (base + p) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[k][e] = po[e * 64 + lane];
      }
    }
#pragma unroll
    for (int k = 0; k < UNR; ++k)
#pragma unroll
      for (int e = 0; e < EPL; ++e) num[e] = fmaf(f[k], o[k][e], num[e]);
  }
  if (lane == 0) sm_x[wave] = den;
#pragma unroll
  for (int e = 0; e < EPL; ++e) sm_num[wave][e * 64 + lane] = num[e];
  __syncthreads();
  if (wave == 0) {
    const float dt = (sm_x[0] + sm_x[1]) + (sm_x[2] + sm_x[3]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = e * 64 + lane;
      const float n = (sm_num[0][i] + sm_num[1][i]) + (sm_num[2][i] + sm_num[3][i]);
      store_out<T>(a.out, ((size_t)s * a.num_q_heads + hq) * D + i, n / dt);
    }
  }
}

template <typename T, int D>
hipError_t launch_reduce(const DecodeArgs& a, hipStream_t st) {
  if (a.max_parts <= 1) return hipSuccess;
  decode_reduce_kernel<T, D><<<dim3(a.num_q_heads, a.num_seqs), 256, 0, st>>>(a);
  return hipGetLastError();
}

// Persistent grid: kDecodeWgPerCu workgroups per CU (the MFMA kernel's
// register budget is sized for 2), never more than there are items.
#ifndef PA_WG_PER_CU
#define PA_WG_PER_CU 2
#endif
constexpr int kDecodeWgPerCu = PA_WG_PER_CU;

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

struct Launch {
  dim3 grid, block;
  size_t lds;
};

Launch decode_launch(const DecodeArgs& a) {
  const int64_t hg = (a.num_kv_heads + kWaves - 1) / kWaves;
  const int64_t items = (int64_t)a.num_seqs * a.max_parts * hg;
  const int64_t wgs = std::min<int64_t>(items, (int64_t)cu_count() * kDecodeWgPerCu);
  return {dim3((unsigned)std::max<int64_t>(wgs, 1)), dim3(kWaves * 64),
          plan_lds_bytes(a.num_seqs, a.partition_tokens)};
}

template <int D>
hipError_t launch_mfma(const DecodeArgs& a, int G, hipStream_t st) {
  const Launch l = decode_launch(a);
  if (G <= 4) decode_mfma_kernel<D, 4, kNBuf><<<l.grid, l.block, l.lds, st>>>(a, G);
  else if (G <= 8) decode_mfma_kernel<D, 8, kNBuf><<<l.grid, l.block, l.lds, st>>>(a, G);
  else decode_mfma_kernel<D, 16, kNBuf><<<l.grid, l.block, l.lds, st>>>(a, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce<__bf16, D>(a, st);
}

template <typename T, int D>
hipError_t launch_valu(const DecodeArgs& a, int G, hipStream_t st) {
  const Launch l = decode_launch(a);
  switch (G) {
    case 1: decode_valu_kernel<T, D, 1, kNBuf><<<l.grid, l.block, l.lds, st>>>(a); break;
    case 2: decode_valu_kernel<T, D, 2, kNBuf><<<l.grid, l.block, l.lds, st>>>(a); break;
    case 3: decode_valu_kernel<T, D, 3, kNBuf><<<l.grid, l.block, l.lds, st>>>(a); break;
    case 4: decode_valu_kernel<T, D, 4, kNBuf><<<l.grid, l.block, l.lds, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce<T, D>(a, st);
}

}  // namespace

DecodePath decode_path(pa_dtype dtype, int head_dim, int group) {
  if (head_dim != 64 && head_dim != 128) return DecodePath::kUnsupported;
  if (group < 1) return DecodePath::kUnsupported;
  if (dtype == PA_BF16) {
    if (group <= 2) return DecodePath::kValu;
    if (group <= kMaxMfmaGroup) return DecodePath::kMfma;
    return DecodePath::kUnsupported;
  }
  if (dtype == PA_F32 && group <= 4) return DecodePath::kValu;
  return DecodePath::kUnsupported;
}

namespace {
hipError_t launch_decode_slice(const DecodeArgs& a, pa_dtype dtype, int head_dim, int group,
                               hipStream_t st) {
  switch (decode_path(dtype, head_dim, group)) {
    case DecodePath::kMfma:
      return head_dim == 128 ? launch_mfma<128>(a, group, st) : launch_mfma<64>(a, group, st);
    case DecodePath::kValu:
      if (dtype == PA_BF16)
        return head_dim == 128 ? launch_valu<__bf16, 128>(a, group, st)
                               : launch_valu<__bf16, 64>(a, group, st);
      return head_dim == 128 ? launch_valu<float, 128>(a, group, st)
                             : launch_valu<float, 64>(a, group, st);
    default:
      return hipErrorInvalidValue;
  }
}
}  // namespace

// Batches larger than kMaxPlanSeqs are launched in slices of that many
// sequences (the per-workgroup plan lives in LDS); every per-sequence array
// is offset to the slice.
hipError_t launch_decode(const DecodeArgs& a, pa_dtype dtype, int head_dim, int group,
                         hipStream_t st) {
  const size_t es = dtype == PA_BF16 ? 2 : 4;
  for (int32_t s0 = 0; s0 < a.num_seqs; s0 += kMaxPlanSeqs) {
    DecodeArgs b = a;
    b.num_seqs = std::min(kMaxPlanSeqs, a.num_seqs - s0);
    const size_t qrow = (size_t)a.num_q_heads * head_dim * es;
    b.q = static_cast<const uint8_t*>(a.q) + (size_t)s0 * qrow;
    b.out = static_cast<uint8_t*>(a.out) + (size_t)s0 * qrow;
    b.block_tables = a.block_tables + (size_t)s0 * a.max_blocks;
    b.context_lens = a.context_lens + s0;
    if (a.part_m) {
      const size_t pr = (size_t)s0 * a.num_q_heads * a.max_parts;
      b.part_m = a.part_m + pr;
      b.part_l = a.part_l + pr;
      b.part_o = a.part_o + pr * head_dim;
    }
    const hipError_t e = launch_decode_slice(b, dtype, head_dim, group, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pakv
