// Paged decode attention for gfx950 (CDNA4, wave64).
//
// What is computed ("How PagedAttention Powers vLLM's KV Cache", section
// "The attention kernel has to read scattered blocks"; attention-lab
// "PagedAttention" page, reference entry "How it works"): for each sequence
// and query head, softmax(scale * q K^T) V over the sequence's logical tokens,
// reading K/V block by block through the sequence's block table.  The
// equation is the textbook one; only the gather is new.
//
// Work decomposition: one workgroup of 4 waves per (partition, kv head,
// sequence).  A partition is `partition_tokens` consecutive logical tokens
// (a multiple of the 16-token block).  The 4 waves take the partition's
// blocks round-robin, each keeping an online-softmax state (running max m,
// running sum l, unnormalised output o) for every query head of the group,
// and merge through LDS at the end.  A sequence that fits one partition is
// finished in place; otherwise the partition writes (m, l, o) to the
// workspace and decode_reduce_kernel combines them:
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
// Both stream each K/V byte of a (block, kv head) from HBM once, with the
// next block's loads issued before the current block is consumed.
#include "pa_internal.h"

namespace pakv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename V>
__device__ __forceinline__ V ldg_stream(const uint8_t* p) {
#if PA_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
#else
  return *reinterpret_cast<const V*>(p);
#endif
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

// Shared tail of both kernels: merge the per-wave states of one workgroup and
// write either the final output or this partition's partials.
//   sm_m, sm_l: [NW][16]; sm_o: [NW][GM][D]
template <typename T, int D, int GM, int NW>
__device__ __forceinline__ void merge_and_store(const DecodeArgs& a, int G, int s, int g,
                                                int part, int nparts, const float* sm_m,
                                                const float* sm_l, const float* sm_o) {
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D, e = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * 16 + h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fexp2(sm_m[w * 16 + h] - M);
      den += f * sm_l[w * 16 + h];
      num += f * sm_o[(w * GM + h) * D + e];
    }
    const int hq = g * G + h;
    if (nparts == 1) {
      store_out<T>(a.out, ((size_t)s * a.num_q_heads + hq) * D + e, num / den);
    } else {
      const size_t pi = ((size_t)s * a.num_q_heads + hq) * a.max_parts + part;
      a.part_o[pi * D + e] = num;
      if (e == 0) {
        a.part_m[pi] = M;
        a.part_l[pi] = den;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel: bf16 pools, G in (GM/2, GM] query heads per kv head.
// ---------------------------------------------------------------------------
template <int D, int GM>
__global__ __launch_bounds__(kWaves * 64) void decode_mfma_kernel(DecodeArgs a, int G) {
  constexpr int B = kBlock, NW = kWaves;
  constexpr int KJ = D / 32;  // q.K MFMAs per block (32 dims each)
  constexpr int NT = D / 16;  // P.V MFMAs per block (16 output dims each)
  constexpr size_t ROW = (size_t)D * 2;  // bytes per K row

  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int L = a.context_lens[s];
  const int P = a.partition_tokens;
  const int t0 = part * P;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + P);
  const int nparts = (L + P - 1) / P;
  const int jb = t0 / B, je = (t1 + B - 1) / B;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = a.num_kv_heads;

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

  const size_t blk_bytes = (size_t)Hkv * B * D * 2;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_pool) + (size_t)g * B * ROW +
                         col * ROW + grp * 16;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_pool) + (size_t)g * D * B * 2 +
                         col * (B * 2) + grp * 8;
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nblk = je - jb;
  const int nmine = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;

  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int cnt = min(64, nmine - c0);
    int tab = 0;
    if (lane < cnt) tab = trow[jb + wave + (c0 + lane) * NW];

    auto load = [&](int i, u32x4* kb, u32x2* vb) {
      const size_t off = (size_t)__builtin_amdgcn_readlane(tab, i) * blk_bytes;
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj)
        kb[kj] = ldg_stream<u32x4>(kbase + off + kj * 64);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        vb[nt] = ldg_stream<u32x2>(vbase + off + nt * 16 * (B * 2));
    };

    auto compute = [&](int i, const u32x4* kb, u32x2* vb) {
      const int j = jb + wave + (c0 + i) * NW;
      const int valid = min(B, L - j * B);
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[kj]),
                                                     qop[kj], sc, 0, 0, 0);
      // sc[r] = score of token 4*grp + r for head col
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[r] = (4 * grp + r < valid) ? sc[r] * a.scale_log2 : kNegInf;
      float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bm = fmaxf(bm, swap16(bm));
      bm = fmaxf(bm, swap32(bm));
      const float m_new = fmaxf(m_run, bm);
      const float alpha = fexp2(m_run - m_new);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fexp2(x[r] - m_new);
      l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m_run = m_new;
      if (__ballot(alpha != 1.f)) {
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = lane_bcast(alpha, 4 * grp + r);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[nt][r] *= ar[r];
      }
      // A operand of P.V: k slots 8*grp+0..3 = high bf16 of p[0..3],
      // 8*grp+4..7 = low bf16 (p - high, rounded to nearest even).
      uint32_t pb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[r] = __float_as_uint(p[r]);
      const bf16x2 lo01 = {static_cast<__bf16>(p[0] - bf16_hi(pb[0])),
                           static_cast<__bf16>(p[1] - bf16_hi(pb[1]))};
      const bf16x2 lo23 = {static_cast<__bf16>(p[2] - bf16_hi(pb[2])),
                           static_cast<__bf16>(p[3] - bf16_hi(pb[3]))};
      const u32x4 pw = {(pb[0] >> 16) | (pb[1] & 0xffff0000u),
                        (pb[2] >> 16) | (pb[3] & 0xffff0000u),
                        __builtin_bit_cast(uint32_t, lo01), __builtin_bit_cast(uint32_t, lo23)};
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
      if (valid < B) {  // zero V of slots past the context so stale bits never reach P.V
        const int t = 4 * grp;
        const uint32_t m0 = (t + 0 < valid ? 0x0000ffffu : 0u) | (t + 1 < valid ? 0xffff0000u : 0u);
        const uint32_t m1 = (t + 2 < valid ? 0x0000ffffu : 0u) | (t + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          vb[nt].x &= m0;
          vb[nt].y &= m1;
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const u32x4 vw = {vb[nt].x, vb[nt].y, vb[nt].x, vb[nt].y};
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop, __builtin_bit_cast(bf16x8, vw),
                                                          acc[nt], 0, 0, 0);
      }
    };

    u32x4 kb[kNBuf][KJ];
    u32x2 vb[kNBuf][NT];
#pragma unroll
    for (int b = 0; b < kNBuf - 1; ++b)
      if (b < cnt) load(b, kb[b], vb[b]);
    for (int i = 0; i < cnt; i += kNBuf) {
#pragma unroll
      for (int b = 0; b < kNBuf; ++b) {
        if (i + b >= cnt) break;
        const int nx = i + b + kNBuf - 1;
        if (nx < cnt) load(nx, kb[(b + kNBuf - 1) % kNBuf], vb[(b + kNBuf - 1) % kNBuf]);
        compute(i + b, kb[b], vb[b]);
      }
    }
  }

  // l over the four lane groups holding the same head
  float l_tot = l_run + swap16(l_run);
  l_tot += swap32(l_tot);

  __shared__ float sm_m[NW * 16], sm_l[NW * 16];
  __shared__ float sm_o[NW * GM * D];
  if (grp == 0) {
    sm_m[wave * 16 + col] = m_run;
    sm_l[wave * 16 + col] = l_tot;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      if (h < GM) sm_o[(wave * GM + h) * D + nt * 16 + col] = acc[nt][r];
    }
  __syncthreads();
  merge_and_store<__bf16, D, GM, NW>(a, G, s, g, part, nparts, sm_m, sm_l, sm_o);
}

// ---------------------------------------------------------------------------
// VALU kernel: fp32 or bf16 pools, G (template) query heads per kv head.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ __launch_bounds__(kWaves * 64) void decode_valu_kernel(DecodeArgs a) {
  constexpr int B = kBlock, NW = kWaves;
  constexpr int ES = sizeof(T);
  constexpr bool BF = ES == 2;
  constexpr int CH = 16 / ES;         // elements per 16-byte chunk
  constexpr int NC = D / CH / 4;      // q.K chunks per lane
  constexpr int QW = NC * 4;          // 32-bit words of q per head per lane
  constexpr int EPL = D / 64;         // output dims per lane
  constexpr int NV = EPL * B * ES / 16;  // 16-byte V loads per lane
  constexpr size_t ROW = (size_t)D * ES;

  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int L = a.context_lens[s];
  const int P = a.partition_tokens;
  const int t0 = part * P;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + P);
  const int nparts = (L + P - 1) / P;
  const int jb = t0 / B, je = (t1 + B - 1) / B;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tok = lane >> 2, qc = lane & 3;
  const int Hkv = a.num_kv_heads;

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

  const size_t blk_bytes = (size_t)Hkv * B * ROW;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_pool) + (size_t)g * B * ROW +
                         tok * ROW + qc * 16;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_pool) + (size_t)g * B * ROW +
                         lane * (EPL * B * ES);
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;

  float m_run[G], l_run[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int nblk = je - jb;
  const int nmine = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;

  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int cnt = min(64, nmine - c0);
    int tab = 0;
    if (lane < cnt) tab = trow[jb + wave + (c0 + lane) * NW];

    auto load = [&](int i, u32x4* kb, u32x4* vb) {
      const size_t off = (size_t)__builtin_amdgcn_readlane(tab, i) * blk_bytes;
#pragma unroll
      for (int jj = 0; jj < NC; ++jj)
        kb[jj] = ldg_stream<u32x4>(kbase + off + jj * 64);
#pragma unroll
      for (int v = 0; v < NV; ++v) vb[v] = ldg_stream<u32x4>(vbase + off + v * 16);
    };

    auto compute = [&](int i, const u32x4* kb, u32x4* vb) {
      const int j = jb + wave + (c0 + i) * NW;
      const int valid = min(B, L - j * B);
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
        sc[h] = tok < valid ? d * a.scale_log2 : kNegInf;
      }
      float p[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float bm = fmaxf(sc[h], dpp<kRowRor4>(sc[h]));
        bm = fmaxf(bm, dpp<kRowRor8>(bm));
        bm = fmaxf(bm, swap16(bm));
        bm = fmaxf(bm, swap32(bm));
        const float m_new = fmaxf(m_run[h], bm);
        const float alpha = fexp2(m_run[h] - m_new);
        p[h] = fexp2(sc[h] - m_new);
        l_run[h] = l_run[h] * alpha + (qc == 0 ? p[h] : 0.f);
        m_run[h] = m_new;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
      }
      if (valid < B) {  // zero V of slots past the context
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          uint32_t* w = reinterpret_cast<uint32_t*>(&vb[v]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // word q of load v covers tokens (word index within the row) ...
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

    u32x4 kb[kNBuf][NC], vb[kNBuf][NV];
#pragma unroll
    for (int b = 0; b < kNBuf - 1; ++b)
      if (b < cnt) load(b, kb[b], vb[b]);
    for (int i = 0; i < cnt; i += kNBuf) {
#pragma unroll
      for (int b = 0; b < kNBuf; ++b) {
        if (i + b >= cnt) break;
        const int nx = i + b + kNBuf - 1;
        if (nx < cnt) load(nx, kb[(b + kNBuf - 1) % kNBuf], vb[(b + kNBuf - 1) % kNBuf]);
        compute(i + b, kb[b], vb[b]);
      }
    }
  }

  __shared__ float sm_m[NW * 16], sm_l[NW * 16];
  __shared__ float sm_o[NW * G * D];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lt = wave_sum(l_run[h]);
    if (lane == 0) {
      sm_m[wave * 16 + h] = m_run[h];
      sm_l[wave * 16 + h] = lt;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_o[(wave * G + h) * D + lane * EPL + e] = acc[h][e];
  }
  __syncthreads();
  merge_and_store<T, D, G, NW>(a, G, s, g, part, nparts, sm_m, sm_l, sm_o);
}

// ---------------------------------------------------------------------------
// Split-context reduce: one wave per (query head, sequence).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, s = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = a.context_lens[s];
  const int P = a.partition_tokens;
  const int np = (L + P - 1) / P;
  if (np <= 1) return;
  const size_t base = ((size_t)s * a.num_q_heads + hq) * a.max_parts;
  float M = kNegInf;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, a.part_m[base + p]);
  M = wave_max(M);
  float den = 0.f;
  for (int p = lane; p < np; p += 64) den += fexp2(a.part_m[base + p] - M) * a.part_l[base + p];
  den = wave_sum(den);
  const float inv = 1.f / den;
  constexpr int EPL = D / 64;
  float num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float f = fexp2(a.part_m[base + p] - M);
    const float* po = a.part_o + (base + p) * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] = fmaf(f, po[e * 64 + lane], num[e]);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    store_out<T>(a.out, ((size_t)s * a.num_q_heads + hq) * D + e * 64 + lane, num[e] * inv);
}

template <typename T, int D>
hipError_t launch_reduce(const DecodeArgs& a, hipStream_t st) {
  if (a.max_parts <= 1) return hipSuccess;
  decode_reduce_kernel<T, D><<<dim3(a.num_q_heads, a.num_seqs), 64, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const DecodeArgs& a, int G, hipStream_t st) {
  const dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs), block(kWaves * 64);
  if (G <= 4) decode_mfma_kernel<D, 4><<<grid, block, 0, st>>>(a, G);
  else if (G <= 8) decode_mfma_kernel<D, 8><<<grid, block, 0, st>>>(a, G);
  else decode_mfma_kernel<D, 16><<<grid, block, 0, st>>>(a, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce<__bf16, D>(a, st);
}

template <typename T, int D>
hipError_t launch_valu(const DecodeArgs& a, int G, hipStream_t st) {
  const dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs), block(kWaves * 64);
  switch (G) {
    case 1: decode_valu_kernel<T, D, 1><<<grid, block, 0, st>>>(a); break;
    case 2: decode_valu_kernel<T, D, 2><<<grid, block, 0, st>>>(a); break;
    case 3: decode_valu_kernel<T, D, 3><<<grid, block, 0, st>>>(a); break;
    case 4: decode_valu_kernel<T, D, 4><<<grid, block, 0, st>>>(a); break;
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

hipError_t launch_decode(const DecodeArgs& a, pa_dtype dtype, int head_dim, int group,
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

}  // namespace pakv
