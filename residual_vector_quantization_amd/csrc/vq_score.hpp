// Nearest-codeword search on one wave (gfx950): approximate scores from one of
// three engines, one value per group of GS consecutive codewords (the group's
// minimum score with the group id packed into its low bits; GS per format,
// Fmt<>::GS), a lane-local top-2 of those values, a merge of the two
// half-waves, then the exact distances of the winning group's codewords and
// the certification test of vq_device.hpp.
//
// Lane layout (shared by all engines): lane = 32*h + j holds the full 8-dim
// residual of vector j of the group; its candidates are the codewords
//   i = 32*tile + 8*(v/4) + 4*h + (v%4),  tile < K/32, v < 16,
// which is exactly the accumulator layout of the 32x32 MFMA instructions with
// codewords on M and vectors on N. Accumulator entries v0 .. v0+GS-1 (v0 a
// multiple of GS) of a tile are GS consecutive codewords: lane-local group id
// g = (16/GS)*tile + v0/GS (group_first gives its first codeword).
#pragma once
#include "vq_device.hpp"

namespace vqk {

enum { ENG_F16X = 1, ENG_F32 = 2, ENG_VALU = 3 };

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

// Per-stage engine tables in LDS.
template <int K, int ENG> struct Tables;
template <int K> struct Tables<K, ENG_F16X> {
  // hi = -2 fp16(c), lo = -2 fp16(c - fp16(c)) (the factor -2 of the score is
  // exact in fp16), nrm = {fp16(n'), fp16(n' - fp16(n')), 0...} with
  // n' = ||c||^2 * 2^-sigma (the matrix-core operands of the split scheme)
  h8 hi[K];
  h8 lo[K];
  h8 nrm[K];
};
template <int K> struct Tables<K, ENG_F32> {
  float a[4][2][K];             // step s: c_i[2s + half]
  alignas(16) float nrm[K];     // ||c_i||^2, the accumulators' initial value
};
template <int K> struct Tables<K, ENG_VALU> {
  float norm[K];     // ||c_i||^2
};

template <int FMT, int ENG, int NST>
struct SearchLds {
  static constexpr int K = Fmt<FMT>::K;
  static constexpr bool QUAD = ENG != ENG_VALU;  // codebook layout (vq_device.hpp)
  // fp32 codebooks: exact distances, residual updates
  alignas(16) float cb[NST][CbFloats<QUAD, K>::N];
  __device__ const float* row(int t, int r) const { return cb[t] + cb_offset<QUAD>(r); }
  __device__ float* row(int t, int r) { return cb[t] + cb_offset<QUAD>(r); }
  Tables<K, ENG> tab[NST];
  float sig[NST];              // 2^sigma of the norm term (F16X)
  uint32_t nmax_bits[NST];
};

// Builds the tables of stages [0, NST) from global fp32 codebooks
// cb_g[NST][K][8] (all threads of the block take part; ends with a barrier).
template <int FMT, int ENG, int NST>
__device__ inline void build_tables(SearchLds<FMT, ENG, NST>& L, const float* cb_g, WsHeader* hdr) {
  constexpr int K = Fmt<FMT>::K;
  const int tid = threadIdx.x, nt = blockDim.x;
  if (tid < NST) L.nmax_bits[tid] = 0u;
  __syncthreads();
  bool bad = false;
  for (int q = tid; q < NST * K; q += nt) {
    const int t = q / K, i = q % K;
    const float4* src = reinterpret_cast<const float4*>(cb_g + (size_t)q * DIM);
    float4 a = src[0], b = src[1];
    float c[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    double n = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      L.row(t, i)[k] = c[k];
      bad |= (__float_as_uint(c[k]) & 0x7FFFFFFFu) > 0x45000000u;  // |c| > 2048, inf or NaN (bit test)
      n += (double)c[k] * (double)c[k];
    }
    float nf = __double2float_rn(n);
    if constexpr (ENG == ENG_F32) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        L.tab[t].a[s][0][i] = c[2 * s];
        L.tab[t].a[s][1][i] = c[2 * s + 1];
      }
      L.tab[t].nrm[i] = nf;
    } else if constexpr (ENG == ENG_VALU) {
      L.tab[t].norm[i] = nf;
    } else {
      atomicMax(&L.nmax_bits[t], __float_as_uint(nf));
      h8 hi, lo;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        _Float16 x = (_Float16)c[k];
        hi[k] = x * (_Float16)(-2.0f);
        lo[k] = (_Float16)(c[k] - (float)x) * (_Float16)(-2.0f);
      }
      L.tab[t].hi[i] = hi;
      L.tab[t].lo[i] = lo;
    }
  }
  if (bad) flag_status(hdr, ST_CODEBOOK_RANGE);
  __syncthreads();
  if constexpr (ENG == ENG_F16X) {
    // sigma keeps n * 2^-sigma below 2^14, inside the fp16 range
    if (tid < NST) {
      int e = 0;
      frexpf(__uint_as_float(L.nmax_bits[tid]), &e);  // nmax < 2^e
      int sg = e > 14 ? e - 14 : 0;
      L.sig[tid] = ldexpf(1.0f, sg);
    }
    __syncthreads();
    for (int q = tid; q < NST * K; q += nt) {
      const int t = q / K, i = q % K;
      double n = 0.0;
#pragma unroll
      for (int k = 0; k < 8; ++k) n += (double)L.row(t, i)[k] * (double)L.row(t, i)[k];
      float ns = __double2float_rn(n) / L.sig[t];  // exact: division by a power of two
      _Float16 nh = (_Float16)ns;
      h8 v = {};
      v[0] = nh;
      v[1] = (_Float16)(ns - (float)nh);
      L.tab[t].nrm[i] = v;
    }
    __syncthreads();
  }
}

// ||r||^2 as the fmaf chain over k = 0..7 starting from 0.
__device__ inline float norm2_8(const float r[8]) {
  float rr = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) rr = __builtin_fmaf(r[k], r[k], rr);
  return rr;
}

// Initial accumulators of the fp32 engine for one 32-codeword tile: lane
// (vector, half h) holds the scores of codewords 8*(v/4) + 4h + v%4 in v, so
// they start from those codewords' ||c||^2 (four 16-byte reads) and the matrix
// products add -2 <r, c> on top.
__device__ inline f16v norm_init(const float* nrm, int tile, int h) {
  f16v acc;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 n4 = *reinterpret_cast<const float4*>(nrm + tile * 32 + 8 * q + 4 * h);
    acc[4 * q] = n4.x;
    acc[4 * q + 1] = n4.y;
    acc[4 * q + 2] = n4.z;
    acc[4 * q + 3] = n4.w;
  }
  return acc;
}

// Lane-local top-2 of the packed group values for stage t (one group of 32
// vectors per wave; both half-waves hold the same vector).
template <int FMT, int ENG, int NST>
__device__ inline void lane_top2(const SearchLds<FMT, ENG, NST>& L, int t, const float r[8], int lane,
                                 float& m1, float& m2) {
  constexpr int TILES = Fmt<FMT>::TILES, PACK = Fmt<FMT>::PACK, GS = Fmt<FMT>::GS, GPT = 16 / GS;
  const int h = lane >> 5, i = lane & 31;
  m1 = __builtin_inff();
  m2 = __builtin_inff();
  if constexpr (ENG == ENG_F16X) {
    h8 b0, b1;
    const _Float16 sg = (_Float16)L.sig[t];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      _Float16 x = (_Float16)r[k];
      _Float16 y = (_Float16)(r[k] - (float)x);
      b0[k] = x;
      b1[k] = h ? (k < 2 ? sg : (_Float16)0.0f) : y;
    }
    const h8* pa0 = h ? L.tab[t].lo : L.tab[t].hi;
    const h8* pa1 = h ? L.tab[t].nrm : L.tab[t].hi;
#pragma unroll
    for (int tile = 0; tile < TILES; ++tile) {
      f16v acc = {};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa0[tile * 32 + i], b0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa1[tile * 32 + i], b1, acc, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < GPT; q += 2)
        top2_pair(m1, m2, group_value<PACK, GS>(acc, GS * q, tile * GPT + q),
                  group_value<PACK, GS>(acc, GS * q + GS, tile * GPT + q + 1));
    }
  } else if constexpr (ENG == ENG_F32) {
    float b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = -2.0f * r[2 * s + h];
#pragma unroll
    for (int tile = 0; tile < TILES; ++tile) {
      f16v acc = norm_init(L.tab[t].nrm, tile, h);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(L.tab[t].a[s][h][tile * 32 + i], b[s], acc, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < GPT; q += 2)
        top2_pair(m1, m2, group_value<PACK, GS>(acc, GS * q, tile * GPT + q),
                  group_value<PACK, GS>(acc, GS * q + GS, tile * GPT + q + 1));
    }
  } else {
    float nr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) nr[k] = -2.0f * r[k];
#pragma unroll 2
    for (int tile = 0; tile < TILES; ++tile) {
      float acc[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ci = tile * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        const float* c = L.row(t, ci);
        float s = L.tab[t].norm[ci];
#pragma unroll
        for (int k = 0; k < 8; ++k) s = __builtin_fmaf(nr[k], c[k], s);
        acc[v] = s;
      }
#pragma unroll
      for (int q = 0; q < GPT; q += 2)
        top2_pair(m1, m2, group_value<PACK, GS>(acc, GS * q, tile * GPT + q),
                  group_value<PACK, GS>(acc, GS * q + GS, tile * GPT + q + 1));
    }
  }
}

// Merge of the two half-waves' top-2 (q0, n0: the low half's set; q1, n1: the
// high half's) into the overall p1 <= p2 and the first codeword of p1's group.
template <int PACK, int GS>
__device__ inline int merge_halves(float q0, float n0, float q1, float n1, float& p1, float& p2) {
  p1 = fmin2(q0, q1);
  p2 = fmin2(fmax2(q0, q1), fmin2(n0, n1));
  const uint32_t pb = __float_as_uint(p1);
  const int hw = (pb == __float_as_uint(q0)) ? 0 : 1;
  return group_first<GS>((int)(pb & ((1u << PACK) - 1u)), hw);
}

// Full stage (one group of 32 vectors per wave): approximate search, merge of
// the half-waves, exact resolution of the winning group, certification and
// residual update. Returns the winner index.
template <int FMT, int ENG, int NST>
__device__ inline int search_stage(const SearchLds<FMT, ENG, NST>& L, int t, float r[8], int lane, bool& flag) {
  constexpr int PACK = Fmt<FMT>::PACK, GS = Fmt<FMT>::GS;
  float m1, m2;
  lane_top2<FMT, ENG, NST>(L, t, r, lane, m1, m2);
  const int h = lane >> 5;
  const float o1 = __shfl_xor(m1, 32);
  const float o2 = __shfl_xor(m2, 32);
  float p1, p2;
  const int j0 = h ? merge_halves<PACK, GS>(o1, o2, m1, m2, p1, p2) : merge_halves<PACK, GS>(m1, m2, o1, o2, p1, p2);
  float rr = norm2_8(r);
  return resolve_group<PACK, GS, SearchLds<FMT, ENG, NST>::QUAD>(L.cb[t], j0, r, p1, p2,
                                                               ENG == ENG_F16X ? L.sig[t] : 0.0f, rr, flag);
}

// Two groups per pass (the matrix-core engines): lane (i, h) owns vector i of
// group h, so the per-vector work after the search (merge, exact resolution,
// certification, residual update, next operand set-up) serves 64 vectors per
// wave instruction. The matrix-core operands of group g need that group's
// residual in both half-waves (the K dimension is split across them); one
// v_permlane32_swap per register broadcasts each half's values to both
// halves. Returns the winner for the lane's own vector.
// rr: ||r||^2 on entry when RR_IN (else computed here); on return ||r'||^2 of
// the updated residual r' = r - C[w] (the winner's exact distance: the same
// fmaf chain over the same differences), so a later stage does not recompute it.
template <int FMT, int ENG, int NST, bool RR_IN>
__device__ inline int search_stage_x2(const SearchLds<FMT, ENG, NST>& L, int t, float r[8], int lane,
                                      bool& flag, float& rr) {
  static_assert(ENG == ENG_F16X || ENG == ENG_F32, "two-group search runs on the matrix-core engines");
  constexpr int TILES = Fmt<FMT>::TILES, PACK = Fmt<FMT>::PACK, GS = Fmt<FMT>::GS, GPT = 16 / GS;
  const int h = lane >> 5, i = lane & 31;
  float m1a = __builtin_inff(), m2a = __builtin_inff(), m1b = __builtin_inff(), m2b = __builtin_inff();
  if constexpr (ENG == ENG_F16X) {
    // own residual split into fp16 hi + lo (pairs converted together; the -2 of
    // the score sits in the codebook tables)
    typedef _Float16 hf2 __attribute__((ext_vector_type(2)));
    typedef float ff2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    // lo = RN16(r - hi) in one mixed-precision fma per element: v_fma_mix
    // forms r * 1 - hi exactly and rounds once to fp16 (into the low / high
    // half). r - hi is itself exact in fp32 (a rounding error of r, a multiple
    // of r's fp32 ulp below 2^13 of them), so these are the bits of converting hi
    // back, subtracting in fp32 and converting again, fp16 subnormals included
    // (the default fp16 denormal mode keeps them).
    u4 hw, lw;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const ff2 rv = {r[2 * q], r[2 * q + 1]};
      const uint32_t hp = __builtin_bit_cast(uint32_t, __builtin_convertvector(rv, hf2));
      uint32_t lo;
      asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(lo) : "v"(rv[0]), "v"(hp));
      asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "+v"(lo) : "v"(rv[1]), "v"(hp));
      hw[q] = hp;
      lw[q] = lo;
    }
    // the high half's operand of the second product: the norm term's factors
    // (2^sigma, 2^sigma, 0, ...)
    h8 cst = {};
    cst[0] = (_Float16)L.sig[t];
    cst[1] = cst[0];
    const u4 cw = __builtin_bit_cast(u4, cst);
    u4 hg0, hg1, lg0, lg1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // swap(x, x): result 0 = the low half's x in both halves, result 1 = the high half's
      const auto a = __builtin_amdgcn_permlane32_swap(hw[q], hw[q], false, false);
      hg0[q] = a[0];
      hg1[q] = a[1];
      // swap(lo, cst): result 0 = [low half's lo | cst], result 1 = [high half's lo | cst]
      const auto b = __builtin_amdgcn_permlane32_swap(lw[q], cw[q], false, false);
      lg0[q] = b[0];
      lg1[q] = b[1];
    }
    const h8 b0g0 = __builtin_bit_cast(h8, hg0), b0g1 = __builtin_bit_cast(h8, hg1);
    const h8 b1g0 = __builtin_bit_cast(h8, lg0), b1g1 = __builtin_bit_cast(h8, lg1);
    const h8* pa0 = h ? L.tab[t].lo : L.tab[t].hi;
    const h8* pa1 = h ? L.tab[t].nrm : L.tab[t].hi;
#pragma unroll
    for (int tile = 0; tile < TILES; ++tile) {
      const h8 a0 = pa0[tile * 32 + i], a1 = pa1[tile * 32 + i];
      f16v acc0 = {}, acc1 = {};
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0g0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0g1, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1g0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1g1, acc1, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < GPT; q += 2) {
        top2_pair(m1a, m2a, group_value<PACK, GS>(acc0, GS * q, tile * GPT + q),
                  group_value<PACK, GS>(acc0, GS * q + GS, tile * GPT + q + 1));
        top2_pair(m1b, m2b, group_value<PACK, GS>(acc1, GS * q, tile * GPT + q),
                  group_value<PACK, GS>(acc1, GS * q + GS, tile * GPT + q + 1));
      }
    }
  } else {
    // fp32 matrix cores (32x32x2): step s < 4 contracts dims 2s (low half) and
    // 2s+1 (high half), step 4 adds ||c||^2. swap(a = r[2s], b = r[2s+1]) gives
    // result 0 = [low half's r[2s] | low half's r[2s+1]] = group 0's operand and
    // result 1 = [high half's r[2s] | high half's r[2s+1]] = group 1's.
    float bg0[4], bg1[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(-2.0f * r[2 * s]),
                                                       __float_as_uint(-2.0f * r[2 * s + 1]), false, false);
      bg0[s] = __uint_as_float(sw[0]);
      bg1[s] = __uint_as_float(sw[1]);
    }
#pragma unroll
    for (int tile = 0; tile < TILES; ++tile) {
      float a[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = L.tab[t].a[s][h][tile * 32 + i];
      f16v acc0 = norm_init(L.tab[t].nrm, tile, h), acc1 = acc0;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], bg0[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], bg1[s], acc1, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < GPT; q += 2) {
        top2_pair(m1a, m2a, group_value<PACK, GS>(acc0, GS * q, tile * GPT + q),
                  group_value<PACK, GS>(acc0, GS * q + GS, tile * GPT + q + 1));
        top2_pair(m1b, m2b, group_value<PACK, GS>(acc1, GS * q, tile * GPT + q),
                  group_value<PACK, GS>(acc1, GS * q + GS, tile * GPT + q + 1));
      }
    }
  }
  // merge: for the lane's own group, q0 = top over the half-0 codeword set,
  // q1 = top over the half-1 set (swap(a, b): result 0 = [a of the low half,
  // b of the low half], result 1 = [a of the high half, b of the high half])
  const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m1a), __float_as_uint(m1b), false, false);
  const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m2a), __float_as_uint(m2b), false, false);
  float p1, p2;
  const int j0 = merge_halves<PACK, GS>(__uint_as_float(s1[0]), __uint_as_float(s2[0]), __uint_as_float(s1[1]),
                                    __uint_as_float(s2[1]), p1, p2);
  if constexpr (!RR_IN) rr = norm2_8(r);
  return resolve_group<PACK, GS, SearchLds<FMT, ENG, NST>::QUAD>(L.cb[t], j0, r, p1, p2,
                                                               ENG == ENG_F16X ? L.sig[t] : 0.0f, rr, flag);
}

// Per-wave staging of flagged vector ids in LDS. The ids of a wave gather in
// its LDS buffer and move to the global list in batches: one atomic on the
// shared list counter per batch instead of one per group with a flagged
// vector, each of which the wave had to wait for. The counter still ends at
// the total number of flagged vectors, and ids past `cap` are dropped as
// before (the overflow is detected from the counter).
constexpr int FLAG_STAGE = 128;  // staged ids per wave

struct FlagStage {
  uint32_t* buf;  // this wave's FLAG_STAGE LDS entries
  int cnt;        // fill, the same in every lane
};

__device__ inline void flag_flush(FlagStage& fs, uint32_t* counter, uint32_t* list, uint32_t cap, int lane) {
  if (fs.cnt == 0) return;
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(counter, (uint32_t)fs.cnt);
  base = __shfl(base, 0);
  for (int i = lane; i < fs.cnt; i += WAVE) {
    const uint32_t pos = base + (uint32_t)i;
    if (pos < cap) list[pos] = fs.buf[i];
  }
  __builtin_amdgcn_wave_barrier();  // the entries are read before they are overwritten
  fs.cnt = 0;
}

__device__ inline void flag_stage(FlagStage& fs, bool f, uint32_t vid, uint32_t* counter, uint32_t* list,
                                  uint32_t cap, int lane) {
  const uint64_t bal = __ballot(f);
  if (bal == 0) return;
  const int n = __popcll(bal);
  if (fs.cnt + n > FLAG_STAGE) flag_flush(fs, counter, list, cap, lane);
  if (f) fs.buf[fs.cnt + __popcll(bal & ((1ull << lane) - 1ull))] = vid;
  __builtin_amdgcn_wave_barrier();
  fs.cnt += n;
}

}  // namespace vqk
