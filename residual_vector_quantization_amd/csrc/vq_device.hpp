// Device-side building blocks shared by the libvq kernels (gfx950, wave64).
//
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace vqk {

constexpr int DIM = 8;
// Layouts of the search's fp32 codebooks in LDS (8 floats used per codeword).
//  - QUAD (the matrix-core engines): quads of 4 consecutive codewords (128
//    bytes), quads CB_QUAD floats (144 bytes) apart. A lane's exact resolution
//    reads the codewords of one group, which starts at a multiple of 4 (VQ3R)
//    or 2 (VQ4P): with evenly spaced rows the group starts of a wave fall on
//    few of the 8 16-byte bank groups (one with 32-byte rows, two with 48-byte
//    rows); quad m starts on bank group m mod 8.
//  - rows CB_ROW floats (48 bytes) apart (the fp32 VALU engine, whose two
//    half-waves read codewords 4 apart: 192 bytes, where quads measured slower).
constexpr int CB_QUAD = 36, CB_ROW = 12;
template <bool QUAD>
__device__ inline int cb_offset(int r) { return QUAD ? CB_QUAD * (r >> 2) + 8 * (r & 3) : CB_ROW * r; }
template <bool QUAD, int K>
struct CbFloats { static constexpr int N = QUAD ? K / 4 * CB_QUAD : K * CB_ROW; };
constexpr int WAVE = 64;

// ---------------------------------------------------------------- status
// Workspace header (first 256 bytes of every workspace).
enum : uint32_t {
  ST_NONFINITE = 1u << 0,       // a non-finite weight
  ST_SCALE_RANGE = 1u << 1,     // a row RMS beyond the fp16 range
  ST_CODEBOOK_RANGE = 1u << 2,  // a codebook entry non-finite or |c| > 2048
  ST_FIXED_POINT = 1u << 3,     // Lloyd fixed-point fraction bits below 16
  ST_ROUTE = 1u << 4,           // a GEMV route id outside [0, n_experts)
  ST_LIST_OVERFLOW = 1u << 8,   // informational: the exact pass covered every vector
  ST_ERROR_MASK = 0xFFu,
};

struct WsHeader {
  uint32_t flags;
  uint32_t n_flag[2];      // fixup-list fill (ping-pong between Lloyd iterations)
  uint32_t maxabs_bits[2]; // max |r| of the Lloyd training residual (ping-pong between stages)
  int32_t fbits;           // Lloyd fixed-point fraction bits of the current stage
  uint32_t pad[58];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

__device__ inline void flag_status(WsHeader* h, uint32_t f) { atomicOr(&h->flags, f); }

// ---------------------------------------------------------------- formats
// VQ3R: [VQ3R page] §2, 3 stages x 256 entries, 8-bit indices.
// VQ4P: [VQ3R page] §5, 4 stages x 64 entries, 6-bit indices in the same 3 bytes.
template <int FMT> struct Fmt;
// The search keeps one value per group of GS consecutive codewords (see
// vq_score.hpp); PACK = bits of the lane-local group id carried in a packed
// value (16 / GS groups per 32-codeword tile and lane: 16 * TILES / GS ids).
constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }
#ifndef VQ_GS_VQ3R
#define VQ_GS_VQ3R 4
#endif
#ifndef VQ_GS_VQ4P
#define VQ_GS_VQ4P 2
#endif
template <> struct Fmt<0> {
  static constexpr int S = 3, K = 256, BITS = 8, TILES = K / 32, GS = VQ_GS_VQ3R;
  static constexpr int PACK = ilog2c(16 * TILES / GS);
};
template <> struct Fmt<1> {
  static constexpr int S = 4, K = 64, BITS = 6, TILES = K / 32, GS = VQ_GS_VQ4P;
  static constexpr int PACK = ilog2c(16 * TILES / GS);
};

// 3-byte record = little-endian 24-bit word sum_t i_t << (t * BITS).
template <int FMT>
__device__ inline uint32_t record_word(const int* idx) {
  uint32_t w = 0;
#pragma unroll
  for (int t = 0; t < Fmt<FMT>::S; ++t) w |= (uint32_t)idx[t] << (t * Fmt<FMT>::BITS);
  return w;
}
template <int FMT>
__device__ inline int record_index(uint32_t word, int t) {
  return (int)((word >> (t * Fmt<FMT>::BITS)) & ((1u << Fmt<FMT>::BITS) - 1u));
}
__device__ inline void store_record(uint8_t* p, uint32_t w) {
  p[0] = (uint8_t)w;
  p[1] = (uint8_t)(w >> 8);
  p[2] = (uint8_t)(w >> 16);
}
__device__ inline uint32_t load_record(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
}

// ---------------------------------------------------------------- inputs
enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// Loads the 8 elements of vector j of a row as fp32 (exact widening).
template <int DT>
__device__ inline void load_vec8(const void* row, int64_t j, float v[8]) {
  if constexpr (DT == DT_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(row) + j * 8);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + j * 8);
    uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (DT == DT_BF16) {
        v[2 * k] = __uint_as_float(u[k] << 16);
        v[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
      } else {
        v[2 * k] = __half2float(__ushort_as_half((unsigned short)(u[k] & 0xFFFFu)));
        v[2 * k + 1] = __half2float(__ushort_as_half((unsigned short)(u[k] >> 16)));
      }
    }
  }
}

__device__ inline float f16_bits_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Non-finite (inf or NaN) test on the bit pattern: an all-ones exponent. The
// search kernels are compiled with NaN-free floating-point semantics (so that
// fminf / fmaxf need no sNaN-quieting operand canonicalization), under which a
// floating-point isfinite may be folded; the bit test cannot be.
__device__ inline bool is_nonfinite_bits(float x) { return (__float_as_uint(x) & 0x7F800000u) == 0x7F800000u; }
__device__ inline uint16_t f32_to_f16_bits(float f) { return __half_as_ushort(__float2half_rn(f)); }

// ---------------------------------------------------------------- row scale
// [VQ3R page] §2: one FP16 scale per row. Reading: the row RMS, fp64 sum of
// squares, sqrt(ss / n) in fp64, rounded fp64 -> fp32 -> fp16 to nearest even.
// One wave computes the scale of one row; returns the fp16 bits and sets
// *bad for a non-finite weight / an RMS beyond fp16.
template <int DT>
__device__ inline uint16_t wave_row_scale(const void* row, int64_t cols, int lane, uint32_t* bad) {
  const int64_t V = cols / DIM;
  double ss = 0.0;
  bool nonfinite = false;
  for (int64_t j = lane; j < V; j += WAVE) {
    float v[8];
    load_vec8<DT>(row, j, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      nonfinite |= is_nonfinite_bits(v[k]);
      ss += (double)v[k] * (double)v[k];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  uint32_t b = __any(nonfinite) ? ST_NONFINITE : 0u;
  double rms = __dsqrt_rn(__ddiv_rn(ss, (double)cols));
  uint16_t h = f32_to_f16_bits(__double2float_rn(rms));
  if ((h & 0x7C00u) == 0x7C00u && !b) b = ST_SCALE_RANGE;
  *bad = b;
  return h;
}

// Normalization ([VQ3R page] §2: codewords live in the row-scaled domain):
// v = w / s, one correctly rounded fp32 division; a zero scale gives v = 0.
__device__ inline float normalize(float w, float s) { return (s == 0.0f) ? 0.0f : __fdiv_rn(w, s); }

// The same quotients for a whole 8-vector, from the row's reciprocal
// y = RN(1/s) (row_recip; 0 for s = 0): q0 = RN(w y), rem = fma(-q0, s, w)
// (exact), q = fma(rem, y, q0) = RN(w / s) -- Markstein's correction step.
// The identity was checked exhaustively for every fp32 significand of w
// against every fp16 significand of s; it is scale-invariant while q, rem and
// the products stay clear of the subnormal range and of overflow, which
// |w| in [2^-100, 2^100] guarantees for an fp16 s. Vectors with an element
// outside that range (zero, tiny, huge, inf, NaN) or s = 0 take the division.
__device__ inline float row_recip(float s) { return (s == 0.0f) ? 0.0f : __fdiv_rn(1.0f, s); }

__device__ inline void normalize8(float r[8], float s, float y) {
  float lo = __builtin_fabsf(r[0]), hi = lo;
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    lo = __builtin_fminf(lo, __builtin_fabsf(r[k]));
    hi = __builtin_fmaxf(hi, __builtin_fabsf(r[k]));
  }
  if (__builtin_expect(lo >= 0x1p-100f && hi <= 0x1p100f && y != 0.0f, 1)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float q0 = r[k] * y;
      const float rem = __builtin_fmaf(-q0, s, r[k]);
      r[k] = __builtin_fmaf(rem, y, q0);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = normalize(r[k], s);
  }
}

// ---------------------------------------------------------------- exact search
// Squared distance in the fixed order of the definition: acc = 0;
// for k = 0..7: e = r_k - c_k; acc = fma(e, e, acc).
__device__ inline float dist8(const float r[8], const float* c) {
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float e = r[k] - c[k];
    acc = __builtin_fmaf(e, e, acc);
  }
  return acc;
}

// Exhaustive nearest codeword, j ascending, strictly smaller wins (ties to the
// lowest index). cb points at LDS [K][8]; all lanes read the same codeword.
template <int K>
__device__ inline int exact_argmin(const float r[8], const float* cb) {
  int best = 0;
  float bd = dist8(r, cb);
  for (int j = 1; j < K; ++j) {
    float d = dist8(r, cb + j * DIM);
    if (d < bd) {
      bd = d;
      best = j;
    }
  }
  return best;
}

// ---------------------------------------------------------------- certification
// The fast scorers produce approximate scores s_j ~ ||c_j||^2 - 2<r, c_j>
// (= T_j - ||r||^2, T_j the exact real distance) with
//   |error| <= ALPHA (||r|| + ||c_j||)^2 + 2^-22.5 (||r|| + ||c_j||) + 2^(sigma-25) + 2^-121.
// For the fp16-split engine: the three split products leave at most
// 6 2^-22 ||r|| ||c|| + 2^-22.5 (||r|| + ||c||) (fp16-subnormal parts round to
// 2^-25 absolute), the split norm term at most 1.25 2^-22 ||c||^2 + 2^(sigma-25)
// (its fp16 lo part is scaled by 2^-sigma), and fp32 accumulation of the 26
// exact products in any order at most 25 2^-24 (||r|| + ||c||)^2: 2^-18.6 in all,
// so ALPHA = 2^-16 has a 6x margin. The fp32 engines stay far inside the same
// bound with sigma = -inf.
// Codewords are taken in groups of GS (1, 2 or 4) consecutive indices; each
// group contributes one value, the minimum of its scores with the low PACK
// bits replaced by a lane-local group id. Let p1 <= p2 be the two smallest
// packed group values, G* the group of p1, d_j the exact fp32 distances (the
// fmaf chain of the definition) of the members of G*, w
// their argmin (lowest index on ties), dmax their maximum and rr = ||r||^2.
// Then the exhaustive search (the oracle) provably picks w whenever
//   p2 - p1 > delta = 1.25 * (2^-18 d_w + ALPHA (M_w + M_D) + 2^(PACK-22) (rr + dmax)
//                             + 2^-21 sqrt(M_D) + 2^-24 2^sigma + 2^-120),
//   M_w = (2 ||r|| + sqrt(1.001 d_w))^2,  M_D = (2 ||r|| + sqrt(1.001 dmax))^2.
// Reason: take j outside G* with d_j <= d_w and s* the member of G* with the
// smallest score (d_s* >= d_w). The chains are within 2^-20.7 relative of the
// real distances, so T_j - T_s* <= 2^-18 d_w, ||c_j|| <= ||r|| + sqrt(1.001 d_w)
// and ||c_s*|| <= ||r|| + sqrt(1.001 dmax), hence ||r|| + ||c|| <= sqrt(M_D) for
// both; their score errors add up to at most ALPHA (M_w + M_D) +
// 2^-21.5 sqrt(M_D) + 2^(sigma-24) + 2^-120, and the packing moves each of the
// two values by at most 2^(PACK-23) (rr + dmax). So p2 <= packed value of j's
// group <= p1 + delta / 1.25. Vectors that fail the test are re-encoded by the
// exact search.
// The test evaluates the bound without square roots (the hardware square root
// issues at a quarter of the VALU rate, and the test runs once per vector and
// stage). For a, b >= 0 and e > 0, 2ab <= e a^2 + b^2 / e, so
// (a + b)^2 <= (1 + e) a^2 + (1 + 1/e) b^2, an equality when b = e a. With
// e = 1/3 for M_w and e = 5/6 for M_D (the ratios sqrt(d)/(2||r||) of the
// encoder's residuals: d_w is about a third of rr, the group's farthest member
// about 2.8 rr), and sqrt(M_D) <= M_D/8 + 2:
//   M_w <= 16/3 rr + 4.004 d_w,  M_D <= 22/3 rr + 2.2022 dmax,
//   delta <= 1.25 (c_rr rr + c_w d_w + c_D dmax + 2^-20 + 2^-24 2^sigma + 2^-120),
// c_rr = 38/3 ALPHA + 2^(PACK-22) + 22/3 2^-24, c_w = 2^-18 + 4.004 ALPHA,
// c_D = 2.2022 (ALPHA + 2^-24) + 2^(PACK-22). On those residuals this is within
// 1 % of the bound with its square roots for half of the vectors and within 4 %
// for 9 in 10. The constants are rounded up (the factor 1 + 2^-20) and each of
// the four fmas adds a non-negative term and rounds once, so the fp32 value is
// at least the real bound.
constexpr float ALPHA = 1.52587890625e-05f;  // 2^-16

// sig = 2^sigma of the split norm term (0 for the fp32 engines).
template <int PACK>
__device__ inline bool certified(float p1, float p2, float rr, float dw, float dmax, float sig) {
  constexpr double A = 1.52587890625e-05, E24 = 5.9604644775390625e-08;  // 2^-16, 2^-24
  constexpr double PK = (double)(1u << PACK) * 2.384185791015625e-07;    // 2^(PACK-22)
  constexpr double UP = 1.25 * (1.0 + 9.5367431640625e-07);              // 1.25 (1 + 2^-20)
  constexpr float c_rr = (float)(UP * (38.0 / 3.0 * A + PK + 22.0 / 3.0 * E24));
  constexpr float c_w = (float)(UP * (3.814697265625e-06 + 4.004 * A));  // 2^-18 + 4.004 ALPHA
  constexpr float c_d = (float)(UP * (2.2022 * (A + E24) + PK));
  constexpr float c_0 = (float)(UP * (9.5367431640625e-07 + 7.52316384526264e-37));  // 2^-20 + 2^-120
  constexpr float c_s = (float)(UP * E24);
  float delta = __builtin_fmaf(c_s, sig, c_0);
  delta = __builtin_fmaf(c_d, dmax, delta);
  delta = __builtin_fmaf(c_w, dw, delta);
  delta = __builtin_fmaf(c_rr, rr, delta);
  return (p2 - p1) > delta;
}

// Packs a lane-local group id into the low PACK bits of a score.
template <int PACK>
__device__ inline float pack_score(float s, uint32_t local) {
  return __uint_as_float((__float_as_uint(s) & ~((1u << PACK) - 1u)) | local);
}

__device__ inline float fmin2(float a, float b) { return __builtin_fminf(a, b); }
__device__ inline float fmin3(float a, float b, float c) { return __builtin_fminf(__builtin_fminf(a, b), c); }
__device__ inline float fmax2(float a, float b) { return __builtin_fmaxf(a, b); }

// Top-2 streaming update with two new packed values x, y (m1 <= m2):
// second smallest of {m1, m2, x, y} = min(m2, med3(m1, x, y)).
__device__ inline void top2_pair(float& m1, float& m2, float x, float y) {
  float s = __builtin_amdgcn_fmed3f(m1, x, y);
  m2 = fmin2(m2, s);
  m1 = fmin3(m1, x, y);
}

// Packed group value of accumulator entries v0 .. v0+GS-1 (GS entries of the
// lane's layout): their minimum (GS = 4: min3 + min; GS = 8: three min3 and a
// min) with the lane-local group id g packed in.
template <int PACK, int GS, typename A>
__device__ inline float group_value(const A& acc, int v0, uint32_t g) {
  float m = acc[v0];
  if constexpr (GS == 2) m = fmin2(acc[v0], acc[v0 + 1]);
  if constexpr (GS == 4) m = fmin3(acc[v0], acc[v0 + 1], fmin2(acc[v0 + 2], acc[v0 + 3]));
  if constexpr (GS == 8)
    m = fmin3(fmin3(acc[v0], acc[v0 + 1], acc[v0 + 2]), fmin3(acc[v0 + 3], acc[v0 + 4], acc[v0 + 5]),
              fmin2(acc[v0 + 6], acc[v0 + 7]));
  return pack_score<PACK>(m, g);
}

// Codeword offset of member u of a group from its first codeword: entries
// v0 + u of the layout (codeword 8 (v / 4) + 4 h + v % 4), i.e. u for groups of
// up to 4 and u % 4 + 8 (u / 4) for groups of 8.
__device__ constexpr int group_member(int u) { return (u & 3) + 8 * (u >> 2); }

// First codeword of lane-local group g in half h (accumulator entries
// v0 = GS * (g mod 16/GS) of tile g / (16/GS)).
template <int GS>
__device__ inline int group_first(int g, int h) {
  constexpr int GPT = 16 / GS;  // groups per tile and lane
  const int tile = g / GPT, v0 = GS * (g % GPT);
  return tile * 32 + 8 * (v0 >> 2) + 4 * h + (v0 & 3);
}

// Exact resolution of the winning group: the exact fp32 distances of its GS
// codewords j0 + group_member(u) (the fmaf chain of the definition; members in
// increasing index order), their argmin with the lowest index on ties, the certificate against the runner-up group value
// p2 (sig: 2^sigma of the split norm term, 0 for the fp32 engines), and the
// residual update r <- r - C[w]. rr holds ||r||^2 on entry and
// ||r'||^2 of the updated residual on return (the winner's exact distance is
// the same fmaf chain over the same differences). Returns w.
template <int PACK, int GS, bool QUAD>
__device__ inline int resolve_group(const float* cbt, int j0, float r[8], float p1, float p2, float sig,
                                    float& rr, bool& flag) {
  float d[GS];
  // members u < 4 lie in j0's quad (j0 is a multiple of GS for GS <= 4), so
  // their rows sit at fixed offsets from the first one's
  const float* base = cbt + cb_offset<QUAD>(j0);
#pragma unroll
  for (int u = 0; u < GS; ++u) {
    const int gm = group_member(u);
    d[u] = dist8(r, gm < 4 ? base + (QUAD ? 8 : CB_ROW) * gm : cbt + cb_offset<QUAD>(j0 + gm));
  }
  int wu = 0;
  float dw = d[0], dmax = d[0];
#pragma unroll
  for (int u = 1; u < GS; ++u) {
    if (d[u] < dw) {  // strictly smaller: ties keep the lower index
      dw = d[u];
      wu = u;
    }
    dmax = __builtin_fmaxf(dmax, d[u]);
  }
  flag |= !certified<PACK>(p1, p2, rr, dw, dmax, sig);
  const int w = j0 + group_member(wu);
  const float* c = cbt + cb_offset<QUAD>(w);
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = r[k] - c[k];
  rr = dw;
  return w;
}

}  // namespace vqk
