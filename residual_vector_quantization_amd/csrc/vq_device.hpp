// Device-side building blocks shared by the libvq kernels (gfx950, wave64).
//
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace vqk {

constexpr int DIM = 8;
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
template <> struct Fmt<0> {
  static constexpr int S = 3, K = 256, BITS = 8, TILES = K / 32, PACK = 7;
};
template <> struct Fmt<1> {
  static constexpr int S = 4, K = 64, BITS = 6, TILES = K / 32, PACK = 5;
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
      nonfinite |= !__builtin_isfinite(v[k]);
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
// The fast scorers produce approximate scores s_i ~ ||c_i||^2 - 2<r, c_i>
// (= d_i - ||r||^2) with |error| <= ALPHA * (||r|| + ||c_i||)^2 + BETA, then
// replace the low PACK bits of each score by its lane-local candidate index.
// With p1 <= p2 the two smallest packed scores, w the index carried by p1,
// d_w the exact fp32 distance to C[w] and rr = ||r||^2, the exhaustive search
// (the oracle) provably picks w whenever
//   p2 - p1 > delta = 1.25 * (2^-18 d_w + 2 ALPHA M + 2^(PACK-22) (rr + d_w)
//                             + 2^-22 sqrt(M) + 2^-120),
//   M = (2 ||r|| + sqrt(1.001 d_w))^2,
// because any codeword at least as close as C[w] has ||c|| <= ||r|| + sqrt(d).
// Vectors that fail the test are re-encoded by the exact search.
constexpr float ALPHA = 1.52587890625e-05f;  // 2^-16, >= 4x the worst-case analysis
// Square root inside the bound only: the hardware instruction (within 1 ulp
// for normal arguments) on an argument raised to at least 2^-100. Its error is
// of the order of the fp32 roundings of the bound itself, which the factors
// 1.001 and 1.25 absorb; raising tiny arguments only makes the bound larger.
__device__ inline float bound_sqrt(float x) {
  return __builtin_amdgcn_sqrtf(__builtin_fmaxf(x, 7.888609052210118e-31f));
}

template <int PACK>
__device__ inline bool certified(float p1, float p2, float rr, float dw) {
  const float m = 2.0f * bound_sqrt(rr) + bound_sqrt(1.001f * dw);  // sqrt(M)
  const float M = m * m;
  const float pk = (float)(1u << PACK) * 2.384185791015625e-07f;  // 2^(PACK-22)
  float delta = 3.814697265625e-06f * dw + 2.0f * ALPHA * M + pk * (rr + dw) + 2.384185791015625e-07f * m +
                7.52316384526264e-37f;
  delta *= 1.25f;
  return (p2 - p1) > delta;
}

// Packs a lane-local candidate index into the low PACK bits of a score.
template <int PACK>
__device__ inline float pack_score(float s, uint32_t local) {
  return __uint_as_float((__float_as_uint(s) & ~((1u << PACK) - 1u)) | local);
}

__device__ inline float fmin2(float a, float b) { return __builtin_fminf(a, b); }

// Top-2 streaming update with two new packed values x, y (m1 <= m2):
// second smallest of {m1, m2, x, y} = min(m2, med3(m1, x, y)).
__device__ inline void top2_pair(float& m1, float& m2, float x, float y) {
  float s = __builtin_amdgcn_fmed3f(m1, x, y);
  m2 = fmin2(m2, s);
  m1 = fmin2(m1, fmin2(x, y));
}

}  // namespace vqk
