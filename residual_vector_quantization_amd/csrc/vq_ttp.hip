// Tied Trit-Planes 9-level codec, from the page "Новый метод квантования Tied
// Trit-Planes сжимает DeepSeek-V4 до 4.0625 бит на вес" ([TTP page]): PTQTP's
// two ternary planes with their scales tied by a factor of 3 form one uniform
// 9-level quantizer w ~ a (3 t1 + t2) = a q, q in -4..4, folded into a 4-bit
// code (summary and "what happened" sections), 4.0625 bits per weight.
//
// A group is 256 consecutive weights of a row with one fp16 scale. The solver
// alternates the two minimisations under the tie: nearest levels
// q = clamp(rint(w / a), -4, 4) for a fixed scale, then the least-squares scale
// a = sum w q / sum q^2 for fixed levels, from a = max|w| / 4, at most 8 rounds,
// stopping when no level changes; the stored scale is fp16(a) and the levels
// are chosen once more for it. The numerator is summed exactly in int64 fixed
// point (W_i = rint(w_i 2^F), F = 52 - e, max|w| < 2^e), so the sum does not
// depend on its order: one wave owns a group (4 weights per lane) and reduces
// across lanes, giving the same scale as a sequential evaluation.
//
// Codes: q + 4 (0..8), two per byte, the even element in the low nibble.
#include "vq_launch.hpp"
#include "vq_ttp.hpp"

namespace vqk {

constexpr int TTP_ITERS = 8;

__device__ inline int ttp_level(float w, float a) {
  if (a == 0.0f) return 0;
  float t = __builtin_rintf(__fdiv_rn(w, a));
  t = t > 4.0f ? 4.0f : t;
  t = t < -4.0f ? -4.0f : t;
  return (int)t;
}

template <int DT>
__device__ inline void load4(const void* W, int64_t i, float v[4]) {
  if constexpr (DT == DT_F32) {
    const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + i);
    v[0] = x.x;
    v[1] = x.y;
    v[2] = x.z;
    v[3] = x.w;
  } else {
    const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(W) + i);
    const uint32_t u[2] = {x.x, x.y};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t b = (uint16_t)(u[k >> 1] >> (16 * (k & 1)));
      v[k] = DT == DT_BF16 ? __uint_as_float((uint32_t)b << 16) : f16_bits_to_f32(b);
    }
  }
}

// Nearest levels from the reciprocal r = RN(1/a) where that provably gives the
// level of the rounded quotient: |w r - w / a| <= 2^-22.9 |w / a|, so for
// |w / a| < 5 the product and the rounded quotient lie within 1e-6 of each
// other and round to the same integer unless the product is within 2^-18 of a
// half-integer; at |w r| >= 5 both clamp to +-4. The weights that test leaves
// open (and every scale whose reciprocal is not a normal number) take the
// division.
__device__ inline bool ttp_recip(float a, float& r) {
  const float aa = __builtin_fabsf(a);
  if (!(aa >= 0x1p-125f && aa <= 0x1p125f)) return false;
  r = __fdiv_rn(1.0f, a);
  return true;
}
// levels of the lane's 4 weights: the reciprocal path, then the division for
// the weights it cannot settle, behind a wave-uniform branch
__device__ inline void ttp_levels4(const float w[4], float a, float r, bool use_r, int q[4]) {
  bool need = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float t = w[k] * r, at = __builtin_fabsf(t);
    float qq = __builtin_rintf(t);
    qq = qq > 4.0f ? 4.0f : (qq < -4.0f ? -4.0f : qq);
    q[k] = (int)qq;
    const float f = at - __builtin_floorf(at);
    need |= !(at >= 5.0f || __builtin_fabsf(f - 0.5f) > 0x1p-18f);
  }
  need |= !use_r;
  if (__builtin_expect(__any(need), 0)) {
    if (need) {
#pragma unroll
      for (int k = 0; k < 4; ++k) q[k] = ttp_level(w[k], a);
    }
  }
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline long long wave_sum_i64(long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ inline int wave_sum_i32(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// one wave per group, groups g = wave id, wave id + total waves, ...
template <int DT>
__global__ __launch_bounds__(256) void k_ttp_quantize(const void* W, int64_t n_groups, uint8_t* codes,
                                                      uint16_t* scales, WsHeader* hdr) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), nw = (int64_t)gridDim.x * 4;
  uint32_t bad = 0;
  for (int64_t g = wid; g < n_groups; g += nw) {
    float w[4];
    load4<DT>(W, g * TTP_GROUP + 4 * lane, w);
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!__builtin_isfinite(w[k])) bad |= ST_NONFINITE;
      am = fmaxf(am, fabsf(w[k]));
    }
    const float amax = wave_max(am);
    float a = amax * 0.25f;
    int e = 0;
    (void)frexpf(amax, &e);
    const int F = 52 - e;
    long long Wf[4];
    int q[4];
    float r = 0.0f;
    bool use_r = ttp_recip(a, r);
#pragma unroll
    for (int k = 0; k < 4; ++k) Wf[k] = (long long)__builtin_rint(ldexp((double)w[k], F));
    ttp_levels4(w, a, r, use_r, q);
    for (int it = 0; it < TTP_ITERS;) {
      long long swq = 0;
      int sqq = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        swq += Wf[k] * q[k];
        sqq += q[k] * q[k];
      }
      swq = wave_sum_i64(swq);
      sqq = wave_sum_i32(sqq);
      if (sqq == 0) break;  // uniform: the sums are the wave's
      a = (float)(ldexp((double)swq, -F) / (double)sqq);
      ++it;
      use_r = ttp_recip(a, r);
      bool changed = false;
      int nq[4];
      ttp_levels4(w, a, r, use_r, nq);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        changed |= nq[k] != q[k];
        q[k] = nq[k];
      }
      if (!__any(changed)) break;
    }
    const uint16_t h = f32_to_f16_bits(a);
    if ((h & 0x7C00u) == 0x7C00u) bad |= ST_SCALE_RANGE;
    const float ah = f16_bits_to_f32(h);
    float rh = 0.0f;
    const bool use_rh = ttp_recip(ah, rh);
    int qf[4];
    ttp_levels4(w, ah, rh, use_rh, qf);
    uint32_t c2 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) c2 |= (uint32_t)(qf[k] + 4) << (4 * k);
    reinterpret_cast<uint16_t*>(codes + g * (TTP_GROUP / 2))[lane] = (uint16_t)c2;
    if (lane == 0) scales[g] = h;
  }
  if (bad) flag_status(hdr, bad);
}

// 4 weights per thread and step: 16 bits of codes -> one float4 store, so each
// store instruction of a wave writes 1 KB of contiguous output
__global__ __launch_bounds__(256) void k_ttp_dequantize(const uint8_t* codes, const uint16_t* scales,
                                                        int64_t n_groups, float* out) {
  const int64_t n4 = n_groups * (TTP_GROUP / 4);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n4; t += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t c = reinterpret_cast<const uint16_t*>(codes)[t];
    const float a = f16_bits_to_f32(scales[t / (TTP_GROUP / 4)]);
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = a * (float)((int)((c >> (4 * k)) & 0xFu) - 4);
    reinterpret_cast<float4*>(out)[t] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// grid (chunks, n_mats): chunk c of matrix m = its groups [64c, 64c + 64); each of
// the 4 waves takes 16 of them; fp64 partials of (w - w_hat)^2 and w^2 per chunk.
template <int DT>
__global__ __launch_bounds__(256) void k_ttp_error(const void* W, const uint8_t* codes, const uint16_t* scales,
                                                   int64_t groups_per_mat, double* partials, WsHeader* hdr) {
  __shared__ double red[2][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m = blockIdx.y, c = blockIdx.x, chunks = gridDim.x;
  double d2 = 0.0, w2 = 0.0;
  bool bad = false;
  for (int i = 0; i < TTP_CHUNK / 4; ++i) {
    const int64_t gl = c * TTP_CHUNK + wave * (TTP_CHUNK / 4) + i;
    if (gl >= groups_per_mat) break;  // uniform over the wave
    const int64_t g = m * groups_per_mat + gl;
    float w[4];
    load4<DT>(W, g * TTP_GROUP + 4 * lane, w);
    const uint32_t cc = reinterpret_cast<const uint16_t*>(codes + g * (TTP_GROUP / 2))[lane];
    const float a = f16_bits_to_f32(scales[g]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bad |= !__builtin_isfinite(w[k]);
      const float wh = a * (float)((int)((cc >> (4 * k)) & 0xFu) - 4);
      const double d = (double)w[k] - (double)wh;
      d2 += d * d;
      w2 += (double)w[k] * (double)w[k];
    }
  }
  if (bad) flag_status(hdr, ST_NONFINITE);
  red[0][threadIdx.x] = d2;
  red[1][threadIdx.x] = w2;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      red[0][threadIdx.x] += red[0][threadIdx.x + o];
      red[1][threadIdx.x] += red[1][threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x < 2) partials[(m * chunks + c) * 2 + threadIdx.x] = red[threadIdx.x][0];
}

__global__ void k_ttp_error_reduce(const double* partials, int64_t chunks, int64_t n_mats, double* sums) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_mats * 2) return;
  const int64_t m = q / 2, t = q % 2;
  double s = 0.0;
  for (int64_t c = 0; c < chunks; ++c) s += partials[(m * chunks + c) * 2 + t];
  sums[q] = s;
}

hipError_t launch_ttp_quantize(const void* W, int dtype, int64_t n_groups, uint8_t* codes, uint16_t* scales,
                               WsHeader* hdr, int ncu, hipStream_t s) {
  hipError_t e0 = launch_reset(hdr, s);
  if (e0 != hipSuccess || n_groups == 0) return e0;
  int64_t blocks = (n_groups + 3) / 4;
  if (blocks > (int64_t)ncu * 32) blocks = (int64_t)ncu * 32;
  if (dtype == DT_F32) k_ttp_quantize<DT_F32><<<(unsigned)blocks, 256, 0, s>>>(W, n_groups, codes, scales, hdr);
  else if (dtype == DT_BF16) k_ttp_quantize<DT_BF16><<<(unsigned)blocks, 256, 0, s>>>(W, n_groups, codes, scales, hdr);
  else k_ttp_quantize<DT_F16><<<(unsigned)blocks, 256, 0, s>>>(W, n_groups, codes, scales, hdr);
  return hipGetLastError();
}

hipError_t launch_ttp_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t n_groups, float* out,
                                 int ncu, hipStream_t s) {
  if (n_groups == 0) return hipSuccess;
  const int64_t n4 = n_groups * (TTP_GROUP / 4);
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > (int64_t)ncu * 16) blocks = (int64_t)ncu * 16;
  k_ttp_dequantize<<<(unsigned)blocks, 256, 0, s>>>(codes, scales, n_groups, out);
  return hipGetLastError();
}

hipError_t launch_ttp_error(const void* W, int dtype, const uint8_t* codes, const uint16_t* scales,
                            int64_t groups_per_mat, int64_t n_mats, double* partials, double* sums, WsHeader* hdr,
                            hipStream_t s) {
  hipError_t e0 = launch_reset(hdr, s);
  if (e0 != hipSuccess) return e0;
  const int64_t chunks = (groups_per_mat + TTP_CHUNK - 1) / TTP_CHUNK;
  if (chunks > 0) {
    const dim3 grid((unsigned)chunks, (unsigned)n_mats);
    if (dtype == DT_F32) k_ttp_error<DT_F32><<<grid, 256, 0, s>>>(W, codes, scales, groups_per_mat, partials, hdr);
    else if (dtype == DT_BF16) k_ttp_error<DT_BF16><<<grid, 256, 0, s>>>(W, codes, scales, groups_per_mat, partials, hdr);
    else k_ttp_error<DT_F16><<<grid, 256, 0, s>>>(W, codes, scales, groups_per_mat, partials, hdr);
  }
  k_ttp_error_reduce<<<(unsigned)((n_mats * 2 + 255) / 256), 256, 0, s>>>(partials, chunks, n_mats, sums);
  return hipGetLastError();
}

}  // namespace vqk
