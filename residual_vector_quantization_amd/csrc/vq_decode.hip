// Decode, reconstruction error and MXFP4 kernels.
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
#include "vq_launch.hpp"

namespace vqk {

// ------------------------------------------------------------------ decode
// [VQ3R page] §2: w_hat = s * (((C1[i1] + C2[i2]) + C3[i3]) [+ C4[i4]]), summed
// left to right in fp32, then one fp32 multiply: one 8-dim vector into two
// float4, from codebooks in LDS.
// The decode and error kernels pad their LDS codebooks to CbPad<FMT>::P floats
// per codeword: with 32-byte rows codeword j starts on 16-byte bank group
// 2j mod 8, one of only 4 of the 8, and the random lookups of a wave collide
// more often; 48-byte rows (group 3j mod 8) spread them over all 8 (VQ3R
// decode 3.33 -> 3.02 ms on a 256-expert layer; relative errors 1.74 -> 1.65 ms).
// VQ4P's 64-entry codebooks gain nothing from it in either kernel and keep
// 32-byte rows.
template <int FMT> struct CbPad { static constexpr int P = FMT == 0 ? 12 : DIM; };

template <int FMT>
__device__ inline void decode_vec(const float (*cb)[Fmt<FMT>::K][CbPad<FMT>::P], uint32_t word, float s, int stages_used,
                                  float4* dst) {
  float acc[8];
  const float* c0 = cb[0][record_index<FMT>(word, 0)];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = c0[k];
  for (int t = 1; t < stages_used; ++t) {
    const float* c = cb[t][record_index<FMT>(word, t)];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = acc[k] + c[k];
  }
  dst[0] = make_float4(s * acc[0], s * acc[1], s * acc[2], s * acc[3]);
  dst[1] = make_float4(s * acc[4], s * acc[5], s * acc[6], s * acc[7]);
}

// A wave decodes chunks of 256 consecutive vectors, four consecutive ones per
// lane: the chunk's 768 record bytes are read as three dwords per lane (one
// contiguous 768-byte piece per wave). The lane's 128 bytes of output go
// through a per-wave LDS stage, slot x stored at x ^ ((x >> 3) & 7) so that
// both the lane-strided writes and the contiguous read-back are free of bank
// conflicts; every store instruction then writes 1 KB of contiguous output.
// The records and scales of the wave's next chunk are loaded before the
// current chunk's stores are issued: vector-memory counters complete in
// order, so loads issued after the stores would make the next chunk wait for
// them. The first chunk is peeled off the loop so that every entry into the
// loop has the same loads and stores in flight.
constexpr int DEC_CHUNK = 256;

__device__ inline int dec_slot(int x) { return x ^ ((x >> 3) & 7); }

template <int FMT, bool DWORD>
__global__ __launch_bounds__(256) void k_decode(const uint8_t* idx, const uint16_t* scales, const float* cb_g,
                                                uint32_t V, uint64_t nvec, int stages_used, float* out) {
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K;
  constexpr int CBP = CbPad<FMT>::P;
  __shared__ __align__(16) float cb[S][K][CBP];
  __shared__ float4 stage[4][2 * DEC_CHUNK];  // per wave: 256 vectors x 32 B
  for (int q = threadIdx.x; q < S * K * DIM; q += blockDim.x) (&cb[0][0][0])[(q >> 3) * CBP + (q & 7)] = cb_g[q];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float4* st = stage[wave];
  const uint64_t nfull = nvec / DEC_CHUNK;  // chunks of 256 vectors
  const uint64_t stride = (uint64_t)gridDim.x * 4;
  // row and in-row position of the chunk the next load() reads, advanced by
  // one wave stride per call without divisions (every call but the clamped
  // last one reads the next chunk of the sequence)
  const uint64_t nrows = nvec / V;
  const uint64_t cfirst = (uint64_t)blockIdx.x * 4 + wave;
  uint64_t lr = cfirst * DEC_CHUNK / V;
  uint32_t lo = (uint32_t)(cfirst * DEC_CHUNK - lr * V);
  const uint64_t dR = stride * DEC_CHUNK / V;
  const uint32_t dO = (uint32_t)(stride * DEC_CHUNK - dR * V);
  // records (one lane: vectors 4 lane .. 4 lane + 3) and scale bits of chunk c < nfull
  auto load = [&](uint64_t c, uint32_t (&d)[3], uint16_t (&sb)[4]) {
    const uint64_t v0 = c * DEC_CHUNK;
    const uint8_t* rec = idx + v0 * 3 + 12 * lane;
    if constexpr (DWORD) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(rec);
      d[0] = src[0];
      d[1] = src[1];
      d[2] = src[2];
    } else {
#pragma unroll
      for (int k = 0; k < 3; ++k)
        d[k] = (uint32_t)rec[4 * k] | ((uint32_t)rec[4 * k + 1] << 8) | ((uint32_t)rec[4 * k + 2] << 16) |
               ((uint32_t)rec[4 * k + 3] << 24);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t off = lo + (uint32_t)(4 * lane + q);  // relative to row lr (< V + 256)
      uint64_t row = lr + (V >= DEC_CHUNK ? (off >= V ? 1u : 0u) : off / V);
      row = row < nrows ? row : nrows - 1;
      sb[q] = scales[row];
    }
    lo += dO;  // the next chunk of the wave: DEC_CHUNK * stride vectors further
    lr += dR;
    if (lo >= V) {
      lo -= V;
      ++lr;
    }
  };
  auto body = [&](uint64_t c, const uint32_t (&d)[3], const uint16_t (&sb)[4], uint32_t (&dn)[3],
                  uint16_t (&sn)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // record q = bytes 3q .. 3q+2 of the lane's 12 bytes
      const int k0 = (3 * q) >> 2, o = (3 * q) & 3;
      const uint32_t w = (o <= 1) ? (d[k0] >> (8 * o)) : ((d[k0] >> (8 * o)) | (d[k0 + 1] << (32 - 8 * o)));
      float4 pr[2];
      decode_vec<FMT>(cb, w, f16_bits_to_f32(sb[q]), stages_used, pr);
      const int x = 2 * (4 * lane + q);
      st[dec_slot(x)] = pr[0];
      st[dec_slot(x + 1)] = pr[1];
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t cn = c + stride < nfull ? c + stride : c;  // clamped: the loads are unconditional
    load(cn, dn, sn);
    float4* dst = reinterpret_cast<float4*>(out + c * DEC_CHUNK * DIM);
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[64 * k + lane] = st[dec_slot(64 * k + lane)];
    __builtin_amdgcn_wave_barrier();
  };
  uint64_t c = (uint64_t)blockIdx.x * 4 + wave;
  if (c < nfull) {
    uint32_t d[3], dn[3];
    uint16_t sb[4], sn[4];
    load(c, d, sb);
    body(c, d, sb, dn, sn);
    for (c += stride; c < nfull; c += stride) {
#pragma unroll
      for (int k = 0; k < 3; ++k) d[k] = dn[k];
#pragma unroll
      for (int q = 0; q < 4; ++q) sb[q] = sn[q];
      body(c, d, sb, dn, sn);
    }
  }
  // the last nvec % 256 vectors: the wave whose chunk sequence reaches nfull
  const uint64_t ntail = nvec - nfull * DEC_CHUNK;
  if (ntail > 0 && c == nfull) {
    const uint64_t v0 = nfull * DEC_CHUNK;
    const int nv = (int)ntail;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = 4 * lane + q;
      if (j < nv) {
        const uint8_t* rec = idx + (v0 + j) * 3;
        const uint32_t w = (uint32_t)rec[0] | ((uint32_t)rec[1] << 8) | ((uint32_t)rec[2] << 16);
        float4 pr[2];
        decode_vec<FMT>(cb, w, f16_bits_to_f32(scales[(v0 + j) / V]), stages_used, pr);
        st[dec_slot(2 * j)] = pr[0];
        st[dec_slot(2 * j + 1)] = pr[1];
      }
    }
    __builtin_amdgcn_wave_barrier();
    float4* dst = reinterpret_cast<float4*>(out + v0 * DIM);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int x = 64 * k + lane;
      if (x < 2 * nv) dst[x] = st[dec_slot(x)];
    }
  }
}

hipError_t launch_decode(const DecodeArgs& a) {
  const uint64_t V = (uint64_t)(a.cols / DIM), nvec = (uint64_t)a.rows * V;
  if (nvec == 0) return hipSuccess;
  const uint64_t nchunks = (nvec + DEC_CHUNK - 1) / DEC_CHUNK;
  uint64_t g = (nchunks + 3) / 4;
  const uint64_t gmax = (uint64_t)a.ncu * 8;
  if (g > gmax) g = gmax;
  if (g < 1) g = 1;
  const bool dw = ((uintptr_t)a.idx & 3) == 0;
  auto go = [&](auto kern) {
    kern<<<(unsigned)g, 256, 0, a.stream>>>(a.idx, a.scales, a.codebooks, (uint32_t)V, nvec, a.stages_used, a.out);
  };
  if (a.format == 0) dw ? go(k_decode<0, true>) : go(k_decode<0, false>);
  else dw ? go(k_decode<1, true>) : go(k_decode<1, false>);
  return hipGetLastError();
}

// ------------------------------------------------------------------ error
// [VQ3R page] §3.1: ||W - W_hat||_F / ||W||_F. Per matrix, fp64 sums of
// (w - w_hat_t)^2 for the partial reconstructions after t = 1..S stages and of
// w^2, each 8-weight vector's terms first summed in fp32 (fp64 where fp32
// would lose range). The sums are grouped by fixed chunks of ERR_CHUNK rows: each chunk's
// partial has its own slot, whichever block computes it, and k_error_reduce
// adds the slots in chunk order. A matrix's result therefore depends only on
// its own data, not on the grid or on how many matrices share a call.
// Raw 8-element vector loads (converted to fp32 only where used, so that a
// load in flight does not force a wait).
template <int DT>
struct RawVec8 {
  uint4 q[DT == DT_F32 ? 2 : 1];
};
template <int DT>
__device__ inline RawVec8<DT> load_raw8(const void* row, int64_t j) {
  RawVec8<DT> r;
  const uint4* p = reinterpret_cast<const uint4*>(static_cast<const char*>(row) + j * 8 * (DT == DT_F32 ? 4 : 2));
#pragma unroll
  for (int h = 0; h < (DT == DT_F32 ? 2 : 1); ++h) r.q[h] = p[h];
  return r;
}
template <int DT>
__device__ inline void raw8_to_f32(const RawVec8<DT>& r, float v[8]) {
  if constexpr (DT == DT_F32) {
    const uint32_t u[8] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w, r.q[1].x, r.q[1].y, r.q[1].z, r.q[1].w};
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(u[k]);
  } else {
    const uint32_t u[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
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
// One item of the error kernel's load stream: its raw inputs.
template <int DT>
struct ErrSlot {
  uint32_t rlo, rhi;
  uint16_t sc;
  RawVec8<DT> w;
};

template <int FMT, int DT>
__global__ __launch_bounds__(256) void k_error(const void* W, const uint8_t* idx, const uint16_t* scales,
                                               const float* cb_g, uint32_t V, int64_t rows_per_mat, int64_t cols,
                                               int64_t nchunks, double* partials, WsHeader* hdr) {
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K;
  // codeword rows padded as in the decode (48 bytes for VQ3R): 4 workgroups fit a CU instead of 6, but the
  // random lookups of 32-byte rows spent about 0.59 of the cycles in bank conflicts
  constexpr int CBP = CbPad<FMT>::P;
  __shared__ __align__(16) float cb[S][K][CBP];
  __shared__ double red[S + 1][4];  // per-wave sums of a chunk
  for (int q = threadIdx.x; q < S * K * DIM; q += blockDim.x) (&cb[0][0][0])[(q >> 3) * CBP + (q & 7)] = cb_g[q];
  __syncthreads();
  const int m = blockIdx.y;
  const size_t esz = DT == DT_F32 ? 4 : 2;
  const uint64_t nvec_per_mat = (uint64_t)rows_per_mat * V;
  const uint8_t* idx_m = idx + (uint64_t)m * nvec_per_mat * 3;
  const uint16_t* sc_m = scales + (uint64_t)m * rows_per_mat;
  const char* W_m = (const char*)W + (uint64_t)m * nvec_per_mat * DIM * esz;
  // the wave index is the same on all lanes: readfirstlane tells the compiler,
  // so the stream bookkeeping below stays in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
  bool nonfinite = false;
  const uint32_t per_row = (V + 63) / 64;  // vector steps of a wave per row
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    double acc[S + 1];
#pragma unroll
    for (int t = 0; t <= S; ++t) acc[t] = 0.0;
    const int64_t r1 = (c + 1) * ERR_CHUNK < rows_per_mat ? (c + 1) * ERR_CHUNK : rows_per_mat;
    // One wave per row (rows c*ERR_CHUNK + wave, + nw, ...), vectors j = lane,
    // lane + 64, ... The wave's (row, j) items form one stream with two items
    // in flight: raw weights, record bytes and row scale are loaded two items
    // ahead, across row boundaries, and converted only when used.
    ErrSlot<DT> sl[2];
    const int64_t rbeg = c * ERR_CHUNK + wave;
    const uint32_t nrows = rbeg < r1 ? (uint32_t)((r1 - rbeg + nw - 1) / nw) : 0u;
    const uint32_t nit = nrows * per_row;  // the wave's items: (row rbeg + nw * (it / per_row), vector it % per_row)
    auto load = [&](ErrSlot<DT>& x, uint32_t it) {
      // unconditional loads from a clamped (row, vector) keep the wait counts
      // exact; items past the chunk or the row are never used
      const uint32_t ic = it < nit ? it : nit - 1;
      const uint32_t rr = ic / per_row;
      const int64_t row = rbeg + (int64_t)nw * rr;
      const uint32_t j = (uint32_t)lane + 64u * (ic - rr * per_row);
      const uint32_t jc = j < V ? j : V - 1;
      x.w = load_raw8<DT>(W_m + (uint64_t)row * cols * esz, jc);
      const uint8_t* pr = idx_m + ((uint64_t)row * V + jc) * 3;
      x.rlo = (uint32_t)pr[0] | ((uint32_t)pr[1] << 8);
      x.rhi = pr[2];
      x.sc = sc_m[row];
    };
    auto use = [&](const ErrSlot<DT>& x, uint32_t it, auto check) {
      if constexpr (decltype(check)::value) {
        const uint32_t rr = it / per_row;
        const uint32_t j = (uint32_t)lane + 64u * (it - rr * per_row);
        if (j >= V) return;
      }
      const float s = f16_bits_to_f32(x.sc);
      float w[8];
      raw8_to_f32<DT>(x.w, w);
      const uint32_t word = x.rlo | (x.rhi << 16);
      // The vector's sums in fp32, then added to the fp64 sums. The difference
      // after stage t is carried from stage to stage, d_t = d_(t-1) - s C_t[i_t]
      // (d_(-1) = w), one fused multiply-add per element. Each d_t is within
      // 2^-24 (|d_0| + ... + |d_t|) of the exact w - s (C_1 + ... + C_t), and
      // the decoder's w - w_hat_t is within 2^-24 (t + 2) |w_hat_t| of it (for
      // partial sums no larger than w_hat_t), so with |d| <= |w| and
      // |w_hat| ~ |w| the two differ by about 7 2^-24 |w| at most. By Cauchy-Schwarz a matrix's sum of d^2 then moves by at most
      // 14 2^-24 sqrt(sum d^2 * sum w^2), and its ratio by at most about
      // 7 2^-24 = 4e-7 in absolute terms (the fp32 sums of each vector's eight
      // terms add 4 2^-24 of the ratio), far inside the 1e-5 bar. Vectors whose
      // fp32 sums could overflow or lose range (non-finite, above 2^120, or sum
      // of w^2 below 2^-100) take the fp64 path instead, which forms w_hat_t as
      // the decoder does. tests/test_error_carry_cpu.py emulates this arithmetic
      // against the oracle, cancelling stages included.
      float dv[8], e[S + 1];
#pragma unroll
      for (int t = 0; t < S; ++t) {
        const float* cw = cb[t][record_index<FMT>(word, t)];
        float et;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          dv[k] = __builtin_fmaf(-s, cw[k], t == 0 ? w[k] : dv[k]);
          et = (k == 0) ? dv[k] * dv[k] : __builtin_fmaf(dv[k], dv[k], et);
        }
        e[t] = et;
      }
      float ew = w[0] * w[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) ew = __builtin_fmaf(w[k], w[k], ew);
      e[S] = ew;
      float emax = e[0];
#pragma unroll
      for (int t = 1; t < S; ++t) emax = fmaxf(emax, e[t]);
      if (emax <= 0x1p120f && ew <= 0x1p120f && ew >= 0x1p-100f) {
#pragma unroll
        for (int t = 0; t <= S; ++t) acc[t] += (double)e[t];
      } else {
        float p2[8];
#pragma unroll
        for (int t = 0; t < S; ++t) {
          const float* cw = cb[t][record_index<FMT>(word, t)];
          double et = 0.0;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            p2[k] = (t == 0) ? cw[k] : p2[k] + cw[k];
            const double d = (double)w[k] - (double)(s * p2[k]);
            et = __builtin_fma(d, d, et);
          }
          acc[t] += et;
        }
        double ewd = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) ewd = __builtin_fma((double)w[k], (double)w[k], ewd);
        acc[S] += ewd;
      }
    };
    // (scheduling barriers keep each reload behind the use of its slot; rows of
    // a multiple of 64 vectors need no per-lane range check, whose divergent
    // branch would make the compiler wait for both slots' loads)
    auto stream = [&](auto check) {
      load(sl[0], 0);
      __builtin_amdgcn_sched_barrier(0);
      load(sl[1], 1);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t it = 0;
      for (; it + 1 < nit; it += 2) {
        use(sl[0], it, check);
        __builtin_amdgcn_sched_barrier(0);
        load(sl[0], it + 2);
        __builtin_amdgcn_sched_barrier(0);
        use(sl[1], it + 1, check);
        __builtin_amdgcn_sched_barrier(0);
        load(sl[1], it + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (it < nit) use(sl[0], it, check);
    };
    if (nit > 0) {
      if ((V & 63) == 0) stream(std::false_type());
      else stream(std::true_type());
    }
    // a non-finite weight makes its thread's sum of squares non-finite; finite
    // weights cannot overflow it (|w| < 2^128 and fewer than 2^32 terms)
    nonfinite |= !__builtin_isfinite(acc[S]);
    // fixed-order reduction (butterfly within each wave, then the 4 waves in
    // order): a small LDS footprint next to the codebooks
#pragma unroll
    for (int t = 0; t <= S; ++t) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc[t] += __shfl_xor(acc[t], o);
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t <= S; ++t) red[t][wave] = acc[t];
    }
    __syncthreads();
    if (threadIdx.x <= S)
      partials[((uint64_t)m * nchunks + c) * (S + 1) + threadIdx.x] =
          ((red[threadIdx.x][0] + red[threadIdx.x][1]) + red[threadIdx.x][2]) + red[threadIdx.x][3];
    __syncthreads();  // red is reused by the next chunk
  }
  if (nonfinite) flag_status(hdr, ST_NONFINITE);
}

__global__ void k_error_reduce(const double* partials, int64_t nchunks, int nv, int64_t n_mats, double* sums) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_mats * nv) return;
  const int64_t m = q / nv, t = q % nv;
  double s = 0.0;
  for (int64_t c = 0; c < nchunks; ++c) s += partials[(m * nchunks + c) * nv + t];
  sums[q] = s;
}

// The Gate-3 metric ([VQ3R page] §3.1) from the sums: rel[m][t] =
// sqrt(sum (w - w_hat_{t+1})^2 / sum w^2) per matrix, and rel_all[t] over all
// matrices (numerator and denominator added over m in order, then the same
// ratio), in fp64 with correctly rounded division and square root. A matrix of
// zeros reconstructed as zeros has error 0. One workgroup; rel / rel_all may be
// NULL.
__global__ __launch_bounds__(256) void k_error_rel(const double* sums, int64_t n_mats, int S, double* rel,
                                                   double* rel_all) {
  auto ratio = [](double num, double den) {
    if (num == 0.0) return 0.0;
    return __dsqrt_rn(__ddiv_rn(num, den));
  };
  if (rel)
    for (int64_t q = threadIdx.x; q < n_mats * S; q += blockDim.x) {
      const int64_t m = q / S, t = q % S;
      rel[q] = ratio(sums[m * (S + 1) + t], sums[m * (S + 1) + S]);
    }
  if (rel_all && threadIdx.x < (unsigned)S) {
    const int t = threadIdx.x;
    double num = 0.0, den = 0.0;
    for (int64_t m = 0; m < n_mats; ++m) {
      num += sums[m * (S + 1) + t];
      den += sums[m * (S + 1) + S];
    }
    rel_all[t] = ratio(num, den);
  }
}

template <int FMT, int DT>
static hipError_t launch_error_t(const ErrorArgs& a) {
  constexpr int S = Fmt<FMT>::S;
  const uint64_t V = (uint64_t)(a.cols / DIM);
  const int64_t nchunks = error_chunks(a.rows);
  dim3 grid((unsigned)a.blocks, (unsigned)a.n_mats);
  k_error<FMT, DT><<<grid, 256, 0, a.stream>>>(a.W, a.idx, a.scales, a.codebooks, (uint32_t)V, a.rows, a.cols,
                                               nchunks, a.partials, a.hdr);
  const int64_t nq = a.n_mats * (S + 1);
  k_error_reduce<<<(unsigned)((nq + 255) / 256), 256, 0, a.stream>>>(a.partials, nchunks, S + 1, a.n_mats, a.sums);
  if (a.rel || a.rel_all) k_error_rel<<<1, 256, 0, a.stream>>>(a.sums, a.n_mats, S, a.rel, a.rel_all);
  return hipGetLastError();
}

hipError_t launch_error(const ErrorArgs& a) {
  hipError_t e0 = launch_reset(a.hdr, a.stream);
  if (e0 != hipSuccess) return e0;
  if (a.format == 0) {
    if (a.dtype == DT_F32) return launch_error_t<0, DT_F32>(a);
    if (a.dtype == DT_BF16) return launch_error_t<0, DT_BF16>(a);
    return launch_error_t<0, DT_F16>(a);
  }
  if (a.dtype == DT_F32) return launch_error_t<1, DT_F32>(a);
  if (a.dtype == DT_BF16) return launch_error_t<1, DT_BF16>(a);
  return launch_error_t<1, DT_F16>(a);
}

// ------------------------------------------------------------------ MXFP4
// [VQ3R page] §3.2 (K3 experts are MXFP4 at the source); the format is the
// OCP Microscaling v1.0 definition: 32-element blocks along the row share the
// E8M0 scale X = 2^(floor(log2 amax) - 2), clamped to [2^-127, 2^127]; elements
// are E2M1(w / X), nearest with ties to the even code, saturated at 6.
__device__ inline float e2m1_round(float a) {
  float q = (a < 2.0f) ? __builtin_rintf(2.0f * a) * 0.5f
                       : ((a < 4.0f) ? __builtin_rintf(a) : 2.0f * __builtin_rintf(0.5f * a));
  return fminf(q, 6.0f);
}

// Output: fp32, or (BF) its upper half as bf16. Every result X * e2m1 has at
// most two significant bits and lies in [2^-128, 1.5 * 2^127], so its fp32 bits
// end in 16 zero bits and the bf16 word holds it exactly.
template <int DT, bool BF>
__global__ __launch_bounds__(256) void k_mxfp4(const void* W, uint64_t nblk, void* out, WsHeader* hdr) {
  // 32 lanes per block of 32 elements (two blocks per wave)
  const int lane = threadIdx.x & 31;
  const uint64_t b0 = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) / 32;
  const uint64_t stride = ((uint64_t)gridDim.x * blockDim.x) / 32;
  for (uint64_t b = b0; b < nblk; b += stride) {  // b is uniform across each 32-lane group
    const uint64_t e = b * 32 + lane;
    float w = 0.0f;
    {
      if constexpr (DT == DT_F32) w = static_cast<const float*>(W)[e];
      else if constexpr (DT == DT_BF16) w = __uint_as_float((uint32_t)static_cast<const uint16_t*>(W)[e] << 16);
      else w = f16_bits_to_f32(static_cast<const uint16_t*>(W)[e]);
    }
    if (!__builtin_isfinite(w)) {
      flag_status(hdr, ST_NONFINITE);
      w = 0.0f;
    }
    float amax = __builtin_fabsf(w);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
    float r = 0.0f;
    if (amax > 0.0f) {
      int ex;
      frexpf(amax, &ex);  // floor(log2 amax) = ex - 1
      int xe = ex - 1 - 2;
      xe = xe < -127 ? -127 : (xe > 127 ? 127 : xe);
      const float X = ldexpf(1.0f, xe);
      const float v = __fdiv_rn(w, X);
      const float q = e2m1_round(__builtin_fabsf(v));
      r = X * (v < 0.0f ? -q : q);
    }
    if constexpr (BF) static_cast<uint16_t*>(out)[e] = (uint16_t)(__float_as_uint(r) >> 16);
    else static_cast<float*>(out)[e] = r;
  }
}

// The same with 8 lanes per block, 4 consecutive elements per lane: one 8- or
// 16-byte load and one 16-byte (fp32) or 8-byte (bf16) store per lane (each
// store instruction of a wave writes 1 KB or 512 B of contiguous output).
// Division by the power of two X is the multiplication by 2^-xe, exact as the
// correctly rounded quotient.
template <int DT, bool BF>
__global__ __launch_bounds__(256) void k_mxfp4_v4(const void* W, uint64_t nblk, void* out, WsHeader* hdr) {
  const int sub = threadIdx.x & 7;
  const uint64_t b0 = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;
  const uint64_t stride = ((uint64_t)gridDim.x * blockDim.x) >> 3;
  bool bad = false;
  for (uint64_t b = b0; b < nblk; b += stride) {  // b is uniform across each 8-lane group
    const uint64_t e = b * 32 + 4 * sub;
    float w[4];
    if constexpr (DT == DT_F32) {
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + e);
      w[0] = x.x;
      w[1] = x.y;
      w[2] = x.z;
      w[3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) + e);
      const uint32_t u[2] = {x.x, x.y};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint16_t h = (uint16_t)(u[k >> 1] >> (16 * (k & 1)));
        w[k] = DT == DT_BF16 ? __uint_as_float((uint32_t)h << 16) : f16_bits_to_f32(h);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!__builtin_isfinite(w[k])) {
        bad = true;
        w[k] = 0.0f;
      }
      amax = fmaxf(amax, __builtin_fabsf(w[k]));
    }
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 8));
    float r[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (amax > 0.0f) {
      int ex;
      frexpf(amax, &ex);  // floor(log2 amax) = ex - 1
      int xe = ex - 1 - 2;
      xe = xe < -127 ? -127 : (xe > 127 ? 127 : xe);
      const float X = ldexpf(1.0f, xe), Xi = ldexpf(1.0f, -xe);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float v = w[k] * Xi;
        const float q = e2m1_round(__builtin_fabsf(v));
        r[k] = X * (v < 0.0f ? -q : q);
      }
    }
    if constexpr (BF) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + e) =
          make_uint2((__float_as_uint(r[0]) >> 16) | (__float_as_uint(r[1]) & 0xFFFF0000u),
                     (__float_as_uint(r[2]) >> 16) | (__float_as_uint(r[3]) & 0xFFFF0000u));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + e) = make_float4(r[0], r[1], r[2], r[3]);
    }
  }
  if (bad) flag_status(hdr, ST_NONFINITE);
}

// ------------------------------------------------------------------ read reference
// A plain streaming read of n16 16-byte words (coalesced dwordx4 loads, grid
// stride, 8 loads in flight per thread): the bandwidth reference that the
// dequant-GEMV's HBM rate is compared with. The XOR of everything read decides
// a store that never happens for the bench's data, so no load is dead.
__global__ __launch_bounds__(512) void k_stream_read(const uint4* src, uint64_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

hipError_t launch_stream_read(const void* src, uint64_t nbytes, uint32_t* out, int ncu, hipStream_t s) {
  const uint64_t n16 = nbytes / 16;
  if (n16 == 0) return hipSuccess;
  uint64_t g = (n16 + 511) / 512;
  if (g > (uint64_t)ncu * 4) g = (uint64_t)ncu * 4;
  k_stream_read<<<(unsigned)g, 512, 0, s>>>(reinterpret_cast<const uint4*>(src), n16, out);
  return hipGetLastError();
}

template <bool BF>
static hipError_t launch_mxfp4_t(const Mxfp4Args& a, uint64_t nblk) {
  const size_t esz = a.dtype == DT_F32 ? 4 : 2;
  const uintptr_t out_align = BF ? 7 : 15;
  if (((uintptr_t)a.W & (4 * esz - 1)) == 0 && ((uintptr_t)a.out & out_align) == 0) {
    uint64_t g = (nblk * 8 + 255) / 256;
    if (g > (uint64_t)a.ncu * 16) g = (uint64_t)a.ncu * 16;
    if (a.dtype == DT_F32) k_mxfp4_v4<DT_F32, BF><<<(unsigned)g, 256, 0, a.stream>>>(a.W, nblk, a.out, a.hdr);
    else if (a.dtype == DT_BF16) k_mxfp4_v4<DT_BF16, BF><<<(unsigned)g, 256, 0, a.stream>>>(a.W, nblk, a.out, a.hdr);
    else k_mxfp4_v4<DT_F16, BF><<<(unsigned)g, 256, 0, a.stream>>>(a.W, nblk, a.out, a.hdr);
    return hipGetLastError();
  }
  uint64_t g = (nblk * 32 + 255) / 256;
  if (g > (uint64_t)a.ncu * 16) g = (uint64_t)a.ncu * 16;
  if (a.dtype == DT_F32) k_mxfp4<DT_F32, BF><<<(unsigned)g, 256, 0, a.stream>>>(a.W, nblk, a.out, a.hdr);
  else if (a.dtype == DT_BF16) k_mxfp4<DT_BF16, BF><<<(unsigned)g, 256, 0, a.stream>>>(a.W, nblk, a.out, a.hdr);
  else k_mxfp4<DT_F16, BF><<<(unsigned)g, 256, 0, a.stream>>>(a.W, nblk, a.out, a.hdr);
  return hipGetLastError();
}

hipError_t launch_mxfp4(const Mxfp4Args& a) {
  hipError_t e0 = launch_reset(a.hdr, a.stream);
  if (e0 != hipSuccess) return e0;
  const uint64_t nblk = (uint64_t)a.rows * (uint64_t)(a.cols / 32);
  if (nblk == 0) return hipGetLastError();
  return a.out_bf16 ? launch_mxfp4_t<true>(a, nblk) : launch_mxfp4_t<false>(a, nblk);
}

}  // namespace vqk
