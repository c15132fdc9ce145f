// Encoder and Lloyd-fit kernels ([VQ3R page] §2 and §4: greedy residual
// encode through the stages, Lloyd k-means codebook fit on sampled experts).
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
#include "vq_launch.hpp"
#include "vq_score.hpp"

namespace vqk {

// ------------------------------------------------------------------ utility
__global__ void k_reset_header(WsHeader* h, int keep_flags) {
  if (threadIdx.x == 0) {
    if (!keep_flags) h->flags = 0;
    h->n_flag[0] = 0;
    h->n_flag[1] = 0;
    h->maxabs_bits[0] = 0;
    h->maxabs_bits[1] = 0;
    h->fbits = 0;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_row_scales(const void* W, int64_t rows, int64_t cols, uint16_t* scales,
                                                    WsHeader* hdr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t esz = DT == DT_F32 ? 4 : 2;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < rows; row += (int64_t)gridDim.x * 4) {
    uint32_t bad;
    uint16_t sb = wave_row_scale<DT>((const char*)W + row * cols * esz, cols, lane, &bad);
    if (lane == 0) {
      if (bad) flag_status(hdr, bad);
      scales[row] = sb;
    }
  }
}

// ------------------------------------------------------------------ encode
// One wave per row: the row scale, then groups of vectors through all
// stages (64 per group with the matrix-core engines, one per lane; 32 with the
// VALU engine, both half-waves working on the same vector). Certified vectors
// get their final record; the others are queued for the exact pass
// (k_encode_exact).
// With the matrix-core engines 8 waves per workgroup share one copy of the LDS
// tables (60 KB for VQ3R fp16-split, 72 KB fp32), so two workgroups give each
// SIMD 4 waves to interleave MFMA and VALU work; the VALU engine uses 4 waves.
constexpr bool two_groups(int eng) { return eng == ENG_F16X || eng == ENG_F32; }
constexpr int enc_waves(int eng) { return two_groups(eng) ? 8 : 4; }

template <int FMT, int ENG, int DT>
__global__ __launch_bounds__(64 * enc_waves(ENG), enc_waves(ENG) / 2) void k_encode(const void* W, int64_t rows, int64_t cols, const float* cb_g,
                                                   uint8_t* idx, uint16_t* scales, WsHeader* hdr, uint32_t* list,
                                                   uint32_t cap) {
  constexpr int S = Fmt<FMT>::S;
  constexpr bool X2 = two_groups(ENG);
  constexpr int GV = X2 ? 64 : 32;  // vectors per group
  constexpr int NWV = enc_waves(ENG);
  __shared__ SearchLds<FMT, ENG, S> L;
  __shared__ uint32_t fbuf[NWV][FLAG_STAGE];
  build_tables<FMT, ENG, S>(L, cb_g, hdr);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int jl = X2 ? lane : (lane & 31);
  const bool writer = X2 || h == 0;
  const int64_t V = cols / DIM;
  const size_t esz = DT == DT_F32 ? 4 : 2;
  FlagStage fs{fbuf[wave], 0};
  for (int64_t row = (int64_t)blockIdx.x * NWV + wave; row < rows; row += (int64_t)gridDim.x * NWV) {
    const void* wrow = (const char*)W + row * cols * esz;
    uint32_t bad;
    const uint16_t sb = wave_row_scale<DT>(wrow, cols, lane, &bad);
    if (lane == 0) {
      scales[row] = sb;
      if (bad) flag_status(hdr, bad);
    }
    if (bad) continue;
    const float s = f16_bits_to_f32(sb), y = row_recip(s);
    for (int64_t g = 0; g < V; g += GV) {
      const int64_t j = g + jl;
      const bool valid = j < V;
      float r[8];
      if (valid) {
        load_vec8<DT>(wrow, j, r);
        normalize8(r, s, y);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = 0.0f;
      }
      uint32_t word = 0;
      bool fl = false;
      float rr = norm2_8(r);
#pragma unroll 1
      for (int t = 0; t < S; ++t) {
        int w;
        if constexpr (X2) w = search_stage_x2<FMT, ENG, S, true>(L, t, r, lane, fl, rr);
        else w = search_stage<FMT, ENG, S>(L, t, r, lane, fl);
        word |= (uint32_t)w << (t * Fmt<FMT>::BITS);
      }
      const uint64_t vid = (uint64_t)row * V + j;
      if (valid && writer) store_record(idx + vid * 3, word);
      flag_stage(fs, fl && valid && writer, (uint32_t)vid, &hdr->n_flag[0], list, cap, lane);
    }
  }
  flag_flush(fs, &hdr->n_flag[0], list, cap, lane);
}

// Exact pass: every queued vector (or every vector when `all` is set or the
// queue overflowed) is re-encoded with the exhaustive fp32 search, one vector
// per thread, codebooks in LDS read in lockstep (broadcast).
template <int FMT, int DT>
__global__ __launch_bounds__(256) void k_encode_exact(const void* W, int64_t rows, int64_t cols, const float* cb_g,
                                                      uint8_t* idx, const uint16_t* scales, WsHeader* hdr,
                                                      const uint32_t* list, uint32_t cap, int all) {
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K;
  __shared__ float cb[S][K][DIM];
  const uint64_t V = (uint64_t)(cols / DIM), nvec = (uint64_t)rows * V;
  const uint32_t n = hdr->n_flag[0];
  const bool full = all || n > cap;
  const uint64_t total = full ? nvec : n;
  if ((uint64_t)blockIdx.x * blockDim.x >= total) return;
  if (full && !all && blockIdx.x == 0 && threadIdx.x == 0) flag_status(hdr, ST_LIST_OVERFLOW);
  for (int q = threadIdx.x; q < S * K * DIM; q += blockDim.x) (&cb[0][0][0])[q] = cb_g[q];
  __syncthreads();
  const size_t esz = DT == DT_F32 ? 4 : 2;
  for (uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t vid = full ? q : list[q];
    const uint64_t row = vid / V, j = vid % V;
    const float s = f16_bits_to_f32(scales[row]);
    float r[8];
    load_vec8<DT>((const char*)W + row * (uint64_t)cols * esz, (int64_t)j, r);
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = normalize(r[k], s);
    int out[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
      const int w = exact_argmin<K>(r, &cb[t][0][0]);
      out[t] = w;
#pragma unroll
      for (int k = 0; k < 8; ++k) r[k] = r[k] - cb[t][w][k];
    }
    store_record(idx + vid * 3, record_word<FMT>(out));
  }
}

// ------------------------------------------------------------------ Lloyd fit
// Training set: R[N][8] fp32, the row-normalized vectors of the sampled
// matrices (matrix, row, vector order). Stage t runs Lloyd on R_t and leaves
// the residual R_{t+1} = R_t - C_t[a] in the other buffer.

template <int DT>
__global__ __launch_bounds__(256) void k_fit_prepare(const void* W, int64_t rows, int64_t cols, float* R,
                                                     WsHeader* hdr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t V = cols / DIM;
  const size_t esz = DT == DT_F32 ? 4 : 2;
  uint32_t mx = 0;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < rows; row += (int64_t)gridDim.x * 4) {
    const void* wrow = (const char*)W + row * cols * esz;
    uint32_t bad;
    const uint16_t sb = wave_row_scale<DT>(wrow, cols, lane, &bad);
    if (bad) {
      if (lane == 0) flag_status(hdr, bad);
      continue;
    }
    const float s = f16_bits_to_f32(sb), y = row_recip(s);
    for (int64_t j = lane; j < V; j += WAVE) {
      float v[8];
      load_vec8<DT>(wrow, j, v);
      normalize8(v, s, y);
#pragma unroll
      for (int k = 0; k < 8; ++k) mx = max(mx, __float_as_uint(__builtin_fabsf(v[k])));
      float4* dst = reinterpret_cast<float4*>(R + (row * V + j) * DIM);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  if (lane == 0 && mx) atomicMax(&hdr->maxabs_bits[0], mx);
}

// Stage start: initial centroids C_t[k] = R_t[init[k]], fixed-point fraction
// bits F = 62 - e - ceil(log2 N) (max|R_t| < 2^e), counter resets.
template <int FMT>
__global__ void k_stage_begin(const float* R, const int64_t* init, float* C, WsHeader* hdr, int cur, int clog2n) {
  constexpr int K = Fmt<FMT>::K;
  for (int q = threadIdx.x; q < K * DIM; q += blockDim.x) C[q] = R[init[q / DIM] * DIM + (q % DIM)];
  if (threadIdx.x == 0) {
    const float mx = __uint_as_float(hdr->maxabs_bits[cur]);
    int e = 0;
    if (mx > 0.0f) frexpf(mx, &e);
    int F = 62 - e - clog2n;
    if (F < 16) {
      flag_status(hdr, ST_FIXED_POINT);
      F = 16;
    }
    hdr->fbits = F;
    hdr->n_flag[0] = 0;
    hdr->n_flag[1] = 0;
    hdr->maxabs_bits[cur ^ 1] = 0;
  }
}

template <int K>
struct FitAccum {
  unsigned long long sum[K][DIM + 1];  // int64 fixed-point sums (two's complement) and counts
};

template <int K>
__device__ inline void accum_vector(FitAccum<K>& A, int w, const float r[8], int F, int k0, int k1, bool count) {
  for (int k = k0; k < k1; ++k)
    atomicAdd(&A.sum[w][k], (unsigned long long)__double2ll_rn(ldexp((double)r[k], F)));
  if (count) atomicAdd(&A.sum[w][DIM], 1ull);
}

// The same sums with a two-instruction conversion, for |r 2^F| < 2^51: the
// fp64 fma x = r 2^F + 1.5 2^52 (the product is exact) lands in [2^52, 2^53),
// where consecutive doubles are consecutive integers, so x = 1.5 2^52 +
// rint(r 2^F) with ties to even, as llrint, and the bit pattern of x is that
// of 1.5 2^52 plus rint(r 2^F) as a two's complement int64. The block adds
// the patterns (mod 2^64) and subtracts count * bits(1.5 2^52) per cluster at
// the flush, leaving the exact sums.
constexpr unsigned long long FIX_BIAS_BITS = 0x4338000000000000ull;  // 1.5 * 2^52

template <int K>
__device__ inline void accum_vector_biased(FitAccum<K>& A, int w, const float r[8], double scale, int k0, int k1,
                                           bool count) {
  for (int k = k0; k < k1; ++k)
    atomicAdd(&A.sum[w][k], (unsigned long long)__double_as_longlong(__builtin_fma((double)r[k], scale, 0x1.8p52)));
  if (count) atomicAdd(&A.sum[w][DIM], 1ull);
}

template <int K>
__device__ inline void flush_accum(FitAccum<K>& A, long long* partials, int slot, bool biased) {
  __syncthreads();
  long long* dst = partials + (size_t)slot * K * (DIM + 1);
  for (int q = threadIdx.x; q < K * (DIM + 1); q += blockDim.x) {
    const int c = q / (DIM + 1), k = q % (DIM + 1);
    unsigned long long v = (&A.sum[0][0])[q];
    if (biased && k < DIM) v -= A.sum[c][DIM] * FIX_BIAS_BITS;
    dst[q] = (long long)v;
  }
}

// Assignment pass over R_cur. MODE 0 (iteration): certified vectors add their
// fixed-point coordinates to the block's cluster sums. MODE 1 (after the last
// update): certified vectors write their residual to R_next. Vectors that fail
// certification are staged per wave in LDS and resolved exactly at the end of
// the block; those that overflow a wave's stage are queued for k_assign_exact.
// Groups of 64 vectors (one per lane) with the matrix-core engines, 32 with the
// VALU engine.
template <int FMT, int ENG, int MODE>
__global__ __launch_bounds__(256, 2) void k_assign(const float* R_cur, float* R_next, int64_t n, const float* C,
                                                   WsHeader* hdr, uint32_t* list, uint32_t cap,
                                                   long long* partials, int parity, int nxt) {
  constexpr int K = Fmt<FMT>::K;
  constexpr bool X2 = two_groups(ENG);
  constexpr int GV = X2 ? 64 : 32;
  __shared__ SearchLds<FMT, ENG, 1> L;
  __shared__ FitAccum<K> A;
  __shared__ uint32_t fbuf[4][FLAG_STAGE];
  if (MODE == 0)
    for (int q = threadIdx.x; q < K * (DIM + 1); q += blockDim.x) (&A.sum[0][0])[q] = 0ull;
  build_tables<FMT, ENG, 1>(L, C, hdr);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int jl = X2 ? lane : (lane & 31);
  const bool writer = X2 || h == 0;
  const int F = hdr->fbits;
  // every |r| of this pass is below 2^e (the stage's residual maximum), so the
  // biased conversion applies when e + F <= 51
  int emax = 0;
  frexpf(__uint_as_float(hdr->maxabs_bits[nxt ^ 1]), &emax);
  const bool biased = emax + F <= 51;
  const double fscale = ldexp(1.0, F);
  uint32_t mx = 0;
  FlagStage fs{fbuf[wave], 0};
  const int64_t ngroups = (n + GV - 1) / GV;
  const int64_t gstride = (int64_t)gridDim.x * 4;
  // the next group's residuals are loaded while the current group is searched
  // (unconditional loads of a clamped vector index keep the wait counts exact)
  float4 na, nb;
  auto load_r = [&](int64_t g) {
    int64_t jj = g * GV + jl;
    jj = jj < n ? jj : n - 1;
    const float4* p = reinterpret_cast<const float4*>(R_cur + jj * DIM);
    na = p[0];
    nb = p[1];
  };
  load_r((int64_t)blockIdx.x * 4 + wave);
  for (int64_t g = (int64_t)blockIdx.x * 4 + wave; g < ngroups; g += gstride) {
    const int64_t j = g * GV + jl;
    const bool valid = j < n;
    float r[8], r0[8];
    r[0] = na.x; r[1] = na.y; r[2] = na.z; r[3] = na.w; r[4] = nb.x; r[5] = nb.y; r[6] = nb.z; r[7] = nb.w;
    if (!valid) {
#pragma unroll
      for (int k = 0; k < 8; ++k) r[k] = 0.0f;
    }
    load_r(g + gstride < ngroups ? g + gstride : g);
#pragma unroll
    for (int k = 0; k < 8; ++k) r0[k] = r[k];
    bool fl = false;
    int w;
    float rr;
    if constexpr (X2) w = search_stage_x2<FMT, ENG, 1, false>(L, 0, r, lane, fl, rr);
    else w = search_stage<FMT, ENG, 1>(L, 0, r, lane, fl);
    const bool ok = valid && !fl;
    if (MODE == 0) {
      if (ok) {
        if (biased) {
          if constexpr (X2) accum_vector_biased<K>(A, w, r0, fscale, 0, DIM, true);
          else accum_vector_biased<K>(A, w, r0, fscale, 4 * h, 4 * h + 4, h == 0);
        } else {
          if constexpr (X2) accum_vector<K>(A, w, r0, F, 0, DIM, true);
          else accum_vector<K>(A, w, r0, F, 4 * h, 4 * h + 4, h == 0);
        }
      }
    } else {
      if (ok) {
        float4* dst = reinterpret_cast<float4*>(R_next + j * DIM);
        if (X2 || h == 0) dst[0] = make_float4(r[0], r[1], r[2], r[3]);
        if (X2 || h == 1) dst[1] = make_float4(r[4], r[5], r[6], r[7]);
#pragma unroll
        for (int k = 0; k < 8; ++k) mx = max(mx, __float_as_uint(__builtin_fabsf(r[k])));
      }
    }
    flag_stage(fs, fl && valid && writer, (uint32_t)j, &hdr->n_flag[parity], list, cap, lane);
  }
  // The wave's flagged vectors still in its LDS stage (those that overflowed
  // it went to the global list for k_assign_exact) are resolved here by the
  // exact search, four lanes per vector, each over a quarter of the codewords
  // in increasing order; combining them keeps the lowest index among equal
  // distances. They are then counted or written like the certified ones.
  {
    constexpr int PARTS = 4, PER = K / PARTS;
    const int part = lane & (PARTS - 1);
    // (rolled loops: the tail is rare work and must not raise the register count)
#pragma unroll 1
    for (int q0 = 0; q0 < fs.cnt; q0 += WAVE / PARTS) {  // fs.cnt is wave-uniform
      const int q = q0 + lane / PARTS;
      const bool act = q < fs.cnt;
      const int64_t vid = fs.buf[act ? q : q0];
      const float4* p = reinterpret_cast<const float4*>(R_cur + vid * DIM);
      const float4 ra = p[0], rb = p[1];
      float r[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
      int best = part * PER;
      float bd = dist8(r, L.row(0, best));
#pragma unroll 1
      for (int c = best + 1; c < (part + 1) * PER; ++c) {
        const float d = dist8(r, L.row(0, c));
        if (d < bd) {
          bd = d;
          best = c;
        }
      }
#pragma unroll
      for (int o = 1; o < PARTS; o <<= 1) {
        const float od = __shfl_xor(bd, o);
        const int oi = __shfl_xor(best, o);
        if (od < bd || (od == bd && oi < best)) {
          bd = od;
          best = oi;
        }
      }
      if (act && part == 0) {
        if (MODE == 0) {
          if (biased) accum_vector_biased<K>(A, best, r, fscale, 0, DIM, true);
          else accum_vector<K>(A, best, r, F, 0, DIM, true);
        } else {
          const float* cw = L.row(0, best);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            r[k] = r[k] - cw[k];
            mx = max(mx, __float_as_uint(__builtin_fabsf(r[k])));
          }
          float4* dst = reinterpret_cast<float4*>(R_next + vid * DIM);
          dst[0] = make_float4(r[0], r[1], r[2], r[3]);
          dst[1] = make_float4(r[4], r[5], r[6], r[7]);
        }
      }
    }
  }
  if (MODE == 0) {
    flush_accum<K>(A, partials, blockIdx.x, biased);
  } else {
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    if (lane == 0 && mx) atomicMax(&hdr->maxabs_bits[nxt], mx);
  }
}

// Exact assignment of the queued vectors (or of all vectors when the queue
// overflowed), one vector per thread. MODE 0 accumulates into this block's own
// partial slot (slot_base + block); MODE 1 writes residuals.
template <int FMT, int MODE>
__global__ __launch_bounds__(256) void k_assign_exact(const float* R_cur, float* R_next, int64_t n, const float* C,
                                                      WsHeader* hdr, const uint32_t* list, uint32_t cap,
                                                      long long* partials, int slot_base, int parity, int nxt) {
  constexpr int K = Fmt<FMT>::K;
  __shared__ float cb[K][DIM];
  __shared__ FitAccum<K> A;
  const uint32_t nf = hdr->n_flag[parity];
  const bool full = nf > cap;
  const uint64_t total = full ? (uint64_t)n : nf;
  // blocks past the queue have no vector to take: they exit without writing
  // their partial slot, which k_update then does not read (same count there)
  if (!full && (uint64_t)blockIdx.x * blockDim.x >= total) return;
  if (MODE == 0)
    for (int q = threadIdx.x; q < K * (DIM + 1); q += blockDim.x) (&A.sum[0][0])[q] = 0ull;
  for (int q = threadIdx.x; q < K * DIM; q += blockDim.x) (&cb[0][0])[q] = C[q];
  if (full && blockIdx.x == 0 && threadIdx.x == 0) flag_status(hdr, ST_LIST_OVERFLOW);
  __syncthreads();
  const int F = hdr->fbits;
  uint32_t mx = 0;
  for (uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t j = full ? q : list[q];
    float r[8];
    const float4* p = reinterpret_cast<const float4*>(R_cur + j * DIM);
    float4 a = p[0], b = p[1];
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w; r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    const int w = exact_argmin<K>(r, &cb[0][0]);
    if (MODE == 0) {
      accum_vector<K>(A, w, r, F, 0, DIM, true);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        r[k] = r[k] - cb[w][k];
        mx = max(mx, __float_as_uint(__builtin_fabsf(r[k])));
      }
      float4* dst = reinterpret_cast<float4*>(R_next + j * DIM);
      dst[0] = make_float4(r[0], r[1], r[2], r[3]);
      dst[1] = make_float4(r[4], r[5], r[6], r[7]);
    }
  }
  if (MODE == 0) {
    flush_accum<K>(A, partials, slot_base + blockIdx.x, false);
  } else {
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    if ((threadIdx.x & 63) == 0 && mx) atomicMax(&hdr->maxabs_bits[nxt], mx);
  }
}

// Centroid update, one block per cluster: exact int64 sums over all partial
// slots (the first n_assign slots are skipped when the exact pass covered
// every vector), then c = (float)(((double)S * 2^-F) / n); empty clusters keep
// their centroid. Block 0 also clears the other parity's queue counter.
constexpr int UPD_THREADS = 256;  // partial slots summed in parallel per cluster

template <int FMT>
__global__ __launch_bounds__(UPD_THREADS) void k_update(float* C, const long long* partials, int n_assign,
                                                        int n_slots, WsHeader* hdr, int parity, uint32_t cap) {
  constexpr int K = Fmt<FMT>::K;
  __shared__ long long red[UPD_THREADS][DIM + 1];
  const int j = blockIdx.x;
  const uint32_t nf = hdr->n_flag[parity];
  const bool full = nf > cap;
  const int s0 = full ? n_assign : 0;
  // exact-pass slots that were written: all when the pass covered every vector,
  // else one per 256 queued vectors (k_assign_exact's blocks past the queue exit)
  if (!full) {
    const int64_t used = ((int64_t)nf + 255) / 256;
    if ((int64_t)n_assign + used < n_slots) n_slots = (int)(n_assign + used);
  }
  long long acc[DIM + 1];
#pragma unroll
  for (int k = 0; k <= DIM; ++k) acc[k] = 0;
  for (int s = s0 + threadIdx.x; s < n_slots; s += UPD_THREADS) {
    const long long* p = partials + ((size_t)s * K + j) * (DIM + 1);
#pragma unroll
    for (int k = 0; k <= DIM; ++k) acc[k] += p[k];
  }
#pragma unroll
  for (int k = 0; k <= DIM; ++k) red[threadIdx.x][k] = acc[k];
  __syncthreads();
  // integer sums: exact in any order
  for (int o = UPD_THREADS / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o)
#pragma unroll
      for (int k = 0; k <= DIM; ++k) red[threadIdx.x][k] += red[threadIdx.x + o][k];
    __syncthreads();
  }
  if (threadIdx.x < DIM) {
    const long long S = red[0][threadIdx.x], cnt = red[0][DIM];
    if (cnt > 0) {
      const double m = __ddiv_rn(ldexp(__ll2double_rn(S), -hdr->fbits), __ll2double_rn(cnt));
      C[j * DIM + threadIdx.x] = __double2float_rn(m);
    }
  }
  if (j == 0 && threadIdx.x == 0) hdr->n_flag[parity ^ 1] = 0;
}

// ------------------------------------------------------------------ launchers
static int grid_rows(int64_t rows, int ncu, int per_cu, int waves = 4) {
  int64_t g = (rows + waves - 1) / waves;
  int64_t m = (int64_t)ncu * per_cu;
  return (int)(g < m ? (g < 1 ? 1 : g) : m);
}

template <int FMT, int ENG, int DT>
static hipError_t launch_encode_t(const EncodeArgs& a) {
  const int g = grid_rows(a.rows, a.ncu, 2, enc_waves(ENG));
  k_encode<FMT, ENG, DT><<<g, 64 * enc_waves(ENG), 0, a.stream>>>(a.W, a.rows, a.cols, a.codebooks, a.idx, a.scales, a.hdr,
                                                  a.list, a.cap);
  return hipGetLastError();
}

template <int FMT, int DT>
static hipError_t launch_encode_dt(const EncodeArgs& a) {
  hipError_t e = hipSuccess;
  k_reset_header<<<1, 64, 0, a.stream>>>(a.hdr, 0);
  const uint64_t nvec = (uint64_t)a.rows * (a.cols / DIM);
  if (a.engine == ENGINE_EXACT) {
    k_row_scales<DT><<<grid_rows(a.rows, a.ncu, 4), 256, 0, a.stream>>>(a.W, a.rows, a.cols, a.scales, a.hdr);
  } else if (a.engine == ENG_F32) {
    e = launch_encode_t<FMT, ENG_F32, DT>(a);
  } else if (a.engine == ENG_VALU) {
    e = launch_encode_t<FMT, ENG_VALU, DT>(a);
  } else {
    e = launch_encode_t<FMT, ENG_F16X, DT>(a);
  }
  if (e != hipSuccess) return e;
  uint64_t gx = (nvec + 256 * 8 - 1) / (256 * 8);
  const uint64_t gmax = (uint64_t)a.ncu * 4;
  if (a.engine == ENGINE_EXACT) {
    gx = (nvec + 255) / 256;
    if (gx > (uint64_t)a.ncu * 16) gx = (uint64_t)a.ncu * 16;
  } else if (gx > gmax) {
    gx = gmax;
  }
  if (gx < 1) gx = 1;
  k_encode_exact<FMT, DT><<<(unsigned)gx, 256, 0, a.stream>>>(a.W, a.rows, a.cols, a.codebooks, a.idx, a.scales,
                                                              a.hdr, a.list, a.cap, a.engine == ENGINE_EXACT);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs& a) {
  if (a.format == 0) {
    if (a.dtype == DT_F32) return launch_encode_dt<0, DT_F32>(a);
    if (a.dtype == DT_BF16) return launch_encode_dt<0, DT_BF16>(a);
    return launch_encode_dt<0, DT_F16>(a);
  }
  if (a.dtype == DT_F32) return launch_encode_dt<1, DT_F32>(a);
  if (a.dtype == DT_BF16) return launch_encode_dt<1, DT_BF16>(a);
  return launch_encode_dt<1, DT_F16>(a);
}

// Assign workgroups launched: at most the workspace's partial slots, and no
// more than the device holds at once. Each workgroup adds a partial-sum slot
// that k_update reads; workgroups past the resident count only add slots (the
// VQ3R assign, 3 workgroups per CU, took the same time with 1024 as with 768,
// and k_update 11.7 instead of 9.6 us).
template <int FMT, int ENG, int MODE>
static int assign_blocks(const FitArgs& a) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_assign<FMT, ENG, MODE>, 256, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int64_t g = (int64_t)per_cu * a.ncu;
  return (int)(g < a.n_assign_blocks ? g : a.n_assign_blocks);
}

template <int FMT, int ENG>
static hipError_t fit_stage_iters(const FitArgs& a, int t, const float* Rc, float* Rn, float* C, int cur) {
  constexpr int K = Fmt<FMT>::K;
  // the iterations' partial slots: [0, ga0) for the assign blocks, then the exact pass's
  const int ga0 = assign_blocks<FMT, ENG, 0>(a), ga1 = assign_blocks<FMT, ENG, 1>(a), gf = a.n_exact_blocks;
  for (int it = 0; it <= a.iters; ++it) {
    const int parity = it & 1;
    if (it < a.iters) {
      k_assign<FMT, ENG, 0><<<ga0, 256, 0, a.stream>>>(Rc, Rn, a.n, C, a.hdr, a.list, a.cap, a.partials, parity,
                                                       cur ^ 1);
      k_assign_exact<FMT, 0><<<gf, 256, 0, a.stream>>>(Rc, Rn, a.n, C, a.hdr, a.list, a.cap, a.partials, ga0,
                                                       parity, cur ^ 1);
      k_update<FMT><<<K, UPD_THREADS, 0, a.stream>>>(C, a.partials, ga0, ga0 + gf, a.hdr, parity, a.cap);
    } else {
      k_assign<FMT, ENG, 1><<<ga1, 256, 0, a.stream>>>(Rc, Rn, a.n, C, a.hdr, a.list, a.cap, a.partials, parity,
                                                       cur ^ 1);
      k_assign_exact<FMT, 1><<<gf, 256, 0, a.stream>>>(Rc, Rn, a.n, C, a.hdr, a.list, a.cap, a.partials, ga1,
                                                       parity, cur ^ 1);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  (void)t;
  return hipSuccess;
}

template <int FMT, int DT>
static hipError_t launch_fit_t(const FitArgs& a) {
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K;
  k_reset_header<<<1, 64, 0, a.stream>>>(a.hdr, 0);
  const int64_t per = a.rows * (a.cols / DIM);
  for (int64_t m = 0; m < a.n_mats; ++m) {
    k_fit_prepare<DT><<<grid_rows(a.rows, a.ncu, 4), 256, 0, a.stream>>>(a.mats[m], a.rows, a.cols,
                                                                         a.R[0] + m * per * DIM, a.hdr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int t = 0; t < S; ++t) {
    const int cur = t & 1;
    float* C = a.codebooks + (size_t)t * K * DIM;
    k_stage_begin<FMT><<<1, 256, 0, a.stream>>>(a.R[cur], a.init + (size_t)t * K, C, a.hdr, cur, a.clog2n);
    if (a.engine == ENG_F32) e = fit_stage_iters<FMT, ENG_F32>(a, t, a.R[cur], a.R[cur ^ 1], C, cur);
    else if (a.engine == ENG_VALU) e = fit_stage_iters<FMT, ENG_VALU>(a, t, a.R[cur], a.R[cur ^ 1], C, cur);
    else e = fit_stage_iters<FMT, ENG_F16X>(a, t, a.R[cur], a.R[cur ^ 1], C, cur);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_fit(const FitArgs& a) {
  if (a.format == 0) {
    if (a.dtype == DT_F32) return launch_fit_t<0, DT_F32>(a);
    if (a.dtype == DT_BF16) return launch_fit_t<0, DT_BF16>(a);
    return launch_fit_t<0, DT_F16>(a);
  }
  if (a.dtype == DT_F32) return launch_fit_t<1, DT_F32>(a);
  if (a.dtype == DT_BF16) return launch_fit_t<1, DT_BF16>(a);
  return launch_fit_t<1, DT_F16>(a);
}

hipError_t launch_reset(WsHeader* hdr, hipStream_t s) {
  k_reset_header<<<1, 64, 0, s>>>(hdr, 0);
  return hipGetLastError();
}

}  // namespace vqk
