// Fused dequantize-GEMV for decode-time expert mat-vecs ([VQ3R page] §1: per
// token only the routed experts' records are read and decoded).
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
//
// y[p][r] = s_r * sum_j sum_t T_t[j][i_t(r, j)],   T_t[j][e] = <C_t[e], x_j>
// where x_j is the j-th 8-element slice of the token's activation. A work tile
// is (token-slot pair p, block of J slices): its workgroup tabulates T for the
// block's slices in LDS with fp32 matrix-core products (codewords x slices),
// then streams the tile's stored records, one row per thread: each index costs
// one table read and one add. Tile partial sums go to the workspace; the last
// tile of a pair to finish adds the blocks in a fixed order and applies the
// row scales, so results are deterministic. This equals sum_c W_hat[r][c] x[c]
// up to fp32 rounding.
#include "vq_launch.hpp"

namespace vqk {

typedef float f16v __attribute__((ext_vector_type(16)));

template <int FMT> struct GemvCfg;
template <> struct GemvCfg<0> { static constexpr int J = 28; };  // 3 x 28 x 256 x 4 B = 84 KB of tables
template <> struct GemvCfg<1> { static constexpr int J = 56; };  // 4 x 56 x 64 x 4 B = 56 KB

constexpr int GEMV_THREADS = 1024;

template <int FMT>
__device__ inline void gemv_build_lut(float* lut, const float* cb_g, const uint16_t* xrow, int64_t j0, int nsl) {
  // LUT[t][m][e] = sum_k C_t[e][k] * x[(j0 + m)*8 + k]  (slices on M, codewords on N)
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K, J = GemvCfg<FMT>::J;
  constexpr int MT = (J + 31) / 32;        // slice tiles of 32
  constexpr int NT = K / 32;               // codeword tiles of 32
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int h = lane >> 5, i = lane & 31;
  for (int task = wave; task < S * MT * NT; task += nw) {
    const int t = task / (MT * NT), mt = (task / NT) % MT, nt = task % NT;
    const int m = mt * 32 + i;                    // slice row of the A operand
    const int e = nt * 32 + i;                    // codeword column of the B operand
    const bool mv = m < nsl;
    f16v acc = {};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = 2 * s + h;
      const float a = mv ? f16_bits_to_f32(xrow[(j0 + m) * DIM + k]) : 0.0f;
      const float b = cb_g[((size_t)t * K + e) * DIM + k];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    // lane (n = codeword, h) holds rows m = 8*(v/4) + 4h + v%4 of the tile
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int mm = mt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (mm < J) lut[((size_t)t * J + mm) * K + e] = acc[v];
    }
  }
}

// Tile order: the tiles of each XCD-sized share are contiguous (pair-major,
// block-minor) so neighbouring blocks of a row, which share cache lines of the
// index stream, run on the same XCD (workgroups are dealt to the 8 XCDs in turn).
__device__ inline int64_t tile_of_block(int64_t bid, int64_t ntiles_pad) {
  const int64_t per_xcd = ntiles_pad / 8;
  return (bid % 8) * per_xcd + bid / 8;
}

template <int FMT, bool FAST>
__global__ __launch_bounds__(GEMV_THREADS) void k_gemv(const uint8_t* idx, int64_t expert_stride,
                                                       const uint16_t* scales, int64_t scale_stride,
                                                       const float* cb_g, int64_t rows, int64_t cols, int n_experts,
                                                       const uint16_t* x, int topk, const int32_t* route, float* y,
                                                       float* partials, uint32_t* counters, int nblk,
                                                       int64_t ntiles, int64_t ntiles_pad, WsHeader* hdr) {
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K, J = GemvCfg<FMT>::J;
  static_assert((3 * J) % 4 == 0, "records of a block end on a dword boundary");
  __shared__ float lut[S * J * K];
  __shared__ int last_flag;
  const int64_t tile = tile_of_block(blockIdx.x, ntiles_pad);
  if (tile >= ntiles) return;
  const int p = (int)(tile / nblk), b = (int)(tile % nblk);
  const int tok = p / topk;
  const int e = route[p];
  const bool bad = e < 0 || e >= n_experts;
  const int64_t V = cols / DIM;
  const int64_t j0 = (int64_t)b * J;
  const int nsl = (int)((V - j0) < J ? (V - j0) : J);
  if (!bad) gemv_build_lut<FMT>(lut, cb_g, x + (int64_t)tok * cols, j0, nsl);
  __syncthreads();
  float* part = partials + ((int64_t)p * nblk + b) * rows;
  if (bad) {
    if (threadIdx.x == 0 && b == 0) flag_status(hdr, ST_ROUTE);
  } else {
    const uint8_t* base = idx + (int64_t)e * expert_stride + j0 * 3;
    for (int64_t r = threadIdx.x; r < rows; r += blockDim.x) {
      const uint8_t* rec = base + r * V * 3;
      float acc = 0.0f;
      if constexpr (FAST) {
        // J records = 3*J bytes, dword aligned: 3*J/4 dwords
        constexpr int ND = 3 * J / 4;
        uint32_t d[ND];
        const uint32_t* p32 = reinterpret_cast<const uint32_t*>(rec);
#pragma unroll
        for (int q = 0; q < ND; ++q) d[q] = __builtin_nontemporal_load(p32 + q);
#pragma unroll
        for (int m = 0; m < J; ++m) {
          // record m = bytes 3m, 3m+1, 3m+2 of the stream
          // (3*J is a multiple of 4, so the last record starts at byte offset 1
          // of the last dword and never needs the dword after it)
          uint32_t w;
          const int byte0 = 3 * m, q0 = byte0 >> 2, o = byte0 & 3;
          if (o <= 1) w = d[q0] >> (8 * o);
          else w = (d[q0] >> (8 * o)) | (d[q0 + 1] << (32 - 8 * o));
          float tsum = 0.0f;
#pragma unroll
          for (int t = 0; t < S; ++t) tsum += lut[(t * J + m) * K + record_index<FMT>(w, t)];
          acc += tsum;
        }
      } else {
        for (int m = 0; m < nsl; ++m) {
          const uint32_t w = load_record(rec + m * 3);
          float tsum = 0.0f;
#pragma unroll
          for (int t = 0; t < S; ++t) tsum += lut[(t * J + m) * K + record_index<FMT>(w, t)];
          acc += tsum;
        }
      }
      part[r] = acc;
    }
  }
  // the last tile of pair p to finish reduces its blocks in order
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last_flag = (atomicAdd(&counters[p], 1u) == (uint32_t)(nblk - 1));
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* pp = partials + (int64_t)p * nblk * rows;
  for (int64_t r = threadIdx.x; r < rows; r += blockDim.x) {
    float acc = 0.0f;
    if (!bad) {
      for (int q = 0; q < nblk; ++q) acc += pp[(int64_t)q * rows + r];
      acc *= f16_bits_to_f32(scales[(int64_t)e * scale_stride + r]);
    }
    y[(int64_t)p * rows + r] = acc;
  }
  if (threadIdx.x == 0) counters[p] = 0u;  // ready for the next call
}

__global__ void k_gemv_reset(WsHeader* hdr, uint32_t* counters, int npairs) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q == 0) hdr->flags = 0;
  if (q < npairs) counters[q] = 0u;
}

template <int FMT>
static hipError_t launch_gemv_t(const GemvArgs& a) {
  constexpr int J = GemvCfg<FMT>::J;
  const int64_t npairs = (int64_t)a.ntok * a.topk;
  const int64_t V = a.cols / DIM;
  const int nblk = (int)((V + J - 1) / J);
  const int64_t ntiles = npairs * nblk;
  const int64_t ntiles_pad = (ntiles + 7) / 8 * 8;
  k_gemv_reset<<<(unsigned)((npairs + 255) / 256), 256, 0, a.stream>>>(a.hdr, a.counters, (int)npairs);
  const bool fast = (V % 4 == 0) && (V % J == 0);
  if (fast)
    k_gemv<FMT, true><<<(unsigned)ntiles_pad, GEMV_THREADS, 0, a.stream>>>(
        a.idx, a.expert_stride, a.scales, a.scale_stride, a.codebooks, a.rows, a.cols, a.n_experts, a.x, a.topk,
        a.route, a.y, a.partials, a.counters, nblk, ntiles, ntiles_pad, a.hdr);
  else
    k_gemv<FMT, false><<<(unsigned)ntiles_pad, GEMV_THREADS, 0, a.stream>>>(
        a.idx, a.expert_stride, a.scales, a.scale_stride, a.codebooks, a.rows, a.cols, a.n_experts, a.x, a.topk,
        a.route, a.y, a.partials, a.counters, nblk, ntiles, ntiles_pad, a.hdr);
  return hipGetLastError();
}

int64_t gemv_partials_floats(int format, int64_t rows, int64_t cols, int64_t npairs) {
  const int J = format == 0 ? GemvCfg<0>::J : GemvCfg<1>::J;
  const int64_t nblk = (cols / DIM + J - 1) / J;
  return npairs * nblk * rows;
}

hipError_t launch_gemv(const GemvArgs& a) {
  if ((int64_t)a.ntok * a.topk == 0 || a.rows == 0) {
    k_gemv_reset<<<1, 64, 0, a.stream>>>(a.hdr, a.counters, 0);
    return hipGetLastError();
  }
  return a.format == 0 ? launch_gemv_t<0>(a) : launch_gemv_t<1>(a);
}

}  // namespace vqk
