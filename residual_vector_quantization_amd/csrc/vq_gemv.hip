// Fused dequantize-GEMV for decode-time expert mat-vecs ([VQ3R page] §1: per
// token only the routed experts' records are read and decoded).
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
//
// y[p][r] = s_r * sum_j sum_t T_t[j][i_t(r, j)],   T_t[j][e] = <C_t[e], x_j>
// where x_j is the j-th 8-element slice of the token's activation: the inner
// products of every codeword with the activation slice are tabulated once per
// block (a lookup table in LDS), after which each stored index costs one table
// read and one add. This equals sum_c W_hat[r][c] x[c] up to fp32 rounding.
#include "vq_launch.hpp"

namespace vqk {

// grid: x = column block (GEMV_SLICES slices), y = (token, slot) pair, z = row chunk of 256
template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_lut(const uint8_t* idx, int64_t expert_stride, const float* cb_g,
                                                  int64_t rows, int64_t cols, int n_experts, const uint16_t* x,
                                                  int topk, const int32_t* route, float* partials, WsHeader* hdr) {
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K, J = GEMV_SLICES;
  __shared__ float lut[S][J][K];
  __shared__ float cb[S][K][DIM];
  __shared__ float xs[J * DIM];
  const int b = blockIdx.x, p = blockIdx.y;
  const int64_t nblk = gridDim.x;
  const int tok = p / topk;
  const int e = route[p];
  const int64_t r = (int64_t)blockIdx.z * 256 + threadIdx.x;
  if (e < 0 || e >= n_experts) {
    if (threadIdx.x == 0 && b == 0 && blockIdx.z == 0) flag_status(hdr, ST_ROUTE);
    if (r < rows) partials[((int64_t)p * nblk + b) * rows + r] = 0.0f;
    return;
  }
  const int64_t V = cols / DIM;
  const int64_t j0 = (int64_t)b * J;
  const int nsl = (int)((V - j0) < J ? (V - j0) : J);
  for (int q = threadIdx.x; q < S * K * DIM; q += blockDim.x) (&cb[0][0][0])[q] = cb_g[q];
  for (int q = threadIdx.x; q < J * DIM; q += blockDim.x)
    xs[q] = (q < nsl * DIM) ? f16_bits_to_f32(x[(int64_t)tok * cols + j0 * DIM + q]) : 0.0f;
  __syncthreads();
  for (int q = threadIdx.x; q < S * J * K; q += blockDim.x) {
    const int t = q / (J * K), sl = (q / K) % J, ee = q % K;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < DIM; ++k) acc = __builtin_fmaf(cb[t][ee][k], xs[sl * DIM + k], acc);
    lut[t][sl][ee] = acc;
  }
  __syncthreads();
  if (r >= rows) return;
  const uint8_t* rec = idx + (int64_t)e * expert_stride + (r * V + j0) * 3;
  float acc = 0.0f;
  for (int sl = 0; sl < nsl; ++sl) {
    const uint32_t word = load_record(rec + sl * 3);
#pragma unroll
    for (int t = 0; t < S; ++t) acc += lut[t][sl][record_index<FMT>(word, t)];
  }
  partials[((int64_t)p * nblk + b) * rows + r] = acc;
}

// y[p][r] = s_r * sum over column blocks (fixed order)
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* partials, const uint16_t* scales,
                                                     int64_t scale_stride, const int32_t* route, int n_experts,
                                                     int64_t rows, int nblk, int64_t npairs, float* y) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= npairs * rows) return;
  const int64_t p = q / rows, r = q % rows;
  const int e = route[p];
  if (e < 0 || e >= n_experts) {
    y[q] = 0.0f;
    return;
  }
  float acc = 0.0f;
  for (int b = 0; b < nblk; ++b) acc += partials[((int64_t)p * nblk + b) * rows + r];
  y[q] = f16_bits_to_f32(scales[(int64_t)e * scale_stride + r]) * acc;
}

hipError_t launch_gemv(const GemvArgs& a) {
  hipError_t e0 = launch_reset(a.hdr, a.stream);
  if (e0 != hipSuccess) return e0;
  const int64_t npairs = (int64_t)a.ntok * a.topk;
  const int nblk = (int)gemv_nblk(a.cols);
  if (npairs == 0 || a.rows == 0) return hipSuccess;
  dim3 grid((unsigned)nblk, (unsigned)npairs, (unsigned)((a.rows + 255) / 256));
  if (a.format == 0)
    k_gemv_lut<0><<<grid, 256, 0, a.stream>>>(a.idx, a.expert_stride, a.codebooks, a.rows, a.cols, a.n_experts, a.x,
                                              a.topk, a.route, a.partials, a.hdr);
  else
    k_gemv_lut<1><<<grid, 256, 0, a.stream>>>(a.idx, a.expert_stride, a.codebooks, a.rows, a.cols, a.n_experts, a.x,
                                              a.topk, a.route, a.partials, a.hdr);
  const int64_t nq = npairs * a.rows;
  k_gemv_reduce<<<(unsigned)((nq + 255) / 256), 256, 0, a.stream>>>(a.partials, a.scales, a.scale_stride, a.route,
                                                                     a.n_experts, a.rows, nblk, npairs, a.y);
  return hipGetLastError();
}

}  // namespace vqk
