// Fused dequantize-GEMV for decode-time expert mat-vecs ([VQ3R page] §1: per
// token only the routed experts' records are read and decoded).
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
//
// y[p][r] = s_r * sum_j sum_t T_t[j][i_t(r, j)],   T_t[j][e] = <C_t[e], x_j>
// where x_j is the j-th 8-element slice of the token's activation. A work tile
// is (token-slot pair p, block of J = 16 slices, chunk of at most 2048 rows):
// its workgroup tabulates T for
// the block's slices in LDS with fp32 matrix-core products (codewords x
// slices), then streams the tile's records, one row per lane: each index
// costs one table read and one add. Tile partial sums go to the workspace and
// a second kernel adds the blocks in a fixed order and applies the row
// scales, so the result is deterministic. It equals sum_c W_hat[r][c] x[c] up
// to fp32 rounding.
//
// Blocks of 16 slices keep a workgroup's tables at 48 KB (VQ3R) / 32 KB
// (VQ4P), so that several 8-wave workgroups share a CU and one's table build
// and start-up latency overlap the others' record streams.
//
// Runtime layout ("packed"): the GEMV reads indices repacked once by
// vq_gemv_pack into blocks of J = 16 slices x 64-row groups. Within a group
// the records are interleaved in 12-byte chunks (4 records of one row), and
// each row's slices are rotated by its lane:
//   packed[b][g][c][lane][12 bytes] = records of row 64g+lane for the slices
//   16b + ((4c + q + lane) mod 16), q = 0..3
// so every wave load is one contiguous 768-byte piece of the stream, a tile's
// data is contiguous, and at step m lane l works on slice (m + l) mod 16 (the
// row-interleave idea of the IQ1_S_R4 format on the ik_llama.cpp page, applied
// to whole waves). The tables are stored slice-minor,
//   T[(e * S + t) * R + replica][slice],
// so the 16 lanes of a quarter-wave read 16 distinct slices (distinct LDS
// banks); VQ4P keeps R = 2 replicas, lanes 16-31 (mod 32) reading the second,
// which makes a half-wave's reads conflict-free; VQ3R keeps one copy.
#include "vq_launch.hpp"

namespace vqk {

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int GJ = 16;     // slices per block
constexpr int GROUP = 64;  // rows per interleaved group (one wave)
constexpr int GEMV_WAVES = 8;
constexpr int GEMV_THREADS = 64 * GEMV_WAVES;

template <int FMT> struct GemvCfg;
template <> struct GemvCfg<0> { static constexpr int R = 1; };  // 256 x 3 x 16 x 4 B = 48 KB
template <> struct GemvCfg<1> { static constexpr int R = 2; };  // 64 x 4 x 2 x 16 x 4 B = 32 KB

int64_t gemv_packed_bytes(int format, int64_t rows, int64_t cols) {
  (void)format;
  const int64_t nblk = (cols / DIM + GJ - 1) / GJ;
  const int64_t ng = (rows + GROUP - 1) / GROUP;
  return nblk * ng * GROUP * GJ * 3;
}

// ------------------------------------------------------------------ repack
// One workgroup (256 threads) per tile (expert, block of 16 slices, group of
// 64 rows): the tile's 64 x 48 record bytes are read row by row (4 threads per
// row, 12 bytes each: three dword loads when the row segment is 4-byte aligned)
// into LDS, then written as the 4 x 64 rotated 12-byte chunks of the packed
// layout, one chunk per thread (contiguous across a wave). Pad rows and slices
// are 0.
__global__ __launch_bounds__(256) void k_gemv_pack(const uint8_t* idx, int64_t rows, int64_t V, int64_t n_experts,
                                                   uint8_t* out, int64_t packed_stride) {
  constexpr int NC = GJ / 4, RB = GJ * 3;  // 4 chunks per row, 48 record bytes per row
  __shared__ uint32_t tile[GROUP][RB / 4 + 1];
  const int64_t ng = (rows + GROUP - 1) / GROUP, nblk = (V + GJ - 1) / GJ;
  const int64_t ntiles = n_experts * nblk * ng;
  const int tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;     // load: row of the group, 12-byte part of its 48 bytes
  const int c = tid >> 6, lane = tid & 63;    // store: chunk c of row `lane`
  const bool dword_ok = ((V * 3) & 3) == 0 && ((uintptr_t)idx & 3) == 0;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t e = t / (nblk * ng), rem = t % (nblk * ng);
    const int64_t b = rem / ng, g = rem % ng;
    const int64_t row = g * GROUP + r;
    const int64_t j0 = b * GJ;
    uint32_t w[3] = {0u, 0u, 0u};
    if (row < rows) {
      const uint8_t* src = idx + ((e * rows + row) * V + j0) * 3 + part * 12;
      const int64_t nbytes = ((V - j0) < GJ ? (V - j0) : GJ) * 3 - part * 12;  // valid bytes of this part
      if (dword_ok && nbytes >= 12) {
        const uint32_t* s4 = reinterpret_cast<const uint32_t*>(src);
        w[0] = s4[0];
        w[1] = s4[1];
        w[2] = s4[2];
      } else {
#pragma unroll
        for (int k = 0; k < 12; ++k)
          if (k < nbytes) w[k >> 2] |= (uint32_t)src[k] << (8 * (k & 3));
      }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) tile[r][part * 3 + k] = w[k];
    __syncthreads();
    const uint8_t* tb = reinterpret_cast<const uint8_t*>(&tile[lane][0]);
    uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sl = (4 * c + q + lane) & (GJ - 1);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int ob = 3 * q + k;
        o[ob >> 2] |= (uint32_t)tb[3 * sl + k] << (8 * (ob & 3));
      }
    }
    uint32_t* dst =
        reinterpret_cast<uint32_t*>(out + e * packed_stride + ((b * ng + g) * NC + c) * (GROUP * 12) + lane * 12);
#pragma unroll
    for (int k = 0; k < 3; ++k) dst[k] = o[k];
    __syncthreads();  // the tile buffer is refilled next
  }
}

// ------------------------------------------------------------------ tables
// T[(e*S + t)*R + rep][m] = sum_k C_t[e][k] * x[(j0 + m)*8 + k] with fp32
// matrix cores (32x32x2): codewords on M, slices on N (lanes 16-31 of each
// half-wave carry zero slices). The operands of a wave's tasks are loaded
// first (lut_load), the MFMAs run later (lut_compute): the first index loads
// are issued in between, so waiting for the table operands never waits for
// the (later) index loads.
template <int FMT>
struct LutOps {
  static constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K, NT = K / 32, TASKS = S * NT;
  static constexpr int PER_WAVE = (TASKS + GEMV_WAVES - 1) / GEMV_WAVES;
  float a[PER_WAVE][4];
  uint32_t xb[4];  // the activation operand (fp16 bits), the same for every task of the wave
};

template <int FMT>
__device__ inline void lut_load(LutOps<FMT>& op, const float* cb_g, const uint16_t* xrow, int64_t j0, int nsl) {
  using O = LutOps<FMT>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, i = lane & 31;
  const int ic = i < nsl ? i : 0;  // clamped slice: loaded but zeroed
#pragma unroll
  for (int u = 0; u < O::PER_WAVE; ++u) {
    const int task = wave + GEMV_WAVES * u;
    const int tk = task < O::TASKS ? task : 0;
    const int t = tk / O::NT, ct = tk % O::NT;
#pragma unroll
    for (int s = 0; s < 4; ++s) op.a[u][s] = cb_g[((size_t)t * O::K + ct * 32 + i) * DIM + 2 * s + h];
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) op.xb[s] = xrow[(j0 + ic) * DIM + 2 * s + h];
}

template <int FMT>
__device__ inline void lut_compute(const LutOps<FMT>& op, float* lut, int nsl) {
  using O = LutOps<FMT>;
  constexpr int R = GemvCfg<FMT>::R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, i = lane & 31;
  const bool sv = i < nsl;  // nsl <= 16: lanes 16-31 of a half-wave compute nothing useful
  float b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) b[s] = sv ? f16_bits_to_f32((uint16_t)op.xb[s]) : 0.0f;
#pragma unroll
  for (int u = 0; u < O::PER_WAVE; ++u) {
    const int task = wave + GEMV_WAVES * u;
    if (task >= O::TASKS) break;  // wave-uniform
    const int t = task / O::NT, ct = task % O::NT;
    f16v acc = {};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(op.a[u][s], b[s], acc, 0, 0, 0);
    // lane (n = slice i, h) holds codewords e = 32ct + 8*(v/4) + 4h + v%4
    if (i < GJ) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int e = ct * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
#pragma unroll
        for (int rep = 0; rep < R; ++rep) lut[((e * O::S + t) * R + rep) * GJ + i] = acc[v];
      }
    }
  }
}

// Tile order: the tiles of each XCD share are contiguous (pair-major, block-minor):
// workgroups are dealt to the 8 XCDs in turn.
__device__ inline int64_t tile_of_block(int64_t bid, int64_t ntiles_pad) {
  const int64_t per_xcd = ntiles_pad / 8;
  return (bid % 8) * per_xcd + bid / 8;
}

// A tile is (slot pair, block of 16 slices, row chunk). Matrices of more than
// 2048 rows are cut into nsplit chunks of near-equal group counts (at most 32
// groups each), so that a tile never streams more than 2048 rows and tall
// matrices still give many tiles. GPW = row groups per wave in a chunk (groups
// g = g0 + wave + 8k, k < GPW), 1..4, fully unrolled.
template <int FMT, int GPW>
__global__ __launch_bounds__(GEMV_THREADS) void k_gemv(const uint8_t* pk, int64_t expert_stride, const float* cb_g,
                                                       int64_t rows, int64_t cols, int n_experts, const uint16_t* x,
                                                       int topk, const int32_t* route, float* partials, int nblk,
                                                       int nsplit, int64_t ntiles, int64_t ntiles_pad) {
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K, R = GemvCfg<FMT>::R, NC = GJ / 4;
  constexpr int NW = GEMV_WAVES;
  __shared__ float lut[K * S * R * GJ];
  const int64_t tile = tile_of_block(blockIdx.x, ntiles_pad);
  if (tile >= ntiles) return;
  const int64_t pb = tile / nsplit, chunk = tile % nsplit;
  const int p = (int)(pb / nblk), b = (int)(pb % nblk);
  const int tok = p / topk;
  const int e = route[p];
  if (e < 0 || e >= n_experts) return;  // flagged and zeroed by k_gemv_reduce
  const int64_t V = cols / DIM;
  const int64_t j0 = (int64_t)b * GJ;
  const int nsl = (int)((V - j0) < GJ ? (V - j0) : GJ);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ng = (rows + GROUP - 1) / GROUP;
  const int64_t g0 = chunk * ng / nsplit, g1 = (chunk + 1) * ng / nsplit;  // this tile's groups [g0, g1)
  const uint8_t* tb = pk + (int64_t)e * expert_stride + (int64_t)b * ng * NC * (GROUP * 12);
  float* part = partials + ((int64_t)p * nblk + b) * rows;
  // unconditional loads with a clamped group index keep the wait counts exact
  uint32_t d[2][NC][3];
  auto load_group = [&](uint32_t (&dg)[NC][3], int64_t g) {
    const int64_t gc = g < g1 ? g : g1 - 1;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tb + gc * NC * (GROUP * 12)) + lane * 3;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int k = 0; k < 3; ++k) dg[c][k] = src[c * (GROUP * 3) + k];
    }
  };
  // byte offset of (slice (m + lane) mod 16, replica) inside one (e, t) row of the table
  const uint32_t rep_off = (R == 2) ? (uint32_t)((lane >> 4) & 1) * (GJ * 4) : 0u;
  constexpr uint32_t E_STRIDE = S * R * GJ * 4, T_STRIDE = R * GJ * 4;
  const char* lbase = reinterpret_cast<const char*>(lut);
  auto consume = [&](const uint32_t (&dg)[NC][3], int64_t g) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // record q of the chunk = bytes 3q .. 3q+2 of the 12 bytes
        const int byte0 = 3 * q, k0 = byte0 >> 2, o = byte0 & 3;
        const uint32_t w =
            (o <= 1) ? (dg[c][k0] >> (8 * o)) : ((dg[c][k0] >> (8 * o)) | (dg[c][k0 + 1] << (32 - 8 * o)));
        const int m = 4 * c + q;
        const uint32_t soff = (((uint32_t)(m + lane) & (GJ - 1)) << 2) + rep_off;
        float tsum = 0.0f;
#pragma unroll
        for (int t = 0; t < S; ++t) {
          const uint32_t ei = (uint32_t)record_index<FMT>(w, t);
          tsum += *reinterpret_cast<const float*>(lbase + (ei * E_STRIDE + soff) + t * T_STRIDE);
        }
        acc += tsum;
      }
    }
    const int64_t row = g * GROUP + lane;
    if (row < rows) part[row] = acc;
  };
  LutOps<FMT> ops;
  lut_load<FMT>(ops, cb_g, x + (int64_t)tok * cols, j0, nsl);
  __builtin_amdgcn_sched_barrier(0);  // keep the table operand loads ahead of the index stream
  load_group(d[0], g0 + wave);
  if (GPW != 1) load_group(d[1], g0 + wave + NW);
  __builtin_amdgcn_sched_barrier(0);
  lut_compute<FMT>(ops, lut, nsl);
  __syncthreads();
  // two groups in flight: the load of group k + 2 follows the consume of group k
#pragma unroll
  for (int k = 0; k < GPW; ++k) {
    const int64_t g = g0 + wave + (int64_t)k * NW;
    if (g < g1) consume(d[k & 1], g);  // wave-uniform
    if (k + 2 < GPW) load_group(d[k & 1], g0 + wave + (int64_t)(k + 2) * NW);
  }
}

// y[p][r] = s_r * sum over blocks in a fixed order. Also writes the status
// flags of the call (route ids outside [0, n_experts)), so no reset is needed.
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* partials, const uint16_t* scales,
                                                     int64_t scale_stride, const int32_t* route, int n_experts,
                                                     int64_t rows, int nblk, int npairs, float* y, WsHeader* hdr) {
  const int p = blockIdx.y;
  const int e = route[p];
  const bool bad = e < 0 || e >= n_experts;
  if (blockIdx.x == 0 && p == 0 && threadIdx.x < 64) {
    bool any = false;
    for (int q = threadIdx.x; q < npairs; q += 64) any |= (route[q] < 0 || route[q] >= n_experts);
    any = __any(any);
    if (threadIdx.x == 0) hdr->flags = any ? ST_ROUTE : 0u;
  }
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.0f;
  if (!bad) {
    const float* pp = partials + (int64_t)p * nblk * rows + r;
    // eight independent loads in flight, added in block order
    int q = 0;
    for (; q + 8 <= nblk; q += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pp[(int64_t)(q + u) * rows];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; q < nblk; ++q) acc += pp[(int64_t)q * rows];
    acc *= f16_bits_to_f32(scales[(int64_t)e * scale_stride + r]);
  }
  y[(int64_t)p * rows + r] = acc;
}

__global__ void k_gemv_clear(WsHeader* hdr) {
  if (threadIdx.x == 0) hdr->flags = 0;
}

template <int FMT>
static hipError_t launch_gemv_t(const GemvArgs& a) {
  const int64_t npairs = (int64_t)a.ntok * a.topk;
  const int64_t V = a.cols / DIM;
  const int nblk = (int)((V + GJ - 1) / GJ);
  const int64_t ng = (a.rows + GROUP - 1) / GROUP;
  const int nsplit = gemv_row_chunks(a.rows);
  const int64_t ntiles = npairs * nblk * nsplit;
  const int64_t ntiles_pad = (ntiles + 7) / 8 * 8;
  const int64_t gpw = (ng / nsplit + (ng % nsplit != 0) + GEMV_WAVES - 1) / GEMV_WAVES;  // largest chunk
  auto go = [&](auto kern) {
    kern<<<(unsigned)ntiles_pad, GEMV_THREADS, 0, a.stream>>>(a.idx, a.expert_stride, a.codebooks, a.rows, a.cols,
                                                               a.n_experts, a.x, a.topk, a.route, a.partials, nblk,
                                                               nsplit, ntiles, ntiles_pad);
  };
  if (gpw == 1) go(k_gemv<FMT, 1>);
  else if (gpw == 2) go(k_gemv<FMT, 2>);
  else if (gpw == 3) go(k_gemv<FMT, 3>);
  else go(k_gemv<FMT, 4>);
  dim3 g2((unsigned)((a.rows + 255) / 256), (unsigned)npairs);
  k_gemv_reduce<<<g2, 256, 0, a.stream>>>(a.partials, a.scales, a.scale_stride, a.route, a.n_experts, a.rows, nblk,
                                          (int)npairs, a.y, a.hdr);
  return hipGetLastError();
}

int gemv_row_chunks(int64_t rows) {
  const int64_t ng = (rows + GROUP - 1) / GROUP;
  return (int)((ng + 4 * GEMV_WAVES - 1) / (4 * GEMV_WAVES));
}

int64_t gemv_tiles(int64_t rows, int64_t cols, int64_t npairs) {
  const int64_t nblk = (cols / DIM + GJ - 1) / GJ;
  return npairs * nblk * gemv_row_chunks(rows);
}

int64_t gemv_partials_floats(int format, int64_t rows, int64_t cols, int64_t npairs) {
  (void)format;
  const int64_t nblk = (cols / DIM + GJ - 1) / GJ;
  return npairs * nblk * rows;
}

hipError_t launch_gemv(const GemvArgs& a) {
  if ((int64_t)a.ntok * a.topk == 0 || a.rows == 0) {
    k_gemv_clear<<<1, 64, 0, a.stream>>>(a.hdr);
    return hipGetLastError();
  }
  return a.format == 0 ? launch_gemv_t<0>(a) : launch_gemv_t<1>(a);
}

hipError_t launch_gemv_pack(int format, const uint8_t* idx, int64_t rows, int64_t cols, int64_t n_experts,
                            uint8_t* out, int ncu, hipStream_t s) {
  const int64_t V = cols / DIM;
  const int64_t ntiles = ((V + GJ - 1) / GJ) * ((rows + GROUP - 1) / GROUP) * n_experts;
  if (ntiles == 0) return hipSuccess;
  int64_t g = ntiles;
  if (g > (int64_t)ncu * 32) g = (int64_t)ncu * 32;
  k_gemv_pack<<<(unsigned)g, 256, 0, s>>>(idx, rows, V, n_experts, out, gemv_packed_bytes(format, rows, cols));
  return hipGetLastError();
}

}  // namespace vqk
