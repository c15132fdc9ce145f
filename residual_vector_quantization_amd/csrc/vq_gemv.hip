// Fused dequantize-GEMV for decode-time expert mat-vecs ([VQ3R page] §1: per
// token only the routed experts' records are read and decoded).
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
//
// y[p][r] = s_r * sum_j sum_t T_t[j][i_t(r, j)],   T_t[j][e] = <C_t[e], x_j>
// where x_j is the j-th 8-element slice of the token's activation. A work tile
// is (token-slot pair p, row chunk of at most 4096 rows, range of NB blocks of
// 16 slices). For each block of its range the workgroup tabulates T for the
// block's slices in LDS with fp32 matrix-core products (codewords x slices),
// then streams the block's records, one row per lane: each index costs one
// table read and one add. Row sums stay in registers across the blocks of the
// range; one partial sum per (pair, range, row) goes to the workspace and a
// second kernel adds the ranges in a fixed order and applies the row scales,
// so the result is deterministic. It equals sum_c W_hat[r][c] x[c] up to fp32
// rounding.
//
// One 16-wave workgroup per CU keeps two table buffers (2 x 64 KB for VQ3R,
// 2 x 32 KB for VQ4P): each step builds the next block's table into one while
// the waves read the current block's from the other, with one barrier per
// block. The record stream of a wave runs two row groups ahead across block
// boundaries, so the first groups of the next block are in flight while its
// table is built.
//
// Runtime layout ("packed"): the GEMV reads indices repacked by
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
// which makes a half-wave's reads conflict-free; VQ3R keeps stage 0 twice
// (below).
//
// The stored-record entry point (vq_dequant_gemv on [rows][cols/8][3]
// records) first lists the distinct routed experts (k_gemv_route_stored), packs
// just those into the workspace (k_gemv_pack over the list) and then runs the
// same two kernels on the packed copies.
#include "vq_launch.hpp"

namespace vqk {

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int GJ = 16;     // slices per block
constexpr int GROUP = 64;  // rows per interleaved group (one wave)
constexpr int GEMV_WAVES = 16;
constexpr int GEMV_THREADS = 64 * GEMV_WAVES;
#ifndef VQ_GEMV_TILES_PER_CU
#define VQ_GEMV_TILES_PER_CU 1
#endif

// Table layouts. VQ3R: T[e][slot][slice] with a 256-byte row per codeword,
// four 16-float slots holding stages 0, 1, 2 and stage 0 again (64 KB): the LDS
// address of a lookup is (e << 8) | (slot*64 + slice*4), so one byte permute
// forms it from the record and a per-lane offset byte. VQ4P:
// T[e][t][replica][slice] (32 KB), two replicas.
template <int FMT> struct GemvCfg;
template <> struct GemvCfg<0> { static constexpr int R = 1, FLOATS = 256 * 64; };
template <> struct GemvCfg<1> { static constexpr int R = 2, FLOATS = 64 * 4 * 2 * 16; };

int64_t gemv_packed_bytes(int format, int64_t rows, int64_t cols) {
  (void)format;
  const int64_t nblk = (cols / DIM + GJ - 1) / GJ;
  const int64_t ng = (rows + GROUP - 1) / GROUP;
  return nblk * ng * GROUP * GJ * 3;
}

// ------------------------------------------------------------------ repack
// One workgroup (256 threads) per tile (expert slot, run of PACK_SB = 4
// consecutive blocks of 16 slices, group of 64 rows). Thread (row r, block q)
// reads the 48 record bytes of block q in row r (three 16-byte loads when the
// records are 16-byte aligned, else dword or byte loads), so the 4 threads of
// a row read its 192 contiguous bytes of the run (three whole 64-byte lines for
// rows of a multiple of 64 slices; one block per tile left most lines partly
// read). The tile goes through LDS and out as the packed layout's rotated
// 12-byte chunks, 4 x 64 per block, one chunk per thread and block (contiguous
// across a wave). Pad rows and slices are 0. Output slot i holds expert list[i]
// (list = NULL: expert i); slots at or past *count (when given) are skipped.
constexpr int PACK_SB = 4;

__global__ __launch_bounds__(256) void k_gemv_pack(const uint8_t* idx, int64_t expert_stride, int64_t rows,
                                                   int64_t V, int64_t n_slots, const int32_t* list,
                                                   const int32_t* count, uint8_t* out, int64_t packed_stride) {
  constexpr int NC = GJ / 4, RB = GJ * 3;  // 4 chunks per row, 48 record bytes per row and block
  __shared__ uint32_t tile[PACK_SB][GROUP][RB / 4 + 1];
  const int64_t ng = (rows + GROUP - 1) / GROUP, nblk = (V + GJ - 1) / GJ;
  const int64_t nsb = (nblk + PACK_SB - 1) / PACK_SB;
  const int64_t ntiles = n_slots * nsb * ng;
  const int64_t used = count ? (int64_t)*count : n_slots;
  const int tid = threadIdx.x;
  const int r = tid >> 2, q = tid & 3;        // load: row of the group, block of the run
  const int c = tid >> 6, lane = tid & 63;    // store: chunk c of row `lane`
  const bool quad_ok = (V & 15) == 0 && ((uintptr_t)idx & 15) == 0 && (expert_stride & 15) == 0;
  const bool dword_ok = ((V * 3) & 3) == 0 && ((uintptr_t)idx & 3) == 0 && (expert_stride & 3) == 0;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t i = t / (nsb * ng), rem = t % (nsb * ng);
    if (i >= used) break;  // tiles are in slot order
    const int64_t e = list ? (int64_t)list[i] : i;
    const int64_t sb = rem / ng, g = rem % ng;
    const int64_t row = g * GROUP + r;
    const int64_t b = sb * PACK_SB + q;
    uint32_t w[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) w[k] = 0u;
    if (row < rows && b < nblk) {
      const int64_t j0 = b * GJ;
      const uint8_t* src = idx + e * expert_stride + (row * V + j0) * 3;
      const int64_t nbytes = ((V - j0) < GJ ? (V - j0) : GJ) * 3;  // valid bytes of this block
      if (quad_ok && nbytes == RB) {
        const uint4* s16 = reinterpret_cast<const uint4*>(src);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const uint4 v = s16[k];
          w[4 * k] = v.x;
          w[4 * k + 1] = v.y;
          w[4 * k + 2] = v.z;
          w[4 * k + 3] = v.w;
        }
      } else if (dword_ok) {
        const uint32_t* s4 = reinterpret_cast<const uint32_t*>(src);
#pragma unroll
        for (int k = 0; k < 12; ++k)
          if (4 * k < nbytes) w[k] = s4[k];  // nbytes is a multiple of 12
      } else {
#pragma unroll
        for (int k = 0; k < RB; ++k)
          if (k < nbytes) w[k >> 2] |= (uint32_t)src[k] << (8 * (k & 3));
      }
    }
#pragma unroll
    for (int k = 0; k < 12; ++k) tile[q][r][k] = w[k];
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < PACK_SB; ++qb) {
      const int64_t bb = sb * PACK_SB + qb;
      if (bb >= nblk) break;  // uniform across the workgroup
      const uint8_t* tb = reinterpret_cast<const uint8_t*>(&tile[qb][lane][0]);
      uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int sl = (4 * c + m + lane) & (GJ - 1);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const int ob = 3 * m + k;
          o[ob >> 2] |= (uint32_t)tb[3 * sl + k] << (8 * (ob & 3));
        }
      }
      uint32_t* dst =
          reinterpret_cast<uint32_t*>(out + i * packed_stride + ((bb * ng + g) * NC + c) * (GROUP * 12) + lane * 12);
#pragma unroll
      for (int k = 0; k < 3; ++k) dst[k] = o[k];
    }
    __syncthreads();  // the tile buffer is refilled next
  }
}

// ------------------------------------------------------------------ stored-record routing
// One workgroup: the distinct valid expert ids of route[] in increasing id
// order (list[0 .. count)), and for every pair the position of its expert in
// that list (slot[p]; 0 for an invalid id, whose output the reduce zeroes).
// mark: n_experts ints of workspace (cleared here).
__global__ __launch_bounds__(1024) void k_gemv_route_stored(const int32_t* route, int npairs, int n_experts,
                                                            int32_t* mark, int32_t* slot, int32_t* list,
                                                            int32_t* count) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (n_experts + 1023) / 1024;
  const int e0 = tid * per, e1 = (e0 + per < n_experts) ? e0 + per : n_experts;
  for (int e = e0; e < e1; ++e) mark[e] = 0;
  __syncthreads();
  for (int p = tid; p < npairs; p += 1024) {
    const int e = route[p];
    if (e >= 0 && e < n_experts) mark[e] = 1;
  }
  __syncthreads();
  int s = 0;
  for (int e = e0; e < e1; ++e) s += mark[e];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan of the per-thread counts
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = part[tid] - s;
  for (int e = e0; e < e1; ++e) {
    const int m = mark[e];
    if (m) list[base] = e;
    mark[e] = base;  // rank of e among the used ids (read only for used ids)
    base += m;
  }
  if (tid == 1023) *count = part[1023];
  __syncthreads();
  for (int p = tid; p < npairs; p += 1024) {
    const int e = route[p];
    slot[p] = (e >= 0 && e < n_experts) ? mark[e] : 0;
  }
}

// ------------------------------------------------------------------ tables
// T[(e*S + t)*R + rep][m] = sum_k C_t[e][k] * x[(j0 + m)*8 + k] with fp32
// matrix cores (16x16x4: 16 codewords on M, the block's 16 slices on N, two
// products over k = 0..3 and 4..7). A task is (stage t, 16 codewords); its
// codebook operands are loaded once per tile (CbOps), the activation operand
// once per block.
template <int FMT, int NW>
struct CbOps {
  static constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K, NT = K / 16, TASKS = S * NT;
  static constexpr int PER_WAVE = (TASKS + NW - 1) / NW;
  float a[PER_WAVE][2];
};

// lane (codeword i = lane % 16, k quarter kq = lane / 16) holds C_t[16ct + i][4h + kq]
template <int FMT, int NW>
__device__ inline void cb_load(CbOps<FMT, NW>& op, const float* cb_g) {
  using O = CbOps<FMT, NW>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int u = 0; u < O::PER_WAVE; ++u) {
    const int task = wave + NW * u;
    const int tk = task < O::TASKS ? task : 0;
    const int t = tk / O::NT, ct = tk % O::NT;
#pragma unroll
    for (int h = 0; h < 2; ++h) op.a[u][h] = cb_g[((size_t)t * O::K + ct * 16 + i) * DIM + 4 * h + kq];
  }
}

// The activation operand of block [j0, j0 + nsl): lane (slice j = lane % 16,
// kq = lane / 16) holds x elements 4h + kq of slice j (fp16 bits), slice
// clamped (its column is zeroed).
__device__ inline void x_load(uint32_t xb[2], const uint16_t* xrow, int64_t j0, int nsl) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, kq = lane >> 4;
  const int jc = j < nsl ? j : 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) xb[h] = xrow[(j0 + jc) * DIM + 4 * h + kq];
}

template <int FMT, int NW>
__device__ inline void lut_compute(const CbOps<FMT, NW>& op, const uint32_t xb[2], float* lut, int nsl) {
  using O = CbOps<FMT, NW>;
  constexpr int R = GemvCfg<FMT>::R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, rg = lane >> 4;
  const bool sv = j < nsl;
  float b[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) b[h] = sv ? f16_bits_to_f32((uint16_t)xb[h]) : 0.0f;
#pragma unroll
  for (int u = 0; u < O::PER_WAVE; ++u) {
    const int task = wave + NW * u;
    if (task >= O::TASKS) break;  // wave-uniform
    const int t = task / O::NT, ct = task % O::NT;
    f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(op.a[u][0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(op.a[u][1], b[1], acc, 0, 0, 0);
    // lane (slice j, rg) holds codewords e = 16ct + 4rg + v
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = ct * 16 + 4 * rg + v;
      if constexpr (FMT == 0) {
        lut[e * 64 + t * GJ + j] = acc[v];
        if (t == 0) lut[e * 64 + 3 * GJ + j] = acc[v];  // stage 0 again in the row's fourth slot
      } else {
#pragma unroll
        for (int rep = 0; rep < R; ++rep) lut[((e * O::S + t) * R + rep) * GJ + j] = acc[v];
      }
    }
  }
}

// Tile order: the tiles of each XCD share are contiguous: workgroups are
// dealt to the 8 XCDs in turn.
__device__ inline uint32_t tile_of_block(uint32_t bid, uint32_t ntiles_pad) {
  const uint32_t per_xcd = ntiles_pad / 8;
  return (bid % 8) * per_xcd + bid / 8;
}

// A tile is (slot pair p, row chunk, range of nb blocks); tile index
// t = (chunk * nrange + range) * npairs + p. Matrices of more than 16 * GPW row
// groups are cut into nsplit chunks of near-equal group counts, so a tile never
// streams more than 16 * GPW * 64 rows and tall matrices still give many tiles.
// GPW = row groups per wave in a chunk (groups g = g0 + wave + 16k, k < GPW),
// fully unrolled. remap (may be NULL): packed slot of pair p (the stored-record
// path packs only the routed experts); else the packed slot is route[p].
template <int FMT, int GPW>
__global__ __launch_bounds__(GEMV_THREADS) void k_gemv(const uint8_t* pk, int64_t expert_stride, const int32_t* remap,
                                                       const float* cb_g, int64_t rows, int64_t cols, int n_experts,
                                                       const uint16_t* x, int topk, const int32_t* route,
                                                       float* partials, int npairs, int nblk, int nb, int nrange,
                                                       int gper, int grem, uint32_t ntiles, uint32_t ntiles_pad) {
  constexpr int S = Fmt<FMT>::S, K = Fmt<FMT>::K, R = GemvCfg<FMT>::R, NC = GJ / 4;
  constexpr int TF = GemvCfg<FMT>::FLOATS, NW = GEMV_WAVES;
  // VQ3R lookups address the tables straight from the record words (below),
  // except with four row groups per wave, where its registers would spill
  constexpr bool DIRECT = FMT == 0 && GPW <= 3;
  __shared__ float lut[2 * TF];
  // 32-bit index arithmetic (the host keeps the grid below 2^31): 64-bit
  // divisions would cost hundreds of scalar instructions per wave here.
  const uint32_t tile = tile_of_block(blockIdx.x, ntiles_pad);
  if (tile >= ntiles) return;
  const uint32_t cq = tile / (uint32_t)npairs, cc = cq / (uint32_t)nrange;
  const int p = (int)(tile - cq * (uint32_t)npairs), q = (int)(cq - cc * (uint32_t)nrange), chunk = (int)cc;
  const int tok = (int)((uint32_t)p / (uint32_t)topk);
  const int64_t V = cols / DIM;
  const int b0 = q * nb, b1 = (b0 + nb < nblk) ? b0 + nb : nblk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ng = (rows + GROUP - 1) / GROUP;
  // this tile's groups [g0, g1): chunks of gper or gper + 1 groups
  const int64_t g0 = (int64_t)chunk * gper + (chunk < grem ? chunk : grem);
  const int64_t g1 = g0 + gper + (chunk < grem ? 1 : 0);
  const uint8_t* eb = pk;  // set once the route id is in
  const uint16_t* xrow = x + (int64_t)tok * cols;
  const int nitems = (b1 - b0) * GPW;  // (block, group) items of this wave, in stream order
  // unconditional loads with a clamped item keep the wait counts exact
  uint32_t d[2][NC][3];
  auto load_item = [&](uint32_t (&dg)[NC][3], int it) {
    const int ic = it < nitems ? it : nitems - 1;
    const int64_t b = b0 + ic / GPW;
    int64_t g = g0 + wave + (int64_t)(ic % GPW) * NW;
    g = g < g1 ? g : g1 - 1;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(eb + (b * ng + g) * NC * (GROUP * 12)) + lane * 3;
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
  // VQ3R lookups. At step m = 4c + qq, lane l reads slice (m + l) mod 16; its
  // half-wave bit h = (l >> 4) & 1 rotates the order of the stages (lanes with
  // h = 1 take stages 1, 2, 0), and its k-th lookup reads slot k + h (slot 3 =
  // stage 0 again). The bank of a lookup is (slot*16 + slice) mod 32, so in
  // each lookup instruction the two 16-lane halves of a half-wave, at slots of
  // different parity, cover all 32 banks whatever the indices (with one copy of
  // stage 0, the third lookup would pair slots 2 and 0: a two-way conflict).
  // sel[qq] extracts record qq of a 12-byte chunk with its stages in the lane's
  // order; soff[k][c] holds, in byte qq, slot*64 + slice*4 for the lane's k-th
  // lookup at step 4c + qq.
  const uint32_t hb = (uint32_t)(lane >> 4) & 1u;
  // Addresses straight from the record words. Record qq of a chunk sits at
  // bytes 3qq .. 3qq+2 of its 12 bytes (stage-minor): qq 0 in word 0, qq 3 in
  // word 2, qq 1 across words 0 and 1, qq 2 across words 1 and 2.
  //  - qq 0 and 3: the lane's k-th lookup reads stage (k + h) mod 3 at slot
  //    k + h, its index byte picked from the word by a per-lane selector.
  //  - qq 1: both halves read stage 0 (word 0, byte 3) first, at slots 0 and 3;
  //    then stages 1 and 2 of word 1, the halves in swapped order (slots 1, 2
  //    and 2, 1). Every instruction still pairs slots of different parity.
  //  - qq 2: its three index bytes are first gathered into one word (as the
  //    gathered form below does for every record), then addressed from it.
  // soffD[par][k][c] holds the offsets slot*64 + slice*4 of the k-th lookups of
  // records 0, 1 and 3 in bytes 0, 1, 3 and the table buffer's bit in byte 2,
  // which every direct address takes as its byte 2; soff2[k] holds record 2's
  // offset of chunk c in byte c.
  uint32_t soffD[2][3][NC], soff2[3], selA[3], selB[3], selC[2], sel2 = 0;
  if constexpr (DIRECT) {
    auto off = [&](uint32_t slot, int m) { return slot * 64u + ((uint32_t)(m + lane) & (GJ - 1)) * 4u; };
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint32_t sl = (uint32_t)k + hb;                                      // records 0, 2, 3
      const uint32_t s1 = k == 0 ? (hb ? 3u : 0u) : (k == 1 ? 1u + hb : 2u - hb);  // record 1
      soff2[k] = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t v = off(sl, 4 * c) | (off(s1, 4 * c + 1) << 8) | (off(sl, 4 * c + 3) << 24);
        soffD[0][k][c] = v;
        soffD[1][k][c] = v | 0x10000u;
        soff2[k] |= off(sl, 4 * c + 2) << (8 * c);
      }
      const uint32_t st = ((uint32_t)k + hb) % 3u;  // stage of the k-th lookup (records 0, 2, 3)
      selA[k] = 0x0c060004u | (st << 8);            // record 0: word 0, byte st
      selB[k] = 0x0c060007u | ((1u + st) << 8);     // record 3: word 2, byte 1 + st
      if (k > 0) selC[k - 1] = 0x0c060005u | (((k == 1) == (hb == 0) ? 0u : 1u) << 8);  // record 1: word 1
    }
    // record 2's bytes within {word 2 : word 1}: stage 0 at 2, 1 at 3, 2 at 4
    sel2 = hb ? (3u | (4u << 8) | (2u << 16) | 0x0c000000u) : (2u | (3u << 8) | (4u << 16) | 0x0c000000u);
  }
  auto row_sum3_direct = [&](const uint32_t (&dg)[NC][3], auto lb) {
    constexpr int LB = decltype(lb)::value;
    auto look = [&](uint32_t a) { return *reinterpret_cast<const float*>(lbase + a); };
    float acc;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t w0 = dg[c][0], w1 = dg[c][1], w2 = dg[c][2];
      // record 0
      float t = look(__builtin_amdgcn_perm(soffD[LB][0][c], w0, selA[0]));
      t += look(__builtin_amdgcn_perm(soffD[LB][1][c], w0, selA[1]));
      t += look(__builtin_amdgcn_perm(soffD[LB][2][c], w0, selA[2]));
      acc = c == 0 ? t : acc + t;
      // record 1 (first lookup: word 0, byte 3, offset byte 1 for both halves)
      t = look(__builtin_amdgcn_perm(soffD[LB][0][c], w0, 0x0c060305u));
      t += look(__builtin_amdgcn_perm(soffD[LB][1][c], w1, selC[0]));
      t += look(__builtin_amdgcn_perm(soffD[LB][2][c], w1, selC[1]));
      acc += t;
      // record 2
      uint32_t w = __builtin_amdgcn_perm(w2, w1, sel2);
      if constexpr (LB == 1) w |= 1u << 24;
      t = look(__builtin_amdgcn_perm(soff2[0], w, 0x0c030004u | (uint32_t)c));
      t += look(__builtin_amdgcn_perm(soff2[1], w, 0x0c030104u | (uint32_t)c));
      t += look(__builtin_amdgcn_perm(soff2[2], w, 0x0c030204u | (uint32_t)c));
      acc += t;
      // record 3
      t = look(__builtin_amdgcn_perm(soffD[LB][0][c], w2, selB[0]));
      t += look(__builtin_amdgcn_perm(soffD[LB][1][c], w2, selB[1]));
      t += look(__builtin_amdgcn_perm(soffD[LB][2][c], w2, selB[2]));
      acc += t;
    }
    return acc;
  };
  uint32_t sel[4], soff[3][NC];
  if constexpr (FMT == 0 && !DIRECT) {
    // bytes of record qq within {hi, lo} (lo = bytes 0-3): qq 0: 0 1 2, 1: 3 4 5 (hi = next dword),
    // 2: 2 3 4 (lo = dword 1), 3: 5 6 7
    constexpr uint32_t b0[4] = {0, 3, 2, 5};
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint32_t x0 = b0[qq], x1 = b0[qq] + 1, x2 = b0[qq] + 2;
      sel[qq] = hb ? (x1 | (x2 << 8) | (x0 << 16) | 0x0c000000u) : (x0 | (x1 << 8) | (x2 << 16) | 0x0c000000u);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint32_t slot = (uint32_t)k + hb;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t v = 0;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) v |= (slot * 64u + ((uint32_t)(4 * c + qq + lane) & (GJ - 1)) * 4u) << (8 * qq);
        soff[k][c] = v;
      }
    }
  }
  // Every record's index bytes gathered into one word w first (used where the
  // direct form needs too many registers: four row groups per wave). lb: the
  // table buffer (the odd one sits 64 KB up, its bit carried in byte 3 of w and
  // moved to address byte 2 by the perm).
  auto row_sum3_perm = [&](const uint32_t (&dg)[NC][3], auto lb) {
    constexpr int LB = decltype(lb)::value;
    float acc;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const uint32_t lo = dg[c][qq < 2 ? 0 : 1], hi = dg[c][qq < 2 ? 1 : 2];
        uint32_t w = __builtin_amdgcn_perm(hi, lo, sel[qq]);  // the lane's stage order in bytes 0-2
        if constexpr (LB == 1) w |= 1u << 24;
        float tsum;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          // byte 0: offset byte qq of soff[k][c]; byte 1: stage index byte k of w;
          // byte 2: the buffer bit (byte 3 of w)
          const uint32_t a = __builtin_amdgcn_perm(soff[k][c], w, 0x0c030004u | ((uint32_t)k << 8) | (uint32_t)qq);
          const float v = *reinterpret_cast<const float*>(lbase + a);
          tsum = k == 0 ? v : tsum + v;
        }
        acc = (c == 0 && qq == 0) ? tsum : acc + tsum;
      }
    }
    return acc;
  };
  auto row_sum3 = [&](const uint32_t (&dg)[NC][3], auto lb) {
    if constexpr (DIRECT) return row_sum3_direct(dg, lb);
    else return row_sum3_perm(dg, lb);
  };
  auto row_sum = [&](const uint32_t (&dg)[NC][3], auto lb) {
    constexpr int LB = decltype(lb)::value;
    if constexpr (FMT == 0) return row_sum3(dg, lb);
    const char* lb_base = lbase + LB * TF * 4;
    float acc;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        // record qq of the chunk = bytes 3qq .. 3qq+2 of the 12 bytes
        const int byte0 = 3 * qq, k0 = byte0 >> 2, o = byte0 & 3;
        const uint32_t w =
            (o <= 1) ? (dg[c][k0] >> (8 * o)) : ((dg[c][k0] >> (8 * o)) | (dg[c][k0 + 1] << (32 - 8 * o)));
        const int m = 4 * c + qq;
        const uint32_t soff = (((uint32_t)(m + lane) & (GJ - 1)) << 2) + rep_off;
        // the stage terms summed in stage order, then added to the row sum
        float tsum = *reinterpret_cast<const float*>(lb_base + ((uint32_t)record_index<FMT>(w, 0) * E_STRIDE + soff));
#pragma unroll
        for (int t = 1; t < S; ++t) {
          const uint32_t ei = (uint32_t)record_index<FMT>(w, t);
          tsum += *reinterpret_cast<const float*>(lb_base + (ei * E_STRIDE + soff) + t * T_STRIDE);
        }
        acc = (c == 0 && qq == 0) ? tsum : acc + tsum;
      }
    }
    return acc;
  };
  float rs[GPW];
#pragma unroll
  for (int k = 0; k < GPW; ++k) rs[k] = 0.0f;
  CbOps<FMT, NW> ops;
  uint32_t xb[2], xb1[2];
  // Item i = (b - b0) * GPW + k sits in ring slot i % 2; the load of item
  // i + 2 follows its consume. Blocks are unrolled by two, which fixes both
  // the slot and the table buffer of every step at compile time.
  auto consume_block = [&](auto u, int i0) {
    constexpr int U = decltype(u)::value;
#pragma unroll
    for (int k = 0; k < GPW; ++k) {
      const int64_t g = g0 + wave + (int64_t)k * NW;
      if (g < g1) rs[k] += row_sum(d[(U * GPW + k) & 1], u);  // wave-uniform
      load_item(d[(U * GPW + k) & 1], i0 + k + 2);
    }
  };
  auto nsl_of = [&](int b) {
    const int64_t j0 = (int64_t)b * GJ;
    return (int)((V - j0) < GJ ? (V - j0) : GJ);
  };
  // Block b's table is in buffer (b - b0) & 1. Each step builds the next
  // block's table into the other buffer, then reads this block's; one barrier
  // per block orders both (the writes of step b + 1 go to the buffer that step
  // b read).
  auto step = [&](auto u, int b) {
    constexpr int U = decltype(u)::value;
    if (b + 1 < b1) {
      lut_compute<FMT, NW>(ops, xb, lut + (U ^ 1) * TF, nsl_of(b + 1));
      if (b + 2 < b1) x_load(xb, xrow, (int64_t)(b + 2) * GJ, nsl_of(b + 2));
    }
    consume_block(u, (b - b0) * GPW);
    __syncthreads();
  };
  // The table operands (codebooks, activations) do not depend on the route id
  // and go out first: issued behind the index stream of every CU they would
  // hold up the first table by several microseconds.
  cb_load<FMT, NW>(ops, cb_g);
  x_load(xb, xrow, (int64_t)b0 * GJ, nsl_of(b0));
  const int bx1 = b0 + 1 < b1 ? b0 + 1 : b0;  // the second block's activations come in with the first's
  x_load(xb1, xrow, (int64_t)bx1 * GJ, nsl_of(bx1));
  __builtin_amdgcn_sched_barrier(0);
  // A route id outside [0, n_experts) is flagged and its outputs zeroed by
  // k_gemv_reduce; its tile runs on expert 0 (there is always one) and stores
  // nothing, so no branch holds up the loads above.
  const int e_raw = route[p];
  const int slot = (remap ? remap : route)[p];
  const bool bad = e_raw < 0 || e_raw >= n_experts;
  eb = pk + (int64_t)(remap || !bad ? slot : 0) * expert_stride;
#pragma unroll
  for (int i = 0; i < 2; ++i) load_item(d[i], i);  // (as a loop: the register allocation comes out far tighter)
  __builtin_amdgcn_sched_barrier(0);
  lut_compute<FMT, NW>(ops, xb, lut, nsl_of(b0));
  xb[0] = xb1[0];
  xb[1] = xb1[1];
  __syncthreads();
  for (int b = b0; b < b1; b += 2) {
    step(std::integral_constant<int, 0>(), b);
    if (b + 1 >= b1) break;
    step(std::integral_constant<int, 1>(), b + 1);
  }
  float* part = partials + ((int64_t)p * nrange + q) * rows;
#pragma unroll
  for (int k = 0; k < GPW; ++k) {
    const int64_t g = g0 + wave + (int64_t)k * NW;
    const int64_t row = g * GROUP + lane;
    if (!bad && g < g1 && row < rows) part[row] = rs[k];
  }
}

// y[p][r] = s_r * sum over the ranges in a fixed order. Also writes the status
// flags of the call (route ids outside [0, n_experts)), so no reset is needed.
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* partials, const uint16_t* scales,
                                                     int64_t scale_stride, const int32_t* route, int n_experts,
                                                     int64_t rows, int nrange, int npairs, float* y, uint32_t* flags) {
  const int p = blockIdx.y;
  const int e = route[p];
  const bool bad = e < 0 || e >= n_experts;
  if (blockIdx.x == 0 && p == 0 && threadIdx.x < 64) {
    bool any = false;
    for (int q = threadIdx.x; q < npairs; q += 64) any |= (route[q] < 0 || route[q] >= n_experts);
    any = __any(any);
    if (threadIdx.x == 0) *flags = any ? ST_ROUTE : 0u;
  }
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.0f;
  if (!bad) {
    const float* pp = partials + (int64_t)p * nrange * rows + r;
    const float sc = f16_bits_to_f32(scales[(int64_t)e * scale_stride + r]);
    // up to sixteen loads in flight, then added in range order
    for (int q = 0; q < nrange; q += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = (q + u < nrange) ? pp[(int64_t)(q + u) * rows] : 0.0f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (q + u < nrange) acc += v[u];  // uniform over the workgroup
      }
    }
    acc *= sc;
  }
  y[(int64_t)p * rows + r] = acc;
}

__global__ void k_gemv_clear(uint32_t* flags) {
  if (threadIdx.x == 0) *flags = 0;
}

// ------------------------------------------------------------------ launch geometry
// Row chunks of a tile column: as few as keep every chunk within 4 groups per
// wave (4096 rows). Cutting small calls' rows further (so that their ranges
// span more blocks) measured no faster with the 16-wave workgroups.
int gemv_row_chunks(int64_t rows, int64_t npairs) {
  (void)npairs;
  const int64_t ng = (rows + GROUP - 1) / GROUP;
  int64_t n = (ng + 4 * GEMV_WAVES - 1) / (4 * GEMV_WAVES);
  if (n > ng) n = ng > 0 ? ng : 1;
  if (n < 1) n = 1;
  return (int)n;
}

// Row groups per wave: the groups of the largest chunk over the 16 waves.
static int gemv_gpw(int64_t rows, int nsplit) {
  const int64_t ng = (rows + GROUP - 1) / GROUP;
  const int64_t per = (ng + nsplit - 1) / nsplit;
  return (int)((per + GEMV_WAVES - 1) / GEMV_WAVES);
}

// Blocks per range: as many as keep about VQ_GEMV_TILES_PER_CU tiles per CU in
// the launch (fewer, longer tiles mean fewer partial sums and fewer table
// start-ups; too few tiles leave CUs idle).
static void gemv_ranges(int64_t npairs, int nsplit, int nblk, int ncu, int* nb, int* nrange) {
  const int64_t target = (int64_t)VQ_GEMV_TILES_PER_CU * (ncu > 0 ? ncu : 1);
  int64_t want = target / (npairs * nsplit > 0 ? npairs * nsplit : 1);
  if (want < 1) want = 1;
  if (want > nblk) want = nblk;
  int b = (int)((nblk + want - 1) / want);
  *nb = b;
  *nrange = (nblk + b - 1) / b;
}

int64_t gemv_tiles(int64_t rows, int64_t cols, int64_t npairs) {
  const int64_t nblk = (cols / DIM + GJ - 1) / GJ;
  return npairs * nblk * gemv_row_chunks(rows, npairs);  // upper bound (one block per range)
}

int64_t gemv_partials_floats(int format, int64_t rows, int64_t cols, int64_t npairs) {
  (void)format;
  const int64_t nblk = (cols / DIM + GJ - 1) / GJ;
  return npairs * nblk * rows;  // upper bound (one block per range)
}

// The partial sums one launch on `ncu` compute units writes: one per (pair,
// range, row).
int64_t gemv_partials_floats_used(int format, int64_t rows, int64_t cols, int64_t npairs, int ncu) {
  (void)format;
  const int nblk = (int)((cols / DIM + GJ - 1) / GJ);
  int nb, nrange;
  gemv_ranges(npairs, gemv_row_chunks(rows, npairs), nblk, ncu, &nb, &nrange);
  return npairs * nrange * rows;
}

template <int FMT>
static hipError_t launch_gemv_t(const GemvArgs& a) {
  const int64_t npairs = (int64_t)a.ntok * a.topk;
  const int64_t V = a.cols / DIM;
  const int nblk = (int)((V + GJ - 1) / GJ);
  const int nsplit = gemv_row_chunks(a.rows, npairs);
  int nb, nrange;
  gemv_ranges(npairs, nsplit, nblk, a.ncu, &nb, &nrange);
  const int64_t ntiles = npairs * nsplit * nrange;
  const int64_t ntiles_pad = (ntiles + 7) / 8 * 8;  // below 2^31 (argument checks)
  const int64_t ng = (a.rows + GROUP - 1) / GROUP;
  const int gpw = gemv_gpw(a.rows, nsplit);
  auto go = [&](auto kern) {
    kern<<<(unsigned)ntiles_pad, GEMV_THREADS, 0, a.stream>>>(a.idx, a.expert_stride, a.remap, a.codebooks, a.rows,
                                                               a.cols, a.n_experts, a.x, a.topk, a.route,
                                                               a.partials, (int)npairs, nblk, nb, nrange,
                                                               (int)(ng / nsplit), (int)(ng % nsplit), (uint32_t)ntiles,
                                                               (uint32_t)ntiles_pad);
  };
  if (gpw == 1) go(k_gemv<FMT, 1>);
  else if (gpw == 2) go(k_gemv<FMT, 2>);
  else if (gpw == 3) go(k_gemv<FMT, 3>);
  else go(k_gemv<FMT, 4>);
  dim3 g2((unsigned)((a.rows + 255) / 256), (unsigned)npairs);
  k_gemv_reduce<<<g2, 256, 0, a.stream>>>(a.partials, a.scales, a.scale_stride, a.route, a.n_experts, a.rows, nrange,
                                          (int)npairs, a.y, a.flags);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs& a) {
  if ((int64_t)a.ntok * a.topk == 0 || a.rows == 0) {
    k_gemv_clear<<<1, 64, 0, a.stream>>>(a.flags);
    return hipGetLastError();
  }
  return a.format == 0 ? launch_gemv_t<0>(a) : launch_gemv_t<1>(a);
}

hipError_t launch_gemv_pack(int format, const uint8_t* idx, int64_t expert_stride, int64_t rows, int64_t cols,
                            int64_t n_slots, const int32_t* list, const int32_t* count, uint8_t* out, int ncu,
                            hipStream_t s) {
  const int64_t V = cols / DIM;
  const int64_t nsb = ((V + GJ - 1) / GJ + PACK_SB - 1) / PACK_SB;
  const int64_t ntiles = nsb * ((rows + GROUP - 1) / GROUP) * n_slots;
  if (ntiles == 0) return hipSuccess;
  int64_t g = ntiles;
  if (g > (int64_t)ncu * 32) g = (int64_t)ncu * 32;
  k_gemv_pack<<<(unsigned)g, 256, 0, s>>>(idx, expert_stride, rows, V, n_slots, list, count, out,
                                          gemv_packed_bytes(format, rows, cols));
  return hipGetLastError();
}

hipError_t launch_gemv_route_stored(const int32_t* route, int npairs, int n_experts, int32_t* mark, int32_t* slot,
                                    int32_t* list, int32_t* count, hipStream_t s) {
  k_gemv_route_stored<<<1, 1024, 0, s>>>(route, npairs, n_experts, mark, slot, list, count);
  return hipGetLastError();
}

}  // namespace vqk
