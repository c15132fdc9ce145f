// Host-side launch interface of the batched dequant-GEMM (vq_gemm.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_device.hpp"

namespace vqk {

// Routing tables in the workspace after the 256-byte header (int32 each):
//   counts[E], offsets[E + 1], tile_offsets[E + 1], list[npairs],
//   tile_expert[max_tiles], tile_m0[max_tiles], n_tiles[1]
struct GemmLayout {
  size_t counts, offsets, tile_offsets, list, tile_expert, tile_m0, n_tiles, total;
  int64_t max_tiles;
};

constexpr int GEMM_MT_MIN = 32;  // smallest pair tile; the workspace is sized for it
constexpr int GEMM_WAVES = 8;    // output rows per workgroup: 32 per wave

GemmLayout gemm_layout(int64_t n_experts, int64_t npairs);
int gemm_msub(int64_t n_experts, int64_t npairs);  // pair sub-tiles of 32 per tile for this call

struct GemmArgs {
  int format;
  const uint8_t* idx;  // [E][rows][cols/8][3] with expert_stride bytes between experts
  int64_t expert_stride;
  const uint16_t* scales;
  int64_t scale_stride;
  const float* codebooks;
  int64_t rows, cols;
  int n_experts;
  const uint16_t* x;  // fp16 [ntok][cols]
  int ntok, topk;
  const int32_t* route;
  float* y;           // [ntok][topk][rows]
  WsHeader* hdr;
  char* ws;           // workspace base (header first)
  GemmLayout L;
  hipStream_t stream;
};

hipError_t launch_gemm(const GemmArgs& a);

}  // namespace vqk
