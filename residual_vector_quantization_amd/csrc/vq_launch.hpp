// Host-side launch interface between the C ABI (vq_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_device.hpp"

namespace vqk {

enum { ENGINE_AUTO = 0, ENGINE_F16X = 1, ENGINE_F32 = 2, ENGINE_VALU = 3, ENGINE_EXACT = 4 };

struct EncodeArgs {
  int format, engine, dtype;
  const void* W;
  int64_t rows, cols;
  const float* codebooks;
  uint8_t* idx;
  uint16_t* scales;
  WsHeader* hdr;
  uint32_t* list;
  uint32_t cap;
  int ncu;
  hipStream_t stream;
};

struct FitArgs {
  int format, engine, dtype;
  const void* const* mats;  // host array of device pointers
  int64_t n_mats, rows, cols, n;
  int iters, clog2n;
  const int64_t* init;      // device copy, [stages][K]
  float* codebooks;
  WsHeader* hdr;
  float* R[2];
  uint32_t* list;
  uint32_t cap;
  long long* partials;
  int n_assign_blocks, n_exact_blocks;
  int ncu;
  hipStream_t stream;
};

struct DecodeArgs {
  int format, stages_used;
  const uint8_t* idx;
  const uint16_t* scales;
  const float* codebooks;
  int64_t rows, cols;
  float* out;
  int ncu;
  hipStream_t stream;
};

struct ErrorArgs {
  int format, dtype;
  const void* W;
  const uint8_t* idx;
  const uint16_t* scales;
  const float* codebooks;
  int64_t n_mats, rows, cols;
  double* sums;
  double* rel;       // [n_mats][stages] relative errors, or NULL
  double* rel_all;   // [stages] over all matrices, or NULL
  double* partials;  // [n_mats][error_chunks(rows)][stages+1]
  int blocks;        // grid width per matrix (does not change the result)
  WsHeader* hdr;
  hipStream_t stream;
};

struct GemvArgs {
  int format;
  const uint8_t* idx;       // packed experts
  int64_t expert_stride;
  const int32_t* remap;     // packed slot of each pair (NULL: the route id itself)
  const uint16_t* scales;
  int64_t scale_stride;
  const float* codebooks;
  int64_t rows, cols;
  int n_experts;
  const uint16_t* x;
  int ntok, topk;
  const int32_t* route;
  float* y;
  float* partials;  // [ntok*topk][nrange][rows]
  uint32_t* flags;  // the call's status word (route ids outside [0, n_experts))
  int ncu;
  hipStream_t stream;
};

struct Mxfp4Args {
  int dtype;
  const void* W;
  int64_t rows, cols;
  void* out;     // fp32, or bf16 when out_bf16
  int out_bf16;
  WsHeader* hdr;
  int ncu;
  hipStream_t stream;
};

// GEMV sizes: floats of tile partial sums (workspace), bytes of one packed expert.
int64_t gemv_partials_floats(int format, int64_t rows, int64_t cols, int64_t npairs);
int64_t gemv_partials_floats_used(int format, int64_t rows, int64_t cols, int64_t npairs, int ncu);
int64_t gemv_packed_bytes(int format, int64_t rows, int64_t cols);
int gemv_row_chunks(int64_t rows, int64_t npairs);                  // row chunks of a GEMV tile column
int64_t gemv_tiles(int64_t rows, int64_t cols, int64_t npairs);     // GEMV workgroups (before padding)
// Packs n_slots experts into the GEMV layout: slot i <- expert list[i] (list
// NULL: expert i) read at idx + expert * expert_stride; slots at or past *count
// (count may be NULL) are skipped.
hipError_t launch_gemv_pack(int format, const uint8_t* idx, int64_t expert_stride, int64_t rows, int64_t cols,
                            int64_t n_slots, const int32_t* list, const int32_t* count, uint8_t* out, int ncu,
                            hipStream_t s);
// Distinct valid expert ids of route[] (list, count) and each pair's position
// in that list (slot); mark = n_experts ints of scratch.
hipError_t launch_gemv_route_stored(const int32_t* route, int npairs, int n_experts, int32_t* mark, int32_t* slot,
                                    int32_t* list, int32_t* count, hipStream_t s);

hipError_t launch_reset(WsHeader* hdr, hipStream_t s);
hipError_t launch_encode(const EncodeArgs& a);
hipError_t launch_fit(const FitArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_error(const ErrorArgs& a);
hipError_t launch_gemv(const GemvArgs& a);

// rows per error chunk and the chunk count of a matrix (fixed by its row count)
constexpr int ERR_CHUNK = 16;
inline int64_t error_chunks(int64_t rows) { return (rows + ERR_CHUNK - 1) / ERR_CHUNK; }
hipError_t launch_mxfp4(const Mxfp4Args& a);
hipError_t launch_stream_read(const void* src, uint64_t nbytes, uint32_t* out, int ncu, hipStream_t s);

}  // namespace vqk
