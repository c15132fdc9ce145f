// Host-side launch interface of the Tied Trit-Planes codec (vq_ttp.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_device.hpp"

namespace vqk {

constexpr int TTP_GROUP = 256;        // weights per fp16 scale
constexpr int TTP_CHUNK = 64;         // groups per error partial

hipError_t launch_ttp_quantize(const void* W, int dtype, int64_t n_groups, uint8_t* codes, uint16_t* scales,
                               WsHeader* hdr, int ncu, hipStream_t s);
hipError_t launch_ttp_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t n_groups, float* out,
                                 int ncu, hipStream_t s);
// partials: [n_mats][chunks][2] fp64 with chunks = ceil(groups_per_mat / TTP_CHUNK)
hipError_t launch_ttp_error(const void* W, int dtype, const uint8_t* codes, const uint16_t* scales,
                            int64_t groups_per_mat, int64_t n_mats, double* partials, double* sums, WsHeader* hdr,
                            hipStream_t s);

}  // namespace vqk
