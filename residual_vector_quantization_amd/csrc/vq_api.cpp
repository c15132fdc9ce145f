// C ABI of libvq (declarations and documentation in include/vq.h): argument
// validation, workspace layout and kernel launches. No allocation happens here.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <unordered_set>
#include <vector>

#include "../../include/vq.h"
#include "vq_gemm.hpp"
#include "vq_ttp.hpp"
#include "vq_launch.hpp"

using namespace vqk;

namespace {

constexpr int kVersion = (1 << 16) | 0;
constexpr size_t kHeader = sizeof(WsHeader);
constexpr int64_t kMaxCols = 1 << 20;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline bool fmt_ok(int f) { return f == VQ_FMT_VQ3R || f == VQ_FMT_VQ4P; }
inline bool dtype_ok(int d) { return d == VQ_DT_F32 || d == VQ_DT_BF16 || d == VQ_DT_F16; }
inline int stages_of(int f) { return f == VQ_FMT_VQ3R ? 3 : 4; }
inline int entries_of(int f) { return f == VQ_FMT_VQ3R ? 256 : 64; }
inline size_t esize(int d) { return d == VQ_DT_F32 ? 4 : 2; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// rows/cols shared checks: cols multiple of 8 and within range; vector count fits 32 bits
int check_shape(int64_t rows, int64_t cols, bool allow_empty_rows = true) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return VQ_EINVAL;
  if (!allow_empty_rows && rows == 0) return VQ_EINVAL;
  if (cols > kMaxCols) return VQ_ERANGE;
  if ((uint64_t)rows * (uint64_t)(cols / 8) >= (1ull << 32)) return VQ_ERANGE;
  return VQ_OK;
}

int device_cus(int* ncu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VQ_EDEVICE;
  if (hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return VQ_EDEVICE;
  if (*ncu < 1) *ncu = 1;
  return VQ_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? VQ_OK : VQ_EDEVICE; }

uint32_t list_capacity(uint64_t nvec) {
  uint64_t cap = nvec / 16;
  if (cap < 4096) cap = 4096;
  if (cap > 0xFFFFFFFFull) cap = 0xFFFFFFFFull;
  return (uint32_t)cap;
}

// ---- fit workspace
struct FitLayout {
  size_t init, r0, r1, list, partials, total;
  uint32_t cap;
  int ga, gf;
};

// The partial-slot counts of the fit are fixed (not taken from the device) so
// that the workspace size does not depend on the GPU it is queried on. The
// assign launches use at most kFitAssignBlocks of them: as many four-wave
// workgroups as the device holds at once (4 per CU where registers and LDS
// allow it, 1024 on a 256-CU part; 512 left 2 per CU and the fit took 2-3 %
// longer).
constexpr int64_t kFitAssignBlocks = 1024, kFitExactBlocks = 256;

FitLayout fit_layout(int format, int64_t n) {
  FitLayout L;
  const int K = entries_of(format), S = stages_of(format);
  L.cap = list_capacity((uint64_t)n);
  int64_t groups = (n + 31) / 32;
  int64_t ga = (groups + 3) / 4;
  if (ga > kFitAssignBlocks) ga = kFitAssignBlocks;
  if (ga < 1) ga = 1;
  int64_t gf = (n / 16 + 255) / 256;
  if (gf > kFitExactBlocks) gf = kFitExactBlocks;
  if (gf < 1) gf = 1;
  L.ga = (int)ga;
  L.gf = (int)gf;
  size_t off = kHeader;
  L.init = off;
  off = align256(off + sizeof(int64_t) * S * K);
  L.r0 = off;
  off = align256(off + sizeof(float) * 8 * (size_t)n);
  L.r1 = off;
  off = align256(off + sizeof(float) * 8 * (size_t)n);
  L.list = off;
  off = align256(off + sizeof(uint32_t) * (size_t)L.cap);
  L.partials = off;
  off = align256(off + sizeof(long long) * (size_t)(L.ga + L.gf) * K * 9);
  L.total = off;
  return L;
}

// grid width per matrix for vq_error: about 2048 blocks in all, at most one per chunk
int error_blocks(int64_t rows, int64_t n_mats) {
  int64_t want = error_chunks(rows);
  int64_t cap = (2048 + n_mats - 1) / n_mats;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return (int)want;
}

size_t error_ws_bytes(int format, int64_t n_mats, int64_t rows) {
  return align256(kHeader + sizeof(double) * (size_t)n_mats * (size_t)error_chunks(rows) * (stages_of(format) + 1));
}


// argument checks shared by the packed and the stored-record GEMV
int gemv_check(int format, int64_t rows, int64_t cols, int32_t n_experts, int64_t expert_stride,
               int64_t min_stride, int64_t scale_stride, int32_t ntok, int32_t topk, const void* recs,
               const void* scales, const void* codebooks, const void* x, const void* route, const void* y) {
  if (!fmt_ok(format)) return VQ_EINVAL;
  int st = check_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (ntok < 0 || topk < 0 || n_experts < 1 || expert_stride < 0 || scale_stride < 0) return VQ_EINVAL;
  if (n_experts > 1 && (expert_stride < min_stride || scale_stride < rows)) return VQ_EINVAL;
  if (!recs || !scales || !codebooks || !x || !route || !y) return VQ_EINVAL;
  if ((int64_t)ntok * topk >= 65536) return VQ_ERANGE;
  if (gemv_tiles(rows, cols, (int64_t)ntok * topk) > ((int64_t)1 << 31) - 64) return VQ_ERANGE;  // grid width
  return VQ_OK;
}

void gemv_fill(GemvArgs& a, int format, const uint16_t* scales, int64_t scale_stride, const float* codebooks,
               int64_t rows, int64_t cols, int32_t n_experts, const uint16_t* x, int32_t ntok, const int32_t* route,
               int32_t topk, float* y, void* workspace, hipStream_t s) {
  a.format = format;
  a.scales = scales;
  a.scale_stride = scale_stride;
  a.codebooks = codebooks;
  a.rows = rows;
  a.cols = cols;
  a.n_experts = n_experts;
  a.x = x;
  a.ntok = ntok;
  a.topk = topk;
  a.route = route;
  a.y = y;
  a.flags = &((WsHeader*)workspace)->flags;
  a.remap = nullptr;
  a.stream = s;
}

size_t gemv_partials_bytes(int format, int64_t rows, int64_t cols, int32_t ntok, int32_t topk) {
  return align256(sizeof(float) * (size_t)gemv_partials_floats(format, rows, cols, (int64_t)ntok * topk));
}

// stored-record GEMV workspace: header, partial sums, expert marks, pair slots,
// expert list and count, then the packed copies of up to min(pairs, experts)
// experts
struct GemvStoredLayout {
  size_t partials, mark, slot, list, count, packed, total;
  int64_t n_slots;
};

GemvStoredLayout gemv_stored_layout(int format, int64_t rows, int64_t cols, int32_t ntok, int32_t topk,
                                    int32_t n_experts) {
  GemvStoredLayout L;
  const int64_t npairs = (int64_t)ntok * topk;
  L.n_slots = npairs < n_experts ? npairs : n_experts;
  size_t off = kHeader;
  L.partials = off;
  off += gemv_partials_bytes(format, rows, cols, ntok, topk);
  L.mark = off;
  off = align256(off + sizeof(int32_t) * (size_t)n_experts);
  L.slot = off;
  off = align256(off + sizeof(int32_t) * (size_t)(npairs > 0 ? npairs : 1));
  L.list = off;
  off = align256(off + sizeof(int32_t) * (size_t)(npairs > 0 ? npairs : 1));
  L.count = off;
  off = align256(off + sizeof(int32_t));
  L.packed = off;
  off = align256(off + (size_t)gemv_packed_bytes(format, rows, cols) * (size_t)L.n_slots);
  L.total = off;
  return L;
}

}  // namespace

// Device scratch of vq_dequant_gemv_packed_noalloc: the status word (when the
// caller passes no status buffer) followed by the split-K partial sums. Each
// GPU the library runs on holds its own copy until the process ends. Host code
// never uses this name as an address: scratch_base() looks the per-device
// address up once with hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[VQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array (looked up on the first call
// on each device, with that device current).
int scratch_base(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VQ_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return VQ_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VQ_OK;
}

}  // namespace

extern "C" {

const char* vq_status_string(int status) {
  switch (status) {
    case VQ_OK: return "ok";
    case VQ_EINVAL: return "invalid argument";
    case VQ_ERANGE: return "size out of supported range";
    case VQ_EWORKSPACE: return "workspace missing, misaligned or too small";
    case VQ_EDEVICE: return "HIP runtime error";
    case VQ_EDATA: return "data error flagged on the device";
    case VQ_EIO: return "container file I/O failed";
    case VQ_EFORMAT: return "container file malformed or corrupt";
    case VQ_ESCRATCH: return "call too large for the no-allocation scratch";
    default: return "unknown status";
  }
}

int vq_version(void) { return kVersion; }

int vq_read_status(const void* workspace, void* stream, uint32_t* flags_out) {
  if (!workspace || !aligned(workspace, 256)) return VQ_EWORKSPACE;
  uint32_t flags = 0;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(&flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return VQ_EDEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return VQ_EDEVICE;
  if (flags_out) *flags_out = flags;
  return (flags & ST_ERROR_MASK) ? VQ_EDATA : VQ_OK;
}

int vq_read_device_status(const void* workspace, void* stream) { return vq_read_status(workspace, stream, nullptr); }

int vq_clear_status(void* workspace, void* stream) {
  if (!workspace || !aligned(workspace, 256)) return VQ_EWORKSPACE;
  return hip_status(launch_reset((WsHeader*)workspace, (hipStream_t)stream));
}

// ---------------------------------------------------------------- encode
size_t vq_encode_workspace_size(int format, int64_t rows, int64_t cols) {
  if (!fmt_ok(format) || check_shape(rows, cols) != VQ_OK) return 0;
  const uint64_t nvec = (uint64_t)rows * (uint64_t)(cols / 8);
  return align256(kHeader + sizeof(uint32_t) * (size_t)list_capacity(nvec));
}

int vq_encode(int format, int engine, const void* W, int dtype, int64_t rows, int64_t cols, const float* codebooks,
              uint8_t* idx, uint16_t* scales, void* workspace, size_t ws_bytes, void* stream) {
  if (!fmt_ok(format) || !dtype_ok(dtype) || engine < VQ_ENGINE_AUTO || engine > VQ_ENGINE_EXACT) return VQ_EINVAL;
  int st = check_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (rows == 0) return VQ_OK;  // empty input: nothing is read or written
  if (!W || !codebooks || !idx || !scales) return VQ_EINVAL;
  if (!aligned(W, 16) || !aligned(codebooks, 16)) return VQ_EINVAL;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < vq_encode_workspace_size(format, rows, cols))
    return VQ_EWORKSPACE;
  EncodeArgs a;
  a.format = format;
  a.engine = engine == VQ_ENGINE_AUTO ? ENGINE_F16X : engine;
  a.dtype = dtype;
  a.W = W;
  a.rows = rows;
  a.cols = cols;
  a.codebooks = codebooks;
  a.idx = idx;
  a.scales = scales;
  a.hdr = (WsHeader*)workspace;
  a.list = (uint32_t*)((char*)workspace + kHeader);
  a.cap = list_capacity((uint64_t)rows * (uint64_t)(cols / 8));
  a.stream = (hipStream_t)stream;
  if ((st = device_cus(&a.ncu)) != VQ_OK) return st;
  return hip_status(launch_encode(a));
}

int vq3r_encode(const void* W, int dtype, int64_t rows, int64_t cols, const float* codebooks, uint8_t* idx,
                uint16_t* scales, void* workspace, size_t ws_bytes, void* stream) {
  return vq_encode(VQ_FMT_VQ3R, VQ_ENGINE_AUTO, W, dtype, rows, cols, codebooks, idx, scales, workspace, ws_bytes,
                   stream);
}

int vq4p_encode(const void* W, int dtype, int64_t rows, int64_t cols, const float* codebooks, uint8_t* idx,
                uint16_t* scales, void* workspace, size_t ws_bytes, void* stream) {
  return vq_encode(VQ_FMT_VQ4P, VQ_ENGINE_AUTO, W, dtype, rows, cols, codebooks, idx, scales, workspace, ws_bytes,
                   stream);
}

// ---------------------------------------------------------------- fit
size_t vq_fit_workspace_size(int format, int64_t n_mats, int64_t rows, int64_t cols) {
  if (!fmt_ok(format) || n_mats < 1 || check_shape(rows, cols, false) != VQ_OK) return 0;
  const uint64_t n = (uint64_t)n_mats * (uint64_t)rows * (uint64_t)(cols / 8);
  if (n >= (1ull << 32)) return 0;
  return fit_layout(format, (int64_t)n).total;
}

int vq_fit_codebooks(int format, const void* const* mats, int dtype, int64_t n_mats, int64_t rows, int64_t cols,
                     int32_t iters, const int64_t* init_idx, float* codebooks, void* workspace, size_t ws_bytes,
                     int engine, void* stream) {
  if (!fmt_ok(format) || !dtype_ok(dtype) || engine < VQ_ENGINE_AUTO || engine > VQ_ENGINE_EXACT) return VQ_EINVAL;
  if (n_mats < 1 || iters < 0 || !mats || !init_idx || !codebooks) return VQ_EINVAL;
  int st = check_shape(rows, cols, false);
  if (st != VQ_OK) return st;
  const uint64_t n = (uint64_t)n_mats * (uint64_t)rows * (uint64_t)(cols / 8);
  if (n >= (1ull << 32)) return VQ_ERANGE;
  const int S = stages_of(format), K = entries_of(format);
  if (n < (uint64_t)K) return VQ_EINVAL;
  for (int64_t m = 0; m < n_mats; ++m)
    if (!mats[m] || !aligned(mats[m], 16)) return VQ_EINVAL;
  if (!aligned(codebooks, 16)) return VQ_EINVAL;
  for (int t = 0; t < S; ++t)
    for (int j = 0; j < K; ++j) {
      const int64_t v = init_idx[t * K + j];
      if (v < 0 || (uint64_t)v >= n) return VQ_EINVAL;
      for (int q = 0; q < j; ++q)
        if (init_idx[t * K + q] == v) return VQ_EINVAL;
    }
  const FitLayout L = fit_layout(format, (int64_t)n);
  if (!workspace || !aligned(workspace, 256) || ws_bytes < L.total) return VQ_EWORKSPACE;
  int ncu = 0;
  if ((st = device_cus(&ncu)) != VQ_OK) return st;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  // the initial indices travel through the workspace; the copy is complete
  // (staged) when hipMemcpyAsync returns for pageable host memory
  if (hipMemcpyAsync(ws + L.init, init_idx, sizeof(int64_t) * S * K, hipMemcpyHostToDevice, s) != hipSuccess)
    return VQ_EDEVICE;
  FitArgs a;
  a.format = format;
  a.engine = (engine == VQ_ENGINE_AUTO) ? ENGINE_F16X : engine;
  if (a.engine == ENGINE_EXACT) a.engine = ENGINE_F16X;  // the fit's exact pass already covers every flagged vector
  a.dtype = dtype;
  a.mats = mats;
  a.n_mats = n_mats;
  a.rows = rows;
  a.cols = cols;
  a.n = (int64_t)n;
  a.iters = iters;
  int c = 0;
  while ((1ull << c) < n) ++c;
  a.clog2n = c;
  a.init = (const int64_t*)(ws + L.init);
  a.codebooks = codebooks;
  a.hdr = (WsHeader*)ws;
  a.R[0] = (float*)(ws + L.r0);
  a.R[1] = (float*)(ws + L.r1);
  a.list = (uint32_t*)(ws + L.list);
  a.cap = L.cap;
  a.partials = (long long*)(ws + L.partials);
  a.n_assign_blocks = L.ga;
  a.n_exact_blocks = L.gf;
  a.ncu = ncu;
  a.stream = s;
  return hip_status(launch_fit(a));
}

int vq_forgy_init(int64_t n_vectors, int32_t entries, int32_t stages, uint64_t seed, int64_t* init_out) {
  if (entries < 1 || stages < 1 || n_vectors < entries || !init_out) return VQ_EINVAL;
  constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
  for (int32_t t = 0; t < stages; ++t) {
    uint64_t x = seed ^ (kGamma * (uint64_t)(t + 1));  // SplitMix64 state of this stage
    std::unordered_set<int64_t> taken;
    int64_t* row = init_out + (int64_t)t * entries;
    for (int32_t have = 0; have < entries;) {
      x += kGamma;
      uint64_t z = x;
      z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
      z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
      z ^= z >> 31;
      const int64_t pick = (int64_t)(uint64_t)(((unsigned __int128)z * (uint64_t)n_vectors) >> 64);
      if (taken.insert(pick).second) row[have++] = pick;
    }
  }
  return VQ_OK;
}

int vq_fit_codebooks_seeded(int format, const void* const* mats, int dtype, int64_t n_mats, int64_t rows,
                            int64_t cols, int32_t iters, uint64_t seed, float* codebooks, void* workspace,
                            size_t ws_bytes, int engine, void* stream) {
  if (!fmt_ok(format) || n_mats < 1 || rows < 1 || cols < 8 || cols % 8 != 0) return VQ_EINVAL;
  if (check_shape(rows, cols, false) != VQ_OK ||
      (uint64_t)n_mats * (uint64_t)rows * (uint64_t)(cols / 8) >= (1ull << 32))
    return VQ_ERANGE;
  const int64_t n = n_mats * rows * (cols / 8);
  const int S = stages_of(format), K = entries_of(format);
  std::vector<int64_t> init((size_t)S * K);
  const int st = vq_forgy_init(n, K, S, seed, init.data());
  if (st != VQ_OK) return st;
  return vq_fit_codebooks(format, mats, dtype, n_mats, rows, cols, iters, init.data(), codebooks, workspace, ws_bytes,
                          engine, stream);
}

// ---------------------------------------------------------------- decode
int vq_decode(int format, const uint8_t* idx, const uint16_t* scales, const float* codebooks, int64_t rows,
              int64_t cols, int32_t stages_used, float* W_out, void* stream) {
  if (!fmt_ok(format)) return VQ_EINVAL;
  int st = check_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (stages_used < 1 || stages_used > stages_of(format)) return VQ_EINVAL;
  if (rows == 0) return VQ_OK;
  if (!idx || !scales || !codebooks || !W_out || !aligned(W_out, 16)) return VQ_EINVAL;
  DecodeArgs a;
  a.format = format;
  a.stages_used = stages_used;
  a.idx = idx;
  a.scales = scales;
  a.codebooks = codebooks;
  a.rows = rows;
  a.cols = cols;
  a.out = W_out;
  a.stream = (hipStream_t)stream;
  if ((st = device_cus(&a.ncu)) != VQ_OK) return st;
  return hip_status(launch_decode(a));
}

int vq3r_decode(const uint8_t* idx, const uint16_t* scales, const float* codebooks, int64_t rows, int64_t cols,
                float* W_out, void* stream) {
  return vq_decode(VQ_FMT_VQ3R, idx, scales, codebooks, rows, cols, 3, W_out, stream);
}

int vq4p_decode(const uint8_t* idx, const uint16_t* scales, const float* codebooks, int64_t rows, int64_t cols,
                float* W_out, void* stream) {
  return vq_decode(VQ_FMT_VQ4P, idx, scales, codebooks, rows, cols, 4, W_out, stream);
}

// ---------------------------------------------------------------- GEMV
size_t vq_gemv_packed_size(int format, int64_t rows, int64_t cols) {
  if (!fmt_ok(format) || check_shape(rows, cols) != VQ_OK) return 0;
  return (size_t)gemv_packed_bytes(format, rows, cols);
}

int vq_gemv_pack(int format, const uint8_t* idx, int64_t rows, int64_t cols, int64_t n_experts, uint8_t* packed,
                 void* stream) {
  if (!fmt_ok(format) || n_experts < 0) return VQ_EINVAL;
  int st = check_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (rows == 0 || n_experts == 0) return VQ_OK;
  if (!idx || !packed || !aligned(packed, 4)) return VQ_EINVAL;
  int ncu = 0;
  if ((st = device_cus(&ncu)) != VQ_OK) return st;
  return hip_status(launch_gemv_pack(format, idx, rows * (cols / 8) * 3, rows, cols, n_experts, nullptr, nullptr,
                                     packed, ncu, (hipStream_t)stream));
}

size_t vq_gemv_packed_workspace_size(int format, int64_t rows, int64_t cols, int32_t ntok, int32_t topk) {
  if (!fmt_ok(format) || check_shape(rows, cols) != VQ_OK || ntok < 0 || topk < 0) return 0;
  return kHeader + gemv_partials_bytes(format, rows, cols, ntok, topk);
}

int vq_dequant_gemv_packed(int format, const uint8_t* packed, int64_t expert_stride, const uint16_t* scales,
                           int64_t scale_stride, const float* codebooks, int64_t rows, int64_t cols,
                           int32_t n_experts, const uint16_t* x, int32_t ntok, const int32_t* route, int32_t topk,
                           float* y, void* workspace, size_t ws_bytes, void* stream) {
  int st = gemv_check(format, rows, cols, n_experts, expert_stride,
                      fmt_ok(format) ? gemv_packed_bytes(format, rows, cols) : 0, scale_stride, ntok, topk, packed,
                      scales, codebooks, x, route, y);
  if (st != VQ_OK) return st;
  if (expert_stride % 4 != 0 || !aligned(packed, 4)) return VQ_EINVAL;
  if (!workspace || !aligned(workspace, 256) ||
      ws_bytes < vq_gemv_packed_workspace_size(format, rows, cols, ntok, topk))
    return VQ_EWORKSPACE;
  GemvArgs a;
  gemv_fill(a, format, scales, scale_stride, codebooks, rows, cols, n_experts, x, ntok, route, topk, y, workspace,
            (hipStream_t)stream);
  a.idx = packed;
  a.expert_stride = expert_stride;
  a.partials = (float*)((char*)workspace + kHeader);
  if ((st = device_cus(&a.ncu)) != VQ_OK) return st;
  return hip_status(launch_gemv(a));
}

int vq_dequant_gemv_packed_noalloc(int format, const uint8_t* packed, int64_t expert_stride, const uint16_t* scales,
                                   int64_t scale_stride, const float* codebooks, int64_t rows, int64_t cols,
                                   int32_t n_experts, const uint16_t* x, int32_t ntok, const int32_t* route,
                                   int32_t topk, float* y, void* status, void* stream) {
  int st = gemv_check(format, rows, cols, n_experts, expert_stride,
                      fmt_ok(format) ? gemv_packed_bytes(format, rows, cols) : 0, scale_stride, ntok, topk, packed,
                      scales, codebooks, x, route, y);
  if (st != VQ_OK) return st;
  if (expert_stride % 4 != 0 || !aligned(packed, 4)) return VQ_EINVAL;
  if (status && !aligned(status, 256)) return VQ_EINVAL;
  GemvArgs a;
  if ((st = device_cus(&a.ncu)) != VQ_OK) return st;
  const size_t need =
      kHeader + sizeof(float) * (size_t)gemv_partials_floats_used(format, rows, cols, (int64_t)ntok * topk, a.ncu);
  if (need > (size_t)VQ_NOALLOC_SCRATCH_BYTES) return VQ_ESCRATCH;
  void* base = nullptr;
  if ((st = scratch_base(&base)) != VQ_OK) return st;
  gemv_fill(a, format, scales, scale_stride, codebooks, rows, cols, n_experts, x, ntok, route, topk, y,
            status ? status : base, (hipStream_t)stream);
  a.idx = packed;
  a.expert_stride = expert_stride;
  a.partials = (float*)((char*)base + kHeader);
  return hip_status(launch_gemv(a));
}

size_t vq_gemv_workspace_size(int format, int64_t rows, int64_t cols, int32_t ntok, int32_t topk,
                              int32_t n_experts) {
  if (!fmt_ok(format) || check_shape(rows, cols) != VQ_OK || ntok < 0 || topk < 0 || n_experts < 1) return 0;
  return gemv_stored_layout(format, rows, cols, ntok, topk, n_experts).total;
}

int vq_dequant_gemv(int format, const uint8_t* idx, int64_t expert_stride, const uint16_t* scales,
                    int64_t scale_stride, const float* codebooks, int64_t rows, int64_t cols, int32_t n_experts,
                    const uint16_t* x, int32_t ntok, const int32_t* route, int32_t topk, float* y, void* workspace,
                    size_t ws_bytes, void* stream) {
  int st = gemv_check(format, rows, cols, n_experts, expert_stride, rows * (cols / 8) * 3, scale_stride, ntok, topk,
                      idx, scales, codebooks, x, route, y);
  if (st != VQ_OK) return st;
  if (!workspace || !aligned(workspace, 256) ||
      ws_bytes < vq_gemv_workspace_size(format, rows, cols, ntok, topk, n_experts))
    return VQ_EWORKSPACE;
  const GemvStoredLayout L = gemv_stored_layout(format, rows, cols, ntok, topk, n_experts);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  GemvArgs a;
  gemv_fill(a, format, scales, scale_stride, codebooks, rows, cols, n_experts, x, ntok, route, topk, y, workspace, s);
  if ((st = device_cus(&a.ncu)) != VQ_OK) return st;
  const int npairs = ntok * topk;
  if (npairs > 0 && rows > 0) {
    int32_t* slot = (int32_t*)(ws + L.slot);
    int32_t* list = (int32_t*)(ws + L.list);
    int32_t* count = (int32_t*)(ws + L.count);
    uint8_t* packed = (uint8_t*)(ws + L.packed);
    hipError_t e = launch_gemv_route_stored(route, npairs, n_experts, (int32_t*)(ws + L.mark), slot, list, count, s);
    if (e == hipSuccess)
      e = launch_gemv_pack(format, idx, expert_stride, rows, cols, L.n_slots, list, count, packed, a.ncu, s);
    if (e != hipSuccess) return VQ_EDEVICE;
    a.idx = packed;
    a.expert_stride = gemv_packed_bytes(format, rows, cols);
    a.remap = slot;
  } else {
    a.idx = idx;
    a.expert_stride = 0;
  }
  a.partials = (float*)(ws + L.partials);
  return hip_status(launch_gemv(a));
}

int vq3r_dequant_gemv(const uint8_t* idx, int64_t expert_stride, const uint16_t* scales, int64_t scale_stride,
                      const float* codebooks, int64_t rows, int64_t cols, int32_t n_experts, const uint16_t* x,
                      int32_t ntok, const int32_t* route, int32_t topk, float* y, void* workspace, size_t ws_bytes,
                      void* stream) {
  return vq_dequant_gemv(VQ_FMT_VQ3R, idx, expert_stride, scales, scale_stride, codebooks, rows, cols, n_experts, x,
                         ntok, route, topk, y, workspace, ws_bytes, stream);
}

int vq4p_dequant_gemv(const uint8_t* idx, int64_t expert_stride, const uint16_t* scales, int64_t scale_stride,
                      const float* codebooks, int64_t rows, int64_t cols, int32_t n_experts, const uint16_t* x,
                      int32_t ntok, const int32_t* route, int32_t topk, float* y, void* workspace, size_t ws_bytes,
                      void* stream) {
  return vq_dequant_gemv(VQ_FMT_VQ4P, idx, expert_stride, scales, scale_stride, codebooks, rows, cols, n_experts, x,
                         ntok, route, topk, y, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------- dequant-GEMM
size_t vq_dequant_gemm_workspace_size(int format, int32_t n_experts, int32_t ntok, int32_t topk) {
  if (!fmt_ok(format) || n_experts < 1 || ntok < 0 || topk < 0) return 0;
  const int64_t npairs = (int64_t)ntok * topk;
  if (npairs >= ((int64_t)1 << 31)) return 0;
  return align256(vqk::gemm_layout(n_experts, npairs).total);
}

int vq_dequant_gemm(int format, const uint8_t* idx, int64_t expert_stride, const uint16_t* scales,
                    int64_t scale_stride, const float* codebooks, int64_t rows, int64_t cols, int32_t n_experts,
                    const uint16_t* x, int32_t ntok, const int32_t* route, int32_t topk, float* y, void* workspace,
                    size_t ws_bytes, void* stream) {
  if (!fmt_ok(format)) return VQ_EINVAL;
  int st = check_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (ntok < 0 || topk < 0 || n_experts < 1 || expert_stride < 0 || scale_stride < 0) return VQ_EINVAL;
  if (n_experts > 1 && (expert_stride < rows * (cols / 8) * 3 || scale_stride < rows)) return VQ_EINVAL;
  const int64_t npairs = (int64_t)ntok * topk;
  if (!idx || !scales || !codebooks) return VQ_EINVAL;
  if (npairs > 0 && (!x || !route || !y || !aligned(x, 16))) return VQ_EINVAL;
  if (npairs >= ((int64_t)1 << 31) || (rows + 255) / 256 > 65535) return VQ_ERANGE;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < vq_dequant_gemm_workspace_size(format, n_experts, ntok, topk))
    return VQ_EWORKSPACE;
  vqk::GemmArgs a;
  a.format = format;
  a.idx = idx;
  a.expert_stride = expert_stride;
  a.scales = scales;
  a.scale_stride = scale_stride;
  a.codebooks = codebooks;
  a.rows = rows;
  a.cols = cols;
  a.n_experts = n_experts;
  a.x = x;
  a.ntok = ntok;
  a.topk = topk;
  a.route = route;
  a.y = y;
  a.hdr = (WsHeader*)workspace;
  a.ws = (char*)workspace;
  a.L = vqk::gemm_layout(n_experts, npairs);
  a.stream = (hipStream_t)stream;
  return hip_status(vqk::launch_gemm(a));
}

// ---------------------------------------------------------------- Tied Trit-Planes
static int ttp_shape(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0 || cols % TTP_GROUP != 0) return VQ_EINVAL;
  if (cols > (1 << 20) || rows > ((int64_t)1 << 40) / cols) return VQ_ERANGE;
  return VQ_OK;
}

int vq_ttp_quantize(const void* W, int dtype, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* scales,
                    void* workspace, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype)) return VQ_EINVAL;
  int st = ttp_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (rows == 0) return VQ_OK;
  if (!W || !codes || !scales || !aligned(W, 16) || !aligned(codes, 4)) return VQ_EINVAL;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < kHeader) return VQ_EWORKSPACE;
  int ncu = 0;
  if ((st = device_cus(&ncu)) != VQ_OK) return st;
  return hip_status(launch_ttp_quantize(W, dtype, rows * (cols / TTP_GROUP), codes, scales, (WsHeader*)workspace,
                                        ncu, (hipStream_t)stream));
}

int vq_ttp_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t cols, float* out,
                      void* stream) {
  int st = ttp_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (rows == 0) return VQ_OK;
  if (!codes || !scales || !out || !aligned(codes, 4) || !aligned(out, 16)) return VQ_EINVAL;
  int ncu = 0;
  if ((st = device_cus(&ncu)) != VQ_OK) return st;
  return hip_status(launch_ttp_dequantize(codes, scales, rows * (cols / TTP_GROUP), out, ncu, (hipStream_t)stream));
}

size_t vq_ttp_error_workspace_size(int64_t n_mats, int64_t rows, int64_t cols) {
  if (n_mats < 1 || ttp_shape(rows, cols) != VQ_OK) return 0;
  const int64_t chunks = (rows * (cols / TTP_GROUP) + TTP_CHUNK - 1) / TTP_CHUNK;
  return align256(kHeader + sizeof(double) * 2 * (size_t)n_mats * (size_t)chunks);
}

int vq_ttp_error(const void* W, int dtype, const uint8_t* codes, const uint16_t* scales, int64_t n_mats,
                 int64_t rows, int64_t cols, double* sums, void* workspace, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || n_mats < 1) return VQ_EINVAL;
  int st = ttp_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (n_mats > 65535 || (rows * (cols / TTP_GROUP) + TTP_CHUNK - 1) / TTP_CHUNK > 0x7FFFFFFF) return VQ_ERANGE;
  if (!sums || (rows > 0 && (!W || !codes || !scales || !aligned(W, 16) || !aligned(codes, 4)))) return VQ_EINVAL;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < vq_ttp_error_workspace_size(n_mats, rows, cols))
    return VQ_EWORKSPACE;
  return hip_status(launch_ttp_error(W, dtype, codes, scales, rows * (cols / TTP_GROUP), n_mats,
                                     (double*)((char*)workspace + kHeader), sums, (WsHeader*)workspace,
                                     (hipStream_t)stream));
}

// ---------------------------------------------------------------- error
size_t vq_error_workspace_size(int format, int64_t n_mats, int64_t rows, int64_t cols) {
  if (!fmt_ok(format) || n_mats < 1 || check_shape(rows, cols) != VQ_OK) return 0;
  return error_ws_bytes(format, n_mats, rows);
}

int vq_error(int format, const void* W, int dtype, const uint8_t* idx, const uint16_t* scales, const float* codebooks,
             int64_t n_mats, int64_t rows, int64_t cols, double* sums, double* rel, double* rel_all, void* workspace,
             size_t ws_bytes, void* stream) {
  if (!fmt_ok(format) || !dtype_ok(dtype) || n_mats < 1) return VQ_EINVAL;
  int st = check_shape(rows, cols);
  if (st != VQ_OK) return st;
  if (n_mats > 65535) return VQ_ERANGE;
  if (!W || !idx || !scales || !codebooks || !sums || !aligned(W, 16)) return VQ_EINVAL;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < error_ws_bytes(format, n_mats, rows)) return VQ_EWORKSPACE;
  const int blocks = error_blocks(rows, n_mats);
  ErrorArgs a;
  a.format = format;
  a.dtype = dtype;
  a.W = W;
  a.idx = idx;
  a.scales = scales;
  a.codebooks = codebooks;
  a.n_mats = n_mats;
  a.rows = rows;
  a.cols = cols;
  a.sums = sums;
  a.rel = rel;
  a.rel_all = rel_all;
  a.partials = (double*)((char*)workspace + kHeader);
  a.blocks = blocks;
  a.hdr = (WsHeader*)workspace;
  a.stream = (hipStream_t)stream;
  return hip_status(launch_error(a));
}

// ---------------------------------------------------------------- MXFP4
static int mxfp4_qdq(const void* W, int dtype, int64_t rows, int64_t cols, void* out, int out_bf16, void* workspace,
                     size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || rows < 0 || cols <= 0 || cols % 32 != 0) return VQ_EINVAL;
  if (!W || !out) return VQ_EINVAL;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < kHeader) return VQ_EWORKSPACE;
  Mxfp4Args a;
  a.dtype = dtype;
  a.W = W;
  a.rows = rows;
  a.cols = cols;
  a.out = out;
  a.out_bf16 = out_bf16;
  a.hdr = (WsHeader*)workspace;
  a.stream = (hipStream_t)stream;
  int st;
  if ((st = device_cus(&a.ncu)) != VQ_OK) return st;
  return hip_status(launch_mxfp4(a));
}

int vq_mxfp4_qdq(const void* W, int dtype, int64_t rows, int64_t cols, float* out, void* workspace, size_t ws_bytes,
                 void* stream) {
  return mxfp4_qdq(W, dtype, rows, cols, out, 0, workspace, ws_bytes, stream);
}

int vq_mxfp4_qdq_bf16(const void* W, int dtype, int64_t rows, int64_t cols, uint16_t* out, void* workspace,
                      size_t ws_bytes, void* stream) {
  return mxfp4_qdq(W, dtype, rows, cols, out, 1, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------- read reference
int vq_stream_read(const void* src, size_t nbytes, uint32_t* out, void* stream) {
  if (nbytes == 0) return VQ_OK;
  if (!src || !out || !aligned(src, 16) || nbytes % 16 != 0) return VQ_EINVAL;
  int ncu = 0, st;
  if ((st = device_cus(&ncu)) != VQ_OK) return st;
  return hip_status(launch_stream_read(src, nbytes, out, ncu, (hipStream_t)stream));
}

}  // extern "C"
