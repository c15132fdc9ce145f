/*
 * vq.h - C ABI of libvq, residual vector quantization (VQ3R and VQ4P) of
 * Mixture-of-Experts expert weights on AMD Instinct MI355X (gfx950).
 *
 * The operations follow the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验"
 * (xdnf.cn), cited as [VQ3R page] with its section numbers:
 *   §2  VQ3R: each weight row gets one FP16 scale; the row is cut into 8-dim
 *       vectors; 3 stages, each a 256-entry codebook with an 8-bit index;
 *       W ~ scale * (C1[i1] + C2[i2] + C3[i3]) at exactly 3.00 bits/weight;
 *       C1 fits the vector, C2 the stage-1 residual, C3 the stage-2 residual;
 *       per-layer codebooks are fit with k-means (Lloyd) on sampled experts.
 *   §3  the relative Frobenius error ||W - W_hat||_F / ||W||_F; MXFP4 experts.
 *   §4  the encoder keeps all 256 distances and writes only the winning index.
 *   §5  VQ4P: 4 stages x 64 entries, 6-bit indices packed in the same bytes.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument that names tensor data is a DEVICE pointer owned
 *     by the caller, unless marked "host". The library never allocates memory:
 *     scratch space is passed in as `workspace` (device memory of at least the
 *     size the matching *_workspace_size() returns, 256-byte aligned).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *     stream) and is asynchronous; the call returns after validating its
 *     arguments and launching.
 *   - Return value: a vq_status. Argument checks happen on the host before any
 *     launch; on error nothing is launched and no output is touched.
 *   - Data errors detected on the device (a non-finite weight, a row RMS beyond
 *     the fp16 range, a codebook entry that is non-finite or larger than 2048 in
 *     magnitude, a GEMV route id out of range) set a flag in the workspace;
 *     vq_read_status() returns it. Outputs of a flagged call are unspecified.
 *   - Layouts (row-major throughout):
 *       weights     [rows][cols] of vq_dtype; cols % 8 == 0
 *       codebooks   fp32 [stages][entries][8]; VQ3R 3 x 256, VQ4P 4 x 64
 *       scales      fp16 bit patterns, one per row
 *       idx         3 bytes per 8-dim vector, [rows][cols/8][3]; the 3 bytes
 *                   are a little-endian 24-bit word sum_t i_t << (t * b) with
 *                   b = 8 (VQ3R: byte t is stage t's index) or b = 6 (VQ4P).
 *   - Limits: 1 <= cols/8, cols <= 2^20, rows * cols / 8 < 2^32 per call.
 *   - Calls on one stream are ordered; the library keeps no global state, so
 *     calls on different streams with different workspaces may overlap.
 */
#ifndef VQ_H
#define VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vq_status {
  VQ_OK = 0,
  VQ_EINVAL = 1,     /* invalid argument (null pointer, bad size, bad enum) */
  VQ_ERANGE = 2,     /* size beyond the supported range */
  VQ_EWORKSPACE = 3, /* workspace missing, misaligned or too small */
  VQ_EDEVICE = 4,    /* a HIP runtime call failed */
  VQ_EDATA = 5,      /* the device flagged a data error (vq_read_status) */
  VQ_EIO = 6,        /* container file: open, read or write failed or was short */
  VQ_EFORMAT = 7,    /* container file: bad header, checksum mismatch, missing record */
  VQ_ESCRATCH = 8    /* call too large for the fixed scratch of the no-allocation entry point */
} vq_status;

typedef enum vq_dtype { VQ_DT_F32 = 0, VQ_DT_BF16 = 1, VQ_DT_F16 = 2 } vq_dtype;

/* VQ3R = 3 stages x 256 entries, 8-bit indices ([VQ3R page] §2);
 * VQ4P = 4 stages x 64 entries, 6-bit packed indices ([VQ3R page] §5). */
typedef enum vq_format { VQ_FMT_VQ3R = 0, VQ_FMT_VQ4P = 1 } vq_format;

/* How the approximate codeword scores of the encoder / Lloyd assignment are
 * computed before the exact check (all engines give identical indices):
 *   MFMA_F16X  fp32 values split into two fp16 halves, fp16 matrix cores
 *   MFMA_F32   fp32 matrix cores (v_mfma_f32_32x32x2_f32)
 *   VALU_F32   fp32 vector FMAs
 *   EXACT      no fast scoring: every vector goes through the exact search
 * AUTO picks the fastest measured engine (MFMA_F16X). */
typedef enum vq_engine {
  VQ_ENGINE_AUTO = 0,
  VQ_ENGINE_MFMA_F16X = 1,
  VQ_ENGINE_MFMA_F32 = 2,
  VQ_ENGINE_VALU_F32 = 3,
  VQ_ENGINE_EXACT = 4
} vq_engine;

/* Human-readable name of a vq_status. Never NULL. */
const char* vq_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
int vq_version(void);

/* Waits for `stream`, then returns VQ_EDATA if the most recent call that used
 * `workspace` flagged a data error, else VQ_OK (every call that takes a
 * workspace clears its flags when it starts). *flags_out (host, may be NULL)
 * receives the raw flag bits (bit 8 is informational: the exact search covered
 * every vector because its queue overflowed). */
int vq_read_status(const void* workspace, void* stream, uint32_t* flags_out);

/* The same without the raw bits: VQ_EDATA if the last call on `workspace`
 * flagged a data error, else VQ_OK (waits for `stream`). */
int vq_read_device_status(const void* workspace, void* stream);

/* Enqueues a reset of the workspace's status flags. */
int vq_clear_status(void* workspace, void* stream);

/* ------------------------------------------------------------------------
 * Codebook fit ([VQ3R page] §2 and §4: per-layer codebooks fit with Lloyd
 * k-means on sampled experts; C1 on the vectors, C2 on the stage-1 residuals,
 * C3 on the stage-2 residuals).
 *
 * mats      host array of n_mats device pointers, each a [rows][cols] matrix
 *           of `dtype`; every row is normalized by its own fp16 RMS scale and
 *           cut into 8-dim vectors, giving N = n_mats*rows*cols/8 training
 *           vectors ordered matrix, row, vector.
 * iters     Lloyd iterations per stage (>= 0); one iteration = nearest-codeword
 *           assignment + centroid update.
 * init_idx  host int64 [stages][entries]: per stage, distinct training-vector
 *           indices in [0, N) whose (residual) vectors are the initial
 *           centroids (Forgy initialization; the caller draws them).
 * codebooks out: fp32 [stages][entries][8].
 * Centroids are cluster means computed from exact int64 fixed-point sums
 * (F = 62 - e - ceil(log2 N) fraction bits, max|r| < 2^e); an empty cluster
 * keeps its centroid. The result is bit-identical for any engine and launch
 * configuration. Requires N >= entries.
 * Workspace: vq_fit_workspace_size(format, n_mats, rows, cols).
 * ---------------------------------------------------------------------- */
size_t vq_fit_workspace_size(int format, int64_t n_mats, int64_t rows, int64_t cols);
int vq_fit_codebooks(int format, const void* const* mats, int dtype, int64_t n_mats, int64_t rows,
                     int64_t cols, int32_t iters, const int64_t* init_idx, float* codebooks,
                     void* workspace, size_t ws_bytes, int engine, void* stream);

/* Seeded Forgy initialization (the configurations' "seeded random vectors";
 * the page names no generator, the reading taken): for stage t (0-based), a
 * SplitMix64 stream (Steele, Lea and Flood, 2014) whose state starts at
 * seed XOR (0x9E3779B97F4A7C15 * (t + 1)) mod 2^64; each output d picks
 * training vector floor(d * n_vectors / 2^64), and a pick already taken for the
 * stage is skipped until `entries` distinct vectors are chosen.
 * init_out: host int64 [stages][entries]. Host-only (no device work); returns
 * VQ_EINVAL when n_vectors < entries or a count is not positive. */
int vq_forgy_init(int64_t n_vectors, int32_t entries, int32_t stages, uint64_t seed, int64_t* init_out);

/* vq_fit_codebooks started from vq_forgy_init(N, entries, stages, seed), N the
 * training-vector count (the call draws the indices on the host). */
int vq_fit_codebooks_seeded(int format, const void* const* mats, int dtype, int64_t n_mats, int64_t rows,
                            int64_t cols, int32_t iters, uint64_t seed, float* codebooks, void* workspace,
                            size_t ws_bytes, int engine, void* stream);

/* ------------------------------------------------------------------------
 * Encode ([VQ3R page] §2 and §4): per row the fp16 scale s = fp16(RMS(row));
 * every vector v = w[8j..8j+7] / s is encoded greedily: for each stage t,
 * i_t = argmin_j ||r - C_t[j]||^2 over the stage's entries (fp32 distance
 * evaluated as sum_k fma(e_k, e_k) in k order, ties to the lowest index),
 * then r <- r - C_t[i_t]. Writes idx and scales. Indices equal those of that
 * exhaustive search exactly; near ties are resolved by the exact evaluation.
 * W         [rows][cols] of dtype;  codebooks fp32 [stages][entries][8]
 * idx       out [rows][cols/8][3];  scales out fp16 bits [rows]
 * Workspace: vq_encode_workspace_size(format, rows, cols).
 * vq_encode selects format and engine; vq3r_encode / vq4p_encode use AUTO.
 * ---------------------------------------------------------------------- */
size_t vq_encode_workspace_size(int format, int64_t rows, int64_t cols);
int vq_encode(int format, int engine, const void* W, int dtype, int64_t rows, int64_t cols,
              const float* codebooks, uint8_t* idx, uint16_t* scales, void* workspace, size_t ws_bytes,
              void* stream);
int vq3r_encode(const void* W, int dtype, int64_t rows, int64_t cols, const float* codebooks, uint8_t* idx,
                uint16_t* scales, void* workspace, size_t ws_bytes, void* stream);
int vq4p_encode(const void* W, int dtype, int64_t rows, int64_t cols, const float* codebooks, uint8_t* idx,
                uint16_t* scales, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode ([VQ3R page] §2, and the container round-trip check of §4):
 * W_out[r][8j+k] = s_r * (((C1[i1][k] + C2[i2][k]) + C3[i3][k]) [+ C4[i4][k]]),
 * summed left to right in fp32, then one fp32 multiply. stages_used < stages
 * gives the partial reconstruction after that many stages (e.g. 2 = "vq2").
 * W_out fp32 [rows][cols], 16-byte aligned (VQ_EINVAL otherwise). No workspace;
 * cannot fail on the device.
 * ---------------------------------------------------------------------- */
int vq_decode(int format, const uint8_t* idx, const uint16_t* scales, const float* codebooks, int64_t rows,
              int64_t cols, int32_t stages_used, float* W_out, void* stream);
int vq3r_decode(const uint8_t* idx, const uint16_t* scales, const float* codebooks, int64_t rows, int64_t cols,
                float* W_out, void* stream);
int vq4p_decode(const uint8_t* idx, const uint16_t* scales, const float* codebooks, int64_t rows, int64_t cols,
                float* W_out, void* stream);

/* ------------------------------------------------------------------------
 * Fused dequantize-GEMV for decode-time expert mat-vecs ([VQ3R page] §1:
 * each token activates a few experts whose stored records are decoded and
 * multiplied): for token b and routed slot k with e = route[b][k],
 *   y[b][k][r] = sum_c W_hat_e[r][c] * x[b][c]   (fp32 accumulation)
 * computed from the indices without materializing W_hat. The result is
 * deterministic (fixed summation order) and within fp32 rounding of the
 * decoded product.
 *
 * Two entry points, same result:
 *   vq_dequant_gemv / vq3r_dequant_gemv / vq4p_dequant_gemv read the stored
 *     records ([rows][cols/8][3], as vq_encode writes them). Each call lists
 *     the distinct routed experts on the device, copies just those into the
 *     workspace in the GEMV layout below, and runs the GEMV on the copies
 *     (about three times the record traffic of the packed call).
 *   vq_dequant_gemv_packed reads experts already in the GEMV layout, built
 *     once with vq_gemv_pack (like loading a container into memory): the path
 *     for repeated decode steps.
 * GEMV layout: blocks of 16 column slices by 64-row groups, each group's
 * records interleaved in 12-byte chunks of 4 records per row and each row's
 * slices rotated by its position in the group; vq_gemv_packed_size() gives the
 * bytes of one packed expert (rows padded to a multiple of 64 and slices to a
 * multiple of 16 with zeros).
 *
 * Arguments of both:
 * idx / packed  base of the experts; expert e at base + e*expert_stride bytes
 *            (stored: expert_stride >= rows*cols/8*3; packed: >=
 *            vq_gemv_packed_size and a multiple of 4; both when n_experts > 1)
 * scales     base of the row scales; expert e at scales + e*scale_stride
 * n_experts  number of experts behind the bases: a route id outside
 *            [0, n_experts) gives y = 0 for that slot and flags a data error
 *            (no expert is read out of bounds)
 * x          fp16 bit patterns [ntok][cols];  route int32 [ntok][topk]
 * y          out fp32 [ntok][topk][rows]
 * ntok * topk < 65536.
 * Workspace: vq_gemv_workspace_size(format, rows, cols, ntok, topk, n_experts)
 * for the stored call (it holds the packed copies of up to
 * min(ntok*topk, n_experts) experts), vq_gemv_packed_workspace_size(...) for
 * the packed call.
 *
 * vq_gemv_pack: idx = n_experts consecutive [rows][cols/8][3] tensors;
 *               packed out = n_experts consecutive packed experts of
 *               vq_gemv_packed_size() bytes each (4-byte aligned).
 * ---------------------------------------------------------------------- */
size_t vq_gemv_workspace_size(int format, int64_t rows, int64_t cols, int32_t ntok, int32_t topk,
                              int32_t n_experts);
int vq_dequant_gemv(int format, const uint8_t* idx, int64_t expert_stride, const uint16_t* scales,
                    int64_t scale_stride, const float* codebooks, int64_t rows, int64_t cols, int32_t n_experts,
                    const uint16_t* x, int32_t ntok, const int32_t* route, int32_t topk, float* y,
                    void* workspace, size_t ws_bytes, void* stream);
int vq3r_dequant_gemv(const uint8_t* idx, int64_t expert_stride, const uint16_t* scales, int64_t scale_stride,
                      const float* codebooks, int64_t rows, int64_t cols, int32_t n_experts, const uint16_t* x,
                      int32_t ntok, const int32_t* route, int32_t topk, float* y, void* workspace, size_t ws_bytes,
                      void* stream);
int vq4p_dequant_gemv(const uint8_t* idx, int64_t expert_stride, const uint16_t* scales, int64_t scale_stride,
                      const float* codebooks, int64_t rows, int64_t cols, int32_t n_experts, const uint16_t* x,
                      int32_t ntok, const int32_t* route, int32_t topk, float* y, void* workspace, size_t ws_bytes,
                      void* stream);
size_t vq_gemv_packed_size(int format, int64_t rows, int64_t cols);
int vq_gemv_pack(int format, const uint8_t* idx, int64_t rows, int64_t cols, int64_t n_experts, uint8_t* packed,
                 void* stream);
size_t vq_gemv_packed_workspace_size(int format, int64_t rows, int64_t cols, int32_t ntok, int32_t topk);
int vq_dequant_gemv_packed(int format, const uint8_t* packed, int64_t expert_stride, const uint16_t* scales,
                           int64_t scale_stride, const float* codebooks, int64_t rows, int64_t cols,
                           int32_t n_experts, const uint16_t* x, int32_t ntok, const int32_t* route, int32_t topk,
                           float* y, void* workspace, size_t ws_bytes, void* stream);

/* vq_dequant_gemv_packed without a workspace, for callers that cannot
 * allocate device memory (code under stream capture, serving loops that keep
 * a fixed memory footprint). Same arguments, result and kernels as
 * vq_dequant_gemv_packed; its partial sums live in a static device array of
 * VQ_NOALLOC_SCRATCH_BYTES that each GPU holds from the first call until the
 * process ends. The call allocates nothing.
 *   status  optional device buffer (256-byte aligned, >= 4 bytes) that
 *           receives the call's status word, readable with vq_read_status;
 *           NULL: the word stays in the scratch
 * Returns VQ_ESCRATCH (nothing launched) when the call's partial sums
 * (ntok*topk * ranges * rows floats, the ranges chosen from the device's
 * compute units, about 2 per compute unit over the pairs) do not fit, e.g.
 * beyond about 2048 pairs at 2048 rows. All calls on one GPU share its array:
 * calls that overlap in time on that GPU (other streams, other threads) race
 * and give wrong results; serialize them. */
#define VQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int vq_dequant_gemv_packed_noalloc(int format, const uint8_t* packed, int64_t expert_stride, const uint16_t* scales,
                                   int64_t scale_stride, const float* codebooks, int64_t rows, int64_t cols,
                                   int32_t n_experts, const uint16_t* x, int32_t ntok, const int32_t* route,
                                   int32_t topk, float* y, void* status, void* stream);

/* ------------------------------------------------------------------------
 * Batched dequantize-GEMM for prompt processing ([VQ3R page] §1: every token
 * reads its routed experts; §2/§5: the weights are w_hat = s * sum_t C_t[i_t]),
 * for many tokens per expert:
 *   y[b][k][r] = sum_c w_hat_{route[b][k]}[r][c] * x[b][c]
 * computed from the stored records (no decoded weights in memory). The pairs
 * (b, k) are grouped by expert on the device; each tile of up to 256 pairs of
 * one expert x 256 rows runs on fp16 matrix cores with fp32 accumulation: the
 * codeword sum u = (C1+C2)+C3 (+C4) of each 8-dim vector is formed in fp32 and
 * rounded once to fp16, and the row scale is applied to the fp32 dot product.
 * Hence |y - y_exact| <= 2^-11 * sum_c |w_hat[r][c] x[c]| plus fp32
 * accumulation error.
 *   idx:     [n_experts][rows][cols/8][3] records as vq_encode writes them,
 *            expert e at idx + e * expert_stride bytes (expert_stride >=
 *            rows*cols/8*3 when n_experts > 1);
 *   scales:  fp16 bits, expert e at scales + e * scale_stride (>= rows);
 *   x:       fp16 bits [ntok][cols], 16-byte aligned;
 *   route:   int32 [ntok][topk], expert ids; an id outside [0, n_experts) sets
 *            the data flag and gives y = 0 for that pair;
 *   y:       fp32 [ntok][topk][rows].
 * rows <= 16,776,960 (the row blocks of 256 fill one launch dimension);
 * ntok * topk < 2^31 (x, route and y may be NULL when it is 0).
 * Workspace: vq_dequant_gemm_workspace_size(...).
 * ---------------------------------------------------------------------- */
size_t vq_dequant_gemm_workspace_size(int format, int32_t n_experts, int32_t ntok, int32_t topk);
int vq_dequant_gemm(int format, const uint8_t* idx, int64_t expert_stride, const uint16_t* scales,
                    int64_t scale_stride, const float* codebooks, int64_t rows, int64_t cols, int32_t n_experts,
                    const uint16_t* x, int32_t ntok, const int32_t* route, int32_t topk, float* y, void* workspace,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Tied Trit-Planes 9-level codec, from the page "Новый метод квантования Tied
 * Trit-Planes сжимает DeepSeek-V4 до 4.0625 бит на вес" ([TTP page]; its summary
 * and "what happened" sections): two ternary planes with scales tied by a
 * factor of 3, i.e. w ~ a * q with q = 3 t1 + t2 in -4..4, folded into one 4-bit
 * code, 4.0625 bits per weight. A 4-bit-class baseline beside rtn4-row.
 * Groups of 256 consecutive weights of a row share one fp16 scale a. The
 * quantizer alternates nearest levels q = clamp(rint(w / a), -4, 4) and the
 * least-squares scale a = sum w q / sum q^2 (numerator summed exactly in int64
 * fixed point), from a = max|w| / 4, at most 8 rounds, stopping when no level
 * changes; the stored scale is fp16(a) and the levels are chosen for it.
 *   W:      [rows][cols] of vq_dtype, 16-byte aligned, cols % 256 == 0;
 *   codes:  [rows][cols/2] bytes, code = q + 4, even element in the low
 *           nibble (4-byte aligned);
 *   scales: fp16 bits [rows][cols/256].
 * Data errors (non-finite weight, scale beyond fp16) set the workspace flag.
 * Workspace of vq_ttp_quantize: 256 bytes. vq_ttp_dequantize writes fp32
 * w_hat = a * q (out 16-byte aligned). vq_ttp_error writes, for n_mats
 * consecutive matrices, sums[m] = {sum (w - w_hat)^2, sum w^2} in fp64, with a
 * summation order fixed by the matrix shape.
 * ---------------------------------------------------------------------- */
int vq_ttp_quantize(const void* W, int dtype, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* scales,
                    void* workspace, size_t ws_bytes, void* stream);
int vq_ttp_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t cols, float* out,
                      void* stream);
size_t vq_ttp_error_workspace_size(int64_t n_mats, int64_t rows, int64_t cols);
int vq_ttp_error(const void* W, int dtype, const uint8_t* codes, const uint16_t* scales, int64_t n_mats,
                 int64_t rows, int64_t cols, double* sums, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Reconstruction error ([VQ3R page] §3.1, the Gate-3 metric
 * ||W - W_hat||_F / ||W||_F, also after fewer stages: "vq2" = 2 stages).
 * For n_mats consecutive matrices (matrix m at W + m*rows*cols elements,
 * idx + m*rows*cols/8*3 bytes, scales + m*rows) writes fp64
 * sums[m][t] = sum (w - w_hat_{t+1})^2 for t = 0..stages-1 (w_hat_t = the
 * partial reconstruction after t stages) and sums[m][stages] = sum w^2, and
 * from them the metric itself:
 *   rel[m][t]   = sqrt(sums[m][t] / sums[m][stages])            (per matrix)
 *   rel_all[t]  = sqrt(sum_m sums[m][t] / sum_m sums[m][stages]) (all matrices)
 * (correctly rounded fp64 division and square root; 0 for a zero matrix
 * reconstructed as zeros). sums: device fp64 [n_mats][stages+1]; rel: device
 * fp64 [n_mats][stages] or NULL; rel_all: device fp64 [stages] or NULL. The
 * sums of a matrix are added in an order fixed by its row count (partials per
 * 16-row chunk, added in chunk order), so they are bit-identical whether the
 * matrix is passed alone or together with others.
 * Workspace: vq_error_workspace_size(format, n_mats, rows, cols).
 * ---------------------------------------------------------------------- */
size_t vq_error_workspace_size(int format, int64_t n_mats, int64_t rows, int64_t cols);
int vq_error(int format, const void* W, int dtype, const uint8_t* idx, const uint16_t* scales,
             const float* codebooks, int64_t n_mats, int64_t rows, int64_t cols, double* sums, double* rel,
             double* rel_all, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * MXFP4 quantize-dequantize of a [rows][cols] matrix (the MXFP4 source format
 * of the K3 experts, [VQ3R page] §3.2; the format is the OCP Microscaling v1.0
 * definition): blocks of 32 along the row share X = 2^(floor(log2 amax) - 2)
 * (E8M0, clamped to 2^-127..2^127); elements are E2M1(w / X) rounded to nearest
 * even and saturated at 6; out = X * e2m1 in fp32 (zero blocks give zeros).
 * cols % 32 == 0. Workspace: 256 bytes (status flags).
 * ---------------------------------------------------------------------- */
int vq_mxfp4_qdq(const void* W, int dtype, int64_t rows, int64_t cols, float* out, void* workspace,
                 size_t ws_bytes, void* stream);

/* The same quantize-dequantize with the result stored as bf16 (out: device
 * uint16 [rows][cols], each word the upper half of the fp32 result above).
 * The format makes this exact: every result X * e2m1 has at most two
 * significant bits and, for finite input, lies in [2^-128, 1.5 * 2^127]
 * (X <= 2^125), so its fp32 bits end in 16 zero bits (2^-128 and 3 * 2^-128
 * are bf16 subnormals). A consumer that reads the MXFP4 source as bf16 gets the
 * same values from half the bytes. Arguments, workspace and errors as
 * vq_mxfp4_qdq. */
int vq_mxfp4_qdq_bf16(const void* W, int dtype, int64_t rows, int64_t cols, uint16_t* out, void* workspace,
                      size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Bandwidth reference (a measurement helper, not a step of the method): a plain
 * coalesced streaming read of nbytes (a multiple of 16; src 16-byte aligned),
 * the read floor that the dequant-GEMV's HBM rate is compared with. out: one
 * device uint32, written only for data whose XOR of all 32-bit words equals
 * 0x9E3779B9 (the read cannot be skipped).
 * ---------------------------------------------------------------------- */
int vq_stream_read(const void* src, size_t nbytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VQ_H */
