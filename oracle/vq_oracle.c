/*
 * CPU oracle for VQ3R / VQ4P residual vector quantization.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library. The product path never calls it.
 *
 * A plain, sequential, obviously-correct statement of what the method computes,
 * written from the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验"
 * (xdnf.cn; cited below as [VQ3R page]) and its sections:
 *   §2  the VQ3R recipe: 3 stages, 256-entry codebooks, 8-bit indices, 8-dim
 *       vectors, one FP16 scale per row; W ~ scale * (C1[i1] + C2[i2] + C3[i3]);
 *       C1 fits the vector, C2 the stage-1 residual, C3 the stage-2 residual;
 *       codebooks fit per layer with Lloyd k-means on sampled experts.
 *   §4  the encoder keeps all 256 distances, holds an 8 KB (fp32) codebook and
 *       writes only the winning index per stage.
 *   §5  VQ4P: 4 stages x 64 entries, 6-bit indices packed into the same bytes.
 * Where the page is silent, each function below states the reading it takes.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math), so
 * every fp32 operation is a single IEEE round-to-nearest-even operation and
 * fmaf() is the correctly rounded fused multiply-add.
 * OpenMP only splits independent rows / vectors; results do not depend on the
 * thread count (the Lloyd sums are exact integers).
 *
 * Status codes: 0 ok, 1 invalid argument, 5 data error (non-finite weight,
 * row RMS beyond the fp16 range, fixed-point range too small).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define VQO_OK 0
#define VQO_EINVAL 1
#define VQO_EDATA 5
#define DIM 8

/* ------------------------------------------------------------------------
 * IEEE 754 binary16 conversion, written from the format definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits; subnormals
 * below 2^-14), rounding to nearest with ties to even.
 * ---------------------------------------------------------------------- */
static uint16_t f32_to_f16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u); /* NaN */
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 rounds to inf */
  int e = (int)(ax >> 23) - 127;
  uint32_t m = (ax & 0x7FFFFFu) | (ax ? 0x800000u : 0u); /* 24-bit significand */
  if (ax == 0) return (uint16_t)sign;
  if ((ax >> 23) == 0) { e = -126; m = ax & 0x7FFFFFu; } /* fp32 subnormal */
  if (e >= -14) {
    /* normal: keep 11 significant bits (implicit + 10) of the 24 */
    uint32_t h = ((uint32_t)(e + 15) << 10) | ((m >> 13) & 0x3FFu);
    uint32_t rem = m & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1; /* carry may bump exponent */
    return (uint16_t)(sign | h);
  }
  /* subnormal result: value = m * 2^(e-23); in units of 2^-24 that is m * 2^(e+1) */
  int sh = -(e + 1); /* > 0 */
  if (sh > 25) return (uint16_t)sign;
  uint32_t q = m >> sh;
  uint32_t rem = m & ((1u << sh) - 1u);
  uint32_t half = 1u << (sh - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1;
  return (uint16_t)(sign | q); /* q may reach 0x400 = smallest normal, still correct */
}

static float f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(m | 0x400), e - 25);
  return sign ? -v : v;
}

uint16_t vqo_f32_to_f16(float f) { return f32_to_f16_rne(f); }
float vqo_f16_to_f32(uint16_t h) { return f16_to_f32(h); }

/* ------------------------------------------------------------------------
 * Row scale, [VQ3R page] §2 "one FP16 per-channel scale per row". The page
 * does not say which statistic; the reading used is the row RMS:
 * ss = sum_k w_k^2 in fp64 (sequential), rms = sqrt(ss / n) in fp64, then
 * rounded fp64 -> fp32 -> fp16 (each step to nearest even).
 * Returns VQO_EDATA for a non-finite weight or an RMS beyond the fp16 range.
 * ---------------------------------------------------------------------- */
static int row_scale(const float* w, int64_t n, uint16_t* s_bits) {
  double ss = 0.0;
  for (int64_t k = 0; k < n; ++k) {
    if (!isfinite(w[k])) return VQO_EDATA;
    ss += (double)w[k] * (double)w[k];
  }
  double rms = sqrt(ss / (double)n);
  uint16_t h = f32_to_f16_rne((float)rms);
  if ((h & 0x7C00u) == 0x7C00u) return VQO_EDATA;
  *s_bits = h;
  return VQO_OK;
}

/* Threads the parallel loops below run on (the OpenMP runtime's setting); no
   arithmetic depends on it. */
int vqo_max_threads(void) { return omp_get_max_threads(); }

int vqo_row_scales(const float* w, int64_t rows, int64_t cols, uint16_t* s_bits) {
  int st = VQO_OK;
  for (int64_t r = 0; r < rows; ++r) {
    int e = row_scale(w + r * cols, cols, &s_bits[r]);
    if (e) st = e;
  }
  return st;
}

/* Normalization, [VQ3R page] §2 (W ~ scale * sum of codewords, so the
 * codewords live in the scaled-down domain): v = w / s as one correctly
 * rounded fp32 division; an all-zero-scale row maps to v = 0. */
static float normalize(float w, float s) { return (s == 0.0f) ? 0.0f : w / s; }

/* ------------------------------------------------------------------------
 * Squared distance of an 8-dim residual to a codeword, [VQ3R page] §4 (the
 * encoder evaluates all codeword distances). Fixed order: acc = 0;
 * for k = 0..7: e = r_k - c_k; acc = fmaf(e, e, acc).
 * ---------------------------------------------------------------------- */
static float dist8(const float* r, const float* c) {
  float acc = 0.0f;
  for (int k = 0; k < DIM; ++k) {
    float e = r[k] - c[k];
    acc = fmaf(e, e, acc);
  }
  return acc;
}

float vqo_dist8(const float* r, const float* c) { return dist8(r, c); }

/* Exhaustive nearest codeword over j = 0..K-1 in increasing order; a strictly
 * smaller distance wins, so ties go to the lowest index. */
static int argmin_codeword(const float* r, const float* cb, int K) {
  int best = 0;
  float bd = dist8(r, cb);
  for (int j = 1; j < K; ++j) {
    float d = dist8(r, cb + (int64_t)j * DIM);
    if (d < bd) { bd = d; best = j; }
  }
  return best;
}

int vqo_argmin(const float* r, const float* cb, int K) { return argmin_codeword(r, cb, K); }

/* Greedy residual encode of one vector, [VQ3R page] §2 (residual relay) and
 * §4 (one pass, the winning index per stage): r <- v; for each stage t:
 * i_t = argmin_j d(r, C_t[j]); r <- r - C_t[i_t] (fp32, elementwise). */
static void encode_vector(const float* v, const float* cb, int stages, int K, int32_t* idx) {
  float r[DIM];
  for (int k = 0; k < DIM; ++k) r[k] = v[k];
  for (int t = 0; t < stages; ++t) {
    const float* C = cb + (int64_t)t * K * DIM;
    int i = argmin_codeword(r, C, K);
    idx[t] = i;
    for (int k = 0; k < DIM; ++k) r[k] = r[k] - C[(int64_t)i * DIM + k];
  }
}

/* Greedy encode of already-normalized vectors v [n][8] (no row scale). */
int vqo_encode_vectors(const float* v, int64_t n, int stages, int K, const float* cb, int32_t* idx_out) {
  if (n < 0 || stages < 1 || K < 1) return VQO_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) encode_vector(v + i * DIM, cb, stages, K, idx_out + i * stages);
  return VQO_OK;
}

/* Encode a [rows x cols] fp32 matrix: per row the fp16 scale, then every
 * 8-element vector v = w[8j .. 8j+7] / s is encoded greedily.
 * idx_out: int32 [rows][cols/8][stages]. */
int vqo_encode(const float* w, int64_t rows, int64_t cols, int stages, int K, const float* cb,
               uint16_t* s_bits, int32_t* idx_out) {
  if (cols % DIM || rows < 0 || stages < 1 || K < 1) return VQO_EINVAL;
  int64_t V = cols / DIM;
  int st = VQO_OK;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < rows; ++r) {
    const float* wr = w + r * cols;
    uint16_t h;
    if (row_scale(wr, cols, &h)) {
#pragma omp atomic write
      st = VQO_EDATA;
      continue;
    }
    s_bits[r] = h;
    float s = f16_to_f32(h);
    for (int64_t j = 0; j < V; ++j) {
      float v[DIM];
      for (int k = 0; k < DIM; ++k) v[k] = normalize(wr[j * DIM + k], s);
      encode_vector(v, cb, stages, K, idx_out + (r * V + j) * stages);
    }
  }
  return st;
}

/* Decode, [VQ3R page] §2: w_hat = s * (((C1[i1] + C2[i2]) + C3[i3]) [+ C4[i4]]),
 * summed left to right in fp32, then one fp32 multiply (no fused operations).
 * With stages_used < stages only the first stages_used codewords are summed
 * (the partial reconstruction after that many stages, e.g. "vq2"). */
int vqo_decode(const int32_t* idx, const uint16_t* s_bits, const float* cb, int64_t rows, int64_t cols,
               int stages, int K, int stages_used, float* w_out) {
  if (cols % DIM || stages_used < 1 || stages_used > stages) return VQO_EINVAL;
  int64_t V = cols / DIM;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float s = f16_to_f32(s_bits[r]);
    for (int64_t j = 0; j < V; ++j) {
      const int32_t* id = idx + (r * V + j) * stages;
      for (int k = 0; k < DIM; ++k) {
        float acc = cb[(int64_t)id[0] * DIM + k];
        for (int t = 1; t < stages_used; ++t) acc = acc + cb[((int64_t)t * K + id[t]) * DIM + k];
        w_out[r * cols + j * DIM + k] = s * acc;
      }
    }
  }
  return VQO_OK;
}

/* ------------------------------------------------------------------------
 * Lloyd codebook fit, [VQ3R page] §2 and §4 (per-layer codebooks fit with
 * k-means / Lloyd iterations on sampled experts; C1 on the vectors, C2 on the
 * stage-1 residuals, C3 on the stage-2 residuals).
 * Readings where the page is silent: stages are fit one after another, stage t on the
 * residuals left by greedy assignment to the final C_1..C_{t-1}; Forgy init
 * from caller-given distinct training-vector indices; one iteration = assign
 * (exhaustive argmin above) + update; a cluster with no members keeps its
 * centroid; the mean is taken from an exact int64 fixed-point sum:
 *   F = 62 - e_max - ceil(log2 N), where max|r| < 2^e_max (frexp exponent),
 *   S_jk = sum_i llrint(r_ik * 2^F),  c_jk = (float)(((double)S_jk * 2^-F) / n_j).
 * After the last update every vector is assigned once more and its residual
 * r - C_t[a] becomes the training set of stage t+1.
 * ---------------------------------------------------------------------- */
static int ceil_log2_i64(int64_t n) {
  int c = 0;
  while (((int64_t)1 << c) < n) ++c;
  return c;
}

int vqo_fixed_point_bits(float maxabs, int64_t n) {
  if (maxabs == 0.0f) return 62 - ceil_log2_i64(n);
  int e;
  frexpf(maxabs, &e); /* maxabs = m * 2^e, m in [0.5, 1): maxabs < 2^e */
  return 62 - e - ceil_log2_i64(n);
}

/* One stage of Lloyd on R (n x 8, fp32), modified in place into the residual.
 * obj (optional, iters+1 entries): sum over vectors of d(r, C[a]) in fp64 after
 * each assignment (the k-means objective). */
static int lloyd_stage(float* R, int64_t n, int K, int iters, const int64_t* init, float* C,
                       int32_t* assign, double* obj) {
  float maxabs = 0.0f;
  for (int64_t i = 0; i < n * DIM; ++i) {
    float a = fabsf(R[i]);
    if (a > maxabs) maxabs = a;
  }
  int F = vqo_fixed_point_bits(maxabs, n);
  if (F < 16) return VQO_EDATA;
  for (int j = 0; j < K; ++j)
    for (int k = 0; k < DIM; ++k) C[j * DIM + k] = R[init[j] * DIM + k];
  int64_t* S = (int64_t*)malloc(sizeof(int64_t) * K * DIM);
  int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * K);
  for (int it = 0; it <= iters; ++it) {
    /* assignment */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) assign[i] = argmin_codeword(R + i * DIM, C, K);
    if (obj) {
      double o = 0.0;
      for (int64_t i = 0; i < n; ++i) o += (double)dist8(R + i * DIM, C + (int64_t)assign[i] * DIM);
      obj[it] = o;
    }
    if (it == iters) break;
    /* update: exact fixed-point cluster sums, then the mean */
    memset(S, 0, sizeof(int64_t) * K * DIM);
    memset(cnt, 0, sizeof(int64_t) * K);
    for (int64_t i = 0; i < n; ++i) {
      int j = assign[i];
      cnt[j] += 1;
      for (int k = 0; k < DIM; ++k) S[j * DIM + k] += llrint(ldexp((double)R[i * DIM + k], F));
    }
    for (int j = 0; j < K; ++j) {
      if (cnt[j] == 0) continue; /* empty cluster keeps its centroid */
      for (int k = 0; k < DIM; ++k)
        C[j * DIM + k] = (float)(ldexp((double)S[j * DIM + k], -F) / (double)cnt[j]);
    }
  }
  for (int64_t i = 0; i < n; ++i)
    for (int k = 0; k < DIM; ++k) R[i * DIM + k] = R[i * DIM + k] - C[(int64_t)assign[i] * DIM + k];
  free(S);
  free(cnt);
  return VQO_OK;
}

/* Fit `stages` codebooks of K entries on the vectors of n_mats matrices
 * [rows x cols] (fp32, each normalized by its own row scales).
 * init: int64 [stages][K] distinct indices into the n = n_mats*rows*cols/8
 * training vectors (matrix-major, then row-major, then vector).
 * cb_out: fp32 [stages][K][8].
 * Optional outputs: assign_out int32 [stages][n] (final assignment per stage),
 * obj_out fp64 [stages][iters+1], energy_out fp64 [stages+1] (sum of squared
 * training residual before stage 1 and after each stage). */
int vqo_fit(const float* const* mats, int n_mats, int64_t rows, int64_t cols, int stages, int K,
            int iters, const int64_t* init, float* cb_out, int32_t* assign_out, double* obj_out,
            double* energy_out) {
  if (cols % DIM || n_mats < 1 || rows < 1 || stages < 1 || K < 1 || iters < 0) return VQO_EINVAL;
  int64_t V = cols / DIM;
  int64_t n = (int64_t)n_mats * rows * V;
  if (n < K) return VQO_EINVAL;
  for (int t = 0; t < stages; ++t)
    for (int j = 0; j < K; ++j) {
      if (init[t * K + j] < 0 || init[t * K + j] >= n) return VQO_EINVAL;
      for (int q = 0; q < j; ++q)
        if (init[t * K + q] == init[t * K + j]) return VQO_EINVAL;
    }
  float* R = (float*)malloc(sizeof(float) * n * DIM);
  int32_t* assign = (int32_t*)malloc(sizeof(int32_t) * n);
  int st = VQO_OK;
  for (int m = 0; m < n_mats && st == VQO_OK; ++m)
    for (int64_t r = 0; r < rows; ++r) {
      const float* wr = mats[m] + r * cols;
      uint16_t h;
      if (row_scale(wr, cols, &h)) { st = VQO_EDATA; break; }
      float s = f16_to_f32(h);
      float* dst = R + ((int64_t)m * rows + r) * cols;
      for (int64_t k = 0; k < cols; ++k) dst[k] = normalize(wr[k], s);
    }
  if (st == VQO_OK && energy_out) {
    double e = 0.0;
    for (int64_t i = 0; i < n * DIM; ++i) e += (double)R[i] * (double)R[i];
    energy_out[0] = e;
  }
  for (int t = 0; t < stages && st == VQO_OK; ++t) {
    st = lloyd_stage(R, n, K, iters, init + (int64_t)t * K, cb_out + (int64_t)t * K * DIM, assign,
                     obj_out ? obj_out + (int64_t)t * (iters + 1) : NULL);
    if (st) break;
    if (assign_out) memcpy(assign_out + (int64_t)t * n, assign, sizeof(int32_t) * n);
    if (energy_out) {
      double e = 0.0;
      for (int64_t i = 0; i < n * DIM; ++i) e += (double)R[i] * (double)R[i];
      energy_out[t + 1] = e;
    }
  }
  free(R);
  free(assign);
  return st;
}

/* ------------------------------------------------------------------------
 * Seeded Forgy init. The configurations ask for Lloyd started from "seeded
 * random vectors" and the page names no generator; the reading taken here:
 * for stage t (0-based), a SplitMix64 stream whose state starts at
 * seed XOR (0x9E3779B97F4A7C15 * (t + 1)) (mod 2^64); each output d picks
 * training vector floor(d * n / 2^64) (the high half of the 128-bit product);
 * a pick already taken for this stage is skipped, until K distinct vectors
 * are chosen. SplitMix64 is the published generator of Steele, Lea and Flood
 * (OOPSLA 2014): the state advances by 0x9E3779B97F4A7C15 and each output is
 * the state mixed by z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 * z *= 0x94D049BB133111EB; z ^= z >> 31.
 * ---------------------------------------------------------------------- */
uint64_t vqo_splitmix64(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ull;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* init out: int64 [stages][K]. Error if n < K. */
int vqo_forgy_init(int64_t n, int K, int stages, uint64_t seed, int64_t* init) {
  if (K < 1 || stages < 1 || n < K) return VQO_EINVAL;
  for (int t = 0; t < stages; ++t) {
    uint64_t state = seed ^ (0x9E3779B97F4A7C15ull * (uint64_t)(t + 1));
    int64_t* out = init + (int64_t)t * K;
    int have = 0;
    while (have < K) {
      uint64_t d = vqo_splitmix64(&state);
      int64_t j = (int64_t)(((unsigned __int128)d * (unsigned __int128)(uint64_t)n) >> 64);
      int taken = 0;
      for (int q = 0; q < have; ++q)
        if (out[q] == j) { taken = 1; break; }
      if (!taken) out[have++] = j;
    }
  }
  return VQO_OK;
}

/* Lloyd on an explicit training set (n x 8 fp32, used as given), for the
 * closed-form pins; same stage semantics as vqo_fit. R is overwritten with the
 * final residual. */
int vqo_lloyd_on_vectors(float* R, int64_t n, int K, int iters, const int64_t* init, float* C,
                         int32_t* assign, double* obj) {
  if (n < K || K < 1 || iters < 0) return VQO_EINVAL;
  return lloyd_stage(R, n, K, iters, init, C, assign, obj);
}

/* ------------------------------------------------------------------------
 * Tied Trit-Planes, from the page "Новый метод квантования Tied Trit-Planes
 * сжимает DeepSeek-V4 до 4.0625 бит на вес" (ai-sphere.ru; cited as [TTP page]).
 * Its summary and "what happened" sections: PTQTP writes a weight group as two
 * ternary planes with one free scale each; tying the scales by a factor of 3
 * turns the pair into a single uniform 9-level (balanced ternary) quantizer,
 *   w ~ a * (3 t1 + t2) = a * q,   t1, t2 in {-1, 0, 1},  q in {-4, ..., 4},
 * and the two planes fold without loss into one 4-bit code plane, 4.0625 bits
 * per weight. Readings taken where the page is silent:
 *   - a group is 256 consecutive weights of a row with one fp16 scale
 *     (4 + 16/256 = 4.0625 bits per weight);
 *   - the solver alternates PTQTP's two minimisations under the tie: for a
 *     fixed scale, each weight takes its nearest level,
 *       q = clamp(rint(w / a), -4, 4)   (fp32 division, ties to even);
 *     for fixed levels, the least-squares scale a = sum_i w_i q_i / sum_i q_i^2,
 *     with the numerator summed exactly in int64 fixed point:
 *       F = 52 - e with max|w| < 2^e (frexp exponent), W_i = llrint(w_i 2^F),
 *       a = (float)(((double) sum_i W_i q_i) 2^-F / sum_i q_i^2);
 *     (|W_i q_i| < 2^54 and 256 terms stay below 2^62; the sum is exact and
 *     does not depend on the order of the terms); starting from
 *     a = max|w| / 4, for at most TTP_ITERS rounds, stopping when no level
 *     changes;
 *   - the stored scale is fp16(a); the levels are then chosen once more for
 *     that stored scale. A zero group gets a = 0 and q = 0;
 *   - code = q + 4 = 3 (t1 + 1) + (t2 + 1) in 0..8; two codes per byte, the
 *     even element in the low nibble.
 * ---------------------------------------------------------------------- */
#define TTP_GROUP 256
#define TTP_ITERS 8

static int ttp_level(float w, float a) {
  if (a == 0.0f) return 0;
  float t = rintf(w / a);
  if (t > 4.0f) t = 4.0f;
  if (t < -4.0f) t = -4.0f;
  return (int)t;
}

/* one group of n <= 256 weights; returns 0 or VQO_EDATA; *rounds = rounds run */
static int ttp_group(const float* w, int n, uint8_t* code, uint16_t* s_bits, int* rounds) {
  int q[TTP_GROUP];
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    if (!isfinite(w[i])) return VQO_EDATA;
    float aw = fabsf(w[i]);
    if (aw > amax) amax = aw;
  }
  float a = amax / 4.0f;
  int e = 0;
  (void)frexpf(amax, &e);
  const int F = 52 - e;
  long long W[TTP_GROUP];
  for (int i = 0; i < n; ++i) W[i] = llrint(ldexp((double)w[i], F));
  for (int i = 0; i < n; ++i) q[i] = ttp_level(w[i], a);
  int it = 0;
  while (it < TTP_ITERS) {
    long long swq = 0, sqq = 0;
    for (int i = 0; i < n; ++i) {
      swq += W[i] * q[i];
      sqq += (long long)q[i] * q[i];
    }
    if (sqq == 0) break;
    a = (float)(ldexp((double)swq, -F) / (double)sqq);
    ++it;
    int changed = 0;
    for (int i = 0; i < n; ++i) {
      int nq = ttp_level(w[i], a);
      changed |= nq != q[i];
      q[i] = nq;
    }
    if (!changed) break;
  }
  uint16_t h = f32_to_f16_rne(a);
  if ((h & 0x7C00u) == 0x7C00u) return VQO_EDATA; /* scale beyond the fp16 range */
  float ah = f16_to_f32(h);
  for (int i = 0; i < n; ++i) code[i] = (uint8_t)(ttp_level(w[i], ah) + 4);
  *s_bits = h;
  if (rounds) *rounds = it;
  return VQO_OK;
}

/* w fp32 [rows][cols], cols % 256 == 0 -> codes [rows][cols/2] (two per byte),
 * scales fp16 bits [rows][cols/256]; rounds (nullable) int32 [rows][cols/256] */
int vqo_ttp_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* scales, int32_t* rounds) {
  if (rows < 0 || cols <= 0 || cols % TTP_GROUP != 0) return VQO_EINVAL;
  const int64_t G = rows * (cols / TTP_GROUP);
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t g = 0; g < G; ++g) {
    uint8_t c[TTP_GROUP];
    int r = 0;
    if (ttp_group(w + g * TTP_GROUP, TTP_GROUP, c, &scales[g], &r) != VQO_OK) {
      bad = 1;
      continue;
    }
    for (int i = 0; i < TTP_GROUP / 2; ++i) codes[g * (TTP_GROUP / 2) + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
    if (rounds) rounds[g] = r;
  }
  return bad ? VQO_EDATA : VQO_OK;
}

/* w_hat = a * (code - 4), fp32 (exact: a has 11 significant bits, |q| <= 4) */
int vqo_ttp_dequantize(const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t cols, float* out) {
  if (rows < 0 || cols <= 0 || cols % TTP_GROUP != 0) return VQO_EINVAL;
  const int64_t n = rows * cols;
  for (int64_t i = 0; i < n; ++i) {
    int c = (codes[i / 2] >> (4 * (i & 1))) & 0xF;
    out[i] = f16_to_f32(scales[i / TTP_GROUP]) * (float)(c - 4);
  }
  return VQO_OK;
}
