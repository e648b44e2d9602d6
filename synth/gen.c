/*
 * Seeded synthetic inputs for the routed MoE FFN layer: activations, router
 * weights and int4-quantised expert weight blobs in the canonical format.
 *
 * This file generates inputs only. It is shared by the CPU oracle's tests,
 * the GPU parity tests and the benchmark, and it holds none of the layer's
 * arithmetic (no routing, no dequantisation, no matmul). Its quantiser exists
 * to turn N(0, std) weights into codes and scales; both the oracle and the GPU
 * library read the stored codes and scales, so quantiser details never affect
 * parity.
 *
 * Randomness: a counter-based generator. Draw i of stream `key` is the
 * SplitMix64 output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) applied to key + (i+1)*gamma,
 * gamma = 0x9E3779B97F4A7C15. Normals come in pairs from the Box-Muller
 * transform (Box & Muller 1958), in single precision, of two 24-bit uniforms
 * taken from one draw.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of the stream for (base, kind, a, b, c): a chain of SplitMix64 mixes. */
uint64_t synth_key(uint64_t base, uint64_t kind, uint64_t a, uint64_t b, uint64_t c) {
  uint64_t k = mix64(base + GAMMA);
  k = mix64(k ^ (kind + 1) * GAMMA);
  k = mix64(k ^ (a + 1) * GAMMA);
  k = mix64(k ^ (b + 1) * GAMMA);
  k = mix64(k ^ (c + 1) * GAMMA);
  return k;
}

uint64_t synth_u64(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* Normal pair number p of stream key: Box-Muller on two 24-bit uniforms. */
static inline void normal_pair(uint64_t key, uint64_t p, float* z0, float* z1) {
  uint64_t r = synth_u64(key, p);
  /* u1 in (0, 1] from the top 24 bits, u2 in [0, 1) from the low 24 bits */
  float u1 = ((float)(uint32_t)(r >> 40) + 1.0f) * (1.0f / 16777216.0f);
  float u2 = ((float)(uint32_t)(r & 0xFFFFFFu)) * (1.0f / 16777216.0f);
  float rad = sqrtf(-2.0f * logf(u1));
  float th = 6.28318530717958647692f * u2;
  *z0 = rad * cosf(th);
  *z1 = rad * sinf(th);
}

/* out[j] = mean + std * N_j, j in [0, n), N_j = normal number (first + j) of stream key. */
void synth_normal_f32(uint64_t key, int64_t first, int64_t n, float mean, float stdv, float* out) {
  for (int64_t j = 0; j < n; ++j) {
    int64_t i = first + j;
    float z0, z1;
    normal_pair(key, (uint64_t)(i >> 1), &z0, &z1);
    out[j] = mean + stdv * ((i & 1) ? z1 : z0);
  }
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* bf16 bits of RNE(mean + std * N_j). */
void synth_normal_bf16(uint64_t key, int64_t first, int64_t n, float mean, float stdv, uint16_t* out) {
  for (int64_t j = 0; j < n; ++j) {
    int64_t i = first + j;
    float z0, z1;
    normal_pair(key, (uint64_t)(i >> 1), &z0, &z1);
    out[j] = f32_to_bf16(mean + stdv * ((i & 1) ? z1 : z0));
  }
}

/* fp32 -> IEEE binary16 bits, round to nearest even. */
uint16_t synth_f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 rounds to inf */
  if (ax < 0x38800000u) {                                   /* below 2^-14: subnormal */
    float a;
    memcpy(&a, &ax, 4);
    uint32_t r = (uint32_t)nearbyintf(a * 16777216.0f);   /* units of 2^-24, exact scaling */
    return (uint16_t)(sign | r);
  }
  uint32_t mant = ax & 0x7FFFFFu;
  uint32_t h = ((uint32_t)((int32_t)(ax >> 23) - 112) << 10) | (mant >> 13);
  uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
  return (uint16_t)(sign | h);
}

float synth_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  float v;
  if (e == 0) {
    v = ldexpf((float)m, -24);
  } else if (e == 31) {
    uint32_t u = 0x7F800000u | (m << 13);
    memcpy(&v, &u, 4);
  } else {
    uint32_t u = ((e + 112) << 23) | (m << 13);
    memcpy(&v, &u, 4);
  }
  uint32_t u;
  memcpy(&u, &v, 4);
  u |= sign;
  memcpy(&v, &u, 4);
  return v;
}

/*
 * Fixture quantiser for one row of K weights, group size G:
 *   amax = max |w| over the group (fp32); s = fp16_rne(amax / 7);
 *   q = clamp(rint_half_even(w / float(s)), -7, 7); s == 0 gives q = 0.
 * Codes go to q[K] (int8), scales to s[K/G] (fp16 bits).
 */
void synth_quantize_row(const float* w, int K, int G, int8_t* q, uint16_t* s) {
  for (int g = 0; g < K / G; ++g) {
    const float* wg = w + (int64_t)g * G;
    float amax = 0.f;
    for (int i = 0; i < G; ++i) amax = fmaxf(amax, fabsf(wg[i]));
    uint16_t sh = synth_f32_to_f16(amax / 7.0f);
    float sf = synth_f16_to_f32(sh);
    s[g] = sh;
    for (int i = 0; i < G; ++i) {
      float r = (sf == 0.f) ? 0.f : nearbyintf(wg[i] / sf);
      r = fminf(fmaxf(r, -7.f), 7.f);
      q[(int64_t)g * G + i] = (int8_t)r;
    }
  }
}

/* Canonical nibble packing: byte j = (q[2j] & 0xF) | (q[2j+1] & 0xF) << 4. */
void synth_pack_int4(const int8_t* q, int64_t n, uint8_t* out) {
  for (int64_t j = 0; j < n / 2; ++j)
    out[j] = (uint8_t)(((uint8_t)q[2 * j] & 0xFu) | (((uint8_t)q[2 * j + 1] & 0xFu) << 4));
}

int64_t synth_expert_bytes(int H, int I, int G) {
  return (int64_t)3 * H * I / 2 + (int64_t)2 * 3 * H * I / G;
}

int64_t synth_expert_bytes_b(int H, int I, int G, int b) {
  return (int64_t)3 * H * I * b / 8 + (int64_t)2 * 3 * H * I / G;
}

/*
 * Fixture quantiser onto b-bit odd levels (b = 2, 3), one row of K weights:
 *   L = 2^b - 1; amax = max |w| over the group; s = fp16_rne(amax / L);
 *   n = clamp(rint_half_even((w / float(s) + L) / 2), 0, 2^b - 1), so that
 *   q = 2n - L is the odd level nearest to w / s; s == 0 gives n = 2^(b-1) (q = 1, weight 0).
 * Codes n go to n[K], scales to s[K/G] (fp16 bits).
 */
void synth_quantize_row_odd(const float* w, int K, int G, int b, uint8_t* n, uint16_t* s) {
  const float L = (float)((1 << b) - 1);
  for (int g = 0; g < K / G; ++g) {
    const float* wg = w + (int64_t)g * G;
    float amax = 0.f;
    for (int i = 0; i < G; ++i) amax = fmaxf(amax, fabsf(wg[i]));
    uint16_t sh = synth_f32_to_f16(amax / L);
    float sf = synth_f16_to_f32(sh);
    s[g] = sh;
    for (int i = 0; i < G; ++i) {
      float r = (sf == 0.f) ? (float)(1 << (b - 1)) : nearbyintf((wg[i] / sf + L) * 0.5f);
      r = fminf(fmaxf(r, 0.f), (float)((1 << b) - 1));
      n[(int64_t)g * G + i] = (uint8_t)r;
    }
  }
}

/* Canonical b-bit packing: code i at bits [b*i, b*i+b) of the little-endian bit string out. */
void synth_pack_bits(const uint8_t* n, int64_t count, int b, uint8_t* out) {
  memset(out, 0, (size_t)((count * b + 7) / 8));
  for (int64_t i = 0; i < count; ++i)
    for (int j = 0; j < b; ++j)
      if ((n[i] >> j) & 1u) out[(i * b + j) >> 3] |= (uint8_t)(1u << ((i * b + j) & 7));
}

/*
 * One canonical expert blob:
 *   q_gate[I][H/2] | q_up[I][H/2] | q_down[H][I/2] | s_gate[I][H/G] | s_up[I][H/G] | s_down[H][I/G]
 * Weights ~ N(0, std) from streams (base, kind=1, layer, expert, tensor) with
 * tensor 0 = gate, 1 = up, 2 = down; row r of a tensor is normals [r*K, (r+1)*K).
 */
static void expert_blob(uint64_t base, int layer, int expert, int H, int I, int G, float stdv,
                        uint8_t* out, float* wrow, int8_t* qrow) {
  int64_t qg = (int64_t)I * H / 2, qd = (int64_t)H * I / 2;
  uint8_t* q_gate = out;
  uint8_t* q_up = out + qg;
  uint8_t* q_down = out + 2 * qg;
  uint16_t* s_gate = (uint16_t*)(out + 2 * qg + qd);
  uint16_t* s_up = s_gate + (int64_t)I * (H / G);
  uint16_t* s_down = s_up + (int64_t)I * (H / G);
  for (int t = 0; t < 3; ++t) {
    int rows = (t < 2) ? I : H, K = (t < 2) ? H : I;
    uint8_t* qd_out = (t == 0) ? q_gate : (t == 1) ? q_up : q_down;
    uint16_t* sd_out = (t == 0) ? s_gate : (t == 1) ? s_up : s_down;
    uint64_t key = synth_key(base, 1, (uint64_t)layer, (uint64_t)expert, (uint64_t)t);
    for (int r = 0; r < rows; ++r) {
      synth_normal_f32(key, (int64_t)r * K, K, 0.f, stdv, wrow);
      synth_quantize_row(wrow, K, G, qrow, sd_out + (int64_t)r * (K / G));
      synth_pack_int4(qrow, K, qd_out + (int64_t)r * (K / 2));
    }
  }
}

/* The same expert's weights quantised onto b-bit odd levels (b = 2, 3), canonical b-bit rows. */
static void expert_blob_b(uint64_t base, int layer, int expert, int H, int I, int G, float stdv, int b,
                          uint8_t* out, float* wrow, uint8_t* nrow) {
  int64_t qg = (int64_t)I * H * b / 8, qd = (int64_t)H * I * b / 8;
  uint8_t* q_gate = out;
  uint8_t* q_up = out + qg;
  uint8_t* q_down = out + 2 * qg;
  uint16_t* s_gate = (uint16_t*)(out + 2 * qg + qd);
  uint16_t* s_up = s_gate + (int64_t)I * (H / G);
  uint16_t* s_down = s_up + (int64_t)I * (H / G);
  for (int t = 0; t < 3; ++t) {
    int rows = (t < 2) ? I : H, K = (t < 2) ? H : I;
    uint8_t* qd_out = (t == 0) ? q_gate : (t == 1) ? q_up : q_down;
    uint16_t* sd_out = (t == 0) ? s_gate : (t == 1) ? s_up : s_down;
    uint64_t key = synth_key(base, 1, (uint64_t)layer, (uint64_t)expert, (uint64_t)t);
    for (int r = 0; r < rows; ++r) {
      synth_normal_f32(key, (int64_t)r * K, K, 0.f, stdv, wrow);
      synth_quantize_row_odd(wrow, K, G, b, nrow, sd_out + (int64_t)r * (K / G));
      synth_pack_bits(nrow, K, b, qd_out + (int64_t)r * K * b / 8);
    }
  }
}

/* Blobs of experts [e0, e0+n) with b bits per code (b = 4: synth_experts). */
void synth_experts_b(uint64_t base, int layer, int e0, int n, int H, int I, int G, float stdv, int b, uint8_t* out) {
  int64_t eb = synth_expert_bytes_b(H, I, G, b);
  int K = H > I ? H : I;
#pragma omp parallel
  {
    float* wrow = (float*)malloc(sizeof(float) * (size_t)K);
    uint8_t* nrow = (uint8_t*)malloc((size_t)K);
#pragma omp for schedule(dynamic, 1)
    for (int e = 0; e < n; ++e)
      expert_blob_b(base, layer, e0 + e, H, I, G, stdv, b, out + (int64_t)e * eb, wrow, nrow);
    free(wrow);
    free(nrow);
  }
}

/*
 * b-bit blobs (b = 2, 3) from 4-bit blobs of the same shape, for throughput runs that
 * need a lower-bit copy of layers already generated: each code keeps the top b bits of
 * its offset form (n_b = (q + 8) >> (4 - b)), the fp16 scales are copied. A seeded
 * synthetic b-bit expert of the same shape (not a re-quantisation of the weights).
 */
void synth_cut_codes(const uint8_t* in4, int64_t n_experts, int H, int I, int G, int b, uint8_t* out) {
  const int64_t eb4 = synth_expert_bytes(H, I, G), ebb = synth_expert_bytes_b(H, I, G, b);
  const int64_t codes4 = (int64_t)3 * H * I / 2, codesb = (int64_t)3 * H * I * b / 8;
  const int64_t rows = (int64_t)2 * I + H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t e = 0; e < n_experts; ++e) {
    const uint8_t* src = in4 + e * eb4;
    uint8_t* dst = out + e * ebb;
    memset(dst, 0, (size_t)codesb);
    for (int64_t r = 0; r < rows; ++r) {
      const int K = r < 2 * I ? H : I;
      const int64_t o4 = r < 2 * I ? r * (H / 2) : 2 * (int64_t)I * (H / 2) + (r - 2 * I) * (I / 2);
      const int64_t ob = r < 2 * I ? r * ((int64_t)H * b / 8) : 2 * (int64_t)I * H * b / 8 + (r - 2 * I) * ((int64_t)I * b / 8);
      for (int i = 0; i < K; ++i) {
        const uint32_t nib = (src[o4 + i / 2] >> (4 * (i & 1))) & 0xFu;
        const uint32_t nb = (nib ^ 8u) >> (4 - b);
        for (int j = 0; j < b; ++j)
          if ((nb >> j) & 1u) dst[ob + (((int64_t)i * b + j) >> 3)] |= (uint8_t)(1u << ((i * b + j) & 7));
      }
    }
    memcpy(dst + codesb, src + codes4, (size_t)(eb4 - codes4));
  }
}

/* Blobs of experts [e0, e0+n) of one layer into out (n * expert_bytes), threaded over experts. */
void synth_experts(uint64_t base, int layer, int e0, int n, int H, int I, int G, float stdv, uint8_t* out) {
  int64_t eb = synth_expert_bytes(H, I, G);
  int K = H > I ? H : I;
#pragma omp parallel
  {
    float* wrow = (float*)malloc(sizeof(float) * (size_t)K);
    int8_t* qrow = (int8_t*)malloc((size_t)K);
#pragma omp for schedule(dynamic, 1)
    for (int e = 0; e < n; ++e)
      expert_blob(base, layer, e0 + e, H, I, G, stdv, out + (int64_t)e * eb, wrow, qrow);
    free(wrow);
    free(qrow);
  }
}

/* Raw fp32 weights of one tensor of one expert (for tests of the quantiser): rows*K normals. */
void synth_expert_tensor_f32(uint64_t base, int layer, int expert, int tensor, int rows, int K, float stdv,
                             float* out) {
  uint64_t key = synth_key(base, 1, (uint64_t)layer, (uint64_t)expert, (uint64_t)tensor);
  synth_normal_f32(key, 0, (int64_t)rows * K, 0.f, stdv, out);
}
