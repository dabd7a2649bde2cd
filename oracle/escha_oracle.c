/*
 * escha_oracle.c -- plain CPU oracle for the trellis-coded ("eschamoe",
 * EXL3-style) routed-expert path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU library shares no
 * code, header, table or helper with it, and neither includes the other.
 *
 * Everything here is written for a reader who checks it against the pages by
 * eye: single-bit loops, fp64 arithmetic, one rounding where the format
 * defines one, no blocking and no fusion. Sources (page title, section):
 *
 *  - "Qwen3.6-35B-A3B-Escha-W2-trellis-mlx" model card, exactness table:
 *    the codebook hash r = ((s*0xCBAC1FED) & 0x8FFF8FFF) ^ 0x3B603B60 and
 *    "two fp16 halves summed RNE"; Hadamard with scale 1/sqrt(128).
 *  - "Escha-W2 port: 2-bit trellis decoded in the GEMV" (hipfire PR),
 *    closing summary "What it is": 16x16 tiles, K bits per weight, code
 *    int16[in/16, out/16, 16K]; overlapping 16-bit windows sliding by K
 *    bits; Sylvester H128 on both sides. Commit notes on the CPU oracle:
 *    state 3 decodes to 0x3ab8 under RNE; gate is the first half of
 *    gate_up; pruned outputs are exactly zero; no zero-activation skip.
 *  - "Qwen3.6-35B-A3B-Escha-W2" model card, Format notes: K comes from
 *    the code tensor's last dimension (2 for gate_up, 3 for down).
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes of the repository):
 *  A1  bit b of a tile's stream is bit (b mod 16) of little-endian word b/16;
 *  A2  windows that run past the tile end wrap to its start (tail-biting);
 *  A3  the first stream bit of a window is the state's least significant bit;
 *  A4  weight i of a tile sits at input row k = i/16, output column n = i%16;
 *  A8  input side: rin first, then H; output side: H first, then rout;
 *  A10 router weights are softmax probabilities over all experts, not
 *      renormalised over the selected k; ties go to the lower expert index;
 *  A17 router logits: the fp16 rounding of the exact gate . x dot product
 *      (the pages fix the fp16 gate and the rounding, not the precision of
 *      the sum; the exact sum is the plainest reading).
 * Real-checkpoint parity of A1-A4 is unpinned: the pages print no decoded
 * tile of real data.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define EO_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* IEEE half / bfloat16 <-> double, written from the format definitions.     */
/* ------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
EO_EXPORT double eo_f16_to_double(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16: the top 16 bits of a binary32. */
EO_EXPORT double eo_bf16_to_double(uint16_t b) {
  int sign = b >> 15;
  int e = (b >> 7) & 255;
  int m = b & 127;
  double v;
  if (e == 0)
    v = ldexp((double)m, -133); /* subnormal: m * 2^-126 * 2^-7 */
  else if (e == 255)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
  return sign ? -v : v;
}

/*
 * Round a finite double to a binary format with `p` fraction bits, exponent
 * bias `bias` and largest finite exponent `emax`, to nearest with ties to
 * even. Returns the encoded bits (sign in bit p + exponent width).
 */
static uint32_t rne_encode(double v, int p, int bias, int emax, int ebits) {
  uint32_t sign = signbit(v) ? 1u : 0u;
  uint32_t sign_bit = sign << (p + ebits);
  uint32_t exp_all_ones = ((1u << ebits) - 1u) << p;
  if (isnan(v)) return exp_all_ones | (1u << (p - 1));
  double a = fabs(v);
  if (a == 0.0) return sign_bit;
  int emin = 1 - bias; /* smallest normal exponent */
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int eu = e - 1;
  if (eu < emin) eu = emin; /* subnormals share the quantum 2^(emin-p) */
  double quantum = ldexp(1.0, eu - p);
  double q = a / quantum; /* exact: division by a power of two */
  double fl = floor(q);
  double rem = q - fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) == 1.0)) fl += 1.0;
  double r = fl * quantum; /* the rounded magnitude */
  /* Overflow: the rounded value exceeds the largest finite number. */
  double maxfin = ldexp((double)((1u << (p + 1)) - 1u), emax - p);
  if (r > maxfin) return sign_bit | exp_all_ones;
  if (r < ldexp(1.0, emin)) /* subnormal, or rounded up to min normal */
    return sign_bit | (uint32_t)fl;
  frexp(r, &e);
  int E = e - 1;
  uint32_t m = (uint32_t)(r / ldexp(1.0, E - p) - ldexp(1.0, p));
  return sign_bit | ((uint32_t)(E + bias) << p) | m;
}

EO_EXPORT uint16_t eo_double_to_f16_rne(double v) {
  return (uint16_t)rne_encode(v, 10, 15, 15, 5);
}

EO_EXPORT uint16_t eo_double_to_bf16_rne(double v) {
  return (uint16_t)rne_encode(v, 7, 127, 127, 8);
}

/* ------------------------------------------------------------------------ */
/* The codebook: one 16-bit trellis state -> one fp16 weight.                */
/* ------------------------------------------------------------------------ */

/*
 * Model card "...-trellis-mlx", exactness table: multiply the state by
 * 0xCBAC1FED (mod 2^32), keep the bits of 0x8FFF8FFF, xor 0x3B603B60, read
 * the low and high 16 bits as two fp16 numbers and add them with one
 * round-to-nearest-even. The sum of two binary16 values is exact in double,
 * so the only rounding is the final one.
 */
EO_EXPORT uint16_t eo_cba_decode_state(uint32_t s) {
  uint64_t prod = (uint64_t)(s & 0xFFFFu) * 0xCBAC1FEDull;
  uint32_t r = (uint32_t)(prod & 0xFFFFFFFFull);
  r = (r & 0x8FFF8FFFu) ^ 0x3B603B60u;
  double lo = eo_f16_to_double((uint16_t)(r & 0xFFFFu));
  double hi = eo_f16_to_double((uint16_t)(r >> 16));
  return eo_double_to_f16_rne(lo + hi);
}

/* ------------------------------------------------------------------------ */
/* One 16x16 tile: 16*K little-endian uint16 words -> 256 fp16 weights.      */
/* ------------------------------------------------------------------------ */

/* Reading A1: bit b of the stream is bit (b % 16) of word b / 16. */
static int stream_bit(const uint16_t* words, int K, int b) {
  int nbits = 256 * K;
  b %= nbits; /* reading A2: windows wrap around the tile */
  return (words[b / 16] >> (b % 16)) & 1;
}

/* Weight i's state: the 16 stream bits starting at K*i (reading A3). */
EO_EXPORT uint32_t eo_tile_state(const uint16_t* words, int K, int i) {
  uint32_t s = 0;
  for (int j = 0; j < 16; j++) s |= (uint32_t)stream_bit(words, K, K * i + j) << j;
  return s;
}

EO_EXPORT void eo_decode_tile(const uint16_t* words, int K, uint16_t* out256) {
  for (int i = 0; i < 256; i++) out256[i] = eo_cba_decode_state(eo_tile_state(words, K, i));
}

/*
 * Reconstruct one projection: code int16 [in/16][out/16][16K] (input-tile
 * index outermost) -> W fp16 bits [out][in]. Reading A4 places weight i of
 * tile (kt, nt) at W[16*nt + i%16][16*kt + i/16].
 * Returns 0, or -1 when the shape is not a whole number of tiles.
 */
EO_EXPORT int eo_reconstruct(const uint16_t* code, int in_f, int out_f, int K, uint16_t* W) {
  if (in_f <= 0 || out_f <= 0 || in_f % 16 || out_f % 16 || (K != 2 && K != 3)) return -1;
  int n_kt = in_f / 16, n_nt = out_f / 16;
  uint16_t tile[256];
  for (int kt = 0; kt < n_kt; kt++) {
    for (int nt = 0; nt < n_nt; nt++) {
      const uint16_t* words = code + ((size_t)kt * n_nt + nt) * (size_t)(16 * K);
      eo_decode_tile(words, K, tile);
      for (int i = 0; i < 256; i++) {
        int k_local = i / 16, n_local = i % 16;
        W[(size_t)(16 * nt + n_local) * in_f + (16 * kt + k_local)] = tile[i];
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* 128-point Sylvester Hadamard, scale 1/sqrt(128), block-diagonal.           */
/* ------------------------------------------------------------------------ */

static int popcount_u32(uint32_t v) {
  int c = 0;
  while (v) {
    c += v & 1u;
    v >>= 1;
  }
  return c;
}

/* Sylvester order: H[i][j] = (-1)^popcount(i & j). */
EO_EXPORT double eo_hadamard_entry(int i, int j) {
  return (popcount_u32((uint32_t)(i & j)) & 1) ? -1.0 : 1.0;
}

/* y = H_n x on each consecutive block of 128 (n a multiple of 128). */
EO_EXPORT void eo_hadamard128(const double* x, int64_t rows, int n, double* y) {
  const double scale = 1.0 / sqrt(128.0);
  for (int64_t r = 0; r < rows; r++) {
    const double* xr = x + r * n;
    double* yr = y + r * n;
    for (int b = 0; b < n / 128; b++) {
      for (int i = 0; i < 128; i++) {
        double acc = 0.0;
        for (int j = 0; j < 128; j++) acc += eo_hadamard_entry(i, j) * xr[128 * b + j];
        yr[128 * b + i] = acc * scale;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* One coded projection, staged: x~ = H(rin*x); z = W x~; y = rout*H(z).    */
/* ------------------------------------------------------------------------ */

/*
 * W fp16 bits [out][in]; rin fp16 bits [in]; rout fp16 bits [out];
 * x double [in] -> y double [out]. No term is skipped: a zero activation
 * still multiplies its weight (0 * NaN stays NaN).
 */
EO_EXPORT void eo_proj(const uint16_t* W, const uint16_t* rin, const uint16_t* rout, int in_f,
                       int out_f, const double* x, double* y) {
  double* xs = (double*)malloc(sizeof(double) * in_f);
  double* xt = (double*)malloc(sizeof(double) * in_f);
  double* z = (double*)malloc(sizeof(double) * out_f);
  double* zt = (double*)malloc(sizeof(double) * out_f);
  for (int k = 0; k < in_f; k++) xs[k] = eo_f16_to_double(rin[k]) * x[k];
  eo_hadamard128(xs, 1, in_f, xt);
  for (int n = 0; n < out_f; n++) {
    double acc = 0.0;
    const uint16_t* row = W + (size_t)n * in_f;
    for (int k = 0; k < in_f; k++) acc += eo_f16_to_double(row[k]) * xt[k];
    z[n] = acc;
  }
  eo_hadamard128(z, 1, out_f, zt);
  for (int n = 0; n < out_f; n++) y[n] = eo_f16_to_double(rout[n]) * zt[n];
  free(xs);
  free(xt);
  free(z);
  free(zt);
}

/*
 * The same projection as one matrix: W_eff = diag(rout) H_n W H_n diag(rin),
 * written out entry by entry. Weff double [out][in].
 */
EO_EXPORT void eo_proj_weff(const uint16_t* W, const uint16_t* rin, const uint16_t* rout, int in_f,
                            int out_f, double* Weff) {
  const double scale = 1.0 / sqrt(128.0);
  /* T = W H_n (right factor): T[n][k] = sum_j W[n][j] H_n[j][k] inside k's block. */
  double* T = (double*)malloc(sizeof(double) * (size_t)out_f * in_f);
  for (int n = 0; n < out_f; n++) {
    for (int k = 0; k < in_f; k++) {
      int kb = k / 128, kl = k % 128;
      double acc = 0.0;
      for (int jl = 0; jl < 128; jl++)
        acc += eo_f16_to_double(W[(size_t)n * in_f + 128 * kb + jl]) * eo_hadamard_entry(jl, kl);
      T[(size_t)n * in_f + k] = acc * scale;
    }
  }
  for (int n = 0; n < out_f; n++) {
    int nb = n / 128, nl = n % 128;
    for (int k = 0; k < in_f; k++) {
      double acc = 0.0;
      for (int il = 0; il < 128; il++)
        acc += eo_hadamard_entry(nl, il) * T[(size_t)(128 * nb + il) * in_f + k];
      Weff[(size_t)n * in_f + k] =
          eo_f16_to_double(rout[n]) * acc * scale * eo_f16_to_double(rin[k]);
    }
  }
  free(T);
}

/* SwiGLU over the gate_up output: gate = first half, up = second half. */
EO_EXPORT void eo_swiglu(const double* y_gu, int inter, double* h) {
  for (int c = 0; c < inter; c++) {
    double g = y_gu[c];
    double u = y_gu[inter + c];
    h[c] = g / (1.0 + exp(-g)) * u;
  }
}

/* ------------------------------------------------------------------------ */
/* Routing: softmax over all experts, top-k, ties to the lower index.        */
/* ------------------------------------------------------------------------ */

EO_EXPORT void eo_route_topk(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  double* p = (double*)malloc(sizeof(double) * E);
  unsigned char* taken = (unsigned char*)malloc(E);
  for (int t = 0; t < T; t++) {
    const float* l = logits + (size_t)t * E;
    double m = -INFINITY;
    for (int e = 0; e < E; e++)
      if ((double)l[e] > m) m = (double)l[e];
    double sum = 0.0;
    for (int e = 0; e < E; e++) {
      p[e] = exp((double)l[e] - m);
      sum += p[e];
    }
    for (int e = 0; e < E; e++) p[e] /= sum;
    memset(taken, 0, E);
    for (int j = 0; j < k; j++) {
      int best = -1;
      for (int e = 0; e < E; e++) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower index on ties */
      }
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
      w[(size_t)t * k + j] = p[best];
    }
  }
  free(p);
  free(taken);
}

/*
 * Router logits, the step before routing: logit[t][e] = the fp16 rounding
 * (round to nearest even) of the dot product of gate row e (fp16, [E][H])
 * with the hidden state of token t (bf16, [T][H]). The model card's
 * exactness table keeps the router gate in fp16; the port's review notes
 * state that the logits are rounded to f16 before the top-k, which makes
 * exact ties that fp32 logits would not have. Every product of an fp16 and
 * a bf16 value is exact in fp64, and the sum is taken in fp64 (error far
 * below half an f16 ulp unless the sum cancels), then rounded once.
 * logits: fp32 holding the f16 value; raw (may be NULL): the fp64 sum.
 */
EO_EXPORT void eo_router_logits(const uint16_t* x_bf16, int T, int H, const uint16_t* gate_f16,
                                int E, float* logits, double* raw) {
  for (int t = 0; t < T; t++)
    for (int e = 0; e < E; e++) {
      double acc = 0.0;
      for (int i = 0; i < H; i++)
        acc += eo_f16_to_double(gate_f16[(size_t)e * H + i]) *
               eo_bf16_to_double(x_bf16[(size_t)t * H + i]);
      logits[(size_t)t * E + e] = (float)eo_f16_to_double(eo_double_to_f16_rne(acc));
      if (raw) raw[(size_t)t * E + e] = acc;
    }
}

/*
 * Group (token, slot) pairs by expert: counts[E], offsets[E+1] (exclusive
 * prefix sums), perm[T*k] = pair indices t*k+j ordered by expert and, within
 * an expert, by pair index.
 */
EO_EXPORT void eo_group(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                        int32_t* perm) {
  int P = T * k;
  for (int e = 0; e < E; e++) counts[e] = 0;
  for (int i = 0; i < P; i++) counts[ids[i]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  int pos = 0;
  for (int e = 0; e < E; e++)
    for (int i = 0; i < P; i++)
      if (ids[i] == e) perm[pos++] = i;
}

/* ------------------------------------------------------------------------ */
/* One MoE layer: per pair gate_up -> SiLU*up -> down, then the weighted sum. */
/* ------------------------------------------------------------------------ */

typedef struct {
  const uint16_t* gu_code; /* [E][hidden/16][2*inter/16][16*k_gu] */
  const uint16_t* gu_rin;  /* [E][hidden] fp16 */
  const uint16_t* gu_rout; /* [E][2*inter] fp16 */
  const uint16_t* dn_code; /* [E][inter/16][hidden/16][16*k_dn] */
  const uint16_t* dn_rin;  /* [E][inter] fp16 */
  const uint16_t* dn_rout; /* [E][hidden] fp16 */
  int32_t n_experts, hidden, inter, k_gu, k_dn, top_k;
} eo_layer_t;

typedef struct {
  const eo_layer_t* L;
  const uint16_t* x_bf16;
  int T;
  const int32_t* ids;
  const int32_t* expert_list; /* distinct experts to process */
  int n_list;
  int next; /* shared work index, guarded by mu */
  pthread_mutex_t mu;
  double* pair_out;  /* [T*k][hidden] */
  double* inter_out; /* [T*k][inter] or NULL */
  int status;
} eo_layer_job_t;

static void* eo_layer_worker(void* arg) {
  eo_layer_job_t* J = (eo_layer_job_t*)arg;
  const eo_layer_t* L = J->L;
  int H = L->hidden, I = L->inter, G = 2 * L->inter, k = L->top_k;
  size_t gu_words = (size_t)(H / 16) * (G / 16) * 16 * L->k_gu;
  size_t dn_words = (size_t)(I / 16) * (H / 16) * 16 * L->k_dn;
  uint16_t* Wgu = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)G * H);
  uint16_t* Wdn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H * I);
  double* x = (double*)malloc(sizeof(double) * H);
  double* ygu = (double*)malloc(sizeof(double) * G);
  double* h = (double*)malloc(sizeof(double) * I);
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int li = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (li >= J->n_list) break;
    int e = J->expert_list[li];
    /* Reconstruct this expert once and serve every pair routed to it. */
    if (eo_reconstruct(L->gu_code + (size_t)e * gu_words, H, G, L->k_gu, Wgu) ||
        eo_reconstruct(L->dn_code + (size_t)e * dn_words, I, H, L->k_dn, Wdn)) {
      J->status = -1;
      continue;
    }
    for (int p = 0; p < J->T * k; p++) {
      if (J->ids[p] != e) continue;
      int t = p / k;
      for (int c = 0; c < H; c++) x[c] = eo_bf16_to_double(J->x_bf16[(size_t)t * H + c]);
      eo_proj(Wgu, L->gu_rin + (size_t)e * H, L->gu_rout + (size_t)e * G, H, G, x, ygu);
      eo_swiglu(ygu, I, h);
      if (J->inter_out)
        for (int c = 0; c < I; c++) J->inter_out[(size_t)p * I + c] = h[c];
      eo_proj(Wdn, L->dn_rin + (size_t)e * I, L->dn_rout + (size_t)e * H, I, H, h,
              J->pair_out + (size_t)p * H);
    }
  }
  free(Wgu);
  free(Wdn);
  free(x);
  free(ygu);
  free(h);
  return NULL;
}

/*
 * y[t] = sum_j w[t][j] * down_e(SiLU(gate_e) * up_e)(x[t]) with e = ids[t][j],
 * summed in slot order. x bf16 bits [T][hidden]; ids [T][k]; w fp32 [T][k];
 * y double [T][hidden]; inter_out (nullable) double [T*k][inter] in pair
 * order; pair_out (nullable) double [T*k][hidden]. n_threads <= 0 uses every
 * online core. Returns 0, -1 on a bad shape, -2 on an expert id out of range.
 */
EO_EXPORT int eo_moe_layer(const eo_layer_t* L, const uint16_t* x_bf16, int T, const int32_t* ids,
                           const float* w, double* y, double* inter_out, double* pair_out_opt,
                           int n_threads) {
  int H = L->hidden, I = L->inter, k = L->top_k, E = L->n_experts;
  if (H % 128 || I % 128 || T < 0 || k <= 0) return -1;
  for (int p = 0; p < T * k; p++)
    if (ids[p] < 0 || ids[p] >= E) return -2;
  double* pair_out = pair_out_opt ? pair_out_opt : (double*)malloc(sizeof(double) * (size_t)T * k * H);
  int32_t* list = (int32_t*)malloc(sizeof(int32_t) * (E > 0 ? E : 1));
  int n_list = 0;
  for (int e = 0; e < E; e++) {
    for (int p = 0; p < T * k; p++) {
      if (ids[p] == e) {
        list[n_list++] = e;
        break;
      }
    }
  }
  eo_layer_job_t J;
  J.L = L;
  J.x_bf16 = x_bf16;
  J.T = T;
  J.ids = ids;
  J.expert_list = list;
  J.n_list = n_list;
  J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  J.pair_out = pair_out;
  J.inter_out = inter_out;
  J.status = 0;
  if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (n_threads > n_list) n_threads = n_list > 0 ? n_list : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * n_threads);
  for (int i = 0; i < n_threads; i++) pthread_create(&th[i], NULL, eo_layer_worker, &J);
  for (int i = 0; i < n_threads; i++) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  for (int t = 0; t < T; t++) {
    for (int c = 0; c < H; c++) {
      double acc = 0.0;
      for (int j = 0; j < k; j++)
        acc += (double)w[(size_t)t * k + j] * pair_out[((size_t)t * k + j) * H + c];
      y[(size_t)t * H + c] = acc;
    }
  }
  if (!pair_out_opt) free(pair_out);
  free(list);
  return J.status;
}

/*
 * One coded projection applied to T tokens of one expert (no routing):
 * code int16 [in/16][out/16][16K], rin/rout fp16 bits, x bf16 bits [T][in]
 * -> y double [T][out]. Returns 0 or -1 on a bad shape.
 */
EO_EXPORT int eo_expert_gemv(const uint16_t* code, const uint16_t* rin, const uint16_t* rout,
                             int in_f, int out_f, int K, const uint16_t* x_bf16, int T, double* y) {
  if (in_f % 128 || out_f % 128) return -1;
  uint16_t* W = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)out_f * in_f);
  double* x = (double*)malloc(sizeof(double) * in_f);
  int rc = eo_reconstruct(code, in_f, out_f, K, W);
  for (int t = 0; rc == 0 && t < T; t++) {
    for (int c = 0; c < in_f; c++) x[c] = eo_bf16_to_double(x_bf16[(size_t)t * in_f + c]);
    eo_proj(W, rin, rout, in_f, out_f, x, y + (size_t)t * out_f);
  }
  free(W);
  free(x);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Dense coded projections: the one-expert case, with additive biases.      */
/* ------------------------------------------------------------------------ */

/*
 * hipfire PR, commit notes on the dense export: every coded projection of an
 * Escha dense export carries an additive output bias, which no weight can
 * absorb; the gate and up biases are added before the SwiGLU, and the down
 * (and out_proj) bias lands on the output (the residual stream). A dense
 * linear is the routed path with one expert, id 0, weight 1. Reading D1:
 * the biases are f32 vectors added to the projection's output after rout
 * (the output side of the coded projection is rout (.) H_n(z)).
 * One projection: y[t] = proj(x[t]) + bias (bias may be NULL).
 */
EO_EXPORT int eo_dense_gemv(const uint16_t* code, const uint16_t* rin, const uint16_t* rout,
                            const float* bias, int in_f, int out_f, int K, const uint16_t* x_bf16,
                            int T, double* y) {
  int rc = eo_expert_gemv(code, rin, rout, in_f, out_f, K, x_bf16, T, y);
  if (rc || !bias) return rc;
  for (int t = 0; t < T; t++)
    for (int n = 0; n < out_f; n++) y[(size_t)t * out_f + n] += (double)bias[n];
  return 0;
}

/*
 * A dense MLP of coded projections: gu = gate_up(x) + gu_bias; g, u = the
 * first and second halves; h = SiLU(g) * u; y = down(h) + dn_bias. Biases
 * f32 (nullable). x bf16 bits [T][hidden]; y double [T][hidden]; h_out
 * (nullable) double [T][inter]. Returns 0 or -1 on a bad shape.
 */
EO_EXPORT int eo_dense_mlp(const uint16_t* gu_code, const uint16_t* gu_rin, const uint16_t* gu_rout,
                           const float* gu_bias, const uint16_t* dn_code, const uint16_t* dn_rin,
                           const uint16_t* dn_rout, const float* dn_bias, int hidden, int inter,
                           int k_gu, int k_dn, const uint16_t* x_bf16, int T, double* y,
                           double* h_out) {
  if (hidden % 128 || inter % 128 || T < 0) return -1;
  int G = 2 * inter;
  uint16_t* Wgu = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)G * hidden);
  uint16_t* Wdn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)hidden * inter);
  double* x = (double*)malloc(sizeof(double) * hidden);
  double* gu = (double*)malloc(sizeof(double) * G);
  double* h = (double*)malloc(sizeof(double) * inter);
  int rc = eo_reconstruct(gu_code, hidden, G, k_gu, Wgu);
  if (!rc) rc = eo_reconstruct(dn_code, inter, hidden, k_dn, Wdn);
  for (int t = 0; rc == 0 && t < T; t++) {
    for (int c = 0; c < hidden; c++) x[c] = eo_bf16_to_double(x_bf16[(size_t)t * hidden + c]);
    eo_proj(Wgu, gu_rin, gu_rout, hidden, G, x, gu);
    if (gu_bias)
      for (int c = 0; c < G; c++) gu[c] += (double)gu_bias[c];
    eo_swiglu(gu, inter, h);
    if (h_out)
      for (int c = 0; c < inter; c++) h_out[(size_t)t * inter + c] = h[c];
    double* yt = y + (size_t)t * hidden;
    eo_proj(Wdn, dn_rin, dn_rout, inter, hidden, h, yt);
    if (dn_bias)
      for (int c = 0; c < hidden; c++) yt[c] += (double)dn_bias[c];
  }
  free(Wgu);
  free(Wdn);
  free(x);
  free(gu);
  free(h);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* The shared expert: int8 weights with f32 group scales (w8a16) and its    */
/* fp16 gate.                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Model card "...-trellis-mlx", exactness table: the shared expert (like
 * the attention and embedding weights) is kept as int8 with f32 scales per
 * group of 128, and its dequantised weight is the f32 product scale * w8;
 * the activations are the 16-bit hidden state (w8a16). The router gates,
 * shared_expert_gate among them, are fp16. Readings (S1-S4 in the design
 * notes): weights int8 [out][in] with scales f32 [out][in/128], weight
 * (o, i) scaled by scales[o][i/128]; the product is rounded once to binary32
 * (it is what the f32 dequantisation computes) and everything after it is
 * exact here (fp64).
 */
EO_EXPORT double eo_q8_weight(int8_t q, float scale) {
  float w = scale * (float)q; /* one binary32 multiply, round to nearest even */
  return (double)w;
}

/* y[o] = sum_i w(o, i) x[i]: W int8 [out][in], scales f32 [out][in/128]. */
EO_EXPORT void eo_q8_linear(const int8_t* W, const float* scales, int in_f, int out_f,
                            const double* x, double* y) {
  int ng = in_f / 128;
  for (int o = 0; o < out_f; o++) {
    double acc = 0.0;
    for (int i = 0; i < in_f; i++)
      acc += eo_q8_weight(W[(size_t)o * in_f + i], scales[(size_t)o * ng + i / 128]) * x[i];
    y[o] = acc;
  }
}

/*
 * The shared expert of one token, added to the routed experts' output:
 *   gu = Wgu x (gate rows [0, inter), up rows [inter, 2 inter));
 *   h = SiLU(gate) * up;  s = Wdn h;
 *   g = sigmoid(gate_f16 . x);  out = g * s.
 * Reading S2: the shared_expert_gate (a single fp16 row over the hidden
 * state) scales the shared expert's output through a sigmoid before it is
 * added to the routed output, as the Qwen MoE blocks do; S3: the gate's dot
 * product is not rounded (unlike the router logits, for which the pages
 * state the f16 rounding). x bf16 bits [T][hidden]; out double [T][hidden];
 * gate_out (nullable) double [T] the sigmoid; h_out (nullable) double
 * [T][inter]. Returns 0, or -1 on a bad shape.
 */
EO_EXPORT int eo_shared_expert(const int8_t* gu_w, const float* gu_s, const int8_t* dn_w,
                               const float* dn_s, const uint16_t* gate_f16, int hidden, int inter,
                               const uint16_t* x_bf16, int T, double* out, double* gate_out,
                               double* h_out) {
  if (hidden % 128 || inter % 128 || hidden <= 0 || inter <= 0 || T < 0) return -1;
  double* x = (double*)malloc(sizeof(double) * hidden);
  double* gu = (double*)malloc(sizeof(double) * 2 * inter);
  double* h = (double*)malloc(sizeof(double) * inter);
  double* sh = (double*)malloc(sizeof(double) * hidden);
  for (int t = 0; t < T; t++) {
    for (int i = 0; i < hidden; i++) x[i] = eo_bf16_to_double(x_bf16[(size_t)t * hidden + i]);
    eo_q8_linear(gu_w, gu_s, hidden, 2 * inter, x, gu);
    eo_swiglu(gu, inter, h);
    eo_q8_linear(dn_w, dn_s, inter, hidden, h, sh);
    double logit = 0.0;
    for (int i = 0; i < hidden; i++) logit += eo_f16_to_double(gate_f16[i]) * x[i];
    double g = 1.0 / (1.0 + exp(-logit));
    for (int i = 0; i < hidden; i++) out[(size_t)t * hidden + i] = g * sh[i];
    if (gate_out) gate_out[t] = g;
    if (h_out)
      for (int c = 0; c < inter; c++) h_out[(size_t)t * inter + c] = h[c];
  }
  free(x);
  free(gu);
  free(h);
  free(sh);
  return 0;
}

/*
 * Between stacked layers: x' = bf16( v / sqrt(mean(v^2) + eps) ), unit
 * weight, no residual. y double [T][n] -> x_out bf16 bits [T][n].
 */
EO_EXPORT void eo_rmsnorm_bf16(const double* y, int T, int n, double eps, uint16_t* x_out) {
  for (int t = 0; t < T; t++) {
    const double* v = y + (size_t)t * n;
    double ss = 0.0;
    for (int c = 0; c < n; c++) ss += v[c] * v[c];
    double inv = 1.0 / sqrt(ss / n + eps);
    for (int c = 0; c < n; c++) x_out[(size_t)t * n + c] = eo_double_to_bf16_rne(v[c] * inv);
  }
}
