/*
 * CPU oracle for the MTP draft step. TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this file's library. The product path (the HIP library under
 * mtp_draft_head_02_amd/) never links, calls or includes anything here, and
 * nothing here includes or calls the product path.
 *
 * What it computes, and where each step comes from (pages are cited by title
 * and the item on the page):
 *   - one draft step of an MTP head: embedding row copy, RMSNorm of the
 *     embedding and of the target's final hidden, concat (embedding first),
 *     the fc projection [h, 2h], final RMSNorm, the draft lm_head GEMV over
 *     the first n_eff rows, argmax
 *       (deepseek_v4_mtp.rs, `forward_one` steps 1, 2, 6, 7; mtp_head.rs module
 *        doc "embed+hidden concat -> fc -> ... -> norm -> lm_head -> argmax";
 *        mtp_head/new.rs, the prefill scratch `embed, normed_embed,
 *        normed_hidden, concat, fc_out, normed2`)
 *   - the weight precisions BF16 / FP8 E4M3 / NVFP4
 *       (mtp_head.rs, `MtpQuantization`, `quantize_proj`, `gemv`)
 *   - the argmax tie rule: scan from index 0 with strict '>' starting at -inf
 *     with token 0, so the lowest index wins and NaN never wins
 *       (deepseek_v4_mtp.rs, `argmax_grammar_masked`)
 *   - BF16 decode: a BF16 is the upper 16 bits of an f32
 *       (deepseek_v4_mtp.rs, `argmax_grammar_masked`)
 *
 * The pages print no quantization recipe, no RMSNorm formula and no rounding
 * points. The readings taken here are listed with the functions below.
 *
 * Floating point: all sums and products are in double (fp64); the BF16 and
 * FP8/FP4 encoders round the exact value once, to nearest, ties to even. The
 * quantizers' scale arithmetic is IEEE f32 (single divisions and multiplies),
 * because the stored scales are f32 and the codes must be reproducible.
 * Build with no fast-math and no FP contraction.
 *
 * Parity status per function is stated at each function; every function here
 * is pinned by tests in tests/test_oracle_*.py except where it says
 * "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* BF16                                                                     */
/* ------------------------------------------------------------------------ */

/* BF16 -> value: the BF16 bits are the upper half of an IEEE f32
 * (deepseek_v4_mtp.rs, `argmax_grammar_masked`, the bf16 -> f32 step).
 * Pinned: closed form, all 65,536 patterns. */
ORACLE_API double oracle_bf16_decode(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round an exact value to the nearest multiple of 2^qexp, ties to even.
 * Returns the integer multiple. Used by every encoder below. The scaled value
 * a / 2^qexp is exact in double for every caller here (a is a double holding
 * an f32 or a product of short significands). */
static double round_half_even_multiple(double a, int qexp) {
  double m = ldexp(a, -qexp); /* exact: scaling by a power of two */
  double fl = floor(m);
  double frac = m - fl; /* exact */
  if (frac > 0.5) return fl + 1.0;
  if (frac < 0.5) return fl;
  /* exact tie: pick the even neighbour */
  return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* value -> BF16 bits, round to nearest, ties to even, with subnormals and
 * overflow to infinity (plain IEEE rounding into 1 sign, 8 exponent and 7
 * fraction bits). NaN -> canonical quiet NaN with the input's sign.
 * Pinned: torch's float32 -> bfloat16 conversion on random and boundary
 * values; exact ties. */
ORACLE_API uint16_t oracle_bf16_encode(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return sign | 0x7FC0u;
  double a = fabs(v);
  if (isinf(a)) return sign | 0x7F80u;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);      /* a = f * 2^e2, f in [0.5, 1) -> floor(log2 a) = e2 - 1 */
  int e = e2 - 1;
  if (e < -126) e = -126; /* subnormal range shares the smallest quantum */
  int qexp = e - 7;       /* 7 fraction bits */
  double r = round_half_even_multiple(a, qexp);
  double rv = ldexp(r, qexp);
  /* largest finite BF16 is (2 - 2^-7) * 2^127; anything that rounds above it
   * is infinity */
  if (rv > ldexp(255.0, 120)) return sign | 0x7F80u;
  if (r == 0.0) return sign;
  /* encode rv exactly */
  int re2;
  frexp(rv, &re2);
  int re = re2 - 1;
  if (re < -126) {
    /* subnormal: fraction = rv / 2^-133 */
    uint32_t frac = (uint32_t)ldexp(rv, 133);
    return sign | (uint16_t)frac;
  }
  uint32_t expf = (uint32_t)(re + 127);
  uint32_t frac = (uint32_t)(ldexp(rv, -re) * 128.0) - 128u;
  return sign | (uint16_t)((expf << 7) | frac);
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (OCP "E4M3FN": bias 7, no infinities, 0x7F/0xFF are NaN,       */
/* largest finite 448) and FP4 E2M1 (bias 1, values 0 0.5 1 1.5 2 3 4 6)     */
/* ------------------------------------------------------------------------ */

/* code -> value. Pinned: closed form over all 256 codes. */
ORACLE_API double oracle_e4m3_decode(uint8_t code) {
  double s = (code & 0x80u) ? -1.0 : 1.0;
  int ef = (code >> 3) & 0xF;
  int mf = code & 0x7;
  if (ef == 0xF && mf == 0x7) return NAN;
  if (ef == 0) return s * ldexp((double)mf, -9); /* subnormal: m/8 * 2^-6 */
  return s * ldexp(8.0 + mf, ef - 7 - 3);
}

/* code -> value. Pinned: closed form over all 16 codes. */
ORACLE_API double oracle_e2m1_decode(uint8_t code) {
  double s = (code & 0x8u) ? -1.0 : 1.0;
  int ef = (code >> 1) & 0x3;
  int mf = code & 0x1;
  if (ef == 0) return s * 0.5 * mf; /* subnormal: m/2 * 2^0 */
  return s * ldexp(2.0 + mf, ef - 1 - 1);
}

/* f32 -> E4M3: round to nearest with ties to the even code, saturate to the
 * largest finite value (448, also for infinities), keep the input's sign bit
 * (so a negative value that rounds to zero gives 0x80), keep subnormals.
 * NaN -> 0x7F with the input's sign. The pages name the FP8 quantizer but print
 * no rounding rule; this is the plainest reading (OCP FP8 satfinite).
 * Pinned: brute-force nearest search over the 127 finite magnitudes; hand
 * table. */
ORACLE_API uint8_t oracle_e4m3_encode(float v) {
  uint8_t sign = signbit(v) ? 0x80u : 0u;
  if (isnan(v)) return sign | 0x7Fu;
  double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7Eu;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);
  int e = e2 - 1;
  if (e < -6) e = -6; /* subnormals share the quantum 2^-9 */
  int qexp = e - 3;   /* 3 mantissa bits */
  double r = round_half_even_multiple(a, qexp);
  double rv = ldexp(r, qexp); /* <= 448 since a < 448 */
  if (rv == 0.0) return sign;
  int re2;
  frexp(rv, &re2);
  int re = re2 - 1;
  if (re < -6) return sign | (uint8_t)ldexp(rv, 9); /* subnormal code = m */
  uint8_t ef = (uint8_t)(re + 7);
  uint8_t mf = (uint8_t)(ldexp(rv, -re) * 8.0 - 8.0);
  return sign | (uint8_t)(ef << 3) | mf;
}

/* f32 -> E2M1, same rules as the E4M3 encoder: nearest, ties to even code,
 * saturate to 6, sign kept, NaN -> 0x7 with sign (E2M1 has no NaN; the
 * quantizer below never feeds it one). Pinned: brute force over the 8
 * magnitudes; hand table. */
ORACLE_API uint8_t oracle_e2m1_encode(float v) {
  uint8_t sign = signbit(v) ? 0x8u : 0u;
  if (isnan(v)) return sign | 0x7u;
  double a = fabs((double)v);
  if (a >= 6.0) return sign | 0x7u;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);
  int e = e2 - 1;
  if (e < 0) e = 0;  /* subnormal quantum 0.5 */
  int qexp = e - 1;  /* 1 mantissa bit */
  double r = round_half_even_multiple(a, qexp);
  double rv = ldexp(r, qexp);
  if (rv >= 6.0) return sign | 0x7u;
  if (rv == 0.0) return sign;
  int re2;
  frexp(rv, &re2);
  int re = re2 - 1;
  if (re < 0) return sign | 0x1u; /* 0.5 */
  uint8_t ef = (uint8_t)(re + 1);
  uint8_t mf = (uint8_t)(ldexp(rv, -re) * 2.0 - 2.0);
  return sign | (uint8_t)(ef << 1) | mf;
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver. Threads split rows statically; every row is still    */
/* computed by the same sequential function, so results do not depend on     */
/* the thread count.                                                         */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void *ctx, int64_t r0, int64_t r1);
struct row_job {
  row_fn fn;
  void *ctx;
  int64_t r0, r1;
};
static void *row_job_main(void *p) {
  struct row_job *j = (struct row_job *)p;
  j->fn(j->ctx, j->r0, j->r1);
  return NULL;
}
static void for_rows(int64_t n, int threads, row_fn fn, void *ctx) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads == 1 || n < 2 * threads) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t tid[256];
  struct row_job jobs[256];
  int started = 0;
  for (int t = 0; t < threads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].r0 = n * t / threads;
    jobs[t].r1 = n * (t + 1) / threads;
    if (pthread_create(&tid[t], NULL, row_job_main, &jobs[t]) == 0) {
      started = t + 1;
    } else {
      /* could not start a thread: do the rest inline */
      fn(ctx, jobs[t].r0, n);
      break;
    }
  }
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* FP8 weight quantization, per-row f32 scale                               */
/* ------------------------------------------------------------------------ */
/* The pages quantize a BF16 [n, k] weight to FP8 at load (mtp_head.rs,
 * `quantize_proj`; glm5next_mtp_head/init.rs, the draft-head shard quantised to
 * FP8, rows only) and keep a per-row scale (mtp_head.rs, `gemv`, the
 * `row_scale` argument). The recipe is not printed. Reading taken:
 *   a_r = max_k |W[r,k]|            (exact)
 *   s_r = f32(a_r / 448)            (IEEE f32 division; 448 = E4M3 max)
 *   s_r = 1 when a_r == 0
 *   q[r,k] = E4M3(f32(W[r,k] / s_r)) (IEEE f32 division, then the encoder)
 * Dequantized weight: e4m3(q) * s_r.
 * Pinned: zero row, single-nonzero row, absmax-448 row (codes = the encoder's
 * hand table), subnormal-BF16 row, absmax element encodes to +-448, error bound. */
struct q8_ctx {
  const uint16_t *w;
  int64_t k;
  uint8_t *codes;
  float *scale;
};
static float bf16_to_f32(uint16_t b) { return (float)oracle_bf16_decode(b); }
static void q8_rows(void *p, int64_t r0, int64_t r1) {
  struct q8_ctx *c = (struct q8_ctx *)p;
  for (int64_t r = r0; r < r1; ++r) {
    const uint16_t *row = c->w + r * c->k;
    float a = 0.0f;
    for (int64_t i = 0; i < c->k; ++i) {
      float v = fabsf(bf16_to_f32(row[i]));
      if (v > a) a = v;
    }
    float s = a / 448.0f; /* f32 division */
    float sr = (a == 0.0f) ? 1.0f : s;
    c->scale[r] = sr;
    for (int64_t i = 0; i < c->k; ++i) {
      float q = bf16_to_f32(row[i]) / sr;
      c->codes[r * c->k + i] = oracle_e4m3_encode(q);
    }
  }
}
ORACLE_API void oracle_quantize_fp8(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes,
                                    float *row_scale, int threads) {
  struct q8_ctx c = {w, k, codes, row_scale};
  for_rows(n, threads, q8_rows, &c);
}

/* ------------------------------------------------------------------------ */
/* NVFP4 weight quantization                                                */
/* ------------------------------------------------------------------------ */
/* The pages run two kernels, a global-absmax pass and the BF16 -> NVFP4
 * quantizer (mtp_head/new.rs, `nvfp4_global_absmax`, `quantize_bf16_to_nvfp4`;
 * mtp_head.rs, `quantize_proj`), store 0.5 B per weight (`MtpQuantization`) and
 * print no recipe. Reading taken (the published two-level NVFP4 form with
 * 16-element blocks, decode-side scales):
 *   G   = max |W| over the whole matrix (exact)
 *   s_g = f32(G / 2688), 2688 = 6 * 448;  s_g = 1 when G == 0
 *   d   = f32(6 * s_g)
 *   per block of 16 along k:   a = max |w|;  sb = E4M3(f32(a / d));
 *                              S = f32(e4m3(sb) * s_g)
 *   per element:               q = E2M1(f32(w / S)),  or signbit(w) << 3 if S == 0
 *   packing: element 2j in the low nibble of byte j, 2j+1 in the high nibble;
 *   block scales row-major [n, k/16].
 * Dequantized weight: e2m1(q) * e4m3(sb) * s_g.
 * Every f32 step is one IEEE operation on f32 operands: s_g and d are rounded
 * before use, a / d and w / S are single f32 divisions.
 * Pinned: the hand example with G = 2688 (s_g = 1); two hand-worked examples
 * with s_g = f32(13/14) and f32(11/12), whose blocks put a / d and w / S on or
 * within an f32 ulp of an encoder tie (tests/golden/nvfp4_example_sg.txt); a
 * brute-force nearest-code search over every block of random heads with
 * outliers and of those examples at power-of-two scalings; the block holding
 * G gets sb = 0x7E and +-G encodes to 0x7/0xF; error bound. */
struct q4_ctx {
  const uint16_t *w;
  int64_t k;
  float sg; /* f32(G / 2688), the stored global scale */
  float d;  /* f32(6 * sg): from the rounded global scale */
  uint8_t *codes;
  uint8_t *bscale;
};
static void q4_rows(void *p, int64_t r0, int64_t r1) {
  struct q4_ctx *c = (struct q4_ctx *)p;
  const float d = c->d;
  for (int64_t r = r0; r < r1; ++r) {
    const uint16_t *row = c->w + r * c->k;
    for (int64_t b0 = 0; b0 < c->k; b0 += 16) {
      float a = 0.0f;
      for (int i = 0; i < 16; ++i) {
        float v = fabsf(bf16_to_f32(row[b0 + i]));
        if (v > a) a = v;
      }
      float ad = a / d; /* f32 division */
      uint8_t sb = oracle_e4m3_encode(ad);
      c->bscale[r * (c->k / 16) + b0 / 16] = sb;
      float S = (float)oracle_e4m3_decode(sb) * c->sg; /* f32 multiply */
      for (int i = 0; i < 16; ++i) {
        float w = bf16_to_f32(row[b0 + i]);
        uint8_t q;
        if (S == 0.0f) {
          q = signbit(w) ? 0x8u : 0x0u;
        } else {
          float t = w / S; /* f32 division */
          q = oracle_e2m1_encode(t);
        }
        int64_t byte = r * (c->k / 2) + (b0 + i) / 2;
        if (((b0 + i) & 1) == 0)
          c->codes[byte] = (uint8_t)((c->codes[byte] & 0xF0u) | q);
        else
          c->codes[byte] = (uint8_t)((c->codes[byte] & 0x0Fu) | (uint8_t)(q << 4));
      }
    }
  }
}
/* Exact max |W| over all rows: per-row maxima (row-parallel), then one
 * sequential max. max is exact, so the order does not matter. */
struct amax_ctx {
  const uint16_t *w;
  int64_t k;
  float *row_max;
};
static void amax_rows(void *p, int64_t r0, int64_t r1) {
  struct amax_ctx *c = (struct amax_ctx *)p;
  for (int64_t r = r0; r < r1; ++r) {
    float a = 0.0f;
    for (int64_t i = 0; i < c->k; ++i) {
      float v = fabsf(bf16_to_f32(c->w[r * c->k + i]));
      if (v > a) a = v;
    }
    c->row_max[r] = a;
  }
}
ORACLE_API float oracle_global_absmax(const uint16_t *w, int64_t n, int64_t k, int threads) {
  float *rm = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  struct amax_ctx c = {w, k, rm};
  for_rows(n, threads, amax_rows, &c);
  float G = 0.0f;
  for (int64_t r = 0; r < n; ++r)
    if (rm[r] > G) G = rm[r];
  free(rm);
  return G;
}
ORACLE_API void oracle_quantize_nvfp4(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes,
                                      uint8_t *block_scale, float *global_scale, int threads) {
  float G = oracle_global_absmax(w, n, k, threads);
  float sg = G / 2688.0f; /* f32 division */
  float s = (G == 0.0f) ? 1.0f : sg;
  float d = 6.0f * s;     /* f32 multiply of the rounded global scale */
  *global_scale = s;
  struct q4_ctx c = {w, k, s, d, codes, block_scale};
  for_rows(n, threads, q4_rows, &c);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm, combiner, final norm                                             */
/* ------------------------------------------------------------------------ */

/* y_i = bf16( v_i * r * (gamma_i + gamma_offset) ), r = 1/sqrt(mean(v^2) + eps).
 * Gamma convention: the shared norm kernel applies (1 + w), the vanilla one
 * plain w (deepseek_v4_mtp.rs, the comment on `rms_norm_k`); gamma_offset is
 * 1 or 0 respectively. eps enters as in the standard RMSNorm (the pages pass
 * only `rms_norm_eps`, deepseek_v4_mtp.rs `forward_one`). Output rounded to
 * BF16 like the pages' BF16 norm buffers (mtp_head/new.rs prefill scratch).
 * Pinned: exact rational arithmetic on small h; scale invariance. */
ORACLE_API void oracle_rms_norm(const uint16_t *v, const uint16_t *gamma, int64_t h, float eps,
                                float gamma_offset, uint16_t *out) {
  double ss = 0.0;
  for (int64_t i = 0; i < h; ++i) {
    double x = oracle_bf16_decode(v[i]);
    ss += x * x;
  }
  double ms = ss / (double)h;
  double r = 1.0 / sqrt(ms + (double)eps);
  for (int64_t i = 0; i < h; ++i) {
    double g = oracle_bf16_decode(gamma[i]) + (double)gamma_offset;
    out[i] = oracle_bf16_encode(oracle_bf16_decode(v[i]) * r * g);
  }
}

/* One draft step's input side for b batch rows (the "combine"):
 *   e_b  = E[t_b]                                (row copy of the shared table)
 *   c_b  = [ rms(e_b, g_e) || rms(h_b, g_h) ]    (BF16, embedding first)
 *   u_b  = bf16( W_fc . c_b ),  W_fc [h, 2h] row-major
 *   x_b  = rms(u_b, g_f)                         (BF16)
 * Sources: deepseek_v4_mtp.rs `forward_one` steps 1-2 and 6 (embedding copy at
 * token * row bytes; two norms; final norm); mtp_head.rs module doc (concat ->
 * fc); mtp_head/new.rs (`fc=[h, 2h]` in the head summary, prefill scratch
 * order embed, normed_embed, normed_hidden, concat [c, 2h], fc_out, normed2).
 * The decoder layer between fc and the final norm is identity here.
 * Writes x [b, h]; if c_out/u_out are not NULL also the intermediates.
 * Pinned: c, u and x each against exact rational arithmetic on small shapes;
 * followed by the lm_head argmax, on a case whose token is known in closed
 * form (a planted peak carried through an fc that selects the hidden half). */
ORACLE_API void oracle_draft_combine(const uint16_t *embed_table, int64_t vocab,
                                     const int32_t *token_ids, const uint16_t *target_hidden,
                                     const uint16_t *gamma_embed, const uint16_t *gamma_hidden,
                                     const uint16_t *fc_w, const uint16_t *gamma_final, int64_t b,
                                     int64_t h, float eps, float gamma_offset, uint16_t *x_out,
                                     uint16_t *c_out, uint16_t *u_out) {
  (void)vocab;
  uint16_t *c = (uint16_t *)malloc((size_t)(2 * h) * sizeof(uint16_t));
  uint16_t *u = (uint16_t *)malloc((size_t)h * sizeof(uint16_t));
  for (int64_t bi = 0; bi < b; ++bi) {
    const uint16_t *e = embed_table + (int64_t)token_ids[bi] * h;
    oracle_rms_norm(e, gamma_embed, h, eps, gamma_offset, c);
    oracle_rms_norm(target_hidden + bi * h, gamma_hidden, h, eps, gamma_offset, c + h);
    for (int64_t j = 0; j < h; ++j) {
      double acc = 0.0;
      const uint16_t *wr = fc_w + j * 2 * h;
      for (int64_t i = 0; i < 2 * h; ++i)
        acc += oracle_bf16_decode(wr[i]) * oracle_bf16_decode(c[i]);
      u[j] = oracle_bf16_encode(acc);
    }
    oracle_rms_norm(u, gamma_final, h, eps, gamma_offset, x_out + bi * h);
    if (c_out) memcpy(c_out + bi * 2 * h, c, (size_t)(2 * h) * sizeof(uint16_t));
    if (u_out) memcpy(u_out + bi * h, u, (size_t)h * sizeof(uint16_t));
  }
  free(c);
  free(u);
}

/* ------------------------------------------------------------------------ */
/* Draft lm_head: logits, tolerance, argmax                                  */
/* ------------------------------------------------------------------------ */

enum { ORACLE_W_BF16 = 0, ORACLE_W_FP8 = 1, ORACLE_W_NVFP4 = 2 };

/* Dequantized weight w[r, i] for the three precisions. All products here are
 * exact in double (at most 2 + 4 + 24 significant bits). */
static double dequant(int wd, const void *w, const void *scale, const float *gscale, int64_t h,
                      int64_t r, int64_t i) {
  if (wd == ORACLE_W_BF16) return oracle_bf16_decode(((const uint16_t *)w)[r * h + i]);
  if (wd == ORACLE_W_FP8)
    return oracle_e4m3_decode(((const uint8_t *)w)[r * h + i]) * (double)((const float *)scale)[r];
  uint8_t byte = ((const uint8_t *)w)[r * (h / 2) + i / 2];
  uint8_t q = (i & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
  uint8_t sb = ((const uint8_t *)scale)[r * (h / 16) + i / 16];
  return oracle_e2m1_decode(q) * oracle_e4m3_decode(sb) * (double)gscale[0];
}

struct lm_ctx {
  int wd;
  const void *w;
  const void *scale;
  const float *gscale;
  const uint16_t *x;
  int64_t b, h, n;
  double *logits;
  double *tau;
};
static void lm_rows(void *p, int64_t r0, int64_t r1) {
  struct lm_ctx *c = (struct lm_ctx *)p;
  for (int64_t r = r0; r < r1; ++r) {
    for (int64_t bi = 0; bi < c->b; ++bi) {
      double acc = 0.0, mag = 0.0;
      for (int64_t i = 0; i < c->h; ++i) {
        double t = dequant(c->wd, c->w, c->scale, c->gscale, c->h, r, i) *
                   oracle_bf16_decode(c->x[bi * c->h + i]);
        acc += t;
        mag += fabs(t);
      }
      c->logits[bi * c->n + r] = acc;
      if (c->tau) c->tau[bi * c->n + r] = 1e-3 * mag;
    }
  }
}

/* L[b, r] = sum_i w^[r, i] * x[b, i] for r < n_eff, in double, and optionally
 * tau[b, r] = 1e-3 * sum_i |w^[r, i] * x[b, i]| (the logit tolerance).
 * n_eff = min(mtp_vocab_size, vocab) when mtp_vocab_size > 0, else vocab
 * (deepseek_v4_mtp.rs `forward_one` step 6; mtp_head/new.rs `effective_vocab`).
 * The lm_head is a GEMV over v rows of a [vocab, hidden] weight with rows
 * packed at hidden (glm5next_mtp_head/init.rs draft-head comment).
 * Pinned: exact rational sums on small shapes; planted rows. */
ORACLE_API int64_t oracle_effective_vocab(int64_t vocab, int64_t mtp_vocab_size) {
  return (mtp_vocab_size > 0 && mtp_vocab_size < vocab) ? mtp_vocab_size : vocab;
}
ORACLE_API void oracle_lmhead_logits(const uint16_t *x, int64_t b, int64_t h, int wd,
                                     const void *w, const void *scale, const float *gscale,
                                     int64_t n_eff, double *logits, double *tau, int threads) {
  struct lm_ctx c = {wd, w, scale, gscale, x, b, h, n_eff, logits, tau};
  for_rows(n_eff, threads, lm_rows, &c);
}

/* Index of the maximum: start at -inf with token 0, scan from 0 upward, take
 * an element only if strictly greater (deepseek_v4_mtp.rs,
 * `argmax_grammar_masked`). Lowest index wins ties; NaN never wins; an all
 * -inf/NaN row gives 0. Pinned: planted maxima, duplicates, permutations,
 * prefixes. */
ORACLE_API int32_t oracle_argmax(const double *v, int64_t n) {
  int32_t best = 0;
  double bv = -INFINITY;
  for (int64_t i = 0; i < n; ++i)
    if (v[i] > bv) {
      bv = v[i];
      best = (int32_t)i;
    }
  return best;
}

/* The whole lm_head + argmax for b rows: token[b] and optionally the logits
 * (caller-sized [b, n_eff]). Returns n_eff. */
ORACLE_API int64_t oracle_lmhead_argmax(const uint16_t *x, int64_t b, int64_t h, int wd,
                                        const void *w, const void *scale, const float *gscale,
                                        int64_t vocab, int64_t mtp_vocab_size, int32_t *token_out,
                                        double *logits_out, int threads) {
  int64_t n = oracle_effective_vocab(vocab, mtp_vocab_size);
  double *lg = logits_out ? logits_out : (double *)malloc((size_t)(b * n) * sizeof(double));
  oracle_lmhead_logits(x, b, h, wd, w, scale, gscale, n, lg, NULL, threads);
  for (int64_t bi = 0; bi < b; ++bi) token_out[bi] = oracle_argmax(lg + bi * n, n);
  if (!logits_out) free(lg);
  return n;
}

/* ------------------------------------------------------------------------ */
/* Top-1 log-probability and the grammar-masked argmax                       */
/* ------------------------------------------------------------------------ */

/* log-probability of the top-1 token under the softmax of one row of logits:
 *   logp = max_i v_i - log sum_i exp(v_i)  =  -log sum_i exp(v_i - max_i v_i)
 * over all n entries (the argmax's domain). The pages emit each row's top-1
 * log-probability next to the argmax, and keep the chain confidence of a
 * propose as the minimum top-1 softmax probability exp(logp) over its drafts
 * (mtp_head.rs, the fields `argmax_batch_lp_k` and `last_conf_bits`). The
 * formula itself is not printed; this is the definition of those words.
 * Reading for non-finite input: a NaN anywhere, or no entry above -inf, gives
 * NaN; -inf entries add nothing. Sum in double, in index order.
 * Pinned: closed forms (uniform, two-point), shift invariance, a 50-digit
 * decimal brute force on small rows. */
ORACLE_API double oracle_top1_logprob(const double *v, int64_t n) {
  double m = -INFINITY;
  for (int64_t i = 0; i < n; ++i) {
    if (isnan(v[i])) return NAN;
    if (v[i] > m) m = v[i];
  }
  if (m == -INFINITY) return NAN;
  double sum = 0.0;
  for (int64_t i = 0; i < n; ++i) sum += exp(v[i] - m);
  return -log(sum);
}

/* Argmax over the entries a grammar bitmask allows: entry i is allowed when
 * word i / 32 exists (i / 32 < mask_words) and its bit i % 32 is set; among
 * allowed entries, scan upward from -inf with token 0 taking only strictly
 * greater values. *any_allowed is 1 if at least one entry is allowed, else 0
 * (and the token is 0). As on the pages, an allowed set whose values are all
 * -inf or NaN also gives token 0 (deepseek_v4_mtp.rs, `argmax_grammar_masked`).
 * Pinned: the full mask equals the plain argmax; empty and short masks; a
 * single allowed entry; masking out the maximum; ties among allowed entries;
 * bit 31 of a word. */
ORACLE_API int32_t oracle_argmax_masked(const double *v, int64_t n, const int32_t *mask,
                                        int64_t mask_words, int32_t *any_allowed) {
  int32_t best = 0;
  double bv = -INFINITY;
  int32_t any = 0;
  for (int64_t i = 0; i < n; ++i) {
    int64_t wi = i / 32;
    if (wi >= mask_words) break;
    if ((((uint32_t)mask[wi]) >> (i % 32) & 1u) == 0u) continue;
    any = 1;
    if (v[i] > bv) {
      bv = v[i];
      best = (int32_t)i;
    }
  }
  if (any_allowed) *any_allowed = any;
  return best;
}

/* ------------------------------------------------------------------------ */
/* Combiner variants                                                         */
/* ------------------------------------------------------------------------ */

/* The combine of oracle_draft_combine with the fc weight stored in any of the
 * three precisions (BF16 / FP8 per-row scale / NVFP4, same layouts and
 * dequantization as the lm_head): u_b[j] = bf16(sum_i fc^[j, i] c_b[i]). The
 * pages quantize the head's projections, the fc among them, to the head's
 * precision at load (mtp_head/new.rs: the fc [h, 2h] goes through the same
 * quantizer as the other projections; mtp_head.rs `quantize_proj`).
 * Pinned: with weights every precision represents exactly, equal to the BF16
 * combine; exact rational fc on small h. */
ORACLE_API void oracle_draft_combine_q(const uint16_t *embed_table, const int32_t *token_ids,
                                       const uint16_t *target_hidden, const uint16_t *gamma_embed,
                                       const uint16_t *gamma_hidden, int fc_wd, const void *fc,
                                       const void *fc_scale, const float *fc_gscale,
                                       const uint16_t *gamma_final, int64_t b, int64_t h, float eps,
                                       float gamma_offset, uint16_t *x_out, uint16_t *u_out) {
  uint16_t *c = (uint16_t *)malloc((size_t)(2 * h) * sizeof(uint16_t));
  uint16_t *u = (uint16_t *)malloc((size_t)h * sizeof(uint16_t));
  for (int64_t bi = 0; bi < b; ++bi) {
    oracle_rms_norm(embed_table + (int64_t)token_ids[bi] * h, gamma_embed, h, eps, gamma_offset, c);
    oracle_rms_norm(target_hidden + bi * h, gamma_hidden, h, eps, gamma_offset, c + h);
    for (int64_t j = 0; j < h; ++j) {
      double acc = 0.0;
      for (int64_t i = 0; i < 2 * h; ++i)
        acc += dequant(fc_wd, fc, fc_scale, fc_gscale, 2 * h, j, i) * oracle_bf16_decode(c[i]);
      u[j] = oracle_bf16_encode(acc);
    }
    oracle_rms_norm(u, gamma_final, h, eps, gamma_offset, x_out + bi * h);
    if (u_out) memcpy(u_out + bi * h, u, (size_t)h * sizeof(uint16_t));
  }
  free(c);
  free(u);
}

/* The split combiner of the DeepSeek-V4 MTP step: two h x h projections, each
 * GEMV output rounded to BF16, then a BF16 residual add:
 *   u_b[j] = bf16( bf16(e_proj[j, :] . rms(e_b)) + bf16(h_proj[j, :] . rms(h_b)) )
 * (deepseek_v4_mtp.rs `forward_one` step 2: the embedding branch into h_in, the
 * hidden branch into a temp, `bf16_residual_add` h_in += temp). The same linear
 * map as the concat form with fc = [e_proj | h_proj], rounded at two more
 * points. x_b = rms(u_b, g_f) as in the concat form.
 * Pinned: exact rational GEMVs on small h; equal to the concat form where
 * both branch sums are exact in BF16; a zero branch. */
ORACLE_API void oracle_draft_combine_split(const uint16_t *embed_table, const int32_t *token_ids,
                                           const uint16_t *target_hidden, const uint16_t *gamma_embed,
                                           const uint16_t *gamma_hidden, const uint16_t *e_proj,
                                           const uint16_t *h_proj, const uint16_t *gamma_final,
                                           int64_t b, int64_t h, float eps, float gamma_offset,
                                           uint16_t *x_out, uint16_t *u_out) {
  uint16_t *ne = (uint16_t *)malloc((size_t)h * sizeof(uint16_t));
  uint16_t *nh = (uint16_t *)malloc((size_t)h * sizeof(uint16_t));
  uint16_t *u = (uint16_t *)malloc((size_t)h * sizeof(uint16_t));
  for (int64_t bi = 0; bi < b; ++bi) {
    oracle_rms_norm(embed_table + (int64_t)token_ids[bi] * h, gamma_embed, h, eps, gamma_offset, ne);
    oracle_rms_norm(target_hidden + bi * h, gamma_hidden, h, eps, gamma_offset, nh);
    for (int64_t j = 0; j < h; ++j) {
      double se = 0.0, sh = 0.0;
      for (int64_t i = 0; i < h; ++i) {
        se += oracle_bf16_decode(e_proj[j * h + i]) * oracle_bf16_decode(ne[i]);
        sh += oracle_bf16_decode(h_proj[j * h + i]) * oracle_bf16_decode(nh[i]);
      }
      double be = oracle_bf16_decode(oracle_bf16_encode(se));
      double bh = oracle_bf16_decode(oracle_bf16_encode(sh));
      u[j] = oracle_bf16_encode(be + bh);
    }
    oracle_rms_norm(u, gamma_final, h, eps, gamma_offset, x_out + bi * h);
    if (u_out) memcpy(u_out + bi * h, u, (size_t)h * sizeof(uint16_t));
  }
  free(ne);
  free(nh);
  free(u);
}

/* out[i] = encode(f32 with bit pattern first_bits + i), i < count, with the
 * encoders above (codec 0: E4M3, 1: E2M1, one byte each; 2: BF16, two bytes
 * each, out read as uint16_t [count]). Used to compare every f32 pattern with
 * another encoder. Pinned through the encoders' own pins. */
struct enc_ctx {
  int codec;
  uint32_t first;
  uint8_t *out;
};
static void enc_rows(void *p, int64_t r0, int64_t r1) {
  struct enc_ctx *c = (struct enc_ctx *)p;
  for (int64_t i = r0; i < r1; ++i) {
    uint32_t u = c->first + (uint32_t)i;
    float f;
    memcpy(&f, &u, sizeof f);
    if (c->codec == 2)
      ((uint16_t *)c->out)[i] = oracle_bf16_encode((double)f);
    else
      c->out[i] = c->codec == 0 ? oracle_e4m3_encode(f) : oracle_e2m1_encode(f);
  }
}
ORACLE_API void oracle_encode_range(int codec, uint32_t first_bits, int64_t count, uint8_t *out,
                                    int threads) {
  struct enc_ctx c = {codec, first_bits, out};
  for_rows(count, threads, enc_rows, &c);
}
