/*
 * mtp_draft.h -- C ABI of the MTP draft-step library (libmtpdraft.so, gfx950).
 *
 * One draft step of a multi-token-prediction (MTP) head, the part that runs on
 * every propose: embed the previous token, RMSNorm it and the target model's
 * final hidden state, concatenate (embedding first), project through fc
 * [h, 2h], RMSNorm again, sweep the draft lm_head [vocab, h] (BF16, FP8 E4M3
 * with a per-row f32 scale, or NVFP4) and take the argmax. Plus the load-time
 * weight quantizers. The pages this follows are cited by title and item:
 *   - deepseek_v4_mtp.rs, module doc and `forward_one` (the draft step: embed,
 *     two norms, combiner, final norm, lm_head over v rows, argmax, 4-byte read
 *     back), `argmax_grammar_masked` (tie rule, BF16 decode);
 *   - mtp_head.rs (spark_model/layers), module doc ("embed+hidden concat -> fc
 *     -> ... -> norm -> lm_head -> argmax"), `MtpQuantization`, `gemv`,
 *     `quantize_proj`, the `draft_token_id_dev` field (deferred read back),
 *     `mtp_vocab_size` (0 = full vocab);
 *   - mtp_head/new.rs, `MtpHead::new` (quantizer kernels, `fc=[h, 2h]`,
 *     `effective_vocab`);
 *   - glm5next_mtp_head/init.rs, the draft-head comment (the sweep over
 *     [vocab, hidden] is most of the drafter's time; rows packed at hidden).
 *
 * Conventions for every call below:
 *   - Pointers are DEVICE pointers unless marked [host]. BF16 values are passed
 *     as uint16_t bit patterns. `stream` is a hipStream_t (NULL = the default
 *     stream).
 *   - Every call validates all arguments on the host first. On any error it
 *     returns the status, enqueues nothing and leaves every output untouched.
 *     On success it enqueues its kernels on `stream` and returns without
 *     synchronizing: results are ready when the stream reaches that point.
 *   - The caller owns every buffer, including workspaces. The library allocates
 *     no device memory; its only state is a per-device cache of device
 *     attributes and kernel occupancies (thread-safe), and the fixed scratch
 *     array of mtp_draft_step_noalloc (part of the loaded code object).
 *   - Arrays are dense and row-major. Bulk arrays (weights, codes, block scales,
 *     activations, outputs, workspaces) must be 16-byte aligned; f32 scales,
 *     token ids and logits 4-byte aligned. Output ranges must not overlap any
 *     input range or each other.
 *   - Workspaces of mtp_draft_combine and mtp_lmhead_argmax must be
 *     zero-filled before their first use. Each call leaves its workspace ready
 *     for the next call (the completion counter in its first bytes is back at
 *     zero when the call's kernels complete), so one zero fill at allocation is
 *     enough. Calls that can run at the same time (different streams) must not
 *     share a workspace.
 */
#ifndef MTP_DRAFT_H
#define MTP_DRAFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTP_ABI_VERSION 1

/* Exported symbols of libmtpdraft.so (the library builds with hidden default
 * visibility). */
#if defined(__GNUC__) || defined(__clang__)
#define MTP_API __attribute__((visibility("default")))
#else
#define MTP_API
#endif

typedef enum {
  MTP_OK = 0,
  MTP_ERR_NULL = 1,      /* a required pointer is NULL */
  MTP_ERR_SHAPE = 2,     /* a size is out of range or not a required multiple */
  MTP_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  MTP_ERR_DTYPE = 4,     /* unknown weight or codec kind, or a scale given/missing */
  MTP_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the query result */
  MTP_ERR_OVERLAP = 6,   /* an output range overlaps an input or another output */
  MTP_ERR_HIP = 7,       /* the HIP runtime refused a launch or attribute call */
  MTP_ERR_RANGE = 8      /* a token id is outside [0, vocab) */
} mtp_status;

/* Weight precision of the draft lm_head (mtp_head.rs, `MtpQuantization`:
 * NVFP4 0.5 B/weight, FP8 1 B/weight, BF16 2 B/weight). */
typedef enum {
  MTP_W_BF16 = 0,          /* w: BF16 [vocab, h]; scale, gscale: NULL */
  MTP_W_FP8_E4M3_ROW = 1,  /* w: E4M3 codes u8 [vocab, h]; scale: f32 [vocab]; gscale: NULL */
  MTP_W_NVFP4 = 2          /* w: E2M1 pairs u8 [vocab, h/2] (element 2j in the low nibble of
                              byte j); scale: E4M3 u8 [vocab, h/16] (one per 16 elements);
                              gscale: f32 [1] */
} mtp_wdtype;

/* Codecs exposed by mtp_codec_encode_range (verification of the on-device
 * encoders used by the quantizers, and of the BF16 rounding of the RMSNorms). */
typedef enum {
  MTP_CODEC_E4M3 = 0, /* f32 -> OCP E4M3FN, nearest, ties to even, satfinite, sign kept */
  MTP_CODEC_E2M1 = 1, /* f32 -> E2M1, nearest, ties to even, satfinite (6), sign kept */
  MTP_CODEC_BF16 = 2  /* f32 -> BF16, nearest, ties to even, subnormals kept, overflow to
                         infinity; a NaN stays NaN with its sign and upper payload bits,
                         quieted (bit 6 of the BF16 set). The packed converter that the
                         normalize passes round their outputs with. */
} mtp_codec;

/* ABI version of the loaded library (MTP_ABI_VERSION at build time). */
MTP_API int mtp_abi_version(void);

/* Static, human-readable text for a status value (never NULL). */
MTP_API const char *mtp_status_string(int status);

/* ---------------------------------------------------------------------------
 * FP8 weight quantization with a per-row f32 scale.
 * The pages quantize a BF16 [n, k] weight to FP8 at load (mtp_head.rs,
 * `quantize_proj`; glm5next_mtp_head/init.rs quantises only the rows a rank
 * sweeps -- any row range is a base-pointer offset) and pass a per-row scale to
 * the FP8 GEMV (mtp_head.rs, `gemv`, `row_scale`). Recipe (not printed on the
 * pages; this library's reading): per row r, a = max|w|, s = f32(a / 448)
 * (IEEE division; s = 1 for an all-zero row), code = E4M3(f32(w / s)).
 *   w         [n, k] BF16, 16-byte aligned, read only.
 *   codes     [n, k] u8 out, 16-byte aligned.
 *   row_scale [n] f32 out, 4-byte aligned.
 *   n >= 1, 16 <= k <= 65536, k % 16 == 0.
 * Deterministic: codes and scales are bit-identical to the published recipe.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_quantize_fp8(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes, float *row_scale,
                     void *stream);

/* ---------------------------------------------------------------------------
 * NVFP4 weight quantization: a global-absmax pass, then E2M1 codes with an
 * E4M3 scale per 16-element block and one f32 global scale (mtp_head/new.rs,
 * `nvfp4_global_absmax` and `quantize_bf16_to_nvfp4`; mtp_head.rs,
 * `quantize_proj`). Recipe (this library's reading of the two-level NVFP4
 * form): G = max|W| over all n rows; s_g = f32(G / 2688) (s_g = 1 if G == 0);
 * d = f32(6 s_g); per block a = max|w|, sb = E4M3(f32(a / d)),
 * S = f32(e4m3(sb) * s_g); code = E2M1(f32(w / S)) (sign only if S == 0).
 *   w            [n, k] BF16, 16-byte aligned.
 *   codes        [n, k/2] u8 out (element 2j low nibble, 2j+1 high nibble).
 *   block_scale  [n, k/16] u8 out (E4M3).
 *   global_scale [1] f32 out.
 *   ws           workspace of at least mtp_quantize_nvfp4_workspace_bytes(n, k)
 *                bytes, 16-byte aligned; any contents (the call clears it).
 *   n >= 1, 256 <= k <= 65536, k % 256 == 0.
 * ------------------------------------------------------------------------- */
MTP_API size_t mtp_quantize_nvfp4_workspace_bytes(int64_t n, int64_t k);
MTP_API int mtp_quantize_nvfp4(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes,
                       uint8_t *block_scale, float *global_scale, void *ws, size_t ws_bytes,
                       void *stream);

/* ---------------------------------------------------------------------------
 * The combine: draft-step input side for b sequences.
 *   e_b = E[t_b]                                  embedding row copy
 *   c_b = [ rms(e_b, g_e) || rms(h_b, g_h) ]      BF16, embedding first
 *   u_b = bf16( W_fc . c_b )                      W_fc [h, 2h] row-major
 *   x_b = rms(u_b, g_f)                           BF16 out
 * rms(v, g)_i = bf16( v_i / sqrt(mean(v^2) + eps) * (g_i + gamma_offset) ).
 * deepseek_v4_mtp.rs `forward_one` steps 1, 2 and 6 (embedding copy at
 * token * row bytes, the two norms, the final norm); mtp_head.rs module doc
 * (concat -> fc); mtp_head/new.rs (`fc=[h, 2h]`; BF16 buffers embed,
 * normed_embed, normed_hidden, concat [c, 2h], fc_out, normed2). Gamma
 * convention: gamma_offset = 1 reproduces the shared norm kernel that applies
 * (1 + w), 0 the vanilla one that applies w (deepseek_v4_mtp.rs, the comment on
 * `rms_norm_k`). The decoder layer between fc and the final norm is not part
 * of this call (identity).
 *   embed_table   [vocab, h] BF16.      token_ids [host] int32 [b], each in [0, vocab).
 *   target_hidden [b, h] BF16.          gamma_embed, gamma_hidden, gamma_final [h] BF16.
 *   fc_w          [h, 2h] BF16.         x_out [b, h] BF16 out.
 *   ws            >= mtp_draft_combine_workspace_bytes(b, h) bytes (a completion
 *                 counter, the concat [b, 2h] and the fc output [b, h]),
 *                 zero-filled before first use. When the call's kernels have
 *                 completed it holds c [b, 2h] BF16 at byte offset
 *                 MTP_COMBINE_WS_C_OFFSET and u [b, h] BF16 at
 *                 MTP_COMBINE_WS_C_OFFSET + round_up(4 b h, 256): the
 *                 intermediates, for verification (read only; the next call
 *                 overwrites them).
 *   1 <= b <= 8, 16 <= h <= 8192, h % 16 == 0, vocab >= 1, eps > 0. Batch
 *   rows whose concat vectors do not fit in LDS together (b (4h + 16) >
 *   131584) run as consecutive launches of fewer rows each.
 * ------------------------------------------------------------------------- */
#define MTP_COMBINE_WS_C_OFFSET 256
MTP_API size_t mtp_draft_combine_workspace_bytes(int64_t b, int64_t h);
MTP_API int mtp_draft_combine(const uint16_t *embed_table, int64_t vocab, const int32_t *token_ids,
                      const uint16_t *target_hidden, const uint16_t *gamma_embed,
                      const uint16_t *gamma_hidden, const uint16_t *fc_w,
                      const uint16_t *gamma_final, int64_t b, int64_t h, float eps,
                      float gamma_offset, uint16_t *x_out, void *ws, size_t ws_bytes,
                      void *stream);

/* ---------------------------------------------------------------------------
 * The combine with device-resident token ids: the embedding row is gathered by
 * a token id read on the device, e.g. the token_out of the previous draft's
 * mtp_lmhead_argmax, so K chained drafts need no host synchronization (the
 * pages keep the draft token on the device, mtp_head.rs `draft_token_id_dev`,
 * and gather the next embedding from the argmax there, mtp_head/new.rs
 * `embed_from_argmax`).
 *   token_ids_dev [b] int32 on the device (4-byte aligned); an id outside
 *                 [0, vocab) is clamped into that range (it cannot be checked
 *                 on the host).
 *   Everything else as mtp_draft_combine.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_draft_combine_dev(const uint16_t *embed_table, int64_t vocab,
                                  const int32_t *token_ids_dev, const uint16_t *target_hidden,
                                  const uint16_t *gamma_embed, const uint16_t *gamma_hidden,
                                  const uint16_t *fc_w, const uint16_t *gamma_final, int64_t b,
                                  int64_t h, float eps, float gamma_offset, uint16_t *x_out,
                                  void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The combine with the fc stored in the head's precision: the pages quantize
 * the head's projections, the fc [h, 2h] among them, to the head's precision
 * at load (mtp_head/new.rs, the fc through the same quantizer as the other
 * projections; mtp_head.rs `quantize_proj`).
 *   u_b = bf16( sum_i fc^[j, i] c_b[i] ), fc^ = the dequantized fc.
 *   fc_wd      mtp_wdtype of fc; fc, fc_scale, fc_gscale as mtp_lmhead_argmax's
 *              w, scale, gscale for [h, 2h] (quantize with mtp_quantize_fp8 /
 *              mtp_quantize_nvfp4 with n = h, k = 2h). NVFP4 needs h % 128 == 0.
 *   Everything else as mtp_draft_combine.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_draft_combine_q(const uint16_t *embed_table, int64_t vocab,
                                const int32_t *token_ids, const uint16_t *target_hidden,
                                const uint16_t *gamma_embed, const uint16_t *gamma_hidden,
                                int fc_wd, const void *fc, const void *fc_scale,
                                const float *fc_gscale, const uint16_t *gamma_final, int64_t b,
                                int64_t h, float eps, float gamma_offset, uint16_t *x_out,
                                void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The split combiner (deepseek_v4_mtp.rs `forward_one` step 2: the embedding
 * branch through e_proj into h_in, the hidden branch through h_proj into a
 * temp, then a BF16 residual add):
 *   u_b[j] = bf16( bf16(e_proj[j, :] . rms(e_b, g_e)) + bf16(h_proj[j, :] . rms(h_b, g_h)) )
 *   x_b    = rms(u_b, g_f)
 * The same linear map as the concat form with fc = [e_proj | h_proj], rounded
 * at the two branch outputs.
 *   e_proj, h_proj [h, h] BF16, row-major, 16-byte aligned.
 *   Everything else as mtp_draft_combine.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_draft_combine_split(const uint16_t *embed_table, int64_t vocab,
                                    const int32_t *token_ids, const uint16_t *target_hidden,
                                    const uint16_t *gamma_embed, const uint16_t *gamma_hidden,
                                    const uint16_t *e_proj, const uint16_t *h_proj,
                                    const uint16_t *gamma_final, int64_t b, int64_t h, float eps,
                                    float gamma_offset, uint16_t *x_out, void *ws,
                                    size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The draft lm_head sweep with a fused argmax.
 *   n_eff = min(mtp_vocab_size, vocab) if mtp_vocab_size > 0, else vocab
 *           (deepseek_v4_mtp.rs `forward_one` step 6; mtp_head/new.rs
 *           `effective_vocab`; rows [0, n_eff) of the same head).
 *   L[b, r] = sum_i w^[r, i] x[b, i], r < n_eff, accumulated in f32, where w^ is
 *           the BF16 weight, e4m3(q) * scale[r], or e2m1(q) * e4m3(sb) * gscale.
 *   token_out[b] = the lowest r attaining max_r L[b, r]; NaN never wins; if no
 *           row is above -inf the token is 0 (deepseek_v4_mtp.rs,
 *           `argmax_grammar_masked`: strict '>' scan from index 0).
 * The result stays on the device for a deferred 4-byte-per-row read back
 * (mtp_head.rs, `draft_token_id_dev`).
 *   x          [b, h] BF16 (the final-normed hidden).
 *   w, scale, gscale: per `wd` (see mtp_wdtype).
 *   token_out  [b] int32 out.
 *   logits_out NULL, or [b, n_eff] f32 out (the f32 logits, for verification).
 *   ws         >= mtp_lmhead_argmax_workspace_bytes(...) bytes (about 384 KB:
 *              a completion counter, a running maximum per batch row and
 *              partial results per thread block), zero-filled before first use.
 *   1 <= b <= 8; 1 <= vocab < 2^31; mtp_vocab_size >= 0; 16 <= h <= 8192 with
 *   h % 16 == 0 (BF16, FP8) or h % 256 == 0 (NVFP4).
 * Deterministic: identical weight rows give bit-identical logits wherever they
 * sit, so exact duplicates resolve to the lower index. The f32 summation order
 * depends on the kernel form the shape takes (mtp_lmhead_kernel_form): calls
 * of one form give a vector the same bits whatever else shares the call;
 * between forms the logits may differ by rounding.
 * ------------------------------------------------------------------------- */
MTP_API size_t mtp_lmhead_argmax_workspace_bytes(int64_t vocab, int64_t h, int64_t b, int wd);
MTP_API int mtp_lmhead_argmax(const uint16_t *x, int64_t b, int64_t h, int wd, const void *w,
                      const void *scale, const float *gscale, int64_t vocab,
                      int64_t mtp_vocab_size, int32_t *token_out, float *logits_out, void *ws,
                      size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Which kernel form the lm_head entry points (and mtp_draft_step) take for b
 * vectors of length h against a `wd` head; a query for profiling and tests,
 * host-only, no device work. Returns 0 for the VALU sweep (per 16-byte weight
 * chunk: decode, then b dot products on the vector ALU), 1 for the matrix-core
 * sweep (16-row tiles against the b vectors as 16 x 16 x 32 MFMAs), taken by
 * FP8 from b = 5 and NVFP4 from b = 3 (FP8 from 3 and NVFP4 from 2 when
 * h % 4096 != 0, where the VALU sweep takes its slower clamped form) when h is
 * a multiple of 512 (FP8) or 1024 (NVFP4) and the b staged vectors plus the
 * per-wave weight tiles fit in LDS (b <= 5 at h = 8192); by BF16 from b = 3
 * when h is a multiple of 1024 and at most 4,096 (four waves share each
 * tile, whose partial sums must fit in LDS beside 8 staged vectors).
 * Both compute the same L[b, r] and token (deepseek_v4_mtp.rs `forward_one`
 * steps 6-7); the matrix-core form exists because at b of 4 to 8 decoding
 * plus b dot products per weight chunk outruns HBM on the vector ALU (for BF16,
 * the b dot products and b reads of the staged vectors per chunk). An NVFP4
 * call of the matrix-core form whose vectors F16 cannot hold exactly (a
 * nonzero element whose binary exponent is more than 31 below that of its
 * vector's largest magnitude, or a non-finite value) runs the VALU sweep
 * inside the same launch.
 * Returns -1 when the arguments are outside the lm_head's limits.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_lmhead_kernel_form(int64_t b, int64_t h, int wd);

/* ---------------------------------------------------------------------------
 * The same sweep and argmax, also giving each row's top-1 log-probability, in
 * the same pass over the weights (mtp_head.rs: `argmax_batch_lp_k`, the batched
 * argmax that also emits each row's top-1 log-probability; `last_conf_bits`,
 * the chain confidence of a propose = the minimum top-1 softmax probability
 * over its drafts, reset to 1.0 when a propose starts).
 *   logprob_out[b] = max_r L[b, r] - log sum_r exp(L[b, r]) over r < n_eff
 *           (f32 logits, f32 online sums; <= 0). NaN when a logit is NaN or no
 *           logit is above -inf. The sums run in the order in which a thread
 *           block's waves take row groups at run time, so repeated calls agree
 *           to rounding (a few f32 ulps); tokens and logits are bit-identical.
 *   conf_inout NULL, or [b] f32 read and written: conf = fminf(conf, exp(logp))
 *           (a NaN log-probability leaves it unchanged). Set it to 1.0 at the
 *           start of a propose; chained drafts then leave the chain confidence.
 *   Other arguments, sizes, workspace and errors as mtp_lmhead_argmax (no
 *   logits output); logprob_out [b] f32 out, non-NULL.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_lmhead_argmax_logprob(const uint16_t *x, int64_t b, int64_t h, int wd,
                                      const void *w, const void *scale, const float *gscale,
                                      int64_t vocab, int64_t mtp_vocab_size, int32_t *token_out,
                                      float *logprob_out, float *conf_inout, void *ws,
                                      size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The sweep with a grammar-masked argmax (deepseek_v4_mtp.rs,
 * `argmax_grammar_masked`): row r < n_eff takes part only when word r / 32
 * exists (r / 32 < mask_words) and its bit r % 32 is set. Among those rows the
 * token is the lowest index attaining the maximum; allowed_out[b] = 1.
 * When the mask allows no row, token 0 and allowed_out[b] = 0 (the pages
 * return 0 as a pad draft). As on the pages, allowed rows whose logits are all
 * -inf or NaN give token 0 with allowed_out[b] = 1.
 *   mask       [b, mask_words] int32, row-major (one mask per batch row);
 *              may be NULL when mask_words == 0; 4-byte aligned.
 *   mask_words 0 <= mask_words <= 2^26 (words past n_eff / 32 are ignored).
 *   allowed_out [b] int32 out, non-NULL.
 *   Other arguments, sizes, workspace and errors as mtp_lmhead_argmax.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_lmhead_argmax_masked(const uint16_t *x, int64_t b, int64_t h, int wd,
                                     const void *w, const void *scale, const float *gscale,
                                     int64_t vocab, int64_t mtp_vocab_size, const int32_t *mask,
                                     int64_t mask_words, int32_t *token_out, int32_t *allowed_out,
                                     void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The whole draft step in one call: a draft from (token, target_hidden)
 * (deepseek_v4_mtp.rs `forward_one`: embed, combiner, final norm, lm_head,
 * argmax; the result left on the device, mtp_head.rs `draft_token_id_dev`).
 * Computes what mtp_draft_combine (BF16 fc) followed by mtp_lmhead_argmax (or
 * mtp_lmhead_argmax_logprob) computes, with the same formulas, in two
 * launches: the combine stops after the fc output u (no completion counter,
 * no separate final-norm pass), and every lm_head thread block applies the
 * final norm to u itself while its first weight loads are in flight.
 *   token_ids   [b] int32: host memory (token_ids_on_device = 0, each id in
 *               [0, embed_vocab)) or device memory (token_ids_on_device = 1,
 *               4-byte aligned, clamped into [0, embed_vocab)), e.g. the
 *               previous draft's token_out.
 *   embed_table, target_hidden, gammas, fc_w, eps, gamma_offset: as
 *               mtp_draft_combine (embed_table has embed_vocab rows).
 *   wd, w, scale, gscale, vocab, mtp_vocab_size, token_out: as mtp_lmhead_argmax.
 *   x_out       NULL, or [b, h] BF16 out (the final-normed hidden).
 *   logprob_out NULL, or [b] f32 out; conf_inout NULL or [b] f32 in/out: as
 *               mtp_lmhead_argmax_logprob.
 *   ws          >= mtp_draft_step_workspace_bytes(b, h) bytes (the lm_head's
 *               counters and partial results, u [b, h] and the concat
 *               [b, 2h]), zero-filled before first use; each call leaves its
 *               counters at zero. When the call's kernels have completed it
 *               holds u [b, h] BF16 at byte offset MTP_STEP_WS_U_OFFSET and
 *               c [b, 2h] BF16 at MTP_STEP_WS_U_OFFSET + round_up(2 b h, 256)
 *               (for verification; read only).
 *   1 <= b <= 8; 16 <= h <= 8192, h % 16 == 0 (h % 256 == 0 for NVFP4);
 *   b * (4h + 16) <= 131584 (the concat vectors in LDS: b <= 8 at h = 4096,
 *   b <= 6 at h = 5120, b <= 4 at h = 8192).
 * ------------------------------------------------------------------------- */
#define MTP_STEP_WS_U_OFFSET 393728
MTP_API size_t mtp_draft_step_workspace_bytes(int64_t b, int64_t h);
MTP_API int mtp_draft_step(const uint16_t *embed_table, int64_t embed_vocab,
                           const int32_t *token_ids, int token_ids_on_device,
                           const uint16_t *target_hidden, const uint16_t *gamma_embed,
                           const uint16_t *gamma_hidden, const uint16_t *fc_w,
                           const uint16_t *gamma_final, int64_t b, int64_t h, float eps,
                           float gamma_offset, int wd, const void *w, const void *scale,
                           const float *gscale, int64_t vocab, int64_t mtp_vocab_size,
                           int32_t *token_out, uint16_t *x_out, float *logprob_out,
                           float *conf_inout, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * mtp_draft_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and kernels without the workspace. The
 * workspace lives in a fixed scratch array of the library (about 0.75 MB per
 * GPU, held until the process ends: mtp_draft_step_workspace_bytes(8, 8192)
 * bytes, enough for every b and h the call accepts; a shape needing more is
 * rejected with MTP_ERR_WORKSPACE). The call allocates nothing. Its first call
 * on a device finds the scratch's address there and clears its counters with
 * a kernel on `stream`; every call leaves them at zero. Every call on one GPU
 * shares that GPU's scratch: calls that can overlap in time (different
 * streams, or other threads) race and must be serialized by the caller.
 * Arguments, limits and errors: as mtp_draft_step (no ws, ws_bytes).
 * ------------------------------------------------------------------------- */
MTP_API int mtp_draft_step_noalloc(const uint16_t *embed_table, int64_t embed_vocab,
                                   const int32_t *token_ids, int token_ids_on_device,
                                   const uint16_t *target_hidden, const uint16_t *gamma_embed,
                                   const uint16_t *gamma_hidden, const uint16_t *fc_w,
                                   const uint16_t *gamma_final, int64_t b, int64_t h, float eps,
                                   float gamma_offset, int wd, const void *w, const void *scale,
                                   const float *gscale, int64_t vocab, int64_t mtp_vocab_size,
                                   int32_t *token_out, uint16_t *x_out, float *logprob_out,
                                   float *conf_inout, void *stream);

/* ---------------------------------------------------------------------------
 * Encoder verification hook: out[i] = encode(f32 with bit pattern
 * first_bits + i), i < count, with the same device encoders the quantizers
 * and the RMSNorms use. Lets a test sweep every f32 pattern against an
 * independent encoder.
 *   codec MTP_CODEC_E4M3 or MTP_CODEC_E2M1: out [count] u8; MTP_CODEC_BF16:
 *   out [count] u16 (2 * count bytes; pattern i is converted in the low half
 *   of a packed pair when i is even and in the high half when i is odd, so
 *   both halves are exercised); out 16-byte aligned;
 *   1 <= count <= 2^32 - first_bits.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_codec_encode_range(int codec, uint32_t first_bits, int64_t count, uint8_t *out,
                           void *stream);

/* ---------------------------------------------------------------------------
 * Measurement aid, not a step of the draft path: the streaming-read ceiling
 * that the lm_head sweeps' fraction of peak HBM bandwidth is set against
 * (the roofline of the pages' lm_head sweep, a memory-bound pass over the
 * [vocab, hidden] weights). Reads the first bytes - bytes % 8192 bytes of buf
 * once, with the sweeps' access pattern (non-temporal 16-byte loads,
 * contiguous units per wave, two in flight, one block per compute unit,
 * grid-stride), in one of six launch shapes: 0: 4 waves per block, 8 KB
 * units; 1: 4 waves, 4 KB; 2: 8 waves, 4 KB; 3: 8 waves, 8 KB; 4: 4 waves,
 * 4 KB units in pairs (8 KB contiguous per wave, as a BF16 row at h = 4096);
 * 5: 8 waves, 4 KB units in pairs. No other work. Each thread folds
 * its reads with xor; if a thread's fold equals magic it stores magic to
 * sink[0] (so a test can plant a chunk and check that it was read; otherwise
 * sink is not written).
 *   buf: device, 16-byte aligned, >= bytes; bytes >= 8192; 0 <= shape <= 5;
 *   sink: device u32[1]. Asynchronous on `stream`; nothing is allocated.
 * ------------------------------------------------------------------------- */
MTP_API int mtp_stream_read(const void *buf, int64_t bytes, int shape, uint32_t magic, uint32_t *sink,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MTP_DRAFT_H */
