/*
 * ssa.h - C ABI of the Skip-Softmax (BLASST) FlashAttention forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every (batch, head) and every query row i the library
 * computes softmax attention O_i = sum_c p_ic v_c with
 * p_ic = exp(s_ic) / sum exp(s_ic), s_ic = scale * (q_i . k_c), in one
 * streaming pass over key tiles of 128 keys ("Skip-Softmax" page of the
 * vLLM-Omni documentation, section "The online-softmax pass"), with the
 * BLASST skip test in front of each tile ("Skip-Softmax" design document of
 * vLLM-Omni, section "Algorithm"): for a block of 64 query rows and a key
 * tile, with tile_max[i] the row's largest score in the tile and m[i] the
 * row's running maximum over the tiles absorbed so far, the tile is skipped
 * when tile_max[i] - m[i] < ln(lambda) holds for every row of the block
 * (strict '<'); a skipped tile's exponentials and P.V product are never
 * computed and it contributes nothing to the row sums.  The scores QK^T are
 * always computed.  lambda = 0 disables the test and gives dense attention.
 *
 * The threshold (design document, section "From configuration to the kernel
 * threshold"; documentation, section "The threshold"):
 *   ssa_fwd             lambda = factor / seqlen
 *   ssa_fwd_threshold   lambda = threshold (the direct control: independent
 *                       of the sequence length)
 *   ssa_fwd_calibrated  lambda = a * exp(b * target_sparsity) / seqlen (the
 *                       calibrated control; only this curve is accepted)
 * ln(lambda) is evaluated once on the host in double precision and rounded
 * to float; the per-tile comparison runs in float.
 *
 * Tiles: 64 query rows x 128 keys, keys visited in ascending order from 0.
 * A last query block shorter than 64 rows votes with its valid rows only;
 * a last key tile shorter than 128 keys is padded with keys of score -inf.
 *
 * Layouts and ownership (all buffers are device memory owned by the caller;
 * the library allocates nothing, never synchronises, and enqueues its work on
 * `stream`, a hipStream_t or NULL for the default stream: one kernel per
 * call, two for ssa_fwd_virtual and ssa_quantize_qk_fp8):
 *   q, k, v, o    bf16, [B, H, S, D] contiguous, 16-byte aligned, D = 128.
 *   lse           float [B, H, S]: LSE_i = m_i + ln(l_i), natural log of the
 *                 row's softmax denominator over the kept tiles. May be NULL.
 *   skip_counts   int32 [B, H, ceil(S/64)]: number of skipped key tiles of
 *                 each 64-row query block. May be NULL.  The two waves of a
 *                 block exchange their halves of the vote with a bounded
 *                 wait (16384 polls of one LDS word; ssa_set_vote_poll_limit
 *                 for the debug entry); a wave that gives up keeps the
 *                 tile, which is always exact, and the block's count is
 *                 then stored as -1 - count, so a negative count flags a
 *                 block whose decisions may differ between its two halves.
 * Inputs o, lse and skip_counts are overwritten; q, k, v are read only.
 *
 * Errors.  Every argument is checked on the host before any HIP call; a bad
 * call returns a negative ssa_status and enqueues nothing.  On a device that
 * is not gfx950 every entry point returns SSA_ERR_DEVICE (no fallback).  A
 * failed launch returns SSA_ERR_LAUNCH.  ssa_strerror() names the code and
 * ssa_last_error() returns a message about the last failure of the calling
 * thread.  B, H or S equal to 0 is a valid empty call that returns SSA_OK.
 */
#ifndef SSA_H_
#define SSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSA_OK = 0,
  SSA_ERR_INVALID_ARG = -1,    /* null or misaligned pointer, negative size, scale not finite and positive */
  SSA_ERR_UNSUPPORTED = -2,    /* head dimension other than 128, sizes beyond the grid limits */
  SSA_ERR_BAD_THRESHOLD = -3,  /* factor / threshold / lambda negative or non-finite, seqlen <= 0 */
  SSA_ERR_NO_CALIBRATION = -4, /* calibrated call with a <= 0 or non-finite a, b: use the threshold entry */
  SSA_ERR_DEVICE = -5,         /* no HIP device, or the current device is not gfx950 */
  SSA_ERR_LAUNCH = -6,         /* the kernel launch failed */
  SSA_ERR_BAD_CONFIG = -7      /* a calibration formula other than a * exp(b * target_sparsity) */
} ssa_status;

/* Threshold controls of ssa_fwd_varlen and ssa_resolve_threshold. */
typedef enum {
  SSA_MODE_FACTOR = 0,     /* p0 = factor: lambda_b = factor / S_b                     */
  SSA_MODE_THRESHOLD = 1,  /* p0 = threshold: lambda_b = threshold                     */
  SSA_MODE_CALIBRATED = 2  /* p0 = a, p1 = b, p2 = target_sparsity:
                              lambda_b = a * exp(b * target_sparsity) / S_b            */
} ssa_mode;

#define SSA_HEAD_DIM 128
#define SSA_BLOCK_Q 64
#define SSA_BLOCK_K 128
#define SSA_VIRTUAL_NOALLOC_BYTES (16u << 20)   /* static workspace of ssa_fwd_virtual_noalloc */

/* lambda = factor / seqlen.  factor >= 0 and finite, seqlen > 0 (normally S). */
int ssa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int B, int H, int S, int D, float scale, float factor, int seqlen,
            int32_t* skip_counts, void* stream);

/* lambda = threshold.  threshold >= 0 and finite; values above 1 are accepted. */
int ssa_fwd_threshold(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int S, int D, float scale, float threshold,
                      int32_t* skip_counts, void* stream);

/* lambda = a * exp(b * target_sparsity) / seqlen.  a > 0, a and b finite
 * (else SSA_ERR_NO_CALIBRATION), target_sparsity finite, seqlen > 0. */
int ssa_fwd_calibrated(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int S, int D, float scale, float a, float b,
                       float target_sparsity, int seqlen, int32_t* skip_counts, void* stream);

/* Packed variable-length batch ("cu_seqlens" layout of the SGLang SubBlock
 * sparse-attention article for the MiniMax-H3 video DiT, section on the
 * varlen path, where a packed batch is split per document by cu_seqlens),
 * with the threshold normalised by each sequence's own length
 * ("Skip-Softmax" page of the vLLM-Omni documentation, section "The
 * threshold"): sequence b holds the
 * tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of q, k, v, o, which are bf16
 * [T, H, D] with T = cu_seqlens[nseq].  cu_seqlens: device int32 [nseq + 1],
 * non-decreasing from 0; every length must be <= max_seqlen (the kernel
 * leaves the rows of a sequence whose length is negative or above
 * max_seqlen unwritten and counts no query block for it).  Attention never
 * crosses sequences and each sequence normalises lambda by its own length
 * S_b (see ssa_mode).  lse: float [H, T] (nullable).  skip_counts: int32
 * [H, sum_b ceil(S_b / 64)], query blocks of sequence b after those of
 * sequences 0..b-1 (nullable).  The work is spread so that each of the
 * eight XCDs gets an eighth of every sequence, whatever the mix of lengths. */
int ssa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int32_t* cu_seqlens, int nseq, int max_seqlen, int H, int D,
                   float scale, int mode, double p0, double p1, double p2,
                   int32_t* skip_counts, void* stream);

/* Any of the three controls (see ssa_mode; S_b = seqlen), with the largest
 * softmax weight of every row as an extra output: max_prob float [B, H, S]
 * (nullable), max_prob_i = exp(m_i - LSE_i) = 1 / l_i with l_i the row's
 * denominator relative to its maximum m_i over the kept keys; near 1 for a
 * row dominated by one key, near 1/N for a flat row (video-attention blog
 * post on Wan 2.2, section "max_prob = 1 / l_i, and why it is free").  It
 * comes from the epilogue at no extra pass over memory; the other outputs
 * are those of ssa_fwd. */
int ssa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int S, int D, float scale, int mode, double p0, double p1, double p2,
               int seqlen, int32_t* skip_counts, float* max_prob, void* stream);

/* Skipped tiles replaced by virtual tiles ("Triage: Skip, Skim, or Refine
 * Attention Tiles in Video Diffusion Transformers", section 6.1 "Skipping
 * with Virtual Tiles").  Same skip test and mask as ssa_fwd (the virtual keys
 * never enter the running maximum the test uses); then each tile t that a
 * query block skipped joins that block's softmax as one key, the mean of
 * the tile's keys with score scale * (q_i . mean k) + ln(n_t), carrying the
 * mean of the tile's values; n_t is the tile's number of keys (128, fewer
 * for a ragged last tile).  o and lse are those of that softmax;
 * skip_counts as for ssa_fwd.  Any of the three controls (see ssa_mode;
 * S_b = seqlen).
 * workspace: device memory of at least ssa_fwd_virtual_workspace_bytes(B, H,
 * S) bytes, 16-byte aligned, owned by the caller, overwritten (the tile
 * means: mean keys bf16 [B, H, ceil(S/128), 2, D] as a hi + lo pair, mean
 * values bf16 [B, H, ceil(S/128), D]).  Enqueues two kernels (tile means,
 * then attention).  At most 2048 key tiles (S <= 262144), else
 * SSA_ERR_UNSUPPORTED. */
size_t ssa_fwd_virtual_workspace_bytes(int B, int H, int S);
int ssa_fwd_virtual(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int S, int D, float scale, int mode, double p0, double p1,
                    double p2, int seqlen, int32_t* skip_counts, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ssa_fwd_virtual for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call without the workspace argument.  The tile means go to a static device
 * array of the library, SSA_VIRTUAL_NOALLOC_BYTES = 16 MiB, one per GPU,
 * held until the process ends; its address is looked up once per
 * device, on the first call there.  The call must fit it: B * H *
 * ceil(S/128) * 768 bytes <= 16 MiB, i.e. at most 21845 (batch, head, key
 * tile) triples, else SSA_ERR_UNSUPPORTED before any HIP call.  Every call
 * on one GPU uses the same array, and every byte a call reads from it is
 * written earlier in the same call, so nothing needs clearing between calls;
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it and must not be issued.  Allocates nothing and calls no allocating
 * routine; the caller passes inputs and outputs as for ssa_fwd_virtual. */
int ssa_fwd_virtual_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int S, int D, float scale, int mode, double p0, double p1,
                            double p2, int seqlen, int32_t* skip_counts, void* stream);

/* FP8 scores.  The score matmul Q K^T runs on 8-bit floating point at the
 * doubled matrix rate while P.V keeps bf16 inputs (video-attention blog post
 * on Wan 2.2, sections "First, the hardware ceiling" and "Where the 1.33x
 * ceiling comes from, exactly": only the score half moves to the low
 * precision).  Format: OCP FP8 E4M3 (bias 7, largest finite value 448).
 *
 * ssa_quantize_qk_fp8: q, k bf16 [B, H, S, D] (16-byte aligned) to E4M3 codes
 * q8, k8 uint8 [B, H, S, D] (8-byte aligned) with q_scale float [B, H, S]
 * (one per token) and k_scale float [B, H, ceil(S/128)] (one per tile of 128
 * keys).  A block's scale is its largest magnitude / 448 (float32 division;
 * 1 for an all-zero block); each value is divided by its scale (float32),
 * clamped to +-448 and rounded to the nearest code, ties to even.  Enqueues
 * two kernels.
 *
 * ssa_fwd_fp8: the method of ssa_fwd with scores
 * s_ic = scale * q_scale_i * k_scale_t(c) * (decode(q8_i) . decode(k8_c)),
 * summed by the E4M3 MFMA in fp32; v, o bf16 [B, H, S, D] as in ssa_fwd;
 * the skip test, threshold controls (ssa_mode), lse and skip_counts as in
 * ssa_fwd_ex.  tile_mask and tile_margin (nullable; tile_margin needs
 * tile_mask) report the decisions as ssa_fwd_debug does.  At most 4096 key
 * tiles (S <= 524288), else SSA_ERR_UNSUPPORTED. */
int ssa_quantize_qk_fp8(const void* q, const void* k, uint8_t* q8, uint8_t* k8, float* q_scale,
                        float* k_scale, int B, int H, int S, int D, void* stream);
int ssa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const float* q_scale, const float* k_scale,
                const void* v, void* o, float* lse, int B, int H, int S, int D, float scale, int mode,
                double p0, double p1, double p2, int seqlen, int32_t* skip_counts,
                uint8_t* tile_mask, float* tile_margin, void* stream);

/* Any of the three controls (see ssa_mode; S_b = seqlen) with every tile
 * decision of the skip test reported ("Skip-Softmax" design document of
 * vLLM-Omni, section "Algorithm": the per-tile test of every row's tile
 * maximum against its running maximum, evaluated in log space):
 * tile_mask uint8 [B, H, ceil(S/64), ceil(S/128)] (1 = skipped, must not be
 * NULL) and tile_margin float (same shape, nullable): the largest
 * tile_max[i] - m[i] over the block's valid rows, +inf on the first tile.
 * Same arithmetic as the other entry points, so o, lse and skip_counts equal
 * theirs bit for bit. */
int ssa_fwd_debug(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int S, int D, float scale, int mode, double p0, double p1,
                  double p2, int seqlen, int32_t* skip_counts, uint8_t* tile_mask,
                  float* tile_margin, void* stream);

/* Host-only: the ln(lambda) the kernels compare against for one sequence of
 * length seqlen, and whether the test is on (lambda > 0).  No HIP call. */
int ssa_resolve_threshold(int mode, double p0, double p1, double p2, int seqlen,
                          float* ln_lambda, int* vote_enabled);

/* ---- Host-side configuration (no HIP call; "Skip-Softmax" design document
 * of vLLM-Omni, sections "From configuration to the kernel threshold" and
 * "Timestep gating").  A layer's factor for one attention call is resolved
 * from the user control, the layer's calibration and the denoising step, and
 * then passed to ssa_fwd (0 = dense). ---- */

/* SSA_OK if formula is exactly "a * exp(b * target_sparsity)", the only
 * accepted calibration curve, else SSA_ERR_BAD_CONFIG (reject at startup). */
int ssa_check_formula(const char* formula);

/* Startup check of the user control: exactly one of threshold and
 * target_sparsity (else SSA_ERR_INVALID_ARG); a threshold finite and >= 0
 * and a target finite (else SSA_ERR_BAD_THRESHOLD); a target needs a
 * calibration in the checkpoint (has_calibration, else
 * SSA_ERR_NO_CALIBRATION: use the threshold control instead). */
int ssa_check_spec(int has_threshold, double threshold, int has_target, double target_sparsity,
                   int has_calibration);

/* *matched = 1 when one of the npatterns fnmatch patterns matches the full
 * module name or the name relative to `component` (what follows
 * "<component>."); such a layer gets no coefficients and stays dense.
 * component may be NULL or empty. */
int ssa_ignore_match(const char* module_name, const char* component, const char* const* patterns,
                     int npatterns, int* matched);

/* The factor one attention call hands to the kernel (*factor_out, 0 = run
 * dense).  Control: threshold (factor = threshold * seqlen, i.e. lambda =
 * threshold) or target_sparsity (factor = a * exp(b * target_sparsity) from
 * the layer's coefficients; a layer without coefficients runs dense).  A
 * layer matched by an ignore pattern (ignored = 1) runs dense under either
 * control.
 * Timestep gate: disabled_until_timestep = 0 turns it off (t not read); a
 * positive cutoff D runs the call dense while t > D or when no t is
 * published (has_t = 0).  Errors: both or neither control
 * (SSA_ERR_INVALID_ARG); a negative or non-finite threshold, target, cutoff
 * or seqlen <= 0 (SSA_ERR_BAD_THRESHOLD); coefficients with a <= 0 or
 * non-finite (SSA_ERR_NO_CALIBRATION). */
int ssa_layer_factor(int has_threshold, double threshold, int has_target, double target_sparsity,
                     int ignored, int has_coefficients, double a, double b, int seqlen, int has_t,
                     double t, double disabled_until_timestep, double* factor_out);

/* *count = number of the n published timesteps t[i] above the cutoff, i.e.
 * the denoising steps that run dense (0 when the cutoff is 0). */
int ssa_dense_steps(const double* t, int n, double disabled_until_timestep, int* count);

/* Published timesteps of a flow-shifted rectified-flow schedule:
 * num_inference_steps uniform positions u from 1 to 0 mapped to
 * t = shift u / (1 + (shift - 1) u); t_out receives the first
 * num_inference_steps - 1 (one per denoiser forward).  shift > 0,
 * num_inference_steps >= 2. */
int ssa_flow_shift_schedule(double shift, int num_inference_steps, double* t_out);

/* SSA_OK when the current HIP device is gfx950. */
int ssa_device_check(void);

/* Debug entry only (ssa_fwd_debug): the bound of the wait for the partner's
 * half of the vote, in polls of one LDS word, for every later call of this
 * process (default 16384, the constant the other entries use).  The two
 * halves are published in the same phase, so the bound only guards against
 * a wave that never arrives; a test sets it to 0 to drive the give-up path
 * from the host (every tile with the test on is then kept and every count
 * comes out as -1 - count, see skip_counts above).  0 <= polls <= 2^24,
 * else SSA_ERR_INVALID_ARG.  Host only; not synchronised with calls already
 * enqueued. */
int ssa_set_vote_poll_limit(int polls);
int ssa_vote_poll_limit(void);

const char* ssa_strerror(int status);
const char* ssa_last_error(void);
int ssa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H_ */
