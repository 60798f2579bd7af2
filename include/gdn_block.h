/*
 * gdn_block.h -- C ABI of the Gated DeltaNet (GDN) decode block for MI355X (gfx950).
 *
 * One gdn_block_decode() call runs a GDN layer's decode front for 1..16 rows,
 * the launch called "K1" on "sgl-amd-mono PR #89" (Modifications) and the "GDN
 * block" on "vLLM PR #60833" (Details / Launches):
 *
 *   1. residual add + Gemma RMSNorm: h = bf16(x + residual), residual <- h,
 *      xn = bf16(h * (mean(h^2) + eps)^-1/2 * (1 + norm_w));
 *   2. in_proj_qkvz and in_proj_ba: y = bf16(W xn), bf16 weights, or MXFP4
 *      in_proj_qkvz with xn quantised to MXFP4 per 32-element block
 *      ("vLLM PR #60833", Details / MoE and MXFP4 layouts), or MXFP6 E2M3
 *      in_proj_qkvz with bf16 xn (W6A16: "vLLM PR #60833", a reviewer's comment
 *      proposing MXFP6 for the GDN projections);
 *   3. causal depthwise conv update (width 4, no bias) + SiLU over the q|k|v
 *      channels, conv state rolled in place;
 *   4. g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b); q, k
 *      L2-normalised, q scaled by dk^-1/2;
 *   5. gated delta rule on the cached state S (dk x dv per value head):
 *      S <- exp(g) S; S <- S + k (beta (v - S^T k))^T; o = S^T q, computed in
 *      f32 and stored back f32 or RNE bf16 ("sgl-amd-mono PR #89", Kernel checks);
 *   6. RMSNormGated over each head, norm before gate:
 *      core = bf16(bf16(o) * rstd * gated_norm_w * SiLU(z)).
 *
 * A row whose state index is <= 0 (or >= num_state_slots) is a pad row: its core row is written as
 * +0.0, and neither conv nor SSM state is touched; its residual row is still
 * written ("sgl-amd-mono PR #89", Modifications; "SGLang PR #43558", Accuracy:
 * pad rows at slot -1).
 *
 * Layouts (all row-major, caller-owned device memory):
 *   x, residual       [rows, H] bf16
 *   norm_w            [H] bf16 (Gemma form: the scale is 1 + norm_w)
 *   w_qkvz (BF16)     [Nqkvz, H] bf16, Nqkvz = 2*nk*dk + 2*nv*dv, K contiguous
 *   w_qkvz (MXFP4)    [Nqkvz, H/2] uint8 e2m1 codes, low nibble = even k,
 *   w_qkvz (MXFP6)    [Nqkvz, H/32, 24] uint8: each block of 32 E2M3 codes (sign at
 *                     bit 5, 2 exponent bits with bias 1, 3 mantissa bits) packed into
 *                     24 bytes, code i at bits 6i..6i+5 of the block read as one
 *                     little-endian number
 *   w_qkvz_scales     [Nqkvz, H/32] uint8 e8m0 (2^(byte-127)), MXFP4 and MXFP6 only
 *                     (MXFP4 and MXFP6 need H to be a multiple of 512)
 *                     Output columns are grouped per key head g:
 *                     [q_g (dk) | k_g (dk) | v_g (r*dv) | z_g (r*dv)], r = nv/nk.
 *   w_ba              [2*nv, H] bf16, grouped per key head: [b_g (r) | a_g (r)]
 *   conv_w            [Cd, W] bf16, Cd = 2*nk*dk + nv*dv channels ordered
 *                     q (nk*dk) | k (nk*dk) | v (nv*dv); tap W-1 multiplies
 *                     the newest input
 *   A_log             [nv] f32;  dt_bias [nv] bf16;  gated_norm_w [dv] bf16
 *   conv_state        [num_state_slots, W-1, Cd] bf16: the W-1 previous raw
 *                     q|k|v projection outputs, oldest first
 *   ssm_state         [num_state_slots, nv, dk, dv] f32 or bf16
 *   state_idx         [rows] int32 in device memory; value head h uses key head h / r
 *   core_out          [rows, nv*dv] bf16
 *
 * Tiled projection weights (optional, faster): gdn_block_pack_weights writes a copy
 * of [in_proj_qkvz; in_proj_ba] cut into 16-row tiles whose K steps are stored as
 * 1 KiB blocks in the operand order of the matrix cores, so every load instruction of
 * the projection reads 1 KiB of contiguous memory: bf16 tiles in 32-wide steps (the
 * in_proj_qkvz blocks ordered [K range][group of 4 tiles][step][tile], so a projection
 * workgroup's share is one contiguous run, and so are the MXFP4 / MXFP6 code and scale
 * blocks below; in_proj_ba tiles one run per tile); MXFP4 code tiles in 128-wide steps, followed by their scales, one
 * dword per lane per 4 steps; MXFP6 tiles in 128-wide steps of 1.5 KiB (each lane's
 * 24 code bytes split as 16 + 8, the 16-byte parts of the 64 lanes first), followed by
 * their scales like MXFP4's. Pass it as w_proj_packed; w_qkvz, w_qkvz_scales and w_ba
 * are then not read. The copy is made once (like the pages' shuffled weight copies
 * made before graph capture, "SGLang PR #43558", Modifications / Weights) and has the
 * size of the matrices it copies.
 *
 * MXFP4 activations: with MXFP4 in_proj_qkvz each xn row is quantised inside the
 * decode, per 32-element block ("vLLM PR #60833", Details / MoE: dynamic MXFP4 in 1x32
 * blocks; Details / MXFP4 layouts: the GDN projections quantise their inputs with one of
 * two scale roundings, matching the FP4 GEMM in use). With the block maximum
 * max|xn| = M * 2^E (1 <= M < 2) the scale is 2^e, e clamped to [-126, 127] (an all-zero
 * block keeps 2^-126), by the config's mx_scale_rule:
 *   GDN_MXSCALE_ROUNDED_MAX (default): the maximum rounded half up at e2m1's one mantissa
 *     bit, e = its exponent - 2, i.e. e = E - 2, or E - 1 when M >= 1.75 (the rule the
 *     same page's reviewer comment proposing MXFP6 gives for dynamic_mxfp4_quant, step 2
 *     of making the weights); elements up to 7 * 2^e occur and round to 6 * 2^e;
 *   GDN_MXSCALE_CEIL: the smallest e with max|xn| <= 6 * 2^e, i.e. E - 2, or E - 1 when
 *     M > 1.5.
 * Each xn / 2^e is rounded to the nearest e2m1 value with ties to the even code, and a
 * zero code carries no sign. gdn_mxfp4_quantize applies the same quantiser to caller rows.
 *
 * Errors: every function returns GDN_OK (0) or a negative code; the message
 * is kept per handle (gdn_block_last_error). A failed check enqueues nothing.
 */
#ifndef GDN_BLOCK_H
#define GDN_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_OK 0
#define GDN_E_INVALID_ARG (-1) /* a null or misaligned pointer, a bad row count or config value */
#define GDN_E_UNSUPPORTED (-2) /* a configuration this library refuses (every reason listed) */
#define GDN_E_HIP (-3)         /* a HIP runtime call failed (message holds hipGetErrorString) */

#define GDN_FMT_BF16 0   /* in_proj_qkvz stored as bf16 */
#define GDN_FMT_MXFP4 1  /* in_proj_qkvz stored as OCP MXFP4: e2m1 codes + e8m0 per 32 K */
#define GDN_FMT_MXFP6 2  /* in_proj_qkvz stored as OCP MXFP6 E2M3 codes + e8m0 per 32 K;
                            the activations stay bf16 */

#define GDN_STATE_F32 0
#define GDN_STATE_BF16 1

#define GDN_MXSCALE_ROUNDED_MAX 0 /* MXFP4 activation scale: rounded block maximum, exponent - 2 */
#define GDN_MXSCALE_CEIL 1        /* MXFP4 activation scale: smallest 2^e with max <= 6 * 2^e */

#define GDN_MAX_ROWS 16

typedef struct gdn_block_config {
  int32_t hidden;          /* H; a multiple of 256 (of 512 with MXFP4 or MXFP6), at most 16384 */
  int32_t num_k_heads;     /* nk */
  int32_t head_k_dim;      /* dk: 32, 64 or 128 */
  int32_t num_v_heads;     /* nv; a multiple of nk */
  int32_t head_v_dim;      /* dv: equal to dk */
  int32_t conv_width;      /* W; must be 4 */
  int32_t num_state_slots; /* slots in the conv and SSM state pools */
  int32_t max_rows;        /* largest row count a decode call may pass, 1..16 */
  int32_t qkvz_format;     /* GDN_FMT_BF16, GDN_FMT_MXFP4 or GDN_FMT_MXFP6 */
  int32_t ssm_state_dtype; /* GDN_STATE_F32 or GDN_STATE_BF16 */
  int32_t has_residual;    /* 0: the layer with no residual input (residual is written = x) */
  float norm_eps;          /* Gemma RMSNorm eps (1e-6) */
  float gated_norm_eps;    /* RMSNormGated eps (1e-6) */
  float l2norm_eps;        /* eps inside the q/k L2 norm's square root (1e-6) */
  int32_t input_normed;    /* 1: x is already the norm's output xn (the "normed" build of
                              "SGLang PR #43558", Modifications): steps 1 (residual add and
                              norm) are skipped, residual and norm_w are neither read nor
                              written (they may be NULL), has_residual must be 0; with MXFP4
                              each projection workgroup quantises its K range of xn itself
                              up to 2 rows, and from 3 rows the launch quantises each row
                              once (the same codes and scales either way) */
  int32_t fold_out_proj;   /* 1: the launch also writes the rank's out_proj partial
                              out = bf16(core W_out^T), [R, H] ("SGLang PR #43558",
                              Modifications: K1 with out_proj folded in); needs nv*dv a
                              multiple of 128 up to 1024; decode with
                              gdn_block_decode_with_out_proj */
  int32_t mx_scale_rule;   /* GDN_MXSCALE_ROUNDED_MAX (0) or GDN_MXSCALE_CEIL (1): the scale
                              rule of the MXFP4 activation quantiser (see above); read only
                              with qkvz_format GDN_FMT_MXFP4 */
} gdn_block_config;

typedef struct gdn_block_weights {
  const void* norm_w;        /* [H] bf16 */
  const void* w_qkvz;        /* [Nqkvz, H] bf16, [Nqkvz, H/2] e2m1 bytes or [Nqkvz, H/32, 24]
                                E2M3 bytes */
  const void* w_qkvz_scales; /* [Nqkvz, H/32] e8m0 bytes (MXFP4 and MXFP6, else ignored) */
  const void* w_ba;          /* [2*nv, H] bf16 */
  const void* conv_w;        /* [Cd, W] bf16 */
  const float* A_log;        /* [nv] f32 */
  const void* dt_bias;       /* [nv] bf16 */
  const void* gated_norm_w;  /* [dv] bf16 */
  const void* w_proj_packed; /* NULL, or the tiled copy from gdn_block_pack_weights */
  const void* w_out;         /* [H, nv*dv] bf16 out_proj (this rank's K slice), fold only */
} gdn_block_weights;

typedef struct gdn_block* gdn_block_t;

/* Validate cfg and build a handle. Every unsupported setting is refused with
 * GDN_E_UNSUPPORTED and all reasons listed in the message (the startup
 * refusals of "sgl-amd-mono PR #89", Modifications / Refusals; "vLLM PR
 * #60833", Details / Refusals). Validation touches no device; on success the
 * handle owns device scratch sized for cfg->max_rows, allocated on the current
 * HIP device. On failure *out is NULL and gdn_block_last_error(NULL) holds
 * the message (per thread). */
int gdn_block_create(const gdn_block_config* cfg, gdn_block_t* out);

/* Enqueue one decode step of `rows` rows on `stream` (a hipStream_t; NULL is
 * the default stream). Asynchronous: no host sync, no allocation, so it can
 * be captured into a HIP graph. All pointers are device pointers aligned to
 * 16 bytes. x is read; residual is read (when the layer has one) and written
 * with h; conv_state and ssm_state are updated in place at the slots named by
 * the valid rows; core_out is written. rows == 0 enqueues nothing and
 * returns GDN_OK; rows < 0 or rows > max_rows is GDN_E_INVALID_ARG.
 * Precondition: the valid state indices of one call are distinct. An index
 * >= num_state_slots is handled like a pad row (zero core, no state access),
 * so no index can make the kernels touch memory outside the pools. The handle's scratch is
 * shared by its calls: calls on one handle must be ordered (one stream). */
int gdn_block_decode(gdn_block_t blk, const void* x, void* residual, const gdn_block_weights* w,
                     void* conv_state, void* ssm_state, const int32_t* state_idx, int32_t rows,
                     void* core_out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): gdn_block_decode, same arguments and
 * results, bit for bit, with the launch's scratch (the hand-off counters, the activation
 * image and the projection partials) taken from a fixed device array that the library
 * holds on each GPU it runs on until the process ends, instead of the handle's own
 * scratch. The array is 8 MiB: 64 KiB of counter lines (at the same place for every
 * handle) and 8128 KiB of data. A handle whose scratch does not fit (a large hidden size
 * or head count at a large max_rows; the TP8-rank and full-width dense shapes fit at
 * max_rows 16) is refused with GDN_E_UNSUPPORTED and both sizes in the message. Its
 * address is looked up (and its counters cleared) once per device by gdn_block_create;
 * if that failed, this call returns GDN_E_HIP with the reason. This call allocates
 * nothing and enqueues one launch. Every such call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other handles, other threads)
 * race and give undefined results; calls ordered on one stream are fine, whatever their
 * handles. Each launch that completes normally leaves the counters at zero; after a
 * wait gives up, gdn_block_check on any handle of that GPU clears them. Not for a
 * handle with fold_out_proj. */
int gdn_block_decode_noalloc(gdn_block_t blk, const void* x, void* residual, const gdn_block_weights* w,
                             void* conv_state, void* ssm_state, const int32_t* state_idx, int32_t rows,
                             void* core_out, void* stream);

/* gdn_block_decode, plus the rank's out_proj partial: out [rows, H] bf16 (device,
 * 16-byte aligned) = bf16(core_out W_out^T) with the sum in f32, one output row per
 * input row (a pad row's partial is zero). Only for a handle created with
 * fold_out_proj = 1 (gdn_block_decode refuses such a handle). */
int gdn_block_decode_with_out_proj(gdn_block_t blk, const void* x, void* residual, const gdn_block_weights* w,
                                   void* conv_state, void* ssm_state, const int32_t* state_idx, int32_t rows,
                                   void* core_out, void* out, void* stream);

/* One launch over `rows` sequences of `tokens` tokens each (a speculative-decoding verify
 * step: the accepted token and its drafts), rows * tokens <= max_rows. Token t of sequence r
 * is row r * tokens + t of x, residual and core_out ([rows * tokens, ...], as in decode).
 * Each sequence starts from the state in slot src_idx[r] (device, [rows] int32) and goes
 * through its tokens in order, with the results that many decode steps would give (at
 * head dim 128 and tokens > 1 in the chunked form: the recurrence unrolled over the step's
 * tokens, the same arithmetic in another rounding order, so equal within rounding, not bit
 * for bit; below 128 one token after the other); after token t the SSM
 * state and the conv window are stored into slot dst_idx[r * tokens + t] (device,
 * [rows, tokens] int32, 16-byte aligned), unless that index is <= 0 or >= num_state_slots
 * (then that snapshot is not kept). The source slot is only read, unless it is also one of
 * the sequence's own destinations. A caller that accepts n tokens continues from
 * dst_idx[r * tokens + n - 1]: a rejected draft leaves nothing to undo (the follow-up
 * "sgl-amd-mono PR #89", Modifications, and "vLLM PR #60833", Limitations, leave open: K1
 * keeps no state per draft token). A sequence with src_idx <= 0 (or >= num_state_slots) is
 * a pad: zero core rows, no state read or written. Preconditions: the valid destination
 * slots of a call are distinct and none is another sequence's source. With tokens == 1 and
 * dst_idx[r] == src_idx[r] the results equal gdn_block_decode's, bit for bit. Not for a
 * handle with fold_out_proj. Asynchronous, allocates nothing; errors as gdn_block_decode. */
int gdn_block_verify(gdn_block_t blk, const void* x, void* residual, const gdn_block_weights* w,
                     void* conv_state, void* ssm_state, const int32_t* src_idx, const int32_t* dst_idx,
                     int32_t rows, int32_t tokens, void* core_out, void* stream);

/* Size in bytes of the tiled projection copy (16-row tiles of [in_proj_qkvz;
 * in_proj_ba], the last b|a tile zero-padded): Nqkvz*H*2 (bf16), Nqkvz*H/2 +
 * Nqkvz*H/32 (MXFP4) or Nqkvz*H*3/4 + Nqkvz*H/32 (MXFP6), plus ceil(2*nv/16) * 16 * H * 2, plus H * nv*dv * 2 with
 * fold_out_proj (W_out in the same tiles). 0 for a NULL handle. */
size_t gdn_block_packed_weight_bytes(gdn_block_t blk);

/* Enqueue on `stream` the write of the tiled copy of w->w_qkvz (with w->w_qkvz_scales
 * for MXFP4 and MXFP6), w->w_ba and, with fold_out_proj, w->w_out, all row-major as above, into
 * `packed` (device memory of gdn_block_packed_weight_bytes bytes, 16-byte aligned,
 * caller-owned). */
int gdn_block_pack_weights(gdn_block_t blk, const gdn_block_weights* w, void* packed, void* stream);

/* Quantise `rows` rows of `cols` bf16 values (x, [rows, cols], device, 16-byte aligned)
 * to OCP MXFP4 with the decode's activation quantiser (see above) under `scale_rule`
 * (GDN_MXSCALE_ROUNDED_MAX or GDN_MXSCALE_CEIL): codes [rows, cols/2] uint8, two per
 * byte, low nibble = even element (device, 4-byte aligned), and scales [rows, cols/32]
 * uint8 e8m0 = e + 127 (device). cols must be a positive multiple of 32; rows == 0
 * enqueues nothing. Asynchronous on `stream`; allocates nothing. Errors are reported
 * like a failed gdn_block_create (gdn_block_last_error(NULL)). */
int gdn_mxfp4_quantize(const void* x, int32_t rows, int32_t cols, void* codes, void* scales, int32_t scale_rule,
                       void* stream);

/* Round `rows` rows of `cols` bf16 weights (w, [rows, cols], device, 16-byte aligned)
 * to MXFP6 E2M3, one block of 32 along a row at a time, and write them in the layout
 * w_qkvz takes: codes [rows, cols/32, 24] uint8 (device, 8-byte aligned) and scales
 * [rows, cols/32] uint8 e8m0 (device). The rule is the one the pages give for making
 * the weights ("vLLM PR #60833", a reviewer's comment proposing MXFP6, step 2): the
 * block maximum is rounded to 3 mantissa bits (a carry moving into the exponent), the
 * scale is 2^(E - 2) with E the exponent of that rounded maximum, clamped to
 * 2^[-126, 127] (an all-zero block keeps 2^-126); each value is rounded to the nearest
 * E2M3 value, ties to the even code, at most 7.5; a zero code carries no sign. cols must
 * be a positive multiple of 32; rows == 0 enqueues nothing. Asynchronous on `stream`;
 * allocates nothing. Errors are reported like gdn_mxfp4_quantize's. */
int gdn_mxfp6_round_weights(const void* w, int32_t rows, int32_t cols, void* codes, void* scales, void* stream);

/* A plain read of `bytes` bytes of device memory at `src`, the reference that the
 * block's achieved bandwidth is compared with (a measurement aid, not a step of the
 * block; the pages measure their kernels against the HBM bandwidth, "vLLM PR #60833",
 * Validation). Every 16-byte word is read once, with 16-byte loads, 8 in flight per
 * thread; workgroup b reads the 32 KiB from byte 32768 b on and folds its 32-bit words by
 * XOR into sink[b], for b < ceil(bytes / 32768) (sink: device, 4-byte aligned,
 * caller-owned), so the XOR of the sink words equals the XOR of all 32-bit words of the
 * input. bytes must be a positive
 * multiple of 16 and src 16-byte aligned. Asynchronous on `stream`; allocates nothing.
 * Errors are reported like gdn_mxfp4_quantize's. */
int gdn_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Read and clear the handle's sticky error word (synchronous: waits for the whole
 * device first; not for the hot path). Inside a decode, every wait for another
 * workgroup is bounded (gdn_block_set_spin_limit); a wait that gives up sets a bit
 * (1: waiting for the norm rows, 2: waiting for a key-head group's projection tiles or,
 * with fold_out_proj, for the core rows, 4: waiting for the other value heads of a key
 * head to read its old q|k conv rows) and lets the launch finish with undefined outputs.
 * Such a launch can also leave the hand-off counters in the handle's scratch uncleared
 * (each launch clears them on the assumption that every workgroup arrived), which would
 * corrupt the handle's next decodes: when the word is not 0, this call also clears every
 * counter, so decodes enqueued after it start clean. The word of the handle's device's
 * gdn_block_decode_noalloc scratch is read, ORed in and cleared the same way. 0 means
 * every decode since the last check completed normally. */
int gdn_block_check(gdn_block_t blk, uint32_t* error_word);

/* Set the poll limit of every bounded wait in this handle's later decodes (default
 * 2^20 polls, each followed by a short sleep: far longer than any launch waits). A
 * smaller limit makes a stalled launch give up sooner; 0 gives up at the first poll
 * that does not find the wait complete (used to test the give-up path). polls < 0 is
 * GDN_E_INVALID_ARG. */
int gdn_block_set_spin_limit(gdn_block_t blk, int32_t polls);

/* Free the handle and its scratch (NULL is a no-op). Waits for nothing: the
 * caller must make sure no enqueued decode still uses it. */
void gdn_block_destroy(gdn_block_t blk);

/* The last error message of a handle, or of this thread's last failed
 * gdn_block_create, gdn_mxfp4_quantize, gdn_mxfp6_round_weights or gdn_read_stream when blk is NULL.
 * Never NULL; "" when there was none. */
const char* gdn_block_last_error(gdn_block_t blk);

#ifdef __cplusplus
}
#endif

#endif /* GDN_BLOCK_H */
