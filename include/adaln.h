/*
 * adaln.h -- C ABI of the MI355X (gfx950) adaLN chain kernels.
 *
 * The operations are the eager diffusion-transformer chain that the pages on
 * SGLang-Diffusion's fused kernels replace with bit-exact fused kernels:
 * affine-free LayerNorm followed by the adaLN modulation, the per-head q/k
 * LayerNorm, the gated residual add, and bias + tanh-GELU.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are bf16 (dtype argument must be ADALN_BF16), except where an
 *    entry point names fp32 tensors.  Every tensor
 *    pointer is a DEVICE pointer, at least 2-byte aligned.  Strides are in
 *    elements, non-negative.  Outputs are written contiguously (row-major).
 *  - Ownership: the caller owns every buffer.  The library never allocates,
 *    frees or synchronises; it keeps no state between calls (beyond cached
 *    device attributes, and the caller-owned workspace of ln_modulate_ws),
 *    so calls are reentrant and thread-safe.
 *  - Execution: each call enqueues its kernel(s) on `stream` (a hipStream_t
 *    passed as void*, NULL = the null stream) and returns at once.
 *  - Errors: 0 = ADALN_OK.  Argument errors are negative codes returned
 *    synchronously BEFORE anything is launched and before any HIP runtime
 *    call is made (so they can be checked on a machine without a GPU).  A
 *    launch failure returns ADALN_ERR_HIP.  adaln_status_str() names a code.
 *  - An empty problem (a zero row count) is a successful no-op.
 *  - Exact aliasing of an output with an input is allowed only where an
 *    entry point says so (same base pointer, identical contiguous layout);
 *    any other overlap between an output and an input is ADALN_ERR_ALIAS.
 *
 * Numerics (every op): fp32 arithmetic in between, results rounded to bf16
 * (round-to-nearest-even) exactly where the eager PyTorch chain rounds, as
 * the "Fused Kernels" page, section "Numerical contracts and quality tiers",
 * requires of its bit-exact kernels.  LayerNorm statistics use the fp32
 * Welford algorithm in one fixed order (see adaln_order_for): lane l of a
 * row pushes the elements of vectors l, l+L, l+2L, ... (V consecutive
 * elements each) in increasing position, with 1/n the correctly rounded
 * reciprocal; lane states are then merged pairwise at offsets 1, 2, 4, ...
 * with the Chan-Golub-LeVeque update, lower lane first, an empty side
 * leaving the other unchanged; var = m2/D, rstd = 1/sqrt(var + eps) with
 * IEEE-correct division and square root.  No fused multiply-add is formed
 * other than the ones this order names.
 */
#ifndef ADALN_H
#define ADALN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADALN_ABI_VERSION 3

/* status codes */
#define ADALN_OK 0
#define ADALN_ERR_NULL -1      /* a required pointer is NULL                      */
#define ADALN_ERR_SHAPE -2     /* negative size, hidden % 4 != 0, bad head size  */
#define ADALN_ERR_DTYPE -3     /* dtype is not ADALN_BF16                        */
#define ADALN_ERR_ALIGN -4     /* a tensor pointer is not 2-byte aligned         */
#define ADALN_ERR_ALIAS -5     /* an output overlaps an input other than allowed */
#define ADALN_ERR_TOO_LARGE -6 /* a size exceeds what the kernels address        */
#define ADALN_ERR_STRIDE -7    /* a stride is negative or unsupported            */
#define ADALN_ERR_HIP -8       /* the HIP runtime reported a launch error        */
#define ADALN_ERR_ARG -9       /* any other invalid argument (unknown op, eps)   */

/* dtypes */
#define ADALN_BF16 1
#define ADALN_F32 2 /* only where an entry point says so (temb_table_slices' temb) */

/* ops, for adaln_order_for */
#define ADALN_OP_LN_MODULATE 1
#define ADALN_OP_QK_HEAD_LAYERNORM 2
#define ADALN_OP_RESIDUAL_GATE_ADD_LN_MODULATE 3
#define ADALN_OP_RMSNORM_SCALE_SHIFT 4
#define ADALN_OP_QK_RMSNORM 5

/*
 * ln_modulate -- out = LN(x) * (1 + scale) + shift, bf16 at every eager op.
 *
 * Source: prhub report on sglang PR #34015 (Sana fused adaLN), 实现拆解 §1
 * and 关键源码片段 (layernorm_modulate.py, pass 2): x_hat = bf16(rstd*(x-mean)),
 * one_plus = bf16(1+scale), y = bf16(x_hat*one_plus), out = bf16(y+shift);
 * hidden % 4 == 0 is the only shape requirement (实现拆解 §1), tails are
 * masked.  Per-sample broadcast: scale and shift hold one row per batch
 * sample (the [B,1,D] adaLN rows passed as [B,D] views).
 *
 *  x        [B,S,D] logical; element (b,s,d) at x + b*sx_b + s*sx_s + d*sx_d.
 *           Any non-negative strides; sx_d == 1 (rows contiguous) and
 *           sx_s == 1 (the transposed [B,D,S] storage of Sana's permuted
 *           activations) are the fast paths.
 *  scale    [B,D] with row stride sscale_b (element stride 1).
 *  shift    [B,D] with row stride sshift_b (element stride 1).
 *  eps      added to the biased variance; must be finite and >= 0.
 *  out      [B,S,D] contiguous.  May be exactly x when x is contiguous
 *           (sx_d == 1, sx_s == D, sx_b == S*D).
 *  mean_out, rstd_out   optional ([B*S] fp32 each, row-major); NULL = skip.
 *  D        % 4 == 0, 4 <= D <= 65536.
 */
int ln_modulate(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                int64_t sshift_b, float eps, int dtype, void* out, float* mean_out,
                float* rstd_out, void* stream);

/* 1 if ln_modulate accepts these sizes/strides/dtype (no pointer is read). */
int ln_modulate_can_use(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s, int64_t sx_d,
                        int64_t sscale_b, int64_t sshift_b, int dtype);

/*
 * ln_modulate_ws -- ln_modulate with a workspace: the same operation, the
 * same arguments and the same bits (the fixed statistics order above, the
 * eager roundings), faster on the transposed storage of Sana's permuted
 * activations (prhub report on sglang PR #34015, 实现拆解 §3: the [B,D,S]
 * layout whose copy aten's LayerNorm pays).
 *
 * With sx_s == 1 the rows of x are strided; a 128-byte line then holds 64
 * consecutive tokens of one hidden position.  This entry point reads such
 * lines whole: 8 blocks share each 64-token group, each block reading
 * lanes 8c .. 8c+7 of the order and merging them at offsets 1, 2, 4, then
 * handing its partial states to the others through `workspace`, where each
 * block takes them and merges at offsets 8, 16, 32 -- the same tree.
 *
 *  workspace        device memory of at least ln_modulate_workspace_size()
 *                   bytes, 16-byte aligned, ZERO-FILLED before its first use
 *                   and then left as the calls leave it (every call returns
 *                   it ready for the next, whatever the shape).  It must not
 *                   overlap x, scale, shift, out, mean_out or rstd_out
 *                   (ADALN_ERR_ALIAS), and calls that share one workspace
 *                   must not run concurrently (their hand-overs would mix).
 *  workspace_bytes  its size.  NULL or fewer bytes than the shape needs:
 *                   the call is ln_modulate (no workspace is touched).
 *  Other arguments, layouts, aliasing and errors: as ln_modulate, plus
 *  ADALN_ERR_ALIGN (workspace not 16-byte aligned) and ADALN_ERR_ARG
 *  (workspace_bytes < 0).
 *
 * The workspace path runs when sx_s == 1, D % 8 == 0, D <= 4096,
 * S % 64 == 0, S < 2^31, sx_d % 8 == 0, sx_b % 8 == 0 (B > 1), x, scale,
 * shift and out are 16-byte aligned and the scale/shift row strides are
 * multiples of 8; any other shape takes ln_modulate's kernels.  Its grid is sized to be
 * resident on the device at once, and a block that waits too long for
 * another's state (ADALN_WS_WAIT_US microseconds, default 200, read at each
 * call; 0 = never wait) recomputes that state from x: same arithmetic,
 * same bits.  Calls on different streams with workspaces of their own may
 * run concurrently; the device may then not hold both grids at once, and
 * the bounded waits keep them correct (same bits, more time).
 */
int ln_modulate_ws(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                   int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                   int64_t sshift_b, float eps, int dtype, void* out, float* mean_out,
                   float* rstd_out, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * ln_modulate_noalloc -- ln_modulate_ws whose workspace is a fixed array of
 * device memory inside the library, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The call itself allocates nothing and frees nothing.
 *
 * Same arguments, bits, layouts and errors as ln_modulate; the shapes that
 * take the workspace path (see ln_modulate_ws) use the library's array of
 * 8454144 bytes = 1024 groups of 64 tokens, so B * S beyond 65536 tokens on
 * that path is ADALN_ERR_TOO_LARGE (returned before any HIP call); other
 * shapes run ln_modulate's kernels and need no array.  Each device the
 * library runs on holds its own array from its first call there until the
 * process ends (its address is looked up once per device, with that device
 * current); every call on a device shares that device's array and leaves it
 * ready for the next call, so calls on one device must be ordered (one
 * stream, or events): calls that overlap on one device race.
 */
int ln_modulate_noalloc(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                        int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                        int64_t sshift_b, float eps, int dtype, void* out, float* mean_out,
                        float* rstd_out, void* stream);

/* Bytes of workspace ln_modulate_ws uses for this shape: 8256 per group of
 * 64 tokens (B * S / 64 groups; group g always uses bytes [8256 g, 8256 g +
 * 8256), so one workspace sized for the largest shape serves every smaller
 * one); 0 when the shape never takes the workspace path (or is not accepted
 * at all).  No pointer is read, no HIP call is made. */
int64_t ln_modulate_workspace_size(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                                   int64_t sx_d);

/*
 * residual_gate_add -- out = residual + gate * update, two eager ops:
 * t = bf16(gate*update), out = bf16(residual + t).
 *
 * Source: "Fused Kernels" page, table "adaLN modulation and gating"
 * (residual_gate_add, bit-exact, replaces residual + gate * update); prhub
 * report on sglang PR #34008, 实现拆解 §2-3 (the GLM-Image ff-gate sites).
 * The gate is per batch sample ([B,1,D] rows as a [B,D] view).
 *
 *  residual [B,S,D], element (b,s,d) at residual + b*sr_b + s*sr_s + d.
 *  gate     [B,D] with row stride sg_b.
 *  update   [B,S,D], element (b,s,d) at update + b*su_b + s*su_s + d.
 *  out      [B,S,D] contiguous; may be exactly residual or exactly update
 *           when that input is contiguous.
 *  D        >= 0, any value.
 */
int residual_gate_add(const void* residual, int64_t sr_b, int64_t sr_s, const void* gate,
                      int64_t sg_b, const void* update, int64_t su_b, int64_t su_s, int64_t B,
                      int64_t S, int64_t D, int dtype, void* out, void* stream);

int residual_gate_add_can_use(int64_t B, int64_t S, int64_t D, int64_t sr_b, int64_t sr_s,
                              int64_t sg_b, int64_t su_b, int64_t su_s, int dtype);

/*
 * ln_modulate_fold -- the single-rounding variant of ln_modulate, one
 * affine LayerNorm op: out = bf16(fma(bf16(1 + scale), n, shift)) with
 * n = (x - mean) * rstd in fp32 (the statistics of ln_modulate, same order).
 * NOT bit-identical to the eager chain ln_modulate reproduces: it skips the
 * rounding of x_hat and of x_hat * (1 + scale).
 *
 * Source: "Fused Kernels" page, the request-gated fusion table ("LayerNorm +
 * modulate": layer_norm(x, weight=(1 + scale), bias=shift) in place of the
 * affine-free LayerNorm plus a separate modulate, mounted only in the
 * high-quality tiers); prhub report on sglang PR #34015, 关联脉络 (the folded
 * path measured against the bit-exact kernel).
 *
 * Arguments, layouts, fast paths and aliasing exactly as ln_modulate.
 */
int ln_modulate_fold(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                     int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                     int64_t sshift_b, float eps, int dtype, void* out, float* mean_out,
                     float* rstd_out, void* stream);

/*
 * ln_modulate_fp8 -- ln_modulate with its bf16 output quantized straight to
 * static OCP FP8 E4M3 (1-4-3, bias 7, largest finite 448, no infinities):
 * q = e4m3(clamp(y * (1 / *qscale), -448, 448)), y the eager chain's bf16
 * output (the bits ln_modulate writes), 1 / *qscale one IEEE fp32 division,
 * the product rounded to fp32, the conversion round-to-nearest-even; NaN
 * stays NaN.  One byte per element: 3 bytes of HBM traffic per element
 * instead of the 4 + 3 of ln_modulate followed by a quantize pass.
 *
 * Source: "Fused Kernels" page, table "Quantized layout producers"
 * (flux2_layernorm_modulate_fp8_quant: LayerNorm plus adaLN modulation
 * directly into static FP8 output).
 *
 *  qscale   device pointer to the fp32 per-tensor scale (> 0), read by the
 *           kernel (so the call needs no host synchronization).
 *  out      [B,S,D] E4M3 bytes, contiguous, V-byte aligned (V as
 *           adaln_order_for reports: 8 when D % 8 == 0, else 4); must not
 *           overlap any input.
 *  Other arguments as ln_modulate (mean_out / rstd_out: the row statistics).
 */
int ln_modulate_fp8(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                    int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                    int64_t sshift_b, float eps, const float* qscale, int dtype, void* out,
                    float* mean_out, float* rstd_out, void* stream);

/*
 * rmsnorm_scale_shift -- out = RMSNorm(x) * (1 + scale) + shift, bf16 at
 * every eager op: x_hat = bf16(x * rinv), then the ln_modulate tail
 * (bf16(1+scale), bf16(x_hat*one_plus), bf16(y+shift)).
 *
 * Source: "Fused Kernels" page, table "Normalization" (rmsnorm_scale_shift:
 * RMSNorm + * (1 + scale) + shift, bit-exact, replaces four eager kernels)
 * and the request-gated fusion table (rms_norm(x) * (1 + scale) + shift in
 * one launch).  RMSNorm without affine: rinv = 1/sqrt(mean(x^2) + eps), no
 * mean subtraction.  Statistics order: lane l of a row accumulates
 * ss = fma(x, x, ss) over the elements of vectors l, l+64, ... in increasing
 * position (V as adaln_order_for reports for ADALN_OP_RMSNORM_SCALE_SHIFT);
 * lane sums are added pairwise at offsets 1, 2, 4, ..., 32; rinv =
 * 1/sqrt(ss/D + eps) with IEEE division and square root.
 *
 * Arguments, layouts, fast paths and aliasing as ln_modulate, except:
 *  rinv_out optional [B*S] fp32 per-row 1/sqrt(mean(x^2) + eps); NULL = skip.
 */
int rmsnorm_scale_shift(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                        int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                        int64_t sshift_b, float eps, int dtype, void* out, float* rinv_out,
                        void* stream);

int rmsnorm_scale_shift_can_use(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                                int64_t sx_d, int64_t sscale_b, int64_t sshift_b, int dtype);

/*
 * residual_gate_add_ln_modulate -- the gated residual update, then
 * ln_modulate of the updated residual, in one pass:
 *   residual_out = bf16(residual + bf16(gate * update))
 *   out          = ln_modulate(residual_out, scale, shift, eps)
 * with the roundings and reduction order of the two unfused entry points,
 * so both results are bit-identical to residual_gate_add followed by
 * ln_modulate (the statistics use the ln_modulate order).
 *
 * Source: "Fused Kernels" page, table "Normalization"
 * (scale_residual_norm_scale_shift: the norm + scale/shift with the
 * preceding residual + gate * update folded in, bit-exact); the two parts
 * are defined where residual_gate_add and ln_modulate cite.  In a DiT block
 * it joins each gated residual add with the LayerNorm that reads its result.
 *
 *  residual [B,S,D], element (b,s,d) at residual + b*sr_b + s*sr_s + d.
 *  gate     [B,D] with row stride sg_b.
 *  update   [B,S,D], element (b,s,d) at update + b*su_b + s*su_s + d.
 *  scale, shift   [B,D] with row strides sscale_b, sshift_b.
 *  eps      added to the biased variance; must be finite and >= 0.
 *  residual_out   [B,S,D] contiguous; may be exactly residual when that
 *           input is contiguous.
 *  out      [B,S,D] contiguous; may be exactly update when that input is
 *           contiguous.  No other overlap between an output and any input
 *           or the other output is accepted.
 *  mean_out, rstd_out   optional statistics of the updated residual
 *           ([B*S] fp32 each); NULL = skip.
 *  D        % 4 == 0, 4 <= D <= 65536.  One launch for 16-byte-aligned rows
 *           with D % 8 == 0 at any D, and for 8-byte-aligned rows with
 *           D % 8 == 4 up to D = 4096; other rows run the two unfused
 *           kernels back to back on the stream (same bits).
 */
int residual_gate_add_ln_modulate(const void* residual, int64_t sr_b, int64_t sr_s,
                                  const void* gate, int64_t sg_b, const void* update, int64_t su_b,
                                  int64_t su_s, int64_t B, int64_t S, int64_t D, const void* scale,
                                  int64_t sscale_b, const void* shift, int64_t sshift_b, float eps,
                                  int dtype, void* residual_out, void* out, float* mean_out,
                                  float* rstd_out, void* stream);

int residual_gate_add_ln_modulate_can_use(int64_t B, int64_t S, int64_t D, int64_t sr_b,
                                          int64_t sr_s, int64_t sg_b, int64_t su_b, int64_t su_s,
                                          int64_t sscale_b, int64_t sshift_b, int dtype);

/*
 * qk_head_layernorm -- per-head affine LayerNorm of q and k in one launch.
 *
 * Source: "Fused Kernels" page, table "Normalization" (qk_head_layernorm,
 * bit-exact, per-head LayerNorm on q/k); prhub report on sglang PR #34008,
 * 实现拆解 §1 and 风险与影响 (head_dim <= 128, % 4 == 0 in the pages' kernel;
 * this library accepts head_dim % 4 == 0 up to 256).  The affine LayerNorm is
 * one eager op, so its output is rounded to bf16 once:
 * out = bf16(fma(w, (x - mean) * rstd, b)), the product (x-mean)*rstd
 * rounded to fp32 first.  With w and b both NULL: out = bf16((x-mean)*rstd).
 *
 *  q        [B,S,H,Dh], element (b,s,h,d) at q + b*sq_b + s*sq_s + h*sq_h + d.
 *  k        [B,S,H,Dh], same with sk_*.
 *  wq,bq    [Dh] each, or both NULL; likewise wk,bk.
 *  q_out, k_out   [B,S,H,Dh] contiguous; q_out may be exactly q (and
 *           k_out exactly k) when that input is contiguous.
 *  Dh       % 4 == 0, 4 <= Dh <= 256.
 */
int qk_head_layernorm(const void* q, int64_t sq_b, int64_t sq_s, int64_t sq_h, const void* k,
                      int64_t sk_b, int64_t sk_s, int64_t sk_h, int64_t B, int64_t S, int64_t H,
                      int64_t Dh, const void* wq, const void* bq, const void* wk, const void* bk,
                      float eps, int dtype, void* q_out, void* k_out, void* stream);

int qk_head_layernorm_can_use(int64_t B, int64_t S, int64_t H, int64_t Dh, int64_t sq_b,
                              int64_t sq_s, int64_t sq_h, int64_t sk_b, int64_t sk_s,
                              int64_t sk_h, int dtype);

/*
 * qk_rmsnorm -- per-head RMSNorm of q and k in one launch, with an optional
 * weight per side: out = bf16((x * rinv) * w), rinv = 1/sqrt(mean(x^2) +
 * eps), each product rounded to fp32 and the result rounded to bf16 once
 * (torch's rms_norm is one eager op computed in fp32).  Without weights:
 * out = bf16(x * rinv).
 *
 * Source: "Fused Kernels" page, table "Normalization" (qk_rmsnorm_native:
 * Z-Image per-head QK RMSNorm, bit-exact) and the request-gated fusion table
 * (HunyuanVideo strided QK RMSNorm over the packed QKV layout).  Statistics:
 * 16 lanes per head, lane l accumulates ss = fma(x, x, ss) over vectors
 * l, l+16, ... in increasing position; lane sums added pairwise at offsets
 * 1, 2, 4, 8; rinv with IEEE division and square root.
 *
 *  q, k, strides, B, S, H, Dh, q_out, k_out, aliasing: as qk_head_layernorm.
 *  wq, wk   [Dh] each, or both NULL.
 */
int qk_rmsnorm(const void* q, int64_t sq_b, int64_t sq_s, int64_t sq_h, const void* k, int64_t sk_b,
               int64_t sk_s, int64_t sk_h, int64_t B, int64_t S, int64_t H, int64_t Dh,
               const void* wq, const void* wk, float eps, int dtype, void* q_out, void* k_out,
               void* stream);

int qk_rmsnorm_can_use(int64_t B, int64_t S, int64_t H, int64_t Dh, int64_t sq_b, int64_t sq_s,
                       int64_t sq_h, int64_t sk_b, int64_t sk_s, int64_t sk_h, int dtype);

/*
 * bias_gelu_tanh -- z = bf16(x + bias); out = bf16(gelu_tanh(z)).
 *
 * Source: PR #37075 report (Wan2.2 NVFP4 bias + GELU), 实现拆解 §1 and
 * 关键源码片段 (bias_gelu.cuh): the bias is added in fp32, the sum is rounded
 * back to the tensor dtype, and tanh-GELU is evaluated in fp32 on that
 * rounded value.  gelu_tanh(z) = 0.5 z (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3)))
 * (Hendrycks & Gimpel), evaluated here as z * sigmoid(2u) with the hardware
 * base-2 exponential; the result is within one bf16 ulp of the correctly
 * rounded value (tanh has no correctly rounded fp32 implementation to match).
 *
 *  x        [rows, width], element (r,j) at x + r*sx_row + j.
 *  bias     [width].
 *  out      [rows, width] contiguous; may be exactly x when x is contiguous.
 *  rows, width >= 0.
 */
int bias_gelu_tanh(const void* x, int64_t rows, int64_t width, int64_t sx_row, const void* bias,
                   int dtype, void* out, void* stream);

int bias_gelu_tanh_can_use(int64_t rows, int64_t width, int64_t sx_row, int dtype);

/*
 * modulate_scale_shift -- out = x * (1 + scale) + shift as three eager bf16
 * ops: one_plus = bf16(1 + scale), y = bf16(x * one_plus),
 * out = bf16(y + shift) (the ln_modulate tail applied to x itself).
 *
 * Source: "Fused Kernels" page, table "adaLN modulation and gating"
 * (modulate_scale_shift replaces x * (1 + scale) + shift, bit-exact) and the
 * note under it (LingBot World's camera conditioning uses one affine row per
 * token).
 *
 *  x        [B,S,D], element (b,s,d) at x + b*sx_b + s*sx_s + d.
 *  scale    element (b,s,d) at scale + b*ssc_b + s*ssc_s + d: ssc_s = 0 for
 *           one adaLN row per sample, ssc_s = D (or any) for one per token.
 *  shift    likewise with ssh_b, ssh_s.
 *  out      [B,S,D] contiguous; may be exactly x when x is contiguous.
 *  D        >= 0, any value (16-byte-aligned rows with D % 8 == 0 take the
 *           vector kernel).
 */
int modulate_scale_shift(const void* x, int64_t sx_b, int64_t sx_s, const void* scale, int64_t ssc_b,
                         int64_t ssc_s, const void* shift, int64_t ssh_b, int64_t ssh_s, int64_t B,
                         int64_t S, int64_t D, int dtype, void* out, void* stream);

int modulate_scale_shift_can_use(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                                 int64_t ssc_b, int64_t ssc_s, int64_t ssh_b, int64_t ssh_s, int dtype);

/*
 * temb_table_slices -- the nmod adaLN slices of table + temb, each written
 * contiguously in one pass: out[m][b,l,d] = table[m,d] + float(temb[b,l,m,d]),
 * one fp32 addition (round-to-nearest-even).
 *
 * Source: "Fused Kernels" page, table "adaLN modulation and gating"
 * (temb_table_slices, bit-exact) and the note under it: it replaces the
 * eager (scale_shift_table + temb.float()).chunk(6, dim=2), whose strided
 * slices the model then copies with .contiguous().
 *
 *  table    fp32 [nmod, D], row m at table + m*st_m (the model's
 *           scale_shift_table, any leading singleton dims dropped).
 *  temb     [B, L, nmod, D], element (b,l,m,d) at temb + b*se_b + l*se_l +
 *           m*se_m + d; dtype ADALN_BF16 or ADALN_F32 (the temb dtype).
 *  out      fp32 [nmod][B*L][D]: slice m is the contiguous block starting at
 *           out + m*B*L*D.  Must not overlap table or temb.
 *  nmod, D  >= 0 (6 slices for the Wan-style table; any count).
 */
int temb_table_slices(const float* table, int64_t st_m, const void* temb, int64_t se_b, int64_t se_l,
                      int64_t se_m, int64_t B, int64_t L, int64_t nmod, int64_t D, int dtype, float* out,
                      void* stream);

int temb_table_slices_can_use(int64_t B, int64_t L, int64_t nmod, int64_t D, int64_t st_m, int64_t se_b,
                              int64_t se_l, int64_t se_m, int dtype);

/*
 * adaln_order_for -- the fixed fp32 reduction order the kernels use for a
 * row of D elements of op ADALN_OP_* (ln_modulate_fold and ln_modulate_fp8
 * use ADALN_OP_LN_MODULATE's order), so that a reference implementation can
 * follow the same order and compare results bit for bit ("Fused Kernels"
 * page, section "Numerical contracts and quality tiers": the bit-exact tier
 * rests on a fixed reduction order).
 *
 *  op           ADALN_OP_*.
 *  D            elements per row (head_dim for the q/k ops); > 0, % 4 == 0.
 *  sx_d         element stride along the row of the storage that will be
 *               passed (1 = contiguous; any value >= 0).
 *  align_bytes  alignment of every row start in bytes (a power of two >= 2).
 *  out          filled on success (caller-owned):
 *    V     elements per vector: 8 when D % 8 == 0, else 4;
 *    W     waves per row: 1 for a q/k head (four heads share a wave); for
 *          the row ops the smallest power of two with 64*W*64 >= D, so a
 *          lane holds at most 64 elements of the row (W = 1 up to D = 4096,
 *          16 at D = 65536);
 *    L     lanes per row: 64*W for the row ops, 16 for a q/k head;
 *    map   ADALN_MAP_INTERLEAVED: vector v (elements v*V .. v*V+V-1) belongs
 *          to lane v mod L, which pushes its vectors in increasing v and the
 *          elements of a vector in increasing position;
 *    fold  ADALN_FOLD_PAIRWISE: lane states are merged at offsets 1, 2, 4,
 *          ..., L/2 (inside a wave, then across its waves through LDS): at
 *          offset o lane l (l % 2o == 0) takes merge(state[l],
 *          state[l + o]), lower lane first; the row's state is lane 0's.
 *          LayerNorm merges Welford states (Chan-Golub-LeVeque, an empty
 *          side leaving the other unchanged), RMSNorm adds the lanes' sums
 *          of squares.
 *  The order depends on op and D only: every storage the entry points
 *  accept (vector loads, transposed tiles, element-wise gathers) is reduced
 *  in this same order, so results are a function of the logical values;
 *  sx_d and align_bytes are checked, not used to pick a different order.
 *  Pure host function.  Returns ADALN_OK; ADALN_ERR_SHAPE for a bad D (or a
 *  q/k head over 256), ADALN_ERR_STRIDE for sx_d < 0, ADALN_ERR_ALIGN for an
 *  align_bytes that is not a power of two >= 2, ADALN_ERR_ARG for an unknown
 *  op, ADALN_ERR_NULL for a NULL out, ADALN_ERR_TOO_LARGE for a row op with
 *  D > 65536.
 */
#define ADALN_MAP_INTERLEAVED 1
#define ADALN_FOLD_PAIRWISE 1

typedef struct adaln_order {
  int V;
  int L;
  int W;
  int map;
  int fold;
} adaln_order;

int adaln_order_for(int op, int64_t D, int64_t sx_d, int align_bytes, adaln_order* out);

/* static string naming a status code (never NULL) */
const char* adaln_status_str(int status);

/* ADALN_ABI_VERSION of the built library */
int adaln_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ADALN_H */
