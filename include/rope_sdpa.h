/*
 * rope_sdpa.h - C ABI of the MI355X (gfx950) fused rotary-embedding + scaled dot-product
 * attention library.
 *
 * What it computes (page "Metal Flash Attention", SimpleTuner docs, section "Fused RoPE + SDPA"):
 *
 *     Q' = R(Q),  K' = R(K)       interleaved-pair rotation with caller-built cos/sin tables:
 *                                 x'_2i = x_2i c_i - x_2i+1 s_i,  x'_2i+1 = x_2i s_i + x_2i+1 c_i
 *     O  = softmax(scale * Q' K'^T + M) V      (softmax accumulated in fp32)
 *
 * with M from a bool mask (True = attend) or an additive float mask, broadcast over up to
 * four dimensions (same page, section "Enable In SimpleTuner"), or a causal (top-left,
 * key j > query i excluded) pattern.  The forward rotates Q and K inside the attention kernel,
 * in registers, on their way from HBM: by default it writes no rotated copy of Q or K to
 * memory.  Two exceptions, both opt-in or forced by the inputs: RS_FLAG_K_PREPASS and the Q/K
 * prologue (RMS-normalized or fp32 Q/K) rotate K once per (batch, K/V head) into the caller's
 * workspace (K' = R(K) rounded to the input dtype, [B, Hkv, S, D]), and the quantized
 * pre-pass mode writes codes.  The backward (16-bit inputs at D = 128) leaves Q' (written by
 * its dQ kernel) and K' (by a rotation pass) in the workspace; at D = 64 and in fp32 it
 * rotates both inside its kernels (the quantized backward: the dequantized Q' and K' in the
 * workspace at either D).  The backward
 * returns gradients with respect to the unrotated Q and K (the inverse rotation, i.e. the
 * same rotation with sin negated, applied to dQ' and dK'), and V.
 *
 * Conventions for every entry point
 *  - All tensors are described by rs_tensor: a DEVICE pointer, a dtype and four sizes and
 *    strides counted in ELEMENTS (not bytes).  Q, K, V, O, dO, dQ, dK, dV are [B, H, S, D]
 *    ("BHSD"); any strides are accepted (e.g. a transpose(1,2) view of a BSHD projection or
 *    an unbind view of a fused QKV tensor) provided stride[3] == 1, the base pointer is
 *    16-byte aligned, strides 0..2 are multiples of 16 bytes and stride[2] < 2^23.
 *  - Ownership: the caller owns every buffer (inputs, outputs, LSE, workspace).  The library
 *    allocates no device memory in these calls and keeps no pointer after a call returns.
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 *    call returns without waiting.  Inputs must stay valid and unmodified, and outputs and
 *    workspace untouched by others, until the stream reaches this work.
 *  - Errors: every argument is validated on the host BEFORE anything is enqueued; on any
 *    error nothing is launched, outputs are untouched and a negative rs_status is returned.
 *    Faults during execution surface at the caller's next synchronisation, as in HIP.
 *  - Thread safety: all entry points are re-entrant; there is no global mode.
 *  - Empty inputs: B, H or S may be 0.  Such a call checks dtypes, sizes, flags and the
 *    mask kind as any other; since no element is addressed, data pointers may be NULL and
 *    strides and alignment are not checked.  It returns RS_OK without launching anything or
 *    touching the workspace (which may be NULL; its size is then 0).
 */
#ifndef ROPE_SDPA_H
#define ROPE_SDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROPE_SDPA_ABI_VERSION 3

typedef enum {
  RS_OK = 0,
  RS_ERR_NULL = -1,        /* a required pointer is NULL */
  RS_ERR_DTYPE = -2,       /* dtype not accepted, or Q/K/V/O dtypes differ */
  RS_ERR_SHAPE = -3,       /* sizes inconsistent or not supported (e.g. D not 64/128) */
  RS_ERR_STRIDE = -4,      /* stride[3] != 1 or a stride not a multiple of 16 bytes */
  RS_ERR_ALIGN = -5,       /* base pointer not 16-byte aligned (workspace: 256-byte) */
  RS_ERR_UNSUPPORTED = -6, /* valid request the library does not implement */
  RS_ERR_WORKSPACE = -7,   /* workspace NULL or smaller than rope_sdpa_workspace_size() */
  RS_ERR_INVALID = -8,     /* bad flag, mask kind, scale, or causal together with a mask */
  RS_ERR_NO_DEVICE = -9,   /* no usable gfx950 device is current */
  RS_ERR_LAUNCH = -10,     /* the HIP launch itself failed */
  RS_ERR_SCRATCH = -11     /* rope_sdpa_fwd_noalloc: the call needs more than its static scratch */
} rs_status;

typedef enum { RS_F32 = 0, RS_F16 = 1, RS_BF16 = 2, RS_BOOL = 3 } rs_dtype;

/* How args->mask is read (section "Enable In SimpleTuner"): a bool mask keeps the score where
 * True and excludes it where False; an additive mask is added to the scaled scores (it is not
 * itself scaled).  A row with every key excluded yields O = 0 and LSE = -inf (never NaN). */
typedef enum { RS_MASK_NONE = 0, RS_MASK_BOOL = 1, RS_MASK_ADDITIVE = 2 } rs_mask_kind;

enum {
  RS_FLAG_CAUSAL = 1u << 0,          /* exclude key j > query i; cannot be combined with a mask */
  RS_FLAG_QUANT_INT8_QK = 1u << 1,   /* forward only: blockwise int8 Q'/K' (see rope_sdpa_fwd) */
  RS_FLAG_QUANT_INT8_PREPASS = 1u << 2, /* with either QUANT flag: codes from a quantizer pass */
  RS_FLAG_QUANT_INT4_QK = 1u << 3,   /* as RS_FLAG_QUANT_INT8_QK with int4 codes (not both flags) */
  RS_FLAG_K_PREPASS = 1u << 4        /* forward: K rotated by a pass of its own (see rope_sdpa_fwd) */
};

typedef struct {
  void* data;        /* device pointer (never dereferenced on the host) */
  int32_t dtype;     /* rs_dtype */
  int32_t reserved;  /* must be 0 */
  int64_t size[4];   /* elements */
  int64_t stride[4]; /* elements; a dimension of size 1 may have any stride */
} rs_tensor;

typedef struct {
  /* Q: [B, H, S, D] in the dtype of v (f32, f16 or bf16), or f32 with v in f16/bf16: the
   * autocast layout of flux-style attention, where RMSNorm hands fp32 Q and K to attention
   * while V stays bf16 (diffusers issue "Flux-family attention: flash-attn and other backends fail in an autocast
   * context", section "Root cause, in order").  Such Q and K are read in fp32, rotated in fp32
   * and rounded to the dtype of v for the matrix products; O is in the dtype of v.
   * rope_sdpa_fwd only (rope_sdpa_bwd returns RS_ERR_UNSUPPORTED), no additive mask, no int8. */
  const rs_tensor* q;
  /* K and V: [B, Hkv, S, D], K in the dtype of q, with H % Hkv == 0.  Hkv < H is grouped-query
   * (Hkv == 1: multi-query) attention: query head h reads K/V head h / (H / Hkv), and K is
   * rotated at its own head count (section "Fused RoPE + SDPA": GQA inputs are rotated at
   * the K/V head count and expanded afterwards); dK and dV of the backward have Hkv heads,
   * each the sum over the query heads that read it. */
  const rs_tensor* k;
  const rs_tensor* v;
  /* Pair-duplicated rotation tables (cos[2i] == cos[2i+1]), fp32, sizes [Bt, 1, S, D] with
   * Bt == 1 (shared) or Bt == B (per sample), stride[3] == 1.  Only the even entries are
   * read; duplication is the caller's precondition (section "Fused RoPE + SDPA").
   * Both NULL: plain attention with Q and K used as given (no rotation; the attention half of
   * the eager path, e.g. after rope_sdpa_rotate).  rope_sdpa_fwd only: rope_sdpa_bwd and
   * RS_FLAG_QUANT_INT8_QK then return RS_ERR_UNSUPPORTED.  Exactly one NULL: RS_ERR_NULL. */
  const rs_tensor* cos;
  const rs_tensor* sin;
  /* Optional mask, sizes [Bm, Hm, Sqm, Skm] with each dimension 1 (broadcast) or full
   * (B, H, S, S).  RS_MASK_BOOL: dtype RS_BOOL (one byte, nonzero = attend).
   * RS_MASK_ADDITIVE: dtype RS_F32 or the dtype of q.  Must be NULL for RS_MASK_NONE.
   * With RS_MASK_BOOL, S <= 262144 (else RS_ERR_SHAPE). */
  const rs_tensor* mask;
  int32_t mask_kind;     /* rs_mask_kind */
  uint32_t flags;        /* RS_FLAG_* */
  float scale;           /* softmax scale; 0 means 1/sqrt(D); otherwise finite and > 0 */
  /* Optional RMSNorm of Q and K over the head dimension before the rotation, as flux-style
   * attention applies it (same diffusers issue, "Describe the bug"): x / sqrt(mean_d x_d^2 +
   * norm_eps) * w_d in fp32, with per-dimension weights w: DEVICE pointers to fp32 [D],
   * 16-byte aligned.  Both NULL: no normalization; both or neither (else RS_ERR_INVALID).
   * norm_eps finite and >= 0.  Same restrictions as fp32 Q/K above (forward, no additive
   * mask, no int8).  Zero-initialized rs_args mean no normalization. */
  const float* q_norm_weight;
  const float* k_norm_weight;
  float norm_eps;
} rs_args;

/* Bytes of device workspace a call needs (0 only for an empty call, B, H or S = 0; otherwise
 * the rotation tables are repacked into it, and a forward with RS_FLAG_K_PREPASS or the Q/K
 * prologue, and the 16-bit backward at D = 128, also hold K' = R(K): B * Hkv * S * D elements
 * of the dtype of v).  `backward` = 0 for rope_sdpa_fwd, 1 for rope_sdpa_bwd. */
rs_status rope_sdpa_workspace_size(const rs_args* args, int backward, size_t* bytes);

/*
 * Forward.  Writes o (dtype of v, sizes of q; any valid strides) and, when lse is not NULL,
 * the natural-log row normaliser lse[b][h][i] = log(sum_j exp(scale q'_i.k'_j + m_ij)) into a
 * contiguous fp32 [B, H, S] buffer (-inf for a row with no valid key); lse is what
 * rope_sdpa_bwd needs.  An all-true bool mask is detected on the device and then costs no
 * per-element mask reads.
 * RS_FLAG_K_PREPASS (bf16/f16, rotating, no quantization, no additive mask; else
 * RS_ERR_UNSUPPORTED): K is rotated once per (batch, K/V head) into the workspace by a pass of
 * its own, with the arithmetic of the in-kernel rotation, and the attention kernel reads K'
 * with no table in its key loop: the same results bit for bit, faster at long sequences,
 * for 2 * B * Hkv * S * D elements more HBM traffic (K' written and read back).
 * RS_FLAG_QUANT_INT8_QK (bf16/f16 inputs; any mask kind or causal; lse may be NULL): after the
 * fp32 rotation (each product and sum rounded), Q' and K' are quantized per (b, h, 64-token
 * block) to int8 codes round-half-even(x * fp32(127/amax)) with scale amax/127, QK^T runs on
 * int8 MFMA with exact int32 accumulation, and P.V stays in the input precision (pages:
 * "Requirements" and "Enable In SimpleTuner" name an int8 blockwise mode; what is quantized
 * is this library's reading).  The attention kernel quantizes in registers: no code reaches
 * memory.  With RS_FLAG_QUANT_INT8_PREPASS as well, a quantizer pass writes the codes and
 * scales of Q' and K' to the workspace first (one byte per element) and the attention kernel
 * streams them: the same codes and the same results bit for bit, faster, because each K
 * block is quantized once instead of once per query tile.
 * RS_FLAG_QUANT_INT4_QK: the same with int4 codes, round-half-even(x * fp32(7/amax)) in
 * [-7, 7] with scale amax/7 (pages: the "-int4" alias sets QUANT_INT4 with blockwise
 * quantization).  CDNA4 has no int4 matrix instruction: the codes, exact as int8 values,
 * take the int8 MFMA (the same speed as int8) and are stored one per byte in the pre-pass
 * mode.
 */
rs_status rope_sdpa_fwd(const rs_args* args, const rs_tensor* o, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * checks and results as rope_sdpa_fwd (bit for bit: the same kernels), without the
 * workspace: the library keeps a device scratch array of rope_sdpa_noalloc_scratch_bytes()
 * bytes (64 MiB) per device, held from the first call on that device until the process ends,
 * and this call allocates nothing (no hipMalloc, no allocating library routine).  A call whose
 * workspace would exceed that size leaves K' out of the scratch where it can
 * (RS_FLAG_K_PREPASS is then ignored: the same results bit for bit); a call that still does
 * not fit, or that needs K' (normalized or fp32 Q/K), returns RS_ERR_SCRATCH and launches
 * nothing.  The caller
 * still owns and passes inputs, o and lse.  Every call on one device shares that device's
 * scratch: calls that overlap on one device (enqueued on different streams without ordering
 * between them, or from several threads onto unordered streams) race and give undefined
 * results; calls on one stream are ordered and safe.  Nothing in the scratch is assumed to
 * start at zero (the kernels clear what they count).
 */
rs_status rope_sdpa_fwd_noalloc(const rs_args* args, const rs_tensor* o, float* lse, void* stream);
size_t rope_sdpa_noalloc_scratch_bytes(void);

/*
 * Backward of rope_sdpa_fwd (section "Fused RoPE + SDPA": gradients with respect to the
 * pre-rotation Q and K).  Inputs: the same args as the forward, its o and lse, and the
 * upstream gradient dout (sizes and dtype of o).  Writes dq (sizes of q), dk and dv (sizes of k),
 * all in the dtype of q.
 * The mask (if any) is a constant: no mask gradient.
 * With RS_FLAG_QUANT_INT8_QK or RS_FLAG_QUANT_INT4_QK (16-bit inputs): the gradients of the
 * quantized forward with the gradient passed
 * straight through the quantizer (the pages name a quantized autograd entry point without
 * saying how gradients cross the quantizer; this is the reading taken).  The quantizer pass
 * writes the dequantized values code * scale of Q' and K', rounded to the input dtype, to the
 * workspace, and the backward runs at those values: dV = P^T dO, dQ' = scale dS K^, dK' =
 * scale dS^T Q^, then the inverse rotation.  RS_FLAG_QUANT_INT8_PREPASS changes nothing here.
 */
rs_status rope_sdpa_bwd(const rs_args* args, const rs_tensor* o, const float* lse,
                        const rs_tensor* dout, const rs_tensor* dq, const rs_tensor* dk,
                        const rs_tensor* dv, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Test-only export of the quantization that rope_sdpa_fwd performs under
 * RS_FLAG_QUANT_INT8_QK or RS_FLAG_QUANT_INT4_QK (same reading, same kernel): writes the codes
 * (int8 storage; int4 codes lie in [-7, 7]) of the rotated Q and
 * K into q_codes / k_codes, contiguous [B, H, S, D] / [B, Hkv, S, D] DEVICE buffers (8-byte
 * aligned), and their fp32 scales into q_scales / k_scales, contiguous [B, H, ceil(S / 64)] /
 * [B, Hkv, ceil(S / 64)] DEVICE buffers.  args
 * must carry one of the QUANT flags (else RS_ERR_INVALID) and pass the same validation as the
 * forward; the workspace is the forward's (rope_sdpa_workspace_size(args, 0, ...)).  It lets a
 * test compare the integer decisions bit for bit and run a reference from exactly these
 * values.  Asynchronous on `stream`; nothing is launched on error.
 */
rs_status rope_sdpa_debug_quantize_qk(const rs_args* args, int8_t* q_codes, int8_t* k_codes,
                                      float* q_scales, float* k_scales, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * The eager rotation pass on its own: out = R(x) for a [B, H, S, D] operand x (f32, f16 or
 * bf16, D = 64 or 128) with the same pair-duplicated fp32 tables as rs_args ([Bt, 1, S, D],
 * Bt == 1 or B): out_2i = x_2i c - x_2i+1 s, out_2i+1 = x_2i s + x_2i+1 c, each product and
 * sum rounded to fp32 (no fused multiply-add), then the result rounded to the dtype of x.
 * out has the sizes and dtype of x, any valid strides (it may alias x exactly: in place).
 * This is the separate pass that the fused forward makes unnecessary (section "Fused RoPE +
 * SDPA"); it serves callers that keep rotated keys, and the fused-versus-eager comparison.
 * Same conventions as the other calls (validated first, asynchronous on `stream`).
 */
rs_status rope_sdpa_rotate(const rs_tensor* x, const rs_tensor* cos, const rs_tensor* sin, const rs_tensor* out,
                           void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* rope_sdpa_status_string(rs_status status);

/* Dispatch counters since load or the last reset (section "Enable In SimpleTuner" describes
 * counters of this kind).  Host counters count successfully enqueued calls; the all-true
 * count is kept on the device and reading it synchronises the current device. */
typedef struct {
  uint64_t fwd_instream;       /* forward calls without LSE (no-grad) */
  uint64_t fwd_autograd;       /* forward calls writing LSE (for a later backward) */
  uint64_t bwd_calls;
  uint64_t masked_bool;        /* calls (fwd or bwd) with a bool mask */
  uint64_t masked_additive;
  uint64_t causal;
  uint64_t quant_int8;         /* quantized forward calls (int8 or int4) */
  uint64_t mask_all_true_skipped; /* bool masks found all-true on the device */
  uint64_t errors;             /* calls rejected with a negative status */
  uint64_t quant_bwd;          /* quantized backward calls (the quantized autograd path) */
} rs_stats;

/* Measurement support (single device): while enabled, every rope_sdpa_fwd call records a pair
 * of HIP events on its stream right before its attention kernel and right after it (not
 * around the K preparation or merge launches), so that a benchmark can time that kernel
 * alone on the stream it runs on.  Enabling (or disabling) forgets the pairs recorded so far.
 * rope_sdpa_debug_kernel_time waits for the recorded pairs and returns the sum of their
 * elapsed times in milliseconds and their number.  rope_sdpa_fwd_noalloc records nothing. */
rs_status rope_sdpa_debug_kernel_timing(int enable);
rs_status rope_sdpa_debug_kernel_time(double* total_ms, uint64_t* launches);

void rope_sdpa_get_stats(rs_stats* out);
void rope_sdpa_reset_stats(void);
int rope_sdpa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ROPE_SDPA_H */
