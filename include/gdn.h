/*
 * gdn.h - C ABI of the frame-wise Gated DeltaNet (GDN) forward scan for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation.  "NVIDIA's New 2.6B World Model Generates Minute-Scale 720p
 * Video on a Single GPU" (section "The Architecture: Replacing Softmax
 * Attention at Scale") describes the layer as a recurrent layer that consumes
 * one entire latent frame per step and keeps a fixed-size state matrix updated
 * by a decay gate and a delta-rule correction; "SANA-WM: democratizing
 * Minute-Scale World Modeling with Hybrid Linear DiT" (section "Methodology",
 * item 1) adds that it scans frames one by one with constant memory.  This
 * library computes the plain reading of that description.  For every batch
 * item b, head h and frame f = 1..F, with N tokens per frame:
 *
 *     k^_i = k_i / max(||k_i||_2, eps)
 *     G_f  = sum_i beta_i k^_i k^_i^T                    (Dk x Dk)
 *     U_f  = sum_i beta_i v_i  k^_i^T                    (Dv x Dk)
 *     S_f  = alpha_f * S_{f-1} (I - G_f) + U_f           (Dv x Dk, fp32)
 *     o_i  = S_f q_i           for every token i of frame f
 *
 * All tokens of a frame read the same S_{f-1}; outputs read the post-update
 * state.  With GDN_FLAG_GATES_ARE_LOGITS the gate inputs are logits and the
 * library applies alpha = sigmoid(a) and beta = sigmoid(b) / N itself.
 *
 * Layouts (row-major, last index fastest, no padding):
 *     q, k   [B][F][N][H][Dk]   io dtype        v, o  [B][F][N][H][Dv]  io dtype
 *     beta   [B][F][N][H]       float32          alpha [B][F][H]         float32
 *     S0, S_final, S_in, S_out  [B][H][Dv][Dk]   float32 (row = value dimension)
 * io dtype is bfloat16 (GDN_BF16) or float32 (GDN_F32); the state is always
 * float32.  Supported: Dk == Dv in {16, 32, 64, 128}.
 *
 * Ownership and execution.  Every pointer is a device pointer owned by the
 * caller; the library keeps none after a call returns, and the scan calls
 * allocate no device memory (the block projections' GEMM library handle is the
 * one exception, see gdn_block_in_proj).  Calls are asynchronous on `stream`
 * (a hipStream_t; NULL is the default stream) and never synchronise it.
 * Scratch memory comes from the
 * caller's workspace (see gdn_workspace_size); calls that share a workspace
 * must be ordered on one stream.
 *
 * Errors.  Every entry point returns a gdn_status; nothing crosses the ABI as
 * an exception.  All checks run on the host before any launch, and a call
 * that fails a check writes nothing.  GDN_ERR_LAUNCH reports a failed kernel
 * launch (hipGetLastError after launching).  Gate values are not range
 * checked: the recurrence is contractive when every alpha is in [0, 1] and the
 * betas of each frame sum to at most 2 (unit keys), which the caller ensures.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,  /* NULL descriptor or required pointer, negative size,
                                 bad eps/dtype/flags, F != 1 in a step call        */
    GDN_ERR_UNSUPPORTED = 2,  /* Dk != Dv, Dk not in {16,32,64,128}, not gfx950   */
    GDN_ERR_ALIGNMENT = 3,    /* q,k,v,o,S*: 16 bytes; beta,alpha: 4; workspace: 256 */
    GDN_ERR_ALIAS = 4,        /* an output overlaps an input, another output or the
                                 workspace (S_final == S0 exactly is allowed)       */
    GDN_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than gdn_workspace_size */
    GDN_ERR_LAUNCH = 6,       /* a kernel launch failed                            */
    GDN_ERR_NO_DEVICE = 7     /* no current HIP device could be queried            */
} gdn_status;

typedef enum gdn_dtype { GDN_BF16 = 0, GDN_F32 = 1, GDN_FP8_E4M3 = 2, GDN_FP4_E2M1 = 3 } gdn_dtype;

/* beta and alpha hold logits; the library applies sigmoid(.)/N and sigmoid(.). */
#define GDN_FLAG_GATES_ARE_LOGITS 0x1u
/* Use the keys as given: k^_i = k_i, no L2 normalisation (and eps is unused).
 * Key normalisation is on by default (flag clear), which is the operator above;
 * a caller whose keys already have unit norm may skip it with this flag. */
#define GDN_FLAG_NO_KEY_NORM 0x2u
/* Reverse direction: the recurrence walks the frames from the last to the
 * first, S0 entering before frame F and S_final leaving after frame 1:
 *     S_f = alpha_f * S_{f+1} (I - G_f) + U_f,   o_i = S_f q_i.
 * The WorldFoundry "SANA-WM" page (sections "What it is for" and "Running in
 * WorldFoundry") names bidirectional weights; each direction is its own scan
 * and the caller combines the two outputs as its model requires. */
#define GDN_FLAG_REVERSE 0x4u

/* Determinism.  Every call is bitwise reproducible: the same inputs on the same
 * device give the same bits, whatever ran before (no atomics, no data-dependent
 * scheduling).  There is no flag for it because there is no other mode. */

typedef struct gdn_desc {
    int32_t B, H, F, N, Dk, Dv; /* batch, heads, frames, tokens per frame, key/value dims */
    int32_t io_dtype;           /* gdn_dtype of q, k, v and o                              */
    uint32_t flags;             /* GDN_FLAG_*                                              */
    float eps;                  /* key-norm floor, finite and > 0 (1e-6 is the convention) */
} gdn_desc;

/* Bytes of device workspace gdn_frame_scan_fwd / gdn_frame_step need for this
 * descriptor (0 when none is needed).  Returns 0 for an invalid descriptor;
 * the compute calls report the reason.
 *
 * The workspace is required, not optional.  The scan runs as three kernels
 * (per-frame Gram and U products over all frames at once, then the serial
 * state recurrence, then the per-frame output products), which hand per-frame
 * d x d operands to each other through this memory: per (b, h, frame) about
 * 10*Dk*Dv bytes in bf16 mode (12*Dk*Dv in fp32 mode), for at most 256 frames
 * per launch, plus one fp32 state per (b, h).  At B1 H16 d128 and 121 frames
 * that is 318 MB (the bf16 intermediates described at gdn_frame_scan_fwd move
 * about 6*Dk*Dv of those bytes per item).  A single persistent kernel holding the state on chip would
 * need none, but it would run on B*H*Dv/16 workgroups (128 at that shape, half
 * the GPU) and re-read every token of K once per row tile of the state; the
 * split design streams each token byte once on every compute unit. */
size_t gdn_workspace_size(const gdn_desc* d);

/* Whole-clip scan: frames 1..F of every (b, h) from S0 (NULL means zeros).
 * Writes o and, when S_final is not NULL, the state after frame F.  S_final
 * may be the same pointer as S0 (in-place carry).  F == 0 copies S0 (or
 * zeros) to S_final; N == 0 applies the decay only.
 *
 * Intermediate precision.  The state is fp32 throughout its recurrence.  With
 * bf16 or block-scaled inputs, Dk >= 64 and N >= 128, the per-frame U_f and
 * the per-frame states handed to the output products are stored in the
 * workspace as bf16 (otherwise U_f as fp32 and the states as bf16 plus an
 * 8-bit remainder, about 16 bits): each adds one bf16 rounding to a value the
 * bf16 products already carry at that precision, and at B1 H16 F121 N880
 * d128 the results stay at about 3.3e-3 (o) and 2.4e-3 (S_final) relative
 * Frobenius error against an fp64 reference.  Small frames keep the finer
 * forms: there a single token's rounding is not averaged with others. */
gdn_status gdn_frame_scan_fwd(const gdn_desc* d,
                              const void* q, const void* k, const void* v,
                              const float* beta, const float* alpha,
                              const float* S0,
                              void* o, float* S_final,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* One frame for streaming use: the same operation with d->F == 1, carrying the
 * state from S_in (NULL means zeros) to S_out.  S_out may equal S_in.  The
 * streaming workflow calls it once per incoming latent frame (the WorldFoundry
 * "SANA-WM" page, section "What it is for": the streaming pipeline advances
 * the rollout window by window).  For bf16 with Dk <= 64, a state kept in two
 * buffers that alternate as S_in and S_out runs as one kernel launch and uses
 * no workspace; an in-place S_out == S_in (and every other shape) takes two
 * launches that pass fp32 partial sums of G and U, one per token range, and a
 * copy of S_in through the workspace, which is why this call takes workspace
 * arguments (gdn_workspace_size with F == 1 gives its size). */
gdn_status gdn_frame_step(const gdn_desc* d,
                          const void* q, const void* k, const void* v,
                          const float* beta, const float* alpha,
                          const float* S_in,
                          void* o, float* S_out,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* Allocation-free scan, for callers that cannot allocate device memory or be
 * handed a workspace: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  The same operation and arguments as
 * gdn_frame_scan_fwd, with the library's own scratch in place of a
 * workspace: a static device array of gdn_static_scratch_bytes() bytes
 * (64 MiB) on every GPU the library runs on, held until the process ends.
 * The frames are processed in chunks sized to fit it, so the results equal
 * gdn_frame_scan_fwd's bit for bit.  GDN_ERR_WORKSPACE when even one frame's
 * operands (about 10*Dk*Dv bytes per (b, h) in bf16 mode, 12*Dk*Dv in fp32
 * mode, plus 4*Dk*Dv per (b, h) of carried state) do not fit.  The scratch
 * needs no clearing: every byte a kernel reads was written earlier in the
 * same call.  All calls on one GPU share its array: calls that can overlap on
 * one GPU (several streams, several host threads) race and must be ordered by
 * the caller.  Calls no allocation routine. */
gdn_status gdn_frame_scan_fwd_static(const gdn_desc* d,
                                     const void* q, const void* k, const void* v,
                                     const float* beta, const float* alpha,
                                     const float* S0,
                                     void* o, float* S_final,
                                     void* stream);

/* Size in bytes of the static scratch array gdn_frame_scan_fwd_static uses. */
size_t gdn_static_scratch_bytes(void);

/* Block-scaled FP8 inputs (io_dtype GDN_FP8_E4M3, Dk = Dv in {32, 64, 128}):
 * the same operation on the dequantised values, for callers whose Q, K and V
 * arrive in low precision (the 4-step distilled model of "NVIDIA's New 2.6B
 * World Model Generates Minute-Scale 720p Video on a Single GPU", section
 * "SANA-WM: One Image, One Minute, One GPU", runs with 4-bit quantization;
 * the scan is bound by HBM bytes, and FP8 halves the bytes of its three
 * input streams).  q, k, v: [B][F][N][H][D] OCP FP8 E4M3 bytes (sign, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinities; 0x7F and 0xFF
 * are NaN); q_scale, k_scale, v_scale: [B][F][N][H][D/32] E8M0 bytes, one per
 * 32 consecutive features of a row: the value of element i is
 * e4m3(x_i) * 2^(s - 127), s its block's scale byte (255 is not a valid
 * scale).  This is the OCP microscaling MXFP8 (E4M3) layout.  o is bfloat16
 * [B][F][N][H][D]; beta, alpha, S0, S_final, the flags, the workspace
 * (gdn_workspace_size of the same descriptor) and every error are as for
 * gdn_frame_scan_fwd.  The kernels turn each loaded value into bf16 exactly,
 * so the result equals gdn_frame_scan_fwd's on bf16 inputs holding the
 * dequantised values.  gdn_frame_scan_fwd and gdn_frame_step refuse this
 * dtype (GDN_ERR_INVALID_ARG), and so does the backward pass
 * (GDN_ERR_UNSUPPORTED). */
gdn_status gdn_frame_scan_fwd_fp8(const gdn_desc* d,
                                  const void* q, const uint8_t* q_scale,
                                  const void* k, const uint8_t* k_scale,
                                  const void* v, const uint8_t* v_scale,
                                  const float* beta, const float* alpha,
                                  const float* S0,
                                  void* o, float* S_final,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Block-scaled FP4 inputs (io_dtype GDN_FP4_E2M1, Dk = Dv in {32, 64, 128}):
 * as gdn_frame_scan_fwd_fp8 with OCP FP4 E2M1 elements (sign, 2 exponent bits
 * with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 * negatives), two per byte: q, k, v are [B][F][N][H][D/2] bytes, byte j of a
 * row holding feature 2j in its lower four bits and feature 2j + 1 in its
 * upper four; the E8M0 scales are laid out as for FP8 (the OCP microscaling
 * MXFP4 layout).  The input streams shrink to a quarter of bf16's; every
 * value is exact in bf16, so the result equals gdn_frame_scan_fwd's on bf16
 * inputs holding the dequantised values.  Each block-scaled entry point
 * accepts its own dtype only (GDN_ERR_INVALID_ARG otherwise). */
gdn_status gdn_frame_scan_fwd_fp4(const gdn_desc* d,
                                  const void* q, const uint8_t* q_scale,
                                  const void* k, const uint8_t* k_scale,
                                  const void* v, const uint8_t* v_scale,
                                  const float* beta, const float* alpha,
                                  const float* S0,
                                  void* o, float* S_final,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ------------------------------------------------------------------ backward
 * Gradients of gdn_frame_scan_fwd, for training on minute-long sequences
 * ("SANA-WM: democratizing Minute-Scale World Modeling with Hybrid Linear
 * DiT", section "Problem & Motivation").  Given the forward call's inputs and
 * flags, the output gradient dO = dL/do and dS_final = dL/dS_final (NULL means
 * zeros), writes
 *     dq, dk, dv  [B][F][N][H][D]  io dtype      dbeta [B][F][N][H]  float32
 *     dalpha      [B][F][H]        float32       dS0   [B][H][Dv][Dk] float32
 * the gradients of the loss with respect to q, k, v, beta, alpha and S0 (with
 * GDN_FLAG_GATES_ARE_LOGITS, dbeta and dalpha are gradients of the logits).
 * dS0 may be NULL (not written) and may be the same pointer as dS_final.  The
 * chain rule of the recurrence in the header comment: walking the frames in
 * the opposite order with X_f = dL/dS_f,
 *     X_f   = sum_i do_i q_i^T + alpha_g X_g (I - G_g)     (g the frame after f)
 *     dq_i  = S_f^T do_i          dv_i = beta_i X_f k^_i
 *     dk^_i = beta_i (X_f^T v_i - alpha_f (M + M^T) k^_i),  M = S_{f-1}^T X_f
 *     dbeta_i = v_i . X_f k^_i - alpha_f k^_i . M k^_i
 *     dalpha_f = <X_f, S_{f-1} (I - G_f)>
 * and dk from dk^ through the key normalisation.  The states S_f are
 * recomputed, not taken from the forward call.  Results are bitwise
 * reproducible.  Pointers, alignment (q,k,v,dO,dq,dk,dv,S0,dS_final,dS0: 16
 * bytes; beta,alpha,dbeta,dalpha: 4), ownership, streams and errors are as for
 * gdn_frame_scan_fwd; every output must be disjoint from every input, from
 * the other outputs and from the workspace. */
size_t gdn_workspace_size_bwd(const gdn_desc* d);
gdn_status gdn_frame_scan_bwd(const gdn_desc* d,
                              const void* q, const void* k, const void* v,
                              const float* beta, const float* alpha,
                              const float* S0,
                              const void* dO, const float* dS_final,
                              void* dq, void* dk, void* dv,
                              float* dbeta, float* dalpha, float* dS0,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* Training with saved states.  gdn_frame_scan_bwd recomputes every per-frame
 * operand of the forward walk (the Gram products, U and the states S_f),
 * which costs about two thirds of a forward call on each backward call.  A
 * caller with the memory to spare (gdn_saved_size bytes per call: at B1 H16
 * F121 N880 d128 about 325 MB) can keep them instead:
 * gdn_frame_scan_fwd_save is gdn_frame_scan_fwd (the same o and S_final, bit
 * for bit when F > 1 and the plain forward keeps full-precision intermediates,
 * i.e. below Dk 64 or 128 tokens per frame; at larger shapes the plain forward
 * hands U and the state planes on in bf16 (see gdn_frame_scan_fwd) while this
 * call keeps the full forms the backward reads, and a one-frame
 * gdn_frame_scan_fwd call runs the streaming step's kernels, which add in
 * another order: in both cases the two agree to rounding, within the
 * forward's tolerance) that leaves in `saved` every frame's operands, the states entering
 * its launch chunks (S0 or zeros first) and every token's key scale, and
 * gdn_frame_scan_bwd_saved is gdn_frame_scan_bwd (the same gradients, bit for
 * bit) that reads them instead of recomputing, so it takes no S0 and needs
 * only gdn_workspace_size_bwd_saved bytes of workspace (about half of
 * gdn_workspace_size_bwd's).  The backward call must see the same descriptor
 * and inputs as the forward call that filled `saved`, which it reads and does
 * not change; `saved` is owned by the caller, must be 256-byte aligned and
 * disjoint from every other argument of both calls.  bf16 and fp32 only
 * (block-scaled inputs: GDN_ERR_UNSUPPORTED).  Sizes are 0 for an invalid
 * descriptor and when there is nothing to save (F == 0 or no (b, h) units). */
size_t gdn_saved_size(const gdn_desc* d);
size_t gdn_workspace_size_bwd_saved(const gdn_desc* d);
gdn_status gdn_frame_scan_fwd_save(const gdn_desc* d,
                                   const void* q, const void* k, const void* v,
                                   const float* beta, const float* alpha,
                                   const float* S0,
                                   void* o, float* S_final,
                                   void* saved, size_t saved_bytes,
                                   void* stream);
gdn_status gdn_frame_scan_bwd_saved(const gdn_desc* d,
                                    const void* q, const void* k, const void* v,
                                    const float* beta, const float* alpha,
                                    const void* dO, const float* dS_final,
                                    void* dq, void* dk, void* dv,
                                    float* dbeta, float* dalpha, float* dS0,
                                    const void* saved, size_t saved_bytes,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ---------------------------------------------------------- block projections
 * The steps either side of the scan inside a GDN block ("NVIDIA's New 2.6B
 * World Model Generates Minute-Scale 720p Video on a Single GPU", section "The
 * Architecture: Replacing Softmax Attention at Scale": the GDN layer sits in
 * transformer blocks of a hybrid backbone).  The pages do not give the
 * block's projections; these calls take the plain reading of a linear
 * attention block: linear maps, without bias, from the hidden states
 * x [B][F][N][C] (bf16, C the model width) to the scan's inputs, and from the
 * scan's output back to width C.
 *
 * Weights are bf16 and stored output-major (one row of inputs per output, the
 * layout of a torch.nn.Linear weight).  gdn_block_in_proj, with
 * w_qkv [3][H][D][C] and w_gate [2][H][C],
 *     q[b,f,n,h,e]        = sum_c x[b,f,n,c] w_qkv[0,h,e,c]   (k: 1, v: 2)
 *     beta_logit[b,f,n,h] = sum_c x[b,f,n,c] w_gate[0,h,c]
 *     alpha_logit[b,f,h]  = (1/N) sum_n sum_c x[b,f,n,c] w_gate[1,h,c]
 * so the decay gate is one per frame, taken from the frame's mean hidden
 * state.  q, k, v [B][F][N][H][D] are bf16; the logits are float32 and feed
 * the scan with GDN_FLAG_GATES_ARE_LOGITS.  N == 0 gives alpha_logit = 0.
 * gdn_block_out_proj, with w_out [C][H*D],
 *     y[b,f,n,c] = sum_{h,e} o[b,f,n,h,e] w_out[c, h*D + e]           (bf16)
 * Products accumulate in float32 and round once to the output type; the
 * results are bitwise reproducible on one device.
 *
 * d gives B, H, F, N and D = Dk (== Dv); io_dtype must be GDN_BF16 and the
 * flags are ignored.  B, F and N may be 0; H, D and C must be at least 1
 * (GDN_ERR_INVALID_ARG), and C and H*D multiples of 8 for 16-byte rows and at
 * most 2^20 (GDN_ERR_UNSUPPORTED, as are io_dtype != GDN_BF16 and Dk != Dv).  Pointers
 * are device pointers owned by the caller: bf16 tensors 16-byte aligned,
 * float32 tensors 4-byte aligned, workspace 256-byte aligned and at least
 * gdn_block_workspace_size bytes (both calls use the same size).  Outputs must
 * be disjoint from the inputs, from each other and from the workspace.  Errors
 * as for the scan; the calls are asynchronous on `stream`.  The GEMMs run in
 * hipBLASLt, whose handle (with whatever device memory hipBLASLt keeps for it)
 * the library creates on a device's first call and keeps until the process
 * ends; the first call on a device may therefore allocate. */
size_t gdn_block_workspace_size(const gdn_desc* d, int32_t C);
gdn_status gdn_block_in_proj(const gdn_desc* d, int32_t C,
                             const void* x, const void* w_qkv, const void* w_gate,
                             void* q, void* k, void* v,
                             float* beta_logit, float* alpha_logit,
                             void* workspace, size_t workspace_bytes,
                             void* stream);
gdn_status gdn_block_out_proj(const gdn_desc* d, int32_t C,
                              const void* o, const void* w_out, void* y,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* Human-readable name of a status code (static storage). */
const char* gdn_status_string(gdn_status s);

/* Library version as 10000*major + 100*minor + patch. */
int32_t gdn_version(void);

/* ------------------------------------------------------------------ profiling
 * Kernel-level timing for benchmarks.  Between gdn_profile_begin and
 * gdn_profile_end every kernel the library launches is bracketed by two
 * hipEvents recorded on the launch stream.  gdn_profile_end waits for the last
 * recorded event, then fills, per kernel kind k < GDN_NUM_KERNELS, the summed
 * duration in milliseconds and the number of launches.  Not thread-safe; at
 * most GDN_PROFILE_MAX_LAUNCHES launches are recorded per session. */
#define GDN_NUM_KERNELS 9
#define GDN_PROFILE_MAX_LAUNCHES 65536
gdn_status gdn_profile_begin(void);
gdn_status gdn_profile_end(double* total_ms, int64_t* launches);
/* Name of kernel kind k ("frame_gram", "state_scan", "frame_output",
 * "state_copy", "frame_step", and for the backward pass "w_gram",
 * "adjoint_scan", "frame_dq", "frame_dkv"), or NULL when k is out of range. */
const char* gdn_kernel_name(int32_t k);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
