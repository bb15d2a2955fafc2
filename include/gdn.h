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
 * caller; the library keeps none after a call returns and allocates no device
 * memory.  Calls are asynchronous on `stream` (a hipStream_t; NULL is the
 * default stream) and never synchronise it.  Scratch memory comes from the
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

typedef enum gdn_dtype { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* beta and alpha hold logits; the library applies sigmoid(.)/N and sigmoid(.). */
#define GDN_FLAG_GATES_ARE_LOGITS 0x1u

typedef struct gdn_desc {
    int32_t B, H, F, N, Dk, Dv; /* batch, heads, frames, tokens per frame, key/value dims */
    int32_t io_dtype;           /* gdn_dtype of q, k, v and o                              */
    uint32_t flags;             /* GDN_FLAG_*                                              */
    float eps;                  /* key-norm floor, finite and > 0 (1e-6 is the convention) */
} gdn_desc;

/* Bytes of device workspace gdn_frame_scan_fwd / gdn_frame_step need for this
 * descriptor (0 when none is needed).  Returns 0 for an invalid descriptor;
 * the compute calls report the reason. */
size_t gdn_workspace_size(const gdn_desc* d);

/* Whole-clip scan: frames 1..F of every (b, h) from S0 (NULL means zeros).
 * Writes o and, when S_final is not NULL, the state after frame F.  S_final
 * may be the same pointer as S0 (in-place carry).  F == 0 copies S0 (or
 * zeros) to S_final; N == 0 applies the decay only. */
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
 * buffers that alternate as S_in and S_out runs as one kernel launch; an
 * in-place S_out == S_in takes two (the state is first copied aside). */
gdn_status gdn_frame_step(const gdn_desc* d,
                          const void* q, const void* k, const void* v,
                          const float* beta, const float* alpha,
                          const float* S_in,
                          void* o, float* S_out,
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
#define GDN_NUM_KERNELS 5
#define GDN_PROFILE_MAX_LAUNCHES 65536
gdn_status gdn_profile_begin(void);
gdn_status gdn_profile_end(double* total_ms, int64_t* launches);
/* Name of kernel kind k ("frame_gram", "state_scan", "frame_output",
 * "state_copy", "frame_step"), or NULL when k is out of range. */
const char* gdn_kernel_name(int32_t k);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
