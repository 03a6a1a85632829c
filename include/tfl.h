/*
 * tfl.h -- C ABI of the MI355X (gfx950) forward pass of a stack of post-LN
 * transformer encoder layers with causal and key-padding masking.
 *
 * Operation (per layer, x one token row of d = d_model values):
 *     x = LN(x + MHA(x))
 *     x = LN(x + W2 GELU(W1 x + b1) + b2)
 * MHA uses H heads of dh = d / H; key j is visible to query i of sequence b
 * iff j <= i and j < valid_len[b] (causal and key-padding masks together).
 * Every row, padded ones included, is computed by that formula.  LN is
 * (z - mean) / sqrt(var + eps) * gamma + beta with the biased variance;
 * GELU uses the exact error function.
 *
 * Where this comes from (three project write-ups on one subject):
 *  - "KernelForge", "Why it matters": 2-4 layer encoder stacks, d_model
 *    32-1024, batch 1 to 10,000, sequences 32 to 100,000 tokens, causal
 *    masking with a padding mask throughout; "What we built": causal and
 *    key-padding masks applied in one attention kernel.
 *  - "KernelForge", "What it does": one frozen plan per (GPU, dtype, shape),
 *    looked up at run time with no autotuning.
 *  - "Hyper-optimized megakernel-hybrid transformer inference", "Problem
 *    decomposition": sequence-resident, task-graph and tiled families
 *    chosen by shape; "Sample prompts": one callable handles all
 *    cases.
 *  - "Implement a GPU Kernel for a Transformer Layer", "What it does": a
 *    shape-aware adapter that routes on sequence length, width and dtype.
 *
 * Ownership: the caller owns every device buffer (weights, x, y, valid_len,
 * workspace).  The library never allocates device memory.  Weights are
 * borrowed from tfl_create until tfl_destroy and read at every forward;
 * x, y, valid_len and workspace are borrowed for the stream-ordered
 * duration of one tfl_forward.  The handle is host memory owned by the
 * library.  One handle may serve several streams at once only with
 * distinct workspaces.
 *
 * Errors: every entry point returns a tfl_status and never aborts; the
 * thread-local text of the last failure is tfl_last_error().
 */
#ifndef TFL_H
#define TFL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tfl_handle tfl_handle;

/* I/O dtype of x, y and every weight, bias and LayerNorm parameter. */
typedef enum { TFL_F32 = 0, TFL_F16 = 1, TFL_BF16 = 2 } tfl_dtype;

typedef enum {
    TFL_OK = 0,
    TFL_E_INVALID = 1,     /* null/misaligned pointer, bad size, overlap, bad length (TFL_CHECK=1) */
    TFL_E_UNSUPPORTED = 2, /* valid but outside the supported shape set */
    TFL_E_WORKSPACE = 3,   /* workspace smaller than tfl_workspace_bytes() */
    TFL_E_HIP = 4,         /* a HIP launch or runtime call failed */
    TFL_E_INTERNAL = 5
} tfl_status;

/* Execution paths the dispatcher chooses among ("Hyper-optimized
 * megakernel-hybrid transformer inference", "Problem decomposition": a
 * sequence-resident family, a task-graph family and a tiled family). */
typedef enum {
    TFL_PATH_AUTO = 0,
    TFL_PATH_SEQ = 1,   /* one workgroup owns whole sequences, whole stack in one launch */
    TFL_PATH_PQ = 2,    /* task list over 64-row tiles (QKV tasks, split-K attention tasks,
                           FFN tasks), one launch per stage of the list */
    TFL_PATH_TILED = 3, /* per-stage kernels: QKV GEMM, attention, GEMM+residual, LayerNorm, FFN */
    TFL_PATH_PQ_SINGLE = 4 /* the PQ tasks in one persistent launch fed by a device queue:
                              disabled, tfl_create returns TFL_E_UNSUPPORTED (its one GPU
                              run did not finish and no cause has been shown) */
} tfl_path;

typedef struct {
    int32_t n_layers;   /* >= 1 */
    int32_t d_model;    /* multiple of 32, <= 1024, odd part <= 7: 32 x {1..8, 10, 12, 14, 16,
                           20, 24, 28, 32} (a LayerNorm row is split over up to 64 lanes of
                           at most 8 four-value chunks each) */
    int32_t n_heads;    /* d_model / n_heads in {16, 32, 64} */
    int32_t d_ffn;      /* multiple of 32 */
    int32_t batch;      /* >= 1 */
    int32_t seq_len;    /* >= 1 */
    int32_t dtype;      /* tfl_dtype */
    float ln_eps;       /* <= 0 selects 1e-5 */
    int32_t force_path; /* tfl_path; TFL_PATH_AUTO lets the dispatcher choose */
} tfl_config;

/* One layer's parameters: device pointers in the I/O dtype, row-major,
 * nn.Linear layout ([out, in]).  w_qkv rows are q | k | v and head h owns
 * rows h*dh .. h*dh+dh-1 of each third.  Every pointer, matrices and
 * vectors alike, must be 16-byte aligned. */
typedef struct {
    const void *w_qkv, *b_qkv; /* [3d, d], [3d] */
    const void *w_o, *b_o;     /* [d, d],  [d]  */
    const void *ln1_g, *ln1_b; /* [d], [d] */
    const void *w_1, *b_1;     /* [f, d],  [f]  */
    const void *w_2, *b_2;     /* [d, f],  [d]  */
    const void *ln2_g, *ln2_b; /* [d], [d] */
} tfl_layer;

/* Validates cfg and the layer pointers, freezes the plan for this shape and
 * returns a handle.  No device call is made.  layers points to n_layers
 * entries, copied into the handle (the weights themselves are borrowed).
 * The plan is a fixed rule over the shape and dtype, evaluated once here
 * ("KernelForge", "What it does": a frozen per-shape table consulted at run
 * time, no autotuning).  Errors: TFL_E_INVALID for null or misaligned
 * pointers and sizes < 1; TFL_E_UNSUPPORTED for shapes outside the supported
 * set or a forced path that cannot run the shape. */
tfl_status tfl_create(const tfl_config *cfg, const tfl_layer *layers, tfl_handle **out);

/* Device workspace one tfl_forward needs, in bytes (0 is possible: the SEQ
 * path keeps everything between x and y on chip).  The caller allocates it;
 * the library never does ("KernelForge", "What it does": memory planned per
 * shape). */
tfl_status tfl_workspace_bytes(const tfl_handle *h, size_t *bytes);

/* Enqueues the forward pass on hip_stream (a hipStream_t; NULL = default
 * stream).  Asynchronous: no host synchronisation, no allocation.  Computes
 * the operation stated at the top of this file: the encoder layers of
 * "Hyper-optimized megakernel-hybrid transformer inference", "Problem
 * decomposition", with the causal and key-padding masks applied together
 * ("KernelForge", "What we built") and the exact-erf GELU ("KernelForge",
 * "How the LLM is used").
 *   x          [batch, seq_len, d_model] I/O dtype, 16-byte aligned
 *   valid_len  [batch] int32 in device memory, each in [1, seq_len]; the
 *              kernels clamp values outside that range (results are those
 *              of the clamped lengths); with the environment variable
 *              TFL_CHECK=1 they are copied to the host (synchronising the
 *              stream) and out-of-range values return TFL_E_INVALID; that
 *              mode also checks the magnitude precondition below (and that
 *              x is finite) with device reductions, returning TFL_E_INVALID
 *   y          [batch, seq_len, d_model] I/O dtype, 16-byte aligned, must
 *              not overlap x or the workspace
 *   workspace  at least tfl_workspace_bytes() bytes, 256-byte aligned, must
 *              not overlap x
 * Errors: TFL_E_INVALID (null or misaligned pointer, overlap, bad length
 * with TFL_CHECK=1), TFL_E_WORKSPACE (too small), TFL_E_HIP (launch failed).
 * Inputs must be finite.  The first layer's products take x rounded to fp16
 * operands, and weights converted to fp16, on the fp16-operand paths (bf16
 * I/O on every path, fp32 I/O on the PQ and layer-wise paths); there |x| and
 * every weight must stay below 65504 in magnitude. */
tfl_status tfl_forward(tfl_handle *h, const void *x, const int32_t *valid_len, void *y,
                       void *workspace, size_t workspace_bytes, void *hip_stream);

/* Size of the static device workspace behind tfl_forward_noalloc (32 MiB). */
#define TFL_STATIC_WORKSPACE_BYTES (32u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as tfl_forward, on the same kernels, with the workspace taken from
 * a static device array of TFL_STATIC_WORKSPACE_BYTES that the library owns
 * (each GPU holds its own copy until the process ends).  No device or host
 * memory is allocated.  Arguments as for tfl_forward; the current HIP device
 * must be the one that x, y, valid_len and the stream belong to.
 * TFL_CHECK is not honoured here (its length check copies to host memory).
 * Errors: TFL_E_WORKSPACE when the plan needs more workspace than the static
 * array holds (tfl_workspace_bytes() > TFL_STATIC_WORKSPACE_BYTES); otherwise
 * as tfl_forward.  All calls on one GPU share that GPU's array: calls that
 * overlap in time on one GPU (several streams, several threads) race and give
 * undefined results; calls ordered on one stream are safe.  Nothing in the
 * array has to start at zero: every forward writes what it reads. */
tfl_status tfl_forward_noalloc(tfl_handle *h, const void *x, const int32_t *valid_len, void *y,
                               void *hip_stream);

/* Frees the handle (host memory only; the borrowed weights stay the
 * caller's).  NULL is accepted. */
tfl_status tfl_destroy(tfl_handle *h);

/* Name of the frozen plan ("TILED", "SEQ", "PQ" plus a tile tag); the
 * string is owned by the handle.  "(null handle)" for NULL. */
const char *tfl_plan_name(const tfl_handle *h);

/* Path of the frozen plan (a tfl_path value), or -1 for a NULL handle. */
int32_t tfl_plan_path(const tfl_handle *h);

/* Kernel stages, for stage timing. */
typedef enum {
    TFL_STAGE_PREP = 1,  /* input staging: x -> fp32 residual + operand planes; weights -> fp16 planes
                            (bf16 / fp32 I/O); V^T padding */
    TFL_STAGE_QKV = 2,   /* fused QKV projection, head-major epilogue */
    TFL_STAGE_ATTN = 3,  /* streaming masked attention */
    TFL_STAGE_OUT = 4,   /* out-projection + bias + residual */
    TFL_STAGE_LN = 5,    /* residual LayerNorm */
    TFL_STAGE_FFN1 = 6,  /* FFN up-projection + exact-erf GELU */
    TFL_STAGE_FFN2 = 7,  /* FFN down-projection + bias + residual */
    TFL_STAGE_FUSED = 8, /* whole-stack kernels of the SEQ and PQ paths */
    TFL_STAGE_ROW = 9    /* layer-wise path, d_model <= 256, 16-bit I/O: one kernel per layer
                            for out-projection + LayerNorm + FFN + LayerNorm + next QKV */
} tfl_stage;

/* Measurement aid.  Arms HIP-event timing of every launch of one stage in
 * the following tfl_forward calls on this handle, up to max_launches
 * launches (the events are recorded on the forward's stream around each
 * launch of that stage, nothing else changes).  Re-arming discards earlier
 * records.  No device memory is allocated (HIP events only). */
tfl_status tfl_timer_arm(tfl_handle *h, int32_t stage, int32_t max_launches);

/* Waits for the recorded events, returns the summed kernel time in ms and
 * the number of launches timed, and disarms the timer. */
tfl_status tfl_timer_read(tfl_handle *h, float *total_ms, int32_t *launches);

/* Thread-local message describing the last non-OK status. */
const char *tfl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TFL_H */
