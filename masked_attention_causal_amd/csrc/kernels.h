// Host-side launchers of the tfl kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tfl {

// Arithmetic mode, fixed by the I/O dtype:
//   F32:  every GEMM/attention operand fp32, fp32 MFMA.
//   F16:  operands fp16 (activations rounded once to fp16), weights fp16.
//   BF16: operands fp16; bf16 weights are widened to fp16 as they are loaded.
// The residual stream, LayerNorm, Q and K are fp32 in every mode.
enum Mode { MODE_F32 = 0, MODE_F16 = 1, MODE_BF16 = 2 };

enum Epi { EPI_QKV = 0, EPI_GELU = 1, EPI_RES = 2 };

struct GemmArgs {
    const void* A;     // [M, K] operand dtype, row-major
    const void* W;     // [N, K] weight dtype (nn.Linear layout)
    const void* bias;  // [N] weight dtype
    int M, N, K;
    // EPI_QKV: N = 3d; writes Q, K [B, H, L, dh] and V^T [B, H, dh, Lp] operand dtype.
    // F32 mode: Q, K fp32.  16-bit modes: Q and K as fp16 planes of M*d
    // elements each: the rounded value (hi) at Q / K and, when split != 0,
    // the rounding remainder (lo) one plane further.
    float* Q;
    float* Kd;
    void* Vt;
    int L, Lp, H, dh, d;
    int split;
    // EPI_QKV: K is written multiplied by kscale (0 means 1).  The head-dim-16
    // attention kernel takes keys pre-multiplied by log2(e)/sqrt(dh), so its
    // score products come out in the exp2 domain.
    float kscale;
    // EPI_GELU: out [M, N] operand dtype
    void* out;
    // EPI_RES: Z = acc + bias + R, [M, N] fp32
    const float* R;
    float* Z;
};

struct AttnArgs {
    const void* Q;     // [B, H, L, dh]: fp32 (F32 mode) or fp16 hi plane (16-bit modes)
    const void* K;     // [B, H, L, dh], same
    const void* Ql;    // 16-bit modes, first layer: fp16 lo planes of Q and K
    const void* Kl;
    const void* Vt;    // [B, H, dh, Lp] operand dtype; columns >= L hold zeros in 16-bit modes
    void* O;           // [B*L, d] operand dtype, head h at columns h*dh
    const int32_t* lens;
    int B, H, L, Lp, d;
    float scale_log2;  // log2(e) / sqrt(dh); the head-dim-16 kernel reads K already multiplied by it
    unsigned long long* audit;  // tile counters of the audit build (null otherwise)
};

// Weight pointers of one layer (same fields as tfl_layer).
struct LayerPtrs {
    const void *w_qkv, *b_qkv, *w_o, *b_o, *ln1_g, *ln1_b, *w_1, *b_1, *w_2, *b_2, *ln2_g, *ln2_b;
};

constexpr int SEQ_MAX_LAYERS = 8;

// Sequence-resident path: whole stack in one launch.
struct SeqArgs {
    const void* x;   // [B, L, d] I/O dtype
    void* y;         // [B, L, d] I/O dtype
    const int32_t* lens;
    int B, L, F, n_layers;
    float eps;
    float scale_log2;
    unsigned long long* audit;  // tile counters of the audit build (null otherwise)
    LayerPtrs lw[SEQ_MAX_LAYERS];
};

// PQ path: the stack as a task list over 64-row tiles (layer-0 QKV
// projection, split-K attention, fused row tasks), run as one launch per
// stage of the list.
struct PqArgs {
    const void* x;   // [B, L, d] I/O dtype
    void* y;         // [B, L, d] I/O dtype
    const int32_t* lens;
    int B, L, Lp, NT, F, n_layers;
    int KS;          // key tiles per attention split
    int Ctot;        // (tile, split) pairs per (sequence, head)
    float eps;
    float scale_log2;
    float* X;        // [B*L, d] fp32 residual stream between layers
    _Float16* Qh;    // [n_layers][B, H, L, dh] fp16 (hi part for layer 0)
    _Float16* Kh;
    _Float16* Ql;    // [B, H, L, dh] fp16 lo parts of layer 0
    _Float16* Kl;
    _Float16* Vt;    // [n_layers][B, H, dh, Lp] fp16
    float* Op;       // [B*H*Ctot][64][dh] fp32 partial attention outputs
    float2* ML;      // [B*H*Ctot][64] (running max in log2 units, sum)
    unsigned long long* audit;  // tile counters of the audit build (null otherwise)
    LayerPtrs lw[SEQ_MAX_LAYERS];
};

// Fused row kernel of the layer-wise path (16-bit I/O, d in {64, 128, 256}):
// for one 64-row tile, the out-projection of the attention output + bias +
// residual + LayerNorm, the FFN (exact-erf GELU) + bias + residual +
// LayerNorm, then the next layer's QKV projection (head-major Q and K, V^T)
// or, after the last layer, y.
struct RowArgs {
    const void* O;   // [B*L, d] fp16 attention output of this layer
    float* X;        // [B*L, d] fp32 residual stream: layer input, overwritten with the layer output
    void* y;         // [B, L, d] I/O dtype, written after the last layer
    _Float16* Q;     // next layer: [B, H, L, dh] fp16
    _Float16* K;     // next layer: [B, H, L, dh] fp16, multiplied by kscale
    _Float16* Vt;    // next layer: [B, H, dh, Lp] fp16
    int B, L, Lp, F;
    float eps;
    float kscale;    // 0 means 1
    int last;        // 1: write y instead of the next layer's Q, K, V^T
    LayerPtrs w;     // this layer
    LayerPtrs wn;    // next layer (unused when last)
};
bool row_supported(Mode m, int d, int dh, int f);
hipError_t launch_row(Mode m, int d, int dh, const RowArgs& a, hipStream_t s);

// Fixed tile shapes shared with the planner.
constexpr int ATT_KT = 64;   // keys per attention tile
constexpr int ATT_BQ = 64;   // queries per attention workgroup

hipError_t launch_prep(Mode m, const void* x, float* Xr, void* A, long n, hipStream_t s);
// Zeroes columns [L, Lp) of every V^T row (rows of Lp fp16).
hipError_t launch_vt_pad(void* Vt, long rows, int L, int Lp, hipStream_t s);
hipError_t launch_gemm(Mode m, Epi e, const GemmArgs& a, hipStream_t s);
// Multi-stage LDS-DMA pipelined GEMM (16-bit operand modes, K % 64 == 0).
bool gemm_pipe_ok(const GemmArgs& a);
hipError_t launch_gemm_pipe(Mode m, Epi e, const GemmArgs& a, hipStream_t s);
hipError_t launch_attn(Mode m, int dh, bool split_qk, const AttnArgs& a, hipStream_t s);
hipError_t launch_ln(Mode m, const float* Z, const void* gamma, const void* beta, float eps,
                     int T, int d, float* Xo, void* Ao, void* Y, hipStream_t s);

hipError_t launch_seq(Mode m, int d, int dh, const SeqArgs& a, hipStream_t s);
// Sequence-resident path for small shapes: one workgroup per sequence, fp32
// VALU arithmetic, any I/O dtype.
bool seq_small_supported(int d, int dh, int f, int L, int n_layers);
hipError_t launch_seq_small(Mode m, int d, int dh, const SeqArgs& a, hipStream_t s);
bool pq_supported(Mode m, int d, int dh, int f, int n_layers);
// One launch per stage of the task list: QKV0, then ATT and ROW per layer.
hipError_t launch_pq(Mode m, int d, int dh, const PqArgs& a, hipStream_t s);
bool seq_supported(Mode m, int d, int dh, int f, int L, int n_layers);

// Row layout of the LayerNorm kernel: lanes per row and float4 chunks per lane.
// Returns false when d is not supported.
bool ln_shape(int d, int* lanes_per_row, int* chunks);

}  // namespace tfl
