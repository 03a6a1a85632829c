// Host-side launchers of the tfl kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tfl {

// Arithmetic mode, fixed by the I/O dtype.  On the layer-wise (TILED) path
// every GEMM and attention operand is fp16 with fp32 accumulation:
//   F32:  operands as two fp16 planes, the rounded value (hi) and the
//         rounding remainder times 2^11 (lo); each product is three MFMAs
//         (hi*hi + (hi*lo + lo*hi) * 2^-11).  Weights are split into the two
//         planes once per forward.
//   F16:  operands fp16 (activations rounded once to fp16), weights as given.
//   BF16: operands fp16; bf16 weights converted to fp16 once per forward.
// The residual stream and LayerNorm are fp32 in every mode.  The fused
// kernels (SEQ, PQ, row) read the weights in their I/O dtype themselves.
enum Mode { MODE_F32 = 0, MODE_F16 = 1, MODE_BF16 = 2 };

enum Epi { EPI_QKV = 0, EPI_GELU = 1, EPI_RES = 2 };

struct GemmArgs {
    const void* A;     // [M, K] fp16 (F32 mode: hi plane, lo plane M*K elements further)
    const void* W;     // [N, K] fp16 (F32 mode: hi plane, lo plane N*K elements further)
    const void* bias;  // [N] I/O dtype
    int M, N, K;       // K % 32 == 0, N % 4 == 0
    // EPI_QKV: N = 3d; writes Q, K [B, H, L, dh] and V^T [B, H, dh, Lp] fp16.
    // Q and K as fp16 planes of M*d elements each: the rounded value (hi) at
    // Q / K and, when split != 0, the rounding remainder (lo) one plane
    // further.
    float* Q;
    float* Kd;
    void* Vt;
    int L, Lp, H, dh, d;
    int split;
    // EPI_QKV: K is written multiplied by kscale (0 means 1).  The attention
    // kernels take keys pre-multiplied by log2(e)/sqrt(dh), so their score
    // products come out in the exp2 domain.
    float kscale;
    // EPI_GELU: out [M, N] fp16 (F32 mode: hi plane, lo plane M*N elements further)
    void* out;
    // EPI_RES: Z = acc + bias + R, [M, N] fp32
    const float* R;
    float* Z;
};

struct AttnArgs {
    const void* Q;     // [B, H, L, dh] fp16 hi plane
    const void* K;     // [B, H, L, dh], same
    const void* Ql;    // fp16 lo planes of Q and K (read when the scores are split)
    const void* Kl;
    const void* Vt;    // [B, H, dh, Lp] fp16; columns >= L hold zeros
    void* O;           // [B*L, d] fp16, head h at columns h*dh
    int o_lo;          // 1: also the remainder times 2^11, B*L*d elements further (F32 mode)
    // Per (sequence, head) row-norm maxima of Q and K written by qk_stats
    // (stats_nch chunks each): each workgroup picks its score variant from
    // them (split or single scores; weights with or without a reference).
    const float2* qk_stats;
    int stats_nch;
    int split_mode;    // 0 single fp16 scores, 1 split where the bound needs it, 2 always split
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

// QKV tasks per 64-row tile and layer on the PQ path.
constexpr int PQ_QKV_PARTS = 3;  // Q, K, V (each split over two head ranges at d >= 128)
constexpr int PQ_FS_MAX = 4;   // PQ FFN tasks per 64-row tile, at most

// A weight matrix converted to fp16 planes: n elements of src (I/O dtype)
// to dst (fp32: hi plane, then the lo plane times 2^11 n elements further).
struct WconvSeg {
    const void* src;
    _Float16* dst;
    long n;
};

// PQ path: the stack as a task list over 64-row tiles (QKV projection,
// split-K attention, out-projection + LayerNorm, FFN parts; the LayerNorm
// after the FFN runs where the rows are next loaded), run as one launch per
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
    float* X1;       // [B*L, d] fp32 rows after attention + LayerNorm (from the FFN tasks of part 0)
    float* FP;       // [FS][B*L, d] fp32 FFN down-projection partials
    int FS;          // FFN tasks per tile (each F / FS hidden features)
    _Float16* Qh;    // [n_layers][B, H, L, dh] fp16 q * log2(e)/sqrt(dh) (hi part for layer 0)
    _Float16* Kh;
    _Float16* Ql;    // [B, H, L, dh] fp16 lo parts of layer 0
    _Float16* Kl;
    _Float16* Vt;    // [n_layers][B, H, dh, Lp] fp16
    _Float16* Op;    // [B*H*Ctot][64][dh] fp16 partial attention outputs, normalised by their sums
    float2* ML;      // [B*H*Ctot][64] (running max in log2 units, sum)
    unsigned long long* audit;  // tile counters of the audit build (null otherwise)
    LayerPtrs lw[SEQ_MAX_LAYERS];
    // fp16 weight matrices per layer (W_qkv, W_o, W_1, W_2): the given ones
    // with fp16 I/O, else converted once per forward; with fp32 I/O each is
    // followed by its lo plane (rounding remainder times 2^11)
    const _Float16* wh[SEQ_MAX_LAYERS][4];
    // bf16 / fp32 I/O: the weights the first attention stage converts into
    // the planes of wh (every weight but the first layer's W_qkv, which the
    // first QKV stage reads as given); nconv = 0 with fp16 I/O
    WconvSeg conv[4 * SEQ_MAX_LAYERS];
    int nconv;
    // [B H][NT] per (sequence, head) and 64-row tile bounds on the largest
    // row norm of the current layer's Q and K (written by the QKV tasks):
    // each attention task's score variant
    float2* qk_stats;
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

// x (I/O dtype) -> fp32 residual Xr and fp16 operand A (F32 mode: hi plane
// at A, lo plane n elements further).
hipError_t launch_prep(Mode m, const void* x, float* Xr, void* A, long n, hipStream_t s);
// Zeroes columns [L, Lp) of every V^T row (rows of Lp fp16).
hipError_t launch_vt_pad(void* Vt, long rows, int L, int Lp, hipStream_t s);
hipError_t launch_gemm(Mode m, Epi e, const GemmArgs& a, hipStream_t s);
// Weight staging of the layer-wise path (BF16 and F32 modes): each segment's
// n source weights (I/O dtype) become n fp16 values at dst (F32 mode: hi at
// dst, lo times 2^11 at dst + n).  n % 8 == 0.
constexpr int WCONV_MAX_SEGS = 32;
struct WconvArgs {
    WconvSeg seg[WCONV_MAX_SEGS];
    int nseg;
};
hipError_t launch_wconv(Mode m, const WconvArgs& a, hipStream_t s);
// atomicMax of the fp32 bits of max |v| over n values (n % 4 == 0) into *out.
hipError_t launch_amax(int dtype_size, bool is_bf16, const void* x, long n, unsigned* out, hipStream_t s);
hipError_t launch_attn(Mode m, int dh, const AttnArgs& a, hipStream_t s);
// Row-norm maxima of the Q and K hi planes ([BH, L, dh] fp16) per (sequence,
// head) and chunk of rows: out [BH][qk_stats_chunks(L)] (max |q|, max |k|).
int qk_stats_chunks(int L);
hipError_t launch_qk_stats(int dh, const void* Q, const void* K, int BH, int L, float2* out, hipStream_t s);
// LayerNorm of fp32 rows Z: optionally to the fp32 residual Xo, the fp16
// operand Ao (F32 mode: hi plane, lo plane T*d elements further) and the I/O
// dtype output Y.
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
