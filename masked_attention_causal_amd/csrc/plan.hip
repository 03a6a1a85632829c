// Plans and launch sequences.
//
// The dispatcher is a fixed rule over (dtype, batch, seq_len, d_model,
// heads, FFN width, layers) evaluated once at tfl_create, never a run-time
// search: "KernelForge", "What it does" (a frozen table consulted at run
// time, no autotuning, no nondeterminism) and "Hyper-optimized
// megakernel-hybrid transformer inference", "Problem decomposition"
// (families by residency and by binding resource).
#include <climits>
#include <cmath>
#include <cstdio>

#include "common.h"
#include "plan.h"

namespace tfl {

size_t dtype_size(int dtype) { return dtype == TFL_F32 ? 4 : 2; }

unsigned long long* audit_counters = nullptr;

static Mode mode_of(int dtype) { return dtype == TFL_F32 ? MODE_F32 : (dtype == TFL_F16 ? MODE_F16 : MODE_BF16); }

// Compute units of the target part (MI355X); the rule below compares the
// number of attention work units against it.
constexpr long PQ_CU_COUNT = 256;

int choose_path(const tfl_config& c) {
    const int dh = c.d_model / c.n_heads;
    const Mode m = mode_of(c.dtype);
    // Short sequences: one workgroup keeps two whole sequences on chip for the
    // whole stack (one launch, no intermediate HBM traffic).
    if (seq_supported(m, c.d_model, dh, c.d_ffn, c.seq_len, c.n_layers)) return TFL_PATH_SEQ;
    // Tiny widths: one workgroup per sequence, one launch for the stack.
    if (seq_small_supported(c.d_model, dh, c.d_ffn, c.seq_len, c.n_layers)) return TFL_PATH_SEQ;
    // Few long sequences: fewer (sequence, head, 64-query tile) units than
    // compute units, so per-stage launches leave most of the chip idle; one
    // task list with split-K attention tasks over 64-row tiles fills it instead.
    const long units = (long)c.batch * c.n_heads * ((c.seq_len + 63) / 64);
    if (units < PQ_CU_COUNT && pq_supported(m, c.d_model, dh, c.d_ffn, c.n_layers)) return TFL_PATH_PQ;
    return TFL_PATH_TILED;
}

static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

tfl_status make_plan(const tfl_config& c, Plan* p, std::string* why) {
    if (c.n_layers < 1 || c.d_model < 1 || c.n_heads < 1 || c.d_ffn < 1 || c.batch < 1 || c.seq_len < 1) {
        *why = "all sizes must be >= 1";
        return TFL_E_INVALID;
    }
    if (c.d_model % c.n_heads != 0) {
        *why = "d_model must be a multiple of n_heads";
        return TFL_E_INVALID;
    }
    if (c.dtype != TFL_F32 && c.dtype != TFL_F16 && c.dtype != TFL_BF16) {
        *why = "unknown dtype";
        return TFL_E_INVALID;
    }
    if (c.force_path < TFL_PATH_AUTO || c.force_path > TFL_PATH_PQ_SINGLE) {
        *why = "unknown force_path";
        return TFL_E_INVALID;
    }
    if (c.force_path == TFL_PATH_PQ_SINGLE) {
        *why = "the single persistent launch of the PQ tasks is disabled: its one GPU run did not finish and "
               "no cause has been shown; TFL_PATH_PQ runs the same tasks as one launch per stage";
        return TFL_E_UNSUPPORTED;
    }
    const int dh = c.d_model / c.n_heads;
    if (dh != 16 && dh != 32 && dh != 64) {
        *why = "head dim must be 16, 32 or 64";
        return TFL_E_UNSUPPORTED;
    }
    int lpr, nc;
    if (c.d_model % 32 != 0 || c.d_model > 1024 || !ln_shape(c.d_model, &lpr, &nc)) {
        *why = "d_model must be a multiple of 32, at most 1024, with an odd part of at most 7 (LayerNorm row split)";
        return TFL_E_UNSUPPORTED;
    }
    if (c.d_ffn % 32 != 0) {
        *why = "d_ffn must be a multiple of 32";
        return TFL_E_UNSUPPORTED;
    }
    const long T = (long)c.batch * c.seq_len;
    if (c.batch > 65535 || T > 65535L * 64) {
        *why = "batch must be <= 65535 and batch*seq_len <= 4194240";
        return TFL_E_UNSUPPORTED;
    }
    int path = c.force_path == TFL_PATH_AUTO ? choose_path(c) : c.force_path;
    const Mode mode = mode_of(c.dtype);
    if ((path == TFL_PATH_PQ && !pq_supported(mode, c.d_model, dh, c.d_ffn, c.n_layers)) ||
        (path == TFL_PATH_SEQ && !seq_supported(mode, c.d_model, dh, c.d_ffn, c.seq_len, c.n_layers) &&
         !seq_small_supported(c.d_model, dh, c.d_ffn, c.seq_len, c.n_layers))) {
        *why = "requested path is not available for this shape";
        return TFL_E_UNSUPPORTED;
    }
    Plan q{};
    q.path = path;
    q.mode = mode;
    q.n_layers = c.n_layers;
    q.d = c.d_model;
    q.H = c.n_heads;
    q.dh = dh;
    q.f = c.d_ffn;
    q.B = c.batch;
    q.L = c.seq_len;
    q.Lp = (c.seq_len + ATT_KT - 1) / ATT_KT * ATT_KT;
    q.T = T;
    q.eps = c.ln_eps > 0.f ? c.ln_eps : 1e-5f;
    q.op = q.mode == MODE_F32 ? 4 : 2;
    if (path == TFL_PATH_SEQ) {
        q.ws_bytes = 0;  // everything stays on chip
        q.seq_kind = seq_supported(mode, c.d_model, dh, c.d_ffn, c.seq_len, c.n_layers) ? 0 : 1;
        if (q.seq_kind == 0)
            std::snprintf(q.name, sizeof(q.name), "SEQ/2x64tok/w8/f16op");
        else
            std::snprintf(q.name, sizeof(q.name), "SEQ/small/1seq/f32");
        *p = q;
        return TFL_OK;
    }
    const size_t Td = (size_t)T * q.d;
    if (path == TFL_PATH_PQ) {
        const int NT = q.Lp / ATT_KT;
        const int BNT = q.B * NT;
        q.pq_ks = 8;
        q.pq_ctot = NT + q.pq_ks * (NT / q.pq_ks) * (NT / q.pq_ks - 1) / 2 + (NT / q.pq_ks) * (NT % q.pq_ks);
        const long n_att = (long)q.B * q.H * q.pq_ctot;
        // FFN tasks per tile: a divisor of the F/128 hidden chunks, up to 4,
        // so the FFN stage has about one workgroup per CU
        const int nch = q.f / 128;
        int fs = 1;
        for (int c = 1; c <= PQ_FS_MAX && c <= nch; c++)
            if (nch % c == 0 && (long)BNT * c <= 256) fs = c;
        q.pq_fs = fs;
        const long n_tasks = (long)q.n_layers * ((2 * PQ_QKV_PARTS + fs) * (long)BNT + n_att) + 8L * BNT;
        if (n_tasks > INT_MAX / 2) {
            *why = "too many tasks for the PQ path";
            return TFL_E_UNSUPPORTED;
        }
        q.pq_tasks = (int)n_tasks;
        const size_t slots = (size_t)n_att;
        size_t o = 0;
        q.off_pX = o;  o += up256(Td * 4);
        q.off_pX1 = o; o += up256(Td * 4);
        q.off_pFP = o; o += up256(Td * 4 * fs);
        q.off_Qh = o;  o += up256(Td * 2 * q.n_layers);
        q.off_Kh = o;  o += up256(Td * 2 * q.n_layers);
        q.off_Ql = o;  o += up256(Td * 2);
        q.off_Kl = o;  o += up256(Td * 2);
        q.off_pVt = o; o += up256((size_t)q.B * q.d * q.Lp * 2 * q.n_layers);
        q.off_Op = o;  o += up256(slots * 64 * q.dh * 2);
        q.off_ML = o;  o += up256(slots * 64 * 8);
        q.off_pS = o;  o += up256((size_t)BNT * q.H * sizeof(float2));
        // fp16 weight planes (bf16 / fp32 I/O; fp32: hi and lo planes)
        q.off_pW = o;
        if (q.mode != MODE_F16)
            o += up256(((size_t)4 * q.d * q.d + (size_t)2 * q.d * q.f) * q.n_layers * (q.mode == MODE_F32 ? 4 : 2));
        q.ws_bytes = o;
        std::snprintf(q.name, sizeof(q.name), "PQ/t64.ks%d.fs%d/staged/%s", q.pq_ks, q.pq_fs,
                      q.mode == MODE_F32 ? "f32io.f16op" : "f16op");
        *p = q;
        return TFL_OK;
    }
    // V^T rows are padded to whole 128-key tiles (the head-dim-16 attention
    // kernel reads 128 keys per tile).
    q.Lp = (c.seq_len + 127) / 128 * 128;
    // d_model <= 256 with 16-bit I/O: after attention, one fused row kernel
    // per layer (out-projection, LayerNorms, FFN, next QKV), so Z, X1 and
    // the FFN activations never reach HBM
    q.row_fused = row_supported(mode, q.d, q.dh, q.f);
    // GEMM operands are fp16 planes: one (16-bit I/O) or two (fp32 I/O: hi
    // and the remainder times 2^11), q.op bytes per element in all
    size_t o = 0;
    q.off_Xr = o; o += up256(Td * 4);
    if (!q.row_fused) {
        q.off_X1 = o; o += up256(Td * 4);
        q.off_Z = o;  o += up256(Td * 4);
    }
    q.off_Q = o;  o += up256(Td * 4);
    q.off_K = o;  o += up256(Td * 4);
    q.off_A = o;  o += up256(Td * q.op);
    q.off_O = o;  o += up256(Td * q.op);
    q.off_Vt = o; o += up256((size_t)q.B * q.d * q.Lp * 2);
    if (!q.row_fused) {
        q.off_G = o;  o += up256((size_t)T * q.f * q.op);
    }
    // weights in their fp16 planes: every GEMM weight of every layer, or,
    // with the fused row kernel (which reads the I/O dtype itself), the
    // first layer's QKV weights only
    q.n_wconv = 0;
    q.off_W = o;
    if (q.mode != MODE_F16) {
        q.n_wconv = q.row_fused ? 1 : q.n_layers;
        const size_t per_layer = q.row_fused ? (size_t)3 * q.d * q.d : (size_t)4 * q.d * q.d + (size_t)2 * q.d * q.f;
        o += up256(per_layer * q.n_wconv * q.op);
    }
    // per-layer Q/K row-norm maxima (the attention's score variant)
    q.off_S = o;
    o += up256((size_t)q.B * q.H * qk_stats_chunks(q.L) * sizeof(float2));
    q.ws_bytes = o;
    std::snprintf(q.name, sizeof(q.name), "TILED/attn.q%d.k%d/%s%s", ATT_BQ, ATT_KT,
                  q.mode == MODE_F32 ? "f32io.f16x3" : "f16op", q.row_fused ? "/rowfused" : "");
    *p = q;
    return TFL_OK;
}

// Records the timer's events around one launch when its stage is armed.
struct Timed {
    StageTimer* t;
    hipStream_t s;
    int idx = -1;
    Timed(StageTimer* t_, int stage, hipStream_t s_) : t(t_), s(s_) {
        if (t && t->stage == stage && t->n < t->cap) {
            idx = t->n++;
            (void)hipEventRecord(t->start[idx], s);
        }
    }
    hipError_t done(hipError_t e) {
        if (idx >= 0) (void)hipEventRecord(t->stop[idx], s);
        return e;
    }
};

// fp16 weight planes of layer l's four GEMM matrices in the workspace (BF16
// and F32 modes), laid out as the plan sized them.
struct WPlanes {
    const void *qkv, *o, *w1, *w2;
};
static WPlanes weight_planes(const Plan& P, char* ws, int l) {
    const size_t ew = P.op / 2;  // fp16 planes per weight
    const size_t dd = (size_t)P.d * P.d, df = (size_t)P.d * P.f;
    const size_t per_layer = P.row_fused ? 3 * dd : 4 * dd + 2 * df;
    const f16* base = (const f16*)(ws + P.off_W) + (size_t)l * per_layer * ew;
    WPlanes w;
    w.qkv = base;
    w.o = base + 3 * dd * ew;
    w.w1 = base + 4 * dd * ew;
    w.w2 = base + (4 * dd + df) * ew;
    return w;
}

static hipError_t run_tiled(const Plan& P, const tfl_layer* layers, const void* x, const int32_t* lens, void* y,
                            char* ws, hipStream_t s, StageTimer* T) {
    float* Xr = (float*)(ws + P.off_Xr);
    float* X1 = (float*)(ws + P.off_X1);
    float* Z = (float*)(ws + P.off_Z);
    float* Q = (float*)(ws + P.off_Q);
    float* K = (float*)(ws + P.off_K);
    void* A = ws + P.off_A;
    void* O = ws + P.off_O;
    void* Vt = ws + P.off_Vt;
    void* G = ws + P.off_G;
    const int M = (int)P.T;
    const bool f32 = P.mode == MODE_F32;
    hipError_t e = hipSuccess;
    {
        Timed tm(T, TFL_STAGE_PREP, s);
        // weights to fp16 planes, up to WCONV_MAX_SEGS matrices per launch
        const size_t dd = (size_t)P.d * P.d, df = (size_t)P.d * P.f;
        WconvArgs wa{};
        for (int l = 0; l < P.n_wconv && e == hipSuccess; l++) {
            const tfl_layer& w = layers[l];
            const WPlanes wp = weight_planes(P, ws, l);
            const void* src[4] = {w.w_qkv, w.w_o, w.w_1, w.w_2};
            const void* dst[4] = {wp.qkv, wp.o, wp.w1, wp.w2};
            const size_t n[4] = {3 * dd, dd, df, df};
            for (int k = 0; k < (P.row_fused ? 1 : 4); k++) {
                wa.seg[wa.nseg++] = WconvSeg{src[k], (f16*)dst[k], (long)n[k]};
                if (wa.nseg == WCONV_MAX_SEGS) {
                    e = launch_wconv(P.mode, wa, s);
                    wa.nseg = 0;
                }
            }
        }
        if (e == hipSuccess) e = launch_wconv(P.mode, wa, s);
        if (e == hipSuccess) e = launch_prep(P.mode, x, Xr, A, (long)P.T * P.d, s);
        if (e == hipSuccess) e = launch_vt_pad(Vt, (long)P.B * P.d, P.L, P.Lp, s);
        e = tm.done(e);
    }
    if (e != hipSuccess) return e;
    for (int l = 0; l < P.n_layers; l++) {
        const tfl_layer& w = layers[l];
        const bool last = l == P.n_layers - 1;
        const WPlanes wp =
            l < P.n_wconv ? weight_planes(P, ws, l) : WPlanes{w.w_qkv, w.w_o, w.w_1, w.w_2};
        // Scores of the first layer see the raw input (up to 1e3 in scale):
        // fp32-accurate there; LayerNorm bounds every later layer's input.
        // With fp32 I/O every layer's scores are split.
        const bool split = f32 || l == 0;
        GemmArgs g{};
        g.A = A; g.W = wp.qkv; g.bias = w.b_qkv;
        g.M = M; g.N = 3 * P.d; g.K = P.d;
        g.Q = Q; g.Kd = K; g.Vt = Vt;
        g.L = P.L; g.Lp = P.Lp; g.H = P.H; g.dh = P.dh; g.d = P.d;
        g.split = split;
        // the attention kernels read K pre-scaled into exp2 units
        g.kscale = (float)(1.4426950408889634 / std::sqrt((double)P.dh));
        // with the fused row kernel, layers after the first get their Q, K
        // and V^T from the previous layer's row kernel
        if (!P.row_fused || l == 0) {
            Timed tm(T, TFL_STAGE_QKV, s);
            if ((e = tm.done(launch_gemm(P.mode, EPI_QKV, g, s))) != hipSuccess) return e;
        }

        AttnArgs a{};
        a.Q = Q; a.K = K; a.Vt = Vt; a.O = O; a.lens = lens;
        a.o_lo = f32;
        // fp16 lo planes follow the hi planes in the same buffers
        a.Ql = (const f16*)Q + (size_t)P.T * P.d;
        a.Kl = (const f16*)K + (size_t)P.T * P.d;
        a.B = P.B; a.H = P.H; a.L = P.L; a.Lp = P.Lp; a.d = P.d;
        a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)P.dh));
        a.audit = audit_counters;
        {
            Timed tm(T, TFL_STAGE_ATTN, s);
            // Q/K magnitudes of each (sequence, head) choose its score
            // variant: with 16-bit I/O the first layer splits only where they
            // need it, fp32 I/O splits every layer; bounded scores take no
            // softmax reference.  The statistics are formed where they can
            // pay: the first layer of 16-bit I/O (the split), and head dim 16
            // (whose softmax work dominates; at head dims 32/64 the bounded
            // weights measured no faster than the statistics launch costs)
            a.split_mode = f32 ? 2 : (l == 0 ? 1 : 0);
            if (a.split_mode == 1 || P.dh == 16) {
                float2* st = (float2*)(ws + P.off_S);
                a.qk_stats = st;
                a.stats_nch = qk_stats_chunks(P.L);
                e = launch_qk_stats(P.dh, Q, K, P.B * P.H, P.L, st, s);
            }
            if (e == hipSuccess) e = launch_attn(P.mode, P.dh, a, s);
            if ((e = tm.done(e)) != hipSuccess) return e;
        }
        if (P.row_fused) {
            // out-projection .. LayerNorm 2 and the next layer's QKV in one launch
            RowArgs r{};
            r.O = O; r.X = Xr; r.y = y;
            r.Q = (f16*)Q; r.K = (f16*)K; r.Vt = (f16*)Vt;
            r.B = P.B; r.L = P.L; r.Lp = P.Lp; r.F = P.f;
            r.eps = P.eps;
            r.kscale = (float)(1.4426950408889634 / std::sqrt((double)P.dh));
            r.last = last ? 1 : 0;
            r.w = LayerPtrs{w.w_qkv, w.b_qkv, w.w_o, w.b_o, w.ln1_g, w.ln1_b, w.w_1, w.b_1, w.w_2, w.b_2, w.ln2_g, w.ln2_b};
            if (!last) {
                const tfl_layer& n = layers[l + 1];
                r.wn = LayerPtrs{n.w_qkv, n.b_qkv, n.w_o, n.b_o, n.ln1_g, n.ln1_b, n.w_1, n.b_1, n.w_2, n.b_2, n.ln2_g,
                                 n.ln2_b};
            }
            Timed tm(T, TFL_STAGE_ROW, s);
            if ((e = tm.done(launch_row(P.mode, P.d, P.dh, r, s))) != hipSuccess) return e;
            continue;
        }

        GemmArgs r{};
        r.A = O; r.W = wp.o; r.bias = w.b_o; r.M = M; r.N = P.d; r.K = P.d; r.R = Xr; r.Z = Z;
        {
            Timed tm(T, TFL_STAGE_OUT, s);
            if ((e = tm.done(launch_gemm(P.mode, EPI_RES, r, s))) != hipSuccess) return e;
        }
        {
            Timed tm(T, TFL_STAGE_LN, s);
            if ((e = tm.done(launch_ln(P.mode, Z, w.ln1_g, w.ln1_b, P.eps, M, P.d, X1, A, nullptr, s))) != hipSuccess)
                return e;
        }

        GemmArgs u{};
        u.A = A; u.W = wp.w1; u.bias = w.b_1; u.M = M; u.N = P.f; u.K = P.d; u.out = G;
        {
            Timed tm(T, TFL_STAGE_FFN1, s);
            if ((e = tm.done(launch_gemm(P.mode, EPI_GELU, u, s))) != hipSuccess) return e;
        }
        GemmArgs dn{};
        dn.A = G; dn.W = wp.w2; dn.bias = w.b_2; dn.M = M; dn.N = P.d; dn.K = P.f; dn.R = X1; dn.Z = Z;
        {
            Timed tm(T, TFL_STAGE_FFN2, s);
            if ((e = tm.done(launch_gemm(P.mode, EPI_RES, dn, s))) != hipSuccess) return e;
        }
        {
            Timed tm(T, TFL_STAGE_LN, s);
            if (last)
                e = launch_ln(P.mode, Z, w.ln2_g, w.ln2_b, P.eps, M, P.d, nullptr, nullptr, y, s);
            else
                e = launch_ln(P.mode, Z, w.ln2_g, w.ln2_b, P.eps, M, P.d, Xr, A, nullptr, s);
            if ((e = tm.done(e)) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

static hipError_t run_seq(const Plan& P, const tfl_layer* layers, const void* x, const int32_t* lens, void* y,
                          hipStream_t s, StageTimer* T) {
    SeqArgs a{};
    a.x = x;
    a.y = y;
    a.lens = lens;
    a.B = P.B;
    a.L = P.L;
    a.F = P.f;
    a.n_layers = P.n_layers;
    a.eps = P.eps;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)P.dh));
    a.audit = audit_counters;
    for (int l = 0; l < P.n_layers; l++) {
        const tfl_layer& w = layers[l];
        a.lw[l] = LayerPtrs{w.w_qkv, w.b_qkv, w.w_o, w.b_o, w.ln1_g, w.ln1_b,
                            w.w_1, w.b_1, w.w_2, w.b_2, w.ln2_g, w.ln2_b};
    }
    Timed tm(T, TFL_STAGE_FUSED, s);
    if (P.seq_kind == 1) return tm.done(launch_seq_small(P.mode, P.d, P.dh, a, s));
    return tm.done(launch_seq(P.mode, P.d, P.dh, a, s));
}

static hipError_t run_pq(const Plan& P, const tfl_layer* layers, const void* x, const int32_t* lens, void* y,
                         char* ws, hipStream_t s, StageTimer* T) {
    PqArgs a{};
    a.x = x;
    a.y = y;
    a.lens = lens;
    a.B = P.B;
    a.L = P.L;
    a.Lp = P.Lp;
    a.NT = P.Lp / ATT_KT;
    a.F = P.f;
    a.n_layers = P.n_layers;
    a.KS = P.pq_ks;
    a.Ctot = P.pq_ctot;
    a.eps = P.eps;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)P.dh));
    a.X = (float*)(ws + P.off_pX);
    a.X1 = (float*)(ws + P.off_pX1);
    a.FP = (float*)(ws + P.off_pFP);
    a.FS = P.pq_fs;
    a.Qh = (_Float16*)(ws + P.off_Qh);
    a.Kh = (_Float16*)(ws + P.off_Kh);
    a.Ql = (_Float16*)(ws + P.off_Ql);
    a.Kl = (_Float16*)(ws + P.off_Kl);
    a.Vt = (_Float16*)(ws + P.off_pVt);
    a.Op = (_Float16*)(ws + P.off_Op);
    a.ML = (float2*)(ws + P.off_ML);
    a.qk_stats = (float2*)(ws + P.off_pS);
    a.audit = audit_counters;
    for (int l = 0; l < P.n_layers; l++) {
        const tfl_layer& w = layers[l];
        a.lw[l] = LayerPtrs{w.w_qkv, w.b_qkv, w.w_o, w.b_o, w.ln1_g, w.ln1_b,
                            w.w_1, w.b_1, w.w_2, w.b_2, w.ln2_g, w.ln2_b};
    }
    // fp16 weights: the given ones with fp16 I/O, else converted here
    const size_t dd = (size_t)P.d * P.d, df = (size_t)P.d * P.f, planes = P.mode == MODE_F32 ? 2 : 1;
    const size_t n[4] = {3 * dd, dd, df, df};
    // (converted by the first attention stage; the first QKV stage reads the
    // first layer's W_qkv as given)
    f16* cw = (f16*)(ws + P.off_pW);
    a.nconv = 0;
    for (int l = 0; l < P.n_layers; l++) {
        const tfl_layer& w = layers[l];
        const void* src[4] = {w.w_qkv, w.w_o, w.w_1, w.w_2};
        for (int k = 0; k < 4; k++) {
            if (P.mode == MODE_F16) {
                a.wh[l][k] = (const f16*)src[k];
            } else if (l == 0 && k == 0) {
                a.wh[l][k] = nullptr;
            } else {
                a.wh[l][k] = cw;
                a.conv[a.nconv++] = WconvSeg{src[k], cw, (long)n[k]};
                cw += n[k] * planes;
            }
        }
    }
    Timed tm(T, TFL_STAGE_FUSED, s);
    return tm.done(launch_pq(P.mode, P.d, P.dh, a, s));
}

hipError_t run_plan(const Plan& p, const tfl_layer* layers, const void* x, const int32_t* lens, void* y, char* ws,
                    hipStream_t s, StageTimer* timer) {
    switch (p.path) {
        case TFL_PATH_SEQ: return run_seq(p, layers, x, lens, y, s, timer);
        case TFL_PATH_PQ: return run_pq(p, layers, x, lens, y, ws, s, timer);
        case TFL_PATH_TILED: return run_tiled(p, layers, x, lens, y, ws, s, timer);
    }
    return hipErrorInvalidValue;
}

}  // namespace tfl
