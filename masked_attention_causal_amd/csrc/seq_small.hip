// Sequence-resident path for small shapes (d <= 64, seq_len <= 64): one
// workgroup per sequence runs the whole layer stack in one launch with the
// sequence held in LDS ("Hyper-optimized megakernel-hybrid transformer
// inference", "Problem decomposition": sequence-resident family; latency-
// bound tiny batches are judged by time, "Headline results").
//
// At these sizes a forward is a few million multiply-adds, so the kernel
// keeps every value in fp32 with no operand rounding at all: projections on
// fp32 MFMA (16 x 16 output blocks spread over 8 or 16 waves, two or four
// per SIMD so they hide one another's latency), attention eight lanes per
// (head, query) with the exact two-pass softmax, LayerNorm eight lanes per
// row.  When every layer's weights fit in LDS beside the
// activations (WL), they are copied there once at the start, as fp32 rows
// padded to 4 floats past a multiple of 32 (the 16 rows of an MFMA operand
// then fall on distinct banks); each phase then waits on LDS, not on a
// global-memory round trip per dependent product.
#include "common.h"
#include "kernels.h"

namespace tfl {

namespace {

// Threads per workgroup: 16 waves (four per SIMD) where the kernel fits the
// 128 registers that allows (head dim 16), else 8 waves.
constexpr int ss_threads(int dh) { return dh == 16 ? 1024 : 512; }
constexpr int SS_MIN_THREADS = 512;

template <class T>
__device__ __forceinline__ float ld(const T* p, int i) { return to_f32(p[i]); }

// Four consecutive stored values (16-, 8- or 8-byte aligned) as fp32.
__device__ __forceinline__ f32x4 load4v(const float* q) { return *(const f32x4*)q; }
template <class T>
__device__ __forceinline__ f32x4 load4v(const T* q) {
    const uint2 r = *(const uint2*)q;
    const T* h = (const T*)&r;
    return f32x4{to_f32(h[0]), to_f32(h[1]), to_f32(h[2]), to_f32(h[3])};
}

// Four consecutive stored values read through a pointer known to be in
// global memory (a generic pointer would be read with a flat load, which the
// compiler orders with LDS work), kept as raw bits until widened, so a batch
// of reads can be in flight before the first conversion.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <class T>
using raw4 = typename std::conditional<sizeof(T) == 4, f32x4, u32x2>::type;
template <class T>
__device__ __forceinline__ raw4<T> load4g(const T* q) {
    return *(const __attribute__((address_space(1))) raw4<T>*)q;
}
__device__ __forceinline__ f32x4 widen4(const float*, f32x4 r) { return r; }
template <class T>
__device__ __forceinline__ f32x4 widen4(const T*, u32x2 r) {
    const T* h = (const T*)&r;
    return f32x4{to_f32(h[0]), to_f32(h[1]), to_f32(h[2]), to_f32(h[3])};
}

}  // namespace

// LDS (rows padded to a multiple of 16 with zeros):
// X [L][D] (layer input / LayerNorm output), B1 [L][max(3D, F)] (QKV, then
// the out-projection sum, then the GELU hidden rows), B2 [L][D] (attention
// output, then the FFN sum).
// Floats of one layer's weights in LDS: W_qkv, W_o, W_1 rows of D + 4, W_2 rows
// of F + 4, then b_qkv | b_o | ln1_g | ln1_b | b_1 | b_2 | ln2_g | ln2_b.
__host__ __device__ inline int ss_layer_floats(int D, int F) {
    return ((3 * D + D + F) * (D + 4) + D * (F + 4) + 9 * D + F + 3) & ~3;
}

template <class WT, int DH, bool WL>
__global__ __launch_bounds__(ss_threads(DH)) void seq_small_kernel(SeqArgs p, int D) {
    constexpr int SS_THREADS = ss_threads(DH);
    extern __shared__ __attribute__((aligned(16))) float ss_lds[];
    const int H = D / DH;
    const int L = p.L, F = p.F;
    const int LR = (L + 15) & ~15;                 // rows incl. padding
    const int W1 = 3 * D > F ? 3 * D : F;
    // Row pitches: 4 floats past a multiple of 32, so 16-byte reads stay
    // aligned and the 16 rows of an MFMA operand fall on 8 bank groups.
    const int PX = D + 4, P1 = W1 + 4;
    float* X = ss_lds;
    float* B1 = X + LR * PX;
    float* B2 = B1 + LR * P1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int b = blockIdx.x;
    int len = p.lens[b];
    len = len < 1 ? 1 : (len > L ? L : len);
    const WT* x = (const WT*)p.x + (size_t)b * L * D;
    // The input rows and (WL) every layer's weights are read as 16-byte
    // units (D is a multiple of 16).  All the loads of a batch are issued
    // before any LDS store, and the first batch's before the LDS is
    // cleared, so the whole prologue costs one memory round trip (a few at
    // d = 64), hidden in part under the clearing.
    constexpr int XB = (1024 + SS_THREADS - 1) / SS_THREADS;  // units per thread (L * D / 4 <= 1024)
    const int D4 = D / 4, F4 = F / 4;
    raw4<WT> xv[XB];
#pragma unroll
    for (int k = 0; k < XB; k++) {
        const int u = k * SS_THREADS + tid;
        xv[k] = load4g(x + 4 * (size_t)(u < L * D4 ? u : 0));  // unconditional: no branch to wait in
    }
    auto clear_and_store_x = [&]() {
        for (int i = tid; i < LR * (2 * PX + P1); i += SS_THREADS) ss_lds[i] = 0.f;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < XB; k++) {
            const int u = k * SS_THREADS + tid;
            if (u < L * D4) {
                const int r = u / D4;
                asm volatile("" : "+v"(xv[k]));  // widened here, after the wait, not at the load
                *(f32x4*)(X + r * PX + 4 * (u - r * D4)) = widen4((const WT*)nullptr, xv[k]);
            }
        }
    };
    float* const WLb = B2 + LR * PX;  // weights of every layer (WL only)
    const int LF = ss_layer_floats(D, F);
    if constexpr (WL) {
        // Each layer's weights and vectors as 16-byte units, in three
        // regions: the rows of W_qkv, W_o and W_1 (D columns each, stored as
        // consecutive LDS rows of D + 4), the rows of W_2 (F columns, rows of
        // F + 4), then the eight vectors.  In the two row regions a thread
        // keeps one column and steps over rows (threads / columns rows a
        // pass), so the layer and region of an iteration are the same for
        // the whole wave.  (F / 4 < 256 since the activations fit 64 KB of
        // LDS.)
        constexpr int WB = 16;  // units per thread per batch
        const int PA = SS_THREADS / D4, PB = SS_THREADS / F4;  // rows per pass
        const int rA = tid / D4, cA = 4 * (tid - rA * D4);
        const int rB = tid / F4, cB = 4 * (tid - rB * F4);
        const int RA = 4 * D + F;
        const int nA = (RA + PA - 1) / PA, nB = (D + PB - 1) / PB, nV = ((9 * D + F) / 4 + SS_THREADS - 1) / SS_THREADS;
        const int nI = nA + nB + nV, NIT = p.n_layers * nI;  // iterations per layer, in all
        const int V0 = RA * (D + 4) + D * (F + 4);  // first vector float
        for (int k0 = 0; k0 < NIT; k0 += WB) {
            raw4<WT> v[WB];
            int dst[WB];
#pragma unroll
            for (int k = 0; k < WB; k++) {
                dst[k] = -1;
                const WT* src = nullptr;
                const int l = (k0 + k) / nI, it = k0 + k - l * nI;  // wave-uniform
                if (l < p.n_layers) {
                    // The layer's pointers, in scalar registers first: a
                    // per-lane choice among them must select values, not
                    // load a pointer per lane from the argument block.
                    const LayerPtrs& w = p.lw[l];
                    if (it < nA) {
                        const WT *q0 = (const WT*)w.w_qkv, *q1 = (const WT*)w.w_o, *q2 = (const WT*)w.w_1;
                        asm volatile("" : "+s"(q0), "+s"(q1), "+s"(q2));
                        const int r = it * PA + rA;
                        if (rA < PA && r < RA) {
                            src = r < 3 * D   ? q0 + r * D + cA
                                  : r < 4 * D ? q1 + (r - 3 * D) * D + cA
                                              : q2 + (r - 4 * D) * D + cA;
                            dst[k] = r * (D + 4) + cA;
                        }
                    } else if (it < nA + nB) {
                        const int r = (it - nA) * PB + rB;
                        if (rB < PB && r < D) {
                            src = (const WT*)w.w_2 + r * F + cB;
                            dst[k] = RA * (D + 4) + r * (F + 4) + cB;
                        }
                    } else {
                        int j = 4 * ((it - nA - nB) * SS_THREADS + tid);  // float of b_qkv | b_o | ln1 | b_1 | b_2 | ln2
                        if (j < 9 * D + F) {
                            const WT* q[8] = {(const WT*)w.b_qkv, (const WT*)w.b_o, (const WT*)w.ln1_g, (const WT*)w.ln1_b,
                                              (const WT*)w.b_1,   (const WT*)w.b_2, (const WT*)w.ln2_g, (const WT*)w.ln2_b};
#pragma unroll
                            for (int e = 0; e < 8; e++) asm volatile("" : "+s"(q[e]));
                            dst[k] = V0 + j;
                            if (j < 3 * D) src = q[0] + j;
                            else if ((j -= 3 * D) < D) src = q[1] + j;
                            else if ((j -= D) < D) src = q[2] + j;
                            else if ((j -= D) < D) src = q[3] + j;
                            else if ((j -= D) < F) src = q[4] + j;
                            else if ((j -= F) < D) src = q[5] + j;
                            else if ((j -= D) < D) src = q[6] + j;
                            else src = q[7] + (j - D);
                        }
                    }
                    if (dst[k] >= 0) {
                        v[k] = load4g(src);
                        dst[k] += l * LF;
                    }
                }
            }
            if (k0 == 0) clear_and_store_x();
#pragma unroll
            for (int k = 0; k < WB; k++)
                if (dst[k] >= 0) *(f32x4*)(WLb + dst[k]) = widen4((const WT*)nullptr, v[k]);
        }
    } else {
        clear_and_store_x();
    }
    __syncthreads();
    // scores in base 2 (scaled by log2 e / sqrt(dh)): the softmax weights are
    // then 2^(s - max) on the hardware exp2, the same values as e^ in base e
    const float scale = rsqrtf((float)DH) * 1.4426950408889634f;

    // out[r][n] = bias[n] + sum_k in[r][k] W[n][k] (+ res[r][n]) on fp32 MFMA
    // (16x16x4: exact fp32 products, fp32 accumulation); one 16 x 16 output
    // block per wave at a time; W rows pw elements apart (global memory in
    // the stored dtype, or the fp32 LDS copy).
    auto linear = [&](const float* in, int pin, int K, auto W, int pw, auto bias, int N, float* out, int pout,
                      const float* res, bool gelu) {
        const int nb16 = N / 16, nblk = (LR / 16) * nb16;
        for (int blk = wave; blk < nblk; blk += SS_THREADS / 64) {
            const int rb = blk / nb16, nb = blk - rb * nb16;
            const float* a = in + (rb * 16 + c16) * pin + g;
            const auto w = W + (size_t)(nb * 16 + c16) * pw + g;
            // result: rows rb*16 + 4g + e, feature nb*16 + c16; its bias and
            // residual (rows below LR, in LDS) are read before the products
            const int n = nb * 16 + c16;
            const float bn = ld(bias, n);
            float rv[4] = {0.f, 0.f, 0.f, 0.f};
            if (res) {
#pragma unroll
                for (int e = 0; e < 4; e++) rv[e] = res[(rb * 16 + 4 * g + e) * PX + n];
            }
            // four accumulators over interleaved K slices (K is a multiple of
            // 32), so four product chains overlap instead of one running K / 4
            // dependent products
            f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0, acc3 = acc0;
#pragma unroll 2
            for (int k = 0; k < K; k += 16) {
                acc0 = mfma_16x16x4(a[k], ld(w, k), acc0);
                acc1 = mfma_16x16x4(a[k + 4], ld(w, k + 4), acc1);
                acc2 = mfma_16x16x4(a[k + 8], ld(w, k + 8), acc2);
                acc3 = mfma_16x16x4(a[k + 12], ld(w, k + 12), acc3);
            }
            const f32x4 acc = (acc0 + acc1) + (acc2 + acc3);
            float vb[4] = {acc[0] + bn, acc[1] + bn, acc[2] + bn, acc[3] + bn};
            if (gelu) gelu_inplace<4>(vb);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = rb * 16 + 4 * g + e;
                if (r >= L) continue;
                out[r * pout + n] = vb[e] + rv[e];
            }
        }
    };
    // rows of Z [L][D] (pitch PZ) -> LayerNorm -> X (two-pass, fp32, biased
    // variance).  Eight lanes share a row (lane i of the 8 takes columns
    // i, i + 8, ...), so a wave normalises 8 rows at once and the row sums
    // reduce over the 8 lanes with DPP moves.
    auto sum8 = [](float v) {
        v += dpp_xor1(v);
        v += dpp_xor2(v);
        return v + dpp_mirror8(v);
    };
    auto layernorm = [&](const float* Z, int PZ, auto gam, auto bet) {
        // A lane's values (at most 8: D <= 64), gamma and beta are read once
        // into registers, all reads issued before the first sum; column
        // j8 + 8e is below D for every lane or for none (D is a multiple of 32).
        const int j8 = lane & 7;
        for (int r = wave * 8 + (lane >> 3); r - (lane >> 3) < L; r += SS_THREADS / 8) {
            const bool live = r < L;
            const int rr = live ? r : 0;
            float zv[8], gv[8], bv[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                zv[e] = gv[e] = bv[e] = 0.f;
                if (8 * e < D) {
                    const int n = j8 + 8 * e;
                    zv[e] = Z[rr * PZ + n];
                    gv[e] = ld(gam, n);
                    bv[e] = ld(bet, n);
                }
            }
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) s += zv[e];
            s = sum8(s);
            const float mean = s / (float)D;
            float q = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++)
                if (8 * e < D) {
                    const float c = zv[e] - mean;
                    q += c * c;
                }
            q = sum8(q);
            const float rstd = 1.0f / sqrtf(q / (float)D + p.eps);
            if (live) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    if (8 * e < D) X[r * PX + j8 + 8 * e] = (zv[e] - mean) * rstd * gv[e] + bv[e];
            }
        }
    };

    for (int l = 0; l < p.n_layers; l++) {
        const LayerPtrs& w = p.lw[l];
        const float* wl = WLb + (size_t)l * LF;
        const float* wv = wl + (3 * D + D + F) * (D + 4) + D * (F + 4);  // vectors of layer l
        if constexpr (WL)
            linear(X, PX, D, wl, D + 4, wv, 3 * D, B1, P1, nullptr, false);
        else
            linear(X, PX, D, (const WT*)w.w_qkv, D, (const WT*)w.b_qkv, 3 * D, B1, P1, nullptr, false);
        __syncthreads();
        // attention: ALN = 8 lanes per (head, query), lane s taking keys
        // j = s mod 8 of j <= min(i, len - 1); exact two-pass softmax,
        // partials combined across the eight lanes by DPP (16 lanes per
        // query with 16 waves measured slower)
        constexpr int ALN = 8, NKL = 64 / ALN;
        auto lanes_max = [](float v) {
            v = fmaxf(v, dpp_xor1(v));
            v = fmaxf(v, dpp_xor2(v));
            return fmaxf(v, dpp_mirror8(v));
        };
        auto lanes_sum = [](float v) {
            v += dpp_xor1(v);
            v += dpp_xor2(v);
            return v + dpp_mirror8(v);
        };
        for (int u = tid / ALN; u < H * L; u += SS_THREADS / ALN) {
            const int s8 = tid & (ALN - 1);
            const int h = u / L, i = u - h * L;
            const int nk = min(i, len - 1);
            float q[DH];
#pragma unroll
            for (int t = 0; t < DH; t += 4) {
                const float4 v4 = *(const float4*)(B1 + i * P1 + h * DH + t);
                q[t] = v4.x; q[t + 1] = v4.y; q[t + 2] = v4.z; q[t + 3] = v4.w;
            }
            auto score = [&](int j) {
                const float* k = B1 + j * P1 + D + h * DH;
                float sc = 0.f;
#pragma unroll
                for (int t = 0; t < DH; t += 4) {
                    const float4 k4 = *(const float4*)(k + t);
                    sc = fmaf(q[t], k4.x, sc);
                    sc = fmaf(q[t + 1], k4.y, sc);
                    sc = fmaf(q[t + 2], k4.z, sc);
                    sc = fmaf(q[t + 3], k4.w, sc);
                }
                return sc * scale;
            };
            // this lane's keys j = s8 + ALN c (c < NKL covers L <= 64): scores
            // kept from the max pass for the exponential pass
            float sc[NKL];
            float m = -INFINITY;
#pragma unroll
            for (int c = 0; c < NKL; c++) {
                const int j = s8 + ALN * c;
                sc[c] = j <= nk ? score(j) : -INFINITY;
                m = fmaxf(m, sc[c]);
            }
            m = lanes_max(m);
            float o[DH];
#pragma unroll
            for (int t = 0; t < DH; t++) o[t] = 0.f;
            float den = 0.f;
#pragma unroll
            for (int c = 0; c < NKL; c++) {
                const int j = s8 + ALN * c;
                if (j > nk) break;
                const float e = __builtin_amdgcn_exp2f(sc[c] - m);
                den += e;
                const float* v = B1 + j * P1 + 2 * D + h * DH;
#pragma unroll
                for (int t = 0; t < DH; t += 4) {
                    const float4 v4 = *(const float4*)(v + t);
                    o[t] = fmaf(e, v4.x, o[t]);
                    o[t + 1] = fmaf(e, v4.y, o[t + 1]);
                    o[t + 2] = fmaf(e, v4.z, o[t + 2]);
                    o[t + 3] = fmaf(e, v4.w, o[t + 3]);
                }
            }
            den = lanes_sum(den);
#pragma unroll
            for (int t = 0; t < DH; t++) o[t] = lanes_sum(o[t]);
            if (s8 == 0) {
                const float inv = 1.0f / den;
#pragma unroll
                for (int t = 0; t < DH; t++) B2[i * PX + h * DH + t] = o[t] * inv;
            }
        }
        __syncthreads();
        // z = X + O Wo^T + b_o  (into B1), LayerNorm -> X
        if constexpr (WL)
            linear(B2, PX, D, wl + 3 * D * (D + 4), D + 4, wv + 3 * D, D, B1, P1, X, false);
        else
            linear(B2, PX, D, (const WT*)w.w_o, D, (const WT*)w.b_o, D, B1, P1, X, false);
        __syncthreads();
        if constexpr (WL)
            layernorm(B1, P1, wv + 4 * D, wv + 5 * D);
        else
            layernorm(B1, P1, (const WT*)w.ln1_g, (const WT*)w.ln1_b);
        __syncthreads();
        // g = GELU(X W1^T + b1) (into B1), z2 = X + g W2^T + b2 (into B2), LayerNorm -> X
        if constexpr (WL)
            linear(X, PX, D, wl + 4 * D * (D + 4), D + 4, wv + 6 * D, F, B1, P1, nullptr, true);
        else
            linear(X, PX, D, (const WT*)w.w_1, D, (const WT*)w.b_1, F, B1, P1, nullptr, true);
        __syncthreads();
        if constexpr (WL)
            linear(B1, P1, F, wl + (4 * D + F) * (D + 4), F + 4, wv + 6 * D + F, D, B2, PX, X, false);
        else
            linear(B1, P1, F, (const WT*)w.w_2, F, (const WT*)w.b_2, D, B2, PX, X, false);
        __syncthreads();
        if constexpr (WL)
            layernorm(B2, PX, wv + 7 * D + F, wv + 8 * D + F);
        else
            layernorm(B2, PX, (const WT*)w.ln2_g, (const WT*)w.ln2_b);
        __syncthreads();
    }
    WT* y = (WT*)p.y + (size_t)b * L * D;
    for (int i = tid; i < L * D; i += SS_THREADS) y[i] = from_f32<WT>(X[(i / D) * PX + i % D]);
}

size_t seq_small_lds(int d, int f, int L) {
    const int w1 = 3 * d > f ? 3 * d : f;
    const int lr = (L + 15) & ~15;
    return (size_t)lr * (2 * (d + 4) + w1 + 4) * sizeof(float);
}

bool seq_small_supported(int d, int dh, int f, int L, int n_layers) {
    return d <= 64 && (dh == 16 || dh == 32 || dh == 64) && L <= 64 && f % 16 == 0 && f < 4 * SS_MIN_THREADS &&
           n_layers <= SEQ_MAX_LAYERS && seq_small_lds(d, f, L) <= 64 * 1024;
}

// Dynamic LDS with every layer's weights copied in (bytes).
static size_t seq_small_lds_wl(int d, int f, int L, int n_layers) {
    return seq_small_lds(d, f, L) + (size_t)n_layers * ss_layer_floats(d, f) * sizeof(float);
}

template <class WT, int DH, bool WL>
static hipError_t small_launch(const SeqArgs& a, int d, size_t lds, hipStream_t s) {
    if (lds > 64 * 1024) {
        // above 64 KB of dynamic LDS the kernel must be allowed it explicitly
        static const hipError_t set = hipFuncSetAttribute((const void*)seq_small_kernel<WT, DH, WL>,
                                                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (set != hipSuccess) return set;
    }
    hipLaunchKernelGGL((seq_small_kernel<WT, DH, WL>), dim3(a.B), dim3(ss_threads(DH)), lds, s, a, d);
    return hipGetLastError();
}

template <class WT>
static hipError_t small_mode(int d, int dh, const SeqArgs& a, hipStream_t s) {
    const size_t lds_wl = seq_small_lds_wl(d, a.F, a.L, a.n_layers);
    const bool wl = lds_wl <= 160 * 1024;
    const size_t lds = wl ? lds_wl : seq_small_lds(d, a.F, a.L);
    switch (dh) {
        case 16: return wl ? small_launch<WT, 16, true>(a, d, lds, s) : small_launch<WT, 16, false>(a, d, lds, s);
        case 32: return wl ? small_launch<WT, 32, true>(a, d, lds, s) : small_launch<WT, 32, false>(a, d, lds, s);
        case 64: return wl ? small_launch<WT, 64, true>(a, d, lds, s) : small_launch<WT, 64, false>(a, d, lds, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_seq_small(Mode m, int d, int dh, const SeqArgs& a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    switch (m) {
        case MODE_F32: return small_mode<float>(d, dh, a, s);
        case MODE_F16: return small_mode<f16>(d, dh, a, s);
        case MODE_BF16: return small_mode<bf16>(d, dh, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tfl
