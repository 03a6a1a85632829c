// Sequence-resident path for small shapes (d <= 64, seq_len <= 64): one
// workgroup per sequence runs the whole layer stack in one launch with the
// sequence held in LDS ("Hyper-optimized megakernel-hybrid transformer
// inference", "Problem decomposition": sequence-resident family; latency-
// bound tiny batches are judged by time, "Headline results").
//
// At these sizes a forward is a few million multiply-adds, so the kernel
// keeps every value in fp32 with no operand rounding at all: projections on
// fp32 MFMA (16 x 16 output blocks spread over the four waves), attention
// one thread per (head, query) with the exact two-pass softmax, LayerNorm
// one wave per row.
#include "common.h"
#include "kernels.h"

namespace tfl {

namespace {

constexpr int SS_THREADS = 256;

template <class T>
__device__ __forceinline__ float ld(const T* p, int i) { return to_f32(p[i]); }

}  // namespace

// LDS (rows padded to a multiple of 16 with zeros):
// X [L][D] (layer input / LayerNorm output), B1 [L][max(3D, F)] (QKV, then
// the out-projection sum, then the GELU hidden rows), B2 [L][D] (attention
// output, then the FFN sum).
template <class WT, int DH>
__global__ __launch_bounds__(SS_THREADS) void seq_small_kernel(SeqArgs p, int D) {
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
    for (int i = tid; i < LR * (2 * PX + P1); i += SS_THREADS) ss_lds[i] = 0.f;
    __syncthreads();
    for (int i = tid; i < L * D; i += SS_THREADS) X[(i / D) * PX + i % D] = ld(x, i);
    __syncthreads();
    const float scale = rsqrtf((float)DH);

    // out[r][n] = bias[n] + sum_k in[r][k] W[n][k] (+ res[r][n]) on fp32 MFMA
    // (16x16x4: exact fp32 products, fp32 accumulation); one 16 x 16 output
    // block per wave at a time, weights straight from global memory.
    auto linear = [&](const float* in, int pin, int K, const WT* W, const WT* bias, int N, float* out, int pout,
                      const float* res, bool gelu) {
        const int nb16 = N / 16, nblk = (LR / 16) * nb16;
        for (int blk = wave; blk < nblk; blk += SS_THREADS / 64) {
            const int rb = blk / nb16, nb = blk - rb * nb16;
            const float* a = in + (rb * 16 + c16) * pin + g;
            const WT* w = W + (size_t)(nb * 16 + c16) * K + g;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int k = 0; k < K; k += 4) acc = mfma_16x16x4(a[k], ld(w, k), acc);
            // result: rows rb*16 + 4g + e, feature nb*16 + c16
            const int n = nb * 16 + c16;
            const float bn = ld(bias, n);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = rb * 16 + 4 * g + e;
                if (r >= L) continue;
                float v = acc[e] + bn;
                if (gelu) v = gelu_erf(v);
                if (res) v += res[r * PX + n];
                out[r * pout + n] = v;
            }
        }
    };
    // rows of Z [L][D] (pitch PZ) -> LayerNorm -> X (two-pass, fp32, biased variance)
    auto layernorm = [&](const float* Z, int PZ, const WT* gam, const WT* bet) {
        for (int r = wave; r < L; r += SS_THREADS / 64) {
            float s = 0.f;
            for (int n = lane; n < D; n += 64) s += Z[r * PZ + n];
            s = wave_sum<64>(s);
            const float mean = s / (float)D;
            float q = 0.f;
            for (int n = lane; n < D; n += 64) {
                const float c = Z[r * PZ + n] - mean;
                q += c * c;
            }
            q = wave_sum<64>(q);
            const float rstd = 1.0f / sqrtf(q / (float)D + p.eps);
            for (int n = lane; n < D; n += 64) X[r * PX + n] = (Z[r * PZ + n] - mean) * rstd * ld(gam, n) + ld(bet, n);
        }
    };

    for (int l = 0; l < p.n_layers; l++) {
        const LayerPtrs& w = p.lw[l];
        linear(X, PX, D, (const WT*)w.w_qkv, (const WT*)w.b_qkv, 3 * D, B1, P1, nullptr, false);
        __syncthreads();
        // attention: four lanes per (head, query), lane s taking keys j = s mod 4
        // of j <= min(i, len - 1); exact two-pass softmax, partials combined
        // across the four lanes
        for (int u = tid >> 2; u < H * L; u += SS_THREADS / 4) {
            const int s4 = tid & 3;
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
            float m = -INFINITY;
            for (int j = s4; j <= nk; j += 4) m = fmaxf(m, score(j));
            m = fmaxf(m, __shfl_xor(m, 1, WAVE));
            m = fmaxf(m, __shfl_xor(m, 2, WAVE));
            float o[DH];
#pragma unroll
            for (int t = 0; t < DH; t++) o[t] = 0.f;
            float den = 0.f;
            for (int j = s4; j <= nk; j += 4) {
                const float e = expf(score(j) - m);
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
            den += __shfl_xor(den, 1, WAVE);
            den += __shfl_xor(den, 2, WAVE);
#pragma unroll
            for (int t = 0; t < DH; t++) {
                o[t] += __shfl_xor(o[t], 1, WAVE);
                o[t] += __shfl_xor(o[t], 2, WAVE);
            }
            if (s4 == 0) {
                const float inv = 1.0f / den;
#pragma unroll
                for (int t = 0; t < DH; t++) B2[i * PX + h * DH + t] = o[t] * inv;
            }
        }
        __syncthreads();
        // z = X + O Wo^T + b_o  (into B1), LayerNorm -> X
        linear(B2, PX, D, (const WT*)w.w_o, (const WT*)w.b_o, D, B1, P1, X, false);
        __syncthreads();
        layernorm(B1, P1, (const WT*)w.ln1_g, (const WT*)w.ln1_b);
        __syncthreads();
        // g = GELU(X W1^T + b1) (into B1), z2 = X + g W2^T + b2 (into B2), LayerNorm -> X
        linear(X, PX, D, (const WT*)w.w_1, (const WT*)w.b_1, F, B1, P1, nullptr, true);
        __syncthreads();
        linear(B1, P1, F, (const WT*)w.w_2, (const WT*)w.b_2, D, B2, PX, X, false);
        __syncthreads();
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
    return d <= 64 && (dh == 16 || dh == 32 || dh == 64) && L <= 64 && f % 16 == 0 &&
           n_layers <= SEQ_MAX_LAYERS && seq_small_lds(d, f, L) <= 64 * 1024;
}

template <class WT>
static hipError_t small_mode(int d, int dh, const SeqArgs& a, hipStream_t s) {
    const size_t lds = seq_small_lds(d, a.F, a.L);
    dim3 grid(a.B);
    switch (dh) {
        case 16: hipLaunchKernelGGL((seq_small_kernel<WT, 16>), grid, dim3(SS_THREADS), lds, s, a, d); break;
        case 32: hipLaunchKernelGGL((seq_small_kernel<WT, 32>), grid, dim3(SS_THREADS), lds, s, a, d); break;
        case 64: hipLaunchKernelGGL((seq_small_kernel<WT, 64>), grid, dim3(SS_THREADS), lds, s, a, d); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
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
