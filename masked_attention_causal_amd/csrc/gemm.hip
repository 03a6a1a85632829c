// Projection GEMMs of the encoder layer on MFMA: C = A W^T + b with an
// epilogue per use.
//   EPI_QKV  : fused QKV projection; Q and K leave in fp32, head-major
//              [B, H, L, dh]; V leaves transposed per head, [B, H, dh, Lp],
//              so the attention kernel reads it as the A operand of P V.
//              (The QKV GEMM with the head-major transpose fused into it is
//              the custom kernel described in "Hyper-optimized megakernel-
//              hybrid transformer inference", "Problem decomposition",
//              hybrid family.)
//   EPI_GELU : FFN up-projection, exact-erf GELU in the epilogue
//              ("KernelForge", "How the LLM is used": exact erf).
//   EPI_RES  : out-projection / FFN down-projection plus bias plus the fp32
//              residual; LayerNorm follows in its own kernel.
//
// Tiling: 256 threads = 4 waves in a 2 x 2 arrangement; a wave owns a
// (BM/2) x (BN/2) block of 16 x 16 MFMA tiles.  A and W tiles are staged in
// LDS, double-buffered, with the next tile's global loads in flight while
// the current one is multiplied.
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace tfl {

template <class OpT, class WT, int EPI, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
    constexpr bool F32 = sizeof(OpT) == 4;
    // fp16 operands: BK = 32 halves per stage, 8-half chunks; fp32: BK = 16, 4-float chunks.
    constexpr int BK = F32 ? 16 : 32;
    constexpr int CH = F32 ? 4 : 8;                  // elements per 16-byte chunk
    constexpr int LDK = F32 ? BK + 1 : BK + 8;       // LDS row pitch (elements)
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int CPR = BK / CH;                     // chunks per tile row
    constexpr int A_CH = BM * CPR / 256, W_CH = BN * CPR / 256;
    static_assert(A_CH >= 1 && W_CH >= 1, "tile too small for 256 threads");
    typedef typename std::conditional<F32, float, f16>::type LT;
    __shared__ __attribute__((aligned(16))) LT As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) LT Ws[2][BN * LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int M = p.M, N = p.N, K = p.K;
    const OpT* __restrict__ A = (const OpT*)p.A;
    const WT* __restrict__ W = (const WT*)p.W;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // staging registers
    f16x8 ra[F32 ? 1 : A_CH], rw[F32 ? 1 : W_CH];
    float4 fa[F32 ? A_CH : 1], fw[F32 ? W_CH : 1];

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CH; i++) {
            const int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * CH;
            const int gm = m0 + r, gk = k0 + kc;
            const bool ok = gm < M && gk < K;
            if constexpr (F32) {
                fa[i] = ok ? *(const float4*)((const float*)A + (size_t)gm * K + gk) : float4{0.f, 0.f, 0.f, 0.f};
            } else {
                ra[i] = ok ? load8_as_f16(A + (size_t)gm * K + gk) : f16x8{};
            }
        }
#pragma unroll
        for (int i = 0; i < W_CH; i++) {
            const int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * CH;
            const int gn = n0 + r, gk = k0 + kc;
            const bool ok = gn < N && gk < K;
            if constexpr (F32) {
                fw[i] = ok ? *(const float4*)((const float*)W + (size_t)gn * K + gk) : float4{0.f, 0.f, 0.f, 0.f};
            } else {
                rw[i] = ok ? load8_as_f16(W + (size_t)gn * K + gk) : f16x8{};
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CH; i++) {
            const int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * CH;
            if constexpr (F32) {
                float* d = (float*)&As[buf][r * LDK + kc];
                d[0] = fa[i].x; d[1] = fa[i].y; d[2] = fa[i].z; d[3] = fa[i].w;
            } else {
                *(f16x8*)&As[buf][r * LDK + kc] = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < W_CH; i++) {
            const int c = tid + i * 256, r = c / CPR, kc = (c % CPR) * CH;
            if constexpr (F32) {
                float* d = (float*)&Ws[buf][r * LDK + kc];
                d[0] = fw[i].x; d[1] = fw[i].y; d[2] = fw[i].z; d[3] = fw[i].w;
            } else {
                *(f16x8*)&Ws[buf][r * LDK + kc] = rw[i];
            }
        }
    };

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const LT* as = As[buf];
        const LT* ws = Ws[buf];
        if constexpr (F32) {
#pragma unroll
            for (int kk = 0; kk < BK / 4; kk++) {
                float a[FM], b[FN];
#pragma unroll
                for (int i = 0; i < FM; i++) a[i] = as[(wm * WM + i * 16 + c16) * LDK + kk * 4 + g];
#pragma unroll
                for (int j = 0; j < FN; j++) b[j] = ws[(wn * WN + j * 16 + c16) * LDK + kk * 4 + g];
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++) acc[i][j] = mfma_16x16x4(a[i], b[j], acc[i][j]);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < BK / 32; kk++) {
                f16x8 a[FM], b[FN];
#pragma unroll
                for (int i = 0; i < FM; i++) a[i] = *(const f16x8*)&as[(wm * WM + i * 16 + c16) * LDK + kk * 32 + g * 8];
#pragma unroll
                for (int j = 0; j < FN; j++) b[j] = *(const f16x8*)&ws[(wn * WN + j * 16 + c16) * LDK + kk * 32 + g * 8];
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++) acc[i][j] = mfma_16x16x32(a[i], b[j], acc[i][j]);
            }
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    const WT* __restrict__ bias = (const WT*)p.bias;
#pragma unroll
    for (int j = 0; j < FN; j++) {
        const int n = n0 + wn * WN + j * 16 + c16;
        if (n >= N) continue;
        const float bn = to_f32(bias[n]);
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int m = m0 + wm * WM + i * 16 + g * 4 + e;
                if (m >= M) continue;
                const float v = acc[i][j][e] + bn;
                if constexpr (EPI == EPI_QKV) {
                    const int which = n / p.d, nn = n - which * p.d;
                    const int h = nn / p.dh, t = nn - h * p.dh;
                    const int b = m / p.L, pos = m - b * p.L;
                    const size_t bh = (size_t)b * p.H + h;
                    const size_t o = (bh * p.L + pos) * p.dh + t;
                    if (which == 2) {
                        ((OpT*)p.Vt)[(bh * p.dh + t) * p.Lp + pos] = from_f32<OpT>(v);
                    } else if constexpr (F32) {
                        (which == 0 ? p.Q : p.Kd)[o] = v;
                    } else {
                        f16* dst = (f16*)(which == 0 ? p.Q : p.Kd);
                        const float vs = (which == 1 && p.kscale != 0.f) ? v * p.kscale : v;
                        const f16 hv = (f16)vs;
                        dst[o] = hv;
                        if (p.split) dst[(size_t)M * p.d + o] = (f16)(vs - (float)hv);
                    }
                } else if constexpr (EPI == EPI_GELU) {
                    ((OpT*)p.out)[(size_t)m * N + n] = from_f32<OpT>(gelu_erf(v));
                } else {
                    const size_t o = (size_t)m * N + n;
                    p.Z[o] = v + p.R[o];
                }
            }
        }
    }
}

template <class OpT, class WT, int EPI>
static hipError_t gemm_dispatch(const GemmArgs& a, hipStream_t s) {
    // Narrow N gets the 64-wide tile so small layers still spread over the chip.
    if (a.N <= 64 || (a.M <= 4096 && a.N <= 512)) {
        dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
        hipLaunchKernelGGL((gemm_kernel<OpT, WT, EPI, 64, 64>), grid, dim3(256), 0, s, a);
    } else {
        dim3 grid((a.N + 127) / 128, (a.M + 127) / 128);
        hipLaunchKernelGGL((gemm_kernel<OpT, WT, EPI, 128, 128>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

template <class OpT, class WT>
static hipError_t gemm_mode(Epi e, const GemmArgs& a, hipStream_t s) {
    switch (e) {
        case EPI_QKV: return gemm_dispatch<OpT, WT, EPI_QKV>(a, s);
        case EPI_GELU: return gemm_dispatch<OpT, WT, EPI_GELU>(a, s);
        case EPI_RES: return gemm_dispatch<OpT, WT, EPI_RES>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(Mode m, Epi e, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipSuccess;
    // TFL_GEMM_BASIC=1 keeps every product on the kernel above (for A/B
    // comparisons of the two GEMM kernels).
    static const bool basic_only = [] {
        const char* v = std::getenv("TFL_GEMM_BASIC");
        return v && v[0] == '1';
    }();
    if (m != MODE_F32 && !basic_only && gemm_pipe_ok(a)) return launch_gemm_pipe(m, e, a, s);
    switch (m) {
        case MODE_F32: return gemm_mode<float, float>(e, a, s);
        case MODE_F16: return gemm_mode<f16, f16>(e, a, s);
        case MODE_BF16: return gemm_mode<f16, bf16>(e, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tfl
