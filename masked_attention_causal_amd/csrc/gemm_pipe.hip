// Pipelined projection GEMM for the 16-bit operand modes: activations fp16,
// weights fp16 or bf16 (widened to fp16 as fragments leave LDS).  Same
// epilogues as gemm.hip (QKV head-major, GELU, bias + residual).
//
// Each workgroup (WGM x WGN waves over tokens x features) owns TT tokens x
// TF features.  Operand tiles of 64 K-columns stream from global memory
// straight into a ring of STAGES LDS buffers with 16-byte global_load_lds,
// STAGES - 1 tiles ahead of the MFMAs, so the loads of several tiles are in
// flight while one is multiplied, and one barrier serves 64 K-columns.
// Rows of every tile are 128 bytes (64 halves) with their eight 16-byte
// chunks XOR-swizzled by the row index (chunk c of row r sits in slot
// c ^ (r & 7)); the swizzle is applied by choosing which global chunk each
// lane loads, since an LDS-DMA lane's destination is fixed.  Eight rows
// read the same chunk through eight different slots, so fragment reads do
// not collide on LDS banks.
//
// The product is formed transposed, OUT^T = W A^T: weight rows are the MFMA
// A operand and token rows the B operand, so a result lane holds four
// consecutive features of one token and the epilogue stores 8 or 16
// contiguous bytes.  The blockIdx -> tile map hands each of the eight XCDs
// a contiguous run of tiles, token-block-major when there are at least as
// many token rows as weight rows (each XCD then reads its own eighth of the
// activations and the whole weight matrix) and feature-block-major
// otherwise; on the d = 1024 stack, token-major cut the FFN-down product's
// fabric traffic from ~4x its algorithmic bytes and the stack from 1,014 to
// 924 us per forward.
#include "common.h"
#include "kernels.h"

namespace tfl {

namespace {

constexpr int PK = 64;        // K-columns per stage
constexpr int PROW = PK * 2;  // bytes per tile row

// Eight stored weights -> eight fp16 operands.
__device__ __forceinline__ f16x8 widen8(const uint4 r, f16) { return *(const f16x8*)&r; }
__device__ __forceinline__ f16x8 widen8(const uint4 r, bf16) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        o[2 * i] = (f16)__uint_as_float(w[i] << 16);
        o[2 * i + 1] = (f16)__uint_as_float(w[i] & 0xFFFF0000u);
    }
    return o;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace

template <class WT, int EPI, int TT, int TF, int STAGES, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_pipe_kernel(GemmArgs p) {
    constexpr int NTHR = 64 * WGM * WGN;            // waves arranged WGM (tokens) x WGN (features)
    constexpr int WTT = TT / WGM, WTF = TF / WGN;   // wave tile
    constexpr int TB = WTT / 16, FB = WTF / 16;     // MFMA blocks per wave
    constexpr int SB = (TT + TF) * PROW;            // bytes per stage
    constexpr int NA = TT * 8 / NTHR, NW = TF * 8 / NTHR;  // 16-byte DMA chunks per thread per stage
    constexpr int NDMA = NA + NW;
    static_assert(NA >= 1 && NW >= 1 && STAGES >= 2 && TB >= 1 && FB >= 1, "tile too small");
    static_assert(NA * NTHR == TT * 8 && NW * NTHR == TF * 8, "tile rows must split evenly over the threads");
    __shared__ __attribute__((aligned(16))) char lds[STAGES * SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int wm = wave / WGN, wn = wave % WGN;
    const int M = p.M, N = p.N, K = p.K;

    // ---- XCD-aware tile order: each XCD takes a contiguous run of tiles,
    // ordered so that the larger operand is split between the XCDs and the
    // smaller one is what every XCD reads whole (token-block-major when the
    // token rows outnumber the weight rows, feature-block-major otherwise)
    const int nTT = (M + TT - 1) / TT, nTF = (N + TF - 1) / TF, ntiles = nTT * nTF;
    int tile = blockIdx.x;
    if (ntiles % 8 == 0) tile = (tile % 8) * (ntiles / 8) + tile / 8;
    int fblk, tblk;
    if (M >= N) {
        tblk = tile / nTF;
        fblk = tile - tblk * nTF;
    } else {
        fblk = tile / nTT;
        tblk = tile - fblk * nTT;
    }
    const int m0 = tblk * TT, n0 = fblk * TF;

    const f16* __restrict__ A = (const f16*)p.A;
    const WT* __restrict__ W = (const WT*)p.W;

    // DMA source addresses of this thread's chunks (row clamped into the
    // matrix; rows past the edge are computed on copies and never stored)
    const char* srcA[NA];
    const char* srcW[NW];
#pragma unroll
    for (int i = 0; i < NA; i++) {
        const int q = i * NTHR + tid, r = q >> 3, slot = q & 7;
        const int gm = min(m0 + r, M - 1);
        srcA[i] = (const char*)(A + (size_t)gm * K) + 16 * (slot ^ (r & 7));
    }
#pragma unroll
    for (int i = 0; i < NW; i++) {
        const int q = i * NTHR + tid, r = q >> 3, slot = q & 7;
        const int gn = min(n0 + r, N - 1);
        srcW[i] = (const char*)(W + (size_t)gn * K) + 16 * (slot ^ (r & 7));
    }
    auto issue = [&](int kt, int buf) {
        char* base = lds + buf * SB;
        const size_t ko = (size_t)kt * PK * 2;
#pragma unroll
        for (int i = 0; i < NA; i++) dma16(srcA[i] + ko, base + (i * NTHR + wave * 64) * 16);
#pragma unroll
        for (int i = 0; i < NW; i++) dma16(srcW[i] + ko, base + TT * PROW + (i * NTHR + wave * 64) * 16);
    };

    f32x4 acc[FB][TB];
#pragma unroll
    for (int i = 0; i < FB; i++)
#pragma unroll
        for (int j = 0; j < TB; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / PK;
#pragma unroll
    for (int s = 0; s < STAGES - 1; s++)
        if (s < nk) issue(s, s);

    for (int kt = 0; kt < nk; kt++) {
        // stage kt has landed once at most (STAGES - 2) later stages are pending
        if (kt + STAGES - 2 < nk)
            wait_vm<(STAGES - 2) * NDMA>();
        else
            wait_vm<0>();
        __syncthreads();  // stage kt visible; every wave is done with stage kt - 1
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
        const char* at = lds + (kt % STAGES) * SB;
        const char* wt = at + TT * PROW;
#pragma unroll
        for (int kk = 0; kk < PK / 32; kk++) {
            const int ch = kk * 4 + g;
            f16x8 wf[FB], af[TB];
#pragma unroll
            for (int i = 0; i < FB; i++) {
                const int r = wn * WTF + i * 16 + c16;
                wf[i] = widen8(*(const uint4*)(wt + r * PROW + 16 * (ch ^ (r & 7))), WT{});
            }
#pragma unroll
            for (int j = 0; j < TB; j++) {
                const int r = wm * WTT + j * 16 + c16;
                af[j] = *(const f16x8*)(at + r * PROW + 16 * (ch ^ (r & 7)));
            }
#pragma unroll
            for (int i = 0; i < FB; i++)
#pragma unroll
                for (int j = 0; j < TB; j++) acc[i][j] = mfma_16x16x32(wf[i], af[j], acc[i][j]);
        }
    }

    // ---------------------------------------------------------------- epilogue
    // lane (c16, g) of block (i, j): features n..n+3, token m
    const WT* __restrict__ bias = (const WT*)p.bias;
#pragma unroll
    for (int i = 0; i < FB; i++) {
        const int n = n0 + wn * WTF + i * 16 + 4 * g;
        if (n >= N) continue;
        float bv[4];
#pragma unroll
        for (int e = 0; e < 4; e++) bv[e] = to_f32(bias[n + e]);
#pragma unroll
        for (int j = 0; j < TB; j++) {
            const int m = m0 + wm * WTT + j * 16 + c16;
            if (m >= M) continue;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; e++) v[e] = acc[i][j][e] + bv[e];
            if constexpr (EPI == EPI_QKV) {
                const int which = n / p.d, nn = n - which * p.d;
                const int h = nn / p.dh, t = nn - h * p.dh;
                const int b = m / p.L, pos = m - b * p.L;
                const size_t bh = (size_t)b * p.H + h;
                if (which < 2) {
                    f16* dst = (f16*)(which == 0 ? p.Q : p.Kd) + (bh * p.L + pos) * p.dh + t;
                    const float ks = (which == 1 && p.kscale != 0.f) ? p.kscale : 1.f;
                    f16x4 hv, lv;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float vs = v[e] * ks;
                        hv[e] = (f16)vs;
                        lv[e] = (f16)(vs - (float)hv[e]);
                    }
                    *(f16x4*)dst = hv;
                    if (p.split) *(f16x4*)(dst + (size_t)M * p.d) = lv;
                } else {
                    f16* vt = (f16*)p.Vt + (bh * p.dh + t) * p.Lp + pos;
#pragma unroll
                    for (int e = 0; e < 4; e++) vt[(size_t)e * p.Lp] = (f16)v[e];
                }
            } else if constexpr (EPI == EPI_GELU) {
                f16x4 o;
#pragma unroll
                for (int e = 0; e < 4; e++) o[e] = (f16)gelu_erf(v[e]);
                *(f16x4*)((f16*)p.out + (size_t)m * N + n) = o;
            } else {
                const size_t o = (size_t)m * N + n;
                const float4 r = *(const float4*)(p.R + o);
                *(float4*)(p.Z + o) = float4{v[0] + r.x, v[1] + r.y, v[2] + r.z, v[3] + r.w};
            }
        }
    }
}

// Whether the pipelined kernel takes this product (16-bit operand modes).
bool gemm_pipe_ok(const GemmArgs& a) {
    return a.K % PK == 0 && a.N % 4 == 0 && a.M >= 128 && a.N >= 128 && (long)a.M * a.N >= (1L << 20);
}

template <class WT, int EPI>
static hipError_t pipe_dispatch(const GemmArgs& a, hipStream_t s) {
    // 128 x 128 tiles, 8 waves (2 token x 4 feature), two 32 KB stages: two
    // workgroups fit one CU, which measured fastest of the tile / wave /
    // stage shapes tried on the FFN and projection shapes.
    const int nt = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    // Products with fewer than two such tiles per CU (the out-projection and
    // FFN-down products of 4096 tokens at d = 1024 have 256) take 64-token
    // tiles with 4 waves (2 x 2, 32 tokens x 64 features each), so a CU holds
    // several workgroups: FFN-down measured 13% faster than with one 128 x 128
    // workgroup per CU; 128 x 64 tiles gained 4%.
    if (nt < 512) {
        const int nt64 = ((a.M + 63) / 64) * ((a.N + 127) / 128);
        hipLaunchKernelGGL((gemm_pipe_kernel<WT, EPI, 64, 128, 2, 2, 2>), dim3(nt64), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemm_pipe_kernel<WT, EPI, 128, 128, 2, 2, 4>), dim3(nt), dim3(512), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm_pipe(Mode m, Epi e, const GemmArgs& a, hipStream_t s) {
    if (m == MODE_F32) return hipErrorInvalidValue;
    const bool b = m == MODE_BF16;
    switch (e) {
        case EPI_QKV: return b ? pipe_dispatch<bf16, EPI_QKV>(a, s) : pipe_dispatch<f16, EPI_QKV>(a, s);
        case EPI_GELU: return b ? pipe_dispatch<bf16, EPI_GELU>(a, s) : pipe_dispatch<f16, EPI_GELU>(a, s);
        case EPI_RES: return b ? pipe_dispatch<bf16, EPI_RES>(a, s) : pipe_dispatch<f16, EPI_RES>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tfl
