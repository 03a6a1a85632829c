// Projection GEMMs of the layer-wise path on MFMA: C = A W^T + b, with an
// epilogue per use.
//   EPI_QKV  : fused QKV projection; Q and K leave head-major [B, H, L, dh]
//              as fp16 planes (hi, and the rounding remainder when split);
//              V leaves transposed per head, [B, H, dh, Lp], the layout the
//              attention kernels read as the A operand of P V.  (The QKV GEMM
//              with the head-major transpose fused into it is the custom
//              kernel of "Hyper-optimized megakernel-hybrid transformer
//              inference", "Problem decomposition", hybrid family.)
//   EPI_GELU : FFN up-projection with exact-erf GELU in the epilogue
//              ("KernelForge", "How the LLM is used": exact erf).
//   EPI_RES  : out-projection / FFN down-projection plus bias plus the fp32
//              residual; LayerNorm follows in its own kernel.
//
// Operands are fp16 in every mode: activations as produced by the previous
// kernel, weights either as given (fp16 I/O) or converted once per forward
// (bf16 I/O: the exact fp16 value; fp32 I/O: an fp16 hi plane and a lo plane
// holding the rounding remainder times 2^11).  With fp32 I/O every product is
// split in three MFMAs, hi*hi + (hi*lo + lo*hi) * 2^-11, so each product
// carries ~22 significant bits instead of fp16's 11: the TF32 idea of
// "Implement a GPU Kernel for a Transformer Layer", "Accomplishments" (tiled
// FP32 on tensor cores), with enough passes to stay accurate for inputs up to
// 1e3 in scale.
//
// Each workgroup (WGM x WGN waves over tokens x features) owns TT tokens x
// TF features.  Operand tiles of 64 K-columns stream from global memory
// straight into a ring of STAGES LDS buffers with 16-byte global_load_lds,
// STAGES - 1 tiles ahead of the MFMAs, so one barrier serves 64 K-columns.
// Rows of every tile are 128 bytes (64 halves) with their eight 16-byte
// chunks XOR-swizzled by the row index (chunk c of row r sits in slot
// c ^ (r & 7)); the swizzle is applied by choosing which global chunk each
// lane loads, since an LDS-DMA lane's destination is fixed.  Eight rows
// read the same chunk through eight different slots, so fragment reads do
// not collide on LDS banks.  When K is an odd multiple of 32 the last stage
// holds 32 columns: its lanes past K reload a valid chunk of their row, and
// only its first 32 columns are multiplied.
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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tfl {

namespace {

constexpr float LO_SCALE = 2048.0f;  // lo planes hold the remainder times 2^11

// Slot of chunk c in row r of a tile whose rows hold CPR 16-byte chunks:
// the chunk index XOR-ed with bits of the row (r mod 8 for 128-byte rows,
// bits 1-2 of r for 64-byte rows), the patterns that make 16-row fragment
// reads conflict-free on this LDS.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    static_assert(CPR == 4 || CPR == 8, "rows of 32 or 64 halves");
    return CPR == 8 ? (r & 7) : ((r >> 1) & 3);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace

template <class PT, int EPI, int TT, int TF, int PK, int STAGES, int WGM, int WGN, bool SPLIT>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_pipe_kernel(GemmArgs p) {
    constexpr int PROW = PK * 2;                    // bytes per tile row
    constexpr int CPR = PK / 8;                     // 16-byte chunks per tile row
    constexpr int NTHR = 64 * WGM * WGN;            // waves arranged WGM (tokens) x WGN (features)
    constexpr int WTT = TT / WGM, WTF = TF / WGN;   // wave tile
    constexpr int TB = WTT / 16, FB = WTF / 16;     // MFMA blocks per wave
    constexpr int NPL = SPLIT ? 2 : 1;              // fp16 planes per operand (hi, lo)
    constexpr int PB = (TT + TF) * PROW;            // bytes per plane of a stage
    constexpr int SB = NPL * PB;                    // bytes per stage
    constexpr int NA = TT * CPR / NTHR, NW = TF * CPR / NTHR;  // 16-byte DMA chunks per thread per plane
    constexpr int NDMA = NPL * (NA + NW);
    static_assert(NA >= 1 && NW >= 1 && STAGES >= 2 && TB >= 1 && FB >= 1, "tile too small");
    static_assert(NA * NTHR == TT * CPR && NW * NTHR == TF * CPR, "tile rows must split evenly over the threads");
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
    const f16* __restrict__ W = (const f16*)p.W;
    const size_t loA = (size_t)M * K * 2, loW = (size_t)N * K * 2;  // byte offsets of the lo planes

    // DMA source addresses of this thread's chunks (row clamped into the
    // matrix; rows past the edge are computed on copies and never stored).
    // hiA / hiW: chunks whose source column lies in the upper half of a
    // stage; in a 32-column last stage they reload the chunk 64 bytes lower.
    const char* srcA[NA];
    const char* srcW[NW];
    unsigned hiA = 0, hiW = 0;
#pragma unroll
    for (int i = 0; i < NA; i++) {
        const int q = i * NTHR + tid, r = q / CPR, c = (q % CPR) ^ swz<CPR>(r);
        const int gm = min(m0 + r, M - 1);
        srcA[i] = (const char*)(A + (size_t)gm * K) + 16 * c;
        hiA |= (unsigned)(PK == 64 && c >= 4) << i;
    }
#pragma unroll
    for (int i = 0; i < NW; i++) {
        const int q = i * NTHR + tid, r = q / CPR, c = (q % CPR) ^ swz<CPR>(r);
        const int gn = min(n0 + r, N - 1);
        srcW[i] = (const char*)(W + (size_t)gn * K) + 16 * c;
        hiW |= (unsigned)(PK == 64 && c >= 4) << i;
    }
    auto issue = [&](int kt, int buf, bool half) {
        char* base = lds + buf * SB;
        const size_t ko = (size_t)kt * PROW;
#pragma unroll
        for (int pl = 0; pl < NPL; pl++) {
#pragma unroll
            for (int i = 0; i < NA; i++) {
                const size_t o = ko + (pl ? loA : 0) - ((half && ((hiA >> i) & 1)) ? 64 : 0);
                dma16(srcA[i] + o, base + pl * PB + (i * NTHR + wave * 64) * 16);
            }
#pragma unroll
            for (int i = 0; i < NW; i++) {
                const size_t o = ko + (pl ? loW : 0) - ((half && ((hiW >> i) & 1)) ? 64 : 0);
                dma16(srcW[i] + o, base + pl * PB + TT * PROW + (i * NTHR + wave * 64) * 16);
            }
        }
    };

    f32x4 acc[FB][TB], acx[SPLIT ? FB : 1][SPLIT ? TB : 1];
#pragma unroll
    for (int i = 0; i < FB; i++)
#pragma unroll
        for (int j = 0; j < TB; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < FB; i++)
#pragma unroll
            for (int j = 0; j < TB; j++) acx[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One stage: wait for its DMA, publish it, issue the stage STAGES - 1
    // ahead, multiply NKK 32-column slices.  Full stages run in the loop; a
    // 32-column last stage (K % 64 == 32) runs once after it, so the loop body
    // has no branch around its products.
    const int nk = (K + PK - 1) / PK;
    const bool halfK = K % PK != 0;
    const int nfull = K / PK;
    auto stage = [&](int kt, auto nkk_c) {
        constexpr int NKK = decltype(nkk_c)::value;
        // stage kt has landed once at most (STAGES - 2) later stages are pending
        if (kt + STAGES - 2 < nk)
            wait_vm<(STAGES - 2) * NDMA>();
        else
            wait_vm<0>();
        __syncthreads();  // stage kt visible; every wave is done with stage kt - 1
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES, halfK && kt + STAGES == nk);
        const char* at = lds + (kt % STAGES) * SB;
        const char* wt = at + TT * PROW;
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) {
            const int ch = kk * 4 + g;
            f16x8 wf[FB], af[TB], wl[SPLIT ? FB : 1], al[SPLIT ? TB : 1];
#pragma unroll
            for (int i = 0; i < FB; i++) {
                const int r = wn * WTF + i * 16 + c16;
                const int off = r * PROW + 16 * (ch ^ swz<CPR>(r));
                wf[i] = *(const f16x8*)(wt + off);
                if constexpr (SPLIT) wl[i] = *(const f16x8*)(wt + PB + off);
            }
#pragma unroll
            for (int j = 0; j < TB; j++) {
                const int r = wm * WTT + j * 16 + c16;
                const int off = r * PROW + 16 * (ch ^ swz<CPR>(r));
                af[j] = *(const f16x8*)(at + off);
                if constexpr (SPLIT) al[j] = *(const f16x8*)(at + PB + off);
            }
#pragma unroll
            for (int i = 0; i < FB; i++)
#pragma unroll
                for (int j = 0; j < TB; j++) {
                    acc[i][j] = mfma_16x16x32(wf[i], af[j], acc[i][j]);
                    if constexpr (SPLIT) {
                        acx[i][j] = mfma_16x16x32(wl[i], af[j], acx[i][j]);
                        acx[i][j] = mfma_16x16x32(wf[i], al[j], acx[i][j]);
                    }
                }
        }
    };
#pragma unroll
    for (int s = 0; s < STAGES - 1; s++)
        if (s < nk) issue(s, s, halfK && s == nk - 1);
    for (int kt = 0; kt < nfull; kt++) stage(kt, std::integral_constant<int, PK / 32>{});
    if (halfK) stage(nfull, std::integral_constant<int, 1>{});

    // ---------------------------------------------------------------- epilogue
    // lane (c16, g) of block (i, j): features n..n+3, token m.  Index
    // arithmetic is split into a token part (per j) and a feature part (per
    // i), each formed once.
    const PT* __restrict__ bias = (const PT*)p.bias;
    int mrow[TB];
#pragma unroll
    for (int j = 0; j < TB; j++) mrow[j] = m0 + wm * WTT + j * 16 + c16;
    // QKV: Q/K element (b, h, pos, t) sits at ((b*H + h)*L + pos)*dh + t =
    // (b*L*d + pos*dh) + (h*L*dh + t) (H*dh = d); V^T element (b, h, t, pos)
    // at (b*d + h*dh + t)*Lp + pos = (b*d*Lp + pos) + (h*dh + t)*Lp.
    size_t qk_m[EPI == EPI_QKV ? TB : 1], vt_m[EPI == EPI_QKV ? TB : 1];
    if constexpr (EPI == EPI_QKV) {
#pragma unroll
        for (int j = 0; j < TB; j++) {
            const int b = mrow[j] / p.L, pos = mrow[j] - b * p.L;
            qk_m[j] = (size_t)b * p.L * p.d + (size_t)pos * p.dh;
            vt_m[j] = (size_t)b * p.d * p.Lp + pos;
        }
    }
#pragma unroll
    for (int i = 0; i < FB; i++) {
        const int n = n0 + wn * WTF + i * 16 + 4 * g;
        if (n >= N) continue;
        float bv[4];
#pragma unroll
        for (int e = 0; e < 4; e++) bv[e] = to_f32(bias[n + e]);
        int which = 0, nn = n;
        size_t qk_n = 0;
        float ks = 1.f;
        if constexpr (EPI == EPI_QKV) {
            which = n >= p.d ? (n >= 2 * p.d ? 2 : 1) : 0;
            nn = n - which * p.d;
            const int h = nn / p.dh, t = nn - h * p.dh;
            qk_n = (size_t)h * p.L * p.dh + t;
            if (which == 1 && p.kscale != 0.f) ks = p.kscale;
        }
#pragma unroll
        for (int j = 0; j < TB; j++) {
            const int m = mrow[j];
            if (m >= M) continue;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                v[e] = acc[i][j][e] + bv[e];
                if constexpr (SPLIT) v[e] += acx[i][j][e] * (1.0f / LO_SCALE);
            }
            if constexpr (EPI == EPI_QKV) {
                if (which < 2) {
                    f16* dst = (f16*)(which == 0 ? p.Q : p.Kd) + qk_m[j] + qk_n;
                    f16x4 hv, lv;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const F16Split sp = split_f16(v[e] * ks, 1.0f);
                        hv[e] = sp.hi;
                        lv[e] = sp.lo;
                    }
                    *(f16x4*)dst = hv;
                    if (p.split) *(f16x4*)(dst + (size_t)M * p.d) = lv;
                } else {
                    f16* vt = (f16*)p.Vt + vt_m[j] + (size_t)nn * p.Lp;
#pragma unroll
                    for (int e = 0; e < 4; e++) vt[(size_t)e * p.Lp] = (f16)v[e];
                }
            } else if constexpr (EPI == EPI_GELU) {
                f16x4 o, ol;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float gv = gelu_full(v[e]);
                    if constexpr (SPLIT) {
                        const F16Split sp = split_f16(gv, LO_SCALE);
                        o[e] = sp.hi;
                        ol[e] = sp.lo;
                    } else {
                        o[e] = (f16)gv;
                    }
                }
                f16* dst = (f16*)p.out + (size_t)m * N + n;
                *(f16x4*)dst = o;
                if constexpr (SPLIT) *(f16x4*)(dst + (size_t)M * N) = ol;
            } else {
                const size_t o = (size_t)m * N + n;
                const float4 r = *(const float4*)(p.R + o);
                *(float4*)(p.Z + o) = float4{v[0] + r.x, v[1] + r.y, v[2] + r.z, v[3] + r.w};
            }
        }
    }
}

// Compute units of the current device (queried once per device).
static int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <class PT, int EPI, bool SPLIT>
static hipError_t pipe_dispatch(const GemmArgs& a, hipStream_t s) {
    // 128 x 128 tiles, 8 waves (2 token x 4 feature), two stages: two
    // workgroups fit one CU with single-plane operands, which measured
    // fastest of the tile / wave / stage shapes tried on the FFN and
    // projection shapes.
    const int nt = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    // 128 x 192 tiles (two workgroups per CU as well, 80 KB of LDS each) where
    // they leave fewer idle workgroup slots: the work is ~rounds x tile width,
    // rounds = tiles / (2 x CUs) rounded up.  The QKV product at d = 1024
    // (4096 x 3072) takes 512 such tiles, one round on 256 CUs, instead of
    // 768 narrower ones in 1.5 rounds: 43 -> 39 us per launch.
    if constexpr (!SPLIT) {
        const long slots = 2L * cu_count();
        const long nt192 = (long)((a.M + 127) / 128) * ((a.N + 191) / 192);
        if (nt >= 512 && ((nt192 + slots - 1) / slots) * 192 < ((nt + slots - 1) / slots) * 128) {
            hipLaunchKernelGGL((gemm_pipe_kernel<PT, EPI, 128, 192, 64, 2, 2, 4, SPLIT>), dim3((unsigned)nt192), dim3(512), 0,
                               s, a);
            return hipGetLastError();
        }
    }
    // Products with fewer than two such tiles per CU (the out-projection and
    // FFN-down products of 4096 tokens at d = 1024 have 256) take 64-token
    // tiles with 4 waves (2 x 2, 32 tokens x 64 features each), so a CU holds
    // several workgroups: FFN-down measured 13% faster than with one 128 x 128
    // workgroup per CU; 128 x 64 tiles gained 4%.
    if (nt < 512) {
        const int nt64 = ((a.M + 63) / 64) * ((a.N + 127) / 128);
        hipLaunchKernelGGL((gemm_pipe_kernel<PT, EPI, 64, 128, 64, 2, 2, 2, SPLIT>), dim3(nt64), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemm_pipe_kernel<PT, EPI, 128, 128, 64, 2, 2, 4, SPLIT>), dim3(nt), dim3(512), 0, s, a);
    return hipGetLastError();
}

template <class PT, bool SPLIT>
static hipError_t gemm_epi(Epi e, const GemmArgs& a, hipStream_t s) {
    switch (e) {
        case EPI_QKV: return pipe_dispatch<PT, EPI_QKV, SPLIT>(a, s);
        case EPI_GELU: return pipe_dispatch<PT, EPI_GELU, SPLIT>(a, s);
        case EPI_RES: return pipe_dispatch<PT, EPI_RES, SPLIT>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(Mode m, Epi e, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipSuccess;
    if (a.K % 32 != 0 || a.N % 4 != 0) return hipErrorInvalidValue;
    switch (m) {
        case MODE_F32: return gemm_epi<float, true>(e, a, s);
        case MODE_F16: return gemm_epi<f16, false>(e, a, s);
        case MODE_BF16: return gemm_epi<bf16, false>(e, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tfl
