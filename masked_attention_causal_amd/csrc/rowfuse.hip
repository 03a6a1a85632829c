// Fused row kernel of the layer-wise path: everything of a layer after
// attention, for one tile of 64 token rows, in one launch -- the out-
// projection + bias + residual + LayerNorm, the FFN up-projection + exact-erf
// GELU, the down-projection + bias + residual + LayerNorm, and then the next
// layer's QKV projection of the same rows (head-major Q and K, V^T), or y
// after the last layer.  This is the launch reduction of "KernelForge",
// "What we built" (fused add + mask + LayerNorm; fewer launches per
// forward): with d_model up to 256 a tile's rows fit in LDS, so the residual
// stream, the LayerNorm outputs and the FFN activations never travel
// through HBM between those steps.
//
// The tile arithmetic is that of the PQ path's row tasks (pq_impl.h): the 64
// rows sit in LDS as fp16 B operands; each of four waves streams its slice
// of weight rows from global memory into A-operand registers; LayerNorm is
// two-pass fp32 over the row with partial sums exchanged through LDS.
// Precision as the rest of the 16-bit path: fp32 residual and LayerNorm,
// fp16 operands (bf16 weights widened exactly), fp32 accumulation.
#include "pq_impl.h"

namespace tfl {

template <class WT, int D, int DH>
__global__ __launch_bounds__(PQ_THREADS, 2) void row_kernel(RowArgs p) {
    typedef PqTile<WT, D, DH> TL;
    constexpr int NB = TL::NB, H = D / DH;
    __shared__ __attribute__((aligned(16))) char smem[TL::ROW_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c16 = lane & 15, g = lane >> 4;
    const int t = blockIdx.x, b = blockIdx.y;
    f16* act = (f16*)(smem + TL::OFF_ACT);
    f16* gs = (f16*)(smem + TL::OFF_GV);
    float* red0 = (float*)(smem + TL::OFF_RED);
    float* red1 = red0 + 256;
    const LayerPtrs& w = p.w;
    const int n0 = wave * (D / 4);          // this wave's output features
    const bool last = p.last != 0;

    // ---- attention output rows of the tile -> LDS (fp16); the out-
    // projection's weight fragments are requested first (d <= 128), so the
    // two memory waits overlap
    constexpr bool PRE = NB <= 2;
    constexpr int NBWO = NB == 1 ? 1 : 2;
    f16x8 ao[PRE ? D / 32 : 1][NBWO];
    if constexpr (PRE) frags_load<NBWO, D / 32>(ao, (const WT*)w.w_o, D, n0, 0, c16, g);
    {
        constexpr int CH = PQ_RT * D / 8;
        const f16* O = (const f16*)p.O;
#pragma unroll
        for (int i = 0; i < CH / PQ_THREADS; i++) {
            const int c = tid + i * PQ_THREADS;
            const int r = c / (D / 8), k = (c % (D / 8)) * 8;
            const int pos = t * PQ_RT + r;
            *(uint4*)(act + r * TL::ALD + k) =
                pos < p.L ? *(const uint4*)(O + ((size_t)b * p.L + pos) * D + k) : uint4{0, 0, 0, 0};
        }
    }
    __syncthreads();

    // ---- out-projection + bias + residual
    f32x4 z[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int rb = 0; rb < 4; rb++) z[nb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (PRE) {
        f32x4 (&zz)[NBWO][4] = *reinterpret_cast<f32x4(*)[NBWO][4]>(&z[0]);
        frags_mma<NBWO, D / 32>(zz, ao, act, TL::ALD, c16, g);
    } else {
#pragma unroll
        for (int half = 0; half < NB / 2; half++) {
            f32x4 (&zz)[2][4] = *reinterpret_cast<f32x4(*)[2][4]>(&z[2 * half]);
            mm_rows<2, D>(zz, (const WT*)w.w_o, D, n0 + 32 * half, 0, act, TL::ALD, c16, g);
        }
    }
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        const int n = n0 + 16 * nb + 4 * g;
        float bv[4];
        load4_f32((const WT*)w.b_o + n, bv);
#pragma unroll
        for (int rb = 0; rb < 4; rb++) {
            const int pos = t * PQ_RT + 16 * rb + c16;
            float xr[4] = {0.f, 0.f, 0.f, 0.f};
            if (pos < p.L) load4_f32(p.X + ((size_t)b * p.L + pos) * D + n, xr);
#pragma unroll
            for (int e = 0; e < 4; e++) z[nb][rb][e] += bv[e] + xr[e];
        }
    }
    row_layernorm<D, NB>(z, (const WT*)w.ln1_g, (const WT*)w.ln1_b, p.eps, red0, red1, n0, wave, c16, g);
    // X1: fp16 operand copy in LDS (every wave is past its out-projection
    // reads: row_sum synchronised) and the fp32 value in this tile's rows of
    // the residual buffer, read back by the same lanes after the FFN
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int rb = 0; rb < 4; rb++) {
            const int r = 16 * rb + c16, pos = t * PQ_RT + r;
            const float v[4] = {z[nb][rb][0], z[nb][rb][1], z[nb][rb][2], z[nb][rb][3]};
            store4(act + r * TL::ALD + n0 + 16 * nb + 4 * g, v);
            if (pos < p.L) store4(p.X + ((size_t)b * p.L + pos) * D + n0 + 16 * nb + 4 * g, v);
        }
    __syncthreads();

    // ---- FFN in chunks of PQ_FC features: G chunk to LDS, then accumulate W2 G^T
    f32x4 y2[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int rb = 0; rb < 4; rb++) y2[nb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nch = p.F / PQ_FC;
    constexpr int NBW2 = NB == 1 ? 1 : 2, NH = NB == 1 ? 1 : NB / 2;
    f16x8 a2[PRE ? NH : 1][PQ_FC / 32][NBW2];
#pragma unroll 1
    for (int c = 0; c < nch; c++) {
        f16* gb = gs + (c & 1) * PQ_RT * TL::GLD;
        const int f0 = c * PQ_FC + wave * (PQ_FC / 4);
        if constexpr (PRE) {
#pragma unroll
            for (int hh = 0; hh < NH; hh++)
                frags_load<NBW2, PQ_FC / 32>(a2[hh], (const WT*)w.w_2, p.F, n0 + 32 * hh, c * PQ_FC, c16, g);
        }
        f32x4 ga[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; nb++)
#pragma unroll
            for (int rb = 0; rb < 4; rb++) ga[nb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        mm_rows<2, D>(ga, (const WT*)w.w_1, D, f0, 0, act, TL::ALD, c16, g);
#pragma unroll
        for (int nb = 0; nb < 2; nb++) {
            float bv[4];
            load4_f32((const WT*)w.b_1 + f0 + 16 * nb + 4 * g, bv);
#pragma unroll
            for (int rb = 0; rb < 4; rb++)
#pragma unroll
                for (int e = 0; e < 4; e++) ga[nb][rb][e] += bv[e];
        }
        static_assert(sizeof(ga) == 32 * sizeof(float), "ga is 32 packed floats");
        gelu_inplace<32, true>((float*)&ga[0][0]);
#pragma unroll
        for (int nb = 0; nb < 2; nb++)
#pragma unroll
            for (int rb = 0; rb < 4; rb++) {
                f16x4 hv;
#pragma unroll
                for (int e = 0; e < 4; e++) hv[e] = (f16)ga[nb][rb][e];
                *(f16x4*)(gb + (16 * rb + c16) * TL::GLD + wave * (PQ_FC / 4) + 16 * nb + 4 * g) = hv;
            }
        __syncthreads();
        if constexpr (NB == 1) {
            frags_mma<1, PQ_FC / 32>(y2, a2[0], gb, TL::GLD, c16, g);
        } else if constexpr (PRE) {
            f32x4 (&yy)[2][4] = *reinterpret_cast<f32x4(*)[2][4]>(&y2[0]);
            frags_mma<2, PQ_FC / 32>(yy, a2[0], gb, TL::GLD, c16, g);
        } else {
#pragma unroll
            for (int hh = 0; hh < NB / 2; hh++) {
                f32x4 (&yy)[2][4] = *reinterpret_cast<f32x4(*)[2][4]>(&y2[2 * hh]);
                mm_rows<2, PQ_FC>(yy, (const WT*)w.w_2, p.F, n0 + 32 * hh, c * PQ_FC, gb, TL::GLD, c16, g);
            }
        }
    }
    // ---- + bias + residual (X1), LayerNorm
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        float bv[4];
        load4_f32((const WT*)w.b_2 + n0 + 16 * nb + 4 * g, bv);
#pragma unroll
        for (int rb = 0; rb < 4; rb++) {
            const int pos = t * PQ_RT + 16 * rb + c16;
            float xr[4] = {0.f, 0.f, 0.f, 0.f};
            if (pos < p.L) load4_f32(p.X + ((size_t)b * p.L + pos) * D + n0 + 16 * nb + 4 * g, xr);
#pragma unroll
            for (int e = 0; e < 4; e++) y2[nb][rb][e] += bv[e] + xr[e];
        }
    }
    row_layernorm<D, NB>(y2, (const WT*)w.ln2_g, (const WT*)w.ln2_b, p.eps, red0, red1, n0, wave, c16, g);

#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        const int n = n0 + 16 * nb + 4 * g;
#pragma unroll
        for (int rb = 0; rb < 4; rb++) {
            const int r = 16 * rb + c16, pos = t * PQ_RT + r;
            const float v[4] = {y2[nb][rb][0], y2[nb][rb][1], y2[nb][rb][2], y2[nb][rb][3]};
            if (pos < p.L) {
                const size_t row = (size_t)b * p.L + pos;
                if (last)
                    store4((WT*)p.y + row * D + n, v);
                else
                    store4(p.X + row * D + n, v);
            }
            if (!last) store4(act + r * TL::ALD + n, v);
        }
    }
    if (last) return;
    __syncthreads();

    // ---- next layer's QKV projection of the tile rows
    f16* vts = gs;   // the FFN chunk buffers are free again: V^T staging [D][64]
    const WT* Wq = (const WT*)p.wn.w_qkv;
    const WT* bq = (const WT*)p.wn.b_qkv;
    const float ks = p.kscale != 0.f ? p.kscale : 1.0f;
#pragma unroll 1
    for (int ps = 0; ps < TL::QPASS; ps++) {
        const int q0 = wave * (3 * D / 4) + ps * 16 * TL::QNB;
        f32x4 acc[TL::QNB][4];
#pragma unroll
        for (int nb = 0; nb < TL::QNB; nb++)
#pragma unroll
            for (int rb = 0; rb < 4; rb++) acc[nb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        mm_rows<TL::QNB, D>(acc, Wq, D, q0, 0, act, TL::ALD, c16, g);
#pragma unroll
        for (int nb = 0; nb < TL::QNB; nb++) {
            const int n = q0 + 16 * nb + 4 * g;         // first of four consecutive features
            float bv[4];
            load4_f32(bq + n, bv);
            const int which = n / D, nn = n - which * D;
            const int h = nn / DH, dd = nn - h * DH;
#pragma unroll
            for (int rb = 0; rb < 4; rb++) {
                const int r = 16 * rb + c16, pos = t * PQ_RT + r;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; e++) v[e] = acc[nb][rb][e] + bv[e];
                if (which == 2) {
#pragma unroll
                    for (int e = 0; e < 4; e++) vts[(nn + e) * TL::VLDT + r] = (f16)v[e];
                } else if (pos < p.L) {
                    const float sc = which == 1 ? ks : 1.0f;
                    f16* dst = (which == 0 ? p.Q : p.K) + (((size_t)b * H + h) * p.L + pos) * DH + dd;
                    *(f16x4*)dst = f16x4{(f16)(v[0] * sc), (f16)(v[1] * sc), (f16)(v[2] * sc), (f16)(v[3] * sc)};
                }
            }
        }
    }
    __syncthreads();
    // V^T block [D][64] of tile t: whole 16-byte runs of keys (columns past L
    // hold finite values of the padded rows; the attention masks them)
    constexpr int CH = D * (PQ_RT / 8);
#pragma unroll
    for (int i = 0; i < (CH + PQ_THREADS - 1) / PQ_THREADS; i++) {
        const int c = tid + i * PQ_THREADS;
        if (CH % PQ_THREADS != 0 && c >= CH) break;
        const int nn = c / (PQ_RT / 8), c8 = (c % (PQ_RT / 8)) * 8;
        const int h = nn / DH, dd = nn - h * DH;
        *(uint4*)(p.Vt + (((size_t)b * H + h) * DH + dd) * p.Lp + t * PQ_RT + c8) =
            *(const uint4*)(vts + nn * TL::VLDT + c8);
    }
}

bool row_supported(Mode m, int d, int dh, int f) {
    if (m == MODE_F32) return false;
    if (d != 64 && d != 128 && d != 256) return false;
    if (dh != 16 && dh != 32 && dh != 64) return false;
    return f % PQ_FC == 0 && f >= PQ_FC;
}

template <class WT, int D>
static hipError_t row_d(int dh, const RowArgs& a, hipStream_t s) {
    dim3 grid((a.L + PQ_RT - 1) / PQ_RT, a.B);
    switch (dh) {
        case 16: hipLaunchKernelGGL((row_kernel<WT, D, 16>), grid, dim3(PQ_THREADS), 0, s, a); break;
        case 32: hipLaunchKernelGGL((row_kernel<WT, D, 32>), grid, dim3(PQ_THREADS), 0, s, a); break;
        case 64: hipLaunchKernelGGL((row_kernel<WT, D, 64>), grid, dim3(PQ_THREADS), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class WT>
static hipError_t row_mode(int d, int dh, const RowArgs& a, hipStream_t s) {
    switch (d) {
        case 64: return row_d<WT, 64>(dh, a, s);
        case 128: return row_d<WT, 128>(dh, a, s);
        case 256: return row_d<WT, 256>(dh, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_row(Mode m, int d, int dh, const RowArgs& a, hipStream_t s) {
    if (a.B <= 0 || a.L <= 0) return hipSuccess;
    if (m == MODE_F16) return row_mode<f16>(d, dh, a, s);
    if (m == MODE_BF16) return row_mode<bf16>(d, dh, a, s);
    return hipErrorInvalidValue;
}

}  // namespace tfl
