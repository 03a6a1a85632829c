// Sequence-resident path: one launch runs the whole layer stack.
//
// "Hyper-optimized megakernel-hybrid transformer inference", "Problem
// decomposition": when sequences are short, a workgroup owns whole
// sequences and keeps them on chip for every layer.  Here a workgroup of 8
// waves (two per SIMD) owns two sequences of up to 64 tokens; wave w owns
// the 16 tokens 16*(w%4) .. of sequence w/4 as one column block (the code
// is written for TPW column blocks per wave).  Each wave keeps
// the fp32 residual rows of its tokens in registers for the whole stack,
// in the MFMA result layout of the transposed products below, so
// LayerNorm, the residual adds and the fp16 operand copies never leave the
// wave.
//
// Every projection is computed transposed, OUT^T = W ACT^T: the weights are
// the A operand, staged through LDS once per workgroup and read as one
// 16-byte fragment that feeds one MFMA per token block; the
// activations are the B operand, straight from registers.  A 16x16 MFMA
// result block leaves lane (g, c) with rows 4g..4g+3 of column c, so two
// adjacent blocks give the lane rows {4g..4g+3, 16+4g..16+4g+3} of a
// 32-row chunk.  Weight tiles are gathered into LDS with their rows
// permuted within every group of 32 (LDS row 16h + 4g + e holds weight row
// 8g + 4h + e), so those result rows are the natural features 8g..8g+7:
// exactly the K slice a lane holds in a 16x16x32 B operand, and the next
// product's fragment is the natural 16 bytes at column 8g.  Activations
// thus pass from one product to the next register to register.
//
// Attention (keys j <= i and j < len_b, "KernelForge", "What we built") is
// computed per head: K and V^T of both sequences go to LDS (their rows
// stored in the same sigma32 order as the weight tiles, so a fragment read
// is a plain row read), each wave forms
// S^T = K Q^T for its queries over at most 64 keys, a plain (not online)
// softmax over the row, and O^T = V^T P^T, which is again a B operand of
// the out-projection.  Key chunks past the wave's last query or past len_b
// are skipped.
//
// Weight tiles (fp16) and the per-layer bias / LayerNorm vectors stream
// from global memory straight into LDS with 16-byte global_load_lds, one
// tile ahead of the MFMAs; bf16 weight tiles go through registers to be
// widened to fp16.
//
// LDS images (weight tiles, K, V^T) are unpadded rows of 16-byte chunks
// with the chunks of row r XOR-permuted by a few bits of r, so a 16-row x
// 16-byte fragment read touches every bank equally.  Rows are a power of two
// chunks long, so the lane -> (row, chunk) split of a tile load is a shift
// and a mask, and the source offsets of one lane's loads differ by
// constants.
//
// Precision matches the tiled path: fp32 residual and LayerNorm, fp16
// operands with fp32 accumulation, first-layer scores from a hi/lo fp16
// split of Q and K, exact-erf GELU.
#include "common.h"
#include "kernels.h"

namespace tfl {

namespace {

constexpr int SEQ_THREADS = 512;  // 8 waves, two per SIMD
constexpr int SEQ_SLOT = 64;      // tokens per sequence slot
constexpr int SEQ_SEQS = 2;       // sequences per workgroup
constexpr int SEQ_TOK = SEQ_SLOT * SEQ_SEQS;
constexpr int TPW = 1;            // 16-token column blocks per wave
constexpr int SEQ_WPS = SEQ_SLOT / (16 * TPW);  // waves per sequence slot
constexpr int SEQ_MAX_F = 4096;   // largest FFN width of the SEQ path
constexpr int FCH = 64;        // FFN width per chunk

constexpr int SEQ_LDS_MAX = 160 * 1024;

// Largest staged weight tile (halves): Q/K/V rows of one head DH x D, W_o
// columns of one head D x DH, W_1 rows of one chunk FCH x D, W_2 columns of
// one chunk D x FCH.
constexpr int seq_tbuf(int D, int DH) { return (DH > FCH ? DH : FCH) * D; }
// Static LDS of the kernel (bytes): two weight tiles, K hi/lo, V^T.
constexpr int seq_static_lds(int D, int DH) {
    return 2 * seq_tbuf(D, DH) * 2 + 2 * SEQ_TOK * DH * 2 + DH * SEQ_TOK * 2;
}
// Dynamic LDS (bytes): per-layer vectors, double-buffered by layer parity.
inline size_t seq_param_lds(int d, int f, size_t elem) { return 2 * (size_t)(((9 * d + f) + 7) & ~7) * elem; }

struct TileDesc {
    int kind;  // 0 Q, 1 K, 2 V rows of a head, 3 W_o columns of a head, 4 W_1 chunk, 5 W_2 chunk
    int layer, h, kc, fc;
};

__device__ __forceinline__ f16x8 pack8(f32x4 a, f32x4 b) {
    return f16x8{(f16)a[0], (f16)a[1], (f16)a[2], (f16)a[3], (f16)b[0], (f16)b[1], (f16)b[2], (f16)b[3]};
}

// Row permutation applied within every 32-row group of a staged tile: LDS
// row 16h + 4g + e holds source row 8g + 4h + e.
__device__ __forceinline__ int sigma32(int r) { return 8 * ((r >> 2) & 3) + 4 * (r >> 4) + (r & 3); }

// Inverse of sigma32: the LDS row that holds source row k of a 32-row group.
__device__ __forceinline__ int sigma32_inv(int k) { return (k & 3) | ((k >> 3) << 2) | (((k >> 2) & 1) << 4); }

// Natural feature held by element e of result block `blk` in lane group g
// (after the sigma32 row gather): 4 consecutive features per block.
__device__ __forceinline__ int feat4(int blk, int g) { return (blk >> 1) * 32 + 8 * g + 4 * (blk & 1); }

// Chunk k of row r of an image with CPR chunks per row sits in slot
// k ^ swz(r).  Measured on this LDS: folding r into the low chunk bits makes
// 16-row fragment reads conflict-free for rows of 128 bytes and more; for
// 64-byte rows (two per 128-byte line) bits 1-2 of r are used instead.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    static_assert(CPR == 4 || CPR == 8 || CPR == 16 || CPR == 32, "rows of 4 to 32 chunks");
    if constexpr (CPR >= 16) return r & 15;
    else if constexpr (CPR == 8) return r & 7;
    else return (r >> 1) & 3;
}
// Byte offset of chunk k of row r.
template <int CPR>
__device__ __forceinline__ int img_off(int r, int k) { return r * (CPR * 16) + ((k ^ swz<CPR>(r)) << 4); }

// A operand fragment: chunk k of row 16 blk + c16 (sw = swz(c16), which is
// swz of that row for every blk).
template <int CPR>
__device__ __forceinline__ f16x8 afrag16(const f16* buf, int blk, int c16, int k, int sw) {
    return *(const f16x8*)((const char*)buf + (blk * 16 + c16) * (CPR * 16) + ((k ^ sw) << 4));
}

// Four consecutive stored values as fp32.
template <class T>
__device__ __forceinline__ f32x4 load4(const T* q) {
    const uint2 r = *(const uint2*)q;
    if constexpr (std::is_same<T, f16>::value) {
        const f16x4 h = *(const f16x4*)&r;
        return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    } else {
        return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
                     __uint_as_float(r.y & 0xFFFF0000u)};
    }
}



// Scheduling order for a fully unrolled product of NM MFMAs fed by NDS LDS
// reads, MPR MFMAs per read: AHEAD reads are issued first, then MPR MFMAs
// and one read alternate, so every fragment is in flight well before use.
template <int NDS, int NM, int MPR, int AHEAD>
__device__ __forceinline__ void pipeline_order() {
#pragma unroll
    for (int i = 0; i < AHEAD; i++) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NM / MPR; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
        if (AHEAD + i < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}
constexpr int SEQ_AHEAD = 8;

}  // namespace

template <class WT, int D, int DH>
__global__ __launch_bounds__(SEQ_THREADS) void seq_kernel(SeqArgs p) {
    constexpr bool DIRECT = std::is_same<WT, f16>::value;  // fp16 weights: global -> LDS directly
    constexpr int H = D / DH;
    constexpr int NDB = D / 16;   // residual blocks per token column
    constexpr int NKC = D / 32;   // 32-wide K chunks over d_model
    constexpr int NQB = DH / 16;  // blocks per head
    constexpr int NHC = DH / 32;  // 32-wide K chunks over the head dim
    constexpr int NCB = NQB > FCH / 16 ? NQB : FCH / 16;  // carried blocks (Q of a head, or a GELU chunk)
    constexpr int KCPR = DH / 8;              // chunks per K row (token)
    constexpr int VCPR = SEQ_TOK / 8;         // chunks per V^T row (feature)
    // Staged weight tiles, rows sigma32-gathered and chunk-swizzled:
    //   kinds 0-2: Q/K/V rows of one head, DH x D;  3: W_o columns of one head, D x DH;
    //   4: W_1 rows of one chunk, FCH x D;          5: W_2 columns of one chunk, D x FCH.
    constexpr int TBUF = seq_tbuf(D, DH);
    constexpr int MAXCH = (TBUF / 8 + SEQ_THREADS - 1) / SEQ_THREADS;  // 16-byte chunks per thread
    static_assert(D % 32 == 0 && DH % 32 == 0 && D % DH == 0, "unsupported SEQ shape");

    __shared__ __attribute__((aligned(16))) f16 Wb0[TBUF];
    __shared__ __attribute__((aligned(16))) f16 Wb1[TBUF];
    __shared__ __attribute__((aligned(16))) f16 Kh[SEQ_TOK * DH];
    __shared__ __attribute__((aligned(16))) f16 Kl[SEQ_TOK * DH];
    __shared__ __attribute__((aligned(16))) f16 Vt[DH * SEQ_TOK];
    static_assert(seq_static_lds(D, DH) == (2 * TBUF + 3 * SEQ_TOK * DH) * 2, "LDS accounting");
    // Small per-layer vectors, raw I/O-dtype bits, double-buffered by layer
    // parity: b_qkv | b_o | ln1_g | ln1_b | b_1 | b_2 | ln2_g | ln2_b.
    constexpr int P_BQKV = 0, P_BO = 3 * D, P_G1 = 4 * D, P_BE1 = 5 * D, P_B1 = 6 * D;
    extern __shared__ __attribute__((aligned(16))) uint16_t seq_dyn_lds[];
    WT* const Pm = (WT*)seq_dyn_lds;  // 2 * PLENP elements

    // Lane coordinates.  With fp16 weights the compiler may keep per-lane
    // addresses derived from them in registers across the tile loop (there is
    // room below the register ceiling); with bf16 weights the staging
    // registers of the tile loads leave none, so there the coordinates are
    // re-derived from an opaque copy of the thread id at every step and the
    // addresses recomputed where they are used.
    int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int c16 = lane & 15, g = lane >> 4;
    const int wave0 = threadIdx.x >> 6;
    const int sq = wave0 / SEQ_WPS;              // sequence slot of this wave
    const int q0 = (wave0 % SEQ_WPS) * 16 * TPW; // first position of this wave's tokens
    const int b = blockIdx.x * SEQ_SEQS + sq;
    auto refresh_lane = [&]() {
        int t = threadIdx.x;
        if constexpr (!std::is_same<WT, f16>::value) asm volatile("" : "+v"(t));
        tid = t;
        lane = t & 63;
        wave = t >> 6;
        c16 = lane & 15;
        g = lane >> 4;
    };
    const int L = p.L;
    int len = b < p.B ? p.lens[b] : 1;
    len = len < 1 ? 1 : (len > L ? L : len);
    const int F = p.F;
    const int NF = F / FCH;
    const int PLEN = 9 * D + F;
    const int PLENP = (PLEN + 7) & ~7;          // 16-byte aligned parity buffers
    const int P_B2 = 6 * D + F, P_G2 = 7 * D + F, P_BE2 = 8 * D + F;

    // Per-layer vectors: 16-byte chunk c of the concatenation (every vector
    // is 16-byte aligned and a multiple of 8 long), fetched straight into LDS.
    auto param_src = [&](const LayerPtrs& w, int j) -> const WT* {
        if (j < 3 * D) return (const WT*)w.b_qkv + j;
        if ((j -= 3 * D) < D) return (const WT*)w.b_o + j;
        if ((j -= D) < D) return (const WT*)w.ln1_g + j;
        if ((j -= D) < D) return (const WT*)w.ln1_b + j;
        if ((j -= D) < F) return (const WT*)w.b_1 + j;
        if ((j -= F) < D) return (const WT*)w.b_2 + j;
        if ((j -= D) < D) return (const WT*)w.ln2_g + j;
        return (const WT*)w.ln2_b + (j - D);
    };
    auto param_fetch = [&](int layer) {
        const LayerPtrs& w = p.lw[layer];
        WT* dst = Pm + (layer & 1) * PLENP;
        for (int i = 0; i * SEQ_THREADS * 8 < PLEN; i++) {
            const int c = i * SEQ_THREADS + tid;
            if (c * 8 < PLEN) dma16(param_src(w, c * 8), (f16*)(dst + (i * SEQ_THREADS + wave * 64) * 8));
        }
    };

    // The tile stream: per layer, for each head h: Q_h, K_h, V_h, W_o(h);
    // then for each FFN chunk: W_1(chunk), W_2(chunk).  next_of gives the
    // tile after d (kind -1 past the last one).
    auto next_of = [&](const TileDesc& d) {
        TileDesc n = d;
        if (d.kind <= 2 || d.kind == 4) {
            n.kind = d.kind + 1;
        } else if (d.kind == 3) {
            if (d.h + 1 < H) {
                n.kind = 0;
                n.h = d.h + 1;
            } else {
                n.kind = 4;
                n.fc = 0;
            }
        } else if (d.fc + 1 < NF) {
            n.kind = 4;
            n.fc = d.fc + 1;
        } else if (d.layer + 1 < p.n_layers) {
            n = TileDesc{0, d.layer + 1, 0, 0, 0};
        } else {
            n.kind = -1;
        }
        return n;
    };
    // Geometry of a tile, passed to fn as compile-time rows and columns of the
    // staged image plus the global base and row stride (elements), so the
    // per-lane chunk -> (row, column) split below divides by constants.
    auto with_geom = [&](const TileDesc& d, auto&& fn) {
        const LayerPtrs& w = p.lw[d.layer];
        if (d.kind <= 2)
            fn(std::integral_constant<int, DH>{}, std::integral_constant<int, D>{},
               (const WT*)w.w_qkv + (size_t)(d.kind * D + d.h * DH) * D, D);
        else if (d.kind == 3)
            fn(std::integral_constant<int, D>{}, std::integral_constant<int, DH>{}, (const WT*)w.w_o + d.h * DH, D);
        else if (d.kind == 4)
            fn(std::integral_constant<int, FCH>{}, std::integral_constant<int, D>{},
               (const WT*)w.w_1 + (size_t)d.fc * FCH * D, D);
        else
            fn(std::integral_constant<int, D>{}, std::integral_constant<int, FCH>{}, (const WT*)w.w_2 + d.fc * FCH, F);
    };

    // Chunk c of a tile's LDS image (row c / CPR, slot c % CPR) is loaded by
    // thread c mod 512, since an LDS-DMA lane's destination is fixed; the
    // slot holds source chunk slot ^ swz(row) of gathered source row
    // gather(row).  512 / CPR rows lie between one thread's loads, a multiple
    // of 16 (rows of up to 32 chunks), so slot, swz and the gather's low part
    // are the same for all of them: the source offsets differ by whole rows.
    uint4 stg[DIRECT ? 1 : MAXCH];
    auto tile_fetch = [&](const TileDesc& t, f16* buf) {
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        with_geom(t, [&](auto R, auto C, const WT* base, int rstride) {
            constexpr int ROWS = decltype(R)::value, CPR = decltype(C)::value / 8, N = ROWS * CPR;
            constexpr int S = SEQ_THREADS / CPR;  // rows between one thread's loads
            static_assert(S % 16 == 0, "rows between loads");
            const int tt = tid & (SEQ_THREADS - 1);
            const int r0 = tt / CPR, slot = tt % CPR;
            const int lane_off = (((r0 & ~31) + sigma32(r0 & 31)) * rstride + ((slot ^ swz<CPR>(r0)) << 3)) * (int)sizeof(WT);
#pragma unroll
            for (int i = 0; i < MAXCH; i++) {
                if (i * SEQ_THREADS < N && tt + i * SEQ_THREADS < N) {
                    // gathered row of r0 + S i: + S i for S >= 32; for S = 16 the
                    // odd half-group adds 4 (sigma32 maps +16 to +4)
                    const int drow = S >= 32 ? S * i : 32 * (i >> 1) + 4 * (i & 1);
                    const WT* sb = base + (size_t)drow * rstride;
                    if constexpr (DIRECT) {
                        dma16s(sb, (unsigned)lane_off, buf + (i * SEQ_THREADS + wv * 64) * 8);
                    } else {
                        stg[i] = *(const uint4*)((const char*)sb + lane_off);
                    }
                }
            }
        });
    };
    auto tile_commit = [&](const TileDesc& t, f16* buf) {
        if constexpr (!DIRECT) {
            with_geom(t, [&](auto R, auto C, const WT*, int) {
                constexpr int N = decltype(R)::value * (decltype(C)::value / 8);
                const int tt = tid & (SEQ_THREADS - 1);
#pragma unroll
                for (int i = 0; i < MAXCH; i++) {
                    const int c = tt + i * SEQ_THREADS;
                    if (i * SEQ_THREADS < N && c < N) *(f16x8*)&buf[c * 8] = load8_as_f16((const WT*)&stg[i]);
                }
            });
        }
        // direct loads of the tile and of the vectors land before the barrier
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    // ---- registers: residual X^T (fp32) and its fp16 B-operand copy, per token block
    f32x4 R[NDB][TPW];
    f16x8 XB[NKC][TPW];
#pragma unroll
    for (int tb = 0; tb < TPW; tb++) {
        const int pos = q0 + tb * 16 + c16;
        const bool live = b < p.B && pos < L;
        const WT* x = (const WT*)p.x + ((size_t)(live ? b : 0) * L + (live ? pos : 0)) * D;
#pragma unroll
        for (int db = 0; db < NDB; db++) {
            const f32x4 v = load4(x + feat4(db, g));
            R[db][tb] = live ? v : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kk = 0; kk < NKC; kk++) XB[kk][tb] = pack8(R[2 * kk][tb], R[2 * kk + 1][tb]);
    }
    // Q^T of the current head (from its tile until attention) or the GELU
    // output of the current FFN chunk (from W_1 to W_2).
    f32x4 carry[NCB][TPW];

    auto layer_norm = [&](const WT* gam, const WT* bet) {  // LDS pointers
#pragma unroll
        for (int tb = 0; tb < TPW; tb++) {
            float s = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; db++) s += (R[db][tb][0] + R[db][tb][1]) + (R[db][tb][2] + R[db][tb][3]);
            s += __shfl_xor(s, 16, WAVE);
            s += __shfl_xor(s, 32, WAVE);
            const float mean = s / (float)D;
            float q = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; db++) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    R[db][tb][e] -= mean;
                    q += R[db][tb][e] * R[db][tb][e];
                }
            }
            q += __shfl_xor(q, 16, WAVE);
            q += __shfl_xor(q, 32, WAVE);
            const float rstd = 1.0f / sqrtf(q / (float)D + p.eps);
#pragma unroll
            for (int db = 0; db < NDB; db++) {
                const f32x4 ga = load4(gam + feat4(db, g)), be = load4(bet + feat4(db, g));
#pragma unroll
                for (int e = 0; e < 4; e++) R[db][tb][e] = R[db][tb][e] * rstd * ga[e] + be[e];
            }
#pragma unroll
            for (int kk = 0; kk < NKC; kk++) XB[kk][tb] = pack8(R[2 * kk][tb], R[2 * kk + 1][tb]);
        }
    };

    auto step = [&](const TileDesc& d, const f16* W) {
        const WT* P = Pm + (d.layer & 1) * PLENP;
        const bool split = d.layer == 0;

        if (d.kind <= 2) {
            // ---- Q^T, K^T or V^T of head h: [DH x tokens] = W rows . X^T
            constexpr int CPR = D / 8;
            const int sw = swz<CPR>(c16);
            f32x4 acc[NQB][TPW];
            const WT* bq = P + P_BQKV + d.kind * D + d.h * DH;
#pragma unroll
            for (int ob = 0; ob < NQB; ob++) {
                const f32x4 bv = load4(bq + feat4(ob, g));
#pragma unroll
                for (int tb = 0; tb < TPW; tb++) acc[ob][tb] = bv;
            }
            // Fragments of the next 32-wide K slice are read before this
            // slice's products, in their own registers, and the issue order
            // below keeps a few more reads in flight (left to the scheduler
            // alone, this step's reads were each waited on before their
            // product).
            f16x8 fa[2][NQB];
#pragma unroll
            for (int ob = 0; ob < NQB; ob++) fa[0][ob] = afrag16<CPR>(W, ob, c16, g, sw);
#pragma unroll
            for (int kk = 0; kk < NKC; kk++) {
                if (kk + 1 < NKC) {
#pragma unroll
                    for (int ob = 0; ob < NQB; ob++) fa[(kk + 1) & 1][ob] = afrag16<CPR>(W, ob, c16, (kk + 1) * 4 + g, sw);
                }
#pragma unroll
                for (int ob = 0; ob < NQB; ob++)
#pragma unroll
                    for (int tb = 0; tb < TPW; tb++) acc[ob][tb] = mfma_16x16x32(fa[kk & 1][ob], XB[kk][tb], acc[ob][tb]);
            }
            pipeline_order<NQB + NKC * NQB, NKC * NQB * TPW, TPW, NQB + 4>();
            if (d.kind == 0) {
#pragma unroll
                for (int ob = 0; ob < NQB; ob++)
#pragma unroll
                    for (int tb = 0; tb < TPW; tb++) carry[ob][tb] = acc[ob][tb];
            } else if (d.kind == 1) {
#pragma unroll
                for (int tb = 0; tb < TPW; tb++) {
                    const int key = sq * SEQ_SLOT + q0 + tb * 16 + c16;
                    const int tok = (key & ~31) + sigma32_inv(key & 31);  // LDS row of this key
#pragma unroll
                    for (int kb = 0; kb < NQB; kb++) {
                        f16x4 hv, lv;
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            hv[e] = (f16)acc[kb][tb][e];
                            lv[e] = (f16)(acc[kb][tb][e] - (float)hv[e]);
                        }
                        // features feat4(kb, g) .. + 3: chunk (kb >> 1) * 4 + g, half kb & 1
                        const int o = img_off<KCPR>(tok, (kb >> 1) * 4 + g) + 8 * (kb & 1);
                        *(f16x4*)((char*)Kh + o) = hv;
                        if (split) *(f16x4*)((char*)Kl + o) = lv;
                    }
                }
            } else {
#pragma unroll
                for (int tb = 0; tb < TPW; tb++) {
                    const int tok = sq * SEQ_SLOT + q0 + tb * 16 + c16;
#pragma unroll
                    for (int vb = 0; vb < NQB; vb++)
#pragma unroll
                        // feature feat4(vb, g) + e sits in LDS row sigma32_inv of it: vb * 16 + 4g + e
                        for (int e = 0; e < 4; e++)
                            *(f16*)((char*)Vt + img_off<VCPR>(vb * 16 + 4 * g + e, tok >> 3) + 2 * (tok & 7)) =
                                (f16)acc[vb][tb][e];
                }
            }
        } else if (d.kind == 3) {
            // ---- attention of head h for this wave's queries
            const int kbase = sq * SEQ_SLOT;
            const int kmax = min(q0 + 16 * TPW, len);
            const int swk = swz<KCPR>(c16);
            const int nch = (kmax + 31) >> 5;  // 32-key chunks that matter (1 or 2)
            if constexpr (MASK_ALL) {
                if (lane == 0 && b < p.B) audit_add(p.audit, AUD_SEQ_WAVE, nch);
            }
            f16x8 qh[NHC][TPW], ql[NHC][TPW];
#pragma unroll
            for (int tb = 0; tb < TPW; tb++)
#pragma unroll
                for (int kk = 0; kk < NHC; kk++) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float a = carry[2 * kk][tb][e], c = carry[2 * kk + 1][tb][e];
                        const f16 ah = (f16)a, ch = (f16)c;
                        qh[kk][tb][e] = ah;
                        qh[kk][tb][4 + e] = ch;
                        ql[kk][tb][e] = (f16)(a - (float)ah);
                        ql[kk][tb][4 + e] = (f16)(c - (float)ch);
                    }
                }
            // At most two 32-key chunks: the scores of both are formed first,
            // then one row max, the weights and the P V products -- a plain
            // softmax over the row, with one cross-lane reduction and no
            // rescaling in the dependent chain.
            f32x4 o[NQB][TPW], s[2][2][TPW];
            float lrun[TPW];
#pragma unroll
            for (int cc = 0; cc < 2; cc++) {
                if (cc < nch) {
#pragma unroll
                    for (int hb = 0; hb < 2; hb++) {
#pragma unroll
                        for (int tb = 0; tb < TPW; tb++) s[cc][hb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                        // LDS row kbase + cc * 32 + hb * 16 + c16 holds key sigma32(hb * 16 + c16)
                        const int kblk = (kbase + cc * 32) / 16 + hb;
#pragma unroll
                        for (int kk = 0; kk < NHC; kk++) {
                            const f16x8 a = afrag16<KCPR>(Kh, kblk, c16, kk * 4 + g, swk);
#pragma unroll
                            for (int tb = 0; tb < TPW; tb++) {
                                s[cc][hb][tb] = mfma_16x16x32(a, qh[kk][tb], s[cc][hb][tb]);
                                if (split) {
                                    s[cc][hb][tb] = mfma_16x16x32(afrag16<KCPR>(Kl, kblk, c16, kk * 4 + g, swk), qh[kk][tb], s[cc][hb][tb]);
                                    s[cc][hb][tb] = mfma_16x16x32(a, ql[kk][tb], s[cc][hb][tb]);
                                }
                            }
                        }
                    }
                    // keys of this chunk can be masked only if it reaches past the
                    // wave's first query or past the sequence end (wave-uniform)
                    const bool need_mask =
                        MASK_ALL ||
                        __builtin_amdgcn_readfirstlane((cc * 32 + 31 > q0) || (cc * 32 + 31 >= len) ? 1 : 0) != 0;
#pragma unroll
                    for (int tb = 0; tb < TPW; tb++) {
                        const int pos = q0 + tb * 16 + c16;
#pragma unroll
                        for (int hb = 0; hb < 2; hb++)
#pragma unroll
                            for (int e = 0; e < 4; e++) {
                                const int key = cc * 32 + 8 * g + 4 * hb + e;
                                float v = s[cc][hb][tb][e] * p.scale_log2;
                                if (need_mask && (key > pos || key >= len)) v = -INFINITY;
                                s[cc][hb][tb][e] = v;
                            }
                    }
                }
            }
#pragma unroll
            for (int tb = 0; tb < TPW; tb++) {
                float mx = -INFINITY;
#pragma unroll
                for (int cc = 0; cc < 2; cc++)
                    if (cc < nch) {
#pragma unroll
                        for (int hb = 0; hb < 2; hb++)
#pragma unroll
                            for (int e = 0; e < 4; e++) mx = fmaxf(mx, s[cc][hb][tb][e]);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
                mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));  // finite: key 0 is in chunk 0
                float ls = 0.f;
#pragma unroll
                for (int cc = 0; cc < 2; cc++)
                    if (cc < nch) {
#pragma unroll
                        for (int hb = 0; hb < 2; hb++)
#pragma unroll
                            for (int e = 0; e < 4; e++) {
                                const float pv = __builtin_amdgcn_exp2f(s[cc][hb][tb][e] - mx);
                                s[cc][hb][tb][e] = pv;
                                ls += pv;
                            }
                    }
                lrun[tb] = ls;
#pragma unroll
                for (int db = 0; db < NQB; db++) o[db][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int cc = 0; cc < 2; cc++)
                if (cc < nch) {
#pragma unroll
                    for (int db = 0; db < NQB; db++) {
                        // LDS row db * 16 + c16 holds feature (db >> 1) * 32 + sigma32((db & 1) * 16 + c16)
                        const f16x8 va = afrag16<VCPR>(Vt, db, c16, (kbase + cc * 32) / 8 + g, c16);
#pragma unroll
                        for (int tb = 0; tb < TPW; tb++)
                            o[db][tb] = mfma_16x16x32(va, pack8(s[cc][0][tb], s[cc][1][tb]), o[db][tb]);
                    }
                }
            f16x8 OB[NHC][TPW];
#pragma unroll
            for (int tb = 0; tb < TPW; tb++) {
                float l = lrun[tb];
                l += __shfl_xor(l, 16, WAVE);
                l += __shfl_xor(l, 32, WAVE);
                const float inv = 1.0f / l;
#pragma unroll
                for (int kk = 0; kk < NHC; kk++) OB[kk][tb] = pack8(o[2 * kk][tb] * inv, o[2 * kk + 1][tb] * inv);
            }

            // ---- out-projection of head h accumulated into the residual
            if (d.h == 0) {
#pragma unroll
                for (int db = 0; db < NDB; db++) {
                    const f32x4 bv = load4(P + P_BO + feat4(db, g));
#pragma unroll
                    for (int tb = 0; tb < TPW; tb++) R[db][tb] += bv;
                }
            }
            const int swo = swz<DH / 8>(c16);
#pragma unroll
            for (int db = 0; db < NDB; db++)
#pragma unroll
                for (int kk = 0; kk < NHC; kk++) {
                    const f16x8 a = afrag16<DH / 8>(W, db, c16, kk * 4 + g, swo);
#pragma unroll
                    for (int tb = 0; tb < TPW; tb++) R[db][tb] = mfma_16x16x32(a, OB[kk][tb], R[db][tb]);
                }
            pipeline_order<NDB * NHC, NDB * NHC * TPW, TPW, SEQ_AHEAD>();
        } else if (d.kind == 4) {
            // ---- FFN up-projection chunk + GELU, carried to the next tile
            const int sw1 = swz<D / 8>(c16);
#pragma unroll
            for (int ob = 0; ob < FCH / 16; ob++) {
                const f32x4 bv = load4(P + P_B1 + d.fc * FCH + feat4(ob, g));
#pragma unroll
                for (int tb = 0; tb < TPW; tb++) carry[ob][tb] = bv;
            }
#pragma unroll
            for (int kk = 0; kk < NKC; kk++)
#pragma unroll
                for (int ob = 0; ob < FCH / 16; ob++) {
                    const f16x8 a = afrag16<D / 8>(W, ob, c16, kk * 4 + g, sw1);
#pragma unroll
                    for (int tb = 0; tb < TPW; tb++) carry[ob][tb] = mfma_16x16x32(a, XB[kk][tb], carry[ob][tb]);
                }
            pipeline_order<FCH / 16 + NKC * FCH / 16, NKC * FCH / 16 * TPW, TPW, SEQ_AHEAD>();
            static_assert(sizeof(carry) == FCH / 16 * TPW * 4 * sizeof(float), "carry is packed floats");
            gelu_inplace<FCH / 16 * TPW * 4, true>((float*)&carry[0][0]);
        } else {
            // ---- FFN down-projection chunk accumulated into the residual
            if (d.fc == 0) {
#pragma unroll
                for (int db = 0; db < NDB; db++) {
                    const f32x4 bv = load4(P + P_B2 + feat4(db, g));
#pragma unroll
                    for (int tb = 0; tb < TPW; tb++) R[db][tb] += bv;
                }
            }
            const int sw2 = swz<FCH / 8>(c16);
            f16x8 gb[FCH / 32][TPW];
#pragma unroll
            for (int kk = 0; kk < FCH / 32; kk++)
#pragma unroll
                for (int tb = 0; tb < TPW; tb++) gb[kk][tb] = pack8(carry[2 * kk][tb], carry[2 * kk + 1][tb]);
#pragma unroll
            for (int db = 0; db < NDB; db++)
#pragma unroll
                for (int kk = 0; kk < FCH / 32; kk++) {
                    const f16x8 a = afrag16<FCH / 8>(W, db, c16, kk * 4 + g, sw2);
#pragma unroll
                    for (int tb = 0; tb < TPW; tb++) R[db][tb] = mfma_16x16x32(a, gb[kk][tb], R[db][tb]);
                }
            pipeline_order<NDB * FCH / 32, NDB * FCH / 32 * TPW, TPW, SEQ_AHEAD>();
        }
        // LayerNorm after the last head (LN1) and after the last FFN chunk (LN2);
        // one call site keeps a single inlined copy.
        if ((d.kind == 3 && d.h == H - 1) || (d.kind == 5 && d.fc == NF - 1))
            layer_norm(P + (d.kind == 3 ? P_G1 : P_G2), P + (d.kind == 3 ? P_BE1 : P_BE2));
    };

    // One step: the next tile streams into the other buffer while this one
    // is multiplied; the first step of a layer also fetches the next layer's
    // vectors into the other parity buffer.  Step kinds are compile-time at
    // every call site below, so each kind is inlined once with no dispatch
    // and the residual stays in the same registers across steps.
    auto run = [&](const TileDesc d, const f16* W, f16* Wn, bool first_of_layer) {
        refresh_lane();
        const TileDesc n = next_of(d);
        if (n.kind >= 0) tile_fetch(n, Wn);
        if (first_of_layer && d.layer + 1 < p.n_layers) param_fetch(d.layer + 1);
        step(d, W);
        if (n.kind >= 0) tile_commit(n, Wn);
        __syncthreads();
    };
    param_fetch(0);
    tile_fetch(TileDesc{0, 0, 0, 0, 0}, Wb0);
    tile_commit(TileDesc{0, 0, 0, 0, 0}, Wb0);
    __syncthreads();
    // Every group (4 tiles per head, 2 per FFN chunk) has an even length, so
    // a group's first tile is always in Wb0.
    for (int l = 0; l < p.n_layers; l++) {
        for (int h = 0; h < H; h++) {
            run(TileDesc{0, l, h, 0, 0}, Wb0, Wb1, h == 0);
            run(TileDesc{1, l, h, 0, 0}, Wb1, Wb0, false);
            run(TileDesc{2, l, h, 0, 0}, Wb0, Wb1, false);
            run(TileDesc{3, l, h, 0, 0}, Wb1, Wb0, false);
        }
        for (int fc = 0; fc < NF; fc++) {
            run(TileDesc{4, l, 0, 0, fc}, Wb0, Wb1, false);
            run(TileDesc{5, l, 0, 0, fc}, Wb1, Wb0, false);
        }
    }

    // ---- output rows
#pragma unroll
    for (int tb = 0; tb < TPW; tb++) {
        const int pos = q0 + tb * 16 + c16;
        if (b < p.B && pos < L) {
            WT* y = (WT*)p.y + ((size_t)b * L + pos) * D;
#pragma unroll
            for (int db = 0; db < NDB; db++) {
                uint2 o;
                WT* ov = (WT*)&o;
#pragma unroll
                for (int e = 0; e < 4; e++) ov[e] = from_f32<WT>(R[db][tb][e]);
                *(uint2*)(y + feat4(db, g)) = o;
            }
        }
    }
}

bool seq_supported(Mode m, int d, int dh, int f, int L, int n_layers) {
    if (m == MODE_F32 || L > SEQ_SLOT || f % FCH != 0 || f > SEQ_MAX_F || n_layers > SEQ_MAX_LAYERS) return false;
    const bool shape = (d == 256 && dh == 64) || (d == 256 && dh == 32) || (d == 128 && dh == 64) ||
                       (d == 128 && dh == 32) || (d == 64 && dh == 64) || (d == 64 && dh == 32);
    // the per-layer vectors (dynamic LDS) must fit beside the static tiles
    return shape && seq_static_lds(d, dh) + seq_param_lds(d, f, 2) <= (size_t)SEQ_LDS_MAX;
}

template <class WT>
static hipError_t seq_mode(int d, int dh, const SeqArgs& a, hipStream_t s) {
    dim3 grid((a.B + SEQ_SEQS - 1) / SEQ_SEQS);
    const size_t pbytes = seq_param_lds(d, a.F, sizeof(WT));
#define TFL_SEQ_CASE(DD, HH)                                                                    \
    if (d == DD && dh == HH) {                                                                  \
        hipLaunchKernelGGL((seq_kernel<WT, DD, HH>), grid, dim3(SEQ_THREADS), pbytes, s, a);   \
        return hipGetLastError();                                                               \
    }
    TFL_SEQ_CASE(256, 64) TFL_SEQ_CASE(256, 32) TFL_SEQ_CASE(128, 64) TFL_SEQ_CASE(128, 32)
    TFL_SEQ_CASE(64, 64) TFL_SEQ_CASE(64, 32)
#undef TFL_SEQ_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_seq(Mode m, int d, int dh, const SeqArgs& a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    if (m == MODE_F16) return seq_mode<f16>(d, dh, a, s);
    if (m == MODE_BF16) return seq_mode<bf16>(d, dh, a, s);
    return hipErrorInvalidValue;
}

}  // namespace tfl
