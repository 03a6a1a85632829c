// Streaming masked attention on MFMA.  Never materialises the L x L score
// matrix ("KernelForge", "Results": the 100k-token shape would need an
// 18.6 TB score matrix; "Implement a GPU Kernel for a Transformer Layer",
// "Accomplishments": a bounded-memory kernel at 100,000 tokens).
//
// Key j is allowed for query i of sequence b iff j <= i and j < len_b: the
// causal and key-padding masks together ("KernelForge", "What we built").
//
// One workgroup = 4 waves = 64 queries of one (sequence, head); every wave
// owns 16 queries.  Key tiles of 64 keys are staged in LDS (double
// buffered) and the workgroup walks them from key 0 up to
// min(query-tile end, len_b): tiles past that are skipped, so a causal
// workload does M(M+1)/2 of the M^2 tile visits ("KernelForge",
// "Challenges": the tiled floor is (M+1)/2M).  The mask predicate is
// evaluated only on tiles that straddle the diagonal or the padding
// boundary; on every other tile it would be a no-op ("KernelForge",
// "Challenges": splitting the loop is bit-identical).
//
// Scores are computed transposed, S^T = K Q^T, so that the MFMA result
// layout (one query per lane column, four keys per lane) is directly the B
// operand of O^T = V^T P^T.  The softmax statistics then live in the lane
// that owns the query, and the running max needs only a reduction across
// the four 16-lane groups of the wave.
//
// Precision: Q and K arrive as fp16 planes written by the QKV epilogue: the
// rounded value and, where the scores need it, the rounding remainder, so
// scores are formed as hi*hi + hi*lo + lo*hi (three MFMAs) at about fp32
// accuracy.  The remainder planes are used for the first layer in the 16-bit
// I/O modes (raw inputs up to 1e3 give scores near 1e5) and for every layer
// with fp32 I/O.  P is rounded to fp16 for the P V product; the row sums use
// the same weights.  With fp32 I/O the output also leaves as two fp16
// planes (hi, and the remainder times 2^11) for the split out-projection.
//
// Two kernels stream K and V^T with LDS-DMA into a ring of three tile
// buffers, two tiles ahead of the MFMAs: attn_ring_kernel (head dim 32 or
// 64, 64-key tiles) and attn_ring16_kernel (head dim 16, 128-key tiles).
#include "common.h"
#include "kernels.h"

namespace tfl {

typedef __attribute__((address_space(3))) char lds_char;

// max(a, b, c) in one instruction (NaN handling as the file's no-NaN build).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Score variant of this workgroup's (sequence, head), from the maxima of
// |q_i| and |k_j| over it (qk_stats; c converts a score to exp2 units).
//  * split: a single fp16 pass rounds each of q and k by at most u = 2^-11
//    relative, so a score moves by at most (2u + u^2) |q| |k| c
//    (Cauchy-Schwarz over the head dimension; the fp32 accumulation of exact
//    fp16 products adds far less).  With split_mode 1 the hi/lo split is
//    taken only when that bound exceeds SPLIT_EXP_ERR = 2^-8 (a relative
//    error of at most 0.27% in any softmax weight); mode 0 never splits,
//    mode 2 always does.
//  * bounded: every score lies within +-|q| |k| c (times 1 + 2^-9 for the
//    lo parts the hi-plane norms leave out).  When that is at most
//    BOUND_EXP = 14 the weights 2^s lie in [2^-14, 2^14]: exact in fp16
//    range with no reference subtracted (softmax is shift-invariant), so the
//    kernels keep no running max and never rescale.
// Every wave forms the same answers.
constexpr float SPLIT_EXP_ERR = 0.00390625f;  // 2^-8
constexpr float BOUND_EXP = 14.f;
__device__ __forceinline__ void score_variant(const AttnArgs& p, float c, bool& split, bool& bounded) {
    if (!p.qk_stats) {  // no statistics: the variant the split mode names, with a reference
        split = p.split_mode == 2;
        bounded = false;
        if constexpr (MASK_ALL) {
            if (threadIdx.x == 0 && split) audit_add(p.audit, AUD_SPLIT_WG, 1);
        }
        return;
    }
    const float2* st = p.qk_stats + (size_t)blockIdx.x * p.stats_nch;
    float mq = 0.f, mk = 0.f;
    for (int i = (int)(threadIdx.x & 63); i < p.stats_nch; i += 64) {
        mq = fmaxf(mq, st[i].x);
        mk = fmaxf(mk, st[i].y);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mq = fmaxf(mq, __shfl_xor(mq, o, WAVE));
        mk = fmaxf(mk, __shfl_xor(mk, o, WAVE));
    }
    const float qk = mq * mk * c;
    const float err = (0.0009765625f + 2.384185791015625e-07f) * qk;  // (2u + u^2) |q| |k| c
    split = p.split_mode == 2 || (p.split_mode == 1 && !(err <= SPLIT_EXP_ERR));  // NaN or inf: split
    bounded = qk * 1.001953125f <= BOUND_EXP;
    if constexpr (MASK_ALL) {
        if (threadIdx.x == 0) {
            if (split) audit_add(p.audit, AUD_SPLIT_WG, 1);
            if (bounded) audit_add(p.audit, AUD_BOUNDED_WG, 1);
        }
    }
}

// ---------------------------------------------------------------- LDS-DMA ring
// Four output values of one query as fp16; with lo_plane != 0 the rounding
// remainders times 2^11 go lo_plane elements further (fp32 I/O).
__device__ __forceinline__ void store_o4(f16* out, const float (&v)[4], size_t lo_plane) {
    f16x4 hv, lv;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const F16Split s = split_f16(v[e], 2048.0f);
        hv[e] = s.hi;
        lv[e] = s.lo;
    }
    *(f16x4*)out = hv;
    if (lo_plane) *(f16x4*)(out + lo_plane) = lv;
}

// Slot swizzle of K row r in the head-dim-32/64 ring (chunk c of the row in
// slot c ^ ksw(r)).  A score block's 16 lanes read key rows
// {0..3, 8..11, 16..19, 24..27} (+4, +32), and LDS serves a 16-byte read
// eight lanes at a time, so the eight rows {0..3, 8..11} (or {16..19,
// 24..27}) of one chunk must fall on eight distinct 16-byte bank groups:
// (r mod 2, slot) distinct for 128-byte rows, (r mod 4, slot) for 64-byte
// rows.  XOR-ing with r mod 8 (as for consecutive rows) put rows r and r + 8
// on the same banks.
template <int DH>
__device__ __forceinline__ int ksw(int r) {
    if constexpr (DH == 64) return ((r >> 1) & 1) | (((r >> 3) & 3) << 1);
    else return (r >> 3) & 3;
}

// LDS bytes of the head-dim-32/64 ring: three stages of K (hi, and lo when
// SPLIT) and V^T, 64 keys each.
template <int DH, bool SPLIT>
constexpr int ring_lds_bytes() { return 3 * (ATT_KT * DH * 2 * (SPLIT ? 2 : 1) + DH * ATT_KT * 2); }

template <int DH, bool SPLIT, bool BOUNDED>
__device__ __forceinline__ void ring_body(const AttnArgs& p, char* lds) {
    constexpr int KT = ATT_KT, ST = 3;
    constexpr int KROW = DH * 2, KCH = KROW / 16;    // bytes and 16-byte chunks per K row
    constexpr int KB = KT * KROW;                    // one K plane tile
    constexpr int VB = DH * KT * 2;                  // V^T tile: DH rows of 64 keys (128 bytes)
    constexpr int SB = KB * (SPLIT ? 2 : 1) + VB;    // bytes per ring stage
    constexpr int NKD = KT * KCH / 256, NVD = DH * 8 / 256;   // DMA chunks per thread per plane
    constexpr int NDMA = NKD * (SPLIT ? 2 : 1) + NVD;
    constexpr int ND = DH / 16, QK = DH / 32;
    static_assert(NKD >= 1 && NVD >= 1 && NKD * 256 == KT * KCH && NVD * 256 == DH * 8, "head dim 32 or 64");
    static_assert(4 * 16 == ATT_BQ, "planner and kernel disagree on the query tile");
    static_assert(ST * SB == ring_lds_bytes<DH, SPLIT>(), "LDS accounting");

    // wave-uniform wave index: the tile skip and mask tests are scalar branches
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;
    // (sequence, head) fastest, heaviest query tiles first (attn_grid)
    const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
    const int b = (int)blockIdx.x / p.H, h = (int)blockIdx.x - b * p.H;
    const int L = p.L, Lp = p.Lp;
    int len = p.lens[b];
    len = len < 1 ? 1 : (len > L ? L : len);
    const int q0 = qt * ATT_BQ, qw0 = q0 + 16 * wave;
    const int kend = min(q0 + ATT_BQ, len);
    const int ntiles = (kend + KT - 1) / KT;
    const size_t bh = (size_t)b * p.H + h;
    const f16* Qh = (const f16*)p.Q + bh * L * DH;
    const f16* Ql = (const f16*)p.Ql + bh * L * DH;
    const char* Khg = (const char*)((const f16*)p.K + bh * L * DH);
    const char* Klg = (const char*)((const f16*)p.Kl + bh * L * DH);
    const char* Vg = (const char*)((const f16*)p.Vt + bh * DH * Lp);

    const int myq = qw0 + c16;
    const bool qok = myq < L;
    f16x8 qh[QK], ql[SPLIT ? QK : 1];
#pragma unroll
    for (int kk = 0; kk < QK; kk++) {
        qh[kk] = qok ? *(const f16x8*)(Qh + (size_t)myq * DH + kk * 32 + 8 * g) : f16x8{};
        if constexpr (SPLIT) ql[kk] = qok ? *(const f16x8*)(Ql + (size_t)myq * DH + kk * 32 + 8 * g) : f16x8{};
    }
    // The query loads complete here, before any tile DMA is issued: passed
    // through an opaque asm, the registers count as written by it, so the
    // compiler does not wait for those loads inside the tile loop -- a wait
    // that would also cover the DMAs issued ahead (its counter does not see
    // them) and stall every tile on the ring's newest load.
#pragma unroll
    for (int kk = 0; kk < QK; kk++) {
        asm volatile("" : "+v"(qh[kk]));
        if constexpr (SPLIT) asm volatile("" : "+v"(ql[kk]));
    }

    // Swizzle: chunk c of K row r lives in slot c ^ ksw(r), of V^T row r in
    // slot c ^ (r % 8).  DMA lane writes slot q of the tile; it fetches the
    // chunk that belongs there.
    int krow[NKD], kchk[NKD], vrow[NVD], vchk[NVD];
#pragma unroll
    for (int i = 0; i < NKD; i++) {
        const int q = i * 256 + tid;
        krow[i] = q / KCH;
        kchk[i] = (q % KCH) ^ ksw<DH>(krow[i]);
    }
#pragma unroll
    for (int i = 0; i < NVD; i++) {
        const int q = i * 256 + tid;
        vrow[i] = q >> 3;
        vchk[i] = (q & 7) ^ (vrow[i] & 7);
    }
    auto issue = [&](int t, int buf) {
        char* base = lds + buf * SB;
        const int k0 = t * KT;
#pragma unroll
        for (int i = 0; i < NKD; i++) {
            const size_t off = (size_t)min(k0 + krow[i], L - 1) * KROW + 16 * kchk[i];   // rows past L: copies
            dma16(Khg + off, base + (i * 256 + wave * 64) * 16);
            if constexpr (SPLIT) dma16(Klg + off, base + KB + (i * 256 + wave * 64) * 16);
        }
#pragma unroll
        for (int i = 0; i < NVD; i++)
            dma16(Vg + ((size_t)vrow[i] * Lp + k0) * 2 + 16 * vchk[i],
                  base + KB * (SPLIT ? 2 : 1) + (i * 256 + wave * 64) * 16);
    };

    f32x4 o[ND];
#pragma unroll
    for (int db = 0; db < ND; db++) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const int ix16 = (lane ^ 16) << 2, ix32 = (lane ^ 32) << 2;  // ds_bpermute byte indices

    int n_vis = 0;  // tiles scored by this wave (audit build)
#pragma unroll
    for (int s = 0; s < ST - 1; s++)
        if (s < ntiles) issue(s, s);
    for (int t = 0; t < ntiles; t++) {
        if (t + ST - 2 < ntiles)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((ST - 2) * NDMA) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // tile t visible; every wave is done with tile t - 1
        if (t + ST - 1 < ntiles) issue(t + ST - 1, (t + ST - 1) % ST);
        const int k0 = t * KT;
        if (k0 > qw0 + 15) continue;  // this wave's queries all precede the tile
        if constexpr (MASK_ALL) n_vis++;
        const char* ks = lds + (t % ST) * SB;
        const char* kls = ks + KB;
        const char* vs = ks + KB * (SPLIT ? 2 : 1);
        // S^T = K Q^T; key of (block kb, group g, element e) = (kb/2)*32 + 8g + 4(kb%2) + e
        f32x4 sc[4];
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
            sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = (kb >> 1) * 32 + (c16 >> 2) * 8 + (kb & 1) * 4 + (c16 & 3);
#pragma unroll
            for (int kk = 0; kk < QK; kk++) {
                const int slot = ((kk * 4 + g) ^ ksw<DH>(r)) * 16;
                const f16x8 a = *(const f16x8*)(ks + r * KROW + slot);
                sc[kb] = mfma_16x16x32(a, qh[kk], sc[kb]);
                if constexpr (SPLIT) {
                    const f16x8 al = *(const f16x8*)(kls + r * KROW + slot);
                    sc[kb] = mfma_16x16x32(al, qh[kk], sc[kb]);
                    sc[kb] = mfma_16x16x32(a, ql[kk], sc[kb]);
                }
            }
        }
        // scores are in exp2 units (K is stored pre-scaled): running max, then
        // one subtraction per score into the hardware exp2 (its flushing of
        // results below 2^-126 is far below the fp16 rounding of the weights
        // and next to a row sum >= 1)
        const bool need_mask = MASK_ALL || (k0 + KT - 1 > qw0) || (k0 + KT > len);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 4; kb++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int key = k0 + (kb >> 1) * 32 + 8 * g + 4 * (kb & 1) + e;
                    if (key > myq || key >= len) sc[kb][e] = -INFINITY;
                }
        }
        // BOUNDED: every score of this (sequence, head) is within +-14 in
        // exp2 units (bound_scores), so the weights 2^s need no reference:
        // no running max, no rescaling, and none overflows or underflows fp16
        float m_use = 0.f, alpha = 1.f;
        if constexpr (!BOUNDED) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; kb++) {
                mx = max3f(mx, sc[kb][0], sc[kb][1]);
                mx = max3f(mx, sc[kb][2], sc[kb][3]);
            }
            mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(ix16, __float_as_int(mx))));
            mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(ix32, __float_as_int(mx))));
            const float m_new = fmaxf(m_run, mx);
            m_use = (m_new == -INFINITY) ? 0.f : m_new;
            alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 0 while m_run is -inf
            m_run = m_new;
        }
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float pv = __builtin_amdgcn_exp2f(BOUNDED ? sc[kb][e] : sc[kb][e] - m_use);
                sc[kb][e] = pv;
                ls += pv;
            }
        if constexpr (BOUNDED) {
            l_run += ls;
        } else {
            l_run = l_run * alpha + ls;
#pragma unroll
            for (int db = 0; db < ND; db++) o[db] *= alpha;
        }
#pragma unroll
        for (int cc = 0; cc < 2; cc++) {
            f16x8 pb;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                pb[e] = (f16)sc[2 * cc][e];
                pb[4 + e] = (f16)sc[2 * cc + 1][e];
            }
#pragma unroll
            for (int db = 0; db < ND; db++) {
                const int r = db * 16 + c16;
                const f16x8 va = *(const f16x8*)(vs + r * (KT * 2) + (((cc * 4 + g) ^ (r & 7)) * 16));
                o[db] = mfma_16x16x32(va, pb, o[db]);
            }
        }
    }

    l_run += __shfl_xor(l_run, 16, WAVE);
    l_run += __shfl_xor(l_run, 32, WAVE);
    if constexpr (MASK_ALL) {
        if (lane == 0) audit_add(p.audit, AUD_TILED_WAVE, n_vis);
        if (tid == 0) audit_add(p.audit, AUD_TILED_WG, ntiles);
    }
    if (!qok) return;
    const float inv = 1.0f / l_run;
    f16* out = (f16*)p.O + ((size_t)b * L + myq) * p.d + (size_t)h * DH;
#pragma unroll
    for (int db = 0; db < ND; db++) {
        float v[4] = {o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv};
        store_o4(out + db * 16 + 4 * g, v, p.o_lo ? (size_t)p.B * L * p.d : 0);
    }
}

// The variant of a workgroup's (sequence, head) is chosen from the row-norm
// maxima of its Q and K (score_variant): split or single scores, bounded or
// referenced weights.
// CAN_SPLIT: launched with split_mode 1 or 2 (the LDS ring then holds the lo
// K planes too); split_mode 0 launches the copy without them.
template <int DH, bool CAN_SPLIT>
__global__ __launch_bounds__(256) void attn_ring_kernel(AttnArgs p) {
    __shared__ __attribute__((aligned(16))) char lds[ring_lds_bytes<DH, CAN_SPLIT>()];
    bool split, bounded;
    score_variant(p, 1.0f, split, bounded);   // K is stored pre-scaled
    if (CAN_SPLIT && split) {
        if constexpr (CAN_SPLIT) {
            if (bounded) ring_body<DH, true, true>(p, lds);
            else ring_body<DH, true, false>(p, lds);
        }
    } else {
        if (bounded) ring_body<DH, false, true>(p, lds);
        else ring_body<DH, false, false>(p, lds);
    }
}

// ---------------------------------------------------------------- head dim 16
// With 16-dim heads the products are a small part of the work and the
// softmax arithmetic dominates ("KernelForge", "Challenges": the 100k-token
// shape), so this variant trims VALU work per score: 128-key tiles per
// barrier (32 scores per lane); keys written by the QKV projection already
// multiplied by log2(e)/sqrt(dh) and score products accumulated onto the
// negated row reference, so each score goes straight into the hardware exp2;
// the reference raised only when a tile passes it by a margin (no per-tile
// rescaling); and the softmax row sums taken on the MFMA by a ones row
// appended to V^T (the sum of the same fp16 weights that multiply V).
// Queries per workgroup of the head-dim-16 kernel: 8 waves of 16, so each
// staged K/V tile serves 128 queries (the first four waves load it).
constexpr int ATT16_WAVES = 8, ATT16_BQ = 16 * ATT16_WAVES;

template <bool SPLIT>
constexpr int ring16_lds_bytes() { return 3 * (128 * 16 * 2 * (SPLIT ? 2 : 1) + 16 * 128 * 2); }

template <bool SPLIT, bool BOUNDED>
__device__ __forceinline__ void ring16_body(const AttnArgs& p, char* lds) {
    constexpr int DH = 16, KT = 128, ST = 3;
    constexpr int KROW = DH * 2;                     // 32-byte K rows: two 16-byte chunks
    constexpr int KB = KT * KROW;                    // 4 KB per K plane tile
    constexpr int VROW = KT * 2;                     // 256-byte V^T rows: sixteen chunks
    constexpr int VB = DH * VROW;
    constexpr int SB = KB * (SPLIT ? 2 : 1) + VB;
    constexpr int NDMA = (SPLIT ? 2 : 1) + 1;        // one K chunk per plane and one V^T chunk per thread
    static_assert(KT * 2 == 256 && DH * 16 == 256, "one DMA chunk per thread per plane");
    static_assert(ST * SB == ring16_lds_bytes<SPLIT>(), "LDS accounting");

    // the wave index is made wave-uniform, so the tile skip and mask tests
    // below are scalar branches
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;
    // (sequence, head) fastest, heaviest query tiles first (attn_grid)
    const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
    const int b = (int)blockIdx.x / p.H, h = (int)blockIdx.x - b * p.H;
    const int L = p.L, Lp = p.Lp;
    int len = p.lens[b];
    len = len < 1 ? 1 : (len > L ? L : len);
    const int q0 = qt * ATT16_BQ, qw0 = q0 + 16 * wave;
    const int kend = min(q0 + ATT16_BQ, len);
    const int ntiles = (kend + KT - 1) / KT;
    const size_t bh = (size_t)b * p.H + h;
    const f16* Qh = (const f16*)p.Q + bh * L * DH;
    const f16* Ql = (const f16*)p.Ql + bh * L * DH;
    const char* Khg = (const char*)((const f16*)p.K + bh * L * DH);
    const char* Klg = (const char*)((const f16*)p.Kl + bh * L * DH);
    const char* Vg = (const char*)((const f16*)p.Vt + bh * DH * Lp);

    const int myq = qw0 + c16;
    const bool qok = myq < L;
    f16x4 qh = qok ? *(const f16x4*)(Qh + (size_t)myq * DH + 4 * g) : f16x4{};
    f16x4 ql = (SPLIT && qok) ? *(const f16x4*)(Ql + (size_t)myq * DH + 4 * g) : f16x4{};
    // the query loads complete here, before any tile DMA (see attn_ring_kernel)
    asm volatile("" : "+v"(qh));
    if constexpr (SPLIT) asm volatile("" : "+v"(ql));

    // DMA: thread tid fetches K chunk slot tid & 1 of LDS row tid >> 1 and V^T
    // row tid >> 4 (chunk slot tid & 15).  LDS K row 16 kb + i holds the key
    // that lane i reads for score block kb (key (kb/2)*32 + 8(i/4) + 4(kb%2) +
    // i%4), so a block's A operand is 16 consecutive 32-byte rows; its two
    // chunks are swapped in rows 8-15 of the block, which puts each half-wave's
    // 8-byte reads on 64 distinct banks.  V^T rows: chunk c in slot c ^ (r mod 16).
    const int krow = tid >> 1, kchk = (tid & 1) ^ ((krow >> 3) & 1);
    const int kkey = ((krow >> 5) * 32) + (((krow & 15) >> 2) * 8) + (((krow >> 4) & 1) * 4) + (krow & 3);
    const int vrow = tid >> 4, vchk = (tid & 15) ^ (vrow & 15);
    auto issue = [&](int t, int buf) {
        char* base = lds + buf * SB;
        const int k0 = t * KT;
        const size_t off = (size_t)min(k0 + kkey, L - 1) * KROW + 16 * kchk;   // keys past L: copies
        dma16(Khg + off, base + wave * 64 * 16);
        if constexpr (SPLIT) dma16(Klg + off, base + KB + wave * 64 * 16);
        dma16(Vg + ((size_t)vrow * Lp + k0) * 2 + 16 * vchk, base + KB * (SPLIT ? 2 : 1) + wave * 64 * 16);
    };

    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 lsum = f32x4{0.f, 0.f, 0.f, 0.f};          // row 0 of (ones . P^T): the weight sums
    const f16 one = (f16)(c16 == 0 ? 1.0f : 0.0f);
    const f16x8 ones = {one, one, one, one, one, one, one, one};
    // Keys arrive multiplied by log2(e)/sqrt(dh), and each score product starts
    // from -m_ref, so the MFMA leaves the exponent of exp2 itself.  m_ref (per
    // query) is the exact row max of the first key tile (every wave computes
    // tile 0, and key 0 is visible to every query); later it is raised only
    // when a tile's max passes it by more than RESCALE, so the row's largest
    // weight stays in [1, 2^RESCALE]: the online softmax is exact for any such
    // reference, and no weight underflows that the running max would keep.
    constexpr float RESCALE = 8.f;
    float m_ref = 0.f;
    int n_vis = 0;  // tiles scored by this wave (audit build)

    // waves 0-3 load the tiles (one chunk per thread per plane); the others
    // issue no loads, so their waits below return at once
    const bool loader = wave < 4;
#pragma unroll
    for (int s = 0; s < ST - 1; s++)
        if (loader && s < ntiles) issue(s, s);
    // Per-lane LDS byte addresses, fixed for the kernel: this lane's K
    // fragment in each score block and its V^T chunk for each 32-key group, in
    // ring buffer 0.  The tile loop below is unrolled over the ST ring buffers,
    // so a buffer's offset is an immediate of the read.  Each K address goes
    // through an opaque copy once: the compiler then keeps the eight reads
    // separate (merged into a two-address read, blocks 512 bytes apart meet on
    // the same banks) without recomputing their addresses at every tile.
    const unsigned lds0 = (unsigned)(size_t)(lds_char*)lds;
    const int koff = c16 * KROW + (((g >> 1) ^ (c16 >> 3)) * 16) + (g & 1) * 8;
    // The lo plane's reads get addresses of their own (opaque as well): from
    // the hi addresses plus 4 KB the compiler forms two-address reads of a hi
    // and a lo fragment, which meet on the same banks.
    unsigned kad[8], kadl[SPLIT ? 8 : 1], vad[4];
#pragma unroll
    for (int kb = 0; kb < 8; kb++) {
        kad[kb] = lds0 + kb * 16 * KROW + koff;
        asm volatile("" : "+v"(kad[kb]));
        if constexpr (SPLIT) {
            kadl[kb] = lds0 + KB + kb * 16 * KROW + koff;
            asm volatile("" : "+v"(kadl[kb]));
        }
    }
#pragma unroll
    for (int cc = 0; cc < 4; cc++) vad[cc] = lds0 + KB * (SPLIT ? 2 : 1) + c16 * VROW + (((cc * 4 + g) ^ c16) * 16);
    // lanes l ^ 16 and l ^ 32 (byte indices for ds_bpermute)
    const int ix16 = (lane ^ 16) << 2, ix32 = (lane ^ 32) << 2;
    typedef const __attribute__((address_space(3))) f16x4 lds_f16x4;
    typedef const __attribute__((address_space(3))) f16x8 lds_f16x8;

    auto tile = [&](const int t, auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        constexpr unsigned BO = BUF * SB;
        if (t + ST - 2 < ntiles)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((ST - 2) * NDMA) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (loader && t + ST - 1 < ntiles) issue(t + ST - 1, (BUF + ST - 1) % ST);
        const int k0 = t * KT;
        if (k0 > qw0 + 15) return;
        if constexpr (MASK_ALL) n_vis++;
        // key of (block kb, group g, element e) = (kb/2)*32 + 8g + 4(kb%2) + e
        f32x4 sc[8];
        f16x4 ka[8], kl[8];
#pragma unroll
        for (int kb = 0; kb < 8; kb++) {
            ka[kb] = *(lds_f16x4*)(size_t)(kad[kb] + BO);
            if constexpr (SPLIT) kl[kb] = *(lds_f16x4*)(size_t)(kadl[kb] + BO);
        }
        const f32x4 c0 = BOUNDED ? f32x4{0.f, 0.f, 0.f, 0.f} : f32x4{-m_ref, -m_ref, -m_ref, -m_ref};
#pragma unroll
        for (int kb = 0; kb < 8; kb++) {
            sc[kb] = mfma_16x16x16(ka[kb], qh, c0);
            if constexpr (SPLIT) {
                sc[kb] = mfma_16x16x16(kl[kb], qh, sc[kb]);
                sc[kb] = mfma_16x16x16(ka[kb], ql, sc[kb]);
            }
        }
        // all K fragments of the tile are read before the first product
#pragma unroll
        for (int i = 0; i < (SPLIT ? 8 : 4); i++) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, SPLIT ? 24 : 8, 0);
        const bool need_mask = MASK_ALL || (k0 + KT - 1 > qw0) || (k0 + KT > len);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 8; kb++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int key = k0 + (kb >> 1) * 32 + 8 * g + 4 * (kb & 1) + e;
                    if (key > myq || key >= len) sc[kb][e] = -INFINITY;
                }
        }
        // BOUNDED: every score of this (sequence, head) is within +-14 in
        // exp2 units (score_variant), so the weights 2^s need no reference:
        // no running max, no raise, and none overflows or underflows fp16
        if constexpr (!BOUNDED) {
        // running max as a chain of three-input maxima (two new values each;
        // left to itself the compiler spends three instructions per four)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 8; kb++) {
            mx = max3f(mx, sc[kb][0], sc[kb][1]);
            mx = max3f(mx, sc[kb][2], sc[kb][3]);
        }
        // mx: the largest exponent among this lane's 32 scores.  The four
        // lanes of a query share its reference (their weights meet in one
        // MFMA), so the row max over them is formed only where the reference
        // is set or raised; the common path needs just this lane's test.
        auto row_max = [&](float v) __attribute__((always_inline)) {
            v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute(ix16, __float_as_int(v))));
            return fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute(ix32, __float_as_int(v))));
        };
        if (t == 0) {
            mx = row_max(mx);
            m_ref = mx;
#pragma unroll
            for (int kb = 0; kb < 8; kb++) sc[kb] -= mx;
        } else if (__ballot(mx > RESCALE) != 0) {
            mx = row_max(mx);
            const float dl = fmaxf(mx, 0.f);
            m_ref += dl;
#pragma unroll
            for (int kb = 0; kb < 8; kb++) sc[kb] -= dl;
            const float alpha = __builtin_amdgcn_exp2f(-dl);
            o *= alpha;
            lsum *= alpha;
        }
        }
#pragma unroll
        for (int cc = 0; cc < 4; cc++) {
            f16x8 pb;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                pb[e] = (f16)__builtin_amdgcn_exp2f(sc[2 * cc][e]);
                pb[4 + e] = (f16)__builtin_amdgcn_exp2f(sc[2 * cc + 1][e]);
            }
            const f16x8 va = *(lds_f16x8*)(size_t)(vad[cc] + BO);
            o = mfma_16x16x32(va, pb, o);
            lsum = mfma_16x16x32(ones, pb, lsum);
        }
    };
    for (int t = 0; t < ntiles; t += ST) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
        if (t + 2 < ntiles) tile(t + 2, std::integral_constant<int, 2>{});
    }
    static_assert(ST == 3, "the tile loop is unrolled over three ring buffers");

    // lsum row 0 (lanes 0..15, element 0) holds the weight sum of query c16
    const float l = __shfl(lsum[0], c16, WAVE);
    if constexpr (MASK_ALL) {
        if (lane == 0) audit_add(p.audit, AUD_TILED_WAVE, n_vis);
        if (tid == 0) audit_add(p.audit, AUD_TILED_WG, ntiles);
    }
    if (!qok) return;
    const float inv = 1.0f / l;
    f16* out = (f16*)p.O + ((size_t)b * L + myq) * p.d + (size_t)h * DH;
    float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    store_o4(out + 4 * g, v, p.o_lo ? (size_t)p.B * L * p.d : 0);
}

// Keys are stored multiplied by log2(e)/sqrt(dh), so their norms are already
// in exp2 units.
template <bool CAN_SPLIT>
__global__ __launch_bounds__(64 * ATT16_WAVES) void attn_ring16_kernel(AttnArgs p) {
    __shared__ __attribute__((aligned(16))) char lds[ring16_lds_bytes<CAN_SPLIT>()];
    bool split, bounded;
    score_variant(p, 1.0f, split, bounded);
    if (CAN_SPLIT && split) {
        if constexpr (CAN_SPLIT) {
            if (bounded) ring16_body<true, true>(p, lds);
            else ring16_body<true, false>(p, lds);
        }
    } else {
        if (bounded) ring16_body<false, true>(p, lds);
        else ring16_body<false, false>(p, lds);
    }
}

// ---------------------------------------------------------------- Q/K statistics
// Maxima of the row norms |q_i| and |k_j| of one (sequence, head) over a
// chunk of QKS_ROWS rows of the hi planes, one workgroup per (sequence
// head, chunk): out[bh * nch + chunk] = (max |q_i|, max |k_j|).
constexpr int QKS_ROWS = 256;  // one row per thread: enough workgroups to fill the chip at B*H = 4

template <int DH>
__global__ __launch_bounds__(256) void qk_stats_kernel(const f16* __restrict__ Q, const f16* __restrict__ K, int L,
                                                       float2* __restrict__ out, int nch) {
    const int bh = blockIdx.x, ch = blockIdx.y;
    const size_t base = (size_t)bh * L * DH;
    const int r1 = min(L, (ch + 1) * QKS_ROWS);
    float mq = 0.f, mk = 0.f;
    for (int r = ch * QKS_ROWS + (int)threadIdx.x; r < r1; r += 256) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < DH / 8; c++) {
            const f16x8 a = *(const f16x8*)(Q + base + (size_t)r * DH + 8 * c);
            const f16x8 k = *(const f16x8*)(K + base + (size_t)r * DH + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                sq = fmaf((float)a[e], (float)a[e], sq);
                sk = fmaf((float)k[e], (float)k[e], sk);
            }
        }
        mq = fmaxf(mq, sq);
        mk = fmaxf(mk, sk);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mq = fmaxf(mq, __shfl_xor(mq, o, WAVE));
        mk = fmaxf(mk, __shfl_xor(mk, o, WAVE));
    }
    __shared__ float2 part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = float2{mq, mk};
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; w++) {
            mq = fmaxf(mq, part[w].x);
            mk = fmaxf(mk, part[w].y);
        }
        // sqrt rounds to nearest; one ulp up keeps the result an upper bound
        out[(size_t)bh * nch + ch] = float2{__uint_as_float(__float_as_uint(sqrtf(mq)) + 1u),
                                            __uint_as_float(__float_as_uint(sqrtf(mk)) + 1u)};
    }
}

int qk_stats_chunks(int L) { return (L + QKS_ROWS - 1) / QKS_ROWS; }

hipError_t launch_qk_stats(int dh, const void* Q, const void* K, int BH, int L, float2* out, hipStream_t s) {
    if (BH <= 0 || L <= 0) return hipSuccess;
    const dim3 grid((unsigned)BH, (unsigned)qk_stats_chunks(L));
    switch (dh) {
        case 16: hipLaunchKernelGGL(qk_stats_kernel<16>, grid, dim3(256), 0, s, (const f16*)Q, (const f16*)K, L, out, (int)grid.y); break;
        case 32: hipLaunchKernelGGL(qk_stats_kernel<32>, grid, dim3(256), 0, s, (const f16*)Q, (const f16*)K, L, out, (int)grid.y); break;
        case 64: hipLaunchKernelGGL(qk_stats_kernel<64>, grid, dim3(256), 0, s, (const f16*)Q, (const f16*)K, L, out, (int)grid.y); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Launch grid: x = (sequence, head), y = query tile.  Workgroups are handed
// to the eight XCDs round-robin in linear order (x fastest), so with
// (sequence, head) fastest every query tile of one (sequence, head) lands on
// the same XCD whenever B*H is a multiple of 8 or divides 8, and its K/V
// tiles are fetched into that XCD's L2 once instead of once per XCD; the
// kernels take query tiles from the last (the most keys) to the first.
static dim3 attn_grid(const AttnArgs& a, int bq) { return dim3((unsigned)(a.B * a.H), (unsigned)((a.L + bq - 1) / bq)); }

hipError_t launch_attn(Mode m, int dh, const AttnArgs& a, hipStream_t s) {
    (void)m;  // every mode takes fp16 Q/K/V planes
    if (a.B <= 0 || a.L <= 0) return hipSuccess;
    if ((a.qk_stats && a.stats_nch < 1) || (!a.qk_stats && a.split_mode == 1)) return hipErrorInvalidValue;
    if ((a.L + ATT_BQ - 1) / ATT_BQ > 65535) return hipErrorInvalidValue;  // query tiles: grid y
    const bool cs = a.split_mode != 0;
    const dim3 g64 = attn_grid(a, ATT_BQ), g16 = attn_grid(a, ATT16_BQ);
    switch (dh) {
        case 64:
            if (cs) hipLaunchKernelGGL((attn_ring_kernel<64, true>), g64, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((attn_ring_kernel<64, false>), g64, dim3(256), 0, s, a);
            break;
        case 32:
            if (cs) hipLaunchKernelGGL((attn_ring_kernel<32, true>), g64, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((attn_ring_kernel<32, false>), g64, dim3(256), 0, s, a);
            break;
        case 16:  // the plan pads V^T rows to whole 128-key tiles
            if (cs) hipLaunchKernelGGL((attn_ring16_kernel<true>), g16, dim3(64 * ATT16_WAVES), 0, s, a);
            else hipLaunchKernelGGL((attn_ring16_kernel<false>), g16, dim3(64 * ATT16_WAVES), 0, s, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tfl
