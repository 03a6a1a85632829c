// Device-side building blocks shared by the tfl kernels (gfx950 / CDNA4).
//
// Storage types: fp32, fp16 and bf16 (bf16 is carried as raw uint16 bits and
// only ever widened to fp32 or narrowed from it).  All narrowing conversions
// round to nearest even.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfl {

typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct bf16 {
    uint16_t u;
};

static constexpr int WAVE = 64;

// ---------------------------------------------------------------- audit build
// A second copy of the library, built with TFL_AUDIT=1 for the tests only,
// checks two claims of "KernelForge", "Challenges" about the attention loop:
// (1) evaluating the mask only on key tiles that reach past the diagonal or
// the padding boundary gives bit-identical results to evaluating it on every
// tile, and (2) the tiles visited are exactly those holding an allowed key,
// M(M+1)/2 of M^2 at full length.  In that build every attention kernel masks
// every tile it visits (MASK_ALL) and adds the tiles it visits to counters in
// device memory (audit_add).  In the product build both compile to nothing.
#ifndef TFL_AUDIT
#define TFL_AUDIT 0
#endif
constexpr bool MASK_ALL = TFL_AUDIT != 0;
// Counter slots (uint64 each).
enum AuditSlot {
    AUD_TILED_WG = 0,    // layer-wise attention: key tiles staged per workgroup
    AUD_TILED_WAVE = 1,  // layer-wise attention: key tiles scored per 16-query wave
    AUD_SEQ_WAVE = 2,    // fused SEQ kernel: 32-key chunks scored per 16-query wave
    AUD_PQ_WG = 3,       // PQ attention tasks: key tiles staged per task
    AUD_PQ_WAVE = 4,     // PQ attention tasks: key tiles scored per 16-query wave
    AUD_SPLIT_WG = 5,    // layer-wise attention workgroups / PQ attention tasks that took the split scores
    AUD_BOUNDED_WG = 6,  // the same whose weights need no reference
    AUD_SLOTS = 8
};
__device__ __forceinline__ void audit_add(unsigned long long* ctr, int slot, unsigned long long v) {
#if TFL_AUDIT
    if (ctr) atomicAdd(ctr + slot, v);
#else
    (void)ctr, (void)slot, (void)v;
#endif
}

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float((uint32_t)v.u << 16); }

template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }  // v_cvt_f16_f32, RNE
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (inputs are finite)
    bf16 r;
    r.u = (uint16_t)(u >> 16);
    return r;
}

// v as an fp16 hi part and the rounding remainder v - hi (exact in fp32)
// times lo_scale, both taken from the same fp32 value.  v passes through an
// empty asm first: where v is the result of a product or an FMA, the compiler
// may otherwise fuse that operation into the fp16 conversion of hi (one
// rounding from the exact result, v_fma_mix) while the remainder is formed
// from the fp32-rounded v; at an fp16 rounding midpoint the two then disagree
// and hi + lo is off by one fp16 ulp instead of ~2^-22 of v.
struct F16Split {
    f16 hi, lo;
};
__device__ __forceinline__ F16Split split_f16(float v, float lo_scale) {
    asm("" : "+v"(v));
    const f16 hi = (f16)v;
    return F16Split{hi, (f16)((v - (float)hi) * lo_scale)};
}

// Eight consecutive stored values -> eight fp16 MFMA operands.
__device__ __forceinline__ f16x8 load8_as_f16(const f16* p) { return *(const f16x8*)p; }
__device__ __forceinline__ f16x8 load8_as_f16(const bf16* p) {
    uint4 r = *(const uint4*)p;
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        o[2 * i] = (f16)__uint_as_float(w[i] << 16);
        o[2 * i + 1] = (f16)__uint_as_float(w[i] & 0xFFFF0000u);
    }
    return o;
}
__device__ __forceinline__ f16x8 load8_as_f16(const float* p) {
    float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    f16x8 o = {(f16)a.x, (f16)a.y, (f16)a.z, (f16)a.w, (f16)b.x, (f16)b.y, (f16)b.z, (f16)b.w};
    return o;
}

// ---------------------------------------------------------------- MFMA
// Lane layouts (lane l, g = l / 16), as used throughout:
//   16x16x32 f16:  A[i][k] in lane i + 16*(k/8), element k%8;  B[k][j] in lane j + 16*(k/8)
//   16x16x16 f16:  A[i][k] in lane i + 16*(k/4), element k%4;  B likewise
//   16x16x4  f32:  A[i][k] in lane i + 16*k;                    B[k][j] in lane j + 16*k
//   result D[i][j] (all three): lane j + 16*(i/4), element i%4

__device__ __forceinline__ f32x4 mfma_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS-DMA

typedef __attribute__((address_space(3))) f16 lds_f16;

// 16-byte global-to-LDS load: lane i of the wave writes its 16 source bytes
// to lds_wave_base + 16 i (lds_wave_base is wave-uniform).  Issued through
// asm so the compiler does not make every later LDS read wait for it; the
// caller waits (s_waitcnt vmcnt) before the barrier that publishes the data.
// M0 is written here and has no other user in the kernels that call this.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_f16*)lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory", "m0");
}
// The same with a wave-uniform base address (SGPRs) and a per-lane 32-bit
// byte offset, so a run of loads from one base differs only in scalar adds.
__device__ __forceinline__ void dma16s(const void* sbase, unsigned voff, void* lds_wave_base) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_f16*)lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(sbase) : "memory", "m0");
}
#pragma clang diagnostic pop

// ---------------------------------------------------------------- wave reductions

template <int WIDTH>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Lane exchanges inside a row of 16 lanes by DPP (a register move with a
// lane pattern; no LDS round trip): partner lane i ^ 1, i ^ 2 within each
// quad, and 7 - i within each group of 8.  After dpp_xor1 and dpp_xor2 sums a
// quad holds its total; dpp_mirror8 then pairs the two quads of an 8-group.
__device__ __forceinline__ float dpp_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_mirror8(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
}

// GELU over the whole range with no branch (the exact-erf GELU of
// "KernelForge", "How the LLM is used", to fp32 rounding): with
// a = |h|/sqrt(2), u = 1/(2 + a) and e = erfc(a)/2 = u 2^(R(u) - a^2 log2 e),
// GELU(h) = h - h e for h >= 0 and h e for h < 0.  R is the degree-9 fit of
// csrc/fit_erf_poly.py over a in [0, 9.3]; past it e < 2^-126 and the
// hardware exp2 flushes it to 0.  In fp32: absolute error <= 2.4e-7, relative
// <= 1.4e-6 for |h| <= 3 (larger relative error only where |GELU| < 5e-9).
// 18 instructions (two transcendental), against ~40 for the library erf with
// both of its branches taken in a wave.
__device__ __forceinline__ float gelu_full(float h) {
    const float a = fabsf(h) * 0.70710678118654752f;
    const float u = __builtin_amdgcn_rcpf(a + 2.0f);
    float r = fmaf(u, 100.67699432373047f, -233.99356079101562f);
    r = fmaf(u, r, 192.95802307128906f);
    r = fmaf(u, r, -50.46892547607422f);
    r = fmaf(u, r, -9.452345848083496f);
    r = fmaf(u, r, 1.5642825365066528f);
    r = fmaf(u, r, 0.13682980835437775f);
    r = fmaf(u, r, 2.2588467597961426f);
    r = fmaf(u, r, 2.879826545715332f);
    r = fmaf(u, r, -1.825615406036377f);
    const float e = u * __builtin_amdgcn_exp2f(fmaf(a * a, -1.4426950408889634f, r));
    const float he = h * e;
    return h >= 0.f ? h - he : he;
}

// GELU for |h| < GELU_SMALL_MAX (erf argument h / sqrt(2) inside [-1, 1]):
// with erf(x) = x P(x^2), P the degree-5 fit of csrc/fit_erf_poly.py
// (relative error 4e-8 in exact arithmetic), GELU(h) = h/2 + u R(u) with
// u = h^2 and R(u) = P(u/2) / (2 sqrt(2)), i.e. coefficient k of P scaled by
// 2^-k / (2 sqrt(2)).  Eight instructions; in fp32 within 10.5 ulp of the
// exact GELU (the error of h/2 (1 + erf) where erf nears -1 cancels), the
// same as evaluating erf first.  No branch.
constexpr float GELU_SMALL_MAX = 1.4142f;
__device__ __forceinline__ float gelu_poly(float h) {
    const float u = h * h;
    float r = fmaf(u, -6.221906e-06f, 0.00010866358f);
    r = fmaf(u, r, -0.0011804844f);
    r = fmaf(u, r, 0.009970365f);
    r = fmaf(u, r, -0.06648983f);
    r = fmaf(u, r, 0.39894226f);
    return fmaf(u, r, 0.5f * h);
}
// The same form with P of degree 3 (csrc/fit_erf_poly.py), for products
// whose GELU output is rounded to fp16 next (the fused kernels' FFN
// activations): within 1.7e-5 of the exact GELU and under 0.7 fp16 ulp of
// its value on |h| < GELU_SMALL_MAX, i.e. one more rounding of at most that
// size before the fp16 one.  Six instructions.
__device__ __forceinline__ float gelu_poly16(float h) {
    const float u = h * h;
    float r = fmaf(u, -0.0008117355173453689f, 0.009531241841614246f);
    r = fmaf(u, r, -0.06631539762020111f);
    r = fmaf(u, r, 0.3989310562610626f);
    return fmaf(u, r, 0.5f * h);
}
// GELU of N values in place: the short-range form when every value of the
// wave is in its range (one wave-uniform test), the whole-range form
// otherwise.  Normalised activations keep to the short range almost always,
// so the common case is straight-line code with no divergent branches.
// FP16_OUT: the values are rounded to fp16 next, so the short range takes
// gelu_poly16.
template <int N, bool FP16_OUT = false>
__device__ __forceinline__ void gelu_inplace(float* v) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < N; i++) m = fmaxf(m, fabsf(v[i]));
    if (__ballot(!(m < GELU_SMALL_MAX)) == 0) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] = FP16_OUT ? gelu_poly16(v[i]) : gelu_poly(v[i]);
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] = gelu_full(v[i]);
    }
}

}  // namespace tfl
