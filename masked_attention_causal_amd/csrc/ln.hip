// Residual LayerNorm and input staging.
//
// LayerNorm is the textbook two-pass one: mean first, then the biased
// variance of the centred values, both in fp32, eps added in fp32, then the
// affine map (the post-LN layer of the PyTorch reference the pages were
// gated against: "Hyper-optimized megakernel-hybrid transformer inference",
// "Challenges").  A row is spread over a group of lanes of one wave
// (up to 64) that read it as coalesced float4 chunks; the reductions are
// butterfly shuffles inside the group.  The row then leaves as fp32 (the
// residual stream), as an fp16 operand copy for the next GEMM (with fp32 I/O
// two planes: the rounded value and the remainder times 2^11), and/or, in
// the last layer, as the I/O dtype output.
//
// Also here: the staging kernels of the layer-wise path (input rows to the
// fp32 residual and the operand planes; weights to fp16 planes; zero padding
// of the V^T rows).
#include "common.h"
#include "kernels.h"

namespace tfl {

namespace {

// Four consecutive stored values as fp32 (one 8- or 16-byte load).
__device__ __forceinline__ void ld4(const float* p, float (&v)[4]) {
    const float4 t = *(const float4*)p;
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void ld4(const f16* p, float (&v)[4]) {
    const f16x4 t = *(const f16x4*)p;
#pragma unroll
    for (int e = 0; e < 4; e++) v[e] = (float)t[e];
}
__device__ __forceinline__ void ld4(const bf16* p, float (&v)[4]) {
    const uint2 t = *(const uint2*)p;
    v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xFFFF0000u);
}
// Four values stored in T, round to nearest even (one 8- or 16-byte store).
template <class T>
__device__ __forceinline__ void st4(T* p, const float (&v)[4]) {
    if constexpr (sizeof(T) == 4) {
        *(float4*)p = float4{v[0], v[1], v[2], v[3]};
    } else {
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const T t = from_f32<T>(v[e]);
            h[e] = *(const uint16_t*)&t;
        }
        *(uint2*)p = uint2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    }
}

}  // namespace

bool ln_shape(int d, int* lanes_per_row, int* chunks) {
    if (d <= 0 || d % 4 != 0) return false;
    const int q = d / 4;
    int lpr = 1;
    while (lpr < 64 && q % (lpr * 2) == 0) lpr *= 2;
    const int nc = q / lpr;
    if (nc > 8) return false;
    *lanes_per_row = lpr;
    *chunks = nc;
    return true;
}

// fp16 rounding of four values and, for LO, the remainders times 2^11.
__device__ __forceinline__ void st4_split(f16* p, size_t lo_plane, const float (&v)[4]) {
    float h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const F16Split s = split_f16(v[e], 2048.0f);
        h[e] = (float)s.hi;
        l[e] = (float)s.lo;
    }
    st4(p, h);
    st4(p + lo_plane, l);
}

template <class PT, int LPR, int NC, bool LO>
__global__ __launch_bounds__(256) void ln_kernel(const float* __restrict__ Z, const PT* __restrict__ gamma,
                                                 const PT* __restrict__ beta, float eps, int T, int d,
                                                 float* __restrict__ Xo, f16* __restrict__ Ao,
                                                 PT* __restrict__ Y) {
    constexpr int RPB = 256 / LPR;  // rows per block
    const int tid = threadIdx.x;
    const int sub = tid % LPR;
    const long row = (long)blockIdx.x * RPB + tid / LPR;
    if (row >= T) return;  // whole lane groups leave together
    const float* z = Z + row * d;
    float4 v[NC];
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        v[c] = *(const float4*)(z + (c * LPR + sub) * 4);
        s += (v[c].x + v[c].y) + (v[c].z + v[c].w);
    }
    s = wave_sum<LPR>(s);
    const float mean = s / (float)d;
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        v[c].x -= mean; v[c].y -= mean; v[c].z -= mean; v[c].w -= mean;
        q += (v[c].x * v[c].x + v[c].y * v[c].y) + (v[c].z * v[c].z + v[c].w * v[c].w);
    }
    q = wave_sum<LPR>(q);
    const float rstd = 1.0f / sqrtf(q / (float)d + eps);
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int col = (c * LPR + sub) * 4;
        float o[4] = {v[c].x, v[c].y, v[c].z, v[c].w}, ga[4], be[4];
        ld4(gamma + col, ga);
        ld4(beta + col, be);
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = o[e] * rstd * ga[e] + be[e];
        if (Xo) *(float4*)(Xo + row * d + col) = float4{o[0], o[1], o[2], o[3]};
        if (Ao) {
            if constexpr (LO)
                st4_split(Ao + row * d + col, (size_t)T * d, o);
            else
                st4(Ao + row * d + col, o);
        }
        if (Y) st4(Y + row * d + col, o);
    }
}

template <class PT, int LPR, bool LO>
static hipError_t ln_nc(int nc, const float* Z, const void* g, const void* b, float eps, int T, int d,
                        float* Xo, void* Ao, void* Y, hipStream_t s) {
    constexpr int RPB = 256 / LPR;
    dim3 grid((T + RPB - 1) / RPB);
#define TFL_LN_CASE(NC)                                                                          \
    case NC:                                                                                     \
        hipLaunchKernelGGL((ln_kernel<PT, LPR, NC, LO>), grid, dim3(256), 0, s, Z, (const PT*)g,  \
                           (const PT*)b, eps, T, d, Xo, (f16*)Ao, (PT*)Y);                        \
        break;
    switch (nc) {
        TFL_LN_CASE(1) TFL_LN_CASE(2) TFL_LN_CASE(3) TFL_LN_CASE(4)
        TFL_LN_CASE(5) TFL_LN_CASE(6) TFL_LN_CASE(7) TFL_LN_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef TFL_LN_CASE
    return hipGetLastError();
}

template <class PT, bool LO>
static hipError_t ln_mode(const float* Z, const void* g, const void* b, float eps, int T, int d, float* Xo,
                          void* Ao, void* Y, hipStream_t s) {
    int lpr, nc;
    if (!ln_shape(d, &lpr, &nc)) return hipErrorInvalidValue;
    switch (lpr) {
        case 1: return ln_nc<PT, 1, LO>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 2: return ln_nc<PT, 2, LO>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 4: return ln_nc<PT, 4, LO>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 8: return ln_nc<PT, 8, LO>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 16: return ln_nc<PT, 16, LO>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 32: return ln_nc<PT, 32, LO>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 64: return ln_nc<PT, 64, LO>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_ln(Mode m, const float* Z, const void* g, const void* b, float eps, int T, int d, float* Xo,
                     void* Ao, void* Y, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    switch (m) {
        case MODE_F32: return ln_mode<float, true>(Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case MODE_F16: return ln_mode<f16, false>(Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case MODE_BF16: return ln_mode<bf16, false>(Z, g, b, eps, T, d, Xo, Ao, Y, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- input staging
// x (I/O dtype) -> fp32 residual stream and fp16 operand copy (fp32 I/O: hi
// plane and the remainder times 2^11 n elements further).
template <class XT>
__global__ __launch_bounds__(256) void prep_kernel(const XT* __restrict__ x, float* __restrict__ Xr,
                                                   f16* __restrict__ A, long n) {
    const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;  // n is a multiple of 4 (d % 4 == 0)
    float v[4];
    ld4(x + i, v);
    *(float4*)(Xr + i) = float4{v[0], v[1], v[2], v[3]};
    if constexpr (sizeof(XT) == 4)
        st4_split(A + i, (size_t)n, v);
    else
        st4(A + i, v);
}

hipError_t launch_prep(Mode m, const void* x, float* Xr, void* A, long n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    dim3 grid((unsigned)((n / 4 + 255) / 256));
    switch (m) {
        case MODE_F32:
            hipLaunchKernelGGL((prep_kernel<float>), grid, dim3(256), 0, s, (const float*)x, Xr, (f16*)A, n);
            break;
        case MODE_F16:
            hipLaunchKernelGGL((prep_kernel<f16>), grid, dim3(256), 0, s, (const f16*)x, Xr, (f16*)A, n);
            break;
        case MODE_BF16:
            hipLaunchKernelGGL((prep_kernel<bf16>), grid, dim3(256), 0, s, (const bf16*)x, Xr, (f16*)A, n);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- weight staging
// Each segment's weights to fp16: bf16 values are exact in fp16 within its
// range (8 significant bits); fp32 values leave as the rounded value and the
// remainder times 2^11 (n elements further), the split operands of the
// three-MFMA products.  Eight weights per thread per step.
template <class WT>
__global__ __launch_bounds__(256) void wconv_kernel(WconvArgs a) {
    const WconvSeg sg = a.seg[blockIdx.y];
    const long step = (long)gridDim.x * 256 * 8;
    for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8; i < sg.n; i += step) {
        float v[8];
        ld4((const WT*)sg.src + i, *(float(*)[4])v);
        ld4((const WT*)sg.src + i + 4, *(float(*)[4])(v + 4));
        if constexpr (sizeof(WT) == 4) {
            st4_split(sg.dst + i, (size_t)sg.n, *(const float(*)[4])v);
            st4_split(sg.dst + i + 4, (size_t)sg.n, *(const float(*)[4])(v + 4));
        } else {
            st4(sg.dst + i, *(const float(*)[4])v);
            st4(sg.dst + i + 4, *(const float(*)[4])(v + 4));
        }
    }
}

hipError_t launch_wconv(Mode m, const WconvArgs& a, hipStream_t s) {
    if (a.nseg <= 0) return hipSuccess;
    if (a.nseg > WCONV_MAX_SEGS) return hipErrorInvalidValue;
    long mx = 0;
    for (int i = 0; i < a.nseg; i++) {
        if (a.seg[i].n % 8 != 0) return hipErrorInvalidValue;
        mx = a.seg[i].n > mx ? a.seg[i].n : mx;
    }
    const long blocks = (mx / 8 + 255) / 256;
    dim3 grid((unsigned)(blocks < 1024 ? (blocks > 0 ? blocks : 1) : 1024), (unsigned)a.nseg);
    switch (m) {
        case MODE_F32: hipLaunchKernelGGL((wconv_kernel<float>), grid, dim3(256), 0, s, a); break;
        case MODE_BF16: hipLaunchKernelGGL((wconv_kernel<bf16>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- magnitude check
// Largest |v| over n stored values, as fp32 bits atomically maxed into *out
// (non-negative floats order like their bit patterns; a NaN has larger bits
// than inf, so it shows as not finite).  Used by the TFL_CHECK=1 argument check.
template <class T>
__global__ __launch_bounds__(256) void amax_kernel(const T* __restrict__ x, long n, unsigned* __restrict__ out) {
    unsigned m = 0;
    const long step = (long)gridDim.x * 256 * 4;
    for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += step) {
        float v[4];
        ld4(x + i, v);
#pragma unroll
        for (int e = 0; e < 4; e++) m = max(m, __float_as_uint(v[e]) & 0x7FFFFFFFu);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, o, WAVE));
    if ((threadIdx.x & 63) == 0 && m) atomicMax(out, m);
}

hipError_t launch_amax(int dtype_size, bool is_bf16, const void* x, long n, unsigned* out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (n % 4 != 0) return hipErrorInvalidValue;
    const long blocks = (n / 4 + 255) / 256;
    dim3 grid((unsigned)(blocks < 2048 ? blocks : 2048));
    if (dtype_size == 4)
        hipLaunchKernelGGL(amax_kernel<float>, grid, dim3(256), 0, s, (const float*)x, n, out);
    else if (is_bf16)
        hipLaunchKernelGGL(amax_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)x, n, out);
    else
        hipLaunchKernelGGL(amax_kernel<f16>, grid, dim3(256), 0, s, (const f16*)x, n, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------- V^T padding
// Columns [L, Lp) of the V^T rows are read as whole 64-key tiles by the
// attention kernel's LDS-DMA; they must hold finite values (zeros), since
// a zero softmax weight times a NaN would still be NaN.
__global__ __launch_bounds__(256) void vt_pad_kernel(f16* __restrict__ Vt, long rows, int L, int Lp) {
    const int pad = Lp - L;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * pad) return;
    const long r = i / pad;
    Vt[r * Lp + L + (i - r * pad)] = (f16)0.f;
}

hipError_t launch_vt_pad(void* Vt, long rows, int L, int Lp, hipStream_t s) {
    const long n = rows * (Lp - L);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(vt_pad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (f16*)Vt, rows, L, Lp);
    return hipGetLastError();
}

}  // namespace tfl
