// Residual LayerNorm and input staging.
//
// LayerNorm is the textbook two-pass one: mean first, then the biased
// variance of the centred values, both in fp32, eps added in fp32, then the
// affine map (the post-LN layer of the PyTorch reference the pages were
// gated against: "Hyper-optimized megakernel-hybrid transformer inference",
// "Challenges").  A row is spread over a group of lanes of one wave
// (up to 64) that read it as coalesced float4 chunks; the reductions are
// butterfly shuffles inside the group.  The row then leaves as fp32 (the
// residual stream), as an operand-dtype copy for the next GEMM, and/or, in
// the last layer, as the I/O dtype output.
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

template <class OpT, class PT, int LPR, int NC>
__global__ __launch_bounds__(256) void ln_kernel(const float* __restrict__ Z, const PT* __restrict__ gamma,
                                                 const PT* __restrict__ beta, float eps, int T, int d,
                                                 float* __restrict__ Xo, OpT* __restrict__ Ao,
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
        if (Ao) st4(Ao + row * d + col, o);
        if (Y) st4(Y + row * d + col, o);
    }
}

template <class OpT, class PT, int LPR>
static hipError_t ln_nc(int nc, const float* Z, const void* g, const void* b, float eps, int T, int d,
                        float* Xo, void* Ao, void* Y, hipStream_t s) {
    constexpr int RPB = 256 / LPR;
    dim3 grid((T + RPB - 1) / RPB);
#define TFL_LN_CASE(NC)                                                                          \
    case NC:                                                                                     \
        hipLaunchKernelGGL((ln_kernel<OpT, PT, LPR, NC>), grid, dim3(256), 0, s, Z, (const PT*)g, \
                           (const PT*)b, eps, T, d, Xo, (OpT*)Ao, (PT*)Y);                        \
        break;
    switch (nc) {
        TFL_LN_CASE(1) TFL_LN_CASE(2) TFL_LN_CASE(3) TFL_LN_CASE(4)
        TFL_LN_CASE(5) TFL_LN_CASE(6) TFL_LN_CASE(7) TFL_LN_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef TFL_LN_CASE
    return hipGetLastError();
}

template <class OpT, class PT>
static hipError_t ln_mode(const float* Z, const void* g, const void* b, float eps, int T, int d, float* Xo,
                          void* Ao, void* Y, hipStream_t s) {
    int lpr, nc;
    if (!ln_shape(d, &lpr, &nc)) return hipErrorInvalidValue;
    switch (lpr) {
        case 1: return ln_nc<OpT, PT, 1>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 2: return ln_nc<OpT, PT, 2>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 4: return ln_nc<OpT, PT, 4>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 8: return ln_nc<OpT, PT, 8>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 16: return ln_nc<OpT, PT, 16>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 32: return ln_nc<OpT, PT, 32>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case 64: return ln_nc<OpT, PT, 64>(nc, Z, g, b, eps, T, d, Xo, Ao, Y, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_ln(Mode m, const float* Z, const void* g, const void* b, float eps, int T, int d, float* Xo,
                     void* Ao, void* Y, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    switch (m) {
        case MODE_F32: return ln_mode<float, float>(Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case MODE_F16: return ln_mode<f16, f16>(Z, g, b, eps, T, d, Xo, Ao, Y, s);
        case MODE_BF16: return ln_mode<f16, bf16>(Z, g, b, eps, T, d, Xo, Ao, Y, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- input staging
// x (I/O dtype) -> fp32 residual stream and operand-dtype copy.
template <class OpT, class XT>
__global__ __launch_bounds__(256) void prep_kernel(const XT* __restrict__ x, float* __restrict__ Xr,
                                                   OpT* __restrict__ A, long n) {
    const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;  // n is a multiple of 4 (d % 4 == 0)
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const float v = to_f32(x[i + e]);
        Xr[i + e] = v;
        A[i + e] = from_f32<OpT>(v);
    }
}

hipError_t launch_prep(Mode m, const void* x, float* Xr, void* A, long n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    dim3 grid((unsigned)((n / 4 + 255) / 256));
    switch (m) {
        case MODE_F32:
            hipLaunchKernelGGL((prep_kernel<float, float>), grid, dim3(256), 0, s, (const float*)x, Xr, (float*)A, n);
            break;
        case MODE_F16:
            hipLaunchKernelGGL((prep_kernel<f16, f16>), grid, dim3(256), 0, s, (const f16*)x, Xr, (f16*)A, n);
            break;
        case MODE_BF16:
            hipLaunchKernelGGL((prep_kernel<f16, bf16>), grid, dim3(256), 0, s, (const bf16*)x, Xr, (f16*)A, n);
            break;
        default: return hipErrorInvalidValue;
    }
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
