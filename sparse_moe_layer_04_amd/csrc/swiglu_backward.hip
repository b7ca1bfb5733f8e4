// Backward of the clamped SwiGLU between the expert matmuls ("HyperParallel
// accelerates DeepSeek-V4.1 ...", section 2.3, MegaMoE: SwiGLU with the V4.1
// clamp).  For h = silu(cg(G)) * cu(U) (the clamps of the forward epilogue)
// and a gradient dh of h:
//   dU = dh * silu(cg(G)) * [U inside [-L, L]],
//   dG = dh * cu(U) * silu'(cg(G)) * [G inside the gate clamp's range],
//   silu'(z) = s (1 + z (1 - s)),  s = 1 / (1 + e^-z);
// a clamp passes its gradient on the closed range.  Elementwise and
// HBM-bound (20 bytes per element): a grid-stride loop over 16-byte groups
// with non-temporal loads, since every input is read once.
#include "moe_internal.h"

namespace moe {
namespace {

// dG and dU of one element (the definition above, fp32)
__device__ __forceinline__ void swiglu_grad(float gv, float uv, float hv, float L, int mode,
                                            float& og, float& ou) {
    const bool g_in = mode == MOE_CLAMP_SYMMETRIC ? (gv >= -L && gv <= L) : (gv <= L);
    const bool u_in = uv >= -L && uv <= L;
    float gc = fminf(gv, L);
    if (mode == MOE_CLAMP_SYMMETRIC) gc = fmaxf(gc, -L);
    const float uc = fminf(fmaxf(uv, -L), L);
    const float s = 1.0f / (1.0f + __expf(-gc));
    ou = u_in ? hv * (gc * s) : 0.0f;
    og = g_in ? hv * uc * (s * (1.0f + gc * (1.0f - s))) : 0.0f;
}

__global__ __launch_bounds__(256) void swiglu_backward_kernel(
    const float* __restrict__ gate, const float* __restrict__ up, const float* __restrict__ dh,
    long long n4, float L, int mode, float* __restrict__ dgate, float* __restrict__ dup) {
    const long long stride = (long long)gridDim.x * 256;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const f32x4 g = __builtin_nontemporal_load((const f32x4*)gate + i);
        const f32x4 u = __builtin_nontemporal_load((const f32x4*)up + i);
        const f32x4 h = __builtin_nontemporal_load((const f32x4*)dh + i);
        f32x4 og, ou;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float a, b;
            swiglu_grad(g[c], u[c], h[c], L, mode, a, b);
            og[c] = a;
            ou[c] = b;
        }
        *((f32x4*)dgate + i) = og;
        *((f32x4*)dup + i) = ou;
    }
}

// rows x F elements (F a multiple of 4); dG and dU rounded to bf16 into
// row r of dgu: [dG (F values) | dU (F values)]
__global__ __launch_bounds__(256) void swiglu_backward_bf16_kernel(
    const float* __restrict__ gate, const float* __restrict__ up, const float* __restrict__ dh,
    long long n4, int F4, float L, int mode, uint16_t* __restrict__ dgu) {
    const long long stride = (long long)gridDim.x * 256;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const f32x4 g = __builtin_nontemporal_load((const f32x4*)gate + i);
        const f32x4 u = __builtin_nontemporal_load((const f32x4*)up + i);
        const f32x4 h = __builtin_nontemporal_load((const f32x4*)dh + i);
        f32x4 og, ou;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float a, b;
            swiglu_grad(g[c], u[c], h[c], L, mode, a, b);
            og[c] = a;
            ou[c] = b;
        }
        const long long r = i / F4, c4 = i % F4;
        uint16_t* row = dgu + (size_t)r * (8 * (size_t)F4);
        *(u32x2*)(row + 4 * c4) =
            u32x2{(uint32_t)f32_to_bf16(og[0]) | ((uint32_t)f32_to_bf16(og[1]) << 16),
                  (uint32_t)f32_to_bf16(og[2]) | ((uint32_t)f32_to_bf16(og[3]) << 16)};
        *(u32x2*)(row + 4 * F4 + 4 * c4) =
            u32x2{(uint32_t)f32_to_bf16(ou[0]) | ((uint32_t)f32_to_bf16(ou[1]) << 16),
                  (uint32_t)f32_to_bf16(ou[2]) | ((uint32_t)f32_to_bf16(ou[3]) << 16)};
    }
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ src,
                                                        long long n, uint16_t* __restrict__ dst) {
    const long long stride = (long long)gridDim.x * 256;
    const long long n4 = n / 4;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const f32x4 v = __builtin_nontemporal_load((const f32x4*)src + i);
        *(u32x2*)(dst + 4 * i) =
            u32x2{(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                  (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
    }
    // the n % 4 tail
    const long long i = 4 * n4 + (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = f32_to_bf16(src[i]);
}

}  // namespace

hipError_t launch_swiglu_backward_bf16(const float* gate, const float* up, const float* dh,
                                       long long rows, int F, float clamp_limit, int clamp_mode,
                                       uint16_t* dgu, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (F % 4) return hipErrorInvalidValue;
    const long long n4 = rows * F / 4;
    const long long blocks = (n4 + 255) / 256;
    const long long cap = 8LL * device_cu_count();
    hipLaunchKernelGGL(swiglu_backward_bf16_kernel, dim3((unsigned)(blocks < cap ? blocks : cap)),
                       dim3(256), 0, stream, gate, up, dh, n4, F / 4, clamp_limit, clamp_mode,
                       dgu);
    return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* src, long long n, uint16_t* dst, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const long long blocks = (n / 4 + 255) / 256 + 1;
    const long long cap = 8LL * device_cu_count();
    hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(256),
                       0, stream, src, n, dst);
    return hipGetLastError();
}

hipError_t launch_swiglu_backward(const float* gate, const float* up, const float* dh,
                                  long long n, float clamp_limit, int clamp_mode, float* dgate,
                                  float* dup, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const long long n4 = n / 4;
    const long long blocks = (n4 + 255) / 256;
    const long long cap = 8LL * device_cu_count();          // 8 workgroups per CU
    hipLaunchKernelGGL(swiglu_backward_kernel, dim3((unsigned)(blocks < cap ? blocks : cap)),
                       dim3(256), 0, stream, gate, up, dh, n4, clamp_limit, clamp_mode, dgate,
                       dup);
    return hipGetLastError();
}

}  // namespace moe
