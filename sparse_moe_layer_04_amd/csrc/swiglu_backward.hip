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
            const float gv = g[c], uv = u[c];
            const bool g_in = mode == MOE_CLAMP_SYMMETRIC ? (gv >= -L && gv <= L) : (gv <= L);
            const bool u_in = uv >= -L && uv <= L;
            float gc = fminf(gv, L);
            if (mode == MOE_CLAMP_SYMMETRIC) gc = fmaxf(gc, -L);
            const float uc = fminf(fmaxf(uv, -L), L);
            const float s = 1.0f / (1.0f + __expf(-gc));
            ou[c] = u_in ? h[c] * (gc * s) : 0.0f;
            og[c] = g_in ? h[c] * uc * (s * (1.0f + gc * (1.0f - s))) : 0.0f;
        }
        *((f32x4*)dgate + i) = og;
        *((f32x4*)dup + i) = ou;
    }
}

}  // namespace

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
