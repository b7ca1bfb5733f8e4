// Backward of the whole layer ("HyperParallel accelerates DeepSeek-V4.1 ...",
// section 2.3: MegaGate's fused backward chain of the gate's normalisation
// gradients and MegaMoE's expert matmuls; section 03: the training run whose
// step this is) and the router projection's gradient kernels.
//
// moe_backward recomputes the forward's intermediates from x (the router
// logits, routes, dispatch permutation, the expert gate/up pre-activations and
// h, the routed expert outputs), as activation recomputation does, then takes
// the output gradient dy back through the layer in reverse order:
//   combine       -> dy_perm = w dy (bf16 for the products), d_topk_w
//   down          -> dW_down = dy_perm^T h,  dH = dy_perm W_down
//   SwiGLU        -> dG, dU (bf16, side by side)
//   gate / up     -> dW_gate = dG^T x_perm, dW_up = dU^T x_perm,
//                    dx_perm = [dG | dU] [W_gate; W_up]
//   dispatch      -> dx = sum over each token's rows of dx_perm (+ shared)
//   routing       -> d_logits (only the k selected entries are non-zero)
//   router        -> dx += d_logits W_g, dW_g = d_logits^T x
//   shared expert -> the same FFN chain on x with dy itself.
// Every product runs on the expert GEMM kernels (packed transposed weights
// for the input gradients) or the grouped weight-gradient kernel.
//
// The router projection's gradients use that d_logits is zero off each
// token's k selected experts:
//   dx[t, :] += sum_j d_logits[t, ids_j] W_g[ids_j, :]    (k rows per token)
//   dW_g[e, :] = sum_{rows r of expert e} d_logits[src_r, e] x[src_r, :]
// in fp32, each sum in a fixed order.
#include "moe_internal.h"

namespace moe {
namespace {

// dx[t, c .. c+3] += sum_j dl[t, ids_j] w_g[ids_j, c .. c+3]: one workgroup
// per token, 4 columns per thread per 1024-column pass, slots in order
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ dl,
                                                        const int32_t* __restrict__ ids,
                                                        const uint16_t* __restrict__ wg, int d,
                                                        int E, int k, float* __restrict__ dx) {
    const int t = blockIdx.x;
    int ej[MOE_MAX_K];
    float sj[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
        ej[j] = -1;
        sj[j] = 0.0f;
        if (j < k) {
            const int e = ids[(size_t)t * k + j];
            if (e >= 0 && e < E) {
                ej[j] = e;
                sj[j] = dl[(size_t)t * E + e];
            }
        }
    }
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        f32x4 acc = *(const f32x4*)(dx + (size_t)t * d + c);
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j) {
            if (ej[j] < 0) continue;
            const u32x2 w = *(const u32x2*)(wg + (size_t)ej[j] * d + c);
            acc[0] = __builtin_fmaf(sj[j], bf16_to_f32((uint16_t)(w[0] & 0xffffu)), acc[0]);
            acc[1] = __builtin_fmaf(sj[j], bf16_to_f32((uint16_t)(w[0] >> 16)), acc[1]);
            acc[2] = __builtin_fmaf(sj[j], bf16_to_f32((uint16_t)(w[1] & 0xffffu)), acc[2]);
            acc[3] = __builtin_fmaf(sj[j], bf16_to_f32((uint16_t)(w[1] >> 16)), acc[3]);
        }
        *(f32x4*)(dx + (size_t)t * d + c) = acc;
    }
}

// dwg[e, c .. c+3] for a 256-column slice: the 4 waves take contiguous
// quarters of the expert's rows (4 columns per lane), then the partial sums
// are added in wave order (the same bits on every run).
__global__ __launch_bounds__(256) void router_dwg_kernel(const float* __restrict__ dl,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ src,
                                                         const uint16_t* __restrict__ x, int d,
                                                         int E, int rows,
                                                         float* __restrict__ dwg) {
    __shared__ f32x4 part[4][64];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.y * 256 + lane * 4;
    const int lo = min(max(offsets[e], 0), rows);
    const int hi = max(lo, min(max(offsets[e + 1], 0), rows));
    const int n = hi - lo;
    const int r0 = lo + (int)((long long)n * wave / 4), r1 = lo + (int)((long long)n * (wave + 1) / 4);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c < d) {
        for (int r = r0; r < r1; ++r) {
            const int t = src[r];
            if (t < 0) continue;
            const float s = dl[(size_t)t * E + e];
            const u32x2 xv = *(const u32x2*)(x + (size_t)t * d + c);
            acc[0] = __builtin_fmaf(s, bf16_to_f32((uint16_t)(xv[0] & 0xffffu)), acc[0]);
            acc[1] = __builtin_fmaf(s, bf16_to_f32((uint16_t)(xv[0] >> 16)), acc[1]);
            acc[2] = __builtin_fmaf(s, bf16_to_f32((uint16_t)(xv[1] & 0xffffu)), acc[2]);
            acc[3] = __builtin_fmaf(s, bf16_to_f32((uint16_t)(xv[1] >> 16)), acc[3]);
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && c < d) {
        f32x4 v = part[0][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += part[w][lane][i];
        *(f32x4*)(dwg + (size_t)e * d + c) = v;
    }
}

}  // namespace

hipError_t launch_router_backward(const float* dl, const int32_t* ids, const int32_t* offsets,
                                  const int32_t* src, const uint16_t* x, const uint16_t* wg,
                                  int T, int d, int E, int k, float* dx, float* dwg,
                                  hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    if (d % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(router_dx_kernel, dim3(T), dim3(256), 0, stream, dl, ids, wg, d, E, k, dx);
    hipLaunchKernelGGL(router_dwg_kernel, dim3(E, (d + 255) / 256), dim3(256), 0, stream, dl,
                       offsets, src, x, d, E, T * k, dwg);
    return hipGetLastError();
}

}  // namespace moe
