// Wavefront router: one 64-lane wave per token.
//
// MegaGate order ("HyperParallel accelerates DeepSeek-V4.1 ...", section 2.3):
// score -> bias ranking -> Top-K -> score extraction -> normalise -> scale,
// with separate text / vision bias rows; HashRouter variant ("Twinkle x
// Ascend ...", section "FSDP2-4D parallel engine adaptation"): ids from
// tid2eid[input_ids], weights still from the gate logits.
//
// Each lane owns experts e = lane + 64 i.  The ranking key of an expert packs
// the order-preserving image of its biased score (high 32 bits) with ~e (low
// 32 bits), so one unsigned 64-bit max picks (score desc, index asc).  Top-k
// is k rounds of a wave-wide max (DPP row operations, then a lane read) over
// the lanes' current best keys.  This translation unit is built with FP
// contraction off: the score function is a fixed sequence of IEEE binary32
// operations.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxPerLane = MOE_MAX_E / 64;

// Binary32 sigmoid as a fixed operation sequence (see moe.h): clamp to
// [-80, 80] (NaN -> -80); z = -x; n = rint(z * log2 e); Cody-Waite
// r = (z - n*C1) - n*C2 by two fmas with C1 = 0x1.62e4p-1 (exact n*C1) and
// C2 = fl32(ln2 - C1); exp(r) by the degree-7 Taylor polynomial (Horner, fma)
// with binary32 coefficients 1/j!; e = p * 2^n; S = 1 / (1 + e), correctly
// rounded division.
__device__ __forceinline__ float score_fn(float x) {
    if (x != x) x = -80.0f;
    if (x < -80.0f) x = -80.0f;
    if (x > 80.0f) x = 80.0f;
    const float log2e = 0x1.715476p+0f;
    const float c1 = 0x1.62e4p-1f;
    const float c2 = 0x1.7f7d1cp-20f;
    float z = -x;
    float t = z * log2e;
    float n = __builtin_rintf(t);
    float r = __builtin_fmaf(-n, c1, z);
    r = __builtin_fmaf(-n, c2, r);
    float p = 0x1.a01a02p-13f;              // 1/5040
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/720
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/120
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/24
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/6
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    float e = __builtin_ldexpf(p, (int)n);
    float den = 1.0f + e;
    return 1.0f / den;
}

// Order-preserving unsigned image of a binary32 value (finite, no -0).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One DPP move of a 64-bit value (both halves through the same lane
// pattern); lanes the pattern leaves unwritten keep v.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROWMASK, 0xf, false);
    const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROWMASK, 0xf, false);
    return ((uint64_t)h2 << 32) | l2;
}

template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
    const uint64_t o = dpp_u64<CTRL, ROWMASK>(v);
    return o > v ? o : v;
}

// Wave-wide maximum of a 64-bit key, returned in every lane (wave-uniform).
// DPP row operations only (no LDS crossbar): quad xor 1 and xor 2, half-row
// and row mirrors leave every lane with its 16-lane row maximum; row
// broadcasts of lanes 15 and 31 carry the row maxima up, so lane 63 ends
// with the wave maximum, which a lane read makes uniform.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_step<0xB1>(v);         // quad_perm [1,0,3,2]
    v = dpp_max_step<0x4E>(v);         // quad_perm [2,3,0,1]
    v = dpp_max_step<0x141>(v);        // row_half_mirror
    v = dpp_max_step<0x140>(v);        // row_mirror
    v = dpp_max_step<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_max_step<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// value of lane `src` (wave-uniform) in every lane
__device__ __forceinline__ float lane_read(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

template <int NPL>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const uint8_t* __restrict__ modality, int T, int E, int k, int n_bias, float scale,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* lt = logits + (size_t)t * E;
    const float* b = nullptr;
    if (bias) {
        int row = (n_bias > 1 && modality && modality[t]) ? 1 : 0;
        b = bias + (size_t)row * E;
    }
    uint64_t keys[NPL];
    float sc[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        int e = lane + 64 * i;
        if (e < E) {
            float s = score_fn(lt[e]);
            float r = b ? s + b[e] : s;
            r = r + 0.0f;  // -0 -> +0
            sc[i] = s;
            keys[i] = ((uint64_t)ordered_bits(r) << 32) | (uint32_t)(~(uint32_t)e);
        } else {
            sc[i] = 0.0f;
            keys[i] = 0;
        }
    }
    float g_mine = 0.0f;  // lane j < k keeps g_j
    int id_mine = -1;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
        float best_s = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            if (keys[i] > best) {
                best = keys[i];
                best_s = sc[i];
            }
        }
        uint64_t win = wave_max_u64(best);
        int e = (int)(~(uint32_t)win);
        const float s = lane_read(best_s, e & 63);
        // owner retires the winner
        if ((e & 63) == lane) {
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (lane + 64 * i == e) keys[i] = 0;
        }
        if (lane == j) {
            g_mine = s;
            id_mine = e;
        }
    }
    // left-to-right fp32 sum of the k gathered (unbiased) scores
    float sum = lane_read(g_mine, 0);
    for (int j = 1; j < k; ++j) sum = sum + lane_read(g_mine, j);
    if (lane < k) {
        float q = g_mine / sum;
        ids_out[(size_t)t * k + lane] = id_mine;
        w_out[(size_t)t * k + lane] = q * scale;
    }
}

__global__ __launch_bounds__(256) void route_hash_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ input_ids,
    const int32_t* __restrict__ tid2eid, int T, int E, int k, int V, float scale,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, uint32_t* __restrict__ flags) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int tok = input_ids[t];
    uint32_t bad = 0;
    int id = -1;
    if (tok < 0 || tok >= V) {
        bad = MOE_FLAG_BAD_INPUT_ID;
    } else {
        if (lane < k) id = tid2eid[(size_t)tok * k + lane];
        bool oob = lane < k && (id < 0 || id >= E);
        if (__any(oob)) bad = MOE_FLAG_BAD_EXPERT_ID;
    }
    if (bad) {
        if (lane == 0 && flags) atomicOr(flags, bad);
        if (lane < k) {
            ids_out[(size_t)t * k + lane] = -1;
            w_out[(size_t)t * k + lane] = 0.0f;
        }
        return;
    }
    float g = 0.0f;
    if (lane < k) g = score_fn(logits[(size_t)t * E + id]);
    float sum = lane_read(g, 0);
    for (int j = 1; j < k; ++j) sum = sum + lane_read(g, j);
    if (lane < k) {
        float q = g / sum;
        ids_out[(size_t)t * k + lane] = id;
        w_out[(size_t)t * k + lane] = q * scale;
    }
}

// Routing backward ("HyperParallel accelerates DeepSeek-V4.1 ...", section
// 2.3, MegaGate: the gradient chain of the gate's normalisation and scaling):
// given dw[t, j] = dLoss/dw_j for the routing weights
//   w_j = scale * g_j / G,  g_j = S(l[t, ids_j]),  G = sum_j g_j,
// the logits' gradient is
//   dl[t, ids_i] = (scale / G) * (dw_i - sum_j dw_j g_j / G) * g_i (1 - g_i)
// and 0 for the E - k experts the token did not select (the choice is
// piecewise constant in the logits; the ranking bias takes no part in w).
// The bracket is evaluated as sum_j g_j (dw_i - dw_j) / G (equal, since
// sum_j g_j = G): no cancellation between dw_i and the weighted mean, and
// exactly 0 when k = 1 or all dw are equal, as the weights are then
// constant.  One wave per token: lane j < k holds slot j; G and the bracket
// are summed in slot order in fp32; then every lane writes its entries
// e = lane + 64 i of the row (each entry written once; an expert listed in
// two slots gets the sum).  A token with an id outside [0, E) gets a zero
// row and sets MOE_FLAG_BAD_EXPERT_ID.
__global__ __launch_bounds__(256) void route_backward_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ids,
    const float* __restrict__ dw, int T, int E, int k, float scale, float* __restrict__ dl,
    uint32_t* __restrict__ flags) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;                          // (wave-uniform)
    int id = -1;
    float dwj = 0.0f;
    if (lane < k) {
        id = ids[(size_t)t * k + lane];
        dwj = dw[(size_t)t * k + lane];
    }
    const bool bad = __builtin_amdgcn_ballot_w64(lane < k && (id < 0 || id >= E)) != 0;
    float* out = dl + (size_t)t * E;
    if (bad) {
        for (int e = lane; e < E; e += 64) out[e] = 0.0f;
        if (lane == 0 && flags) atomicOr(flags, MOE_FLAG_BAD_EXPERT_ID);
        return;
    }
    const float g = lane < k ? score_fn(logits[(size_t)t * E + id]) : 0.0f;
    float G = lane_read(g, 0);
    float br = lane_read(g, 0) * (dwj - lane_read(dwj, 0));
    for (int j = 1; j < k; ++j) {
        G = G + lane_read(g, j);
        br = br + lane_read(g, j) * (dwj - lane_read(dwj, j));
    }
    float dlj = 0.0f;
    if (lane < k) {
        const float dg = scale / G * (br / G);
        dlj = dg * (g * (1.0f - g));
    }
    // the k (id, gradient) pairs, wave-uniform, read once for the whole row
    int sid[MOE_MAX_K];
    float sdl[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
        sid[j] = j < k ? __builtin_amdgcn_readlane(id, j) : -1;
        sdl[j] = j < k ? lane_read(dlj, j) : 0.0f;
    }
    for (int e = lane; e < E; e += 64) {
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j)
            if (sid[j] == e) v = v + sdl[j];
        out[e] = v;
    }
}

template <int NPL>
void launch_topk(dim3 grid, const float* logits, const float* bias, const uint8_t* modality,
                 int T, int E, int k, int n_bias, float scale, int32_t* ids, float* w,
                 hipStream_t stream) {
    hipLaunchKernelGGL(route_topk_kernel<NPL>, grid, dim3(256), 0, stream, logits, bias,
                       modality, T, E, k, n_bias, scale, ids, w);
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, const uint8_t* modality,
                        const int32_t* input_ids, const int32_t* tid2eid, int T, int E, int k,
                        int n_bias, int V, int mode, float scale, int32_t* ids, float* w,
                        uint32_t* flags, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    if (mode == MOE_MODE_HASH) {
        hipLaunchKernelGGL(route_hash_kernel, grid, dim3(256), 0, stream, logits, input_ids,
                           tid2eid, T, E, k, V, scale, ids, w, flags);
        return hipGetLastError();
    }
    int npl = (E + 63) / 64;
    if (npl <= 1)
        launch_topk<1>(grid, logits, bias, modality, T, E, k, n_bias, scale, ids, w, stream);
    else if (npl <= 2)
        launch_topk<2>(grid, logits, bias, modality, T, E, k, n_bias, scale, ids, w, stream);
    else if (npl <= 4)
        launch_topk<4>(grid, logits, bias, modality, T, E, k, n_bias, scale, ids, w, stream);
    else if (npl <= 6)
        launch_topk<6>(grid, logits, bias, modality, T, E, k, n_bias, scale, ids, w, stream);
    else if (npl <= 8)
        launch_topk<8>(grid, logits, bias, modality, T, E, k, n_bias, scale, ids, w, stream);
    else
        launch_topk<kMaxPerLane>(grid, logits, bias, modality, T, E, k, n_bias, scale, ids, w,
                                 stream);
    return hipGetLastError();
}

hipError_t launch_route_backward(const float* logits, const int32_t* ids, const float* dw,
                                 int T, int E, int k, float scale, float* dl, uint32_t* flags,
                                 hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(route_backward_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits,
                       ids, dw, T, E, k, scale, dl, flags);
    return hipGetLastError();
}

}  // namespace moe
