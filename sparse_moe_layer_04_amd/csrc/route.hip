// Wavefront router: one 64-lane wave per token (top-k), 64/k tokens per wave
// (hash).
//
// MegaGate order ("HyperParallel accelerates DeepSeek-V4.1 ...", section 2.3):
// score -> bias ranking -> Top-K -> score extraction -> normalise -> scale,
// with separate text / vision bias rows; HashRouter variant ("Twinkle x
// Ascend ...", section "FSDP2-4D parallel engine adaptation"): ids from
// tid2eid[input_ids], weights still from the gate logits.
//
// Each lane owns experts e = lane + 64 i.  The ranking key of an expert is
// the order-preserving 32-bit image of its biased score; top-k is k rounds
// of a wave-wide maximum (DPP row operations, then a lane read) over the
// lanes' largest keys, ties between lanes going to the lowest expert index
// (see route_topk_kernel).  This translation unit is built with FP
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
    x = __builtin_fminf(__builtin_fmaxf(x, -80.0f), 80.0f);  // maxNum: NaN -> -80
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

// Order-preserving unsigned image of a binary32 value (finite, no -0):
// negative values have every bit flipped, the others the sign bit set.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// One DPP move; lanes the pattern leaves unwritten get `fill`.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t fill, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, ROWMASK, 0xf, false);
}

// Wave-wide maximum (MIN = false) or minimum of v, wave-uniform.  DPP row
// operations only: quad xor 1 and xor 2, half-row and row mirrors leave every
// lane with its 16-lane row's extreme; row broadcasts of lanes 15 and 31
// carry the row extremes up, so lane 63 ends with the wave's, which a lane
// read makes uniform.  Lanes a broadcast does not write see the identity of
// the operation (0 for the maximum, all ones for the minimum).
template <bool MIN>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
#define MOE_STEP(CTRL, RM)                                   \
    {                                                        \
        const uint32_t o = dpp_u32<CTRL, RM>(MIN ? ~0u : 0u, v); \
        v = MIN ? (o < v ? o : v) : (o > v ? o : v);         \
    }
    MOE_STEP(0xB1, 0xf)    // quad_perm [1,0,3,2]
    MOE_STEP(0x4E, 0xf)    // quad_perm [2,3,0,1]
    MOE_STEP(0x141, 0xf)   // row_half_mirror
    MOE_STEP(0x140, 0xf)   // row_mirror
    MOE_STEP(0x142, 0xa)   // row_bcast:15 into rows 1 and 3
    MOE_STEP(0x143, 0xc)   // row_bcast:31 into rows 2 and 3
#undef MOE_STEP
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// value of lane `src` (wave-uniform) in every lane
__device__ __forceinline__ float lane_read(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Top-k by (biased score descending, expert index ascending).  Lane l holds
// experts e = l + 64 i (i < NPL) as 32-bit keys (the order-preserving image
// of r; 0 for e >= E, below every real value) with their unbiased scores.
// Round j: m = the wave's largest key (each lane's largest, then a DPP wave
// maximum).  Usually one lane holds m: its keys and scores are read into
// scalar registers and the first i with key m (the lowest expert of that
// lane among equal keys) is the winner.  When several lanes hold m the
// smallest index e among them wins (a wave minimum over each such lane's
// lowest e with key m).  The winner's key is then cleared in its lane.
// All loads of a token (its logits, then the bias row that its modality
// picks) are issued before any score is computed.
template <int NPL>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const uint8_t* __restrict__ modality, int T, int E, int k, int n_bias, float scale,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= T) return;
    const float* lt = logits + (size_t)t * E;
    float lv[NPL], bv[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) lv[i] = lt[min(lane + 64 * i, E - 1)];
    if (bias && n_bias > 1 && modality) {
        // both bias rows are loaded beside the modality byte, so the row
        // choice waits for no second round trip
        float b1[NPL];
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            bv[i] = bias[min(lane + 64 * i, E - 1)];
            b1[i] = bias[E + min(lane + 64 * i, E - 1)];
        }
        if (modality[t]) {
#pragma unroll
            for (int i = 0; i < NPL; ++i) bv[i] = b1[i];
        }
    } else if (bias) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) bv[i] = bias[min(lane + 64 * i, E - 1)];
    } else {
#pragma unroll
        for (int i = 0; i < NPL; ++i) bv[i] = 0.0f;
    }
    uint32_t key[NPL];
    float sc[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const float s = score_fn(lv[i]);
        const float r = (s + bv[i]) + 0.0f;  // (s > 0: adding a zero bias is exact; -0 -> +0)
        sc[i] = s;
        key[i] = lane + 64 * i < E ? ordered_bits(r) : 0u;
    }
    float g_mine = 0.0f;  // lane j < k keeps g_j
    int id_mine = -1;
    for (int j = 0; j < k; ++j) {
        uint32_t lm = key[0];
#pragma unroll
        for (int i = 1; i < NPL; ++i) lm = key[i] > lm ? key[i] : lm;
        const uint32_t m = wave_reduce_u32<false>(lm);
        const uint64_t holders = __builtin_amdgcn_ballot_w64(lm == m);
        int w, wi = 0, sbits = 0;  // winner lane, its slot, its score's bits
        if (__popcll(holders) == 1) {
            w = __builtin_ctzll(holders);
#pragma unroll
            for (int i = NPL - 1; i >= 0; --i) {
                const uint32_t kv = (uint32_t)__builtin_amdgcn_readlane((int)key[i], w);
                const int sv = __builtin_amdgcn_readlane(__float_as_int(sc[i]), w);
                if (kv == m) {
                    wi = i;
                    sbits = sv;
                }
            }
        } else {
            uint32_t fe = 0xffffffffu;
#pragma unroll
            for (int i = NPL - 1; i >= 0; --i)
                if (key[i] == m) fe = (uint32_t)(lane + 64 * i);
            const uint32_t e = wave_reduce_u32<true>(fe);
            w = (int)(e & 63);
            wi = (int)(e >> 6);
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (i == wi) sbits = __builtin_amdgcn_readlane(__float_as_int(sc[i]), w);
        }
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (i == wi) key[i] = lane == w ? 0u : key[i];
        if (lane == j) {
            g_mine = __int_as_float(sbits);
            id_mine = w + 64 * wi;
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

// Hash routing packs P = 64 / k tokens into a wave: lane l < P k holds slot
// j = l % k of token t = P w + l / k, so the three dependent loads (input
// id, table entry, logit) of every slot are in flight at once.  A token
// whose input id is outside [0, V), or any of whose k table entries is
// outside [0, E), gets ids -1 and weights 0 (ballots over the token's lanes).
__global__ __launch_bounds__(256) void route_hash_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ input_ids,
    const int32_t* __restrict__ tid2eid, int T, int E, int k, int V, float scale,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, uint32_t* __restrict__ flags) {
    const int lane = threadIdx.x & 63;
    const int P = 64 / k;
    const int q = lane / k, j = lane - q * k;
    const int t = (blockIdx.x * 4 + (threadIdx.x >> 6)) * P + q;
    const bool live = q < P && t < T;
    int tok = -1, id = -1;
    if (live) tok = input_ids[t];
    const bool tok_ok = live && tok >= 0 && tok < V;
    if (tok_ok) id = tid2eid[(size_t)tok * k + j];
    const uint64_t seg = ((1ull << k) - 1) << (q * k);  // this token's lanes
    const uint64_t bad_id = __builtin_amdgcn_ballot_w64(tok_ok && (id < 0 || id >= E));
    const bool ok = tok_ok && (bad_id & seg) == 0;
    float g = 0.0f;
    if (ok) g = score_fn(logits[(size_t)t * E + id]);
    // left-to-right fp32 sum of the token's k scores
    const int base = q * k;
    float sum = __shfl(g, base, 64);
    for (int jj = 1; jj < k; ++jj) sum = sum + __shfl(g, base + jj, 64);
    if (live) {
        ids_out[(size_t)t * k + j] = ok ? id : -1;
        w_out[(size_t)t * k + j] = ok ? (g / sum) * scale : 0.0f;
    }
    const bool bad_tok = __builtin_amdgcn_ballot_w64(live && !tok_ok) != 0;
    if (lane == 0 && flags && (bad_tok || bad_id))
        atomicOr(flags, (bad_tok ? MOE_FLAG_BAD_INPUT_ID : 0u) |
                            (bad_id ? MOE_FLAG_BAD_EXPERT_ID : 0u));
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
        const int per_wave = 64 / k;
        const int waves = (T + per_wave - 1) / per_wave;
        hipLaunchKernelGGL(route_hash_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, logits,
                           input_ids, tid2eid, T, E, k, V, scale, ids, w, flags);
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
