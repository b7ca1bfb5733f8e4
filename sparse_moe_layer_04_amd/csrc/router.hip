// Router projection l = x W_g^T (+ logit_offset) on packed router weights
// ("HyperParallel accelerates DeepSeek-V4.1 ...", section 2.3, MegaGate:
// the projection matmul stays outside the fused gate; "Twinkle x Ascend
// ...", section "FSDP2-4D parallel engine adaptation": the router computes
// logits from the hidden states).
//
// Shape: N = E is small (384) against T (8192) and K = d (4096).  Every
// workgroup streams its tokens' rows of x and its experts' rows of W_g once
// through K, so the traffic between L2 and the CUs is
//   T E K 2 B (1 / tokens per workgroup + 1 / experts per workgroup),
// smallest for a square-ish tile.  Tile: 128 tokens x 96 experts (three
// 32-row weight blocks), T / 128 x ceil(E / 96) workgroups (256 at the
// 384-expert layer): ~0.47 GB of operand reads instead of ~1 GB for
// 32 tokens x all experts.  The workgroups of one token tile run together
// on one XCD (see the order below), so x comes from memory once.
//   - workgroup: 4 waves (one per SIMD); wave w owns tokens 32 w .. 32 w + 31
//     of the tile and all of its (up to) three weight blocks;
//   - per 16-wide K substep: one activation fragment (16 bytes per lane,
//     straight from x) and three weight fragments (1 KB contiguous each in
//     the moe_pack_weights panel layout, shared by the four waves through
//     L1), loaded kRing substeps ahead into a register ring; one
//     v_mfma_f32_32x32x16_bf16 per weight block.
// Each output accumulates its K substeps in ascending order with the same
// instruction and operand order as the plain-layout kernel, so both layouts
// give the same bits.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterPanel = 256;   // panel rows of the packed router weights
constexpr int kRing = 8;            // substeps in flight
constexpr int kBlocks = 3;          // 32-row weight blocks per workgroup
constexpr int kTokens = 128;        // tokens per workgroup (32 per wave)

__global__ __launch_bounds__(256, 1) void router_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ wg,
                                                        const float* __restrict__ offset, int T,
                                                        int K, int E, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    // XCD-aware order: workgroup id mod 8 is its XCD; on each XCD the
    // consecutive workgroups take the expert groups of one token tile, so
    // the tile's rows of x are read from memory once and then hit that
    // XCD's L2 (and every XCD keeps all of W_g in its L2)
    const int NB = (E + 31) / 32;                 // 32-row weight blocks
    const int groups = (NB + kBlocks - 1) / kBlocks;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tile = (slot / groups) * 8 + xcd, group = slot % groups;
    const int t0 = tile * kTokens + wave * 32;
    if (t0 >= T) return;                          // (wave-uniform; no barrier below)
    const int eb0 = group * kBlocks;              // this workgroup's first block
    const int nb = min(kBlocks, NB - eb0);        // its blocks (>= 1)
    const int S = K / 16;                         // 16-wide K substeps

    // activation row of this lane (rows past T read the last row; not stored)
    const uint16_t* arow = x + (size_t)min(t0 + l32, T - 1) * K + 8 * half;
    // weight fragment of block eb, substep ks: panel eb / 8, 64-wide stage
    // ks / 4, block eb % 8, substep ks % 4, 8 elements per lane
    const size_t pstride = (size_t)kRouterPanel * K;
    const uint16_t* wb[kBlocks];
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
        const int eb = min(eb0 + j, NB - 1);
        wb[j] = wg + (size_t)(eb / 8) * pstride + (eb % 8) * 2048 + lane * 8;
    }
    auto w_off = [](int ks) { return (size_t)(ks >> 2) * (8 * 2048) + (ks & 3) * 512; };

    f32x16 acc[kBlocks];
#pragma unroll
    for (int j = 0; j < kBlocks; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    bf16x8 ar[kRing], wr[kRing][kBlocks];
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
        const int ks = min(u, S - 1);
        ar[u] = *(const bf16x8*)(arow + 16 * ks);
#pragma unroll
        for (int j = 0; j < kBlocks; ++j) wr[u][j] = *(const bf16x8*)(wb[j] + w_off(ks));
    }
    // Loads and MFMAs are unconditional (blocks past the last read its
    // rows again; their outputs are not stored): straight-line code lets the
    // compiler count the ring's outstanding loads exactly instead of draining
    // them at every turn.
    const int S8 = S / kRing * kRing;             // whole ring turns; S % 4 == 0
    for (int s0 = 0; s0 < S8; s0 += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
#pragma unroll
            for (int j = 0; j < kBlocks; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[u][j], ar[u], acc[j], 0, 0, 0);
            // refill the slot with substep s0 + u + kRing (the last substep
            // again past the end, so the loads stay in bounds)
            const int ks = min(s0 + u + kRing, S - 1);
            ar[u] = *(const bf16x8*)(arow + 16 * ks);
#pragma unroll
            for (int j = 0; j < kBlocks; ++j) wr[u][j] = *(const bf16x8*)(wb[j] + w_off(ks));
        }
    }
    if (S8 < S) {                                 // last 4 substeps: slots 0 .. 3
#pragma unroll
        for (int u = 0; u < kRing / 2; ++u)
#pragma unroll
            for (int j = 0; j < kBlocks; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[u][j], ar[u], acc[j], 0, 0, 0);
    }

    // acc[j] element 4 qq + i of lane l: token t0 + l % 32, expert
    // 32 (eb0 + j) + 8 qq + 4 (l / 32) + i
    const int t = t0 + l32;
    if (t >= T) return;
    float* out = logits + (size_t)t * E;
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
        if (j >= nb) continue;
        const int e_blk = 32 * (eb0 + j);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int e = e_blk + 8 * qq + 4 * half;
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[j][4 * qq + i];
            if ((E & 3) == 0 && e + 3 < E) {
                if (offset)
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = v[i] + offset[e + i];
                *(f32x4*)(out + e) = v;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (e + i < E) out[e + i] = offset ? v[i] + offset[e + i] : v[i];
            }
        }
    }
}

}  // namespace

bool router_packed_preferred(int T, int E) {
    // each workgroup's time is set by its own load latency chain, so the
    // kernel wins while its grid is at most two rounds over the CUs; larger
    // grids go to the persistent grouped GEMM (same bits either way)
    const long long groups = ((E + 31) / 32 + kBlocks - 1) / kBlocks;
    const long long wgs = ((T + kTokens - 1) / kTokens + 7) / 8 * 8 * groups;
    return wgs <= 2LL * device_cu_count();
}

hipError_t launch_router_packed(const uint16_t* x, const uint16_t* wg_packed, const float* offset,
                                int T, int K, int E, float* logits, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    if (K % 64 || E < 1 || E > MOE_MAX_E) return hipErrorInvalidValue;
    const int groups = ((E + 31) / 32 + kBlocks - 1) / kBlocks;
    const long long tiles8 = ((T + kTokens - 1) / kTokens + 7) / 8 * 8;   // whole XCD rounds
    hipLaunchKernelGGL(router_kernel, dim3((unsigned)(tiles8 * groups)), dim3(256), 0, stream, x,
                       wg_packed, offset, T, K, E, logits);
    return hipGetLastError();
}

}  // namespace moe
