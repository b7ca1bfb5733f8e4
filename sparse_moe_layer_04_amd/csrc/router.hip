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
// 32 tokens x all experts.  Where that grid would not cover the CUs (few
// tokens or experts), a workgroup takes 2 or 1 weight blocks instead: more,
// shorter workgroups.  The workgroups of one token tile run together on one
// XCD (see the order below), so x comes from memory once.
//   - workgroup: 4 waves (one per SIMD); wave w owns tokens 32 w .. 32 w + 31
//     of the tile and all of its (up to) three weight blocks;
//   - per 16-wide K substep: one activation fragment and three weight
//     fragments (1 KB contiguous each in the moe_pack_weights panel layout,
//     shared by the four waves through L1, loaded kRing substeps ahead into
//     a register ring); one v_mfma_f32_32x32x16_bf16 per weight block;
//   - the activation fragments (lane l: row l % 32, 8 consecutive K) would
//     touch 32 cache lines per load instruction straight from x, and the L1
//     lookups of those loads bounded the kernel; instead each wave loads its
//     32 rows 64 columns at a time (8 lanes per 128-byte row segment, so 8
//     lines per instruction), two stages ahead, into a private 2-slot LDS
//     ring (XOR-swizzled 16-byte chunks), and reads the fragments from
//     there.  The wave's LDS is its own, so its in-order LDS accesses need
//     no barrier.
// Each output accumulates its K substeps in ascending order with the same
// instruction and operand order as the plain-layout kernel, so both layouts
// give the same bits.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterPanel = 256;   // panel rows of the packed router weights
constexpr int kRing = 8;            // substeps in flight
constexpr int kTokens = 128;        // tokens per workgroup (32 per wave)
constexpr int kXSlot = 32 * 128;    // LDS bytes per wave per 64-column stage of x

// KB: 32-row weight blocks per workgroup (3, or fewer when the grid would
// not cover the CUs)
template <int KB>
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
    const int groups = (NB + KB - 1) / KB;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tile = (slot / groups) * 8 + xcd, group = slot % groups;
    const int t0 = tile * kTokens + wave * 32;
    if (t0 >= T) return;                          // (wave-uniform; no barrier below)
    const int eb0 = group * KB;              // this workgroup's first block
    const int nb = min(KB, NB - eb0);        // its blocks (>= 1)
    const int S = K / 16;                         // 16-wide K substeps

    __shared__ __align__(16) unsigned char xs_all[4 * 2 * kXSlot];
    unsigned char* xs = xs_all + wave * 2 * kXSlot;
    // x staging: lane l copies 16-byte chunk l % 8 of rows l / 8 + 8 i
    // (i < 4) of the wave's 32 rows (rows past T read the last row; their
    // outputs are not stored); chunk c of row r sits at c ^ ((r >> 1) & 7)
    const int xc = lane & 7;
    const uint16_t* xrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xrow[i] = x + (size_t)min(t0 + (lane >> 3) + 8 * i, T - 1) * K + 8 * xc;
    const int NS = S / 4;                         // 64-wide stages
    u32x4 xr[2][4];
    auto load_x = [&](int st, u32x4 (&d)[4]) {
        const int sc = min(st, NS - 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = *(const u32x4*)(xrow[i] + 64 * sc);
    };
    auto store_x = [&](int slot, const u32x4 (&d)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (lane >> 3) + 8 * i;
            *(u32x4*)(xs + slot * kXSlot + r * 128 + ((xc ^ ((r >> 1) & 7)) << 4)) = d[i];
        }
    };
    // the activation fragment of substep ks (stage ks / 4 in slot (ks / 4) % 2):
    // row l32, K chunk 2 (ks % 4) + half of the stage
    auto read_a = [&](int ks) {
        const int c = 2 * (ks & 3) + half;
        return *(const bf16x8*)(xs + ((ks >> 2) & 1) * kXSlot + l32 * 128 +
                                ((c ^ ((l32 >> 1) & 7)) << 4));
    };
    // weight fragment of block eb, substep ks: panel eb / 8, 64-wide stage
    // ks / 4, block eb % 8, substep ks % 4, 8 elements per lane
    const size_t pstride = (size_t)kRouterPanel * K;
    const uint16_t* wb[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        const int eb = min(eb0 + j, NB - 1);
        wb[j] = wg + (size_t)(eb / 8) * pstride + (eb % 8) * 2048 + lane * 8;
    }
    auto w_off = [](int ks) { return (size_t)(ks >> 2) * (8 * 2048) + (ks & 3) * 512; };

    f32x16 acc[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    bf16x8 wr[kRing][KB];
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
        const int ks = min(u, S - 1);
#pragma unroll
        for (int j = 0; j < KB; ++j) wr[u][j] = *(const bf16x8*)(wb[j] + w_off(ks));
    }
    // x stages 0 and 1 into registers, stage 0 into slot 0, stage 2 into the
    // freed registers
    load_x(0, xr[0]);
    load_x(1, xr[1]);
    store_x(0, xr[0]);
    load_x(2, xr[0]);
    // Loads and MFMAs are unconditional (blocks past the last read its
    // rows again, stages past the end the last stage; those outputs are not
    // used): straight-line code lets the compiler count the outstanding
    // loads exactly instead of draining them at every turn.
    // stage st (4 substeps) from slot st % 2; then stage st + 1 goes from its
    // registers into the other slot and those registers take stage st + 3
    auto stage = [&](int st, auto par) {
        constexpr int P = decltype(par)::value;   // st % 2
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
            const int u = 4 * P + uu;             // ring slot of substep 4 st + uu
            const bf16x8 a = read_a(4 * st + uu);
#pragma unroll
            for (int j = 0; j < KB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[u][j], a, acc[j], 0, 0, 0);
            // refill the slot with substep 4 st + uu + kRing (the last
            // substep again past the end, so the loads stay in bounds)
            const int ks = min(4 * st + uu + kRing, S - 1);
#pragma unroll
            for (int j = 0; j < KB; ++j) wr[u][j] = *(const bf16x8*)(wb[j] + w_off(ks));
        }
        store_x(P ^ 1, xr[P ^ 1]);
        load_x(st + 3, xr[P ^ 1]);
    };
    const int NS2 = NS / 2 * 2;                   // whole ring turns (two stages)
    for (int st = 0; st < NS2; st += 2) {
        stage(st, std::integral_constant<int, 0>());
        stage(st + 1, std::integral_constant<int, 1>());
    }
    if (NS2 < NS) stage(NS2, std::integral_constant<int, 0>());   // last 4 substeps

    // acc[j] element 4 qq + i of lane l: token t0 + l % 32, expert
    // 32 (eb0 + j) + 8 qq + 4 (l / 32) + i
    const int t = t0 + l32;
    if (t >= T) return;
    float* out = logits + (size_t)t * E;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
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

namespace {
// workgroups of the router grid with kb weight blocks per workgroup
long long router_wgs(int T, int E, int kb) {
    const long long groups = ((E + 31) / 32 + kb - 1) / kb;
    return ((T + kTokens - 1) / kTokens + 7) / 8 * 8 * groups;
}
// the most weight blocks per workgroup (3, 2, 1) whose grid still covers the
// CUs, else 1: fewer blocks per workgroup mean more, shorter workgroups
// (64-expert layer with 4096 tokens: 29 -> 20 us with 1 block)
int router_blocks(int T, int E) {
    const long long cus = device_cu_count();
    for (int kb = 3; kb > 1; --kb)
        if (router_wgs(T, E, kb) >= cus) return kb;
    return 1;
}
}  // namespace

bool router_packed_preferred(int T, int E) {
    // each workgroup's time is set by its own load latency chain, so the
    // kernel wins while its grid is at most two rounds over the CUs; larger
    // grids go to the persistent grouped GEMM (same bits either way)
    return router_wgs(T, E, router_blocks(T, E)) <= 2LL * device_cu_count();
}

hipError_t launch_router_packed(const uint16_t* x, const uint16_t* wg_packed, const float* offset,
                                int T, int K, int E, float* logits, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    if (K % 64 || E < 1 || E > MOE_MAX_E) return hipErrorInvalidValue;
    const int kb = router_blocks(T, E);
    const unsigned grid = (unsigned)router_wgs(T, E, kb);
    if (kb == 3)
        hipLaunchKernelGGL(router_kernel<3>, dim3(grid), dim3(256), 0, stream, x, wg_packed,
                           offset, T, K, E, logits);
    else if (kb == 2)
        hipLaunchKernelGGL(router_kernel<2>, dim3(grid), dim3(256), 0, stream, x, wg_packed,
                           offset, T, K, E, logits);
    else
        hipLaunchKernelGGL(router_kernel<1>, dim3(grid), dim3(256), 0, stream, x, wg_packed,
                           offset, T, K, E, logits);
    return hipGetLastError();
}

}  // namespace moe
