// Grouped GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), used for
// the router projection, the expert gate/up projection with the clamped
// SwiGLU epilogue, and the expert down projection ("HyperParallel
// accelerates DeepSeek-V4.1 ...", section 2.3, MegaMoE: two expert matmuls
// with the V4.1 SwiGLU clamp between them).
//
// Problem: for each group g and activation row r in [lo_g, hi_g),
//   out[r, n] = sum_k A[r, k] * W[g, n, k]      (W stored [out, in])
// Tiling (one workgroup = 4 waves = 256 threads):
//   - a tile is up to 256 activation rows x 256 weight rows (SwiGLU: 128
//     features x {gate, up}); each wave owns 64 weight rows (two 32-row MFMA
//     blocks) against all rows of the tile (eight 32-row blocks, or four when
//     the tile holds at most 128 valid rows): up to 16 accumulators of 32x32.
//     An expert with up to 256 rows is one tile, so its weights are streamed
//     from memory once.
//   - K advances in 64-wide stages, 4 MFMA substeps of 16 each.  Substep q
//     pairs k-chunk 2q (lanes 0-31) and 2q+1 (lanes 32-63) of both operands.
//   - Weights: every weight element is used by exactly one wave, so they go
//     straight from memory into the MFMA operand registers through a 3-deep
//     register ring (stage j computes while j+1 and j+2 are in flight).
//     Every load is issued unconditionally (tail stages and padding rows read
//     clamped, valid addresses), so the in-order vmcnt accounting never
//     collapses to a full drain.
//   - Activations: each stage's tile goes global -> registers -> LDS (2-slot
//     LDS ring, rows padded to 144 B; loads issued one stage ahead), one
//     barrier per stage.
//   - Weight layouts: [out, in] row-major, or the packed panel layout written
//     by moe_pack_weights: the 16-byte fragments one wave loads for one
//     substep are 1 KB contiguous in lane order (fully coalesced loads), and a
//     workgroup's whole weight panel for one stage is contiguous, so each
//     workgroup streams one sequential range per weight tensor.
//   - MFMA operand A = weights (D rows = weight rows), operand B = the
//     activation rows (D cols = activation rows): lane l holds activation row
//     l % 32 and weight rows 8 (i / 4) + 4 (l / 32) + i % 4 of accumulator
//     element i, so epilogue stores are 4 consecutive outputs per lane.
// Scheduling: persistent grid; every workgroup builds the per-group m-tile
// prefix in LDS from the device offsets (no host sync); work items are
// ordered (group, n-tile, m-tile) and split into 8 contiguous ranges, one
// per XCD (workgroup id mod 8), so the tiles of one expert run together on
// one XCD and share its L2 for the activation rows and weights.
#include "moe_internal.h"

namespace moe {
namespace {

// Tile shape and pipeline depths (defaults; the build may override them)
#ifndef MOE_GEMM_MAXNTB
#define MOE_GEMM_MAXNTB 4   // 32-row activation blocks per expert tile
#endif
#ifndef MOE_GEMM_RING
#define MOE_GEMM_RING 4     // weight register ring depth (stages)
#endif
#ifndef MOE_GEMM_APRE
#define MOE_GEMM_APRE 2     // activation prefetch depth (stages)
#endif
constexpr int BM = 256;                // LDS rows per activation slot (max tile height)
constexpr int BK = 64;
constexpr int kLdsRow = BK * 2 + 16;   // bytes per activation row in LDS
constexpr int kLdsStage = BM * kLdsRow;
constexpr int kLdsStages = 2;

__device__ __forceinline__ float clamp_sym(float v, float L) { return fminf(fmaxf(v, -L), L); }

template <int EPI, bool PACKED>
struct TileCtx {
    const GemmArgs* args;
    unsigned char* smem;
    int tid, lane, wave, half, l32;
    int S, N, K;
    int row0, grp_hi;
    int n_wave;
    bool active;
    const uint16_t* w_ptr0;
    const uint16_t* w_ptr1;
};

// One tile: rows [row0, row0 + 32*NTB) (clamped to grp_hi) x this wave's 64
// weight rows.  K loop with an R-deep weight register ring and an AD-deep
// activation register staging ring feeding a 2-slot LDS ring.  Stage j
// issues A(j+AD) then W(j+R-1) (into the slot W(j-1) used), computes stage j,
// stores A(j+1) to LDS and hits one barrier.  vmcnt retires loads in issue
// order, so waiting for A(j+1) also retires every weight load issued before
// it: a weight stage can stay in flight for up to AD+1 stages.
template <int EPI, bool PACKED, int NTB, int R, int AD>
__device__ __forceinline__ void run_tile(TileCtx<EPI, PACKED>& c) {
    constexpr int kPanel = (EPI == EPI_SWIGLU_BF16) ? 128 : 256;
    const GemmArgs& args = *c.args;
    const int tid = c.tid, half = c.half, l32 = c.l32;
    const int S = c.S, K = c.K, N = c.N;
    // activation tile: thread loads 16 B chunks (row = tid/8 + 32 i, chunk = tid % 8)
    const uint16_t* a_ptr[NTB];
#pragma unroll
    for (int i = 0; i < NTB; ++i) {
        const int r = min(c.row0 + (tid >> 3) + 32 * i, c.grp_hi - 1);
        a_ptr[i] = args.a + (size_t)r * K + (tid & 7) * 8;
    }
    f32x16 acc[2][NTB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;

    u32x4 areg[AD][NTB];
    bf16x8 wr[R][2][4];

    auto load_a = [&](int j, u32x4* dst) {
        const int k0 = min(j, S - 1) * BK;
#pragma unroll
        for (int i = 0; i < NTB; ++i) dst[i] = *(const u32x4*)(a_ptr[i] + k0);
    };
    auto store_a = [&](int j, const u32x4* src) {
        unsigned char* base = c.smem + (j & 1) * kLdsStage;
#pragma unroll
        for (int i = 0; i < NTB; ++i)
            *(u32x4*)(base + ((tid >> 3) + 32 * i) * kLdsRow + (tid & 7) * 16) = src[i];
    };
    auto load_w = [&](int j, bf16x8 (*dst)[4]) {
        const int js = min(j, S - 1);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const size_t off = PACKED ? (size_t)js * (kPanel / 32) * 2048 + qq * 512
                                      : (size_t)js * BK + qq * 16;
            dst[0][qq] = *(const bf16x8*)(c.w_ptr0 + off);
            dst[1][qq] = *(const bf16x8*)(c.w_ptr1 + off);
        }
    };
    auto compute = [&](int j, bf16x8 (*w)[4]) {
        const unsigned char* base = c.smem + (j & 1) * kLdsStage + l32 * kLdsRow + half * 16;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            bf16x8 bt[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
                bt[tb] = *(const bf16x8*)(base + tb * 32 * kLdsRow + qq * 32);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[0][qq], bt[tb], acc[0][tb],
                                                                      0, 0, 0);
                acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[1][qq], bt[tb], acc[1][tb],
                                                                      0, 0, 0);
            }
        }
    };

    // prologue: the loads the stages v < 0 would have issued, in the
    // steady-state order (A(v+AD) then W(v+R-1)); then A(0) to LDS slot 0
    constexpr int V0 = (AD > R - 1) ? AD : R - 1;
#pragma unroll
    for (int v = -V0; v < 0; ++v) {
        if (v + AD >= 0) load_a(v + AD, areg[(v + AD) % AD]);
        __builtin_amdgcn_sched_barrier(0);
        if (v + R - 1 >= 0) load_w(v + R - 1, wr[(v + R - 1) % R]);
        __builtin_amdgcn_sched_barrier(0);
    }
    store_a(0, areg[0]);
    __syncthreads();
    constexpr int UNROLL = (R % AD == 0) ? R : R * AD;
    for (int s = 0;; s += UNROLL) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int j = s + u;
            if (j >= S) goto k_done;
            load_a(j + AD, areg[(u + AD) % AD]);
            __builtin_amdgcn_sched_barrier(0);
            load_w(j + R - 1, wr[(u + R - 1) % R]);
            __builtin_amdgcn_sched_barrier(0);
            if (c.active) compute(j, wr[u % R]);
            __builtin_amdgcn_sched_barrier(0);
            store_a(j + 1, areg[(u + 1) % AD]);
            __syncthreads();
        }
    }
k_done:

    if (!c.active) return;
    // ---- epilogue ----
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int r = c.row0 + tb * 32 + l32;
        if (r >= c.grp_hi) continue;
        if (EPI == EPI_SWIGLU_BF16) {
            const float L = args.clamp_limit;
            uint16_t* orow = (uint16_t*)args.out + (size_t)r * N;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int n = c.n_wave + 8 * qq + 4 * half;
                uint32_t packed[2];
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    uint16_t hb[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        float gv = acc[0][tb][4 * qq + i + u];
                        float uv = acc[1][tb][4 * qq + i + u];
                        gv = args.clamp_mode == MOE_CLAMP_SYMMETRIC ? clamp_sym(gv, L)
                                                                    : fminf(gv, L);
                        uv = clamp_sym(uv, L);
                        const float silu = gv / (1.0f + __expf(-gv));
                        hb[u] = f32_to_bf16(silu * uv);
                    }
                    packed[i >> 1] = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
                }
                *(u32x2*)(orow + n) = u32x2{packed[0], packed[1]};
            }
        } else {
            float* orow = (float*)args.out + (size_t)r * N;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int n = c.n_wave + 32 * b + 8 * qq + 4 * half;
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = acc[b][tb][4 * qq + i];
                    if (EPI == EPI_F32_OFFSET) {
                        if ((N & 3) == 0 && n + 3 < N) {
                            if (args.offset)
#pragma unroll
                                for (int i = 0; i < 4; ++i) v[i] = v[i] + args.offset[n + i];
                            *(f32x4*)(orow + n) = v;
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (n + i < N)
                                    orow[n + i] = args.offset ? v[i] + args.offset[n + i] : v[i];
                        }
                    } else {
                        if (n < N) *(f32x4*)(orow + n) = v;
                    }
                }
        }
    }
}

// MAXNTB: 32-row activation blocks per tile (8 for the expert GEMMs; the
// router projection uses 4, which keeps its offset epilogue out of spills)
template <int EPI, bool PACKED, int MAXNTB, int RING, int APRE>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs args) {
    constexpr int TM = MAXNTB * 32;
    extern __shared__ __align__(16) unsigned char smem[];
    int* tile_prefix = (int*)(smem + kLdsStages * kLdsStage);
    __shared__ int scan_sh[4];

    TileCtx<EPI, PACKED> c;
    c.args = &args;
    c.smem = smem;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wave = c.tid >> 6;
    c.half = c.lane >> 5;
    c.l32 = c.lane & 31;
    const int tid = c.tid, lane = c.lane, wave = c.wave;
    const int G = args.G, rows = args.rows, K = args.K, N = args.N;
    c.K = K;
    c.N = N;
    const int* offs = args.offsets;

    // ---- per-group m-tile counts -> exclusive prefix in LDS ----
    {
        const int per = (G + 255) / 256;
        const int g0 = tid * per;
        int local = 0;
        for (int g = g0; g < g0 + per && g < G; ++g) {
            int lo = 0, hi = rows;
            if (offs) {
                lo = min(max(offs[g], 0), rows);
                hi = max(lo, min(max(offs[g + 1], 0), rows));
            }
            const int mt = (hi - lo + TM - 1) / TM;
            tile_prefix[g] = mt;  // temporarily the count
            local += mt;
        }
        int x = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) scan_sh[wave] = x;
        __syncthreads();
        int wbase = 0, total = 0;
        for (int w = 0; w < 4; ++w) {
            if (w < wave) wbase += scan_sh[w];
            total += scan_sh[w];
        }
        int run = wbase + x - local;
        for (int g = g0; g < g0 + per && g < G; ++g) {
            const int mt = tile_prefix[g];
            tile_prefix[g] = run;
            run += mt;
        }
        if (tid == 0) tile_prefix[G] = total;
        __syncthreads();
    }

    constexpr int kRowsPerWg = (EPI == EPI_SWIGLU_BF16) ? 128 : 256;
    const int NT = (N + kRowsPerWg - 1) / kRowsPerWg;
    const long long Q = (long long)tile_prefix[G] * NT;
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const long long q_lo = Q * xcd / 8, q_hi = Q * (xcd + 1) / 8;

    c.S = K / BK;                         // K is a multiple of 64
    const int NB = (N + 31) >> 5;         // 32-row weight blocks per group
    // packed weights are panels of kPanelRows rows: 128 (gate / up, four
    // features blocks of one workgroup) or 256 (down / router)
    constexpr int kPanelRows = (EPI == EPI_SWIGLU_BF16) ? 128 : 256;
    const size_t w_group =
        PACKED ? (size_t)((N + kPanelRows - 1) / kPanelRows) * kPanelRows * K : (size_t)N * K;

    for (long long q = q_lo + (blockIdx.x >> 3); q < q_hi; q += per_xcd) {
        // ---- decode (group, n-tile, m-tile) ----
        const int qm = (int)(q / NT);
        int g = 0;
        {
            int lo = 0, hi = G;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (tile_prefix[mid] <= qm) lo = mid; else hi = mid - 1;
            }
            g = lo;
        }
        const int mt = tile_prefix[g + 1] - tile_prefix[g];
        const int local = (int)(q - (long long)tile_prefix[g] * NT);
        const int n_tile = local / mt;
        const int m_tile = local % mt;
        int grp_lo = 0, grp_hi = rows;
        if (offs) {
            grp_lo = min(max(offs[g], 0), rows);
            grp_hi = max(grp_lo, min(max(offs[g + 1], 0), rows));
        }
        c.row0 = grp_lo + m_tile * TM;
        c.grp_hi = grp_hi;
        // weight rows of this wave: blocks nb0, nb1 (32 rows each)
        c.n_wave = (EPI == EPI_SWIGLU_BF16) ? n_tile * 128 + wave * 32 : n_tile * 256 + wave * 64;
        c.active = c.n_wave < N;
        {
            const uint16_t* base1 = args.w1 + (size_t)g * w_group;
            const uint16_t* base2 = (EPI == EPI_SWIGLU_BF16 ? args.w2 : args.w1) +
                                    (size_t)g * w_group;
            const int nb0 = min(c.n_wave >> 5, NB - 1);
            const int nb1 = (EPI == EPI_SWIGLU_BF16) ? nb0 : min((c.n_wave >> 5) + 1, NB - 1);
            if (PACKED) {
                // panel layout [panel][stage][block in panel][substep][lane][8]
                constexpr int BPP = kPanelRows / 32;
                const size_t pstride = (size_t)kPanelRows * K;
                c.w_ptr0 = base1 + (size_t)(nb0 / BPP) * pstride + (nb0 % BPP) * 2048 + lane * 8;
                c.w_ptr1 = base2 + (size_t)(nb1 / BPP) * pstride + (nb1 % BPP) * 2048 + lane * 8;
            } else {
                const int r0 = min(nb0 * 32 + c.l32, N - 1);
                const int r1 = min(nb1 * 32 + c.l32, N - 1);
                c.w_ptr0 = base1 + (size_t)r0 * K + c.half * 8;
                c.w_ptr1 = base2 + (size_t)r1 * K + c.half * 8;
            }
        }
        // the tile computes only as many 32-row blocks as it has valid rows
        // (4-block granularity above 128 rows)
        const int valid = grp_hi - c.row0;
        if (valid <= 32)
            run_tile<EPI, PACKED, 1, RING, APRE>(c);
        else if (valid <= 64)
            run_tile<EPI, PACKED, 2, RING, APRE>(c);
        else if (valid <= 96)
            run_tile<EPI, PACKED, 3, RING, APRE>(c);
        else if (MAXNTB == 4 || valid <= 128)
            run_tile<EPI, PACKED, 4, RING, APRE>(c);
        else
            run_tile<EPI, PACKED, MAXNTB, RING, APRE>(c);
    }
}

// Packed weight layout for panels of P rows (P = 128 or 256):
// [G][ceil(N/P)][S = K/64][P/32][4][64 lanes][8 bf16]; fragment
// (panel, s, b, q, lane) = W[panel*P + b*32 + lane%32][s*64 + 16 q + 8 (lane/32) .. +8],
// rows >= N zero-filled.  One workgroup's weight panel is contiguous per stage.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ src,
                                                           uint16_t* __restrict__ dst, int N,
                                                           int K, int P, long long nfrag_group,
                                                           long long nfrag) {
    const long long f = (long long)blockIdx.x * 256 + threadIdx.x;
    if (f >= nfrag) return;
    const long long g = f / nfrag_group;
    long long r = f - g * nfrag_group;
    const int lane = (int)(r & 63);
    r >>= 6;
    const int qq = (int)(r & 3);
    r >>= 2;
    const int bpp = P / 32;
    const int b = (int)(r % bpp);
    r /= bpp;
    const int S = K / BK;
    const int s = (int)(r % S);
    const int panel = (int)(r / S);
    const int row = panel * P + b * 32 + (lane & 31);
    const int col = s * BK + 16 * qq + 8 * (lane >> 5);
    u32x4 v = {0, 0, 0, 0};
    if (row < N) v = *(const u32x4*)(src + ((size_t)g * N + row) * K + col);
    *(u32x4*)(dst + (size_t)f * 8) = v;
}

template <int EPI, bool PACKED>
hipError_t launch_epi(const GemmArgs& g, hipStream_t stream) {
    constexpr int MAXNTB = EPI == EPI_F32_OFFSET ? 4 : MOE_GEMM_MAXNTB;
    constexpr int RING = MOE_GEMM_RING;
    constexpr int APRE = MOE_GEMM_APRE;
    const size_t lds = kLdsStages * kLdsStage + (size_t)(MOE_MAX_GROUPS + 1) * sizeof(int);
    // per device, once: the dynamic LDS limit and the grid (all resident
    // workgroups, whole rounds of the 8 XCDs)
    static DeviceSetup setup;
    long long grid = 0, unused = 0;
    const hipError_t err = device_setup(setup, grid, unused, [](int, long long& gr, long long&) {
        hipError_t e = hipFuncSetAttribute(
            (const void*)grouped_gemm_kernel<EPI, PACKED, MAXNTB, RING, APRE>,
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        int occ = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ, grouped_gemm_kernel<EPI, PACKED, MAXNTB, RING, APRE>, 256, lds);
        if (e != hipSuccess) return e;
        if (occ < 1) occ = 1;
        gr = ((long long)device_cu_count() * occ + 7) & ~7LL;
        return hipSuccess;
    });
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((grouped_gemm_kernel<EPI, PACKED, MAXNTB, RING, APRE>), dim3((unsigned)grid),
                       dim3(256), lds, stream, g);
    return hipGetLastError();
}

}  // namespace

size_t packed_weight_elems(int G, int N, int K, int P) {
    return (size_t)G * (size_t)((N + P - 1) / P) * P * (size_t)K;
}

hipError_t launch_pack_weights(const uint16_t* src, uint16_t* dst, int G, int N, int K, int P,
                               hipStream_t stream) {
    const long long nfrag_group = (long long)((N + P - 1) / P) * P / 32 * (K / BK) * 4 * 64;
    const long long nfrag = nfrag_group * G;
    if (nfrag == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((nfrag + 255) / 256)), dim3(256), 0,
                       stream, src, dst, N, K, P, nfrag_group, nfrag);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(int epilogue, const GemmArgs& g, hipStream_t stream) {
    if (g.packed) {
        switch (epilogue) {
            case EPI_SWIGLU_BF16: return launch_epi<EPI_SWIGLU_BF16, true>(g, stream);
            case EPI_F32: return launch_epi<EPI_F32, true>(g, stream);
            case EPI_F32_OFFSET: return launch_epi<EPI_F32_OFFSET, true>(g, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (epilogue) {
        case EPI_SWIGLU_BF16: return launch_epi<EPI_SWIGLU_BF16, false>(g, stream);
        case EPI_F32: return launch_epi<EPI_F32, false>(g, stream);
        case EPI_F32_OFFSET: return launch_epi<EPI_F32_OFFSET, false>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
