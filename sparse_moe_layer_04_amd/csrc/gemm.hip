// Grouped GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), used for
// the router projection, the expert gate/up projection with the clamped
// SwiGLU epilogue, and the expert down projection ("HyperParallel
// accelerates DeepSeek-V4.1 ...", section 2.3, MegaMoE: two expert matmuls
// with the V4.1 SwiGLU clamp between them).
//
// Problem: for each group g and activation row r in [lo_g, hi_g),
//   out[r, n] = sum_k A[r, k] * W[g, n, k]      (W stored [out, in])
// Tiling (one workgroup = 4 waves = 256 threads):
//   - a tile is 128 activation rows x 256 weight rows (SwiGLU: 128 features
//     x {gate, up}); each wave owns 64 weight rows (two 32-row MFMA blocks)
//     against all 128 rows (four 32-row blocks): 8 accumulators of 32x32.
//   - K advances in 64-wide stages, 4 MFMA substeps of 16 each.  Substep q
//     pairs k-chunk 2q (lanes 0-31) and 2q+1 (lanes 32-63) of both operands.
//   - Weights: every weight element is used by exactly one wave, so they go
//     straight from memory into the MFMA operand registers through a 4-deep
//     register ring (stage j computes while stages j+1..j+3 are in flight:
//     96 KB per CU).  Every load is issued unconditionally (tail stages and
//     padding rows read clamped, valid addresses), so the in-order vmcnt
//     accounting never collapses to a full drain.
//   - Activations: each stage's 128 x 64 tile goes global -> registers -> LDS
//     (3-deep LDS ring, rows padded to 144 B; loads issued two stages ahead),
//     one barrier per stage.
//   - Weight layouts: [out, in] row-major, or the packed layout written by
//     moe_pack_weights, in which the 16-byte fragments one wave loads for one
//     substep are 1 KB contiguous in lane order (fully coalesced loads).
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

constexpr int BM = 128;
constexpr int BK = 64;
constexpr int kLdsRow = BK * 2 + 16;   // bytes per activation row in LDS
constexpr int kLdsStage = BM * kLdsRow;
constexpr int kLdsStages = 3;
constexpr int kWRing = 4;

__device__ __forceinline__ float clamp_sym(float v, float L) { return fminf(fmaxf(v, -L), L); }

template <int EPI, bool PACKED>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs args) {
    extern __shared__ __align__(16) unsigned char smem[];
    int* tile_prefix = (int*)(smem + kLdsStages * kLdsStage);
    __shared__ int scan_sh[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int G = args.G, rows = args.rows, K = args.K, N = args.N;
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
            const int mt = (hi - lo + BM - 1) / BM;
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

    const int S = K / BK;                 // K is a multiple of 64
    const int NB = (N + 31) >> 5;         // 32-row weight blocks per group
    const size_t w_group = PACKED ? (size_t)NB * 32 * K : (size_t)N * K;

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
        const int row0 = grp_lo + m_tile * BM;

        // activation tile: thread loads 16 B chunks (row = tid/8 + 32 i, chunk = tid % 8)
        const uint16_t* a_ptr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = min(row0 + (tid >> 3) + 32 * i, grp_hi - 1);
            a_ptr[i] = args.a + (size_t)r * K + (tid & 7) * 8;
        }
        // weight rows of this wave: blocks nb0, nb1 (32 rows each)
        const int n_wave = (EPI == EPI_SWIGLU_BF16) ? n_tile * 128 + wave * 32
                                                    : n_tile * 256 + wave * 64;
        const bool active = n_wave < N;
        const uint16_t* w_ptr0;
        const uint16_t* w_ptr1;
        {
            const uint16_t* base1 = args.w1 + (size_t)g * w_group;
            const uint16_t* base2 = (EPI == EPI_SWIGLU_BF16 ? args.w2 : args.w1) +
                                    (size_t)g * w_group;
            int nb0 = min(n_wave >> 5, NB - 1);
            int nb1 = (EPI == EPI_SWIGLU_BF16) ? nb0 : min((n_wave >> 5) + 1, NB - 1);
            if (PACKED) {
                // [nb][stage][substep][lane][8]
                w_ptr0 = base1 + (size_t)nb0 * 32 * K + lane * 8;
                w_ptr1 = base2 + (size_t)nb1 * 32 * K + lane * 8;
            } else {
                const int r0 = min(nb0 * 32 + l32, N - 1);
                const int r1 = min(nb1 * 32 + l32, N - 1);
                w_ptr0 = base1 + (size_t)r0 * K + half * 8;
                w_ptr1 = base2 + (size_t)r1 * K + half * 8;
            }
        }

        f32x16 acc[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;

        u32x4 areg[2][4];
        bf16x8 wr[kWRing][2][4];

        auto load_a = [&](int j, u32x4* dst) {
            const int k0 = min(j, S - 1) * BK;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = *(const u32x4*)(a_ptr[i] + k0);
        };
        auto store_a = [&](int j, const u32x4* src) {
            unsigned char* base = smem + (j % kLdsStages) * kLdsStage;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(u32x4*)(base + ((tid >> 3) + 32 * i) * kLdsRow + (tid & 7) * 16) = src[i];
        };
        auto load_w = [&](int j, bf16x8 (*dst)[4]) {
            const int js = min(j, S - 1);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                if (PACKED) {
                    const size_t off = (size_t)js * 2048 + qq * 512;
                    dst[0][qq] = *(const bf16x8*)(w_ptr0 + off);
                    dst[1][qq] = *(const bf16x8*)(w_ptr1 + off);
                } else {
                    const size_t off = (size_t)js * BK + qq * 16;
                    dst[0][qq] = *(const bf16x8*)(w_ptr0 + off);
                    dst[1][qq] = *(const bf16x8*)(w_ptr1 + off);
                }
            }
        };
        auto compute = [&](int j, bf16x8 (*w)[4]) {
            const unsigned char* base =
                smem + (j % kLdsStages) * kLdsStage + l32 * kLdsRow + half * 16;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                bf16x8 bt[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    bt[tb] = *(const bf16x8*)(base + tb * 32 * kLdsRow + qq * 32);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[0][qq], bt[tb],
                                                                          acc[0][tb], 0, 0, 0);
                    acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[1][qq], bt[tb],
                                                                          acc[1][tb], 0, 0, 0);
                }
            }
        };

        // ---- prologue: LDS holds A(0); areg[1] = A(1); wr[0..2] = W(0..2) ----
        // (issue order A(0) W(0) W(1) A(1) W(2) matches the steady state, in
        // which A(j+1) is followed by W(j+2) and the next stage's A, W)
        load_a(0, areg[0]);
        __builtin_amdgcn_sched_barrier(0);
        load_w(0, wr[0]);
        load_w(1, wr[1]);
        __builtin_amdgcn_sched_barrier(0);
        load_a(1, areg[1]);
        __builtin_amdgcn_sched_barrier(0);
        load_w(2, wr[2]);
        __builtin_amdgcn_sched_barrier(0);
        store_a(0, areg[0]);
        __syncthreads();

        // ---- main loop: 4 stages per iteration (static register rings) ----
        // stage j: issue A(j+2) -> areg[j%2], W(j+3) -> wr[(j+3)%4]; compute j;
        // store A(j+1) (areg[(j+1)%2]) into LDS slot (j+1)%3; barrier.
        for (int s = 0; s < S; s += 4) {
// (scheduling barriers keep each stage's loads in issue order A then W, so
// the in-order vmcnt waits for A(j+1) never cover W(j+2) or W(j+3))
#define MOE_GEMM_STAGE(U)                                              \
    {                                                                  \
        const int j = s + (U);                                         \
        load_a(j + 2, areg[(U) & 1]);                                  \
        __builtin_amdgcn_sched_barrier(0);                             \
        load_w(j + 3, wr[((U) + 3) & 3]);                              \
        __builtin_amdgcn_sched_barrier(0);                             \
        if (active && j < S) compute(j, wr[(U) & 3]);                  \
        __builtin_amdgcn_sched_barrier(0);                             \
        store_a(j + 1, areg[((U) + 1) & 1]);                           \
        __syncthreads();                                               \
    }
            MOE_GEMM_STAGE(0)
            MOE_GEMM_STAGE(1)
            MOE_GEMM_STAGE(2)
            MOE_GEMM_STAGE(3)
#undef MOE_GEMM_STAGE
        }

        if (!active) continue;
        // ---- epilogue ----
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int r = row0 + tb * 32 + l32;
            if (r >= grp_hi) continue;
            if (EPI == EPI_SWIGLU_BF16) {
                const float L = args.clamp_limit;
                uint16_t* orow = (uint16_t*)args.out + (size_t)r * N;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int n = n_wave + 8 * qq + 4 * half;
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
                        const int n = n_wave + 32 * b + 8 * qq + 4 * half;
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
                                        orow[n + i] =
                                            args.offset ? v[i] + args.offset[n + i] : v[i];
                            }
                        } else {
                            if (n < N) *(f32x4*)(orow + n) = v;
                        }
                    }
            }
        }
    }
}

// Packed weight layout: [G][NB = ceil(N/32)][S = K/64][4][64 lanes][8 bf16];
// fragment (nb, s, q, lane) = W[nb*32 + lane%32][s*64 + 16 q + 8 (lane/32) .. +8],
// rows >= N zero-filled.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ src,
                                                           uint16_t* __restrict__ dst, int N,
                                                           int K, long long nfrag_group,
                                                           long long nfrag) {
    const long long f = (long long)blockIdx.x * 256 + threadIdx.x;
    if (f >= nfrag) return;
    const long long g = f / nfrag_group;
    long long r = f - g * nfrag_group;
    const int lane = (int)(r & 63);
    r >>= 6;
    const int qq = (int)(r & 3);
    r >>= 2;
    const int S = K / BK;
    const int s = (int)(r % S);
    const int nb = (int)(r / S);
    const int row = nb * 32 + (lane & 31);
    const int col = s * BK + 16 * qq + 8 * (lane >> 5);
    u32x4 v = {0, 0, 0, 0};
    if (row < N) v = *(const u32x4*)(src + ((size_t)g * N + row) * K + col);
    *(u32x4*)(dst + (size_t)f * 8) = v;
}

template <int EPI, bool PACKED>
hipError_t launch_epi(const GemmArgs& g, hipStream_t stream) {
    static int configured_device = -1;
    static int grid = 0;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const size_t lds = kLdsStages * kLdsStage + (size_t)(MOE_MAX_GROUPS + 1) * sizeof(int);
    if (configured_device != dev) {
        err = hipFuncSetAttribute((const void*)grouped_gemm_kernel<EPI, PACKED>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        int occ = 0;
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, grouped_gemm_kernel<EPI, PACKED>,
                                                           256, lds);
        if (err != hipSuccess) return err;
        if (occ < 1) occ = 1;
        grid = device_cu_count() * occ;
        grid = (grid + 7) & ~7;
        configured_device = dev;
    }
    hipLaunchKernelGGL((grouped_gemm_kernel<EPI, PACKED>), dim3(grid), dim3(256), lds, stream, g);
    return hipGetLastError();
}

}  // namespace

size_t packed_weight_elems(int G, int N, int K) {
    return (size_t)G * (size_t)((N + 31) / 32) * 32 * (size_t)K;
}

hipError_t launch_pack_weights(const uint16_t* src, uint16_t* dst, int G, int N, int K,
                               hipStream_t stream) {
    const long long nfrag_group = (long long)((N + 31) / 32) * (K / BK) * 4 * 64;
    const long long nfrag = nfrag_group * G;
    if (nfrag == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((nfrag + 255) / 256)), dim3(256), 0,
                       stream, src, dst, N, K, nfrag_group, nfrag);
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
