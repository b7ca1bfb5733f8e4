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
//   - K advances in 128-wide stages.  The activation tile of a stage goes
//     global -> registers -> LDS (double buffered, rows padded to 272 B);
//     every weight element is used by exactly one wave, so weights go
//     straight from global memory into the MFMA operand registers, double
//     buffered one stage ahead (no LDS round trip for the streamed operand).
//   - K order inside a stage: lane half h (lane / 32) holds k in
//     [64 h, 64 h + 64); substep q uses k = 64 h + 8 q + [0, 8) from both
//     operands, so each lane streams 128 contiguous weight bytes per stage.
//   - MFMA operand A = weights (D rows = weight rows), operand B = the
//     activation rows (D cols = activation rows): lane l holds activation row
//     l % 32 and weight rows 8 (i / 4) + 4 (l / 32) + i % 4 of accumulator
//     element i, so epilogue stores are 4 consecutive outputs per lane.
// Scheduling: persistent grid; every workgroup builds the per-group m-tile
// prefix in LDS from the device offsets (no host sync), work items are
// ordered (group, n-tile, m-tile) and split into 8 contiguous ranges, one
// per XCD (workgroup id mod 8), so the m-tiles and n-tiles of one expert run
// together on one XCD and share its L2 for the activation rows and weights.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 128;
constexpr int BK = 128;
constexpr int kLdsRow = BK * 2 + 16;   // bytes per activation row in LDS
constexpr int kLdsStage = BM * kLdsRow;

__device__ __forceinline__ float clamp_sym(float v, float L) { return fminf(fmaxf(v, -L), L); }

template <int EPI>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs args) {
    extern __shared__ __align__(16) unsigned char smem[];
    int* tile_prefix = (int*)(smem + 2 * kLdsStage);
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

    const size_t KN = (size_t)K * N;
    const int S = (K + BK - 1) / BK;

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

        // ---- operand pointers ----
        // activation tile: thread loads 16 B chunks (row = tid/16 + 16 i, col16 = tid % 16)
        const uint16_t* a_ptr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = min(row0 + (tid >> 4) + 16 * i, grp_hi - 1);
            a_ptr[i] = args.a + (size_t)r * K + (tid & 15) * 8;
        }
        const int n_wave = (EPI == EPI_SWIGLU_BF16) ? n_tile * 128 + wave * 32
                                                    : n_tile * 256 + wave * 64;
        const bool active = n_wave < N;
        const uint16_t* w_ptr0;
        const uint16_t* w_ptr1;
        {
            const uint16_t* wbase1 = args.w1 + (size_t)g * KN;
            int r0, r1;
            if (EPI == EPI_SWIGLU_BF16) {
                r0 = min(n_wave + l32, N - 1);
                r1 = r0;
                w_ptr1 = args.w2 + (size_t)g * KN + (size_t)r1 * K + half * 64;
            } else {
                r0 = min(n_wave + l32, N - 1);
                r1 = min(n_wave + 32 + l32, N - 1);
                w_ptr1 = wbase1 + (size_t)r1 * K + half * 64;
            }
            w_ptr0 = wbase1 + (size_t)r0 * K + half * 64;
        }

        f32x16 acc[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;

        u32x4 areg[8];
        bf16x8 wa0[8], wa1[8], wb0[8], wb1[8];

        auto load_a = [&](int s) {
            const int k0 = s * BK;
            const int kval = K - k0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if ((tid & 15) * 8 < kval)
                    areg[i] = *(const u32x4*)(a_ptr[i] + k0);
                else
                    areg[i] = u32x4{0, 0, 0, 0};
            }
        };
        auto store_a = [&](int buf) {
            unsigned char* base = smem + buf * kLdsStage;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *(u32x4*)(base + ((tid >> 4) + 16 * i) * kLdsRow + (tid & 15) * 16) = areg[i];
        };
        auto load_w = [&](int s, bf16x8* w0, bf16x8* w1) {
            const int k0 = s * BK;
            if (half * 64 < K - k0) {
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    w0[v] = *(const bf16x8*)(w_ptr0 + k0 + v * 8);
                    w1[v] = *(const bf16x8*)(w_ptr1 + k0 + v * 8);
                }
            } else {
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    w0[v] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
                    w1[v] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
                }
            }
        };
        auto compute = [&](int buf, const bf16x8* w0, const bf16x8* w1) {
            const unsigned char* base = smem + buf * kLdsStage + l32 * kLdsRow + half * 128;
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) {
                bf16x8 bt[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    bt[tb] = *(const bf16x8*)(base + tb * 32 * kLdsRow + qq * 16);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0[qq], bt[tb],
                                                                          acc[0][tb], 0, 0, 0);
                    acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1[qq], bt[tb],
                                                                          acc[1][tb], 0, 0, 0);
                }
            }
        };

        // ---- K loop: two stages per iteration (static register buffers) ----
        load_a(0);
        if (active) {
            load_w(0, wa0, wa1);
            if (S > 1) load_w(1, wb0, wb1);
        }
        store_a(0);
        __syncthreads();
        for (int s = 0; s < S; s += 2) {
            if (s + 1 < S) load_a(s + 1);
            if (active) {
                compute(0, wa0, wa1);
                if (s + 2 < S) load_w(s + 2, wa0, wa1);
            }
            if (s + 1 < S) store_a(1);
            __syncthreads();
            if (s + 1 >= S) break;
            if (s + 2 < S) load_a(s + 2);
            if (active) {
                compute(1, wb0, wb1);
                if (s + 3 < S) load_w(s + 3, wb0, wb1);
            }
            if (s + 2 < S) store_a(0);
            __syncthreads();
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

template <int EPI>
hipError_t launch_epi(const GemmArgs& g, hipStream_t stream) {
    static int configured_device = -1;
    static int grid = 0;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const size_t lds = 2 * kLdsStage + (size_t)(MOE_MAX_GROUPS + 1) * sizeof(int);
    if (configured_device != dev) {
        err = hipFuncSetAttribute((const void*)grouped_gemm_kernel<EPI>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        int occ = 0;
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, grouped_gemm_kernel<EPI>, 256,
                                                           lds);
        if (err != hipSuccess) return err;
        if (occ < 1) occ = 1;
        grid = device_cu_count() * occ;
        grid = (grid + 7) & ~7;
        configured_device = dev;
    }
    hipLaunchKernelGGL(grouped_gemm_kernel<EPI>, dim3(grid), dim3(256), lds, stream, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(int epilogue, const GemmArgs& g, hipStream_t stream) {
    switch (epilogue) {
        case EPI_SWIGLU_BF16: return launch_epi<EPI_SWIGLU_BF16>(g, stream);
        case EPI_F32: return launch_epi<EPI_F32>(g, stream);
        case EPI_F32_OFFSET: return launch_epi<EPI_F32_OFFSET>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
