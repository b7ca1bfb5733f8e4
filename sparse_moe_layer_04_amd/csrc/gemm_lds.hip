// Grouped expert GEMM for packed weights: 256 x 256 tiles, both operands
// staged in LDS by direct-to-LDS DMA loads ("HyperParallel accelerates
// DeepSeek-V4.1 ...", section 2.3, MegaMoE: the two expert matmuls and the
// clamped SwiGLU between them).
//
// Problem: for each expert g and activation row r in [lo_g, hi_g),
//   out[r, n] = sum_k A[r, k] * W[g, n, k]
// with W in the moe_pack_weights panel layout (P = 128 rows for the gate and
// up matrices, P = 256 for the down matrix).
//
// One workgroup = 8 waves (two per SIMD); a tile is up to 256 activation rows
// x 256 weight rows (SwiGLU: 128 features x {gate, up}).  Wave w = (wm, wn),
// wm = w / 4 picks the 128-row half of the tile, wn = w % 4 the 64 weight
// rows (two 32-row MFMA blocks: SwiGLU gate block wn and up block wn; down
// blocks 2wn, 2wn+1).  An expert with up to 256 rows is one tile, so its
// weights are read from memory once.  Per 32-wide K stage one LDS slot holds
//   - the activation tile, 256 rows x 64 B, the 16-byte chunks of row r
//     XOR-swizzled by ((r / 2) mod 4) so that MFMA operand reads spread
//     over the banks;
//   - the weight panel half-stage, 16 KB in matrix-core fragment order
//     (copied from the packed layout in 1 KB runs; the operand reads are
//     1 KB contiguous per wave).
// A 4-slot LDS ring keeps three stages (96 KB) in flight per CU.  Each of
// the 8 waves issues 2 activation and 2 weight DMA instructions of 1 KB per
// stage (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16 l).  The
// DMA is issued from inline assembly, so the compiler does not see LDS
// writes it would otherwise guard with a full vmcnt drain before every LDS
// read; explicit vmcnt waits + one barrier per stage are the complete
// synchronisation.
// Scheduling: persistent grid, per-expert tile prefix built in LDS from the
// device offsets, items ordered (expert, n-tile, m-tile) and split into 8
// contiguous ranges, one per XCD.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TM = 256;                      // activation rows per tile
constexpr int BK = 32;                       // K per pipeline stage
constexpr int kSlotA = TM * 64;              // 16 KB activation tile per stage
constexpr int kSlotW = 16 * 1024;            // 16 KB weight panel half-stage
constexpr int kSlot = kSlotA + kSlotW;
constexpr int kSlots = 4;                    // LDS ring: 3 stages in flight
constexpr int kThreads = 512;

__device__ __forceinline__ float clamp_sym(float v, float L) { return fminf(fmaxf(v, -L), L); }

// 1 KB direct-to-LDS copy: lane l's 16 bytes from gaddr go to LDS byte
// lds_byte + 16 l.
// (lds_byte must be wave-uniform; readfirstlane makes that visible)
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_byte) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(m0v), "v"(gaddr)
                 : "memory", "m0");
}

// wait until at most N of this wave's memory operations are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int EPI>
struct LdsTile {
    const GemmArgs* args;
    uint32_t lds0;         // LDS byte address of slot 0
    unsigned char* smem;
    int lane, wave, wm, wn, half, l32;
    int K, N, S;
    int row0, grp_hi, valid;
    int n0;                // first weight row / feature of this wave's blocks
    const uint16_t* wsrc0; // weight panel (gate panel for SwiGLU)
    const uint16_t* wsrc1; // up panel (SwiGLU) or the same panel
    size_t wstride;        // packed elements per 64-wide K stage of one panel
};

// DMA of pipeline stage j (32 k) into `slot`: 2 activation and 2 weight
// instructions per wave, always issued (rows past the tile read the last
// valid row), so every stage costs each wave exactly 4 vmcnt entries.
//   activations: wave w copies rows [32 w, 32 w + 32), 16 rows x 64 B per
//     instruction; chunk c of row r is stored at position c ^ ((r >> 1) & 3).
//   weights: the 64-wide packed stage s = j / 2 holds, per 32-row block b,
//     4 substeps x 1 KB; this half-stage (h = j % 2) takes substeps 2h, 2h+1
//     of all 8 blocks: instruction n = 2 w + i copies block n / 2, substep
//     2h + n % 2 to LDS fragment slot n.
template <int EPI>
__device__ __forceinline__ void issue_stage(const LdsTile<EPI>& t, int j, int slot) {
    const uint32_t base = t.lds0 + slot * kSlot;
    const int kcol = j * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r0 = 32 * t.wave + 16 * i;
        const int r = r0 + (t.lane >> 2);
        const int c = (t.lane & 3) ^ ((t.lane >> 3) & 3);
        const int grow = t.row0 + min(r, t.valid - 1);
        dma16(t.args->a + (size_t)grow * t.K + kcol + c * 8, base + r0 * 64);
    }
    const int s64 = j >> 1, h2 = j & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int n = 2 * t.wave + i;
        const int b = n >> 1;
        const int sub = 2 * h2 + (n & 1);
        const uint16_t* src;
        if (EPI == EPI_SWIGLU_BF16)
            src = (b < 4 ? t.wsrc0 + (size_t)b * 2048 : t.wsrc1 + (size_t)(b - 4) * 2048);
        else
            src = t.wsrc0 + (size_t)b * 2048;
        dma16(src + (size_t)s64 * t.wstride + sub * 512 + t.lane * 8, base + kSlotA + n * 1024);
    }
}

template <int EPI, int NTB>
__device__ __forceinline__ void compute_stage(const LdsTile<EPI>& t, int slot,
                                              f32x16 (&acc)[2][4]) {
    const unsigned char* base = t.smem + slot * kSlot;
    // weight blocks of this wave (fragment slots 2 b + substep)
    const int b0 = (EPI == EPI_SWIGLU_BF16) ? t.wn : 2 * t.wn;
    const int b1 = (EPI == EPI_SWIGLU_BF16) ? 4 + t.wn : 2 * t.wn + 1;
    const unsigned char* wbase = base + kSlotA + t.lane * 16;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const bf16x8 w0 = *(const bf16x8*)(wbase + (b0 * 2 + q) * 1024);
        const bf16x8 w1 = *(const bf16x8*)(wbase + (b1 * 2 + q) * 1024);
        bf16x8 at[NTB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const int r = t.wm * 128 + tb * 32 + t.l32;
            const int c = (2 * q + t.half) ^ ((r >> 1) & 3);
            at[tb] = *(const bf16x8*)(base + r * 64 + c * 16);
        }
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, at[tb], acc[0][tb], 0, 0, 0);
            acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, at[tb], acc[1][tb], 0, 0, 0);
        }
    }
}

template <int EPI, int NTB>
__device__ __forceinline__ void epilogue(const LdsTile<EPI>& t, const f32x16 (&acc)[2][4]) {
    const GemmArgs& args = *t.args;
    const int N = t.N;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int rl = t.wm * 128 + tb * 32 + t.l32;
        if (rl >= t.valid) continue;
        const int r = t.row0 + rl;
        if (EPI == EPI_SWIGLU_BF16) {
            const float L = args.clamp_limit;
            uint16_t* orow = (uint16_t*)args.out + (size_t)r * N;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int n = t.n0 + 8 * qq + 4 * t.half;
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
                    const int n = t.n0 + 32 * b + 8 * qq + 4 * t.half;
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = acc[b][tb][4 * qq + i];
                    *(f32x4*)(orow + n) = v;
                }
        }
    }
}

// K loop of one tile for a wave computing NTB 32-row blocks (0: DMA only).
// Stages j+1 and j+2 stay in flight while stage j computes: wait for stage j
// (this wave's own DMA: at most 8 newer entries outstanding), barrier (all
// waves' DMA of stage j landed, and all waves are done reading the slot the
// next DMA overwrites), issue stage j+3, compute stage j.
template <int EPI, int NTB>
__device__ __forceinline__ void run_tile(const LdsTile<EPI>& t) {
    f32x16 acc[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;
    const int S = t.S;
    wait_vm<0>();  // retire the previous tile's stores before counting DMA entries
    issue_stage<EPI>(t, 0, 0);
    issue_stage<EPI>(t, min(1, S - 1), 1);
    issue_stage<EPI>(t, min(2, S - 1), 2);
    for (int j = 0; j < S; ++j) {
        wait_vm<8>();
        __syncthreads();
        issue_stage<EPI>(t, min(j + 3, S - 1), (j + 3) & 3);
        if constexpr (NTB > 0) compute_stage<EPI, NTB>(t, j & 3, acc);
    }
    wait_vm<0>();
    __syncthreads();
    if constexpr (NTB > 0) epilogue<EPI, NTB>(t, acc);
}

template <int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_lds_kernel(GemmArgs args) {
    extern __shared__ __align__(16) unsigned char smem[];
    int* tile_prefix = (int*)(smem + kSlots * kSlot);
    __shared__ int scan_sh[8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = args.G, rows = args.rows, K = args.K, N = args.N;
    const int* offs = args.offsets;

    // ---- per-group m-tile counts -> exclusive prefix in LDS ----
    {
        const int per = (G + kThreads - 1) / kThreads;
        const int g0 = tid * per;
        int local = 0;
        for (int g = g0; g < g0 + per && g < G; ++g) {
            int lo = 0, hi = rows;
            if (offs) {
                lo = min(max(offs[g], 0), rows);
                hi = max(lo, min(max(offs[g + 1], 0), rows));
            }
            const int mt = (hi - lo + TM - 1) / TM;
            tile_prefix[g] = mt;
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
        for (int w = 0; w < 8; ++w) {
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

    constexpr int kPanel = (EPI == EPI_SWIGLU_BF16) ? 128 : 256;  // packed panel rows
    const int NT = (N + kPanel - 1) / kPanel;
    const long long Q = (long long)tile_prefix[G] * NT;
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const long long q_lo = Q * xcd / 8, q_hi = Q * (xcd + 1) / 8;
    const size_t w_group = (size_t)NT * kPanel * K;   // packed elements per expert

    LdsTile<EPI> t;
    t.args = &args;
    t.smem = smem;
    t.lds0 = (uint32_t)(uintptr_t)smem;
    t.lane = lane;
    t.wave = wave;
    t.wm = wave >> 2;
    t.wn = wave & 3;
    t.half = lane >> 5;
    t.l32 = lane & 31;
    t.K = K;
    t.N = N;
    t.S = K / BK;

    for (long long q = q_lo + (blockIdx.x >> 3); q < q_hi; q += per_xcd) {
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
        t.row0 = grp_lo + m_tile * TM;
        t.grp_hi = grp_hi;
        t.valid = min(TM, grp_hi - t.row0);
        // weight panel of this n-tile: stage chunks of kPanel/32 blocks x 4 KB
        const size_t pbase = (size_t)g * w_group + (size_t)n_tile * kPanel * K;
        t.wsrc0 = args.w1 + pbase;
        t.wsrc1 = (EPI == EPI_SWIGLU_BF16 ? args.w2 : args.w1) + pbase;
        t.wstride = (size_t)(kPanel / 32) * 2048;
        t.n0 = (EPI == EPI_SWIGLU_BF16) ? n_tile * 128 + t.wn * 32 : n_tile * 256 + t.wn * 64;
        // this wave computes the valid 32-row blocks of its 128-row half
        const int wrows = min(max(t.valid - t.wm * 128, 0), 128);
        const bool wact = t.n0 < N;
        const int ntb = wact ? (wrows + 31) / 32 : 0;
        switch (ntb) {
            case 0: run_tile<EPI, 0>(t); break;
            case 1: run_tile<EPI, 1>(t); break;
            case 2: run_tile<EPI, 2>(t); break;
            case 3: run_tile<EPI, 3>(t); break;
            default: run_tile<EPI, 4>(t); break;
        }
    }
}

template <int EPI>
hipError_t launch_lds_epi(const GemmArgs& g, hipStream_t stream) {
    static int configured_device = -1;
    static int grid = 0;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const size_t lds = kSlots * kSlot + (size_t)(MOE_MAX_GROUPS + 1) * sizeof(int);
    if (configured_device != dev) {
        err = hipFuncSetAttribute((const void*)grouped_gemm_lds_kernel<EPI>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        grid = (device_cu_count() + 7) & ~7;
        configured_device = dev;
    }
    hipLaunchKernelGGL(grouped_gemm_lds_kernel<EPI>, dim3(grid), dim3(kThreads), lds, stream, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm_lds(int epilogue, const GemmArgs& g, hipStream_t stream) {
    switch (epilogue) {
        case EPI_SWIGLU_BF16: return launch_lds_epi<EPI_SWIGLU_BF16>(g, stream);
        case EPI_F32: return launch_lds_epi<EPI_F32>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
