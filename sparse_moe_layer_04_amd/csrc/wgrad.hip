// Grouped weight gradient ("HyperParallel accelerates DeepSeek-V4.1 ...",
// section 2.3, MegaMoE: the expert matmuls, whose weights a training step
// updates; section 03: the training run):
//   dw[g, m, k] = sum_{offsets[g] <= r < offsets[g+1]} dy[r, m] * a[r, k]
// for the forward out = a W_g^T per group.  dy [rows, M] and a [rows, K] bf16
// row-major, fp32 accumulation on the matrix cores, dw [G, M, K] fp32 (a group
// without rows gets zeros).  One kernel gives the expert down projection's
// dW_down = dY^T H, the gate/up matrices' dW_gate = dG^T X and dW_up = dU^T X,
// the shared expert's (one group) and the router projection's dW_g =
// dlogits^T x (one group of T rows).
//
// The contraction runs over each group's rows, the slow index of both inputs.
// A workgroup (4 waves) computes a 128 (m) x 128 (k) tile of one group's dw,
// walking the group's rows in chunks of 32:
//   - a chunk of dy (32 rows x 128 m) and of a (32 rows x 128 k) is loaded
//     two chunks ahead into registers (16-byte coalesced loads; rows past the
//     group end are zeros) and copied row-major into one of two LDS slots,
//     one barrier per chunk;
//   - the MFMA operands need 8 consecutive rows of one column per lane
//     (v_mfma_f32_32x32x16_bf16: operand A = a, so each lane's accumulator
//     holds 4 consecutive k of one m and the stores are 16 bytes); two LDS
//     transpose reads (ds_read_b64_tr_b16) give a lane its 8 rows from the
//     row-major chunk; LDS rows are padded to 288 bytes;
//   - wave (wm, wk) owns 64 m x 64 k (2 x 2 accumulators);
//   - the fp32 tile (64 KB, as many bytes as the tile reads at 128 rows, so
//     the writes dominate the traffic) leaves through LDS in two halves of
//     64 rows: every store instruction writes two whole 512-byte row
//     segments, non-temporal (the gradient is not read again by this step).
// Four waves per SIMD (the register budget is capped for it): a tile's
// chunks are few, so the memory latency is hidden by the other tiles.
// Grid: one workgroup per (group, m-tile, k-tile), mapped so that each XCD
// (workgroup id mod 8) takes a contiguous range of tiles: the tiles of one
// group share that XCD's L2 for their dy and a rows.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int WT = 128;                 // tile: m and k extent
constexpr int WR = 32;                  // rows per chunk
constexpr int kWThreads = 256;
constexpr int kWRow = WT * 2 + 32;      // LDS bytes per staged row (padded)
constexpr int kWOperand = WR * kWRow;   // one operand chunk
constexpr int kWSlot = 2 * kWOperand;   // dy + a chunk

struct WgradArgs {
    const uint16_t* dy;
    const uint16_t* a;
    const int32_t* offsets;  // [G + 1] or NULL (one group [0, rows))
    int G, rows, M, K;
    int ld_dy, ld_a;         // row strides (elements) of dy and a
    int mt, kt;              // tiles per group along m and k
    long long tiles;         // G * mt * kt
    float* dw;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The MFMA operand of lane l from a staged row-major chunk: rows row0 +
// 8 (l / 32) + t (t = 0..7) of column col0 + l % 32, by two LDS transpose
// reads.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane j of a group
// receives 16-bit element j % 4 of the 8-byte pieces addressed by lanes
// 4 m + j / 4 of the group, m = 0..3 (established on the GPU by a one-wave
// probe).  Lane i of group gp therefore addresses row i / 4 (of the group's
// 4-row block) and columns 16 (gp % 2) + 4 (i % 4) .. + 3, so lane j's
// values are 4 consecutive rows of column 16 (gp % 2) + j.
__device__ __forceinline__ bf16x8 gather8(const unsigned char* chunk, int row0, int col0,
                                          int lane) {
    const int gp = lane >> 4, i = lane & 15;
    const int r = row0 + 8 * (gp >> 1) + (i >> 2);
    const int c = col0 + 16 * (gp & 1) + 4 * (i & 3);
    const unsigned char* p = chunk + r * kWRow + c * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * kWRow));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void grouped_wgrad_kernel(WgradArgs args) {
    __shared__ __align__(16) unsigned char lds[2 * kWSlot];
    // XCD-contiguous tile order: workgroup b runs on XCD b % 8
    const long long per = (long long)gridDim.x / 8;
    const long long tile = (long long)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (tile >= args.tiles) return;
    const int kt_i = (int)(tile % args.kt);
    const int mt_i = (int)((tile / args.kt) % args.mt);
    const int g = (int)(tile / ((long long)args.kt * args.mt));
    const int M = args.M, K = args.K;
    const int m0 = mt_i * WT, k0 = kt_i * WT;
    int lo = 0, hi = args.rows;
    if (args.offsets) {
        lo = min(max(args.offsets[g], 0), args.rows);
        hi = max(lo, min(max(args.offsets[g + 1], 0), args.rows));
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wk = wave & 1;
    const int half = lane >> 5, l32 = lane & 31;

    f32x16 acc[2][2];   // [k block][m block]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // staging: thread tid copies 16-byte chunk (tid % 16) of chunk rows
    // tid / 16 and tid / 16 + 16 of both operands (columns past M / K and rows
    // past the group end stage zeros)
    const int sc = tid & 15, sr = tid >> 4;
    const int cm = m0 + 8 * sc, ck = k0 + 8 * sc;
    const bool m_in = cm < M, k_in = ck < K;
    u32x4 st[2][2][2];  // [register set][operand: dy, a][row group]
    auto load_chunk = [&](int r0, auto set) {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = r0 + sr + 16 * i;
            const bool in = r < hi;
            u32x4 z = {0u, 0u, 0u, 0u};
            st[S][0][i] = (in && m_in) ? *(const u32x4*)(args.dy + (size_t)r * args.ld_dy + cm) : z;
            st[S][1][i] = (in && k_in) ? *(const u32x4*)(args.a + (size_t)r * args.ld_a + ck) : z;
        }
    };
    auto store_chunk = [&](int slot, auto set) {
        constexpr int S = decltype(set)::value;
        unsigned char* base = lds + slot * kWSlot;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *(u32x4*)(base + (sr + 16 * i) * kWRow + sc * 16) = st[S][0][i];
            *(u32x4*)(base + kWOperand + (sr + 16 * i) * kWRow + sc * 16) = st[S][1][i];
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // chunk c is staged from register set c % 2 into LDS slot c % 2; its
    // global loads are issued two chunks ahead
    const int nchunks = (hi - lo + WR - 1) / WR;
    if (nchunks > 0) load_chunk(lo, I0());
    if (nchunks > 1) load_chunk(lo + WR, I1());
    if (nchunks > 0) store_chunk(0, I0());
    auto step = [&](int c, auto par) {
        constexpr int P = decltype(par)::value;
        __syncthreads();
        if (c + 2 < nchunks) load_chunk(lo + (c + 2) * WR, par);
        const unsigned char* dyc = lds + P * kWSlot;
        const unsigned char* ac = dyc + kWOperand;
#pragma unroll
        for (int s = 0; s < WR / 16; ++s) {
            bf16x8 fa[2], fd[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i] = gather8(ac, 16 * s, 64 * wk + 32 * i, lane);
                fd[i] = gather8(dyc, 16 * s, 64 * wm + 32 * i, lane);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fd[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (c + 1 < nchunks) store_chunk(P ^ 1, std::integral_constant<int, P ^ 1>());
    };
    for (int c = 0; c < nchunks; c += 2) {
        step(c, I0());
        if (c + 1 < nchunks) step(c + 1, I1());
    }

    // output through LDS in two halves of 64 m rows (the chunk slots hold
    // 64 rows x 128 k fp32): the waves of half wm write their accumulators
    // (element e of lane l: k = 8 (e / 4) + 4 half + e % 4 of the k block,
    // m = l32 of the m block), then all 256 threads store whole 512-byte row
    // segments
    float* out = args.dw + (size_t)g * M * K;
    constexpr int kORow = WT * 4 + 16;
    static_assert(64 * kORow <= 2 * kWSlot, "output half fits the chunk slots");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __syncthreads();
        if (wm == h) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        f32x4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * qq + e];
                        const int r = 32 * j + l32;
                        const int kk = 64 * wk + 32 * i + 8 * qq + 4 * half;
                        *(f32x4*)(lds + r * kORow + kk * 4) = v;
                    }
        }
        __syncthreads();
        const int c4 = tid & 31;
        const int k = k0 + 4 * c4;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int r = 8 * p + (tid >> 5);
            const int m = m0 + 64 * h + r;
            if (m < M && k < K) {
                const f32x4 v = *(const f32x4*)(lds + r * kORow + c4 * 16);
                __builtin_nontemporal_store(v, (f32x4*)(out + (size_t)m * K + k));
            }
        }
    }
}

}  // namespace

hipError_t launch_grouped_wgrad(const uint16_t* dy, const uint16_t* a, const int32_t* offsets,
                                int G, int rows, int M, int K, float* dw, hipStream_t stream,
                                int ld_dy, int ld_a) {
    WgradArgs args;
    args.ld_dy = ld_dy > 0 ? ld_dy : M;
    args.ld_a = ld_a > 0 ? ld_a : K;
    if (args.ld_dy < M || args.ld_a < K || args.ld_dy % 8 || args.ld_a % 8)
        return hipErrorInvalidValue;
    args.dy = dy;
    args.a = a;
    args.offsets = offsets;
    args.G = G;
    args.rows = rows;
    args.M = M;
    args.K = K;
    args.mt = (M + WT - 1) / WT;
    args.kt = (K + WT - 1) / WT;
    args.tiles = (long long)G * args.mt * args.kt;
    args.dw = dw;
    const long long per = (args.tiles + 7) / 8;
    if (8 * per > 0x7fffffffll) return hipErrorInvalidValue;
    hipLaunchKernelGGL(grouped_wgrad_kernel, dim3((unsigned)(8 * per)), dim3(kWThreads), 0, stream,
                       args);
    return hipGetLastError();
}

}  // namespace moe
