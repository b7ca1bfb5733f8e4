// Grouped expert GEMM on packed bf16 weights, "flat" form: weights stream
// from memory straight into the MFMA operand registers of the one wave that
// uses them; only the activation rows go through LDS ("HyperParallel
// accelerates DeepSeek-V4.1 ...", section 2.3, MegaMoE: the two expert
// matmuls and the clamped SwiGLU between them).
//
// Problem: for each expert g and activation row r in [lo_g, hi_g),
//   out[r, n] = sum_k A[r, k] * W[g, n, k]
// with W in the moe_pack_weights panel layout (P = 128 rows for the gate and
// up matrices, P = 256 for the down matrix) and A row-major, in the blocked
// activation layout, or gathered (row r of A is row gather[r] of a row-major
// matrix: the dispatch permutation applied while loading).
//
// Why this shape.  With a few hundred rows per expert the expert GEMMs are
// bound by streaming the weights from HBM: every weight element is used
// against all rows of its tile, once.  So:
//   - a tile is up to 128 activation rows x 512 weight rows (SwiGLU: 256
//     features x {gate, up}); wave w of the 8 owns 64 weight rows (SwiGLU: the
//     gate and up rows of 32 features, so the epilogue needs no exchange;
//     down: two 32-row blocks) against every row of the tile: up to 2 x 4
//     MFMA 32x32 accumulators per wave;
//   - each weight element feeds exactly one wave, so the packed 1 KB
//     fragments (one per 16-wide K substep and 32-row block, lane-ordered)
//     are loaded by that wave straight into its operand registers, one
//     64-wide stage (4 substeps) ahead: plain coalesced 16-byte loads, no
//     LDS round trip and no second read of the weights by another wave;
//   - the activation rows are shared by all 8 waves, so they go through a
//     2-slot LDS ring: each stage (128 rows x 64 columns, 16 KB) is loaded
//     into registers two stages ahead and written to LDS one stage ahead,
//     one barrier per stage.  512 weight rows per tile halve how often an
//     expert's rows are restaged compared with 256-row tiles.
// Every memory operation is an ordinary compiler-visible load or store, so
// the compiler's vmcnt/lgkmcnt waits are exact; loads past the end of K or of
// a group read clamped, valid addresses so the load count per stage is fixed.
//
// LDS swizzle: row r of a slot is 128 bytes (8 chunks of 16 B); chunk c is
// stored at c ^ ((r >> 1) & 7), so the 16 lanes one LDS cycle serves in an
// MFMA operand read (16 rows of one chunk index) hit distinct banks.
//
// Scheduling: persistent grid (one workgroup per CU); every workgroup builds
// the per-expert item prefix in LDS from the device offsets; items are
// ordered (expert, n-tile, m-tile), the 8 XCDs take contiguous ranges of
// equal item count and inside an XCD the workgroups claim items from a
// per-XCD counter (or, without counters, take every (grid/8)-th item).
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int FM = 128;                  // activation rows per tile
constexpr int FN = 512;                  // weight rows per tile
constexpr int FK = 64;                   // K columns per stage
constexpr int FQ = FK / 16;              // MFMA substeps per stage
constexpr int FNTB = FM / 32;            // 32-row activation blocks per tile
constexpr int kFThreads = 512;           // 8 waves
constexpr int kRowBytes = FK * 2;        // LDS bytes per activation row
constexpr int kSlotBytes = FM * kRowBytes;
constexpr int kRingBytes = 2 * kSlotBytes;
// fp32 epilogue staging: one 32-row block of the tile's outputs, rows padded
// by 16 bytes so that the 32 rows one MFMA accumulator spans land in
// distinct banks
constexpr int kEpiRow = FN * 4 + 16;
constexpr int kEpiBytes = 32 * kEpiRow;
// A8W4: fp8 activations, 128 K columns per stage (128 bytes per row, the
// bf16 stage's slot size) and their scale bytes (4 MX blocks per row)
constexpr int FK8 = 128;
constexpr int kScaleSlot = FM * 4;
constexpr int kLdsFixed = kRingBytes + kEpiBytes + 2 * kScaleSlot;
constexpr int kFLdsLimit = 160 * 1024;
constexpr int kFStaticLds = 256;

enum FAMode : int { FA_ROW = 0, FA_BLK = 1, FA_GATHER = 2 };

template <int EPI>
struct FPanel {
    static constexpr int P = (EPI == EPI_SWIGLU_BF16) ? 128 : 256;  // packed panel rows
    static constexpr int BPP = P / 32;                               // 32-row blocks per panel
    // outputs (features for SwiGLU, output rows for down) per tile
    static constexpr int TN = (EPI == EPI_SWIGLU_BF16) ? FN / 2 : FN;
};

__device__ __forceinline__ float fclamp_sym(float v, float L) { return fminf(fmaxf(v, -L), L); }

__device__ __forceinline__ int fswz(int r) { return (r >> 1) & 7; }

// Buffer resource over [base, base + bytes), base and bytes wave-uniform
// (read from the first lane, so the resource lives in scalar registers):
// the weight loads address their panel as a scalar base plus the lane's
// 16-byte offset and a scalar stage offset, which keeps the 64-bit address
// arithmetic out of the vector registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t flat_rsrc(const void* base, size_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)min(bytes, (size_t)0x7fffffff));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), 0, n,
                                             0x00020000);
}

// Per-workgroup state of one tile.
struct FlatTile {
    int lane, wave, half, l32, tid;
    int K, N;
    int row0, valid;       // first activation row of the tile, rows in it
    int ntb;               // 32-row activation blocks holding a valid row
    int n0;                // first output (feature / output row) of this wave
    const uint16_t* wp0;   // this wave's block-0 fragments at stage 0 (lane offset included)
    const uint16_t* wp1;   // block 1 (SwiGLU: the up block)
    size_t wstage;         // elements per 64-wide K stage of one panel
    size_t a_off[2];       // this thread's activation source (elements) at stage 0
    int a_rows;            // activation rows this thread stages (0..2, wave-uniform)
    int a_step;            // elements per stage of the activation source
    // MXFP8 / MXFP4 weights: this wave's code chunks and scale bytes
    const uint8_t* cp0;    // block 0 codes at K block 0 (lane offset included)
    const uint8_t* cp1;    // block 1
    size_t cstage;         // fp8: bytes per 64-wide K stage of a panel; fp4: per K block
    const uint8_t* sp0;    // block 0 scale byte of this lane's row at K block 0
    const uint8_t* sp1;
    int sstep;             // scale bytes per K block (the panel's rows)
    size_t s_off;          // A8W4: scale bytes of the activation row this thread stages
};

template <int NTB>
struct FOps {
    bf16x8 a[NTB];
};

// activation fragments of substep q (one 16-wide K slice) of the slot
template <int NTB>
__device__ __forceinline__ void read_act(const unsigned char* slot, const FlatTile& t, int q,
                                         FOps<NTB>& o) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int r = tb * 32 + t.l32;
        const int c = (2 * q + t.half) ^ fswz(r);
        o.a[tb] = *(const bf16x8*)(slot + r * kRowBytes + c * 16);
    }
}

template <int NTB>
__device__ __forceinline__ void mfma_step(const bf16x8& w0, const bf16x8& w1, const FOps<NTB>& o,
                                          f32x16 (&acc)[2][FNTB]) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, o.a[tb], acc[0][tb], 0, 0, 0);
        acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, o.a[tb], acc[1][tb], 0, 0, 0);
    }
}

// fp32 outputs (down projection): each 32-row block goes through LDS so that
// every store instruction writes 1 KB of one output row (the accumulator
// layout gives each lane 16 bytes in each of 32 rows 4 * N bytes apart).
// Barrier-uniform: every wave runs it whatever its columns.  NT_OUT: stores
// with the streaming hint (the routed expert outputs, larger than the caches
// and read once by the combine).
template <int NTB, bool NT_OUT>
__device__ __forceinline__ void flat_epilogue_f32(const GemmArgs& args, const FlatTile& t,
                                                  const f32x16 (&acc)[2][FNTB],
                                                  unsigned char* stg) {
    const int N = t.N;
    const int nl0 = 64 * t.wave;                   // this wave's first column in the tile
    const int nbase = t.n0 - nl0;                  // the tile's first output column
    float* out = (float*)args.out;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        __syncthreads();                           // the previous block's reads are done
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int c = nl0 + 32 * b + 8 * qq + 4 * t.half;
                f32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = acc[b][tb][4 * qq + i];
                *(f32x4*)(stg + t.l32 * kEpiRow + c * 4) = v;
            }
        __syncthreads();
        // wave w stores rows 4 w .. 4 w + 3 of the block: 2 x 1 KB per row
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = 4 * t.wave + rr;
            const int rl = tb * 32 + row;
            if (rl >= t.valid) continue;
            float* orow = out + (size_t)(t.row0 + rl) * N + nbase;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 256 * h + 4 * t.lane;
                if (nbase + c < N) {
                    const f32x4 v = *(const f32x4*)(stg + row * kEpiRow + c * 4);
                    if constexpr (NT_OUT) {
                        __builtin_nontemporal_store(v, (f32x4*)(orow + c));
                    } else {
                        *(f32x4*)(orow + c) = v;
                    }
                }
            }
        }
    }
}

template <int EPI, int AM, int NTB>
__device__ __forceinline__ void flat_epilogue(const GemmArgs& args, const FlatTile& t,
                                              const f32x16 (&acc)[2][FNTB]) {
    const int N = t.N;
    if (t.n0 >= N) return;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int rl = tb * 32 + t.l32;
        if (rl >= t.valid) continue;
        const size_t r = (size_t)(t.row0 + rl);
        if constexpr (EPI == EPI_SWIGLU_BF16) {
            const float L = args.clamp_limit;
            uint16_t* out = (uint16_t*)args.out;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int n = t.n0 + 8 * qq + 4 * t.half;
                if (args.out_g) {
                    // the fp32 pre-activations, before the clamps (saved for
                    // the backward)
                    f32x4 gs, us;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        gs[i] = acc[0][tb][4 * qq + i];
                        us[i] = acc[1][tb][4 * qq + i];
                    }
                    *(f32x4*)(args.out_g + r * N + n) = gs;
                    *(f32x4*)(args.out_u + r * N + n) = us;
                }
                uint32_t packed[2];
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    uint16_t hb[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        float gv = acc[0][tb][4 * qq + i + u];
                        float uv = acc[1][tb][4 * qq + i + u];
                        gv = args.clamp_mode == MOE_CLAMP_SYMMETRIC ? fclamp_sym(gv, L)
                                                                    : fminf(gv, L);
                        uv = fclamp_sym(uv, L);
                        const float silu = gv / (1.0f + __expf(-gv));
                        hb[u] = f32_to_bf16(silu * uv);
                    }
                    packed[i >> 1] = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
                }
                uint16_t* dst = AM != FA_ROW ? out + blocked_index(r, n, N) : out + r * N + n;
                *(u32x2*)dst = u32x2{packed[0], packed[1]};
            }
        } else {
            float* orow = (float*)args.out + r * N;
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

// Pipeline depths (defaults; the build may override them):
//   FLAT_R   weight substeps in flight per wave (register ring; 4 or 8)
//   FLAT_AD  stages the activation loads run ahead of their LDS write (1, 2)
//   FLAT_OB  activation operand buffers (2: read one substep ahead)
#ifndef FLAT_R
#define FLAT_R 4
#endif
#ifndef FLAT_AD
#define FLAT_AD 2
#endif
#ifndef FLAT_OB
#define FLAT_OB 2
#endif

// K loop and epilogue of one tile for NTB valid 32-row blocks.
//   stage j: barrier (slot j % 2 holds stage j); load the activations of
//   stage j + AD into registers; for each substep u = 4 j + q: read its
//   activation fragments from LDS and multiply (with two operand buffers the
//   multiply lags the read by one substep, so every LDS read latency hides
//   behind the other substep's MFMAs); after the MFMAs of substep u, its weight
//   register slot (u % R) takes the weights of substep u + R.  Finally stage
//   j + 1's activations (loaded AD - 1 stages earlier) go to slot (j + 1) % 2.
// The stage loop is unrolled by two, so every ring index is static.
template <int EPI, int AM, int NTB, int WF>
__device__ __forceinline__ void flat_tile(const GemmArgs& args, const FlatTile& t,
                                          unsigned char* ring) {
    // (MX weights: one stage of code chunks in flight, operands read one
    // substep ahead)
    constexpr int R = WF ? 4 : FLAT_R, AD = FLAT_AD, OB = WF ? 2 : FLAT_OB;
    static_assert(R == 4 || R == 8, "weight ring of one or two stages");
    static_assert(AD == 1 || AD == 2, "activation depth");
    static_assert(OB == 1 || OB == 2, "operand buffers");
    f32x16 acc[2][FNTB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int tb = 0; tb < FNTB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;
    const int S = t.K / FK;
    const uint16_t* a = args.a;

    bf16x8 w0[WF ? 1 : R], w1[WF ? 1 : R];
    u32x4 areg[AD][2];
    // MX weights: the code chunks (32 K columns = one MX block, both of its
    // substeps) of one stage for both blocks, and their scale bytes X + 127
    using CodeT = typename std::conditional<WF == 2, u32x2, u32x4>::type;
    CodeT cw0[2], cw1[2];
    uint32_t sc0[2], sc1[2];
    // (through buffer resources over the blocks' codes and scale bytes, as
    // the bf16 weights: the lane offsets are t.lane * 16 or 8 bytes of code
    // and t.l32 scale bytes; a panel of codes stays under 2 GiB for K up to
    // kFlatMaxK)
    const int lane_c = t.lane * (WF == 1 ? 16 : 8);
    const __amdgpu_buffer_rsrc_t cr0 = flat_rsrc(t.cp0 - lane_c, (size_t)0x7fffffff);
    const __amdgpu_buffer_rsrc_t cr1 = flat_rsrc(t.cp1 - lane_c, (size_t)0x7fffffff);
    const __amdgpu_buffer_rsrc_t sr0 = flat_rsrc(t.sp0 - t.l32, (size_t)0x7fffffff);
    const __amdgpu_buffer_rsrc_t sr1 = flat_rsrc(t.sp1 - t.l32, (size_t)0x7fffffff);
    auto load_c = [&](int j, int c) {
        const int jj = min(j, S - 1);
        const int kb = 2 * jj + c;
        const int off = WF == 1 ? jj * (int)t.cstage + c * 1024 : kb * (int)t.cstage;
        if constexpr (WF == 1) {
            cw0[c] = __builtin_bit_cast(CodeT, __builtin_amdgcn_raw_buffer_load_b128(cr0, lane_c, off, 0));
            cw1[c] = __builtin_bit_cast(CodeT, __builtin_amdgcn_raw_buffer_load_b128(cr1, lane_c, off, 0));
        } else if constexpr (WF == 2) {
            cw0[c] = __builtin_bit_cast(CodeT, __builtin_amdgcn_raw_buffer_load_b64(cr0, lane_c, off, 0));
            cw1[c] = __builtin_bit_cast(CodeT, __builtin_amdgcn_raw_buffer_load_b64(cr1, lane_c, off, 0));
        }
        sc0[c] = __builtin_amdgcn_raw_buffer_load_b8(sr0, t.l32, kb * t.sstep, 0);
        sc1[c] = __builtin_amdgcn_raw_buffer_load_b8(sr1, t.l32, kb * t.sstep, 0);
    };
    // the bf16 operands of substep pq of the stage in the code ring: exact
    // (the scaled code is a bf16 value)
    auto decode = [&](int pq, bf16x8& d0, bf16x8& d1) {
        const int c = pq >> 1, hh = pq & 1;
        const float f0 = __uint_as_float(sc0[c] << 23), f1 = __uint_as_float(sc1[c] << 23);
        if constexpr (WF == 1) {
            d0 = fp8x8_to_bf16x8(u32x2{cw0[c][2 * hh], cw0[c][2 * hh + 1]}, f0);
            d1 = fp8x8_to_bf16x8(u32x2{cw1[c][2 * hh], cw1[c][2 * hh + 1]}, f1);
        } else if constexpr (WF == 2) {
            d0 = fp4x8_to_bf16x8(cw0[c][hh], f0);
            d1 = fp4x8_to_bf16x8(cw1[c][hh], f1);
        }
    };

    // weights of global substep u (stage u / 4, substep u % 4), clamped to K,
    // through buffer resources over this wave's two blocks (the launch keeps
    // a panel under 2 GiB)
    const size_t wbytes = (size_t)S * t.wstage * 2;
    const __amdgpu_buffer_rsrc_t wr0 = flat_rsrc(t.wp0 - t.lane * 8, wbytes);
    const __amdgpu_buffer_rsrc_t wr1 = flat_rsrc(t.wp1 - t.lane * 8, wbytes);
    auto load_w = [&](int u, bf16x8& d0, bf16x8& d1) {
        const int j = min(u >> 2, S - 1);
        const int so = (int)(((size_t)j * t.wstage + (size_t)(u & 3) * 512) * 2);
        d0 = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wr0, t.lane * 16, so, 0));
        d1 = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wr1, t.lane * 16, so, 0));
    };
    auto load_a = [&](int j, u32x4 (&d)[2]) {
        const size_t off = (size_t)min(j, S - 1) * t.a_step;
        d[0] = *(const u32x4*)(a + t.a_off[0] + off);
        if (t.a_rows > 1) d[1] = *(const u32x4*)(a + t.a_off[1] + off);
    };
    auto store_a = [&](int j, const u32x4 (&d)[2]) {
        unsigned char* slot = ring + (j & 1) * kSlotBytes;
        const int c = t.tid & 7;
        const int r0 = t.tid >> 3;
        *(u32x4*)(slot + r0 * kRowBytes + ((c ^ fswz(r0)) << 4)) = d[0];
        if (t.a_rows > 1) {
            const int r1 = r0 + 64;
            *(u32x4*)(slot + r1 * kRowBytes + ((c ^ fswz(r1)) << 4)) = d[1];
        }
    };

    // prologue: weights of substeps 0 .. R - 1; activations of stages
    // 0 .. AD - 1 (stage 0 into slot 0)
    if constexpr (WF) {
        load_c(0, 0);
        load_c(0, 1);
    } else {
#pragma unroll
        for (int u = 0; u < R; ++u) load_w(u, w0[u], w1[u]);
    }
    if (t.a_rows > 0) {
#pragma unroll
        for (int p = 0; p < AD; ++p) load_a(p, areg[p]);
        store_a(0, areg[0]);
    }

    FOps<NTB> o[OB];
    auto stage = [&](int j, auto par) {
        constexpr int P = decltype(par)::value;   // j % 2
        __syncthreads();
        const unsigned char* slot = ring + P * kSlotBytes;
        // activation registers: stage j's set was written to LDS at the end
        // of stage j - 1; it now takes stage j + AD
        if (t.a_rows > 0) load_a(j + AD, areg[AD == 2 ? P : 0]);
#pragma unroll
        for (int q = 0; q < FQ; ++q) {
            const int u = 4 * j + q;
            if constexpr (OB == 2) {
                read_act<NTB>(slot, t, q, o[q & 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (q > 0 || j > 0) {
                    if constexpr (WF) {
                        // previous substep pq of stage jp; after the second
                        // substep of a code chunk the chunk takes stage jp + 1
                        const int pq = (q + 3) & 3;
                        const int jp = q > 0 ? j : j - 1;
                        bf16x8 d0, d1;
                        decode(pq, d0, d1);
                        mfma_step<NTB>(d0, d1, o[(q + 1) & 1], acc);
                        if (pq & 1) load_c(jp + 1, pq >> 1);
                    } else {
                        // previous substep u - 1, its weight slot, then refill
                        const int ps = (P * 4 + q + R - 1) % R;
                        mfma_step<NTB>(w0[ps], w1[ps], o[(q + 1) & 1], acc);
                        load_w(u - 1 + R, w0[ps], w1[ps]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
                read_act<NTB>(slot, t, q, o[0]);
                const int cs = (P * 4 + q) % R;
                mfma_step<NTB>(w0[cs], w1[cs], o[0], acc);
                load_w(u + R, w0[cs], w1[cs]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (t.a_rows > 0 && j + 1 < S) {
            if constexpr (AD == 2) {
                store_a(j + 1, areg[P ^ 1]);
            } else {
                store_a(j + 1, areg[0]);
            }
        }
        // the last substep of the K loop (its operands were read at q = 3)
        if constexpr (OB == 2) {
            if (j == S - 1) {
                if constexpr (WF) {
                    bf16x8 d0, d1;
                    decode(3, d0, d1);
                    mfma_step<NTB>(d0, d1, o[1], acc);
                } else {
                    constexpr int ls = (P * 4 + 3) % R;
                    mfma_step<NTB>(w0[ls], w1[ls], o[1], acc);
                }
            }
        }
    };
    for (int j = 0; j < S; j += 2) {
        stage(j, std::integral_constant<int, 0>());
        if (j + 1 < S) stage(j + 1, std::integral_constant<int, 1>());
    }
    if constexpr (EPI == EPI_F32) {
        // (the blocked activations are the routed h of the forward)
        flat_epilogue_f32<NTB, AM == FA_BLK>(args, t, acc, ring + kRingBytes);
    } else {
        flat_epilogue<EPI, AM, NTB>(args, t, acc);
    }
}

// ---------------------------------------------------------------- A8W4 ----
// MXFP8 activations x MXFP4 weights on the scaled MX matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4: D[n, t] += sum over 64 K of A[n, k]
// 2^(sa - 127) B[k, t] 2^(sb - 127), the scales per 32-wide K block).
// Operand lanes (lane l: row / column l % 32, h = l / 32):
//   A, E2M1 weights: the 32 values K [32 h, 32 h + 32) of the step, 8 per
//     dword, low nibble first (dwords 0-3);
//   B, E4M3 activations: bytes 0-15 are K [16 h, 16 h + 16), bytes 16-31 are
//     K [32 + 16 h, 32 + 16 h + 16);
//   scale operand of lane l: the E8M0 scale of K block h of its row / column.
// The MXFP4 packed weights hold, per K block and 32-row block, 8 bytes for
// lane l' (row l' % 32): K [8 h', 8 h' + 8) and [16 + 8 h', 16 + 8 h' + 8);
// lane (n, h) therefore takes the bytes of lanes n and n + 32 of block
// 4 j + 2 s + h (stage j, step s) and interleaves their dwords into K order.
// Each output accumulates over ascending 64-wide steps; the accumulator
// layout is the bf16 kernel's, so the epilogues are shared (SwiGLU writes h
// as MXFP8 codes and scales for the down projection).
// activation operands of step s of the stage in `slot` (32 bytes per lane
// per 32-row block); the scale operands come from one 4-byte word per row
template <int NTB>
__device__ __forceinline__ void read_b8(const unsigned char* slot, const FlatTile& t, int s,
                                        v8i (&b)[NTB]) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int r = tb * 32 + t.l32;
        const int c1 = (4 * s + t.half) ^ fswz(r), c2 = (4 * s + 2 + t.half) ^ fswz(r);
        const u32x4 lo = *(const u32x4*)(slot + r * kRowBytes + (c1 << 4));
        const u32x4 hi = *(const u32x4*)(slot + r * kRowBytes + (c2 << 4));
        b[tb] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
}

// the 2 x NTB scaled MFMAs of step S.  The weight fragments stay as loaded
// (the bytes of lanes n and n + 32: two u32x2 per block) until here, where
// they are interleaved into K order two stages after their loads were
// issued (interleaving them at load time made the moves wait on the loads
// just issued); the weight scale bytes sit alone in their registers; the
// activation scale words are shifted so that byte 2 S is this lane's block.
template <int NTB, int S>
__device__ __forceinline__ void mfma_a8w4(const u32x2 (&w)[2][2], const uint32_t (&ws)[2],
                                          const v8i (&b)[NTB], const uint32_t (&as)[NTB],
                                          f32x16 (&acc)[2][FNTB]) {
    const v8i a0 = {(int)w[0][0][0], (int)w[0][1][0], (int)w[0][0][1], (int)w[0][1][1],
                    0, 0, 0, 0};
    const v8i a1 = {(int)w[1][0][0], (int)w[1][1][0], (int)w[1][0][1], (int)w[1][1][1],
                    0, 0, 0, 0};
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        acc[0][tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a0, b[tb], acc[0][tb], 4, 0, 0, (int)ws[0], 2 * S, (int)as[tb]);
        acc[1][tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a1, b[tb], acc[1][tb], 4, 0, 0, (int)ws[1], 2 * S, (int)as[tb]);
    }
}

// SwiGLU epilogue of the A8W4 gate/up GEMM: h = SwiGLU(clamped g, u) rounded
// to bf16 (as the bf16 path's h), then MXFP8 along the features: the wave's
// 32 features of a row are one MX block, held by lanes l and l ^ 32.
template <int NTB>
__device__ __forceinline__ void flat_epilogue_h8(const GemmArgs& args, const FlatTile& t,
                                                 const f32x16 (&acc)[2][FNTB]) {
    const int N = t.N;
    if (t.n0 >= N) return;                         // (wave-uniform)
    const float L = args.clamp_limit;
    uint8_t* out = (uint8_t*)args.out;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        float hv[16];
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float gv = acc[0][tb][e], uv = acc[1][tb][e];
            gv = args.clamp_mode == MOE_CLAMP_SYMMETRIC ? fclamp_sym(gv, L) : fminf(gv, L);
            uv = fclamp_sym(uv, L);
            const float silu = gv / (1.0f + __expf(-gv));
            hv[e] = bf16_to_f32(f32_to_bf16(silu * uv));
            amax = fmaxf(amax, fabsf(hv[e]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int X = mx8_exponent(amax);
        const float inv = __builtin_ldexpf(1.0f, -X);
        const int rl = tb * 32 + t.l32;
        if (rl >= t.valid) continue;
        const size_t r = (size_t)(t.row0 + rl);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) word |= e4m3_rne(hv[4 * qq + i] * inv) << (8 * i);
            *(uint32_t*)(out + r * N + t.n0 + 8 * qq + 4 * t.half) = word;
        }
        if (t.half == 0) args.out_scale[r * (N / 32) + t.n0 / 32] = (uint8_t)(X + 127);
    }
}

// K loop and epilogue of one A8W4 tile: 128-wide stages, one barrier each;
// per stage and wave two 64-wide steps of 2 x NTB scaled MFMAs.  The
// activation codes (and scale words) of stage j + 2 are loaded during stage
// j and written to LDS at the end of stage j + 1; the weights of stage j + 2
// are loaded into the register set of stage j right after its MFMAs.
template <int EPI, int AM, int NTB>
__device__ __forceinline__ void flat_tile_a8(const GemmArgs& args, const FlatTile& t,
                                             unsigned char* ring) {
    f32x16 acc[2][FNTB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int tb = 0; tb < FNTB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;
    const int S = t.K / FK8;
    const uint8_t* a8 = args.a8;
    unsigned char* sring = ring + kRingBytes + kEpiBytes;

    u32x2 wq[2][2][2][2];    // [set][step][block][bytes of lane n, lane n + 32]
    uint32_t wsc[2][2][2];   // [set][step][block] scale byte
    auto load_w = [&](int j, auto set) {
        constexpr int W = decltype(set)::value;
        const int jj = min(j, S - 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const size_t kb = (size_t)(4 * jj + 2 * s);
            const size_t off = kb * t.cstage;
            wq[W][s][0][0] = *(const u32x2*)(t.cp0 + off);
            wq[W][s][0][1] = *(const u32x2*)(t.cp0 + off + 256);
            wq[W][s][1][0] = *(const u32x2*)(t.cp1 + off);
            wq[W][s][1][1] = *(const u32x2*)(t.cp1 + off + 256);
            wsc[W][s][0] = t.sp0[kb * t.sstep];
            wsc[W][s][1] = t.sp1[kb * t.sstep];
        }
    };
    u32x4 areg[2][2];
    uint32_t sreg[2];
    auto load_a = [&](int j, u32x4 (&d)[2], uint32_t& sd) {
        // (unconditional: clamped rows are valid addresses, and the same
        // load count on every path keeps the compiler's vmcnt waits from
        // falling to the shortest path's; measured 6% faster)
        const size_t jj = (size_t)min(j, S - 1);
        d[0] = *(const u32x4*)(a8 + t.a_off[0] + jj * FK8);
        d[1] = *(const u32x4*)(a8 + t.a_off[1] + jj * FK8);
        sd = *(const uint32_t*)(args.a_scale + t.s_off + 4 * jj);
    };
    auto store_a = [&](int j, const u32x4 (&d)[2], uint32_t sd) {
        unsigned char* slot = ring + (j & 1) * kSlotBytes;
        const int c = t.tid & 7;
        const int r0 = t.tid >> 3;
        if (t.a_rows > 0) *(u32x4*)(slot + r0 * kRowBytes + ((c ^ fswz(r0)) << 4)) = d[0];
        if (t.a_rows > 1) {
            const int r1 = r0 + 64;
            *(u32x4*)(slot + r1 * kRowBytes + ((c ^ fswz(r1)) << 4)) = d[1];
        }
        if (t.tid < FM) *(uint32_t*)(sring + (j & 1) * kScaleSlot + t.tid * 4) = sd;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // (the loads in the order of the loop's own, so that the waits at the
    // loop head are the steady state's)
    load_a(0, areg[0], sreg[0]);
    load_w(0, I0());
    load_a(1, areg[1], sreg[1]);
    load_w(1, I1());
    store_a(0, areg[0], sreg[0]);

    v8i b[NTB];
    uint32_t as[NTB];
    auto stage = [&](int j, auto par) {
        constexpr int P = decltype(par)::value;   // j % 2
        __syncthreads();
        const unsigned char* slot = ring + P * kSlotBytes;
        const unsigned char* sslot = sring + P * kScaleSlot;
        load_a(j + 2, areg[P], sreg[P]);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
            as[tb] = *(const uint32_t*)(sslot + (tb * 32 + t.l32) * 4) >> (8 * t.half);
        read_b8<NTB>(slot, t, 0, b);
        mfma_a8w4<NTB, 0>(wq[P][0], wsc[P][0], b, as, acc);
        read_b8<NTB>(slot, t, 1, b);
        mfma_a8w4<NTB, 1>(wq[P][1], wsc[P][1], b, as, acc);
        load_w(j + 2, par);
        if (j + 1 < S) store_a(j + 1, areg[P ^ 1], sreg[P ^ 1]);
    };
    for (int j = 0; j < S; j += 2) {
        stage(j, I0());
        if (j + 1 < S) stage(j + 1, I1());
    }
    if constexpr (EPI == EPI_F32) {
        flat_epilogue_f32<NTB, true>(args, t, acc, ring + kRingBytes);
    } else {
        flat_epilogue_h8<NTB>(args, t, acc);
    }
}

template <int EPI, int AM, int NT, int WF>
__device__ __forceinline__ void flat_tile_ntb(const GemmArgs& args, const FlatTile& t,
                                              unsigned char* ring) {
    if constexpr (NT == 1) {
        if constexpr (WF == 3) flat_tile_a8<EPI, AM, 1>(args, t, ring);
        else flat_tile<EPI, AM, 1, WF>(args, t, ring);
    } else {
        if (t.ntb >= NT) {
            if constexpr (WF == 3) flat_tile_a8<EPI, AM, NT>(args, t, ring);
            else flat_tile<EPI, AM, NT, WF>(args, t, ring);
        } else {
            flat_tile_ntb<EPI, AM, NT - 1, WF>(args, t, ring);
        }
    }
}

// Set up and run the tile of item `local` of group g (rows [grp_lo, grp_hi)).
// A group's rows split evenly over its ceil(n / 128) m-tiles (rounded up to
// 32 rows), so its m-tiles run at the same pace.
template <int EPI, int AM, int WF>
__device__ __forceinline__ void flat_item(const GemmArgs& args, FlatTile& t, unsigned char* ring,
                                          int g, int local, int grp_lo, int grp_hi) {
    using Pn = FPanel<EPI>;
    const int n = grp_hi - grp_lo;
    const int mt = (n + FM - 1) / FM;
    const int per = ((n + mt - 1) / mt + 31) & ~31;
    const int n_tile = local / mt, m_tile = local % mt;
    t.row0 = grp_lo + m_tile * per;
    t.valid = min(per, grp_hi - t.row0);
    t.ntb = (t.valid + 31) >> 5;
    // this wave's weight blocks
    const int np = (t.N + Pn::P - 1) / Pn::P;
    const size_t pstride = (size_t)Pn::P * t.K;
    const size_t ebase = (size_t)g * np * pstride;
    t.wstage = (size_t)Pn::BPP * 2048;
    const uint16_t* m0;
    const uint16_t* m1;
    int blk0, blk1;
    if constexpr (EPI == EPI_SWIGLU_BF16) {
        // features [32 fb, 32 fb + 32) of the gate and the up matrix
        const int fb = n_tile * (Pn::TN / 32) + t.wave;
        t.n0 = fb * 32;
        m0 = args.w1 + ebase;
        m1 = args.w2 + ebase;
        blk0 = blk1 = fb;
    } else {
        // output rows [32 wb, 32 wb + 64)
        const int wb = n_tile * (Pn::TN / 32) + 2 * t.wave;
        t.n0 = wb * 32;
        m0 = m1 = args.w1 + ebase;
        blk0 = wb;
        blk1 = wb + 1;
    }
    // (blocks past the matrix end read the last panel; never stored)
    const int p0 = min(blk0 / Pn::BPP, np - 1), p1 = min(blk1 / Pn::BPP, np - 1);
    t.wp0 = m0 + (size_t)p0 * pstride + (size_t)(blk0 % Pn::BPP) * 2048 + t.lane * 8;
    t.wp1 = m1 + (size_t)p1 * pstride + (size_t)(blk1 % Pn::BPP) * 2048 + t.lane * 8;
    if constexpr (WF) {
        // MX codes: fp8 [panel][K/64][P/32][2 chunks][64 lanes][16 B]; fp4
        // [panel][K/32][P/32][64 lanes][8 B]; scales [panel][K/32][P/32][32]
        const size_t pstride_b = (size_t)Pn::P * t.K / (WF >= 2 ? 2 : 1);
        const size_t ebase_b = (size_t)g * np * pstride_b;
        const uint8_t* c0 = (const uint8_t*)args.w1 + ebase_b;
        const uint8_t* c1 =
            (const uint8_t*)(EPI == EPI_SWIGLU_BF16 ? args.w2 : args.w1) + ebase_b;
        const size_t bsz = WF == 1 ? 2048 : 512;        // bytes per block per stage / K block
        const size_t lsz = WF == 1 ? 16 : 8;            // bytes per lane
        t.cstage = (size_t)Pn::BPP * bsz;
        // (A8W4: lane (n, h) reads the bytes of lanes n and n + 32 of K block
        // 2 s' + h, so the lane offset is n's and block h is folded in)
        const size_t lane_b = WF == 3 ? (size_t)t.l32 * lsz + (size_t)t.half * t.cstage
                                      : (size_t)t.lane * lsz;
        t.cp0 = c0 + (size_t)p0 * pstride_b + (size_t)(blk0 % Pn::BPP) * bsz + lane_b;
        t.cp1 = c1 + (size_t)p1 * pstride_b + (size_t)(blk1 % Pn::BPP) * bsz + lane_b;
        const size_t sstride = (size_t)(t.K / 32) * Pn::P;
        const uint8_t* s0 = args.s1 + (size_t)g * np * sstride;
        const uint8_t* s1 = (EPI == EPI_SWIGLU_BF16 ? args.s2 : args.s1) + (size_t)g * np * sstride;
        const size_t lane_s = (size_t)t.l32 + (WF == 3 ? (size_t)t.half * Pn::P : 0);
        t.sp0 = s0 + (size_t)p0 * sstride + (size_t)(blk0 % Pn::BPP) * 32 + lane_s;
        t.sp1 = s1 + (size_t)p1 * sstride + (size_t)(blk1 % Pn::BPP) * 32 + lane_s;
        t.sstep = Pn::P;
    }
    // activation staging: thread tid copies 16 B chunk (tid % 8) of rows
    // tid / 8 and tid / 8 + 64 (rows past the tile read its last valid row);
    // a wave stages its second row group only if the tile reaches it
    const int c = t.tid & 7;
    const int r0 = t.tid >> 3;
    const int rows_needed = t.ntb * 32;
    t.a_rows = (r0 - (t.lane >> 3) < rows_needed) + (r0 - (t.lane >> 3) + 64 < rows_needed);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const size_t grow = (size_t)(t.row0 + min(r0 + 64 * i, t.valid - 1));
        size_t e;
        if constexpr (WF == 3) {
            // fp8 codes: bytes, 16 per chunk
            const size_t src = AM == FA_GATHER ? (size_t)args.gather[grow] : grow;
            e = src * t.K + c * 16;
        } else if (AM == FA_BLK) {
            e = blocked_index(grow, c * 8, t.K);
        } else if (AM == FA_GATHER) {
            e = (size_t)args.gather[grow] * t.K + c * 8;
        } else {
            e = grow * t.K + c * 8;
        }
        t.a_off[i] = e;
    }
    if constexpr (WF == 3) {
        // scale bytes of tile row tid (threads 0 .. FM - 1 store them; the
        // others load a valid row too)
        const size_t grow = (size_t)(t.row0 + min(t.tid, t.valid - 1));
        const size_t src = AM == FA_GATHER ? (size_t)args.gather[grow] : grow;
        t.s_off = src * (size_t)(t.K / 32);
    }
    // per 64-wide stage: two 32-column blocks (blocked) or 64 elements
    t.a_step = AM == FA_BLK ? 1024 : FK;
    flat_tile_ntb<EPI, AM, FNTB, WF>(args, t, ring);
}

template <int EPI, int AM, int WF>
__global__ __launch_bounds__(kFThreads) void grouped_gemm_flat_kernel(GemmArgs args) {
    using Pn = FPanel<EPI>;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int scan_sh[8];
    __shared__ int next_item;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = args.G, rows = args.rows, N = args.N;
    const int* offs = args.offsets;
    int* item_prefix = (int*)(smem + kLdsFixed);   // [G + 1]
    const int NT = (N + Pn::TN - 1) / Pn::TN;

    auto group_rows = [&](int g, int& lo, int& hi) {
        lo = 0;
        hi = rows;
        if (offs) {
            lo = min(max(offs[g], 0), rows);
            hi = max(lo, min(max(offs[g + 1], 0), rows));
        }
    };

    // per-group item counts -> exclusive prefix in LDS
    {
        const int per = (G + kFThreads - 1) / kFThreads;
        const int g0 = tid * per;
        int local = 0;
        for (int g = g0; g < g0 + per && g < G; ++g) {
            int lo, hi;
            group_rows(g, lo, hi);
            const int items = NT * ((hi - lo + FM - 1) / FM);
            item_prefix[g] = items;
            local += items;
        }
        int x = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
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
            const int v = item_prefix[g];
            item_prefix[g] = run;
            run += v;
        }
        if (tid == 0) item_prefix[G] = total;
        __syncthreads();
    }

    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const long long Q = item_prefix[G];
    const int item_lo = (int)(Q * xcd / 8), item_hi = (int)(Q * (xcd + 1) / 8);

    FlatTile t;
    t.tid = tid;
    t.lane = lane;
    t.wave = wave;
    t.half = lane >> 5;
    t.l32 = lane & 31;
    t.K = args.K;
    t.N = N;
    unsigned* ctr = args.sched ? args.sched + xcd * 32 : nullptr;

    int q;
    if (ctr) {
        if (tid == 0) next_item = claimed_item(item_lo, item_hi, atomicAdd(ctr, 1u));
        __syncthreads();
        q = next_item;
    } else {
        q = item_lo + (blockIdx.x >> 3);
    }
    while (q < item_hi) {
        // claim the next item now; its id is published after this tile
        unsigned claimed = 0;
        if (ctr && tid == 0) claimed = atomicAdd(ctr, 1u);
        int g = 0;
        {
            int lo = 0, hi = G;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (item_prefix[mid] <= q) lo = mid; else hi = mid - 1;
            }
            g = lo;
        }
        int grp_lo, grp_hi;
        group_rows(g, grp_lo, grp_hi);
        flat_item<EPI, AM, WF>(args, t, smem, g, q - item_prefix[g], grp_lo, grp_hi);
        // every wave is past its last LDS read of this tile before the next
        // tile's prologue writes slot 0, and the claimed id is visible
        __syncthreads();
        if (ctr && tid == 0) next_item = claimed_item(item_lo, item_hi, claimed);
        __syncthreads();
        q = ctr ? next_item : q + per_xcd;
    }
}

template <int EPI, int AM, int WF = 0>
hipError_t launch_flat(const GemmArgs& g, hipStream_t stream) {
    static DeviceSetup setup;
    long long grid = 0, static_lds = 0;
    const hipError_t err = device_setup(setup, grid, static_lds, [](int, long long& gr,
                                                                    long long& st) {
        hipFuncAttributes fa;
        hipError_t e = hipFuncGetAttributes(&fa, (const void*)grouped_gemm_flat_kernel<EPI, AM, WF>);
        if (e != hipSuccess) return e;
        if (fa.sharedSizeBytes > (size_t)kFStaticLds) return hipErrorInvalidValue;
        e = hipFuncSetAttribute((const void*)grouped_gemm_flat_kernel<EPI, AM, WF>,
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                kFLdsLimit - (int)fa.sharedSizeBytes);
        if (e != hipSuccess) return e;
        st = (long long)fa.sharedSizeBytes;
        gr = (device_cu_count() + 7) & ~7;
        return hipSuccess;
    });
    if (err != hipSuccess) return err;
    const size_t lds = kLdsFixed + (size_t)(g.G + 1) * sizeof(int);
    if (lds + (size_t)static_lds > (size_t)kFLdsLimit) return hipErrorInvalidValue;
    hipLaunchKernelGGL((grouped_gemm_flat_kernel<EPI, AM, WF>), dim3((unsigned)grid), dim3(kFThreads),
                       lds, stream, g);
    return hipGetLastError();
}

}  // namespace

int grouped_gemm_flat_max_groups() {
    return (kFLdsLimit - kFStaticLds - kLdsFixed) / (int)sizeof(int) - 1;
}

hipError_t launch_grouped_gemm_flat(int epilogue, const GemmArgs& g, hipStream_t stream) {
    if (g.K % FK != 0 || g.G < 1) return hipErrorInvalidValue;
    // one weight panel (at most 256 rows) within a buffer resource's range
    if (g.K > kFlatMaxK) return hipErrorInvalidValue;
    if (g.wfp8 == 3) {
        // A8W4: gate/up on MXFP8 rows (gathered or row-major) into MXFP8 h,
        // down on row-major MXFP8 h; MXFP4 weights
        if (g.K % FK8 || !g.a8 || !g.a_scale || !g.s1 || g.out_g || g.a_blocked ||
            g.out_blocked)
            return hipErrorInvalidValue;
        if (epilogue == EPI_SWIGLU_BF16 && g.s2 && g.out_scale && g.N % 32 == 0)
            return g.gather ? launch_flat<EPI_SWIGLU_BF16, FA_GATHER, 3>(g, stream)
                            : launch_flat<EPI_SWIGLU_BF16, FA_ROW, 3>(g, stream);
        if (epilogue == EPI_F32 && !g.gather) return launch_flat<EPI_F32, FA_ROW, 3>(g, stream);
        return hipErrorInvalidValue;
    }
    if (g.wfp8) {
        // MX weights: the two routed expert GEMMs of moe_forward (gate/up on
        // gathered token rows, down on the blocked h)
        if (g.wfp8 != 1 && g.wfp8 != 2) return hipErrorInvalidValue;
        if (!g.s1 || (epilogue == EPI_SWIGLU_BF16 && !g.s2) || g.out_g) return hipErrorInvalidValue;
        const bool gu = epilogue == EPI_SWIGLU_BF16 && g.gather && g.out_blocked && !g.a_blocked;
        const bool dn = epilogue == EPI_F32 && !g.gather && g.a_blocked;
        if (g.wfp8 == 1) {
            if (gu) return launch_flat<EPI_SWIGLU_BF16, FA_GATHER, 1>(g, stream);
            if (dn) return launch_flat<EPI_F32, FA_BLK, 1>(g, stream);
        } else {
            if (gu) return launch_flat<EPI_SWIGLU_BF16, FA_GATHER, 2>(g, stream);
            if (dn) return launch_flat<EPI_F32, FA_BLK, 2>(g, stream);
        }
        return hipErrorInvalidValue;
    }
    if ((g.out_g != nullptr) != (g.out_u != nullptr)) return hipErrorInvalidValue;
    if (g.out_g && epilogue != EPI_SWIGLU_BF16) return hipErrorInvalidValue;
    if (g.gather && g.a_blocked) return hipErrorInvalidValue;
    const int am = g.gather ? FA_GATHER : g.a_blocked ? FA_BLK : FA_ROW;
    switch (epilogue) {
        case EPI_SWIGLU_BF16:
            // h is blocked exactly when the activations are not plain row-major
            if (g.out_blocked != (am != FA_ROW)) return hipErrorInvalidValue;
            if (am == FA_GATHER) return launch_flat<EPI_SWIGLU_BF16, FA_GATHER>(g, stream);
            if (am == FA_BLK) return launch_flat<EPI_SWIGLU_BF16, FA_BLK>(g, stream);
            return launch_flat<EPI_SWIGLU_BF16, FA_ROW>(g, stream);
        case EPI_F32:
            if (am == FA_GATHER) return launch_flat<EPI_F32, FA_GATHER>(g, stream);
            if (am == FA_BLK) return launch_flat<EPI_F32, FA_BLK>(g, stream);
            return launch_flat<EPI_F32, FA_ROW>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
