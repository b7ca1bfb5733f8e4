// Grouped expert GEMM for packed weights, both operands staged in LDS by
// direct-to-LDS DMA loads ("HyperParallel accelerates DeepSeek-V4.1 ...",
// section 2.3, MegaMoE: the two expert matmuls and the clamped SwiGLU
// between them).
//
// Problem: for each expert g and activation row r in [lo_g, hi_g),
//   out[r, n] = sum_k A[r, k] * W[g, n, k]
// with W in the moe_pack_weights panel layout (P = 128 rows for the gate and
// up matrices, P = 256 for the down matrix) and A row-major or in the
// blocked activation layout (16 x 32 blocks of 1 KB).
//
// Two tile shapes, one workgroup of 8 waves (two per SIMD) per tile; every
// wave owns two 32-row weight blocks (SwiGLU: gate block and the up block of
// the same 32 features; down: two adjacent output blocks) times up to four
// 32-row activation blocks (acc: 2 x NTB MFMA 32x32 tiles):
//   - square: up to TM = 256 activation rows x 256 weight rows (SwiGLU: 128
//     features).  Wave w = (wm, wn): wm = w / 4 takes one half of the tile's
//     valid rows (rounded to 32-row blocks), wn = w % 4 its weight blocks.
//   - wide: up to 128 activation rows x 512 weight rows (SwiGLU: 256
//     features); all 8 waves share the activation rows, wave w takes weight
//     blocks of index w.  Each activation byte staged feeds twice the MFMA
//     work, so experts with at most 128 rows move half the activation bytes
//     per weight byte.
// An expert with up to TM rows is one tile row, so its weights are read from
// memory once.  Per 32-wide K stage one LDS slot holds
//   - the activation tile, TM rows x 64 B, the 16-byte chunks of row r
//     XOR-swizzled by sw(r) = ((r >> 1) ^ (r >> 3)) & 3, so that the 16
//     lanes an LDS cycle serves (256 B over 64 banks: rows r, r+4, r+8,
//     r+12 share banks) hit distinct banks in MFMA operand reads;
//   - the weight half-stage in matrix-core fragment order (copied from the
//     packed layout in 1 KB runs; operand reads are 1 KB contiguous per
//     wave).
// A ring of SLOTS LDS slots keeps SLOTS - 1 stages in flight per CU.  The
// DMA (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16 l) moves
// 1 KB per instruction: weight instructions and blocked-layout activation
// instructions each read 1 KB of contiguous memory (8 full cache lines);
// row-major activations cost 16 half-used lines per instruction.  Each wave
// issues NW weight instructions and na activation instructions per stage
// (only the 16-row groups that hold valid rows are copied); both are fixed
// for a tile, so vmcnt counts stay exact.  The DMA is issued from inline
// assembly, so the compiler does not see LDS writes it would otherwise guard
// with a full vmcnt drain before every LDS read; explicit vmcnt waits + one
// barrier per stage are the complete synchronisation.
// Scheduling: persistent grid; per-expert item and cost prefixes built in
// LDS from the device offsets; cost-balanced contiguous item ranges per XCD,
// claimed in order by the XCD's workgroups (see grouped_gemm_lds_kernel).
#include "moe_internal.h"

#ifndef MOE_LDS_TM
#define MOE_LDS_TM 256
#endif
#ifndef MOE_LDS_SLOTS
#define MOE_LDS_SLOTS 4
#endif

namespace moe {
namespace {

constexpr int BK = 32;                       // K per pipeline stage
constexpr int kThreads = 512;
constexpr int kLdsLimit = 160 * 1024;
constexpr int kStaticLds = 256;              // reserve for static LDS (scan_sh, next_item)

template <int EPI, bool WIDE>
struct Shape {
    static constexpr int TM = WIDE ? 128 : MOE_LDS_TM;      // activation rows per tile
    static_assert(TM % 64 == 0 && TM >= 64 && TM <= 256, "TM: 64..256, multiple of 64");
    static constexpr int MH = WIDE ? TM : TM / 2;           // max rows per wave
    static constexpr int MAXNTB = MH / 32;                  // activation blocks per wave
    static constexpr int WBLK = WIDE ? 16 : 8;              // 32-row weight blocks per tile
    static constexpr int NW = WBLK / 4;                     // weight DMA instrs per wave per stage
    static constexpr int WAVES_N = WIDE ? 8 : 4;            // waves along the weight rows
    static constexpr int SLOTA = TM * 64;
    static constexpr int SLOTW = WBLK * 2 * 1024;           // 2 substeps x 1 KB per block
    static constexpr int SLOT = SLOTA + SLOTW;
    static constexpr int SLOTS = WIDE ? 3 : MOE_LDS_SLOTS;
    static constexpr int AHEAD = SLOTS - 1;                 // stages in flight
    static_assert(SLOTS >= 2 && SLOTS <= 8, "ring depth");
    static constexpr int AINSTR = TM / 16;                  // activation instrs per stage
    static constexpr int APW = (AINSTR + 7) / 8;            // ... per wave (max)
    static constexpr int PANEL = (EPI == EPI_SWIGLU_BF16) ? 128 : 256;
    static constexpr int BPP = PANEL / 32;                  // blocks per panel
    // weight rows (per matrix) and panels (per matrix) of one n-tile
    static constexpr int TN = (EPI == EPI_SWIGLU_BF16) ? WBLK * 16 : WBLK * 32;
    static constexpr int PPT = TN / PANEL;
    static constexpr int RING = SLOTS * SLOT;
    static_assert(RING + kStaticLds < kLdsLimit, "LDS ring");
};

__device__ __forceinline__ float clamp_sym(float v, float L) { return fminf(fmaxf(v, -L), L); }

// position swizzle of the four 16-byte chunks of activation row r in LDS
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

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

// wait for the oldest in-flight stage of a wave that issues na + NW
// instructions per stage (AHEAD - 1 newer stages may stay outstanding)
template <int NW, int AHEAD>
__device__ __forceinline__ void wait_stage(int na) {
    if (na == 2) wait_vm<(AHEAD - 1) * (NW + 2)>();
    else if (na == 1) wait_vm<(AHEAD - 1) * (NW + 1)>();
    else wait_vm<(AHEAD - 1) * NW>();
}

struct LdsTile {
    const GemmArgs* args;
    uint32_t lds0;         // LDS byte address of slot 0
    unsigned char* smem;
    int lane, wave, wm, wn, half, l32;
    int K, N, S;
    int row0, valid;
    int mh;                // activation rows per wave half (multiple of 32)
    int na;                // activation DMA instructions of this wave per stage
    int n0;                // first weight row / feature of this wave's blocks
    const uint16_t* wsrc0; // first panel of this n-tile (gate matrix for SwiGLU)
    const uint16_t* wsrc1; // up matrix panel (SwiGLU) or the same
    int np_left;           // panels of this n-tile that exist (1..PPT)
    size_t pstride;        // packed elements per panel
    size_t wstride;        // packed elements per 64-wide K stage of one panel
    unsigned* ctr;         // this XCD's item counter (dynamic scheduling) or NULL
    int* next_item;        // LDS slot receiving the claimed next item
    int item_lo;           // first item of this XCD's range
};

// DMA of pipeline stage j (32 k) into the LDS slot at byte offset `sbase`.
//   activations: instruction n (rows [16 n, 16 n + 16) of the tile) belongs
//     to wave n % 8 and is issued only if the group holds a valid row; rows
//     past the tile read the last valid row.  Chunk c of row r is stored at
//     position c ^ sw(r).
//   weights: the 64-wide packed stage s = j / 2 holds, per 32-row block,
//     4 substeps x 1 KB; this half-stage (h = j % 2) takes substeps 2h, 2h+1
//     of all WBLK blocks: instruction n = NW w + i copies tile block n / 2,
//     substep 2h + n % 2 to LDS fragment slot n.  SwiGLU tile blocks
//     [0, WBLK/2) are gate rows, the rest up rows; a block of a panel past
//     the matrix end re-reads the last panel (its outputs are never stored).
template <int EPI, bool WIDE>
__device__ __forceinline__ void issue_stage(const LdsTile& t, int j, uint32_t sbase) {
    using C = Shape<EPI, WIDE>;
    const uint32_t base = t.lds0 + sbase;
    const int kcol = j * BK;
    const GemmArgs& args = *t.args;
#pragma unroll
    for (int i = 0; i < C::APW; ++i) {
        if (i < t.na) {
            const int r0 = 16 * (t.wave + 8 * i);
            const int r = r0 + (t.lane >> 2);
            const int c = (t.lane & 3) ^ swz(r);
            const size_t grow = (size_t)(t.row0 + min(r, t.valid - 1));
            const uint16_t* src = args.a_blocked ? args.a + blocked_index(grow, kcol + c * 8, t.K)
                                                 : args.a + grow * t.K + kcol + c * 8;
            dma16(src, base + r0 * 64);
        }
    }
    const int s64 = j >> 1, h2 = j & 1;
#pragma unroll
    for (int i = 0; i < C::NW; ++i) {
        const int n = C::NW * t.wave + i;
        const int b = n >> 1;
        const int sub = 2 * h2 + (n & 1);
        const uint16_t* mat = t.wsrc0;
        int bb = b;
        if (EPI == EPI_SWIGLU_BF16 && b >= C::WBLK / 2) {
            mat = t.wsrc1;
            bb = b - C::WBLK / 2;
        }
        const int panel = min(bb / C::BPP, t.np_left - 1);
        const uint16_t* src = mat + (size_t)panel * t.pstride + (size_t)s64 * t.wstride +
                              (bb % C::BPP) * 2048 + sub * 512 + t.lane * 8;
        dma16(src, base + C::SLOTA + n * 1024);
    }
}

// MFMA operands of one 16-wide K substep q of a stage: this wave's two weight
// fragments and its NTB activation fragments.
template <int NTB>
struct Operands {
    bf16x8 w0, w1, a[NTB];
};

template <int EPI, bool WIDE, int NTB>
__device__ __forceinline__ void read_operands(const LdsTile& t, uint32_t sbase, int q,
                                              Operands<NTB>& o) {
    using C = Shape<EPI, WIDE>;
    const unsigned char* base = t.smem + sbase;
    // weight blocks of this wave (fragment slots 2 b + substep)
    const int b0 = (EPI == EPI_SWIGLU_BF16) ? t.wn : 2 * t.wn;
    const int b1 = (EPI == EPI_SWIGLU_BF16) ? C::WBLK / 2 + t.wn : 2 * t.wn + 1;
    const unsigned char* wbase = base + C::SLOTA + t.lane * 16;
    o.w0 = *(const bf16x8*)(wbase + (b0 * 2 + q) * 1024);
    o.w1 = *(const bf16x8*)(wbase + (b1 * 2 + q) * 1024);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int r = t.wm * t.mh + tb * 32 + t.l32;
        const int c = (2 * q + t.half) ^ swz(r);
        o.a[tb] = *(const bf16x8*)(base + r * 64 + c * 16);
    }
}

template <int NTB, int MAXNTB>
__device__ __forceinline__ void mfma_substep(const Operands<NTB>& o, f32x16 (&acc)[2][MAXNTB]) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w0, o.a[tb], acc[0][tb], 0, 0, 0);
        acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w1, o.a[tb], acc[1][tb], 0, 0, 0);
    }
}

template <int EPI, bool WIDE, int NTB>
__device__ __forceinline__ void epilogue(const LdsTile& t,
                                         const f32x16 (&acc)[2][Shape<EPI, WIDE>::MAXNTB]) {
    const GemmArgs& args = *t.args;
    const int N = t.N;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int rl = t.wm * t.mh + tb * 32 + t.l32;
        if (rl >= t.valid) continue;
        const size_t r = (size_t)(t.row0 + rl);
        if (EPI == EPI_SWIGLU_BF16) {
            const float L = args.clamp_limit;
            uint16_t* out = (uint16_t*)args.out;
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
                uint16_t* dst = args.out_blocked ? out + blocked_index(r, n, N) : out + r * N + n;
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

// K loop of one tile for a wave computing NTB 32-row blocks (0: DMA only).
// Stages j+1 .. j+AHEAD-1 stay in flight while stage j computes: wait for
// stage j (this wave's own DMA), barrier (all waves' DMA of stage j landed,
// and all waves are done reading the slot the next DMA overwrites), issue
// stage j + AHEAD into the slot stage j - 1 used, compute stage j.  Stages
// past the end re-issue the last stage, so every iteration issues the same
// number of instructions.
template <int EPI, bool WIDE, int NTB>
__device__ __forceinline__ void run_tile(const LdsTile& t) {
    using C = Shape<EPI, WIDE>;
    f32x16 acc[2][C::MAXNTB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int tb = 0; tb < C::MAXNTB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;
    const int S = t.S;
    wait_vm<0>();  // retire the previous tile's stores before counting DMA entries
#pragma unroll
    for (int p = 0; p < C::AHEAD; ++p) issue_stage<EPI, WIDE>(t, min(p, S - 1), p * C::SLOT);
    uint32_t s_cmp = 0, s_iss = C::AHEAD * C::SLOT;
    // Operand reads run one half-stage ahead of the MFMAs: after the barrier
    // of stage j the wave reads substep 0 of stage j while it multiplies
    // substep 1 of stage j - 1 (read before this barrier), then reads
    // substep 1 of stage j while it multiplies substep 0.  Every LDS read
    // latency hides behind MFMAs of the same wave; the reads of a slot
    // complete before the next barrier, so the DMA that reuses the slot
    // after that barrier never races them.
    Operands<NTB> o0, o1;
    for (int j = 0; j < S; ++j) {
        wait_stage<C::NW, C::AHEAD>(t.na);
        __syncthreads();
        issue_stage<EPI, WIDE>(t, min(j + C::AHEAD, S - 1), s_iss);
        s_iss = (s_iss + C::SLOT == C::RING) ? 0 : s_iss + C::SLOT;
        if constexpr (NTB > 0) {
            read_operands<EPI, WIDE, NTB>(t, s_cmp, 0, o0);
            __builtin_amdgcn_sched_barrier(0);
            if (j > 0) mfma_substep<NTB, C::MAXNTB>(o1, acc);
            __builtin_amdgcn_sched_barrier(0);
            read_operands<EPI, WIDE, NTB>(t, s_cmp, 1, o1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_substep<NTB, C::MAXNTB>(o0, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        s_cmp = (s_cmp + C::SLOT == C::RING) ? 0 : s_cmp + C::SLOT;
    }
    if constexpr (NTB > 0) mfma_substep<NTB, C::MAXNTB>(o1, acc);
    // dynamic scheduling: thread 0 claims the workgroup's next item here,
    // after the last stage wait, so no claim is in flight while the K loop
    // counts DMA entries
    const bool claim = t.ctr != nullptr && threadIdx.x == 0;
    unsigned claimed = 0;
    if (claim) claimed = atomicAdd(t.ctr, 1u);
    wait_vm<0>();
    if (claim) *t.next_item = t.item_lo + (int)claimed;
    __syncthreads();
    if constexpr (NTB > 0) epilogue<EPI, WIDE, NTB>(t, acc);
}

// run_tile for ntb in [0, NT] (ntb is wave-uniform)
template <int EPI, bool WIDE, int NT>
__device__ __forceinline__ void run_tile_ntb(const LdsTile& t, int ntb) {
    if constexpr (NT == 0) {
        run_tile<EPI, WIDE, 0>(t);
    } else {
        if (ntb >= NT) run_tile<EPI, WIDE, NT>(t);
        else run_tile_ntb<EPI, WIDE, NT - 1>(t, ntb);
    }
}

// Tile of item (group g, local item index) in the given shape: set up the
// per-tile fields of t and run it.
template <int EPI, bool WIDE>
__device__ __forceinline__ void do_tile(LdsTile& t, const GemmArgs& args, int g, int local,
                                        int grp_lo, int grp_hi) {
    using C = Shape<EPI, WIDE>;
    const int N = args.N;
    int n_tile = local, m_tile = 0;
    if (!WIDE) {
        const int mt = (grp_hi - grp_lo + C::TM - 1) / C::TM;
        n_tile = local / mt;
        m_tile = local % mt;
    }
    t.row0 = grp_lo + m_tile * C::TM;
    t.valid = min(C::TM, grp_hi - t.row0);
    // activation instructions n = wave + 8 i with a valid row (16 n < valid)
    t.na = 0;
#pragma unroll
    for (int i = 0; i < C::APW; ++i)
        t.na += (t.wave + 8 * i < C::AINSTR && 16 * (t.wave + 8 * i) < t.valid) ? 1 : 0;
    t.wm = WIDE ? 0 : t.wave >> 2;
    t.wn = WIDE ? t.wave : t.wave & 3;
    // weight panels of this n-tile
    const int NP = (N + C::PANEL - 1) / C::PANEL;
    const int p0 = n_tile * C::PPT;
    t.pstride = (size_t)C::PANEL * t.K;
    const size_t pbase = ((size_t)g * NP + p0) * t.pstride;
    t.wsrc0 = args.w1 + pbase;
    t.wsrc1 = (EPI == EPI_SWIGLU_BF16 ? args.w2 : args.w1) + pbase;
    t.np_left = min(C::PPT, NP - p0);
    t.wstride = (size_t)C::BPP * 2048;
    t.n0 = (EPI == EPI_SWIGLU_BF16) ? n_tile * C::TN + t.wn * 32 : n_tile * C::TN + t.wn * 64;
    // square tiles split the valid rows evenly (in 32-row blocks) between
    // the two wave halves, so both waves of a SIMD compute
    t.mh = WIDE ? C::MH : min(C::MH, (((t.valid + 1) >> 1) + 31) & ~31);
    const int wrows = min(max(t.valid - t.wm * t.mh, 0), t.mh);
    const int ntb = t.n0 < N ? (wrows + 31) / 32 : 0;
    run_tile_ntb<EPI, WIDE, C::MAXNTB>(t, ntb);
}

template <int EPI>
constexpr int ring_bytes() {
    return Shape<EPI, false>::RING > Shape<EPI, true>::RING ? Shape<EPI, false>::RING
                                                             : Shape<EPI, true>::RING;
}

// Work items: a group with at most 128 rows (when args.wide) is wide-tiled,
// ceil(N / TN_wide) items; any other non-empty group is square-tiled,
// ceil(N / TN_square) x ceil(rows / 256) items.  An item's cost is its
// weight rows (wide 2, square 1 units of 256 rows x K), since every item
// streams its weight panels through the CU.  Items are ordered (group,
// n-tile, m-tile); the 8 XCDs take contiguous ranges of equal cost, and
// inside an XCD the workgroups claim items in order from a per-XCD counter
// (args.sched, zeroed before the launch) or, without counters, take every
// 32nd item.  Workgroups of one XCD thus work on neighbouring items (the
// n-tiles of the same experts) at the same time and share their
// activations in L2.
template <int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_lds_kernel(GemmArgs args) {
    using SQ = Shape<EPI, false>;
    using WD = Shape<EPI, true>;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int scan_sh[2][8];
    __shared__ int next_item;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int G = args.G, rows = args.rows, K = args.K, N = args.N;
    const int* offs = args.offsets;
    int* item_prefix = (int*)(smem + ring_bytes<EPI>());  // [G + 1]
    int* cost_prefix = item_prefix + (G + 1);               // [G + 1]
    const int NTs = (N + SQ::TN - 1) / SQ::TN;
    const int NTw = (N + WD::TN - 1) / WD::TN;

    auto group_rows = [&](int g, int& lo, int& hi) {
        lo = 0;
        hi = rows;
        if (offs) {
            lo = min(max(offs[g], 0), rows);
            hi = max(lo, min(max(offs[g + 1], 0), rows));
        }
    };
    auto is_wide = [&](int n) { return args.wide && n <= WD::TM; };

    // ---- per-group item counts and costs -> exclusive prefixes in LDS ----
    {
        const int per = (G + kThreads - 1) / kThreads;
        const int g0 = tid * per;
        int li = 0, lc = 0;
        for (int g = g0; g < g0 + per && g < G; ++g) {
            int lo, hi;
            group_rows(g, lo, hi);
            const int n = hi - lo;
            const int items = n == 0 ? 0 : is_wide(n) ? NTw : NTs * ((n + SQ::TM - 1) / SQ::TM);
            item_prefix[g] = items;
            cost_prefix[g] = items * (is_wide(n) ? 2 : 1);
            li += items;
            lc += cost_prefix[g];
        }
        int xi = li, xc = lc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int yi = __shfl_up(xi, off, 64), yc = __shfl_up(xc, off, 64);
            if (lane >= off) {
                xi += yi;
                xc += yc;
            }
        }
        if (lane == 63) {
            scan_sh[0][wave] = xi;
            scan_sh[1][wave] = xc;
        }
        __syncthreads();
        int bi = 0, bc = 0, ti = 0, tc = 0;
        for (int w = 0; w < 8; ++w) {
            if (w < wave) {
                bi += scan_sh[0][w];
                bc += scan_sh[1][w];
            }
            ti += scan_sh[0][w];
            tc += scan_sh[1][w];
        }
        int ri = bi + xi - li, rc = bc + xc - lc;
        for (int g = g0; g < g0 + per && g < G; ++g) {
            const int vi = item_prefix[g], vc = cost_prefix[g];
            item_prefix[g] = ri;
            cost_prefix[g] = rc;
            ri += vi;
            rc += vc;
        }
        if (tid == 0) {
            item_prefix[G] = ti;
            cost_prefix[G] = tc;
        }
        __syncthreads();
    }

    // first item whose cost starts at or after `target`
    auto boundary = [&](long long target) -> int {
        int lo = 0, hi = G;  // largest g with cost_prefix[g] <= target
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cost_prefix[mid] <= target) lo = mid; else hi = mid - 1;
        }
        if (lo == G) return item_prefix[G];
        const int items = item_prefix[lo + 1] - item_prefix[lo];
        if (items == 0) return item_prefix[lo];
        const int unit = (cost_prefix[lo + 1] - cost_prefix[lo]) / items;
        const long long rem = target - cost_prefix[lo];
        return item_prefix[lo] + (int)min((long long)items, (rem + unit - 1) / unit);
    };
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const long long total_cost = cost_prefix[G];
    const int item_lo = boundary(total_cost * xcd / 8);
    const int item_hi = boundary(total_cost * (xcd + 1) / 8);

    LdsTile t;
    t.args = &args;
    t.smem = smem;
    t.lds0 = (uint32_t)(uintptr_t)smem;
    t.lane = lane;
    t.wave = wave;
    t.half = lane >> 5;
    t.l32 = lane & 31;
    t.K = K;
    t.N = N;
    t.S = K / BK;
    t.ctr = args.sched ? args.sched + xcd * 32 : nullptr;
    t.next_item = &next_item;
    t.item_lo = item_lo;

    int q;
    if (t.ctr) {
        if (tid == 0) next_item = item_lo + (int)atomicAdd(t.ctr, 1u);
        __syncthreads();
        q = next_item;
    } else {
        q = item_lo + (blockIdx.x >> 3);
    }
    while (q < item_hi) {
        int g = 0;
        {
            int lo = 0, hi = G;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (item_prefix[mid] <= q) lo = mid; else hi = mid - 1;
            }
            g = lo;
        }
        const int local = q - item_prefix[g];
        int grp_lo, grp_hi;
        group_rows(g, grp_lo, grp_hi);
        if (is_wide(grp_hi - grp_lo)) do_tile<EPI, true>(t, args, g, local, grp_lo, grp_hi);
        else do_tile<EPI, false>(t, args, g, local, grp_lo, grp_hi);
        q = t.ctr ? next_item : q + per_xcd;
    }
}

template <int EPI>
hipError_t launch_lds(const GemmArgs& g, hipStream_t stream) {
    static int configured_device = -1;
    static int grid = 0;
    static size_t static_lds = 0;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (configured_device != dev) {
        hipFuncAttributes fa;
        err = hipFuncGetAttributes(&fa, (const void*)grouped_gemm_lds_kernel<EPI>);
        if (err != hipSuccess) return err;
        static_lds = fa.sharedSizeBytes;
        if (static_lds > (size_t)kStaticLds) return hipErrorInvalidValue;
        err = hipFuncSetAttribute((const void*)grouped_gemm_lds_kernel<EPI>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  kLdsLimit - (int)static_lds);
        if (err != hipSuccess) return err;
        grid = (device_cu_count() + 7) & ~7;
        configured_device = dev;
    }
    const size_t lds = ring_bytes<EPI>() + 2 * (size_t)(g.G + 1) * sizeof(int);
    if (lds + static_lds > (size_t)kLdsLimit) return hipErrorInvalidValue;
    hipLaunchKernelGGL((grouped_gemm_lds_kernel<EPI>), dim3(grid), dim3(kThreads), lds, stream,
                       g);
    return hipGetLastError();
}

}  // namespace

int grouped_gemm_lds_max_groups() {
    constexpr int ring = ring_bytes<EPI_SWIGLU_BF16>() > ring_bytes<EPI_F32>()
                             ? ring_bytes<EPI_SWIGLU_BF16>()
                             : ring_bytes<EPI_F32>();
    return (kLdsLimit - kStaticLds - ring) / (2 * (int)sizeof(int)) - 1;
}

hipError_t launch_grouped_gemm_lds(int epilogue, const GemmArgs& g, hipStream_t stream) {
    if (g.K % BK != 0 || g.G < 1) return hipErrorInvalidValue;
    switch (epilogue) {
        case EPI_SWIGLU_BF16: return launch_lds<EPI_SWIGLU_BF16>(g, stream);
        case EPI_F32: return launch_lds<EPI_F32>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
