// Grouped expert GEMM for packed weights, both operands staged in LDS by
// direct-to-LDS DMA loads ("HyperParallel accelerates DeepSeek-V4.1 ...",
// section 2.3, MegaMoE: the two expert matmuls and the clamped SwiGLU
// between them).
//
// Problem: for each expert g and activation row r in [lo_g, hi_g),
//   out[r, n] = sum_k A[r, k] * W[g, n, k]
// with W in the moe_pack_weights panel layout (P = 128 rows for the gate and
// up matrices, P = 256 for the down matrix) and A row-major, in the blocked
// activation layout (16 x 32 blocks of 1 KB), or gathered: row r of A is row
// gather[r] of a row-major matrix (the dispatch permutation applied while
// loading, so the permuted copy of the tokens is never written).
//
// Tiles of up to 256 activation rows x 256 weight rows (SwiGLU: 128 features
// x {gate, up}), one workgroup of 8 waves (two per SIMD) per tile.  Wave
// w = (wm, wn): wn = w % 4 owns two 32-row weight blocks (SwiGLU: gate block
// wn and the up block of the same 32 features; down: blocks 2 wn, 2 wn + 1),
// wm = w / 4 one half of the tile's valid rows, split in 32-row blocks so
// that both waves of a SIMD compute (acc: 2 x NTB MFMA 32x32 tiles,
// NTB <= 4).  An expert with up to 256 rows is one tile row, so its weights
// are streamed from memory once.  (Taller or wider tiles for mid-size or
// very small experts stage more activation bytes per weight byte or hold
// fewer stages in flight; measured on MI355X they were slower.)
// Per 32-wide K stage one LDS slot holds
//   - the activation tile, 256 rows x 64 B, the 16-byte chunks of row r
//     XOR-swizzled by sw(r) = ((r >> 1) ^ (r >> 3)) & 3, so that the 16
//     lanes an LDS cycle serves (256 B over 64 banks: rows r, r+4, r+8,
//     r+12 share banks) hit distinct banks in MFMA operand reads;
//   - the weight half-stage, 16 KB in matrix-core fragment order (copied
//     from the packed layout in 1 KB runs; operand reads are 1 KB
//     contiguous per wave).
// A ring of 4 slots keeps 3 stages (96 KB) in flight per CU.  The DMA
// (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16 l) moves 1 KB
// per instruction: weight instructions and blocked-layout activation
// instructions each read 1 KB of contiguous memory (8 full cache lines);
// row-major activations cost 16 half-used lines per instruction.  Each wave
// issues 2 weight instructions and na in {0, 1, 2} activation instructions
// per stage (only the 16-row groups that hold valid rows are copied); na is
// fixed for a tile, so vmcnt counts stay exact.  The DMA is issued from
// inline assembly, so the compiler does not see LDS writes it would
// otherwise guard with a full vmcnt drain before every LDS read; explicit
// vmcnt waits + one barrier per stage are the complete synchronisation, and
// the kernel keeps every other value in registers (a spill reload would make
// the compiler drain vmcnt inside the pipeline).
// Scheduling: see grouped_gemm_lds_kernel.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TM = 256;                      // activation rows per tile
constexpr int MH = TM / 2;                   // max rows per wave
constexpr int MAXNTB = MH / 32;              // activation blocks per wave
constexpr int WBLK = 8;                      // 32-row weight blocks per tile
constexpr int BK = 32;                       // K per pipeline stage
constexpr int kSlotA = TM * 64;              // activation tile per stage
constexpr int kSlotW = WBLK * 2 * 1024;      // weight half-stage: 2 substeps x 1 KB per block
constexpr int kSlot = kSlotA + kSlotW;
constexpr int kSlots = 4;                    // LDS ring
constexpr int kAhead = kSlots - 1;           // stages in flight
constexpr int kRing = kSlots * kSlot;
constexpr int kAInstr = TM / 16;             // activation DMA instructions per stage
constexpr int kAPerWave = kAInstr / 8;
constexpr int kThreads = 512;
constexpr int kLdsLimit = 160 * 1024;
constexpr int kStaticLds = 256;              // reserve for static LDS (scan_sh, next_item)

// activation addressing: row-major a, the blocked layout, or row-major a
// with row r of the problem taken from row gather[r] (the dispatch
// permutation applied while loading).  The SwiGLU output is written in the
// blocked layout unless the activations are plain row-major.
enum AMode : int { A_ROW = 0, A_BLK = 1, A_GATHER = 2 };

template <int EPI>
struct Panel {
    static constexpr int P = (EPI == EPI_SWIGLU_BF16) ? 128 : 256;  // packed panel rows
    static constexpr int BPP = P / 32;                               // blocks per panel
    // weight blocks per matrix in a tile (SwiGLU: 4 gate blocks, then 4 up)
    static constexpr int BPM = (EPI == EPI_SWIGLU_BF16) ? WBLK / 2 : WBLK;
    static constexpr int TN = BPM * 32;                              // rows of one matrix
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

// wait for the oldest in-flight stage of a wave that issues na + 2
// instructions per stage (kAhead - 1 newer stages may stay outstanding)
__device__ __forceinline__ void wait_stage(int na) {
    if (na == 2) wait_vm<(kAhead - 1) * 4>();
    else if (na == 1) wait_vm<(kAhead - 1) * 3>();
    else wait_vm<(kAhead - 1) * 2>();
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
    uint32_t a_off[kAPerWave];  // lane's stage-0 source of activation instruction i (16 B units)
    uint32_t a_step;       // ... advance per stage (16 B units)
    int n0;                // first weight row / feature of this wave's blocks
    const uint16_t* wsrc0; // this expert's packed matrix (gate matrix for SwiGLU)
    const uint16_t* wsrc1; // up matrix (SwiGLU) or the same
    int blk0;              // first 32-row block of this n-tile in each matrix
    int np;                // packed panels per matrix
    size_t pstride;        // packed elements per panel
    size_t wstride;        // packed elements per 64-wide K stage of one panel
    unsigned* ctr;         // this XCD's item counter (dynamic scheduling) or NULL
    int* next_item;        // LDS slot receiving the claimed next item
    int item_lo;           // first item of this XCD's range
};

// DMA of pipeline stage j (32 k) into the LDS slot at byte offset `sbase`.
//   activations: instruction n (rows [16 n, 16 n + 16) of the tile) belongs
//     to wave n % 8 and is issued only if the group holds a valid row (the
//     per-lane sources are set up per tile in t.a_off).
//   weights: the 64-wide packed stage s = j / 2 holds, per 32-row block,
//     4 substeps x 1 KB; this half-stage (h = j % 2) takes substeps 2h, 2h+1
//     of all 8 blocks: instruction n = 2 w + i copies tile block n / 2,
//     substep 2h + n % 2 to LDS fragment slot n.  SwiGLU tile blocks [0, 4)
//     are gate rows, [4, 8) up rows; a block of a panel past the matrix end
//     re-reads the last panel (its outputs are never stored).
template <int EPI>
__device__ __forceinline__ void issue_stage(const LdsTile& t, int j, uint32_t sbase) {
    using Pn = Panel<EPI>;
    const uint32_t base = t.lds0 + sbase;
    const GemmArgs& args = *t.args;
#pragma unroll
    for (int i = 0; i < kAPerWave; ++i) {
        if (i < t.na) {
            const int r0 = 16 * (t.wave + 8 * i);
            const uint32_t off = t.a_off[i] + (uint32_t)j * t.a_step;
            dma16((const u32x4*)args.a + off, base + r0 * 64);
        }
    }
    const int s64 = j >> 1, h2 = j & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int n = 2 * t.wave + i;
        const int b = n >> 1;
        const int sub = 2 * h2 + (n & 1);
        const uint16_t* mat = t.wsrc0;
        int gb = t.blk0 + b;
        if (EPI == EPI_SWIGLU_BF16 && b >= Pn::BPM) {
            mat = t.wsrc1;
            gb -= Pn::BPM;
        }
        const int panel = min(gb / Pn::BPP, t.np - 1);
        const uint16_t* src = mat + (size_t)panel * t.pstride + (size_t)s64 * t.wstride +
                              (gb % Pn::BPP) * 2048 + sub * 512 + t.lane * 8;
        dma16(src, base + kSlotA + n * 1024);
    }
}

// MFMA operands of one 16-wide K substep q of a stage: this wave's two weight
// fragments and its NTB activation fragments.
template <int NTB>
struct Operands {
    bf16x8 w0, w1, a[NTB];
};

template <int EPI, int NTB>
__device__ __forceinline__ void read_operands(const LdsTile& t, uint32_t sbase, int q,
                                              Operands<NTB>& o) {
    const unsigned char* base = t.smem + sbase;
    // weight blocks of this wave (fragment slots 2 b + substep)
    const int b0 = (EPI == EPI_SWIGLU_BF16) ? t.wn : 2 * t.wn;
    const int b1 = (EPI == EPI_SWIGLU_BF16) ? Panel<EPI>::BPM + t.wn : 2 * t.wn + 1;
    const unsigned char* wbase = base + kSlotA + t.lane * 16;
    o.w0 = *(const bf16x8*)(wbase + (b0 * 2 + q) * 1024);
    o.w1 = *(const bf16x8*)(wbase + (b1 * 2 + q) * 1024);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int r = t.wm * t.mh + tb * 32 + t.l32;
        const int c = (2 * q + t.half) ^ swz(r);
        o.a[tb] = *(const bf16x8*)(base + r * 64 + c * 16);
    }
}

template <int NTB>
__device__ __forceinline__ void mfma_substep(const Operands<NTB>& o, f32x16 (&acc)[2][MAXNTB]) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w0, o.a[tb], acc[0][tb], 0, 0, 0);
        acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w1, o.a[tb], acc[1][tb], 0, 0, 0);
    }
}

template <int EPI, int AM, int NTB>
__device__ __forceinline__ void epilogue(const LdsTile& t, const f32x16 (&acc)[2][MAXNTB]) {
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
                uint16_t* dst = AM != A_ROW ? out + blocked_index(r, n, N) : out + r * N + n;
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
// Stages j+1 .. j+kAhead-1 stay in flight while stage j computes: wait for
// stage j (this wave's own DMA), barrier (all waves' DMA of stage j landed,
// and all waves are done reading the slot the next DMA overwrites), issue
// stage j + kAhead into the slot stage j - 1 used, compute stage j.  Stages
// past the end re-issue the last stage, so every iteration issues the same
// number of instructions.
template <int EPI, int AM, int NTB>
__device__ __forceinline__ void run_tile(const LdsTile& t) {
    f32x16 acc[2][MAXNTB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int tb = 0; tb < MAXNTB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;
    const int S = t.S;
    wait_vm<0>();  // retire the previous tile's stores before counting DMA entries
#pragma unroll
    for (int p = 0; p < kAhead; ++p) issue_stage<EPI>(t, min(p, S - 1), p * kSlot);
    uint32_t s_cmp = 0, s_iss = kAhead * kSlot;
    // Operand reads run one half-stage ahead of the MFMAs: after the barrier
    // of stage j the wave reads substep 0 of stage j while it multiplies
    // substep 1 of stage j - 1 (read before this barrier), then reads
    // substep 1 of stage j while it multiplies substep 0.  Every LDS read
    // latency hides behind MFMAs of the same wave; the reads of a slot
    // complete before the next barrier, so the DMA that reuses the slot
    // after that barrier never races them.
    Operands<NTB> o0, o1;
    for (int j = 0; j < S; ++j) {
        wait_stage(t.na);
        __syncthreads();
        issue_stage<EPI>(t, min(j + kAhead, S - 1), s_iss);
        s_iss = (s_iss + kSlot == kRing) ? 0 : s_iss + kSlot;
        if constexpr (NTB > 0) {
            read_operands<EPI, NTB>(t, s_cmp, 0, o0);
            __builtin_amdgcn_sched_barrier(0);
            if (j > 0) mfma_substep<NTB>(o1, acc);
            __builtin_amdgcn_sched_barrier(0);
            read_operands<EPI, NTB>(t, s_cmp, 1, o1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_substep<NTB>(o0, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        s_cmp = (s_cmp + kSlot == kRing) ? 0 : s_cmp + kSlot;
    }
    if constexpr (NTB > 0) mfma_substep<NTB>(o1, acc);
    // dynamic scheduling: thread 0 claims the workgroup's next item here,
    // after the last stage wait, so no claim is in flight while the K loop
    // counts DMA entries
    const bool claim = t.ctr != nullptr && threadIdx.x == 0;
    unsigned claimed = 0;
    if (claim) claimed = atomicAdd(t.ctr, 1u);
    wait_vm<0>();
    if (claim) *t.next_item = t.item_lo + (int)claimed;
    __syncthreads();
    if constexpr (NTB > 0) epilogue<EPI, AM, NTB>(t, acc);
}

// run_tile for ntb in [0, NT] (ntb is wave-uniform)
template <int EPI, int AM, int NT>
__device__ __forceinline__ void run_tile_ntb(const LdsTile& t, int ntb) {
    if constexpr (NT == 0) {
        run_tile<EPI, AM, 0>(t);
    } else {
        if (ntb >= NT) run_tile<EPI, AM, NT>(t);
        else run_tile_ntb<EPI, AM, NT - 1>(t, ntb);
    }
}

// Tile of item (group g, local item index): set up the per-tile fields of t
// and run it.
template <int EPI, int AM>
__device__ __forceinline__ void do_tile(LdsTile& t, const GemmArgs& args, int g, int local,
                                        int grp_lo, int grp_hi) {
    using Pn = Panel<EPI>;
    const int N = args.N;
    const int mt = (grp_hi - grp_lo + TM - 1) / TM;
    const int n_tile = local / mt, m_tile = local % mt;
    t.row0 = grp_lo + m_tile * TM;
    t.valid = min(TM, grp_hi - t.row0);
    // activation instructions n = wave + 8 i with a valid row (16 n < valid);
    // lane l copies 16 bytes of row r = 16 n + l / 4: chunk c = (l % 4) ^ sw(r)
    // of the stage's 32 columns (rows past the tile read the last valid row)
    t.na = 0;
#pragma unroll
    for (int i = 0; i < kAPerWave; ++i) {
        t.na += (16 * (t.wave + 8 * i) < t.valid) ? 1 : 0;
        const int r = 16 * (t.wave + 8 * i) + (t.lane >> 2);
        const int c = (t.lane & 3) ^ swz(r);
        const size_t grow = (size_t)(t.row0 + min(r, t.valid - 1));
        size_t e;
        if (AM == A_BLK) e = blocked_index(grow, c * 8, t.K);
        else if (AM == A_GATHER) e = (size_t)args.gather[grow] * t.K + c * 8;
        else e = grow * t.K + c * 8;
        t.a_off[i] = (uint32_t)(e >> 3);
    }
    t.a_step = AM == A_BLK ? 512 / 8 : BK / 8;
    // this expert's packed matrices and the n-tile's first block
    t.np = (N + Pn::P - 1) / Pn::P;
    t.pstride = (size_t)Pn::P * t.K;
    const size_t ebase = (size_t)g * t.np * t.pstride;
    t.wsrc0 = args.w1 + ebase;
    t.wsrc1 = (EPI == EPI_SWIGLU_BF16 ? args.w2 : args.w1) + ebase;
    t.blk0 = n_tile * Pn::BPM;
    t.wstride = (size_t)Pn::BPP * 2048;
    t.n0 = n_tile * Pn::TN + t.wn * ((EPI == EPI_SWIGLU_BF16) ? 32 : 64);
    // the valid rows split evenly (in 32-row blocks) over the two wave halves
    t.mh = min(MH, (((t.valid + 1) >> 1) + 31) & ~31);
    const int wrows = min(max(t.valid - t.wm * t.mh, 0), t.mh);
    const int ntb = t.n0 < N ? (wrows + 31) / 32 : 0;
    run_tile_ntb<EPI, AM, MAXNTB>(t, ntb);
}

// Work items: a group of n > 0 rows has ceil(N / TN) x ceil(n / 256) items
// (n-tile major); every item streams the same weight bytes (one tile's
// panels).  Items are ordered (group, n-tile, m-tile) and the 8 XCDs take
// contiguous ranges of equal item count; inside an XCD the workgroups claim
// items in order from a per-XCD counter (args.sched, zeroed before the
// launch) or, without counters, take every 32nd item.  Workgroups of one XCD
// thus work on neighbouring items (the n-tiles of the same experts) at the
// same time and share their activations in L2, and a workgroup that drew
// cheap tiles (few valid rows) takes more of them.
template <int EPI, int AM>
__global__ __launch_bounds__(kThreads) void grouped_gemm_lds_kernel(GemmArgs args) {
    using Pn = Panel<EPI>;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int scan_sh[8];
    __shared__ int next_item;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int G = args.G, rows = args.rows, K = args.K, N = args.N;
    const int* offs = args.offsets;
    int* item_prefix = (int*)(smem + kRing);  // [G + 1]
    const int NT = (N + Pn::TN - 1) / Pn::TN;

    auto group_rows = [&](int g, int& lo, int& hi) {
        lo = 0;
        hi = rows;
        if (offs) {
            lo = min(max(offs[g], 0), rows);
            hi = max(lo, min(max(offs[g + 1], 0), rows));
        }
    };

    // ---- per-group item counts -> exclusive prefix in LDS ----
    {
        const int per = (G + kThreads - 1) / kThreads;
        const int g0 = tid * per;
        int local = 0;
        for (int g = g0; g < g0 + per && g < G; ++g) {
            int lo, hi;
            group_rows(g, lo, hi);
            const int items = NT * ((hi - lo + TM - 1) / TM);
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

    LdsTile t;
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
        int grp_lo, grp_hi;
        group_rows(g, grp_lo, grp_hi);
        do_tile<EPI, AM>(t, args, g, q - item_prefix[g], grp_lo, grp_hi);
        q = t.ctr ? next_item : q + per_xcd;
    }
}

template <int EPI, int AM>
hipError_t launch_lds(const GemmArgs& g, hipStream_t stream) {
    static int configured_device = -1;
    static int grid = 0;
    static size_t static_lds = 0;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (configured_device != dev) {
        hipFuncAttributes fa;
        err = hipFuncGetAttributes(&fa, (const void*)grouped_gemm_lds_kernel<EPI, AM>);
        if (err != hipSuccess) return err;
        static_lds = fa.sharedSizeBytes;
        if (static_lds > (size_t)kStaticLds) return hipErrorInvalidValue;
        err = hipFuncSetAttribute((const void*)grouped_gemm_lds_kernel<EPI, AM>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  kLdsLimit - (int)static_lds);
        if (err != hipSuccess) return err;
        grid = (device_cu_count() + 7) & ~7;
        configured_device = dev;
    }
    const size_t lds = kRing + (size_t)(g.G + 1) * sizeof(int);
    if (lds + static_lds > (size_t)kLdsLimit) return hipErrorInvalidValue;
    hipLaunchKernelGGL((grouped_gemm_lds_kernel<EPI, AM>), dim3(grid), dim3(kThreads), lds,
                       stream, g);
    return hipGetLastError();
}

}  // namespace

int grouped_gemm_lds_max_groups() {
    return (kLdsLimit - kStaticLds - kRing) / (int)sizeof(int) - 1;
}

hipError_t launch_grouped_gemm_lds(int epilogue, const GemmArgs& g, hipStream_t stream) {
    if (g.K % BK != 0 || g.G < 1) return hipErrorInvalidValue;
    // activation sources are 32-bit offsets in 16-byte units (a gathered a
    // has at most g.a_rows rows)
    const size_t a_rows = g.gather ? (size_t)g.a_rows : (size_t)g.rows;
    if (a_rows * g.K / 8 + 2 * (size_t)g.K >= (1ull << 32)) return hipErrorInvalidValue;
    if (g.gather && g.a_blocked) return hipErrorInvalidValue;
    const int am = g.gather ? A_GATHER : g.a_blocked ? A_BLK : A_ROW;
    switch (epilogue) {
        case EPI_SWIGLU_BF16:
            // h is blocked exactly when the activations are not plain row-major
            if (g.out_blocked != (am != A_ROW)) return hipErrorInvalidValue;
            if (am == A_GATHER) return launch_lds<EPI_SWIGLU_BF16, A_GATHER>(g, stream);
            if (am == A_BLK) return launch_lds<EPI_SWIGLU_BF16, A_BLK>(g, stream);
            return launch_lds<EPI_SWIGLU_BF16, A_ROW>(g, stream);
        case EPI_F32:
            if (am == A_GATHER) return launch_lds<EPI_F32, A_GATHER>(g, stream);
            if (am == A_BLK) return launch_lds<EPI_F32, A_BLK>(g, stream);
            return launch_lds<EPI_F32, A_ROW>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
