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
// The K loop runs in stages; the LDS ring (128 KB) holds either 4 slots of
// 32-wide stages (3 in flight, for tiles of at most 192 valid rows: few MFMAs
// per weight byte, so the deeper lookahead hides more memory latency) or 2
// slots of 64-wide stages (1 in flight while one computes, for fuller tiles:
// half the barriers and waits per K).  Measured on MI355X, the split beats
// either width alone on every workload tried.  Per stage one slot holds
//   - the activation tile, 256 rows x KB columns, the 16-byte chunks of row
//     r XOR-swizzled (swz), so that the 16 lanes an LDS cycle serves (256 B
//     over 64 banks) hit distinct banks in MFMA operand reads;
//   - the weight stage, KB / 16 substeps x 1 KB per 32-row block in
//     matrix-core fragment order (copied from the packed layout in 1 KB runs;
//     operand reads are 1 KB contiguous per wave).
// The DMA (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16 l)
// moves 1 KB per instruction: weight instructions and blocked-layout
// activation instructions read whole cache lines; row-major activations read
// 64 of 128 bytes per line at KB = 32, whole lines at KB = 64.  Each wave issues KB / 16 weight instructions and na
// activation instructions per stage (only the row groups that hold valid
// rows are copied); na is fixed for a tile, so vmcnt counts stay exact.  The
// DMA is issued from inline assembly, so the compiler does not see LDS writes
// it would otherwise guard with a full vmcnt drain before every LDS read;
// explicit vmcnt waits + one barrier per stage are the complete
// synchronisation, and the kernel keeps every other value in registers (a
// spill reload would make the compiler drain vmcnt inside the pipeline).
// Scheduling: see grouped_gemm_lds_kernel.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TM = 256;                      // activation rows per tile
constexpr int MH = TM / 2;                   // max rows per wave
constexpr int MAXNTB = MH / 32;              // activation blocks per wave
constexpr int WBLK = 8;                      // 32-row weight blocks per tile
constexpr int kRing = 128 * 1024;            // LDS operand ring (either stage width)
constexpr int kThreads = 512;
constexpr int kLdsLimit = 160 * 1024;
constexpr int kStaticLds = 256;              // reserve for static LDS (scan_sh, next_item)
// tiles with more valid rows than this take the 64-wide stages (MFMA-heavy),
// the others the 32-wide ones (memory-bound: deeper lookahead)
constexpr int kWideStageRows = 192;
// (MXFP8 weights: half the weight bytes per stage, so the 64-wide stages pay
// off from 129 valid rows; measured 2% faster at the 384-expert workload)
constexpr int kWideStageRowsFp8 = 128;


// Pipeline of one stage width KB (32 or 64 columns of K per stage).
//   KB = 32: 4 slots of 32 KB (16 KB activations + 16 KB weights), 3 stages
//            in flight; per stage 2 activation + 2 weight DMA instructions
//            per wave; the waits count the instructions of later stages.
//   KB = 64: 2 slots of 64 KB, 1 stage in flight while one computes; per
//            stage 4 + 4 instructions per wave; every wait is vmcnt(0).
//   WF = 2 (MXFP4 weights): a quarter of the bytes: one 512-byte chunk per
//            32-row block per 32 columns (a 16-byte DMA by lanes 0-31).
//   WF = 1 (MXFP8 weights): the weight stage is half as many bytes (one 1 KB
//            chunk per 32-row block per 32 columns of K) plus the 8 blocks'
//            scale bytes (256 per 32 columns: one more DMA instruction for
//            waves 0 .. KB/32 - 1), same slot count.
template <int KB, int WF = 0>
struct Stage {
    static_assert(KB == 32 || KB == 64, "stage width");
    static constexpr int ROWB = KB * 2;                    // LDS bytes per activation row
    static constexpr int LPR = ROWB / 16;                  // lanes per row in one DMA
    static constexpr int RPI = 64 / LPR;                   // rows per DMA instruction
    static constexpr int APW = TM / RPI / 8;               // activation instrs per wave (max)
    static constexpr int Q = KB / 16;                      // MFMA substeps per stage
    static constexpr int WI = WF ? KB / 32 : Q;            // weight instrs per wave (1 KB each)
    // (waves w < WI also issue one scale instruction per stage)
    static constexpr int SLOTA = TM * ROWB;
    static constexpr int CHUNK = WF == 2 ? 512 : 1024;    // bytes per weight instruction
    static constexpr int SLOTW = WBLK * WI * CHUNK;
    static constexpr int SLOTS_B = WF ? WBLK * (KB / 32) * 32 : 0;   // MXFP8 scale bytes
    static constexpr int SLOT = SLOTA + SLOTW + SLOTS_B;
    static constexpr int SLOTS = KB == 32 ? 4 : 2;
    static constexpr int AHEAD = SLOTS - 1;                // stages in flight
    static_assert(SLOTS * SLOT <= kRing, "ring");
};

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

// position swizzle of the 16-byte chunks of activation row r in LDS: the 16
// lanes an LDS cycle serves (256 B over 64 banks) read 16 rows of one chunk
// index and must hit distinct banks.  64-byte rows (KB = 32): rows r, r+4,
// r+8, r+12 share banks; 128-byte rows (KB = 64): rows of equal parity do.
template <int KB>
__device__ __forceinline__ int swz(int r) {
    return KB == 32 ? ((r >> 1) ^ (r >> 3)) & 3 : (r >> 1) & 7;
}

// 1 KB direct-to-LDS copy: lane l's 16 bytes from gaddr go to LDS byte
// lds_byte + 16 l.
// (lds_byte must be wave-uniform; readfirstlane makes that visible)
// M0 carries the LDS address of the copy.  The compiler may keep a value of
// its own in M0, so the block saves M0 in an SGPR of its own, sets it, issues
// the copy (one wait state after the M0 write, as the hardware requires) and
// restores it: M0 leaves the block as it came in.  The copy takes its LDS
// address from M0 when it issues, so the restore does not disturb it.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_byte) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0v), "v"(gaddr)
        : "memory");
}

// 4-byte direct-to-LDS copy: lane l's 4 bytes from gaddr go to LDS byte
// lds_byte + 4 l (only the active lanes copy); M0 handled as in dma16
__device__ __forceinline__ void dma4(const void* gaddr, uint32_t lds_byte) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0v), "v"(gaddr)
        : "memory");
}

// wait until at most N of this wave's memory operations are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait for the oldest in-flight stage (AHEAD - 1 later stages of na + NW
// instructions each may stay outstanding)
// instructions per stage: na activation + NW weight (+ sc scale)
template <int KB, int WF>
__device__ __forceinline__ void wait_stage(int na, int sc) {
    constexpr int A1 = Stage<KB, WF>::AHEAD - 1, NW = Stage<KB, WF>::WI;
    if constexpr (A1 == 0) {
        wait_vm<0>();
    } else if constexpr (WF) {
        const int n = na + sc;
        if (n == 3) wait_vm<A1 * (NW + 3)>();
        else if (n == 2) wait_vm<A1 * (NW + 2)>();
        else if (n == 1) wait_vm<A1 * (NW + 1)>();
        else wait_vm<A1 * NW>();
    } else {
        if (na == 2) wait_vm<A1 * (NW + 2)>();
        else if (na == 1) wait_vm<A1 * (NW + 1)>();
        else wait_vm<A1 * NW>();
    }
}

struct LdsTile {
    const GemmArgs* args;
    uint32_t lds0;         // LDS byte address of slot 0
    unsigned char* smem;
    int lane, wave, wm, wn, half, l32;
    int K, N;
    int row0, valid;
    int mh;                // activation rows per wave half (multiple of 32)
    int na;                // activation DMA instructions of this wave per stage
    uint32_t a_off[4];     // lane's stage-0 source of activation instruction i (16 B units)
    uint32_t a_step;       // ... advance per stage (16 B units)
    int n0;                // first weight row / feature of this wave's blocks
    const uint16_t* wsrc0; // this expert's packed matrix (gate matrix for SwiGLU)
    const uint16_t* wsrc1; // up matrix (SwiGLU) or the same
    const uint8_t* bsrc0;  // fp8 weights: this expert's code matrices (gate / the one)
    const uint8_t* bsrc1;  // fp8 weights: up matrix (SwiGLU) or the same
    size_t pstride_b;      // fp8 weights: bytes per panel
    size_t wstride_b;      // fp8 weights: bytes per 64-wide K stage of one panel
    const uint8_t* ssrc0;  // fp8 weights: MX block scale bytes of this expert (gate / the one)
    const uint8_t* ssrc1;  // fp8 weights: MX block scale bytes of the up matrix (SwiGLU)
    size_t sstride;        // fp8 weights: scale bytes per panel
    int blk0;              // first 32-row block of this n-tile in each matrix
    int np;                // packed panels per matrix
    size_t pstride;        // packed elements per panel
    size_t wstride;        // packed elements per 64-wide K stage of one panel
    unsigned* ctr;         // this XCD's item counter (dynamic scheduling) or NULL
    int* next_item;        // LDS slot receiving the claimed next item
    int item_lo;           // first item of this XCD's range
    int item_hi;           // end of this XCD's range
};

// DMA of pipeline stage j (KB columns of K) into the LDS slot at byte offset
// `sbase`.
//   activations: instruction n (rows [RPI n, RPI n + RPI) of the tile)
//     belongs to wave n % 8 and is issued only if the group holds a valid
//     row (the per-lane sources are set up per tile in t.a_off).
//   weights: the 64-wide packed stage holds, per 32-row block, 4 substeps x
//     1 KB; the stage takes Q of them from all 8 blocks: instruction
//     n = Q w + i copies tile block n / Q, substep n % Q (KB = 32: the half
//     j % 2 of the packed stage j / 2) to LDS fragment slot n.  SwiGLU tile
//     blocks [0, 4) are gate rows, [4, 8) up rows; a block of a panel past
//     the matrix end re-reads the last panel (its outputs are never stored).
template <int EPI, int KB, int WF>
__device__ __forceinline__ void issue_stage(const LdsTile& t, int j, uint32_t sbase) {
    using Pn = Panel<EPI>;
    using St = Stage<KB, WF>;
    const uint32_t base = t.lds0 + sbase;
    const GemmArgs& args = *t.args;
#pragma unroll
    for (int i = 0; i < St::APW; ++i) {
        if (i < t.na) {
            const int r0 = St::RPI * (t.wave + 8 * i);
            const uint32_t off = t.a_off[i] + (uint32_t)j * t.a_step;
            dma16((const u32x4*)args.a + off, base + r0 * St::ROWB);
        }
    }
    const int s64 = (j * KB) >> 6, sub0 = ((j * KB) & 63) >> 4;
    if constexpr (WF == 2) {
        // fp4 codes: wave w copies block w's 512-byte chunks of MX blocks
        // kb0 .. kb0 + WI - 1 (lanes 0-31, 16 bytes each) to slot WI w + i
        const int b = t.wave;
        const uint8_t* mat = t.bsrc0;
        int gb = t.blk0 + b;
        if (EPI == EPI_SWIGLU_BF16 && b >= Pn::BPM) {
            mat = t.bsrc1;
            gb -= Pn::BPM;
        }
        const int panel = min(gb / Pn::BPP, t.np - 1);
        const int kb0 = (j * KB) / 32;
        if (t.lane < 32) {
#pragma unroll
            for (int i = 0; i < St::WI; ++i) {
                const uint8_t* src = mat + (size_t)panel * t.pstride_b +
                                     (size_t)(kb0 + i) * (Pn::BPP * 512) + (gb % Pn::BPP) * 512 +
                                     t.lane * 16;
                dma16(src, base + St::SLOTA + (b * St::WI + i) * 512);
            }
        }
    }
    if constexpr (WF) {
        // fp8 codes: wave w copies block w, chunks c0 .. c0 + WI - 1 (each the
        // 32 columns of one 32-wide K slice, both substeps) to fragment slot
        // WI w + i
        const int b = t.wave;
        const uint8_t* mat = t.bsrc0;
        int gb = t.blk0 + b;
        if (EPI == EPI_SWIGLU_BF16 && b >= Pn::BPM) {
            mat = t.bsrc1;
            gb -= Pn::BPM;
        }
        const int panel = min(gb / Pn::BPP, t.np - 1);
        const int c0 = ((j * KB) & 63) >> 5;
        if constexpr (WF == 1) {
#pragma unroll
            for (int i = 0; i < St::WI; ++i) {
                const uint8_t* src = mat + (size_t)panel * t.pstride_b +
                                     (size_t)s64 * t.wstride_b + (gb % Pn::BPP) * 2048 +
                                     (c0 + i) * 1024 + t.lane * 16;
                dma16(src, base + St::SLOTA + (b * St::WI + i) * 1024);
            }
        }
        // scale bytes of MX block kb = j KB / 32 + w for all 8 weight blocks
        // (wave w < WI): lanes 8 b' .. 8 b' + 7 copy the 32 rows of block b'
        if (t.wave < St::WI) {
            const int bs = t.lane >> 3;
            const uint8_t* smat2 = t.ssrc0;
            int gs = t.blk0 + bs;
            if (EPI == EPI_SWIGLU_BF16 && bs >= Pn::BPM) {
                smat2 = t.ssrc1;
                gs -= Pn::BPM;
            }
            const int pans = min(gs / Pn::BPP, t.np - 1);
            const int kb = (j * KB) / 32 + t.wave;
            const uint8_t* ssrc = smat2 + (size_t)pans * t.sstride + (size_t)kb * Pn::P +
                                  (gs % Pn::BPP) * 32 + (t.lane & 7) * 4;
            dma4(ssrc, base + St::SLOTA + St::SLOTW + t.wave * 256);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < St::Q; ++i) {
        const int n = St::Q * t.wave + i;
        const int b = n / St::Q;
        const int sub = sub0 + n % St::Q;
        const uint16_t* mat = t.wsrc0;
        int gb = t.blk0 + b;
        if (EPI == EPI_SWIGLU_BF16 && b >= Pn::BPM) {
            mat = t.wsrc1;
            gb -= Pn::BPM;
        }
        const int panel = min(gb / Pn::BPP, t.np - 1);
        const uint16_t* src = mat + (size_t)panel * t.pstride + (size_t)s64 * t.wstride +
                              (gb % Pn::BPP) * 2048 + sub * 512 + t.lane * 8;
        dma16(src, base + St::SLOTA + n * 1024);
    }
}

// MFMA operands of one 16-wide K substep q of a stage: this wave's two weight
// fragments and its NTB activation fragments.
template <int NTB>
struct Operands {
    bf16x8 w0, w1, a[NTB];
};


template <int EPI, int KB, int NTB, int WF>
__device__ __forceinline__ void read_operands(const LdsTile& t, uint32_t sbase, int q,
                                              Operands<NTB>& o, float (&msc)[2]) {
    using St = Stage<KB, WF>;
    const unsigned char* base = t.smem + sbase;
    // weight blocks of this wave (bf16: fragment slots Q b + substep; fp8:
    // chunk slots WI b + substep / 2, substep parity selects the 8-byte half)
    const int b0 = (EPI == EPI_SWIGLU_BF16) ? t.wn : 2 * t.wn;
    const int b1 = (EPI == EPI_SWIGLU_BF16) ? Panel<EPI>::BPM + t.wn : 2 * t.wn + 1;
    if constexpr (WF) {
        // scale byte X + 127 of this lane's row and MX block -> 2^X
        // (scale region: [MX block of the stage][8 weight blocks][32 rows])
        if ((q & 1) == 0) {
            const unsigned char* sbase =
                base + St::SLOTA + St::SLOTW + (q >> 1) * 256 + (t.lane & 31);
            msc[0] = __uint_as_float((uint32_t)sbase[b0 * 32] << 23);
            msc[1] = __uint_as_float((uint32_t)sbase[b1 * 32] << 23);
        }
        if constexpr (WF == 2) {
            // fp4: lane l's 8 bytes at 8 l of the chunk, substep parity
            // selects the 4-byte half
            const unsigned char* wbase = base + St::SLOTA + t.lane * 8 + (q & 1) * 4;
            o.w0 = fp4x8_to_bf16x8(*(const uint32_t*)(wbase + (b0 * St::WI + (q >> 1)) * 512),
                                   msc[0]);
            o.w1 = fp4x8_to_bf16x8(*(const uint32_t*)(wbase + (b1 * St::WI + (q >> 1)) * 512),
                                   msc[1]);
        } else {
            const unsigned char* wbase = base + St::SLOTA + t.lane * 16 + (q & 1) * 8;
            o.w0 = fp8x8_to_bf16x8(*(const u32x2*)(wbase + (b0 * St::WI + (q >> 1)) * 1024),
                                   msc[0]);
            o.w1 = fp8x8_to_bf16x8(*(const u32x2*)(wbase + (b1 * St::WI + (q >> 1)) * 1024),
                                   msc[1]);
        }
    } else {
        const unsigned char* wbase = base + St::SLOTA + t.lane * 16;
        o.w0 = *(const bf16x8*)(wbase + (b0 * St::Q + q) * 1024);
        o.w1 = *(const bf16x8*)(wbase + (b1 * St::Q + q) * 1024);
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        const int r = t.wm * t.mh + tb * 32 + t.l32;
        const int c = (2 * q + t.half) ^ swz<KB>(r);
        o.a[tb] = *(const bf16x8*)(base + r * St::ROWB + c * 16);
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

template <int EPI, int AM, int NTB, int WF>
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

// K loop of one tile for a wave computing NTB 32-row blocks (0: DMA only),
// in stages of KB columns.  Stages j+1 .. j+AHEAD-1 stay in flight while
// stage j computes: wait for stage j (this wave's own DMA), barrier (all
// waves' DMA of stage j landed, and all waves are done reading the slot the
// next DMA overwrites), issue stage j + AHEAD into the slot stage j - 1 used,
// compute stage j.  With more than one stage in flight, stages past the end
// re-issue the last stage, so every iteration issues the same number of
// instructions and the vmcnt counts of wait_stage stay exact.
// Operand reads run one substep ahead of the MFMAs: after the barrier of
// stage j the wave reads substep 0 of stage j while it multiplies the last
// substep of stage j - 1 (read before this barrier), and so on.  Every LDS
// read latency hides behind MFMAs of the same wave; the reads of a slot
// complete before the next barrier, so the DMA that reuses the slot after
// that barrier never races them.
template <int EPI, int AM, int KB, int NTB, int WF>
__device__ __forceinline__ void run_tile(const LdsTile& t) {
    using St = Stage<KB, WF>;
    f32x16 acc[2][MAXNTB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int tb = 0; tb < MAXNTB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][tb][i] = 0.0f;
    const int S = t.K / KB;
    wait_vm<0>();  // retire the previous tile's stores before counting DMA entries
#pragma unroll
    for (int p = 0; p < St::AHEAD; ++p) issue_stage<EPI, KB, WF>(t, min(p, S - 1), p * St::SLOT);
    uint32_t s_cmp = 0, s_iss = St::AHEAD * St::SLOT;
    Operands<NTB> o[2];
    float msc[2] = {1.0f, 1.0f};
    for (int j = 0; j < S; ++j) {
        wait_stage<KB, WF>(t.na, WF && t.wave < St::WI ? 1 : 0);
        __syncthreads();
        // (one stage in flight: every wait is vmcnt(0), nothing to re-issue)
        if (St::AHEAD > 1 || j + 1 < S)
            issue_stage<EPI, KB, WF>(t, min(j + St::AHEAD, S - 1), s_iss);
        s_iss = (s_iss + St::SLOT == St::SLOTS * St::SLOT) ? 0 : s_iss + St::SLOT;
        if constexpr (NTB > 0) {
#pragma unroll
            for (int q = 0; q < St::Q; ++q) {
                read_operands<EPI, KB, NTB, WF>(t, s_cmp, q, o[q & 1], msc);
                __builtin_amdgcn_sched_barrier(0);
                if (q > 0 || j > 0) mfma_substep<NTB>(o[(q + 1) & 1], acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        s_cmp = (s_cmp + St::SLOT == St::SLOTS * St::SLOT) ? 0 : s_cmp + St::SLOT;
    }
    if constexpr (NTB > 0) mfma_substep<NTB>(o[(St::Q - 1) & 1], acc);
    // dynamic scheduling: thread 0 claims the workgroup's next item here,
    // after the last stage wait, so no claim is in flight while the K loop
    // counts DMA entries
    const bool claim = t.ctr != nullptr && threadIdx.x == 0;
    unsigned claimed = 0;
    if (claim) claimed = atomicAdd(t.ctr, 1u);
    wait_vm<0>();
    if (claim) *t.next_item = claimed_item(t.item_lo, t.item_hi, claimed);
    __syncthreads();
    if constexpr (NTB > 0) epilogue<EPI, AM, NTB, WF>(t, acc);
}

// run_tile for ntb in [0, NT] (ntb is wave-uniform)
template <int EPI, int AM, int KB, int NT, int WF>
__device__ __forceinline__ void run_tile_ntb(const LdsTile& t, int ntb) {
    if constexpr (NT == 0) {
        run_tile<EPI, AM, KB, 0, WF>(t);
    } else {
        if (ntb >= NT) run_tile<EPI, AM, KB, NT, WF>(t);
        else run_tile_ntb<EPI, AM, KB, NT - 1, WF>(t, ntb);
    }
}

// activation sources of a tile for stage width KB: instruction n = wave + 8 i
// (rows [RPI n, RPI n + RPI)) is issued if it holds a valid row; lane l
// copies 16 bytes of row r = RPI n + l / LPR: chunk c = (l % LPR) ^ swz(r) of
// the stage's KB columns (rows past the tile read the last valid row)
template <int AM, int KB>
__device__ __forceinline__ void setup_a(LdsTile& t, const GemmArgs& args) {
    using St = Stage<KB>;
    t.na = 0;
#pragma unroll
    for (int i = 0; i < St::APW; ++i) {
        t.na += (St::RPI * (t.wave + 8 * i) < t.valid) ? 1 : 0;
        const int r = St::RPI * (t.wave + 8 * i) + t.lane / St::LPR;
        const int c = (t.lane % St::LPR) ^ swz<KB>(r);
        const size_t grow = (size_t)(t.row0 + min(r, t.valid - 1));
        size_t e;
        if (AM == A_BLK) e = blocked_index(grow, c * 8, t.K);
        else if (AM == A_GATHER) e = (size_t)args.gather[grow] * t.K + c * 8;
        else e = grow * t.K + c * 8;
        t.a_off[i] = (uint32_t)(e >> 3);
    }
    // per stage: KB / 32 blocks of 512 elements (blocked) or KB elements
    t.a_step = AM == A_BLK ? KB * 2 : KB / 8;
}

// Tile of item (group g, local item index): set up the per-tile fields of t
// and run it.
template <int EPI, int AM, int WF>
__device__ __forceinline__ void do_tile(LdsTile& t, const GemmArgs& args, int g, int local,
                                        int grp_lo, int grp_hi) {
    using Pn = Panel<EPI>;
    const int N = args.N;
    // bf16 weights: m-tiles of TM rows, the last one shorter.  MX weights:
    // the group's rows split evenly over its mt m-tiles (per rows each,
    // rounded up to 16, the last tile shorter), so the m-tiles of one n-tile
    // run at the same pace and share their weight reads in L2; measured on
    // MI355X, 3% faster for MXFP8 weights at the 384-expert workload and 1%
    // slower for bf16.  Either way per <= TM, and the last tile holds a row:
    // n > TM (mt - 1) >= per (mt - 1).
    const int n = grp_hi - grp_lo;
    const int mt = (n + TM - 1) / TM;
    const int per = WF != 0 ? ((n + mt - 1) / mt + 15) & ~15 : TM;
    const int n_tile = local / mt, m_tile = local % mt;
    t.row0 = grp_lo + m_tile * per;
    t.valid = min(per, grp_hi - t.row0);
    // this expert's packed matrices and the n-tile's first block
    t.np = (N + Pn::P - 1) / Pn::P;
    t.pstride = (size_t)Pn::P * t.K;
    const size_t ebase = (size_t)g * t.np * t.pstride;
    t.wsrc0 = args.w1 + ebase;
    t.wsrc1 = (EPI == EPI_SWIGLU_BF16 ? args.w2 : args.w1) + ebase;
    t.blk0 = n_tile * Pn::BPM;
    t.wstride = (size_t)Pn::BPP * 2048;
    if constexpr (WF) {
        // fp8 codes: one byte per weight, panels of P rows x K bytes (fp4:
        // half a byte per weight)
        t.pstride_b = (size_t)Pn::P * t.K / (WF == 2 ? 2 : 1);
        const size_t ebase_b = (size_t)g * t.np * t.pstride_b;
        t.bsrc0 = (const uint8_t*)args.w1 + ebase_b;
        t.bsrc1 = (const uint8_t*)(EPI == EPI_SWIGLU_BF16 ? args.w2 : args.w1) + ebase_b;
        t.wstride_b = (size_t)Pn::BPP * 2048;
        t.sstride = (size_t)(t.K / 32) * Pn::P;
        t.ssrc0 = args.s1 + (size_t)g * t.np * t.sstride;
        t.ssrc1 = (EPI == EPI_SWIGLU_BF16 ? args.s2 : args.s1) + (size_t)g * t.np * t.sstride;
    }
    t.n0 = n_tile * Pn::TN + t.wn * ((EPI == EPI_SWIGLU_BF16) ? 32 : 64);
    // the valid rows split evenly (in 32-row blocks) over the two wave halves
    t.mh = min(MH, (((t.valid + 1) >> 1) + 31) & ~31);
    const int wrows = min(max(t.valid - t.wm * t.mh, 0), t.mh);
    const int ntb = t.n0 < N ? (wrows + 31) / 32 : 0;
    if (t.valid > (WF ? kWideStageRowsFp8 : kWideStageRows)) {
        setup_a<AM, 64>(t, args);
        run_tile_ntb<EPI, AM, 64, MAXNTB, WF>(t, ntb);
    } else {
        setup_a<AM, 32>(t, args);
        run_tile_ntb<EPI, AM, 32, MAXNTB, WF>(t, ntb);
    }
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
template <int EPI, int AM, int WF>
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
    t.ctr = args.sched ? args.sched + xcd * 32 : nullptr;
    t.next_item = &next_item;
    t.item_lo = item_lo;
    t.item_hi = item_hi;

    int q;
    if (t.ctr) {
        if (tid == 0) next_item = claimed_item(item_lo, item_hi, atomicAdd(t.ctr, 1u));
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
        do_tile<EPI, AM, WF>(t, args, g, q - item_prefix[g], grp_lo, grp_hi);
        q = t.ctr ? next_item : q + per_xcd;
    }
}

template <int EPI, int AM, int WF = 0>
hipError_t launch_lds(const GemmArgs& g, hipStream_t stream) {
    // per device, once: the dynamic LDS limit and the grid (one workgroup per
    // CU, whole rounds of the 8 XCDs)
    static DeviceSetup setup;
    long long grid = 0, static_lds = 0;
    const hipError_t err = device_setup(setup, grid, static_lds, [](int, long long& gr,
                                                                    long long& st) {
        hipFuncAttributes fa;
        hipError_t e = hipFuncGetAttributes(&fa, (const void*)grouped_gemm_lds_kernel<EPI, AM, WF>);
        if (e != hipSuccess) return e;
        if (fa.sharedSizeBytes > (size_t)kStaticLds) return hipErrorInvalidValue;
        e = hipFuncSetAttribute((const void*)grouped_gemm_lds_kernel<EPI, AM, WF>,
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                kLdsLimit - (int)fa.sharedSizeBytes);
        if (e != hipSuccess) return e;
        st = (long long)fa.sharedSizeBytes;
        gr = (device_cu_count() + 7) & ~7;
        return hipSuccess;
    });
    if (err != hipSuccess) return err;
    const size_t lds = kRing + (size_t)(g.G + 1) * sizeof(int);
    if (lds + (size_t)static_lds > (size_t)kLdsLimit) return hipErrorInvalidValue;
    hipLaunchKernelGGL((grouped_gemm_lds_kernel<EPI, AM, WF>), dim3((unsigned)grid), dim3(kThreads),
                       lds, stream, g);
    return hipGetLastError();
}

}  // namespace

int grouped_gemm_lds_max_groups() {
    return (kLdsLimit - kStaticLds - kRing) / (int)sizeof(int) - 1;
}

hipError_t launch_grouped_gemm_lds(int epilogue, const GemmArgs& g, hipStream_t stream) {
    if (g.K % 64 != 0 || g.G < 1) return hipErrorInvalidValue;
    // activation sources are 32-bit offsets in 16-byte units (a gathered a
    // has at most g.a_rows rows)
    const size_t a_rows = g.gather ? (size_t)g.a_rows : (size_t)g.rows;
    if (a_rows * g.K / 8 + 2 * (size_t)g.K >= (1ull << 32)) return hipErrorInvalidValue;
    if (g.gather && g.a_blocked) return hipErrorInvalidValue;
    const int am = g.gather ? A_GATHER : g.a_blocked ? A_BLK : A_ROW;
    if (g.wfp8) {
        // fp8 weights: the two routed expert GEMMs of moe_forward (gate/up
        // on gathered token rows, down on the blocked h)
        if (!g.s1 || (epilogue == EPI_SWIGLU_BF16 && !g.s2)) return hipErrorInvalidValue;
        if (g.wfp8 == 2) {
            if (epilogue == EPI_SWIGLU_BF16 && am == A_GATHER && g.out_blocked)
                return launch_lds<EPI_SWIGLU_BF16, A_GATHER, 2>(g, stream);
            if (epilogue == EPI_F32 && am == A_BLK) return launch_lds<EPI_F32, A_BLK, 2>(g, stream);
            return hipErrorInvalidValue;
        }
        if (epilogue == EPI_SWIGLU_BF16 && am == A_GATHER && g.out_blocked)
            return launch_lds<EPI_SWIGLU_BF16, A_GATHER, 1>(g, stream);
        if (epilogue == EPI_F32 && am == A_BLK) return launch_lds<EPI_F32, A_BLK, 1>(g, stream);
        return hipErrorInvalidValue;
    }
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
