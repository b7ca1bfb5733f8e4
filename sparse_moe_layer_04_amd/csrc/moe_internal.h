// Internal declarations shared by the HIP translation units of the MoE
// library: kernel launchers (host side) and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- device ----
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

// fp32 -> bf16 bits, round to nearest even (quiet NaN kept NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// eight E4M3 codes (bytes of v, in order) times the MX block scale sc (a
// power of two in [2^-110, 2^110]) -> bf16x8.  The products have at most 4
// significant bits and a normal exponent, so the conversion is exact (on
// MI355X it gives the upper halves of the exact fp32 products, checked for
// every code and scales 2^-110 .. 2^110).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 v, float sc) {
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], sc, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], sc, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], sc, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], sc, true);
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, p0);
    r[1] = __builtin_bit_cast(uint32_t, p1);
    r[2] = __builtin_bit_cast(uint32_t, p2);
    r[3] = __builtin_bit_cast(uint32_t, p3);
    return __builtin_bit_cast(bf16x8, r);
}

// eight E2M1 codes (nibbles of v, low nibble first) times the MX block scale
// -> bf16x8 (exact: at most 2 significant bits, normal range; checked on
// MI355X for every byte and scales 2^-110 .. 2^110)
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t v, float sc) {
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 3));
    return __builtin_bit_cast(bf16x8, r);
}

// ----------------------------------------------------------------- host -----
// Number of compute units of the current device (cached per device).
int device_cu_count();

// Per-device one-time set-up (kernel attributes, grid sizes) that is safe
// when several host threads make their first calls at once: the set-up of a
// device runs exactly once (std::call_once), later callers wait for it and
// then read its error code and the two values it stored.  A failed set-up
// is not retried.
constexpr int kMaxDevices = 64;

struct DeviceSetup {
    std::once_flag once[kMaxDevices];
    hipError_t err[kMaxDevices] = {};
    long long v0[kMaxDevices] = {};
    long long v1[kMaxDevices] = {};
};

// setup(dev, v0, v1) -> hipError_t runs once for the current device.
template <class F>
inline hipError_t device_setup(DeviceSetup& s, long long& v0, long long& v1, F&& setup) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(s.once[dev], [&] { s.err[dev] = setup(dev, s.v0[dev], s.v1[dev]); });
    v0 = s.v0[dev];
    v1 = s.v1[dev];
    return s.err[dev];
}

// Grouped GEMM epilogues.
enum GemmEpilogue : int {
    EPI_SWIGLU_BF16 = 0,  // out = bf16(silu(clamp(A W1^T)) * clamp(A W2^T))
    EPI_F32 = 1,          // out = fp32(A W1^T)
    EPI_F32_OFFSET = 2,   // out = fp32(A W1^T + offset[n])
};

// OCP E4M3 code of a finite v: round to nearest, ties to even, saturating
// at +-448 (subnormal codes below 2^-6, spacing 2^-9)
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a >= 448.0f) return sign | 0x7eu;
    if (a < 0x1p-6f) {
        const float m = __builtin_rintf(a * 512.0f);   // exact product; 0 .. 8
        return sign | (uint32_t)m;                     // 8 = code 0x08, the smallest normal
    }
    const uint32_t ua = __float_as_uint(a);
    int E = (int)(ua >> 23) - 127;
    const uint32_t mant = ua & 0x7fffffu;
    uint32_t r = (mant + 0x7ffffu + ((mant >> 20) & 1u)) >> 20;   // 3 bits, ties to even
    if (r == 8u) {
        r = 0u;
        E += 1;
    }
    if (E > 8 || (E == 8 && r > 6u)) return sign | 0x7eu;
    return sign | ((uint32_t)(E + 7) << 3) | r;
}

// MXFP8 block exponent X = floor(log2 amax) - 8 clamped to [-110, 110], 0
// for an all-zero block (the scale byte is X + 127).  floor(log2) from the
// exponent field: a subnormal amax is below 2^-126 and clamps anyway.
__device__ __forceinline__ int mx8_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xff) - 127;
    return min(max(e - 8, -110), 110);
}

struct GemmArgs {
    const uint16_t* a;        // [rows, K] bf16 activations ([a_rows, K] when gathered)
    const int32_t* offsets;   // [G+1] device group row offsets, or NULL: one group [0, rows)
    int G;
    int rows;
    int K;
    int N;                    // weight rows per group (outputs per row)
    const uint16_t* w1;       // [G, N, K] bf16
    const uint16_t* w2;       // [G, N, K] bf16 (SWIGLU: up projection)
    const float* offset;      // [N] (EPI_F32_OFFSET) or NULL
    float clamp_limit;
    int clamp_mode;
    int packed;               // weights in the moe_pack_weights layout
    void* out;                // [rows, N] bf16 (SWIGLU) or fp32
    int a_blocked;            // a in the blocked activation layout (below)
    const int32_t* gather;    // LDS kernel: row r of A is row gather[r] of a (or NULL)
    int a_rows;               // rows of a when gathered
    int out_blocked;          // SWIGLU out in the blocked activation layout
    uint32_t* sched;          // LDS kernel: 8 per-XCD item counters, 128 B apart,
                              // zero at launch (NULL: static schedule)
    int wfp8;                 // LDS kernel: 1: w1 / w2 hold MXFP8 codes (moe_pack_weights_fp8),
                              // 2: MXFP4 codes (moe_pack_weights_fp4); block scales in s1 / s2
    const uint8_t* s1;        // MXFP8 block scale bytes of w1
    const uint8_t* s2;        // MXFP8 block scale bytes of w2 (SWIGLU)
    float* out_g;             // flat kernel, SWIGLU: [rows, N] fp32 gate pre-activations
    float* out_u;             // ... and up pre-activations (both or neither; NULL: not saved)
    // A8W4 (wfp8 == 3, flat kernel): MXFP8 activations and MXFP4 weights
    const uint8_t* a8;        // [rows (a_rows when gathered), K] E4M3 codes
    const uint8_t* a_scale;   // [.., K / 32] block scale bytes X + 127 of a8
    uint8_t* out_scale;       // SWIGLU: out is [rows, N] E4M3 codes of h, these its
                              // [rows, N / 32] scale bytes
};
// per-launch scheduling counters of the LDS-staged expert GEMM
constexpr int kSchedWords = 8 * 32;
// largest contraction length K of the flat expert GEMM: one 256-row packed
// weight panel (K 256 bf16 values) stays within a buffer resource's 2 GiB
constexpr int kFlatMaxK = (0x7fffffff / (256 * 2)) / 64 * 64;

// The item a workgroup claims from its XCD's counter: item_lo plus the
// counter's previous value, or item_hi (no item) when that value is past the
// XCD's range, so a counter that was not cleared before the launch cannot
// send a workgroup outside its items.
__device__ __forceinline__ int claimed_item(int item_lo, int item_hi, unsigned claimed) {
    return claimed < (unsigned)(item_hi - item_lo) ? item_lo + (int)claimed : item_hi;
}

// Blocked activation layout (internal to moe_forward): a [rows, K] bf16
// matrix stored as 1 KB blocks of 16 rows x 32 columns, blocks ordered by row
// block then column block, each block row-major:
//   elem(r, c) at ((r / 16) * (K / 32) + c / 32) * 512 + (r % 16) * 32 + c % 32.
// K must be a multiple of 32 and the buffer must hold ceil(rows / 16) * 16
// rows.  Sixteen consecutive rows of a 32-wide K slice are then 1 KB of
// contiguous memory, which is what the expert GEMM copies per DMA
// instruction.
__host__ __device__ __forceinline__ size_t blocked_index(size_t r, size_t c, size_t K) {
    return ((r >> 4) * (K >> 5) + (c >> 5)) * 512 + (r & 15) * 32 + (c & 31);
}
inline size_t blocked_rows(size_t rows) { return (rows + 15) & ~size_t(15); }

hipError_t launch_grouped_gemm(int epilogue, const GemmArgs& g, hipStream_t stream);
// Router projection on packed router weights (panel_rows 256): logits[T,E] =
// x W_g^T (+ offset), every output accumulated like the grouped GEMM's.
hipError_t launch_router_packed(const uint16_t* x, const uint16_t* wg_packed, const float* offset,
                                int T, int K, int E, float* logits, hipStream_t stream);
// whether launch_router_packed is the faster router for T tokens, E experts
bool router_packed_preferred(int T, int E);
// Expert GEMMs on packed weights (EPI_SWIGLU_BF16 with 128-row panels,
// EPI_F32 with 256-row panels): tiles staged in LDS by DMA.  Takes
// G <= grouped_gemm_lds_max_groups().
hipError_t launch_grouped_gemm_lds(int epilogue, const GemmArgs& g, hipStream_t stream);
int grouped_gemm_lds_max_groups();
// Expert GEMMs on packed bf16 weights, weights streamed into registers and
// only the activation rows staged in LDS (128 x 512 tiles).  Takes
// G <= grouped_gemm_flat_max_groups().
hipError_t launch_grouped_gemm_flat(int epilogue, const GemmArgs& g, hipStream_t stream);
int grouped_gemm_flat_max_groups();
size_t packed_weight_elems(int G, int N, int K, int P);
hipError_t launch_pack_weights(const uint16_t* src, uint16_t* dst, int G, int N, int K, int P,
                               hipStream_t stream);

// MXFP8 expert weights (E4M3 codes, one power-of-two scale per 32 values of K)
size_t packed_fp8_weight_bytes(int G, int N, int K, int P);
size_t packed_fp8_scale_bytes(int G, int N, int K, int P);
// MXFP8 quantisation of bf16 rows [rows, K] (K multiple of 32): E4M3 codes
// [rows, K] and scale bytes X + 127 [rows, K / 32]
hipError_t launch_quant_rows_mxfp8(const uint16_t* a, long long rows, int K, uint8_t* codes,
                                   uint8_t* scales, hipStream_t stream);
hipError_t launch_pack_weights_fp8(const uint16_t* src, uint8_t* dst, uint8_t* scales, int G,
                                   int N, int K, int P, hipStream_t stream);
// MXFP4 expert weights (E2M1 codes, two per byte; the same scale layout)
size_t packed_fp4_weight_bytes(int G, int N, int K, int P);
hipError_t launch_pack_weights_fp4(const uint16_t* src, uint8_t* dst, uint8_t* scales, int G,
                                   int N, int K, int P, hipStream_t stream);

hipError_t launch_route(const float* logits, const float* bias, const uint8_t* modality,
                        const int32_t* input_ids, const int32_t* tid2eid, int T, int E, int k,
                        int n_bias, int V, int mode, float scale, int32_t* ids, float* w,
                        uint32_t* flags, hipStream_t stream);

hipError_t launch_swiglu_backward(const float* gate, const float* up, const float* dh,
                                  long long n, float clamp_limit, int clamp_mode, float* dgate,
                                  float* dup, hipStream_t stream);

hipError_t launch_combine_backward(const float* dy, const float* y_perm, const int32_t* dest,
                                   const float* w, int T, int d, int k, int rows, float* dy_perm,
                                   float* dw, hipStream_t stream);
// the same with the gradient rows written as bf16 (d a multiple of 4)
hipError_t launch_combine_backward_bf16(const float* dy, const float* y_perm,
                                        const int32_t* dest, const float* w, int T, int d, int k,
                                        int rows, uint16_t* dy_perm, float* dw,
                                        hipStream_t stream);

hipError_t launch_route_backward(const float* logits, const int32_t* ids, const float* dw,
                                 int T, int E, int k, float scale, float* dl, uint32_t* flags,
                                 hipStream_t stream);

// dw[g] = dy[rows of g]^T a[rows of g] (fp32), every group's dw written;
// row r of dy at dy + r * ld_dy, of a at a + r * ld_a
hipError_t launch_grouped_wgrad(const uint16_t* dy, const uint16_t* a, const int32_t* offsets,
                                int G, int rows, int M, int K, float* dw, hipStream_t stream,
                                int ld_dy = 0, int ld_a = 0);
// the clamped-SwiGLU backward for rows x F pre-activations with bf16 outputs
// side by side: dgu[r, f] = dG, dgu[r, F + f] = dU (row stride 2F); the same
// fp32 arithmetic as launch_swiglu_backward, rounded once to bf16
hipError_t launch_swiglu_backward_bf16(const float* gate, const float* up, const float* dh,
                                       long long rows, int F, float clamp_limit, int clamp_mode,
                                       uint16_t* dgu, hipStream_t stream);
// dst[i] = bf16(src[i]) (nearest even), n values
hipError_t launch_cast_bf16(const float* src, long long n, uint16_t* dst, hipStream_t stream);
// router projection gradients from the logits' gradient dl [T, E] (fp32),
// using that dl is zero off each token's selected experts:
//   dx[t, :] += sum_j dl[t, ids_j] w_g[ids_j, :]          (accumulated into dx)
//   dwg[e, :] = sum_{rows r of expert e} dl[src_r, e] x[src_r, :]
hipError_t launch_router_backward(const float* dl, const int32_t* ids, const int32_t* offsets,
                                  const int32_t* src, const uint16_t* x, const uint16_t* wg,
                                  int T, int d, int E, int k, float* dx, float* dwg,
                                  hipStream_t stream);

size_t permute_workspace_bytes(int T, int k, int E);
// moe_permute's argument checks other than the workspace (MOE_OK or the
// error code)
int permute_arg_checks(const int32_t* topk_ids, const uint16_t* x, int T, int d, int E, int k,
                       const int32_t* counts, const int32_t* offsets, const int32_t* dest,
                       const int32_t* src, const uint16_t* x_perm);
hipError_t launch_permute(const int32_t* ids, const uint16_t* x, int T, int d, int E, int k,
                          int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                          uint16_t* x_perm, uint32_t* flags, void* ws, hipStream_t stream,
                          uint32_t* zero = nullptr, int nzero = 0);
// (x_perm may be NULL: dest/src only; the rank kernel also clears
// zero[0, nzero): the expert GEMMs' counters)

// (w may be NULL: every weight 1, the dispatch gather's backward)
hipError_t launch_combine(const float* y_perm, const int32_t* dest, const float* w,
                          const float* y_shared, int T, int d, int k, int rows, int out_dtype,
                          void* y, hipStream_t stream);

}  // namespace moe
