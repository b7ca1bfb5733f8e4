// One-time quantisation of bf16 expert weights to MXFP8 (and MXFP4, below)
// for the 8-bit and 4-bit weight modes of the expert GEMMs.
//
// The pages name MXFP8 / MXFP4 weights as the low-precision direction
// ("CANN DeepSeek-V4 training optimisation": outlook section,
// functional-expansion bullets; FP4/FP8 checkpoints in the quick start of
// "Twinkle x Ascend ... DeepSeek-V4 training").  MXFP8 (OCP
// Microscaling): blocks of 32 values along K share one power-of-two scale,
// each value an OCP E4M3 float (bias 7, subnormals, no infinities, largest
// finite 448).  Scale rule of the OCP specification: X = floor(log2(block
// max |v|)) - 8, clamped here to [-110, 110] (0 for an all-zero block);
// q = E4M3(v / 2^X), round to nearest even, saturating at +-448.  The
// dequantised value E4M3(q) * 2^X is exactly a bf16 value; the GEMM decodes
// codes and scale together (v_cvt_scalef32_pk_f32_fp8, exact for these
// scales) into the bf16 operands of the matrix cores.
//
// Layout of the codes (per matrix, panels of P rows, K multiple of 64):
//   [G][ceil(N/P)][K/64][P/32][2][64 lanes][16 bytes]; chunk c of 32-row
//   block b, lane l holds row panel*P + b*32 + l%32, columns
//   64 s + 32 c + 8 (l/32) + {0..7} (bytes 0-7) and the same + 16 (bytes
//   8-15): the operand fragments of the two 16-wide MFMA substeps of that
//   32-wide K slice, which is one MX block.  Rows >= N are zero codes.
// Scales: one byte X + 127 per (row, block), [G][ceil(N/P)][K/32][P/32][32]:
//   the 32 rows of one 32-row weight block for one K block are contiguous.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxExp = 110;

// One thread per 16-byte chunk of codes (16 values of one MX block of one
// row): block exponent from all 32 values of the block, then its 16 codes;
// the lane holding columns 0-7 of the block also writes the scale byte.
__global__ __launch_bounds__(256) void mxfp8_pack_kernel(const uint16_t* __restrict__ src,
                                                         uint8_t* __restrict__ dst,
                                                         uint8_t* __restrict__ scales, int N,
                                                         int K, int P, long long nchunks) {
    const long long f = (long long)blockIdx.x * 256 + threadIdx.x;
    if (f >= nchunks) return;
    const int lane = (int)(f & 63);
    const int c = (int)((f >> 6) & 1);
    long long r = f >> 7;
    const int bpp = P / 32;
    const int b = (int)(r % bpp);
    r /= bpp;
    const int S = K / 64;
    const int s = (int)(r % S);
    r /= S;
    const int np = (N + P - 1) / P;
    const int panel = (int)(r % np);
    const long long g = r / np;
    const int row = panel * P + b * 32 + (lane & 31);
    const int kb = 2 * s + c;                             // MX block (32 columns)
    u32x4 out = {0u, 0u, 0u, 0u};
    int X = 0;
    if (row < N) {
        const uint16_t* bp = src + (g * N + row) * (long long)K + 32 * kb;
        float amax = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const u32x4 w = *(const u32x4*)(bp + 8 * v);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
                amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
            }
        }
        X = mx8_exponent(amax);
        const float inv = __builtin_ldexpf(1.0f, -X);   // exact power of two
        const uint16_t* rp = bp + 8 * (lane >> 5);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 w = *(const u32x4*)(rp + 16 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = e4m3_rne(__uint_as_float(w[i] << 16) * inv);
                const uint32_t hi = e4m3_rne(__uint_as_float(w[i] & 0xffff0000u) * inv);
                const int byte = 8 * h + 2 * i;           // elements 2i, 2i+1 of half h
                out[byte >> 2] |= (lo | (hi << 8)) << (8 * (byte & 3));
            }
        }
    }
    *(u32x4*)(dst + f * 16) = out;
    if (lane < 32)
        scales[((g * np + panel) * (K / 32) + kb) * (long long)P + b * 32 + lane] =
            (uint8_t)(X + 127);
}

// E2M1 code of a finite v: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to
// the even code (mantissa bit 0), saturating at 6.  Every threshold is an
// exact midpoint; at a tie the comparison direction picks the even code.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
    const float a = fabsf(v);
    const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return sign | m;
}

// MXFP4 codes: [G][ceil(N/P)][K/32][P/32][64 lanes][8 bytes]; lane l of the
// 512-byte chunk of (K block kb, 32-row block b) holds row b*32 + l%32,
// columns 32 kb + 8 (l/32) + {0..7} in bytes 0-3 and the same + 16 in bytes
// 4-7, two values per byte, the lower column in the low nibble.  One thread
// per (row, K block): block exponent, 32 codes (two lanes' 8 bytes), scale.
__global__ __launch_bounds__(256) void mxfp4_pack_kernel(const uint16_t* __restrict__ src,
                                                         uint8_t* __restrict__ dst,
                                                         uint8_t* __restrict__ scales, int N,
                                                         int K, int P, long long nthreads) {
    const long long f = (long long)blockIdx.x * 256 + threadIdx.x;
    if (f >= nthreads) return;
    const int r = (int)(f & 31);
    long long q = f >> 5;
    const int bpp = P / 32;
    const int b = (int)(q % bpp);
    q /= bpp;
    const int KB = K / 32;
    const int kb = (int)(q % KB);
    q /= KB;
    const int np = (N + P - 1) / P;
    const int panel = (int)(q % np);
    const long long g = q / np;
    const int row = panel * P + b * 32 + r;
    uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};   // lane r, lane r + 32: bytes 0-3, 4-7
    int X = 0;
    if (row < N) {
        const uint16_t* bp = src + (g * N + row) * (long long)K + 32 * kb;
        float v[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 w = *(const u32x4*)(bp + 8 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
        if (amax > 0.0f) {
            const int e = (int)((__float_as_uint(amax) >> 23) & 0xff) - 127;
            X = min(max(e - 2, -kMaxExp), kMaxExp);
        }
        const float inv = __builtin_ldexpf(1.0f, -X);
        // column c of the block: lane half h = (c / 8) % 2, word (c / 16),
        // nibble position c % 8 within that word
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const uint32_t code = e2m1_rne(v[c] * inv);
            const int h = (c >> 3) & 1, word = c >> 4, nib = c & 7;
            if (word == 0) (h ? lo[1] : lo[0]) |= code << (4 * nib);
            else (h ? hi[1] : hi[0]) |= code << (4 * nib);
        }
    }
    uint8_t* chunk = dst + ((((g * np + panel) * KB + kb) * bpp + b) * 512);
    *(u32x2*)(chunk + 8 * r) = u32x2{lo[0], hi[0]};
    *(u32x2*)(chunk + 8 * (r + 32)) = u32x2{lo[1], hi[1]};
    scales[((g * np + panel) * KB + kb) * (long long)P + b * 32 + r] = (uint8_t)(X + 127);
}

// MXFP8 quantisation of activation rows (the A8W4 mode's x): one thread per
// MX block of 32 values of one row, 64 bytes in (four 16-byte loads), 32
// codes and one scale byte out.
__global__ __launch_bounds__(256) void mxfp8_rows_kernel(const uint16_t* __restrict__ a,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         long long nblocks) {
    const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    const uint16_t* bp = a + b * 32;
    u32x4 w[4];
    float amax = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        w[v] = *(const u32x4*)(bp + 8 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(__uint_as_float(w[v][i] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(w[v][i] & 0xffff0000u)));
        }
    }
    const int X = mx8_exponent(amax);
    const float inv = __builtin_ldexpf(1.0f, -X);       // exact power of two
    u32x4 out[2];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            // elements 8 v + 2 i .. 8 v + 2 i + 3: one 32-bit word of codes
            uint32_t word = 0;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t lo = e4m3_rne(__uint_as_float(w[v][i + u] << 16) * inv);
                const uint32_t hi = e4m3_rne(__uint_as_float(w[v][i + u] & 0xffff0000u) * inv);
                word |= (lo | (hi << 8)) << (16 * u);
            }
            out[v >> 1][2 * (v & 1) + (i >> 1)] = word;
        }
    *(u32x4*)(codes + b * 32) = out[0];
    *(u32x4*)(codes + b * 32 + 16) = out[1];
    scales[b] = (uint8_t)(X + 127);
}

}  // namespace

hipError_t launch_quant_rows_mxfp8(const uint16_t* a, long long rows, int K, uint8_t* codes,
                                   uint8_t* scales, hipStream_t stream) {
    if (rows < 0 || K % 32) return hipErrorInvalidValue;
    const long long nblocks = rows * (K / 32);
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL(mxfp8_rows_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0,
                       stream, a, codes, scales, nblocks);
    return hipGetLastError();
}

size_t packed_fp8_weight_bytes(int G, int N, int K, int P) {
    return (size_t)G * (size_t)((N + P - 1) / P) * P * (size_t)K;
}

size_t packed_fp8_scale_bytes(int G, int N, int K, int P) {
    return packed_fp8_weight_bytes(G, N, K, P) / 32;
}

size_t packed_fp4_weight_bytes(int G, int N, int K, int P) {
    return packed_fp8_weight_bytes(G, N, K, P) / 2;
}

hipError_t launch_pack_weights_fp4(const uint16_t* src, uint8_t* dst, uint8_t* scales, int G,
                                   int N, int K, int P, hipStream_t stream) {
    const long long nthreads = (long long)packed_fp8_weight_bytes(G, N, K, P) / 32;
    if (nthreads == 0) return hipSuccess;
    hipLaunchKernelGGL(mxfp4_pack_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0,
                       stream, src, dst, scales, N, K, P, nthreads);
    return hipGetLastError();
}

hipError_t launch_pack_weights_fp8(const uint16_t* src, uint8_t* dst, uint8_t* scales, int G,
                                   int N, int K, int P, hipStream_t stream) {
    const long long nchunks = (long long)packed_fp8_weight_bytes(G, N, K, P) / 16;
    if (nchunks == 0) return hipSuccess;
    hipLaunchKernelGGL(mxfp8_pack_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0,
                       stream, src, dst, scales, N, K, P, nchunks);
    return hipGetLastError();
}

}  // namespace moe
