// One-time quantisation of bf16 expert weights to 8-bit floats for the fp8
// weight mode of the expert GEMMs.
//
// The pages name FP8 expert weights as the low-precision direction
// ("Twinkle x Ascend ... DeepSeek-V4 training": MXFP8 / MXFP4 in the
// functional-expansion section, FP4/FP8 checkpoints in the quick start) but
// fix no encoding.  Encoding used: OCP E4M3 (bias 7, subnormals, no
// infinities, largest finite 448) with one power-of-two scale per output
// row: e = the smallest integer with max_k |W[n,k]| <= 448 * 2^e (0 for a
// zero row, clamped to [-110, 110]); q = E4M3(W / 2^e), round to nearest
// even, saturating at +-448.  The dequantised weight E4M3(q) * 2^e is
// exactly a bf16 value, so the GEMM multiplies the bf16 activations by the
// decoded codes and applies 2^e to the fp32 accumulator (exact).
//
// Layout of the codes (per matrix, panels of P rows, K multiple of 64):
//   [G][ceil(N/P)][K/64][P/32][2][64 lanes][16 bytes]; chunk c of 32-row
//   block b, lane l holds row panel*P + b*32 + l%32, columns
//   64 s + 32 c + 8 (l/32) + {0..7} (bytes 0-7) and the same + 16 (bytes
//   8-15): the operand fragments of the two 16-wide MFMA substeps of that
//   32-wide K slice.  Rows >= N are zero codes.  Scales: fp32 2^e, [G, N].
#include "moe_internal.h"

namespace moe {
namespace {

constexpr float kE4M3Max = 448.0f;
constexpr int kMaxExp = 110;

// E4M3 code of a finite v, round to nearest even, saturating
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a >= kE4M3Max) return sign | 0x7eu;
    if (a < 0x1p-6f) {                          // subnormal codes, spacing 2^-9
        const float m = __builtin_rintf(a * 512.0f);   // exact product; 0 .. 8
        return sign | (uint32_t)m;              // 8 = code 0x08, the smallest normal
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

// one wave per row: amax -> e -> scales[row] = 2^e
__global__ __launch_bounds__(256) void fp8_row_scale_kernel(const uint16_t* __restrict__ src,
                                                            long long rows, int K,
                                                            float* __restrict__ scales) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const u32x4* p = (const u32x4*)(src + row * K);
    float amax = 0.0f;
    for (int v = lane; v < K / 8; v += 64) {
        const u32x4 w = p[v];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane != 0) return;
    int e = 0;
    if (amax > 0.0f) {
        // 2^(x-1) <= amax < 2^x, then the smallest e with amax <= 448 * 2^e
        int x = (int)((__float_as_uint(amax) >> 23) & 0xff) - 126;
        if ((__float_as_uint(amax) >> 23) == 0) x = -125;   // (bf16 subnormal amax)
        e = x - 9;
        while (e < kMaxExp && amax > __builtin_ldexpf(kE4M3Max, e)) ++e;
        while (e > -kMaxExp && amax <= __builtin_ldexpf(kE4M3Max, e - 1)) --e;
        e = min(max(e, -kMaxExp), kMaxExp);
    }
    scales[row] = __builtin_ldexpf(1.0f, e);
}

// one thread per 16-byte chunk of the packed codes
__global__ __launch_bounds__(256) void fp8_pack_kernel(const uint16_t* __restrict__ src,
                                                       const float* __restrict__ scales,
                                                       uint8_t* __restrict__ dst, int N, int K,
                                                       int P, long long nchunks) {
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
    u32x4 out = {0u, 0u, 0u, 0u};
    if (row < N) {
        const long long grow = g * N + row;
        const float inv = 1.0f / scales[grow];            // exact: a power of two
        const int col = s * 64 + 32 * c + 8 * (lane >> 5);
        const uint16_t* rp = src + grow * K + col;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 w = *(const u32x4*)(rp + 16 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = e4m3_rne(__uint_as_float(w[i] << 16) * inv);
                const uint32_t hi = e4m3_rne(__uint_as_float(w[i] & 0xffff0000u) * inv);
                const uint32_t pair = lo | (hi << 8);
                const int byte = 8 * h + 2 * i;           // element 2i, 2i+1 of half h
                out[byte >> 2] |= pair << (8 * (byte & 3));
            }
        }
    }
    *(u32x4*)(dst + f * 16) = out;
}

}  // namespace

size_t packed_fp8_weight_bytes(int G, int N, int K, int P) {
    return (size_t)G * (size_t)((N + P - 1) / P) * P * (size_t)K;
}

hipError_t launch_pack_weights_fp8(const uint16_t* src, uint8_t* dst, float* scales, int G, int N,
                                   int K, int P, hipStream_t stream) {
    const long long rows = (long long)G * N;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(fp8_row_scale_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                       src, rows, K, scales);
    const long long nchunks = (long long)packed_fp8_weight_bytes(G, N, K, P) / 16;
    hipLaunchKernelGGL(fp8_pack_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0,
                       stream, src, scales, dst, N, K, P, nchunks);
    return hipGetLastError();
}

}  // namespace moe
