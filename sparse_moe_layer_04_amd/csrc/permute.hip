// Token dispatch as a stable counting sort on the device (no host sync).
//
// The expert-parallel all-to-all ("Twinkle x Ascend ...", section "FSDP2-4D
// parallel engine adaptation": route tokens to the owner of each selected
// expert through one dispatch flow) becomes, on one device, a permutation
// that groups token copies by expert, tokens ascending inside each expert.
//
//   K1 rank:    each wave owns a chunk of kChunk flattened (t, j) entries and
//               walks it 64 at a time; lanes holding the same expert find
//               each other with bit-sliced ballots (one ballot per id bit),
//               so a lane's rank inside its chunk is the running LDS count
//               of its expert plus the number of lower lanes with the same
//               id.  Writes rank[i] and the chunk histogram hist[c][e].
//   K2 scan:    one workgroup per expert scans its column of hist over
//               chunks (chunk bases) and writes counts[e].
//   K3 scatter: every workgroup first scans counts into the expert offsets
//               in LDS (E <= 1024 values: cheaper than a grid-wide ticket
//               for a last-block scan, whose single contended atomic took
//               most of K2's time); workgroup 0 also writes offsets[E+1]
//               and marks the unused tail of src.  Then one wave per token:
//               dest/src for its k pairs and k copies of its row of x into
//               x_perm (16-byte vector loads and stores; the row is read
//               once).  Without x_perm (moe_forward with packed weights: the
//               expert GEMM gathers rows through src) only dest and src are
//               written.
#include "moe_internal.h"

namespace moe {
namespace {

// short chunks: the rank kernel is a serial ballot chain per wave, so it
// needs many waves (49,152 entries: 384 chunks) more than long walks
constexpr int kChunkSteps = 2;               // 64-entry steps per chunk
constexpr int kChunk = 64 * kChunkSteps;     // entries per chunk (one wave)

struct PermWs {
    int32_t* rank;   // [N]
    int32_t* hist;   // [nchunks, E]
    int32_t* base;   // [nchunks, E]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline PermWs carve(void* ws, int N, int E) {
    int nchunks = (N + kChunk - 1) / kChunk;
    char* p = (char*)ws;
    PermWs w;
    w.rank = (int32_t*)p;
    p += align256((size_t)N * 4);
    w.hist = (int32_t*)p;
    p += align256((size_t)nchunks * E * 4);
    w.base = (int32_t*)p;
    return w;
}

__global__ __launch_bounds__(256) void perm_rank_kernel(const int32_t* __restrict__ ids, int N,
                                                        int E, int nchunks, int id_bits,
                                                        int32_t* __restrict__ rank,
                                                        int32_t* __restrict__ hist,
                                                        uint32_t* __restrict__ flags,
                                                        uint32_t* __restrict__ zero, int nzero) {
    extern __shared__ int cnt_all[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = blockIdx.x * 4 + wave;
    int* cnt = cnt_all + wave * E;
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0u;
    for (int e = lane; e < E; e += 64) cnt[e] = 0;
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    bool bad = false;
    for (int s = 0; s < kChunkSteps; ++s) {
        const long long i = (long long)c * kChunk + s * 64 + lane;
        int id = -1;
        if (c < nchunks && i < N) id = ids[i];
        const bool valid = (unsigned)id < (unsigned)E;
        if (c < nchunks && i < N && !valid) bad = true;
        uint64_t m = __ballot(valid);
        for (int b = 0; b < id_bits; ++b) {
            const bool bit = (id >> b) & 1;
            const uint64_t bb = __ballot(valid && bit);
            m &= bit ? bb : ~bb;
        }
        const int r = __popcll(m & lt_mask);
        const int tot = __popcll(m);
        // cnt is this wave's own: its LDS reads and writes execute in program
        // order, so no barrier is needed between the steps
        int base = 0;
        if (valid) base = cnt[id];
        if (valid) {
            rank[i] = base + r;
            if (r == 0) cnt[id] = base + tot;
        }
    }
    if (__any(bad) && lane == 0 && flags) atomicOr(flags, MOE_FLAG_BAD_EXPERT_ID);
    if (c < nchunks)
        for (int e = lane; e < E; e += 64) hist[(size_t)c * E + e] = cnt[e];
}

// Exclusive scan of v over the 256 threads of a block; returns the prefix,
// *total gets the block sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int wbase = 0, sum = 0;
    for (int w = 0; w < 4; ++w) {
        int t = sh[w];
        if (w < wave) wbase += t;
        sum += t;
    }
    __syncthreads();
    *total = sum;
    return wbase + x - v;
}

__global__ __launch_bounds__(256) void perm_scan_kernel(const int32_t* __restrict__ hist,
                                                        int nchunks, int E,
                                                        int32_t* __restrict__ base,
                                                        int32_t* __restrict__ counts) {
    __shared__ int sh[4];
    const int e = blockIdx.x;
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 256) {
        const int c = c0 + threadIdx.x;
        const int v = c < nchunks ? hist[(size_t)c * E + e] : 0;
        int tot;
        const int ex = block_exclusive_scan(v, sh, &tot);
        if (c < nchunks) base[(size_t)c * E + e] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) counts[e] = carry;
}

// tokens per scatter workgroup (4 waves x kTokPerWave)
constexpr int kTokPerWave = 4;
constexpr int kTokPerBlock = 4 * kTokPerWave;

__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t* __restrict__ ids, const uint16_t* __restrict__ x, int T, int d, int E, int k,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ dest, int32_t* __restrict__ src, uint16_t* __restrict__ x_perm) {
    __shared__ int off_sh[MOE_MAX_E + 1];
    __shared__ int sh[4];
    const int lane = threadIdx.x & 63;
    // expert offsets = exclusive scan of counts (every workgroup)
    int run = 0;
    for (int e0 = 0; e0 < E; e0 += 256) {
        const int ee = e0 + threadIdx.x;
        const int v = ee < E ? counts[ee] : 0;
        int tot;
        const int ex = block_exclusive_scan(v, sh, &tot);
        if (ee < E) off_sh[ee] = run + ex;
        run += tot;
    }
    if (threadIdx.x == 0) off_sh[E] = run;
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int e = threadIdx.x; e <= E; e += 256) offsets[e] = off_sh[e];
        for (int r = run + threadIdx.x; r < T * k; r += 256) src[r] = -1;
    }
    for (int tt = 0; tt < kTokPerWave; ++tt) {
        const int t = blockIdx.x * kTokPerBlock + tt * 4 + (threadIdx.x >> 6);
        if (t >= T) return;
        int row = -1;
        if (lane < k) {
            const long long i = (long long)t * k + lane;
            const int e = ids[i];
            if ((unsigned)e < (unsigned)E) {
                const int c = (int)(i / kChunk);
                row = off_sh[e] + base[(size_t)c * E + e] + rank[i];
                src[row] = t;
            }
            dest[i] = row;
        }
        if (x_perm == nullptr) continue;
        int rows[MOE_MAX_K];
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j) rows[j] = __shfl(row, j, 64);
        // copy the row of x to each slot, 8 x 16 B per lane per segment
        const int nvec = d >> 3;  // 16-byte vectors per row
        const u32x4* xs = (const u32x4*)(x + (size_t)t * d);
        for (int v0 = 0; v0 < nvec; v0 += 512) {
            u32x4 buf[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int v = v0 + u * 64 + lane;
                if (v < nvec) buf[u] = xs[v];
            }
#pragma unroll
            for (int j = 0; j < MOE_MAX_K; ++j) {
                if (j >= k || rows[j] < 0) continue;
                u32x4* xd = (u32x4*)(x_perm + (size_t)rows[j] * d);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int v = v0 + u * 64 + lane;
                    if (v < nvec) xd[v] = buf[u];
                }
            }
        }
    }
}

}  // namespace

size_t permute_workspace_bytes(int T, int k, int E) {
    const long long N = (long long)T * k;
    const long long nchunks = (N + kChunk - 1) / kChunk;
    return align256((size_t)N * 4) + 2 * align256((size_t)nchunks * E * 4);
}

hipError_t launch_permute(const int32_t* ids, const uint16_t* x, int T, int d, int E, int k,
                          int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                          uint16_t* x_perm, uint32_t* flags, void* ws, hipStream_t stream,
                          uint32_t* zero, int nzero) {
    const int N = T * k;
    PermWs w = carve(ws, N, E);
    const int nchunks = (N + kChunk - 1) / kChunk;
    int id_bits = 0;
    while ((1 << id_bits) < E) ++id_bits;
    {
        // (with N = 0 one block still runs: it only clears the counters)
        const int blocks = N > 0 ? (nchunks + 3) / 4 : 1;
        hipLaunchKernelGGL(perm_rank_kernel, dim3(blocks), dim3(256), 4 * E * sizeof(int),
                           stream, ids, N, E, nchunks, id_bits, w.rank, w.hist, flags, zero,
                           nzero);
    }
    hipLaunchKernelGGL(perm_scan_kernel, dim3(E), dim3(256), 0, stream, w.hist, nchunks, E,
                       w.base, counts);
    // (with T = 0 one block still runs: it writes the all-zero offsets)
    const int sblocks = T > 0 ? (T + kTokPerBlock - 1) / kTokPerBlock : 1;
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(sblocks), dim3(256), 0, stream, ids, x, T, d, E,
                       k, w.rank, w.base, counts, offsets, dest, src, x_perm);
    return hipGetLastError();
}

}  // namespace moe
