// Token dispatch as a stable counting sort on the device (no host sync).
//
// The expert-parallel all-to-all ("Twinkle x Ascend ...", section "FSDP2-4D
// parallel engine adaptation": route tokens to the owner of each selected
// expert through one dispatch flow) becomes, on one device, a permutation
// that groups token copies by expert, tokens ascending inside each expert.
//
// The N = T k flattened (t, j) entries are cut into chunks of 1024 S
// entries (S 64-entry steps per wave, S <= 16 chosen so that there are at
// most 64 chunks where possible), one workgroup of 16 waves per chunk in both
// kernels:
//   K1 rank:    each wave walks its 64 S entries 64 at a time; lanes holding
//               the same expert find each other with bit-sliced ballots (one
//               ballot per id bit), so an entry's rank inside its wave is the
//               wave's running LDS count of its expert plus the number of
//               lower lanes with the same id.  After a barrier one thread per
//               expert scans that expert's 16 wave counts (the chunk's
//               histogram entry is their sum), and each entry adds the counts
//               of the lower waves: its rank inside the chunk.
//   K2 scatter: every workgroup sums the histogram's columns over all chunks
//               (expert counts) and over the chunks before its own (its
//               chunk's base per expert), scans the counts into the expert
//               offsets in LDS, and writes dest and src for its entries:
//               row = offset[e] + base[e] + rank.  Workgroup 0 also writes
//               counts, offsets[E+1] and marks the unused tail of src.  The
//               entry loads and all histogram loads of a thread are issued
//               together, so each kernel waits for memory about once.
//   K3 gather (only when x_perm is wanted): one wave per token copies its row
//               of x to its k rows of x_perm (16-byte loads and stores, the
//               row read once).  moe_forward gathers the rows inside the
//               expert GEMM through src instead.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxChunks = 64;
constexpr int kWaves = 16;                 // waves per workgroup (both kernels)
constexpr int kThreads = 64 * kWaves;
constexpr int kHistRows = kMaxChunks / 4;  // histogram rows per thread (E <= 1024)
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 64-entry steps per wave: the smallest power of two up to 16 that cuts the
// N entries into at most kMaxChunks chunks of 1024 S (beyond 2^20 entries
// there are more chunks, and the scatter reads the histogram in passes)
int perm_steps(long long N) {
    int S = 1;
    while (S < 16 && (N + (long long)kThreads * S - 1) / ((long long)kThreads * S) > kMaxChunks)
        S *= 2;
    return S;
}

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
__host__ __device__ inline int round4(int e) { return (e + 3) & ~3; }

struct PermWs {
    int32_t* rank;   // [N]
    int32_t* hist;   // [nchunks, E4]
};

inline PermWs carve(void* ws, int N) {
    char* p = (char*)ws;
    PermWs w;
    w.rank = (int32_t*)p;
    p += align256((size_t)N * 4);
    w.hist = (int32_t*)p;
    return w;
}

template <int S>
__global__ __launch_bounds__(kThreads) void perm_rank_kernel(
    const int32_t* __restrict__ ids, int N, int E, int E4, int nchunks, int id_bits,
    int32_t* __restrict__ rank, int32_t* __restrict__ hist, uint32_t* __restrict__ flags,
    uint32_t* __restrict__ zero, int nzero) {
    extern __shared__ int cnt_all[];  // [kWaves][E4]: each wave's counts
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = blockIdx.x;
    int* cnt = cnt_all + wave * E4;
    if (c == 0)
        for (int i = threadIdx.x; i < nzero; i += kThreads) zero[i] = 0u;
    const long long i0 = (long long)c * (kThreads * S) + wave * (64 * S) + lane;
    int id[S];
#pragma unroll
    for (int s = 0; s < S; ++s) id[s] = i0 + 64 * s < N ? ids[i0 + 64 * s] : -1;
    for (int e = lane; e < E4; e += 64) cnt[e] = 0;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    bool bad = false;
    int r[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bool in = i0 + 64 * s < N;
        const bool valid = (unsigned)id[s] < (unsigned)E;
        if (in && !valid) bad = true;
        uint64_t m = __ballot(valid);
        for (int b = 0; b < id_bits; ++b) {
            const bool bit = (id[s] >> b) & 1;
            const uint64_t bb = __ballot(valid && bit);
            m &= bit ? bb : ~bb;
        }
        const int below = __popcll(m & lt_mask);
        // cnt is this wave's own: its LDS reads and writes execute in program
        // order, so no barrier is needed between the steps
        const int base = valid ? cnt[id[s]] : 0;
        r[s] = base + below;
        if (valid && below == 0) cnt[id[s]] = base + __popcll(m);
    }
    __syncthreads();
    // per expert: exclusive prefix of the wave counts (in place), total ->
    // the chunk histogram
    if ((int)threadIdx.x < E4) {
        const int e = threadIdx.x;
        int v[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v[w] = cnt_all[w * E4 + e];
        int run = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            cnt_all[w * E4 + e] = run;
            run += v[w];
        }
        if (c < nchunks) hist[(size_t)c * E4 + e] = run;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < S; ++s)
        if ((unsigned)id[s] < (unsigned)E) rank[i0 + 64 * s] = r[s] + cnt[id[s]];
    if (__any(bad) && lane == 0 && flags) atomicOr(flags, MOE_FLAG_BAD_EXPERT_ID);
}

// Exclusive scan of v over the kThreads threads of a block; returns the
// prefix, *total gets the block sum.
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
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int t = sh[w];
        if (w < wave) wbase += t;
        sum += t;
    }
    __syncthreads();
    *total = sum;
    return wbase + x - v;
}

template <int S>
__global__ __launch_bounds__(kThreads) void perm_scatter_kernel(
    const int32_t* __restrict__ ids, int N, int k, int E, int E4, int nchunks,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ dest,
    int32_t* __restrict__ src) {
    __shared__ __align__(16) int pre_sh[4 * MOE_MAX_E];  // [G][E4] partial sums
    __shared__ __align__(16) int tot_sh[4 * MOE_MAX_E];
    __shared__ int base_sh[MOE_MAX_E], off_sh[MOE_MAX_E];
    __shared__ int sh[kWaves];
    const int tid = threadIdx.x;
    const int c = blockIdx.x;
    // this chunk's entries (with up to 4 per thread loaded before the
    // histogram, in flight together with it; more would not fit the
    // registers beside the histogram rows)
    constexpr int SP = S <= 4 ? S : 1;
    const long long i0 = (long long)c * (kThreads * S) + tid;
    int id[SP], rk[SP];
    if (S <= 4) {
#pragma unroll
        for (int s = 0; s < SP; ++s) {
            const long long i = i0 + kThreads * s;
            id[s] = i < N ? ids[i] : -1;
            rk[s] = i < N ? rank[i] : 0;
        }
    }
    // histogram columns: thread (g, q) sums expert quad q over the chunks
    // g, g + G, ... (at most kHistRows of them, all loads in flight at once):
    // all chunks (counts) and those before c (chunk base)
    const int quads = E4 / 4;
    const int G = kThreads / quads;
    const int g = tid / quads, q = tid - g * quads;
    if (g < G) {
        i32x4 pre = {0, 0, 0, 0}, tot = {0, 0, 0, 0};
        // (one pass while nchunks <= kHistRows G, i.e. up to 64 chunks)
        for (int c0 = 0; c0 < nchunks; c0 += kHistRows * G) {
            i32x4 hv[kHistRows];
#pragma unroll
            for (int b = 0; b < kHistRows; ++b) {
                const int cc = c0 + g + b * G;
                hv[b] = cc < nchunks ? *(const i32x4*)(hist + (size_t)cc * E4 + 4 * q)
                                     : i32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int b = 0; b < kHistRows; ++b) {
                tot += hv[b];
                if (c0 + g + b * G < c) pre += hv[b];
            }
        }
        *(i32x4*)(pre_sh + g * E4 + 4 * q) = pre;
        *(i32x4*)(tot_sh + g * E4 + 4 * q) = tot;
    }
    __syncthreads();
    // thread e < E4: base and count of expert e, then the exclusive scan of
    // the counts into the offsets
    int n = 0, b = 0;
    if (tid < E4)
        for (int gg = 0; gg < G; ++gg) {
            b += pre_sh[gg * E4 + tid];
            n += tot_sh[gg * E4 + tid];
        }
    int total;
    const int ex = block_exclusive_scan(n, sh, &total);
    if (tid < E4) {
        base_sh[tid] = b;
        off_sh[tid] = ex;
        if (c == 0 && tid < E) {
            offsets[tid] = ex;
            counts[tid] = n;
        }
    }
    if (c == 0) {
        if (tid == 0) offsets[E] = total;
        for (long long r = total + tid; r < N; r += kThreads) src[r] = -1;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const long long i = i0 + kThreads * s;
        if (i >= N) continue;
        const int e = S <= 4 ? id[s % SP] : ids[i];
        int row = -1;
        if ((unsigned)e < (unsigned)E) {
            row = off_sh[e] + base_sh[e] + (S <= 4 ? rk[s % SP] : rank[i]);
            src[row] = (int)(i / k);
        }
        dest[i] = row;
    }
}

// one wave per token: its row of x to each of its k rows of x_perm,
// 8 x 16 B per lane per 8 KB segment
__global__ __launch_bounds__(256) void perm_gather_kernel(const uint16_t* __restrict__ x, int T,
                                                          int d, int k,
                                                          const int32_t* __restrict__ dest,
                                                          uint16_t* __restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int rows[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) rows[j] = j < k ? dest[(size_t)t * k + j] : -1;
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
            if (rows[j] < 0) continue;
            u32x4* xd = (u32x4*)(x_perm + (size_t)rows[j] * d);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int v = v0 + u * 64 + lane;
                if (v < nvec) xd[v] = buf[u];
            }
        }
    }
}

template <int S>
void launch_rank_scatter(const int32_t* ids, int N, int k, int E, int E4, int nchunks,
                         int id_bits, const PermWs& w, int32_t* counts, int32_t* offsets,
                         int32_t* dest, int32_t* src, uint32_t* flags, uint32_t* zero, int nzero,
                         hipStream_t stream) {
    // (with N = 0 one block of each still runs: the first clears the
    // counters, the second writes the all-zero counts and offsets)
    const int blocks = nchunks > 0 ? nchunks : 1;
    hipLaunchKernelGGL(perm_rank_kernel<S>, dim3(blocks), dim3(kThreads),
                       kWaves * E4 * sizeof(int), stream, ids, N, E, E4, nchunks, id_bits, w.rank,
                       w.hist, flags, zero, nzero);
    hipLaunchKernelGGL(perm_scatter_kernel<S>, dim3(blocks), dim3(kThreads), 0, stream, ids, N, k,
                       E, E4, nchunks, w.rank, w.hist, counts, offsets, dest, src);
}

}  // namespace

size_t permute_workspace_bytes(int T, int k, int E) {
    const long long N = (long long)T * k;
    const int S = perm_steps(N);
    const long long nchunks = (N + (long long)kThreads * S - 1) / ((long long)kThreads * S);
    return align256((size_t)N * 4) + align256((size_t)nchunks * round4(E) * 4);
}

hipError_t launch_permute(const int32_t* ids, const uint16_t* x, int T, int d, int E, int k,
                          int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                          uint16_t* x_perm, uint32_t* flags, void* ws, hipStream_t stream,
                          uint32_t* zero, int nzero) {
    const int N = T * k;
    const PermWs w = carve(ws, N);
    const int S = perm_steps(N);
    const int nchunks = (int)(((long long)N + (long long)kThreads * S - 1) / ((long long)kThreads * S));
    const int E4 = round4(E);
    int id_bits = 0;
    while ((1 << id_bits) < E) ++id_bits;
#define MOE_PERM_CASE(SV)                                                                   \
    case SV:                                                                                \
        launch_rank_scatter<SV>(ids, N, k, E, E4, nchunks, id_bits, w, counts, offsets, dest, \
                                src, flags, zero, nzero, stream);                           \
        break;
    switch (S) {
        MOE_PERM_CASE(1)
        MOE_PERM_CASE(2)
        MOE_PERM_CASE(4)
        MOE_PERM_CASE(8)
        MOE_PERM_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef MOE_PERM_CASE
    if (x_perm != nullptr && T > 0)
        hipLaunchKernelGGL(perm_gather_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, x, T, d, k,
                           dest, x_perm);
    return hipGetLastError();
}

}  // namespace moe
