// C ABI of the MoE layer library: argument validation (complete before any
// launch), workspace layout and the launch sequence of the forward pass.
#include <math.h>
#include <string.h>

#include "moe_internal.h"

namespace moe {

int device_cu_count() {
    // (256, the MI355X count, if the query fails)
    static DeviceSetup setup;
    long long cus = 0, unused = 0;
    const hipError_t err = device_setup(setup, cus, unused, [](int dev, long long& v, long long&) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 0;
        v = n > 0 ? n : 256;
        return hipSuccess;
    });
    return err == hipSuccess ? (int)cus : 256;
}

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }

int route_checks(const float* logits, const float* bias, const int32_t* input_ids,
                 const int32_t* tid2eid, int T, int E, int k, int n_bias, int V, int mode,
                 float scale, const int32_t* ids, const float* w) {
    if (T < 0 || E < 1 || k < 1) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_E || k > MOE_MAX_K || k > E) return MOE_ERR_UNSUPPORTED;
    if (mode != MOE_MODE_TOPK && mode != MOE_MODE_HASH) return MOE_ERR_UNSUPPORTED;
    if (!(scale == scale)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!logits || !ids || !w) return MOE_ERR_NULL;
    if (mode == MOE_MODE_TOPK) {
        if (n_bias < 0 || n_bias > 2) return MOE_ERR_SHAPE;
        if (n_bias > 0 && !bias) return MOE_ERR_NULL;
    } else {
        if (!input_ids || !tid2eid) return MOE_ERR_NULL;
        if (V < 1) return MOE_ERR_SHAPE;
    }
    return MOE_OK;
}

int ffn_checks(int rows, int d, int F, float clamp_limit, int clamp_mode) {
    if (rows < 0 || d < 64 || F < 64) return MOE_ERR_SHAPE;
    if (d % 64 || F % 64) return MOE_ERR_UNSUPPORTED;
    if (d > kFlatMaxK || F > kFlatMaxK) return MOE_ERR_UNSUPPORTED;
    if (!(clamp_limit > 0.0f)) return MOE_ERR_SHAPE;  // also rejects NaN
    if (clamp_mode != MOE_CLAMP_SYMMETRIC && clamp_mode != MOE_CLAMP_GATE_UPPER)
        return MOE_ERR_UNSUPPORTED;
    if ((long long)rows * d >= (1ll << 40) || (long long)rows * F >= (1ll << 40))
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// expert GEMMs: packed weights take the LDS-staged kernel when its LDS holds
// the group table, else (and for plain weights) the register-direct kernel
inline bool lds_gemm_ok(int packed, int G) {
    return packed && G <= grouped_gemm_lds_max_groups();
}
#ifndef MOE_EXPERT_GEMM_FLAT
#define MOE_EXPERT_GEMM_FLAT 1
#endif
// packed bf16 weights without a workspace (static schedule): the flat kernel
// when its LDS holds the group table, else the LDS-staged one
inline hipError_t packed_gemm(int epi, const GemmArgs& g, hipStream_t s) {
    if (MOE_EXPERT_GEMM_FLAT && g.G <= grouped_gemm_flat_max_groups())
        return launch_grouped_gemm_flat(epi, g, s);
    return launch_grouped_gemm_lds(epi, g, s);
}
#ifndef MOE_EXPERT_GEMM_FLAT_MX
#define MOE_EXPERT_GEMM_FLAT_MX 1
#endif
// the flat kernel takes MX weights in the two routed GEMMs of the forward:
// gate/up on gathered token rows into blocked h, down on blocked h
inline bool flat_mx_ok(int epi, const GemmArgs& g) {
    return MOE_EXPERT_GEMM_FLAT_MX && !g.out_g &&
           ((epi == EPI_SWIGLU_BF16 && g.gather && g.out_blocked && !g.a_blocked) ||
            (epi == EPI_F32 && !g.gather && g.a_blocked));
}
inline hipError_t expert_gemm(int epi, const GemmArgs& g, hipStream_t s) {
    if (g.wfp8 == 3) return launch_grouped_gemm_flat(epi, g, s);   // A8W4: flat kernel only
    if (MOE_EXPERT_GEMM_FLAT && g.packed && g.G <= grouped_gemm_flat_max_groups() &&
        (!g.wfp8 || flat_mx_ok(epi, g)))
        return launch_grouped_gemm_flat(epi, g, s);
    return lds_gemm_ok(g.packed, g.G) ? launch_grouped_gemm_lds(epi, g, s)
                                      : launch_grouped_gemm(epi, g, s);
}

// moe_forward workspace layout
struct FwdWs {
    float* logits;
    int32_t* ids;
    float* w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* dest;
    int32_t* src;
    uint16_t* x_perm;
    uint16_t* h;
    float* y_perm;
    uint16_t* hs;
    float* ys;
    void* perm;
    uint32_t* sched;  // 4 x kSchedWords expert GEMM counters
    uint8_t* x8;      // A8W4: [T, d] MXFP8 codes of x
    uint8_t* x8s;     // [T, d / 32] their scale bytes
    uint8_t* h8s;     // [T k, F / 32] scale bytes of the MXFP8 h (codes in h)
    size_t total;
};

FwdWs forward_layout(const moe_cfg* c, char* base) {
    const size_t T = (size_t)c->T, N = (size_t)c->T * c->k;
    size_t off = 0;
    FwdWs w;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += align256(bytes);
        return (void*)p;
    };
    w.logits = (float*)take(T * c->E * 4);
    w.ids = (int32_t*)take(N * 4);
    w.w = (float*)take(N * 4);
    w.counts = (int32_t*)take((size_t)c->E * 4);
    w.offsets = (int32_t*)take((size_t)(c->E + 1) * 4);
    w.dest = (int32_t*)take(N * 4);
    w.src = (int32_t*)take(N * 4);
    w.x_perm = (uint16_t*)take(N * c->d * 2);  // plain-weight path only
    w.h = (uint16_t*)take(blocked_rows(N) * c->F * 2);
    w.y_perm = (float*)take(N * c->d * 4);
    w.hs = (uint16_t*)take(T * (size_t)(c->F_shared > 0 ? c->F_shared : 0) * 2);
    w.ys = (float*)take(c->F_shared > 0 ? T * c->d * 4 : 0);
    w.perm = take(permute_workspace_bytes(c->T, c->k, c->E));
    w.sched = (uint32_t*)take(4 * kSchedWords * sizeof(uint32_t));
    w.x8 = (uint8_t*)take(T * c->d);
    w.x8s = (uint8_t*)take(T * (c->d / 32));
    w.h8s = (uint8_t*)take(N * (c->F / 32));
    w.total = off;
    return w;
}

// moe_backward workspace layout (N = T k routed rows)
struct BwdWs {
    float* logits;      // [T, E]
    int32_t* ids;       // [T, k]
    float* w;           // [T, k]
    float* dtw;         // [T, k] routing-weight gradient
    float* dl;          // [T, E] logit gradient
    int32_t* counts;    // [E]
    int32_t* offsets;   // [E + 1]
    int32_t* dest;      // [N]
    int32_t* src;       // [N]
    uint16_t* x_perm;   // [N, d] bf16
    float* g;           // [N, F] gate pre-activations
    float* u;           // [N, F] up pre-activations
    uint16_t* h;        // [N, F] bf16
    float* y_perm;      // [N, d]
    float* dyp;         // [N, d] fp32 dx_perm (the gate/up input gradient rows)
    uint16_t* dyp16;    // [N, d] bf16
    float* dh;          // [N, F]
    uint16_t* dgu;      // [N, 2F] bf16
    float* gs;          // [T, Fs]
    float* us;          // [T, Fs]
    uint16_t* hs;       // [T, Fs] bf16
    uint16_t* dy16;     // [T, d] bf16
    float* dhs;         // [T, Fs]
    uint16_t* dgus;     // [T, 2Fs] bf16
    float* dxs;         // [T, d] shared expert's input gradient
    void* perm;
    uint32_t* sched;    // 8 x kSchedWords expert GEMM counters
    size_t total;
};

BwdWs backward_layout(const moe_cfg* c, char* base) {
    const size_t T = (size_t)c->T, N = (size_t)c->T * c->k, d = c->d, F = c->F;
    const size_t Fs = c->F_shared > 0 ? c->F_shared : 0;
    size_t off = 0;
    BwdWs w;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += align256(bytes);
        return (void*)p;
    };
    w.logits = (float*)take(T * c->E * 4);
    w.ids = (int32_t*)take(N * 4);
    w.w = (float*)take(N * 4);
    w.dtw = (float*)take(N * 4);
    w.dl = (float*)take(T * c->E * 4);
    w.counts = (int32_t*)take((size_t)c->E * 4);
    w.offsets = (int32_t*)take((size_t)(c->E + 1) * 4);
    w.dest = (int32_t*)take(N * 4);
    w.src = (int32_t*)take(N * 4);
    w.x_perm = (uint16_t*)take(N * d * 2);
    w.g = (float*)take(N * F * 4);
    w.u = (float*)take(N * F * 4);
    w.h = (uint16_t*)take(N * F * 2);
    w.y_perm = (float*)take(N * d * 4);
    w.dyp = (float*)take(N * d * 4);
    w.dyp16 = (uint16_t*)take(N * d * 2);
    w.dh = (float*)take(N * F * 4);
    w.dgu = (uint16_t*)take(N * 2 * F * 2);
    w.gs = (float*)take(T * Fs * 4);
    w.us = (float*)take(T * Fs * 4);
    w.hs = (uint16_t*)take(T * Fs * 2);
    w.dy16 = (uint16_t*)take(T * d * 2);
    w.dhs = (float*)take(T * Fs * 4);
    w.dgus = (uint16_t*)take(T * 2 * Fs * 2);
    w.dxs = (float*)take(Fs ? T * d * 4 : 0);
    w.perm = take(permute_workspace_bytes(c->T, c->k, c->E));
    w.sched = (uint32_t*)take(8 * kSchedWords * sizeof(uint32_t));
    w.total = off;
    return w;
}

// one expert GEMM on the flat kernel with row-major activations
hipError_t flat_gemm(int epi, const uint16_t* a, const int32_t* offsets, int G, int rows, int K,
                     int N, const uint16_t* w1, const uint16_t* w2, float L, int cmode, void* out,
                     float* out_g, float* out_u, uint32_t* sched, hipStream_t s) {
    GemmArgs g{};
    g.a = a;
    g.offsets = offsets;
    g.G = G;
    g.rows = rows;
    g.K = K;
    g.N = N;
    g.w1 = w1;
    g.w2 = w2;
    g.packed = 1;
    g.clamp_limit = L;
    g.clamp_mode = cmode;
    g.out = out;
    g.out_g = out_g;
    g.out_u = out_u;
    g.sched = sched;
    return launch_grouped_gemm_flat(epi, g, s);
}

}  // namespace

int permute_arg_checks(const int32_t* topk_ids, const uint16_t* x, int T, int d, int E, int k,
                       const int32_t* counts, const int32_t* offsets, const int32_t* dest,
                       const int32_t* src, const uint16_t* x_perm) {
    if (T < 0 || d < 8 || E < 1 || k < 1) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_E || k > MOE_MAX_K || d % 8) return MOE_ERR_UNSUPPORTED;
    if ((long long)T * k >= (1ll << 31)) return MOE_ERR_SHAPE;
    if (!counts || !offsets) return MOE_ERR_NULL;
    if (T > 0 && (!topk_ids || !x || !dest || !src || !x_perm)) return MOE_ERR_NULL;
    if (T > 0 && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
        case MOE_ERR_UNSUPPORTED: return "unsupported mode or size";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case MOE_ERR_SCRATCH:
            return "the call needs more scratch than the library's static scratch array holds";
        default: return "unknown status";
    }
}

int moe_gate_logits(const uint16_t* x, const uint16_t* w_g, const float* logit_offset, int T,
                    int d, int E, float* logits, void* stream) {
    if (T < 0 || E < 1 || d < 64) return MOE_ERR_SHAPE;
    if (d % 64) return MOE_ERR_UNSUPPORTED;
    if (E > MOE_MAX_GROUPS) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_g || !logits) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_g)) return MOE_ERR_ALIGN;
    GemmArgs g{};
    g.a = x;
    g.offsets = nullptr;
    g.G = 1;
    g.rows = T;
    g.K = d;
    g.N = E;
    g.w1 = w_g;
    g.w2 = nullptr;
    g.offset = logit_offset;
    g.out = logits;
    return hip_status(launch_grouped_gemm(EPI_F32_OFFSET, g, as_stream(stream)));
}

int moe_route(const float* logits, const float* score_bias, const uint8_t* modality,
              const int32_t* input_ids, const int32_t* tid2eid, int T, int E, int k, int n_bias,
              int V, int mode, float scale, int32_t* topk_ids, float* topk_w, uint32_t* d_flags,
              void* stream) {
    int st = route_checks(logits, score_bias, input_ids, tid2eid, T, E, k, n_bias, V, mode, scale,
                          topk_ids, topk_w);
    if (st != MOE_OK || T == 0) return st;
    return hip_status(launch_route(logits, n_bias > 0 ? score_bias : nullptr, modality, input_ids,
                                   tid2eid, T, E, k, n_bias, V, mode, scale, topk_ids, topk_w,
                                   d_flags, as_stream(stream)));
}

int moe_route_backward(const float* logits, const int32_t* topk_ids, const float* d_topk_w,
                       int T, int E, int k, float scale, float* d_logits, uint32_t* d_flags,
                       void* stream) {
    if (T < 0 || E < 1 || k < 1) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_E || k > MOE_MAX_K || k > E) return MOE_ERR_UNSUPPORTED;
    if (!(scale == scale)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !d_topk_w || !d_logits) return MOE_ERR_NULL;
    return hip_status(launch_route_backward(logits, topk_ids, d_topk_w, T, E, k, scale, d_logits,
                                            d_flags, as_stream(stream)));
}

size_t moe_permute_workspace_size(int T, int k, int E) {
    if (T < 0 || k < 1 || E < 1) return 0;
    return permute_workspace_bytes(T, k, E);
}

int moe_permute(const int32_t* topk_ids, const uint16_t* x, int T, int d, int E, int k,
                int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src, uint16_t* x_perm,
                uint32_t* d_flags, void* ws, size_t ws_bytes, void* stream) {
    int st = permute_arg_checks(topk_ids, x, T, d, E, k, counts, offsets, dest, src, x_perm);
    if (st != MOE_OK) return st;
    if (!ws && permute_workspace_bytes(T, k, E) > 0) return MOE_ERR_NULL;
    if (((uintptr_t)ws & 255u) || ws_bytes < permute_workspace_bytes(T, k, E))
        return MOE_ERR_WORKSPACE;
    return hip_status(launch_permute(topk_ids, x, T, d, E, k, counts, offsets, dest, src, x_perm,
                                     d_flags, ws, as_stream(stream)));
}

int moe_expert_ffn(const uint16_t* a, const int32_t* offsets, int G, int rows, int d, int F,
                   const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                   float clamp_limit, int clamp_mode, uint16_t* h, float* y, void* stream) {
    if (G < 1) return MOE_ERR_SHAPE;
    if (G > MOE_MAX_GROUPS) return MOE_ERR_UNSUPPORTED;
    int st = ffn_checks(rows, d, F, clamp_limit, clamp_mode);
    if (st != MOE_OK) return st;
    if (rows == 0) return MOE_OK;
    if (!a || !offsets || !w_gate || !w_up || !w_down || !h || !y) return MOE_ERR_NULL;
    if (!aligned16(a) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
        !aligned16(h) || !aligned16(y))
        return MOE_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    GemmArgs g1{};
    g1.a = a;
    g1.offsets = offsets;
    g1.G = G;
    g1.rows = rows;
    g1.K = d;
    g1.N = F;
    g1.w1 = w_gate;
    g1.w2 = w_up;
    g1.clamp_limit = clamp_limit;
    g1.clamp_mode = clamp_mode;
    g1.out = h;
    hipError_t e = launch_grouped_gemm(EPI_SWIGLU_BF16, g1, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    GemmArgs g2{};
    g2.a = h;
    g2.offsets = offsets;
    g2.G = G;
    g2.rows = rows;
    g2.K = F;
    g2.N = d;
    g2.w1 = w_down;
    g2.out = y;
    return hip_status(launch_grouped_gemm(EPI_F32, g2, s));
}

int moe_expert_ffn_packed(const uint16_t* a, const int32_t* offsets, int G, int rows, int d,
                          int F, const uint16_t* w_gate, const uint16_t* w_up,
                          const uint16_t* w_down, float clamp_limit, int clamp_mode, uint16_t* h,
                          float* y, void* stream) {
    if (G < 1) return MOE_ERR_SHAPE;
    if (G > MOE_MAX_GROUPS || G > grouped_gemm_lds_max_groups()) return MOE_ERR_UNSUPPORTED;
    int st = ffn_checks(rows, d, F, clamp_limit, clamp_mode);
    if (st != MOE_OK) return st;
    if (rows == 0) return MOE_OK;
    if (!a || !offsets || !w_gate || !w_up || !w_down || !h || !y) return MOE_ERR_NULL;
    if (!aligned16(a) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
        !aligned16(h) || !aligned16(y))
        return MOE_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    // no workspace: both GEMMs take the static schedule (sched = NULL)
    GemmArgs g1{};
    g1.a = a;
    g1.offsets = offsets;
    g1.G = G;
    g1.rows = rows;
    g1.K = d;
    g1.N = F;
    g1.w1 = w_gate;
    g1.w2 = w_up;
    g1.packed = 1;
    g1.clamp_limit = clamp_limit;
    g1.clamp_mode = clamp_mode;
    g1.out = h;
    hipError_t e = packed_gemm(EPI_SWIGLU_BF16, g1, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    GemmArgs g2{};
    g2.a = h;
    g2.offsets = offsets;
    g2.G = G;
    g2.rows = rows;
    g2.K = F;
    g2.N = d;
    g2.w1 = w_down;
    g2.packed = 1;
    g2.out = y;
    return hip_status(packed_gemm(EPI_F32, g2, s));
}

size_t moe_packed_weight_bytes(int G, int N, int K, int panel_rows) {
    if (G < 1 || N < 1 || K < 64 || K % 64) return 0;
    if (panel_rows != 128 && panel_rows != 256) return 0;
    return packed_weight_elems(G, N, K, panel_rows) * 2;
}

int moe_pack_weights(const uint16_t* src, int G, int N, int K, int panel_rows, uint16_t* dst,
                     void* stream) {
    if (G < 1 || N < 1 || K < 64) return MOE_ERR_SHAPE;
    if (K % 64 || (panel_rows != 128 && panel_rows != 256)) return MOE_ERR_UNSUPPORTED;
    if (!src || !dst) return MOE_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_ALIGN;
    return hip_status(launch_pack_weights(src, dst, G, N, K, panel_rows, as_stream(stream)));
}

size_t moe_packed_fp8_weight_bytes(int G, int N, int K, int panel_rows) {
    if (G < 1 || N < 1 || K < 64 || K % 64) return 0;
    if (panel_rows != 128 && panel_rows != 256) return 0;
    return packed_fp8_weight_bytes(G, N, K, panel_rows);
}

size_t moe_packed_fp8_scale_bytes(int G, int N, int K, int panel_rows) {
    if (G < 1 || N < 1 || K < 64 || K % 64) return 0;
    if (panel_rows != 128 && panel_rows != 256) return 0;
    return packed_fp8_scale_bytes(G, N, K, panel_rows);
}

int moe_pack_weights_fp8(const uint16_t* src, int G, int N, int K, int panel_rows, uint8_t* dst,
                         uint8_t* scales, void* stream) {
    if (G < 1 || N < 1 || K < 64) return MOE_ERR_SHAPE;
    if (K % 64 || (panel_rows != 128 && panel_rows != 256)) return MOE_ERR_UNSUPPORTED;
    if (!src || !dst || !scales) return MOE_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst) || !aligned16(scales)) return MOE_ERR_ALIGN;
    return hip_status(
        launch_pack_weights_fp8(src, dst, scales, G, N, K, panel_rows, as_stream(stream)));
}

size_t moe_packed_fp4_weight_bytes(int G, int N, int K, int panel_rows) {
    if (G < 1 || N < 1 || K < 64 || K % 64) return 0;
    if (panel_rows != 128 && panel_rows != 256) return 0;
    return packed_fp4_weight_bytes(G, N, K, panel_rows);
}

int moe_pack_weights_fp4(const uint16_t* src, int G, int N, int K, int panel_rows, uint8_t* dst,
                         uint8_t* scales, void* stream) {
    if (G < 1 || N < 1 || K < 64) return MOE_ERR_SHAPE;
    if (K % 64 || (panel_rows != 128 && panel_rows != 256)) return MOE_ERR_UNSUPPORTED;
    if (!src || !dst || !scales) return MOE_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst) || !aligned16(scales)) return MOE_ERR_ALIGN;
    return hip_status(
        launch_pack_weights_fp4(src, dst, scales, G, N, K, panel_rows, as_stream(stream)));
}

int moe_quantize_mxfp8(const uint16_t* a, long long rows, int K, uint8_t* codes, uint8_t* scales,
                       void* stream) {
    if (rows < 0 || K <= 0 || K % 32 || rows * (long long)K >= (1ll << 40)) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!a || !codes || !scales) return MOE_ERR_NULL;
    if (!aligned16(a) || !aligned16(codes)) return MOE_ERR_ALIGN;
    return hip_status(launch_quant_rows_mxfp8(a, rows, K, codes, scales, as_stream(stream)));
}

int moe_combine(const float* y_perm, const int32_t* dest, const float* topk_w,
                const float* y_shared, int T, int d, int k, int rows, int out_dtype, void* y,
                void* stream) {
    if (T < 0 || d < 8 || k < 1 || rows < 0) return MOE_ERR_SHAPE;
    if (k > MOE_MAX_K || d % 8) return MOE_ERR_UNSUPPORTED;
    if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!dest || !topk_w || !y || (rows > 0 && !y_perm)) return MOE_ERR_NULL;
    if ((y_perm && !aligned16(y_perm)) || (y_shared && !aligned16(y_shared)) || !aligned16(y))
        return MOE_ERR_ALIGN;
    return hip_status(launch_combine(y_perm, dest, topk_w, y_shared, T, d, k, rows, out_dtype, y,
                                     as_stream(stream)));
}

int moe_combine_backward(const float* dy, const float* y_perm, const int32_t* dest,
                         const float* topk_w, int T, int d, int k, int rows, float* dy_perm,
                         float* d_topk_w, void* stream) {
    if (T < 0 || d < 8 || k < 1 || rows < 0) return MOE_ERR_SHAPE;
    if (k > MOE_MAX_K || d % 8) return MOE_ERR_UNSUPPORTED;
    if ((long long)rows * d >= (1ll << 40) || (long long)T * d >= (1ll << 40)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!dy || !dest || !topk_w || !d_topk_w || (rows > 0 && (!y_perm || !dy_perm)))
        return MOE_ERR_NULL;
    if (!aligned16(dy) || (y_perm && !aligned16(y_perm)) || (dy_perm && !aligned16(dy_perm)))
        return MOE_ERR_ALIGN;
    return hip_status(launch_combine_backward(dy, y_perm, dest, topk_w, T, d, k, rows, dy_perm,
                                              d_topk_w, as_stream(stream)));
}

int moe_expert_ffn_a8w4(const uint8_t* a8, const uint8_t* a_scale, const int32_t* offsets, int G,
                        int rows, int d, int F, const uint8_t* w_gate, const uint8_t* w_up,
                        const uint8_t* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                        const uint8_t* s_down, float clamp_limit, int clamp_mode, uint8_t* h8,
                        uint8_t* h_scale, float* y, void* stream) {
    if (G < 1) return MOE_ERR_SHAPE;
    if (G > MOE_MAX_GROUPS || G > grouped_gemm_flat_max_groups()) return MOE_ERR_UNSUPPORTED;
    int st = ffn_checks(rows, d, F, clamp_limit, clamp_mode);
    if (st != MOE_OK) return st;
    if (d % 128 || F % 128) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!a8 || !a_scale || !offsets || !w_gate || !w_up || !w_down || !s_gate || !s_up ||
        !s_down || !h8 || !h_scale || !y)
        return MOE_ERR_NULL;
    if (!aligned16(a8) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
        !aligned16(h8) || !aligned16(y) || ((uintptr_t)a_scale & 3u) || ((uintptr_t)h_scale & 3u))
        return MOE_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    // no workspace: static schedule (sched = NULL)
    GemmArgs g1{};
    g1.a8 = a8;
    g1.a_scale = a_scale;
    g1.offsets = offsets;
    g1.G = G;
    g1.rows = rows;
    g1.K = d;
    g1.N = F;
    g1.w1 = (const uint16_t*)w_gate;
    g1.w2 = (const uint16_t*)w_up;
    g1.s1 = s_gate;
    g1.s2 = s_up;
    g1.packed = 1;
    g1.wfp8 = 3;
    g1.clamp_limit = clamp_limit;
    g1.clamp_mode = clamp_mode;
    g1.out = h8;
    g1.out_scale = h_scale;
    hipError_t e = launch_grouped_gemm_flat(EPI_SWIGLU_BF16, g1, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    GemmArgs g2{};
    g2.a8 = h8;
    g2.a_scale = h_scale;
    g2.offsets = offsets;
    g2.G = G;
    g2.rows = rows;
    g2.K = F;
    g2.N = d;
    g2.w1 = (const uint16_t*)w_down;
    g2.s1 = s_down;
    g2.packed = 1;
    g2.wfp8 = 3;
    g2.out = y;
    return hip_status(launch_grouped_gemm_flat(EPI_F32, g2, s));
}

int moe_grouped_gemm_packed(const uint16_t* a, const int32_t* offsets, int G, int rows, int K,
                            int N, const uint16_t* w_packed, float* out, void* stream) {
    if (G < 1 || rows < 0 || K < 64 || N < 64) return MOE_ERR_SHAPE;
    if (K % 64 || N % 64 || K > kFlatMaxK) return MOE_ERR_UNSUPPORTED;
    if (G > MOE_MAX_GROUPS || G > grouped_gemm_lds_max_groups()) return MOE_ERR_UNSUPPORTED;
    if ((long long)rows * K >= (1ll << 40) || (long long)rows * N >= (1ll << 40))
        return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!a || !offsets || !w_packed || !out) return MOE_ERR_NULL;
    if (!aligned16(a) || !aligned16(w_packed) || !aligned16(out)) return MOE_ERR_ALIGN;
    // the LDS-staged expert GEMM, fp32 output, static schedule (no workspace)
    GemmArgs g{};
    g.a = a;
    g.offsets = offsets;
    g.G = G;
    g.rows = rows;
    g.K = K;
    g.N = N;
    g.w1 = w_packed;
    g.packed = 1;
    g.out = out;
    return hip_status(packed_gemm(EPI_F32, g, as_stream(stream)));
}

int moe_grouped_wgrad(const uint16_t* dy, const uint16_t* a, const int32_t* offsets, int G,
                      int rows, int M, int K, float* dw, void* stream) {
    if (G < 1 || rows < 0 || M < 8 || K < 8) return MOE_ERR_SHAPE;
    if (M % 8 || K % 8) return MOE_ERR_UNSUPPORTED;
    if ((long long)rows * M >= (1ll << 40) || (long long)rows * K >= (1ll << 40) ||
        (long long)G * M * K >= (1ll << 40))
        return MOE_ERR_SHAPE;
    if (!dw || (rows > 0 && (!dy || !a))) return MOE_ERR_NULL;
    if (G > 1 && !offsets) return MOE_ERR_NULL;
    if ((dy && !aligned16(dy)) || (a && !aligned16(a)) || !aligned16(dw)) return MOE_ERR_ALIGN;
    return hip_status(launch_grouped_wgrad(dy, a, offsets, G, rows, M, K, dw, as_stream(stream)));
}

int moe_swiglu_backward(const float* gate, const float* up, const float* dh, int64_t n,
                        float clamp_limit, int clamp_mode, float* dgate, float* dup,
                        void* stream) {
    if (n < 0) return MOE_ERR_SHAPE;
    if (n % 4) return MOE_ERR_UNSUPPORTED;
    if (!(clamp_limit > 0.0f)) return MOE_ERR_SHAPE;  // also rejects NaN
    if (clamp_mode != MOE_CLAMP_SYMMETRIC && clamp_mode != MOE_CLAMP_GATE_UPPER)
        return MOE_ERR_UNSUPPORTED;
    if (n == 0) return MOE_OK;
    if (!gate || !up || !dh || !dgate || !dup) return MOE_ERR_NULL;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(dh) || !aligned16(dgate) ||
        !aligned16(dup))
        return MOE_ERR_ALIGN;
    return hip_status(launch_swiglu_backward(gate, up, dh, (long long)n, clamp_limit, clamp_mode,
                                             dgate, dup, as_stream(stream)));
}

static int forward_checks(const moe_cfg* c, const moe_weights* w) {
    if (!c || !w) return MOE_ERR_NULL;
    if (c->T < 0 || c->E < 1 || c->k < 1 || c->F_shared < 0) return MOE_ERR_SHAPE;
    if (c->E > MOE_MAX_E || c->k > MOE_MAX_K || c->k > c->E) return MOE_ERR_UNSUPPORTED;
    // (before T k is formed as an int)
    if ((long long)c->T * c->k >= (1ll << 31)) return MOE_ERR_SHAPE;
    int st = ffn_checks(c->T * c->k, c->d, c->F, c->clamp_limit, c->clamp_mode);
    if (st != MOE_OK) return st;
    if (c->F_shared % 64 || c->F_shared > kFlatMaxK) return MOE_ERR_UNSUPPORTED;
    if (c->mode != MOE_MODE_TOPK && c->mode != MOE_MODE_HASH) return MOE_ERR_UNSUPPORTED;
    if (c->out_dtype != MOE_OUT_BF16 && c->out_dtype != MOE_OUT_F32) return MOE_ERR_UNSUPPORTED;
    if (!(c->scale == c->scale)) return MOE_ERR_SHAPE;
    if (w->packed != 0 && w->packed != 1 && w->packed != MOE_WEIGHTS_FP8 &&
        w->packed != MOE_WEIGHTS_FP4 && w->packed != MOE_WEIGHTS_A8W4)
        return MOE_ERR_UNSUPPORTED;
    if (w->packed == MOE_WEIGHTS_A8W4) {
        // the flat expert GEMM on 128-wide K stages
        if (c->E > grouped_gemm_flat_max_groups() || c->d % 128 || c->F % 128)
            return MOE_ERR_UNSUPPORTED;
        return MOE_OK;
    }
    // 8- and 4-bit routed weights need the group table of the LDS-staged
    // expert GEMM (their fallback)
    if (w->packed >= MOE_WEIGHTS_FP8 && !lds_gemm_ok(1, c->E)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

size_t moe_forward_workspace_size(const moe_cfg* cfg) {
    if (!cfg || cfg->T < 0 || cfg->E < 1 || cfg->k < 1) return 0;
    return forward_layout(cfg, nullptr).total;
}

size_t moe_workspace_size(const moe_cfg* cfg) { return moe_forward_workspace_size(cfg); }

int moe_read_error_flags(const uint32_t* d_flags, void* stream, uint32_t* out) {
    if (!d_flags || !out) return MOE_ERR_NULL;
    uint32_t v = 0;
    hipStream_t s = as_stream(stream);
    if (hipMemcpyAsync(&v, d_flags, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
        return MOE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    *out = v;
    return MOE_OK;
}

int moe_forward(const moe_cfg* c, const moe_weights* w, const uint16_t* x,
                const int32_t* input_ids, const uint8_t* modality, void* y, float* logits_out,
                int32_t* ids_out, float* w_out, uint32_t* d_flags, void* ws, size_t ws_bytes,
                void* stream) {
    return moe_forward_timed(c, w, x, input_ids, modality, y, logits_out, ids_out, w_out, d_flags,
                             ws, ws_bytes, stream, nullptr);
}

int moe_forward_timed(const moe_cfg* c, const moe_weights* w, const uint16_t* x,
                      const int32_t* input_ids, const uint8_t* modality, void* y,
                      float* logits_out, int32_t* ids_out, float* w_out, uint32_t* d_flags,
                      void* ws, size_t ws_bytes, void* stream, void* const* events) {
    int st = forward_checks(c, w);
    if (st != MOE_OK) return st;
    if (c->T == 0) return MOE_OK;
    if (!x || !y || !w->w_g || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_NULL;
    if (c->F_shared > 0 && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_NULL;
    // routed weight format of the expert GEMMs: 0 bf16, 1 MXFP8, 2 MXFP4
    const int wfmt = w->packed == MOE_WEIGHTS_FP8    ? 1
                     : w->packed == MOE_WEIGHTS_FP4  ? 2
                     : w->packed == MOE_WEIGHTS_A8W4 ? 3
                                                     : 0;
    if (wfmt && (!w->w_gate_scale || !w->w_up_scale || !w->w_down_scale)) return MOE_ERR_NULL;
    if (wfmt && (!aligned16(w->w_gate_scale) || !aligned16(w->w_up_scale) ||
                 !aligned16(w->w_down_scale)))
        return MOE_ERR_ALIGN;
    // layout of the bf16 matrices (router, shared expert; routed unless MX)
    const int wpk = wfmt ? 1 : w->packed;
    if (c->mode == MOE_MODE_TOPK) {
        if (c->n_bias < 0 || c->n_bias > 2) return MOE_ERR_SHAPE;
        if (c->n_bias > 0 && !w->score_bias) return MOE_ERR_NULL;
    } else {
        if (!input_ids || !w->tid2eid) return MOE_ERR_NULL;
        if (c->V < 1) return MOE_ERR_SHAPE;
    }
    if (!ws) return MOE_ERR_NULL;
    FwdWs L = forward_layout(c, (char*)ws);
    if (((uintptr_t)ws & 255u) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(y) || !aligned16(w->w_g) || !aligned16(w->w_gate) ||
        !aligned16(w->w_up) || !aligned16(w->w_down))
        return MOE_ERR_ALIGN;
    if (c->F_shared > 0 && (!aligned16(w->s_gate) || !aligned16(w->s_up) || !aligned16(w->s_down)))
        return MOE_ERR_ALIGN;

    hipStream_t s = as_stream(stream);
    const int T = c->T, d = c->d, E = c->E, k = c->k, F = c->F, Fs = c->F_shared;
    float* logits = logits_out ? logits_out : L.logits;
    int32_t* ids = ids_out ? ids_out : L.ids;
    float* wts = w_out ? w_out : L.w;
    hipError_t e;
    auto mark = [&](int i) -> bool {
        return !events || hipEventRecord((hipEvent_t)events[i], s) == hipSuccess;
    };
    if (!mark(0)) return MOE_ERR_HIP;

    // 1. router projection (+ logit offset)
    GemmArgs gl{};
    gl.a = x;
    gl.G = 1;
    gl.rows = T;
    gl.K = d;
    gl.N = E;
    gl.w1 = w->w_g;
    gl.packed = wpk;
    gl.offset = w->logit_offset;
    gl.out = logits;
    if (wpk && router_packed_preferred(T, E))
        e = launch_router_packed(x, w->w_g, w->logit_offset, T, d, E, logits, s);
    else e = launch_grouped_gemm(EPI_F32_OFFSET, gl, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (!mark(1)) return MOE_ERR_HIP;
    // 2. routing
    if ((e = launch_route(logits, c->n_bias > 0 ? w->score_bias : nullptr, modality, input_ids,
                          w->tid2eid, T, E, k, c->n_bias, c->V, c->mode, c->scale, ids, wts,
                          d_flags, s)) != hipSuccess)
        return MOE_ERR_HIP;
    if (!mark(2)) return MOE_ERR_HIP;
    // 3. dispatch permutation + row gather
    // The LDS-staged expert GEMM gathers the token rows through src (no
    // x_perm copy) and passes h in the blocked layout; the register-direct
    // kernel (plain weights) reads a row-major x_perm.  The permutation's
    // first kernel also clears the expert GEMMs' scheduling counters.  A8W4:
    // the rows of x are quantised to MXFP8 once, and gathered as codes.
    const bool a8 = wfmt == 3;
    const bool lds = lds_gemm_ok(wpk, E) && !a8;
    if ((e = launch_permute(ids, x, T, d, E, k, L.counts, L.offsets, L.dest, L.src,
                            lds || a8 ? nullptr : L.x_perm, d_flags, L.perm, s, L.sched,
                            4 * kSchedWords)) != hipSuccess)
        return MOE_ERR_HIP;
    if (a8 && (e = launch_quant_rows_mxfp8(x, T, d, L.x8, L.x8s, s)) != hipSuccess)
        return MOE_ERR_HIP;
    if (!mark(3)) return MOE_ERR_HIP;
    const int rows = T * k;
    // 4. routed experts: gate/up + clamped SwiGLU
    GemmArgs g1{};
    g1.a = lds ? x : L.x_perm;
    g1.gather = lds ? L.src : nullptr;
    g1.a_rows = T;
    g1.offsets = L.offsets;
    g1.G = E;
    g1.rows = rows;
    g1.K = d;
    g1.N = F;
    g1.w1 = w->w_gate;
    g1.w2 = w->w_up;
    g1.packed = wpk;
    g1.wfp8 = wfmt;
    g1.s1 = w->w_gate_scale;
    g1.s2 = w->w_up_scale;
    g1.clamp_limit = c->clamp_limit;
    g1.clamp_mode = c->clamp_mode;
    g1.out = L.h;
    g1.out_blocked = lds;
    g1.sched = L.sched;
    if (a8) {
        // MXFP8 x rows through src, h written as MXFP8 codes (in h) + scales
        g1.gather = L.src;
        g1.a8 = L.x8;
        g1.a_scale = L.x8s;
        g1.out_scale = L.h8s;
    }
    if ((e = expert_gemm(EPI_SWIGLU_BF16, g1, s)) != hipSuccess) return MOE_ERR_HIP;
    if (!mark(4)) return MOE_ERR_HIP;
    // 5. shared expert gate/up
    if (Fs > 0) {
        GemmArgs gs{};
        gs.a = x;
        gs.G = 1;
        gs.rows = T;
        gs.K = d;
        gs.N = Fs;
        gs.w1 = w->s_gate;
        gs.w2 = w->s_up;
        gs.packed = wpk;
        gs.clamp_limit = c->clamp_limit;
        gs.clamp_mode = c->clamp_mode;
        gs.out = L.hs;
        gs.sched = L.sched + kSchedWords;
        if ((e = expert_gemm(EPI_SWIGLU_BF16, gs, s)) != hipSuccess) return MOE_ERR_HIP;
    }
    if (!mark(5)) return MOE_ERR_HIP;
    // 6. routed experts: down projection
    GemmArgs g2{};
    g2.a = L.h;
    g2.offsets = L.offsets;
    g2.G = E;
    g2.rows = rows;
    g2.K = F;
    g2.N = d;
    g2.w1 = w->w_down;
    g2.packed = wpk;
    g2.wfp8 = wfmt;
    g2.s1 = w->w_down_scale;
    g2.out = L.y_perm;
    g2.a_blocked = lds;
    g2.sched = L.sched + 2 * kSchedWords;
    if (a8) {
        g2.a8 = (const uint8_t*)L.h;
        g2.a_scale = L.h8s;
    }
    if ((e = expert_gemm(EPI_F32, g2, s)) != hipSuccess) return MOE_ERR_HIP;
    if (!mark(6)) return MOE_ERR_HIP;
    // 7. shared expert down
    if (Fs > 0) {
        GemmArgs gs{};
        gs.a = L.hs;
        gs.G = 1;
        gs.rows = T;
        gs.K = Fs;
        gs.N = d;
        gs.w1 = w->s_down;
        gs.packed = wpk;
        gs.out = L.ys;
        gs.sched = L.sched + 3 * kSchedWords;
        if ((e = expert_gemm(EPI_F32, gs, s)) != hipSuccess) return MOE_ERR_HIP;
    }
    if (!mark(7)) return MOE_ERR_HIP;
    // 8. weighted combine + shared add
    if ((e = launch_combine(L.y_perm, L.dest, wts, Fs > 0 ? L.ys : nullptr, T, d, k, rows,
                            c->out_dtype, y, s)) != hipSuccess)
        return MOE_ERR_HIP;
    if (!mark(8)) return MOE_ERR_HIP;
    return MOE_OK;
}

size_t moe_backward_workspace_size(const moe_cfg* cfg) {
    if (!cfg || cfg->T < 0 || cfg->E < 1 || cfg->k < 1 || cfg->F_shared < 0) return 0;
    return backward_layout(cfg, nullptr).total;
}

int moe_backward(const moe_cfg* c, const moe_weights* w, const moe_bwd_weights* bw,
                 const uint16_t* x, const int32_t* input_ids, const uint8_t* modality,
                 const float* dy, const moe_grads* gr, uint32_t* d_flags, void* ws,
                 size_t ws_bytes, void* stream) {
    int st = forward_checks(c, w);
    if (st != MOE_OK) return st;
    if (!bw || !gr) return MOE_ERR_NULL;
    if (w->packed != 1) return MOE_ERR_UNSUPPORTED;   // bf16 packed weights only
    // (the gate/up input gradient contracts over 2F and 2 F_shared)
    if (2LL * c->F > kFlatMaxK || 2LL * c->F_shared > kFlatMaxK) return MOE_ERR_UNSUPPORTED;
    if (c->E > grouped_gemm_flat_max_groups()) return MOE_ERR_UNSUPPORTED;
    if (c->T == 0) return MOE_OK;
    const int Fs = c->F_shared;
    if (!x || !dy || !w->w_g || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_NULL;
    if (!bw->w_g || !bw->w_down_t || !bw->w_gu_t) return MOE_ERR_NULL;
    if (!gr->dx || !gr->dw_g || !gr->dw_gate || !gr->dw_up || !gr->dw_down) return MOE_ERR_NULL;
    if (Fs > 0 && (!w->s_gate || !w->s_up || !w->s_down || !bw->s_down_t || !bw->s_gu_t ||
                   !gr->ds_gate || !gr->ds_up || !gr->ds_down))
        return MOE_ERR_NULL;
    if (c->mode == MOE_MODE_TOPK) {
        if (c->n_bias < 0 || c->n_bias > 2) return MOE_ERR_SHAPE;
        if (c->n_bias > 0 && !w->score_bias) return MOE_ERR_NULL;
    } else {
        if (!input_ids || !w->tid2eid) return MOE_ERR_NULL;
        if (c->V < 1) return MOE_ERR_SHAPE;
    }
    if (c->d % 8) return MOE_ERR_UNSUPPORTED;
    if (!ws) return MOE_ERR_NULL;
    BwdWs L = backward_layout(c, (char*)ws);
    if (((uintptr_t)ws & 255u) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    const void* al[] = {x, dy, w->w_g, w->w_gate, w->w_up, w->w_down, bw->w_g, bw->w_down_t,
                        bw->w_gu_t, gr->dx, gr->dw_g, gr->dw_gate, gr->dw_up, gr->dw_down};
    for (const void* p : al)
        if (!aligned16(p)) return MOE_ERR_ALIGN;
    if (Fs > 0) {
        const void* as[] = {w->s_gate, w->s_up, w->s_down, bw->s_down_t, bw->s_gu_t, gr->ds_gate,
                            gr->ds_up, gr->ds_down};
        for (const void* p : as)
            if (!aligned16(p)) return MOE_ERR_ALIGN;
    }

    hipStream_t s = as_stream(stream);
    const int T = c->T, d = c->d, E = c->E, k = c->k, F = c->F;
    const int N = T * k;
    const float Lc = c->clamp_limit;
    const int cm = c->clamp_mode;
    uint32_t* sch = L.sched;
    auto ok = [](hipError_t e) { return e == hipSuccess; };

    // ---- recompute the forward's intermediates
    if (router_packed_preferred(T, E)) {
        if (!ok(launch_router_packed(x, w->w_g, w->logit_offset, T, d, E, L.logits, s)))
            return MOE_ERR_HIP;
    } else {
        GemmArgs gl{};
        gl.a = x;
        gl.G = 1;
        gl.rows = T;
        gl.K = d;
        gl.N = E;
        gl.w1 = w->w_g;
        gl.packed = 1;
        gl.offset = w->logit_offset;
        gl.out = L.logits;
        if (!ok(launch_grouped_gemm(EPI_F32_OFFSET, gl, s))) return MOE_ERR_HIP;
    }
    if (!ok(launch_route(L.logits, c->n_bias > 0 ? w->score_bias : nullptr, modality, input_ids,
                         w->tid2eid, T, E, k, c->n_bias, c->V, c->mode, c->scale, L.ids, L.w,
                         d_flags, s)))
        return MOE_ERR_HIP;
    if (!ok(launch_permute(L.ids, x, T, d, E, k, L.counts, L.offsets, L.dest, L.src, L.x_perm,
                           d_flags, L.perm, s, sch, 8 * kSchedWords)))
        return MOE_ERR_HIP;
    // gate/up with the pre-activations saved, h row-major; then y_perm
    if (!ok(flat_gemm(EPI_SWIGLU_BF16, L.x_perm, L.offsets, E, N, d, F, w->w_gate, w->w_up, Lc,
                      cm, L.h, L.g, L.u, sch, s)))
        return MOE_ERR_HIP;
    if (!ok(flat_gemm(EPI_F32, L.h, L.offsets, E, N, F, d, w->w_down, nullptr, Lc, cm, L.y_perm,
                      nullptr, nullptr, sch + kSchedWords, s)))
        return MOE_ERR_HIP;

    // ---- combine -> expert outputs and routing weights
    if (!ok(launch_combine_backward_bf16(dy, L.y_perm, L.dest, L.w, T, d, k, N, L.dyp16, L.dtw,
                                         s)))
        return MOE_ERR_HIP;
    // ---- down projection: weight and input gradients
    if (!ok(launch_grouped_wgrad(L.dyp16, L.h, L.offsets, E, N, d, F, gr->dw_down, s)))
        return MOE_ERR_HIP;
    if (!ok(flat_gemm(EPI_F32, L.dyp16, L.offsets, E, N, d, F, bw->w_down_t, nullptr, Lc, cm,
                      L.dh, nullptr, nullptr, sch + 2 * kSchedWords, s)))
        return MOE_ERR_HIP;
    // ---- clamped SwiGLU, then gate/up weight and input gradients
    if (!ok(launch_swiglu_backward_bf16(L.g, L.u, L.dh, N, F, Lc, cm, L.dgu, s)))
        return MOE_ERR_HIP;
    if (!ok(launch_grouped_wgrad(L.dgu, L.x_perm, L.offsets, E, N, F, d, gr->dw_gate, s, 2 * F)))
        return MOE_ERR_HIP;
    if (!ok(launch_grouped_wgrad(L.dgu + F, L.x_perm, L.offsets, E, N, F, d, gr->dw_up, s, 2 * F)))
        return MOE_ERR_HIP;
    float* dxp = L.dyp;
    if (!ok(flat_gemm(EPI_F32, L.dgu, L.offsets, E, N, 2 * F, d, bw->w_gu_t, nullptr, Lc, cm, dxp,
                      nullptr, nullptr, sch + 3 * kSchedWords, s)))
        return MOE_ERR_HIP;

    // ---- shared expert on x with dy
    if (Fs > 0) {
        if (!ok(flat_gemm(EPI_SWIGLU_BF16, x, nullptr, 1, T, d, Fs, w->s_gate, w->s_up, Lc, cm,
                          L.hs, L.gs, L.us, sch + 4 * kSchedWords, s)))
            return MOE_ERR_HIP;
        if (!ok(launch_cast_bf16(dy, (long long)T * d, L.dy16, s))) return MOE_ERR_HIP;
        if (!ok(launch_grouped_wgrad(L.dy16, L.hs, nullptr, 1, T, d, Fs, gr->ds_down, s)))
            return MOE_ERR_HIP;
        if (!ok(flat_gemm(EPI_F32, L.dy16, nullptr, 1, T, d, Fs, bw->s_down_t, nullptr, Lc, cm,
                          L.dhs, nullptr, nullptr, sch + 5 * kSchedWords, s)))
            return MOE_ERR_HIP;
        if (!ok(launch_swiglu_backward_bf16(L.gs, L.us, L.dhs, T, Fs, Lc, cm, L.dgus, s)))
            return MOE_ERR_HIP;
        if (!ok(launch_grouped_wgrad(L.dgus, x, nullptr, 1, T, Fs, d, gr->ds_gate, s, 2 * Fs)))
            return MOE_ERR_HIP;
        if (!ok(launch_grouped_wgrad(L.dgus + Fs, x, nullptr, 1, T, Fs, d, gr->ds_up, s, 2 * Fs)))
            return MOE_ERR_HIP;
        if (!ok(flat_gemm(EPI_F32, L.dgus, nullptr, 1, T, 2 * Fs, d, bw->s_gu_t, nullptr, Lc, cm,
                          L.dxs, nullptr, nullptr, sch + 6 * kSchedWords, s)))
            return MOE_ERR_HIP;
    }
    // ---- dx = (each token's dx_perm rows, unit weights) + shared expert's
    if (!ok(launch_combine(dxp, L.dest, nullptr, Fs > 0 ? L.dxs : nullptr, T, d, k, N, MOE_OUT_F32,
                           gr->dx, s)))
        return MOE_ERR_HIP;
    // ---- routing weights -> logits -> router projection
    if (!ok(launch_route_backward(L.logits, L.ids, L.dtw, T, E, k, c->scale, L.dl, d_flags, s)))
        return MOE_ERR_HIP;
    if (!ok(launch_router_backward(L.dl, L.ids, L.offsets, L.src, x, bw->w_g, T, d, E, k, gr->dx,
                                   gr->dw_g, s)))
        return MOE_ERR_HIP;
    return MOE_OK;
}

}  // extern "C"
