/*
 * CPU oracle for the forward pass of a fine-grained Mixture-of-Experts layer
 * (DeepSeek-V4 / V4.1-Flash style: sigmoid-scored, bias-ranked top-k routing,
 * hash routing through a tid2eid table, token dispatch, two expert GEMMs with a
 * clamped SwiGLU, a shared expert, and a routing-weight combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source with
 * the HIP path and must never be used as a fallback for it.
 *
 * Every step is written as its plain definition, in the order the pages give:
 *   - "HyperParallel accelerates DeepSeek-V4.1 multimodal 1M long-sequence
 *     training", section 2.3 (MegaKernel), MegaGate bullet: scoring, bias
 *     ranking, Top-K, score extraction, normalisation, scaling; separate text
 *     and vision routing bias; projection matmul kept outside the gate.
 *   - same page, section 2.3, MegaMoE bullet: token dispatch, two expert
 *     matmuls, SwiGLU activation with the V4.1 clamp, result return.
 *   - "Twinkle x Ascend ... DeepSeek-V4 training", section "FSDP2-4D parallel
 *     engine adaptation": the router returns logits / routing weights /
 *     selected experts; HashRouter takes ids from tid2eid[input_ids] and still
 *     weights them from the gate logits; one dispatch path for both; results
 *     merged by routing weight.
 *   - "MindSpore HyperParallel one-click DeepSeek-V4.1-Flash", section 01:
 *     1 shared expert + 384 routed experts, 6 routed experts per token.
 * Readings of what the pages leave open (score function = sigmoid, clamp
 * limit L, clamp form, tie order, shared-expert form) are the ones listed in
 * the design notes; each function below states the one it uses.
 *
 * Floating point: fp64 everywhere the pages do not fix a precision, except
 * the routing decision, which both sides take in IEEE binary32 with the pinned
 * score function S() below.  Build with -ffp-contract=off and without
 * fast-math; x86-64 SSE arithmetic is IEEE binary32/binary64 with RNE.
 *
 * Parity pins (see tests/test_oracle_*.py): S() against fp64 sigmoid over
 * every binary32 input in [-80, 80]; top-k against brute-force subset
 * enumeration with forced ties; weights against the textbook normalised
 * sigmoid ratio; the permutation against a library stable argsort and its
 * invariants; the FFN against a numpy fp64 dense FFN and the clamp's closed
 * form; the combine against the dense reductions (single forced expert,
 * identical experts, scale 0); the MXFP8 encoding against torch's
 * float8_e4m3fn (every code, RNE casts, saturated block codes) and numpy's
 * frexp for the block exponent; the MXFP4 encoding against the E2M1 value
 * table of the OCP specification and brute force over its 16 codes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MODE_TOPK 0
#define ORC_MODE_HASH 1
#define ORC_FLAG_BAD_INPUT_ID 1u
#define ORC_FLAG_BAD_EXPERT_ID 2u

/* ---------------------------------------------------------------- bf16 ---- */

static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary64 value to the nearest bfloat16 (8 significant bits, binary32
 * exponent range), ties to even, in one step (no intermediate binary32). */
uint16_t orc_f64_to_bf16(double v)
{
    if (v != v)
        return 0x7FC0u;
    uint16_t sign = (uint16_t)(signbit(v) ? 0x8000u : 0u);
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    double r;
    if (a < ldexp(1.0, -126)) {
        /* subnormal bfloat16: spacing 2^-133 */
        r = nearbyint(ldexp(a, 133));
        r = ldexp(r, -133);
    } else {
        int e;
        double m = frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1 */
        r = nearbyint(ldexp(m, 8)); /* 8 significant bits */
        r = ldexp(r, e - 8);
    }
    /* largest finite bfloat16 is (2 - 2^-7) * 2^127 */
    if (r > ldexp(2.0 - ldexp(1.0, -7), 127))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* ------------------------------------------------- pinned score function ---- */
/*
 * S(x) = 1 / (1 + exp(-x)) in IEEE binary32, evaluated as a fixed sequence of
 * correctly rounded binary32 operations so that any IEEE machine reproduces
 * the same bits (the routing decision depends on them):
 *   1. x <- clamp(x, -80, 80) (NaN -> -80); keeps every intermediate normal.
 *   2. z = -x; n = rint(z * log2(e)) (round to nearest even).
 *   3. Cody-Waite additive reduction (Cody & Waite, Software Manual for the
 *      Elementary Functions, 1980): r = z - n*C1 - n*C2 with C1 + C2 = ln 2,
 *      C1 carrying few enough bits that n*C1 is exact; each step one fma.
 *   4. exp(r) by the degree-7 Taylor polynomial in Horner form with fma
 *      (coefficients 1/j! rounded to binary32); |r| <= ~ln2/2, so the
 *      truncation error is below 2^-27 relative.
 *   5. e = p * 2^n (exact), S = 1 / (1 + e) with correctly rounded division.
 */
float orc_score(float x)
{
    if (x != x)
        x = -80.0f;
    if (x < -80.0f)
        x = -80.0f;
    if (x > 80.0f)
        x = 80.0f;
    const float log2e = (float)1.4426950408889634;     /* 1/ln 2 */
    const float c1 = 0.693145751953125f;               /* 0x3F317200 */
    const float c2 = (float)(0.69314718055994531 - 0.693145751953125);
    float z = -x;
    float t = z * log2e;
    float n = rintf(t);
    float r = fmaf(-n, c1, z);
    r = fmaf(-n, c2, r);
    float p = (float)(1.0 / 5040.0);
    p = fmaf(p, r, (float)(1.0 / 720.0));
    p = fmaf(p, r, (float)(1.0 / 120.0));
    p = fmaf(p, r, (float)(1.0 / 24.0));
    p = fmaf(p, r, (float)(1.0 / 6.0));
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    float e = ldexpf(p, (int)n);
    float den = 1.0f + e;
    return 1.0f / den;
}

void orc_score_array(const float* x, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_score(x[i]);
}

/* ------------------------------------------------------ router projection -- */
/* Router logits l[t,e] = fl32( sum_i x[t,i] * Wg[e,i] + off[e] ), sum in fp64.
 * (Projection stays outside the gate: MegaGate bullet, section 2.3.) */
void orc_gate_logits(const uint16_t* x, const uint16_t* wg, const float* off,
                     int T, int d, int E, float* logits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int i = 0; i < d; ++i)
                s += bf16_value(x[(size_t)t * d + i]) * bf16_value(wg[(size_t)e * d + i]);
            if (off)
                s += (double)off[e];
            logits[(size_t)t * E + e] = (float)s;
        }
    }
}

/* ---------------------------------------------------------------- routing -- */
/*
 * MegaGate order: score -> bias ranking -> Top-K -> score extraction ->
 * normalise -> scale.  TopK mode:
 *   s[e] = S(l[t,e]);  r[e] = fl32(s[e] + b[m(t), e])  (m(t) = modality, 0 text,
 *   1 vision; always row 0 when n_bias == 1; no bias when b == NULL);
 *   ids = the k experts greatest under (r descending, expert index ascending),
 *   listed in that order.
 * Hash mode (HashRouter): ids[t,j] = tid2eid[input_ids[t], j] in table order,
 *   no bias, no ranking.
 * Both: g_j = s[ids_j] (unbiased score); S_t = left-to-right fp32 sum of g;
 *   w_j = fl32( fl32(g_j / S_t) * scale ).
 * A token whose input id is outside [0, V) or whose table row holds an id
 * outside [0, E) gets ids = -1, w = 0 and sets a flag bit.
 * Returns the OR of flag bits.
 */
unsigned orc_route(const float* logits, const float* bias, const uint8_t* modality,
                   const int32_t* input_ids, const int32_t* tid2eid,
                   int T, int E, int k, int n_bias, int V, int mode, float scale,
                   int32_t* ids, float* w)
{
    unsigned flags = 0;
    float* s = (float*)malloc(sizeof(float) * (size_t)E);
    float* r = (float*)malloc(sizeof(float) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float* lt = logits + (size_t)t * E;
        int32_t* it = ids + (size_t)t * k;
        float* wt = w + (size_t)t * k;
        for (int e = 0; e < E; ++e)
            s[e] = orc_score(lt[e]);
        int valid = 1;
        if (mode == ORC_MODE_TOPK) {
            const float* b = NULL;
            if (bias) {
                int row = 0;
                if (n_bias > 1 && modality)
                    row = modality[t] ? 1 : 0;
                b = bias + (size_t)row * E;
            }
            for (int e = 0; e < E; ++e) {
                r[e] = b ? s[e] + b[e] : s[e];
                taken[e] = 0;
            }
            for (int j = 0; j < k; ++j) {
                int best = -1;
                for (int e = 0; e < E; ++e) {
                    if (taken[e])
                        continue;
                    if (best < 0 || r[e] > r[best])
                        best = e;
                }
                taken[best] = 1;
                it[j] = best;
            }
        } else {
            int32_t tok = input_ids[t];
            if (tok < 0 || tok >= V) {
                flags |= ORC_FLAG_BAD_INPUT_ID;
                valid = 0;
            } else {
                for (int j = 0; j < k; ++j) {
                    int32_t e = tid2eid[(size_t)tok * k + j];
                    if (e < 0 || e >= E) {
                        flags |= ORC_FLAG_BAD_EXPERT_ID;
                        valid = 0;
                    }
                    it[j] = e;
                }
            }
        }
        if (!valid) {
            for (int j = 0; j < k; ++j) {
                it[j] = -1;
                wt[j] = 0.0f;
            }
            continue;
        }
        float sum = s[it[0]];
        for (int j = 1; j < k; ++j)
            sum = sum + s[it[j]];
        for (int j = 0; j < k; ++j) {
            float q = s[it[j]] / sum;
            wt[j] = q * scale;
        }
    }
    free(s);
    free(r);
    free(taken);
    return flags;
}

/* ------------------------------------------------------ routing backward -- */
/*
 * Gradient of the routing weights with respect to the router logits: the
 * first link of MegaGate's backward ("HyperParallel accelerates DeepSeek-V4.1
 * ...", section 2.3: the gate's normalisation and scaling steps, whose
 * gradients the fused backward chain carries).  The forward gives
 *   g_j = S(l[t, ids_j])  (the pinned binary32 sigmoid),
 *   w_j = scale * g_j / sum_i g_i.
 * The expert choice is piecewise constant in the logits and the ranking
 * bias takes no part in w, so only the k selected logits of a token get a
 * gradient:
 *   dg_i = (scale / G) * (dw_i - sum_j dw_j g_j / G),   G = sum_j g_j,
 *        = (scale / G) * sum_j g_j (dw_i - dw_j) / G   (evaluated so: exactly
 *          0 for k = 1 or equal dw, where the weights are constant),
 *   dl[t, ids_i] += dg_i * g_i * (1 - g_i)   (the logistic derivative at the
 *                                             forward's score value),
 * and every other entry of the row is 0.  A token whose ids are not all in
 * [0, E) (dropped by the forward) gets a zero row and sets
 * ORC_FLAG_BAD_EXPERT_ID.  All arithmetic after S() is fp64.
 */
unsigned orc_route_backward(const float* logits, const int32_t* ids, const float* dw,
                            int T, int E, int k, float scale, double* dl)
{
    unsigned flags = 0;
    double g[64];
    for (int t = 0; t < T; ++t) {
        const float* lt = logits + (size_t)t * E;
        const int32_t* it = ids + (size_t)t * k;
        const float* dwt = dw + (size_t)t * k;
        double* out = dl + (size_t)t * E;
        for (int e = 0; e < E; ++e)
            out[e] = 0.0;
        int valid = 1;
        for (int j = 0; j < k; ++j)
            if (it[j] < 0 || it[j] >= E)
                valid = 0;
        if (!valid) {
            flags |= ORC_FLAG_BAD_EXPERT_ID;
            continue;
        }
        double G = 0.0;
        for (int j = 0; j < k; ++j) {
            g[j] = (double)orc_score(lt[it[j]]);
            G += g[j];
        }
        for (int i = 0; i < k; ++i) {
            double br = 0.0;
            for (int j = 0; j < k; ++j)
                br += g[j] * ((double)dwt[i] - (double)dwt[j]);
            double dg = (double)scale / G * (br / G);
            out[it[i]] += dg * g[i] * (1.0 - g[i]);
        }
    }
    return flags;
}

/* ------------------------------------------------------------ permutation -- */
/*
 * Dispatch (Twinkle: ids from either router become global expert ids ->
 * expert_mask -> one token-dispatch flow; the all-to-all of expert parallelism
 * is, on one device, a permutation of token copies grouped by expert).
 * Stable counting sort of the flattened pairs (t, j), t-major, by expert id:
 *   counts[e] = #{(t,j) : ids = e};  offsets = exclusive prefix sum,
 *   offsets[E] = number of valid pairs;
 *   dest[t*k+j] = offsets[e] + #{earlier pairs with the same expert};
 *   src[row] = t for every filled row, -1 for rows in [offsets[E], T*k).
 * Pairs with an id outside [0, E) get dest = -1 and set a flag bit.
 */
unsigned orc_permute(const int32_t* ids, int T, int k, int E,
                     int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src)
{
    unsigned flags = 0;
    int64_t n = (int64_t)T * k;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = ids[i];
        if (e >= 0 && e < E)
            counts[e] += 1;
        else
            flags |= ORC_FLAG_BAD_EXPERT_ID;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int64_t i = 0; i < n; ++i)
        src[i] = -1;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = ids[i];
        if (e < 0 || e >= E) {
            dest[i] = -1;
            continue;
        }
        int32_t row = cursor[e]++;
        dest[i] = row;
        src[row] = (int32_t)(i / k);
    }
    free(cursor);
    return flags;
}

/* x_perm[row] = x[src[row]] for rows with src >= 0 (exact copy). */
void orc_gather(const uint16_t* x, const int32_t* src, int64_t rows, int d, uint16_t* x_perm)
{
    for (int64_t r = 0; r < rows; ++r) {
        if (src[r] < 0)
            continue;
        memcpy(x_perm + r * d, x + (int64_t)src[r] * d, sizeof(uint16_t) * (size_t)d);
    }
}

/* ---------------------------------------------------------- grouped GEMM -- */
/*
 * One grouped matmul of the expert FFN's shape, out = A W_g^T per group
 * ("HyperParallel accelerates DeepSeek-V4.1 ...", section 2.3, MegaMoE: the
 * expert matmuls; in the backward the same product gives the input
 * gradients, dH = dY W_down = dY (W_down^T)^T):
 *   out[r, n] = sum_k a[r, k] * w[g, n, k]   for offsets[g] <= r < offsets[g+1],
 * a and w bf16, exact products summed in fp64.  Rows outside every group
 * are left as they are.
 */
void orc_grouped_gemm(const uint16_t* a, const int32_t* offsets, int G, int K, int N,
                      const uint16_t* w, double* out)
{
    for (int g = 0; g < G; ++g) {
        const uint16_t* wg = w + (size_t)g * N * K;
#pragma omp parallel for schedule(static)
        for (int r = offsets[g]; r < offsets[g + 1]; ++r) {
            for (int n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int k = 0; k < K; ++k)
                    acc += bf16_value(a[(size_t)r * K + k]) * bf16_value(wg[(size_t)n * K + k]);
                out[(size_t)r * N + n] = acc;
            }
        }
    }
}

/* ------------------------------------------------ grouped weight gradient -- */
/*
 * Weight gradient of a grouped matmul ("HyperParallel accelerates
 * DeepSeek-V4.1 ...", section 2.3, MegaMoE: the expert matmuls, whose weights
 * a training step updates; section 03: the training run).  For the forward
 * out = A W_g^T per group (orc_grouped_gemm) and a gradient dy of out, the
 * chain rule gives
 *   dw[g, m, k] = sum_{offsets[g] <= r < offsets[g+1]} dy[r, m] * a[r, k],
 * dy and a bf16, exact products summed in fp64.  A group without rows gets a
 * zero gradient.  With dy = dY, a = H it is the down projection's dW_down;
 * with dy = dG or dU, a = X (the dispatched tokens) dW_gate or dW_up; with a
 * single group of T rows, dy = the router logits' gradient and a = x, it is
 * the router projection's dW_g.
 */
void orc_grouped_wgrad(const uint16_t* dy, const uint16_t* a, const int32_t* offsets, int G,
                       int M, int K, double* dw)
{
    for (int g = 0; g < G; ++g) {
        const int lo = offsets[g], hi = offsets[g + 1];
        double* dwg = dw + (size_t)g * M * K;
#pragma omp parallel for schedule(static)
        for (int m = 0; m < M; ++m) {
            for (int k = 0; k < K; ++k) {
                double acc = 0.0;
                for (int r = lo; r < hi; ++r)
                    acc += bf16_value(dy[(size_t)r * M + m]) * bf16_value(a[(size_t)r * K + k]);
                dwg[(size_t)m * K + k] = acc;
            }
        }
    }
}

/* The same definition at n listed entries (g[i], m[i], k[i]) only, for
 * sampled checks at sizes where the whole gradient is too large. */
void orc_grouped_wgrad_entries(const uint16_t* dy, const uint16_t* a, const int32_t* offsets,
                               int M, int K, const int32_t* g, const int32_t* m, const int32_t* k,
                               int64_t n, double* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int r = offsets[g[i]]; r < offsets[g[i] + 1]; ++r)
            acc += bf16_value(dy[(size_t)r * M + m[i]]) * bf16_value(a[(size_t)r * K + k[i]]);
        out[i] = acc;
    }
}

/* ---------------------------------------------------- router backward -- */
/*
 * Gradients of the router projection l = x W_g^T ("HyperParallel accelerates
 * DeepSeek-V4.1 ...", section 2.3, MegaGate: the projection matmul that
 * feeds the gate) for a gradient dl of the logits:
 *   dx[t, i]  = sum_e dl[t, e] * w_g[e, i]
 *   dwg[e, i] = sum_t dl[t, e] * x[t, i]
 * dl in fp64 (the routing backward's output), x and w_g bf16, fp64 sums over
 * every expert / token (the plain dense definition).
 */
void orc_router_backward(const double* dl, const uint16_t* x, const uint16_t* wg, int T, int d,
                         int E, double* dx, double* dwg)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int e = 0; e < E; ++e)
                acc += dl[(size_t)t * E + e] * bf16_value(wg[(size_t)e * d + i]);
            dx[(size_t)t * d + i] = acc;
        }
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e)
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int t = 0; t < T; ++t)
                acc += dl[(size_t)t * E + e] * bf16_value(x[(size_t)t * d + i]);
            dwg[(size_t)e * d + i] = acc;
        }
}

/* n values rounded to bf16 (nearest, ties to even): the precision in which a
 * gradient enters the matrix cores in the backward. */
void orc_round_bf16_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(v[i]);
}

/* out = a + b elementwise (fp64): the sum of the gradient contributions that
 * reach the same tensor along different paths of the layer. */
void orc_add_f64(const double* a, const double* b, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = a[i] + b[i];
}

/* ------------------------------------------------------ SwiGLU backward -- */
/*
 * Backward of the clamped SwiGLU between the expert matmuls ("HyperParallel
 * accelerates DeepSeek-V4.1 ...", section 2.3, MegaMoE: SwiGLU with the V4.1
 * clamp).  For h = silu(cg(G)) * cu(U) with the clamps of ffn_row and a
 * gradient dh of h:
 *   dU = dh * silu(cg(G)) * [U inside [-L, L]],
 *   dG = dh * cu(U) * silu'(cg(G)) * [G inside the gate clamp's range],
 *   silu'(z) = s (1 + z (1 - s)),  s = 1 / (1 + exp(-z)),
 * a clamp passing its gradient on the closed range (as at the limits the
 * clamp is the identity from the inside).  fp64 from fp32 inputs.
 */
void orc_swiglu_backward(const float* gate, const float* up, const float* dh, int64_t n,
                         double L, int clamp_mode, double* dgate, double* dup)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double g = gate[i], u = up[i], gh = dh[i];
        int g_in = clamp_mode == 0 ? (g >= -L && g <= L) : (g <= L);
        int u_in = (u >= -L && u <= L);
        double gc = g, uc = u;
        if (gc > L) gc = L;
        if (clamp_mode == 0 && gc < -L) gc = -L;
        if (uc > L) uc = L;
        if (uc < -L) uc = -L;
        double sg = 1.0 / (1.0 + exp(-gc));
        double silu = gc * sg;
        dup[i] = u_in ? gh * silu : 0.0;
        dgate[i] = g_in ? gh * uc * sg * (1.0 + gc * (1.0 - sg)) : 0.0;
    }
}

/* ------------------------------------------------------------- expert FFN -- */
/*
 * One expert on one activation row a[0..d):
 *   G_f = sum_i a_i * Wgate[f,i],  U_f = sum_i a_i * Wup[f,i]   (fp64)
 *   clamp (limit L > 0; L = +inf disables it):
 *     mode 0 (symmetric):  G <- min(max(G,-L),L),  U <- min(max(U,-L),L)
 *     mode 1 (gate above): G <- min(G, L),          U <- min(max(U,-L),L)
 *   h_f = bf16_rne( silu(G_f) * U_f ),  silu(z) = z / (1 + exp(-z))   (fp64)
 *   y_o = sum_f h_f * Wdown[o,f]   (fp64, from the bf16-rounded h)
 * Weights are stored [out, in]: Wgate/Wup [F,d], Wdown [d,F].  The bf16
 * rounding of h is kept because h is the bf16 input of the second matmul.
 */
static void ffn_row(const uint16_t* a, int d, int F,
                    const uint16_t* wgate, const uint16_t* wup, const uint16_t* wdown,
                    double L, int clamp_mode, uint16_t* h_out, double* y_out, double* hbuf)
{
    for (int f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        const uint16_t* rg = wgate + (size_t)f * d;
        const uint16_t* ru = wup + (size_t)f * d;
        for (int i = 0; i < d; ++i) {
            double ai = bf16_value(a[i]);
            g += ai * bf16_value(rg[i]);
            u += ai * bf16_value(ru[i]);
        }
        if (clamp_mode == 0) {
            if (g > L) g = L;
            if (g < -L) g = -L;
        } else {
            if (g > L) g = L;
        }
        if (u > L) u = L;
        if (u < -L) u = -L;
        double silu = g / (1.0 + exp(-g));
        uint16_t hb = orc_f64_to_bf16(silu * u);
        if (h_out)
            h_out[f] = hb;
        hbuf[f] = bf16_value(hb);
    }
    if (!y_out)
        return;
    for (int o = 0; o < d; ++o) {
        double acc = 0.0;
        const uint16_t* rd = wdown + (size_t)o * F;
        for (int f = 0; f < F; ++f)
            acc += hbuf[f] * bf16_value(rd[f]);
        y_out[o] = acc;
    }
}

/*
 * Grouped expert FFN over a permuted activation matrix a[rows, d]: rows
 * [offsets[g], offsets[g+1]) go through expert g (weights at g*F*d and
 * g*d*F).  h[rows,F] (bf16 bits) and y[rows,d] (fp64) are written for those
 * rows only.  The shared expert is the G = 1, offsets = {0, T} case on x.
 */
void orc_expert_ffn(const uint16_t* a, const int32_t* offsets, int G, int d, int F,
                    const uint16_t* wgate, const uint16_t* wup, const uint16_t* wdown,
                    double L, int clamp_mode, uint16_t* h, double* y)
{
    for (int g = 0; g < G; ++g) {
        int64_t lo = offsets[g], hi = offsets[g + 1];
        const uint16_t* wg = wgate + (size_t)g * F * d;
        const uint16_t* wu = wup + (size_t)g * F * d;
        const uint16_t* wd = wdown + (size_t)g * d * F;
#pragma omp parallel
        {
            double* hbuf = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = lo; r < hi; ++r)
                ffn_row(a + r * d, d, F, wg, wu, wd, L, clamp_mode,
                        h ? h + r * F : NULL, y ? y + r * d : NULL, hbuf);
            free(hbuf);
        }
    }
}

/*
 * Same FFN for an explicit list of rows: row rows[i] of a goes through expert
 * experts[i].  Outputs are packed: h_out[i*F..], y_out[i*d..].  Used to check
 * sampled rows of full-size runs.
 */
void orc_expert_ffn_rows(const uint16_t* a, const int64_t* rows, const int32_t* experts, int n,
                         int d, int F, const uint16_t* wgate, const uint16_t* wup,
                         const uint16_t* wdown, double L, int clamp_mode,
                         uint16_t* h_out, double* y_out)
{
#pragma omp parallel
    {
        double* hbuf = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; ++i) {
            int64_t e = experts[i];
            ffn_row(a + rows[i] * d, d, F, wgate + e * F * d, wup + e * F * d,
                    wdown + e * d * F, L, clamp_mode,
                    h_out ? h_out + (int64_t)i * F : NULL,
                    y_out ? y_out + (int64_t)i * d : NULL, hbuf);
        }
        free(hbuf);
    }
}

/* ---------------------------------------------------------------- combine -- */
/*
 * Result return, merged by routing weight, plus the always-on shared expert
 * (weight 1):  y[t,o] = ysh[t,o] + sum_j w[t,j] * y_perm[dest[t,j], o]  (fp64).
 * Pairs with dest < 0 are skipped; ysh may be NULL (no shared expert).
 */
void orc_combine(const double* y_perm, const int32_t* dest, const float* w, const double* ysh,
                 int T, int d, int k, double* y)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int o = 0; o < d; ++o) {
            double acc = ysh ? ysh[(size_t)t * d + o] : 0.0;
            for (int j = 0; j < k; ++j) {
                int32_t row = dest[(size_t)t * k + j];
                if (row < 0)
                    continue;
                acc += (double)w[(size_t)t * k + j] * y_perm[(size_t)row * d + o];
            }
            y[(size_t)t * d + o] = acc;
        }
    }
}

/*
 * Backward of the combine (the result return merged by routing weight,
 * "Twinkle x Ascend ...", section "FSDP2-4D parallel engine adaptation"):
 * for y[t] = y_shared[t] + sum_j w[t,j] Y_perm[dest[t,j]] and a gradient dy
 * of the output,
 *   dY_perm[dest[t,j], o] = w[t,j] * dy[t,o]          (not rounded),
 *   dw[t,j]               = sum_o dy[t,o] * Y_perm[dest[t,j], o],
 * and dy_shared = dy.  A pair with dest outside [0, rows) gets dw = 0 and
 * writes no row; rows no pair maps to are left as they are.  fp64.
 */
void orc_combine_backward(const float* dy, const float* y_perm, const int32_t* dest,
                          const float* w, int T, int d, int k, int rows,
                          double* dy_perm, double* dw)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t row = dest[(size_t)t * k + j];
            double acc = 0.0;
            if (row >= 0 && row < rows) {
                for (int o = 0; o < d; ++o) {
                    double g = (double)dy[(size_t)t * d + o];
                    acc += g * (double)y_perm[(size_t)row * d + o];
                    dy_perm[(size_t)row * d + o] = (double)w[(size_t)t * k + j] * g;
                }
            }
            dw[(size_t)t * k + j] = acc;
        }
    }
}

/*
 * The layer output for a list of tokens, from their routing (ids, w):
 *   y[t] = FFN_shared(x[t]) + sum_j w[t,j] * FFN_{ids[t,j]}(x[t]).
 * Identical by definition to permute -> grouped FFN -> combine, because every
 * dispatched row is an exact copy of its token's row; used for sampled checks
 * of full-size runs.  Shared weights may be NULL (no shared expert).
 */
void orc_tokens_forward(const uint16_t* x, const int64_t* tokens, int n, int d, int F, int k,
                        const int32_t* ids, const float* w,
                        const uint16_t* wgate, const uint16_t* wup, const uint16_t* wdown,
                        const uint16_t* sgate, const uint16_t* sup, const uint16_t* sdown, int Fs,
                        double L, int clamp_mode, double* y_out)
{
#pragma omp parallel
    {
        int Fmax = F > Fs ? F : Fs;
        double* hbuf = (double*)malloc(sizeof(double) * (size_t)Fmax);
        double* ye = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; ++i) {
            int64_t t = tokens[i];
            const uint16_t* a = x + t * d;
            double* yt = y_out + (int64_t)i * d;
            for (int o = 0; o < d; ++o)
                yt[o] = 0.0;
            if (sgate) {
                ffn_row(a, d, Fs, sgate, sup, sdown, L, clamp_mode, NULL, ye, hbuf);
                for (int o = 0; o < d; ++o)
                    yt[o] += ye[o];
            }
            for (int j = 0; j < k; ++j) {
                int64_t e = ids[t * k + j];
                if (e < 0)
                    continue;
                double wj = (double)w[t * k + j];
                ffn_row(a, d, F, wgate + e * F * d, wup + e * F * d, wdown + e * d * F,
                        L, clamp_mode, NULL, ye, hbuf);
                for (int o = 0; o < d; ++o)
                    yt[o] += wj * ye[o];
            }
        }
        free(hbuf);
        free(ye);
    }
}

/* ------------------------------------------------------ fp8 expert weights -- */
/*
 * 8-bit expert weights.  The pages name MXFP8 / MXFP4 as the low-precision
 * direction ("CANN DeepSeek-V4 training optimisation", outlook section,
 * functional-expansion bullets; the V4-Flash checkpoints ship in FP4/FP8,
 * quick-start section of "Twinkle x Ascend ... DeepSeek-V4 training") without restating the format.  MXFP8 is the OCP Microscaling
 * format: blocks of 32 consecutive values along K share one power-of-two
 * scale (E8M0), each value an OCP 8-bit float E4M3 ("E4M3FN": 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities,
 * S.1111.111 is NaN, largest finite 448).  Conversion, per the OCP MX
 * specification's rule:
 *   X    = floor(log2(max |v| over the block)) - 8   (8 = E4M3's largest
 *          exponent), clamped here to [-110, 110] (X = 0 for an all-zero
 *          block);
 *   q[i] = E4M3(v[i] / 2^X), round to nearest, ties to even, values beyond
 *          448 saturated to +-448;
 *   dequantised value = E4M3 value of q[i] * 2^X.
 * With X in [-110, 110] the dequantised value has at most 4 significant bits
 * and a binary exponent inside bfloat16's normal range, so it is exactly a
 * bf16 value: the FFN of the fp8 mode is the bf16 FFN on the dequantised
 * weights.
 */

/* value of an E4M3 code (NaN for S.1111.111) */
double orc_e4m3_decode(uint8_t c)
{
    const double s = (c & 0x80) ? -1.0 : 1.0;
    const int E = (c >> 3) & 15, M = c & 7;
    if ((c & 0x7f) == 0x7f)
        return NAN;
    if (E == 0)
        return s * ldexp((double)M, -9);          /* subnormal: M/8 * 2^-6 */
    return s * ldexp(1.0 + M / 8.0, E - 7);
}

/* E4M3 code of v: round to nearest, ties to even; |v| > 448 saturates */
uint8_t orc_e4m3_encode(double v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7e;
    if (a < ldexp(1.0, -6)) {                     /* subnormal range, spacing 2^-9 */
        const double m = nearbyint(ldexp(a, 9)); /* 0 .. 8 (8 = smallest normal) */
        return sign | (uint8_t)m;                 /* m = 8 encodes as E = 1, M = 0 */
    }
    int x;
    frexp(a, &x);                                 /* a = f * 2^x, f in [0.5, 1) */
    int E = x - 1;                                /* 2^E <= a < 2^(E+1), E >= -6 */
    double m = nearbyint((ldexp(a, -E) - 1.0) * 8.0);   /* 0 .. 8 */
    if (m == 8.0) {
        m = 0.0;
        E += 1;
    }
    if (E > 8 || (E == 8 && m > 6.0))             /* above 448 after rounding */
        return sign | 0x7e;
    return sign | (uint8_t)(((E + 7) << 3) | (int)m);
}

/* MXFP8 quantisation of bf16 weights [R, K] (K multiple of 32): codes
 * [R, K], block exponents X [R, K/32] */
void orc_quant_mxfp8(const uint16_t* w, int64_t R, int K, uint8_t* q, int32_t* x)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int b = 0; b < K / 32; ++b) {
            const uint16_t* v = w + r * K + 32 * b;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                const double a = fabs(bf16_value(v[i]));
                if (a > amax)
                    amax = a;
            }
            int X = 0;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);                 /* 2^(ex-1) <= amax < 2^ex */
                X = (ex - 1) - 8;
                if (X < -110)
                    X = -110;
                if (X > 110)
                    X = 110;
            }
            x[r * (K / 32) + b] = X;
            for (int i = 0; i < 32; ++i)
                q[r * K + 32 * b + i] = orc_e4m3_encode(ldexp(bf16_value(v[i]), -X));
        }
    }
}

/* dequantised MXFP8 weights as bf16 bit patterns (exact; see above) */
void orc_dequant_mxfp8(const uint8_t* q, const int32_t* x, int64_t R, int K, uint16_t* w)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int k = 0; k < K; ++k)
            w[r * K + k] = orc_f64_to_bf16(
                ldexp(orc_e4m3_decode(q[r * K + k]), x[r * (K / 32) + k / 32]));
}

/* ------------------------------------------------------ fp4 expert weights -- */
/*
 * MXFP4 (the pages' "MxFP4", OCP Microscaling): blocks of 32 values along K
 * share one power-of-two scale, each value an OCP E2M1 float (1 sign bit, 2
 * exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6; no infinities or NaN).  Scale rule of the OCP specification:
 *   X = floor(log2(max |v| over the block)) - 2   (2 = E2M1's largest
 *       exponent), clamped here to [-110, 110] (0 for an all-zero block);
 *   q = E2M1(v / 2^X), round to nearest, ties to the even code (mantissa
 *       bit 0), magnitudes beyond 6 saturated to 6.
 * The dequantised value E2M1(q) * 2^X has at most 2 significant bits and a
 * normal bf16 exponent, so it is exactly a bf16 value.
 */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_decode(uint8_t c)
{
    return ((c & 8) ? -1.0 : 1.0) * e2m1_mag[c & 7];
}

/* nearest magnitude code, ties to the even code; |v| > 6 saturates */
uint8_t orc_e2m1_encode(double v)
{
    const uint8_t sign = signbit(v) ? 8 : 0;
    const double a = fmin(fabs(v), 6.0);          /* saturate first */
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        const double dc = fabs(a - e2m1_mag[c]), db = fabs(a - e2m1_mag[best]);
        if (dc < db || (dc == db && (c & 1) == 0))
            best = c;
    }
    return sign | (uint8_t)best;
}

/* MXFP4 quantisation of bf16 weights [R, K] (K multiple of 32): codes [R, K]
 * (one per byte, 0..15), block exponents X [R, K/32] */
void orc_quant_mxfp4(const uint16_t* w, int64_t R, int K, uint8_t* q, int32_t* x)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int b = 0; b < K / 32; ++b) {
            const uint16_t* v = w + r * K + 32 * b;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                const double a = fabs(bf16_value(v[i]));
                if (a > amax)
                    amax = a;
            }
            int X = 0;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);                 /* 2^(ex-1) <= amax < 2^ex */
                X = (ex - 1) - 2;
                if (X < -110)
                    X = -110;
                if (X > 110)
                    X = 110;
            }
            x[r * (K / 32) + b] = X;
            for (int i = 0; i < 32; ++i)
                q[r * K + 32 * b + i] = orc_e2m1_encode(ldexp(bf16_value(v[i]), -X));
        }
    }
}

/* dequantised MXFP4 weights as bf16 bit patterns (exact) */
void orc_dequant_mxfp4(const uint8_t* q, const int32_t* x, int64_t R, int K, uint16_t* w)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int k = 0; k < K; ++k)
            w[r * K + k] = orc_f64_to_bf16(
                ldexp(orc_e2m1_decode(q[r * K + k]), x[r * (K / 32) + k / 32]));
}
