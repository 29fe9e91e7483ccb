/*
 * pw_oracle.c -- plain fp64 CPU oracle for the fused mixed-precision MoE
 * expert path of PagedWeight.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only tests/, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * What is computed (PagedWeight pages: "Technical summary: PagedWeight",
 * "Core components" 1 and 3 -- per-expert linear blocks (layer, expert,
 * gate_up | down) held as Any-Precision bit-planes with per-row LUTs, each
 * block read at its own committed width q_i by one fused MoE operation;
 * "Problem statement" -- each token activates only a subset of experts).
 * The pages fix only this vocabulary.  The concrete definition used here:
 *
 *   route   : per token, the k experts with the largest logit, ordered by
 *             (logit descending, expert index ascending); gate weights are a
 *             softmax over those k logits, in fp64.
 *   permute : stable counting sort of assignments a = t*k + j by expert.
 *   decode  : parent code width p = 8; the q-bit child code is code8 >> (8-q)
 *             and the weight is LUT_q[row][child code].
 *   FFN     : g = W_gate x, u = W_up x (rows [0,I) and [I,2I) of gate_up),
 *             h = silu(g) * u, d = W_down h, y_t = sum_j w[t][j] d_(t,j)
 *             (+ the shared expert's d with weight 1 when present).
 * All sums run in fp64, in ascending index order, with no blocking or
 * reordering.  Build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    const uint8_t *code8; /* [R][K] parent codes                      */
    const double *lut;    /* [R][2^q] LUT_q of each row, widened fp16 */
    int32_t R, K, q;
} pwo_block;

/* q-bit child code of an 8-bit parent code. */
static inline int child_code(uint8_t code8, int q) { return (int)(code8 >> (8 - q)); }

/* decoded weight W(r, c) of a block at its committed width */
static inline double weight_at(const pwo_block *b, int64_t r, int64_t c)
{
    return b->lut[r * ((int64_t)1 << b->q) + child_code(b->code8[r * b->K + c], b->q)];
}

int pwo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void pwo_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* child codes of n parent codes at width q */
int pwo_decode_codes(const uint8_t *code8, int64_t n, int q, uint8_t *out)
{
    if (q < 1 || q > 8) return 1;
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)child_code(code8[i], q);
    return 0;
}

/* dense decoded weights W [R][K] of one block */
int pwo_decode_block(const pwo_block *b, double *W)
{
    if (b->q < 1 || b->q > 8) return 1;
    for (int64_t r = 0; r < b->R; ++r)
        for (int64_t c = 0; c < b->K; ++c) W[r * b->K + c] = weight_at(b, r, c);
    return 0;
}

/* top-k selection per token: (logit desc, index asc); softmax over the k */
int pwo_route_topk(const float *logits, int64_t T, int E, int k, int32_t *idx, double *w)
{
    if (k < 1 || k > E) return 1;
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        int32_t *sel = idx + t * k;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int jj = 0; jj < j; ++jj) taken |= (sel[jj] == e);
                if (taken) continue;
                if (best < 0 || l[e] > l[best]) best = e; /* ties keep the lower index */
            }
            sel[j] = best;
        }
        double m = (double)l[sel[0]];
        double z = 0.0;
        for (int j = 0; j < k; ++j) z += exp((double)l[sel[j]] - m);
        for (int j = 0; j < k; ++j) w[t * k + j] = exp((double)l[sel[j]] - m) / z;
    }
    return 0;
}

/* stable counting sort of assignments by expert */
int pwo_permute(const int32_t *idx, int64_t T, int k, int E, int32_t *offsets, int32_t *sorted)
{
    int64_t n = T * k;
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!fill) return 2;
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t a = 0; a < n; ++a) {
        if (idx[a] < 0 || idx[a] >= E) { free(fill); return 1; }
        offsets[idx[a] + 1] += 1;
    }
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int64_t a = 0; a < n; ++a) {
        int e = idx[a];
        sorted[offsets[e] + fill[e]] = (int32_t)a;
        fill[e] += 1;
    }
    free(fill);
    return 0;
}

/* d = W_down * (silu(W_gate x) * (W_up x)) for one expert and one token */
static void expert_ffn(const pwo_block *gu, const pwo_block *dn, int H, int I,
                       const double *x, double *h, double *d)
{
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) g += weight_at(gu, i, c) * x[c];
        for (int c = 0; c < H; ++c) u += weight_at(gu, (int64_t)I + i, c) * x[c];
        h[i] = g / (1.0 + exp(-g)) * u;
    }
    #pragma omp parallel for schedule(static)
    for (int o = 0; o < H; ++o) {
        double s = 0.0;
        for (int i = 0; i < I; ++i) s += weight_at(dn, o, i) * h[i];
        d[o] = s;
    }
}

static int check_block(const pwo_block *b, int R, int K)
{
    if (!b || !b->code8 || !b->lut) return 1;
    if (b->R != R || b->K != K || b->q < 1 || b->q > 8) return 1;
    return 0;
}

/*
 * y[n][H] for the tokens listed in `tokens` (n_tokens of them; NULL = all T),
 * given the routing (idx, w) of all T tokens.  gate_up/down hold E blocks;
 * sh_gate_up/sh_down may be NULL (no shared expert).
 */
int pwo_moe_layer(int64_t T, int H, int I, int E, int k, int I_shared,
                  const double *x, const int32_t *idx, const double *w,
                  const pwo_block *gate_up, const pwo_block *down,
                  const pwo_block *sh_gate_up, const pwo_block *sh_down,
                  const int32_t *tokens, int64_t n_tokens, double *y)
{
    int64_t nt = tokens ? n_tokens : T;
    int Imax = I > I_shared ? I : I_shared;
    double *h = (double *)malloc(sizeof(double) * (size_t)(Imax > 0 ? Imax : 1));
    double *d = (double *)malloc(sizeof(double) * (size_t)H);
    if (!h || !d) { free(h); free(d); return 2; }
    int rc = 0;
    for (int64_t n = 0; n < nt && !rc; ++n) {
        int64_t t = tokens ? tokens[n] : n;
        if (t < 0 || t >= T) { rc = 1; break; }
        double *yt = y + n * H;
        for (int o = 0; o < H; ++o) yt[o] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = idx[t * k + j];
            if (e < 0 || e >= E || check_block(&gate_up[e], 2 * I, H) ||
                check_block(&down[e], H, I)) { rc = 1; break; }
            expert_ffn(&gate_up[e], &down[e], H, I, x + t * H, h, d);
            double wj = w[t * k + j];
            for (int o = 0; o < H; ++o) yt[o] += wj * d[o];
        }
        if (!rc && I_shared > 0) {
            if (check_block(sh_gate_up, 2 * I_shared, H) || check_block(sh_down, H, I_shared)) {
                rc = 1;
                break;
            }
            expert_ffn(sh_gate_up, sh_down, H, I_shared, x + t * H, h, d);
            for (int o = 0; o < H; ++o) yt[o] += d[o];
        }
    }
    free(h);
    free(d);
    return rc;
}
