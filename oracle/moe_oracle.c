/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle of the
 * single-GPU Mixture-of-Experts forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library: it is written from the
 * definitions below and nothing else.
 *
 * Source of the definitions.  [R] is the Pith review page of
 * "Cross-Platform Fused MoE Dispatch in Triton: Portable Expert Routing
 * Without CUDA" (arXiv 2605.23911), which also carries the paper's abstract.
 *   - [R] "The reading": the path scores tokens, reorders them onto experts,
 *     runs variable-size per-expert GEMMs and scatters results back with the
 *     routing weights.
 *   - [R] "Assumptions & free parameters" (paper section 2.1, Eq. (1)-(4)):
 *     the standard softmax/sigmoid router, top-k selection and SwiGLU expert
 *     FFN; the equations are named there but not printed, so the standard
 *     forms are written out here.
 *   - [R] "What carries the argument" and "Referee Report" (Algorithm 1):
 *     fixed-size blocks of rows mapped to (expert, token-offset) pairs.
 *   - [R] abstract: router scoring, token permutation, expert GEMMs and a
 *     weighted output combination.
 * Where the page leaves a step open, the plainest reading is taken; each
 * such reading is marked "Reading:" below.
 *
 * Precision: fp32 arithmetic with fp32 accumulation in ascending index
 * order, libm expf, one token at a time.  bf16 inputs are widened exactly
 * (bits << 16).  Build with -O2 -ffp-contract=off and no fast-math so the
 * stated summation order is the one executed.
 *
 * Parity pins: every function here is checked by tests that do not call
 * it twice -- numpy float64 dense brute force, numpy/scipy closed forms,
 * invariants and special cases that reduce to a textbook SwiGLU MLP.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_ENOMEM (-2)  /* a working buffer could not be allocated */

enum { ORC_SCORE_SOFTMAX = 0, ORC_SCORE_SIGMOID = 1 };

/* Exact widening of a bf16 bit pattern to fp32. */
static float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest-even fp32 -> bf16, NaN kept NaN (quiet bit set). */
static uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

int orc_abi_version(void) { return 1; }

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the following parallel regions (OpenMP over tokens only: the
 * results do not depend on it). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* "a ranks before b" for the top-k order of one token's logits.
 * Reading: the selection key is the raw fp32 logit (softmax and sigmoid are
 * strictly increasing, so the selected set is the same in exact arithmetic);
 * equal logits (IEEE equality, so -0 == +0) rank the lower expert first. */
static int orc_ranks_before(const float *l, int a, int b)
{
    if (l[a] > l[b]) return 1;
    if (l[a] == l[b] && a < b) return 1;
    return 0;
}

/* O1 -- top-k selection ([R] "The reading": tokens are scored; [R] paper
 * Eq. (1)-(4): top-k of the router scores).  ids[t*k + j] is the j-th expert
 * of token t in descending logit order, ties to the lower index.  Plain k
 * passes of selection over the E experts. */
int orc_select_topk(const float *logits, int T, int E, int k, int32_t *ids)
{
    if (!logits || !ids || T < 0 || E < 1 || k < 1 || k > E) return ORC_EARG;
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int i = 0; i < j; ++i)
                    if (ids[(size_t)t * k + i] == e) taken = 1;
                if (taken) continue;
                if (best < 0 || orc_ranks_before(l, e, best)) best = e;
            }
            ids[(size_t)t * k + j] = best;
        }
    }
    return ORC_OK;
}

/* O2 -- routing weights of the selected experts ([R] "Assumptions & free
 * parameters": softmax or sigmoid router, Eq. (1)-(4)).
 *   softmax, renormalize=1: softmax over the k selected logits,
 *       m = l[ids0] (the largest), w_j = exp(l_j - m) / sum_{i<k} exp(l_i - m).
 *   softmax, renormalize=0: softmax over all E logits, then take the k
 *       selected entries: w_j = exp(l_j - m) / sum_{e<E} exp(l_e - m).
 *   sigmoid: s_j = 1 / (1 + exp(-l_j)); renormalize=1 divides by sum_i s_i.
 * Sums run in ascending j (or e) order in fp32. */
int orc_weights(const float *logits, const int32_t *ids, int T, int E, int k,
                int score, int renormalize, float *w)
{
    if (!logits || !ids || !w || T < 0 || E < 1 || k < 1 || k > E) return ORC_EARG;
    if (score != ORC_SCORE_SOFTMAX && score != ORC_SCORE_SIGMOID) return ORC_EARG;
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        const int32_t *id = ids + (size_t)t * k;
        float *wt = w + (size_t)t * k;
        if (score == ORC_SCORE_SOFTMAX) {
            float m = l[id[0]];
            float z = 0.0f;
            if (renormalize) {
                for (int j = 0; j < k; ++j) z += expf(l[id[j]] - m);
            } else {
                for (int e = 0; e < E; ++e) z += expf(l[e] - m);
            }
            for (int j = 0; j < k; ++j) wt[j] = expf(l[id[j]] - m) / z;
        } else {
            float s = 0.0f;
            for (int j = 0; j < k; ++j) {
                wt[j] = 1.0f / (1.0f + expf(-l[id[j]]));
                s += wt[j];
            }
            if (renormalize)
                for (int j = 0; j < k; ++j) wt[j] = wt[j] / s;
        }
    }
    return ORC_OK;
}

/* O3 -- per-expert row counts and their exclusive prefix sum ([R] "The
 * reading": variable-size per-expert GEMMs need each expert's row count;
 * the token-offset of "What carries the argument" is a running sum of them).
 * offsets has E+1 entries, offsets[E] = A. */
int orc_counts_offsets(const int32_t *ids, int A, int E, int32_t *counts, int32_t *offsets)
{
    if (!ids || !counts || !offsets || A < 0 || E < 1) return ORC_EARG;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int i = 0; i < A; ++i) {
        if (ids[i] < 0 || ids[i] >= E) return ORC_EARG;
        counts[ids[i]] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    return ORC_OK;
}

/* O4 -- the reordering onto experts ([R] "The reading"; abstract: token
 * permutation).  Flat row i = t*k + j goes to sorted row p; perm[p] = i and
 * inv[i] = p.  Reading: rows of one expert keep ascending i (a stable
 * counting sort), which makes the permutation unique. */
int orc_permute(const int32_t *ids, int A, int E, const int32_t *offsets,
                int32_t *perm, int32_t *inv)
{
    if (!ids || !offsets || !perm || !inv || A < 0 || E < 1) return ORC_EARG;
    int32_t cursor[E];
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int i = 0; i < A; ++i) {
        int p = cursor[ids[i]]++;
        perm[p] = i;
        inv[i] = p;
    }
    return ORC_OK;
}

/* O5 -- the block schedule ([R] "What carries the argument": fixed-size
 * program blocks mapped onto (expert, token-offset) pairs; "Assumptions &
 * free parameters": BLOCK_M fixed for one launch).  Reading: the
 * token-offset is the absolute first sorted row of the block; blocks never
 * span two experts; an expert with no rows has no block.  For e ascending,
 * for r = 0, BM, 2BM, ... < counts[e]: emit (e, offsets[e] + r). */
int orc_block_table(const int32_t *counts, const int32_t *offsets, int E, int BM,
                    int32_t *blocks, int max_blocks, int32_t *nb)
{
    if (!counts || !offsets || !blocks || !nb || E < 1 || BM < 1) return ORC_EARG;
    int n = 0;
    for (int e = 0; e < E; ++e) {
        for (int r = 0; r < counts[e]; r += BM) {
            if (n >= max_blocks) return ORC_EARG;
            blocks[2 * n] = e;
            blocks[2 * n + 1] = offsets[e] + r;
            ++n;
        }
    }
    *nb = n;
    return ORC_OK;
}

/* O5b -- a launch order of the blocks.  The pages fix no order in which the
 * blocks are run ([R] "Assumptions & free parameters": BLOCK_M is fixed and
 * load imbalance under skew is the stated weakness).  Reading: longest
 * first -- the block indices sorted by decreasing row count
 * (min(BM, end of the expert's rows - first row)), equal counts in
 * ascending block index.  A plain stable insertion sort. */
int orc_block_order(const int32_t *blocks, int nb, const int32_t *offsets, int BM,
                    int32_t *order)
{
    if ((nb > 0 && (!blocks || !offsets || !order)) || nb < 0 || BM < 1) return ORC_EARG;
    int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
    if (!rows) return ORC_EARG;
    for (int b = 0; b < nb; ++b) {
        const int e = blocks[2 * b], first = blocks[2 * b + 1];
        const int left = offsets[e + 1] - first;
        rows[b] = left < BM ? left : BM;
        order[b] = b;
    }
    for (int i = 1; i < nb; ++i) {
        const int key = order[i];
        int j = i - 1;
        while (j >= 0 && rows[order[j]] < rows[key]) {
            order[j + 1] = order[j];
            --j;
        }
        order[j + 1] = key;
    }
    free(rows);
    return ORC_OK;
}

/* O5c -- a block table with a variable block size per expert for the
 * gate/up GEMM.  The pages leave the assignment of blocks to experts under
 * skew as future work ([R] abstract: dynamic block-to-expert assignment;
 * "Editorial extensions"); this is the library's reading of it, written
 * out plainly.  With `tiles` column tiles per block and a round of `round`
 * workgroups: the fixed cutting has F = sum_e ceil(counts[e] / BM) blocks;
 * the merged cutting gives an expert with more than BM rows blocks of 2 BM
 * rows (the last holding the rest) and the others blocks of BM rows, M
 * blocks in all.  mode 2 always merges; mode 1 merges when F * tiles >
 * round and M * tiles <= round.  Merged: vb[3 n] = (e, offsets[e] + r,
 * min(size, counts[e] - r)) for e ascending, r = 0, size, 2 size, ... and
 * *vnb = M; not merged: *vnb = -1 and vb is not written. */
int orc_var_block_table(const int32_t *counts, const int32_t *offsets, int E, int BM, int tiles,
                        int mode, int round, int32_t *vb, int max_blocks, int32_t *vnb)
{
    if (!counts || !offsets || !vnb || E < 1 || BM < 1 || tiles < 1 || round < 1 ||
        (mode != 1 && mode != 2))
        return ORC_EARG;
    long long fixed = 0, merged = 0;
    for (int e = 0; e < E; ++e) {
        fixed += (counts[e] + BM - 1) / BM;
        const int size = counts[e] > BM ? 2 * BM : BM;
        merged += (counts[e] + size - 1) / size;
    }
    const int merge = mode == 2 || (fixed * tiles > round && merged * tiles <= round);
    if (!merge) {
        *vnb = -1;
        return ORC_OK;
    }
    if (!vb) return ORC_EARG;
    int n = 0;
    for (int e = 0; e < E; ++e) {
        const int size = counts[e] > BM ? 2 * BM : BM;
        for (int r = 0; r < counts[e]; r += size) {
            if (n >= max_blocks) return ORC_EARG;
            vb[3 * n] = e;
            vb[3 * n + 1] = offsets[e] + r;
            vb[3 * n + 2] = counts[e] - r < size ? counts[e] - r : size;
            ++n;
        }
    }
    *vnb = n;
    return ORC_OK;
}

/* O6 -- per-token expert FFN and weighted combination ([R] "What carries the
 * argument": SwiGLU with a gate and an up projection; abstract: expert GEMMs
 * and weighted output combination; Eq. (1)-(4)).  For token t:
 *     out[t] = sum_j w[t,j] * Wd[e_j] (silu(Wg[e_j] x_t) * (Wu[e_j] x_t)),
 * silu(z) = z / (1 + exp(-z)).
 * Reading: W_gate_up[e] holds the gate rows [0, F) and then the up rows
 * [F, 2F), each row d long; W_down[e] is [d, F].  The routing weight is
 * applied after the down projection, at the combination.
 *
 * The weights are passed per expert (wgu[e] -> [2F, d], wd[e] -> [d, F]) so
 * a caller can hand over only the experts the chosen tokens use; an expert
 * that a chosen token routes to must not be NULL.  Only the ntok tokens
 * listed in `tokens` are evaluated; out32 is [ntok, d]. */
int orc_ffn_tokens(const uint16_t *x, const int32_t *ids, const float *w,
                   const uint16_t *const *wgu, const uint16_t *const *wd,
                   int T, int d, int F, int E, int k,
                   const int32_t *tokens, int ntok, float *out32)
{
    if (!x || !ids || !w || !wgu || !wd || !tokens || !out32) return ORC_EARG;
    if (T < 0 || d < 1 || F < 1 || E < 1 || k < 1 || k > E || ntok < 0) return ORC_EARG;
    for (int s = 0; s < ntok; ++s) {
        int t = tokens[s];
        if (t < 0 || t >= T) return ORC_EARG;
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            if (e < 0 || e >= E || !wgu[e] || !wd[e]) return ORC_EARG;
        }
    }
    int bad = 0, oom = 0;
    /* per-thread working rows (x_t, the accumulator, h) on the heap: d and F
     * can be large enough to overflow a worker thread's stack */
#pragma omp parallel reduction(| : bad, oom)
    {
    float *buf = (float *)malloc(sizeof(float) * ((size_t)2 * d + (size_t)F));
    if (!buf) oom = 1;
#pragma omp for schedule(static)
    for (int s = 0; s < ntok; ++s) {
        if (!buf) continue;
        int t = tokens[s];
        float *xt = buf;
        float *acc = buf + d;
        float *h = buf + (size_t)2 * d;
        for (int c = 0; c < d; ++c) xt[c] = orc_bf16_to_f32(x[(size_t)t * d + c]);
        for (int o = 0; o < d; ++o) acc[o] = 0.0f;
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            const uint16_t *wg = wgu[e];
            const uint16_t *wu = wgu[e] + (size_t)F * d;
            const uint16_t *wdn = wd[e];
            for (int f = 0; f < F; ++f) {
                float g = 0.0f, u = 0.0f;
                for (int c = 0; c < d; ++c) {
                    g += orc_bf16_to_f32(wg[(size_t)f * d + c]) * xt[c];
                    u += orc_bf16_to_f32(wu[(size_t)f * d + c]) * xt[c];
                }
                h[f] = (g / (1.0f + expf(-g))) * u;
            }
            float wj = w[(size_t)t * k + j];
            for (int o = 0; o < d; ++o) {
                float y = 0.0f;
                for (int f = 0; f < F; ++f)
                    y += orc_bf16_to_f32(wdn[(size_t)o * F + f]) * h[f];
                acc[o] += wj * y;
            }
        }
        for (int o = 0; o < d; ++o) {
            out32[(size_t)s * d + o] = acc[o];
            if (!isfinite(acc[o])) bad |= 1;
        }
    }
    free(buf);
    }
    (void)bad; /* non-finite values are returned as computed */
    return oom ? ORC_ENOMEM : ORC_OK;
}

/* O0 -- router scores ([R] "The reading": tokens are scored before they are
 * routed; "Assumptions & free parameters", Eq. (1)-(4): the standard router,
 * a linear map of the token's hidden state to one score per expert):
 *   logits[t][e] = sum_c x[t][c] * W_r[e][c].
 * Reading: W_r is [E, d] with each expert's row contiguous, like the expert
 * weights; x and W_r are bf16.  The precision is not fixed by the page:
 * here the products are summed in fp64 in ascending c and the sum is
 * rounded once to fp32, i.e. the exact dot product to within d * 2^-53 of
 * sum_c |x[t][c] * W_r[e][c]| before that one rounding. */
int orc_router_logits(const uint16_t *x, const uint16_t *wr, int T, int d, int E, float *logits)
{
    if ((!x || !wr || !logits) && T > 0) return ORC_EARG;
    if (T < 0 || d < 1 || E < 1) return ORC_EARG;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int c = 0; c < d; ++c)
                s += (double)orc_bf16_to_f32(x[(size_t)t * d + c]) *
                     (double)orc_bf16_to_f32(wr[(size_t)e * d + c]);
            logits[(size_t)t * E + e] = (float)s;
        }
    }
    return ORC_OK;
}

/* O7 -- the bf16 output: round-to-nearest-even of the fp32 result. */
int orc_round_bf16(const float *in, uint16_t *out, long n)
{
    if ((!in || !out) && n > 0) return ORC_EARG;
    for (long i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
    return ORC_OK;
}
