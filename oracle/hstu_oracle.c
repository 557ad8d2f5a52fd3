/*
 * hstu_oracle.c -- fp64 CPU oracle of the HSTU pointwise aggregated attention
 * path (attention core and its gradients, LayerNorm*U gate and its gradients,
 * layer with f1/f2, M-FALCON scores, and a brute-force enumeration of the
 * non-empty (query tile, key tile) set).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or helper with the HIP path.
 *
 * Everything is a plain loop in double precision, written from the
 * definitions, with no blocking, fusion or reordering:
 *   - "生成式推荐（一）：HSTU", section "高性能自注意力Encoder：HSTU": a layer is
 *     pointwise projection -> spatial aggregation -> pointwise transformation;
 *     f1 and f2 are single linear layers, phi1 = phi2 = SiLU, Norm = LayerNorm,
 *     rab^{p,t} combines position and time.
 *   - same page, section "Pointwise aggregated attention": the aggregated
 *     output enters the layer as Norm(A(X)V(X)) (.) U(X); weights are not
 *     normalised over the sequence (no softmax).
 *   - "Meta HSTU: как действия пользователя стали основой большой
 *     рекомендательной модели", section "Что меняется внутри HSTU по сравнению
 *     с обычным Transformer": Q, K, V and U are built together; aggregation
 *     uses relative position and time biases; the result is normalised, gated
 *     by U, transformed, and added through a residual.
 *   - "行动胜于言语：万亿参数序列转导器用于生成式推荐", section "7. 模型细节":
 *     normalised attention without softmax (a fixed 1/n scale, given here as
 *     alpha); section "2.3 M-FALCON算法" and the page "生成式推荐（一）：HSTU",
 *     section "M-FALCON": b_m candidates share one pass through a modified
 *     mask and bias.
 * Readings taken where the pages are silent are listed in the design notes
 * and repeated at each function below.
 *
 * Parallelism: OpenMP over independent (head, query row) pairs of a sequence,
 * and over rows in the row-wise functions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ACT_SILU 0
#define ORACLE_ACT_IDENTITY 1

/* ------------------------------------------------------------------------ */
/* Scalar definitions                                                        */
/* ------------------------------------------------------------------------ */

/* Number of significant bits of x (0 for x == 0). */
static int bit_length_u64(uint64_t x) {
    int n = 0;
    while (x != 0) {
        ++n;
        x >>= 1;
    }
    return n;
}

/* Time bucket of a pair: log2 buckets of the absolute time gap in seconds,
 * bucket = min(NT - 1, bit_length(|t_i - t_j|)).  Reading of "rab^{p,t}"
 * ("生成式推荐（一）：HSTU", symbol list of the layer equations). */
int32_t hstu_oracle_time_bucket(int64_t t_i, int64_t t_j, int32_t num_time_buckets) {
    uint64_t gap = (t_i >= t_j) ? (uint64_t)t_i - (uint64_t)t_j : (uint64_t)t_j - (uint64_t)t_i;
    int b = bit_length_u64(gap);
    return b < num_time_buckets - 1 ? b : num_time_buckets - 1;
}

/* Position of row i in a sequence with n_hist history rows: history rows keep
 * their index, every candidate row sits at position n_hist (just after the
 * history).  Reading of the M-FALCON bias change ("生成式推荐（一）：HSTU",
 * section "M-FALCON"): each candidate sees the history exactly as a single
 * appended target would. */
static int32_t position_of(int32_t i, int32_t n_hist) { return i < n_hist ? i : n_hist; }

/* Position bucket: min(p(i) - p(j), P - 1); p(i) >= p(j) for visible pairs. */
int32_t hstu_oracle_pos_bucket(int32_t i, int32_t j, int32_t n_hist, int32_t num_pos_buckets) {
    int32_t diff = position_of(i, n_hist) - position_of(j, n_hist);
    if (diff < 0) diff = 0; /* never reached for a visible pair */
    return diff < num_pos_buckets - 1 ? diff : num_pos_buckets - 1;
}

/* Visibility of key j from query i in a sequence of L rows whose first n_hist
 * rows are history (n_hist == L: plain causal sequence).
 *   history row i:   sees j <= i (causal: an event sees itself and the past);
 *   candidate row i: sees every history row and itself, no other candidate.
 */
int32_t hstu_oracle_visible(int32_t i, int32_t j, int32_t L, int32_t n_hist) {
    if (i < 0 || j < 0 || i >= L || j >= L) return 0;
    if (i < n_hist) return j <= i;
    return (j < n_hist) || (j == i);
}

/* SiLU(x) = x * sigmoid(x) = x / (1 + e^{-x}). */
double hstu_oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/* ------------------------------------------------------------------------ */
/* Jagged batch helpers                                                      */
/* ------------------------------------------------------------------------ */

static int32_t seq_len(const int32_t* offsets, const int32_t* lengths, int32_t b) {
    return lengths ? lengths[b] : offsets[b + 1] - offsets[b];
}

static int32_t seq_hist(const int32_t* offsets, const int32_t* lengths,
                        const int32_t* num_candidates, int32_t b) {
    int32_t L = seq_len(offsets, lengths, b);
    return num_candidates ? L - num_candidates[b] : L;
}

static void set_threads(int32_t num_threads) {
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
}

int32_t hstu_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Attention core                                                            */
/*   O[i, h, :] = alpha * sum_{j visible from i} act(S_ij) * V[j, h, :]       */
/*   S_ij = <Q[i, h, :], K[j, h, :]> + rab_pos[pb(i,j)] + rab_time[tb(i,j)]   */
/* Sums run over j ascending.  Row r of sequence b is offsets[b] + r.        */
/* Tables are per head when rab_head_stride > 0, shared when it is 0.        */
/* ------------------------------------------------------------------------ */
/* One output row of one head: acc = sum over visible j (ascending) of
 * act(S_ij) V[j], then O[i] = alpha * acc. */
static void attn_row(int32_t i, int32_t h, int32_t L, int32_t n_hist, int64_t base, int32_t d_qk,
                     int32_t d_v, const double* q, int64_t q_stride, const double* k, int64_t k_stride,
                     const double* v, int64_t v_stride, const int64_t* timestamps,
                     const double* rab_pos, int32_t num_pos_buckets, const double* rab_time,
                     int32_t num_time_buckets, int64_t rab_pos_head_stride,
                     int64_t rab_time_head_stride, double alpha, int32_t act, double* acc,
                     double* oi) {
    const double* rp = rab_pos + (int64_t)h * rab_pos_head_stride;
    const double* rt = rab_time + (int64_t)h * rab_time_head_stride;
    const double* qi = q + (base + i) * q_stride + (int64_t)h * d_qk;
    for (int32_t c = 0; c < d_v; ++c) acc[c] = 0.0;
    for (int32_t j = 0; j < L; ++j) {
        if (!hstu_oracle_visible(i, j, L, n_hist)) continue;
        const double* kj = k + (base + j) * k_stride + (int64_t)h * d_qk;
        double s = 0.0;
        for (int32_t c = 0; c < d_qk; ++c) s += qi[c] * kj[c];
        s += rp[hstu_oracle_pos_bucket(i, j, n_hist, num_pos_buckets)];
        s += rt[hstu_oracle_time_bucket(timestamps[base + i], timestamps[base + j], num_time_buckets)];
        double a = (act == ORACLE_ACT_IDENTITY) ? s : hstu_oracle_silu(s);
        const double* vj = v + (base + j) * v_stride + (int64_t)h * d_v;
        for (int32_t c = 0; c < d_v; ++c) acc[c] += a * vj[c];
    }
    for (int32_t c = 0; c < d_v; ++c) oi[c] = alpha * acc[c];
}

void hstu_oracle_attn(int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                      const int32_t* offsets, const int32_t* lengths,
                      const int32_t* num_candidates,
                      const double* q, int64_t q_stride,
                      const double* k, int64_t k_stride,
                      const double* v, int64_t v_stride,
                      const int64_t* timestamps,
                      const double* rab_pos, int32_t num_pos_buckets,
                      const double* rab_time, int32_t num_time_buckets,
                      int64_t rab_pos_head_stride, int64_t rab_time_head_stride,
                      double alpha, int32_t act,
                      double* o, int64_t o_stride, int32_t num_threads) {
    set_threads(num_threads);
    for (int32_t b = 0; b < B; ++b) {
        int32_t L = seq_len(offsets, lengths, b);
        int32_t n_hist = seq_hist(offsets, lengths, num_candidates, b);
        int64_t base = offsets[b];
        /* every (head, query row) of the sequence is independent */
#pragma omp parallel
        {
            double* acc = (double*)malloc(sizeof(double) * (size_t)(d_v > 0 ? d_v : 1));
#pragma omp for collapse(2) schedule(dynamic, 4)
            for (int32_t h = 0; h < H; ++h) {
                for (int32_t i = 0; i < L; ++i) {
                    attn_row(i, h, L, n_hist, base, d_qk, d_v, q, q_stride, k, k_stride, v, v_stride,
                             timestamps, rab_pos, num_pos_buckets, rab_time, num_time_buckets,
                             rab_pos_head_stride, rab_time_head_stride, alpha, act, acc,
                             o + (base + i) * o_stride + (int64_t)h * d_v);
                }
            }
            free(acc);
        }
    }
}

/* The same outputs for selected rows only: rows[r] is a row of the jagged
 * batch (offsets[b] <= rows[r] < offsets[b] + L_b); out[r, h, :] receives
 * its O for every head.  For checks of batches too large for the full
 * oracle: each row costs O(L d), not O(L^2 d). */
void hstu_oracle_attn_rows(int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                           const int32_t* offsets, const int32_t* lengths,
                           const int32_t* num_candidates,
                           const double* q, int64_t q_stride,
                           const double* k, int64_t k_stride,
                           const double* v, int64_t v_stride,
                           const int64_t* timestamps,
                           const double* rab_pos, int32_t num_pos_buckets,
                           const double* rab_time, int32_t num_time_buckets,
                           int64_t rab_pos_head_stride, int64_t rab_time_head_stride,
                           double alpha, int32_t act, int64_t nrows, const int64_t* rows,
                           double* out, int32_t num_threads) {
    set_threads(num_threads);
#pragma omp parallel
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)(d_v > 0 ? d_v : 1));
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            for (int32_t h = 0; h < H; ++h) {
                int32_t b = 0;
                while (b + 1 < B && offsets[b + 1] <= rows[r]) ++b;
                const int32_t L = seq_len(offsets, lengths, b);
                const int32_t n_hist = seq_hist(offsets, lengths, num_candidates, b);
                const int32_t i = (int32_t)(rows[r] - offsets[b]);
                attn_row(i, h, L, n_hist, offsets[b], d_qk, d_v, q, q_stride, k, k_stride, v, v_stride,
                         timestamps, rab_pos, num_pos_buckets, rab_time, num_time_buckets,
                         rab_pos_head_stride, rab_time_head_stride, alpha, act, acc,
                         out + (r * H + h) * d_v);
            }
        }
        free(acc);
    }
}

/* ------------------------------------------------------------------------ */
/* Pointwise transformation gate: Y = LayerNorm(o) (.) U per row.            */
/* LayerNorm over the row's `width` values (all heads concatenated), biased  */
/* variance, no affine parameters, eps added to the variance.                */
/* ------------------------------------------------------------------------ */
void hstu_oracle_ln_gate(int64_t rows, int32_t width,
                         const double* o, int64_t o_stride,
                         const double* u, int64_t u_stride,
                         double eps, double* y, int64_t y_stride, int32_t num_threads) {
    set_threads(num_threads);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double* orow = o + r * o_stride;
        const double* urow = u + r * u_stride;
        double* yrow = y + r * y_stride;
        double mean = 0.0;
        for (int32_t c = 0; c < width; ++c) mean += orow[c];
        mean /= (double)width;
        double var = 0.0;
        for (int32_t c = 0; c < width; ++c) var += (orow[c] - mean) * (orow[c] - mean);
        var /= (double)width;
        double inv = 1.0 / sqrt(var + eps);
        for (int32_t c = 0; c < width; ++c) yrow[c] = (orow[c] - mean) * inv * urow[c];
    }
}

/* ------------------------------------------------------------------------ */
/* Attention core, gradients.  With dO = dLoss/dO given, the chain rule      */
/* through O[i] = alpha * sum_j act(S_ij) V[j] gives, per visible pair:      */
/*   dV[j]           += alpha * act(S_ij) * dO[i]                            */
/*   G_ij             = alpha * <dO[i], V[j]> * act'(S_ij)   (= dLoss/dS_ij) */
/*   dQ[i]           += G_ij * K[j]          dK[j] += G_ij * Q[i]            */
/*   drab_pos[pb(i,j)] += G_ij             drab_time[tb(i,j)] += G_ij       */
/* act' of SiLU: sigma(x) (1 + x (1 - sigma(x))); of the identity: 1.         */
/* The S_ij, masks and buckets are those of the forward above ("生成式推荐   */
/* （一）：HSTU", sections "高性能自注意力Encoder：HSTU" and "Pointwise      */
/* aggregated attention").  Valid rows of dQ, dK, dV are overwritten          */
/* (padding rows untouched); the table gradients are overwritten: [P] / [NT]  */
/* summed over heads for shared tables, [H][P] / [H][NT] for per-head ones.   */
/* Loops run i ascending, then j ascending, within one (sequence, head).      */
/* ------------------------------------------------------------------------ */
static double act_value(double s, int32_t act) {
    return act == ORACLE_ACT_IDENTITY ? s : hstu_oracle_silu(s);
}

static double act_slope(double s, int32_t act) {
    if (act == ORACLE_ACT_IDENTITY) return 1.0;
    double sg = 1.0 / (1.0 + exp(-s));
    return sg * (1.0 + s * (1.0 - sg));
}

/* The chain rule at one visible pair (i, j) of head h: S_ij, A_ij =
 * act(S_ij), dov = <dO_i, V_j> and G_ij = alpha dov act'(S_ij). */
typedef struct {
    double a, g;
    int32_t pb, tb;
} bwd_pair_t;

static bwd_pair_t bwd_pair(int32_t i, int32_t j, int32_t h, int32_t n_hist, int64_t base, int32_t d_qk,
                           int32_t d_v, const double* q, const double* k, const double* v,
                           int64_t qk_stride, int64_t v_stride, const int64_t* timestamps,
                           const double* rab_pos, int32_t P, const double* rab_time, int32_t NT,
                           int64_t rab_pos_head_stride, int64_t rab_time_head_stride, double alpha,
                           int32_t act, const double* dout) {
    const double* rp = rab_pos + (int64_t)h * rab_pos_head_stride;
    const double* rt = rab_time + (int64_t)h * rab_time_head_stride;
    const double* qi = q + (base + i) * qk_stride + (int64_t)h * d_qk;
    const double* gi = dout + (base + i) * v_stride + (int64_t)h * d_v;
    const double* kj = k + (base + j) * qk_stride + (int64_t)h * d_qk;
    const double* vj = v + (base + j) * v_stride + (int64_t)h * d_v;
    bwd_pair_t r;
    r.pb = hstu_oracle_pos_bucket(i, j, n_hist, P);
    r.tb = hstu_oracle_time_bucket(timestamps[base + i], timestamps[base + j], NT);
    double s = rp[r.pb] + rt[r.tb];
    for (int32_t c = 0; c < d_qk; ++c) s += qi[c] * kj[c];
    r.a = act_value(s, act);
    double dov = 0.0;
    for (int32_t c = 0; c < d_v; ++c) dov += gi[c] * vj[c];
    r.g = alpha * dov * act_slope(s, act);
    return r;
}

void hstu_oracle_attn_bwd(int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                          const int32_t* offsets, const int32_t* lengths,
                          const int32_t* num_candidates,
                          const double* q, const double* k, const double* v,
                          int64_t qk_stride, int64_t v_stride,
                          const int64_t* timestamps,
                          const double* rab_pos, int32_t num_pos_buckets,
                          const double* rab_time, int32_t num_time_buckets,
                          int64_t rab_pos_head_stride, int64_t rab_time_head_stride,
                          double alpha, int32_t act, const double* dout,
                          double* dq, double* dk, double* dv,
                          double* drab_pos, double* drab_time, int32_t num_threads) {
    set_threads(num_threads);
    const int32_t P = num_pos_buckets, NT = num_time_buckets;
    /* per-head table gradients, summed over heads at the end when shared */
    double* gp = (double*)calloc((size_t)H * (size_t)P, sizeof(double));
    double* gt = (double*)calloc((size_t)H * (size_t)NT, sizeof(double));
    for (int32_t b = 0; b < B; ++b) {
        int32_t L = seq_len(offsets, lengths, b);
        int32_t n_hist = seq_hist(offsets, lengths, num_candidates, b);
        int64_t base = offsets[b];
        for (int32_t r = 0; r < L; ++r) {
            for (int32_t c = 0; c < H * d_qk; ++c) {
                dq[(base + r) * qk_stride + c] = 0.0;
                dk[(base + r) * qk_stride + c] = 0.0;
            }
            for (int32_t c = 0; c < H * d_v; ++c) dv[(base + r) * v_stride + c] = 0.0;
        }
        /* heads are independent: each writes its own columns and table row */
#pragma omp parallel for schedule(dynamic, 1)
        for (int32_t h = 0; h < H; ++h) {
            for (int32_t i = 0; i < L; ++i) {
                const double* qi = q + (base + i) * qk_stride + (int64_t)h * d_qk;
                const double* gi = dout + (base + i) * v_stride + (int64_t)h * d_v;
                double* dqi = dq + (base + i) * qk_stride + (int64_t)h * d_qk;
                for (int32_t j = 0; j < L; ++j) {
                    if (!hstu_oracle_visible(i, j, L, n_hist)) continue;
                    const bwd_pair_t pr = bwd_pair(i, j, h, n_hist, base, d_qk, d_v, q, k, v, qk_stride,
                                                   v_stride, timestamps, rab_pos, P, rab_time, NT,
                                                   rab_pos_head_stride, rab_time_head_stride, alpha, act,
                                                   dout);
                    const double* kj = k + (base + j) * qk_stride + (int64_t)h * d_qk;
                    double* dvj = dv + (base + j) * v_stride + (int64_t)h * d_v;
                    for (int32_t c = 0; c < d_v; ++c) dvj[c] += alpha * pr.a * gi[c];
                    double* dkj = dk + (base + j) * qk_stride + (int64_t)h * d_qk;
                    for (int32_t c = 0; c < d_qk; ++c) {
                        dqi[c] += pr.g * kj[c];
                        dkj[c] += pr.g * qi[c];
                    }
                    gp[(int64_t)h * P + pr.pb] += pr.g;
                    gt[(int64_t)h * NT + pr.tb] += pr.g;
                }
            }
        }
    }
    if (rab_pos_head_stride > 0) {
        for (int64_t e = 0; e < (int64_t)H * P; ++e) drab_pos[e] = gp[e];
    } else {
        for (int32_t e = 0; e < P; ++e) {
            double t = 0.0;
            for (int32_t h = 0; h < H; ++h) t += gp[(int64_t)h * P + e];
            drab_pos[e] = t;
        }
    }
    if (rab_time_head_stride > 0) {
        for (int64_t e = 0; e < (int64_t)H * NT; ++e) drab_time[e] = gt[e];
    } else {
        for (int32_t e = 0; e < NT; ++e) {
            double t = 0.0;
            for (int32_t h = 0; h < H; ++h) t += gt[(int64_t)h * NT + e];
            drab_time[e] = t;
        }
    }
    free(gp);
    free(gt);
}

/* The same dQ, dK and dV for selected rows only (no table gradients): the
 * query rows qrows[r] get dQ (sum over their visible keys, ascending), the
 * key rows krows[r] get dK and dV (sum over the rows that see them,
 * ascending) -- the full oracle's sums, in its order.  O(L d) per row. */
void hstu_oracle_attn_bwd_rows(int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                               const int32_t* offsets, const int32_t* lengths,
                               const int32_t* num_candidates,
                               const double* q, const double* k, const double* v,
                               int64_t qk_stride, int64_t v_stride,
                               const int64_t* timestamps,
                               const double* rab_pos, int32_t num_pos_buckets,
                               const double* rab_time, int32_t num_time_buckets,
                               int64_t rab_pos_head_stride, int64_t rab_time_head_stride,
                               double alpha, int32_t act, const double* dout,
                               int64_t nq, const int64_t* qrows, double* dq_out,
                               int64_t nk, const int64_t* krows, double* dk_out, double* dv_out,
                               int32_t num_threads) {
    set_threads(num_threads);
    const int32_t P = num_pos_buckets, NT = num_time_buckets;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t r = 0; r < nq + nk; ++r) {
        for (int32_t h = 0; h < H; ++h) {
            const int64_t row = r < nq ? qrows[r] : krows[r - nq];
            int32_t b = 0;
            while (b + 1 < B && offsets[b + 1] <= row) ++b;
            const int32_t L = seq_len(offsets, lengths, b);
            const int32_t n_hist = seq_hist(offsets, lengths, num_candidates, b);
            const int64_t base = offsets[b];
            const int32_t x = (int32_t)(row - base);
            if (r < nq) {
                double* acc = dq_out + (r * H + h) * d_qk;
                for (int32_t c = 0; c < d_qk; ++c) acc[c] = 0.0;
                for (int32_t j = 0; j < L; ++j) {
                    if (!hstu_oracle_visible(x, j, L, n_hist)) continue;
                    const bwd_pair_t pr = bwd_pair(x, j, h, n_hist, base, d_qk, d_v, q, k, v, qk_stride,
                                                   v_stride, timestamps, rab_pos, P, rab_time, NT,
                                                   rab_pos_head_stride, rab_time_head_stride, alpha, act,
                                                   dout);
                    const double* kj = k + (base + j) * qk_stride + (int64_t)h * d_qk;
                    for (int32_t c = 0; c < d_qk; ++c) acc[c] += pr.g * kj[c];
                }
            } else {
                double* dka = dk_out + ((r - nq) * H + h) * d_qk;
                double* dva = dv_out + ((r - nq) * H + h) * d_v;
                for (int32_t c = 0; c < d_qk; ++c) dka[c] = 0.0;
                for (int32_t c = 0; c < d_v; ++c) dva[c] = 0.0;
                for (int32_t i = 0; i < L; ++i) {
                    if (!hstu_oracle_visible(i, x, L, n_hist)) continue;
                    const bwd_pair_t pr = bwd_pair(i, x, h, n_hist, base, d_qk, d_v, q, k, v, qk_stride,
                                                   v_stride, timestamps, rab_pos, P, rab_time, NT,
                                                   rab_pos_head_stride, rab_time_head_stride, alpha, act,
                                                   dout);
                    const double* qi = q + (base + i) * qk_stride + (int64_t)h * d_qk;
                    const double* gi = dout + (base + i) * v_stride + (int64_t)h * d_v;
                    for (int32_t c = 0; c < d_v; ++c) dva[c] += alpha * pr.a * gi[c];
                    for (int32_t c = 0; c < d_qk; ++c) dka[c] += pr.g * qi[c];
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Gate gradients.  With y = xhat (.) u, xhat = (o - mean) / sqrt(var + eps) */
/* over the row and dY given:                                                */
/*   dU = xhat (.) dY;   g = dY (.) u;                                       */
/*   dO = (g - mean(g) - xhat * mean(g (.) xhat)) / sqrt(var + eps)          */
/* (the derivative of a LayerNorm without affine parameters, biased          */
/* variance, of the forward gate above).                                     */
/* ------------------------------------------------------------------------ */
void hstu_oracle_ln_gate_bwd(int64_t rows, int32_t width,
                             const double* o, int64_t o_stride,
                             const double* u, int64_t u_stride,
                             const double* dy, int64_t dy_stride, double eps,
                             double* dout, int64_t dout_stride,
                             double* du, int64_t du_stride, int32_t num_threads) {
    set_threads(num_threads);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double* orow = o + r * o_stride;
        const double* urow = u + r * u_stride;
        const double* dyrow = dy + r * dy_stride;
        double mean = 0.0;
        for (int32_t c = 0; c < width; ++c) mean += orow[c];
        mean /= (double)width;
        double var = 0.0;
        for (int32_t c = 0; c < width; ++c) var += (orow[c] - mean) * (orow[c] - mean);
        var /= (double)width;
        double inv = 1.0 / sqrt(var + eps);
        double mg = 0.0, mgx = 0.0;
        for (int32_t c = 0; c < width; ++c) {
            double xh = (orow[c] - mean) * inv;
            double g = dyrow[c] * urow[c];
            du[r * du_stride + c] = xh * dyrow[c];
            mg += g;
            mgx += g * xh;
        }
        mg /= (double)width;
        mgx /= (double)width;
        for (int32_t c = 0; c < width; ++c) {
            double xh = (orow[c] - mean) * inv;
            double g = dyrow[c] * urow[c];
            dout[r * dout_stride + c] = inv * (g - mg - xh * mgx);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Linear layer: out[t, n] = bias[n] + sum_k x[t, k] * w[n, k]  (w is out x in) */
/* ------------------------------------------------------------------------ */
static void linear(int64_t rows, int32_t n_out, int32_t n_in, const double* x, int64_t x_stride,
                   const double* w, const double* bias, double* out, int64_t out_stride) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < rows; ++t) {
        for (int32_t n = 0; n < n_out; ++n) {
            double s = bias ? bias[n] : 0.0;
            for (int32_t kk = 0; kk < n_in; ++kk) s += x[t * x_stride + kk] * w[(int64_t)n * n_in + kk];
            out[t * out_stride + n] = s;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* One HSTU layer over a packed jagged batch (rows offsets[0] .. offsets[B]). */
/*   Z = SiLU(X W1^T + b1), split by columns into U | V | Q | K (each H*d,    */
/*   head h at sub-columns h*d .. h*d+d-1);                                   */
/*   O = attention(Q, K, V);  Y = LayerNorm(O) (.) U;                         */
/*   X_out = X + Y W2^T + b2.                                                 */
/* ------------------------------------------------------------------------ */
void hstu_oracle_layer(int32_t B, int32_t H, int32_t d, int32_t D,
                       const int32_t* offsets, const int32_t* num_candidates,
                       const double* x, const double* w1, const double* b1,
                       const double* w2, const double* b2,
                       const int64_t* timestamps,
                       const double* rab_pos, int32_t num_pos_buckets,
                       const double* rab_time, int32_t num_time_buckets,
                       double alpha, double eps, double* x_out, int32_t num_threads) {
    set_threads(num_threads);
    int64_t row0 = offsets[0];
    int64_t T = (int64_t)offsets[B] - row0;
    int32_t hd = H * d;
    int32_t zw = 4 * hd;
    double* z = (double*)malloc(sizeof(double) * (size_t)(T * zw + 1));
    double* ob = (double*)malloc(sizeof(double) * (size_t)(T * hd + 1));
    double* yb = (double*)malloc(sizeof(double) * (size_t)(T * hd + 1));
    /* offsets rebased to the start of the packed buffers */
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B + 1));
    for (int32_t b = 0; b <= B; ++b) off[b] = (int32_t)(offsets[b] - row0);

    linear(T, zw, D, x + row0 * D, D, w1, b1, z, zw);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < T * zw; ++e) z[e] = hstu_oracle_silu(z[e]);

    const double* U = z + 0 * hd;
    const double* V = z + 1 * hd;
    const double* Q = z + 2 * hd;
    const double* K = z + 3 * hd;
    hstu_oracle_attn(B, H, d, d, off, NULL, num_candidates, Q, zw, K, zw, V, zw,
                     timestamps + row0, rab_pos, num_pos_buckets, rab_time, num_time_buckets,
                     0, 0, alpha, ORACLE_ACT_SILU, ob, hd, num_threads);
    hstu_oracle_ln_gate(T, hd, ob, hd, U, zw, eps, yb, hd, num_threads);
    linear(T, D, hd, yb, hd, w2, b2, x_out + row0 * D, D);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int32_t m = 0; m < D; ++m) x_out[(row0 + t) * D + m] += x[(row0 + t) * D + m];
    free(off);
    free(yb);
    free(ob);
    free(z);
}

/* ------------------------------------------------------------------------ */
/* Layer gradients: with dX_out = dLoss/dX_out given, the chain rule through */
/* the layer above, in reverse:                                               */
/*   f2:   dY = dX_out W2;  dW2 = dX_out^T Y;  db2 = sum_t dX_out             */
/*   gate and attention: dO, dU, then dQ, dK, dV and the table gradients     */
/*         (hstu_oracle_ln_gate_bwd, hstu_oracle_attn_bwd)                     */
/*   f1:   dP = dZ (.) SiLU'(P) with P = X W1^T + b1 and dZ = dU | dV | dQ | dK */
/*         dX = dX_out + dP W1;  dW1 = dP^T X;  db1 = sum_t dP               */
/* (the residual passes dX_out straight through).  Shared tables.  Sums over */
/* tokens run in row order.                                                   */
/* ------------------------------------------------------------------------ */
void hstu_oracle_layer_bwd(int32_t B, int32_t H, int32_t d, int32_t D,
                           const int32_t* offsets, const int32_t* num_candidates,
                           const double* x, const double* w1, const double* b1,
                           const double* w2, const double* b2,
                           const int64_t* timestamps,
                           const double* rab_pos, int32_t num_pos_buckets,
                           const double* rab_time, int32_t num_time_buckets,
                           double alpha, double eps, const double* dx_out,
                           double* dx, double* dw1, double* db1, double* dw2, double* db2,
                           double* drab_pos, double* drab_time, int32_t num_threads) {
    set_threads(num_threads);
    (void)b2;
    int64_t row0 = offsets[0];
    int64_t T = (int64_t)offsets[B] - row0;
    int32_t hd = H * d;
    int32_t zw = 4 * hd;
    size_t tz = (size_t)(T * zw + 1), th = (size_t)(T * hd + 1);
    double* pre = (double*)malloc(sizeof(double) * tz);
    double* z = (double*)malloc(sizeof(double) * tz);
    double* dz = (double*)calloc(tz, sizeof(double));
    double* gz = (double*)calloc(tz, sizeof(double));   /* dO at the V columns' stride */
    double* ob = (double*)malloc(sizeof(double) * th);
    double* yb = (double*)malloc(sizeof(double) * th);
    double* dy = (double*)malloc(sizeof(double) * th);
    double* dob = (double*)malloc(sizeof(double) * th);
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B + 1));
    for (int32_t b = 0; b <= B; ++b) off[b] = (int32_t)(offsets[b] - row0);
    const double* xr = x + row0 * D;
    const double* gr = dx_out + row0 * D;

    /* forward intermediates */
    linear(T, zw, D, xr, D, w1, b1, pre, zw);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < T * zw; ++e) z[e] = hstu_oracle_silu(pre[e]);
    hstu_oracle_attn(B, H, d, d, off, NULL, num_candidates, z + 2 * hd, zw, z + 3 * hd, zw, z + hd, zw,
                     timestamps + row0, rab_pos, num_pos_buckets, rab_time, num_time_buckets,
                     0, 0, alpha, ORACLE_ACT_SILU, ob, hd, num_threads);
    hstu_oracle_ln_gate(T, hd, ob, hd, z, zw, eps, yb, hd, num_threads);

    /* f2 (each sum accumulates its terms in index order: m for dY, t for
       dW2 and db2; the loops are ordered for contiguous reads) */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* dyr = dy + t * hd;
        for (int32_t h = 0; h < hd; ++h) dyr[h] = 0.0;
        for (int32_t m = 0; m < D; ++m) {
            const double a = gr[t * D + m];
            const double* w2r = w2 + (int64_t)m * hd;
            for (int32_t h = 0; h < hd; ++h) dyr[h] += a * w2r[h];
        }
    }
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < D; ++m) {
        double* dw2r = dw2 + (int64_t)m * hd;
        for (int32_t h = 0; h < hd; ++h) dw2r[h] = 0.0;
        double sb = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double a = gr[t * D + m];
            const double* yr = yb + t * hd;
            for (int32_t h = 0; h < hd; ++h) dw2r[h] += a * yr[h];
            sb += a;
        }
        if (db2) db2[m] = sb;
    }

    /* gate (dU into dZ's U columns) and attention (dV, dQ, dK into theirs) */
    hstu_oracle_ln_gate_bwd(T, hd, ob, hd, z, zw, dy, hd, eps, dob, hd, dz, zw, num_threads);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < hd; ++h) gz[t * zw + h] = dob[t * hd + h];
    hstu_oracle_attn_bwd(B, H, d, d, off, NULL, num_candidates, z + 2 * hd, z + 3 * hd, z + hd, zw, zw,
                         timestamps + row0, rab_pos, num_pos_buckets, rab_time, num_time_buckets, 0, 0,
                         alpha, ORACLE_ACT_SILU, gz, dz + 2 * hd, dz + 3 * hd, dz + hd, drab_pos, drab_time,
                         num_threads);

    /* f1 + SiLU */
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < T * zw; ++e) {
        double sg = 1.0 / (1.0 + exp(-pre[e]));
        dz[e] *= sg * (1.0 + pre[e] * (1.0 - sg));
    }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* dxr = dx + (row0 + t) * D;
        for (int32_t k = 0; k < D; ++k) dxr[k] = gr[t * D + k];
        for (int32_t n = 0; n < zw; ++n) {
            const double a = dz[t * zw + n];
            const double* w1r = w1 + (int64_t)n * D;
            for (int32_t k = 0; k < D; ++k) dxr[k] += a * w1r[k];
        }
    }
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < zw; ++n) {
        double* dw1r = dw1 + (int64_t)n * D;
        for (int32_t k = 0; k < D; ++k) dw1r[k] = 0.0;
        double sb = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double a = dz[t * zw + n];
            const double* xrow = xr + t * D;
            for (int32_t k = 0; k < D; ++k) dw1r[k] += a * xrow[k];
            sb += a;
        }
        if (db1) db1[n] = sb;
    }
    free(off); free(dob); free(dy); free(yb); free(ob); free(gz); free(dz); free(z); free(pre);
}

/* ------------------------------------------------------------------------ */
/* M-FALCON ranking scores: for candidate c of sequence b,                    */
/*   s[b, c] = < Y[n_b + c, :], w >,  Y = LayerNorm(O) (.) U over H*d_v.       */
/* The attention output is computed for all rows in one pass (history rows   */
/* causal, candidates see the history and themselves).                        */
/* ------------------------------------------------------------------------ */
void hstu_oracle_mfalcon_score(int32_t B, int32_t H, int32_t d,
                               const int32_t* offsets, const int32_t* num_candidates,
                               const double* q, const double* k, const double* v,
                               const double* u, int64_t stride,
                               const int64_t* timestamps,
                               const double* rab_pos, int32_t num_pos_buckets,
                               const double* rab_time, int32_t num_time_buckets,
                               double alpha, double eps, const double* w,
                               double* scores, int32_t score_stride, int32_t num_threads) {
    set_threads(num_threads);
    int64_t T = offsets[B];
    int32_t hd = H * d;
    double* ob = (double*)malloc(sizeof(double) * (size_t)(T * hd + 1));
    double* yrow = (double*)malloc(sizeof(double) * (size_t)hd);
    hstu_oracle_attn(B, H, d, d, offsets, NULL, num_candidates, q, stride, k, stride, v, stride,
                     timestamps, rab_pos, num_pos_buckets, rab_time, num_time_buckets, 0, 0,
                     alpha, ORACLE_ACT_SILU, ob, hd, num_threads);
    for (int32_t b = 0; b < B; ++b) {
        int32_t L = offsets[b + 1] - offsets[b];
        int32_t c_b = num_candidates[b];
        int32_t n_b = L - c_b;
        for (int32_t c = 0; c < c_b; ++c) {
            int64_t row = (int64_t)offsets[b] + n_b + c;
            hstu_oracle_ln_gate(1, hd, ob + row * hd, hd, u + row * stride, stride, eps, yrow, hd, 1);
            double s = 0.0;
            for (int32_t m = 0; m < hd; ++m) s += yrow[m] * w[m];
            scores[(int64_t)b * score_stride + c] = s;
        }
    }
    free(yrow);
    free(ob);
}

/* ------------------------------------------------------------------------ */
/* The last layer of an M-FALCON stack, scores only: Z = SiLU(X W1^T + b1)   */
/* split into U | V | Q | K as in hstu_oracle_layer, then the M-FALCON       */
/* scores of that attention ("生成式推荐（一）：HSTU", section "M-FALCON").    */
/* ------------------------------------------------------------------------ */
void hstu_oracle_layer_scores(int32_t B, int32_t H, int32_t d, int32_t D,
                              const int32_t* offsets, const int32_t* num_candidates,
                              const double* x, const double* w1, const double* b1,
                              const int64_t* timestamps,
                              const double* rab_pos, int32_t num_pos_buckets,
                              const double* rab_time, int32_t num_time_buckets,
                              double alpha, double eps, const double* w,
                              double* scores, int32_t score_stride, int32_t num_threads) {
    set_threads(num_threads);
    int64_t row0 = offsets[0];
    int64_t T = (int64_t)offsets[B] - row0;
    int32_t hd = H * d;
    int32_t zw = 4 * hd;
    double* z = (double*)malloc(sizeof(double) * (size_t)(T * zw + 1));
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B + 1));
    for (int32_t b = 0; b <= B; ++b) off[b] = (int32_t)(offsets[b] - row0);
    linear(T, zw, D, x + row0 * D, D, w1, b1, z, zw);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < T * zw; ++e) z[e] = hstu_oracle_silu(z[e]);
    hstu_oracle_mfalcon_score(B, H, d, off, num_candidates, z + 2 * hd, z + 3 * hd, z + 1 * hd, z, zw,
                              timestamps + row0, rab_pos, num_pos_buckets, rab_time, num_time_buckets,
                              alpha, eps, w, scores, score_stride, num_threads);
    free(off);
    free(z);
}

/* ------------------------------------------------------------------------ */
/* Brute-force set of non-empty tiles: (b, query tile, key tile) such that   */
/* some visible pair (i, j) has i / tile_m == query tile and j / tile_n ==    */
/* key tile.  Written in ascending (b, qt, kt) order; returns the count.     */
/* ------------------------------------------------------------------------ */
int64_t hstu_oracle_tiles(int32_t B, const int32_t* offsets, const int32_t* lengths,
                          const int32_t* num_candidates, int32_t tile_m, int32_t tile_n,
                          int32_t* out, int64_t cap) {
    int64_t count = 0;
    for (int32_t b = 0; b < B; ++b) {
        int32_t L = seq_len(offsets, lengths, b);
        int32_t n_hist = seq_hist(offsets, lengths, num_candidates, b);
        int32_t nq = (L + tile_m - 1) / tile_m;
        int32_t nk = (L + tile_n - 1) / tile_n;
        unsigned char* mark = (unsigned char*)calloc((size_t)nq * nk + 1, 1);
        for (int32_t i = 0; i < L; ++i)
            for (int32_t j = 0; j < L; ++j)
                if (hstu_oracle_visible(i, j, L, n_hist)) mark[(i / tile_m) * nk + (j / tile_n)] = 1;
        for (int32_t qt = 0; qt < nq; ++qt)
            for (int32_t kt = 0; kt < nk; ++kt)
                if (mark[qt * nk + kt]) {
                    if (count < cap) {
                        out[3 * count + 0] = b;
                        out[3 * count + 1] = qt;
                        out[3 * count + 2] = kt;
                    }
                    ++count;
                }
        free(mark);
    }
    return count;
}

/* Number of visible (i, j) pairs over the batch, by enumeration. */
int64_t hstu_oracle_count_visible(int32_t B, const int32_t* offsets, const int32_t* lengths,
                                  const int32_t* num_candidates) {
    int64_t count = 0;
    for (int32_t b = 0; b < B; ++b) {
        int32_t L = seq_len(offsets, lengths, b);
        int32_t n_hist = seq_hist(offsets, lengths, num_candidates, b);
        for (int32_t i = 0; i < L; ++i)
            for (int32_t j = 0; j < L; ++j) count += hstu_oracle_visible(i, j, L, n_hist);
    }
    return count;
}
