/*
 * orc.c - the parity oracle: exact causal (or full) grouped-query softmax
 * attention, forward and backward, written out from its definition in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library and never calls it.
 *
 * What it computes, and where the pages state it:
 *   - A query token attends to the key/value tokens that precede it or sit at
 *     the same position (FPDT talk summary, "Technical Deep Dive", the
 *     paragraph on the auto-regressive nature of LLMs).  That is the causal
 *     set J(i) = {0..i}; non-causal uses J(i) = {0..S-1}.
 *   - Attention is exact softmax attention whose pairwise query/key
 *     interactions give the quadratic cost (Road to 5 Million Tokens summary,
 *     "Main Topics and Challenges"); stable softmax keeps the maximum logit as
 *     a statistic (FPDT summary, "Technical Deep Dive").
 *   - Partial outputs over key trunks are combined by updating those softmax
 *     statistics until every trunk of the current query trunk is done (same
 *     section).  orc_attn_fwd_trunked follows that order: query trunk outer,
 *     key trunks 0..m inner, merge by log-sum-exp.
 *   - Heads are walked a chunk at a time through one reused buffer set (Road
 *     to 5 Million Tokens talk, the U-Pipe paragraph): orc_attn_fwd_chunked.
 *   - The backward needs Q, K, V, O and the incoming gradient (FPDT summary,
 *     "Background").  The pages print no backward formulas; the gradients here
 *     are the plain derivative of L = sum(O * dO), taken by hand.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - GQA: query head h reads key/value head h / g, g = Hq / Hkv.
 *   - softmax scale c = 1 / sqrt(D); LSE is the natural log of the sum of
 *     exp(scaled score) over J(i).
 *   - layout token-major: q, o, dout [S][Hq][D]; k, v [S][Hkv][D]; batch 1.
 *
 * Definition (per query head h, kv = h / g):
 *   s_ij    = c * <q_i, k_j>                       j in J(i)
 *   LSE_i   = log(sum_{j in J(i)} exp(s_ij))
 *   P_ij    = exp(s_ij - LSE_i)
 *   O_i     = sum_j P_ij v_j
 *   dP_ij   = <dO_i, v_j>
 *   Delta_i = sum_j P_ij dP_ij
 *   dS_ij   = P_ij (dP_ij - Delta_i)
 *   dQ_i    = c * sum_j dS_ij k_j
 *   dK_j    = c * sum_{h in G(kv)} sum_{i : j in J(i)} dS^h_ij q^h_i
 *   dV_j    = sum_{h in G(kv)} sum_{i : j in J(i)} P^h_ij dO^h_i
 *
 * All inputs and outputs are fp64 (callers widen bf16/fp32 values exactly);
 * exp/log come from libm.  No blocking or reordering beyond the definition:
 * each sum is a plain loop.  OpenMP runs over (head, query row) for row
 * quantities and over (kv head, key) for dK/dV, so no two threads write one
 * output element.
 *
 * Every entry point returns 0 on success and -1 on an invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef int64_t i64;

static int bad_shape(i64 S, int Hq, int Hkv, int D, int causal) {
    return S < 1 || Hq < 1 || Hkv < 1 || D < 1 || (Hq % Hkv) != 0 ||
           (causal != 0 && causal != 1);
}

/* last key (inclusive) that query row i may attend to */
static i64 last_key(i64 i, i64 S, int causal) { return causal ? i : S - 1; }

static double dot(const double* a, const double* b, int D) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += a[d] * b[d];
    return s;
}

static const double* krow(const double* k, i64 j, int kv, int Hkv, int D) {
    return k + ((size_t)j * Hkv + kv) * D;
}

/* LSE of query row qi against keys [j0, j1] of kv head kv; -inf if empty */
static double row_lse(const double* qi, const double* k, i64 j0, i64 j1, int kv, int Hkv,
                      int D, double c) {
    if (j1 < j0) return -INFINITY;
    double m = -INFINITY;
    for (i64 j = j0; j <= j1; ++j) {
        double s = c * dot(qi, krow(k, j, kv, Hkv, D), D);
        if (s > m) m = s;
    }
    double l = 0.0;
    for (i64 j = j0; j <= j1; ++j) l += exp(c * dot(qi, krow(k, j, kv, Hkv, D), D) - m);
    return m + log(l);
}

/* output row over keys [j0, j1] given that key range's LSE */
static void row_out(const double* qi, const double* k, const double* v, i64 j0, i64 j1,
                    int kv, int Hkv, int D, double c, double lse, double* out) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    for (i64 j = j0; j <= j1; ++j) {
        double p = exp(c * dot(qi, krow(k, j, kv, Hkv, D), D) - lse);
        const double* vj = krow(v, j, kv, Hkv, D);
        for (int d = 0; d < D; ++d) out[d] += p * vj[d];
    }
}

/* Delta_i = sum_{j <= j1} P_ij dP_ij (definition form) */
static double row_delta(const double* qi, const double* doi, const double* k, const double* v,
                        i64 j1, int kv, int Hkv, int D, double c, double lse) {
    double delta = 0.0;
    for (i64 j = 0; j <= j1; ++j) {
        double p = exp(c * dot(qi, krow(k, j, kv, Hkv, D), D) - lse);
        delta += p * dot(doi, krow(v, j, kv, Hkv, D), D);
    }
    return delta;
}

/* dQ_i (unscaled sum then times c) for one row */
static void row_dq(const double* qi, const double* doi, const double* k, const double* v,
                   i64 j1, int kv, int Hkv, int D, double c, double lse, double delta,
                   double* out) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    for (i64 j = 0; j <= j1; ++j) {
        const double* kj = krow(k, j, kv, Hkv, D);
        double p = exp(c * dot(qi, kj, D) - lse);
        double ds = p * (dot(doi, krow(v, j, kv, Hkv, D), D) - delta);
        for (int d = 0; d < D; ++d) out[d] += ds * kj[d];
    }
    for (int d = 0; d < D; ++d) out[d] *= c;
}

/* ------------------------------------------------------------------ forward */

int orc_attn_fwd(const double* q, const double* k, const double* v, i64 S, int Hq, int Hkv,
                 int D, int causal, double* o, double* lse) {
    if (bad_shape(S, Hq, Hkv, D, causal)) return -1;
    const double c = 1.0 / sqrt((double)D);
    const int g = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int h = 0; h < Hq; ++h)
        for (i64 i = 0; i < S; ++i) {
            const double* qi = q + ((size_t)i * Hq + h) * D;
            i64 j1 = last_key(i, S, causal);
            double L = row_lse(qi, k, 0, j1, h / g, Hkv, D, c);
            lse[(size_t)h * S + i] = L;
            row_out(qi, k, v, 0, j1, h / g, Hkv, D, c, L, o + ((size_t)i * Hq + h) * D);
        }
    return 0;
}

/*
 * Forward for chosen query rows.  q_rows [n][Hq][D] holds the query rows at
 * positions rows[0..n); k, v hold the whole sequence.  Writes o_rows
 * [n][Hq][D] and lse_rows [Hq][n].
 */
int orc_attn_fwd_rows(const double* q_rows, const i64* rows, i64 n, const double* k,
                      const double* v, i64 S, int Hq, int Hkv, int D, int causal,
                      double* o_rows, double* lse_rows) {
    if (bad_shape(S, Hq, Hkv, D, causal) || n < 0) return -1;
    for (i64 r = 0; r < n; ++r)
        if (rows[r] < 0 || rows[r] >= S) return -1;
    const double c = 1.0 / sqrt((double)D);
    const int g = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int h = 0; h < Hq; ++h)
        for (i64 r = 0; r < n; ++r) {
            const double* qi = q_rows + ((size_t)r * Hq + h) * D;
            i64 j1 = last_key(rows[r], S, causal);
            double L = row_lse(qi, k, 0, j1, h / g, Hkv, D, c);
            lse_rows[(size_t)h * n + r] = L;
            row_out(qi, k, v, 0, j1, h / g, Hkv, D, c, L, o_rows + ((size_t)r * Hq + h) * D);
        }
    return 0;
}

/*
 * Key-trunked forward in the FPDT order: for query trunk m (rows [mT, mT+T)),
 * for key trunk t = 0..m (t = 0..N-1 when non-causal), take the trunk's
 * partial (O_t, LSE_t) over the keys of trunk t that row i may see and merge
 * it into the running (O, LSE):
 *     L = log(exp(LSE_run) + exp(LSE_t))      (shifted by the larger one)
 *     O = exp(LSE_run - L) O_run + exp(LSE_t - L) O_t
 * A trunk with no visible key for a row has LSE_t = -inf, weight 0, and is
 * skipped, which is the same as merging it.
 */
int orc_attn_fwd_trunked(const double* q, const double* k, const double* v, i64 S, int Hq,
                         int Hkv, int D, int causal, i64 T, double* o, double* lse) {
    if (bad_shape(S, Hq, Hkv, D, causal) || T < 1) return -1;
    const double c = 1.0 / sqrt((double)D);
    const int g = Hq / Hkv;
    const i64 N = (S + T - 1) / T;
    int rc = 0;
#pragma omp parallel
    {
        double* ot = (double*)malloc(sizeof(double) * (size_t)D);
        if (!ot) {
#pragma omp atomic write
            rc = -1;
        }
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int h = 0; h < Hq; ++h)
            for (i64 i = 0; i < S; ++i) {
                if (!ot) continue;
                const double* qi = q + ((size_t)i * Hq + h) * D;
                double* orow = o + ((size_t)i * Hq + h) * D;
                i64 tlast = causal ? i / T : N - 1;
                double Lrun = -INFINITY;
                for (int d = 0; d < D; ++d) orow[d] = 0.0;
                for (i64 t = 0; t <= tlast; ++t) {
                    i64 j0 = t * T, j1 = (t + 1) * T - 1;
                    if (j1 > last_key(i, S, causal)) j1 = last_key(i, S, causal);
                    double Lt = row_lse(qi, k, j0, j1, h / g, Hkv, D, c);
                    if (Lt == -INFINITY) continue;
                    row_out(qi, k, v, j0, j1, h / g, Hkv, D, c, Lt, ot);
                    if (Lrun == -INFINITY) {
                        Lrun = Lt;
                        for (int d = 0; d < D; ++d) orow[d] = ot[d];
                        continue;
                    }
                    double mx = Lrun > Lt ? Lrun : Lt;
                    double L = mx + log(exp(Lrun - mx) + exp(Lt - mx));
                    double wr = exp(Lrun - L), wt = exp(Lt - L);
                    for (int d = 0; d < D; ++d) orow[d] = wr * orow[d] + wt * ot[d];
                    Lrun = L;
                }
                lse[(size_t)h * S + i] = Lrun;
            }
        free(ot);
    }
    return rc;
}

/*
 * Head-chunked forward: for each chunk of hc consecutive query heads, copy
 * the chunk's query heads and the kv heads they read into one set of chunk
 * buffers (allocated once, sized for the widest chunk, reused by every
 * chunk), run attention on the chunk buffers, and store the chunk's output.
 * Heads are independent, so the numbers equal orc_attn_fwd's exactly.
 */
int orc_attn_fwd_chunked(const double* q, const double* k, const double* v, i64 S, int Hq,
                         int Hkv, int D, int causal, int hc, double* o, double* lse) {
    if (bad_shape(S, Hq, Hkv, D, causal) || hc < 1) return -1;
    const int g = Hq / Hkv;
    if (hc > Hq) hc = Hq;
    int kvmax = (hc + g - 1) / g + 1;
    if (kvmax > Hkv) kvmax = Hkv;
    double* qc = (double*)malloc(sizeof(double) * (size_t)S * hc * D);
    double* kc = (double*)malloc(sizeof(double) * (size_t)S * kvmax * D);
    double* vc = (double*)malloc(sizeof(double) * (size_t)S * kvmax * D);
    double* oc = (double*)malloc(sizeof(double) * (size_t)S * hc * D);
    double* lc = (double*)malloc(sizeof(double) * (size_t)S * hc);
    int rc = 0;
    if (!qc || !kc || !vc || !oc || !lc) rc = -1;
    for (int h0 = 0; rc == 0 && h0 < Hq; h0 += hc) {
        int nh = (h0 + hc <= Hq) ? hc : Hq - h0;
        int kv0 = h0 / g, nkv = (h0 + nh - 1) / g - kv0 + 1;
        for (i64 s = 0; s < S; ++s) {
            memcpy(qc + (size_t)s * nh * D, q + ((size_t)s * Hq + h0) * D, sizeof(double) * (size_t)nh * D);
            memcpy(kc + (size_t)s * nkv * D, k + ((size_t)s * Hkv + kv0) * D, sizeof(double) * (size_t)nkv * D);
            memcpy(vc + (size_t)s * nkv * D, v + ((size_t)s * Hkv + kv0) * D, sizeof(double) * (size_t)nkv * D);
        }
        const double c = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
        for (int hh = 0; hh < nh; ++hh)
            for (i64 i = 0; i < S; ++i) {
                const double* qi = qc + ((size_t)i * nh + hh) * D;
                int kvl = (h0 + hh) / g - kv0;
                i64 j1 = last_key(i, S, causal);
                double L = row_lse(qi, kc, 0, j1, kvl, nkv, D, c);
                lc[(size_t)hh * S + i] = L;
                row_out(qi, kc, vc, 0, j1, kvl, nkv, D, c, L, oc + ((size_t)i * nh + hh) * D);
            }
        for (i64 s = 0; s < S; ++s)
            memcpy(o + ((size_t)s * Hq + h0) * D, oc + (size_t)s * nh * D, sizeof(double) * (size_t)nh * D);
        for (int hh = 0; hh < nh; ++hh)
            memcpy(lse + (size_t)(h0 + hh) * S, lc + (size_t)hh * S, sizeof(double) * (size_t)S);
    }
    free(qc); free(kc); free(vc); free(oc); free(lc);
    return rc;
}

/* ----------------------------------------------------------------- backward */

/* dK_j, dV_j of kv head kv from every head of its group and every row i in
 * [i0, S) that sees key j; q_tail/dout_tail hold rows [i0, S); L and Dl hold
 * LSE and Delta of those rows, [Hq][S - i0]. */
static void col_dkdv(const double* q_tail, const double* dout_tail, i64 i0, const double* k,
                     const double* v, const double* L, const double* Dl, i64 S, int Hq, int Hkv,
                     int D, int causal, i64 j, int kv, double* dkj, double* dvj) {
    const double c = 1.0 / sqrt((double)D);
    const int g = Hq / Hkv;
    const i64 nr = S - i0;
    const double* kj = krow(k, j, kv, Hkv, D);
    const double* vj = krow(v, j, kv, Hkv, D);
    for (int d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
    for (int h = kv * g; h < kv * g + g; ++h)
        for (i64 i = causal ? j : 0; i < S; ++i) {
            const double* qi = q_tail + ((size_t)(i - i0) * Hq + h) * D;
            const double* doi = dout_tail + ((size_t)(i - i0) * Hq + h) * D;
            double p = exp(c * dot(qi, kj, D) - L[(size_t)h * nr + (i - i0)]);
            double ds = p * (dot(doi, vj, D) - Dl[(size_t)h * nr + (i - i0)]);
            for (int d = 0; d < D; ++d) {
                dkj[d] += ds * qi[d];
                dvj[d] += p * doi[d];
            }
        }
    for (int d = 0; d < D; ++d) dkj[d] *= c;
}

/*
 * Full backward of L = sum(O * dout).  Row pass (parallel over head, row):
 * LSE_i, Delta_i, dQ_i.  Column pass (parallel over kv head, key): dK_j, dV_j,
 * recomputing P from the row pass's LSE.  lse_out, delta_out ([Hq][S]) may be
 * NULL.
 */
int orc_attn_bwd(const double* q, const double* k, const double* v, const double* dout, i64 S,
                 int Hq, int Hkv, int D, int causal, double* dq, double* dk, double* dv,
                 double* lse_out, double* delta_out) {
    if (bad_shape(S, Hq, Hkv, D, causal)) return -1;
    const double c = 1.0 / sqrt((double)D);
    const int g = Hq / Hkv;
    double* L = (double*)malloc(sizeof(double) * (size_t)Hq * S);
    double* Dl = (double*)malloc(sizeof(double) * (size_t)Hq * S);
    if (!L || !Dl) { free(L); free(Dl); return -1; }
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int h = 0; h < Hq; ++h)
        for (i64 i = 0; i < S; ++i) {
            const double* qi = q + ((size_t)i * Hq + h) * D;
            const double* doi = dout + ((size_t)i * Hq + h) * D;
            i64 j1 = last_key(i, S, causal);
            double Li = row_lse(qi, k, 0, j1, h / g, Hkv, D, c);
            double di = row_delta(qi, doi, k, v, j1, h / g, Hkv, D, c, Li);
            L[(size_t)h * S + i] = Li;
            Dl[(size_t)h * S + i] = di;
            row_dq(qi, doi, k, v, j1, h / g, Hkv, D, c, Li, di, dq + ((size_t)i * Hq + h) * D);
        }
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int kv = 0; kv < Hkv; ++kv)
        for (i64 j = 0; j < S; ++j)
            col_dkdv(q, dout, 0, k, v, L, Dl, S, Hq, Hkv, D, causal, j, kv,
                     dk + ((size_t)j * Hkv + kv) * D, dv + ((size_t)j * Hkv + kv) * D);
    if (lse_out) memcpy(lse_out, L, sizeof(double) * (size_t)Hq * S);
    if (delta_out) memcpy(delta_out, Dl, sizeof(double) * (size_t)Hq * S);
    free(L);
    free(Dl);
    return 0;
}

/*
 * dQ for chosen rows: q_rows, dout_rows [n][Hq][D] hold rows rows[0..n);
 * writes dq_rows [n][Hq][D] and, if not NULL, delta_rows [Hq][n].
 */
int orc_attn_dq_rows(const double* q_rows, const double* dout_rows, const i64* rows, i64 n,
                     const double* k, const double* v, i64 S, int Hq, int Hkv, int D,
                     int causal, double* dq_rows, double* delta_rows) {
    if (bad_shape(S, Hq, Hkv, D, causal) || n < 0) return -1;
    for (i64 r = 0; r < n; ++r)
        if (rows[r] < 0 || rows[r] >= S) return -1;
    const double c = 1.0 / sqrt((double)D);
    const int g = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int h = 0; h < Hq; ++h)
        for (i64 r = 0; r < n; ++r) {
            const double* qi = q_rows + ((size_t)r * Hq + h) * D;
            const double* doi = dout_rows + ((size_t)r * Hq + h) * D;
            i64 j1 = last_key(rows[r], S, causal);
            double Li = row_lse(qi, k, 0, j1, h / g, Hkv, D, c);
            double di = row_delta(qi, doi, k, v, j1, h / g, Hkv, D, c, Li);
            if (delta_rows) delta_rows[(size_t)h * n + r] = di;
            row_dq(qi, doi, k, v, j1, h / g, Hkv, D, c, Li, di, dq_rows + ((size_t)r * Hq + h) * D);
        }
    return 0;
}

/*
 * dK, dV for chosen keys cols[0..n).  q_tail, dout_tail [S - i0][Hq][D] hold
 * query rows [i0, S); every row that sees one of the keys must be there
 * (causal: i0 <= min(cols); non-causal: i0 == 0).  LSE and Delta of those rows
 * are computed here from the definition.  Writes dk_cols, dv_cols [n][Hkv][D].
 */
int orc_attn_dkdv_cols(const double* q_tail, const double* dout_tail, i64 i0, const double* k,
                       const double* v, i64 S, int Hq, int Hkv, int D, int causal,
                       const i64* cols, i64 n, double* dk_cols, double* dv_cols) {
    if (bad_shape(S, Hq, Hkv, D, causal) || n < 0 || i0 < 0 || i0 >= S) return -1;
    if (!causal && i0 != 0) return -1;
    for (i64 r = 0; r < n; ++r)
        if (cols[r] < i0 || cols[r] >= S) return -1;
    const double c = 1.0 / sqrt((double)D);
    const int g = Hq / Hkv;
    const i64 nr = S - i0;
    double* L = (double*)malloc(sizeof(double) * (size_t)Hq * nr);
    double* Dl = (double*)malloc(sizeof(double) * (size_t)Hq * nr);
    if (!L || !Dl) { free(L); free(Dl); return -1; }
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int h = 0; h < Hq; ++h)
        for (i64 i = i0; i < S; ++i) {
            const double* qi = q_tail + ((size_t)(i - i0) * Hq + h) * D;
            const double* doi = dout_tail + ((size_t)(i - i0) * Hq + h) * D;
            i64 j1 = last_key(i, S, causal);
            double Li = row_lse(qi, k, 0, j1, h / g, Hkv, D, c);
            L[(size_t)h * nr + (i - i0)] = Li;
            Dl[(size_t)h * nr + (i - i0)] = row_delta(qi, doi, k, v, j1, h / g, Hkv, D, c, Li);
        }
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (i64 r = 0; r < n; ++r)
        for (int kv = 0; kv < Hkv; ++kv)
            col_dkdv(q_tail, dout_tail, i0, k, v, L, Dl, S, Hq, Hkv, D, causal, cols[r], kv,
                     dk_cols + ((size_t)r * Hkv + kv) * D, dv_cols + ((size_t)r * Hkv + kv) * D);
    free(L);
    free(Dl);
    return 0;
}

/* ------------------------------------------------- attention layer (NEXT) */

/*
 * The attention layer around the attention itself, as the U-Pipe paragraph
 * of the Road to 5 Million Tokens talk describes the chunk loop: for a group
 * of heads, the heads' projections are (re)computed, attention runs on them,
 * and the group's partial result is stored before the buffers are reused.
 * The pages name no projection shapes; the readings here (each listed in the
 * design notes): weights in the [out][in] convention, no bias, no rotary
 * embedding, batch 1, d_model = dm:
 *     q = x Wq^T  [S][Hq*D]     Wq [Hq*D][dm]
 *     k = x Wk^T  [S][Hkv*D]    Wk [Hkv*D][dm]
 *     v = x Wv^T  [S][Hkv*D]    Wv [Hkv*D][dm]
 *     o = attention(q, k, v)    (the definition above, heads as [S][H][D])
 *     y = o Wo^T  [S][dm]       Wo [dm][Hq*D]
 * and the gradients of L = sum(y * dy).
 */

/* out[s][n] = sum_c a[s][c] w[n][c]   (a [S][K], w [N][K]) */
static void matmul_nt(const double* a, const double* w, i64 S, int K, int N, double* out) {
#pragma omp parallel for schedule(static)
    for (i64 s = 0; s < S; ++s)
        for (int n = 0; n < N; ++n)
            out[(size_t)s * N + n] = dot(a + (size_t)s * K, w + (size_t)n * K, K);
}

/* out[s][c] = sum_n g[s][n] w[n][c]   (g [S][N], w [N][K]); accumulate if acc */
static void matmul_nn(const double* g, const double* w, i64 S, int N, int K, double* out, int acc) {
#pragma omp parallel for schedule(static)
    for (i64 s = 0; s < S; ++s)
        for (int c = 0; c < K; ++c) {
            double t = 0.0;
            for (int n = 0; n < N; ++n) t += g[(size_t)s * N + n] * w[(size_t)n * K + c];
            out[(size_t)s * K + c] = acc ? out[(size_t)s * K + c] + t : t;
        }
}

/* out[n][c] = sum_s g[s][n] a[s][c]   (g [S][N], a [S][K]) */
static void matmul_tn(const double* g, const double* a, i64 S, int N, int K, double* out) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; ++n)
        for (int c = 0; c < K; ++c) {
            double t = 0.0;
            for (i64 s = 0; s < S; ++s) t += g[(size_t)s * N + n] * a[(size_t)s * K + c];
            out[(size_t)n * K + c] = t;
        }
}

int orc_layer_fwd(const double* x, const double* wq, const double* wk, const double* wv,
                  const double* wo, i64 S, int dm, int Hq, int Hkv, int D, int causal,
                  double* y, double* lse) {
    if (bad_shape(S, Hq, Hkv, D, causal) || dm < 1) return -1;
    const int nq = Hq * D, nk = Hkv * D;
    double* q = (double*)malloc(sizeof(double) * (size_t)S * nq);
    double* k = (double*)malloc(sizeof(double) * (size_t)S * nk);
    double* v = (double*)malloc(sizeof(double) * (size_t)S * nk);
    double* o = (double*)malloc(sizeof(double) * (size_t)S * nq);
    double* l = (double*)malloc(sizeof(double) * (size_t)Hq * S);
    int rc = (q && k && v && o && l) ? 0 : -1;
    if (rc == 0) {
        matmul_nt(x, wq, S, dm, nq, q);
        matmul_nt(x, wk, S, dm, nk, k);
        matmul_nt(x, wv, S, dm, nk, v);
        rc = orc_attn_fwd(q, k, v, S, Hq, Hkv, D, causal, o, l);
    }
    if (rc == 0) {
        matmul_nt(o, wo, S, nq, dm, y);
        if (lse) memcpy(lse, l, sizeof(double) * (size_t)Hq * S);
    }
    free(q); free(k); free(v); free(o); free(l);
    return rc;
}

/*
 * The same layer walked a head chunk at a time in the U-Pipe order: for the
 * chunk's query heads [h0, h0 + nh) and the kv heads they read, project only
 * those heads from x into one set of chunk buffers (allocated once, reused by
 * every chunk), run attention on the chunk, and add the chunk's share of the
 * output projection, o_c Wo[:, chunk columns]^T, into y.
 */
int orc_layer_fwd_chunked(const double* x, const double* wq, const double* wk, const double* wv,
                          const double* wo, i64 S, int dm, int Hq, int Hkv, int D, int causal,
                          int hc, double* y) {
    if (bad_shape(S, Hq, Hkv, D, causal) || dm < 1 || hc < 1) return -1;
    const int g = Hq / Hkv;
    if (hc > Hq) hc = Hq;
    int kvmax = (hc + g - 1) / g + 1;
    if (kvmax > Hkv) kvmax = Hkv;
    double* qc = (double*)malloc(sizeof(double) * (size_t)S * hc * D);
    double* kc = (double*)malloc(sizeof(double) * (size_t)S * kvmax * D);
    double* vc = (double*)malloc(sizeof(double) * (size_t)S * kvmax * D);
    double* oc = (double*)malloc(sizeof(double) * (size_t)S * hc * D);
    double* lc = (double*)malloc(sizeof(double) * (size_t)S * hc);
    double* woc = (double*)malloc(sizeof(double) * (size_t)dm * hc * D);
    int rc = (qc && kc && vc && oc && lc && woc) ? 0 : -1;
    for (size_t i = 0; rc == 0 && i < (size_t)S * dm; ++i) y[i] = 0.0;
    for (int h0 = 0; rc == 0 && h0 < Hq; h0 += hc) {
        const int nh = (h0 + hc <= Hq) ? hc : Hq - h0;
        const int kv0 = h0 / g, nkv = (h0 + nh - 1) / g - kv0 + 1;
        /* the chunk's rows of Wq / Wk / Wv are contiguous: heads h0.. and kv0.. */
        matmul_nt(x, wq + (size_t)h0 * D * dm, S, dm, nh * D, qc);
        matmul_nt(x, wk + (size_t)kv0 * D * dm, S, dm, nkv * D, kc);
        matmul_nt(x, wv + (size_t)kv0 * D * dm, S, dm, nkv * D, vc);
        /* attention of the chunk: query head hh reads local kv head (h0+hh)/g - kv0 */
        const double c = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
        for (int hh = 0; hh < nh; ++hh)
            for (i64 i = 0; i < S; ++i) {
                const double* qi = qc + ((size_t)i * nh + hh) * D;
                const int kvl = (h0 + hh) / g - kv0;
                const i64 j1 = last_key(i, S, causal);
                const double L = row_lse(qi, kc, 0, j1, kvl, nkv, D, c);
                lc[(size_t)hh * S + i] = L;
                row_out(qi, kc, vc, 0, j1, kvl, nkv, D, c, L, oc + ((size_t)i * nh + hh) * D);
            }
        /* y += o_c Wo[:, h0*D .. (h0+nh)*D]^T */
        for (int m = 0; m < dm; ++m)
            for (int n = 0; n < nh * D; ++n) woc[(size_t)m * nh * D + n] = wo[(size_t)m * Hq * D + (size_t)h0 * D + n];
#pragma omp parallel for schedule(static)
        for (i64 s = 0; s < S; ++s)
            for (int m = 0; m < dm; ++m)
                y[(size_t)s * dm + m] += dot(oc + (size_t)s * nh * D, woc + (size_t)m * nh * D, nh * D);
    }
    free(qc); free(kc); free(vc); free(oc); free(lc); free(woc);
    return rc;
}

/*
 * Backward of L = sum(y * dy) through the layer:
 *     do  = dy Wo,          dWo = dy^T o
 *     (dq, dk, dv) = attention backward with do
 *     dx  = dq Wq + dk Wk + dv Wv
 *     dWq = dq^T x,  dWk = dk^T x,  dWv = dv^T x
 */
int orc_layer_bwd(const double* x, const double* wq, const double* wk, const double* wv,
                  const double* wo, const double* dy, i64 S, int dm, int Hq, int Hkv, int D,
                  int causal, double* dx, double* dwq, double* dwk, double* dwv, double* dwo) {
    if (bad_shape(S, Hq, Hkv, D, causal) || dm < 1) return -1;
    const int nq = Hq * D, nk = Hkv * D;
    double* q = (double*)malloc(sizeof(double) * (size_t)S * nq);
    double* k = (double*)malloc(sizeof(double) * (size_t)S * nk);
    double* v = (double*)malloc(sizeof(double) * (size_t)S * nk);
    double* o = (double*)malloc(sizeof(double) * (size_t)S * nq);
    double* l = (double*)malloc(sizeof(double) * (size_t)Hq * S);
    double* dov = (double*)malloc(sizeof(double) * (size_t)S * nq);
    double* dq = (double*)malloc(sizeof(double) * (size_t)S * nq);
    double* dk = (double*)malloc(sizeof(double) * (size_t)S * nk);
    double* dv = (double*)malloc(sizeof(double) * (size_t)S * nk);
    int rc = (q && k && v && o && l && dov && dq && dk && dv) ? 0 : -1;
    if (rc == 0) {
        matmul_nt(x, wq, S, dm, nq, q);
        matmul_nt(x, wk, S, dm, nk, k);
        matmul_nt(x, wv, S, dm, nk, v);
        rc = orc_attn_fwd(q, k, v, S, Hq, Hkv, D, causal, o, l);
    }
    if (rc == 0) {
        matmul_nn(dy, wo, S, dm, nq, dov, 0);
        matmul_tn(dy, o, S, dm, nq, dwo);
        rc = orc_attn_bwd(q, k, v, dov, S, Hq, Hkv, D, causal, dq, dk, dv, NULL, NULL);
    }
    if (rc == 0) {
        matmul_nn(dq, wq, S, nq, dm, dx, 0);
        matmul_nn(dk, wk, S, nk, dm, dx, 1);
        matmul_nn(dv, wv, S, nk, dm, dx, 1);
        matmul_tn(dq, x, S, nq, dm, dwq);
        matmul_tn(dk, x, S, nk, dm, dwk);
        matmul_tn(dv, x, S, nk, dm, dwv);
    }
    free(q); free(k); free(v); free(o); free(l); free(dov); free(dq); free(dk); free(dv);
    return rc;
}

/*
 * The layer's output for chosen rows: y_rows [n][dm] at positions rows[0..n)
 * (and lse_rows [Hq][n]).  The query projections of those rows and the key /
 * value projections of every position are taken from x (the whole
 * sequence); then each row's attention and its output projection, as in
 * orc_layer_fwd.
 */
int orc_layer_fwd_rows(const double* x, const double* wq, const double* wk, const double* wv,
                       const double* wo, i64 S, int dm, int Hq, int Hkv, int D, int causal,
                       const i64* rows, i64 n, double* y_rows, double* lse_rows) {
    if (bad_shape(S, Hq, Hkv, D, causal) || dm < 1 || n < 0) return -1;
    for (i64 r = 0; r < n; ++r)
        if (rows[r] < 0 || rows[r] >= S) return -1;
    const int nq = Hq * D, nk = Hkv * D;
    double* xr = (double*)malloc(sizeof(double) * (size_t)(n ? n : 1) * dm);
    double* q = (double*)malloc(sizeof(double) * (size_t)(n ? n : 1) * nq);
    double* k = (double*)malloc(sizeof(double) * (size_t)S * nk);
    double* v = (double*)malloc(sizeof(double) * (size_t)S * nk);
    double* o = (double*)malloc(sizeof(double) * (size_t)(n ? n : 1) * nq);
    int rc = (xr && q && k && v && o) ? 0 : -1;
    if (rc == 0) {
        for (i64 r = 0; r < n; ++r)
            memcpy(xr + (size_t)r * dm, x + (size_t)rows[r] * dm, sizeof(double) * (size_t)dm);
        matmul_nt(xr, wq, n, dm, nq, q);
        matmul_nt(x, wk, S, dm, nk, k);
        matmul_nt(x, wv, S, dm, nk, v);
        rc = orc_attn_fwd_rows(q, rows, n, k, v, S, Hq, Hkv, D, causal, o, lse_rows);
    }
    if (rc == 0) matmul_nt(o, wo, n, nq, dm, y_rows);
    free(xr); free(q); free(k); free(v); free(o);
    return rc;
}
