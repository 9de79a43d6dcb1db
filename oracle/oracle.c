/*
 * oracle.c - plain, slow CPU reference for quantized cross-loop decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code, header, table or constant with the HIP path.
 *
 * Sources (pages about "FlashLoop: Fast and Memory-Efficient Looped Transformers
 * via Lazy Updates"):
 *   [P1] PyPI project page, "Configuration and supported scope" (defaults: 4-bit K/V,
 *        group 64, 64-token BF16 tail, 10% key retention in sparse loops).
 *   [P2] project page, "The Method", STEP 01 (inactive tokens reuse the previous
 *        loop's K/V), STEP 02 (columns chosen from the preceding loop; their global
 *        probability mass under the preceding loop's full distribution is cached),
 *        STEP 03 (loop-1 K/V quantized as the base, later loops store the residual
 *        against the reconstructed previous loop).
 *   [P5] flozi.net explainer, section 3 "What FlashLoop actually computes" (INT4,
 *        group-wise asymmetric, group 64, per-channel post-RoPE keys, per-token values,
 *        most recent 64 tokens kept in BF16; residual X^(r) - Xhat^(r-1) on active
 *        tokens only; top-K columns from the previous loop's statistics and a rank-K
 *        correction of the previous loop's output that keeps the cached mass).
 *
 * Precision: attention arithmetic is fp64.  The codec is specified in fp32 (scales and
 * zeros are stored as fp32 and the GPU must match them bit for bit), so each codec
 * step below is one IEEE fp32 operation: this file must be built without fast-math
 * and with -ffp-contract=off so that no two of them are fused.
 *
 * Readings where the pages are silent:
 *   - quantizer: s = (max-min)/15, z = min, code = rint((x-z)/s) clamped to [0,15],
 *     round-half-even, s == 0 gives code 0; -0 is canonicalised to +0 in s and z;
 *   - dequantised value = fmaf(code, s, z) (single rounding);
 *   - selection key is the fp32 score, descending, ties to the lower index;
 *   - the sparse update keeps the cached mass m for the selected set and
 *     re-distributes it by a softmax over the selected columns' new scores.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GROUP 64

/* ---------------------------------------------------------------------------------
 * Quantizer [P5 section 3]: asymmetric min/max over one group of m <= 64 values
 * x[0], x[stride], ... with 2^bits levels (bits = 4 for the pages' INT4 codec; 2 for
 * the 2-bit residual setting of the project page's precision sweep, "Main Results", and
 * of the explainer's section 5).  Writes m codes (one per byte) and the group's fp32 s, z.
 * ------------------------------------------------------------------------------- */
void orc_quantize_group(const float* x, int m, long stride, int bits,
                        uint8_t* code, long code_stride, float* s_out, float* z_out)
{
    const float top = (float)((1 << bits) - 1);  /* largest code: 15 or 3 */
    float mn = x[0], mx = x[0];
    for (int i = 1; i < m; ++i) {
        float v = x[(long)i * stride];
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    float range = mx - mn;          /* one fp32 subtraction */
    float s = range / top;          /* one fp32 division    */
    s = s + 0.0f;                   /* -0 -> +0             */
    float z = mn + 0.0f;            /* -0 -> +0             */
    for (int i = 0; i < m; ++i) {
        uint8_t c = 0;
        if (s != 0.0f) {
            float t = x[(long)i * stride] - z;  /* fp32 subtraction */
            float u = t / s;                    /* fp32 division    */
            float r = rintf(u);                 /* half to even     */
            if (r < 0.0f) r = 0.0f;
            if (r > top) r = top;
            c = (uint8_t)r;
        }
        code[(long)i * code_stride] = c;
    }
    *s_out = s;
    *z_out = z;
}

float orc_dequant(uint8_t c, float s, float z) { return fmaf((float)c, s, z); }

/* ---------------------------------------------------------------------------------
 * One loop's encode of the rows stored by one call [P2 STEP 03, P5 section 3].
 * Rows are the call's stored (active) rows in ascending position order.
 *   X[nrows][d]  : this loop's K (or V) values of those rows (bf16 values held in fp32)
 *   P[nrows][d]  : the previous loop's reconstruction of the same rows, NULL at loop 1
 * The residual D = X - P (fp32) is quantized:
 *   keys   (is_key=1): per channel over each run of 64 consecutive stored rows
 *                      -> s[ngroups][d], z[ngroups][d]
 *   values (is_key=0): per row over each run of 64 consecutive channels
 *                      -> s[nrows][d/64], z[nrows][d/64]
 * code[nrows][d] one code per byte, `bits` bits each.  R[nrows][d] receives the new
 * reconstruction (loop 1: dequantised value; later loops: P + dequantised residual,
 * fp32 add).  With P == NULL the rows' own values are quantized, which is also how the
 * per-loop full-state INT4 ablation (explainer section 4, "Per-loop KIVI4") stores
 * every loop.
 * ------------------------------------------------------------------------------- */
void orc_encode_rows(int nrows, int d, int is_key, int bits, const float* X, const float* P,
                     uint8_t* code, float* s, float* z, float* R)
{
    float* D = (float*)malloc(sizeof(float) * (size_t)(nrows > 0 ? nrows : 1) * d);
    for (long i = 0; i < (long)nrows * d; ++i)
        D[i] = P ? (X[i] - P[i]) : X[i];

    if (is_key) {
        int ngroups = (nrows + ORC_GROUP - 1) / ORC_GROUP;
        for (int g = 0; g < ngroups; ++g) {
            int r0 = g * ORC_GROUP;
            int m = nrows - r0 < ORC_GROUP ? nrows - r0 : ORC_GROUP;
            for (int c = 0; c < d; ++c)
                orc_quantize_group(D + (long)r0 * d + c, m, d, bits,
                                   code + (long)r0 * d + c, d,
                                   s + (long)g * d + c, z + (long)g * d + c);
        }
        for (int i = 0; i < nrows; ++i)
            for (int c = 0; c < d; ++c) {
                int g = i / ORC_GROUP;
                float deq = orc_dequant(code[(long)i * d + c], s[(long)g * d + c], z[(long)g * d + c]);
                R[(long)i * d + c] = P ? (P[(long)i * d + c] + deq) : deq;
            }
    } else {
        int gpr = d / ORC_GROUP;
        for (int i = 0; i < nrows; ++i)
            for (int g = 0; g < gpr; ++g)
                orc_quantize_group(D + (long)i * d + g * ORC_GROUP, ORC_GROUP, 1, bits,
                                   code + (long)i * d + g * ORC_GROUP, 1,
                                   s + (long)i * gpr + g, z + (long)i * gpr + g);
        for (int i = 0; i < nrows; ++i)
            for (int c = 0; c < d; ++c) {
                int g = c / ORC_GROUP;
                float deq = orc_dequant(code[(long)i * d + c], s[(long)i * gpr + g], z[(long)i * gpr + g]);
                R[(long)i * d + c] = P ? (P[(long)i * d + c] + deq) : deq;
            }
    }
    free(D);
}

/* ---------------------------------------------------------------------------------
 * Dense attention of one query over n columns [P5 section 1: decode attention reads
 * every cached column]: the textbook softmax attention in fp64.
 *   s_j = sm * sum_d q_d K[j][d];  lse = log sum_j exp(s_j);  o = sum_j exp(s_j-lse) V[j]
 * K, V are the loop's reconstructed keys/values (fp32), q the bf16 query in fp32.
 * ------------------------------------------------------------------------------- */
void orc_attend_dense(int n, int d, const float* q, double sm, const float* K, const float* V,
                      double* o, double* scores, double* lse_out)
{
    double mx = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)q[c] * (double)K[(long)j * d + c];
        scores[j] = sm * acc;
        if (scores[j] > mx) mx = scores[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) l += exp(scores[j] - mx);
    double lse = mx + log(l);
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int j = 0; j < n; ++j) {
        double p = exp(scores[j] - lse);
        for (int c = 0; c < d; ++c) o[c] += p * (double)V[(long)j * d + c];
    }
    *lse_out = lse;
}

/* ---------------------------------------------------------------------------------
 * Column selection [P2 STEP 02, P5 section 3]: the k columns with the largest fp32
 * score (ties: lower index first), returned in ascending index order, with each
 * column's probability under the preceding distribution, p_j = exp(s_j - lse), and
 * their total mass m = sum p_j.  k >= n takes every column, k = 0 none.
 * ------------------------------------------------------------------------------- */
typedef struct { float key; int32_t index; } orc_keyed;

static int cmp_desc_then_index(const void* a, const void* b)
{
    const orc_keyed* x = (const orc_keyed*)a;
    const orc_keyed* y = (const orc_keyed*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->index < y->index) ? -1 : (x->index > y->index);
}
static int cmp_index(const void* a, const void* b)
{
    int ia = *(const int32_t*)a, ib = *(const int32_t*)b;
    return (ia < ib) ? -1 : (ia > ib);
}

int orc_select(int n, const float* scores, double lse, int k,
               int32_t* idx, double* p_sel, double* mass)
{
    if (k > n) k = n;
    if (k < 0) k = 0;
    orc_keyed* order = (orc_keyed*)malloc(sizeof(orc_keyed) * (size_t)(n > 0 ? n : 1));
    for (int j = 0; j < n; ++j) { order[j].key = scores[j]; order[j].index = j; }
    qsort(order, (size_t)n, sizeof(orc_keyed), cmp_desc_then_index);
    for (int i = 0; i < k; ++i) idx[i] = order[i].index;
    qsort(idx, (size_t)k, sizeof(int32_t), cmp_index);
    double m = 0.0;
    for (int i = 0; i < k; ++i) {
        p_sel[i] = exp((double)scores[idx[i]] - lse);
        m += p_sel[i];
    }
    *mass = m;
    free(order);
    return k;
}

/* ---------------------------------------------------------------------------------
 * Sparse loop r [P2 STEP 02, P5 section 3 "rank-K correction"]:
 *   s_j  = sm * q . Kr_j for j in S;   alpha = softmax over S of s;
 *   o^(r) = o^(r-1) + sum_{j in S} ( m * alpha_j * Vr_j  -  p_j * Vrm1_j )
 * i.e. the selected columns' old contributions p_j * v^(r-1)_j are removed from the
 * previous output and their cached total mass m is re-assigned by the new in-set
 * softmax over the loop-r values.  scores[j] for j in S is replaced by the logit of
 * that new probability on the previous lse scale: lse + log m + s_j - lse_S, so that
 * sum_j exp(scores_j - lse) stays 1.  Other scores and lse are unchanged.
 * ------------------------------------------------------------------------------- */
void orc_attend_sparse(int n, int d, const float* q, double sm,
                       const float* Kr, const float* Vr, const float* Vrm1,
                       const int32_t* idx, int k, const double* p_sel, double mass,
                       const double* o_prev, double lse, double* scores, double* o)
{
    (void)n;
    for (int c = 0; c < d; ++c) o[c] = o_prev[c];
    if (k <= 0) return;
    double* s = (double*)malloc(sizeof(double) * (size_t)k);
    double mx = -INFINITY;
    for (int i = 0; i < k; ++i) {
        long j = idx[i];
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)q[c] * (double)Kr[j * d + c];
        s[i] = sm * acc;
        if (s[i] > mx) mx = s[i];
    }
    double l = 0.0;
    for (int i = 0; i < k; ++i) l += exp(s[i] - mx);
    double lse_s = mx + log(l);
    for (int i = 0; i < k; ++i) {
        long j = idx[i];
        double alpha = exp(s[i] - lse_s);
        for (int c = 0; c < d; ++c)
            o[c] += mass * alpha * (double)Vr[j * d + c] - p_sel[i] * (double)Vrm1[j * d + c];
        scores[j] = lse + log(mass) + s[i] - lse_s;
    }
    free(s);
}

/* ---------------------------------------------------------------------------------
 * Token selection score [P5 section 3 "Cross-loop token-sparse updates": after the dense
 * loops, each loop ranks the tokens updated in the preceding loop by their normalized
 * hidden-state change and keeps a top-k subset; P2 STEP 01].  Reading: the change of
 * token t is the relative one, ||H_cur[t] - H_prev[t]||_2 / ||H_prev[t]||_2, in fp64
 * (a zero previous state gives +inf for a nonzero change and 0 otherwise).  Tokens not
 * active in the preceding loop (act_prev[t] == 0) score -inf, so the sets nest.
 *   H_cur, H_prev [n][dm]: the preceding loop's output and input states (bf16 values
 *   held in fp32); score[n] out.
 * ------------------------------------------------------------------------------- */
void orc_token_change(int n, int dm, const float* H_cur, const float* H_prev, const uint8_t* act_prev,
                      double* score)
{
    for (int t = 0; t < n; ++t) {
        if (act_prev && !act_prev[t]) { score[t] = -INFINITY; continue; }
        double dd = 0.0, pp = 0.0;
        for (int c = 0; c < dm; ++c) {
            double a = (double)H_cur[(long)t * dm + c], b = (double)H_prev[(long)t * dm + c];
            dd += (a - b) * (a - b);
            pp += b * b;
        }
        if (pp > 0.0) score[t] = sqrt(dd) / sqrt(pp);
        else score[t] = dd > 0.0 ? INFINITY : 0.0;
    }
}

/* ---------------------------------------------------------------------------------
 * Prefill-side sparse loop over compact buffers [P2, The Method, after STEP 03: selected
 * tokens and keys gathered into compact buffers so that the work stays regular GEMMs;
 * P2 STEP 02 and P5 section 3: the rank-K correction that keeps the cached mass].
 * Reading: during prefill a sparse loop updates its active tokens only (nq query rows at
 * ascending positions qpos) against one set of selected columns per head (nc keys at
 * ascending positions cpos); a row sees the columns at or before its own position (causal).
 * For row i and its visible columns j:
 *   s_ij  = sm q_i . K_j            (this loop's query and keys)
 *   p_ij  = exp(sm q0_i . K0_j - lse0_i)   (the preceding loop's probability, from its
 *                                           query, keys and log-sum-exp of row i)
 *   m_i   = sum_j p_ij;   alpha_ij = softmax over the visible j of s_ij
 *   o_i   = o0_i + sum_j (m_i alpha_ij V_j - p_ij V0_j)
 * A row with no visible column keeps o0_i (m_i = 0).  fp64 throughout; inputs fp32
 * (bf16 values held in fp32).  Shapes: Q, Q0 [nq][d]; K, V, K0, V0 [nc][d]; lse0 [nq];
 * O0, O [nq][d]; mass [nq].
 * ------------------------------------------------------------------------------- */
void orc_prefill_sparse(int nq, int nc, int d, const float* Q, const float* Q0, const int32_t* qpos,
                        const double* lse0, const double* O0, const float* K, const float* V, const float* K0,
                        const float* V0, const int32_t* cpos, double sm, double* O, double* mass)
{
    double* s = (double*)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
    for (int i = 0; i < nq; ++i) {
        int nv = 0;
        while (nv < nc && cpos[nv] <= qpos[i]) ++nv;   /* visible columns: a prefix */
        double mx = -INFINITY, m = 0.0;
        for (int j = 0; j < nv; ++j) {
            double a = 0.0, b = 0.0;
            for (int c = 0; c < d; ++c) {
                a += (double)Q[(long)i * d + c] * (double)K[(long)j * d + c];
                b += (double)Q0[(long)i * d + c] * (double)K0[(long)j * d + c];
            }
            s[j] = sm * a;
            p[j] = exp(sm * b - lse0[i]);
            m += p[j];
            if (s[j] > mx) mx = s[j];
        }
        for (int c = 0; c < d; ++c) O[(long)i * d + c] = O0[(long)i * d + c];
        mass[i] = m;
        if (nv == 0) continue;
        double l = 0.0;
        for (int j = 0; j < nv; ++j) l += exp(s[j] - mx);
        for (int j = 0; j < nv; ++j) {
            double alpha = exp(s[j] - mx) / l;
            for (int c = 0; c < d; ++c)
                O[(long)i * d + c] += m * alpha * (double)V[(long)j * d + c] - p[j] * (double)V0[(long)j * d + c];
        }
    }
    free(s);
    free(p);
}

/* ---------------------------------------------------------------------------------
 * Rebuild of one loop's reconstruction from its stored plane [P2 STEP 03; P5 section 3]:
 * for every stored slot s (position pos[s] >= 0) of loop r's plane, the dequantised codes
 * are added to the previous loop's reconstruction (first = 1: loop 1, the base, or every
 * loop of the full-state codec, where they replace it).  K groups are 64 consecutive slots
 * (metadata per group), V groups 64 consecutive channels (metadata per slot).
 *   X[cap][d] holds loop r-1's reconstruction on entry (any value if first) and loop r's on
 *   exit for the stored positions; other positions are left as they are.
 * ------------------------------------------------------------------------------- */
void orc_rebuild_plane(int nslots, int d, const int32_t* pos, const uint8_t* kc, const float* ks, const float* kz,
                       const uint8_t* vc, const float* vs, const float* vz, int first, float* Kx, float* Vx)
{
    int gpr = d / ORC_GROUP;
    for (int s = 0; s < nslots; ++s) {
        long p = pos[s];
        if (p < 0) continue;
        int g = s / ORC_GROUP;
        for (int c = 0; c < d; ++c) {
            float dk = orc_dequant(kc[(long)s * d + c], ks[(long)g * d + c], kz[(long)g * d + c]);
            float dv = orc_dequant(vc[(long)s * d + c], vs[(long)s * gpr + c / ORC_GROUP], vz[(long)s * gpr + c / ORC_GROUP]);
            Kx[p * d + c] = first ? dk : Kx[p * d + c] + dk;
            Vx[p * d + c] = first ? dv : Vx[p * d + c] + dv;
        }
    }
}
