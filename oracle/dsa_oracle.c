/*
 * dsa_oracle.c -- plain, slow, obviously-correct fp64 CPU oracle for the DSA
 * hot path (lightning indexer -> causal top-k -> absorbed sparse MLA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * path: geometry constants below are restated from the pages on purpose.
 *
 * Sources (pages, by title and section):
 *  [P1] "GLM-5.1 架构深度拆解" (cctoctofx.netlify.app, GLM-5.1 architecture
 *       teardown): CH3 §3.2 "Indexer 公式" steps 4-7, CH3 §3.6
 *       "GlmMoeDsaIndexer.forward" steps 4, 5 and 7, CH4 §4.1 and §4.5
 *       "GlmMoeDsaAttention.forward" steps 2, 6 and 7.
 *  [P2] GLM-5 explainer (ailearn.mscapital.top): the indexer paragraph
 *       ("32 x 128 index queries, one 128-d key per position, ReLU, 32
 *       weights, causal Top-2,048"), the "shorter than 2,048 keeps all"
 *       paragraph and the 202,752-token window table.
 *  [P5] "GLM-5.2 架构 QA" (pillumina.github.io), Q1.1 config listing
 *       (qk_nope_head_dim 192 + qk_rope_head_dim 64 = qk_head_dim 256).
 *
 * Every floating-point input arrives as the exact bytes the GPU path reads
 * (bf16 bit patterns as uint16, fp32 weights); each is widened exactly to
 * fp64 and all arithmetic below is fp64 in the plain loop order written.
 * Parallelism is only over independent query rows (OpenMP); the arithmetic
 * inside a row is a single ordered loop nest.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Geometry, restated from [P1] CH3 §3.6 step 1-2 (32 index heads x 128 dims,
 * one 128-d key per position) and CH4 §4.1 (kv_lora_rank 512 + rope 64). */
#define OR_IDX_HEADS 32
#define OR_IDX_DIM 128
#define OR_HEADS 64
#define OR_LATENT 512
#define OR_ROW 576

static double bf16_to_f64(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

const char* oracle_version(void) { return "dsa-oracle fp64 1"; }

/*
 * Lightning-indexer scores ([P1] §3.6 step 5, §3.2 steps 4-5; [P2] indexer
 * paragraph):
 *     d_h    = scale * sum_d q[r,h,d] * K[base_r + t, d]
 *     s[r,t] = sum_h w[r,h] * max(0, d_h)          for 0 <= t < n_r
 * The causal mask of [P1] §3.2 step 6 is the loop bound t < n_r: a query sees
 * its own position and every earlier one.  w is taken as given (already
 * multiplied by 32^-1/2 upstream, [P1] §3.6 step 4).
 *
 * q: [R,32,128] bf16 bits; w: [R,32] fp32; k: packed key cache [*,128] bf16
 * bits; out: [R, ld] fp64, only columns [0, n_r) are written.
 */
/* Thread count of later parallel regions (the OpenMP runtime reads
 * OMP_NUM_THREADS only once, at its first parallel region).  No arithmetic. */
void oracle_set_threads(int32_t n) { omp_set_num_threads(n < 1 ? 1 : n); }

void oracle_indexer_scores(int32_t R, const int32_t* n, const int64_t* base, const uint16_t* q,
                           const float* w, const uint16_t* k, double scale, double* out, int64_t ld)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < R; r++) {
        double qd[OR_IDX_HEADS][OR_IDX_DIM];
        double wd[OR_IDX_HEADS];
        for (int h = 0; h < OR_IDX_HEADS; h++) {
            wd[h] = (double)w[(int64_t)r * OR_IDX_HEADS + h];
            for (int d = 0; d < OR_IDX_DIM; d++)
                qd[h][d] = bf16_to_f64(q[((int64_t)r * OR_IDX_HEADS + h) * OR_IDX_DIM + d]);
        }
        for (int32_t t = 0; t < n[r]; t++) {
            const uint16_t* krow = k + (base[r] + t) * OR_IDX_DIM;
            double kd[OR_IDX_DIM];
            for (int d = 0; d < OR_IDX_DIM; d++) kd[d] = bf16_to_f64(krow[d]);
            double s = 0.0;
            for (int h = 0; h < OR_IDX_HEADS; h++) {
                double dot = 0.0;
                for (int d = 0; d < OR_IDX_DIM; d++) dot += qd[h][d] * kd[d];
                double dh = scale * dot;
                if (dh > 0.0) s += wd[h] * dh;
            }
            out[(int64_t)r * ld + t] = s;
        }
    }
}

/* Round fp64 scores to fp32 with round-to-nearest-even (the C conversion
 * under the default rounding mode), to feed the top-k exactly like the GPU
 * path's fp32 scores. */
void oracle_round_to_f32(int64_t count, const double* in, float* out)
{
    for (int64_t i = 0; i < count; i++) out[i] = (float)in[i];
}

/*
 * Top-k ordering key ([P1] §3.6 step 7 "topk = min(index_topk, total_len)",
 * §3.4 determinism requirement; [P2] "shorter than 2,048 keeps all"):
 * larger score first; IEEE comparison so -0.0 equals +0.0; equal scores are
 * broken toward the lower position; NaN orders below every number.
 */
typedef struct {
    float s;
    int32_t t;
} oracle_entry;

static int cmp_entry(const void* pa, const void* pb)
{
    const oracle_entry* a = (const oracle_entry*)pa;
    const oracle_entry* b = (const oracle_entry*)pb;
    int an = isnan(a->s), bn = isnan(b->s);
    if (an != bn) return an ? 1 : -1;
    if (!an) {
        if (a->s > b->s) return -1;
        if (a->s < b->s) return 1;
    }
    return (a->t < b->t) ? -1 : (a->t > b->t ? 1 : 0);
}

static int cmp_i32(const void* pa, const void* pb)
{
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a < b) ? -1 : (a > b);
}

/*
 * For each row: sort positions [0, n_r) by the key above, keep the first
 * k_r = min(k, n_r), return them in ascending position order, pad with -1.
 * scores: [R, ld] fp32; idx: [R, k] int32.
 */
void oracle_topk(int32_t R, const int32_t* n, const float* scores, int64_t ld, int32_t k, int32_t* idx)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < R; r++) {
        int32_t nr = n[r];
        oracle_entry* e = (oracle_entry*)malloc(sizeof(oracle_entry) * (size_t)(nr > 0 ? nr : 1));
        for (int32_t t = 0; t < nr; t++) {
            e[t].s = scores[(int64_t)r * ld + t];
            e[t].t = t;
        }
        qsort(e, (size_t)nr, sizeof(oracle_entry), cmp_entry);
        int32_t kr = nr < k ? nr : k;
        int32_t* out = idx + (int64_t)r * k;
        for (int32_t j = 0; j < kr; j++) out[j] = e[j].t;
        qsort(out, (size_t)kr, sizeof(int32_t), cmp_i32);
        for (int32_t j = kr; j < k; j++) out[j] = -1;
        free(e);
    }
}

/*
 * Absorbed-MLA attention over a given index list ([P1] §4.5 steps 2, 6, 7;
 * [P2] "the Top-2,048 IDs only drive the gather"; [P5] Q1.1 qk_head_dim 256):
 *     z_j    = softmax_scale * sum_{d<576} qa[r,h,d] * L[base_r + idx_j, d]
 *     p_j    = exp(z_j - m) / sum_j exp(z_j - m),   m = max_j z_j
 *     o[h,c] = sum_j p_j * L[base_r + idx_j, c]      for c < 512
 *     lse[h] = m + log sum_j exp(z_j - m)
 * over the entries idx_j >= 0 of the row (entries < 0 are padding).  The
 * absorbed query qa = [W_UK^T q_nope (512) || q_pe (64)] and the 576-wide
 * latent row [c_kv (512) || k_pe (64)] make the 64-head dot products equal to
 * the expanded 192+64 ones, because kv_b_proj is linear; values are the
 * 512-wide c_kv part, before the per-head V up-projection.
 *
 * qa: [R,64,576] bf16 bits; kv: packed latent cache [*,576] bf16 bits;
 * idx: [R, k] int32; out: [R,64,512] fp64; lse: [R,64] fp64 (may be NULL).
 */
void oracle_sparse_mla(int32_t R, const int64_t* base, const uint16_t* qa, const uint16_t* kv,
                       const int32_t* idx, int32_t k, double softmax_scale, double* out, double* lse)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < R; r++) {
        const int32_t* ir = idx + (int64_t)r * k;
        int32_t m_valid = 0;
        for (int32_t j = 0; j < k; j++)
            if (ir[j] >= 0) m_valid++;
        double* z = (double*)malloc(sizeof(double) * (size_t)(m_valid > 0 ? m_valid : 1));
        const uint16_t** rows = (const uint16_t**)malloc(sizeof(void*) * (size_t)(m_valid > 0 ? m_valid : 1));
        int32_t jj = 0;
        for (int32_t j = 0; j < k; j++)
            if (ir[j] >= 0) rows[jj++] = kv + (base[r] + ir[j]) * OR_ROW;
        for (int h = 0; h < OR_HEADS; h++) {
            const uint16_t* qh = qa + ((int64_t)r * OR_HEADS + h) * OR_ROW;
            double qd[OR_ROW];
            for (int d = 0; d < OR_ROW; d++) qd[d] = bf16_to_f64(qh[d]);
            double m = -INFINITY;
            for (int32_t j = 0; j < m_valid; j++) {
                double dot = 0.0;
                for (int d = 0; d < OR_ROW; d++) dot += qd[d] * bf16_to_f64(rows[j][d]);
                z[j] = softmax_scale * dot;
                if (z[j] > m) m = z[j];
            }
            double denom = 0.0;
            for (int32_t j = 0; j < m_valid; j++) denom += exp(z[j] - m);
            double* o = out + ((int64_t)r * OR_HEADS + h) * OR_LATENT;
            for (int c = 0; c < OR_LATENT; c++) o[c] = 0.0;
            for (int32_t j = 0; j < m_valid; j++) {
                double p = exp(z[j] - m) / denom;
                for (int c = 0; c < OR_LATENT; c++) o[c] += p * bf16_to_f64(rows[j][c]);
            }
            if (lse) lse[(int64_t)r * OR_HEADS + h] = m + log(denom);
        }
        free(rows);
        free(z);
    }
}

/* Per-head kv_b_proj geometry ([P1] CH4 §4.1: kv_b_proj expands the 512-d
 * latent into 64 heads x (192 non-RoPE key dims + 256 value dims); §4.5 step 2
 * splits each head's 448 outputs as [k_nope (192) || value (256)];
 * [P5] Q1.1: qk_nope_head_dim 192, v_head_dim 256). */
#define OR_NOPE 192
#define OR_VDIM 256
#define OR_KVB_ROWS (OR_NOPE + OR_VDIM)
#define OR_ROPE 64

/*
 * Query absorption (the step before the path).  kv_b_proj is linear, so for
 * the non-RoPE part of head h, with W_UK,h the first 192 rows of its 448 output
 * rows ([P1] §4.1, §4.5 step 2):
 *     q_nope . k_nope = q_nope . (W_UK,h c) = (W_UK,h^T q_nope) . c
 * and the absorbed query is the 576-wide [W_UK,h^T q_nope || q_pe]:
 *     q_abs[r,h,c]       = sum_{d<192} W[h,d,c] * q_nope[r,h,d]    (c < 512)
 *     q_abs[r,h,512 + i] = q_pe[r,h,i]                              (i < 64)
 * q_nope: [R,64,192] bf16 bits; q_pe: [R,64,64] bf16 bits; kvb: kv_b_proj
 * weight [64,448,512] bf16 bits; q_abs: [R,64,576] fp64.
 */
void oracle_absorb_queries(int32_t R, const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* kvb,
                           double* q_abs)
{
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < R; r++) {
        for (int h = 0; h < OR_HEADS; h++) {
            const uint16_t* qn = q_nope + ((int64_t)r * OR_HEADS + h) * OR_NOPE;
            const uint16_t* qp = q_pe + ((int64_t)r * OR_HEADS + h) * OR_ROPE;
            const uint16_t* W = kvb + (int64_t)h * OR_KVB_ROWS * OR_LATENT;
            double* o = q_abs + ((int64_t)r * OR_HEADS + h) * OR_ROW;
            for (int c = 0; c < OR_LATENT; c++) {
                double acc = 0.0;
                for (int d = 0; d < OR_NOPE; d++) acc += bf16_to_f64(W[(int64_t)d * OR_LATENT + c]) * bf16_to_f64(qn[d]);
                o[c] = acc;
            }
            for (int i = 0; i < OR_ROPE; i++) o[OR_LATENT + i] = bf16_to_f64(qp[i]);
        }
    }
}

/*
 * V up-projection (the step after the path): the values are W_UV,h c with
 * W_UV,h the last 256 of head h's 448 kv_b_proj rows ([P1] §4.1, §4.5 step 2),
 * and attention weights sum linearly, so the head output is W_UV,h applied to
 * the latent output o[r,h,:]:
 *     out[r,h,v] = sum_{c<512} W[h, 192 + v, c] * o[r,h,c]           (v < 256)
 * o: [R,64,512] fp64 (given as the caller hands it); kvb: [64,448,512] bf16
 * bits; out: [R,64,256] fp64.
 */
void oracle_v_up_proj(int32_t R, const double* o, const uint16_t* kvb, double* out)
{
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < R; r++) {
        for (int h = 0; h < OR_HEADS; h++) {
            const double* oh = o + ((int64_t)r * OR_HEADS + h) * OR_LATENT;
            const uint16_t* W = kvb + ((int64_t)h * OR_KVB_ROWS + OR_NOPE) * OR_LATENT;
            double* y = out + ((int64_t)r * OR_HEADS + h) * OR_VDIM;
            for (int v = 0; v < OR_VDIM; v++) {
                double acc = 0.0;
                for (int c = 0; c < OR_LATENT; c++) acc += bf16_to_f64(W[(int64_t)v * OR_LATENT + c]) * oh[c];
                y[v] = acc;
            }
        }
    }
}

/* ---- cache rows written per new token ------------------------------------
 *
 * [P1] CH3 §3.6 step 2: the indexer key is LayerNorm(128) of wk(hidden),
 * whose first 64 dims then get RoPE and whose last 64 pass through:
 *     k = [RoPE(LN(wk x)[0:64]) || LN(wk x)[64:128]].
 * [P1] CH4 §4.1 / §4.5 steps 2-3: kv_a_proj_with_mqa maps the hidden state to
 * 576 = 512 (compressed kv) + 64 (single-head k_pe); the 512 part goes
 * through kv_a_layernorm (RMSNorm over 512) and k_pe through RoPE:
 *     latent = [RMSNorm(c_kv) || RoPE(k_pe)].
 * RoPE ([P5] Q1.4): the pair (i, i + 32) of a 64-dim block is rotated by the
 * angle m * base^(-2i/64), m the token position, base = rope_theta.  The pages
 * use HF's apply_rotary_pos_emb, which pairs dimension i with i + 32 (the two
 * halves), and which this follows:
 *     y[i]      = x[i] cos(a_i) - x[i + 32] sin(a_i)
 *     y[i + 32] = x[i + 32] cos(a_i) + x[i] sin(a_i)          (i < 32)
 * LayerNorm: (v - mean) / sqrt(var + eps) * g + b with the population
 * variance; RMSNorm: v / sqrt(mean(v^2) + eps) * g.
 * hidden [N, 6144] bf16 bits; wk [128, 6144] and kv_a [576, 6144] bf16 bits
 * (nn.Linear layout: one output per row); k_g, k_b [128], kv_g [512] fp32;
 * pos [N]; outputs key [N, 128] and latent [N, 576] in fp64.
 */
#define OR_HIDDEN 6144

static void or_rope64(double* v, int64_t m, double base)
{
    for (int i = 0; i < 32; i++) {
        const double a = (double)m * pow(base, -2.0 * i / 64.0);
        const double c = cos(a), s = sin(a);
        const double x0 = v[i], x1 = v[i + 32];
        v[i] = x0 * c - x1 * s;
        v[i + 32] = x1 * c + x0 * s;
    }
}

void oracle_cache_rows(int32_t N, const uint16_t* hidden, const uint16_t* wk, const float* k_g, const float* k_b,
                       double k_eps, const uint16_t* kv_a, const float* kv_g, double kv_eps, const int64_t* pos,
                       double rope_theta, double* key, double* latent)
{
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < N; t++) {
        const uint16_t* x = hidden + (int64_t)t * OR_HIDDEN;
        double kx[OR_IDX_DIM], lx[OR_ROW];
        for (int c = 0; c < OR_IDX_DIM; c++) {
            double acc = 0.0;
            for (int d = 0; d < OR_HIDDEN; d++) acc += bf16_to_f64(wk[(int64_t)c * OR_HIDDEN + d]) * bf16_to_f64(x[d]);
            kx[c] = acc;
        }
        for (int c = 0; c < OR_ROW; c++) {
            double acc = 0.0;
            for (int d = 0; d < OR_HIDDEN; d++) acc += bf16_to_f64(kv_a[(int64_t)c * OR_HIDDEN + d]) * bf16_to_f64(x[d]);
            lx[c] = acc;
        }
        /* indexer key: LayerNorm(128), then RoPE on dims 0..63 */
        double mean = 0.0, var = 0.0;
        for (int c = 0; c < OR_IDX_DIM; c++) mean += kx[c];
        mean /= OR_IDX_DIM;
        for (int c = 0; c < OR_IDX_DIM; c++) var += (kx[c] - mean) * (kx[c] - mean);
        var /= OR_IDX_DIM;
        const double inv = 1.0 / sqrt(var + k_eps);
        for (int c = 0; c < OR_IDX_DIM; c++) kx[c] = (kx[c] - mean) * inv * (double)k_g[c] + (double)k_b[c];
        or_rope64(kx, pos[t], rope_theta);
        /* latent row: RMSNorm over c_kv, RoPE on k_pe */
        double ms = 0.0;
        for (int c = 0; c < OR_LATENT; c++) ms += lx[c] * lx[c];
        ms /= OR_LATENT;
        const double rinv = 1.0 / sqrt(ms + kv_eps);
        for (int c = 0; c < OR_LATENT; c++) lx[c] = lx[c] * rinv * (double)kv_g[c];
        or_rope64(lx + OR_LATENT, pos[t], rope_theta);
        memcpy(key + (int64_t)t * OR_IDX_DIM, kx, sizeof kx);
        memcpy(latent + (int64_t)t * OR_ROW, lx, sizeof lx);
    }
}
