/*
 * oracle.c -- plain, slow CPU reference for paged KV-cache attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py use it.  It shares no code with the HIP library.
 *
 * What it computes, and where that is stated:
 *   - A KV cache kept in fixed-size pages ("blocks"); a per-sequence block
 *     table maps logical block j to a physical block id.
 *       tiny-vLLM paper-digest page, "Core Mechanics" (PagedAttention splits
 *       the KV cache into page units); tiny-vllm README (Korean translation),
 *       table of contents "Paged Attention", "Paged KV cache"; the nano-vLLM
 *       guide announcement, ch. 4 "PagedAttention" (virtual memory for the
 *       KV cache).
 *   - Writing each new token's K and V once, so later steps look them up
 *     instead of recomputing them: README table of contents "Why KV cache
 *     exists"; guide ch. 3 "KV Cache".
 *   - Scaled dot-product attention, grouped-query heads, softmax and the
 *     causal mask: README table of contents "Attention", "GQA", "Softmax",
 *     "Causal mask".  The pages name these steps but do not print them, so
 *     the textbook definitions are written out here:
 *         s_j  = scale * sum_d q[d] * k_j[d]
 *         p_j  = exp(s_j - max_i s_i) / sum_i exp(s_i - max_i s_i)
 *         out  = sum_j p_j * v_j
 *     computed in two passes (max first, then exponentials), NOT online.
 *   - The FlashAttention-style online softmax named in the README feature
 *     list and table of contents ("Online softmax") appears here only as a
 *     separate routine (oracle_decode_online) that tests compare against the
 *     two-pass definition.
 *   - Split-context partitions and their log-sum-exp merge are the
 *     online-softmax identity applied to whole partitions; they are written
 *     out (oracle_decode_partials, oracle_lse_merge) so tests can check the
 *     algebra of a split path.
 *
 * Readings taken where the pages are silent:
 *   - pool layout [num_blocks][Hkv][block_size][D] of bf16 bit patterns,
 *     one layout for K and for V;
 *   - query head h reads KV head h / (Hq / Hkv) (contiguous groups);
 *   - context_lens counts the valid tokens of each sequence after this
 *     step's append, and a decode query attends to all of them;
 *   - in causal prefill, query t of sequence b sits at absolute position
 *     context_lens[b] - q_len_b + t and sees keys 0..pos inclusive;
 *   - an empty context gives a zero output row.
 *
 * Arithmetic: bf16 inputs are widened exactly (bits << 16) and every sum,
 * exponential and division is done in double precision, in ascending key
 * and ascending d order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_INPUT (-1)

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Paging: logical token j of a sequence lives in physical block
 * table[j / block_size] at row j % block_size.  Returns the element offset of
 * that token's D-vector for KV head g, or -1 if the table does not cover j. */
static long token_offset(const int32_t *table_row, int32_t max_blocks_per_seq,
                         int32_t num_blocks, int32_t Hkv, int32_t block_size,
                         int32_t D, int32_t g, int32_t j)
{
    int32_t logical_block = j / block_size;
    if (j < 0 || logical_block >= max_blocks_per_seq)
        return -1;
    int32_t phys = table_row[logical_block];
    if (phys < 0 || phys >= num_blocks)
        return -1;
    int32_t row = j % block_size;
    return (((long)phys * Hkv + g) * block_size + row) * (long)D;
}

/* Store each new token's K and V rows at its slot in the paged pools.
 * Token t (0-based) of the n_b new tokens of sequence b has logical
 * position context_lens[b] - n_b + t.  cu_new_lens == NULL means one new
 * token per sequence.  Pure byte copy. */
int oracle_kv_append(uint16_t *k_cache, uint16_t *v_cache,
                     const uint16_t *k_new, const uint16_t *v_new,
                     const int32_t *block_tables, const int32_t *context_lens,
                     const int32_t *cu_new_lens, int32_t B, int32_t Hkv,
                     int32_t D, int32_t block_size, int32_t max_blocks_per_seq,
                     int32_t num_blocks)
{
    for (int32_t b = 0; b < B; b++) {
        int32_t first = cu_new_lens ? cu_new_lens[b] : b;
        int32_t n = cu_new_lens ? cu_new_lens[b + 1] - cu_new_lens[b] : 1;
        for (int32_t t = 0; t < n; t++) {
            int32_t pos = context_lens[b] - n + t;
            const int32_t *row = block_tables + (long)b * max_blocks_per_seq;
            for (int32_t h = 0; h < Hkv; h++) {
                long dst = token_offset(row, max_blocks_per_seq, num_blocks,
                                        Hkv, block_size, D, h, pos);
                if (dst < 0)
                    return ORACLE_BAD_INPUT;
                long src = ((long)(first + t) * Hkv + h) * D;
                memcpy(k_cache + dst, k_new + src, (size_t)D * sizeof(uint16_t));
                memcpy(v_cache + dst, v_new + src, (size_t)D * sizeof(uint16_t));
            }
        }
    }
    return ORACLE_OK;
}

/* Everything one attention row needs to find its keys. */
typedef struct {
    const uint16_t *k_cache, *v_cache;
    const int32_t *table_row;
    int32_t max_blocks_per_seq, num_blocks, Hkv, block_size, D;
} paged_seq;

/* One query vector q[D] of KV group g against logical keys [0, n_keys):
 * two-pass softmax.  out[D] receives the result; zero when n_keys == 0. */
static int attend_two_pass(double *out, const uint16_t *q, const paged_seq *s,
                           int32_t g, int32_t n_keys, double scale)
{
    int32_t D = s->D;
    for (int32_t d = 0; d < D; d++)
        out[d] = 0.0;
    if (n_keys <= 0)
        return ORACLE_OK;

    double *score = (double *)malloc((size_t)n_keys * sizeof(double));
    if (!score)
        return ORACLE_BAD_INPUT;

    /* scores */
    for (int32_t j = 0; j < n_keys; j++) {
        long off = token_offset(s->table_row, s->max_blocks_per_seq,
                                s->num_blocks, s->Hkv, s->block_size, D, g, j);
        if (off < 0) {
            free(score);
            return ORACLE_BAD_INPUT;
        }
        double dot = 0.0;
        for (int32_t d = 0; d < D; d++)
            dot += widen_bf16(q[d]) * widen_bf16(s->k_cache[off + d]);
        score[j] = scale * dot;
    }

    /* pass 1: the maximum score */
    double m = score[0];
    for (int32_t j = 1; j < n_keys; j++)
        if (score[j] > m)
            m = score[j];

    /* pass 2: exponentials and their sum */
    double l = 0.0;
    for (int32_t j = 0; j < n_keys; j++) {
        score[j] = exp(score[j] - m);
        l += score[j];
    }

    /* weighted sum of values with the normalised weights */
    for (int32_t j = 0; j < n_keys; j++) {
        long off = token_offset(s->table_row, s->max_blocks_per_seq,
                                s->num_blocks, s->Hkv, s->block_size, D, g, j);
        double p = score[j] / l;
        for (int32_t d = 0; d < D; d++)
            out[d] += p * widen_bf16(s->v_cache[off + d]);
    }
    free(score);
    return ORACLE_OK;
}

static int check_heads(int32_t Hq, int32_t Hkv)
{
    return (Hq > 0 && Hkv > 0 && Hq % Hkv == 0) ? ORACLE_OK : ORACLE_BAD_INPUT;
}

/* Decode: one query token per sequence, q[B][Hq][D]; it attends to all
 * context_lens[b] keys.  out[B][Hq][D] in double. */
int oracle_decode(double *out, const uint16_t *q, const uint16_t *k_cache,
                  const uint16_t *v_cache, const int32_t *block_tables,
                  const int32_t *context_lens, int32_t B, int32_t Hq,
                  int32_t Hkv, int32_t D, int32_t block_size,
                  int32_t max_blocks_per_seq, int32_t num_blocks, double scale)
{
    if (check_heads(Hq, Hkv) != ORACLE_OK)
        return ORACLE_BAD_INPUT;
    int32_t group = Hq / Hkv;
    for (int32_t b = 0; b < B; b++) {
        paged_seq s = {k_cache, v_cache, block_tables + (long)b * max_blocks_per_seq,
                       max_blocks_per_seq, num_blocks, Hkv, block_size, D};
        for (int32_t h = 0; h < Hq; h++) {
            int rc = attend_two_pass(out + ((long)b * Hq + h) * D,
                                     q + ((long)b * Hq + h) * D, &s, h / group,
                                     context_lens[b], scale);
            if (rc != ORACLE_OK)
                return rc;
        }
    }
    return ORACLE_OK;
}

/* Causal prefill over packed queries q[T][Hq][D]; cu_q_lens[B+1] delimits the
 * sequences.  Query t of sequence b is at absolute position
 * pos = context_lens[b] - q_len_b + t and sees keys 0..pos.  If rows != NULL
 * only the n_rows listed token indices are computed (other rows of out are
 * left untouched); otherwise all T rows are. */
int oracle_prefill_causal(double *out, const uint16_t *q, const uint16_t *k_cache,
                          const uint16_t *v_cache, const int32_t *block_tables,
                          const int32_t *context_lens, const int32_t *cu_q_lens,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t num_blocks, double scale,
                          const int32_t *rows, int32_t n_rows)
{
    if (check_heads(Hq, Hkv) != ORACLE_OK)
        return ORACLE_BAD_INPUT;
    int32_t group = Hq / Hkv;
    int32_t T = cu_q_lens[B];
    int32_t count = rows ? n_rows : T;
    for (int32_t r = 0; r < count; r++) {
        int32_t t = rows ? rows[r] : r;
        if (t < 0 || t >= T)
            return ORACLE_BAD_INPUT;
        int32_t b = 0;
        while (!(cu_q_lens[b] <= t && t < cu_q_lens[b + 1]))
            b++;
        int32_t q_len = cu_q_lens[b + 1] - cu_q_lens[b];
        int32_t pos = context_lens[b] - q_len + (t - cu_q_lens[b]);
        paged_seq s = {k_cache, v_cache, block_tables + (long)b * max_blocks_per_seq,
                       max_blocks_per_seq, num_blocks, Hkv, block_size, D};
        for (int32_t h = 0; h < Hq; h++) {
            int rc = attend_two_pass(out + ((long)t * Hq + h) * D,
                                     q + ((long)t * Hq + h) * D, &s, h / group,
                                     pos + 1, scale);
            if (rc != ORACLE_OK)
                return rc;
        }
    }
    return ORACLE_OK;
}

/* Online (single-pass) softmax, FlashAttention style: a running maximum m,
 * a running sum l and a running weighted value sum acc are rescaled by
 * exp(m_old - m_new) whenever the maximum grows.  Used only to check that it
 * agrees with the two-pass definition above. */
int oracle_decode_online(double *out, const uint16_t *q, const uint16_t *k_cache,
                         const uint16_t *v_cache, const int32_t *block_tables,
                         const int32_t *context_lens, int32_t B, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t block_size,
                         int32_t max_blocks_per_seq, int32_t num_blocks,
                         double scale)
{
    if (check_heads(Hq, Hkv) != ORACLE_OK)
        return ORACLE_BAD_INPUT;
    int32_t group = Hq / Hkv;
    double *acc = (double *)malloc((size_t)D * sizeof(double));
    if (!acc)
        return ORACLE_BAD_INPUT;
    for (int32_t b = 0; b < B; b++) {
        const int32_t *row = block_tables + (long)b * max_blocks_per_seq;
        for (int32_t h = 0; h < Hq; h++) {
            const uint16_t *qv = q + ((long)b * Hq + h) * D;
            double *o = out + ((long)b * Hq + h) * D;
            double m = -INFINITY, l = 0.0;
            for (int32_t d = 0; d < D; d++)
                acc[d] = 0.0;
            for (int32_t j = 0; j < context_lens[b]; j++) {
                long off = token_offset(row, max_blocks_per_seq, num_blocks, Hkv,
                                        block_size, D, h / group, j);
                if (off < 0) {
                    free(acc);
                    return ORACLE_BAD_INPUT;
                }
                double dot = 0.0;
                for (int32_t d = 0; d < D; d++)
                    dot += widen_bf16(qv[d]) * widen_bf16(k_cache[off + d]);
                double s = scale * dot;
                double m_new = s > m ? s : m;
                double alpha = exp(m - m_new); /* 0 on the first key */
                double p = exp(s - m_new);
                l = l * alpha + p;
                for (int32_t d = 0; d < D; d++)
                    acc[d] = acc[d] * alpha + p * widen_bf16(v_cache[off + d]);
                m = m_new;
            }
            for (int32_t d = 0; d < D; d++)
                o[d] = context_lens[b] > 0 ? acc[d] / l : 0.0;
        }
    }
    free(acc);
    return ORACLE_OK;
}

/* Split-context partials: partition p of sequence b holds logical keys
 * [p * partition_size, min((p+1) * partition_size, context_lens[b])).
 * For each (b, h, p): m = max score, l = sum exp(s - m), o = softmax-weighted
 * value mean of that partition alone (o = sum exp(s - m) v / l).
 * An empty partition has m = -inf, l = 0, o = 0.
 * Outputs: o[B][Hq][P][D], m[B][Hq][P], l[B][Hq][P] (natural-log units). */
int oracle_decode_partials(double *o, double *m, double *l, const uint16_t *q,
                           const uint16_t *k_cache, const uint16_t *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t num_blocks, double scale,
                           int32_t partition_size, int32_t P)
{
    if (check_heads(Hq, Hkv) != ORACLE_OK || partition_size <= 0)
        return ORACLE_BAD_INPUT;
    int32_t group = Hq / Hkv;
    for (int32_t b = 0; b < B; b++) {
        const int32_t *row = block_tables + (long)b * max_blocks_per_seq;
        for (int32_t h = 0; h < Hq; h++) {
            const uint16_t *qv = q + ((long)b * Hq + h) * D;
            for (int32_t p = 0; p < P; p++) {
                long idx = ((long)b * Hq + h) * P + p;
                double *op = o + idx * D;
                int32_t j0 = p * partition_size;
                int32_t j1 = j0 + partition_size;
                if (j1 > context_lens[b])
                    j1 = context_lens[b];
                for (int32_t d = 0; d < D; d++)
                    op[d] = 0.0;
                m[idx] = -INFINITY;
                l[idx] = 0.0;
                if (j0 >= j1)
                    continue;
                int32_t n = j1 - j0;
                double *score = (double *)malloc((size_t)n * sizeof(double));
                if (!score)
                    return ORACLE_BAD_INPUT;
                for (int32_t j = j0; j < j1; j++) {
                    long off = token_offset(row, max_blocks_per_seq, num_blocks,
                                            Hkv, block_size, D, h / group, j);
                    if (off < 0) {
                        free(score);
                        return ORACLE_BAD_INPUT;
                    }
                    double dot = 0.0;
                    for (int32_t d = 0; d < D; d++)
                        dot += widen_bf16(qv[d]) * widen_bf16(k_cache[off + d]);
                    score[j - j0] = scale * dot;
                }
                double mx = score[0];
                for (int32_t i = 1; i < n; i++)
                    if (score[i] > mx)
                        mx = score[i];
                double sum = 0.0;
                for (int32_t i = 0; i < n; i++) {
                    score[i] = exp(score[i] - mx);
                    sum += score[i];
                }
                for (int32_t j = j0; j < j1; j++) {
                    long off = token_offset(row, max_blocks_per_seq, num_blocks,
                                            Hkv, block_size, D, h / group, j);
                    for (int32_t d = 0; d < D; d++)
                        op[d] += score[j - j0] / sum * widen_bf16(v_cache[off + d]);
                }
                m[idx] = mx;
                l[idx] = sum;
                free(score);
            }
        }
    }
    return ORACLE_OK;
}

/* Log-sum-exp merge of partials over their P partitions:
 *   M = max_p m_p,  w_p = l_p * exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
 * Rows whose partitions are all empty give zero.  n_rows = B * Hq. */
int oracle_lse_merge(double *out, const double *o, const double *m,
                     const double *l, int32_t n_rows, int32_t P, int32_t D)
{
    for (int32_t r = 0; r < n_rows; r++) {
        double *dst = out + (long)r * D;
        for (int32_t d = 0; d < D; d++)
            dst[d] = 0.0;
        double M = -INFINITY;
        for (int32_t p = 0; p < P; p++)
            if (l[(long)r * P + p] > 0.0 && m[(long)r * P + p] > M)
                M = m[(long)r * P + p];
        if (M == -INFINITY)
            continue;
        double wsum = 0.0;
        for (int32_t p = 0; p < P; p++) {
            double lp = l[(long)r * P + p];
            if (lp <= 0.0)
                continue;
            double w = lp * exp(m[(long)r * P + p] - M);
            wsum += w;
            for (int32_t d = 0; d < D; d++)
                dst[d] += w * o[((long)r * P + p) * D + d];
        }
        for (int32_t d = 0; d < D; d++)
            dst[d] /= wsum;
    }
    return ORACLE_OK;
}

/* ---- Rotary position embedding ------------------------------------------
 *
 * The pages list RoPE among the components of the model they run (README
 * feature list and table of contents "RoPE") but print no formula.  Reading
 * taken: the rotary embedding of that model in the layout of its
 * Safetensors checkpoint, where the rotated pairs are (i, i + D/2): the
 * 2-vector (x[i], x[i + D/2]) is multiplied by the rotation matrix of the
 * position's angle,
 *     [ cos  -sin ] [ x[i]       ]
 *     [ sin   cos ] [ x[i + D/2] ],
 * i.e. the complex number x[i] + i x[i + D/2] times e^(i angle).  The
 * angle's cosine and sine are the caller's tables, indexed [pos][i]; the
 * position of a new token is the kv_append rule above.  Arithmetic in double
 * precision from the widened bf16 inputs and the fp32 table entries. */

/* Absolute position pos[t] and sequence seq[t] of every new token t: token
 * t of the n_b new tokens of sequence b is at context_lens[b] - n_b + t.
 * cu_new_lens == NULL means one new token per sequence (T_new == B). */
int oracle_token_positions(int32_t *pos, int32_t *seq, const int32_t *context_lens,
                           const int32_t *cu_new_lens, int32_t B, int32_t T_new)
{
    for (int32_t b = 0; b < B; b++) {
        int32_t first = cu_new_lens ? cu_new_lens[b] : b;
        int32_t n = cu_new_lens ? cu_new_lens[b + 1] - cu_new_lens[b] : 1;
        if (first < 0 || n < 0 || first + n > T_new)
            return ORACLE_BAD_INPUT;
        for (int32_t t = 0; t < n; t++) {
            pos[first + t] = context_lens[b] - n + t;
            seq[first + t] = b;
        }
    }
    return ORACLE_OK;
}

/* Rotate the rows x[rows][heads][D] (bf16 bits); row r is at position
 * pos[r].  out[rows][heads][D] receives the rotated values. */
int oracle_rope(double *out, const uint16_t *x, const int32_t *pos, const float *cos_tab,
                const float *sin_tab, int32_t rows, int32_t heads, int32_t D,
                int32_t max_position)
{
    if (D <= 0 || D % 2 != 0)
        return ORACLE_BAD_INPUT;
    int32_t half = D / 2;
    for (int32_t r = 0; r < rows; r++) {
        if (pos[r] < 0 || pos[r] >= max_position)
            return ORACLE_BAD_INPUT;
        const float *cr = cos_tab + (long)pos[r] * half;
        const float *sr = sin_tab + (long)pos[r] * half;
        for (int32_t h = 0; h < heads; h++) {
            const uint16_t *src = x + ((long)r * heads + h) * D;
            double *dst = out + ((long)r * heads + h) * D;
            for (int32_t i = 0; i < half; i++) {
                double a = widen_bf16(src[i]), b = widen_bf16(src[i + half]);
                double c = (double)cr[i], s = (double)sr[i];
                dst[i] = a * c - b * s;
                dst[i + half] = b * c + a * s;
            }
        }
    }
    return ORACLE_OK;
}

/* Round doubles to bf16 bit patterns, to nearest with ties to even, straight
 * from the double (no intermediate float rounding): 8 significant bits for
 * normal values, a fixed step of 2^-133 below 2^-126, infinity past the
 * largest finite bf16; NaN gives the quiet NaN 0x7FC0 with its sign. */
int oracle_round_bf16(uint16_t *out, const double *x, long n)
{
    for (long k = 0; k < n; k++) {
        double v = x[k];
        uint16_t sign = signbit(v) ? 0x8000u : 0u;
        double a = fabs(v);
        if (isnan(v)) {
            out[k] = (uint16_t)(sign | 0x7FC0u);
            continue;
        }
        double r;
        if (a < ldexp(1.0, -126)) {
            r = ldexp(nearbyint(ldexp(a, 133)), -133);
        } else {
            int e;
            double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
            r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
        }
        float f = (float)r; /* exact: at most 8 significant bits; inf past the range */
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        out[k] = (uint16_t)(sign | (u >> 16));
    }
    return ORACLE_OK;
}

/* ---- Block copies (copy on write of shared blocks) ------------------------
 * The guide's ch. 7 ("Prefix Caching") shares KV blocks between sequences;
 * a sequence about to write into a shared block first gets its own copy.
 * Block dst[i] of both pools receives the bytes of block src[i] (every KV
 * head and row), in pair order. */
int oracle_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int32_t *src,
                       const int32_t *dst, int32_t n_pairs, int32_t Hkv, int32_t block_size,
                       int32_t D, int32_t num_blocks)
{
    long per_block = (long)Hkv * block_size * D;
    for (int32_t i = 0; i < n_pairs; i++) {
        if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks)
            return ORACLE_BAD_INPUT;
        memcpy(k_cache + dst[i] * per_block, k_cache + src[i] * per_block,
               (size_t)per_block * sizeof(uint16_t));
        memcpy(v_cache + dst[i] * per_block, v_cache + src[i] * per_block,
               (size_t)per_block * sizeof(uint16_t));
    }
    return ORACLE_OK;
}
