/*
 * CPU oracle for absorbed Multi-head Latent Attention (MLA) over a latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the GPU
 * library is checked against.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header or table with the GPU
 * library (deepseek_mla_amd/csrc).
 *
 * Source of the method: the page "ik_llama.cpp MLA matrix absorption ..."
 * (czykbl.com/news/93068), sections 1 (low-rank KV compression and explicit
 * decompression), 3 (K absorption), 4 (V absorption, late decompression, the three
 * einsum forms), 5 (move elision: scores as a RoPE term plus a latent term).
 *
 * Precision: float32 inputs and outputs; every dot product, softmax sum and GEMM
 * accumulates in double.  RoPE angles are computed in double.
 *
 * Layouts (row-major, innermost last):
 *   q_nope [T][H][Dn], q_rope [T][H][Dr], pos [T], wk_b [H][R][Dn], wv_b [H][Dv][R],
 *   wo [D][H*Dv] (input column h*Dv+d), cache rows [N][R+Dr] = [c_kv | k_rope],
 *   q_cat [T][H][R+Dr] = [q_lat | RoPE(q_rope)], o_lat [T][H][R], lse [T][H].
 * The wk_b / wv_b layouts are the split-tensor layouts of the page
 * "ik_llama.cpp PR #394" section 3.2 (ggml {Dn,R,H} and {R,Dv,H}).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Thread count of the parallel loops below (the timing of the CPU baseline sets it;
 * results do not depend on it: every output element is summed by one thread). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- RoPE ---
 * Rotary position embedding of one vector of even length dr at position pos.
 * Pair i = (x[2i], x[2i+1]) is rotated by angle pos * base^(-2i/dr), the
 * original RoPE formulation with adjacent pairs.  The pages fix no pairing
 * convention; this is the reading used everywhere in this project. */
void orc_rope(const float *x, int dr, double pos, double base, float *y)
{
    for (int i = 0; i < dr / 2; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)dr);
        double ang = pos * theta;
        double c = cos(ang), s = sin(ang);
        double a = x[2 * i], b = x[2 * i + 1];
        y[2 * i] = (float)(a * c - b * s);
        y[2 * i + 1] = (float)(a * s + b * c);
    }
}

/* ------------------------------------------------------ K absorption ---
 * Section 3 of the absorption page: q^T k = q_nope^T W_UK c, so the nope query
 * is projected into the latent space once: q_lat[l] = sum_d wk_b[h][l][d] *
 * q_nope[d] (the mul_mat(wk_b, q_nope) of section 4).  The RoPE query part is
 * not absorbable (RoPE breaks associativity) and is rotated and kept apart.
 * Writes q_cat[t][h] = [q_lat | RoPE(q_rope, pos[t])]. */
void orc_absorb_q(int H, int R, int Dn, int Dr, double rope_base,
                  const float *q_nope, const float *q_rope, const int32_t *pos,
                  const float *wk_b, int T, float *q_cat)
{
    const int W = R + Dr;
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            const float *qn = q_nope + ((size_t)t * H + h) * Dn;
            const float *qr = q_rope + ((size_t)t * H + h) * Dr;
            float *out = q_cat + ((size_t)t * H + h) * W;
            for (int l = 0; l < R; ++l) {
                const float *w = wk_b + ((size_t)h * R + l) * Dn;
                double acc = 0.0;
                for (int d = 0; d < Dn; ++d)
                    acc += (double)w[d] * (double)qn[d];
                out[l] = (float)acc;
            }
            orc_rope(qr, Dr, (double)pos[t], rope_base, out + R);
        }
    }
}

/* ------------------------------------------ attention on the latent cache ---
 * Sections 4 and 5 of the absorption page.  For query row (t, h):
 *   s_j = scale * (q_lat . c_kv[j] + q_rope' . k_rope[j])   for visible j,
 * the two-term score of "move elision" (section 5) computed over the adjacent
 * [c_kv | k_rope] parts of cache row j.  Key j is visible iff j <= pos[t] and
 * j < N (causal; the query's own latent is already in the cache).
 *   p_j = exp(s_j - m) / Z,   m = max_j s_j,   Z = sum_j exp(s_j - m)
 *   o_lat = sum_j p_j c_kv[j]     (einsum bhql,blc->bhqc of section 4)
 *   lse   = m + ln Z
 * A row with no visible key gets o_lat = 0 and lse = -inf.
 * Scores are held in a double buffer of N entries per thread. */
void orc_attention(int H, int R, int Dr, double scale,
                   const float *q_cat, const int32_t *pos, int T,
                   const float *cache, int N, float *o_lat, float *lse)
{
    const int W = R + Dr;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)R);
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int t = 0; t < T; ++t) {
            for (int h = 0; h < H; ++h) {
                const float *q = q_cat + ((size_t)t * H + h) * W;
                int nvis = pos[t] + 1;
                if (nvis > N) nvis = N;
                if (nvis < 0) nvis = 0;
                float *orow = o_lat + ((size_t)t * H + h) * R;
                if (nvis == 0) {
                    for (int l = 0; l < R; ++l) orow[l] = 0.0f;
                    if (lse) lse[(size_t)t * H + h] = -INFINITY;
                    continue;
                }
                double m = -INFINITY;
                for (int j = 0; j < nvis; ++j) {
                    const float *row = cache + (size_t)j * W;
                    double lat = 0.0, rot = 0.0;
                    for (int l = 0; l < R; ++l) lat += (double)q[l] * (double)row[l];
                    for (int r = 0; r < Dr; ++r) rot += (double)q[R + r] * (double)row[R + r];
                    s[j] = scale * (lat + rot);
                    if (s[j] > m) m = s[j];
                }
                double Z = 0.0;
                for (int j = 0; j < nvis; ++j) {
                    s[j] = exp(s[j] - m);
                    Z += s[j];
                }
                for (int l = 0; l < R; ++l) o[l] = 0.0;
                for (int j = 0; j < nvis; ++j) {
                    const float *row = cache + (size_t)j * W;
                    double p = s[j] / Z;
                    for (int l = 0; l < R; ++l) o[l] += p * (double)row[l];
                }
                for (int l = 0; l < R; ++l) orow[l] = (float)o[l];
                if (lse) lse[(size_t)t * H + h] = (float)(m + log(Z));
            }
        }
        free(s);
        free(o);
    }
}

/* --------------------------------------------- late V decompression + wo ---
 * Section 4 of the absorption page: the weighted sum stays latent and wv_b is
 * applied afterwards, v[t][h][d] = sum_l wv_b[h][d][l] o_lat[t][h][l]
 * (einsum bhqc,hdc->bhqd), then out[t][e] = sum_{h,d} wo[e][h*Dv+d] v[t][h][d]
 * (einsum hdD,bhqd->bqD; the heads are concatenated as in reshape_2d to
 * n_embd_head_v*n_head).  v may be NULL. */
void orc_out_proj(int H, int R, int Dv, int D, const float *o_lat, const float *wv_b,
                  const float *wo, int T, float *v, float *out)
{
    const int HDv = H * Dv;
    double *vd = (double *)malloc(sizeof(double) * (size_t)T * HDv);
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h)
            for (int d = 0; d < Dv; ++d) {
                const float *w = wv_b + ((size_t)h * Dv + d) * R;
                const float *o = o_lat + ((size_t)t * H + h) * R;
                double acc = 0.0;
                for (int l = 0; l < R; ++l) acc += (double)w[l] * (double)o[l];
                vd[(size_t)t * HDv + h * Dv + d] = acc;
                if (v) v[(size_t)t * HDv + h * Dv + d] = (float)acc;
            }
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < D; ++e) {
            const float *w = wo + (size_t)e * HDv;
            double acc = 0.0;
            for (int k = 0; k < HDv; ++k) acc += (double)w[k] * vd[(size_t)t * HDv + k];
            out[(size_t)t * D + e] = (float)acc;
        }
    free(vd);
}

/* ------------------------------------------------ unabsorbed reference ---
 * Section 1 of the absorption page ("standard" MLA, mode 0): decompress every
 * cached latent explicitly, k_nope[j][h] = W_UK[h] c_kv[j] with
 * W_UK[h][d][l] = wk_b[h][l][d], and v[j][h] = wv_b[h] c_kv[j]; then ordinary
 * multi-head attention with K = [k_nope | k_rope] (Dn+Dr wide) and
 * Q = [q_nope | RoPE(q_rope)], the same scale and causal rule, and
 * out = wo . concat_h(O).  Written independently of the absorbed functions so
 * that their agreement is the associativity identity of section 3.
 * attn_v [T][H][Dv] (may be NULL), out [T][D]. */
void orc_mla_unabsorbed(int H, int R, int Dn, int Dr, int Dv, int D, double scale,
                        double rope_base, const float *q_nope, const float *q_rope,
                        const int32_t *pos, int T, const float *cache, int N,
                        const float *wk_b, const float *wv_b, const float *wo,
                        float *attn_v, float *out)
{
    const int W = R + Dr;
    const int HDv = H * Dv;
    double *K = (double *)malloc(sizeof(double) * (size_t)N * H * Dn);
    double *V = (double *)malloc(sizeof(double) * (size_t)N * H * Dv);
    double *O = (double *)malloc(sizeof(double) * (size_t)T * HDv);
#pragma omp parallel for collapse(2) schedule(static)
    for (int j = 0; j < N; ++j)
        for (int h = 0; h < H; ++h) {
            const float *c = cache + (size_t)j * W;
            for (int d = 0; d < Dn; ++d) {
                double acc = 0.0;
                for (int l = 0; l < R; ++l)
                    acc += (double)wk_b[((size_t)h * R + l) * Dn + d] * (double)c[l];
                K[((size_t)j * H + h) * Dn + d] = acc;
            }
            for (int d = 0; d < Dv; ++d) {
                double acc = 0.0;
                for (int l = 0; l < R; ++l)
                    acc += (double)wv_b[((size_t)h * Dv + d) * R + l] * (double)c[l];
                V[((size_t)j * H + h) * Dv + d] = acc;
            }
        }
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        float *qr = (float *)malloc(sizeof(float) * (size_t)Dr);
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h) {
                const float *qn = q_nope + ((size_t)t * H + h) * Dn;
                orc_rope(q_rope + ((size_t)t * H + h) * Dr, Dr, (double)pos[t], rope_base, qr);
                int nvis = pos[t] + 1;
                if (nvis > N) nvis = N;
                if (nvis < 0) nvis = 0;
                double *o = O + (size_t)t * HDv + (size_t)h * Dv;
                for (int d = 0; d < Dv; ++d) o[d] = 0.0;
                if (nvis == 0) continue;
                double m = -INFINITY;
                for (int j = 0; j < nvis; ++j) {
                    const double *k = K + ((size_t)j * H + h) * Dn;
                    const float *kr = cache + (size_t)j * W + R;
                    double acc = 0.0;
                    for (int d = 0; d < Dn; ++d) acc += (double)qn[d] * k[d];
                    for (int r = 0; r < Dr; ++r) acc += (double)qr[r] * (double)kr[r];
                    s[j] = scale * acc;
                    if (s[j] > m) m = s[j];
                }
                double Z = 0.0;
                for (int j = 0; j < nvis; ++j) {
                    s[j] = exp(s[j] - m);
                    Z += s[j];
                }
                for (int j = 0; j < nvis; ++j) {
                    const double *v = V + ((size_t)j * H + h) * Dv;
                    for (int d = 0; d < Dv; ++d) o[d] += s[j] / Z * v[d];
                }
            }
        free(s);
        free(qr);
    }
    if (attn_v)
        for (size_t i = 0; i < (size_t)T * HDv; ++i) attn_v[i] = (float)O[i];
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < D; ++e) {
            double acc = 0.0;
            for (int k = 0; k < HDv; ++k)
                acc += (double)wo[(size_t)e * HDv + k] * O[(size_t)t * HDv + k];
            out[(size_t)t * D + e] = (float)acc;
        }
    free(K);
    free(V);
    free(O);
}

/* ------------------------------------------------------- IEEE half ---
 * binary16 <-> binary32 conversion from the IEEE 754 encoding (1 sign bit,
 * 5 exponent bits with bias 15, 10 fraction bits), round to nearest even. */
float orc_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + (double)f, e - 25); /* (1 + f/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

uint16_t orc_float_to_half(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return sign | 0x7E00;
    if (a == 0.0) return sign;
    /* value = a; find the binary16 quantum for its binade */
    int e2;
    frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1) -> unbiased exponent e2-1 */
    int ue = e2 - 1;
    if (ue < -14) ue = -14; /* subnormal range shares the quantum 2^-24 */
    double quantum = ldexp(1.0, ue - 10);
    double n = a / quantum; /* exact: power-of-two scaling */
    double fl = floor(n);
    double rem = n - fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * quantum;
    if (r >= 65520.0 || r > 65504.0) return sign | 0x7C00; /* overflow to inf */
    /* encode r */
    if (r < ldexp(1.0, -14)) return sign | (uint16_t)(r / ldexp(1.0, -24));
    int re;
    double rm = frexp(r, &re); /* r = rm * 2^re */
    int be = re - 1 + 15;
    uint16_t frac = (uint16_t)((rm * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)(be << 10) | frac;
}

/* ------------------------------------------------------------- Q8_0 ---
 * 8-bit latent cache (the Q8_0 KV cache of the absorption page's section 8.1,
 * PR 206, used with -ctk q8_0 in the DeepSeek-V3 run of the KV-cache-rm page).
 * Each run of 32 values is one 34-byte block: a binary16 scale d (little
 * endian) followed by 32 signed 8-bit codes, value = d * code.  A 576-wide
 * row is 18 blocks = 612 bytes.  Quantizer (the pages fix only the format):
 * amax = max |x| over the block, d = amax / 127 in float32,
 * code = round-half-away-from-zero(x / d) clamped to [-127, 127] (0 if d == 0),
 * stored scale = binary16(d) rounded to nearest even. */
void orc_q8_0_quantize(const float *x, int64_t n_rows, int width, uint8_t *out)
{
    const int nb = width / 32;
    const size_t row_bytes = (size_t)nb * 34;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const float *v = x + (size_t)r * width + (size_t)b * 32;
            uint8_t *blk = out + (size_t)r * row_bytes + (size_t)b * 34;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            uint16_t hd = orc_float_to_half(d);
            blk[0] = (uint8_t)(hd & 0xFF);
            blk[1] = (uint8_t)(hd >> 8);
            for (int i = 0; i < 32; ++i) {
                int q = 0;
                if (d != 0.0f) {
                    float y = v[i] / d; /* float32 quotient, correctly rounded */
                    double ry = (y >= 0.0f) ? floor((double)y + 0.5) : -floor(-(double)y + 0.5);
                    if (ry > 127.0) ry = 127.0;
                    if (ry < -127.0) ry = -127.0;
                    q = (int)ry;
                }
                blk[2 + i] = (uint8_t)(int8_t)q;
            }
        }
    }
}

void orc_q8_0_dequantize(const uint8_t *in, int64_t n_rows, int width, float *out)
{
    const int nb = width / 32;
    const size_t row_bytes = (size_t)nb * 34;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r)
        for (int b = 0; b < nb; ++b) {
            const uint8_t *blk = in + (size_t)r * row_bytes + (size_t)b * 34;
            float d = orc_half_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int i = 0; i < 32; ++i)
                out[(size_t)r * width + (size_t)b * 32 + i] = d * (float)(int8_t)blk[2 + i];
        }
}

/* ------------------------------------------------- head-chunk planner ---
 * The -amb rule of the absorption page, section 8.3: when the K x Q
 * intermediate (size_mib) exceeds the cap, use the smallest iteration count
 * niter >= 2 that divides n_head and brings size/niter within the cap, and
 * process n_head/niter heads per iteration; if none qualifies, one head at a
 * time.  cap 0 means unlimited; a cap in (0, 128) is raised to 128 (the
 * KV-cache-rm page's parameter table).  Returns heads per chunk. */
int orc_heads_per_chunk(int n_head, double size_mib, int cap_mib)
{
    if (cap_mib <= 0) return n_head;
    if (cap_mib < 128) cap_mib = 128;
    if (!(size_mib > (double)cap_mib)) return n_head;
    int n_max_head = 1;
    for (int niter = 2; niter <= n_head; ++niter) {
        if (n_head % niter == 0 && size_mib / niter <= (double)cap_mib) {
            n_max_head = n_head / niter;
            break;
        }
    }
    return n_max_head;
}
