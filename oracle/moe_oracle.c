/*
 * moe_oracle.c -- plain, slow, double-precision reference of one routed-expert
 * MoE layer at decode.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load or run this code.  It shares no source with the
 * GPU library: it reads the packed bytes through its own indexing below.
 *
 * What one layer computes, per token (sources are the pages' own wording,
 * restated):
 *   - router logits from an 8-bit router held in memory
 *       (TurboFieldfare article, "Arsitektur eksekusi ..." and
 *        "Proses pembuatan token": the router is 8-bit and runs on resident
 *        weights; Colibri analysis report section 2, "Route")
 *   - exact top-8 selection of routed experts
 *       (Inferno README, "Current Scope"; TurboFieldfare, "Proses pembuatan
 *        token": the 8 top expert ids; Colibri analysis section 3: exact
 *        routing semantics by default)
 *   - gate weights renormalised over the selected experts (softmax over the
 *     selected logits; the pages name no formula, this is the plainest reading)
 *   - per selected expert, its gate, up and down matrices (Inferno README,
 *     "Model": each routed expert's gate/up/down stored next to each other),
 *     dequantised on use from affine 4-bit, group 64, one scale and one bias
 *     per group (TurboFieldfare, "Arsitektur eksekusi ...": MLX affine 4-bit
 *     group 64; Colibri README, "What's implemented": dequant-on-use), then
 *     h = silu(G x) * (U x) and y_e = D h
 *   - an always-resident shared expert whose output is added to the routed
 *     outputs (TurboFieldfare, "Proses pembuatan token": shared-expert branch,
 *     then shared and routed outputs combined)
 *   - y = sum_j w_j y_{S_j} + y_shared
 *
 * Parity status of each function is listed in its comment; all are pinned by
 * tests/test_oracle_pins.py except where it says "parity unpinned".
 *
 * Packed expert record (hidden H, intermediate I, both multiples of 64).
 * G and U are [I][H] (input dim H), D is [H][I] (input dim I).  A weight is
 * W = scale * q + bias, q the code (0..15 for 4-bit records, 0..3 for 2-bit),
 * with one fp16 (scale, bias) pair per row and per group of 64 inputs.
 *
 * The record is a sequence of 3*H*I/4096 segments.  A segment covers one tile
 * of 64 rows x 64 inputs: its codes (2048 bytes at 4 bits, 1024 at 2 bits),
 * then 256 bytes of (scale, bias) pairs, one per row r < 64, in row order.
 *   gate/up segments first: segment b*(H/64) + g, for b < I/32, g < H/64:
 *     tile row r < 32 is G row 32b+r, r >= 32 is U row 32b+r-32; inputs
 *     [64g, 64g+64) of H
 *   down segments next: segment (I/32)*(H/64) + t*(I/64) + g, for t < H/64,
 *     g < I/64: tile row r is D row 64t+r; inputs [64g, 64g+64) of I
 * Codes of a segment, 4-bit: [half c < 2][row r < 64][16 bytes], the 16 bytes
 * holding inputs [64g+32c, 64g+32c+32) of row r, input 2m of those 32 in the
 * low nibble of byte m and 2m+1 in its high nibble.  2-bit (our own format:
 * the pages name 2-bit models but define no 2-bit container): [row r < 64][16
 * bytes] holding inputs [64g, 64g+64), input 4m+j in bits [2j, 2j+2) of byte m.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads used by the row loops; returns the count in effect (1 without OpenMP). */
int oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ---- number formats --------------------------------------------------- */

/* IEEE binary16 -> double, exactly (normals, subnormals, zeros, inf, nan). */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int mant = h & 0x3FF;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);                 /* subnormal: m * 2^-24 */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(mant + 1024), expo - 25);  /* (1024+m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* bfloat16 -> double, exactly: bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Activations in the layer's dtype (0 = fp32, 1 = bf16 bits) -> double. */
void oracle_act_to_f64(int act_dtype, const void *x, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) {
        if (act_dtype == 0)
            out[i] = (double)((const float *)x)[i];
        else
            out[i] = oracle_bf16_to_f64(((const uint16_t *)x)[i]);
    }
}

/* ---- packed record indexing (see the header comment) ------------------- */

static int nibble_at(const uint8_t *rec, size_t byte_off, int elem)
{
    uint8_t byte = rec[byte_off];
    return (elem & 1) ? (byte >> 4) : (byte & 0x0F);
}

/* bytes of a segment's codes, and of a whole segment (codes + 64 pairs) */
static size_t seg_codes(int bits) { return bits == 2 ? 1024 : 2048; }
static size_t seg_bytes(int bits) { return seg_codes(bits) + 256; }

/* start of gate/up segment (b, g) and of down segment (t, g) */
static size_t gu_segment(int bits, int H, int b, int g)
{
    return ((size_t)b * (H / 64) + g) * seg_bytes(bits);
}

static size_t d_segment(int bits, int H, int I, int t, int g)
{
    return ((size_t)(I / 32) * (H / 64) + (size_t)t * (I / 64) + g) * seg_bytes(bits);
}

/* quantised value of gate (which = 0) or up (which = 1) at row i, input k */
static int q_gate_up(const uint8_t *rec, int H, int which, int i, int k)
{
    int b = i / 32, r = i % 32 + 32 * which, g = k / 64, c = (k % 64) / 32, e = k % 32;
    size_t off = gu_segment(4, H, b, g) + (size_t)c * 1024 + (size_t)r * 16 + e / 2;
    return nibble_at(rec, off, e);
}

static int q_down(const uint8_t *rec, int H, int I, int o, int i)
{
    int t = o / 64, r = o % 64, g = i / 64, c = (i % 64) / 32, e = i % 32;
    size_t off = d_segment(4, H, I, t, g) + (size_t)c * 1024 + (size_t)r * 16 + e / 2;
    return nibble_at(rec, off, e);
}

/* 2-bit codes: input e of a run sits in bits [2(e%4), 2(e%4)+2) of byte e/4 */
static int crumb_at(const uint8_t *rec, size_t byte_off, int elem)
{
    return (rec[byte_off] >> (2 * (elem & 3))) & 3;
}

static int q_gate_up2(const uint8_t *rec, int H, int which, int i, int k)
{
    int b = i / 32, r = i % 32 + 32 * which, g = k / 64, e = k % 64;
    size_t off = gu_segment(2, H, b, g) + (size_t)r * 16 + e / 4;
    return crumb_at(rec, off, e);
}

static int q_down2(const uint8_t *rec, int H, int I, int o, int i)
{
    int t = o / 64, r = o % 64, g = i / 64, e = i % 64;
    size_t off = d_segment(2, H, I, t, g) + (size_t)r * 16 + e / 4;
    return crumb_at(rec, off, e);
}

/* the code width in use: 4 (nibbles) or 2 */
static int q_gu(int bits, const uint8_t *rec, int H, int which, int i, int k)
{
    return bits == 2 ? q_gate_up2(rec, H, which, i, k) : q_gate_up(rec, H, which, i, k);
}

static int q_d(int bits, const uint8_t *rec, int H, int I, int o, int i)
{
    return bits == 2 ? q_down2(rec, H, I, o, i) : q_down(rec, H, I, o, i);
}

static void sb_read(const uint8_t *rec, size_t off, double *s, double *bias)
{
    uint16_t sv, bv;
    memcpy(&sv, rec + off, 2);
    memcpy(&bv, rec + off + 2, 2);
    *s = oracle_f16_to_f64(sv);
    *bias = oracle_f16_to_f64(bv);
}

/* scale/bias of gate (which = 0) or up (which = 1) row i, input group h */
static void sb_gate_up(int bits, const uint8_t *rec, int H, int which, int i, int h,
                       double *s, double *bias)
{
    int b = i / 32, r = i % 32 + 32 * which;
    size_t off = gu_segment(bits, H, b, h) + seg_codes(bits) + (size_t)r * 4;
    sb_read(rec, off, s, bias);
}

/* scale/bias of down row o, input group g */
static void sb_down(int bits, const uint8_t *rec, int H, int I, int o, int g, double *s, double *bias)
{
    size_t off = d_segment(bits, H, I, o / 64, g) + seg_codes(bits) + (size_t)(o % 64) * 4;
    sb_read(rec, off, s, bias);
}

size_t oracle_record_bytes_bits(int bits, int H, int I)
{
    return (size_t)3 * (H / 64) * (I / 64) * seg_bytes(bits);
}

size_t oracle_record_bytes(int H, int I) { return oracle_record_bytes_bits(4, H, I); }

/* Dense dequantisation of one record: W = scale * q + bias per 64-group of the
 * input dim.  G, U are [I][H] row-major, D is [H][I].  Pinned against an
 * independently written packer and its dense source matrices. */
void oracle_dequant_record_bits(int bits, int H, int I, const uint8_t *rec, double *G, double *U,
                                double *D)
{
    double s, bias;
    for (int i = 0; i < I; ++i)
        for (int k = 0; k < H; ++k) {
            sb_gate_up(bits, rec, H, 0, i, k / 64, &s, &bias);
            G[(size_t)i * H + k] = s * q_gu(bits, rec, H, 0, i, k) + bias;
            sb_gate_up(bits, rec, H, 1, i, k / 64, &s, &bias);
            U[(size_t)i * H + k] = s * q_gu(bits, rec, H, 1, i, k) + bias;
        }
    for (int o = 0; o < H; ++o)
        for (int i = 0; i < I; ++i) {
            sb_down(bits, rec, H, I, o, i / 64, &s, &bias);
            D[(size_t)o * I + i] = s * q_d(bits, rec, H, I, o, i) + bias;
        }
}

void oracle_dequant_record(int H, int I, const uint8_t *rec, double *G, double *U, double *D)
{
    oracle_dequant_record_bits(4, H, I, rec, G, U, D);
}

/* ---- the layer --------------------------------------------------------- */

/* Router: logit_e = scale_e * sum_h q[e][h] * x_h  (8-bit rows, one fp16 scale
 * per row, scale applied after the sum).  TurboFieldfare article, "Arsitektur
 * eksekusi ...": the router is 8-bit. */
void oracle_router_logits(int H, int E, const int8_t *rq, const uint16_t *rs,
                          const double *x, double *logits)
{
    #pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h)
            acc += (double)rq[(size_t)e * H + h] * x[h];
        logits[e] = oracle_f16_to_f64(rs[e]) * acc;
    }
}

/* Exact top-k: the first k experts in the order (logit descending, then id
 * ascending).  Inferno README "Current Scope" and TurboFieldfare "Proses
 * pembuatan token" fix k = 8 and exact (not approximate) selection. */
void oracle_select_topk(int E, int k, const double *logits, int32_t *ids)
{
    char *taken = (char *)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || logits[e] > logits[best])
                best = e;            /* strict '>' keeps the lower id on ties */
        }
        taken[best] = 1;
        ids[j] = best;
    }
    free(taken);
}

/* Gate weights renormalised over the selected experts:
 * w_j = exp(l_j - m) / sum_{j'} exp(l_j' - m), m = max of the selected logits.
 * (Equal to a softmax over all experts, renormalised over the selection.) */
void oracle_softmax_gates(int k, const double *sel_logits, double *w)
{
    double m = sel_logits[0], z = 0.0;
    for (int j = 1; j < k; ++j)
        if (sel_logits[j] > m)
            m = sel_logits[j];
    for (int j = 0; j < k; ++j) {
        w[j] = exp(sel_logits[j] - m);
        z += w[j];
    }
    for (int j = 0; j < k; ++j)
        w[j] /= z;
}

/* Sigmoid router with a selection bias and a routed scaling factor: the
 * DeepSeek-V3-style router that the Colibri README ("What's implemented")
 * names for GLM (noaux_tc, routed_scaling_factor); the pages give no formula,
 * so this is the published scheme's plainest reading:
 *   score s_e = 1 / (1 + exp(-l_e));
 *   selection: the k largest keys s_e + b_e (b = per-expert correction bias,
 *     zero when bias is NULL), in the order (key descending, id ascending);
 *   gates from the unbiased scores of the selection,
 *     w_j = scale * s_{S_j} / sum_{j'} s_{S_j'}.
 * Group-limited selection is not modelled (a single group). */
void oracle_sigmoid_route(int E, int k, const double *logits, const double *bias,
                          double scale, int32_t *ids, double *w)
{
    double *key = (double *)malloc(sizeof(double) * (size_t)E);
    for (int e = 0; e < E; ++e)
        key[e] = 1.0 / (1.0 + exp(-logits[e])) + (bias ? bias[e] : 0.0);
    oracle_select_topk(E, k, key, ids);
    double z = 0.0;
    for (int j = 0; j < k; ++j) {
        w[j] = 1.0 / (1.0 + exp(-logits[ids[j]]));
        z += w[j];
    }
    for (int j = 0; j < k; ++j)
        w[j] = scale * (w[j] / z);
    free(key);
}

double oracle_silu(double v) { return v / (1.0 + exp(-v)); }

/* One expert's SwiGLU FFN on a dequantised-on-use record:
 *   g = G x, u = U x, h = silu(g) * u, y = D h.
 * Each 64-input group's scale and bias are decoded once and applied to every
 * element of the group as W = scale * q + bias.  Rows are independent, so the
 * row loops may run on several threads (OpenMP) without changing any sum.
 * Optional outputs g, u, h (length I) for the pins; pass NULL to skip. */
void oracle_expert_ffn_bits(int bits, int H, int I, const uint8_t *rec, const double *x,
                            double *y, double *g_out, double *u_out, double *h_out)
{
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0, sg, bg, su, bu;
        for (int grp = 0; grp < H / 64; ++grp) {
            sb_gate_up(bits, rec, H, 0, i, grp, &sg, &bg);
            sb_gate_up(bits, rec, H, 1, i, grp, &su, &bu);
            for (int k = 64 * grp; k < 64 * grp + 64; ++k) {
                g += (sg * q_gu(bits, rec, H, 0, i, k) + bg) * x[k];
                u += (su * q_gu(bits, rec, H, 1, i, k) + bu) * x[k];
            }
        }
        h[i] = oracle_silu(g) * u;
        if (g_out) g_out[i] = g;
        if (u_out) u_out[i] = u;
        if (h_out) h_out[i] = h[i];
    }
    #pragma omp parallel for schedule(static)
    for (int o = 0; o < H; ++o) {
        double acc = 0.0, s, bias;
        for (int grp = 0; grp < I / 64; ++grp) {
            sb_down(bits, rec, H, I, o, grp, &s, &bias);
            for (int i = 64 * grp; i < 64 * grp + 64; ++i)
                acc += (s * q_d(bits, rec, H, I, o, i) + bias) * h[i];
        }
        y[o] = acc;
    }
    free(h);
}

void oracle_expert_ffn(int H, int I, const uint8_t *rec, const double *x, double *y,
                       double *g_out, double *u_out, double *h_out)
{
    oracle_expert_ffn_bits(4, H, I, rec, x, y, g_out, u_out, h_out);
}

/* y = sum_j w_j * y_routed[j] + y_shared, summed in the order j = 0..k-1 and
 * then the shared expert (weight 1, no gate).  y_shared may be NULL. */
void oracle_combine(int k, int H, const double *w, const double *y_routed,
                    const double *y_shared, double *y)
{
    for (int o = 0; o < H; ++o) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j)
            acc += w[j] * y_routed[(size_t)j * H + o];
        if (y_shared)
            acc += y_shared[o];
        y[o] = acc;
    }
}

/* A whole layer for one token, with every routed record reachable at
 * pool + e * record_bytes(H, I).  shared may be NULL (no shared expert).
 * Writes ids[k], w[k], y[H] and, if logits != NULL, logits[E]. */
void oracle_layer_token(int H, int E, int I, int k, int I_shared,
                        const int8_t *rq, const uint16_t *rs,
                        const uint8_t *pool, const uint8_t *shared,
                        const double *x, int32_t *ids, double *w, double *y,
                        double *logits)
{
    double *lg = (double *)malloc(sizeof(double) * (size_t)E);
    double *sel = (double *)malloc(sizeof(double) * (size_t)k);
    double *yr = (double *)malloc(sizeof(double) * (size_t)k * H);
    double *ys = shared ? (double *)malloc(sizeof(double) * (size_t)H) : NULL;
    size_t rb = oracle_record_bytes(H, I);

    oracle_router_logits(H, E, rq, rs, x, lg);
    oracle_select_topk(E, k, lg, ids);
    for (int j = 0; j < k; ++j)
        sel[j] = lg[ids[j]];
    oracle_softmax_gates(k, sel, w);
    for (int j = 0; j < k; ++j)
        oracle_expert_ffn(H, I, pool + (size_t)ids[j] * rb, x, yr + (size_t)j * H,
                          NULL, NULL, NULL);
    if (shared)
        oracle_expert_ffn(H, I_shared, shared, x, ys, NULL, NULL, NULL);
    oracle_combine(k, H, w, yr, ys, y);
    if (logits)
        memcpy(logits, lg, sizeof(double) * (size_t)E);
    free(lg); free(sel); free(yr); free(ys);
}
