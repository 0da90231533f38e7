/*
 * CPU oracle for the routed mixture-of-experts FFN over block-scaled FP4
 * expert weights.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain reference that the
 * GPU path is checked against. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header, table
 * or constant generator with the GPU library, and the GPU library never
 * calls it.
 *
 * Sources (cited by title and section):
 *  [Q] "Running a 133 GB MoE model on an 8 GB GPU at 11 tokens/s by streaming
 *      experts from NVMe" (aiwithghost.com).
 *  [D] "Running the 510 GB DeepSeek-V4.1-Flash on an 8 GB GPU, and three bugs
 *      that never raise an error" (dev.to).
 *  [OCP-FP8] OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding.
 *  [OCP-MX]  OCP Microscaling Formats (MX) Specification v1.0: E2M1 element
 *            encoding, E8M0 scale, and the conversion of a block of values.
 *
 * Arithmetic: weights are dequantised to fp32 by the closed-form decode of
 * each code (no lookup tables shared with anyone); matrix-vector products,
 * SiLU, softmax and the combine run in fp64.
 *
 * Parity pins: see tests/test_oracle_*.py. Every function here is pinned by
 * closed forms, exhaustive enumeration against library decoders, brute force
 * on tiny inputs, or integer-exact special cases; none is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_NVFP4 1 /* e2m1 codes, one E4M3 scale per 16 codes */
#define ORC_MXFP4 2 /* e2m1 codes, one UE8M0 scale per 32 codes */

/* ------------------------------------------------------------------------ */
/* Formats                                                                   */
/* ------------------------------------------------------------------------ */

/* E2M1 ([OCP-MX] element format FP4): 1 sign bit, 2 exponent bits (bias 1),
 * 1 mantissa bit; exponent 0 is subnormal with value 0.5 * m. Magnitudes of
 * the codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6; code 8 is -0. */
double orc_e2m1(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3 ([OCP-FP8] E4M3, the "FN" variant: no infinities): 1 sign bit,
 * 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal
 * (M/8) * 2^-6; S.1111.111 is NaN. This is the per-16 scale of NVFP4 ([Q]
 * "The engine", item 4). */
double orc_e4m3(int byte)
{
    int s = (byte >> 7) & 1, E = (byte >> 3) & 15, M = byte & 7;
    double mag;
    if (E == 15 && M == 7)
        return NAN;
    if (E == 0)
        mag = ldexp(M / 8.0, -6);
    else
        mag = ldexp(1.0 + M / 8.0, E - 7);
    return s ? -mag : mag;
}

/* UE8M0 ([OCP-MX] E8M0 scale; "ue8m0" in [D] "Three bugs", item 2):
 * unsigned exponent with bias 127, 0xFF is NaN. */
double orc_ue8m0(int byte)
{
    if ((byte & 0xFF) == 0xFF)
        return NAN;
    return ldexp(1.0, (byte & 0xFF) - 127);
}

static int group_of(int fmt) { return fmt == ORC_NVFP4 ? 16 : 32; }

static double scale_value(int fmt, int byte)
{
    return fmt == ORC_NVFP4 ? orc_e4m3(byte) : orc_ue8m0(byte);
}

/* ------------------------------------------------------------------------ */
/* Expert block layout                                                       */
/* ------------------------------------------------------------------------ */

/* One block per expert, in the order gate | up | down | gate_scale |
 * up_scale | down_scale ([Q] "The engine", item 1). gate and up are [I][H]
 * and down is [H][I], row-major, 4-bit codes packed along the row (element 2i
 * in the low nibble of byte i); scales are row-major [rows][cols/G].
 * off[0..5] receive the byte offsets of the six regions, off[6] the total. */
int orc_layout(int fmt, int H, int I, int64_t *off)
{
    int G = group_of(fmt);
    if (H <= 0 || I <= 0 || H % G || I % G)
        return -1;
    int64_t mat_codes = (int64_t)H * I / 2, mat_scales = (int64_t)H * I / G;
    off[0] = 0;
    off[1] = mat_codes;
    off[2] = 2 * mat_codes;
    off[3] = 3 * mat_codes;
    off[4] = 3 * mat_codes + mat_scales;
    off[5] = 3 * mat_codes + 2 * mat_scales;
    off[6] = 3 * mat_codes + 3 * mat_scales;
    return 0;
}

/* The 4-bit code of element (r, c) of a [rows][cols] matrix. */
static int code_at(const uint8_t *codes, int cols, int r, int c)
{
    uint8_t b = codes[(int64_t)r * (cols / 2) + c / 2];
    return (c & 1) ? (b >> 4) : (b & 15);
}

/* W[r][c] = e2m1(code) * scale(S[r][c / G]), evaluated in fp64 and stored in
 * fp32 (the product has at most 6 significant bits, so it is exact). */
static float weight_at(int fmt, const uint8_t *codes, const uint8_t *scales, int cols, int r, int c)
{
    int G = group_of(fmt);
    double s = scale_value(fmt, scales[(int64_t)r * (cols / G) + c / G]);
    return (float)(orc_e2m1(code_at(codes, cols, r, c)) * s);
}

static void dequant_matrix(int fmt, const uint8_t *codes, const uint8_t *scales, int rows, int cols, float *out)
{
    for (int r = 0; r < rows; r++)
        for (int c = 0; c < cols; c++)
            out[(int64_t)r * cols + c] = weight_at(fmt, codes, scales, cols, r, c);
}

/* Dequantise the three matrices of one block to fp32. */
int orc_dequant_block(int fmt, int H, int I, const uint8_t *blk, float *gate, float *up, float *down)
{
    int64_t off[7];
    if (orc_layout(fmt, H, I, off))
        return -1;
    dequant_matrix(fmt, blk + off[0], blk + off[3], I, H, gate);
    dequant_matrix(fmt, blk + off[1], blk + off[4], I, H, up);
    dequant_matrix(fmt, blk + off[2], blk + off[5], H, I, down);
    return 0;
}

/* sum_c W[r][c] * x[c] in fp64, weights decoded on the fly. */
static double row_dot(int fmt, const uint8_t *codes, const uint8_t *scales, int cols, int r, const double *x)
{
    double acc = 0.0;
    for (int c = 0; c < cols; c++)
        acc += (double)weight_at(fmt, codes, scales, cols, r, c) * x[c];
    return acc;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------------ */
/* A minimal parallel-for over a range, used only to time the oracle on many */
/* cores. Each index is computed independently, so results do not depend on */
/* the thread count.                                                         */
/* ------------------------------------------------------------------------ */

typedef void (*range_fn)(void *ctx, int64_t i);
struct range_job { range_fn fn; void *ctx; int64_t lo, hi; };

static void *range_worker(void *p)
{
    struct range_job *j = (struct range_job *)p;
    for (int64_t i = j->lo; i < j->hi; i++)
        j->fn(j->ctx, i);
    return NULL;
}

static void parallel_for(int64_t n, int nthreads, range_fn fn, void *ctx)
{
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > n)
        nthreads = (int)n;
    if (nthreads <= 1) {
        for (int64_t i = 0; i < n; i++)
            fn(ctx, i);
        return;
    }
    pthread_t th[256];
    int running[256];
    struct range_job jobs[256];
    for (int t = 0; t < nthreads; t++) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].lo = n * t / nthreads;
        jobs[t].hi = n * (t + 1) / nthreads;
        running[t] = pthread_create(&th[t], NULL, range_worker, &jobs[t]) == 0;
        if (!running[t])
            range_worker(&jobs[t]); /* no thread available: run the share inline */
    }
    for (int t = 0; t < nthreads; t++)
        if (running[t])
            pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Router: logits, softmax, top-k, renormalised weights                      */
/* ------------------------------------------------------------------------ */

/* logits[t][e] = sum_h Wr[e][h] * x[t][h], fp64 accumulation of fp32 inputs. */
void orc_logits(int T, int H, int E, const float *x, const float *Wr, double *logits)
{
    for (int t = 0; t < T; t++)
        for (int e = 0; e < E; e++) {
            double acc = 0.0;
            for (int h = 0; h < H; h++)
                acc += (double)Wr[(int64_t)e * H + h] * (double)x[(int64_t)t * H + h];
            logits[(int64_t)t * E + e] = acc;
        }
}

/* Ranking used by the router: a higher logit first; equal logits go to the
 * lower expert index first. */
static int ranks_before(const double *l, int a, int b)
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

struct ranked { double l; int i; };
static int cmp_ranked(const void *pa, const void *pb)
{
    const struct ranked *a = pa, *b = pb;
    if (a->l > b->l) return -1;
    if (a->l < b->l) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

/* Top-k by sorting all E (logit, index) pairs. */
void orc_topk_sort(int E, int k, const double *l, int32_t *idx)
{
    struct ranked *v = malloc(sizeof(*v) * (size_t)E);
    for (int e = 0; e < E; e++) {
        v[e].l = l[e];
        v[e].i = e;
    }
    qsort(v, (size_t)E, sizeof(*v), cmp_ranked);
    for (int j = 0; j < k; j++)
        idx[j] = v[j].i;
    free(v);
}

/* Top-k by brute force over all k-subsets (E <= 20): the chosen set is the
 * one whose every member ranks before every non-member. Returns the number
 * of such subsets found (always 1 for finite logits). */
int orc_topk_brute(int E, int k, const double *l, int32_t *idx)
{
    if (E > 20 || k > E)
        return -1;
    int found = 0;
    for (uint32_t mask = 0; mask < (1u << E); mask++) {
        if (__builtin_popcount(mask) != k)
            continue;
        int ok = 1;
        for (int a = 0; a < E && ok; a++)
            for (int b = 0; b < E && ok; b++)
                if ((mask >> a & 1) && !(mask >> b & 1) && !ranks_before(l, a, b))
                    ok = 0;
        if (!ok)
            continue;
        found++;
        /* order the members: member m goes to position = number of members
         * that rank before it */
        for (int a = 0; a < E; a++) {
            if (!(mask >> a & 1))
                continue;
            int pos = 0;
            for (int b = 0; b < E; b++)
                if ((mask >> b & 1) && b != a && ranks_before(l, b, a))
                    pos++;
            idx[pos] = a;
        }
    }
    return found;
}

/* Softmax over all E logits (max-subtracted, fp64), top-k, and weights
 * renormalised over the chosen k ([Q] "Why this model, of all models":
 * top-10 routing over 512 experts; [D] "Bytes per token decide everything":
 * 6 chosen of 384). */
void orc_route(int T, int H, int E, int k, const float *x, const float *Wr, double *logits, int32_t *idx, double *w)
{
    orc_logits(T, H, E, x, Wr, logits);
    double *p = malloc(sizeof(double) * (size_t)E);
    for (int t = 0; t < T; t++) {
        const double *l = logits + (int64_t)t * E;
        double mx = l[0], z = 0.0;
        for (int e = 1; e < E; e++)
            if (l[e] > mx) mx = l[e];
        for (int e = 0; e < E; e++) {
            p[e] = exp(l[e] - mx);
            z += p[e];
        }
        for (int e = 0; e < E; e++)
            p[e] /= z;
        int32_t *it = idx + (int64_t)t * k;
        orc_topk_sort(E, k, l, it);
        double sel = 0.0;
        for (int j = 0; j < k; j++)
            sel += p[it[j]];
        for (int j = 0; j < k; j++)
            w[(int64_t)t * k + j] = p[it[j]] / sel;
    }
    free(p);
}

/* ------------------------------------------------------------------------ */
/* Expert SwiGLU: y = down( silu(gate x) * (up x) )                          */
/* ------------------------------------------------------------------------ */

/* h[i] = silu(g[i]) * u[i] with g = Wg x, u = Wu x (fp64). */
static void expert_hidden(int fmt, int H, int I, const uint8_t *blk, const double *x, double *h)
{
    int64_t off[7];
    orc_layout(fmt, H, I, off);
    for (int i = 0; i < I; i++) {
        double g = row_dot(fmt, blk + off[0], blk + off[3], H, i, x);
        double u = row_dot(fmt, blk + off[1], blk + off[4], H, i, x);
        h[i] = silu(g) * u;
    }
}

/* y[r] = sum_i Wd[r][i] * h[i] (fp64). */
static void expert_down(int fmt, int H, int I, const uint8_t *blk, const double *h, double *y)
{
    int64_t off[7];
    orc_layout(fmt, H, I, off);
    for (int r = 0; r < H; r++)
        y[r] = row_dot(fmt, blk + off[2], blk + off[5], I, r, h);
}

/* One expert on one fp64 input, no intermediate rounding. */
int orc_expert(int fmt, int H, int I, const uint8_t *blk, const double *x, double *h_out, double *y)
{
    int64_t off[7];
    if (orc_layout(fmt, H, I, off))
        return -1;
    double *h = h_out ? h_out : malloc(sizeof(double) * (size_t)I);
    expert_hidden(fmt, H, I, blk, x, h);
    expert_down(fmt, H, I, blk, h, y);
    if (!h_out)
        free(h);
    return 0;
}

double orc_bf16_value(uint16_t b)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)b << 16;
    return (double)v.f;
}

/* Dense bf16 SwiGLU (the shared expert): h = silu(Wg x) * (Wu x); y += Wd h. */
static void shared_expert_add(int H, int I, const uint16_t *sg, const uint16_t *su, const uint16_t *sd,
                              const double *x, double *y)
{
    double *h = malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < I; i++) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; c++) {
            g += orc_bf16_value(sg[(int64_t)i * H + c]) * x[c];
            u += orc_bf16_value(su[(int64_t)i * H + c]) * x[c];
        }
        h[i] = silu(g) * u;
    }
    for (int r = 0; r < H; r++) {
        double acc = 0.0;
        for (int i = 0; i < I; i++)
            acc += orc_bf16_value(sd[(int64_t)r * I + i]) * h[i];
        y[r] += acc;
    }
    free(h);
}

/* ------------------------------------------------------------------------ */
/* Decode: one token through one MoE layer                                   */
/* ------------------------------------------------------------------------ */

struct decode_ctx {
    int fmt, H, I, k;
    const uint8_t *const *blocks;
    const double *x;
    double *h;   /* [k][I] */
    double *yj;  /* [k][H] */
};

static void decode_hidden_task(void *p, int64_t n)
{
    struct decode_ctx *c = p;
    int j = (int)(n / c->I), i = (int)(n % c->I);
    int64_t off[7];
    orc_layout(c->fmt, c->H, c->I, off);
    const uint8_t *b = c->blocks[j];
    double g = row_dot(c->fmt, b + off[0], b + off[3], c->H, i, c->x);
    double u = row_dot(c->fmt, b + off[1], b + off[4], c->H, i, c->x);
    c->h[(int64_t)j * c->I + i] = silu(g) * u;
}

static void decode_down_task(void *p, int64_t n)
{
    struct decode_ctx *c = p;
    int j = (int)(n / c->H), r = (int)(n % c->H);
    int64_t off[7];
    orc_layout(c->fmt, c->H, c->I, off);
    const uint8_t *b = c->blocks[j];
    c->yj[(int64_t)j * c->H + r] = row_dot(c->fmt, b + off[2], b + off[5], c->I, r, c->h + (int64_t)j * c->I);
}

/* y = sum_j w[j] * expert_{blocks[j]}(x) (+ shared expert if sg != NULL).
 * blocks[j] points at the block of the j-th chosen expert. h_out, if not
 * NULL, receives the k x I SwiGLU hidden vectors. */
int orc_moe_decode(int fmt, int H, int I, int k, const float *x, const uint8_t *const *blocks, const double *w,
                   const uint16_t *sg, const uint16_t *su, const uint16_t *sd, double *y, double *h_out,
                   int nthreads)
{
    int64_t off[7];
    if (orc_layout(fmt, H, I, off) || k < 1)
        return -1;
    double *xd = malloc(sizeof(double) * (size_t)H);
    for (int c = 0; c < H; c++)
        xd[c] = x[c];
    struct decode_ctx c = {fmt, H, I, k, blocks, xd,
                           malloc(sizeof(double) * (size_t)k * I), malloc(sizeof(double) * (size_t)k * H)};
    parallel_for((int64_t)k * I, nthreads, decode_hidden_task, &c);
    parallel_for((int64_t)k * H, nthreads, decode_down_task, &c);
    for (int r = 0; r < H; r++) {
        double acc = 0.0;
        for (int j = 0; j < k; j++)
            acc += w[j] * c.yj[(int64_t)j * H + r];
        y[r] = acc;
    }
    if (sg)
        shared_expert_add(H, I, sg, su, sd, xd, y);
    if (h_out)
        memcpy(h_out, c.h, sizeof(double) * (size_t)k * I);
    free(c.h);
    free(c.yj);
    free(xd);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Activation rounding used by prefill                                       */
/* ------------------------------------------------------------------------ */

/* Round a real value to bfloat16 (8 significant bits, fp32 exponent range),
 * to nearest, ties to even. Returns the bf16 bit pattern. */
uint16_t orc_bf16_rne(double v)
{
    union { uint32_t u; float f; } out;
    if (isnan(v))
        return 0x7FC0;
    double a = fabs(v), r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        frexp(a, &e);                     /* a = m * 2^e, m in [0.5, 1) */
        int q = e - 8;                    /* 8 significant bits: quantum 2^(e-8) */
        if (q < -133)
            q = -133;                     /* smallest bf16 subnormal step */
        r = nearbyint(ldexp(a, -q));      /* default rounding: to nearest, ties to even */
        r = ldexp(r, q);
        if (r >= ldexp(1.0, 128))         /* beyond the largest finite bf16 */
            r = INFINITY;
    }
    out.f = (float)(signbit(v) ? -r : r); /* exact: r has at most 8 significant bits */
    return (uint16_t)(out.u >> 16);
}

/* e2m1 code of the real value t (already divided by the block scale):
 * nearest grid value, ties to the code with an even mantissa bit,
 * magnitudes above 6 saturate to 6 ([OCP-MX] conversion with saturation). */
static int e2m1_round(double t)
{
    double a = fabs(t);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs(a - orc_e2m1(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    if (a > 6.0)
        best = 7;
    return (t < 0 || (t == 0 && signbit(t))) ? (best | 8) : best;
}

/* MXFP4 conversion of one block of n <= 32 values ([OCP-MX] section on
 * converting a vector to an MX block): shared exponent
 * X = floor(log2(max |v|)) - 2 (2 = largest exponent of e2m1), clamped to
 * [-127, 127]; scale byte X + 127; codes = e2m1_round(v / 2^X). An all-zero
 * block gets scale byte 0 and zero codes. */
void orc_mxfp4_quant(const double *v, int n, uint8_t *codes, uint8_t *scale_byte)
{
    double amax = 0.0;
    for (int i = 0; i < n; i++)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    if (amax == 0.0) {
        *scale_byte = 0;
        for (int i = 0; i < n; i++)
            codes[i] = signbit(v[i]) ? 8 : 0;
        return;
    }
    int e;
    frexp(amax, &e);                      /* amax in [2^(e-1), 2^e) */
    int X = (e - 1) - 2;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    *scale_byte = (uint8_t)(X + 127);
    for (int i = 0; i < n; i++)
        codes[i] = (uint8_t)e2m1_round(ldexp(v[i], -X));
}

/* Value of an MXFP4-rounded block, for the oracle's own use. */
static void mxfp4_roundtrip(const double *v, int n, double *out)
{
    uint8_t codes[32], sb;
    orc_mxfp4_quant(v, n, codes, &sb);
    double s = orc_ue8m0(sb);
    for (int i = 0; i < n; i++)
        out[i] = orc_e2m1(codes[i]) * s;
}

/* Row-wise activation quantisers (for the bit-exact check of the GPU's x~):
 * bf16: out16[T][n]; MXFP4: codes packed [T][n/2] (element 2i in the low
 * nibble), scales [T][n/32]. */
void orc_quant_bf16_rows(int T, int n, const float *x, uint16_t *out16)
{
    for (int64_t i = 0; i < (int64_t)T * n; i++)
        out16[i] = orc_bf16_rne(x[i]);
}

int orc_quant_mxfp4_rows(int T, int n, const float *x, uint8_t *packed, uint8_t *scales)
{
    if (n % 32)
        return -1;
    double v[32];
    uint8_t c[32];
    for (int t = 0; t < T; t++)
        for (int b = 0; b < n / 32; b++) {
            for (int i = 0; i < 32; i++)
                v[i] = x[(int64_t)t * n + b * 32 + i];
            orc_mxfp4_quant(v, 32, c, &scales[(int64_t)t * (n / 32) + b]);
            for (int i = 0; i < 16; i++)
                packed[(int64_t)t * (n / 2) + b * 16 + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 activation quantiser with a UE8M0 scale per block                     */
/* ------------------------------------------------------------------------ */

#define ORC_SCALE_FLOOR 0 /* [OCP-MX]: X = floor(log2 amax) - 8 (may saturate) */
#define ORC_SCALE_CEIL  1 /* smallest X with amax <= 448 * 2^X (never saturates) */

/* E4M3 code of the real value t: the nearest of the finite E4M3 values
 * (codes 0..126 and their negatives), found by searching the whole grid;
 * ties go to the code with an even mantissa bit; magnitudes above 448
 * saturate to 448 (code 0x7E). Negative values that round to zero keep the
 * sign (code 0x80). */
static int e4m3_round(double t)
{
    double a = fabs(t);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 127; c++) {
        double d = fabs(a - orc_e4m3(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    if (a > 448.0)
        best = 0x7E;
    return (t < 0 || (t == 0 && signbit(t))) ? (best | 0x80) : best;
}

/* One block of n values to E4M3 codes with a shared UE8M0 scale ([D] "Three
 * bugs", item 2: DeepSeek's activation quantiser writes FP8 with ue8m0
 * scales; [OCP-MX] MXFP8 is the same format with blocks of 32). The shared
 * exponent X is clamped to [-127, 127] and stored as the byte X + 127; the
 * codes are e4m3_round(v / 2^X). An all-zero block gets scale byte 0 and
 * zero codes. */
void orc_fp8_quant(const double *v, int n, int rule, uint8_t *codes, uint8_t *scale_byte)
{
    double amax = 0.0;
    for (int i = 0; i < n; i++)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    if (amax == 0.0) {
        *scale_byte = 0;
        for (int i = 0; i < n; i++)
            codes[i] = signbit(v[i]) ? 0x80 : 0;
        return;
    }
    int e;
    frexp(amax, &e);                      /* amax in [2^(e-1), 2^e) */
    int X = (e - 1) - 8;                  /* 8 = largest exponent of E4M3 */
    if (rule == ORC_SCALE_CEIL) {
        X = (e - 1) - 9;
        while (amax > ldexp(448.0, X))
            X++;
    }
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    *scale_byte = (uint8_t)(X + 127);
    for (int i = 0; i < n; i++)
        codes[i] = (uint8_t)e4m3_round(ldexp(v[i], -X));
}

/* Rows of n values, blocks of `block` consecutive values: codes [T][n],
 * scales [T][n/block]. */
int orc_quant_fp8_rows(int T, int n, int block, int rule, const float *x, uint8_t *codes, uint8_t *scales)
{
    if (block <= 0 || block > 1024 || n % block)
        return -1;
    double v[1024];
    for (int t = 0; t < T; t++)
        for (int b = 0; b < n / block; b++) {
            for (int i = 0; i < block; i++)
                v[i] = x[(int64_t)t * n + (int64_t)b * block + i];
            orc_fp8_quant(v, block, rule, codes + (int64_t)t * n + (int64_t)b * block,
                          &scales[(int64_t)t * (n / block) + b]);
        }
    return 0;
}

/* Row-scaled FP8 matrix-vector product ([Q] "The engine", item 4; [Q] "Why
 * this model, of all models": dense matrices in FP8 with one scale per
 * row): y[r] = s[r] * sum_c e4m3(W[r][c]) * x[c], in fp64. */
void orc_gemv_fp8(int rows, int cols, const uint8_t *W, const float *s, const float *x, double *y)
{
    for (int r = 0; r < rows; r++) {
        double acc = 0.0;
        for (int c = 0; c < cols; c++)
            acc += orc_e4m3(W[(int64_t)r * cols + c]) * (double)x[c];
        y[r] = (double)s[r] * acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Grouping of (token, slot) assignments by expert                           */
/* ------------------------------------------------------------------------ */

/* count[e] = number of assignments to expert e; off = exclusive prefix sum
 * (off[E] = T*k); perm lists assignment ids a = t*k + j grouped by expert,
 * in increasing a within each expert (a stable counting sort). */
int orc_group(int T, int k, int E, const int32_t *idx, int32_t *count, int32_t *off, int32_t *perm)
{
    for (int e = 0; e < E; e++)
        count[e] = 0;
    for (int64_t a = 0; a < (int64_t)T * k; a++) {
        if (idx[a] < 0 || idx[a] >= E)
            return -1;
        count[idx[a]]++;
    }
    off[0] = 0;
    for (int e = 0; e < E; e++)
        off[e + 1] = off[e] + count[e];
    int32_t *next = malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; e++)
        next[e] = off[e];
    for (int64_t a = 0; a < (int64_t)T * k; a++)
        perm[next[idx[a]]++] = (int32_t)a;
    free(next);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Prefill: every token through one layer, with the declared activation      */
/* rounding points                                                           */
/* ------------------------------------------------------------------------ */

#define ACT_NONE 0
#define ACT_BF16 1
#define ACT_MXFP4 2

static void round_activation(int act, const double *v, int n, double *out)
{
    if (act == ACT_BF16) {
        for (int i = 0; i < n; i++)
            out[i] = orc_bf16_value(orc_bf16_rne(v[i]));
    } else if (act == ACT_MXFP4) {
        for (int b = 0; b < n; b += 32)
            mxfp4_roundtrip(v + b, n - b < 32 ? n - b : 32, out + b);
    } else {
        for (int i = 0; i < n; i++)
            out[i] = v[i];
    }
}

struct prefill_ctx {
    int fmt, H, I, k, T, act, out_bf16;
    const float *x;
    const uint8_t *const *blocks;
    const int32_t *idx;
    const float *w;
    double *out, *h_pre, *h_q;
};

static void prefill_token_task(void *p, int64_t t)
{
    struct prefill_ctx *c = p;
    int H = c->H, I = c->I, k = c->k;
    double *xt = malloc(sizeof(double) * (size_t)H);
    double *xq = malloc(sizeof(double) * (size_t)H);
    double *h = malloc(sizeof(double) * (size_t)I);
    double *hq = malloc(sizeof(double) * (size_t)I);
    double *y = malloc(sizeof(double) * (size_t)H);
    double *acc = calloc((size_t)H, sizeof(double));
    for (int c0 = 0; c0 < H; c0++)
        xt[c0] = c->x[t * H + c0];
    round_activation(c->act, xt, H, xq);                 /* x~ */
    for (int j = 0; j < k; j++) {
        const uint8_t *b = c->blocks[c->idx[t * k + j]];
        expert_hidden(c->fmt, H, I, b, xq, h);            /* h = silu(g) * u */
        round_activation(c->act, h, I, hq);               /* h~ */
        expert_down(c->fmt, H, I, b, hq, y);
        double wj = c->w[t * k + j];
        for (int r = 0; r < H; r++)
            acc[r] += wj * y[r];
        if (c->h_pre)
            memcpy(c->h_pre + (t * k + j) * (int64_t)I, h, sizeof(double) * (size_t)I);
        if (c->h_q)
            memcpy(c->h_q + (t * k + j) * (int64_t)I, hq, sizeof(double) * (size_t)I);
    }
    for (int r = 0; r < H; r++)
        c->out[t * H + r] = c->out_bf16 ? orc_bf16_value(orc_bf16_rne(acc[r])) : acc[r];
    free(xt); free(xq); free(h); free(hq); free(y); free(acc);
}

/* out[t] = sum_j w[t][j] * down_e( Q( silu(gate_e Q(x_t)) * up_e Q(x_t) ) ),
 * e = idx[t][j], where Q is the activation rounding act (none, bf16 RNE, or
 * MXFP4 per 32 along the row), and out is optionally rounded to bf16.
 * blocks[e] points at expert e's block. h_pre / h_q (optional, [T][k][I])
 * receive h before and after rounding. */
int orc_moe_prefill(int fmt, int H, int I, int E, int k, int T, const float *x, const uint8_t *const *blocks,
                    const int32_t *idx, const float *w, int act, int out_bf16, double *out, double *h_pre,
                    double *h_q, int nthreads)
{
    int64_t off[7];
    if (orc_layout(fmt, H, I, off) || k < 1 || k > E || T < 0)
        return -1;
    if (act == ACT_MXFP4 && (H % 32 || I % 32))
        return -1;
    for (int64_t a = 0; a < (int64_t)T * k; a++)
        if (idx[a] < 0 || idx[a] >= E)
            return -1;
    struct prefill_ctx c = {fmt, H, I, k, T, act, out_bf16, x, blocks, idx, w, out, h_pre, h_q};
    parallel_for(T, nthreads, prefill_token_task, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Prefill, stage by stage                                                   */
/*                                                                           */
/* The same per-token definition as orc_moe_prefill, cut at the rounding     */
/* point of h so that each stage can be checked on its own: the gate/up      */
/* stage on a list of assignments, and the down projection + combine on a    */
/* caller-given h~ (for instance the one the GPU rounded). Every expert      */
/* matrix a stage needs is dequantised to fp32 once (the same exact values   */
/* weight_at gives) and each output element is the same fp64 sum over the    */
/* input index in increasing order, so the results equal orc_moe_prefill's   */
/* bit for bit where the inputs are the same.                                */
/* ------------------------------------------------------------------------ */

/* Rows of n values through the activation rounding act (ACT_NONE, ACT_BF16:
 * bf16 round-to-nearest-even, ACT_MXFP4: MXFP4 per 32 along the row),
 * returned as the rounded values in fp64. */
int orc_round_rows(int act, int rows, int n, const double *in, double *out)
{
    if (act == ACT_MXFP4 && n % 32)
        return -1;
    for (int64_t r = 0; r < rows; r++)
        round_activation(act, in + r * n, n, out + r * n);
    return 0;
}

/* One assignment to evaluate: its expert, its id a = t*k + j and the caller's
 * output row. Workers take them sorted by (expert, id, row), so that each
 * meets an expert in one run and dequantises its matrices once. */
struct stage_item { int32_t e, a, row; };
static int cmp_stage_item(const void *pa, const void *pb)
{
    const struct stage_item *x = pa, *y = pb;
    if (x->e != y->e) return (x->e > y->e) - (x->e < y->e);
    if (x->a != y->a) return (x->a > y->a) - (x->a < y->a);
    return (x->row > y->row) - (x->row < y->row);
}

static struct stage_item *sorted_items(int n, const int32_t *ids, const int32_t *idx)
{
    struct stage_item *it = malloc(sizeof(*it) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; i++) {
        it[i].e = idx[ids[i]];
        it[i].a = ids[i];
        it[i].row = i;
    }
    qsort(it, (size_t)n, sizeof(*it), cmp_stage_item);
    return it;
}

struct stage_ctx {
    int fmt, H, I, k, act, nparts, n, out_bf16;
    const float *x;
    const uint8_t *const *blocks;
    const struct stage_item *items;
    const double *h_in;              /* down stage: h~ [n][I] */
    double *h_pre, *h_q, *gu, *agu;  /* hidden stage outputs, [n][...] */
    double *y;                       /* down stage: [n][H] */
};

static void stage_hidden_worker(void *p, int64_t part)
{
    struct stage_ctx *c = p;
    int H = c->H, I = c->I;
    int64_t lo = (int64_t)c->n * part / c->nparts, hi = (int64_t)c->n * (part + 1) / c->nparts;
    if (lo >= hi)
        return;
    int64_t off[7];
    orc_layout(c->fmt, H, I, off);
    float *Wg = malloc(sizeof(float) * (size_t)I * H), *Wu = malloc(sizeof(float) * (size_t)I * H);
    double *xt = malloc(sizeof(double) * (size_t)H), *xq = malloc(sizeof(double) * (size_t)H);
    double *h = malloc(sizeof(double) * (size_t)I);
    int cur = -1;
    for (int64_t i = lo; i < hi; i++) {
        const struct stage_item *it = &c->items[i];
        int t = it->a / c->k;
        int64_t row = it->row;
        if (it->e != cur) {
            const uint8_t *b = c->blocks[it->e];
            dequant_matrix(c->fmt, b + off[0], b + off[3], I, H, Wg);
            dequant_matrix(c->fmt, b + off[1], b + off[4], I, H, Wu);
            cur = it->e;
        }
        for (int q = 0; q < H; q++)
            xt[q] = c->x[(int64_t)t * H + q];
        round_activation(c->act, xt, H, xq);                 /* x~ */
        for (int r = 0; r < I; r++) {
            double g = 0.0, u = 0.0, ag = 0.0, au = 0.0;
            const float *wg = Wg + (int64_t)r * H, *wu = Wu + (int64_t)r * H;
            for (int q = 0; q < H; q++) {
                double pg = (double)wg[q] * xq[q], pu = (double)wu[q] * xq[q];
                g += pg;
                u += pu;
                ag += fabs(pg);
                au += fabs(pu);
            }
            h[r] = silu(g) * u;                              /* h = silu(g) * u */
            if (c->gu) {
                c->gu[(row * 2 + 0) * I + r] = g;
                c->gu[(row * 2 + 1) * I + r] = u;
            }
            if (c->agu) {
                c->agu[(row * 2 + 0) * I + r] = ag;
                c->agu[(row * 2 + 1) * I + r] = au;
            }
        }
        memcpy(c->h_pre + row * I, h, sizeof(double) * (size_t)I);
        if (c->h_q)
            round_activation(c->act, h, I, c->h_q + row * I); /* h~ */
    }
    free(Wg); free(Wu); free(xt); free(xq); free(h);
}

static int check_ids(int n, const int32_t *ids, const int32_t *idx, int T, int k, int E)
{
    for (int i = 0; i < n; i++)
        if (ids[i] < 0 || ids[i] >= (int64_t)T * k || idx[ids[i]] < 0 || idx[ids[i]] >= E)
            return -1;
    return 0;
}

/* The gate/up stage of prefill for n assignments ids[i] = t*k + j: with
 * x~ = Q(x_t) and e = idx[t][j], h = silu(Wg_e x~) * (Wu_e x~) (fp64) into
 * h_pre[i][I], and h~ = Q(h) into h_q[i][I] (may be NULL). gu (may be
 * NULL) receives [i][0][I] = g and [i][1][I] = u; agu (may be NULL) the sums
 * of the absolute values of the same products, sum_c |W[r][c] x~[c]|: the
 * magnitude that bounds the rounding error of any finite-precision
 * evaluation of that dot product. */
int orc_prefill_stage_hidden(int fmt, int H, int I, int E, int k, int T, const float *x,
                             const uint8_t *const *blocks, const int32_t *idx, int act, int n, const int32_t *ids,
                             double *h_pre, double *h_q, double *gu, double *agu, int nthreads)
{
    int64_t off[7];
    if (orc_layout(fmt, H, I, off) || k < 1 || k > E || n < 0 || check_ids(n, ids, idx, T, k, E))
        return -1;
    if (act == ACT_MXFP4 && (H % 32 || I % 32))
        return -1;
    struct stage_item *items = sorted_items(n, ids, idx);
    int parts = nthreads < 1 ? 1 : (nthreads > n ? (n > 0 ? n : 1) : nthreads);
    struct stage_ctx c = {fmt, H, I, k, act, parts, n, 0, x, blocks, items, NULL, h_pre, h_q, gu, agu, NULL};
    parallel_for(parts, parts, stage_hidden_worker, &c);
    free(items);
    return 0;
}

static void stage_down_worker(void *p, int64_t part)
{
    struct stage_ctx *c = p;
    int H = c->H, I = c->I;
    int64_t lo = (int64_t)c->n * part / c->nparts, hi = (int64_t)c->n * (part + 1) / c->nparts;
    if (lo >= hi)
        return;
    int64_t off[7];
    orc_layout(c->fmt, H, I, off);
    float *Wd = malloc(sizeof(float) * (size_t)H * I);
    int cur = -1;
    for (int64_t i = lo; i < hi; i++) {
        const struct stage_item *it = &c->items[i];
        if (it->e != cur) {
            const uint8_t *b = c->blocks[it->e];
            dequant_matrix(c->fmt, b + off[2], b + off[5], H, I, Wd);
            cur = it->e;
        }
        const double *hq = c->h_in + (int64_t)it->row * I;
        double *y = c->y + (int64_t)it->row * H;
        for (int r = 0; r < H; r++) {
            double acc = 0.0;
            const float *wd = Wd + (int64_t)r * I;
            for (int q = 0; q < I; q++)
                acc += (double)wd[q] * hq[q];
            y[r] = acc;                                      /* y_j = Wd_e h~_j */
        }
    }
    free(Wd);
}

/* The down projection and combine of prefill on a given h~: for tokens
 * t < T, out[t] = sum_j w[t][j] * Wd_e h_q[t][j] with e = idx[t][j] (fp64,
 * j increasing), rounded to bf16 when out_bf16 is set (the value of the
 * rounded bf16 is stored). h_q is [T][k][I] in token order: the rounded
 * hidden vectors of some evaluation of the gate/up stage. */
int orc_prefill_down_combine(int fmt, int H, int I, int E, int k, int T, const uint8_t *const *blocks,
                             const int32_t *idx, const float *w, const double *h_q, int out_bf16, double *out,
                             int nthreads)
{
    int64_t off[7];
    if (orc_layout(fmt, H, I, off) || k < 1 || k > E || T < 0)
        return -1;
    int n = T * k;
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    for (int a = 0; a < n; a++)
        ids[a] = a;
    if (check_ids(n, ids, idx, T, k, E)) {
        free(ids);
        return -1;
    }
    struct stage_item *items = sorted_items(n, ids, idx);
    double *y = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * H);
    int parts = nthreads < 1 ? 1 : (nthreads > n ? (n > 0 ? n : 1) : nthreads);
    struct stage_ctx c = {fmt, H, I, k, ACT_NONE, parts, n, out_bf16, NULL, blocks, items, h_q, NULL, NULL, NULL, NULL, y};
    parallel_for(parts, parts, stage_down_worker, &c);
    for (int t = 0; t < T; t++)
        for (int r = 0; r < H; r++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++)
                acc += (double)w[t * k + j] * y[((int64_t)t * k + j) * H + r];
            out[(int64_t)t * H + r] = out_bf16 ? orc_bf16_value(orc_bf16_rne(acc)) : acc;
        }
    free(items);
    free(ids);
    free(y);
    return 0;
}
