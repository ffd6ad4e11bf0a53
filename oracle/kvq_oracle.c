/*
 * kvq_oracle.c -- plain, slow CPU oracle for Block-GTQ key-cache quantization
 * and packed-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do.  It shares no source, header, table or generator with the HIP library.
 *
 * The method is described on the page "RoPE-Aware Bit Allocation for KV-Cache
 * Quantization" (abstract only).  The abstract fixes the outline:
 *   - under RoPE a key's contribution to a logit splits into 2-D frequency blocks;
 *   - per layer and KV head, a label-free energy score is computed per block;
 *   - integer bit widths are allocated greedily by marginal gain under a budget;
 *   - the base quantizer is TurboQuant-MSE (TQ-MSE);
 *   - a packed-cache decode path reads the compressed cache.
 * Every concrete numeric choice below is the reading documented alongside the
 * code (per-token L2 norm, per-block scale, Gaussian Lloyd-Max codebooks, the
 * bit layout).  Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

typedef unsigned __int128 u128;

/* ------------------------------------------------------------------------- */
/* Scalar helpers                                                            */
/* ------------------------------------------------------------------------- */

/* fp16 bit pattern -> exact double (IEEE binary16). */
static double h2d(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* double -> binary16, round to nearest even (finite inputs of modest size). */
static uint16_t d2h(double x)
{
    uint16_t sign = 0;
    if (x < 0) { sign = 0x8000; x = -x; }
    if (x == 0) return sign;
    int e;
    frexp(x, &e);                 /* x = f * 2^e, f in [0.5, 1) */
    int ex = e - 1;               /* x in [2^ex, 2^(ex+1)) */
    if (ex < -14) ex = -14;       /* subnormal range uses the fixed scale 2^-24 */
    double m = rint(ldexp(x, 10 - ex)); /* significand in units of 2^(ex-10) */
    if (m >= 2048.0) { m /= 2.0; ex += 1; }
    if (ex > 15) return sign | 0x7C00;
    if (m < 1024.0) return sign | (uint16_t)m; /* subnormal */
    return sign | (uint16_t)(((ex + 15) << 10) | ((int)m - 1024));
}

static double phi(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }
/* upper tail Q(x) = P[X >= x], accurate for large x */
static double qtail(double x) { return 0.5 * erfc(x / sqrt(2.0)); }

/* ------------------------------------------------------------------------- */
/* Lloyd-Max codebooks for N(0,1)                                            */
/* ------------------------------------------------------------------------- */
/*
 * TQ-MSE's scalar quantizer is read as the MSE-optimal (Lloyd-Max) quantizer of
 * a standard Gaussian coordinate with 2^w levels.  Optimality conditions:
 *   threshold between levels j-1 and j is their midpoint;
 *   level j is the conditional mean of X on its cell.
 * The codebook is symmetric, so only the positive half is solved: cells
 * [t_0 = 0, t_1), ..., [t_{h-1}, +inf) with h = 2^(w-1) levels c_0 < ... < c_{h-1}.
 * Solved by Lloyd iterations from the companding start, then Newton's method on
 * F_j(c) = c_j - mean(t_j, t_{j+1}), whose Jacobian is tridiagonal.
 */

/* conditional mean of X on [a, b) with a >= 0 (b may be +inf) */
static void cell_mean(double a, double b, double *mean, double *prob)
{
    double pa = phi(a), pb = isinf(b) ? 0.0 : phi(b);
    double P = qtail(a) - (isinf(b) ? 0.0 : qtail(b));
    *prob = P;
    *mean = (pa - pb) / P;
}

static void thresholds(const double *c, int h, double *t)
{
    t[0] = 0.0;
    for (int j = 1; j < h; j++) t[j] = 0.5 * (c[j - 1] + c[j]);
    t[h] = INFINITY;
}

/* inverse of the standard normal CDF by bisection (used only for the start) */
static double ndtri_bisect(double p)
{
    double lo = -40, hi = 40;
    for (int i = 0; i < 200; i++) {
        double mid = 0.5 * (lo + hi);
        double cdf = 1.0 - qtail(mid);
        if (cdf < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

/*
 * Solve the w-bit codebook.  Outputs all 2^w levels ascending in cent[],
 * the mean squared error D in *D, and the max fixed-point residual in *resid.
 * Returns the number of Newton steps, or -1 on failure.
 */
int or_lloyd_max(int w, double *cent, double *D, double *resid)
{
    if (w < 1 || w > 8) return -1;
    int n = 1 << w, h = n / 2;
    double c[128], t[129], cn[128];
    /* companding start: level density proportional to phi^(1/3), i.e. N(0, 3) */
    for (int j = 0; j < h; j++) c[j] = sqrt(3.0) * ndtri_bisect((h + j + 0.5) / n);
    for (int it = 0; it < 3000; it++) {
        thresholds(c, h, t);
        for (int j = 0; j < h; j++) { double P; cell_mean(t[j], t[j + 1], &cn[j], &P); }
        memcpy(c, cn, sizeof(double) * h);
    }
    int steps = 0;
    for (; steps < 50; steps++) {
        double F[128], lo[128], di[128], up[128];
        thresholds(c, h, t);
        double maxF = 0;
        for (int j = 0; j < h; j++) {
            double a = t[j], b = t[j + 1], m, P;
            cell_mean(a, b, &m, &P);
            F[j] = c[j] - m;
            if (fabs(F[j]) > maxF) maxF = fabs(F[j]);
            /* d mean / d a = phi(a) (m - a) / P ; d mean / d b = phi(b) (b - m) / P */
            double dma = (j == 0) ? 0.0 : phi(a) * (m - a) / P;       /* t_0 = 0 is fixed */
            double dmb = isinf(b) ? 0.0 : phi(b) * (b - m) / P;
            /* t_j = (c_{j-1} + c_j)/2, t_{j+1} = (c_j + c_{j+1})/2 */
            lo[j] = -0.5 * dma;
            di[j] = 1.0 - 0.5 * dma - 0.5 * dmb;
            up[j] = -0.5 * dmb;
        }
        if (maxF < 1e-13) break;   /* the evaluation noise floor is ~1e-14 */
        /* Thomas algorithm for the tridiagonal system J dx = F */
        double cp[128], dp[128];
        cp[0] = up[0] / di[0];
        dp[0] = F[0] / di[0];
        for (int j = 1; j < h; j++) {
            double den = di[j] - lo[j] * cp[j - 1];
            cp[j] = up[j] / den;
            dp[j] = (F[j] - lo[j] * dp[j - 1]) / den;
        }
        double dx[128];
        dx[h - 1] = dp[h - 1];
        for (int j = h - 2; j >= 0; j--) dx[j] = dp[j] - cp[j] * dx[j + 1];
        for (int j = 0; j < h; j++) c[j] -= dx[j];
    }
    /* residual and distortion */
    thresholds(c, h, t);
    double r = 0, dsum = 0;
    for (int j = 0; j < h; j++) {
        double a = t[j], b = t[j + 1], m, P;
        cell_mean(a, b, &m, &P);
        if (fabs(c[j] - m) > r) r = fabs(c[j] - m);
        /* E[(X - c)^2 ; a <= X < b] = P - (b phi(b) - a phi(a)) - c^2 P  for c = mean */
        double bpb = isinf(b) ? 0.0 : b * phi(b);
        dsum += P - (bpb - a * phi(a)) - c[j] * c[j] * P;
    }
    *D = 2.0 * dsum;
    *resid = r;
    for (int j = 0; j < h; j++) { cent[h + j] = c[j]; cent[h - 1 - j] = -c[j]; }
    return steps;
}

/* round a codebook to binary16 (bit patterns) */
void or_round_fp16(const double *x, int n, uint16_t *out)
{
    for (int i = 0; i < n; i++) out[i] = d2h(x[i]);
}

void or_h2d(const uint16_t *h, int n, double *out)
{
    for (int i = 0; i < n; i++) out[i] = h2d(h[i]);
}

/* ------------------------------------------------------------------------- */
/* Block map                                                                 */
/* ------------------------------------------------------------------------- */
/*
 * Under RoPE the head dimension d splits into d/2 two-dimensional rotation
 * planes ("blocks").  pairing 0 (half split, rotate_half convention): block i
 * holds coordinates (i, i + d/2); pairing 1 (interleaved): (2i, 2i + 1).
 */
static void block_coords(int d, int pairing, int i, int *p, int *q)
{
    if (pairing == 0) { *p = i; *q = i + d / 2; }
    else { *p = 2 * i; *q = 2 * i + 1; }
}

/* ------------------------------------------------------------------------- */
/* Block energy                                                              */
/* ------------------------------------------------------------------------- */
/*
 * Label-free energy of block i: sum over the supplied tokens of the squared
 * norm of the block, k_p^2 + k_q^2.  Every binary16 square is an integer
 * multiple of 2^-48, so the sum is kept exactly as a 128-bit integer in units
 * of 2^-48.  For a binary16 pattern with exponent field e and fraction m the
 * value is M * 2^(e-25) with M = 1024 + m (e >= 1) or M * 2^-24 with M = m
 * (e == 0), so the square is M^2 << (2e - 2) units (M^2 << 0 when e == 0).
 * The same formula is applied to every pattern, including e == 31.
 */
static u128 sq_units(uint16_t h)
{
    int e = (h >> 10) & 31, m = h & 1023;
    u128 M = (e == 0) ? (u128)m : (u128)(1024 + m);
    int sh = (e == 0) ? 0 : 2 * e - 2;
    return (M * M) << sh;
}

/*
 * x: binary16 patterns, element (t, h, c) at x[t*stride_tok + h*stride_head + c].
 * energy: [n_heads][d/2][2] uint64 limbs (low, high); accumulated into.
 */
void or_block_energy(const uint16_t *x, int64_t n_tok, int64_t stride_tok, int64_t stride_head,
                     int n_heads, int d, int pairing, uint64_t *energy)
{
    int nb = d / 2;
    for (int h = 0; h < n_heads; h++) {
        for (int i = 0; i < nb; i++) {
            int p, q;
            block_coords(d, pairing, i, &p, &q);
            u128 acc = (u128)energy[(h * nb + i) * 2] | ((u128)energy[(h * nb + i) * 2 + 1] << 64);
            for (int64_t t = 0; t < n_tok; t++) {
                const uint16_t *row = x + t * stride_tok + (int64_t)h * stride_head;
                acc += sq_units(row[p]) + sq_units(row[q]);
            }
            energy[(h * nb + i) * 2] = (uint64_t)acc;
            energy[(h * nb + i) * 2 + 1] = (uint64_t)(acc >> 64);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Greedy bit allocation                                                     */
/* ------------------------------------------------------------------------- */

/* exact unsigned 128-bit integer -> double, round to nearest even */
static double u128_to_double(u128 v)
{
    if (v == 0) return 0.0;
    int top = 127;
    while (!((v >> top) & 1)) top--;
    if (top < 53) return (double)(uint64_t)v;          /* exact */
    int drop = top - 52;                               /* bits below the 53-bit significand */
    u128 keep = v >> drop;
    u128 rem = v - (keep << drop);
    u128 half = (u128)1 << (drop - 1);
    if (rem > half || (rem == half && (keep & 1))) keep += 1;
    return ldexp((double)(uint64_t)keep, drop);        /* keep <= 2^53, exact */
}

/*
 * Per unit (layer, KV head):
 *   E_i  = RN_fp64(energy_i * 2^-48)
 *   GREEDY (mode 0): start from b = 0 and, budget times, give one more bit to the
 *     block with the largest gain E_i * dD[b_i] among blocks with b_i < 8;
 *     gains are RN_fp64 products; ties go to the lowest block index.
 *   UNIFORM (mode 1): b_i = budget / nb (budget divisible by nb).
 *   budget == 16*nb: every block is 16 (raw binary16 passthrough).
 *   sigma_i = RN_fp32(sqrt(E_i / (2 E_tot))), E_tot = RN_fp64(sum_i energy_i * 2^-48);
 *   sigma = 0 when E_tot = 0.
 * dD[b] (b = 0..7) is the drop in Gaussian Lloyd-Max distortion from b to b+1
 * bits, as a binary32 value.  Returns 0, or -3 for an invalid budget.
 */
int or_allocate(const uint64_t *energy, int n_units, int nb, int budget, int mode,
                const float *dD, uint8_t *bits, float *sigma)
{
    int pass = (budget == 16 * nb);
    if (!pass) {
        if (budget < 0 || budget > 8 * nb) return -3;
        if (mode == 1 && budget % nb) return -3;
    }
    for (int u = 0; u < n_units; u++) {
        double E[128];
        u128 tot = 0;
        for (int i = 0; i < nb; i++) {
            u128 e = (u128)energy[(u * nb + i) * 2] | ((u128)energy[(u * nb + i) * 2 + 1] << 64);
            tot += e;
            E[i] = ldexp(u128_to_double(e), -48);
        }
        double Etot = ldexp(u128_to_double(tot), -48);
        uint8_t *b = bits + (size_t)u * nb;
        if (pass) {
            for (int i = 0; i < nb; i++) b[i] = 16;
        } else if (mode == 1) {
            for (int i = 0; i < nb; i++) b[i] = (uint8_t)(budget / nb);
        } else {
            for (int i = 0; i < nb; i++) b[i] = 0;
            for (int step = 0; step < budget; step++) {
                int best = -1;
                double bg = 0;
                for (int i = 0; i < nb; i++) {
                    if (b[i] >= 8) continue;
                    double g = E[i] * (double)dD[b[i]];
                    if (best < 0 || g > bg) { best = i; bg = g; }
                }
                b[best] += 1;
            }
        }
        for (int i = 0; i < nb; i++)
            sigma[(size_t)u * nb + i] = (Etot > 0) ? (float)sqrt(E[i] / (2.0 * Etot)) : 0.0f;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Per-token scale and codes                                                 */
/* ------------------------------------------------------------------------- */

/*
 * Per-token scale s = sqrt_RN_fp32(T(x_0^2, ..., x_{d-1}^2)) where each square is
 * formed in binary32 (exact for binary16 inputs) and T is the balanced pairwise
 * binary32 sum in coordinate order: (0+1), (2+3), ... then pairs of those, up to
 * the root.  d must be a power of two.
 */
float or_token_scale(const uint16_t *x, int d)
{
    float buf[256];
    for (int c = 0; c < d; c++) { float v = (float)h2d(x[c]); buf[c] = v * v; }
    for (int n = d; n > 1; n /= 2)
        for (int j = 0; j < n / 2; j++) buf[j] = buf[2 * j] + buf[2 * j + 1];
    return sqrtf(buf[0]);
}

/*
 * Code of one coordinate x in a block of width w (1..8) with block scale sig and
 * token scale s: the number of thresholds j = 1..2^w-1 with
 *   x >= RN32(s * RN32(sig * thr[j])),
 * where thr[j] is the binary32 midpoint of binary16 levels j-1 and j.
 * (IEEE comparisons: -0 == +0, NaN compares false.)
 */
static int code_of(float x, int w, float sig, float s, const float *thr)
{
    int n = 0;
    for (int j = 1; j < (1 << w); j++) {
        float a = sig * thr[j];
        float b = s * a;
        if (x >= b) n++;
    }
    return n;
}

/*
 * Encode n tokens of one KV head.
 *   x         : binary16 rows, token t at x + t*stride_tok (d contiguous values)
 *   width     : per-coordinate widths [d] (0..8 or 16)
 *   sig       : per-coordinate block scale [d]
 *   thr_tab   : thresholds for widths 1..8 concatenated; width w starts at
 *               thr_off[w] and holds 2^w entries (index 0 unused)
 * Outputs codes[n][d] (uint16: raw bits for width 16, 0 for width 0) and scale[n].
 */
void or_encode(const uint16_t *x, int64_t n, int64_t stride_tok, int d, const int *width,
               const float *sig, const float *thr_tab, const int *thr_off,
               uint16_t *codes, float *scale)
{
    for (int64_t t = 0; t < n; t++) {
        const uint16_t *row = x + t * stride_tok;
        float s = or_token_scale(row, d);
        scale[t] = s;
        for (int c = 0; c < d; c++) {
            int w = width[c];
            uint16_t code;
            if (w == 0) code = 0;
            else if (w == 16) code = row[c];
            else code = (uint16_t)code_of((float)h2d(row[c]), w, sig[c], s, thr_tab + thr_off[w]);
            codes[t * d + c] = code;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Packed layout, version 1                                                  */
/* ------------------------------------------------------------------------- */
/*
 * Per (sequence, layer) region: [H_kv][capacity/64 tiles][tile bytes].
 * A tile holds 64 token slots:
 *   K section  : 64 records of SK bytes, SK = 16*ceil(2*k_budget/128);
 *                record p is slot p's K codes as an LSB-first bitstream (bit b of
 *                the stream is bit b%8 of byte b/8) in K order: blocks sorted by
 *                width descending (stable, lower block index first), each block
 *                contributing its two coordinates p(i) then q(i), width-0 blocks
 *                omitted; each field is w bits (16 bits for passthrough).
 *   V section  : d runs of 8*v bytes; run c holds the 64 slots' codes of
 *                coordinate c, slot p at bits [p*v, p*v+v) of the run.
 *   K scales   : 64 binary32
 *   V scales   : 64 binary32
 * Unused slots are all-zero bytes.
 */
int64_t or_tile_bytes(int d, int k_budget, int v_bits)
{
    int64_t sk = 16 * ((2 * (int64_t)k_budget + 127) / 128);
    return 64 * sk + (int64_t)d * 8 * v_bits + 2 * 64 * 4;
}

static void put_bits(uint8_t *buf, int64_t bitpos, uint32_t val, int w)
{
    for (int b = 0; b < w; b++)
        if ((val >> b) & 1) buf[(bitpos + b) >> 3] |= (uint8_t)(1u << ((bitpos + b) & 7));
}

static uint32_t get_bits(const uint8_t *buf, int64_t bitpos, int w)
{
    uint32_t v = 0;
    for (int b = 0; b < w; b++) v |= (uint32_t)((buf[(bitpos + b) >> 3] >> ((bitpos + b) & 7)) & 1) << b;
    return v;
}

/* K order: list of coordinates; returns its length */
int or_k_order(int d, int pairing, const uint8_t *bits_blk, int *order)
{
    int nb = d / 2, len = 0;
    for (int w = 16; w >= 1; w--)
        for (int i = 0; i < nb; i++)
            if (bits_blk[i] == w) {
                int p, q;
                block_coords(d, pairing, i, &p, &q);
                order[len++] = p;
                order[len++] = q;
            }
    return len;
}

/*
 * Pack tokens into one head's tile sequence (ORs into zero-initialised memory).
 * region points at this head's first tile.  Token t (0..n-1) goes to slot
 * first_slot + t.  kcodes/vcodes are [n][d]; kscale/vscale are [n].
 */
void or_pack(uint8_t *region, int d, int pairing, int k_budget, int v_bits,
             const uint8_t *kbits_blk, int64_t first_slot, int64_t n,
             const uint16_t *kcodes, const uint16_t *vcodes, const float *kscale, const float *vscale)
{
    int order[256];
    int nk = or_k_order(d, pairing, kbits_blk, order);
    int width[256];
    for (int i = 0; i < d / 2; i++) {
        int p, q;
        block_coords(d, pairing, i, &p, &q);
        width[p] = width[q] = kbits_blk[i];
    }
    int64_t tile = or_tile_bytes(d, k_budget, v_bits);
    int64_t sk = 16 * ((2 * (int64_t)k_budget + 127) / 128);
    for (int64_t t = 0; t < n; t++) {
        int64_t slot = first_slot + t;
        uint8_t *tb = region + (slot / 64) * tile;
        int p = (int)(slot % 64);
        uint8_t *rec = tb + p * sk;
        int64_t pos = 0;
        for (int f = 0; f < nk; f++) {
            int c = order[f];
            put_bits(rec, pos, kcodes[t * d + c], width[c]);
            pos += width[c];
        }
        uint8_t *vsec = tb + 64 * sk;
        for (int c = 0; c < d; c++)
            put_bits(vsec + (int64_t)c * 8 * v_bits, (int64_t)p * v_bits, vcodes[t * d + c], v_bits);
        float *ks = (float *)(tb + 64 * sk + (int64_t)d * 8 * v_bits);
        ks[p] = kscale[t];
        ks[64 + p] = vscale[t];
    }
}

/* Inverse of or_pack for slots [first_slot, first_slot + n). */
void or_unpack(const uint8_t *region, int d, int pairing, int k_budget, int v_bits,
               const uint8_t *kbits_blk, int64_t first_slot, int64_t n,
               uint16_t *kcodes, uint16_t *vcodes, float *kscale, float *vscale)
{
    int order[256];
    int nk = or_k_order(d, pairing, kbits_blk, order);
    int width[256];
    for (int i = 0; i < d / 2; i++) {
        int p, q;
        block_coords(d, pairing, i, &p, &q);
        width[p] = width[q] = kbits_blk[i];
    }
    int64_t tile = or_tile_bytes(d, k_budget, v_bits);
    int64_t sk = 16 * ((2 * (int64_t)k_budget + 127) / 128);
    for (int64_t t = 0; t < n; t++) {
        int64_t slot = first_slot + t;
        const uint8_t *tb = region + (slot / 64) * tile;
        int p = (int)(slot % 64);
        const uint8_t *rec = tb + p * sk;
        for (int c = 0; c < d; c++) kcodes[t * d + c] = 0;
        int64_t pos = 0;
        for (int f = 0; f < nk; f++) {
            int c = order[f];
            kcodes[t * d + c] = (uint16_t)get_bits(rec, pos, width[c]);
            pos += width[c];
        }
        const uint8_t *vsec = tb + 64 * sk;
        for (int c = 0; c < d; c++)
            vcodes[t * d + c] = (uint16_t)get_bits(vsec + (int64_t)c * 8 * v_bits, (int64_t)p * v_bits, v_bits);
        const float *ks = (const float *)(tb + 64 * sk + (int64_t)d * 8 * v_bits);
        kscale[t] = ks[p];
        vscale[t] = ks[64 + p];
    }
}

/* ------------------------------------------------------------------------- */
/* Dequantization and exact attention                                        */
/* ------------------------------------------------------------------------- */

/*
 * Dequantized value of one coordinate, in fp64:
 *   width 0  -> 0
 *   width 16 -> the binary16 value itself
 *   else     -> s * sig * level_w[code]   (level_w = binary16-rounded Lloyd-Max level)
 * levels: binary16 patterns for widths 1..8 concatenated, width w at lev_off[w].
 */
static double dequant(uint16_t code, int w, double s, double sig, const uint16_t *levels, const int *lev_off)
{
    if (w == 0) return 0.0;
    if (w == 16) return h2d(code);
    return s * sig * h2d(levels[lev_off[w] + code]);
}

void or_dequant(const uint16_t *codes, int64_t n, int d, const int *width, const float *sig,
                const float *scale, const uint16_t *levels, const int *lev_off, double *out)
{
    for (int64_t t = 0; t < n; t++)
        for (int c = 0; c < d; c++)
            out[t * d + c] = dequant(codes[t * d + c], width[c], scale[t], sig[c], levels, lev_off);
}

/*
 * Exact softmax attention of one query over n dequantized keys/values (fp64):
 *   z_t = scale * sum_c q_c khat_{t,c};  p = softmax(z);  o = sum_t p_t vhat_t.
 * n == 0 gives o = 0.
 */
void or_attend(const double *q, const double *khat, const double *vhat, int64_t n, int d,
               double scale, double *o)
{
    for (int c = 0; c < d; c++) o[c] = 0;
    if (n == 0) return;
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int64_t t = 0; t < n; t++) {
        double s = 0;
        for (int c = 0; c < d; c++) s += q[c] * khat[t * d + c];
        z[t] = scale * s;
        if (z[t] > m) m = z[t];
    }
    double l = 0;
    for (int64_t t = 0; t < n; t++) { z[t] = exp(z[t] - m); l += z[t]; }
    for (int64_t t = 0; t < n; t++)
        for (int c = 0; c < d; c++) o[c] += z[t] * vhat[t * d + c];
    for (int c = 0; c < d; c++) o[c] /= l;
    free(z);
}

/*
 * Decode attention straight from one sequence's packed region for every query
 * head (GQA: query head h reads KV head h / (n_q_heads / n_kv_heads)).
 *   region   : [n_kv][n_tiles][tile] bytes
 *   q        : binary16 [n_q][d]
 *   kbits    : [n_kv][d/2] block widths, ksig/vsig: [n_kv][d/2] block scales
 *   out      : fp64 [n_q][d]
 * Heads run in parallel (OpenMP); each head is the plain computation above.
 */
void or_decode_attention(const uint8_t *region, int64_t n_tiles, int n_kv, int n_q, int d, int pairing,
                         int k_budget, int v_bits, const uint8_t *kbits, const float *ksig,
                         const float *vsig, const uint16_t *levels, const int *lev_off,
                         const uint16_t *q, int64_t seq_len, double scale, double *out)
{
    int64_t tile = or_tile_bytes(d, k_budget, v_bits);
    int g = n_q / n_kv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < n_q; h++) {
        int kv = h / g;
        const uint8_t *reg = region + (int64_t)kv * n_tiles * tile;
        int nb = d / 2;
        int kw[256], vw[256];
        float ks[256], vs[256];
        for (int i = 0; i < nb; i++) {
            int p, qq;
            block_coords(d, pairing, i, &p, &qq);
            kw[p] = kw[qq] = kbits[kv * nb + i];
            vw[p] = vw[qq] = v_bits;
            ks[p] = ks[qq] = ksig[kv * nb + i];
            vs[p] = vs[qq] = vsig[kv * nb + i];
        }
        uint16_t *kc = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(seq_len > 0 ? seq_len : 1) * d);
        uint16_t *vc = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(seq_len > 0 ? seq_len : 1) * d);
        float *kscale = (float *)malloc(sizeof(float) * (size_t)(seq_len > 0 ? seq_len : 1));
        float *vscale = (float *)malloc(sizeof(float) * (size_t)(seq_len > 0 ? seq_len : 1));
        double *kh = (double *)malloc(sizeof(double) * (size_t)(seq_len > 0 ? seq_len : 1) * d);
        double *vh = (double *)malloc(sizeof(double) * (size_t)(seq_len > 0 ? seq_len : 1) * d);
        or_unpack(reg, d, pairing, k_budget, v_bits, kbits + kv * nb, 0, seq_len, kc, vc, kscale, vscale);
        or_dequant(kc, seq_len, d, kw, ks, kscale, levels, lev_off, kh);
        or_dequant(vc, seq_len, d, vw, vs, vscale, levels, lev_off, vh);
        double qd[256];
        for (int c = 0; c < d; c++) qd[c] = h2d(q[h * d + c]);
        or_attend(qd, kh, vh, seq_len, d, scale, out + (int64_t)h * d);
        free(kc); free(vc); free(kscale); free(vscale); free(kh); free(vh);
    }
}

/*
 * Decode attention over a packed prefix plus an fp16 window of the most recent
 * tokens (the recent-key buffer variant: those tokens are kept unquantized).
 *   slots [0, n_packed) of the packed region, dequantized as above, followed by
 *   the n_win window tokens wk/wv : binary16 [n_win][n_kv][d] in sequence order,
 *   taken at their exact binary16 values;
 * then the same exact softmax attention over all n_packed + n_win tokens.
 */
void or_decode_attention_window(const uint8_t *region, int64_t n_tiles, int n_kv, int n_q, int d, int pairing,
                                int k_budget, int v_bits, const uint8_t *kbits, const float *ksig,
                                const float *vsig, const uint16_t *levels, const int *lev_off,
                                const uint16_t *q, int64_t n_packed, const uint16_t *wk, const uint16_t *wv,
                                int64_t n_win, double scale, double *out)
{
    int64_t tile = or_tile_bytes(d, k_budget, v_bits);
    int g = n_q / n_kv;
    int64_t n = n_packed + n_win;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < n_q; h++) {
        int kv = h / g;
        const uint8_t *reg = region + (int64_t)kv * n_tiles * tile;
        int nb = d / 2;
        int kw[256], vw[256];
        float ks[256], vs[256];
        for (int i = 0; i < nb; i++) {
            int p, qq;
            block_coords(d, pairing, i, &p, &qq);
            kw[p] = kw[qq] = kbits[kv * nb + i];
            vw[p] = vw[qq] = v_bits;
            ks[p] = ks[qq] = ksig[kv * nb + i];
            vs[p] = vs[qq] = vsig[kv * nb + i];
        }
        size_t np1 = (size_t)(n_packed > 0 ? n_packed : 1), n1 = (size_t)(n > 0 ? n : 1);
        uint16_t *kc = (uint16_t *)malloc(sizeof(uint16_t) * np1 * d);
        uint16_t *vc = (uint16_t *)malloc(sizeof(uint16_t) * np1 * d);
        float *kscale = (float *)malloc(sizeof(float) * np1);
        float *vscale = (float *)malloc(sizeof(float) * np1);
        double *kh = (double *)malloc(sizeof(double) * n1 * d);
        double *vh = (double *)malloc(sizeof(double) * n1 * d);
        or_unpack(reg, d, pairing, k_budget, v_bits, kbits + kv * nb, 0, n_packed, kc, vc, kscale, vscale);
        or_dequant(kc, n_packed, d, kw, ks, kscale, levels, lev_off, kh);
        or_dequant(vc, n_packed, d, vw, vs, vscale, levels, lev_off, vh);
        for (int64_t t = 0; t < n_win; t++)
            for (int c = 0; c < d; c++) {
                kh[(n_packed + t) * d + c] = h2d(wk[(t * n_kv + kv) * d + c]);
                vh[(n_packed + t) * d + c] = h2d(wv[(t * n_kv + kv) * d + c]);
            }
        double qd[256];
        for (int c = 0; c < d; c++) qd[c] = h2d(q[h * d + c]);
        or_attend(qd, kh, vh, n, d, scale, out + (int64_t)h * d);
        free(kc); free(vc); free(kscale); free(vscale); free(kh); free(vh);
    }
}

/*
 * Chunked prefill attention over the packed cache (causal): a chunk of n_tok
 * queries whose first sits at position q_start; query j (position q_start + j)
 * attends slots [0, q_start + j] of the packed region -- the chunk's own tokens are
 * read from the packed cache too, so they must have been packed before the call.
 * Each query row is the same exact softmax attention as decode at length
 * q_start + j + 1 (the page's packed-cache serving path, with the causal mask of
 * ordinary prefill).
 *   q   : binary16 [n_tok][n_q][d]
 *   out : fp64     [n_tok][n_q][d]
 */
void or_prefill_attention(const uint8_t *region, int64_t n_tiles, int n_kv, int n_q, int d, int pairing,
                          int k_budget, int v_bits, const uint8_t *kbits, const float *ksig, const float *vsig,
                          const uint16_t *levels, const int *lev_off, const uint16_t *q, int64_t q_start,
                          int64_t n_tok, double scale, double *out)
{
    int64_t tile = or_tile_bytes(d, k_budget, v_bits);
    int g = n_q / n_kv;
    int64_t n = q_start + n_tok;  /* slots any query of the chunk may read */
    size_t n1 = (size_t)(n > 0 ? n : 1);
#pragma omp parallel for schedule(dynamic, 1)
    for (int kv = 0; kv < n_kv; kv++) {
        const uint8_t *reg = region + (int64_t)kv * n_tiles * tile;
        int nb = d / 2;
        int kw[256], vw[256];
        float ks[256], vs[256];
        for (int i = 0; i < nb; i++) {
            int p, qq;
            block_coords(d, pairing, i, &p, &qq);
            kw[p] = kw[qq] = kbits[kv * nb + i];
            vw[p] = vw[qq] = v_bits;
            ks[p] = ks[qq] = ksig[kv * nb + i];
            vs[p] = vs[qq] = vsig[kv * nb + i];
        }
        uint16_t *kc = (uint16_t *)malloc(sizeof(uint16_t) * n1 * d);
        uint16_t *vc = (uint16_t *)malloc(sizeof(uint16_t) * n1 * d);
        float *kscale = (float *)malloc(sizeof(float) * n1);
        float *vscale = (float *)malloc(sizeof(float) * n1);
        double *kh = (double *)malloc(sizeof(double) * n1 * d);
        double *vh = (double *)malloc(sizeof(double) * n1 * d);
        or_unpack(reg, d, pairing, k_budget, v_bits, kbits + kv * nb, 0, n, kc, vc, kscale, vscale);
        or_dequant(kc, n, d, kw, ks, kscale, levels, lev_off, kh);
        or_dequant(vc, n, d, vw, vs, vscale, levels, lev_off, vh);
        double qd[256];
        for (int64_t j = 0; j < n_tok; j++)
            for (int h = kv * g; h < (kv + 1) * g; h++) {
                for (int c = 0; c < d; c++) qd[c] = h2d(q[(j * n_q + h) * d + c]);
                or_attend(qd, kh, vh, q_start + j + 1, d, scale, out + (j * n_q + h) * d);
            }
        free(kc); free(vc); free(kscale); free(vscale); free(kh); free(vh);
    }
}

/* ------------------------------------------------------------------------- */
/* Split attention and the log-sum-exp merge                                 */
/* ------------------------------------------------------------------------- */
/*
 * A long sequence is attended in chunks whose partial results are combined
 * afterwards (the split-K softmax merge).  The partial of one query over a chunk of
 * n tokens is, with logits taken in log2 units (z_t = scale * log2(e) * q.khat_t):
 *   m = max_t z_t   (-inf for an empty chunk),
 *   l = sum_t 2^(z_t - m),
 *   o_c = sum_t 2^(z_t - m) vhat_{t,c}   (unnormalised).
 * Any reference value in place of the maximum gives the same merged result, as long
 * as l and o use the same one.
 */
void or_attend_partial(const double *q, const double *khat, const double *vhat, int64_t n, int d,
                       double scale, double *m, double *l, double *o)
{
    for (int c = 0; c < d; c++) o[c] = 0;
    *m = -INFINITY;
    *l = 0;
    if (n == 0) return;
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; t++) {
        double s = 0;
        for (int c = 0; c < d; c++) s += q[c] * khat[t * d + c];
        z[t] = scale * M_LOG2E * s;
        if (z[t] > mx) mx = z[t];
    }
    double lsum = 0;
    for (int64_t t = 0; t < n; t++) {
        double w = exp2(z[t] - mx);
        lsum += w;
        for (int c = 0; c < d; c++) o[c] += w * vhat[t * d + c];
    }
    *m = mx;
    *l = lsum;
    free(z);
}

/*
 * Merge of n_split partials of rows, in the library's partials format:
 *   part[(row * n_split + j) * (d + 2) + {0: m_j, 1: l_j, 2 + c: o_j,c}]  (binary32)
 * out[row][c] = sum_j 2^(m_j - M) o_j,c / sum_j 2^(m_j - M) l_j with M = max_j m_j,
 * computed in fp64; a row whose partials are all empty (M = -inf) or whose weight sum
 * is 0 gives 0.
 */
void or_merge_partials(const float *part, int64_t n_rows, int n_split, int d, double *out)
{
    for (int64_t r = 0; r < n_rows; r++) {
        const float *p = part + r * n_split * (int64_t)(d + 2);
        double M = -INFINITY;
        for (int j = 0; j < n_split; j++)
            if ((double)p[j * (d + 2)] > M) M = p[j * (d + 2)];
        double L = 0;
        double *o = out + r * d;
        for (int c = 0; c < d; c++) o[c] = 0;
        if (M == -INFINITY) continue;
        for (int j = 0; j < n_split; j++) {
            const float *pj = p + j * (d + 2);
            if ((double)pj[0] == -INFINITY) continue;
            double w = exp2((double)pj[0] - M);
            L += w * (double)pj[1];
            for (int c = 0; c < d; c++) o[c] += w * (double)pj[2 + c];
        }
        for (int c = 0; c < d; c++) o[c] = (L > 0) ? o[c] / L : 0.0;
    }
}

/* ------------------------------------------------------------------------- */
/* Randomized Walsh-Hadamard rotation (TurboQuant-MSE proper)                */
/* ------------------------------------------------------------------------- */
/*
 * TQ-MSE rotates each vector by a random orthogonal matrix before scalar
 * quantization, so that every rotated coordinate of a unit vector follows (about)
 * N(0, 1/d) and one Gaussian codebook serves all coordinates.  The rotation read
 * here is R = H diag(sg) / sqrt(d): H the d x d Sylvester Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)), sg a seeded vector of signs (an input: sg_j =
 * -1 where signs[j] is 1, else +1).  R is orthogonal, so ||R x|| = ||x||.
 *
 * Exact rotated sums: for binary16 x, S_i = sum_j H[i][j] sg_j x_j = sqrt(d) (R x)_i
 * is a sum of +-multiples of 2^-24 below 2^47 in magnitude, kept exactly as an
 * integer count of 2^-24 and rounded once to binary32.
 */
static int hsign(int i, int j) { return __builtin_popcount((unsigned)(i & j)) & 1 ? -1 : 1; }

/* integer value of a finite binary16 in units of 2^-24 */
static int64_t h2units(uint16_t h)
{
    int e = (h >> 10) & 31, m = h & 1023;
    int64_t M = (e == 0) ? m : (1024 + m);
    int64_t v = (e == 0) ? M : (M << (e - 1));
    return (h >> 15) ? -v : v;
}

/* exact S_i = sum_j H[i][j] sg_j x_j (units of 2^-24) for a binary16 row x[d] */
void or_hadamard_units(const uint16_t *x, int d, const uint8_t *signs, int64_t *S)
{
    for (int i = 0; i < d; i++) {
        int64_t acc = 0;
        for (int j = 0; j < d; j++) {
            int64_t t = h2units(x[j]);
            if (signs[j]) t = -t;
            acc += hsign(i, j) * t;
        }
        S[i] = acc;
    }
}

/* the rotated sums rounded once to binary32: RN32(S_i * 2^-24) */
void or_hadamard_f32(const uint16_t *x, int d, const uint8_t *signs, float *S)
{
    int64_t u[256];
    or_hadamard_units(x, d, signs, u);
    for (int i = 0; i < d; i++) S[i] = ldexpf((float)u[i], -24);  /* int64 -> float is RN; the scaling is exact */
}

/*
 * Codes of n binary16 rows under the rotation (all coordinates at width w, 1..8):
 *   s = or_token_scale(x) (the norm of the unrotated row; R keeps it);
 *   code_i = #{ j in 1..2^w-1 : S_i >= RN32(s * t_w[j]) }.
 * In exact arithmetic this compares the normalised rotated coordinate
 * (R x)_i sqrt(d) / s with the Gaussian thresholds t_w: the codebook N(0, 1/d) at
 * scale s.  Outputs codes [n][d] and scale [n].
 */
void or_rot_encode(const uint16_t *x, int64_t n, int64_t stride_tok, int d, int w, const uint8_t *signs,
                   const float *thr_tab, const int *thr_off, uint16_t *codes, float *scale)
{
    float S[256];
    for (int64_t t = 0; t < n; t++) {
        const uint16_t *row = x + t * stride_tok;
        float s = or_token_scale(row, d);
        scale[t] = s;
        or_hadamard_f32(row, d, signs, S);
        const float *thr = thr_tab + thr_off[w];
        for (int c = 0; c < d; c++) {
            int k = 0;
            for (int j = 1; j < (1 << w); j++) {
                float b = s * thr[j];
                if (S[c] >= b) k++;
            }
            codes[t * d + c] = (uint16_t)k;
        }
    }
}

/* binary16 query rotated once: RN16(RN32(RN32(S_i) * sigma)), sigma = RN32(1/sqrt(d)) */
void or_rot_query(const uint16_t *q, int d, const uint8_t *signs, float sigma, uint16_t *out)
{
    float S[256];
    or_hadamard_f32(q, d, signs, S);
    for (int i = 0; i < d; i++) {
        float p = S[i] * sigma;
        out[i] = d2h((double)p);
    }
}

/* x = R^T y = diag(sg) H y / sqrt(d), fp64 (the output rotated back) */
void or_rot_back(const double *y, int d, const uint8_t *signs, double *x)
{
    for (int j = 0; j < d; j++) {
        double acc = 0;
        for (int i = 0; i < d; i++) acc += hsign(i, j) * y[i];
        acc /= sqrt((double)d);
        x[j] = signs[j] ? -acc : acc;
    }
}

/* thread count of the OpenMP loops above (a timing control: results do not depend on it) */
void or_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int or_max_threads(void) { return omp_get_max_threads(); }
