/*
 * lct_oracle.c -- plain, serial CPU oracle of the LCT lossless BF16 exponent codec.
 *
 * TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  Plain C99, one
 * thread, no SIMD intrinsics, no tables shared with the HIP library.
 * Compile without -ffast-math and with -ffp-contract=off: the SGD step relies
 * on the C library's correctly rounded fmaf and on IEEE subnormals.
 *
 * Page citations (title, then passage):
 *   [LCT-abs]     "LCT: Losslessly Compressed Tensors with GPU friendly execution
 *                 for Training", abstract.
 *   [EXP-split]   "LCT paper - Lossless Huffman coding of BF16 training tensors",
 *                 paragraph that splits the 16 bits into a sign-fraction byte and
 *                 an exponent byte, caps codes at 8 bits, adds one escape prefix
 *                 with an 8-bit literal, and shifts a precomputed codebook.
 *   [EXP-streams] same page, paragraph on 65,536 / 32,768-element blocks cut into
 *                 256 round-robin streams of fixed length, with an overflow
 *                 region whose start is marked.
 *   [EXP-train]   same page, paragraph on training traffic and the fused SGD
 *                 update W_{t+1} = W_t - eta * M_t.
 *   [EXP-ideal]   same page, paragraph with the idealized arithmetic (16/11,
 *                 1.4382x for CLEAN).
 *   [EXP-jargon]  same page, jargon entry "Optimizer state": the momentum
 *                 buffer of SGD with momentum, kept for every weight.
 */
#include "lct_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define NSTREAM 256
#define MAXLEN 8

/* ------------------------------------------------------------------------ */
/* Byte split ([EXP-split]): 1 sign + 8 exponent + 7 fraction bits.  The     */
/* sign-fraction byte keeps BF16's own bit order: sign at bit 7, fraction in */
/* bits 6..0.                                                                */
/* ------------------------------------------------------------------------ */
uint8_t lcto_exponent(uint16_t v) { return (uint8_t)((v >> 7) & 0xFFu); }
uint8_t lcto_signfrac(uint16_t v) { return (uint8_t)(((v >> 8) & 0x80u) | (v & 0x7Fu)); }
uint16_t lcto_join(uint8_t sf, uint8_t e)
{
    return (uint16_t)(((unsigned)(sf & 0x80u) << 8) | ((unsigned)e << 7) | (sf & 0x7Fu));
}

/* ------------------------------------------------------------------------ */
/* Model ([EXP-split]: the user picks a Gaussian, Laplace or power-law       */
/* model).  The power-law model is a Student-t with shape = degrees of       */
/* freedom.  All three are symmetric, so only |X| matters.                   */
/* ------------------------------------------------------------------------ */

static const double TINY = 1e-300;

/* g = 1 + d1/(1 + d2/(1 + ...)), the continued fraction of the regularized
 * incomplete beta function, evaluated with the modified Lentz method. */
static double incbeta_cf(double a, double b, double x)
{
    double g = 1.0, C = 1.0, D = 0.0;
    for (int j = 1; j <= 100000; j++) {
        int m = j / 2;
        double dj;
        if (j & 1)
            dj = -(a + m) * (a + b + m) * x / ((a + 2.0 * m) * (a + 2.0 * m + 1.0));
        else
            dj = m * (b - m) * x / ((a + 2.0 * m - 1.0) * (a + 2.0 * m));
        D = 1.0 + dj * D;
        if (fabs(D) < TINY) D = TINY;
        D = 1.0 / D;
        C = 1.0 + dj / C;
        if (fabs(C) < TINY) C = TINY;
        double delta = C * D;
        g *= delta;
        if (fabs(delta - 1.0) < 1e-16) break;
    }
    return g;
}

/* I_x(a, b) with x and y = 1 - x both given (y is passed separately so that
 * values of x near 1 keep their precision). */
static double incbeta(double a, double b, double x, double y)
{
    if (x <= 0.0) return 0.0;
    if (y <= 0.0) return 1.0;
    double lnbeta = lgamma(a) + lgamma(b) - lgamma(a + b);
    if (x < (a + 1.0) / (a + b + 2.0)) {
        double lnpre = a * log(x) + b * log(y) - lnbeta;
        return exp(lnpre) / (a * incbeta_cf(a, b, x));
    }
    double lnpre = b * log(y) + a * log(x) - lnbeta;
    return 1.0 - exp(lnpre) / (b * incbeta_cf(b, a, y));
}

double lcto_model_survival(int family, double scale, double shape, double t)
{
    switch (family) {
    case LCTO_GAUSSIAN: /* P(|X| > t), X ~ N(0, scale^2) */
        return erfc(t / (scale * sqrt(2.0)));
    case LCTO_LAPLACE:  /* P(|X| > t), X ~ Laplace(0, scale) */
        return exp(-t / scale);
    case LCTO_POWERLAW: { /* P(|T| > t), T = scale * t_nu */
        double u = t / scale, nu = shape;
        double x = nu / (nu + u * u), y = (u * u) / (nu + u * u);
        return incbeta(0.5 * nu, 0.5, x, y);
    }
    default:
        return NAN;
    }
}

/* Exponent field e in 1..254 holds |x| in [2^(e-127), 2^(e-126)); field 0
 * holds zero and the subnormals (|x| < 2^-126); field 255 (inf, NaN) has no
 * model mass. */
int lcto_model_pmf(int family, double scale, double shape, double p[256])
{
    if (family < LCTO_GAUSSIAN || family > LCTO_POWERLAW) return LCTO_EINVAL;
    if (!(scale > 0.0) || !isfinite(scale)) return LCTO_EINVAL;
    if (family == LCTO_POWERLAW && (!(shape > 0.0) || !isfinite(shape))) return LCTO_EINVAL;
    p[0] = 1.0 - lcto_model_survival(family, scale, shape, ldexp(1.0, -126));
    for (int e = 1; e <= 254; e++) {
        double lo = lcto_model_survival(family, scale, shape, ldexp(1.0, e - 127));
        double hi = lcto_model_survival(family, scale, shape, ldexp(1.0, e - 126));
        double q = lo - hi;
        p[e] = q > 0.0 ? q : 0.0;
    }
    p[255] = 0.0;
    return LCTO_OK;
}

void lcto_weights(const double p[256], uint64_t w[256])
{
    for (int e = 0; e < 256; e++) w[e] = (uint64_t)floor(p[e] * 1099511627776.0 + 0.5);
}

/* ------------------------------------------------------------------------ */
/* Length-limited Huffman code ([EXP-split]: codes capped at 8 bits), by     */
/* package-merge (Larmore and Hirschberg, 1990), in its coin-collector form: */
/* level L holds the leaves; each shallower level holds the leaves merged    */
/* with pairs of consecutive items of the level below.  The first 2n-2 items */
/* of level 1 are kept, and a leaf's code length is how often it occurs in   */
/* them once every package is expanded.                                      */
/* ------------------------------------------------------------------------ */

typedef struct {
    uint64_t w;
    int leaf;   /* leaf index, or -1 for a package */
    int a, b;   /* for a package: its two items, on the level below */
} pm_item;

#define PM_MAXN 512
static pm_item pm_lvl[MAXLEN + 2][2 * PM_MAXN];
static int pm_cnt[MAXLEN + 2];

static void pm_expand(int d, int i, uint8_t *len)
{
    const pm_item *it = &pm_lvl[d][i];
    if (it->leaf >= 0) {
        len[it->leaf]++;
        return;
    }
    pm_expand(d + 1, it->a, len);
    pm_expand(d + 1, it->b, len);
}

int lcto_package_merge(int n, const uint64_t *w, const int *id, int L, uint8_t *len)
{
    if (L < 1 || L > MAXLEN || n < 2 || n > PM_MAXN || n > (1 << L)) return LCTO_EINVAL;

    /* leaves ordered by (weight, id): insertion sort, n is small */
    int order[PM_MAXN];
    for (int i = 0; i < n; i++) {
        int j = i;
        while (j > 0) {
            int o = order[j - 1];
            if (w[o] > w[i] || (w[o] == w[i] && id[o] > id[i])) {
                order[j] = o;
                j--;
            } else {
                break;
            }
        }
        order[j] = i;
    }

    for (int i = 0; i < n; i++) {
        pm_lvl[L][i].w = w[order[i]];
        pm_lvl[L][i].leaf = order[i];
        pm_lvl[L][i].a = pm_lvl[L][i].b = -1;
    }
    pm_cnt[L] = n;

    for (int d = L - 1; d >= 1; d--) {
        int npk = pm_cnt[d + 1] / 2;   /* an odd last item is dropped */
        int li = 0, pi = 0, k = 0;
        while (li < n || pi < npk) {
            uint64_t pw = 0;
            if (pi < npk) pw = pm_lvl[d + 1][2 * pi].w + pm_lvl[d + 1][2 * pi + 1].w;
            /* at equal weight the leaf goes first */
            if (li < n && (pi >= npk || w[order[li]] <= pw)) {
                pm_lvl[d][k].w = w[order[li]];
                pm_lvl[d][k].leaf = order[li];
                pm_lvl[d][k].a = pm_lvl[d][k].b = -1;
                li++;
            } else {
                pm_lvl[d][k].w = pw;
                pm_lvl[d][k].leaf = -1;
                pm_lvl[d][k].a = 2 * pi;
                pm_lvl[d][k].b = 2 * pi + 1;
                pi++;
            }
            k++;
        }
        pm_cnt[d] = k;
    }

    memset(len, 0, (size_t)n);
    if (pm_cnt[1] < 2 * n - 2) return LCTO_EINVAL;
    for (int i = 0; i < 2 * n - 2; i++) pm_expand(1, i, len);
    return LCTO_OK;
}

/* ------------------------------------------------------------------------ */
/* Escape set ([EXP-split]: rare exponents grouped under one escape prefix   */
/* followed by an 8-bit literal).  "Rare" is read as: all but the k heaviest */
/* symbols, with k chosen to minimise the expected bits.                     */
/* ------------------------------------------------------------------------ */
uint64_t lcto_build_escape(int nsym, const uint64_t *w, int L, int lit_bits,
                           uint8_t *len, uint8_t *esc_len, int *k_out)
{
    if (nsym < 2 || nsym > PM_MAXN - 1 || L < 1 || L > MAXLEN || lit_bits < 0) return UINT64_MAX;

    /* symbols ranked by (weight descending, id ascending) */
    int rank[PM_MAXN];
    for (int i = 0; i < nsym; i++) {
        int j = i;
        while (j > 0) {
            int o = rank[j - 1];
            if (w[o] < w[i] || (w[o] == w[i] && o > i)) {
                rank[j] = o;
                j--;
            } else {
                break;
            }
        }
        rank[j] = i;
    }
    int nz = 0;
    for (int i = 0; i < nsym; i++) nz += (w[i] > 0);
    int kmax = nz > 1 ? nz : 1;
    if (kmax > nsym - 1) kmax = nsym - 1;
    if (kmax > (1 << L) - 1) kmax = (1 << L) - 1;

    uint64_t best = UINT64_MAX;
    int bestk = 0;
    uint8_t bestlen[PM_MAXN];
    for (int k = 1; k <= kmax; k++) {
        uint64_t lw[PM_MAXN];
        int lid[PM_MAXN];
        uint8_t ll[PM_MAXN];
        uint64_t rest = 0;
        for (int i = 0; i < k; i++) {
            lw[i] = w[rank[i]];
            lid[i] = rank[i];
        }
        for (int i = k; i < nsym; i++) rest += w[rank[i]];
        lw[k] = rest;
        lid[k] = nsym; /* the escape symbol's id follows every real one */
        if (lcto_package_merge(k + 1, lw, lid, L, ll) != LCTO_OK) return UINT64_MAX;
        uint64_t cost = 0;
        for (int i = 0; i < k; i++) cost += lw[i] * ll[i];
        cost += rest * (uint64_t)(ll[k] + lit_bits);
        if (cost < best) {
            best = cost;
            bestk = k;
            memcpy(bestlen, ll, (size_t)(k + 1));
        }
    }
    memset(len, 0, (size_t)nsym);
    for (int i = 0; i < bestk; i++) len[rank[i]] = bestlen[i];
    *esc_len = bestlen[bestk];
    if (k_out) *k_out = bestk;
    return best;
}

uint64_t lcto_build_base(const uint64_t w[256], uint8_t len[256], uint8_t *esc_len, int *k_out)
{
    return lcto_build_escape(256, w, MAXLEN, 8, len, esc_len, k_out);
}

/* ------------------------------------------------------------------------ */
/* Shift ([EXP-split]: a small shift, sampled from up to 4096 elements,      */
/* follows the tensor's scale; [LCT-abs]: adaptation to magnitude shifts).   */
/* Read as an integer offset k of the exponent field: field e is coded with  */
/* the base code of field e - k.                                             */
/* ------------------------------------------------------------------------ */
static unsigned base_cost(const uint8_t len_base[256], uint8_t esc_len, int x)
{
    if (x >= 0 && x <= 255 && len_base[x] > 0) return len_base[x];
    return (unsigned)esc_len + 8u;
}

uint64_t lcto_shift_cost(const uint8_t len_base[256], uint8_t esc_len, const uint8_t *e, size_t m, int k)
{
    uint64_t bits = 0;
    for (size_t i = 0; i < m; i++) bits += base_cost(len_base, esc_len, (int)e[i] - k);
    return bits;
}

int lcto_best_shift(const uint8_t len_base[256], uint8_t esc_len, const uint8_t *e, size_t m)
{
    int bestk = 0;
    uint64_t best = UINT64_MAX;
    for (int k = -255; k <= 255; k++) {
        uint64_t c = lcto_shift_cost(len_base, esc_len, e, m, k);
        int better = c < best ||
                     (c == best && (abs(k) < abs(bestk) || (abs(k) == abs(bestk) && k < bestk)));
        if (better) {
            best = c;
            bestk = k;
        }
    }
    return bestk;
}

/* ------------------------------------------------------------------------ */
/* Canonical codes, as in DEFLATE (RFC 1951, section 3.2.2): code values     */
/* increase with (length, symbol id); the escape symbol has id 256.          */
/* ------------------------------------------------------------------------ */
void lcto_canonical(const uint8_t len[257], uint32_t code[257])
{
    unsigned bl_count[MAXLEN + 1] = {0}, next_code[MAXLEN + 2] = {0};
    for (int i = 0; i < 257; i++)
        if (len[i]) bl_count[len[i]]++;
    unsigned c = 0;
    for (int bits = 1; bits <= MAXLEN; bits++) {
        c = (c + bl_count[bits - 1]) << 1;
        next_code[bits] = c;
    }
    for (int i = 0; i < 257; i++) code[i] = len[i] ? next_code[len[i]]++ : 0;
}

void lcto_codebook_from_base(const uint8_t len_base[256], uint8_t esc_len, int shift, lcto_codebook *cb)
{
    uint8_t l[257];
    for (int e = 0; e < 256; e++) {
        int x = e - shift;
        l[e] = (x >= 0 && x <= 255) ? len_base[x] : 0;
        cb->len[e] = l[e];
    }
    l[256] = esc_len;
    memcpy(cb->len_base, len_base, 256);
    cb->esc_len = esc_len;
    cb->shift = shift;
    lcto_canonical(l, cb->code);
}

int lcto_codebook_build(int family, double scale, double shape,
                        const uint16_t *x, uint64_t n, lcto_codebook *cb)
{
    double p[256];
    uint64_t w[256];
    uint8_t len_base[256], esc_len;
    int k;
    int rc = lcto_model_pmf(family, scale, shape, p);
    if (rc != LCTO_OK) return rc;
    lcto_weights(p, w);
    if (lcto_build_base(w, len_base, &esc_len, &k) == UINT64_MAX) return LCTO_EINVAL;

    size_t m = n < 4096 ? (size_t)n : 4096;
    uint8_t *smp = (uint8_t *)malloc(m ? m : 1);
    if (!smp) return LCTO_EINVAL;
    for (size_t i = 0; i < m; i++) smp[i] = lcto_exponent(x[(uint64_t)i * n / m]);
    int shift = lcto_best_shift(len_base, esc_len, smp, m);
    free(smp);
    lcto_codebook_from_base(len_base, esc_len, shift, cb);
    return LCTO_OK;
}

/* ------------------------------------------------------------------------ */
/* Block format ([EXP-streams]).  Block element r goes to stream r mod 256,  */
/* position r div 256.  Each stream has 32*cap_words bits; bit k of a stream */
/* is bit (k mod 32) of its word k div 32, and word w of stream s sits at    */
/* pay[w*256 + s].  Codes go in MSB first; an escaped field follows its ESC  */
/* code as 8 bits, least significant first.  The longest prefix of a stream */
/* that fits is coded; the rest of its fields spill, raw, to the overflow.   */
/* ------------------------------------------------------------------------ */

static void put_bit(uint32_t *pay, int s, uint32_t pos, unsigned bit)
{
    if (bit) pay[(pos / 32u) * NSTREAM + (unsigned)s] |= 1u << (pos % 32u);
}

static unsigned get_bit(const uint32_t *pay, int s, uint32_t pos)
{
    return (pay[(pos / 32u) * NSTREAM + (unsigned)s] >> (pos % 32u)) & 1u;
}

static unsigned code_cost(const lcto_codebook *cb, uint8_t e)
{
    return cb->len[e] ? cb->len[e] : (unsigned)cb->esc_len + 8u;
}

static uint32_t stream_len(uint32_t nb, int s)
{
    return nb > (uint32_t)s ? (nb - (uint32_t)s + NSTREAM - 1) / NSTREAM : 0;
}

int lcto_encode_block(const lcto_codebook *cb, const uint16_t *x, uint32_t nb,
                      uint32_t cap_words, uint8_t *sf, uint32_t *pay, uint16_t *cnt,
                      uint8_t *spill, uint32_t *nspill)
{
    uint32_t cap_bits = 32u * cap_words;
    memset(pay, 0, sizeof(uint32_t) * cap_words * NSTREAM);
    for (uint32_t r = 0; r < nb; r++) sf[r] = lcto_signfrac(x[r]);
    uint32_t ns = 0;
    for (int s = 0; s < NSTREAM; s++) {
        uint32_t n_s = stream_len(nb, s), c_s = n_s, pos = 0;
        for (uint32_t j = 0; j < n_s; j++) {
            uint8_t e = lcto_exponent(x[j * NSTREAM + (uint32_t)s]);
            if (pos + code_cost(cb, e) > cap_bits) {
                c_s = j;
                break;
            }
            if (cb->len[e]) {
                for (int t = cb->len[e] - 1; t >= 0; t--) put_bit(pay, s, pos++, (cb->code[e] >> t) & 1u);
            } else {
                for (int t = cb->esc_len - 1; t >= 0; t--) put_bit(pay, s, pos++, (cb->code[256] >> t) & 1u);
                for (int t = 0; t < 8; t++) put_bit(pay, s, pos++, (e >> t) & 1u);
            }
        }
        cnt[s] = (uint16_t)c_s;
        for (uint32_t j = c_s; j < n_s; j++) spill[ns++] = lcto_exponent(x[j * NSTREAM + (uint32_t)s]);
    }
    *nspill = ns;
    return LCTO_OK;
}

/* Canonical decoding, one bit at a time: after reading l bits the value is a
 * code word if it lies in [first[l], first[l] + count[l]). */
typedef struct {
    unsigned count[MAXLEN + 1], first[MAXLEN + 1], offset[MAXLEN + 1];
    int sym[257];
} canon_dec;

static void canon_dec_init(const lcto_codebook *cb, canon_dec *d)
{
    uint8_t l[257];
    memcpy(l, cb->len, 256);
    l[256] = cb->esc_len;
    memset(d, 0, sizeof *d);
    for (int i = 0; i < 257; i++)
        if (l[i]) d->count[l[i]]++;
    unsigned c = 0, off = 0;
    for (int bits = 1; bits <= MAXLEN; bits++) {
        c = (c + d->count[bits - 1]) << 1;
        d->first[bits] = c;
        d->offset[bits] = off;
        off += d->count[bits];
    }
    unsigned fill[MAXLEN + 1] = {0};
    for (int i = 0; i < 257; i++)
        if (l[i]) d->sym[d->offset[l[i]] + fill[l[i]]++] = i;
}

int lcto_decode_block(const lcto_codebook *cb, const uint8_t *sf, const uint32_t *pay,
                      const uint16_t *cnt, const uint8_t *spill, uint32_t nb,
                      uint32_t cap_words, uint16_t *y)
{
    canon_dec d;
    canon_dec_init(cb, &d);
    uint32_t cap_bits = 32u * cap_words, ns = 0;
    for (int s = 0; s < NSTREAM; s++) {
        uint32_t n_s = stream_len(nb, s), c_s = cnt[s], pos = 0;
        if (c_s > n_s) return LCTO_EDECODE;
        for (uint32_t j = 0; j < c_s; j++) {
            unsigned v = 0;
            int sym = -1;
            for (int l = 1; l <= MAXLEN; l++) {
                if (pos >= cap_bits) return LCTO_EDECODE;
                v = (v << 1) | get_bit(pay, s, pos++);
                if (d.count[l] && v >= d.first[l] && v - d.first[l] < d.count[l]) {
                    sym = d.sym[d.offset[l] + v - d.first[l]];
                    break;
                }
            }
            if (sym < 0) return LCTO_EDECODE;
            uint8_t e;
            if (sym == 256) {
                unsigned lit = 0;
                for (int t = 0; t < 8; t++) {
                    if (pos >= cap_bits) return LCTO_EDECODE;
                    lit |= get_bit(pay, s, pos++) << t;
                }
                e = (uint8_t)lit;
            } else {
                e = (uint8_t)sym;
            }
            uint32_t r = j * NSTREAM + (uint32_t)s;
            y[r] = lcto_join(sf[r], e);
        }
        for (uint32_t j = c_s; j < n_s; j++) {
            uint32_t r = j * NSTREAM + (uint32_t)s;
            y[r] = lcto_join(sf[r], spill[ns++]);
        }
    }
    return LCTO_OK;
}

/* ------------------------------------------------------------------------ */
/* Whole tensors: blocks of block_elems, the last one possibly short; the    */
/* marker obase[b] is where block b's spilled bytes start in the overflow    */
/* region, obase[nblk] the total.                                            */
/* ------------------------------------------------------------------------ */
static int layout_ok(uint32_t block_elems, uint32_t cap_words)
{
    return block_elems >= NSTREAM && block_elems % NSTREAM == 0 &&
           block_elems / NSTREAM <= 65535u && cap_words >= 1;
}

int lcto_encode(const lcto_codebook *cb, const uint16_t *x, uint64_t n,
                uint32_t block_elems, uint32_t cap_words,
                uint8_t *sf, uint32_t *pay, uint16_t *cnt, uint64_t *obase,
                uint8_t *ovf, uint64_t ovf_cap)
{
    if (!layout_ok(block_elems, cap_words)) return LCTO_EINVAL;
    uint64_t nblk = (n + block_elems - 1) / block_elems;
    uint8_t *spill = (uint8_t *)malloc(block_elems);
    if (!spill) return LCTO_EINVAL;
    obase[0] = 0;
    for (uint64_t b = 0; b < nblk; b++) {
        uint64_t r0 = b * block_elems;
        uint32_t nb = (uint32_t)((n - r0) < block_elems ? (n - r0) : block_elems);
        uint32_t ns = 0;
        lcto_encode_block(cb, x + r0, nb, cap_words, sf + r0,
                          pay + b * (uint64_t)cap_words * NSTREAM, cnt + b * NSTREAM, spill, &ns);
        for (uint32_t i = 0; i < ns; i++)
            if (obase[b] + i < ovf_cap) ovf[obase[b] + i] = spill[i];
        obase[b + 1] = obase[b] + ns;
    }
    free(spill);
    return obase[nblk] > ovf_cap ? LCTO_OVF_FULL : LCTO_OK;
}

int lcto_decode(const lcto_codebook *cb, const uint8_t *sf, const uint32_t *pay,
                const uint16_t *cnt, const uint64_t *obase, const uint8_t *ovf,
                uint64_t n, uint32_t block_elems, uint32_t cap_words, uint16_t *y)
{
    if (!layout_ok(block_elems, cap_words)) return LCTO_EINVAL;
    uint64_t nblk = (n + block_elems - 1) / block_elems;
    for (uint64_t b = 0; b < nblk; b++) {
        uint64_t r0 = b * block_elems;
        uint32_t nb = (uint32_t)((n - r0) < block_elems ? (n - r0) : block_elems);
        int rc = lcto_decode_block(cb, sf + r0, pay + b * (uint64_t)cap_words * NSTREAM,
                                   cnt + b * NSTREAM, ovf + obase[b], nb, cap_words, y + r0);
        if (rc != LCTO_OK) return rc;
    }
    return LCTO_OK;
}

/* ------------------------------------------------------------------------ */
/* Shift re-estimation ([LCT-abs]: adaptation to magnitude shifts;           */
/* [EXP-split]: the shift is sampled from up to 4096 elements; [EXP-limits]: */
/* a distribution that no longer fits the tensor raises storage).  The       */
/* tensor is decoded in full, the sample is taken at the build's positions,  */
/* and only the shift changes: the base code is kept as it is.               */
/* ------------------------------------------------------------------------ */
int lcto_reshift(const lcto_codebook *cb, const uint8_t *sf, const uint32_t *pay,
                 const uint16_t *cnt, const uint64_t *obase, const uint8_t *ovf,
                 uint64_t n, uint32_t block_elems, uint32_t cap_words, lcto_codebook *out)
{
    if (!layout_ok(block_elems, cap_words)) return LCTO_EINVAL;
    uint16_t *y = (uint16_t *)malloc(sizeof(uint16_t) * (n ? n : 1));
    size_t m = n < 4096 ? (size_t)n : 4096;
    uint8_t *smp = (uint8_t *)malloc(m ? m : 1);
    int rc = (y && smp) ? LCTO_OK : LCTO_EINVAL;
    if (rc == LCTO_OK) rc = lcto_decode(cb, sf, pay, cnt, obase, ovf, n, block_elems, cap_words, y);
    if (rc == LCTO_OK) {
        for (size_t i = 0; i < m; i++) smp[i] = lcto_exponent(y[(uint64_t)i * n / m]);
        int shift = lcto_best_shift(cb->len_base, cb->esc_len, smp, m);
        lcto_codebook_from_base(cb->len_base, cb->esc_len, shift, out);
    }
    free(y);
    free(smp);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* SGD update ([EXP-train]): W_{t+1} = W_t - eta * M_t, read as one fp32     */
/* fused multiply-add fmaf(-eta, m, w), rounded to nearest-even BF16.  A NaN */
/* result is written as the canonical quiet NaN 0x7FC0.                      */
/* ------------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t v)
{
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float lcto_fmaf(float a, float b, float c) { return fmaf(a, b, c); }

uint16_t lcto_rne_bf16(float r)
{
    uint32_t u;
    memcpy(&u, &r, 4);
    if (isnan(r)) return 0x7FC0u;
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

uint16_t lcto_sgd_elem(uint16_t w, uint16_t m, float eta)
{
    return lcto_rne_bf16(fmaf(-eta, bf16_to_f32(m), bf16_to_f32(w)));
}

int lcto_sgd(const lcto_codebook *cw, const uint8_t *w_sf, const uint32_t *w_pay,
             const uint16_t *w_cnt, const uint64_t *w_obase, const uint8_t *w_ovf,
             const lcto_codebook *cm, const uint8_t *m_sf, const uint32_t *m_pay,
             const uint16_t *m_cnt, const uint64_t *m_obase, const uint8_t *m_ovf,
             float eta, const lcto_codebook *cw_out, uint64_t n, uint32_t block_elems,
             uint32_t cap_words, uint8_t *o_sf, uint32_t *o_pay, uint16_t *o_cnt, uint64_t *o_obase,
             uint8_t *o_ovf, uint64_t ovf_cap)
{
    if (!layout_ok(block_elems, cap_words)) return LCTO_EINVAL;
    if (!cw_out) cw_out = cw;
    uint64_t nblk = (n + block_elems - 1) / block_elems;
    uint16_t *wd = (uint16_t *)malloc(sizeof(uint16_t) * block_elems);
    uint16_t *md = (uint16_t *)malloc(sizeof(uint16_t) * block_elems);
    uint8_t *spill = (uint8_t *)malloc(block_elems);
    int rc = LCTO_OK;
    if (!wd || !md || !spill) rc = LCTO_EINVAL;
    if (rc == LCTO_OK) o_obase[0] = 0;
    for (uint64_t b = 0; b < nblk && rc == LCTO_OK; b++) {
        uint64_t r0 = b * block_elems, po = b * (uint64_t)cap_words * NSTREAM;
        uint32_t nb = (uint32_t)((n - r0) < block_elems ? (n - r0) : block_elems);
        rc = lcto_decode_block(cw, w_sf + r0, w_pay + po, w_cnt + b * NSTREAM, w_ovf + w_obase[b],
                               nb, cap_words, wd);
        if (rc != LCTO_OK) break;
        rc = lcto_decode_block(cm, m_sf + r0, m_pay + po, m_cnt + b * NSTREAM, m_ovf + m_obase[b],
                               nb, cap_words, md);
        if (rc != LCTO_OK) break;
        for (uint32_t r = 0; r < nb; r++) wd[r] = lcto_sgd_elem(wd[r], md[r], eta);
        uint32_t ns = 0;
        lcto_encode_block(cw_out, wd, nb, cap_words, o_sf + r0, o_pay + po, o_cnt + b * NSTREAM, spill, &ns);
        for (uint32_t i = 0; i < ns; i++)
            if (o_obase[b] + i < ovf_cap) o_ovf[o_obase[b] + i] = spill[i];
        o_obase[b + 1] = o_obase[b] + ns;
    }
    free(wd);
    free(md);
    free(spill);
    if (rc != LCTO_OK) return rc;
    return o_obase[nblk] > ovf_cap ? LCTO_OVF_FULL : LCTO_OK;
}

/* ------------------------------------------------------------------------ */
/* Momentum step ([EXP-jargon], [EXP-train]).  The pages name the momentum   */
/* buffer of SGD with momentum as optimizer state stored compressed, but no  */
/* update rule; this is the plain heavy-ball form M' = mu*M + g, then        */
/* W' = W - eta*M', each a single fused multiply-add rounded to fp32, then   */
/* to BF16 (a NaN written as 0x7FC0); the W update uses M' as stored.        */
/* ------------------------------------------------------------------------ */
void lcto_momentum_elem(uint16_t w, uint16_t m, uint16_t g, float mu, float eta,
                        uint16_t *w_out, uint16_t *m_out)
{
    uint16_t m2 = lcto_rne_bf16(fmaf(mu, bf16_to_f32(m), bf16_to_f32(g)));
    *m_out = m2;
    *w_out = lcto_rne_bf16(fmaf(-eta, bf16_to_f32(m2), bf16_to_f32(w)));
}

/* Encode one block's values and append its spilled bytes to ovf at obase[b]. */
static void encode_block_out(const lcto_codebook *cb, const uint16_t *x, uint32_t nb, uint32_t cap_words,
                             uint64_t b, uint64_t r0, uint64_t po, uint8_t *spill,
                             uint8_t *sf, uint32_t *pay, uint16_t *cnt, uint64_t *obase,
                             uint8_t *ovf, uint64_t ovf_cap)
{
    uint32_t ns = 0;
    lcto_encode_block(cb, x, nb, cap_words, sf + r0, pay + po, cnt + b * NSTREAM, spill, &ns);
    for (uint32_t i = 0; i < ns; i++)
        if (obase[b] + i < ovf_cap) ovf[obase[b] + i] = spill[i];
    obase[b + 1] = obase[b] + ns;
}

int lcto_momentum(const lcto_codebook *cw, const uint8_t *w_sf, const uint32_t *w_pay,
                  const uint16_t *w_cnt, const uint64_t *w_obase, const uint8_t *w_ovf,
                  const lcto_codebook *cm, const uint8_t *m_sf, const uint32_t *m_pay,
                  const uint16_t *m_cnt, const uint64_t *m_obase, const uint8_t *m_ovf,
                  const uint16_t *g, float mu, float eta,
                  const lcto_codebook *cw_out, const lcto_codebook *cm_out,
                  uint64_t n, uint32_t block_elems, uint32_t cap_words,
                  uint8_t *ow_sf, uint32_t *ow_pay, uint16_t *ow_cnt, uint64_t *ow_obase,
                  uint8_t *ow_ovf, uint64_t ow_ovf_cap,
                  uint8_t *om_sf, uint32_t *om_pay, uint16_t *om_cnt, uint64_t *om_obase,
                  uint8_t *om_ovf, uint64_t om_ovf_cap)
{
    if (!layout_ok(block_elems, cap_words)) return LCTO_EINVAL;
    if (!cw_out) cw_out = cw;
    if (!cm_out) cm_out = cm;
    uint64_t nblk = (n + block_elems - 1) / block_elems;
    uint16_t *wd = (uint16_t *)malloc(sizeof(uint16_t) * block_elems);
    uint16_t *md = (uint16_t *)malloc(sizeof(uint16_t) * block_elems);
    uint8_t *spill = (uint8_t *)malloc(block_elems);
    int rc = LCTO_OK;
    if (!wd || !md || !spill) rc = LCTO_EINVAL;
    if (rc == LCTO_OK) {
        ow_obase[0] = 0;
        om_obase[0] = 0;
    }
    for (uint64_t b = 0; b < nblk && rc == LCTO_OK; b++) {
        uint64_t r0 = b * block_elems, po = b * (uint64_t)cap_words * NSTREAM;
        uint32_t nb = (uint32_t)((n - r0) < block_elems ? (n - r0) : block_elems);
        rc = lcto_decode_block(cw, w_sf + r0, w_pay + po, w_cnt + b * NSTREAM, w_ovf + w_obase[b],
                               nb, cap_words, wd);
        if (rc != LCTO_OK) break;
        rc = lcto_decode_block(cm, m_sf + r0, m_pay + po, m_cnt + b * NSTREAM, m_ovf + m_obase[b],
                               nb, cap_words, md);
        if (rc != LCTO_OK) break;
        for (uint32_t r = 0; r < nb; r++) lcto_momentum_elem(wd[r], md[r], g[r0 + r], mu, eta, &wd[r], &md[r]);
        encode_block_out(cw_out, wd, nb, cap_words, b, r0, po, spill, ow_sf, ow_pay, ow_cnt, ow_obase, ow_ovf,
                         ow_ovf_cap);
        encode_block_out(cm_out, md, nb, cap_words, b, r0, po, spill, om_sf, om_pay, om_cnt, om_obase, om_ovf,
                         om_ovf_cap);
    }
    free(wd);
    free(md);
    free(spill);
    if (rc != LCTO_OK) return rc;
    return (ow_obase[nblk] > ow_ovf_cap || om_obase[nblk] > om_ovf_cap) ? LCTO_OVF_FULL : LCTO_OK;
}
