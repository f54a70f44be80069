// codebook.cpp -- host construction of the exponent codebook.
//
// Explainer "LCT paper - Lossless Huffman coding of BF16 training tensors",
// paragraph on bits: exponents are Huffman-coded with codes of at most 8 bits;
// rare exponents share one escape code followed by the 8-bit field; the
// code is fixed ahead of training from a Gaussian, Laplace or power-law model
// chosen by the user, with an exponent offset estimated on at most 4096
// sampled values.  The LCT
// abstract names the adaptation to magnitude shifts.
//
// Readings taken where the passage is silent:
//   - weights are floor(p * 2^40 + 0.5) of the model probability of each
//     8-bit exponent field (field e in 1..254 covers |x| in [2^(e-127),
//     2^(e-126)), field 0 zero and subnormals, field 255 nothing);
//   - "rare" = every field but the k heaviest, k chosen for the least
//     expected bits (an escaped field costs esc_len + 8);
//   - the 8-bit cap is met by an optimal length-limited code (package-merge),
//     leaves ordered by (weight, id), a leaf before a package of equal weight;
//   - the shift is the integer exponent offset k that minimises the coded
//     bits of the sample under the base code (ties: smallest |k|, then the
//     smaller k);
//   - canonical code values follow DEFLATE's convention (RFC 1951, 3.2.2);
//   - re-estimating the shift during training keeps the base code and runs
//     the same shift search over a sample of the tensor's current values
//     (explainer, paragraph on the limits: a model that no longer fits the
//     tensor raises storage).
#include <math.h>
#include <string.h>

// The model weights must not depend on contraction of a*b+c into fma.
#pragma clang fp contract(off)

#include <algorithm>
#include <vector>

#include "lct_internal.h"

namespace lct {
namespace {

constexpr int kCap = 8;          // longest code
constexpr int kLit = 8;          // literal bits after the escape code
constexpr int kEsc = 256;        // escape symbol id

// ---------------------------------------------------------------- model
//
// The probability of each exponent field's range of |x| under the model.
// Gaussian and Laplace use their survival functions, P(|X| > t) = erfc(t /
// (sigma sqrt 2)) and exp(-t / b).  Student-t integrates its density over
// the range by Gauss-Legendre quadrature (no survival function, so no
// difference of two nearly equal tails near zero): the range is cut into
// pieces over each of which the log-density drops by at most one, so the
// integrand is smooth on the scale of a piece and the rule is exact to
// rounding; pieces whose mass is certainly below 2^-70 count as zero (their
// weights are zero either way).

// Gauss-Legendre rule with kGl nodes on [-1, 1]: the nodes are the roots of
// the Legendre polynomial P_n, found by Newton's method from the estimates
// cos(pi (i + 3/4) / (n + 1/2)), P_n and P_n' from the three-term recurrence;
// the weights are 2 / ((1 - x^2) P_n'(x)^2).
constexpr int kGl = 24;
struct GaussLegendre {
    double x[kGl], w[kGl];
    GaussLegendre() {
        const double pi = 3.14159265358979323846;
        for (int i = 0; i < kGl; ++i) {
            double z = cos(pi * (i + 0.75) / (kGl + 0.5)), dp = 0.0;
            for (int it = 0; it < 100; ++it) {
                double p0 = 1.0, p1 = z;          // P_{k-1}(z), P_k(z)
                for (int k = 2; k <= kGl; ++k) {
                    const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
                    p0 = p1;
                    p1 = p2;
                }
                dp = kGl * (z * p1 - p0) / (z * z - 1.0);
                const double dz = p1 / dp;
                z -= dz;
                if (fabs(dz) <= 1e-16) break;
            }
            double p0 = 1.0, p1 = z;
            for (int k = 2; k <= kGl; ++k) {
                const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
                p0 = p1;
                p1 = p2;
            }
            dp = kGl * (z * p1 - p0) / (z * z - 1.0);
            x[i] = z;
            w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
        }
    }
};
const GaussLegendre &gauss_legendre() {
    static const GaussLegendre rule;
    return rule;
}

// log Gamma(x + 1/2) - log Gamma(x).  For x >= 15 from Stirling's series
// log Gamma(z) = (z - 1/2) log z - z + log(2 pi)/2 + sum B_2k / (2k (2k-1)
// z^(2k-1)), taken as one difference (five terms: error below 1e-16
// relative), since the two lgamma values, each about x log x, would cancel
// to about 1e-16 x log x of absolute error.
double lgamma_half_step(double x) {
    if (x < 15.0) return lgamma(x + 0.5) - lgamma(x);
    auto series = [](double z) {
        const double r = 1.0 / z, r2 = r * r;
        return r * (1.0 / 12 - r2 * (1.0 / 360 - r2 * (1.0 / 1260 - r2 * (1.0 / 1680 - r2 / 1188))));
    };
    return x * log1p(0.5 / x) + 0.5 * log(x) - 0.5 + (series(x + 0.5) - series(x));
}

// Student-t with nu degrees of freedom, unit scale: the density at u is
// exp(lc - g(u)) with g(u) = (nu + 1)/2 log(1 + u^2/nu).
struct StudentT {
    double nu, lc;
    explicit StudentT(double nu_)
        : nu(nu_), lc(lgamma_half_step(0.5 * nu_) - 0.5 * log(nu_ * 3.14159265358979323846)) {}
    double g(double u) const { return 0.5 * (nu + 1.0) * log1p(u * u / nu); }
    double density(double u) const { return exp(lc - g(u)); }
    // g' is largest at u = sqrt(nu)
    double max_slope(double a, double b) const {
        const double u = std::min(std::max(sqrt(nu), a), b);
        return (nu + 1.0) * u / (nu + u * u);
    }
    // P(a <= |T| < b), 0 <= a < b
    double mass(double a, double b) const {
        if (!(b > a)) return 0.0;
        if (2.0 * density(a) * (b - a) < 0x1p-70) return 0.0;
        const double drop = max_slope(a, b) * (b - a);
        const int pieces = (int)std::min(65536.0, std::max(1.0, ceil(drop)));
        const GaussLegendre &r = gauss_legendre();
        const double h = (b - a) / pieces;
        double sum = 0.0;
        for (int j = 0; j < pieces; ++j) {
            const double x0 = a + j * h, half = 0.5 * h, mid = x0 + half;
            if (2.0 * density(x0) * h < 0x1p-70) break;      // the density decreases from here
            double q = 0.0;
            for (int i = 0; i < kGl; ++i) q += r.w[i] * density(mid + half * r.x[i]);
            sum += q * half;
        }
        return 2.0 * sum;
    }
    // P(|T| < b): octaves down to where the density is flat, then the rest
    double below(double b) const {
        const double flat = std::min(sqrt(nu), 1.0) / 8.0;
        double sum = 0.0, hi = b;
        while (hi > flat) {
            sum += mass(0.5 * hi, hi);
            hi *= 0.5;
        }
        return sum + mass(0.0, hi);
    }
};

bool model_ok(const lct_model &m) {
    if (m.family < LCT_GAUSSIAN || m.family > LCT_POWERLAW) return false;
    if (!(m.scale > 0.0) || !std::isfinite(m.scale)) return false;
    if (m.family == LCT_POWERLAW && (!(m.shape > 0.0) || !std::isfinite(m.shape))) return false;
    return true;
}

}  // namespace

// Field e in 1..254 covers |x| in [2^(e-127), 2^(e-126)); field 0 zero and
// the subnormals (|x| < 2^-126); field 255 has no mass.
void model_pmf(const lct_model &m, double p[256]) {
    const double r2 = sqrt(2.0);
    auto edge = [&](int e) { return ldexp(1.0, e - 127) / m.scale; };   // in units of the scale
    switch (m.family) {
    case LCT_GAUSSIAN:
        p[0] = erf(edge(1) / r2);
        for (int e = 1; e <= 254; ++e) p[e] = erfc(edge(e) / r2) - erfc(edge(e + 1) / r2);
        break;
    case LCT_LAPLACE:
        p[0] = -expm1(-edge(1));
        for (int e = 1; e <= 254; ++e) p[e] = exp(-edge(e)) - exp(-edge(e + 1));
        break;
    default: {
        const StudentT t(m.shape);
        p[0] = t.below(edge(1));
        for (int e = 1; e <= 254; ++e) p[e] = t.mass(edge(e), edge(e + 1));
    }
    }
    for (int e = 0; e <= 254; ++e)
        if (!(p[e] > 0.0)) p[e] = 0.0;
    p[255] = 0.0;
}

namespace {

void model_weights(const lct_model &m, uint64_t w[256]) {
    double p[256];
    model_pmf(m, p);
    for (int e = 0; e < 256; ++e) w[e] = (uint64_t)floor(p[e] * 1099511627776.0 + 0.5);
}

// ---------------------------------------------------------------- package-merge
//
// Coin-collector form: level kCap holds the leaves in (weight, id) order;
// every shallower level is the leaves merged with the pairs of consecutive
// items of the level below.  Only each level's item kinds are kept: of the
// first 2n-2 items of level 1, the leaves are the lightest leaves and the
// packages expand to the first items of the next level, so a leaf's length
// is the number of levels whose selected prefix reaches it.

struct Leaf {
    uint64_t w;
    int id;
};

void limited_lengths(std::vector<Leaf> &leaves, std::vector<int> &len_out) {
    const int n = (int)leaves.size();
    std::sort(leaves.begin(), leaves.end(), [](const Leaf &a, const Leaf &b) {
        return a.w != b.w ? a.w < b.w : a.id < b.id;
    });
    // kind[d][i]: true = package; levels 1..kCap (index 0 unused)
    std::vector<std::vector<uint8_t>> kind(kCap + 1);
    std::vector<uint64_t> cur(n), nxt;
    for (int i = 0; i < n; ++i) cur[i] = leaves[i].w;
    kind[kCap].assign(n, 0);
    for (int d = kCap - 1; d >= 1; --d) {
        const int npk = (int)cur.size() / 2;
        nxt.clear();
        kind[d].clear();
        int li = 0, pi = 0;
        while (li < n || pi < npk) {
            const bool take_leaf =
                li < n && (pi >= npk || leaves[li].w <= cur[2 * pi] + cur[2 * pi + 1]);
            if (take_leaf) {
                nxt.push_back(leaves[li++].w);
                kind[d].push_back(0);
            } else {
                nxt.push_back(cur[2 * pi] + cur[2 * pi + 1]);
                kind[d].push_back(1);
                ++pi;
            }
        }
        cur.swap(nxt);
    }
    std::vector<int> len_sorted(n, 0);
    int take = 2 * n - 2;
    for (int d = 1; d <= kCap && take > 0; ++d) {
        int nleaf = 0, npack = 0;
        for (int i = 0; i < take; ++i) (kind[d][i] ? npack : nleaf)++;
        for (int i = 0; i < nleaf; ++i) ++len_sorted[i];
        take = 2 * npack;
    }
    len_out.assign(n, 0);
    for (int i = 0; i < n; ++i) len_out[i] = len_sorted[i];
}

// Base code: lengths len[256] (0 = escaped) and esc_len for the weights.
bool base_code(const uint64_t w[256], uint8_t len[256], uint8_t *esc_len) {
    int order[256];
    for (int i = 0; i < 256; ++i) order[i] = i;
    std::sort(order, order + 256, [&](int a, int b) { return w[a] != w[b] ? w[a] > w[b] : a < b; });
    int nonzero = 0;
    for (int i = 0; i < 256; ++i) nonzero += w[i] != 0;
    const int kmax = std::min(255, std::max(1, nonzero));

    // suffix sums of the ranked weights: weight escaped when keeping k
    uint64_t rest[257];
    rest[256] = 0;
    for (int r = 255; r >= 0; --r) rest[r] = rest[r + 1] + w[order[r]];

    uint64_t best = ~uint64_t(0);
    int best_k = 0;
    std::vector<int> best_len;
    std::vector<Leaf> leaves;
    std::vector<int> ln;
    for (int k = 1; k <= kmax; ++k) {
        leaves.clear();
        for (int r = 0; r < k; ++r) leaves.push_back({w[order[r]], order[r]});
        leaves.push_back({rest[k], kEsc});
        limited_lengths(leaves, ln);   // leaves are now sorted; ln follows that order
        uint64_t cost = 0;
        for (size_t i = 0; i < leaves.size(); ++i) {
            if (leaves[i].id == kEsc) {
                cost += leaves[i].w * (uint64_t)(ln[i] + kLit);
            } else {
                cost += leaves[i].w * (uint64_t)ln[i];
            }
        }
        if (cost < best) {
            best = cost;
            best_k = k;
            best_len.assign(257, 0);
            for (size_t i = 0; i < leaves.size(); ++i) best_len[leaves[i].id] = ln[i];
        }
    }
    if (best_k == 0) return false;
    for (int e = 0; e < 256; ++e) len[e] = (uint8_t)best_len[e];
    *esc_len = (uint8_t)best_len[kEsc];
    return true;
}

// Shift k minimising the sample's coded bits; the histogram of the sample's
// exponent fields is all that matters.
int best_shift(const uint8_t base[256], uint8_t esc_len, const uint16_t *sample, uint32_t m) {
    uint64_t hist[256] = {0};
    for (uint32_t i = 0; i < m; ++i) ++hist[(sample[i] >> 7) & 0xFF];
    auto bits_for = [&](int k) {
        uint64_t total = 0;
        for (int e = 0; e < 256; ++e) {
            if (!hist[e]) continue;
            const int x = e - k;
            const unsigned c = (x >= 0 && x < 256 && base[x]) ? base[x] : esc_len + kLit;
            total += hist[e] * c;
        }
        return total;
    };
    int best_k = 0;
    uint64_t best = bits_for(0);
    // visiting 0, -1, +1, -2, +2, ... and keeping strict improvements gives
    // the smallest |k|, then the smaller k, among equal costs
    for (int a = 1; a <= 255; ++a) {
        for (int k : {-a, a}) {
            const uint64_t c = bits_for(k);
            if (c < best) {
                best = c;
                best_k = k;
            }
        }
    }
    return best_k;
}

uint32_t reverse_bits(uint32_t v, int n) {
    uint32_t r = 0;
    for (int i = 0; i < n; ++i) r |= ((v >> i) & 1u) << (n - 1 - i);
    return r;
}

// Canonical codes, lookup tables and summary fields from cb->len / esc_len.
void finish(lct_codebook *cb) {
    // symbols with a code in (length, id) order; code values count up and
    // shift left whenever the length grows
    std::vector<std::pair<int, int>> syms;   // (length, id)
    for (int e = 0; e < 256; ++e)
        if (cb->len[e]) syms.push_back({cb->len[e], e});
    syms.push_back({cb->esc_len, kEsc});
    std::sort(syms.begin(), syms.end());
    memset(cb->code, 0, sizeof cb->code);
    uint32_t c = 0;
    for (size_t i = 0; i < syms.size(); ++i) {
        if (i > 0) c = (c + 1) << (syms[i].first - syms[i - 1].first);
        cb->code[syms[i].second] = c;
    }
    uint32_t kept = 0, maxl = cb->esc_len;
    for (int e = 0; e < 256; ++e) {
        if (cb->len[e]) {
            ++kept;
            maxl = std::max<uint32_t>(maxl, cb->len[e]);
            cb->enc_bits[e] = reverse_bits(cb->code[e], cb->len[e]);
            cb->enc_len[e] = cb->len[e];
        } else {
            cb->enc_bits[e] = reverse_bits(cb->code[kEsc], cb->esc_len) | ((uint32_t)e << cb->esc_len);
            cb->enc_len[e] = (uint8_t)(cb->esc_len + kLit);
        }
    }
    cb->kept = kept;
    cb->max_len = (uint8_t)maxl;
    // peek table: every 8-bit window whose low L bits are a code's stream bits
    for (int p = 0; p < 256; ++p) cb->dec[p] = (uint16_t)((kCap << 8) | (1u << 14));
    for (const auto &s : syms) {
        const int L = s.first;
        const uint32_t r = reverse_bits(cb->code[s.second], L);
        const uint16_t ent = s.second == kEsc
                                 ? (uint16_t)(((L + kLit) << 8) | (1u << 13))
                                 : (uint16_t)(s.second | (L << 8));
        for (uint32_t h = 0; h < (1u << (kCap - L)); ++h) cb->dec[r | (h << L)] = ent;
    }
}

}  // namespace

lct_status build_codebook(const lct_model &model, const uint16_t *sample, uint32_t m,
                          lct_codebook *out) {
    if (!model_ok(model)) return LCT_EINVAL;
    uint64_t w[256];
    model_weights(model, w);
    uint8_t base[256], esc_len = 0;
    if (!base_code(w, base, &esc_len)) return LCT_EINVAL;
    const int k = best_shift(base, esc_len, sample, m);
    lct_status st = codebook_from_lengths(base, esc_len, k, out);
    out->model = model;
    return st;
}

lct_status codebook_from_lengths(const uint8_t len_base[256], uint8_t esc_len, int32_t shift,
                                 lct_codebook *out) {
    if (!len_base || !out || esc_len < 1 || esc_len > kCap || shift < -255 || shift > 255)
        return LCT_EINVAL;
    uint32_t kraft = 1u << (kCap - esc_len);
    for (int e = 0; e < 256; ++e) {
        if (len_base[e] > kCap) return LCT_EINVAL;
        if (len_base[e]) kraft += 1u << (kCap - len_base[e]);
    }
    if (kraft > (1u << kCap)) return LCT_EINVAL;
    memset(out, 0, sizeof *out);
    for (int e = 0; e < 256; ++e) {
        const int x = e - shift;
        out->len[e] = (x >= 0 && x < 256) ? len_base[x] : 0;
    }
    memcpy(out->len_base, len_base, sizeof out->len_base);
    out->esc_len = esc_len;
    out->shift = (int16_t)shift;
    finish(out);
    return LCT_OK;
}

lct_status reshift_codebook(const lct_codebook &cb, const uint16_t *sample, uint32_t m,
                            lct_codebook *out) {
    const lct_codebook in = cb;   // out may be &cb
    const int k = best_shift(in.len_base, in.esc_len, sample, m);
    lct_status st = codebook_from_lengths(in.len_base, in.esc_len, k, out);
    if (st == LCT_OK) out->model = in.model;
    return st;
}

bool tables_ok(const lct_codebook &cb) {
    if (cb.esc_len < 1 || cb.esc_len > kCap) return false;
    for (int e = 0; e < 256; ++e) {
        const uint32_t L = cb.enc_len[e];
        if (L < 1 || L > kCap + kLit || (cb.enc_bits[e] >> L) != 0) return false;
        if (((cb.dec[e] >> 8) & 0x1F) > kCap + kLit) return false;
    }
    return true;
}

void fill_enc(const lct_codebook &cb, EncTab *t) {
    memcpy(t->bits, cb.enc_bits, sizeof t->bits);
    memcpy(t->len, cb.enc_len, sizeof t->len);
}

void fill_enc_packed(const lct_codebook &cb, uint32_t t[256]) {
    for (int e = 0; e < 256; ++e) t[e] = cb.enc_bits[e] | ((uint32_t)cb.enc_len[e] << 24);
}

void fill_dec(const lct_codebook &cb, DecTab *t) {
    memcpy(t->dec, cb.dec, sizeof t->dec);
    t->esc_len = cb.esc_len;
}

}  // namespace lct
