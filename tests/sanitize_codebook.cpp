// sanitize_codebook.cpp -- the library's host codebook builder, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py
// together with the oracle, and checked against it: for a grid of models
// (Gaussian, Laplace, Student-t at several scales) and seeded samples of
// several sizes, the final lengths, escape length, shift and canonical codes
// of lct::build_codebook equal lcto_codebook_build's; the model pmfs agree
// bin by bin; codebooks from given
// base lengths equal lcto_codebook_from_base's; shift re-estimation and the
// table fills run over every codebook.  Test infrastructure: the sanitizers
// report any out-of-bounds access or undefined operation on the way.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../lossless_bf16_tensor_split_amd/csrc/lct_internal.h"
extern "C" {
#include "../oracle/lct_oracle.h"
}

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {   // xorshift64*
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return g_state * 0x2545F4914F6CDD1Dull;
}
double uniform01() { return ((next_u64() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
double normal() { return sqrt(-2.0 * log(uniform01())) * cos(6.283185307179586 * uniform01()); }

// fp32 bits -> BF16 bits, round to nearest even (an input generator only)
uint16_t bf16_of(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace

// The library's model pmf (Student-t: quadrature of the density over each
// field's range) against the oracle's (differences of the survival
// function), bin by bin: within 1e-12 relative or 1e-15 absolute, and the
// integer weights equal except by one where the oracle's p * 2^40 lies
// within 2e-3 of a rounding boundary.  Returns the bins that differ.
int check_pmfs(int *checked) {
    const double scales[] = {3.7e-12, 1e-3, 0.02, 1.0, 7.5, 1e30};
    // past nu of about 100 the oracle's normalising constant (a difference of
    // two lgamma values) loses 1e-12; the library's is printed for larger nu
    // (below) and checked against 50-digit values by the calling test
    const double shapes[] = {0.5, 1.0, 2.0, 3.0, 5.5, 30.0};
    int bad = 0;
    for (int fam = 0; fam < 3; ++fam) {
        for (double scale : scales) {
            for (double shape : shapes) {
                if (fam != 2 && shape != 1.0) continue;
                const lct_model model{fam, scale, fam == 2 ? shape : 0.0};
                double pl[256], po[256];
                lct::model_pmf(model, pl);
                if (lcto_model_pmf(fam, scale, model.shape, po) != 0) {
                    ++bad;
                    continue;
                }
                double sum = 0.0;
                for (int e = 0; e < 256; ++e) {
                    sum += pl[e];
                    const double d = fabs(pl[e] - po[e]);
                    bool ok = d <= 1e-15 || d <= 1e-12 * fabs(po[e]);
                    const double xl = pl[e] * 1099511627776.0, xo = po[e] * 1099511627776.0;
                    const double wl = floor(xl + 0.5), wo = floor(xo + 0.5);
                    if (wl != wo) ok = ok && fabs(wl - wo) == 1.0 && fabs(xo - floor(xo) - 0.5) < 2e-3;
                    if (!ok) {
                        ++bad;
                        printf("pmf: family %d scale %g shape %g field %d: library %.17g oracle %.17g\n", fam,
                               scale, model.shape, e, pl[e], po[e]);
                    }
                }
                if (fabs(sum - 1.0) > 1e-12 && scale > 1e-30 && scale < 1e30) {
                    ++bad;
                    printf("pmf: family %d scale %g shape %g sums to %.17g\n", fam, scale, model.shape, sum);
                }
                ++*checked;
            }
        }
    }
    // the library's Student-t pmf at large nu, every bin above 1e-9
    const double big[][2] = {{1000.0, 0.02}, {1e4, 7.5}, {1e6, 1.0}};
    for (const auto &ns : big) {
        const lct_model model{2, ns[1], ns[0]};
        double pl[256];
        lct::model_pmf(model, pl);
        for (int e = 0; e < 256; ++e)
            if (pl[e] > 1e-9) printf("libpmf %.17g %.17g %d %.17g\n", ns[0], ns[1], e, pl[e]);
    }
    return bad;
}

int main() {
    int pmfs = 0;
    const int pmf_bad = check_pmfs(&pmfs);
    printf("pmfs checked: %d, differing bins: %d\n", pmfs, pmf_bad);
    const double scales[] = {1e-3, 0.02, 1.0, 7.5};
    const double shapes[] = {1.0, 2.0, 3.0, 5.5};
    const uint32_t sizes[] = {0, 1, 100, 4096};
    int checked = 0, bad = 0;
    static uint16_t sample[4096];
    for (int fam = 0; fam < 3; ++fam) {
        for (double scale : scales) {
            for (double shape : shapes) {
                if (fam != 2 && shape != 1.0) continue;
                for (uint32_t m : sizes) {
                    const double spread = scale * (0.25 + 4.0 * uniform01());
                    for (uint32_t i = 0; i < m; ++i) {
                        double v = spread * normal();
                        if (i % 97 == 3) v *= 1e6;          // a few far out: escapes
                        if (i % 211 == 5) v = 0.0;
                        sample[i] = bf16_of(v);
                    }
                    lct_model model{fam, scale, fam == 2 ? shape : 0.0};
                    lct_codebook cb;
                    if (lct::build_codebook(model, sample, m, &cb) != LCT_OK) {
                        ++bad;
                        continue;
                    }
                    lcto_codebook ocb;
                    lcto_codebook_build(fam, scale, model.shape, sample, m, &ocb);
                    bool same = cb.esc_len == ocb.esc_len && cb.shift == ocb.shift;
                    for (int e = 0; e < 256; ++e) same = same && cb.len[e] == ocb.len[e];
                    for (int e = 0; e < 257; ++e) same = same && cb.code[e] == ocb.code[e];
                    // the same base code with another shift
                    lct_codebook c2;
                    lcto_codebook o2;
                    const int32_t k = (int32_t)(next_u64() % 21) - 10;
                    lct::codebook_from_lengths(cb.len_base, cb.esc_len, k, &c2);
                    lcto_codebook_from_base(ocb.len_base, ocb.esc_len, k, &o2);
                    for (int e = 0; e < 256; ++e) same = same && c2.len[e] == o2.len[e];
                    for (int e = 0; e < 257; ++e) same = same && c2.code[e] == o2.code[e];
                    lct_codebook c3;
                    lct::reshift_codebook(c2, sample, m, &c3);
                    same = same && c3.shift == cb.shift;
                    lct::EncTab et;
                    lct::DecTab dt;
                    lct::fill_enc(c3, &et);
                    lct::fill_dec(c3, &dt);
                    ++checked;
                    if (!same) {
                        ++bad;
                        printf("mismatch: family %d scale %g shape %g m %u\n", fam, scale, model.shape, m);
                    }
                }
            }
        }
    }
    printf("codebooks checked: %d, mismatches: %d\n", checked, bad);
    return bad || pmf_bad ? 1 : 0;
}
