/*
 * lct_oracle.h -- plain, serial CPU oracle of the LCT lossless BF16 exponent codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP library; the two meet only through the
 * seeded input generators, which hold none of the codec's arithmetic.
 *
 * Sources, cited by page and passage:
 *   [LCT-abs]     "LCT: Losslessly Compressed Tensors with GPU friendly execution
 *                 for Training" (scholarbro.com), abstract.
 *   [EXP-split]   "LCT paper - Lossless Huffman coding of BF16 training tensors"
 *                 (learnaivisually.com), the paragraph on the bits of a BF16 value
 *                 (byte split, exponent entropy, capped Huffman codes, escape).
 *   [EXP-streams] same page, paragraph on blocks of 65,536 / 32,768 and 256 streams.
 *   [EXP-train]   same page, paragraph on training traffic and the fused SGD update.
 *   [EXP-ideal]   same page, the paragraph on idealized arithmetic (16/11; 1.4382).
 *   [EXP-limits]  same page, paragraph on the longer-context claim and the limits
 *                 (a distribution that does not fit the tensor raises storage).
 *   [EXP-jargon]  same page, jargon entry "Optimizer state".
 *
 * Where the pages are silent, a convention had to be fixed; every function
 * below states the reading it takes.
 *
 * Parity status: every function here is pinned by tests/test_oracle_*.py.
 * The model probability mass (lcto_model_pmf) and the integer weights
 * (lcto_weights) are pinned bin by bin against 50-digit evaluations of the
 * survival functions written from their definitions (erfc, exp, the
 * regularized incomplete beta), for Gaussian, Laplace and Student-t models
 * with 1, 2, 3 and 5.5 degrees of freedom at several scales.  The
 * Student-t normalising constant is a difference of two lgamma values: past
 * about 100 degrees of freedom it loses 1e-12 (2e-12 at 1000).
 */
#ifndef LCT_ORACLE_H
#define LCT_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LCTO_GAUSSIAN = 0, LCTO_LAPLACE = 1, LCTO_POWERLAW = 2 };

/* Return codes. */
enum {
    LCTO_OK = 0,
    LCTO_OVF_FULL = 1,      /* spill total exceeds ovf_cap; markers still complete */
    LCTO_EINVAL = -1,
    LCTO_EDECODE = -2       /* bit pattern that is no code word */
};

/* A complete codebook: final lengths after the shift plus the canonical codes.
 * len[e] == 0 means exponent field e is escaped (ESC code, then its 8-bit field). */
typedef struct {
    uint8_t  len[256];
    uint8_t  esc_len;
    int32_t  shift;
    uint32_t code[257];     /* canonical code values, MSB-first; [256] = ESC */
    uint8_t  len_base[256]; /* the base code the shift was applied to */
} lcto_codebook;

/* ---- model and codebook construction ([EXP-split]) ---------------------- */

/* Survival function 1 - F(t) of |X| for the model (t >= 0). */
double lcto_model_survival(int family, double scale, double shape, double t);
/* Probability of each 8-bit exponent field under the model. */
int  lcto_model_pmf(int family, double scale, double shape, double p[256]);
/* Integer symbol weights: floor(p * 2^40 + 0.5). */
void lcto_weights(const double p[256], uint64_t w[256]);

/* Length-limited optimal prefix code (package-merge).  n leaves with weights
 * w[i] and tie-break ids id[i]; lengths <= L; needs 2 <= n <= 2^L.
 * Leaves are ordered by (weight, id); at equal weight a leaf precedes a package. */
int  lcto_package_merge(int n, const uint64_t *w, const int *id, int L, uint8_t *len);

/* Escape-set choice on a generic alphabet: keep the k heaviest symbols (ties by
 * smaller id) plus one escape leaf whose weight is the rest; escaped symbols
 * cost len_esc + lit_bits.  Picks the k in 1..min(nsym-1, max(1, #nonzero))
 * with the least cost, the smaller k on ties.  len[i] = 0 for escaped symbols.
 * Returns the cost, or UINT64_MAX on bad input. */
uint64_t lcto_build_escape(int nsym, const uint64_t *w, int L, int lit_bits,
                           uint8_t *len, uint8_t *esc_len, int *k_out);

/* Base code over the 256 exponent fields: L = 8, 8-bit literal. */
uint64_t lcto_build_base(const uint64_t w[256], uint8_t len[256], uint8_t *esc_len, int *k_out);

/* Integer exponent shift minimising the coded bits of the sample exponents
 * under the base code; ties: smallest |k|, then the smaller k. */
int  lcto_best_shift(const uint8_t len_base[256], uint8_t esc_len, const uint8_t *e, size_t m);
/* Bits the sample exponents cost under the base code shifted by k. */
uint64_t lcto_shift_cost(const uint8_t len_base[256], uint8_t esc_len, const uint8_t *e, size_t m, int k);

/* Canonical code values (sorted by (length, id), ESC id 256). */
void lcto_canonical(const uint8_t len[257], uint32_t code[257]);

/* Whole build: pmf -> weights -> base code -> shift from the sample
 * x[floor(i*n/m)], m = min(n, 4096) -> final lengths -> canonical codes. */
int  lcto_codebook_build(int family, double scale, double shape,
                         const uint16_t *x, uint64_t n, lcto_codebook *cb);
/* Final codebook from a base code and a shift (no sampling). */
void lcto_codebook_from_base(const uint8_t len_base[256], uint8_t esc_len, int shift,
                             lcto_codebook *cb);

/* ---- shift re-estimation ([LCT-abs], [EXP-split], [EXP-limits]) ----------- */

/* New shift for a compressed tensor, keeping the base code: decode the tensor
 * (codebook cb), take its sample x[floor(i*n/m)], m = min(n, 4096), pick the
 * shift that minimises the sample's coded bits under cb's base code (same
 * search and tie rule as the build), and apply it: out has cb's base code and
 * escape length with the new shift.  No Huffman code is rebuilt. */
int  lcto_reshift(const lcto_codebook *cb, const uint8_t *sf, const uint32_t *pay,
                  const uint16_t *cnt, const uint64_t *obase, const uint8_t *ovf,
                  uint64_t n, uint32_t block_elems, uint32_t cap_words, lcto_codebook *out);

/* ---- the format ([EXP-split], [EXP-streams]) ----------------------------- */

/* Split / join of one BF16 bit pattern. */
uint8_t  lcto_exponent(uint16_t v);
uint8_t  lcto_signfrac(uint16_t v);
uint16_t lcto_join(uint8_t sf, uint8_t e);

/* One block of nb elements (1..block_elems).  Outputs are block-local:
 * sf[nb]; pay[cap_words*256] word-interleaved (word w of stream s at w*256+s);
 * cnt[256]; spilled exponent bytes to spill[] in (stream, position) order,
 * their number to *nspill (spill must hold nb bytes). */
int  lcto_encode_block(const lcto_codebook *cb, const uint16_t *x, uint32_t nb,
                       uint32_t cap_words, uint8_t *sf, uint32_t *pay, uint16_t *cnt,
                       uint8_t *spill, uint32_t *nspill);
/* Inverse of lcto_encode_block; spill points at this block's spilled bytes. */
int  lcto_decode_block(const lcto_codebook *cb, const uint8_t *sf, const uint32_t *pay,
                       const uint16_t *cnt, const uint8_t *spill, uint32_t nb,
                       uint32_t cap_words, uint16_t *y);

/* Whole tensor.  nblk = ceil(n / block_elems); sf[n]; pay[nblk*cap_words*256];
 * cnt[nblk*256]; obase[nblk+1]; ovf[ovf_cap].  Overflow bytes beyond ovf_cap
 * are not written; obase is always complete. */
int  lcto_encode(const lcto_codebook *cb, const uint16_t *x, uint64_t n,
                 uint32_t block_elems, uint32_t cap_words,
                 uint8_t *sf, uint32_t *pay, uint16_t *cnt, uint64_t *obase,
                 uint8_t *ovf, uint64_t ovf_cap);
int  lcto_decode(const lcto_codebook *cb, const uint8_t *sf, const uint32_t *pay,
                 const uint16_t *cnt, const uint64_t *obase, const uint8_t *ovf,
                 uint64_t n, uint32_t block_elems, uint32_t cap_words, uint16_t *y);

/* ---- SGD update ([EXP-train]) -------------------------------------------- */

float    lcto_fmaf(float a, float b, float c);
uint16_t lcto_rne_bf16(float r);
/* One element: rne(fmaf(-eta, f32(m), f32(w))). */
uint16_t lcto_sgd_elem(uint16_t w, uint16_t m, float eta);

/* Naive round trip of one SGD step: decode W (codebook cw) and M (cm) fully,
 * update densely, re-encode W' with cw_out (cw when NULL).  Input and output
 * compressed tensors share n, block_elems and cap_words. */
int  lcto_sgd(const lcto_codebook *cw, const uint8_t *w_sf, const uint32_t *w_pay,
              const uint16_t *w_cnt, const uint64_t *w_obase, const uint8_t *w_ovf,
              const lcto_codebook *cm, const uint8_t *m_sf, const uint32_t *m_pay,
              const uint16_t *m_cnt, const uint64_t *m_obase, const uint8_t *m_ovf,
              float eta, const lcto_codebook *cw_out, uint64_t n, uint32_t block_elems, uint32_t cap_words,
              uint8_t *o_sf, uint32_t *o_pay, uint16_t *o_cnt, uint64_t *o_obase,
              uint8_t *o_ovf, uint64_t ovf_cap);

/* ---- Momentum step ([EXP-jargon], [EXP-train]) ---------------------------- */

/* One element of SGD with momentum: m' = rne(fmaf(mu, f32(m), f32(g))), then
 * w' = rne(fmaf(-eta, f32(m'), f32(w))) with m' as stored (BF16). */
void lcto_momentum_elem(uint16_t w, uint16_t m, uint16_t g, float mu, float eta,
                        uint16_t *w_out, uint16_t *m_out);

/* Naive round trip of one momentum step: decode W (codebook cw) and M (cm)
 * fully, update densely with the dense gradient g, re-encode W' with cw_out
 * and M' with cm_out (cw and cm when NULL).  Inputs and outputs share n,
 * block_elems and cap_words.
 * Returns LCTO_OVF_FULL if either output's spill exceeds its ovf_cap. */
int  lcto_momentum(const lcto_codebook *cw, const uint8_t *w_sf, const uint32_t *w_pay,
                   const uint16_t *w_cnt, const uint64_t *w_obase, const uint8_t *w_ovf,
                   const lcto_codebook *cm, const uint8_t *m_sf, const uint32_t *m_pay,
                   const uint16_t *m_cnt, const uint64_t *m_obase, const uint8_t *m_ovf,
                   const uint16_t *g, float mu, float eta,
                   const lcto_codebook *cw_out, const lcto_codebook *cm_out,
                   uint64_t n, uint32_t block_elems, uint32_t cap_words,
                   uint8_t *ow_sf, uint32_t *ow_pay, uint16_t *ow_cnt, uint64_t *ow_obase,
                   uint8_t *ow_ovf, uint64_t ow_ovf_cap,
                   uint8_t *om_sf, uint32_t *om_pay, uint16_t *om_cnt, uint64_t *om_obase,
                   uint8_t *om_ovf, uint64_t om_ovf_cap);

#ifdef __cplusplus
}
#endif
#endif
