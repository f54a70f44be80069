/*
 * lct.h -- C ABI of the LCT lossless BF16 exponent codec for MI355X (gfx950).
 *
 * A BF16 tensor is stored as a raw sign-fraction byte per element plus its
 * exponents, Huffman-coded with a precomputed, length-limited codebook (codes
 * of at most 8 bits; rare exponents take one escape code followed by the 8-bit
 * field).  Each block of elements is dealt round-robin into 256 streams of a
 * fixed capacity; the exponents that do not fit spill, raw, to an overflow
 * region whose start is recorded per block.  Sources:
 *   "LCT: Losslessly Compressed Tensors with GPU friendly execution for
 *    Training" (scholarbro.com), abstract;
 *   "LCT paper - Lossless Huffman coding of BF16 training tensors"
 *    (learnaivisually.com): the paragraph on bits (byte split, 8-bit cap,
 *    escape, precomputed codebook and sampled shift), the paragraph on blocks
 *    and streams (65,536 / 32,768 elements, 256 streams, fixed capacity,
 *    overflow and its marker), the paragraph on training traffic (the
 *    fused SGD update W_{t+1} = W_t - eta * M_t), the jargon entry
 *    "Optimizer state" (the momentum buffer is stored compressed too) and the
 *    paragraph on the limits (a distribution that does not fit the tensor
 *    raises storage).
 *
 * Conventions (common to every call):
 *   - Every function returns lct_status (0 = LCT_OK) and never throws.
 *   - Pointers named d_* and every pointer inside lct_tensor are DEVICE
 *     pointers on the current HIP device; every other pointer is host memory.
 *   - The caller allocates and frees every device buffer, sized by lct_sizes().
 *     The library allocates no device memory of its own, except two static
 *     arrays per device: 8 KiB used by lct_codebook_build() and
 *     lct_codebook_reshift() for their sample, and the working memory of
 *     lct_sgd_step_noalloc() (LCT_NOALLOC_SCRATCH_BYTES).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     lct_encode, lct_decode and the update calls (lct_sgd_step*,
 *     lct_momentum_step*) only enqueue work on it and return at once, as do
 *     the group calls and lct_group_fit; lct_codebook_build,
 *     lct_codebook_reshift, lct_codebook_reshift_dense, lct_tensor_sample
 *     and lct_codebook_adapt synchronise it (they read a sample back), and
 *     lct_group_bind copies its table with a blocking copy.
 *   - Errors found on the host (null pointer, bad size, misalignment, illegal
 *     aliasing, a current device that is not gfx950) are returned before
 *     anything is enqueued.  Which device a buffer lives on is not checked:
 *     every buffer must be on the current device.
 *     Sizes are bounded so that nothing computed from them wraps: n (of a
 *     tensor, a group member or a dense input) at most 2^48 elements, at
 *     most 2^32 - 1 blocks, ovf_cap at most 2^56 bytes; larger ones give
 *     LCT_EINVAL.
 *     The only data-dependent failure is a too-small overflow region: it is
 *     reported through the device status word (LCT_ST_* bits), never by a
 *     fault.  n == 0 (for a group: no blocks) is a no-op that returns LCT_OK
 *     and writes nothing; the empty encoding is obase = [0] with status 0, so
 *     storage whose obase and status start zeroed already holds it.
 *   - Thread-safe: the global state is the sample array (guarded by a lock),
 *     per-device caches of constants (guarded), and the working memory of
 *     lct_sgd_step_noalloc, which calls overlapping on one device share.
 */
#ifndef LCT_H
#define LCT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LCT_OK = 0,
    LCT_EINVAL = -1,  /* null pointer, bad layout, bad model, size mismatch */
    LCT_EALIGN = -2,  /* device pointer not aligned as documented */
    LCT_EALIAS = -3,  /* output overlaps an input it must not overlap */
    LCT_EHIP = -4,    /* a HIP runtime call failed (message via lct_last_hip_error) */
    LCT_EARCH = -5,   /* current device is not gfx950 */
    LCT_ESIZE = -6    /* lct_sgd_step_noalloc: the tensor needs more working memory
                         than its static scratch holds */
} lct_status;

/* Device status word bits, OR-ed in by the kernels (the word is cleared at the
 * start of every lct_encode and every update call that writes the tensor). */
#define LCT_ST_OVF_FULL 0x1u   /* total spill > ovf_cap: the overflow region is incomplete;
                                  obase[nblk] still holds the size needed */
#define LCT_ST_LOOKBACK 0x2u   /* overflow-offset scan gave up waiting (never expected) */

/* Codebook model picked by the user (explainer, paragraph on bits: a
 * Gaussian, Laplace or power-law distribution).  scale = sigma (Gaussian),
 * b (Laplace) or the t scale (power law = Student-t, shape = degrees of
 * freedom). */
typedef enum { LCT_GAUSSIAN = 0, LCT_LAPLACE = 1, LCT_POWERLAW = 2 } lct_family;
typedef struct {
    int32_t family;   /* lct_family */
    double scale;
    double shape;
} lct_model;

/* Block layouts (explainer, paragraph on blocks and streams: 65,536-element
 * blocks in CLEAN, 32,768 in MEDIUM and HIGH).  cap_words is each stream's
 * capacity in 32-bit words: CLEAN 25 (16 / (8 + 800/256) = 1.4382x, the
 * bound printed for CLEAN), MEDIUM 12 (8 + 3 bits per value, 16/11), HIGH 11.
 * Any block_elems that is a multiple of 4096 in [4096, 65536] and any
 * cap_words in [1, 64] is accepted. */
typedef enum { LCT_CLEAN = 0, LCT_MEDIUM = 1, LCT_HIGH = 2 } lct_mode;
typedef struct {
    uint32_t block_elems;
    uint32_t cap_words;
} lct_layout;

/* Host-side codebook (plain old data, about 4 KiB).  len[e] is the code
 * length of exponent field e, 0 when e is escaped (then it costs esc_len + 8
 * bits: the escape code, then the field's 8 bits, least significant first).
 * code[] holds canonical code values (ordered by length, then field; the
 * escape symbol has id 256); codes enter a stream most significant bit first.
 * len_base[] is the base code the shift was applied to: len[e] =
 * len_base[e - shift] where 0 <= e - shift <= 255, else 0; shift re-estimation
 * keeps it.  The remaining members are lookup tables derived from
 * len/esc_len by the library: treat them as opaque.  Every call that takes a
 * codebook returns LCT_EINVAL for one whose tables break the ranges the
 * kernels rely on (escape code of 1..8 bits, every field 1..16 bits with no
 * bits past its length, decode lengths at most 16), such as a zeroed struct
 * that was never built. */
typedef struct {
    uint8_t  len[256];
    uint8_t  esc_len;
    uint8_t  max_len;
    int16_t  shift;        /* exponent offset applied to the base code */
    uint32_t kept;         /* number of exponent fields with a code */
    lct_model model;
    uint32_t code[257];
    uint32_t enc_bits[256];   /* stream bits of each field, LSB-first (code reversed, literal) */
    uint8_t  enc_len[256];    /* bits each field costs */
    uint16_t dec[256];        /* 8-bit peek -> field | bits << 8 | escape << 13 | invalid << 14 */
    uint8_t  len_base[256];   /* base code lengths before the shift */
} lct_codebook;

/* A compressed tensor: every pointer is a caller-owned device buffer.
 *   n          number of BF16 elements
 *   layout     block_elems, cap_words;  nblk = ceil(n / block_elems)
 *   sf         uint8[n]      sign-fraction bytes in element order (16-byte aligned)
 *   pay        uint32[nblk * cap_words * 256]  word w of stream s of block b at
 *              (b * cap_words + w) * 256 + s; stream bit k is bit (k mod 32) of
 *              its word k / 32; unused bits are 0 (16-byte aligned)
 *   cnt        uint16[nblk * 256]  coded prefix length of each stream; the rest
 *              of the stream's elements are in the overflow region (4-byte aligned)
 *   obase      uint64[nblk + 1]  where block b's spilled bytes start in ovf;
 *              obase[nblk] = total spilled bytes (8-byte aligned)
 *   ovf        uint8[ovf_cap]  spilled exponent fields, raw, in (block,
 *              stream, position) order.  ovf_cap = n always suffices; with
 *              ovf_cap >= nblk * block_elems the writing calls stage spilled
 *              fields at fixed places in scratch instead of claiming space
 *              from one shared counter, which is much faster when many
 *              streams spill
 *   status     uint32[1]  LCT_ST_* bits
 *   scratch    lct_sizes().scratch bytes of working memory (256-byte aligned);
 *              only lct_encode and the output of lct_sgd_step and
 *              lct_momentum_step use it.  It may be shared by
 *              calls that do not overlap in time.
 * Element r of block b (r < block_elems) is position r / 256 of stream r % 256. */
typedef struct {
    uint64_t n;
    lct_layout layout;
    uint8_t  *sf;
    uint32_t *pay;
    uint16_t *cnt;
    uint64_t *obase;
    uint8_t  *ovf;
    uint64_t ovf_cap;
    uint32_t *status;
    void     *scratch;
} lct_tensor;

typedef struct {
    uint64_t nblk;
    uint64_t sf, pay, cnt, obase;   /* bytes */
    uint64_t scratch;               /* bytes, for the given ovf_cap */
    uint64_t fixed;                 /* sf + pay + cnt + obase: compressed size before spills */
} lct_sizes_t;

/* Layout of a mode.  Errors: LCT_EINVAL for an unknown mode or null out. */
lct_status lct_layout_init(int32_t mode, lct_layout *out);

/* Buffer sizes of an n-element tensor.  Errors: LCT_EINVAL for a layout
 * outside the accepted range, a null pointer, or sizes past the limits that
 * every call checks (see the conventions). */
lct_status lct_sizes(uint64_t n, const lct_layout *layout, uint64_t ovf_cap, lct_sizes_t *out);

/* Codebook build (explainer, paragraph on bits: the code is fixed ahead of
 * training from a model distribution chosen by the user, and an exponent
 * offset estimated on at most 4096 sampled values adapts it to the tensor's
 * magnitude).
 * Steps: model probability of every exponent field -> integer weights
 * floor(p * 2^40 + 0.5) -> escape set (the k heaviest fields kept, k chosen
 * for the least expected bits) with length-limited Huffman (package-merge,
 * 8-bit cap) -> integer shift k minimising the coded bits of the sample
 * d_x[floor(i * n / m)], m = min(n, 4096) (ties: smallest |k|, then the smaller
 * k) -> final lengths len[e] = base[e - k] -> canonical codes -> lookup tables.
 * d_x: device BF16 bit patterns, n elements (may be NULL when n == 0: shift 0).
 * Synchronises `stream`.  Errors: LCT_EINVAL (bad model, null out),
 * LCT_EARCH, LCT_EHIP. */
lct_status lct_codebook_build(const lct_model *model, const uint16_t *d_x, uint64_t n,
                              void *stream, lct_codebook *out);

/* Codebook from given base lengths and shift (no model, no sampling): the
 * final lengths are len_base[e - shift].  len_base[] must be a prefix code
 * together with esc_len (Kraft sum <= 1, lengths <= 8, esc_len in 1..8).
 * Errors: LCT_EINVAL. */
lct_status lct_codebook_from_lengths(const uint8_t len_base[256], uint8_t esc_len, int32_t shift,
                                     lct_codebook *out);

/* Shift re-estimation (abstract: adaptation to magnitude shifts; explainer,
 * paragraph on bits: an exponent offset estimated on at most 4096 sampled
 * values adapts the code to the tensor's magnitude; paragraph on the limits:
 * a distribution that no longer fits the tensor raises storage).  Takes the current values of the
 * compressed tensor *t (decoded with *cb) at positions floor(i * n / m),
 * m = min(n, 4096), as lct_codebook_build does, and picks the shift that
 * minimises their coded bits under cb's base code (same search and ties).
 * *out gets cb's base code, escape length and model with the new shift; no
 * Huffman code is rebuilt.  n == 0 gives shift 0.  The tensor keeps its
 * encoding: it moves to *out when it is next written (lct_encode, or an
 * update call with *out as its output codebook).  Synchronises `stream`.
 * Errors: LCT_EINVAL, LCT_EALIGN, LCT_EARCH, LCT_EHIP. */
lct_status lct_codebook_reshift(const lct_codebook *cb, const lct_tensor *t, void *stream,
                                lct_codebook *out);

/* The shift sample of a compressed tensor, as lct_codebook_reshift takes it:
 * out[i] = element floor(i * n / m) of *t (decoded with *cb), i < m =
 * min(n, 4096), as BF16 bit patterns in host memory (out holds 4096 values);
 * *m_out (may be NULL) gets m.  Synchronises `stream`.  Errors: as
 * lct_codebook_reshift. */
lct_status lct_tensor_sample(const lct_codebook *cb, const lct_tensor *t, void *stream,
                             uint16_t *out, uint32_t *m_out);

/* Shift re-estimation from a dense tensor: d_x (device BF16 bit patterns, n
 * elements) sampled at floor(i * n / m), m = min(n, 4096), as
 * lct_codebook_build does, and cb's base code, escape length and model kept
 * with the shift that minimises the sample's coded bits.  For a codebook
 * built from a model this equals lct_codebook_build(model, d_x) without
 * building the Huffman code again: the per-tensor codebook of a saved
 * activation (abstract: activations are compressed too).  n == 0 gives shift
 * 0.  Synchronises `stream`.  Errors: LCT_EINVAL, LCT_EARCH, LCT_EHIP. */
lct_status lct_codebook_reshift_dense(const lct_codebook *cb, const uint16_t *d_x, uint64_t n,
                                      void *stream, lct_codebook *out);

/* Re-estimation when the spill has grown: reads t's spilled total
 * (obase[nblk]); if it exceeds max_spill_per_elem * n bytes, *out is
 * lct_codebook_reshift(cb, t), else a copy of *cb.  *changed (may be NULL)
 * is set to 1 when out's shift differs from cb's, else 0.  Synchronises
 * `stream`.  Errors: as lct_codebook_reshift; LCT_EINVAL for a negative or
 * NaN limit. */
lct_status lct_codebook_adapt(const lct_codebook *cb, const lct_tensor *t, double max_spill_per_elem,
                              void *stream, lct_codebook *out, int32_t *changed);

/* Encode (explainer, paragraphs on bits and on blocks and streams).
 * d_x: device BF16 bit patterns, out->n elements, 16-byte aligned.  Writes
 * every buffer of *out (all of sf, pay, cnt, obase, status; ovf below ovf_cap).
 * If the spill exceeds out->ovf_cap, LCT_ST_OVF_FULL is set in *out->status
 * and obase[nblk] holds the capacity needed: allocate more and encode again.
 * The fixed side (sf, pay, cnt, obase) is complete even then; ovf is never
 * written past ovf_cap, and its content is unspecified.
 * Safe bound: ovf_cap = n.  Errors: LCT_EINVAL, LCT_EALIGN, LCT_EALIAS (d_x
 * overlapping an output), LCT_EARCH, LCT_EHIP. */
lct_status lct_encode(const lct_codebook *cb, const uint16_t *d_x, const lct_tensor *out,
                      void *stream);

/* Decode: the inverse of lct_encode (explainer, first paragraph: every
 * value decodes exactly).  d_y: device uint16[in->n], 16-byte aligned, must
 * not overlap *in.  Errors: LCT_EINVAL, LCT_EALIGN, LCT_EALIAS, LCT_EARCH,
 * LCT_EHIP. */
lct_status lct_decode(const lct_codebook *cb, const lct_tensor *in, uint16_t *d_y, void *stream);

/* Fused SGD step (explainer, paragraph on training traffic: read the
 * compressed operands once, do the arithmetic, and store the re-encoded
 * result, all in a single pass).  W' = W - eta * M, element by element as
 * rne_bf16(fmaf(-eta, f32(m), f32(w))) with a NaN result written as 0x7FC0;
 * W' is encoded with cw (the codebook of W).  w_in, m, w_out share n and
 * layout.  w_out's sf, pay, cnt and obase may be w_in's own (in-place update);
 * w_out's ovf, status and scratch must not overlap any buffer of w_in or m, and
 * m must not overlap w_out.  If LCT_ST_OVF_FULL is set after an in-place
 * update, W is lost: callers that cannot bound the spill update out of place.
 * Errors: LCT_EINVAL, LCT_EALIGN, LCT_EALIAS, LCT_EARCH, LCT_EHIP. */
lct_status lct_sgd_step(const lct_codebook *cw, const lct_tensor *w_in,
                        const lct_codebook *cm, const lct_tensor *m,
                        float eta, const lct_tensor *w_out, void *stream);

/* lct_sgd_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step, arguments, rules and errors, except that w_out->scratch is
 * ignored (it may be NULL) and the library's own static working memory is used
 * instead: one array of LCT_NOALLOC_SCRATCH_BYTES per device, reserved when the
 * library is loaded and held until the process ends.  The call allocates
 * nothing.  The working memory needed is lct_sizes(n, layout,
 * w_out->ovf_cap).scratch; more than LCT_NOALLOC_SCRATCH_BYTES returns
 * LCT_ESIZE before anything is enqueued (16 MiB holds, e.g., a 2^24-element
 * tensor with ovf_cap up to 8,314,624 bytes, or ovf_cap = n up to about 8.3M
 * elements).  Every call on a device shares
 * that device's array: calls that overlap in time on one device (on
 * different streams, or from several host threads without ordering) race and
 * give undefined results.  The array keeps the last call's contents; what must
 * start at zero is cleared by a kernel on `stream` at the start of each call. */
#define LCT_NOALLOC_SCRATCH_BYTES (16u << 20)
lct_status lct_sgd_step_noalloc(const lct_codebook *cw, const lct_tensor *w_in,
                                const lct_codebook *cm, const lct_tensor *m,
                                float eta, const lct_tensor *w_out, void *stream);

/* lct_sgd_step with W' encoded with cw_out instead of cw (W is still decoded
 * with cw): the step that moves W onto a codebook from lct_codebook_reshift.
 * Same arguments, rules and errors otherwise; cw_out == cw is lct_sgd_step. */
lct_status lct_sgd_step_recode(const lct_codebook *cw, const lct_tensor *w_in,
                               const lct_codebook *cm, const lct_tensor *m, float eta,
                               const lct_codebook *cw_out, const lct_tensor *w_out, void *stream);

/* Momentum step (explainer, jargon entry "Optimizer state": the momentum
 * buffer of SGD with momentum is stored compressed like the weights; paragraph
 * on training traffic: decode, update, re-encode in one pass).  Element by
 * element, m' = rne_bf16(fmaf(mu, f32(m), f32(g))), then
 * w' = rne_bf16(fmaf(-eta, f32(m'), f32(w))) with m' as rounded to BF16 (the
 * value M' stores); a NaN result is written as 0x7FC0.  W' is encoded with
 * cw, M' with cm.
 * d_g: the dense gradient, device BF16 bit patterns, n elements, 16-byte
 * aligned, overlapping no output.  w_in, m_in, w_out, m_out share n and
 * layout.  Each output's sf, pay, cnt and obase may be its own input's
 * (in-place step) or disjoint from every input; its ovf, status and scratch
 * must not overlap any input, and the two outputs must not overlap each other.
 * Each output has its own status word (LCT_ST_OVF_FULL as for lct_encode).
 * The step is one pass: W' is computed from M' as rounded, not from M''s
 * stored form, so an overflow of m_out's region leaves W' complete and
 * w_out's status clean (and the other way round).  After an in-place step
 * whose output overflowed, that input is lost: callers that cannot bound the
 * spill step out of place or size ovf_cap = n.
 * Errors: LCT_EINVAL, LCT_EALIGN, LCT_EALIAS, LCT_EARCH, LCT_EHIP. */
lct_status lct_momentum_step(const lct_codebook *cw, const lct_tensor *w_in,
                             const lct_codebook *cm, const lct_tensor *m_in,
                             const uint16_t *d_g, float mu, float eta,
                             const lct_tensor *w_out, const lct_tensor *m_out, void *stream);

/* lct_momentum_step with W' encoded with cw_out and M' with cm_out (W and M
 * are still decoded with cw and cm).  Same arguments, rules and errors
 * otherwise. */
lct_status lct_momentum_step_recode(const lct_codebook *cw, const lct_tensor *w_in,
                                    const lct_codebook *cm, const lct_tensor *m_in,
                                    const uint16_t *d_g, float mu, float eta,
                                    const lct_codebook *cw_out, const lct_codebook *cm_out,
                                    const lct_tensor *w_out, const lct_tensor *m_out, void *stream);

/* ---- tensor groups ---------------------------------------------------------
 * Many tensors in one launch, with one shared overflow region (explainer,
 * paragraph on the idealized arithmetic: measured memory includes the shared
 * overflow buffer).  A group lays its tensors side by side: tensor k's blocks
 * follow tensor k-1's in one set of arrays (pay, cnt and obase indexed by the
 * group's block number), its sign-fraction bytes start at a multiple of 256 in
 * one sf array, and every spilled byte goes to one overflow region, in tensor
 * order; obase values are offsets into that shared region.  Each tensor keeps
 * its own codebook and its own dense buffer.  Tensor k alone is an ordinary
 * lct_tensor (lct_group_tensor) that every other call accepts.
 *
 * The group's storage is one lct_tensor whose n is the group's sf_bytes and
 * whose arrays are sized by lct_group_sizes; its status word and scratch
 * serve the whole group.  The sf bytes between one member's last element and
 * the next member's start (the padding to a multiple of 256) are never read
 * or written by any call: storage whose sf array was zeroed once keeps zero
 * padding, as the format's reference layout has it. */
typedef struct {
    uint32_t count;              /* tensors */
    lct_layout layout;
    uint64_t nblk;               /* blocks of all tensors */
    uint64_t sf_bytes;           /* sf array: every n[k] rounded up to a multiple of 256 */
    uint64_t shape_hash;         /* fingerprint of (layout, n[]) */
    const uint64_t *n;           /* host, caller-owned, count entries, alive while the group is used */
    uint16_t *const *d_dense;    /* host array of device pointers, caller-owned (may be NULL) */
    void *d_table;               /* device descriptor table */
} lct_group;

/* Bytes of the device descriptor table of a group (count tensors of n[k]
 * elements in `layout`).  Errors: LCT_EINVAL. */
lct_status lct_group_table_bytes(uint32_t count, const uint64_t *n, const lct_layout *layout,
                                 uint64_t *bytes);

/* Set up a group: tensor k has n[k] elements (0 allowed), codebook cbs[k]
 * (used to encode and decode it; for a group used as M in an update, to
 * decode it) and dense buffer d_dense[k] (device BF16, 16-byte aligned, the
 * source of lct_encode_group and the target of lct_decode_group; d_dense may
 * be NULL for a group that is only updated).  Dense buffers must not overlap
 * each other.  Writes the descriptor table to d_table (device,
 * lct_group_table_bytes bytes, 256-byte aligned) with a blocking copy and
 * fills *out, which keeps the n and d_dense pointers.  The copy is not
 * ordered with work queued on other streams: no such work may still use
 * d_table's memory.  Errors: LCT_EINVAL, LCT_EALIGN, LCT_EALIAS, LCT_EARCH,
 * LCT_EHIP. */
lct_status lct_group_bind(uint32_t count, const uint64_t *n, const lct_layout *layout,
                          const lct_codebook *cbs, uint16_t *const *d_dense, void *d_table,
                          lct_group *out);

/* A one-tensor group whose codebook is fitted on the device, for callers
 * that must not wait for it (a tensor saved for backward): the shift of the
 * dense tensor's sample over base's base code is chosen on the device, as
 * lct_codebook_reshift_dense chooses it, and the shifted code's tables are
 * built there and written to d_table (lct_group_table_bytes(1, n, layout)
 * bytes, 256-byte aligned) with the tensor's record.  n and d_dense are
 * one-element host arrays owned by the caller (kept in *out); d_shift (device
 * int32, may be NULL) receives the shift, so that the host codebook
 * (lct_codebook_from_lengths(base->len_base, base->esc_len, shift)) can be
 * made once it is read.  Enqueues only.  Errors: LCT_EINVAL, LCT_EALIGN,
 * LCT_EARCH, LCT_EHIP. */
lct_status lct_group_fit(const lct_codebook *base, const uint64_t *n, uint16_t *const *d_dense,
                         const lct_layout *layout, void *d_table, int32_t *d_shift, void *stream,
                         lct_group *out);

/* Sizes of a group's storage arrays (as lct_sizes for one tensor). */
lct_status lct_group_sizes(const lct_group *g, uint64_t ovf_cap, lct_sizes_t *out);

/* Tensor k of a group as an lct_tensor: views into the storage `all` (its
 * ovf, ovf_cap, status and scratch are all's; its obase values point into
 * the shared overflow region, so its spilled bytes are obase[nblk] -
 * obase[0]).  Use it as the input of any call (decode, sample, an update's
 * input); write a group only with the group calls, since a single-tensor
 * output rewrites the overflow region from its start. */
lct_status lct_group_tensor(const lct_group *g, const lct_tensor *all, uint32_t k, lct_tensor *out);

/* Encode every tensor of the group from its dense buffer, in one launch
 * (plus the clear and the overflow scan).  As lct_encode otherwise: the
 * status word reports a too-small shared overflow region.  Errors:
 * LCT_EINVAL (no dense buffers, storage not sized for g), LCT_EALIGN,
 * LCT_EALIAS (a dense buffer overlapping the storage), LCT_EARCH, LCT_EHIP. */
lct_status lct_encode_group(const lct_group *g, const lct_tensor *all, void *stream);

/* Decode every tensor of the group into its dense buffer, in one launch. */
lct_status lct_decode_group(const lct_group *g, const lct_tensor *all, void *stream);

/* Fused SGD step on a group, in one launch: W' = W - eta * M per tensor as
 * lct_sgd_step, with gw's codebooks for W and W' and gm's for M.  gw and gm
 * must have the same layout and sizes.  Storage aliasing rules as
 * lct_sgd_step (w_out may be w_all in place).  Errors: as lct_sgd_step. */
lct_status lct_sgd_step_group(const lct_group *gw, const lct_tensor *w_all, const lct_group *gm,
                              const lct_tensor *m_all, float eta, const lct_tensor *w_out,
                              void *stream);

/* Momentum step on groups (lct_momentum_step per tensor, in one launch):
 * gw's codebooks for W and W', gm's for M and M', and the gradients are gg's
 * dense buffers (gg's codebooks are not used).  The three groups must have the
 * same layout and sizes; the gradients must not overlap an output.  Storage aliasing rules as lct_momentum_step.  Errors: as
 * lct_momentum_step. */
lct_status lct_momentum_step_group(const lct_group *gw, const lct_tensor *w_all, const lct_group *gm,
                                   const lct_tensor *m_all, const lct_group *gg, float mu, float eta,
                                   const lct_tensor *w_out, const lct_tensor *m_out, void *stream);

/* Message for a status code (static string). */
const char *lct_strerror(lct_status st);
/* Text of the last HIP error seen on this thread (static per thread). */
const char *lct_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LCT_H */
