// lct_internal.h -- parameter blocks shared by the C ABI (api.cpp) and the
// HIP kernels (kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lct.h"

namespace lct {

constexpr uint32_t kStreams = 256;          // streams per block
constexpr uint32_t kChunk = 16;             // positions per stream processed per loop step
constexpr uint32_t kMinBlock = kStreams * kChunk;
constexpr uint32_t kMaxBlock = 65536;
constexpr uint32_t kMaxCapWords = 64;

constexpr uint32_t kMaxUnits = 4;           // units a block is split into
constexpr uint32_t kUnitStreams = kStreams / kMaxUnits;   // streams per unit: one wave's lanes

// Scratch layout (bytes).  The header and the scan's look-back flags are
// cleared by a fill kernel before each encode / SGD launch.  Every unit of the
// main kernel writes its record (spilled bytes, where they sit in the second
// staging area, whether its counts were parked).  Spilled exponent fields are
// parked per stream in the first staging area while a unit runs, copied into
// one contiguous piece per unit at its end, and placed in the overflow region
// by the placing kernel once the scan has given every block its offset.  An
// in-place update parks its counts too, so that no unit overwrites counts
// another unit of the same block has yet to read; the placing kernel puts
// them in place.
constexpr uint64_t kScrTicket2 = 4;   // uint32: next group of the scan kernel
constexpr uint64_t kScrStage = 8;     // uint64: bytes claimed in the first staging area
constexpr uint64_t kScrStage2 = 16;   // uint64: bytes claimed in the second
constexpr uint64_t kScrParked = 24;   // uint32: nonzero when some unit parked its counts
constexpr uint64_t kScrFullUnits = 28;  // uint32: units the update ran on its full-block path
                                        // (read by tests to show which path ran)
constexpr uint64_t kScrFlags = 64;    // uint64[groups + 1]: the scan's look-back flags
constexpr uint32_t kScanGroup = 256;  // blocks per scan workgroup (the flags are sized for
                                      // one group per 256 units, more than it needs)
__host__ __device__ inline uint64_t scr_units(uint64_t nblk) { return kMaxUnits * nblk; }
__host__ __device__ inline uint64_t scr_clear_bytes(uint64_t nblk) {
    return kScrFlags + 8 * ((scr_units(nblk) + kScanGroup - 1) / kScanGroup + 1);
}
__host__ __device__ inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }
__host__ __device__ inline uint64_t scr_rec_offset(uint64_t nblk) { return align256(scr_clear_bytes(nblk)); }
__host__ __device__ inline uint64_t scr_cnt_offset(uint64_t nblk) {
    return align256(scr_rec_offset(nblk) + 16 * scr_units(nblk));
}
__host__ __device__ inline uint64_t scr_stage_offset(uint64_t nblk) {
    return align256(scr_cnt_offset(nblk) + 2 * kStreams * nblk);
}
__host__ __device__ inline uint64_t scr_stage2_offset(uint64_t nblk, uint64_t ovf_cap) {
    return align256(scr_stage_offset(nblk) + ovf_cap);
}
__host__ __device__ inline uint64_t scr_bytes(uint64_t nblk, uint64_t ovf_cap) {
    return scr_stage2_offset(nblk, ovf_cap) + ovf_cap;
}

// A unit's record: where its spilled bytes sit in the second staging area,
// how many there are, and flags (bit 0: its counts are parked in scratch).
struct UnitRec {
    uint64_t base;
    uint32_t total, flags;
};

// Encoder tables: stream bits of each exponent field and their count.
struct EncTab {
    uint32_t bits[256];
    uint8_t len[256];
};

// Decoder table: 8-bit peek -> field | bits << 8 | escape << 13 | invalid << 14
// (the kernels expand it in LDS).
struct DecTab {
    uint16_t dec[256];
    uint32_t esc_len;
};

// Tensor groups: tensor k's blocks follow tensor k-1's in one set of arrays
// (pay, cnt, obase indexed by the group's block number; sf at the tensor's
// own offset e0, a multiple of 256), one overflow region for all.  The device
// table holds a record per tensor, the tensor of every block and every
// tensor's code tables.
struct GroupEntry {
    uint16_t *dense;      // encode source and decode target (null: none)
    uint64_t n;           // elements
    uint64_t e0;          // first sign-fraction byte in the group's sf array
    uint32_t blk0, nblk;  // first block in the group, blocks
};
// blk_tab[b]: the first tensor whose code tables are byte-identical to those
// of block b's tensor (tensors with one model and one shift share tables, so
// an update that walks many tensors stages them only when they change).
struct GroupRef {
    const GroupEntry *ent;
    const EncTab *enc;
    const DecTab *dec;
    const uint32_t *blk_tensor;
    const uint32_t *blk_tab;
};
// Offsets of the parts of a group's device table.
struct GroupTableLayout {
    uint64_t ent, enc, dec, blk_tensor, blk_tab, bytes;
};
inline GroupTableLayout group_table_layout(uint64_t count, uint64_t nblk) {
    auto up = [](uint64_t v) { return (v + 255) & ~uint64_t(255); };
    GroupTableLayout t;
    t.ent = 0;
    t.enc = up(t.ent + count * sizeof(GroupEntry));
    t.dec = up(t.enc + count * sizeof(EncTab));
    t.blk_tensor = up(t.dec + count * sizeof(DecTab));
    t.blk_tab = up(t.blk_tensor + nblk * sizeof(uint32_t));
    t.bytes = up(t.blk_tab + nblk * sizeof(uint32_t));
    return t;
}

struct EncodeParams {
    const uint16_t *x;
    uint64_t n;
    uint32_t block_elems, cap_words, nblk, pad0;
    uint8_t *sf;
    uint32_t *pay;
    uint16_t *cnt;
    uint64_t *obase;
    uint8_t *ovf;
    uint64_t ovf_cap;
    uint32_t *status;
    uint8_t *scratch;
    GroupRef grp;         // used by the group kernels only
    EncTab enc;
};

struct DecodeParams {
    const uint8_t *sf;
    const uint32_t *pay;
    const uint16_t *cnt;
    const uint64_t *obase;
    const uint8_t *ovf;
    uint64_t ovf_cap;
    uint16_t *y;
    uint64_t n;
    uint32_t block_elems, cap_words, nblk, pad0;
    GroupRef grp;         // used by the group kernels only
    DecTab dec;
};

struct SgdParams {
    // inputs: W (codebook cw) and M (codebook cm)
    const uint8_t *w_sf;
    const uint32_t *w_pay;
    const uint16_t *w_cnt;
    const uint64_t *w_obase;
    const uint8_t *w_ovf;
    uint64_t w_ovf_cap;
    const uint8_t *m_sf;
    const uint32_t *m_pay;
    const uint16_t *m_cnt;
    const uint64_t *m_obase;
    const uint8_t *m_ovf;
    uint64_t m_ovf_cap;
    // output W'
    uint8_t *o_sf;
    uint32_t *o_pay;
    uint16_t *o_cnt;
    uint64_t *o_obase;
    uint8_t *o_ovf;
    uint64_t ovf_cap;
    uint32_t *status;
    uint8_t *scratch;
    uint64_t n;
    uint32_t block_elems, cap_words, nblk;
    float mul;           // the product's factor: -eta, for W - eta*M
    uint32_t park_cnt;   // the result's counts overwrite W's: park them in scratch
    GroupRef gw, gm;     // used by the group kernels only (W's codes for W and W';
                         // M's for M)
    EncTab wenc;
    DecTab wdec;
    DecTab mdec;
};

// The fused momentum step: W and M decoded, g dense; M' = rne(mu*M + g) and
// W' = rne(W - eta*M') (M' as rounded), both re-encoded in one pass.  Encode
// tables travel packed (stream bits | bit count << 24) to keep the arguments
// small.
struct MomParams {
    const uint8_t *w_sf;
    const uint32_t *w_pay;
    const uint16_t *w_cnt;
    const uint64_t *w_obase;
    const uint8_t *w_ovf;
    uint64_t w_ovf_cap;
    const uint8_t *m_sf;
    const uint32_t *m_pay;
    const uint16_t *m_cnt;
    const uint64_t *m_obase;
    const uint8_t *m_ovf;
    uint64_t m_ovf_cap;
    const uint16_t *g;
    // outputs W' (ow_*) and M' (om_*), each with its own overflow side
    uint8_t *ow_sf;
    uint32_t *ow_pay;
    uint16_t *ow_cnt;
    uint64_t *ow_obase;
    uint8_t *ow_ovf;
    uint64_t ow_ovf_cap;
    uint32_t *ow_status;
    uint8_t *ow_scratch;
    uint8_t *om_sf;
    uint32_t *om_pay;
    uint16_t *om_cnt;
    uint64_t *om_obase;
    uint8_t *om_ovf;
    uint64_t om_ovf_cap;
    uint32_t *om_status;
    uint8_t *om_scratch;
    uint64_t n;
    uint32_t block_elems, cap_words, nblk;
    float mu, neg_eta;
    uint32_t park_w, park_m;   // an output's counts overwrite its input's: park them
    uint32_t pad0;
    GroupRef gw, gm, gg;       // group kernels: W's and M's codes, the gradients' buffers
    uint32_t wenc[256], menc[256];   // packed: bits | len << 24 (W' and M')
    DecTab wdec, mdec;
};

// Shift sample of a compressed tensor: the values at floor(i * n / m), i < m.
struct SampleParams {
    const uint8_t *sf;
    const uint32_t *pay;
    const uint16_t *cnt;
    const uint64_t *obase;
    const uint8_t *ovf;
    uint64_t ovf_cap;
    uint64_t n;
    uint32_t block_elems, cap_words, m, pad0;
    DecTab dec;
};

// Fit of a codebook on the device: the shift of x's sample over the base
// code, the shifted code's tables, and x's record, written as a one-tensor
// group table.
struct FitParams {
    uint16_t *x;
    uint64_t n;
    uint32_t m, nblk;        // sample size min(n, 4096); x's blocks
    uint32_t esc_len, pad0;
    uint8_t base[256];       // base code lengths (0: escaped)
    GroupEntry *ent;
    EncTab *enc;
    DecTab *dec;
    uint32_t *blk_tensor;
    uint32_t *blk_tab;
    int32_t *shift_out;      // may be null
};

// The allocation-free update's static working memory (per device).
constexpr uint64_t kNoAllocScratch = LCT_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
// Device address of the current device's static working memory, looked up
// once per device (hipGetSymbolAddress).  Returns a hipError_t.
int noalloc_scratch(uint8_t **out);

// Host-side launchers (kernels.hip).  Each returns the hipError_t of the launch.
int launch_clear(uint8_t *scratch, uint64_t nblk, uint32_t *status, void *stream);
int launch_scan(uint8_t *scratch, uint64_t nblk, uint64_t *obase, uint8_t *ovf, uint64_t ovf_cap,
                uint32_t *status, uint16_t *cnt, void *stream);
int launch_encode(const EncodeParams &p, void *stream, bool group = false);
int launch_decode(const DecodeParams &p, void *stream, bool group = false);
int launch_sgd(const SgdParams &p, void *stream, bool group = false);
int launch_mom(const MomParams &p, void *stream, bool group = false);
int launch_gather(const uint16_t *x, uint64_t n, uint32_t m, void *stream, uint16_t *host_out);
// The shift sample of a compressed tensor, copied to host_out; synchronises.
int launch_sample(const SampleParams &p, void *stream, uint16_t *host_out);
// The device fit (enqueues only).
int launch_fit(const FitParams &p, void *stream);

// Host codebook construction (codebook.cpp).
// The model's probability of each exponent field (its range of |x|).
void model_pmf(const lct_model &model, double p[256]);
lct_status build_codebook(const lct_model &model, const uint16_t *sample, uint32_t m,
                          lct_codebook *out);
lct_status codebook_from_lengths(const uint8_t len_base[256], uint8_t esc_len, int32_t shift,
                                 lct_codebook *out);
// cb's base code with the shift that minimises the sample's coded bits.
lct_status reshift_codebook(const lct_codebook &cb, const uint16_t *sample, uint32_t m,
                            lct_codebook *out);
// The ranges the kernels rely on hold in cb's lookup tables: an escape code
// of 1..8 bits, every field costing 1..16 bits with no bits past its length,
// every decode entry's length at most 16 (a codebook not made by the
// library, e.g. one left zeroed, fails).
bool tables_ok(const lct_codebook &cb);
void fill_enc(const lct_codebook &cb, EncTab *t);
void fill_enc_packed(const lct_codebook &cb, uint32_t t[256]);
void fill_dec(const lct_codebook &cb, DecTab *t);

}  // namespace lct
