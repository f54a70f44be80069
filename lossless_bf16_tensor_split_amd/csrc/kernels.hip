// kernels.hip -- encode, decode, fused SGD and fused momentum kernels of the
// LCT exponent codec, written for CDNA4 (gfx950, wave64), and the small
// kernels around them (overflow scan and placement, shift sample, device
// codebook fit).
//
// Format (explainer "LCT paper - Lossless Huffman coding of BF16 training
// tensors", paragraphs on bits and on blocks and streams): a BF16 value splits
// into a raw sign-fraction byte and an 8-bit exponent field; exponents are
// coded with a precomputed code of at most 8 bits per field (escaped fields:
// escape code + the 8-bit field); a block is dealt round-robin into 256
// streams of fixed capacity, and the fields that do not fit spill, raw, to an
// overflow region whose start per block is recorded.  The fused SGD kernel
// follows the paragraph on training traffic: read the compressed W and M,
// compute W - eta * M, write the new bytes in one pass.
//
// Mapping.  A "unit" is 64 streams of one block and one wave does it, one
// lane per stream, so at step j lane s touches element j*256 + s of its block
// and a wave's accesses cover contiguous bytes.  The waves of a workgroup
// share the code tables in LDS and nothing else, so no wave ever waits for
// another.  Encode and decode run one unit per wave (a workgroup is a block's
// four units); the fused update's waves are persistent and take units
// round-robin, so its three tables are staged once per workgroup (at the
// CLEAN capacity a block's four units at a time, M's rows through an LDS
// ring); the momentum kernel's persistent workgroups are a block's four units
// at a time and share its four tables.  The updates' blocks that are partial
// or have spilled input fields go to general kernels of their own.  The
// block's stream words are interleaved (word w of stream s at
// w*256 + s): a unit's payload rows move between HBM and LDS with 16-byte
// accesses and every lane works on its own column of the wave's LDS rows
// (a row's lanes hit distinct banks).  Kernels are specialised on the stream
// capacity of the three modes, so row counts and table offsets are constants.
//
// Bit reader: a code starts at stream bit q+2; the two LDS words around q give
// a 32-bit window by one funnel shift (v_alignbit), whose bits 2..9 are the
// 8-bit peek and index the decode table directly as a byte offset.  A table
// entry holds the field (bits 30..23), the bits the code takes (bits 15..8)
// and a shift (bits 4..0) that moves an escape's literal from the window to
// bits 30..23 (31 for ordinary codes, which shifts everything out of that
// range).  Several codes are read from one window; there is no refill logic.
// Row -1 of each input column is zero for the first codes.  (The ring kernel
// reads M through slots of a ring and refills it by halves; a window past
// the rows in the ring is read from memory.)
//
// Bit writer: a 64-bit buffer; after every second code it is stored at the
// current row, and it advances by a word when the first one is full.  The
// encoder's rows are the wave's LDS rows (both words stored, by ds_write2st64,
// so there is no final flush; two sink rows past the stream capacity absorb
// the stores of a full stream), copied out at the unit's end.  The fused
// update writes the first word straight to the payload array through a buffer
// resource spanning the unit's rows (its range check drops the stores of a
// full stream past the last row), stores the last word at the unit's end and
// clears the rows after it; that keeps its LDS to the inputs' rows.  The
// encode table has one 8-byte entry per field: stream bits, bit count.
//
// Overflow offsets: spilled fields are parked per stream in a staging area,
// gathered per unit at its end, then given their offsets by a separate scan
// kernel, an exclusive scan over the units' spill totals with a decoupled
// look-back across its workgroups (Merrill and Garland, "Single-pass Parallel
// Prefix Scan with Decoupled Look-back", 2016), and copied to their place by
// a placing kernel, a wave per unit, so that the fields land in (block,
// stream, position) order.
//
// Every loop step handles 16 positions per lane while the next 16 are loaded
// into a second buffer (two buffers alternate, so loads are waited for one
// step after they were issued).  Full blocks whose inputs carry no spilled
// fields take a path with no overflow reads at all; partial blocks and inputs
// with spills take a general path with per-element checks.  The fused
// update's full-block path moves the sign-fraction bytes through a per-wave
// LDS slab: one 16-byte global access per lane covers 16 positions of 16
// streams, where a lane-per-stream access would move one byte per instruction.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "lct_internal.h"

namespace lct {
namespace {

constexpr uint32_t NS = kStreams;
constexpr uint32_t CH = kChunk;
constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagIncl = 2ull << 62;
constexpr uint64_t kFlagVal = (1ull << 62) - 1;
constexpr uint32_t kSpinLimit = 1u << 21;
// Staging of spilled fields.  In the encoder, with room for every element in
// the overflow region (ovf_cap >= nblk * block_elems), a stream's fields have
// a fixed place in its unit's slice of each staging area (position j of
// stream s of unit u at u * 64 * npos + s * npos + j), so no wave contends
// for a shared counter; otherwise (and in the updates, whose outputs rarely
// spill and whose registers the extra code would cost) space is claimed from
// a counter as streams start to spill.
constexpr uint64_t kClaim = ~0ull;
// A unit's slice of a staging area under fixed staging, or 0 when the
// region is too small for it (space is then claimed).
__device__ __forceinline__ uint64_t fixed_stride(uint64_t nblk, uint32_t block_elems, uint64_t ovf_cap) {
    return nblk * block_elems <= ovf_cap ? (uint64_t)(block_elems / kStreams) * kUnitStreams : 0;
}

// The dynamic LDS region (named only to declare it: the kernels address it
// by byte offset, below).
extern __shared__ uint32_t lds[] __attribute__((unused));

// LDS accessed by byte offset.  These kernels declare no static LDS, so the
// dynamic region starts at LDS address 0 and an offset is an address: the
// accesses take it (plus a constant folded into the instruction) directly.
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x2 lds_u64;
typedef __attribute__((address_space(3))) u32x4 lds_u128;
__device__ __forceinline__ uint32_t ld32(uint32_t off) { return *reinterpret_cast<lds_u32 *>(off); }
__device__ __forceinline__ u32x2 ld64(uint32_t off) { return *reinterpret_cast<lds_u64 *>(off); }
__device__ __forceinline__ u32x4 ld128(uint32_t off) { return *reinterpret_cast<lds_u128 *>(off); }
__device__ __forceinline__ void st128(uint32_t off, u32x4 v) { *reinterpret_cast<lds_u128 *>(off) = v; }
__device__ __forceinline__ void st32(uint32_t off, uint32_t v) { *reinterpret_cast<lds_u32 *>(off) = v; }
// byte 2 of v
__device__ __forceinline__ void st8hi(uint32_t off, uint32_t v) {
    *reinterpret_cast<lds_u8 *>(off) = (uint8_t)(v >> 16);
}
__device__ __forceinline__ void st8(uint32_t off, uint32_t v) {
    *reinterpret_cast<lds_u8 *>(off) = (uint8_t)v;
}

constexpr uint32_t log2c(uint32_t v) { return v <= 1 ? 0 : 1 + log2c(v / 2); }

__device__ __forceinline__ uint32_t lane() { return __lane_id(); }

// True when c holds in every active lane (one ballot compared with exec).
__device__ __forceinline__ bool wave_all(bool c) {
    return __builtin_amdgcn_ballot_w64(c) == __builtin_amdgcn_read_exec();
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t t = __shfl_up(v, d, 64);
        if ((int)lane() >= d) v += t;
    }
    return v;
}

// The wave's minimum of v, in every lane: within each row of 16 lanes by
// shifts of 1, 2, 4 and 8 lanes, then across rows by the broadcasts of
// lanes 15 and 31, which leaves it in lane 63 (a lane whose shift source
// lies outside its row keeps its own value).
__device__ __forceinline__ int32_t wave_min(int32_t v) {
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x111, 0xF, 0xF, false));   // row_shr:1
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x112, 0xF, 0xF, false));   // row_shr:2
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x114, 0xF, 0xF, false));   // row_shr:4
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xF, 0xF, false));   // row_shr:8
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));   // row_bcast:15
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));   // row_bcast:31
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// Decoupled look-back for scan group u, run by one whole wave: publishes the
// group's total, walks back over the predecessors' descriptors 64 at a time
// until an inclusive prefix is found, publishes its own inclusive prefix and
// returns the exclusive one.  Groups come from a ticket counter, so every
// predecessor is already running and never waits on u.  The wait is bounded:
// on time-out the status word records it and the group goes on.
__device__ uint64_t lookback(uint64_t *flags, uint32_t u, uint64_t agg, uint32_t *status) {
    if (u == 0) {
        if (lane() == 0)
            __hip_atomic_store(&flags[0], kFlagIncl | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
    }
    if (lane() == 0)
        __hip_atomic_store(&flags[u], kFlagAgg | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t excl = 0;
    int64_t top = (int64_t)u - 1;
    uint32_t spins = 0;
    while (true) {
        const int64_t idx = top - (int64_t)lane();
        const uint64_t f = idx >= 0 ? __hip_atomic_load(&flags[idx], __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : kFlagIncl;
        const uint64_t st = f >> 62;
        const uint64_t incl = __ballot(st == 2);
        const uint64_t empty = __ballot(st == 0);
        const int first = incl ? __ffsll((unsigned long long)incl) - 1 : 64;
        const uint64_t need = first >= 63 ? ~0ull : ((2ull << first) - 1);
        if (empty & need) {
            if (++spins > kSpinLimit) {
                if (lane() == 0) atomicOr(status, LCT_ST_LOOKBACK);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
            continue;
        }
        excl += wave_sum64((int)lane() <= first ? (f & kFlagVal) : 0);
        if (first < 64) break;
        top -= 64;
    }
    if (lane() == 0)
        __hip_atomic_store(&flags[u], kFlagIncl | (excl + agg), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return excl;
}

__device__ __forceinline__ uint32_t stream_len(uint32_t nb, uint32_t s) {
    return nb > s ? (nb - s + NS - 1) / NS : 0;
}

// Sign-fraction byte of BF16 bits v: sign (bit 15) to bit 7, fraction kept.
__device__ __forceinline__ uint32_t sf_of(uint32_t v) {
    return (v & 0x7Fu) | ((v >> 8) & ~0x7Fu);
}

// fp32 bits of the BF16 value (sf, e): sf copied to bytes 3 and 2, then the
// exponent field (bits 30..23 of e23; its other bits are ignored) inserted.
__device__ __forceinline__ uint32_t join32(uint32_t sf, uint32_t e23) {
    const uint32_t sfx = __builtin_amdgcn_perm(0u, sf, 0x00000C0Cu);
    uint32_t r;
    // one bit-field insert; written out because the compiler otherwise
    // spends a mask and an and-or on it
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(0x7F800000u), "v"(e23), "v"(sfx));
    return r;
}
// The same with the sign-fraction byte as byte s of word w, sel being
// s * 0x01010000 | 0x0C0C.
__device__ __forceinline__ uint32_t join32s(uint32_t w, uint32_t e23, uint32_t sel) {
    const uint32_t sfx = __builtin_amdgcn_perm(0u, w, sel);
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(0x7F800000u), "v"(e23), "v"(sfx));
    return r;
}

// ------------------------------------------------------------------ code tables in LDS

// Decode table at byte offset `tab`, indexed by peek*4 (see the bit reader).
__device__ __forceinline__ void stage_dec(const DecTab &t, uint32_t tab) {
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) {
        const uint32_t d = t.dec[i];
        const bool esc = (d >> 13) & 1u;
        const uint32_t field = esc ? 0u : (d & 0xFFu);
        const uint32_t sh = esc ? 21u - t.esc_len : 31u;
        st32(tab + 4 * i, (field << 23) | (((d >> 8) & 0x1Fu) << 8) | sh);
    }
}

// Encode table at byte offset `tab`: 8-byte entries {stream bits, bit count}.
__device__ __forceinline__ void stage_enc(const EncTab &t, uint32_t tab) {
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) {
        st32(tab + 8 * i, t.bits[i]);
        st32(tab + 8 * i + 4, t.len[i]);
    }
}

// ------------------------------------------------------------------ stream reader

// Rows are one wave's: 64 streams of 4 bytes.
constexpr uint32_t US = kUnitStreams;
constexpr uint32_t ROWB = US * 4;
static_assert(ROWB == 256, "a unit row is 256 bytes: paired LDS accesses step one row per unit");

struct Reader {
    // q: stream bit position of the next code, minus 2, plus 32 times the
    // index of the stream's row 0 in LDS (row0 / ROWB), so that q / 32 is
    // the LDS row to read and q % 32 the bit within it.
    int32_t q;
    uint32_t tcol;   // this lane's byte in a row

    __device__ __forceinline__ static int32_t bias(uint32_t row0) { return (int32_t)(row0 / ROWB) * 32; }
    __device__ __forceinline__ void init(uint32_t row0, uint32_t lane_) {
        q = bias(row0) - 2;
        tcol = 4 * lane_;
    }
    // The 32-bit window at q: stream bits q .. q+31 (the code at bit 2).  Rows
    // -1 and `cap` are zero.
    __device__ __forceinline__ uint32_t window() const {
        const uint32_t off = (((uint32_t)q << 3) & ~(ROWB - 1)) | tcol;
        const uint32_t a = ld32(off), b = ld32(off + ROWB);
        return __builtin_amdgcn_alignbit(b, a, (uint32_t)q);
    }
    // Next exponent field in bits 30..23 of the result (other bits garbage);
    // tab: the decode table.
    __device__ __forceinline__ uint32_t next(uint32_t tab) {
        const uint32_t win = window();
        const uint32_t en = ld32(tab + (win & 0x3FCu));
        q += (en >> 8) & 0xFFu;
        return (win << (en & 31u)) | en;
    }
    // The next N fields from one window: field k is read from the window
    // shifted by the bits of fields 0..k-1.  The window holds 30 bits past the
    // first code, so the results are exact when all N fields (codes and
    // literals) take at most 30 bits together; the bits they take are
    // returned, and a caller that gets more than 30 must decode the same
    // fields again with next().  q is kept at most qmax so that a bad group
    // never addresses past the stream's zero row.
    template <uint32_t N>
    __device__ __forceinline__ uint32_t next_n(uint32_t tab, int32_t qmax, uint32_t (&e23)[N]) {
        const uint32_t win = window();
        uint32_t c = 0;
#pragma unroll
        for (uint32_t k = 0; k < N; ++k) {
            const uint32_t wk = win >> c;
            const uint32_t en = ld32(tab + (wk & 0x3FCu));
            e23[k] = (wk << (en & 31u)) | en;
            c += (en >> 8) & 0xFFu;
        }
        q = min(q + (int32_t)c, qmax);
        return c;
    }
};

// ------------------------------------------------------------------ stream writer
// A buffer resource over `bytes` bytes from p, which must be the same in
// every lane: its registers are taken as the wave's scalars (the compiler
// cannot see that a unit's base is uniform, and a resource in vector
// registers makes every access a loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void *p, uint32_t bytes) {
    // (the builtin returns a signed int: widen each half through uint32_t,
    // or a low half with bit 31 set would fill the high half with ones)
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t s = ((uint64_t)hi << 32) | lo;
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(s), (short)0, (int)bytes, 0x00020000);
}


// Where a writer's rows go.  LdsRows: the wave's LDS rows (ROWB bytes apart),
// both words of the buffer stored at each step (the second is overwritten
// until complete).  PayRows: the unit's rows of the payload array in memory
// (4 * NS bytes apart), through a buffer resource spanning exactly the unit's
// cap rows; only the first word is stored at each step (each word is stored
// again until it is complete, and the last one once more at the end), and a
// store past the last row, left by a full stream, is dropped by the range
// check.
struct LdsRows {
    static constexpr uint32_t kStride = ROWB;
    __device__ __forceinline__ void store(uint32_t woff, uint64_t buf) const {
        st32(woff, (uint32_t)buf);
        st32(woff + ROWB, (uint32_t)(buf >> 32));
    }
};
struct PayRows {
    static constexpr uint32_t kStride = 4 * NS;
    __amdgpu_buffer_rsrc_t r;
    // rows of unit h of block b (cap rows of the payload array)
    __device__ __forceinline__ void init(uint32_t *pay, uint32_t b, uint32_t h, uint32_t cap) {
        r = wave_rsrc(pay + ((uint64_t)b * cap * NS + h * US), (cap - 1) * kStride + 4 * US);
    }
    __device__ __forceinline__ void store(uint32_t woff, uint64_t buf) const {
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)buf, r, woff, 0, 0);
    }
};

template <class Rows>
struct WriterT {
    static constexpr uint32_t kSh = log2c(Rows::kStride) - 5;
    uint64_t buf;     // pending bits, LSB first (< 32 at every store step)
    uint32_t used;    // bits in buf
    uint32_t woff;    // address of the current row of this lane's column
    uint32_t tadj;    // column address >> kSh, so that total() = (woff >> kSh) - tadj + used
    uint32_t live;    // no field has failed to fit yet
    uint32_t cs;      // coded prefix length
    uint32_t claimed; // staging space claimed for the spilled fields
    uint64_t soff;    // start of this stream's spilled fields in the staging area
    uint64_t sbase;   // fixed staging: where the stream's position 0 would go (kClaim: claim space)
    uint32_t slot;    // fixed staging: positions of a stream's place
    Rows rows;

    // row0: address of the output's row 0 (a multiple of the row stride).
    __device__ __forceinline__ void init(uint32_t row0, uint32_t lane_, uint32_t n_s) {
        buf = 0;
        used = 0;
        woff = row0 + 4 * lane_;
        tadj = woff >> kSh;
        live = 1;
        cs = n_s;
        claimed = 0;
        soff = 0;
        sbase = kClaim;
        slot = 0;
    }
    // fixed staging: this lane's stream takes positions [base, base + npos)
    __device__ __forceinline__ void fixed(uint64_t base, uint32_t npos) {
        sbase = base;
        slot = npos;
    }
    __device__ __forceinline__ void put(uint32_t bits, uint32_t len) {
        buf |= (uint64_t)bits << used;
        used += len;
    }
    // Store the buffer at the current row; move on by a word when the first
    // is full.
    __device__ __forceinline__ void flush() {
        rows.store(woff, buf);
        const uint32_t t = used & 32u;
        buf >>= t;
        woff += t << kSh;
        used &= 31u;
    }
    __device__ __forceinline__ uint32_t total() const { return (woff >> kSh) - tadj + used; }
};
using Writer = WriterT<LdsRows>;
using PayWriter = WriterT<PayRows>;

// Code the CH fields at positions j0..j0+CH-1, given as encode-table offsets
// e8[] (8 * field); with CHECKED, positions at or past n_s are absent.  One
// capacity test per step in the common case.  When some lane's stream runs
// out of room in this step, every lane codes the longest prefix of its
// fields that fits (the greedy prefix: the first field that does not fit
// and all after it spill), with the fields past its cut given no bits, so
// that the wave takes one pass of pair puts instead of a test per field.
// Without GREEDY a stream that runs out of room tests its fields one by one
// (fewer registers: the updates, whose outputs rarely run out, take this).
template <bool CHECKED, bool GREEDY, class W>
__device__ __forceinline__ void writer_chunk(W &st, const uint32_t (&e8)[CH], uint32_t j0,
                                             uint32_t n_s, uint32_t capbits, uint32_t etab) {
    uint32_t cb[CH], cl[CH];
#pragma unroll
    for (uint32_t i = 0; i < CH; ++i) {
        const u32x2 c = ld64(etab + e8[i]);
        cb[i] = c.x;
        cl[i] = c.y;
        if (CHECKED && j0 + i >= n_s) {
            cb[i] = 0;
            cl[i] = 0;
        }
    }
    if constexpr (!GREEDY) {
        if (!st.live) return;
        const uint32_t tot = st.total();
        bool fits = tot + CH * 16 <= capbits;
        if (!fits) {
            uint32_t sum = 0;
#pragma unroll
            for (uint32_t i = 0; i < CH; ++i) sum += cl[i];
            fits = tot + sum <= capbits;
        }
        if (fits) {
#pragma unroll
            for (uint32_t k = 0; k < CH; k += 2) {
                st.put(cb[k], cl[k]);
                st.put(cb[k + 1], cl[k + 1]);
                st.flush();
            }
        } else {
#pragma unroll
            for (uint32_t i = 0; i < CH; ++i) {
                if (st.live) {
                    if (st.total() + cl[i] <= capbits) {
                        st.put(cb[i], cl[i]);
                        st.flush();
                    } else {
                        st.live = 0;
                        st.cs = j0 + i;
                    }
                }
            }
        }
        return;
    }
    const bool live = st.live;
    const uint32_t tot = st.total();
    bool fits = tot + CH * 16 <= capbits;
    if (live && !fits) {
        uint32_t sum = 0;
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) sum += cl[i];
        fits = tot + sum <= capbits;
    }
    if (!wave_all(fits || !live)) {
        // cut: the first field whose code does not fit (CH when all do)
        const uint32_t room = capbits - tot;
        uint32_t run = 0, cut = CH;
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) {
            run += cl[i];
            cut = (run > room && cut == CH) ? i : cut;
        }
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) {
            cb[i] = i < cut ? cb[i] : 0u;
            cl[i] = i < cut ? cl[i] : 0u;
        }
        if (live && cut < CH) {
            st.live = 0;
            st.cs = j0 + cut;
        }
    }
    if (live) {
#pragma unroll
        for (uint32_t k = 0; k < CH; k += 2) {
            st.put(cb[k], cl[k]);
            st.put(cb[k + 1], cl[k + 1]);
            st.flush();
        }
    }
}

// Claim staging space for streams that started spilling in this step (one
// atomic per wave), then park this step's N spilled fields (e8[] = 8 * field)
// there.  Every lane of the wave must reach it.
template <bool CHECKED, uint32_t N, class W>
__device__ __forceinline__ void writer_spill(W &st, const uint32_t (&e8)[N], uint32_t j0,
                                             uint32_t n_s, uint64_t *stage_ctr, uint8_t *stage,
                                             uint64_t stage_cap) {
    const bool fresh = !st.live && !st.claimed;
    if (st.sbase != kClaim) {
        // fixed places: the step's N fields go out in one store of N bytes
        // at the stream's position j0 (aligned: j0, the unit's slice and the
        // stream's share of it are multiples of N); the bytes before the
        // stream's cut are never read
        static_assert(N == 4 || N == 16, "one dword or one 16-byte store");
        if (fresh) {
            st.soff = st.sbase + st.cs;
            st.claimed = 1;
        }
        if (!st.live && j0 + N <= st.slot) {
            uint32_t wd[N / 4];
#pragma unroll
            for (uint32_t q = 0; q < N / 4; ++q)
                wd[q] = ((e8[4 * q] >> 3) & 0xFFu) | (((e8[4 * q + 1] >> 3) & 0xFFu) << 8) |
                        (((e8[4 * q + 2] >> 3) & 0xFFu) << 16) | (((e8[4 * q + 3] >> 3) & 0xFFu) << 24);
            uint8_t *at = stage + st.sbase + j0;
            if constexpr (N == 16)
                *reinterpret_cast<u32x4 *>(at) = u32x4{wd[0], wd[1], wd[2], wd[3]};
            else
                *reinterpret_cast<uint32_t *>(at) = wd[0];
        }
        return;
    } else if (__any(fresh)) {
        const uint32_t amt = fresh ? n_s - st.cs : 0;
        const uint32_t inc = wave_incl_scan(amt);
        const uint32_t tot = __shfl(inc, 63, 64);
        unsigned long long base = 0;
        if (lane() == 0) base = atomicAdd((unsigned long long *)stage_ctr, (unsigned long long)tot);
        base = __shfl(base, 0, 64);
        if (fresh) {
            st.soff = base + inc - amt;
            st.claimed = 1;
        }
    }
    if (!st.live) {
#pragma unroll
        for (uint32_t i = 0; i < N; ++i) {
            const uint32_t j = j0 + i;
            if (j >= st.cs && (!CHECKED || j < n_s)) {
                const uint64_t k = st.soff + (j - st.cs);
                if (k < stage_cap) stage[k] = (uint8_t)(e8[i] >> 3);
            }
        }
    }
}

// ------------------------------------------------------------------ units

// Unit u is streams (u % kMaxUnits) * US .. +US of block u / kMaxUnits.
__device__ __forceinline__ uint32_t unit_block(uint32_t u) { return u / kMaxUnits; }
__device__ __forceinline__ uint32_t unit_part(uint32_t u) { return u % kMaxUnits; }

// Wave g of the grid does unit g; persistent waves then take units g + S,
// g + 2S, ... with S the number of waves in the grid (units are alike in
// work, so round-robin spreads them evenly).
__device__ __forceinline__ uint32_t wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ uint32_t first_unit(uint32_t waves) { return blockIdx.x * waves + wave_id(); }


// Copy a unit's payload rows (cap rows of 64 words: cap * 16 pieces of 16
// bytes, piece p of row p / 16) to LDS from row0; with TWO, the rows of a
// second array (pay2) go to row2 as well.  Up to 8 pieces per lane and source
// are loaded before any is stored, so a unit's start waits for memory about
// once.  The loads go through buffer resources spanning the unit's rows; a
// lane past the last piece loads from past the range (nothing, no traffic),
// so no branch splits the loads; only the stores are skipped.
template <bool TWO>
__device__ __forceinline__ void rows_to_lds(const uint32_t *pay, uint32_t row0, const uint32_t *pay2,
                                            uint32_t row2, uint32_t b, uint32_t h, uint32_t cap) {
    const uint32_t np = cap * 16;
    const uint64_t u0 = (uint64_t)b * cap * NS + h * US;
    const uint32_t span = (cap - 1) * 4 * NS + 4 * US;
    const __amdgpu_buffer_rsrc_t r1 = wave_rsrc(pay + u0, span);
    const __amdgpu_buffer_rsrc_t r2 = wave_rsrc((TWO ? pay2 : pay) + u0, span);
    for (uint32_t base = 0; base < np; base += 8 * 64) {
        u32x4 v[8], v2[8];
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) {
            const uint32_t p = base + k * 64 + lane();
            const uint32_t off = p < np ? (p / 16) * (4 * NS) + (p % 16) * 16 : 0x80000000u;
            if (base + k * 64 < np) {
                v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, 0));
                if (TWO) v2[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r2, off, 0, 0));
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) {
            const uint32_t p = base + k * 64 + lane();
            if (p < np) {
                st128(row0 + 16 * p, v[k]);
                if (TWO) st128(row2 + 16 * p, v2[k]);
            }
        }
    }
}

// Spill layout of a block (general paths): this lane's stream's coded count
// and the number of spilled fields of the block's streams before it.
__device__ __forceinline__ void unit_spills(const uint16_t *cnt_b, uint32_t nb, uint32_t h,
                                            uint32_t &c_own, uint32_t &excl) {
    uint32_t before = 0;
    c_own = 0;
    excl = 0;
#pragma unroll
    for (uint32_t k = 0; k < kMaxUnits; ++k) {
        const uint32_t s = k * US + lane();
        const uint32_t n_s = stream_len(nb, s);
        const uint32_t c = min<uint32_t>(cnt_b[s], n_s);
        const uint32_t sp = n_s - c;
        const uint32_t inc = wave_incl_scan(sp);
        if (k < h) before += __shfl(inc, 63, 64);
        if (k == h) {
            c_own = c;
            excl = inc - sp;
        }
    }
    excl += before;
}

// Where a unit's results go.
struct UnitOut {
    uint32_t *pay;       // whole array
    uint16_t *cnt;       // whole array (or the parking area in scratch)
    uint8_t *scratch;
    uint64_t nblk, ovf_cap;
    uint32_t cap, parked;
    uint64_t ustride;    // fixed staging: bytes of a unit's slice (0: claimed)
};

// After a unit's stream loop: its payload rows go out (LdsRows: the wave's
// LDS rows from address row0 are copied; PayRows: the last word is stored
// and the rows after it are cleared); its spilled fields, if any, are gathered from the
// per-stream staging pieces into one piece of the second staging area in
// (stream, position) order; its record says where; then its counts.  The
// overflow offsets are the scan kernel's work, the fields' final places the
// placing kernel's.
template <class Rows>
__device__ __forceinline__ void unit_finish(const WriterT<Rows> &st, uint32_t n_s, uint32_t u, uint32_t b,
                                            uint32_t h, uint32_t row0, const UnitOut &o) {
    const uint32_t l = lane();
    const uint32_t spill = n_s - st.cs;
    const uint32_t inc = wave_incl_scan(spill);
    const uint32_t total = __shfl(inc, 63, 64);
    const uint32_t excl = inc - spill;
    if constexpr (Rows::kStride == ROWB) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(o.pay);
        for (uint32_t p = l; p < o.cap * 16; p += 64)
            dst[(((uint64_t)b * o.cap + p / 16) * NS + h * US) / 4 + p % 16] = ld128(row0 + 16 * p);
    } else {
        st.rows.store(st.woff, st.buf);
        for (uint32_t w = st.woff + Rows::kStride; w < o.cap * Rows::kStride; w += Rows::kStride)
            st.rows.store(w, 0);
    }
    uint64_t base = 0;
    if (total && o.ustride) {
        // fixed places: the unit's slice of the second staging area; the
        // wave copies the piece together, a byte a lane, each destination
        // byte d from the stream s whose range [excl_s, excl_s + spill_s)
        // holds it (the last stream with excl_s <= d, found by halving)
        base = (uint64_t)u * o.ustride;
        const uint8_t *stage = o.scratch + scr_stage_offset(o.nblk);
        uint8_t *stage2 = o.scratch + scr_stage2_offset(o.nblk, o.ovf_cap);
        const uint64_t src = spill ? st.soff : 0;
        for (uint32_t d0 = 0; d0 < total; d0 += 64) {
            const uint32_t d = d0 + l;
            uint32_t sel = 0;
#pragma unroll
            for (uint32_t step = 32; step >= 1; step >>= 1) {
                const uint32_t c = sel + step;
                sel = (uint32_t)__shfl((int)excl, (int)c, 64) <= d ? c : sel;
            }
            const uint64_t from = __shfl(src, (int)sel, 64) + (d - (uint32_t)__shfl((int)excl, (int)sel, 64));
            if (d < total && from < o.ovf_cap && base + d < o.ovf_cap) stage2[base + d] = stage[from];
        }
    } else if (total) {
        unsigned long long t = 0;
        if (l == 0)
            t = atomicAdd(reinterpret_cast<unsigned long long *>(o.scratch + kScrStage2),
                          (unsigned long long)total);
        base = __shfl(t, 0, 64);
        const uint8_t *stage = o.scratch + scr_stage_offset(o.nblk);
        uint8_t *stage2 = o.scratch + scr_stage2_offset(o.nblk, o.ovf_cap);
        // a byte at a time per lane: rare in the updates, whose outputs
        // seldom spill, and cheap in registers there
        for (uint32_t k = 0; k < spill; ++k) {
            const uint64_t from = st.soff + k, to = base + excl + k;
            if (from < o.ovf_cap && to < o.ovf_cap) stage2[to] = stage[from];
        }
    }
    if (l == 0) {
        UnitRec *rec = reinterpret_cast<UnitRec *>(o.scratch + scr_rec_offset(o.nblk));
        rec[u] = UnitRec{base, total, o.parked};
    }
    o.cnt[(uint64_t)b * NS + h * US + l] = (uint16_t)st.cs;
}

// ------------------------------------------------------------------ small kernels

// A scratch header and the status word, cleared by a fill kernel (no
// memset node if a caller captures the call in a graph).
__global__ void k_clear(uint64_t *words, uint64_t nwords, uint32_t *status) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nwords) words[i] = 0;
    if (i == 0) *status = 0u;
}

// Overflow offsets: an exclusive scan of the blocks' spill totals (each the
// sum of its units' records), one block per thread, groups chained by the
// look-back.  Writes obase and flags a too-small overflow region; the
// placing kernel finds a unit's place within its block from the records.
__global__ __launch_bounds__(kScanGroup) void k_scan(uint8_t *scratch, uint64_t nblk, uint64_t *obase,
                                                     uint64_t ovf_cap, uint32_t *status) {
    __shared__ uint32_t s_g;
    __shared__ uint64_t s_wave[kScanGroup / 64], s_excl;
    const uint32_t t = threadIdx.x;
    if (t == 0) s_g = atomicAdd(reinterpret_cast<uint32_t *>(scratch + kScrTicket2), 1u);
    __syncthreads();
    const uint32_t g = s_g;
    // one thread per block: its units' records are contiguous
    const uint64_t b = (uint64_t)g * kScanGroup + t;
    const UnitRec *rec = reinterpret_cast<const UnitRec *>(scratch + scr_rec_offset(nblk));
    uint64_t total = 0;
    uint32_t parked = 0;
    if (b < nblk) {
        UnitRec r[kMaxUnits];
#pragma unroll
        for (uint32_t k = 0; k < kMaxUnits; ++k) r[k] = rec[b * kMaxUnits + k];
#pragma unroll
        for (uint32_t k = 0; k < kMaxUnits; ++k) {
            total += r[k].total;
            parked |= r[k].flags & 1u;
        }
    }
    // group scan of the totals (64-bit sums)
    uint64_t inc = total;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t x = __shfl_up(inc, d, 64);
        if ((int)lane() >= d) inc += x;
    }
    if (lane() == 63) s_wave[t >> 6] = inc;
    __syncthreads();
    uint64_t before = 0, agg = 0;
#pragma unroll
    for (uint32_t k = 0; k < kScanGroup / 64; ++k) {
        before += k < (t >> 6) ? s_wave[k] : 0;
        agg += s_wave[k];
    }
    inc += before;
    if (t < 64) {
        uint64_t *flags = reinterpret_cast<uint64_t *>(scratch + kScrFlags);
        const uint64_t ex = lookback(flags, g, agg, status);
        if (t == 0) s_excl = ex;
    }
    __syncthreads();
    const uint64_t ex = s_excl + inc - total;
    if (b < nblk) obase[b] = ex;
    if (b + 1 == nblk) {
        obase[nblk] = ex + total;
        if (ex + total > ovf_cap) atomicOr(status, LCT_ST_OVF_FULL);
    }
    // parked counts are put in place by the placing kernel: tell it
    if (__any(parked != 0) && lane() == 0)
        atomicOr(reinterpret_cast<uint32_t *>(scratch + kScrParked), 1u);
}

// After the scan: every unit's spilled bytes go from the second staging area
// to the overflow region at its block's offset plus the spills of the block's
// earlier units, and parked counts go in place.  One wave per unit, the
// workgroups taking units round-robin; nothing to do (no spills, nothing
// parked) ends every wave at once.
__global__ __launch_bounds__(256) void k_place(const uint8_t *scratch, uint64_t nblk, const uint64_t *obase,
                                               uint8_t *ovf, uint64_t ovf_cap, uint16_t *cnt) {
    const uint32_t parked = *reinterpret_cast<const uint32_t *>(scratch + kScrParked);
    if (obase[nblk] == 0 && parked == 0) return;
    const uint64_t nunits = nblk * kMaxUnits;
    const UnitRec *rec = reinterpret_cast<const UnitRec *>(scratch + scr_rec_offset(nblk));
    const uint8_t *stage2 = scratch + scr_stage2_offset(nblk, ovf_cap);
    const uint16_t *parked_cnt = reinterpret_cast<const uint16_t *>(scratch + scr_cnt_offset(nblk));
    const uint32_t l = lane();
    for (uint64_t u = (uint64_t)blockIdx.x * 4 + wave_id(); u < nunits; u += (uint64_t)gridDim.x * 4) {
        const UnitRec r = rec[u];
        const uint64_t b = u / kMaxUnits;
        if (r.flags & 1u) {
            const uint64_t at = b * NS + (u % kMaxUnits) * US;
            cnt[at + l] = parked_cnt[at + l];
        }
        if (r.total == 0) continue;
        uint64_t to = obase[b];
        for (uint64_t v = b * kMaxUnits; v < u; ++v) to += rec[v].total;
        for (uint64_t i = l; i < r.total; i += 64)
            if (r.base + i < ovf_cap && to + i < ovf_cap) ovf[to + i] = stage2[r.base + i];
    }
}

__device__ uint16_t g_sample[4096];

__global__ void k_gather(const uint16_t *x, uint64_t n, uint32_t m) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < m) g_sample[i] = x[(uint64_t)i * n / m];
}

// Shift re-estimation sample of a compressed tensor: thread i < m takes
// element floor(i * n / m).  Its stream's words are copied to the thread's
// LDS column first (independent loads, no barrier: a thread reads only its own
// column), then the stream is walked one code at a time up to the element's
// position; a spilled element is read from the overflow region, whose bytes
// are in (block, stream, position) order.  The decode table sits below the
// columns.
constexpr uint32_t kSampleDec = 0, kSampleCols = 1024;

__global__ __launch_bounds__(64) void k_sample(const SampleParams p) {
    for (uint32_t k = threadIdx.x; k < 256; k += 64) st32(kSampleDec + 4 * k, p.dec.dec[k]);
    __syncthreads();
    const uint32_t l = threadIdx.x;
    const uint32_t i = blockIdx.x * 64 + l;
    if (i >= p.m) return;
    const uint64_t r = (uint64_t)i * p.n / p.m;
    const uint64_t b = r / p.block_elems;
    const uint32_t j = (uint32_t)(r - b * p.block_elems);
    const uint32_t s = j % NS, pos = j / NS;
    const uint32_t cap = p.cap_words;
    const uint32_t c = p.cnt[b * NS + s];
    uint32_t e = 0;
    if (pos < c) {
        const uint32_t *col = p.pay + b * cap * NS + s;
        for (uint32_t w = 0; w < cap; ++w) st32(kSampleCols + (w * 64 + l) * 4, col[(size_t)w * NS]);
        uint32_t q = 0;
        for (uint32_t k = 0; k <= pos; ++k) {
            const uint32_t w = q >> 5;
            if (w >= cap) break;     // never for a valid stream: its first c codes fit
            const uint32_t lo = ld32(kSampleCols + (w * 64 + l) * 4);
            const uint32_t hi = w + 1 < cap ? ld32(kSampleCols + ((w + 1) * 64 + l) * 4) : 0u;
            const uint32_t win = (uint32_t)((((uint64_t)hi << 32) | lo) >> (q & 31));
            const uint32_t ent = ld32(kSampleDec + 4 * (win & 0xFFu));
            if (ent & (1u << 14)) break;   // no code word: not a valid stream
            e = (ent & (1u << 13)) ? (win >> p.dec.esc_len) & 0xFFu : ent & 0xFFu;
            q += (ent >> 8) & 0x1Fu;
        }
    } else {
        const uint32_t nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - b * p.block_elems);
        uint64_t k = p.obase[b] + (pos - c);
        for (uint32_t t = 0; t < s; ++t) k += stream_len(nb, t) - p.cnt[b * NS + t];
        e = k < p.ovf_cap ? p.ovf[k] : 0u;
    }
    const uint32_t sf = p.sf[r];
    g_sample[i] = (uint16_t)(((sf & 0x80u) << 8) | (e << 7) | (sf & 0x7Fu));
}

// Codebook fit on the device, for callers that must not wait for it: one
// workgroup takes x's 4096-element sample (positions floor(i * n / m)), costs
// every shift k in -255..255 over the base code (a field e costs base[e - k],
// or the escape plus its 8-bit literal), keeps the cheapest (ties: smaller
// |k|, then negative k), and builds the shifted code's canonical codes
// (RFC 1951 order: by length, then field, the escape last as id 256), its
// encode table and its 8-bit peek decode table, as the host builder does.
__global__ __launch_bounds__(256) void k_fit(const FitParams p) {
    __shared__ uint32_t hist[256], base[256], lenf[256], code[257], cnt[17], key[4], wcount[4];
    __shared__ uint32_t bins[256], syms[256], bylen[257], nbins, nsyms;
    const uint32_t t = threadIdx.x;
    hist[t] = 0;
    base[t] = p.base[t];
    if (t < 17) cnt[t] = 0;   // codes per length in cnt[1..8], first codes in cnt[9..16]
    __syncthreads();
    // the sample's 16 loads per thread all go out before any is counted;
    // the position floor(i * n / m) without a 64-bit division in the usual
    // cases (m = 4096 for n >= 4096, m = n below)
    uint32_t es[16];
    const uint32_t mode = p.m == 4096u ? 0u : p.m == p.n ? 1u : 2u;
#pragma unroll
    for (uint32_t j = 0; j < 16; ++j) {
        const uint32_t i = t + 256 * j;
        const uint64_t at = mode == 0u ? ((uint64_t)i * p.n) >> 12 : mode == 1u ? (uint64_t)i
                                                                                  : (uint64_t)i * p.n / p.m;
        es[j] = i < p.m ? (p.x[at] >> 7) & 0xFFu : 256u;
    }
#pragma unroll
    for (uint32_t j = 0; j < 16; ++j)
        if (es[j] < 256) atomicAdd(&hist[es[j]], 1u);
    __syncthreads();
    // keep the entries t with flag set, in order of t, in out[0..*count)
    auto compact = [&](bool flag, uint32_t value, uint32_t *out, uint32_t *count) {
        const uint64_t m = __ballot(flag);
        const uint32_t l = t & 63, w = t >> 6;
        if (l == 0) wcount[w] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t off = (uint32_t)__popcll(m & ((1ull << l) - 1));
        for (uint32_t v = 0; v < w; ++v) off += wcount[v];
        if (flag) out[off] = value;
        if (t == 0) *count = wcount[0] + wcount[1] + wcount[2] + wcount[3];
        __syncthreads();
    };
    // the sample's fields (few for a tensor the model fits): field | count << 8
    compact(hist[t] != 0, t | (hist[t] << 8), bins, &nbins);
    const uint32_t esc_cost = p.esc_len + 8;
    // cost first, then |k|, then the negative of a pair
    auto key_of = [](uint32_t c, int32_t k) {
        return (c << 10) | ((uint32_t)(k < 0 ? -k : k) << 1) | (k > 0 ? 1u : 0u);
    };
    // Shifts k0 = t - 255 and k1 = t + 1 (t < 255) costed together, eight
    // bins at a time so that the table reads of a batch are in flight at once
    // (a bin past nbins reads as a zero count; j0 + 7 < 256 since j0 <= 248).
    const int32_t k0 = (int32_t)t - 255, k1 = (int32_t)t + 1;
    uint32_t c0 = 0, c1 = 0;
    for (uint32_t j0 = 0; j0 < nbins; j0 += 8) {
        uint32_t v[8];
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) v[i] = j0 + i < nbins ? bins[j0 + i] : 0u;
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) {
            const int32_t x0 = (int32_t)(v[i] & 0xFFu) - k0, x1 = (int32_t)(v[i] & 0xFFu) - k1;
            const uint32_t b0 = (x0 >= 0 && x0 < 256) ? base[x0] : 0u;
            const uint32_t b1 = (x1 >= 0 && x1 < 256) ? base[x1] : 0u;
            c0 += (v[i] >> 8) * (b0 ? b0 : esc_cost);
            c1 += (v[i] >> 8) * (b1 ? b1 : esc_cost);
        }
    }
    uint32_t best = key_of(c0, k0);
    if (t < 255) best = min(best, key_of(c1, k1));
    for (uint32_t o = 32; o > 0; o >>= 1) best = min(best, (uint32_t)__shfl_xor((int)best, (int)o));
    if ((t & 63) == 0) key[t >> 6] = best;
    __syncthreads();
    best = min(min(key[0], key[1]), min(key[2], key[3]));
    const uint32_t mag = (best >> 1) & 511u;
    const int32_t k = (best & 1u) ? (int32_t)mag : -(int32_t)mag;
    // the shifted code: lengths, counts per length, canonical codes
    const int32_t x = (int32_t)t - k;
    const uint32_t L = (x >= 0 && x < 256) ? base[x] : 0u;
    lenf[t] = L;
    if (L) atomicAdd(&cnt[L], 1u);
    if (t == 0) atomicAdd(&cnt[p.esc_len], 1u);
    compact(L != 0, t | (L << 9), syms, &nsyms);      // the coded fields, by field
    if (t == 0) {
        uint32_t c = 0;
        cnt[0] = 0;
        for (uint32_t bits = 1; bits <= 8; ++bits) {
            c = (c + cnt[bits - 1]) << 1;
            cnt[8 + bits] = c;      // first code of each length
        }
    }
    __syncthreads();
    auto first_code = [&](uint32_t len) { return cnt[8 + len]; };
    // a code is its length's first code plus the coded fields before it of
    // that length; the escape comes after every field of its length
    // (eight entries of syms at a time; j0 + 7 < 256 as above)
    {
        uint32_t rank = 0, erank = 0;
        for (uint32_t j0 = 0; j0 < nsyms; j0 += 8) {
#pragma unroll
            for (uint32_t i = 0; i < 8; ++i) {
                const uint32_t v = j0 + i < nsyms ? syms[j0 + i] : 0u;   // length 0: never counted
                rank += (v & 0x1FFu) < t && (v >> 9) == L;
                erank += (v >> 9) == p.esc_len;
            }
        }
        if (L) code[t] = first_code(L) + rank;
        if (t == 0) code[256] = first_code(p.esc_len) + erank;
        // the symbols in canonical order: those of length L (the escape the
        // last of its length) from the number of codes shorter than L
        uint32_t before = 0;
        for (uint32_t b = 1; b < 8; ++b) before += b < L ? cnt[b] : 0u;
        if (L) bylen[before + rank] = t;
        if (t == 0) {
            uint32_t eb = 0;
            for (uint32_t b = 1; b < p.esc_len; ++b) eb += cnt[b];
            bylen[eb + erank] = 256;
        }
    }
    __syncthreads();
    auto rev = [](uint32_t v, uint32_t n) { return __brev(v) >> (32 - n); };
    // encode table: stream bits (code reversed; an escape then the literal)
    if (L) {
        p.enc->bits[t] = rev(code[t], L);
        p.enc->len[t] = (uint8_t)L;
    } else {
        p.enc->bits[t] = rev(code[256], p.esc_len) | (t << p.esc_len);
        p.enc->len[t] = (uint8_t)(p.esc_len + 8);
    }
    // decode table: the symbol whose code the peek t starts with.  The
    // stream holds each code reversed, so the peek's first l bits read
    // backwards are a code of length l when they fall in that length's range
    // of canonical values; the shortest such l is the code (no code is a
    // prefix of another).  Its symbol is bylen[codes shorter than l + offset
    // in the range].
    uint32_t d = (8u << 8) | (1u << 14);
    {
        uint32_t before = 0, found = 0, at = 0, fl = 0;
#pragma unroll
        for (uint32_t l = 1; l <= 8; ++l) {
            const uint32_t c = rev(t & ((1u << l) - 1), l);
            const uint32_t f = first_code(l);
            if (!found && cnt[l] && c >= f && c - f < cnt[l]) {
                found = 1;
                at = before + (c - f);
                fl = l;
            }
            before += cnt[l];
        }
        if (found) {
            const uint32_t s = bylen[at];
            d = s < 256 ? (s | (fl << 8)) : (((fl + 8) << 8) | (1u << 13));
        }
    }
    p.dec->dec[t] = (uint16_t)d;
    if (t == 0) {
        p.dec->esc_len = p.esc_len;
        *p.ent = GroupEntry{p.x, p.n, 0, 0, p.nblk};
        if (p.shift_out) *p.shift_out = k;
    }
    for (uint32_t b = t; b < p.nblk; b += 256) {
        p.blk_tensor[b] = 0;
        p.blk_tab[b] = 0;
    }
}

// ------------------------------------------------------------------ step driver

// Positions [j0, j0+CH) of one lane's stream from base (the lane's position 0,
// positions NS apart); with GUARD, positions at or past n_s read as 0.
// The second half of a chunk is addressed from its own base, so that every
// access's offset fits the instruction's immediate (16 positions of 2-byte
// values span 7.5 KiB).
template <bool GUARD, typename T>
__device__ __forceinline__ void load_chunk(uint32_t (&dst)[CH], const T *base, uint32_t j0,
                                           uint32_t n_s) {
    const T *p = base + (size_t)j0 * NS;
    const T *p2 = p + (CH / 2) * NS;
#pragma unroll
    for (uint32_t i = 0; i < CH; ++i) {
        const T *q = i < CH / 2 ? p + i * NS : p2 + (i - CH / 2) * NS;
        dst[i] = (!GUARD || j0 + i < n_s) ? (uint32_t)*q : 0u;
    }
}

// Runs step(buf, j0) over the positions of a stream, CH at a time, with the
// next step's inputs loaded (load(buf, j0)) while the current one works.  Two
// buffers alternate, so no value is copied between steps and the waits for a
// load fall one step after it was issued.  The load for the step past the end
// re-reads the last step's positions.
template <typename Buf, typename Load, typename Step>
__device__ __forceinline__ void double_buffered(uint32_t npos, Load load, Step step) {
    Buf a, b;
    load(a, 0u);
    for (uint32_t j0 = 0; j0 < npos; j0 += 2 * CH) {
        load(b, min(j0 + CH, npos - CH));
        step(a, j0);
        if (j0 + CH >= npos) break;
        load(a, min(j0 + 2 * CH, npos - CH));
        step(b, j0 + CH);
    }
}

// The same with the loads two chunks ahead (three buffers): a wave's stream
// waits less on memory when few waves share a compute unit (small tensors).
template <typename Buf, typename Load, typename Step>
__device__ __forceinline__ void triple_buffered(uint32_t npos, Load load, Step step) {
    Buf a, b, c;
    load(a, 0u);
    load(b, min(CH, npos - CH));
    for (uint32_t j0 = 0; j0 < npos; j0 += 3 * CH) {
        load(c, min(j0 + 2 * CH, npos - CH));
        step(a, j0);
        if (j0 + CH >= npos) break;
        load(a, min(j0 + 3 * CH, npos - CH));
        step(b, j0 + CH);
        if (j0 + 2 * CH >= npos) break;
        load(b, min(j0 + 4 * CH, npos - CH));
        step(c, j0 + 2 * CH);
    }
}

struct Buf1 {
    uint32_t v[CH];
};
struct Buf2 {
    uint32_t w[CH], m[CH];
};

template <uint32_t CAPT>
__device__ __forceinline__ uint32_t cap_of(uint32_t rt) { return CAPT ? CAPT : rt; }

// ------------------------------------------------------------------ encode

// LDS: encode table, then per wave the output rows (cap + 2 sink rows).
constexpr uint32_t kEncWaves = 4;
constexpr uint32_t kEncTab = 256, kEncWave0 = 2304;
__host__ __device__ constexpr uint32_t enc_wave_bytes(uint32_t cap) { return (cap + 2) * ROWB; }

// One lane's stream of a unit; xu and sfu point at the unit's first element
// (stream 0, position 0) in the values and in the sign-fraction bytes.
template <bool FULL, uint32_t CAPT>
__device__ __forceinline__ void encode_stream(const EncodeParams &p, Writer &st, uint32_t n_s,
                                              const uint16_t *xu, uint8_t *sfu) {
    const uint32_t s = lane();
    const uint32_t npos = p.block_elems / NS;
    const uint32_t capbits = 32 * cap_of<CAPT>(p.cap_words);
    const uint16_t *xs = xu + s;
    uint8_t *sfs = sfu + s;
    uint64_t *stage_ctr = reinterpret_cast<uint64_t *>(p.scratch + kScrStage);
    uint8_t *stage = p.scratch + scr_stage_offset(p.nblk);
    triple_buffered<Buf1>(
        npos, [&](Buf1 &bf, uint32_t j0) { load_chunk<!FULL>(bf.v, xs, j0, n_s); },
        [&](Buf1 &bf, uint32_t j0) {
            uint32_t e[CH];
            uint8_t *o = sfs + (size_t)j0 * NS;
#pragma unroll
            for (uint32_t i = 0; i < CH; ++i) {
                e[i] = (bf.v[i] >> 4) & 0x7F8u;   // 8 * exponent field
                if (FULL || j0 + i < n_s) o[i * NS] = (uint8_t)sf_of(bf.v[i]);
            }
            writer_chunk<!FULL, true>(st, e, j0, n_s, capbits, kEncTab);
            writer_spill<!FULL>(st, e, j0, n_s, stage_ctr, stage, p.ovf_cap);
        });
}

// Where a block's elements live: its values (encode source, decode target),
// the offset of its sign-fraction bytes, and its length.  A flat tensor's
// block b starts at element b * block_elems; in a group, block b belongs to
// tensor blk_tensor[b] and starts (b - blk0) * block_elems into that tensor.
struct BlockSpan {
    uint16_t *dense;
    uint64_t sf0;
    uint32_t nb;
};
__device__ __forceinline__ BlockSpan flat_span(uint16_t *dense, uint64_t n, uint32_t block_elems, uint32_t b) {
    const uint64_t r0 = (uint64_t)b * block_elems;
    return {dense + r0, r0, (uint32_t)min<uint64_t>(block_elems, n - r0)};
}
__device__ __forceinline__ BlockSpan group_span(const GroupRef &g, uint32_t k, uint32_t block_elems, uint32_t b) {
    const GroupEntry e = g.ent[k];
    const uint64_t loc = (uint64_t)(b - e.blk0) * block_elems;
    return {e.dense + loc, e.e0 + loc, (uint32_t)min<uint64_t>(block_elems, e.n - loc)};
}

template <uint32_t CAPT, bool GROUP>
__global__ __launch_bounds__(64 * kEncWaves) void k_encode(const EncodeParams p) {
    const uint32_t u = first_unit(kEncWaves);
    const uint32_t b = unit_block(u), h = unit_part(u);
    // a workgroup is one block, so one tensor of a group
    const uint32_t k = GROUP ? p.grp.blk_tensor[min(b, p.nblk - 1)] : 0u;
    stage_enc(GROUP ? p.grp.enc[k] : p.enc, kEncTab);
    __syncthreads();
    const uint32_t l = lane();
    const uint32_t cap = cap_of<CAPT>(p.cap_words);
    const uint32_t out0 = kEncWave0 + wave_id() * enc_wave_bytes(cap);
    if (u >= p.nblk * kMaxUnits) return;
    for (uint32_t w = 0; w < cap; ++w) st32(out0 + w * ROWB + 4 * l, 0);
    const BlockSpan sp = GROUP ? group_span(p.grp, k, p.block_elems, b)
                               : flat_span(const_cast<uint16_t *>(p.x), p.n, p.block_elems, b);
    const uint32_t nb = sp.nb;
    const uint32_t n_s = stream_len(nb, h * US + l);
    Writer st;
    st.init(out0, l, n_s);
    const uint64_t ustride = fixed_stride(p.nblk, p.block_elems, p.ovf_cap);
    if (ustride) st.fixed((uint64_t)u * ustride + (uint64_t)l * (p.block_elems / NS), p.block_elems / NS);
    if (nb == p.block_elems)
        encode_stream<true, CAPT>(p, st, n_s, sp.dense + h * US, p.sf + sp.sf0 + h * US);
    else
        encode_stream<false, CAPT>(p, st, n_s, sp.dense + h * US, p.sf + sp.sf0 + h * US);
    const UnitOut o{p.pay, p.cnt, p.scratch, p.nblk, p.ovf_cap, cap, 0, ustride};
    unit_finish(st, n_s, u, b, h, out0, o);
}

// ------------------------------------------------------------------ decode

// LDS: decode table, then per wave: zero row -1, rows 0..cap-1, zero row cap.
constexpr uint32_t kDecWaves = 4;
constexpr uint32_t kDecTab = 256, kDecWave0 = 1280;
__host__ __device__ constexpr uint32_t dec_wave_bytes(uint32_t cap) { return (cap + 2) * ROWB; }

template <bool FAST, uint32_t CAPT>
__device__ __forceinline__ void decode_stream(const DecodeParams &p, uint32_t row0, uint32_t n_s,
                                              uint32_t c_s, const uint8_t *sfu, uint16_t *yu,
                                              uint64_t sp0) {
    const uint32_t s = lane();
    const uint32_t npos = p.block_elems / NS;
    const int32_t qmax = Reader::bias(row0) + 32 * (int32_t)cap_of<CAPT>(p.cap_words) - 2;
    const uint8_t *sfs = sfu + s;
    uint16_t *ys = yu + s;
    Reader rd;
    rd.init(row0, s);
    triple_buffered<Buf1>(
        npos, [&](Buf1 &bf, uint32_t j0) { load_chunk<!FAST>(bf.v, sfs, j0, n_s); },
        [&](Buf1 &bf, uint32_t j0) {
            uint16_t *o = ys + (size_t)j0 * NS;
            uint16_t *o2 = o + (CH / 2) * NS;
            auto out = [&](uint32_t i) -> uint16_t & { return i < CH / 2 ? o[i * NS] : o2[(i - CH / 2) * NS]; };
            if (FAST) {
                // four fields per window; a chunk where some window ran out
                // (long escapes) is decoded again one field per window
                const int32_t q0 = rd.q;
                uint32_t cmax = 0;
#pragma unroll
                for (uint32_t g = 0; g < CH; g += 4) {
                    uint32_t e23[4];
                    cmax = max(cmax, rd.next_n<4>(kDecTab, qmax, e23));
#pragma unroll
                    for (uint32_t k = 0; k < 4; ++k)
                        out(g + k) = (uint16_t)(join32(bf.v[g + k], e23[k]) >> 16);
                }
                if (__builtin_expect(!__all(cmax <= 30), 0)) {
                    rd.q = q0;
#pragma unroll
                    for (uint32_t i = 0; i < CH; ++i) {
                        const uint32_t e23 = rd.next(kDecTab);
                        rd.q = min(rd.q, qmax);
                        out(i) = (uint16_t)(join32(bf.v[i], e23) >> 16);
                    }
                }
                return;
            }
            // chunks where no stream of the wave has a spilled field take a
            // copy of the loop with no memory read in it (a read under a
            // per-element branch makes every later element wait for all of
            // the wave's memory operations)
            auto elems = [&](auto SP_) {
                constexpr bool SP = decltype(SP_)::value;
#pragma unroll
                for (uint32_t i = 0; i < CH; ++i) {
                    const uint32_t j = j0 + i;
                    uint32_t e23 = rd.next(kDecTab);
                    rd.q = min(rd.q, qmax);
                    if (SP && j >= c_s && j < n_s) {
                        const uint64_t k = sp0 + (j - c_s);
                        e23 = (k < p.ovf_cap ? (uint32_t)p.ovf[k] : 0u) << 23;
                    }
                    // the BF16 value is the top half of its fp32 form
                    if (j < n_s) out(i) = (uint16_t)(join32(bf.v[i], e23) >> 16);
                }
            };
            if (wave_all(j0 + CH <= c_s || c_s >= n_s))
                elems(std::false_type{});
            else
                elems(std::true_type{});
        });
}

template <uint32_t CAPT, bool GROUP>
__global__ __launch_bounds__(64 * kDecWaves) void k_decode(const DecodeParams p) {
    const uint32_t u = first_unit(kDecWaves);
    const uint32_t b = unit_block(u), h = unit_part(u);
    const uint32_t k = GROUP ? p.grp.blk_tensor[min(b, p.nblk - 1)] : 0u;
    stage_dec(GROUP ? p.grp.dec[k] : p.dec, kDecTab);
    __syncthreads();
    const uint32_t l = lane();
    const uint32_t cap = cap_of<CAPT>(p.cap_words);
    const uint32_t base = kDecWave0 + wave_id() * dec_wave_bytes(cap);
    const uint32_t row0 = base + ROWB;
    st32(base + 4 * l, 0);                      // row -1
    st32(row0 + cap * ROWB + 4 * l, 0);         // row cap
    if (u >= p.nblk * kMaxUnits) return;
    rows_to_lds<false>(p.pay, row0, nullptr, 0, b, h, cap);
    const BlockSpan sp = GROUP ? group_span(p.grp, k, p.block_elems, b)
                               : flat_span(p.y, p.n, p.block_elems, b);
    const uint32_t nb = sp.nb;
    const uint32_t n_s = stream_len(nb, h * US + l);
    const uint64_t ob0 = p.obase[b], ob1 = p.obase[b + 1];
    const uint8_t *sfu = p.sf + sp.sf0 + h * US;
    uint16_t *yu = sp.dense + h * US;
    if (nb == p.block_elems && ob0 == ob1) {
        decode_stream<true, CAPT>(p, row0, n_s, n_s, sfu, yu, 0);
    } else {
        uint32_t c_s, excl;
        unit_spills(p.cnt + (uint64_t)b * NS, nb, h, c_s, excl);
        decode_stream<false, CAPT>(p, row0, n_s, c_s, sfu, yu, ob0 + excl);
    }
}

// ------------------------------------------------------------------ fused SGD

constexpr uint32_t kSgdWaves = 2;
// The general update kernel: a block's four units per workgroup, so that a
// partial block's units walk at once.
constexpr uint32_t kSgdGenWaves = 4;
template <bool GEN> constexpr uint32_t sgd_waves() { return GEN ? kSgdGenWaves : kSgdWaves; }
// Sign-fraction regions of the full-block path: per wave and tensor, two
// regions of one half (CH positions of its 64 streams) each; W's also take
// the result's bytes, written in place.
constexpr uint32_t kRegB = CH * US;
constexpr uint32_t kSlabB = 2 * kRegB;
// LDS: W and M decode tables, the W encode table, then per wave the slabs and
// the rows.
constexpr uint32_t kSgdETab = 0, kSgdNone = 2048, kSgdWTab = 2304, kSgdMTab = 3328, kSgdWave0 = 4352;
// kSgdNone: an encode-table entry of no bits and length 0 (a field that codes
// to nothing), as an offset from kSgdETab
constexpr uint32_t kSgdNoField = kSgdNone - kSgdETab;

// A wave's region (from `base`): the slabs; W's zero row -1 and rows
// 0..cap-1; a zero row (W's row cap and M's row -1); M's rows; a zero row.
// The result's rows are not staged: they go to memory as they fill.
struct SgdLayout {
    uint32_t sw, sm, z0, w0, z1, m0, z2, end;
    __host__ __device__ constexpr SgdLayout(uint32_t cap, uint32_t base)
        : sw(base),
          sm(base + kSlabB),
          z0(base + 2 * kSlabB),
          w0(z0 + ROWB),
          z1(w0 + cap * ROWB),
          m0(z1 + ROWB),
          z2(m0 + cap * ROWB),
          end(z2 + ROWB) {}
};
__host__ __device__ constexpr uint32_t sgd_wave_bytes(uint32_t cap) { return SgdLayout(cap, 0).end; }

// One element: rne_bf16(fmaf(-eta, m, w)) in bits 31..16 of the result (bits
// 15..0 hold rounding garbage); a NaN gives 0x7FC0.
__device__ __forceinline__ uint32_t sgd_round(uint32_t wf, uint32_t mf, float a) {
    const float r = __builtin_fmaf(a, __uint_as_float(mf), __uint_as_float(wf));
    const uint32_t u = __float_as_uint(r);
    const uint32_t R = u + 0x7FFFu + ((u >> 16) & 1u);
    return r != r ? 0x7FC00000u : R;
}

// Sign-fraction byte of the rounded result R in bits 23..16: the sign moves
// from bit 31 to bit 23, the fraction stays in bits 22..16.
__device__ __forceinline__ uint32_t sgd_sf16(uint32_t R) {
    return (R & ~0x00800000u) | ((R >> 8) & 0x00800000u);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even BF16 by the hardware conversion
// (a in bits 15..0, b in bits 31..16).  It agrees with the integer rounding of
// sgd_round for every value but NaN, whose sign and payload it keeps: callers
// check for NaN and take sgd_round where one occurs.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- The update at the CLEAN capacity with three waves per SIMD.
//
// At 25 words a stream, W's and M's rows and the sign-fraction regions take
// 17.6 KB a wave, which leaves room for two waves per SIMD.  The ring kernel
// keeps W's rows whole in LDS (an update in place overwrites them in memory)
// but passes M's, which the update only reads, through a ring of kRing rows:
// slot r % kRing holds row r, and a slot past the last repeats slot 0 so that
// a window's second word never wraps.  At the start of every half the ring
// takes the rows loaded during the previous half, and rows are loaded for
// the slots whose rows lie below the wave's slowest reader.  A window that
// reaches a row not yet in the ring is read from memory instead (rows past
// the last read as zero).  M's sign-fraction bytes take one region.  With the
// tables shared by four waves this is 12 KiB a wave: three waves per SIMD.
constexpr uint32_t kRing = 8;
constexpr uint32_t kRingMask = (kRing * ROWB - 1) & ~(ROWB - 1);
constexpr uint32_t kRingFill = 2;   // rows loaded per half, at most
constexpr uint32_t kRingCap = 25;
constexpr uint32_t kRingWaves = 4;

struct RingLayout {
    uint32_t ring, z0, w0, z1, sw, sm, end;
    __host__ __device__ constexpr RingLayout(uint32_t cap, uint32_t base)
        : ring(base),
          z0(base + (kRing + 1) * ROWB),
          w0(z0 + ROWB),
          z1(w0 + cap * ROWB),
          sw(z1 + ROWB),
          sm(sw + kSlabB),
          end(sm + kRegB) {}
};
// a wave's bytes, a whole number of rings so that every ring is aligned to
// its size (its slots are found by masking)
constexpr uint32_t kRingWaveB = (RingLayout(kRingCap, 0).end + kRing * ROWB - 1) / (kRing * ROWB) * (kRing * ROWB);
// the tables, at the update's offsets from here
constexpr uint32_t kRingTab = kRingWaves * kRingWaveB;
constexpr uint32_t kRingLds = kRingTab + kSgdWave0;
static_assert(kRingLds * 3 <= 160 * 1024, "three four-wave workgroups per CU");

struct RingReader {
    int32_t q;          // stream bit position of the next code, minus 2
    uint32_t tcol;      // the ring's address | this lane's byte in a row
    int32_t hi;         // rows below hi have come in (those at or above the slowest reader's are held)
    int32_t qlim;       // every lane's window is held while q < qlim
    int32_t ncome;      // rows hi .. hi + ncome - 1 are on their way, in rr
    int32_t cap;
    uint32_t rr[kRingFill];
    __amdgpu_buffer_rsrc_t src;   // the unit's rows in memory

    // The ring holds rows 0 .. kRing-2, row -1 (zero) in slot kRing-1 and
    // row 0 again in slot kRing.
    __device__ __forceinline__ void init(uint32_t ring, uint32_t lane_, const uint32_t *rows, uint32_t cap_) {
        q = -2;
        tcol = ring | (4 * lane_);
        hi = kRing - 1;
        qlim = 32 * (hi - 1);
        ncome = 0;
        cap = (int32_t)cap_;
        src = wave_rsrc(rows, (cap_ - 1) * 4 * NS + 4 * US);
#pragma unroll
        for (uint32_t k = 0; k < kRingFill; ++k) rr[k] = 0;
    }
    // this lane's word of row r >= 0 from memory (zero past the last row)
    __device__ __forceinline__ uint32_t word(int32_t r) const {
        return __builtin_amdgcn_raw_buffer_load_b32(src, (uint32_t)r * (4 * NS) + (tcol & (ROWB - 1)), 0, 0);
    }
    __device__ __forceinline__ uint32_t window() const {
        const uint32_t off = (((uint32_t)q << 3) & kRingMask) | tcol;
        uint32_t a, b;
        if (__builtin_expect(wave_all(q < qlim), 1)) {
            a = ld32(off);
            b = ld32(off + ROWB);
        } else {
            const int32_t r = q >> 5;
            a = r < hi ? ld32(off) : word(r);
            b = r + 1 < hi ? ld32(off + ROWB) : word(r + 1);
            // wait for the two loads here (vmcnt(0), other counters left
            // alone), so that the paths join with no load of theirs
            // outstanding; otherwise every window after the join would wait
            // for all of the wave's memory operations
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        return __builtin_amdgcn_alignbit(b, a, (uint32_t)q);
    }
    __device__ __forceinline__ uint32_t next(uint32_t tab) {
        const uint32_t win = window();
        const uint32_t en = ld32(tab + (win & 0x3FCu));
        q += (en >> 8) & 0xFFu;
        return (win << (en & 31u)) | en;
    }
    // The rows that came in go to their slots; then rows are loaded for the
    // slots whose rows every reader has left (row r's slot held row r - kRing).
    __device__ __forceinline__ void refill() {
#pragma unroll
        for (uint32_t k = 0; k < kRingFill; ++k) {
            if ((int32_t)k < ncome) {
                const uint32_t slot = (uint32_t)(hi + (int32_t)k) & (kRing - 1);
                st32(tcol + slot * ROWB, rr[k]);
                if (slot == 0) st32(tcol + kRing * ROWB, rr[k]);
            }
        }
        hi += ncome;
        int32_t lo = wave_min(q >> 5);
        const int32_t n = max(0, min(min((int32_t)kRingFill, lo + (int32_t)kRing - hi), cap + 1 - hi));
#pragma unroll
        for (uint32_t k = 0; k < kRingFill; ++k)
            if ((int32_t)k < n) rr[k] = word(hi + (int32_t)k);
        ncome = n;
        qlim = 32 * (hi - 1);
    }
};

// General path: partial blocks and inputs with spilled fields; byte-wide
// accesses with per-element checks.
template <uint32_t CAPT>
__device__ __forceinline__ void sgd_stream_general(const SgdParams &p, const SgdLayout &lay, PayWriter &st,
                                                   uint32_t n_s, uint32_t cw_s, uint32_t cm_s,
                                                   uint64_t r0, uint64_t wsp, uint64_t msp) {
    const uint32_t s = lane();
    const uint32_t npos = p.block_elems / NS;
    const uint32_t cap = cap_of<CAPT>(p.cap_words);
    const uint32_t capbits = 32 * cap;
    const int32_t qwmax = Reader::bias(lay.w0) + (int32_t)capbits - 2;
    const int32_t qmmax = Reader::bias(lay.m0) + (int32_t)capbits - 2;
    const uint8_t *wsf = p.w_sf + r0 + s;
    const uint8_t *msf = p.m_sf + r0 + s;
    uint8_t *osf = p.o_sf + r0 + s;
    uint64_t *stage_ctr = reinterpret_cast<uint64_t *>(p.scratch + kScrStage);
    uint8_t *stage = p.scratch + scr_stage_offset(p.nblk);
    Reader rw, rm;
    rw.init(lay.w0, s);
    rm.init(lay.m0, s);
    double_buffered<Buf2>(
        npos,
        [&](Buf2 &bf, uint32_t j0) {
            load_chunk<true>(bf.w, wsf, j0, n_s);
            load_chunk<true>(bf.m, msf, j0, n_s);
        },
        [&](Buf2 &bf, uint32_t j0) {
            uint32_t e[CH];
            uint8_t *o = osf + (size_t)j0 * NS;
            // SP: some stream of the wave has a spilled input field in this
            // chunk.  The other chunks (nearly all) take a copy of the loop
            // with no memory read in it: a read under a per-element branch
            // makes every element after it wait for all of the wave's memory
            // operations, the prefetched chunk and the stores included.
            auto elems = [&](auto SP_) {
                constexpr bool SP = decltype(SP_)::value;
#pragma unroll
                for (uint32_t i = 0; i < CH; ++i) {
                    const uint32_t j = j0 + i;
                    uint32_t ew = rw.next(kSgdWTab);
                    rw.q = min(rw.q, qwmax);
                    if (SP && j >= cw_s && j < n_s) {
                        const uint64_t k = wsp + (j - cw_s);
                        ew = (k < p.w_ovf_cap ? (uint32_t)p.w_ovf[k] : 0u) << 23;
                    }
                    uint32_t em = rm.next(kSgdMTab);
                    rm.q = min(rm.q, qmmax);
                    if (SP && j >= cm_s && j < n_s) {
                        const uint64_t k = msp + (j - cm_s);
                        em = (k < p.m_ovf_cap ? (uint32_t)p.m_ovf[k] : 0u) << 23;
                    }
                    const uint32_t R = sgd_round(join32(bf.w[i], ew), join32(bf.m[i], em), p.mul);
                    if (j < n_s) o[i * NS] = (uint8_t)(sgd_sf16(R) >> 16);
                    e[i] = (R >> 20) & 0x7F8u;   // 8 * exponent field
                }
            };
            if (wave_all((j0 + CH <= cw_s || cw_s >= n_s) && (j0 + CH <= cm_s || cm_s >= n_s))) {
                // no spilled field: four fields per window, a group of four
                // positions at a time (a group whose window ran out is
                // decoded again a field per window); fields past a stream's
                // end decode to values that are not stored
#pragma unroll
                for (uint32_t g = 0; g < CH; g += 4) {
                    const int32_t qw0 = rw.q, qm0 = rm.q;
                    uint32_t ew[4], em[4];
                    const uint32_t cw = rw.next_n<4>(kSgdWTab, qwmax, ew);
                    const uint32_t cm = rm.next_n<4>(kSgdMTab, qmmax, em);
                    if (__builtin_expect(!wave_all(max(cw, cm) <= 30), 0)) {
                        rw.q = qw0;
                        rm.q = qm0;
#pragma unroll
                        for (uint32_t k = 0; k < 4; ++k) {
                            ew[k] = rw.next(kSgdWTab);
                            rw.q = min(rw.q, qwmax);
                            em[k] = rm.next(kSgdMTab);
                            rm.q = min(rm.q, qmmax);
                        }
                    }
#pragma unroll
                    for (uint32_t k = 0; k < 4; ++k) {
                        const uint32_t i = g + k;
                        const uint32_t R = sgd_round(join32(bf.w[i], ew[k]), join32(bf.m[i], em[k]), p.mul);
                        if (j0 + i < n_s) o[i * NS] = (uint8_t)(sgd_sf16(R) >> 16);
                        e[i] = (R >> 20) & 0x7F8u;
                    }
                }
            } else {
                elems(std::true_type{});
            }
            writer_chunk<true, false>(st, e, j0, n_s, capbits, kSgdETab);
            writer_spill<true>(st, e, j0, n_s, stage_ctr, stage, p.ovf_cap);
        });
}

// Full-block path (every stream has npos elements and no input field spilled).
//
// One software pipeline over the unit's groups of four positions: stage s
// decodes group s (both readers, four fields per window), does the
// arithmetic of group s-1 and splits its results, and codes the fields of
// group s-2.  Nothing goes back: a group whose window ran out (long escapes)
// is decoded again right after its own decode, and a NaN result, which the
// hardware conversion rounds to the same exponent field as the integer
// rounding, only has its sign-fraction byte made again right after its
// arithmetic; so the writer can follow two groups behind.
//
// The sign-fraction bytes of W and M move through two LDS regions per
// tensor, one per half (16 positions) in turn: lane l carries the 16 bytes of
// position l/4, streams 16*(l%4).. of the unit, with one 16-byte load per
// tensor and half, issued two halves ahead; the result's bytes overwrite W's
// in the region and leave with one 16-byte store, half a half later.
// A half's inputs on their way to LDS: W's sign-fraction bytes and M's.
struct HalfRegs {
    u32x4 w, m;
};

// RING: M's rows come through a ring (the ring kernel's layout, Lay =
// RingLayout, its tables from kRingTab); M's sign-fraction bytes then take
// one region, refilled at the end of each half.  mrows: this unit's row 0 of
// M's payload (ring only).
template <uint32_t CAPT, bool RING, class Lay>
__device__ __forceinline__ void sgd_stream_full(const SgdParams &p, const Lay &lay, PayWriter &st,
                                                uint64_t r0, const uint32_t *mrows) {
    constexpr uint32_t TB = RING ? kRingTab : 0u;
    constexpr uint32_t tabE = TB + kSgdETab, tabW = TB + kSgdWTab, tabM = TB + kSgdMTab;
    const uint32_t l = lane();
    const uint32_t npos = p.block_elems / NS;
    const uint32_t nh = npos / CH;                // halves (the block size is a multiple of 4096)
    const uint32_t cap = cap_of<CAPT>(p.cap_words);
    const uint32_t capbits = 32 * cap;
    const int32_t qwmax = Reader::bias(lay.w0) + (int32_t)capbits - 2;
    int32_t qmmax;
    const uint32_t mine = 16 * l;                 // this lane's 16 bytes of a region
    const uint32_t lw = l & ~3u;                  // its sign-fraction byte's word in a region row
    const uint32_t jsel = (l & 3u) * 0x01010000u | 0x0C0Cu;
    // The unit's sign-fraction bytes of W, M and the result through buffer
    // resources spanning them: 32-bit offsets, and an offset past the range
    // makes a load that returns nothing (no traffic) or a store that is
    // dropped.
    const uint32_t span = (npos - 1) * NS + US;
    const __amdgpu_buffer_rsrc_t rws = wave_rsrc(p.w_sf + r0, span);
    const __amdgpu_buffer_rsrc_t rms = wave_rsrc(p.m_sf + r0, span);
    const __amdgpu_buffer_rsrc_t ros = wave_rsrc(p.o_sf + r0, span);
    constexpr uint32_t kNone = 0x80000000u;
    constexpr uint32_t kHalfB = CH * NS;          // sign-fraction bytes of a half
    const uint32_t g = (l >> 2) * NS + 16 * (l & 3);
    uint64_t *stage_ctr = reinterpret_cast<uint64_t *>(p.scratch + kScrStage);
    uint8_t *stage = p.scratch + scr_stage_offset(p.nblk);
    Reader rw;
    std::conditional_t<RING, RingReader, Reader> rm;
    rw.init(lay.w0, l);
    if constexpr (RING) {
        rm.init(lay.ring, l, mrows, cap);
        qmmax = (int32_t)capbits - 2;
    } else {
        rm.init(lay.m0, l);
        qmmax = Reader::bias(lay.m0) + (int32_t)capbits - 2;
    }

    auto load_w = [&](HalfRegs &r, uint32_t h) {
        const uint32_t o = h < nh ? h * kHalfB + g : kNone;
        r.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rws, o, 0, 0));
    };
    auto load_m = [&](HalfRegs &r, uint32_t h) {
        const uint32_t o = h < nh ? h * kHalfB + g : kNone;
        r.m = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rms, o, 0, 0));
    };
    auto region = [&](uint32_t h) { return (h & 1u) * kRegB; };
    // M's region of half h (one region in turn with the ring)
    auto region_m = [&](uint32_t h) { return RING ? 0u : region(h); };
    // a half's inputs into the regions of half h
    auto to_lds_w = [&](const HalfRegs &r, uint32_t h) { st128(lay.sw + region(h) + mine, r.w); };
    auto to_lds_m = [&](const HalfRegs &r, uint32_t h) { st128(lay.sm + region_m(h) + mine, r.m); };

    // Carried from stage to stage: the inputs of the group whose arithmetic
    // comes next (sign-fraction words and decoded fields), the codes (and
    // fields) of the group the writer codes next, the result bytes of the
    // half that leaves next.  Before the first group they stand for a group
    // that codes to nothing.
    uint32_t wsP[4] = {0, 0, 0, 0}, msP[4] = {0, 0, 0, 0}, ewP[4] = {0, 0, 0, 0}, emP[4] = {0, 0, 0, 0};
    u32x2 wc[4] = {{0u, 0u}, {0u, 0u}, {0u, 0u}, {0u, 0u}};
    uint32_t ew8[4] = {kSgdNoField, kSgdNoField, kSgdNoField, kSgdNoField};
    uint32_t jw = 0;                              // position of the writer's group
    u32x4 outv = {0u, 0u, 0u, 0u};
    bool wall = true;

    // The writer's group coded with a check per field (a stream near its end
    // may run out of room); its codes are then spent.
    auto code_checked = [&]() {
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            if (st.live) {
                if (st.total() + wc[k].y <= capbits) {
                    st.put(wc[k].x, wc[k].y);
                    st.flush();
                } else {
                    st.live = 0;
                    st.cs = jw + k;
                }
            }
            wc[k] = u32x2{0u, 0u};
        }
        writer_spill<false>(st, ew8, jw, npos, stage_ctr, stage, p.ovf_cap);
    };

    // One stage.  DEC: group s exists (decode it).  GS = s % 4; h = s / 4.
    // The arithmetic is for group s-1 (in half (s-1)/4, region of that half),
    // the writer codes group s-2 (its codes in wc, fields in ew8, positions
    // jw..).
    auto stage_fn = [&](auto DEC_, auto GS_, uint32_t h) {
        constexpr bool DEC = decltype(DEC_)::value;
        constexpr uint32_t GS = decltype(GS_)::value;
        const uint32_t rc = region(h) + GS * 4 * US;                       // group s's rows
        const uint32_t rcm = region_m(h) + GS * 4 * US;
        const uint32_t rp = (GS ? region(h) : region(h + 1)) + ((GS + 3) % 4) * 4 * US;   // group s-1's rows
        uint32_t wsC[4], msC[4], ewC[4], emC[4];
        uint32_t winw = 0, winm = 0, cw = 0, cm = 0;
        const int32_t qw0 = rw.q, qm0 = rm.q;
        if (DEC) {
            winw = rw.window();
            winm = rm.window();
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                wsC[k] = ld32(lay.sw + rc + k * US + lw);
                msC[k] = ld32(lay.sm + rcm + k * US + lw);
            }
        }
        // the writer's group, with checks when some stream is near its end
        if (!wall && !__all(st.live && st.total() + 4 * 16 <= capbits)) code_checked();
        uint32_t ep[4];
        float r[4];
        bool nan = false;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            uint32_t enw = 0, enm = 0, wkw = 0, wkm = 0;
            if (DEC) {
                wkw = winw >> cw;
                enw = ld32(tabW + (wkw & 0x3FCu));
                wkm = winm >> cm;
                enm = ld32(tabM + (wkm & 0x3FCu));
            }
            r[k] = __builtin_fmaf(p.mul, __uint_as_float(join32s(msP[k], emP[k], jsel)),
                                  __uint_as_float(join32s(wsP[k], ewP[k], jsel)));
            nan |= r[k] != r[k];
            if (k & 1) {
                uint32_t hh = cvt_bf16x2(r[k - 1], r[k]);
                asm volatile("" : "+v"(hh));
                ep[k - 1] = (hh >> 4) & 0x7F8u;
                ep[k] = (hh >> 20) & 0x7F8u;
                uint32_t b;
                asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b) : "s"(0x00800080u), "v"(hh >> 8), "v"(hh));
                st8(lay.sw + rp + (k - 1) * US + l, b);
                st8hi(lay.sw + rp + k * US + l, b);
                // a pair of codes (at most 16 bits each) as one put
                st.put(wc[k - 1].x | (wc[k].x << wc[k - 1].y), wc[k - 1].y + wc[k].y);
                st.flush();
            }
            if (DEC) {
                ewC[k] = (wkw << (enw & 31u)) | enw;
                cw += (enw >> 8) & 0xFFu;
                emC[k] = (wkm << (enm & 31u)) | enm;
                cm += (enm >> 8) & 0xFFu;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // All fields of a full block are valid: a window that held its four
        // fields moves the reader at most to the stream's end, so no clamp is
        // needed here; a window that ran out is decoded again (with clamps).
        if (DEC) {
            rw.q += (int32_t)cw;
            rm.q += (int32_t)cm;
        }
        if (__builtin_expect(!wave_all((!DEC || max(cw, cm) <= 30) && !nan), 0)) {
            if (DEC && !wave_all(max(cw, cm) <= 30)) {
                // a window ran out: group s again, one field per window
                rw.q = qw0;
                rm.q = qm0;
#pragma unroll
                for (uint32_t k = 0; k < 4; ++k) {
                    ewC[k] = rw.next(tabW);
                    rw.q = min(rw.q, qwmax);
                    emC[k] = rm.next(tabM);
                    rm.q = min(rm.q, qmmax);
                }
            }
            // group s-1 with the integer rounding (same fields; a NaN's byte
            // becomes the canonical one's)
#pragma unroll
            for (uint32_t k = 0; k < 4; k += 2) {
                const uint32_t R0 =
                    sgd_round(join32s(wsP[k], ewP[k], jsel), join32s(msP[k], emP[k], jsel), p.mul);
                const uint32_t R1 = sgd_round(join32s(wsP[k + 1], ewP[k + 1], jsel),
                                              join32s(msP[k + 1], emP[k + 1], jsel), p.mul);
                const uint32_t hh = (R0 >> 16) | (R1 & 0xFFFF0000u);
                ep[k] = (hh >> 4) & 0x7F8u;
                ep[k + 1] = (hh >> 20) & 0x7F8u;
                uint32_t b;
                asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b) : "s"(0x00800080u), "v"(hh >> 8), "v"(hh));
                st8(lay.sw + rp + k * US + l, b);
                st8hi(lay.sw + rp + (k + 1) * US + l, b);
            }
        }
        // the writer codes group s-1 next stage
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            wc[k] = ld64(tabE + ep[k]);
            ew8[k] = ep[k];
        }
        jw = 4 * (4 * h + GS) - 4;
        if (DEC) {
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                wsP[k] = wsC[k];
                msP[k] = msC[k];
                ewP[k] = ewC[k];
                emP[k] = emC[k];
            }
        }
    };
    // Half h: its four stages.  At the end of its first stage the last group
    // of half h-1 has been split: that half's bytes are read out, its region
    // takes half h+1 (loaded two halves earlier into `next`), and the loads
    // of half h+3 go out into the same registers.  Half h-1's bytes leave in
    // the third stage.  With the ring, M's one region takes half h+1 after
    // the half's last stage (which read the last of half h), and the ring
    // takes the rows that came in during the previous half first.
    auto half = [&](uint32_t h, HalfRegs &next) {
        if constexpr (RING) rm.refill();
        wall = __all(st.live && st.total() + CH * 16 <= capbits);
        stage_fn(std::true_type{}, std::integral_constant<uint32_t, 0>{}, h);
        if (h == 0) {
            // the group before the first codes to nothing
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                wc[k] = u32x2{0u, 0u};
                ew8[k] = kSgdNoField;
            }
            jw = 0;
        } else {
            outv = ld128(lay.sw + region(h - 1) + mine);
        }
        to_lds_w(next, h + 1);
        load_w(next, h + 3);
        if (!RING) {
            to_lds_m(next, h + 1);
            load_m(next, h + 3);
        }
        stage_fn(std::true_type{}, std::integral_constant<uint32_t, 1>{}, h);
        if (h != 0) __builtin_amdgcn_raw_buffer_store_b128(outv, ros, (h - 1) * kHalfB + g, 0, 0);
        stage_fn(std::true_type{}, std::integral_constant<uint32_t, 2>{}, h);
        stage_fn(std::true_type{}, std::integral_constant<uint32_t, 3>{}, h);
        if (RING) {
            to_lds_m(next, h + 1);
            load_m(next, h + 3);
        }
    };
    HalfRegs a, b;
    load_w(a, 0);
    load_m(a, 0);
    load_w(b, 1);
    load_m(b, 1);
    to_lds_w(a, 0);
    to_lds_m(a, 0);
    load_w(a, 2);
    load_m(a, 2);
    for (uint32_t h = 0; h < nh; h += 2) {
        half(h, b);
        if (h + 1 < nh) half(h + 1, a);
    }
    // the last group's arithmetic, the writer's last two groups, the last
    // half's bytes
    wall = false;
    stage_fn(std::false_type{}, std::integral_constant<uint32_t, 0>{}, nh);
    code_checked();
    outv = ld128(lay.sw + region(nh - 1) + mine);
    __builtin_amdgcn_raw_buffer_store_b128(outv, ros, (nh - 1) * kHalfB + g, 0, 0);
}

// A block takes the full-block path when it is whole and neither input has
// a spilled field in it.  The update and the momentum step run that path and
// the general one in kernels of their own (the general path's registers
// would otherwise set the budget of the common one): the first skips the
// other blocks, the second finds them with one test per lane for 64 blocks
// at a time and does only those.
template <bool GROUP, class P>
__device__ __forceinline__ uint32_t block_len(const P &p, uint32_t b) {
    if (GROUP) return group_span(p.gw, p.gw.blk_tensor[b], p.block_elems, b).nb;
    return (uint32_t)min<uint64_t>(p.block_elems, p.n - (uint64_t)b * p.block_elems);
}
template <class P>
__device__ __forceinline__ bool block_full(const P &p, uint32_t b, uint32_t nb, uint64_t wob, uint64_t wob1,
                                           uint64_t mob, uint64_t mob1) {
    return nb == p.block_elems && wob == wob1 && mob == mob1;
}
// The general kernel's walk: f(i) for every i < count taken by this
// workgroup (i = blockIdx.x, + gridDim.x, ...) whose block is not full;
// blk(i) names i's block.  Every wave of the workgroup takes the same i in
// the same order.
template <bool GROUP, class P, class Blk, class F>
__device__ __forceinline__ void for_general(const P &p, uint32_t count, Blk blk, F f) {
    const uint32_t G = gridDim.x;
    for (uint64_t base = blockIdx.x; base < count; base += 64ull * G) {
        const uint64_t i = base + (uint64_t)lane() * G;
        bool gen = false;
        if (i < count) {
            const uint32_t b = blk((uint32_t)i);
            gen = !block_full(p, b, block_len<GROUP>(p, b), p.w_obase[b], p.w_obase[b + 1], p.m_obase[b],
                              p.m_obase[b + 1]);
        }
        for (uint64_t mask = __ballot(gen); mask; mask &= mask - 1)
            f((uint32_t)(base + (uint64_t)__builtin_ctzll(mask) * G));
    }
}

// At least two waves per SIMD (at most 256 registers a lane, AGPRs
// included); the full-block kernel of the MEDIUM and HIGH capacities needs
// about 150, so LDS lets three share a SIMD.  GEN: the general kernel
// (blocks that are not full); otherwise the full-block kernel (the CLEAN
// capacity's is the ring kernel).
template <uint32_t CAPT, bool GROUP, bool GEN>
__global__ __launch_bounds__(64 * sgd_waves<GEN>()) __attribute__((amdgpu_waves_per_eu(2)))
void k_sgd(const SgdParams p) {
    if (!GROUP) {
        stage_dec(p.wdec, kSgdWTab);
        stage_dec(p.mdec, kSgdMTab);
        stage_enc(p.wenc, kSgdETab);
    }
    if (threadIdx.x < 2) st32(kSgdNone + 4 * threadIdx.x, 0);
    __syncthreads();
    uint64_t staged = ~0ull;   // the group tables in LDS: W's (and W''s) and M's, as table indices
    const uint32_t l = lane();
    const uint32_t cap = cap_of<CAPT>(p.cap_words);
    const SgdLayout lay(cap, kSgdWave0 + wave_id() * sgd_wave_bytes(cap));
    st32(lay.z0 + 4 * l, 0);
    st32(lay.z1 + 4 * l, 0);
    st32(lay.z2 + 4 * l, 0);
    const uint32_t nunits = p.nblk * kMaxUnits;
    uint16_t *cnt_out = p.park_cnt ? reinterpret_cast<uint16_t *>(p.scratch + scr_cnt_offset(p.nblk))
                                   : p.o_cnt;
    // The two waves of a workgroup take units 2i and 2i+1 of one block, whose
    // sign-fraction bytes share every 128-byte line (the general kernel's four
    // waves a block's four units).  Left free, the waves drift apart over many
    // units and the second read of a line misses L2, so they meet at the
    // start of each unit (an execution barrier only: they share no data).
    // All take the same number of trips, the unit count being even.
    static_assert(kSgdWaves == 2 && kMaxUnits % kSgdWaves == 0 && kSgdGenWaves == kMaxUnits,
                  "pairs of units per workgroup; the general kernel's: a block's units");
    uint32_t nfull = 0;   // units done on the full-block path
    // One unit (the full-block kernel leaves the others to the general one).
    auto unit = [&](uint32_t u) {
        __builtin_amdgcn_s_barrier();
        const uint32_t b = unit_block(u), h = unit_part(u);
        uint32_t k = 0;
        if (GROUP) {
            // both waves work on one block, so on one tensor; the barrier
            // above means neither still reads the tables being replaced.
            // Tensors with identical tables share an index: a pair that moves
            // to another tensor stages tables only when they differ.
            k = p.gw.blk_tensor[b];
            const uint32_t tw = p.gw.blk_tab[b], tm = p.gm.blk_tab[b];
            const uint64_t key = ((uint64_t)tm << 32) | tw;
            if (key != staged) {
                stage_dec(p.gw.dec[tw], kSgdWTab);
                stage_dec(p.gm.dec[tm], kSgdMTab);
                stage_enc(p.gw.enc[tw], kSgdETab);
                __syncthreads();
                staged = key;
            }
        }
        // the block's overflow offsets are read along with the rows (one
        // memory round trip for both)
        const uint64_t wob = p.w_obase[b], wob1 = p.w_obase[b + 1];
        const uint64_t mob = p.m_obase[b], mob1 = p.m_obase[b + 1];
        rows_to_lds<true>(p.w_pay, lay.w0, p.m_pay, lay.m0, b, h, cap);
        uint64_t r0;
        uint32_t nb;
        if (GROUP) {
            const BlockSpan sp = group_span(p.gw, k, p.block_elems, b);
            r0 = sp.sf0;
            nb = sp.nb;
        } else {
            r0 = (uint64_t)b * p.block_elems;
            nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
        }
        if (!GEN && !block_full(p, b, nb, wob, wob1, mob, mob1)) return;
        const uint32_t n_s = stream_len(nb, h * US + l);
        // The result's rows go straight to memory: W's rows, which an update
        // in place overwrites, are all in LDS by now.
        PayWriter st;
        st.init(0, l, n_s);
        st.rows.init(p.o_pay, b, h, cap);
        if (!GEN) {
            sgd_stream_full<CAPT, false>(p, lay, st, r0 + h * US, nullptr);
            ++nfull;
            const UnitOut o{p.o_pay, p.o_cnt, p.scratch, p.nblk, p.ovf_cap, cap, 0, 0};
            unit_finish(st, n_s, u, b, h, 0, o);
        } else {
            uint32_t cw_s, cm_s, wex, mex;
            unit_spills(p.w_cnt + (uint64_t)b * NS, nb, h, cw_s, wex);
            unit_spills(p.m_cnt + (uint64_t)b * NS, nb, h, cm_s, mex);
            sgd_stream_general<CAPT>(p, lay, st, n_s, cw_s, cm_s, r0 + h * US, wob + wex, mob + mex);
            // The result's counts overwrite W's when the update is in place:
            // other units of this block may still read W's, so they are
            // parked and put in place by the placing kernel.  (The
            // full-block kernel reads no counts.)
            const UnitOut o{p.o_pay, cnt_out, p.scratch, p.nblk, p.ovf_cap, cap, p.park_cnt, 0};
            unit_finish(st, n_s, u, b, h, 0, o);
        }
    };
    if (!GEN) {
        const uint32_t stride = gridDim.x * kSgdWaves;
        for (uint32_t u = first_unit(kSgdWaves); u < nunits; u += stride) unit(u);
        if (l == 0 && nfull) atomicAdd(reinterpret_cast<uint32_t *>(p.scratch + kScrFullUnits), nfull);
    } else {
        for_general<GROUP>(p, p.nblk, [](uint32_t i) { return i; },
                           [&](uint32_t b) { unit(kMaxUnits * b + wave_id()); });
    }
}

// W's rows (cap) and M's first kRing-1 rows into the ring kernel's LDS with
// one wait: row 0 goes to the ring's last slot too, and the slot before it
// (row -1) is cleared.
__device__ __forceinline__ void rows_ring_to_lds(const uint32_t *wpay, const uint32_t *mpay, const RingLayout &lay,
                                                 uint32_t b, uint32_t h) {
    constexpr uint32_t np = kRingCap * 16, nr = (kRing - 1) * 16;
    constexpr uint32_t kw = (np + 63) / 64, km = (nr + 63) / 64;
    const uint64_t u0 = (uint64_t)b * kRingCap * NS + h * US;
    const uint32_t span = (kRingCap - 1) * 4 * NS + 4 * US;
    const __amdgpu_buffer_rsrc_t rw = wave_rsrc(wpay + u0, span);
    const __amdgpu_buffer_rsrc_t rm = wave_rsrc(mpay + u0, span);
    u32x4 v[kw], m[km];
#pragma unroll
    for (uint32_t k = 0; k < kw; ++k) {
        const uint32_t p = k * 64 + lane();
        const uint32_t off = p < np ? (p / 16) * (4 * NS) + (p % 16) * 16 : 0x80000000u;
        v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
    }
#pragma unroll
    for (uint32_t k = 0; k < km; ++k) {
        const uint32_t p = k * 64 + lane();
        const uint32_t off = p < nr ? (p / 16) * (4 * NS) + (p % 16) * 16 : 0x80000000u;
        m[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rm, off, 0, 0));
    }
#pragma unroll
    for (uint32_t k = 0; k < kw; ++k) {
        const uint32_t p = k * 64 + lane();
        if (p < np) st128(lay.w0 + 16 * p, v[k]);
    }
#pragma unroll
    for (uint32_t k = 0; k < km; ++k) {
        const uint32_t p = k * 64 + lane();
        if (p < nr) st128(lay.ring + 16 * p, m[k]);
        if (p < 16) st128(lay.ring + kRing * ROWB + 16 * p, m[k]);
    }
    st32(lay.ring + (kRing - 1) * ROWB + 4 * lane(), 0);
}

// The full-block update at the CLEAN capacity: four waves, one block's
// units, per workgroup (they share the tables and meet at every block),
// three waves per SIMD.  Blocks that are not full are left to the general
// kernel.
template <bool GROUP>
__global__ __launch_bounds__(64 * kRingWaves) __attribute__((amdgpu_waves_per_eu(3)))
void k_sgd_ring(const SgdParams p) {
    constexpr uint32_t cap = kRingCap;
    if (!GROUP) {
        stage_dec(p.wdec, kRingTab + kSgdWTab);
        stage_dec(p.mdec, kRingTab + kSgdMTab);
        stage_enc(p.wenc, kRingTab + kSgdETab);
    }
    if (threadIdx.x < 2) st32(kRingTab + kSgdNone + 4 * threadIdx.x, 0);
    __syncthreads();
    uint64_t staged = ~0ull;
    const uint32_t l = lane(), h = wave_id();
    const RingLayout lay(cap, h * kRingWaveB);
    st32(lay.z0 + 4 * l, 0);
    st32(lay.z1 + 4 * l, 0);
    static_assert(kRingWaves == kMaxUnits, "a workgroup is one block's units");
    uint32_t nfull = 0;
    for (uint32_t b = blockIdx.x; b < p.nblk; b += gridDim.x) {
        __builtin_amdgcn_s_barrier();
        uint32_t k = 0;
        if (GROUP) {
            k = p.gw.blk_tensor[b];
            const uint32_t tw = p.gw.blk_tab[b], tm = p.gm.blk_tab[b];
            const uint64_t key = ((uint64_t)tm << 32) | tw;
            if (key != staged) {
                stage_dec(p.gw.dec[tw], kRingTab + kSgdWTab);
                stage_dec(p.gm.dec[tm], kRingTab + kSgdMTab);
                stage_enc(p.gw.enc[tw], kRingTab + kSgdETab);
                __syncthreads();
                staged = key;
            }
        }
        const uint64_t wob = p.w_obase[b], wob1 = p.w_obase[b + 1];
        const uint64_t mob = p.m_obase[b], mob1 = p.m_obase[b + 1];
        rows_ring_to_lds(p.w_pay, p.m_pay, lay, b, h);
        uint64_t r0;
        uint32_t nb;
        if (GROUP) {
            const BlockSpan sp = group_span(p.gw, k, p.block_elems, b);
            r0 = sp.sf0;
            nb = sp.nb;
        } else {
            r0 = (uint64_t)b * p.block_elems;
            nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
        }
        if (!block_full(p, b, nb, wob, wob1, mob, mob1)) continue;
        const uint32_t n_s = stream_len(nb, h * US + l);
        PayWriter st;
        st.init(0, l, n_s);
        st.rows.init(p.o_pay, b, h, cap);
        sgd_stream_full<cap, true>(p, lay, st, r0 + h * US, p.m_pay + ((uint64_t)b * cap * NS + h * US));
        ++nfull;
        const UnitOut o{p.o_pay, p.o_cnt, p.scratch, p.nblk, p.ovf_cap, cap, 0, 0};
        unit_finish(st, n_s, b * kMaxUnits + h, b, h, 0, o);
    }
    if (l == 0 && nfull) atomicAdd(reinterpret_cast<uint32_t *>(p.scratch + kScrFullUnits), nfull);
}

// ------------------------------------------------------------------ fused momentum step

// One pass for the momentum step (explainer, jargon entry "Optimizer state":
// the momentum buffer is kept compressed like the weights; paragraph on
// training traffic: decode, update and re-encode in one pass): W and M are
// decoded, g is read dense, and per element m' = rne(fmaf(mu, m, g)) and
// w' = rne(fmaf(-eta, m', w)) with m' as rounded, each NaN written as 0x7FC0;
// M' is coded with M's output code and W' with W's, each by its own writer
// into its own output.  The update's pipeline carries both: stage s decodes
// group s of W and M (and loads its g values), does both products of group
// s-1 and splits both results, and codes both outputs' fields of group s-2.
// M''s sign-fraction bytes take the place of M's in M's LDS regions, W''s
// those of W, and each leaves with its own 16-byte stores.
//
// Four waves per workgroup, the four units of a block, share the four code
// tables (two waves per SIMD, eight per CU); units 2i and 2i+1 share their
// sign-fraction lines, so the workgroup meets at every block.
constexpr uint32_t kMomWaves = 4;
constexpr uint32_t kMWE = 0, kMME = 2048, kMNone = 4096, kMWD = 4352, kMMD = 5376, kMWave0 = 6400;
constexpr uint32_t kMWNoField = kMNone - kMWE, kMMNoField = kMNone - kMME;

// Encode table from its packed form (bits | len << 24) into 8-byte entries.
__device__ __forceinline__ void stage_enc_packed(const uint32_t *t, uint32_t tab) {
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) {
        const uint32_t e = t[i];
        st32(tab + 8 * i, e & 0xFFFFFFu);
        st32(tab + 8 * i + 4, e >> 24);
    }
}

// General path (partial blocks and inputs with spilled fields): byte-wide
// accesses with per-element checks.
template <uint32_t CAPT>
__device__ __forceinline__ void mom_stream_general(const MomParams &p, const SgdLayout &lay, PayWriter &stw,
                                                   PayWriter &stm, uint32_t n_s, uint32_t cw_s, uint32_t cm_s,
                                                   uint64_t r0, const uint16_t *gu, uint64_t wsp, uint64_t msp) {
    const uint32_t s = lane();
    const uint32_t npos = p.block_elems / NS;
    const uint32_t cap = cap_of<CAPT>(p.cap_words);
    const uint32_t capbits = 32 * cap;
    const int32_t qwmax = Reader::bias(lay.w0) + (int32_t)capbits - 2;
    const int32_t qmmax = Reader::bias(lay.m0) + (int32_t)capbits - 2;
    const uint8_t *wsf = p.w_sf + r0 + s;
    const uint8_t *msf = p.m_sf + r0 + s;
    const uint16_t *gs = gu + s;
    uint8_t *owsf = p.ow_sf + r0 + s;
    uint8_t *omsf = p.om_sf + r0 + s;
    uint64_t *wctr = reinterpret_cast<uint64_t *>(p.ow_scratch + kScrStage);
    uint8_t *wstage = p.ow_scratch + scr_stage_offset(p.nblk);
    uint64_t *mctr = reinterpret_cast<uint64_t *>(p.om_scratch + kScrStage);
    uint8_t *mstage = p.om_scratch + scr_stage_offset(p.nblk);
    Reader rw, rm;
    rw.init(lay.w0, s);
    rm.init(lay.m0, s);
    struct Buf3 {
        uint32_t w[CH], m[CH], g[CH];
    };
    double_buffered<Buf3>(
        npos,
        [&](Buf3 &bf, uint32_t j0) {
            load_chunk<true>(bf.w, wsf, j0, n_s);
            load_chunk<true>(bf.m, msf, j0, n_s);
            load_chunk<true>(bf.g, gs, j0, n_s);
        },
        [&](Buf3 &bf, uint32_t j0) {
            uint32_t ew[CH], em[CH];
            uint8_t *ow = owsf + (size_t)j0 * NS;
            uint8_t *om = omsf + (size_t)j0 * NS;
            // as in the update: chunks with no spilled input field take a
            // copy of the loop with no memory read in it
            auto elems = [&](auto SP_) {
                constexpr bool SP = decltype(SP_)::value;
#pragma unroll
                for (uint32_t i = 0; i < CH; ++i) {
                    const uint32_t j = j0 + i;
                    uint32_t fw = rw.next(kMWD);
                    rw.q = min(rw.q, qwmax);
                    if (SP && j >= cw_s && j < n_s) {
                        const uint64_t k = wsp + (j - cw_s);
                        fw = (k < p.w_ovf_cap ? (uint32_t)p.w_ovf[k] : 0u) << 23;
                    }
                    uint32_t fm = rm.next(kMMD);
                    rm.q = min(rm.q, qmmax);
                    if (SP && j >= cm_s && j < n_s) {
                        const uint64_t k = msp + (j - cm_s);
                        fm = (k < p.m_ovf_cap ? (uint32_t)p.m_ovf[k] : 0u) << 23;
                    }
                    const uint32_t Rm = sgd_round(bf.g[i] << 16, join32(bf.m[i], fm), p.mu);
                    const uint32_t Rw = sgd_round(join32(bf.w[i], fw), Rm & 0xFFFF0000u, p.neg_eta);
                    if (j < n_s) {
                        ow[i * NS] = (uint8_t)(sgd_sf16(Rw) >> 16);
                        om[i * NS] = (uint8_t)(sgd_sf16(Rm) >> 16);
                    }
                    ew[i] = (Rw >> 20) & 0x7F8u;
                    em[i] = (Rm >> 20) & 0x7F8u;
                }
            };
            if (wave_all((j0 + CH <= cw_s || cw_s >= n_s) && (j0 + CH <= cm_s || cm_s >= n_s))) {
                // no spilled field: four fields per window, a group of four
                // positions at a time, as in the update's general path
#pragma unroll
                for (uint32_t g4 = 0; g4 < CH; g4 += 4) {
                    const int32_t qw0 = rw.q, qm0 = rm.q;
                    uint32_t fw[4], fm[4];
                    const uint32_t cw = rw.next_n<4>(kMWD, qwmax, fw);
                    const uint32_t cm = rm.next_n<4>(kMMD, qmmax, fm);
                    if (__builtin_expect(!wave_all(max(cw, cm) <= 30), 0)) {
                        rw.q = qw0;
                        rm.q = qm0;
#pragma unroll
                        for (uint32_t k = 0; k < 4; ++k) {
                            fw[k] = rw.next(kMWD);
                            rw.q = min(rw.q, qwmax);
                            fm[k] = rm.next(kMMD);
                            rm.q = min(rm.q, qmmax);
                        }
                    }
#pragma unroll
                    for (uint32_t k = 0; k < 4; ++k) {
                        const uint32_t i = g4 + k;
                        const uint32_t Rm = sgd_round(bf.g[i] << 16, join32(bf.m[i], fm[k]), p.mu);
                        const uint32_t Rw = sgd_round(join32(bf.w[i], fw[k]), Rm & 0xFFFF0000u, p.neg_eta);
                        if (j0 + i < n_s) {
                            ow[i * NS] = (uint8_t)(sgd_sf16(Rw) >> 16);
                            om[i * NS] = (uint8_t)(sgd_sf16(Rm) >> 16);
                        }
                        ew[i] = (Rw >> 20) & 0x7F8u;
                        em[i] = (Rm >> 20) & 0x7F8u;
                    }
                }
            } else {
                elems(std::true_type{});
            }
            writer_chunk<true, false>(stw, ew, j0, n_s, capbits, kMWE);
            writer_spill<true>(stw, ew, j0, n_s, wctr, wstage, p.ow_ovf_cap);
            writer_chunk<true, false>(stm, em, j0, n_s, capbits, kMME);
            writer_spill<true>(stm, em, j0, n_s, mctr, mstage, p.om_ovf_cap);
        });
}

// Full-block path (every stream has npos elements and no input field
// spilled): the update's pipeline with both products and both writers.
template <uint32_t CAPT>
__device__ __forceinline__ void mom_stream_full(const MomParams &p, const SgdLayout &lay, PayWriter &stw,
                                                PayWriter &stm, uint64_t r0, const uint16_t *gu) {
    const uint32_t l = lane();
    const uint32_t npos = p.block_elems / NS;
    const uint32_t nh = npos / CH;
    const uint32_t cap = cap_of<CAPT>(p.cap_words);
    const uint32_t capbits = 32 * cap;
    const int32_t qwmax = Reader::bias(lay.w0) + (int32_t)capbits - 2;
    const int32_t qmmax = Reader::bias(lay.m0) + (int32_t)capbits - 2;
    const uint32_t mine = 16 * l;
    const uint32_t lw = l & ~3u;
    const uint32_t jsel = (l & 3u) * 0x01010000u | 0x0C0Cu;
    const uint32_t span = (npos - 1) * NS + US;
    const __amdgpu_buffer_rsrc_t rws = wave_rsrc(p.w_sf + r0, span);
    const __amdgpu_buffer_rsrc_t rms = wave_rsrc(p.m_sf + r0, span);
    const __amdgpu_buffer_rsrc_t rows_ = wave_rsrc(p.ow_sf + r0, span);
    const __amdgpu_buffer_rsrc_t roms = wave_rsrc(p.om_sf + r0, span);
    const __amdgpu_buffer_rsrc_t rg = wave_rsrc(gu, 2 * span);
    constexpr uint32_t kNone = 0x80000000u;
    constexpr uint32_t kHalfB = CH * NS;
    const uint32_t piece = (l >> 2) * NS + 16 * (l & 3);
    uint64_t *wctr = reinterpret_cast<uint64_t *>(p.ow_scratch + kScrStage);
    uint8_t *wstage = p.ow_scratch + scr_stage_offset(p.nblk);
    uint64_t *mctr = reinterpret_cast<uint64_t *>(p.om_scratch + kScrStage);
    uint8_t *mstage = p.om_scratch + scr_stage_offset(p.nblk);
    Reader rw, rm;
    rw.init(lay.w0, l);
    rm.init(lay.m0, l);

    struct Halves {
        u32x4 w, m;
    };
    auto load = [&](Halves &r, uint32_t h) {
        const uint32_t o = h < nh ? h * kHalfB + piece : kNone;
        r.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rws, o, 0, 0));
        r.m = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rms, o, 0, 0));
    };
    auto region = [&](uint32_t h) { return (h & 1u) * kRegB; };
    auto to_lds = [&](const Halves &r, uint32_t h) {
        st128(lay.sw + region(h) + mine, r.w);
        st128(lay.sm + region(h) + mine, r.m);
    };
    // g of group s (positions 4s..4s+3 of this lane's stream), as BF16 bits
    auto gload = [&](uint32_t s, uint32_t (&gv)[4]) {
        const uint32_t o = 2 * (4 * s * NS + l);
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k)
            gv[k] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rg, o + 2 * k * NS, 0, 0);
    };

    uint32_t wsP[4] = {0, 0, 0, 0}, msP[4] = {0, 0, 0, 0}, ewP[4] = {0, 0, 0, 0}, emP[4] = {0, 0, 0, 0};
    uint32_t gP[4] = {0, 0, 0, 0}, gC[4] = {0, 0, 0, 0};
    u32x2 wcw[4] = {{0u, 0u}, {0u, 0u}, {0u, 0u}, {0u, 0u}}, wcm[4] = {{0u, 0u}, {0u, 0u}, {0u, 0u}, {0u, 0u}};
    uint32_t ew8[4] = {kMWNoField, kMWNoField, kMWNoField, kMWNoField};
    uint32_t em8[4] = {kMMNoField, kMMNoField, kMMNoField, kMMNoField};
    uint32_t jw = 0;
    u32x4 outw = {0u, 0u, 0u, 0u}, outm = {0u, 0u, 0u, 0u};
    bool wall = true;

    // a writer's group coded with a check per field; its codes are then spent
    auto checked = [&](PayWriter &st, u32x2 (&wc)[4], const uint32_t (&e8)[4], uint64_t *ctr, uint8_t *stg,
                       uint64_t stg_cap) {
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            if (st.live) {
                if (st.total() + wc[k].y <= capbits) {
                    st.put(wc[k].x, wc[k].y);
                    st.flush();
                } else {
                    st.live = 0;
                    st.cs = jw + k;
                }
            }
            wc[k] = u32x2{0u, 0u};
        }
        writer_spill<false>(st, e8, jw, npos, ctr, stg, stg_cap);
    };
    auto code_checked = [&]() {
        checked(stw, wcw, ew8, wctr, wstage, p.ow_ovf_cap);
        checked(stm, wcm, em8, mctr, mstage, p.om_ovf_cap);
    };

    auto stage_fn = [&](auto DEC_, auto GS_, uint32_t h) {
        constexpr bool DEC = decltype(DEC_)::value;
        constexpr uint32_t GS = decltype(GS_)::value;
        const uint32_t rc = region(h) + GS * 4 * US;
        const uint32_t rp = (GS ? region(h) : region(h + 1)) + ((GS + 3) % 4) * 4 * US;
        uint32_t wsC[4], msC[4], ewC[4], emC[4];
        uint32_t winw = 0, winm = 0, cw = 0, cm = 0;
        const int32_t qw0 = rw.q, qm0 = rm.q;
        if (DEC) {
            winw = rw.window();
            winm = rm.window();
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                wsC[k] = ld32(lay.sw + rc + k * US + lw);
                msC[k] = ld32(lay.sm + rc + k * US + lw);
            }
            gload(4 * h + GS, gC);
        }
        if (!wall && !wave_all(stw.live && stw.total() + 4 * 16 <= capbits &&
                               stm.live && stm.total() + 4 * 16 <= capbits))
            code_checked();
        uint32_t epw[4], epm[4];
        float rmv[4], rwv[4];
        bool nan = false;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            uint32_t enw = 0, enm = 0, wkw = 0, wkm = 0;
            if (DEC) {
                wkw = winw >> cw;
                enw = ld32(kMWD + (wkw & 0x3FCu));
                wkm = winm >> cm;
                enm = ld32(kMMD + (wkm & 0x3FCu));
            }
            rmv[k] = __builtin_fmaf(p.mu, __uint_as_float(join32s(msP[k], emP[k], jsel)),
                                    __uint_as_float(gP[k] << 16));
            if (k & 1) {
                // M' of the pair, rounded; W' from M' as rounded
                uint32_t hm = cvt_bf16x2(rmv[k - 1], rmv[k]);
                asm volatile("" : "+v"(hm));
                rwv[k - 1] = __builtin_fmaf(p.neg_eta, __uint_as_float(hm << 16),
                                            __uint_as_float(join32s(wsP[k - 1], ewP[k - 1], jsel)));
                rwv[k] = __builtin_fmaf(p.neg_eta, __uint_as_float(hm & 0xFFFF0000u),
                                        __uint_as_float(join32s(wsP[k], ewP[k], jsel)));
                uint32_t hw = cvt_bf16x2(rwv[k - 1], rwv[k]);
                asm volatile("" : "+v"(hw));
                nan |= (rmv[k - 1] != rmv[k - 1]) | (rmv[k] != rmv[k]) | (rwv[k - 1] != rwv[k - 1]) |
                       (rwv[k] != rwv[k]);
                epm[k - 1] = (hm >> 4) & 0x7F8u;
                epm[k] = (hm >> 20) & 0x7F8u;
                epw[k - 1] = (hw >> 4) & 0x7F8u;
                epw[k] = (hw >> 20) & 0x7F8u;
                uint32_t bm, bw;
                asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(bm) : "s"(0x00800080u), "v"(hm >> 8), "v"(hm));
                asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(bw) : "s"(0x00800080u), "v"(hw >> 8), "v"(hw));
                st8(lay.sm + rp + (k - 1) * US + l, bm);
                st8hi(lay.sm + rp + k * US + l, bm);
                st8(lay.sw + rp + (k - 1) * US + l, bw);
                st8hi(lay.sw + rp + k * US + l, bw);
                stw.put(wcw[k - 1].x | (wcw[k].x << wcw[k - 1].y), wcw[k - 1].y + wcw[k].y);
                stw.flush();
                stm.put(wcm[k - 1].x | (wcm[k].x << wcm[k - 1].y), wcm[k - 1].y + wcm[k].y);
                stm.flush();
            }
            if (DEC) {
                ewC[k] = (wkw << (enw & 31u)) | enw;
                cw += (enw >> 8) & 0xFFu;
                emC[k] = (wkm << (enm & 31u)) | enm;
                cm += (enm >> 8) & 0xFFu;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // every field of a full block is valid: a window that held its four
        // fields moves a reader at most to its stream's end (no clamp)
        if (DEC) {
            rw.q += (int32_t)cw;
            rm.q += (int32_t)cm;
        }
        if (__builtin_expect(!wave_all((!DEC || max(cw, cm) <= 30) && !nan), 0)) {
            if (DEC && !wave_all(max(cw, cm) <= 30)) {
                // a window ran out: group s again, one field per window
                rw.q = qw0;
                rm.q = qm0;
#pragma unroll
                for (uint32_t k = 0; k < 4; ++k) {
                    ewC[k] = rw.next(kMWD);
                    rw.q = min(rw.q, qwmax);
                    emC[k] = rm.next(kMMD);
                    rm.q = min(rm.q, qmmax);
                }
            }
            // group s-1 with the integer rounding (same fields; a NaN's byte
            // becomes the canonical one's)
#pragma unroll
            for (uint32_t k = 0; k < 4; k += 2) {
                const uint32_t Rm0 = sgd_round(gP[k] << 16, join32s(msP[k], emP[k], jsel), p.mu);
                const uint32_t Rm1 = sgd_round(gP[k + 1] << 16, join32s(msP[k + 1], emP[k + 1], jsel), p.mu);
                const uint32_t Rw0 = sgd_round(join32s(wsP[k], ewP[k], jsel), Rm0 & 0xFFFF0000u, p.neg_eta);
                const uint32_t Rw1 = sgd_round(join32s(wsP[k + 1], ewP[k + 1], jsel), Rm1 & 0xFFFF0000u,
                                               p.neg_eta);
                const uint32_t hm = (Rm0 >> 16) | (Rm1 & 0xFFFF0000u);
                const uint32_t hw = (Rw0 >> 16) | (Rw1 & 0xFFFF0000u);
                epm[k] = (hm >> 4) & 0x7F8u;
                epm[k + 1] = (hm >> 20) & 0x7F8u;
                epw[k] = (hw >> 4) & 0x7F8u;
                epw[k + 1] = (hw >> 20) & 0x7F8u;
                uint32_t bm, bw;
                asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(bm) : "s"(0x00800080u), "v"(hm >> 8), "v"(hm));
                asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(bw) : "s"(0x00800080u), "v"(hw >> 8), "v"(hw));
                st8(lay.sm + rp + k * US + l, bm);
                st8hi(lay.sm + rp + (k + 1) * US + l, bm);
                st8(lay.sw + rp + k * US + l, bw);
                st8hi(lay.sw + rp + (k + 1) * US + l, bw);
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            wcw[k] = ld64(kMWE + epw[k]);
            ew8[k] = epw[k];
            wcm[k] = ld64(kMME + epm[k]);
            em8[k] = epm[k];
        }
        jw = 4 * (4 * h + GS) - 4;
        if (DEC) {
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                wsP[k] = wsC[k];
                msP[k] = msC[k];
                ewP[k] = ewC[k];
                emP[k] = emC[k];
                gP[k] = gC[k];
            }
        }
    };
    auto half = [&](uint32_t h, Halves &next) {
        wall = wave_all(stw.live && stw.total() + CH * 16 <= capbits && stm.live &&
                        stm.total() + CH * 16 <= capbits);
        stage_fn(std::true_type{}, std::integral_constant<uint32_t, 0>{}, h);
        if (h == 0) {
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                wcw[k] = u32x2{0u, 0u};
                wcm[k] = u32x2{0u, 0u};
                ew8[k] = kMWNoField;
                em8[k] = kMMNoField;
            }
            jw = 0;
        } else {
            outw = ld128(lay.sw + region(h - 1) + mine);
            outm = ld128(lay.sm + region(h - 1) + mine);
        }
        to_lds(next, h + 1);
        load(next, h + 2);
        stage_fn(std::true_type{}, std::integral_constant<uint32_t, 1>{}, h);
        if (h != 0) {
            __builtin_amdgcn_raw_buffer_store_b128(outw, rows_, (h - 1) * kHalfB + piece, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(outm, roms, (h - 1) * kHalfB + piece, 0, 0);
        }
        stage_fn(std::true_type{}, std::integral_constant<uint32_t, 2>{}, h);
        stage_fn(std::true_type{}, std::integral_constant<uint32_t, 3>{}, h);
    };
    Halves a;
    load(a, 0);
    to_lds(a, 0);
    load(a, 1);
    for (uint32_t h = 0; h < nh; ++h) half(h, a);
    wall = false;
    stage_fn(std::false_type{}, std::integral_constant<uint32_t, 0>{}, nh);
    code_checked();
    outw = ld128(lay.sw + region(nh - 1) + mine);
    outm = ld128(lay.sm + region(nh - 1) + mine);
    __builtin_amdgcn_raw_buffer_store_b128(outw, rows_, (nh - 1) * kHalfB + piece, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(outm, roms, (nh - 1) * kHalfB + piece, 0, 0);
}

// GEN: the general kernel (blocks that are not full), as for the update.
template <uint32_t CAPT, bool GROUP, bool GEN>
__global__ __launch_bounds__(64 * kMomWaves) __attribute__((amdgpu_waves_per_eu(2)))
void k_mom(const MomParams p) {
    if (!GROUP) {
        stage_dec(p.wdec, kMWD);
        stage_dec(p.mdec, kMMD);
        stage_enc_packed(p.wenc, kMWE);
        stage_enc_packed(p.menc, kMME);
    }
    if (threadIdx.x < 2) st32(kMNone + 4 * threadIdx.x, 0);
    __syncthreads();
    uint64_t staged = ~0ull;
    const uint32_t l = lane();
    const uint32_t cap = cap_of<CAPT>(p.cap_words);
    const SgdLayout lay(cap, kMWave0 + wave_id() * sgd_wave_bytes(cap));
    st32(lay.z0 + 4 * l, 0);
    st32(lay.z1 + 4 * l, 0);
    st32(lay.z2 + 4 * l, 0);
    uint16_t *wcnt_out = p.park_w ? reinterpret_cast<uint16_t *>(p.ow_scratch + scr_cnt_offset(p.nblk)) : p.ow_cnt;
    uint16_t *mcnt_out = p.park_m ? reinterpret_cast<uint16_t *>(p.om_scratch + scr_cnt_offset(p.nblk)) : p.om_cnt;
    static_assert(kMomWaves == kMaxUnits, "a workgroup is one block's units");
    // Workgroups take blocks round-robin; the four waves meet at every block
    // (the units share sign-fraction lines and, in a group, the tables).
    uint32_t nfull = 0;   // units done on the full-block path
    auto block = [&](uint32_t b) {
        __builtin_amdgcn_s_barrier();
        const uint32_t h = wave_id();
        const uint32_t u = b * kMaxUnits + h;
        uint32_t k = 0;
        if (GROUP) {
            k = p.gw.blk_tensor[b];
            const uint32_t tw = p.gw.blk_tab[b], tm = p.gm.blk_tab[b];
            const uint64_t key = ((uint64_t)tm << 32) | tw;
            if (key != staged) {
                stage_dec(p.gw.dec[tw], kMWD);
                stage_dec(p.gm.dec[tm], kMMD);
                stage_enc(p.gw.enc[tw], kMWE);
                stage_enc(p.gm.enc[tm], kMME);
                __syncthreads();
                staged = key;
            }
        }
        const uint64_t wob = p.w_obase[b], wob1 = p.w_obase[b + 1];
        const uint64_t mob = p.m_obase[b], mob1 = p.m_obase[b + 1];
        rows_to_lds<true>(p.w_pay, lay.w0, p.m_pay, lay.m0, b, h, cap);
        uint64_t r0;
        uint32_t nb;
        const uint16_t *gu;
        if (GROUP) {
            const BlockSpan sp = group_span(p.gw, k, p.block_elems, b);
            r0 = sp.sf0;
            nb = sp.nb;
            gu = group_span(p.gg, k, p.block_elems, b).dense + h * US;
        } else {
            r0 = (uint64_t)b * p.block_elems;
            nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
            gu = p.g + r0 + h * US;
        }
        if (!GEN && !block_full(p, b, nb, wob, wob1, mob, mob1)) return;
        const uint32_t n_s = stream_len(nb, h * US + l);
        PayWriter stw, stm;
        stw.init(0, l, n_s);
        stw.rows.init(p.ow_pay, b, h, cap);
        stm.init(0, l, n_s);
        stm.rows.init(p.om_pay, b, h, cap);
        if (!GEN) {
            mom_stream_full<CAPT>(p, lay, stw, stm, r0 + h * US, gu);
            ++nfull;
        } else {
            uint32_t cw_s, cm_s, wex, mex;
            unit_spills(p.w_cnt + (uint64_t)b * NS, nb, h, cw_s, wex);
            unit_spills(p.m_cnt + (uint64_t)b * NS, nb, h, cm_s, mex);
            mom_stream_general<CAPT>(p, lay, stw, stm, n_s, cw_s, cm_s, r0 + h * US, gu, wob + wex, mob + mex);
        }
        // in place, the general kernel parks the counts (other units of the
        // block still read the inputs'); the full-block kernel reads none
        const UnitOut ow{p.ow_pay, GEN ? wcnt_out : p.ow_cnt, p.ow_scratch, p.nblk,
                         p.ow_ovf_cap, cap, GEN ? p.park_w : 0u, 0};
        unit_finish(stw, n_s, u, b, h, 0, ow);
        const UnitOut om{p.om_pay, GEN ? mcnt_out : p.om_cnt, p.om_scratch, p.nblk,
                         p.om_ovf_cap, cap, GEN ? p.park_m : 0u, 0};
        unit_finish(stm, n_s, u, b, h, 0, om);
    };
    if (!GEN) {
        for (uint32_t b = blockIdx.x; b < p.nblk; b += gridDim.x) block(b);
        if (l == 0 && nfull) {
            atomicAdd(reinterpret_cast<uint32_t *>(p.ow_scratch + kScrFullUnits), nfull);
            atomicAdd(reinterpret_cast<uint32_t *>(p.om_scratch + kScrFullUnits), nfull);
        }
    } else {
        for_general<GROUP>(p, p.nblk, [](uint32_t i) { return i; }, block);
    }
}

// ------------------------------------------------------------------ launches

// Dynamic LDS beyond 64 KiB must be requested per kernel; remember the
// largest size granted so far so the runtime is asked only when it grows.
int ensure_lds(const void *kernel, size_t bytes, std::atomic<size_t> &granted) {
    if (bytes <= 64 * 1024 || bytes <= granted.load()) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)bytes);
    if (e == hipSuccess) granted.store(bytes);
    return (int)e;
}

// The capacities of the three modes get their own kernels; others run the
// kernel that reads the capacity at run time.
template <template <uint32_t> class K>
struct ByCap {
    static const void *pick(uint32_t cap) {
        switch (cap) {
        case 25: return K<25>::fn();
        case 12: return K<12>::fn();
        case 11: return K<11>::fn();
        default: return K<0>::fn();
        }
    }
};
template <uint32_t C> struct EncK { static const void *fn() { return reinterpret_cast<const void *>(&k_encode<C, false>); } };
template <uint32_t C> struct DecK { static const void *fn() { return reinterpret_cast<const void *>(&k_decode<C, false>); } };
template <uint32_t C> struct SgdK { static const void *fn() { return reinterpret_cast<const void *>(&k_sgd<C, false, false>); } };
// the CLEAN capacity's full-block update is the ring kernel
template <> struct SgdK<kRingCap> { static const void *fn() { return nullptr; } };
template <uint32_t C> struct SgdXK { static const void *fn() { return reinterpret_cast<const void *>(&k_sgd<C, false, true>); } };
template <uint32_t C> struct EncGK { static const void *fn() { return reinterpret_cast<const void *>(&k_encode<C, true>); } };
template <uint32_t C> struct DecGK { static const void *fn() { return reinterpret_cast<const void *>(&k_decode<C, true>); } };
template <uint32_t C> struct SgdGK { static const void *fn() { return reinterpret_cast<const void *>(&k_sgd<C, true, false>); } };
template <> struct SgdGK<kRingCap> { static const void *fn() { return nullptr; } };
template <uint32_t C> struct SgdGXK { static const void *fn() { return reinterpret_cast<const void *>(&k_sgd<C, true, true>); } };

// per kernel (encode, decode, update, the group encode, decode and update,
// the update's general kernel, flat and group) and capacity slot
std::atomic<size_t> g_lds_granted[8][4];

int cap_slot(uint32_t cap) { return cap == 25 ? 0 : cap == 12 ? 1 : cap == 11 ? 2 : 3; }

// One wave per unit, or (persistent) as many workgroups as the device holds
// at once, never more than there are units to go round.
template <typename P>
int launch(const void *fn, uint64_t nunits, uint32_t waves, bool persistent, size_t lds_bytes,
           const P &p, void *stream, std::atomic<size_t> &granted) {
    const int attr = ensure_lds(fn, lds_bytes, granted);
    if (attr != hipSuccess) return attr;
    const uint64_t want = (nunits + waves - 1) / waves;
    uint32_t grid = (uint32_t)want;
    hipError_t e = hipSuccess;
    if (persistent) {
        int dev = 0, cus = 0, per_cu = 0;
        e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, (int)(64 * waves), lds_bytes);
        if (e != hipSuccess) return (int)e;
        if (per_cu < 1) return (int)hipErrorInvalidConfiguration;
        grid = (uint32_t)std::min<uint64_t>(want, (uint64_t)per_cu * cus);
    }
    void *args[] = {const_cast<P *>(&p)};
    e = hipLaunchKernel(fn, dim3(grid), dim3(64 * waves), args, lds_bytes, (hipStream_t)stream);
    if (e != hipSuccess) return (int)e;
    return (int)hipGetLastError();
}

}  // namespace

size_t encode_lds(uint32_t cap) { return kEncWave0 + (size_t)kEncWaves * enc_wave_bytes(cap); }
size_t decode_lds(uint32_t cap) { return kDecWave0 + (size_t)kDecWaves * dec_wave_bytes(cap); }
size_t sgd_lds(uint32_t cap, uint32_t waves) { return kSgdWave0 + (size_t)waves * sgd_wave_bytes(cap); }

int launch_clear(uint8_t *scratch, uint64_t nblk, uint32_t *status, void *stream) {
    const uint64_t words = (scr_clear_bytes(nblk) + 7) / 8;
    const uint32_t grid = (uint32_t)((words + 255) / 256);
    hipLaunchKernelGGL(k_clear, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<uint64_t *>(scratch), words, status);
    return (int)hipGetLastError();
}

int launch_scan(uint8_t *scratch, uint64_t nblk, uint64_t *obase, uint8_t *ovf, uint64_t ovf_cap,
                uint32_t *status, uint16_t *cnt, void *stream) {
    const uint64_t groups = (nblk + kScanGroup - 1) / kScanGroup;
    hipLaunchKernelGGL(k_scan, dim3((uint32_t)groups), dim3(kScanGroup), 0, (hipStream_t)stream,
                       scratch, nblk, obase, ovf_cap, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const uint32_t place = (uint32_t)std::min<uint64_t>(nblk, 2048);
    hipLaunchKernelGGL(k_place, dim3(place), dim3(256), 0, (hipStream_t)stream, scratch, nblk, obase, ovf,
                       ovf_cap, cnt);
    return (int)hipGetLastError();
}

int launch_encode(const EncodeParams &p, void *stream, bool group) {
    const void *fn = group ? ByCap<EncGK>::pick(p.cap_words) : ByCap<EncK>::pick(p.cap_words);
    return launch(fn, (uint64_t)p.nblk * kMaxUnits, kEncWaves, false, encode_lds(p.cap_words), p, stream,
                  g_lds_granted[group ? 3 : 0][cap_slot(p.cap_words)]);
}

template <uint32_t C> struct MomK { static const void *fn() { return reinterpret_cast<const void *>(&k_mom<C, false, false>); } };
template <uint32_t C> struct MomGK { static const void *fn() { return reinterpret_cast<const void *>(&k_mom<C, true, false>); } };
template <uint32_t C> struct MomXK { static const void *fn() { return reinterpret_cast<const void *>(&k_mom<C, false, true>); } };
template <uint32_t C> struct MomGXK { static const void *fn() { return reinterpret_cast<const void *>(&k_mom<C, true, true>); } };
// flat, group, and their general kernels
std::atomic<size_t> g_mom_lds_granted[4][4];

// The full-block kernel, then the general one (which ends at once when every
// block is full).
int launch_mom(const MomParams &p, void *stream, bool group) {
    const size_t lds = kMWave0 + (size_t)kMomWaves * sgd_wave_bytes(p.cap_words);
    const int slot = cap_slot(p.cap_words);
    // persistent: one workgroup is one block at a time
    const void *fn = group ? ByCap<MomGK>::pick(p.cap_words) : ByCap<MomK>::pick(p.cap_words);
    int e = launch(fn, (uint64_t)p.nblk * kMomWaves, kMomWaves, true, lds, p, stream,
                   g_mom_lds_granted[group ? 1 : 0][slot]);
    if (e != hipSuccess) return e;
    fn = group ? ByCap<MomGXK>::pick(p.cap_words) : ByCap<MomXK>::pick(p.cap_words);
    return launch(fn, (uint64_t)p.nblk * kMomWaves, kMomWaves, true, lds, p, stream,
                  g_mom_lds_granted[group ? 3 : 2][slot]);
}

int launch_decode(const DecodeParams &p, void *stream, bool group) {
    const void *fn = group ? ByCap<DecGK>::pick(p.cap_words) : ByCap<DecK>::pick(p.cap_words);
    return launch(fn, (uint64_t)p.nblk * kMaxUnits, kDecWaves, false, decode_lds(p.cap_words), p, stream,
                  g_lds_granted[group ? 4 : 1][cap_slot(p.cap_words)]);
}

std::atomic<size_t> g_ring_granted[2];

// The full-block kernel (the ring kernel at the CLEAN capacity), then the
// general one (which ends at once when every block is full).
int launch_sgd(const SgdParams &p, void *stream, bool group) {
    const int slot = cap_slot(p.cap_words);
    int e;
    if (p.cap_words == kRingCap) {
        const void *fn = group ? reinterpret_cast<const void *>(&k_sgd_ring<true>)
                               : reinterpret_cast<const void *>(&k_sgd_ring<false>);
        e = launch(fn, (uint64_t)p.nblk * kRingWaves, kRingWaves, true, kRingLds, p, stream,
                   g_ring_granted[group ? 1 : 0]);
    } else {
        const void *fn = group ? ByCap<SgdGK>::pick(p.cap_words) : ByCap<SgdK>::pick(p.cap_words);
        e = launch(fn, (uint64_t)p.nblk * kMaxUnits, kSgdWaves, true, sgd_lds(p.cap_words, kSgdWaves), p, stream,
                   g_lds_granted[group ? 5 : 2][slot]);
    }
    if (e != hipSuccess) return e;
    const void *fn;
    fn = group ? ByCap<SgdGXK>::pick(p.cap_words) : ByCap<SgdXK>::pick(p.cap_words);
    return launch(fn, (uint64_t)p.nblk * kMaxUnits, kSgdGenWaves, true, sgd_lds(p.cap_words, kSgdGenWaves), p,
                  stream,
                  g_lds_granted[group ? 7 : 6][slot]);
}


int launch_sample(const SampleParams &p, void *stream, uint16_t *host_out) {
    hipStream_t st = (hipStream_t)stream;
    if (p.m == 0) return hipSuccess;
    const size_t lds_bytes = kSampleCols + (size_t)p.cap_words * 64 * 4;
    hipLaunchKernelGGL(k_sample, dim3((p.m + 63) / 64), dim3(64), lds_bytes, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    e = hipMemcpyFromSymbolAsync(host_out, HIP_SYMBOL(g_sample), p.m * sizeof(uint16_t), 0,
                                 hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return (int)e;
    return (int)hipStreamSynchronize(st);
}

int launch_fit(const FitParams &p, void *stream) {
    hipLaunchKernelGGL(k_fit, dim3(1), dim3(256), 0, (hipStream_t)stream, p);
    return (int)hipGetLastError();
}

// The allocation-free update's working memory: one static array per device,
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it only stands for the symbol); the device address is
// taken once per device with hipGetSymbolAddress and kept.
namespace noalloc {
static __device__ __align__(256) uint8_t scratch[kNoAllocScratch];
std::mutex g_mu;
void *g_ptr[kMaxDevices];
}  // namespace noalloc

int noalloc_scratch(uint8_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(noalloc::g_mu);
    if (!noalloc::g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc::scratch));
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        noalloc::g_ptr[dev] = p;
    }
    *out = static_cast<uint8_t *>(noalloc::g_ptr[dev]);
    return hipSuccess;
}

int launch_gather(const uint16_t *x, uint64_t n, uint32_t m, void *stream, uint16_t *host_out) {
    hipStream_t st = (hipStream_t)stream;
    if (m == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather, dim3((m + 255) / 256), dim3(256), 0, st, x, n, m);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    e = hipMemcpyFromSymbolAsync(host_out, HIP_SYMBOL(g_sample), m * sizeof(uint16_t), 0,
                                 hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return (int)e;
    return (int)hipStreamSynchronize(st);
}

}  // namespace lct
