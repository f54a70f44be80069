// kernels.hip -- encode, decode and fused SGD kernels of the LCT exponent
// codec, written for CDNA4 (gfx950, wave64).
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
// Mapping.  One lane per stream, so at step j lane s touches element
// j*256 + s of its block and a wave's accesses cover contiguous bytes.  A
// workgroup ("unit") owns SW = 256/H streams of one block.  The block's
// stream words are interleaved (word w of stream s at w*256 + s), so a unit's
// payload rows move between HBM and LDS with 16-byte accesses and every lane
// works on its own column of LDS rows (a row's lanes hit distinct banks).
//
// Bit reader: a code starts at stream bit q+2; the two LDS words around q give
// a 32-bit window by one funnel shift (v_alignbit), whose bits 2..9 are the
// 8-bit peek and index the decode table directly as a byte offset.  The
// window is re-read for every code, so there is no refill logic.  Row -1 of
// each input column is zero for the first codes.
//
// Bit writer: a 64-bit buffer; after every second code both of its words are
// stored (ds_write2st64) at the current row and the next, and the buffer
// advances by a word when the first one is full, so there is no final flush.
// Two sink rows past the stream capacity absorb the stores of a full stream.
//
// Overflow offsets come from a scan of the per-stream spill counts over the
// unit and a decoupled look-back across units (Merrill and Garland,
// "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016); units
// take tickets in order, so spilled fields land in (block, stream, position)
// order in one pass.  Fields that spill are parked in a staging area until
// their offset is known.
//
// Every loop step handles 16 positions per lane and loads the next 16 ahead.
// Full blocks whose inputs carry no spilled fields take a path with no
// overflow reads at all; partial blocks and inputs with spills take a general
// path with per-element checks.
#include <hip/hip_runtime.h>

#include <atomic>

#include "lct_internal.h"

namespace lct {
namespace {

constexpr uint32_t NS = kStreams;
constexpr uint32_t CH = kChunk;
constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagIncl = 2ull << 62;
constexpr uint64_t kFlagVal = (1ull << 62) - 1;
constexpr uint32_t kSpinLimit = 1u << 21;

__device__ __forceinline__ uint32_t lane() { return __lane_id(); }

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t t = __shfl_up(v, d, 64);
        if ((int)lane() >= d) v += t;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// Exclusive scan over the SW threads of the workgroup; the total too.  Every
// thread must call it (it holds two barriers).
template <uint32_t SW>
__device__ __forceinline__ uint32_t group_excl_scan(uint32_t v, uint32_t *s_tmp, uint32_t &total) {
    constexpr uint32_t NW = SW / 64;
    const uint32_t inc = wave_incl_scan(v);
    const uint32_t wid = threadIdx.x >> 6;
    if (lane() == 63) s_tmp[wid] = inc;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (uint32_t k = 0; k < NW; ++k) {
        const uint32_t t = s_tmp[k];
        base += k < wid ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return base + inc - v;
}

// Decoupled look-back for unit u, run by one whole wave: publishes the unit's
// spill total, walks back over the predecessors' descriptors 64 at a time
// until an inclusive prefix is found, publishes its own inclusive prefix and
// returns the exclusive one.  Units come from a ticket counter, so every
// predecessor is already running and never waits on u.  The wait is bounded:
// on time-out the status word records it and the unit goes on.
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

// BF16 bits from a sign-fraction byte and an exponent in bits 30..23 of e23
// (other bits of e23 are ignored): sign to bit 15, fraction to bits 6..0.
__device__ __forceinline__ uint32_t join16(uint32_t sf, uint32_t e23) {
    const uint32_t sfx = sf * 0x101u;
    return (sfx & 0x807Fu) | ((e23 >> 16) & 0x7F80u);
}

// fp32 bits of the BF16 value (sf, e): sf in bytes 3 and 2, e in 30..23.
__device__ __forceinline__ uint32_t join32(uint32_t sf, uint32_t e23) {
    const uint32_t sfx = __builtin_amdgcn_perm(0u, sf, 0x00000C0Cu);
    return (sfx & 0x807FFFFFu) | (e23 & 0x7F800000u);
}

// ------------------------------------------------------------------ code tables in LDS

// Decode table, indexed by peek*4: e << 23 | bits consumed, and a mask that
// selects the literal field (escape codes).
__device__ __forceinline__ void stage_dec(const DecTab &t, uint32_t *ent, uint32_t *msk) {
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) {
        const uint32_t d = t.dec[i];
        ent[i] = ((d & 0xFFu) << 23) | ((d >> 8) & 0x1Fu);
        msk[i] = (d >> 13) & 1u ? 0x7F800000u : 0u;
    }
}

__device__ __forceinline__ void stage_enc(const EncTab &t, uint32_t *bits, uint8_t *len) {
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) {
        bits[i] = t.bits[i];
        len[i] = t.len[i];
    }
}

// ------------------------------------------------------------------ stream reader

template <uint32_t SW>
struct Reader {
    int32_t q;   // stream bit position of the next code, minus 2

    __device__ __forceinline__ void init() { q = -2; }
    // Next exponent field in bits 30..23 of the result (other bits garbage).
    // col: this stream's word in row 0; rows -1 and `cap` are zero.
    __device__ __forceinline__ uint32_t next(const uint32_t *col, const uint32_t *ent,
                                             const uint32_t *msk, uint32_t litsh) {
        const uint32_t *p = col + (q >> 5) * (int32_t)SW;
        const uint32_t a = p[0], b = p[SW];
        const uint32_t win = __builtin_amdgcn_alignbit(b, a, (uint32_t)q);
        const uint32_t k = win & 0x3FCu;
        const uint32_t en = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(ent) + k);
        const uint32_t mk = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(msk) + k);
        q += en & 0xFFu;
        return ((win << litsh) & mk) | en;
    }
};

// ------------------------------------------------------------------ stream writer

template <uint32_t SW>
struct Writer {
    static constexpr uint32_t kRowShift = SW == 256 ? 10 : SW == 128 ? 9 : 8;   // log2(row bytes)
    uint64_t buf;     // pending bits, LSB first (< 32 at every store step)
    uint32_t used;    // bits in buf
    uint32_t *wp;     // LDS word of this stream being filled
    uint32_t live;    // no field has failed to fit yet
    uint32_t cs;      // coded prefix length
    uint32_t claimed; // staging space claimed for the spilled fields
    uint64_t soff;    // start of this stream's spilled fields in the staging area

    __device__ __forceinline__ void init(uint32_t *col0, uint32_t n_s) {
        buf = 0;
        used = 0;
        wp = col0;
        live = 1;
        cs = n_s;
        claimed = 0;
        soff = 0;
    }
    __device__ __forceinline__ void put(uint32_t bits, uint32_t len) {
        buf |= (uint64_t)bits << used;
        used += len;
    }
    // Store both words of the buffer at the current row and the next; move
    // on by a word when the first is full.
    __device__ __forceinline__ void flush() {
        wp[0] = (uint32_t)buf;
        wp[SW] = (uint32_t)(buf >> 32);
        const uint32_t t = used & 32u;
        buf >>= t;
        wp = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(wp) + (t << (kRowShift - 5)));
        used &= 31u;
    }
    __device__ __forceinline__ uint32_t total(const uint32_t *col0) const {
        return (uint32_t)((reinterpret_cast<const char *>(wp) - reinterpret_cast<const char *>(col0)) >>
                          (kRowShift - 5)) + used;
    }
};

// Code the CH fields e[] at positions j0..j0+CH-1; with CHECKED, positions at
// or past n_s are absent.  One capacity test per step in the common case.
template <uint32_t SW, bool CHECKED>
__device__ __forceinline__ void writer_chunk(Writer<SW> &st, const uint32_t (&e)[CH], uint32_t j0,
                                             uint32_t n_s, uint32_t capbits, const uint32_t *ebits,
                                             const uint8_t *elen, const uint32_t *col0) {
    uint32_t cb[CH], cl[CH];
#pragma unroll
    for (uint32_t i = 0; i < CH; ++i) {
        cb[i] = ebits[e[i]];
        cl[i] = elen[e[i]];
        if (CHECKED && j0 + i >= n_s) {
            cb[i] = 0;
            cl[i] = 0;
        }
    }
    if (!st.live) return;
    const uint32_t tot = st.total(col0);
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
                if (st.total(col0) + cl[i] <= capbits) {
                    st.put(cb[i], cl[i]);
                    st.flush();
                } else {
                    st.live = 0;
                    st.cs = j0 + i;
                }
            }
        }
    }
}

// Claim staging space for streams that started spilling in this step (one
// atomic per wave), then park this step's spilled fields there.  Every lane of
// the wave must reach it.
template <uint32_t SW, bool CHECKED>
__device__ __forceinline__ void writer_spill(Writer<SW> &st, const uint32_t (&e)[CH], uint32_t j0,
                                             uint32_t n_s, uint64_t *stage_ctr, uint8_t *stage,
                                             uint64_t stage_cap) {
    const bool fresh = !st.live && !st.claimed;
    if (__any(fresh)) {
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
        for (uint32_t i = 0; i < CH; ++i) {
            const uint32_t j = j0 + i;
            if (j >= st.cs && (!CHECKED || j < n_s)) {
                const uint64_t k = st.soff + (j - st.cs);
                if (k < stage_cap) stage[k] = (uint8_t)e[i];
            }
        }
    }
}

// Where a unit's results go.
struct UnitOut {
    uint32_t *pay;       // whole array
    uint16_t *cnt;       // whole array
    uint64_t *obase;     // whole array
    uint8_t *ovf;
    uint64_t ovf_cap;
    uint32_t *status;
    uint8_t *scratch;
    uint32_t nblk, nunits, cap;
};

// After the stream loop: the unit's payload rows, the overflow offset
// (look-back) and the spilled fields, then counts and the block's marker.
// `before` runs just before cnt / obase are written (the fused update waits
// there until the block's other units have read theirs).
template <uint32_t SW, typename Before>
__device__ void writer_finish(Writer<SW> &st, uint32_t n_s, uint32_t u, uint32_t b, uint32_t h,
                              const uint32_t *s_out, uint32_t *s_tmp, uint64_t *s_ob,
                              const UnitOut &o, Before before) {
    const uint32_t t = threadIdx.x;
    const uint32_t spill = n_s - st.cs;
    uint32_t total;
    const uint32_t excl = group_excl_scan<SW>(spill, s_tmp, total);   // barriers: LDS rows complete
    // payload: cap rows of SW words (16-byte pieces)
    constexpr uint32_t Q = SW / 4;
    const uint4 *src = reinterpret_cast<const uint4 *>(s_out);
    uint4 *dst = reinterpret_cast<uint4 *>(o.pay);
    for (uint32_t i = t; i < o.cap * Q; i += SW) {
        const uint32_t row = i / Q, c = i % Q;
        dst[(((uint64_t)b * o.cap + row) * NS + h * SW) / 4 + c] = src[i];
    }
    if (t < 64) {
        uint64_t *flags = reinterpret_cast<uint64_t *>(o.scratch + kScrFlags);
        const uint64_t ob = lookback(flags, u, total, o.status);
        if (t == 0) *s_ob = ob;
    }
    __syncthreads();
    const uint64_t ob = *s_ob;
    if (spill) {
        const uint8_t *stage = o.scratch + scr_stage_offset(o.nblk);
        for (uint32_t k = 0; k < spill; ++k) {
            const uint64_t from = st.soff + k, to = ob + excl + k;
            if (from < o.ovf_cap && to < o.ovf_cap) o.ovf[to] = stage[from];
        }
    }
    before();
    o.cnt[(uint64_t)b * NS + h * SW + t] = (uint16_t)st.cs;
    if (t == 0) {
        if (h == 0) o.obase[b] = ob;
        if (u == o.nunits - 1) {
            o.obase[o.nblk] = ob + total;
            if (ob + total > o.ovf_cap) atomicOr(o.status, LCT_ST_OVF_FULL);
        }
    }
}

// Copy rows [0, cap) of a unit's columns of a block's payload into LDS rows of
// SW words.
template <uint32_t SW>
__device__ __forceinline__ void stage_rows(const uint32_t *pay, uint64_t b, uint32_t h, uint32_t cap,
                                           uint32_t *dst_row0) {
    constexpr uint32_t Q = SW / 4;
    uint4 *dst = reinterpret_cast<uint4 *>(dst_row0);
    const uint4 *src = reinterpret_cast<const uint4 *>(pay);
    for (uint32_t i = threadIdx.x; i < cap * Q; i += SW) {
        const uint32_t row = i / Q, c = i % Q;
        dst[i] = src[((b * cap + row) * NS + h * SW) / 4 + c];
    }
}

// Spill layout of a block as unit h sees it: this stream's coded count, the
// number of spilled fields of the block's streams before it, the block total.
template <uint32_t SW, uint32_t H>
__device__ __forceinline__ void block_spills(const uint16_t *cnt_b, uint32_t nb, uint32_t h,
                                             uint32_t *s_tmp, uint32_t &c_own, uint32_t &excl,
                                             uint32_t &block_total) {
    uint32_t base = 0, mine = 0, all = 0;
    c_own = 0;
#pragma unroll
    for (uint32_t k = 0; k < H; ++k) {
        const uint32_t s = k * SW + threadIdx.x;
        const uint32_t n_s = stream_len(nb, s);
        const uint32_t c = min<uint32_t>(cnt_b[s], n_s);
        uint32_t tot;
        const uint32_t ex = group_excl_scan<SW>(n_s - c, s_tmp, tot);
        if (k < h) base += tot;
        if (k == h) {
            mine = ex;
            c_own = c;
        }
        all += tot;
    }
    excl = base + mine;
    block_total = all;
}

// ------------------------------------------------------------------ small kernels

__global__ void k_clear(uint64_t *words, uint64_t nwords, uint32_t *status) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nwords) words[i] = 0;
    if (i == 0) *status = 0;
}

__device__ uint16_t g_sample[4096];

__global__ void k_gather(const uint16_t *x, uint64_t n, uint32_t m) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < m) g_sample[i] = x[(uint64_t)i * n / m];
}

// ------------------------------------------------------------------ encode

constexpr uint32_t kEncH = 1, kEncSW = NS / kEncH;

template <bool FULL>
__device__ __forceinline__ void encode_stream(const EncodeParams &p, Writer<kEncSW> &st,
                                              uint32_t n_s, uint64_t r0, const uint32_t *ebits,
                                              const uint8_t *elen, const uint32_t *col0) {
    const uint32_t s = threadIdx.x;
    const uint32_t npos = p.block_elems / NS;
    const uint32_t capbits = 32 * p.cap_words;
    const uint16_t *xs = p.x + r0 + s;
    uint8_t *sfs = p.sf + r0 + s;
    uint64_t *stage_ctr = reinterpret_cast<uint64_t *>(p.scratch + kScrStage);
    uint8_t *stage = p.scratch + scr_stage_offset(p.nblk);
    uint32_t v[CH], vn[CH];
#pragma unroll
    for (uint32_t i = 0; i < CH; ++i) v[i] = (FULL || i < n_s) ? xs[i * NS] : 0;
    for (uint32_t j0 = 0; j0 < npos; j0 += CH) {
        if (j0 + CH < npos) {
#pragma unroll
            for (uint32_t i = 0; i < CH; ++i) {
                const uint32_t j = j0 + CH + i;
                vn[i] = (FULL || j < n_s) ? xs[j * NS] : 0;
            }
        }
        uint32_t e[CH];
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) {
            e[i] = (v[i] >> 7) & 0xFFu;
            if (FULL || j0 + i < n_s)
                sfs[(j0 + i) * NS] = (uint8_t)(((v[i] >> 8) & 0x80u) | (v[i] & 0x7Fu));
        }
        writer_chunk<kEncSW, !FULL>(st, e, j0, n_s, capbits, ebits, elen, col0);
        writer_spill<kEncSW, !FULL>(st, e, j0, n_s, stage_ctr, stage, p.ovf_cap);
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) v[i] = vn[i];
    }
}

__global__ __launch_bounds__(256) void k_encode(const EncodeParams p) {
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_tmp[4];
    __shared__ uint32_t s_ticket;
    __shared__ uint64_t s_ob;
    constexpr uint32_t SW = kEncSW;
    const uint32_t t = threadIdx.x;
    const uint32_t cap = p.cap_words;
    uint32_t *s_out = lds;                                    // cap rows + 2 sink rows
    uint32_t *s_bits = lds + (cap + 2) * SW;                  // 256 words
    uint8_t *s_len = reinterpret_cast<uint8_t *>(s_bits + 256);
    stage_enc(p.enc, s_bits, s_len);
    uint32_t *col0 = s_out + t;
    for (uint32_t w = 0; w < cap; ++w) col0[w * SW] = 0;
    if (t == 0) s_ticket = atomicAdd(reinterpret_cast<uint32_t *>(p.scratch + kScrTicket), 1u);
    __syncthreads();
    const uint32_t u = s_ticket;
    const uint32_t nunits = p.nblk * kEncH;
    if (u >= nunits) return;   // only if the scratch header was not cleared
    const uint32_t b = u / kEncH, h = u % kEncH;
    const uint64_t r0 = (uint64_t)b * p.block_elems;
    const uint32_t nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
    const uint32_t n_s = stream_len(nb, h * SW + t);
    Writer<SW> st;
    st.init(col0, n_s);
    if (nb == p.block_elems)
        encode_stream<true>(p, st, n_s, r0 + h * SW, s_bits, s_len, col0);
    else
        encode_stream<false>(p, st, n_s, r0 + h * SW, s_bits, s_len, col0);
    const UnitOut o{p.pay, p.cnt, p.obase, p.ovf, p.ovf_cap, p.status, p.scratch,
                    p.nblk, nunits, cap};
    writer_finish<SW>(st, n_s, u, b, h, s_out, s_tmp, &s_ob, o, [] {});
}

// ------------------------------------------------------------------ decode

template <bool FAST>
__device__ __forceinline__ void decode_stream(const DecodeParams &p, uint32_t n_s, uint32_t c_s,
                                              uint64_t r0, uint64_t sp0, const uint32_t *col,
                                              const uint32_t *ent, const uint32_t *msk) {
    const uint32_t s = threadIdx.x;
    const uint32_t npos = p.block_elems / NS;
    const int32_t qmax = 32 * (int32_t)p.cap_words - 2;
    const uint32_t litsh = 21 - p.dec.esc_len;
    const uint8_t *sfs = p.sf + r0 + s;
    uint16_t *ys = p.y + r0 + s;
    Reader<NS> rd;
    rd.init();
    uint32_t f[CH], fn[CH];
#pragma unroll
    for (uint32_t i = 0; i < CH; ++i) f[i] = (FAST || i < n_s) ? sfs[i * NS] : 0;
    for (uint32_t j0 = 0; j0 < npos; j0 += CH) {
        if (j0 + CH < npos) {
#pragma unroll
            for (uint32_t i = 0; i < CH; ++i) {
                const uint32_t j = j0 + CH + i;
                fn[i] = (FAST || j < n_s) ? sfs[j * NS] : 0;
            }
        }
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) {
            const uint32_t j = j0 + i;
            uint32_t e23 = rd.next(col, ent, msk, litsh);
            if (!FAST) {
                rd.q = min(rd.q, qmax);
                if (j >= c_s && j < n_s) {
                    const uint64_t k = sp0 + (j - c_s);
                    e23 = (k < p.ovf_cap ? (uint32_t)p.ovf[k] : 0u) << 23;
                }
            }
            if (FAST || j < n_s) ys[j * NS] = (uint16_t)join16(f[i], e23);
        }
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) f[i] = fn[i];
    }
}

__global__ __launch_bounds__(256) void k_decode(const DecodeParams p) {
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_tmp[4];
    const uint32_t t = threadIdx.x, b = blockIdx.x;
    const uint32_t cap = p.cap_words;
    uint32_t *s_in = lds + NS;                                // row -1 at lds, rows 0..cap-1, row cap
    uint32_t *s_ent = lds + (cap + 2) * NS;
    uint32_t *s_msk = s_ent + 256;
    stage_dec(p.dec, s_ent, s_msk);
    stage_rows<NS>(p.pay, b, 0, cap, s_in);
    lds[t] = 0;
    s_in[cap * NS + t] = 0;
    const uint64_t r0 = (uint64_t)b * p.block_elems;
    const uint32_t nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
    const uint32_t n_s = stream_len(nb, t);
    uint32_t c_s, excl, total;
    block_spills<NS, 1>(p.cnt + (uint64_t)b * NS, nb, 0, s_tmp, c_s, excl, total);  // barriers
    const uint64_t sp0 = p.obase[b] + excl;
    if (nb == p.block_elems && total == 0)
        decode_stream<true>(p, n_s, c_s, r0, sp0, s_in + t, s_ent, s_msk);
    else
        decode_stream<false>(p, n_s, c_s, r0, sp0, s_in + t, s_ent, s_msk);
}

// ------------------------------------------------------------------ fused SGD

constexpr uint32_t kSgdH = 2, kSgdSW = NS / kSgdH;

// One element: rne_bf16(fmaf(-eta, m, w)) in bits 31..16 of the result (bits
// 15..0 hold rounding garbage); a NaN gives 0x7FC0.
__device__ __forceinline__ uint32_t sgd_round(uint32_t wf, uint32_t mf, float neg_eta) {
    const float r = __builtin_fmaf(neg_eta, __uint_as_float(mf), __uint_as_float(wf));
    const uint32_t u = __float_as_uint(r);
    uint32_t R = u + 0x7FFFu + ((u >> 16) & 1u);
    const bool nan = r != r;
    if (__builtin_expect(__any(nan), 0)) R = nan ? 0x7FC00000u : R;
    return R;
}

template <bool FAST>
__device__ __forceinline__ void sgd_stream(const SgdParams &p, Writer<kSgdSW> &st, uint32_t n_s,
                                           uint32_t cw_s, uint32_t cm_s, uint64_t r0, uint64_t wsp,
                                           uint64_t msp, const uint32_t *wcol, const uint32_t *mcol,
                                           const uint32_t *went, const uint32_t *wmsk,
                                           const uint32_t *ment, const uint32_t *mmsk,
                                           const uint32_t *ebits, const uint8_t *elen,
                                           const uint32_t *ocol0) {
    constexpr uint32_t SW = kSgdSW;
    const uint32_t s = threadIdx.x;
    const uint32_t npos = p.block_elems / NS;
    const uint32_t capbits = 32 * p.cap_words;
    const int32_t qmax = (int32_t)capbits - 2;
    const uint32_t wlit = 21 - p.wdec.esc_len, mlit = 21 - p.mdec.esc_len;
    const uint8_t *wsf = p.w_sf + r0 + s;
    const uint8_t *msf = p.m_sf + r0 + s;
    uint8_t *osf = p.o_sf + r0 + s;
    uint64_t *stage_ctr = reinterpret_cast<uint64_t *>(p.scratch + kScrStage);
    uint8_t *stage = p.scratch + scr_stage_offset(p.nblk);
    Reader<SW> rw, rm;
    rw.init();
    rm.init();
    uint32_t fw[CH], fm[CH], fwn[CH], fmn[CH];
#pragma unroll
    for (uint32_t i = 0; i < CH; ++i) {
        fw[i] = (FAST || i < n_s) ? wsf[i * NS] : 0;
        fm[i] = (FAST || i < n_s) ? msf[i * NS] : 0;
    }
    for (uint32_t j0 = 0; j0 < npos; j0 += CH) {
        if (j0 + CH < npos) {
#pragma unroll
            for (uint32_t i = 0; i < CH; ++i) {
                const uint32_t j = j0 + CH + i;
                fwn[i] = (FAST || j < n_s) ? wsf[j * NS] : 0;
                fmn[i] = (FAST || j < n_s) ? msf[j * NS] : 0;
            }
        }
        uint32_t e[CH];
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) {
            const uint32_t j = j0 + i;
            uint32_t ew = rw.next(wcol, went, wmsk, wlit);
            uint32_t em = rm.next(mcol, ment, mmsk, mlit);
            if (!FAST) {
                rw.q = min(rw.q, qmax);
                rm.q = min(rm.q, qmax);
                if (j >= cw_s && j < n_s) {
                    const uint64_t k = wsp + (j - cw_s);
                    ew = (k < p.w_ovf_cap ? (uint32_t)p.w_ovf[k] : 0u) << 23;
                }
                if (j >= cm_s && j < n_s) {
                    const uint64_t k = msp + (j - cm_s);
                    em = (k < p.m_ovf_cap ? (uint32_t)p.m_ovf[k] : 0u) << 23;
                }
            }
            const uint32_t R = sgd_round(join32(fw[i], ew), join32(fm[i], em), p.neg_eta);
            // sign-fraction byte of the result: move the sign (bit 31) to bit
            // 23, then store bits 23..16
            const uint32_t sfr = (R & ~0x00800000u) | ((R >> 8) & 0x00800000u);
            if (FAST || j < n_s) osf[j * NS] = (uint8_t)(sfr >> 16);
            e[i] = (R >> 23) & 0xFFu;
        }
        writer_chunk<SW, !FAST>(st, e, j0, n_s, capbits, ebits, elen, ocol0);
        writer_spill<SW, !FAST>(st, e, j0, n_s, stage_ctr, stage, p.ovf_cap);
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) {
            fw[i] = fwn[i];
            fm[i] = fmn[i];
        }
    }
}

__global__ __launch_bounds__(128) void k_sgd(const SgdParams p) {
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_tmp[4];
    __shared__ uint32_t s_ticket;
    __shared__ uint64_t s_ob;
    constexpr uint32_t SW = kSgdSW, H = kSgdH;
    const uint32_t t = threadIdx.x;
    const uint32_t cap = p.cap_words;
    // LDS rows (SW words each): the output's rows 0..cap-1 and its two sink
    // rows; W's zero row -1 and rows 0..cap-1; a zero row (W's row cap and M's
    // row -1); M's rows; a zero row.  With cap >= 18 the output's sink rows
    // are W's row -1 and row 0: a stream's output reaches row cap-1 only after
    // 2*(cap-1) >= 34 fields, when its own W reader has left rows -1 and 0.
    const bool alias = cap >= 18;
    uint32_t *s_out = lds;
    uint32_t *z0 = lds + (alias ? cap : cap + 2) * SW;
    uint32_t *s_w = z0 + SW;
    uint32_t *z1 = s_w + cap * SW;
    uint32_t *s_m = z1 + SW;
    uint32_t *z2 = s_m + cap * SW;
    uint32_t *tabs = z2 + SW;
    uint32_t *went = tabs, *wmsk = tabs + 256, *ment = tabs + 512, *mmsk = tabs + 768;
    uint32_t *ebits = tabs + 1024;
    uint8_t *elen = reinterpret_cast<uint8_t *>(tabs + 1280);
    stage_dec(p.wdec, went, wmsk);
    stage_dec(p.mdec, ment, mmsk);
    stage_enc(p.wenc, ebits, elen);
    if (t == 0) s_ticket = atomicAdd(reinterpret_cast<uint32_t *>(p.scratch + kScrTicket), 1u);
    __syncthreads();
    const uint32_t u = s_ticket;
    const uint32_t nunits = p.nblk * H;
    if (u >= nunits) return;   // only if the scratch header was not cleared
    const uint32_t b = u / H, h = u % H;
    stage_rows<SW>(p.w_pay, b, h, cap, s_w);
    stage_rows<SW>(p.m_pay, b, h, cap, s_m);
    z0[t] = 0;
    z1[t] = 0;
    z2[t] = 0;
    uint32_t *ocol0 = s_out + t;
    for (uint32_t w = 0; w < cap; ++w) ocol0[w * SW] = 0;
    const uint64_t r0 = (uint64_t)b * p.block_elems;
    const uint32_t nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
    const uint32_t n_s = stream_len(nb, h * SW + t);
    uint32_t cw_s, cm_s, wex, mex, wtot, mtot;
    block_spills<SW, H>(p.w_cnt + (uint64_t)b * NS, nb, h, s_tmp, cw_s, wex, wtot);   // barriers
    block_spills<SW, H>(p.m_cnt + (uint64_t)b * NS, nb, h, s_tmp, cm_s, mex, mtot);
    const uint64_t wsp = p.w_obase[b] + wex, msp = p.m_obase[b] + mex;
    // this unit has read what the block's other units may overwrite in place
    uint32_t *readers = reinterpret_cast<uint32_t *>(p.scratch + scr_readers_offset(p.nblk));
    __syncthreads();
    if (t == 0) __hip_atomic_fetch_add(&readers[b], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    Writer<SW> st;
    st.init(ocol0, n_s);
    if (nb == p.block_elems && wtot == 0 && mtot == 0)
        sgd_stream<true>(p, st, n_s, cw_s, cm_s, r0 + h * SW, wsp, msp, s_w + t, s_m + t, went,
                         wmsk, ment, mmsk, ebits, elen, ocol0);
    else
        sgd_stream<false>(p, st, n_s, cw_s, cm_s, r0 + h * SW, wsp, msp, s_w + t, s_m + t, went,
                          wmsk, ment, mmsk, ebits, elen, ocol0);
    const UnitOut o{p.o_pay, p.o_cnt, p.o_obase, p.o_ovf, p.ovf_cap, p.status, p.scratch,
                    p.nblk, nunits, cap};
    uint32_t *status = p.status;
    writer_finish<SW>(st, n_s, u, b, h, s_out, s_tmp, &s_ob, o, [readers, b, status, t] {
        // counts and offsets of W may be this block's own buffers: wait until
        // every unit of the block has read them (they all hold tickets, so
        // they are running, and they read before anything else)
        if (t == 0) {
            uint32_t spins = 0;
            while (__hip_atomic_load(&readers[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < H) {
                if (++spins > kSpinLimit) {
                    atomicOr(status, LCT_ST_LOOKBACK);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
    });
}

// Dynamic LDS beyond 64 KiB must be requested per kernel; remember the
// largest size granted so far so the runtime is asked only when it grows.
template <typename K>
int ensure_lds(K kernel, size_t bytes, std::atomic<size_t> &granted) {
    if (bytes <= 64 * 1024 || bytes <= granted.load()) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) granted.store(bytes);
    return (int)e;
}

std::atomic<size_t> g_enc_lds{0}, g_dec_lds{0}, g_sgd_lds{0};

}  // namespace

size_t encode_lds(uint32_t cap) { return (size_t)(cap + 2) * kEncSW * 4 + 256 * 4 + 256; }
size_t decode_lds(uint32_t cap) { return (size_t)(cap + 2) * NS * 4 + 2 * 256 * 4; }
size_t sgd_lds(uint32_t cap) {
    const uint32_t rows = (cap >= 18 ? cap : cap + 2) + 1 + cap + 1 + cap + 1;
    return (size_t)rows * kSgdSW * 4 + 1280 * 4 + 256;
}

int launch_clear(uint8_t *scratch, uint64_t nblk, uint32_t *status, void *stream) {
    const uint64_t words = (scr_clear_bytes(nblk) + 7) / 8;
    const uint32_t grid = (uint32_t)((words + 255) / 256);
    hipLaunchKernelGGL(k_clear, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<uint64_t *>(scratch), words, status);
    return (int)hipGetLastError();
}

int launch_encode(const EncodeParams &p, void *stream) {
    const int attr = ensure_lds(k_encode, encode_lds(p.cap_words), g_enc_lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_encode, dim3(p.nblk * kEncH), dim3(kEncSW), encode_lds(p.cap_words),
                       (hipStream_t)stream, p);
    return (int)hipGetLastError();
}

int launch_decode(const DecodeParams &p, void *stream) {
    const int attr = ensure_lds(k_decode, decode_lds(p.cap_words), g_dec_lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_decode, dim3(p.nblk), dim3(NS), decode_lds(p.cap_words), (hipStream_t)stream, p);
    return (int)hipGetLastError();
}

int launch_sgd(const SgdParams &p, void *stream) {
    const int attr = ensure_lds(k_sgd, sgd_lds(p.cap_words), g_sgd_lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_sgd, dim3(p.nblk * kSgdH), dim3(kSgdSW), sgd_lds(p.cap_words),
                       (hipStream_t)stream, p);
    return (int)hipGetLastError();
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
