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
// Mapping: one workgroup (4 waves) per block and one lane per stream, so lane
// s reads element j*256 + s of its block at step j and a wave's reads cover
// 128 contiguous bytes.  A stream's 32-bit words are interleaved with the other
// streams' (word w of stream s at w*256 + s), so a block's payload is one
// contiguous range that moves between HBM and LDS with 16-byte accesses; the
// per-lane bit writer and reader work on that LDS copy, where the 256 lanes of
// a row hit distinct banks.  The code tables sit in LDS.  Overflow offsets
// come from a block scan of per-stream spill counts and a decoupled look-back
// across blocks (Merrill and Garland, "Single-pass Parallel Prefix Scan with
// Decoupled Look-back", 2016), so spilled fields land in (block, stream,
// position) order in one pass.
#include <hip/hip_runtime.h>

#include <atomic>

#include "lct_internal.h"

namespace lct {
namespace {

constexpr uint32_t NS = kStreams;
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

// Exclusive scan over the 256 lanes of the workgroup; total returned too.
// All 256 threads must call it.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *s_tmp, uint32_t &total) {
    const uint32_t inc = wave_incl_scan(v);
    const uint32_t wid = threadIdx.x >> 6;
    if (lane() == 63) s_tmp[wid] = inc;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        const uint32_t t = s_tmp[k];
        base += k < wid ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return base + inc - v;
}

// Decoupled look-back for block b, run by one whole wave: publishes the
// block's spill total, walks back over the predecessors' descriptors 64 at a
// time until an inclusive prefix is found, publishes its own inclusive prefix
// and returns the exclusive one.  Block indices come from a ticket counter,
// so every predecessor is already running and never waits on b.
__device__ uint64_t lookback(uint64_t *flags, uint32_t b, uint64_t agg, uint32_t *status) {
    if (b == 0) {
        if (lane() == 0)
            __hip_atomic_store(&flags[0], kFlagIncl | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
    }
    if (lane() == 0)
        __hip_atomic_store(&flags[b], kFlagAgg | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t excl = 0;
    int64_t top = (int64_t)b - 1;
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
        __hip_atomic_store(&flags[b], kFlagIncl | (excl + agg), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return excl;
}

__device__ __forceinline__ uint32_t sf_byte(uint32_t v) { return ((v >> 8) & 0x80u) | (v & 0x7Fu); }
__device__ __forceinline__ uint32_t join16(uint32_t sf, uint32_t e) {
    return ((sf & 0x80u) << 8) | (e << 7) | (sf & 0x7Fu);
}

// ------------------------------------------------------------------ stream writer

struct Writer {
    uint64_t buf;     // pending bits, LSB first
    uint32_t used;    // pending bit count (< 32 between steps)
    uint32_t w;       // index of the word being filled
    uint32_t live;    // still coding (no field has failed to fit yet)
    uint32_t cs;      // coded prefix length once a field failed to fit
    uint32_t claimed; // staging space claimed for the spilled fields
    uint64_t soff;    // start of this stream's spilled fields in the staging area

    __device__ void init(uint32_t n_s) {
        buf = 0;
        used = w = 0;
        live = 1;
        cs = n_s;
        claimed = 0;
        soff = 0;
    }
    __device__ __forceinline__ void put(uint32_t bits, uint32_t len) {
        buf |= (uint64_t)bits << used;
        used += len;
    }
    // Store the current word (partial words are rewritten until complete);
    // advance when it is full.  col points at this stream's column in LDS.
    __device__ __forceinline__ void flush(uint32_t *col) {
        col[w * NS] = (uint32_t)buf;
        if (used >= 32) {
            ++w;
            buf >>= 32;
            used -= 32;
        }
    }
};

// Code the 8 fields e[] at positions j0..j0+7 (those at or past n_s are
// absent).  The common case is one capacity test per 8 fields.
template <bool FULL>
__device__ __forceinline__ void writer_chunk(Writer &st, const uint32_t (&e)[kChunk], uint32_t j0,
                                             uint32_t n_s, uint32_t capbits, const uint32_t *s_bits,
                                             const uint8_t *s_len, uint32_t *col) {
    uint32_t cb[kChunk], cl[kChunk], sum = 0;
#pragma unroll
    for (uint32_t i = 0; i < kChunk; ++i) {
        cb[i] = s_bits[e[i]];
        cl[i] = s_len[e[i]];
        if (!FULL && j0 + i >= n_s) {
            cb[i] = 0;
            cl[i] = 0;
        }
        sum += cl[i];
    }
    if (st.live && st.w * 32 + st.used + sum <= capbits) {
#pragma unroll
        for (uint32_t k = 0; k < kChunk; k += 2) {
            st.put(cb[k], cl[k]);
            st.put(cb[k + 1], cl[k + 1]);
            st.flush(col);
        }
    } else if (st.live) {
#pragma unroll
        for (uint32_t i = 0; i < kChunk; ++i) {
            if (st.live) {
                if (st.w * 32 + st.used + cl[i] <= capbits) {
                    st.put(cb[i], cl[i]);
                    st.flush(col);
                } else {
                    st.live = 0;
                    st.cs = j0 + i;
                }
            }
        }
    }
}

// Claim staging space for streams that started spilling in this step (one
// atomic per wave), then park this step's spilled fields there.  Must be
// reached by every lane of the wave.
template <bool FULL>
__device__ __forceinline__ void writer_spill(Writer &st, const uint32_t (&e)[kChunk], uint32_t j0,
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
        for (uint32_t i = 0; i < kChunk; ++i) {
            const uint32_t j = j0 + i;
            if (j >= st.cs && (FULL || j < n_s)) {
                const uint64_t k = st.soff + (j - st.cs);
                if (k < stage_cap) stage[k] = (uint8_t)e[i];
            }
        }
    }
}

// After the stream loop: store the last partial word, write cnt, the block's
// payload, the overflow offsets (look-back) and the spilled fields.
struct BlockOut {
    uint32_t *pay;       // this block's payload (cap * 256 words)
    uint16_t *cnt;       // this block's 256 counts
    uint64_t *obase;     // whole array
    uint8_t *ovf;
    uint64_t ovf_cap;
    uint32_t *status;
    uint8_t *scratch;
    uint8_t *stage;
    uint64_t stage_cap;
    uint32_t nblk;
};

__device__ void writer_finish(Writer &st, uint32_t n_s, uint32_t b, uint32_t cap, uint32_t *s_pay,
                              uint32_t *col, uint32_t *s_tmp, uint64_t *s_ob, const BlockOut &o) {
    const uint32_t s = threadIdx.x;
    col[st.w * NS] = (uint32_t)st.buf;    // row cap is a sink when the stream is exactly full
    o.cnt[s] = (uint16_t)st.cs;
    const uint32_t spill = n_s - st.cs;
    uint32_t total;
    const uint32_t excl = block_excl_scan(spill, s_tmp, total);   // has barriers
    // payload: cap rows of 256 words, contiguous in HBM
    const uint4 *src = reinterpret_cast<const uint4 *>(s_pay);
    uint4 *dst = reinterpret_cast<uint4 *>(o.pay);
    for (uint32_t i = s; i < cap * (NS / 4); i += NS) dst[i] = src[i];
    if (s < 64) {
        uint64_t *flags = reinterpret_cast<uint64_t *>(o.scratch + kScrFlags);
        const uint64_t ob = lookback(flags, b, total, o.status);
        if (s == 0) *s_ob = ob;
    }
    __syncthreads();
    const uint64_t ob = *s_ob;
    if (spill) {
        for (uint32_t t = 0; t < spill; ++t) {
            const uint64_t from = st.soff + t, to = ob + excl + t;
            if (from < o.stage_cap && to < o.ovf_cap) o.ovf[to] = o.stage[from];
        }
    }
    if (s == 0) {
        o.obase[b] = ob;
        if (b == o.nblk - 1) {
            o.obase[o.nblk] = ob + total;
            if (ob + total > o.ovf_cap) atomicOr(o.status, LCT_ST_OVF_FULL);
        }
    }
}

// ------------------------------------------------------------------ stream reader

struct Reader {
    uint64_t buf;   // next bits of the stream, LSB first
    uint32_t nb;    // valid bits in buf (>= 32 at the start of every pair of symbols)
    uint32_t wr;    // next word to load (row `cap` of the LDS copy is zero)

    __device__ __forceinline__ void init(const uint32_t *col, uint32_t cap) {
        buf = (uint64_t)col[0] | ((uint64_t)col[min(1u, cap) * NS] << 32);
        nb = 64;
        wr = min(2u, cap);
    }
    // Next exponent field: peek 8 bits, look up (field, bits, escape mask);
    // an escaped field is the 8 bits after the escape code.
    __device__ __forceinline__ uint32_t next(const uint8_t *s_sym, const uint8_t *s_len,
                                             const uint8_t *s_msk, uint32_t esc_len) {
        const uint32_t pk = (uint32_t)buf & 0xFFu;
        const uint32_t lit = ((uint32_t)buf >> esc_len) & 0xFFu;
        const uint32_t e = (lit & s_msk[pk]) | s_sym[pk];
        const uint32_t l = s_len[pk];
        buf >>= l;
        nb -= l;
        return e;
    }
    __device__ __forceinline__ void refill(const uint32_t *col, uint32_t cap) {
        if (nb < 32) {
            buf |= (uint64_t)col[wr * NS] << nb;
            nb += 32;
            wr = min(wr + 1, cap);
        }
    }
};

__device__ __forceinline__ void stage_dec(const DecTab &t, uint8_t *s_sym, uint8_t *s_len,
                                          uint8_t *s_msk) {
    const uint32_t s = threadIdx.x;
    const uint32_t ent = t.dec[s];
    s_sym[s] = (uint8_t)(ent & 0xFFu);
    s_len[s] = (uint8_t)((ent >> 8) & 0x1Fu);
    s_msk[s] = (ent >> 13) & 1u ? 0xFF : 0x00;
}

__device__ __forceinline__ void stage_payload(const uint32_t *pay, uint32_t cap, uint32_t *s_pay) {
    const uint4 *src = reinterpret_cast<const uint4 *>(pay);
    uint4 *dst = reinterpret_cast<uint4 *>(s_pay);
    for (uint32_t i = threadIdx.x; i < cap * (NS / 4); i += NS) dst[i] = src[i];
    s_pay[cap * NS + threadIdx.x] = 0;
}

__device__ __forceinline__ uint32_t stream_len(uint32_t nb, uint32_t s) {
    return nb > s ? (nb - s + NS - 1) / NS : 0;
}

// ------------------------------------------------------------------ kernels

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

template <bool FULL>
__device__ __forceinline__ void encode_stream(const EncodeParams &p, Writer &st, uint32_t n_s,
                                              uint64_t r0, const uint32_t *s_bits,
                                              const uint8_t *s_len, uint32_t *col) {
    const uint32_t s = threadIdx.x;
    const uint32_t npos = p.block_elems / NS;
    const uint32_t capbits = 32 * p.cap_words;
    const uint16_t *xs = p.x + r0 + s;
    uint8_t *sfs = p.sf + r0 + s;
    uint64_t *stage_ctr = reinterpret_cast<uint64_t *>(p.scratch + kScrStage);
    uint8_t *stage = p.scratch + scr_stage_offset(p.nblk);
    uint32_t v[kChunk], vn[kChunk];
#pragma unroll
    for (uint32_t i = 0; i < kChunk; ++i) v[i] = (FULL || i < n_s) ? xs[i * NS] : 0;
    for (uint32_t j0 = 0; j0 < npos; j0 += kChunk) {
        if (j0 + kChunk < npos) {
#pragma unroll
            for (uint32_t i = 0; i < kChunk; ++i) {
                const uint32_t j = j0 + kChunk + i;
                vn[i] = (FULL || j < n_s) ? xs[j * NS] : 0;
            }
        }
        uint32_t e[kChunk];
#pragma unroll
        for (uint32_t i = 0; i < kChunk; ++i) {
            e[i] = (v[i] >> 7) & 0xFFu;
            if (FULL || j0 + i < n_s) sfs[(j0 + i) * NS] = (uint8_t)sf_byte(v[i]);
        }
        writer_chunk<FULL>(st, e, j0, n_s, capbits, s_bits, s_len, col);
        writer_spill<FULL>(st, e, j0, n_s, stage_ctr, stage, p.ovf_cap);
#pragma unroll
        for (uint32_t i = 0; i < kChunk; ++i) v[i] = vn[i];
    }
}

__global__ __launch_bounds__(256) void k_encode(const EncodeParams p) {
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_tmp[4];
    __shared__ uint32_t s_ticket;
    __shared__ uint64_t s_ob;
    const uint32_t s = threadIdx.x;
    const uint32_t cap = p.cap_words;
    uint32_t *s_pay = lds;                                   // (cap + 1) rows
    uint32_t *s_bits = lds + (cap + 1) * NS;                 // 256 words
    uint8_t *s_len = reinterpret_cast<uint8_t *>(s_bits + NS);   // 256 bytes
    s_bits[s] = p.enc.bits[s];
    s_len[s] = p.enc.len[s];
    uint32_t *col = s_pay + s;
    for (uint32_t w = 0; w <= cap; ++w) col[w * NS] = 0;
    if (s == 0) s_ticket = atomicAdd(reinterpret_cast<uint32_t *>(p.scratch + kScrTicket), 1u);
    __syncthreads();
    const uint32_t b = s_ticket;
    if (b >= p.nblk) return;   // only if the scratch header was not cleared
    const uint64_t r0 = (uint64_t)b * p.block_elems;
    const uint32_t nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
    const uint32_t n_s = stream_len(nb, s);
    Writer st;
    st.init(n_s);
    if (nb == p.block_elems)
        encode_stream<true>(p, st, n_s, r0, s_bits, s_len, col);
    else
        encode_stream<false>(p, st, n_s, r0, s_bits, s_len, col);
    BlockOut o{p.pay + (uint64_t)b * cap * NS, p.cnt + (uint64_t)b * NS, p.obase, p.ovf,
               p.ovf_cap, p.status, p.scratch, p.scratch + scr_stage_offset(p.nblk), p.ovf_cap,
               p.nblk};
    __syncthreads();
    writer_finish(st, n_s, b, cap, s_pay, col, s_tmp, &s_ob, o);
}

template <bool FULL>
__device__ __forceinline__ void decode_stream(const DecodeParams &p, uint32_t n_s, uint32_t c_s,
                                              uint64_t r0, uint64_t sp0, const uint32_t *col,
                                              const uint8_t *s_sym, const uint8_t *s_len,
                                              const uint8_t *s_msk) {
    const uint32_t s = threadIdx.x;
    const uint32_t npos = p.block_elems / NS;
    const uint32_t cap = p.cap_words;
    const uint32_t esc = p.dec.esc_len;
    const uint8_t *sfs = p.sf + r0 + s;
    uint16_t *ys = p.y + r0 + s;
    Reader rd;
    rd.init(col, cap);
    uint32_t f[kChunk], fn[kChunk];
#pragma unroll
    for (uint32_t i = 0; i < kChunk; ++i) f[i] = (FULL || i < n_s) ? sfs[i * NS] : 0;
    for (uint32_t j0 = 0; j0 < npos; j0 += kChunk) {
        if (j0 + kChunk < npos) {
#pragma unroll
            for (uint32_t i = 0; i < kChunk; ++i) {
                const uint32_t j = j0 + kChunk + i;
                fn[i] = (FULL || j < n_s) ? sfs[j * NS] : 0;
            }
        }
#pragma unroll
        for (uint32_t i = 0; i < kChunk; ++i) {
            const uint32_t j = j0 + i;
            uint32_t e = rd.next(s_sym, s_len, s_msk, esc);
            if (j >= c_s && (FULL || j < n_s)) {
                const uint64_t k = sp0 + (j - c_s);
                e = k < p.ovf_cap ? p.ovf[k] : 0;
            }
            if (FULL || j < n_s) ys[j * NS] = (uint16_t)join16(f[i], e);
            if (i & 1) rd.refill(col, cap);
        }
#pragma unroll
        for (uint32_t i = 0; i < kChunk; ++i) f[i] = fn[i];
    }
}

__global__ __launch_bounds__(256) void k_decode(const DecodeParams p) {
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_tmp[4];
    const uint32_t s = threadIdx.x, b = blockIdx.x;
    const uint32_t cap = p.cap_words;
    uint32_t *s_pay = lds;                                        // (cap + 1) rows
    uint8_t *s_sym = reinterpret_cast<uint8_t *>(lds + (cap + 1) * NS);
    uint8_t *s_len = s_sym + NS;
    uint8_t *s_msk = s_len + NS;
    stage_dec(p.dec, s_sym, s_len, s_msk);
    stage_payload(p.pay + (uint64_t)b * cap * NS, cap, s_pay);
    const uint64_t r0 = (uint64_t)b * p.block_elems;
    const uint32_t nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
    const uint32_t n_s = stream_len(nb, s);
    const uint32_t c_s = min<uint32_t>(p.cnt[(uint64_t)b * NS + s], n_s);
    uint32_t total;
    const uint32_t excl = block_excl_scan(n_s - c_s, s_tmp, total);   // barriers also publish LDS
    const uint64_t sp0 = p.obase[b] + excl;
    if (nb == p.block_elems)
        decode_stream<true>(p, n_s, c_s, r0, sp0, s_pay + s, s_sym, s_len, s_msk);
    else
        decode_stream<false>(p, n_s, c_s, r0, sp0, s_pay + s, s_sym, s_len, s_msk);
}

// One SGD element: rne_bf16(fmaf(-eta, m, w)); NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t sgd_elem(uint32_t w16, uint32_t m16, float neg_eta) {
    const float w = __uint_as_float(w16 << 16);
    const float m = __uint_as_float(m16 << 16);
    const uint32_t u = __float_as_uint(__builtin_fmaf(neg_eta, m, w));
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool FULL>
__device__ __forceinline__ void sgd_stream(const SgdParams &p, Writer &st, uint32_t n_s,
                                           uint32_t cw_s, uint32_t cm_s, uint64_t r0, uint64_t wsp,
                                           uint64_t msp, const uint32_t *wcol, const uint32_t *mcol,
                                           uint32_t *ocol, const uint8_t *s_wd, const uint8_t *s_md,
                                           const uint32_t *s_bits, const uint8_t *s_elen) {
    const uint32_t s = threadIdx.x;
    const uint32_t npos = p.block_elems / NS;
    const uint32_t cap = p.cap_words;
    const uint32_t capbits = 32 * cap;
    const uint32_t wesc = p.wdec.esc_len, mesc = p.mdec.esc_len;
    const uint8_t *wsf = p.w_sf + r0 + s;
    const uint8_t *msf = p.m_sf + r0 + s;
    uint8_t *osf = p.o_sf + r0 + s;
    uint64_t *stage_ctr = reinterpret_cast<uint64_t *>(p.scratch + kScrStage);
    uint8_t *stage = p.scratch + scr_stage_offset(p.nblk);
    Reader rw, rm;
    rw.init(wcol, cap);
    rm.init(mcol, cap);
    uint32_t fw[kChunk], fm[kChunk], fwn[kChunk], fmn[kChunk];
#pragma unroll
    for (uint32_t i = 0; i < kChunk; ++i) {
        fw[i] = (FULL || i < n_s) ? wsf[i * NS] : 0;
        fm[i] = (FULL || i < n_s) ? msf[i * NS] : 0;
    }
    for (uint32_t j0 = 0; j0 < npos; j0 += kChunk) {
        if (j0 + kChunk < npos) {
#pragma unroll
            for (uint32_t i = 0; i < kChunk; ++i) {
                const uint32_t j = j0 + kChunk + i;
                fwn[i] = (FULL || j < n_s) ? wsf[j * NS] : 0;
                fmn[i] = (FULL || j < n_s) ? msf[j * NS] : 0;
            }
        }
        uint32_t e[kChunk];
#pragma unroll
        for (uint32_t i = 0; i < kChunk; ++i) {
            const uint32_t j = j0 + i;
            uint32_t ew = rw.next(s_wd, s_wd + NS, s_wd + 2 * NS, wesc);
            uint32_t em = rm.next(s_md, s_md + NS, s_md + 2 * NS, mesc);
            if (j >= cw_s && (FULL || j < n_s)) {
                const uint64_t k = wsp + (j - cw_s);
                ew = k < p.w_ovf_cap ? p.w_ovf[k] : 0;
            }
            if (j >= cm_s && (FULL || j < n_s)) {
                const uint64_t k = msp + (j - cm_s);
                em = k < p.m_ovf_cap ? p.m_ovf[k] : 0;
            }
            const uint32_t w2 = sgd_elem(join16(fw[i], ew), join16(fm[i], em), p.neg_eta);
            if (FULL || j < n_s) osf[j * NS] = (uint8_t)sf_byte(w2);
            e[i] = (w2 >> 7) & 0xFFu;
            if (i & 1) {
                rw.refill(wcol, cap);
                rm.refill(mcol, cap);
            }
        }
        writer_chunk<FULL>(st, e, j0, n_s, capbits, s_bits, s_elen, ocol);
        writer_spill<FULL>(st, e, j0, n_s, stage_ctr, stage, p.ovf_cap);
#pragma unroll
        for (uint32_t i = 0; i < kChunk; ++i) {
            fw[i] = fwn[i];
            fm[i] = fmn[i];
        }
    }
}

__global__ __launch_bounds__(256) void k_sgd(const SgdParams p) {
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_tmp[4];
    __shared__ uint32_t s_ticket;
    __shared__ uint64_t s_ob;
    const uint32_t s = threadIdx.x;
    const uint32_t cap = p.cap_words;
    const uint32_t rows = cap + 1;
    uint32_t *s_wpay = lds;                       // W, M: cap rows + a zero row
    uint32_t *s_mpay = lds + rows * NS;
    uint32_t *s_opay = lds + 2 * rows * NS;       // W': cap rows + a sink row
    uint32_t *s_bits = lds + 3 * rows * NS;
    uint8_t *s_elen = reinterpret_cast<uint8_t *>(s_bits + NS);
    uint8_t *s_wd = s_elen + NS;                  // field, bits, mask tables of W
    uint8_t *s_md = s_wd + 3 * NS;                // same for M
    s_bits[s] = p.wenc.bits[s];
    s_elen[s] = p.wenc.len[s];
    stage_dec(p.wdec, s_wd, s_wd + NS, s_wd + 2 * NS);
    stage_dec(p.mdec, s_md, s_md + NS, s_md + 2 * NS);
    if (s == 0) s_ticket = atomicAdd(reinterpret_cast<uint32_t *>(p.scratch + kScrTicket), 1u);
    __syncthreads();
    const uint32_t b = s_ticket;
    if (b >= p.nblk) return;   // only if the scratch header was not cleared
    stage_payload(p.w_pay + (uint64_t)b * cap * NS, cap, s_wpay);
    stage_payload(p.m_pay + (uint64_t)b * cap * NS, cap, s_mpay);
    uint32_t *ocol = s_opay + s;
    for (uint32_t w = 0; w <= cap; ++w) ocol[w * NS] = 0;
    const uint64_t r0 = (uint64_t)b * p.block_elems;
    const uint32_t nb = (uint32_t)min<uint64_t>(p.block_elems, p.n - r0);
    const uint32_t n_s = stream_len(nb, s);
    const uint32_t cw_s = min<uint32_t>(p.w_cnt[(uint64_t)b * NS + s], n_s);
    const uint32_t cm_s = min<uint32_t>(p.m_cnt[(uint64_t)b * NS + s], n_s);
    uint32_t wtot, mtot;
    const uint32_t wex = block_excl_scan(n_s - cw_s, s_tmp, wtot);
    const uint32_t mex = block_excl_scan(n_s - cm_s, s_tmp, mtot);
    const uint64_t wsp = p.w_obase[b] + wex, msp = p.m_obase[b] + mex;
    Writer st;
    st.init(n_s);
    if (nb == p.block_elems)
        sgd_stream<true>(p, st, n_s, cw_s, cm_s, r0, wsp, msp, s_wpay + s, s_mpay + s, ocol, s_wd,
                         s_md, s_bits, s_elen);
    else
        sgd_stream<false>(p, st, n_s, cw_s, cm_s, r0, wsp, msp, s_wpay + s, s_mpay + s, ocol, s_wd,
                          s_md, s_bits, s_elen);
    BlockOut o{p.o_pay + (uint64_t)b * cap * NS, p.o_cnt + (uint64_t)b * NS, p.o_obase, p.o_ovf,
               p.ovf_cap, p.status, p.scratch, p.scratch + scr_stage_offset(p.nblk), p.ovf_cap,
               p.nblk};
    // every lane has read W's payload, counts and offsets before any is overwritten
    __syncthreads();
    writer_finish(st, n_s, b, cap, s_opay, ocol, s_tmp, &s_ob, o);
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

size_t encode_lds(uint32_t cap) { return (size_t)(cap + 1) * NS * 4 + NS * 4 + NS; }
size_t decode_lds(uint32_t cap) { return (size_t)(cap + 1) * NS * 4 + 3 * NS; }
size_t sgd_lds(uint32_t cap) { return (size_t)3 * (cap + 1) * NS * 4 + NS * 4 + NS + 6 * NS; }

int launch_clear(uint8_t *scratch, uint64_t nblk, uint32_t *status, void *stream) {
    const uint64_t words = scr_clear_bytes(nblk) / 8;
    const uint32_t grid = (uint32_t)((words + 255) / 256);
    hipLaunchKernelGGL(k_clear, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<uint64_t *>(scratch), words, status);
    return (int)hipGetLastError();
}

int launch_encode(const EncodeParams &p, void *stream) {
    const int attr = ensure_lds(k_encode, encode_lds(p.cap_words), g_enc_lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_encode, dim3(p.nblk), dim3(NS), encode_lds(p.cap_words), (hipStream_t)stream, p);
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
    hipLaunchKernelGGL(k_sgd, dim3(p.nblk), dim3(NS), sgd_lds(p.cap_words), (hipStream_t)stream, p);
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
