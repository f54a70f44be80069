// api.cpp -- the extern "C" entry points declared in include/lct.h:
// argument checks, size accounting and kernel launches.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <vector>

#include "lct_internal.h"

namespace {

using namespace lct;

thread_local char g_hip_msg[256] = "";

lct_status hip_fail(int err, const char *what) {
    snprintf(g_hip_msg, sizeof g_hip_msg, "%s: %s", what, hipGetErrorString((hipError_t)err));
    return LCT_EHIP;
}

// gfx950 check, cached per device.
lct_status check_arch() {
    static std::mutex mu;
    static int known[64] = {0};   // 0 unknown, 1 ok, -1 other arch
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return LCT_EARCH;
    std::lock_guard<std::mutex> lock(mu);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return known[dev] == 1 ? LCT_OK : LCT_EARCH;
}

bool layout_ok(const lct_layout &l) {
    return l.block_elems >= kMinBlock && l.block_elems <= kMaxBlock &&
           l.block_elems % kMinBlock == 0 && l.cap_words >= 1 && l.cap_words <= kMaxCapWords;
}

uint64_t nblocks(uint64_t n, const lct_layout &l) { return (n + l.block_elems - 1) / l.block_elems; }

// The largest sizes a call accepts, so that no size or address computed from
// them wraps: n elements (blocks are indexed by 32 bits) and ovf_cap bytes.
constexpr uint64_t kMaxElems = 1ull << 48;
constexpr uint64_t kMaxOvfCap = 1ull << 56;
bool sizes_ok(uint64_t n, const lct_layout &l, uint64_t ovf_cap) {
    return n <= kMaxElems && nblocks(n, l) <= 0xFFFFFFFFull && ovf_cap <= kMaxOvfCap;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};
Range rng(const void *p, uint64_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

struct Parts {
    Range sf, pay, cnt, obase, ovf, status, scratch;
};

// The ranges of a tensor's buffers; nb overrides the block count (a group's
// storage has more blocks than its n implies).
Parts parts(const lct_tensor &t, uint64_t nb = ~0ull) {
    if (nb == ~0ull) nb = nblocks(t.n, t.layout);
    Parts p;
    p.sf = rng(t.sf, t.n);
    p.pay = rng(t.pay, nb * t.layout.cap_words * kStreams * 4);
    p.cnt = rng(t.cnt, nb * kStreams * 2);
    p.obase = rng(t.obase, (nb + 1) * 8);
    p.ovf = rng(t.ovf, t.ovf_cap);
    p.status = rng(t.status, 4);
    p.scratch = rng(t.scratch, scr_bytes(nb, t.ovf_cap));
    return p;
}

// Pointers a call reads or writes must be non-null and aligned.
lct_status check_tensor(const lct_tensor *t, bool writes, uint64_t nb = ~0ull) {
    if (!t || !layout_ok(t->layout) || !sizes_ok(t->n, t->layout, t->ovf_cap)) return LCT_EINVAL;
    if (nb != ~0ull && nb > 0xFFFFFFFFull) return LCT_EINVAL;
    if (!t->sf || !t->pay || !t->cnt || !t->obase) return LCT_EINVAL;
    if (t->ovf_cap && !t->ovf) return LCT_EINVAL;
    if (!aligned(t->sf, 16) || !aligned(t->pay, 16) || !aligned(t->cnt, 4) || !aligned(t->obase, 8))
        return LCT_EALIGN;
    if (writes) {
        if (!t->status || !t->scratch) return LCT_EINVAL;
        if (!aligned(t->status, 4) || !aligned(t->scratch, 256)) return LCT_EALIGN;
        // the output's own parts must be disjoint
        const Parts p = parts(*t, nb);
        const Range all[] = {p.sf, p.pay, p.cnt, p.obase, p.ovf, p.status, p.scratch};
        for (int i = 0; i < 7; ++i)
            for (int j = i + 1; j < 7; ++j)
                if (overlap(all[i], all[j])) return LCT_EALIAS;
    }
    return LCT_OK;
}

bool overlaps_any(Range r, const Parts &p, bool with_writable = true) {
    const Range all[] = {p.sf, p.pay, p.cnt, p.obase, p.ovf};
    for (const Range &a : all)
        if (overlap(r, a)) return true;
    if (with_writable && (overlap(r, p.status) || overlap(r, p.scratch))) return true;
    return false;
}

std::mutex g_sample_mu;

// ---- groups

uint64_t shape_hash(uint32_t count, const uint64_t *n, const lct_layout &l) {
    uint64_t h = 1469598103934665603ull;   // FNV-1a over the layout and sizes
    auto mix = [&](uint64_t v) {
        for (int i = 0; i < 8; ++i) {
            h ^= (v >> (8 * i)) & 0xFF;
            h *= 1099511628211ull;
        }
    };
    mix(l.block_elems);
    mix(l.cap_words);
    mix(count);
    for (uint32_t k = 0; k < count; ++k) mix(n[k]);
    return h;
}

uint64_t round256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// The group's block count and sf bytes; false on overflow of the 32-bit block index.
bool group_extent(uint32_t count, const uint64_t *n, const lct_layout &l, uint64_t *nblk, uint64_t *sf) {
    uint64_t nb = 0, s = 0;
    for (uint32_t k = 0; k < count; ++k) {
        if (n[k] > kMaxElems) return false;
        nb += nblocks(n[k], l);
        if (nb > 0xFFFFFFFFull) return false;   // checked as it grows: it cannot wrap
        s += round256(n[k]);
    }
    *nblk = nb;
    *sf = s;
    return true;
}

GroupRef group_ref(const lct_group &g) {
    const GroupTableLayout t = group_table_layout(g.count, g.nblk);
    const uint8_t *base = static_cast<const uint8_t *>(g.d_table);
    return {reinterpret_cast<const GroupEntry *>(base + t.ent), reinterpret_cast<const EncTab *>(base + t.enc),
            reinterpret_cast<const DecTab *>(base + t.dec), reinterpret_cast<const uint32_t *>(base + t.blk_tensor),
            reinterpret_cast<const uint32_t *>(base + t.blk_tab)};
}

// A bound group and storage sized for it.
lct_status check_group(const lct_group *g, const lct_tensor *all, bool writes) {
    if (!g || !all || !g->d_table || !g->n || g->count == 0 || !layout_ok(g->layout)) return LCT_EINVAL;
    if (all->n != g->sf_bytes || all->layout.block_elems != g->layout.block_elems ||
        all->layout.cap_words != g->layout.cap_words)
        return LCT_EINVAL;
    uint64_t nb = 0, sf = 0;
    if (!group_extent(g->count, g->n, g->layout, &nb, &sf) || nb != g->nblk || sf != g->sf_bytes ||
        shape_hash(g->count, g->n, g->layout) != g->shape_hash)
        return LCT_EINVAL;
    return check_tensor(all, writes, g->nblk);
}

// Every dense buffer of the group, disjoint from the storage's parts.
lct_status check_group_dense(const lct_group &g, const Parts &p) {
    if (!g.d_dense) return LCT_EINVAL;
    for (uint32_t k = 0; k < g.count; ++k) {
        if (g.n[k] == 0) continue;
        if (!g.d_dense[k]) return LCT_EINVAL;
        if (!aligned(g.d_dense[k], 16)) return LCT_EALIGN;
        if (overlaps_any(rng(g.d_dense[k], g.n[k] * 2), p)) return LCT_EALIAS;
    }
    return LCT_OK;
}

// The buffers of an update: W and M (both decoded) and the result.
void sgd_params(SgdParams &p, const lct_tensor &w_in, const lct_tensor &m, const lct_tensor &w_out,
                uint64_t nb, float mul) {
    p.w_sf = w_in.sf;
    p.w_pay = w_in.pay;
    p.w_cnt = w_in.cnt;
    p.w_obase = w_in.obase;
    p.w_ovf = w_in.ovf;
    p.w_ovf_cap = w_in.ovf_cap;
    p.m_sf = m.sf;
    p.m_pay = m.pay;
    p.m_cnt = m.cnt;
    p.m_obase = m.obase;
    p.m_ovf = m.ovf;
    p.m_ovf_cap = m.ovf_cap;
    p.o_sf = w_out.sf;
    p.o_pay = w_out.pay;
    p.o_cnt = w_out.cnt;
    p.o_obase = w_out.obase;
    p.o_ovf = w_out.ovf;
    p.ovf_cap = w_out.ovf_cap;
    p.status = w_out.status;
    p.scratch = (uint8_t *)w_out.scratch;
    p.n = w_in.n;
    p.block_elems = w_in.layout.block_elems;
    p.cap_words = w_in.layout.cap_words;
    p.nblk = (uint32_t)nb;
    p.mul = mul;
    p.park_cnt = p.o_cnt == p.w_cnt;
}

// Clear, update, scan.
lct_status sgd_launch(const SgdParams &p, uint64_t nb, bool group, void *stream) {
    int e = launch_clear(p.scratch, nb, p.status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear launch");
    e = launch_sgd(p, stream, group);
    if (e != hipSuccess) return hip_fail(e, "sgd launch");
    e = launch_scan(p.scratch, nb, p.o_obase, p.o_ovf, p.ovf_cap, p.status, p.o_cnt, stream);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    return LCT_OK;
}

// The buffers of a fused momentum step.
void mom_params(MomParams &p, const lct_tensor &w_in, const lct_tensor &m_in, const uint16_t *g,
                const lct_tensor &w_out, const lct_tensor &m_out, uint64_t nb, float mu, float eta) {
    p.w_sf = w_in.sf;
    p.w_pay = w_in.pay;
    p.w_cnt = w_in.cnt;
    p.w_obase = w_in.obase;
    p.w_ovf = w_in.ovf;
    p.w_ovf_cap = w_in.ovf_cap;
    p.m_sf = m_in.sf;
    p.m_pay = m_in.pay;
    p.m_cnt = m_in.cnt;
    p.m_obase = m_in.obase;
    p.m_ovf = m_in.ovf;
    p.m_ovf_cap = m_in.ovf_cap;
    p.g = g;
    p.ow_sf = w_out.sf;
    p.ow_pay = w_out.pay;
    p.ow_cnt = w_out.cnt;
    p.ow_obase = w_out.obase;
    p.ow_ovf = w_out.ovf;
    p.ow_ovf_cap = w_out.ovf_cap;
    p.ow_status = w_out.status;
    p.ow_scratch = (uint8_t *)w_out.scratch;
    p.om_sf = m_out.sf;
    p.om_pay = m_out.pay;
    p.om_cnt = m_out.cnt;
    p.om_obase = m_out.obase;
    p.om_ovf = m_out.ovf;
    p.om_ovf_cap = m_out.ovf_cap;
    p.om_status = m_out.status;
    p.om_scratch = (uint8_t *)m_out.scratch;
    p.n = w_in.n;
    p.block_elems = w_in.layout.block_elems;
    p.cap_words = w_in.layout.cap_words;
    p.nblk = (uint32_t)nb;
    p.mu = mu;
    p.neg_eta = -eta;
    p.park_w = p.ow_cnt == p.w_cnt;
    p.park_m = p.om_cnt == p.m_cnt;
}

// Clear both outputs' scratch headers and status words, the fused kernel,
// both outputs' overflow scans.
lct_status mom_launch(const MomParams &p, uint64_t nb, bool group, void *stream) {
    int e = launch_clear(p.ow_scratch, nb, p.ow_status, stream);
    if (e == hipSuccess) e = launch_clear(p.om_scratch, nb, p.om_status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear launch");
    e = launch_mom(p, stream, group);
    if (e != hipSuccess) return hip_fail(e, "momentum launch");
    e = launch_scan(p.ow_scratch, nb, p.ow_obase, p.ow_ovf, p.ow_ovf_cap, p.ow_status, p.ow_cnt, stream);
    if (e == hipSuccess)
        e = launch_scan(p.om_scratch, nb, p.om_obase, p.om_ovf, p.om_ovf_cap, p.om_status, p.om_cnt, stream);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    return LCT_OK;
}

// The momentum step's aliasing rules (nb: the block count, ~0 for n's): the
// outputs are disjoint from each other; each output's fixed side is its own
// input's buffers, exactly, or disjoint from every input; its overflow,
// status and scratch overlap no input.
bool momentum_alias_ok(const lct_tensor &w_in, const lct_tensor &m_in, const lct_tensor &w_out,
                       const lct_tensor &m_out, uint64_t nb) {
    const Parts pw = parts(w_in, nb), pm = parts(m_in, nb), qw = parts(w_out, nb), qm = parts(m_out, nb);
    const Range qws[] = {qw.sf, qw.pay, qw.cnt, qw.obase, qw.ovf, qw.status, qw.scratch};
    for (const Range &r : qws)
        if (overlaps_any(r, qm)) return false;
    auto check_out = [&](const Parts &own, const Parts &other, const Parts &q) {
        const Range in[] = {own.sf, own.pay, own.cnt, own.obase};
        const Range out[] = {q.sf, q.pay, q.cnt, q.obase};
        for (int i = 0; i < 4; ++i) {
            for (int j = 0; j < 4; ++j) {
                const bool same = i == j && in[i].lo == out[j].lo;
                if (!same && overlap(in[i], out[j])) return false;
            }
            if (overlap(own.ovf, out[i])) return false;
            if (overlaps_any(out[i], other, false)) return false;
        }
        const Range rest[] = {q.ovf, q.status, q.scratch};
        for (const Range &r : rest)
            if (overlaps_any(r, own, false) || overlaps_any(r, other, false)) return false;
        return true;
    };
    return check_out(pw, pm, qw) && check_out(pm, pw, qm);
}

// Aliasing rules, parameters and launches of an update (a tensor, or a
// group's storage when `group`); p's tables (or group references) are set.
lct_status sgd_run(SgdParams &p, const lct_tensor &w_in, const lct_tensor &m, const lct_tensor &w_out,
                   uint64_t nb, float eta, bool group, void *stream) {
    const Parts pw = parts(w_in, nb), pm = parts(m, nb), po = parts(w_out, nb);
    // M is read-only and must not share memory with the output
    const Range mr[] = {pm.sf, pm.pay, pm.cnt, pm.obase, pm.ovf};
    for (const Range &r : mr)
        if (overlaps_any(r, po)) return LCT_EALIAS;
    // the output's fixed side may be W's own buffers, exactly, or disjoint from W
    const Range wf[] = {pw.sf, pw.pay, pw.cnt, pw.obase};
    const Range of[] = {po.sf, po.pay, po.cnt, po.obase};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j) {
            const bool same = i == j && wf[i].lo == of[j].lo;
            if (!same && overlap(wf[i], of[j])) return LCT_EALIAS;
        }
        if (overlap(pw.ovf, of[i])) return LCT_EALIAS;
    }
    // overflow, status and scratch of the output never overlap an input
    const Range ow[] = {po.ovf, po.status, po.scratch};
    for (const Range &r : ow)
        if (overlaps_any(r, pw, false) || overlaps_any(r, pm, false)) return LCT_EALIAS;
    lct_status st = check_arch();
    if (st != LCT_OK) return st;
    sgd_params(p, w_in, m, w_out, nb, -eta);
    return sgd_launch(p, nb, group, stream);
}

}  // namespace

extern "C" {

lct_status lct_layout_init(int32_t mode, lct_layout *out) {
    if (!out) return LCT_EINVAL;
    switch (mode) {
    case LCT_CLEAN: *out = {65536, 25}; return LCT_OK;
    case LCT_MEDIUM: *out = {32768, 12}; return LCT_OK;
    case LCT_HIGH: *out = {32768, 11}; return LCT_OK;
    }
    return LCT_EINVAL;
}

lct_status lct_sizes(uint64_t n, const lct_layout *layout, uint64_t ovf_cap, lct_sizes_t *out) {
    if (!layout || !out || !layout_ok(*layout) || !sizes_ok(n, *layout, ovf_cap)) return LCT_EINVAL;
    const uint64_t nb = nblocks(n, *layout);
    out->nblk = nb;
    out->sf = n;
    out->pay = nb * layout->cap_words * kStreams * 4;
    out->cnt = nb * kStreams * 2;
    out->obase = (nb + 1) * 8;
    out->scratch = scr_bytes(nb, ovf_cap);
    out->fixed = out->sf + out->pay + out->cnt + out->obase;
    return LCT_OK;
}

lct_status lct_codebook_build(const lct_model *model, const uint16_t *d_x, uint64_t n, void *stream,
                              lct_codebook *out) {
    if (!model || !out || (n > 0 && !d_x) || n > kMaxElems) return LCT_EINVAL;
    const uint32_t m = (uint32_t)std::min<uint64_t>(n, 4096);
    uint16_t sample[4096];
    if (m > 0) {
        lct_status st = check_arch();
        if (st != LCT_OK) return st;
        std::lock_guard<std::mutex> lock(g_sample_mu);
        const int e = launch_gather(d_x, n, m, stream, sample);
        if (e != hipSuccess) return hip_fail(e, "sample gather");
    }
    return build_codebook(*model, sample, m, out);
}

lct_status lct_codebook_from_lengths(const uint8_t len_base[256], uint8_t esc_len, int32_t shift,
                                     lct_codebook *out) {
    return codebook_from_lengths(len_base, esc_len, shift, out);
}

lct_status lct_tensor_sample(const lct_codebook *cb, const lct_tensor *t, void *stream,
                             uint16_t *sample, uint32_t *m_out) {
    if (!cb || !t || !sample || !tables_ok(*cb)) return LCT_EINVAL;
    const uint32_t m = (uint32_t)std::min<uint64_t>(t->n, 4096);
    if (m > 0) {
        lct_status st = check_tensor(t, false);
        if (st != LCT_OK) return st;
        if (t->n >= (1ull << 52)) return LCT_EINVAL;   // i * n stays within 64 bits
        st = check_arch();
        if (st != LCT_OK) return st;
        SampleParams p;
        memset(&p, 0, sizeof p);
        p.sf = t->sf;
        p.pay = t->pay;
        p.cnt = t->cnt;
        p.obase = t->obase;
        p.ovf = t->ovf;
        p.ovf_cap = t->ovf_cap;
        p.n = t->n;
        p.block_elems = t->layout.block_elems;
        p.cap_words = t->layout.cap_words;
        p.m = m;
        fill_dec(*cb, &p.dec);
        std::lock_guard<std::mutex> lock(g_sample_mu);
        const int e = launch_sample(p, stream, sample);
        if (e != hipSuccess) return hip_fail(e, "compressed sample");
    }
    if (m_out) *m_out = m;
    return LCT_OK;
}

lct_status lct_codebook_reshift(const lct_codebook *cb, const lct_tensor *t, void *stream,
                                lct_codebook *out) {
    if (!cb || !t || !out || !tables_ok(*cb)) return LCT_EINVAL;
    uint16_t sample[4096];
    uint32_t m = 0;
    const lct_status st = lct_tensor_sample(cb, t, stream, sample, &m);
    if (st != LCT_OK) return st;
    return reshift_codebook(*cb, sample, m, out);
}

lct_status lct_codebook_reshift_dense(const lct_codebook *cb, const uint16_t *d_x, uint64_t n,
                                      void *stream, lct_codebook *out) {
    if (!cb || !out || (n > 0 && !d_x) || n > kMaxElems || !tables_ok(*cb)) return LCT_EINVAL;
    const uint32_t m = (uint32_t)std::min<uint64_t>(n, 4096);
    uint16_t sample[4096];
    if (m > 0) {
        lct_status st = check_arch();
        if (st != LCT_OK) return st;
        std::lock_guard<std::mutex> lock(g_sample_mu);
        const int e = launch_gather(d_x, n, m, stream, sample);
        if (e != hipSuccess) return hip_fail(e, "sample gather");
    }
    return reshift_codebook(*cb, sample, m, out);
}

lct_status lct_codebook_adapt(const lct_codebook *cb, const lct_tensor *t, double max_spill_per_elem,
                              void *stream, lct_codebook *out, int32_t *changed) {
    if (!cb || !t || !out || !(max_spill_per_elem >= 0) || !tables_ok(*cb)) return LCT_EINVAL;
    const lct_codebook in = *cb;   // out may be cb
    bool reshift = false;
    if (t->n > 0) {
        lct_status st = check_tensor(t, false);
        if (st != LCT_OK) return st;
        st = check_arch();
        if (st != LCT_OK) return st;
        uint64_t spilled = 0;
        hipStream_t hs = (hipStream_t)stream;
        hipError_t e = hipMemcpyAsync(&spilled, t->obase + nblocks(t->n, t->layout), sizeof spilled,
                                      hipMemcpyDeviceToHost, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        if (e != hipSuccess) return hip_fail(e, "spill total read");
        reshift = (double)spilled > max_spill_per_elem * (double)t->n;
    }
    if (reshift) {
        lct_status st = lct_codebook_reshift(&in, t, stream, out);
        if (st != LCT_OK) return st;
    } else {
        *out = in;
    }
    if (changed) *changed = out->shift != in.shift;
    return LCT_OK;
}

lct_status lct_encode(const lct_codebook *cb, const uint16_t *d_x, const lct_tensor *out,
                      void *stream) {
    if (!cb || !out || !tables_ok(*cb)) return LCT_EINVAL;
    if (out->n == 0) return LCT_OK;
    lct_status st = check_tensor(out, true);
    if (st != LCT_OK) return st;
    if (!d_x) return LCT_EINVAL;
    if (!aligned(d_x, 16)) return LCT_EALIGN;
    if (overlaps_any(rng(d_x, out->n * 2), parts(*out))) return LCT_EALIAS;
    st = check_arch();
    if (st != LCT_OK) return st;

    const uint64_t nb = nblocks(out->n, out->layout);
    if (nb > 0xFFFFFFFFull) return LCT_EINVAL;
    EncodeParams p;
    memset(&p, 0, sizeof p);
    p.x = d_x;
    p.n = out->n;
    p.block_elems = out->layout.block_elems;
    p.cap_words = out->layout.cap_words;
    p.nblk = (uint32_t)nb;
    p.sf = out->sf;
    p.pay = out->pay;
    p.cnt = out->cnt;
    p.obase = out->obase;
    p.ovf = out->ovf;
    p.ovf_cap = out->ovf_cap;
    p.status = out->status;
    p.scratch = (uint8_t *)out->scratch;
    fill_enc(*cb, &p.enc);
    int e = launch_clear(p.scratch, nb, p.status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear launch");
    e = launch_encode(p, stream);
    if (e != hipSuccess) return hip_fail(e, "encode launch");
    e = launch_scan(p.scratch, nb, p.obase, p.ovf, p.ovf_cap, p.status, p.cnt, stream);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    return LCT_OK;
}

lct_status lct_decode(const lct_codebook *cb, const lct_tensor *in, uint16_t *d_y, void *stream) {
    if (!cb || !in || !tables_ok(*cb)) return LCT_EINVAL;
    if (in->n == 0) return LCT_OK;
    lct_status st = check_tensor(in, false);
    if (st != LCT_OK) return st;
    if (!d_y) return LCT_EINVAL;
    if (!aligned(d_y, 16)) return LCT_EALIGN;
    if (overlaps_any(rng(d_y, in->n * 2), parts(*in), false)) return LCT_EALIAS;
    st = check_arch();
    if (st != LCT_OK) return st;
    const uint64_t nb = nblocks(in->n, in->layout);
    if (nb > 0xFFFFFFFFull) return LCT_EINVAL;
    DecodeParams p;
    memset(&p, 0, sizeof p);
    p.sf = in->sf;
    p.pay = in->pay;
    p.cnt = in->cnt;
    p.obase = in->obase;
    p.ovf = in->ovf;
    p.ovf_cap = in->ovf_cap;
    p.y = d_y;
    p.n = in->n;
    p.block_elems = in->layout.block_elems;
    p.cap_words = in->layout.cap_words;
    p.nblk = (uint32_t)nb;
    fill_dec(*cb, &p.dec);
    const int e = launch_decode(p, stream);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return LCT_OK;
}

lct_status lct_sgd_step(const lct_codebook *cw, const lct_tensor *w_in, const lct_codebook *cm,
                        const lct_tensor *m, float eta, const lct_tensor *w_out, void *stream) {
    return lct_sgd_step_recode(cw, w_in, cm, m, eta, cw, w_out, stream);
}

lct_status lct_sgd_step_recode(const lct_codebook *cw, const lct_tensor *w_in, const lct_codebook *cm,
                               const lct_tensor *m, float eta, const lct_codebook *cw_out,
                               const lct_tensor *w_out, void *stream) {
    if (!cw || !cm || !cw_out || !w_in || !m || !w_out) return LCT_EINVAL;
    if (!tables_ok(*cw) || !tables_ok(*cm) || !tables_ok(*cw_out)) return LCT_EINVAL;
    if (w_in->n != m->n || w_in->n != w_out->n) return LCT_EINVAL;
    if (w_in->layout.block_elems != m->layout.block_elems ||
        w_in->layout.block_elems != w_out->layout.block_elems ||
        w_in->layout.cap_words != m->layout.cap_words ||
        w_in->layout.cap_words != w_out->layout.cap_words)
        return LCT_EINVAL;
    if (w_in->n == 0) return LCT_OK;
    lct_status st = check_tensor(w_in, false);
    if (st == LCT_OK) st = check_tensor(m, false);
    if (st == LCT_OK) st = check_tensor(w_out, true);
    if (st != LCT_OK) return st;
    const uint64_t nb = nblocks(w_in->n, w_in->layout);
    if (nb > 0xFFFFFFFFull) return LCT_EINVAL;
    SgdParams p;
    memset(&p, 0, sizeof p);
    fill_enc(*cw_out, &p.wenc);
    fill_dec(*cw, &p.wdec);
    fill_dec(*cm, &p.mdec);
    return sgd_run(p, *w_in, *m, *w_out, nb, eta, false, stream);
}

lct_status lct_sgd_step_noalloc(const lct_codebook *cw, const lct_tensor *w_in, const lct_codebook *cm,
                                const lct_tensor *m, float eta, const lct_tensor *w_out, void *stream) {
    if (!cw || !cm || !w_in || !m || !w_out || !tables_ok(*cw) || !tables_ok(*cm)) return LCT_EINVAL;
    if (w_out->n == 0) return lct_sgd_step(cw, w_in, cm, m, eta, w_out, stream);
    if (!layout_ok(w_out->layout) || !sizes_ok(w_out->n, w_out->layout, w_out->ovf_cap)) return LCT_EINVAL;
    if (scr_bytes(nblocks(w_out->n, w_out->layout), w_out->ovf_cap) > kNoAllocScratch) return LCT_ESIZE;
    lct_status st = check_arch();
    if (st != LCT_OK) return st;
    uint8_t *scr = nullptr;
    const int e = noalloc_scratch(&scr);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    lct_tensor out = *w_out;
    out.scratch = scr;
    return lct_sgd_step(cw, w_in, cm, m, eta, &out, stream);
}

lct_status lct_momentum_step(const lct_codebook *cw, const lct_tensor *w_in, const lct_codebook *cm,
                             const lct_tensor *m_in, const uint16_t *d_g, float mu, float eta,
                             const lct_tensor *w_out, const lct_tensor *m_out, void *stream) {
    return lct_momentum_step_recode(cw, w_in, cm, m_in, d_g, mu, eta, cw, cm, w_out, m_out, stream);
}

lct_status lct_momentum_step_recode(const lct_codebook *cw, const lct_tensor *w_in,
                                    const lct_codebook *cm, const lct_tensor *m_in,
                                    const uint16_t *d_g, float mu, float eta,
                                    const lct_codebook *cw_out, const lct_codebook *cm_out,
                                    const lct_tensor *w_out, const lct_tensor *m_out, void *stream) {
    if (!cw || !cm || !cw_out || !cm_out || !w_in || !m_in || !w_out || !m_out) return LCT_EINVAL;
    if (!tables_ok(*cw) || !tables_ok(*cm) || !tables_ok(*cw_out) || !tables_ok(*cm_out)) return LCT_EINVAL;
    const lct_tensor *all[] = {w_in, m_in, w_out, m_out};
    for (const lct_tensor *t : all)
        if (t->n != w_in->n || t->layout.block_elems != w_in->layout.block_elems ||
            t->layout.cap_words != w_in->layout.cap_words)
            return LCT_EINVAL;
    if (w_in->n == 0) return LCT_OK;
    if (!d_g) return LCT_EINVAL;
    if (!aligned(d_g, 16)) return LCT_EALIGN;
    lct_status st = check_tensor(w_in, false);
    if (st == LCT_OK) st = check_tensor(m_in, false);
    if (st == LCT_OK) st = check_tensor(w_out, true);
    if (st == LCT_OK) st = check_tensor(m_out, true);
    if (st != LCT_OK) return st;
    if (overlaps_any(rng(d_g, w_in->n * 2), parts(*w_out)) || overlaps_any(rng(d_g, w_in->n * 2), parts(*m_out)))
        return LCT_EALIAS;   // the gradient is read only: no output may overlap it
    if (!momentum_alias_ok(*w_in, *m_in, *w_out, *m_out, ~0ull)) return LCT_EALIAS;
    st = check_arch();
    if (st != LCT_OK) return st;

    const uint64_t nb = nblocks(w_in->n, w_in->layout);
    if (nb > 0xFFFFFFFFull) return LCT_EINVAL;
    // One pass: W and M decoded, M' = rne(mu * M + g) and W' = rne(W - eta * M')
    // with M' as rounded, both re-encoded by the fused kernel.
    MomParams p;
    memset(&p, 0, sizeof p);
    mom_params(p, *w_in, *m_in, d_g, *w_out, *m_out, nb, mu, eta);
    fill_enc_packed(*cw_out, p.wenc);
    fill_enc_packed(*cm_out, p.menc);
    fill_dec(*cw, &p.wdec);
    fill_dec(*cm, &p.mdec);
    return mom_launch(p, nb, false, stream);
}

// ---- groups

lct_status lct_group_table_bytes(uint32_t count, const uint64_t *n, const lct_layout *layout,
                                 uint64_t *bytes) {
    if (!layout || !bytes || !layout_ok(*layout) || (count > 0 && !n)) return LCT_EINVAL;
    uint64_t nb = 0, sf = 0;
    if (!group_extent(count, n, *layout, &nb, &sf)) return LCT_EINVAL;
    *bytes = group_table_layout(count, nb).bytes;
    return LCT_OK;
}

lct_status lct_group_bind(uint32_t count, const uint64_t *n, const lct_layout *layout,
                          const lct_codebook *cbs, uint16_t *const *d_dense, void *d_table,
                          lct_group *out) {
    if (!layout || !out || !cbs || !n || !d_table || count == 0 || !layout_ok(*layout))
        return LCT_EINVAL;
    for (uint32_t k = 0; k < count; ++k)
        if (!tables_ok(cbs[k])) return LCT_EINVAL;
    if (!aligned(d_table, 256)) return LCT_EALIGN;
    uint64_t nb = 0, sf = 0;
    if (!group_extent(count, n, *layout, &nb, &sf)) return LCT_EINVAL;
    if (d_dense) {
        std::vector<Range> rs;
        for (uint32_t k = 0; k < count; ++k) {
            if (n[k] == 0) continue;
            if (!d_dense[k]) return LCT_EINVAL;
            if (!aligned(d_dense[k], 16)) return LCT_EALIGN;
            rs.push_back(rng(d_dense[k], n[k] * 2));
        }
        std::sort(rs.begin(), rs.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
        for (size_t i = 1; i < rs.size(); ++i)
            if (rs[i].lo < rs[i - 1].hi) return LCT_EALIAS;
    }
    lct_status st = check_arch();
    if (st != LCT_OK) return st;
    const GroupTableLayout t = group_table_layout(count, nb);
    std::vector<uint8_t> host(t.bytes, 0);
    auto *ent = reinterpret_cast<GroupEntry *>(host.data() + t.ent);
    auto *enc = reinterpret_cast<EncTab *>(host.data() + t.enc);
    auto *dec = reinterpret_cast<DecTab *>(host.data() + t.dec);
    auto *owner = reinterpret_cast<uint32_t *>(host.data() + t.blk_tensor);
    auto *tabs = reinterpret_cast<uint32_t *>(host.data() + t.blk_tab);
    // tensors whose tables are byte-identical share the first one's index
    std::map<std::vector<uint8_t>, uint32_t> first_with;
    uint64_t b0 = 0, e0 = 0;
    for (uint32_t k = 0; k < count; ++k) {
        const uint64_t nbk = nblocks(n[k], *layout);
        ent[k].dense = d_dense ? d_dense[k] : nullptr;
        ent[k].n = n[k];
        ent[k].e0 = e0;
        ent[k].blk0 = (uint32_t)b0;
        ent[k].nblk = (uint32_t)nbk;
        fill_enc(cbs[k], &enc[k]);
        fill_dec(cbs[k], &dec[k]);
        std::vector<uint8_t> key(sizeof(EncTab) + sizeof(DecTab));
        memcpy(key.data(), &enc[k], sizeof(EncTab));
        memcpy(key.data() + sizeof(EncTab), &dec[k], sizeof(DecTab));
        const uint32_t tab = first_with.emplace(std::move(key), k).first->second;
        for (uint64_t j = 0; j < nbk; ++j) {
            owner[b0 + j] = k;
            tabs[b0 + j] = tab;
        }
        b0 += nbk;
        e0 += round256(n[k]);
    }
    const hipError_t e = hipMemcpy(d_table, host.data(), t.bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "group table copy");
    out->count = count;
    out->layout = *layout;
    out->nblk = nb;
    out->sf_bytes = sf;
    out->shape_hash = shape_hash(count, n, *layout);
    out->n = n;
    out->d_dense = d_dense;
    out->d_table = d_table;
    return LCT_OK;
}

lct_status lct_group_fit(const lct_codebook *base, const uint64_t *n, uint16_t *const *d_dense,
                         const lct_layout *layout, void *d_table, int32_t *d_shift, void *stream,
                         lct_group *out) {
    if (!base || !n || !d_dense || !layout || !d_table || !out || !layout_ok(*layout)) return LCT_EINVAL;
    // the device builds the tables from the base code: its lengths must make one
    lct_codebook check;
    if (codebook_from_lengths(base->len_base, base->esc_len, 0, &check) != LCT_OK) return LCT_EINVAL;
    if (n[0] > 0 && !d_dense[0]) return LCT_EINVAL;
    if (!aligned(d_table, 256) || (n[0] > 0 && !aligned(d_dense[0], 16)) || (d_shift && !aligned(d_shift, 4)))
        return LCT_EALIGN;
    uint64_t nb = 0, sf = 0;
    if (!group_extent(1, n, *layout, &nb, &sf)) return LCT_EINVAL;
    lct_status st = check_arch();
    if (st != LCT_OK) return st;
    const GroupTableLayout t = group_table_layout(1, nb);
    uint8_t *tab = static_cast<uint8_t *>(d_table);
    FitParams p;
    memset(&p, 0, sizeof p);
    p.x = d_dense[0];
    p.n = n[0];
    p.m = (uint32_t)std::min<uint64_t>(n[0], 4096);
    p.nblk = (uint32_t)nb;
    p.esc_len = base->esc_len;
    memcpy(p.base, base->len_base, sizeof p.base);
    p.ent = reinterpret_cast<GroupEntry *>(tab + t.ent);
    p.enc = reinterpret_cast<EncTab *>(tab + t.enc);
    p.dec = reinterpret_cast<DecTab *>(tab + t.dec);
    p.blk_tensor = reinterpret_cast<uint32_t *>(tab + t.blk_tensor);
    p.blk_tab = reinterpret_cast<uint32_t *>(tab + t.blk_tab);
    p.shift_out = d_shift;
    const int e = launch_fit(p, stream);
    if (e != hipSuccess) return hip_fail(e, "fit launch");
    out->count = 1;
    out->layout = *layout;
    out->nblk = nb;
    out->sf_bytes = sf;
    out->shape_hash = shape_hash(1, n, *layout);
    out->n = n;
    out->d_dense = d_dense;
    out->d_table = d_table;
    return LCT_OK;
}

lct_status lct_group_sizes(const lct_group *g, uint64_t ovf_cap, lct_sizes_t *out) {
    if (!g || !out || !layout_ok(g->layout) || g->nblk > 0xFFFFFFFFull || ovf_cap > kMaxOvfCap)
        return LCT_EINVAL;
    out->nblk = g->nblk;
    out->sf = g->sf_bytes;
    out->pay = g->nblk * g->layout.cap_words * kStreams * 4;
    out->cnt = g->nblk * kStreams * 2;
    out->obase = (g->nblk + 1) * 8;
    out->scratch = scr_bytes(g->nblk, ovf_cap);
    out->fixed = out->sf + out->pay + out->cnt + out->obase;
    return LCT_OK;
}

lct_status lct_group_tensor(const lct_group *g, const lct_tensor *all, uint32_t k, lct_tensor *out) {
    if (!g || !all || !out || !g->n || k >= g->count) return LCT_EINVAL;
    uint64_t b0 = 0, e0 = 0;
    for (uint32_t j = 0; j < k; ++j) {
        b0 += nblocks(g->n[j], g->layout);
        e0 += round256(g->n[j]);
    }
    *out = *all;
    out->n = g->n[k];
    out->sf = all->sf + e0;
    out->pay = all->pay + b0 * g->layout.cap_words * kStreams;
    out->cnt = all->cnt + b0 * kStreams;
    out->obase = all->obase + b0;
    return LCT_OK;
}

lct_status lct_encode_group(const lct_group *g, const lct_tensor *all, void *stream) {
    lct_status st = check_group(g, all, true);
    if (st != LCT_OK) return st;
    st = check_group_dense(*g, parts(*all, g->nblk));
    if (st != LCT_OK) return st;
    st = check_arch();
    if (st != LCT_OK) return st;
    if (g->nblk == 0) return LCT_OK;
    EncodeParams p;
    memset(&p, 0, sizeof p);
    p.n = all->n;
    p.block_elems = g->layout.block_elems;
    p.cap_words = g->layout.cap_words;
    p.nblk = (uint32_t)g->nblk;
    p.sf = all->sf;
    p.pay = all->pay;
    p.cnt = all->cnt;
    p.obase = all->obase;
    p.ovf = all->ovf;
    p.ovf_cap = all->ovf_cap;
    p.status = all->status;
    p.scratch = (uint8_t *)all->scratch;
    p.grp = group_ref(*g);
    int e = launch_clear(p.scratch, g->nblk, p.status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear launch");
    e = launch_encode(p, stream, true);
    if (e != hipSuccess) return hip_fail(e, "group encode launch");
    e = launch_scan(p.scratch, g->nblk, p.obase, p.ovf, p.ovf_cap, p.status, p.cnt, stream);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    return LCT_OK;
}

lct_status lct_decode_group(const lct_group *g, const lct_tensor *all, void *stream) {
    lct_status st = check_group(g, all, false);
    if (st != LCT_OK) return st;
    st = check_group_dense(*g, parts(*all, g->nblk));
    if (st != LCT_OK) return st;
    st = check_arch();
    if (st != LCT_OK) return st;
    if (g->nblk == 0) return LCT_OK;
    DecodeParams p;
    memset(&p, 0, sizeof p);
    p.sf = all->sf;
    p.pay = all->pay;
    p.cnt = all->cnt;
    p.obase = all->obase;
    p.ovf = all->ovf;
    p.ovf_cap = all->ovf_cap;
    p.n = all->n;
    p.block_elems = g->layout.block_elems;
    p.cap_words = g->layout.cap_words;
    p.nblk = (uint32_t)g->nblk;
    p.grp = group_ref(*g);
    const int e = launch_decode(p, stream, true);
    if (e != hipSuccess) return hip_fail(e, "group decode launch");
    return LCT_OK;
}

lct_status lct_sgd_step_group(const lct_group *gw, const lct_tensor *w_all, const lct_group *gm,
                              const lct_tensor *m_all, float eta, const lct_tensor *w_out,
                              void *stream) {
    lct_status st = check_group(gw, w_all, false);
    if (st == LCT_OK) st = check_group(gm, m_all, false);
    if (st == LCT_OK) st = check_group(gw, w_out, true);
    if (st != LCT_OK) return st;
    if (gm->shape_hash != gw->shape_hash || gm->count != gw->count || gm->nblk != gw->nblk ||
        gm->sf_bytes != gw->sf_bytes)
        return LCT_EINVAL;
    for (uint32_t k = 0; k < gw->count; ++k)
        if (gw->n[k] != gm->n[k]) return LCT_EINVAL;
    if (gw->nblk == 0) return LCT_OK;
    SgdParams p;
    memset(&p, 0, sizeof p);
    p.gw = group_ref(*gw);
    p.gm = group_ref(*gm);
    return sgd_run(p, *w_all, *m_all, *w_out, gw->nblk, eta, true, stream);
}

lct_status lct_momentum_step_group(const lct_group *gw, const lct_tensor *w_all, const lct_group *gm,
                                   const lct_tensor *m_all, const lct_group *gg, float mu, float eta,
                                   const lct_tensor *w_out, const lct_tensor *m_out, void *stream) {
    lct_status st = check_group(gw, w_all, false);
    if (st == LCT_OK) st = check_group(gm, m_all, false);
    if (st == LCT_OK) st = check_group(gw, w_out, true);
    if (st == LCT_OK) st = check_group(gm, m_out, true);
    if (st != LCT_OK) return st;
    if (!gg || !gg->d_table || !gg->n) return LCT_EINVAL;
    for (const lct_group *o : {gm, gg}) {
        if (o->shape_hash != gw->shape_hash || o->count != gw->count || o->nblk != gw->nblk ||
            o->sf_bytes != gw->sf_bytes)
            return LCT_EINVAL;
        for (uint32_t k = 0; k < gw->count; ++k)
            if (o->n[k] != gw->n[k]) return LCT_EINVAL;
    }
    // the gradients (gg's dense buffers) are read only: no output may overlap them
    st = check_group_dense(*gg, parts(*w_out, gw->nblk));
    if (st == LCT_OK) st = check_group_dense(*gg, parts(*m_out, gw->nblk));
    if (st != LCT_OK) return st;
    if (!momentum_alias_ok(*w_all, *m_all, *w_out, *m_out, gw->nblk)) return LCT_EALIAS;
    st = check_arch();
    if (st != LCT_OK) return st;
    if (gw->nblk == 0) return LCT_OK;
    const uint64_t nb = gw->nblk;
    MomParams p;
    memset(&p, 0, sizeof p);
    mom_params(p, *w_all, *m_all, nullptr, *w_out, *m_out, nb, mu, eta);
    p.gw = group_ref(*gw);
    p.gm = group_ref(*gm);
    p.gg = group_ref(*gg);
    return mom_launch(p, nb, true, stream);
}

const char *lct_strerror(lct_status st) {
    switch (st) {
    case LCT_OK: return "ok";
    case LCT_EINVAL: return "invalid argument";
    case LCT_EALIGN: return "misaligned device pointer";
    case LCT_EALIAS: return "illegal buffer overlap";
    case LCT_EHIP: return "HIP runtime error";
    case LCT_EARCH: return "device is not gfx950";
    case LCT_ESIZE: return "working memory needed exceeds the static scratch of the allocation-free call";
    }
    return "unknown status";
}

const char *lct_last_hip_error(void) { return g_hip_msg; }

}  // extern "C"
