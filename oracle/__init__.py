"""ctypes view of the plain C oracle of the LCT codec (``lct_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package; the product
path never does.  Arrays are numpy arrays; every call is serial C.

Page citations are in ``lct_oracle.h``: "LCT: Losslessly Compressed Tensors
with GPU friendly execution for Training" (abstract) and the explainer "LCT
paper - Lossless Huffman coding of BF16 training tensors" (paragraphs on the
byte split and codebook, on blocks and streams, and on training traffic).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lct_oracle.c")
_LIB = os.path.join(_HERE, "liblct_oracle.so")
# A different build of the same source (the sanitizer test's) may be loaded
# instead; build() still writes the default one.
_LOAD = os.environ.get("LCT_ORACLE_LIB") or _LIB

GAUSSIAN, LAPLACE, POWERLAW = 0, 1, 2
OK, OVF_FULL, EINVAL, EDECODE = 0, 1, -1, -2
NSTREAM = 256


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Codebook(C.Structure):
    _fields_ = [("len", C.c_uint8 * 256), ("esc_len", C.c_uint8),
                ("shift", C.c_int32), ("code", C.c_uint32 * 257), ("len_base", C.c_uint8 * 256)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LOAD == _LIB and not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LOAD)
        P = C.c_void_p
        u64, u32, i32 = C.c_uint64, C.c_uint32, C.c_int
        L.lcto_model_survival.restype = C.c_double
        L.lcto_model_survival.argtypes = [i32, C.c_double, C.c_double, C.c_double]
        L.lcto_model_pmf.argtypes = [i32, C.c_double, C.c_double, P]
        L.lcto_weights.argtypes = [P, P]
        L.lcto_package_merge.argtypes = [i32, P, P, i32, P]
        L.lcto_build_escape.restype = u64
        L.lcto_build_escape.argtypes = [i32, P, i32, i32, P, P, P]
        L.lcto_build_base.restype = u64
        L.lcto_build_base.argtypes = [P, P, P, P]
        L.lcto_best_shift.argtypes = [P, C.c_uint8, P, C.c_size_t]
        L.lcto_shift_cost.restype = u64
        L.lcto_shift_cost.argtypes = [P, C.c_uint8, P, C.c_size_t, i32]
        L.lcto_canonical.argtypes = [P, P]
        L.lcto_codebook_build.argtypes = [i32, C.c_double, C.c_double, P, u64, P]
        L.lcto_codebook_from_base.argtypes = [P, C.c_uint8, i32, P]
        L.lcto_exponent.restype = C.c_uint8
        L.lcto_exponent.argtypes = [C.c_uint16]
        L.lcto_signfrac.restype = C.c_uint8
        L.lcto_signfrac.argtypes = [C.c_uint16]
        L.lcto_join.restype = C.c_uint16
        L.lcto_join.argtypes = [C.c_uint8, C.c_uint8]
        L.lcto_encode_block.argtypes = [P, P, u32, u32, P, P, P, P, P]
        L.lcto_decode_block.argtypes = [P, P, P, P, P, u32, u32, P]
        L.lcto_encode.argtypes = [P, P, u64, u32, u32, P, P, P, P, P, u64]
        L.lcto_decode.argtypes = [P, P, P, P, P, P, u64, u32, u32, P]
        L.lcto_fmaf.restype = C.c_float
        L.lcto_fmaf.argtypes = [C.c_float, C.c_float, C.c_float]
        L.lcto_rne_bf16.restype = C.c_uint16
        L.lcto_rne_bf16.argtypes = [C.c_float]
        L.lcto_sgd_elem.restype = C.c_uint16
        L.lcto_sgd_elem.argtypes = [C.c_uint16, C.c_uint16, C.c_float]
        L.lcto_sgd.argtypes = ([P, P, P, P, P, P] + [P, P, P, P, P, P] +
                               [C.c_float, P, u64, u32, u32, P, P, P, P, P, u64])
        L.lcto_momentum_elem.restype = None
        L.lcto_momentum_elem.argtypes = [C.c_uint16, C.c_uint16, C.c_uint16, C.c_float, C.c_float,
                                         C.POINTER(C.c_uint16), C.POINTER(C.c_uint16)]
        L.lcto_momentum.argtypes = ([P, P, P, P, P, P] + [P, P, P, P, P, P] +
                                    [P, C.c_float, C.c_float, P, P, u64, u32, u32] +
                                    [P, P, P, P, P, u64] + [P, P, P, P, P, u64])
        L.lcto_reshift.argtypes = [P, P, P, P, P, P, u64, u32, u32, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- codebook

@dataclass
class Codebook:
    """Final code: len[e] (0 = escaped), esc_len, shift, canonical codes, and
    the base code len_base the shift was applied to."""
    len: np.ndarray      # uint8[256]
    esc_len: int
    shift: int
    code: np.ndarray     # uint32[257], [256] = ESC
    len_base: np.ndarray  # uint8[256]

    def _c(self) -> _Codebook:
        cb = _Codebook()
        C.memmove(cb.len, self.len.astype(np.uint8).tobytes(), 256)
        cb.esc_len = int(self.esc_len)
        cb.shift = int(self.shift)
        C.memmove(cb.code, self.code.astype(np.uint32).tobytes(), 257 * 4)
        C.memmove(cb.len_base, self.len_base.astype(np.uint8).tobytes(), 256)
        return cb

    @staticmethod
    def _from_c(cb: _Codebook) -> "Codebook":
        return Codebook(np.frombuffer(bytes(cb.len), np.uint8).copy(), int(cb.esc_len),
                        int(cb.shift), np.frombuffer(bytes(cb.code), np.uint32).copy(),
                        np.frombuffer(bytes(cb.len_base), np.uint8).copy())

    def cost(self, e: int) -> int:
        return int(self.len[e]) if self.len[e] else self.esc_len + 8


def survival(family: int, scale: float, shape: float, t: float) -> float:
    return lib().lcto_model_survival(family, scale, shape, t)


def model_pmf(family: int, scale: float, shape: float = 0.0) -> np.ndarray:
    p = np.zeros(256, np.float64)
    rc = lib().lcto_model_pmf(family, scale, shape, _p(p))
    if rc != OK:
        raise ValueError("bad model")
    return p


def weights(p: np.ndarray) -> np.ndarray:
    w = np.zeros(256, np.uint64)
    lib().lcto_weights(_p(np.ascontiguousarray(p, np.float64)), _p(w))
    return w


def package_merge(w, L: int, ids=None) -> np.ndarray:
    w = np.ascontiguousarray(w, np.uint64)
    n = len(w)
    ids = np.arange(n, dtype=np.int32) if ids is None else np.ascontiguousarray(ids, np.int32)
    out = np.zeros(n, np.uint8)
    rc = lib().lcto_package_merge(n, _p(w), _p(ids), L, _p(out))
    if rc != OK:
        raise ValueError("package_merge: bad input")
    return out


def build_escape(w, L: int, lit_bits: int):
    """Returns (len[nsym], esc_len, k, cost)."""
    w = np.ascontiguousarray(w, np.uint64)
    n = len(w)
    ln = np.zeros(n, np.uint8)
    esc = C.c_uint8(0)
    k = C.c_int(0)
    cost = lib().lcto_build_escape(n, _p(w), L, lit_bits, _p(ln), C.byref(esc), C.byref(k))
    if cost == 2**64 - 1:
        raise ValueError("build_escape: bad input")
    return ln, int(esc.value), int(k.value), int(cost)


def build_base(w):
    return build_escape(w, 8, 8)


def best_shift(len_base, esc_len: int, exps) -> int:
    e = np.ascontiguousarray(exps, np.uint8)
    return lib().lcto_best_shift(_p(np.ascontiguousarray(len_base, np.uint8)), esc_len, _p(e), len(e))


def shift_cost(len_base, esc_len: int, exps, k: int) -> int:
    e = np.ascontiguousarray(exps, np.uint8)
    return int(lib().lcto_shift_cost(_p(np.ascontiguousarray(len_base, np.uint8)), esc_len,
                                     _p(e), len(e), k))


def canonical(len257) -> np.ndarray:
    code = np.zeros(257, np.uint32)
    lib().lcto_canonical(_p(np.ascontiguousarray(len257, np.uint8)), _p(code))
    return code


def codebook_from_base(len_base, esc_len: int, shift: int) -> Codebook:
    cb = _Codebook()
    lib().lcto_codebook_from_base(_p(np.ascontiguousarray(len_base, np.uint8)), esc_len, shift,
                                  C.byref(cb))
    return Codebook._from_c(cb)


def sample_positions(n: int) -> np.ndarray:
    """Positions floor(i * n / m), m = min(n, 4096), of the shift sample."""
    m = min(n, 4096)
    return (np.arange(m, dtype=np.uint64) * np.uint64(n)) // np.uint64(max(m, 1))


def codebook_from_sample(family: int, scale: float, shape: float, sample: np.ndarray) -> Codebook:
    """Codebook from the model and the already gathered sample (BF16 bits at
    sample_positions(n)); same result as codebook_build on the whole tensor."""
    lens, esc, _, _ = build_base(weights(model_pmf(family, scale, shape)))
    e = ((np.ascontiguousarray(sample, np.uint16) >> 7) & 0xFF).astype(np.uint8)
    return codebook_from_base(lens, esc, best_shift(lens, esc, e))


def codebook_build(family: int, scale: float, shape: float, x: np.ndarray) -> Codebook:
    x = np.ascontiguousarray(x, np.uint16)
    cb = _Codebook()
    rc = lib().lcto_codebook_build(family, scale, shape, _p(x), x.size, C.byref(cb))
    if rc != OK:
        raise ValueError("codebook_build: bad model")
    return Codebook._from_c(cb)


# ---------------------------------------------------------------- format

def exponent(v: int) -> int:
    return lib().lcto_exponent(v)


def signfrac(v: int) -> int:
    return lib().lcto_signfrac(v)


def join(sf: int, e: int) -> int:
    return lib().lcto_join(sf, e)


@dataclass
class Compressed:
    n: int
    block_elems: int
    cap_words: int
    sf: np.ndarray       # uint8[n]
    pay: np.ndarray      # uint32[nblk*cap_words*256]
    cnt: np.ndarray      # uint16[nblk*256]
    obase: np.ndarray    # uint64[nblk+1]
    ovf: np.ndarray      # uint8[ovf_cap]
    status: int = 0

    @property
    def nblk(self) -> int:
        return -(-self.n // self.block_elems)

    @property
    def spilled(self) -> int:
        return int(self.obase[-1])

    def nbytes(self) -> int:
        """Compressed size: sf + payload + markers + spilled bytes."""
        return (self.n + self.pay.nbytes + self.cnt.nbytes + self.obase.nbytes + self.spilled)

    def ratio(self) -> float:
        return 2.0 * self.n / self.nbytes() if self.n else 0.0


def _alloc(n: int, block_elems: int, cap_words: int, ovf_cap: int) -> Compressed:
    nblk = -(-n // block_elems)
    return Compressed(n, block_elems, cap_words, np.zeros(n, np.uint8),
                      np.zeros(nblk * cap_words * NSTREAM, np.uint32),
                      np.zeros(nblk * NSTREAM, np.uint16), np.zeros(nblk + 1, np.uint64),
                      np.zeros(max(ovf_cap, 1), np.uint8))


def encode(cb: Codebook, x: np.ndarray, block_elems: int, cap_words: int,
           ovf_cap: int | None = None) -> Compressed:
    x = np.ascontiguousarray(x, np.uint16).reshape(-1)
    n = x.size
    ovf_cap = n if ovf_cap is None else ovf_cap
    t = _alloc(n, block_elems, cap_words, ovf_cap)
    c = cb._c()
    rc = lib().lcto_encode(C.byref(c), _p(x), n, block_elems, cap_words, _p(t.sf), _p(t.pay),
                           _p(t.cnt), _p(t.obase), _p(t.ovf), ovf_cap)
    if rc < 0:
        raise ValueError("encode: bad arguments")
    t.status = rc
    return t


def decode(cb: Codebook, t: Compressed) -> np.ndarray:
    y = np.zeros(t.n, np.uint16)
    c = cb._c()
    rc = lib().lcto_decode(C.byref(c), _p(t.sf), _p(t.pay), _p(t.cnt), _p(t.obase), _p(t.ovf),
                           t.n, t.block_elems, t.cap_words, _p(y))
    if rc != OK:
        raise ValueError("decode: stream error %d" % rc)
    return y


def encode_block(cb: Codebook, x: np.ndarray, cap_words: int):
    """One block: returns (sf, pay, cnt, spill bytes)."""
    x = np.ascontiguousarray(x, np.uint16).reshape(-1)
    nb = x.size
    sf = np.zeros(nb, np.uint8)
    pay = np.zeros(cap_words * NSTREAM, np.uint32)
    cnt = np.zeros(NSTREAM, np.uint16)
    spill = np.zeros(max(nb, 1), np.uint8)
    ns = C.c_uint32(0)
    c = cb._c()
    lib().lcto_encode_block(C.byref(c), _p(x), nb, cap_words, _p(sf), _p(pay), _p(cnt),
                            _p(spill), C.byref(ns))
    return sf, pay, cnt, spill[:ns.value].copy()


def decode_block(cb: Codebook, sf, pay, cnt, spill, cap_words: int) -> np.ndarray:
    sf = np.ascontiguousarray(sf, np.uint8)
    nb = sf.size
    y = np.zeros(nb, np.uint16)
    spill = np.ascontiguousarray(spill, np.uint8)
    if spill.size == 0:
        spill = np.zeros(1, np.uint8)
    c = cb._c()
    rc = lib().lcto_decode_block(C.byref(c), _p(sf), _p(np.ascontiguousarray(pay, np.uint32)),
                                 _p(np.ascontiguousarray(cnt, np.uint16)), _p(spill), nb,
                                 cap_words, _p(y))
    if rc != OK:
        raise ValueError("decode_block: stream error %d" % rc)
    return y


# ---------------------------------------------------------------- SGD

def fmaf(a: float, b: float, c: float) -> float:
    return lib().lcto_fmaf(a, b, c)


def rne_bf16(r: float) -> int:
    return lib().lcto_rne_bf16(r)


def sgd_elem(w: int, m: int, eta: float) -> int:
    return lib().lcto_sgd_elem(w, m, eta)


def sgd_dense(w: np.ndarray, m: np.ndarray, eta: float) -> np.ndarray:
    """Element-wise update on raw BF16 bit patterns (serial C, via the block path)."""
    L = lib()
    w = np.ascontiguousarray(w, np.uint16).reshape(-1)
    m = np.ascontiguousarray(m, np.uint16).reshape(-1)
    return np.fromiter((L.lcto_sgd_elem(int(a), int(b), eta) for a, b in zip(w, m)),
                       np.uint16, count=w.size)


def _cb_ref(cb: Codebook | None):
    return None if cb is None else C.byref(cb._c())


def sgd(cw: Codebook, w: Compressed, cm: Codebook, m: Compressed, eta: float,
        ovf_cap: int | None = None, cw_out: Codebook | None = None) -> Compressed:
    """Naive round trip of one SGD step; W' is encoded with cw_out (cw if None)."""
    assert (w.n, w.block_elems, w.cap_words) == (m.n, m.block_elems, m.cap_words)
    ovf_cap = w.n if ovf_cap is None else ovf_cap
    o = _alloc(w.n, w.block_elems, w.cap_words, ovf_cap)
    a, b = cw._c(), cm._c()
    rc = lib().lcto_sgd(C.byref(a), _p(w.sf), _p(w.pay), _p(w.cnt), _p(w.obase), _p(w.ovf),
                        C.byref(b), _p(m.sf), _p(m.pay), _p(m.cnt), _p(m.obase), _p(m.ovf),
                        eta, _cb_ref(cw_out), w.n, w.block_elems, w.cap_words, _p(o.sf), _p(o.pay), _p(o.cnt),
                        _p(o.obase), _p(o.ovf), ovf_cap)
    if rc < 0:
        raise ValueError("sgd: error %d" % rc)
    o.status = rc
    return o


# ---------------------------------------------------------------- momentum step

def momentum_elem(w: int, m: int, g: int, mu: float, eta: float):
    """(w', m') of one element: m' = rne(fmaf(mu, m, g)), w' = rne(fmaf(-eta, m', w))."""
    wo, mo = C.c_uint16(), C.c_uint16()
    lib().lcto_momentum_elem(w, m, g, mu, eta, C.byref(wo), C.byref(mo))
    return wo.value, mo.value


def momentum_dense(w: np.ndarray, m: np.ndarray, g: np.ndarray, mu: float, eta: float):
    """Element-wise momentum step on raw BF16 bit patterns (serial C)."""
    w = np.ascontiguousarray(w, np.uint16).reshape(-1)
    m = np.ascontiguousarray(m, np.uint16).reshape(-1)
    g = np.ascontiguousarray(g, np.uint16).reshape(-1)
    wo = np.empty_like(w)
    mo = np.empty_like(m)
    for i in range(w.size):
        wo[i], mo[i] = momentum_elem(int(w[i]), int(m[i]), int(g[i]), mu, eta)
    return wo, mo


def momentum(cw: Codebook, w: Compressed, cm: Codebook, m: Compressed, g: np.ndarray,
             mu: float, eta: float, ovf_cap: int | None = None,
             cw_out: Codebook | None = None, cm_out: Codebook | None = None):
    """Naive round trip of one momentum step on compressed W and M and dense g:
    returns (W', M') encoded with cw_out and cm_out (cw and cm if None)."""
    assert (w.n, w.block_elems, w.cap_words) == (m.n, m.block_elems, m.cap_words)
    g = np.ascontiguousarray(g, np.uint16).reshape(-1)
    assert g.size == w.n
    ovf_cap = w.n if ovf_cap is None else ovf_cap
    ow = _alloc(w.n, w.block_elems, w.cap_words, ovf_cap)
    om = _alloc(w.n, w.block_elems, w.cap_words, ovf_cap)
    a, b = cw._c(), cm._c()
    rc = lib().lcto_momentum(C.byref(a), _p(w.sf), _p(w.pay), _p(w.cnt), _p(w.obase), _p(w.ovf),
                             C.byref(b), _p(m.sf), _p(m.pay), _p(m.cnt), _p(m.obase), _p(m.ovf),
                             _p(g), mu, eta, _cb_ref(cw_out), _cb_ref(cm_out), w.n, w.block_elems, w.cap_words,
                             _p(ow.sf), _p(ow.pay), _p(ow.cnt), _p(ow.obase), _p(ow.ovf), ovf_cap,
                             _p(om.sf), _p(om.pay), _p(om.cnt), _p(om.obase), _p(om.ovf), ovf_cap)
    if rc < 0:
        raise ValueError("momentum: error %d" % rc)
    ow.status = int(ow.obase[-1] > ovf_cap)
    om.status = int(om.obase[-1] > ovf_cap)
    return ow, om


# ---------------------------------------------------------------- shift re-estimation

def reshift(cb: Codebook, t: Compressed) -> Codebook:
    """cb's base code with the shift re-estimated from the compressed tensor t
    (decoded with cb; sample at sample_positions(t.n))."""
    out = _Codebook()
    rc = lib().lcto_reshift(C.byref(cb._c()), _p(t.sf), _p(t.pay), _p(t.cnt), _p(t.obase),
                            _p(t.ovf), t.n, t.block_elems, t.cap_words, C.byref(out))
    if rc != OK:
        raise ValueError("reshift: error %d" % rc)
    return Codebook._from_c(out)


# ---------------------------------------------------------------- tensor groups

def group(ts, ovf_cap: int | None = None) -> Compressed:
    """Tensors laid side by side with one shared overflow region (explainer,
    paragraph on the idealized arithmetic: the shared overflow buffer).  Tensor
    k's blocks follow tensor k-1's; its sign-fraction bytes start at the sum of
    the earlier sizes, each rounded up to a multiple of 256 (the padding is
    zero); its spilled bytes follow the earlier tensors' in the shared region
    and its block offsets are shifted by their total.  Every tensor is encoded
    on its own (each with every spilled byte kept); this only places them.
    The result's n is the sf array's length."""
    B, cw = ts[0].block_elems, ts[0].cap_words
    assert all((t.block_elems, t.cap_words) == (B, cw) for t in ts)
    sf, pay, cnt, ob, ovf = [], [], [], [], []
    base = 0
    for t in ts:
        assert t.spilled <= len(t.ovf), "encode each tensor with room for every spill"
        pad = -(-t.n // 256) * 256
        sf.append(np.concatenate([t.sf[:t.n], np.zeros(pad - t.n, np.uint8)]))
        pay.append(t.pay)
        cnt.append(t.cnt)
        ob.append(t.obase[:-1] + np.uint64(base))
        ovf.append(t.ovf[:t.spilled])
        base += t.spilled
    ob.append(np.array([base], np.uint64))
    total = base
    ovf_cap = total if ovf_cap is None else ovf_cap
    region = np.zeros(max(ovf_cap, 1), np.uint8)
    keep = min(total, ovf_cap)
    region[:keep] = np.concatenate(ovf)[:keep] if ovf else region[:0]
    g = Compressed(sum(len(a) for a in sf), B, cw, np.concatenate(sf), np.concatenate(pay),
                   np.concatenate(cnt), np.concatenate(ob), region)
    g.status = int(total > ovf_cap)
    return g


def group_member(g: Compressed, ns, k: int) -> Compressed:
    """Tensor k of a group (sizes ns) as a tensor whose block offsets index
    the group's shared overflow region."""
    B, cw = g.block_elems, g.cap_words
    b0 = sum(-(-n // B) for n in ns[:k])
    e0 = sum(-(-n // 256) * 256 for n in ns[:k])
    nb = -(-ns[k] // B)
    return Compressed(ns[k], B, cw, g.sf[e0:e0 + ns[k]], g.pay[b0 * cw * NSTREAM:(b0 + nb) * cw * NSTREAM],
                      g.cnt[b0 * NSTREAM:(b0 + nb) * NSTREAM], g.obase[b0:b0 + nb + 1], g.ovf)


def encode_group(cbs, xs, block_elems: int, cap_words: int, ovf_cap: int | None = None) -> Compressed:
    """Every tensor encoded with its own codebook, then placed as a group."""
    return group([encode(cb, x, block_elems, cap_words) for cb, x in zip(cbs, xs)], ovf_cap)


# ---------------------------------------------------------------- block-range driver

def _at(a: np.ndarray, i: int) -> C.c_void_p:
    """Pointer to element i of a contiguous numpy array."""
    return C.c_void_p(a.ctypes.data + int(i) * a.itemsize)


def _ranges(nblk: int, pieces: int):
    pieces = max(1, min(pieces, nblk))
    cuts = [nblk * i // pieces for i in range(pieces + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(pieces) if cuts[i + 1] > cuts[i]]


def _in_view(t: Compressed, b0: int, b1: int):
    """Blocks [b0, b1) of t as the serial routines take a tensor: element
    range, pointers into t's arrays and offsets rebased to the range."""
    B, cw = t.block_elems, t.cap_words
    e0, e1 = b0 * B, min(b1 * B, t.n)
    ob = (t.obase[b0:b1 + 1] - t.obase[b0]).astype(np.uint64)
    ovf = _at(t.ovf, int(t.obase[b0])) if int(t.obase[b0]) < t.ovf.size else _at(t.ovf, 0)
    return e0, e1, (_at(t.sf, e0), _at(t.pay, b0 * cw * NSTREAM), _at(t.cnt, b0 * NSTREAM), _p(ob), ovf), ob


def _stitch(out: Compressed, ranges, parts, ovf_cap: int):
    """Offsets and spilled bytes of the block ranges, placed in block order
    (the serial scan over the ranges' totals)."""
    base = 0
    for (b0, b1), (ob, ov) in zip(ranges, parts):
        out.obase[b0:b1] = ob[:-1] + np.uint64(base)
        tot = int(ob[-1])
        keep = max(0, min(tot, ovf_cap - base))
        if keep:
            out.ovf[base:base + keep] = ov[:keep]
        base += tot
    out.obase[out.nblk] = base
    out.status = int(base > ovf_cap)
    return out


def _run(fn, ranges, threads: int):
    """fn over the block ranges on `threads` host threads (the C calls release
    the interpreter lock, so the ranges run in parallel)."""
    from concurrent.futures import ThreadPoolExecutor
    if threads <= 1:
        return [fn(r) for r in ranges]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, ranges))


def encode_threads(cb: Codebook, x: np.ndarray, block_elems: int, cap_words: int,
                   threads: int, ovf_cap: int | None = None, pieces: int | None = None) -> Compressed:
    """lcto_encode over ranges of whole blocks on several host threads, then
    the overflow offsets by a serial scan over the ranges: the same bytes as
    encode() (blocks are coded independently; only the offsets chain)."""
    x = np.ascontiguousarray(x, np.uint16).reshape(-1)
    n = x.size
    ovf_cap = n if ovf_cap is None else ovf_cap
    out = _alloc(n, block_elems, cap_words, ovf_cap)
    ranges = _ranges(out.nblk, pieces or 4 * threads)
    c = cb._c()

    def work(r):
        b0, b1 = r
        e0, e1 = b0 * block_elems, min(b1 * block_elems, n)
        ob = np.zeros(b1 - b0 + 1, np.uint64)
        ov = np.zeros(max(e1 - e0, 1), np.uint8)
        rc = lib().lcto_encode(C.byref(c), _at(x, e0), e1 - e0, block_elems, cap_words, _at(out.sf, e0),
                               _at(out.pay, b0 * cap_words * NSTREAM), _at(out.cnt, b0 * NSTREAM), _p(ob),
                               _p(ov), e1 - e0)
        if rc < 0:
            raise ValueError("encode: bad arguments")
        return ob, ov

    return _stitch(out, ranges, _run(work, ranges, threads), ovf_cap)


def sgd_threads(cw: Codebook, w: Compressed, cm: Codebook, m: Compressed, eta: float, threads: int,
                ovf_cap: int | None = None, pieces: int | None = None) -> Compressed:
    """sgd() over ranges of whole blocks on several host threads (each range
    the naive round trip on its own), offsets stitched serially."""
    assert (w.n, w.block_elems, w.cap_words) == (m.n, m.block_elems, m.cap_words)
    B, cwd = w.block_elems, w.cap_words
    ovf_cap = w.n if ovf_cap is None else ovf_cap
    out = _alloc(w.n, B, cwd, ovf_cap)
    ranges = _ranges(out.nblk, pieces or 4 * threads)
    a, b = cw._c(), cm._c()

    def work(r):
        b0, b1 = r
        e0, e1, wp, wob = _in_view(w, b0, b1)
        _, _, mp, mob = _in_view(m, b0, b1)
        ob = np.zeros(b1 - b0 + 1, np.uint64)
        ov = np.zeros(max(e1 - e0, 1), np.uint8)
        rc = lib().lcto_sgd(C.byref(a), *wp, C.byref(b), *mp, eta, None, e1 - e0, B, cwd,
                            _at(out.sf, e0), _at(out.pay, b0 * cwd * NSTREAM), _at(out.cnt, b0 * NSTREAM),
                            _p(ob), _p(ov), e1 - e0)
        if rc < 0:
            raise ValueError("sgd: error %d" % rc)
        return ob, ov

    return _stitch(out, ranges, _run(work, ranges, threads), ovf_cap)


def decode_threads(cb: Codebook, t: Compressed, threads: int, pieces: int | None = None) -> np.ndarray:
    """decode() over ranges of whole blocks on several host threads."""
    y = np.zeros(t.n, np.uint16)
    ranges = _ranges(t.nblk, pieces or 4 * threads)
    c = cb._c()

    def work(r):
        b0, b1 = r
        e0, e1, tp, _ = _in_view(t, b0, b1)
        rc = lib().lcto_decode(C.byref(c), *tp, e1 - e0, t.block_elems, t.cap_words, _at(y, e0))
        if rc != OK:
            raise ValueError("decode: stream error %d" % rc)

    _run(work, ranges, threads)
    return y
