"""Python binding of the LCT codec's C ABI (``include/lct.h``, ``liblct.so``).

Argument marshalling only: every step of the codec runs in the HIP library.
torch provides device memory (``torch.empty`` on the GPU) and the stream
(``torch.cuda.current_stream()``); nothing else of torch is used.  Importing
the package needs the built library; there is no fallback.

Functions keep the C names:
    lct_layout_init(mode) -> Layout
    lct_sizes(n, layout, ovf_cap) -> Sizes
    lct_codebook_build(model, x) -> Codebook
    lct_codebook_from_lengths(len_base, esc_len, shift) -> Codebook
    lct_tensor_sample(cb, t) -> numpy uint16 array (the shift sample)
    lct_codebook_reshift(cb, t) -> Codebook
    lct_codebook_reshift_dense(cb, x) -> Codebook
    lct_codebook_adapt(cb, t, max_spill_per_elem) -> (Codebook, changed)
    lct_encode(cb, x, out)            (out: LctTensor from alloc_tensor)
    lct_decode(cb, t, y)
    lct_sgd_step(cw, w_in, cm, m, eta, w_out)
    lct_sgd_step_recode(cw, w_in, cm, m, eta, cw_out, w_out)
    lct_sgd_step_noalloc(cw, w_in, cm, m, eta, w_out)   (static working memory)
    lct_momentum_step(cw, w_in, cm, m_in, g, mu, eta, w_out, m_out)
    lct_momentum_step_recode(cw, w_in, cm, m_in, g, mu, eta, cw_out, cm_out, w_out, m_out)
    LctGroup(ns, layout, codebooks, dense)  (lct_group_table_bytes + lct_group_bind)
    lct_encode_group(g, all) / lct_decode_group(g, all)
    lct_sgd_step_group(gw, w_all, gm, m_all, eta, w_out)
    lct_momentum_step_group(gw, w_all, gm, m_all, gg, mu, eta, w_out, m_out)
plus ``alloc_tensor`` and the convenience wrappers ``encode`` / ``decode`` /
``sgd_step`` / ``momentum_step`` that allocate their outputs.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblct.so")

GAUSSIAN, LAPLACE, POWERLAW = 0, 1, 2
CLEAN, MEDIUM, HIGH = 0, 1, 2
ST_OVF_FULL, ST_LOOKBACK = 0x1, 0x2
OK, EINVAL, EALIGN, EALIAS, EHIP, EARCH, ESIZE = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED = ["lct_layout_init", "lct_sizes", "lct_codebook_build", "lct_codebook_from_lengths",
            "lct_tensor_sample", "lct_codebook_reshift", "lct_codebook_reshift_dense",
            "lct_codebook_adapt", "lct_encode", "lct_decode",
            "lct_sgd_step", "lct_sgd_step_recode", "lct_sgd_step_noalloc", "lct_momentum_step", "lct_momentum_step_recode",
            "lct_group_table_bytes", "lct_group_bind", "lct_group_fit", "lct_group_sizes", "lct_group_tensor",
            "lct_encode_group", "lct_decode_group", "lct_sgd_step_group", "lct_momentum_step_group",
            "lct_strerror", "lct_last_hip_error"]


class Model(C.Structure):
    _fields_ = [("family", C.c_int32), ("scale", C.c_double), ("shape", C.c_double)]


class Layout(C.Structure):
    _fields_ = [("block_elems", C.c_uint32), ("cap_words", C.c_uint32)]


class Codebook(C.Structure):
    _fields_ = [("len", C.c_uint8 * 256), ("esc_len", C.c_uint8), ("max_len", C.c_uint8),
                ("shift", C.c_int16), ("kept", C.c_uint32), ("model", Model),
                ("code", C.c_uint32 * 257), ("enc_bits", C.c_uint32 * 256),
                ("enc_len", C.c_uint8 * 256), ("dec", C.c_uint16 * 256),
                ("len_base", C.c_uint8 * 256)]


class _Tensor(C.Structure):
    _fields_ = [("n", C.c_uint64), ("layout", Layout), ("sf", C.c_void_p), ("pay", C.c_void_p),
                ("cnt", C.c_void_p), ("obase", C.c_void_p), ("ovf", C.c_void_p),
                ("ovf_cap", C.c_uint64), ("status", C.c_void_p), ("scratch", C.c_void_p)]


class Sizes(C.Structure):
    _fields_ = [("nblk", C.c_uint64), ("sf", C.c_uint64), ("pay", C.c_uint64),
                ("cnt", C.c_uint64), ("obase", C.c_uint64), ("scratch", C.c_uint64),
                ("fixed", C.c_uint64)]


class Group(C.Structure):
    _fields_ = [("count", C.c_uint32), ("layout", Layout), ("nblk", C.c_uint64),
                ("sf_bytes", C.c_uint64), ("shape_hash", C.c_uint64), ("n", C.c_void_p),
                ("d_dense", C.c_void_p), ("d_table", C.c_void_p)]


class LctError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblct.so is not built: run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    L = C.CDLL(LIB_PATH)
    P, u64, i32 = C.c_void_p, C.c_uint64, C.c_int32
    L.lct_layout_init.argtypes = [i32, C.POINTER(Layout)]
    L.lct_sizes.argtypes = [u64, C.POINTER(Layout), u64, C.POINTER(Sizes)]
    L.lct_codebook_build.argtypes = [C.POINTER(Model), P, u64, P, C.POINTER(Codebook)]
    L.lct_codebook_from_lengths.argtypes = [P, C.c_uint8, i32, C.POINTER(Codebook)]
    CB, T = C.POINTER(Codebook), C.POINTER(_Tensor)
    L.lct_tensor_sample.argtypes = [CB, T, P, P, C.POINTER(C.c_uint32)]
    L.lct_codebook_reshift.argtypes = [CB, T, P, CB]
    L.lct_codebook_reshift_dense.argtypes = [CB, P, u64, P, CB]
    L.lct_codebook_adapt.argtypes = [CB, T, C.c_double, P, CB, C.POINTER(i32)]
    L.lct_sgd_step_recode.argtypes = [CB, T, CB, T, C.c_float, CB, T, P]
    L.lct_momentum_step_recode.argtypes = [CB, T, CB, T, P, C.c_float, C.c_float, CB, CB, T, T, P]
    G = C.POINTER(Group)
    L.lct_group_table_bytes.argtypes = [C.c_uint32, P, C.POINTER(Layout), C.POINTER(u64)]
    L.lct_group_bind.argtypes = [C.c_uint32, P, C.POINTER(Layout), P, P, P, G]
    L.lct_group_fit.argtypes = [CB, P, P, C.POINTER(Layout), P, P, P, G]
    L.lct_group_sizes.argtypes = [G, u64, C.POINTER(Sizes)]
    L.lct_group_tensor.argtypes = [G, T, C.c_uint32, T]
    L.lct_encode_group.argtypes = [G, T, P]
    L.lct_decode_group.argtypes = [G, T, P]
    L.lct_sgd_step_group.argtypes = [G, T, G, T, C.c_float, T, P]
    L.lct_momentum_step_group.argtypes = [G, T, G, T, G, C.c_float, C.c_float, T, T, P]
    L.lct_encode.argtypes = [C.POINTER(Codebook), P, C.POINTER(_Tensor), P]
    L.lct_decode.argtypes = [C.POINTER(Codebook), C.POINTER(_Tensor), P, P]
    L.lct_sgd_step.argtypes = [C.POINTER(Codebook), C.POINTER(_Tensor), C.POINTER(Codebook),
                               C.POINTER(_Tensor), C.c_float, C.POINTER(_Tensor), P]
    L.lct_sgd_step_noalloc.argtypes = [C.POINTER(Codebook), C.POINTER(_Tensor), C.POINTER(Codebook),
                                       C.POINTER(_Tensor), C.c_float, C.POINTER(_Tensor), P]
    L.lct_momentum_step.argtypes = [C.POINTER(Codebook), C.POINTER(_Tensor), C.POINTER(Codebook),
                                    C.POINTER(_Tensor), P, C.c_float, C.c_float, C.POINTER(_Tensor),
                                    C.POINTER(_Tensor), P]
    L.lct_strerror.restype = C.c_char_p
    L.lct_strerror.argtypes = [i32]
    L.lct_last_hip_error.restype = C.c_char_p
    for name in EXPORTED:
        if name not in ("lct_strerror", "lct_last_hip_error"):
            getattr(L, name).restype = i32
    return L


lib = _load()


def _check(rc: int, what: str):
    if rc != OK:
        msg = lib.lct_strerror(rc).decode()
        if rc == EHIP:
            msg += " (" + lib.lct_last_hip_error().decode() + ")"
        raise LctError("%s failed: %s [%d]" % (what, msg, rc))


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ layout, sizes

def lct_layout_init(mode: int) -> Layout:
    out = Layout()
    _check(lib.lct_layout_init(mode, C.byref(out)), "lct_layout_init")
    return out


def layout(block_elems: int, cap_words: int) -> Layout:
    return Layout(block_elems, cap_words)


def lct_sizes(n: int, lay: Layout, ovf_cap: int = 0) -> Sizes:
    out = Sizes()
    _check(lib.lct_sizes(n, C.byref(lay), ovf_cap, C.byref(out)), "lct_sizes")
    return out


# ------------------------------------------------------------------ codebook

def lct_codebook_build(model: Model, x: torch.Tensor | None, stream=None) -> Codebook:
    """Codebook for model, shift sampled from x (BF16 or 16-bit tensor on the GPU)."""
    out = Codebook()
    n = 0 if x is None else x.numel()
    if n:
        _bits16(x)
    st = _stream(stream) if n else None     # no sample: nothing runs on the device
    _check(lib.lct_codebook_build(C.byref(model), _ptr(x), n, st, C.byref(out)),
           "lct_codebook_build")
    return out


def lct_codebook_from_lengths(len_base, esc_len: int, shift: int = 0) -> Codebook:
    arr = (C.c_uint8 * 256)(*[int(v) for v in len_base])
    out = Codebook()
    _check(lib.lct_codebook_from_lengths(arr, esc_len, shift, C.byref(out)),
           "lct_codebook_from_lengths")
    return out


def lct_tensor_sample(cb: Codebook, t: "LctTensor", stream=None):
    """BF16 bit patterns (numpy uint16) of the shift sample of t."""
    import numpy as np
    out = np.zeros(4096, np.uint16)
    m = C.c_uint32(0)
    ct = t.c()
    st = _stream(stream) if t.n else None
    _check(lib.lct_tensor_sample(C.byref(cb), C.byref(ct), st, out.ctypes.data_as(C.c_void_p),
                                 C.byref(m)), "lct_tensor_sample")
    return out[:m.value].copy()


def lct_codebook_reshift(cb: Codebook, t: "LctTensor", stream=None) -> Codebook:
    """cb's base code with the shift re-estimated from the compressed tensor t."""
    out = Codebook()
    ct = t.c()
    st = _stream(stream) if t.n else None
    _check(lib.lct_codebook_reshift(C.byref(cb), C.byref(ct), st, C.byref(out)),
           "lct_codebook_reshift")
    return out


def lct_codebook_reshift_dense(cb: Codebook, x: torch.Tensor, stream=None) -> Codebook:
    """cb's base code with the shift re-estimated from the dense tensor x."""
    n = x.numel()
    if n:
        _bits16(x)
    out = Codebook()
    st = _stream(stream) if n else None
    _check(lib.lct_codebook_reshift_dense(C.byref(cb), _ptr(x), n, st, C.byref(out)),
           "lct_codebook_reshift_dense")
    return out


def lct_codebook_adapt(cb: Codebook, t: "LctTensor", max_spill_per_elem: float, stream=None):
    """(codebook, changed): re-estimated when t spills more than the limit."""
    out = Codebook()
    changed = C.c_int32(0)
    ct = t.c()
    st = _stream(stream) if t.n else None
    _check(lib.lct_codebook_adapt(C.byref(cb), C.byref(ct), max_spill_per_elem, st, C.byref(out),
                                  C.byref(changed)), "lct_codebook_adapt")
    return out, bool(changed.value)


# ------------------------------------------------------------------ compressed tensors

class LctTensor:
    """Device buffers of one compressed tensor (torch-owned memory)."""

    def __init__(self, n: int, lay: Layout, ovf_cap: int, device="cuda", scratch=None, ovf=None):
        sz = lct_sizes(n, lay, ovf_cap)
        dev = torch.device(device)
        u8 = torch.uint8
        self.n, self.layout, self.ovf_cap, self.sizes = n, Layout(lay.block_elems, lay.cap_words), ovf_cap, sz
        self.sf = torch.empty(max(sz.sf, 16), dtype=u8, device=dev)
        self.pay = torch.empty(max(sz.pay // 4, 4), dtype=torch.int32, device=dev)
        self.cnt = torch.empty(max(sz.cnt // 2, 2), dtype=torch.int16, device=dev)
        # zeroed: the calls write nothing for an empty tensor, whose encoding
        # is obase = [0]
        self.obase = torch.zeros(sz.obase // 8, dtype=torch.int64, device=dev)
        if ovf is None:
            ovf = torch.empty(max(ovf_cap, 16), dtype=u8, device=dev)
        elif ovf.numel() < ovf_cap:
            raise ValueError("ovf too small: %d < %d" % (ovf.numel(), ovf_cap))
        self.ovf = ovf
        self.status = torch.zeros(4, dtype=torch.int32, device=dev)
        if scratch is None:
            scratch = torch.empty(sz.scratch, dtype=u8, device=dev)
        elif scratch.numel() < sz.scratch:
            raise ValueError("scratch too small: %d < %d" % (scratch.numel(), sz.scratch))
        self.scratch = scratch

    @classmethod
    def wrap(cls, n: int, lay: Layout, ovf_cap: int, sizes: Sizes, sf, pay, cnt, obase, ovf, status,
             scratch) -> "LctTensor":
        """A descriptor over existing buffers (views of a group's storage)."""
        t = cls.__new__(cls)
        t.n, t.layout, t.ovf_cap, t.sizes = n, Layout(lay.block_elems, lay.cap_words), ovf_cap, sizes
        t.sf, t.pay, t.cnt, t.obase, t.ovf, t.status, t.scratch = sf, pay, cnt, obase, ovf, status, scratch
        return t

    def c(self, need_scratch: bool = True) -> _Tensor:
        """The C descriptor.  Every buffer must be a contiguous device tensor
        of at least the bytes lct_sizes gives (the library cannot see a
        buffer's size; a missing one is left to the call to refuse)."""
        sz = self.sizes
        for name, need in (("sf", sz.sf), ("pay", sz.pay), ("cnt", sz.cnt), ("obase", sz.obase),
                           ("ovf", self.ovf_cap), ("status", 4), ("scratch", sz.scratch if need_scratch else 0)):
            b = getattr(self, name)
            if b is None:
                continue
            if not b.is_cuda or not b.is_contiguous():
                raise ValueError("%s must be a contiguous device tensor" % name)
            if b.numel() * b.element_size() < need:
                raise ValueError("%s holds %d bytes; the tensor needs %d" % (name, b.numel() * b.element_size(), need))
        return _Tensor(self.n, self.layout, _ptr(self.sf), _ptr(self.pay), _ptr(self.cnt),
                       _ptr(self.obase), _ptr(self.ovf), self.ovf_cap, _ptr(self.status),
                       _ptr(self.scratch))

    # host views (synchronise the current stream)
    def status_word(self) -> int:
        return int(self.status[0].item()) & 0xFFFFFFFF

    def spilled(self) -> int:
        """Spilled bytes of this tensor (a group member's offsets start where
        the earlier members' spills end)."""
        if self.obase.numel() == 1:
            return 0
        ends = self.obase[[0, -1]].cpu()
        return int(ends[1]) - int(ends[0])

    def full_path_units(self) -> int:
        """Units (64 streams of a block) that the last update writing this
        tensor ran on its full-block path: a counter the update keeps in the
        header of its working memory (byte offset 28), for tests."""
        return int(self.scratch[28:32].view(torch.int32).item())

    def nbytes(self) -> int:
        return int(self.sizes.fixed) + self.spilled()

    def ratio(self) -> float:
        return 2.0 * self.n / self.nbytes() if self.n else 0.0


def full_ovf_cap(n: int, lay: Layout) -> int:
    """An overflow region for every element of n rounded up to whole blocks:
    no spill can exceed it, and with it the kernels stage spilled fields at
    fixed places (no shared counter), which is faster when many streams spill."""
    b = int(lay.block_elems)
    return -(-n // b) * b if n else 0


def alloc_tensor(n: int, lay: Layout, ovf_cap: int | None = None, device="cuda",
                 scratch=None, ovf=None) -> LctTensor:
    """Buffers of a compressed tensor (ovf_cap: full_ovf_cap(n, lay) when None)."""
    return LctTensor(n, lay, full_ovf_cap(n, lay) if ovf_cap is None else ovf_cap, device, scratch, ovf)


def _bits16(x: torch.Tensor) -> torch.Tensor:
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("expected BF16 (or 16-bit pattern) tensor, got %s" % x.dtype)
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if not x.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return x


def _gradient(g: torch.Tensor, n: int) -> torch.Tensor:
    _bits16(g)
    if g.numel() != n:
        raise ValueError("g has %d elements, the tensors %d" % (g.numel(), n))
    return g


def lct_encode(cb: Codebook, x: torch.Tensor, out: LctTensor, stream=None) -> None:
    _bits16(x)
    if x.numel() != out.n:
        raise ValueError("x has %d elements, output tensor %d" % (x.numel(), out.n))
    t = out.c()
    _check(lib.lct_encode(C.byref(cb), _ptr(x), C.byref(t), _stream(stream)), "lct_encode")


def lct_decode(cb: Codebook, t: LctTensor, y: torch.Tensor, stream=None) -> None:
    _bits16(y)
    if y.numel() != t.n:
        raise ValueError("y has %d elements, tensor %d" % (y.numel(), t.n))
    ct = t.c()
    _check(lib.lct_decode(C.byref(cb), C.byref(ct), _ptr(y), _stream(stream)), "lct_decode")


def lct_sgd_step(cw: Codebook, w_in: LctTensor, cm: Codebook, m: LctTensor, eta: float,
                 w_out: LctTensor, stream=None) -> None:
    a, b, o = w_in.c(), m.c(), w_out.c()
    _check(lib.lct_sgd_step(C.byref(cw), C.byref(a), C.byref(cm), C.byref(b), eta, C.byref(o),
                            _stream(stream)), "lct_sgd_step")


def lct_sgd_step_noalloc(cw: Codebook, w_in: LctTensor, cm: Codebook, m: LctTensor, eta: float,
                         w_out: LctTensor, stream=None) -> None:
    """lct_sgd_step with the library's static working memory (w_out's
    scratch is not used)."""
    a, b, o = w_in.c(), m.c(), w_out.c(need_scratch=False)
    _check(lib.lct_sgd_step_noalloc(C.byref(cw), C.byref(a), C.byref(cm), C.byref(b), eta, C.byref(o),
                                    _stream(stream)), "lct_sgd_step_noalloc")


def lct_sgd_step_recode(cw: Codebook, w_in: LctTensor, cm: Codebook, m: LctTensor, eta: float,
                        cw_out: Codebook, w_out: LctTensor, stream=None) -> None:
    a, b, o = w_in.c(), m.c(), w_out.c()
    _check(lib.lct_sgd_step_recode(C.byref(cw), C.byref(a), C.byref(cm), C.byref(b), eta,
                                   C.byref(cw_out), C.byref(o), _stream(stream)),
           "lct_sgd_step_recode")


def lct_momentum_step_recode(cw: Codebook, w_in: LctTensor, cm: Codebook, m_in: LctTensor,
                             g: torch.Tensor, mu: float, eta: float, cw_out: Codebook,
                             cm_out: Codebook, w_out: LctTensor, m_out: LctTensor,
                             stream=None) -> None:
    _gradient(g, w_in.n)
    a, b, ow, om = w_in.c(), m_in.c(), w_out.c(), m_out.c()
    _check(lib.lct_momentum_step_recode(C.byref(cw), C.byref(a), C.byref(cm), C.byref(b), _ptr(g),
                                        mu, eta, C.byref(cw_out), C.byref(cm_out), C.byref(ow),
                                        C.byref(om), _stream(stream)), "lct_momentum_step_recode")


def lct_momentum_step(cw: Codebook, w_in: LctTensor, cm: Codebook, m_in: LctTensor, g: torch.Tensor,
                      mu: float, eta: float, w_out: LctTensor, m_out: LctTensor, stream=None) -> None:
    _gradient(g, w_in.n)
    a, b, ow, om = w_in.c(), m_in.c(), w_out.c(), m_out.c()
    _check(lib.lct_momentum_step(C.byref(cw), C.byref(a), C.byref(cm), C.byref(b), _ptr(g), mu, eta,
                                 C.byref(ow), C.byref(om), _stream(stream)), "lct_momentum_step")


# ------------------------------------------------------------------ conveniences

def encode(cb: Codebook, x: torch.Tensor, lay: Layout, ovf_cap: int | None = None,
           scratch=None) -> LctTensor:
    out = alloc_tensor(x.numel(), lay, ovf_cap, x.device, scratch)
    lct_encode(cb, x, out)
    return out


def decode(cb: Codebook, t: LctTensor) -> torch.Tensor:
    y = torch.empty(max(t.n, 1), dtype=torch.bfloat16, device=t.sf.device)[:t.n]
    lct_decode(cb, t, y)
    return y


def sgd_step(cw: Codebook, w: LctTensor, cm: Codebook, m: LctTensor, eta: float,
             out: LctTensor | None = None, ovf_cap: int | None = None) -> LctTensor:
    if out is None:
        out = alloc_tensor(w.n, w.layout, ovf_cap, w.sf.device)
    lct_sgd_step(cw, w, cm, m, eta, out)
    return out


def momentum_step(cw: Codebook, w: LctTensor, cm: Codebook, m: LctTensor, g: torch.Tensor,
                  mu: float, eta: float, w_out: LctTensor | None = None, m_out: LctTensor | None = None,
                  ovf_cap: int | None = None):
    if w_out is None:
        w_out = alloc_tensor(w.n, w.layout, ovf_cap, w.sf.device)
    if m_out is None:
        m_out = alloc_tensor(m.n, m.layout, ovf_cap, m.sf.device)
    lct_momentum_step(cw, w, cm, m, g, mu, eta, w_out, m_out)
    return w_out, m_out


# ------------------------------------------------------------------ tensor groups

class LctGroup:
    """A bound group: the device table, the host arrays the C struct points
    at (kept alive here), the codebooks and the dense tensors."""

    def __init__(self, ns, lay: Layout, codebooks, dense=None, device="cuda", fit=False, shift=None,
                 stream=None):
        """fit: one tensor (ns[0] elements, dense[0]) whose codebook is fitted
        on the device from codebooks[0]'s base code (lct_group_fit); the shift
        goes to the device int32 tensor `shift`."""
        count = len(ns)
        if len(codebooks) != count or (dense is not None and len(dense) != count):
            raise ValueError("one codebook (and one dense tensor) per size")
        self.count, self.layout = count, Layout(lay.block_elems, lay.cap_words)
        self.ns = (C.c_uint64 * count)(*[int(v) for v in ns])
        self.codebooks = (Codebook * count)(*codebooks)
        self.dense = list(dense) if dense is not None else None
        self.dense_ptrs = None
        if dense is not None:
            for t, nk in zip(dense, ns):
                _bits16(t)
                if t.numel() < int(nk):
                    raise ValueError("a dense tensor has %d elements, its member %d" % (t.numel(), int(nk)))
            self.dense_ptrs = (C.c_void_p * count)(*[t.data_ptr() for t in dense])
        nbytes = C.c_uint64(0)
        _check(lib.lct_group_table_bytes(count, self.ns, C.byref(self.layout), C.byref(nbytes)),
               "lct_group_table_bytes")
        self.table = torch.empty(max(int(nbytes.value), 256), dtype=torch.uint8, device=device)
        self.g = Group()
        if fit:
            if count != 1 or dense is None:
                raise ValueError("a fitted group holds one tensor with its dense buffer")
            _check(lib.lct_group_fit(C.byref(self.codebooks[0]), self.ns, self.dense_ptrs, C.byref(self.layout),
                                     _ptr(self.table), _ptr(shift), _stream(stream), C.byref(self.g)),
                   "lct_group_fit")
        else:
            # the table's memory may come from a tensor freed while work that
            # uses it is still queued on the current stream, and the bind's
            # blocking copy is not ordered with that stream
            torch.cuda.current_stream(self.table.device).synchronize()
            _check(lib.lct_group_bind(count, self.ns, C.byref(self.layout), self.codebooks,
                                      self.dense_ptrs, _ptr(self.table), C.byref(self.g)), "lct_group_bind")

    def sizes(self, ovf_cap: int = 0) -> Sizes:
        out = Sizes()
        _check(lib.lct_group_sizes(C.byref(self.g), ovf_cap, C.byref(out)), "lct_group_sizes")
        return out

    def alloc_storage(self, ovf_cap: int, device="cuda", scratch=None, ovf=None) -> LctTensor:
        sz = self.sizes(ovf_cap)
        dev = torch.device(device)
        u8 = torch.uint8
        if scratch is None:
            scratch = torch.empty(sz.scratch, dtype=u8, device=dev)
        elif scratch.numel() < sz.scratch:
            raise ValueError("scratch too small: %d < %d" % (scratch.numel(), sz.scratch))
        if ovf is None:
            ovf = torch.empty(max(ovf_cap, 16), dtype=u8, device=dev)
        elif ovf.numel() < ovf_cap:
            raise ValueError("ovf too small: %d < %d" % (ovf.numel(), ovf_cap))
        # the padding after each member is zeroed once: no call writes it,
        # so it stays zero; obase is zeroed because a group with no blocks
        # is a no-op whose encoding is obase = [0]
        sf = torch.empty(max(sz.sf, 16), dtype=u8, device=dev)
        if self.count == 1:
            if int(self.ns[0]) % 256:
                sf[int(self.ns[0]):].zero_()
        else:
            sf.zero_()
        return LctTensor.wrap(int(self.g.sf_bytes), self.layout, ovf_cap, sz, sf,
                              torch.empty(max(sz.pay // 4, 4), dtype=torch.int32, device=dev),
                              torch.empty(max(sz.cnt // 2, 2), dtype=torch.int16, device=dev),
                              torch.zeros(sz.obase // 8, dtype=torch.int64, device=dev),
                              ovf, torch.zeros(4, dtype=torch.int32, device=dev), scratch)

    def tensor(self, all_: LctTensor, k: int) -> LctTensor:
        """Tensor k as views of the storage (its obase values index the shared
        overflow region; read it with any call, write the group with the
        group calls)."""
        t = _Tensor()
        a = all_.c()
        _check(lib.lct_group_tensor(C.byref(self.g), C.byref(a), k, C.byref(t)), "lct_group_tensor")
        n = int(self.ns[k])
        sz = lct_sizes(n, self.layout, all_.ovf_cap)
        sf0 = (t.sf or 0) - all_.sf.data_ptr()
        pay0 = ((t.pay or 0) - all_.pay.data_ptr()) // 4
        cnt0 = ((t.cnt or 0) - all_.cnt.data_ptr()) // 2
        ob0 = ((t.obase or 0) - all_.obase.data_ptr()) // 8
        return LctTensor.wrap(n, self.layout, all_.ovf_cap, sz, all_.sf[sf0:sf0 + max(n, 1)],
                              all_.pay[pay0:pay0 + sz.pay // 4], all_.cnt[cnt0:cnt0 + sz.cnt // 2],
                              all_.obase[ob0:ob0 + sz.obase // 8], all_.ovf, all_.status, all_.scratch)


def lct_encode_group(g: LctGroup, all_: LctTensor, stream=None) -> None:
    a = all_.c()
    _check(lib.lct_encode_group(C.byref(g.g), C.byref(a), _stream(stream)), "lct_encode_group")


def lct_decode_group(g: LctGroup, all_: LctTensor, stream=None) -> None:
    a = all_.c()
    _check(lib.lct_decode_group(C.byref(g.g), C.byref(a), _stream(stream)), "lct_decode_group")


def lct_sgd_step_group(gw: LctGroup, w_all: LctTensor, gm: LctGroup, m_all: LctTensor, eta: float,
                       w_out: LctTensor, stream=None) -> None:
    a, b, o = w_all.c(), m_all.c(), w_out.c()
    _check(lib.lct_sgd_step_group(C.byref(gw.g), C.byref(a), C.byref(gm.g), C.byref(b), eta,
                                  C.byref(o), _stream(stream)), "lct_sgd_step_group")


def lct_momentum_step_group(gw: LctGroup, w_all: LctTensor, gm: LctGroup, m_all: LctTensor,
                            gg: LctGroup, mu: float, eta: float, w_out: LctTensor, m_out: LctTensor,
                            stream=None) -> None:
    a, b, ow, om = w_all.c(), m_all.c(), w_out.c(), m_out.c()
    _check(lib.lct_momentum_step_group(C.byref(gw.g), C.byref(a), C.byref(gm.g), C.byref(b), C.byref(gg.g),
                                       mu, eta, C.byref(ow), C.byref(om), _stream(stream)),
           "lct_momentum_step_group")
