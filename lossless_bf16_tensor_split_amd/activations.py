"""Compressed saving of activations for backward.

The LCT abstract lists activations among the tensors LCT keeps compressed
during training, next to weights and optimizer state; the explainer's results
paragraph credits part of NanoGPT's memory saving to them.  Here autograd's
saved-tensor hooks do it: a BF16 tensor on the GPU that autograd saves for
backward is encoded when it is saved and decoded when backward asks for it.
The encode, the decode and the per-tensor codebook fit all run in the HIP
library; this module only decides what to encode and owns the buffers.

Per saved tensor:
  - codebook: the context's base code (from the model the user picks) with
    the shift chosen from the tensor's own 4096-element sample, the same
    choice as lct_codebook_reshift_dense, made and turned into tables on the
    device (lct_group_fit), so a save never waits for the device;
  - buffers: the fixed side at its exact size; the spilled bytes land in a
    staging region (large enough for every element, in whole blocks, to
    spill) taken from a small pool.  The shift and the spilled total are copied to pinned host
    memory behind an event; once the event has passed, the spilled bytes move
    to a buffer of exactly their size, the staging region returns to the
    pool, and the host codebook for the decode is made from the shift.  A
    save that finds the pool empty waits for the oldest save's event; the
    block's end and a backward read of a save still in flight wait for it.
  - streams: a save runs on the current stream.  Each staging slot has its
    own scratch, and a slot taken again waits (on the device) for the trim
    that last read it, so saves made on different streams do not race; a
    restore on another stream than its save's waits for the trim and keeps
    the saved buffers alive until its decode is done.

Tensors that are not BF16, not on the GPU, not contiguous, smaller than
`min_elems`, or leaves that require grad (parameters, which autograd saves by
reference at no cost) are saved as they are.

A codec keeps its staging pool, pinned words and base code across uses:
a training loop makes one and enters it once per step (`with codec:`), so
only the first step pays for the setup.  `compressed_activations` makes a
fresh codec for one block.
"""
from __future__ import annotations

import time
from collections import deque
from contextlib import contextmanager
from dataclasses import dataclass

import torch

from . import (CLEAN, POWERLAW, Codebook, LctGroup, LctTensor, Model, full_ovf_cap, lct_codebook_build,
               lct_codebook_from_lengths, lct_decode, lct_encode_group, lct_layout_init, lct_sizes)


_BASE = {}


def _base_code(model: Model) -> Codebook:
    """The model's base code (shift 0), built once per model: it depends on
    the model alone, and codecs only read it."""
    key = (int(model.family), float(model.scale), float(model.shape))
    cb = _BASE.get(key)
    if cb is None:
        cb = _BASE[key] = lct_codebook_build(model, None)
    return cb


@dataclass
class _Saved:
    t: LctTensor                 # the tensor (n elements) over the group storage's buffers
    grp: LctGroup | None         # its one-tensor group (device tables), until the encode is done
    shape: torch.Size
    cb: Codebook | None = None   # host codebook, once the shift is known
    stream: torch.cuda.Stream | None = None   # the stream its buffers were made and written on
    ready: torch.cuda.Event | None = None     # recorded on it once the spills are trimmed


class ActivationCodec:
    """pack/unpack hooks with their staging buffers and byte counts."""

    def __init__(self, model: Model | None = None, mode: int = CLEAN, min_elems: int = 1 << 16,
                 pool: int = 3):
        # Default: Student-t with 3 degrees of freedom.  Products of activations
        # (a gated MLP's silu(g) * u) have heavy tails that a Gaussian code sends
        # to the escape and, past a stream's capacity, to the overflow region;
        # the t code keeps near-Gaussian tensors at the same size.
        self.model = Model(POWERLAW, 1.0, 3.0) if model is None else model
        self.base = _base_code(self.model)
        self.len_base = list(self.base.len_base)
        self.layout = lct_layout_init(mode)
        self.min_elems = int(min_elems)
        self._stage = [None] * pool          # staging regions
        self._scratch = [None] * pool        # each slot's scratch
        self._slot_ev = [None] * pool        # recorded after the trim that last read each slot
        self._free = list(range(pool))
        self._shift = None                   # device int32 per slot: the fitted shift
        self._pin_shift = None               # pinned host copies: shift (int32) and
        self._pin_spill = None               # spilled total (int64) per slot
        self._pending = deque()              # (handle, slot, event, stream), oldest first
        self.saved = 0           # tensors encoded
        self.passed = 0          # tensors kept as they are
        self.raw_bytes = 0       # BF16 bytes of the encoded tensors
        self.stored_bytes = 0    # their fixed sides plus spilled bytes
        self.pack_s = 0.0        # host time spent in pack (waits for the device included)
        self.unpack_s = 0.0      # host time spent in unpack
        self._hooks = None

    def _wants(self, x: torch.Tensor) -> bool:
        return (x.dtype == torch.bfloat16 and x.is_cuda and x.is_contiguous()
                and x.numel() >= self.min_elems and not (x.is_leaf and x.requires_grad))

    def _finish(self, entry):
        """A save whose event has passed: its shift and spilled total are in
        pinned memory; trim its spills, make its host codebook, free its slot."""
        h, slot, _, stream = entry
        shift, spilled = int(self._pin_shift[slot]), int(self._pin_spill[slot])
        h.grp = None                         # its table and the reference to the input go
        with torch.cuda.stream(stream):
            h.t.ovf = self._stage[slot][:max(spilled, 16)].clone()
            h.ready = torch.cuda.Event()
            h.ready.record(stream)
        self._slot_ev[slot] = h.ready
        h.t.ovf_cap = spilled
        h.cb = lct_codebook_from_lengths(self.len_base, self.base.esc_len, shift)
        self.stored_bytes += int(h.t.sizes.fixed) + spilled
        self._free.append(slot)

    def _reap(self, wait_one: bool = False):
        """Finish every save whose event has passed, in order; with wait_one,
        wait for the oldest if none has."""
        while self._pending:
            e = self._pending[0][2]
            if not e.query():
                if not wait_one:
                    break
                e.synchronize()
            wait_one = False
            self._finish(self._pending.popleft())

    def pack(self, x: torch.Tensor):
        if not self._wants(x):
            self.passed += 1
            return x
        t0 = time.perf_counter()
        dev = x.device
        n = x.numel()
        xd = x.detach().view(-1)
        stream = torch.cuda.current_stream(dev)
        self._reap()
        if not self._free:
            self._reap(wait_one=True)
        slot = self._free.pop()
        if self._slot_ev[slot] is not None:
            # the slot's last trim may have run on another stream
            stream.wait_event(self._slot_ev[slot])
        if self._shift is None:
            self._pin_shift = torch.zeros(len(self._stage), dtype=torch.int32, pin_memory=True)
            self._pin_spill = torch.zeros(len(self._stage), dtype=torch.int64, pin_memory=True)
            self._shift = torch.zeros(len(self._stage), dtype=torch.int32, device=dev)
        # room for every element in whole blocks: the encode stages spilled
        # fields at fixed places (see full_ovf_cap)
        cap = full_ovf_cap(n, self.layout)
        st = self._stage[slot]
        if st is None or st.numel() < cap or st.device != dev:
            self._stage[slot] = st = torch.empty(max(cap, 16), dtype=torch.uint8, device=dev)
        sz = lct_sizes(n, self.layout, cap)
        scr = self._scratch[slot]
        if scr is None or scr.numel() < sz.scratch or scr.device != dev:
            self._scratch[slot] = scr = torch.empty(sz.scratch, dtype=torch.uint8, device=dev)
        # the codebook fitted on the device, then the encode with its tables
        grp = LctGroup([n], self.layout, [self.base], [xd], device=dev, fit=True,
                       shift=self._shift[slot:slot + 1], stream=stream)
        all_ = grp.alloc_storage(cap, dev, scr, st)
        lct_encode_group(grp, all_, stream)
        self._pin_shift[slot:slot + 1].copy_(self._shift[slot:slot + 1], non_blocking=True)
        self._pin_spill[slot:slot + 1].copy_(all_.obase[-1:], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        t = LctTensor.wrap(n, self.layout, cap, lct_sizes(n, self.layout, cap), all_.sf, all_.pay, all_.cnt,
                           all_.obase, st, all_.status, None)
        h = _Saved(t, grp, x.shape, stream=stream)
        self._pending.append((h, slot, ev, stream))
        self.saved += 1
        self.raw_bytes += 2 * n
        self.pack_s += time.perf_counter() - t0
        return h

    def unpack(self, h):
        if not isinstance(h, _Saved):
            return h
        t0 = time.perf_counter()
        while h.cb is None:                  # still in flight: finish saves up to it
            self._reap(wait_one=True)
        cur = torch.cuda.current_stream(h.t.sf.device)
        if cur != h.stream:
            cur.wait_event(h.ready)
            for b in (h.t.sf, h.t.pay, h.t.cnt, h.t.obase, h.t.ovf):
                b.record_stream(cur)
        y = torch.empty(h.shape, dtype=torch.bfloat16, device=h.t.sf.device)
        lct_decode(h.cb, h.t, y.view(-1))
        self.unpack_s += time.perf_counter() - t0
        return y

    def close(self):
        """Finish every save still in flight (waits for their events)."""
        while self._pending:
            self._reap(wait_one=True)

    def __enter__(self):
        """Install the pack/unpack hooks for the block (one step's forward;
        backward may run inside or after it)."""
        if self._hooks is not None:
            raise RuntimeError("the codec is already entered")
        self._hooks = torch.autograd.graph.saved_tensors_hooks(self.pack, self.unpack)
        self._hooks.__enter__()
        return self

    def __exit__(self, *exc):
        try:
            self._hooks.__exit__(*exc)
        finally:
            self._hooks = None
            self.close()
        return False

    def ratio(self) -> float:
        return self.raw_bytes / self.stored_bytes if self.stored_bytes else 0.0


@contextmanager
def compressed_activations(model: Model | None = None, mode: int = CLEAN, min_elems: int = 1 << 16):
    """Within the block, tensors autograd saves for backward are stored
    compressed (see the module docstring); yields the codec for its counts."""
    with ActivationCodec(model, mode, min_elems) as codec:
        yield codec
