"""Compressed saving of activations for backward.

The LCT abstract lists activations among the tensors LCT keeps compressed
during training, next to weights and optimizer state; the explainer's results
paragraph credits part of NanoGPT's memory saving to them.  Here autograd's
saved-tensor hooks do it: a BF16 tensor on the GPU that autograd saves for
backward is encoded when it is saved and decoded when backward asks for it.
The encode, the decode and the per-tensor shift sample all run in the HIP
library; this module only decides what to encode and owns the buffers.

Per saved tensor:
  - codebook: the context's base code (from the model the user picks) with
    the shift re-estimated from the tensor's own 4096-element sample
    (lct_codebook_reshift_dense, no Huffman rebuild);
  - buffers: the fixed side at its exact size; the spilled bytes land in a
    staging region shared by the context, large enough for every element to
    spill, and are then copied into a buffer of exactly their size.

A save waits twice for the device: for the sample that sets the shift, and
for the spilled total that sizes the kept overflow buffer.

Tensors that are not BF16, not on the GPU, not contiguous, smaller than
`min_elems`, or leaves that require grad (parameters, which autograd saves by
reference at no cost) are saved as they are.
"""
from __future__ import annotations

import time
from contextlib import contextmanager
from dataclasses import dataclass

import torch

from . import (CLEAN, GAUSSIAN, Codebook, LctTensor, Model, alloc_tensor,
               lct_codebook_build, lct_codebook_reshift_dense, lct_decode, lct_encode,
               lct_layout_init, lct_sizes)


@dataclass
class _Saved:
    t: LctTensor
    cb: Codebook
    shape: torch.Size


class ActivationCodec:
    """pack/unpack hooks with their staging buffers and byte counts."""

    def __init__(self, model: Model | None = None, mode: int = CLEAN, min_elems: int = 1 << 16):
        self.model = Model(GAUSSIAN, 1.0, 0.0) if model is None else model
        self.base = lct_codebook_build(self.model, None)
        self.layout = lct_layout_init(mode)
        self.min_elems = int(min_elems)
        self._scratch = None
        self._ovf = None
        self.saved = 0           # tensors encoded
        self.passed = 0          # tensors kept as they are
        self.raw_bytes = 0       # BF16 bytes of the encoded tensors
        self.stored_bytes = 0    # their fixed sides plus spilled bytes
        self.pack_s = 0.0        # host time spent in pack (waits for the device included)
        self.unpack_s = 0.0      # host time spent in unpack

    def _wants(self, x: torch.Tensor) -> bool:
        return (x.dtype == torch.bfloat16 and x.is_cuda and x.is_contiguous()
                and x.numel() >= self.min_elems and not (x.is_leaf and x.requires_grad))

    def _staging(self, n: int, need_ovf: int, device):
        sz = lct_sizes(n, self.layout, need_ovf)
        if self._scratch is None or self._scratch.numel() < sz.scratch or self._scratch.device != device:
            self._scratch = torch.empty(sz.scratch, dtype=torch.uint8, device=device)
        if self._ovf is None or self._ovf.numel() < need_ovf or self._ovf.device != device:
            self._ovf = torch.empty(max(need_ovf, 16), dtype=torch.uint8, device=device)

    def pack(self, x: torch.Tensor):
        if not self._wants(x):
            self.passed += 1
            return x
        t0 = time.perf_counter()
        n = x.numel()
        xd = x.detach()
        cb = lct_codebook_reshift_dense(self.base, xd.view(-1))
        # a staging region of n bytes holds every possible spill: one encode
        self._staging(n, n, x.device)
        t = alloc_tensor(n, self.layout, n, x.device, self._scratch, self._ovf)
        lct_encode(cb, xd.view(-1), t)
        spilled = t.spilled()                # synchronises
        # keep the spilled bytes in a buffer of their own size
        t.ovf = self._ovf[:max(spilled, 16)].clone()
        t.ovf_cap = spilled
        t.scratch = None
        self.saved += 1
        self.raw_bytes += 2 * n
        self.stored_bytes += int(t.sizes.fixed) + spilled
        self.pack_s += time.perf_counter() - t0
        return _Saved(t, cb, x.shape)

    def unpack(self, h):
        if not isinstance(h, _Saved):
            return h
        t0 = time.perf_counter()
        y = torch.empty(h.shape, dtype=torch.bfloat16, device=h.t.sf.device)
        lct_decode(h.cb, h.t, y.view(-1))
        self.unpack_s += time.perf_counter() - t0
        return y

    def ratio(self) -> float:
        return self.raw_bytes / self.stored_bytes if self.stored_bytes else 0.0


@contextmanager
def compressed_activations(model: Model | None = None, mode: int = CLEAN, min_elems: int = 1 << 16):
    """Within the block, tensors autograd saves for backward are stored
    compressed (see the module docstring); yields the codec for its counts."""
    codec = ActivationCodec(model, mode, min_elems)
    with torch.autograd.graph.saved_tensors_hooks(codec.pack, codec.unpack):
        yield codec
