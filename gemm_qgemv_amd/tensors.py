"""torch helpers around the C ABI: put a packed weight set on the device and
allocate a workspace of the size the library asks for. torch only provides
device memory here; no arithmetic happens in this module."""
from __future__ import annotations

import dataclasses

import numpy as np

from . import _binding as B


@dataclasses.dataclass
class DeviceWeights:
    fmt: int
    M: int
    K: int
    codes: "object"   # torch tensor (int8 or uint8)
    scales: "object"  # torch tensor (float32, or int16 holding bf16/fp16 bits)
    biases: "object"  # torch tensor (int16 holding bf16 bits) or None

    @property
    def nbytes(self) -> int:
        n = self.codes.numel() * self.codes.element_size()
        n += self.scales.numel() * self.scales.element_size()
        if self.biases is not None:
            n += self.biases.numel() * self.biases.element_size()
        return n


def _dev(a: np.ndarray, device):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)   # same bits; torch's int16 copies everywhere
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(w, device="cuda") -> DeviceWeights:
    """Copy a synth.QWeights (numpy) to the device."""
    return DeviceWeights(w.fmt, w.M, w.K, _dev(w.codes, device), _dev(w.scales, device),
                         None if w.biases is None else _dev(w.biases, device))


def workspace(op: int, fmt: int, M: int, K: int, rows: int, device="cuda"):
    """A device workspace of qg_workspace_bytes(...) bytes (None if 0). Its
    contents on entry do not matter (every kernel launch claims the
    completion words it counts on), so it is left uninitialised."""
    import torch
    n = B.qg_workspace_bytes(op, fmt, M, K, rows)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)
