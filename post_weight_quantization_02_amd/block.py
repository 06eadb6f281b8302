"""Several layers quantized in one call order, as a transformer block's
linear layers are: one Hessian per calibration stream, one Hinv per
stream shared by every layer that reads that stream, and one workspace for
every call.

The pages quantize layer after layer, each from the Hessian of its own
inputs ("GPTQ: fixing errors as you go", "The algorithm, in words"); layers
that read the same inputs (a block's q, k and v projections; its gate and up
projections) share that Hessian, so H, its preparation and Hinv are formed
once per stream. This module only sequences entry points of the library;
every step runs in its kernels.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Optional

from . import _lib


@dataclasses.dataclass
class BlockLayer:
    """One layer: W (rows x cols, fp16/fp32, on the device), its quantizer,
    and its preallocated outputs (codes, scales, zeros, losses[, g_idx])."""
    W: object
    bits: int = 4
    groupsize: int = 128
    blocksize: int = 128
    out: Optional[tuple] = None


@dataclasses.dataclass
class BlockStream:
    """One calibration stream: X (tokens x d fp16), the H and Hinv buffers
    (d x d fp32), perm (d int32) for act-order, and the layers it feeds."""
    X: object
    H: object
    U: object
    layers: List[BlockLayer]
    percdamp: float = 0.01
    perm: object = None


def allocate_outputs(torch, W, groupsize: int, act_order: bool = False):
    rows, cols = W.shape
    g = cols if groupsize <= 0 else groupsize
    ng = (cols + g - 1) // g
    dev = W.device
    out = (torch.empty((rows, cols), dtype=torch.uint8, device=dev),
           torch.empty((rows, ng), dtype=torch.float32, device=dev),
           torch.empty((rows, ng), dtype=torch.float32, device=dev),
           torch.empty((cols,), dtype=torch.float32, device=dev))
    if act_order:
        out = out + (torch.empty((cols,), dtype=torch.int32, device=dev),)
    return out


def workspace_bytes(streams: List[BlockStream], act_order: bool = False) -> int:
    """The largest workspace any call of the sequence needs."""
    op = _lib.OP_QUANTIZE_PERM if act_order else _lib.OP_QUANTIZE
    need = 0
    for st in streams:
        n, d = st.X.shape
        need = max(need, _lib.workspace_bytes(_lib.OP_ACCUMULATE, 0, d, n),
                   _lib.workspace_bytes(_lib.OP_PREPARE, 0, d, 0))
        for ly in st.layers:
            need = max(need, _lib.workspace_bytes(op, ly.W.shape[0], d, 0))
    return need


def quantize_streams(streams: List[BlockStream], workspace, act_order: bool = False,
                     stream=None, mark: Optional[Callable[[str, bool], None]] = None):
    """For each stream in order: H = 0, H += 2 X^T X, Hinv (with act-order,
    the order of decreasing diag(H) first), then every layer of the stream in
    order with that Hinv. `mark(phase, begin)` is called around the
    accumulate ("acc"), the preparation ("prep") and each layer ("quant")."""
    note = mark if mark is not None else (lambda phase, begin: None)
    for st in streams:
        st.H.zero_()
        note("acc", True)
        _lib.hessian_accumulate(st.H, st.X, 2.0, workspace=workspace, stream=stream)
        note("acc", False)
        note("prep", True)
        if act_order:
            _lib.act_order(st.H, out=st.perm, stream=stream)
            _lib.prepare_hinv_perm(st.H, st.perm, st.percdamp, out=st.U, workspace=workspace,
                                   stream=stream)
        else:
            _lib.prepare_hinv(st.H, st.percdamp, out=st.U, workspace=workspace, stream=stream)
        note("prep", False)
        for ly in st.layers:
            note("quant", True)
            if act_order:
                _lib.quantize_layer_perm(ly.W, st.perm, st.U, ly.bits, ly.groupsize, ly.blocksize,
                                         out=ly.out, workspace=workspace, stream=stream)
            else:
                _lib.quantize_layer(ly.W, st.U, ly.bits, ly.groupsize, ly.blocksize, out=ly.out,
                                    workspace=workspace, stream=stream)
            note("quant", False)
