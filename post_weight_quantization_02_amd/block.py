"""Several layers quantized in one call order, as a transformer block's
linear layers are: one Hessian per calibration stream, one Hinv per
stream shared by every layer that reads that stream, and one workspace for
every call.

The pages quantize layer after layer, each from the Hessian of its own
inputs ("GPTQ: fixing errors as you go", "The algorithm, in words"); layers
that read the same inputs (a block's q, k and v projections; its gate and up
projections) share that Hessian, so H, its preparation and Hinv are formed
once per stream. The streams of a block are independent, so they may also
run concurrently, in lanes of their own (quantize_streams_concurrent). This
module only sequences entry points of the library; every step runs in its
kernels.
"""
from __future__ import annotations

import dataclasses
import threading
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
    three_step: bool = False  # Hinv by the pages' three steps (no act-order)


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


def stream_workspace_bytes(st: BlockStream, act_order: bool = False) -> int:
    """The largest workspace any call of one stream's sequence needs."""
    op = _lib.OP_QUANTIZE_PERM if act_order else _lib.OP_QUANTIZE
    n, d = st.X.shape
    need = max(_lib.workspace_bytes(_lib.OP_ACCUMULATE, 0, d, n),
               _lib.workspace_bytes(_lib.OP_PREPARE, 0, d, 0))
    for ly in st.layers:
        need = max(need, _lib.workspace_bytes(op, ly.W.shape[0], d, 0))
    return need


def workspace_bytes(streams: List[BlockStream], act_order: bool = False) -> int:
    """The largest workspace any call of the sequence needs."""
    return max([stream_workspace_bytes(st, act_order) for st in streams] + [0])


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
        elif st.three_step:
            _lib.prepare_hinv_three_step(st.H, st.percdamp, out=st.U, workspace=workspace,
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


def lane_assignment(streams: List[BlockStream], lanes: int) -> List[List[int]]:
    """Calibration streams grouped into `lanes` lanes: largest stream
    (tokens x channels x channels) first, each to the lane with the least
    work so far; the lane keeps the streams' original order."""
    work = [st.X.shape[0] * st.X.shape[1] * st.X.shape[1] for st in streams]
    lanes = max(1, min(lanes, len(streams)))
    load = [0] * lanes
    out = [[] for _ in range(lanes)]
    for i in sorted(range(len(streams)), key=lambda i: -work[i]):
        j = min(range(lanes), key=lambda j: load[j])
        out[j].append(i)
        load[j] += work[i]
    return [sorted(l) for l in out if l]


def quantize_streams_concurrent(streams: List[BlockStream], workspaces, act_order: bool = False,
                                device_streams=None,
                                mark: Optional[Callable[[str, bool], None]] = None):
    """quantize_streams with the calibration streams in lanes, each lane on a
    device stream of its own, driven by a host thread of its own (the
    preparation waits on its stream for the pivot flag, and the library calls
    release the GIL), so the lanes' work overlaps on the GPU: one stream's
    serial factorization chain and latency-bound sweeps leave most CUs to the
    others. len(workspaces) is the number of lanes (see lane_assignment); a
    lane runs its streams in order with workspaces[lane], at least the
    largest stream_workspace_bytes of its streams, and the lanes share no
    buffer, so the results are those of quantize_streams. device_streams:
    one torch.cuda.Stream per lane (created when None). The work starts after
    what is queued on the caller's current stream, and that stream waits for
    all of it on return. `mark` is called from the lane's own thread, with
    its device stream current."""
    from ._lib import _torch
    torch = _torch()
    if not streams:
        return
    lanes = lane_assignment(streams, len(workspaces))
    if len(lanes) != len(workspaces):
        raise ValueError("more workspaces than streams")
    dev = streams[0].X.device
    caller = torch.cuda.current_stream(dev)
    if device_streams is None:
        device_streams = [torch.cuda.Stream(device=dev) for _ in lanes]
    if len(device_streams) < len(lanes):
        raise ValueError("one device stream per lane is needed")
    ready = torch.cuda.Event()
    ready.record(caller)
    errors = [None] * len(lanes)

    def run(j):
        try:
            torch.cuda.set_device(dev)
            s = device_streams[j]
            with torch.cuda.stream(s):
                s.wait_event(ready)
                quantize_streams([streams[i] for i in lanes[j]], workspaces[j], act_order,
                                 stream=s, mark=mark)
        except BaseException as e:  # re-raised in the caller's thread
            errors[j] = e

    threads = [threading.Thread(target=run, args=(j,)) for j in range(len(lanes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for s in device_streams:
        caller.wait_stream(s)
    for e in errors:
        if e is not None:
            raise e


def lane_workspace_bytes(streams: List[BlockStream], lanes: int, act_order: bool = False):
    """Workspace bytes of each lane of lane_assignment(streams, lanes)."""
    return [max(stream_workspace_bytes(streams[i], act_order) for i in l)
            for l in lane_assignment(streams, lanes)]
