"""Layer-by-layer quantization of an up -> ReLU -> down block on the GPU.

Quantization proceeds one layer at a time: the calibration data is run
through the model as it stands, the next layer's inputs are recorded, its H is
formed and it is quantized ("GPTQ: fixing errors as you go", "The algorithm,
in words"; "GPTQ > The GPTQ Algorithm", the procedure's first step). So the
second layer's inputs are the outputs of the already quantized first layer,
y1 = fp16(max(x W1_hat^T, 0)), produced from the first layer's stored form.

Every step runs in the library's kernels (accumulate, prepare, quantize, pack,
forward product); this module only sequences the entry points and owns the
intermediate buffers.
"""
from __future__ import annotations

import contextlib

from . import _lib


def quantize_relu_block(x, W1, W2, bits: int = 4, groupsize: int = 128, blocksize: int = 128,
                        percdamp: float = 0.01, timer=None):
    """x: n x d fp16 calibration inputs of the block; W1: m x d and W2: d_out x m
    (fp16 or fp32) on the GPU. Returns a dict with, per layer, codes, scales,
    zeros, losses and H, plus y1 (n x m fp16, the recorded inputs of the
    second layer) and the first layer's packed codes.

    ``timer``, if given, is a context-manager factory ``timer(name)`` wrapped
    around each phase (the benchmark's event pairs)."""
    torch = _lib._torch()
    if bits not in (4, 8):
        raise ValueError("the block's forward product takes 4- or 8-bit codes")
    d, m = x.shape[1], W1.shape[0]
    if W1.shape[1] != d or W2.shape[1] != m:
        raise ValueError("shapes: x n x d, W1 m x d, W2 d_out x m")

    def phase(name):
        return contextlib.nullcontext() if timer is None else timer(name)

    out = {}
    with phase("acc1"):
        H1 = torch.zeros((d, d), dtype=torch.float32, device=x.device)
        _lib.hessian_accumulate(H1, x, 2.0)
    with phase("prep1"):
        U1 = _lib.prepare_hinv(H1, percdamp)
    with phase("quant1"):
        c1, s1, z1, l1 = _lib.quantize_layer(W1, U1, bits, groupsize, blocksize)
    with phase("pack1"):
        p1 = _lib.pack_codes(c1, bits)
    with phase("forward1"):
        y1 = _lib.linear_forward(x, p1, bits, d, s1, z1, groupsize, relu=True)
    with phase("acc2"):
        H2 = torch.zeros((m, m), dtype=torch.float32, device=x.device)
        _lib.hessian_accumulate(H2, y1, 2.0)
    with phase("prep2"):
        U2 = _lib.prepare_hinv(H2, percdamp)
    with phase("quant2"):
        c2, s2, z2, l2 = _lib.quantize_layer(W2, U2, bits, groupsize, blocksize)
    out["first"] = dict(codes=c1, scales=s1, zeros=z1, losses=l1, H=H1, packed=p1)
    out["second"] = dict(codes=c2, scales=s2, zeros=z2, losses=l2, H=H2)
    out["y1"] = y1
    return out
