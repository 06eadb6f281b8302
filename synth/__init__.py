"""Seeded synthetic inputs for one GPTQ layer: weights W and calibration
activations X.

This module is shared by the HIP path's tests/bench and by the fp64 oracle.
It holds no arithmetic of the quantization method itself: it only draws
random numbers and shapes them into the workloads the pages describe.

Workloads (stand-ins for the pages' calibration setting of 128 sequences x
2048 tokens of web text, page "GPTQ: fixing errors as you go", section
"a 4-bit Llama layer"; the corpus is not available, so X is drawn from a
low-rank-plus-noise model instead):

* ``tiny``     W 64x256 fp32 ~N(0, 0.02^2); X 512 tokens x 256 channels,
               Z(512x32)N(0,1) . A(32x256)N(0,1/32) + 0.1 N(0,1),
               channels 0-3 scaled x20.
* ``attn``     Llama-7B attention projection: W 4096x4096 fp16 ~N(0,0.02^2);
               X 262144 tokens x 4096, rank 256 + 0.1 noise, 40 random
               outlier channels scaled x20.
* ``mlp_up``   W 11008x4096 fp16 ~N(0,0.02^2), int3; X identical to ``attn``.
* ``mlp_down`` W 4096x11008 fp16 ~N(0,0.015^2); X 262144 x 11008, rank 256 +
               0.1 noise, shifted ReLU so that 60% of entries are zero, and
               220 (2%) dead channels that are all zero.

X is produced token-major (tokens x channels, the layout a forward hook
records) in chunks of ``CHUNK`` tokens. Every chunk has its own seed, so any
chunk can be regenerated alone and chunks can be produced in parallel.
The fp16 bytes returned here are the single source of truth: the GPU and the
oracle both consume exactly these values.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Iterator, Optional

import numpy as np

CHUNK = 8192

# seed stream ids
_S_W, _S_A, _S_Z, _S_NOISE, _S_OUTLIER, _S_DEAD = 1, 2, 3, 4, 5, 6

# Phi^{-1}(0.6): the standard-normal quantile below which 60% of the mass lies.
_PROBIT_0_6 = 0.2533471031357997


@dataclasses.dataclass(frozen=True)
class XSpec:
    """Low-rank-plus-noise activation model, tokens x d."""
    key: int                 # seed key of this activation stream
    d: int                   # channels (= W columns)
    n: int                   # tokens
    rank: int                # rank of the structured part Z.A
    noise: float = 0.1       # std of the isotropic noise
    outliers: int = 0        # number of randomly chosen outlier channels
    outlier_channels: tuple = ()  # fixed outlier channels (used by ``tiny``)
    outlier_scale: float = 20.0
    zero_frac: float = 0.0   # fraction of zeros made by a shifted ReLU
    dead: int = 0            # number of all-zero channels

    def scaled(self, d: Optional[int] = None, n: Optional[int] = None,
               rank: Optional[int] = None) -> "XSpec":
        """Same structure at a smaller size (for tests the oracle finishes fast)."""
        d2 = self.d if d is None else d
        fr = d2 / self.d
        return dataclasses.replace(
            self, d=d2, n=self.n if n is None else n,
            rank=self.rank if rank is None else rank,
            outliers=int(round(self.outliers * fr)) if self.outliers else 0,
            outlier_channels=tuple(c for c in self.outlier_channels if c < d2),
            dead=int(math.floor(self.dead * fr)) if self.dead else 0)


@dataclasses.dataclass(frozen=True)
class WSpec:
    key: int
    rows: int
    cols: int
    std: float
    dtype: str = "f16"       # "f16" or "f32"

    def scaled(self, rows: Optional[int] = None, cols: Optional[int] = None) -> "WSpec":
        return dataclasses.replace(self, rows=self.rows if rows is None else rows,
                                   cols=self.cols if cols is None else cols)


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    w: WSpec
    x: XSpec
    bits: int = 4
    groupsize: int = 128
    blocksize: int = 128
    percdamp: float = 0.01

    def scaled(self, rows=None, cols=None, n=None, rank=None) -> "Layer":
        return dataclasses.replace(self, w=self.w.scaled(rows, cols),
                                   x=self.x.scaled(cols, n, rank))


X_TINY = XSpec(key=100, d=256, n=512, rank=32, outlier_channels=(0, 1, 2, 3))
X_ATTN = XSpec(key=200, d=4096, n=128 * 2048, rank=256, outliers=40)
X_DOWN = XSpec(key=400, d=11008, n=128 * 2048, rank=256, zero_frac=0.6, dead=220)
# the other two activation streams of a Llama-7B block (o input, MLP input)
X_O = dataclasses.replace(X_ATTN, key=210)
X_MLP = dataclasses.replace(X_ATTN, key=220)

LAYERS = {
    "tiny": Layer("tiny", WSpec(10, 64, 256, 0.02, "f32"), X_TINY),
    "attn": Layer("attn", WSpec(20, 4096, 4096, 0.02), X_ATTN),
    "mlp_up": Layer("mlp_up", WSpec(30, 11008, 4096, 0.02), X_ATTN, bits=3),
    "mlp_down": Layer("mlp_down", WSpec(40, 4096, 11008, 0.015), X_DOWN),
}

# Llama-7B-shaped block: seven layers, four activation streams.
BLOCK = [
    Layer("q", WSpec(51, 4096, 4096, 0.02), X_ATTN),
    Layer("k", WSpec(52, 4096, 4096, 0.02), X_ATTN),
    Layer("v", WSpec(53, 4096, 4096, 0.02), X_ATTN),
    Layer("o", WSpec(54, 4096, 4096, 0.02), X_O),
    Layer("gate", WSpec(55, 11008, 4096, 0.02), X_MLP),
    Layer("up", WSpec(56, 11008, 4096, 0.02), X_MLP),
    Layer("down", WSpec(57, 4096, 11008, 0.02), X_DOWN),
]


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def weights(w: WSpec) -> np.ndarray:
    """W (rows x cols), ~N(0, std^2), returned as fp16 or fp32."""
    g = _rng(w.key, _S_W, w.rows, w.cols)
    a = g.standard_normal((w.rows, w.cols), dtype=np.float32) * np.float32(w.std)
    return a.astype(np.float16) if w.dtype == "f16" else a


def _mixing(x: XSpec) -> np.ndarray:
    g = _rng(x.key, _S_A, x.d, x.rank)
    return g.standard_normal((x.rank, x.d)) / math.sqrt(x.rank)


def _channel_sets(x: XSpec):
    out = np.array(x.outlier_channels, dtype=np.int64)
    if x.outliers:
        out = np.sort(_rng(x.key, _S_OUTLIER, x.d).choice(x.d, x.outliers, replace=False))
    dead = np.zeros(0, dtype=np.int64)
    if x.dead:
        dead = np.sort(_rng(x.key, _S_DEAD, x.d).choice(x.d, x.dead, replace=False))
    return out, dead


def dead_channels(x: XSpec) -> np.ndarray:
    return _channel_sets(x)[1]


def outlier_channels(x: XSpec) -> np.ndarray:
    return _channel_sets(x)[0]


def _chunk(x: XSpec, A: np.ndarray, out: np.ndarray, dead: np.ndarray,
           c: int, t0: int, t1: int) -> np.ndarray:
    m = t1 - t0
    Z = _rng(x.key, _S_Z, x.d, c).standard_normal((m, x.rank))
    N = _rng(x.key, _S_NOISE, x.d, c).standard_normal((m, x.d), dtype=np.float32)
    G = Z @ A
    G += x.noise * N
    if x.zero_frac:
        sigma = math.sqrt(1.0 + x.noise * x.noise)
        thr = _PROBIT_0_6 * sigma if abs(x.zero_frac - 0.6) < 1e-12 else None
        if thr is None:
            from scipy.special import ndtri
            thr = float(ndtri(x.zero_frac)) * sigma
        G -= thr
        np.maximum(G, 0.0, out=G)
    if out.size:
        G[:, out] *= x.outlier_scale
    if dead.size:
        G[:, dead] = 0.0
    return G.astype(np.float16)


def activation_chunks(x: XSpec, chunk: int = CHUNK,
                      t_begin: int = 0, t_end: Optional[int] = None) -> Iterator[np.ndarray]:
    """Yield X[t_begin:t_end] as fp16 (tokens x d) chunks of at most ``chunk``
    tokens. Chunk boundaries are fixed multiples of CHUNK, so the values do not
    depend on how the caller slices the token range."""
    assert chunk % CHUNK == 0 or CHUNK % chunk == 0
    t_end = x.n if t_end is None else min(t_end, x.n)
    A = _mixing(x)
    out, dead = _channel_sets(x)
    t = t_begin
    while t < t_end:
        c = t // CHUNK
        c0 = c * CHUNK
        c1 = min(c0 + CHUNK, x.n)
        blk = _chunk(x, A, out, dead, c, c0, c1)
        lo, hi = t - c0, min(t_end, c1) - c0
        yield blk[lo:hi]
        t = c0 + hi


def activations(x: XSpec, threads: int = 8, out: Optional[np.ndarray] = None) -> np.ndarray:
    """All of X (n x d, fp16). Chunks are generated on ``threads`` threads."""
    A = _mixing(x)
    ochan, dead = _channel_sets(x)
    if out is None:
        out = np.empty((x.n, x.d), dtype=np.float16)
    nchunks = (x.n + CHUNK - 1) // CHUNK

    def job(c):
        c0 = c * CHUNK
        c1 = min(c0 + CHUNK, x.n)
        out[c0:c1] = _chunk(x, A, ochan, dead, c, c0, c1)

    if threads <= 1 or nchunks == 1:
        for c in range(nchunks):
            job(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(job, range(nchunks)))
    return out
