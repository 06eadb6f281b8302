"""Packed storage and the dequantizing product on the GPU against the oracle.

Inputs come from the oracle (its round-to-nearest codes, scales and zeros,
seeded fp16 activations) and go to both sides. Packing is integer work and
must be bit-exact. The product is compared output by output within the
rounding bound of its arithmetic. Two kernels compute it (K = floor(32 /
bits) codes per word, nw words per row, 64 lanes whose partial sums are
added in a tree of depth 6):
  * the general one forms W_hat in fp32 (one rounding) and sums x * W_hat,
    a lane over the K columns of each of at most ceil(nw / 64) words;
  * the 2/4/8-bit one sums the exact products x * q and x over runs of 4K
    columns inside one group and adds s * (sum x q - z sum x) per run, a lane
    over at most ceil(nw / 256) runs.
  * for two tokens or more with 4-bit codes, groups of whole 128-column
    chunks and cols % 128 == 0, an MFMA kernel sums the exact products x * q
    and x over each chunk (128 terms) and adds s * (sum x q - z sum x) per
    chunk to sums over at most ceil(cols / 512) chunks, four of which are
    added at the end.
The first two are within

    |y_gpu - y| <= F * 2^-24 * sum_c |x_c| (|q_c| + |z_c|) s_c,
    F = max(ceil(nw / 64) K, 4K + ceil(nw / 256)) + 8,

which bounds either sum since |q - z| <= |q| + |z|; the MFMA kernel within
the same form with F = 128 + ceil(cols / 512) + 8 (each MFMA's sum no less
accurate than sequential fp32 additions).
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import post_weight_quantization_02_amd as gq
    return torch, gq


def _cuda(env, a, dtype=None):
    torch, _ = env
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).cuda()


def _layer(rows, cols, bits, g, seed):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((rows, cols)) * 0.02
    r = oracle.rtn(W, bits, g)
    return r["codes"], r["scales"], r["zeros"]


def _mfma_path(m, cols, bits, g, g_idx):
    gg = cols if g <= 0 else g
    return bits == 4 and m >= 2 and g_idx is None and cols % 128 == 0 and \
        (gg % 128 == 0 or gg >= cols)


def _bound(x, codes, scales, zeros, cols, bits, g, g_idx=None):
    k = 32 // bits
    nw = -(-cols // k)
    f = max(-(-nw // 64) * k, 4 * k + -(-nw // 256)) + 8
    if _mfma_path(np.asarray(x).shape[0], cols, bits, g, g_idx):
        f = 128 + -(-cols // 512) + 8
    if g_idx is None:
        gi = np.arange(cols) // (cols if g <= 0 else g)
    else:
        gi = np.asarray(g_idx, np.int64)
    mag = (np.abs(codes) + np.abs(zeros[:, gi])) * np.abs(scales[:, gi])
    return f * 2.0 ** -24 * (np.abs(np.asarray(x, np.float64)) @ mag.T)


@pytest.mark.parametrize("bits,rows,cols", [(4, 37, 300), (3, 5, 1001), (2, 8, 17), (8, 3, 4096),
                                            (5, 2, 77), (4, 1, 5)])
def test_pack_bit_exact(env, bits, rows, cols):
    torch, gq = env
    rng = np.random.default_rng(bits * 1000 + cols)
    codes = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)  # high bits must be masked
    p = gq.pack_codes(_cuda(env, codes), bits)
    torch.cuda.synchronize()
    ref = oracle.pack_codes(codes & ((1 << bits) - 1), bits)
    assert np.array_equal(p.cpu().numpy().view(np.uint32), ref)
    assert p.shape[1] == gq.packed_words(cols, bits) == ref.shape[1]


def _gemm_case(env, rows, cols, bits, g, m, seed, act_order=False):
    torch, gq = env
    codes, scales, zeros = _layer(rows, cols, bits, g, seed)
    g_idx = None
    if act_order:
        perm = np.random.default_rng(seed + 1).permutation(cols)
        g_idx = np.empty(cols, np.int64)
        g_idx[perm] = np.arange(cols) // g
    rng = np.random.default_rng(seed + 2)
    x = rng.standard_normal((m, cols)).astype(np.float16)
    packed = gq.pack_codes(_cuda(env, codes.astype(np.uint8)), bits)
    y = gq.dequant_gemm(_cuda(env, x), packed, bits, cols, _cuda(env, scales, np.float32),
                        _cuda(env, zeros, np.float32), g,
                        None if g_idx is None else _cuda(env, g_idx, np.int32))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    s32 = scales.astype(np.float32).astype(np.float64)
    z32 = zeros.astype(np.float32).astype(np.float64)
    ref = oracle.dequant_matmul(x, oracle.pack_codes(codes, bits), bits, cols, s32, z32, g, g_idx)
    err = np.abs(y - ref)
    bound = _bound(x, codes, s32, z32, cols, bits, g, g_idx)
    assert np.all(err <= bound), (err.max(), bound[err > bound][:5])
    return float((err / np.maximum(bound, 1e-300)).max())


@pytest.mark.parametrize("rows,cols,bits,g,m", [
    (64, 256, 4, 128, 1),
    (37, 300, 4, 128, 3),      # ragged rows, ragged last word and group, one pass of 3 tokens
    (50, 1000, 3, 128, 5),     # 10 codes per word, words straddle groups; two passes
    (16, 512, 2, 32, 2),
    (9, 640, 8, 64, 4),
    (7, 200, 4, 200, 9),       # per-channel, three passes
    (1, 5, 4, 128, 1),         # a single row, one partial word
])
def test_dequant_gemm_matches_oracle(env, rows, cols, bits, g, m):
    _gemm_case(env, rows, cols, bits, g, m, seed=rows * 7 + cols)


@pytest.mark.parametrize("rows,cols,g,m", [
    (64, 256, 128, 2),         # two tokens: the MFMA path
    (37, 384, 128, 5),         # ragged rows, three chunks over four waves
    (50, 1024, 256, 17),       # two token tiles, groups of two chunks
    (16, 512, 512, 3),         # one group per row
    (9, 128, 128, 16),         # one chunk: three waves with nothing to do
    (40, 640, 128, 40),        # two passes (32 + 8 tokens)
])
def test_dequant_gemm_mfma_path(env, rows, cols, g, m):
    """Several tokens at 4 bits: the MFMA kernel, every output within the
    bound of its arithmetic."""
    assert _mfma_path(m, cols, 4, g, None)
    _gemm_case(env, rows, cols, 4, g, m, seed=rows * 5 + cols + m)


@pytest.mark.parametrize("bits", [3, 4])
def test_dequant_gemm_with_g_idx(env, bits):
    """Act-order groups: the group of each column comes from g_idx."""
    _gemm_case(env, 40, 768, bits, 128, 2, seed=5, act_order=True)


@pytest.mark.parametrize("rows,cols,m", [(4096, 4096, 1), (4096, 4096, 4), (11008, 4096, 1),
                                         (4096, 11008, 2), (4096, 4096, 16), (11008, 4096, 32),
                                         (4096, 11008, 16)])
def test_dequant_gemm_full_layer_shapes(env, rows, cols, m):
    """The Llama-7B-shaped projections of the decode benchmark, int4 g128,
    every output compared."""
    _gemm_case(env, rows, cols, 4, 128, m, seed=rows + cols + m)


def test_dequant_gemm_zero_tokens_is_a_no_op(env):
    torch, gq = env
    codes, scales, zeros = _layer(8, 128, 4, 128, 1)
    packed = gq.pack_codes(_cuda(env, codes.astype(np.uint8)), 4)
    y = gq.dequant_gemm(torch.empty((0, 128), dtype=torch.float16, device="cuda"), packed, 4, 128,
                        _cuda(env, scales, np.float32), _cuda(env, zeros, np.float32), 128)
    torch.cuda.synchronize()
    assert y.shape == (0, 8)


def test_quantize_pack_product_end_to_end(env):
    """The GPU's own quantizer output, packed and multiplied on the GPU,
    equals the dense product with the GPU's dequantized weights (a property
    of the GPU outputs, no oracle input from them)."""
    torch, gq = env
    import synth
    from parity import dequant
    L = synth.LAYERS["tiny"]
    X = synth.activations(L.x)
    W = synth.weights(L.w)
    H = torch.zeros((L.x.d, L.x.d), dtype=torch.float32, device="cuda")
    gq.hessian_accumulate(H, _cuda(env, X), 2.0)
    U = gq.prepare_hinv(H, 0.01)
    codes, scales, zeros, _ = gq.quantize_layer(_cuda(env, W), U, 4, 128, 128)
    x = _cuda(env, X[:3])
    y = gq.dequant_gemm(x, gq.pack_codes(codes, 4), 4, L.x.d, scales, zeros, 128)
    torch.cuda.synchronize()
    c, sc, zr = codes.cpu().numpy(), scales.cpu().numpy(), zeros.cpu().numpy()
    Wq = dequant(c, sc, zr, 128)
    xd = X[:3].astype(np.float64)
    ref = xd @ Wq.T
    bound = _bound(xd, c.astype(np.float64), sc.astype(np.float64), zr.astype(np.float64),
                   L.x.d, 4, 128)
    assert np.all(np.abs(y.cpu().numpy() - ref) <= bound)


def test_dequant_gemm_graph_replay(env):
    """The decode products captured in a HIP graph: every replay, with eager
    work changing x in between, equals the eager result bit for bit."""
    torch, gq = env
    mats = []
    for rows, cols, seed in ((96, 512, 1), (40, 1024, 2)):
        codes, scales, zeros = _layer(rows, cols, 4, 128, seed)
        mats.append((cols, gq.pack_codes(_cuda(env, codes.astype(np.uint8)), 4),
                     _cuda(env, scales, np.float32), _cuda(env, zeros, np.float32),
                     torch.empty((2, rows), dtype=torch.float32, device="cuda")))
    xs = {c: torch.zeros((2, c), dtype=torch.float16, device="cuda") for c in (512, 1024)}

    def step():
        for cols, p, sc, zr, y in mats:
            gq.dequant_gemm(xs[cols], p, 4, cols, sc, zr, 128, out=y)

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    for rep in range(4):
        for c, xt in xs.items():  # eager work between replays
            xt.copy_(torch.from_numpy(rng.standard_normal((2, c)).astype(np.float16)).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [m[4].clone() for m in mats]
        step()
        torch.cuda.synchronize()
        for a, m in zip(got, mats):
            assert torch.equal(a, m[4]), rep
