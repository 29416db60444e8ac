"""GPU parity of the Swish gradient over non-contiguous tensors (swish_grad_strided through
the C ABI, reached from swish_grad for any non-contiguous argument) against the float64
oracle evaluated on the same logical values.  Layouts: transposed, sliced with a step,
permuted 3-D and 5-D views, broadcast (zero-stride) inputs, a non-contiguous output whose
gaps must stay untouched, more than 8 dimensions (merged before launch), in-place on a
view, empty views, a view of more than 2^32 elements (the 64-bit index path), and a
seeded sweep of random layouts."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.ref as R
import swish_activation_backward_amd as swg
from gpu_util import device, note
from parity import compare, swish_abs_model
from workloads.gen import DTYPES, swish_inputs

pytestmark = pytest.mark.gpu


def _values(dt, shape, seed):
    """grad, x of the given shape (CPU, contiguous), from the seeded Swish generator."""
    n = int(np.prod(shape))
    inp = swish_inputs(dt, L=max(n, 1), seed=seed)
    return inp["grad"][:n].reshape(shape), inp["x"][:n].reshape(shape)


def _check(name, out, grad_view, x_view, dt, beta):
    """Compare the logical values of out with the oracle on the views' logical values."""
    g64 = grad_view.detach().cpu().contiguous().double().numpy()
    x64 = x_view.detach().cpu().contiguous().double().numpy()
    ref = R.swish_grad_ref(g64, x64, beta)
    compare(name, out.detach().cpu().contiguous(), ref, dt,
            model_abs=swish_abs_model(g64, x64, beta))


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("beta", [None, 1.702, -0.5])
def test_transposed_inputs(dt, beta):
    dev = device()
    G, X = _values(dt, (513, 1031), 21)
    g, x = G.to(dev).t(), X.to(dev).t()          # logical [1031, 513], strides (1, 1031)
    note(f"strided swish: transposed {dt} beta={beta}")
    out = swg.swish_grad(g, x, beta=beta)
    torch.cuda.synchronize()
    assert out.is_contiguous() and out.shape == (1031, 513)
    _check("transposed", out, g, x, dt, beta)


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_transposed_with_aligned_strides(dt):
    """Strides that are multiples of 4: the 4-element-vector tile kernel, with partial
    tiles on both edges."""
    dev = device()
    G, X = _values(dt, (1028, 516), 31)
    g, x = G.to(dev).t(), X.to(dev).t()          # [516, 1028], strides (1, 516)
    note(f"strided swish: transposed, aligned strides {dt}")
    out = swg.swish_grad(g, x, beta=1.702)
    torch.cuda.synchronize()
    _check("transposed aligned", out, g, x, dt, 1.702)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_transposed_partial_vectors(dt):
    """Rows and columns that are not multiples of 4 (vectors cut by the edge fall back to
    elements); the output's padding columns must stay untouched."""
    dev = device()
    G, X = _values(dt, (1026, 516), 32)
    g = G.to(dev)[:, :515].t()                   # [515, 1026], strides (1, 516)
    x = X.to(dev)[:, :515].t()
    base = torch.full((515, 1028), float("nan"), dtype=DTYPES[dt], device=dev)
    out = base[:, :1026]                         # strides (1028, 1)
    note(f"strided swish: partial vectors {dt}")
    swg.swish_grad(g, x, grad_x=out, beta=-0.5)
    torch.cuda.synchronize()
    assert torch.isnan(base[:, 1026:]).all(), "the kernel wrote past the view"
    _check("partial vectors", out, g, x, dt, -0.5)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_sliced_with_step_and_gapped_output(dt):
    """Inputs sliced with a step of 2; the output is every other column of a buffer whose
    other columns hold a sentinel that must survive."""
    dev = device()
    G, X = _values(dt, (300, 514), 22)
    g, x = G.to(dev)[:, ::2], X.to(dev)[:, 1::2]
    base = torch.full((300, 514), float("nan"), dtype=DTYPES[dt], device=dev)
    out = base[:, 1::2]
    note(f"strided swish: sliced, gapped output {dt}")
    swg.swish_grad(g, x, grad_x=out, beta=1.702)
    torch.cuda.synchronize()
    assert torch.isnan(base[:, ::2]).all(), "the kernel wrote into the output's gaps"
    _check("sliced", out, g, x, dt, 1.702)


@pytest.mark.parametrize("shape,perm", [((7, 33, 65), (2, 0, 1)),
                                        ((3, 4, 5, 6, 7), (4, 2, 0, 3, 1)),
                                        ((65537, 3), (1, 0)),
                                        ((2, 3, 5, 7, 11, 13), (5, 3, 1, 0, 2, 4))])
def test_permuted_views(shape, perm):
    """Permutations with odd sizes (every dimension's division is exercised)."""
    dev = device()
    G, X = _values("bf16", shape, 23)
    g = G.to(dev).permute(*perm)
    x = X.to(dev).permute(*perm)
    out = torch.empty(g.shape, dtype=torch.bfloat16, device=dev).permute(
        *[int(i) for i in np.argsort(perm)]).contiguous().permute(*perm)   # own buffer
    note(f"strided swish: permuted {shape} {perm}")
    swg.swish_grad(g, x, grad_x=out, beta=0.75)
    torch.cuda.synchronize()
    _check("permuted", out, g, x, "bf16", 0.75)


def test_broadcast_inputs():
    """x broadcast along rows (stride 0) and grad along columns."""
    dev = device()
    G, X = _values("fp32", (1, 1000), 24)
    _, Xc = _values("fp32", (777, 1), 25)
    g = G.to(dev).expand(777, 1000)
    x = Xc.to(dev).expand(777, 1000)
    note("strided swish: broadcast inputs")
    out = swg.swish_grad(g, x, beta=1.0)
    torch.cuda.synchronize()
    _check("broadcast", out, g, x, "fp32", 1.0)


def test_more_than_eight_dims():
    """Ten dimensions: contiguous ones merge into one (the contiguous kernel runs); with the
    last two transposed in grad only, three dimensions remain."""
    dev = device()
    shape = (2, 3, 2, 3, 2, 3, 2, 3, 4, 5)
    G, X = _values("bf16", shape, 26)
    g, x = G.to(dev), X.to(dev)
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    note("strided swish: 10-D contiguous through the strided entry point")
    swg.swish_grad_strided(g, x, out, beta=1.702)
    torch.cuda.synchronize()
    _check("10-D contiguous", out, g, x, "bf16", 1.702)
    gt = G.transpose(-1, -2).contiguous().to(dev).transpose(-1, -2)   # same values
    note("strided swish: 10-D with a transposed pair")
    out2 = swg.swish_grad(gt, x, beta=1.702)
    torch.cuda.synchronize()
    _check("10-D transposed pair", out2, gt, x, "bf16", 1.702)


def test_nine_unmergeable_dims_are_refused():
    dev = device()
    g = torch.zeros([2] * 9, dtype=torch.bfloat16, device=dev)
    x = torch.zeros([2] * 9, dtype=torch.bfloat16, device=dev).permute(*range(8, -1, -1))
    with pytest.raises(swg.SwgError, match="UNSUPPORTED"):
        swg.swish_grad(g, x)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_in_place_on_a_view(dt):
    dev = device()
    G, X = _values(dt, (129, 257), 27)
    gbase = G.to(dev)
    g = gbase.t()
    x = X.to(dev).t()
    want_in = g.detach().cpu().clone()
    note(f"strided swish: in place on a transposed view {dt}")
    swg.swish_grad(g, x, grad_x=g, beta=1.702)
    torch.cuda.synchronize()
    _check("in-place view", g, want_in, x, dt, 1.702)


def test_overlapping_output_is_refused():
    dev = device()
    buf = torch.zeros(64, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(8, 8, dtype=torch.bfloat16, device=dev)
    out = buf.as_strided((8, 8), (4, 1))          # rows overlap
    with pytest.raises(swg.SwgError, match="INVALID"):
        swg.swish_grad(g, g, grad_x=out)
    with pytest.raises(swg.SwgError, match="INVALID"):
        swg.swish_grad(g.t(), g, grad_x=g)       # aliases grad with other strides


def test_empty_views():
    dev = device()
    g = torch.zeros(0, 5, dtype=torch.bfloat16, device=dev).t()
    out = swg.swish_grad(g, g)
    torch.cuda.synchronize()
    assert out.shape == (5, 0)


def test_more_than_2_32_elements_2d():
    """A broadcast view of 65537 x 65537 > 2^32 elements into an 8.6 GB output (the 2-D
    tiled kernel, its tile loop past 2^20 tiles).  Sampled outputs (the first and last rows
    and columns included)."""
    dev = device()
    gs, _ = _values("bf16", (65537,), 28)
    _, xs = _values("bf16", (65537,), 29)
    n = 65537
    g = gs.to(dev).view(1, n).expand(n, n)
    x = xs.to(dev).view(n, 1).expand(n, n)
    out = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    note("strided swish: 65537 x 65537 broadcast (64-bit indices)")
    swg.swish_grad(g, x, grad_x=out, beta=1.702)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.concatenate([[0, 1, n - 1], rng.integers(0, n, 4000)])
    cols = np.concatenate([[0, n - 1, 1], rng.integers(0, n, 4000)])
    got = out[torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)].cpu()
    del out
    gsel = gs[torch.from_numpy(cols)]
    xsel = xs[torch.from_numpy(rows)]
    _check("2^32+ broadcast", got, gsel, xsel, "bf16", 1.702)


def test_more_than_2_32_elements_3d():
    """2 x 65537 x 32769 > 2^32 elements that stay three dimensions after merging: the
    gather kernel's 64-bit index path."""
    dev = device()
    R, C = 65537, 32769
    gs, _ = _values("bf16", (C,), 30)
    _, xs = _values("bf16", (R,), 31)
    g = gs.to(dev).view(1, 1, C).expand(2, R, C)
    x = xs.to(dev).view(1, R, 1).expand(2, R, C)
    out = torch.empty(2, R, C, dtype=torch.bfloat16, device=dev)
    note("strided swish: 2 x 65537 x 32769 broadcast (64-bit indices, 3-D)")
    swg.swish_grad(g, x, grad_x=out, beta=0.9)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    b = np.concatenate([[0, 1, 1], rng.integers(0, 2, 4000)])
    rows = np.concatenate([[0, R - 1, R - 1], rng.integers(0, R, 4000)])
    cols = np.concatenate([[0, C - 1, 0], rng.integers(0, C, 4000)])
    idx = [torch.from_numpy(v).to(dev) for v in (b, rows, cols)]
    got = out[idx[0], idx[1], idx[2]].cpu()
    del out
    _check("2^32+ broadcast 3-D", got, gs[torch.from_numpy(cols)], xs[torch.from_numpy(rows)],
           "bf16", 0.9)



def _random_view(base, rng, shape):
    """A view of ``base`` (1-D, contiguous, at least 8 x the view's elements) with logical
    ``shape``: a random permutation of a strided slice (steps 1..3, their product at most
    8) of a larger block."""
    nd = len(shape)
    steps = [1] * nd
    for i in rng.permutation(nd):
        st = int(rng.integers(1, 4))
        if int(np.prod(steps)) * st <= 8:
            steps[int(i)] = st
    perm = [int(p) for p in rng.permutation(nd)]
    # the block, in the permuted order, that the sliced view is cut from
    block = [shape[perm[i]] * steps[perm[i]] for i in range(nd)]
    t = base[:int(np.prod(block))].view(*block)
    t = t[tuple(slice(None, None, steps[perm[i]]) for i in range(nd))]
    inv = [perm.index(i) for i in range(nd)]
    v = t.permute(*inv)
    assert tuple(v.shape) == tuple(shape)
    return v


@pytest.mark.parametrize("seed", range(40))
def test_random_strided_views(seed):
    """Seeded random layouts: 1 to 7 dimensions, every tensor a random permutation of a
    random step slice, inputs sometimes broadcast along a dimension, the output a view of
    a larger buffer whose other elements must stay untouched; all three dtypes."""
    dev = device()
    rng = np.random.default_rng(7000 + seed)
    dt = ["bf16", "fp16", "fp32"][seed % 3]
    tdt = DTYPES[dt]
    nd = int(rng.integers(1, 8))
    shape = [int(rng.integers(1, 9 if nd > 4 else 40)) for _ in range(nd)]
    n = int(np.prod(shape))
    beta = [None, 1.702, 0.5, -1.3][seed % 4]
    G, X = _values(dt, (n * 8,), 300 + seed)
    grad = _random_view(G.to(dev), rng, shape)
    x = _random_view(X.to(dev), rng, shape)
    if nd > 1 and rng.random() < 0.3:        # a broadcast input along one dimension
        d = int(rng.integers(0, nd))
        idx = [slice(None)] * nd
        idx[d] = slice(0, 1)
        x = x[tuple(idx)].expand(*shape)
    sentinel = {torch.bfloat16: 0x7FA5, torch.float16: 0x7DA5, torch.float32: 0x7FA5A5A5}[tdt]
    ibits = torch.int32 if tdt == torch.float32 else torch.int16
    out_base = torch.empty(n * 8, dtype=tdt, device=dev)
    out_base.view(ibits).fill_(sentinel)
    out = _random_view(out_base, rng, shape)
    note(f"strided sweep {seed}: {dt} shape={shape} grad={grad.stride()} x={x.stride()} "
         f"out={out.stride()} beta={beta}")
    swg.swish_grad(grad, x, grad_x=out, beta=beta)
    torch.cuda.synchronize()
    _check("strided sweep", out, grad, x, dt, beta)
    # every element outside the output view is untouched
    touched = torch.zeros(n * 8, dtype=torch.int32, device=dev)
    offs = torch.zeros(shape, dtype=torch.int64, device=dev)
    for d_, (sz, st) in enumerate(zip(shape, out.stride())):
        ar = torch.arange(sz, device=dev, dtype=torch.int64) * st
        offs = offs + ar.view(*([1] * d_ + [sz] + [1] * (nd - d_ - 1)))
    base_off = out.storage_offset() - out_base.storage_offset()
    touched[(offs + base_off).reshape(-1)] = 1
    rest = out_base.view(ibits)[touched == 0]
    assert torch.all(rest == torch.tensor(sentinel, dtype=ibits, device=dev).view(ibits)), \
        "elements outside the output view were written"
