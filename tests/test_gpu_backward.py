"""GPU parity of had_backward (the straight-through backward) through the C
ABI against the oracle's backward().

The GPU takes D_i = dout_i . out_i from had_attention's own output (float32);
everything else is recomputed.  Tolerance (the forward's reading of "1e-5
relative" for float32 outputs, elementwise against the natural magnitude):
|g - g*| <= 1e-5 * E, where E is the sum of the absolute values of the terms
that make up the element (the oracle's e_dq, e_dk, e_dv).  Every case prints
its parameters first.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_had_amd as had
from had_workloads import WORKLOADS, make_inputs
from parity_util import log, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()


def _check(got, want, mag, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    tol = TOL * mag + 1e-30
    bad = err > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r} tol {tol[i]!r}")
    return float((err / (mag + 1e-30)).max())


def _run(B, H, n, d, topn, causal, vdt, scale, seed, with_sigma=False, heads=None):
    inp = make_inputs(B, H, n, d, rank=8, noise="t3", seed=seed, v_dtype=vdt)
    q, k, v = to_dev(inp)
    qb, sq = had.pack(q)
    kb, sk = had.pack(k)
    out = had.attention(qb, kb, v, topn, scale, causal)
    dout_np = np.random.default_rng(seed + 1).standard_normal((B, H, n, d)).astype(np.float32)
    dout = torch.from_numpy(dout_np).cuda()
    kw = {"sigma_q": sq, "sigma_k": sk} if with_sigma else {}
    dq, dk, dv = had.backward(qb, kb, v, out, dout, topn, scale, causal, **kw)
    dq, dk, dv = (t.cpu().numpy() for t in (dq, dk, dv))
    sig_q = float(sq.item()) if with_sigma else 1.0
    sig_k = float(sk.item()) if with_sigma else 1.0
    worst = 0.0
    for bh in (range(B * H) if heads is None else heads):
        b, h = divmod(bh, H)
        r = oracle.backward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], dout_np[b, h], topn, scale,
                            causal, sigma_q=sig_q, sigma_k=sig_k)
        for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
            worst = max(worst, _check(g[b, h], r[name], r["e_" + name], f"slice {bh} {name}"))
    return worst


CASES = [
    # B, H, n, d, topn, causal, v dtype, scale
    (1, 1, 128, 64, 32, False, "f32", 0.125),
    (2, 2, 300, 64, 37, True, "bf16", 0.125),
    (1, 2, 200, 128, 50, True, "f32", 1 / np.sqrt(128)),
    (1, 1, 97, 5, 10, True, "f32", 0.9),        # ties everywhere
    (1, 1, 97, 5, 10, False, "bf16", 0.9),
    (1, 1, 70, 33, 70, False, "f32", 0.3),      # N = n: dense
    (1, 1, 50, 96, 80, True, "bf16", 0.2),      # N > visible
    (1, 1, 130, 64, 1, False, "f32", 0.125),    # N = 1
    (1, 1, 1, 64, 4, True, "f32", 0.125),       # one token
    (2, 1, 257, 32, 20, True, "bf16", 0.5),     # one word per row, ragged tail
    (1, 1, 33, 1, 5, False, "f32", 1.0),        # d = 1
    (1, 2, 160, 100, 30, False, "bf16", 2.0),   # sharp softmax, d not a multiple of 32
    # the bf16-product kernels at the other feature widths
    (1, 2, 150, 128, 20, False, "bf16", 0.09),  # d = 128
    (1, 1, 90, 33, 12, True, "bf16", 0.3),      # d = 33: padded features
    (1, 1, 40, 1, 7, True, "bf16", 1.0),        # d = 1
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_oracle(case):
    B, H, n, d, topn, causal, vdt, scale = case
    log(f"backward {case}")
    worst = _run(B, H, n, d, topn, causal, vdt, scale, seed=n * 5 + d + topn)
    log(f"  worst |err| / E {worst:.3e}")


def test_backward_with_sigma_and_is_deterministic():
    B, H, n, d, topn = 2, 2, 200, 64, 24
    log(f"backward sigma/determinism {(B, H, n, d, topn)}")
    _run(B, H, n, d, topn, True, "bf16", 0.125, seed=77, with_sigma=True)
    inp = make_inputs(B, H, n, d, rank=8, noise="t3", seed=78, v_dtype="bf16")
    q, k, v = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    out = had.attention(qb, kb, v, topn, 0.125, True)
    dout = torch.randn(B, H, n, d, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    g1 = [t.clone() for t in had.backward(qb, kb, v, out, dout, topn, 0.125, True)]
    g2 = had.backward(qb, kb, v, out, dout, topn, 0.125, True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


@pytest.mark.parametrize("name,heads", [("t5-base-n1024", (0, 50, 95)), ("causal-n16384", (13,))])
def test_backward_at_full_size(name, heads):
    """The long workloads' full shapes and launch, whole slices checked (every
    row of dq, every key of dk and dv)."""
    w = WORKLOADS[name]
    log(f"backward full size {name}: B={w.batch} H={w.heads} n={w.seq} d={w.dim} N={w.topn} "
        f"causal={w.causal} seed={w.seed}")
    worst = _run(w.batch, w.heads, w.seq, w.dim, w.topn, w.causal, w.v_dtype, w.scale, seed=w.seed,
                 heads=heads)
    log(f"  worst |err| / E {worst:.3e}")
