"""GPU: had_forward_noalloc (the forward call for callers that cannot
allocate: sigma partials in the library's own device array) through the C
ABI, against had_forward with a caller workspace: bits, sigma and out equal
bit for bit, on calls in a row whose second input is smaller (the array keeps
the first call's contents), with and without sigma; sigma also against the
oracle.  Every case prints its shape and seed first."""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_had_amd as had
from had_workloads import make_inputs
from parity_util import bits_np, check_out, log, oracle_head, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()


CALLS = [
    # B, H, n, d, topn, causal, v dtype, seed (the second is smaller than the first)
    (8, 12, 1024, 64, 256, False, "bf16", 41),
    (1, 2, 300, 128, 40, True, "f32", 42),
    (2, 1, 77, 40, 9, False, "bf16", 43),
]


def test_noalloc_equals_forward_on_calls_in_a_row():
    for case in CALLS:
        B, H, n, d, topn, causal, vdt, seed = case
        log(f"forward_noalloc {case}")
        inp = make_inputs(B, H, n, d, rank=4, noise="t3", seed=seed, v_dtype=vdt)
        q, k, v = to_dev(inp)
        scale = 1.0 / np.sqrt(d)
        ref = had.forward(q, k, v, topn, scale, causal)
        got = had.forward_noalloc(q, k, v, topn, scale, causal)
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("out", "qbits", "kbits", "sigma_q", "sigma_k")):
            assert torch.equal(a, b), f"{case}: {name} differs from had_forward"
        sq = oracle.sigma(inp["q"])
        assert abs(float(got[3].item()) - sq) <= 1e-6 * sq
        assert np.array_equal(bits_np(got[1]), oracle.pack_bits(oracle.binarize(inp["q"])))
        r = oracle_head(inp, B - 1, H - 1, topn, scale, causal, rows=np.arange(min(n, 40)))
        check_out(got[0].cpu().numpy()[B - 1, H - 1][r["rows"]], r["out"], r["E"], inp["v"], vdt,
                  where=f"{case} last slice")


def test_noalloc_without_sigma_and_with_status():
    B, H, n, d, topn = 1, 2, 96, 64, 16
    log(f"forward_noalloc no sigma {(B, H, n, d, topn)}")
    inp = make_inputs(B, H, n, d, rank=4, noise="normal", seed=44, v_dtype="bf16")
    q, k, v = to_dev(inp)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, qb, kb, none_q, none_k = had.forward_noalloc(q, k, v, topn, 0.2, False, with_sigma=False,
                                                      dev_status=st)
    ref = had.forward(q, k, v, topn, 0.2, False, with_sigma=False)
    torch.cuda.synchronize()
    assert none_q is None and none_k is None and int(st.item()) == 0
    assert torch.equal(out, ref[0]) and torch.equal(qb, ref[1]) and torch.equal(kb, ref[2])
