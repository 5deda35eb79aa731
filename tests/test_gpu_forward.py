"""GPU: had_forward (pack of Q and K in one launch, attention with the sigma
finalize folded in) against the separate calls and against the oracle.

had_forward must reproduce had_pack(q), had_pack(k), had_attention(...) bit
for bit (bits, sigma, out); one case is also checked against the oracle
directly.  Every case prints its name, shape and seed first.
"""

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


CASES = [
    # B, H, n, d, topn, causal, v dtype, seed
    (1, 1, 128, 64, 32, False, "f32", 11),
    (2, 3, 300, 64, 40, True, "bf16", 12),
    (1, 2, 77, 40, 9, False, "bf16", 13),
    (2, 2, 250, 128, 64, True, "bf16", 14),
    (1, 1, 33, 256, 5, False, "f32", 15),
    (4, 4, 1024, 64, 256, False, "bf16", 16),
]


@pytest.mark.parametrize("case", CASES)
def test_forward_equals_separate_calls(case):
    B, H, n, d, topn, causal, vdt, seed = case
    log(f"forward vs separate {case}")
    inp = make_inputs(B, H, n, d, rank=4, noise="t3", seed=seed, v_dtype=vdt)
    q, k, v = to_dev(inp)
    scale = 1.0 / np.sqrt(d)
    qb, sq = had.pack(q)
    kb, sk = had.pack(k)
    ref = had.attention(qb, kb, v, topn, scale, causal)
    out, fqb, fkb, fsq, fsk = had.forward(q, k, v, topn, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(fqb, qb) and torch.equal(fkb, kb)
    assert torch.equal(fsq, sq) and torch.equal(fsk, sk)
    assert torch.equal(out, ref)


def test_forward_against_oracle_and_without_sigma():
    B, H, n, d, topn = 2, 2, 200, 64, 24
    log(f"forward oracle {(B, H, n, d, topn)}")
    inp = make_inputs(B, H, n, d, rank=8, noise="t3", seed=21, v_dtype="bf16")
    q, k, v = to_dev(inp)
    scale = 1.0 / np.sqrt(d)
    out, qb, kb, sq, sk = had.forward(q, k, v, topn, scale, True)
    out2, _, _, none_q, none_k = had.forward(q, k, v, topn, scale, True, with_sigma=False)
    torch.cuda.synchronize()
    assert none_q is None and none_k is None
    assert torch.equal(out, out2)
    assert np.array_equal(bits_np(qb), oracle.pack_bits(oracle.binarize(inp["q"])))
    assert np.array_equal(bits_np(kb), oracle.pack_bits(oracle.binarize(inp["k"])))
    assert abs(float(sq.item()) - oracle.sigma(inp["q"])) <= 1e-6 * oracle.sigma(inp["q"])
    assert abs(float(sk.item()) - oracle.sigma(inp["k"])) <= 1e-6 * oracle.sigma(inp["k"])
    got = out.cpu().numpy()
    for b in range(B):
        for h in range(H):
            r = oracle_head(inp, b, h, topn, scale, True)
            check_out(got[b, h], r["out"], r["E"], inp["v"], "bf16", where=f"b{b}h{h}")


def test_forward_unaligned_q_and_nan_flag():
    """Q at a 4- but not 16-byte aligned address packs on the scalar path in its
    own launch; K keeps the vector path.  A NaN in K sets the status bit."""
    B, H, n, d, topn = 1, 2, 96, 64, 16
    log(f"forward unaligned {(B, H, n, d, topn)}")
    inp = make_inputs(B, H, n, d, rank=4, noise="normal", seed=31, v_dtype="bf16")
    q, k, v = to_dev(inp)
    buf = torch.zeros(q.numel() + 1, dtype=torch.float32, device="cuda")
    buf[1:] = q.reshape(-1)
    qu = buf[1:].view(q.shape)
    assert qu.data_ptr() % 16 != 0
    scale = 0.2
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, qb, kb, sq, sk = had.forward(qu, k, v, topn, scale, False, dev_status=st)
    qb2, sq2 = had.pack(qu)
    ref = had.attention(qb2, kb, v, topn, scale, False)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(qb, qb2) and torch.equal(sq, sq2) and torch.equal(out, ref)
    k2 = k.clone()
    k2[0, 1, 5, 7] = float("nan")
    had.forward(q, k2, v, topn, scale, False, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & had.DEV_NAN_INPUT
