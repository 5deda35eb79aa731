"""GPU: a seeded sweep of random small shapes through every compute call of
the C ABI (had_forward, had_attention, had_select, had_logits, had_pack,
had_decode, had_decode_forward, had_topn_mass), each compared with the
oracle: packed bits, logits and kept indices bit-exact, sigma within 1e-6
relative, outputs within the fp32 / bf16 tolerances, top-N mass exact up to
decisions within rounding; had_decode_forward equal to had_pack + had_decode
bit for bit.  The shapes mix feature counts around the 32-bit word
boundaries (1 ... 256), sequence lengths around the 16-key chunk and 128-row
tile boundaries, N from 1 to beyond n, both masks, both V types, sharp and
flat softmax scales and both noise families.  Every case prints its
parameters first.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_had_amd as had
from had_workloads import make_inputs
from parity_util import bits_np, check_out, check_topn_mass, log

pytestmark = pytest.mark.gpu

DIMS = [1, 2, 5, 8, 16, 31, 32, 33, 40, 63, 64, 65, 96, 100, 127, 128, 160, 200, 255, 256]
SEQS = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256, 257, 300, 511, 700]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()


def _cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        d = int(rng.choice(DIMS))
        n = int(rng.choice(SEQS))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        topn = int(rng.choice([1, 2, 3, max(1, n // 4), max(1, n // 2), n, n + 5]))
        causal = bool(rng.integers(0, 2))
        vdt = "f32" if rng.random() < 0.3 else "bf16"
        scale = float(rng.choice([0.01, 0.1, 1 / np.sqrt(d), 0.5, 2.0]))
        noise = str(rng.choice(["normal", "t3"]))
        nq = int(min(n, rng.integers(1, 5)))
        seed = int(rng.integers(0, 1 << 30))
        mass = float(rng.choice([0.5, 0.9, 0.99]))
        out.append((B, H, n, d, topn, causal, vdt, scale, noise, nq, seed, mass))
    return out


@pytest.mark.parametrize("block", range(6))
def test_random_shapes_against_the_oracle(block):
    for case in _cases(7000 + block, 50):
        B, H, n, d, topn, causal, vdt, scale, noise, nq, seed, mass = case
        log(f"random {case}")
        inp = make_inputs(B, H, n, d, rank=min(4, d), noise=noise, seed=seed, v_dtype=vdt)
        q = torch.from_numpy(inp["q"]).cuda()
        k = torch.from_numpy(inp["k"]).cuda()
        v = torch.from_numpy(inp["v"])
        v = (v.to(torch.bfloat16) if vdt == "bf16" else v).cuda()
        out, qb, kb, sq, _ = had.forward(q, k, v, topn, scale, causal)
        idx = had.select(qb, kb, d, topn, causal).cpu().numpy()
        out2 = had.attention(qb, kb, v, topn, scale, causal)
        p0 = n - nq
        qn = np.ascontiguousarray(inp["q"][:, :, p0:])
        qnb, _ = had.pack(torch.from_numpy(qn).cuda(), with_sigma=False)
        odt = had.decode(qnb, kb, v, topn, scale, q_pos0=p0, causal=causal)
        odf = had.decode_forward(torch.from_numpy(qn).cuda(), kb, v, topn, scale, q_pos0=p0, causal=causal)
        lg = had.logits(qb, kb, d).cpu().numpy()
        nm = had.topn_mass(qb, kb, d, scale, mass, causal).cpu().numpy()
        torch.cuda.synchronize()
        assert torch.equal(out, out2), f"{case}: had_forward and had_attention differ"
        assert torch.equal(odt, odf), f"{case}: had_decode_forward and had_pack + had_decode differ"
        od = odt.cpu().numpy()
        assert np.array_equal(bits_np(qb), oracle.pack_bits(oracle.binarize(inp["q"]))), f"{case}: bits"
        ref_sigma = oracle.sigma(inp["q"])
        assert abs(float(sq.item()) - ref_sigma) <= 1e-6 * ref_sigma, f"{case}: sigma"
        o = out.cpu().numpy()
        for b in range(B):
            for h in range(H):
                r = oracle.forward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], topn, scale,
                                   causal=causal)
                assert np.array_equal(idx[b * H + h].astype(np.int64), r["idx"]), f"{case}: select {(b, h)}"
                S = oracle.logits(oracle.binarize(inp["q"][b, h]), oracle.binarize(inp["k"][b, h]))
                assert np.array_equal(lg[b * H + h].astype(np.int64), S.astype(np.int64)), f"{case}: logits {(b, h)}"
                check_topn_mass(nm[b * H + h], S, float(np.float32(scale)), mass, causal, where=f"{case} {(b, h)}")
                check_out(o[b, h], r["out"], r["E"], inp["v"], vdt, where=f"{case} slice {(b, h)}")
                rd = oracle.decode(qn[b, h], inp["k"][b, h], inp["v"][b, h], topn, scale,
                                   q_pos0=p0, causal=causal)
                check_out(od[b, h], rd["out"], rd["E"], inp["v"], vdt, where=f"{case} decode {(b, h)}")
