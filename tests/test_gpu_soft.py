"""GPU parity of had_soft_forward / had_soft_select (the scaled-tanh soft
forward) through the C ABI against the oracle's soft_forward().

The GPU forms tanh in float32 and the logits on the fp32 matrix cores, so its
logit s~_ij differs from the oracle's float64 S_ij by at most delta_i =
2 * (12 + d) * 2^-24 * B_i, with B_i the largest sum over features of
|Bq_ic| |Bk_jc| in the row: each float32 soft sign is within 6 * 2^-24 of
its value relatively (the argument x * (1 / (sigma c)) rounded twice, which
tanh's slope z sech^2 z <= tanh z does not amplify, and the function within
2 ulp), and the fp32 accumulation of d products adds at most d * 2^-24 * B_i;
doubled for safety.  Where floating point decides
the kept set, the test compares what is unique and checks the rest is valid:
with thr the oracle's N_i-th largest logit of the row, every key with S >
thr + 2 delta must be kept, every key with S < thr - 2 delta dropped, and the
row keeps exactly N_i keys.  Outputs: a row whose window holds just the keys
still needed has one valid kept set, the oracle's; otherwise every valid
choice is evaluated by the oracle and the GPU row must match one of them.
Output tolerance: (4 * scale * delta_i + 2e-5) * E (the logit error moves each
weight by at most 2 * scale * delta relatively, Z likewise; 2e-5 covers the
float32 weights and sums over up to 1024 keys).  With c so small that every
|x| / (sigma c) exceeds 20, both sides have exactly +-1 soft signs and integer
logits: there the kept sets must equal the oracle's (and the sign path's) bit
for bit, ties by lower index.  Every case prints its parameters first.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_had_amd as had
from had_workloads import make_inputs
from parity_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()


def _dev(inp):
    q = torch.from_numpy(inp["q"]).cuda()
    k = torch.from_numpy(inp["k"]).cuda()
    v = torch.from_numpy(inp["v"])
    v = (v.to(torch.bfloat16) if inp["v_dtype"] == "bf16" else v).cuda()
    return q, k, v


def _sigmas(inp):
    """The oracle's sigma of each tensor, rounded to float32: both sides use it."""
    sq = np.float32(oracle.sigma(inp["q"]))
    sk = np.float32(oracle.sigma(inp["k"]))
    return sq, sk, torch.tensor([sq], device="cuda"), torch.tensor([sk], device="cuda")


def _check_slice(r, bq, bk, v, keep, out, topn, scale, causal, d, where):
    """Kept-set validity and outputs of one slice; returns (rows, ambiguous rows)."""
    S = r["S"]
    n = S.shape[1]
    B = np.abs(bq[r["rows"]]) @ np.abs(bk).T
    amb = 0
    for ri, i in enumerate(r["rows"]):
        nv = oracle.visible_count(int(i), n, causal)
        Ni = min(topn, nv)
        Sv = S[ri, :nv]
        thr = Sv[np.argsort(-Sv, kind="stable")[Ni - 1]]
        delta = 2.0 * (12 + d) * 2.0 ** -24 * float(B[ri, :nv].max())
        must_keep = Sv > thr + 2 * delta
        must_drop = Sv < thr - 2 * delta
        window = np.nonzero(~must_keep & ~must_drop)[0]
        if keep is not None:
            gk = keep[ri].astype(bool)
            assert not gk[nv:].any(), f"{where} row {i}: a key past the visible range is kept"
            gk = gk[:nv]
            assert int(gk.sum()) == Ni, f"{where} row {i}: {int(gk.sum())} kept, want {Ni}"
            assert gk[must_keep].all(), f"{where} row {i}: a key clear of the threshold is dropped"
            assert not gk[must_drop].any(), f"{where} row {i}: a key clear below the threshold is kept"
        if out is None:
            continue
        need = Ni - int(must_keep.sum())
        base = np.nonzero(must_keep)[0]
        if need == len(window):
            alts = [np.sort(np.concatenate([base, window]))]
        else:
            amb += 1
            combos = list(itertools.islice(itertools.combinations(window, need), 64))
            assert len(combos) < 64, f"{where} row {i}: window of {len(window)} keys for {need} places"
            alts = [np.sort(np.concatenate([base, np.array(cmb, dtype=np.int64)])) for cmb in combos]
        tol_rel = 4.0 * scale * delta + 2e-5
        ok = False
        worst = np.inf
        for idx in alts:
            o, E = oracle.sparse_softmax_av(S[ri:ri + 1], idx[None, :], v, scale)
            err = np.abs(out[ri].astype(np.float64) - o[0])
            excess = float(np.max(err - (tol_rel * E[0] + 1e-30)))
            worst = min(worst, excess)
            if excess <= 0:
                ok = True
                break
        assert ok, f"{where} row {i}: output outside tolerance by {worst:.3e} for every valid kept set"
    return len(r["rows"]), amb


def _run(shape, topn, c, causal, v_dtype, seed, scale=None, slices=None, rows=None, mask=True,
         rank=8, noise="t3"):
    B, H, n, d = shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    log(f"soft forward {shape} topn={topn} c={c} causal={causal} v={v_dtype} seed={seed}")
    inp = make_inputs(B, H, n, d, v_dtype=v_dtype, rank=rank, noise=noise, seed=seed)
    q, k, v = _dev(inp)
    sq, sk, tsq, tsk = _sigmas(inp)
    out = had.soft_forward(q, k, v, topn, scale, c, causal, sigma_q=tsq, sigma_k=tsk)
    out2 = had.soft_forward(q, k, v, topn, scale, c, causal, sigma_q=tsq, sigma_k=tsk)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "two calls differ"
    out = out.cpu().numpy()
    slices = range(B * H) if slices is None else slices
    keep = had.soft_select(q, k, topn, c, causal, sigma_q=tsq, sigma_k=tsk).cpu().numpy() if mask else None
    total = amb = 0
    for bh in slices:
        b, h = divmod(bh, H)
        r = oracle.soft_forward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], topn, scale, c, causal,
                                sigma_q=float(sq), sigma_k=float(sk), rows=rows)
        bq = oracle.soft_binarize(inp["q"][b, h], float(sq), c)
        bk = oracle.soft_binarize(inp["k"][b, h], float(sk), c)
        kr = keep[bh][r["rows"]] if keep is not None else None
        t, a = _check_slice(r, bq, bk, inp["v"][b, h], kr, out[b, h][r["rows"]], topn, scale, causal, d,
                            where=f"{shape} slice {bh}")
        total += t
        amb += a
    log(f"  rows {total}, rows with several valid kept sets {amb}")
    return total, amb


CASES = [
    ((1, 2, 77, 64), 9, 0.7, False, "f32", 1),
    ((1, 2, 77, 64), 9, 0.7, True, "f32", 2),
    ((2, 3, 200, 40), 50, 0.3, True, "bf16", 3),
    ((1, 2, 130, 128), 33, 1.0, False, "f32", 4),
    ((1, 1, 97, 100), 20, 2.0, False, "bf16", 5),
    ((1, 3, 64, 5), 7, 0.5, False, "f32", 6),
    ((1, 2, 45, 1), 4, 0.5, True, "f32", 7),
    ((1, 1, 300, 32), 1, 0.4, False, "f32", 8),
    ((1, 1, 150, 64), 150, 0.4, False, "f32", 9),
    ((1, 1, 150, 64), 400, 0.4, True, "f32", 10),
    ((1, 1, 1, 64), 3, 0.4, False, "f32", 11),
    ((1, 2, 1024, 64), 256, 0.5, False, "f32", 12),
    ((1, 1, 1024, 128), 200, 0.8, True, "bf16", 13),
    ((1, 2, 333, 64), 40, 30.0, False, "f32", 14),
    ((1, 2, 77, 64), 9, 0.7, True, "bf16", 15),
    ((1, 1, 100, 32), 12, 0.6, False, "bf16", 16),
    ((2, 1, 150, 48), 30, 0.9, True, "bf16", 17),
    ((1, 1, 600, 128), 70, 0.5, True, "f32", 18),
    # 8-wave work-groups with bf16 V: d = 64 takes the asynchronous V copies (causal and
    # ragged: tiles past the diagonal are skipped), d = 48 clamps the copies' features past d,
    # d = 32 stages V through registers
    ((1, 2, 700, 64), 90, 0.6, True, "bf16", 19),
    ((1, 1, 520, 48), 64, 0.5, False, "bf16", 20),
    ((1, 1, 400, 32), 50, 0.7, True, "bf16", 21),
]


@pytest.mark.parametrize("shape,topn,c,causal,v_dtype,seed", CASES)
def test_soft_forward_matches_oracle(shape, topn, c, causal, v_dtype, seed):
    total, amb = _run(shape, topn, c, causal, v_dtype, seed)
    assert amb <= max(2, total // 5)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,n,topn", [(64, 200, 17), (24, 130, 30), (128, 64, 8)])
def test_soft_forward_small_c_is_the_sign_path_exactly(d, n, topn, causal):
    """Every |x| >= 0.05 sigma and c = 1e-3: |x / (sigma c)| >= 50, so both the
    float32 tanh and the float64 one are exactly +-1, the logits are the
    integers of the sign path, and the kept sets must match the oracle's bit
    for bit (lower index first among the many equal logits)."""
    log(f"soft forward sign limit d={d} n={n} topn={topn} causal={causal}")
    inp = make_inputs(1, 2, n, d, v_dtype="f32", rank=4, noise="t3", seed=40 + d + n)
    for name in ("q", "k"):
        x = inp[name]
        floor = 0.06 * oracle.sigma(x) + 0.06 * 3 * np.abs(x).max()
        inp[name] = np.where(x >= 0, x + floor, x - floor).astype(np.float32)
    q, k, v = _dev(inp)
    sq, sk, tsq, tsk = _sigmas(inp)
    assert np.abs(inp["q"]).min() >= 0.05 * sq and np.abs(inp["k"]).min() >= 0.05 * sk
    scale = 0.3
    out = had.soft_forward(q, k, v, topn, scale, 1e-3, causal, sigma_q=tsq, sigma_k=tsk).cpu().numpy()
    keep = had.soft_select(q, k, topn, 1e-3, causal, sigma_q=tsq, sigma_k=tsk).cpu().numpy()
    for h in range(2):
        r = oracle.soft_forward(inp["q"][0, h], inp["k"][0, h], inp["v"][0, h], topn, scale, 1e-3, causal,
                                sigma_q=float(sq), sigma_k=float(sk))
        hard = oracle.forward(inp["q"][0, h], inp["k"][0, h], inp["v"][0, h], topn, scale, causal)
        assert np.array_equal(r["idx"], hard["idx"])
        want = np.zeros((n, n), dtype=np.uint8)
        for i in range(n):
            kept = r["idx"][i][r["idx"][i] >= 0]
            want[i, kept] = 1
        assert np.array_equal(keep[h], want), f"slice {h}: kept sets differ"
        err = np.abs(out[0, h] - r["out"])
        assert np.all(err <= 2e-5 * r["E"] + 1e-30), f"slice {h}: output error {err.max():.3e}"


def test_soft_forward_full_t5_shape_sampled_slices():
    """The t5-base-n1024 shape (8 x 12 heads, n = 1024, d = 64, N = 256) in one
    launch; every row of two slices checked, kept sets of both."""
    total, amb = _run((8, 12, 1024, 64), 256, 0.5, False, "bf16", 21, scale=0.125, slices=[0, 95],
                      rank=16, noise="normal")
    assert amb <= total // 5


def test_soft_forward_sigma_is_applied():
    """The same inputs with sigma given as 2 * sigma and c halved give the
    same soft rows (x / (2 sigma * c / 2)), hence the same output bit for bit;
    sigma = NULL means 1."""
    log("soft forward sigma scaling")
    inp = make_inputs(1, 2, 100, 64, v_dtype="f32", rank=4, noise="t3", seed=3)
    q, k, v = _dev(inp)
    one = torch.ones(1, device="cuda")
    a = had.soft_forward(q, k, v, 11, 0.2, 0.5, False, sigma_q=one, sigma_k=one)
    b = had.soft_forward(q, k, v, 11, 0.2, 0.5, False)
    assert torch.equal(a, b)
    two = torch.full((1,), 2.0, device="cuda")
    c2 = had.soft_forward(q, k, v, 11, 0.2, 0.25, False, sigma_q=two, sigma_k=two)
    assert torch.equal(a, c2)


def test_soft_select_slice_range_equals_the_full_export():
    """had_soft_select on slices [1, 3) of 4 gives those slices of the full export."""
    log("soft select slice range")
    inp = make_inputs(2, 2, 300, 64, v_dtype="f32", rank=4, noise="t3", seed=9)
    q, k, _ = _dev(inp)
    _, _, tsq, tsk = _sigmas(inp)
    full = had.soft_select(q, k, 40, 0.5, True, sigma_q=tsq, sigma_k=tsk)
    part = had.soft_select(q, k, 40, 0.5, True, sigma_q=tsq, sigma_k=tsk, bh_begin=1, bh_count=2)
    assert torch.equal(part, full[1:3])
    assert int(full.sum()) == sum(min(40, i + 1) for i in range(300)) * 4


def test_soft_forward_with_sigma_zero_is_finite():
    """A sigma of 0 (the sigma had_pack reports for a constant tensor) takes
    1 / (sigma c) as FLT_MAX: the soft signs are the signs, 0 for an element
    equal to 0, so with every query element 0 all logits are 0 and each row is
    the mean of its N_i lowest-index visible V rows."""
    log("soft forward sigma 0")
    n, d, topn = 70, 64, 9
    q = torch.zeros((1, 1, n, d), device="cuda")
    k = torch.randn((1, 1, n, d), device="cuda")
    v = torch.randn((1, 1, n, d), device="cuda")
    zero = torch.zeros(1, device="cuda")
    out = had.soft_forward(q, k, v, topn, 0.3, 0.5, True, sigma_q=zero, sigma_k=zero).cpu().numpy()[0, 0]
    vv = v.cpu().numpy()[0, 0].astype(np.float64)
    for i in range(n):
        want = vv[: min(topn, i + 1)].mean(0)
        assert np.all(np.abs(out[i] - want) <= 1e-5 * np.abs(vv[: min(topn, i + 1)]).mean(0) + 1e-6)
