"""Pins for the CPU oracle: checks against facts fixed by the pages and by
mathematics, never against the oracle's own formulas retyped.

Every pin names the mistake it is meant to catch.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from had_workloads import make_inputs


# ---------------------------------------------------------------- sigma ----
def test_sigma_textbook_example():
    # Population std of 2,4,4,4,5,5,7,9 is exactly 2 (sample std would be
    # 2.138...): catches ddof=1 and a missing square root.
    assert oracle.sigma(np.array([2, 4, 4, 4, 5, 5, 7, 9], dtype=np.float32)) == 2.0


def test_sigma_two_points_and_constant():
    # sigma{a, b} = |a - b| / 2; a constant tensor has sigma 0.
    assert oracle.sigma(np.array([[-3.0], [5.0]])) == pytest.approx(4.0, rel=1e-15)
    assert oracle.sigma(np.full((3, 7), 2.5)) == 0.0


def test_sigma_invariances():
    # sigma(aX) = |a| sigma(X); sigma(X + c) = sigma(X) catches a missing
    # mean subtraction (root mean square instead of std).
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 9, 13))
    s = oracle.sigma(x)
    assert oracle.sigma(-3.0 * x) == pytest.approx(3.0 * s, rel=1e-12)
    assert oracle.sigma(x + 17.0) == pytest.approx(s, rel=1e-10)


def test_sigma_rejects_nan():
    with pytest.raises(ValueError):
        oracle.sigma(np.array([1.0, np.nan]))


# ------------------------------------------------------------- binarize ----
def test_binarize_special_values():
    # x >= 0 -> +1: both zeros give +1 (value compare, not the sign bit),
    # infinities keep their sign.
    x = np.array([-2.0, -0.0, 0.0, 3.0, np.inf, -np.inf, -1e-30, 1e-30], dtype=np.float32)
    assert oracle.binarize(x).tolist() == [-1, 1, 1, 1, 1, -1, -1, 1]


def test_binarize_rejects_nan():
    with pytest.raises(ValueError):
        oracle.binarize(np.array([0.0, np.nan]))


def test_binarize_is_sigma_invariant():
    # The standardization divides by sigma > 0 and cannot change a sign.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 40)).astype(np.float32)
    s = oracle.sigma(x)
    assert np.array_equal(oracle.binarize(x / s), oracle.binarize(x))
    assert np.array_equal(oracle.binarize(x * 1e-20), oracle.binarize(x))


# ----------------------------------------------------------------- pack ----
def _pack_bruteforce(row):
    """Python-int packing, one bit at a time (independent of numpy shifts)."""
    d = len(row)
    words = []
    for w in range((d + 31) // 32):
        value = 0
        for c in range(32 * w, min(d, 32 * w + 32)):
            if row[c] == -1:
                value += 2 ** (c - 32 * w)
        words.append(value)
    return words


@pytest.mark.parametrize("d", [1, 5, 31, 32, 33, 40, 64, 100, 128, 256])
def test_pack_matches_bruteforce(d):
    rng = np.random.default_rng(d)
    b = np.where(rng.random((7, d)) < 0.5, -1, 1).astype(np.int8)
    packed = oracle.pack_bits(b)
    assert packed.shape == (7, (d + 31) // 32)
    for r in range(7):
        assert [int(x) for x in packed[r]] == _pack_bruteforce(b[r].tolist())
    assert np.array_equal(oracle.unpack_bits(packed, d), b)


def test_pack_hand_examples():
    # d=5: signs [-,+,-,-,+] -> bits 0,2,3 -> 13.  d=33: element 32 is bit 0
    # of word 1.  Catches reversed bit order and flipped polarity.
    assert oracle.pack_bits(np.array([-1, 1, -1, -1, 1])).tolist() == [13]
    b = np.ones(33, dtype=np.int8)
    b[32] = -1
    b[0] = -1
    assert oracle.pack_bits(b).tolist() == [1, 1]


def test_pack_pad_bits_zero_and_negation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 40)).astype(np.float32)
    p = oracle.pack_bits(oracle.binarize(x))
    assert np.all(p[:, 1] < (1 << 8))  # 8 data bits in the last word
    pn = oracle.pack_bits(oracle.binarize(-x))
    data_mask = np.array([0xFFFFFFFF, 0xFF], dtype=np.uint32)
    assert np.array_equal(pn, (~p) & data_mask)  # no zeros in x
    assert np.array_equal(oracle.pack_bits(oracle.binarize(7.5 * x)), p)


# --------------------------------------------------------------- logits ----
@pytest.mark.parametrize("d", [1, 3, 32, 33, 64, 128])
def test_logits_equal_xnor_popcount_identity(d):
    # The pages' statement: the +-1 product is computed by XNOR + popcount,
    # i.e. s = d - 2 * popcount(q XOR k).  Python-int popcount of the packed
    # words is an independent route to the same integers.
    rng = np.random.default_rng(100 + d)
    bq = np.where(rng.random((9, d)) < 0.5, -1, 1).astype(np.int8)
    bk = np.where(rng.random((11, d)) < 0.5, -1, 1).astype(np.int8)
    S = oracle.logits(bq, bk)
    pq, pk = oracle.pack_bits(bq), oracle.pack_bits(bk)
    for i in range(9):
        for j in range(11):
            ham = sum(bin(int(a) ^ int(b)).count("1") for a, b in zip(pq[i], pk[j]))
            assert S[i, j] == d - 2 * ham
    # brute-force sum of products on a few entries
    for i, j in [(0, 0), (3, 7), (8, 10)]:
        assert S[i, j] == sum(int(a) * int(b) for a, b in zip(bq[i], bk[j]))


def test_logits_range_parity_symmetry():
    rng = np.random.default_rng(8)
    d = 37
    b = np.where(rng.random((12, d)) < 0.5, -1, 1).astype(np.int8)
    S = oracle.logits(b, b)
    assert S.dtype == np.int64
    assert np.all(np.abs(S) <= d) and np.all((S - d) % 2 == 0)
    assert np.array_equal(S, S.T)
    assert np.all(np.diag(S) == d)
    assert np.all(np.diag(oracle.logits(b, -b)) == -d)


# --------------------------------------------------------------- select ----
def _brute_select(s_row, topn, nv):
    """First (lexicographically smallest) index set of size min(N, nv)
    maximizing the sum of logits: the top-N set with lower-index tie wins."""
    best = None
    for comb in itertools.combinations(range(nv), min(topn, nv)):
        tot = sum(s_row[j] for j in comb)
        if best is None or tot > best[0]:
            best = (tot, comb)
    return list(best[1])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,n,topn", [(3, 8, 3), (2, 9, 4), (5, 7, 2), (1, 6, 3), (4, 8, 8), (3, 5, 9)])
def test_select_matches_subset_bruteforce(d, n, topn, causal):
    # Small d gives many equal logits, so the tie rule is exercised.
    rng = np.random.default_rng(d * 100 + n * 10 + topn)
    bq = np.where(rng.random((n, d)) < 0.5, -1, 1).astype(np.int8)
    bk = np.where(rng.random((n, d)) < 0.5, -1, 1).astype(np.int8)
    S = oracle.logits(bq, bk)
    idx = oracle.select_topn(S, topn, causal)
    for i in range(n):
        nv = i + 1 if causal else n
        want = _brute_select(S[i].tolist(), topn, nv)
        got = [int(j) for j in idx[i] if j >= 0]
        assert got == want, (i, S[i].tolist())
        assert len(got) == min(topn, nv)
        assert all(j == -1 for j in idx[i][len(got):])


def test_select_threshold_separation_and_ties():
    rng = np.random.default_rng(21)
    bq = np.where(rng.random((64, 16)) < 0.5, -1, 1).astype(np.int8)
    bk = np.where(rng.random((200, 16)) < 0.5, -1, 1).astype(np.int8)
    S = oracle.logits(bq, bk)
    idx = oracle.select_topn(S, 37)
    for i in range(64):
        kept = idx[i]
        assert np.all(np.diff(kept) > 0)
        dropped = np.setdiff1d(np.arange(200), kept)
        kmin, dmax = S[i, kept].min(), S[i, dropped].max()
        assert kmin >= dmax
        if kmin == dmax:  # every kept tie has a lower index than every dropped tie
            kt = kept[S[i, kept] == kmin]
            dt = dropped[S[i, dropped] == kmin]
            assert kt.max() < dt.min()


def test_select_rejects_nonpositive_topn():
    with pytest.raises(ValueError):
        oracle.select_topn(np.zeros((2, 3), dtype=np.int64), 0)


# ------------------------------------------------------- softmax and AV ----
def test_full_topn_reduces_to_dense_softmax_attention():
    # N >= n (non-causal) keeps every key: the result must equal dense
    # softmax(scale * S) V, with scipy's softmax as the library routine.
    rng = np.random.default_rng(4)
    n, d = 24, 16
    bq = np.where(rng.random((n, d)) < 0.5, -1, 1).astype(np.int8)
    bk = np.where(rng.random((n, d)) < 0.5, -1, 1).astype(np.int8)
    v = rng.standard_normal((n, 5))
    S = oracle.logits(bq, bk)
    for topn in (n, n + 5):
        idx = oracle.select_topn(S, topn)
        out, _ = oracle.sparse_softmax_av(S, idx, v, 0.3)
        dense = scipy.special.softmax(0.3 * S.astype(np.float64), axis=1) @ v
        np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-14)


def test_rows_sum_to_one_and_convexity():
    # V = ones gives 1 exactly when the softmax is renormalized over the kept
    # set (a global softmax followed by a mask would give less than 1).
    rng = np.random.default_rng(9)
    bq = np.where(rng.random((30, 8)) < 0.5, -1, 1).astype(np.int8)
    bk = np.where(rng.random((50, 8)) < 0.5, -1, 1).astype(np.int8)
    S = oracle.logits(bq, bk)
    idx = oracle.select_topn(S, 7)
    out, mag = oracle.sparse_softmax_av(S, idx, np.ones((50, 3)), 0.9)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-12)
    vpos = rng.random((50, 4))
    out, mag = oracle.sparse_softmax_av(S, idx, vpos, 0.9)
    np.testing.assert_allclose(out, mag, rtol=1e-14)
    for i in range(30):  # convex combination of the kept rows only
        kept = idx[i]
        assert np.all(out[i] <= vpos[kept].max(0) + 1e-12)
        assert np.all(out[i] >= vpos[kept].min(0) - 1e-12)


def test_two_kept_keys_follow_the_logistic_closed_form():
    # With V = identity rows the output is the probability row itself; with
    # two kept keys the softmax is the logistic function of the logit gap.
    bq = np.array([[1, 1, 1, 1]], dtype=np.int8)
    bk = np.array([[1, 1, 1, -1], [1, -1, -1, -1], [1, 1, 1, 1], [-1, -1, -1, -1]], dtype=np.int8)
    S = oracle.logits(bq, bk)
    assert S.tolist() == [[2, -2, 4, -4]]
    idx = oracle.select_topn(S, 2)
    assert idx.tolist() == [[0, 2]]
    out, _ = oracle.sparse_softmax_av(S, idx, np.eye(4), 0.7)
    p2 = 1.0 / (1.0 + math.exp(-0.7 * (4 - 2)))
    np.testing.assert_allclose(out[0], [1 - p2, 0.0, p2, 0.0], rtol=1e-14, atol=1e-15)


def test_equal_logits_or_tiny_scale_give_the_mean_of_kept_rows():
    rng = np.random.default_rng(13)
    bq = np.where(rng.random((10, 6)) < 0.5, -1, 1).astype(np.int8)
    bk = np.where(rng.random((40, 6)) < 0.5, -1, 1).astype(np.int8)
    v = rng.standard_normal((40, 3))
    S = oracle.logits(bq, bk)
    idx = oracle.select_topn(S, 9)
    out, _ = oracle.sparse_softmax_av(S, idx, v, 1e-13)
    for i in range(10):
        np.testing.assert_allclose(out[i], v[idx[i]].mean(0), rtol=1e-9, atol=1e-11)
    Seq = np.full((3, 40), 5, dtype=np.int64)
    idx = oracle.select_topn(Seq, 4)
    assert idx.tolist() == [[0, 1, 2, 3]] * 3  # all tied: the lowest indices
    out, _ = oracle.sparse_softmax_av(Seq, idx, v, 2.0)
    np.testing.assert_allclose(out, np.tile(v[:4].mean(0), (3, 1)), rtol=1e-13)


# ------------------------------------------------------- golden fixture ----
def test_hand_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_example_d4_n4.json")))
    q = np.array(g["q"], dtype=np.float32)
    k = np.array(g["k"], dtype=np.float32)
    v = np.array(g["v"], dtype=np.float64)
    r = oracle.forward(q, k, v, g["topn"], g["scale"])
    assert r["qbits"][:, 0].tolist() == g["qbits"]
    assert r["kbits"][:, 0].tolist() == g["kbits"]
    assert r["S"].tolist() == g["S"]
    assert r["idx"].tolist() == g["idx"]
    np.testing.assert_allclose(r["out"], g["out"], rtol=1e-14, atol=1e-15)
    rc = oracle.forward(q, k, v, g["topn"], g["scale"], causal=True)
    assert rc["idx"].tolist() == g["causal_idx"]
    np.testing.assert_allclose(rc["out"], g["causal_out"], rtol=1e-14, atol=1e-15)


def test_forward_row_subset_matches_full():
    w = make_inputs(1, 1, 70, 40, v_dtype="bf16", rank=3, noise="t3", seed=77)
    q, k, v = w["q"][0, 0], w["k"][0, 0], w["v"][0, 0]
    full = oracle.forward(q, k, v, 9, 0.2, causal=True)
    rows = np.array([0, 5, 33, 69])
    part = oracle.forward(q, k, v, 9, 0.2, causal=True, rows=rows)
    assert np.array_equal(part["idx"], full["idx"][rows])
    np.testing.assert_allclose(part["out"], full["out"][rows], rtol=0, atol=0)


# --------------------------------------------------------------- decode ----
def test_decode_rows_match_the_same_rows_of_the_full_sequence():
    # New rows at positions p0..p0+m-1 against the cache of the first n_k
    # tokens: exactly the rows p0.. of the full-sequence path (catches an
    # off-by-one in the query positions or the causal limit).
    inp = make_inputs(1, 1, 80, 40, rank=4, noise="t3", seed=12, v_dtype="f32")
    q, k, v = inp["q"][0, 0], inp["k"][0, 0], inp["v"][0, 0]
    for causal in (False, True):
        for p0, m in ((0, 1), (17, 5), (75, 5)):
            rows = np.arange(p0, p0 + m)
            full = oracle.forward(q, k, v, 9, 0.3, causal=causal, rows=rows)
            dec = oracle.decode(q[rows], k, v, 9, 0.3, q_pos0=p0, causal=causal)
            assert np.array_equal(dec["idx"], full["idx"])
            np.testing.assert_array_equal(dec["out"], full["out"])


def test_decode_first_position_sees_only_the_first_key():
    # Causal row at position 0: one visible key, so the output is V[0]
    # itself whatever N and the logits (closed form).
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 33))
    k = rng.standard_normal((50, 33))
    v = rng.standard_normal((50, 7))
    r = oracle.decode(q, k, v, 5, 0.4, q_pos0=0, causal=True)
    assert r["idx"][0].tolist() == [0, -1, -1, -1, -1]
    np.testing.assert_allclose(r["out"][0], v[0], rtol=0, atol=0)


def test_decode_with_every_visible_key_is_dense_softmax_over_the_prefix():
    # N >= visible keys: softmax over the visible prefix (scipy) times V.
    rng = np.random.default_rng(9)
    n_k, d = 30, 24
    q = rng.standard_normal((3, d))
    k = rng.standard_normal((n_k, d))
    v = rng.standard_normal((n_k, 4))
    r = oracle.decode(q, k, v, 64, 0.25, q_pos0=10, causal=True)
    sq = np.where(q >= 0, 1.0, -1.0)
    sk = np.where(k >= 0, 1.0, -1.0)
    for i in range(3):
        vis = 10 + i + 1
        s = sk[:vis] @ sq[i]
        want = scipy.special.softmax(0.25 * s) @ v[:vis]
        np.testing.assert_allclose(r["out"][i], want, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------ top-N mass ----
def test_topn_mass_equal_logits_closed_form():
    # Equal logits: every weight is 1/n, so N = ceil(mass * n).
    S = np.zeros((1, 40))
    for mass in (0.01, 0.3, 0.5, 0.97):
        assert oracle.topn_mass(S, 0.7, mass)[0] == math.ceil(mass * 40 - 1e-12)


def test_topn_mass_two_levels_closed_form():
    # a keys at logit 1, b keys at logit 0: each top key weighs e/(a e + b).
    a, b, scale = 3, 9, 2.0
    S = np.array([[1.0] * a + [0.0] * b])
    wt = math.exp(scale) / (a * math.exp(scale) + b)
    wl = 1.0 / (a * math.exp(scale) + b)
    for mass in (0.1, 0.4, 0.6, 0.9, 0.99):
        k = math.ceil(mass / wt - 1e-12)
        want = k if k <= a else a + math.ceil((mass - a * wt) / wl - 1e-12)
        assert oracle.topn_mass(S, scale, mass)[0] == want


def test_topn_mass_brute_force_and_limits():
    # Brute force over subsets: the smallest subset whose softmax mass reaches
    # the target (any subset, not only prefixes); mass >= 1 keeps everything;
    # a causal row sees its prefix only.
    rng = np.random.default_rng(21)
    S = rng.integers(-4, 5, size=(6, 7)).astype(np.float64)
    for mass in (0.25, 0.5, 0.8):
        got = oracle.topn_mass(S, 0.6, mass)
        for r in range(6):
            p = np.exp(0.6 * S[r]) / np.exp(0.6 * S[r]).sum()
            best = min(len(c) for k in range(1, 8) for c in itertools.combinations(range(7), k)
                       if p[list(c)].sum() >= mass - 1e-15)
            assert got[r] == best
    assert oracle.topn_mass(S, 0.6, 1.0).tolist() == [7] * 6
    assert oracle.topn_mass(S, 0.6, 1.0, causal=True).tolist() == [1, 2, 3, 4, 5, 6]


# ------------------------------------------------- straight-through backward ----
def _pm1(x):
    # {-1, +1} with x >= 0 -> +1, written here independently of oracle.binarize
    return np.where(np.asarray(x) >= 0, 1.0, -1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_with_every_key_kept_matches_torch_autograd(causal):
    """N >= n keeps every visible key, so the path is dense (masked) softmax
    attention on the +-1 matrices; with the straight-through estimator on the
    standardized inputs (sign's derivative taken as 1, sigma constant) its
    gradients are what torch's float64 autograd gives for
    u = x / sigma;  b = u + (sign(u) - u).detach().  Catches a dropped -D_i
    term, a transposed dS, a missing scale or 1/sigma, and dV from the wrong
    weights."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(31 + causal)
    n, d, scale, sq, sk = 9, 7, 0.37, 1.7, 0.6
    q, k, v, dout = (rng.standard_normal((n, d)) for _ in range(4))
    r = oracle.backward(q, k, v, dout, n + 3, scale, causal, sigma_q=sq, sigma_k=sk)
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    uq, uk = tq / sq, tk / sk
    bq = uq + (torch.where(uq >= 0, 1.0, -1.0) - uq).detach()
    bk = uk + (torch.where(uk >= 0, 1.0, -1.0) - uk).detach()
    z = scale * (bq @ bk.T)
    if causal:
        z = z.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    out = torch.softmax(z, dim=-1) @ tv
    (out * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("d,n,topn,causal", [(5, 11, 4, False), (5, 11, 4, True), (3, 8, 2, False),
                                              (33, 10, 5, True)])
def test_backward_matches_finite_differences_with_the_kept_sets_fixed(d, n, topn, causal):
    """Central differences (float64) of f = sum(dout * out) with the kept
    sets held at the oracle's choice, the +-1 matrices and V perturbed as real
    numbers.  f is written here as a masked dense softmax (keep mask -> -inf
    elsewhere), not with the oracle's per-row loop; few feature values (small
    d) make ties at the threshold common."""
    rng = np.random.default_rng(100 * d + n + topn + causal)
    q, k, v, dout = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 0.45
    r = oracle.backward(q, k, v, dout, topn, scale, causal)
    keep = np.zeros((n, n), dtype=bool)
    for i in range(n):
        keep[i, r["idx"][i][r["idx"][i] >= 0]] = True

    def f(bq, bk, vv):
        z = np.where(keep, scale * (bq @ bk.T), -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return float(np.sum(dout * (p @ vv)))

    bq0, bk0 = _pm1(q), _pm1(k)
    h = 1e-6
    for name, base, grad in (("bq", bq0, r["dq"]), ("bk", bk0, r["dk"]), ("v", v, r["dv"])):
        for i, c in [(0, 0), (n // 2, d - 1), (n - 1, d // 2), (1, 1 % d)]:
            plus, minus = base.copy(), base.copy()
            plus[i, c] += h
            minus[i, c] -= h
            args_p = {"bq": (plus, bk0, v), "bk": (bq0, plus, v), "v": (bq0, bk0, plus)}[name]
            args_m = {"bq": (minus, bk0, v), "bk": (bq0, minus, v), "v": (bq0, bk0, minus)}[name]
            fd = (f(*args_p) - f(*args_m)) / (2 * h)
            assert abs(fd - grad[i, c]) <= 1e-7 * (1 + abs(fd)), (name, i, c, fd, grad[i, c])


def test_backward_two_kept_keys_closed_form():
    """One row keeping two keys with logits s1 > s2: p1 = logistic(scale (s1 - s2)),
    dS_1 = -dS_2 = scale p1 p2 dout.(V1 - V2), dV_1 = p1 dout, dV_2 = p2 dout,
    and the dropped key gets nothing."""
    q = np.array([[1.0, 1.0, 1.0, 1.0]])
    k = np.array([[1.0, 1.0, 1.0, 1.0],      # s = 4
                  [1.0, 1.0, 1.0, -1.0],     # s = 2
                  [-1.0, -1.0, -1.0, -1.0]])  # s = -4, dropped
    v = np.array([[0.5, -1.0, 2.0, 0.0], [1.5, 0.25, -1.0, 3.0], [9.0, 9.0, 9.0, 9.0]])
    dout = np.array([[1.0, -2.0, 0.5, 1.0]])
    scale = 0.3
    p1 = 1.0 / (1.0 + math.exp(-scale * 2.0))
    p2 = 1.0 - p1
    g = scale * p1 * p2 * float(dout[0] @ (v[0] - v[1]))
    r = oracle.backward(q, k, v, dout, 2, scale)
    np.testing.assert_allclose(r["dv"], [p1 * dout[0], p2 * dout[0], np.zeros(4)], rtol=1e-14, atol=1e-15)
    # dq = dS_1 Bk_1 + dS_2 Bk_2;  dk_j = dS_j Bq
    np.testing.assert_allclose(r["dq"][0], g * k[0] - g * k[1], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r["dk"], [g * q[0], -g * q[0], np.zeros(4)], rtol=1e-13, atol=1e-15)


def test_backward_invariants():
    """Softmax gradients sum to zero over a row's kept keys (so sum_i dq_i .
    1-direction checks hold), dV sums to sum_i dout_i over the keys, the
    gradient is linear in dout, and the row-block size changes nothing."""
    rng = np.random.default_rng(5)
    n, d, topn = 40, 6, 9
    q, k, v, dout = (rng.standard_normal((n, d)) for _ in range(4))
    bq, bk = oracle.binarize(q), oracle.binarize(k)
    S = oracle.logits(bq, bk)
    idx = oracle.select_topn(S, topn, True)
    ds, dv, e_ds, _ = oracle.sparse_softmax_av_backward(S, idx, v, dout, 0.5)
    assert np.all(np.abs(ds.sum(axis=1)) <= 1e-13 * (1 + e_ds.sum(axis=1)))
    kept = np.zeros(ds.shape, dtype=bool)
    for i in range(n):
        kept[i, idx[i][idx[i] >= 0]] = True
    assert np.all(ds[~kept] == 0) and np.count_nonzero(kept, axis=1).tolist() == \
        [min(topn, i + 1) for i in range(n)]
    np.testing.assert_allclose(dv.sum(axis=0), dout.sum(axis=0), rtol=0, atol=1e-12)
    r1 = oracle.backward(q, k, v, dout, topn, 0.5, True)
    r2 = oracle.backward(q, k, v, 2.5 * dout, topn, 0.5, True, block=7)
    for x in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r2[x], 2.5 * r1[x], rtol=1e-12, atol=1e-13)
    assert np.all(r1["e_dq"] >= np.abs(r1["dq"])) and np.all(r1["e_dv"] >= np.abs(r1["dv"]))


# ------------------------------------------ scaled-tanh (soft) forward ----
def _away_from_zero(x, floor):
    """Move every element at least `floor` away from 0, keeping its sign."""
    return np.where(x >= 0, x + floor, x - floor)


@pytest.mark.parametrize("causal", [False, True])
def test_soft_forward_small_c_is_the_sign_path(causal):
    # tanh(u / c) is exactly +-1 in float64 once |u / c| > 19.1; with every
    # |x| >= 0.05 sigma and c = 1e-3 that holds for all elements, so the soft
    # path must give the sign path's logits, kept sets and outputs exactly.
    # Catches tanh(u * c) in place of tanh(u / c) and a missing standardization
    # factor that pushes |u / c| back into tanh's curved range.
    w = make_inputs(1, 1, 60, 24, v_dtype="f32", rank=3, noise="t3", seed=31)
    q, k, v = w["q"][0, 0], w["k"][0, 0], w["v"][0, 0]
    q = _away_from_zero(q, 0.05 * oracle.sigma(q) + 0.05 * 3 * np.abs(q).max())
    k = _away_from_zero(k, 0.05 * oracle.sigma(k) + 0.05 * 3 * np.abs(k).max())
    assert np.abs(q).min() >= 0.05 * oracle.sigma(q) and np.abs(k).min() >= 0.05 * oracle.sigma(k)
    for topn in (1, 7, 60):
        soft = oracle.soft_forward(q, k, v, topn, 0.3, 1e-3, causal=causal)
        hard = oracle.forward(q, k, v, topn, 0.3, causal=causal)
        assert np.array_equal(soft["S"], hard["S"].astype(np.float64))
        assert np.array_equal(soft["idx"], hard["idx"])
        np.testing.assert_array_equal(soft["out"], hard["out"])


def test_soft_forward_large_c_is_topn_attention_on_the_standardized_inputs():
    # c^2 tanh(a / c) tanh(b / c) = a b (1 - (a^2 + b^2) / (3 c^2) + ...), so
    # with scale * c^2 and c = 1e4 the soft path is top-N softmax attention
    # over the dot products of x / sigma, up to ~1e-7 relative.  The reference
    # here is built directly: standardized products, argsort, scipy softmax.
    # Catches a dropped or squared sigma (the inputs have sigma far from 1).
    rng = np.random.default_rng(5)
    n, d, topn, scale, c = 48, 16, 9, 0.2, 1.0e4
    q = 3.0 * rng.standard_normal((n, d)) + 0.4
    k = 0.5 * rng.standard_normal((n, d)) - 0.1
    v = rng.standard_normal((n, 6))
    soft = oracle.soft_forward(q, k, v, topn, scale * c * c, c)
    u = (q / q.std()) @ (k / k.std()).T
    for i in range(n):
        kept = np.sort(np.argsort(-u[i], kind="stable")[:topn])
        assert soft["idx"][i].tolist() == kept.tolist()
        p = scipy.special.softmax(scale * u[i, kept])
        np.testing.assert_allclose(soft["out"][i], p @ v[kept], rtol=1e-5, atol=1e-7)


def test_soft_forward_two_keys_closed_form():
    # atanh inverts the soft sign at c = 1, sigma = 1: q = atanh(0.8) and keys
    # atanh(+-0.5) give logits +-0.4, and the two kept keys mix by the logistic
    # function of the gap 0.8 * scale.
    q = np.array([[math.atanh(0.8)]])
    k = np.array([[math.atanh(0.5)], [math.atanh(-0.5)], [math.atanh(0.1)]])
    v = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, 5.0]])
    r = oracle.soft_forward(q, k, v, 2, 1.5, 1.0, sigma_q=1.0, sigma_k=1.0)
    np.testing.assert_allclose(r["S"], [[0.4, -0.4, 0.08]], rtol=1e-14)
    assert r["idx"].tolist() == [[0, 2]]
    p0 = 1.0 / (1.0 + math.exp(-1.5 * (0.4 - 0.08)))
    np.testing.assert_allclose(r["out"][0], p0 * v[0] + (1 - p0) * v[2], rtol=1e-14)


def test_soft_forward_symmetries_and_bounds():
    # tanh is odd: negating both q and k leaves the logits and the output
    # unchanged, negating q alone negates every logit; |S| <= d always.
    rng = np.random.default_rng(17)
    n, d = 30, 12
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, 4))
    a = oracle.soft_forward(q, k, v, 5, 0.7, 0.6)
    b = oracle.soft_forward(-q, -k, v, 5, 0.7, 0.6)
    np.testing.assert_array_equal(a["S"], b["S"])
    np.testing.assert_array_equal(a["out"], b["out"])
    neg = oracle.soft_forward(-q, k, v, 5, 0.7, 0.6)
    np.testing.assert_array_equal(neg["S"], -a["S"])
    assert np.abs(a["S"]).max() <= d
    tiny = oracle.soft_forward(q, k, v, 5, 0.7, 1e-9)
    assert np.abs(tiny["S"]).max() <= d and np.all(np.abs(np.rint(tiny["S"]) - tiny["S"]) == 0)
    with pytest.raises(ValueError):
        oracle.soft_forward(q, k, v, 5, 0.7, 0.0)
