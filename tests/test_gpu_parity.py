"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bits, integer logits and selected indices must match bit for bit; outputs
must be within 1e-5 * sum(p|V|) (fp32 V) or 2e-3 * max|V| (bf16 V); sigma
within 1e-6 relative.  Every case prints its name, shape and seed first.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_had_amd as had
from had_workloads import WORKLOADS, make_inputs, workload_inputs
from parity_util import bits_np, check_out, check_topn_mass, log, oracle_head, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()


# --------------------------------------------------------------------- pack
@pytest.mark.parametrize("shape", [(1, 1, 128, 64), (2, 3, 77, 128), (1, 2, 50, 40), (3, 1, 9, 33),
                                   (1, 1, 5, 5), (1, 2, 31, 256), (1, 1, 1, 1), (4, 4, 300, 32),
                                   (1, 1, 999, 32), (2, 3, 1001, 64), (1, 4, 8192, 128),
                                   (2, 8, 8192, 128)])
def test_pack_bits_and_sigma(shape):
    log(f"pack {shape}")
    rng = np.random.default_rng(sum(shape))
    x = (rng.standard_normal(shape) * 3 + 0.7).astype(np.float32)
    flat = x.reshape(-1)
    flat[:: 7] = 0.0
    flat[3:: 11] = -0.0
    if flat.size > 20:
        flat[5] = np.inf
        flat[6] = -np.inf
        x_sig = x.copy()
        x_sig.reshape(-1)[5:7] = 0.0
    else:
        x_sig = x
    xt = torch.from_numpy(x).cuda()
    bits, sig = had.pack(xt)
    torch.cuda.synchronize()
    want = oracle.pack_bits(oracle.binarize(x))
    assert np.array_equal(bits_np(bits), want)
    # sigma on a finite copy (infinities make sigma meaningless)
    xs = torch.from_numpy(x_sig).cuda()
    _, sig2 = had.pack(xs)
    ref = oracle.sigma(x_sig)
    assert abs(float(sig2.item()) - ref) <= 1e-6 * ref + 1e-30


@pytest.mark.parametrize("shape,offset,spread", [((2, 3, 77, 64), 1.0e4, 1.0), ((1, 4, 1000, 128), -3.0e5, 2.0),
                                                  ((3, 1, 9, 33), 2.5e4, 0.5), ((2, 2, 300, 64), 1.0e4, 1.0e-2)])
def test_pack_sigma_with_a_large_common_offset(shape, offset, spread):
    """x = offset + spread * N(0, 1): the mean is 1e4 to 1e6 times the spread,
    where a one-pass sum of raw squares would lose the digits sigma needs.
    Sigma must still be within 1e-6 relative of the oracle's two-pass value,
    through had_pack, had_forward and the running calibration."""
    log(f"pack sigma offset {shape} {offset} {spread}")
    rng = np.random.default_rng(int(abs(offset)) + shape[2])
    x = (offset + spread * rng.standard_normal(shape)).astype(np.float32)
    ref = oracle.sigma(x)
    xt = torch.from_numpy(x).cuda()
    _, sig = had.pack(xt)
    assert abs(float(sig.item()) - ref) <= 1e-6 * ref, (float(sig.item()), ref)
    v = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    _, _, _, sq, _ = had.forward(xt, xt, v, 4, 0.1, False)
    assert abs(float(sq.item()) - ref) <= 1e-6 * ref, (float(sq.item()), ref)
    # calibration over two halves of the batch, then the whole tensor
    state = had.sigma_state()
    half = shape[0] // 2 or 1
    parts = [x[:half], x[half:]] if shape[0] > 1 else [x]
    for part in parts:
        had.pack_calibrate(torch.from_numpy(np.ascontiguousarray(part)).cuda(), state)
    sc = float(had.sigma_from_state(state).item())
    assert abs(sc - ref) <= 1e-6 * ref, (sc, ref)


@pytest.mark.parametrize("shape", [(2, 3, 77, 64), (1, 1, 999, 32)])
def test_pack_unaligned_input(shape):
    """x at a 4-byte but not 16-byte aligned address takes the scalar path."""
    log(f"pack unaligned {shape}")
    rng = np.random.default_rng(7 + shape[2])
    x = rng.standard_normal(shape).astype(np.float32)
    buf = torch.zeros(x.size + 1, dtype=torch.float32, device="cuda")
    buf[1:] = torch.from_numpy(x.reshape(-1)).cuda()
    xt = buf[1:].view(shape)
    assert xt.data_ptr() % 16 != 0
    bits, sig = had.pack(xt)
    torch.cuda.synchronize()
    assert np.array_equal(bits_np(bits), oracle.pack_bits(oracle.binarize(x)))
    ref = oracle.sigma(x)
    assert abs(float(sig.item()) - ref) <= 1e-6 * ref


def test_pack_flags_nan_and_is_deterministic():
    log("pack nan/determinism")
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 2, 100, 64)).astype(np.float32)
    xt = torch.from_numpy(x).cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    b1, s1 = had.pack(xt, dev_status=st)
    b2, s2 = had.pack(xt, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(b1, b2) and torch.equal(s1, s2)
    x[1, 1, 7, 3] = np.nan
    had.pack(torch.from_numpy(x).cuda(), dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & had.DEV_NAN_INPUT


def test_pack_without_sigma_and_constant_input():
    log("pack constant")
    x = torch.full((1, 1, 64, 64), -2.5, device="cuda")
    bits, sig = had.pack(x)
    torch.cuda.synchronize()
    assert float(sig.item()) == 0.0
    assert np.all(bits_np(bits) == 0xFFFFFFFF)
    bits2, none = had.pack(x, with_sigma=False)
    assert none is None and torch.equal(bits, bits2)


# ------------------------------------------------------------------- logits
@pytest.mark.parametrize("shape", [(1, 1, 128, 64), (2, 3, 300, 64), (1, 2, 77, 128), (1, 1, 50, 40),
                                   (1, 1, 70, 256), (1, 1, 33, 1), (1, 1, 200, 96)])
def test_logits_bit_exact(shape):
    log(f"logits {shape}")
    B, H, n, d = shape
    inp = make_inputs(B, H, n, d, rank=4, noise="t3", seed=n + d)
    q, k, _ = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    s = had.logits(qb, kb, d).cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = oracle.logits(oracle.binarize(inp["q"][b, h]), oracle.binarize(inp["k"][b, h]))
            assert np.array_equal(s[b * H + h].astype(np.int64), ref), (b, h)


def test_logits_row_and_slice_ranges():
    log("logits ranges")
    inp = make_inputs(2, 2, 260, 64, rank=4, seed=9)
    q, k, _ = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    s = had.logits(qb, kb, 64, bh_begin=1, bh_count=2, row_begin=130, row_count=70).cpu().numpy()
    for t, bh in enumerate((1, 2)):
        b, h = divmod(bh, 2)
        ref = oracle.logits(oracle.binarize(inp["q"][b, h][130:200]), oracle.binarize(inp["k"][b, h]))
        assert np.array_equal(s[t].astype(np.int64), ref)


# ------------------------------------------------------------------- select
SELECT_CASES = [
    # B, H, n, d, topn, causal
    (1, 1, 128, 64, 32, False),
    (2, 3, 300, 64, 37, False),
    (2, 3, 300, 64, 37, True),
    (1, 2, 200, 128, 50, True),
    (1, 1, 97, 5, 10, False),     # tiny d: ties everywhere
    (1, 1, 97, 5, 10, True),
    (1, 2, 64, 64, 64, False),    # N = n: every key
    (1, 1, 50, 64, 80, True),     # N > n
    (1, 1, 130, 33, 1, False),    # N = 1
    (1, 1, 40, 256, 7, True),
    (1, 1, 1, 64, 4, True),       # single token
]


@pytest.mark.parametrize("case", SELECT_CASES)
def test_select_bit_exact(case):
    B, H, n, d, topn, causal = case
    log(f"select {case}")
    inp = make_inputs(B, H, n, d, rank=4, noise="normal", seed=n * 7 + d + topn)
    q, k, _ = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    idx = had.select(qb, kb, d, topn, causal).cpu().numpy()
    for b in range(B):
        for h in range(H):
            S = oracle.logits(oracle.binarize(inp["q"][b, h]), oracle.binarize(inp["k"][b, h]))
            ref = oracle.select_topn(S, topn, causal)
            got = idx[b * H + h].astype(np.int64)
            if not np.array_equal(got, ref):
                r = int(np.argwhere((got != ref).any(1))[0][0])
                raise AssertionError(f"slice {(b, h)} row {r}: got {got[r].tolist()} want {ref[r].tolist()}")


# ---------------------------------------------------------------- attention
ATTN_CASES = [
    # B, H, n, d, topn, causal, v_dtype, scale
    (1, 1, 128, 64, 32, False, "f32", 0.125),
    (1, 1, 128, 64, 32, False, "bf16", 0.125),
    (2, 3, 300, 64, 37, False, "bf16", 0.125),
    (2, 3, 300, 64, 37, True, "bf16", 0.125),
    (2, 2, 300, 64, 37, True, "f32", 0.4),
    (1, 2, 200, 128, 50, True, "bf16", 1 / np.sqrt(128)),
    (1, 2, 200, 128, 50, False, "f32", 1 / np.sqrt(128)),
    (1, 1, 97, 40, 10, False, "bf16", 0.3),
    (1, 1, 97, 5, 10, True, "f32", 0.9),
    (1, 1, 70, 256, 20, False, "bf16", 1 / 16),
    (1, 1, 64, 64, 64, False, "bf16", 0.125),
    (1, 1, 50, 64, 80, True, "bf16", 0.125),
    (1, 1, 130, 64, 1, False, "f32", 0.125),
    (1, 1, 1, 64, 4, True, "bf16", 0.125),
    (1, 1, 100, 64, 16, False, "bf16", 3.0),   # sharp softmax
    (2, 2, 177, 32, 20, True, "bf16", 0.2),    # d = 32: one word per row
    (1, 2, 160, 96, 30, False, "bf16", 0.1),   # d = 96: three words per row
    (1, 1, 90, 256, 40, True, "f32", 1 / 16),  # fp32 V at d = 256
    (1, 1, 100, 64, 16, False, "f32", 60.0),   # weights past the first bin underflow to 0
    (1, 2, 150, 128, 30, True, "bf16", 60.0),
]


@pytest.mark.parametrize("case", ATTN_CASES)
def test_attention_matches_oracle(case):
    B, H, n, d, topn, causal, vdt, scale = case
    log(f"attention {case}")
    inp = make_inputs(B, H, n, d, v_dtype=vdt, rank=8, noise="t3", seed=n * 3 + d + topn)
    q, k, v = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    out = had.attention(qb, kb, v, topn, scale, causal).cpu().numpy()
    for b in range(B):
        for h in range(H):
            r = oracle_head(inp, b, h, topn, scale, causal)
            check_out(out[b, h], r["out"], r["E"], inp["v"], vdt, where=f"slice {(b, h)}")


def test_attention_is_deterministic():
    log("attention determinism")
    inp = make_inputs(2, 2, 400, 64, v_dtype="bf16", rank=8, noise="t3", seed=5)
    q, k, v = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    o1 = had.attention(qb, kb, v, 50, 0.125, True).clone()
    o2 = had.attention(qb, kb, v, 50, 0.125, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_attention_invariants():
    log("attention invariants")
    inp = make_inputs(1, 2, 150, 64, v_dtype="bf16", rank=8, seed=17)
    q, k, _ = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    ones = torch.ones((1, 2, 150, 64), dtype=torch.bfloat16, device="cuda")
    o = had.attention(qb, kb, ones, 20, 0.125, True)
    torch.cuda.synchronize()
    assert torch.allclose(o, torch.ones_like(o), atol=1e-5, rtol=0)
    # tiny scale: the mean of the selected V rows
    v = torch.from_numpy(inp["v"]).cuda().to(torch.float32)
    o = had.attention(qb, kb, v, 20, 1e-9, False).cpu().numpy()
    idx = had.select(qb, kb, 64, 20, False).cpu().numpy()
    for h in range(2):
        mean = inp["v"][0, h][idx[h]].mean(axis=1)
        np.testing.assert_allclose(o[0, h], mean, rtol=0, atol=1e-5)


@pytest.mark.parametrize("case", [(1, 2, 64, 64, 20, False, 0.3), (1, 1, 200, 256, 37, True, 0.2),
                                  (2, 1, 128, 128, 128, False, 0.05), (1, 1, 100, 100, 1, True, 1.0)])
def test_attention_onehot_v_gives_the_weight_row(case):
    """V = identity rows (n <= d, fp32): out_i is row i of the sparse softmax
    matrix itself, so its non-zero positions are exactly the kept set the
    attend path chose (N_i of them) and its values the oracle's weights."""
    B, H, n, d, topn, causal, scale = case
    log(f"attention one-hot V {case}")
    inp = make_inputs(B, H, n, d, rank=4, noise="t3", seed=n + d + topn)
    q, k, _ = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    eye = np.zeros((B, H, n, d), dtype=np.float32)
    eye[:, :, np.arange(n), np.arange(n)] = 1.0
    out = had.attention(qb, kb, torch.from_numpy(eye).cuda(), topn, scale, causal).cpu().numpy()
    for b in range(B):
        for h in range(H):
            r = oracle.forward(inp["q"][b, h], inp["k"][b, h], eye[b, h], topn, scale, causal=causal)
            check_out(out[b, h], r["out"], r["E"], eye, "f32", where=f"slice {(b, h)}")
            for i in range(n):
                kept = r["idx"][i][r["idx"][i] >= 0]
                nz = np.nonzero(out[b, h, i])[0]
                assert np.array_equal(nz, kept), f"slice {(b, h)} row {i}: non-zeros {nz[:10]} kept {kept[:10]}"
                assert nz.size == min(topn, i + 1 if causal else n)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_at_the_sequence_limit(causal):
    """n = 65536 (the limit) with d = 5: six possible logits, so the threshold
    bin holds thousands of ties, each lane-half's 16-bit histogram counter
    sees up to 32768 keys and the tie count in the selection key reaches its
    bound.  Sampled rows against the oracle: indices bit-exact, outputs within
    the bf16 tolerance."""
    B, H, n, d, topn, scale = 1, 1, 65536, 5, 300, 0.3
    log(f"attention at the limit {(B, H, n, d, topn, causal)}")
    inp = make_inputs(B, H, n, d, rank=4, noise="normal", seed=99, v_dtype="bf16")
    q, k, v = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    out = had.attention(qb, kb, v, topn, scale, causal).cpu().numpy()
    idx = had.select(qb, kb, d, topn, causal)[0].cpu().numpy()
    rows = np.array([0, 1, 2, 37, 299, 300, 32767, 32768, 40000, 65534, 65535])
    r = oracle_head(inp, 0, 0, topn, scale, causal, rows=rows)
    assert np.array_equal(idx[r["rows"]].astype(np.int64), r["idx"])
    check_out(out[0, 0][r["rows"]], r["out"], r["E"], inp["v"], "bf16", where=f"n={n} causal={causal}")


# --------------------------------------------------------------- workloads
def _workload_check(name, sample_rows=None, select_heads=None):
    w = WORKLOADS[name]
    log(f"workload {name}: B={w.batch} H={w.heads} n={w.seq} d={w.dim} N={w.topn} "
        f"causal={w.causal} v={w.v_dtype} seed={w.seed}")
    inp = workload_inputs(w)
    q, k, v = to_dev(inp)
    qb, sq = had.pack(q)
    kb, sk = had.pack(k)
    out = had.attention(qb, kb, v, w.topn, w.scale, w.causal)
    torch.cuda.synchronize()
    log(f"  gpu done; checking sigma and bits")
    assert abs(sq.item() - oracle.sigma(inp["q"])) <= 1e-6 * oracle.sigma(inp["q"])
    assert abs(sk.item() - oracle.sigma(inp["k"])) <= 1e-6 * oracle.sigma(inp["k"])
    qbn, kbn = bits_np(qb), bits_np(kb)
    out = out.cpu().numpy()
    worst = 0.0
    BH = w.batch * w.heads
    for bh in range(BH):
        b, h = divmod(bh, w.heads)
        assert np.array_equal(qbn[b, h], oracle.pack_bits(oracle.binarize(inp["q"][b, h])))
        assert np.array_equal(kbn[b, h], oracle.pack_bits(oracle.binarize(inp["k"][b, h])))
        rows = None if sample_rows is None else sample_rows(bh)
        r = oracle_head(inp, b, h, w.topn, w.scale, w.causal, rows=rows)
        got = out[b, h] if rows is None else out[b, h][r["rows"]]
        worst = max(worst, check_out(got, r["out"], r["E"], inp["v"], w.v_dtype, where=f"{name} slice {bh}"))
        if select_heads is not None and bh in select_heads:
            idx = had.select(qb, kb, w.dim, w.topn, w.causal, bh_begin=bh, bh_count=1)[0].cpu().numpy()
            ref_rows = r["rows"]
            assert np.array_equal(idx[ref_rows].astype(np.int64), r["idx"]), f"{name} select slice {bh}"
    log(f"  max abs error {worst:.3e}")


def test_workload_single_head_n128():
    _workload_check("single-head-n128", select_heads={0})


def test_workload_bert_base_n128():
    _workload_check("bert-base-n128", select_heads={0, 383})


def test_workload_deit_s_n197():
    _workload_check("deit-s-n197", select_heads={0, 200})


def test_workload_t5_base_n1024_sampled():
    rng = np.random.default_rng(44)
    _workload_check("t5-base-n1024",
                    sample_rows=lambda bh: np.unique(np.r_[0, 1023, rng.integers(0, 1024, 14)]),
                    select_heads={0, 95})


def test_workload_causal_n16384_sampled():
    rng = np.random.default_rng(55)
    _workload_check("causal-n16384",
                    sample_rows=lambda bh: np.unique(np.r_[0, 1, 2047, 2048, 16383,
                                                           rng.integers(0, 16384, 4)]),
                    select_heads={7})


# ------------------------------------------------------------ top-N mass
MASS_CASES = [
    # B, H, n, d, causal, scale
    (1, 2, 300, 64, False, 0.125),
    (2, 1, 257, 64, True, 0.125),
    (1, 1, 97, 5, False, 0.9),     # few distinct logits: large tie bins
    (1, 2, 200, 128, True, 1 / np.sqrt(128)),
    (1, 1, 64, 40, False, 2.0),    # sharp softmax
]


@pytest.mark.parametrize("case", MASS_CASES)
def test_topn_mass_matches_oracle(case):
    B, H, n, d, causal, scale = case
    log(f"topn mass {case}")
    inp = make_inputs(B, H, n, d, rank=8, noise="t3", seed=n + d)
    q, k, _ = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    sc = float(np.float32(scale))
    for mass in (0.5, 0.9, 0.99, 1.0):
        got = had.topn_mass(qb, kb, d, scale, mass, causal).cpu().numpy().astype(np.int64)
        for b in range(B):
            for h in range(H):
                S = oracle.logits(oracle.binarize(inp["q"][b, h]), oracle.binarize(inp["k"][b, h]))
                check_topn_mass(got[b * H + h], S, sc, mass, causal, where=f"slice {(b, h)}")


# ------------------------------------------------------- sigma calibration
def test_sigma_calibration_over_batches():
    """Running calibration over several minibatches equals the population
    std of all their elements together; bits are had_pack's."""
    log("sigma calibration")
    rng = np.random.default_rng(77)
    shapes = [(2, 3, 77, 64), (1, 2, 300, 64), (4, 1, 5, 33), (1, 1, 1, 1), (3, 2, 64, 128)]
    xs = [(rng.standard_normal(sh) * 1.7 + 0.4).astype(np.float32) for sh in shapes]
    state = had.sigma_state()
    assert float(had.sigma_from_state(state).item()) == 0.0
    for x in xs:
        bits = had.pack_calibrate(torch.from_numpy(x).cuda(), state)
        assert np.array_equal(bits_np(bits), oracle.pack_bits(oracle.binarize(x)))
    sig = float(had.sigma_from_state(state).item())
    ref = oracle.sigma(np.concatenate([x.reshape(-1) for x in xs]))
    assert abs(sig - ref) <= 1e-6 * ref
    again = had.sigma_state()
    for x in xs:
        had.pack_calibrate(torch.from_numpy(x).cuda(), again)
    torch.cuda.synchronize()
    assert torch.equal(state, again)
    assert float(state[0].item()) == sum(x.size for x in xs)
