"""GPU: the attend path's own kept sets at the full sizes of the long workloads.

With bf16 V the output tolerance (2e-3 * max|V|) is larger than what one
wrong tie choice moves an output by (the threshold key's weight w_T / Z is
about 2e-3 at t5-base-n1024 and 2e-4 at causal-n16384, times |V_j - V_j'|), so
the workload checks of test_gpu_parity.py cannot see a tie error in the
attention kernel.  These checks can:

* fp32 V with the same Q/K (same generator and seed) at the full shapes:
  the tolerance is 1e-5 * sum(p |V|), hundreds of times below a tie swap;
* bf16 V whose row j is the unit vector of feature j mod d, run through
  had_forward exactly as bench.py times it (bf16 V, rows copied straight into
  LDS): every output is then a sum of kept weights over one residue class of
  keys, V is exact, and the only rounding is the weights' two-term bf16 split
  (relative error < 2^-15) and float32 sums, so the tolerance derived from that
  arithmetic, (2^-14 + (N + d + 2) * 2^-24) * sum(p |V|), sits far below a swap;
* had_select compared on whole heads (every row) against the oracle;
* the same two V variants for the decode workload at its full size.

Every case prints its name, shape and seed first.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_had_amd as had
from had_workloads import DECODE_WORKLOADS, WORKLOADS, make_inputs
from parity_util import bits_np, check_out, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()


def _inputs(w, v_dtype):
    # the workload's own generator and seed; V is drawn after Q and K, so Q and
    # K are those of the workload whatever V's type
    return make_inputs(w.batch, w.heads, w.seq, w.dim, v_dtype=v_dtype, rank=w.rank,
                       noise=w.noise, seed=w.seed)


def _residue_onehot(B, H, n, d):
    """V[b, h, j, c] = 1 if c == j mod d else 0 (float32 array)."""
    v = np.zeros((B, H, n, d), dtype=np.float32)
    j = np.arange(n)
    v[:, :, j, j % d] = 1.0
    return v


def _sample_rows(n, extra, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, n // 8 - 1, n // 8, n // 2, n - 2, n - 1]
    return np.unique(np.r_[[r for r in fixed if 0 <= r < n], rng.integers(0, n, extra)])


def _check_onehot(got, ref, N, d, where):
    """Tolerance from the arithmetic of the bf16 path with exact one-hot V."""
    E = ref["E"]
    tol = (2.0 ** -14 + (N + d + 2) * 2.0 ** -24) * E + 1e-30
    err = np.abs(np.asarray(got, dtype=np.float64) - ref["out"])
    bad = err > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{where}: {int(bad.sum())} outputs outside tolerance; first at {i}: "
                             f"got {got[i]!r} want {ref['out'][i]!r} tol {tol[i]!r}")
    return float(err.max())


@pytest.mark.parametrize("name,extra", [("t5-base-n1024", 24), ("causal-n16384", 8)])
def test_fp32_v_at_full_size(name, extra):
    w = WORKLOADS[name]
    log(f"fp32 V at full size {name}: B={w.batch} H={w.heads} n={w.seq} d={w.dim} N={w.topn} "
        f"causal={w.causal} seed={w.seed}")
    inp = _inputs(w, "f32")
    q = torch.from_numpy(inp["q"]).cuda()
    k = torch.from_numpy(inp["k"]).cuda()
    v = torch.from_numpy(inp["v"]).cuda()
    out, qb, kb, _, _ = had.forward(q, k, v, w.topn, w.scale, w.causal)
    out = out.cpu().numpy()
    log("  gpu done")
    worst = 0.0
    for bh in range(w.batch * w.heads):
        b, h = divmod(bh, w.heads)
        rows = _sample_rows(w.seq, extra, 1000 + bh)
        r = oracle.forward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], w.topn, w.scale,
                           causal=w.causal, rows=rows)
        worst = max(worst, check_out(out[b, h][rows], r["out"], r["E"], inp["v"], "f32",
                                     where=f"{name} fp32 V slice {bh}"))
    log(f"  max abs error {worst:.3e}")


@pytest.mark.parametrize("name,extra", [("t5-base-n1024", 24), ("causal-n16384", 8)])
def test_onehot_v_in_the_bench_launch(name, extra):
    w = WORKLOADS[name]
    log(f"one-hot residue V, had_forward, bf16 {name}: B={w.batch} H={w.heads} n={w.seq} "
        f"d={w.dim} N={w.topn} causal={w.causal} seed={w.seed}")
    inp = _inputs(w, "bf16")
    vo = _residue_onehot(w.batch, w.heads, w.seq, w.dim)
    q = torch.from_numpy(inp["q"]).cuda()
    k = torch.from_numpy(inp["k"]).cuda()
    v = torch.from_numpy(vo).to(torch.bfloat16).cuda()
    out, _, _, _, _ = had.forward(q, k, v, w.topn, w.scale, w.causal)
    out = out.cpu().numpy()
    log("  gpu done")
    worst = 0.0
    for bh in range(w.batch * w.heads):
        b, h = divmod(bh, w.heads)
        rows = _sample_rows(w.seq, extra, 2000 + bh)
        r = oracle.forward(inp["q"][b, h], inp["k"][b, h], vo[b, h], w.topn, w.scale,
                           causal=w.causal, rows=rows)
        worst = max(worst, _check_onehot(out[b, h][rows], r, w.topn, w.dim,
                                         where=f"{name} one-hot V slice {bh}"))
    log(f"  max abs error {worst:.3e}")


@pytest.mark.parametrize("name,heads", [("t5-base-n1024", (0, 57, 95)), ("causal-n16384", (7,))])
def test_select_on_whole_heads(name, heads):
    """Every row of the named (batch, head) slices, indices bit for bit."""
    w = WORKLOADS[name]
    log(f"select whole heads {name} {heads}: n={w.seq} d={w.dim} N={w.topn} causal={w.causal} "
        f"seed={w.seed}")
    inp = _inputs(w, "bf16")
    q = torch.from_numpy(inp["q"]).cuda()
    k = torch.from_numpy(inp["k"]).cuda()
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    for bh in heads:
        b, h = divmod(bh, w.heads)
        idx = had.select(qb, kb, w.dim, w.topn, w.causal, bh_begin=bh, bh_count=1)[0].cpu().numpy()
        assert np.array_equal(bits_np(qb)[b, h], oracle.pack_bits(oracle.binarize(inp["q"][b, h])))
        bq = oracle.binarize(inp["q"][b, h])
        bk = oracle.binarize(inp["k"][b, h])
        for r0 in range(0, w.seq, 2048):
            rows = np.arange(r0, min(w.seq, r0 + 2048))
            S = oracle.logits(bq[rows], bk)
            ref = oracle.select_topn(S, w.topn, w.causal, row_index=rows)
            got = idx[rows].astype(np.int64)
            if not np.array_equal(got, ref):
                r = int(np.argwhere((got != ref).any(1))[0][0])
                raise AssertionError(f"{name} slice {bh} row {rows[r]}: got {got[r][:8].tolist()}... "
                                     f"want {ref[r][:8].tolist()}...")
        log(f"  slice {bh}: all {w.seq} rows equal")


@pytest.mark.parametrize("variant", ["f32", "onehot"])
def test_decode_workload_kept_sets(variant):
    """decode-n16384 at full size in bench.py's launch configuration
    (had_decode_forward), with fp32 V or with one-hot residue bf16 V."""
    w = DECODE_WORKLOADS["decode-n16384"]
    log(f"decode {w.name} {variant}: B={w.batch} H={w.heads} n_k={w.n_k} n_q={w.n_q} d={w.dim} "
        f"N={w.topn} seed={w.seed}")
    inp = make_inputs(w.batch, w.heads, w.n_k, w.dim, v_dtype="f32", rank=w.rank, noise=w.noise,
                      seed=w.seed)
    qn = np.ascontiguousarray(inp["q"][:, :, w.n_k - w.n_q:])
    if variant == "onehot":
        vnp = _residue_onehot(w.batch, w.heads, w.n_k, w.dim)
        v = torch.from_numpy(vnp).to(torch.bfloat16).cuda()
    else:
        vnp = inp["v"]
        v = torch.from_numpy(vnp).cuda()
    kb, _ = had.pack(torch.from_numpy(inp["k"]).cuda(), with_sigma=False)
    out = had.decode_forward(torch.from_numpy(qn).cuda(), kb, v, w.topn, w.scale, q_pos0=w.q_pos0,
                             causal=w.causal).cpu().numpy()
    log("  gpu done")
    BH = w.batch * w.heads
    rng = np.random.default_rng(77)
    for bh in np.unique(np.r_[0, BH - 1, rng.integers(0, BH, 10)]):
        b, h = divmod(int(bh), w.heads)
        r = oracle.decode(qn[b, h], inp["k"][b, h], vnp[b, h], w.topn, w.scale, q_pos0=w.q_pos0,
                          causal=w.causal)
        if variant == "onehot":
            _check_onehot(out[b, h], r, w.topn, w.dim, where=f"decode one-hot slice {bh}")
        else:
            check_out(out[b, h], r["out"], r["E"], vnp, "f32", where=f"decode fp32 V slice {bh}")
