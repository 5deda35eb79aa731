"""GPU parity of had_decode (new query rows against a key/value cache)
through the C ABI, against the CPU oracle's decode(); had_decode_forward
(float32 new rows, sign words built inside the first launch) must equal
had_pack + had_decode bit for bit.

Cache rows past n_k hold large finite garbage so that a read of an unused
row shows up in the outputs.  Outputs must be within 1e-5 * sum(p|V|) (fp32
V) or 2e-3 * max|V| (bf16 V, max over the valid cache).  Every case prints
its name, shape and seed first.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_had_amd as had
from had_workloads import DECODE_WORKLOADS, decode_inputs, make_inputs
from parity_util import check_out, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()


CASES = [
    # B, H, n_q, n_k, k_stride, d, topn, q_pos0, causal, v dtype, scale
    (1, 1, 1, 16384, 16384, 128, 2048, 16383, True, "bf16", 1 / np.sqrt(128)),
    (2, 3, 4, 300, 320, 64, 37, 296, True, "bf16", 0.125),
    (1, 2, 16, 1000, 1000, 64, 100, 0, False, "f32", 0.2),
    (1, 1, 64, 5000, 5000, 5, 50, 4936, True, "bf16", 0.9),   # d = 5: ties everywhere
    (1, 1, 3, 1, 8, 256, 4, 0, True, "f32", 1 / 16),          # one cached key
    (2, 2, 5, 4097, 4100, 96, 512, 3000, True, "bf16", 0.1),  # rows see a prefix
    (1, 2, 2, 70000, 70000, 64, 256, 69998, True, "bf16", 0.125),  # n_k > 65536
    (1, 1, 2, 50, 50, 64, 80, 48, True, "bf16", 0.125),       # N > visible
    (1, 1, 2, 100, 100, 64, 10, 500, True, "f32", 0.3),       # every key visible
    (3, 1, 17, 777, 800, 33, 20, 760, False, "bf16", 0.25),   # two row batches
    (1, 8, 64, 1000, 1000, 64, 100, 936, True, "bf16", 0.125),    # 2 splits of 512 keys, recomputed
    (1, 64, 1, 16384, 16384, 32, 1024, 16383, True, "bf16", 0.18),  # full cache, single launch, 4 parts
    (1, 32, 1, 16384, 16384, 32, 1024, 16383, True, "bf16", 0.18),  # full cache, single launch, 4 parts
    # hundreds of (slice, row) pairs: the single launch with one work-group per pair
    # (more than 16 new rows per slice, or caches above 16384 keys, take the split launches)
    (1, 520, 1, 3000, 3000, 32, 300, 2999, True, "bf16", 0.25),
    (2, 300, 2, 2048, 2048, 64, 256, 2046, True, "f32", 0.125),
    (1, 600, 1, 1000, 1024, 5, 40, 999, False, "bf16", 0.9),         # d = 5 ties
    # the single launch's placement by slice (8 slices or more) with several parts and rows:
    (2, 4, 3, 900, 900, 64, 90, 897, True, "bf16", 0.125),           # 8 slices x 3 rows, 4 parts
    (3, 3, 2, 700, 704, 64, 70, 698, True, "f32", 0.2),              # 9 slices: a padded group of 8
]


@pytest.mark.parametrize("case", CASES)
def test_decode_matches_oracle(case):
    B, H, nq, nk, ks, d, topn, p0, causal, vdt, scale = case
    seed = nk + 7 * nq + d
    log(f"decode {case} seed {seed}")
    total = max(nk, p0 + nq)
    inp = make_inputs(B, H, total, d, v_dtype=vdt, rank=8, noise="t3", seed=seed)
    rows = np.arange(p0, p0 + nq) % total
    qn = np.ascontiguousarray(inp["q"][:, :, rows])
    kc = np.full((B, H, ks, d), 3.0e5, dtype=np.float32)
    kc[:, :, :nk] = inp["k"][:, :, :nk]
    kc[:, :, nk:, ::2] = -3.0e5
    vc = np.full((B, H, ks, d), 1.0e6, dtype=np.float32)
    vc[:, :, :nk] = inp["v"][:, :, :nk]
    q_t = torch.from_numpy(qn).cuda()
    k_t = torch.from_numpy(kc).cuda()
    v_t = torch.from_numpy(vc)
    v_t = (v_t.to(torch.bfloat16) if vdt == "bf16" else v_t).cuda()
    qb, _ = had.pack(q_t, with_sigma=False)
    kb, _ = had.pack(k_t, with_sigma=False)
    out_t = had.decode(qb, kb, v_t, topn, scale, q_pos0=p0, causal=causal, n_k=nk)
    fwd_t = had.decode_forward(q_t, kb, v_t, topn, scale, q_pos0=p0, causal=causal, n_k=nk)
    torch.cuda.synchronize()
    assert torch.equal(out_t, fwd_t), "decode_forward differs from pack + decode"
    out = out_t.cpu().numpy()
    vvalid = inp["v"][:, :, :nk]
    for b in range(B):
        for h in range(H):
            r = oracle.decode(qn[b, h], inp["k"][b, h, :nk], vvalid[b, h], topn, scale,
                              q_pos0=p0, causal=causal)
            check_out(out[b, h], r["out"], r["E"], vvalid, vdt, where=f"slice {(b, h)}")


@pytest.mark.parametrize("nq", [1, 3])
def test_decode_d256_key_opposite_to_every_query_sign(nq):
    """d = 256: a key whose signs all differ from a row's has Hamming distance
    256, which does not fit the per-key distance byte of the few-row path; the
    row's output must still match the oracle (that key is the least similar
    one, weight exp(-2 * scale * 256) relative to an equal key)."""
    B, H, nk, d, topn = 1, 2, 600, 256, 599
    log(f"decode d=256 opposite key nq={nq}")
    inp = make_inputs(B, H, nk, d, v_dtype="f32", rank=4, noise="normal", seed=256 + nq)
    qn = np.ascontiguousarray(inp["q"][:, :, nk - nq:])
    k = inp["k"].copy()
    for i in range(nq):
        k[:, :, 10 + i] = -np.where(qn[:, :, i] >= 0, 1.0, -1.0) * (1.0 + np.abs(k[:, :, 10 + i]))
        k[:, :, 20 + i] = np.where(qn[:, :, i] >= 0, 1.0, -1.0)
    kb, _ = had.pack(torch.from_numpy(k).cuda(), with_sigma=False)
    v = torch.from_numpy(inp["v"]).cuda()
    for scale in (1e-3, 0.01):
        out = had.decode_forward(torch.from_numpy(qn).cuda(), kb, v, topn, scale, q_pos0=nk - nq,
                                 causal=True).cpu().numpy()
        for h in range(H):
            r = oracle.decode(qn[0, h], k[0, h], inp["v"][0, h], topn, scale, q_pos0=nk - nq, causal=True)
            assert (r["S"][np.arange(nq), 10 + np.arange(nq)] == -d).all()
            check_out(out[0, h], r["out"], r["E"], inp["v"], "f32", where=f"head {h} scale {scale}")


@pytest.mark.parametrize("case", [(2, 3, 300, 64, 37, True, "f32"), (1, 2, 257, 128, 40, False, "bf16"),
                                  (1, 1, 97, 5, 10, True, "f32"), (4, 4, 1024, 64, 256, False, "f32")])
def test_decode_of_the_whole_sequence_is_the_attention(case):
    """n_q = n_k = n and q_pos0 = 0: had_decode gathers the kept V rows of every
    row of the sequence, which is had_attention's computation in another form;
    both match the oracle (fp32 V: 1e-5 * E, far below a tie swap)."""
    B, H, n, d, topn, causal, vdt = case
    log(f"decode whole sequence {case}")
    inp = make_inputs(B, H, n, d, v_dtype=vdt, rank=8, noise="t3", seed=3 * n + d)
    q_t = torch.from_numpy(inp["q"]).cuda()
    k_t = torch.from_numpy(inp["k"]).cuda()
    v_t = torch.from_numpy(inp["v"])
    v_t = (v_t.to(torch.bfloat16) if vdt == "bf16" else v_t).cuda()
    qb, _ = had.pack(q_t, with_sigma=False)
    kb, _ = had.pack(k_t, with_sigma=False)
    scale = 1.0 / np.sqrt(d)
    out = had.decode(qb, kb, v_t, topn, scale, q_pos0=0, causal=causal).cpu().numpy()
    att = had.attention(qb, kb, v_t, topn, scale, causal).cpu().numpy()
    for b in range(B):
        for h in range(H):
            rows = np.arange(n) if n <= 300 else np.unique(np.r_[0, n - 1, np.arange(0, n, 37)])
            r = oracle.forward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], topn, scale,
                               causal=causal, rows=rows)
            check_out(out[b, h][rows], r["out"], r["E"], inp["v"], vdt, where=f"decode slice {(b, h)}")
            check_out(att[b, h][rows], r["out"], r["E"], inp["v"], vdt, where=f"attention slice {(b, h)}")


def test_decode_is_deterministic_and_reuses_its_workspace():
    B, H, nq, nk, d = 2, 4, 8, 3000, 64
    log(f"decode determinism {(B, H, nq, nk, d)}")
    inp = make_inputs(B, H, nk, d, v_dtype="bf16", rank=8, noise="t3", seed=5)
    q_t = torch.from_numpy(np.ascontiguousarray(inp["q"][:, :, -nq:])).cuda()
    k_t = torch.from_numpy(inp["k"]).cuda()
    v_t = torch.from_numpy(inp["v"]).to(torch.bfloat16).cuda()
    qb, _ = had.pack(q_t, with_sigma=False)
    kb, _ = had.pack(k_t, with_sigma=False)
    ws = torch.empty(had.decode_workspace_bytes(B, H, nq, nk, nk, d), dtype=torch.uint8, device="cuda")
    o1 = had.decode(qb, kb, v_t, 300, 0.125, q_pos0=nk - nq, workspace=ws).clone()
    o2 = had.decode(qb, kb, v_t, 300, 0.125, q_pos0=nk - nq, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("name", sorted(DECODE_WORKLOADS))
def test_decode_workload_sampled(name):
    """The decode workloads at full size, in the launch configuration bench.py
    times (both take the single launch: 128 rows x 16384 keys with two
    work-groups per row, 2048 rows with one), checked against the oracle on
    sampled (batch, head) slices, all new rows of each."""
    w = DECODE_WORKLOADS[name]
    log(f"decode workload {name}: B={w.batch} H={w.heads} n_k={w.n_k} n_q={w.n_q} d={w.dim} "
        f"N={w.topn} seed={w.seed}")
    inp = decode_inputs(w)
    qn = torch.from_numpy(inp["q_new"]).cuda()
    kc = torch.from_numpy(inp["k"]).cuda()
    v_t = torch.from_numpy(inp["v"])
    v_t = (v_t.to(torch.bfloat16) if w.v_dtype == "bf16" else v_t).cuda()
    qb, _ = had.pack(qn, with_sigma=False)
    kb, _ = had.pack(kc, with_sigma=False)
    del kc
    ws = torch.empty(had.decode_workspace_bytes(w.batch, w.heads, w.n_q, w.n_k, w.n_k, w.dim),
                     dtype=torch.uint8, device="cuda")
    out_t = had.decode_forward(qn, kb, v_t, w.topn, w.scale, q_pos0=w.q_pos0, causal=w.causal,
                               workspace=ws)
    ref_t = had.decode(qb, kb, v_t, w.topn, w.scale, q_pos0=w.q_pos0, causal=w.causal)
    torch.cuda.synchronize()
    assert torch.equal(out_t, ref_t), "decode_forward differs from pack + decode"
    out = out_t.cpu().numpy()
    log("  gpu done")
    BH = w.batch * w.heads
    rng = np.random.default_rng(66)
    for bh in np.unique(np.r_[0, BH - 1, rng.integers(0, BH, 4)]):
        b, h = divmod(int(bh), w.heads)
        r = oracle.decode(inp["q_new"][b, h], inp["k"][b, h], inp["v"][b, h], w.topn, w.scale,
                          q_pos0=w.q_pos0, causal=w.causal)
        check_out(out[b, h], r["out"], r["E"], inp["v"], w.v_dtype, where=f"{name} slice {(b, h)}")
