"""CPU: the host logic of bench.py.  The work models that turn a measured
launch time into a roofline fraction are checked against counts written out
by hand for the headline workload and against enumeration over rows on small
shapes; the HBM traffic record is used only while the kernel sources are the
ones it was taken on; the headline metric string is the one its numbers are
quoted under; more than one GPU is refused with a message.
"""

import os
import subprocess
import sys
import types

import numpy as np

import pytest

import bench
from had_workloads import DECODE_WORKLOADS, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_work_model_by_hand():
    # 8 x 12 slices, n = 1024, d = 64 (W = 2 words), N = 256, bf16 V, not causal
    m = bench.work_model(WORKLOADS["t5-base-n1024"])
    slices, n, d, N = 96, 1024, 64, 256
    assert m["visible_pairs"] == slices * n * n == 100_663_296
    assert m["kept"] == slices * n * N == 25_165_824
    # XOR + popcount per word (2 x 2) and histogram + compaction (2) per pair,
    # weight + index per kept pair (2)
    assert m["int_ops"] == 100_663_296 * 6 + 25_165_824 * 2
    assert m["flops"] == 2 * 25_165_824 * d
    assert m["lane_ops"] == m["int_ops"] + m["flops"] / 4
    # bits of Q and K (2 words each), bf16 V, fp32 out
    assert m["hbm_bytes"] == slices * n * (2 * 2 * 4 + d * 2 + d * 4) == 39_321_600


@pytest.mark.parametrize("n,N,causal,d,vdt", [(1, 1, False, 1, "f32"), (7, 3, True, 33, "bf16"),
                                              (16, 20, True, 64, "f32"), (50, 8, False, 100, "bf16"),
                                              (129, 128, True, 256, "bf16")])
def test_work_model_against_enumeration(n, N, causal, d, vdt):
    w = types.SimpleNamespace(batch=2, heads=3, seq=n, dim=d, topn=N, causal=causal, v_dtype=vdt)
    W = -(-d // 32)
    vis = kept = 0
    for i in range(n):
        v = i + 1 if causal else n
        vis += v
        kept += min(N, v)
    m = bench.work_model(w)
    assert m["visible_pairs"] == 6 * vis
    assert m["kept"] == 6 * kept
    assert m["int_ops"] == 6 * (vis * (2 * W + 2) + 2 * kept)
    assert m["flops"] == 6 * 2 * kept * d
    assert m["hbm_bytes"] == 6 * n * (2 * W * 4 + d * (2 if vdt == "bf16" else 4) + d * 4)


def test_decode_model_by_hand():
    w = DECODE_WORKLOADS["decode-n16384"]
    # 4 x 32 slices, one new row seeing all 16384 keys, d = 128 (4 words), N = 2048, bf16 V
    slices, nk, d, N = 128, 16384, 128, 2048
    assert (w.batch * w.heads, w.n_k, w.dim, w.topn, w.n_q) == (slices, nk, d, N, 1)
    key_words = slices * nk * 4 * 4
    kept_rows = slices * N * d * 2
    m = bench.decode_model(w, fp32_rows=True)
    assert m["kept"] == slices * N
    assert m["hbm_bytes"] == key_words + kept_rows + slices * (d * 4 + d * 4) == 100_794_368
    # with packed new rows: their words instead of float32 rows
    assert bench.decode_model(w)["hbm_bytes"] == key_words + kept_rows + slices * (4 * 4 + d * 4)


def test_traffic_record_only_on_matching_sources(monkeypatch):
    import sparse_attention_had_amd.profiling as prof

    got = bench.traffic_for("t5-base-n1024")
    assert got is not None and got > 0, "the committed traffic record is stale for these kernel sources"
    monkeypatch.setattr(prof, "source_hash", lambda: "0" * 16)
    assert bench.traffic_for("t5-base-n1024") is None
    assert bench.traffic_for("no-such-workload") is None


def test_headline_metric_string():
    w = WORKLOADS["t5-base-n1024"]
    assert bench.METRIC.format(n=w.seq, topn=w.topn) == \
        "query rows/sec of HAD attention at n=1024,N=256; % of HBM/VALU roofline"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_mfma_model_at_the_headline_workload():
    """384 matrix-core instructions per wave at t5-base-n1024 (the SQ_INSTS_MFMA
    count the counter pass reads): 32 int8 logit tiles of 2 instructions in each
    pass, and 8 bf16 products (hi and lo weights, 2 K-steps, 2 feature tiles) per
    pass-2 tile."""
    w = WORKLOADS["t5-base-n1024"]
    m = bench.mfma_model(w)
    waves = 96 * (1024 // 32)
    assert m["int8_instr"] == waves * (32 * 2 + 32 * 2)
    assert m["bf16_instr"] == waves * 32 * 8
    assert (m["int8_instr"] + m["bf16_instr"]) / waves == 384
    assert m["fp32_instr"] == 0
    r = bench.mfma_roofline(w, 51.6e-6)
    busy = m["int8_ops"] / 5.0e15 + m["bf16_flops"] / 2.5e15
    assert abs(r["frac"] - busy / 51.6e-6) < 1e-12
    assert 0.25 < r["frac"] < 0.35


def test_mfma_model_causal_counts_only_visible_chunks():
    # one slice, n = 256, causal, d = 64: work-group t (128 rows) sees keys [0, 128(t+1))
    w = types.SimpleNamespace(batch=1, heads=1, seq=256, dim=64, topn=16, causal=True, v_dtype="bf16")
    m = bench.mfma_model(w)
    int8 = bf16 = 0
    for t in range(2):
        kend = 128 * (t + 1)
        nchunk = (((kend + 1) // 2 + 15) & ~15) // 16
        for wv in range(4):
            wch = min(nchunk, (min(256, 128 * t + 32 * wv + 32) + 15) // 16)
            p2 = -(-wch // 4) * 4
            int8 += 2 * (wch + p2)
            bf16 += 8 * p2
    assert (m["int8_instr"], m["bf16_instr"]) == (int8, bf16)


def test_host_workers_and_baseline_record(monkeypatch):
    assert 1 <= bench.host_workers() <= 16
    w = types.SimpleNamespace(batch=1, heads=2, seq=40, dim=8, topn=5, causal=False, scale=0.3)
    rng = np.random.default_rng(0)
    inp = {"q": rng.standard_normal((1, 2, 40, 8)), "k": rng.standard_normal((1, 2, 40, 8)),
           "v": rng.standard_normal((1, 2, 40, 8))}
    monkeypatch.setattr(bench, "host_workers", lambda: 1)
    rec = bench.cpu_baseline(w, inp, 0.5)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["workers"] == 1
    assert rec["value"] > 0 and rec["os_cpu_count"] == os.cpu_count()


def test_forked_workers_run_every_slice(monkeypatch):
    w = types.SimpleNamespace(batch=2, heads=3, seq=30, dim=8, topn=4, causal=True, scale=0.3)
    rng = np.random.default_rng(1)
    inp = {x: rng.standard_normal((2, 3, 30, 8)) for x in ("q", "k", "v")}
    monkeypatch.setattr(bench, "host_workers", lambda: 2)
    rec = bench.cpu_baseline(w, inp, 30.0, 30.0)
    assert rec["cores"] == 2 and rec["workers"] == 2
    assert rec["sample"].startswith("6 of 6 ") and rec["single_core"]["sample"].startswith("6 of 6 ")


def test_backward_model_by_hand():
    w = WORKLOADS["t5-base-n1024"]
    m = bench.backward_model(w)
    assert m["kept"] == 96 * 1024 * 256
    assert m["flops"] == 8 * 64 * m["kept"]
    assert m["mfma_fp32_flops"] == 10 * 64 * 96 * 1024 * 1024  # every 32 x 32 tile is visible
    c = bench.backward_model(types.SimpleNamespace(batch=1, heads=1, seq=64, dim=32, topn=8,
                                                    causal=True, v_dtype="bf16"))
    assert c["mfma_fp32_flops"] == 10 * 32 * 3 * 1024  # tiles (0,0), (1,0), (1,1)


def test_soft_model_by_hand():
    w = WORKLOADS["t5-base-n1024"]
    m = bench.soft_model(w)
    pairs, kept = 96 * 1024 * 1024, 96 * 1024 * 256
    assert m["flops"] == 2 * 64 * (pairs + kept)
    assert m["mfma_fp32_flops"] == 4 * 64 * pairs  # logits and V product over every tile
    # Q and K read (4 B), their 64-feature soft rows written and read (2 x 4 B each), V bf16, out fp32
    assert m["hbm_bytes"] == 96 * 1024 * (2 * 64 * 4 + 4 * 64 * 4 + 64 * 2 + 64 * 4)
    c = bench.soft_model(types.SimpleNamespace(batch=1, heads=1, seq=64, dim=40, topn=8,
                                                causal=True, v_dtype="f32"))
    assert c["mfma_fp32_flops"] == 4 * 64 * 3 * 1024  # 40 features padded to 64; 3 visible tiles
