"""Helpers shared by the GPU parity tests: they move data, call the oracle or
the GPU library, and compare (tolerances, and for the top-N mass the float64
prefix sums that show a decision lies within rounding)."""

import sys

import numpy as np
import torch

import oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp, device="cuda"):
    q = torch.from_numpy(inp["q"]).to(device)
    k = torch.from_numpy(inp["k"]).to(device)
    v = torch.from_numpy(inp["v"])
    v = (v.to(torch.bfloat16) if inp["v_dtype"] == "bf16" else v).to(device)
    return q, k, v


def bits_np(t):
    return t.cpu().numpy().view(np.uint32)


def oracle_head(inp, b, h, topn, scale, causal, rows=None):
    return oracle.forward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], topn, scale,
                          causal=causal, rows=rows)


def check_out(got, ref, E, v_all, v_dtype, where=""):
    """Tolerance: fp32 V -> |o - o*| <= 1e-5 * E (E = sum p |V|) + 1e-30;
    bf16 V -> |o - o*| <= 2e-3 * max|V| (max over the whole V tensor)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    if v_dtype == "f32":
        tol = 1e-5 * E + 1e-30
    else:
        tol = 2e-3 * float(np.max(np.abs(v_all)))
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{where}: {int(bad.sum())} outputs outside tolerance; first at {tuple(i)}: "
            f"got {got[tuple(i)]!r} want {ref[tuple(i)]!r} tol {np.broadcast_to(tol, err.shape)[tuple(i)]!r}")
    return float(err.max()) if err.size else 0.0


def check_topn_mass(got, S, scale, mass, causal, where=""):
    """got [rows] against oracle.topn_mass(S, scale, mass, causal); a row may
    differ by one only where a prefix sum lies within 1e-12 of mass (a
    decision inside the rounding of the float64 sums)."""
    want = oracle.topn_mass(S, scale, mass, causal)
    got = np.asarray(got, dtype=np.int64)
    n = S.shape[1]
    for r in np.nonzero(got != want)[0]:
        nv = oracle.visible_count(int(r), n, causal)
        z = scale * S[r, :nv].astype(np.float64)
        e = np.exp(z - z.max())
        c = np.cumsum(np.sort(e / e.sum())[::-1])
        margin = min(abs(c[want[r] - 1] - mass), abs(c[want[r] - 2] - mass) if want[r] >= 2 else 1.0)
        assert abs(int(got[r]) - int(want[r])) == 1 and margin < 1e-12, \
            f"{where}: mass {mass} row {r}: got {got[r]} want {want[r]}"

