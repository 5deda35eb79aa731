"""CPU: the selection scheme of the soft forward's GPU kernel, restated in
Python, against a stable sort.

The kernel keeps, per row, exactly the N_i largest float32 logits, the lower
key index first among equal ones, by a radix select over the composite
(order-preserving bits of the logit, inverted key index): four levels over the
bytes of the logit's order key, then two over 5-bit digits of the key index,
each finding the digit that holds the row's remaining quota.  A row is
resolved as soon as its quota takes a whole bin (its threshold becomes that
bin's lowest composite); keys the row does not see get key 0, below every
visible key.  This test restates those steps (not the kernel's code) and
checks that they select exactly what a stable descending sort selects, on
random, heavily tied and signed-zero logits, with and without a visibility
limit.  It pins the scheme; the GPU parity tests pin the kernel.
"""

import numpy as np
import pytest


def order_key(s):
    u = (np.asarray(s, dtype=np.float32) + np.float32(0)).view(np.uint32).astype(np.int64)
    return np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000).astype(np.int64)


def scheme_select(s, lim, topn):
    """Kept key indices of one row (keys j < lim visible) by the radix scheme."""
    n = len(s)
    j = np.arange(n)
    k = np.where(j < lim, order_key(s), 0)
    need = min(topn, lim)
    if need == lim:  # every visible key kept: threshold key 1
        kst, jst, done = 1, 2**31 - 1, True
    else:
        kst, jst, done = 0, 0, False
    for level in range(6):
        if done:
            break
        if level == 0:
            match, digit = np.ones(n, bool), k >> 24
        elif level < 4:
            match, digit = (k >> (32 - 8 * level)) == kst, (k >> (24 - 8 * level)) & 255
        elif level == 4:
            match, digit = k == kst, 31 - (j >> 5)
        else:
            match, digit = (k == kst) & ((j >> 5) == jst), 31 - (j & 31)
        hist = np.bincount(digit[match], minlength=256)
        above = 0
        for t in range(255, -1, -1):  # the digit holding the remaining quota
            if above + hist[t] >= need:
                break
            above += hist[t]
        rem = need - above
        whole = rem == hist[t] or level == 5
        if level < 4:
            key = t if level == 0 else (kst << 8) | t
            kst = key << (24 - 8 * level) if whole else key
            if whole:
                jst = 2**31 - 1
        elif level == 4:
            jst = 32 * (31 - t) + 31 if whole else 31 - t
        else:
            jst = 32 * jst + (31 - t)
        need = 0 if whole else rem
        done = whole
    keep = (k > kst) | ((k == kst) & (j <= jst))
    return np.nonzero(keep)[0]


def stable_top(s, lim, topn):
    sv = np.asarray(s[:lim], dtype=np.float64)
    return np.sort(np.argsort(-sv, kind="stable")[: min(topn, lim)])


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "narrow"])
def test_scheme_equals_a_stable_sort(kind):
    rng = np.random.default_rng({"normal": 1, "ties": 2, "zeros": 3, "narrow": 4}[kind])
    for trial in range(600):
        n = int(rng.integers(1, 1025))
        topn = int(rng.integers(1, 300))
        if kind == "normal":
            s = rng.standard_normal(n).astype(np.float32) * 4
        elif kind == "ties":  # integer logits: the sign limit, many equal values
            s = rng.integers(-8, 9, n).astype(np.float32)
        elif kind == "zeros":  # +0 and -0 are equal logits
            s = np.where(rng.random(n) < 0.5, np.float32(-0.0), np.float32(0.0))
            s[rng.random(n) < 0.1] = np.float32(1.0)
        else:  # values that share their top key bytes
            s = (3.0 + rng.standard_normal(n) * 1e-4).astype(np.float32)
        lim = int(rng.integers(1, n + 1)) if trial % 2 else n
        got = scheme_select(s, lim, topn)
        want = stable_top(s, lim, topn)
        assert np.array_equal(got, want), (kind, trial, n, topn, lim)


def test_scheme_keeps_exactly_n_and_only_visible_keys():
    rng = np.random.default_rng(7)
    for lim in (1, 2, 31, 32, 33, 500):
        s = rng.standard_normal(600).astype(np.float32)
        got = scheme_select(s, lim, 40)
        assert len(got) == min(40, lim) and got.max() < lim
