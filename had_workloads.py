"""Seeded synthetic inputs for HAD attention (shared by tests, smoke and bench).

This module only draws random numbers.  It holds none of the method's
arithmetic: no sign, no packing, no logits, no selection, no softmax.  Both the
CPU oracle and the GPU library consume exactly the arrays produced here.

The pages evaluate on GLUE (BERT), ImageNet (DeiT) and QuALITY (T5), none of
which is available; these generators stand in for them with the same tensor
shapes.  Q and K are Gaussian, following the pages' own modelling assumption
that keys and queries are roughly Gaussian (Pith review, "Assumptions & free
parameters"), plus a low-rank component shared by Q and K so that the top-N
sets depend on the query, and, for the long-context shapes, heavy-tailed
(Student-t, 3 degrees of freedom) per-element noise.

Recipe for one (batch, head) slice with rank r (r = 0 means plain iid):
    A  ~ N(0, 1/r)  of shape (r, d), shared by Q and K of the slice
    Cq ~ N(0, 1)    (n, r);  Eq ~ noise (n, d);  Q = Eq + 0.5 * Cq @ A
    Ck ~ N(0, 1)    (n, r);  Ek ~ noise (n, d);  K = Ek + 0.5 * Ck @ A
drawn slice by slice in (b, h) order from numpy default_rng(seed), then V ~
N(0, 1) of shape (B, H, n, d) in one draw.  Q and K are rounded to float32,
V to float32 or to bfloat16 (round to nearest even).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq: int
    dim: int
    topn: int
    causal: bool
    v_dtype: str  # "f32" or "bf16"
    rank: int  # 0 => iid N(0,1) Q and K
    noise: str  # "normal" or "t3"
    seed: int
    note: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        return self.batch * self.heads * self.seq

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.dim))


# Shapes of the pages' encoder, ViT and long-context workloads.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("single-head-n128", 1, 1, 128, 64, 32, False, "f32", 0, "normal", 1,
                 "one head, iid N(0,1) Q/K/V, fp32 V"),
        Workload("bert-base-n128", 32, 12, 128, 64, 32, False, "bf16", 4, "normal", 2,
                 "BERT-base encoder attention shape"),
        Workload("deit-s-n197", 64, 6, 197, 64, 50, False, "bf16", 8, "normal", 3,
                 "DeiT-S ViT attention shape (196 patches + CLS)"),
        Workload("t5-base-n1024", 8, 12, 1024, 64, 256, False, "bf16", 8, "t3", 4,
                 "T5-base long-document encoder shape, N = n/4"),
        Workload("causal-n16384", 1, 32, 16384, 128, 2048, True, "bf16", 8, "t3", 5,
                 "long-context causal decoder stress, N = n/8"),
    ]
}

HEADLINE = "t5-base-n1024"


@dataclass(frozen=True)
class DecodeWorkload:
    """New query rows at the end of a sequence against its key/value cache."""

    name: str
    batch: int
    heads: int
    n_k: int  # cached tokens (the new rows are the last n_q of them)
    n_q: int
    dim: int
    topn: int
    causal: bool
    v_dtype: str
    rank: int
    noise: str
    seed: int
    note: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        return self.batch * self.heads * self.n_q

    @property
    def q_pos0(self) -> int:
        return self.n_k - self.n_q

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.dim))


# Decoding shapes next to the long-context causal workload: the same head
# size and N = n/8, one new token (or a block of 16 being verified) per
# sequence.
DECODE_WORKLOADS = {
    w.name: w
    for w in [
        DecodeWorkload("decode-n16384", 4, 32, 16384, 1, 128, 2048, True, "bf16", 8, "t3", 6,
                       "one new token per sequence against a 16384-token cache"),
        DecodeWorkload("decode-n16384-q16", 4, 32, 16384, 16, 128, 2048, True, "bf16", 8, "t3", 7,
                       "16 new tokens per sequence against a 16384-token cache"),
    ]
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint32(0x7FC00000)
    return r.view(np.float32).reshape(a.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly representable in bf16."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _noise(rng, kind: str, shape):
    if kind == "normal":
        return rng.standard_normal(shape)
    if kind == "t3":
        return rng.standard_t(3.0, shape)
    raise ValueError(f"unknown noise kind {kind!r}")


def make_qk(batch, heads, seq, dim, rank, noise, rng):
    q = np.empty((batch, heads, seq, dim), dtype=np.float32)
    k = np.empty((batch, heads, seq, dim), dtype=np.float32)
    for b in range(batch):
        for h in range(heads):
            if rank > 0:
                a = rng.standard_normal((rank, dim)) / np.sqrt(rank)
                cq = rng.standard_normal((seq, rank))
                q[b, h] = _noise(rng, noise, (seq, dim)) + 0.5 * (cq @ a)
                ck = rng.standard_normal((seq, rank))
                k[b, h] = _noise(rng, noise, (seq, dim)) + 0.5 * (ck @ a)
            else:
                q[b, h] = _noise(rng, noise, (seq, dim))
                k[b, h] = _noise(rng, noise, (seq, dim))
    return q, k


def make_inputs(batch, heads, seq, dim, *, v_dtype="bf16", rank=8, noise="normal", seed=0):
    """Q, K (float32) and V (float32 holding bf16-exact values when v_dtype='bf16')."""
    rng = np.random.default_rng(seed)
    q, k = make_qk(batch, heads, seq, dim, rank, noise, rng)
    v = rng.standard_normal((batch, heads, seq, dim)).astype(np.float32)
    if v_dtype == "bf16":
        v = round_to_bf16(v)
    elif v_dtype != "f32":
        raise ValueError(f"unknown v_dtype {v_dtype!r}")
    return {"q": q, "k": k, "v": v, "v_dtype": v_dtype}


def workload_inputs(w: Workload):
    return make_inputs(w.batch, w.heads, w.seq, w.dim, v_dtype=w.v_dtype,
                       rank=w.rank, noise=w.noise, seed=w.seed)


def decode_inputs(w: DecodeWorkload):
    """The whole sequence (recipe above); the new rows' queries are its last n_q rows."""
    inp = make_inputs(w.batch, w.heads, w.n_k, w.dim, v_dtype=w.v_dtype, rank=w.rank,
                      noise=w.noise, seed=w.seed)
    inp["q_new"] = np.ascontiguousarray(inp["q"][:, :, w.n_k - w.n_q:])
    return inp
