"""GPU: libhad_popcount.so, the build whose attention kernel takes its logit
tiles from XOR + popcount on the vector ALU, gives exactly what libhad.so (the
int8 matrix-core logit stage) gives.  Both tiles hold the same integers
cin + k*(2h - d), so logits, kept sets and outputs must be bit-identical; the
popcount library exists to measure the logit-stage choice against.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import sparse_attention_had_amd as had
from had_workloads import make_inputs
from parity_util import log

pytestmark = pytest.mark.gpu

# B, H, n, d, topn, causal, v dtype: tile and word boundaries, both masks, both V types
CASES = [
    (1, 2, 128, 64, 32, False, "bf16"),
    (2, 1, 200, 64, 50, True, "bf16"),
    (1, 1, 1024, 64, 256, False, "bf16"),
    (1, 2, 300, 33, 40, True, "f32"),
    (1, 1, 257, 128, 64, False, "bf16"),
    (1, 1, 100, 256, 10, True, "bf16"),
    (1, 1, 17, 5, 3, False, "f32"),
]


@pytest.fixture(scope="module")
def poplib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()
    path = os.path.join(os.path.dirname(os.path.abspath(had.__file__)), "libhad_popcount.so")
    assert os.path.exists(path), f"{path} not built (python -m sparse_attention_had_amd.build)"
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.had_attention.argtypes = [P, P, P, I, had.Shape, I64, ctypes.c_float, I, P, P]
    lib.had_attention.restype = I
    lib.had_select.argtypes = [P, P, had.Shape, I64, I, I64, I64, P, P]
    lib.had_select.restype = I
    lib.had_logits.argtypes = [P, P, had.Shape, I64, I64, I64, I64, P, P]
    lib.had_logits.restype = I
    return lib


@pytest.mark.parametrize("case", CASES)
def test_popcount_logit_build_matches(poplib, case):
    B, H, n, d, topn, causal, vdt = case
    log(f"popcount logits {case}")
    scale = float(1.0 / np.sqrt(d))
    inp = make_inputs(B, H, n, d, rank=min(4, d), noise="t3", seed=11 * n + d, v_dtype=vdt)
    q = torch.from_numpy(inp["q"]).cuda()
    k = torch.from_numpy(inp["k"]).cuda()
    v = torch.from_numpy(inp["v"])
    v = (v.to(torch.bfloat16) if vdt == "bf16" else v).cuda()
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    out = had.attention(qb, kb, v, topn, scale, causal)
    idx = had.select(qb, kb, d, topn, causal)
    lg = had.logits(qb, kb, d)
    stream = torch.cuda.current_stream().cuda_stream
    shape = had.Shape(B, H, n, d)
    out2 = torch.empty_like(out)
    idx2 = torch.empty_like(idx)
    lg2 = torch.empty_like(lg)
    assert poplib.had_attention(qb.data_ptr(), kb.data_ptr(), v.data_ptr(),
                                had.HAD_BF16 if vdt == "bf16" else had.HAD_F32, shape, topn, scale, int(causal),
                                out2.data_ptr(), stream) == 0
    assert poplib.had_select(qb.data_ptr(), kb.data_ptr(), shape, topn, int(causal), 0, B * H,
                             idx2.data_ptr(), stream) == 0
    assert poplib.had_logits(qb.data_ptr(), kb.data_ptr(), shape, 0, B * H, 0, n,
                             lg2.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(lg, lg2), f"{case}: logits differ"
    assert torch.equal(idx, idx2), f"{case}: kept sets differ"
    assert torch.equal(out, out2), f"{case}: outputs differ"
