"""GPU: libhad_fusedq.so, the build whose had_forward packs only K in a launch
of its own and forms Q's sign words inside the attention launch (one sigma
partial pair per wave, sigma_Q finalized by a third small launch), gives what
libhad.so gives: sign words, outputs and sigma_K bit for bit, sigma_Q within
1e-6 relative of the oracle (its float64 partial sums are grouped
differently), and the NaN flag for a NaN in Q.  The build exists to measure
that fusion against had_forward's separate pack launch.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_had_amd as had
from had_workloads import make_inputs
from parity_util import log, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, n, d, topn, causal, v dtype, aligned q
    (1, 2, 128, 64, 32, False, "bf16", True),
    (2, 1, 300, 64, 50, True, "bf16", True),
    (4, 4, 1024, 64, 256, False, "bf16", True),
    (1, 2, 300, 33, 40, True, "f32", True),
    (1, 1, 257, 128, 64, False, "bf16", True),
    (1, 1, 100, 256, 10, True, "bf16", True),
    (1, 2, 96, 64, 16, False, "bf16", False),
]


@pytest.fixture(scope="module")
def fqlib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    had.load_library()
    path = os.path.join(os.path.dirname(os.path.abspath(had.__file__)), "libhad_fusedq.so")
    assert os.path.exists(path), f"{path} not built (python -m sparse_attention_had_amd.build)"
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.had_forward_workspace_bytes.argtypes = [had.Shape]
    lib.had_forward_workspace_bytes.restype = ctypes.c_size_t
    lib.had_forward.argtypes = [P, P, P, I, had.Shape, I64, ctypes.c_float, I, P, P, P, P, P, P,
                                ctypes.c_size_t, P, P]
    lib.had_forward.restype = I
    lib.had_attention.argtypes = [P, P, P, I, had.Shape, I64, ctypes.c_float, I, P, P]
    lib.had_attention.restype = I
    return lib


def _fused_forward(lib, q, k, v, topn, scale, causal, st=None):
    B, H, n, d = q.shape
    W = had.words_per_row(d)
    shape = had.Shape(B, H, n, d)
    qb = torch.empty((B, H, n, W), dtype=torch.int32, device="cuda")
    kb = torch.empty_like(qb)
    out = torch.empty((B, H, n, d), dtype=torch.float32, device="cuda")
    sq = torch.empty(1, dtype=torch.float32, device="cuda")
    sk = torch.empty(1, dtype=torch.float32, device="cuda")
    nb = int(lib.had_forward_workspace_bytes(shape))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    rc = lib.had_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), had._v_dtype(v), shape, topn, scale,
                         int(causal), qb.data_ptr(), kb.data_ptr(), out.data_ptr(), sq.data_ptr(),
                         sk.data_ptr(), ws.data_ptr(), nb, None if st is None else st.data_ptr(),
                         torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    return out, qb, kb, sq, sk


@pytest.mark.parametrize("case", CASES)
def test_fused_q_pack_build_matches(fqlib, case):
    B, H, n, d, topn, causal, vdt, al = case
    log(f"fused q pack {case}")
    scale = float(1.0 / np.sqrt(d))
    inp = make_inputs(B, H, n, d, rank=min(4, d), noise="t3", seed=13 * n + d, v_dtype=vdt)
    q, k, v = to_dev(inp)
    if not al:
        buf = torch.zeros(q.numel() + 1, dtype=torch.float32, device="cuda")
        buf[1:] = q.reshape(-1)
        q = buf[1:].view(q.shape)
    ref = had.forward(q, k, v, topn, scale, causal)
    got = _fused_forward(fqlib, q, k, v, topn, scale, causal)
    torch.cuda.synchronize()
    for a, b, name in zip(got[:3], ref[:3], ("out", "qbits", "kbits")):
        assert torch.equal(a, b), f"{case}: {name} differs"
    assert torch.equal(got[4], ref[4]), "sigma_k differs"
    sq = oracle.sigma(inp["q"])
    assert abs(float(got[3].item()) - sq) <= 1e-6 * sq


def test_fused_q_pack_flags_nan(fqlib):
    log("fused q pack nan")
    inp = make_inputs(1, 2, 100, 64, rank=4, noise="normal", seed=5, v_dtype="bf16")
    q, k, v = to_dev(inp)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    _fused_forward(fqlib, q, k, v, 8, 0.2, False, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    q2 = q.clone()
    q2[0, 1, 17, 5] = float("nan")
    _fused_forward(fqlib, q2, k, v, 8, 0.2, False, st)
    torch.cuda.synchronize()
    assert int(st.item()) & had.DEV_NAN_INPUT


def test_fused_build_attention_call_reads_sign_words(fqlib):
    """had_attention of the fused build (no float32 rows passed) reads the
    sign words as libhad.so does."""
    B, H, n, d, topn = 2, 3, 300, 64, 40
    log(f"fused build had_attention {(B, H, n, d, topn)}")
    inp = make_inputs(B, H, n, d, rank=4, noise="t3", seed=9, v_dtype="bf16")
    q, k, v = to_dev(inp)
    qb, _ = had.pack(q, with_sigma=False)
    kb, _ = had.pack(k, with_sigma=False)
    ref = had.attention(qb, kb, v, topn, 0.125, True)
    out = torch.empty_like(ref)
    rc = fqlib.had_attention(qb.data_ptr(), kb.data_ptr(), v.data_ptr(), had._v_dtype(v),
                             had.Shape(B, H, n, d), topn, 0.125, 1, out.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(out, ref)
