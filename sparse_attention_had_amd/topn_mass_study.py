"""How many of a row's largest attention weights hold a given softmax mass?

    python -m sparse_attention_had_amd.topn_mass_study [--dims 64] [--seqs 256 1024 4096 16384]

For each sequence length n it reports, over the rows of seeded synthetic
heads, the mean and 90th percentile of N/n, where N is the smallest number of
largest softmax weights that reach 90 %, 95 % and 99 % of the mass:

* "had": the HAD path's integer logits (sign bits of Q and K, s = d - 2h,
  softmax of s/sqrt(d)), measured by had_topn_mass on the GPU;
* "float": real-valued logits q.k/sqrt(d) of the same Q and K, with a
  sort + cumulative sum in PyTorch on the GPU.

Inputs: iid N(0, 1) Q and K (the Gaussian setting of the pages' mass
figure) and the long-document generator (rank-8 shared component plus
Student-t noise).  The question is whether N must grow linearly with n to
keep the mass.
"""

from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import sparse_attention_had_amd as had  # noqa: E402
from had_workloads import make_inputs  # noqa: E402

MASSES = (0.9, 0.95, 0.99)


def float_topn_mass(q: torch.Tensor, k: torch.Tensor, scale: float, mass: float) -> torch.Tensor:
    """Smallest N per row for real-valued logits (rows of one head at a time)."""
    out = []
    for bh in range(q.shape[0]):
        z = (q[bh].double() @ k[bh].double().T) * scale
        p = torch.softmax(z, dim=1)
        c = torch.cumsum(torch.sort(p, dim=1, descending=True).values, dim=1)
        out.append((c < mass).sum(dim=1) + 1)
    return torch.stack(out).clamp(max=q.shape[1])


def study(dims, seqs, heads, seed):
    rows = []
    for d in dims:
        for n in seqs:
            for gen, kw in (("iid", dict(rank=0, noise="normal")), ("rank8-t3", dict(rank=8, noise="t3"))):
                inp = make_inputs(1, heads, n, d, v_dtype="f32", seed=seed + n + d, **kw)
                q = torch.from_numpy(inp["q"]).cuda()
                k = torch.from_numpy(inp["k"]).cuda()
                qb, _ = had.pack(q, with_sigma=False)
                kb, _ = had.pack(k, with_sigma=False)
                scale = 1.0 / float(np.sqrt(d))
                for mass in MASSES:
                    nh = had.topn_mass(qb, kb, d, scale, mass).float().cpu().numpy() / n
                    nf = float_topn_mass(q[0], k[0], scale, mass).float().cpu().numpy() / n
                    rows.append({"d": d, "n": n, "inputs": gen, "mass": mass,
                                 "had_mean": float(nh.mean()), "had_p90": float(np.quantile(nh, 0.9)),
                                 "float_mean": float(nf.mean()), "float_p90": float(np.quantile(nf, 0.9))})
                    print(json.dumps(rows[-1]), flush=True)
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--dims", type=int, nargs="+", default=[64])
    ap.add_argument("--seqs", type=int, nargs="+", default=[256, 1024, 4096, 16384])
    ap.add_argument("--heads", type=int, default=4)
    ap.add_argument("--seed", type=int, default=100)
    a = ap.parse_args(argv)
    study(a.dims, a.seqs, a.heads, a.seed)


if __name__ == "__main__":
    main()
