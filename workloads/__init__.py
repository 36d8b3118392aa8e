"""Seeded synthetic inputs for paged chunk attention.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic: no attention, no selection, no page summaries. Both the HIP
path and the CPU oracle consume the tensors produced here, byte for byte.

The workloads stand in for the Qwen2.5-7B training runs that the OOMB pages report
(gist.science explainer, "4. Experimental Results"): 28 query heads sharing 4 KV
heads, head dimension 128, bf16, 128-token pages. No dataset or trained weights are
involved; every value is N(0, 1) from a seeded generator, rounded to the input dtype
with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

# One generator per input, seeded independently, so that a change in one
# tensor's shape never changes another tensor's values.
SEEDS = {"q": 1, "k": 2, "v": 3, "do": 4, "perm": 5, "gperm": 6, "needle": 7}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hq: int                 # query heads
    hkv: int                # key/value heads
    d: int                  # head dimension
    page: int               # tokens per page
    chunk: int              # queries in the chunk under test
    total: int              # tokens in the sequence, chunk included
    dtype: torch.dtype
    top_k: Optional[int]    # pages kept by the selector; None = dense (all prior pages)
    needles: int = 0        # prior pages whose keys are pushed toward the chunk's mean query
    needle_gain: float = 1.5
    sweep: bool = False     # True: every chunk of the sequence, forward then reverse
    window: int = 0         # local attention: each query sees its `window` latest positions

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def t0(self) -> int:
        """Position of the first query of the (last) chunk = number of prior tokens."""
        return self.total - self.chunk

    @property
    def pages_per_head(self) -> int:
        return -(-self.total // self.page)

    @property
    def pool_pages(self) -> int:
        return self.hkv * self.pages_per_head

    @property
    def n_chunks(self) -> int:
        return self.total // self.chunk

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    # 2 query heads on 1 KV head, D=64 fp32, 16-token pages, 16 chunks of 64.
    "tiny": Workload("tiny", 2, 1, 64, 16, 64, 1024, torch.float32, None, sweep=True),
    # last 4096-token chunk of a 128K context, all 992 prior pages attended.
    "dense128k": Workload("dense128k", 28, 4, 128, 128, 4096, 131072, torch.bfloat16, None),
    # 4096-token chunk after 1M prior tokens, top-64 pages + the chunk's own 32.
    "sparse1m": Workload("sparse1m", 28, 4, 128, 128, 4096, 1048576 + 4096, torch.bfloat16, 64,
                         needles=32),
    # 8192-token chunk closing a 4M-token context, top-128 pages + 64 local.
    "sparse4m": Workload("sparse4m", 28, 4, 128, 128, 8192, 4194304, torch.bfloat16, 128,
                         needles=32),
    # local attention (sparse layers of sparse-native models): the sparse-1M chunk with
    # each query seeing its 128 latest positions instead of a page selection.
    "local1m": Workload("local1m", 28, 4, 128, 128, 4096, 1048576 + 4096, torch.bfloat16, None,
                        window=128),
    # 256K tokens in 32 chunks of 8192, every chunk forward then reverse.
    "sweep256k": Workload("sweep256k", 28, 4, 128, 128, 8192, 262144, torch.bfloat16, None,
                          sweep=True),
    "sweep256k_top64": Workload("sweep256k_top64", 28, 4, 128, 128, 8192, 262144,
                                torch.bfloat16, 64, sweep=True),
}


def custom(base_name: str, **kw) -> Workload:
    """A reduced workload with the same structure (for parity tests at small sizes)."""
    base = dataclasses.asdict(WORKLOADS[base_name])
    base.update(kw)
    base["name"] = kw.get("name", base_name + "_custom")
    return Workload(**base)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, dtype: torch.dtype, device="cpu") -> torch.Tensor:
    """N(0,1) drawn in fp32 then rounded once to `dtype` (round-to-nearest-even)."""
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def permutation(n: int, seed: int) -> torch.Tensor:
    """Seeded permutation of 0..n-1 (int64, CPU): physical placement of pages."""
    return torch.randperm(n, generator=_gen(seed, "cpu"))


def page_tables(w: Workload):
    """Logical->physical page tables [hkv, pages_per_head] for K/V and for dK/dV.

    The pool is shared by all KV heads; its physical pages are a shuffle of
    0..pool_pages-1, and the gradient pool has its own independent shuffle."""
    n = w.pool_pages
    kv = permutation(n, SEEDS["perm"]).to(torch.int32).reshape(w.hkv, w.pages_per_head)
    gr = permutation(n, SEEDS["gperm"]).to(torch.int32).reshape(w.hkv, w.pages_per_head)
    return kv, gr


def needle_pages(w: Workload) -> torch.Tensor:
    """The same seeded set of distinct prior logical pages for every KV head."""
    n_prior = w.t0 // w.page
    if w.needles == 0 or n_prior == 0:
        return torch.zeros(0, dtype=torch.int64)
    m = min(w.needles, n_prior)
    return torch.sort(torch.randperm(n_prior, generator=_gen(SEEDS["needle"], "cpu"))[:m]).values


def make_inputs(w: Workload, device="cpu", with_grad=True):
    """All inputs of one workload.

    Returns a dict:
      q, do : [hq, n_q, d]  (n_q = chunk, or total for a sweep)  in w.dtype
      k, v  : [hkv, total, d] in w.dtype
      table, gtable : int32 [hkv, pages_per_head]
      needles : int64 logical page ids
    For a sweep, q/do cover the whole sequence; chunk c is q[:, c*chunk:(c+1)*chunk].

    Needles: for each KV head, the fp32 keys of every token in the needle pages get
    `needle_gain` times the mean of that head group's chunk queries added before the
    cast to the input dtype. The mean is a plain fp64 average used only to shape
    the input; it is not the selector's query summary.
    """
    n_q = w.total if w.sweep else w.chunk
    out = {}
    out["q"] = normal((w.hq, n_q, w.d), SEEDS["q"], w.dtype, device)
    needles = needle_pages(w)
    if len(needles):
        k32 = normal((w.hkv, w.total, w.d), SEEDS["k"], torch.float32, device)
        qc = out["q"][:, -w.chunk:].to(torch.float64)
        direction = qc.reshape(w.hkv, w.group * w.chunk, w.d).mean(dim=1).to(torch.float32)
        tok = (needles[:, None] * w.page + torch.arange(w.page)[None, :]).reshape(-1).to(device)
        k32[:, tok] += w.needle_gain * direction[:, None, :]
        out["k"] = k32.to(w.dtype)
        del k32
    else:
        out["k"] = normal((w.hkv, w.total, w.d), SEEDS["k"], w.dtype, device)
    out["v"] = normal((w.hkv, w.total, w.d), SEEDS["v"], w.dtype, device)
    if with_grad:
        out["do"] = normal((w.hq, n_q, w.d), SEEDS["do"], w.dtype, device)
    out["table"], out["gtable"] = page_tables(w)
    out["needles"] = needles
    return out
