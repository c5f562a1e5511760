"""Seeded synthetic inputs for HiKVP attention: clustered-Gaussian key trees,
leaf values, queries and causal sequence K/V.

This module draws random numbers and lays out the tree topology; it holds none
of the attention arithmetic.  Both the GPU tests/benchmark and the CPU oracle
consume the tensors it materialises.

Recipe (the stand-in for encoder embeddings of a knowledge graph, whose data
and encoders are not available here):
  * root keys ~ N(0, 1) per element;
  * every mid key = its parent root key + 0.3 * N(0, 1);
  * every leaf key = its parent mid key + 0.3 * N(0, 1);
  * leaf values, queries and sequence K/V ~ N(0, 1);
  * each KV head drawn independently over one shared topology;
  * draws in fp32 on the target device with torch.Generator(seed), fixed order
    root -> mid -> leaf keys -> leaf values -> q -> seq_k -> seq_v, each
    tensor rounded once to the storage dtype;
  * balanced fanouts: the first (children mod parents) parents get one extra
    child; "ragged" trees draw random fanouts (zeros allowed) instead.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

# Level sizes follow the clustering section of the AtlasKV digest page
# (S = ceil(cbrt M), M_I = ceil(M^(2/3)), M_R = ceil(M_I / cbrt M)); the tests
# check these constants against the oracle's integer evaluation.
CONFIGS = {
    "tiny": dict(dtype="f32", B=1, N=16, S_kv=16, Hq=4, Hkv=4, d=64,
                 M_R=10, M_I=100, M=1000, K=(2, 2, 4), seed=0),
    "m1e4": dict(dtype="bf16", B=1, N=128, S_kv=128, Hq=32, Hkv=8, d=128,
                 M_R=22, M_I=465, M=10_000, K=(4, 4, 16), seed=1),
    "m1e6": dict(dtype="bf16", B=1, N=512, S_kv=512, Hq=32, Hkv=8, d=128,
                 M_R=100, M_I=10_000, M=1_000_000, K=(8, 8, 32), seed=2),
    "m1e7_decode": dict(dtype="bf16", B=64, N=1, S_kv=4096, Hq=32, Hkv=8, d=128,
                        M_R=216, M_I=46_416, M=10_000_000, K=(8, 8, 32), seed=3),
    "m1e8_slice": dict(dtype="bf16", B=1, N=1024, S_kv=1024, Hq=4, Hkv=1, d=128,
                       M_R=465, M_I=215_444, M=100_000_000, K=(16, 16, 64), seed=4),
}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_CHUNK_ROWS = 1 << 21          # leaf rows drawn per chunk (bounds fp32 temporaries)
_CHILD_SIGMA = 0.3


@dataclass
class Case:
    name: str
    dtype: str
    B: int
    N: int
    S_kv: int
    Hq: int
    Hkv: int
    d: int
    M_R: int
    M_I: int
    M: int
    K: Tuple[int, int, int]
    q: torch.Tensor
    root_k: torch.Tensor
    mid_k: torch.Tensor
    leaf_k: torch.Tensor
    leaf_v: torch.Tensor
    root_off: torch.Tensor
    mid_off: torch.Tensor
    seq_k: Optional[torch.Tensor]
    seq_v: Optional[torch.Tensor]
    q_kg: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.B * self.N * self.Hq


def balanced_offsets(parents: int, children: int) -> torch.Tensor:
    """CSR offsets [parents + 1] (int64, CPU) with near-equal fanouts."""
    base, extra = divmod(children, parents) if parents else (0, 0)
    counts = torch.full((parents,), base, dtype=torch.int64)
    counts[:extra] += 1
    off = torch.zeros(parents + 1, dtype=torch.int64)
    torch.cumsum(counts, 0, out=off[1:])
    return off


def ragged_offsets(parents: int, children: int, gen: torch.Generator) -> torch.Tensor:
    """CSR offsets with random fanouts summing to `children` (zeros allowed)."""
    cuts = torch.randint(0, children + 1, (max(parents - 1, 0),), generator=gen).sort().values
    off = torch.cat([torch.zeros(1, dtype=torch.int64), cuts.to(torch.int64),
                     torch.full((1,), children, dtype=torch.int64)])
    return off


def _parent_index(off: torch.Tensor, lo: int, hi: int, device) -> torch.Tensor:
    """Parent of each child lo..hi-1 given CSR offsets."""
    child = torch.arange(lo, hi, dtype=torch.int64, device=device)
    return torch.searchsorted(off.to(device), child, right=True) - 1


def make_case(name: str = "tiny", device="cpu", seed: Optional[int] = None,
              ragged: bool = False, **overrides) -> Case:
    """Materialise one configuration (overrides replace any config field)."""
    cfg = dict(CONFIGS[name]) if name in CONFIGS else {}
    cfg.update(overrides)
    if seed is None:
        seed = cfg.get("seed", 0)
    dt = _TORCH_DTYPE[cfg["dtype"]]
    B, N, S, Hq, Hkv, d = (cfg[k] for k in ("B", "N", "S_kv", "Hq", "Hkv", "d"))
    MR, MI, M = cfg["M_R"], cfg["M_I"], cfg["M"]
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    if ragged:
        tgen = torch.Generator()
        tgen.manual_seed(seed + 7919)
        root_off = ragged_offsets(MR, MI, tgen)
        mid_off = ragged_offsets(MI, M, tgen)
    else:
        root_off = balanced_offsets(MR, MI)
        mid_off = balanced_offsets(MI, M)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    root32 = randn(Hkv, MR, d)
    mid_par = _parent_index(root_off, 0, MI, device)
    mid32 = root32[:, mid_par, :] + _CHILD_SIGMA * randn(Hkv, MI, d)
    leaf_k = torch.empty(Hkv, M, d, dtype=dt, device=device)
    for g in range(Hkv):
        for lo in range(0, M, _CHUNK_ROWS):
            hi = min(M, lo + _CHUNK_ROWS)
            par = _parent_index(mid_off, lo, hi, device)
            leaf_k[g, lo:hi] = (mid32[g, par, :] + _CHILD_SIGMA * randn(hi - lo, d)).to(dt)
    leaf_v = torch.empty(Hkv, M, d, dtype=dt, device=device)
    for g in range(Hkv):
        for lo in range(0, M, _CHUNK_ROWS):
            hi = min(M, lo + _CHUNK_ROWS)
            leaf_v[g, lo:hi] = randn(hi - lo, d).to(dt)
    q = randn(B, N, Hq, d).to(dt)
    seq_k = randn(B, S, Hkv, d).to(dt) if S > 0 else None
    seq_v = randn(B, S, Hkv, d).to(dt) if S > 0 else None
    return Case(name=name, dtype=cfg["dtype"], B=B, N=N, S_kv=S, Hq=Hq, Hkv=Hkv, d=d,
                M_R=MR, M_I=MI, M=M, K=tuple(cfg["K"]), q=q, root_k=root32.to(dt),
                mid_k=mid32.to(dt), leaf_k=leaf_k, leaf_v=leaf_v,
                root_off=root_off.to(device), mid_off=mid_off.to(device),
                seq_k=seq_k, seq_v=seq_v)
