"""Seeded synthetic inputs for the MoE layer.

This module is the only code shared by the CPU oracle side (tests, the CPU
baseline) and the GPU side.  It holds no arithmetic of the layer itself: it
only produces pseudo-random input tensors.

Recipe
------
Every tensor is a *stream* identified by ``(seed, stream_id)``.  Element ``i``
(flat, row-major) of a stream is a pure function of ``(seed, stream_id, i)``:

* a 32-bit integer hash of the counter (two rounds of an xorshift-multiply
  mixer, all arithmetic on non-negative int64 values masked to 32 bits, so it
  is exact on any device);
* the top ``TABLE_BITS`` bits of the hash index a table of standard-normal
  quantiles ``Phi^-1((j + 0.5) / 2**TABLE_BITS)`` computed once in float64 and
  stored as float32 (a discretised N(0, 1) with 2**20 levels, tails cut at
  about +-4.9 sigma);
* the quantile is multiplied by ``std`` in float32 (a correctly rounded IEEE
  operation) and, for bf16 tensors, rounded to nearest-even bf16.

Because every step is exact or correctly rounded, the same call gives the
same bits on the CPU and on the GPU, and any slice (one expert's weights, a
handful of tokens) can be regenerated on its own from its flat offset.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

TABLE_BITS = 20
_M32 = 0xFFFFFFFF

# stream ids
S_LOGITS, S_X, S_WGATE, S_WUP, S_WDOWN, S_SGATE, S_SUP, S_SDOWN, S_DY, S_PERM, S_ROUTER = range(1, 12)

_TABLES: dict = {}


def normal_table(device="cpu") -> torch.Tensor:
    """float32 [2**TABLE_BITS] standard-normal quantiles at cell midpoints."""
    key = str(torch.device(device))
    if key not in _TABLES:
        if "cpu" not in _TABLES:
            from scipy.special import ndtri

            n = 1 << TABLE_BITS
            p = (np.arange(n, dtype=np.float64) + 0.5) / n
            _TABLES["cpu"] = torch.from_numpy(ndtri(p).astype(np.float32))
        _TABLES[key] = _TABLES["cpu"].to(device)
    return _TABLES[key]


def _mix32(x: torch.Tensor) -> torch.Tensor:
    # multipliers are below 2**31, so products of 32-bit values fit in int64
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & _M32
    x = x ^ (x >> 15)
    x = (x * 0x2C1B3C6D) & _M32
    x = x ^ (x >> 16)
    return x


def _key(seed: int, stream: int) -> tuple[int, int]:
    a = (seed * 0x9E3779B1 + stream * 0x85EBCA77 + 0x165667B1) & _M32
    t = _mix32(torch.tensor([a, a ^ 0x27D4EB2F], dtype=torch.int64))
    return int(t[0]), int(t[1])


def uniform_bits(n: int, seed: int, stream: int, offset: int = 0, device="cpu") -> torch.Tensor:
    """int64 tensor of n hashed 32-bit values for counters offset .. offset+n-1."""
    k0, k1 = _key(seed, stream)
    i = torch.arange(offset, offset + n, dtype=torch.int64, device=device)
    h = _mix32((i & _M32) ^ k0)
    h = _mix32(h ^ (i >> 32) ^ k1)
    return h


def normal(shape, seed: int, stream: int, std: float = 1.0, dtype=torch.float32,
           device="cpu", offset: int = 0, chunk: int = 1 << 24) -> torch.Tensor:
    """Discretised N(0, std) tensor of `shape`; element j has counter offset + j."""
    shape = tuple(int(s) for s in shape)
    n = math.prod(shape)
    out = torch.empty(n, dtype=dtype, device=device)
    table = normal_table(device)
    s = torch.tensor(std, dtype=torch.float32, device=device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        h = uniform_bits(c1 - c0, seed, stream, offset + c0, device)
        v = table[h >> (32 - TABLE_BITS)]
        if std != 1.0:
            v = v * s
        out[c0:c1] = v.to(dtype)
    return out.view(shape)


def zipf_bias(E: int, s: float = 1.1) -> torch.Tensor:
    """float32 [E]: b_e = 2 ln p_(e+1), p_r = r^-s / sum_q q^-s (expert 0 hottest)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p = p / p.sum()
    return torch.from_numpy((2.0 * np.log(p)).astype(np.float32))


def permutation(n: int, seed: int, stream: int, device="cpu") -> torch.Tensor:
    """A seeded permutation of range(n) (argsort of distinct hashed keys)."""
    h = uniform_bits(n, seed, stream, 0, device)
    key = (h << 32) | torch.arange(n, dtype=torch.int64, device=device)
    return torch.argsort(key)


# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    seed: int
    n_shared: int = 0
    macrobatch: int = 0   # tokens; 0 = T
    minibatch: int = 0    # tokens; 0 = macrobatch
    zipf: bool = False
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def S(self) -> int:
        return self.T * self.k


SHAPES = {
    # tiny forward/backward, several GEMM tiles and ragged groups
    "tiny": MoEShape("tiny", T=256, H=256, I=128, E=8, k=2, seed=0),
    # 512 experts, H 4096, I 1024, top-10, 2048 tokens, all experts on one GPU;
    # the backward's upstream gradient dy uses seed 3
    "e512_t2048": MoEShape("e512_t2048", T=2048, H=4096, I=1024, E=512, k=10, seed=1,
                           extra={"dy_seed": 3}),
    # long Zipf-imbalanced stream through the ring buffer, with a shared expert
    "e512_t65536_zipf": MoEShape("e512_t65536_zipf", T=65536, H=4096, I=1024, E=512, k=10,
                                 seed=4, n_shared=1, macrobatch=16384, minibatch=4096,
                                 zipf=True),
    # one GPU's expert-parallel share of the 512-expert layer (64 ranks x 2048
    # tokens x top-10 / 512): 8 local experts, exactly 2560 rows each; every row
    # is routed top-1 to its expert by one-hot logits from a seeded balanced
    # assignment (weight 1), so dispatch, GEMMs and combine see that share
    "e8_ep_share": MoEShape("e8_ep_share", T=20480, H=4096, I=1024, E=8, k=1, seed=2,
                            extra={"balanced": True}),
}


def balanced_assignment(shape: MoEShape, device="cpu") -> torch.Tensor:
    """int64 [T]: row t's expert, exactly T/E rows each (rank in a seeded permutation // (T/E))."""
    per = shape.T // shape.E
    rank = torch.empty(shape.T, dtype=torch.int64, device=device)
    rank[permutation(shape.T, shape.seed, S_PERM, device)] = torch.arange(shape.T, device=device)
    return rank // per


def logits(shape: MoEShape, device="cpu") -> torch.Tensor:
    """fp32 [T, E] router logits: N(0,1), plus the Zipf bias per expert if shape.zipf;
    one-hot (1 at the assigned expert, 0 elsewhere) for a balanced shape."""
    if shape.extra.get("balanced"):
        L = torch.zeros((shape.T, shape.E), dtype=torch.float32, device=device)
        L[torch.arange(shape.T, device=device), balanced_assignment(shape, device)] = 1.0
        return L
    L = normal((shape.T, shape.E), shape.seed, S_LOGITS, 1.0, torch.float32, device)
    if shape.zipf:
        L = L + zipf_bias(shape.E).to(device)
    return L


def tokens(shape: MoEShape, device="cpu", rows=None) -> torch.Tensor:
    """bf16 [T, H] (or the listed rows) activations, N(0,1)."""
    if rows is None:
        return normal((shape.T, shape.H), shape.seed, S_X, 1.0, torch.bfloat16, device)
    return torch.stack([normal((shape.H,), shape.seed, S_X, 1.0, torch.bfloat16, device,
                               offset=int(t) * shape.H) for t in rows])


def grad_out(shape: MoEShape, device="cpu", rows=None) -> torch.Tensor:
    """bf16 [T, H] upstream gradient dy, N(0,1)."""
    seed = shape.extra.get("dy_seed", shape.seed + 100)
    if rows is None:
        return normal((shape.T, shape.H), seed, S_DY, 1.0, torch.bfloat16, device)
    return torch.stack([normal((shape.H,), seed, S_DY, 1.0, torch.bfloat16, device,
                               offset=int(t) * shape.H) for t in rows])


def expert_weights(shape: MoEShape, e: int, device="cpu"):
    """bf16 (W_gate[e] [I,H], W_up[e] [I,H], W_down[e] [H,I]); std 1/sqrt(fan_in)."""
    H, I = shape.H, shape.I
    wg = normal((I, H), shape.seed, S_WGATE, 1.0 / math.sqrt(H), torch.bfloat16, device, offset=e * I * H)
    wu = normal((I, H), shape.seed, S_WUP, 1.0 / math.sqrt(H), torch.bfloat16, device, offset=e * I * H)
    wd = normal((H, I), shape.seed, S_WDOWN, 1.0 / math.sqrt(I), torch.bfloat16, device, offset=e * H * I)
    return wg, wu, wd


def all_expert_weights(shape: MoEShape, device="cpu"):
    """bf16 W_gate, W_up [E,I,H] and W_down [E,H,I], generated in chunks."""
    H, I, E = shape.H, shape.I, shape.E
    wg = normal((E, I, H), shape.seed, S_WGATE, 1.0 / math.sqrt(H), torch.bfloat16, device)
    wu = normal((E, I, H), shape.seed, S_WUP, 1.0 / math.sqrt(H), torch.bfloat16, device)
    wd = normal((E, H, I), shape.seed, S_WDOWN, 1.0 / math.sqrt(I), torch.bfloat16, device)
    return wg, wu, wd


def shared_weights(shape: MoEShape, device="cpu"):
    """bf16 shared expert (W_gate [I,H], W_up [I,H], W_down [H,I]) or None."""
    if not shape.n_shared:
        return None
    H, I = shape.H, shape.I
    wg = normal((I, H), shape.seed, S_SGATE, 1.0 / math.sqrt(H), torch.bfloat16, device)
    wu = normal((I, H), shape.seed, S_SUP, 1.0 / math.sqrt(H), torch.bfloat16, device)
    wd = normal((H, I), shape.seed, S_SDOWN, 1.0 / math.sqrt(I), torch.bfloat16, device)
    return wg, wu, wd


def router_weights(shape: MoEShape, device="cpu") -> torch.Tensor:
    """bf16 [E, H] router projection (row e = expert e), std 1/sqrt(H)."""
    return normal((shape.E, shape.H), shape.seed, S_ROUTER, 1.0 / math.sqrt(shape.H), torch.bfloat16, device)


def custom_shape(name, T, H, I, E, k, seed, **kw) -> MoEShape:
    return MoEShape(name, T=T, H=H, I=I, E=E, k=k, seed=seed, **kw)
