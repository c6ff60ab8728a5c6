"""Seeded synthetic inputs for the exact-attention workloads.

This module only draws and rounds random inputs; it holds none of the attention
arithmetic. Both the HIP path (through the tests and the bench) and the CPU
oracle consume what it returns, so each side sees exactly the same bytes.

Recipe (one numpy PCG64 generator per case, seeded):
  1. Q, K, V, dO  = standard_normal((B, H, N, d), float32), drawn in that order;
  2. key-padding cases: key_len = integers(lo, hi + 1, size=B)  (uniform, inclusive);
  3. block-sparse cases: for every block pair i < j draw u ~ U[0, 1) (row-major
     order over the upper triangle) and keep the pair iff u < p; mirror to (j, i);
     every diagonal block is kept.
  4. bf16 cases round Q, K, V, dO from float32 to bfloat16 with
     round-to-nearest-even; the float32 arrays returned hold those rounded values.

The shapes stand in for the attention layers of the pages' workloads
(BERT-large at sequence 512, GPT-2 at 1K, long-context GPT-2 / LRA at 4K-8K,
block-sparse long sequences): FlashAttention reading notes (hackmd),
§Experiments › 4.2 and 4.4. Values are N(0, 1) because the pages give no
activation statistics.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"

# Named workloads: (B, H, N, d), dtype, mask kind and default seed.
CONFIGS: dict[str, dict] = {
    "C1": dict(B=1, H=1, N=128, d=64, dtype=F32, mask="none", seed=1, fwd_only=True,
               desc="forward only, fp32, no mask"),
    "C2": dict(B=16, H=16, N=512, d=64, dtype=BF16, mask="key_len", key_len_range=(384, 512),
               seed=2, desc="BERT-large-shaped, key-padding mask"),
    "C3": dict(B=8, H=12, N=1024, d=64, dtype=BF16, mask="causal", seed=3,
               desc="GPT-2-shaped, causal"),
    "C4a": dict(B=2, H=16, N=4096, d=128, dtype=BF16, mask="causal", seed=4,
                desc="long-sequence causal, N=4096"),
    "C4b": dict(B=2, H=16, N=8192, d=128, dtype=BF16, mask="causal", seed=5,
                desc="long-sequence causal, N=8192"),
    "C5": dict(B=1, H=8, N=16384, d=64, dtype=BF16, mask="block", block_size=128, block_p=0.125,
               seed=6, desc="block-sparse, 128x128 blocks, diagonal + symmetric p=1/8"),
    # Long sequences (the pages' 64K-token tasks): measured, and parity-tested on sampled rows.
    "L64K": dict(B=1, H=16, N=65536, d=64, dtype=BF16, mask="causal", seed=7,
                 desc="long-sequence causal, N=65536"),
    "L64Ks": dict(B=1, H=16, N=65536, d=64, dtype=BF16, mask="block", block_size=256, block_p=0.125,
                  seed=8, desc="long-sequence block-sparse, N=65536, 256x256 blocks, p=1/8"),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even, NaN kept quiet."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    bits = (rounded >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        bits = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16), bits)
    return bits


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_block_mask(rng: np.random.Generator, nb: int, p: float) -> np.ndarray:
    """Symmetric block mask: diagonal kept, each pair i<j kept i.i.d. with probability p."""
    iu, ju = np.triu_indices(nb, k=1)
    keep = rng.random(iu.size) < p
    m = np.zeros((nb, nb), dtype=np.uint8)
    m[iu[keep], ju[keep]] = 1
    m[ju[keep], iu[keep]] = 1
    m[np.arange(nb), np.arange(nb)] = 1
    return m


@dataclass
class Case:
    """One seeded attention problem. Float arrays are [B, H, N, d] float32, holding
    exactly the values the device receives (bf16-rounded for bf16 cases)."""
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    scale: np.float32
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    key_len: Optional[np.ndarray] = None      # int32 [B]
    block_mask: Optional[np.ndarray] = None   # uint8 [N/bs, N/bs]
    block_size: Optional[int] = None
    seed: int = 0
    meta: dict = field(default_factory=dict)

    def bits(self, name: str) -> np.ndarray:
        """bf16 bit patterns of q/k/v/do (bf16 cases only)."""
        assert self.dtype == BF16
        return f32_to_bf16_bits(getattr(self, name))


def make_case(B: int, H: int, N: int, d: int, dtype: str = BF16, mask: str = "none", seed: int = 0,
              key_len_range: Optional[tuple[int, int]] = None, block_size: Optional[int] = None,
              block_p: Optional[float] = None, scale: Optional[float] = None, name: str = "custom",
              std: float = 1.0) -> Case:
    """Draw one case following the module recipe. mask: "none", or kinds from {causal, key_len,
    block} joined by "+" (e.g. "block+causal"); the draws happen in the order Q, K, V, dO, key
    lengths, block mask whatever the order of the kinds."""
    kinds = set() if mask == "none" else set(mask.split("+"))
    assert kinds <= {"causal", "key_len", "block"}, mask
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    arrs = [rng.standard_normal(shape, dtype=np.float32) for _ in range(4)]
    if std != 1.0:
        arrs = [a * np.float32(std) for a in arrs]
    key_len = None
    if "key_len" in kinds:
        lo, hi = key_len_range if key_len_range is not None else (0, N)
        key_len = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    block_mask = None
    if "block" in kinds:
        assert block_size is not None and N % block_size == 0
        block_mask = draw_block_mask(rng, N // block_size, 0.125 if block_p is None else block_p)
    if dtype == BF16:
        arrs = [bf16_round(a) for a in arrs]
    sc = np.float32(1.0 / np.sqrt(d)) if scale is None else np.float32(scale)
    return Case(name=name, B=B, H=H, N=N, d=d, dtype=dtype, causal="causal" in kinds, scale=sc,
                q=arrs[0], k=arrs[1], v=arrs[2], do=arrs[3], key_len=key_len, block_mask=block_mask,
                block_size=block_size if "block" in kinds else None, seed=seed)


def make_config(name: str, seed: Optional[int] = None) -> Case:
    """The named workload (C1 ... C5) with its default seed unless one is given."""
    c = CONFIGS[name]
    s = c["seed"] if seed is None else seed
    return make_case(c["B"], c["H"], c["N"], c["d"], dtype=c["dtype"], mask=c["mask"], seed=s,
                     key_len_range=c.get("key_len_range"), block_size=c.get("block_size"),
                     block_p=c.get("block_p"), name=name)
