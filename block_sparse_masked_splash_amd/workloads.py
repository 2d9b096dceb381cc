"""Seeded synthetic inputs for the attention workloads.

This module holds random draws, shapes and plain mask descriptions only; it
contains none of the attention arithmetic. Both the GPU path (through the
binding) and the CPU oracle consume what it produces, and neither is imported
here.

Recipe (shared by every test and by the benchmark):
  * ``numpy.random.default_rng(seed)`` (PCG64); q, k, v are drawn in that order
    as float32 ``standard_normal`` of shape [B, H, S, D] (k and v with
    kv_heads instead of H heads for grouped-query workloads), times sigma.
  * bf16 workloads round those float32 values to bfloat16 with
    round-to-nearest-even (``torch.Tensor.to(torch.bfloat16)``); the oracle
    receives the rounded values upcast exactly to float64.
  * Backward workloads: after v, with the same generator, the output
    gradient d_o as float32 ``standard_normal`` of q's shape (sigma 1).
  * Packed documents (segment ids): after that, with the same generator, each
    batch row draws integer document lengths uniformly in [lo, hi] until the
    running total reaches S, the last document is cut at S, and documents are
    numbered 0, 1, 2, ... along the row; q and kv share the ids.

A dense mask is an explicit boolean [S, S] array shared by all heads; the one
workload kind here ("tril") is the causal pattern written out as such an
array, the form in which "hstu_ops.py" (``pointwise_splash_attention``)
accepts an arbitrary numpy mask.

A head mask is a plain triple ``(causal, window_left, window_right)``: causal
means key position <= query position; a window bound of -1 is unbounded,
otherwise keys in [q - window_left, q + window_right] are allowed. This is the
shape of the per-head masks that "hstu_ops.py" (RecML,
``pointwise_splash_attention``) composes from CausalMask, FullMask and
LocalMask((w, w), offset=0).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

CAUSAL = (1, -1, -1)
FULL = (0, -1, -1)


def local_causal(window: int) -> tuple:
    """Causal mask ANDed with a symmetric local window of ``window`` keys."""
    return (1, int(window), int(window))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str              # "f32" or "bf16" (storage type of q, k, v)
    sigma: float            # standard deviation of q, k, v
    head_masks: tuple       # one triple (broadcast) or H triples
    block_q: int
    block_kv: int
    segments: bool          # packed documents (causal AND same segment)
    pointwise: bool         # SiLU pointwise attention instead of softmax
    seed: int
    kv_heads: int = 0       # K/V heads (0: H, plain multi-head attention)
    dense: str = ""         # "" (none) or "tril": the causal pattern as a dense [S, S] array
    backward: bool = False  # also an output gradient d_o (the pointwise backward's input)

    @property
    def n_kv_heads(self) -> int:
        return self.kv_heads or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["head_masks"] = [list(m) for m in self.head_masks]
        return d


_LOCAL_MIX = tuple([CAUSAL] * 8 + [local_causal(1024)] * 8)

WORKLOADS = {
    # tiny fp32 causal attention
    "c1": Workload("c1", 1, 1, 256, 64, "f32", 1.0, (CAUSAL,), 64, 64, False, False, 1),
    # causal MHA, S=2048
    "c2": Workload("c2", 4, 16, 2048, 128, "bf16", 1.0, (CAUSAL,), 128, 128, False, False, 2),
    # causal MHA, S=8192, H=32, D=128 (the throughput workload)
    "c3h": Workload("c3h", 2, 32, 8192, 128, "bf16", 1.0, (CAUSAL,), 128, 128, False, False, 3),
    # causal AND same document, packed documents of length 256..2048
    "c3": Workload("c3", 2, 32, 8192, 128, "bf16", 1.0, (CAUSAL,), 128, 128, True, False, 3),
    # 8 causal heads + 8 causal local-window-1024 heads, S=32768
    "c4": Workload("c4", 1, 16, 32768, 128, "bf16", 1.0, _LOCAL_MIX, 128, 128, False, False, 4),
    # pointwise SiLU attention, causal, N(0, 0.5^2)
    "c5": Workload("c5", 8, 8, 4096, 64, "bf16", 0.5, (CAUSAL,), 128, 128, False, True, 5),
    # grouped-query form of c3h: 32 query heads over 8 K/V heads
    "g3h": Workload("g3h", 2, 32, 8192, 128, "bf16", 1.0, (CAUSAL,), 128, 128, False, False, 6, kv_heads=8),
    # c3h's attention with its causal pattern handed over as a dense mask array
    "d3h": Workload("d3h", 2, 32, 8192, 128, "bf16", 1.0, (FULL,), 128, 128, False, False, 7, dense="tril"),
    # c5's pointwise attention with its causal pattern as a dense mask array
    "d5": Workload("d5", 8, 8, 4096, 64, "bf16", 0.5, (FULL,), 128, 128, False, True, 8, dense="tril"),
    # the pointwise backward at c5's shape, output gradient N(0, 1)
    "b5": Workload("b5", 8, 8, 4096, 64, "bf16", 0.5, (CAUSAL,), 128, 128, False, True, 9, backward=True),
    # the pointwise backward at D = 128: B=2 H=16 S=4096
    "b5h": Workload("b5h", 2, 16, 4096, 128, "bf16", 0.5, (CAUSAL,), 128, 128, False, True, 10, backward=True),
    # the softmax backward at the causal S=8192 shape
    "s3h": Workload("s3h", 2, 32, 8192, 128, "bf16", 1.0, (CAUSAL,), 128, 128, False, False, 11, backward=True),
}


def dense_mask(w: Workload, S: int):
    """The workload's dense boolean [S, S] mask as a CPU torch tensor, or None."""
    if not w.dense:
        return None
    if w.dense != "tril":
        raise ValueError(f"unknown dense mask kind {w.dense!r}")
    import torch
    return torch.from_numpy(np.tri(S, S, dtype=bool))


def draw_qkv_f32(rng: np.random.Generator, B: int, H: int, Sq: int, Skv: int, D: int,
                 sigma: float, kv_heads: int | None = None):
    """float32 q [B,H,Sq,D], k [B,Hk,Skv,D], v [B,Hk,Skv,D] (Hk = kv_heads or
    H), drawn in that order."""
    Hk = H if kv_heads is None else kv_heads
    q = rng.standard_normal((B, H, Sq, D), dtype=np.float32) * np.float32(sigma)
    k = rng.standard_normal((B, Hk, Skv, D), dtype=np.float32) * np.float32(sigma)
    v = rng.standard_normal((B, Hk, Skv, D), dtype=np.float32) * np.float32(sigma)
    return q, k, v


def draw_documents(rng: np.random.Generator, B: int, S: int, lo: int = 256,
                   hi: int = 2048) -> np.ndarray:
    """int32 [B, S] document ids: lengths uniform in [lo, hi], last one cut at S."""
    ids = np.empty((B, S), dtype=np.int32)
    for b in range(B):
        pos, doc = 0, 0
        while pos < S:
            n = int(rng.integers(lo, hi, endpoint=True))
            ids[b, pos:min(S, pos + n)] = doc
            pos += n
            doc += 1
    return ids


def _store(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.to(torch.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def generate(w: Workload, *, B: int | None = None, H: int | None = None,
             S: int | None = None, seed: int | None = None) -> dict:
    """CPU torch tensors for workload ``w`` (sizes overridable for small cases).

    Returns dict(q, k, v, q_segment_ids, kv_segment_ids, dense, d_o) where the
    segment ids are int32 torch tensors [B, S] or None, ``dense`` is the
    boolean [S, S] mask or None and ``d_o`` the output gradient (backward
    workloads) or None.
    """
    B = w.B if B is None else B
    Hk = w.n_kv_heads if H is None else max(1, H // (w.H // w.n_kv_heads))
    H = w.H if H is None else H
    S = w.S if S is None else S
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q, k, v = draw_qkv_f32(rng, B, H, S, S, w.D, w.sigma, Hk)
    out = dict(q=_store(q, w.dtype), k=_store(k, w.dtype), v=_store(v, w.dtype),
               q_segment_ids=None, kv_segment_ids=None, dense=dense_mask(w, S), d_o=None)
    if w.backward:
        out["d_o"] = _store(rng.standard_normal(q.shape, dtype=np.float32), w.dtype)
    del q, k, v
    if w.segments:
        import torch
        ids = torch.from_numpy(draw_documents(rng, B, S))
        out["q_segment_ids"] = ids
        out["kv_segment_ids"] = ids.clone()
    return out


def random_case(seed: int, B: int, H: int, Sq: int, Skv: int, D: int, dtype: str,
                sigma: float = 1.0, segments: str | None = None,
                doc_len: tuple = (1, 64)) -> dict:
    """Small seeded case with independent sizes for parity tests.

    ``segments``: None, "docs" (packed documents with lengths in ``doc_len``,
    same ids for q and kv when Sq == Skv) or "random" (arbitrary int32 ids drawn
    from a small set, independently for q and kv).
    """
    rng = np.random.default_rng(seed)
    q, k, v = draw_qkv_f32(rng, B, H, Sq, Skv, D, sigma)
    out = dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
               q_segment_ids=None, kv_segment_ids=None)
    if segments is not None:
        import torch
        if segments == "docs":
            qs = draw_documents(rng, B, Sq, doc_len[0], doc_len[1])
            ks = qs.copy() if Skv == Sq else draw_documents(rng, B, Skv, doc_len[0], doc_len[1])
        elif segments == "random":
            vals = rng.integers(-2**31, 2**31 - 1, size=3, dtype=np.int64).astype(np.int32)
            qs = vals[rng.integers(0, 3, size=(B, Sq))]
            ks = vals[rng.integers(0, 3, size=(B, Skv))]
        else:
            raise ValueError(segments)
        out["q_segment_ids"] = torch.from_numpy(np.ascontiguousarray(qs, dtype=np.int32))
        out["kv_segment_ids"] = torch.from_numpy(np.ascontiguousarray(ks, dtype=np.int32))
    return out
