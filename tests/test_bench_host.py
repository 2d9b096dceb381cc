"""Host-side pieces of bench.py, checked against the oracle (no GPU).

bench.py counts the allowed (query, key) pairs row by row from the band of
each head mask and the document bounds; the oracle counts them from its
element masks (``oracle.element_flops``). The two must agree on every kind
of workload the benchmark runs.
"""

import dataclasses

import numpy as np
import pytest
import torch

import bench
import oracle
from block_sparse_masked_splash_amd import workloads as wl


@pytest.mark.parametrize("name", ["c1", "c2", "c3h", "c3", "c4", "c5", "g3h", "d3h", "b5", "s3h"])
def test_allowed_pairs_match_oracle_element_flops(name):
    w = wl.WORKLOADS[name]
    H = min(w.H, 16)
    small = dataclasses.replace(w, B=min(w.B, 2), H=H, S=600 if w.segments else 333,
                                kv_heads=(H // (w.H // w.n_kv_heads)) if w.kv_heads else 0)
    gen = wl.generate(small)
    if w.name == "c4":  # the window of the full workload (1024) would cover every row here
        heads = tuple([wl.CAUSAL] * 8 + [wl.local_causal(40)] * 8)
        small = dataclasses.replace(small, head_masks=heads)
    qs = None if gen["q_segment_ids"] is None else gen["q_segment_ids"].numpy()
    dense = None if gen["dense"] is None else gen["dense"].numpy()
    want = oracle.element_flops(small.B, small.H, small.S, small.S, small.D, small.head_masks, qs, qs, dense=dense)
    assert 4 * small.D * bench.allowed_pairs(small, gen) == want


def test_allowed_pairs_short_documents_and_windows():
    """Many short documents (lengths 1..40) under causal and windowed heads."""
    rng = np.random.default_rng(5)
    S = 257
    ids = torch.from_numpy(wl.draw_documents(rng, 3, S, 1, 40))
    heads = (wl.CAUSAL, wl.local_causal(7), wl.FULL, (0, 3, 9))
    w = dataclasses.replace(wl.WORKLOADS["c3"], B=3, H=4, S=S, head_masks=heads)
    gen = {"q_segment_ids": ids, "dense": None}
    want = oracle.element_flops(3, 4, S, S, w.D, heads, ids.numpy(), ids.numpy())
    assert 4 * w.D * bench.allowed_pairs(w, gen) == want


def test_allowed_pairs_full_size_causal():
    """The S=8192 causal workload: 2*32 heads of S(S+1)/2 pairs (1.0997e12
    element FLOPs at D=128)."""
    w = wl.WORKLOADS["c3h"]
    n = w.S
    assert bench.allowed_pairs(w, {"q_segment_ids": None, "dense": None}) == 64 * n * (n + 1) // 2
