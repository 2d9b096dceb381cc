"""Plain fp64 definitions of block-sparse masked attention (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.

Everything here is written from the pages' definitions, in float64, with no
blocking, fusion or reordering beyond what a definition states:

* Element mask: "hstu_ops.py" (RecML), ``pointwise_splash_attention`` builds
  a CausalMask or FullMask, optionally ANDed with LocalMask((w, w), offset=0);
  ``_apply_mask`` ANDs that with segment equality ``q_ids == kv_ids``.
* Dense masks: "hstu_ops.py", ``pointwise_splash_attention`` (a numpy array
  mask of shape (q_len, kv_len) becomes a NumpyMask) and the forward's mask
  block index map (partial blocks fetch their mask through ``mask_next``).
* Block metadata: "hstu_ops.py", ``_next_nonzero`` (a block runs when its
  ``block_mask`` entry is > 0, needs no element mask when it is not 1, and the
  kv block fetched at grid step j is ``data_next[h, i, j]``); page 3
  "JAX 到 VLIW ... 复习笔记", section 21 (sparse indirection: a fully masked kv
  block is skipped by pointing at the next valid block).
* Softmax attention: page 3, section 12 (naive attention: scores, max, exp,
  sum, divide, times V) and section 15 (Out = sum_t e^{a_t - M} v_t /
  sum_t e^{a_t - M}).
* Online softmax: page 3, sections 15.1-15.3 (m, L, O per kv block and the
  correction alpha = e^{m_A - m_AB}).
* Grouped-query attention: page 3, section 21 (query head h reads K/V head
  h // q_heads_per_kv_head).
* Pointwise backward: "hstu_ops.py", ``_pointwise_splash_attention_bwd_kernel_impl``
  (per kv block: scores qk = scale * k q^T, sigmoid masked to 0,
  p = qk * sigmoid / seq_len, dv += p do, dp = v do^T,
  ds = dp * sigmoid * (1 + qk (1 - sigmoid)) / seq_len, dk += scale ds q,
  dq += scale ds^T k) and ``_pointwise_splash_attention_bwd_kernel`` (grid over
  kv blocks, then heads, then q blocks; the q block fetched at step i is
  ``data_next[h, i, j]`` of the dK/dV metadata, ``_next_nonzero(next_i=True)``).
* Softmax log-sum-exp and backward: page 3, section 15 (per row, the running
  max m and sum L give log sum e^a = m + log L) and section 12's definition of
  softmax attention, differentiated; "hstu_ops.py" (``custom_vjp``: the
  forward hands the backward its residuals). The pages give no softmax
  backward kernel: the reading taken is the gradient of the definition, with
  the forward's log-sum-exp as the residual.
* Pointwise attention: "hstu_ops.py", ``_pointwise_splash_attention_fwd_kernel_impl``
  (scores times scale, times logistic(scores), divided by the query sequence
  length, masked entries set to 0, then times V), with the contributions of
  all kv blocks summed (page 3, section 14: kv tiles add, they do not
  concatenate).

Where the pages are silent, the reading taken is stated at the function that
relies on it.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------


def _allowed(qpos: np.ndarray, kpos: np.ndarray, head) -> np.ndarray:
    """Boolean [len(qpos), len(kpos)] base mask of one head.

    ``head = (causal, window_left, window_right)``. causal: key <= query
    (top-left aligned). Window bounds of -1 are unbounded; otherwise a key is
    allowed when q - window_left <= k <= q + window_right (the symmetric
    LocalMask((w, w)) of "hstu_ops.py" is (w, w), read as inclusive bounds).
    """
    causal, wl, wr = (int(x) for x in head)
    q = np.asarray(qpos, dtype=np.int64)[:, None]
    k = np.asarray(kpos, dtype=np.int64)[None, :]
    m = np.ones((q.shape[0], k.shape[1]), dtype=bool)
    if causal:
        m &= k <= q
    if wl >= 0:
        m &= k >= q - wl
    if wr >= 0:
        m &= k <= q + wr
    return m


def element_mask(q_len: int, kv_len: int, head, q_seg=None, kv_seg=None,
                 rows=None, dense=None) -> np.ndarray:
    """Boolean element mask [len(rows), kv_len] of one (batch, head).

    ``q_seg`` / ``kv_seg`` are the segment ids of this batch row ([q_len],
    [kv_len]) or None; with ids, a pair is allowed only when they are equal.
    ``dense`` is an arbitrary boolean [q_len, kv_len] mask of this head or
    None ("hstu_ops.py", ``pointwise_splash_attention``: a numpy array mask
    becomes a NumpyMask, which the local window is ANDed onto). All parts are
    combined with logical AND ("hstu_ops.py", ``_apply_mask``). ``rows``
    selects query positions (default: all).
    """
    qpos = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    kpos = np.arange(kv_len)
    m = _allowed(qpos, kpos, head)
    if dense is not None:
        d = np.asarray(dense, dtype=bool)
        if d.shape != (q_len, kv_len):
            raise ValueError(f"dense mask shape {d.shape} is not ({q_len}, {kv_len})")
        m &= d[qpos]
    if (q_seg is None) != (kv_seg is None):
        raise ValueError("q and kv segment ids must be given together or not at all")
    if q_seg is not None:
        qs = np.asarray(q_seg)[qpos]
        ks = np.asarray(kv_seg)
        m &= qs[:, None] == ks[None, :]
    return m


def padded_element_mask(q_len: int, kv_len: int, bq: int, bkv: int, head,
                        q_seg=None, kv_seg=None, q_block=None, dense=None) -> np.ndarray:
    """Element mask over whole blocks: [nq*bq, nk*bkv], or [bq, nk*bkv] for the
    single query block ``q_block``. Positions past the sequence ends are not
    allowed (reading for lengths that are not a multiple of the block size)."""
    nq = -(-q_len // bq)
    nk = -(-kv_len // bkv)
    blocks = range(nq) if q_block is None else [int(q_block)]
    out = np.zeros((len(blocks) * bq, nk * bkv), dtype=bool)
    for n, i in enumerate(blocks):
        rows = np.arange(i * bq, min(q_len, (i + 1) * bq))
        if rows.size:
            out[n * bq:n * bq + rows.size, :kv_len] = element_mask(
                q_len, kv_len, head, q_seg, kv_seg, rows=rows, dense=dense)
    return out


# ---------------------------------------------------------------------------
# block metadata
# ---------------------------------------------------------------------------


def next_nonempty(block_mask_row) -> np.ndarray:
    """data_next for one row of block classes.

    For each j: the smallest j' >= j whose block is not empty, or nk when
    there is none (page 3, section 21: a fully masked kv block points at the
    next valid block; the sentinel nk is the reading for "no next block").
    """
    row = np.asarray(block_mask_row)
    nk = row.shape[0]
    out = np.empty(nk, dtype=np.int32)
    for j in range(nk):
        later = [jj for jj in range(j, nk) if row[jj] != 0]
        out[j] = later[0] if later else nk
    return out


def mask_info_row(q_len: int, kv_len: int, bq: int, bkv: int, head, i: int,
                  q_seg=None, kv_seg=None, dense=None):
    """(block_mask [nk] int8, data_next [nk] int32) of query block ``i`` of one
    (batch, head).

    For block (i, j), c counts the allowed (q, k) pairs of the padded element
    mask; block_mask is 0 when c == 0, 2 when c == bq*bkv (no element mask
    needed) and 1 otherwise ("hstu_ops.py" ``_next_nonzero``: > 0 runs, != 1
    skips the element mask; the value 2 for "full" is the reading taken).
    """
    nk = -(-kv_len // bkv)
    m = padded_element_mask(q_len, kv_len, bq, bkv, head, q_seg, kv_seg, q_block=i, dense=dense)
    counts = m.reshape(bq, nk, bkv).sum(axis=(0, 2), dtype=np.int64)
    cls = np.where(counts == 0, 0, np.where(counts == bq * bkv, 2, 1)).astype(np.int8)
    return cls, next_nonempty(cls)


def _dense_heads(dense, H):
    """None, or a list of per-head boolean masks (1 broadcast, or H)."""
    if dense is None:
        return None
    d = np.asarray(dense, dtype=bool)
    if d.ndim == 2:
        d = d[None]
    if d.shape[0] not in (1, H):
        raise ValueError("need one dense mask or one per head")
    return [d[n] for n in range(d.shape[0])]


def mask_info(B: int, H: int, q_len: int, kv_len: int, bq: int, bkv: int, heads,
              q_seg=None, kv_seg=None, dense=None):
    """Block metadata (block_mask int8, data_next int32), [Bm, Hm, nq, nk].

    Hm = max(len(heads), number of dense masks) (1 broadcasts over all H
    heads, "hstu_ops.py" ``_next_nonzero`` forces the head index to 0 for
    one-head metadata); Bm = B with segment ids, else 1. Each row is
    ``mask_info_row``.
    """
    heads = [tuple(h) for h in heads]
    if len(heads) not in (1, H):
        raise ValueError("need one head mask or one per head")
    if (q_seg is None) != (kv_seg is None):
        raise ValueError("q and kv segment ids must be given together or not at all")
    dh = _dense_heads(dense, H)
    Bm = B if q_seg is not None else 1
    Hm = max(len(heads), 1 if dh is None else len(dh))
    nq = -(-q_len // bq)
    nk = -(-kv_len // bkv)
    bmask = np.zeros((Bm, Hm, nq, nk), dtype=np.int8)
    dnext = np.zeros((Bm, Hm, nq, nk), dtype=np.int32)
    for b in range(Bm):
        qs = None if q_seg is None else np.asarray(q_seg)[b]
        ks = None if kv_seg is None else np.asarray(kv_seg)[b]
        for hm in range(Hm):
            head = heads[0] if len(heads) == 1 else heads[hm]
            dm = None if dh is None else (dh[0] if len(dh) == 1 else dh[hm])
            for i in range(nq):
                bmask[b, hm, i], dnext[b, hm, i] = mask_info_row(
                    q_len, kv_len, bq, bkv, head, i, qs, ks, dense=dm)
    return bmask, dnext


def mask_info_dkv(B: int, H: int, q_len: int, kv_len: int, bq: int, bkv: int, heads,
                  q_seg=None, kv_seg=None, dense=None):
    """(block_mask, data_next) of the dK/dV pass, both [Bm, Hm, nq, nk].

    "hstu_ops.py", ``_pointwise_splash_attention_bwd_kernel``: the grid runs
    over kv blocks j, then heads, then q steps i, and the q block fetched at
    step i is ``data_next[h, i, j]`` (``_next_nonzero(..., next_i=True)``),
    from metadata that ``process_mask_dkv`` builds for the same mask. Reading:
    the classes are those of the forward (they only depend on the block's
    pairs), and ``data_next[..., i, j]`` is the first q block i' >= i of
    column j that is not empty, else nq (the sentinel read as for the
    forward's walk).
    """
    bm, _ = mask_info(B, H, q_len, kv_len, bq, bkv, heads, q_seg, kv_seg, dense=dense)
    dn = np.empty(bm.shape, dtype=np.int32)
    for b in range(bm.shape[0]):
        for h in range(bm.shape[1]):
            for j in range(bm.shape[3]):
                dn[b, h, :, j] = next_nonempty(bm[b, h, :, j])
    return bm, dn


def partial_blocks(H: int, q_len: int, kv_len: int, bq: int, bkv: int, heads, dense):
    """Element masks of the partial blocks under a dense mask, and how many
    distinct ones there are.

    Returns (blocks, distinct): ``blocks`` maps (hm, i, j) of every class-1
    block to its padded element mask [bq, bkv]; ``distinct`` is the number of
    different such masks. "hstu_ops.py" fetches the mask of a partial block
    through an index (``mask_next``, the m index map of the forward) into a
    store of [bq, bkv] mask blocks, so equal blocks can share one entry.
    """
    heads = [tuple(h) for h in heads]
    dh = _dense_heads(dense, H)
    Hm = max(len(heads), len(dh))
    nq = -(-q_len // bq)
    nk = -(-kv_len // bkv)
    blocks, seen = {}, set()
    for hm in range(Hm):
        head = heads[0] if len(heads) == 1 else heads[hm]
        dm = dh[0] if len(dh) == 1 else dh[hm]
        for i in range(nq):
            m = padded_element_mask(q_len, kv_len, bq, bkv, head, q_block=i, dense=dm)
            for j in range(nk):
                blk = m[:, j * bkv:(j + 1) * bkv]
                c = int(blk.sum())
                if 0 < c < bq * bkv:
                    blocks[(hm, i, j)] = blk.copy()
                    seen.add(blk.tobytes())
    return blocks, len(seen)


def block_flops(block_mask: np.ndarray, B: int, H: int, bq: int, bkv: int, D: int) -> int:
    """4*bq*bkv*D per non-empty block, summed over every (batch, head).

    Metadata with one head or one batch row is broadcast (counted H or B
    times)."""
    Bm, Hm = block_mask.shape[:2]
    per = np.count_nonzero(np.asarray(block_mask), axis=(2, 3))  # [Bm, Hm]
    per = np.broadcast_to(per, (B if Bm == 1 else Bm, H if Hm == 1 else Hm))
    return int(per.sum()) * 4 * bq * bkv * D


def element_flops(B: int, H: int, q_len: int, kv_len: int, D: int, heads,
                  q_seg=None, kv_seg=None, dense=None) -> int:
    """4*D per allowed (q, k) pair, summed over every (batch, head): the
    element-exact count of the two products' FLOPs (2*D for q.k and 2*D for
    p*v per allowed pair), as against ``block_flops``, which counts whole
    non-empty blocks.

    The allowed pairs of one (batch, head) are those of ``element_mask``;
    (batch, head) pairs with the same head mask, segment ids and dense mask
    have the same count, which is taken once.
    """
    heads = _heads_list(heads, H)
    dh = _dense_heads(dense, H)
    counts = {}
    total = 0
    for b in range(B):
        qs = None if q_seg is None else np.asarray(q_seg)[b]
        ks = None if kv_seg is None else np.asarray(kv_seg)[b]
        for h in range(H):
            hd = heads[0] if len(heads) == 1 else heads[h]
            hdn = None if dh is None else (0 if len(dh) == 1 else h)
            key = (hd, b if q_seg is not None else None, hdn)
            if key not in counts:
                dm = None if dh is None else dh[hdn]
                counts[key] = int(element_mask(q_len, kv_len, hd, qs, ks, dense=dm).sum())
            total += counts[key]
    return 4 * D * total


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------


def softmax_attention_rows(q_rows, k, v, scale: float, mask_rows) -> np.ndarray:
    """Masked softmax attention of some query rows, fp64.

    q_rows [R, D], k [Skv, D], v [Skv, Dv], mask_rows bool [R, Skv].
    Page 3, section 12 (naive attention) and section 15: scores = scale*q.k,
    masked scores are excluded (set to -inf, weight exactly 0), M = row max,
    Out = sum e^{a-M} v / sum e^{a-M}. A row with no allowed key returns 0
    (reading: nothing to average).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q_rows @ k.T) * float(scale)
    s = np.where(mask_rows, s, -np.inf)
    out = np.zeros((q_rows.shape[0], v.shape[1]), dtype=np.float64)
    has = np.asarray(mask_rows).any(axis=1)
    if has.any():
        sh = s[has]
        m = sh.max(axis=1, keepdims=True)
        w = np.exp(sh - m)
        out[has] = (w @ v) / w.sum(axis=1, keepdims=True)
    return out


def pointwise_attention_rows(q_rows, k, v, scale: float, mask_rows, seq_len: int) -> np.ndarray:
    """Pointwise (SiLU) attention of some query rows, fp64.

    "hstu_ops.py" ``_pointwise_splash_attention_fwd_kernel_impl``:
    x = scale*q.k; p = x * logistic(x) / seq_len with seq_len the query
    sequence length; masked entries -> 0; out = sum_k p v_k, summed over all kv
    blocks (the printed per-slice overwrite of the output is read as an
    accumulation, as the backward on the same page and page 3 section 14
    imply).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    x = (q_rows @ k.T) * float(scale)
    with np.errstate(over="ignore"):
        p = x / (1.0 + np.exp(-x)) / float(seq_len)
    p = np.where(mask_rows, p, 0.0)
    return p @ v


def online_softmax_rows(q_rows, k, v, scale: float, mask_rows, block_kv: int) -> np.ndarray:
    """The same result as ``softmax_attention_rows`` by the blockwise recurrence.

    Page 3, sections 15.1-15.3: for each kv block B after blocks A,
    m_AB = max(m_A, m_B), alpha = e^{m_A - m_AB}, L_B = sum e^{a - m_AB},
    O_B = sum e^{a - m_AB} v, L_AB = alpha L_A + L_B, O_AB = alpha O_A + O_B;
    finally Out = O / L. Excluded entries carry no weight; a row that has
    seen no allowed key yet keeps m = -inf, L = 0, O = 0.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask_rows = np.asarray(mask_rows)
    R, Skv = mask_rows.shape
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    for r in range(R):
        m_a = -np.inf
        l_a = 0.0
        o_a = np.zeros(v.shape[1], dtype=np.float64)
        for j0 in range(0, Skv, block_kv):
            sel = np.nonzero(mask_rows[r, j0:j0 + block_kv])[0] + j0
            if sel.size == 0:
                continue
            a = (k[sel] @ q_rows[r]) * float(scale)
            m_b = a.max()
            m_ab = max(m_a, m_b)
            alpha = np.exp(m_a - m_ab)          # 0 when m_a = -inf
            e = np.exp(a - m_ab)
            l_a = alpha * l_a + e.sum()
            o_a = alpha * o_a + e @ v[sel]
            m_a = m_ab
        if l_a > 0:
            out[r] = o_a / l_a
    return out


def kv_head_of(h: int, H: int, kv_heads: int) -> int:
    """KV head read by query head ``h`` when ``H`` query heads share
    ``kv_heads`` K/V heads (page 3, section 21, GQA/MQA: the K/V index map
    takes head h // q_heads_per_kv_head, with q_heads_per_kv_head = H /
    kv_heads, so consecutive query heads share a K/V head)."""
    if kv_heads < 1 or H % kv_heads:
        raise ValueError("the query heads must split evenly over the kv heads")
    return h // (H // kv_heads)


def _heads_list(heads, H):
    heads = [tuple(h) for h in heads]
    if len(heads) not in (1, H):
        raise ValueError("need one head mask or one per head")
    return heads


def _attention(kind: str, q, k, v, scale, heads, q_seg, kv_seg, row_chunk: int, dense=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Sq, _ = q.shape
    Skv = k.shape[2]
    kv_heads = k.shape[1]
    heads = _heads_list(heads, H)
    dh = _dense_heads(dense, H)
    out = np.zeros((B, H, Sq, v.shape[3]), dtype=np.float64)
    for b in range(B):
        qs = None if q_seg is None else np.asarray(q_seg)[b]
        ks = None if kv_seg is None else np.asarray(kv_seg)[b]
        for h in range(H):
            hd = heads[0] if len(heads) == 1 else heads[h]
            hk = kv_head_of(h, H, kv_heads)
            dm = None if dh is None else (dh[0] if len(dh) == 1 else dh[h])
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                m = element_mask(Sq, Skv, hd, qs, ks, rows=rows, dense=dm)
                if kind == "softmax":
                    out[b, h, rows] = softmax_attention_rows(q[b, h, rows], k[b, hk], v[b, hk], scale, m)
                else:
                    out[b, h, rows] = pointwise_attention_rows(q[b, h, rows], k[b, hk], v[b, hk], scale, m, Sq)
    return out


def softmax_attention(q, k, v, scale: float, heads, q_seg=None, kv_seg=None,
                      row_chunk: int = 512, dense=None) -> np.ndarray:
    """Masked softmax attention [B, H, Sq, Dv] (fp64); rows are independent, so
    the full-score definition is evaluated ``row_chunk`` rows at a time. k and
    v may have fewer heads than q (grouped-query attention, ``kv_head_of``)."""
    return _attention("softmax", q, k, v, scale, heads, q_seg, kv_seg, row_chunk, dense)


def pointwise_attention(q, k, v, scale: float, heads, q_seg=None, kv_seg=None,
                        row_chunk: int = 512, dense=None) -> np.ndarray:
    """Pointwise SiLU attention [B, H, Sq, Dv] (fp64), divided by Sq; k and v
    may have fewer heads than q (``kv_head_of``)."""
    return _attention("pointwise", q, k, v, scale, heads, q_seg, kv_seg, row_chunk, dense)


# ---------------------------------------------------------------------------
# pointwise backward
# ---------------------------------------------------------------------------


def _logistic(x):
    """1 / (1 + e^-x) without overflow warnings (e^-x = inf gives 0)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def pointwise_attention_bwd_rows(q_rows, k, v, do_rows, scale: float, mask_rows, seq_len: int):
    """Contributions of some query rows to the pointwise attention gradients.

    q_rows, do_rows [R, D]; k, v [Skv, D]; mask_rows bool [R, Skv]. Returns
    (dq_rows [R, D], dk [Skv, D], dv [Skv, D]): dq of these rows, and what
    these rows add to dk and dv. "hstu_ops.py",
    ``_pointwise_splash_attention_bwd_kernel_impl``, in its orientation (keys
    x queries):
      qk = scale * k q^T; sig = logistic(qk), 0 where masked;
      p = qk * sig / seq_len; dv = p do;
      dp = v do^T; ds = dp * sig * (1 + qk (1 - sig)) / seq_len;
      dk = scale * ds q; dq = scale * ds^T k.
    This is the derivative of ``pointwise_attention_rows`` (d/dx of
    x logistic(x) is logistic(x) (1 + x (1 - logistic(x)))).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do_rows = np.asarray(do_rows, dtype=np.float64)
    qk = (k @ q_rows.T) * float(scale)                    # [Skv, R]
    sig = np.where(np.asarray(mask_rows).T, _logistic(qk), 0.0)
    p = qk * sig / float(seq_len)
    dv = p @ do_rows
    dp = v @ do_rows.T
    ds = dp * sig * (1.0 + qk * (1.0 - sig)) / float(seq_len)
    dk = float(scale) * (ds @ q_rows)
    dq = float(scale) * (ds.T @ k)
    return dq, dk, dv


def pointwise_attention_bwd(q, k, v, do, scale: float, heads, q_seg=None, kv_seg=None,
                            row_chunk: int = 512, dense=None):
    """Gradients (dq [B, H, Sq, D], dk, dv [B, Hk, Skv, D]) of
    ``pointwise_attention`` for the output gradient ``do``, fp64.

    Query rows are taken ``row_chunk`` at a time and their contributions to dk
    and dv summed (the kernel's sum over q blocks for each kv block). With
    fewer K/V heads than query heads (``kv_head_of``), a K/V head's dk and dv
    sum over the query heads that read it. ``dense``: an optional boolean
    [Sq, Skv] or [H, Sq, Skv] mask ANDed into every head's element mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, Sq, _ = q.shape
    Skv = k.shape[2]
    kv_heads = k.shape[1]
    heads = _heads_list(heads, H)
    dh = _dense_heads(dense, H)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        qs = None if q_seg is None else np.asarray(q_seg)[b]
        ks = None if kv_seg is None else np.asarray(kv_seg)[b]
        for h in range(H):
            hd = heads[0] if len(heads) == 1 else heads[h]
            hk = kv_head_of(h, H, kv_heads)
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                dm = None if dh is None else dh[0 if len(dh) == 1 else h]
                m = element_mask(Sq, Skv, hd, qs, ks, rows=rows, dense=dm)
                a, bk, bv = pointwise_attention_bwd_rows(q[b, h, rows], k[b, hk], v[b, hk], do[b, h, rows],
                                                         scale, m, Sq)
                dq[b, h, rows] = a
                dk[b, hk] += bk
                dv[b, hk] += bv
    return dq, dk, dv


# ---------------------------------------------------------------------------
# softmax log-sum-exp and backward
# ---------------------------------------------------------------------------


def softmax_lse_rows(q_rows, k, scale: float, mask_rows) -> np.ndarray:
    """log sum_k e^{a_k} over the allowed keys of each row, a = scale q.k
    (page 3, section 15: with M the row max, log sum e^a = M + log sum
    e^{a - M}); -inf for a row with no allowed key (nothing to sum)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    a = (q_rows @ k.T) * float(scale)
    mask_rows = np.asarray(mask_rows)
    out = np.full(q_rows.shape[0], -np.inf)
    has = mask_rows.any(axis=1)
    if has.any():
        ah = np.where(mask_rows[has], a[has], -np.inf)
        m = ah.max(axis=1)
        out[has] = m + np.log(np.exp(ah - m[:, None]).sum(axis=1))
    return out


def softmax_attention_bwd_rows(q_rows, k, v, do_rows, scale: float, mask_rows):
    """Contributions of some query rows to the softmax attention gradients:
    (dq_rows, dk, dv), the derivative of ``softmax_attention_rows``.

    With P the row softmax of the allowed scores a = scale q.k (0 elsewhere,
    and 0 for a row with no allowed key), O = P v:
      dv = P^T do;  dP = do v^T;  delta = rowsum(do * O);
      dS = P (dP - delta);  dq = scale dS k;  dk = scale dS^T q.
    (d softmax: dS_j = P_j (dP_j - sum_l P_l dP_l), and sum_l P_l dP_l =
    do . O.)
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do_rows = np.asarray(do_rows, dtype=np.float64)
    mask_rows = np.asarray(mask_rows)
    a = (q_rows @ k.T) * float(scale)
    P = np.zeros_like(a)
    has = mask_rows.any(axis=1)
    if has.any():
        ah = np.where(mask_rows[has], a[has], -np.inf)
        e = np.exp(ah - ah.max(axis=1, keepdims=True))
        P[has] = e / e.sum(axis=1, keepdims=True)
    O = P @ v
    dv = P.T @ do_rows
    dP = do_rows @ v.T
    delta = (do_rows * O).sum(axis=1, keepdims=True)
    dS = P * (dP - delta)
    dq = float(scale) * (dS @ k)
    dk = float(scale) * (dS.T @ q_rows)
    return dq, dk, dv


def softmax_lse(q, k, scale: float, heads, q_seg=None, kv_seg=None, dense=None) -> np.ndarray:
    """Log-sum-exp [B, H, Sq] of every row (``softmax_lse_rows``); k may have
    fewer heads than q (``kv_head_of``); ``dense`` as for
    ``pointwise_attention_bwd``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, Sq, _ = q.shape
    Skv = k.shape[2]
    heads = _heads_list(heads, H)
    dh = _dense_heads(dense, H)
    out = np.zeros((B, H, Sq))
    for b in range(B):
        qs = None if q_seg is None else np.asarray(q_seg)[b]
        ks = None if kv_seg is None else np.asarray(kv_seg)[b]
        for h in range(H):
            hd = heads[0] if len(heads) == 1 else heads[h]
            dm = None if dh is None else dh[0 if len(dh) == 1 else h]
            m = element_mask(Sq, Skv, hd, qs, ks, dense=dm)
            out[b, h] = softmax_lse_rows(q[b, h], k[b, kv_head_of(h, H, k.shape[1])], scale, m)
    return out


def softmax_attention_bwd(q, k, v, do, scale: float, heads, q_seg=None, kv_seg=None,
                          row_chunk: int = 512, dense=None):
    """Gradients (dq [B, H, Sq, D], dk, dv [B, Hk, Skv, D]) of
    ``softmax_attention`` for the output gradient ``do``, fp64; rows are
    taken ``row_chunk`` at a time and their dk, dv contributions summed, and
    a K/V head's gradients sum over the query heads that read it; ``dense``
    as for ``pointwise_attention_bwd``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, Sq, _ = q.shape
    Skv = k.shape[2]
    kv_heads = k.shape[1]
    heads = _heads_list(heads, H)
    dh = _dense_heads(dense, H)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        qs = None if q_seg is None else np.asarray(q_seg)[b]
        ks = None if kv_seg is None else np.asarray(kv_seg)[b]
        for h in range(H):
            hd = heads[0] if len(heads) == 1 else heads[h]
            hk = kv_head_of(h, H, kv_heads)
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                dm = None if dh is None else dh[0 if len(dh) == 1 else h]
                m = element_mask(Sq, Skv, hd, qs, ks, rows=rows, dense=dm)
                a, bk, bv = softmax_attention_bwd_rows(q[b, h, rows], k[b, hk], v[b, hk], do[b, h, rows], scale, m)
                dq[b, h, rows] = a
                dk[b, hk] += bk
                dv[b, hk] += bv
    return dq, dk, dv
