"""Plain fp64 CPU oracle for prefix-masked attention and its split-KV form.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, constants or helpers with the HIP
library; it depends on numpy alone (plus ``math`` for the brute force).

What is computed, and where the pages fix it
--------------------------------------------
* Page "Rewrite prefix key-padding masks as k/v truncation to keep SDPA on the
  flash path (PyTorch)" (google-research/tabfm PR #80), section "Fix": when the
  key-padding mask is a prefix (the first n key rows valid), masking the
  remaining keys gives exactly the same attention as cutting k and v down to
  their first n rows and attending with no mask.  Section "Tests" adds that a
  ragged mask (a different n per batch element) equals per-element truncated
  forwards.  So the oracle is the plain softmax-attention definition applied
  to the truncated keys, one batch element at a time -- not an online or
  tiled algorithm.
* Page "Add sequence-parallel multi-GPU inference (PyTorch and JAX) and a cuDNN
  flash attention option" (google-research/tabfm PR #81), section
  "Sequence-parallel inference": partial attention results over disjoint key
  sets are merged exactly with log-sum-exp weights, and unequal key sets are
  allowed; the JAX variant walks the keys in chunks.  ``ref_splitkv_partial``
  and ``ref_lse_combine`` state that merge directly.
* Same page, section "cuDNN flash attention (JAX backend)": a boolean prefix
  mask is equivalent to one valid-key count per batch element, which is the
  ``kv_len`` argument used here.

Readings where the pages are silent (each is listed in the design notes):
* the log-sum-exp statistic is the natural log of sum_j exp(scale * q.k_j) over
  the valid keys;
* n = 0 (an all-False mask row) gives out = 0 and lse = -inf, and so does an
  empty chunk and a merge in which every partial is -inf;
* ``scale`` is rounded to fp32 first, because the kernels receive an fp32;
* every query row is valid (no causal mask) and T_q is independent of S;
* the backward pass (gradients for training on ragged, packed batches) is the
  exact derivative of the forward above with respect to q, k and v; padded key
  slots do not enter the function, so their gradient is exactly zero, and a row
  block with n = 0 (constant output 0) has zero gradients everywhere.

Parity pins for every function live in ``tests/test_oracle_pins.py``; none of
the functions here is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "ref_prefix_bwd",
    "ref_prefix_mask_to_kv_len",
    "scale64",
    "ref_prefix_fwd",
    "ref_splitkv_partial",
    "ref_lse_combine",
    "brute_force",
    "num_chunks",
]

# Query rows handled per block: bounds the [rows, n] score block kept in memory.
_ROW_BLOCK = 1024


def scale64(scale: float) -> float:
    """The softmax scale as the kernels see it: rounded to fp32, then widened."""
    return float(np.float64(np.float32(scale)))


def _attend_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, s64: float):
    """Softmax attention of query rows ``q`` [T, D] over keys ``k``/``v`` [n, D].

    Plain definition, two passes with the exact row maximum:
        scores = s64 * q k^T ; m = rowmax ; e = exp(scores - m) ; z = rowsum(e)
        out = (e v) / z ; lse = m + ln z
    With n == 0 the result is out = 0, lse = -inf.
    """
    t, d = q.shape
    n = k.shape[0]
    out = np.zeros((t, v.shape[1]), dtype=np.float64)
    lse = np.full((t,), -np.inf, dtype=np.float64)
    if n == 0 or t == 0:
        return out, lse
    kt = k.T  # [D, n]
    for r0 in range(0, t, _ROW_BLOCK):
        r1 = min(t, r0 + _ROW_BLOCK)
        scores = s64 * (q[r0:r1] @ kt)  # [rows, n]
        m = scores.max(axis=1, keepdims=True)
        e = np.exp(scores - m)
        z = e.sum(axis=1, keepdims=True)
        out[r0:r1] = (e @ v) / z
        lse[r0:r1] = (m + np.log(z))[:, 0]
    return out, lse


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def ref_prefix_fwd(q, k, v, kv_len, scale: float):
    """Prefix-masked attention forward (the truncation identity of PR #80, "Fix").

    q: [B, H, T_q, D]; k, v: [B, H, S, D]; kv_len: [B] ints with 0 <= n_b <= S.
    Returns (out [B, H, T_q, D] fp64, lse [B, H, T_q] fp64).

    Keys are sliced to their first n_b rows *before* any arithmetic, so the
    contents of the padded slots can never reach the result.  Any subset of
    query rows may be passed in ``q``: rows are independent, so the result for
    a subset is the matching subset of the full result.
    """
    q = _as64(q)
    b_, h_, t_, d_ = q.shape
    kv_len = np.asarray(kv_len).reshape(-1)
    assert kv_len.shape[0] == b_, "kv_len needs one entry per batch element"
    assert k.shape[:2] == (b_, h_) and v.shape[:3] == k.shape[:3]
    s_slots = k.shape[2]
    s64 = scale64(scale)
    out = np.zeros((b_, h_, t_, v.shape[3]), dtype=np.float64)
    lse = np.full((b_, h_, t_), -np.inf, dtype=np.float64)
    for b in range(b_):
        n = int(kv_len[b])
        assert 0 <= n <= s_slots, f"kv_len[{b}]={n} outside [0, {s_slots}]"
        for h in range(h_):
            kk = _as64(k[b, h, :n])
            vv = _as64(v[b, h, :n])
            out[b, h], lse[b, h] = _attend_one(q[b, h], kk, vv, s64)
    return out, lse


def num_chunks(s_slots: int, chunk: int) -> int:
    """Number of key chunks covering the S allocated slots (ceil(S / chunk))."""
    return -(-s_slots // chunk)


def ref_splitkv_partial(q, k, v, kv_len, scale: float, chunk: int):
    """Per-chunk partial attention (PR #81, "Sequence-parallel inference").

    Chunk c covers keys [c*chunk, min((c+1)*chunk, n_b)).  For each chunk the
    result is the *normalized* partial output O_c and its statistic L_c (the
    natural-log LSE over that chunk's keys).  An empty chunk gives (0, -inf).
    Returns (part_out [B, H, C, T_q, D], part_lse [B, H, C, T_q]), fp64.
    """
    q = _as64(q)
    b_, h_, t_, d_ = q.shape
    s_slots = k.shape[2]
    c_ = num_chunks(s_slots, chunk)
    kv_len = np.asarray(kv_len).reshape(-1)
    s64 = scale64(scale)
    part_out = np.zeros((b_, h_, c_, t_, v.shape[3]), dtype=np.float64)
    part_lse = np.full((b_, h_, c_, t_), -np.inf, dtype=np.float64)
    for b in range(b_):
        n = int(kv_len[b])
        assert 0 <= n <= s_slots
        for h in range(h_):
            for c in range(c_):
                lo = c * chunk
                hi = min((c + 1) * chunk, n)
                if hi <= lo:
                    continue  # empty chunk: (0, -inf) as initialised
                kk = _as64(k[b, h, lo:hi])
                vv = _as64(v[b, h, lo:hi])
                part_out[b, h, c], part_lse[b, h, c] = _attend_one(q[b, h], kk, vv, s64)
    return part_out, part_lse


def ref_lse_combine(part_out, part_lse, axis: int = 2):
    """Exact log-sum-exp merge of partials over ``axis`` (PR #81).

    Accepts any partition of the keys into parts, equal or not, including empty
    parts (L = -inf).  With M = max_c L_c:
        M == -inf          -> out = 0, lse = -inf
        otherwise  w_c = exp(L_c - M), W = sum_c w_c,
                   out = sum_c w_c O_c / W, lse = M + ln W.
    part_out has the part axis at ``axis`` and D last; part_lse has the same
    shape without D.
    """
    po = np.moveaxis(_as64(part_out), axis, 0)  # [C, ..., D]
    pl = np.moveaxis(_as64(part_lse), axis, 0)  # [C, ...]
    m = pl.max(axis=0)  # [...]
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.where(np.isneginf(pl), 0.0, np.exp(pl - m_safe[None]))  # [C, ...]
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    out = (w[..., None] * po).sum(axis=0) / wsum_safe[..., None]
    out = np.where(empty[..., None], 0.0, out)
    lse = np.where(empty, -np.inf, m_safe + np.log(wsum_safe))
    return out, lse


def _grad_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, s64: float):
    """Gradients of out = softmax(s64 * q k^T) v for one (b, h), keys already truncated.

    Plain definition, in query-row blocks (dk and dv sum over the blocks):
        P = softmax(s64 q k^T) ; dv = P^T dout ; dP = dout v^T
        delta = rowsum(P * dP)  (equal to rowsum(dout * out))
        dS = P * (dP - delta) ; dq = s64 dS k ; dk = s64 dS^T q
    With n == 0 every gradient is zero.
    """
    t = q.shape[0]
    n = k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if n == 0 or t == 0:
        return dq, dk, dv
    for r0 in range(0, t, _ROW_BLOCK):
        r1 = min(t, r0 + _ROW_BLOCK)
        scores = s64 * (q[r0:r1] @ k.T)
        e = np.exp(scores - scores.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        do = dout[r0:r1]
        dv += p.T @ do
        dp = do @ v.T
        delta = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[r0:r1] = s64 * (ds @ k)
        dk += s64 * (ds.T @ q[r0:r1])
    return dq, dk, dv


def ref_prefix_bwd(q, k, v, kv_len, scale: float, dout):
    """Backward of the prefix-masked forward: returns (dq, dk, dv) in fp64.

    Shapes as in ``ref_prefix_fwd``; dout is [B, H, T_q, D].  Keys are sliced to
    their first n_b rows before any arithmetic, so dk and dv are exactly zero on
    the padded slots j >= n_b whatever those slots hold (the truncation identity
    of PR #80, section Fix, carried to the gradients).
    """
    q = _as64(q)
    dout = _as64(dout)
    b_, h_, t_, d_ = q.shape
    kv_len = np.asarray(kv_len).reshape(-1)
    assert kv_len.shape[0] == b_
    s_slots = k.shape[2]
    s64 = scale64(scale)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(b_):
        n = int(kv_len[b])
        assert 0 <= n <= s_slots
        for h in range(h_):
            gq, gk, gv = _grad_one(q[b, h], _as64(k[b, h, :n]), _as64(v[b, h, :n]), dout[b, h], s64)
            dq[b, h] = gq
            dk[b, h, :n] = gk
            dv[b, h, :n] = gv
    return dq, dk, dv


def ref_prefix_mask_to_kv_len(mask):
    """Lengths of prefix key-padding masks, or -1 for rows that are not prefixes.

    The page on tabfm PR #80 (section Fix) rewrites a boolean key mask only when its
    valid keys are exactly the first n rows; PR #81 (section cuDNN flash attention)
    maps such masks onto one length per batch element.  mask: [B, S] or [B, 1, 1, S]
    booleans, True = attend.  Row b gives n_b = the number of leading True entries if
    every later entry is False, and -1 otherwise (a hole, or a True after a False).
    An all-False row is a valid prefix of length 0.
    """
    m = np.asarray(mask).astype(bool)
    m = m.reshape(m.shape[0], -1)
    out = np.empty(m.shape[0], dtype=np.int64)
    for b in range(m.shape[0]):
        row = m[b].tolist()
        n = 0
        while n < len(row) and row[n]:
            n += 1
        out[b] = n if not any(row[n:]) else -1
    return out


def brute_force(q, k, v, kv_len, scale: float):
    """Pure-Python prefix-masked attention for tiny shapes (no numpy arithmetic).

    Nested loops over (b, h, i); for each query row the valid keys j < n_b are
    scored, exponentiated against the row maximum with ``math.exp`` and summed
    with ``math.fsum``.  Returns nested lists (out[b][h][i][d], lse[b][h][i]).
    """
    q = np.asarray(q, dtype=np.float64).tolist()
    k = np.asarray(k, dtype=np.float64).tolist()
    v = np.asarray(v, dtype=np.float64).tolist()
    lens = [int(x) for x in np.asarray(kv_len).reshape(-1)]
    s64 = scale64(scale)
    outs, lses = [], []
    for b, qb in enumerate(q):
        n = lens[b]
        ob, lb = [], []
        for h, qbh in enumerate(qb):
            oh, lh = [], []
            dv = len(v[b][h][0]) if len(v[b][h]) else len(qbh[0]) if qbh else 0
            for qi in qbh:
                if n == 0:
                    oh.append([0.0] * dv)
                    lh.append(-math.inf)
                    continue
                sc = [s64 * math.fsum(a * c for a, c in zip(qi, k[b][h][j])) for j in range(n)]
                mx = max(sc)
                ex = [math.exp(x - mx) for x in sc]
                z = math.fsum(ex)
                oh.append([math.fsum(ex[j] * v[b][h][j][d] for j in range(n)) / z for d in range(dv)])
                lh.append(mx + math.log(z))
            ob.append(oh)
            lb.append(lh)
        outs.append(ob)
        lses.append(lb)
    return outs, lses
