"""Plain float64 CPU oracle for grouped-query attention with a learned per-head softmax sink.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. The HIP library never calls it, shares no code with it, and
this module imports nothing from the HIP package.

What it computes (source: the blog post "GPT-OSS on Day 0", Perplexity, 2025; section "Kernels for
GPT-OSS", subsection "Sink attention"):

* The sink-attention formula: every attention head owns one learned scalar, its sink, that enters
  the softmax taken over the scaled query-key products; the softmax output then weights V.
* The max-subtracted ("safe") softmax identity that the same subsection states.
* The online form described there: a running maximum ``m`` and a running scale ``d`` per query
  row, with ``m`` started at the head's sink value so the sink lands in the denominator once.
* When attention is split into blocks along the KV sequence, the sink is taken into the first
  chunk only.

Readings taken where the page is silent or garbled (each one is also listed in the design notes):

* The sink is ONE extra logit per head appended to each score row; it has no value vector, so its
  column is dropped after the softmax and the remaining weights are not renormalised.  (The formula
  as printed adds the sink to every logit, which a softmax would ignore; the initialisation
  paragraph, m := sink with d := 1, puts exactly one term e^(sink - m) in the denominator.)
* The sink is not multiplied by the softmax scale (operator order in the printed formula; the
  initialisation compares it directly with the running max of scaled logits).
* Exponentials are natural (the page writes e^x).  ``lse`` and the chunk maxima are natural-log.
* GQA: query head h reads KV head floor(h / G), G = Hq / Hkv (contiguous groups).
* Causal masking is bottom-right aligned: query i of a sequence with Lq queries and Lk keys sees
  keys j <= i + (Lk - Lq).  Decode (one query) sees every cached key below its length.
* A row with no key and a finite sink puts all its weight on the value-less sink: out = 0.  A row
  whose every term is -inf (no key and sink = -inf) is defined as out = 0, lse = -inf.
* Split-KV state per chunk is (m, d, o): m the chunk's max logit (with the sink when the chunk is
  the first), d = sum of e^(z - m) over the chunk's terms, o = the chunk's softmax-weighted mean of
  V.  An empty chunk that is not the first is (-inf, 0, 0).  Merging weighs chunk c by
  d_c * e^(m_c - M), M the largest m_c (the log-sum-exp merge).  Prefill split along the KV length
  follows the same first-chunk rule: only split 0 of a sequence carries the sink.

Every function here is pinned by tests that do not call back into it for their expected values:
closed forms, a 50-digit brute force, the float64 PyTorch SDPA library routine, identities, and
invariances.  No function is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def sink_softmax(z, sink):
    """Softmax over the row ``[z_0 .. z_{n-1}, sink]`` with the sink column then dropped.

    Follows the safe-softmax identity of the "Sink attention" subsection: subtract the row max,
    exponentiate, divide by the sum.

    z:    float64 ``[..., n]`` scaled logits; masked entries are ``-inf``.
    sink: float64 scalar or array broadcastable to ``z.shape[:-1]``; finite or ``-inf``.
    Returns ``(p [..., n], p_sink [...], lse [...])`` where ``p`` are the key weights,
    ``p_sink`` the weight the sink absorbed and ``lse`` = log of the full denominator.
    A row whose every term is ``-inf`` returns zeros and ``lse = -inf``.
    """
    z = _f64(z)
    sink = np.broadcast_to(_f64(sink), z.shape[:-1])
    full = np.concatenate([z, sink[..., None]], axis=-1)
    row_max = full.max(axis=-1)
    dead = np.isneginf(row_max)
    shift = np.where(dead, 0.0, row_max)
    e = np.exp(full - shift[..., None])
    total = e.sum(axis=-1)
    safe_total = np.where(dead, 1.0, total)
    p_full = np.where(dead[..., None], 0.0, e / safe_total[..., None])
    lse = np.where(dead, NEG_INF, shift + np.log(safe_total))
    return p_full[..., :-1], p_full[..., -1], lse


def attend(q_rows, keys, values, sink, scale, allowed=None):
    """Sink attention for a block of query rows of one head against one KV head.

    q_rows [n, D]; keys, values [L, D]; sink scalar; allowed: optional bool [n, L] mask.
    Returns ``(out [n, D], lse [n])``.  Step order is the page's formula: scaled Q.K^T, mask,
    append the sink, softmax, drop the sink column, weight V.
    """
    q_rows, keys, values = _f64(q_rows), _f64(keys), _f64(values)
    z = scale * (q_rows @ keys.T)
    if allowed is not None:
        z = np.where(allowed, z, NEG_INF)
    p, _, lse = sink_softmax(z, sink)
    return p @ values, lse


def causal_allowed(rows, num_q: int, num_k: int) -> np.ndarray:
    """Bottom-right causal mask: query ``i`` (0-based in its sequence) may see keys ``j <= i + num_k - num_q``."""
    rows = np.asarray(rows, dtype=np.int64)
    return np.arange(num_k)[None, :] <= (rows[:, None] + (num_k - num_q))


def _group(num_q_heads: int, num_kv_heads: int) -> int:
    if num_kv_heads <= 0 or num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    return num_q_heads // num_kv_heads


def prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal=True, row_block=512):
    """Varlen (packed) prefill: every sequence b attends its own keys only.

    q [Tq, Hq, D]; k, v [Tk, Hkv, D]; sinks [Hq]; cu_seqlens_q/k [B+1] prefix sums of lengths.
    Returns ``(out [Tq, Hq, D], lse [Tq, Hq])`` in float64.  Rows are processed in blocks of
    ``row_block`` only to bound memory; rows are independent, so this changes no arithmetic.
    """
    q, k, v, sinks = _f64(q), _f64(k), _f64(v), _f64(sinks)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    t_q, h_q, dim = q.shape
    group = _group(h_q, k.shape[1])
    out = np.zeros((t_q, h_q, dim))
    lse = np.full((t_q, h_q), NEG_INF)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        n_q, n_k = q1 - q0, k1 - k0
        for h in range(h_q):
            g = h // group
            keys, values = k[k0:k1, g], v[k0:k1, g]
            for r0 in range(0, n_q, row_block):
                rows = np.arange(r0, min(r0 + row_block, n_q))
                allowed = causal_allowed(rows, n_q, n_k) if causal else None
                o, l = attend(q[q0 + rows, h], keys, values, sinks[h], scale, allowed)
                out[q0 + rows, h] = o
                lse[q0 + rows, h] = l
    return out, lse


def prefill_at(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal, tokens, heads):
    """The prefill output at selected (token, head) pairs only, one row at a time.

    Used to check full-size problems where the whole output would take the CPU too long.
    Returns ``(out [n, D], lse [n])`` for ``n = len(tokens)`` pairs.
    """
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    h_q = q.shape[1]
    group = _group(h_q, k.shape[1])
    outs, lses = [], []
    for t, h in zip(np.asarray(tokens).tolist(), np.asarray(heads).tolist()):
        b = int(np.searchsorted(cu_q, t, side="right") - 1)
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        g = h // group
        allowed = causal_allowed([t - q0], q1 - q0, k1 - k0) if causal else None
        o, l = attend(_f64(q[t, h])[None], _f64(k[k0:k1, g]), _f64(v[k0:k1, g]),
                      float(sinks[h]), scale, allowed)
        outs.append(o[0])
        lses.append(l[0])
    return np.array(outs), np.array(lses)


def decode(q, k, v, sinks, seqlens_k, scale):
    """Single-token decode against a KV cache, unsplit.

    q [B, Hq, D]; k, v [B, Lcap, Hkv, D]; seqlens_k [B] (keys ``0 .. len_b - 1`` are valid).
    Returns ``(out [B, Hq, D], lse [B, Hq])``.
    """
    q, sinks = _f64(q), _f64(sinks)
    batch, h_q, dim = q.shape
    group = _group(h_q, k.shape[2])
    out = np.zeros((batch, h_q, dim))
    lse = np.full((batch, h_q), NEG_INF)
    for b in range(batch):
        n = int(seqlens_k[b])
        for h in range(h_q):
            g = h // group
            o, l = attend(q[b, h][None], _f64(k[b, :n, g]), _f64(v[b, :n, g]), sinks[h], scale)
            out[b, h], lse[b, h] = o[0], l[0]
    return out, lse


def chunk_state(z, values, sink=None):
    """Softmax state ``(m, d, o)`` of one KV chunk of one query row.

    z [L] scaled logits (L may be 0), values [L, D]; ``sink`` is the head's sink logit when this
    is the first chunk (the only chunk that carries it) and ``None`` otherwise.
    m = max of the chunk's terms, d = sum of e^(term - m), o = (sum_j e^(z_j - m) v_j) / d.
    A chunk with no finite term is ``(-inf, 0, 0)``.
    """
    z, values = _f64(z), _f64(values)
    terms = z if sink is None else np.append(z, float(sink))
    if terms.size == 0 or np.isneginf(terms.max()):
        return NEG_INF, 0.0, np.zeros(values.shape[-1])
    m = float(terms.max())
    e = np.exp(z - m)
    d = float(e.sum()) + (math.exp(float(sink) - m) if sink is not None else 0.0)
    return m, d, (e @ values) / d


def chunk_size(capacity: int, num_chunks: int) -> int:
    """Keys per chunk: ceil(capacity / num_chunks)."""
    return -(-int(capacity) // int(num_chunks))


def decode_split(q, k, v, sinks, seqlens_k, num_chunks, scale):
    """Split-KV decode partials: chunk ``c`` covers keys ``[c*cs, min((c+1)*cs, len))``.

    The sink is folded into chunk 0 only, whatever the sequence length (the first-chunk rule).
    Returns ``(partial_o [B, Hq, C, D], partial_m [B, Hq, C], partial_d [B, Hq, C])``.
    """
    q, sinks = _f64(q), _f64(sinks)
    batch, h_q, dim = q.shape
    cap = k.shape[1]
    group = _group(h_q, k.shape[2])
    cs = chunk_size(cap, num_chunks)
    po = np.zeros((batch, h_q, num_chunks, dim))
    pm = np.full((batch, h_q, num_chunks), NEG_INF)
    pd = np.zeros((batch, h_q, num_chunks))
    for b in range(batch):
        n = int(seqlens_k[b])
        for h in range(h_q):
            g = h // group
            for c in range(num_chunks):
                lo, hi = c * cs, min((c + 1) * cs, n)
                keys = _f64(k[b, lo:hi, g]) if hi > lo else np.zeros((0, dim))
                vals = _f64(v[b, lo:hi, g]) if hi > lo else np.zeros((0, dim))
                z = scale * (keys @ q[b, h])
                m, d, o = chunk_state(z, vals, sinks[h] if c == 0 else None)
                po[b, h, c], pm[b, h, c], pd[b, h, c] = o, m, d
    return po, pm, pd


def decode_multi(q, k, v, sinks, seqlens_k, scale):
    """Multi-token decode: the last T rows of each sequence, against a KV cache that holds them.

    q [B, T, Hq, D]; k, v [B, Lcap, Hkv, D]; seqlens_k [B] counts the T new tokens. Token t of
    sequence b is query row t of a block of T queries against L = seqlens_k[b] keys, under the
    bottom-right causal rule: it sees keys j <= L - T + t.
    Returns ``(out [B, T, Hq, D], lse [B, T, Hq])``.
    """
    q, sinks = _f64(q), _f64(sinks)
    batch, q_len, h_q, dim = q.shape
    group = _group(h_q, k.shape[2])
    out = np.zeros((batch, q_len, h_q, dim))
    lse = np.full((batch, q_len, h_q), NEG_INF)
    for b in range(batch):
        n = int(seqlens_k[b])
        allowed = causal_allowed(np.arange(q_len), q_len, n)
        for h in range(h_q):
            g = h // group
            o, l = attend(q[b, :, h], _f64(k[b, :n, g]), _f64(v[b, :n, g]), sinks[h], scale, allowed)
            out[b, :, h], lse[b, :, h] = o, l
    return out, lse


def decode_multi_split(q, k, v, sinks, seqlens_k, num_chunks, scale):
    """Split-KV partials of multi-token decode, by the chunk definition.

    Chunk ``c`` covers keys ``[c*cs, (c+1)*cs)``, cs = ceil(Lcap / C), intersected with the keys
    token t may see (``j <= L - T + t``); chunk 0 carries the sink. Row ``b*T + t`` of the
    partials holds token t of sequence b: ``(partial_o [B*T, Hq, C, D], partial_m [B*T, Hq, C],
    partial_d [B*T, Hq, C])``.
    """
    q, sinks = _f64(q), _f64(sinks)
    batch, q_len, h_q, dim = q.shape
    cap = k.shape[1]
    group = _group(h_q, k.shape[2])
    cs = chunk_size(cap, num_chunks)
    po = np.zeros((batch * q_len, h_q, num_chunks, dim))
    pm = np.full((batch * q_len, h_q, num_chunks), NEG_INF)
    pd = np.zeros((batch * q_len, h_q, num_chunks))
    for b in range(batch):
        n = int(seqlens_k[b])
        for t in range(q_len):
            seen = max(0, min(n, n - q_len + 1 + t))  # keys 0 .. seen - 1
            for h in range(h_q):
                g = h // group
                for c in range(num_chunks):
                    lo, hi = c * cs, min((c + 1) * cs, seen)
                    keys = _f64(k[b, lo:hi, g]) if hi > lo else np.zeros((0, dim))
                    vals = _f64(v[b, lo:hi, g]) if hi > lo else np.zeros((0, dim))
                    z = scale * (keys @ q[b, t, h])
                    m, d, o = chunk_state(z, vals, sinks[h] if c == 0 else None)
                    row = b * q_len + t
                    po[row, h, c], pm[row, h, c], pd[row, h, c] = o, m, d
    return po, pm, pd


def split_size(num_keys: int, num_splits: int, align: int = 64) -> int:
    """Keys per KV split of one prefill sequence: ceil(Lk / S) rounded up to a multiple of ``align``.

    A convention of the split-KV prefill call (its splits start on whole key tiles), not of the
    method: any split with the sink in split 0 merges to the same result.
    """
    per = -(-int(num_keys) // int(num_splits))
    return -(-per // align) * align


def prefill_split(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal, num_splits, align=64):
    """Split-KV prefill partials: split ``j`` of sequence b covers its keys
    ``[j*ks_b, min((j+1)*ks_b, Lk_b))`` with ``ks_b = split_size(Lk_b, S)``; a query row's state in
    a split is taken over the split's keys that the row may see (causal reading as in ``prefill``),
    with the sink in split 0 only (the first-chunk rule, applied to prefill).

    Each state is computed from its definition: the split's scaled logits, the sink column appended
    when j = 0, m = their max, d = sum of e^(term - m), o = the e^(z - m)-weighted mean of V. A split
    with no finite term is (-inf, 0, 0).
    Returns ``(partial_o [Tq, Hq, S, D], partial_m [Tq, Hq, S], partial_d [Tq, Hq, S])``.
    """
    q, k, v, sinks = _f64(q), _f64(k), _f64(v), _f64(sinks)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    t_q, h_q, dim = q.shape
    group = _group(h_q, k.shape[1])
    po = np.zeros((t_q, h_q, num_splits, dim))
    pm = np.full((t_q, h_q, num_splits), NEG_INF)
    pd = np.zeros((t_q, h_q, num_splits))
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        n_q, n_k = q1 - q0, k1 - k0
        if n_q == 0:
            continue
        ks = split_size(n_k, num_splits, align) if n_k > 0 else 1
        rows = np.arange(n_q)
        allowed = causal_allowed(rows, n_q, n_k) if causal else np.ones((n_q, n_k), dtype=bool)
        for h in range(h_q):
            g = h // group
            z = scale * (q[q0:q1, h] @ k[k0:k1, g].T)  # [n_q, n_k]
            z = np.where(allowed, z, NEG_INF)
            for j in range(num_splits):
                lo, hi = min(j * ks, n_k), min((j + 1) * ks, n_k)
                zj = z[:, lo:hi]
                terms = zj if j > 0 else np.concatenate([zj, np.full((n_q, 1), sinks[h])], axis=1)
                m = terms.max(axis=1, initial=NEG_INF)
                live = ~np.isneginf(m)
                shift = np.where(live, m, 0.0)
                e = np.exp(zj - shift[:, None])  # e^(-inf) = 0 for keys the row may not see
                d = e.sum(axis=1) + (np.exp(sinks[h] - shift) if j == 0 else 0.0)
                d = np.where(live, d, 0.0)
                o = np.where(live[:, None], (e @ v[k0 + lo:k0 + hi, g]) / np.where(live, d, 1.0)[:, None], 0.0)
                po[q0:q1, h, j], pm[q0:q1, h, j], pd[q0:q1, h, j] = o, m, d
    return po, pm, pd


def merge(partial_o, partial_m, partial_d):
    """Log-sum-exp merge of chunk states over the chunk axis (second to last of ``partial_o``).

    M = max_c m_c, w_c = d_c e^(m_c - M), out = sum_c w_c o_c / sum_c w_c,
    lse = M + ln sum_c w_c.  Chunks with m_c = -inf weigh 0; if all do, out = 0, lse = -inf.
    """
    o, m, d = _f64(partial_o), _f64(partial_m), _f64(partial_d)
    big = m.max(axis=-1)
    dead = np.isneginf(big)
    shift = np.where(dead, 0.0, big)
    w = np.where(np.isneginf(m), 0.0, d * np.exp(m - shift[..., None]))
    total = w.sum(axis=-1)
    alive = total > 0
    safe_total = np.where(alive, total, 1.0)
    out = np.where(alive[..., None], (w[..., None] * o).sum(axis=-2) / safe_total[..., None], 0.0)
    lse = np.where(alive, shift + np.log(safe_total), NEG_INF)
    return out, lse


def online_row(z_tiles, value_tiles, sink, initial_scale=1.0):
    """The page's online recurrence for one query row, tile by tile.

    State: running max ``m`` started at the head's sink value and running scale ``d`` started at
    1 (that 1 is the sink's own term e^(sink - sink)).  Per tile: m' = max(m, max z);
    alpha = e^(m - m'); p = e^(z - m'); d = alpha d + sum p; acc = alpha acc + p V.
    Returns ``(out, m, d)``.  Kept beside the plain definition so that tests can pin the page's
    initialisation rule against it; ``initial_scale`` is the starting ``d`` (1 on the page; the
    tests set 0 to check that dropping the sink's own term is caught).
    """
    m, d = float(sink), float(initial_scale)
    acc = None
    for z, vals in zip(z_tiles, value_tiles):
        z, vals = _f64(z), _f64(vals)
        if acc is None:
            acc = np.zeros(vals.shape[-1])
        if z.size == 0:
            continue
        m_new = max(m, float(z.max()))
        if np.isneginf(m_new):
            continue
        alpha = 0.0 if np.isneginf(m) else math.exp(m - m_new)
        p = np.exp(z - m_new)
        d = alpha * d + float(p.sum())
        acc = alpha * acc + p @ vals
        m = m_new
    if acc is None:
        acc = np.zeros(0)
    out = acc / d if d > 0 else np.zeros_like(acc)
    return out, m, d
