"""Plain CPU oracle for Hidden Decoding's Stream-Factorized Attention (SFA).

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct reference
that the HIP path is checked against.  Only ``tests/``, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py`` may import it; the library itself never
does, and it shares no code with the HIP sources.

Everything here is float64 NumPy computed from the exact bf16 input bits.  Each
function names the passage it follows:

* "Hidden Decoding at Scale" review (romaanj.github.io), section *Method*: each
  token becomes n streams, each read from an embedding table of its own, and
  the backbone runs once over the length-nL sequence; in the majority of layers
  a position sees only its own stream (cost of order nL^2), and a few layers let
  streams see each other with the base model's (full causal) pattern; the
  intermediate streams' KV is retained so later tokens read it as context.
* arXiv 2607.08186 abstract page: SFA makes the attention cost grow roughly
  linearly in n instead of quadratically.
* Tencent/Sequential-Hidden-Decoding README, *Key Idea* items 1, 2 and 4.

Readings where the pages are silent (each listed in the design notes):
  R1 expanded position of (token t, stream s) is p = t*n + s (token-major
     interleave, stream 0 first);
  R2 table s feeds stream s;
  R3 a within-stream query sees its own position (t' <= t);
  R4 a mixing query at (t, s) sees (t, s') for s' <= s (causal in the
     interleaved order);
  R5 the softmax scale is an explicit argument;
  R6 query head h reads KV head h // (Hq / Hkv);
  R7 an out-of-range token id yields an all-zero row and raises a flag;
  R13 a sliding-window mixing layer (review, *Method*: the mixing layers
     keep the base model's pattern, sliding-window or full) has a window
     W counted in positions of the interleaved order: position i sees
     i - W < j <= i (the pages give no W; a base window of w tokens is W = n*w).

No function here is "parity unpinned": every one is pinned in
``tests/test_oracle.py`` against brute force, a library routine, a closed form
or an invariant.
"""
from __future__ import annotations

import numpy as np

WITHIN = 0  # within-stream layer
MIX = 1     # mixing layer, causal over the interleaved order (full, or with a window)


# ---------------------------------------------------------------------------
# bf16 handling
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16/int16) to float64 exactly.

    A bf16 value is the upper half of an IEEE float32, so shifting the 16 bits
    into the high half of a 32-bit word gives the float32 with the same value;
    widening float32 -> float64 is exact.
    """
    b = np.asarray(bits)
    u32 = b.astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# (1) Embedding expansion + interleave
# ---------------------------------------------------------------------------
def expanded_position(t, s, n):
    """Position of token t, stream s in the length-nL sequence (reading R1)."""
    return t * n + s


def expand_ref(ids, tables):
    """Hidden Decoding embedding expansion (review, *Method*; README *Key Idea* 1-2).

    ids    : int array [B, L] of token ids
    tables : uint16 bf16 bits [n, V, H], table s is stream s's own embedding
             table (reading R2)
    returns (out, bad): out uint16 [B, n*L, H] with
             out[b, t*n + s, :] = tables[s, ids[b, t], :]
             and ``bad`` True when some id lies outside [0, V); such a token's
             n rows are zero (reading R7).

    Pure byte copy: no floating-point arithmetic is involved.
    """
    ids = np.asarray(ids)
    tables = np.asarray(tables, dtype=np.uint16)
    B, L = ids.shape
    n, V, H = tables.shape
    out = np.zeros((B, n * L, H), dtype=np.uint16)
    bad = False
    for b in range(B):
        for t in range(L):
            tok = int(ids[b, t])
            if tok < 0 or tok >= V:
                bad = True
                continue
            for s in range(n):
                out[b, expanded_position(t, s, n), :] = tables[s, tok, :]
    return out, bad


def final_stream_rows_ref(x, n):
    """Rows of the final stream, the only positions whose next-token loss is
    taken (review, *Method*; README *Key Idea* 3): x[:, t*n + n-1, ...]."""
    x = np.asarray(x)
    L = x.shape[1] // n
    idx = [expanded_position(t, n - 1, n) for t in range(L)]
    return x[:, idx]


def cyclic_replicate_ref(tables, n_new):
    """Cyclic Replication Initialization (review, *Method*): when the number of
    streams grows, the new tables are copies of the existing ones, cycling over
    them: new table s = old table (s mod n_old)."""
    tables = np.asarray(tables)
    n_old = tables.shape[0]
    return np.stack([tables[s % n_old] for s in range(n_new)], axis=0)


# ---------------------------------------------------------------------------
# (2) The SFA visibility rule
# ---------------------------------------------------------------------------
def visible(i, j, n, mode, window=None):
    """True where key position j is visible to query position i.

    Within-stream (review, *Method*: a position sees only its own stream):
        j and i hold the same stream (j = i mod n) and j is not later than i
        (reading R3, so a query sees itself).
    Mixing, full pattern (review, *Method*: the base model's full causal
        pattern, here over the interleaved order, reading R4): j <= i.
    Mixing, sliding-window pattern (same passage; reading R13): additionally
        j > i - window.

    Works elementwise on NumPy integer arrays (broadcasting).
    """
    i = np.asarray(i)
    j = np.asarray(j)
    causal = j <= i
    if mode == WITHIN:
        if window is not None:
            raise ValueError("a window applies to mixing layers only")
        return causal & ((j % n) == (i % n))
    if mode == MIX:
        if window is None:
            return causal
        if window < 1:
            raise ValueError("window must be >= 1")
        return causal & (j > i - window)
    raise ValueError(f"unknown mode {mode}")


def count_pairs(N, n, mode, window=None):
    """Number of visible (query, key) pairs in one (batch, head) of length N,
    counted by enumerating the visibility rule (used to check the closed forms
    n*L*(L+1)/2, N*(N+1)/2 and, with a window W <= N, W(W+1)/2 + (N-W)W, and
    the review's O(nL^2) vs O(n^2 L^2) orders)."""
    j = np.arange(N)[None, :]
    total = 0
    for r0 in range(0, N, 1024):
        i = np.arange(r0, min(N, r0 + 1024))[:, None]
        total += int(np.count_nonzero(visible(i, j, n, mode, window)))
    return total


# ---------------------------------------------------------------------------
# (3) Masked softmax attention, the plain definition
# ---------------------------------------------------------------------------
def _softmax_rows(scores):
    """Row softmax of a float64 matrix whose masked entries are -inf.  Every row
    holds at least one finite entry (the query's own position)."""
    m = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - m)
    return p / p.sum(axis=1, keepdims=True)


def attention_rows(q_rows, q_pos, k, v, n, mode, scale, window=None, k_pos=None):
    """softmax(scale * q k^T + mask) v for some query rows of one head.

    q_rows : float64 [R, D]   the queries
    q_pos  : int [R]          their positions in the expanded sequence
    k, v   : float64 [Nk, D]  keys/values
    k_pos  : int [Nk]         their positions (default 0..Nk-1)
    returns (out [R, D], probs [R, Nk]) in float64.
    """
    j = (np.arange(k.shape[0]) if k_pos is None else np.asarray(k_pos))[None, :]
    mask = visible(np.asarray(q_pos)[:, None], j, n, mode, window)
    scores = scale * (q_rows @ k.T)
    scores = np.where(mask, scores, -np.inf)
    probs = _softmax_rows(scores)
    return probs @ v, probs


def prefill_ref(q, k, v, n, mode, scale, rows=None, heads=None, batches=None,
                chunk=1024, window=None):
    """Prefill SFA layer (review, *Method*; abstract; README *Key Idea*).

    q      : bf16 bits [B, N, Hq, D]; k, v : bf16 bits [B, N, Hkv, D];
             N = n*L in the interleaved order (reading R1)
    mode   : WITHIN or MIX
    window : MIX only: sliding window W (reading R13); None = full pattern
    rows   : optional int array of query positions to compute (default all)
    heads  : optional query heads (default all); batches likewise
    returns float64 [len(batches), len(rows), len(heads), D]

    Query head h reads KV head h // (Hq // Hkv) (reading R6).  Rows are handled
    ``chunk`` at a time only to bound memory; each row's arithmetic is the
    definition above, independent of the others.  Within-stream rows are taken
    one stream at a time and given only that stream's keys: the visibility
    rule removes every other key, so leaving them out changes no value (it
    only spares the work of scores that the mask discards).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    rows = np.arange(N) if rows is None else np.asarray(rows)
    heads = list(range(Hq)) if heads is None else list(heads)
    batches = list(range(B)) if batches is None else list(batches)
    out = np.zeros((len(batches), len(rows), len(heads), D))
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            g = h // G
            kf = bf16_bits_to_f64(k[b, :, g, :])
            vf = bf16_bits_to_f64(v[b, :, g, :])
            groups = [np.arange(len(rows))] if mode != WITHIN else \
                [np.nonzero(rows % n == s)[0] for s in range(n)]
            for sel in groups:
                for c0 in range(0, len(sel), chunk):
                    idx = sel[c0:c0 + chunk]
                    r = rows[idx]
                    # keys later than the last requested row are never visible
                    nk = int(r.max()) + 1
                    kp = np.arange(nk) if mode != WITHIN else np.arange(int(r[0]) % n, nk, n)
                    qf = bf16_bits_to_f64(q[b, r, h, :])
                    o, _ = attention_rows(qf, r, kf[kp], vf[kp], n, mode, scale, window, k_pos=kp)
                    out[bi, idx, hi, :] = o
    return out


# ---------------------------------------------------------------------------
# (3b) Gradients of a prefill layer (training)
# ---------------------------------------------------------------------------
def attention_backward_head(qf, kf, vf, dof, n, mode, scale, window=None, chunk=512):
    """Gradients of O = softmax(scale * Q K^T + mask) V for one query head,
    float64 in and out, written out from the definition (the review's
    *Results* numbers are training costs of the expanded sequence, so the
    layer's gradient is part of the method's cost).  For queries i, keys j:

        P = masked softmax of scale * Q K^T (rows i),   O = P V
        dV = P^T dO,   dP = dO V^T,   delta_i = sum_d dO_id O_id
        dS = P * (dP - delta)        (the softmax Jacobian applied to dP)
        dQ = scale * dS K,   dK = scale * dS^T Q

    qf, dof : [N, D] queries and upstream gradient of the output
    kf, vf  : [N, D] keys and values (positions 0..N-1)
    returns (dq [N, D], dk [N, D], dv [N, D], lse [N]) with lse_i the natural
    log of sum over visible j of exp(scale * q_i . k_j).
    """
    N = qf.shape[0]
    dq = np.zeros_like(qf)
    dk = np.zeros_like(kf)
    dv = np.zeros_like(vf)
    lse = np.zeros(N)
    j = np.arange(N)[None, :]
    for r0 in range(0, N, chunk):
        r = np.arange(r0, min(N, r0 + chunk))
        s = scale * (qf[r] @ kf.T)
        s = np.where(visible(r[:, None], j, n, mode, window), s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        p = e / z
        lse[r] = (m + np.log(z))[:, 0]
        o = p @ vf
        delta = np.sum(dof[r] * o, axis=1, keepdims=True)
        dp = dof[r] @ vf.T
        ds = p * (dp - delta)
        dq[r] = scale * (ds @ kf)
        dk += scale * (ds.T @ qf[r])
        dv += p.T @ dof[r]
    return dq, dk, dv, lse


def prefill_backward_ref(q, k, v, dout, n, mode, scale, window=None, heads=None, batches=None):
    """Gradients of a prefill SFA layer (the forward is ``prefill_ref``).

    q, dout : bf16 bits [B, N, Hq, D];  k, v : bf16 bits [B, N, Hkv, D]
    heads   : optional KV heads to compute (default all); batches likewise
    returns float64 (dq [b, N, Hq', D], dk [b, N, Hkv', D], dv [b, N, Hkv', D],
    lse [b, N, Hq']) over the selected batches and KV heads (Hq' = G * Hkv'),
    query heads in order.  dK and dV of KV head g sum the contributions of its
    G query heads (reading R6).
    """
    q, k, v, dout = (np.asarray(t) for t in (q, k, v, dout))
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    heads = list(range(Hkv)) if heads is None else list(heads)
    batches = list(range(B)) if batches is None else list(batches)
    dq = np.zeros((len(batches), N, G * len(heads), D))
    dk = np.zeros((len(batches), N, len(heads), D))
    dv = np.zeros_like(dk)
    lse = np.zeros((len(batches), N, G * len(heads)))
    for bi, b in enumerate(batches):
        for gi, g in enumerate(heads):
            kf = bf16_bits_to_f64(k[b, :, g, :])
            vf = bf16_bits_to_f64(v[b, :, g, :])
            for hh in range(G):
                h = g * G + hh
                r = attention_backward_head(bf16_bits_to_f64(q[b, :, h, :]), kf, vf,
                                            bf16_bits_to_f64(dout[b, :, h, :]), n, mode,
                                            scale, window)
                dq[bi, :, gi * G + hh] = r[0]
                dk[bi, :, gi] += r[1]
                dv[bi, :, gi] += r[2]
                lse[bi, :, gi * G + hh] = r[3]
    return dq, dk, dv, lse


# ---------------------------------------------------------------------------
# (4) Decode step over the retained KV cache
# ---------------------------------------------------------------------------
def decode_append_ref(k_cache, v_cache, k_new, v_new, tokens_before, n):
    """Retained-KV append (review, *Method* and *Limitations*: every stream's
    KV stays in the cache).  For sequence q with T = tokens_before[q] tokens
    already cached, new stream s goes to entry T*n + s.  Returns new copies."""
    kc = np.array(k_cache, dtype=np.uint16, copy=True)
    vc = np.array(v_cache, dtype=np.uint16, copy=True)
    S = kc.shape[0]
    for qi in range(S):
        T = int(tokens_before[qi])
        for s in range(n):
            kc[qi, expanded_position(T, s, n)] = k_new[qi, s]
            vc[qi, expanded_position(T, s, n)] = v_new[qi, s]
    return kc, vc


def gather_pages_ref(pool, page_table, entries):
    """Contiguous cache rows [S, entries, ...] from a paged pool: entry e of
    sequence q lives in page page_table[q, e // P], slot e % P, with P the
    page size (pool [num_pages, P, ...]).  Serving stacks keep the retained
    KV in such pages; the review's *Limitations* count the cache's size, not
    its layout, so paging is a storage choice that leaves every decode value
    unchanged."""
    pool = np.asarray(pool)
    pt = np.asarray(page_table)
    P = pool.shape[1]
    S = pt.shape[0]
    out = np.zeros((S, entries) + pool.shape[2:], dtype=pool.dtype)
    for q in range(S):
        for e in range(entries):
            out[q, e] = pool[pt[q, e // P], e % P]
    return out


def scatter_pages_ref(pool, page_table, q, e, row):
    """The inverse placement for one row: a copy of ``pool`` with entry e of
    sequence q set to ``row``."""
    pool = np.array(pool, copy=True)
    P = pool.shape[1]
    pool[int(page_table[q, e // P]), e % P] = row
    return pool


def decode_ref(q_new, k_cache, v_cache, tokens_before, n, mode, scale,
               seqs=None, window=None):
    """Decode attention for the n new stream positions of one token.

    q_new  : bf16 bits [S, n, Hq, D], query of new stream s of sequence q sits
             at position T*n + s with T = tokens_before[q]
    k_cache, v_cache : bf16 bits [S, C, Hkv, D] already holding the appended
             entries (see decode_append_ref); entries 0 .. T*n + n - 1 are live
    returns float64 [len(seqs), n, Hq, D]

    The visibility rule is the prefill one restricted to the new queries: the
    within-stream query (T, s) reads entries t'*n + s, t' <= T; the mixing
    query reads every entry up to and including T*n + s (review, *Method*;
    small-batch decode being bandwidth-bound is the review's *Notes*).  With
    ``window`` (mixing only, reading R13) it reads the entries p - W < j <= p.
    """
    q_new = np.asarray(q_new)
    S, _, Hq, D = q_new.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    seqs = list(range(S)) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), n, Hq, D))
    for si, qi in enumerate(seqs):
        T = int(tokens_before[qi])
        live = T * n + n
        pos = np.array([expanded_position(T, s, n) for s in range(n)])
        for h in range(Hq):
            g = h // G
            kf = bf16_bits_to_f64(k_cache[qi, :live, g, :])
            vf = bf16_bits_to_f64(v_cache[qi, :live, g, :])
            qf = bf16_bits_to_f64(q_new[qi, :, h, :])
            o, _ = attention_rows(qf, pos, kf, vf, n, mode, scale, window)
            out[si, :, h, :] = o
    return out


# ---------------------------------------------------------------------------
# (5) Useful work (closed forms checked against count_pairs in the tests)
# ---------------------------------------------------------------------------
def useful_flops(B, n, L, Hq, D, mode, window=None):
    """4*D FLOPs per visible (query, key) pair per query head: 2*D for the
    score, 2*D for the value accumulation."""
    N = n * L
    pairs = count_pairs(N, n, mode, window)
    return 4 * D * Hq * B * pairs
