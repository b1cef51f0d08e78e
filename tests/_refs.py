"""Oracle results for the GPU parity tests, paired with the magnitude sums
that the max-abs part of the floating-point bar needs (``tests/_check``).

For each call the oracle runs twice on the same bits: once as given, and once
with |V| in place of V, which yields sum_j p_j |v_j| for every output element
(the weights p are the same; only the values lose their sign).  The GPU path
rounds each p_j to bf16 before the value product, so that sum bounds what
those roundings can move the output.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

import oracle
from tests._check import abs_bits

THREADS = min(16, os.cpu_count() or 1)


def prefill_pair(q, k, v, n, mode, scale, **kw):
    return (oracle.prefill_ref(q, k, v, n, mode, scale, **kw),
            oracle.prefill_ref(q, k, abs_bits(v), n, mode, scale, **kw))


def decode_pair(q_new, k_cache, v_cache, tokens_before, n, mode, scale, **kw):
    return (oracle.decode_ref(q_new, k_cache, v_cache, tokens_before, n, mode, scale, **kw),
            oracle.decode_ref(q_new, k_cache, abs_bits(v_cache), tokens_before, n, mode, scale, **kw))


def pool_map(fn, units):
    """fn over units in a thread pool, one BLAS thread per worker."""
    with threadpool_limits(1):
        with ThreadPoolExecutor(THREADS) as ex:
            return list(ex.map(fn, units))


def prefill_pair_all(qb, kb, vb, n, mode, scale, window=None, batches=None, heads=None):
    """prefill_pair over every (batch, head) unit in parallel -> two arrays
    [B', N, H', D] (bits in, as numpy uint16)."""
    batches = list(range(qb.shape[0])) if batches is None else list(batches)
    heads = list(range(qb.shape[2])) if heads is None else list(heads)
    units = [(bi, hi) for bi in range(len(batches)) for hi in range(len(heads))]
    res = pool_map(lambda u: prefill_pair(qb, kb, vb, n, mode, scale, window=window,
                                          batches=[batches[u[0]]], heads=[heads[u[1]]]), units)
    shape = (len(batches), qb.shape[1], len(heads), qb.shape[3])
    ref, ref_abs = np.empty(shape), np.empty(shape)
    for (bi, hi), (r, ra) in zip(units, res):
        ref[bi, :, hi] = r[0, :, 0]
        ref_abs[bi, :, hi] = ra[0, :, 0]
    return ref, ref_abs
