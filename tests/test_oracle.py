"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: the pure-Python brute
force (a different formulation of the visibility rule and of the softmax), a
library routine (torch SDPA in float64, torch embedding), a closed form, an
invariant, or a number the pages state.  The ``planted`` tests plant plausible
mistakes in the oracle (on the CPU) and check that a pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute, sfa
from oracle.sfa import MIX, WITHIN

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bits(rng, shape, std=1.0):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * std)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f(bits):
    return sfa.bf16_bits_to_f64(bits)


def _sdpa_causal(qf, kf, vf, scale):
    """float64 torch SDPA, causal. qf [B, N, Hq, D], kf/vf [B, N, Hkv, D]."""
    G = qf.shape[2] // kf.shape[2]
    q = torch.from_numpy(qf).permute(0, 2, 1, 3)
    k = torch.from_numpy(kf).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    v = torch.from_numpy(vf).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                         scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


# ---------------------------------------------------------------------------
# bf16 widening
# ---------------------------------------------------------------------------
def test_bf16_known_values():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x0001, 0x7F80,
                     0x3C00], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 0.0, -0.0, 2.0 ** -133, math.inf, 2.0 ** -7]
    got = _f(bits)
    assert list(got) == want


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(1)
    b = _rand_bits(rng, (4096,), 3.0)
    t = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    assert np.array_equal(_f(b), t.numpy())


# ---------------------------------------------------------------------------
# expansion
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_expand_matches_brute(n):
    rng = np.random.default_rng(10 + n)
    V, H, B, L = 37, 6, 2, 9
    tab = rng.integers(0, 65536, size=(n, V, H), dtype=np.uint16)
    ids = rng.integers(0, V, size=(B, L))
    out, bad = oracle.expand_ref(ids, tab)
    assert not bad
    ref = brute.brute_expand(ids.tolist(), tab.tolist())
    assert out.tolist() == ref


def test_expand_layout_is_token_major_interleave():
    rng = np.random.default_rng(3)
    n, V, H, B, L = 3, 50, 8, 2, 7
    tab = rng.integers(0, 65536, size=(n, V, H), dtype=np.uint16)
    ids = rng.integers(0, V, size=(B, L))
    out, _ = oracle.expand_ref(ids, tab)
    # [B, L, n, H] view: gather every table at once with fancy indexing
    want = np.transpose(tab[:, ids], (1, 2, 0, 3)).reshape(B, n * L, H)
    assert np.array_equal(out, want)


def test_expand_n1_is_embedding():
    rng = np.random.default_rng(4)
    V, H = 100, 16
    w = _rand_bits(rng, (1, V, H), 0.02)
    ids = rng.integers(0, V, size=(3, 11))
    out, _ = oracle.expand_ref(ids, w)
    emb = torch.nn.functional.embedding(torch.from_numpy(ids),
                                        torch.from_numpy(w[0].view(np.int16)))
    assert np.array_equal(out, emb.numpy().view(np.uint16))


def test_expand_out_of_range_ids_zero_and_flag():
    rng = np.random.default_rng(5)
    tab = rng.integers(1, 65536, size=(2, 10, 4), dtype=np.uint16)
    ids = np.array([[0, 10, 3, -1]])
    out, bad = oracle.expand_ref(ids, tab)
    assert bad
    assert np.all(out[0, 2:4] == 0) and np.all(out[0, 6:8] == 0)
    assert np.array_equal(out[0, 0], tab[0, 0]) and np.array_equal(out[0, 5], tab[1, 3])


def test_final_stream_rows_and_cyclic_replication():
    x = np.arange(2 * 12 * 3).reshape(2, 12, 3)   # n=4, L=3
    fs = oracle.final_stream_rows_ref(x, 4)
    assert np.array_equal(fs, x[:, [3, 7, 11]])
    tab = np.arange(2 * 5 * 3).reshape(2, 5, 3)
    rep = oracle.cyclic_replicate_ref(tab, 4)
    assert rep.shape == (4, 5, 3)
    assert np.array_equal(rep[2], tab[0]) and np.array_equal(rep[3], tab[1])
    # n = 1: the final stream is every row
    y = np.arange(2 * 5 * 4).reshape(2, 5, 4)
    assert np.array_equal(oracle.final_stream_rows_ref(y, 1), y)
    # growth that is not a doubling: 3 -> 8 tables cycle 0,1,2,0,1,2,0,1
    tab3 = np.arange(3 * 2 * 2).reshape(3, 2, 2)
    rep8 = oracle.cyclic_replicate_ref(tab3, 8)
    assert [int(r[0, 0]) for r in rep8] == [0, 4, 8, 0, 4, 8, 0, 4]
    # 1 -> 2 -> 4 -> 8 (the pages' schedule) leaves every table a copy of table 0
    t1 = np.arange(6).reshape(1, 2, 3)
    t8 = oracle.cyclic_replicate_ref(oracle.cyclic_replicate_ref(oracle.cyclic_replicate_ref(t1, 2), 4), 8)
    assert all(np.array_equal(t, t1[0]) for t in t8)


# ---------------------------------------------------------------------------
# visibility rule: closed forms and the pages' cost orders
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,L", [(1, 1), (1, 17), (2, 64), (3, 10), (4, 33), (8, 20)])
def test_pair_count_closed_forms(n, L):
    N = n * L
    assert oracle.count_pairs(N, n, WITHIN) == n * L * (L + 1) // 2
    assert oracle.count_pairs(N, n, MIX) == N * (N + 1) // 2


def test_pair_counts_of_the_workloads():
    # tiny workload (n=2, L=64): closed forms at n*L = 128
    assert oracle.count_pairs(128, 2, WITHIN) == 4160
    assert oracle.count_pairs(128, 2, MIX) == 8256
    # n4 workload (n=4, L=1024)
    assert oracle.count_pairs(4096, 4, WITHIN) == 2_099_200
    assert oracle.count_pairs(4096, 4, MIX) == 8_390_656


def test_cost_orders_stated_on_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "cost_orders.json")))
    n = g["n"]
    L = 256
    base = oracle.count_pairs(L, 1, MIX)
    within = oracle.count_pairs(n * L, n, WITHIN)
    mix = oracle.count_pairs(n * L, n, MIX)
    # within-stream cost is exactly the linear reference
    assert within / base == g["linear_reference_ratio"]
    # full mixing tends to the dense n^2 figure: n*(nL+1)/(L+1)
    assert abs(mix / base - g["dense_attention_ratio"]) < g["dense_attention_ratio"] * 0.25 / (L + 1) * n
    assert mix / base < g["dense_attention_ratio"]
    # the whole-model costs bracket the linear reference and sit far under dense
    for r in (g["whole_model_cost_ratio_80B"], g["whole_model_cost_ratio_617B"]):
        assert g["linear_reference_ratio"] < r < g["dense_attention_ratio"]


def test_useful_flops_closed_form():
    assert oracle.useful_flops(2, 4, 64, 8, 16, WITHIN) == 4 * 16 * 8 * 2 * (4 * 64 * 65 // 2)


# ---------------------------------------------------------------------------
# attention: brute force, library routine, invariants
# ---------------------------------------------------------------------------
SHAPES = [
    # n, L, Hq, Hkv, D
    (1, 5, 1, 1, 4),
    (2, 4, 2, 1, 8),
    (3, 3, 4, 2, 4),
    (5, 2, 2, 2, 8),
    (4, 6, 4, 1, 4),
    (2, 1, 1, 1, 4),
]


def _qkv(rng, B, n, L, Hq, Hkv, D, std=1.0):
    N = n * L
    return (_rand_bits(rng, (B, N, Hq, D), std), _rand_bits(rng, (B, N, Hkv, D), std),
            _rand_bits(rng, (B, N, Hkv, D), std))


@pytest.mark.parametrize("n,L,Hq,Hkv,D", SHAPES)
@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_prefill_matches_brute_force(n, L, Hq, Hkv, D, mode):
    rng = np.random.default_rng(100 + 7 * n + L)
    q, k, v = _qkv(rng, 2, n, L, Hq, Hkv, D)
    scale = 0.7
    got = oracle.prefill_ref(q, k, v, n, mode, scale)
    ref = np.array(brute.brute_attention(_f(q).tolist(), _f(k).tolist(), _f(v).tolist(),
                                         n, mode == WITHIN, scale))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# gradients of a prefill layer
# ---------------------------------------------------------------------------
def _autograd_grads(qf, kf, vf, dof, n, mode, scale, window=None):
    """float64 torch autograd through masked softmax attention of one head."""
    N = qf.shape[0]
    q = torch.tensor(qf, requires_grad=True)
    k = torch.tensor(kf, requires_grad=True)
    v = torch.tensor(vf, requires_grad=True)
    mask = torch.tensor(sfa.visible(np.arange(N)[:, None], np.arange(N)[None, :], n, mode, window))
    s = (scale * q @ k.T).masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=1) @ v
    o.backward(torch.tensor(dof))
    lse = torch.logsumexp(s, dim=1)
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), lse.detach().numpy()


@pytest.mark.parametrize("n,L,mode,window", [(1, 9, MIX, None), (2, 6, WITHIN, None),
                                             (3, 5, MIX, None), (4, 4, MIX, 5), (2, 7, WITHIN, None)])
def test_backward_matches_autograd(n, L, mode, window):
    rng = np.random.default_rng(900 + n * 10 + L)
    N, D = n * L, 8
    qf, kf, vf, dof = (rng.standard_normal((N, D)) for _ in range(4))
    got = sfa.attention_backward_head(qf, kf, vf, dof, n, mode, 0.7, window, chunk=5)
    want = _autograd_grads(qf, kf, vf, dof, n, mode, 0.7, window)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)


def test_backward_matches_finite_differences():
    """Central differences of L = sum(dO * O) through the forward definition
    (attention_rows), entry by entry, against the backward formulas."""
    rng = np.random.default_rng(950)
    n, L, D, scale = 2, 5, 4, 0.9
    N = n * L
    qf, kf, vf, dof = (rng.standard_normal((N, D)) for _ in range(4))

    def loss(mode, qq, kk, vv):
        o, _ = sfa.attention_rows(qq, np.arange(N), kk, vv, n, mode, scale)
        return float(np.sum(dof * o))

    eps = 1e-6
    for mode in (WITHIN, MIX):
        dq, dk, dv, _ = sfa.attention_backward_head(qf, kf, vf, dof, n, mode, scale)
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            for (i, d) in ((0, 0), (3, 1), (N - 1, 3), (N // 2, 2)):
                args = [qf.copy(), kf.copy(), vf.copy()]
                args[which][i, d] += eps
                lp = loss(mode, *args)
                args[which][i, d] -= 2 * eps
                lm = loss(mode, *args)
                assert abs((lp - lm) / (2 * eps) - grad[i, d]) < 1e-7, (mode, which, i, d)


def test_backward_invariants():
    """Shifting every key by the same vector leaves each row's softmax
    unchanged (the shift adds a per-row constant to the scores), so the key
    gradients of each query row sum to zero; and with dO = V-independent
    constant rows the value gradient is the column sums of P times dO."""
    rng = np.random.default_rng(960)
    n, L, D = 3, 6, 8
    N = n * L
    qf, kf, vf, dof = (rng.standard_normal((N, D)) for _ in range(4))
    for mode in (WITHIN, MIX):
        dq, dk, dv, lse = sfa.attention_backward_head(qf, kf, vf, dof, n, mode, 0.5)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
        _, p = sfa.attention_rows(qf, np.arange(N), kf, vf, n, mode, 0.5)
        ones = np.ones((N, D))
        _, _, dv1, _ = sfa.attention_backward_head(qf, kf, vf, ones, n, mode, 0.5)
        np.testing.assert_allclose(dv1, np.repeat(p.sum(axis=0)[:, None], D, axis=1), atol=1e-12)
        s = 0.5 * qf @ kf.T
        mask = sfa.visible(np.arange(N)[:, None], np.arange(N)[None, :], n, mode)
        np.testing.assert_allclose(np.exp(np.where(mask, s, -np.inf) - lse[:, None]).sum(axis=1),
                                   1.0, atol=1e-12)


def test_backward_ref_sums_query_heads_into_kv_heads():
    rng = np.random.default_rng(970)
    n, L, Hq, Hkv, D = 2, 4, 4, 2, 8
    q, k, v = _qkv(rng, 1, n, L, Hq, Hkv, D)
    do = _rand_bits(rng, (1, n * L, Hq, D))
    dq, dk, dv, lse = oracle.prefill_backward_ref(q, k, v, do, n, MIX, 0.6)
    for g in range(Hkv):
        acc = np.zeros((n * L, D))
        for hh in range(Hq // Hkv):
            h = g * (Hq // Hkv) + hh
            r = sfa.attention_backward_head(_f(q)[0, :, h], _f(k)[0, :, g], _f(v)[0, :, g],
                                            _f(do)[0, :, h], n, MIX, 0.6)
            np.testing.assert_allclose(dq[0, :, h], r[0], atol=0)
            acc += r[1]
        np.testing.assert_allclose(dk[0, :, g], acc, atol=1e-13)


@pytest.mark.parametrize("n,L,Hq,Hkv,mode,window", [(2, 5, 4, 2, MIX, None), (3, 4, 6, 2, WITHIN, None),
                                                    (2, 6, 8, 2, MIX, 5), (1, 9, 3, 1, MIX, None)])
def test_backward_ref_gqa_matches_autograd_through_repeated_kv(n, L, Hq, Hkv, mode, window):
    """prefill_backward_ref (every head, the query heads of a group summed
    into its dK / dV) against float64 torch autograd of a whole multi-head
    layer whose K and V reach the heads through repeat_interleave over the
    head axis (query head h reads KV head h // (Hq / Hkv), reading R6):
    autograd sums the repeated copies' gradients by itself, with no per-head
    loop of the oracle's."""
    rng = np.random.default_rng(1000 + 10 * n + L + Hq)
    D, scale = 8, 0.55
    q, k, v = _qkv(rng, 1, n, L, Hq, Hkv, D)
    do = _rand_bits(rng, (1, n * L, Hq, D))
    dq, dk, dv, lse = oracle.prefill_backward_ref(q, k, v, do, n, mode, scale, window=window)
    N, G = n * L, Hq // Hkv
    qt = torch.tensor(_f(q)[0], requires_grad=True)          # [N, Hq, D]
    kt = torch.tensor(_f(k)[0], requires_grad=True)          # [N, Hkv, D]
    vt = torch.tensor(_f(v)[0], requires_grad=True)
    kr = kt.repeat_interleave(G, dim=1)                     # [N, Hq, D]
    vr = vt.repeat_interleave(G, dim=1)
    mask = torch.tensor(sfa.visible(np.arange(N)[:, None], np.arange(N)[None, :], n, mode, window))
    s = scale * torch.einsum("ihd,jhd->hij", qt, kr)
    s = s.masked_fill(~mask[None], float("-inf"))
    o = torch.einsum("hij,jhd->ihd", torch.softmax(s, dim=2), vr)
    o.backward(torch.tensor(_f(do)[0]))
    np.testing.assert_allclose(dq[0], qt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk[0], kt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv[0], vt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], torch.logsumexp(s, dim=2).T.detach().numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# sliding-window mixing (reading R13)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,W", [(1, 1), (17, 1), (17, 5), (64, 64), (64, 100), (130, 64),
                                 (4096, 1024)])
def test_window_pair_count_closed_form(N, W):
    """Row i sees min(i+1, W) keys: W(W+1)/2 + (N-W)W pairs when W <= N."""
    want = W * (W + 1) // 2 + (N - W) * W if W <= N else N * (N + 1) // 2
    assert oracle.count_pairs(N, 4, MIX, window=W) == want


def test_window_one_is_identity():
    """W = 1: each position sees only itself, so the output is its own v."""
    rng = np.random.default_rng(31)
    q, k, v = _qkv(rng, 2, 3, 11, 4, 2, 16)
    got = oracle.prefill_ref(q, k, v, 3, MIX, 0.9, window=1)
    vf = _f(v)
    want = np.repeat(vf, 2, axis=2)            # query head h reads KV head h // 2
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_window_two_is_a_logistic_blend():
    """W = 2: position i > 0 blends v_{i-1} and v_i with weights sigma(a) and
    sigma(-a), a = scale * q_i . (k_{i-1} - k_i); position 0 returns v_0."""
    rng = np.random.default_rng(32)
    n, L, scale = 2, 9, 0.6
    q, k, v = _qkv(rng, 1, n, L, 2, 1, 8)
    got = oracle.prefill_ref(q, k, v, n, MIX, scale, window=2)
    qf, kf, vf = _f(q)[0], _f(k)[0, :, 0], _f(v)[0, :, 0]
    for i in range(n * L):
        for h in range(2):
            if i == 0:
                want = vf[0]
            else:
                a = scale * float(qf[i, h] @ (kf[i - 1] - kf[i]))
                w = 1.0 / (1.0 + math.exp(-a))
                want = w * vf[i - 1] + (1.0 - w) * vf[i]
            np.testing.assert_allclose(got[0, i, h], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,L,W", [(1, 20, 3), (2, 12, 1), (2, 12, 5), (3, 8, 7), (4, 6, 24),
                                   (4, 6, 40)])
def test_window_matches_brute_force(n, L, W):
    rng = np.random.default_rng(500 + W + n)
    q, k, v = _qkv(rng, 1, n, L, 4, 2, 8)
    got = oracle.prefill_ref(q, k, v, n, MIX, 0.8, window=W)
    ref = np.array(brute.brute_attention(_f(q).tolist(), _f(k).tolist(), _f(v).tolist(),
                                         n, False, 0.8, window=W))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_window_planted_off_by_one_is_caught(monkeypatch):
    real = sfa.visible

    def wide(i, j, n, mode, window=None):     # j >= i - W: one key too many
        if window is None:
            return real(i, j, n, mode)
        return real(i, j, n, mode) | ((np.asarray(j) <= np.asarray(i)) &
                                       (np.asarray(j) == np.asarray(i) - window))

    monkeypatch.setattr(sfa, "visible", wide)
    with pytest.raises(AssertionError):
        test_window_one_is_identity()
    with pytest.raises(AssertionError):
        test_window_pair_count_closed_form(17, 5)
    monkeypatch.setattr(sfa, "visible", real)


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_n1_is_ordinary_causal_attention(mode):
    rng = np.random.default_rng(7)
    q, k, v = _qkv(rng, 2, 1, 40, 4, 2, 16)
    got = oracle.prefill_ref(q, k, v, 1, mode, 0.25)
    ref = _sdpa_causal(_f(q), _f(k), _f(v), 0.25)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 4])
def test_within_is_n_independent_causal_attentions(n):
    rng = np.random.default_rng(20 + n)
    L = 30
    q, k, v = _qkv(rng, 2, n, L, 4, 2, 16)
    got = oracle.prefill_ref(q, k, v, n, WITHIN, 0.3)
    for s in range(n):
        ref = _sdpa_causal(_f(q[:, s::n]), _f(k[:, s::n]), _f(v[:, s::n]), 0.3)
        np.testing.assert_allclose(got[:, s::n], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 8])
def test_mix_is_causal_attention_over_nL(n):
    rng = np.random.default_rng(30 + n)
    q, k, v = _qkv(rng, 1, n, 12, 4, 4, 8)
    got = oracle.prefill_ref(q, k, v, n, MIX, 0.5)
    ref = _sdpa_causal(_f(q), _f(k), _f(v), 0.5)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_softmax_rows_sum_to_one_and_respect_mask(mode):
    rng = np.random.default_rng(40)
    n, L, D = 3, 9, 8
    N = n * L
    qf = rng.standard_normal((N, D))
    kf = rng.standard_normal((N, D))
    vf = rng.standard_normal((N, D))
    _, p = oracle.attention_rows(qf, np.arange(N), kf, vf, n, mode, 1.0)
    assert np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-12)
    for i in range(N):
        t, s = divmod(i, n)
        for j in range(N):
            t2, s2 = divmod(j, n)
            if not brute.sees(t, s, t2, s2, mode == WITHIN):
                assert p[i, j] == 0.0
            else:
                assert p[i, j] > 0.0


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_v_ones_gives_ones(mode):
    rng = np.random.default_rng(41)
    q, k, _ = _qkv(rng, 1, 4, 16, 2, 1, 8, std=2.0)
    v = np.full(k.shape, 0x3F80, dtype=np.uint16)
    got = oracle.prefill_ref(q, k, v, 4, mode, 1.0)
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_k_zero_gives_prefix_means(mode):
    rng = np.random.default_rng(42)
    n, L = 3, 11
    q, _, v = _qkv(rng, 1, n, L, 2, 2, 8)
    k = np.zeros(v.shape, dtype=np.uint16)
    got = oracle.prefill_ref(q, k, v, n, mode, 1.0)
    vf = _f(v)[0]
    if mode == MIX:
        want = np.cumsum(vf, axis=0) / np.arange(1, n * L + 1)[:, None, None]
    else:
        want = np.empty_like(vf)
        for s in range(n):
            want[s::n] = np.cumsum(vf[s::n], axis=0) / np.arange(1, L + 1)[:, None, None]
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-13)


def test_stream_one_hot_values_pin_the_within_mask():
    rng = np.random.default_rng(43)
    n, L, D = 5, 7, 8
    q, k, _ = _qkv(rng, 1, n, L, 2, 1, D, std=3.0)
    v = np.zeros(k.shape, dtype=np.uint16)
    for i in range(n * L):
        v[0, i, :, i % n] = 0x3F80
    got = oracle.prefill_ref(q, k, v, n, WITHIN, 1.0)
    for i in range(n * L):
        want = np.zeros(D)
        want[i % n] = 1.0
        np.testing.assert_allclose(got[0, i, 0], want, rtol=0, atol=1e-14)
        np.testing.assert_allclose(got[0, i, 1], want, rtol=0, atol=1e-14)


def test_first_token_sees_only_itself():
    rng = np.random.default_rng(44)
    n = 4
    q, k, v = _qkv(rng, 1, n, 5, 4, 2, 8)
    w = oracle.prefill_ref(q, k, v, n, WITHIN, 1.0)
    m = oracle.prefill_ref(q, k, v, n, MIX, 1.0)
    vf = _f(v)
    for h in range(4):
        for s in range(n):
            assert np.array_equal(w[0, s, h], vf[0, s, h // 2])
        assert np.array_equal(m[0, 0, h], vf[0, 0, h // 2])


def test_stream_relabel_equivariance():
    rng = np.random.default_rng(45)
    n, L = 4, 6
    q, k, v = _qkv(rng, 1, n, L, 2, 1, 8)
    perm = np.array([2, 0, 3, 1])

    def relabel(x):
        y = x.reshape(x.shape[0], L, n, *x.shape[2:])
        return y[:, :, perm].reshape(x.shape)

    a = oracle.prefill_ref(relabel(q), relabel(k), relabel(v), n, WITHIN, 1.0)
    b = relabel(oracle.prefill_ref(q, k, v, n, WITHIN, 1.0))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_row_subset_equals_full():
    rng = np.random.default_rng(46)
    n = 3
    q, k, v = _qkv(rng, 2, n, 20, 4, 2, 8)
    full = oracle.prefill_ref(q, k, v, n, MIX, 1.0)
    rows = np.array([0, 7, 31, 59])
    part = oracle.prefill_ref(q, k, v, n, MIX, 1.0, rows=rows, heads=[1, 3], batches=[1],
                              chunk=2)
    np.testing.assert_array_equal(part[0], full[1][rows][:, [1, 3]])


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def test_decode_append_positions():
    rng = np.random.default_rng(50)
    S, n, Hkv, D = 3, 4, 2, 4
    C = 6 * n
    kc = rng.integers(0, 65536, size=(S, C, Hkv, D), dtype=np.uint16)
    vc = rng.integers(0, 65536, size=(S, C, Hkv, D), dtype=np.uint16)
    kn = rng.integers(0, 65536, size=(S, n, Hkv, D), dtype=np.uint16)
    vn = rng.integers(0, 65536, size=(S, n, Hkv, D), dtype=np.uint16)
    tb = np.array([0, 2, 5])
    k2, v2 = oracle.decode_append_ref(kc, vc, kn, vn, tb, n)
    for qi in range(S):
        for e in range(C):
            t, s = divmod(e, n)
            if t == tb[qi]:
                assert np.array_equal(k2[qi, e], kn[qi, s]) and np.array_equal(v2[qi, e], vn[qi, s])
            else:
                assert np.array_equal(k2[qi, e], kc[qi, e]) and np.array_equal(v2[qi, e], vc[qi, e])


def test_page_gather_and_scatter():
    """Hand-placed pages: page size 2, sequence 0 on pages [3, 0], sequence 1
    on [1, 2]; entry e of sequence q is pool[pt[q, e // 2], e % 2]."""
    pool = np.arange(4 * 2 * 3).reshape(4, 2, 3)          # 4 pages x 2 slots x 3 values
    pt = np.array([[3, 0], [1, 2]])
    g = oracle.gather_pages_ref(pool, pt, 4)
    assert np.array_equal(g[0], np.stack([pool[3, 0], pool[3, 1], pool[0, 0], pool[0, 1]]))
    assert np.array_equal(g[1], np.stack([pool[1, 0], pool[1, 1], pool[2, 0], pool[2, 1]]))
    assert int(g[0, 2, 0]) == 0 and int(g[1, 3, 2]) == 17     # values computed by hand
    p2 = oracle.scatter_pages_ref(pool, pt, 1, 2, np.array([-1, -2, -3]))
    assert np.array_equal(p2[2, 0], [-1, -2, -3]) and np.array_equal(np.delete(p2.reshape(-1, 3), 4, 0),
                                                                     np.delete(pool.reshape(-1, 3), 4, 0))


def test_decode_window_equals_windowed_prefill_tail():
    """With a sliding window the decode rows are the last n rows of the
    windowed prefill (windows shorter than, equal to and longer than the cache)."""
    rng = np.random.default_rng(70)
    S, n, Hq, Hkv, D = 3, 3, 4, 2, 8
    tb = np.array([0, 5, 2])
    C = 7 * n
    kc = _rand_bits(rng, (S, C, Hkv, D))
    vc = _rand_bits(rng, (S, C, Hkv, D))
    qn = _rand_bits(rng, (S, n, Hq, D))
    kn = _rand_bits(rng, (S, n, Hkv, D))
    vn = _rand_bits(rng, (S, n, Hkv, D))
    k2, v2 = oracle.decode_append_ref(kc, vc, kn, vn, tb, n)
    for W in (1, 4, 7, 18, 100):
        got = oracle.decode_ref(qn, k2, v2, tb, n, MIX, 0.35, window=W)
        for qi in range(S):
            T = int(tb[qi])
            N = (T + 1) * n
            q = _rand_bits(rng, (1, N, Hq, D))
            q[0, T * n:] = qn[qi]
            ref = oracle.prefill_ref(q, k2[qi:qi + 1, :N], v2[qi:qi + 1, :N], n, MIX, 0.35, window=W)
            np.testing.assert_allclose(got[qi], ref[0, T * n:], rtol=0, atol=1e-13)
        if W == 1:   # only the query's own (just appended) entry
            G = Hq // Hkv
            for qi in range(S):
                T = int(tb[qi])
                want = np.repeat(_f(v2[qi, T * n:T * n + n]), G, axis=1)
                np.testing.assert_allclose(got[qi], want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_equals_prefill_tail(mode):
    """Decoding token T over a cache of T tokens equals the last n rows of a
    prefill over T+1 tokens, sequence by sequence (ragged T)."""
    rng = np.random.default_rng(60 + mode)
    S, n, Hq, Hkv, D = 3, 3, 4, 2, 8
    tb = np.array([0, 5, 2])
    C = 7 * n
    kc = _rand_bits(rng, (S, C, Hkv, D))
    vc = _rand_bits(rng, (S, C, Hkv, D))
    qn = _rand_bits(rng, (S, n, Hq, D))
    kn = _rand_bits(rng, (S, n, Hkv, D))
    vn = _rand_bits(rng, (S, n, Hkv, D))
    k2, v2 = oracle.decode_append_ref(kc, vc, kn, vn, tb, n)
    got = oracle.decode_ref(qn, k2, v2, tb, n, mode, 0.35)
    for qi in range(S):
        T = int(tb[qi])
        N = (T + 1) * n
        q = _rand_bits(rng, (1, N, Hq, D))
        q[0, T * n:] = qn[qi]
        ref = oracle.prefill_ref(q, k2[qi:qi + 1, :N], v2[qi:qi + 1, :N], n, mode, 0.35)
        np.testing.assert_allclose(got[qi], ref[0, T * n:], rtol=0, atol=1e-13)


def test_decode_matches_brute_force():
    rng = np.random.default_rng(70)
    S, n, Hq, Hkv, D, T = 1, 2, 2, 1, 4, 3
    C = (T + 1) * n
    kc = _rand_bits(rng, (S, C, Hkv, D))
    vc = _rand_bits(rng, (S, C, Hkv, D))
    qn = _rand_bits(rng, (S, n, Hq, D))
    tb = np.array([T])
    for mode in (WITHIN, MIX):
        got = oracle.decode_ref(qn, kc, vc, tb, n, mode, 1.0)
        q = np.zeros((1, C, Hq, D), dtype=np.uint16)
        q[0, T * n:] = qn[0]
        ref = np.array(brute.brute_attention(_f(q).tolist(), _f(kc).tolist(),
                                             _f(vc).tolist(), n, mode == WITHIN, 1.0))
        np.testing.assert_allclose(got[0], ref[0, T * n:], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin above
# ---------------------------------------------------------------------------
def _pins_pass():
    """Run a compact subset of the pins against the (possibly patched) oracle."""
    try:
        test_prefill_matches_brute_force(3, 3, 4, 2, 4, WITHIN)
        test_prefill_matches_brute_force(3, 3, 4, 2, 4, MIX)
        test_within_is_n_independent_causal_attentions(3)
        test_mix_is_causal_attention_over_nL(3)
        test_pair_count_closed_forms(4, 33)
        test_decode_equals_prefill_tail(WITHIN)
    except AssertionError:
        return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    assert _pins_pass()
    real = sfa.visible

    def strict(i, j, n, mode, window=None):         # forgets the query's own position
        return real(i, j, n, mode, window) & (np.asarray(j) != np.asarray(i))

    def no_stream(i, j, n, mode, window=None):      # within-stream without the stream test
        return np.asarray(j) <= np.asarray(i)

    def token_stream(i, j, n, mode, window=None):   # stream taken as i // n
        i, j = np.asarray(i), np.asarray(j)
        c = j <= i
        return c & ((j // n) == (i // n)) if mode == WITHIN else c

    def anti(i, j, n, mode, window=None):           # causality reversed
        return real(j, i, n, mode, window)

    for bad in (strict, no_stream, token_stream, anti):
        monkeypatch.setattr(sfa, "visible", bad)
        # a planted mask can leave a row with no visible key (a NaN row)
        with np.errstate(invalid="ignore"):
            assert not _pins_pass(), bad.__name__
        monkeypatch.setattr(sfa, "visible", real)

    real_softmax = sfa._softmax_rows

    def no_norm(s):                    # drops the denominator
        return np.exp(s - s.max(axis=1, keepdims=True))

    monkeypatch.setattr(sfa, "_softmax_rows", no_norm)
    assert not _pins_pass()
    monkeypatch.setattr(sfa, "_softmax_rows", real_softmax)

    real_widen = sfa.bf16_bits_to_f64

    def low_half(bits):                # bf16 bits read as the low half
        return (np.asarray(bits).astype(np.uint32)).view(np.float32).astype(np.float64)

    monkeypatch.setattr(sfa, "bf16_bits_to_f64", low_half)
    try:
        test_bf16_known_values()
        caught = False
    except AssertionError:
        caught = True
    monkeypatch.setattr(sfa, "bf16_bits_to_f64", real_widen)
    assert caught
    assert _pins_pass()
