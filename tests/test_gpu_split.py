"""Key-split prefill (sfa_attn_split) against the oracle on the GPU.

A launch with no more causal work items than compute units takes each item
with two or more key tiles as two units (its first and second half of the
key tiles) on different workgroups; the second unit to finish merges the two
partial softmax states and writes the output and lse.  These tests compare
every row with the oracle over packings of 1, 2, 4 and 8 query heads, both
layer kinds, head_dim 64 and 128 and partial last tiles, the n = 1 stack
baseline layer on every row of two KV groups, and check that a second call
gives the same bits (the merge does not depend on which half finishes
last), that the workspace counters are zero again after each call, that the
grid size changes no bit, and that a launch with more items than compute
units is the plain forward, bit for bit, and leaves the workspace untouched.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import sequence_length_latent_amd as hd
import sfa_inputs as si
from tests._check import assert_close
from tests._refs import prefill_pair, prefill_pair_all

pytestmark = pytest.mark.gpu
DEV = "cuda"
WITHIN, MIX = oracle.WITHIN, oracle.MIX


def f64(t):
    return oracle.bf16_bits_to_f64(si.bits(t.cpu()))


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _split_items(B, n, L, Hq, Hkv, mode):
    """Items with two or more key tiles, restated: items cover 32 * 8 / P
    query rows of a view (P query heads packed, the largest of 8, 4, 2, 1
    dividing the group size), and an item whose rows end past key row 64
    reaches a second 64-key tile."""
    G = Hq // Hkv
    P = next(p for p in (8, 4, 2, 1) if G % p == 0)
    BT = 32 * 8 // P
    ln = L if mode == WITHIN else n * L
    per = B * (n if mode == WITHIN else 1) * Hkv * (G // P)
    qtiles = -(-ln // BT)
    return sum(per for qt in range(qtiles) if min(ln, (qt + 1) * BT) > 64)


def _counters_zero(ws, items):
    cbytes = -(-items * 8 * 4 // 256) * 256
    return bool((ws[:cbytes] == 0).all())


def _lse_ref(q, k, v, n, mode, scale):
    do = torch.zeros_like(q)
    return oracle.prefill_backward_ref(si.bits(q.cpu()), si.bits(k.cpu()), si.bits(v.cpu()),
                                       si.bits(do.cpu()), n, mode, scale)[3]


SWEEP = [
    # n, B, L, Hq, Hkv, D, mode
    (1, 1, 300, 8, 2, 128, MIX),       # P = 4, a partial last key tile
    (2, 1, 70, 4, 2, 128, WITHIN),     # P = 2: 128-row items, waves past their last tile
    (3, 2, 45, 8, 2, 64, MIX),         # head_dim 64
    (5, 1, 140, 16, 2, 128, WITHIN),   # P = 8: 32-row items
    (1, 2, 129, 2, 2, 128, MIX),       # P = 1
    (4, 1, 65, 8, 8, 128, WITHIN),
    (2, 1, 257, 8, 2, 64, WITHIN),     # odd tile counts: halves of unequal length
]


@pytest.mark.parametrize("n,B,L,Hq,Hkv,D,mode", SWEEP)
def test_split_sweep_every_row(n, B, L, Hq, Hkv, D, mode):
    seed = 9100 + 17 * n + L + Hq + D + mode
    N = n * L
    scale = D ** -0.5
    q = si.randn_bf16((B, N, Hq, D), 1.0, seed, DEV)
    k = si.randn_bf16((B, N, Hkv, D), 1.0, seed + 1, DEV)
    v = si.randn_bf16((B, N, Hkv, D), 1.0, seed + 2, DEV)
    items = _split_items(B, n, L, Hq, Hkv, mode)
    assert items > 0
    ws = hd.split_workspace(q, k, n, mode)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=DEV)
    out = hd.attn_split(q, k, v, n, scale, mode, ws, lse=lse)
    torch.cuda.synchronize()
    assert _counters_zero(ws, items)
    ref, ref_abs = prefill_pair(si.bits(q.cpu()), si.bits(k.cpu()), si.bits(v.cpu()), n, mode,
                                scale)
    what = f"split n={n} B={B} L={L} H={Hq}/{Hkv} D={D} mode={mode}"
    assert_close(f64(out), ref, what, ref_abs=ref_abs)
    lref = _lse_ref(q, k, v, n, mode, scale)
    got = lse.permute(0, 2, 1).cpu().numpy().astype(np.float64)
    err = np.abs(got - lref)
    assert np.all(err <= 1e-3 + 1e-4 * np.abs(lref)), f"{what}: max lse error {err.max():.3g}"
    # the same bits on a second call, whichever half merges each item
    out2 = hd.attn_split(q, k, v, n, scale, mode, ws)
    torch.cuda.synchronize()
    assert _same(out, out2)
    assert _counters_zero(ws, items)


def test_split_n1_stack_layer_two_kv_groups():
    """The n = 1 causal layer of the stack baseline (L = 2048, 32 / 8 heads,
    256 items on 256 compute units), every row of KV groups 0 and 7."""
    cfg = si.N8STACK
    q, k, v = si.prefill_qkv(cfg, B=1, L=cfg.L)
    q, k, v = (t[:, :cfg.L].contiguous() for t in (q, k, v))
    ws = hd.split_workspace(q.to(DEV), k.to(DEV), 1, MIX)
    out = hd.attn_split(q.to(DEV), k.to(DEV), v.to(DEV), 1, cfg.scale, MIX, ws)
    G = cfg.Hq // cfg.Hkv
    heads = list(range(G)) + list(range(cfg.Hq - G, cfg.Hq))
    ref, ref_abs = prefill_pair_all(si.bits(q), si.bits(k), si.bits(v), 1, MIX, cfg.scale,
                                    heads=heads)
    assert_close(f64(out[:, :, heads]), ref, "split n=1 L=2048 KV groups 0, 7", ref_abs=ref_abs)
    plain = hd.mix_attn(q.to(DEV), k.to(DEV), v.to(DEV), 1, cfg.scale)
    assert_close(f64(plain[:, :, heads]), ref, "plain n=1 L=2048 KV groups 0, 7", ref_abs=ref_abs)


class _grid:
    def __init__(self, count):
        self.count = count

    def __enter__(self):
        self.old = os.environ.get("HD_SFA_PREFILL_WORKGROUPS")
        os.environ["HD_SFA_PREFILL_WORKGROUPS"] = str(self.count)

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("HD_SFA_PREFILL_WORKGROUPS", None)
        else:
            os.environ["HD_SFA_PREFILL_WORKGROUPS"] = self.old


def test_split_grid_size_changes_no_bit():
    """256 items: split on every grid of at least 256 workgroups (up to one
    unit per workgroup); every unit is computed the same way wherever it
    runs and the merge is symmetric."""
    cfg = si.N8STACK
    q, k, v = si.prefill_qkv(cfg, B=1, L=cfg.L, device=DEV)
    q, k, v = (t[:, :cfg.L].contiguous() for t in (q, k, v))
    ws = hd.split_workspace(q, k, 1, MIX)
    lse = torch.empty((1, cfg.Hq, cfg.L), dtype=torch.float32, device=DEV)
    with _grid(256):
        ref = hd.attn_split(q, k, v, 1, cfg.scale, MIX, ws, lse=lse)
        lref = lse.clone()
    for g in (300, 504, 1000):
        with _grid(g):
            got = hd.attn_split(q, k, v, 1, cfg.scale, MIX, ws, lse=lse)
        torch.cuda.synchronize()
        assert _same(got, ref), g
        assert torch.equal(lse, lref), g
    assert _counters_zero(ws, _split_items(1, 1, cfg.L, cfg.Hq, cfg.Hkv, MIX))


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_split_full_launch_is_the_plain_forward(mode):
    """1024 items on 256 compute units: no split; the call is sfa_attn_fwd
    bit for bit and the workspace is not written."""
    cfg = si.N4
    q, k, v = si.prefill_qkv(cfg, device=DEV)
    ws = hd.split_workspace(q, k, cfg.n, mode)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.n * cfg.L), dtype=torch.float32, device=DEV)
    with _grid(256):
        out = hd.attn_split(q, k, v, cfg.n, cfg.scale, mode, ws, lse=lse)
        ref, lref = hd.attn_fwd(q, k, v, cfg.n, cfg.scale, mode)
    torch.cuda.synchronize()
    assert _same(out, ref)
    assert torch.equal(lse, lref)
    assert not bool(ws.any())
