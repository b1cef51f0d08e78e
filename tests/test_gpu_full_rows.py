"""Element-complete GPU parity where each persistent workgroup runs several
work items, and invariance of the prefill results under the grid size.

The prefill kernel is persistent: with one workgroup per compute unit, the n4
workload gives every workgroup four items per layer and the long-context one
thirty-two.  The code between items (the next item's Q and first K/V tiles
requested during the last key tile, the LDS ring slots carried across items,
the output leaving through a free V slot) runs only there, so these tests
compare every row of every head (long context: every row of one full
(batch, KV head) group) with the oracle at those shapes (gradients: every KV
group of the n4 layers and one of the n8 stack's mixing layer), and check that
running the same call on other grid sizes (1, 7, 100 and 300 workgroups, set
through HD_SFA_PREFILL_WORKGROUPS) changes no output bit.  The oracle runs
over (batch, head) units in a thread pool with one BLAS thread each.
"""
import os
import pytest
import torch

import oracle
import sequence_length_latent_amd as hd
import sfa_inputs as si
from tests._check import assert_close
from tests._refs import pool_map, prefill_pair_all

pytestmark = pytest.mark.gpu
DEV = "cuda"
WITHIN, MIX = oracle.WITHIN, oracle.MIX
FNS = {WITHIN: hd.stream_attn, MIX: hd.mix_attn}


def f64(t):
    return oracle.bf16_bits_to_f64(si.bits(t))


def _prefill_oracle(q, k, v, n, mode, scale, window=None, batches=None, heads=None):
    return prefill_pair_all(si.bits(q), si.bits(k), si.bits(v), n, mode, scale, window=window,
                            batches=batches, heads=heads)


# ---------------------------------------------------------------------------
# every row, every head, at the full n4 size (4 items per workgroup)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_prefill_n4_every_row_every_head(mode):
    cfg = si.N4
    q, k, v = si.prefill_qkv(cfg)
    out = FNS[mode](q.to(DEV), k.to(DEV), v.to(DEV), cfg.n, cfg.scale)
    ref, ref_abs = _prefill_oracle(q, k, v, cfg.n, mode, cfg.scale)
    assert_close(f64(out), ref, f"n4 every row mode={mode}", ref_abs=ref_abs)


def test_prefill_n4_window_every_row_every_head():
    cfg = si.N4
    q, k, v = si.prefill_qkv(cfg)
    out = hd.mix_attn_window(q.to(DEV), k.to(DEV), v.to(DEV), cfg.n, cfg.scale, 1024)
    ref, ref_abs = _prefill_oracle(q, k, v, cfg.n, MIX, cfg.scale, window=1024)
    assert_close(f64(out), ref, "n4 window 1024 every row", ref_abs=ref_abs)


# ---------------------------------------------------------------------------
# long context: every row of one full (batch, KV head) group (32 items per
# workgroup; the group's 16 query heads are two packs of 8)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_prefill_long_one_kv_group_every_row(mode):
    cfg = si.LONG
    q, k, v = si.prefill_qkv(cfg)
    out = FNS[mode](q.to(DEV), k.to(DEV), v.to(DEV), cfg.n, cfg.scale)
    G = cfg.Hq // cfg.Hkv
    kvh = 2
    heads = list(range(kvh * G, (kvh + 1) * G))
    ref, ref_abs = _prefill_oracle(q, k, v, cfg.n, mode, cfg.scale, heads=heads)
    assert_close(f64(out[:, :, heads]), ref, f"long KV group {kvh} every row mode={mode}",
                 ref_abs=ref_abs)


# ---------------------------------------------------------------------------
# gradients of the n4 workload, every KV group
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_attn_bwd_n4_every_kv_group(mode):
    cfg = si.N4
    q, k, v = si.prefill_qkv(cfg, device=DEV)
    do = si.randn_bf16(q.shape, 1.0, 6900 + mode, DEV)
    _, lse = hd.attn_fwd(q, k, v, cfg.n, cfg.scale, mode)
    dq, dk, dv = hd.attn_bwd(q, k, v, do, lse, cfg.n, cfg.scale, mode)
    torch.cuda.synchronize()
    qb, kb, vb, db = (si.bits(t) for t in (q, k, v, do))
    G = cfg.Hq // cfg.Hkv
    units = [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    res = pool_map(lambda u: oracle.prefill_backward_ref(qb, kb, vb, db, cfg.n, mode, cfg.scale,
                                                          heads=[u[1]], batches=[u[0]]), units)
    gq, gk, gv = f64(dq), f64(dk), f64(dv)
    for (b, g), (rq, rk, rv, _) in zip(units, res):
        w = f"n4 b={b} g={g} mode={mode}"
        assert_close(gq[b:b + 1, :, g * G:(g + 1) * G], rq, "dq " + w, c10=False)
        assert_close(gk[b:b + 1, :, g:g + 1], rk, "dk " + w, c10=False)
        assert_close(gv[b:b + 1, :, g:g + 1], rv, "dv " + w, c10=False)


# ---------------------------------------------------------------------------
# gradients of the n8 stack's mixing layer (16384 positions): a key there sums
# dS over four times as many query rows as in the n4 layer, which is where the
# bf16 operands' rounding error grows; one full (batch, KV head) group
# ---------------------------------------------------------------------------
def test_attn_bwd_n8_mixing_one_kv_group():
    cfg = si.N8STACK
    q, k, v = si.prefill_qkv(cfg, device=DEV)
    do = si.randn_bf16(q.shape, 1.0, 7100, DEV)
    _, lse = hd.attn_fwd(q, k, v, cfg.n, cfg.scale, MIX)
    dq, dk, dv = hd.attn_bwd(q, k, v, do, lse, cfg.n, cfg.scale, MIX)
    torch.cuda.synchronize()
    G = cfg.Hq // cfg.Hkv
    g = 3
    rq, rk, rv, _ = oracle.prefill_backward_ref(*(si.bits(t) for t in (q, k, v, do)), cfg.n, MIX,
                                                 cfg.scale, heads=[g], batches=[0])
    w = f"n8 mixing b=0 g={g}"
    assert_close(f64(dq[:, :, g * G:(g + 1) * G]), rq, "dq " + w, c10=False)
    assert_close(f64(dk[:, :, g:g + 1]), rk, "dk " + w, c10=False)
    assert_close(f64(dv[:, :, g:g + 1]), rv, "dv " + w, c10=False)


# ---------------------------------------------------------------------------
# grid size: no output bit depends on which workgroup runs an item
# ---------------------------------------------------------------------------
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


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("cfg,kind", [(si.N4, "within"), (si.N4, "mix"), (si.N4, "window"),
                                      (si.N4, "fwd_lse"), (si.LONG, "within"), (si.LONG, "mix")],
                         ids=lambda x: getattr(x, "name", str(x)))
def test_prefill_grid_size_changes_no_bit(cfg, kind):
    q, k, v = si.prefill_qkv(cfg, device=DEV)

    def run():
        if kind == "within":
            return hd.stream_attn(q, k, v, cfg.n, cfg.scale), None
        if kind == "mix":
            return hd.mix_attn(q, k, v, cfg.n, cfg.scale), None
        if kind == "window":
            return hd.mix_attn_window(q, k, v, cfg.n, cfg.scale, 1024), None
        return hd.attn_fwd(q, k, v, cfg.n, cfg.scale, MIX)

    ref, ref_lse = run()
    for count in (1, 7, 100, 300):
        with _grid(count):
            got, got_lse = run()
        torch.cuda.synchronize()
        assert _same(ref, got), f"{cfg.name} {kind}: output differs on {count} workgroups"
        if ref_lse is not None:
            assert torch.equal(ref_lse, got_lse), f"{cfg.name} {kind}: lse differs on {count} workgroups"


SMALL = [
    # n, B, L, Hq, Hkv, D, W (None: full pattern)
    (3, 2, 333, 8, 2, 128, None),      # P=4: odd and even item lengths, ragged last tile
    (5, 1, 130, 4, 4, 64, None),       # P=1, D=64
    (2, 1, 500, 16, 2, 128, 200),      # P=8, windowed items
    (4, 1, 257, 32, 8, 128, None),     # the n4 head layout
]


@pytest.mark.parametrize("n,B,L,Hq,Hkv,D,W", SMALL)
def test_prefill_three_workgroups_every_row(n, B, L, Hq, Hkv, D, W):
    """Three workgroups for the whole call: each runs tens of items in snake
    order, through every item length the shape has, against the oracle on
    every element."""
    seed = 8100 + 17 * n + L + D
    N = n * L
    q = si.randn_bf16((B, N, Hq, D), D ** -0.5, seed)
    k = si.randn_bf16((B, N, Hkv, D), 1.0, seed + 1)
    v = si.randn_bf16((B, N, Hkv, D), 1.0, seed + 2)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    modes = (WITHIN, MIX) if W is None else (MIX,)
    for mode in modes:
        with _grid(3):
            if W is None:
                out = FNS[mode](qd, kd, vd, n, 1.0)
            else:
                out = hd.mix_attn_window(qd, kd, vd, n, 1.0, W)
        ref, ref_abs = _prefill_oracle(q, k, v, n, mode, 1.0, window=W)
        assert_close(f64(out), ref, f"3 workgroups n={n} L={L} H={Hq}/{Hkv} D={D} W={W} mode={mode}",
                     ref_abs=ref_abs)
