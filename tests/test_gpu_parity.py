"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case draws seeded synthetic inputs (``sfa_inputs``), runs the library on
the GPU, and compares with ``oracle`` on the very same bf16 bits: bit-exact for
the expansion and the cache append, the floating-point bar of ``_check`` for
attention.  Full-size workloads are checked on sampled rows that the oracle
computes one by one, in the launch configuration the bench uses.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_length_latent_amd as hd
import sfa_inputs as si
from tests._check import assert_close, close_report
from tests._refs import decode_pair, prefill_pair

pytestmark = pytest.mark.gpu
DEV = "cuda"
WITHIN, MIX = oracle.WITHIN, oracle.MIX
FNS = {WITHIN: hd.stream_attn, MIX: hd.mix_attn}


def f64(t):
    return oracle.bf16_bits_to_f64(si.bits(t))


def _rand(shape, std, seed, device=DEV):
    return si.randn_bf16(shape, std, seed, device)


# ---------------------------------------------------------------------------
# expansion (bit-exact)
# ---------------------------------------------------------------------------
def test_expand_tiny_bit_exact():
    ids, tab = si.expand_inputs(si.TINY)
    out = hd.expand(ids.to(DEV), tab.to(DEV))
    ref, bad = oracle.expand_ref(ids.numpy(), si.bits(tab))
    assert not bad
    assert np.array_equal(si.bits(out), ref)


@pytest.mark.parametrize("n,B,L,V,H", [(1, 1, 1, 7, 8), (3, 2, 33, 50, 24), (8, 1, 100, 300, 64),
                                       (5, 3, 17, 1000, 4096), (2, 1, 1024, 64, 136),
                                       # around the one-row-per-workgroup limit of 512 chunks:
                                       # 256 chunks (two rows per workgroup), 513 (a second pass
                                       # for one thread), 1024 (two chunks per thread)
                                       (2, 1, 50, 30, 2048), (1, 2, 9, 11, 4104), (1, 1, 40, 20, 8192)])
def test_expand_shapes_bit_exact(n, B, L, V, H):
    seed = 1000 + n * 7 + L
    tab = _rand((n, V, H), 0.02, seed, "cpu")
    g = torch.Generator().manual_seed(seed)
    ids = torch.randint(0, V, (B, L), generator=g, dtype=torch.int64).to(torch.int32)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = hd.expand(ids.to(DEV), tab.to(DEV), err_flag=flag)
    ref, bad = oracle.expand_ref(ids.numpy(), si.bits(tab))
    assert np.array_equal(si.bits(out), ref)
    assert int(flag.item()) == 0 and not bad


def test_expand_out_of_range_ids():
    n, V, H = 3, 20, 16
    tab = _rand((n, V, H), 1.0, 77, "cpu")
    ids = torch.tensor([[0, 20, 5, -3, 19]], dtype=torch.int32)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = hd.expand(ids.to(DEV), tab.to(DEV), err_flag=flag)
    ref, bad = oracle.expand_ref(ids.numpy(), si.bits(tab))
    assert bad and int(flag.item()) == 1
    assert np.array_equal(si.bits(out), ref)


def test_expand_n4_full_size_sampled():
    """n=4 workload at full size: vocab 151936, hidden 4096 (4.98 GB of tables)."""
    cfg = si.N4
    ids, tab = si.expand_inputs(cfg, device=DEV)
    out = hd.expand(ids, tab)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(5)
    tsel = torch.cat([torch.tensor([0, 1, cfg.L - 1]),
                      torch.randint(0, cfg.L, (61,), generator=g)]).unique()
    ids_h = ids.cpu()
    # oracle over the sampled tokens, reading only the table rows they use
    used = ids_h[:, tsel].unique()
    sub_tab = si.bits(tab[:, used.to(DEV)])
    remap = {int(t): i for i, t in enumerate(used)}
    sub_ids = np.vectorize(lambda x: remap[int(x)])(ids_h[:, tsel].numpy())
    ref, bad = oracle.expand_ref(sub_ids, sub_tab)
    assert not bad
    pos = (tsel[:, None] * cfg.n + torch.arange(cfg.n)[None, :]).reshape(-1)
    got = si.bits(out[:, pos.to(DEV)])
    assert np.array_equal(got, ref)
    # and the whole output once, against a second gather route on the GPU
    want = tab[torch.arange(cfg.n, device=DEV)[None, None, :], ids.long()[:, :, None]]
    assert torch.equal(out.view(torch.int16), want.reshape(cfg.B, cfg.N, cfg.hidden).view(torch.int16))


# ---------------------------------------------------------------------------
# final-stream rows and cyclic replication (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,n,L,H", [(1, 1, 5, 8), (2, 4, 33, 136), (3, 8, 7, 64), (1, 3, 1000, 24)])
def test_final_stream_rows_bit_exact(B, n, L, H):
    x = _rand((B, n * L, H), 1.0, 5000 + n + L)
    out = hd.final_stream_rows(x, n)
    ref = oracle.final_stream_rows_ref(si.bits(x), n)
    assert np.array_equal(si.bits(out), ref)


def test_final_stream_rows_n4_full_size():
    """The n4 workload's expanded hidden size: [2, 4096, 4096] -> [2, 1024, 4096]."""
    cfg = si.N4
    x = _rand((cfg.B, cfg.N, cfg.hidden), 1.0, 5100)
    out = hd.final_stream_rows(x, cfg.n)
    ref = oracle.final_stream_rows_ref(si.bits(x), cfg.n)
    assert np.array_equal(si.bits(out), ref)


@pytest.mark.parametrize("n_old,n_new,V,H", [(1, 2, 7, 8), (2, 4, 100, 64), (3, 8, 33, 24),
                                             (4, 2, 10, 16), (2, 5, 1000, 4096)])
def test_cyclic_replicate_bit_exact(n_old, n_new, V, H):
    tab = _rand((n_old, V, H), 0.02, 5200 + n_old * 10 + n_new)
    out = hd.cyclic_replicate(tab, n_new)
    ref = oracle.cyclic_replicate_ref(si.bits(tab), n_new)
    assert np.array_equal(si.bits(out), ref)


def test_cyclic_replicate_in_place_growth():
    """1 -> 2 -> 4 -> 8 in one allocation (the pages' schedule): table 0 is
    never written and every table ends a copy of it."""
    V, H = 257, 128
    buf = torch.zeros((8, V, H), dtype=torch.bfloat16, device=DEV)
    buf[0] = _rand((V, H), 0.02, 5300)
    before = si.bits(buf[0:1]).copy()
    for n_old, n_new in ((1, 2), (2, 4), (4, 8)):
        hd.cyclic_replicate(buf[:n_old], n_new, out=buf[:n_new])
        ref = oracle.cyclic_replicate_ref(before, n_new)
        assert np.array_equal(si.bits(buf[:n_new]), ref), (n_old, n_new)


def test_cyclic_replicate_n4_vocab_sampled():
    """The n4 workload's tables: 2 -> 4 tables of 151936 x 4096 in place; all
    rows compared on the GPU, sampled rows against the oracle."""
    cfg = si.N4
    buf = torch.empty((4, cfg.vocab, cfg.hidden), dtype=torch.bfloat16, device=DEV)
    buf[:2] = si.tables(2, cfg.vocab, cfg.hidden, cfg.table_std, 5400, device=DEV)
    hd.cyclic_replicate(buf[:2], 4, out=buf)
    torch.cuda.synchronize()
    assert torch.equal(buf[2].view(torch.int16), buf[0].view(torch.int16))
    assert torch.equal(buf[3].view(torch.int16), buf[1].view(torch.int16))
    rows = torch.tensor([0, 1, 77, 4095, cfg.vocab - 1], device=DEV)
    ref = oracle.cyclic_replicate_ref(si.bits(buf[:2, rows]), 4)
    assert np.array_equal(si.bits(buf[:, rows]), ref)


# ---------------------------------------------------------------------------
# prefill attention
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_prefill_tiny_all_rows(mode):
    cfg = si.TINY
    q, k, v = si.prefill_qkv(cfg)
    out = FNS[mode](q.to(DEV), k.to(DEV), v.to(DEV), cfg.n, cfg.scale)
    ref, ref_abs = prefill_pair(si.bits(q), si.bits(k), si.bits(v), cfg.n, mode, cfg.scale)
    assert_close(f64(out), ref, f"tiny mode={mode}", ref_abs=ref_abs)


SWEEP = [
    # n, B, L, Hq, Hkv, D
    (1, 1, 1, 1, 1, 64),
    (1, 2, 65, 4, 2, 128),
    (2, 1, 7, 8, 1, 128),
    (3, 1, 64, 4, 2, 64),
    (5, 1, 65, 8, 2, 128),
    (8, 1, 100, 4, 4, 128),
    (2, 2, 257, 8, 8, 64),
    (4, 1, 129, 32, 8, 128),
    (3, 1, 96, 16, 1, 128),
    (8, 1, 33, 2, 2, 64),
    (2, 1, 65, 6, 2, 128),      # 3 query heads per KV head: packs of 1
    (3, 1, 50, 12, 2, 64),      # 6 per KV head: packs of 2
]


@pytest.mark.parametrize("n,B,L,Hq,Hkv,D", SWEEP)
@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_prefill_sweep(n, B, L, Hq, Hkv, D, mode):
    seed = 2000 + 97 * n + 13 * L + Hq + D
    N = n * L
    q = _rand((B, N, Hq, D), D ** -0.5, seed, "cpu")
    k = _rand((B, N, Hkv, D), 1.0, seed + 1, "cpu")
    v = _rand((B, N, Hkv, D), 1.0, seed + 2, "cpu")
    out = FNS[mode](q.to(DEV), k.to(DEV), v.to(DEV), n, 1.0)
    ref, ref_abs = prefill_pair(si.bits(q), si.bits(k), si.bits(v), n, mode, 1.0)
    assert_close(f64(out), ref, f"sweep n={n} L={L} H={Hq}/{Hkv} D={D} mode={mode}", ref_abs=ref_abs)


# sliding-window mixing: n, B, L, Hq, Hkv, D, W (W in interleaved positions)
WINDOW_SWEEP = [
    (4, 1, 40, 4, 1, 128, 1),          # own position only
    (2, 1, 100, 8, 2, 128, 7),         # window inside one tile
    (3, 1, 70, 16, 4, 128, 64),        # one tile wide
    (4, 2, 65, 32, 8, 128, 65),        # a tile and one
    (5, 1, 57, 8, 1, 64, 100),         # P=8 packing, D=64
    (2, 1, 300, 4, 2, 64, 129),        # P=2 packing
    (1, 1, 333, 2, 2, 128, 200),       # P=1 packing, n=1
    (8, 1, 40, 16, 1, 128, 319),       # W = N - 1
    (4, 1, 129, 32, 8, 128, 1024),     # W > N: the causal kernel
]


@pytest.mark.parametrize("n,B,L,Hq,Hkv,D,W", WINDOW_SWEEP)
def test_prefill_window_sweep(n, B, L, Hq, Hkv, D, W):
    seed = 4000 + 31 * n + 7 * L + W
    N = n * L
    q = _rand((B, N, Hq, D), D ** -0.5, seed, "cpu")
    k = _rand((B, N, Hkv, D), 1.0, seed + 1, "cpu")
    v = _rand((B, N, Hkv, D), 1.0, seed + 2, "cpu")
    out = hd.mix_attn_window(q.to(DEV), k.to(DEV), v.to(DEV), n, 1.0, W)
    ref, ref_abs = prefill_pair(si.bits(q), si.bits(k), si.bits(v), n, MIX, 1.0, window=W)
    assert_close(f64(out), ref, f"window W={W} n={n} L={L} H={Hq}/{Hkv} D={D}", ref_abs=ref_abs)


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_window_scale_modes(D):
    """The same windowed product through the three scale modes of the kernel."""
    n, B, L, Hq, Hkv, W = 3, 1, 90, 8, 2, 77
    seed = 4500 + D
    N = n * L
    q = _rand((B, N, Hq, D), 1.0, seed, "cpu")
    k = _rand((B, N, Hkv, D), 1.0, seed + 1, "cpu")
    v = _rand((B, N, Hkv, D), 1.0, seed + 2, "cpu")
    scale = D ** -0.5
    ref, ref_abs = prefill_pair(si.bits(q), si.bits(k), si.bits(v), n, MIX, scale, window=W)
    kd, vd = k.to(DEV), v.to(DEV)
    out0 = hd.mix_attn_window(q.to(DEV), kd, vd, n, scale, W)
    assert_close(f64(out0), ref, f"window any-scale D={D}", ref_abs=ref_abs)
    out1 = hd.mix_attn_window((q.float() * scale).to(torch.bfloat16).to(DEV), kd, vd, n, 1.0, W)
    assert_close(f64(out1), ref, f"window unit-scale D={D}", ref_abs=ref_abs)
    out2 = hd.mix_attn_window((q.float() * (scale * si.LOG2E)).to(torch.bfloat16).to(DEV), kd, vd,
                              n, si.LN2, W)
    assert_close(f64(out2), ref, f"window log2 units D={D}", ref_abs=ref_abs)


def test_prefill_window_one_returns_v_exactly():
    """W = 1: one visible key with probability exactly 1, so the output is that
    key's value row, bit for bit."""
    n, B, L, Hq, Hkv, D = 4, 1, 70, 8, 2, 128
    N = n * L
    q = _rand((B, N, Hq, D), 1.0, 4600)
    k = _rand((B, N, Hkv, D), 1.0, 4601)
    v = _rand((B, N, Hkv, D), 1.0, 4602)
    out = hd.mix_attn_window(q, k, v, n, 1.0, 1)
    want = v.repeat_interleave(Hq // Hkv, dim=2)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


def test_prefill_window_at_least_n_is_mix_bitwise():
    cfg = si.TINY
    q, k, v = (t.to(DEV) for t in si.prefill_qkv(cfg))
    a = hd.mix_attn(q, k, v, cfg.n, cfg.scale)
    for W in (cfg.N, cfg.N + 1, 1 << 40):
        b = hd.mix_attn_window(q, k, v, cfg.n, cfg.scale, W)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), W


def test_prefill_window_full_size_sampled():
    """The n4 workload's mixing layer with a window of 1024 positions (256
    tokens x 4 streams), sampled rows and heads, in the bench's launch."""
    cfg, W = si.N4, 1024
    q, k, v = si.prefill_qkv(cfg, device=DEV)
    out = hd.mix_attn_window(q, k, v, cfg.n, cfg.scale, W)
    torch.cuda.synchronize()
    rows = _sample_rows(cfg.N, cfg.n, 40, 17)
    rows = np.unique(np.concatenate([rows, [W - 2, W - 1, W, W + 1, W + 63, W + 64]]))
    G = cfg.Hq // cfg.Hkv
    heads = sorted({0, G - 1, G, cfg.Hq - 1})
    ref, ref_abs = prefill_pair(si.bits(q[:1].cpu()), si.bits(k[:1].cpu()), si.bits(v[:1].cpu()),
                                cfg.n, MIX, cfg.scale, rows=rows, heads=heads, window=W)
    got = f64(out[:1, torch.as_tensor(rows, device=DEV)][:, :, heads].cpu())
    assert_close(got, ref, f"n4 window {W} sampled", ref_abs=ref_abs)


# ---------------------------------------------------------------------------
# training: forward with log-sum-exp, gradients
# ---------------------------------------------------------------------------
def _assert_lse(got, ref, what):
    err = np.abs(got - ref)
    assert np.all(err <= 1e-3 + 1e-4 * np.abs(ref)), f"{what}: max lse error {err.max():.3g}"


@pytest.mark.parametrize("n,B,L,Hq,Hkv,D,mode", [(2, 1, 70, 4, 2, 128, WITHIN), (3, 2, 33, 8, 2, 64, MIX),
                                                  (1, 1, 200, 16, 2, 128, MIX), (4, 1, 65, 8, 8, 128, WITHIN)])
def test_attn_fwd_lse(n, B, L, Hq, Hkv, D, mode):
    seed = 6000 + 13 * n + L + mode
    N = n * L
    q = _rand((B, N, Hq, D), D ** -0.5, seed)
    k = _rand((B, N, Hkv, D), 1.0, seed + 1)
    v = _rand((B, N, Hkv, D), 1.0, seed + 2)
    out, lse = hd.attn_fwd(q, k, v, n, 1.0, mode)
    plain = FNS[mode](q, k, v, n, 1.0)
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    do = torch.zeros_like(q)
    _, _, _, ref = oracle.prefill_backward_ref(si.bits(q.cpu()), si.bits(k.cpu()), si.bits(v.cpu()),
                                               si.bits(do.cpu()), n, mode, 1.0)
    _assert_lse(lse.permute(0, 2, 1).cpu().numpy().astype(np.float64), ref, f"lse n={n} mode={mode}")


BWD_SWEEP = [
    # n, B, L, Hq, Hkv, D, mode
    (2, 1, 70, 4, 2, 128, WITHIN),
    (2, 1, 70, 4, 2, 128, MIX),
    (3, 2, 45, 8, 2, 64, WITHIN),
    (3, 1, 45, 8, 2, 64, MIX),
    (4, 1, 129, 8, 1, 128, MIX),       # a partial last key tile of 128
    (5, 1, 40, 16, 2, 128, WITHIN),    # P = 8 packing
    (1, 1, 300, 2, 2, 128, MIX),       # P = 1
    (4, 1, 96, 32, 2, 128, MIX),       # 16 query heads per KV head (the long-context ratio): two packs of 8
    (2, 1, 100, 6, 2, 64, WITHIN),     # 3 query heads per KV head: three packs of 1
]


@pytest.mark.parametrize("n,B,L,Hq,Hkv,D,mode", BWD_SWEEP)
def test_attn_bwd_sweep(n, B, L, Hq, Hkv, D, mode):
    seed = 6500 + 31 * n + 7 * L + Hq + D + mode
    N = n * L
    scale = D ** -0.5
    q = _rand((B, N, Hq, D), 1.0, seed)
    k = _rand((B, N, Hkv, D), 1.0, seed + 1)
    v = _rand((B, N, Hkv, D), 1.0, seed + 2)
    do = _rand((B, N, Hq, D), 1.0, seed + 3)
    out, lse = hd.attn_fwd(q, k, v, n, scale, mode)
    dq, dk, dv = hd.attn_bwd(q, k, v, do, lse, n, scale, mode)
    rq, rk, rv, _ = oracle.prefill_backward_ref(si.bits(q.cpu()), si.bits(k.cpu()), si.bits(v.cpu()),
                                                si.bits(do.cpu()), n, mode, scale)
    what = f"bwd n={n} L={L} H={Hq}/{Hkv} D={D} mode={mode}"
    assert_close(f64(dq.cpu()), rq, "dq " + what, c10=False)
    assert_close(f64(dk.cpu()), rk, "dk " + what, c10=False)
    assert_close(f64(dv.cpu()), rv, "dv " + what, c10=False)


def test_attn_bwd_single_position():
    """One position: P = 1, so dV = dO and dQ = dK = 0 (dS = P (dP - delta)
    vanishes up to rounding)."""
    q = _rand((1, 1, 2, 64), 1.0, 6400)
    k = _rand((1, 1, 1, 64), 1.0, 6401)
    v = _rand((1, 1, 1, 64), 1.0, 6402)
    do = _rand((1, 1, 2, 64), 1.0, 6403)
    out, lse = hd.attn_fwd(q, k, v, 1, 0.125, MIX)
    dq, dk, dv = hd.attn_bwd(q, k, v, do, lse, 1, 0.125, MIX)
    # P = 1 up to the rounding of lse (stored in natural-log units): dV equals
    # the sum of the two heads' dO within one bf16 rounding
    want = do[:, :, 0].float() + do[:, :, 1].float()
    assert torch.all((dv[:, :, 0].float() - want).abs() <= want.abs() * 2.0 ** -8 + 1e-6)
    assert float(dq.float().abs().max()) < 1e-5 and float(dk.float().abs().max()) < 1e-5


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_attn_bwd_n4_full_size_one_group(mode):
    """The n4 workload at full size; the oracle computes batch 0, KV head 0
    (its four query heads) over every row."""
    cfg = si.N4
    q, k, v = si.prefill_qkv(cfg, device=DEV)
    do = _rand(q.shape, 1.0, 6900 + mode)
    out, lse = hd.attn_fwd(q, k, v, cfg.n, cfg.scale, mode)
    dq, dk, dv = hd.attn_bwd(q, k, v, do, lse, cfg.n, cfg.scale, mode)
    torch.cuda.synchronize()
    G = cfg.Hq // cfg.Hkv
    rq, rk, rv, _ = oracle.prefill_backward_ref(si.bits(q[:1].cpu()), si.bits(k[:1].cpu()),
                                                si.bits(v[:1].cpu()), si.bits(do[:1].cpu()),
                                                cfg.n, mode, cfg.scale, heads=[0])
    assert_close(f64(dq[:1, :, :G].cpu()), rq, f"n4 dq mode={mode}", c10=False)
    assert_close(f64(dk[:1, :, :1].cpu()), rk, f"n4 dk mode={mode}", c10=False)
    assert_close(f64(dv[:1, :, :1].cpu()), rv, f"n4 dv mode={mode}", c10=False)


WIN_BWD_SWEEP = [
    # n, B, L, Hq, Hkv, D, W (positions of the interleaved order)
    (2, 1, 70, 4, 2, 128, 7),        # inside a 64-row tile
    (3, 1, 45, 8, 2, 64, 64),        # one tile
    (4, 1, 129, 8, 1, 128, 65),      # a tile and one; partial last 128-key tile
    (4, 1, 129, 8, 1, 128, 300),     # across 128-key tiles
    (2, 2, 100, 16, 2, 128, 199),    # W = N - 1, P = 8 packing
    (1, 1, 300, 2, 2, 128, 129),     # P = 1
]


@pytest.mark.parametrize("n,B,L,Hq,Hkv,D,W", WIN_BWD_SWEEP)
def test_attn_window_training_sweep(n, B, L, Hq, Hkv, D, W):
    """Sliding-window mixing layer: the training forward equals the plain
    windowed forward bit for bit, its lse and the gradients match the oracle."""
    seed = 7300 + 31 * n + 7 * L + Hq + D + W
    N = n * L
    scale = D ** -0.5
    q = _rand((B, N, Hq, D), 1.0, seed)
    k = _rand((B, N, Hkv, D), 1.0, seed + 1)
    v = _rand((B, N, Hkv, D), 1.0, seed + 2)
    do = _rand((B, N, Hq, D), 1.0, seed + 3)
    out, lse = hd.attn_fwd(q, k, v, n, scale, MIX, window=W)
    plain = hd.mix_attn_window(q, k, v, n, scale, W)
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    dq, dk, dv = hd.attn_bwd(q, k, v, do, lse, n, scale, MIX, window=W)
    rq, rk, rv, rl = oracle.prefill_backward_ref(si.bits(q.cpu()), si.bits(k.cpu()), si.bits(v.cpu()),
                                                 si.bits(do.cpu()), n, MIX, scale, window=W)
    what = f"window bwd n={n} L={L} H={Hq}/{Hkv} D={D} W={W}"
    _assert_lse(lse.permute(0, 2, 1).cpu().numpy().astype(np.float64), rl, "lse " + what)
    assert_close(f64(dq.cpu()), rq, "dq " + what, c10=False)
    assert_close(f64(dk.cpu()), rk, "dk " + what, c10=False)
    assert_close(f64(dv.cpu()), rv, "dv " + what, c10=False)


def test_attn_window_one_training():
    """W = 1: every query sees only its own key, so P = 1, dV_j = the sum of
    dO_j over the KV group's query heads, and dQ = dK = 0 (up to the rounding
    of lse)."""
    n, L, Hq, Hkv, D = 2, 40, 4, 2, 64
    N = n * L
    q = _rand((1, N, Hq, D), 1.0, 7400)
    k = _rand((1, N, Hkv, D), 1.0, 7401)
    v = _rand((1, N, Hkv, D), 1.0, 7402)
    do = _rand((1, N, Hq, D), 1.0, 7403)
    out, lse = hd.attn_fwd(q, k, v, n, 0.125, MIX, window=1)
    dq, dk, dv = hd.attn_bwd(q, k, v, do, lse, n, 0.125, MIX, window=1)
    want = do.float().reshape(1, N, Hkv, Hq // Hkv, D).sum(3)
    assert torch.all((dv.float() - want).abs() <= want.abs() * 2.0 ** -7 + 1e-5)
    assert float(dq.float().abs().max()) < 1e-4 and float(dk.float().abs().max()) < 1e-4


def test_attn_window_training_long_window_is_full():
    """W >= N: the windowed training forward and gradients are bitwise those
    of the full mixing layer."""
    n, B, L, Hq, Hkv, D = 3, 1, 50, 8, 2, 128
    N = n * L
    q = _rand((B, N, Hq, D), 1.0, 7450)
    k = _rand((B, N, Hkv, D), 1.0, 7451)
    v = _rand((B, N, Hkv, D), 1.0, 7452)
    do = _rand((B, N, Hq, D), 1.0, 7453)
    out, lse = hd.attn_fwd(q, k, v, n, D ** -0.5, MIX)
    outw, lsew = hd.attn_fwd(q, k, v, n, D ** -0.5, MIX, window=N)
    assert torch.equal(out.view(torch.int16), outw.view(torch.int16)) and torch.equal(lse, lsew)
    a = hd.attn_bwd(q, k, v, do, lse, n, D ** -0.5, MIX)
    b = hd.attn_bwd(q, k, v, do, lse, n, D ** -0.5, MIX, window=N + 5)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_attn_window_training_n4_full_size_one_group():
    """The n4 workload at W = 1024 (256 tokens at n = 4), full size; the oracle
    computes batch 0, KV head 0 (its four query heads) over every row."""
    cfg = si.N4
    W = 1024
    q, k, v = si.prefill_qkv(cfg, device=DEV)
    do = _rand(q.shape, 1.0, 7500)
    out, lse = hd.attn_fwd(q, k, v, cfg.n, cfg.scale, MIX, window=W)
    dq, dk, dv = hd.attn_bwd(q, k, v, do, lse, cfg.n, cfg.scale, MIX, window=W)
    torch.cuda.synchronize()
    G = cfg.Hq // cfg.Hkv
    rq, rk, rv, _ = oracle.prefill_backward_ref(si.bits(q[:1].cpu()), si.bits(k[:1].cpu()),
                                                si.bits(v[:1].cpu()), si.bits(do[:1].cpu()),
                                                cfg.n, MIX, cfg.scale, window=W, heads=[0])
    assert_close(f64(dq[:1, :, :G].cpu()), rq, "n4 window dq", c10=False)
    assert_close(f64(dk[:1, :, :1].cpu()), rk, "n4 window dk", c10=False)
    assert_close(f64(dv[:1, :, :1].cpu()), rv, "n4 window dv", c10=False)


def test_attn_bwd_deterministic():
    n, B, L, Hq, Hkv, D = 3, 1, 90, 8, 2, 128
    N = n * L
    q = _rand((B, N, Hq, D), 1.0, 6950)
    k = _rand((B, N, Hkv, D), 1.0, 6951)
    v = _rand((B, N, Hkv, D), 1.0, 6952)
    do = _rand((B, N, Hq, D), 1.0, 6953)
    out, lse = hd.attn_fwd(q, k, v, n, D ** -0.5, MIX)
    a = hd.attn_bwd(q, k, v, do, lse, n, D ** -0.5, MIX)
    b = hd.attn_bwd(q, k, v, do, lse, n, D ** -0.5, MIX)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_prefill_nonunit_scale(D, mode):
    """Unscaled Q with the softmax scale 1/sqrt(D) passed to the call: the
    general-scale kernel.  The same product through the two specialised ones:
    scale 1 (Q carries the scale) and scale ln 2 (Q also carries log2(e), so
    scale * log2(e) == 1 in float32)."""
    n, B, L, Hq, Hkv = 3, 1, 70, 8, 2
    seed = 3100 + D + mode
    N = n * L
    q = _rand((B, N, Hq, D), 1.0, seed, "cpu")
    k = _rand((B, N, Hkv, D), 1.0, seed + 1, "cpu")
    v = _rand((B, N, Hkv, D), 1.0, seed + 2, "cpu")
    scale = D ** -0.5
    out = FNS[mode](q.to(DEV), k.to(DEV), v.to(DEV), n, scale)
    ref, ref_abs = prefill_pair(si.bits(q), si.bits(k), si.bits(v), n, mode, scale)
    assert_close(f64(out), ref, f"scale={scale:.4f} D={D} mode={mode}", ref_abs=ref_abs)
    # the same product through the unit-scale kernel: Q pre-scaled on the host
    out1 = FNS[mode]((q.float() * scale).to(torch.bfloat16).to(DEV), k.to(DEV), v.to(DEV), n, 1.0)
    assert_close(f64(out1), ref, f"pre-scaled D={D} mode={mode}", ref_abs=ref_abs)
    # and with log2(e) folded in as well: scores arrive in log2 units
    out2 = FNS[mode]((q.float() * (scale * si.LOG2E)).to(torch.bfloat16).to(DEV), k.to(DEV), v.to(DEV),
                     n, si.LN2)
    assert_close(f64(out2), ref, f"log2 units D={D} mode={mode}", ref_abs=ref_abs)


def _sample_rows(N, n, count, seed):
    g = np.random.default_rng(seed)
    fixed = [0, 1, n - 1, n, 31, 32, 63, 64, 127, 128, N // 2, N - n - 1, N - 2, N - 1]
    rows = np.unique(np.concatenate([np.array([r for r in fixed if 0 <= r < N]),
                                     g.integers(0, N, count)]))
    return rows


FULL = [
    (si.N4, 0, WITHIN), (si.N4, 0, MIX),
    (si.N8STACK, 0, WITHIN), (si.N8STACK, 3, MIX),
    (si.LONG, 0, WITHIN), (si.LONG, 0, MIX),
]


@pytest.mark.parametrize("cfg,layer,mode", FULL, ids=lambda x: getattr(x, "name", str(x)))
def test_prefill_full_size_sampled(cfg, layer, mode):
    q, k, v = si.prefill_qkv(cfg, layer=layer, device=DEV)
    out = FNS[mode](q, k, v, cfg.n, cfg.scale)
    torch.cuda.synchronize()
    rows = _sample_rows(cfg.N, cfg.n, 40, 11 + layer)
    G = cfg.Hq // cfg.Hkv
    heads = sorted({0, G - 1, G, cfg.Hq - 1})
    for b in range(cfg.B):
        ref, ref_abs = prefill_pair(si.bits(q[b:b + 1]), si.bits(k[b:b + 1]), si.bits(v[b:b + 1]),
                                    cfg.n, mode, cfg.scale, rows=rows, heads=heads)
        got = f64(out[b:b + 1][:, torch.as_tensor(rows, device=DEV)][:, :, heads])
        assert_close(got, ref, f"{cfg.name} b={b} mode={mode}", ref_abs=ref_abs)


def test_prefill_literal_scaling_reading():
    """Second reading of 'Q/K/V ~N(0,1) pre-scaled by 1/sqrt(128)': all three scaled."""
    cfg = si.N4
    s = 128 ** -0.5
    q, k, v = si.prefill_qkv(cfg, device=DEV, q_std=s, kv_std=s, B=1, L=256)
    for mode in (WITHIN, MIX):
        out = FNS[mode](q, k, v, cfg.n, 1.0)
        ref, ref_abs = prefill_pair(si.bits(q), si.bits(k), si.bits(v), cfg.n, mode, 1.0,
                                    heads=[0, 5, 31])
        assert_close(f64(out[:, :, [0, 5, 31]]), ref, f"literal scaling mode={mode}", ref_abs=ref_abs)


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_prefill_peaked_softmax(mode):
    """Q ~ N(0,1) with scale 1: logits of std ~ sqrt(D), exercising the max rescale."""
    n, L, Hq, Hkv, D = 4, 200, 8, 2, 128
    q = _rand((1, n * L, Hq, D), 1.0, 31, "cpu")
    k = _rand((1, n * L, Hkv, D), 1.0, 32, "cpu")
    v = _rand((1, n * L, Hkv, D), 1.0, 33, "cpu")
    out = FNS[mode](q.to(DEV), k.to(DEV), v.to(DEV), n, 1.0)
    ref, ref_abs = prefill_pair(si.bits(q), si.bits(k), si.bits(v), n, mode, 1.0)
    assert_close(f64(out), ref, "peaked", ref_abs=ref_abs)


def test_prefill_exact_pins():
    n, L, Hq, Hkv, D = 4, 70, 8, 2, 128
    N = n * L
    q = _rand((1, N, Hq, D), 1.0, 41)
    k = _rand((1, N, Hkv, D), 1.0, 42)
    v = _rand((1, N, Hkv, D), 1.0, 43)
    vrep = v.repeat_interleave(Hq // Hkv, dim=2)
    # L = 1 within-stream: every query sees only itself -> O == V bitwise
    o1 = hd.stream_attn(q[:, :n].contiguous(), k[:, :n].contiguous(), v[:, :n].contiguous(), n, 1.0)
    assert torch.equal(o1.view(torch.int16), vrep[:, :n].view(torch.int16))
    # first token of every stream (within) and position 0 (mixing) -> O == V bitwise
    ow = hd.stream_attn(q, k, v, n, 1.0)
    om = hd.mix_attn(q, k, v, n, 1.0)
    assert torch.equal(ow[:, :n].view(torch.int16), vrep[:, :n].view(torch.int16))
    assert torch.equal(om[:, :1].view(torch.int16), vrep[:, :1].view(torch.int16))
    # V == 1 -> O == 1 (softmax rows sum to one).  The weights enter P V as
    # bf16 and the row sum in fp32, so O may sit one bf16 ulp (2^-8) from 1.
    ones = torch.ones_like(v)
    for fn in (hd.stream_attn, hd.mix_attn):
        o = fn(q, k, ones, n, 1.0)
        assert torch.all((o.float() - 1.0).abs() <= 2.0 ** -8)


def test_prefill_stream_one_hot_pin():
    """V[p(t,s)] = e_s: within-stream output must be e_s for every query."""
    n, L, Hq, Hkv, D = 5, 90, 4, 2, 64
    N = n * L
    q = _rand((1, N, Hq, D), 1.0, 51)
    k = _rand((1, N, Hkv, D), 1.0, 52)
    v = torch.zeros((1, N, Hkv, D), dtype=torch.bfloat16, device=DEV)
    pos = torch.arange(N, device=DEV)
    v[0, pos, :, pos % n] = 1.0
    o = hd.stream_attn(q, k, v, n, 1.0)
    want = torch.zeros((1, N, Hq, D), dtype=torch.float64, device=DEV)
    want[0, pos, :, pos % n] = 1.0
    # sum_j p_j |v_j| is the same one-hot vector
    assert_close(o.double().cpu().numpy(), want.cpu().numpy(), "one-hot", ref_abs=want.cpu().numpy())


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_prefill_k_zero_prefix_means(mode):
    n, L, Hq, Hkv, D = 3, 150, 4, 4, 128
    N = n * L
    q = _rand((1, N, Hq, D), 1.0, 61)
    k = torch.zeros((1, N, Hkv, D), dtype=torch.bfloat16, device=DEV)
    v = _rand((1, N, Hkv, D), 1.0, 62)
    o = FNS[mode](q, k, v, n, 1.0)
    vf = f64(v)[0]

    def prefix_means(x):
        if mode == MIX:
            return np.cumsum(x, axis=0) / np.arange(1, N + 1)[:, None, None]
        m = np.empty_like(x)
        for s in range(n):
            m[s::n] = np.cumsum(x[s::n], axis=0) / np.arange(1, L + 1)[:, None, None]
        return m

    assert_close(f64(o)[0], prefix_means(vf), "prefix means", ref_abs=prefix_means(np.abs(vf)))


def test_negative_controls_fail_the_bar():
    cfg = si.TINY
    q, k, v = si.prefill_qkv(cfg, L=64)
    q2 = _rand(q.shape, 1.0, 71, "cpu")   # peaked, so outputs are not all tiny
    ref_w = oracle.prefill_ref(si.bits(q2), si.bits(k), si.bits(v), cfg.n, WITHIN, 1.0)
    ref_m = oracle.prefill_ref(si.bits(q2), si.bits(k), si.bits(v), cfg.n, MIX, 1.0)
    ow = f64(hd.stream_attn(q2.to(DEV), k.to(DEV), v.to(DEV), cfg.n, 1.0))
    om = f64(hd.mix_attn(q2.to(DEV), k.to(DEV), v.to(DEV), cfg.n, 1.0))
    assert close_report(ow, ref_w)[0] and close_report(om, ref_m)[0]
    assert not close_report(np.zeros_like(ow), ref_w)[0]              # zero output
    assert not close_report(np.roll(ow, 1, axis=1), ref_w)[0]         # rolled by one stream
    assert not close_report(om, ref_w)[0]                             # mixing fed to within
    assert not close_report(ow, ref_m)[0]


def test_determinism():
    cfg = si.N4
    q, k, v = si.prefill_qkv(cfg, device=DEV, B=1, L=512)
    for fn in (hd.stream_attn, hd.mix_attn):
        a = fn(q, k, v, cfg.n, 1.0)
        b = fn(q, k, v, cfg.n, 1.0)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def _decode_case(cfg, S, T, tb, mode, seqs=None, max_tokens=None, device=DEV, window=None):
    qn, kn, vn, kc, vc, tbt = si.decode_inputs(cfg, device=device, S=S, T=T, tokens_before=tb)
    max_tokens = T if max_tokens is None else max_tokens
    kc0, vc0 = kc.clone(), vc.clone()
    out = hd.decode_step(qn, kn, vn, kc, vc, tbt, cfg.n, max_tokens, mode, cfg.scale, window=window)
    torch.cuda.synchronize()
    seqs = list(range(S)) if seqs is None else seqs
    tbh = tbt.cpu().numpy()
    for qi in seqs:
        sl = slice(qi, qi + 1)
        k2, v2 = oracle.decode_append_ref(si.bits(kc0[sl]), si.bits(vc0[sl]), si.bits(kn[sl]),
                                          si.bits(vn[sl]), tbh[sl], cfg.n)
        assert np.array_equal(si.bits(kc[sl]), k2), f"k append seq {qi}"
        assert np.array_equal(si.bits(vc[sl]), v2), f"v append seq {qi}"
        ref, ref_abs = decode_pair(si.bits(qn[sl]), k2, v2, tbh[sl], cfg.n, mode, cfg.scale,
                                   window=window)
        assert_close(f64(out[sl]), ref, f"decode seq {qi} T={tbh[qi]} mode={mode} window={window}",
                     ref_abs=ref_abs)
    return out


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_small_ragged(mode):
    _decode_case(si.DECODE, S=5, T=300, tb=[300, 0, 1, 129, 255], mode=mode)


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_first_token_empty_caches(mode):
    """The first decode step: every cache is empty (max_tokens 0), so token 0's
    n rows are appended and attend to themselves only (mixing: stream s sees
    streams 0..s of token 0; within-stream: each sees its own row, out = v)."""
    out = _decode_case(si.DECODE, S=4, T=0, tb=[0, 0, 0, 0], mode=mode)
    if mode == WITHIN:
        cfg = si.DECODE
        _, kn, vn, _, _, _ = si.decode_inputs(cfg, device=DEV, S=4, T=0, tokens_before=[0, 0, 0, 0])
        G = cfg.Hq // cfg.Hkv
        want = vn.repeat_interleave(G, dim=2)
        assert torch.equal(out.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_other_shapes(mode):
    # n=3 (not a power of two), G=8 -> 24 rows; D=64
    cfg = si.DecodeCfg("d3", 9, S=3, n=3, T=200, Hq=16, Hkv=2, D=64, scale=0.125)
    _decode_case(cfg, S=3, T=200, tb=[200, 77, 3], mode=mode)
    # n=8, G=8 -> 64 rows in mixing mode (two 32-row blocks)
    cfg = si.DecodeCfg("d8", 10, S=2, n=8, T=70, Hq=8, Hkv=1, D=128, scale=0.09)
    _decode_case(cfg, S=2, T=70, tb=[70, 31], mode=mode)
    # G=3 (odd): 12 rows in mixing mode, 3 per stream view
    cfg = si.DecodeCfg("d3g", 19, S=3, n=4, T=150, Hq=6, Hkv=2, D=128, scale=0.1)
    _decode_case(cfg, S=3, T=150, tb=[150, 64, 1], mode=mode)


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_many_streams(mode):
    """Stream counts where a stream has several keys per 32-key wave slice
    (n=5), or at most one (n=40 > 32), exercising the within-stream row mask."""
    cfg = si.DecodeCfg("d5", 15, S=3, n=5, T=90, Hq=4, Hkv=2, D=64, scale=0.11)
    _decode_case(cfg, S=3, T=90, tb=[90, 41, 0], mode=mode)
    cfg = si.DecodeCfg("d40", 16, S=2, n=40, T=20, Hq=1, Hkv=1, D=128, scale=0.09)
    _decode_case(cfg, S=2, T=20, tb=[20, 7], mode=mode)


def test_decode_window_split_plan_capped():
    """37 sequences x 2 KV heads (74 units, ~7 splits wanted), 250 tokens x 4
    streams: the full view gets 4 splits of 256 entries, and a window of 797
    would on its own get 7 splits of 128.  The window plan is capped at the
    full view's split count (the workspace stride), so the partials of one
    row never reach the next row's."""
    cfg = si.DecodeCfg("dcap", 17, S=37, n=4, T=249, Hq=8, Hkv=2, D=128, scale=0.09)
    tb = [249 - (i * 37) % 250 for i in range(37)]
    _decode_case(cfg, S=37, T=249, tb=tb, mode=MIX, seqs=[0, 1, 18, 36], window=797)


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_full_size_sampled(mode):
    """Decode workload at full size: 64 sequences x 16384 cached entries."""
    cfg = si.DECODE
    _decode_case(cfg, S=cfg.S, T=cfg.T, tb=None, mode=mode, seqs=[0, 31, 63])


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_long_context_sampled(mode):
    """Long-context decode at full size: 32 sequences x 32768 tokens x 4
    streams (a 17.2 GB K+V cache), ragged token counts, in the launch the
    bench times; two sequences checked against the oracle (each ~131k
    entries), the appends of those sequences bit-exact."""
    cfg = si.DECODE_LONG
    tb = [cfg.T - (i * 1031) % 4096 for i in range(cfg.S)]
    qn, kn, vn, kc, vc, tbt = si.decode_inputs(cfg, device=DEV, tokens_before=tb)
    seqs = [0, 19]
    before = {qi: (si.bits(kc[qi:qi + 1]), si.bits(vc[qi:qi + 1])) for qi in seqs}
    out = hd.decode_step(qn, kn, vn, kc, vc, tbt, cfg.n, cfg.T, mode, cfg.scale)
    torch.cuda.synchronize()
    tbh = np.asarray(tb, dtype=np.int32)
    for qi in seqs:
        sl = slice(qi, qi + 1)
        k2, v2 = oracle.decode_append_ref(before[qi][0], before[qi][1], si.bits(kn[sl]),
                                          si.bits(vn[sl]), tbh[sl], cfg.n)
        assert np.array_equal(si.bits(kc[sl]), k2), f"k append seq {qi}"
        assert np.array_equal(si.bits(vc[sl]), v2), f"v append seq {qi}"
        ref, ref_abs = decode_pair(si.bits(qn[sl]), k2, v2, tbh[sl], cfg.n, mode, cfg.scale)
        assert_close(f64(out[sl]), ref, f"long decode seq {qi} T={tbh[qi]} mode={mode}", ref_abs=ref_abs)
    del qn, kn, vn, kc, vc, tbt, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("window", [1, 3, 64, 129, 500, 1 << 20])
def test_decode_window_ragged(window):
    """Sliding-window mixing decode over ragged caches (windows inside one
    token's streams, one tile, past a tile edge, longer than some caches)."""
    _decode_case(si.DECODE, S=5, T=300, tb=[300, 0, 1, 129, 255], mode=MIX, window=window)


def test_decode_window_other_shapes():
    cfg = si.DecodeCfg("d3w", 12, S=3, n=3, T=200, Hq=16, Hkv=2, D=64, scale=0.125)
    _decode_case(cfg, S=3, T=200, tb=[200, 77, 3], mode=MIX, window=50)
    cfg = si.DecodeCfg("d8w", 13, S=2, n=8, T=70, Hq=8, Hkv=1, D=128, scale=0.09)
    _decode_case(cfg, S=2, T=70, tb=[70, 31], mode=MIX, window=130)


def test_decode_window_full_size_sampled():
    """The decode workload (64 sequences x 16384 entries) with a window of
    4096 positions (1024 tokens x 4 streams)."""
    cfg = si.DECODE
    _decode_case(cfg, S=cfg.S, T=cfg.T, tb=None, mode=MIX, seqs=[0, 31, 63], window=4096)


def test_decode_window_long_equals_mix_bitwise():
    cfg = si.DECODE
    S, T = 3, 90
    qn, kn, vn, kc, vc, tb = si.decode_inputs(cfg, device=DEV, S=S, T=T, tokens_before=[90, 4, 50])
    a = hd.decode_step(qn, kn, vn, kc, vc, tb, cfg.n, T, MIX, cfg.scale)
    b = hd.decode_step(qn, kn, vn, kc, vc, tb, cfg.n, T, MIX, cfg.scale, window=(T + 1) * cfg.n)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _paged_from(kc, vc, P, seed, spare=3):
    """A page pool holding the contiguous caches' rows in shuffled pages (plus
    spare pages filled with noise) and the page table that maps them back."""
    S, C, Hkv, D = kc.shape
    mp = (C + P - 1) // P
    num_pages = S * mp + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(num_pages, generator=g)[: S * mp].reshape(S, mp).to(torch.int32)
    kp = _rand((num_pages, P, Hkv, D), 1.0, seed + 1)
    vp = _rand((num_pages, P, Hkv, D), 1.0, seed + 2)
    pad = mp * P - C
    kpad = torch.cat([kc, kc[:, :pad]], dim=1) if pad else kc
    vpad = torch.cat([vc, vc[:, :pad]], dim=1) if pad else vc
    pt = perm.to(DEV)
    kp[pt.reshape(-1).long()] = kpad.reshape(S * mp, P, Hkv, D)
    vp[pt.reshape(-1).long()] = vpad.reshape(S * mp, P, Hkv, D)
    return kp, vp, pt


@pytest.mark.parametrize("P,mode,window", [(16, WITHIN, None), (16, MIX, None), (64, MIX, 300),
                                           (1, MIX, None), (128, WITHIN, None), (4, MIX, 7)])
def test_decode_paged_equals_contiguous(P, mode, window):
    """Paged decode over shuffled pages gives the contiguous decode bit for
    bit, and the append lands in the right page slots (checked against the
    oracle's scatter)."""
    cfg = si.DECODE
    S, T = 5, 300
    tb = [300, 0, 1, 129, 255]
    qn, kn, vn, kc, vc, tbt = si.decode_inputs(cfg, device=DEV, S=S, T=T, tokens_before=tb)
    kp, vp, pt = _paged_from(kc, vc, P, 7000 + P + mode)
    kp0 = kp.clone()
    ref = hd.decode_step(qn, kn, vn, kc, vc, tbt, cfg.n, T, mode, cfg.scale, window=window)
    got = hd.decode_step_paged(qn, kn, vn, kp, vp, pt, tbt, cfg.n, T, mode, cfg.scale, window=window)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    want = si.bits(kp0)
    pth = pt.cpu().numpy()
    for q in range(S):
        for s_ in range(cfg.n):
            want = oracle.scatter_pages_ref(want, pth, q, tb[q] * cfg.n + s_, si.bits(kn[q, s_]))
    assert np.array_equal(si.bits(kp), want)


@pytest.mark.parametrize("n,Hq,Hkv,D,mode,P", [(8, 64, 8, 128, MIX, 32),     # 64 query rows
                                                (8, 64, 8, 128, WITHIN, 32),
                                                (3, 16, 2, 64, MIX, 8),        # head_dim 64
                                                (3, 16, 2, 64, WITHIN, 64)])
def test_decode_paged_other_shapes(n, Hq, Hkv, D, mode, P):
    """Paged decode with 64 query rows per KV head (two 32-row blocks) and with
    head_dim 64: bitwise the contiguous decode on the same rows."""
    cfg = si.DecodeCfg("dpo", 15, S=3, n=n, T=150, Hq=Hq, Hkv=Hkv, D=D, scale=D ** -0.5)
    tb = [150, 17, 0]
    qn, kn, vn, kc, vc, tbt = si.decode_inputs(cfg, device=DEV, S=3, T=150, tokens_before=tb)
    kp, vp, pt = _paged_from(kc, vc, P, 7150 + n + D + mode)
    ref = hd.decode_step(qn, kn, vn, kc, vc, tbt, n, 150, mode, cfg.scale)
    got = hd.decode_step_paged(qn, kn, vn, kp, vp, pt, tbt, n, 150, mode, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_error_flag_token_counts(mode):
    """A tokens_before value outside [0, max_tokens] is clamped into it on the
    device (every access stays in the cache) and raises the caller's flag; the
    step is then the step with the clamped counts, bit for bit.  In-range
    counts leave the flag at zero."""
    cfg = si.DECODE
    S, T = 3, 100
    qn, kn, vn, kc, vc, _ = si.decode_inputs(cfg, device=DEV, S=S, T=T)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    good = torch.tensor([100, 0, 40], dtype=torch.int32, device=DEV)
    kc1, vc1 = kc.clone(), vc.clone()
    ref = hd.decode_step(qn, kn, vn, kc1, vc1, good, cfg.n, T, mode, cfg.scale, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    bad = torch.tensor([130, -4, 40], dtype=torch.int32, device=DEV)
    kc2, vc2 = kc.clone(), vc.clone()
    got = hd.decode_step(qn, kn, vn, kc2, vc2, bad, cfg.n, T, mode, cfg.scale, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16))


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_paged_error_flag_page_ids(mode):
    """A page id outside the pool, on a page the step reads, is clamped into
    the pool (-1 -> page 0, num_pages + 5 -> the last page) and raises the
    flag; the result equals the step over a table holding the clamped ids.
    Garbage in table slots past a sequence's live entries is never read and
    leaves the flag at zero."""
    cfg = si.DECODE
    S, T, P = 3, 100, 16
    tb = [100, 20, 55]
    qn, kn, vn, kc, vc, tbt = si.decode_inputs(cfg, device=DEV, S=S, T=T, tokens_before=tb)
    kp, vp, pt = _paged_from(kc, vc, P, 7300 + mode)
    num_pages = kp.shape[0]
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    # sequence 1 holds (20 + 1) * 4 = 84 entries: pages 0..5; slots 6.. are unused
    pt_unused = pt.clone()
    pt_unused[1, 7:] = -7
    out0 = hd.decode_step_paged(qn, kn, vn, kp.clone(), vp.clone(), pt_unused, tbt, cfg.n, T, mode,
                                cfg.scale, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    bad = pt.clone()
    bad[0, 3] = -1
    bad[2, 1] = num_pages + 5
    clamped = pt.clone()
    clamped[0, 3] = 0
    clamped[2, 1] = num_pages - 1
    ref = hd.decode_step_paged(qn, kn, vn, kp.clone(), vp.clone(), clamped, tbt, cfg.n, T, mode,
                               cfg.scale)
    got = hd.decode_step_paged(qn, kn, vn, kp.clone(), vp.clone(), bad, tbt, cfg.n, T, mode,
                               cfg.scale, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    assert torch.equal(out0.view(torch.int16),
                       hd.decode_step_paged(qn, kn, vn, kp.clone(), vp.clone(), pt, tbt, cfg.n, T,
                                            mode, cfg.scale).view(torch.int16))


def test_decode_paged_oracle_on_gathered_pages():
    """Paged decode against the oracle on the rows gathered back through the
    page table (page size 32, mixing with a window)."""
    cfg = si.DecodeCfg("dpg", 14, S=3, n=4, T=120, Hq=16, Hkv=4, D=128, scale=128 ** -0.5)
    qn, kn, vn, kc, vc, tbt = si.decode_inputs(cfg, device=DEV, S=3, T=120, tokens_before=[120, 9, 64])
    kp, vp, pt = _paged_from(kc, vc, 32, 7100)
    out = hd.decode_step_paged(qn, kn, vn, kp, vp, pt, tbt, cfg.n, 120, MIX, cfg.scale, window=200)
    torch.cuda.synchronize()
    C = kc.shape[1]
    k2 = oracle.gather_pages_ref(si.bits(kp), pt.cpu().numpy(), C)
    v2 = oracle.gather_pages_ref(si.bits(vp), pt.cpu().numpy(), C)
    ref, ref_abs = decode_pair(si.bits(qn), k2, v2, tbt.cpu().numpy(), cfg.n, MIX, cfg.scale, window=200)
    assert_close(f64(out), ref, "paged decode vs oracle", ref_abs=ref_abs)


def test_decode_stack_graph_replays_match_eager():
    """The layer-schedule step recorded as a HIP graph: three replays, each on
    new rows and new cache lengths written into the captured buffers, with an
    eager step between them, give the eager step's outputs and pools bit for bit."""
    from sequence_length_latent_amd import schedule as sch
    S, n, Hq, Hkv, D, P, T, W = 3, 4, 16, 4, 128, 16, 60, 90
    kinds = [sch.WITHIN_STREAM, sch.SLIDING, sch.FULL]
    mp = -(-((T + 1) * n) // P)
    g = torch.Generator().manual_seed(7600)
    pt = torch.randperm(S * mp + 3, generator=g)[: S * mp].reshape(S, mp).to(torch.int32).to(DEV)
    st = sch.PagedDecodeStack(kinds, S, n, Hq, Hkv, D, P, mp, W, device=DEV, page_table=pt,
                              num_pages=S * mp + 3)
    for i in range(len(kinds)):
        st.k_pools[i].copy_(_rand(st.k_pools[i].shape, 1.0, 7610 + i))
        st.v_pools[i].copy_(_rand(st.v_pools[i].shape, 1.0, 7620 + i))
    qs = [torch.empty((S, n, Hq, D), dtype=torch.bfloat16, device=DEV) for _ in kinds]
    ks = [torch.empty((S, n, Hkv, D), dtype=torch.bfloat16, device=DEV) for _ in kinds]
    vs = [torch.empty((S, n, Hkv, D), dtype=torch.bfloat16, device=DEV) for _ in kinds]
    tb = torch.zeros(S, dtype=torch.int32, device=DEV)
    outs = [torch.empty_like(q) for q in qs]
    ws = st.workspace(T)

    def fill(r):
        for i in range(len(kinds)):
            qs[i].copy_(_rand(qs[i].shape, 1.0, 7700 + 10 * r + i))
            ks[i].copy_(_rand(ks[i].shape, 1.0, 7800 + 10 * r + i))
            vs[i].copy_(_rand(vs[i].shape, 1.0, 7900 + 10 * r + i))
        tb.copy_(torch.tensor([[60, 5, 33], [12, 60, 0], [59, 1, 47]][r], dtype=torch.int32))

    fill(0)
    graph = st.capture(qs, ks, vs, tb, T, D ** -0.5, outs, ws)
    torch.cuda.synchronize()
    for r in range(3):
        fill(r)
        before = [(kp.clone(), vp.clone()) for kp, vp in zip(st.k_pools, st.v_pools)]
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        got_pools = [(kp.clone(), vp.clone()) for kp, vp in zip(st.k_pools, st.v_pools)]
        for (kp, vp), (kb, vb) in zip(zip(st.k_pools, st.v_pools), before):
            kp.copy_(kb)
            vp.copy_(vb)
        st.step(qs, ks, vs, tb, T, D ** -0.5, outs, ws)
        torch.cuda.synchronize()
        for i in range(len(kinds)):
            assert torch.equal(got[i].view(torch.int16), outs[i].view(torch.int16)), (r, i)
            assert torch.equal(got_pools[i][0], st.k_pools[i]) and torch.equal(got_pools[i][1], st.v_pools[i])


def test_decode_stack_three_layer_kinds():
    """A paged multi-layer decode step (within-stream, sliding-window and full
    mixing layers sharing one page table), each layer against the oracle."""
    from sequence_length_latent_amd import schedule as sch
    S, n, Hq, Hkv, D, P, T, W = 3, 4, 16, 4, 128, 16, 90, 150
    kinds = [sch.WITHIN_STREAM, sch.SLIDING, sch.FULL]
    mp = -(-((T + 1) * n) // P)
    g = torch.Generator().manual_seed(7200)
    pt = torch.randperm(S * mp + 5, generator=g)[: S * mp].reshape(S, mp).to(torch.int32).to(DEV)
    st = sch.PagedDecodeStack(kinds, S, n, Hq, Hkv, D, P, mp, W, device=DEV, page_table=pt,
                              num_pages=S * mp + 5)
    for i in range(len(kinds)):
        st.k_pools[i].copy_(_rand(st.k_pools[i].shape, 1.0, 7210 + i))
        st.v_pools[i].copy_(_rand(st.v_pools[i].shape, 1.0, 7220 + i))
    kp0 = [si.bits(x) for x in st.k_pools]
    vp0 = [si.bits(x) for x in st.v_pools]
    tb = torch.tensor([90, 3, 47], dtype=torch.int32, device=DEV)
    qs = [_rand((S, n, Hq, D), 1.0, 7230 + i) for i in range(3)]
    ks = [_rand((S, n, Hkv, D), 1.0, 7240 + i) for i in range(3)]
    vs = [_rand((S, n, Hkv, D), 1.0, 7250 + i) for i in range(3)]
    outs = [torch.empty_like(q) for q in qs]
    st.step(qs, ks, vs, tb, T, D ** -0.5, outs, st.workspace(T))
    torch.cuda.synchronize()
    pth, tbh = pt.cpu().numpy(), tb.cpu().numpy()
    C = mp * P
    for i, kind in enumerate(kinds):
        kc = oracle.gather_pages_ref(kp0[i], pth, C)
        vc = oracle.gather_pages_ref(vp0[i], pth, C)
        k2, v2 = oracle.decode_append_ref(kc, vc, si.bits(ks[i]), si.bits(vs[i]), tbh, n)
        mode, window = st.layer_call(i)
        ref, ref_abs = decode_pair(si.bits(qs[i]), k2, v2, tbh, n, mode, D ** -0.5, window=window)
        assert_close(f64(outs[i]), ref, f"stack layer {i} ({kind})", ref_abs=ref_abs)


def test_decode_idempotent_append_and_modes_share_cache():
    cfg = si.DECODE
    S, T = 4, 64
    qn, kn, vn, kc, vc, tb = si.decode_inputs(cfg, device=DEV, S=S, T=T)
    a = hd.decode_step(qn, kn, vn, kc, vc, tb, cfg.n, T, WITHIN, cfg.scale)
    kc1 = kc.clone()
    b = hd.decode_step(qn, kn, vn, kc, vc, tb, cfg.n, T, WITHIN, cfg.scale)
    assert torch.equal(kc.view(torch.int16), kc1.view(torch.int16))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("mode", [WITHIN, MIX])
def test_decode_matches_prefill_tail_on_gpu(mode):
    """Decode of token T equals the last n rows of a prefill over T+1 tokens."""
    n, Hq, Hkv, D, T = 4, 32, 8, 128, 150
    cfg = si.DecodeCfg("dp", 11, S=1, n=n, T=T, Hq=Hq, Hkv=Hkv, D=D, scale=D ** -0.5)
    qn, kn, vn, kc, vc, tb = si.decode_inputs(cfg, device=DEV, S=1, T=T)
    out = hd.decode_step(qn, kn, vn, kc, vc, tb, n, T, mode, cfg.scale)
    N = (T + 1) * n
    qp = _rand((1, N, Hq, D), 1.0, 81)
    qp[0, T * n:] = qn[0]
    pre = FNS[mode](qp, kc[:, :N].contiguous(), vc[:, :N].contiguous(), n, cfg.scale)
    # two GPU results, each with its own bf16 roundings: the base bar only
    assert_close(f64(out[0]), f64(pre[0, T * n:]), "decode vs prefill tail", c10=False)
