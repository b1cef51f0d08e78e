"""sfa_decode_step_noalloc (split partials in the library's static per-device
scratch, no workspace) against sfa_decode_step with a caller's workspace.

Two calls in a row, the second on a smaller input, in both modes, at shapes
whose views are split (so the scratch holds partials); every output and every
appended cache row must be bit-for-bit those of the workspace entry point
(the same kernels and split plan; only the partials' stride differs).  Both
entry points are called through the C ABI with raw device pointers.
"""
import ctypes

import pytest
import torch

import sequence_length_latent_amd as hd
import sfa_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _call_both(cfg, S, T, tb, mode):
    lib = hd.load()
    qn, kn, vn, kc, vc, tbt = si.decode_inputs(cfg, device=DEV, S=S, T=T, tokens_before=tb)
    C = kc.shape[1]
    need = lib.sfa_decode_workspace_size(S, cfg.n, cfg.Hq, cfg.Hkv, cfg.D, T)
    ws = torch.empty(max(int(need), 16), dtype=torch.uint8, device=DEV)
    kc_a, vc_a = kc.clone(), vc.clone()
    kc_b, vc_b = kc.clone(), vc.clone()
    out_a = torch.empty_like(qn)
    out_b = torch.full_like(qn, float("nan"))
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.sfa_decode_step(_ptr(qn), _ptr(kn), _ptr(vn), _ptr(kc_a), _ptr(vc_a), _ptr(tbt), S, cfg.n,
                             cfg.Hq, cfg.Hkv, cfg.D, C, T, mode, cfg.scale, _ptr(ws),
                             ws.numel(), _ptr(out_a), None, stream)
    assert st == 0, hd._lib.load().hd_status_string(st)
    st = lib.sfa_decode_step_noalloc(_ptr(qn), _ptr(kn), _ptr(vn), _ptr(kc_b), _ptr(vc_b), _ptr(tbt),
                                     S, cfg.n, cfg.Hq, cfg.Hkv, cfg.D, C, T, mode, cfg.scale,
                                     _ptr(out_b), _ptr(flag), stream)
    assert st == 0, hd._lib.load().hd_status_string(st)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), (S, T, mode)
    assert torch.equal(kc_a.view(torch.int16), kc_b.view(torch.int16))
    assert torch.equal(vc_a.view(torch.int16), vc_b.view(torch.int16))


@pytest.mark.parametrize("mode", [0, 1])
def test_noalloc_matches_workspace_entry_point_twice(mode):
    cfg = si.DECODE
    # 3 sequences x 8 KV heads: views split into many 128-entry pieces, so the
    # partials (several MB) live in the scratch; then a smaller call reuses it
    _call_both(cfg, S=3, T=2000, tb=[2000, 17, 1203], mode=mode)
    _call_both(cfg, S=2, T=700, tb=[5, 700], mode=mode)


def test_noalloc_other_shapes_and_single_split():
    # D=64, n=3, 24 query rows per KV head, split views
    cfg = si.DecodeCfg("na3", 18, S=2, n=3, T=900, Hq=16, Hkv=2, D=64, scale=0.125)
    _call_both(cfg, S=2, T=900, tb=[900, 333], mode=1)
    _call_both(cfg, S=2, T=400, tb=[0, 400], mode=0)
    # enough (sequence, KV head) views that no view is split: the scratch is
    # not used at all, the attention kernel writes the rows itself
    _call_both(si.DECODE, S=64, T=64, tb=[64 - (i % 7) for i in range(64)], mode=1)
