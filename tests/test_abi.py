"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and rejects invalid arguments on the host before launching
anything (these paths return before any HIP call)."""
import os
import re

import pytest

import sequence_length_latent_amd as hd
from sequence_length_latent_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hd_sfa.h")

OK, NULL, SHAPE, UNSUP, CAP, LAUNCH, WS, SCRATCH = range(8)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hd_\w+|sfa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return hd.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == {"hd_status_string", "hd_abi_version", "hd_expand",
                          "hd_final_stream_rows", "hd_cyclic_replicate", "sfa_stream_attn",
                          "sfa_mix_attn", "sfa_mix_attn_window", "sfa_attn_fwd",
                          "sfa_attn_bwd_workspace_size", "sfa_attn_bwd",
                          "sfa_attn_fwd_window", "sfa_attn_bwd_window",
                          "sfa_decode_workspace_size", "sfa_decode_step",
                          "sfa_decode_step_window", "sfa_decode_step_paged",
                          "sfa_decode_step_noalloc", "sfa_attn_split_workspace_size",
                          "sfa_attn_split"}
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_status_strings(lib):
    assert lib.hd_abi_version() == 2
    seen = set()
    for code in range(8):
        s = lib.hd_status_string(code).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.hd_status_string(99).decode() == "unknown status"
    assert lib.hd_status_string(-1).decode() == "unknown status"


FAKE = 0x10000  # 16-byte aligned non-null host value; never dereferenced on error paths


def test_expand_validation(lib):
    assert lib.hd_expand(None, 1, 4, FAKE, 2, 10, 8, FAKE, None, None) == NULL
    assert lib.hd_expand(FAKE, 1, 4, FAKE, 2, 10, 12, FAKE, None, None) == SHAPE   # H % 8
    assert lib.hd_expand(FAKE, 1, 4, FAKE + 2, 2, 10, 8, FAKE, None, None) == SHAPE  # align
    assert lib.hd_expand(FAKE, 1, 4, FAKE, 0, 10, 8, FAKE, None, None) == SHAPE    # n = 0
    assert lib.hd_expand(FAKE, -1, 4, FAKE, 2, 10, 8, FAKE, None, None) == SHAPE
    # zero work: OK without touching anything, even with NULL buffers
    assert lib.hd_expand(None, 0, 4, None, 2, 10, 8, None, None, None) == OK
    assert lib.hd_expand(None, 3, 0, None, 2, 10, 8, None, None, None) == OK
    # one workgroup per output row: B*L*n must stay below 2^31
    assert lib.hd_expand(FAKE, 1 << 16, 1 << 14, FAKE, 2, 10, 8, FAKE, None, None) == UNSUP


@pytest.mark.parametrize("fn", ["sfa_stream_attn", "sfa_mix_attn"])
def test_prefill_validation(lib, fn):
    f = getattr(lib, fn)
    assert f(None, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, 1.0, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 3, 128, 1.0, None) == SHAPE     # Hq % Hkv
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 96, 1.0, None) == UNSUP      # D
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 0, 8, 4, 2, 128, 1.0, None) == SHAPE     # n
    assert f(FAKE, FAKE + 8, FAKE, FAKE, 1, 2, 8, 4, 2, 128, 1.0, None) == SHAPE  # align
    assert f(None, None, None, None, 0, 2, 8, 4, 2, 128, 1.0, None) == OK
    assert f(None, None, None, None, 2, 2, 0, 4, 2, 128, 1.0, None) == OK


def test_stream_copy_validation(lib):
    f, c = lib.hd_final_stream_rows, lib.hd_cyclic_replicate
    assert f(FAKE, 1, 0, 4, 8, FAKE + 4096, None) == SHAPE         # n
    assert f(FAKE, 1, 2, 4, 12, FAKE + 4096, None) == SHAPE        # H % 8
    assert f(FAKE + 8, 1, 2, 4, 8, FAKE + 4096, None) == SHAPE     # alignment
    assert f(FAKE, 1, 2, 4, 8, FAKE + 16, None) == SHAPE           # out overlaps x
    assert f(None, 1, 2, 4, 8, FAKE, None) == NULL
    assert f(None, 0, 2, 4, 8, None, None) == OK                   # empty
    assert c(FAKE, 0, 5, 8, FAKE + 4096, 2, None) == SHAPE         # n_old
    assert c(FAKE, 2, 5, 8, FAKE + 16, 4, None) == SHAPE           # partial overlap
    assert c(FAKE, 2, 5, 12, FAKE + 4096, 4, None) == SHAPE        # H % 8
    assert c(None, 2, 5, 8, FAKE, 4, None) == NULL
    assert c(FAKE, 4, 5, 8, FAKE, 2, None) == OK                   # in place, nothing to add
    assert c(None, 2, 0, 8, None, 4, None) == OK                   # empty tables


def test_training_entry_validation(lib):
    f, b, ws = lib.sfa_attn_fwd, lib.sfa_attn_bwd, lib.sfa_attn_bwd_workspace_size
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, 1.0, 2, None) == SHAPE     # mode
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 1, 2, 8, 4, 2, 128, 1.0, 1, None) == SHAPE  # lse align
    assert f(None, FAKE, FAKE, FAKE, None, 1, 2, 8, 4, 2, 128, 1.0, 0, None) == NULL
    assert f(None, None, None, None, None, 0, 2, 8, 4, 2, 128, 1.0, 0, None) == OK
    assert ws(2, 4, 1024, 32) == 2 * 32 * 4096 * 4
    assert ws(-1, 4, 8, 2) == 0
    args = [FAKE] * 8
    assert b(*args, 1, 2, 8, 4, 2, 128, 1.0, 3, FAKE, 1 << 20, None) == SHAPE           # mode
    assert b(*args, 1, 2, 8, 4, 3, 128, 1.0, 0, FAKE, 1 << 20, None) == SHAPE           # Hq % Hkv
    assert b(*args, 1, 2, 8, 4, 2, 96, 1.0, 0, FAKE, 1 << 20, None) == UNSUP            # D
    assert b(*args, 1, 2, 8, 4, 2, 128, 1.0, 0, FAKE, 16, None) == WS                   # workspace
    assert b(None, *args[1:], 1, 2, 8, 4, 2, 128, 1.0, 0, FAKE, 1 << 20, None) == NULL
    assert b(*args, 0, 2, 8, 4, 2, 128, 1.0, 0, FAKE, 0, None) == OK                    # empty


def test_training_window_validation(lib):
    f, b = lib.sfa_attn_fwd_window, lib.sfa_attn_bwd_window
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, 1.0, 0, None) == SHAPE     # window < 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 1, 2, 8, 4, 2, 128, 1.0, 4, None) == SHAPE  # lse align
    assert f(None, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, 1.0, 4, None) == NULL
    assert f(None, None, None, None, None, 0, 2, 8, 4, 2, 128, 1.0, 4, None) == OK        # empty
    args = [FAKE] * 8
    assert b(*args, 1, 2, 8, 4, 2, 128, 1.0, 0, FAKE, 1 << 20, None) == SHAPE           # window < 1
    assert b(*args, 1, 2, 8, 4, 2, 128, 1.0, 1 << 40, FAKE, 1 << 20, None) == SHAPE     # > 2^31 - 1
    assert b(*args, 1, 2, 8, 4, 3, 128, 1.0, 4, FAKE, 1 << 20, None) == SHAPE           # Hq % Hkv
    assert b(*args, 1, 2, 8, 4, 2, 96, 1.0, 4, FAKE, 1 << 20, None) == UNSUP            # D
    assert b(*args, 1, 2, 8, 4, 2, 128, 1.0, 4, FAKE, 16, None) == WS                   # workspace
    assert b(*args, 0, 2, 8, 4, 2, 128, 1.0, 4, FAKE, 0, None) == OK                    # empty


def test_window_validation(lib):
    f = lib.sfa_mix_attn_window
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, 1.0, 0, None) == SHAPE      # window < 1
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, 1.0, -5, None) == SHAPE
    assert f(None, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, 1.0, 16, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 3, 128, 1.0, 16, None) == SHAPE     # Hq % Hkv
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 96, 1.0, 16, None) == UNSUP      # D
    assert f(None, None, None, None, 0, 2, 8, 4, 2, 128, 1.0, 16, None) == OK        # empty


def test_decode_workspace_size(lib):
    # n4 decode workload: 64 sequences, 4096 cached tokens, 32/8 heads, D=128
    size = lib.sfa_decode_workspace_size(64, 4, 32, 8, 128, 4096)
    rows = 4 * (32 // 8)
    per = 64 * 8 * rows * (128 + 2) * 4
    assert size > 0 and size % per == 0
    assert lib.sfa_decode_workspace_size(64, 4, 32, 8, 96, 4096) == 0       # D
    assert lib.sfa_decode_workspace_size(64, 4, 32, 7, 128, 4096) == 0      # Hq % Hkv
    assert lib.sfa_decode_workspace_size(64, 8, 128, 8, 128, 4096) == 0     # rows > 64


def test_decode_validation(lib):
    args = dict(S=2, n=4, Hq=8, Hkv=2, D=128, C=4 * 11, maxT=10, mode=1)

    def call(**kw):
        a = dict(args, **kw)
        ws = kw.get("ws", FAKE)
        wsb = kw.get("wsb", 1 << 30)
        return lib.sfa_decode_step(kw.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, a["S"], a["n"],
                                   a["Hq"], a["Hkv"], a["D"], a["C"], a["maxT"], a["mode"], 0.1,
                                   ws, wsb, FAKE, None, None)

    assert call(q=None) == NULL
    assert call(C=4 * 11 - 1) == CAP
    assert call(mode=2) == SHAPE
    assert call(Hkv=3) == SHAPE
    assert call(D=80) == UNSUP
    assert call(ws=None) == WS
    assert call(wsb=16) == WS
    assert call(S=0, q=None) == OK


def test_decode_noalloc_validation(lib):
    """The no-workspace decode validates like sfa_decode_step and rejects, on
    the host and before any launch, a call whose split partials would not fit
    its 16 MiB static scratch."""
    def call(S=2, n=4, Hq=8, Hkv=2, D=128, C=4 * 11, maxT=10, mode=1, q=FAKE):
        return lib.sfa_decode_step_noalloc(q, FAKE, FAKE, FAKE, FAKE, FAKE, S, n, Hq, Hkv, D, C, maxT,
                                           mode, 0.1, FAKE, None, None)

    assert call(q=None) == NULL
    assert call(C=4 * 11 - 1) == CAP
    assert call(mode=2) == SHAPE
    assert call(Hkv=3) == SHAPE
    assert call(D=80) == UNSUP
    assert call(S=0, q=None) == OK
    # 16 sequences x 8 KV heads (128 views, 4 splits each) x 64 query rows x
    # 130 floats: 17.0 MB of partials > 16 MiB
    big = dict(S=16, n=8, Hq=64, Hkv=8, D=128, maxT=4095, C=8 * 4096)
    assert call(**big) == SCRATCH
    assert lib.hd_status_string(SCRATCH).decode().startswith("call needs more")


def test_decode_window_validation(lib):
    def call(window, C=4 * 11, ws=FAKE, wsb=1 << 30, q=FAKE, S=2):
        return lib.sfa_decode_step_window(q, FAKE, FAKE, FAKE, FAKE, FAKE, S, 4, 8, 2, 128, C, 10,
                                          window, 0.1, ws, wsb, FAKE, None, None)

    assert call(0) == SHAPE
    assert call(-3) == SHAPE
    assert call(16, q=None) == NULL
    assert call(16, C=4 * 11 - 1) == CAP
    assert call(16, wsb=16) == WS
    assert call(16, S=0, q=None) == OK


def test_decode_paged_validation(lib):
    def call(P=16, num_pages=64, mpps=8, mode=1, window=0, C=None, pt=FAKE, q=FAKE, S=2, wsb=1 << 30):
        return lib.sfa_decode_step_paged(q, FAKE, FAKE, FAKE, FAKE, pt, FAKE, S, 4, 8, 2, 128, P,
                                         num_pages, mpps, 10, mode, window, 0.1, FAKE, wsb, FAKE, None,
                                         None)

    assert call(P=12) == SHAPE                  # not a power of two
    assert call(P=0) == SHAPE
    assert call(num_pages=0) == SHAPE
    assert call(mode=0, window=8) == SHAPE      # window on a within-stream layer
    assert call(window=-1) == SHAPE
    assert call(mpps=2) == CAP                  # 2 pages x 16 < 11 tokens x 4 streams
    assert call(pt=None) == NULL
    assert call(wsb=16) == WS
    assert call(S=0, q=None, pt=None) == OK
    assert call(P=1 << 16, num_pages=(1 << 16) + 1) == UNSUP   # pool rows past 32 bits


def test_layer_schedules():
    """The pages' counts (80B: 6 full + 23 sliding-window + 20 within-stream of
    49; 617B: 25 full + 69 within-stream of 94), each kind spread evenly."""
    from sequence_length_latent_amd import schedule as sch
    for name, total in (("80B", 49), ("617B", 94)):
        kinds = sch.layer_kinds(name)
        assert len(kinds) == total
        for kind, count in sch.SCHEDULES[name].items():
            at = [i for i, k in enumerate(kinds) if k == kind]
            assert len(at) == count
            gaps = [b - a for a, b in zip(at, at[1:])]
            assert max(gaps, default=0) <= -(-total // count) + 1, (name, kind, gaps)


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        hd.stream_attn(q, q, q, 2, 1.0)
    with pytest.raises(ValueError):
        hd.expand(torch.zeros(1, 2, dtype=torch.int32), torch.zeros(2, 5, 8, dtype=torch.bfloat16))


def test_library_is_gfx950_only():
    """The shared object carries only gfx950 device code."""
    data = open(_lib.LIB_PATH, "rb").read()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100", b"sm_"):
        assert other + b"\x00" not in data and b"amdgcn-amd-amdhsa--" + other not in data


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "sequence_length_latent_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_no_kernel_spills_to_scratch():
    """Every kernel of the library keeps its working set in registers and LDS:
    no scratch memory and no VGPR spills (from the compiler's resource report
    that the build writes next to the library).  SGPR spills are allowed: with
    no scratch they go to lanes of a VGPR (the prefill kernels park the
    diagonal tile's hoisted lane masks there, read once per work item)."""
    import json
    import os
    from sequence_length_latent_amd import build as b
    assert os.path.exists(b.RESOURCES), "build the library first (python -m sequence_length_latent_amd.build)"
    res = json.load(open(b.RESOURCES))
    kernels = [k for k in res if "_kernel" in k]
    # every kernel family of the path is reported
    for fam in ("expand_kernel", "sfa_prefill_kernel", "decode_append_kernel", "decode_attend_kernel",
                "decode_combine_kernel", "rowcopy_kernel", "dq_kernel", "dkv_kernel"):
        assert any(fam in k for k in kernels), fam
    for k in kernels:
        r = res[k]
        assert r.get("scratch_bytes_per_lane", 0) == 0, (k, r)
        assert r.get("vgpr_spill", 0) == 0, (k, r)
        assert r.get("lds_bytes", 0) <= 160 * 1024, (k, r)


def test_softmax_scale_must_be_finite_and_positive(lib):
    """The kernels mask with -inf and track the max of raw scores times the
    scale, so every attention entry point rejects a scale that is zero,
    negative, infinite or NaN before any launch."""
    bad = (0.0, -0.125, float("inf"), float("nan"))
    args8 = [FAKE] * 8
    for sc in bad:
        assert lib.sfa_stream_attn(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, sc, None) == SHAPE
        assert lib.sfa_mix_attn(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, sc, None) == SHAPE
        assert lib.sfa_mix_attn_window(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, sc, 4, None) == SHAPE
        assert lib.sfa_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, sc, 1, None) == SHAPE
        assert lib.sfa_attn_fwd_window(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 4, 2, 128, sc, 4, None) == SHAPE
        assert lib.sfa_attn_bwd(*args8, 1, 2, 8, 4, 2, 128, sc, 1, FAKE, 1 << 20, None) == SHAPE
        assert lib.sfa_attn_bwd_window(*args8, 1, 2, 8, 4, 2, 128, sc, 4, FAKE, 1 << 20, None) == SHAPE
        assert lib.sfa_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 8, 2, 128, 44, 10, 1, sc,
                                   FAKE, 1 << 30, FAKE, None, None) == SHAPE
        assert lib.sfa_decode_step_window(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 8, 2, 128, 44, 10, 8, sc,
                                          FAKE, 1 << 30, FAKE, None, None) == SHAPE
        assert lib.sfa_decode_step_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 8, 2, 128, 16, 64, 8,
                                         10, 1, 0, sc, FAKE, 1 << 30, FAKE, None, None) == SHAPE


def _split_bytes(items_split, D):
    """Workspace of the key-split forward, restated: a 4-byte counter per
    (item, wave) rounded up to 256 bytes, then two slots per (item, wave) of
    64 lanes x (D/2 accumulators + m + l) floats."""
    counters = -(-items_split * 8 * 4 // 256) * 256
    return counters + items_split * 2 * 8 * 64 * (D // 2 + 2) * 4


def test_split_workspace_size(lib):
    f = lib.sfa_attn_split_workspace_size
    # n = 1, L = 2048, 32 / 8 heads: 32 query tiles of 64 rows x 8 KV heads;
    # all but the first query tile have two or more key tiles
    assert f(1, 1, 2048, 32, 8, 128, 1) == _split_bytes(31 * 8, 128)
    # within-stream, n = 4, L = 1024, batch 2: 16 query tiles x 2 x 4 x 8 views
    assert f(2, 4, 1024, 32, 8, 128, 0) == _split_bytes(15 * 2 * 4 * 8, 128)
    # G = 8 packs 32 query rows per item: tiles 0 and 1 end inside key tile 0
    assert f(1, 1, 256, 16, 2, 64, 1) == _split_bytes(6 * 2, 64)
    # G = 2 packs 128 rows per item: every item has two or more key tiles
    assert f(1, 2, 200, 4, 2, 128, 1) == _split_bytes(4 * 2, 128)
    assert f(1, 1, 64, 8, 2, 128, 1) == 0          # one key tile: nothing to split
    for bad in ((0, 1, 64, 8, 2, 128, 1), (1, 1, 64, 8, 3, 128, 1), (1, 1, 64, 8, 2, 96, 1),
                (1, 1, 64, 8, 2, 128, 2), (1, 0, 64, 8, 2, 128, 1)):
        assert f(*bad) == 0, bad


def test_split_validation(lib):
    f = lib.sfa_attn_split
    need = lib.sfa_attn_split_workspace_size(1, 1, 2048, 32, 8, 128, 1)
    args = (1, 1, 2048, 32, 8, 128, 1.0)
    assert f(FAKE, FAKE, FAKE, FAKE, None, *args, 2, FAKE, need, None) == SHAPE      # mode
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 2, *args, 1, FAKE, need, None) == SHAPE  # lse align
    assert f(FAKE, FAKE, FAKE, FAKE, None, *args, 1, None, need, None) == WS         # no workspace
    assert f(None, FAKE, FAKE, FAKE, None, *args, 1, FAKE, need, None) == NULL
    # 256 items: split on a GPU of 256 compute units (the count taken when
    # none can be queried): a short or misaligned workspace is refused
    assert f(FAKE, FAKE, FAKE, FAKE, None, *args, 1, FAKE, need - 1, None) == WS
    assert f(FAKE, FAKE, FAKE, FAKE, None, *args, 1, FAKE + 8, need, None) == WS
    assert f(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 2048, 32, 8, 96, 1.0, 1, FAKE, need, None) == UNSUP
    # a one-tile layer needs no workspace: the check passes it on (zero work: OK)
    assert f(None, None, None, None, None, 0, 1, 64, 8, 2, 128, 1.0, 1, None, 0, None) == OK
