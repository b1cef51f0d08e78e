"""Host logic of bench.py that needs no GPU: the one-GPU guard and the rule
that measured HBM traffic is reported only for the kernel sources it was
taken on."""
import hashlib
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CSRC = os.path.join(ROOT, "sequence_length_latent_amd", "csrc")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("key", sorted(bench.KERNEL_SOURCES))
def test_source_hash_covers_every_source_file(key):
    h = hashlib.sha256()
    for f in bench.KERNEL_SOURCES[key]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    assert bench.kernel_source_sha256(key) == h.hexdigest()
    # the prefill kernel's generated assembly is part of its source
    if key == "prefill_source_sha256":
        assert "prefill_asm.h" in bench.KERNEL_SOURCES[key]


def _fake_tree(tmp_path):
    """A copy of the kernel sources and a traffic summary taken on them."""
    csrc = tmp_path / "sequence_length_latent_amd" / "csrc"
    csrc.mkdir(parents=True)
    for files in bench.KERNEL_SOURCES.values():
        for f in files:
            shutil.copy(os.path.join(CSRC, f), csrc / f)
    (tmp_path / "profiles").mkdir()
    return csrc


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    csrc = _fake_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    t = {"prefill_source_sha256": bench.kernel_source_sha256("prefill_source_sha256"),
         "decode_source_sha256": bench.kernel_source_sha256("decode_source_sha256"),
         "sfa_prefill_kernel_n4": {"within": {"read": 100.0, "write": 50.0},
                                   "mix": {"read": 300.0, "write": 50.0}},
         "decode_attend_kernel": {"within": {"read": 7.0, "write": 1.0},
                                  "mix": {"read": 9.0, "write": 1.0}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(t))
    assert bench.measured_traffic("sfa_prefill_kernel_n4", "prefill.hip") == 250
    assert bench.measured_traffic("decode_attend_kernel", "decode.hip") == 9
    # any change to a source the kernel is built from voids its figures
    with open(csrc / "prefill_asm.h", "a") as fh:
        fh.write("\n")
    assert bench.measured_traffic("sfa_prefill_kernel_n4", "prefill.hip") is None
    assert bench.measured_traffic("decode_attend_kernel", "decode.hip") == 9
    with open(csrc / "common.h", "a") as fh:
        fh.write("\n")
    assert bench.measured_traffic("decode_attend_kernel", "decode.hip") is None


def test_traffic_missing_summary_is_none(tmp_path, monkeypatch):
    _fake_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("sfa_prefill_kernel_n4", "prefill.hip") is None
