"""Run the host-side validation tests of the C ABI against the library built
with AddressSanitizer + UndefinedBehaviorSanitizer on its host code.

    LD_PRELOAD=<asan runtime> python tests/_sanitized_abi.py <sanitized .so>

The sanitized library is loaded first, so every `load()` of the binding
returns it, then pytest runs the ABI tests that call entry points (status
strings, every validation path, workspace sizing, the scale checks): each
returns its status on the host before any device work, with the sanitizers
watching every host-side access and arithmetic step.  Started as a child
process by tests/test_host_sanitizers.py.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import pytest  # noqa: E402

from sequence_length_latent_amd import _lib  # noqa: E402

lib = _lib.load(sys.argv[1])
assert lib._name == sys.argv[1]
sys.exit(pytest.main([os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-p", "no:cacheprovider",
                      "-k", "exported or status or validation or workspace or softmax_scale"]))
