"""Parity of the opt-in persistent prefill kernel (GQA_ATTN_PERSIST=1).

The kernel choice is read from the environment once per process, so the
plain-case parity tests (16-bit, online softmax, no mask: every form pair and
causal kind, head groups and head sizes, batch sizes of the dispatch map,
ragged batches with empty sequences, packed = padded bitwise, the bf16
ragged causal workload at full size, and the split-KV path) run once more in
one child process with the persistent kernel selected.  Same bar as the
parity tests themselves: elementwise against the oracle.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

SELECT = ("test_forms_causal or test_head_groups_and_head_size or test_dispatch_map_batch_sizes "
          "or test_ragged_with_empty_sequences or test_packed_equals_padded "
          "or test_workload_sampled and 2 or test_split")


def test_persistent_kernel_parity():
    env = dict(os.environ, GQA_ATTN_PERSIST="1")
    print("persistent kernel parity: child pytest", flush=True)
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "gpu",
         os.path.join(ROOT, "tests", "test_gpu_parity.py"), "-k", SELECT],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    m = re.search(r"(\d+) passed", r.stdout)
    assert m and int(m.group(1)) >= 40, tail  # the selection ran (about 45 cases)
    print(m.group(0), flush=True)
