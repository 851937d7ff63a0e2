"""One HIP runtime and one OpenMP runtime per process, whatever the order in
which the binding and the oracle are loaded (each child process below starts
from a clean interpreter; no GPU is touched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
order = sys.argv[2].split(",")
for what in order:
    if what == "oracle":
        from oracle import oracle
        oracle._load()
        oracle.trigger_due(0, 64)
    elif what == "lsa":
        import sparse_kv_cache_lsa_amd as lsa
        lsa.load()
    elif what == "torch":
        import torch
from sparse_kv_cache_lsa_amd._abi import mapped_runtimes
print(json.dumps({k: sorted(v) for k, v in mapped_runtimes().items()}))
"""


@pytest.mark.parametrize("order", ["oracle,lsa", "lsa,oracle", "oracle,torch,lsa",
                                   "lsa,torch,oracle"])
def test_single_runtime_of_each_kind(order):
    import json
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, order], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    maps = json.loads(r.stdout.strip().splitlines()[-1])
    assert len(maps["libamdhip64"]) == 1, maps
    assert len(maps["libhsa-runtime64"]) == 1, maps
    assert len(maps["libgomp"]) == 1, maps
