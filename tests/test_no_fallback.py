"""The Python binding has no implementation of its own: without libdsa.so it
raises, and it refuses host tensors instead of computing on the CPU."""
import subprocess
import sys

import pytest
import torch

import long_context_02_amd as dsa


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(dsa, "_lib", None)
    monkeypatch.setattr(dsa, "_LIB_PATH", str(tmp_path / "libdsa.so"))
    with pytest.raises(RuntimeError, match="is missing"):
        dsa.lib()


def test_host_tensors_are_refused():
    scores = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        dsa.topk_select(scores, 8, 60)
    q = torch.zeros(1, 2, 128, 576, dtype=torch.bfloat16)
    kv = torch.zeros(1, 64, 576, dtype=torch.bfloat16)
    idx = torch.zeros(1, 2, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        dsa.sparse_mla_attn(q, kv, idx, 512, 0.04)


def test_package_imports_nothing_from_the_oracle():
    # the product modules must not reach the CPU reference implementation
    code = ("import sys, long_context_02_amd, long_context_02_amd.synth, long_context_02_amd.build; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=str(__import__("pathlib").Path(dsa.__file__).resolve().parents[1]))
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "False"
