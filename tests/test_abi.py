"""The C-ABI library loads on a machine without a GPU and exports every symbol the headers in
include/ declare; size queries are host arithmetic and need no device."""
import ctypes
import os
import re

import pytest

import post_weight_quantization_amd as pwq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"\b(gptq_\w+)\s*\(", src)
    return sorted(set(names))


def test_headers_declare_the_boundary():
    names = _declared()
    for n in ("gptq_fold", "gptq_ladder", "gptq_sweep", "gptq_fold_workspace_size",
              "gptq_sweep_workspace_size", "gptq_status_string"):
        assert n in names


@pytest.mark.parametrize("name", _declared())
def test_library_exports_declared_symbol(name):
    lib = ctypes.CDLL(pwq.LIB_PATH)
    assert hasattr(lib, name), name


def test_workspace_sizes_are_host_arithmetic():
    lib = pwq.load()
    assert lib.gptq_fold_workspace_size(0) == 0
    np_ = 17408
    assert lib.gptq_fold_workspace_size(17408) >= 2 * 4 * np_ * np_
    assert lib.gptq_fold_workspace_size(100) >= 2 * 4 * 128 * 128
    assert lib.gptq_sweep_workspace_size(5120, 17408) >= 4 * 5120 * 17408
    assert lib.gptq_status_string(4).decode().startswith("damping")


def test_product_path_has_no_cpu_fallback(monkeypatch):
    """Without a visible GPU the binding refuses instead of computing anything elsewhere."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(RuntimeError):
        pwq.require_native()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with a message before touching one."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_packed_layout_is_the_pages_poff():
    """The packed Hessian layout: element (i, j >= i) at poff(i) + (j - i) with
    poff(r) = r (2n - r + 1) / 2 (page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs", poff),
    n (n + 1) / 2 floats; the tests' packing helper produces exactly that order, and the
    header's marker value is the binding's."""
    import re

    import torch

    from packing import pack_upper, unpack_upper
    for n in (1, 2, 5, 17, 64):
        H = torch.arange(n * n, dtype=torch.float64).reshape(n, n)
        Hp = pack_upper(H)
        assert Hp.numel() == n * (n + 1) // 2
        for i in range(n):
            poff = i * (2 * n - i + 1) // 2
            for j in range(i, n):
                assert Hp[poff + j - i] == H[i, j]
        assert torch.equal(unpack_upper(Hp, n), torch.triu(H))
    hdr = open(os.path.join(ROOT, "include", "gptq.h")).read()
    m = re.search(r"#define GPTQ_PACKED_UPPER \(\(int64_t\)(-?\d+)\)", hdr)
    assert m and int(m.group(1)) == pwq.GPTQ_PACKED_UPPER
    with pytest.raises(ValueError):
        pwq._hessian(torch.zeros(11))  # 11 is not n (n + 1) / 2
