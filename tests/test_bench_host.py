"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic flop
counts of the timed step, and the kernel-class map of the counter summaries."""

import os
import subprocess
import sys

import bench
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_side_sums_closed_forms():
    # 4096 = 8 whole blocks of 512; 5461 = 21 blocks of 256 and one of 85
    assert bench.side_sums(4096, 512) == (8 * 512**2, 8 * 512**3)
    assert bench.side_sums(5461, 256) == (21 * 256**2 + 85**2, 21 * 256**3 + 85**3)
    assert bench.side_sums(100, 128) == (100**2, 100**3)


def test_llama8b_step_flops():
    """W~ contractions 4 T m n per linear, block products 6 T (sum r^2 of both
    sides) per linear (forward, backward apply and block gradients), CNP 16 sum
    r^3 (build 4, chain rule 12)."""
    wl = WORKLOADS["llama8b"]
    g, a, c = bench.step_flops(wl, wl.T)
    T = 8192
    lin = [(4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096), (4096, 14336), (4096, 14336), (14336, 4096)]
    assert g == sum(4.0 * T * m * n for m, n in lin)
    r2 = lambda d: (d // 512) * 512**2
    r3 = lambda d: (d // 512) * 512**3
    assert a == sum(6.0 * T * (r2(m) + r2(n)) for m, n in lin)
    assert c == sum(16.0 * (r3(m) + r3(n)) for m, n in lin)
    assert abs((g + a + c) / 1e12 - 9.552) < 1e-3


def test_kernel_classes():
    k = bench.kernel_class
    assert k("void (anonymous namespace)::k_gemm<px::DCfg<256, 256, 64>>(...)") == "W~ contractions"
    assert k("void (anonymous namespace)::k_gemm_group<px::DCfg<256, 256, 64>>(GemmTable)") == "W~ contractions"
    assert k("k_apply_stream<512, 32, 3, false>") == "block products"
    assert k("k_scatter_lds<unsigned short>") == "permutations"
    assert k("k_permute_lds<unsigned short>") == "permutations"
    assert k("k_adam<4>") == "optimiser step"
    assert k("k_cnp_grad1<...>") == "CNP products"
    assert k("at::native::vectorized_elementwise_kernel") is None
