"""The partial kernels' page-range clamp on the CPU (no GPU): whatever a
device page table holds (offsets outside [0, nnz), fewer pages than the
length needs, negative lengths or partitions), every page-id index a kernel
reads for partition p of a request, page0 + start/P .. page0 + (end-1)/P,
lies in [0, nnz); a well-formed table gives the unclamped range. The clamp
is built for the host from the same header the kernels include."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("clamp") / "part_range")
    subprocess.run([hipcc, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROOT}/include", f"-I{ROOT}/paged_split_kv_v2_amd/csrc",
                    os.path.join(ROOT, "tests", "part_range_harness.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def run(exe, cases):
    text = "\n".join(" ".join(str(int(v)) for v in c) for c in cases) + "\n"
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return np.array([[int(v) for v in line.split()] for line in out.splitlines()])


def test_every_read_stays_in_the_page_ids(harness):
    rng = np.random.default_rng(7)
    big = 2**31 - 1
    cases = []
    for _ in range(4000):
        nnz = int(rng.integers(0, 50))
        P = int(rng.choice([1, 16, 64]))
        S = P * int(rng.integers(1, 5))
        pick = lambda: int(rng.choice([rng.integers(-60, 60), -big, big, nnz]))
        cases.append((pick(), pick(), int(rng.choice([rng.integers(-100, 3000), big, -big])),
                      nnz, S, P, int(rng.choice([rng.integers(-5, 40), big // 2, -big]))))
    got = run(harness, cases)
    for (lo, hi, n, nnz, S, P, p), (page0, start, end) in zip(cases, got):
        assert 0 <= page0 <= nnz and 0 <= start <= end
        if end > start:
            first, last = page0 + start // P, page0 + (end - 1) // P
            assert 0 <= first and last < nnz, (lo, hi, n, nnz, S, P, p)
            assert end - start <= S


def test_well_formed_tables_are_unchanged(harness):
    rng = np.random.default_rng(8)
    cases, want = [], []
    for _ in range(2000):
        P = int(rng.choice([1, 16, 64]))
        S = P * int(rng.integers(1, 5))
        n = int(rng.integers(0, 2000))
        pages = -(-n // P)
        lo = int(rng.integers(0, 100))
        nnz = lo + pages + int(rng.integers(0, 10))
        p = int(rng.integers(0, max(1, -(-n // S))))
        cases.append((lo, lo + pages, n, nnz, S, P, p))
        want.append((lo, p * S, max(p * S, min(p * S + S, n))))
    assert run(harness, cases).tolist() == [list(w) for w in want]
