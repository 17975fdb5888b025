"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and its host-side integer work agrees bit for bit with the oracle."""
import os
import re

import numpy as np
import pytest

import paged_split_kv_v2_amd as pdk
from oracle import attention as oatt
from oracle import planner as oplan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(pdk_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    lib = pdk.lib()
    names = declared_functions()
    assert len(names) >= 25
    missing = [n for n in names if not hasattr(lib, n)]
    assert missing == []
    # the binding declares a signature for each one
    assert set(names) <= set(pdk._SIGS)


def test_partition_indptr_matches_oracle():
    rng = np.random.default_rng(1)
    for S in (16, 32, 512):
        kv = rng.integers(0, 3000, size=57)
        assert np.array_equal(pdk.partition_indptr(kv, S), oatt.partition_indptr(kv, S))
    with pytest.raises(pdk.PdkError):
        pdk.partition_indptr([5, -1], 16)
    with pytest.raises(pdk.PdkError):
        pdk.partition_indptr([5], 0)


def test_validate_csr():
    pdk.validate_csr([0, 2, 3], [4, 5, 6], [20, 16], 16, 7)
    for bad in ([[1, 2, 3], [4, 5, 6], [20, 16]],   # indptr[0] != 0
                [[0, 1, 3], [4, 5, 6], [20, 16]],   # page count vs length
                [[0, 2, 3], [4, 5, 9], [20, 16]]):  # id outside the pool
        with pytest.raises(pdk.PdkError) as e:
            pdk.validate_csr(*bad, 16, 7)
        assert e.value.status == -2


def test_kill_switch_matches_oracle():
    for v in (None, "", "0", "false", "OFF", " no ", "1", "true", "On", " YES", "2", "enable"):
        assert pdk.parse_switch(v) == oplan.enabled_from_env(v)
    os.environ["PDK_TEST_SWITCH"] = " on "
    assert pdk.cascade_enabled_from_env("PDK_TEST_SWITCH") == 1
    del os.environ["PDK_TEST_SWITCH"]
    assert pdk.cascade_enabled_from_env("PDK_TEST_SWITCH") == -1


@pytest.mark.parametrize("M,Hkv,G", [(3, 2, 4), (16, 8, 4), (1, 1, 128), (5, 4, 1)])
def test_stacked_head_map_matches_oracle(M, Hkv, G):
    assert np.array_equal(pdk.stacked_head_map(M, Hkv, G), oplan.stacked_head_map(M, Hkv, G))


def test_gpu_entry_points_reject_bad_arguments_before_launch():
    lib = pdk.lib()
    # NULL pool / NULL arrays: argument errors, no device work
    assert lib.pdk_paged_decode_partial(None, None, None, 0, 8, 1.0, 32, None, 0, None, None,
                                        None) == -1
    assert lib.pdk_merge_states(None, None, 3, None, 4, 2, 6, None, None, None) == -2  # D % 4
    assert lib.pdk_merge_states(None, None, 3, None, 4, 2, 8, None, None, None) == -1
    assert b"NULL" in lib.pdk_last_error()
    assert lib.pdk_fp8_dequant_bf16(None, -1, 1.0, None, None) == -1
