"""Argument checks of the C ABI (no GPU work): every call below must be
refused on the host, before any launch or copy, with the documented status
and a message. Device pointers are stand-in addresses that are never
dereferenced when the checks hold. The module is skipped where a GPU is
visible, so that a missing check could never send those addresses to a
kernel."""
import ctypes

import numpy as np
import pytest
import torch

import paged_split_kv_v2_amd as pdk

if torch.cuda.device_count() > 0:
    pytest.skip("host-side argument checks run where no GPU is visible", allow_module_level=True)

ERR_ARG, ERR_SHAPE, ERR_WORKSPACE = -1, -2, -5
FAKE = 0x100000  # 16-byte aligned stand-in for a device address


def lib():
    return pdk.lib()


BF16 = 1  # pdk_dtype


def pool(P=16, Hkv=2, D=64, dtype=BF16):
    return pdk._Pool(k=FAKE, v=FAKE, num_blocks=64, page_size=P, num_kv_heads=Hkv,
                     head_dim_k=D, head_dim_v=D, dtype=dtype, k_scale=1.0, v_scale=1.0)


def dev_csr(batch=2):
    return pdk._CSR(indptr=FAKE, indices=FAKE, kv_len=FAKE, batch=batch, nnz=8)


def status(rc, code, word):
    assert rc == code, (rc, lib().pdk_last_error())
    assert word.encode() in lib().pdk_last_error().lower(), lib().pdk_last_error()


def test_multi_token_partial_rejects_bad_token_count_and_causal_flag():
    p, c = pool(), dev_csr()
    for T, causal in ((0, 1), (2, 2)):
        rc = lib().pdk_paged_multi_token_partial(ctypes.byref(p), ctypes.byref(c), FAKE, 1, 4, T,
                                                 causal, 0.125, 32, FAKE, 4, FAKE, FAKE, None)
        status(rc, ERR_ARG, "q_tokens")


def test_partition_size_must_be_a_multiple_of_the_page():
    p, c = pool(), dev_csr()
    rc = lib().pdk_paged_decode_partial(ctypes.byref(p), ctypes.byref(c), FAKE, 1, 4, 0.125, 24,
                                        FAKE, 4, FAKE, FAKE, None)
    status(rc, ERR_ARG, "multiple of page_size")


def test_flat_decode_rejects_a_small_workspace():
    p, c = pool(), dev_csr()
    need = lib().pdk_decode_flat_workspace_bytes(4, 4, 64)
    assert need > 0
    rc = lib().pdk_decode_flat(ctypes.byref(p), ctypes.byref(c), FAKE, 1, 4, 0.125, 32, FAKE, 4,
                               FAKE, FAKE, FAKE, need - 1, None)
    status(rc, ERR_WORKSPACE, "workspace")
    rc = lib().pdk_multi_token_flat(ctypes.byref(p), ctypes.byref(c), FAKE, 1, 4, 2, 1, 0.125, 32,
                                    FAKE, 4, FAKE, FAKE, FAKE,
                                    lib().pdk_decode_flat_workspace_bytes(4, 8, 64) - 1, None)
    status(rc, ERR_WORKSPACE, "workspace")


def host_csr(lists, lens):
    indptr = np.cumsum([0] + [len(x) for x in lists]).astype(np.int32)
    indices = np.asarray([p for x in lists for p in x], np.int32)
    kv_len = np.asarray(lens, np.int32)
    keep = (indptr, indices, kv_len)
    return pdk._CSR(indptr=indptr.ctypes.data, indices=indices.ctypes.data,
                    kv_len=kv_len.ctypes.data, batch=len(lens), nnz=int(indptr[-1])), keep


def params(**kw):
    pr = pdk._Params()
    lib().pdk_cascade_params_default(ctypes.byref(pr))
    for k, v in kw.items():
        setattr(pr, k, v)
    return pr


@pytest.mark.parametrize("kw,word", [
    (dict(l1_partition_tokens=24), "multiples of page_size"),
    (dict(l0_partition_tokens=0), "multiples of page_size"),
    (dict(min_members=1), "thresholds"),
    (dict(fuse_levels=2), "fuse_levels"),
])
def test_cascade_plan_rejects_bad_parameters(kw, word):
    c, keep = host_csr([[0, 1, 2], [0, 1, 3]], [40, 40])
    plan = ctypes.c_void_p()
    rc = lib().pdk_cascade_plan_create(ctypes.byref(c), 16, ctypes.byref(params(**kw)),
                                       ctypes.byref(plan))
    status(rc, ERR_ARG, word)
    assert not plan.value


def test_cascade_plan_must_be_uploaded_to_the_workspace_it_runs_from():
    c, keep = host_csr([[0, 1, 2], [0, 1, 3]], [40, 40])
    plan = ctypes.c_void_p()
    assert lib().pdk_cascade_plan_create(ctypes.byref(c), 16,
                                         ctypes.byref(params(enabled=1, min_shared_pages=1)),
                                         ctypes.byref(plan)) == 0
    try:
        p = pool()
        need = lib().pdk_cascade_workspace_bytes(plan, 4, 64)
        assert need > 0
        # too small to upload into: refused before the copy
        status(lib().pdk_cascade_plan_upload(plan, FAKE, 16, None), ERR_WORKSPACE, "workspace")
        # never uploaded: the run is refused
        rc = lib().pdk_run_cascade_decode(plan, ctypes.byref(p), FAKE, 1, 4, 0.125, FAKE, FAKE,
                                          FAKE, need, None)
        status(rc, ERR_WORKSPACE, "uploaded")
    finally:
        lib().pdk_cascade_plan_free(plan)


def test_page_table_checks_name_the_violation():
    # page count disagrees with the length; an id outside the pool
    for lists, lens in (([[0, 1], [2]], [40, 10]), ([[0, 1, 9], [2]], [40, 10])):
        c, keep = host_csr(lists, lens)
        assert lib().pdk_validate_csr(ctypes.byref(c), 16, 8) == ERR_SHAPE
        assert lib().pdk_last_error()
    c, keep = host_csr([[0, 1, 2], [3]], [40, 10])
    assert lib().pdk_validate_csr(ctypes.byref(c), 16, 8) == 0


ERR_UNSUPPORTED = -4
FP8 = 2  # pdk_dtype (PDK_FP8_E4M3)


@pytest.mark.parametrize("P,Hkv,Hq,D,Dv,dtype,limit", [
    (16, 8, 32, 128, 128, BF16, 1023),   # vector path (4 rows per KV head)
    (16, 2, 32, 128, 128, BF16, 511),    # LDS-ring path (16 rows per KV head)
    (2, 1, 32, 128, 128, BF16, 1023),    # matrix-core path on 2-token pages (32 rows)
    (64, 1, 128, 576, 512, FP8, 255),    # latent fp8 path (128 rows)
])
def test_partition_spanning_too_many_pages_is_unsupported(P, Hkv, Hq, D, Dv, dtype, limit):
    """Each partial kernel stages a partition's page ids in LDS, so a
    partition of more pages than its table holds is refused on the host with
    PDK_ERR_UNSUPPORTED (one page over the limit that
    pdk_paged_decode_partial documents for the path)."""
    p = pdk._Pool(k=FAKE, v=None if Dv != D else FAKE, num_blocks=4096, page_size=P,
                  num_kv_heads=Hkv, head_dim_k=D, head_dim_v=Dv, dtype=dtype, k_scale=0.01,
                  v_scale=0.01)
    c = dev_csr()
    rc = lib().pdk_paged_decode_partial(ctypes.byref(p), ctypes.byref(c), FAKE, BF16, Hq, 0.125,
                                        (limit + 1) * P, FAKE, 4, FAKE, FAKE, None)
    status(rc, ERR_UNSUPPORTED, f"more than {limit} pages")


def test_step_graph_calls_check_their_arguments():
    """Capture needs a stream other than the null stream; a NULL graph is
    refused by launch and by the node count; freeing NULL is a no-op."""
    status(lib().pdk_graph_begin(None), ERR_ARG, "null stream")
    status(lib().pdk_graph_end(None, None), ERR_ARG, "null stream")
    status(lib().pdk_graph_launch(None, None), ERR_ARG, "null graph")
    k, o = ctypes.c_int32(), ctypes.c_int32()
    status(lib().pdk_graph_nodes(None, ctypes.byref(k), ctypes.byref(o)), ERR_ARG, "null")
    lib().pdk_graph_free(None)


def test_an_empty_batch_is_a_no_op():
    """Batch 0 (no partitions, no output rows) succeeds without touching any
    buffer: the partial launch, the flat decode and the merge each return
    PDK_OK before reading an address (all stand-ins here)."""
    p, c = pool(), dev_csr(batch=0)
    rc = lib().pdk_paged_decode_partial(ctypes.byref(p), ctypes.byref(c), FAKE, BF16, 4, 0.125, 32,
                                        FAKE, 0, FAKE, FAKE, None)
    assert rc == 0, lib().pdk_last_error()
    rc = lib().pdk_decode_flat(ctypes.byref(p), ctypes.byref(c), FAKE, BF16, 4, 0.125, 32, FAKE,
                               0, FAKE, FAKE, None, 0, None)
    assert rc == 0, lib().pdk_last_error()
    rc = lib().pdk_merge_states(FAKE, FAKE, 0, FAKE, 0, 4, 64, FAKE, FAKE, None)
    assert rc == 0, lib().pdk_last_error()


@pytest.mark.parametrize("D,Dv,v,word", [
    (96, 96, True, "no vector kernel"),          # head dim without an instance
    (128, 64, True, "head_dim_k == head_dim_v"),  # separate V of another width, few rows
])
def test_head_dims_without_a_kernel_are_unsupported(D, Dv, v, word):
    """A valid pool whose head dims no kernel is instantiated for is refused
    with PDK_ERR_UNSUPPORTED on the host, before any launch."""
    p = pdk._Pool(k=FAKE, v=FAKE if v else None, num_blocks=64, page_size=16, num_kv_heads=2,
                  head_dim_k=D, head_dim_v=Dv, dtype=BF16, k_scale=1.0, v_scale=1.0)
    c = dev_csr()
    rc = lib().pdk_paged_decode_partial(ctypes.byref(p), ctypes.byref(c), FAKE, BF16, 4, 0.125, 32,
                                        FAKE, 4, FAKE, FAKE, None)
    status(rc, ERR_UNSUPPORTED, word)
