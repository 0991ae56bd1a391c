"""The C-ABI library loads, exports every function include/dspark.h declares,
and rejects bad arguments on the host (no GPU work is launched by these calls)."""

import ctypes
import os

import pytest

from lossless_rejection_sampling_amd import dspark as ds


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ds.LIB_PATH):
        from lossless_rejection_sampling_amd import build
        build.build()
    return ds.lib()


def test_exports_every_declared_function(lib):
    names = ds.declared_functions()
    assert {"dspark_draft_round", "dspark_verify", "dspark_schedule", "dspark_pack_w2",
            "dspark_peak_mfma_bf16"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_signatures_match_the_header():
    # every declared function has a ctypes signature with the header's number of
    # parameters, and the binding declares nothing the header does not
    arity = ds.declared_functions(with_arity=True)
    assert len(arity) >= 20
    for n, k in arity.items():
        assert n in ds._SIG, n
        assert len(ds._SIG[n][1]) == k, (n, len(ds._SIG[n][1]), k)
    assert set(ds._SIG) <= set(arity), set(ds._SIG) - set(arity)


def test_version_and_error_strings(lib):
    assert ds.dspark_abi_version() == 5
    assert ds.error_string(0) == "ok"
    assert "argument" in ds.error_string(-1)
    assert "device" in ds.error_string(-3)


def test_last_hip_error_is_per_thread_and_starts_clear(lib):
    # a thread that has had no DSPARK_EHIP return reads 0 (no HIP call is made
    # when the name is not asked for)
    import threading

    seen = []
    t = threading.Thread(target=lambda: seen.append(lib.dspark_last_hip_error(None)))
    t.start()
    t.join()
    assert seen == [0]


def test_workspace_size_rules(lib):
    assert ds.dspark_workspace_bytes(256, 5, 151936, 256) > 0
    assert ds.dspark_workspace_bytes(0, 5, 100, 8) == 0
    assert ds.dspark_workspace_bytes(4, 0, 100, 8) == 0
    assert ds.dspark_workspace_bytes(4, 17, 100, 8) == 0
    assert ds.dspark_workspace_bytes(4, 5, 0, 8) == 0
    small = ds.dspark_workspace_bytes(4, 4, 1024, 16)
    assert small % 256 == 0 and small < ds.dspark_workspace_bytes(8, 4, 1024, 16)
    # the scheduler's own part: header + one int per candidate + one float64 per
    # cut (each part 256-byte aligned), within the full workspace
    up = lambda x: (x + 255) // 256 * 256
    assert ds.dspark_schedule_workspace_bytes(256, 5) == 256 + up(256 * 5 * 4) + up((256 * 5 + 1) * 8)
    assert ds.dspark_schedule_workspace_bytes(1024, 8) == 256 + up(1024 * 8 * 4) + up((1024 * 8 + 1) * 8)
    assert ds.dspark_schedule_workspace_bytes(1024, 9) == 0      # B * gamma > 8192
    assert ds.dspark_schedule_workspace_bytes(0, 4) == 0
    for B, g, V, r in [(1, 1, 8, 1), (7, 16, 65, 20), (256, 5, 151936, 256)]:
        assert ds.dspark_schedule_workspace_bytes(B, g) <= ds.dspark_workspace_bytes(B, g, V, r)


def test_host_argument_checks_return_einval(lib):
    P = ctypes.c_void_p
    nul = P(None)
    fake = P(256)  # never dereferenced: the checks fail before any launch
    VM, RM = ds.DSPARK_W_VOCAB_MAJOR, ds.DSPARK_W_RANK_MAJOR
    # B = 0
    rc = lib.dspark_draft_round(fake, 0, fake, fake, 0, VM, fake, fake, 1, nul, 0, 5, 100, 16,
                                fake, fake, fake, fake, nul)
    assert rc == ds.DSPARK_EINVAL
    # unknown dtype
    rc = lib.dspark_draft_round(fake, 7, fake, fake, 0, VM, fake, fake, 1, nul, 4, 5, 100, 16,
                                fake, fake, fake, fake, nul)
    assert rc == ds.DSPARK_EINVAL
    # W2 declared [r, V] (the pages' layout): the round reads only the packed layout
    rc = lib.dspark_draft_round(fake, 0, fake, fake, 0, RM, fake, fake, 1, nul, 4, 5, 100, 16,
                                fake, fake, fake, fake, nul)
    assert rc == ds.DSPARK_EINVAL
    rc = lib.dspark_draft_round(fake, 0, fake, fake, 0, 5, fake, fake, 1, nul, 4, 5, 100, 16,
                                fake, fake, fake, fake, nul)
    assert rc == ds.DSPARK_EINVAL
    rc = lib.dspark_verify(fake, fake, 0, fake, fake, 0, RM, fake, fake, fake, fake, nul, fake, 1, nul,
                           4, 5, 100, 16, fake, fake, fake, nul, nul, fake, nul)
    assert rc == ds.DSPARK_EINVAL
    rc = lib.dspark_acceptance(fake, fake, 0, fake, fake, 0, RM, fake, fake, fake, fake, 4, 5, 100, 16,
                               fake, fake, nul)
    assert rc == ds.DSPARK_EINVAL
    # missing workspace
    rc = lib.dspark_verify(fake, fake, 0, fake, fake, 0, VM, fake, fake, fake, fake, nul, fake, 1, nul,
                           4, 5, 100, 16, fake, fake, fake, nul, nul, nul, nul)
    assert rc == ds.DSPARK_EINVAL
    # misaligned workspace
    rc = lib.dspark_verify(fake, fake, 0, fake, fake, 0, VM, fake, fake, fake, fake, nul, fake, 1, nul,
                           4, 5, 100, 16, fake, fake, fake, nul, nul, P(257), nul)
    assert rc == ds.DSPARK_EINVAL
    # packing W2: pointers, sizes and dtype are checked before any launch
    assert lib.dspark_pack_w2(nul, 0, 100, 16, fake, nul) == ds.DSPARK_EINVAL
    assert lib.dspark_pack_w2(fake, 0, 100, 16, nul, nul) == ds.DSPARK_EINVAL
    assert lib.dspark_pack_w2(fake, 0, 0, 16, fake, nul) == ds.DSPARK_EINVAL
    assert lib.dspark_pack_w2(fake, 0, 100, 0, fake, nul) == ds.DSPARK_EINVAL
    assert lib.dspark_pack_w2(fake, 3, 100, 16, fake, nul) == ds.DSPARK_EINVAL
    # scheduler limits: too many candidates, too few table points
    assert lib.dspark_schedule(fake, fake, fake, 16, 1025, 8, fake, fake, nul) == ds.DSPARK_EINVAL
    assert lib.dspark_schedule(fake, fake, fake, 1, 4, 4, fake, fake, nul) == ds.DSPARK_EINVAL
    # unknown rule, NaN parameter, missing table for a rule that reads it
    ex = lib.dspark_schedule_ex
    assert ex(fake, nul, fake, fake, 16, 4, 4, 9, 0.0, fake, fake, nul) == ds.DSPARK_EINVAL
    assert ex(fake, nul, nul, nul, 0, 4, 4, 2, float("nan"), fake, fake, nul) == ds.DSPARK_EINVAL
    assert ex(fake, nul, nul, nul, 0, 4, 4, 1, 0.0, fake, fake, nul) == ds.DSPARK_EINVAL
    # draft + schedule in one call: the checks of both calls, before anything is enqueued
    dsch = lib.dspark_draft_schedule
    assert dsch(fake, 0, fake, fake, 0, VM, fake, fake, 1, nul, 4, 5, 100, 16, fake, fake, fake,
                fake, nul, fake, fake, 16, 9, 0.0, fake, fake, nul) == ds.DSPARK_EINVAL      # unknown rule
    assert dsch(fake, 0, fake, fake, 0, VM, fake, fake, 1, nul, 4, 5, 100, 16, fake, fake, fake,
                nul, nul, fake, fake, 16, 0, 0.0, fake, fake, nul) == ds.DSPARK_EINVAL       # no scores
    assert dsch(fake, 7, fake, fake, 0, VM, fake, fake, 1, nul, 4, 5, 100, 16, fake, fake, fake,
                fake, nul, fake, fake, 16, 0, 0.0, fake, fake, nul) == ds.DSPARK_EINVAL      # unknown dtype
    assert dsch(fake, 0, fake, fake, 0, RM, fake, fake, 1, nul, 4, 5, 100, 16, fake, fake, fake,
                fake, nul, fake, fake, 16, 0, 0.0, fake, fake, nul) == ds.DSPARK_EINVAL      # [r, V] W2
    assert lib.dspark_status(nul, nul) == ds.DSPARK_EINVAL
    assert lib.dspark_profile_enable(99, 1) == ds.DSPARK_EINVAL


def test_draft_path_switch(lib):
    # no device work: the switch is process state of the library
    prev = lib.dspark_set_draft_path(1)
    assert prev == 0  # per-position launches are the default
    assert lib.dspark_set_draft_path(0) == 1
    assert lib.dspark_set_draft_path(2) == -1 and lib.dspark_set_draft_path(-1) == -1
    assert lib.dspark_set_draft_path(0) == 0


def test_resident_wait_bound_setter():
    # process state too: a bound in [0, 60] s, default 0.2 s
    prev = ds.dspark_set_resident_wait_bound(0.05)
    assert prev == pytest.approx(0.2)
    assert ds.dspark_set_resident_wait_bound(prev) == pytest.approx(0.05)
    for bad in (-1e-9, 60.5, float("nan"), float("inf")):
        with pytest.raises(ds.DsparkError):
            ds.dspark_set_resident_wait_bound(bad)
    assert ds.dspark_set_resident_wait_bound(0.2) == pytest.approx(0.2)


def test_binding_reads_the_layout_from_the_shape():
    import torch
    U = torch.zeros((100, 16))
    assert ds._w_layout(U, torch.zeros((100, 16)), 100, None) == ds.DSPARK_W_VOCAB_MAJOR
    assert ds._w_layout(U, torch.zeros((16, 100)), 100, None) == ds.DSPARK_W_RANK_MAJOR
    with pytest.raises(ValueError):
        ds._w_layout(U, torch.zeros((50, 16)), 100, None)
