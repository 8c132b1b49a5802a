"""The C++ chunk-metadata builder against the oracle's brute-force labeler (bit-exact),
the examples from the pages, and its error paths.  CPU only."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import chunk_metadata
from selective_state_space_mamba2_amd import api
from selective_state_space_mamba2_amd._abi import (SSD_ERR_BAD_METADATA, SSD_ERR_BAD_SHAPE,
                                                   SSD_ERR_CAPACITY, SSD_ERR_NULL_POINTER,
                                                   SSDError, lib)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", ["warmup_single_chunk", "partial_first_chunks"])
def test_examples(name):
    f = json.load(open(os.path.join(GOLDEN, "metadata_examples.json")))[name]
    cu, sidx, last = api.ssd_build_chunk_metadata(f["cu_seqlens"], f["num_computed"],
                                                  f["chunk_size"])
    assert cu.tolist() == f["cu_chunk_seqlens"]
    assert sidx.tolist() == f["seq_idx"]
    assert last.tolist() == f["last_chunk_indices"]


def _compare(lengths, nc, cs):
    cu_seq = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    got = api.ssd_build_chunk_metadata(cu_seq, nc, cs)
    ref = chunk_metadata(cu_seq, nc, cs)
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)
    assert api.ssd_chunk_metadata_count(cu_seq, nc, cs) == len(ref[1])


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 300), st.lists(st.tuples(st.integers(1, 700), st.integers(0, 2000)),
                                     min_size=1, max_size=12))
def test_random_batches_match_the_labeler(cs, seqs):
    _compare([a for a, _ in seqs], [b for _, b in seqs], cs)


@pytest.mark.parametrize("cs", [64, 256, 2048])
def test_workload_structures(cs):
    rng = np.random.default_rng(cs)
    lengths = rng.integers(512, 8193, size=16)
    nc = rng.integers(0, 4097, size=16)
    _compare(lengths, nc, cs)
    _compare(lengths, None, cs)


def test_edge_cases():
    _compare([1], [0], 1)               # chunk size 1: a chunk per token
    _compare([1, 1, 1], [5, 0, 7], 4)   # single-token sequences, unaligned
    _compare([255, 256, 257], [1, 0, 255], 256)
    _compare([3], [254], 256)           # the open chunk is longer than the new tokens
    cu, sidx, last = api.ssd_build_chunk_metadata([0], None, 256)   # empty batch
    assert cu.tolist() == [0] and len(sidx) == 0 and len(last) == 0


def test_errors():
    with pytest.raises(SSDError) as e:
        api.ssd_build_chunk_metadata([0, 4, 4], None, 4)      # an empty sequence
    assert e.value.status == SSD_ERR_BAD_METADATA
    with pytest.raises(SSDError) as e:
        api.ssd_build_chunk_metadata([1, 4], None, 4)         # cu_seqlens[0] != 0
    assert e.value.status == SSD_ERR_BAD_METADATA
    with pytest.raises(SSDError) as e:
        api.ssd_build_chunk_metadata([0, 4], [-1], 4)
    assert e.value.status == SSD_ERR_BAD_METADATA
    with pytest.raises(SSDError) as e:
        api.ssd_build_chunk_metadata([0, 4], None, 0)
    assert e.value.status == SSD_ERR_BAD_SHAPE
    with pytest.raises(SSDError) as e:                        # absolute positions past int32
        api.ssd_build_chunk_metadata([0, 20], [2**31 - 10], 64)
    assert e.value.status == SSD_ERR_BAD_METADATA
    assert len(api.ssd_build_chunk_metadata([0, 10], [2**31 - 11], 64)[1]) == 1
    # capacity too small: the status says so and reports the count
    import ctypes
    cu = np.array([0, 10], dtype=np.int32)
    out = ctypes.c_int32(-1)
    buf = np.zeros(8, dtype=np.int32)
    st_ = lib().ssd_build_chunk_metadata(1, cu.ctypes.data, None, 4, 2, buf.ctypes.data,
                                         buf.ctypes.data, buf.ctypes.data, ctypes.byref(out))
    assert st_ == SSD_ERR_CAPACITY and out.value == 3
    assert lib().ssd_build_chunk_metadata(1, cu.ctypes.data, None, 4, 3, None, None, None,
                                          ctypes.byref(out)) == SSD_ERR_NULL_POINTER
