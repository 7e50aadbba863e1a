"""The seeded input generator: the C fast path against its numpy restatement."""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("mode", ["uniform", "int"])
def test_c_generator_matches_numpy_definition(mode):
    rows = np.array([0, 1, 2, 63, 64, 1000, 131071, 262180, 2**40 + 3], dtype=np.int64)
    got = synth.rows_of(rows, 97, seed=4001, tensor=synth.TENSOR_A, mode=mode)
    ref = synth.reference_rows(rows, 97, seed=4001, tensor=synth.TENSOR_A, mode=mode)
    assert np.array_equal(got, ref)


def test_layouts_hold_the_same_logical_matrix():
    a = synth.matrix(37, 53, seed=7, tensor=1, order="row")
    t = synth.matrix(37, 53, seed=7, tensor=1, order="col")
    assert t.shape == (53, 37)
    assert np.array_equal(a, t.T)
    sub = synth.rows_of([5, 36, 0], 53, seed=7, tensor=1)
    assert np.array_equal(sub, a[[5, 36, 0]])


def test_value_ranges():
    u = synth.matrix(300, 300, seed=1, tensor=0).view(np.float16).astype(np.float64)
    assert np.all(np.abs(u) <= 1.0) and np.all(u != 0.0)
    assert abs(u.mean()) < 0.01 and abs(u.std() - 1 / np.sqrt(3)) < 0.01
    i = synth.matrix(300, 300, seed=1, tensor=0, mode="int").view(np.float16).astype(np.float64)
    assert set(np.unique(i).tolist()) == set(range(-4, 5))


def test_seed_and_tensor_change_the_stream():
    a = synth.matrix(16, 16, seed=1, tensor=0)
    assert not np.array_equal(a, synth.matrix(16, 16, seed=2, tensor=0))
    assert not np.array_equal(a, synth.matrix(16, 16, seed=1, tensor=1))
    assert np.array_equal(a, synth.matrix(16, 16, seed=1, tensor=0, nthreads=3))


def test_group_sizes_partition():
    for G, total, seed in ((1, 5, 0), (8, 1000, 3), (32, 131072, 11), (7, 3, 2)):
        s = synth.group_sizes(G, total, seed)
        assert s.shape == (G,) and s.min() >= 0 and int(s.sum()) == total
        assert np.array_equal(s, synth.group_sizes(G, total, seed))   # seeded


@pytest.mark.parametrize("mode", ["uniform", "int"])
def test_bf16_format_matches_the_numpy_torch_restatement(mode):
    rows = np.array([0, 1, 7, 1000, 123456])
    got = synth.rows_of(rows, 300, 77, 3, mode, fmt="bf16")
    assert np.array_equal(got, synth.reference_rows(rows, 300, 77, 3, mode, fmt="bf16"))
    # the same logical values as the binary16 matrix, rounded to bfloat16
    f16 = synth.rows_of(rows, 300, 77, 3, mode).view(np.float16).astype(np.float64)
    bf = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(bf - f16) <= np.abs(f16) * 2.0 ** -8 + 2.0 ** -24)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("mode", ["uniform", "int"])
def test_f8_formats_match_the_torch_restatement(fmt, mode):
    rows = np.array([0, 1, 7, 1000, 123456])
    got = synth.rows_of(rows, 300, 78, 3, mode, fmt=fmt)
    assert got.dtype == np.uint8
    assert np.array_equal(got, synth.reference_rows(rows, 300, 78, 3, mode, fmt=fmt))
    a = synth.matrix(50, 20, 78, 3, mode, fmt=fmt)
    at = synth.matrix(50, 20, 78, 3, mode, fmt=fmt, order="col")
    assert np.array_equal(a, at.T)
