"""The seeded generators: determinism, shapes and the clustered structure."""
import numpy as np

import workloads


def test_same_seed_same_bytes():
    a = workloads.clustered([3, 4], 8, 2, 32, [100, 70], "f16", n_dirs=4)
    b = workloads.clustered([3, 4], 8, 2, 32, [100, 70], "f16", n_dirs=4)
    for x, y in zip(a.k + a.v + [a.q], b.k + b.v + [b.q]):
        assert x.tobytes() == y.tobytes()
    c = workloads.gaussian(9, 2, 4, 2, 16, [10, 20], "i8")
    d = workloads.gaussian(9, 2, 4, 2, 16, [10, 20], "i8")
    assert c.k[1].tobytes() == d.k[1].tobytes() and c.q.tobytes() == d.q.tobytes()


def test_shapes_and_dtypes():
    w = workloads.gaussian(1, 2, 8, 2, 16, [5, 9], "f16")
    assert w.k[0].shape == (2, 5, 16) and w.k[1].dtype == np.float16
    assert w.q.shape == (2, 8, 16) and w.q.dtype == np.float32
    w8 = workloads.gaussian(1, 1, 8, 2, 16, [5], "i8")
    assert w8.k[0].dtype == np.float32


def test_clustered_keys_share_a_direction_within_a_block():
    w = workloads.clustered([2], 4, 1, 128, [640], "f16", n_dirs=16, amp=4.0)
    k = w.k[0][0].astype(np.float32)
    means = k.reshape(10, 64, 128).mean(axis=1)
    norms = np.linalg.norm(means, axis=1)
    assert np.all(np.abs(norms - 4.0) < 0.8)       # amp * unit dir + averaged noise


def test_config4_lengths():
    lens = workloads.lengths_config4()
    assert len(lens) == 16 and all(16384 <= L <= 65536 for L in lens)
    assert lens == workloads.lengths_config4()
