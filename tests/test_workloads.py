"""The seeded input generator: determinism, chunking, shapes and recipe."""
import numpy as np

import workloads


def test_blocks_independent_of_threads_and_prefix(monkeypatch):
    w = workloads.WORKLOADS["rms_17x257"]
    monkeypatch.setattr(workloads, "_CHUNK_ELEMS", 257 * 3)   # 3-row blocks
    a = workloads.generate(w)
    monkeypatch.setattr(workloads, "_THREADS", 1)
    b = workloads.generate(w)
    c = workloads.generate(w, N=7)
    for k in a:
        assert (a[k].view(np.uint16) == b[k].view(np.uint16)).all(), k
        if a[k].ndim == 2:
            assert (a[k][:7].view(np.uint16) == c[k].view(np.uint16)).all(), k


def test_recipe_matches_plain_numpy():
    w = workloads.WORKLOADS["ln_128x1024"]
    got = workloads.generate(w)
    X = (0.5 + np.random.default_rng([0, 0, 0]).standard_normal((128, 1024))).astype(np.float16)
    g = (1 + 0.1 * np.random.default_rng([0, 1]).standard_normal(1024)).astype(np.float16)
    b = (0.1 * np.random.default_rng([0, 2]).standard_normal(1024)).astype(np.float16)
    dY = np.random.default_rng([0, 3, 0]).standard_normal((128, 1024)).astype(np.float16)
    for k, v in (("X", X), ("gamma", g), ("beta", b), ("dY", dY)):
        assert (got[k].view(np.uint16) == v.view(np.uint16)).all(), k


def test_outlier_channels():
    w = workloads.WORKLOADS["rms_16384x4096"]
    ch = w.outlier_channels()
    assert len(ch) == 41 and len(np.unique(ch)) == 41 and (np.diff(ch) > 0).all()
    d = workloads.generate(w, N=256)
    a = np.abs(d["X"].astype(np.float64))
    ratio = a[:, ch].mean() / np.delete(a, ch, axis=1).mean()
    assert 15 < ratio < 25


def test_shapes_and_dtypes():
    for name, w in workloads.WORKLOADS.items():
        d = workloads.generate(w, N=3)
        for spec in w.tensors:
            a = d[spec.name]
            assert a.dtype == np.float16 and a.flags.c_contiguous
            want = ((w.D, w.Nout) if spec.matrix else (w.B, w.D) if spec.per_sample
                    else (w.channels,) if spec.per_channel
                    else (3, w.D) if spec.per_row else (w.D,))
            assert a.shape == want, (name, spec.name)


def test_sample_rows():
    s = workloads.sample_rows(1000, 50)
    assert s[0] == 0 and s[-1] == 999 and len(s) == 50 and (np.diff(s) > 0).all()
    assert (workloads.sample_rows(10, 50) == np.arange(10)).all()
