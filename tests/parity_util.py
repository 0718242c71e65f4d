"""Helpers shared by the GPU parity tests.

whole_rel_err computes the parity metric max |x - x_ref| / max |x_ref| over
EVERY element of a full-size output, copying the device tensor to the host
one slice at a time, so that a 1M-token output never needs a second full
host copy; a non-finite element fails it outright.  OracleCache keeps one
full-size oracle result between the tests (and the prefill paths) that
compare against it.
"""
import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def whole_rel_err(got, ref, dim=0, name="output"):
    """max |got - ref| / max |ref| over the whole tensor.  got: a torch tensor
    (any device), ref: a numpy array of the same shape.  Slices along `dim`
    are compared one at a time."""
    assert tuple(got.shape) == tuple(ref.shape), (tuple(got.shape), ref.shape)
    num = den = 0.0
    for i in range(ref.shape[dim]):
        a = host(got.select(dim, i)).astype(np.float64)
        r = np.take(ref, i, axis=dim)
        if not np.isfinite(a).all():
            raise AssertionError("%s: non-finite elements in slice %d of dim %d" % (name, i, dim))
        if a.size:
            num = max(num, float(np.abs(a - r).max()))
            den = max(den, float(np.abs(r).max()))
    return num / (den if den > 0 else 1.0)


class OracleCache:
    """One cached oracle result (the full-size references are GBs; a new key
    drops the previous one)."""

    def __init__(self):
        self.key = None
        self.val = None

    def clear(self):
        self.key, self.val = None, None

    def get(self, key, compute):
        if self.key != key:
            self.key, self.val = None, None
            self.val = compute()
            self.key = key
        return self.val


ORACLE_CACHE = OracleCache()
