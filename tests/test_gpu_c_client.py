"""GPU: a plain C client of the ABI (tests/c_client.c: hipMalloc'd buffers,
the owner map built on the device, one bucket flush (searched, and again
from a plan made on the host) and one reduce-scatter, no Python or torch in
the client), bit-exact against the oracle."""
import ctypes
import os
import random

import numpy as np
import pytest

import oracle
import synth
from gradient_reduction_amd import dc
from synth import workloads as wl

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def client():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dc.lib()  # loads torch's HIP runtime first: the client resolves to the same one
    path = os.path.join(HERE, "libc_client.so")
    assert os.path.exists(path), "build first: python -c 'import __graft_entry__ as g; g.build()'"
    L = ctypes.CDLL(path)
    f = L.c_client_run
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.argtypes = [i32, i32, vp, i64, i32, vp, i32, i32, vp, vp, i64, vp, vp]
    f.restype = ctypes.c_int
    return f


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


CASES = [(8, wl.DT_BF16, 1, 1), (8, wl.DT_BF16, 0, 1), (4, wl.DT_F32, 1, 0),
         (16, wl.DT_F32, 1, 1), (3, wl.DT_BF16, 1, 1), (1, wl.DT_F32, 0, 0)]


@pytest.mark.parametrize("W,dtype,owner,pre", CASES, ids=lambda v: str(v))
def test_c_client_matches_oracle(client, W, dtype, owner, pre):
    rng = random.Random(W * 100 + dtype * 10 + owner)
    numel = np.array([rng.choice([1, 7, 64, 999, 4096, 30_000, 120_000]) for _ in range(40)],
                     np.int64)
    total = int(numel.sum())
    ld = wl.round_up(total, 64)
    scale = wl.sigma_scale(1e-2)
    print("c client", W, dtype, owner, pre, total, flush=True)
    hin = synth.fill_slab(dtype, 70 + W, 0, scale, W, ld, total)
    ld_rs = (total // W) // 64 * 64
    P = len(numel)
    owner_out = np.full(P, -7, np.int32)
    flush_out = np.zeros_like(hin)
    planned_out = np.zeros_like(hin)
    rs_out = np.zeros((W, max(ld_rs, 64)), hin.dtype)
    rc = client(W, dtype, _ptr(hin), ld, P, _ptr(numel), owner, pre, _ptr(owner_out),
                _ptr(flush_out), ld_rs, _ptr(rs_out) if ld_rs else None, _ptr(planned_out))
    assert rc == 0, rc

    flat, ps, off, pids = oracle.partition_ids(list(numel), [0, P], [W])
    want_owner, _ = oracle.owner_map(off, pids, [0, P], [1])
    assert np.array_equal(owner_out, want_owner)
    want = hin.copy()   # the client's output slab starts as a copy of the input
    offs = np.concatenate([[0], np.cumsum(numel)[:-1]])
    oracle.flush(W, dtype, hin, want, 0, list(offs), list(numel), list(range(P)), [0] * P,
                 want_owner if owner else None, [W], [1], pre)
    bits = np.uint16 if dtype == wl.DT_BF16 else np.uint32
    assert np.array_equal(flush_out.view(bits), want.view(bits))
    assert np.array_equal(planned_out.view(bits), want.view(bits))
    if ld_rs:
        want_rs = np.zeros_like(rs_out)
        oracle.reduce_scatter(W, dtype, hin, want_rs, W * ld_rs, pre)
        assert np.array_equal(rs_out.view(bits), want_rs.view(bits))


def test_c_client_reports_library_errors(client):
    """An argument the library rejects comes back to the C caller as its
    DC_ERR_* code (here a communicator size that does not match W)."""
    numel = np.array([100, 200], np.int64)
    hin = np.zeros((4, 320), np.float32)
    out = np.zeros_like(hin)
    own = np.zeros(2, np.int32)
    assert client(0, wl.DT_F32, _ptr(hin), 320, 2, _ptr(numel), 1, 0, _ptr(own), _ptr(out), 0,
                  None, None) == dc.DC_ERR_ARG
    assert client(4, 7, _ptr(hin), 320, 2, _ptr(numel), 1, 0, _ptr(own), _ptr(out), 0,
                  None, _ptr(out)) == dc.DC_ERR_DTYPE
