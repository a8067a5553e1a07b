"""The allocation-free activation entry point (rq_rotate_quant_noalloc)
against rq_rotate_quant with a caller workspace, through the C ABI: codes,
scales and top-r coefficients bit for bit, on two calls in a row (the second
smaller, so stale scratch contents from the first call must not leak in),
for the dense path that stages in the library's scratch and for RPBH."""
import sys

import numpy as np
import pytest

from rotated_w4a4_quantized_amd import datagen, rq
from tests import _layer as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_both(w, inp):
    L = H.GpuLayer(w, inp)
    L.rotate_quant()
    codes = torch.full_like(L.codes, 0x5A)
    scale = torch.full_like(L.scale, -3.0)
    top = None if L.top is None else torch.full_like(L.top, 7)
    rq.rotate_quant_noalloc(L.drot, L.q, L.X, codes, scale, top)
    torch.cuda.synchronize()
    assert torch.equal(codes, L.codes), "codes differ"
    assert torch.equal(scale.view(torch.int32), L.scale.view(torch.int32)), "scales differ"
    if top is not None:
        assert torch.equal(top, L.top), "top-r coefficients differ"
    return L


@pytest.mark.parametrize("name,first,second", [
    ("pixart", dict(T=300, N=64), dict(T=77, N=64)),
    ("pixart", dict(), dict(T=1000, N=64)),           # full 8192 x 1152 first
    ("tiny", dict(T=300, N=64), dict(T=45, N=64)),    # RPBH: no scratch
])
def test_noalloc_matches_workspace_entry(name, first, second):
    for i, shape in enumerate((first, second)):
        w = datagen.WORKLOADS[name].with_shape(**shape) if shape else datagen.WORKLOADS[name]
        say(f"[noalloc] call {i}: {w}")
        inp = datagen.make_inputs(w, seed_offset=17 * i)
        run_both(w, inp)


def test_noalloc_rejects_oversize_dense():
    w = datagen.WORKLOADS["pixart"].with_shape(T=16, N=64)
    inp = datagen.make_inputs(w)
    L = H.GpuLayer(w, inp)
    Tbig = (64 << 20) // (4 * w.K) + 1
    X = torch.zeros((Tbig, w.K), dtype=torch.int16, device="cuda")
    codes = torch.empty((Tbig, w.Kq // 2), dtype=torch.uint8, device="cuda")
    scale = torch.empty((Tbig,), dtype=torch.float32, device="cuda")
    top = torch.empty((Tbig, w.r), dtype=torch.int16, device="cuda")
    with pytest.raises(rq.RQError) as e:
        rq.rotate_quant_noalloc(L.drot, L.q, X, codes, scale, top)
    assert e.value.status == -2 and "limit" in str(e.value)
