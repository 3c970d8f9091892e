"""The allocation-free entry point ozaki2_dgemm_noalloc, through the C ABI, against
ozaki2_dgemm on the same inputs: the same kernels run on a workspace held in a fixed
device array, so C must be bit-identical.  Two calls in a row share that array, the
second on a smaller product (what the first left behind must not leak into it), and
neither may allocate device memory."""
import numpy as np
import pytest

from fp64_gemm_emulation_amd.workloads import generate
from tests.gpu_helpers import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oz():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from fp64_gemm_emulation_amd import binding
    return binding


def _noalloc(oz, Ad, Bd, C, s, mode):
    import torch
    p, q = Ad.shape
    r = Bd.shape[1]
    return oz.ozaki2_dgemm_noalloc(p, q, r, Ad.data_ptr(), Ad.stride(1), Bd.data_ptr(), Bd.stride(1),
                                   C.data_ptr(), C.stride(1), s, oz.MODES[mode],
                                   torch.cuda.current_stream().cuda_stream)


CASES = [  # (p, q, r, s, mode, phi): the second smaller than the first
    (1500, 1200, 1400, 14, "fast", 1.0),
    (600, 500, 400, 8, "accu", 2.0),
]


def test_noalloc_matches_dgemm_on_two_calls(oz):
    import torch
    inputs = []
    for k, (p, q, r, s, mode, phi) in enumerate(CASES):
        A = generate(p, q, phi, 700 + k)
        B = generate(q, r, phi, 800 + k)
        Ad, Bd = to_device(A), to_device(B)
        want = oz.dgemm(Ad, Bd, s, mode)                   # the existing entry point
        C = oz.empty_colmajor(p, r)
        C.fill_(float("nan"))
        inputs.append((Ad, Bd, C, want, s, mode))
    torch.cuda.synchronize()
    # module loaded and the scratch address resolved by a first call; then no call may
    # take device memory (the library-owned workspace is released first, and nothing of
    # torch runs between the two readings of free memory)
    assert _noalloc(oz, *inputs[1][:3], inputs[1][4], inputs[1][5]) == oz.OZ2_OK
    torch.cuda.synchronize()
    assert oz.ozaki2_release() == oz.OZ2_OK
    for Ad, Bd, C, want, s, mode in inputs:
        C.fill_(float("nan"))
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for k, (Ad, Bd, C, want, s, mode) in enumerate(inputs):
        assert _noalloc(oz, Ad, Bd, C, s, mode) == oz.OZ2_OK
        torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 >= free0 - (1 << 20), f"device memory taken: {(free0 - free1) >> 20} MiB"
    for k, (Ad, Bd, C, want, s, mode) in enumerate(inputs):
        p, q = Ad.shape
        log(f"[noalloc] call {k}: p,q,r={p},{q},{Bd.shape[1]} s={s} mode={mode} "
            f"workspace {oz.ozaki2_workspace_size(p, q, Bd.shape[1], s, oz.MODES[mode]) >> 20} MiB")
        assert torch.equal(C, want), f"call {k}: C differs from ozaki2_dgemm"
    # the smaller call again after the larger one, and an oversized call that is refused
    # before anything is launched (C untouched)
    Ad, Bd, C, want, s, mode = inputs[0]
    C.fill_(float("nan"))
    assert _noalloc(oz, Ad, Bd, C, s, mode) == oz.OZ2_OK
    Ad, Bd, C, want, s, mode = inputs[1]
    C.fill_(float("nan"))
    assert _noalloc(oz, Ad, Bd, C, s, mode) == oz.OZ2_OK
    torch.cuda.synchronize()
    assert torch.equal(C, want)
    n = 4096
    big = torch.zeros((n, n), dtype=torch.float64, device="cuda")
    out = torch.full((n, n), 3.0, dtype=torch.float64, device="cuda")
    assert oz.ozaki2_dgemm_noalloc(n, n, n, big.data_ptr(), n, big.data_ptr(), n, out.data_ptr(), n, 14, 0,
                                   torch.cuda.current_stream().cuda_stream) == oz.OZ2_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    log("[noalloc] ok")
