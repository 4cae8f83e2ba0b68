"""fwd_gemm_noalloc, the projection entry point for callers that cannot allocate: the
same result as fwd_gemm bit for bit (same kernels, same split of `in`, partials in the
library's static device scratch instead of memory allocated for the call), checked on
two calls in a row, the second smaller (the scratch keeps the first call's partials),
plus the error for a product whose partials exceed the scratch and a check that a call
leaves the device's free memory unchanged."""
import sys

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32
from synth import workloads as wl
from tests.gpu_util import err_over_scale, to_device

pytestmark = pytest.mark.gpu

# Both products are split over `in` (few output tiles, `in` >= 8192): 2 ranges each,
# 0.79M and 0.13M partial floats of the 4M the scratch holds.
SHAPES = [(256, 8192, 1536), (128, 8192, 512)]


@pytest.fixture(scope="module")
def fwd():
    import torch
    from decoder_only_transformer_bf16_amd import fwd as F
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    torch.cuda.set_device(0)
    assert F.available(), "libfwd.so sees no gfx950 device"
    return F


def test_noalloc_gemm_equals_fwd_gemm_on_two_calls(fwd):
    import torch
    for P, K, N in SHAPES:
        print(f"fwd_gemm_noalloc [{P},{K},{N}]", flush=True)
        sys.stdout.flush()
        Xh, Wh = wl.draw_gemm(P, K, N)
        X, W = to_device(Xh), to_device(Wh)
        want = fwd.gemm(X, W)
        got = torch.full((P, N), float("nan"), dtype=torch.float32, device="cuda")
        fwd.gemm(X, W, got, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(got, want), "fwd_gemm_noalloc must equal fwd_gemm bit for bit"
        ref = oracle.gemm(bf16_bits_to_f32(Xh), bf16_bits_to_f32(Wh))
        err = err_over_scale(got.cpu().numpy(), ref)
        assert err < 1e-5, err  # bf16-exact inputs: only the fp32 summation order differs


def test_noalloc_gemm_allocates_nothing(fwd):
    import torch
    P, K, N = SHAPES[0]
    Xh, Wh = wl.draw_gemm(P, K, N)
    X, W = to_device(Xh), to_device(Wh)
    Y = torch.empty((P, N), dtype=torch.float32, device="cuda")
    fwd.gemm(X, W, Y, noalloc=True)  # first use on this device: symbol lookup, kernel loading
    torch.cuda.synchronize()
    before = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        fwd.gemm(X, W, Y, noalloc=True)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == before


def test_noalloc_gemm_rejects_partials_beyond_the_scratch(fwd):
    import torch
    # 240 output tiles of 128 x 128 over `in` 8192: 2 ranges of 1024 x 3840 partials = 7.9M floats
    P, K, N = 1024, 8192, 3840
    X = torch.zeros((P, K), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((P, N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(fwd.FwdError) as e:
        fwd.gemm(X, W, Y, noalloc=True)
    assert e.value.code == fwd.FWD_E_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all()), "a rejected call computes nothing"
