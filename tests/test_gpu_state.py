"""la_state_init on the GPU: every element of S, z and the mLSTM stabiliser
becomes exactly 0, for sizes that are and are not multiples of four and a
stabiliser that starts off a 16-byte boundary (the kernel stores 16 bytes at
a time over the aligned body and single floats at both ends)."""
import ctypes

import pytest
import torch

import fixed_state_sequence_amd as la
from conftest import gpu_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,dp,dv", [(1, 8, 128, 128), (3, 5, 6, 4), (2, 3, 7, 4), (1, 1, 1, 4)])
def test_state_init_zeroes_every_element(B, H, dp, dv):
    dev = gpu_device()
    nan = float("nan")
    S = torch.full((B, H, dp, dv), nan, device=dev)
    z = torch.full((B, H, dp), nan, device=dev)
    mbuf = torch.full((B * H + 2,), nan, device=dev)
    m = mbuf[1:1 + B * H]                       # 4 bytes past a 16-byte boundary
    g = torch.empty(1, device=dev)
    desc = la.make_desc(B, H, 0, dp, dv, la._lib.LA_F32, phi="identity", igate=g, fgate=g, stab=m)
    la._lib.check(la._lib.lib().la_state_init(ctypes.byref(desc), la._ptr(S), la._ptr(z),
                                              la._stream(dev)))
    torch.cuda.synchronize()
    assert (S == 0).all() and (z == 0).all() and (m == 0).all()
    assert mbuf[0].isnan() and mbuf[-1].isnan()   # nothing outside the stabiliser
