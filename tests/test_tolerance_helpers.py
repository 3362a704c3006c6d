"""Host checks of the rounding bound the GPU parity tests grade the bf16
output with: round-to-nearest-even into bf16 (8 significant bits) errs by
at most half the bf16 spacing of the value's binade, and reaches it on ties."""
import numpy as np
import torch

from tests.gpu_util import bf16_half_ulp


def test_half_ulp_bounds_torch_rounding():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(200000, generator=g) * torch.exp2(torch.randint(-20, 20, (200000,), generator=g).float())
    r = x.to(torch.bfloat16).float()
    err = (r.double() - x.double()).abs().numpy()
    bound = bf16_half_ulp(x.double().numpy())
    assert (err <= bound).all()
    assert (err > 0.5 * bound).any()  # the bound is not loose by a factor of two


def test_half_ulp_reached_on_ties():
    for e in (-10, 0, 2, 7):
        base = 2.0 ** e
        tie = np.float32(base * (1 + 2.0 ** -8))  # halfway between 2^e and the next bf16 value
        r = float(torch.tensor([tie]).to(torch.bfloat16).float()[0])
        assert r == base  # ties go to the even neighbour
        assert abs(r - float(tie)) == float(bf16_half_ulp(np.array([tie], np.float64))[0])


def test_half_ulp_values():
    assert bf16_half_ulp(np.array([1.0]))[0] == 2.0 ** -8
    assert bf16_half_ulp(np.array([4.0, 7.99]))[0] == 2.0 ** -6
    assert bf16_half_ulp(np.array([-0.75]))[0] == 2.0 ** -9
