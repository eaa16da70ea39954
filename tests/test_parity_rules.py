"""CPU checks of the GPU-vs-oracle comparison helpers themselves."""
import numpy as np
import pytest
import torch

from parity import bf16_ulp, ulp_check


def test_bf16_ulp_is_the_spacing_of_bf16_values():
    xs = torch.tensor([1.0, 0.75, 3.0, 1e-3, -2.5, 6e-38], dtype=torch.float32)
    b = xs.to(torch.bfloat16)
    up = (b.view(torch.int16) + 1).view(torch.bfloat16)  # next bf16 away from zero
    spacing = (up.float() - b.float()).abs().double().numpy()
    assert np.array_equal(bf16_ulp(b.float().numpy()), spacing)
    assert bf16_ulp(1.0) == 2.0 ** -7 and bf16_ulp(0.75) == 2.0 ** -8


def test_ulp_check_accepts_one_step_and_rejects_two():
    old = np.array([[0.5, -0.25, 0.125]])
    ora = np.array([[0.5078125, -0.25, 0.125]])          # values in [0.5, 1) are 2^-8 apart in bf16
    one = ora + np.array([[2.0 ** -8, 0.0, 0.0]])        # one bf16 step above
    two = ora + np.array([[2.0 ** -7, 0.0, 0.0]])        # two steps
    ulp_check(one, ora, old, "one step", arith=0.0)
    with pytest.raises(AssertionError):
        ulp_check(two, ora, old, "two steps", arith=0.0)
