"""Parity sweep over seeded random layer configurations (tests/random_layers.py): the forward
against the oracle on every token (routing bit for bit, y and the losses within the layer
dtype's tolerance), and the backward against the backward oracle on every other case, with
the same checks as the named layers."""
import pytest

import random_layers

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("i", range(random_layers.N_CASES))
def test_random_layer_forward(i):
    import gpu_harness
    gpu_harness.full_check(random_layers.CASES[i])


@pytest.mark.parametrize("i", range(0, random_layers.N_CASES, 2))
def test_random_layer_backward(i):
    import test_gpu_backward
    test_gpu_backward.check(random_layers.CASES[i])
