"""The seeded input generator's device fill equals its host twin bit for bit."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("shape,sigma,key", [
    ((4680, 12, 128), 0.5, (2, 0, 29, 79, 3)),    # a rollout chunk tensor
    ((23400, 1536), 1.0, (3, 10, 0)),            # recache hidden states
    ((1,), 3.0, (9,)),
    ((3,), 1.0, (9, 1)),
    ((5, 1), 0.25, (9, 2)),
    ((1001,), 1.0, (2 ** 40, 7)),
])
def test_device_fill_equals_host_twin(torch_gpu, shape, sigma, key):
    dev = synth.to_bits(synth.normal_bf16_device(shape, sigma, *key))
    host = synth.normal_bf16_philox(shape, sigma, *key)
    assert dev.shape == host.shape
    bad = int((dev != host).sum())
    assert bad == 0, f"{bad} of {dev.size} values differ"
