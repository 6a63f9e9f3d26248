import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)

import synth  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size CPU checks that take tens of seconds")


@pytest.fixture(scope="session")
def ckpt_gpt2():
    """Seed-0 GPT-2 124M checkpoint: N(0, 0.02) matrices, gamma 1, beta 0, biases 0."""
    return synth.make_checkpoint(0, synth.GPT2)


@pytest.fixture(scope="session")
def ckpt_tiny_robust():
    return synth.make_checkpoint(3, synth.TINY, robust=True)


def golden_path(name: str) -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
