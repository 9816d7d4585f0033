import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: large CPU work (full-vocabulary oracle rows)")


# ------------------------------------------------------------------ GPU side --
# Shared, session-scoped workloads for the GPU tests.  Each is generated once
# from its seed (see invariant_selected_token_amd/synth.py) and kept on the
# device; the oracle runs on sampled rows only where a full run would take
# minutes.

import numpy as np  # noqa: E402


def _torch():
    import torch
    return torch


@pytest.fixture(scope="session")
def dev():
    torch = _torch()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev_bf16(x, dev):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)


def to_dev_i32(x, dev):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)


class DevCase:
    def __init__(self, case, dev):
        self.case = case
        self.hidden = to_dev_bf16(case.hidden, dev)
        self.weight = to_dev_bf16(case.weight, dev)
        self.targets = to_dev_i32(case.targets, dev)


@pytest.fixture(scope="session")
def tiny(dev):
    from invariant_selected_token_amd import synth
    return DevCase(synth.tiny_case(), dev)


@pytest.fixture(scope="session")
def prefill(dev):
    from invariant_selected_token_amd import synth
    return DevCase(synth.prefill_case(), dev)


@pytest.fixture(scope="session")
def adversarial(dev):
    from invariant_selected_token_amd import synth
    return DevCase(synth.adversarial_case(), dev)


@pytest.fixture(scope="session")
def rollout(dev):
    from invariant_selected_token_amd import synth
    return DevCase(synth.long_rollout_case(), dev)
