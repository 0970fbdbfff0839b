import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running case at a full workload size")


@pytest.fixture(scope="session")
def gpu():
    """The GPU binding, loaded from the in-tree library. Fails (never skips)
    when no GPU or no built library is present: a GPU test must run the HIP
    path or fail."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import transformer_attention_05_amd as attn
    attn.load()
    return attn
