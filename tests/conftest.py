import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library (built here on first use if it is missing)."""
    from decode_attention_kv_04_amd import binding
    from decode_attention_kv_04_amd import build as _build
    if not os.path.exists(binding.library_path()):
        _build.build_library()
    return binding.load()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


# The two full-size batches with their oracle outputs, built once per session
# (the oracle over a whole batch takes seconds of host time; the workloads
# themselves are deterministic for their seeds). Tests must not modify them.
@pytest.fixture(scope="session")
def long_batch(gpu):
    return _full_size("long_batch", gpu)


@pytest.fixture(scope="session")
def mixed_window(gpu):
    return _full_size("mixed_window", gpu)


def _full_size(name, gpu):
    import oracle
    from decode_attention_kv_04_amd import workloads as wl
    print(f"[fixture] {name}: workload and oracle", file=sys.stderr, flush=True)
    w = wl.make_workload(wl.NAMED[name], gpu)
    a = wl.to_numpy_inputs(w, attended_only=True)
    ref = oracle.decode_attention(a["q"], a["k_pool"], a["v_pool"], a["page_table"], a["seq_lens"],
                                  a["page_size"], a["scale"], a["window"])
    return w, ref
