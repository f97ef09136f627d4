import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _reload_tuning_after_test():
    """Tests that force a kernel through a MOE_* variable set it with
    monkeypatch and make the library re-read it; once monkeypatch has
    restored the environment, the library reads it again here (through the
    binding, which also drops the workspace sizes it cached under the
    test's setting)."""
    yield
    from top_routing_dispatch_amd import binding
    if binding._lib is not None:
        binding.moe_reload_tuning()
