import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (HIP device)")
    # The oracle is test infrastructure; build it if nothing is built yet.
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(lib):
        from oracle import build_oracle
        build_oracle.build()
    # The HIP library is built ahead of time (__graft_entry__.build());
    # build it here only if nothing is built yet.
    tide_lib = os.path.join(ROOT, "parameter_layout_collectives_amd", "libtide.so")
    if not os.path.exists(tide_lib):
        from parameter_layout_collectives_amd import build as tide_build
        tide_build.build()


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()
