"""Shared fixtures.  Tests marked ``gpu`` need an MI355X; every other test runs on
the CPU (oracle pins, host-side logic, C-ABI load/export checks)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    import oracle as orc
    if not os.path.exists(orc.LIB):
        orc.build()
    return orc.Oracle(orc.LIB)


@pytest.fixture(scope="session")
def planted(tmp_path_factory):
    """Factory for oracle builds that carry one deliberate mistake (negative
    controls for the statistical tests)."""
    import oracle as orc
    cache = {}

    def get(plant: int):
        if plant not in cache:
            path = str(tmp_path_factory.mktemp(f"plant{plant}") / f"liboracle_plant{plant}.so")
            orc.build(path, plant=plant)
            cache[plant] = orc.Oracle(path)
            assert cache[plant].plant == plant
        return cache[plant]

    return get
