import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    from oracle import oracle
    return oracle


@pytest.fixture(scope="session")
def ling_seed1():
    """The seed-1 Ling-shape layer (numpy, plain layout), generated once per
    session and shared by every GPU test module that needs it."""
    from w4a16_grouped_quantized_amd import synth
    print("generating Ling-shape layer (seed 1)", flush=True)
    return synth.make_layer(synth.LING, 1, threads=16)


@pytest.fixture(scope="session")
def ling_seed23():
    """Seeds 2 and 3 of the Ling-shape layer (the second and third layers of
    the stacked-layer tests)."""
    from w4a16_grouped_quantized_amd import synth
    print("generating Ling-shape layers (seeds 2, 3)", flush=True)
    return [synth.make_layer(synth.LING, s, threads=16) for s in (2, 3)]
