import pytest

from layer_sliding_offloaded_amd import runtime as rt


@pytest.fixture(autouse=True)
def poisoned_buffers():
    """Every workspace, pool, activation region, slot and output buffer the
    parity tests allocate starts as NaN bytes, so a result that depends on
    memory nothing wrote fails its comparison."""
    rt.POISON = True
    yield
    rt.POISON = False
