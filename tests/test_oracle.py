"""The CPU oracle against its pins (brute force, library routine, invariants,
closed forms, hand-worked examples, pair counts)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib_path():
    oracle.lib()
    return oracle._LIB


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib_path):
    fails = pin(lib_path)
    assert not fails, "\n".join(fails[:20])


def test_union_totals_of_svg_geometry(lib_path):
    """Key unions of 64-row query blocks on the SVG head-routing geometry
    (13 frames of 30x52, anchor frame 0, radius 2) equal the totals computed by
    hand from that geometry: 967,200 for a spatial head (frame-major),
    1,092,806 for a temporal head in frame-major order and 192,088 for a
    temporal head in temporal-major order."""
    import workloads as wl
    a, b = wl.svg("A"), wl.svg("B")
    assert oracle.union_total(a, 0, 0) == 967200
    assert oracle.union_total(a, 0, 12) == 1092806
    assert oracle.union_total(b, 0, 12) == 192088
    assert oracle.union_total(b, 0, 0) == 967200
