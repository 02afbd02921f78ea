"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import json
import os

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_reported_fp64_figures(capsys):
    """Report our fp64 figures beside the pages' (2.2e-16 and 5.7e-14,
    'Expanding Attention' abstract); the asserted bounds live in the pins."""
    g = json.load(open(os.path.join(pins.GOLDEN, "page_numbers.json")))
    rec = pins.pin_recurrent_vs_quadratic()
    add = pins.pin_chunk_additivity()
    with capsys.disabled():
        print(f"\n  recurrence vs quadratic fp64: {rec:.2e} (pages: {g['recursion_vs_truncated_kernel_fp64']['value']:.1e})"
              f"\n  chunk additivity fp64:        {add:.2e} (pages: {g['chunk_additivity_fp64']['value']:.1e})")
