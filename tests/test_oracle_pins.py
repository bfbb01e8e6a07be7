"""The oracle against its pins (closed forms, exact rationals, invariants,
hand-unrolled recurrences); see oracle_pins.py for what each pin fixes."""
import json
import os

import pytest

import oracle
from oracle import muon as oracle_muon
from tests import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle_muon)


def test_defaults_match_pages():
    """Oracle defaults are the Training Guide's dmuon.Muon defaults."""
    with open(os.path.join(HERE, "golden", "pages_hyperparameters.json")) as f:
        pages = json.load(f)
    import inspect
    sig = inspect.signature(oracle.muon_step)
    for key in ("lr", "momentum", "nesterov", "ns_steps", "weight_decay", "ns_backend"):
        assert sig.parameters[key].default == pages[key], key
    assert pages["ns_backend"] in pages["ns_backends"]
