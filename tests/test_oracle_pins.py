"""The FP64 oracle against hand-worked values, closed forms, invariants,
independent definitions and brute force (CPU only)."""

import pytest

import pins


@pytest.mark.parametrize("name", sorted(pins.ALL_PINS))
def test_pin(name):
    pins.ALL_PINS[name]()


def test_bruteforce_tiny_all_parent_vectors():
    pins.pin_bruteforce_tiny()
