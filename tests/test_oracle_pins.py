"""The oracle against its pins (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_tree_bruteforce_seven_nodes():
    """All 720 topologically ordered 7-node trees x 64 match patterns."""
    pins.check_accept_tree_bruteforce(max_nodes=7)
