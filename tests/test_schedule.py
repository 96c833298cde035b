"""Anchor schedule of a layer stack (host logic, no GPU)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from long_context_amd import kascade as K  # noqa: E402


def test_roles_follow_the_nearest_preceding_anchor():
    roles = K.anchor_schedule(12, [2, 6, 10])
    assert roles[:2] == [("dense", None)] * 2
    assert roles[2] == ("anchor", 2) and roles[6] == ("anchor", 6) and roles[10] == ("anchor", 10)
    assert [r for r in roles[3:6]] == [("reuse", 2)] * 3
    assert [r for r in roles[7:10]] == [("reuse", 6)] * 3
    assert roles[11] == ("reuse", 10)


def test_anchor_at_layer_zero_and_unsorted_duplicates():
    assert K.anchor_schedule(4, [3, 0, 0]) == [("anchor", 0), ("reuse", 0), ("reuse", 0), ("anchor", 3)]


def test_every_layer_an_anchor():
    assert K.anchor_schedule(3, [0, 1, 2]) == [("anchor", 0), ("anchor", 1), ("anchor", 2)]


@pytest.mark.parametrize("anchors", [[], [-1], [4]])
def test_bad_anchor_lists(anchors):
    with pytest.raises(ValueError):
        K.anchor_schedule(4, anchors)
