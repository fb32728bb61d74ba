"""The literal parameter-block offsets of the synthetic workloads agree with
the oracle's compute_offsets (itself pinned to the page's worked example), and
each bias block follows its weight block."""

import pytest

import oracle
import workloads


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5, 6])
def test_layer_offsets_are_the_compute_offsets_of_the_blocks(key):
    wl = workloads.make(key)
    flat = []
    for L in wl.layers:
        flat.append(L.w_offset)
        if L.bias is not None:
            flat.append(L.b_offset)
        assert L.b_offset == L.w_offset + L.out_features * L.in_features
    assert oracle.compute_offsets(wl.shapes) == flat


def test_three_layer_offsets_literal():
    assert [o for pair in workloads.LAYER_OFFSETS[4] for o in pair] == [0, 200704, 200960, 266496, 266752, 269312]
