"""Pins of the oracle's window / flush placement (CPU)."""

import pytest

from oracle import placement


def simulate(n, s_sink, s_keep, s_flush):
    """Literal step-by-step reading of the flush rule: append one token at a
    time; after each append, while the un-quantized tail beyond the sink is at
    least S_keep + S_flush long, quantize the oldest S_flush tokens of it."""
    sq = s_sink
    history = []
    for length in range(1, n + 1):
        while length - sq >= s_keep + s_flush and sq >= s_sink:
            sq += s_flush
        history.append(sq)
    return history


@pytest.mark.parametrize("s_sink,s_keep,s_flush", [
    (4, 128, 16), (64, 256, 16), (64, 256, 256), (0, 0, 1), (0, 5, 1), (3, 7, 5),
    (64, 256, 8), (1, 1, 1), (16, 0, 16)])
def test_closed_form_matches_simulator(s_sink, s_keep, s_flush):
    hist = simulate(2000, s_sink, s_keep, s_flush)
    for length, sq in enumerate(hist, start=1):
        assert placement.s_quant(length, s_sink, s_keep, s_flush) == sq


def test_flush_one_is_single_token_demotion():
    # S_flush = 1: each new token beyond the windows demotes exactly the oldest one
    for length in range(1, 600):
        sq = placement.s_quant(length, 4, 100, 1)
        assert sq == max(4, length - 100)


@pytest.mark.parametrize("s_sink,s_keep,s_flush", [(4, 128, 16), (64, 256, 256), (3, 7, 5)])
def test_segments_partition_and_ring_slots_unique(s_sink, s_keep, s_flush):
    cap = placement.ring_capacity(s_keep, s_flush)
    assert cap % 16 == 0 and cap >= s_keep + s_flush
    for length in range(1, 1200, 7):
        sink, int2, recent = placement.segments(length, s_sink, s_keep, s_flush)
        covered = list(range(*sink)) + list(range(*int2)) + list(range(*recent))
        assert covered == list(range(length))
        if length >= s_sink + s_keep:
            assert s_keep <= recent[1] - recent[0] <= s_keep + s_flush - 1
        slots = [placement.where(p, length, s_sink, s_keep, s_flush) for p in range(*recent)]
        assert len(set(slots)) == len(slots)
        assert (int2[1] - int2[0]) % s_flush == 0


def test_where_pages():
    # position -> (logical page, slot) of the INT2 region starts right after the sink
    assert placement.where(64, 2000, 64, 256, 16) == ("int2", 0, 0)
    assert placement.where(64 + 16 * 7 + 3, 2000, 64, 256, 16) == ("int2", 7, 3)
    assert placement.where(3, 2000, 64, 256, 16) == ("sink", 3)
    assert placement.n_int2_pages(2000, 64, 256, 16) == (placement.s_quant(2000, 64, 256, 16) - 64) // 16
