"""O2: where each cached position lives (sink / INT2 / recent ring).

Test infrastructure (see ``oracle/__init__.py``).

Sources:
* OSCAR summary page, section 4 "KV Cache Layout": the first S0 tokens (sink)
  and the most recent W tokens stay in BF16; the middle context is INT2.
* OSCAR summary page, section 4 "KV Cache Update": new tokens enter the BF16
  recent window and the oldest ones are demoted into the INT2 middle region.
* WUSH-KV notes, "method step details" (inference, Algorithm 2): keep a
  quantized right boundary S_quant; quantize the S_flush-aligned segments that
  lie beyond the S_sink and S_keep windows, then move S_quant.

Reading taken: after every append, while len - S_quant >= S_keep + S_flush,
quantize [S_quant, S_quant + S_flush) and advance S_quant by S_flush.  Its
closed form is ``s_quant`` below.  S_flush = 1 is OSCAR's one-token demotion.
The recent window is a ring of R = roundup16(S_keep + S_flush) rows; position
p sits in ring slot (p - S_sink) mod R.  INT2 position p sits in logical page
(p - S_sink) // 16, slot (p - S_sink) % 16.
"""

PAGE = 16


def s_quant(length, s_sink, s_keep, s_flush):
    """Quantized right boundary after ``length`` tokens have been appended."""
    k = (length - s_sink - s_keep) // s_flush
    return s_sink + s_flush * max(0, k)


def ring_capacity(s_keep, s_flush):
    return -(-(s_keep + s_flush) // PAGE) * PAGE


def segments(length, s_sink, s_keep, s_flush):
    """(sink, int2, recent) half-open position ranges of a length-``length`` cache."""
    sq = s_quant(length, s_sink, s_keep, s_flush)
    sink = (0, min(length, s_sink))
    int2 = (s_sink, sq) if sq > s_sink else (s_sink, s_sink)
    lo = max(sq, s_sink)
    recent = (lo, length) if length > lo else (lo, lo)
    return sink, int2, recent


def where(p, length, s_sink, s_keep, s_flush):
    """('sink', slot) | ('int2', logical_page, slot) | ('ring', slot) for position p."""
    assert 0 <= p < length
    sink, int2, recent = segments(length, s_sink, s_keep, s_flush)
    if p < sink[1]:
        return ("sink", p)
    if int2[0] <= p < int2[1]:
        m = p - s_sink
        return ("int2", m // PAGE, m % PAGE)
    assert recent[0] <= p < recent[1]
    return ("ring", (p - s_sink) % ring_capacity(s_keep, s_flush))


def n_int2_pages(length, s_sink, s_keep, s_flush):
    sq = s_quant(length, s_sink, s_keep, s_flush)
    return -(-(sq - s_sink) // PAGE) if sq > s_sink else 0
