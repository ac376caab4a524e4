"""Chunk policy of the streaming vocoder, written from the pages (oracle side).

TEST INFRASTRUCTURE: see ``oracle/__init__.py``.

Source: AI-infra handbook, "Qwen3-TTS" case, section "third stop: the
streaming vocoder".  The vocoder decodes when the number of *generated*
frames (all frames received minus the reference frames prefixed once)
reaches the next threshold; the final chunk always decodes.  Thresholds grow
by the chunk ramp (1, 2, 4 frames) and then by the steady stride (8).  The
stateless variant re-decodes each chunk with up to 16 frames of left context,
and the section lists the window lengths that occur.  A per-request initial
chunk size is validated and capped at the steady size.
"""
from __future__ import annotations

import operator


def initial_chunk_size(requested, steady: int, fallback: int = 0) -> int:
    """Size of a request's first decode, in frames.

    A request may name its own first-chunk size; without one (``None``) the
    server's ``fallback`` applies.  The size is a whole number of frames, at
    least 0, and never larger than the steady chunk: a larger request is cut
    down to ``steady``.  The steady chunk itself must be at least one frame.

    Errors: ``ValueError`` for a steady size below 1 or a negative request;
    ``TypeError`` for a request that is not an integer (``bool`` and
    non-integral numbers included).
    """
    if steady < 1:
        raise ValueError(f"steady chunk size {steady} is below one frame")
    chosen = fallback if requested is None else requested
    if isinstance(chosen, bool):
        raise TypeError("a chunk size is a frame count, not a flag")
    try:
        frames = operator.index(chosen)
    except TypeError:
        raise TypeError(f"chunk size {chosen!r} is not an integer frame count") from None
    if frames < 0:
        raise ValueError(f"chunk size {frames} is negative")
    return steady if frames > steady else frames


def strides(ramp, steady: int, initial: int = 0):
    """Yield new-frame counts per decode: the first is ``initial`` when it is
    positive, else ramp[0]; then the remaining ramp entries, each clamped to
    the steady stride; then the steady stride forever."""
    first = initial if initial > 0 else (ramp[0] if ramp else steady)
    yield min(first, steady)
    for s in ramp[1:]:
        yield min(s, steady)
    while True:
        yield steady


def chunk_plan(total_generated: int, ramp=(1, 2, 4), steady: int = 8, initial: int = 0) -> list[int]:
    """New frames per decode for an utterance of ``total_generated`` frames
    arriving one at a time: decode whenever the generated count reaches the
    next threshold, and decode the remainder when the utterance ends."""
    out: list[int] = []
    it = strides(ramp, steady, initial)
    threshold = next(it)
    done = 0
    for g in range(1, total_generated + 1):
        if g >= threshold:
            out.append(g - done)
            done = g
            threshold = g + next(it)
    if done < total_generated:
        out.append(total_generated - done)
    return out


def decode_points(plan: list[int]) -> list[int]:
    """Cumulative generated-frame counts at which each decode happens."""
    pts, acc = [], 0
    for n in plan:
        acc += n
        pts.append(acc)
    return pts


def window_frame_counts(left_context: int, ramp=(1, 2, 4), steady: int = 8) -> tuple[int, ...]:
    """Window lengths of the stateless re-decode: each decode covers its new
    frames plus up to ``left_context`` earlier frames.  While the left
    context is still filling, the ramp's cumulative counts occur; once it is
    full, any stride from 1 to the steady stride can occur (arrival jitter)."""
    sizes = set()
    prior = 0
    it = strides(ramp, steady)
    while prior < left_context:
        n = next(it)
        sizes.add(min(prior, left_context) + n)
        prior += n
    for k in range(1, steady + 1):
        sizes.add(left_context + k)
    return tuple(sorted(sizes))
