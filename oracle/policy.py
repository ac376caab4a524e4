"""Chunk policy of the streaming vocoder, written from the pages (oracle side).

TEST INFRASTRUCTURE: see ``oracle/__init__.py``.

Source: AI-infra handbook, "Qwen3-TTS" case, section "third stop: the
streaming vocoder".  The vocoder decodes when the number of *generated*
frames (all frames received minus the reference frames prefixed once)
reaches the next threshold; the final chunk always decodes.  Thresholds grow
by the chunk ramp (1, 2, 4 frames) and then by the steady stride (8).  The
stateless variant re-decodes each chunk with up to 16 frames of left context,
and the section lists the window lengths that occur.  A per-request initial
chunk size is validated and clamped to the steady size (the section's
``resolve_initial_codec_chunk_frames``).
"""
from __future__ import annotations


def resolve_initial_chunk_frames(value, steady_chunk_frames: int, default_frames: int = 0) -> int:
    """Per-request initial chunk size: None -> default; must be an integer
    >= 0; the result is clamped to the steady size (which must be positive)."""
    if steady_chunk_frames <= 0:
        raise ValueError(f"steady_chunk_frames must be positive, got {steady_chunk_frames}")
    if value is None:
        value = default_frames
    try:
        frames = int(value)
    except (TypeError, ValueError) as exc:
        raise TypeError("initial chunk frames must be an integer") from exc
    if frames < 0:
        raise ValueError("initial chunk frames must be >= 0")
    return min(frames, int(steady_chunk_frames))


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
