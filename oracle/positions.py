"""Reference 3-axis (T, H, W) position ids for a run of text and visual segments.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

H3 encoder page, ``_get_rope_index`` and ``_get_vision_position_ids``: tokens
are grouped into runs of one modality. A text run of n tokens takes positions
current, current+1, ..., current+n-1 on all three axes and advances current
by n. A visual run with merged grid (t, h, w) takes, for the token at frame f,
row r, column c (row-major within a frame, frames in order), the position
(current + f, current + r, current + c), and advances current by max(h, w).
"""

from __future__ import annotations

from typing import Iterable, Tuple, Union

import numpy as np

Segment = Tuple[str, Union[int, Tuple[int, int, int]]]


def text_and_grid_positions(segments: Iterable[Segment]) -> np.ndarray:
    """Positions [3, S] (int64) for segments ``("text", n)`` / ``("visual", (t, h, w))``."""
    cols = []
    current = 0
    for kind, spec in segments:
        if kind == "text":
            n = int(spec)
            for i in range(n):
                cols.append((current + i, current + i, current + i))
            current += n
        elif kind == "visual":
            t, h, w = (int(x) for x in spec)
            for f in range(t):
                for r in range(h):
                    for c in range(w):
                        cols.append((current + f, current + r, current + c))
            current += max(h, w)
        else:
            raise ValueError(f"unknown segment kind {kind!r}")
    if not cols:
        return np.zeros((3, 0), dtype=np.int64)
    return np.asarray(cols, dtype=np.int64).T.copy()
