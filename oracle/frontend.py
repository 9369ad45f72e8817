"""Token-level front end of the encoder, as plain reference code.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

H3 encoder page, ``_encode`` and the helpers it calls:

* token types: an id equal to the image token id is type 1, the video token
  id type 2, anything else text (type 0);
* ``embed_tokens`` followed by ``masked_scatter``: every token starts as its
  embedding-table row, then the image (video) token rows, in ascending token
  order, are replaced by the image (video) feature rows in order; the feature
  count must equal the placeholder count (``_get_placeholder_mask`` raises
  otherwise);
* ``_aggregate_deepstack``: with both images and videos, DeepStack level l is
  one array over all visual tokens in ascending order, each row taken from the
  image or the video features of that level according to the token's type;
  with one modality it is that modality's features and mask;
* ``_get_rope_index`` with ``_get_vision_position_ids``: the token types are
  cut into runs of equal type. A text run of n tokens takes positions
  cur .. cur+n-1 on all three axes and advances cur by n. A visual run takes
  the next grid of its modality (a video of t frames is t grids of one frame);
  with merge size m the grid (t, h, w) has t x h/m x w/m tokens, the token at
  frame f, row r, column c (row-major) gets (cur+f, cur+r, cur+c), and cur
  advances by max(h, w) / m. The position delta is max position + 1 - S.

Reading where the page is silent: a visual run must hold exactly the tokens
of one grid (the page's processor always brackets each image and each video
frame with text tokens); a run of another length, or a run with no grid left,
is an error, as the page's final position assignment would fail. Grids left
over after the last run are ignored, as on the page.
"""

from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np


def token_types(ids: np.ndarray, image_token_id: int, video_token_id: int) -> np.ndarray:
    """0 text, 1 image, 2 video, per token."""
    ids = np.asarray(ids)
    types = np.zeros(ids.shape, dtype=np.int64)
    types[ids == image_token_id] = 1
    types[ids == video_token_id] = 2
    return types


def _runs(types: np.ndarray) -> List[Tuple[int, int, int]]:
    """(type, start, end) of each maximal run of equal type, in order."""
    out = []
    s = 0
    n = len(types)
    while s < n:
        e = s
        while e < n and types[e] == types[s]:
            e += 1
        out.append((int(types[s]), s, e))
        s = e
    return out


def rope_index(ids, image_token_id: int, video_token_id: int,
               image_grid_thw: Optional[Sequence[Sequence[int]]],
               video_grid_thw: Optional[Sequence[Sequence[int]]],
               spatial_merge: int) -> Tuple[np.ndarray, int]:
    """(positions [3, S] int64 rows T, H, W; position delta)."""
    types = token_types(ids, image_token_id, video_token_id)
    image_grids = [tuple(int(v) for v in g) for g in (image_grid_thw or [])]
    video_frames = []
    for g in (video_grid_thw or []):
        t, h, w = (int(v) for v in g)
        video_frames.extend([(1, h, w)] * t)
    pending = {1: list(image_grids), 2: list(video_frames)}
    cols = []
    cur = 0
    for kind, s, e in _runs(types):
        n = e - s
        if kind == 0:
            for i in range(n):
                cols.append((cur + i, cur + i, cur + i))
            cur += n
            continue
        if not pending[kind]:
            raise ValueError(f"visual run at token {s} has no grid left")
        t, h, w = pending[kind].pop(0)
        lt, lh, lw = t, h // spatial_merge, w // spatial_merge
        if lt * lh * lw != n:
            raise ValueError(f"visual run at token {s} has {n} tokens, its grid {lt * lh * lw}")
        for f in range(lt):
            for r in range(lh):
                for c in range(lw):
                    cols.append((cur + f, cur + r, cur + c))
        cur += max(h, w) // spatial_merge
    if not cols:
        return np.zeros((3, 0), dtype=np.int64), 0
    pos = np.asarray(cols, dtype=np.int64).T.copy()
    return pos, int(pos.max()) + 1 - pos.shape[1]


def embed_and_scatter(table: np.ndarray, ids, image_token_id: int, video_token_id: int,
                      image_embeds: Optional[np.ndarray] = None,
                      video_embeds: Optional[np.ndarray] = None) -> np.ndarray:
    """inputs_embeds [S, hidden]: table rows, visual placeholders overwritten."""
    ids = np.asarray(ids)
    out = np.array(table[ids], dtype=np.float64)
    types = token_types(ids, image_token_id, video_token_id)
    for kind, feats in ((1, image_embeds), (2, video_embeds)):
        if feats is None:
            continue
        rows = [t for t in range(len(ids)) if types[t] == kind]
        if len(rows) != feats.shape[0]:
            raise ValueError(f"{len(rows)} placeholder tokens for {feats.shape[0]} features")
        for r, t in enumerate(rows):
            out[t] = feats[r]
    return out


def aggregate_deepstack(image_mask: Optional[np.ndarray], video_mask: Optional[np.ndarray],
                        ds_image: Optional[Sequence[np.ndarray]],
                        ds_video: Optional[Sequence[np.ndarray]]):
    """(visual_mask [S] bool or None, list of DeepStack levels or None)."""
    if image_mask is not None and video_mask is not None:
        visual = np.asarray(image_mask, bool) | np.asarray(video_mask, bool)
        vis_rows = [t for t in range(len(visual)) if visual[t]]
        levels = []
        for img, vid in zip(ds_image, ds_video):
            joint = np.zeros((len(vis_rows), img.shape[1]), dtype=np.float64)
            i = v = 0
            for r, t in enumerate(vis_rows):
                if image_mask[t]:
                    joint[r] = img[i]
                    i += 1
                else:
                    joint[r] = vid[v]
                    v += 1
            levels.append(joint)
        return visual, levels
    if image_mask is not None:
        return np.asarray(image_mask, bool), ds_image
    if video_mask is not None:
        return np.asarray(video_mask, bool), ds_video
    return None, None
