"""Greedy speculative accept and the draft-window rule (test oracle).

Source: Hugging Face "Assisted Generation" page, section "Assisted Generation
loop":

* the assistant drafts a short candidate window greedily, 5 tokens at first;
* the base model scores the whole window in one pass (logits at every
  position);
* its predicted tokens are compared with the candidates from the left;
* at the first mismatch the base model's own token is kept and the later
  candidates are dropped;
* the window grows by 2 when every candidate matched and shrinks by 1
  otherwise.

Readings taken:

* the base model's prediction at a position is the argmax of that row's
  logits; among equal maxima the lowest index wins; a NaN counts as the
  maximum and the first NaN wins (numpy's rule; callers pass finite logits);
* row ``i`` (``i < n``) of a sequence predicts the token after window token
  ``i`` and is compared with draft ``i``; row ``n`` is the bonus row;
* the accepted count includes the kept base-model token: ``m + 1``, where
  ``m`` is the first mismatching draft index (``m = n`` if all match); the
  next token is the argmax of row ``m``;
* the window never drops below 1; zero drafts count as a full match.

Layouts: logits float32 [sum(n_draft + 1), V] packed by sequence; draft_ids
int32 packed [sum(n_draft)]; n_draft int32 [B].
"""

import numpy as np


def argmax_rows(logits):
    """Index of each row's maximum (lowest index among ties, first NaN wins)."""
    x = np.asarray(logits, dtype=np.float32)
    return np.argmax(x, axis=1).astype(np.int64)


def accept(logits, draft_ids, n_draft):
    """Returns (accepted[B], next_token[B], first_mismatch[B]) as int32."""
    n_draft = np.asarray(n_draft, dtype=np.int64)
    draft_ids = np.asarray(draft_ids, dtype=np.int64)
    rows_needed = int(np.sum(n_draft + 1))
    if logits.shape[0] != rows_needed or draft_ids.shape[0] != int(np.sum(n_draft)):
        raise ValueError("logits rows must be sum(n_draft + 1) and drafts sum(n_draft)")
    pred = argmax_rows(logits)
    B = len(n_draft)
    accepted = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    first = np.zeros(B, dtype=np.int32)
    r0 = 0
    d0 = 0
    for b in range(B):
        n = int(n_draft[b])
        m = n
        for i in range(n):                   # compare from the left
            if pred[r0 + i] != draft_ids[d0 + i]:
                m = i
                break
        first[b] = m
        accepted[b] = m + 1                  # matched drafts + the base model's token
        nxt[b] = pred[r0 + m]
        r0 += n + 1
        d0 += n
    return accepted, nxt, first


def window_next(window, n_draft, accepted):
    """Next draft window: +2 after a full match, otherwise -1 (at least 1)."""
    window = np.asarray(window, dtype=np.int64)
    full = np.asarray(accepted, dtype=np.int64) == np.asarray(n_draft, dtype=np.int64) + 1
    return np.where(full, window + 2, np.maximum(1, window - 1)).astype(np.int32)
