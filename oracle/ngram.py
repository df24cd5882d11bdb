"""Prompt-lookup / n-gram drafting (TEST INFRASTRUCTURE ONLY).

Two definitions on the pages:
- "7.6 Speculative Decoding: Draft Models, Medusa, EAGLE & Lookahead",
  Exercise 4 (`ngram_draft`): the key is the last token; find its most recent
  earlier occurrence and propose the gamma tokens that followed it; a position
  past the end of the sequence, or every position when there is no earlier
  occurrence, proposes the last token again. Always gamma tokens, each with a
  one-hot q.
- "Medusa, EAGLE and self-speculation", "Copying, verified against plain greedy"
  (`lookup_draft`): the key is the last `ngram` tokens; scan the earlier
  start positions from right to left for the same n-gram and propose what
  followed it, at most k tokens and fewer where the sequence ends; no proposal
  when the sequence is shorter than ngram + 1 or the n-gram has no earlier
  occurrence.

Here both are one search with a switch: the last `ngram` tokens are looked up
at start positions i = T - ngram - 1 down to 0 (for ngram = 1 that is the
exercise's scan from T - 2 down), and then
- pad = True: gamma tokens, those past the end (or all, without a match)
  replaced by the last token (the exercise; for ngram > 1 its fill rule on top
  of the n-gram search);
- pad = False: the continuation, cut at the end of the sequence (the lookup
  page).
Plain Python loops, written from the two definitions.
"""
from __future__ import annotations

import numpy as np


def ngram_draft_one(seq, ngram: int, gamma: int, pad: bool):
    """One sequence (a list of ints). Returns (draft list, match start or -1).
    With pad, len(draft) == gamma; without, 0 .. gamma. An empty sequence has
    no last token to pad with: (None, -1) in pad mode, ([], -1) otherwise."""
    T = len(seq)
    if T == 0:
        return (None, -1) if pad else ([], -1)
    # The key is the n-gram that ends the sequence, starting at T - ngram. An
    # earlier occurrence starts at some i < T - ngram (it may overlap the key);
    # every start is compared token by token, in increasing order, and a later
    # match replaces an earlier one, so the most recent occurrence is kept.
    key = T - ngram
    match = -1
    for i in range(max(key, 0)):
        if all(seq[i + j] == seq[key + j] for j in range(ngram)):
            match = i
    # The proposal is what followed the occurrence, at most gamma tokens.
    follow = seq[match + ngram:match + ngram + gamma] if match >= 0 else []
    if pad:
        # The exercise's fill: the last token wherever the copy runs short.
        return follow + [seq[-1]] * (gamma - len(follow)), match
    return follow, match


def ngram_draft(tokens: np.ndarray, lengths: np.ndarray, ngram: int, gamma: int, pad: bool):
    """Batched: tokens [B, stride] int32, lengths [B]. Returns draft [B, gamma]
    (-1 past the count), count [B] (-1 for an invalid length: below 0, above
    the stride, or 0 in pad mode) and match [B] (start of the matched n-gram,
    -1 when none)."""
    B = tokens.shape[0]
    draft = np.full((B, gamma), -1, np.int32)
    count = np.zeros(B, np.int32)
    match = np.full(B, -1, np.int32)
    for b in range(B):
        T = int(lengths[b])
        if T < 0 or T > tokens.shape[1]:
            count[b] = -1
            continue
        d, m = ngram_draft_one([int(x) for x in tokens[b, :T]], ngram, gamma, pad)
        if d is None:
            count[b] = -1
            continue
        draft[b, :len(d)] = d
        count[b] = len(d)
        match[b] = m
    return draft, count, match
