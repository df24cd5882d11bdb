"""Pins of the oracle's n-gram drafter against the two definitions on the
pages ([SB] Exercise 4 `ngram_draft`; [SS] "Copying, verified against plain
greedy", `lookup_draft`) and a brute force written another way (a substring
search over a fixed-width text encoding of the tokens). No GPU."""
import numpy as np

from oracle import ngram as og


def test_last_token_key_copies_what_followed_and_pads_with_it():
    """[SB] Exercise 4: the most recent earlier occurrence of the last token,
    the gamma tokens after it, the last token where the sequence runs out or
    when nothing matches."""
    assert og.ngram_draft_one([5, 7, 9, 5], 1, 3, pad=True) == ([7, 9, 5], 0)
    assert og.ngram_draft_one([5, 7, 9, 5], 1, 5, pad=True) == ([7, 9, 5, 5, 5], 0)
    assert og.ngram_draft_one([4, 5, 8, 5, 6, 5], 1, 2, pad=True) == ([6, 5], 3)  # the most recent one
    assert og.ngram_draft_one([1, 2, 3], 1, 2, pad=True) == ([3, 3], -1)
    assert og.ngram_draft_one([3], 1, 4, pad=True) == ([3, 3, 3, 3], -1)


def test_lookup_is_empty_without_an_earlier_ngram():
    """[SS]: nothing when the sequence is shorter than ngram + 1 or the last
    ngram tokens do not occur earlier; otherwise at most k tokens, cut where
    the sequence ends."""
    assert og.ngram_draft_one([1, 2, 3], 3, 4, pad=False) == ([], -1)
    assert og.ngram_draft_one([1, 2, 3, 4, 2, 3], 3, 4, pad=False) == ([], -1)
    assert og.ngram_draft_one([1, 2, 3, 4, 9, 1, 2, 3], 3, 4, pad=False) == ([4, 9, 1, 2], 0)
    assert og.ngram_draft_one([1, 2, 3, 4, 1, 2, 3], 3, 4, pad=False) == ([4, 1, 2, 3], 0)
    # the match may overlap the key itself: a a a a -> match at 0, one token left
    assert og.ngram_draft_one([7, 7, 7, 7], 3, 4, pad=False) == ([7], 0)
    assert og.ngram_draft_one([], 2, 3, pad=False) == ([], -1)
    assert og.ngram_draft_one([], 1, 3, pad=True) == (None, -1)


def _brute(seq, ngram, gamma, pad):
    """The same rules through str.rfind over '%07d,' per token: a match can
    only start on a token boundary (the commas line up), and the window ends
    where a match would run into the last token."""
    T = len(seq)
    if T == 0:
        return (None, -1) if pad else ([], -1)
    text = "".join("%07d," % t for t in seq)
    w = 8
    m = -1
    if T >= ngram + 1:
        at = text.rfind(text[(T - ngram) * w:], 0, (T - 1) * w)
        m = at // w if at >= 0 else -1
    cont = seq[m + ngram:m + ngram + gamma] if m >= 0 else []
    if pad:
        cont = cont + [seq[-1]] * (gamma - len(cont))
    return cont, m


def test_matches_the_brute_force_on_random_sequences():
    rng = np.random.default_rng(0)
    checked = matched = 0
    for trial in range(3000):
        T = int(rng.integers(0, 40))
        alpha = int(rng.integers(2, 6))
        seq = [int(x) for x in rng.integers(0, alpha, T)]
        ngram = int(rng.integers(1, 5))
        gamma = int(rng.integers(1, 7))
        pad = bool(trial % 2)
        got = og.ngram_draft_one(seq, ngram, gamma, pad)
        assert got == _brute(seq, ngram, gamma, pad), (seq, ngram, gamma, pad, got)
        checked += 1
        matched += got[1] >= 0
    assert matched > checked // 3


def test_batched_form_and_invalid_lengths():
    tokens = np.array([[5, 7, 9, 5, 0, 0], [1, 2, 3, 4, 1, 2], [1, 1, 1, 1, 1, 1]], np.int32)
    draft, count, match = og.ngram_draft(tokens, np.array([4, 6, 7]), 2, 3, pad=False)
    assert count.tolist() == [0, 3, -1] and match.tolist() == [-1, 0, -1]
    assert draft.tolist() == [[-1, -1, -1], [3, 4, 1], [-1, -1, -1]]
    draft, count, match = og.ngram_draft(tokens, np.array([4, 5, 6]), 2, 3, pad=False)
    # row 1 no longer ends in an earlier bigram; row 2 (six 1s) matches at 3 with one token left
    assert count.tolist() == [0, 0, 1] and match.tolist() == [-1, -1, 3] and draft[2].tolist() == [1, -1, -1]
    draft, count, match = og.ngram_draft(tokens, np.array([4, 0, -1]), 1, 3, pad=True)
    assert count.tolist() == [3, -1, -1] and draft[0].tolist() == [7, 9, 5]
    assert np.all(draft[1:] == -1)
