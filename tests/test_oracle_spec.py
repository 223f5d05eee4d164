"""Pins of the oracle's speculative-verification rule ("GLM-5.3 推理全链路
(七)", section 投机解码的输出行: k+1 sampled rows per request, accepted
tokens kept and the rejected suffix rolled back; "SGLang 源码完全拆解(十)",
section 逐 token 推进: rollback from the first mismatching position; "04 · 结构
化输出", 4.4 推进与终止: the tail past a terminator dropped).

The rule is pinned by what it must preserve: the emitted tokens are
distributed as the target model's own samples, whatever the drafts (the
chance that a draft token is accepted is the target's probability of it,
and after an acceptance the next token follows the next row's
distribution), checked by chi-square over seeds with the oracle's sampler
against closed-form probabilities; and by the page's accounting example
(2 of 6 drafts accepted, or all 6).  CPU only."""
import numpy as np
import scipy.special
import scipy.stats

import oracle


def _draws(z, n, offset):
    return np.array([oracle.sample_row(z, T=1.0, seed=s, offset=offset)["id"]
                     for s in range(1, n + 1)])


def test_acceptance_is_lossless_chi_square():
    z0 = np.array([1.0, 0.2, -0.5, 1.4, 0.0, -1.0], np.float32)
    z1 = np.array([-0.3, 0.9, 0.4, -1.2, 1.1, 0.0], np.float32)
    p0 = scipy.special.softmax(z0.astype(np.float64))
    p1 = scipy.special.softmax(z1.astype(np.float64))
    n = 30000
    y0, y1 = _draws(z0, n, 0), _draws(z1, n, 1)
    for d1 in (3, 5):
        counts = np.array([oracle.spec_accept([a, b], [d1])[1] for a, b in zip(y0, y1)])
        acc = counts == 2
        # P(accept) = p0(d1)
        k = int(acc.sum())
        assert scipy.stats.binomtest(k, n, p0[d1]).pvalue > 1e-4
        # after an acceptance the emitted second token follows row 1
        obs = np.bincount(y1[acc], minlength=6)
        assert scipy.stats.chisquare(obs, p1 * k).pvalue > 1e-4
        # on a rejection the emitted token follows row 0 without the draft
        q = p0.copy()
        q[d1] = 0.0
        q /= q.sum()
        obs = np.bincount(y0[~acc], minlength=6)
        m = obs.sum()
        keep = q > 0
        assert obs[d1] == 0
        assert scipy.stats.chisquare(obs[keep], q[keep] * m).pvalue > 1e-4


def test_page_accounting_examples():
    """k = 6 drafts: the first 2 accepted (3 tokens emitted: 2 drafts and the
    row's own token at the mismatch, 4 positions rolled back), or all 6 (7
    emitted with the bonus token, nothing rolled back)."""
    draft = [11, 12, 13, 14, 15, 16]
    tok, n, rb = oracle.spec_accept([11, 12, 99, 14, 15, 16, 17], draft)
    assert n == 3 and rb == 4 and list(tok) == [11, 12, 99]
    tok, n, rb = oracle.spec_accept([11, 12, 13, 14, 15, 16, 17], draft)
    assert n == 7 and rb == 0 and list(tok) == draft + [17]


def test_terminator_and_status_cut_the_emission():
    draft = [4, 5, 6]
    # a terminator among the accepted tokens: nothing after it is kept
    tok, n, rb = oracle.spec_accept([4, 5, 6, 7], draft, eos=5)
    assert list(tok) == [4, 5] and n == 2 and rb == 2
    # the terminator as the row's own token at a mismatch
    tok, n, rb = oracle.spec_accept([4, 8, 6, 7], draft, eos=8)
    assert list(tok) == [4, 8] and rb == 2
    # a row without a token (INVALID / OVERFLOW) ends the emission before it
    tok, n, rb = oracle.spec_accept([4, 5, -1, 7], draft, status=[0, 0, 2, 0])
    assert list(tok) == [4, 5] and rb == 2
    tok, n, rb = oracle.spec_accept([-1, 5, 6, 7], draft, status=[1, 0, 0, 0])
    assert n == 0 and rb == 4
    # k = 0: the bonus token alone
    tok, n, rb = oracle.spec_accept([9], [])
    assert list(tok) == [9] and rb == 0
