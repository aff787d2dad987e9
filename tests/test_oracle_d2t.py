"""Pins of the reduced-draft-vocabulary widening (CPU): by hand, the identity table, the
probability mass it carries over, and the tables it refuses."""
import numpy as np
import pytest

from oracle.sampling import truncated_distribution, widen_draft_logits


def test_widening_by_hand():
    # V = 6, V_d = 3, offsets (1, 2, 2): draft ids 0, 1, 2 -> target ids 1, 3, 4
    dl = np.array([[0.5, -1.0, 2.0], [3.0, 0.0, -2.5]], dtype=np.float32)
    out = widen_draft_logits(dl, [1, 2, 2], 6)
    ninf = -np.inf
    assert out.tolist() == [[ninf, 0.5, ninf, -1.0, 2.0, ninf],
                            [ninf, 3.0, ninf, 0.0, -2.5, ninf]]


def test_identity_table_changes_nothing():
    rng = np.random.default_rng(1)
    dl = rng.standard_normal((4, 50)).astype(np.float32)
    assert np.array_equal(widen_draft_logits(dl, np.zeros(50, np.int64), 50), dl)


@pytest.mark.parametrize("temperature,top_k,top_p", [(1.0, 0, 1.0), (0.7, 20, 0.9)])
def test_widened_distribution_is_the_draft_distribution_moved(temperature, top_k, top_p):
    """The widened row's (truncated) probabilities at the mapped ids are the draft row's,
    and every other target id gets exactly 0."""
    rng = np.random.default_rng(2)
    vocab, dvocab = 300, 64
    target = np.sort(rng.choice(vocab, size=dvocab, replace=False))
    d2t = target - np.arange(dvocab)
    dl = (2.0 * rng.standard_normal(dvocab)).astype(np.float32)
    wide = widen_draft_logits(dl[None], d2t, vocab)[0]
    q_d = truncated_distribution(dl, temperature, top_k, top_p).probs
    q_w = truncated_distribution(wide, temperature, top_k, top_p).probs
    # equal up to the order of the fp64 normalizing sums (the wide row adds exact zeros)
    assert np.allclose(q_w[target], q_d, rtol=1e-14, atol=0)
    off = np.ones(vocab, bool)
    off[target] = False
    assert np.all(q_w[off] == 0.0)
    assert abs(q_w.sum() - 1.0) < 1e-12


@pytest.mark.parametrize("d2t,vocab", [([0, 0, -1], 5),      # two draft ids -> target 1
                                       ([0, 5, 0], 5),       # target 6 outside V = 5
                                       ([-1, 0, 0], 5),      # target -1
                                       ([0, 0], 5)])         # one offset missing
def test_refuses_bad_tables(d2t, vocab):
    with pytest.raises(ValueError):
        widen_draft_logits(np.zeros((1, 3), np.float32), d2t, vocab)
