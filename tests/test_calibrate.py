"""Host-side tests of the cost-model calibration (no GPU): the planner's
share/fold decision on the calibration trees follows the closed form of its
rule, and the fitting helpers pick what they should."""
import pytest

from decode_attention_prefix_amd import calibrate as cal

G = cal.HQ // cal.HKV
PARTIAL_ROW_BYTES = 2 * cal.D + 8          # fp16 o/l + fp32 m + fp32 l
HEAD_TOKEN_BYTES = 4 * cal.D               # K + V of one token, one KV head


@pytest.mark.parametrize("c", [2, 4, 8])
@pytest.mark.parametrize("ell", [16, 32, 48, 64])
@pytest.mark.parametrize("margin", [1.0, 4.0, 16.0, 64.0])
def test_planner_decision_is_the_closed_form(c, ell, margin):
    # small roots are one page run (one chunk), so the rule reads:
    # share iff (c - 1) * l * 4D > margin * 2 * (c * G rows) * (2D + 8)
    saved = (c - 1) * ell * HEAD_TOKEN_BYTES
    added = 2 * c * G * PARTIAL_ROW_BYTES
    if abs(saved - margin * added) < 0.05 * saved:
        pytest.skip("too close to the threshold")
    # 64 subtrees, as the calibration uses: enough work that a root of at
    # most four pages stays one page run
    t = cal.family_tree(ell, c, subtrees=64)
    assert cal.planner_shares_roots(t, 64, c, share_margin=margin) == (saved > margin * added)


def test_forced_modes_are_seen():
    t = cal.family_tree(1024, 4, subtrees=8)
    assert cal.planner_shares_roots(t, 8, 4, share_mode=1)
    assert not cal.planner_shares_roots(t, 8, 4, share_mode=0)


def test_measured_side_and_crossover():
    assert cal.measured_side(90.0, 100.0) == "share"
    assert cal.measured_side(100.0, 90.0) == "fold"
    assert cal.measured_side(100.0, 99.0) == "tie"
    lengths = [16, 64, 256, 1024, 4096]
    assert cal.crossover(lengths, ["fold", "fold", "share", "tie", "share"]) == 256
    assert cal.crossover(lengths, ["share"] * 5) == 16
    assert cal.crossover(lengths, ["share", "share", "share", "share", "fold"]) is None
    assert cal.crossover(lengths, ["fold", "share", "fold", "share", "share"]) == 1024


def test_fit_margin_recovers_a_planted_threshold():
    # toy model: share iff length > margin * 10; "measured": share from 100 up
    points = [((ell,), "share" if ell >= 100 else "fold") for ell in (10, 30, 50, 70, 100, 200, 400)]
    m, acc = cal.fit_margin(points, lambda k, m: k[0] > m * 10)
    assert acc == 1.0 and m == 8.0
    # all margins agree on ties: the one closest to 1 wins
    m, acc = cal.fit_margin([((5,), "tie")], lambda k, m: True)
    assert m == 1.0 and acc == 1.0
