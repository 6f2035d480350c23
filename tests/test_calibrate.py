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
    # the traffic part of the rule alone (item term off, no reread
    # discount); small roots are one page run (one chunk), so it reads:
    # share iff (c - 1) * l * 4D > margin * 2 * (c * G rows) * (2D + 8)
    saved = (c - 1) * ell * HEAD_TOKEN_BYTES
    added = 2 * c * G * PARTIAL_ROW_BYTES
    if abs(saved - margin * added) < 0.05 * saved:
        pytest.skip("too close to the threshold")
    # 64 subtrees, as the calibration uses: enough work that a root of at
    # most four pages stays one page run
    t = cal.family_tree(ell, c, subtrees=64)
    assert cal.planner_shares_roots(t, 64, c, share_margin=margin, item_us=-1.0,
                                    reread_factor=1.0) == (saved > margin * added)


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


def _committed_grid():
    """(c, root tokens, measured side) rows of the committed calibration
    summary, as measured on the GPU."""
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                        "cost_model_calibration.txt")
    rows = []
    for line in open(path):
        f = line.split()
        if len(f) == 7 and f[0].isdigit() and f[4] in ("share", "fold", "tie"):
            rows.append((int(f[0]), int(f[1]), f[4]))
    return rows


def test_default_rule_reproduces_the_measured_sides():
    """The planner's default share/fold rule (its per-item start-cost term
    and reread discount included) takes the side the GPU measured as faster
    at (nearly) every point of the committed calibration grid: at least 14
    of 15, ties counting as agreement.  The rule of bytes alone (item term
    off, no reread discount) agrees at far fewer."""
    rows = _committed_grid()
    assert len(rows) == 15
    ok = sum(cal.agrees(cal.planner_shares_roots(cal.family_tree(ell, c), 64, c), side) for c, ell, side in rows)
    assert ok >= 14, f"default rule agrees at {ok} of {len(rows)}"
    bytes_only = sum(cal.agrees(cal.planner_shares_roots(cal.family_tree(ell, c), 64, c, item_us=-1.0,
                                                         reread_factor=1.0), side) for c, ell, side in rows)
    assert bytes_only < ok


@pytest.mark.parametrize("c", [2, 4, 8])
@pytest.mark.parametrize("ell", [16, 48, 64, 256, 1024])
def test_rule_with_item_term_is_its_closed_form(c, ell):
    # share iff (c - 1) l 4D / rho > 2 (c G) (2D + 8) + items x item_bytes,
    # one page run and one row group per root; item_bytes = t_round x
    # 7.2e6 B/us / (2 x 256 CUs)
    rho, t_round = 3.0, 4.7
    saved = (c - 1) * ell * HEAD_TOKEN_BYTES / rho
    added = 2 * c * G * PARTIAL_ROW_BYTES + t_round * 7.2e6 / 512
    if abs(saved - added) < 0.05 * added:
        pytest.skip("too close to the threshold")
    t = cal.family_tree(ell, c, subtrees=64)
    assert cal.planner_shares_roots(t, 64, c) == (saved > added)
    assert cal.planner_shares_roots(t, 64, c, item_us=t_round, reread_factor=rho) == (saved > added)
