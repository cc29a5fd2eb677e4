"""The speculation cost governor (host C++; TensorSharp speculative decoding
page, protocol section and governor paragraphs), driven on the CPU with
scripted step timings.  Each expected decision string is written out from
the page's numbers: a full probe of 8 speculative steps, a re-probe of 3
after a loss, parks of 32 -> 64 -> 128 -> 256 steps, four zero-accept
speculative steps ending a probe, a hold re-checked on its last 8 steps and
refreshed by 3 plain steps every 64, and a new request capping a park at 32.
P = plain step, S = speculative step."""
import pytest

from draft_verify_amd import specv


def run(gov, n, cost):
    """n steps; cost(decision, i) -> (committed, accepted, seconds).  Returns
    the decision string."""
    out = []
    for i in range(n):
        d = gov.should_draft()
        c, a, s = cost(d, i)
        gov.record(d, c, a, s)
        out.append("S" if d else "P")
    return "".join(out)


def losing(d, i):   # speculative: 2 tokens in 5 ms (2.5 ms/token) against 1 ms/token plain
    return (2, 1, 5e-3) if d else (1, 0, 1e-3)


def winning(d, i):  # speculative: 3 tokens in 1.5 ms (0.5 ms/token)
    return (3, 2, 1.5e-3) if d else (1, 0, 1e-3)


def zero_accept(d, i):  # speculative steps that accept nothing: one token each, a little dearer
    return (1, 0, 1.1e-3) if d else (1, 0, 1e-3)


def test_losing_pairing_parks_with_backoff():
    g = specv.Governor()
    seq = run(g, 3 + 8 + 32 + 3 + 64 + 3 + 128 + 3 + 256 + 3 + 256 + 3, losing)
    expect = ("PPP" + "S" * 8 + "P" * 32 + "SSS" + "P" * 64 + "SSS" + "P" * 128 + "SSS" + "P" * 256
              + "SSS" + "P" * 256 + "SSS")
    assert seq == expect
    st = g.stats()
    assert st["losses"] == 6 and st["wins"] == 0
    assert st["parked_steps"] == 32 + 64 + 128 + 256 + 256
    # parked steps feed the baseline except the first of each park
    assert st["plain_samples"] == 3 + (32 + 64 + 128 + 256 + 256) - 5
    assert abs(st["plain_ms_per_token"] - 1.0) < 1e-9


def test_four_zero_accept_steps_end_a_probe():
    g = specv.Governor()
    seq = run(g, 3 + 4 + 32 + 3 + 2, zero_accept)
    # the full probe of 8 ends after 4; the short re-probe of 3 ends before the
    # zero-accept limit and loses on its verdict (1.1 against 1 ms/token), parking 64
    assert seq == "PPP" + "SSSS" + "P" * 32 + "SSS" + "PP"
    assert g.stats()["losses"] == 2


def test_winning_pairing_holds_and_refreshes_its_baseline():
    g = specv.Governor()
    seq = run(g, 3 + 8 + 64 + 3 + 64 + 3, winning)
    assert seq == "PPP" + "S" * 8 + "S" * 64 + "PPP" + "S" * 64 + "PPP"
    st = g.stats()
    assert st["wins"] == 1 and st["losses"] == 0 and st["parked_steps"] == 0
    assert abs(st["spec_ms_per_token"] - 0.5) < 1e-9


def test_a_held_win_that_turns_into_a_loss_parks_within_eight_steps():
    g = specv.Governor()

    def turn(d, i):  # wins for 20 steps, then speculation loses
        return winning(d, i) if i < 20 else losing(d, i)
    seq = run(g, 3 + 8 + 9 + 8 + 32, turn)
    # steps 11..19 hold on winning samples; from step 20 the window of the last
    # 8 turns: 3 winning + 5 losing = 14.5 ms / 19 tokens > 1 ms -> park at the
    # 5th losing step
    k = seq.index("P", 11)
    assert seq[:k] == "PPP" + "S" * (k - 3)
    assert 20 <= k - 1 <= 27
    assert seq[k:k + 32] == "P" * 32


def test_a_win_resets_the_backoff():
    g = specv.Governor()
    phase = {"lose": True}

    def cost(d, i):
        return losing(d, i) if phase["lose"] else winning(d, i)
    seq = run(g, 3 + 8 + 32 + 3 + 64, cost)      # two losses: next park would be 128
    phase["lose"] = False
    seq2 = run(g, 3, cost)                       # short re-probe wins
    assert seq2 == "SSS" and g.stats()["wins"] == 1
    phase["lose"] = True
    seq3 = run(g, 8 + 32 + 3, cost)              # the hold turns: a loss parks 32 (not 128),
    p = seq3.index("P")                          # then the short re-probe of a losing verdict
    assert seq3[p:p + 32] == "P" * 32 and seq3[p + 32:p + 35] == "SSS"


def test_new_request_caps_the_park_and_keeps_the_short_probe():
    g = specv.Governor()
    run(g, 3 + 8 + 32 + 3 + 10, losing)          # in the middle of a 64-step park
    g.new_request()
    seq = run(g, 32 + 3 + 32, losing)
    assert seq == "P" * 32 + "SSS" + "P" * 32   # capped at 32, short re-probe, backoff restarted


def test_record_must_follow_the_decision():
    g = specv.Governor()
    assert not g.should_draft()
    with pytest.raises(specv.SpecError) as e:
        g.record(True, 2, 1, 1e-3)
    assert e.value.code == specv.SPEC_ESTATE
    with pytest.raises(specv.SpecError):
        g.record(False, 0, 0, 1e-3)              # a step commits at least one token


def test_custom_numbers():
    p = specv.spec_governor_params(probe_spec=2, probe_spec_short=1, probe_plain=1, park_first=4,
                                   park_max=8, zero_accept_exit=4, hold_window=2, hold_refresh=5)
    g = specv.Governor(p)
    assert run(g, 1 + 2 + 4 + 1 + 8 + 1 + 8, losing) == "P" + "SS" + "PPPP" + "S" + "P" * 8 + "S" + "P" * 8
    bad = specv.spec_governor_params(0, 1, 1, 4, 8, 4, 2, 5)
    with pytest.raises(specv.SpecError):
        specv.Governor(bad)
