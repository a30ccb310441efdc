"""The bidirectional oracle's pins catch plausible mistakes (CPU only).

Each case replaces one function of ``oracle.bidirectional`` with a version that
makes a mistake a reading of the reverse scan could plausibly make, then runs
the behavioural pins of ``test_oracle_bidirectional`` (closed forms and
invariants; not the pin on ``successor_decays`` itself): at least one must
fail.  The readings pinned are those of the SGLang-diffusion "SANA-WM" page's
dense bidirectional mode as stated in the oracle: a reverse scan whose decays
sit on the forward scan's frame boundaries, summed with the forward scan.
"""
import numpy as np
import pytest

import test_oracle_bidirectional as pins
from oracle import bidirectional as BD
from oracle.recurrence import gdn_recurrence

PINS = [
    pins.test_closed_form_orthonormal_keys,
    pins.test_reverse_scan_exit_state_closed_form,
    pins.test_single_token_is_twice_the_forward,
    pins.test_zero_gate_cuts_both_directions,
    pins.test_mirrored_sequence_mirrors_the_output,
]

_orig_reverse_scan = BD.reverse_scan
_orig_bidirectional = BD.bidirectional


def _no_shift(g):
    # each token keeps its own decay in reverse
    return np.asarray(g, np.float64).copy()


def _predecessor_shift(g):
    # shifted the wrong way: token t takes token t - 1's decay
    g = np.asarray(g, np.float64)
    out = np.zeros_like(g)
    out[:, 1:] = g[:, :-1]
    return out


def _last_token_decays(g):
    # the scan also decays on entering the last token (by that token's gate)
    g = np.asarray(g, np.float64)
    out = np.zeros_like(g)
    out[:, :-1] = g[:, 1:]
    out[:, -1] = g[:, -1] - 0.5
    return out


def _not_reversed_back(q, k, v, g, beta, state_in=None, **kw):
    rev = lambda a: np.ascontiguousarray(np.asarray(a)[:, ::-1])  # noqa: E731
    return gdn_recurrence(rev(q), rev(k), rev(v), rev(BD.successor_decays(g)), rev(beta), state_in, **kw)


def _average(q, k, v, g, beta, **kw):
    return 0.5 * _orig_bidirectional(q, k, v, g, beta, **kw)


def _reverse_is_forward(q, k, v, g, beta, **kw):
    kw = dict(kw, want_state=False)
    o_f, _ = gdn_recurrence(q, k, v, g, beta, None, **kw)
    return 2.0 * o_f


def _reverse_without_own_write(q, k, v, g, beta, **kw):
    # the reverse scan reads out before writing its own token (exclusive)
    kw = dict(kw, want_state=False)
    o_f, _ = gdn_recurrence(q, k, v, g, beta, None, **kw)
    o_r, _ = _orig_reverse_scan(q, k, v, g, beta, None, **kw)
    # with every gate -inf the state is cleared before each token: o_t is token t's own write
    own, _ = gdn_recurrence(q, k, v, np.full(np.shape(g), -np.inf), beta, None, **kw)
    return o_f + o_r - own


MUTATIONS = {
    "no_shift": ("successor_decays", _no_shift),
    "shift_wrong_way": ("successor_decays", _predecessor_shift),
    "decay_entering_last_token": ("successor_decays", _last_token_decays),
    "output_not_reversed_back": ("reverse_scan", _not_reversed_back),
    "average_not_sum": ("bidirectional", _average),
    "reverse_scan_is_forward": ("bidirectional", _reverse_is_forward),
    "reverse_exclusive": ("bidirectional", _reverse_without_own_write),
}


def test_pins_pass_unmutated():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_fails_a_pin(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(BD, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    print(f"{name}: fails {len(failed)} of {len(PINS)} pins: {failed}")
    assert failed, f"mutation {name} passes every pin"
