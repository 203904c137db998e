"""Planted mistakes in the oracle (CPU only) must each fail at least one pin.

Each mutant replaces one of the oracle's named readings with a plausible wrong
version (a dropped term, a wrong index, an off-by-one mask, a transposed operand)
and runs the pins of tests/test_oracle_attention.py against it.
"""
import numpy as np
import pytest

import oracle.attention as oa
import tests.test_oracle_attention as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _mla_pins():
    return [
        _fails(pins.test_mla_prefill_vs_torch_sdpa_concat),
        _fails(pins.test_mla_prefill_brute_force),
        _fails(pins.test_per_token_scale_algebra),
        _fails(pins.test_mla_prefill_per_head_rope),
    ]


MUTANTS = {
    "gqa_modulo_instead_of_group": ("kv_head", lambda h, Hq, Hkv: h % Hkv),
    "causal_strict_less": ("causal_visible",
                           lambda rows, Sq, Skv: np.arange(Skv)[None, :] < (rows[:, None] + (Skv - Sq))),
    "causal_top_left": ("causal_visible", lambda rows, Sq, Skv: np.arange(Skv)[None, :] <= rows[:, None]),
    "mla_rope_dropped": ("mla_logits", lambda qn, kn, qr, kr, qs, ks, s: s * ((qn @ kn.T) * qs[:, None] * ks[None, :])),
    "mla_scale_outside_rope": ("mla_logits",
                               lambda qn, kn, qr, kr, qs, ks, s: s * ((qn @ kn.T) + qr @ kr.T) * qs[:, None] * ks[None, :]),
    "mla_k_scale_squared": ("mla_logits",
                            lambda qn, kn, qr, kr, qs, ks, s: s * ((qn @ kn.T) * qs[:, None] * ks[None, :] ** 2 + qr @ kr.T)),
    "mla_softmax_scale_on_nope_only": ("mla_logits",
                                       lambda qn, kn, qr, kr, qs, ks, s: s * (qn @ kn.T) * qs[:, None] * ks[None, :] + qr @ kr.T),
    "mla_decode_v_last_columns": ("mla_value", lambda kv, Dv: kv[..., -Dv:]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    if attr == "kv_head":
        caught = [_fails(pins.test_prefill_vs_torch_sdpa, False, 8, 2),
                  _fails(pins.test_decode_vs_torch_sdpa_with_lengths)]
    elif attr == "causal_visible":
        caught = [_fails(pins.test_prefill_vs_torch_sdpa, True, 4, 4),
                  _fails(pins.test_causal_bottom_right_suffix),
                  _fails(pins.test_prefill_brute_force, True, 1, 3, 6, 4, 2, 3, 2)]
    elif attr == "mla_logits":
        caught = _mla_pins()
    else:
        caught = [_fails(pins.test_mla_decode_vs_torch_sdpa), _fails(pins.test_mla_decode_brute_force)]
    assert any(caught), f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_the_same_pins():
    assert not any(_mla_pins())
    assert not _fails(pins.test_prefill_vs_torch_sdpa, True, 8, 2)
    assert not _fails(pins.test_causal_bottom_right_suffix)
    assert not _fails(pins.test_mla_decode_vs_torch_sdpa)


def test_sdpa_without_max_subtraction_is_caught(monkeypatch):
    """A softmax that skips the max shift overflows on logits of order 1e3."""
    def unshifted(q, k, v, visible, logits=None, scale=1.0):
        x = scale * (q @ k.T) if logits is None else logits
        if visible is not None:
            x = np.where(visible, x, -np.inf)
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(x)
            s = e.sum(1, keepdims=True)
            return (e / s) @ v, np.log(s[:, 0])
    monkeypatch.setattr(oa, "sdpa_rows", unshifted)
    assert _fails(pins.test_prefill_large_logits_no_overflow)
