"""The fp64 oracle against brute force, a library routine, finite differences,
closed forms, invariants and the pages' streaming identity; plus planted
mistakes in a copy of the oracle that the pins must catch.  CPU only."""
import importlib.util
import os
import types

import pytest

import oracle.reference as ref
from tests import pins

ORACLE_SRC = os.path.join(os.path.dirname(ref.__file__), "reference.py")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ref)


def _mutant(old: str, new: str) -> types.ModuleType:
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


MUTANTS = {
    # log-softmax without the log-sum-exp term
    "dropped_lse": ("return s - lse, lse[:, 0]", "return s - m, lse[:, 0]"),
    # KL weighted by the student's probabilities
    "wrong_weight": ("p1 = np.exp(lp1)\n    with np.errstate", "p1 = np.exp(lp2)\n    with np.errstate"),
    # Setting 1 gradient with the wrong sign
    "set1_sign": ("ds = g[:, None] * (np.exp(lp2) - p1)", "ds = g[:, None] * (p1 - np.exp(lp2))"),
    # Setting 2 gradient without the -KL term
    "set2_drop_kl": ("ds = g[:, None] * p1 * (r - kl[:, None])", "ds = g[:, None] * p1 * r"),
    # the two settings swapped
    "swapped_settings": ("if setting == 1:\n        ds =", "if setting == 2:\n        ds ="),
    # dK built from the keys instead of the queries (transposed operand)
    "dk_operand": ("dk += scale * (ds.T @ q_t[r])", "dk += scale * (ds.T @ k_t[r])"),
    # dQ without the softmax scale
    "dq_no_scale": ("dq[r] = scale * (ds @ k_t)", "dq[r] = ds @ k_t"),
    # causal mask aligned top-left instead of bottom-right
    "causal_top_left": ("return j <= (rows[:, None] + (n_k - n_q))", "return j <= rows[:, None]"),
    # causal mask off by one
    "causal_off_by_one": ("return j <= (rows[:, None] + (n_k - n_q))", "return j < (rows[:, None] + (n_k - n_q))"),
    # teacher logits built from the student's keys
    "s1_operand": ("s1 = scale * (q1[rows] @ k1.T)", "s1 = scale * (q1[rows] @ k2.T)"),
    # dK from saved statistics with the student's LSE in the teacher's log-probabilities
    "state_wrong_lse": ("lp1 = np.where(mask, s1 - lse1[r, None], -np.inf)",
                        "lp1 = np.where(mask, s1 - lse2[r, None], -np.inf)"),
    # dK from saved statistics ignoring the causal mask
    "state_no_mask": ("mask = allowed_mask(r, n_q, n_k, causal, keys)",
                      "mask = allowed_mask(r, n_q, n_k, False, keys)"),
    # upstream weight ignored in Setting 2
    "set2_drop_g": ("ds = g[:, None] * p1 * (r - kl[:, None])", "ds = p1 * (r - kl[:, None])"),
    # the full logit gradient without the upstream weights
    "dlogits_drop_g": ("return _dlogits(setting, mask, lp1, lp2, kl, g)",
                       "return _dlogits(setting, mask, lp1, lp2, kl, np.ones(n_q))"),
    # the full logit gradient of the other setting
    "dlogits_swapped_setting": ("return _dlogits(setting, mask, lp1, lp2, kl, g)",
                                "return _dlogits(3 - setting, mask, lp1, lp2, kl, g)"),
    # the full logit gradient with the KL of a different row block (rows shifted by one)
    "dlogits_wrong_kl": ("return _dlogits(setting, mask, lp1, lp2, kl, g)",
                         "return _dlogits(setting, mask, lp1, lp2, np.roll(kl, 1), g)"),
    # multi-head forward reading head 0's keys for every head
    "multihead_wrong_head": ("forward_head(q1[h], k1[h], q2[h], k2[h], scale, causal)",
                             "forward_head(q1[h], k1[0], q2[h], k2[h], scale, causal)"),
    # multi-head backward with head 0's upstream weights for every head
    "multihead_wrong_g": ("None if dkl is None else dkl[h])", "None if dkl is None else dkl[0])"),
}


# a mutant may produce NaN on the way to failing a pin (an empty causal row)
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"


def test_page_memory_figure():
    """The pages' closed-form figure: materialising P1 and P2 at 64K context,
    32 heads, BF16 takes about 512 GB (StreamKL gist.science technical summary,
    Problem Statement)."""
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")) as f:
        golden = json.load(f)
    f = golden["materialized_p1_p2_bytes"]
    n, heads, bytes_per = f["context"], f["heads"], f["bytes_per_element"]
    total = 2 * n * n * heads * bytes_per
    assert total == 2 ** 39                      # 512 GiB exactly
    assert abs(total / 2 ** 30 - f["approx_gb"]) < 1e-9
