"""Host-side checks of the verification-cost model (no GPU)."""
import importlib.util
import math
import os

import pytest

# loaded by path: the model is plain host arithmetic and needs neither the
# package's HIP library nor torch
_spec = importlib.util.spec_from_file_location(
    "cost_model", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                               "speculative_decoding_verification_w4a16_amd", "cost_model.py"))
cm = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(cm)


def test_plain_decoding_is_unit_speedup():
    # verifying one row with no draft emits one token per plain step
    assert cm.speedup(1, 1.0, 0.0) == 1.0


def test_break_even_is_where_speedup_is_one():
    for r in (1.07, 1.93, 2.5):
        for d in (0.0, 0.1, 0.5):
            assert math.isclose(cm.speedup(cm.break_even(r, d), r, d), 1.0)


def test_monotone_in_each_argument():
    assert cm.speedup(4, 1.5, 0.1) > cm.speedup(3, 1.5, 0.1)
    assert cm.speedup(4, 1.5, 0.1) > cm.speedup(4, 2.0, 0.1)
    assert cm.speedup(4, 1.5, 0.1) > cm.speedup(4, 1.5, 0.3)


def test_table_from_pass_times():
    t = cm.table({1: 10000.0, 5: 10700.0, 64: 19300.0}, accepted=(2, 4), draft_costs=(0.0, 0.5))
    assert t["t_over_t1"] == {"5": 1.07, "64": 1.93}
    assert t["speedup"]["5"][0] == [round(2 / 1.07, 3), round(4 / 1.07, 3)]
    assert t["speedup"]["64"][1] == [round(2 / 2.43, 3), round(4 / 2.43, 3)]
    assert t["break_even_accepted"]["64"] == [1.93, 2.43]
    # string keys (as in the bench JSON) work too
    assert cm.table({"1": 1.0, "5": 2.0})["t_over_t1"] == {"5": 2.0}


def test_rejects_nonsense():
    with pytest.raises(ValueError):
        cm.speedup(1, 0.0, 0.0)
    with pytest.raises(ValueError):
        cm.speedup(-1, 1.0, 0.0)
