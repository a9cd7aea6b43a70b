"""The per-dtype forward bars (bars.py) on the CPU: the formula 2 u max|V|, the cap at the stated bar,
the float32 bar and the dtype taken from the tensor."""
import torch

from bars import LSE_BAR, STATED_LSE, STATED_O, o_bar


def test_o_bar_formula_cap_and_dtypes():
    v = torch.tensor([[-4.0, 1.0], [0.5, 2.0]])
    assert abs(o_bar("f16", v) - (2 * 2.0 ** -11 * 4.0 + 1e-5)) < 1e-12
    assert o_bar("bf16", v) == STATED_O  # 2 * 2^-8 * 4 = 3.1e-2 is looser than the stated bar
    assert abs(o_bar("bf16", v / 8) - (2 * 2.0 ** -8 * 0.5 + 1e-5)) < 1e-12
    assert o_bar("f32", v) == 1e-4
    assert o_bar(None, v.to(torch.float16)) == o_bar("f16", v)
    assert o_bar(None, v.to(torch.bfloat16)) == o_bar("bf16", v)
    assert o_bar("f16", torch.zeros(0)) == 1e-5
    assert LSE_BAR < STATED_LSE


def test_o_bound_is_the_uncapped_formula():
    from bars import o_bound

    v = torch.tensor([4.5, -1.0])
    assert abs(o_bound("bf16", v) - (2 * 2.0 ** -8 * 4.5 + 1e-5)) < 1e-12
    assert o_bar("bf16", v) == STATED_O < o_bound("bf16", v)
    assert o_bound("f16", v) == o_bar("f16", v)
