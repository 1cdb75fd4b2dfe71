"""The delayed-scaling recipe object of the binding (host logic only)."""
import pytest

import mxfp4_precision_numerics_amd as mxq


def test_default_recipe_is_the_pages_recipe():
    # FP8 guide, "Transformer Engine: a fundacao de software": margin 0,
    # HYBRID formats, history of 16 amax values reduced with max
    r = mxq.DelayedScaling()
    assert (r.margin, r.fmt, r.amax_history_len, r.amax_compute_algo) == (0, mxq.HYBRID, 16, "max")
    assert r.format_for(backward=False) == mxq.E4M3
    assert r.format_for(backward=True) == mxq.E5M2


def test_single_format_recipes():
    assert mxq.DelayedScaling(fmt="E4M3").format_for(True) == mxq.E4M3
    assert mxq.DelayedScaling(fmt="E5M2").format_for(False) == mxq.E5M2


@pytest.mark.parametrize("kw", [dict(margin=1), dict(amax_compute_algo="most_recent"), dict(fmt="E2M1"),
                                dict(amax_history_len=0), dict(amax_history_len=1025)])
def test_unsupported_recipes_are_refused(kw):
    with pytest.raises(ValueError):
        mxq.DelayedScaling(**kw)
