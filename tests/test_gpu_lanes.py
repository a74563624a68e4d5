"""The wave primitives the selection and attention kernels are built on (register lane
exchanges through DPP and v_permlane*_swap, wave scans and reductions) agree bit for bit with
the general shuffle forms they replace, for every check and thread (grw_selftest_lanes)."""
import pytest

import generative_recommendation_wide_amd as grw
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_wave_primitives_match_shuffles():
    say("selftest_lanes: 14 checks x 256 threads")
    assert grw.selftest_lanes() == 0
