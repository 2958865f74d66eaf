"""The persistent grids with workgroups that run several tiles, every output compared with the
fp64 oracle.  The preparation kernel keeps two workgroups per CU, each walking chunks with the
next chunk's q, k and g loaded while the current one is computed; GSA's pass-1 backward keeps
one per CU and carries its next tile's gates and dZ.  With 720 chunk tiles some workgroups run
one tile and others two or three, and the last round's loads are the harmless repeats of a
tile's first row."""
import pytest

import workloads as W
from tests.test_gla_bwd_gpu import check_bwd
from tests.test_gla_fwd_gpu import check_fwd
from tests.test_gsa_gpu import check_gsa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_gla_amd as m
    m.lib()
    return m


def test_gla_tiles_past_one_round(gla):
    # N = 24 chunks (the last ragged) x 30 sequences = 720 tiles
    w = W.GlaWorkload("persist-gla", 6, 5, 64 * 23 + 17, 64, 64, 64, "bf16", 911, h0=True, gate_law="iid")
    x = W.gla_inputs(w)
    check_fwd(gla, w, x)
    check_bwd(gla, w, x)


@pytest.mark.parametrize("saved", [False, True])
def test_gsa_tiles_past_one_round(gla, saved):
    w = W.GsaWorkload("persist-gsa", 6, 5, 64 * 23 + 17, 64, 64, 32, 64, "bf16", 912, h0=True)
    check_gsa(gla, w, W.gsa_inputs(w), saved=saved)
