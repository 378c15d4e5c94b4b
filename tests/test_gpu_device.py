"""gdn2_device_info: the part's compute-unit count and peak clock, which the
benchmark states beside the published peaks."""

import pytest

import gated_delta_rule_47_amd as g

pytestmark = pytest.mark.gpu


def test_device_info_matches_runtime():
    import torch
    cus, khz = g.device_info(0)
    assert cus == torch.cuda.get_device_properties(0).multi_processor_count
    assert 500_000 <= khz <= 5_000_000  # a peak engine clock between 0.5 and 5 GHz


def test_device_info_bad_device_is_an_error():
    import torch
    with pytest.raises(g.Gdn2Error):
        g.device_info(torch.cuda.device_count() + 7)
