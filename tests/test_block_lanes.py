"""Host logic of the concurrent block: how calibration streams are grouped
into lanes (no GPU)."""
from post_weight_quantization_02_amd import block


class _X:
    def __init__(self, n, d):
        self.shape = (n, d)


class _Stream:
    def __init__(self, n, d):
        self.X = _X(n, d)


def test_lanes_of_the_seven_layer_block():
    # attention input, o input, MLP input (d = 4096), down input (d = 11008)
    sts = [_Stream(262144, 4096), _Stream(262144, 4096), _Stream(262144, 4096),
           _Stream(262144, 11008)]
    assert block.lane_assignment(sts, 1) == [[0, 1, 2, 3]]
    assert block.lane_assignment(sts, 2) == [[3], [0, 1, 2]]
    assert block.lane_assignment(sts, 4) == [[3], [0], [1], [2]]
    assert block.lane_assignment(sts, 9) == [[3], [0], [1], [2]]


def test_lanes_cover_every_stream_once_in_order():
    sts = [_Stream(n, d) for n, d in ((100, 64), (5000, 512), (300, 128), (5000, 512), (7, 8))]
    for lanes in range(1, 7):
        got = block.lane_assignment(sts, lanes)
        assert sorted(i for l in got for i in l) == list(range(len(sts)))
        assert all(l == sorted(l) for l in got)
        assert len(got) == min(lanes, len(sts))
