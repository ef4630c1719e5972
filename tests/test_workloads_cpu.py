"""The seeded input helpers of the position-order tests: the within-segment shuffle keeps every token
in its own segment and moves the position ids with the tokens."""
import torch

import workloads


def test_position_ids_restart_per_segment():
    pos = workloads.position_ids([3, 1, 4])
    assert pos.dtype == torch.int32
    assert pos.tolist() == [0, 1, 2, 0, 0, 1, 2, 3]
    assert workloads.position_ids([]).numel() == 0


def test_shuffle_stays_within_segments_and_is_seeded():
    lens = [300, 129, 1, 64]
    seg = workloads.segment_ids(lens)
    p = workloads.shuffle_within_segments(lens, 5)
    assert sorted(p.tolist()) == list(range(sum(lens)))
    assert torch.equal(seg[p], seg)                      # nobody leaves their segment
    assert not torch.equal(p, torch.arange(sum(lens)))   # and it is a real shuffle
    assert torch.equal(p, workloads.shuffle_within_segments(lens, 5))
    pos = workloads.position_ids(lens)[p]
    t0 = 0
    for L in lens:                                       # each segment's ids stay a permutation of 0..L-1
        assert sorted(pos[t0:t0 + L].tolist()) == list(range(L))
        t0 += L
