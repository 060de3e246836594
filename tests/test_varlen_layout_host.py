"""The per-side storage helper the GPU addressing tests use (tests/
varlen_layout.py), pinned on hand-worked placements: start rows, rooms,
arrays, and scatter / gather as inverses on the used rows."""
import numpy as np
import torch

from varlen_layout import LEN_ARRAY, LEN_CUMSUM, LEN_UNIFORM, POS_ARRAY, POS_CUMSUM, POS_UNIFORM, ST, gather, \
    scatter, side_layout


def test_start_array_reverse_order_with_gaps():
    s = side_layout(ST | LEN_ARRAY | POS_ARRAY, [2, 0, 3], gap=3)
    # sequence 2 first at row 3, then (after a 3-row gap) the empty sequence 1
    # at row 9, then sequence 0 at row 12; 3 unused rows at the end
    assert s.starts == [12, 9, 3] and s.total == 17
    assert list(s.start) == [12, 9, 3] and list(s.used) == [2, 0, 3]
    assert s.cu is None and s.rooms == [None, None, None]
    assert list(s.rows(0)) == [12, 13] and list(s.rows(2)) == [3, 4, 5]
    assert len(s.room_rows(0)) == 0


def test_cumulative_rooms_with_used_lengths():
    s = side_layout(ST | LEN_ARRAY | POS_CUMSUM, [2, 1], rooms=[4, 2])
    assert list(s.cu) == [0, 4, 6] and s.starts == [0, 4] and s.total == 6
    assert list(s.used) == [2, 1] and s.rooms == [4, 2]
    assert list(s.room_rows(0)) == [2, 3] and list(s.room_rows(1)) == [5]
    t = side_layout(ST | LEN_CUMSUM | POS_CUMSUM, [2, 1])
    assert list(t.cu) == [0, 2, 3] and t.used is None and t.rooms == [2, 1]


def test_uniform_rooms():
    p = side_layout(LEN_ARRAY, [1, 3], rooms=[3, 3])
    assert p.S == 3 and p.starts == [0, 0] and not p.stacked and p.rooms == [3, 3]
    assert list(p.rows(1)) == [0, 1, 2] and list(p.room_rows(0)) == [1, 2]
    u = side_layout(ST | LEN_UNIFORM | POS_UNIFORM, [5, 5])
    assert u.S == 5 and u.starts == [0, 5] and u.total == 10 and u.cu is None and u.used is None
    c = side_layout(ST | LEN_CUMSUM | POS_UNIFORM, [2, 4])
    assert c.S == 4 and c.starts == [0, 4] and list(c.cu) == [0, 2, 6] and c.rooms == [4, 4]


def test_scatter_gather_inverse():
    rng = np.random.default_rng(0)
    lens = [3, 0, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    compact = torch.from_numpy(rng.standard_normal((int(cu[-1]), 2, 4))).float()
    for mode, rooms in ((ST | LEN_ARRAY | POS_ARRAY, None), (ST | LEN_ARRAY | POS_CUMSUM, [4, 2, 6]),
                        (LEN_ARRAY, [6, 6, 6]), (ST | LEN_CUMSUM | POS_UNIFORM, None)):
        s = side_layout(mode, lens, rooms)
        stored = scatter(compact, cu, s, 2)
        assert torch.equal(gather(stored, s), compact)
        # exactly the used rows hold values
        assert int((~torch.isnan(stored)).sum()) == compact.numel()
