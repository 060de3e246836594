"""Per-side storage of a packed problem under the ATTN_VARLEN modes (test
helper, no attention arithmetic): where each sequence's rows sit in a padded
or stacked tensor, which arrays the mode reads, and the scatter of compact
packed rows into that storage (every other row NaN)."""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

ST = 0x01
LEN_UNIFORM, LEN_CUMSUM, LEN_ARRAY = 0x00, 0x02, 0x04
POS_UNIFORM, POS_CUMSUM, POS_ARRAY = 0x00, 0x08, 0x10


@dataclasses.dataclass
class SideLayout:
    """One side: mode byte, lengths, and the storage rows of each sequence."""
    mode: int
    lens: List[int]              # rows each sequence uses
    rooms: List[Optional[int]]   # rows each sequence owns (None: not known)
    S: int                       # seqlen field (uniform length / room, or the largest length)
    starts: List[int]            # storage row of local row 0 (padded: 0 within its batch entry)
    total: int                   # stacked: rows of the tensor
    cu: Optional[np.ndarray]     # int32 [B+1] when the mode reads it
    used: Optional[np.ndarray]   # int32 [B] when the mode reads it
    start: Optional[np.ndarray]  # int32 [B] when the mode reads it

    @property
    def stacked(self) -> bool:
        return bool(self.mode & ST)

    def rows(self, b: int) -> np.ndarray:
        """Storage rows of sequence b's used rows (stacked: tensor rows;
        padded: rows inside batch entry b)."""
        return self.starts[b] + np.arange(self.lens[b])

    def room_rows(self, b: int) -> np.ndarray:
        """Storage rows of sequence b's room past its length."""
        if self.rooms[b] is None:
            return np.zeros(0, dtype=np.int64)
        return self.starts[b] + np.arange(self.lens[b], self.rooms[b])


def side_layout(mode: int, lens: List[int], rooms: Optional[List[int]] = None, gap: int = 3) -> SideLayout:
    """Storage for sequences of `lens` rows under `mode`.  `rooms` (>= lens)
    sets the room of each sequence where the mode keeps one (padded and
    uniform starts use max(rooms) for every sequence); with POS_ARRAY the
    sequences are stored in reverse order with `gap` unused rows between
    them."""
    B = len(lens)
    lens = [int(x) for x in lens]
    rooms = list(lens) if rooms is None else [int(x) for x in rooms]
    assert all(r >= n for r, n in zip(rooms, lens))
    ls, ps = (mode >> 1) & 3, (mode >> 3) & 3
    stacked = bool(mode & ST)
    cu = used = start = None
    if not stacked or ps == 0:  # uniform room S
        S = max(rooms + [0]) if ls != 0 else max(lens + [0])
        if ls == 0:
            lens = [S] * B
        rooms_out: List[Optional[int]] = [S] * B
        starts = [b * S for b in range(B)] if stacked else [0] * B
        total = B * S if stacked else 0
        if ls == 1:
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    elif ps == 1:  # cumulative starts: the room is the cu range
        if ls == 1:
            rooms = list(lens)
        cu = np.concatenate([[0], np.cumsum(rooms)]).astype(np.int32)
        rooms_out = list(rooms)
        starts = [int(x) for x in cu[:-1]]
        total = int(cu[-1])
        S = max(lens + [0]) if ls != 0 else max(rooms + [0])
        if ls == 0:
            lens = [S] * B
            assert all(r >= S for r in rooms), "uniform lengths need rooms of at least S"
    else:  # start array: sequences stored in reverse order with gaps
        S = max(lens + [0])
        if ls == 0:
            lens = [S] * B
        if ls == 1:
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        starts = [0] * B
        row = gap
        for b in reversed(range(B)):
            starts[b] = row
            row += lens[b] + gap
        total = row
        rooms_out = [None] * B
        start = np.asarray(starts, dtype=np.int32)
    if ls == 2:
        used = np.asarray(lens, dtype=np.int32)
    return SideLayout(mode, lens, rooms_out, S, starts, total, cu, used, start)


def scatter(compact: torch.Tensor, cu_compact: np.ndarray, side: SideLayout, heads: int) -> torch.Tensor:
    """The compact packed [T, H, D] rows placed into the side's storage
    ([total, H, D] stacked, [B, H, S, D] padded); every other row NaN."""
    D = compact.shape[-1]
    B = len(side.lens)
    if side.stacked:
        out = torch.full((side.total, heads, D), float("nan"), dtype=compact.dtype)
        for b in range(B):
            out[torch.from_numpy(side.rows(b))] = compact[int(cu_compact[b]):int(cu_compact[b + 1])]
    else:
        out = torch.full((B, heads, side.S, D), float("nan"), dtype=compact.dtype)
        for b in range(B):
            out[b, :, torch.from_numpy(side.rows(b))] = compact[int(cu_compact[b]):int(cu_compact[b + 1])].transpose(0, 1)
    return out


def gather(stored: torch.Tensor, side: SideLayout) -> torch.Tensor:
    """The used rows of every sequence, back in compact packed [T, H, D]
    order (inverse of scatter on those rows)."""
    parts = []
    for b in range(len(side.lens)):
        r = torch.from_numpy(side.rows(b))
        parts.append(stored[r] if side.stacked else stored[b, :, r].transpose(0, 1))
    return torch.cat(parts, 0) if parts else stored.reshape(0, *stored.shape[-2:])
