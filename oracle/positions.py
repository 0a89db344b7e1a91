"""Global token positions of the rows one simulated device holds (oracle side).

Test infrastructure only; see the package docstring.

* Contiguous: device r of n holds tokens [r*c, (r+1)*c) — the naive split of
  the sequence into n equal blocks ("Ring Attention vs tensor parallelism",
  standard answer: 128K over 8 cards is 16K per card; lecture 30, section 3.2
  walk-through: GPU i holds Q_i, K_i, V_i).
* Zigzag: the sequence is cut into 2n chunks of g = c/2 tokens and device r
  holds chunk r followed by chunk 2n-1-r ("Ring Attention and Sequence
  Parallelism", section 4 item 2, which names segments i and n-1-i; with n
  segments that would give each segment to two devices, so the reading taken
  is 2n chunks — the 8-device workload names chunks i and 15-i).
* Striped: token t goes to device t mod n (lecture 30, section 3.2, which
  describes GPU 0 holding tokens 0, 4, 8, ... with 4 GPUs).
"""
from __future__ import annotations

import numpy as np


def device_positions(partition: str, world: int, rank: int, local_len: int) -> np.ndarray:
    """Global positions (int64) of the local rows of device ``rank``, in local row order."""
    if not (0 <= rank < world):
        raise ValueError("rank out of range")
    c = int(local_len)
    if partition == "contiguous":
        return np.arange(rank * c, (rank + 1) * c, dtype=np.int64)
    if partition == "zigzag":
        if c % 2:
            raise ValueError("zigzag needs an even local length")
        g = c // 2
        first = np.arange(rank * g, (rank + 1) * g, dtype=np.int64)
        mirror = 2 * world - 1 - rank
        second = np.arange(mirror * g, (mirror + 1) * g, dtype=np.int64)
        return np.concatenate([first, second])
    if partition == "striped":
        return np.arange(c, dtype=np.int64) * world + rank
    raise ValueError(f"unknown partition {partition!r}")


def partition_table(partition: str, world: int, local_len: int) -> np.ndarray:
    """[world, local_len] table of positions: row r is device r's local rows."""
    return np.stack([device_positions(partition, world, r, local_len) for r in range(world)])
