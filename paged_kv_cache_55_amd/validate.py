"""Opt-in host check of the device-value contracts of the C ABI.

The library does not read device-resident lengths or table entries on the
host (that would need a synchronisation). This validator checks, on host
copies, the conditions the kernels rely on:
  * 0 <= seq_lens[b] <= MB * block_size;
  * every table entry a sequence uses is a block id in [0, NB);
  * write slots are distinct, and non-negative ones are < NB * block_size;
  * copy pairs name blocks in [0, NB), destinations are distinct, and no
    destination is also a source in the same call;
  * for the fused decode step (``append_rows=True``): slot_mapping[b] is
    negative or the slot of position seq_lens[b] - 1 of row b.
It raises ValueError on the first violation.
"""

from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


def _host(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy()
    return np.asarray(x)


def validate(num_blocks, block_tables=None, seq_lens=None, slot_mapping=None,
             block_mapping=None, append_rows=False, block_size=BLOCK_SIZE) -> None:
    nb = int(num_blocks)
    bsz = int(block_size)
    if block_tables is not None or seq_lens is not None:
        bt = _host(block_tables)
        lens = _host(seq_lens).astype(np.int64)
        if bt.ndim != 2 or lens.shape != (bt.shape[0],):
            raise ValueError("block_tables must be [B, MB] and seq_lens [B]")
        mb = bt.shape[1]
        if (lens < 0).any() or (lens > mb * bsz).any():
            raise ValueError("seq_lens out of [0, MB * block_size]")
        for b, L in enumerate(lens.tolist()):
            used = bt[b, :-(-L // bsz)] if L else bt[b, :0]
            if used.size and ((used < 0).any() or (used >= nb).any()):
                raise ValueError(f"sequence {b}: table entry out of [0, {nb})")
    if slot_mapping is not None:
        s = _host(slot_mapping).astype(np.int64)
        live = s[s >= 0]
        if (live >= nb * bsz).any():
            raise ValueError("slot out of range")
        if len(np.unique(live)) != len(live):
            raise ValueError("duplicate write slots race")
    if append_rows:
        bt = _host(block_tables)
        lens = _host(seq_lens).astype(np.int64)
        s = _host(slot_mapping).astype(np.int64)
        if s.shape != lens.shape:
            raise ValueError("the fused step takes one slot per row")
        for b, (slot, L) in enumerate(zip(s.tolist(), lens.tolist())):
            if slot < 0:
                continue
            if L == 0:
                raise ValueError(f"row {b}: padded row appends a token")
            pos = L - 1
            want = int(bt[b, pos // bsz]) * bsz + pos % bsz
            if slot != want:
                raise ValueError(f"row {b}: slot {slot} is not the slot of position {pos}")
    if block_mapping is not None:
        m = _host(block_mapping).astype(np.int64).reshape(-1, 2)
        if m.size and ((m < 0).any() or (m >= nb).any()):
            raise ValueError("copy pair names a block out of range")
        src, dst = m[:, 0], m[:, 1]
        if len(np.unique(dst)) != len(dst):
            raise ValueError("duplicate copy destinations race")
        if np.intersect1d(src, dst).size:
            raise ValueError("a copy destination is also a source")
