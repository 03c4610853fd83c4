"""copy_missing: gather every missing expert's rows from the host banks into its slot.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FreeToken MoE benchmark guide §4.2 and §4.4: host banks are supplied per bank
as a list of per-layer tensors; the cache is indifferent to layout and only
moves rows; for each miss, every bank contributes one contiguous row.
"""
import numpy as np


def copy_missing(misses, host_banks, slot_banks, num_experts: int):
    """Apply the miss list to the slot banks in place.

    misses      - [(slot, flat_id)] as returned by SlotTable.ensure
    host_banks  - host_banks[b][layer] is a uint8 array of shape [E, row_bytes_b]
                  (or None for a layer with no source)
    slot_banks  - slot_banks[b] is a uint8 array of shape [S, row_bytes_b]
    Returns the number of bytes moved.
    """
    moved = 0
    for slot, fid in misses:
        layer, expert = divmod(int(fid), num_experts)
        for b in range(len(slot_banks)):
            src = host_banks[b][layer]
            if src is None:
                raise ValueError(f"bank {b} has no source for layer {layer}")
            row = np.asarray(src[expert], dtype=np.uint8)
            slot_banks[b][slot, :] = row
            moved += row.size
    return moved
