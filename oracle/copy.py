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


def resize_slots(slot_banks, src, fill: int = 0xA5):
    """Slot banks after a pool resize (see SlotTable.resize): new slot i takes the
    bytes of old slot src[i]; a new empty slot (src[i] = -1) holds `fill` here,
    standing for bytes that no step reads before a copy writes them.
    Returns new arrays; the inputs are not changed."""
    out = []
    for bank in slot_banks:
        new = np.full((len(src), bank.shape[1]), fill, dtype=np.uint8)
        for i, s in enumerate(src):
            if s >= 0:
                new[i, :] = bank[s]
        out.append(new)
    return out
