"""Whole-layer streaming for prefill: a two-deep buffer of every expert of a layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FreeToken architecture walk-through §5: prefill streams whole layers through a
double buffer so that copy and compute overlap.  Layer l's E experts are
copied, in expert order (buffer row e = expert e), into buffer[l % 2] while the
FFN of the previous layer runs on the other buffer; the FFN of layer l then
reads buffer[l % 2].  This is separate from the LRU slot pool.
"""
import numpy as np

from . import ffn, route


def buffer_after_prefetch(host_banks, layer):
    """Content of the buffer that holds `layer`: per bank, the layer's whole host bank (a byte copy)."""
    return [np.array(host_banks[b][layer], dtype=np.uint8, copy=True) for b in range(len(host_banks))]


def prefill_layer(fmt, hidden, inter, x_bits, logits32, k, buffer_banks):
    """Route from given logits, then run the expert FFN with slot = expert on the layer buffer.

    Returns (ids, w, y) with y float64 [n, H].
    """
    ids, w = route.topk_softmax(logits32, k)
    y = ffn.expert_ffn(fmt, hidden, inter, x_bits, ids, w,
                       lambda e: [buffer_banks[b][e] for b in range(len(buffer_banks))])
    return ids, w, y
