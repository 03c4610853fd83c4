"""Per-format bank lists: one host bank per schema tensor, one row per expert.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FreeToken MoE benchmark guide §4.2 and FreeToken architecture walk-through §5:
each quantisation format declares its own bank schema; bf16 is the pair
(gate_up, down); NVFP4 is six banks (packed codes, an e4m3 scale per 16-element
block, an fp16 global per output row, for gate_up and for down); the MXFP4
format is six transposed banks (_blocks, _scales, _bias for each matrix).  The
FP8 block format (e4m3 weights with fp32 scales per 128x128 block) is listed on
the architecture page; its bank split (weights and scales as separate banks)
is the reading taken here.  GGUF Q4_0 is the fifth format the architecture page
lists; its values follow the published GGUF block_q4_0 definition (32 weights
share one fp16 scale d, weight = (q - 8) * d) and its bank split - the 4-bit
codes and the fp16 scales as separate banks, as for NVFP4 - is a reading.

Weights use the [out, in] convention: gate_up is [2I, H] and down is [H, I].
Rows [0, I) of gate_up are the gate projection, rows [I, 2I) the up
projection (a reading: the pages do not say).

Each entry is (name, element tag, row shape, row bytes).  The element tag says
how to read a row: "bf16", "e4m3", "f32", "fp4x2" (two e2m1 codes per byte),
"fp16", "e8m0", "u8", "q4x2" (GGUF Q4_0 codes: in every 16 bytes, byte j holds
element j in its low nibble and element j + 16 in its high nibble).
"""

BF16, FP8_BLOCK128, NVFP4, MXFP4_T, Q4_0 = "bf16", "fp8_block128", "nvfp4", "mxfp4_t", "q4_0"
FORMATS = (BF16, FP8_BLOCK128, NVFP4, MXFP4_T, Q4_0)

_ELEM_BYTES = {"bf16": 2, "e4m3": 1, "f32": 4, "fp16": 2, "e8m0": 1, "u8": 1}


def _bytes(elem, shape):
    n = 1
    for d in shape:
        n *= d
    if elem in ("fp4x2", "q4x2"):
        return n  # shape already counts bytes (two codes per byte)
    return n * _ELEM_BYTES[elem]


def bank_specs(fmt: str, hidden: int, inter: int):
    """Ordered bank list for one expert of the given format.

    Returns a list of (name, elem, row_shape, row_bytes).
    """
    H, I = hidden, inter
    if fmt == BF16:
        banks = [("gate_up", "bf16", (2 * I, H)), ("down", "bf16", (H, I))]
    elif fmt == FP8_BLOCK128:
        if H % 128 or I % 128:
            raise ValueError("fp8 block format needs H and I divisible by 128")
        banks = [("gate_up", "e4m3", (2 * I, H)),
                 ("gate_up_scale", "f32", (2 * I // 128, H // 128)),
                 ("down", "e4m3", (H, I)),
                 ("down_scale", "f32", (H // 128, I // 128))]
    elif fmt == NVFP4:
        if H % 16 or I % 16:
            raise ValueError("nvfp4 needs H and I divisible by 16")
        banks = [("gate_up_codes", "fp4x2", (2 * I, H // 2)),
                 ("gate_up_scale", "e4m3", (2 * I, H // 16)),
                 ("gate_up_global", "fp16", (2 * I,)),
                 ("down_codes", "fp4x2", (H, I // 2)),
                 ("down_scale", "e4m3", (H, I // 16)),
                 ("down_global", "fp16", (H,))]
    elif fmt == MXFP4_T:
        if H % 32 or I % 32:
            raise ValueError("mxfp4 needs H and I divisible by 32")
        banks = [("gate_up_blocks", "u8", (H // 32, 2 * I, 16)),
                 ("gate_up_scales", "e8m0", (H // 32, 2 * I)),
                 ("gate_up_bias", "bf16", (2 * I,)),
                 ("down_blocks", "u8", (I // 32, H, 16)),
                 ("down_scales", "e8m0", (I // 32, H)),
                 ("down_bias", "bf16", (H,))]
    elif fmt == Q4_0:
        if H % 32 or I % 32:
            raise ValueError("q4_0 needs H and I divisible by 32")
        banks = [("gate_up_q", "q4x2", (2 * I, H // 2)),
                 ("gate_up_d", "fp16", (2 * I, H // 32)),
                 ("down_q", "q4x2", (H, I // 2)),
                 ("down_d", "fp16", (H, I // 32))]
    else:
        raise ValueError(f"unknown format {fmt!r}")
    return [(name, elem, shape, _bytes(elem, shape)) for name, elem, shape in banks]


def bytes_per_expert(fmt: str, hidden: int, inter: int) -> int:
    """Sum of one expert's row bytes over every bank of the schema."""
    return sum(b[3] for b in bank_specs(fmt, hidden, inter))
