"""CPU oracle of the ternary quantized linear layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
library (``quantized_gemv_gemm_amd``) never imports it, and this package imports
nothing from the library: the two share no code.  Inputs come from ``synth``.

Source of the method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, the
write-up of the ternary 27B model on two RTX 5070 under vLLM TP=2.  Cited below
as [P1] with its section headings.

Every function is the plain definition, written with numpy in binary64 unless a
step is an integer decision; there is no blocking, fusion or reordering beyond
what the definition states.  Readings of points the page leaves open are marked
READING; each reading is stated where it is used.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, textbook identities, exact rational arithmetic and brute force.
"""
from .ternary import (  # noqa: F401
    GROUP,
    HBLOCK,
    sylvester_hadamard,
    rotate_exact,
    rotate_f32,
    half_block_stage,
    half_block_join,
    encode_words,
    decode_words,
    packed_size_words,
    pack_codes,
    unpack_codes,
    decompose_scales,
    int8_weight,
    quant_act_int8,
    gemv_ternary,
    gemv_ternary_q8,
    gemm_int8_acc,
    rescale,
    rel_fro,
    bf16_round,
)
