"""Closed form for the materialised attention-matrix memory.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[HF] "¿Por qué la paralelización de secuencias?": a standard (materialising)
attention needs sequence_length x sequence_length weights of 2 bytes each in
bf16, per head; at a 128k sequence that is about 32 GB per head.  Chunked
attention never allocates this matrix.
"""


def attn_matrix_bytes(L: int, heads: int = 1, elem_bytes: int = 2) -> int:
    return L * L * elem_bytes * heads
