"""Algorithmic bytes of one decode step and the HBM roofline.

A decode step at batch B reads every weight once and, for every batch row,
the K and V rows of every earlier position in every layer; the bandwidth
floor is bytes / peak bandwidth (the speed-of-light definition on the page
"Megakernels: Deleting the Kernel Boundary to Win Back Microseconds", opening
paragraph, and the Gemma TPU megakernel page's speed-of-light table).
"""
from __future__ import annotations

MI355X_HBM_PEAK_GBPS = 8000.0  # published HBM3E peak, GB/s


def weight_bytes_read(shape, batch: int, matrix_bytes: int = 2) -> int:
    """Weight bytes streamed per step: every layer matrix (matrix_bytes per element:
    2 for bf16, 1 for FP8 codes), every norm gain (bf16), the LM head (the embedding
    matrix when tied; a matrix too) and the final norm gain, plus one bf16 embedding
    row per batch row."""
    H, D = shape.hidden, shape.head_dim
    mats = (shape.n_q_heads * D * H + 2 * shape.n_kv_heads * D * H + H * shape.n_q_heads * D
            + 3 * shape.ffn * H)
    return matrix_bytes * (shape.n_layers * mats + shape.vocab * H) + 2 * (shape.n_layers * 2 * H + H + batch * H)


def kv_bytes_read(shape, batch: int, keys: float) -> float:
    """bf16 K and V bytes read per step when every row attends to `keys` positions."""
    return batch * keys * shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * 2


def step_bytes(shape, batch: int, keys: float, matrix_bytes: int = 2) -> float:
    return weight_bytes_read(shape, batch, matrix_bytes) + kv_bytes_read(shape, batch, keys)


def mean_keys(prompt: int, first_step: int, n_steps: int) -> float:
    """Average attended positions over steps first_step .. first_step+n_steps-1
    after a `prompt`-token cache: step i writes slot prompt+i and reads prompt+i+1 keys."""
    return prompt + first_step + (n_steps - 1) / 2.0 + 1.0


def floor_us(bytes_per_step: float, peak_gbps: float = MI355X_HBM_PEAK_GBPS) -> float:
    return bytes_per_step / (peak_gbps * 1e3)
