"""W_UV up-projection of the latent attention output, with the sigmoid gate.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows ``_v_up_proj`` on the ``vllm.models.kimi_k3.nvidia.mla`` page: the
[T, H, 512] latent output, viewed per head, times ``W_UV`` (the (N, L, V) =
[H, 512, 128] weight ``process_weights_after_loading`` splits out of
``kv_b_proj``), then the layer's ``_gate_sigmoid_mul(attn_out, gate)`` with
the g_proj output ``gate`` [T, H * 128].  Reading taken: the gate multiplies by the logistic sigmoid elementwise, column
``128 h + v`` of the gate belonging to head h, value v.  Computed in float64
on the bf16 inputs (a per-head matrix product serves as the step).
"""

import numpy as np

from .records import bf16_bits_to_f32

V_HEAD_DIM = 128


def v_up_proj(latent_bits, w_uv_bits, gate_bits=None):
    """float64 [T, H, 128] = latent[t, h, :512] @ W_UV[h] (* sigmoid(gate)).

    latent_bits uint16 [T, H, 512]; w_uv_bits uint16 [H, 512, 128];
    gate_bits uint16 [T, H * 128] or None.
    """
    x = bf16_bits_to_f32(latent_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_uv_bits).astype(np.float64)
    t, h = x.shape[0], x.shape[1]
    y = np.matmul(x.transpose(1, 0, 2), w).transpose(1, 0, 2)  # per head: [T, 512] @ [512, 128]
    if gate_bits is not None:
        g = bf16_bits_to_f32(gate_bits).astype(np.float64).reshape(t, h, V_HEAD_DIM)
        y = y * (1.0 / (1.0 + np.exp(-g)))
    return y
