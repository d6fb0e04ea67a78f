"""Token-selective (sparse) SwiGLU FFN, fp64.

Pages: paooo.com "RedKnot的主要功能" (dense FFN for the top-k tokens by
attention score, residual identity for the rest) and "RedKnot的技术原理" (FFN
and attention optimised orthogonally); RedKnot README "About" (Elastic
Sparsity / sparse FFN).

Reading: no normalisation layer; SwiGLU is silu(W_gate h) * (W_up h), and the
one declared rounding point is the bf16 activation between the two
projections (the tensor handed from the first GEMM to the second):
    out_i = h_i + W_down . bf16(silu(W_gate h_i) * (W_up h_i))   for i in idx
    out_i = h_i                                                  otherwise.
Weights are [out_features, in_features].
"""
import numpy as np

from .bf16 import bf16_bits_to_f64, round_bf16


def _silu(x):
    return x / (1.0 + np.exp(-x))


def swiglu_activation(hidden_bits, idx, w_gate_bits, w_up_bits):
    """silu(W_gate h) * (W_up h) for the rows idx, fp64, before its bf16 rounding."""
    X = bf16_bits_to_f64(hidden_bits)[np.asarray(idx, dtype=np.int64)]
    return _silu(X @ bf16_bits_to_f64(w_gate_bits).T) * (X @ bf16_bits_to_f64(w_up_bits).T)


def sparse_ffn(hidden_bits, idx, w_gate_bits, w_up_bits, w_down_bits):
    """Returns the fp64 output rows [n, hidden] (before the final bf16 store)."""
    H = bf16_bits_to_f64(hidden_bits)
    out = H.copy()
    idx = np.asarray(idx, dtype=np.int64)
    if len(idx) == 0:
        return out
    a = round_bf16(swiglu_activation(hidden_bits, idx, w_gate_bits, w_up_bits))
    out[idx] = H[idx] + a @ bf16_bits_to_f64(w_down_bits).T
    return out
