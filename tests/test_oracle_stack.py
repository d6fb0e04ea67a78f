"""CPU: the elastic-stack oracle pinned to things other than itself.

1. Zero output and down projections make every layer the identity.
2. A deep layer chooses the rows a pure-Python sort by (-importance, row)
   picks from the query slice of the (pinned) importance vector, and a
   shallow layer chooses every row.
3. A one-layer deep stack with k = every row equals the (pinned) layer glue
   followed by the dense SwiGLU FFN written with torch on every row.
4. The shallow layout with a window covering the whole context gives the same
   result as an all-global class map.
"""
import dataclasses

import numpy as np
import torch

import oracle
import workloads


def _layers(n, hidden=128, inter=256, seed=0):
    ws = [workloads.tiny(seed=100 + i) for i in range(n)]
    h, wts = workloads.stack_inputs(ws[0], n, hidden, inter, seed=seed)
    return h, list(zip(ws, wts))


def test_zero_projections_are_identity():
    h, layers = _layers(3)
    for _, wt in layers:
        wt["w_o"][:] = 0
        wt["w_down"][:] = 0
    out, _, _ = oracle.stack(layers, h, n_shallow=1, shallow_window=16, k=8, n_last=16)
    assert np.array_equal(out, oracle.bf16_bits_to_f64(h))


def test_selection_rule():
    h, layers = _layers(3, seed=1)
    _, chosen, imps = oracle.stack(layers, h, n_shallow=1, shallow_window=16, k=8, n_last=16)
    assert np.array_equal(chosen[0], np.arange(32))
    for idx, imp in zip(chosen[1:], imps[1:]):
        order = sorted(range(len(imp)), key=lambda j: (-imp[j], j))[:8]
        assert list(idx) == sorted(order)


def test_dense_ffn_on_every_row():
    h, layers = _layers(1, seed=2)
    out, chosen, _ = oracle.stack(layers, h, n_shallow=0, shallow_window=16, k=32, n_last=16)
    assert np.array_equal(chosen[0], np.arange(32))
    w, wt = layers[0]
    o, _ = oracle.layer(w, h, wt["w_qkv"], wt["w_o"])
    x = torch.from_numpy(oracle.round_bf16(o))
    f = lambda a: torch.from_numpy(oracle.bf16_bits_to_f64(a))
    act = torch.nn.functional.silu(x @ f(wt["w_gate"]).T) * (x @ f(wt["w_up"]).T)
    ref = x + torch.from_numpy(oracle.round_bf16(act.numpy())) @ f(wt["w_down"]).T
    assert np.allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_wide_shallow_window_equals_global():
    h, layers = _layers(2, seed=3)
    out1, _, _ = oracle.stack(layers, h, n_shallow=2, shallow_window=1 << 20, k=8, n_last=16)
    glob = [(dataclasses.replace(w, head_class=np.zeros_like(w.head_class)), wt) for w, wt in layers]
    out2, _, _ = oracle.stack(glob, h, n_shallow=0, shallow_window=16, k=32, n_last=16)
    assert np.allclose(out1, out2, rtol=0, atol=1e-12)
