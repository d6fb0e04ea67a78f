"""GPU: segpaged_attn_prefill_noalloc (split-KV partials in the library's fixed
device scratch) against segpaged_attn_prefill (caller workspace), through the
C-ABI, on consecutive calls with shrinking inputs. Both run the same kernels
with the same plan, so out and lse must be bit-identical; the later, smaller
calls also show that the scratch left by an earlier call does not leak in."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import bits, build
from head_aware_paged_amd import segpaged_attn_prefill_noalloc

pytestmark = pytest.mark.gpu

G_, L_, R_, D_ = workloads.GLOBAL, workloads.LOCAL, workloads.RETRIEVAL, workloads.DENSE


def _cases():
    yield workloads.make("mistral7b_32k")
    yield workloads.make_custom("g4_d128_q512", Hq=16, Hkv=4, D=128, theta=1e6,
                                seg_lens_per_req=[[2048, 2048, 512]], orig_starts_per_req=[[0, 0, None]],
                                classes=[G_, L_, R_, D_], windows=[0, 1024, 0, 0], retr=[None, None, (1, 0), None])
    yield workloads.tiny(window=8)


def test_noalloc_matches_workspace_entry():
    for w in _cases():
        layer, dev = build(w)
        print(f"case {w.name}: workspace {layer.sizes['attn_workspace_bytes']} B", flush=True)
        out, lse = layer.attention(dev.q, dev.k_work, dev.v_work)
        out2 = torch.full_like(out, float("nan"))
        lse2 = torch.full_like(lse, float("nan"))
        segpaged_attn_prefill_noalloc(layer.dims, layer.meta, dev.q, dev.k_work, dev.v_work, layer.page_ids,
                                      layer.page_pos, layer.plan, layer.scale, out2, lse2)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out2), bits(out)), w.name
        assert np.array_equal(lse2.cpu().numpy().view(np.uint32), lse.cpu().numpy().view(np.uint32)), w.name
        del layer, dev, out, lse, out2, lse2
