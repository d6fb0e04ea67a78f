"""CPU: the device buffers of a layout carry no query-rows x keys term.

paooo.com "RedKnot的技术原理" and "RedKnot的同类竞品对比": the fused varlen
kernel reads per-head page tables and never builds an attention mask, whose
size would be Hkv x T_q x L_k. The sizes the library asks for are checked on
a grid of query lengths T and context lengths L (one global and seven local
kv heads, D = 128):
- the attention plan grows additively in T and L: its mixed second
  difference, the signature of a T x L term, stays within twice the bound of
  the one region that depends on both, the work-item list (64-byte items, at
  most four rounds of one item per compute unit, holes of the XCD-aware
  order at most doubling the count);
- the split-KV workspace is bounded by the work-item cap (four rounds of one
  item per compute unit, one 256-row partial each), independent of T and L;
- the importance workspace is exactly one fp32 per (kv head, key).
"""
import os

import pytest

import head_aware_paged_amd as hk

pytestmark = pytest.mark.skipif(not os.path.exists(hk.LIB_PATH), reason="libsegkv.so not built")

HQ, HKV, D = 32, 8, 128
TS = [512, 4096, 32768]
LS = [8192, 131072, 1048576]


def sizes(T, L):
    d = hk.dims(1, HQ, HKV, D, 16, 2)
    m = hk.HostMeta([0, 2], [0, L], [L, T], [hk.GLOBAL] + [hk.LOCAL] * (HKV - 1), [0] + [1024] * (HKV - 1),
                    [-1] * (2 * HKV))
    return hk.segkv_plan_sizes(d, m)


def test_no_query_by_key_term():
    s = {(T, L): sizes(T, L) for T in TS for L in LS}
    slots = 256  # compute units of the part (the host default without a device)
    partial = 256 * D * 2 + 256 * 8  # bf16 O rows + fp32 (m, l) of one 256-row chunk
    for (T, L), v in s.items():
        assert v["attn_workspace_bytes"] <= 4 * slots * partial == 69206016, (T, L, v)  # the no-alloc scratch
        assert v["importance_workspace_bytes"] == HKV * (T + L) * 4
    big = s[(TS[-1], LS[-1])]
    assert big["plan_bytes"] + big["attn_workspace_bytes"] < HKV * TS[-1] * LS[-1] // 8 // 1000  # vs a 1-bit mask
    item_region = 64 * 4 * slots * 2
    for T0, T1 in zip(TS, TS[1:]):
        for L0, L1 in zip(LS, LS[1:]):
            p = lambda T, L: s[(T, L)]["plan_bytes"]
            mixed = p(T1, L1) - p(T0, L1) - p(T1, L0) + p(T0, L0)
            # a T x L term would make this grow with (T1 - T0)(L1 - L0); a
            # 1-bit mask's share of it is Hkv (T1 - T0)(L1 - L0) / 8 bytes
            assert abs(mixed) <= 2 * item_region, (T0, T1, L0, L1, mixed)
            assert 2 * item_region * 1000 < HKV * (T1 - T0) * (L1 - L0) // 8
