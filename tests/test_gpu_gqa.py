"""GPU parity of grouped-query decode: with G = q_heads / kv_heads > 1 query
heads per KV head, one workgroup serves all G heads and reads the KV head's
packed planes once, the logits and value sums running on matrix cores.
Every query head must match the fp64 oracle on its KV head's slice (1e-3
relative L2, 2e-3 max-abs), for group ratios 2 to 16 (3 leaves MFMA columns
idle), every head_dim, the residual, direct and chained modes, ragged rows
and a paged pool."""
import numpy as np
import pytest
import torch

from decode_attention_int4_amd import rq
from decode_attention_int4_amd.synth import Workload
from decode_attention_int4_amd.workload import RQDecode
from tests.gpu_common import assert_close_attention, bits16, encode_kept, oracle_attention, say

pytestmark = pytest.mark.gpu

CASES = [
    # d, kv heads, query heads, mode, tokens
    (128, 2, 8, 0, 333),
    (128, 1, 16, 0, 200),
    (128, 2, 6, 0, 150),
    (96, 2, 8, 0, 300),
    (64, 3, 6, 0, 257),
    (128, 2, 16, 1, 190),
    (64, 2, 8, 1, 100),
    (128, 2, 8, 2, 222),
    # long enough for several splits per (row, KV head), so the partial states
    # of more than 8 heads pass through the workspace and the final merge
    (128, 1, 16, 0, 2100),
    (128, 1, 12, 0, 1500),
]


@pytest.mark.parametrize("d,kvh,hq,mode,n", CASES,
                         ids=[f"d{c[0]}-g{c[2] // c[1]}-mode{c[3]}-n{c[4]}" for c in CASES])
def test_grouped_query_heads(d, kvh, hq, mode, n):
    w = Workload(f"gqa_d{d}_{kvh}x{hq // kvh}_m{mode}", batch=2, loops=4, layers=1, kv_heads=kvh,
                 q_heads=hq, head_dim=d, n_tokens=n, seed=d + hq + mode, mode=mode)
    G = hq // kvh
    keep = [(1, 0, kvh - 1), (0, 0, 0)]
    say(f"[gqa] {w.name}")
    run = RQDecode(w, keep=keep, chunk_tokens=128)
    run.step()
    torch.cuda.synchronize()
    out = run.out.cpu().numpy()
    for key in keep:
        b, layer, head = key
        ek, ev, HK, HV = encode_kept(w, run.kept[key], layer)
        for loop in range(w.loops):
            for h in range(head * G, (head + 1) * G):
                ref = oracle_attention(w, ek, ev, HK, HV, bits16(run.q[loop, layer, b, h]), loop, n)
                assert_close_attention(out[loop, layer, b, h], ref, f"{w.name} loop {loop} head {h}")


def test_grouped_query_ragged_and_lengths():
    """Per-row lengths through the grouped kernel, with a row of length 0 and a
    row shorter than one split."""
    w = Workload("gqa_ragged", batch=3, loops=4, layers=1, kv_heads=2, q_heads=8, head_dim=128,
                 n_tokens=700, seed=3)
    keep = [(b, 0, h) for b in range(3) for h in range(2)]
    run = RQDecode(w, keep=keep, chunk_tokens=256)
    lengths = torch.tensor([700, 37, 0], dtype=torch.int32, device="cuda")
    ws = rq.alloc_workspace(rq.decode_workspace_bytes(run.desc, w.q_heads, 700))
    enc = {k: encode_kept(w, run.kept[k], 0) for k in keep}
    for loop in range(w.loops):
        out = rq.decode_attention_ragged(run.desc, run.cache, run.signs, loop, 0, run.q[loop, 0],
                                         lengths, 700, w.softmax_scale, ws).cpu().numpy()
        for (b, layer, head) in keep:
            n = int(lengths[b])
            for h in range(4 * head, 4 * head + 4):
                if n == 0:
                    assert np.all(out[b, h] == 0)
                    continue
                ek, ev, HK, HV = enc[(b, layer, head)]
                ref = oracle_attention(w, ek, ev, HK, HV, bits16(run.q[loop, 0, b, h]), loop, n)
                assert_close_attention(out[b, h], ref, f"ragged gqa row {b} n {n} loop {loop} head {h}")


def test_grouped_query_paged_equals_contiguous():
    """The grouped kernel over a paged pool gives the outputs of the
    contiguous cache holding the same tokens, up to fp32 summation order (the
    waves claim their tiles dynamically, so the order in which a wave sums
    its tiles varies from call to call)."""
    base = Workload("gqa_paged", batch=2, loops=4, layers=1, kv_heads=2, q_heads=8, head_dim=128,
                    n_tokens=300, seed=4)
    run = RQDecode(base, chunk_tokens=300)
    paged = RQDecode(base.with_(page_tokens=32), chunk_tokens=300)
    run.step()
    paged.step()
    torch.cuda.synchronize()
    a, b = run.out.double(), paged.out.double()
    rel = ((a - b).norm() / a.norm()).item()
    assert rel < 1e-6, rel
    assert (a - b).abs().max().item() < 1e-5


@pytest.mark.parametrize("hq", [2, 8])
def test_queries_with_extreme_group_sums(hq):
    """Queries whose 16-element group sums reach 16 x their largest element
    (all elements equal and positive), one dominant element, and mixed signs
    around a large offset: every query head still matches the oracle (the
    grouped kernel holds such sums in fp16 only after a power-of-two scale)."""
    w = Workload(f"gqa_extreme_{hq}", batch=1, loops=4, layers=1, kv_heads=2, q_heads=hq,
                 head_dim=128, n_tokens=200, seed=21)
    keep = [(0, 0, 0), (0, 0, 1)]
    run = RQDecode(w, keep=keep, chunk_tokens=200)
    d = w.head_dim
    patterns = [torch.ones(d), torch.full((d,), -3.0), torch.zeros(d).index_fill_(0, torch.tensor([5]), 40.0),
                2.0 + 0.01 * torch.arange(d, dtype=torch.float32)]
    for h in range(hq):
        run.q[:, :, :, h] = patterns[h % len(patterns)].to(torch.bfloat16).cuda()
    run.step()
    torch.cuda.synchronize()
    out = run.out.cpu().numpy()
    assert np.isfinite(out).all()
    G = hq // 2
    for key in keep:
        b, layer, head = key
        ek, ev, HK, HV = encode_kept(w, run.kept[key], layer)
        for loop in range(w.loops):
            for h in range(head * G, (head + 1) * G):
                ref = oracle_attention(w, ek, ev, HK, HV, bits16(run.q[loop, layer, b, h]), loop, 200)
                assert_close_attention(out[loop, layer, b, h], ref, f"{w.name} loop {loop} head {h}")
