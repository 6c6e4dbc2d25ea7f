"""GPU parity at long contexts and with many token splits, against the fp64
oracle on sampled slices (every loop of each slice):

  * split merges over more than 16 splits (merged in rounds of 16), at
    head_dim 64, 96 and 128 with few (batch row, head) pairs;
  * balanced split plans, where some rows take one split fewer than the
    others so that the grid fills its workgroup target;
  * 64k and 128k tokens with 8-16 splits per row, and single-split calls
    (a whole row per workgroup) at 32k and 128k tokens, in residual and
    direct mode: the longest accumulation per lane.

The decode kernel's value sums carry the magic-number constant (1024 per
unit weight) that the code unpack adds; it is folded out every few tiles,
so rounding does not grow with the tokens a lane sums.  Each case prints its
worst relative L2 error."""
import gc

import numpy as np
import pytest
import torch

from decode_attention_int4_amd import rq
from decode_attention_int4_amd.synth import Workload
from decode_attention_int4_amd.workload import RQDecode
from tests.gpu_common import (assert_close_attention, bits16, check_slice_planes, oracle_attention,
                              POOL, say)

pytestmark = pytest.mark.gpu


def _run(w, keep, expect_splits=None, check_planes=True):
    say(f"[longctx] {w.name}: fill {w.n_tokens} tokens, batch {w.batch}")
    run = RQDecode(w, keep=keep)
    torch.cuda.synchronize()
    splits = {loop: rq.decode_splits(run.desc, loop, w.q_heads, run.N) for loop in range(w.loops)}
    if expect_splits is not None:
        cmp, n = expect_splits
        assert all(cmp(s, n) for s in splits.values()), f"split plan {splits}"
    out = {}
    for loop in range(w.loops):
        out[loop] = run.attend(loop, 0).cpu().numpy()
    worst = 0.0
    for key in keep:
        b, layer, head = key
        if check_planes:
            from tests.gpu_common import encode_kept
            ek, ev, HK, HV = check_slice_planes(w, run, key)
        else:
            from tests.gpu_common import encode_kept
            ek, ev, HK, HV = encode_kept(w, run.kept[key], layer)
        futs = {loop: POOL.submit(oracle_attention, w, ek, ev, HK, HV,
                                  bits16(run.q[loop, layer, b, head]), loop, run.N)
                for loop in range(w.loops)}
        for loop, f in futs.items():
            rel, _ = assert_close_attention(out[loop][b, head], f.result(),
                                            f"{w.name} slice {key} loop {loop}")
            worst = max(worst, rel)
    say(f"[longctx] {w.name}: splits {sorted(set(splits.values()))}, worst rel-L2 {worst:.2e}")
    del run
    gc.collect()
    torch.cuda.empty_cache()
    return worst


MANY = {
    # (d, batch, heads, tokens): fewer (row, head) pairs than the grid's workgroups
    "splits_d64": (64, 1, 2, 8192),
    "splits_d96": (96, 1, 4, 8192),
    "splits_d128": (128, 1, 2, 8192),
}


@pytest.mark.parametrize("name", list(MANY))
def test_many_splits(name):
    d, batch, heads, n = MANY[name]
    w = Workload(name, batch=batch, loops=4, layers=1, kv_heads=heads, q_heads=heads, head_dim=d,
                 n_tokens=n, seed=d + 1)
    _run(w, [(0, 0, heads - 1)], expect_splits=(lambda s, k: s > k, 16))


BALANCED = {
    # (d, batch, heads, tokens, rows_lo, splits): four-wave calls whose rows do
    # not divide the workgroup target; the first rows_lo rows take one split
    # fewer than the others
    "balanced_d96": (96, 2, 55, 8192, 2, 7),    # 110 rows, 768 target: 2 x 6 + 108 x 7
    "balanced_d64": (64, 4, 25, 8192, 88, 6),   # 100 rows, 512 target: 88 x 5 + 12 x 6
}


@pytest.mark.parametrize("name", list(BALANCED))
def test_balanced_plan(name):
    """Rows on both sides of the boundary between the two split counts, and
    the last row, match the oracle in every loop."""
    d, batch, heads, n, rows_lo, hi = BALANCED[name]
    w = Workload(name, batch=batch, loops=4, layers=1, kv_heads=heads, q_heads=heads, head_dim=d,
                 n_tokens=n, seed=d + 3)
    rows = [rows_lo - 1, rows_lo, batch * heads - 1]
    keep = [(r // heads, 0, r % heads) for r in rows]
    _run(w, keep, expect_splits=(lambda s, k: s == k, hi))


LONG = {
    # name: (batch, tokens, mode, expected splits: (compare, value))
    "ctx64k_b1": (1, 65536, 0, (lambda s, k: s >= k, 8)),
    "ctx128k_b2": (2, 131072, 0, (lambda s, k: s >= k, 4)),
    "ctx128k_b2_direct": (2, 131072, 1, (lambda s, k: s >= k, 4)),
    "ctx32k_b16_one_split": (16, 32768, 0, (lambda s, k: s == k, 1)),
    "ctx128k_b16_one_split": (16, 131072, 0, (lambda s, k: s == k, 1)),
    "ctx128k_b16_one_split_direct": (16, 131072, 1, (lambda s, k: s == k, 1)),
}


@pytest.mark.parametrize("name", list(LONG))
def test_long_context(name):
    batch, n, mode, splits = LONG[name]
    w = Workload(name, batch=batch, loops=4, layers=1, kv_heads=16, q_heads=16, head_dim=128,
                 n_tokens=n, seed=7, mode=mode)
    free, _ = torch.cuda.mem_get_info()
    need = 1.2 * batch * n * 16 * 940 + 6e9
    if free < need:
        pytest.skip(f"needs {need / 1e9:.0f} GB free, have {free / 1e9:.0f} GB")
    _run(w, [(batch - 1, 0, 5)], expect_splits=splits, check_planes=(n <= 65536))
