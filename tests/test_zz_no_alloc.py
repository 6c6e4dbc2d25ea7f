"""rq_decode_attention_noalloc through the raw C ABI: the decode entry point
whose split-K partial states and counters live in the library's own device
array (for callers that cannot allocate).  Two calls in a row, the second
with a smaller input, each compared with rq_decode_attention (caller
workspace) on the same inputs to the attention bar (1e-3 relative L2, 2e-3
max-abs; the two run the same kernels and differ only in summation order), and
with the fp64 oracle; a call that would need more than the library's array is
refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from decode_attention_int4_amd import rq
from decode_attention_int4_amd.synth import Workload
from decode_attention_int4_amd.workload import RQDecode
from tests.gpu_common import (assert_close_attention, bits16, encode_kept, oracle_attention, say)

pytestmark = pytest.mark.gpu


def _noalloc(run, loop, layer, q, n, out):
    return rq.lib().rq_decode_attention_noalloc(
        ctypes.byref(run.desc), ctypes.c_void_p(run.cache.data_ptr()),
        ctypes.c_void_p(run.signs.data_ptr()), loop, layer, ctypes.c_void_p(q.data_ptr()),
        q.shape[1], n, ctypes.c_float(run.w.softmax_scale), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_entry_point():
    w = Workload("noalloc", batch=2, loops=4, layers=2, kv_heads=4, q_heads=4, head_dim=128,
                 n_tokens=3000, seed=21)
    key = (1, 1, 2)
    run = RQDecode(w, keep=[key])
    ek, ev, HK, HV = encode_kept(w, run.kept[key], key[1])
    b, layer, head = key
    for call, (loop, n) in enumerate(((0, 3000), (3, 1000))):
        assert rq.decode_splits(run.desc, loop, w.q_heads, n) > 1, "the call must use split states"
        q = run.q[loop, layer].contiguous()
        got = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device="cuda")
        status = _noalloc(run, loop, layer, q, n, got)
        assert status == 0, rq.STATUS_NAMES.get(status, status)
        want = rq.decode_attention(run.desc, run.cache, run.signs, loop, layer, q, n,
                                   w.softmax_scale, run.ws)
        torch.cuda.synchronize()
        g, r = got.double().cpu().numpy(), want.double().cpu().numpy()
        assert np.isfinite(g).all()
        assert_close_attention(g, r, f"call {call}: noalloc vs workspace entry point")
        ref = oracle_attention(w, ek, ev, HK, HV, bits16(q[b, head]), loop, n)
        assert_close_attention(g[b, head], ref, f"call {call}: noalloc vs oracle")
        say(f"[noalloc] call {call} (loop {loop}, {n} tokens): rel-L2 to the workspace call "
            f"{np.linalg.norm(g - r) / np.linalg.norm(r):.2e}")


def test_noalloc_refuses_calls_beyond_its_array():
    # grouped-query heads (16 per KV head) over 16 (row, KV head) pairs at 8k
    # tokens: the split states need about 4 MB, more than the 2 MiB array
    desc = rq.make_desc(2, 4, 1, 8, 8193, 128)
    assert rq.decode_workspace_bytes(desc, 128, 8192) > (2 << 20)
    fake = ctypes.c_void_p(1 << 20)
    status = rq.lib().rq_decode_attention_noalloc(ctypes.byref(desc), fake, fake, 0, 0, fake, 128,
                                                  8192, ctypes.c_float(0.088), fake, None)
    assert status == 4, rq.STATUS_NAMES.get(status, status)   # RQ_ERR_WORKSPACE
