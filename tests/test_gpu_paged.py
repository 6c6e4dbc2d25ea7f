"""GPU parity of the paged cache (vLLM-style block tables; ai4snews summary,
paragraph 4, places the method inside a batching inference server).

Sequences of different lengths are appended through scattered pool blocks:
the codes, FP8 bytes and alphas found at each token's block and in-block
position must equal the oracle's encoding of that token bit for bit, and paged
decode attention must match the fp64 oracle on each sequence's logical tokens
(1e-3 relative L2, 2e-3 max-abs).  The same data in a contiguous cache, read
by the ragged call, must give the same outputs up to fp32 summation order:
the block table changes where the bytes live, not what is computed.  Calls
that run the same kernel shape on both caches agree to rounding (well under
1e-6); a d = 128 anchor call runs eight-wave workgroups on the contiguous
cache and four on the paged one, with its own split plan, and its value sums
then differ by the fp32 rounding of a different summation order, amplified
by the magic-number unpack: each sum accumulates w (1024 + code) and drops
1024 sum(w) at the end, about 1024 / 7.5 = 137 times the mean code term, so
tens of fp32 adds per lane give differences of order 1e-5.  The bound is
1e-4 relative L2; a paging mistake (a wrong block or position) moves the
output by order one."""
import numpy as np
import pytest
import torch

from decode_attention_int4_amd import rq
from decode_attention_int4_amd.synth import Workload, kv_chunk
from decode_attention_int4_amd.workload import RQDecode, desc_for
from tests.gpu_common import (assert_close_attention, assert_planes_equal, bits16, encode_kept,
                              oracle_attention, say)
from tests.layout_decode import Geom, Planes, decode_slice

pytestmark = pytest.mark.gpu


class Pool:
    """A paged cache holding the same logical tokens as `run`'s contiguous one:
    sequence s owns ceil(fill[s] / bt) blocks taken from a random permutation
    of the pool (plus `spare` blocks nobody owns); unused table entries are -1,
    so the appends past a sequence's blocks are skipped."""

    def __init__(self, run: RQDecode, bt: int, fill, chunk: int, seed: int, spare: int = 3):
        w = run.w
        self.bt, self.fill = bt, list(fill)
        need = [-(-n // bt) for n in self.fill]
        n_blocks = sum(need) + spare
        rng = np.random.default_rng(seed)
        perm = rng.permutation(n_blocks).astype(np.int32)
        self.table = np.full((w.batch, max(need) + 1), -1, np.int32)
        k = 0
        for s, m in enumerate(need):
            self.table[s, :m] = perm[k:k + m]
            k += m
        self.desc = desc_for(w, bt)
        self.desc.batch = n_blocks
        self.cache = rq.alloc_cache(self.desc)
        self.cache.zero_()
        self.table_dev = torch.from_numpy(self.table).cuda()
        # the same chunks as the contiguous fill, so the generated states agree
        for t0 in range(0, run.N, chunk):
            t1 = min(run.N, t0 + chunk)
            x = kv_chunk(w, t0, t1, "cuda", run.lam)
            pos = torch.full((w.batch,), t0, dtype=torch.int32, device="cuda")
            rq.paged_quantize_append(self.desc, self.cache, x, self.table_dev, pos, run.signs)
        torch.cuda.synchronize()

    def planes(self, kv: int, s: int, layer: int, head: int, n: int) -> Planes:
        """Logical planes of sequence s's first n tokens, gathered block by block."""
        geom = Geom.of(self.desc)
        parts = []
        for j in range(-(-n // self.bt)):
            m = min(self.bt, n - j * self.bt)
            parts.append(decode_slice(self.cache, geom, kv, int(self.table[s, j]), layer, head, m))
        return Planes(*(np.concatenate([getattr(p, f) for p in parts], axis=1)
                        for f in ("codes", "s8", "z8", "alpha")))


CASES = [
    # d, block tokens, mode, per-sequence fill, lengths attended, query heads per KV head
    # (2: the grouped kernel serves every call but a chained loop's several
    # planes; 1: the per-head kernel, eight waves for d = 128 residual calls)
    (128, 16, 0, (333, 200, 17, 333), (333, 200, 0, 101), 2),
    (128, 64, 0, (333, 333, 70, 5), (320, 1, 70, 5), 2),
    (96, 32, 0, (300, 129, 300, 64), (300, 129, 255, 64), 2),
    (64, 32, 0, (300, 96, 31, 300), (300, 96, 31, 0), 2),
    (64, 128, 1, (300, 250, 300, 3), (299, 250, 128, 3), 2),
    (128, 32, 2, (290, 290, 40, 160), (290, 200, 40, 160), 2),
    (128, 16, 0, (600, 333, 17, 560), (600, 333, 0, 421), 1),
    (96, 32, 0, (500, 129, 300, 64), (500, 129, 255, 64), 1),
    (128, 64, 1, (520, 250, 300, 3), (519, 250, 128, 3), 1),
    (64, 32, 2, (450, 97, 300, 33), (450, 96, 300, 0), 1),
]


@pytest.mark.parametrize("d,bt,mode,fill,lengths,G", CASES,
                         ids=[f"d{c[0]}-bt{c[1]}-mode{c[2]}-G{c[5]}" for c in CASES])
def test_paged_append_and_decode(d, bt, mode, fill, lengths, G):
    N = max(fill)
    w = Workload(f"paged_d{d}_bt{bt}_m{mode}_g{G}", batch=len(fill), loops=4, layers=2, kv_heads=2,
                 q_heads=2 * G, head_dim=d, n_tokens=N, seed=d + bt + mode + G, mode=mode)
    keep = [(s, 1, 1) for s in range(w.batch)] + [(0, 0, 0)]
    chunk = 100
    say(f"[paged] {w.name} fill {fill} lengths {lengths}")
    run = RQDecode(w, keep=keep, chunk_tokens=chunk)
    pool = Pool(run, bt, fill, chunk, seed=d * 7 + bt)

    # planes: every kept slice, through the block table
    for (s, layer, head) in keep:
        n = fill[s]
        ek, ev, _, _ = encode_kept(w, run.kept[(s, layer, head)][:, :, :n], layer)
        for kv, enc in ((0, ek), (1, ev)):
            assert_planes_equal(pool.planes(kv, s, layer, head, n), enc,
                                f"{w.name} kv={kv} seq={s} layer={layer} head={head}")

    # attention: oracle on the logical tokens, and the contiguous ragged call
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    max_n = max(lengths)
    ws = rq.alloc_workspace(rq.paged_decode_workspace_bytes(pool.desc, w.q_heads, w.batch, max_n))
    ws_c = rq.alloc_workspace(rq.decode_workspace_bytes(run.desc, w.q_heads, max_n))
    enc = {k: encode_kept(w, run.kept[k], k[1]) for k in keep}
    for loop in range(w.loops):
        for layer in range(w.layers):
            q = run.q[loop, layer]
            got = rq.paged_decode_attention(pool.desc, pool.cache, run.signs, loop, layer, q,
                                            pool.table_dev, lens, max_n, w.softmax_scale, ws)
            ref_c = rq.decode_attention_ragged(run.desc, run.cache, run.signs, loop, layer, q,
                                               lens, max_n, w.softmax_scale, ws_c)
            got, ref_c = got.cpu().numpy().astype(np.float64), ref_c.cpu().numpy().astype(np.float64)
            diff = np.linalg.norm(got - ref_c) / max(np.linalg.norm(ref_c), 1e-30)
            assert diff <= 1e-4, f"{w.name} loop {loop} layer {layer}: paged vs contiguous rel-L2 {diff:.2e}"
            for (s, lay, head) in keep:
                if lay != layer:
                    continue
                n = lengths[s]
                for hq in range(G * head, G * head + G):
                    if n == 0:
                        assert np.all(got[s, hq] == 0)
                        continue
                    ek, ev, HK, HV = enc[(s, lay, head)]
                    ref = oracle_attention(w, ek, ev, HK, HV, bits16(q[s, hq]), loop, n)
                    assert_close_attention(got[s, hq], ref,
                                           f"{w.name} seq {s} n {n} loop {loop} hq {hq}")


def test_paged_append_crosses_blocks_and_skips_unmapped():
    """A multi-token append that crosses a block boundary lands in both blocks;
    tokens whose block id is outside the pool, and sequences whose range does
    not fit their table, are not written anywhere."""
    d, bt = 128, 16
    w = Workload("paged_cross", batch=3, loops=4, layers=1, kv_heads=2, q_heads=2, head_dim=d,
                 n_tokens=20, seed=5)
    run = RQDecode(w, keep=[(s, 0, h) for s in range(3) for h in range(2)], chunk_tokens=20)
    table = np.array([[4, 1], [0, 7], [2, -1]], np.int32)   # block 7 is outside the pool
    desc = desc_for(w, bt)
    desc.batch = 6
    cache = rq.alloc_cache(desc)
    cache.zero_()
    x = kv_chunk(w, 0, 20, "cuda", run.lam)
    # seq 0: tokens 5..24 span blocks 4 and 1; seq 1: tokens 10..29, the part in
    # table entry 1 (block 7) is skipped; seq 2 starts at 20 > 32 - 20: skipped
    pos = torch.tensor([5, 10, 20], dtype=torch.int32, device="cuda")
    rq.paged_quantize_append(desc, cache, x, torch.from_numpy(table).cuda(), pos, run.signs)
    torch.cuda.synchronize()
    geom = Geom.of(desc)
    for s, ranges in ((0, [(4, 5, 11), (1, 0, 9)]), (1, [(0, 10, 6)])):
        for head in range(2):
            ek, ev, _, _ = encode_kept(w, run.kept[(s, 0, head)], 0)
            t = 0
            for blk, start, m in ranges:
                for kv, e in ((0, ek), (1, ev)):
                    g = decode_slice(cache, geom, kv, blk, 0, head, m, start)
                    for f in ("codes", "s8", "z8", "alpha"):
                        assert np.array_equal(getattr(g, f), getattr(e, f)[:, t:t + m]), \
                            (s, blk, kv, f)
                t += m
    # blocks 2, 3 and 5 were never the target of a mapped token: still zero
    for blk in (2, 3, 5):
        for kv in range(2):
            for head in range(2):
                g = decode_slice(cache, geom, kv, blk, 0, head, bt)
                assert not g.codes.any() and not g.s8.any() and not g.alpha.any(), (blk, kv, head)
