"""Shared pieces of the GPU parity tests: oracle runs on kept BF16 slices,
plane comparison through the documented layout, and the error metrics."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import oracle as O
from decode_attention_int4_amd.synth import Workload, rotation_signs
from tests.layout_decode import Geom, decode_slice

# Attention outputs must be within 1e-3 relative L2 and 2e-3 max-abs of the
# fp64 oracle computed on the same BF16 inputs.
REL_L2 = 1e-3
MAX_ABS = 2e-3

POOL = cf.ThreadPoolExecutor(max_workers=8)   # ctypes calls release the GIL


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def params(w: Workload) -> O.Params:
    return O.Params(d=w.head_dim, g=16, P=w.loops_per_group, anchor_bits=w.anchor_bits,
                    residual_bits=w.residual_bits, mode=w.mode, alpha_mode=w.alpha_mode,
                    rotate=1 if (w.rotation == 1 and w.mode != 1) else 0)


def rotations(w: Workload, layer: int):
    """Sign vectors of K and V at `layer` (the oracle builds H from them)."""
    s = rotation_signs(w).numpy()
    return s[0, layer].copy(), s[1, layer].copy()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def encode_kept(w: Workload, kept: torch.Tensor, layer: int):
    """kept: BF16 [2, loops, N, d] -> (enc K, enc V, HK, HV) from the oracle."""
    p = params(w)
    HK, HV = rotations(w, layer)
    fk = POOL.submit(O.encode_slice, p, bits16(kept[0]), HK)
    fv = POOL.submit(O.encode_slice, p, bits16(kept[1]), HV)
    return fk.result(), fv.result(), HK, HV


def assert_planes_equal(gpu: "Planes", enc: O.Encoded, what: str, loops=None, dump=None):
    loops = range(enc.codes.shape[0]) if loops is None else loops
    msgs = []
    for l in loops:
        for name in ("codes", "s8", "z8", "alpha"):
            a, b = getattr(gpu, name)[l], getattr(enc, name)[l]
            if not np.array_equal(a, b):
                bad = np.argwhere(a != b)
                msgs.append(f"{what} loop {l} {name}: {len(bad)} mismatches, first at "
                            f"{bad[0].tolist()}: gpu {a[tuple(bad[0])]} oracle "
                            f"{b[tuple(bad[0])]}")
    if msgs:
        if dump is not None:
            dump(gpu, enc)
        raise AssertionError("; ".join(msgs))


def check_slice_planes(w, run, key, t0=0, n=None):
    b, layer, head = key
    geom = Geom.of(run.desc)
    n = run.N if n is None else n
    ek, ev, HK, HV = encode_kept(w, run.kept[key], layer)
    for kv, enc, H in ((0, ek, HK), (1, ev, HV)):
        gpu = decode_slice(run.cache, geom, kv, b, layer, head, n, t0)

        def dump(g, e, kv=kv, H=H):
            # inputs and both encodings of a mismatching slice, for offline study
            out_dir = os.environ.get("RQ_MISMATCH_DIR", "mismatch_dumps")
            os.makedirs(out_dir, exist_ok=True)
            path = f"{out_dir}/mismatch_{w.name}_kv{kv}_{b}_{layer}_{head}.npz"
            np.savez_compressed(path, x=bits16(run.kept[key][kv]), H=H,
                                gpu_codes=g.codes, gpu_s8=g.s8, gpu_z8=g.z8, gpu_alpha=g.alpha,
                                o_codes=e.codes, o_s8=e.s8, o_z8=e.z8, o_alpha=e.alpha)
            say(f"[dump] wrote {path}")

        assert_planes_equal(gpu, enc, f"{w.name} kv={kv} slice={key}", dump=dump)
    return ek, ev, HK, HV


def attention_errors(gpu: np.ndarray, ref: np.ndarray):
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)
    return rel, np.abs(gpu - ref).max()


def assert_close_attention(gpu, ref, what, scale=1.0):
    """rel-L2 <= 1e-3 and max-abs <= 2e-3 * scale.  The max-abs bound is for
    outputs of unit scale; a caller whose outputs are far larger (hand-built
    inputs of magnitude ~10^3) passes scale = max|ref|."""
    rel, mx = attention_errors(np.asarray(gpu, np.float64), ref)
    assert rel <= REL_L2 and mx <= MAX_ABS * scale, f"{what}: rel-L2 {rel:.3e}, max-abs {mx:.3e}"
    return rel, mx


def oracle_attention(w, ek, ev, HK, HV, q_bits, loop, n):
    return O.attention_slice(params(w), ek, ev, HK, HV, q_bits, loop, n, w.softmax_scale)


def check_reconstruct(w, run, encs, t0, t1, loops=None, tol_rel=2e-5):
    """rq_reconstruct over tokens [t0, t1), fp32 and BF16 outputs, compared
    element by element with the oracle's reconstruction of the same planes
    (ai4snews summary, paragraph 3: anchor plus alpha H^T times the residual).

    encs: {(batch row, layer, kv head): (enc K, enc V, signs K, signs V)}.
    fp32: within tol_rel of max(1, max |ref|) (fp32 arithmetic of the FWHT and
    the alpha products against the fp64 oracle); BF16: bit-equal to the
    round-to-nearest-even of the library's own fp32 result, and within one
    BF16 half-ulp of the fp64 reference plus the fp32 tolerance.  Returns the
    worst fp32 error relative to max(1, max |ref|)."""
    from decode_attention_int4_amd import rq
    loops = range(w.loops) if loops is None else loops
    out32 = rq.reconstruct(run.desc, run.cache, run.signs, t0, t1)
    out16 = rq.reconstruct(run.desc, run.cache, run.signs, t0, t1, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    p = params(w)
    worst = 0.0
    for (b, layer, head), (ek, ev, HK, HV) in encs.items():
        g32 = out32[:, b, :, layer, head].cpu().numpy()
        g16 = bits16(out16[:, b, :, layer, head])
        for kv, e, H in ((0, ek, HK), (1, ev, HV)):
            for loop in loops:
                ref = O.reconstruct_slice(p, e, H, loop, t0, t1)
                got = g32[kv, loop].astype(np.float64)
                scale = max(1.0, float(np.abs(ref).max()))
                err = float(np.abs(got - ref).max()) / scale
                worst = max(worst, err)
                where = f"{w.name} kv {kv} slice {(b, layer, head)} loop {loop} tokens [{t0},{t1})"
                assert err <= tol_rel, f"{where}: fp32 error {err:.3e} of max |ref|"
                mine = O.bf16_encode(got)
                assert np.array_equal(g16[kv, loop], mine), f"{where}: BF16 is not RNE of the fp32 output"
                half_ulp = np.abs(O.bf16_decode(O.bf16_encode(ref)) - ref) + 2.0 ** -9 * np.abs(ref)
                assert np.all(np.abs(O.bf16_decode(g16[kv, loop]) - ref) <= half_ulp + tol_rel * scale), where
    del out32, out16
    return worst
