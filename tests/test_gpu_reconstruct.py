"""GPU parity of rq_reconstruct (ai4snews summary, paragraph 3: a loop is
rebuilt from the shared anchor plus alpha H^T times its own residual, two
reads) against the oracle, element by element, in fp32 and BF16, for head_dim
64, 96 (block-diagonal 64 + 32 transform) and 128, in residual, direct and
chained modes and the bit-width / alpha / rotation variants.  Whole token
ranges and a ragged interior window are rebuilt."""
import pytest
import torch

from decode_attention_int4_amd.synth import Workload
from decode_attention_int4_amd.workload import RQDecode
from tests.gpu_common import check_reconstruct, encode_kept, say

pytestmark = pytest.mark.gpu

MODES = {
    "residual": {},
    "direct": dict(mode=1),
    "chained": dict(mode=2),
    "chained_no_rotation": dict(mode=2, rotation=0),
    "uniform_int4": dict(residual_bits=4),
    "int2_anchor": dict(anchor_bits=2),
    "norm_ratio": dict(alpha_mode=1),
    "no_rotation": dict(rotation=0),
}


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("mode", list(MODES))
def test_reconstruct_modes(d, mode):
    w = Workload(f"recon_{mode}_{d}", batch=2, loops=8, layers=2, kv_heads=2, q_heads=2,
                 head_dim=d, n_tokens=200, seed=3 * d + len(mode), **MODES[mode])
    keep = [(1, 1, 0), (0, 0, 1)]
    say(f"[reconstruct] {w.name}")
    run = RQDecode(w, keep=keep, chunk_tokens=96)
    torch.cuda.synchronize()
    encs = {k: encode_kept(w, run.kept[k], k[1]) for k in keep}
    worst = 0.0
    for t0, t1 in ((0, 200), (37, 101), (199, 200)):
        worst = max(worst, check_reconstruct(w, run, encs, t0, t1))
    say(f"[reconstruct] {w.name}: worst fp32 error {worst:.2e} of max |x|")
