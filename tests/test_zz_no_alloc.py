"""GPU: the allocation-free step (gdn_step_noalloc, the library's static
scratch in place of a workspace) against gdn_step on the same inputs, through
the C ABI: two calls in a row, the second on a smaller input, each
bit-identical to gdn_step (same kernels, same plan, same rows) and within the
bf16 bar of the oracle."""
import numpy as np
import pytest

from gdn_inputs import WORKLOADS, make_inputs
from oracle import gdn_oracle as O
from tests.gpu_util import TOL, oracle_args, rel_err, to_device, to_numpy

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_step_noalloc_matches_step_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_frame_amd as G
    cases = [
        (WORKLOADS[3].resized(frames=1, h0_sigma=0.1), 0),                         # one frame, 20 x 112
        (WORKLOADS[4].resized(frames=1, tokens_per_frame=300, heads=3), 1),       # smaller: 300 tokens, 3 x 64
    ]
    for w, seed in cases:
        x = make_inputs(w, seed)
        d = to_device(x, w.qkv_dtype)
        args = [d[n] for n in ("q", "k", "v", "log_gate", "beta")]
        ref_out, ref_state = G.step(*args, d["h0"].clone(), None)
        out = torch.empty_like(ref_out)
        state = torch.empty_like(ref_state)
        o, s = G.step_noalloc(*args, d["h0"].clone(), state, out=out)
        torch.cuda.synchronize()
        assert o is out and s is state
        print(f"[noalloc] {w.name} {w.batch}x{w.heads}x{w.d_k} {w.tokens} tokens: "
              f"equal={torch.equal(out, ref_out) and torch.equal(state, ref_state)}", flush=True)
        assert torch.equal(out, ref_out) and torch.equal(state, ref_state)
        ro, rH = O.fwd(*oracle_args(x)[0], x["h0"])
        assert rel_err(to_numpy(out), ro) <= TOL["bf16"] and rel_err(to_numpy(state), rH) <= TOL["bf16"]
