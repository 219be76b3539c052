"""The allocation-free entry point, lmoe_static_forward, through the C ABI
(needs a gfx950 GPU): two calls in a row, the second on fewer tokens, each
bit-identical to latentmoe_forward with a workspace of its own; the second
call changes no device allocation."""
import sys

import pytest
import torch

from sparse_moe_layer_06_amd import binding as B
from sparse_moe_layer_06_amd import synth

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS
CASES = {
    # many rows per expert with a shared expert (192-row tiles, fused dense GEMMs)
    "bf16_deep": CFG["tiny_f32"].with_(name="bf16_deep", T=500, d=512, l=128, E=8, k=2, f=256, f_s=320,
                                       act="bf16", experts="bf16"),
    # NVFP4 experts with the router in the latent space
    "nvfp4_latent": CFG["tiny_f32"].with_(name="nvfp4_latent", T=300, d=512, l=128, E=16, k=3, f=256, f_s=0,
                                          act="bf16", experts="nvfp4", router_latent=True),
    # the decode workload at full size (skewed routing, split-K GEMMs and tails)
    "decode_bf16_zipf": CFG["decode_bf16_zipf"],
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", list(CASES))
def test_static_forward_equals_workspace_forward_on_two_calls(name):
    cfg = CASES[name]
    first = synth.make_inputs(cfg, 0, "cuda")
    second = synth.make_inputs(cfg.with_(T=max(1, cfg.T // 4)), 1, "cuda")
    for call, inp in (("first", first), ("second", second)):
        T = inp["x"].shape[0]
        log(f"case {name} call {call} T={T}")
        ref = B.forward(cfg, inp)
        got = torch.empty_like(ref)
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        B.static_forward(cfg, inp, out=got)
        torch.cuda.synchronize()
        free_after = torch.cuda.mem_get_info()[0]
        assert torch.equal(got, ref), (name, call)
        if call == "second":  # the scratch array is the library's since load: nothing allocated per call
            assert free_after == free_before, (free_before, free_after)
