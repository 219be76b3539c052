"""The forward recorded into a HIP graph and replayed (needs a gfx950 GPU).

The library enqueues only kernels on the caller's stream (no allocation, no
memset nodes, no host synchronisation), so one forward can be captured with
torch's graph API and replayed.  Every replay must equal the eager call bit
for bit, also when eager calls on other inputs, sharing the workspace, run
between the replays: the tile table, the split-K counters and the partial sums
live in that workspace and are rewritten by every call.
"""
import sys

import pytest
import torch

from sparse_moe_layer_06_amd import binding as B
from sparse_moe_layer_06_amd import synth

pytestmark = pytest.mark.gpu

TINY = synth.CONFIGS["tiny_f32"]
CASES = {
    "bf16_deep": TINY.with_(name="bf16_deep", T=500, d=512, l=128, E=8, k=2, f=256, f_s=320,
                            act="bf16", experts="bf16"),
    # 64 x 128 expert tiles with split-K items finished by the last block
    "few_rows_wide": TINY.with_(name="few_rows_wide", T=24, d=4096, l=1024, E=32, k=4, f=1280, f_s=0,
                                act="bf16", experts="bf16"),
    # full rounds of expert items, then tail items split along K
    "few_rows_rounds": TINY.with_(name="few_rows_rounds", T=64, d=5120, l=1280, E=64, k=8, f=2304, f_s=0,
                                    act="bf16", experts="bf16"),
    "latent_nvfp4_zipf": TINY.with_(name="latent_nvfp4_zipf", T=40, d=256, l=64, E=32, k=5, f=128, f_s=0,
                                    act="bf16", experts="nvfp4", zipf_bias=True, router_latent=True),
    "fp8_shared": TINY.with_(name="fp8_shared", T=150, d=512, l=128, E=16, k=3, f=192, f_s=256,
                             act="bf16", experts="bf16", shared_fp8=True),
    "standard_bf16": TINY.with_(name="standard_bf16", T=150, d=256, l=256, E=16, k=3, f=128, f_s=128,
                                act="bf16", experts="bf16", standard_moe=True),
    "f32_ragged": TINY.with_(name="f32_ragged", T=77, d=256, l=64, E=9, k=3, f=192, f_s=128),
    "nvfp4_2d_few_wide": TINY.with_(name="nvfp4_2d_few_wide", T=16, d=4096, l=1024, E=16, k=2, f=1280, f_s=0,
                                    act="bf16", experts="nvfp4_2d"),
    "mxfp8_proj_few": TINY.with_(name="mxfp8_proj_few", T=20, d=1024, l=256, E=8, k=2, f=128, f_s=256,
                                 act="bf16", experts="nvfp4", proj_mxfp8=True, shared_fp8=True, router_latent=True),
    # split-K fp8 GEMMs (fp8 projections and shared expert at few rows)
    "fp8_proj_few": TINY.with_(name="fp8_proj_few", T=20, d=1024, l=256, E=8, k=2, f=128, f_s=256,
                               act="bf16", experts="nvfp4", proj_fp8=True, shared_fp8=True, router_latent=True),
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


def small_inputs(cfg, seed):
    inp = synth.make_inputs(cfg, seed, "cpu")
    return {k: (v.cuda() if v is not None else None) for k, v in inp.items()}


def replay_check(cfg, inp, inp2, replays=3):
    ws = B.alloc_workspace(cfg)
    out = torch.empty((cfg.T, cfg.d), dtype=B.act_dtype(cfg), device="cuda")
    out2 = torch.empty_like(out)
    ref = B.forward(cfg, inp, out=out, workspace=ws).clone()
    ref2 = B.forward(cfg, inp2, out=out2, workspace=ws).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.Call(cfg, inp, out, ws)()
    torch.cuda.synchronize()
    for i in range(replays):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        # eager work between replays, on other inputs and the same workspace
        out2.zero_()
        B.forward(cfg, inp2, out=out2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref2), f"eager call after replay {i}"
    del g


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    cfg = CASES[name]
    log(f"case graph {name} {cfg}")
    replay_check(cfg, small_inputs(cfg, 0), small_inputs(cfg, 1))


@pytest.mark.timeout(900)
def test_graph_replays_match_eager_decode_full_size():
    # 64 tokens, 512 experts, top-22 with the skewed bias: the 64 x 128 expert
    # tiles with the split last round, expert weights in the tiled layout
    cfg = synth.CONFIGS["decode_bf16_zipf"]
    log(f"case graph {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    cfg_t, inp_t = B.pack_experts(cfg, inp)
    inp2 = dict(inp_t)
    inp2["x"] = -inp["x"]  # other logits, so other experts behind expert 0
    replay_check(cfg_t, inp_t, inp2)
