"""HIP path vs the CPU oracle, through the C ABI (needs a gfx950 GPU).

Every case, small or full-size, checks the routing, the permutation and the
outputs (z, c, out) of every token; the full-size workloads run at the sizes
and in the launch configuration the benchmark times, and the oracle
evaluates them expert by expert.
"""
import sys

import numpy as np
import pytest
import torch

import parity as P
from oracle import latentmoe_oracle as O
from sparse_moe_layer_06_amd import binding as B
from sparse_moe_layer_06_amd import synth

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS
TINY = CFG["tiny_f32"]
# Small layers that still span several MFMA tiles with ragged edges.
SMALL = {
    "bf16_ragged": TINY.with_(name="bf16_ragged", T=193, d=256, l=64, E=12, k=3, f=192, f_s=192,
                              act="bf16", experts="bf16"),
    # >= 96 rows per expert on average: the 192-row expert tiles, each expert
    # in one partly filled tile
    "bf16_deep": TINY.with_(name="bf16_deep", T=500, d=512, l=128, E=8, k=2, f=256, f_s=320,
                            act="bf16", experts="bf16"),
    "nvfp4_deep": TINY.with_(name="nvfp4_deep", T=300, d=512, l=128, E=4, k=2, f=256, f_s=0,
                             act="bf16", experts="nvfp4"),
    # more than 192 rows per expert: full and partly filled 192-row tiles
    "bf16_deep192": TINY.with_(name="bf16_deep192", T=450, d=512, l=128, E=4, k=2, f=320, f_s=192,
                               act="bf16", experts="bf16"),
    "nvfp4_deep192": TINY.with_(name="nvfp4_deep192", T=400, d=512, l=128, E=4, k=2, f=256, f_s=0,
                                act="bf16", experts="nvfp4"),
    # the register-weight expert GEMM (192-row tiles, N a multiple of 256, K
    # steps a multiple of 4): ragged experts in one or two tiles, one item per
    # block; and 64 experts over 3 N tiles with K of 4 and 12 steps, several
    # items per block
    "bf16_regw": TINY.with_(name="bf16_regw", T=600, d=1024, l=256, E=4, k=2, f=512, f_s=256,
                            act="bf16", experts="bf16"),
    "bf16_regw_items": TINY.with_(name="bf16_regw_items", T=4096, d=1024, l=256, E=64, k=6, f=768, f_s=0,
                                  act="bf16", experts="bf16"),
    # the register-decode NVFP4 expert GEMM (192-row tiles, N a multiple of
    # 256, K steps a multiple of 4), 1-D and 2-D scale blocks
    "nvfp4_regw": TINY.with_(name="nvfp4_regw", T=600, d=1024, l=256, E=4, k=2, f=512, f_s=0,
                             act="bf16", experts="nvfp4"),
    "nvfp4_2d_regw": TINY.with_(name="nvfp4_2d_regw", T=600, d=1024, l=256, E=4, k=2, f=512, f_s=0,
                                act="bf16", experts="nvfp4_2d"),
    "nvfp4_regw_items": TINY.with_(name="nvfp4_regw_items", T=4096, d=1024, l=256, E=64, k=6, f=768, f_s=0,
                                   act="bf16", experts="nvfp4"),
    "nvfp4_sparse": TINY.with_(name="nvfp4_sparse", T=70, d=256, l=64, E=16, k=3, f=128, f_s=0,
                               act="bf16", experts="nvfp4"),
    "zipf_small": TINY.with_(name="zipf_small", T=64, d=512, l=128, E=64, k=6, f=256, f_s=0,
                             act="bf16", experts="bf16", zipf_bias=True),
    "f32_ragged": TINY.with_(name="f32_ragged", T=77, d=256, l=64, E=9, k=3, f=192, f_s=128),
    "T1_bf16": TINY.with_(name="T1_bf16", T=1, d=256, l=64, E=16, k=4, f=128, f_s=64, act="bf16",
                          experts="bf16"),
    "k1_bf16": TINY.with_(name="k1_bf16", T=128, d=256, l=64, E=8, k=1, f=128, act="bf16", experts="bf16"),
    "kE_bf16": TINY.with_(name="kE_bf16", T=64, d=256, l=64, E=5, k=5, f=64, act="bf16", experts="bf16"),
    # few rows per expert (the 64-row, 4-stage expert tiles), short K (l=128,
    # f=192) and deep K (l=f=512)
    "few_rows_ragged": TINY.with_(name="few_rows_ragged", T=37, d=512, l=128, E=32, k=5, f=192, f_s=64,
                                  act="bf16", experts="bf16"),
    "few_rows_deepK": TINY.with_(name="few_rows_deepK", T=20, d=2048, l=512, E=16, k=4, f=512, f_s=0,
                                 act="bf16", experts="bf16"),
    # few rows per expert and outputs >= 1024 wide (the 64 x 128 expert
    # tiles, two blocks per CU): fewer items than blocks, so GEMM1 runs whole
    # items and GEMM2 splits them along K
    "few_rows_wide": TINY.with_(name="few_rows_wide", T=24, d=4096, l=1024, E=32, k=4, f=1280, f_s=0,
                                act="bf16", experts="bf16"),
    # the same with both expert GEMMs' outputs (f = 1216, l = 1088) ending in
    # a partly filled 128-wide N tile
    "few_rows_wide_ragged": TINY.with_(name="few_rows_wide_ragged", T=24, d=4352, l=1088, E=32, k=4, f=1216,
                                       f_s=0, act="bf16", experts="bf16"),
    # more 64 x 128 expert items than blocks, not in whole rounds (about 1150
    # items in GEMM1 and 640 in GEMM2 over 512 blocks on 256 CUs): full
    # rounds, then the tail items split along K
    "few_rows_rounds": TINY.with_(name="few_rows_rounds", T=64, d=5120, l=1280, E=64, k=8, f=2304, f_s=0,
                                    act="bf16", experts="bf16"),
    "nvfp4_few_wide": TINY.with_(name="nvfp4_few_wide", T=16, d=4096, l=1024, E=16, k=2, f=1280, f_s=0,
                                 act="bf16", experts="nvfp4"),
    "nvfp4_few_wide_ragged": TINY.with_(name="nvfp4_few_wide_ragged", T=16, d=4352, l=1088, E=16, k=2, f=1216,
                                        f_s=0, act="bf16", experts="nvfp4"),
    # top-k beyond one register slot per lane: k = 100 of E = 256, and E = 1024
    "k100_E256": TINY.with_(name="k100_E256", T=16, d=256, l=64, E=256, k=100, f=64, act="bf16",
                            experts="bf16"),
    "E1024": TINY.with_(name="E1024", T=32, d=256, l=64, E=1024, k=8, f=64, act="bf16", experts="bf16"),
    # the router reading the stored latent z (W_r [E][l])
    "latent_bf16": TINY.with_(name="latent_bf16", T=150, d=512, l=128, E=24, k=4, f=192, f_s=128,
                              act="bf16", experts="bf16", router_latent=True),
    "latent_f32": TINY.with_(name="latent_f32", T=70, E=12, k=3, f_s=64, router_latent=True),
    "latent_nvfp4_zipf": TINY.with_(name="latent_nvfp4_zipf", T=40, d=256, l=64, E=32, k=5, f=128, f_s=0,
                                    act="bf16", experts="nvfp4", zipf_bias=True, router_latent=True),
    # FP8 shared expert (E4M3 weights, per-token E4M3 inputs, fp8 MFMA GEMMs)
    "fp8_shared": TINY.with_(name="fp8_shared", T=150, d=512, l=128, E=16, k=3, f=192, f_s=256,
                             act="bf16", experts="bf16", shared_fp8=True),
    "fp8_shared_few": TINY.with_(name="fp8_shared_few", T=5, d=1024, l=256, E=8, k=2, f=128, f_s=384,
                                 act="bf16", experts="nvfp4", shared_fp8=True, router_latent=True),
    # the standard MoE comparison layer (no latent projections, experts in d)
    "standard_bf16": TINY.with_(name="standard_bf16", T=150, d=256, l=256, E=16, k=3, f=128, f_s=128,
                                act="bf16", experts="bf16", standard_moe=True),
    "standard_f32": TINY.with_(name="standard_f32", T=40, l=256, E=8, k=2, f_s=64, standard_moe=True),
    "standard_fp8_zipf": TINY.with_(name="standard_fp8_zipf", T=24, d=512, l=512, E=32, k=6, f=256, f_s=256,
                                    act="bf16", experts="bf16", shared_fp8=True, zipf_bias=True,
                                    standard_moe=True),
    # FP8 down- and up-projections (E4M3 weights, per-token E4M3 inputs):
    # many rows (256x256 fp8 tiles) with a bf16 shared expert added after
    # the fp8 up-projection; few rows (split-K fp8 GEMMs) with everything
    # else fp8 too; skewed routing without a shared expert
    "fp8_proj": TINY.with_(name="fp8_proj", T=150, d=512, l=128, E=16, k=3, f=192, f_s=128,
                           act="bf16", experts="bf16", proj_fp8=True),
    "fp8_proj_few": TINY.with_(name="fp8_proj_few", T=20, d=1024, l=256, E=8, k=2, f=128, f_s=256,
                               act="bf16", experts="nvfp4", proj_fp8=True, shared_fp8=True, router_latent=True),
    "fp8_proj_zipf": TINY.with_(name="fp8_proj_zipf", T=64, d=2048, l=512, E=64, k=6, f=256, f_s=0,
                                act="bf16", experts="bf16", proj_fp8=True, zipf_bias=True),
    # NVFP4 with 16 x 16 scale blocks: 192-row tiles, and the 64 x 128 tiles
    # of few rows (split along K in GEMM2)
    "nvfp4_2d_deep": TINY.with_(name="nvfp4_2d_deep", T=300, d=512, l=128, E=4, k=2, f=256, f_s=0,
                                act="bf16", experts="nvfp4_2d"),
    "nvfp4_2d_deep192": TINY.with_(name="nvfp4_2d_deep192", T=400, d=512, l=128, E=4, k=2, f=256, f_s=0,
                                   act="bf16", experts="nvfp4_2d"),
    "nvfp4_2d_few_wide": TINY.with_(name="nvfp4_2d_few_wide", T=16, d=4096, l=1024, E=16, k=2, f=1280, f_s=0,
                                    act="bf16", experts="nvfp4_2d"),
    # MXFP8 projections (E4M3 with E8M0 scales per 32 elements, applied by
    # the scaled MFMA): many rows, few rows (split-K), skewed routing
    "mxfp8_proj": TINY.with_(name="mxfp8_proj", T=150, d=512, l=128, E=16, k=3, f=192, f_s=128,
                             act="bf16", experts="bf16", proj_mxfp8=True),
    "mxfp8_proj_few": TINY.with_(name="mxfp8_proj_few", T=20, d=1024, l=256, E=8, k=2, f=128, f_s=256,
                                 act="bf16", experts="nvfp4", proj_mxfp8=True, shared_fp8=True, router_latent=True),
    "mxfp8_proj_zipf": TINY.with_(name="mxfp8_proj_zipf", T=64, d=2048, l=512, E=64, k=6, f=256, f_s=0,
                                  act="bf16", experts="bf16", proj_mxfp8=True, zipf_bias=True),
    "E1_f32": TINY.with_(name="E1_f32", T=33, E=1, k=1),
    "E1_bf16": TINY.with_(name="E1_bf16", T=150, E=1, k=1, act="bf16", experts="bf16", f_s=64),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def small_inputs(cfg, seed=0):
    inp = synth.make_inputs(cfg, seed, "cpu")
    return {k: (v.cuda() if v is not None else None) for k, v in inp.items()}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.empty_cache()


def test_tiny_f32_matches_oracle_everywhere():
    log("case tiny_f32 T=64 d=256 E=16 k=4")
    errs, _, _ = P.run_and_check(TINY, small_inputs(TINY), report=log)
    assert errs["tokens_checked"] == TINY.T - errs["tie_substitutions"]


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layers_match_oracle(name):
    cfg = SMALL[name]
    log(f"case {name} {cfg}")
    P.run_and_check(cfg, small_inputs(cfg), report=log)


def test_all_tokens_to_one_expert():
    cfg = SMALL["bf16_ragged"]
    inp = small_inputs(cfg)
    bias = torch.full((cfg.E,), -30.0, dtype=torch.float32)
    bias[[3, 7, 1]] = torch.tensor([30.0, 20.0, 10.0])  # every token: experts 3, 7, 1 in that order
    inp["b_r"] = bias.cuda()
    log("case one-expert-takes-all")
    errs, _, dbg = P.run_and_check(cfg, inp, report=log)
    counts = dbg["counts"].cpu().numpy()
    assert counts[3] == counts[7] == counts[1] == cfg.T and counts.sum() == cfg.T * cfg.k


@pytest.mark.parametrize("name", ["bf16_deep", "nvfp4_deep", "nvfp4_2d_deep", "bf16_deep192", "nvfp4_deep192",
                                  "nvfp4_2d_deep192", "bf16_regw", "nvfp4_regw", "nvfp4_2d_regw"])
def test_experts_spanning_several_tiles(name):
    # every token routed to the same two experts (a large bias on them): 500
    # rows each, so each expert takes two full 192-row tiles and a 116-row
    # partial one; all tokens are compared
    cfg = SMALL[name].with_(T=500)
    inp = small_inputs(cfg)
    bias = torch.full((cfg.E,), -30.0, dtype=torch.float32)
    bias[[2, 1]] = torch.tensor([30.0, 20.0])
    inp["b_r"] = bias.cuda()
    log(f"case {name} forced to experts 2, 1 T={cfg.T}")
    errs, _, dbg = P.run_and_check(cfg, inp, report=log)
    counts = dbg["counts"].cpu().numpy()
    assert counts[2] == counts[1] == cfg.T and errs["tokens_checked"] == cfg.T


@pytest.mark.parametrize("experts", ["nvfp4", "nvfp4_2d"])
def test_nvfp4_items_of_one_k_step(experts):
    # l = 64: the NVFP4 expert GEMM1 has a single K step per item (its fill
    # side moves to the next item on every step) and GEMM2 two; 100 rows per
    # expert, so the 192-row tiles (three A stages) run, one item per block
    cfg = TINY.with_(name=f"{experts}_one_k_step", T=400, d=256, l=64, E=4, k=1, f=128, f_s=0, act="bf16",
                     experts=experts)
    inp = small_inputs(cfg)
    log(f"case {cfg.name}")
    errs, _, _ = P.run_and_check(cfg, inp, report=log)
    assert errs["tokens_checked"] == cfg.T


@pytest.mark.parametrize("T,d", [(193, 256), (64, 1024)], ids=["router_kernel", "in_gemm_reduction"])
def test_exact_logit_ties_break_to_lower_id(T, d):
    # x = 0 makes every logit equal to its bias; equal biases must pick the
    # lower ids.  64 tokens with d = 1024 take the top-k inside the first
    # GEMM's split-K reduction.
    cfg = SMALL["bf16_ragged"].with_(f_s=0, T=T, d=d, l=d // 4)
    inp = small_inputs(cfg)
    inp["x"].zero_()
    inp["b_r"] = torch.tensor([0.5, 1.0, 1.0, 0.0, 1.0, 0.5, 2.0, 1.0, 0, 0, 0, 0], dtype=torch.float32).cuda()
    dbg = P.debug_buffers(cfg, cfg.T)
    with B.KernelTimer() as kt:
        B.forward(cfg, inp, debug=dbg)
        torch.cuda.synchronize()
    idx = dbg["topk_idx"].cpu().numpy()
    assert np.all(idx == np.array([6, 1, 2])), idx[:2]
    ran = kt.by_kernel()
    # 64 tokens: the reduction also permutes (its last token block), so no
    # router or permutation kernel of its own runs
    fused = "splitk_reduce_topk_perm" in ran
    assert fused == (T == 64) and fused != ("topk_softmax" in ran)
    assert fused != any(n.startswith("perm_") for n in ran)


def test_staged_entry_points_compose_to_forward():
    for name in ("bf16_deep", "nvfp4_sparse", "f32_ragged", "few_rows_wide", "latent_bf16", "fp8_shared",
                 "standard_bf16", "fp8_proj", "fp8_proj_few", "mxfp8_proj", "mxfp8_proj_few"):
        cfg = SMALL[name]
        log(f"case staged {name}")
        inp = small_inputs(cfg)
        ws = B.alloc_workspace(cfg)
        fused = B.forward(cfg, inp, workspace=ws)
        r = B.project_route(cfg, inp, ws)
        p = B.permute(cfg, r["idx"], ws)
        z = inp["x"] if cfg.standard_moe else r["z"]  # a standard MoE computes on x
        Y = B.experts_ffn(cfg, inp, z, p["offsets"], p["perm"], ws)
        o = B.combine_up(cfg, inp, Y, p["inv"], r["gate"], r["hs"], ws, cfg.T)
        torch.cuda.synchronize()
        assert torch.equal(o["out"], fused), name


@pytest.mark.parametrize("name", ["bf16_deep", "few_rows_wide", "few_rows_rounds"])
def test_repeated_runs_are_bit_identical(name):
    # few_rows_wide: expert GEMMs with split-K items, whose partial sums are
    # added by whichever block finishes last
    cfg = SMALL[name]
    inp = small_inputs(cfg)
    ws = B.alloc_workspace(cfg)
    a = B.forward(cfg, inp, workspace=ws).clone()
    for _ in range(5):
        b = B.forward(cfg, inp, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_context_owned_workspace():
    # the optional context: reserved for 8 tokens it refuses a 500-token call
    # (it never allocates in the forward), reserved again it grows and gives
    # the same bytes as a caller-provided workspace; it does not shrink
    cfg = SMALL["bf16_deep"]
    inp = small_inputs(cfg)
    ref = B.forward(cfg, inp).clone()
    with B.Context(0) as ctx:
        ctx.reserve(cfg, 8)
        small = ctx.workspace_bytes()
        out = torch.empty_like(ref)
        with pytest.raises(B.LatentMoEError):
            ctx.forward(cfg, inp, out)
        ctx.reserve(cfg)
        assert ctx.workspace_bytes() > small
        ctx.forward(cfg, inp, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        big = ctx.workspace_bytes()
        ctx.reserve(cfg, 8)
        assert ctx.workspace_bytes() == big
    assert not ctx.h  # closed on leaving the block


def test_invalid_expert_ids_are_left_out_of_the_permutation():
    cfg = SMALL["bf16_ragged"]
    ws = B.alloc_workspace(cfg)
    idx = torch.randint(0, cfg.E, (cfg.T, cfg.k), dtype=torch.int32, generator=torch.Generator().manual_seed(3))
    idx[5, 1] = cfg.E + 3
    idx[9, 0] = -1
    p = B.permute(cfg, idx.cuda(), ws)
    torch.cuda.synchronize()
    inv = p["inv"].cpu().numpy()
    assert inv[5 * cfg.k + 1] == -1 and inv[9 * cfg.k] == -1
    valid = idx.numpy().reshape(-1)
    valid = valid[(valid >= 0) & (valid < cfg.E)]
    assert np.array_equal(p["counts"].cpu().numpy(), np.bincount(valid, minlength=cfg.E))


@pytest.mark.parametrize("T,k,E", [(4096, 8, 256), (4097, 8, 256), (300, 22, 1024), (1, 1, 1), (2048, 1, 7)])
def test_permutation_matches_oracle_on_both_paths(T, k, E):
    # 4096 x 8 = 32768 pairs is the largest single-block permutation; 4097 x 8
    # takes the histogram / chunk-scan / scatter kernels.
    cfg = TINY.with_(name="perm", T=T, k=k, E=E, act="bf16", experts="bf16")
    log(f"case permutation T={T} k={k} E={E}")
    ws = B.alloc_workspace(cfg)
    g = torch.Generator().manual_seed(T * 31 + E)
    idx = torch.argsort(torch.rand(T, E, generator=g), dim=1)[:, :k].to(torch.int32).contiguous()
    p = B.permute(cfg, idx.cuda(), ws)
    torch.cuda.synchronize()
    rc, ro, rp, ri = O.permutation(idx.numpy(), E)
    assert np.array_equal(p["counts"].cpu().numpy(), rc)
    assert np.array_equal(p["offsets"].cpu().numpy(), ro)
    assert np.array_equal(p["perm"].cpu().numpy(), rp)
    assert np.array_equal(p["inv"].cpu().numpy(), ri)


@pytest.mark.parametrize("name", ["bf16_deep", "bf16_regw", "bf16_regw_items", "zipf_small", "few_rows_ragged", "few_rows_wide", "few_rows_wide_ragged",
                                  "few_rows_rounds", "k100_E256", "E1_bf16"])
def test_tiled_expert_weights(name):
    # the packed layout holds the same values: outputs bit-identical to the
    # row-major stacks, and the oracle (row-major weights) agrees
    # (few_rows_wide, few_rows_wide_ragged, few_rows_rounds: 64 x 128 tiles with the split tail)
    cfg = SMALL[name]
    log(f"case tiled {name}")
    inp = small_inputs(cfg)
    ref = B.forward(cfg, inp).clone()
    cfg_t, inp_t = B.pack_experts(cfg, inp)
    out = B.forward(cfg_t, inp_t)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    P.run_and_check(cfg_t, inp, gpu_inp=inp_t, report=log)


@pytest.mark.parametrize("rows,cols", [(37, 1000), (1100, 264), (64, 8192)])
def test_quantize_rows_fp8_matches_oracle(rows, cols):
    # rows of very different magnitudes, an all-zero row, and ragged widths;
    # up to 1024 rows take the block-per-row kernel, more the wave-per-row one
    g = torch.Generator().manual_seed(5)
    v = torch.randn(rows, cols, generator=g) * torch.exp2(torch.randint(-20, 20, (rows, 1), generator=g).float())
    v[4] = 0.0
    v[6, :cols // 2] *= 1e-4  # values near the E4M3 subnormal range of that row
    src = v.to(torch.bfloat16)
    codes, scales = B.quantize_rows_fp8(src.cuda())
    torch.cuda.synchronize()
    rc, rs = O.quantize_rows_fp8(O.as_f64(synth.host_view(src)))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("name", ["mxfp8_proj", "mxfp8_proj_few"])
def test_mxfp8_projections_with_varied_block_scales(name):
    # x scaled per 32-element block by 2^-6 .. 2^6 (exact in bf16), so
    # neighbouring blocks of every row carry different E8M0 scales and a
    # scale applied to the wrong block of the MFMA shows
    cfg = SMALL[name]
    inp = small_inputs(cfg)
    g = torch.Generator().manual_seed(23)
    f = torch.exp2(torch.randint(-6, 7, (cfg.T, cfg.d // 32), generator=g).float()).repeat_interleave(32, dim=1)
    inp["x"] = (inp["x"].float().cpu() * f).to(torch.bfloat16).cuda()
    log(f"case {name} with varied block scales")
    P.run_and_check(cfg, inp, report=log)


@pytest.mark.parametrize("rows,cols", [(37, 1024), (1100, 256)])
def test_quantize_rows_mxfp8_matches_oracle(rows, cols):
    # blocks of very different magnitudes (2^-40 .. 2^40), an all-zero
    # block, a saturating block and values near the E4M3 subnormal range
    g = torch.Generator().manual_seed(17)
    v = torch.randn(rows, cols, generator=g)
    v = v * torch.exp2(torch.randint(-40, 40, (rows, cols // 32), generator=g).float()).repeat_interleave(32, dim=1)
    v[2, 32:64] = 0.0
    v[3, :32] = torch.linspace(-1, 1, 32) * 0.99
    v[3, 7] = 1.97  # 1.97 * 2^8 = 504: saturates to 448
    v[5, :32] *= 1e-3
    src = v.to(torch.bfloat16)
    codes, scales = B.quantize_rows_mxfp8(src.cuda())
    torch.cuda.synchronize()
    rc, rs = O.quantize_blocks_mxfp8(O.as_f64(synth.host_view(src)))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


# ---- full-size workloads --------------------------------------------------

@pytest.mark.timeout(900)
def test_mid_bf16_full_size():
    cfg = CFG["mid_bf16"]
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_prefill_bf16_full_size():
    cfg = CFG["prefill_bf16"]
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_decode_zipf_full_size():
    cfg = CFG["decode_bf16_zipf"]
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    errs, _, dbg = P.run_and_check(cfg, inp, lazy_experts=True, report=log)
    counts = dbg["counts"].cpu().numpy()
    log(f"experts touched {int((counts > 0).sum())}, expert 0 rows {counts[0]}")
    assert counts[0] == cfg.T  # the largest bias: every token picks expert 0


@pytest.mark.timeout(900)
def test_tiled_experts_full_size_match_row_major():
    for name in ("decode_bf16_zipf", "prefill_bf16"):
        cfg = CFG[name]
        log(f"case tiled full size {cfg}")
        inp = synth.make_inputs(cfg, 0, "cuda")
        ref = B.forward(cfg, inp).clone()
        cfg_t, inp_t = B.pack_experts(cfg, inp)
        out = B.forward(cfg_t, inp_t)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), name
        if name == "decode_bf16_zipf":
            P.run_and_check(cfg_t, inp, lazy_experts=True, report=log, gpu_inp=inp_t)
        del inp, inp_t, ref, out
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_decode_latent_router_full_size():
    cfg = CFG["decode_bf16_zipf"].with_(name="decode_latent_router", router_latent=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_prefill_latent_router_2048_tokens():
    # many-token latent router: its own split-K GEMM (64 tiles of 256 x 256)
    cfg = CFG["prefill_bf16"].with_(name="prefill_latent_router", T=2048, router_latent=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_mid_fp8_shared_full_size():
    cfg = CFG["mid_bf16"].with_(name="mid_fp8_shared", shared_fp8=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_prefill_fp8_shared_full_size():
    cfg = CFG["prefill_bf16"].with_(name="prefill_fp8_shared", shared_fp8=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_decode_standard_moe_full_size():
    # the comparison layer at decode: 128 experts of d -> 2048 -> d, top-6
    cfg = CFG["decode_bf16_zipf"].with_(name="decode_standard_moe", l=8192, E=128, k=6, standard_moe=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_prefill_nvfp4_full_size():
    cfg = CFG["prefill_nvfp4"]
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_prefill_nvfp4_2d_full_size():
    cfg = CFG["prefill_nvfp4"].with_(name="prefill_nvfp4_2d", experts="nvfp4_2d")
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_decode_fp8_projections_full_size():
    # split-K fp8 GEMMs for both projections at d = 8192, 64 tokens
    cfg = CFG["decode_bf16_zipf"].with_(name="decode_fp8_proj", proj_fp8=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    errs, _, dbg = P.run_and_check(cfg, inp, lazy_experts=True, report=log)
    assert int(dbg["counts"].cpu()[0]) == cfg.T


@pytest.mark.timeout(900)
def test_prefill_fp8_projections_2048_tokens():
    cfg = CFG["prefill_bf16"].with_(name="prefill_fp8_proj", T=2048, proj_fp8=True, shared_fp8=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)


@pytest.mark.timeout(900)
def test_decode_mxfp8_projections_full_size():
    cfg = CFG["decode_bf16_zipf"].with_(name="decode_mxfp8_proj", proj_mxfp8=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    errs, _, dbg = P.run_and_check(cfg, inp, lazy_experts=True, report=log)
    assert int(dbg["counts"].cpu()[0]) == cfg.T


@pytest.mark.timeout(900)
def test_prefill_mxfp8_projections_2048_tokens():
    cfg = CFG["prefill_bf16"].with_(name="prefill_mxfp8_proj", T=2048, proj_mxfp8=True, shared_fp8=True)
    log(f"case {cfg}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    P.run_and_check(cfg, inp, lazy_experts=True, report=log)
