"""Seeded synthetic inputs for the LatentMoE layer forward.

This module only draws random tensors and stores them in the formats the
layer consumes (bf16, fp32, NVFP4 codes).  It contains none of the layer's
arithmetic: no projection, routing, expert or combine step.  Both the HIP
path and the CPU oracle read the bytes produced here.

Recipe (one stream per tensor, so every tensor is reproducible alone):
  * generator = torch.Generator(device).manual_seed(seed * 1000 + tensor_id)
    with tensor_id: x=0, W_down=1, W_r=2, W1=3, W2=4, W_up=5, W_s1=6,
    W_s2=7, W1 block scales=8, W2 block scales=9.
  * x ~ N(0, 1); every weight ~ N(0, 1/fan_in) with fan_in the input width
    of that matrix (d for W_down, W_r, W_s1; l for W1, W_up and a latent
    router's W_r; f for W2; f_s for W_s2).  Draws are fp32, then rounded to
    bf16 (round to nearest even) for bf16 tensors.
  * FP8 shared-expert weights (shared_fp8) and FP8 projection weights
    (proj_fp8, W_down and W_up): the same fp32 draws, stored as E4M3 codes
    with one fp32 scale per output row (max |row| / 448).  MXFP8 projection
    weights (proj_mxfp8): E4M3 codes with one E8M0 scale per 32 fan-in
    elements, 2^(floor(log2 max|block|) - 8), codes saturated to +-448.
  * The skewed-routing workload adds a per-expert router bias
    b_e = 2 * log(1 / (e + 1)), stored in fp32.
  * NVFP4 expert weights: W ~ N(0, 1/fan_in) in fp32, a block scale
    s ~ U[0.5, 2] per 16 consecutive fan-in elements rounded to the E4M3
    grid, a per-matrix fp32 tensor scale ts = 1/sqrt(fan_in), and the
    element code is W / (s * ts) clamped to [-6, 6] and rounded to the
    nearest E2M1 value (ties to the even mantissa).  Two codes per byte,
    the even element in the low nibble.  The 2-D variant (nvfp4_2d) draws
    one block scale per 16 x 16 block (16 weight rows by 16 fan-in
    elements) instead of per 16 fan-in elements of one row.

The random draws depend on the torch device's generator: CPU and GPU
streams differ.  Whatever is drawn, both sides of a comparison read the
same bytes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

TENSOR_IDS = dict(x=0, W_down=1, W_r=2, W1=3, W2=4, W_up=5, W_s1=6, W_s2=7,
                  W1_scale=8, W2_scale=9)


@dataclasses.dataclass(frozen=True)
class LayerDims:
    """Shape of one LatentMoE layer call.

    T tokens, hidden width d, latent width l (= d/4), E routed experts, top-k,
    expert intermediate width f, shared-expert intermediate width f_s
    (0 = no shared expert).  act is the activation/storage dtype ('f32' or
    'bf16'); experts is the routed-expert weight format ('f32', 'bf16',
    'nvfp4' or 'nvfp4_2d'); zipf_bias adds the skewed router bias; router_latent makes the
    router read the latent z (W_r [E][l]) instead of x (W_r [E][d]);
    shared_fp8 stores the shared expert's weights as E4M3 codes with one fp32
    scale per output row; standard_moe is the comparison layer without the
    latent projections (l = d, no W_down / W_up); proj_fp8 stores W_down and
    W_up that way too; proj_mxfp8 stores them as MXFP8 (E4M3 with an E8M0
    scale per 32 fan-in elements) instead.
    """
    name: str
    T: int
    d: int
    l: int
    E: int
    k: int
    f: int
    f_s: int
    act: str
    experts: str
    zipf_bias: bool = False
    router_latent: bool = False
    shared_fp8: bool = False
    standard_moe: bool = False
    proj_fp8: bool = False
    proj_mxfp8: bool = False

    def with_(self, **kw) -> "LayerDims":
        return dataclasses.replace(self, **kw)

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs of one forward: projections, router, experts, shared."""
        T, d, l, E, k, f, fs = self.T, self.d, self.l, self.E, self.k, self.f, self.f_s
        router_in = l if self.router_latent else d
        proj = 0.0 if self.standard_moe else 4.0 * T * d * l  # down- and up-projection
        return proj + 2.0 * T * router_in * E + 4.0 * T * k * l * f + 4.0 * T * d * fs


# The five workloads.  Sizes follow the Ultra layer (d = 8192, 512 experts,
# top-22) and two smaller variants; l = d/4 everywhere.
CONFIGS: Dict[str, LayerDims] = {
    "tiny_f32": LayerDims("tiny_f32", T=64, d=256, l=64, E=16, k=4, f=128, f_s=0,
                          act="f32", experts="f32"),
    "mid_bf16": LayerDims("mid_bf16", T=2048, d=4096, l=1024, E=128, k=8, f=1024, f_s=4096,
                          act="bf16", experts="bf16"),
    "prefill_bf16": LayerDims("prefill_bf16", T=8192, d=8192, l=2048, E=512, k=22, f=2048,
                              f_s=8192, act="bf16", experts="bf16"),
    "decode_bf16_zipf": LayerDims("decode_bf16_zipf", T=64, d=8192, l=2048, E=512, k=22,
                                  f=2048, f_s=0, act="bf16", experts="bf16", zipf_bias=True),
    "prefill_nvfp4": LayerDims("prefill_nvfp4", T=8192, d=8192, l=2048, E=512, k=22, f=2048,
                               f_s=0, act="bf16", experts="nvfp4"),
}


def _gen(device, seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + TENSOR_IDS[name])
    return g


def _normal(shape, std: float, g: torch.Generator, device, out_dtype) -> torch.Tensor:
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(out_dtype)


def _act_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


# --- NVFP4 encoding (input preparation only; the layer decodes) ------------

# E2M1 magnitudes indexed by the 3-bit magnitude code, and the midpoints
# between neighbours (used for round-to-nearest).
_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _round_to_e4m3_grid(s: torch.Tensor) -> torch.Tensor:
    """Round positive values in [2^-6, 448] to the E4M3 grid (nearest, ties even)."""
    e = torch.floor(torch.log2(s))
    step = torch.exp2(e - 3)
    return torch.round(s / step) * step


def _e4m3_bytes(s: torch.Tensor) -> torch.Tensor:
    """Encode positive normal E4M3-grid values (as produced above) into bytes."""
    e = torch.floor(torch.log2(s))
    mant = torch.round((s / torch.exp2(e) - 1.0) * 8.0)
    return ((e + 7).to(torch.int32) * 8 + mant.to(torch.int32)).to(torch.uint8)


def _e2m1_codes(v: torch.Tensor) -> torch.Tensor:
    """Nearest E2M1 code (ties to even mantissa) for v already clamped to [-6, 6]."""
    a = v.abs()
    code = torch.zeros_like(a, dtype=torch.int32)
    for i, m in enumerate(_E2M1_MIDPOINTS):
        # above the midpoint -> the upper neighbour; at the midpoint only when the
        # upper neighbour's code is even (i + 1 even).
        up = (a > m) | ((a == m) & ((i + 1) % 2 == 0))
        code += up.to(torch.int32)
    return code | ((v < 0).to(torch.int32) << 3)


def _nvfp4_quantize(W: torch.Tensor, scale_u: torch.Tensor, fan_in: int, rows_per_scale: int = 1):
    """W [R][K] fp32, scale_u [R/rows_per_scale][K/16] in [0.5, 2] ->
    (codes [R][K/2] u8, scales [R/rows_per_scale][K/16] u8, ts)."""
    ts = torch.tensor(1.0 / math.sqrt(fan_in), dtype=torch.float32).item()
    s = _round_to_e4m3_grid(scale_u)
    v = W / (s.repeat_interleave(16, dim=-1).repeat_interleave(rows_per_scale, dim=-2) * ts)
    v = v.clamp_(-6.0, 6.0)
    code = _e2m1_codes(v)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).to(torch.uint8)
    return packed, _e4m3_bytes(s), ts


def _expert_stack(cfg: LayerDims, which: str, seed: int, device, chunk: int = 32):
    """Routed expert weights W1 [E][f][l] or W2 [E][l][f] in cfg.experts format."""
    E = cfg.E
    rows, fan_in = (cfg.f, cfg.l) if which == "W1" else (cfg.l, cfg.f)
    std = 1.0 / math.sqrt(fan_in)
    g = _gen(device, seed, which)
    if cfg.experts in ("f32", "bf16"):
        dt = _act_dtype(cfg.experts)
        out = torch.empty((E, rows, fan_in), dtype=dt, device=device)
        for e0 in range(0, E, chunk):
            e1 = min(E, e0 + chunk)
            out[e0:e1] = _normal((e1 - e0, rows, fan_in), std, g, device, dt)
        return {which: out}
    assert cfg.experts in ("nvfp4", "nvfp4_2d")
    assert fan_in % 16 == 0
    rps = 16 if cfg.experts == "nvfp4_2d" else 1  # weight rows per block scale
    assert rows % rps == 0
    gs = _gen(device, seed, which + "_scale")
    codes = torch.empty((E, rows, fan_in // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((E, rows // rps, fan_in // 16), dtype=torch.uint8, device=device)
    ts_all = torch.empty((E,), dtype=torch.float32, device=device)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        W = torch.randn((e1 - e0, rows, fan_in), generator=g, device=device, dtype=torch.float32).mul_(std)
        su = torch.rand((e1 - e0, rows // rps, fan_in // 16), generator=gs, device=device,
                        dtype=torch.float32).mul_(1.5).add_(0.5)
        c, s, ts = _nvfp4_quantize(W, su, fan_in, rps)
        codes[e0:e1] = c
        scales[e0:e1] = s
        ts_all[e0:e1] = ts
        del W, su, c, s
    return {which + "_codes": codes, which + "_scales": scales, which + "_ts": ts_all}


def make_inputs(cfg: LayerDims, seed: int = 0, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """All inputs of one layer call, as torch tensors on `device`."""
    dev = torch.device(device)
    act = _act_dtype(cfg.act)
    T, d, l, E, f, fs = cfg.T, cfg.d, cfg.l, cfg.E, cfg.f, cfg.f_s
    inp: Dict[str, Optional[torch.Tensor]] = {}
    inp["x"] = _normal((T, d), 1.0, _gen(dev, seed, "x"), dev, act)
    inp["W_down"] = (None if cfg.standard_moe
                     else _proj_weight(cfg, (l, d), d, _gen(dev, seed, "W_down"), dev, act, inp, "W_down"))
    r_in = l if cfg.router_latent else d
    inp["W_r"] = _normal((E, r_in), 1.0 / math.sqrt(r_in), _gen(dev, seed, "W_r"), dev, act)
    if cfg.zipf_bias:
        e = torch.arange(E, dtype=torch.float64)
        inp["b_r"] = (2.0 * torch.log(1.0 / (e + 1.0))).to(torch.float32).to(dev)
    else:
        inp["b_r"] = None
    inp.update(_expert_stack(cfg, "W1", seed, dev))
    inp.update(_expert_stack(cfg, "W2", seed, dev))
    inp["W_up"] = (None if cfg.standard_moe
                   else _proj_weight(cfg, (d, l), l, _gen(dev, seed, "W_up"), dev, act, inp, "W_up"))
    if fs > 0 and cfg.shared_fp8:
        for name, shape, fan_in in (("W_s1", (fs, d), d), ("W_s2", (d, fs), fs)):
            W = _normal(shape, 1.0 / math.sqrt(fan_in), _gen(dev, seed, name), dev, torch.float32)
            inp[name], inp[name + "_scale"] = _fp8_rows(W)
    elif fs > 0:
        inp["W_s1"] = _normal((fs, d), 1.0 / math.sqrt(d), _gen(dev, seed, "W_s1"), dev, act)
        inp["W_s2"] = _normal((d, fs), 1.0 / math.sqrt(fs), _gen(dev, seed, "W_s2"), dev, act)
    else:
        inp["W_s1"] = None
        inp["W_s2"] = None
    return inp


def _proj_weight(cfg: LayerDims, shape, fan_in: int, gen, dev, act, inp, name: str):
    """A projection weight in the activation dtype, or as E4M3 codes (its
    per-row scales stored under name + '_scale') with proj_fp8."""
    if cfg.proj_mxfp8:
        codes, inp[name + "_mxscale"] = _mxfp8_rows(_normal(shape, 1.0 / math.sqrt(fan_in), gen, dev,
                                                            torch.float32))
        return codes
    if not cfg.proj_fp8:
        return _normal(shape, 1.0 / math.sqrt(fan_in), gen, dev, act)
    codes, inp[name + "_scale"] = _fp8_rows(_normal(shape, 1.0 / math.sqrt(fan_in), gen, dev, torch.float32))
    return codes


def _mxfp8_rows(W: torch.Tensor):
    """fp32 W [rows][K] -> (E4M3 codes uint8 [rows][K], E8M0 scale bytes
    uint8 [rows][K/32]): per 32 consecutive elements e = floor(log2 max|w|)
    - 8 (clamped to [-127, 127]; 0 for an all-zero block), codes = torch's
    float8_e4m3fn cast of w / 2^e saturated to +-448."""
    rows, K = W.shape
    b = W.reshape(rows, K // 32, 32)
    amax = b.abs().amax(dim=2)
    _, p = torch.frexp(amax)
    e = torch.where(amax > 0, p - 9, torch.zeros_like(p)).clamp(-127, 127)
    q = (b / torch.ldexp(torch.ones_like(amax), e)[..., None]).clamp(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(rows, K)
    return codes.contiguous(), (e + 127).to(torch.uint8).contiguous()


def _fp8_rows(W: torch.Tensor):
    """fp32 W [rows][cols] -> (E4M3 codes as uint8, fp32 scale per row):
    scale = max|row| / 448, code = E4M3(w / scale) by torch's float8_e4m3fn
    cast (round to nearest even)."""
    amax = W.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (W / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def host_view(t: Optional[torch.Tensor]):
    """numpy copy of a tensor in the layout the oracle reads: bf16 as uint16 bits."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view("uint16")
    return t.cpu().numpy()


class LazyExperts:
    """Index-on-demand host copy of an expert stack [E][...] (for large stacks
    that stay on the device: only the experts a check touches are copied)."""

    def __init__(self, t: torch.Tensor):
        self._t = t
        self.shape = tuple(t.shape)
        self._cache = {}

    def __len__(self):
        return self.shape[0]

    def __getitem__(self, e):
        e = int(e)
        if e not in self._cache:
            self._cache[e] = host_view(self._t[e])
        return self._cache[e]
