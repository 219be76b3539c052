"""CPU oracle of the LatentMoE layer forward -- TEST INFRASTRUCTURE ONLY.

Plain, slow float64 reference of what the layer computes.  Only the test
suite, the package's smoke check and the benchmark's CPU-baseline leg may
import it; the HIP library never does, and this file shares no code,
constants or helpers with it.  numpy's matmul and stable argsort are used as
library steps; everything else is written out from the definitions below.

The layer (sources: the Nemotron 3 overview article, section 2.2 "LatentMoE",
steps 1-3 and the paragraph after its table; the Nemotron 3 Super blog,
section "Latent MoE"; the Nemotron 3 Ultra release news, architecture
paragraph):
  1. z_t = W_down x_t, the token's hidden vector (width d) projected down to
     the latent width l = d/4                                (overview s2.2 step 1)
  2. s_t = W_r x_t + b, router logits over E experts; the router reads x in d
     (the routing gate stays in d per the paragraph after the s2.2 table).
     The pages also place routing in the latent space (s2.2 step 2; Super
     blog, "Latent MoE"): with W_r of width l the router reads the latent
     z_t as the layer stores it (rounded to the activation format), which
     the width of W_r selects
  3. I_t = the k largest logits, ordered by (logit desc, expert id asc);
     Ultra uses E = 512, k = 22                           (release news, architecture)
  4. g_t = softmax over the k selected logits (the gate form is this layer's
     specification; the pages do not give one)
  5. y_{t,j} = W2_e (max(0, W1_e z_t))^2 for e = I_t[j]: each routed expert is
     a ReLU^2 FFN l -> f -> l run in the latent space       (overview s2.2 step 2)
  6. c_t = sum_j g_{t,j} y_{t,j}, then out_t = W_up c_t, back to width d
                                                            (overview s2.2 step 3)
  7. optional shared expert in d: out_t += W_s2 (max(0, W_s1 x_t))^2
                                   (overview s2.2, paragraph after the table).
     With FP8 shared weights (the Ultra release news lists FP8 shared
     experts): W_s1, W_s2 are E4M3 codes times one scale per output row, and
     each of the shared expert's inputs (x_t, then its hidden layer as stored
     in bf16) is quantised per token to E4M3 with scale max|v|/448 before
     its product
  FP8 projections (the Ultra model card, "Model design", keeps the latent
  projections out of NVFP4, in BF16 or MXFP8): either the shared expert's
  scheme (W_down and W_up as E4M3 codes times one scale per output row,
  each input quantised per token), or MXFP8 (OCP microscaling: E4M3
  elements sharing one power-of-two E8M0 scale per 32 consecutive fan-in
  elements, for the weights and for each input row).  The inputs are x
  before W_down and c as stored in bf16 before W_up.
  Without W_down and W_up the same steps describe the standard MoE layer the
  overview compares against (section 2.2 table: 128 experts, top-6, experts
  in the hidden width): z_t = x_t and out_t = c_t (+ shared expert).
  Integer side: counts[e] = #{(t, j): I_t[j] = e}, offsets = exclusive prefix
  sum of counts, perm = stable counting sort of the row-major (t, j) pairs by
  expert, inv = perm^-1.

Precision: all arithmetic in float64 on the exact values of the stored
inputs; the one intermediate taken at its stored precision is the latent z
a latent router reads (the layer stores z before the router reads it).  The
one place floating point decides an integer (the top-k) takes the decision
on float32 logits, the precision the layer stores its logits in; ties in
float32 are broken by the lower expert id.

Data format: bf16 tensors are numpy uint16 arrays of bf16 bit patterns;
fp32 tensors are float32 arrays.  NVFP4 expert weights are byte arrays of
E2M1 codes (two per byte, even element in the low nibble), E4M3 block scales
(one per 16 consecutive fan-in elements, or one per 16 x 16 block of the 2-D
variant) and one fp32 tensor scale per expert matrix (overview s3.1.1, NVFP4
format: E2M1 elements, 16-element micro-blocks, E4M3 block scale; release
news: two-dimensional weight blocks).
"""
from __future__ import annotations

from collections import OrderedDict

import numpy as np


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64.  A bf16 number is the upper half of an
    IEEE-754 binary32 with the lower 16 mantissa bits zero."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """float64 values rounded to the nearest bf16 value (ties to the even
    mantissa), returned as float64.  bf16 keeps the binary32 exponent range
    and 8 significant bits, so this drops the low 45 of the 52 stored
    fraction bits of a float64 with round-to-nearest-even (normal numbers of
    the binary32 range, the only ones the layer produces)."""
    u = np.asarray(v, dtype=np.float64).view(np.uint64)
    drop = np.uint64(45)
    lsb = (u >> drop) & np.uint64(1)
    u = u + (np.uint64((1 << 44) - 1) + lsb)
    u = u & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64)


def store_round(v, like) -> np.ndarray:
    """float64 values rounded to the storage format of the array `like`
    (bf16 bit patterns or float32), returned as float64."""
    if np.asarray(like).dtype == np.uint16:
        return round_to_bf16(v)
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported array dtype {a.dtype}")


def e2m1_value(code) -> np.ndarray:
    """Value of a 4-bit E2M1 code: bit 3 sign, bits 2-1 exponent (bias 1),
    bit 0 mantissa.  Exponent field 0 is subnormal: 0.5 * mantissa."""
    code = np.asarray(code).astype(np.int64)
    sign = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.exp2(e - 1.0) * (1.0 + 0.5 * m))
    return np.where(sign == 1, -mag, mag)


def e4m3_value(byte) -> np.ndarray:
    """Value of an 8-bit E4M3 (FN variant) pattern: bit 7 sign, bits 6-3
    exponent (bias 7), bits 2-0 mantissa; exponent field 0 is subnormal
    2^-6 * m/8; no infinities; exponent 15 with mantissa 7 is NaN."""
    byte = np.asarray(byte).astype(np.int64)
    sign = (byte >> 7) & 1
    e = (byte >> 3) & 15
    m = byte & 7
    mag = np.where(e == 0, np.exp2(-6.0) * (m / 8.0), np.exp2(e - 7.0) * (1.0 + m / 8.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 (FN) code of each value, ties to the even mantissa:
    normal numbers 2^(e-7) (1 + m/8), subnormals 2^-6 m/8.  Magnitudes must
    stay below 464 (the midpoint above the largest finite value 448)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a >= 464.0) or not np.all(np.isfinite(v)):
        raise ValueError("value outside the E4M3 range")
    frac, p = np.frexp(a)                     # a = frac * 2^p, frac in [0.5, 1)
    e = p.astype(np.int64) - 1                # a = (2 frac) * 2^e
    m = np.rint((2.0 * frac - 1.0) * 8.0)     # mantissa steps, ties to even
    carry = m == 8.0
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0.0, m)
    field = e + 7
    sub = field < 1                           # below 2^-6: steps of 2^-9
    q = np.rint(a * 512.0)
    field = np.where(sub, np.where(q == 8.0, 1, 0), field)
    m = np.where(sub, np.where(q == 8.0, 0.0, q), m)
    code = (field.astype(np.int64) << 3) | m.astype(np.int64)
    code = np.where(a == 0.0, 0, code)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def quantize_rows_fp8(v) -> tuple:
    """Per-row E4M3 quantisation of float32-representable values [n][K]:
    scale = max|row| / 448 and code = E4M3(v / scale), both quotients taken in
    float32 (the precision the layer takes this decision in); scale 1 for an
    all-zero row.  Returns (codes uint8 [n][K], scales float32 [n])."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(v32), axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (v32 / scale[:, None]).astype(np.float32)
    return e4m3_encode(q.astype(np.float64)), scale


def e8m0_value(byte) -> np.ndarray:
    """E8M0 scale byte -> float64: 2^(byte - 127); 255 is NaN."""
    b = np.asarray(byte).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def quantize_blocks_mxfp8(v) -> tuple:
    """MXFP8 quantisation of the rows of v [n][K] (K a multiple of 32), per
    block of 32 consecutive elements: shared exponent e = floor(log2 max|v|)
    minus 8 (the largest E4M3 exponent), clamped to [-127, 127], so the
    block's largest magnitude lands in [256, 512) times 2^-e; the scale is
    the E8M0 byte e + 127 (127 for an all-zero block); each element is the
    E4M3 code (nearest, ties to even) of v / 2^e saturated to +-448.  The
    division by a power of two is exact.  Returns (codes uint8 [n][K],
    scales uint8 [n][K/32])."""
    v = np.asarray(v, dtype=np.float64)
    n, K = v.shape
    blocks = v.reshape(n, K // 32, 32)
    amax = np.max(np.abs(blocks), axis=2)
    _, p = np.frexp(amax)                      # amax = f 2^p, f in [0.5, 1)
    e = np.where(amax > 0, p.astype(np.int64) - 1 - 8, 0)
    e = np.clip(e, -127, 127)
    q = np.clip(blocks / np.ldexp(1.0, e)[..., None], -448.0, 448.0)
    codes = e4m3_encode(q).reshape(n, K)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3(code) * E8M0(scale of its 32-element block) for [rows][K]."""
    return e4m3_value(codes) * np.repeat(e8m0_value(scales), 32, axis=-1)


def mxfp8_product(v: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """v W^T with MXFP8 weights W (codes, E8M0 block scales), the rows of v
    quantised to MXFP8 first (quantize_blocks_mxfp8)."""
    qv, sv = quantize_blocks_mxfp8(as_f64(v))
    return mxfp8_dequant(qv, sv) @ mxfp8_dequant(codes, scales).T


def nvfp4_dequant(codes: np.ndarray, scales: np.ndarray, tensor_scale: float) -> np.ndarray:
    """w[r][c] = E2M1(code[r][c]) * E4M3(scale[r][c // 16]) * tensor_scale,
    or with 2-D blocks (one scale per 16 rows x 16 columns, scales
    [R/16][K/16]; the Ultra release news describes the pretrained weights as
    quantised in two-dimensional blocks) E4M3(scale[r // 16][c // 16]).
    The codes and scale bytes are decoded through tables of e2m1_value over
    the 16 codes and e4m3_value over the 256 bytes: the same values, looked
    up instead of recomputed per element."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    e2m1_table = e2m1_value(np.arange(16))
    e4m3_table = e4m3_value(np.arange(256))
    q = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.float64)
    q[..., 0::2] = e2m1_table[codes & 0x0F]
    q[..., 1::2] = e2m1_table[codes >> 4]
    s = np.repeat(e4m3_table[scales], 16, axis=-1)
    if scales.shape[-2] != codes.shape[-2]:
        if scales.shape[-2] * 16 != codes.shape[-2]:
            raise ValueError("block scales neither per row nor per 16 rows")
        s = np.repeat(s, 16, axis=-2)
    return q * s * float(tensor_scale)


# --------------------------------------------------------------------------
# Expert weights
# --------------------------------------------------------------------------

class ExpertWeights:
    """float64 W1_e [f][l] and W2_e [l][f], decoded on demand from the input
    dict (dense stacks 'W1'/'W2', or NVFP4 '<W>_codes', '<W>_scales', '<W>_ts').
    Decoded experts are memoised (a cache of decoded values, not a change of
    arithmetic)."""

    def __init__(self, inp: dict, cache_size: int = 64):
        self.inp = inp
        self.nvfp4 = inp.get("W1_codes") is not None
        self.cache: "OrderedDict[int, tuple]" = OrderedDict()
        self.cache_size = cache_size

    def _decode(self, which: str, e: int) -> np.ndarray:
        if self.nvfp4:
            return nvfp4_dequant(self.inp[which + "_codes"][e], self.inp[which + "_scales"][e],
                                 float(np.asarray(self.inp[which + "_ts"])[e]))
        return as_f64(self.inp[which][e])

    def __call__(self, e: int):
        e = int(e)
        if e in self.cache:
            self.cache.move_to_end(e)
            return self.cache[e]
        w = (self._decode("W1", e), self._decode("W2", e))
        self.cache[e] = w
        if len(self.cache) > self.cache_size:
            self.cache.popitem(last=False)
        return w


# --------------------------------------------------------------------------
# The steps
# --------------------------------------------------------------------------

def down_project(x: np.ndarray, W_down: np.ndarray) -> np.ndarray:
    """Step 1: z_t = W_down x_t for every row t of x.  [n][d] -> [n][l]."""
    return as_f64(x) @ as_f64(W_down).T


def fp8_product(v: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """v W^T for E4M3 weights W = codes times one scale per output row, with
    the rows of v quantised per row to E4M3 first (quantize_rows_fp8): the
    product of the decoded codes, times the row scale of v and the column
    scale of W."""
    qv, sv = quantize_rows_fp8(as_f64(v))
    sw = np.asarray(scales, dtype=np.float64)
    return (e4m3_value(qv) @ e4m3_value(codes).T) * sv.astype(np.float64)[:, None] * sw[None, :]


def project(v: np.ndarray, inp: dict, name: str) -> np.ndarray:
    """v W^T for the projection weight inp[name] (W_down or W_up) in its
    stored format: bf16 / fp32 values, or E4M3 codes (uint8) with per-row
    fp32 scales under name + '_scale', or MXFP8 codes with E8M0 block scales
    (uint8 [rows][K/32]) under name + '_mxscale'."""
    W = np.asarray(inp[name])
    if W.dtype == np.uint8 and inp.get(name + "_mxscale") is not None:
        return mxfp8_product(v, W, np.asarray(inp[name + "_mxscale"]))
    if W.dtype == np.uint8:
        return fp8_product(v, W, inp[name + "_scale"])
    return as_f64(v) @ as_f64(W).T


def router_logits(x: np.ndarray, W_r: np.ndarray, b_r=None) -> np.ndarray:
    """Step 2: s_t = W_r x_t (+ b) in float64, returned as float32 (the
    precision in which the top-k decision is taken)."""
    s = as_f64(x) @ as_f64(W_r).T
    if b_r is not None:
        s = s + as_f64(b_r)[None, :]
    return s.astype(np.float32)


def select_topk(s: np.ndarray, k: int) -> np.ndarray:
    """Step 3: per row, the k expert ids with the largest logits, in the order
    (logit desc, id asc).  A stable sort of -s keeps equal logits in id order."""
    order = np.argsort(-np.asarray(s, dtype=np.float32), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gate_weights(s: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Step 4: g_{t,j} = exp(s_{t,I_j}) / sum_j' exp(s_{t,I_j'}) over the k
    selected logits (shifted by the row's top logit for range)."""
    sel = np.take_along_axis(np.asarray(s, dtype=np.float64), idx.astype(np.int64), axis=1)
    w = np.exp(sel - sel[:, :1])
    return w / w.sum(axis=1, keepdims=True)


def expert_ffn(z_t: np.ndarray, W1_e: np.ndarray, W2_e: np.ndarray) -> np.ndarray:
    """Step 5: y = W2_e (max(0, W1_e z_t))^2, a ReLU^2 FFN in the latent space."""
    h = np.maximum(W1_e @ z_t, 0.0) ** 2
    return W2_e @ h


def permutation(idx: np.ndarray, E: int):
    """Integer side: counts [E], offsets [E+1] (exclusive prefix sum with the
    total at the end), perm [n*k] (stable sort of the flat pair index
    t*k + j by expert) and inv [n*k] = perm^-1, all int32."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable")
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
            inv.astype(np.int32))


def router_input(x: np.ndarray, inp: dict) -> np.ndarray:
    """What the router reads for the rows x: x itself when W_r is [E][d], or
    the latent z = W_down x as stored (rounded to x's format) when W_r is
    [E][l]."""
    width = np.asarray(inp["W_r"]).shape[1]
    if width == np.asarray(x).shape[1]:
        return x
    if width != np.asarray(inp["W_down"]).shape[0]:
        raise ValueError("W_r width is neither d nor l")
    return store_round(project(x, inp, "W_down"), x)


def route(inp: dict, k: int):
    """Steps 2-4 for every token: logits (float32), idx, gates (float64)."""
    s = router_logits(router_input(inp["x"], inp), inp["W_r"], inp.get("b_r"))
    idx = select_topk(s, k)
    return s, idx, gate_weights(s, idx)


def forward(inp: dict, k: int, tokens=None, experts: ExpertWeights = None, idx=None) -> dict:
    """The layer forward for the given token rows (all rows by default).

    Returns float64 z [n][l], c [n][l], out [n][d], and the routing of those
    rows: logits (float32) [n][E], idx [n][k], gate [n][k].  Tokens are
    independent (no capacity limit, every routed pair is computed), so any
    subset of rows gives the same values as the full call for those rows.

    idx, if given ([n][k] expert ids of those rows), replaces the top-k
    selection of step 3: the rows are evaluated with those experts, gated by
    the softmax over their own logits (step 4).  This evaluates a row with
    another valid selection of its top-k where logits tie or nearly tie.
    """
    x = np.asarray(inp["x"])
    if tokens is not None:
        x = x[np.asarray(tokens)]
    experts = experts or ExpertWeights(inp)
    # a standard MoE (no W_down / W_up, experts in d) routes and computes on x
    z = project(x, inp, "W_down") if inp.get("W_down") is not None else as_f64(x)
    s = router_logits(router_input(x, inp), inp["W_r"], inp.get("b_r"))
    idx = select_topk(s, k) if idx is None else np.asarray(idx, dtype=np.int32).reshape(len(x), k)
    g = gate_weights(s, idx)
    n, l = z.shape
    c = np.zeros((n, l), dtype=np.float64)
    for t in range(n):
        for j in range(k):
            W1_e, W2_e = experts(idx[t, j])
            c[t] += g[t, j] * expert_ffn(z[t], W1_e, W2_e)
    return dict(z=z, logits=s, idx=idx, gate=g, c=c, out=up_project(c, x, inp))


def forward_batched(inp: dict, k: int, idx=None, experts: ExpertWeights = None) -> dict:
    """forward() for every token, with step 5 taken one expert at a time over
    all the rows routed to it: H = max(0, Z_e W1_e^T)^2 and Y = H W2_e^T for
    the stacked latent rows Z_e of that expert's tokens, then each row added
    into its token's c with its gate.  The same arithmetic as forward(),
    grouped by expert instead of by token (a token holds each expert at
    most once), so only the order of the float64 additions into c differs.
    idx, if given ([T][k]), replaces the top-k selection as in forward()."""
    x = np.asarray(inp["x"])
    experts = experts or ExpertWeights(inp, cache_size=1)
    z = project(x, inp, "W_down") if inp.get("W_down") is not None else as_f64(x)
    s = router_logits(router_input(x, inp), inp["W_r"], inp.get("b_r"))
    idx = select_topk(s, k) if idx is None else np.asarray(idx, dtype=np.int32).reshape(len(x), k)
    g = gate_weights(s, idx)
    c = np.zeros(z.shape, dtype=np.float64)
    for e in np.unique(idx):
        t, j = np.nonzero(idx == e)
        W1_e, W2_e = experts(e)
        H = np.maximum(z[t] @ W1_e.T, 0.0) ** 2
        c[t] += g[t, j][:, None] * (H @ W2_e.T)
    return dict(z=z, logits=s, idx=idx, gate=g, c=c, out=up_project(c, x, inp))


def up_project(c: np.ndarray, x: np.ndarray, inp: dict) -> np.ndarray:
    """Step 6's up-projection out = W_up c (c itself without W_up: the
    standard MoE layer), plus the shared expert of step 7 if there is one.
    An E4M3 W_up reads c as stored (rounded to x's format)."""
    if inp.get("W_up") is None:
        out = c.copy()
    elif np.asarray(inp["W_up"]).dtype == np.uint8:
        out = project(store_round(c, x), inp, "W_up")
    else:
        out = project(c, inp, "W_up")
    if inp.get("W_s1") is not None:
        out = out + shared_expert(x, inp)
    return out


def shared_expert(x: np.ndarray, inp: dict) -> np.ndarray:
    """Step 7 for the rows x: W_s2 (max(0, W_s1 x))^2; with E4M3 weights
    (uint8 codes, per-row scales) both products take per-token E4M3 inputs:
    x, then the hidden layer as stored (bf16)."""
    W1, W2 = np.asarray(inp["W_s1"]), np.asarray(inp["W_s2"])
    if W1.dtype != np.uint8:
        hs = np.maximum(as_f64(x) @ as_f64(W1).T, 0.0) ** 2
        return hs @ as_f64(W2).T
    hs = round_to_bf16(np.maximum(fp8_product(x, W1, inp["W_s1_scale"]), 0.0) ** 2)
    return fp8_product(hs, W2, inp["W_s2_scale"])
