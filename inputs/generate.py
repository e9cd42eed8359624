"""Seeded generators for the window-attention workloads.

Workload shapes stand in for the pages' measured settings (no dataset or trained
weights are used anywhere):

* FlashSwin-T stage 1 at 256 px and patch 4 is a 64x64 token grid with C = 96 = 3 heads
  x 32; patch 2 makes it 128x128 (FlashSwin page, efficiency and accuracy results).
* SST super-resolution windows reach 96x96 tokens (RIB/SST page, key contributions).

Q, K, V are i.i.d. N(0, 1) drawn in float32 and rounded once to bfloat16 (round to
nearest even) for the bf16 workloads; the arrays returned are float32 holding exactly
those bf16 values, so the oracle and the device see identical numbers.

Learned-parameter inputs:

* ``theta_table``: theta = exp(omega) per rotation pair, omega from the geometric RoPE
  schedule (FlashSwin page, "How it works", second change: frequencies are
  parameterised as exp(omega) and initialised from the standard geometric schedule),
  optionally perturbed by N(0, sigma^2) noise.  The default ("shared") reading gives the
  y half and the x half the same d/4 frequencies, stored as a d/2-entry table per head.
* ``rib_factors``: the rank-r bias factors U, V of the RIB page (section 2.1): window-local
  token coordinates -> Fourier features -> small seeded MLP -> (U, V).  This is an input
  generator, not part of what the operator computes.
* ``block_gate``: per-block gate values in [0, 1] for the gated local path (HSMLA page,
  section 2: a learned gate per spatial block, about 30% of the blocks above the threshold).
  The gate network itself is a learned model part; the synthetic gates are i.i.d. uniform,
  so a threshold tau selects a fraction 1 - tau of the blocks in expectation.
* ``cla_params``: seeded weights of the convolutional gate (RIB/SST page, section 2.2): a
  3x3 depth-wise kernel per channel ~ N(0, 1/9), a C x C point-wise matrix ~ N(0, 1/C), and
  biases ~ N(0, 0.1^2), so the gate logits of an N(0, 1) input are O(1).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    dtype: str          # "bf16" or "fp32"
    B: int
    Hg: int
    Wg: int
    M: int
    shift: int
    H: int
    d: int
    r: int              # bias rank (0 = no bias)
    rope: bool
    omega_noise: float  # std of the N(0, s^2) perturbation of omega
    seed: int           # base seed; q/k/v use seed, omega noise seed+1000, MLP seed+2000

    @property
    def tokens(self) -> int:
        return self.B * self.Hg * self.Wg

    @property
    def N(self) -> int:
        return self.M * self.M

    def dense_flops(self) -> float:
        """4 * T * N * d * H: QK^T plus PV over every (query, key) pair of each window."""
        return 4.0 * self.tokens * self.N * self.d * self.H

    def io_bytes(self) -> int:
        """q, k, v read once and out written once."""
        esize = 2 if self.dtype == "bf16" else 4
        return 4 * self.tokens * self.H * self.d * esize


def _cfg(name, dtype, B, Hg, Wg, M, shift, H, d, r, rope, noise, seed):
    return WorkloadConfig(name, dtype, B, Hg, Wg, M, shift, H, d, r, rope, noise, seed)


# The workloads: a tiny fp32 case, a Swin-T stage-1-like layer, a large-window layer,
# the dense patch-2 grid at M = 32 (plus its M sweep) and the SR-style M = 96 layer with
# a rank-16 bias.
CONFIGS = {
    "tiny_fp32": _cfg("tiny_fp32", "fp32", 1, 16, 16, 8, 0, 2, 32, 0, True, 0.0, 1001),
    "swin_t_m8": _cfg("swin_t_m8", "bf16", 64, 64, 64, 8, 4, 3, 32, 0, True, 0.1, 1002),
    "large_m32": _cfg("large_m32", "bf16", 64, 64, 64, 32, 16, 3, 32, 0, True, 0.1, 1003),
    "dense_p2_m32": _cfg("dense_p2_m32", "bf16", 16, 128, 128, 32, 16, 3, 32, 0, True, 0.1, 1004),
    "dense_p2_m16": _cfg("dense_p2_m16", "bf16", 16, 128, 128, 16, 8, 3, 32, 0, True, 0.1, 1004),
    "dense_p2_m8": _cfg("dense_p2_m8", "bf16", 16, 128, 128, 8, 4, 3, 32, 0, True, 0.1, 1004),
    "sr_m96_rib": _cfg("sr_m96_rib", "bf16", 8, 192, 192, 96, 0, 6, 32, 16, False, 0.0, 1005),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    NaN stays NaN; values beyond the bf16 range round to +-inf as IEEE rounding does.  The
    32-bit sum cannot wrap for a non-NaN input (the largest pattern, -inf = 0xFF800000, plus
    0x8000 stays below 2^32).
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    bits = a.view(np.uint32)
    rounded = bits + (np.uint32(0x7FFF) + ((bits >> 16) & np.uint32(1)))
    rounded &= np.uint32(0xFFFF0000)
    out = rounded.view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.nan
    return out.reshape(a.shape)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def qkv(shape, seed: int, dtype: str = "bf16"):
    """Three i.i.d. N(0,1) tensors of ``shape`` ([B, Hg, Wg, H, d]), drawn in the order q, k, v."""
    rng = _rng(seed)
    out = []
    for _ in range(3):
        t = rng.standard_normal(size=shape, dtype=np.float32)
        out.append(round_bf16(t) if dtype == "bf16" else t)
    return tuple(out)


def omega_schedule(H: int, d: int, shared: bool = True) -> np.ndarray:
    """Initial log-frequencies omega per head, float64.

    shared=True: d/4 values per head (one set used by both axes), omega_j = -(4j/d) ln 10000,
    i.e. the geometric base-10000 schedule of a rotary subspace of d/2 dimensions.
    shared=False: d/2 values, omega_j = -(2j/d) ln 10000 (the 1D schedule over all d dims).
    """
    n = d // 4 if shared else d // 2
    step = 4.0 / d if shared else 2.0 / d
    w = -np.arange(n, dtype=np.float64) * step * math.log(10000.0)
    return np.broadcast_to(w, (H, n)).copy()


def theta_table(H: int, d: int, noise_std: float = 0.0, seed: int = 0, shared: bool = True) -> np.ndarray:
    """Per-rotation-pair frequencies theta[h][j], j in [0, d/2), as float32.

    Pairs j < d/4 rotate the first half of the head dimension (y), pairs j >= d/4 the
    second half (x).  With shared=True both halves use the same theta = exp(omega).
    """
    w = omega_schedule(H, d, shared)
    if noise_std > 0:
        w = w + _rng(seed).normal(0.0, noise_std, size=w.shape)
    th = np.exp(w)
    if shared:
        th = np.concatenate([th, th], axis=1)
    return th.astype(np.float32)


def _gelu_erf(x: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def rib_factors(H: int, M: int, r: int, seed: int, dtype: str = "bf16", n_freq: int = 4, hidden: int = 64):
    """Rank-r bias factors U, V of shape [H, M*M, r] for window-local coordinates.

    Coordinates (row, col) in [0, M) are mapped to [-1, 1]; the features are
    sin/cos(2^k pi yhat), sin/cos(2^k pi xhat) for k < n_freq (16 features for n_freq=4);
    a seeded two-layer MLP (hidden 64, exact-erf GELU, weights N(0, 1/fan_in), zero
    biases) maps them to 2*H*r outputs, split into U[h] and V[h].  Computed in float64,
    then rounded to the workload dtype.
    """
    n = np.arange(M * M)
    rr = (n // M).astype(np.float64)
    cc = (n % M).astype(np.float64)
    den = max(M - 1, 1)
    yh = 2.0 * rr / den - 1.0
    xh = 2.0 * cc / den - 1.0
    feats = []
    for kk in range(n_freq):
        f = (2.0 ** kk) * math.pi
        feats += [np.sin(f * yh), np.cos(f * yh), np.sin(f * xh), np.cos(f * xh)]
    F = np.stack(feats, axis=1)                                  # [N, 4*n_freq]
    rng = _rng(seed)
    W1 = rng.normal(0.0, 1.0 / math.sqrt(F.shape[1]), size=(F.shape[1], hidden))
    W2 = rng.normal(0.0, 1.0 / math.sqrt(hidden), size=(hidden, 2 * H * r))
    hdn = _gelu_erf(F @ W1)
    o = hdn @ W2                                                 # [N, 2*H*r]
    U = o[:, : H * r].reshape(M * M, H, r).transpose(1, 0, 2)
    V = o[:, H * r:].reshape(M * M, H, r).transpose(1, 0, 2)
    U = np.ascontiguousarray(U.astype(np.float32))
    V = np.ascontiguousarray(V.astype(np.float32))
    if dtype == "bf16":
        U, V = round_bf16(U), round_bf16(V)
    return U, V


@dataclasses.dataclass(frozen=True)
class GatedConfig:
    """A workload of the gated local path: the token grid, heads, window w, threshold tau
    and the denominator guard eps of the linear attention."""
    name: str
    B: int
    Hg: int
    Wg: int
    H: int
    d: int
    w: int
    tau: float
    eps: float
    seed: int           # q/k/v use seed, the gate seed+3000, the base output seed+4000

    @property
    def tokens(self) -> int:
        return self.B * self.Hg * self.Wg

    @property
    def blocks(self) -> int:
        return self.B * (self.Hg // self.w) * (self.Wg // self.w)


# The dense patch-2 grid with 8x8 and 16x16 local windows, 30% of the blocks selected.
GATED_CONFIGS = {
    "gated_p2_w8": GatedConfig("gated_p2_w8", 16, 128, 128, 3, 32, 8, 0.7, 1e-6, 1006),
    "gated_p2_w16": GatedConfig("gated_p2_w16", 16, 128, 128, 3, 32, 16, 0.7, 1e-6, 1006),
}


def block_gate(B: int, nWy: int, nWx: int, seed: int) -> np.ndarray:
    """Gate values in [0, 1) per block, [B][nWy][nWx] float32, i.i.d. uniform."""
    return _rng(seed).random(size=(B, nWy, nWx), dtype=np.float32)


def make_gated_inputs(cfg: GatedConfig, batch: int | None = None):
    """q, k, v (bf16-exact float32), the block gate and a base output ~ N(0, 1) (float32)."""
    B = cfg.B if batch is None else batch
    shape = (B, cfg.Hg, cfg.Wg, cfg.H, cfg.d)
    q, k, v = qkv(shape, cfg.seed, "bf16")
    gate = block_gate(B, cfg.Hg // cfg.w, cfg.Wg // cfg.w, cfg.seed + 3000)
    base = _rng(cfg.seed + 4000).standard_normal(size=shape, dtype=np.float32)
    return dict(q=q, k=k, v=v, gate=gate, base=base)


@dataclasses.dataclass(frozen=True)
class StackConfig:
    """A stack of window-attention layers with a per-layer window schedule (RIB/SST page,
    section 2.3), the convolutional gate on every layer's output (section 2.2) and a rank-r
    bias per layer (section 2.1).  ``layers`` lists (M, shift) per layer."""
    name: str
    B: int
    Hg: int
    Wg: int
    H: int
    d: int
    layers: tuple
    r: int
    seed: int

    @property
    def tokens(self) -> int:
        return self.B * self.Hg * self.Wg

    @property
    def C(self) -> int:
        return self.H * self.d


# The SR-style grid (8 x 192 x 192 tokens, 6 heads x 32) through six layers whose windows
# cycle 16, 32, 64, shifted on every second layer, each with a rank-16 bias and the gate.
STACK_CONFIGS = {
    "sst_cycle_sr": StackConfig("sst_cycle_sr", 8, 192, 192, 6, 32,
                                ((16, 0), (32, 16), (64, 0), (16, 8), (32, 0), (64, 32)), 16, 1007),
}


def make_stack_layer(cfg: StackConfig, layer: int, batch: int | None = None):
    """Inputs of one layer of a stack: q, k, v and the layer input x (bf16-exact float32), the
    gate's convolution weights, and the bias factors for the layer's window side."""
    B = cfg.B if batch is None else batch
    M = cfg.layers[layer][0]
    seed = cfg.seed + 10 * layer
    q, k, v = qkv((B, cfg.Hg, cfg.Wg, cfg.H, cfg.d), seed, "bf16")
    x = round_bf16(_rng(seed + 4).standard_normal(size=(B, cfg.Hg, cfg.Wg, cfg.C), dtype=np.float32))
    w_dw, b_dw, w_pw, b_pw = cla_params(cfg.C, seed + 5)
    U, V = rib_factors(cfg.H, M, cfg.r, seed + 7, "bf16") if cfg.r else (None, None)
    return dict(q=q, k=k, v=v, x=x, w_dw=w_dw, b_dw=b_dw, w_pw=w_pw, b_pw=b_pw, bias_u=U, bias_v=V)


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """A FlashSwin-T forward pass: image side, patch size p (stem kernel 2p - 1, stride p), window
    side M, embedding C, depths and heads per stage (d = C_s / heads_s = 32), classes."""
    name: str
    B: int
    img: int
    p: int
    M: int
    C: int = 96
    depths: tuple = (2, 2, 6, 2)
    heads: tuple = (3, 6, 12, 24)
    n_classes: int = 1000
    seed: int = 1008

    @property
    def tokens(self) -> int:
        return self.B * (self.img // self.p) ** 2


# FlashSwin-T at 256 px: patch 4 with M = 32, and the dense patch-2 grid with M = 32.
MODEL_CONFIGS = {
    "flashswin_t_p4_m32": ModelConfig("flashswin_t_p4_m32", 64, 256, 4, 32),
    "flashswin_t_p2_m32": ModelConfig("flashswin_t_p2_m32", 16, 256, 2, 32),
}


def _block_params(rng, C: int, dtype: str):
    def w(o, i):
        return rng.normal(0.0, 1.0 / math.sqrt(i), size=(o, i)).astype(np.float32)

    def small(n):
        return rng.normal(0.0, 0.02, size=n).astype(np.float32)

    P = dict(ln1_g=1.0 + small(C), ln1_b=small(C), w_qkv=w(3 * C, C), b_qkv=small(3 * C),
             w_proj=w(C, C), b_proj=small(C), ln2_g=1.0 + small(C), ln2_b=small(C),
             w_fc1=w(4 * C, C), b_fc1=small(4 * C), w_fc2=w(C, 4 * C), b_fc2=small(C))
    if dtype == "bf16":
        for key in ("w_qkv", "w_proj", "w_fc1", "w_fc2"):
            P[key] = round_bf16(P[key])
    return {k: np.asarray(v, np.float32) for k, v in P.items()}


def block_params(C: int, seed: int, dtype: str = "bf16"):
    """Seeded weights of one block: matrices ~ N(0, 1/fan_in) (rounded to bf16 for the bf16
    path), norm gains 1 + N(0, 0.02^2), biases N(0, 0.02^2), all float32 arrays."""
    return _block_params(_rng(seed), C, dtype)


def model_params(cfg: ModelConfig, dtype: str = "bf16"):
    """Seeded weights of the whole FlashSwin-T forward pass (structure as flashswin_forward
    expects): stem convolution and norm, per stage its blocks, RoPE table and patch merging,
    the final norm and the head."""
    rng = _rng(cfg.seed)
    k = 2 * cfg.p - 1
    rb = (lambda a: round_bf16(a)) if dtype == "bf16" else (lambda a: a)
    params = dict(stem_w=rb(rng.normal(0.0, 1.0 / math.sqrt(3 * k * k), size=(cfg.C, 3, k, k)).astype(np.float32)),
                  stem_b=rng.normal(0.0, 0.02, size=cfg.C).astype(np.float32),
                  stem_ln_g=(1.0 + rng.normal(0.0, 0.02, size=cfg.C)).astype(np.float32),
                  stem_ln_b=rng.normal(0.0, 0.02, size=cfg.C).astype(np.float32), stages=[])
    C = cfg.C
    for s, (depth, heads) in enumerate(zip(cfg.depths, cfg.heads)):
        st = dict(heads=heads, blocks=[_block_params(rng, C, dtype) for _ in range(depth)],
                  theta=theta_table(heads, C // heads, 0.1, cfg.seed + 100 + s), merge=None)
        if s + 1 < len(cfg.depths):
            st["merge"] = dict(ln_g=(1.0 + rng.normal(0.0, 0.02, size=4 * C)).astype(np.float32),
                               ln_b=rng.normal(0.0, 0.02, size=4 * C).astype(np.float32),
                               w=rb(rng.normal(0.0, 1.0 / math.sqrt(4 * C), size=(2 * C, 4 * C)).astype(np.float32)))
            C *= 2
        params["stages"].append(st)
    params["norm_g"] = (1.0 + rng.normal(0.0, 0.02, size=C)).astype(np.float32)
    params["norm_b"] = rng.normal(0.0, 0.02, size=C).astype(np.float32)
    params["head_w"] = rb(rng.normal(0.0, 1.0 / math.sqrt(C), size=(cfg.n_classes, C)).astype(np.float32))
    params["head_b"] = np.zeros(cfg.n_classes, np.float32)
    return params


def images(B: int, side: int, seed: int, dtype: str = "bf16"):
    """[B][side][side][3] images ~ N(0, 1) (NHWC), bf16-exact for the bf16 path."""
    a = _rng(seed).standard_normal(size=(B, side, side, 3), dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def cla_params(C: int, seed: int):
    """(w_dw [C][3][3], b_dw [C], w_pw [C][C], b_pw [C]) as float32."""
    rng = _rng(seed)
    w_dw = rng.normal(0.0, 1.0 / 3.0, size=(C, 3, 3)).astype(np.float32)
    b_dw = rng.normal(0.0, 0.1, size=C).astype(np.float32)
    w_pw = rng.normal(0.0, 1.0 / math.sqrt(C), size=(C, C)).astype(np.float32)
    b_pw = rng.normal(0.0, 0.1, size=C).astype(np.float32)
    return w_dw, b_dw, w_pw, b_pw


def make_inputs(cfg: WorkloadConfig, batch: int | None = None, shared_theta: bool = True):
    """All inputs of a workload as float32 numpy arrays (bf16-exact for bf16 workloads).

    Returns dict(q, k, v, theta or None, bias_u or None, bias_v or None).  ``batch``
    overrides B (a prefix of the same random stream is NOT implied; it is a new draw).
    """
    B = cfg.B if batch is None else batch
    shape = (B, cfg.Hg, cfg.Wg, cfg.H, cfg.d)
    q, k, v = qkv(shape, cfg.seed, cfg.dtype)
    theta = theta_table(cfg.H, cfg.d, cfg.omega_noise, cfg.seed + 1000, shared_theta) if cfg.rope else None
    U = V = None
    if cfg.r > 0:
        U, V = rib_factors(cfg.H, cfg.M, cfg.r, cfg.seed + 2000, cfg.dtype)
    return dict(q=q, k=k, v=v, theta=theta, bias_u=U, bias_v=V)
