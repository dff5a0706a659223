"""Seeded synthetic workloads for the contextual-sparsity FFN step.

Input generation only: this module draws weights and tokens and holds none of the method's
arithmetic.  The pages measure on trained models (OPT-175B, OPT-30B, LLaMA/Mistral-class) that
are not available here; these stand-ins copy their shapes and the structure the method relies on:

  * W1 = U V + small noise, so the active set is predictable from a cheap low-rank projection
    ("Contextual Sparsity and Activation Predictors": the set is predictable from the layer input
    by something far cheaper than the layer);
  * a bias calibrated so a chosen fraction of pre-activations is positive (the sparsity level);
  * clustered tokens, so that the active sets of a batch overlap ("When it breaks");
  * optionally, per-neuron biases that make firing frequency follow a power law, a few neurons
    active for almost every token and a long rare tail ("Static locality: hot and cold neurons").

Normal draws N(0, s) use s as the standard deviation.  Every tensor is drawn from its own
torch.Generator seeded with seed(config, role, layer) = 1_000_000*config + 1_000*role + layer,
in float32, and rounded once (nearest-even) to the storage type.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

ROLE_U, ROLE_V, ROLE_W1_NOISE, ROLE_W2T, ROLE_WUP, ROLE_TOKENS = 1, 2, 3, 4, 5, 6
ROLE_CALIB, ROLE_CENTROIDS, ROLE_CLUSTER_IDS, ROLE_CLUSTER_NOISE = 7, 8, 9, 10
ROLE_POWERLAW, ROLE_PROFILE = 11, 12

RELU, REGLU, SILU, SWIGLU = 0, 1, 2, 3
GATED = (REGLU, SWIGLU)


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    d: int
    f: int
    r: int
    dtype: torch.dtype
    act: int
    k: Optional[int]                 # top-k size, or None for threshold mode
    tau: Optional[float]             # threshold on the sigmoid score
    uv_std: float                    # std of the low-rank factors U, V
    noise_std: float                 # std of the W1 noise elements
    w2t_std: float
    wup_std: float
    bias: Optional[float]            # fixed bias, or None to calibrate
    positive_frac: Optional[float]   # calibrated fraction of positive pre-activations
    tokens: int
    layers: int = 1

    def scaled(self, d: int, f: int, r: int, k: Optional[int] = None, tokens: int = 4) -> "Config":
        """The same recipe at another shape (parity tests); k defaults to the same fraction of f."""
        if k is None and self.k is not None:
            k = int(math.floor(f * self.k / self.f + 0.5))
        gated = self.act in GATED
        # ReLU recipes: unit-scale factors (the bias sets the sparsity).  SiLU recipes keep the
        # gate's spread, std(W1 x) = uv_std^2 sqrt(r d), which sets the functional sparsity.
        uv = (1.0 / math.sqrt(r) if self.act in (RELU, REGLU)
              else self.uv_std * (self.r * self.d / (r * d)) ** 0.25)
        return dataclasses.replace(self, d=d, f=f, r=r, k=k, tokens=tokens,
                                   uv_std=uv, noise_std=0.1 / d,
                                   w2t_std=1.0 / math.sqrt(d if gated else f),
                                   wup_std=1.0 / math.sqrt(d) if gated else 0.0)


# The workloads: a tiny float32 layer; the OPT-175B FFN shape at 5% (the headline case); a
# LLaMA-class gated (ReGLU) layer in bfloat16 with a sigmoid >= 0.5 threshold; the OPT-30B FFN shape
# at 20% for batch-union studies; a 48-layer stack of that shape; and the SwiGLU form of the
# LLaMA-class layer (functional sparsity).
CONFIGS = {
    0: Config(0, "tiny-relu-f32", 256, 1024, 64, torch.float32, RELU, 102, None,
              uv_std=1 / 8, noise_std=0.1 / 256, w2t_std=1 / 32, wup_std=0.0, bias=-0.5,
              positive_frac=None, tokens=64),
    1: Config(1, "opt175b-relu-f16", 12288, 49152, 1024, torch.float16, RELU, 2458, None,
              uv_std=1 / 32, noise_std=0.1 / 12288, w2t_std=1 / math.sqrt(49152), wup_std=0.0,
              bias=None, positive_frac=0.05, tokens=256),
    2: Config(2, "llama-reglu-bf16", 4096, 14336, 256, torch.bfloat16, REGLU, None, 0.5,
              uv_std=1 / 16, noise_std=0.1 / 4096, w2t_std=1 / 64, wup_std=1 / 64, bias=None,
              positive_frac=0.10, tokens=256),
    3: Config(3, "opt30b-relu-f16", 7168, 28672, 512, torch.float16, RELU, 5734, None,
              uv_std=1 / math.sqrt(512), noise_std=0.1 / 7168, w2t_std=1 / math.sqrt(28672),
              wup_std=0.0, bias=None, positive_frac=0.20, tokens=256),
    4: Config(4, "opt30b-relu-f16-stack48", 7168, 28672, 512, torch.float16, RELU, 5734, None,
              uv_std=1 / math.sqrt(512), noise_std=0.1 / 7168, w2t_std=1 / math.sqrt(28672),
              wup_std=0.0, bias=None, positive_frac=0.20, tokens=128, layers=48),
    # The LLaMA-class block before ReLU-fication: SwiGLU, no bias, the gate's spread chosen so
    # that |silu(W1 x)| > 0.1 for about half of the neurons (std(W1 x) = 0.3), the ~50%
    # functional sparsity the pages give for SiLU models; top-k keeps half of the neurons.
    5: Config(5, "llama-swiglu-bf16", 4096, 14336, 256, torch.bfloat16, SWIGLU, 7168, None,
              uv_std=(0.09 / (256 * 4096)) ** 0.25, noise_std=0.1 / 4096, w2t_std=1 / 64,
              wup_std=1 / 64, bias=0.0, positive_frac=None, tokens=256),
}

TINY_F32 = CONFIGS[0]          # d 256, f 1024, r 64, float32, top-k 102
OPT175B = CONFIGS[1]           # d 12288, f 49152, r 1024, float16, top-k 2458 (5%)
LLAMA_REGLU = CONFIGS[2]       # d 4096, f 14336, r 256, bfloat16, ReGLU, threshold 0.5
OPT30B = CONFIGS[3]            # d 7168, f 28672, r 512, float16, top-k 5734 (20%)
OPT30B_STACK48 = CONFIGS[4]    # 48 blocks of the OPT-30B shape
LLAMA_SWIGLU = CONFIGS[5]      # the LLaMA-class shape with SwiGLU, top-k 7168


def seed(config: int, role: int, layer: int = 0) -> int:
    return 1_000_000 * config + 1_000 * role + layer


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def normal(shape, std, device, s) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(device, s), device=device, dtype=torch.float32) * std


@dataclasses.dataclass
class Layer:
    cfg: Config
    V: torch.Tensor         # [r, d]  predictor down projection
    U: torch.Tensor         # [f, r]  predictor up projection
    W1: torch.Tensor        # [f, d]  gate (or up) projection
    b1: torch.Tensor        # [f]     float32
    Wup: Optional[torch.Tensor]  # [f, d] for the gated form
    W2T: torch.Tensor       # [f, d]  down projection, neuron-major

    @property
    def weight_bytes(self) -> int:
        n = self.W1.numel() + self.W2T.numel() + (self.Wup.numel() if self.Wup is not None else 0)
        return n * self.W1.element_size()


def make_layer(cfg: Config, device="cpu", layer: int = 0, config_id: Optional[int] = None) -> Layer:
    """Draw one layer's predictor and FFN weights on `device` (float32 draws, one rounding)."""
    c = cfg.index if config_id is None else config_id
    d, f, r, dt = cfg.d, cfg.f, cfg.r, cfg.dtype
    U32 = normal((f, r), cfg.uv_std, device, seed(c, ROLE_U, layer))
    V32 = normal((r, d), cfg.uv_std, device, seed(c, ROLE_V, layer))
    W1_32 = normal((f, d), cfg.noise_std, device, seed(c, ROLE_W1_NOISE, layer))
    W1_32.addmm_(U32, V32)
    W1 = W1_32.to(dt)
    del W1_32
    W2T = normal((f, d), cfg.w2t_std, device, seed(c, ROLE_W2T, layer)).to(dt)
    Wup = None
    if cfg.act in GATED:
        Wup = normal((f, d), cfg.wup_std, device, seed(c, ROLE_WUP, layer)).to(dt)
    V, U = V32.to(dt), U32.to(dt)
    del U32, V32
    if cfg.bias is not None:
        b = cfg.bias
    else:
        b = calibrate_bias(cfg, W1, device, c, layer)
    b1 = torch.full((f,), b, dtype=torch.float32, device=device)
    return Layer(cfg, V, U, W1, b1, Wup, W2T)


def calibrate_bias(cfg: Config, W1: torch.Tensor, device, c: int, layer: int,
                   n_tokens: int = 64) -> float:
    """Scalar bias -q with q the (1 - positive_frac) quantile of W1 x over calibration tokens, so
    that about positive_frac of the pre-activations are positive."""
    X = normal((n_tokens, cfg.d), 1.0, device, seed(c, ROLE_CALIB, layer)).to(cfg.dtype)
    P = (X.float() @ W1.float().t()).reshape(-1)
    kth = int(math.ceil((1.0 - cfg.positive_frac) * P.numel()))
    kth = min(max(kth, 1), P.numel())
    q = torch.kthvalue(P.cpu(), kth).values.item()
    return float(-q)


def powerlaw_firing(f: int, mean: float, alpha: float, device, s: int) -> torch.Tensor:
    """Target firing probability of each neuron: q = 0.99 / (1 + (rank / knee)^alpha) over a seeded
    random ranking, the knee set (by bisection) so that the mean probability is `mean`."""
    rank = torch.randperm(f, generator=_gen(device, s), device=device).to(torch.float64)

    def q_of(knee):
        return 0.99 / (1.0 + (rank / knee) ** alpha)

    lo, hi = 1e-3, float(f)
    for _ in range(80):
        mid = math.sqrt(lo * hi)
        if float(q_of(mid).mean()) < mean:
            lo = mid
        else:
            hi = mid
    return q_of(hi)


def make_powerlaw_layer(cfg: Config, device="cpu", layer: int = 0, alpha: float = 2.0,
                        config_id: Optional[int] = None) -> Layer:
    """A layer of the same recipe whose per-neuron bias gives neuron j the firing probability q_j
    of powerlaw_firing (mean cfg.positive_frac): for x ~ N(0, I), W1_j.x ~ N(0, |W1_j|^2), so
    b1_j = |W1_j| * Phi^-1(q_j).  The predictor is bias-free, so it does not see this structure."""
    c = cfg.index if config_id is None else config_id
    L = make_layer(cfg, device=device, layer=layer, config_id=config_id)
    sigma = L.W1.float().norm(dim=1).to(torch.float64)
    q = powerlaw_firing(cfg.f, cfg.positive_frac, alpha, device, seed(c, ROLE_POWERLAW, layer))
    b1 = (sigma * torch.special.ndtri(q)).to(torch.float32)
    return Layer(cfg, L.V, L.U, L.W1, b1, L.Wup, L.W2T)


def make_profile_tokens(cfg: Config, n: int, device="cpu", config_id: Optional[int] = None):
    """n tokens for profiling firing frequencies, seeded apart from the measured tokens."""
    c = cfg.index if config_id is None else config_id
    return normal((n, cfg.d), 1.0, device, seed(c, ROLE_PROFILE)).to(cfg.dtype)


def make_tokens(cfg: Config, n: int, device="cpu", config_id: Optional[int] = None) -> torch.Tensor:
    """n tokens x ~ N(0, 1), rounded to the storage type: [n, d]."""
    c = cfg.index if config_id is None else config_id
    return normal((n, cfg.d), 1.0, device, seed(c, ROLE_TOKENS)).to(cfg.dtype)


def make_clustered_tokens(cfg: Config, n: int, device="cpu", n_centroids: int = 8,
                          noise: float = 0.3, config_id: Optional[int] = None) -> torch.Tensor:
    """n tokens drawn as centroid[Uniform{0..n_centroids-1}] + N(0, noise): [n, d]."""
    c = cfg.index if config_id is None else config_id
    cent = normal((n_centroids, cfg.d), 1.0, device, seed(c, ROLE_CENTROIDS))
    ids = torch.randint(0, n_centroids, (n,), generator=_gen(device, seed(c, ROLE_CLUSTER_IDS)),
                        device=device)
    X = cent[ids] + normal((n, cfg.d), noise, device, seed(c, ROLE_CLUSTER_NOISE))
    return X.to(cfg.dtype)


def touched_bytes(cfg: Config, count: int) -> int:
    """Algorithmic bytes one batch-1 layer step reads: predictor V and U, `count` active rows of W1
    (and W_up) and W2T, and x."""
    es = torch.tensor([], dtype=cfg.dtype).element_size()
    rows = 3 if cfg.act in GATED else 2
    return es * (cfg.r * cfg.d + cfg.f * cfg.r + count * rows * cfg.d + cfg.d)


def dense_bytes(cfg: Config) -> int:
    es = torch.tensor([], dtype=cfg.dtype).element_size()
    rows = 3 if cfg.act in GATED else 2
    return es * rows * cfg.f * cfg.d


# ------------------------------------------------------------------------------------------------
# Attention-head sparsity workload
# ------------------------------------------------------------------------------------------------
ROLE_A_U, ROLE_A_V, ROLE_A_DIR, ROLE_A_QNOISE, ROLE_A_WK, ROLE_A_WV, ROLE_A_WO = 21, 22, 23, 24, 25, 26, 27
ROLE_A_KC, ROLE_A_VC, ROLE_A_CALIB, ROLE_A_TOKENS = 28, 29, 30, 31


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    """A decode step of multi-head attention with a KV cache of `context` past tokens per head.

    Head relevance is made input-dependent the way the pages describe silent heads: every head's
    cache starts with a sink position whose value is zero.  A head's query has a component along
    the sink key equal to beta * (theta - g_h(x)) + log(context) + q_std^2 / 2, with
    g = U_a (V_a x) a low-rank projection of the input: where g_h(x) < theta the sink takes almost
    all of the attention and the head's output is near zero; where g_h(x) > theta the head attends
    to its content (the constant is the log of the content's total softmax weight, so the switch
    sits at g_h = theta).  theta is set so that
    `active_frac` of the (token, head) pairs have g_h > theta.  The predictor's factors are the
    same U_a, V_a, so the active heads are predictable from x by a cheap low-rank network."""
    index: int
    name: str
    d: int
    H: int
    dh: int
    r: int
    dtype: torch.dtype
    k: int                  # heads kept by top-k
    context: int            # cached past tokens per head (the sink included)
    extra: int              # free cache positions beyond the context (Tmax = context + extra)
    active_frac: float
    beta: float = 16.0      # sink strength
    q_std: float = 1.5      # spread of the content logits
    tokens: int = 64

    @property
    def Tmax(self) -> int:
        return self.context + self.extra

    def scaled(self, d, H, dh, r, context, k=None, extra=8, tokens=4) -> "AttnConfig":
        if k is None:
            k = max(1, int(math.floor(H * self.k / self.H + 0.5)))
        return dataclasses.replace(self, d=d, H=H, dh=dh, r=r, context=context, k=k, extra=extra,
                                   tokens=tokens)


# OPT-175B attention shape (d 12288 = 96 heads x 128), a 2048-token context, a fifth of the heads
# active per token (the pages: a fifth to a third matter; over 80% can be silenced).
ATTN_CONFIGS = {
    0: AttnConfig(100, "tiny-attn-f32", 256, 8, 32, 32, torch.float32, 2, 64, 8, 0.25),
    1: AttnConfig(101, "opt175b-attn-f16", 12288, 96, 128, 256, torch.float16, 19, 2048, 64, 0.20),
}
ATTN_TINY_F32 = ATTN_CONFIGS[0]
ATTN_OPT175B = ATTN_CONFIGS[1]


@dataclasses.dataclass
class AttnLayer:
    cfg: AttnConfig
    Vp: torch.Tensor        # [r, d]      head predictor down projection (= V_a)
    Up: torch.Tensor        # [H, r]      head predictor up projection (= U_a)
    Wq: torch.Tensor        # [H*dh, d]
    Wk: torch.Tensor
    Wv: torch.Tensor
    WoT: torch.Tensor       # [H*dh, d]  output projection, head-dimension major
    bq: torch.Tensor        # [H*dh] float32
    Kc: torch.Tensor        # [H, Tmax, dh]
    Vc: torch.Tensor
    lens: torch.Tensor      # [H] int32, all = context

    @property
    def weight_bytes(self) -> int:
        return 4 * self.Wq.numel() * self.Wq.element_size()


def make_attention_layer(cfg: AttnConfig, device="cpu", layer: int = 0) -> AttnLayer:
    """Draw one attention layer and its filled caches (float32 draws, one rounding)."""
    c = cfg.index
    d, H, dh, r, dt, T = cfg.d, cfg.H, cfg.dh, cfg.r, cfg.dtype, cfg.context
    HD = H * dh
    uv = (1.0 / (r * d)) ** 0.25                       # g = U_a (V_a x) has unit spread
    Ua = normal((H, r), uv, device, seed(c, ROLE_A_U, layer))
    Va = normal((r, d), uv, device, seed(c, ROLE_A_V, layer))
    e = normal((H, dh), 1.0, device, seed(c, ROLE_A_DIR, layer))
    e = e / e.norm(dim=1, keepdim=True)                 # the sink direction of each head
    theta = _attn_theta(cfg, Ua, Va, device, layer)
    A = Ua @ Va                                         # [H, d]
    Wq = normal((HD, d), cfg.q_std / math.sqrt(d), device, seed(c, ROLE_A_QNOISE, layer))
    Wq.view(H, dh, d).add_(-cfg.beta * e[:, :, None] * A[:, None, :])
    # at g_h = theta the sink logit equals the log of the content's total weight (context
    # positions with logits of spread q_std), so the sink then holds about half of the attention
    c0 = math.log(T) + 0.5 * cfg.q_std ** 2
    bq = ((cfg.beta * theta + c0) * e).reshape(HD).to(torch.float32)
    Wk = normal((HD, d), 1.0 / math.sqrt(d), device, seed(c, ROLE_A_WK, layer))
    Wv = normal((HD, d), 1.0 / math.sqrt(d), device, seed(c, ROLE_A_WV, layer))
    WoT = normal((HD, d), 1.0 / math.sqrt(HD), device, seed(c, ROLE_A_WO, layer))
    Kc = normal((H, cfg.Tmax, dh), 1.0, device, seed(c, ROLE_A_KC, layer))
    Vc = normal((H, cfg.Tmax, dh), 1.0, device, seed(c, ROLE_A_VC, layer))
    Kc -= (Kc * e[:, None, :]).sum(-1, keepdim=True) * e[:, None, :]   # content keys avoid the sink
    Kc[:, 0, :] = math.sqrt(dh) * e                     # the sink: key along e_h, value zero
    Vc[:, 0, :] = 0.0
    Kc[:, T:, :] = 0.0
    Vc[:, T:, :] = 0.0
    lens = torch.full((H,), T, dtype=torch.int32, device=device)
    cast = lambda t: t.to(dt).contiguous()
    return AttnLayer(cfg, cast(Va), cast(Ua), cast(Wq), cast(Wk), cast(Wv), cast(WoT), bq,
                     cast(Kc), cast(Vc), lens)


def _attn_theta(cfg: AttnConfig, Ua, Va, device, layer, n_tokens: int = 64) -> float:
    """The (1 - active_frac) quantile of g = U_a (V_a x) over calibration tokens."""
    X = normal((n_tokens, cfg.d), 1.0, device, seed(cfg.index, ROLE_A_CALIB, layer)).to(cfg.dtype)
    G = (X.float() @ Va.to(cfg.dtype).float().t()) @ Ua.to(cfg.dtype).float().t()
    G = G.reshape(-1).cpu()
    kth = min(max(int(math.ceil((1.0 - cfg.active_frac) * G.numel())), 1), G.numel())
    return float(torch.kthvalue(G, kth).values)


def make_attn_tokens(cfg: AttnConfig, n: int, device="cpu") -> torch.Tensor:
    """n tokens x ~ N(0, 1), rounded to the storage type: [n, d]."""
    return normal((n, cfg.d), 1.0, device, seed(cfg.index, ROLE_A_TOKENS)).to(cfg.dtype)


def attn_touched_bytes(cfg: AttnConfig, heads: int, lens: int) -> int:
    """Algorithmic bytes of one decode step over `heads` heads with `lens` cached positions each
    (before the step): predictor Vp, Up; Wq, Wk, Wv rows and WoT rows of the heads; their cached
    keys and values (with the new token); x; the appended k, v."""
    es = torch.tensor([], dtype=cfg.dtype).element_size()
    pred = (cfg.r * cfg.d + cfg.H * cfg.r) * es
    weights = 4 * heads * cfg.dh * cfg.d * es
    cache = 2 * heads * (lens + 1) * cfg.dh * es
    return pred + weights + cache + cfg.d * es
