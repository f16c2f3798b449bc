"""Seeded synthetic inputs for the SERQ linear layer.

This module only draws random numbers.  It holds none of the method's
arithmetic (no scaling, permutation or quantization), so both the CPU oracle
and the HIP path can be fed from it without sharing any of the computation.

The shapes are the public LLaMA-2-7B / LLaMA-3-8B layer shapes (hidden 4096,
intermediate 14336, 8 KV heads x 128 = 1024) at 2048-token prefill, the
setting the SERQ notes page (dihengye.cn) measures in its GPU performance
table.  Trained weights and calibration corpora are not available, so:

* weights are N(0, 0.02) draws;
* activations are N(0, 1) draws with a fixed set of outlier channels
  multiplied by a factor (sign kept).  The same channel indices are used in
  the runtime activations and in the calibration rows: channel-persistent
  outliers are the premise of static activation flattening (SERQ notes page,
  Stage 1; gist.science summaries, section 2.1);
* the down-projection input is shaped like silu(G) * U with G, U ~ N(0, 1);
* calibration sets are independent 512-row draws of the same distribution,
  standing in for the 32-512 calibration samples the pages use.

Every workload is reproducible from ``numpy.random.SeedSequence(1000 + c)``;
child streams are spawned in a fixed order per workload.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

FMT_INT4 = "int4"    # 4-bit weights, 4-bit per-token activations (W4A4)
FMT_W4A8 = "w4a8"    # 4-bit weights, 8-bit per-token activations
FMT_MXFP4 = "mxfp4"  # E2M1 elements, E8M0 scale per 32-element block
FMT_MXW4A8 = "mxw4a8"  # MXFP4 weights and R, E4M3 activations with E8M0 block scales


@dataclass
class LinearCase:
    """One linear layer Y = X @ W with its calibration rows.

    W is [d_in][d_out] (rows are input channels), X is [M][d_in] in original
    channel order, X_cal is [n_cal][d_in].
    """

    name: str
    fmt: str
    r: int
    W: np.ndarray
    X: np.ndarray
    X_cal: np.ndarray
    group: str = ""          # layers with the same group share their input X
    extra: dict = field(default_factory=dict)

    @property
    def d_in(self) -> int:
        return int(self.W.shape[0])

    @property
    def d_out(self) -> int:
        return int(self.W.shape[1])

    @property
    def M(self) -> int:
        return int(self.X.shape[0])


def _weights(rng: np.random.Generator, d_in: int, d_out: int, std: float = 0.02) -> np.ndarray:
    return (rng.standard_normal((d_in, d_out)) * std).astype(np.float32)


def _acts(rng: np.random.Generator, m: int, d_in: int, idx: np.ndarray, factor: float,
          kind: str = "normal") -> np.ndarray:
    if kind == "normal":
        x = rng.standard_normal((m, d_in))
    elif kind == "silu":
        g = rng.standard_normal((m, d_in))
        u = rng.standard_normal((m, d_in))
        x = g / (1.0 + np.exp(-g)) * u
    else:
        raise ValueError(kind)
    x[:, idx] *= factor
    return x.astype(np.float32)


def correlated_case(c: LinearCase, n_cal: int = 2048, rank: int = 64, noise: float = 0.3, factor: float = 50.0,
                    seed: int = 2000) -> LinearCase:
    """The layer of ``c`` with activations whose channels are correlated, as
    an LLM's are: a rank-``rank`` latent factor (N(0, 1) mixing weights over
    sqrt(rank)) plus isotropic noise, 1 % outlier channels times ``factor``;
    the same mixing for the M input tokens and ``n_cal`` calibration tokens.
    Error-compensating weight quantizers (GPTQ) exploit exactly this
    structure, which the independent-channel recipe lacks."""
    ss = np.random.SeedSequence(seed + c.d_in)
    k_mix, k_x, k_c, k_i = [np.random.default_rng(x) for x in ss.spawn(4)]
    A = k_mix.standard_normal((rank, c.d_in)) / np.sqrt(rank)
    idx = k_i.choice(c.d_in, n_outliers(c.d_in), replace=False)

    def draw(g, m):
        x = g.standard_normal((m, rank)) @ A + noise * g.standard_normal((m, c.d_in))
        x[:, idx] *= factor
        return x.astype(np.float32)

    return LinearCase(c.name + "_correlated", c.fmt, c.r, c.W, draw(k_x, c.M), draw(k_c, n_cal), group=c.group)


def n_outliers(d_in: int, frac: float = 0.01) -> int:
    """1 % of the channels, rounded up (41 of 4096, 144 of 14336)."""
    return int(np.ceil(frac * d_in))


def random_case(seed: int, M: int, d_in: int, d_out: int, r: int, fmt: str,
                n_out: int = 3, factor: float = 40.0, n_cal: Optional[int] = None,
                kind: str = "normal", name: str = "random") -> LinearCase:
    """A small seeded case of any shape (parity tests: ragged M, tails, r=0, r=d_in)."""
    ss = np.random.SeedSequence(seed)
    k_w, k_x, k_c, k_i = [np.random.default_rng(s) for s in ss.spawn(4)]
    idx = k_i.choice(d_in, min(n_out, d_in), replace=False)
    W = _weights(k_w, d_in, d_out)
    X = _acts(k_x, M, d_in, idx, factor, kind)
    X_cal = X if n_cal is None else _acts(k_c, n_cal, d_in, idx, factor, kind)
    return LinearCase(name, fmt, r, W, X, X_cal)


# --- the five workloads ------------------------------------------------------

def tiny_int4() -> List[LinearCase]:
    """16 tokens, 256 -> 128, r = 16, 3 outlier channels x40, X_cal = X."""
    ss = np.random.SeedSequence(1000)
    k_w, k_x, k_i = [np.random.default_rng(s) for s in ss.spawn(3)]
    W = _weights(k_w, 256, 128)
    idx = k_i.choice(256, 3, replace=False)
    X = _acts(k_x, 16, 256, idx, 40.0)
    return [LinearCase("tiny", FMT_INT4, 16, W, X, X)]


def attn_proj_int4(M: int = 2048) -> List[LinearCase]:
    """LLaMA-2-7B attention projection, 4096 -> 4096, 2048 tokens, r = 128, INT4."""
    ss = np.random.SeedSequence(1001)
    k_w, k_x, k_c, k_i = [np.random.default_rng(s) for s in ss.spawn(4)]
    W = _weights(k_w, 4096, 4096)
    idx = k_i.choice(4096, n_outliers(4096), replace=False)
    X = _acts(k_x, M, 4096, idx, 50.0)
    X_cal = _acts(k_c, 512, 4096, idx, 50.0)
    return [LinearCase("attn_proj", FMT_INT4, 128, W, X, X_cal)]


def llama3_mlp_int4(M: int = 2048) -> List[LinearCase]:
    """LLaMA-3-8B MLP: gate, up 4096 -> 14336 sharing X; down 14336 -> 4096 on a
    silu-shaped input.  r = 128, INT4."""
    ss = np.random.SeedSequence(1002)
    (k_wg, k_wu, k_wd, k_x, k_xc, k_h, k_hc, k_ix, k_ih) = [
        np.random.default_rng(s) for s in ss.spawn(9)]
    Wg = _weights(k_wg, 4096, 14336)
    Wu = _weights(k_wu, 4096, 14336)
    Wd = _weights(k_wd, 14336, 4096)
    ix = k_ix.choice(4096, n_outliers(4096), replace=False)
    ih = k_ih.choice(14336, n_outliers(14336), replace=False)
    X = _acts(k_x, M, 4096, ix, 50.0)
    Xc = _acts(k_xc, 512, 4096, ix, 50.0)
    H = _acts(k_h, M, 14336, ih, 50.0, "silu")
    Hc = _acts(k_hc, 512, 14336, ih, 50.0, "silu")
    return [LinearCase("gate", FMT_INT4, 128, Wg, X, Xc, group="mlp_in"),
            LinearCase("up", FMT_INT4, 128, Wu, X, Xc, group="mlp_in"),
            LinearCase("down", FMT_INT4, 128, Wd, H, Hc, group="down_in")]


def llama3_layer_mxfp4(M: int = 2048, fmt: str = FMT_MXFP4) -> List[LinearCase]:
    """LLaMA-3-8B decoder-layer linear set in an MX format (MXFP4, or MXFP4
    weights with MXFP8 E4M3 activations), 2048 tokens, r = 128."""
    ss = np.random.SeedSequence(1003)
    ks = [np.random.default_rng(s) for s in ss.spawn(19)]
    shapes = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
              ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
    Ws = {n: _weights(ks[i], di, do) for i, (n, di, do) in enumerate(shapes)}
    groups = [("attn_in", 4096, "normal"), ("o_in", 4096, "normal"),
              ("mlp_in", 4096, "normal"), ("down_in", 14336, "silu")]
    acts = {}
    for j, (g, d, kind) in enumerate(groups):
        k_x, k_c, k_i = ks[7 + 3 * j], ks[8 + 3 * j], ks[9 + 3 * j]
        idx = k_i.choice(d, n_outliers(d), replace=False)
        acts[g] = (_acts(k_x, M, d, idx, 50.0, kind), _acts(k_c, 512, d, idx, 50.0, kind))
    member = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in",
              "gate": "mlp_in", "up": "mlp_in", "down": "down_in"}
    return [LinearCase(n, fmt, 128, Ws[n], *acts[member[n]], group=member[n])
            for n, _, _ in shapes]


def decode_llama3(fmt: str = FMT_INT4, M: int = 16) -> List[LinearCase]:
    """Decode-shaped LLaMA-3-8B MLP: fused gate+up 4096 -> 28672 and down
    14336 -> 4096, M tokens, r = 256, activations with 3 outlier channels x40."""
    ss = np.random.SeedSequence(1004)
    k_wgu, k_wd, k_x, k_xc, k_h, k_hc, k_ix, k_ih = [
        np.random.default_rng(s) for s in ss.spawn(8)]
    Wgu = _weights(k_wgu, 4096, 28672)
    Wd = _weights(k_wd, 14336, 4096)
    ix = k_ix.choice(4096, 3, replace=False)
    ih = k_ih.choice(14336, 3, replace=False)
    X = _acts(k_x, M, 4096, ix, 40.0)
    Xc = _acts(k_xc, 512, 4096, ix, 40.0)
    H = _acts(k_h, M, 14336, ih, 40.0)
    Hc = _acts(k_hc, 512, 14336, ih, 40.0)
    return [LinearCase("gate_up", fmt, 256, Wgu, X, Xc, group="mlp_in"),
            LinearCase("down", fmt, 256, Wd, H, Hc, group="down_in")]


def concat_shared(cases: List[LinearCase], name: str) -> LinearCase:
    """Layers that read the same input share one flattening scale and one
    permutation; they are prepared as one wide layer [W_a | W_b | ...]."""
    first = cases[0]
    W = np.concatenate([c.W for c in cases], axis=1)
    return LinearCase(name, first.fmt, first.r, W, first.X, first.X_cal, group=first.group,
                      extra={"splits": [c.d_out for c in cases], "names": [c.name for c in cases]})


def _mlp_int4() -> List[LinearCase]:
    g, u, d = llama3_mlp_int4()
    return [concat_shared([g, u], "gate_up"), d]


def _layer_mx(fmt: str = FMT_MXFP4) -> List[LinearCase]:
    cs = {c.name: c for c in llama3_layer_mxfp4(fmt=fmt)}
    return [concat_shared([cs["q"], cs["k"], cs["v"]], "qkv"), cs["o"],
            concat_shared([cs["gate"], cs["up"]], "gate_up"), cs["down"]]


# Named workloads of the benchmark: name -> (description, layer-list factory,
# roofline bound, weight copies rotated per step so that decode weights come
# from HBM rather than the 256 MB last-level cache).
NAMED = {
    "attn_proj_int4": ("LLaMA-2-7B attention projection, 2048 tokens, 4096->4096, r=128, W4A4 INT4",
                       attn_proj_int4, "mfma", 1),
    "llama3_mlp_int4": ("LLaMA-3-8B MLP, 2048 tokens, gate|up 4096->28672 and down 14336->4096, r=128, "
                        "W4A4 INT4", _mlp_int4, "mfma", 1),
    "llama3_layer_mxfp4": ("LLaMA-3-8B decoder-layer linears (q|k|v, o, gate|up, down), 2048 tokens, r=128, "
                           "MXFP4", _layer_mx, "mfma", 1),
    "llama3_layer_mxw4a8": ("LLaMA-3-8B decoder-layer linears (q|k|v, o, gate|up, down), 2048 tokens, r=128, "
                            "MXFP4 weights, MXFP8 E4M3 activations", lambda: _layer_mx(FMT_MXW4A8), "mfma", 1),
    "decode_int4_m16": ("LLaMA-3-8B decode, 16 tokens, gate|up 4096->28672 and down 14336->4096, r=256, W4A4",
                        lambda: decode_llama3(FMT_INT4, 16), "hbm", 6),
    "decode_int4_m1": ("LLaMA-3-8B decode, 1 token, gate|up 4096->28672 and down 14336->4096, r=256, W4A4",
                       lambda: decode_llama3(FMT_INT4, 1), "hbm", 6),
    "decode_w4a8_m16": ("LLaMA-3-8B decode, 16 tokens, gate|up 4096->28672 and down 14336->4096, r=256, W4A8",
                        lambda: decode_llama3(FMT_W4A8, 16), "hbm", 6),
    "decode_mxfp4_m16": ("LLaMA-3-8B decode, 16 tokens, gate|up 4096->28672 and down 14336->4096, r=256, MXFP4",
                         lambda: decode_llama3(FMT_MXFP4, 16), "hbm", 6),
    "decode_mxw4a8_m16": ("LLaMA-3-8B decode, 16 tokens, gate|up 4096->28672 and down 14336->4096, r=256, "
                          "MXFP4 weights, MXFP8 E4M3 activations", lambda: decode_llama3(FMT_MXW4A8, 16), "hbm", 6),
}
