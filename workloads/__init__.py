"""Seeded synthetic inputs for the CSA2 layer step.

This module only draws random numbers and lays them out; it holds none of the
layer step's arithmetic (no compression, quantization, scoring, selection or
attention).  Both the CPU oracle and the GPU path consume exactly the tensors
built here.  FP8 inputs that the workloads define as "N(0,1) rounded to E4M3"
(indexer keys and queries) are produced with torch's
own float8_e4m3fn cast of clamped normals.

Sizes follow the five workloads of the layer step:
  0  decode, 1 Full layer, batch 1, 4,096-token context (1,024 entries)
  1  prefill chunk of 2,048 tokens at positions 30,720..32,767 (8,192 entries)
  2  decode, batch 64 x 131,072 tokens (32,768 entries), Full + 5 Reuse
  3  decode, batch 32 x 1,048,576 tokens (262,144 entries), Full + pool + 3 Reindex
  4  prefill chunk of 4,096 tokens after 262,144 tokens (65,536 entries),
     Full(+pool), Reuse, Reuse, Reindex, Reuse
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

D = 512          # latent width (key = value)
H = 16           # attention query heads
H_I = 8          # indexer heads
D_I = 128        # indexer head width
M = 4            # tokens per compressed entry
ROPE_DIM = 64    # rotated channels (the last 64)
ROPE_BASE = 10000.0
N_WIN = 128
TOP_K = 512
POOL_BLOCKS = 2048
BLOCK = 8
EPS = 1e-6


@dataclass
class Config:
    cid: int
    name: str
    kind: str                 # "decode" or "prefill"
    n_seq: int                # sequences
    ctx_tokens: int           # tokens before the queries (prefill) / total (decode)
    chunk: int                # queries per sequence (decode: 1)
    layers: List[str]         # layer modes: "F", "U" (Reuse), "I" (Reindex)
    build_pool: bool
    synthetic_cache: bool     # prior entries drawn as MXFP4 bytes
    extra: dict = field(default_factory=dict)
    window_per_layer: bool = False   # every layer its own window (else one per group)

    @property
    def n_queries(self):
        return self.n_seq * self.chunk

    @property
    def entries_total(self):
        """Entries per sequence after the step."""
        if self.kind == "decode":
            return self.ctx_tokens // M
        return (self.ctx_tokens + self.chunk) // M

    @property
    def prior_entries(self):
        """Entries that exist before the step's compression runs."""
        if self.kind == "decode":
            return self.ctx_tokens // M - 1
        return self.ctx_tokens // M

    @property
    def new_entries(self):
        return self.entries_total - self.prior_entries


CONFIGS = {
    0: Config(0, "decode_b1_4k_full", "decode", 1, 4096, 1, ["F"], False, False),
    1: Config(1, "prefill_2048_at_32k_full", "prefill", 1, 30720, 2048, ["F"], False, False),
    2: Config(2, "decode_b64_128k_full_5reuse", "decode", 64, 131072, 1,
              ["F", "U", "U", "U", "U", "U"], False, True),
    3: Config(3, "decode_b32_1m_full_pool_3reindex", "decode", 32, 1048576, 1,
              ["F", "I", "I", "I"], True, True),
    4: Config(4, "prefill_4096_at_256k_FUUIU", "prefill", 1, 262144, 4096,
              ["F", "U", "U", "I", "U"], True, True),
}


def small_config(kind="decode", n_seq=2, ctx_tokens=1024, chunk=1, layers=("F",),
                 build_pool=False, synthetic_cache=False, cid=100):
    """A reduced workload of the same structure (tests)."""
    return Config(cid, f"small_{kind}", kind, n_seq, ctx_tokens, chunk, list(layers),
                  build_pool, synthetic_cache)


# The V4.1 CSA2 layer schedule ("DeepSeek-V4.1 架构解析" §02, layer modes): the 18 CSA2 encoder
# layers form three groups of one Full layer and five Reuse layers; the 20
# decoder layers are a Full layer and three Reuse layers, then four times a
# Reindex layer and three Reuse layers, and the decoder's Full layer builds
# the block pool its Reindex layers search.  Every group has its own global
# KV (entries and indexer keys, from its Full layer); every layer has its own
# 128-token window ("DeepSeek-V4.1 架构解析" §03: the window state is per layer).
V41_ENCODER_GROUP = ["F"] + ["U"] * 5
V41_DECODER_GROUP = ["F", "U", "U", "U"] + ["I", "U", "U", "U"] * 4
V41_GROUPS = [(V41_ENCODER_GROUP, False)] * 3 + [(V41_DECODER_GROUP, True)]


def v41_schedule(kind="decode", n_seq=2, ctx_tokens=4096, chunk=1, synthetic_cache=False, cid=200,
                 name="v41"):
    """Workload configs of the four groups of the schedule (decode: a new token
    passes through every layer)."""
    return [Config(cid + 10 * g, f"{name}_g{g}", kind, n_seq, ctx_tokens, chunk, list(layers), pool,
                   synthetic_cache, window_per_layer=True)
            for g, (layers, pool) in enumerate(V41_GROUPS)]


# The schedule at the 1M-context decode shape (batch 32): 38 layers, four
# global KV caches of 262,144 entries per sequence.
SCHEDULES = {
    "decode_b32_1m_v41_38layers": dict(kind="decode", n_seq=32, ctx_tokens=1048576, synthetic_cache=True,
                                       cid=300, name="decode_b32_1m_v41"),
}


# ------------------------------------------------------------ primitives ----

def _gen(cid, tid, device):
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (cid + 1) + 7919 * tid + 17)
    return g


def normal(shape, cid, tid, device="cpu", std=1.0):
    g = _gen(cid, tid, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def uniform(shape, cid, tid, device="cpu"):
    g = _gen(cid, tid, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def e4m3_normal(shape, cid, tid, device="cpu"):
    """N(0,1) rounded to E4M3 by torch's cast; returned as uint8 bytes."""
    x = normal(shape, cid, tid, device).clamp_(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def mxfp4_bytes(n_rows, cid, tid, device="cpu"):
    """Synthetic MXFP4 entries: random codes, scales 2**-2 .. 2**-1.

    Every code nibble is uniform over the 16 E2M1 codes; every scale byte is
    uniform over the E4M3 bytes 0x28..0x30 (0.25 .. 0.5), which gives entries
    of RMS ~1 like an RMSNorm output.  Shapes: codes [*n_rows, 256], scales
    [*n_rows, 32].
    """
    rows = tuple(n_rows) if isinstance(n_rows, (tuple, list)) else (n_rows,)
    g = _gen(cid, tid, device)
    codes = torch.randint(0, 256, rows + (D // 2,), generator=g, device=device,
                          dtype=torch.uint8)
    g2 = _gen(cid, tid + 1000, device)
    scales = torch.randint(0x28, 0x31, rows + (D // 16,), generator=g2, device=device,
                           dtype=torch.uint8)
    return codes, scales


def rope_table(positions, rope_dim=ROPE_DIM, base=ROPE_BASE):
    """(cos, sin) of pos * base**(-2i/rope_dim), computed in float64, stored fp32.

    Returns a float32 numpy array [len(positions), rope_dim/2, 2].
    """
    pos = np.asarray(positions, dtype=np.float64)[:, None]
    inv = base ** (-np.arange(0, rope_dim, 2, dtype=np.float64) / rope_dim)
    ang = pos * inv[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


# -------------------------------------------------------------- workload ----

@dataclass
class Workload:
    cfg: Config
    tensors: dict

    def __getitem__(self, k):
        return self.tensors[k]


def make_workload(cfg, device="cpu"):
    """All inputs of one layer step of ``cfg`` on ``device``.

    Keys (S sequences, Q = S * chunk queries, cap = entries per sequence):
      x_tail     fp32 [S, 127 + n_step, 512]: the latest token latents, i.e. the
                 127 tokens before the step's tokens, then the step's tokens
                 (decode: n_step = 1; prefill: n_step = chunk).  The window holds
                 them; the step compresses the last 4 * new_entries rows.
      x_prior    fp32 [S, 4 * prior, 512]: tokens of the prior entries (only when
                 the cache is not synthetic; shares its tail with x_tail).
      rope_prior fp32 [S, prior, 32, 2] (only when the cache is not synthetic)
      w          fp32 [4, 512, 512] ~ N(0, 1/(512*4))
      rope_cs    fp32 [S, new_entries, 32, 2]: table of the step's new entries
      codes/scales  uint8 [S, cap, 256] / [S, cap, 32]; synthetic caches have
                 their prior rows filled here, the rest is written by the step
      k_fp8      uint8 [S, cap, 128] ~ E4M3(N(0,1))
      q_pos      int32 [Q]
      q_fp8 / w_idx   per layer (None for Reuse): uint8 [Q, 8, 128] / fp32 [Q, 8]
      q_attn     per layer fp32 [Q, 16, 512] ~ N(0,1)
      x_win      (window_per_layer only) fp32 [L, S, 127 + n_step, 512]: every
                 layer's own window latents, laid out like x_tail
    """
    S, chunk = cfg.n_seq, cfg.chunk
    cap = cfg.entries_total
    prior, new = cfg.prior_entries, cfg.new_entries
    cid = cfg.cid
    t = {}
    n_step = 1 if cfg.kind == "decode" else chunk
    tail = N_WIN - 1 + n_step
    total_tokens = M * cap
    if cfg.synthetic_cache:
        t["x_tail"] = normal((S, tail, D), cid, 0, device)
        c, s = mxfp4_bytes((S, prior), cid, 60, device)
        codes = torch.zeros((S, cap, D // 2), dtype=torch.uint8, device=device)
        scales = torch.zeros((S, cap, D // 16), dtype=torch.uint8, device=device)
        codes[:, :prior] = c
        scales[:, :prior] = s
    else:
        x_full = normal((S, total_tokens, D), cid, 0, device)
        t["x_tail"] = x_full[:, total_tokens - tail:].contiguous()
        t["x_prior"] = x_full[:, :M * prior].contiguous()
        prior_pos = [M * j + M - 1 for j in range(prior)]
        rp = torch.from_numpy(rope_table(prior_pos)).to(device)
        t["rope_prior"] = rp.unsqueeze(0).expand(S, -1, -1, -1).contiguous()
        codes = torch.zeros((S, cap, D // 2), dtype=torch.uint8, device=device)
        scales = torch.zeros((S, cap, D // 16), dtype=torch.uint8, device=device)
    t["codes"], t["scales"] = codes, scales
    t["w"] = normal((M, D, D), cid, 1, device, std=1.0 / np.sqrt(D * M))
    new_pos = [M * (prior + j) + M - 1 for j in range(new)]
    rc = torch.from_numpy(rope_table(new_pos)).to(device)
    t["rope_cs"] = rc.unsqueeze(0).expand(S, -1, -1, -1).contiguous()
    t["k_fp8"] = e4m3_normal((S, cap, D_I), cid, 2, device)
    if cfg.kind == "decode":
        t["q_pos"] = torch.full((S,), cfg.ctx_tokens - 1, dtype=torch.int32, device=device)
    else:
        pos = torch.arange(cfg.ctx_tokens, cfg.ctx_tokens + chunk, dtype=torch.int32,
                           device=device)
        t["q_pos"] = pos.repeat(S)
    Q = cfg.n_queries
    if cfg.window_per_layer:
        t["x_win"] = normal((len(cfg.layers), S, tail, D), cid, 80, device)
    t["q_attn"] = [normal((Q, H, D), cid, 5 + li, device) for li in range(len(cfg.layers))]
    t["q_fp8"], t["w_idx"] = [], []
    for li, mode in enumerate(cfg.layers):
        if mode in ("F", "I"):
            t["q_fp8"].append(e4m3_normal((Q, H_I, D_I), cid, 20 + li, device))
            t["w_idx"].append(uniform((Q, H_I), cid, 40 + li, device))
        else:
            t["q_fp8"].append(None)
            t["w_idx"].append(None)
    return Workload(cfg, t)


def window_capacity(cfg):
    """Rows of the per-sequence window ring (token t lives in row t % cap)."""
    return N_WIN if cfg.kind == "decode" else cfg.chunk + N_WIN
