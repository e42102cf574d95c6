"""Seeded synthetic inputs for the GDN streaming core.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the method's arithmetic (no normalisation, no scan), so both the
GPU tests and the CPU oracle can take their inputs from it.

Workload shapes follow the SANA-Streaming pages: 1280x704 frames through the
DCAE-V F32T4C32 autoencoder give 22 x 40 = 880 latent tokens per latent frame
(SANA-Video blog, section 3.2, and the Chinese summary's "Motivation"), a
streaming chunk is 3 latent frames (Chinese summary, "Method steps" step 2),
the head dimension is 112 (SANA-Video blog, section 3.1 table), and the hybrid
DiT has 15 GDN blocks (Chinese summary, "Core method").

Distributions (per token and head):
  q, k, v ~ N(0, 1), rounded to bf16 (round-to-nearest-even) unless io="f32";
  a = exp(-0.1 * softplus(z_a)), beta = sigmoid(z_b), z ~ N(0, 1), kept in fp32;
  S0 ~ N(0, 0.1^2) in fp32 where a carried state is needed.
q and k are drawn raw: the per-token L2 normalisation is part of the path.
Seeds: numpy SeedSequence([cfg, stream, layer, chunk, step]) -> PCG64; draw order
q, k, v, z_a, z_b, then S0.  The tiny fp32 case uses default_rng(0).
"""
from __future__ import annotations

import numpy as np

TOKENS_PER_FRAME = 22 * 40          # 1280x704 at 32x spatial compression
FRAMES_PER_CHUNK = 3
CHUNK_TOKENS = TOKENS_PER_FRAME * FRAMES_PER_CHUNK   # 2640
HEAD_DIM = 112
HEADS = 20
GDN_LAYERS = 15


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs cannot wrap: the largest finite pattern plus 0x8000 stays below 2^32
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-exact float32 values (the bf16 storage pattern)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _softplus(z):
    return np.logaddexp(0.0, z)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def draw(rng: np.random.Generator, T: int, H: int, Dk: int, Dv: int, *, io: str = "bf16",
         with_state: bool = False, gates: str = "default"):
    """Draw one stream's chunk: q, k [T, H, Dk], v [T, H, Dv], a, beta [T, H] (+ S0 [H, Dv, Dk])."""
    q = rng.standard_normal((T, H, Dk)).astype(np.float32)
    k = rng.standard_normal((T, H, Dk)).astype(np.float32)
    v = rng.standard_normal((T, H, Dv)).astype(np.float32)
    za = rng.standard_normal((T, H))
    zb = rng.standard_normal((T, H))
    if io == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif io != "f32":
        raise ValueError(f"unknown io dtype {io!r}")
    if gates == "default":
        a = np.exp(-0.1 * _softplus(za)).astype(np.float32)
    elif gates == "stress":           # slow forgetting: the carried state matters for a whole chunk
        a = np.full((T, H), 1.0 - 1e-3, dtype=np.float32)
    else:
        raise ValueError(f"unknown gate recipe {gates!r}")
    beta = _sigmoid(zb).astype(np.float32)
    out = dict(q=q, k=k, v=v, a=a, beta=beta)
    if with_state:
        out["S0"] = (0.1 * rng.standard_normal((H, Dv, Dk))).astype(np.float32)
    return out


def rng_for(cfg: int, stream: int = 0, layer: int = 0, chunk: int = 0, step: int = 0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, stream, layer, chunk, step])))


def batch(cfg: int, B: int, T: int, H: int, D: int, *, layer: int = 0, chunk: int = 0, step: int = 0,
          io: str = "bf16", with_state: bool = False, gates: str = "default", stream0: int = 0):
    """Stack B independent streams along a leading batch axis: q [B, T, H, D], ..., S0 [B, H, D, D]."""
    parts = [draw(rng_for(cfg, stream0 + b, layer, chunk, step), T, H, D, D, io=io,
                  with_state=with_state, gates=gates) for b in range(B)]
    return {key: np.stack([p[key] for p in parts]) for key in parts[0]}


def tiny_fp32():
    """16-dim single-head 64-token fp32 case (zero initial state), seed 0."""
    rng = np.random.default_rng(0)
    d = draw(rng, 64, 1, 16, 16, io="f32")
    return {key: val[None] for key, val in d.items()}


def stream_chunk_torch(cfg: int, chunk: int, B: int, T: int, H: int, D: int, *, device="cuda",
                       with_state: bool = False, stream0: int = 0):
    """Same distributions as `batch`, drawn on the device with torch's generator (for long
    streams whose host-side generation would dominate a test).  Seed: the first word of
    SeedSequence([cfg, stream0, 0, chunk, 0]).  Returns bf16 q, k, v [B, T, H, D], fp32 a, beta
    [B, T, H] and, if asked, an fp32 S0 [B, H, D, D], all on `device`."""
    import torch
    seed = int(np.random.SeedSequence([cfg, stream0, 0, chunk, 0]).generate_state(1)[0])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    for key in ("q", "k", "v"):
        out[key] = torch.randn((B, T, H, D), generator=gen, device=device).to(torch.bfloat16)
    za = torch.randn((B, T, H), generator=gen, device=device)
    zb = torch.randn((B, T, H), generator=gen, device=device)
    out["a"] = torch.exp(-0.1 * torch.nn.functional.softplus(za))
    out["beta"] = torch.sigmoid(zb)
    if with_state:
        out["S0"] = 0.1 * torch.randn((B, H, D, D), generator=gen, device=device)
    return out


ATTN_CFG = 10   # seed tag of the softmax-block attention inputs


def attn_chunk(chunk: int, B: int, T: int, H: int, D: int, *, stream: int = 0, step: int = 0,
               q_scale: float = 1.0) -> dict:
    """q, k, v [B, T, H, D] of one chunk for the softmax block's attention: N(0, 1) entries
    (q times ``q_scale``: the logits scale*q.k then have standard deviation q_scale at the
    default scale 1/sqrt(D)), rounded to bf16, returned as float32.
    Seed: SeedSequence([10, stream, 0, chunk, step]); draw order q, k, v."""
    rng = rng_for(ATTN_CFG, stream=stream, chunk=chunk, step=step)
    q = round_bf16(q_scale * rng.standard_normal((B, T, H, D), dtype=np.float32))
    k = round_bf16(rng.standard_normal((B, T, H, D), dtype=np.float32))
    v = round_bf16(rng.standard_normal((B, T, H, D), dtype=np.float32))
    return {"q": q, "k": k, "v": v}


def proj_inputs(cfg: int, M: int, K: int, N: int):
    """Inputs of a projection GEMM of the GDN block: activations x [M, K] ~ N(0, 1) and weights w [N, K] ~
    N(0, 1/K), both rounded to bf16 (float32 arrays of bf16 values).  SeedSequence([cfg, 0, 0, 0, 0]) -> PCG64,
    drawn in that order."""
    rng = rng_for(cfg)
    x = round_bf16(rng.standard_normal((M, K)).astype(np.float32))
    w = round_bf16((rng.standard_normal((N, K)) / np.sqrt(max(K, 1))).astype(np.float32))
    return x, w
