"""Seeded synthetic inputs for the verify step.

Both the HIP path (its tests and ``bench.py``) and the fp64 oracle take their
inputs from here. This module holds none of the verification method's
arithmetic: it draws random numbers, rounds generated values to bfloat16,
names the workload shapes, and stands in for the draft model with a Gumbel-max
draw from the draft logits (the drafter is outside the verify step).

Random streams are numpy's Philox4x64-10 counter-based generator (Salmon et
al., "Parallel random numbers: as easy as 1, 2, 3", SC'11), keyed by
(seed, stream name). Uniforms are float32 values k * 2^-24 in [0, 1), exactly
representable in float32 and float64, so both sides see identical draws.

Workloads (all synthetic, no trained weights):

* ``tiny``: batch 1, K = 4, V = 1000; target logits i.i.d. N(0, 2^2), draft
  logits = target + N(0, 0.5^2); one bf16 linear 256 -> 1000 on a 5 x 256
  activation with x ~ N(0, 1), w ~ N(0, 0.02^2).
* ``LLAMA_8B``: 32 layers of QKV 4096->6144, O 4096->4096, gate/up
  4096->2*14336, down 14336->4096, plus an lm-head 4096->128256 (the
  Llama-3.1-8B linear shapes).
* ``LLAMA_70B_16L``: 16 layers of QKV 8192->10240, O 8192->8192, gate/up
  8192->2*28672, down 28672->8192, plus an lm-head 8192->128256.
* sampling stress: batch 64, K = 8, V = 128256, logits N(0, 3^2), draft
  noise set for alpha in {0.6, 0.81, 0.9}.

Draft-noise standard deviations for a target acceptance rate are read from
``draft_noise.json``, written by a calibration script that lives with the
oracle.
"""

import json
import os
import zlib

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))


# --------------------------------------------------------------------------
# Random streams
# --------------------------------------------------------------------------

def stream(seed, name):
    """Philox generator keyed by (seed, name)."""
    tag = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([int(seed), tag])))


def uniforms(seed, name, shape):
    """float32 uniforms on [0, 1), each a multiple of 2^-24."""
    return stream(seed, name).random(shape, dtype=np.float32)


def normals(seed, name, shape, std=1.0):
    """float32 normals N(0, std^2)."""
    z = stream(seed, name).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return z


def bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even);
    returns the uint16 bit patterns. Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_normal_bits(seed, name, shape, std=1.0):
    """bf16 bit patterns of N(0, std^2) draws."""
    return bf16_bits(normals(seed, name, shape, std))


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

class Stack:
    """Linear shapes of a decoder stack: (name, d_in, d_out) per layer."""

    def __init__(self, name, hidden, layers, linears, vocab):
        self.name = name
        self.hidden = hidden
        self.layers = layers
        self.linears = linears
        self.vocab = vocab

    def all_linears(self):
        """Every linear of one step in execution order, lm-head last."""
        out = []
        for layer in range(self.layers):
            for nm, d_in, d_out in self.linears:
                out.append((f"layer{layer}.{nm}", d_in, d_out))
        out.append(("lm_head", self.hidden, self.vocab))
        return out

    def weight_bytes(self):
        return sum(2 * d_in * d_out for _, d_in, d_out in self.all_linears())


LLAMA_8B = Stack("llama3.1-8b", 4096, 32,
                 [("qkv", 4096, 6144), ("o", 4096, 4096),
                  ("gate_up", 4096, 2 * 14336), ("down", 14336, 4096)], 128256)

LLAMA_70B_16L = Stack("llama-70b-16l", 8192, 16,
                      [("qkv", 8192, 10240), ("o", 8192, 8192),
                       ("gate_up", 8192, 2 * 28672), ("down", 28672, 8192)], 128256)

WEIGHT_STD = 0.02


# --------------------------------------------------------------------------
# Draft model stand-in
# --------------------------------------------------------------------------

# Weight-only 8-bit storage: FP8 E4M3 codes with one float32 scale per output
# row. Codes are N(0, W8_CODE_STD^2) draws rounded to the format, and the
# scales bring the dequantised weights to about N(0, WEIGHT_STD^2), with a
# seeded spread across rows.
W8_CODE_STD = 64.0


def e4m3_normal_codes(seed, name, shape, std=W8_CODE_STD):
    """uint8 FP8 E4M3 codes of N(0, std^2) draws, clamped to the finite range
    [-448, 448] and rounded to the format by torch's float8_e4m3fn cast."""
    import torch
    z = normals(seed, name, shape, std)
    np.clip(z, -448.0, 448.0, out=z)
    return torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def w8_row_scales(seed, name, d_out):
    """float32 [d_out]: WEIGHT_STD / W8_CODE_STD * (0.75 + 0.5 u), u uniform."""
    u = uniforms(seed, name, (d_out,))
    base = np.float32(WEIGHT_STD / W8_CODE_STD)
    return (base * (np.float32(0.75) + np.float32(0.5) * u)).astype(np.float32)


def gumbel_max_tokens(draft_logits, seed, name="draft_tokens"):
    """One draw per draft row from softmax(draft logits) by the Gumbel-max
    trick: argmax_v (l_v + g_v) with g_v = -log(-log U_v) i.i.d. Gumbel.

    draft_logits: float32 [B][K][V] -> int32 [B][K].
    """
    l = np.asarray(draft_logits, dtype=np.float32)
    u = uniforms(seed, name, l.shape).astype(np.float64)
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))
    return np.argmax(l.astype(np.float64) + g, axis=-1).astype(np.int32)


# --------------------------------------------------------------------------
# Draft noise for a target acceptance rate
# --------------------------------------------------------------------------

def draft_noise_table():
    with open(os.path.join(_HERE, "draft_noise.json")) as f:
        return json.load(f)


def draft_noise_sigma(key, alpha):
    """Noise std that gives the requested mean acceptance rate for the
    logit distribution named by key (see draft_noise.json)."""
    entry = draft_noise_table()[key]
    for row in entry["sigmas"]:
        if abs(row["alpha"] - alpha) < 1e-9:
            return row["sigma"]
    raise KeyError(f"no calibrated sigma for {key} at alpha={alpha}")


# --------------------------------------------------------------------------
# Whole inputs
# --------------------------------------------------------------------------

def sampling_inputs(seed, B, K, V, logit_std, sigma):
    """Target logits [B][K+1][V] ~ N(0, logit_std^2) i.i.d.; draft logits
    [B][K][V] = target rows 0..K-1 + sigma * N(0, 1); draft tokens drawn from
    the draft logits; u_accept [B][K] and u_sample [B][K+1]."""
    tl = normals(seed, "target_logits", (B, K + 1, V), logit_std)
    dl = tl[:, :K, :] + normals(seed, "draft_noise", (B, K, V), sigma)
    return {
        "B": B, "K": K, "V": V,
        "target_logits": tl,
        "draft_logits": dl.astype(np.float32),
        "draft_tokens": gumbel_max_tokens(dl, seed),
        "u_accept": uniforms(seed, "u_accept", (B, K)),
        "u_sample": uniforms(seed, "u_sample", (B, K + 1)),
    }


def tiny(seed):
    """The tiny workload: sampling inputs at B=1, K=4, V=1000 plus one bf16
    linear 256 -> 1000 on a 5 x 256 activation."""
    d = sampling_inputs(seed, 1, 4, 1000, 2.0, 0.5)
    d["x_bits"] = bf16_normal_bits(seed, "x", (5, 256), 1.0)
    d["w_bits"] = bf16_normal_bits(seed, "w", (1000, 256), WEIGHT_STD)
    return d


def linear_inputs(seed, name, M, d_in, d_out):
    """bf16 activation [M][d_in] ~ N(0,1) and weight [d_out][d_in] ~
    N(0, 0.02^2), as uint16 bit patterns (host arrays)."""
    return (bf16_normal_bits(seed, name + ".x", (M, d_in), 1.0),
            bf16_normal_bits(seed, name + ".w", (d_out, d_in), WEIGHT_STD))
