"""Seeded synthetic workloads drawn on the GPU (inputs only, no scoring arithmetic).

The full-cache workload (Phi-3-mini shaped: 32 layers, Hq = Hkv = 32, d = 96,
n = 131072, about 48 GiB of K/V) would take minutes to draw on the host, so this
module draws the same recipe as ``workload.make_layer`` on the device with
torch's counter-based Philox generator, seeded per layer (seed + layer):

* Q [Hq][w][d], K [Hkv][n][d], V [Hkv][n][d] i.i.d. standard normal float32,
  drawn in that order;
* 4 channels of K scaled by 8 in every KV head (channels from ``randperm``);
* keys 0..3 of every KV head raised by the least-norm b_g with
  q . b_g / sqrt(d) = 6 for all G*w window queries of the group (float64 solve);
* rounded to bfloat16 (round to nearest, ties to even).

The values differ from the numpy draws of ``workload`` (a different generator),
the distribution and structure do not.  Like ``workload``, this module holds
none of the method's arithmetic; the oracle gets host copies of exactly the
bytes the device path reads.
"""
from __future__ import annotations

import math

import torch


def fill_layer(cfg, layer: int, q_out, k_out, v_out):
    """Draw one layer into device int16 tensors q_out [Hq][w][d], k_out and
    v_out [Hkv][n][d] (bf16 bit patterns)."""
    Hq, Hkv, d, n, w = cfg.Hq, cfg.Hkv, cfg.d, cfg.n, cfg.w
    G = Hq // Hkv
    dev = k_out.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed + layer)
    q32 = torch.randn((Hq, w, d), generator=gen, device=dev, dtype=torch.float32)
    k32 = torch.randn((Hkv, n, d), generator=gen, device=dev, dtype=torch.float32)
    q_out.copy_(q32.to(torch.bfloat16).view(torch.int16))
    v_out.copy_(torch.randn((Hkv, n, d), generator=gen, device=dev,
                            dtype=torch.float32).to(torch.bfloat16).view(torch.int16))
    n_s = min(4, n)
    rhs = torch.full((G * w,), 6.0 * math.sqrt(d), dtype=torch.float64, device=dev)
    for g in range(Hkv):
        ch = torch.randperm(d, generator=gen, device=dev)[:4]
        k32[g][:, ch] *= 8.0
        qg = q32[g * G:(g + 1) * G].reshape(G * w, d).double()
        # least-norm solution of qg b = rhs (G*w equations, d unknowns)
        b = qg.t() @ torch.linalg.solve(qg @ qg.t(), rhs)
        k32[g][:n_s] += b.float()[None, :]
    k_out.copy_(k32.to(torch.bfloat16).view(torch.int16))


def make_cache(cfg, device="cuda"):
    """All layers folded into heads on the device: (q [L*Hq][w][d],
    k, v [L*Hkv][n][d]) int16 tensors holding bf16 bit patterns."""
    L, Hq, Hkv, d, n, w = cfg.layers, cfg.Hq, cfg.Hkv, cfg.d, cfg.n, cfg.w
    q = torch.empty((L * Hq, w, d), dtype=torch.int16, device=device)
    k = torch.empty((L * Hkv, n, d), dtype=torch.int16, device=device)
    v = torch.empty((L * Hkv, n, d), dtype=torch.int16, device=device)
    for layer in range(L):
        fill_layer(cfg, layer, q[layer * Hq:(layer + 1) * Hq], k[layer * Hkv:(layer + 1) * Hkv],
                   v[layer * Hkv:(layer + 1) * Hkv])
    return q, k, v
