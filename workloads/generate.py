"""Seeded synthetic Q, K, V, G for one attention layer or a stacked 4-layer group.

Recipe (same for every workload):
  * one independent random stream per (layer, tensor) -- or per (layer, tensor,
    b, h) slab for the on-device generator -- derived from the workload seed with
    numpy's SeedSequence spawn keys, tensor ids Q=0, K=1, V=2, G=3, heavy-row
    set=4;
  * standard normal draws in float32, scaled to the workload's distribution
    (Q, K, V ~ N(0,1) or N(0,1)/sqrt(d); G ~ N(g_mean, 1));
  * heavy-tailed workloads scale round(heavy_frac * N) token rows of K and V by
    heavy_scale; the rows are drawn without replacement, shared by K and V, by
    every batch item and head of one layer;
  * rounding to the storage dtype with round-to-nearest-even (torch's float32 ->
    bfloat16 conversion).
The host generator (numpy PCG64) and the device generator (torch Philox, used
where host generation of multi-GB tensors would take minutes) draw different
numbers for the same seed; a check always hands the oracle the exact values the
GPU saw, copied back from device memory.
"""
import math

import numpy as np
import torch

from .configs import Workload

TENSORS = ("Q", "K", "V", "G")
_TID = {"Q": 0, "K": 1, "V": 2, "G": 3, "heavy": 4, "x": 5, "W_in": 6, "W_out": 7}
_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(w: Workload):
    return _TORCH_DTYPE[w.dtype]


def _std(w: Workload, name: str) -> float:
    if name == "G":
        return 1.0
    return 1.0 if w.qkv_std == "unit" else 1.0 / math.sqrt(w.d)


def _mean(w: Workload, name: str) -> float:
    return w.g_mean if name == "G" else 0.0


def _seed_seq(w: Workload, layer: int, name: str, *slab):
    return np.random.SeedSequence(w.seed, spawn_key=(layer, _TID[name]) + tuple(slab))


def heavy_token_positions(w: Workload, layer: int, N: int | None = None) -> np.ndarray:
    """Sorted token indices whose K and V rows are scaled (empty if none)."""
    N = w.N if N is None else N
    n_heavy = int(round(w.heavy_frac * N))
    if n_heavy == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(_seed_seq(w, layer, "heavy")))
    return np.sort(rng.choice(N, size=n_heavy, replace=False)).astype(np.int64)


def layer_inputs_host(w: Workload, layer: int = 0, *, B=None, H=None, N=None,
                      device="cpu") -> dict:
    """Q, K, V, G of one layer drawn on the host, returned as torch tensors of the
    workload dtype on `device`.  B, H, N override the workload's sizes (tests use
    smaller shapes with the same distributions)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    heavy = heavy_token_positions(w, layer, N)
    out = {}
    for name in TENSORS:
        rng = np.random.Generator(np.random.PCG64(_seed_seq(w, layer, name)))
        x = rng.standard_normal((B, H, N, w.d), dtype=np.float32)
        x *= np.float32(_std(w, name))
        if _mean(w, name) != 0.0:
            x += np.float32(_mean(w, name))
        if name in ("K", "V") and heavy.size:
            x[:, :, heavy, :] *= np.float32(w.heavy_scale)
        out[name] = torch.from_numpy(x).to(torch_dtype(w)).to(device)
    return out


def _torch_seed(w: Workload, layer: int, name: str, *slab) -> int:
    return int(_seed_seq(w, layer, name, *slab).generate_state(1, np.uint64)[0] >> 1)


def layer_inputs_device(w: Workload, layer: int = 0, device="cuda", *, out=None) -> dict:
    """Q, K, V, G of one layer drawn on the GPU, one (b, h) slab at a time so the
    float32 staging buffer stays at N*d elements.  `out` may hold preallocated
    [B, H, N, d] tensors (e.g. views into a stacked group buffer)."""
    heavy = heavy_token_positions(w, layer)
    heavy_t = torch.from_numpy(heavy).to(device) if heavy.size else None
    res = {}
    gen = torch.Generator(device=device)
    for name in TENSORS:
        t = out[name] if out is not None else torch.empty(
            (w.B, w.H, w.N, w.d), dtype=torch_dtype(w), device=device)
        for b in range(w.B):
            for h in range(w.H):
                gen.manual_seed(_torch_seed(w, layer, name, b, h))
                x = torch.randn((w.N, w.d), generator=gen, device=device, dtype=torch.float32)
                x.mul_(_std(w, name))
                if _mean(w, name) != 0.0:
                    x.add_(_mean(w, name))
                if name in ("K", "V") and heavy_t is not None:
                    x[heavy_t] *= w.heavy_scale
                t[b, h].copy_(x)
                del x
        res[name] = t
    return res


def group_inputs_device(w: Workload, device="cuda", layers: int = 4) -> dict:
    """Stacked [layers, B, H, N, d] Q, K, V, G for a group, drawn on the GPU."""
    stacked = {n: torch.empty((layers, w.B, w.H, w.N, w.d), dtype=torch_dtype(w), device=device)
               for n in TENSORS}
    for layer in range(layers):
        layer_inputs_device(w, layer, device, out={n: stacked[n][layer] for n in TENSORS})
    return stacked


# ---------------------------------------------------------------------------
# Attention block: residual stream x [B, N, C] ~ N(0, 1) and, per sub-layer l,
# W_in[l] [4C, C] and W_out[l] [C, C] ~ N(0, 1/C) (fan-in scaling, so that the
# projected Q, K, V, G are about N(0, 1)), C = H * d.  One stream per (layer,
# tensor) on the host; per (layer, tensor, slab) on the device.

def block_inputs_host(w: Workload, *, B=None, H=None, N=None, d=None, layers: int = 4,
                      device="cpu", out_scale: float = 1.0) -> dict:
    """x [B, N, C], W_in [layers, 4C, C], W_out [layers, C, C] drawn on the host.
    out_scale multiplies W_out (tests use it to give the update the size of x)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    d = w.d if d is None else d
    C = H * d
    dt = torch_dtype(w)
    rng = np.random.Generator(np.random.PCG64(_seed_seq(w, 0, "x")))
    x = rng.standard_normal((B, N, C), dtype=np.float32)
    W_in = np.empty((layers, 4 * C, C), dtype=np.float32)
    W_out = np.empty((layers, C, C), dtype=np.float32)
    for l in range(layers):
        W_in[l] = np.random.Generator(np.random.PCG64(_seed_seq(w, l, "W_in"))).standard_normal(
            (4 * C, C), dtype=np.float32) * np.float32(1.0 / math.sqrt(C))
        W_out[l] = np.random.Generator(np.random.PCG64(_seed_seq(w, l, "W_out"))).standard_normal(
            (C, C), dtype=np.float32) * np.float32(out_scale / math.sqrt(C))
    return {"x": torch.from_numpy(x).to(dt).to(device),
            "W_in": torch.from_numpy(W_in).to(dt).to(device),
            "W_out": torch.from_numpy(W_out).to(dt).to(device)}


def block_inputs_device(w: Workload, device="cuda", layers: int = 4) -> dict:
    """The block inputs at the workload's full size, drawn on the GPU (x one
    batch item at a time, each weight matrix as one slab)."""
    C = w.H * w.d
    dt = torch_dtype(w)
    gen = torch.Generator(device=device)
    x = torch.empty((w.B, w.N, C), dtype=dt, device=device)
    for b in range(w.B):
        gen.manual_seed(_torch_seed(w, 0, "x", b))
        x[b].copy_(torch.randn((w.N, C), generator=gen, device=device, dtype=torch.float32))
    W_in = torch.empty((layers, 4 * C, C), dtype=dt, device=device)
    W_out = torch.empty((layers, C, C), dtype=dt, device=device)
    for l in range(layers):
        gen.manual_seed(_torch_seed(w, l, "W_in"))
        W_in[l].copy_(torch.randn((4 * C, C), generator=gen, device=device, dtype=torch.float32) / math.sqrt(C))
        gen.manual_seed(_torch_seed(w, l, "W_out"))
        W_out[l].copy_(torch.randn((C, C), generator=gen, device=device, dtype=torch.float32) / math.sqrt(C))
    return {"x": x, "W_in": W_in, "W_out": W_out}


def to_f64(t) -> np.ndarray:
    """Exact widening of a float32/bfloat16 tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
