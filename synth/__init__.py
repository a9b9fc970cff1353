"""Seeded synthetic inputs for Taylor-truncated attention.

This module only draws and rounds inputs; it holds none of the attention
arithmetic, and both the oracle checks and the library runs take their inputs
from here.

Recipe (host, numpy):

* each (config id, b, h) slice has its own stream,
  ``numpy.random.default_rng(SeedSequence([cfg_id, b, h, salt]))`` (PCG64);
* q and k rows are drawn N(0, 1) in float64 and divided by their L2 norm
  (``unit_norm=True``; the raw variant keeps the draws), v is drawn N(0, 1);
* values are rounded to float32 (round to nearest even); for bfloat16 the
  float32 values are rounded again to bfloat16 (round to nearest even);
* the float64 copy handed to the oracle holds exactly the rounded values.

Recipe (device, torch; for inputs too large to draw on the host, e.g. a
65,536-token decode prefix over 1,024 heads): a ``torch.Generator`` on the
device seeded with ``seed_of(cfg_id, salt)`` draws float32 N(0, 1) in order
batch by batch; q/k rows are normalised in float64 and rounded back to
float32.  Checks copy the slices they need back to the host, so the oracle
sees exactly the device values.
"""

import numpy as np

F32 = "f32"
BF16 = "bf16"


def _rng(cfg_id, b, h, salt):
    return np.random.default_rng(np.random.SeedSequence([int(cfg_id), int(b), int(h), int(salt)]))


def round_to_bf16_bits(x32):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_values(x64, dtype):
    """Round float64 values as the device will see them. Returns (device-format array, float64 copy)."""
    x32 = x64.astype(np.float32)
    if dtype == F32:
        return x32, x32.astype(np.float64)
    if dtype == BF16:
        bits = round_to_bf16_bits(x32)
        return bits, bf16_bits_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def draw_head(cfg_id, b, h, N, d_k, d_v, unit_norm=True, salt=0):
    """float64 q [N, d_k], k [N, d_k], v [N, d_v] for one (b, h) slice, before rounding."""
    rng = _rng(cfg_id, b, h, salt)
    q = rng.standard_normal((N, d_k))
    k = rng.standard_normal((N, d_k))
    v = rng.standard_normal((N, d_v))
    if unit_norm:
        q = q / np.linalg.norm(q, axis=1, keepdims=True)
        k = k / np.linalg.norm(k, axis=1, keepdims=True)
    return q, k, v


class QKV:
    """Rounded inputs in device format (``q``, ``k``, ``v``) and their float64 copies (``q64`` ...)."""

    def __init__(self, q, k, v, q64, k64, v64, dtype):
        self.q, self.k, self.v = q, k, v
        self.q64, self.k64, self.v64 = q64, k64, v64
        self.dtype = dtype

    def torch(self, device):
        """Device tensors [B, H, N, d]: float32, or bfloat16 carrying the same bits."""
        import torch

        def up(a):
            if self.dtype == BF16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)

        return up(self.q), up(self.k), up(self.v)


def make_qkv(cfg_id, B, H, N, d_k, d_v, dtype=F32, unit_norm=True, salt=0):
    """Seeded [B, H, N, d] inputs, rounded to ``dtype`` (host recipe in the module docstring)."""
    shape_k = (B, H, N, d_k)
    shape_v = (B, H, N, d_v)
    q64 = np.empty(shape_k)
    k64 = np.empty(shape_k)
    v64 = np.empty(shape_v)
    for b in range(B):
        for h in range(H):
            q64[b, h], k64[b, h], v64[b, h] = draw_head(cfg_id, b, h, N, d_k, d_v, unit_norm, salt)
    q, q64 = round_values(q64, dtype)
    k, k64 = round_values(k64, dtype)
    v, v64 = round_values(v64, dtype)
    return QKV(q, k, v, q64, k64, v64, dtype)


def seed_of(cfg_id, salt=0):
    """64-bit seed for the device-side generator, derived from the same SeedSequence scheme."""
    return int(np.random.SeedSequence([int(cfg_id), int(salt)]).generate_state(1, dtype=np.uint64)[0] >> 1)


def device_qkv(cfg_id, B, H, N, d_k, d_v, device, unit_norm=True, salt=0, need_q=True, slab=None):
    """Seeded float32 [B, H, N, d] tensors drawn on ``device`` (device recipe in the module docstring).

    Draws batch row by batch row (``slab`` sequences at a time) so that the
    float64 normalisation never holds more than one slab.  Returns (q or None, k, v).
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed_of(cfg_id, salt))
    slab = slab or max(1, min(B, (1 << 26) // max(1, H * N * (d_k + d_v))))
    q = torch.empty((B, H, N, d_k), dtype=torch.float32, device=device) if need_q else None
    k = torch.empty((B, H, N, d_k), dtype=torch.float32, device=device)
    v = torch.empty((B, H, N, d_v), dtype=torch.float32, device=device)

    def unit(x):
        x64 = x.double()
        return (x64 / x64.norm(dim=-1, keepdim=True)).float()

    for b0 in range(0, B, slab):
        b1 = min(B, b0 + slab)
        if need_q:
            t = torch.randn((b1 - b0, H, N, d_k), generator=g, device=device)
            q[b0:b1] = unit(t) if unit_norm else t
        t = torch.randn((b1 - b0, H, N, d_k), generator=g, device=device)
        k[b0:b1] = unit(t) if unit_norm else t
        v[b0:b1] = torch.randn((b1 - b0, H, N, d_v), generator=g, device=device)
    return q, k, v


def ragged_lengths(cfg_id, n_seqs, lo, hi, salt=0):
    """Seeded sequence lengths drawn uniformly from [lo, hi] (a mix of short and long prompts)."""
    rng = np.random.default_rng(np.random.SeedSequence([int(cfg_id), int(salt), 7]))
    return [int(x) for x in rng.integers(lo, hi + 1, size=n_seqs)]


class Ragged(QKV):
    """A ragged batch packed head-major: q, k [H, T, d_k] and v [H, T, d_v] in device format (float64
    copies q64 ...), and offsets ``cu`` [n_seqs + 1] (int32): sequence b is tokens cu[b] .. cu[b+1]-1."""

    def __init__(self, q, k, v, q64, k64, v64, dtype, cu):
        super().__init__(q, k, v, q64, k64, v64, dtype)
        self.cu = cu

    @property
    def lengths(self):
        return [int(b - a) for a, b in zip(self.cu[:-1], self.cu[1:])]

    def seq(self, b):
        """float64 (q, k, v) of sequence b, each [H, len_b, d]."""
        a, e = int(self.cu[b]), int(self.cu[b + 1])
        return self.q64[:, a:e], self.k64[:, a:e], self.v64[:, a:e]

    def torch_cu(self, device):
        import torch

        return torch.from_numpy(self.cu).to(device)


def make_ragged(cfg_id, lengths, H, d_k, d_v, dtype=F32, unit_norm=True, salt=0):
    """Seeded ragged batch: sequence b, head h draws its rows as draw_head(cfg_id, b, h, len_b, ...)."""
    lengths = [int(n) for n in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q64 = np.empty((H, T, d_k))
    k64 = np.empty((H, T, d_k))
    v64 = np.empty((H, T, d_v))
    for b, n in enumerate(lengths):
        for h in range(H):
            q64[h, cu[b] : cu[b + 1]], k64[h, cu[b] : cu[b + 1]], v64[h, cu[b] : cu[b + 1]] = draw_head(
                cfg_id, b, h, n, d_k, d_v, unit_norm, salt)
    q, q64 = round_values(q64, dtype)
    k, k64 = round_values(k64, dtype)
    v, v64 = round_values(v64, dtype)
    return Ragged(q, k, v, q64, k64, v64, dtype, cu)
