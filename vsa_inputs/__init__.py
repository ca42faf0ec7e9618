"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path.

This module draws random numbers and nothing else: it holds none of the
block-sparse attention arithmetic (no token-to-block index formula, no pooling,
scoring, selection or attention).  Both sides of every parity test receive the
very same host tensors from here.

Workloads stand in for the activations of the video DiT self-attention layers
the "FastVideo VSA" user guide describes (its intro and its routing log line
under "Choose top-k": a (31, 22, 40) post-patch latent grid cut into (4, 8, 8)
blocks), for the long-horizon Wan 2.1 1.3B runs in the "lvsa-tuning" listing's
latency table, and for the text-prefix + 64-token-tile maps of the sm_100a
route entry in FastVideo's h3-perf-stack commit log.  No trained weights,
real activations or benchmark suites are used.

Value recipe (per tensor Q, K, V, in that order, from one CPU generator):
  mu  ~ N(0, 0.5^2), one D-vector per (batch, head, coarse grid cell), where
        the coarse grid has cells of size block_size over the latent grid;
  eps ~ N(0, 1), shape [B, S, heads, D];
  x   = eps + mu broadcast over its cell  -> cast to bf16 (round to nearest even).
The mean field is built by repeating the coarse grid along each axis and
cropping to the latent grid, i.e. a piecewise-constant field; it is input
structure that makes the pooled block scores informative, like real DiT
activations whose neighbouring tokens are correlated.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "make_tile64_map",
           "make_planted_block_means"]


@dataclass(frozen=True)
class Workload:
    name: str
    dit_seq_shape: tuple
    block_size: tuple
    batch: int
    heads: int
    head_dim: int
    topk: int | None          # None: the block map is given (map mode)
    seed: int
    map_seed: int | None = None
    prefix_tiles: int = 0     # map mode: text-prefix tiles kept by every row
    max_video_k: int = 0      # map mode: video rows draw k ~ U{0..max_video_k}
    zero_row_every: int = 0   # map mode: 1 in N video rows emptied (0 = never)

    @property
    def seq_len(self) -> int:
        t, h, w = self.dit_seq_shape
        return t * h * w


# The five measured shapes plus two small parity shapes.  Sizes follow the
# pages: 27280-token Wan2.2-TI2V-5B layer with topk=64 (and its topk sweep),
# a tile-64 text-prefix map (512-token prefix + 32768 video tokens), and the
# 321-frame Wan 2.1 1.3B latent (81, 30, 52) at 12 heads.
WORKLOADS = {
    "tiny": Workload("tiny", (8, 16, 16), (4, 8, 8), 1, 2, 128, 4, seed=0),
    "wan5b_k64": Workload("wan5b_k64", (31, 22, 40), (4, 8, 8), 1, 24, 128, 64, seed=1),
    "wan5b_k16": Workload("wan5b_k16", (31, 22, 40), (4, 8, 8), 1, 24, 128, 16, seed=1),
    "wan5b_k32": Workload("wan5b_k32", (31, 22, 40), (4, 8, 8), 1, 24, 128, 32, seed=1),
    "wan5b_k120": Workload("wan5b_k120", (31, 22, 40), (4, 8, 8), 1, 24, 128, 120, seed=1),
    # one GPU's share of the 27280-token layer sharded over 8 (4, 2) GPUs by heads
    "wan5b_k64_h3": Workload("wan5b_k64_h3", (31, 22, 40), (4, 8, 8), 1, 3, 128, 64, seed=1),
    "wan5b_k64_h6": Workload("wan5b_k64_h6", (31, 22, 40), (4, 8, 8), 1, 6, 128, 64, seed=1),
    "wan5b_k64_h12": Workload("wan5b_k64_h12", (31, 22, 40), (4, 8, 8), 1, 12, 128, 64, seed=1),
    "tile64_csr": Workload("tile64_csr", (1, 1, 33280), (1, 1, 64), 1, 24, 128, None,
                           seed=3, map_seed=1003, prefix_tiles=8, max_video_k=64),
    "tile64_csr_zero": Workload("tile64_csr_zero", (1, 1, 33280), (1, 1, 64), 1, 24, 128,
                                None, seed=3, map_seed=1003, prefix_tiles=8,
                                max_video_k=64, zero_row_every=16),
    "wan13b_long": Workload("wan13b_long", (81, 30, 52), (4, 8, 8), 1, 12, 128, 64, seed=4),
    # small parity shapes
    "padded_tiny": Workload("padded_tiny", (7, 13, 10), (4, 8, 8), 1, 2, 128, 4, seed=7),
    "tile64_tiny": Workload("tile64_tiny", (1, 1, 640), (1, 1, 64), 1, 2, 128, None,
                            seed=8, map_seed=1008, prefix_tiles=2, max_video_k=4,
                            zero_row_every=3),
    # the other block volumes the kernels implement (128, 192, 3-D 64), one
    # with two batches
    "vol128_b2": Workload("vol128_b2", (8, 16, 16), (2, 8, 8), 2, 2, 128, 5, seed=9),
    "vol192_padded": Workload("vol192_padded", (7, 13, 10), (3, 8, 8), 1, 2, 128, 5, seed=10),
    "vol64_3d": Workload("vol64_3d", (4, 16, 16), (1, 8, 8), 1, 2, 128, 6, seed=11),
}


def _coarse_cells(dit_seq_shape, block_size):
    return tuple(-(-g // b) for g, b in zip(dit_seq_shape, block_size))


def _piecewise_field(mu, dit_seq_shape, block_size):
    """mu: [B, heads, ct, ch, cw, D] -> [B, S, heads, D] piecewise-constant field."""
    t, h, w = dit_seq_shape
    bt, bh, bw = block_size
    f = mu.repeat_interleave(bt, dim=2)[:, :, :t]
    f = f.repeat_interleave(bh, dim=3)[:, :, :, :h]
    f = f.repeat_interleave(bw, dim=4)[:, :, :, :, :w]
    b, nh = f.shape[0], f.shape[1]
    return f.permute(0, 2, 3, 4, 1, 5).reshape(b, t * h * w, nh, f.shape[-1])


def make_qkv(wl: Workload, dtype=torch.bfloat16):
    """Return (q, k, v) host tensors [B, S, heads, D] in ``dtype`` (bf16 default)."""
    nh = wl.heads
    g = torch.Generator("cpu").manual_seed(wl.seed)
    cells = _coarse_cells(wl.dit_seq_shape, wl.block_size)
    out = []
    for _ in range(3):
        mu = torch.randn(wl.batch, nh, *cells, wl.head_dim, generator=g) * 0.5
        eps = torch.randn(wl.batch, wl.seq_len, nh, wl.head_dim, generator=g)
        x = eps + _piecewise_field(mu, wl.dit_seq_shape, wl.block_size)
        out.append(x.to(dtype).contiguous())
        del mu, eps, x
    return tuple(out)


def make_tile64_map(wl: Workload):
    """Seeded non-uniform block map for the 1-D tile workloads, as CSR.

    Rows are ordered (batch, head, query tile).  Query tiles below
    ``prefix_tiles`` (the text prefix) keep every tile.  Every other row keeps
    the prefix tiles plus k ~ U{0..max_video_k} distinct video tiles drawn
    without replacement; with ``zero_row_every = n`` a seeded one in n of the
    video rows is emptied (count 0).  Column lists are ascending.

    Returns (row_ptr int32 [rows+1], col_idx int32 [nnz], num_tiles).
    """
    assert wl.map_seed is not None
    n_tiles = wl.dit_seq_shape[2] // wl.block_size[2]
    rng = np.random.default_rng(wl.map_seed)
    counts, cols = [], []
    prefix = np.arange(wl.prefix_tiles, dtype=np.int64)
    video = np.arange(wl.prefix_tiles, n_tiles, dtype=np.int64)
    for _b in range(wl.batch):
        for _h in range(wl.heads):
            for i in range(n_tiles):
                if i < wl.prefix_tiles:
                    row = np.arange(n_tiles, dtype=np.int64)
                else:
                    k = int(rng.integers(0, wl.max_video_k + 1))
                    pick = np.sort(rng.choice(video, size=k, replace=False))
                    row = np.concatenate([prefix, pick])
                    if wl.zero_row_every and int(rng.integers(0, wl.zero_row_every)) == 0:
                        row = row[:0]
                counts.append(len(row))
                cols.append(row)
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int64)
    return row_ptr.astype(np.int32), col_idx.astype(np.int32), n_tiles


def make_planted_block_means(seed, batch, heads, dit_seq_shape, block_size,
                             head_dim, lo=-4, hi=4, dtype=torch.bfloat16):
    """Inputs whose every token equals its coarse cell's integer mean vector.

    Returns (x [B,S,heads,D] in ``dtype``, mu [B,heads,cells...,D] int64).
    Small integers are exact in bf16 and fp32, so any correct block mean of x
    equals mu exactly, whatever the summation order.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    cells = _coarse_cells(dit_seq_shape, block_size)
    mu = torch.randint(lo, hi + 1, (batch, heads, *cells, head_dim), generator=g)
    x = _piecewise_field(mu.to(torch.float32), dit_seq_shape, block_size)
    return x.to(dtype).contiguous(), mu


def bf16_to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact upcast of a host tensor to a float64 numpy array."""
    return x.detach().to("cpu", torch.float64).numpy()

