"""Seeded synthetic workloads for the NVFP4 W4A4 prefill linear layer.

This module only draws inputs.  It holds none of the layer's arithmetic, so
both the CPU oracle and the HIP path can consume exactly the same bytes.
Everything is drawn in float32 with numpy's PCG64 generator and rounded to
BF16 (round-to-nearest-even) on the host.

Shapes follow the five layer configurations the library is measured on
(prefill token counts M, hidden sizes and projection widths of Qwen3-8B- and
larger dense- and MoE-shaped models).  Weights are stored N x K (the
transpose of a K x N projection matrix), K contiguous.

Seeds: tensor t of configuration c uses ``SeedSequence([1000 * c + t, chunk])``
for rows [chunk * CHUNK, (chunk + 1) * CHUNK) and ``SeedSequence([1000 * c + t,
OUTLIER_KEY])`` for its outlier channels, so any row range can be
regenerated on its own (the oracle checks sampled rows of large tensors).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1024                 # rows per independently seeded chunk
OUTLIER_KEY = 0x0517
OUTLIER_FRACTION = 0.005     # 0.5% of K-channels
OUTLIER_GAIN = 50.0


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1)))
    return (u >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Tensor:
    """One synthetic tensor: ``rows x cols`` BF16, drawn chunk by chunk."""
    cfg: int
    index: int
    rows: int
    cols: int
    dist: str                 # "normal", "student_t4", "silu_glu"
    std: float = 1.0
    outliers: bool = False

    def seed(self, chunk: int):
        return np.random.SeedSequence([1000 * self.cfg + self.index, chunk])

    def outlier_channels(self) -> np.ndarray:
        if not self.outliers:
            return np.zeros(0, dtype=np.int64)
        n = int(round(OUTLIER_FRACTION * self.cols))
        rng = np.random.default_rng(
            np.random.SeedSequence([1000 * self.cfg + self.index, OUTLIER_KEY]))
        return np.sort(rng.choice(self.cols, n, replace=False))

    def _draw(self, rng, n_rows: int) -> np.ndarray:
        shape = (n_rows, self.cols)
        if self.dist == "normal":
            x = rng.standard_normal(shape, dtype=np.float32)
            if self.std != 1.0:
                x *= np.float32(self.std)
        elif self.dist == "student_t4":
            x = rng.standard_t(4.0, shape).astype(np.float32)
            if self.std != 1.0:
                x *= np.float32(self.std)
        elif self.dist == "silu_glu":
            # H = SiLU(G) * U with G and U drawn independently, each with the
            # tensor's outlier channels; computed in float32 on the host.
            g = rng.standard_normal(shape, dtype=np.float32)
            u = rng.standard_normal(shape, dtype=np.float32)
            ch = self.outlier_channels()
            g[:, ch] *= np.float32(OUTLIER_GAIN)
            u[:, ch] *= np.float32(OUTLIER_GAIN)
            with np.errstate(over="ignore"):
                x = g / (np.float32(1.0) + np.exp(-g)) * u
            return x
        else:
            raise ValueError(self.dist)
        ch = self.outlier_channels()
        if ch.size:
            x[:, ch] *= np.float32(OUTLIER_GAIN)
        return x

    def chunk(self, c: int) -> np.ndarray:
        lo = c * CHUNK
        n = min(CHUNK, self.rows - lo)
        rng = np.random.default_rng(self.seed(c))
        return bf16_bits(self._draw(rng, n))

    def rows_of(self, row_ids) -> np.ndarray:
        """BF16 bits of the given rows (regenerating only their chunks)."""
        row_ids = np.asarray(row_ids, dtype=np.int64)
        out = np.empty((row_ids.size, self.cols), dtype=np.uint16)
        for c in np.unique(row_ids // CHUNK):
            blk = self.chunk(int(c))
            sel = np.nonzero(row_ids // CHUNK == c)[0]
            out[sel] = blk[row_ids[sel] - c * CHUNK]
        return out

    def full(self, workers: int | None = None) -> np.ndarray:
        """The whole tensor (chunks drawn in parallel host threads)."""
        out = np.empty((self.rows, self.cols), dtype=np.uint16)
        n_chunks = (self.rows + CHUNK - 1) // CHUNK

        def fill(c):
            out[c * CHUNK:c * CHUNK + CHUNK] = self.chunk(c)

        workers = workers or min(16, os.cpu_count() or 1, n_chunks)
        if workers <= 1 or n_chunks == 1:
            for c in range(n_chunks):
                fill(c)
        else:
            with ThreadPoolExecutor(workers) as ex:
                list(ex.map(fill, range(n_chunks)))
        return out


@dataclass(frozen=True)
class Gemm:
    """One projection: ``act`` (M x K) times ``weight`` (N x K) transposed."""
    name: str
    act: str
    weight: str
    grouped: bool = False


@dataclass
class Workload:
    cfg: int
    title: str
    tensors: dict = field(default_factory=dict)
    gemms: list = field(default_factory=list)
    # grouped (MoE) layers
    experts: int = 0
    topk: int = 0
    tokens: int = 0

    def flops(self) -> float:
        tot = 0.0
        for g in self.gemms:
            if g.grouped:
                w = self.tensors[g.weight + "[0]"]
                m = self.tokens * self.topk
                tot += 2.0 * m * w.rows * w.cols
            else:
                a, w = self.tensors[g.act], self.tensors[g.weight]
                tot += 2.0 * a.rows * w.rows * w.cols
        return tot

    def routing(self):
        """Top-k expert choice per token, drawn uniformly from the seed.

        Returns (token_of_row int32 [tokens*topk], group_offsets int64
        [experts+1]): routed rows sorted by expert, tokens ascending within an
        expert (a stable sort).
        """
        rng = np.random.default_rng(np.random.SeedSequence([1000 * self.cfg, 0x707E]))
        keys = rng.random((self.tokens, self.experts))
        choice = np.argsort(keys, axis=1, kind="stable")[:, :self.topk]
        tok = np.repeat(np.arange(self.tokens, dtype=np.int64), self.topk)
        exp = choice.reshape(-1)
        order = np.lexsort((tok, exp))
        counts = np.bincount(exp, minlength=self.experts)
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        return tok[order].astype(np.int32), offsets


def _add(w: Workload, name, idx, rows, cols, dist, std=1.0, outliers=False):
    w.tensors[name] = Tensor(w.cfg, idx, rows, cols, dist, std, outliers)


def workload(cfg: int) -> Workload:
    """Configurations 1..5 (see the module docstring)."""
    if cfg == 1:
        w = Workload(1, "single linear 256x1024 -> 1024")
        _add(w, "X", 0, 256, 1024, "normal")
        _add(w, "W", 1, 1024, 1024, "normal", 0.02)
        w.gemms = [Gemm("linear", "X", "W")]
    elif cfg == 2:
        w = Workload(2, "Qwen3-8B-shaped attention projections, M=8192")
        m, h = 8192, 4096
        _add(w, "X_qkv", 0, m, h, "normal", outliers=True)
        _add(w, "X_o", 1, m, h, "normal", outliers=True)
        _add(w, "W_q", 2, 4096, h, "normal", 0.02)
        _add(w, "W_k", 3, 1024, h, "normal", 0.02)
        _add(w, "W_v", 4, 1024, h, "normal", 0.02)
        _add(w, "W_o", 5, h, 4096, "normal", 0.02)
        w.gemms = [Gemm("q_proj", "X_qkv", "W_q"), Gemm("k_proj", "X_qkv", "W_k"),
                   Gemm("v_proj", "X_qkv", "W_v"), Gemm("o_proj", "X_o", "W_o")]
    elif cfg == 3:
        w = Workload(3, "Qwen3-8B-shaped MLP, M=32768")
        m, h, f = 32768, 4096, 12288
        _add(w, "X", 0, m, h, "normal", outliers=True)
        _add(w, "H", 1, m, f, "silu_glu", outliers=True)
        _add(w, "W_gate", 2, f, h, "normal", 0.02)
        _add(w, "W_up", 3, f, h, "normal", 0.02)
        _add(w, "W_down", 4, h, f, "normal", 0.02)
        w.gemms = [Gemm("gate_proj", "X", "W_gate"), Gemm("up_proj", "X", "W_up"),
                   Gemm("down_proj", "H", "W_down")]
    elif cfg == 4:
        w = Workload(4, "large dense linear stack, M=16384, hidden 5120")
        m, h = 16384, 5120
        _add(w, "X_qkv", 0, m, h, "student_t4")
        _add(w, "X_o", 1, m, h, "student_t4")
        _add(w, "X_gu", 2, m, h, "student_t4")
        _add(w, "H", 3, m, 25600, "student_t4")
        _add(w, "W_qkv", 4, 7168, h, "normal", 0.015)
        _add(w, "W_o", 5, h, h, "normal", 0.015)
        _add(w, "W_gu", 6, 51200, h, "normal", 0.015)
        _add(w, "W_down", 7, h, 25600, "normal", 0.015)
        w.gemms = [Gemm("qkv_proj", "X_qkv", "W_qkv"), Gemm("o_proj", "X_o", "W_o"),
                   Gemm("gate_up_proj", "X_gu", "W_gu"), Gemm("down_proj", "H", "W_down")]
    elif cfg == 5:
        w = Workload(5, "MoE grouped layer: 16384 tokens, 64 experts, top-8")
        w.tokens, w.experts, w.topk = 16384, 64, 8
        _add(w, "X", 0, 16384, 2816, "normal", outliers=True)
        _add(w, "H", 1, 16384 * 8, 1408, "normal", outliers=True)
        for e in range(64):
            _add(w, f"W_gu[{e}]", 100 + e, 2816, 2816, "normal", 0.02)
            _add(w, f"W_down[{e}]", 200 + e, 2816, 1408, "normal", 0.02)
        w.gemms = [Gemm("gate_up_proj", "X", "W_gu", grouped=True),
                   Gemm("down_proj", "H", "W_down", grouped=True)]
    else:
        raise ValueError(f"no configuration {cfg}")
    return w
