"""Seeded synthetic inputs for Gist Sparse Attention (GSA) decode and prefill.

This module is shared by the tests, the benchmark and the smoke check. It
only *makes inputs*: Gaussian queries and an interleaved K/V cache (C raw
rows, then one gist row per chunk), with a few gist keys moved along the
mean-query direction so that the top-k chunk choice has a clear margin.
It never selects chunks and never computes attention; the projections onto
the mean-query direction below exist only to place the planted keys.

Shapes follow the workloads the pages describe (long contexts, chunk size 16,
compression ratio 8x to 32x, a handful of relevant chunks among many
distractors: gist.science explainer, section 2 'Key Concepts' and section 4
'Experimental Results'; Taki-lab slide deck, slide 3).

Randomness comes from ``torch.Generator`` on the requested device, so the
values differ between CPU and GPU for the same seed; every consumer passes
the very same tensors (or host copies of them) to both the GPU path and the
CPU oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = [
    "DecodeConfig", "HierConfig", "PrefillConfig", "GistConfig", "VarlenConfig", "CONFIGS",
    "DecodeInputs", "HierInputs", "PrefillInputs",
    "make_decode", "make_hier", "make_prefill", "make_gist", "TokenStream", "make_token_stream",
    "make_levels", "level_sizes", "varlen_lengths", "to_pages",
    "raw_row", "gist_row", "n_rows",
]


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str            # "f32" | "bf16"
    n_raw: int            # N raw tokens per sequence
    chunk: int            # C
    topk: int             # k
    tail: int             # T trailing raw tokens always attended
    plant: str = "margin"  # "margin" | "literal" | "none"
    margin: float = 0.5   # minimum planted gap in scaled group score
    n_gist: Optional[int] = None  # default floor(N / C)

    @property
    def M(self) -> int:
        return self.n_raw // self.chunk if self.n_gist is None else self.n_gist

    @property
    def R(self) -> int:
        return self.n_raw + self.M


@dataclasses.dataclass(frozen=True)
class HierConfig:
    base: DecodeConfig    # level-1 cache and k1 (= base.topk)
    fanout: int           # G level-1 gists per level-2 gist
    topk2: int            # k2

    @property
    def name(self) -> str:
        return self.base.name

    @property
    def M2(self) -> int:
        return self.base.M // self.fanout


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    n_raw: int
    chunk: int
    topk: int
    window: int
    n_q: int              # queries are raw positions [n_raw - n_q, n_raw)
    q_block: int = 64
    alpha: float = 8.0    # weight of the per-block shared query direction
    margin: float = 0.5
    n_gist: Optional[int] = None
    values: str = "gauss"  # "int": q/K/V entries uniform in {-2..2} (exact scores, many ties)

    @property
    def M(self) -> int:
        return self.n_raw // self.chunk if self.n_gist is None else self.n_gist

    @property
    def R(self) -> int:
        return self.n_raw + self.M

    @property
    def q_start(self) -> int:
        return self.n_raw - self.n_q


@dataclasses.dataclass(frozen=True)
class VarlenConfig:
    """A decode step over sequences of different lengths (uniform in
    [n_min, n_max] raw tokens)."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    n_min: int
    n_max: int
    chunk: int
    topk: int
    tail: int
    page_chunks: int = 0   # > 0: the caches live in shuffled pages of this many chunk slots


@dataclasses.dataclass(frozen=True)
class GistConfig:
    """Cache-building step of one prompt: every raw and gist row appended to an
    empty cache, then the attention of every gist token."""
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    n_raw: int
    chunk: int

    @property
    def M(self) -> int:
        return self.n_raw // self.chunk

    @property
    def R(self) -> int:
        return self.n_raw + self.M


CONFIGS = {
    # tiny single-query decode, fp32, D=64: parity config
    "tiny_f32": DecodeConfig("tiny_f32", 1, 1, 1, 64, "f32", 4096, 16, 8, 16,
                             plant="literal", margin=0.05),
    # batched GQA decode step at 32K context, 16x compression
    "gqa_32k": DecodeConfig("gqa_32k", 32, 32, 8, 128, "bf16", 32768, 16, 16, 64),
    # compression-ratio sweep at 131K context
    "c8_131k": DecodeConfig("c8_131k", 8, 32, 8, 128, "bf16", 131072, 8, 64, 64),
    "c32_131k": DecodeConfig("c32_131k", 8, 32, 8, 128, "bf16", 131072, 32, 16, 64),
    # two-level gist-of-gist decode at 1M context
    "hier_1m": HierConfig(DecodeConfig("hier_1m", 4, 32, 8, 128, "bf16", 1048576,
                                       16, 16, 64), fanout=16, topk2=8),
    # causal block-sparse prefill of the last 4096 positions of a 64K sequence
    "prefill_64k": PrefillConfig("prefill_64k", 32, 8, 128, "bf16", 65536, 16, 16,
                                 64, 4096),
    # cache append + gist-token attention of a 64K-token prompt (4096 gists)
    "gist_64k": GistConfig("gist_64k", 32, 8, 128, "bf16", 65536, 16),
    # the batched GQA decode step with sequence lengths uniform in [4K, 32K]
    "varlen_32k": VarlenConfig("varlen_32k", 32, 32, 8, 128, "bf16", 4096, 32768, 16, 16, 64),
    # the same batch with its caches in shuffled pages of 16 chunk slots (272 rows)
    "paged_32k": VarlenConfig("paged_32k", 32, 32, 8, 128, "bf16", 4096, 32768, 16, 16, 64, page_chunks=16),
}


# --------------------------------------------------------------------------
# layout helpers (pure index math of the interleaved cache; no attention)
# --------------------------------------------------------------------------

def n_rows(n_raw: int, n_gist: int) -> int:
    return n_raw + n_gist


def gist_row(m: int, chunk: int) -> int:
    """Row of gist m: it follows the C raw rows of chunk m."""
    return m * (chunk + 1) + chunk


def raw_row(p: int, chunk: int, n_gist: int) -> int:
    """Row of raw position p (raw rows past the last gist are stored last)."""
    if p < n_gist * chunk:
        return (p // chunk) * (chunk + 1) + p % chunk
    return n_gist * (chunk + 1) + (p - n_gist * chunk)


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round float32/float64 values to the storage dtype (bf16: nearest-even)."""
    return x.to(torch.float32).to(_TORCH_DT[dtype])


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _plant_margin(keys: torch.Tensor, chosen: torch.Tensor, u: torch.Tensor,
                  unit_gain: float, margin: float) -> None:
    """Move rows ``chosen`` of ``keys`` (in place, fp64) along unit vector u.

    The i-th chosen row gets projection on u equal to the largest projection
    among the other rows plus (margin + 0.01 i) / unit_gain, so the chosen rows
    end up above every other row by at least ``margin`` once the projection is
    multiplied by ``unit_gain``.
    """
    proj = keys @ u
    mask = torch.ones(keys.shape[0], dtype=torch.bool, device=keys.device)
    mask[chosen] = False
    top = proj[mask].max() if bool(mask.any()) else torch.zeros((), dtype=keys.dtype,
                                                                 device=keys.device)
    steps = torch.arange(chosen.numel(), dtype=keys.dtype, device=keys.device)
    target = top + (margin + 0.01 * steps) / unit_gain
    keys[chosen] += (target - proj[chosen])[:, None] * u[None, :]


def _gap(keys64: torch.Tensor, chosen: torch.Tensor, u: torch.Tensor,
         unit_gain: float) -> float:
    """(min over chosen - max over the rest) of unit_gain * (row . u)."""
    proj = (keys64 @ u) * unit_gain
    mask = torch.ones(keys64.shape[0], dtype=torch.bool, device=keys64.device)
    mask[chosen] = False
    if not bool(mask.any()) or chosen.numel() == 0:
        return math.inf
    return float(proj[chosen].min() - proj[mask].max())


def _scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


# --------------------------------------------------------------------------
# decode inputs
# --------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    q: torch.Tensor          # [B, Hq, D]
    k_cache: torch.Tensor    # [B, Hkv, R, D]
    v_cache: torch.Tensor    # [B, Hkv, R, D]
    planted: Optional[torch.Tensor]  # [B, Hkv, k] chunk ids (ascending), or None
    seed: int                # seed actually used
    min_gap: float           # realized planted margin (scaled group score), inf if none


def _eligible_chunks(n_raw: int, chunk: int, n_gist: int, tail: int) -> int:
    """Number of leading chunks with no raw row inside the tail."""
    return max(0, min(n_gist, (n_raw - tail) // chunk))


def _decode_once(cfg: DecodeConfig, seed: int, device) -> DecodeInputs:
    B, Hq, Hkv, D = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    g = Hq // Hkv
    M, R, C, k = cfg.M, cfg.R, cfg.chunk, cfg.topk
    gen = _gen(device, seed)
    dt = _TORCH_DT[cfg.dtype]
    q = _store(torch.randn(B, Hq, D, generator=gen, device=device), cfg.dtype)
    k_cache = torch.empty(B, Hkv, R, D, dtype=dt, device=device)
    v_cache = torch.empty(B, Hkv, R, D, dtype=dt, device=device)
    n_elig = _eligible_chunks(cfg.n_raw, C, M, cfg.tail)
    do_plant = cfg.plant != "none" and 0 < k <= n_elig
    planted = torch.empty(B, Hkv, k, dtype=torch.long, device=device) if do_plant else None
    gist_rows = torch.arange(M, device=device) * (C + 1) + C
    scale = _scale(D)
    min_gap = math.inf
    for b in range(B):
        for j in range(Hkv):
            ks = torch.randn(R, D, generator=gen, device=device)
            vs = torch.randn(R, D, generator=gen, device=device)
            if do_plant:
                qbar = q[b, j * g:(j + 1) * g].double().mean(0)
                qn = float(qbar.norm())
                u = qbar / qn
                chosen = torch.randperm(n_elig, generator=gen, device=device)[:k]
                gk = ks[gist_rows].double()
                if cfg.plant == "literal":
                    # gist key = 3 * q/|q| + N(0, 0.1^2)
                    noise = torch.randn(k, D, generator=gen, device=device).double()
                    gk[chosen] = 3.0 * u[None, :] + 0.1 * noise
                else:
                    _plant_margin(gk, chosen, u, scale * qn, cfg.margin + 0.05)
                ks[gist_rows] = gk.float()
                planted[b, j] = torch.sort(chosen).values
            kq = _store(ks, cfg.dtype)
            k_cache[b, j] = kq
            v_cache[b, j] = _store(vs, cfg.dtype)
            if do_plant:
                qbar = q[b, j * g:(j + 1) * g].double().mean(0)
                qn = float(qbar.norm())
                min_gap = min(min_gap, _gap(kq[gist_rows].double(), planted[b, j],
                                            qbar / qn, scale * qn))
    return DecodeInputs(cfg, q, k_cache, v_cache, planted, seed, min_gap)


def make_decode(cfg: DecodeConfig, seed: int, device="cpu", max_tries: int = 64) -> DecodeInputs:
    """Seeded decode inputs; re-seeds (seed+1, seed+2, ...) until the realized
    planted gap reaches ``cfg.margin``. The seed used is recorded."""
    for t in range(max_tries):
        inp = _decode_once(cfg, seed + t, device)
        if inp.planted is None or inp.min_gap >= cfg.margin:
            return inp
    raise RuntimeError(f"{cfg.name}: no seed in [{seed}, {seed + max_tries}) reached "
                       f"planted gap {cfg.margin}")


# --------------------------------------------------------------------------
# two-level (gist-of-gist) inputs
# --------------------------------------------------------------------------

@dataclasses.dataclass
class HierInputs:
    cfg: HierConfig
    q: torch.Tensor          # [B, Hq, D]
    k_cache: torch.Tensor    # [B, Hkv, R, D] level-1 interleaved cache
    v_cache: torch.Tensor
    k_l2: torch.Tensor       # [B, Hkv, M2, D] level-2 gists
    v_l2: torch.Tensor
    planted2: Optional[torch.Tensor]  # [B, Hkv, k2] level-2 group ids (ascending)
    planted1: Optional[torch.Tensor]  # [B, Hkv, k1] level-1 chunk ids (ascending)
    seed: int
    min_gap2: float
    min_gap1: float


def _hier_once(cfg: HierConfig, seed: int, device) -> HierInputs:
    base = cfg.base
    B, Hq, Hkv, D = base.batch, base.n_q_heads, base.n_kv_heads, base.head_dim
    g = Hq // Hkv
    M, R, C = base.M, base.R, base.chunk
    G, k1, k2, M2 = cfg.fanout, base.topk, cfg.topk2, cfg.M2
    gen = _gen(device, seed)
    dt = _TORCH_DT[base.dtype]
    q = _store(torch.randn(B, Hq, D, generator=gen, device=device), base.dtype)
    k_cache = torch.empty(B, Hkv, R, D, dtype=dt, device=device)
    v_cache = torch.empty(B, Hkv, R, D, dtype=dt, device=device)
    k_l2 = torch.empty(B, Hkv, M2, D, dtype=dt, device=device)
    v_l2 = torch.empty(B, Hkv, M2, D, dtype=dt, device=device)
    # groups whose every child chunk lies before the tail
    n_elig_groups = max(0, min(M2, ((base.n_raw - base.tail) // C) // G))
    per = k1 // k2 if k2 > 0 else 0
    do_plant = (base.plant != "none" and 0 < k2 <= n_elig_groups and per >= 1
                and per * k2 == k1 and per <= G)
    planted2 = torch.empty(B, Hkv, k2, dtype=torch.long, device=device) if do_plant else None
    planted1 = torch.empty(B, Hkv, k1, dtype=torch.long, device=device) if do_plant else None
    scale = _scale(D)
    gap2 = gap1 = math.inf
    for b in range(B):
        for j in range(Hkv):
            ks = torch.randn(R, D, generator=gen, device=device)
            vs = torch.randn(R, D, generator=gen, device=device)
            k2s = torch.randn(M2, D, generator=gen, device=device)
            v2s = torch.randn(M2, D, generator=gen, device=device)
            qbar = q[b, j * g:(j + 1) * g].double().mean(0)
            qn = float(qbar.norm())
            u = qbar / qn
            if do_plant:
                ch2 = torch.sort(torch.randperm(n_elig_groups, generator=gen,
                                                device=device)[:k2]).values
                g2 = k2s.double()
                _plant_margin(g2, ch2, u, scale * qn, base.margin + 0.05)
                k2s = g2.float()
                # children of the planted groups: plant `per` per group
                cand = (ch2[:, None] * G + torch.arange(G, device=device)[None, :]).reshape(-1)
                pick = torch.stack([torch.randperm(G, generator=gen, device=device)[:per]
                                    for _ in range(k2)])          # [k2, per]
                ch1_local = (torch.arange(k2, device=device)[:, None] * G + pick).reshape(-1)
                rows = cand * (C + 1) + C
                g1 = ks[rows].double()
                _plant_margin(g1, ch1_local, u, scale * qn, base.margin + 0.05)
                ks[rows] = g1.float()
                planted2[b, j] = ch2
                planted1[b, j] = torch.sort(cand[ch1_local]).values
            kq = _store(ks, base.dtype)
            k2q = _store(k2s, base.dtype)
            k_cache[b, j] = kq
            v_cache[b, j] = _store(vs, base.dtype)
            k_l2[b, j] = k2q
            v_l2[b, j] = _store(v2s, base.dtype)
            if do_plant:
                gap2 = min(gap2, _gap(k2q.double(), planted2[b, j], u, scale * qn))
                cand = (planted2[b, j][:, None] * G
                        + torch.arange(G, device=device)[None, :]).reshape(-1)
                rows = cand * (C + 1) + C
                local = torch.searchsorted(cand, planted1[b, j])
                gap1 = min(gap1, _gap(kq[rows].double(), local, u, scale * qn))
    return HierInputs(cfg, q, k_cache, v_cache, k_l2, v_l2, planted2, planted1, seed,
                      gap2, gap1)


def make_hier(cfg: HierConfig, seed: int, device="cpu", max_tries: int = 64) -> HierInputs:
    for t in range(max_tries):
        inp = _hier_once(cfg, seed + t, device)
        if inp.planted2 is None or min(inp.min_gap2, inp.min_gap1) >= cfg.base.margin:
            return inp
    raise RuntimeError(f"{cfg.name}: no seed reached the planted gap")


# --------------------------------------------------------------------------
# prefill inputs
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillInputs:
    cfg: PrefillConfig
    q: torch.Tensor          # [Hq, n_q, D] queries at raw positions q_start + i
    k_cache: torch.Tensor    # [Hkv, R, D]
    v_cache: torch.Tensor
    planted: Optional[torch.Tensor]  # [n_blocks, Hkv, k] chunk ids per query block
    seed: int
    min_gap: float           # realized min over (query, kv-head) of planted gap


def _prefill_once(cfg: PrefillConfig, seed: int, device, check: bool) -> PrefillInputs:
    Hq, Hkv, D, C = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.chunk
    g = Hq // Hkv
    M, R, k, W = cfg.M, cfg.R, cfg.topk, cfg.window
    nq, qb, q0 = cfg.n_q, cfg.q_block, cfg.q_start
    nblk = (nq + qb - 1) // qb
    gen = _gen(device, seed)
    dt = _TORCH_DT[cfg.dtype]
    scale = _scale(D)
    if cfg.values == "int":
        # small integers: every dot product is exact in fp32 and fp64, so equal
        # group scores are equal on both sides and ties are decided by index
        def ints(*shape):
            return torch.randint(-2, 3, shape, generator=gen, device=device).to(torch.float32)
        q = _store(ints(Hq, nq, D), cfg.dtype)
        k_cache = _store(ints(Hkv, R, D), cfg.dtype)
        v_cache = _store(ints(Hkv, R, D), cfg.dtype)
        return PrefillInputs(cfg, q, k_cache, v_cache, None, seed, math.inf)
    # chunks complete before the first query and clear of every window
    n_far = max(0, min(M, (q0 - W) // C))
    do_plant = k > 0 and nblk * k <= n_far
    z = torch.randn(Hq, nq, D, generator=gen, device=device)
    ks = torch.randn(Hkv, R, D, generator=gen, device=device)
    vs = torch.randn(Hkv, R, D, generator=gen, device=device)
    planted = None
    min_gap = math.inf
    if do_plant:
        planted = torch.empty(nblk, Hkv, k, dtype=torch.long, device=device)
        # one direction per query block; orthonormal across the blocks of a kv
        # group (when there are at most D blocks) so that a block's planted keys
        # do not lift the scores another block sees
        u = torch.empty(nblk, Hkv, D, dtype=torch.float64, device=device)
        for j in range(Hkv):
            a = torch.randn(D, nblk, generator=gen, device=device).double()
            if nblk <= D:
                qmat, _ = torch.linalg.qr(a.cpu())
                u[:, j] = qmat.T.to(device)
            else:
                u[:, j] = (a / a.norm(dim=0, keepdim=True)).T
        # shared direction per (query block, kv group) on every head of the group
        qf = z.double().view(Hkv, g, nq, D)
        ublk = u.repeat_interleave(qb, dim=0)[:nq]                 # [nq, Hkv, D]
        qf = qf + cfg.alpha * ublk.permute(1, 0, 2)[:, None, :, :]
        q = _store(qf.view(Hq, nq, D), cfg.dtype)
        gist_rows = torch.arange(M, device=device) * (C + 1) + C
        for j in range(Hkv):
            perm = torch.randperm(n_far, generator=gen, device=device)[:nblk * k].view(nblk, k)
            planted[:, j] = torch.sort(perm, dim=1).values
        # planted key of block b = tau_b * u_b + 0.25 * noise; tau_b from the
        # block's weakest query so every query of the block clears the margin
        qbar = q.double().view(Hkv, g, nq, D).mean(1)             # [Hkv, nq, D]
        gk = ks[:, gist_rows].double()                            # [Hkv, M, D]
        noise = torch.randn(nblk, Hkv, k, D, generator=gen, device=device).double() * 0.25
        for j in range(Hkv):
            for b in range(nblk):
                gk[j, planted[b, j]] = noise[b, j]
        for _ in range(3):
            for j in range(Hkv):
                for b in range(nblk):
                    t0, t1 = b * qb, min(nq, (b + 1) * qb)
                    qq = qbar[j, t0:t1]                          # [nb, D]
                    s = (qq @ gk[j].T) * scale                    # [nb, M]
                    mask = torch.ones(M, dtype=torch.bool, device=device)
                    mask[planted[b, j]] = False
                    # eligible gists of query t: m < floor(t / C)
                    pos = q0 + torch.arange(t0, t1, device=device)
                    elig = torch.arange(M, device=device)[None, :] < (pos // C)[:, None]
                    other = torch.where(mask[None, :] & elig, s, torch.full_like(s, -math.inf))
                    need = other.max(dim=1).values + cfg.margin + 0.3
                    along = (qq @ u[b, j]) * scale                # [nb]
                    base = (qq @ noise[b, j].T) * scale            # [nb, k]
                    tau = float(((need[:, None] - base) / along[:, None]).max())
                    tau = max(tau, 1.0)
                    gk[j, planted[b, j]] = tau * u[b, j][None, :] + noise[b, j]
        ks[:, gist_rows] = gk.float()
    else:
        q = _store(z, cfg.dtype)
    k_cache = _store(ks, cfg.dtype)
    v_cache = _store(vs, cfg.dtype)
    if do_plant and check:
        gkq = k_cache[:, torch.arange(M, device=device) * (C + 1) + C].double()
        qbar = q.double().view(Hkv, g, nq, D).mean(1)
        for j in range(Hkv):
            s = (qbar[j] @ gkq[j].T) * scale                          # [nq, M]
            pos = q0 + torch.arange(nq, device=device)
            elig = torch.arange(M, device=device)[None, :] < (pos // C)[:, None]
            blk = torch.arange(nq, device=device) // qb
            pmask = torch.zeros(nq, M, dtype=torch.bool, device=device)
            pmask[torch.arange(nq, device=device)[:, None], planted[blk, j]] = True
            lo = torch.where(pmask, s, torch.full_like(s, math.inf)).min(1).values
            hi = torch.where(~pmask & elig, s, torch.full_like(s, -math.inf)).max(1).values
            min_gap = min(min_gap, float((lo - hi).min()))
    return PrefillInputs(cfg, q, k_cache, v_cache, planted, seed, min_gap)


def make_prefill(cfg: PrefillConfig, seed: int, device="cpu", max_tries: int = 16,
                 check: bool = True) -> PrefillInputs:
    for t in range(max_tries):
        inp = _prefill_once(cfg, seed + t, device, check)
        if inp.planted is None or not check or inp.min_gap >= cfg.margin:
            return inp
    raise RuntimeError(f"{cfg.name}: no seed reached the planted gap")


# --------------------------------------------------------------------------
# gist-token queries and token streams (plain Gaussian values)
# --------------------------------------------------------------------------

def make_gist(n_q_heads: int, n_kv_heads: int, head_dim: int, n_raw: int, n_gist: int,
              n_q: int, seed: int, device="cpu", dtype: str = "bf16"):
    """Gist-token queries q [Hq, n_q, D] and a one-sequence interleaved cache
    k, v [Hkv, N + M, D], all i.i.d. standard normal, rounded to `dtype`."""
    g = _gen(device, seed)
    R = n_raw + n_gist
    q = torch.randn(n_q_heads, n_q, head_dim, generator=g, device=device)
    k = torch.randn(n_kv_heads, R, head_dim, generator=g, device=device)
    v = torch.randn(n_kv_heads, R, head_dim, generator=g, device=device)
    return _store(q, dtype), _store(k, dtype), _store(v, dtype)


@dataclasses.dataclass
class TokenStream:
    """K/V rows of a batch of sequences generated token by token."""
    raw_k: torch.Tensor      # [steps, B, Hkv, D] row of raw token p at [p]
    raw_v: torch.Tensor
    gist_k: torch.Tensor     # [n_chunks, B, Hkv, D] row of the gist of chunk m at [m]
    gist_v: torch.Tensor
    gist_q: torch.Tensor     # [n_chunks, B, Hq, D] query of the gist token of chunk m
    q: torch.Tensor          # [B, Hq, D] query of the token after the stream


def make_token_stream(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, steps: int,
                      chunk: int, seed: int, device="cpu", dtype: str = "bf16") -> TokenStream:
    g = _gen(device, seed)
    nc = steps // chunk

    def r(*shape):
        return _store(torch.randn(*shape, head_dim, generator=g, device=device), dtype)
    return TokenStream(r(steps, batch, n_kv_heads), r(steps, batch, n_kv_heads),
                       r(nc, batch, n_kv_heads), r(nc, batch, n_kv_heads),
                       r(nc, batch, n_q_heads), r(batch, n_q_heads))


# --------------------------------------------------------------------------
# L-level decode inputs
# --------------------------------------------------------------------------

def level_sizes(n_gist: int, fanout: int, n_levels: int):
    """[M_1, ..., M_L], M_l = floor(M_{l-1} / G)."""
    sizes = [n_gist]
    for _ in range(n_levels - 1):
        sizes.append(sizes[-1] // fanout)
    return sizes


def make_levels(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, n_raw: int, n_gist: int,
                chunk: int, fanout: int, n_levels: int, seed: int, device="cpu", dtype: str = "bf16",
                values: str = "int"):
    """q [B, Hq, D], the interleaved cache [B, Hkv, N + M, D] and the level
    arrays [B, Hkv, M_l, D] for l = 2..L. values="int": entries uniform in
    {-2..2} (exact group scores, many ties); "gauss": N(0, 1). Built in
    slices so that long caches need no full-size float32 temporaries."""
    g = _gen(device, seed)
    D = head_dim

    def draw(*shape):
        out = torch.empty(*shape, D, dtype=_TORCH_DT[dtype], device=device)
        flat = out.view(-1, D)
        step = 1 << 20
        for i in range(0, flat.shape[0], step):
            n = min(step, flat.shape[0] - i)
            if values == "int":
                x = torch.randint(-2, 3, (n, D), generator=g, device=device).float()
            else:
                x = torch.randn(n, D, generator=g, device=device)
            flat[i:i + n] = x.to(out.dtype)
        return out
    R = n_raw + n_gist
    q = draw(batch, n_q_heads)
    k = draw(batch, n_kv_heads, R)
    v = draw(batch, n_kv_heads, R)
    sizes = level_sizes(n_gist, fanout, n_levels)
    k_up = [draw(batch, n_kv_heads, m) for m in sizes[1:]]
    v_up = [draw(batch, n_kv_heads, m) for m in sizes[1:]]
    return q, k, v, k_up, v_up


def to_pages(k_cache, v_cache, rows, page_chunks: int, chunk: int, seed: int, spare: int = 3):
    """Scatter dense caches [B, Hkv, cap, D] into shuffled page pools: sequence
    b's first rows[b] rows go page by page (P(C+1) rows each) to distinct
    random pages of one pool, `spare` unused pages (random values) mixed in.
    Returns (k_pool, v_pool [n_pages, Hkv, P(C+1), D], block_table [B,
    max_pages] int32 with -1 past a sequence's pages)."""
    B, Hkv, cap, D = k_cache.shape
    rpp = page_chunks * (chunk + 1)
    need = [-(-int(r) // rpp) for r in rows]
    max_pages = max(1, max(need))
    n_pages = sum(need) + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages)
    g = torch.Generator(device="cpu").manual_seed(seed)
    k_pool = torch.randn(n_pages, Hkv, rpp, D, generator=g).to(k_cache.dtype).to(k_cache.device)
    v_pool = torch.randn(n_pages, Hkv, rpp, D, generator=g).to(k_cache.dtype).to(k_cache.device)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    nxt = 0
    for b in range(B):
        for i in range(need[b]):
            pg = int(perm[nxt])
            nxt += 1
            table[b, i] = pg
            r0, r1 = i * rpp, min(int(rows[b]), (i + 1) * rpp)
            k_pool[pg, :, :r1 - r0] = k_cache[b, :, r0:r1]
            v_pool[pg, :, :r1 - r0] = v_cache[b, :, r0:r1]
    return k_pool, v_pool, table


def varlen_lengths(batch: int, n_min: int, n_max: int, chunk: int, seed: int):
    """Per-sequence (n_raw, n_gist) with n_raw uniform in [n_min, n_max] and
    every complete chunk gisted, except that a sequence ending on a chunk
    boundary leaves its last chunk's gist out half of the time (a full chunk
    waiting for its gist)."""
    rng = np.random.default_rng(seed)
    n = rng.integers(n_min, n_max + 1, size=batch)
    m = n // chunk
    drop = (n % chunk == 0) & (rng.random(batch) < 0.5) & (m > 0)
    m = m - drop.astype(n.dtype)
    return [int(x) for x in n], [int(x) for x in m]

