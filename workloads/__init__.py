"""Seeded synthetic inputs for the verification pass.

This module only draws random numbers and stores them; it holds none of the
verification arithmetic. Both the CPU oracle's tests and the GPU path's tests
and benchmark take their inputs from here.

The pages' workloads are trained-model logits on public benchmarks
([DualDiffusion] §4 "Results": MMLU and GSM8K; [COVER] "Results": HumanEval,
MBPP, GSM8K, MATH500 at generation length 512; [SPOT] §3: SDAR-8B). No
weights or datasets are used here: synthetic logits stand in for them, with
the pages' sequence lengths and vocabulary sizes of that size class.

Recipes (values drawn in float32, then rounded to bfloat16 round-to-nearest-
even where the workload is bf16; the drafter is formed from the float32
verifier before rounding and each tensor is rounded on its own):

* ``peaked``  (workloads 1, 3, 4, 5): verifier a ~ N(0, 2^2) plus +6 at one
  uniformly chosen token per row; drafter b = a + N(0, 0.5^2).
* ``spiked``  (workload 2): a ~ N(0, 1); in 90% of rows (Bernoulli) +8 at a
  uniformly chosen token; b = a + N(0, 1). In 15% of the spiked rows the
  drafter's spike moves: -8 at the old token and +8 at another uniformly
  chosen token.

Random streams: numpy PCG64 seeded by SeedSequence(seed, spawn_key=(workload,
sequence, stream)); the torch backend (used for sizes numpy would take minutes
to draw) seeds a device generator from the same SeedSequence, so its values
follow the same recipe but not the same stream.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["WORKLOADS", "Workload", "workload", "rng_for", "round_bf16_bits",
           "peaked_logits", "spiked_logits", "make_logits_numpy", "make_logits_torch",
           "subject_rows", "committed_rows", "diffusion_inputs", "positions"]

# stream ids inside one (workload, sequence) seed
_S_LOGITS, _S_SUBJECT, _S_COMMITTED, _S_DIN, _S_DOUT = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    """Shape and parameters of one synthetic workload."""
    name: str
    number: int
    B: int                 # sequences (or candidates x ... see ``rows``)
    L: int                 # rows per sequence
    V: int
    dtype: str             # "fp32" or "bf16"
    recipe: str            # "peaked" or "spiked"
    temperature: float
    seed: int = 0
    tau_kl: float = 0.0
    conf_thr: float = 0.0
    pos_period: int = 0    # 0: position = row index; >0: position = row % pos_period
    group_len: int = 0     # rows per candidate for coupled-noise acceptance
    n_subject: int = 0     # rows flagged as newly drafted (0: all rows)
    n_committed: int = 0   # rows with seed-score inputs (0: none)
    topk: int = 0
    rules: tuple = field(default_factory=tuple)

    @property
    def rows(self) -> int:
        return self.B * self.L

    @property
    def elt(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def input_bytes(self) -> int:
        return 2 * self.rows * self.V * self.elt


WORKLOADS = {
    1: Workload("tiny-fp32", 1, 1, 64, 1024, "fp32", "peaked", 0.0, tau_kl=0.1, conf_thr=0.9,
                n_subject=16, rules=("KL", "CONF", "KL_OR_CONF", "TRUST")),
    2: Workload("single-seq-remask", 2, 1, 512, 126464, "bf16", "spiked", 0.0, tau_kl=0.05,
                conf_thr=0.9, rules=("KL", "CONF", "KL_OR_CONF")),
    3: Workload("cover-revision", 3, 1, 512, 152064, "bf16", "peaked", 0.0, conf_thr=0.9,
                n_committed=256, topk=32, rules=("COVER",)),
    4: Workload("spot-tree-coupled", 4, 64, 32, 151936, "bf16", "peaked", 1.0, pos_period=32,
                group_len=32, rules=("COUPLED_ACCEPT",)),
    5: Workload("throughput-32x1024", 5, 32, 1024, 126464, "bf16", "peaked", 1.0, topk=64,
                rules=("KL",)),
}


def workload(n: int) -> Workload:
    return WORKLOADS[int(n)]


def rng_for(number: int, seq: int, stream: int, seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(number, seq, stream))))


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def peaked_logits(rows: int, V: int, rng: np.random.Generator, sigma: float = 2.0,
                  boost: float = 6.0, drafter_sigma: float = 0.5):
    """float32 (a, b) for the ``peaked`` recipe."""
    a = (rng.standard_normal((rows, V), dtype=np.float32) * np.float32(sigma))
    tok = rng.integers(0, V, size=rows)
    a[np.arange(rows), tok] += np.float32(boost)
    b = a + rng.standard_normal((rows, V), dtype=np.float32) * np.float32(drafter_sigma)
    return a, b


def spiked_logits(rows: int, V: int, rng: np.random.Generator, p_spike: float = 0.9,
                  spike: float = 8.0, drafter_sigma: float = 1.0, p_move: float = 0.15):
    """float32 (a, b) for the ``spiked`` recipe."""
    a = rng.standard_normal((rows, V), dtype=np.float32)
    spiked = rng.random(rows) < p_spike
    tok = rng.integers(0, V, size=rows)
    r = np.nonzero(spiked)[0]
    a[r, tok[r]] += np.float32(spike)
    b = a + rng.standard_normal((rows, V), dtype=np.float32) * np.float32(drafter_sigma)
    move = spiked & (rng.random(rows) < p_move)
    other = (tok + 1 + rng.integers(0, V - 1, size=rows)) % V
    m = np.nonzero(move)[0]
    b[m, tok[m]] -= np.float32(spike)
    b[m, other[m]] += np.float32(spike)
    return a, b


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "fp32" else round_bf16_bits(x)


def make_logits_numpy(w: Workload, seqs=None):
    """(verifier, drafter) arrays [len(seqs) * L, V] as stored on the device:
    float32 values for fp32 workloads, uint16 bfloat16 bit patterns for bf16.
    """
    seqs = range(w.B) if seqs is None else seqs
    L = w.L
    va, vb = [], []
    for s in seqs:
        g = rng_for(w.number, s, _S_LOGITS, w.seed)
        if w.recipe == "peaked":
            a, b = peaked_logits(L, w.V, g)
        else:
            a, b = spiked_logits(L, w.V, g)
        va.append(_store(a, w.dtype))
        vb.append(_store(b, w.dtype))
    return np.concatenate(va), np.concatenate(vb)


def make_logits_torch(w: Workload, device, seqs=None, out=None):
    """(verifier, drafter) torch tensors [len(seqs) * L, V] on ``device``,
    bfloat16 or float32, drawn with the recipe on the device.

    When ``out`` = (va, vb) is given the rows are written into those tensors.
    """
    import torch

    seqs = list(range(w.B)) if seqs is None else list(seqs)
    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    n = len(seqs) * w.L
    if out is None:
        va = torch.empty((n, w.V), dtype=tdt, device=device)
        vb = torch.empty((n, w.V), dtype=tdt, device=device)
    else:
        va, vb = out
    gen = torch.Generator(device=device)
    for j, s in enumerate(seqs):
        ss = np.random.SeedSequence(w.seed, spawn_key=(w.number, s, _S_LOGITS))
        gen.manual_seed(int(ss.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF))
        L, V = w.L, w.V
        if w.recipe == "peaked":
            a = torch.randn((L, V), generator=gen, device=device, dtype=torch.float32) * 2.0
            tok = torch.randint(0, V, (L,), generator=gen, device=device)
            a[torch.arange(L, device=device), tok] += 6.0
            b = a + torch.randn((L, V), generator=gen, device=device, dtype=torch.float32) * 0.5
        else:
            a = torch.randn((L, V), generator=gen, device=device, dtype=torch.float32)
            spiked = torch.rand((L,), generator=gen, device=device) < 0.9
            tok = torch.randint(0, V, (L,), generator=gen, device=device)
            ar = torch.arange(L, device=device)
            a[ar[spiked], tok[spiked]] += 8.0
            b = a + torch.randn((L, V), generator=gen, device=device, dtype=torch.float32)
            move = spiked & (torch.rand((L,), generator=gen, device=device) < 0.15)
            other = (tok + 1 + torch.randint(0, V - 1, (L,), generator=gen, device=device)) % V
            b[ar[move], tok[move]] -= 8.0
            b[ar[move], other[move]] += 8.0
        va[j * w.L:(j + 1) * w.L].copy_(a.to(tdt))
        vb[j * w.L:(j + 1) * w.L].copy_(b.to(tdt))
        del a, b
    return va, vb


def subject_rows(w: Workload) -> np.ndarray | None:
    """uint8 [rows] mask of rows flagged as newly drafted (None: all rows)."""
    if not w.n_subject:
        return None
    m = np.zeros(w.rows, np.uint8)
    for s in range(w.B):
        perm = rng_for(w.number, s, _S_SUBJECT, w.seed).permutation(w.L)[:w.n_subject]
        m[s * w.L + perm] = 1
    return m


def committed_rows(w: Workload) -> np.ndarray | None:
    """uint8 [rows] mask of committed positions that may become seeds."""
    if not w.n_committed:
        return None
    m = np.zeros(w.rows, np.uint8)
    for s in range(w.B):
        perm = rng_for(w.number, s, _S_COMMITTED, w.seed).permutation(w.L)[:w.n_committed]
        m[s * w.L + perm] = 1
    return m


def diffusion_inputs(w: Workload):
    """float32 (d_in, d_out) per row, each ~ U[0, 1)."""
    d_in = np.concatenate([rng_for(w.number, s, _S_DIN, w.seed).random(w.L, dtype=np.float32)
                           for s in range(w.B)])
    d_out = np.concatenate([rng_for(w.number, s, _S_DOUT, w.seed).random(w.L, dtype=np.float32)
                            for s in range(w.B)])
    return d_in, d_out


def positions(w: Workload) -> np.ndarray:
    """int32 position of every row (what the noise is keyed on)."""
    r = np.arange(w.rows, dtype=np.int64)
    if w.pos_period:
        r = r % w.pos_period
    return r.astype(np.int32)
