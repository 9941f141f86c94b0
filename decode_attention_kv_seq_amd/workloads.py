"""Seeded synthetic inputs for single-query decode attention.

This module only draws numbers: it holds none of the attention arithmetic
(no dot products, no softmax, no weighted sums).  It is the one place that
both the GPU path's callers (tests, bench) and the CPU oracle's callers get
their inputs from, so the two sides always see the same bits.

Generator
---------
Every value is a pure function of ``(seed, stream, flat element index)``:

* ``word(i)`` is the SplitMix64 output for counter ``i``: the state
  ``key + (i + 1) * GAMMA`` (mod 2**64) passed through the 64-bit finaliser
  published by Steele, Lea and Flood ("Fast splittable pseudorandom number
  generators", OOPSLA 2014; constants of Stafford's "variant 13" mixer).
* ``key = mix64(seed * GAMMA + stream * GAMMA2 + 1)`` separates the streams
  (0 = Q, 1 = K, 2 = V, 3 = extra draws such as positions).
* An approximately normal value is the standardised Irwin-Hall sum of the
  word's four 16-bit fields: ``c = sum(u_j) - 2*65535`` (an integer, exact
  in fp32), ``x = fp32(c) * fp32(sigma / sd)`` with
  ``sd = sqrt(4 * (65536**2 - 1) / 12)``, then rounded to fp16
  (round-to-nearest-even).  Mean 0, standard deviation ``sigma``, support
  bounded at about +-3.46 sigma.

All steps are integer operations, one fp32 multiply and one fp32->fp16
rounding, so a CPU tensor and a GPU tensor built from the same indices hold
identical bits.  That lets the GPU fill multi-GiB caches in a fraction of a
second while the oracle regenerates, on the host, only the heads it checks.

Workloads
---------
Five shapes of single-query decode attention over an fp16 cache laid out
``[seq_len, n_heads, head_dim]`` (batched: ``[batch, capacity, n_heads,
head_dim]``), with Q and output ``[n_heads, head_dim]``.  The page "Developing
Apple Metal Kernels in Rust - A Deep Dive Through Attention" (section "The
MSL, briefly") fixes these layouts and the ``current_pos`` mask; its
"Testing" section fixes the three small cases in ``PAGE_CASES``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

_U64 = 1 << 64


def _s64(x: int) -> int:
    """Two's-complement int64 view of an unsigned 64-bit constant."""
    x %= _U64
    return x - _U64 if x >= (1 << 63) else x


GAMMA = 0x9E3779B97F4A7C15
GAMMA2 = 0xD1B54A32D192ED03
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB

STREAM_Q, STREAM_K, STREAM_V, STREAM_EXTRA = 0, 1, 2, 3

# standard deviation of a sum of four independent uniform 16-bit integers
IRWIN_HALL_SD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
IRWIN_HALL_CENTRE = 2 * 65535


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    # logical right shift of an int64 tensor holding uint64 bits
    return torch.bitwise_and(torch.bitwise_right_shift(z, s), (1 << (64 - s)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 finaliser on int64 tensors (wrapping arithmetic)."""
    z = torch.bitwise_xor(z, _lsr(z, 30)) * _s64(M1)
    z = torch.bitwise_xor(z, _lsr(z, 27)) * _s64(M2)
    return torch.bitwise_xor(z, _lsr(z, 31))


def _mix64_int(z: int) -> int:
    z %= _U64
    z = ((z ^ (z >> 30)) * M1) % _U64
    z = ((z ^ (z >> 27)) * M2) % _U64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    """int64 view of the per-stream key."""
    return _s64(_mix64_int(seed * GAMMA + stream * GAMMA2 + 1))


def words(seed: int, stream: int, index: torch.Tensor) -> torch.Tensor:
    """uint64 words (as int64 bits) for the given int64 counters."""
    state = (index + 1) * _s64(GAMMA) + stream_key(seed, stream)
    return mix64(state)


_CPU_CHUNK = 1 << 16   # keeps the int64 temporaries cache-resident on the host


def normal_f16(seed: int, stream: int, index: torch.Tensor, sigma: float) -> torch.Tensor:
    """fp16 approximately-N(0, sigma^2) values for int64 counters ``index``."""
    if index.device.type == "cpu" and index.numel() > _CPU_CHUNK:
        flat = index.reshape(-1)
        out = torch.empty(flat.shape, dtype=torch.float16)
        for lo in range(0, flat.numel(), _CPU_CHUNK):
            out[lo:lo + _CPU_CHUNK] = _normal_f16(seed, stream, flat[lo:lo + _CPU_CHUNK], sigma)
        return out.view(index.shape)
    return _normal_f16(seed, stream, index, sigma)


def _normal_f16(seed: int, stream: int, index: torch.Tensor, sigma: float) -> torch.Tensor:
    w = words(seed, stream, index)
    total = torch.bitwise_and(w, 0xFFFF)
    for shift in (16, 32, 48):
        total = total + torch.bitwise_and(torch.bitwise_right_shift(w, shift), 0xFFFF)
    c = (total - IRWIN_HALL_CENTRE).to(torch.float32)
    scale = torch.tensor(sigma / IRWIN_HALL_SD, dtype=torch.float32, device=index.device)
    return (c * scale).to(torch.float16)


def normal_f32(seed: int, stream: int, index: torch.Tensor, sigma: float) -> torch.Tensor:
    """The same values as ``normal_f16`` before its final rounding: fp32."""
    if index.device.type == "cpu" and index.numel() > _CPU_CHUNK:
        flat = index.reshape(-1)
        out = torch.empty(flat.shape, dtype=torch.float32)
        for lo in range(0, flat.numel(), _CPU_CHUNK):
            out[lo:lo + _CPU_CHUNK] = _normal_f32(seed, stream, flat[lo:lo + _CPU_CHUNK], sigma)
        return out.view(index.shape)
    return _normal_f32(seed, stream, index, sigma)


def _normal_f32(seed: int, stream: int, index: torch.Tensor, sigma: float) -> torch.Tensor:
    w = words(seed, stream, index)
    total = torch.bitwise_and(w, 0xFFFF)
    for shift in (16, 32, 48):
        total = total + torch.bitwise_and(torch.bitwise_right_shift(w, shift), 0xFFFF)
    c = (total - IRWIN_HALL_CENTRE).to(torch.float32)
    return c * torch.tensor(sigma / IRWIN_HALL_SD, dtype=torch.float32, device=index.device)


def uniform_u64(seed: int, stream: int, index: torch.Tensor) -> torch.Tensor:
    return words(seed, stream, index)


def fill_normal_(out: torch.Tensor, seed: int, stream: int, sigma: float,
                 start: int = 0, chunk: int = 1 << 26) -> torch.Tensor:
    """Fill a contiguous fp16 tensor: element i gets value(start + i)."""
    assert out.dtype == torch.float16 and out.is_contiguous()
    flat = out.view(-1)
    n = flat.numel()
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        idx = torch.arange(start + lo, start + hi, dtype=torch.int64, device=out.device)
        flat[lo:hi] = normal_f16(seed, stream, idx, sigma)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode-attention problem.

    ``cur_pos`` is the index of the newest cached token for a single
    sequence; ``None`` means a ragged batch whose per-sequence positions are
    drawn uniformly from ``[0, capacity-1]`` on the extra stream.
    """
    name: str
    n_heads: int
    head_dim: int
    seq_len: int                      # capacity per sequence
    cur_pos: Optional[int]
    seed: int
    batch: int = 1
    sigma_q: float = 1.0
    sigma_kv: float = 1.0
    garbage_sigma: Optional[float] = None   # K/V rows beyond cur_pos
    spike_fraction: float = 0.0             # share of K rows scaled
    spike_scale: float = 8.0
    page_size: int = 0                      # > 0: the cache lives in a paged pool

    @property
    def batched(self) -> bool:
        return self.cur_pos is None

    def positions(self) -> torch.Tensor:
        """Per-sequence current_pos as int64 [batch] (host)."""
        if not self.batched:
            return torch.full((self.batch,), self.cur_pos, dtype=torch.int64)
        idx = torch.arange(self.batch, dtype=torch.int64)
        w = uniform_u64(self.seed, STREAM_EXTRA, idx)
        # capacity is a power of two in every workload that uses this
        assert self.seq_len & (self.seq_len - 1) == 0
        return torch.bitwise_and(w, self.seq_len - 1)

    def valid_len(self, b: int = 0) -> int:
        cp = int(self.positions()[b])
        return min(cp, self.seq_len - 1) + 1

    def spike_rows(self) -> torch.Tensor:
        """Sorted K row indices (positions) that get scaled, host int64."""
        n = int(round(self.spike_fraction * self.seq_len))
        if n == 0:
            return torch.zeros(0, dtype=torch.int64)
        idx = torch.arange(self.seq_len, dtype=torch.int64)
        w = uniform_u64(self.seed, STREAM_EXTRA, idx + (1 << 40))
        # rank by the word as unsigned: flip the sign bit so signed order matches
        key = torch.bitwise_xor(w, -(1 << 63))
        order = torch.argsort(key, stable=True)
        return torch.sort(order[:n]).values

    @property
    def kv_shape(self):
        return (self.batch, self.seq_len, self.n_heads, self.head_dim)

    @property
    def q_shape(self):
        return (self.batch, self.n_heads, self.head_dim)

    @property
    def paged(self) -> bool:
        return self.page_size > 0

    @property
    def max_blocks(self) -> int:
        return -(-self.seq_len // self.page_size)

    @property
    def num_blocks(self) -> int:
        """Pool pages: exactly enough for every sequence's full capacity."""
        return self.batch * self.max_blocks

    @property
    def pool_shape(self):
        return (self.num_blocks, self.page_size, self.n_heads, self.head_dim)

    def block_table(self) -> torch.Tensor:
        """int64 [batch, max_blocks]: a seeded permutation of all pool pages,
        so each sequence's pages are scattered through the pool."""
        n = self.num_blocks
        w = uniform_u64(self.seed, STREAM_EXTRA, torch.arange(n, dtype=torch.int64) + (1 << 41))
        order = torch.argsort(torch.bitwise_xor(w, -(1 << 63)), stable=True)
        return order.view(self.batch, self.max_blocks)

    def kv_bytes_read(self) -> int:
        """Algorithmic K+V bytes: rows p <= current_pos of every head."""
        lens = torch.clamp(self.positions(), max=self.seq_len - 1) + 1
        return int(lens.sum()) * self.n_heads * self.head_dim * 2 * 2


def make_q(w: Workload, device="cpu") -> torch.Tensor:
    q = torch.empty(w.q_shape, dtype=torch.float16, device=device)
    return fill_normal_(q, w.seed, STREAM_Q, w.sigma_q)


def _fill_kv(t: torch.Tensor, w: Workload, stream: int, device) -> None:
    fill_normal_(t, w.seed, stream, w.sigma_kv)
    row = w.n_heads * w.head_dim
    if w.garbage_sigma is not None and not w.batched:
        lo = min(w.cur_pos, w.seq_len - 1) + 1
        if lo < w.seq_len:
            for b in range(w.batch):
                base = (b * w.seq_len + lo) * row
                fill_normal_(t[b, lo:], w.seed, stream, w.garbage_sigma, start=base)
    if stream == STREAM_K and w.spike_fraction > 0:
        rows = w.spike_rows().to(device)
        t[:, rows] = t[:, rows] * w.spike_scale


def make_kv(w: Workload, device="cpu"):
    """Full K and V caches [batch, seq_len, n_heads, head_dim] fp16."""
    k = torch.empty(w.kv_shape, dtype=torch.float16, device=device)
    v = torch.empty(w.kv_shape, dtype=torch.float16, device=device)
    _fill_kv(k, w, STREAM_K, device)
    _fill_kv(v, w, STREAM_V, device)
    return k, v


def make_kv_paged(w: Workload, device="cpu"):
    """K and V page pools [num_blocks, page_size, n_heads, head_dim] fp16;
    element i of a pool gets value(i) of its stream."""
    assert w.paged
    k = torch.empty(w.pool_shape, dtype=torch.float16, device=device)
    v = torch.empty(w.pool_shape, dtype=torch.float16, device=device)
    fill_normal_(k, w.seed, STREAM_K, w.sigma_kv)
    fill_normal_(v, w.seed, STREAM_V, w.sigma_kv)
    return k, v


def head_slice_paged(w: Workload, b: int, h: int, block_table: Optional[torch.Tensor] = None):
    """Host copies of one (sequence, head) of a paged workload, gathered
    through the block table into the dense layout: q [1,1,D], k/v [L,1,D]."""
    H, D, P = w.n_heads, w.head_dim, w.page_size
    if block_table is None:
        block_table = w.block_table()
    L = w.valid_len(b)
    d = torch.arange(D, dtype=torch.int64)
    q = normal_f16(w.seed, STREAM_Q, (b * H + h) * D + d, w.sigma_q).view(1, 1, D)
    p = torch.arange(L, dtype=torch.int64)
    page = block_table[b, p // P]
    idx = (((page * P + p % P) * H + h) * D)[:, None] + d[None, :]
    k = normal_f16(w.seed, STREAM_K, idx, w.sigma_kv).view(L, 1, D)
    v = normal_f16(w.seed, STREAM_V, idx, w.sigma_kv).view(L, 1, D)
    return q, k, v


def head_slice(w: Workload, b: int, h: int, n_rows: Optional[int] = None):
    """Host copies of one (sequence, head): q [1,1,D], k/v [n_rows,1,D].

    Values are bit-identical to the same elements of ``make_q``/``make_kv``.
    ``n_rows`` defaults to the sequence's valid length (rows 0..current_pos).
    """
    H, D, S = w.n_heads, w.head_dim, w.seq_len
    if n_rows is None:
        n_rows = w.valid_len(b)
    d = torch.arange(D, dtype=torch.int64)
    q = normal_f16(w.seed, STREAM_Q, (b * H + h) * D + d, w.sigma_q).view(1, 1, D)
    p = torch.arange(n_rows, dtype=torch.int64)
    idx = ((b * S + p[:, None]) * H + h) * D + d[None, :]
    out = []
    for stream in (STREAM_K, STREAM_V):
        t = normal_f16(w.seed, stream, idx, w.sigma_kv)
        if w.garbage_sigma is not None and not w.batched:
            lo = min(w.cur_pos, S - 1) + 1
            if lo < n_rows:
                t[lo:] = normal_f16(w.seed, stream, idx[lo:], w.garbage_sigma)
        if stream == STREAM_K and w.spike_fraction > 0:
            rows = w.spike_rows()
            rows = rows[rows < n_rows]
            t[rows] = t[rows] * w.spike_scale
        out.append(t.view(n_rows, 1, D))
    return q, out[0], out[1]


def make_normal(w: Workload, device, chunk_rows: int = 2048):
    """True normal inputs of the workload's shape and structure: q
    [B, H, D] ~ N(0, sigma_q^2); k, v [B, S, H, D] ~ N(0, sigma_kv^2), rows
    after current_pos ~ N(0, garbage_sigma^2) where the workload has
    garbage, the K rows of ``spike_rows()`` times ``spike_scale``; all fp16
    (nearest even).  Drawn with torch.randn from a generator seeded by the
    workload, on ``device``, so the values depend on the device type: a
    check against the oracle takes host copies of these tensors.  (The
    counter-based generator above is bounded at +-3.46 sigma; these draws
    have the normal tails.)"""
    assert not w.paged
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * w.seed + 17)
    q = (torch.randn(w.q_shape, generator=g, device=device) * w.sigma_q).half()
    B, S, H, D = w.kv_shape
    k = torch.empty(w.kv_shape, dtype=torch.float16, device=device)
    v = torch.empty(w.kv_shape, dtype=torch.float16, device=device)
    lo_garbage = S
    if w.garbage_sigma is not None and not w.batched:
        lo_garbage = min(w.cur_pos, S - 1) + 1
    for t in (k, v):
        for b in range(B):
            for r0 in range(0, S, chunk_rows):
                r1 = min(S, r0 + chunk_rows)
                x = torch.randn((r1 - r0, H, D), generator=g, device=device)
                sig = torch.full((r1 - r0, 1, 1), w.sigma_kv, device=device)
                if r1 > lo_garbage:
                    sig[max(0, lo_garbage - r0):] = w.garbage_sigma
                t[b, r0:r1] = (x * sig).half()
    if w.spike_fraction > 0:
        rows = w.spike_rows().to(device)
        k[:, rows] = k[:, rows] * w.spike_scale
    return q, k, v


# The five decode-attention workloads, named by shape.
WORKLOADS = {
    wl.name: wl for wl in [
        Workload("h4_d64_s128_cp100", n_heads=4, head_dim=64, seq_len=128,
                 cur_pos=100, seed=1),
        Workload("h32_d128_s4096_full", n_heads=32, head_dim=128, seq_len=4096,
                 cur_pos=4095, seed=2),
        Workload("h32_d128_s32768_cp20000_garbage", n_heads=32, head_dim=128,
                 seq_len=32768, cur_pos=20000, seed=3, sigma_q=2.0,
                 garbage_sigma=10.0),
        Workload("b64_h32_d128_cap8192_ragged", n_heads=32, head_dim=128,
                 seq_len=8192, cur_pos=None, seed=4, batch=64),
        Workload("h64_d64_s131072_spikes", n_heads=64, head_dim=64,
                 seq_len=131072, cur_pos=131071, seed=5, spike_fraction=0.01),
        # the ragged batch again, its caches cut into 16-position pages
        # scattered through one pool
        Workload("b64_h32_d128_cap8192_ragged_paged16", n_heads=32, head_dim=128,
                 seq_len=8192, cur_pos=None, seed=4, batch=64, page_size=16),
        # a batch of short capacity: one launch, one chunk per sequence and
        # head block
        Workload("b256_h32_d128_cap64_ragged", n_heads=32, head_dim=128,
                 seq_len=64, cur_pos=None, seed=6, batch=256),
    ]
}

# Workload timed by the bench: the largest single-sequence cache at
# seq_len >= 32768 (2 GiB of K+V, far beyond the 256 MB last-level cache).
BENCH_WORKLOAD = "h64_d64_s131072_spikes"


def page_pattern_f16(n: int) -> torch.Tensor:
    """The Testing section's deterministic fill: element i holds (i % 10) * 0.1
    rounded to fp16 (the page converts an f32 value with f16::from_f32)."""
    i = torch.arange(n, dtype=torch.int64)
    return ((i % 10).to(torch.float32) * 0.1).to(torch.float16)


# ------------------------------------------------------------ row softmax
# The softmax step on its own (the Foundry notes' fm_softmax over a
# [rows, cols] fp32 tensor) on the score matrices of the decode workloads:
# row r is (sequence r // n_heads, head r % n_heads), column p a cache
# position.  Values are seeded stand-ins for scaled scores: approximately
# N(0, sigma^2), the decode workload's spike positions scaled the same way,
# and -inf after each row's last valid position (the masked score of the
# page's attention_qk_f16).

STREAM_SCORES = 4


@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    of: str          # the decode workload whose shape, lengths and spikes it takes
    seed: int
    sigma: float

    @property
    def decode(self) -> Workload:
        return WORKLOADS[self.of]

    @property
    def rows(self) -> int:
        return self.decode.batch * self.decode.n_heads

    @property
    def cols(self) -> int:
        return self.decode.seq_len

    def row_lengths(self) -> torch.Tensor:
        """Valid (not -inf) columns of each row, int64 [rows] (host)."""
        d = self.decode
        lens = torch.clamp(d.positions(), max=d.seq_len - 1) + 1
        return lens.repeat_interleave(d.n_heads)

    def bytes_moved(self) -> int:
        """Algorithmic bytes of one softmax: x read once, out written once."""
        return self.rows * self.cols * 4 * 2


def score_rows(w: SoftmaxWorkload, rows, device="cpu") -> torch.Tensor:
    """fp32 [len(rows), cols]: the given rows of the workload's input."""
    rows = torch.as_tensor(rows, dtype=torch.int64)
    cols = w.cols
    idx = rows.to(device)[:, None] * cols + torch.arange(cols, dtype=torch.int64, device=device)[None, :]
    x = normal_f32(w.seed, STREAM_SCORES, idx, w.sigma)
    d = w.decode
    if d.spike_fraction > 0:
        sp = d.spike_rows().to(device)
        x[:, sp] = x[:, sp] * d.spike_scale
    lens = w.row_lengths()[rows].to(device)
    x[torch.arange(cols, device=device)[None, :] >= lens[:, None]] = -math.inf
    return x


def make_scores(w: SoftmaxWorkload, device="cpu", chunk_rows: int = 256) -> torch.Tensor:
    """The whole input [rows, cols] fp32."""
    x = torch.empty((w.rows, w.cols), dtype=torch.float32, device=device)
    for lo in range(0, w.rows, chunk_rows):
        hi = min(w.rows, lo + chunk_rows)
        x[lo:hi] = score_rows(w, torch.arange(lo, hi), device)
    return x


SOFTMAX_WORKLOADS = {
    sw.name: sw for sw in [
        # the seq-32768 scores: q of sigma 2 gives scaled scores of sigma ~2
        SoftmaxWorkload("sm_h32_s32768_masked", of="h32_d128_s32768_cp20000_garbage",
                        seed=13, sigma=2.0),
        SoftmaxWorkload("sm_b64_h32_cap8192_ragged", of="b64_h32_d128_cap8192_ragged",
                        seed=14, sigma=1.0),
        SoftmaxWorkload("sm_h64_s131072_spikes", of="h64_d64_s131072_spikes", seed=15,
                        sigma=1.0),
    ]
}
