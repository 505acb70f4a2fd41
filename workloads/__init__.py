"""Seeded synthetic inputs for the multi-LoRA shrink / expand path.

This module only draws random inputs and encodes them as 16-bit patterns.  It
holds none of the method's arithmetic: no shrink, expand or segment logic.  The
oracle (``oracle/``) and the HIP path (``lora_serving_build_amd``) both consume
exactly the bits produced here, and neither is imported by it.

Recipe (the pages fix shapes and value ranges only loosely; these readings are
listed with the design notes):
  * numpy ``Generator(PCG64(seed))``; named workloads use seed 1000 + k.
  * Values are drawn as float32 and rounded once, round-to-nearest-even, to
    IEEE binary16 (numpy's conversion) or bfloat16 (rounding the binary32 bit
    pattern).
  * x ~ N(0, 1); weights N(0, 1/fan_in): A ~ N(0, 1/H), B ~ N(0, 1/r_i) on the
    adapter's live rank and exact zeros on its padding; y0 ~ N(0, 1), except
    the 16-token decode case where y0 = x . W0 with W0 ~ N(0, 1/H) evaluated in
    fp64 on the rounded x and W0 and rounded once.
  * Sequence lengths uniform in {1..m} drawn until the total reaches T, the
    last one cut to hit T exactly; an adapter id per sequence (uniform or Zipf
    with P(k) proportional to (k+1)^-s); a fraction of whole sequences take
    id -1 (Bernoulli per sequence).
  * Weight layouts: A is [L][r][H] (each adapter's H x r matrix stored
    transposed, H contiguous) and B is [L][n][r] (each adapter's r x n matrix
    stored transposed, r contiguous), i.e. the contraction index is contiguous.
Draw order inside a workload: sequence structure (lengths, ids, -1 flags,
ranks), then x, then A, then every slice's B in order, then every output's y0,
then W0 where used.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

_CHUNK = 1 << 24


# ---------------------------------------------------------------- encodings
def f32_to_bits(a, dtype: str) -> np.ndarray:
    """Round float32 values once (RNE) to binary16 / bfloat16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        # uint32 arithmetic cannot wrap here except for NaN patterns, which
        # are replaced by the canonical quiet NaN below.
        u = a.view(np.uint32)
        out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(a)
        if nan.any():
            out[nan] = 0x7FC0
        return out
    raise ValueError(dtype)


def bits_to_f32(bits, dtype: str) -> np.ndarray:
    """float32 value of binary16 / bfloat16 bit patterns (both widen exactly)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def normal_bits(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    """N(0, std^2) draws, encoded, filled in chunks to bound host memory."""
    out = np.empty(int(np.prod(shape)), np.uint16)
    for s in range(0, out.size, _CHUNK):
        e = min(out.size, s + _CHUNK)
        out[s:e] = f32_to_bits(rng.standard_normal(e - s, dtype=np.float32) * np.float32(std), dtype)
    return out.reshape(shape)


def int_bits(rng: np.random.Generator, shape, lo: int, hi: int, dtype: str) -> np.ndarray:
    """Integer values uniform in [lo, hi], encoded exactly."""
    return f32_to_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32), dtype)


# ---------------------------------------------------------------- containers
@dataclass
class Slice:
    n: int                 # slice width
    col_off: int           # first column of the slice in its output
    B: np.ndarray          # uint16 [L][n][r]


@dataclass
class Output:
    name: str
    y0: np.ndarray         # uint16 [T][ldy], the output before the call
    slices: list[Slice]

    @property
    def ldy(self) -> int:
        return int(self.y0.shape[1])


@dataclass
class Workload:
    name: str
    dtype: str             # "f16" | "bf16"
    T: int
    H: int
    r: int                 # rank as passed (after any padding)
    L: int
    ids: np.ndarray        # int32 [T]; -1 = no adapter
    x: np.ndarray          # uint16 [T][H]
    A: np.ndarray          # uint16 [L][r][H]
    outputs: list[Output]
    add: bool = True
    ranks: np.ndarray | None = None      # live rank per adapter (<= r)
    seq_lens: list[int] = field(default_factory=list)
    seed: int = 0

    @property
    def active(self) -> np.ndarray:
        return (self.ids >= 0) & (self.ids < self.L)

    @property
    def T_a(self) -> int:
        return int(self.active.sum())

    @property
    def distinct(self) -> int:
        return int(np.unique(self.ids[self.active]).size)

    # Algorithmic bytes and flops of one pass (unique weights, -1 rows excluded).
    def shrink_bytes(self) -> int:
        e = 2
        return self.T_a * self.H * e + self.distinct * self.r * self.H * e + self.T_a * self.r * 4

    def output_bytes(self, o: "Output") -> int:
        """Algorithmic bytes of the one expand / expand_slice call that writes
        output o: v read, the present adapters' weights, y read (add) and
        written."""
        e = 2
        n = sum(s.n for s in o.slices)
        return self.T_a * self.r * 4 + self.distinct * self.r * n * e + (2 if self.add else 1) * self.T_a * n * e

    def expand_bytes(self) -> int:
        return sum(self.output_bytes(o) for o in self.outputs)

    def shrink_flops(self) -> int:
        return 2 * self.T_a * self.H * self.r

    def expand_flops(self) -> int:
        return sum(2 * self.T_a * self.r * sum(s.n for s in o.slices) for o in self.outputs)

    def host_bytes(self) -> int:
        b = self.x.nbytes + self.A.nbytes + self.ids.nbytes
        for o in self.outputs:
            b += o.y0.nbytes + sum(s.B.nbytes for s in o.slices)
        return b


# ---------------------------------------------------------------- structure
def seq_lengths(rng, T: int, max_len: int) -> list[int]:
    lens, tot = [], 0
    while tot < T:
        n = int(rng.integers(1, max_len + 1))
        lens.append(n)
        tot += n
    lens[-1] -= tot - T
    return lens


def zipf_probs(L: int, s: float) -> np.ndarray:
    w = (np.arange(L, dtype=np.float64) + 1.0) ** (-s)
    return w / w.sum()


def make(name: str, dtype: str, T: int, H: int, r: int, L: int,
         slices_per_output: list[list[int]], *, seed: int,
         seq_len: int | tuple[int, int] = 1, id_dist: str = "uniform",
         zipf_s: float = 1.1, neg_frac: float = 0.0, sort_by_id: bool = False,
         ranks_from: list[int] | None = None, add: bool = True,
         y0_mode: str = "normal", integer: bool = False) -> Workload:
    """Build one workload.

    seq_len: an int = fixed length per sequence; (1, m) = uniform in {1..m}.
    slices_per_output: e.g. [[4096, 1024, 1024], [14336, 14336]] = two outputs,
    the first with three slices side by side.
    ranks_from: draw each adapter's live rank from this list (padded to r).
    integer: small integer-valued inputs, for exact comparisons."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if isinstance(seq_len, int):
        nseq = -(-T // seq_len)
        lens = [seq_len] * nseq
        lens[-1] -= nseq * seq_len - T
    else:
        lens = seq_lengths(rng, T, seq_len[1])
    nseq = len(lens)
    if id_dist == "uniform":
        seq_ids = rng.integers(0, L, size=nseq).astype(np.int32)
    elif id_dist == "zipf":
        seq_ids = rng.choice(L, size=nseq, p=zipf_probs(L, zipf_s)).astype(np.int32)
    else:
        raise ValueError(id_dist)
    if neg_frac > 0:
        neg = rng.random(nseq) < neg_frac
        seq_ids[neg] = -1
    if sort_by_id:
        order = np.argsort(seq_ids, kind="stable")
        seq_ids = seq_ids[order]
        lens = [lens[i] for i in order]
    ids = np.repeat(seq_ids, lens).astype(np.int32)
    assert ids.shape[0] == T
    if ranks_from is not None:
        ranks = rng.choice(np.array(ranks_from), size=L).astype(np.int32)
        assert ranks.max() <= r
    else:
        ranks = np.full(L, r, np.int32)

    if integer:
        x = int_bits(rng, (T, H), -2, 2, dtype)
        A = int_bits(rng, (L, r, H), -2, 2, dtype)
    else:
        x = normal_bits(rng, (T, H), 1.0, dtype)
        A = normal_bits(rng, (L, r, H), 1.0 / np.sqrt(H), dtype)
    for l in range(L):
        A[l, ranks[l]:, :] = 0
    outputs = []
    b_list = []
    for oi, widths in enumerate(slices_per_output):
        sl, off = [], 0
        for n in widths:
            if integer:
                B = int_bits(rng, (L, n, r), -2, 2, dtype)
            else:
                B = np.empty((L, n, r), np.uint16)
                for l in range(L):
                    B[l] = normal_bits(rng, (n, r), 1.0 / np.sqrt(ranks[l]), dtype)
            for l in range(L):
                B[l, :, ranks[l]:] = 0
            sl.append(Slice(n=n, col_off=off, B=B))
            off += n
        b_list.append(sl)
    for oi, sl in enumerate(b_list):
        ldy = sum(s.n for s in sl)
        if integer:
            y0 = int_bits(rng, (T, ldy), -4, 4, dtype)
        elif y0_mode == "normal":
            y0 = normal_bits(rng, (T, ldy), 1.0, dtype)
        elif y0_mode == "base":
            W0 = normal_bits(rng, (H, ldy), 1.0 / np.sqrt(H), dtype)
            base = bits_to_f32(x, dtype).astype(np.float64) @ bits_to_f32(W0, dtype).astype(np.float64)
            y0 = f32_to_bits(base.astype(np.float32), dtype) if dtype == "bf16" else \
                base.astype(np.float16).view(np.uint16)
        else:
            raise ValueError(y0_mode)
        outputs.append(Output(name=f"y{oi}", y0=y0, slices=sl))
    return Workload(name=name, dtype=dtype, T=T, H=H, r=r, L=L, ids=ids, x=x, A=A,
                    outputs=outputs, add=add, ranks=ranks, seq_lens=lens, seed=seed)


# ---------------------------------------------------------------- named cases
CONFIG_NAMES = {
    1: "bgmv_decode_f16_T16_H1024_r16_L4",
    2: "llama3_8b_decode_bgmv_f16_T256_H4096_r16_L4",
    3: "sgmv_prefill_bf16_T2048_seq8_H4096_r16_L4_sorted",
    4: "sgmv_expand_slice_bf16_T1024_mixed_rank128_L16_qkv_gateup",
    5: "llama3_70b_layer_bf16_T8192_H8192_r64_L64_zipf",
}


def config(k: int) -> Workload:
    """The five named workloads (seed 1000 + k)."""
    seed = 1000 + k
    name = CONFIG_NAMES[k]
    if k == 1:
        return make(name, "f16", 16, 1024, 16, 4, [[1024]], seed=seed, y0_mode="base")
    if k == 2:
        return make(name, "f16", 256, 4096, 16, 4, [[4096]], seed=seed)
    if k == 3:
        return make(name, "bf16", 2048, 4096, 16, 4, [[4096]], seed=seed, seq_len=8,
                    sort_by_id=True)
    if k == 4:
        return make(name, "bf16", 1024, 4096, 128, 16, [[4096, 1024, 1024], [14336, 14336]],
                    seed=seed, seq_len=(1, 64), neg_frac=0.10,
                    ranks_from=[8, 16, 32, 64, 128])
    if k == 5:
        return make(name, "bf16", 8192, 8192, 64, 64, [[8192, 1024, 1024], [28672, 28672]],
                    seed=seed, seq_len=(1, 512), id_dist="zipf", zipf_s=1.1, neg_frac=0.05)
    raise KeyError(k)


def sweep_point(kind: str, T: int, H: int, r: int, L: int = 4, seed: int = 7,
                dtype: str = "f16") -> Workload:
    """Micro-benchmark sweep shape (4 adapters, sorted by id; BGMV one token per
    sequence, SGMV eight): shrink H -> r, expand r -> H."""
    sl = 1 if kind == "bgmv" else 8
    return make(f"{kind}_T{T}_H{H}_r{r}_L{L}", dtype, T, H, r, L, [[H]], seed=seed,
                seq_len=sl, sort_by_id=True)


def make_mixed(name: str, dtype: str, n_prefill: int, prefill_loras: int, n_decode: int, L: int,
               H: int, r: int, slices_per_output: list[list[int]], *, seed: int, max_len: int = 64,
               neg_frac: float = 0.0, integer: bool = False) -> Workload:
    """A batch that mixes prefill and decode: prefill sequences of U{1..max_len}
    tokens (n_prefill in all) on adapters drawn uniformly from the first
    prefill_loras, and n_decode one-token requests whose adapters are drawn
    without replacement from the other L - prefill_loras (each is a segment of
    one token).  Sequences in shuffled order; a fraction of whole sequences
    take id -1.  x, weights and y0 are those of make() with the same seed."""
    if n_decode > L - prefill_loras:
        raise ValueError("each decode token needs an adapter of its own")
    T = n_prefill + n_decode
    w = make(name, dtype, T, H, r, L, slices_per_output, seed=seed, integer=integer)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    lens = seq_lengths(rng, n_prefill, max_len) if n_prefill else []
    seq_ids = rng.integers(0, prefill_loras, size=len(lens)) if lens else np.zeros(0, np.int64)
    dec_ids = prefill_loras + rng.permutation(L - prefill_loras)[:n_decode]
    seqs = [(int(n), int(i)) for n, i in zip(lens, seq_ids)] + [(1, int(d)) for d in dec_ids]
    order = rng.permutation(len(seqs))
    neg = rng.random(len(seqs)) < neg_frac
    ids = np.concatenate([np.full(seqs[k][0], -1 if neg[k] else seqs[k][1], np.int32) for k in order])
    assert ids.shape[0] == T
    w.ids = ids.astype(np.int32)
    w.seq_lens = [seqs[k][0] for k in order]
    return w
