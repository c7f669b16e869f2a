"""Seeded synthetic inputs for the indexer -> Top-K -> sparse MLA attention path.

This module only draws random numbers and lays them out in the paged-cache
format; it holds none of the method's arithmetic. Both the CPU oracle (through
the tests) and the HIP library read what it produces.

Layout produced (all row-major, contiguous):
  seq_lens   int32 [B]                      context length n_b of each sequence
  page_table int32 [B, max_pages]           physical page of logical page p (-1 = none)
  idx_k      [num_pages, 64, d_I]           index-K rows: bfloat16, or uint8 holding
                                            OCP float8 e4m3fn codes
  idx_scale  float32 [num_pages, 64]        per-token scale (fp8 index cache only)
  kv         bfloat16 [num_pages, 64, 576]  latent KV rows (512 latent + 64 rope)
  q_idx      bfloat16 [Q, H_I, d_I]         indexer query heads
  w          float32 [Q, H_I]               per-token head weights
  q_attn     bfloat16 [Q, H_A, 576]         attention queries in the latent space
  q_seq      int32 [Q]                      sequence of each query token
  q_pos      int32 [Q]                      absolute position t_j (sees 0..t_j)

Both caches share one page table. Physical pages are a seeded shuffle. With
``poison=True`` every row no sequence owns (tails of last pages and a few
spare pages) is filled with NaN so that any read past n_b shows up.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

PAGE = 64
DIM_KV = 576
D_V = 512


@dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    ctx_lo: int
    ctx_hi: int
    q_per_seq: int          # decode: trailing query tokens per sequence; 0 = prefill
    heads_idx: int
    dim_idx: int
    idx_fp8: bool
    w_std: float
    topk: int
    heads_attn: int
    sm_scale: float
    chunk: int = 0          # chunked prefill: queries per chunk (0 = single shot)
    seed: int = 20260000

    @property
    def prefill(self) -> bool:
        return self.q_per_seq == 0


# The five workloads: tiny decode, batch-32 decode, 128K speculative decode,
# 16K causal prefill, 128K chunked prefill (8192-query chunks).
SPECS = {
    "tiny_decode": Spec("tiny_decode", 1, 4096, 4096, 1, 4, 64, False, 0.5, 256, 16,
                        1.0 / 24.0, seed=20260000),
    "decode_b32": Spec("decode_b32", 32, 8192, 32768, 1, 64, 128, True, 1.0 / 8.0, 2048,
                       128, 1.0 / 24.0, seed=20260001),
    "spec_decode_128k": Spec("spec_decode_128k", 64, 131072, 131072, 2, 64, 128, True,
                             1.0 / 8.0, 2048, 128, 1.0 / 24.0, seed=20260002),
    "prefill_16k": Spec("prefill_16k", 1, 16384, 16384, 0, 64, 128, False, 1.0 / 8.0, 2048,
                        128, 1.0 / 24.0, seed=20260003),
    "chunked_prefill_128k": Spec("chunked_prefill_128k", 1, 131072, 131072, 0, 64, 128, True,
                                 1.0 / 8.0, 2048, 128, 1.0 / 24.0, chunk=8192, seed=20260004),
}


def spec(name: str, **overrides) -> Spec:
    """A named workload, optionally shrunk (e.g. ``batch=2, ctx_lo=3000``)."""
    s = SPECS[name]
    return replace(s, **overrides) if overrides else s


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn_chunked(shape, std, gen, device, out_dtype, chunk_elems=1 << 27):
    """N(0, std^2) drawn in fp32 and rounded (RNE) to ``out_dtype``."""
    numel = math.prod(shape)
    out = torch.empty(numel, dtype=out_dtype, device=device)
    for s in range(0, numel, chunk_elems):
        e = min(numel, s + chunk_elems)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[s:e] = x.to(out_dtype)
    return out.view(shape)


def _e4m3fn_codes(shape, gen, device, chunk_elems=1 << 26):
    """N(0,1) in fp32 cast (RNE) to OCP float8 e4m3fn; returned as uint8 codes.

    The cast runs on the device when torch supports it there, else on the host."""
    numel = math.prod(shape)
    out = torch.empty(numel, dtype=torch.uint8, device=device)
    for s in range(0, numel, chunk_elems):
        e = min(numel, s + chunk_elems)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        try:
            c = x.to(torch.float8_e4m3fn).view(torch.uint8)
        except (RuntimeError, TypeError):
            c = x.cpu().to(torch.float8_e4m3fn).view(torch.uint8).to(device)
        out[s:e] = c
    return out.view(shape)


@dataclass
class Workload:
    spec: Spec
    seq_lens: torch.Tensor
    page_table: torch.Tensor
    idx_k: torch.Tensor
    idx_scale: Optional[torch.Tensor]
    kv: torch.Tensor
    q_idx: torch.Tensor
    w: torch.Tensor
    q_attn: torch.Tensor
    q_seq: torch.Tensor
    q_pos: torch.Tensor
    num_pages: int

    @property
    def num_q(self) -> int:
        return int(self.q_seq.numel())

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def queries(self, start: int, stop: int) -> "Workload":
        """The same caches with only queries [start, stop)."""
        return replace(self, q_idx=self.q_idx[start:stop], w=self.w[start:stop],
                       q_attn=self.q_attn[start:stop], q_seq=self.q_seq[start:stop],
                       q_pos=self.q_pos[start:stop])

    def to(self, device) -> "Workload":
        def mv(t):
            return None if t is None else t.to(device)
        return replace(self, seq_lens=mv(self.seq_lens), page_table=mv(self.page_table),
                       idx_k=mv(self.idx_k), idx_scale=mv(self.idx_scale), kv=mv(self.kv),
                       q_idx=mv(self.q_idx), w=mv(self.w), q_attn=mv(self.q_attn),
                       q_seq=mv(self.q_seq), q_pos=mv(self.q_pos))


def make(s: Spec, device="cpu", poison: bool = False, shuffle: bool = True,
         spare_pages: int = 2, with_attn: bool = True) -> Workload:
    """Draw the workload ``s`` with its seed. Host-side structure (lengths, page
    permutation) always comes from numpy so that it is identical on any device;
    bulk tensors come from a torch generator on ``device``."""
    ss = np.random.SeedSequence(s.seed)
    rng_len, rng_perm = [np.random.default_rng(c) for c in ss.spawn(2)]
    B = s.batch
    if s.ctx_lo == s.ctx_hi:
        lens = np.full(B, s.ctx_lo, dtype=np.int64)
    else:
        lens = rng_len.integers(s.ctx_lo, s.ctx_hi + 1, size=B)
    pages_per_seq = (lens + PAGE - 1) // PAGE
    max_pages = int(pages_per_seq.max())
    used = int(pages_per_seq.sum())
    num_pages = used + spare_pages
    phys = rng_perm.permutation(num_pages) if shuffle else np.arange(num_pages)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        table[b, :n] = phys[off:off + n]
        off += n

    # query tokens
    if s.prefill:
        assert B == 1
        q_seq = np.zeros(int(lens[0]), dtype=np.int32)
        q_pos = np.arange(int(lens[0]), dtype=np.int32)
    else:
        q_seq = np.repeat(np.arange(B, dtype=np.int32), s.q_per_seq)
        q_pos = np.concatenate([np.arange(int(n) - s.q_per_seq, int(n)) for n in lens]).astype(np.int32)
    Q = len(q_seq)

    seeds = [int(x.generate_state(1)[0]) for x in ss.spawn(8)[2:8]]
    dev = torch.device(device)
    rows = num_pages * PAGE
    if s.idx_fp8:
        idx_k = _e4m3fn_codes((num_pages, PAGE, s.dim_idx), _gen(dev, seeds[0]), dev)
        g = _gen(dev, seeds[1])
        idx_scale = (torch.rand(rows, generator=g, device=dev, dtype=torch.float32) * 1.5 + 0.5)
        idx_scale = idx_scale.view(num_pages, PAGE)
    else:
        idx_k = _randn_chunked((num_pages, PAGE, s.dim_idx), 1.0, _gen(dev, seeds[0]), dev,
                               torch.bfloat16)
        idx_scale = None
    q_idx = _randn_chunked((Q, s.heads_idx, s.dim_idx), 1.0, _gen(dev, seeds[2]), dev,
                           torch.bfloat16)
    w = torch.randn((Q, s.heads_idx), generator=_gen(dev, seeds[3]), device=dev,
                    dtype=torch.float32) * s.w_std
    if with_attn:
        kv = _randn_chunked((num_pages, PAGE, DIM_KV), 1.0, _gen(dev, seeds[4]), dev,
                            torch.bfloat16)
        q_attn = _randn_chunked((Q, s.heads_attn, DIM_KV), 1.0, _gen(dev, seeds[5]), dev,
                                torch.bfloat16)
    else:
        kv = torch.empty((num_pages, PAGE, DIM_KV), dtype=torch.bfloat16, device=dev)
        q_attn = torch.empty((Q, s.heads_attn, DIM_KV), dtype=torch.bfloat16, device=dev)

    wl = Workload(s, torch.from_numpy(lens.astype(np.int32)).to(dev),
                  torch.from_numpy(table).to(dev), idx_k, idx_scale, kv, q_idx, w, q_attn,
                  torch.from_numpy(q_seq).to(dev), torch.from_numpy(q_pos).to(dev), num_pages)
    if poison:
        poison_unowned(wl)
    return wl


@dataclass
class MxInputs:
    """Synthetic MXFP8 index-path inputs for a workload with an fp8 index
    cache: its e4m3 codes serve as the MXFP8 rows; the E8M0 block scales and
    an MXFP8 query are drawn here (no quantizer involved)."""
    k_scales: torch.Tensor   # uint8 [num_pages, 64, d_I / 32]
    q_codes: torch.Tensor    # uint8 [Q, H_I, d_I] (e4m3 codes of N(0,1) draws)
    q_scales: torch.Tensor   # uint8 [Q, H_I, d_I / 32]

    def queries(self, start: int, stop: int) -> "MxInputs":
        return replace(self, q_codes=self.q_codes[start:stop], q_scales=self.q_scales[start:stop])

    def to(self, device) -> "MxInputs":
        return MxInputs(self.k_scales.to(device), self.q_codes.to(device), self.q_scales.to(device))


def make_mx(wl: Workload, scale_lo: int = 124, scale_hi: int = 130, poison: bool = False) -> MxInputs:
    """MXFP8 inputs for ``wl`` (whose index cache holds e4m3 codes): block
    scale bytes uniform in [scale_lo, scale_hi] (2^-3 .. 2^3), query codes from
    N(0,1) cast to e4m3 and their scale bytes likewise. Seeded from the
    workload's seed. With ``poison``, rows no sequence owns get the E8M0 NaN
    byte 0xFF."""
    s = wl.spec
    assert s.idx_fp8 and s.dim_idx % 32 == 0
    seeds = [int(x.generate_state(1)[0]) for x in np.random.SeedSequence([s.seed, 0x4D58]).spawn(3)]
    dev = wl.idx_k.device
    nb = s.dim_idx // 32
    k_scales = torch.randint(scale_lo, scale_hi + 1, (wl.num_pages, PAGE, nb), generator=_gen(dev, seeds[0]),
                             device=dev, dtype=torch.int32).to(torch.uint8)
    Q = wl.num_q
    q_codes = _e4m3fn_codes((Q, s.heads_idx, s.dim_idx), _gen(dev, seeds[1]), dev)
    q_scales = torch.randint(scale_lo, scale_hi + 1, (Q, s.heads_idx, nb), generator=_gen(dev, seeds[2]),
                             device=dev, dtype=torch.int32).to(torch.uint8)
    if poison:
        bad = (~owned_rows_mask(wl)).to(dev)
        k_scales[bad] = 0xFF
    return MxInputs(k_scales, q_codes, q_scales)


KV8_ROW = 656   # fp8 latent row: 512 e4m3 codes, 4 fp32 block scales, 64 bf16 rope values


def make_kv8(wl: Workload, poison: bool = False) -> torch.Tensor:
    """A synthetic FP8 latent cache [num_pages, 64, 656] (uint8) for ``wl``:
    per row and block of 128 latent elements a scale ~ U(0.5, 2) / 64, codes of
    N(0,1) * 64 cast to e4m3fn (so the values are about N(0,1) times the
    block's U(0.5, 2)), rope values N(0,1) in bf16. Seeded from the workload's
    seed. With ``poison``, rows no sequence owns get NaN codes and scales."""
    s = wl.spec
    seeds = [int(x.generate_state(1)[0]) for x in np.random.SeedSequence([s.seed, 0x4B56]).spawn(3)]
    dev = wl.kv.device
    rows = wl.num_pages * PAGE
    codes = _randn_chunked((rows, D_V), 64.0, _gen(dev, seeds[0]), dev, torch.float8_e4m3fn).view(torch.uint8)
    scales = (torch.rand((rows, 4), generator=_gen(dev, seeds[1]), device=dev, dtype=torch.float32) * 1.5
              + 0.5) / 64.0
    rope = _randn_chunked((rows, DIM_KV - D_V), 1.0, _gen(dev, seeds[2]), dev, torch.bfloat16)
    out = torch.empty((rows, KV8_ROW), dtype=torch.uint8, device=dev)
    out[:, :512] = codes
    out[:, 512:528] = scales.view(torch.uint8).view(rows, 16)
    out[:, 528:] = rope.view(torch.uint8).view(rows, 128)
    out = out.view(wl.num_pages, PAGE, KV8_ROW)
    if poison:
        bad = (~owned_rows_mask(wl)).to(dev)
        out[bad, :512] = 0x7F
        out[bad, 512:528] = torch.tensor([float("nan")] * 4, device=dev).view(torch.uint8)
    return out


def owned_rows_mask(wl: Workload) -> torch.Tensor:
    """bool [num_pages, 64]: True where some sequence owns the row."""
    table = wl.page_table.cpu().numpy()
    lens = wl.seq_lens.cpu().numpy()
    own = np.zeros((wl.num_pages, PAGE), dtype=bool)
    for b in range(table.shape[0]):
        n = int(lens[b])
        for p in range((n + PAGE - 1) // PAGE):
            own[table[b, p], :min(PAGE, n - p * PAGE)] = True
    return torch.from_numpy(own)


def poison_unowned(wl: Workload) -> None:
    """Fill every row no sequence owns with NaN (bf16 0x7FC0, e4m3fn 0x7F)."""
    bad = (~owned_rows_mask(wl)).to(wl.kv.device)
    wl.kv[bad] = float("nan")
    if wl.spec.idx_fp8:
        wl.idx_k[bad] = 0x7F
        wl.idx_scale[bad] = float("nan")
    else:
        wl.idx_k[bad] = float("nan")


def with_seq_lens(wl: Workload, lens) -> Workload:
    """Same caches, different context lengths (chunked prefill grows n_b)."""
    t = torch.as_tensor(lens, dtype=torch.int32).to(wl.seq_lens.device)
    return replace(wl, seq_lens=t)


def chunk_queries(wl: Workload, c: int) -> Workload:
    """Chunk ``c`` of a chunked prefill: queries [c*chunk, (c+1)*chunk) against a
    cache holding positions < (c+1)*chunk (the chunk's own rows are written before
    its indexer runs)."""
    ch = wl.spec.chunk
    sub = wl.queries(c * ch, (c + 1) * ch)
    return with_seq_lens(sub, [(c + 1) * ch])


def subset(wl: Workload, seqs, device="cpu") -> Workload:
    """The queries of sequences ``seqs`` with compact caches holding only those
    sequences' pages. The pages are renumbered contiguously in logical order, so
    the subset's page table is the identity placement (page placement itself is
    covered by its own tests). Used to hand a slice of a large workload to the
    CPU."""
    seqs = [int(s) for s in seqs]
    table = wl.page_table.cpu()
    lens = wl.seq_lens.cpu()
    q_seq = wl.q_seq.cpu()
    keep_q = torch.zeros(q_seq.numel(), dtype=torch.bool)
    for s in seqs:
        keep_q |= q_seq == s
    qi = torch.nonzero(keep_q).flatten()
    npg = [int((int(lens[s]) + PAGE - 1) // PAGE) for s in seqs]
    phys = torch.cat([table[s, :n] for s, n in zip(seqs, npg)]).long()
    new_table = torch.full((len(seqs), max(npg)), -1, dtype=torch.int32)
    off = 0
    for i, n in enumerate(npg):
        new_table[i, :n] = torch.arange(off, off + n, dtype=torch.int32)
        off += n
    src = phys.to(wl.idx_k.device)
    remap = {s: i for i, s in enumerate(seqs)}
    new_qseq = torch.tensor([remap[int(s)] for s in q_seq[qi]], dtype=torch.int32)
    return Workload(
        wl.spec, lens[seqs].clone().to(device), new_table.to(device),
        wl.idx_k[src].to(device), None if wl.idx_scale is None else wl.idx_scale[src].to(device),
        wl.kv[src].to(device), wl.q_idx[qi.to(wl.q_idx.device)].to(device),
        wl.w[qi.to(wl.w.device)].to(device), wl.q_attn[qi.to(wl.q_attn.device)].to(device),
        new_qseq.to(device), wl.q_pos.cpu()[qi].to(device), len(phys))
