"""Synthetic workloads: shapes, value distributions and structure.

Shapes follow the pages: 64 indexer heads of width 128 with one shared key head
(page "DeepSeekV3.2之DSA", part 3.1-3.2), 128 attention heads over a shared
576-wide latent row (512 latent + 64 rotary, part 5.1), k = 2048 selected
positions (part 5.3).  No trained weights or real activations exist here, so
every tensor is drawn from seeded normal distributions:

* indexer q [nq, 64, 128] and keys [R, 128]: N(0, 1) fp32 (quantised later);
* head weights w [nq, 64]: N(0, 1) / 8;
* attention q [nq, 128, 576] and latent cache [R, 576]: N(0, 1) rounded to bf16;
* planted keys (decode batches 16x32K and 64x128K): in each sequence
  floor(0.01 * L) key rows are replaced by mean_over_heads(q_idx of that
  sequence's query) + 0.5 * N(0, 1), so the top-k is not a random subset.

Layouts: contiguous per-sequence caches (row0[s] = first row), or caches paged
in 64-token blocks whose physical order is a random permutation, with one block
table shared by both caches.  Big tensors are drawn chunk by chunk (65536 rows),
each chunk from its own seed, so peak temporary memory stays small.
"""

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

H_I, D_I, H, D = 64, 128, 128, 576
TOPK = 2048
SOFTMAX_SCALE = 1.0 / math.sqrt(192.0)
CHUNK = 65536

CONFIG_NAMES = {
    0: "decode 1 x 4096",
    1: "decode 16 x 32768 (planted)",
    2: "decode 64 x 131072 (planted)",
    3: "prefill 16384 (causal)",
    4: "ragged paged decode 128 x logU[1024,131072]",
}


@dataclass
class Workload:
    name: str
    nq: int
    num_seqs: int
    rows: int
    q_idx: torch.Tensor          # fp32 [nq, 64, 128]
    w: torch.Tensor              # fp32 [nq, 64]
    k_idx: torch.Tensor          # fp32 [R, 128]
    q_mla: torch.Tensor          # bf16 [nq, 128, 576]
    kv: torch.Tensor             # bf16 [R, 576]
    q_seq: torch.Tensor          # int32 [nq]
    q_nvis: torch.Tensor         # int32 [nq]
    seq_len: np.ndarray          # host int64 [num_seqs]
    block_size: int = 0
    row0: Optional[torch.Tensor] = None         # int64 [num_seqs] (contiguous)
    block_table: Optional[torch.Tensor] = None  # int32 [num_seqs, max_blocks] (paged)
    k: int = TOPK
    softmax_scale: float = SOFTMAX_SCALE
    planted: dict = field(default_factory=dict)  # seq -> host int64 positions

    @property
    def max_nvis(self) -> int:
        return int(self.q_nvis.max().item()) if self.nq else 0


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _normal(shape, device, seed, dtype=torch.float32, std=1.0):
    """N(0, std^2) drawn in row chunks, each chunk with its own seed."""
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    flat = out.view(rows, -1)
    for c0 in range(0, rows, CHUNK):
        c1 = min(rows, c0 + CHUNK)
        g = _gen(device, seed * 7919 + c0 // CHUNK)
        x = torch.randn((c1 - c0, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[c0:c1].copy_(x.to(dtype))
    return out


def make_custom(*, seq_lens, device="cpu", seed=1, prefill=False, paged=False,
                plant=False, k=TOPK, block_size=64, name="custom", queries_per_seq=None):
    """Build a workload.

    Decode (prefill=False): one query per sequence with n_vis = L.
    Prefill (prefill=True): every token t of every sequence is a query with
    n_vis = t (strictly earlier positions), or the last ``queries_per_seq``
    tokens of each sequence if given."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    num_seqs = len(seq_lens)
    rng = np.random.default_rng(seed)
    # --- cache layout -------------------------------------------------------
    if paged:
        nblk = (seq_lens + block_size - 1) // block_size
        total = int(nblk.sum())
        perm = rng.permutation(total).astype(np.int32)
        maxb = int(nblk.max()) if num_seqs else 0
        bt = np.full((num_seqs, max(maxb, 1)), -1, np.int32)
        off = 0
        for s in range(num_seqs):
            bt[s, : nblk[s]] = perm[off: off + nblk[s]]
            off += int(nblk[s])
        rows = total * block_size
        row0 = None
        block_table = torch.from_numpy(bt).to(device)
    else:
        starts = np.concatenate([[0], np.cumsum(seq_lens)[:-1]]).astype(np.int64)
        rows = int(seq_lens.sum())
        row0 = torch.from_numpy(starts).to(device)
        block_table = None
    # --- queries ------------------------------------------------------------
    if prefill:
        qs, qn = [], []
        for s, L in enumerate(seq_lens):
            first = 0 if queries_per_seq is None else max(0, int(L) - queries_per_seq)
            ts = np.arange(first, int(L))
            qs.append(np.full(ts.size, s))
            qn.append(ts)
        q_seq = np.concatenate(qs) if qs else np.zeros(0, np.int64)
        q_nvis = np.concatenate(qn) if qn else np.zeros(0, np.int64)
    else:
        q_seq = np.arange(num_seqs)
        q_nvis = seq_lens.copy()
    nq = int(q_seq.size)
    # --- values -------------------------------------------------------------
    q_idx = _normal((nq, H_I, D_I), device, seed * 10 + 1)
    w = _normal((nq, H_I), device, seed * 10 + 2, std=1.0 / 8.0)
    k_idx = _normal((rows, D_I), device, seed * 10 + 3)
    q_mla = _normal((nq, H, D), device, seed * 10 + 4, dtype=torch.bfloat16)
    kv = _normal((rows, D), device, seed * 10 + 5, dtype=torch.bfloat16)
    planted = {}
    if plant:
        for s in range(num_seqs):
            L = int(seq_lens[s])
            npl = int(math.floor(0.01 * L))
            if npl == 0:
                continue
            pos = np.sort(np.random.default_rng(seed * 1000 + s).choice(L, npl, replace=False))
            qi = int(np.nonzero(q_seq == s)[0][-1])  # the sequence's (last) query
            mean = q_idx[qi].mean(dim=0)
            noise = _normal((npl, D_I), device, seed * 100000 + 7 * s + 6, std=0.5)
            if paged:
                prow = bt[s, pos // block_size].astype(np.int64) * block_size + pos % block_size
            else:
                prow = int(row0[s].item()) + pos
            k_idx[torch.from_numpy(prow).to(device)] = mean[None, :] + noise
            planted[s] = pos
    return Workload(
        name=name, nq=nq, num_seqs=num_seqs, rows=rows, q_idx=q_idx, w=w, k_idx=k_idx,
        q_mla=q_mla, kv=kv,
        q_seq=torch.from_numpy(q_seq.astype(np.int32)).to(device),
        q_nvis=torch.from_numpy(q_nvis.astype(np.int32)).to(device),
        seq_len=seq_lens, block_size=block_size if paged else 0, row0=row0,
        block_table=block_table, k=k, planted=planted)


def config_seq_lens(cfg: int, seed: int):
    if cfg == 0:
        return [4096]
    if cfg == 1:
        return [32768] * 16
    if cfg == 2:
        return [131072] * 64
    if cfg == 3:
        return [16384]
    if cfg == 4:
        rng = np.random.default_rng(seed + 4_000_000)
        u = rng.uniform(math.log(1024), math.log(131072), 128)
        return np.minimum(np.floor(np.exp(u)), 131072).astype(np.int64).tolist()
    raise ValueError(f"unknown config {cfg}")


def make_config(cfg: int, device="cpu", seed: Optional[int] = None, **kw):
    """The five named workloads (decode 1x4K, 16x32K, 64x128K, prefill 16K,
    ragged paged 128 sequences).  seed defaults to 20260000 + cfg."""
    seed = 20260000 + cfg if seed is None else seed
    lens = config_seq_lens(cfg, seed)
    opts = dict(seq_lens=lens, device=device, seed=seed, name=CONFIG_NAMES[cfg])
    if cfg in (1, 2):
        opts["plant"] = True
    if cfg == 3:
        opts["prefill"] = True
    if cfg == 4:
        opts["paged"] = True
    opts.update(kw)
    return make_custom(**opts)
