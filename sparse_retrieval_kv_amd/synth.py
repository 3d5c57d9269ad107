"""Seeded synthetic workloads for retrieval-sparse paged decode attention.

This module only builds inputs: paged K/V pools, block tables, lengths,
per-step queries and per-step appended tokens.  It holds none of the method's
arithmetic (no representation, scoring, selection or attention), so both the
HIP library's tests/bench and the CPU oracle can consume what it makes.

Values are drawn in float32 and rounded once to bf16 (round to nearest even,
through torch's conversion); the library and the oracle read the same bits.
Seeds are ``1000 * config + stream`` with one stream per kind of value.

Pool layout (the library's ABI layout):
  k_pages  int16 bit patterns of bf16, [P, Hkv, 128 tokens, 128 dims]
  v_pages  int16 bit patterns of bf16, [P, Hkv, 128 dims, 128 tokens]
  block_table int32 [B, max_blocks], logical block -> physical page, -1 unused

A sequence of context N holds N - 1 prefill tokens in the pool; decode step t
appends the token at position N - 1 + t, so the length at step t is N + t and
counts the token being decoded.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

BLOCK = 128
HEAD_DIM = 128
BF16_QNAN = 0x7FC0  # written into never-filled slots to catch missing masks

# stream ids for the seeds
S_Q, S_K, S_V, S_PLANT, S_LEN, S_PERM, S_NEW, S_OFFSET = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class Spec:
    """Shape and structure of one workload."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    context: tuple = ()            # L at step 0 per sequence (fixed lengths)
    len_range: tuple | None = None  # (lo, hi) inclusive, drawn per sequence
    steps: int = 1
    init_tokens: int = 1024
    local_tokens: int = 7192
    topk_ppm: int = 200_000
    dense_boundary: int = 32768
    plant_count: int = 0           # planted offload blocks per sequence
    plant_range: tuple = (0, 0)    # offload block range at step 0 (hand-derived)
    plant_mode: str = "none"       # "qmean" (one step) or "shared_u" (multi-step)
    shuffle: bool = False          # shuffled physical page order
    shared_prefix_pages: int = 0   # pages shared by every sequence
    key_head_offset: bool = False  # per-KV-head random mean added to keys
    host_offload: bool = False     # offload pages live in pinned host memory
    config_id: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


# The five workloads.  plant_range is the offload block range at step 0,
# worked out by hand from the region rule (init = ceil(init/128) blocks,
# local starts at floor((L - local)/128)):
#   tiny (1 x 4K): L=4096, init 256, local 512 -> init blocks 2, local start 28 -> [2, 28)
#   8B layer (1 x 64K): L=65536, 1024/7192 -> 8, floor(58344/128)=455 -> [8, 455)
#   host tier (4 x 256K): L=262144 -> 8, floor(254952/128)=1991 -> [8, 1991)
CONFIGS = {
    1: Spec("tiny sparse decode, 1 x 4K, 8/2 heads", 1, 8, 2, context=(4096,),
            steps=1, init_tokens=256, local_tokens=512, dense_boundary=0,
            plant_count=2, plant_range=(2, 28), plant_mode="qmean",
            config_id=1),
    2: Spec("Llama-3-8B-shaped layer, 1 x 64K, 32/8 heads", 1, 32, 8,
            context=(65536,), steps=64, plant_count=23, plant_range=(8, 455),
            plant_mode="shared_u", config_id=2),
    3: Spec("batched paged decode, 16 x U[32K,128K], 32/8 heads, shuffled pool",
            16, 32, 8, len_range=(32768, 131072), steps=32, shuffle=True,
            config_id=3),
    4: Spec("70B-shaped layer, 8 x 128K, 64/8 heads, 16K shared prefix",
            8, 64, 8, context=(131072,) * 8, steps=16, shuffle=True,
            shared_prefix_pages=128, key_head_offset=True, config_id=4),
    5: Spec("host-offload tier, 4 x 256K, 32/8 heads", 4, 32, 8,
            context=(262144,) * 4, steps=16, plant_count=60,
            plant_range=(8, 1991), plant_mode="shared_u", host_offload=True,
            config_id=5),
}


def np_rng(spec: Spec, stream: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        [1000 * spec.config_id + stream, salt]))


def torch_gen(spec: Spec, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1000 * spec.config_id + stream)
    return g


def to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """float32 -> bf16 (round to nearest even) -> int16 bit pattern."""
    return x.to(torch.bfloat16).view(torch.int16)


class PagePool:
    """Host-side page allocator with reference counts (pages shared by
    several block tables are stored once and freed when the count is 0)."""

    def __init__(self, n_pages: int, order: np.ndarray | None = None):
        self.n_pages = n_pages
        self.refcount = np.zeros(n_pages, dtype=np.int64)
        self._free = list(order if order is not None else range(n_pages))
        self._free.reverse()

    def allocate(self) -> int:
        p = self._free.pop()
        self.refcount[p] = 1
        return p

    def acquire(self, p: int) -> int:
        assert self.refcount[p] > 0
        self.refcount[p] += 1
        return p

    def release(self, p: int) -> None:
        assert self.refcount[p] > 0
        self.refcount[p] -= 1
        if self.refcount[p] == 0:
            self._free.append(p)


@dataclass
class Batch:
    spec: Spec
    device: torch.device
    k_pages: torch.Tensor          # int16 [P, Hkv, 128, 128]
    v_pages: torch.Tensor          # int16 [P, Hkv, 128, 128] (dim-major)
    block_table: torch.Tensor      # int32 [B, max_blocks]
    table_np: np.ndarray           # same, on the host
    context: np.ndarray            # int64 [B], L at step 0
    max_blocks: int
    n_pages: int
    planted: dict                  # b -> array of planted logical blocks
    refcount: np.ndarray
    u: np.ndarray | None           # [B, Hkv, d] per-group planting direction
    head_offset: np.ndarray | None  # [Hkv, d]
    q0: np.ndarray | None = None   # float32 [B, Hq, d], step-0 query (qmean mode)
    host_pages: np.ndarray | None = None  # bool [P]: page lives in host memory
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return self.spec.batch

    def lens_at(self, t: int) -> np.ndarray:
        return (self.context + t).astype(np.int32)

    def q_f32(self, t: int) -> np.ndarray:
        """float32 query [B, Hq, d] of decode step t."""
        s = self.spec
        if s.plant_mode == "qmean" and t == 0:
            return self.q0
        z = np_rng(s, S_Q, t).standard_normal(
            (s.batch, s.n_q_heads, HEAD_DIM), dtype=np.float32)
        if s.plant_mode == "shared_u":
            u = np.repeat(self.u, s.group, axis=1)
            z = ((u + z) / np.float32(math.sqrt(2.0))).astype(np.float32)
        return z

    def q_bits(self, t: int) -> torch.Tensor:
        return to_bf16_bits(torch.from_numpy(self.q_f32(t))).to(self.device)

    def new_kv_f32(self, t: int):
        """float32 K and V [B, Hkv, d] of the token appended at step t."""
        s = self.spec
        r = np_rng(s, S_NEW, t)
        k = r.standard_normal((s.batch, s.n_kv_heads, HEAD_DIM), dtype=np.float32)
        v = r.standard_normal((s.batch, s.n_kv_heads, HEAD_DIM), dtype=np.float32)
        if self.head_offset is not None:
            k = (k + self.head_offset[None]).astype(np.float32)
        return k, v

    def new_kv_bits(self, t: int):
        k, v = self.new_kv_f32(t)
        return (to_bf16_bits(torch.from_numpy(k)).to(self.device),
                to_bf16_bits(torch.from_numpy(v)).to(self.device))


def _plant_blocks(spec: Spec, rng: np.random.Generator) -> dict:
    out = {}
    lo, hi = spec.plant_range
    for b in range(spec.batch):
        if spec.plant_count > 0:
            out[b] = np.sort(rng.choice(np.arange(lo, hi), spec.plant_count,
                                        replace=False))
        else:
            out[b] = np.zeros(0, dtype=np.int64)
    return out


def make_batch(spec: Spec, device="cpu", poison_tail: bool = True,
               extra_pages: int = 0) -> Batch:
    """Build the pools, tables and per-step generators of a workload.
    `extra_pages` NaN-filled pages are appended to the pools (e.g. staging
    pages for the host tier); they belong to no block table."""
    device = torch.device(device)
    B, Hkv, G = spec.batch, spec.n_kv_heads, spec.group
    if spec.len_range is not None:
        lo, hi = spec.len_range
        context = np_rng(spec, S_LEN).integers(lo, hi + 1, size=B)
    else:
        context = np.asarray(spec.context, dtype=np.int64)
        assert context.shape == (B,)
    final_len = context + spec.steps - 1
    nblk = -(-final_len // BLOCK)
    max_blocks = int(nblk.max())
    shared = spec.shared_prefix_pages
    # every sequence extends past the shared prefix: its decoded tokens (and
    # the padding after its end) go to pages of its own, never to a shared one
    assert shared == 0 or int(context.min()) > shared * BLOCK, \
        "every context must extend past the shared prefix"
    n_pages = int(shared + (nblk - shared).sum())

    order = None
    if spec.shuffle:
        order = np_rng(spec, S_PERM).permutation(n_pages)
    pool = PagePool(n_pages, order)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    prefix = [pool.allocate() for _ in range(shared)]
    for b in range(B):
        for j in range(int(nblk[b])):
            table[b, j] = pool.acquire(prefix[j]) if j < shared else pool.allocate()
    if shared:
        for p in prefix:  # the allocation's own reference is not a table's
            pool.release(p)

    # Pool values: N(0,1) per element, drawn page by page on the device.
    k_pages = torch.empty((n_pages, Hkv, BLOCK, HEAD_DIM), dtype=torch.int16,
                          device=device)
    v_pages = torch.empty_like(k_pages)
    gk, gv = torch_gen(spec, S_K, device), torch_gen(spec, S_V, device)
    head_offset = None
    if spec.key_head_offset:
        head_offset = np_rng(spec, S_OFFSET).standard_normal(
            (Hkv, HEAD_DIM), dtype=np.float32)
        off_t = torch.from_numpy(head_offset).to(device)[None, :, None, :]
    chunk = max(1, (1 << 27) // (Hkv * BLOCK * HEAD_DIM))
    for p0 in range(0, n_pages, chunk):
        p1 = min(n_pages, p0 + chunk)
        shp = (p1 - p0, Hkv, BLOCK, HEAD_DIM)
        k = torch.randn(shp, generator=gk, device=device, dtype=torch.float32)
        if head_offset is not None:
            k += off_t
        k_pages[p0:p1] = to_bf16_bits(k)
        del k
        v = torch.randn(shp, generator=gv, device=device, dtype=torch.float32)
        v_pages[p0:p1] = to_bf16_bits(v)
        del v

    prng = np_rng(spec, S_PLANT)
    planted = _plant_blocks(spec, prng)
    u = q0 = None
    if spec.plant_mode == "shared_u":
        u = prng.standard_normal((B, Hkv, HEAD_DIM), dtype=np.float32)
    elif spec.plant_mode == "qmean":
        q0 = np_rng(spec, S_Q, 0).standard_normal(
            (B, spec.n_q_heads, HEAD_DIM), dtype=np.float32)
    gp = torch.Generator(device=device)
    gp.manual_seed(1000 * spec.config_id + S_PLANT)
    for b in range(B):
        for j in planted[b]:
            page = int(table[b, j])
            if spec.plant_mode == "qmean":
                # K = 0.5 * mean of the group's step-0 queries + N(0, 1)
                qm = q0[b].reshape(Hkv, G, HEAD_DIM).mean(axis=1)
                shift = 0.5 * qm
            else:
                # K = N(0, 1) + 0.5 * u / sqrt(2), u the group's query direction
                shift = 0.5 * u[b] / np.float32(math.sqrt(2.0))
            noise = torch.randn((Hkv, BLOCK, HEAD_DIM), generator=gp,
                                device=device, dtype=torch.float32)
            noise += torch.from_numpy(shift.astype(np.float32)).to(device)[:, None, :]
            k_pages[page] = to_bf16_bits(noise)

    if poison_tail:
        # slots at and after the first decode position were never written by
        # the prefill: fill them with NaN so a missing mask shows up
        for b in range(B):
            first = int(context[b]) - 1
            for j in range(first // BLOCK, int(nblk[b])):
                page = int(table[b, j])
                s0 = max(first - j * BLOCK, 0)
                k_pages[page, :, s0:, :] = BF16_QNAN
                v_pages[page, :, :, s0:] = BF16_QNAN

    host_pages = None
    if spec.host_offload:
        host_pages = np.zeros(n_pages, dtype=bool)
        lo, hi = spec.plant_range
        for b in range(B):
            host_pages[table[b, lo:hi]] = True

    if extra_pages:
        pad = torch.full((extra_pages, Hkv, BLOCK, HEAD_DIM), BF16_QNAN,
                         dtype=torch.int16, device=device)
        k_pages = torch.cat([k_pages, pad])
        v_pages = torch.cat([v_pages, pad])
        del pad

    return Batch(spec, device, k_pages, v_pages,
                 torch.from_numpy(table).to(device), table, context,
                 max_blocks, n_pages, planted, pool.refcount.copy(), u,
                 head_offset, q0, host_pages)


@dataclass
class HostPools:
    host_k: torch.Tensor       # pinned int16 [P_host, Hkv, 128, 128]
    host_v: torch.Tensor       # pinned int16 [P_host, Hkv, 128, 128] (dim-major)
    host_table: torch.Tensor   # int32 [B, max_blocks] on the device, -1 = in HBM
    host_table_np: np.ndarray


def plan_host_pools(batch: Batch) -> HostPools:
    """Pinned host pools (uninitialised) and the host page of every offload
    block of the spec's block range at step 0: sequence b's blocks
    [lo, hi) take host pages b * (hi - lo) + 0, 1, ...; -1 elsewhere."""
    spec = batch.spec
    lo, hi = spec.plant_range
    B, Hkv = spec.batch, spec.n_kv_heads
    host_table = np.full_like(batch.table_np, -1)
    for b in range(B):
        host_table[b, lo:hi] = b * (hi - lo) + np.arange(hi - lo)
    n_host = B * (hi - lo)
    host_k = torch.empty((n_host, Hkv, BLOCK, HEAD_DIM), dtype=torch.int16,
                         pin_memory=True)
    host_v = torch.empty_like(host_k, pin_memory=True)
    return HostPools(host_k, host_v,
                     torch.from_numpy(host_table).to(batch.k_pages.device),
                     host_table)


def poison_device_copies(batch: Batch, host: HostPools) -> None:
    """Fill the device pages of host-resident blocks with NaN, so that only
    the host copies carry their data."""
    pages = batch.table_np[host.host_table_np >= 0]
    idx = torch.as_tensor(pages.astype(np.int64), device=batch.k_pages.device)
    for s0 in range(0, len(pages), 1024):
        sl = idx[s0:s0 + 1024]
        batch.k_pages[sl] = BF16_QNAN
        batch.v_pages[sl] = BF16_QNAN
    if batch.k_pages.is_cuda:
        torch.cuda.synchronize(batch.k_pages.device)


def move_offload_to_host(batch: Batch) -> HostPools:
    """Place the offload blocks (the spec's block range at step 0) of every
    sequence in pinned host memory: copy their pages to host pools (torch
    copies), record the host page of each block, and fill the device copies
    with NaN so that only the host copies carry the data."""
    host = plan_host_pools(batch)
    B = batch.spec.batch
    pages = np.concatenate([batch.table_np[b][host.host_table_np[b] >= 0]
                            for b in range(B)])
    idx = torch.as_tensor(pages.astype(np.int64), device=batch.k_pages.device)
    n_host = len(pages)
    for s0 in range(0, n_host, 1024):
        sl = idx[s0:s0 + 1024]
        host.host_k[s0:s0 + 1024].copy_(batch.k_pages.index_select(0, sl))
        host.host_v[s0:s0 + 1024].copy_(batch.v_pages.index_select(0, sl))
    poison_device_copies(batch, host)
    return host


def custom(name="custom", batch=1, n_q_heads=8, n_kv_heads=2, context=(4096,),
           steps=1, config_id=90, **kw) -> Spec:
    """A workload with chosen sizes, for tests at oracle-friendly scale."""
    return Spec(name, batch, n_q_heads, n_kv_heads, context=tuple(context),
                steps=steps, config_id=config_id, **kw)


def scaled(spec: Spec, **kw) -> Spec:
    return replace(spec, **kw)
