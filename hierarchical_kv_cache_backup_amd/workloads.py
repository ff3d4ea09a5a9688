"""Seeded synthetic workloads for the cross-tier KV transfer.

This module only describes shapes and draws random index sets and data; it
holds none of the transfer's arithmetic (no address maps, no copies). Tests,
the smoke check and the benchmark all draw their inputs from here.

Shapes follow the pages' workloads (an MLA latent KV of 78 layers x 576 at
page size 64 and a 32K-token prefix: "Tuning SGLang HiCache L2 on Kunlunxin
P800/P900", section 2.1; a GQA K/V pool of 32 layers x 8 heads x 128 in bf16;
a mixed batch of prefix lengths with reuse rate 0.82: same page, section 3).
No dataset is used: the pages' production traces are replaced by the seeded
draws below.

Seeds: numpy.random.default_rng([config, purpose]) with purpose
  0 data, 1 device slots, 2 reload slots, 3 host slots, 4 lengths, 5 offset.
"""
from dataclasses import dataclass, field

import numpy as np

LAYER_FIRST, PAGE_FIRST, PAGE_FIRST_DIRECT = 0, 1, 2
LAYOUT_NAMES = {LAYER_FIRST: "layer_first", PAGE_FIRST: "page_first",
                PAGE_FIRST_DIRECT: "page_first_direct"}

P_DATA, P_DEV, P_RELOAD, P_HOST, P_LEN, P_OFFSET = range(6)

SENTINEL = 0xA5


def rng(cfg, purpose):
    return np.random.default_rng([int(cfg), int(purpose)])


@dataclass
class Shape:
    """Pool shape. row_bytes = heads * head_dim * elem_bytes."""
    name: str
    layers: int
    components: int
    heads: int
    head_dim: int
    elem_bytes: int
    device_slots: int
    host_slots: int
    page_size: int
    dtype: str = "bf16"
    layouts: tuple = (LAYER_FIRST,)
    extra: dict = field(default_factory=dict)

    @property
    def row_bytes(self):
        return self.heads * self.head_dim * self.elem_bytes

    def bytes_per_token(self, nlayers=None):
        nl = self.layers if nlayers is None else nlayers
        return nl * self.components * self.row_bytes

    def device_pool_bytes(self):
        return self.layers * self.components * self.device_slots * self.row_bytes

    def host_pool_bytes(self):
        return self.layers * self.components * self.host_slots * self.row_bytes

    def scaled(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Shape(**d)


# ---- the five workloads ---------------------------------------------------

def tiny():
    """4 layers, K/V [256 slots, 2 heads, 64] bf16, page 16; 16 pages backed up
    from a seeded token-level slot permutation, reloaded into fresh slots."""
    return Shape("tiny", 4, 2, 2, 64, 2, 256, 256, 16, "bf16",
                 (LAYER_FIRST, PAGE_FIRST, PAGE_FIRST_DIRECT))


def llama8b():
    """Llama-3-8B-shaped K/V: 32 layers, [131072 slots, 8 heads, 128] bf16, page 64;
    D2H of an 8192-token prefix from fragmented device pages into page_first."""
    return Shape("llama8b", 32, 2, 8, 128, 2, 131072, 8192, 64, "bf16",
                 (PAGE_FIRST, LAYER_FIRST, PAGE_FIRST_DIRECT), {"tokens": 8192})


def mla32k():
    """MLA-latent-shaped KV: 78 layers, one latent [65536 slots, 1, 576] bf16, page 64;
    H2D load of a 32768-token prefix (512 pages)."""
    return Shape("mla32k", 78, 1, 1, 576, 2, 65536, 32768, 64, "bf16",
                 (PAGE_FIRST_DIRECT, LAYER_FIRST, PAGE_FIRST), {"tokens": 32768})


def mixed():
    """64 requests, lengths ~ lognormal(median 4096, sigma 1.0) clipped to
    [64, 32768] and rounded up to whole pages, 32 layers x 8 x 128 bf16 K/V,
    page 64; per request the first floor(0.82*len/64)*64 tokens are L2 hits
    (H2D) and the rest are new (D2H)."""
    return Shape("mixed", 32, 2, 8, 128, 2, 0, 0, 64, "bf16",
                 (LAYER_FIRST, PAGE_FIRST), {"requests": 64, "median": 4096, "sigma": 1.0,
                                             "max_len": 32768, "reuse": 0.82})


def streamed():
    """61 layers, K/V [262144 slots, 8 heads, 128] fp8 e4m3 (random bytes), page 64;
    per-layer H2D of a 131072-token prefix overlapped with an HBM-bound kernel."""
    return Shape("streamed", 61, 2, 8, 128, 1, 262144, 131072, 64, "fp8",
                 (LAYER_FIRST, PAGE_FIRST_DIRECT), {"tokens": 131072})


CONFIGS = {1: tiny, 2: llama8b, 3: mla32k, 4: mixed, 5: streamed}


# ---- index sets -------------------------------------------------------------

def tiny_indices(shape, cfg=1):
    """Backup: a token-level permutation of all device slots -> host slots 0..n-1.
    Reload: an independent permutation of the device slots of a fresh pool."""
    n = shape.device_slots
    dev = rng(cfg, P_DEV).permutation(n).astype(np.int64)
    host = np.arange(n, dtype=np.int64)
    reload = rng(cfg, P_RELOAD).permutation(n).astype(np.int64)
    return dev, host, reload


def page_indices(pages, page_size):
    """Token slots of whole pages, in the given page order."""
    pages = np.asarray(pages, dtype=np.int64)
    return (pages[:, None] * page_size + np.arange(page_size, dtype=np.int64)[None, :]).reshape(-1)


def fragmented_pages(cfg, total_pages, count, purpose=P_DEV):
    """`count` distinct pages drawn at random from `total_pages`, in random order."""
    return rng(cfg, purpose).choice(total_pages, size=count, replace=False).astype(np.int64)


def contiguous_pages_at_offset(cfg, total_pages, count):
    off = int(rng(cfg, P_OFFSET).integers(0, total_pages - count + 1))
    return np.arange(off, off + count, dtype=np.int64)


def prefix_indices(shape, cfg, tokens, fragmented, device_pages_available=None):
    """(dev_idx, host_idx) for a prefix of `tokens` tokens (whole pages).
    Device: contiguous pages at a seeded offset, or (fragmented) random distinct
    pages in random order. Host: slots 0..tokens-1."""
    ps = shape.page_size
    assert tokens % ps == 0
    npages = tokens // ps
    total = (shape.device_slots // ps) if device_pages_available is None else device_pages_available
    if fragmented:
        pages = fragmented_pages(cfg, total, npages)
    else:
        pages = contiguous_pages_at_offset(cfg, total, npages)
    return page_indices(pages, ps), np.arange(tokens, dtype=np.int64)


def mixed_requests(shape, cfg=4, scale=1.0):
    """Lengths, hit tokens and new tokens of the mixed batch (see mixed())."""
    ex = shape.extra
    r = rng(cfg, P_LEN)
    nreq = max(1, int(round(ex["requests"] * scale)))
    raw = r.lognormal(mean=np.log(ex["median"] * scale), sigma=ex["sigma"], size=nreq)
    ps = shape.page_size
    lens = np.clip(raw, ps, ex["max_len"] * scale)
    lens = (np.ceil(lens / ps) * ps).astype(np.int64)
    hits = (np.floor(ex["reuse"] * lens / ps) * ps).astype(np.int64)
    new = lens - hits
    return lens, hits, new


def mixed_plan(shape, cfg=4, scale=1.0, fragmented=False):
    """Index sets of the mixed batch. Every request owns a fresh contiguous run
    of device slots (or random pages); its hit tokens come from a random
    permutation of host pages; its new tokens go to the next free host pages.
    Returns dict with total sizes and the concatenated H2D and D2H index sets."""
    lens, hits, new = mixed_requests(shape, cfg, scale)
    ps = shape.page_size
    total_tokens = int(lens.sum())
    dev_slots = total_tokens
    host_slots = total_tokens
    dev_pages_all = np.arange(dev_slots // ps, dtype=np.int64)
    if fragmented:
        dev_pages_all = rng(cfg, P_DEV).permutation(dev_pages_all)
    host_pages_all = rng(cfg, P_HOST).permutation(host_slots // ps).astype(np.int64)
    h2d_dev, h2d_host, d2h_dev, d2h_host = [], [], [], []
    dp = 0
    hp = 0
    for ln, ht, nw in zip(lens, hits, new):
        npg = int(ln // ps)
        dpages = dev_pages_all[dp:dp + npg]
        dp += npg
        hpages = host_pages_all[hp:hp + npg]
        hp += npg
        hpg = int(ht // ps)
        h2d_dev.append(page_indices(dpages[:hpg], ps))
        h2d_host.append(page_indices(hpages[:hpg], ps))
        d2h_dev.append(page_indices(dpages[hpg:], ps))
        d2h_host.append(page_indices(hpages[hpg:], ps))
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)
    return {"lens": lens, "hits": hits, "new": new, "device_slots": dev_slots,
            "host_slots": host_slots, "h2d": (cat(h2d_dev), cat(h2d_host)),
            "d2h": (cat(d2h_dev), cat(d2h_host))}


def churn_requests(shape, cfg, count, device_pages, max_pages):
    """A stream of `count` write-back requests for a free-list churn: each has a
    length in whole pages, drawn like the mixed batch's (lognormal, median 4096
    tokens, sigma 1.0, at most `max_pages` pages), and a contiguous run of device
    pages at a seeded offset (the request's own KV in a fresh device pool).
    Returns a list of (npages, first_device_page)."""
    ex = mixed().extra
    ps = shape.page_size
    r_len = rng(cfg, P_LEN)
    r_off = rng(cfg, P_OFFSET)
    out = []
    for _ in range(count):
        tokens = r_len.lognormal(mean=np.log(ex["median"]), sigma=ex["sigma"])
        npg = int(min(max_pages, max(1, np.ceil(tokens / ps))))
        first = int(r_off.integers(0, device_pages - npg + 1))
        out.append((npg, first))
    return out


# ---- data -------------------------------------------------------------------

def host_rows_random(cfg, nbytes):
    """Seeded random bytes (CPU), e.g. for small device pools built on the host."""
    return rng(cfg, P_DATA).integers(0, 256, size=nbytes, dtype=np.uint8)


def fill_device_buffer(tensor_u8, shape, cfg, layer, comp, torch):
    """Fill one device buffer (uint8 tensor of S_dev*R bytes) with seeded data:
    bf16 N(0,1) for bf16 shapes, uniform random bytes for fp8 shapes. Data is
    generated on the device with a torch generator seeded per (cfg, layer, comp)."""
    g = torch.Generator(device=tensor_u8.device)
    g.manual_seed(int(cfg) * 1_000_003 + int(layer) * 131 + int(comp) * 7 + 1)
    if shape.dtype == "bf16":
        v = tensor_u8.view(torch.bfloat16)
        v.normal_(0.0, 1.0, generator=g)
    else:
        tensor_u8.random_(0, 256, generator=g)
