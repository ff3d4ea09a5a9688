"""Oracle of the write-through-selective filter with a Ghost List.

TEST INFRASTRUCTURE ONLY. Tests, the smoke check and the benchmark's CPU
baseline may use this module; the library never does, and this module imports
nothing from the library.

What it computes ("Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section
2.6, "Write-policy semantic fix + Ghost List"; "Baidu's KVCache Overhaul",
"write_through_selective with Ghost List"):

* Page-boundary hashes. A request's tokens are cut into pages; the hash at the
  end of page k covers every token from the root up to that boundary, so it
  names both the page's content and its position in the prefix. Readings
  where the pages leave the step open: the hash is 64-bit FNV-1a (its
  published definition: offset basis 0xcbf29ce484222325, prime
  0x100000001b3, per byte xor then multiply modulo 2**64) over the token ids
  as 4-byte little-endian signed integers; a trailing partial page has no
  hash.
* The Ghost List. When pages leave L1 their KV is dropped but their hashes are
  kept in a bounded map in least-recently-inserted order: inserting a hash
  that is present makes it the most recent; inserting into a full list first
  drops the least recent. Reading: a lookup does not change the order.
* The reuse proof. When a prefix is rebuilt, its page hashes are scanned from
  the last page backwards; the first hash found in the Ghost List ends the
  longest prefix proven to be reused, and only that prefix is written back.

Every function here is written from the definitions above, without the
incremental or table-driven shortcuts the library takes.
"""
from collections import OrderedDict

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data, h=FNV_OFFSET):
    """64-bit FNV-1a of a byte string."""
    for b in bytes(data):
        h ^= b
        h = (h * FNV_PRIME) & MASK64
    return h


def token_bytes(tokens):
    return b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)


def page_hashes(tokens, page_size):
    """Hash at the end of every full page: FNV-1a over all tokens from the root
    to that page boundary (recomputed from the root for each page)."""
    assert page_size >= 1
    tokens = list(tokens)
    return [fnv1a64(token_bytes(tokens[:(k + 1) * page_size]))
            for k in range(len(tokens) // page_size)]


class GhostList:
    """Bounded set of page hashes in least-recently-inserted order."""

    def __init__(self, capacity):
        assert capacity >= 1
        self.capacity = capacity
        self.d = OrderedDict()

    def insert(self, hashes):
        """Record evicted pages, in the given order."""
        for h in hashes:
            h = int(h) & MASK64
            if h in self.d:
                self.d.move_to_end(h)
            else:
                if len(self.d) == self.capacity:
                    self.d.popitem(last=False)
                self.d[h] = None

    def contains(self, h):
        return (int(h) & MASK64) in self.d

    def reuse_prefix(self, hashes):
        """Pages in the longest prefix whose last page hash is in the list: scan
        from the last page back; 0 when none is."""
        for k in range(len(hashes) - 1, -1, -1):
            if self.contains(hashes[k]):
                return k + 1
        return 0

    def size(self):
        return len(self.d)

    def order(self):
        """Hashes from least to most recent."""
        return list(self.d)
