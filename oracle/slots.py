"""Oracle of the host pool's page allocator (FIFO or LIFO free list).

TEST INFRASTRUCTURE ONLY. Tests and the benchmark's CPU baseline may use this
module; the library never does, and this module imports nothing from it.

What it computes ("Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section
2.4, "LIFO free list"; "Baidu's KVCache Overhaul", "LIFO slot allocation"): the
host pool is handed out in pages from a free list. With the default FIFO policy
pages freed go to the tail, so under churn allocation walks the whole pool;
with LIFO the pages freed last are reused first, so writes stay on a small set
of hot pages. The policy changes which pages a write-back lands on, nothing
else.

Readings where the pages leave the steps open:

* the free list starts as pages 0, 1, ..., P-1;
* an allocation of k pages removes the first k entries of the list and returns
  them in list order; it fails (changing nothing) if fewer than k are free;
* a free inserts its batch, in the batch's order, at the tail (FIFO) or at the
  head (LIFO) of the list;
* a free is refused, changing nothing, if a page is out of range (checked over
  the whole batch first), not allocated, or listed twice.

The free list here is a plain Python list, edited by slicing.
"""
OK, EINVAL, ERANGE, ENOMEM = 0, -1, -2, -4
FIFO, LIFO = 0, 1


class FreeList:
    def __init__(self, num_pages, policy):
        assert num_pages >= 1 and policy in (FIFO, LIFO)
        self.num_pages = num_pages
        self.policy = policy
        self.free = list(range(num_pages))
        self.allocated = set()

    def alloc(self, k):
        """(status, pages): the first k pages of the free list."""
        if k < 0:
            return EINVAL, []
        if k > len(self.free):
            return ENOMEM, []
        taken = self.free[:k]
        self.free = self.free[k:]
        self.allocated.update(taken)
        return OK, taken

    def release(self, pages):
        """Status of returning a batch of pages to the free list."""
        pages = [int(p) for p in pages]
        for p in pages:
            if p < 0 or p >= self.num_pages:
                return ERANGE
        seen = set()
        for p in pages:
            if p not in self.allocated or p in seen:
                return EINVAL
            seen.add(p)
        for p in pages:
            self.allocated.remove(p)
        if self.policy == FIFO:
            self.free = self.free + pages
        else:
            self.free = pages + self.free
        return OK

    def available(self):
        return len(self.free)

    def order(self):
        """The free list, head first."""
        return list(self.free)
