"""NumPy cross-derivation of the cross-tier KV copies — TEST INFRASTRUCTURE ONLY.

Independent of the C oracle's host-row formula: the host pool is reshaped into
each layout's dimension order, outermost first, and rows are assigned through
fancy indexing.

* layer_first        (layer, comp, slot, row)        — "(layer, size, 1, kv_dim)",
                      Kunlunxin tuning page, section 2.1.
* page_first         (slot, layer, comp, row)        — a page is contiguous and is
                      moved one token per layer ("HiCache system design",
                      section "data transfer optimisation"); token-outer reading.
* page_first_direct  (page, layer, comp, offset, row) — "(page_num, layer_num,
                      page_size, 1, kv_dim)", Kunlunxin tuning page, section 2.1.

The component axis (K/V) sits directly inside the layer axis in all three (the
pages give MLA shapes with a single latent; this is the reading used here).
The device pool is a stacked (L, C, S_dev, R) uint8 array.
"""
import numpy as np

LAYER_FIRST, PAGE_FIRST, PAGE_FIRST_DIRECT = 0, 1, 2


def host_view(host, layout, L, C, S_host, ps, R):
    """The host pool as an array in the layout's own dimension order (a view, no copy)."""
    if layout == LAYER_FIRST:
        return host.reshape(L, C, S_host, R)
    if layout == PAGE_FIRST:
        return host.reshape(S_host, L, C, R)
    if layout == PAGE_FIRST_DIRECT:
        return host.reshape(S_host // ps, L, C, ps, R)
    raise ValueError(layout)


def _host_rows(view, layout, host_idx, l0, l1, ps):
    """Index expression selecting rows (n, nl, C, R) of the view, as (key, order)."""
    h = np.asarray(host_idx, dtype=np.int64)
    if layout == LAYER_FIRST:
        return (slice(l0, l1), slice(None), h), "lcn"
    if layout == PAGE_FIRST:
        return (h, slice(l0, l1), slice(None)), "nlc"
    page, offset = np.divmod(h, ps)
    return (page, slice(l0, l1), slice(None), offset), "nlc"


def backup(dev, host, layout, L, C, S_host, ps, R, dev_idx, host_idx, l0=0, l1=None):
    """host (flat uint8, modified in place) <- dev (L, C, S_dev, R)."""
    l1 = L if l1 is None else l1
    view = host_view(host, layout, L, C, S_host, ps, R)
    src = dev[l0:l1, :, np.asarray(dev_idx, dtype=np.int64), :]          # (nl, C, n, R)
    key, order = _host_rows(view, layout, host_idx, l0, l1, ps)
    view[key] = src if order == "lcn" else src.transpose(2, 0, 1, 3)


def load(dev, host, layout, L, C, S_host, ps, R, dev_idx, host_idx, l0=0, l1=None):
    """dev (L, C, S_dev, R, modified in place) <- host (flat uint8)."""
    l1 = L if l1 is None else l1
    view = host_view(host, layout, L, C, S_host, ps, R)
    key, order = _host_rows(view, layout, host_idx, l0, l1, ps)
    rows = view[key]
    if order == "nlc":
        rows = rows.transpose(1, 2, 0, 3)                                  # -> (nl, C, n, R)
    dev[l0:l1, :, np.asarray(dev_idx, dtype=np.int64), :] = rows


def row_id_table(layout, L, C, S_host, ps):
    """(L, C, S_host) table of host row numbers, obtained by enumerating the
    rows of the host pool in storage order and viewing them in the layout's
    dimension order (no address formula)."""
    ids = np.arange(L * C * S_host, dtype=np.int64)
    if layout == LAYER_FIRST:
        return ids.reshape(L, C, S_host)
    if layout == PAGE_FIRST:
        return ids.reshape(S_host, L, C).transpose(1, 2, 0)
    v = ids.reshape(S_host // ps, L, C, ps).transpose(1, 2, 0, 3)          # (L, C, P, ps)
    return v.reshape(L, C, S_host)


def count_segments(layout, L, C, S_host, ps, dev_idx, host_idx, l0=0, l1=None):
    """DMA segments counted from the row-id table: a segment breaks wherever the
    device slot or the host row fails to advance by one."""
    l1 = L if l1 is None else l1
    d = np.asarray(dev_idx, dtype=np.int64)
    n = d.size
    if n == 0 or l1 <= l0:
        return 0
    table = row_id_table(layout, L, C, S_host, ps)
    rows = table[l0:l1, :, np.asarray(host_idx, dtype=np.int64)]        # (nl, C, n)
    dev_cont = np.diff(d) == 1                                            # (n-1,)
    host_cont = np.diff(rows, axis=2) == 1                                # (nl, C, n-1)
    continues = host_cont & dev_cont[None, None, :]
    return int(rows.shape[0] * rows.shape[1] * n - continues.sum())
