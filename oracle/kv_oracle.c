/*
 * kv_oracle.c — plain, slow, obviously-correct CPU definition of the
 * cross-tier KV transfer (device KV pool <-> pinned host KV pool).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library links or calls this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no code, header or table with the GPU path.
 *
 * Sources (the web pages this method is described on):
 *  - "Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section 2.1: the
 *    device side is one buffer per layer; layer_first host dims are
 *    (layer, size, 1, kv_dim); page_first_direct host dims are
 *    (page_num, layer_num, page_size, 1, kv_dim); DMA segments are maximal
 *    contiguous copies, page_num*layer_num of them for page_first_direct and
 *    layer_num for layer_first.
 *  - "HiCache system design", section "data transfer optimisation":
 *    page_first keeps a page contiguous and moves one token per layer at a
 *    time.
 * Readings where the pages are silent (component axis directly inside the
 * layer axis; page_first token-outer; duplicates rejected; half-open layer
 * range) are the same as the library's and are listed in the design notes.
 *
 * Everything is byte copies with memcpy; no value is ever interpreted.
 */
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define KVO_OK 0
#define KVO_EINVAL (-1)
#define KVO_ERANGE (-2)
#define KVO_EDUP (-3)

#define KVO_LAYER_FIRST 0
#define KVO_PAGE_FIRST 1
#define KVO_PAGE_FIRST_DIRECT 2

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* Geometry preconditions. */
int kvo_check_geometry(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps, int layout)
{
    if (L < 1 || C < 1 || ps < 1) return KVO_EINVAL;
    if (R < 16 || R % 16 != 0) return KVO_EINVAL;
    if (S_dev < 1 || S_host < 1) return KVO_EINVAL;
    if (S_host % ps != 0) return KVO_EINVAL;
    if (layout != KVO_LAYER_FIRST && layout != KVO_PAGE_FIRST && layout != KVO_PAGE_FIRST_DIRECT)
        return KVO_EINVAL;
    return KVO_OK;
}

/*
 * Host row holding (layer l, component c, host token slot h), by writing the
 * position out in the layout's dimension order (outermost first):
 *   layer_first        (layer, comp, slot)
 *   page_first         (slot, layer, comp)
 *   page_first_direct  (page, layer, comp, offset-in-page)
 */
int64_t kvo_host_row(int layout, int L, int C, int64_t S_host, int ps, int l, int c, int64_t h)
{
    if (layout == KVO_LAYER_FIRST) {
        int64_t layer_block = (int64_t)l * C * S_host; /* rows before layer l */
        int64_t comp_block = (int64_t)c * S_host;      /* rows before comp c inside layer l */
        return layer_block + comp_block + h;
    }
    if (layout == KVO_PAGE_FIRST) {
        int64_t token_block = h * L * C;               /* rows before token h */
        int64_t layer_block = (int64_t)l * C;          /* rows before layer l inside token h */
        return token_block + layer_block + c;
    }
    /* page_first_direct */
    int64_t page = h / ps;
    int64_t offset = h % ps;
    int64_t page_block = page * L * C * ps;            /* rows before page `page` */
    int64_t layer_block = (int64_t)l * C * ps;         /* rows before layer l inside the page */
    int64_t comp_block = (int64_t)c * ps;              /* rows before comp c inside the layer */
    return page_block + layer_block + comp_block + offset;
}

/*
 * Request validation. direction 0 = backup (D2H, destination = host slots),
 * 1 = load (H2D, destination = device slots). Order of the rules: argument
 * errors, then any index out of range, then a repeated destination.
 */
int kvo_validate(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps, int layout,
                 int direction, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
                 int l0, int l1, int check_unique)
{
    int rc = kvo_check_geometry(L, C, R, S_dev, S_host, ps, layout);
    if (rc != KVO_OK) return rc;
    if (direction != 0 && direction != 1) return KVO_EINVAL;
    if (n < 0) return KVO_EINVAL;
    if (n > 0 && (dev_idx == NULL || host_idx == NULL)) return KVO_EINVAL;
    if (l0 < 0 || l0 > l1 || l1 > L) return KVO_EINVAL;

    for (int64_t i = 0; i < n; i++) {
        if (dev_idx[i] < 0 || dev_idx[i] >= S_dev) return KVO_ERANGE;
        if (host_idx[i] < 0 || host_idx[i] >= S_host) return KVO_ERANGE;
    }
    if (check_unique && n > 1) {
        /* sort a copy of the destinations; a repeat shows up as equal neighbours */
        const int64_t *dst = (direction == 0) ? host_idx : dev_idx;
        int64_t *sorted = (int64_t *)malloc((size_t)n * sizeof(int64_t));
        if (sorted == NULL) return KVO_EINVAL;
        memcpy(sorted, dst, (size_t)n * sizeof(int64_t));
        qsort(sorted, (size_t)n, sizeof(int64_t), cmp_i64);
        int dup = 0;
        for (int64_t i = 1; i < n; i++)
            if (sorted[i] == sorted[i - 1]) dup = 1;
        free(sorted);
        if (dup) return KVO_EDUP;
    }
    return KVO_OK;
}

/*
 * D2H write-back. dev_bufs[l*C + c] is the host mirror of device buffer
 * B[l][c] (S_dev rows of R bytes); host is the host pool (L*C*S_host rows).
 * For each request position i, layer l in [l0,l1) and component c: copy
 * device row dev_idx[i] of B[l][c] to host row host_row(l, c, host_idx[i]).
 */
int kvo_backup(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps, int layout,
               uint8_t *const *dev_bufs, uint8_t *host, const int64_t *dev_idx,
               const int64_t *host_idx, int64_t n, int l0, int l1, int check_unique)
{
    int rc = kvo_validate(L, C, R, S_dev, S_host, ps, layout, 0, dev_idx, host_idx, n, l0, l1,
                          check_unique);
    if (rc != KVO_OK) return rc;
    for (int64_t i = 0; i < n; i++)
        for (int l = l0; l < l1; l++)
            for (int c = 0; c < C; c++) {
                const uint8_t *src = dev_bufs[l * C + c] + dev_idx[i] * R;
                uint8_t *dst = host + kvo_host_row(layout, L, C, S_host, ps, l, c, host_idx[i]) * R;
                memcpy(dst, src, (size_t)R);
            }
    return KVO_OK;
}

/* H2D load: the reverse copy, host row -> device row. */
int kvo_load(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps, int layout,
             uint8_t *const *dev_bufs, const uint8_t *host, const int64_t *dev_idx,
             const int64_t *host_idx, int64_t n, int l0, int l1, int check_unique)
{
    int rc = kvo_validate(L, C, R, S_dev, S_host, ps, layout, 1, dev_idx, host_idx, n, l0, l1,
                          check_unique);
    if (rc != KVO_OK) return rc;
    for (int64_t i = 0; i < n; i++)
        for (int l = l0; l < l1; l++)
            for (int c = 0; c < C; c++) {
                const uint8_t *src =
                    host + kvo_host_row(layout, L, C, S_host, ps, l, c, host_idx[i]) * R;
                uint8_t *dst = dev_bufs[l * C + c] + dev_idx[i] * R;
                memcpy(dst, src, (size_t)R);
            }
    return KVO_OK;
}

/*
 * DMA segments: for every (l, c) buffer pair, walk the request in order and
 * start a new segment whenever the device row or the host row does not
 * continue the previous one by exactly one row. Segments never span two
 * (l, c) buffers. Returns the count (>= 0) or a negative error code.
 */
int64_t kvo_count_segments(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps,
                           int layout, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
                           int l0, int l1)
{
    int rc = kvo_validate(L, C, R, S_dev, S_host, ps, layout, 0, dev_idx, host_idx, n, l0, l1, 0);
    if (rc != KVO_OK) return rc;
    int64_t segments = 0;
    for (int l = l0; l < l1; l++)
        for (int c = 0; c < C; c++) {
            for (int64_t i = 0; i < n; i++) {
                int starts_new = 1;
                if (i > 0) {
                    int64_t prev_host = kvo_host_row(layout, L, C, S_host, ps, l, c, host_idx[i - 1]);
                    int64_t this_host = kvo_host_row(layout, L, C, S_host, ps, l, c, host_idx[i]);
                    int dev_continues = (dev_idx[i] == dev_idx[i - 1] + 1);
                    int host_continues = (this_host == prev_host + 1);
                    starts_new = !(dev_continues && host_continues);
                }
                segments += starts_new;
            }
        }
    return segments;
}
