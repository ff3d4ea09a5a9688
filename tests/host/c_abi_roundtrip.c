/*
 * c_abi_roundtrip.c — a client of libkvtier.so written against include/kvtier.h
 * alone: no Python, no torch. Device buffers and streams come from the HIP
 * runtime, transfers from the C ABI, and the expected bytes from the C oracle
 * (oracle/kv_oracle.c, compiled into this test program). For every host layout
 * and path: a backup into a sentinel-filled host pool and a load into other
 * device slots, both compared byte for byte, per-layer waits through
 * kv_load_layer on a library stream, and one refused request. Prints
 * "<n> failures".
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvtier.h"

int kvo_backup(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps, int layout,
               uint8_t *const *dev_bufs, uint8_t *host, const int64_t *dev_idx,
               const int64_t *host_idx, int64_t n, int l0, int l1, int check_unique);
int kvo_load(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps, int layout,
             uint8_t *const *dev_bufs, const uint8_t *host, const int64_t *dev_idx,
             const int64_t *host_idx, int64_t n, int l0, int l1, int check_unique);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static uint64_t next_u64(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545f4914f6cdd1dull;
}

static void random_bytes(uint8_t *p, size_t n) {
  for (size_t i = 0; i < n; i++) p[i] = (uint8_t)(next_u64() >> 56);
}

/* n distinct values of [0, range) in random order (partial Fisher-Yates). */
static void distinct(int64_t *out, int64_t n, int64_t range) {
  int64_t *all = malloc(sizeof(int64_t) * (size_t)range);
  for (int64_t i = 0; i < range; i++) all[i] = i;
  for (int64_t i = 0; i < n; i++) {
    int64_t j = i + (int64_t)(next_u64() % (uint64_t)(range - i));
    int64_t t = all[i];
    all[i] = all[j];
    all[j] = t;
    out[i] = all[i];
  }
  free(all);
}

static int failures = 0;

static void check(int ok, const char *what, int layout, int path) {
  if (!ok) {
    if (failures < 20) printf("failure: %s (layout %d, path %d): %s\n", what, layout, path,
                              kv_last_error());
    failures++;
  }
}

int main(void) {
  const int L = 3, C = 2, ps = 16;
  const int64_t R = 272, S_dev = 700, S_host = 640, n = 500;
  const size_t buf_bytes = (size_t)(S_dev * R);
  const int paths[] = {KV_PATH_KERNEL, KV_PATH_KERNEL_LDS, KV_PATH_DMA, KV_PATH_STAGED,
                       KV_PATH_AUTO};
  int64_t *dev_idx = malloc(sizeof(int64_t) * n), *dev2 = malloc(sizeof(int64_t) * n);
  int64_t *host_idx = malloc(sizeof(int64_t) * n);
  void *dev_bufs[2 * 3];
  uint8_t *mirrors[2 * 3];
  uint8_t *readback = malloc(buf_bytes);
  if (hipSetDevice(0) != hipSuccess) {
    printf("no device\n");
    return 2;
  }
  for (int layout = KV_LAYER_FIRST; layout <= KV_PAGE_FIRST_DIRECT; layout++) {
    for (size_t pi = 0; pi < sizeof paths / sizeof paths[0]; pi++) {
      const int path = paths[pi];
      for (int k = 0; k < L * C; k++) {
        mirrors[k] = malloc(buf_bytes);
        random_bytes(mirrors[k], buf_bytes);
        if (hipMalloc(&dev_bufs[k], buf_bytes) != hipSuccess ||
            hipMemcpy(dev_bufs[k], mirrors[k], buf_bytes, hipMemcpyHostToDevice) != hipSuccess) {
          printf("device buffer setup failed\n");
          return 2;
        }
      }
      kv_pool_desc_t desc;
      memset(&desc, 0, sizeof desc);
      desc.geom.num_layers = L;
      desc.geom.num_components = C;
      desc.geom.row_bytes = R;
      desc.geom.device_slots = S_dev;
      desc.geom.host_slots = S_host;
      desc.geom.page_size = ps;
      desc.geom.host_layout = layout;
      desc.device_buffers = dev_bufs;
      desc.device = 0;
      desc.numa_node = -1;
      desc.flags = KV_F_CHECK_UNIQUE;
      kv_pool_t *pool = NULL;
      check(kv_pool_create(&desc, &pool) == KV_OK, "kv_pool_create", layout, path);
      if (!pool) continue;
      check(kv_set_path(pool, path) == KV_OK, "kv_set_path", layout, path);
      const int64_t hbytes = kv_pool_host_bytes(pool);
      uint8_t *host = kv_pool_host_ptr(pool);
      uint8_t *want = malloc((size_t)hbytes);
      memset(host, 0xA5, (size_t)hbytes);
      memset(want, 0xA5, (size_t)hbytes);
      void *s = NULL, *s2 = NULL;
      check(kv_stream_create(0, &s) == KV_OK && kv_stream_create(0, &s2) == KV_OK,
            "kv_stream_create", layout, path);

      /* backup */
      distinct(dev_idx, n, S_dev);
      distinct(host_idx, n, S_host);
      check(kv_backup(pool, dev_idx, host_idx, n, 0, L, s) == KV_OK, "kv_backup", layout, path);
      check(hipStreamSynchronize((hipStream_t)s) == hipSuccess, "sync", layout, path);
      check(kvo_backup(L, C, R, S_dev, S_host, ps, layout, mirrors, want, dev_idx, host_idx, n,
                       0, L, 1) == 0, "oracle backup", layout, path);
      check(memcmp(host, want, (size_t)hbytes) == 0, "host pool after backup", layout, path);

      /* load into other slots, consumer stream gated layer by layer */
      random_bytes(host, (size_t)hbytes);
      memcpy(want, host, (size_t)hbytes);
      distinct(dev2, n, S_dev);
      check(kv_load(pool, dev2, host_idx, n, 0, L, s) == KV_OK, "kv_load", layout, path);
      for (int l = 0; l < L; l++)
        check(kv_load_layer(pool, l, s2) == KV_OK, "kv_load_layer", layout, path);
      check(hipStreamSynchronize((hipStream_t)s2) == hipSuccess &&
            hipStreamSynchronize((hipStream_t)s) == hipSuccess, "sync", layout, path);
      check(kvo_load(L, C, R, S_dev, S_host, ps, layout, mirrors, want, dev2, host_idx, n, 0, L,
                     1) == 0, "oracle load", layout, path);
      for (int k = 0; k < L * C; k++) {
        check(hipMemcpy(readback, dev_bufs[k], buf_bytes, hipMemcpyDeviceToHost) == hipSuccess,
              "readback", layout, path);
        check(memcmp(readback, mirrors[k], buf_bytes) == 0, "device buffer after load", layout,
              path);
      }

      /* a refused request changes nothing and says why */
      host_idx[1] = host_idx[0];
      memcpy(want, host, (size_t)hbytes);
      check(kv_backup(pool, dev_idx, host_idx, n, 0, L, s) == KV_EDUP, "duplicate refused",
            layout, path);
      check(strlen(kv_last_error()) > 0, "error message", layout, path);
      check(hipStreamSynchronize((hipStream_t)s) == hipSuccess &&
            memcmp(host, want, (size_t)hbytes) == 0, "refused call left the pool", layout, path);

      check(kv_stream_destroy(s) == KV_OK && kv_stream_destroy(s2) == KV_OK, "kv_stream_destroy",
            layout, path);
      check(kv_pool_destroy(pool) == KV_OK, "kv_pool_destroy", layout, path);
      free(want);
      for (int k = 0; k < L * C; k++) {
        (void)hipFree(dev_bufs[k]);
        free(mirrors[k]);
      }
    }
  }
  free(dev_idx);
  free(dev2);
  free(host_idx);
  free(readback);
  printf("%d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
