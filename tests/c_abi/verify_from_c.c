/* One tree-verify call from a C99 program, with nothing but the library's
 * header and the HIP runtime's C API: the way a C or C++ serving stack calls
 * the boundary.
 *
 *   verify_from_c DIR
 *
 * DIR/problem.txt holds the tv_problem fields (batch num_heads total_q
 * max_q_len max_kv_len num_slots total_kv total_mask num_splits out_dtype
 * flags) and sm_scale; DIR/q.bin, kv.bin, kv_indices.bin, kv_indptr.bin,
 * qo_indptr.bin, mask.bin and mask_indptr.bin the inputs in the header's
 * layouts.  Every file must hold exactly the bytes the problem implies.  The
 * program copies them to the device, runs tv_check_inputs and tv_verify_attn
 * on a stream of its own with a workspace of tv_workspace_bytes, and writes
 * DIR/out.bin and DIR/lse.bin.  Exit status 0 on success; otherwise it names
 * the step that failed. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "treeverify.h"

static int fail(const char* step, const char* why) {
  printf("FAILED: %s: %s\n", step, why);
  return 1;
}

/* reads DIR/name, which must hold exactly n bytes; a buffer of at least 4 */
static void* read_exact(const char* dir, const char* name, size_t n) {
  char path[4096];
  FILE* f;
  void* buf;
  long sz;
  snprintf(path, sizeof path, "%s/%s", dir, name);
  f = fopen(path, "rb");
  if (!f) return NULL;
  if (fseek(f, 0, SEEK_END) != 0 || (sz = ftell(f)) < 0 || (size_t)sz != n ||
      fseek(f, 0, SEEK_SET) != 0) {
    fclose(f);
    return NULL;
  }
  buf = calloc(n > 4 ? n : 4, 1);
  if (buf && n > 0 && fread(buf, 1, n, f) != n) {
    free(buf);
    buf = NULL;
  }
  fclose(f);
  return buf;
}

static int write_all(const char* dir, const char* name, const void* buf, size_t n) {
  char path[4096];
  FILE* f;
  size_t w;
  snprintf(path, sizeof path, "%s/%s", dir, name);
  f = fopen(path, "wb");
  if (!f) return 0;
  w = fwrite(buf, 1, n, f);
  return fclose(f) == 0 && w == n;
}

enum { IN_Q, IN_KV, IN_KVI, IN_KVP, IN_QOP, IN_MASK, IN_MASKP, N_IN };

int main(int argc, char** argv) {
  static const char* names[N_IN] = {"q.bin",         "kv.bin",   "kv_indices.bin",
                                    "kv_indptr.bin", "qo_indptr.bin", "mask.bin",
                                    "mask_indptr.bin"};
  const char* dir;
  char path[4096];
  FILE* f;
  tv_problem p;
  long long tq, ns, tk, tm;
  float sm_scale;
  size_t bytes[N_IN], out_bytes, lse_bytes, ws_bytes;
  void* host[N_IN] = {0};
  void* dev[N_IN] = {0};
  void *d_out = NULL, *d_ws = NULL, *h_out = NULL;
  float *d_lse = NULL, *h_lse = NULL;
  hipStream_t stream = NULL;
  int32_t bad = -2;
  tv_status st;
  int i, rc = 1;

  if (argc != 2) return fail("arguments", "usage: verify_from_c DIR");
  dir = argv[1];
  memset(&p, 0, sizeof p);
  snprintf(path, sizeof path, "%s/problem.txt", dir);
  f = fopen(path, "r");
  if (!f) return fail("problem.txt", "cannot open");
  if (fscanf(f, "%d %d %lld %d %d %lld %lld %lld %d %d %d %f", &p.batch, &p.num_heads, &tq,
             &p.max_q_len, &p.max_kv_len, &ns, &tk, &tm, &p.num_splits, &p.out_dtype, &p.flags,
             &sm_scale) != 12) {
    fclose(f);
    return fail("problem.txt", "expected 12 numbers");
  }
  fclose(f);
  p.total_q = tq;
  p.num_slots = ns;
  p.total_kv = tk;
  p.total_mask = tm;
  if (p.batch < 1 || p.num_heads < 1 || tq < 0 || ns < 1 || tk < 0 || tm < 0)
    return fail("problem.txt", "sizes out of range");

  bytes[IN_Q] = (size_t)tq * p.num_heads * TV_QK_DIM * 2;
  bytes[IN_KV] = (size_t)ns * TV_QK_DIM * 2;
  bytes[IN_KVI] = (size_t)tk * 4;
  bytes[IN_KVP] = bytes[IN_QOP] = bytes[IN_MASKP] = (size_t)(p.batch + 1) * 4;
  bytes[IN_MASK] = (size_t)tm;
  out_bytes = (size_t)tq * p.num_heads * TV_V_DIM * (p.out_dtype == TV_OUT_F32 ? 4 : 2);
  lse_bytes = (size_t)tq * p.num_heads * 4;

  for (i = 0; i < N_IN; ++i) {
    host[i] = read_exact(dir, names[i], bytes[i]);
    if (!host[i]) {
      fail(names[i], "missing, or not the size the problem implies");
      goto done;
    }
  }
  if (hipSetDevice(0) != hipSuccess) {
    fail("hipSetDevice", "no device");
    goto done;
  }
  for (i = 0; i < N_IN; ++i) {
    /* (a buffer of at least 4 bytes, so that an empty one is still a valid pointer) */
    if (hipMalloc(&dev[i], bytes[i] > 4 ? bytes[i] : 4) != hipSuccess ||
        hipMemcpy(dev[i], host[i], bytes[i] > 4 ? bytes[i] : 4, hipMemcpyHostToDevice) !=
            hipSuccess) {
      fail(names[i], "device allocation or copy");
      goto done;
    }
  }
  if (hipMalloc(&d_out, out_bytes) != hipSuccess ||
      hipMalloc((void**)&d_lse, lse_bytes) != hipSuccess ||
      hipStreamCreate(&stream) != hipSuccess) {
    fail("outputs", "device allocation or stream");
    goto done;
  }
  /* every output byte 0xff beforehand (NaN in either output type): a row the
   * call leaves unwritten shows */
  if (hipMemsetAsync(d_out, 0xff, out_bytes, stream) != hipSuccess ||
      hipMemsetAsync(d_lse, 0xff, lse_bytes, stream) != hipSuccess) {
    fail("outputs", "fill");
    goto done;
  }

  st = tv_check_inputs(&p, (const int32_t*)dev[IN_KVI], (const int32_t*)dev[IN_KVP],
                       (const int32_t*)dev[IN_QOP], (const int32_t*)dev[IN_MASKP], stream, &bad);
  if (st != TV_OK || bad != -1) {
    printf("tv_check_inputs: %s, request %d\n", tv_status_str(st), (int)bad);
    fail("tv_check_inputs", "inputs rejected");
    goto done;
  }
  ws_bytes = tv_workspace_bytes(&p);
  if (ws_bytes > 0 && hipMalloc(&d_ws, ws_bytes) != hipSuccess) {
    fail("workspace", "device allocation");
    goto done;
  }
  st = tv_verify_attn(&p, dev[IN_Q], dev[IN_KV], (const int32_t*)dev[IN_KVI],
                      (const int32_t*)dev[IN_KVP], (const int32_t*)dev[IN_QOP],
                      (const uint8_t*)dev[IN_MASK], (const int32_t*)dev[IN_MASKP], sm_scale,
                      d_out, d_lse, d_ws, ws_bytes, stream);
  if (st != TV_OK) {
    fail("tv_verify_attn", tv_status_str(st));
    goto done;
  }
  h_out = malloc(out_bytes);
  h_lse = (float*)malloc(lse_bytes);
  if (!h_out || !h_lse || hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(h_out, d_out, out_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(h_lse, d_lse, lse_bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    fail("results", "synchronize or copy back");
    goto done;
  }
  if (!write_all(dir, "out.bin", h_out, out_bytes) || !write_all(dir, "lse.bin", h_lse, lse_bytes)) {
    fail("results", "cannot write");
    goto done;
  }
  printf("ok: workspace %lu bytes\n", (unsigned long)ws_bytes);
  rc = 0;

done:
  if (stream) (void)hipStreamDestroy(stream);
  for (i = 0; i < N_IN; ++i) {
    if (dev[i]) (void)hipFree(dev[i]);
    free(host[i]);
  }
  if (d_out) (void)hipFree(d_out);
  if (d_lse) (void)hipFree(d_lse);
  if (d_ws) (void)hipFree(d_ws);
  free(h_out);
  free(h_lse);
  return rc;
}
