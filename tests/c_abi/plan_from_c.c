/* A C99 caller of the library's host-side entry points: it uses only
 * include/treeverify.h and links against libtreeverify.so, the way a C or C++
 * serving stack would.  No kernel is launched and no device memory is touched.
 *
 *   plan_from_c B H total_q max_q_len max_kv_len num_slots total_kv total_mask
 *               num_splits out_dtype flags
 *       prints "status split_keys max_splits row_blocks merge workspace_bytes
 *       tv_workspace_bytes" for that problem
 *   plan_from_c layout
 *       prints "name offset size" for every field of tv_problem, tv_plan and
 *       tv_append_problem, and each struct's size, as this compiler lays them out
 *   plan_from_c errors
 *       checks the argument errors of every entry point that validates on the
 *       host; prints "ok" and exits 0, or names the first failed check and
 *       exits 1
 */
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "treeverify.h"

static int fail(const char* what) {
  printf("FAILED: %s\n", what);
  return 1;
}

static tv_problem live_shape(void) {
  tv_problem p;
  memset(&p, 0, sizeof p);
  p.batch = 1;
  p.num_heads = 8;
  p.total_q = 9;
  p.max_q_len = 9;
  p.max_kv_len = 30;
  p.num_slots = 4096;
  p.total_kv = 30;
  p.total_mask = 270;
  p.out_dtype = TV_OUT_BF16;
  return p;
}

static int errors(void) {
  tv_plan pl;
  tv_problem p = live_shape();
  int s;
  int32_t bad = -7;
  if (tv_get_plan(NULL, &pl) != TV_ERR_NULL) return fail("tv_get_plan(NULL, plan)");
  if (tv_get_plan(&p, NULL) != TV_ERR_NULL) return fail("tv_get_plan(p, NULL)");
  if (tv_get_plan(&p, &pl) != TV_OK || pl.max_splits != 1 || pl.merge != 0)
    return fail("tv_get_plan(live shape)");
  p.num_heads = 0;
  if (tv_get_plan(&p, &pl) != TV_ERR_SHAPE) return fail("num_heads = 0");
  if (tv_workspace_bytes(&p) != 0) return fail("tv_workspace_bytes(invalid)");
  p = live_shape();
  p.flags = 64;
  if (tv_get_plan(&p, &pl) != TV_ERR_UNSUPPORTED) return fail("unknown flag bit");
  p = live_shape();
  p.out_dtype = 7;
  if (tv_get_plan(&p, &pl) != TV_ERR_UNSUPPORTED) return fail("unknown out_dtype");
  p = live_shape();
  p.reserved = 1;
  if (tv_get_plan(&p, &pl) != TV_ERR_UNSUPPORTED) return fail("reserved != 0");
  p = live_shape();
  if (tv_workspace_bytes(NULL) != 0) return fail("tv_workspace_bytes(NULL)");
  /* the compute entry points reject bad arguments before they touch the
   * runtime: the addresses below are never dereferenced */
  if (tv_verify_attn(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1.0f, NULL, NULL, NULL, 0,
                     NULL) != TV_ERR_NULL)
    return fail("tv_verify_attn(NULL problem)");
  if (tv_verify_attn(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1.0f, NULL, NULL, NULL, 0,
                     NULL) != TV_ERR_NULL)
    return fail("tv_verify_attn(NULL buffers)");
  {
    void* a = (void*)(uintptr_t)0x100000; /* aligned, never read */
    float* f = (float*)a;
    const int32_t* i = (const int32_t*)a;
    const uint8_t* m = (const uint8_t*)a;
    tv_problem c3 = live_shape(); /* one request, 32 drafts, 32k prefix, 16 heads */
    c3.num_heads = 16;
    c3.total_q = 32;
    c3.max_q_len = 32;
    c3.max_kv_len = 32800;
    c3.num_slots = 200000;
    c3.total_kv = 32800;
    c3.total_mask = 32 * 32800;
    if (tv_verify_attn(&p, a, a, i, i, i, m, i, 0.0f, a, f, NULL, 0, NULL) != TV_ERR_SHAPE)
      return fail("sm_scale = 0");
    if (tv_verify_attn(&p, (char*)a + 4, a, i, i, i, m, i, 1.0f, a, f, NULL, 0, NULL) !=
        TV_ERR_SHAPE)
      return fail("q not 16-byte aligned");
    if (tv_workspace_bytes(&c3) == 0) return fail("tv_workspace_bytes(C3 shape)");
    if (tv_verify_attn(&c3, a, a, i, i, i, m, i, 1.0f, a, f, NULL, 0, NULL) != TV_ERR_WORKSPACE)
      return fail("no workspace where one is needed");
    if (tv_verify_attn(&c3, a, a, i, i, i, m, i, 1.0f, a, f, a, tv_workspace_bytes(&c3) - 256,
                       NULL) != TV_ERR_WORKSPACE)
      return fail("workspace too small");
  }
  s = tv_check_inputs(NULL, NULL, NULL, NULL, NULL, NULL, &bad);
  if (s != TV_ERR_NULL) return fail("tv_check_inputs(NULL problem)");
  for (s = TV_OK; s <= TV_ERR_HIP; ++s) {
    const char* t = tv_status_str((tv_status)s);
    if (t == NULL || t[0] == '\0' || strcmp(t, "unknown status") == 0)
      return fail("tv_status_str of a defined status");
  }
  if (strcmp(tv_status_str((tv_status)99), "unknown status") != 0)
    return fail("tv_status_str(99)");
  printf("ok\n");
  return 0;
}

#define TV_FIELD(T, f) printf(#T "." #f " %u %u\n", (unsigned)offsetof(T, f), (unsigned)sizeof(((T*)0)->f))

static int layout(void) {
  TV_FIELD(tv_problem, batch);
  TV_FIELD(tv_problem, num_heads);
  TV_FIELD(tv_problem, total_q);
  TV_FIELD(tv_problem, max_q_len);
  TV_FIELD(tv_problem, max_kv_len);
  TV_FIELD(tv_problem, num_slots);
  TV_FIELD(tv_problem, total_kv);
  TV_FIELD(tv_problem, total_mask);
  TV_FIELD(tv_problem, num_splits);
  TV_FIELD(tv_problem, out_dtype);
  TV_FIELD(tv_problem, flags);
  TV_FIELD(tv_problem, reserved);
  printf("tv_problem %u\n", (unsigned)sizeof(tv_problem));
  TV_FIELD(tv_plan, split_keys);
  TV_FIELD(tv_plan, max_splits);
  TV_FIELD(tv_plan, row_blocks);
  TV_FIELD(tv_plan, merge);
  TV_FIELD(tv_plan, workspace_bytes);
  printf("tv_plan %u\n", (unsigned)sizeof(tv_plan));
  TV_FIELD(tv_append_problem, batch);
  TV_FIELD(tv_append_problem, max_q_len);
  TV_FIELD(tv_append_problem, max_kv_len);
  TV_FIELD(tv_append_problem, flags);
  TV_FIELD(tv_append_problem, total_q);
  TV_FIELD(tv_append_problem, num_slots);
  TV_FIELD(tv_append_problem, total_prefix);
  TV_FIELD(tv_append_problem, total_kv);
  TV_FIELD(tv_append_problem, total_mask);
  printf("tv_append_problem %u\n", (unsigned)sizeof(tv_append_problem));
  return 0;
}

int main(int argc, char** argv) {
  tv_problem p;
  tv_plan pl;
  tv_status s;
  if (argc == 2 && strcmp(argv[1], "errors") == 0) return errors();
  if (argc == 2 && strcmp(argv[1], "layout") == 0) return layout();
  if (argc != 12) {
    fprintf(stderr, "usage: see the header comment of plan_from_c.c\n");
    return 2;
  }
  memset(&p, 0, sizeof p);
  p.batch = atoi(argv[1]);
  p.num_heads = atoi(argv[2]);
  p.total_q = atoll(argv[3]);
  p.max_q_len = atoi(argv[4]);
  p.max_kv_len = atoi(argv[5]);
  p.num_slots = atoll(argv[6]);
  p.total_kv = atoll(argv[7]);
  p.total_mask = atoll(argv[8]);
  p.num_splits = atoi(argv[9]);
  p.out_dtype = atoi(argv[10]);
  p.flags = atoi(argv[11]);
  memset(&pl, 0, sizeof pl);
  s = tv_get_plan(&p, &pl);
  printf("%d %d %d %d %d %lld %llu\n", (int)s, pl.split_keys, pl.max_splits, pl.row_blocks,
         pl.merge, (long long)pl.workspace_bytes, (unsigned long long)tv_workspace_bytes(&p));
  return 0;
}
