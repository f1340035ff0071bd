/*
 * The C ABI used from plain C99, with no device work (runs on a machine
 * without a GPU).  Built and run by tests/test_c_abi.py.
 *
 * stdin: planner cases, one per line:
 *   num_tokens tokens_per_cta ctas_per_token_tile num_cus ctas_per_cu min_split_tokens
 *   table_tokens table_offset
 * stdout: one line per case, the analytic plan and then the plan with a
 * one-entry measured table {table_tokens: table_offset}, each as
 *   status prefix suffix offset waves_unsplit waves_prefix waves_suffix reason
 * then the results of the argument checks below, one "name status" line each,
 * and "done" last.  Exit status 0 unless a check of this program's own fails.
 */
#include <stdio.h>
#include <string.h>

#include "tokenweave.h"

static int report(const char* name, tw_status s) {
  printf("%s %d\n", name, (int)s);
  if (s != TW_OK && tw_last_error()[0] == '\0') {
    fprintf(stderr, "%s: status %d without detail\n", name, (int)s);
    return 1;
  }
  return 0;
}

int main(void) {
  int fail = 0;
  long long T, tpc, tiles, thr, tab_t;
  int cus, occ, tab_off;
  char line[256];

  if (tw_abi_version() != TW_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", (int)tw_abi_version(), TW_ABI_VERSION);
    return 1;
  }
  while (fgets(line, sizeof line, stdin) != NULL) {
    tw_split_problem p;
    tw_split_plan_result r;
    tw_status s;
    tw_split_entry e;
    if (sscanf(line, "%lld %lld %lld %d %d %lld %lld %d", &T, &tpc, &tiles, &cus, &occ, &thr,
               &tab_t, &tab_off) != 8)
      continue;
    memset(&p, 0, sizeof p);
    p.num_tokens = T;
    p.tokens_per_cta = tpc;
    p.ctas_per_token_tile = tiles;
    p.num_cus = cus;
    p.ctas_per_cu = occ;
    p.min_split_tokens = thr;
    p.offsets = NULL; /* the default offset set */
    p.num_offsets = 0;
    s = tw_split_plan(&p, &r);
    printf("%d %lld %lld %d %d %d %d %d ", (int)s, (long long)r.prefix_tokens,
           (long long)r.suffix_tokens, (int)r.offset, (int)r.waves_unsplit, (int)r.waves_prefix,
           (int)r.waves_suffix, (int)r.reason);
    e.num_tokens = tab_t;
    e.offset = tab_off;
    s = tw_split_plan_measured(&p, &e, 1, &r);
    printf("%d %lld %lld %d %d %d %d %d\n", (int)s, (long long)r.prefix_tokens,
           (long long)r.suffix_tokens, (int)r.offset, (int)r.waves_unsplit, (int)r.waves_prefix,
           (int)r.waves_suffix, (int)r.reason);
  }

  {
    /* Argument checks that fail before any device call.  The pointers are
     * never dereferenced: validation rejects each call first. */
    static unsigned char buf[6][4096] __attribute__((aligned(16)));
    const void* parts[2] = {buf[0], buf[1]};
    tw_split_problem p;
    tw_split_plan_result r;
    fail |= report("null_partials",
                   tw_fused_reduce_rmsnorm(NULL, 2, buf[2], buf[3], buf[4], buf[5], 4, 64, 1e-5f,
                                           TW_BF16, NULL));
    fail |= report("hidden_not_16_bytes",
                   tw_fused_reduce_rmsnorm(parts, 2, buf[2], buf[3], buf[4], buf[5], 4, 12, 1e-5f,
                                           TW_BF16, NULL));
    fail |= report("negative_eps",
                   tw_fused_reduce_rmsnorm(parts, 2, buf[2], buf[3], buf[4], buf[5], 4, 64, -1.0f,
                                           TW_BF16, NULL));
    fail |= report("shard_index_out_of_range",
                   tw_shard_rmsnorm(parts, 2, buf[2], buf[3], buf[4], buf[5], 4, 64, 1e-5f,
                                    TW_BF16, 2, NULL));
    fail |= report("out_overlaps_partial",
                   tw_fused_reduce_rmsnorm(parts, 2, buf[2], buf[3], buf[0], buf[5], 4, 64, 1e-5f,
                                           TW_BF16, NULL));
    fail |= report("empty_batch",
                   tw_fused_reduce_rmsnorm(parts, 2, buf[2], buf[3], buf[4], buf[5], 0, 64, 1e-5f,
                                           TW_BF16, NULL));
    fail |= report("plan_null_problem", tw_split_plan(NULL, &r));
    memset(&p, 0, sizeof p);
    p.num_tokens = 100;
    p.tokens_per_cta = 0;
    p.ctas_per_token_tile = 1;
    p.num_cus = 256;
    p.ctas_per_cu = 1;
    fail |= report("plan_zero_tile", tw_split_plan(&p, &r));
    {
      tw_split_entry t[2];
      p.tokens_per_cta = 1;
      t[0].num_tokens = 200;
      t[0].offset = 0;
      t[1].num_tokens = 100;
      t[1].offset = 0;
      fail |= report("plan_table_not_ascending", tw_split_plan_measured(&p, t, 2, &r));
      t[0].num_tokens = 100;
      t[0].offset = 50;
      fail |= report("plan_table_offset_at_half", tw_split_plan_measured(&p, t, 1, &r));
      fail |= report("plan_table_null", tw_split_plan_measured(&p, NULL, 1, &r));
    }
  }
  {
    /* Randomized argument sets, each invalid by construction (an output
     * starting exactly at another tensor, a misaligned pointer, or a bad
     * scalar), so that argument validation must refuse every call.  As a
     * second guard the pointer checks are on for the loop: a call that got
     * past validation would be refused as unknown memory, never launched.
     * The fake addresses are never dereferenced.  Exercises the validation
     * code under the sanitizers this program may be built with. */
    unsigned long long st = 88172645463325252ULL;
    int it, refused = 0;
    tw_set_pointer_checks(1);
    for (it = 0; it < 2000; ++it) {
      const void* parts[16];
      unsigned long long base = 0x7f0000000000ULL, r;
      long long T, h;
      int n, i, kind, victim;
      size_t row;
      const unsigned char* p[5];
      tw_status s;
#define NEXT() (st ^= st << 13, st ^= st >> 7, st ^= st << 17, st)
      r = NEXT();
      n = 1 + (int)(r % 16);
      T = 1 + (long long)((r >> 8) % 64);
      h = 8 * (1 + (long long)((r >> 16) % 32));
      row = (size_t)(T * h * 2);
      for (i = 0; i < n; ++i) parts[i] = (const void*)(base + (unsigned long long)i * (row + 4096));
      for (i = 0; i < 4; ++i) p[i] = (const unsigned char*)(base + (unsigned long long)(n + i) * (row + 4096));
      p[4] = p[0];
      kind = (int)((r >> 24) % 4);
      victim = (int)((r >> 32) % (unsigned long long)(n + 2));
      if (kind == 0) {          /* out starts at an input */
        p[2] = victim < n ? (const unsigned char*)parts[victim] : p[victim - n];
      } else if (kind == 1) {   /* residual_out starts at a partial or the weight */
        p[3] = victim < n ? (const unsigned char*)parts[victim] : p[1];
      } else if (kind == 2) {   /* misaligned output */
        p[2] = p[2] + 8;
      } else {                  /* a bad scalar */
        h = (r >> 40) % 2 ? h + 1 : h;
        if (h % 8 == 0) T = -T;
      }
      s = tw_fused_reduce_rmsnorm(parts, n, p[0], p[1], (void*)p[2], (void*)p[3], T, h, 1e-5f,
                                  TW_BF16, NULL);
      if (s != TW_OK && tw_last_error()[0] != '\0' && strstr(tw_last_error(), "memory") == NULL &&
          strstr(tw_last_error(), "allocation") == NULL)
        ++refused;
      else {
        fprintf(stderr, "case %d (kind %d) not refused by validation: status %d (%s)\n", it, kind,
                (int)s, tw_last_error());
        fail = 1;
        break;
      }
#undef NEXT
    }
    tw_set_pointer_checks(0);
    printf("randomized_refused %d\n", refused == 2000 ? 0 : 1);
  }
  {
    int k;
    for (k = 0; k <= 3; ++k)
      if (tw_status_string((tw_status)k) == NULL || tw_status_string((tw_status)k)[0] == '\0') {
        fprintf(stderr, "no text for status %d\n", k);
        fail = 1;
      }
  }
  printf("done\n");
  return fail;
}
