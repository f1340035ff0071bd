/*
 * The C ABI used from plain C99, with no device work (runs on a machine
 * without a GPU).  Built and run by tests/test_c_abi.py.
 *
 * stdin: planner cases, one per line:
 *   num_tokens tokens_per_cta ctas_per_token_tile num_cus ctas_per_cu min_split_tokens
 * stdout: one line per case,
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
  long long T, tpc, tiles, thr;
  int cus, occ;
  char line[256];

  if (tw_abi_version() != TW_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", (int)tw_abi_version(), TW_ABI_VERSION);
    return 1;
  }
  while (fgets(line, sizeof line, stdin) != NULL) {
    tw_split_problem p;
    tw_split_plan_result r;
    tw_status s;
    if (sscanf(line, "%lld %lld %lld %d %d %lld", &T, &tpc, &tiles, &cus, &occ, &thr) != 6) continue;
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
