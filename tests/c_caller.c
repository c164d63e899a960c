/* A plain C99 caller of libgdn.so: the host-side calls of the C ABI (no device work), printed one per
 * line for tests/test_c_caller.py. Built with gcc against include/gdn.h only. */
#include <stdio.h>
#include <string.h>

#include "gdn.h"

static gdn_desc layer(int n_k, int n_v, int d_k, int d_v) {
  gdn_desc d;
  memset(&d, 0, sizeof d);
  d.n_k = n_k;
  d.n_v = n_v;
  d.d_k = d_k;
  d.d_v = d_v;
  d.conv_k = 4;
  d.act_dtype = GDN_BF16;
  d.l2_eps = 1e-6f;
  d.rms_eps = 1e-6f;
  d.out_dtype = GDN_OUT_ACT;
  return d;
}

int main(void) {
  gdn_desc d = layer(16, 32, 128, 128);
  printf("version %s\n", gdn_version());
  printf("record %zu\n", gdn_state_record_bytes(&d));
  printf("workspace %zu\n", gdn_prefill_workspace_bytes(&d, 1, 4096));
  /* a NULL argument is rejected before any device work */
  int rc = gdn_decode_step(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL);
  printf("decode_null %d %s\n", rc, gdn_last_error());
  /* head dims outside {32, 64, 128} are reported as unsupported */
  gdn_desc bad = layer(2, 4, 48, 48);
  rc = gdn_conv_chunk(&bad, NULL, NULL, NULL, NULL, NULL, 1, 1, NULL);
  printf("conv_unsupported %d %s\n", rc, gdn_last_error());
  /* key and value heads of different dims are built: the workspace of the zero-padded call */
  gdn_desc mixed = layer(2, 4, 64, 128);
  printf("workspace_unequal %zu\n", gdn_prefill_workspace_bytes(&mixed, 2, 300));
  /* the prefix-state cache planner is host code: create, plan an empty row, read the counters */
  gdn_pcache* cache = NULL;
  rc = gdn_pcache_create(8, 2048, 16, 64, 2048, 0, &cache);
  int32_t info[4] = {0, 0, 0, 0};
  int rc2 = rc == 0 ? gdn_pcache_row(cache, NULL, 0, 0, 0, info, NULL, NULL, NULL) : -99;
  int64_t stats[GDN_PCACHE_NSTATS];
  memset(stats, 0, sizeof stats);
  int rc3 = rc == 0 ? gdn_pcache_stats(cache, stats) : -99;
  printf("pcache %d %d %d plain=%lld\n", rc, rc2, rc3, (long long)stats[GDN_PCACHE_PLAIN]);
  if (cache) gdn_pcache_destroy(cache);
  return 0;
}
