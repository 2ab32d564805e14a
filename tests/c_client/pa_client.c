/* pa_client.c: a plain C99 client of the library's host-side ABI.
 *
 * It includes include/pa.h as C, links libpa.so, and drives the calls that
 * need no GPU: version and error strings, pool and workspace sizes, and a
 * block manager with prefix caching, fork, copy-on-write, a refused and an
 * accepted swap, and frees.  Every result is printed as "name v1 v2 ..." so
 * that the test can compare the run with the block-manager oracle.  Exit
 * status 0 unless a call fails in a way the scenario does not expect. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pa.h"

static void print_i64(const char* name, const int64_t* v, int n) {
  int i;
  printf("%s", name);
  for (i = 0; i < n; ++i) printf(" %lld", (long long)v[i]);
  printf("\n");
}

static int check(int32_t rc, const char* what) {
  if (rc != PA_OK) {
    fprintf(stderr, "%s: %s (%s)\n", what, pa_strerror(rc), pa_last_error());
    return 1;
  }
  return 0;
}

int main(void) {
  int32_t prompt1[10], prompt2[9], toks[2], rc, ncached = 0, ncow = 0, npairs = 0, i;
  int64_t slots[16], cow[8], pairs[32], ids[3] = {1, 2, 3}, app[2] = {1, 3};
  int32_t tables[3 * 8], lens[3];
  uint64_t h;
  pa_block_manager* bm;

  printf("version %d\n", (int)pa_version());
  printf("strerror_invalid %s\n", pa_strerror(PA_ERR_INVALID));
  printf("pool_bytes %llu\n", (unsigned long long)pa_pool_bytes(10, 8, 16, 128, PA_BF16));

  for (i = 0; i < 10; ++i) prompt1[i] = 1000 + i;
  for (i = 0; i < 9; ++i) prompt2[i] = i < 8 ? 1000 + i : 77;
  h = pa_bm_block_hash(0, prompt1, 4, 7);
  printf("block_hash %llu\n", (unsigned long long)h);

  bm = pa_bm_create_swap(32, 16, 4);
  if (!bm) return 1;
  if (check(pa_bm_enable_prefix_caching(bm), "enable_prefix_caching")) return 1;

  if (check(pa_bm_add_prompt(bm, 1, prompt1, 10, 7, slots, &ncached), "add_prompt 1")) return 1;
  print_i64("prompt1_slots", slots, 10);
  printf("prompt1_cached %d\n", (int)ncached);
  if (check(pa_bm_add_prompt(bm, 2, prompt2, 9, 7, slots, &ncached), "add_prompt 2")) return 1;
  print_i64("prompt2_slots", slots, 9);
  printf("prompt2_cached %d\n", (int)ncached);

  if (check(pa_bm_fork(bm, 1, 3), "fork")) return 1;
  toks[0] = 100;
  toks[1] = 101;
  if (check(pa_bm_append_tokens(bm, 2, app, toks, slots, cow, &ncow), "append_tokens")) return 1;
  print_i64("append_slots", slots, 2);
  print_i64("append_cow", cow, 2 * ncow);

  if (check(pa_bm_block_tables(bm, 3, ids, 8, tables, lens), "block_tables")) return 1;
  for (i = 0; i < 3; ++i) {
    int64_t row[8];
    int j;
    for (j = 0; j < 8; ++j) row[j] = tables[i * 8 + j];
    printf("len%d %d\n", i + 1, (int)lens[i]);
    print_i64(i == 0 ? "table1" : i == 1 ? "table2" : "table3", row, 8);
  }
  printf("num_free %d\n", (int)pa_bm_num_free(bm));
  printf("num_cached %d\n", (int)pa_bm_num_cached_blocks(bm));

  /* Sequence 2 shares its cached prefix with 1 and 3: alone it cannot move. */
  rc = pa_bm_swap_out(bm, 1, ids + 1, pairs, 16, &npairs);
  printf("swap_out_2 %d\n", (int)rc);
  if (check(pa_bm_swap_out(bm, 3, ids, pairs, 16, &npairs), "swap_out all")) return 1;
  print_i64("swap_out_pairs", pairs, 2 * npairs);
  printf("num_free_host %d\n", (int)pa_bm_num_free_host(bm));
  printf("is_swapped_3 %d\n", (int)pa_bm_is_swapped(bm, 3));
  if (check(pa_bm_swap_in(bm, 3, ids, pairs, 16, &npairs), "swap_in all")) return 1;
  print_i64("swap_in_pairs", pairs, 2 * npairs);

  for (i = 0; i < 3; ++i)
    if (check(pa_bm_free(bm, ids[i]), "free")) return 1;
  printf("num_free_end %d\n", (int)pa_bm_num_free(bm));
  printf("num_cached_end %d\n", (int)pa_bm_num_cached_blocks(bm));
  pa_bm_destroy(bm);
  return 0;
}
