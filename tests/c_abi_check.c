/* Plain C99 user of include/sigattn.h: compiles the header as C, links
 * libsigattn, and exercises the host-only calls (no GPU needed): status
 * strings, tile shapes, the schedule statistics and argument validation with
 * fake, never-dereferenced device addresses.  Prints one line per check and
 * returns the number of failed checks. */
#include <stdint.h>
#include <stdio.h>

#include "sigattn.h"

static int fails = 0;
static void check(int ok, const char *what) {
  printf("%s %s\n", ok ? "ok" : "FAIL", what);
  if (!ok) ++fails;
}

int main(void) {
  const int32_t lens[3] = {300, 1, 0};
  sigattn_args a = {0};
  a.B = 3;
  a.H = 2;
  a.Lmax = 300;
  a.d = 64;
  a.seqlens = lens;
  a.bias_mode = SIGATTN_BIAS_NEG_LOG_SEQLEN;
  a.precision = SIGATTN_PREC_FAST;
  a.mask = SIGATTN_MASK_NONE;
  a.dtype = SIGATTN_DTYPE_BF16;

  int64_t items = -1, pairs = -1;
  int32_t launches = -1;
  check(sigattn_plan_stats(&a, SIGATTN_PASS_FWD, &items, &pairs, &launches) == SIGATTN_OK, "plan_stats ok");
  /* closed forms: 300 rows -> 3 query tiles x 5 key tiles; 1 row -> 1 x 1 */
  check(items == 2 * (3 + 1) && pairs == 2 * (3 * 5 + 1 * 1), "plan_stats closed form");
  int32_t outer = 0, inner = 0;
  check(sigattn_tile_shape(SIGATTN_PASS_BWD_DKDV, 64, &outer, &inner) == SIGATTN_OK && outer == 128 && inner == 64,
        "tile_shape");
  check(sigattn_status_str(SIGATTN_ERR_ALIAS) != 0 && sigattn_status_str((sigattn_status)999) != 0, "status_str");

  const uintptr_t base = (uintptr_t)1 << 44, gap = (uintptr_t)1 << 36;
  const void *t[6];
  for (int i = 0; i < 6; ++i) t[i] = (const void *)(base + i * gap);
  check(sigattn_validate(&a, SIGATTN_PASS_BWD_DKDV, t) == SIGATTN_OK, "validate ok");
  t[5] = t[4];
  check(sigattn_validate(&a, SIGATTN_PASS_BWD_DKDV, t) == SIGATTN_ERR_ALIAS, "validate alias");
  a.d = 96;
  check(sigattn_validate(&a, SIGATTN_PASS_FWD, t) == SIGATTN_ERR_SHAPE, "validate shape");
  a.d = 64;
  a.dtype = 7;
  check(sigattn_fwd(&a, t[0], t[1], t[2], (void *)t[3]) == SIGATTN_ERR_DTYPE, "fwd rejects dtype before launch");
  return fails;
}
