/* A plain C consumer of include/pkv.h: compiled as C11 against the header alone and linked against libpkv.so, it
 * exercises the host-only entry points (no device call) -- the version, the dispatcher with an explicit CU count,
 * the workspace size, and argument validation -- and prints one line per check. */
#include <stdio.h>
#include <string.h>

#include "pkv.h"

static int failures = 0;

static void check(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    if (!ok)
        failures++;
}

int main(void) {
    const char *v = pkv_version();
    check(v != NULL && strlen(v) > 0, "pkv_version");

    pkv_decode_plan plan;
    memset(&plan, 0, sizeof plan);
    /* Llama-3-8B-shaped batch on 256 CUs: 32 x 8 tiles fill one round, so a single pass */
    int rc = pkv_plan_decode(32, 32, 8, 128, 16, 128, 2048, 0, 256, &plan);
    check(rc == PKV_OK && plan.num_splits == 1 && plan.workspace_bytes == 0, "plan: one round is a single pass");
    /* four long sequences: splits, and a workspace that holds their partials */
    rc = pkv_plan_decode(4, 32, 8, 128, 16, 2048, 32768, 0, 256, &plan);
    check(rc == PKV_OK && plan.num_splits > 1 &&
              plan.workspace_bytes == pkv_decode_workspace_bytes(4, 32, 128, plan.num_splits),
          "plan: long sequences split, workspace sized");
    check(pkv_decode_workspace_bytes(4, 32, 128, 1) == 0, "no workspace for a single pass");

    /* validation happens before any device work */
    pkv_pool_desc pool = {8, 128, 16, 100};
    rc = pkv_paged_decode_attention(NULL, NULL, NULL, pool, NULL, 128, NULL, 4, 32, 0.1f, NULL, 0, 0, NULL);
    check(rc == PKV_EINVAL && strlen(pkv_last_error()) > 0, "null pointers are PKV_EINVAL with a message");
    pkv_pool_desc odd = {8, 100, 16, 100}; /* head_dim not a multiple of 8 */
    rc = pkv_plan_decode(4, 32, 8, 96, 16, 128, 0, 0, 256, &plan);
    check(rc == PKV_EUNSUPPORTED, "head_dim 96 is PKV_EUNSUPPORTED");
    rc = pkv_paged_kv_append(NULL, NULL, NULL, 1, NULL, NULL, odd, NULL);
    check(rc == PKV_EUNSUPPORTED, "append into head_dim 100 pools is PKV_EUNSUPPORTED");
    rc = pkv_paged_kv_append(NULL, NULL, NULL, -1, NULL, NULL, pool, NULL);
    check(rc == PKV_EINVAL, "a negative token count is PKV_EINVAL");
    return failures == 0 ? 0 : 1;
}
