/* Host paths of libpkv under AddressSanitizer and UndefinedBehaviorSanitizer: the dispatcher over a grid of shapes
 * (every plan it returns is checked for its own rules and its workspace size against pkv_decode_workspace_bytes),
 * the workspace size at extreme shapes, and every argument error an entry point must report before it enqueues
 * anything.  Linked against the host-only build whose kernel launchers are stubs that count their calls
 * (pkv_test_stub_launches): none may be called.  Prints one line per check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pkv.h"

int pkv_test_stub_launches(void);

static int failures = 0;
static void check(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    if (!ok)
        failures++;
}

/* 16-byte aligned stand-ins for device pointers: the host paths check and pass them on but never dereference
 * them, and every call below fails before a launch. */
static uint16_t h16[64] __attribute__((aligned(256)));
static int32_t h32[64] __attribute__((aligned(256)));
static float hf[64] __attribute__((aligned(256)));

int main(void) {
    /* the dispatcher over a grid of shapes */
    static const int32_t Bs[] = {1, 2, 7, 32, 255, 256, 2048, 16384, 100000};
    static const int32_t heads[][2] = {{32, 8}, {64, 8}, {16, 16}, {4, 1}, {8, 2}, {32, 1}, {6, 4}};
    static const int32_t Ds[] = {64, 96, 128, 256};
    static const int32_t BSs[] = {16, 32, 48, 64};
    static const int32_t Ms[] = {1, 8, 128, 2048};
    static const int32_t hints[] = {0, 1, 100, 32768};
    static const int32_t splits[] = {0, 1, 2, 7, 64};
    static const int32_t cus[] = {1, 80, 256, 304};
    long plans = 0, bad = 0, refused = 0;
    for (size_t b = 0; b < sizeof Bs / sizeof *Bs; ++b)
        for (size_t h = 0; h < sizeof heads / sizeof *heads; ++h)
            for (size_t d = 0; d < sizeof Ds / sizeof *Ds; ++d)
                for (size_t bs = 0; bs < sizeof BSs / sizeof *BSs; ++bs)
                    for (size_t m = 0; m < sizeof Ms / sizeof *Ms; ++m)
                        for (size_t x = 0; x < sizeof hints / sizeof *hints; ++x)
                            for (size_t s = 0; s < sizeof splits / sizeof *splits; ++s)
                                for (size_t c = 0; c < sizeof cus / sizeof *cus; ++c) {
                                    pkv_decode_plan p;
                                    memset(&p, 0x5A, sizeof p);
                                    const int rc = pkv_plan_decode(Bs[b], heads[h][0], heads[h][1], Ds[d], BSs[bs],
                                                                   Ms[m], hints[x], splits[s], cus[c], &p);
                                    if (rc != PKV_OK) {
                                        refused += rc == PKV_EUNSUPPORTED || rc == PKV_EINVAL;
                                        bad += !(rc == PKV_EUNSUPPORTED || rc == PKV_EINVAL);
                                        continue;
                                    }
                                    ++plans;
                                    const int w = p.waves_per_group;
                                    const int ok = p.num_splits >= 1 && p.num_splits <= 65535 &&
                                                   p.chunk_blocks >= 0 && (w == 1 || w == 2 || w == 4 || w == 8) &&
                                                   (Ds[d] < 256 || w <= 4) &&
                                                   (splits[s] == 0 || p.num_splits == splits[s]) &&
                                                   p.workspace_bytes == pkv_decode_workspace_bytes(
                                                                            Bs[b], heads[h][0], Ds[d], p.num_splits);
                                    bad += !ok;
                                }
    printf("# %ld plans, %ld refused\n", plans, refused);
    check(bad == 0 && plans > 0 && refused > 0, "every plan keeps its rules; refusals are EINVAL or EUNSUPPORTED");

    check(pkv_decode_workspace_bytes(1, 1, 64, 1) == 0 && pkv_decode_workspace_bytes(0, 32, 128, 8) <= 3 * 256 &&
              pkv_decode_workspace_bytes(16384, 64, 256, 64) >= (size_t)16384 * 64 * 64 * 256 * 4,
          "workspace bytes at the extremes");

    pkv_decode_plan plan;
    check(pkv_plan_decode(32, 32, 8, 128, 16, 128, 0, 0, 256, NULL) == PKV_EINVAL, "plan: NULL output");
    check(pkv_plan_decode(-1, 32, 8, 128, 16, 128, 0, 0, 256, &plan) == PKV_EINVAL, "plan: negative batch");
    check(pkv_plan_decode(32, 30, 8, 128, 16, 128, 0, 0, 256, &plan) == PKV_EINVAL, "plan: Hq % Hkv != 0");
    check(pkv_plan_decode(32, 32, 8, 128, 16, -4, 0, 0, 256, &plan) == PKV_EINVAL, "plan: negative table width");

    pkv_pool_desc pool = {8, 128, 16, 64}, odd = {8, 100, 16, 64}, wide = {8, 512, 16, 64}, bs8 = {8, 128, 8, 64};
    pkv_pool_desc d40 = {8, 40, 16, 64};
    /* append */
    check(pkv_paged_kv_append(h16, h16, h32, -1, h16, h16, pool, NULL) == PKV_EINVAL, "append: negative tokens");
    check(pkv_paged_kv_append(h16, h16, h32, 0, h16, h16, pool, NULL) == PKV_OK, "append: zero tokens is a no-op");
    check(pkv_paged_kv_append(NULL, h16, h32, 4, h16, h16, pool, NULL) == PKV_EINVAL, "append: NULL k");
    check(pkv_paged_kv_append(h16, h16, h32, 4, h16, h16, odd, NULL) == PKV_EUNSUPPORTED, "append: head_dim 100");
    check(pkv_paged_kv_append(h16, h16, h32, 4, h16, h16, d40, NULL) == PKV_EUNSUPPORTED, "append: head_dim 40");
    check(pkv_paged_kv_append(h16, h16, h32, 4, h16, h16, bs8, NULL) == PKV_EUNSUPPORTED, "append: block_size 8");
    check(pkv_paged_kv_append(h16 + 1, h16, h32, 4, h16, h16, pool, NULL) == PKV_EINVAL, "append: misaligned k");
    /* attention and its variants */
    check(pkv_paged_decode_attention(h16, h16, h16, pool, h32, 8, h32, 0, 32, 0.1f, h16, 0, 0, NULL) == PKV_OK,
          "attention: zero sequences is a no-op");
    check(pkv_paged_decode_attention(NULL, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, 0, 0, NULL) == PKV_EINVAL,
          "attention: NULL q");
    check(pkv_paged_decode_attention(h16, h16, h16, pool, h32, 8, h32, 4, 30, 0.1f, h16, 0, 0, NULL) == PKV_EINVAL,
          "attention: Hq % Hkv != 0");
    check(pkv_paged_decode_attention(h16, h16, h16, odd, h32, 8, h32, 4, 32, 0.1f, h16, 0, 0, NULL) ==
              PKV_EUNSUPPORTED, "attention: head_dim 100");
    check(pkv_paged_decode_attention(h16, h16, h16, wide, h32, 8, h32, 4, 32, 0.1f, h16, 0, 0, NULL) ==
              PKV_EUNSUPPORTED, "attention: head_dim 512");
    check(pkv_paged_decode_attention(h16, h16, h16, pool, h32, 8, h32, 4, 256, 0.1f, h16, 0, 0, NULL) ==
              PKV_EUNSUPPORTED, "attention: group of 32");
    check(pkv_paged_decode_attention(h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, -2, 0, NULL) == PKV_EINVAL,
          "attention: negative split count");
    check(pkv_paged_decode_attention_ws(h16, h16, h16, pool, h32, 8, h32, -1, 32, 0.1f, h16, 0, 0, NULL, 0, NULL) ==
              PKV_EINVAL, "attention (caller workspace): negative batch");
    check(pkv_paged_decode_attention_noalloc(h16, h16, NULL, pool, h32, 8, h32, 4, 32, 0.1f, h16, 0, 0, NULL) ==
              PKV_EINVAL, "attention (no allocation): NULL v_pool");
    check(pkv_paged_decode_attention_window(h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, 0, -5, 0, NULL) ==
              PKV_EINVAL, "windowed attention: negative window");
    pkv_decode_plan bad_plan = {0, 0, 8, 0, 0};
    check(pkv_paged_decode_attention_planned(h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, &bad_plan, NULL, 0,
                                             NULL) == PKV_EINVAL, "planned attention: zero splits");
    pkv_decode_plan bad_waves = {1, 0, 3, 0, 0};
    check(pkv_paged_decode_attention_planned(h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, &bad_waves, NULL,
                                             0, NULL) == PKV_EINVAL, "planned attention: three waves");
    pkv_decode_plan short_chunks = {2, 1, 8, 0, 0};
    check(pkv_paged_decode_attention_planned(h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, &short_chunks, NULL,
                                             0, NULL) == PKV_EINVAL, "planned attention: chunks cover too few blocks");
    check(pkv_paged_decode_attention_planned(h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, NULL, NULL, 0,
                                             NULL) == PKV_EINVAL, "planned attention: NULL plan");
    /* steps */
    check(pkv_paged_decode_step(h16, NULL, h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, 0, 0, NULL) ==
              PKV_EINVAL, "decode step: NULL k_new");
    check(pkv_paged_decode_step_window(h16, h16, h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, h16, 0, -1, 0,
                                       NULL) == PKV_EINVAL, "windowed step: negative window");
    check(pkv_paged_decode_step_qkv(h16, h16, h16, hf, hf, 128, 1e-6f, 2, h16, h16, h16, pool, h32, 8, h32, 4, 32,
                                    0.1f, h16, 0, 0, NULL) == PKV_EINVAL, "QKV step: qk_mode 2");
    check(pkv_paged_decode_step_qkv(h16, h16, h16, hf, hf, 0, 1e-6f, 1, h16, h16, h16, pool, h32, 8, h32, 4, 32,
                                    0.1f, h16, 0, 0, NULL) == PKV_EINVAL, "QKV step: no positions");
    /* varlen */
    check(pkv_paged_varlen_attention(h16, h16, h16, pool, h32, 8, NULL, h32, 4, 9, 32, 0.1f, h16, 0, 0, 0, NULL) ==
              PKV_EINVAL, "varlen attention: NULL prefix sums");
    check(pkv_paged_varlen_attention(h16, h16, h16, pool, h32, 8, h32, h32, 4, -9, 32, 0.1f, h16, 0, 0, 0, NULL) ==
              PKV_EINVAL, "varlen attention: negative token count");
    check(pkv_paged_varlen_step(h16, h16, h16, h16, h16, pool, h32, 8, h32, h32, 4, 9, 32, 0.1f, h16, 0, 0, 0,
                                NULL) == PKV_EINVAL, "varlen step: max_q_len 0");
    /* QKV to cache */
    check(pkv_split_qkv_norm_rope_into_paged_cache_varlen(h16, h16, h16, hf, hf, 128, h16, h16, h16, pool, h32, 8,
                                                          h32, h32, 4, 9, 32, -1.0f, 1, NULL) == PKV_EINVAL,
          "QKV to cache: negative eps");
    check(pkv_split_qkv_norm_rope_into_paged_cache(h16, h16, h16, hf, hf, 128, h16, h16, h16, pool, h32, 8, 4, 32,
                                                   126, 0, 1e-6f, 1, NULL) == PKV_EINVAL,
          "QKV to cache: positions past the table");
    check(pkv_split_qkv_norm_rope_into_paged_cache(h16, h16, h16, hf, hf, 1024, h16, h16, h16, pool, h32, 8, 4, 32,
                                                   0, 126, 1e-6f, 1, NULL) == PKV_EINVAL,
          "QKV to cache: cache rows past the table");
    /* split-K pieces */
    check(pkv_paged_decode_split_partials(h16, h16, h16, pool, h32, 8, h32, 4, 32, 0.1f, 0, 0, hf, hf, hf, NULL) ==
              PKV_EINVAL, "split partials: zero splits");
    check(pkv_paged_decode_split_combine(hf, hf, NULL, h32, 4, 32, 128, 16, 8, 2, 0, h16, NULL) == PKV_EINVAL,
          "split combine: NULL partial_l");
    /* input checks and utilities */
    check(pkv_check_decode_inputs(h32, 8, h32, -1, pool, 0, h32, NULL) == PKV_EINVAL, "input check: negative batch");
    check(pkv_check_slot_mapping(h32, 4, bs8, h32, NULL) == PKV_EUNSUPPORTED, "slot check: block_size 8");
    check(pkv_device_cu_count(NULL) == PKV_EINVAL, "cu count: NULL");
    check(strlen(pkv_last_error()) > 0 && strlen(pkv_version()) > 0, "messages and version");

    check(pkv_test_stub_launches() == 0, "nothing was enqueued by any failing call");
    return failures == 0 ? 0 : 1;
}
