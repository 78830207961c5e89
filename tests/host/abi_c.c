/* abi_c.c -- the C ABI from plain C99: include/kvattn.h compiled as C and
 * the library's host-only entry points called from a C program (no GPU work,
 * no handle).  Built and run by tests/test_c_abi.py with gcc; exit status 0
 * and a last line "ok" mean every check held. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/kvattn.h"

static int failures = 0;
#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "check failed at line %d: ", __LINE__);       \
            fprintf(stderr, __VA_ARGS__);                                 \
            fprintf(stderr, "\n");                                        \
            failures++;                                                   \
        }                                                                 \
    } while (0)

/* The 40-query-head, 8-KV-head geometry with 256-position pages. */
static kvattn_params workload_params(uint32_t k_type, uint32_t v_type) {
    kvattn_params p;
    memset(&p, 0, sizeof p);
    p.struct_size = sizeof p;
    p.n_layers = 2;
    p.n_q_heads = 40;
    p.n_kv_heads = 8;
    p.head_dim = 128;
    p.page_tokens = 256;
    p.k_type = k_type;
    p.v_type = v_type;
    p.n_pool_pages = 16;
    p.n_ring_slots = 4;
    p.max_pages_per_layer = 8;
    p.max_rows = 6;
    return p;
}

int main(void) {
    /* supported pairs, and the ones that fail closed */
    CHECK(kvattn_supported(KVATTN_TYPE_Q8_0, KVATTN_TYPE_Q4_0, 128) == 1, "Q8_0/Q4_0");
    CHECK(kvattn_supported(KVATTN_TYPE_Q8_0, KVATTN_TYPE_Q8_0, 128) == 1, "Q8_0/Q8_0");
    CHECK(kvattn_supported(KVATTN_TYPE_Q4_0, KVATTN_TYPE_Q4_0, 128) == 1, "Q4_0/Q4_0");
    CHECK(kvattn_supported(KVATTN_TYPE_F16, KVATTN_TYPE_F16, 128) == 1, "F16/F16");
    CHECK(kvattn_supported(KVATTN_TYPE_Q4_0, KVATTN_TYPE_Q8_0, 128) == 0, "Q4_0/Q8_0 must fail closed");
    CHECK(kvattn_supported(KVATTN_TYPE_Q8_0, KVATTN_TYPE_Q4_0, 64) == 0, "head_dim 64 must fail closed");

    /* page sizes: H * T * (kc + 8 + vc + 8) for block pairs, H * T * 512 for F16 */
    kvattn_params p = workload_params(KVATTN_TYPE_Q8_0, KVATTN_TYPE_Q4_0);
    CHECK(kvattn_page_bytes(&p) == 425984u, "Q8_0/Q4_0 page %zu", kvattn_page_bytes(&p));
    kvattn_params f = workload_params(KVATTN_TYPE_F16, KVATTN_TYPE_F16);
    CHECK(kvattn_page_bytes(&f) == 8u * 256u * 512u, "F16 page %zu", kvattn_page_bytes(&f));
    kvattn_params q8 = workload_params(KVATTN_TYPE_Q8_0, KVATTN_TYPE_Q8_0);
    CHECK(kvattn_page_bytes(&q8) == 8u * 256u * (128u + 8u + 128u + 8u), "Q8_0/Q8_0 page %zu", kvattn_page_bytes(&q8));
    kvattn_params bad = p;
    bad.head_dim = 64;
    CHECK(kvattn_page_bytes(&bad) == 0 && kvattn_workspace_bytes(&bad) == 0, "invalid geometry must size 0");
    CHECK(strlen(kvattn_global_error()) > 0, "an invalid call leaves a message");
    bad = p;
    bad.n_q_heads = 42; /* not a multiple of the KV heads */
    CHECK(kvattn_page_bytes(&bad) == 0, "GQA ratio must divide");

    /* the workspace grows with the rows it must hold */
    const size_t ws6 = kvattn_workspace_bytes(&p);
    kvattn_params wide = p;
    wide.max_rows = 64;
    CHECK(ws6 > 0 && kvattn_workspace_bytes(&wide) > ws6, "workspace %zu then %zu", ws6, kvattn_workspace_bytes(&wide));

    /* page-table validation: ok, duplicate physical page, pool id out of
     * range, ring slot out of range, host entries without a history */
    const uint32_t n_tokens = 3 * 256 - 5;
    uint32_t t[3] = {2, 0, KVATTN_PT_RING(1)};
    CHECK(kvattn_validate_page_table(&p, t, n_tokens, 0) == KVATTN_OK, "valid table: %s", kvattn_global_error());
    t[1] = 2;
    CHECK(kvattn_validate_page_table(&p, t, n_tokens, 0) == KVATTN_E_PLAN, "duplicate page");
    t[1] = 16;
    CHECK(kvattn_validate_page_table(&p, t, n_tokens, 0) == KVATTN_E_RANGE, "pool id past the pool");
    t[1] = 0;
    t[2] = KVATTN_PT_RING(4);
    CHECK(kvattn_validate_page_table(&p, t, n_tokens, 0) == KVATTN_E_RANGE, "ring slot past the ring");
    t[2] = KVATTN_PT_HOST;
    CHECK(kvattn_validate_page_table(&p, t, n_tokens, 0) != KVATTN_OK, "streamed page without a history");

    /* the streaming planner: two streamed layers, called in order twice */
    const uint32_t counts[2] = {5, 3}, calls[4] = {0, 1, 0, 1};
    int64_t ops[256 * 7];
    uint32_t n_ops = 0;
    CHECK(kvattn_sched_simulate(2, 4, 2, counts, calls, 4, ops, 256, &n_ops) == KVATTN_OK, "planner: %s",
          kvattn_global_error());
    uint32_t computed = 0, merged = 0;
    for (uint32_t i = 0; i < n_ops; i++) {
        if (ops[7 * i] == 2) computed += (uint32_t)ops[7 * i + 3];
        if (ops[7 * i] == 4) merged++;
    }
    CHECK(computed == 2 * (5 + 3) && merged == 4, "planner computed %u streamed pages, %u merges", computed, merged);

    /* one policy step: a history that fits stays resident */
    kvattn_policy_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.n_layers = 4;
    cfg.page_tokens = 256;
    cfg.budget_pages = 64;
    cfg.min_ring_slots = 2;
    cfg.max_ring_slots = 8;
    cfg.ring_step = 2;
    cfg.grow_after = 1;
    cfg.shrink_after = 1;
    cfg.miss_rate_high = 0.5f;
    cfg.busy_high = 0.9f;
    cfg.occupancy_low = 0.25f;
    kvattn_policy_state st, next;
    memset(&st, 0, sizeof st);
    kvattn_policy_observation ob;
    memset(&ob, 0, sizeof ob);
    ob.n_tokens = 10 * 256;
    kvattn_policy_decision d;
    uint32_t resident[4];
    CHECK(kvattn_policy_step(&cfg, &st, &ob, &next, &d, resident) == KVATTN_OK, "policy: %s", kvattn_global_error());
    CHECK(d.reason == KVATTN_POLICY_FITS && d.ring_slots == 0 && d.resident_pages == 40 && d.streamed_pages == 0,
          "policy fits: reason %u ring %u resident %u", d.reason, d.ring_slots, d.resident_pages);
    /* a budget that holds half the pages streams whole layers */
    ob.n_tokens = 32 * 256;
    CHECK(kvattn_policy_step(&cfg, &st, &ob, &next, &d, resident) == KVATTN_OK, "policy: %s", kvattn_global_error());
    CHECK(d.streamed_pages > 0 && d.resident_pages + d.ring_slots <= 64 && d.resident_pages + d.streamed_pages == 128,
          "policy streams: resident %u ring %u streamed %u", d.resident_pages, d.ring_slots, d.streamed_pages);

    /* handle calls on a null handle fail with an argument error */
    CHECK(kvattn_decode(NULL, 0, NULL, NULL) == KVATTN_E_ARG, "null handle");
    CHECK(kvattn_destroy(NULL) == KVATTN_OK, "destroying a null handle is a no-op");
    CHECK(strlen(kvattn_last_error(NULL)) > 0, "static text for a null handle");

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
