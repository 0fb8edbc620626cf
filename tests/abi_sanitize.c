/*
 * Driver for the library's host code (argument checks, workspace layout, plan objects, the
 * status strings) under AddressSanitizer / UndefinedBehaviorSanitizer, on a machine without a
 * GPU.  Every call below returns before anything would be enqueued: device pointers are fake
 * addresses the host code only checks and stores, never dereferences.  Each descriptor, weight
 * table and expert array lives in a heap block of exactly its size, so a read past one of them
 * is reported; every plan is destroyed, so a leak or a double free is reported too.
 * Returns non-zero (and prints the case) on any unexpected status.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/ffn_sparse.h"

static int failures = 0;

#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        ffn_status got_ = (call);                                                             \
        if (got_ != (want)) {                                                                 \
            printf("FAIL line %d: %s -> %s (%s), want %s\n", __LINE__, #call,                 \
                   ffn_status_string(got_), ffn_last_error(), ffn_status_string(want));       \
            ++failures;                                                                       \
        }                                                                                     \
        if (ffn_last_error() == NULL) {                                                       \
            printf("FAIL line %d: ffn_last_error() is NULL\n", __LINE__);                     \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

static ffn_layer_desc *new_desc(int32_t d, int32_t ffn, int32_t rank, int32_t act,
                                int32_t w_dtype, int32_t max_batch)
{
    ffn_layer_desc *p = (ffn_layer_desc *)malloc(sizeof(ffn_layer_desc));
    p->d = d;
    p->ffn = ffn;
    p->rank = rank;
    p->act = act;
    p->w_dtype = w_dtype;
    p->x_dtype = w_dtype == FFN_F32 ? FFN_F32 : FFN_F16;
    p->p_dtype = p->x_dtype;
    p->threshold = 0.5f;
    p->max_batch = max_batch;
    return p;
}

/* fake, 16-byte aligned device addresses */
#define DEV(k) ((const void *)(uintptr_t)(0x100000u * (k)))

static ffn_layer_weights *new_weights(int gate, int i4)
{
    ffn_layer_weights *w = (ffn_layer_weights *)calloc(1, sizeof(ffn_layer_weights));
    w->w_up = DEV(1);
    w->w_gate = gate ? DEV(2) : NULL;
    w->w_down_t = DEV(3);
    if (i4) {
        w->s_up = DEV(4);
        w->s_gate = gate ? DEV(5) : NULL;
        w->s_down_t = DEV(6);
    }
    w->p1 = DEV(7);
    w->p2 = DEV(8);
    return w;
}

int main(int argc, char **argv)
{
    if (argc > 1 && strcmp(argv[1], "planted") == 0) {
        /* a descriptor cut short by its last field: the library's check reads max_batch one
         * block past the allocation, which AddressSanitizer must report from the library */
        ffn_layer_desc *cut = (ffn_layer_desc *)malloc(offsetof(ffn_layer_desc, max_batch));
        memcpy(cut, new_desc(768, 3072, 64, FFN_ACT_RELU, FFN_F32, 1),
               offsetof(ffn_layer_desc, max_batch));
        size_t b = 0;
        ffn_workspace_size(cut, &b);
        printf("planted read not reported\n");
        return 0;
    }
    /* status strings: every value, and out-of-range values */
    for (int s = -2; s <= 7; ++s) {
        const char *t = ffn_status_string((ffn_status)s);
        if (!t || !*t) {
            printf("FAIL: status string of %d\n", s);
            ++failures;
        }
    }
    if (strcmp(ffn_status_string(FFN_ERR_WORKSPACE_TOO_SMALL), "FFN_ERR_WORKSPACE_TOO_SMALL")) {
        printf("FAIL: status string text\n");
        ++failures;
    }

    /* workspace sizes: valid shapes of every storage type, and rejected ones */
    size_t bytes = 0;
    static const int32_t shapes[][6] = {
        /* d, ffn, rank, act, w_dtype, max_batch */
        {768, 3072, 64, FFN_ACT_RELU, FFN_F32, 1},
        {4096, 11008, 256, FFN_ACT_REGLU, FFN_F16, 1},
        {4096, 14336, 512, FFN_ACT_DRELU, FFN_F16, 32},
        {4096, 14336, 256, FFN_ACT_DRELU, FFN_I4G32, 1},
        {8192, 32768, 1024, FFN_ACT_RELU, FFN_F16, 512},
        {256, 1024, 32, FFN_ACT_REGLU, FFN_F16, 4096},
        {64, 256, 0, FFN_ACT_RELU, FFN_F32, 3},
    };
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
        const int32_t *s = shapes[i];
        ffn_layer_desc *d = new_desc(s[0], s[1], s[2], s[3], s[4], s[5]);
        EXPECT(ffn_workspace_size(d, &bytes), FFN_OK);
        free(d);
    }
    static const int32_t bad[][7] = {
        /* d, ffn, rank, act, w_dtype, max_batch, expected */
        {0, 3072, 64, FFN_ACT_RELU, FFN_F32, 1, FFN_ERR_INVALID_ARGUMENT},
        {768, 3072, 64, 9, FFN_F32, 1, FFN_ERR_INVALID_ARGUMENT},
        {4100, 11008, 256, FFN_ACT_REGLU, FFN_F16, 1, FFN_ERR_UNSUPPORTED},
        {4096, 11000, 256, FFN_ACT_REGLU, FFN_F16, 1, FFN_ERR_UNSUPPORTED},
        {4096, 11008, 100, FFN_ACT_REGLU, FFN_F16, 1, FFN_ERR_UNSUPPORTED},
        {16384, 11008, 256, FFN_ACT_REGLU, FFN_F16, 1, FFN_ERR_UNSUPPORTED},
        {4096, 11008, 256, FFN_ACT_REGLU, FFN_F16, 5000, FFN_ERR_UNSUPPORTED},
        {4096, 11008, 256, FFN_ACT_REGLU, FFN_F16, 0, FFN_ERR_INVALID_ARGUMENT},
    };
    for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
        const int32_t *s = bad[i];
        ffn_layer_desc *d = new_desc(s[0], s[1], s[2], s[3], s[4], s[5]);
        EXPECT(ffn_workspace_size(d, &bytes), (ffn_status)s[6]);
        free(d);
    }
    EXPECT(ffn_workspace_size(NULL, &bytes), FFN_ERR_INVALID_ARGUMENT);

    /* plans over fake device pointers: host-only calls on them, then destroy */
    ffn_plan *plan = NULL;
    ffn_layer_desc *d = new_desc(4096, 11008, 256, FFN_ACT_REGLU, FFN_F16, 512);
    ffn_layer_weights *w = new_weights(1, 0);
    EXPECT(ffn_workspace_size(d, &bytes), FFN_OK);
    void *ws = (void *)(uintptr_t)0x40000000u;
    EXPECT(ffn_sparse_plan(d, w, ws, bytes - 1, NULL, 0, &plan), FFN_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(ffn_sparse_plan(d, w, (void *)((uintptr_t)ws + 8), bytes, NULL, 0, &plan),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_sparse_plan(d, w, ws, bytes, NULL, 0, &plan), FFN_OK);
    float rho = 0.0f;
    for (int B = 1; B <= 4096; B *= 2) EXPECT(ffn_plan_crossover(plan, B, &rho), FFN_OK);
    EXPECT(ffn_plan_set_crossover(plan, 64, 0.3f), FFN_OK);
    EXPECT(ffn_plan_set_crossover(plan, 64, 1.5f), FFN_ERR_INVALID_ARGUMENT);
    const int32_t *flag = NULL;
    EXPECT(ffn_plan_path_flag(plan, &flag), FFN_OK);
    EXPECT(ffn_plan_set_hot_head(plan, 33), FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_plan_set_hot_head(plan, 256), FFN_OK);
    EXPECT(ffn_plan_set_decode_variant(plan, 1), FFN_OK);
    EXPECT(ffn_plan_set_decode_variant(plan, 2), FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_plan_set_timing_events(plan, FFN_STAGE_GATHER, NULL, NULL), FFN_OK);
    EXPECT(ffn_plan_set_timing_events(plan, 42, NULL, NULL), FFN_ERR_INVALID_ARGUMENT);
    /* forward argument checks (nothing is enqueued) */
    float *y = (float *)(uintptr_t)0x50000000u;
    EXPECT(ffn_sparse_forward(plan, DEV(9), 0, y, NULL, NULL, NULL, NULL, FFN_PATH_AUTO, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_sparse_forward(plan, DEV(9), 513, y, NULL, NULL, NULL, NULL, FFN_PATH_AUTO, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_sparse_forward(plan, DEV(9), 1, NULL, NULL, NULL, NULL, NULL, FFN_PATH_AUTO, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_sparse_forward(plan, DEV(9), 1, y, NULL, NULL, NULL, NULL, 7, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_sparse_forward(plan, DEV(9), 1, y, (const uint8_t *)(uintptr_t)0x60000001u, NULL,
                              NULL, NULL, FFN_PATH_SPARSE, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_dense_forward(plan, DEV(9), 600, y, NULL, NULL), FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_dense_forward(plan, NULL, 1, y, NULL, NULL), FFN_ERR_INVALID_ARGUMENT);

    /* a mixture over three plans of the same descriptor (and one that differs) */
    ffn_layer_desc *de = new_desc(4096, 14336, 256, FFN_ACT_DRELU, FFN_I4G32, 1);
    ffn_layer_weights *we = new_weights(1, 1);
    ffn_plan **experts = (ffn_plan **)calloc(3, sizeof(ffn_plan *));
    size_t eb = 0;
    EXPECT(ffn_workspace_size(de, &eb), FFN_OK);
    for (int e = 0; e < 3; ++e)
        EXPECT(ffn_sparse_plan(de, we, ws, eb, NULL, 0, &experts[e]), FFN_OK);
    size_t mb = 0;
    EXPECT(ffn_moe_workspace_size(3, 2, experts[0], &mb), FFN_OK);
    EXPECT(ffn_moe_workspace_size(17, 2, experts[0], &mb), FFN_ERR_UNSUPPORTED);
    EXPECT(ffn_moe_workspace_size(3, 2, experts[0], &mb), FFN_OK);
    ffn_moe *moe = NULL;
    EXPECT(ffn_moe_plan(3, 2, DEV(10), experts, ws, mb - 256, &moe), FFN_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(ffn_moe_plan(3, 2, DEV(10), experts, ws, mb, &moe), FFN_OK);
    EXPECT(ffn_moe_forward(moe, DEV(9), 2, y, NULL, NULL, NULL, NULL), FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_moe_destroy(moe), FFN_OK);
    ffn_plan *odd = NULL;
    ffn_layer_desc *dodd = new_desc(4096, 14336, 128, FFN_ACT_DRELU, FFN_I4G32, 1);
    EXPECT(ffn_sparse_plan(dodd, we, ws, eb, NULL, 0, &odd), FFN_OK);
    ffn_plan *pair[2] = {experts[0], odd};
    ffn_plan **pairs = (ffn_plan **)malloc(sizeof(pair));
    memcpy(pairs, pair, sizeof(pair));
    EXPECT(ffn_moe_plan(2, 1, DEV(10), pairs, ws, mb, &moe), FFN_ERR_INVALID_ARGUMENT);
    free(pairs);
    EXPECT(ffn_plan_destroy(odd), FFN_OK);
    for (int e = 0; e < 3; ++e) EXPECT(ffn_plan_destroy(experts[e]), FFN_OK);
    free(experts);

    /* the neuron-cache plan rejects rows that are not pinned host memory */
    size_t ob = 0;
    ffn_layer_desc *d1 = new_desc(4096, 11008, 256, FFN_ACT_REGLU, FFN_F16, 1);
    EXPECT(ffn_offload_workspace_size(d1, 2048, &ob), FFN_OK);
    EXPECT(ffn_offload_workspace_size(d1, 48, &ob), FFN_ERR_INVALID_ARGUMENT);
    ffn_plan *op = NULL;
    EXPECT(ffn_offload_plan(d1, w, 2048, 0, ws, ob, NULL, &op), FFN_ERR_INVALID_ARGUMENT);

    /* the allocation-free entry point: its checks, and the size limit of its scratch */
    EXPECT(ffn_sparse_forward_static(d1, w, DEV(9), 2, y, NULL, NULL, NULL, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    ffn_layer_desc *dbig = new_desc(8192, 32768, 1024, FFN_ACT_RELU, FFN_F16, 1);
    EXPECT(ffn_sparse_forward_static(dbig, w, DEV(9), 1, y, NULL, NULL, NULL, NULL),
           FFN_ERR_WORKSPACE_TOO_SMALL);

    /* the attention block: descriptor checks, workspace size, plan and the forward's checks */
    ffn_attn_desc *ad = (ffn_attn_desc *)malloc(sizeof(ffn_attn_desc));
    ad->d = 4096;
    ad->heads = 32;
    ad->kv_heads = 8;
    ad->head_dim = 128;
    ad->rank = 128;
    ad->max_seq = 512;
    ad->threshold = 0.5f;
    ffn_attn_weights *aw = (ffn_attn_weights *)calloc(1, sizeof(ffn_attn_weights));
    aw->w_q = DEV(1);
    aw->w_k = DEV(2);
    aw->w_v = DEV(3);
    aw->w_o_t = DEV(4);
    aw->p1 = DEV(5);
    aw->p2 = DEV(6);
    size_t ab = 0;
    EXPECT(ffn_attn_workspace_size(ad, &ab), FFN_OK);
    EXPECT(ffn_attn_workspace_size(ad, NULL), FFN_ERR_INVALID_ARGUMENT);
    ad->kv_heads = 5;
    EXPECT(ffn_attn_workspace_size(ad, &ab), FFN_ERR_UNSUPPORTED);
    ad->kv_heads = 8;
    ad->head_dim = 96;
    EXPECT(ffn_attn_workspace_size(ad, &ab), FFN_ERR_UNSUPPORTED);
    ad->head_dim = 128;
    ffn_attn *ap = NULL;
    EXPECT(ffn_attn_plan(ad, aw, ws, ab - 1, &ap), FFN_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(ffn_attn_plan(ad, aw, ws, ab, &ap), FFN_OK);
    EXPECT(ffn_attn_forward(ap, DEV(9), 512, DEV(10), DEV(11), y, NULL, NULL, NULL, NULL, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_attn_forward(ap, DEV(9), 0, NULL, DEV(11), y, NULL, NULL, NULL, NULL, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_attn_forward(NULL, DEV(9), 0, DEV(10), DEV(11), y, NULL, NULL, NULL, NULL, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_attn_set_timing_events(ap, FFN_STAGE_GATHER, NULL, NULL),
           FFN_ERR_INVALID_ARGUMENT);
    EXPECT(ffn_attn_destroy(ap), FFN_OK);
    EXPECT(ffn_attn_destroy(NULL), FFN_OK);
    free(ad);
    free(aw);

    EXPECT(ffn_plan_destroy(plan), FFN_OK);
    EXPECT(ffn_plan_destroy(NULL), FFN_OK);
    free(d);
    free(w);
    free(de);
    free(we);
    free(dodd);
    free(d1);
    free(dbig);
    if (failures) {
        printf("abi sanitizer run: %d failure(s)\n", failures);
        return 1;
    }
    printf("abi sanitizer run: OK\n");
    return 0;
}
