/*
 * fs_c_client.c -- a plain C99 program that uses the engine only through
 * include/fs.h and the HIP runtime, the way a C or C++ training runtime
 * would.  Test program, not part of the library.
 *
 *   fs_c_client host   plan the worked example of "FSDP1 vs FSDP2" (Table 3:
 *                      two parameters of 3 and 5 elements, N = 4, bf16) under
 *                      FSDP1 (use_orig_params false / true) and FSDP2, and
 *                      the documented error returns; the fp32 twin of the
 *                      use_orig_params plan beside the plan made directly
 *                      with FS_FP32 (the twin keeps the bf16 alignment, the
 *                      direct plan aligns fp32 elements); print one JSON
 *                      line.  Makes no GPU call.
 *   fs_c_client gpu    on device 0: plan the tiny 2-layer MLP group (FSDP1,
 *                      use_orig_params, N = 4, grad_acc = 2), pack every
 *                      shard, unpack, reduce 8 constant gradient slices and
 *                      take one AdamW step from zero moments; check each
 *                      result against what the method fixes (placement
 *                      given by the plan's segments, pads zero, the round
 *                      trip, the exact average, the first-step closed
 *                      form).  Prints "ok" and exits 0, or names the first
 *                      mismatch and exits 1.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fs.h"

static int plan_shapes(int32_t n, const int32_t *ndim, const int64_t *dims, int32_t world, int32_t uo,
                       fs_mode mode, int32_t grad_acc, fs_plan_t *p) {
    return fs_plan(n, ndim, dims, FS_BF16, world, uo, mode, grad_acc, p);
}

/* ------------------------------------------------------------------ host -- */

static void print_plan(const char *name, fs_plan_t p) {
    fs_plan_info_t I;
    if (fs_plan_info(p, &I) != FS_OK) {
        printf("\"%s\": null", name);
        return;
    }
    printf("\"%s\": {\"shard_numel\": %lld, \"gathered_numel\": %lld, \"align_pad\": %lld, "
           "\"tail_pad\": %lld, \"segments\": [",
           name, (long long)I.shard_numel, (long long)I.gathered_numel, (long long)I.align_pad,
           (long long)I.tail_pad);
    int64_t n = 0;
    fs_plan_segments(p, NULL, 0, &n);
    fs_segment_t *s = (fs_segment_t *)calloc((size_t)(n > 0 ? n : 1), sizeof(fs_segment_t));
    fs_plan_segments(p, s, n, &n);
    for (int64_t i = 0; i < n; ++i)
        printf("%s[%lld, %lld, %lld, %d, %d]", i ? ", " : "", (long long)s[i].dst_off, (long long)s[i].src_off,
               (long long)s[i].len, s[i].param, s[i].rank);
    printf("]}");
    free(s);
}

static int run_host(void) {
    const int32_t ndim[2] = {1, 1};
    const int64_t dims[2] = {3, 5};
    fs_plan_t f1f = NULL, f1t = NULL, f2 = NULL, bad = NULL;
    int rc1 = plan_shapes(2, ndim, dims, 4, 0, FS_FSDP1_FLAT, 1, &f1f);
    int rc2 = plan_shapes(2, ndim, dims, 4, 1, FS_FSDP1_FLAT, 1, &f1t);
    int rc3 = plan_shapes(2, ndim, dims, 4, 0, FS_FSDP2_PER_PARAM, 1, &f2);
    printf("{\"rc\": [%d, %d, %d], ", rc1, rc2, rc3);
    print_plan("fsdp1_use_orig_params_false", f1f);
    printf(", ");
    print_plan("fsdp1_use_orig_params_true", f1t);
    printf(", ");
    print_plan("fsdp2", f2);
    fs_plan_t twin = NULL, f1t32 = NULL;
    int rc_twin = fs_plan_twin(f1t, FS_FP32, &twin);
    int rc_f32 = fs_plan(2, ndim, dims, FS_FP32, 4, 1, FS_FSDP1_FLAT, 1, &f1t32);
    fs_plan_info_t It;
    int eb_twin = (rc_twin == FS_OK && fs_plan_info(twin, &It) == FS_OK) ? It.elem_bytes : 0;
    printf(", \"twin_rc\": [%d, %d], \"twin_elem_bytes\": %d, ", rc_twin, rc_f32, eb_twin);
    print_plan("fsdp1_use_orig_params_true_fp32_twin", twin);
    printf(", ");
    print_plan("fsdp1_use_orig_params_true_fp32_direct", f1t32);
    fs_plan_t none = NULL;
    int e_twin_dtype = fs_plan_twin(f1t, (fs_dtype)7, &none);
    int e_twin_null = fs_plan_twin(NULL, FS_FP32, &none);
    int e_world = plan_shapes(2, ndim, dims, 0, 0, FS_FSDP1_FLAT, 1, &bad);
    int e_uo = plan_shapes(2, ndim, dims, 4, 1, FS_FSDP2_PER_PARAM, 1, &bad);
    const int64_t neg[2] = {3, -5};
    int e_dim = plan_shapes(2, ndim, neg, 4, 0, FS_FSDP1_FLAT, 1, &bad);
    int e_acc = plan_shapes(2, ndim, dims, 4, 0, FS_FSDP1_FLAT, 0, &bad);
    const char *msg = fs_last_error();
    printf(", \"errors\": {\"world_0\": %d, \"use_orig_params_fsdp2\": %d, \"negative_dim\": %d, "
           "\"grad_acc_0\": %d, \"twin_bad_dtype\": %d, \"twin_null\": %d, \"last_error_nonempty\": %d}}\n",
           e_world, e_uo, e_dim, e_acc, e_twin_dtype, e_twin_null, msg != NULL && msg[0] != '\0');
    fs_plan_destroy(f1f);
    fs_plan_destroy(f1t);
    fs_plan_destroy(f2);
    fs_plan_destroy(twin);
    fs_plan_destroy(f1t32);
    return 0;
}

/* ------------------------------------------------------------------- gpu -- */

#define CHECK_HIP(x)                                                                 \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            return 1;                                                                \
        }                                                                            \
    } while (0)

#define CHECK_FS(x)                                                                  \
    do {                                                                             \
        int r_ = (x);                                                                \
        if (r_ != FS_OK) {                                                           \
            printf("fs error %d (%s) at line %d\n", r_, fs_last_error(), __LINE__);  \
            return 1;                                                                \
        }                                                                            \
    } while (0)

static uint32_t xorshift32(uint32_t *s) {
    uint32_t x = *s;
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return *s = x;
}

static uint16_t bf16_bits(float f) { /* exact for the values used here */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static uint16_t bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static int run_gpu(void) {
    int ndev = 0;
    CHECK_HIP(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        printf("no GPU\n");
        return 1;
    }
    CHECK_HIP(hipSetDevice(0));
    /* the tiny 2-layer MLP: W_in 64x256, W_out 256x64, bias 256, LN weight 64 */
    const int32_t ndim[4] = {2, 2, 1, 1};
    const int64_t dims[6] = {64, 256, 256, 64, 256, 64};
    const int32_t np = 4, N = 4, A = 2;
    fs_plan_t plan = NULL;
    CHECK_FS(plan_shapes(np, ndim, dims, N, 1, FS_FSDP1_FLAT, A, &plan));
    fs_plan_info_t I;
    CHECK_FS(fs_plan_info(plan, &I));
    void *ws = NULL;
    CHECK_HIP(hipMalloc(&ws, (size_t)I.workspace_bytes));
    CHECK_FS(fs_plan_upload(plan, ws, (size_t)I.workspace_bytes, NULL));

    int64_t numel[4];
    uint16_t *h_par[4];
    void *d_par[4], *d_out[4];
    uint32_t seed = 0x9E3779B9u;
    for (int i = 0; i < np; ++i) {
        fs_param_layout_t pl;
        CHECK_FS(fs_plan_param(plan, i, &pl));
        numel[i] = pl.numel;
        h_par[i] = (uint16_t *)malloc((size_t)numel[i] * 2);
        for (int64_t e = 0; e < numel[i]; ++e) h_par[i][e] = (uint16_t)xorshift32(&seed);
        CHECK_HIP(hipMalloc(&d_par[i], (size_t)numel[i] * 2));
        CHECK_HIP(hipMalloc(&d_out[i], (size_t)numel[i] * 2));
        CHECK_HIP(hipMemcpy(d_par[i], h_par[i], (size_t)numel[i] * 2, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemset(d_out[i], 0x5A, (size_t)numel[i] * 2));
    }
    void **d_tab_in = NULL, **d_tab_out = NULL;
    CHECK_HIP(hipMalloc((void **)&d_tab_in, sizeof(void *) * np));
    CHECK_HIP(hipMalloc((void **)&d_tab_out, sizeof(void *) * np));
    CHECK_HIP(hipMemcpy(d_tab_in, d_par, sizeof(void *) * np, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_tab_out, d_out, sizeof(void *) * np, hipMemcpyHostToDevice));

    /* pack all N shards, then check every element against the plan's segments */
    const int64_t G = I.gathered_numel;
    void *d_gath = NULL;
    CHECK_HIP(hipMalloc(&d_gath, (size_t)G * 2));
    CHECK_HIP(hipMemset(d_gath, 0x5A, (size_t)G * 2));
    CHECK_FS(fs_pack(plan, (const void *const *)d_tab_in, d_gath, -1, NULL));
    CHECK_FS(fs_unpack(plan, d_gath, (void *const *)d_tab_out, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    uint16_t *h_gath = (uint16_t *)malloc((size_t)G * 2);
    unsigned char *covered = (unsigned char *)calloc((size_t)G, 1);
    CHECK_HIP(hipMemcpy(h_gath, d_gath, (size_t)G * 2, hipMemcpyDeviceToHost));
    int64_t nseg = 0;
    fs_plan_segments(plan, NULL, 0, &nseg);
    fs_segment_t *segs = (fs_segment_t *)calloc((size_t)nseg, sizeof(fs_segment_t));
    CHECK_FS(fs_plan_segments(plan, segs, nseg, &nseg));
    for (int64_t s = 0; s < nseg; ++s)
        for (int64_t k = 0; k < segs[s].len; ++k) {
            const int64_t d = segs[s].dst_off + k;
            covered[d] = 1;
            if (h_gath[d] != h_par[segs[s].param][segs[s].src_off + k]) {
                printf("pack: gathered[%lld] differs\n", (long long)d);
                return 1;
            }
        }
    for (int64_t d = 0; d < G; ++d)
        if (!covered[d] && h_gath[d] != 0) {
            printf("pack: pad gathered[%lld] is not zero\n", (long long)d);
            return 1;
        }
    for (int i = 0; i < np; ++i) {
        uint16_t *h = (uint16_t *)malloc((size_t)numel[i] * 2);
        CHECK_HIP(hipMemcpy(h, d_out[i], (size_t)numel[i] * 2, hipMemcpyDeviceToHost));
        if (memcmp(h, h_par[i], (size_t)numel[i] * 2) != 0) {
            printf("unpack: parameter %d differs\n", i);
            return 1;
        }
        free(h);
    }

    /* reduce: slice t (= j*N + k) holds 0.25*(t+1) everywhere; the average
     * over N of the A*N terms is 0.25 * (A*N)(A*N+1)/2 / N, exact in fp32 */
    const int64_t S = I.shard_numel;
    const int T = A * N;
    void *d_sl[8];
    uint16_t *h_sl = (uint16_t *)malloc((size_t)S * 2);
    for (int t = 0; t < T; ++t) {
        for (int64_t e = 0; e < S; ++e) h_sl[e] = bf16_bits(0.25f * (float)(t + 1));
        CHECK_HIP(hipMalloc(&d_sl[t], (size_t)S * 2));
        CHECK_HIP(hipMemcpy(d_sl[t], h_sl, (size_t)S * 2, hipMemcpyHostToDevice));
    }
    float *d_g = NULL, *d_th = NULL, *d_m = NULL, *d_v = NULL;
    uint16_t *d_p16 = NULL;
    CHECK_HIP(hipMalloc((void **)&d_g, (size_t)S * 4));
    CHECK_HIP(hipMalloc((void **)&d_th, (size_t)S * 4));
    CHECK_HIP(hipMalloc((void **)&d_m, (size_t)S * 4));
    CHECK_HIP(hipMalloc((void **)&d_v, (size_t)S * 4));
    CHECK_HIP(hipMalloc((void **)&d_p16, (size_t)S * 2));
    CHECK_FS(fs_reduce_shard(S, N, A, (const uint16_t *const *)d_sl, d_g, NULL));
    float *h_f = (float *)malloc((size_t)S * 4);
    const float want_g = 0.25f * (float)(T * (T + 1) / 2) / (float)N;
    CHECK_HIP(hipMemcpy(h_f, d_g, (size_t)S * 4, hipMemcpyDeviceToHost));
    for (int64_t e = 0; e < S; ++e)
        if (h_f[e] != want_g) {
            printf("reduce: out[%lld] = %.9g, want %.9g\n", (long long)e, h_f[e], want_g);
            return 1;
        }

    /* AdamW, step 1 from zero moments: m = (1-b1) g, v = (1-b2) g^2, the
     * bias-corrected ratio is g/|g|, so theta' = theta (1 - lr wd) - lr g/(|g| + eps) */
    for (int64_t e = 0; e < S; ++e) h_f[e] = 1.0f;
    CHECK_HIP(hipMemcpy(d_th, h_f, (size_t)S * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_m, 0, (size_t)S * 4));
    CHECK_HIP(hipMemset(d_v, 0, (size_t)S * 4));
    fs_adamw_hparams_t hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 0, 1};
    CHECK_FS(fs_adamw_step(S, d_th, d_m, d_v, d_g, FS_FP32, d_p16, &hp, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    const double lr = hp.lr, b1 = hp.beta1, b2 = hp.beta2, eps = hp.eps, wd = hp.weight_decay, g = want_g;
    const double th_want = 1.0 * (1.0 - lr * wd) - lr * g / (fabs(g) + eps);
    const double m_want = (1.0 - b1) * g, v_want = (1.0 - b2) * g * g;
    float *h_m = (float *)malloc((size_t)S * 4), *h_v = (float *)malloc((size_t)S * 4);
    uint16_t *h_p = (uint16_t *)malloc((size_t)S * 2);
    CHECK_HIP(hipMemcpy(h_f, d_th, (size_t)S * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_m, d_m, (size_t)S * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_v, d_v, (size_t)S * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_p, d_p16, (size_t)S * 2, hipMemcpyDeviceToHost));
    for (int64_t e = 0; e < S; ++e) {
        if (fabs(h_f[e] - th_want) > 1e-6 * fabs(th_want) || fabs(h_m[e] - m_want) > 1e-6 * fabs(m_want) ||
            fabs(h_v[e] - v_want) > 1e-6 * fabs(v_want) || h_p[e] != bf16_rne(h_f[e])) {
            printf("adamw: element %lld: theta %.9g (want %.9g), m %.9g (want %.9g), v %.9g (want %.9g)\n",
                   (long long)e, h_f[e], th_want, h_m[e], m_want, h_v[e], v_want);
            return 1;
        }
    }

    for (int t = 0; t < T; ++t) CHECK_HIP(hipFree(d_sl[t]));
    for (int i = 0; i < np; ++i) {
        CHECK_HIP(hipFree(d_par[i]));
        CHECK_HIP(hipFree(d_out[i]));
        free(h_par[i]);
    }
    CHECK_HIP(hipFree(d_tab_in));
    CHECK_HIP(hipFree(d_tab_out));
    CHECK_HIP(hipFree(d_gath));
    CHECK_HIP(hipFree(d_g));
    CHECK_HIP(hipFree(d_th));
    CHECK_HIP(hipFree(d_m));
    CHECK_HIP(hipFree(d_v));
    CHECK_HIP(hipFree(d_p16));
    CHECK_HIP(hipFree(ws));
    fs_plan_destroy(plan);
    free(h_gath);
    free(covered);
    free(segs);
    free(h_sl);
    free(h_f);
    free(h_m);
    free(h_v);
    free(h_p);
    printf("ok\n");
    return 0;
}

int main(int argc, char **argv) {
    if (argc == 2 && strcmp(argv[1], "host") == 0) return run_host();
    if (argc == 2 && strcmp(argv[1], "gpu") == 0) return run_gpu();
    fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
    return 2;
}
