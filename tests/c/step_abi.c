/* step_abi.c -- the library used from C through include/flatparam.h alone
 * (no Python, no torch): device buffers from hipMalloc, two micro-batches of
 * one rank's shard step in each of its forms (one-pass kernel, two phases,
 * speculative with separate output state), with and without an overflow,
 * each compared element by element with the serial CPU oracle on the same
 * input bytes.  Test infrastructure: the oracle (liboracle.so) is linked
 * here only to check the results.  Built as a shared library whose one
 * entry point, step_abi_run(), a test calls in its own process.
 *
 * The step follows "Infra: Data Parallel", ZeRO-1 / ZeRO-2 paragraphs
 * (reduce-scatter with averaging, AdamW on the rank's slice, all-gather of
 * the bf16 parameters) and "PyTorch FSDP" section 3.5 (overflow check of the
 * sharded gradient scaler).
 *
 * Bars: the reduced gradient bitwise, the fp32 state within 1e-6 relative /
 * 1e-9 absolute, the own bf16 slice within 1 ulp, the other ranks' slices
 * and the flag exactly.  step_abi_run() returns the number of failed cases
 * (0 when every case holds; 100 without a GPU) and prints one line per case
 * on stdout; a failed call ends its case (its buffers are not freed) but
 * never the process. */

#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flatparam.h"

/* the oracle's entry points (oracle/oracle.c) */
void or_reduce(int64_t shard, int32_t world, const uint16_t* const* grads, float scale, int32_t accumulate,
               float* acc);
void or_adamw(int64_t n, double lr, double beta1, double beta2, double eps, double weight_decay, int64_t step,
              const float* grad, float* master, float* exp_avg, float* exp_avg_sq, int32_t skip);
void or_f32_to_bf16_array(int64_t n, const float* x, uint16_t* y);

enum { WORLD = 8, RANK = 3, MICRO = 2 };
static const int64_t S = 1000003; /* odd: rows off the 8-byte grid, a ragged last tile */
static const double LR = 1e-3, B1 = 0.9, B2 = 0.999, EPS = 1e-8, WD = 0.01;
static const int64_t STEP = 3;

/* A failed HIP or library call ends the case with an error (returned to the
 * caller, which is a test in its own process: nothing here exits). */
#define HIP_OK(x)                                                                      \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_));  \
            return CASE_ERROR;                                                         \
        }                                                                              \
    } while (0)

#define CHECK_FP(x)                                                                      \
    do {                                                                                 \
        fp_status s_ = (x);                                                              \
        if (s_ != FP_OK) {                                                               \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, fp_status_string(s_), \
                    fp_last_error());                                                    \
            return CASE_ERROR;                                                           \
        }                                                                                \
    } while (0)

enum { CASE_ERROR = 1000 };

/* splitmix64: seeded inputs, the same bytes for the GPU and the oracle */
static uint64_t mix(uint64_t* s) {
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float uniform(uint64_t* s, float lo, float hi) {
    return lo + (hi - lo) * (float)((mix(s) >> 40) * (1.0 / 16777216.0));
}

static int dev_copy(void** p, const void* host, size_t bytes) {
    HIP_OK(hipMalloc(p, bytes));
    HIP_OK(hipMemcpy(*p, host, bytes, hipMemcpyHostToDevice));
    return 0;
}

static int ulp_distance_over_one(uint16_t a, uint16_t b) {
    /* ordered-integer distance of two bf16 patterns */
    int32_t x = (a & 0x8000) ? -(int32_t)(a & 0x7FFF) : (int32_t)a;
    int32_t y = (b & 0x8000) ? -(int32_t)(b & 0x7FFF) : (int32_t)b;
    return abs(x - y) > 1;
}

/* one case: form = 0 one pass, 1 two phases, 2 speculative; inf = plant an
 * overflow in the second micro-batch */
static int run_case(int form, int inf, int32_t want_path) {
    uint64_t seed = 20240601u + (uint64_t)(form * 2 + inf);
    const size_t nb = (size_t)S * sizeof(uint16_t), nf = (size_t)S * sizeof(float);
    uint16_t* grads = malloc((size_t)MICRO * WORLD * nb);
    float* tmp = malloc(nf);
    float* master = malloc(nf);
    float* exp_avg = malloc(nf);
    float* exp_avg_sq = malloc(nf);
    uint16_t* others = malloc((size_t)WORLD * nb);
    for (int m = 0; m < MICRO; ++m)
        for (int q = 0; q < WORLD; ++q) {
            for (int64_t i = 0; i < S; ++i) tmp[i] = uniform(&seed, -1e-3f, 1e-3f);
            or_f32_to_bf16_array(S, tmp, grads + ((size_t)m * WORLD + q) * S);
        }
    if (inf) grads[((size_t)1 * WORLD + 5) * S + S / 2] = 0x7F80; /* +inf, micro-batch 1, rank 5 */
    for (int64_t i = 0; i < S; ++i) {
        master[i] = uniform(&seed, -0.05f, 0.05f);
        exp_avg[i] = uniform(&seed, -1e-4f, 1e-4f);
        exp_avg_sq[i] = uniform(&seed, 0.0f, 1e-8f);
    }
    for (int q = 0; q < WORLD; ++q) {
        for (int64_t i = 0; i < S; ++i) tmp[i] = uniform(&seed, -0.05f, 0.05f);
        or_f32_to_bf16_array(S, tmp, others + (size_t)q * S);
    }

    /* device side: one buffer of rows per micro-batch, as a bucket would hold them */
    uint16_t *d_grads = NULL, *d_others = NULL;
    float *d_master = NULL, *d_m = NULL, *d_v = NULL;
    if (dev_copy((void**)&d_grads, grads, (size_t)MICRO * WORLD * nb) ||
        dev_copy((void**)&d_others, others, (size_t)WORLD * nb) || dev_copy((void**)&d_master, master, nf) ||
        dev_copy((void**)&d_m, exp_avg, nf) || dev_copy((void**)&d_v, exp_avg_sq, nf))
        return CASE_ERROR;
    float *d_acc = NULL, *d_out[3] = {NULL, NULL, NULL};
    uint16_t* d_full = NULL;
    int32_t* d_flag = NULL;
    void* d_ws = NULL;
    HIP_OK(hipMalloc((void**)&d_acc, nf));
    HIP_OK(hipMalloc((void**)&d_full, (size_t)WORLD * nb));
    HIP_OK(hipMalloc((void**)&d_flag, sizeof(int32_t)));
    HIP_OK(hipMemset(d_flag, 0, sizeof(int32_t)));
    const int64_t ws_bytes = fp_workspace_bytes(S);
    HIP_OK(hipMalloc(&d_ws, (size_t)ws_bytes));
    HIP_OK(hipMemset(d_ws, 0, (size_t)ws_bytes));
    if (form == 2)
        for (int k = 0; k < 3; ++k) HIP_OK(hipMalloc((void**)&d_out[k], nf));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    const uint16_t* rows[MICRO][WORLD];
    const uint16_t* shard_ptrs[WORLD];
    for (int m = 0; m < MICRO; ++m)
        for (int q = 0; q < WORLD; ++q) rows[m][q] = d_grads + ((size_t)m * WORLD + q) * S;
    for (int q = 0; q < WORLD; ++q) shard_ptrs[q] = q == RANK ? NULL : d_others + (size_t)q * S;
    const float scale = 1.0f / (float)(WORLD * MICRO);

    /* micro-batch 0: the reduce alone */
    CHECK_FP(fp_reduce_shard(S, WORLD, rows[0], scale, 0, d_acc, d_flag, NULL, NULL, stream));
    /* micro-batch 1: the step */
    fp_step_args a;
    memset(&a, 0, sizeof a);
    a.shard = S;
    a.world = WORLD;
    a.rank = RANK;
    a.grads = rows[1];
    a.scale = scale;
    a.accumulate = 1;
    a.acc = d_acc;
    a.master = d_master;
    a.exp_avg = d_m;
    a.exp_avg_sq = d_v;
    a.hp.lr = LR;
    a.hp.beta1 = B1;
    a.hp.beta2 = B2;
    a.hp.eps = EPS;
    a.hp.weight_decay = WD;
    a.hp.step = STEP;
    a.shards = shard_ptrs;
    a.full = d_full;
    a.found_inf = d_flag;
    a.workspace = d_ws;
    a.flags = FP_STEP_EXACT_SKIP | (form == 0 ? 0 : FP_STEP_NO_COOP) | (form == 1 ? FP_STEP_KEEP_GRAD : 0);
    if (form == 2) {
        a.master_out = d_out[0];
        a.exp_avg_out = d_out[1];
        a.exp_avg_sq_out = d_out[2];
    }
    int32_t path = -1;
    CHECK_FP(fp_step_path(&a, &path));
    CHECK_FP(fp_shard_step(&a, stream));
    HIP_OK(hipStreamSynchronize(stream));

    /* results */
    float* g_state[3] = {malloc(nf), malloc(nf), malloc(nf)};
    float* g_acc = malloc(nf);
    uint16_t* g_full = malloc((size_t)WORLD * nb);
    int32_t g_flag = -1;
    HIP_OK(hipMemcpy(g_state[0], form == 2 ? d_out[0] : d_master, nf, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_state[1], form == 2 ? d_out[1] : d_m, nf, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_state[2], form == 2 ? d_out[2] : d_v, nf, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_acc, d_acc, nf, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g_full, d_full, (size_t)WORLD * nb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&g_flag, d_flag, sizeof g_flag, hipMemcpyDeviceToHost));

    /* the oracle on the same bytes */
    float* o_acc = malloc(nf);
    const uint16_t* h_rows[MICRO][WORLD];
    for (int m = 0; m < MICRO; ++m)
        for (int q = 0; q < WORLD; ++q) h_rows[m][q] = grads + ((size_t)m * WORLD + q) * S;
    or_reduce(S, WORLD, h_rows[0], scale, 0, o_acc);
    or_reduce(S, WORLD, h_rows[1], scale, 1, o_acc);
    int32_t o_flag = 0;
    for (int64_t i = 0; i < S; ++i)
        if (!isfinite(o_acc[i])) o_flag = 1;
    or_adamw(S, LR, B1, B2, EPS, WD, STEP, o_acc, master, exp_avg, exp_avg_sq, o_flag);
    uint16_t* o_own = malloc(nb);
    or_f32_to_bf16_array(S, master, o_own);

    int64_t bad_acc = 0, bad_state = 0, bad_own = 0, bad_other = 0;
    const float* o_state[3] = {master, exp_avg, exp_avg_sq};
    for (int64_t i = 0; i < S; ++i) {
        if (form == 1 && !o_flag && memcmp(&g_acc[i], &o_acc[i], sizeof(float)) != 0) ++bad_acc;
        for (int k = 0; k < 3; ++k) {
            const double got = g_state[k][i], want = o_state[k][i];
            if (!(fabs(got - want) <= 1e-9 + 1e-6 * fabs(want))) ++bad_state;
        }
        if (ulp_distance_over_one(g_full[(size_t)RANK * S + i], o_own[i])) ++bad_own;
        for (int q = 0; q < WORLD; ++q)
            if (q != RANK && g_full[(size_t)q * S + i] != others[(size_t)q * S + i]) ++bad_other;
    }
    const int ok = path == want_path && (g_flag & 1) == o_flag && (g_flag & FP_FLAG_GAVE_UP) == 0 &&
                   bad_acc == 0 && bad_state == 0 && bad_own == 0 && bad_other == 0;
    printf("%s form=%s overflow=%d path=%d (want %d) flag=%d (oracle %d) mismatches: acc %lld state %lld "
           "own bf16 %lld other shards %lld\n",
           ok ? "ok  " : "FAIL", form == 0 ? "one-pass" : form == 1 ? "two-phase" : "speculative", inf, path,
           want_path, g_flag, o_flag, (long long)bad_acc, (long long)bad_state, (long long)bad_own,
           (long long)bad_other);

    HIP_OK(hipStreamDestroy(stream));
    (void)hipFree(d_grads);
    (void)hipFree(d_others);
    (void)hipFree(d_master);
    (void)hipFree(d_m);
    (void)hipFree(d_v);
    (void)hipFree(d_acc);
    (void)hipFree(d_full);
    (void)hipFree(d_flag);
    (void)hipFree(d_ws);
    for (int k = 0; k < 3; ++k) {
        if (d_out[k] != NULL) (void)hipFree(d_out[k]);
        free(g_state[k]);
    }
    free(grads);
    free(tmp);
    free(master);
    free(exp_avg);
    free(exp_avg_sq);
    free(others);
    free(g_acc);
    free(g_full);
    free(o_acc);
    free(o_own);
    return ok ? 0 : 1;
}

int step_abi_run(void) {
    int device_count = 0;
    if (hipGetDeviceCount(&device_count) != hipSuccess || device_count < 1) {
        fprintf(stderr, "no GPU\n");
        return 100;
    }
    int failures = 0;
    for (int inf = 0; inf < 2; ++inf) {
        const int32_t want[3] = {FP_PATH_ONE_PASS, FP_PATH_TWO_PHASE, FP_PATH_SPECULATIVE};
        for (int form = 0; form < 3; ++form) {
            const int r = run_case(form, inf, want[form]);
            if (r == CASE_ERROR) printf("FAIL form=%d overflow=%d: a call failed (above)\n", form, inf);
            failures += r != 0;
        }
    }
    printf("%s: %d case(s) failed\n", failures ? "FAIL" : "ok", failures);
    fflush(stdout);
    return failures;
}
