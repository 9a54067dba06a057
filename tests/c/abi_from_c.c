/*
 * A plain C caller of the library's ABI (include/os_softmax.h): device
 * buffers from the HIP runtime's C API, os_softmax_fwd on the AUTO path for
 * three shapes (one per path: resident, stream, split with a workspace the
 * caller sizes with os_softmax_workspace_bytes), checked against the fp64
 * oracle (oracle/oracle.h, test infrastructure) on the same input bytes:
 * fp32 y within 1e-6 + 1e-5 |y|, bf16 y within one bf16 step of the
 * rounded reference, m equal to the row max bit for bit, lse within
 * 1e-5 + 2 ulp.  Inputs come from a 64-bit linear congruential generator
 * (data only).  Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "os_softmax.h"
#include "../../oracle/oracle.h"

static uint64_t lcg_state;
static double uniform01(void) {
    lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(lcg_state >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

static float bf16_to_f32(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ordered distance between two bf16 bit patterns of finite values */
static int32_t bf16_steps(uint16_t a, uint16_t b) {
    const int32_t ia = (a & 0x8000) ? -(int32_t)(a & 0x7fff) : (int32_t)a;
    const int32_t ib = (b & 0x8000) ? -(int32_t)(b & 0x7fff) : (int32_t)b;
    return ia > ib ? ia - ib : ib - ia;
}

#define HIP_OK(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));      \
            return 1;                                                       \
        }                                                                   \
    } while (0)

static int run_case(int64_t M, int64_t N, os_dtype dt, uint64_t seed) {
    const size_t es = dt == OS_F32 ? 4 : 2, n = (size_t)(M * N);
    void *xh = malloc(n * es), *yh = malloc(n * es);
    double *yr = malloc(n * sizeof(double));
    double *mr = malloc((size_t)M * sizeof(double)), *lr = malloc((size_t)M * sizeof(double));
    float *mh = malloc((size_t)M * 4), *lh = malloc((size_t)M * 4);
    if (!xh || !yh || !yr || !mr || !lr || !mh || !lh) return 1;
    lcg_state = seed;
    for (size_t i = 0; i < n; ++i) {
        const float v = (float)(8.0 * uniform01() - 4.0);
        if (dt == OS_F32) ((float *)xh)[i] = v;
        else ((uint16_t *)xh)[i] = f32_to_bf16_rne(v);
    }

    void *x, *y, *ws = NULL;
    float *m, *lse;
    HIP_OK(hipMalloc(&x, n * es));
    HIP_OK(hipMalloc(&y, n * es));
    HIP_OK(hipMalloc((void **)&m, (size_t)M * 4));
    HIP_OK(hipMalloc((void **)&lse, (size_t)M * 4));
    const size_t wsb = os_softmax_workspace_bytes(M, N, dt, OS_PATH_AUTO);
    if (wsb) HIP_OK(hipMalloc(&ws, wsb));
    HIP_OK(hipMemcpy(x, xh, n * es, hipMemcpyHostToDevice));
    const os_path path = os_softmax_select_path(M, N, dt);
    const os_status st = os_softmax_fwd(x, N, y, N, M, N, dt, m, NULL, lse,
                                        ws, wsb, NULL);
    if (st != OS_OK) {
        fprintf(stderr, "os_softmax_fwd: %s\n", os_status_string(st));
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(yh, y, n * es, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(mh, m, (size_t)M * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lh, lse, (size_t)M * 4, hipMemcpyDeviceToHost));

    if (oracle_softmax(xh, N, M, N, dt == OS_F32 ? ORACLE_F32 : ORACLE_BF16,
                       yr, mr, NULL, lr) != ORACLE_OK)
        return 1;
    double worst = 0.0;
    int32_t worst_steps = 0;
    for (size_t i = 0; i < n; ++i) {
        if (dt == OS_F32) {
            const double e = fabs((double)((float *)yh)[i] - yr[i]);
            if (!(e <= 1e-6 + 1e-5 * fabs(yr[i]))) {
                fprintf(stderr, "y[%zu] = %.9g, oracle %.17g\n", i,
                        (double)((float *)yh)[i], yr[i]);
                return 1;
            }
            if (e > worst) worst = e;
        } else {
            const uint16_t want = f32_to_bf16_rne((float)yr[i]);
            const int32_t s = bf16_steps(((uint16_t *)yh)[i], want);
            if (s > 1) {
                fprintf(stderr, "y[%zu] = %.9g, oracle %.17g (%d bf16 steps)\n", i,
                        (double)bf16_to_f32(((uint16_t *)yh)[i]), yr[i], s);
                return 1;
            }
            if (s > worst_steps) worst_steps = s;
        }
    }
    for (int64_t r = 0; r < M; ++r) {
        if ((double)mh[r] != mr[r]) {
            fprintf(stderr, "m[%lld] = %.9g, row max %.17g\n", (long long)r,
                    (double)mh[r], mr[r]);
            return 1;
        }
        const double tol = 1e-5 + 2.0 * (nextafterf(fabsf((float)lr[r]), INFINITY) - fabsf((float)lr[r]));
        if (!(fabs((double)lh[r] - lr[r]) <= tol)) {
            fprintf(stderr, "lse[%lld] = %.9g, oracle %.17g\n", (long long)r,
                    (double)lh[r], lr[r]);
            return 1;
        }
    }
    printf("%s %lldx%lld path %d (workspace %zu B): y within %s %.3g, m exact, lse within bound\n",
           dt == OS_F32 ? "fp32" : "bf16", (long long)M, (long long)N, (int)path, wsb,
           dt == OS_F32 ? "abs" : "bf16 steps", dt == OS_F32 ? worst : (double)worst_steps);
    HIP_OK(hipFree(x));
    HIP_OK(hipFree(y));
    HIP_OK(hipFree(m));
    HIP_OK(hipFree(lse));
    if (ws) HIP_OK(hipFree(ws));
    free(xh); free(yh); free(yr); free(mr); free(lr); free(mh); free(lh);
    return 0;
}

int main(void) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        fprintf(stderr, "no HIP device\n");
        return 2;
    }
    HIP_OK(hipSetDevice(0));
    if (run_case(600, 3001, OS_F32, 11)) return 1;    /* resident */
    if (run_case(520, 40000, OS_BF16, 12)) return 1;  /* stream (many long rows) */
    if (run_case(3, 300001, OS_F32, 13)) return 1;    /* split, with a workspace */
    printf("C caller: all checks hold\n");
    return 0;
}
