/*
 * worked_example.c -- drive libmha through its C ABI alone: device memory
 * from hipMalloc, the pages' hand-worked attention example in, the output
 * checked against that example's exact value.  No Python or torch.
 *
 * The example ("序列建模架构的演进与变革（二）" §4.3): one query q = [1, 0]
 * against four keys K = [[1,0],[0,1],[.7,.7],[1,0]] with values
 * V = [[2,1],[0,3],[1,2],[0,0]] and scale 1/sqrt(2).  Its exact output is
 * [0.850672, 1.240767] (the page rounds its intermediates and prints
 * [0.85, 1.25]).  The library takes heads of d = 64, so the vectors are
 * zero-padded: zero features add nothing to any dot product and give zero
 * output features.
 *
 * Build: gcc worked_example.c -I<include> -I/opt/rocm/include
 *        -D__HIP_PLATFORM_AMD__ -L<lib dir> -lmha -L/opt/rocm/lib -lamdhip64
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "libmha.h"

#define D 64
#define M 4

static int fail(const char *what, int code) {
    fprintf(stderr, "worked_example: %s (%d)\n", what, code);
    return 1;
}

int main(void) {
    float q[D] = {0}, k[M * D] = {0}, v[M * D] = {0}, o[D];
    const float K2[M][2] = {{1, 0}, {0, 1}, {0.7f, 0.7f}, {1, 0}};
    const float V2[M][2] = {{2, 1}, {0, 3}, {1, 2}, {0, 0}};
    const double want[2] = {0.850672, 1.240767};
    q[0] = 1.0f;
    for (int j = 0; j < M; ++j) {
        k[j * D] = K2[j][0];
        k[j * D + 1] = K2[j][1];
        v[j * D] = V2[j][0];
        v[j * D + 1] = V2[j][1];
    }
    const float scale = (float)(1.0 / sqrt(2.0));

    /* the host-side check alone needs no device memory */
    int st = mha_validate((void *)0x1000, (void *)0x2000, (void *)0x3000, NULL, 0, scale,
                          (void *)0x4000, 1, 1, 1, M, D, D, MHA_F32);
    if (st != MHA_OK) return fail(mha_status_string(st), st);
    st = mha_validate((void *)0x1000, (void *)0x2000, (void *)0x3000, NULL, 0, -1.0f,
                      (void *)0x4000, 1, 1, 1, M, D, D, MHA_F32);
    if (st != MHA_ERR_SCALE) return fail("a negative scale was not refused", st);

    void *dq, *dk, *dv, *dout;
    if (hipMalloc(&dq, sizeof q) != hipSuccess || hipMalloc(&dk, sizeof k) != hipSuccess ||
        hipMalloc(&dv, sizeof v) != hipSuccess || hipMalloc(&dout, sizeof o) != hipSuccess)
        return fail("hipMalloc", 0);
    hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice);
    hipMemcpy(dk, k, sizeof k, hipMemcpyHostToDevice);
    hipMemcpy(dv, v, sizeof v, hipMemcpyHostToDevice);

    st = mha_forward(dq, dk, dv, NULL, 0, scale, dout, 1, 1, 1, M, D, D, MHA_F32, NULL);
    if (st != MHA_OK) return fail(mha_status_string(st), st);
    if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", 0);
    hipMemcpy(o, dout, sizeof o, hipMemcpyDeviceToHost);

    int bad = 0;
    for (int c = 0; c < 2; ++c)
        if (fabs((double)o[c] - want[c]) > 1e-5) bad = 1;
    for (int c = 2; c < D; ++c)
        if (o[c] != 0.0f) bad = 1;
    printf("worked_example: O = [%.6f, %.6f], expected [%.6f, %.6f]\n", o[0], o[1], want[0],
           want[1]);

    /* bf16 (the round to nearest even is exact for these inputs but
       0.7, which rounds to 0.69921875; the check allows the bf16 budget) */
    unsigned short qb[D], kb[M * D], vb[M * D], ob[D];
    for (int c = 0; c < D; ++c) {
        unsigned int u;
        memcpy(&u, &q[c], 4);
        qb[c] = (unsigned short)((u + 0x7fff + ((u >> 16) & 1)) >> 16);
    }
    for (int e = 0; e < M * D; ++e) {
        unsigned int u;
        memcpy(&u, &k[e], 4);
        kb[e] = (unsigned short)((u + 0x7fff + ((u >> 16) & 1)) >> 16);
        memcpy(&u, &v[e], 4);
        vb[e] = (unsigned short)((u + 0x7fff + ((u >> 16) & 1)) >> 16);
    }
    hipMemcpy(dq, qb, sizeof qb, hipMemcpyHostToDevice);
    hipMemcpy(dk, kb, sizeof kb, hipMemcpyHostToDevice);
    hipMemcpy(dv, vb, sizeof vb, hipMemcpyHostToDevice);
    st = mha_forward(dq, dk, dv, NULL, 0, scale, dout, 1, 1, 1, M, D, D, MHA_BF16, NULL);
    if (st != MHA_OK) return fail(mha_status_string(st), st);
    if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", 0);
    hipMemcpy(ob, dout, sizeof ob, hipMemcpyDeviceToHost);
    for (int c = 0; c < 2; ++c) {
        unsigned int u = (unsigned int)ob[c] << 16;
        float f;
        memcpy(&f, &u, 4);
        printf("worked_example: bf16 O[%d] = %.6f\n", c, f);
        if (fabs((double)f - want[c]) > 1.5e-2) bad = 1;
    }

    hipFree(dq);
    hipFree(dk);
    hipFree(dv);
    hipFree(dout);
    if (bad) return fail("output differs from the worked example", 0);
    printf("worked_example: ok\n");
    return 0;
}
