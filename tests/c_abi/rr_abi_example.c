/*
 * rr_abi_example.c -- the relay library driven from plain C11, with no
 * Python and no torch: device memory from hipMalloc, one HIP stream, and
 * the entry points declared in include/rr.h.  Expected values come from the
 * CPU oracle's C library (test infrastructure) on the same input bytes.
 *
 *   rr_abi_example host   checks that need no GPU: ABI version, geometry of
 *                         the A=2 epilogue configuration (count 2^25, eight
 *                         chunks of 2^22), and argument errors reported
 *                         before any HIP call
 *   rr_abi_example gpu    runs a batched A=2 allreduce helper reduction, the
 *                         A=4 reduce-scatter pass 1 and a ragged all-to-all
 *                         pack and unpack on the GPU and compares every
 *                         output element bit for bit with the oracle
 *
 * Exit status 0 on success; otherwise the first failing check is printed.
 */
#include <hip/hip_runtime_api.h>
#include <inttypes.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rr.h"

/* The oracle library's entry points used here (oracle/oracle.c). */
void orc_ar2_helper(int dt, int op, const void *slot0, const void *slot1, int64_t n, void *out);
void orc_rs4_pass1(int dt, int A, int64_t chunk, const void *scratch, void *out);
void orc_a2a_pack(int es, int A, int64_t seg, int64_t chunk, int h, const void *const *src,
                  void *const *dst);
void orc_a2a_unpack(int es, int A, int64_t seg, int64_t chunk, int h, const void *const *recv,
                    void *const *out);

static int failures = 0;

#define CHECK(cond, ...)                                                                   \
    do {                                                                                   \
        if (!(cond)) {                                                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);                           \
            fprintf(stderr, __VA_ARGS__);                                                  \
            fprintf(stderr, "\n");                                                         \
            ++failures;                                                                    \
            return 1;                                                                      \
        }                                                                                  \
    } while (0)

#define HIP(call)                                                                          \
    do {                                                                                   \
        hipError_t e_ = (call);                                                            \
        CHECK(e_ == hipSuccess, "%s: %s", #call, hipGetErrorString(e_));                   \
    } while (0)

/* splitmix64: the input generator of this program (inputs only). */
static uint64_t mix_state;
static uint64_t mix_next(void)
{
    uint64_t z = (mix_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Finite bf16 patterns of magnitude 2^-7 .. 2^7, both signs. */
static void fill_bf16(uint16_t *p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = mix_next();
        uint16_t sign = (uint16_t)(r & 1), expo = (uint16_t)(120 + (r >> 1) % 15);
        p[i] = (uint16_t)(sign << 15 | expo << 7 | ((r >> 8) & 0x7F));
    }
}

static void fill_bits(uint16_t *p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        p[i] = (uint16_t)mix_next();
}

static int same(const void *a, const void *b, size_t bytes, const char *what)
{
    const unsigned char *x = a, *y = b;
    for (size_t i = 0; i < bytes; ++i)
        CHECK(x[i] == y[i], "%s: byte %zu differs (%u vs %u)", what, i, x[i], y[i]);
    return 0;
}

/* ------------------------------------------------------------------------ */

static int host_checks(void)
{
    CHECK(rr_abi_version() == RR_ABI_VERSION, "ABI version %d", rr_abi_version());

    rr_relay r = {2, 6, 8, 0, INT64_C(1) << 25};
    rr_geom g;
    CHECK(rr_geometry(&r, RR_ALLREDUCE, RR_BF16, &g) == RR_OK, "geometry: %s", rr_last_error());
    CHECK(g.chunk == (INT64_C(1) << 22), "chunk %" PRId64, g.chunk);
    CHECK(g.relay_total == 6 * g.chunk && g.dirA_off == 6 * g.chunk && g.dirA_len == g.chunk &&
              g.dirB_off == 7 * g.chunk && g.dirB_len == g.chunk && !g.pure_direct,
          "A=2 regions");

    rr_relay bad = {3, 5, 8, 0, 4096};
    CHECK(rr_geometry(&bad, RR_ALLREDUCE, RR_BF16, &g) == RR_EINVAL, "A=3 accepted");
    CHECK(strlen(rr_last_error()) > 0, "no message for A=3");
    CHECK(rr_geometry(NULL, RR_ALLREDUCE, RR_BF16, &g) == RR_EINVAL, "null relay accepted");

    /* Fake, aligned addresses: every call below is rejected during validation,
     * before anything could touch them. */
    const uintptr_t B = (uintptr_t)1 << 40;
    const void *slots[2] = {(const void *)B, (const void *)(B + (16u << 20))};
    rr_relay r2 = {2, 6, 8, 0, 8 << 20};
    CHECK(rr_helper_reduce(&r2, RR_ALLREDUCE, RR_BF16, RR_SUM, 0, slots, 3,
                           (void *)(B + (64u << 20)), NULL) == RR_EINVAL,
          "nSlots=3 accepted");
    CHECK(rr_helper_reduce(&r2, RR_ALLREDUCE, RR_BF16, RR_SUM, 0, slots, 2, (void *)(B + 2),
                           NULL) == RR_EALIAS,
          "partial overlap accepted");
    CHECK(rr_helper_reduce(&r2, RR_REDUCE_SCATTER, RR_BF16, RR_SUM, 0, slots, 2,
                           (void *)(B + (64u << 20)), NULL) == RR_EINVAL,
          "A=2 reduce-scatter helper reduction accepted");
    rr_relay r4 = {4, 4, 5, 0, 5 * 128 * 4};
    const void *src[4] = {(const void *)B, (const void *)(B + 4096), (const void *)(B + 8192),
                          (const void *)(B + 12288)};
    void *dst[4] = {(void *)B, (void *)(B + 65536), (void *)(B + 131072), (void *)(B + 196608)};
    CHECK(rr_a2a_pack(&r4, RR_BF16, 0, src, dst, NULL) == RR_EALIAS, "in-place pack accepted");
    CHECK(rr_helper_reduce_many(RR_ALLREDUCE, RR_BF16, RR_SUM, NULL, 1, NULL) == RR_EINVAL,
          "null job array accepted");
    CHECK(rr_phase_reduce_many(RR_ALLREDUCE, RR_BF16, RR_SUM, NULL, 0, NULL, 1, NULL) == RR_EINVAL,
          "null active job array accepted");
    /* plans: sizes, and misuse rejected before anything runs */
    CHECK(rr_plan_bytes(0) == 0 && rr_plan_bytes(RR_PLAN_MAX_LAUNCHES + 1) == 0 &&
              rr_plan_bytes(2) > rr_plan_bytes(1), "plan sizes");
    CHECK(rr_plan_end(NULL) == RR_EINVAL, "plan end without a recording accepted");
    CHECK(rr_plan_launch(NULL, NULL) == RR_EINVAL, "null plan launched");
    {
        uint64_t small[4] = {0, 0, 0, 0};
        CHECK(rr_plan_begin(small, sizeof small) == RR_EINVAL, "plan buffer without room accepted");
        CHECK(rr_plan_launch(small, NULL) == RR_EINVAL, "a buffer that is no plan launched");
    }
    CHECK(rr_phase_reduce_many(RR_ALLREDUCE, RR_BF16, RR_SUM, NULL, 0, NULL, 0, NULL) == RR_OK,
          "empty phase call rejected: %s", rr_last_error());
    return 0;
}

/* ------------------------------------------------------------------------ */

static int gpu_helper_reduce(hipStream_t st)
{
    const int H = 6;
    const int64_t count = (INT64_C(1) << 22) + 12345;
    rr_relay r = {2, H, 8, 0, count};
    rr_geom g;
    CHECK(rr_geometry(&r, RR_ALLREDUCE, RR_BF16, &g) == RR_OK, "%s", rr_last_error());
    const int64_t c = g.chunk;
    const size_t bytes = (size_t)count * 2, cb = (size_t)c * 2;

    uint16_t *x0 = malloc(bytes), *x1 = malloc(bytes), *got = malloc(cb), *ref = malloc(cb);
    CHECK(x0 && x1 && got && ref, "host allocation");
    fill_bf16(x0, count);
    fill_bf16(x1, count);
    void *d0, *d1, *dout;
    HIP(hipMalloc(&d0, bytes));
    HIP(hipMalloc(&d1, bytes));
    HIP(hipMalloc(&dout, cb * H));
    HIP(hipMemcpy(d0, x0, bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d1, x1, bytes, hipMemcpyHostToDevice));

    rr_helper_job jobs[6];
    for (int k = 0; k < H; ++k) {
        memset(&jobs[k], 0, sizeof jobs[k]);
        jobs[k].relay = r;
        jobs[k].helper = k;
        jobs[k].nSlots = 2;
        jobs[k].slots[0] = (char *)d0 + k * cb;
        jobs[k].slots[1] = (char *)d1 + k * cb;
        jobs[k].out = (char *)dout + k * cb;
    }
    CHECK(rr_helper_reduce_many(RR_ALLREDUCE, RR_BF16, RR_AVG, jobs, H, st) == RR_OK, "%s",
          rr_last_error());
    HIP(hipStreamSynchronize(st));
    for (int k = 0; k < H; ++k) {
        HIP(hipMemcpy(got, (char *)dout + k * cb, cb, hipMemcpyDeviceToHost));
        orc_ar2_helper(RR_BF16, RR_AVG, x0 + k * c, x1 + k * c, c, ref);
        if (same(got, ref, cb, "A=2 helper reduce"))
            return 1;
    }
    HIP(hipFree(d0));
    HIP(hipFree(d1));
    HIP(hipFree(dout));
    free(x0), free(x1), free(got), free(ref);
    printf("A=2 allreduce helpers (6 jobs, one call): bit-exact\n");
    return 0;
}

static int gpu_rs4_pass1(hipStream_t st)
{
    const int A = 4;
    const int64_t R = (INT64_C(1) << 20) + 8 * 128 * 3;
    rr_relay r = {A, 4, 0, 500, R};
    rr_geom g;
    CHECK(rr_geometry(&r, RR_REDUCE_SCATTER, RR_BF16, &g) == RR_OK, "%s", rr_last_error());
    const int64_t c = g.chunk, n_in = (int64_t)A * (A - 1) * c;
    const size_t sb = (size_t)(2 * R) * 2, ob = (size_t)(A * c) * 2;
    uint16_t *scratch = calloc((size_t)(2 * R), 2), *got = malloc(ob), *ref = malloc(ob);
    CHECK(scratch && got && ref, "host allocation");
    fill_bf16(scratch, n_in);
    void *ds;
    HIP(hipMalloc(&ds, sb));
    HIP(hipMemcpy(ds, scratch, sb, hipMemcpyHostToDevice));
    const void *in[1] = {ds};
    CHECK(rr_rs_multi_reduce(&r, RR_BF16, RR_SUM, 1, 2, in, 1, (char *)ds + n_in * 2, st) == RR_OK,
          "%s", rr_last_error());
    HIP(hipStreamSynchronize(st));
    HIP(hipMemcpy(got, (char *)ds + n_in * 2, ob, hipMemcpyDeviceToHost));
    orc_rs4_pass1(RR_BF16, A, c, scratch, ref);
    if (same(got, ref, ob, "A=4 reduce-scatter pass 1"))
        return 1;
    HIP(hipFree(ds));
    free(scratch), free(got), free(ref);
    printf("A=4 reduce-scatter pass 1: bit-exact\n");
    return 0;
}

static int gpu_a2a(hipStream_t st)
{
    enum { A = 4, H = 4 };
    const int64_t seg = 5 * 128 * 300 + 3; /* off the 16-byte grid: realigned moves */
    rr_relay r = {A, H, 5, 0, seg};
    rr_geom g;
    CHECK(rr_geometry(&r, RR_ALLTOALL, RR_BF16, &g) == RR_OK, "%s", rr_last_error());
    const int64_t c = g.chunk;
    const size_t full = (size_t)(A * seg) * 2, packed = (size_t)((A - 1) * c) * 2;

    uint16_t *hs[A], *hout[A], *ref_out[A], *got = malloc(full), *ref_pk[A];
    void *ds[A], *dpk[H][A], *dout[A];
    CHECK(got != NULL, "host allocation");
    for (int s = 0; s < A; ++s) {
        hs[s] = malloc(full);
        hout[s] = malloc(full);
        ref_out[s] = calloc(1, full);
        ref_pk[s] = malloc(packed);
        CHECK(hs[s] && hout[s] && ref_out[s] && ref_pk[s], "host allocation");
        fill_bits(hs[s], A * seg);
        HIP(hipMalloc(&ds[s], full));
        HIP(hipMalloc(&dout[s], full));
        HIP(hipMemcpy(ds[s], hs[s], full, hipMemcpyHostToDevice));
        HIP(hipMemset(dout[s], 0, full));
    }
    for (int h = 0; h < H; ++h)
        for (int d = 0; d < A; ++d)
            HIP(hipMalloc(&dpk[h][d], packed));

    /* one job per helper slice; each job points at host arrays of A device pointers */
    const void *pin[H][A], *uin[H][A];
    void *pout[H][A], *uout[H][A];
    rr_a2a_job pj[H], uj[H];
    for (int h = 0; h < H; ++h) {
        for (int s = 0; s < A; ++s) {
            pin[h][s] = ds[s];
            pout[h][s] = dpk[h][s];
            uin[h][s] = dpk[h][s];
            uout[h][s] = dout[s];
        }
        memset(&pj[h], 0, sizeof pj[h]);
        pj[h].relay = r;
        pj[h].helper = h;
        uj[h] = pj[h];
        pj[h].in = pin[h];
        pj[h].out = pout[h];
        uj[h].in = uin[h];
        uj[h].out = uout[h];
    }
    /* both calls recorded into one caller-owned plan (validated once), then
       launched with a single call */
    const size_t plan_bytes = rr_plan_bytes(8);
    void *plan = malloc(plan_bytes);
    int32_t launches = -1;
    CHECK(plan != NULL && plan_bytes > 0, "plan allocation");
    CHECK(rr_plan_begin(plan, plan_bytes) == RR_OK, "%s", rr_last_error());
    CHECK(rr_a2a_pack_many(RR_BF16, pj, H, st) == RR_OK, "%s", rr_last_error());
    CHECK(rr_a2a_unpack_many(RR_BF16, uj, H, st) == RR_OK, "%s", rr_last_error());
    CHECK(rr_plan_end(&launches) == RR_OK && launches == 2, "plan end: %d launches, %s", launches,
          rr_last_error());
    HIP(hipStreamSynchronize(st));
    for (int d = 0; d < A; ++d) {  /* recording enqueued nothing */
        HIP(hipMemcpy(hout[d], dout[d], full, hipMemcpyDeviceToHost));
        if (same(hout[d], ref_out[d], full, "all-to-all output before the plan is launched"))
            return 1;
    }
    CHECK(rr_plan_launch(plan, st) == RR_OK, "%s", rr_last_error());
    HIP(hipStreamSynchronize(st));
    free(plan);

    const void *srcs[A] = {hs[0], hs[1], hs[2], hs[3]};
    void *pks[A] = {ref_pk[0], ref_pk[1], ref_pk[2], ref_pk[3]};
    void *outs[A] = {ref_out[0], ref_out[1], ref_out[2], ref_out[3]};
    for (int h = 0; h < H; ++h) {
        orc_a2a_pack(2, A, seg, c, h, srcs, pks);
        for (int d = 0; d < A; ++d) {
            HIP(hipMemcpy(got, dpk[h][d], packed, hipMemcpyDeviceToHost));
            if (same(got, ref_pk[d], packed, "all-to-all pack"))
                return 1;
        }
        orc_a2a_unpack(2, A, seg, c, h, (const void *const *)pks, outs);
    }
    for (int d = 0; d < A; ++d) {
        HIP(hipMemcpy(hout[d], dout[d], full, hipMemcpyDeviceToHost));
        if (same(hout[d], ref_out[d], full, "all-to-all unpack"))
            return 1;
    }
    for (int s = 0; s < A; ++s) {
        HIP(hipFree(ds[s]));
        HIP(hipFree(dout[s]));
        free(hs[s]), free(hout[s]), free(ref_out[s]), free(ref_pk[s]);
    }
    for (int h = 0; h < H; ++h)
        for (int d = 0; d < A; ++d)
            HIP(hipFree(dpk[h][d]));
    free(got);
    printf("A=4 all-to-all pack + unpack, segmentCount %" PRId64 ", one recorded plan: bit-exact\n", seg);
    return 0;
}

int main(int argc, char **argv)
{
    mix_state = 0x5EEDull;
    if (argc != 2 || (strcmp(argv[1], "host") && strcmp(argv[1], "gpu"))) {
        fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
        return 2;
    }
    if (!strcmp(argv[1], "host")) {
        host_checks();
    } else {
        hipStream_t st;
        if (hipStreamCreate(&st) != hipSuccess) {
            fprintf(stderr, "FAIL: no HIP device\n");
            return 1;
        }
        if (!gpu_helper_reduce(st) && !gpu_rs4_pass1(st))
            gpu_a2a(st);
        (void)hipStreamDestroy(st);
    }
    if (failures == 0)
        printf("%s checks passed\n", argv[1]);
    return failures ? 1 : 0;
}
