/*
 * oracle.c -- plain, slow, scalar CPU oracle for the per-GPU local work of the
 * link-balanced sharded relay collectives (torchrec pull request #4570,
 * "Link-balance the sharded relay schedules (up to 3.2x vs NCCL)").
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the CPU
 * baseline leg of bench.py may load this library.  It shares no code, header,
 * table or constant with the HIP library under pack_rr_helper_amd/csrc/, and it
 * never reads anything that library produced.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (oracle/build.py).
 * No FMA contraction, no fast-math: every float operation below is one IEEE-754
 * binary32 operation in round-to-nearest-even, performed in the order written.
 *
 * Arithmetic contract (the reading this oracle implements):
 *   - inputs are fp32 or bf16; every reduction converts each input to fp32,
 *     folds left in ascending source-rank order in fp32, multiplies once by the
 *     op scale (SUM: 1, AVG: 1/A), and rounds once to the buffer dtype with
 *     round-to-nearest-even.
 *   - the A=4 reduce-scatter helper emits its partial sum in the buffer dtype
 *     (it travels over the wire), so that path rounds twice; it is *not* the
 *     plain reduce-scatter, and the tests bound its distance from it.
 *   - all-to-all pack/unpack move raw element bit patterns, never via float.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_*.py against
 * closed forms, printed constants, exact rational brute force or library
 * routines -- never against this file's own formulas.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_SUM = 0, ORC_AVG = 1 };
enum { ORC_ALLREDUCE = 0, ORC_REDUCE_SCATTER = 1, ORC_ALLTOALL = 2 };

/* ------------------------------------------------------------------------- */
/* bf16 codec.  bf16 is the top half of an IEEE binary32.                      */
/* ------------------------------------------------------------------------- */

float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest-even from binary32 to bf16.  A NaN keeps its sign and its
 * top payload bits and is made quiet. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* Correct rounding of a double to the buffer dtype, used only by the plain
 * (fp64) collective definitions.  binary64 -> binary32 uses round-to-odd and
 * then binary32 -> bf16 uses round-to-nearest-even; rounding to odd with at
 * least two extra bits before the final rounding gives the correctly rounded
 * result (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
 * proved algorithms using rounding to odd", IEEE TC 2008). */
static float f64_to_f32_odd(double d)
{
    float t = (float)d;
    if (isnan(d) || isinf(d) || (double)t == d)
        return t;
    if (isinf(t))  /* overflowed in nearest mode: take the largest finite */
        t = copysignf(3.40282347e+38f, t);
    else if (fabs((double)t) > fabs(d))
        t = nextafterf(t, 0.0f);
    uint32_t u;
    memcpy(&u, &t, sizeof u);
    u |= 1u;
    memcpy(&t, &u, sizeof t);
    return t;
}

static float ld(const void *p, int dt, int64_t i)
{
    if (dt == ORC_F32)
        return ((const float *)p)[i];
    return orc_bf16_to_f32(((const uint16_t *)p)[i]);
}

static void st(void *p, int dt, int64_t i, float v)
{
    if (dt == ORC_F32)
        ((float *)p)[i] = v;
    else
        ((uint16_t *)p)[i] = orc_f32_to_bf16(v);
}

static void st64(void *p, int dt, int64_t i, double v)
{
    if (dt == ORC_F32)
        ((float *)p)[i] = (float)v; /* one rounding, nearest-even */
    else
        ((uint16_t *)p)[i] = orc_f32_to_bf16(f64_to_f32_odd(v));
}

static int64_t esize(int dt) { return dt == ORC_F32 ? 4 : 2; }

static int64_t align_down_128(int64_t x) { return (x / 128) * 128; }

/* ------------------------------------------------------------------------- */
/* Geometry.                                                                   */
/* ------------------------------------------------------------------------- */

typedef struct {
    int64_t chunk;        /* per-helper relay chunk, elements; 0 = pure direct */
    int64_t relay_total;  /* relay region [0, relay_total) */
    int64_t direct_off;
    int64_t direct_len;
    int64_t dirA_off, dirA_len, dirB_off, dirB_len; /* A=2 direct split */
    int64_t dslice;       /* A=4: per-active direct slice (last one takes the rest) */
    int64_t helper_elems; /* helper scratch contract, elements */
    int32_t pure_direct;
    int32_t status;       /* 0 ok, 1 invalid */
} orc_geom;

/* The pages' Python helper sizing for passthrough helpers: A slots of one
 * 128-aligned chunk of count_g / num_chunks, never more than count_g itself
 * (sharded relay reduce-scatter tests commit and the all-to-all distributed
 * layer commit of the pull request). */
int64_t orc_passthrough_helper_size(int64_t count_g, int32_t A, int32_t num_chunks)
{
    int64_t slots = (int64_t)A * align_down_128(count_g / num_chunks);
    return count_g < slots ? count_g : slots;
}

/*
 * Geometry of one group, in the pages' terms.
 *   A=2, every collective (section 1 of the summary): chunk =
 *     align_down(count / numChunks, 128) with numChunks = H+2; chunks 0..H-1 are
 *     relayed through helper k; the direct exchange covers the rest, dirA = the
 *     chunk at index H and dirB = everything after it.  A zero chunk falls back
 *     to pure direct with dirA = half and dirB = the remainder (zero-chunk
 *     direct-fallback commit).
 *   A=4 allreduce (section 4): oChunk = align_down(count * permille / (1000 H), 128);
 *     per-rank inputs under 2 MiB take the pure-direct path.  The direct region
 *     is split evenly over the A actives, remainder to the last one.
 *   A=4 reduce-scatter (section 6): the same offload chunk of recvCount; the
 *     helper holds A(A-1) input chunks plus A reduced chunks inside the
 *     2 * recvCount contract.
 *   A=4 all-to-all (reverted section, all-to-all distributed layer commit):
 *     chunk = align_down(segmentCount / numChunks, 128), numChunks = H+1.
 */
int orc_geometry(int32_t A, int32_t H, int32_t numChunks, int32_t permille,
                 int64_t count, int32_t coll, int32_t dtype, orc_geom *g)
{
    memset(g, 0, sizeof *g);
    g->status = 1;
    if ((A != 2 && A != 4) || H < 1 || count < 0)
        return 1;
    if (coll < 0 || coll > 2 || (dtype != ORC_F32 && dtype != ORC_BF16))
        return 1;

    int64_t chunk = 0;
    if (A == 2) {
        if (numChunks < H + 2)
            return 1;
        chunk = align_down_128(count / numChunks);
    } else if (coll == ORC_ALLTOALL) {
        if (numChunks < H + 1)
            return 1;
        chunk = align_down_128(count / numChunks);
    } else {
        if (permille <= 0 || permille > 1000)
            return 1;
        int under_floor = (coll == ORC_ALLREDUCE) &&
                          (count * esize(dtype) < (int64_t)2 * 1024 * 1024);
        chunk = under_floor ? 0 : align_down_128(count * permille / (1000 * (int64_t)H));
        if (coll == ORC_REDUCE_SCATTER && (int64_t)A * A * chunk > 2 * count)
            return 1; /* scratch would not fit the 2 * recvCount contract */
    }

    g->chunk = chunk;
    g->pure_direct = chunk == 0;
    g->relay_total = (int64_t)H * chunk;
    g->direct_off = g->relay_total;
    g->direct_len = count - g->relay_total;

    if (A == 2) {
        if (chunk > 0) {
            g->dirA_off = (int64_t)H * chunk;
            g->dirA_len = chunk;
            g->dirB_off = (int64_t)(H + 1) * chunk;
            g->dirB_len = count - g->dirB_off;
        } else {
            g->dirA_off = 0;
            g->dirA_len = count / 2;
            g->dirB_off = g->dirA_len;
            g->dirB_len = count - g->dirA_len;
        }
        g->helper_elems = (int64_t)A * chunk;
    } else {
        if (coll != ORC_ALLTOALL)
            g->dslice = g->direct_len / A;
        if (coll == ORC_ALLREDUCE || coll == ORC_REDUCE_SCATTER)
            g->helper_elems = 2 * count;
        else
            g->helper_elems = (int64_t)A * (A - 1) * chunk;
    }
    g->status = 0;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* The one reduction rule every step uses:                                     */
/*   out[i] = RND( scale * ((in_0[i] + in_1[i]) + ... + in_{k-1}[i]) )         */
/* with fp32 adds in the listed order and one rounding to the dtype.           */
/* ------------------------------------------------------------------------- */

static void fold(int dt, int nin, const void *const *in, const int64_t *in_off,
                 int64_t n, float scale, void *out, int64_t out_off)
{
    for (int64_t i = 0; i < n; i++) {
        float acc = ld(in[0], dt, in_off[0] + i);
        for (int k = 1; k < nin; k++)
            acc = acc + ld(in[k], dt, in_off[k] + i);
        acc = acc * scale;
        st(out, dt, out_off + i, acc);
    }
}

static float op_scale(int op, int A) { return op == ORC_AVG ? 1.0f / (float)A : 1.0f; }

/* ------------------------------------------------------------------------- */
/* Steps, one per role (summary sections 2, 4, 6 and the reverted all-to-all).  */
/* Every buffer uses the layout of the rank that owns it.                      */
/* ------------------------------------------------------------------------- */

/* A=2 allreduce helper (section 2): both actives send chunk k, so the sum of
 * the two slots is already the allreduced chunk; the helper returns it to both.
 * For AVG the helper applies the 1/2 so the actives do no work over the
 * relayed part of the buffer. */
void orc_ar2_helper(int dt, int op, const void *slot0, const void *slot1,
                    int64_t n, void *out)
{
    const void *in[2] = {slot0, slot1};
    int64_t off[2] = {0, 0};
    fold(dt, 2, in, off, n, op_scale(op, 2), out, 0);
}

/* A>2 allreduce helper (section 4, flat helper-reduce-and-broadcast): the
 * helper sums the A active ranks' copies of its position slice. */
void orc_ar4_helper(int dt, int op, int A, const void *const *slots, int64_t n,
                    void *out)
{
    int64_t off[8] = {0};
    fold(dt, A, slots, off, n, op_scale(op, A), out, 0);
}

/* Active allreduce epilogue: the direct-exchange region.
 *   A=2: both actives reduce the whole direct region [direct_off, count).
 *   A=4: active a reduces its slice of the direct region (reduce-scatter over
 *        the intra links; the all-gather that follows moves bits only).
 * x[s] is source rank s's full buffer (count elements), out is the active's
 * full output; nothing outside the region is written. */
void orc_ar_active(int dt, int op, int A, int H, int numChunks, int permille,
                   int64_t count, int a, const void *const *x, void *out)
{
    orc_geom g;
    if (orc_geometry(A, H, numChunks, permille, count, ORC_ALLREDUCE, dt, &g))
        return;
    int64_t lo = g.direct_off, n = g.direct_len;
    if (A > 2) {
        lo = g.direct_off + (int64_t)a * g.dslice;
        n = (a == A - 1) ? g.direct_off + g.direct_len - lo : g.dslice;
    }
    int64_t off[8];
    for (int s = 0; s < A; s++)
        off[s] = lo;
    fold(dt, A, x, off, n, op_scale(op, A), out, lo);
}

/* A=2 reduce-scatter active epilogue (the fused add + scale of the relayed
 * chunks and the final reduction of the direct chunks): owner o adds the
 * other active's contribution to its own block.  blk[s] is source s's block
 * destined for this owner (recvCount elements). */
void orc_rs2_active(int dt, int op, const void *blk0, const void *blk1,
                    int64_t R, void *out)
{
    const void *in[2] = {blk0, blk1};
    int64_t off[2] = {0, 0};
    fold(dt, 2, in, off, R, op_scale(op, 2), out, 0);
}

/* A=4 reduce-scatter pass 1 at helper h (section 6): the scratch holds one
 * chunk per (owner, source) pair, owner-major, the sources of owner o being
 * the A-1 ranks other than o in ascending order.  Each owner's A-1 chunks are
 * summed into one reduced chunk; no scale here (it is applied once, by the
 * owner).  out holds A chunks, owner-major. */
void orc_rs4_pass1(int dt, int A, int64_t chunk, const void *scratch, void *out)
{
    for (int o = 0; o < A; o++) {
        const void *in[8];
        int64_t off[8];
        for (int j = 0; j < A - 1; j++) {
            in[j] = scratch;
            off[j] = ((int64_t)o * (A - 1) + j) * chunk;
        }
        fold(dt, A - 1, in, off, chunk, 1.0f, out, (int64_t)o * chunk);
    }
}

/* A=4 reduce-scatter pass 2 at owner o: the direct region sums the A sources'
 * blocks (blk[s] = source s's recvCount-element block destined for o); offload
 * slice h adds the owner's own block and helper h's reduced chunk red[h]. */
void orc_rs4_pass2(int dt, int op, int A, int H, int permille, int64_t R, int o,
                   const void *const *blk, const void *const *red, void *out)
{
    orc_geom g;
    if (orc_geometry(A, H, 0, permille, R, ORC_REDUCE_SCATTER, dt, &g))
        return;
    float scale = op_scale(op, A);
    for (int h = 0; h < H && g.chunk > 0; h++) {
        const void *in[2] = {blk[o], red[h]};
        int64_t off[2] = {(int64_t)h * g.chunk, 0};
        fold(dt, 2, in, off, g.chunk, scale, out, (int64_t)h * g.chunk);
    }
    int64_t off[8];
    for (int s = 0; s < A; s++)
        off[s] = g.direct_off;
    fold(dt, A, blk, off, g.direct_len, scale, out, g.direct_off);
}

/* All-to-all coalescing at helper slice h (reverted section: sources and destinations are both
 * laid out with a segmentCount stride).  src[s] holds A segments of seg elements, segment
 * d destined for rank d.  The per-destination buffer dst[d] receives the slice
 * h of every source other than d, in ascending source order. */
void orc_a2a_pack(int es, int A, int64_t seg, int64_t chunk, int h,
                  const void *const *src, void *const *dst)
{
    for (int d = 0; d < A; d++) {
        int j = 0;
        for (int s = 0; s < A; s++) {
            if (s == d)
                continue;
            const char *from = (const char *)src[s] + ((int64_t)d * seg + (int64_t)h * chunk) * es;
            char *to = (char *)dst[d] + ((int64_t)j * chunk) * es;
            for (int64_t b = 0; b < chunk * es; b++)
                to[b] = from[b];
            j++;
        }
    }
}

/* Inverse scatter: recv[d] (as packed for destination d) lands in rank d's
 * output at segment s_j, slice h. */
void orc_a2a_unpack(int es, int A, int64_t seg, int64_t chunk, int h,
                    const void *const *recv, void *const *out)
{
    for (int d = 0; d < A; d++) {
        int j = 0;
        for (int s = 0; s < A; s++) {
            if (s == d)
                continue;
            const char *from = (const char *)recv[d] + ((int64_t)j * chunk) * es;
            char *to = (char *)out[d] + ((int64_t)s * seg + (int64_t)h * chunk) * es;
            for (int64_t b = 0; b < chunk * es; b++)
                to[b] = from[b];
            j++;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Whole-group compositions: every rank of one group simulated in host memory, */
/* each point-to-point hop a plain copy.  scratch must hold the number of      */
/* bytes documented per function.                                              */
/* ------------------------------------------------------------------------- */

static void copy_elems(void *dst, int64_t doff, const void *src, int64_t soff,
                       int64_t n, int64_t es)
{
    memcpy((char *)dst + doff * es, (const char *)src + soff * es, (size_t)(n * es));
}

/* A=2 allreduce, reduce-at-helper (sections 1-2).  scratch: 2*chunk elements. */
int orc_ar2_group(int dt, int op, int H, int numChunks, int64_t count,
                  const void *x0, const void *x1, void *out0, void *out1,
                  void *scratch)
{
    orc_geom g;
    if (orc_geometry(2, H, numChunks, 0, count, ORC_ALLREDUCE, dt, &g))
        return 1;
    int64_t es = esize(dt);
    for (int k = 0; k < H && g.chunk > 0; k++) {
        /* phase 1: each active scatters chunk k to helper k's two slots */
        void *slot0 = scratch;
        void *slot1 = (char *)scratch + g.chunk * es;
        copy_elems(slot0, 0, x0, (int64_t)k * g.chunk, g.chunk, es);
        copy_elems(slot1, 0, x1, (int64_t)k * g.chunk, g.chunk, es);
        /* the helper reduces in place over slot 0 and returns it to both */
        orc_ar2_helper(dt, op, slot0, slot1, g.chunk, slot0);
        copy_elems(out0, (int64_t)k * g.chunk, slot0, 0, g.chunk, es);
        copy_elems(out1, (int64_t)k * g.chunk, slot0, 0, g.chunk, es);
    }
    const void *x[2] = {x0, x1};
    orc_ar_active(dt, op, 2, H, numChunks, 0, count, 0, x, out0);
    orc_ar_active(dt, op, 2, H, numChunks, 0, count, 1, x, out1);
    return 0;
}

/* A=2 reduce-scatter with passthrough helpers (section 2, last paragraph, and
 * the five phases of the reduce-scatter core commit).  x_a holds 2 blocks of R;
 * block b is destined for active b.  scratch: 4*R elements (two receive
 * buffers and the two helper slots). */
int orc_rs2_group(int dt, int op, int H, int numChunks, int64_t R,
                  const void *x0, const void *x1, void *out0, void *out1,
                  void *scratch)
{
    orc_geom g;
    if (orc_geometry(2, H, numChunks, 0, R, ORC_REDUCE_SCATTER, dt, &g))
        return 1;
    int64_t es = esize(dt);
    void *recv0 = scratch;                        /* a1's block 0, for a0 */
    void *recv1 = (char *)scratch + R * es;       /* a0's block 1, for a1 */
    void *slot0 = (char *)scratch + 2 * R * es;
    void *slot1 = (char *)scratch + 3 * R * es;
    for (int k = 0; k < H && g.chunk > 0; k++) {
        /* slot 0 carries what a0 adds into a1's block and slot 1 what a1 adds
         * into a0's block: they belong to different outputs, so the helper
         * forwards them unsummed */
        copy_elems(slot0, 0, x0, R + (int64_t)k * g.chunk, g.chunk, es);
        copy_elems(slot1, 0, x1, 0 + (int64_t)k * g.chunk, g.chunk, es);
        copy_elems(recv1, (int64_t)k * g.chunk, slot0, 0, g.chunk, es);
        copy_elems(recv0, (int64_t)k * g.chunk, slot1, 0, g.chunk, es);
    }
    /* direct exchange of the rest of each block */
    copy_elems(recv1, g.direct_off, x0, R + g.direct_off, g.direct_len, es);
    copy_elems(recv0, g.direct_off, x1, 0 + g.direct_off, g.direct_len, es);
    /* owners add in source-rank order */
    orc_rs2_active(dt, op, x0, recv0, R, out0);
    orc_rs2_active(dt, op, recv1, (const char *)x1 + R * es, R, out1);
    return 0;
}

/* A=4 allreduce (section 4; flat helper reduce and broadcast).
 * scratch: (A+1)*oChunk elements. */
int orc_ar4_group(int dt, int op, int H, int permille, int64_t count,
                  const void *const *x, void *const *out, void *scratch)
{
    const int A = 4;
    orc_geom g;
    if (orc_geometry(A, H, 0, permille, count, ORC_ALLREDUCE, dt, &g))
        return 1;
    int64_t es = esize(dt);
    for (int h = 0; h < H && g.chunk > 0; h++) {
        const void *slots[4];
        for (int a = 0; a < A; a++) {
            copy_elems(scratch, (int64_t)a * g.chunk, x[a], (int64_t)h * g.chunk, g.chunk, es);
            slots[a] = (char *)scratch + (int64_t)a * g.chunk * es;
        }
        void *red = (char *)scratch + (int64_t)A * g.chunk * es;
        orc_ar4_helper(dt, op, A, slots, g.chunk, red);
        for (int a = 0; a < A; a++)
            copy_elems(out[a], (int64_t)h * g.chunk, red, 0, g.chunk, es);
    }
    for (int a = 0; a < A; a++)
        orc_ar_active(dt, op, A, H, 0, permille, count, a, x, out[a]);
    /* all-gather of the reduced direct slices over the intra links */
    for (int a = 0; a < A; a++) {
        int64_t lo = g.direct_off + (int64_t)a * g.dslice;
        int64_t n = (a == A - 1) ? g.direct_off + g.direct_len - lo : g.dslice;
        for (int b = 0; b < A; b++)
            if (b != a)
                copy_elems(out[b], lo, out[a], lo, n, es);
    }
    return 0;
}

/* A=4 reduce-scatter, flat reduce-at-helper (section 6).  x[s] holds A blocks
 * of R.  scratch: 2*R elements (the helper contract) plus A*H*chunk elements
 * for the reduced chunks as delivered to the owners. */
int orc_rs4_group(int dt, int op, int H, int permille, int64_t R,
                  const void *const *x, void *const *out, void *scratch)
{
    const int A = 4;
    orc_geom g;
    if (orc_geometry(A, H, 0, permille, R, ORC_REDUCE_SCATTER, dt, &g))
        return 1;
    int64_t es = esize(dt);
    char *hbuf = (char *)scratch;                  /* one helper's 2R scratch */
    char *delivered = (char *)scratch + 2 * R * es; /* [owner][helper] chunks */
    for (int h = 0; h < H && g.chunk > 0; h++) {
        for (int o = 0; o < A; o++) {
            int j = 0;
            for (int s = 0; s < A; s++) {
                if (s == o)
                    continue;
                copy_elems(hbuf, ((int64_t)o * (A - 1) + j) * g.chunk, x[s],
                           (int64_t)o * R + (int64_t)h * g.chunk, g.chunk, es);
                j++;
            }
        }
        char *red = hbuf + (int64_t)A * (A - 1) * g.chunk * es;
        orc_rs4_pass1(dt, A, g.chunk, hbuf, red);
        for (int o = 0; o < A; o++)
            copy_elems(delivered, ((int64_t)o * H + h) * g.chunk, red,
                       (int64_t)o * g.chunk, g.chunk, es);
    }
    for (int o = 0; o < A; o++) {
        const void *blk[4];
        const void *red[16];
        for (int s = 0; s < A; s++)
            blk[s] = (const char *)x[s] + (int64_t)o * R * es;
        for (int h = 0; h < H; h++)
            red[h] = delivered + ((int64_t)o * H + h) * g.chunk * es;
        orc_rs4_pass2(dt, op, A, H, permille, R, o, blk, red, out[o]);
    }
    return 0;
}

/* A=4 all-to-all with helper coalescing: every helper slice packed and
 * unpacked, the direct region and the rank's own segment copied straight.
 * scratch: A*(A-1)*chunk*es bytes. */
int orc_a2a_group(int es, int A, int H, int numChunks, int64_t seg,
                  const void *const *src, void *const *out, void *scratch)
{
    orc_geom g;
    if (orc_geometry(A, H, numChunks, 0, seg, ORC_ALLTOALL,
                     es == 4 ? ORC_F32 : ORC_BF16, &g))
        return 1;
    void *dst[8];
    for (int d = 0; d < A; d++)
        dst[d] = (char *)scratch + (int64_t)d * (A - 1) * g.chunk * es;
    for (int h = 0; h < H && g.chunk > 0; h++) {
        orc_a2a_pack(es, A, seg, g.chunk, h, src, dst);
        orc_a2a_unpack(es, A, seg, g.chunk, h, (const void *const *)dst, out);
    }
    for (int d = 0; d < A; d++)
        for (int s = 0; s < A; s++) {
            int64_t lo = (s == d) ? 0 : g.direct_off;
            copy_elems(out[d], (int64_t)s * seg + lo, src[s], (int64_t)d * seg + lo,
                       seg - lo, es);
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Plain collective definitions, fp64 accumulation, one correct rounding.      */
/* ------------------------------------------------------------------------- */

/* out[i] = RND(scale * sum_s x_s[off + i]) */
void orc_plain_sum(int dt, int op, int A, const void *const *x, int64_t off,
                   int64_t n, void *out)
{
    double scale = op == ORC_AVG ? 1.0 / (double)A : 1.0;
    for (int64_t i = 0; i < n; i++) {
        double acc = 0.0;
        for (int s = 0; s < A; s++)
            acc += (double)ld(x[s], dt, off + i);
        st64(out, dt, i, acc * scale);
    }
}

/* out_d[s*seg + p] = x_s[d*seg + p] */
void orc_plain_all_to_all(int es, int A, int64_t seg, int d,
                          const void *const *x, void *out)
{
    for (int s = 0; s < A; s++)
        copy_elems(out, (int64_t)s * seg, x[s], (int64_t)d * seg, seg, es);
}

/* Element-wise codec over arrays (for the exhaustive codec pins). */
void orc_bf16_to_f32_array(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_bf16_to_f32(in[i]);
}

void orc_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_f32_to_bf16(in[i]);
}

int orc_abi_version(void) { return 1; }
