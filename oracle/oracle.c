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
/* Plain collective definitions: the exact sum, rounded once.                  */
/* ------------------------------------------------------------------------- */

/*
 * Every finite binary32 value (and so every bf16 value) is an integer multiple
 * of 2^-149, the least binary32 subnormal, and is smaller than 2^128 in
 * magnitude.  The plain definition therefore sums the inputs exactly as a
 * two's complement fixed-point integer whose unit is 2^-149: FX_LIMBS words of
 * 32 bits hold 2^277 times any number of terms up to 2^42 with room for the
 * sign.  No floating-point operation is involved until the single rounding.
 */
#define FX_LIMBS 10
typedef struct { uint32_t w[FX_LIMBS]; } fx_int;  /* w[0] least significant */

/* acc += sign * (mag << sh), mag < 2^32, 0 <= sh < 32*FX_LIMBS - 64. */
static void fx_add_shifted(fx_int *acc, int negative, uint32_t mag, int sh)
{
    int limb = sh / 32;
    uint64_t v = (uint64_t)mag << (sh % 32);  /* at most 63 bits */
    uint32_t part[3] = {(uint32_t)v, (uint32_t)(v >> 32), 0};
    if (!negative) {
        uint64_t carry = 0;
        for (int i = limb; i < FX_LIMBS; i++) {
            uint64_t t = (uint64_t)acc->w[i] + (i - limb < 3 ? part[i - limb] : 0) + carry;
            acc->w[i] = (uint32_t)t;
            carry = t >> 32;
        }
    } else {
        uint64_t borrow = 0;
        for (int i = limb; i < FX_LIMBS; i++) {
            uint64_t sub = (uint64_t)(i - limb < 3 ? part[i - limb] : 0) + borrow;
            borrow = (uint64_t)acc->w[i] < sub;
            acc->w[i] = (uint32_t)((uint64_t)acc->w[i] - sub);
        }
    }
}

static int fx_is_negative(const fx_int *a) { return (a->w[FX_LIMBS - 1] >> 31) & 1u; }

static int fx_is_zero(const fx_int *a)
{
    for (int i = 0; i < FX_LIMBS; i++)
        if (a->w[i])
            return 0;
    return 1;
}

static void fx_negate(fx_int *a)
{
    uint64_t carry = 1;
    for (int i = 0; i < FX_LIMBS; i++) {
        uint64_t t = (uint64_t)(uint32_t)~a->w[i] + carry;
        a->w[i] = (uint32_t)t;
        carry = t >> 32;
    }
}

/* a = a / d (a >= 0, 0 < d < 2^31); returns the remainder. */
static uint32_t fx_divmod_small(fx_int *a, uint32_t d)
{
    uint64_t rem = 0;
    for (int i = FX_LIMBS - 1; i >= 0; i--) {
        uint64_t cur = (rem << 32) | a->w[i];
        a->w[i] = (uint32_t)(cur / d);
        rem = cur % d;
    }
    return (uint32_t)rem;
}

static int fx_bit(const fx_int *a, int i) { return (int)((a->w[i / 32] >> (i % 32)) & 1u); }

/* Number of significant bits of a >= 0 (0 for a == 0). */
static int fx_bitlen(const fx_int *a)
{
    for (int i = FX_LIMBS - 1; i >= 0; i--)
        if (a->w[i])
            for (int b = 31; b >= 0; b--)
                if ((a->w[i] >> b) & 1u)
                    return 32 * i + b + 1;
    return 0;
}

/* Any of bits [0, n) of a >= 0 set. */
static int fx_any_below(const fx_int *a, int n)
{
    for (int i = 0; i < n; i++)
        if (fx_bit(a, i))
            return 1;
    return 0;
}

/* Bits [lo, lo + 32) of a >= 0 (lo >= 0). */
static uint32_t fx_bits_at(const fx_int *a, int lo)
{
    uint32_t r = 0;
    for (int b = 0; b < 32 && lo + b < 32 * FX_LIMBS; b++)
        r |= (uint32_t)fx_bit(a, lo + b) << b;
    return r;
}

/*
 * Round the exact value  sign * (q + rem/d) * 2^-149  to the binary format
 * with p significant bits (24: binary32, 8: bf16), exponent range
 * [-126, 127], round-to-nearest with ties to even (IEEE 754-2019 clause
 * 4.3.1), gradual underflow, overflow to infinity.  Returns the format's bit
 * pattern (32 or 16 bits wide).
 */
static uint32_t fx_round(const fx_int *q, uint32_t rem, uint32_t d, int negative, int p)
{
    const int width = p == 24 ? 32 : 16, man = p - 1;
    const uint32_t sign = negative ? 1u << (width - 1) : 0u;
    const int L = fx_bitlen(q);
    /* exponent of the leading bit, in units of 2^-149; values under 2^-126 use
       the subnormal quantum */
    int lead = L - 1 - 149;
    if (L == 0 || lead < -126)
        lead = -126;
    const int s = lead - (p - 1) + 149;  /* quantum = 2^(s - 149), s >= 0 */
    /* q >> s: at most p bits, since s >= L - p */
    uint64_t r = (uint64_t)fx_bits_at(q, s) & ((1ull << p) - 1);
    int above_half, at_half;
    if (s == 0) {
        above_half = 2ull * rem > d;
        at_half = 2ull * rem == d;
    } else {
        const int round_bit = fx_bit(q, s - 1);
        const int sticky = fx_any_below(q, s - 1) || rem != 0;
        above_half = round_bit && sticky;
        at_half = round_bit && !sticky;
    }
    if (above_half || (at_half && (r & 1u)))
        r += 1;
    int e = s;
    if (r == (1ull << p)) {  /* carried into the next binade */
        r >>= 1;
        e += 1;
    }
    if (r == 0)
        return sign;  /* underflow to a zero of the value's sign */
    if (r < (1ull << man))  /* subnormal: exponent field 0 */
        return sign | (uint32_t)r;
    const int biased = e - 149 + (p - 1) + 127;  /* exponent of r * 2^(e-149) */
    if (biased >= 255)
        return sign | (0xFFu << man);
    return sign | ((uint32_t)biased << man) | ((uint32_t)r - (1u << man));
}

/* out[i] = RND(sum_s x_s[off + i] / D), D = A for AVG and 1 for SUM: the
 * inputs summed exactly, then rounded once to the buffer dtype.  NaN inputs,
 * and +inf with -inf, give the default quiet NaN; otherwise an infinite input
 * gives that infinity.  An exact zero sum is -0 only when every input is -0. */
void orc_plain_sum(int dt, int op, int A, const void *const *x, int64_t off,
                   int64_t n, void *out)
{
    const uint32_t d = op == ORC_AVG ? (uint32_t)A : 1u;
    const int p = dt == ORC_F32 ? 24 : 8;
    for (int64_t i = 0; i < n; i++) {
        fx_int acc;
        memset(&acc, 0, sizeof acc);
        int nan = 0, pinf = 0, ninf = 0, all_neg_zero = 1;
        for (int s = 0; s < A; s++) {
            uint32_t u;
            if (dt == ORC_F32)
                memcpy(&u, (const float *)x[s] + off + i, sizeof u);
            else
                u = (uint32_t)((const uint16_t *)x[s])[off + i] << 16;
            const int neg = (int)(u >> 31), ef = (int)((u >> 23) & 0xFFu);
            const uint32_t mf = u & 0x7FFFFFu;
            if (u != 0x80000000u)
                all_neg_zero = 0;
            if (ef == 0xFF) {
                if (mf)
                    nan = 1;
                else if (neg)
                    ninf = 1;
                else
                    pinf = 1;
                continue;
            }
            /* value = M * 2^sh units of 2^-149 */
            const uint32_t M = ef ? (mf | 0x800000u) : mf;
            const int sh = ef ? ef - 1 : 0;
            if (M)
                fx_add_shifted(&acc, neg, M, sh);
        }
        uint32_t bits;
        if (nan || (pinf && ninf)) {
            bits = p == 24 ? 0x7FC00000u : 0x7FC0u;
        } else if (pinf || ninf) {
            bits = p == 24 ? 0x7F800000u : 0x7F80u;
            if (ninf)
                bits |= p == 24 ? 0x80000000u : 0x8000u;
        } else if (fx_is_zero(&acc)) {
            bits = all_neg_zero ? (p == 24 ? 0x80000000u : 0x8000u) : 0u;
        } else {
            const int negative = fx_is_negative(&acc);
            if (negative)
                fx_negate(&acc);
            const uint32_t rem = fx_divmod_small(&acc, d);
            bits = fx_round(&acc, rem, d, negative, p);
        }
        if (dt == ORC_F32)
            memcpy((float *)out + i, &bits, sizeof bits);
        else
            ((uint16_t *)out)[i] = (uint16_t)bits;
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
