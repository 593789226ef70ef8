/*
 * rr.h -- C ABI of the MI355X (gfx950) kernels for the per-GPU local work of the
 * link-balanced sharded relay collectives, as described in the pull request
 * "Link-balance the sharded relay schedules (up to 3.2x vs NCCL)" (torchrec #4570)
 * and the commit messages of its stack.
 *
 * Terms follow the pull request:
 *   A          active ranks per sparse group (2 or 4)
 *   H          helpers per group: the other local ranks, local_size - A (>= 1)
 *   numChunks  relay chunk divisor (A=2: H+2 in the link-balanced schedule;
 *              A=4 all-to-all: H+1)
 *   permille   A=4 allreduce / reduce-scatter offload fraction in 1/1000
 *              (500 = the balanced split of summary section 4)
 *   count      the per-group element count the kernel receives: the per-rank
 *              element count for allreduce, recvCount for reduce-scatter,
 *              segmentCount for all-to-all
 *
 * Conventions for every entry point:
 *   - Buffers are device memory owned by the caller (for example torch
 *     tensors).  The library allocates, frees, retains and synchronises
 *     nothing; it never reads a buffer on the host.
 *   - Pointer arguments of the form `const void* const* p` are HOST arrays of
 *     DEVICE pointers.
 *   - Kernels are enqueued on `stream` (a hipStream_t passed as void*; NULL =
 *     the null stream) and run asynchronously.  A call enqueues kernel
 *     launches only -- no allocation, memset, copy or synchronisation -- so
 *     calls can be captured in a HIP graph and replayed.  Calls that overlap
 *     on different streams must not write the same buffers.
 *   - Buffer sizes are the caller's contract (they are stated per entry
 *     point); the library cannot check them.
 *   - Every device pointer must be aligned to the element size (RR_EINVAL
 *     otherwise); any such offset is served by 16-byte vector loads and
 *     stores.  Buffers at 16-byte boundaries take the direct path; views at
 *     other offsets are realigned in registers, and the few elements before
 *     the first and after the last whole 16-byte output vector are computed
 *     one by one.
 *   - Every call validates its arguments before any HIP call and returns an
 *     rr_status; a thread-local message is available from rr_last_error().
 *     No exception crosses the ABI.  RR_EHIP means a HIP launch failed.
 *   - A relay chunk of zero elements (count below numChunks * 128, or an A=4
 *     allreduce under the 2 MiB floor) is not an error: the group is served by
 *     the direct path, helper work is a no-op and returns RR_OK (the zero-chunk
 *     direct-fallback commit of the stack).
 *   - Reductions read the buffer dtype, accumulate in fp32 in ascending source
 *     rank order, multiply once by the op scale (SUM 1, AVG 1/A) and round once
 *     to the buffer dtype (round-to-nearest-even).  A NaN result is a NaN of
 *     unspecified payload.  Pack and unpack copy raw bit patterns.
 */
#ifndef RR_H
#define RR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RR_ABI_VERSION 1

typedef enum {
    RR_OK = 0,
    RR_EINVAL = 1,        /* argument outside the method's domain */
    RR_EALIAS = 2,        /* forbidden overlap between inputs and outputs */
    RR_EUNSUPPORTED = 3,  /* reserved for calls valid in the method but not provided;
                             no entry point of this version returns it */
    RR_EHIP = 4           /* the HIP runtime reported an error */
} rr_status;

typedef enum { RR_F32 = 0, RR_BF16 = 1 } rr_dtype;

/* Only SUM and AVG exist in the method (reduce-scatter core commit). */
typedef enum { RR_SUM = 0, RR_AVG = 1 } rr_op;

typedef enum { RR_ALLREDUCE = 0, RR_REDUCE_SCATTER = 1, RR_ALLTOALL = 2 } rr_coll;

typedef struct {
    int32_t A;
    int32_t H;
    int32_t numChunks;
    int32_t permille;
    int64_t count;
} rr_relay;

/* Largest accepted count (2^48 elements, far beyond any device memory): every
 * product the geometry forms (count * elemsize * permille, A*A*chunk, byte
 * offsets) then stays inside int64_t. */
#define RR_MAX_COUNT (INT64_C(1) << 48)

/* Geometry of one group, in elements.  The relay region comes first:
 * helper k owns [k*chunk, (k+1)*chunk) of every buffer it relays, so
 * relay_total = H*chunk; the direct region is [direct_off, direct_off +
 * direct_len) = [relay_total, count). */
typedef struct {
    int64_t chunk;        /* per-helper relay chunk (A=4 allreduce: oChunk); 0 = pure direct */
    int64_t relay_total;
    int64_t direct_off;
    int64_t direct_len;
    int64_t dirA_off, dirA_len; /* A=2: the direct piece riding with relay group 1 */
    int64_t dirB_off, dirB_len; /* A=2: the direct piece riding with relay group 2 */
    int64_t dslice;       /* A=4 allreduce / reduce-scatter: direct slice per active
                             (active A-1 also takes direct_len - A*dslice) */
    int64_t helper_elems; /* helper scratch contract for this collective */
    int32_t pure_direct;
    int32_t reserved;
} rr_geom;

/* ABI version compiled into the library (RR_ABI_VERSION). */
int rr_abi_version(void);

/* Message of the last failing call on this thread ("" if none). */
const char *rr_last_error(void);

/*
 * rr_geometry -- the chunk geometry of one group (summary section 1 for A=2,
 * section 4 for the A=4 allreduce, section 6 for the A=4 reduce-scatter, the
 * all-to-all distributed-layer commit for the all-to-all chunk, and the
 * zero-chunk direct-fallback commit for chunk == 0).
 *   A=2, any collective: numChunks >= H+2; chunk = align_down(count/numChunks, 128);
 *     dirA = the chunk at index H, dirB = the rest of the buffer.  chunk == 0:
 *     dirA = [0, count/2), dirB = the remainder.  helper_elems = 2*chunk (two
 *     slots; the allreduce helper writes its reduced chunk over slot 0).
 *   A=4 allreduce: chunk = align_down(count*permille/(1000*H), 128); 0 when
 *     count*elemsize < 2 MiB.  helper_elems = 2*count, which covers the
 *     (A+1)*chunk the flat helper-reduce-and-broadcast needs.
 *   A=4 reduce-scatter: chunk = align_down(recvCount*permille/(1000*H), 128);
 *     helper_elems = 2*recvCount, holding A*(A-1) input chunks and A reduced
 *     chunks (RR_EINVAL if A*A*chunk exceeds it).
 *   A=4 all-to-all: numChunks >= H+1; chunk = align_down(segmentCount/numChunks, 128);
 *     helper_elems = A*(A-1)*chunk, one chunk per (destination, source) pair.
 * Errors: RR_EINVAL for A not in {2,4}, H < 1, count < 0 or above
 * RR_MAX_COUNT, numChunks or permille out of range, unknown collective or
 * dtype, null pointers.
 */
rr_status rr_geometry(const rr_relay *relay, int coll, int dtype, rr_geom *out);

/*
 * rr_passthrough_helper_size -- the helper buffer size for passthrough helpers
 * used by the distributed layer: min(count_g, A * align_down(count_g / num_chunks, 128))
 * elements, count_g being the count the kernel receives (reduce-scatter tests
 * commit and all-to-all distributed-layer commit).  Returns -1 if count_g < 0,
 * A < 1 or num_chunks < 1.
 */
int64_t rr_passthrough_helper_size(int64_t count_g, int32_t A, int32_t num_chunks);

/*
 * rr_helper_reduce -- reduce-at-helper for the allreduce (summary section 2
 * for A=2; section 4 and the 4-active allreduce commit, "flat
 * helper-reduce-and-broadcast", for A=4).
 *   coll must be RR_ALLREDUCE: the A=2 reduce-scatter helpers are passthrough
 *   (their two slots feed different outputs and are not summable), the A=4
 *   reduce-scatter helper uses rr_rs_multi_reduce, and all-to-all has no
 *   reduction -- all three return RR_EINVAL.
 *   helper:  k in [0, H); selects nothing in memory (the slots are given) but
 *            is validated against the geometry.
 *   slots:   nSlots == A device pointers; slots[a] holds active a's copy of
 *            relay chunk k (chunk elements each, buffer dtype).
 *   out:     chunk elements: out[i] = RND(scale * sum_a slots[a][i]), scale 1
 *            (SUM) or 1/A (AVG).  The helper returns it unchanged to every
 *            active, whose relay region then needs no further work.
 *   Aliasing: out may equal one of the slots exactly (the A=2 helper buffer
 *   holds just the two slots); any other overlap is RR_EALIAS.
 */
rr_status rr_helper_reduce(const rr_relay *relay, int coll, int dtype, int op,
                           int helper, const void *const *slots, int nSlots,
                           void *out, void *stream);

/*
 * rr_active_add_scale -- the active rank's fused add + scale epilogue.
 *   RR_ALLREDUCE (A=2 or 4): in[s] (nIn == A) is source rank s's full count-
 *     element buffer; out is active `activeIdx`'s count-element output.
 *     A=2 writes the whole direct region [direct_off, count) (dirA and dirB,
 *     summary section 1); A=4 writes active activeIdx's direct slice (the
 *     intra-link reduce-scatter of section 4).  out[i] = RND(scale * sum_s in[s][i]).
 *     Elements outside that region are not touched (the relay region holds
 *     what the helpers returned).
 *   RR_REDUCE_SCATTER (A=2 only): in[s] (nIn == 2) is source s's block destined
 *     for owner activeIdx (recvCount elements: the own block, and the other
 *     active's block as assembled from the helpers' passthrough forwards and
 *     the direct exchange); out is the owner's recvCount-element output, all of
 *     which is written.  This fuses the add + scale of the relayed chunks and
 *     the final reduction of the direct chunks (reduce-scatter core commit,
 *     phases 3 and 5) into one pass.  A=4 uses rr_rs_multi_reduce (RR_EINVAL).
 *   Aliasing: out's region may equal the same region of one input exactly
 *   (in-place, normally in[activeIdx]); any other overlap is RR_EALIAS.
 */
rr_status rr_active_add_scale(const rr_relay *relay, int coll, int dtype, int op,
                              int activeIdx, const void *const *in, int nIn,
                              void *out, void *stream);

/*
 * rr_rs_multi_reduce -- the A=4 reduce-scatter "two fused multi-input passes"
 * of the flat reduce-at-helper schedule (summary section 6).  A must be 4.
 *   pass 1, at helper idx (in [0, H)): nIn == 1; in[0] is the helper scratch
 *     holding one chunk per (owner o, source) pair at element offset
 *     (o*(A-1) + j)*chunk, j indexing the sources other than o in ascending
 *     order.  out (A*chunk elements, owner-major) receives
 *     out[o*chunk + i] = RND(sum_j scratch[(o*(A-1)+j)*chunk + i]) -- unscaled,
 *     the owner applies the scale.  Within the 2*recvCount contract out
 *     conventionally sits at scratch + A*(A-1)*chunk.  out must not overlap
 *     the A*(A-1) input chunks (RR_EALIAS).
 *   pass 2, at owner idx (in [0, A)): nIn == A + H; in[s] (s < A) is source s's
 *     recvCount-element block destined for owner idx (in[idx] is the owner's
 *     own block); in[A+h] is helper h's reduced chunk for this owner (chunk
 *     elements).  out (recvCount elements):
 *       offload slice h, [h*chunk, (h+1)*chunk): RND(scale*(in[idx][i] + in[A+h][i-h*chunk]))
 *       direct region [H*chunk, recvCount):      RND(scale*sum_s in[s][i])
 *     out may equal in[idx] exactly (in-place); any other overlap is RR_EALIAS.
 *     With chunk == 0 the whole output is the direct sum and in[A..A+H-1]
 *     are not read.
 */
rr_status rr_rs_multi_reduce(const rr_relay *relay, int dtype, int op, int pass,
                             int idx, const void *const *in, int nIn, void *out,
                             void *stream);

/*
 * rr_a2a_pack -- strided gather that coalesces helper slice h's all-to-all
 * traffic per destination (the reverted all-to-all paragraph of the summary: the
 * open lead needs gather/scatter kernels because sources and destinations are
 * both laid out with a segmentCount stride).  Out-of-place only.
 *   src[s] (A pointers): source s's input, A segments of count elements,
 *     segment d destined for rank d.
 *   dst[d] (A pointers): (A-1)*chunk elements; chunk j holds the slice
 *     [helper*chunk, (helper+1)*chunk) of segment d of the j-th source other
 *     than d, sources ascending:
 *       dst[d][j*chunk + i] = src[s_j][d*count + helper*chunk + i].
 *   Bit copies of dtype-sized elements.  chunk == 0: no-op.  Any overlap
 *   between a dst range and a src range or another dst range is RR_EALIAS.
 */
rr_status rr_a2a_pack(const rr_relay *relay, int dtype, int helper,
                      const void *const *src, void *const *dst, void *stream);

/*
 * rr_a2a_unpack -- the inverse scatter on receive:
 *       out[d][s_j*count + helper*chunk + i] = recv[d][j*chunk + i]
 *   recv[d]: (A-1)*chunk elements as packed for destination d; out[d]: rank d's
 *   A*count-element output.  Only helper slice positions of the segments from
 *   other ranks are written.  Any overlap between an out slice and a recv
 *   range or another out slice is RR_EALIAS.
 */
rr_status rr_a2a_unpack(const rr_relay *relay, int dtype, int helper,
                        const void *const *recv, void *const *out, void *stream);

/*
 * Batched forms -- one fused call for all the groups a GPU serves in one
 * phase (the fused multi-group call of the reduce-scatter distributed-layer
 * commit: one fused call covers every sparse group at once), with
 * a per-group geometry: each job carries its own rr_relay, so groups of
 * different sizes mix freely and a job whose chunk aligns down to zero is a
 * no-op (zero-chunk direct-fallback commit: every group picks its schedule
 * independently).
 *
 * Each job means exactly what the single-job call with the same fields means.
 * All jobs are validated before anything is enqueued: first each job's
 * arguments, in job order (the first invalid job fails the whole call with
 * the status and message of its single-job call, prefixed "job j: "), then
 * the aliasing over all jobs together (RR_EALIAS, prefixed "job j: " for an
 * alias within one job, "jobs i and j: " for memory two jobs share).  The
 * jobs of one call run concurrently: one kernel launch for up to 40 reduction
 * segments (a helper or active job is one, an A=4 reduce-scatter pass-1 job
 * A, an owner pass with the balanced split 2H) or 64 chunk moves whose
 * buffers are 16-byte aligned, one more for those at other offsets, and
 * further launches on the same stream for larger calls.  So no job may write
 * memory another job of the call reads or writes (RR_EALIAS); the exact
 * in-place aliases of the single-job calls stay allowed within a job.
 * Pointer arrays inside the job structs are host memory, read during the
 * call only.
 */
typedef struct {
    rr_relay relay;
    int32_t helper;
    int32_t nSlots;
    const void *slots[4];
    void *out;
} rr_helper_job;

typedef struct {
    rr_relay relay;
    int32_t activeIdx;
    int32_t nIn;
    const void *in[4];
    void *out;
} rr_active_job;

typedef struct {
    rr_relay relay;
    int32_t pass;            /* 1 helper, 2 owner */
    int32_t idx;
    int32_t nIn;
    int32_t reserved;
    const void *const *in;   /* nIn device pointers (host array) */
    void *out;
} rr_rs_job;

typedef struct {
    rr_relay relay;
    int32_t helper;
    int32_t reserved;
    const void *const *in;   /* pack: src[A]; unpack: recv[A] (host arrays) */
    void *const *out;        /* pack: dst[A]; unpack: out[A] */
} rr_a2a_job;

rr_status rr_helper_reduce_many(int coll, int dtype, int op, const rr_helper_job *jobs, int nJobs,
                                void *stream);
rr_status rr_active_add_scale_many(int coll, int dtype, int op, const rr_active_job *jobs, int nJobs,
                                   void *stream);
rr_status rr_rs_multi_reduce_many(int dtype, int op, const rr_rs_job *jobs, int nJobs, void *stream);
rr_status rr_a2a_pack_many(int dtype, const rr_a2a_job *jobs, int nJobs, void *stream);
rr_status rr_a2a_unpack_many(int dtype, const rr_a2a_job *jobs, int nJobs, void *stream);

/*
 * rr_phase_reduce_many -- every helper and active reduction a GPU runs in one
 * phase, in one batched call.  In the fused A=4 allreduce (summary section 4,
 * groups of 4 consecutive ranks) a rank is an active of its own group and a
 * helper of the other one; after the first serialized group of hops it reduces
 * its own direct slice (the intra-link reduce-scatter) and its position slice
 * of the other group's offload region (the helper's 4->1 sum) before the
 * second group returns both.  The two reductions read different buffers and
 * are ready at the same time, so they share one launch.
 *   helperJobs[0..nHelper): as rr_helper_reduce_many (numbered as jobs
 *     0..nHelper-1 in messages); activeJobs[0..nActive): as
 *     rr_active_add_scale_many (jobs nHelper..nHelper+nActive-1).  All jobs
 *     share coll, dtype and op.
 *   Each job means what its single-job call means; validation, aliasing over
 *   all jobs of both arrays, and launch batching follow the batched forms
 *   above.  nHelper == nActive == 0 is a no-op.  Either array may be null when
 *   its count is zero.
 */
rr_status rr_phase_reduce_many(int coll, int dtype, int op,
                               const rr_helper_job *helperJobs, int nHelper,
                               const rr_active_job *activeJobs, int nActive,
                               void *stream);

/*
 * Plans -- validate once, launch many times.  For callers that issue the same
 * relay steps on the same buffers over and over (a training or serving loop at
 * small messages, where the host's per-call work -- argument checks, geometry,
 * aliasing, segment tables -- would otherwise take longer than the kernels),
 * every entry point above can be recorded into a plan and the plan re-issued
 * with one call.  A plan is a HOST buffer owned by the caller; the library
 * allocates nothing and keeps no pointer to it after rr_plan_end.
 *
 *   rr_plan_bytes(n): bytes a plan buffer needs to hold n kernel launches
 *     (1 <= n <= RR_PLAN_MAX_LAUNCHES; 0 otherwise).  A call is one launch per
 *     kernel body it uses (reductions: aligned and realigned items; copies:
 *     one), or more when it exceeds a launch's segment table (40 reduction
 *     items, 64 chunk moves) or 2^22 tiles.
 *   rr_plan_begin(plan, bytes): starts recording on the calling thread into
 *     `plan` (8-byte aligned, at least rr_plan_bytes(1) bytes).  Until
 *     rr_plan_end, every entry point called on this thread validates its
 *     arguments as usual (a rejected call records nothing and returns its
 *     status) and appends its launches to the plan instead of enqueuing them;
 *     their `stream` argument is ignored.  RR_EINVAL if this thread is already
 *     recording.
 *   rr_plan_end(&launches): stops recording; stores the number of recorded
 *     launches if `launches` is not null.  RR_EINVAL if the thread is not
 *     recording, or if a call ran out of records (that call returned RR_EINVAL
 *     too); such a plan cannot be launched.
 *   rr_plan_append(plan, bytes, other): appends the launches of the finished
 *     plan `other` to the finished plan `plan` (whose buffer is `bytes` long),
 *     so that one rr_plan_launch issues both in order -- for instance every
 *     relay step of one phase or of one benchmark step.  RR_EINVAL, with
 *     nothing changed, if either is not a finished, unbroken plan, if they are
 *     the same buffer, or if `plan` lacks room.
 *   rr_plan_launch(plan, stream): enqueues the recorded launches, in recording
 *     order, on `stream`, with no validation: the device buffers named by the
 *     recorded calls must still be allocated at the same addresses with the
 *     same sizes.  RR_EINVAL for a buffer that is not a finished, unbroken
 *     plan; RR_EHIP if a launch fails.  Launching is read-only on the plan, so
 *     one plan may be launched from several threads (on streams that do not
 *     write the same buffers concurrently), and the plan buffer may be copied.
 */
#define RR_PLAN_MAX_LAUNCHES 4096

size_t rr_plan_bytes(int32_t max_launches);
rr_status rr_plan_begin(void *plan, size_t bytes);
rr_status rr_plan_end(int32_t *launches);
rr_status rr_plan_append(void *plan, size_t bytes, const void *other);
rr_status rr_plan_launch(const void *plan, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RR_H */
