/*
 * ar.h -- C ABI of the barrier-free small/medium-message AllReduce (sum) for N ranks emulated on
 * one MI355X (gfx950).
 *
 * Each emulated rank is a group of co-resident workgroups with its own input, output and block
 * of a symmetric scratch allocation (Every µs Matters: Achieving Near Speed-of-Light Latency in
 * GPU Collectives, §II.B "symmetric memory": every participant's object has the same size and
 * layout and is addressed by participant index plus offset). Ranks exchange data only through
 * global stores into each other's scratch and polling of their own; no device-wide barrier is
 * used (§IV "Designing Barrier-Free Collectives"). Latencies measured through this interface are
 * on-chip (L2 / MALL / HBM), not interconnect latencies.
 *
 * Conventions for every entry point:
 *   - Device pointers are plain `void*` from any HIP allocator (hipMalloc, torch); host pointers
 *     are ordinary host memory. `stream` is a hipStream_t passed as `void*` (NULL = null stream).
 *   - Integer returns are AR_OK (0) or a negative AR_E* code; ar_last_error() then holds a
 *     message for the calling thread. Functions returning a pointer return NULL on error.
 *   - A handle is not thread-safe. Calls on one handle must be issued in order on one stream:
 *     the sequence number and the scratch reuse depend on call order (as with a communicator).
 *   - Every workgroup of a call's grid waits for others, so a grid must be resident as a whole.
 *     Each call is planned to fit the GPU on its own; two calls in flight at once on one GPU
 *     (two handles on two streams) may each get only part of the GPU and then wait for each
 *     other forever (each side's poll times out after AR_OPT_TIMEOUT_US). Keep the calls of all
 *     handles on one GPU on one stream, or order the streams.
 */
#ifndef LATENCY_COLLECTIVES_AR_H
#define LATENCY_COLLECTIVES_AR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { AR_FLOAT32 = 0, AR_BFLOAT16 = 1, AR_INT32 = 2 } ar_dtype;

/*
 * Algorithms (Every µs Matters, §III.A and §IV; the LL128 atomic two-shot of Fig. 5 as described
 * in the Pith review of the paper):
 *   AR_ONESHOT_LL       one-shot push; each 8 bytes travel with their step's sequence number in
 *                       one 16-byte store, polled as one line (§IV "LL").
 *   AR_ONESHOT_SENTINEL one-shot push into sentinel-filled scratch, polled until the sentinel is
 *                       gone, then re-armed (§IV "Sentinel").
 *   AR_TWOSHOT          reduce-scatter to partition owners + all-gather, sentinel synchronised
 *                       (§III.A "Two-shot AllReduce"). For int32 the all-gather carries sums,
 *                       any of which may equal the sentinel, so int32 always runs the
 *                       bandwidth kernel, whose per-wave completion flags ignore the data; so
 *                       do fp32 and bf16 messages whose slots do not fit the near pages with up
 *                       to 8 ranks, and with more over 1 MiB per rank. With more than 8 ranks,
 *                       messages whose slots need two near
 *                       pages per region keep the one-pass kernel on two-page near slots
 *                       (AR_OPT_TWO_PAGE). The bandwidth kernel's owners store their reduced partition
 *                       into every rank's output directly (the outputs are all kernel
 *                       arguments), except in an ar_bench launch whose output sets overlap its
 *                       input sets.
 *   AR_LL128_ATOMIC     reduce-scatter by atomic adds into the owner's shared destination, then
 *                       an all-gather with completion flags: the owners store their sums
 *                       straight into every rank's output (as the bandwidth kernel above; the
 *                       peer-split kernels of small messages keep the sentinel all-gather).
 *                       bf16 adds two elements per atomic and rounds to bf16 at every addition.
 *                       The fp32 and bf16 summation order is not deterministic: per element
 *                       |result - rank-order fold| <= N * 2^-23 * sum_r |x_r| (fp32),
 *                       <= N * 2^-8 * sum_r |x_r| (bf16).
 *   AR_LL128_DET        the deterministic variant (the Pith review's "per-chunk grouping or
 *                       hierarchical accumulation"): ranks form groups of AR_OPT_GROUP
 *                       consecutive ranks; each group's values are added into the owner's
 *                       group destination in rank order (ticket-ordered atomics), and the owner
 *                       adds the group sums in group order; binary32 throughout (bf16 inputs
 *                       widened, rounded once). Bit-reproducible; fp32 and bf16 (int32 runs
 *                       AR_LL128_ATOMIC, whose integer sum does not depend on the order).
 *   AR_BARRIER2         one-shot push between two cross-rank flag barriers: the conventional
 *                       design whose barrier cost the pages measure (§III.B). A baseline.
 *   AR_BARRIER_ONLY     (ar_bench only) one cross-rank barrier per iteration, no data: the
 *                       barrier latency versus N (§III.B, Fig. 3).
 *   AR_ALGO_AUTO        picks one-shot LL, one-shot sentinel, two-shot or (int32 only) the
 *                       LL128-style kernel from the dtype, the rank count and the message size,
 *                       by tables of the fastest measured on MI355X; for fp32 and bf16 only
 *                       fixed-order kernels, so the result stays bit-reproducible.
 * Every algorithm except AR_LL128_ATOMIC and AR_LL128_DET adds in rank order 0..N-1 (fp32
 * accumulation for bf16, rounded once to nearest even; wrapping int32) and is bit-reproducible.
 * Double buffering (§IV "Bidirectional Communication Double Buffering", Fig. 4) is used by
 * every algorithm except AR_BARRIER2: step s uses scratch buffer s & 1.
 */
typedef enum {
  AR_ALGO_AUTO = 0,
  AR_ONESHOT_LL = 1,
  AR_ONESHOT_SENTINEL = 2,
  AR_TWOSHOT = 3,
  AR_LL128_ATOMIC = 4,
  AR_BARRIER2 = 5,
  AR_BARRIER_ONLY = 6,
  /* values 7..11, 15..20 and 22..36 are internal kernel families (see ar_plan_info); the standalone
     collectives below are called through their own entry points and named by these ids in
     ar_bench, ar_alg_bytes and ar_plan_info */
  AR_REDUCESCATTER = 12,
  AR_ALLGATHER = 13,
  AR_BROADCAST = 14,
  AR_LL128_DET = 21
} ar_algo;

enum {
  AR_OK = 0,
  AR_EINVAL = -1,   /* bad argument */
  AR_ETOOBIG = -2,  /* count * sizeof(dtype) > max_bytes of the handle */
  AR_ENOTSUP = -3,  /* algorithm / dtype combination not provided */
  AR_EHIP = -4,     /* a HIP runtime call failed */
  AR_ETIMEOUT = -5, /* a poll timed out on the device; the handle is poisoned (sticky) */
  AR_ENORES = -6    /* the workgroups of all ranks cannot be co-resident */
};

/* Placement of the emulated ranks on the XCDs (ar_set_option AR_OPT_PLACEMENT, ar_sol). */
typedef enum { AR_PLACE_XCD = 0, AR_PLACE_SAME = 1, AR_PLACE_LINEAR = 2 } ar_placement;

typedef struct ar_handle ar_handle;

/*
 * ar_create: build a handle for `nranks` emulated ranks (1..16) exchanging messages of up to
 * `max_bytes` bytes per rank (1..2^31-1) of `dtype`.
 *
 * Allocates the symmetric scratch in device memory (one allocation, rank r's block at
 * base + r * stride) and fills it: LL lines, atomic destinations, counters and barrier flags
 * with zeros, sentinel slots with the dtype's sentinel (fp32 0xFFFFFFFF, bf16 0xFFFF: negative
 * quiet NaNs, compared bitwise; int32 INT32_MIN). The sequence number starts at 1. Scratch
 * per rank per protocol is capped by the environment variables AR_SCRATCH_ONESHOT (default
 * 4 MiB) and AR_SCRATCH_TWOSHOT (default 16 MiB; also the LL128 cap): the outcome of a
 * scratch-size sweep on MI355X, the counterpart of the pages' Fig. 12 (the Pith review lists
 * 4 MiB / 64 MiB for their hardware, "Assumptions & free parameters"); larger messages are sent
 * in equal chunks.
 * AR_POLL_TIMEOUT_US sets the initial poll timeout (default 2000000).
 * Synchronous on the current device. Returns NULL on error (see ar_last_error()).
 *
 * Caller obligation (§IV "Sentinel"): input values must never equal the sentinel bit pattern
 * (AR_OPT_CHECK_INPUTS checks it). Only inputs travel through sentinel slots as they are; the
 * sums that the two-shot all-gather sends are fp32 / bf16 values that a fold of such inputs
 * can produce (a fold of finite values never yields a NaN; a NaN input may propagate, so
 * callers keep NaNs out of float inputs) or int32 sums, which use completion flags instead.
 */
ar_handle* ar_create(int nranks, size_t max_bytes, ar_dtype dtype);

/*
 * ar_allreduce: out[r][i] = in[0][i] + in[1][i] + ... + in[N-1][i] for every rank r and element
 * i < count (Every µs Matters, §III.A: after the collective every rank holds the complete
 * reduction).
 *   in, out : host arrays of N device pointers, each to count * sizeof(dtype) bytes, 16-byte
 *             aligned. out[r] == in[r] (in place) is allowed; any other overlap is AR_EINVAL.
 *   count   : elements per rank; 0 is a no-op (the sequence number still advances).
 *   algo    : see ar_algo; AR_BARRIER_ONLY is not accepted here.
 *   stream  : hipStream_t; the call only enqueues work and returns.
 * The caller keeps ownership of every buffer; they must stay valid until the stream has run
 * the work. Device timeouts are reported asynchronously through ar_check().
 */
int ar_allreduce(ar_handle* h, const void* const in[], void* const out[], size_t count,
                 ar_algo algo, void* stream);

/*
 * ar_allreduce_noalloc: ar_allreduce for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation. It makes no
 * allocation of any kind; there is no handle. The symmetric scratch is a static device array
 * of 40 MiB that the library holds on every GPU it runs on until the process ends (scratch per
 * rank per protocol 256 KiB, so larger messages run in more chunks than through a handle).
 *   nranks, dtype          : as for ar_create (1..16; AR_FLOAT32, AR_BFLOAT16, AR_INT32).
 *   in, out, count, algo   : as for ar_allreduce (count * sizeof(dtype) < 2^31 bytes per rank,
 *                            AR_ETOOBIG beyond; every algorithm of ar_allreduce is accepted).
 *   stream                 : hipStream_t; the call only enqueues work on it.
 * The array keeps the last call's state (sequence number, armed slots). When nranks or dtype
 * differs from the previous call on the current GPU, the call first clears the array and
 * re-arms its slots on `stream`. Calls on one GPU must not overlap: two calls in flight at once
 * on one GPU (on different streams, or from different threads) race on the shared array, and
 * calls must be issued in order, as on one handle. Device poll timeouts are not reported to the
 * host (there is no status block to read without allocating): the timed-out kernel raises the
 * abort word in the array, every later call on that GPU then exits without writing its outputs,
 * until a call with another (nranks, dtype) sets the array up again. Argument errors are
 * synchronous return codes, as for ar_allreduce.
 */
int ar_allreduce_noalloc(int nranks, ar_dtype dtype, const void* const in[], void* const out[],
                         size_t count, ar_algo algo, void* stream);

/*
 * Standalone collectives from the same barrier-free primitives. The paper notes that AllReduce is
 * commonly decomposed into ReduceScatter + AllGather or Reduce + Broadcast (Every µs Matters,
 * §III opening paragraph), and the Pith review of it ("If this is right") expects these
 * collectives to be rebuilt with the same LL / sentinel / double-buffering pattern. All three
 * push raw 16-byte units into sentinel-armed scratch slots, poll until the sentinel is gone,
 * consume and re-arm (§IV "Sentinel"), with step s on scratch buffer s & 1 (§IV "Bidirectional
 * Communication Double Buffering"). Common rules: host arrays of N device pointers, every
 * buffer 16-byte aligned; outputs of different ranks must not overlap; count 0 is a no-op that
 * still advances the sequence number; the call only enqueues work on `stream` (ordering and
 * ownership as for ar_allreduce); device timeouts are reported through ar_check(); AR_ETOOBIG
 * when an input or output exceeds the handle's max_bytes per rank.
 *
 * ar_reducescatter: out[r][i] = in[0][r*recvcount + i] + ... + in[N-1][r*recvcount + i] for
 *   i < recvcount (the AllReduce fold: rank order, fp32 accumulation for bf16, one rounding).
 *   in[r] holds N * recvcount elements, out[r] recvcount; recvcount * sizeof(dtype) must be a
 *   multiple of 16 bytes (AR_EINVAL otherwise). In place: out[r] == in[r] + r * recvcount
 *   elements; any other overlap of an output with an input is AR_EINVAL.
 */
int ar_reducescatter(ar_handle* h, const void* const in[], void* const out[], size_t recvcount,
                     void* stream);

/*
 * ar_allgather: out[r][q*sendcount + i] = in[q][i] for every rank r, source q and i < sendcount.
 *   in[r] holds sendcount elements, out[r] N * sendcount; sendcount * sizeof(dtype) must be a
 *   multiple of 16 bytes (AR_EINVAL otherwise). In place: in[r] == out[r] + r * sendcount
 *   elements; any other overlap of an output with an input is AR_EINVAL.
 */
int ar_allgather(ar_handle* h, const void* const in[], void* const out[], size_t sendcount,
                 void* stream);

/*
 * ar_broadcast: out[r][i] = in[i] for every rank r and i < count, where `in` is the input of
 *   rank `root` (0..N-1; AR_EINVAL otherwise). Any count. out[root] == in is allowed; any other
 *   overlap of an output with `in` is AR_EINVAL. Only the root sends data, so each receiver hands
 *   its scratch buffer back to the root with a flag after consuming a step (the root reuses a
 *   buffer only after every receiver's flag of two steps before).
 */
int ar_broadcast(ar_handle* h, const void* in, void* const out[], size_t count, int root,
                 void* stream);

/* ar_destroy: synchronise the handle's last stream and free everything. NULL is ignored. */
void ar_destroy(ar_handle* h);

/* ar_last_error: message of the last failing call on this thread ("" if none). */
const char* ar_last_error(void);

/*
 * ar_check: wait for the work of the handle's last stream and report a device-side poll
 * timeout. Returns AR_OK, AR_ETIMEOUT (the message names rank, peer, step and algorithm; the
 * handle stays poisoned and every later call returns AR_ETIMEOUT) or AR_EHIP.
 * A timed-out launch raises a device abort word: every launch on the handle enqueued after it
 * (before ar_check has seen the timeout) exits at entry without reading or writing anything,
 * so its outputs keep whatever they held before the call.
 */
int ar_check(ar_handle* h);

/*
 * ar_bench: run `iters` AllReduces back to back inside ONE persistent launch, with no host
 * involvement between iterations (a persistent loop measures µs-scale latency without the
 * launch overhead; the pages' latency is that of back-to-back collectives). Iteration k uses
 * input/output set k % nsets:
 *   in_sets, out_sets : host arrays of nsets * N device pointers, set-major (set j, rank r at
 *                       index j * N + r); nsets in [1, 65536].
 *   t_start, t_end    : host arrays of iters * N entries (iteration-major) receiving, per
 *                       iteration and rank, the device wall-clock tick at which the rank's
 *                       first wave entered the iteration (before its first input load) and the
 *                       tick at which its last wave had completed its last output store.
 *                       Either may be NULL to skip timestamps.
 * Synchronous. Ticks convert to seconds with ar_wallclock_hz(). AR_BARRIER_ONLY measures one
 * cross-rank barrier per iteration and ignores the data arguments (they may be NULL).
 * AR_REDUCESCATTER, AR_ALLGATHER and AR_BROADCAST run the standalone collectives instead, with
 * `count` as their entry points take it (recvcount, sendcount, count) and buffers sized as
 * there; the broadcast root is AR_OPT_ROOT (only the root's input pointers are read).
 */
int ar_bench(ar_handle* h, const void* const* in_sets, void* const* out_sets, int nsets,
             size_t count, ar_algo algo, int iters, uint64_t* t_start, uint64_t* t_end,
             void* stream);

/* ar_bench_ex: ar_bench that also returns the launch's duration from HIP events recorded on
 * `stream` around it (*elapsed_ms, if not NULL). */
int ar_bench_ex(ar_handle* h, const void* const* in_sets, void* const* out_sets, int nsets,
                size_t count, ar_algo algo, int iters, uint64_t* t_start, uint64_t* t_end,
                double* elapsed_ms, void* stream);

/* Rate of the device wall clock used by ar_bench and ar_sol, in Hz (0 on error). */
double ar_wallclock_hz(void);

/*
 * Per-handle options (defaults in brackets). Values are checked; AR_EINVAL when out of range.
 *   AR_OPT_TIMEOUT_US    poll timeout in microseconds [AR_POLL_TIMEOUT_US or 2000000]
 *   AR_OPT_WITHHOLD_RANK fault injection: this rank sends nothing, so its peers' polls time out
 *                        and ar_check reports AR_ETIMEOUT [-1 = off]
 *   AR_OPT_CTAS          workgroups per rank [0 = chosen from the message size]
 *   AR_OPT_THREADS       threads per workgroup, 64, 128 or 256 [0 = chosen]
 *   AR_OPT_PLACEMENT     ar_placement of ranks on XCDs [AR_PLACE_XCD]
 *   AR_OPT_DRIFT         ar_bench only: each rank sleeps a pseudo-random 0..value units of ~3 µs
 *                        before each iteration, to stress the double-buffer credits [0]
 *   AR_OPT_NARROW        1: when the launch shape is not forced (AR_OPT_CTAS and AR_OPT_THREADS
 *                        are 0), the one-pass sentinel kernels (one-shot and two-shot) move
 *                        8-byte units if the message still fits one pass of co-resident lanes
 *                        (twice the lanes, half the fold per lane); 0: always 16-byte units [1]
 *   AR_OPT_ROOT          ar_bench of AR_BROADCAST only: the root rank [0]
 *   AR_OPT_CHECK_INPUTS  1: every ar_allreduce / ar_reducescatter / ar_allgather / ar_broadcast
 *                        first scans the inputs for the sentinel bit pattern on `stream`, waits
 *                        for the scan, and returns AR_EINVAL (naming the first rank and element)
 *                        instead of launching when one is found. A debugging aid: it makes
 *                        every call synchronous [0]
 *   AR_OPT_RECORD_LAUNCH 1: every launch writes, per workgroup, its XCC id and the rank and
 *                        workgroup index it decoded into region 13 of rank 0 (ar_read_region)
 *                        [0]
 *   AR_OPT_GROUP         AR_LL128_DET: ranks per group, 2..16; the result depends on it (it is
 *                        the summation order) [2]
 *   AR_OPT_COOPERATIVE   1: kernels are started with the cooperative launch, which makes the
 *                        runtime check that the whole grid can be resident at once (every
 *                        workgroup waits for others, Every µs Matters §II.B) and refuse it
 *                        otherwise (AR_ENORES) instead of starting part of it; no grid-wide
 *                        synchronisation is used. Costs launch time, not device time [0]
 *   AR_OPT_SPLIT         1: with 5..16 ranks, when the launch shape is not forced, the one-pass
 *                        one-shot LL, one-shot sentinel and two-shot kernels and the fp32 / bf16
 *                        LL128-style kernel give each 64 units of a chunk a workgroup of 4
 *                        waves, each pushing to (adding into) and polling a quarter of the
 *                        peers (the kernel families 26..33 of ar_plan_info), while those
 *                        workgroups get a compute unit each; 0: one wave per 64 units with every
 *                        peer [1]
 *   AR_OPT_TWO_HALVES    1: a one-shot sentinel message whose ranks span two XCDs (one in each
 *                        half of the chip) and whose slots fit a near page when every 8 KiB
 *                        granule is used puts each workgroup's units in the granules homed in
 *                        its own XCD's half (ar_plan_info near = 2); 0: regular slots [1]
 *   AR_OPT_TWO_PAGE      1: a two-shot or one-shot LL message of more than 8 ranks, or a one-shot
 *                        sentinel message of 8 or more (AR_PLACE_XCD), whose 2 N slots need more
 *                        than one near page but whose N slots of one double buffer fit one uses
 *                        two-page near slots, buffer b in page b of the p1 and p2 (two-shot), ll
 *                        (LL) or p1 (sentinel) near regions
 *                        (ar_plan_info near = 3); buffer 1 starts one granule before its page
 *                        where that page's calibration shows it mirrors the first; 0: regular
 *                        slots [1]. The two-page regions exist in handles whose ranks and
 *                        max_bytes need them (2 MiB more scratch per rank and region).
 */
typedef enum {
  AR_OPT_TIMEOUT_US = 0,
  AR_OPT_WITHHOLD_RANK = 1,
  AR_OPT_CTAS = 2,
  AR_OPT_THREADS = 3,
  AR_OPT_PLACEMENT = 4,
  AR_OPT_DRIFT = 5,
  AR_OPT_NARROW = 6,
  AR_OPT_ROOT = 7,
  AR_OPT_CHECK_INPUTS = 8,
  AR_OPT_RECORD_LAUNCH = 9,
  AR_OPT_GROUP = 10,
  AR_OPT_COOPERATIVE = 11,
  AR_OPT_SPLIT = 12,
  AR_OPT_TWO_HALVES = 13,
  AR_OPT_TWO_PAGE = 14
} ar_option;
int ar_set_option(ar_handle* h, ar_option opt, int64_t value);

/*
 * Scratch regions (for tests that check that sentinel slots are re-armed after a call).
 * ar_read_region copies `bytes` bytes of region `region` of rank `rank` to host memory
 * (synchronous, after the handle's last stream has finished); ar_region_bytes gives the size.
 *   0 = one-shot / reduce-scatter sentinel slots  1 = all-gather sentinel slots
 *   2 = LL lines  3 = atomic destination  4 = arrival counters  5 = barrier flags
 *   6 = barrier-baseline data
 *   7, 8, 9 = the near LL, one-shot / reduce-scatter and all-gather regions that small messages
 *   use (slot data in 8 KiB chunks, each in the granule homed near its rank)
 *   10, 11 = bulk two-shot reduce-scatter and all-gather data slots  12 = their completion flags
 *   13 = launch record (rank 0 only): one uint32 per workgroup of the last launch made with
 *        AR_OPT_RECORD_LAUNCH, XCC id in bits 7:0, rank + 1 in bits 15:8 (0: the workgroup maps
 *        to no rank and exits), workgroup index within the rank in bits 31:16
 *   14 = sink: 16 KiB that idle lanes of the bf16 LL128-style kernel add zero into (stays zero)
 */
int64_t ar_region_bytes(ar_handle* h, int region);

/*
 * ar_alg_bytes: the algorithmic bytes one ar_allreduce of `count` elements with `algo` moves on
 * handle h, summed over all ranks, for the kernel and protocol the library would launch: every
 * logical read and write counted once (inputs, pushes to peers, slot reads, sentinel re-arms,
 * outputs; an LL line is 16 bytes per 8 bytes of payload). One-shot LL 2NS + 4N(N-1)S; one-shot
 * sentinel 2NS + 3N(N-1)S; two-shot (one pass) (N+1)S + 7(N-1)S; two-shot (bulk, completion
 * flags) (N+1)S + 5(N-1)S; LL128-style 2NS + 3S + 4(N-1)S; two-barrier 2NS + 2N(N-1)S, with S
 * the bytes per rank. For AR_REDUCESCATTER and AR_ALLGATHER (count as their entry points take
 * it, x = count * sizeof(dtype)): N ((N+1) x + 3 (N-1) x); for AR_BROADCAST (N+1) x + 3 (N-1) x.
 * Returns the count, or a negative error code (bad handle or algorithm, AR_ETOOBIG).
 */
int64_t ar_alg_bytes(ar_handle* h, size_t count, ar_algo algo);

/*
 * ar_plan_info: the launch that an ar_allreduce (or, for AR_REDUCESCATTER, AR_ALLGATHER and
 * AR_BROADCAST, the standalone collective with `count` as its entry point takes it) of `count`
 * elements with `algo` would make on handle h, written to *info. Host only: nothing is launched.
 * Returns AR_OK, or AR_EINVAL / AR_ETOOBIG / AR_ENOTSUP / AR_ENORES as the call itself would.
 */
typedef struct {
  int kernel;     /* kernel family: the public algorithm id (21 = AR_LL128_DET), or an internal one:
                     22 / 23 LL128-style with one / two word slices per lane (24 / 25
                     deterministic), 7 bulk
                     two-shot; 8 / 9 multi-pass LL / sentinel one-shot; 10 / 11 one-pass sentinel
                     one-shot / two-shot with 8-byte units; 12 / 13 / 14 the reduce-scatter /
                     all-gather / broadcast loop kernels; 15 / 16 reduce-scatter / all-gather as
                     one half of the one-pass two-shot (17 / 18 with 8-byte units); 19 / 20
                     one-pass broadcast with 16- / 8-byte units; 26 / 27 peer-split one-shot
                     sentinel, 28 / 29 peer-split two-shot, with 16- / 8-byte units; 30 / 31 /
                     32 peer-split LL128-style with 4 / 1 / 2 word slices per lane; 33
                     peer-split one-shot LL; 34 / 35 / 36 one-pass two-shot / one-shot LL /
                     one-shot sentinel on two-page near slots */
  int chunks;     /* steps per call (the message is cut into equal chunks at the scratch cap) */
  int ctas;       /* workgroups per rank */
  int threads;    /* threads per workgroup */
  int grid;       /* workgroups launched; those beyond the ranks' (on XCDs no rank uses) exit at
                     once */
  int unit_bytes; /* payload bytes per lane and unit: 16, or 8 for LL and the 8-byte kernels */
  int near;       /* 1: the slots are in the near regions; 2: two-half near p1 slots;
                     3: two-page near p1 and p2 slots */
  int resident_per_cu; /* workgroups of this kernel and block size that one compute unit holds at
                          once (the HIP occupancy query); the plan leaves one of them free per
                          compute unit whenever this is above 1 */
  int cu_count;   /* compute units of the device (8 XCDs share them equally) */
} ar_plan;
int ar_plan_info(ar_handle* h, size_t count, ar_algo algo, ar_plan* info);
int ar_read_region(ar_handle* h, int rank, int region, void* host_dst, size_t bytes);

/* Sequence number the next step will use. */
uint64_t ar_epoch(ar_handle* h);

/*
 * ar_sol: speed-of-light microbenchmarks on the current device (the pages' bound
 * L_SoL = 2 * L_L2 + L_remote_store; Every µs Matters §VI as summarised in the Pith review).
 * `placement` is AR_PLACE_XCD (the two workgroups of the ping-pong on different XCDs) or
 * AR_PLACE_SAME (same XCD). Writes out_ns[0] = L_fence (store + agent-scope release fence),
 * out_ns[1] = L_L2 (dependent-load L2 latency), out_ns[2] = L_store (store -> poll half round
 * trip on the nearest memory position), all in nanoseconds; the floor is
 * 2 * out_ns[1] + out_ns[2]. Synchronous. ar_sol_ex returns every probe.
 */
int ar_sol(int placement, double* out_ns);

/* ar_sol_ex: the same probes with all their results in `res`. */
typedef struct {
  double fence_ns;         /* plain store + agent-scope release fence, per iteration        */
  double l2_load_ns;       /* dependent load, 1 MiB footprint (L2 hit, per-CU cache miss)    */
  double coherent_load_ns; /* dependent load with the agent-coherent (sc1) policy, 1 MiB     */
  double mall_load_ns;     /* dependent load, 64 MiB footprint (beyond L2)                   */
  double hbm_load_ns;      /* dependent load, 1 GiB footprint (beyond the 256 MiB MALL)      */
  double store_half_rtt_ns;/* store -> poll ping-pong (sc1 store, sc1 poll), half round trip,
                              on a line homed in the workgroups' half of the chip            */
  double store_half_rtt_far_ns; /* the same on a line homed in the other half                */
  double floor_ns;         /* 2 * l2_load_ns + store_half_rtt_ns                             */
  double floor_fence_ns;   /* the pages' form: 2 * fence_ns + store_half_rtt_ns              */
  int xcc_a, xcc_b;        /* XCC ids the two ping-pong workgroups ran on                     */
} ar_sol_result;
int ar_sol_ex(int placement, ar_sol_result* res);

/*
 * ar_sol_ranks: the store term of the floor for the XCD pairs an N-rank placement uses. The
 * latency of one AllReduce is a maximum over ranks (the last rank's data decides), so the
 * floor of an N-rank configuration takes the slowest sender -> receiver pair among the ranks'
 * XCDs (the Pith review's referee comment on §VII.C: the bound grows with the rank count). For
 * every ordered pair of XCDs holding ranks (the same XCD twice when two ranks share one), a
 * store -> poll ping-pong on a fresh 2 MiB page at the position the planner would pick for the
 * receiving XCD (the fastest for its partner XCD x ^ 1). nranks 2..16, placement AR_PLACE_XCD
 * or AR_PLACE_SAME. Synchronous.
 */
typedef struct {
  double store_half_rtt_worst_ns; /* slowest pair: the store term of the N-rank floor           */
  double store_half_rtt_best_ns;  /* fastest pair                                               */
  int worst_sender_xcc, worst_receiver_xcc;
  int pairs;                      /* distinct (sender XCD, receiver XCD) pairs measured         */
} ar_sol_ranks_result;
int ar_sol_ranks(int nranks, int placement, ar_sol_ranks_result* res);

/*
 * ar_pingpong: the store -> poll ping-pong alone with explicit cache policies, for studying
 * the coherence options. store_policy / load_policy: 0 plain, 1 sc0, 2 nt, 16 sc1, 17 sc0|sc1.
 * Returns the half round trip in nanoseconds through *half_rtt_ns; xcc ids through xcc[2].
 */
int ar_pingpong(int placement, int store_policy, int load_policy, int rounds, double* half_rtt_ns,
                int* xcc);

/*
 * ar_torn_lines: 16-byte single-copy atomicity probe. One workgroup rewrites `nlines` 16-byte
 * lines (1..64) `gens` times with one 16-byte store each while a workgroup on another XCD
 * (placement AR_PLACE_XCD) or the same XCD reads them; *torn counts reads whose four words came
 * from different writes, *reads the reads made. Synchronous.
 */
int ar_torn_lines(int placement, int nlines, int gens, uint64_t* torn, uint64_t* reads);

/*
 * ar_stream_copy: copy `bytes` (a multiple of 16) from device `src` to device `dst` (both 16-byte
 * aligned, not overlapping) on `stream`, with non-temporal 16-byte loads and stores in launches
 * of at most 1 GiB each. It is the device's reference for achievable HBM bandwidth (every byte read
 * once and written once) and the kernel of known size that scales rocprof's HBM byte counters.
 * Asynchronous; AR_EINVAL for null, misaligned or ragged arguments.
 */
int ar_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LATENCY_COLLECTIVES_AR_H */
