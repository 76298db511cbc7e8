// Barrier-free AllReduce (sum) kernels for N ranks emulated on one gfx950 device.
//
// Every emulated rank is a group of `ctas` co-resident workgroups with its own input, output and
// block of the symmetric scratch allocation. Ranks exchange data only through global stores into
// another rank's scratch block and polling of their own block; no kernel uses a device-wide
// barrier. Workgroup c of rank r only ever talks to workgroup c of the other ranks, and inside
// it a unit (8 or 16 bytes of payload) is always handled by the same lane, so every credit of
// the double-buffering scheme is a per-lane fact.
//
// One launch runs `iters` AllReduces back to back (1 for an ordinary call); an AllReduce whose
// message does not fit the scratch slots is split into `chunks` equal chunks. Each (iteration,
// chunk) pair is a step with its own sequence number s = e0 + it * chunks + k; step s uses
// scratch buffer s & 1.
//
// Sources: Every µs Matters: Achieving Near Speed-of-Light Latency in GPU Collectives —
// §III.A (one-shot push and two-shot AllReduce), §III.B (memory-barrier cost; the baseline),
// §IV (LL, Sentinel, Bidirectional Communication Double Buffering, Fig. 4); the two-shot
// LL128 atomic AllReduce (Fig. 5) as described in the Pith review of the same paper
// ("Assumptions & free parameters", referee report on §IV.4).

#pragma once

#include "ar_args.h"
#include "ar_device.h"

namespace ar {

struct Ctx {
  int rank, cta, wave, lane, wpb;
  uint32_t T;   // threads per rank
  uint32_t t0;  // first unit index of this wave inside a chunk (lane adds its own offset)
};

__device__ __forceinline__ bool decode(const Args& a, Ctx& c) {
  const int w = blockIdx.x;
  int rank, cta;
  if (a.placement == PLACE_XCD) {
    // Dispatch round j puts workgroup 8j + x on XCD x. With N > 8, R ranks share every XCD; with
    // N dividing 8, XCDs x, x + N, ... all belong to rank x and its workgroups alternate over them.
    const int xcd = w & 7, j = w >> 3, R = a.ranks_per_xcd, X = a.xcds_per_rank;
    if (X > 1) {
      rank = xcd % a.nranks;
      cta = j * X + xcd / a.nranks;
    } else {
      rank = xcd + 8 * (j % R);
      cta = j / R;
    }
  } else if (a.placement == PLACE_SAME) {
    if ((w & 7) != 0) return false;
    const int j = w >> 3;
    rank = j / a.ctas;
    cta = j % a.ctas;
  } else {
    rank = w / a.ctas;
    cta = w % a.ctas;
  }
  if (rank >= a.nranks || cta >= a.ctas) return false;
  c.rank = rank;
  c.cta = cta;
  c.wave = threadIdx.x >> 6;
  c.lane = threadIdx.x & 63;
  c.wpb = blockDim.x >> 6;
  c.T = a.ctas * blockDim.x;
  c.t0 = cta * blockDim.x + c.wave * kWave;
  return true;
}

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Start of region g in rank `rank`'s block; in a near region every slot's data starts at the
// rank's position inside the slot's pitch; in a two-half near region at the granule of each pitch
// homed near the XCD half `half` of the workgroups that poll it (0: the rank's first XCD). In a
// two-page near region the descriptor of double buffer `buf` = 1 is moved so that the slot
// offsets of buffer 1 (from N slots on) land in the second page: at its start, or one granule
// before it where bit 3 of the rank's position says that page's granule homes are mirrored.
__device__ __forceinline__ uint8_t* region_base(const Args& a, int rank, const Region& g,
                                                uint32_t half = 0, uint32_t buf = 0) {
  const uint32_t nib = static_cast<uint32_t>((g.home_pos >> (4 * rank)) & 15u);
  const uint32_t pos = nib & 7u;
  const uint32_t lead = g.near == kNearTwoHalves ? ((pos ^ half) & 1u) * kGranule : pos * kNearSub;
  const int64_t second =
      buf != 0 && g.bstride != 0
          ? static_cast<int64_t>(g.bstride) - static_cast<int64_t>((nib >> 3) * kGranule) -
                static_cast<int64_t>(a.nranks) * g.slot
          : 0;
  return a.base + static_cast<uint64_t>(rank) * a.stride + g.off + lead + second;
}

// Byte offset of unit i (UB bytes) inside a slot: contiguous in the regular regions; in a near
// region, 8 KiB chunks of units, one per 16 KiB (2 granules) of the slot's pitch. In a two-half
// near region (a rank on two XCDs, one in each half of the chip, its workgroups alternating over
// them) workgroup w's units go to the granules of w's half: workgroups 2k and 2k + 1 share the
// k-th block of their granules, and region_base picks the granule.
template <int UB = 16>
__device__ __forceinline__ uint32_t slot_off(const Region& g, uint32_t i) {
  const uint32_t byte = i * static_cast<uint32_t>(UB);
  if (g.near == kNearTwoHalves) {
    const uint32_t T = blockDim.x, bw = T * static_cast<uint32_t>(UB);
    const uint32_t w = i / T, k = w >> 1, m = kGranule / bw;
    return (k / m) * (2 * kGranule) + (k % m) * bw + (byte - w * bw);
  }
  return g.near ? ((byte / kGranule) * (2 * kGranule) + byte % kGranule) : byte;
}

__device__ __forceinline__ rsrc_t region_rsrc(const Args& a, int rank, const Region& g,
                                              uint32_t half = 0, uint32_t buf = 0) {
  return make_rsrc(region_base(a, rank, g, half, buf), g.bytes);
}

// Region of the j-th peer after rank r (q = (r + j) mod N), or a descriptor that drops every
// access when j >= N (the peer does not exist); keeps the push loops free of branches.
__device__ __forceinline__ rsrc_t peer_rsrc(const Args& a, int r, int j, const Region& g,
                                            uint32_t half = 0, uint32_t buf = 0) {
  int q = r + j;
  if (q >= a.nranks) q -= a.nranks;
  const bool live = j < a.nranks;
  return make_rsrc(region_base(a, live ? q : 0, g, half, buf), live ? g.bytes : 0u);
}

// Where a poll loop reports a timeout: the few kernel arguments the slow path needs, passed by
// value so that the argument block never has to be copied to private memory.
struct PollEnv {
  uint32_t* ctl;
  uint32_t* status;
  uint64_t timeout_ticks;
  int algo;
};

__device__ __forceinline__ PollEnv poll_env(const Args& a) {
  return PollEnv{a.ctl, a.status, a.timeout_ticks, a.algo};
}

__device__ __noinline__ uint64_t poll_check_call(PollEnv e, uint64_t t_first, int rank, int peer,
                                                 uint64_t step);

// Called after every 1024 unsuccessful polls with the clock value of the first such call (0 on
// the first call). Returns that start value (set now if it was 0) while the wave may keep
// polling, and 0 when it must give up: either another wave already aborted, or this poll has
// waited longer than the timeout, in which case this wave raises the abort flag and, if it is
// the first, records where it stopped. Everything is passed by value so that no kernel keeps
// state in private memory for it. The result is the same in every lane and is handed back in
// scalar registers: returned in vector registers it would make every poll loop a divergent loop
// (exec-mask bookkeeping in each round, exits merged behind extra waits), measured 4-11 % higher
// p50 on the 2-, 4- and 8-rank latency workloads.
__device__ __forceinline__ uint64_t poll_check(PollEnv e, uint64_t t_first, int rank, int peer,
                                               uint64_t step) {
  const uint64_t t = poll_check_call(e, t_first, rank, peer, step);
  return (static_cast<uint64_t>(uni(static_cast<uint32_t>(t >> 32))) << 32) |
         uni(static_cast<uint32_t>(t));
}

// The out-of-line body of poll_check (kept out of the poll loops' code).
__device__ __noinline__ uint64_t poll_check_call(PollEnv e, uint64_t t_first, int rank, int peer,
                                                 uint64_t step) {
  const uint64_t now = wall_clock64();
  if (t_first == 0) return now == 0 ? 1 : now;
  const uint32_t ab = uni(__hip_atomic_load(&e.ctl[CTL_ABORT], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT));
  if (ab != 0) return 0;
  if (now - t_first <= e.timeout_ticks) return t_first;
  if (threadIdx.x % kWave == static_cast<unsigned>(__builtin_ctzll(__ballot(1)))) {
    if (__hip_atomic_exchange(&e.ctl[CTL_ABORT], 1u, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT) == 0) {
      __hip_atomic_store(&e.status[ST_RANK], static_cast<uint32_t>(rank), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&e.status[ST_PEER], static_cast<uint32_t>(peer), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&e.status[ST_STEP_LO], static_cast<uint32_t>(step), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&e.status[ST_STEP_HI], static_cast<uint32_t>(step >> 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&e.status[ST_ALGO], static_cast<uint32_t>(e.algo), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&e.status[ST_CODE], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
  return 0;
}

// Issue one round of poll loads: one 16-byte coherent load per possible source into t[q], in
// one basic block. Sources already received (or that do not exist) read the drop offset.
template <int NMAX>
__device__ __forceinline__ void poll_issue(rsrc_t own, uint32_t off0, uint32_t qstride,
                                           uint32_t pend, u32x4 (&t)[NMAX]) {
#pragma unroll
  for (int q = 0; q < NMAX; ++q)
    t[q] = ld16<kCoh>(own, ((pend >> q) & 1u) ? off0 + static_cast<uint32_t>(q) * qstride : kDrop);
}

// Finish polling the sources in `pend`, whose first round of loads is already in t[]: keep each
// line that `ready` accepts in v[] and load the others again until none is missing.
template <int NMAX, class Ready>
__device__ __forceinline__ bool poll_rest(const Args& a, rsrc_t own, uint32_t off0,
                                          uint32_t qstride, uint32_t pend, u32x4 (&t)[NMAX],
                                          u32x4 (&v)[NMAX], Ready ready, int rank, uint64_t step) {
  uint32_t spins = 0;
  uint64_t t_first = 0;
  while (true) {
    compiler_fence();
#pragma unroll
    for (int q = 0; q < NMAX; ++q) {
      if ((pend >> q) & 1u) {
        v[q] = t[q];
        if (ready(t[q])) pend &= ~(1u << q);
      }
    }
    const uint64_t waiting = __ballot(pend != 0);
    if (waiting == 0) return true;
    if ((++spins & 1023u) == 0) {
      const int lane = __builtin_ctzll(waiting);
      const uint32_t p = __shfl(pend, lane);
      t_first = poll_check(poll_env(a), t_first, rank, __builtin_ctz(p), step);
      if (t_first == 0) return false;
    }
    poll_issue<NMAX>(own, off0, qstride, pend, t);
  }
}

// Latency-path poll: every source in `mask` is loaded straight into v[q] each round, whether
// or not it has arrived (a slot that has arrived keeps its value until this rank re-arms it),
// until all of them pass `ready`. No per-source branches or copies: after the last load returns
// only the readiness test and the ballot stand between the data and the fold. V is the unit
// (u32x4 or u32x2).
template <int NMAX, class Ready, class V>
__device__ __forceinline__ bool poll_all(const Args& a, rsrc_t own, uint32_t off0,
                                         uint32_t qstride, uint32_t mask, V (&v)[NMAX],
                                         Ready ready, int rank, uint64_t step) {
  uint32_t spins = 0;
  uint64_t t_first = 0;
  while (true) {
#pragma unroll
    for (int q = 0; q < NMAX; ++q)
      ld_vec<kCoh>(own, ((mask >> q) & 1u) ? off0 + static_cast<uint32_t>(q) * qstride : kDrop,
                   v[q]);
    compiler_fence();
    bool ok = true;
#pragma unroll
    for (int q = 0; q < NMAX; ++q) ok = ok & ((((mask >> q) & 1u) == 0u) | ready(v[q]));
    const uint64_t waiting = __ballot(!ok);
    if (waiting == 0) return true;
    if ((++spins & 1023u) == 0) {
      t_first = poll_check(poll_env(a), t_first, rank, -1, step);
      if (t_first == 0) return false;
    }
  }
}

// The same with two rounds of loads in flight, the second issued about half a coherent round trip
// after the first: a line that lands just after one round passed the coherence point is seen by
// the other round half a round trip later instead of a whole one. Each round is NMAX loads, so
// "the older round has returned" is `vmcnt <= NMAX` (vector memory operations complete in issue
// order). A round still in flight at exit writes only its own registers.
template <int NMAX, class Ready>
__device__ __forceinline__ bool poll_all2(const Args& a, rsrc_t own, uint32_t off0,
                                          uint32_t qstride, uint32_t mask, u32x4 (&v)[NMAX],
                                          Ready ready, int rank, uint64_t step) {
  u32x4 w[NMAX];
  auto issue = [&](u32x4 (&t)[NMAX]) {
#pragma unroll
    for (int q = 0; q < NMAX; ++q)
      t[q] = ld16<kCoh>(own, ((mask >> q) & 1u) ? off0 + static_cast<uint32_t>(q) * qstride : kDrop);
  };
  auto all_ready = [&](const u32x4 (&t)[NMAX]) {
    bool ok = true;
#pragma unroll
    for (int q = 0; q < NMAX; ++q) ok = ok & ((((mask >> q) & 1u) == 0u) | ready(t[q]));
    return __ballot(!ok) == 0;
  };
  uint32_t spins = 0;
  uint64_t t_first = 0;
  issue(v);
  compiler_fence();
  __builtin_amdgcn_s_sleep(2);
  while (true) {
    issue(w);  // round B of this pass, issued only here so that it never needs a copy
    compiler_fence();
    wait_vm<NMAX>();  // round A has returned
    compiler_fence();
    if (all_ready(v)) return true;
    issue(v);
    compiler_fence();
    wait_vm<NMAX>();  // round B has returned
    compiler_fence();
    if (all_ready(w)) {
#pragma unroll
      for (int q = 0; q < NMAX; ++q) v[q] = w[q];
      return true;
    }
    if ((++spins & 511u) == 0) {
      t_first = poll_check(poll_env(a), t_first, rank, -1, step);
      if (t_first == 0) return false;
    }
  }
}

template <int NMAX, class Ready>
__device__ __forceinline__ bool poll_lines(const Args& a, rsrc_t own, uint32_t off0,
                                           uint32_t qstride, uint32_t pend, u32x4 (&v)[NMAX],
                                           Ready ready, int rank, uint64_t step) {
  u32x4 t[NMAX];
  poll_issue<NMAX>(own, off0, qstride, pend, t);
  return poll_rest<NMAX>(a, own, off0, qstride, pend, t, v, ready, rank, step);
}

// Fold the N sources of one unit in rank order 0..N-1; the rank's own value is `x`. The first W
// words of each v[q] are payload. Sources q >= N (the kernel is built for NMAX >= N ranks) add
// the additive identity of the fold, -0.0 for binary32 (x + -0.0 is x for every x, +0 and -0
// included) and 0 for int32, so the fold needs no branch on the run-time rank count.
template <int DT, int NMAX, int W, class V>
__device__ __forceinline__ void fold_rank_order(int N, int r, const uint32_t* x,
                                                const V (&v)[NMAX], uint32_t* o) {
  // identity word: two bf16 -0.0 (each widens to binary32 -0.0), one binary32 -0.0, int32 0
  constexpr uint32_t kId = DT == DT_I32 ? 0u : DT == DT_BF16 ? 0x80008000u : 0x80000000u;
  Fold<DT, W> f;
#pragma unroll
  for (int q = 0; q < NMAX; ++q) {
    uint32_t src[W];
#pragma unroll
    for (int i = 0; i < W; ++i) src[i] = (q == r) ? x[i] : (q < N ? v[q][i] : kId);
    if (q == 0)
      f.init(src);
    else
      f.add(src);
  }
  f.pack(o);
}

__device__ __forceinline__ uint32_t peer_mask(int N, int r) {
  return ((N >= 32) ? 0xFFFFFFFFu : ((1u << N) - 1u)) & ~(1u << r);
}

// Write the sentinel unit back into the slots of the sources in `mask` (source q's unit at
// off0 + q * qstride): NMAX stores, branch-free.
template <int NMAX, class V>
__device__ __forceinline__ void rearm(rsrc_t own, uint32_t off0, uint32_t qstride, uint32_t mask,
                                      V sent) {
#pragma unroll
  for (int q = 0; q < NMAX; ++q)
    st_vec<kCoh>(own, ((mask >> q) & 1u) ? off0 + static_cast<uint32_t>(q) * qstride : kDrop,
                 sent);
}

// Push one unit (a 16-byte line or an 8-byte unit) to the j-th peer after r, for j = 1..NMAX-1
// (NMAX-1 stores, branch-free; peers that do not exist and idle lanes drop their store).
template <int NMAX, class V>
__device__ __forceinline__ void push_peers(const Args& a, int r, const Region& g, uint32_t off,
                                           V line, uint32_t half = 0, uint32_t buf = 0) {
#pragma unroll
  for (int j = 1; j < NMAX; ++j) st_vec<kCoh>(peer_rsrc(a, r, j, g, half, buf), off, line);
}

// Ordering of a step (every step function follows it):
//  * Before its first push a step waits until every store of the previous step has completed.
//    The re-arm (or clearing) stores of step s must be visible before this rank's push of step
//    s+1, because that push is the credit that lets a peer write the same buffer again in step
//    s+2. Coherent stores are visible once they have completed.
//  * A step returns only after its output stores have completed.
// In the latency path (each lane owns at most one unit) a single wait after the input load
// covers both: the load and every older store have completed when the pushes are issued. The
// polls follow the pushes: in lockstep a poll issued before this rank's own push reaches memory
// before the peers' data can have landed and only costs a round trip.

// ------------------------------------------------------------------ one-shot, LL protocol
//
// Push: every 8 bytes of the rank's chunk go to every peer as one 16-byte line {payload, s}
// (§IV "LL"). Receive: poll each peer's line until its flag equals s, then fold in rank order.
// Nothing needs resetting: an old line carries an older sequence number.
template <int DT, int NMAX, bool kMulti, bool TWO_PAGE = false>
__device__ bool step_oneshot_ll(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                rsrc_t out_r, int k, uint64_t& t0,
                                uint64_t& t1) {
  static_assert(!TWO_PAGE || !kMulti, "two-page near slots are planned for the one-pass kernel");
  const int N = a.nranks, r = c.rank;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  // two-page near ll region (TWO_PAGE, the only instance planned on it): the step's ll
  // descriptors are those of buffer b
  const uint32_t bd = TWO_PAGE ? b : 0u;
  const uint32_t elo = static_cast<uint32_t>(s), ehi = static_cast<uint32_t>(s >> 32);
  const uint32_t slot = a.ll.slot, CU = a.chunk_units;
  const uint32_t unit0 = static_cast<uint32_t>(k) * CU;
  const bool sends = r != a.withhold;
  const uint32_t mine = (b * N + r) * slot;
  const rsrc_t own = region_rsrc(a, r, a.ll, 0, bd);
  const uint32_t peers = peer_mask(N, r);
  auto ready = [elo, ehi](u32x4 l) { return (l.z == elo) & (l.w == ehi); };
  auto finish = [&](uint32_t i, bool act, const uint32_t* x, const u32x4 (&v)[NMAX]) {
    uint32_t o[2];
    fold_rank_order<DT, NMAX, 2>(N, r, x, v, o);
    store_unit<DT, 8, kOut>(out_r, act ? (unit0 + i) * 8u : kDrop, a.nbytes, o);
  };
  if constexpr (!kMulti) {
    // one pass: the plan gives this rank at least one lane per unit of the chunk
    const uint32_t i = c.t0 + c.lane;
    const bool act = i < CU;
    uint32_t off0 = b * N * slot + slot_off(a.ll, i);
    uint32_t in_off = act ? (unit0 + i) * 8u : kDrop;
    uint32_t push_off = act ? mine + slot_off(a.ll, i) : kDrop;
    pin(off0);
    pin(in_off);
    pin(push_off);
    stamp_start(t0, k);
    uint32_t x[2];
    load_unit<DT, 8>(in_r, in_off, a.nbytes, x);
    compiler_fence();
    wait_vm<0>();
    if (sends) push_peers<NMAX>(a, r, a.ll, push_off, u32x4{x[0], x[1], elo, ehi}, 0, bd);
    u32x4 v[NMAX];
    if constexpr (NMAX <= 8) {
      if (!poll_all2<NMAX>(a, own, off0, slot, act ? peers : 0u, v, ready, r, s)) return false;
    } else {
      if (!poll_all<NMAX>(a, own, off0, slot, act ? peers : 0u, v, ready, r, s)) return false;
    }
    finish(i, act, x, v);
    wait_all_mem();
    t1 = now_ticks();
    return true;
  } else {
    stamp_start(t0, k);
    wait_all_mem();
    if (sends) {
      for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
        const uint32_t i = i0 + c.lane;
        const bool act = i < CU;
        uint32_t w[2];
        load_unit<DT, 8>(in_r, act ? (unit0 + i) * 8u : kDrop, a.nbytes, w);
        push_peers<NMAX>(a, r, a.ll, act ? mine + slot_off(a.ll, i) : kDrop,
                         u32x4{w[0], w[1], elo, ehi});
      }
    }
    for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CU;
      uint32_t x[2];
      load_unit<DT, 8>(in_r, act ? (unit0 + i) * 8u : kDrop, a.nbytes, x);
      u32x4 v[NMAX];
      if (!poll_lines<NMAX>(a, own, b * N * slot + slot_off(a.ll, i), slot, act ? peers : 0u, v,
                            ready, r, s))
        return false;
      finish(i, act, x, v);
    }
    wait_all_mem();
    t1 = now_ticks();
    return true;
  }
}

// ------------------------------------------------------------------ one-shot, sentinel protocol
//
// Push raw units into every peer's slot (§IV "Sentinel"). Receive: poll until no element of a
// peer's unit equals the sentinel, fold in rank order, then write the sentinel back so the slot
// is armed for step s+2 (the same buffer). The output store is issued before the re-arm so that
// the step can return as soon as the output has landed. A unit is UB = 16 bytes, or 8 bytes in
// the narrow one-pass kernel: twice the lanes, each folding half as many words, which shortens
// the serial fold of every wave (the fold is one dependent add chain per word and source).
template <int DT, int NMAX, bool kMulti, int UB = 16, bool TWO_PAGE = false>
__device__ bool step_oneshot_sentinel(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                      rsrc_t out_r, int k, uint64_t& t0,
                                      uint64_t& t1) {
  static_assert(!kMulti || UB == 16, "the multi-pass path moves 16-byte units");
  static_assert(!TWO_PAGE || !kMulti, "two-page near slots are planned for the one-pass kernel");
  using V = unit_t<UB>;
  constexpr int W = UB / 4;
  const int N = a.nranks, r = c.rank;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot = a.p1.slot, CU = a.chunk_units;
  const uint32_t unit0 = static_cast<uint32_t>(k) * CU;
  const bool sends = r != a.withhold;
  const uint32_t mine = (b * N + r) * slot;
  // the XCD half of this workgroup (two-half near slots; 0 elsewhere)
  const uint32_t half = a.p1.near == kNearTwoHalves ? static_cast<uint32_t>(c.cta) & 1u : 0u;
  // two-page near p1 region (TWO_PAGE, the only instance planned on it): the step's p1
  // descriptors are those of buffer b
  const uint32_t bd = TWO_PAGE ? b : 0u;
  const rsrc_t own = region_rsrc(a, r, a.p1, half, bd);
  const uint32_t peers = peer_mask(N, r);
  const V sent = sentinel_unit<DT, UB>();
  auto ready = [](V l) { return vec_clear<DT>(l); };
  auto finish = [&](uint32_t i, bool act, const uint32_t* x, const V (&v)[NMAX],
                    uint32_t off0) {
    uint32_t o[W];
    fold_rank_order<DT, NMAX, W>(N, r, x, v, o);
    store_unit<DT, UB, kOut>(out_r, act ? (unit0 + i) * UB : kDrop, a.nbytes, o);
    rearm<NMAX>(own, off0, slot, act ? peers : 0u, sent);
  };
  if constexpr (!kMulti) {
    // one pass: the plan gives this rank at least one lane per unit of the chunk
    const uint32_t i = c.t0 + c.lane;
    const bool act = i < CU;
    uint32_t off0 = b * N * slot + slot_off<UB>(a.p1, i);
    uint32_t in_off = act ? (unit0 + i) * UB : kDrop;
    uint32_t push_off = act ? mine + slot_off<UB>(a.p1, i) : kDrop;
    pin(off0);
    pin(in_off);
    pin(push_off);
    stamp_start(t0, k);
    uint32_t x[W];
    load_unit<DT, UB>(in_r, in_off, a.nbytes, x);
    compiler_fence();
    wait_vm<0>();
    if (sends) {
      V line;
#pragma unroll
      for (int e = 0; e < W; ++e) line[e] = x[e];
      push_peers<NMAX>(a, r, a.p1, push_off, line, half, bd);
    }
    V v[NMAX];
    // one round of polls at a time: with a second round in flight the sentinel path measured
    // slower (the exit then waits for the other round's loads)
    if (!poll_all<NMAX>(a, own, off0, slot, act ? peers : 0u, v, ready, r, s)) return false;
    uint32_t o[W];
    fold_rank_order<DT, NMAX, W>(N, r, x, v, o);
    store_unit<DT, UB, kOut>(out_r, act ? (unit0 + i) * UB : kDrop, a.nbytes, o);
    compiler_fence();
    wait_vm<0>();  // the output has landed: the AllReduce is complete for this lane
    t1 = now_ticks();
    // Re-arm the slots for step s + 2 after the output: the next step's first push waits for
    // these stores, and the credit chain only needs them before that push.
    rearm<NMAX>(own, off0, slot, act ? peers : 0u, sent);
    return true;
  } else {
    stamp_start(t0, k);
    wait_all_mem();
    if (sends) {
      for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
        const uint32_t i = i0 + c.lane;
        const bool act = i < CU;
        uint32_t w[4];
        load_unit<DT, 16>(in_r, act ? (unit0 + i) * 16u : kDrop, a.nbytes, w);
        push_peers<NMAX>(a, r, a.p1, act ? mine + slot_off(a.p1, i) : kDrop,
                         u32x4{w[0], w[1], w[2], w[3]});
      }
    }
    for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CU;
      const uint32_t off0 = b * N * slot + slot_off(a.p1, i);
      uint32_t x[4];
      load_unit<DT, 16>(in_r, act ? (unit0 + i) * 16u : kDrop, a.nbytes, x);
      u32x4 v[NMAX];
      if (!poll_lines<NMAX>(a, own, off0, slot, act ? peers : 0u, v, ready, r, s)) return false;
      finish(i, act, x, v, off0);
    }
    wait_all_mem();
    t1 = now_ticks();
    return true;
  }
}

// ------------------------------------------------------------------ two-shot helpers
//
// The message is cut into N partitions of `part_units` units (the last ones padded with zeros);
// partition p belongs to owner p. Chunk k of every partition moves in step k. Lane i of a wave
// handles unit i of the chunk in every partition.

// Load unit i of the chunk in the partition of the j-th peer after rank r into w[j], for
// j = jfirst..NMAX-1 (zeros for peers that do not exist or an idle lane): NMAX-jfirst loads.
template <int DT, int NMAX, int CP = kPlain, int UB = 16>
__device__ __forceinline__ void load_partitions(const Args& a, int r, rsrc_t in_r, int k,
                                                uint32_t i, bool act, int jfirst,
                                                uint32_t (&w)[NMAX][UB / 4]) {
  const int N = a.nranks;
  const uint32_t CU = a.chunk_units, P = a.part_units;
#pragma unroll
  for (int j = 0; j < NMAX; ++j) {
    if (j < jfirst) {
#pragma unroll
      for (int e = 0; e < UB / 4; ++e) w[j][e] = 0u;
      continue;
    }
    int p = r + j;
    if (p >= N) p -= N;
    const bool live = act && j < N;
    load_unit<DT, UB, CP, false>(in_r, live ? (p * P + k * CU + i) * UB : kDrop, a.nbytes, w[j]);
  }
  // all loads are in flight before the one scalar branch for an odd bf16 tail
  if (odd_tail<DT>(a.nbytes)) {
    asm volatile("");
#pragma unroll
    for (int j = jfirst; j < NMAX; ++j) {
      int p = r + j;
      if (p >= N) p -= N;
      clear_odd_tail<UB>((p * P + k * CU + i) * UB, a.nbytes, w[j]);
    }
  }
}

// Store the reduced unit i of every owner in `mask` (already in v[]) into the output; an odd bf16
// tail is written after all of them, behind one branch.
template <int DT, int NMAX, int UB = 16>
__device__ __forceinline__ void allgather_store(const Args& a, rsrc_t out_r, uint32_t mask, int k,
                                                uint32_t i, const unit_t<UB> (&v)[NMAX]) {
  const uint32_t CU = a.chunk_units, P = a.part_units;
#pragma unroll
  for (int p = 0; p < NMAX; ++p) {
    const uint32_t off = ((mask >> p) & 1u) ? (p * P + k * CU + i) * UB : kDrop;
    if constexpr (UB == 16)
      st16<kOut>(out_r, off, v[p]);
    else
      st8<kOut>(out_r, off, v[p]);
  }
  if (odd_tail<DT>(a.out_nbytes)) {
    asm volatile("");
    const uint32_t last = a.out_nbytes & ~3u;
#pragma unroll
    for (int p = 0; p < NMAX; ++p) {
      const uint32_t off = (p * P + k * CU + i) * UB;
      const bool tail = ((mask >> p) & 1u) && off <= last && last < off + UB;
      uint32_t word = v[p][0];
#pragma unroll
      for (int e = 1; e < UB / 4; ++e) word = (off + 4u * e == last) ? v[p][e] : word;
      st2<kOut>(out_r, tail ? last : kDrop, static_cast<uint16_t>(word & 0xFFFFu));
    }
  }
}

// All-gather receive of unit i: the reduced unit of every other owner, already polled into v[],
// is copied to `out` and its slot re-armed.
template <int DT, int NMAX, int UB = 16>
__device__ __forceinline__ void allgather_out(const Args& a, int r, rsrc_t out_r, rsrc_t own2,
                                              uint32_t off0, uint32_t mask, int k, uint32_t i,
                                              const unit_t<UB> (&v)[NMAX], unit_t<UB> sent) {
  allgather_store<DT, NMAX, UB>(a, out_r, mask, k, i, v);
  rearm<NMAX>(own2, off0, a.p2.slot, mask, sent);
}

// ------------------------------------------------------------------ two-shot (RS + AG)
//
// Reduce-scatter: partition p's chunk goes to owner p's slot r. The owner folds its partition in
// rank order, writes it to its own output and pushes the result to every peer's all-gather slot
// r; every rank copies the other owners' results into its output (§III.A "Two-shot").
// MODE 0 is that AllReduce. The standalone collectives run one half of it on the same slots:
// MODE 1 the reduce-scatter alone (the folded partition is the whole output), MODE 2 the
// all-gather alone (the rank's input is the partition it owns). Their partitions are exact, so
// the last chunk may be short; an AllReduce's partitions are padded to whole chunks.
template <int DT, int NMAX, int UB = 16, int MODE = 0, bool TWO_PAGE = false>
__device__ bool step_twoshot(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r, rsrc_t out_r,
                             int k, uint64_t& t0,
                             uint64_t& t1) {
  using V = unit_t<UB>;
  constexpr int W = UB / 4;
  const int N = a.nranks, r = c.rank;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot1 = a.p1.slot, slot2 = a.p2.slot, CU = a.chunk_units, P = a.part_units;
  const bool sends = r != a.withhold;
  // two-page near regions (TWO_PAGE, the only instance planned on them): every p1 / p2
  // descriptor of the step is that of buffer b
  const uint32_t bd = TWO_PAGE ? b : 0u;
  const rsrc_t own1 = region_rsrc(a, r, a.p1, 0, bd);
  const rsrc_t own2 = region_rsrc(a, r, a.p2, 0, bd);
  const uint32_t peers = peer_mask(N, r);
  const V sent = sentinel_unit<DT, UB>();
  auto ready = [](V l) { return vec_clear<DT>(l); };
  const uint32_t mine1 = (b * N + r) * slot1, mine2 = (b * N + r) * slot2;
  // one pass: the plan gives this rank at least one lane per unit of the chunk (wider chunks
  // run step_twoshot_bulk, or the loop kernels of the standalone collectives)
  {
    const uint32_t i = c.t0 + c.lane;
    const bool act = i < CU && k * CU + i < P;
    const uint32_t mask = act ? peers : 0u;
    uint32_t off1 = b * N * slot1 + slot_off<UB>(a.p1, i);
    const uint32_t off2 = b * N * slot2 + slot_off<UB>(a.p2, i);
    const uint32_t uoff = (r * P + k * CU + i) * UB;
    // Address arithmetic of the step before its start stamp: the input offset of unit i in the
    // partition of the j-th rank after r, and the push offsets of both phases.
    uint32_t in_off[NMAX];
#pragma unroll
    for (int j = 0; j < NMAX; ++j) {
      int p = r + j;
      if (p >= N) p -= N;
      in_off[j] = act && j < N ? (p * P + k * CU + i) * UB : kDrop;
      pin(in_off[j]);
    }
    uint32_t push1 = act ? mine1 + slot_off<UB>(a.p1, i) : kDrop;
    uint32_t push2 = act ? mine2 + slot_off<UB>(a.p2, i) : kDrop;
    pin(off1);
    pin(push1);
    pin(push2);
    stamp_start(t0, k);
    uint32_t o[W];
    if constexpr (MODE == 2) {
      load_unit<DT, UB>(in_r, act ? (k * CU + i) * UB : kDrop, a.nbytes, o);
      compiler_fence();
      wait_vm<0>();
    } else {
      uint32_t w[NMAX][W];
#pragma unroll
      for (int j = 0; j < NMAX; ++j)
        load_unit<DT, UB, kPlain, false>(in_r, in_off[j], a.nbytes, w[j]);  // w[0]: own partition
      // all loads are in flight before the one scalar branch for an odd bf16 tail
      if (odd_tail<DT>(a.nbytes)) {
        asm volatile("");
#pragma unroll
        for (int j = 0; j < NMAX; ++j) clear_odd_tail<UB>(in_off[j], a.nbytes, w[j]);
      }
      compiler_fence();
      wait_vm<0>();
      if (sends) {
        const uint32_t off = push1;
#pragma unroll
        for (int j = 1; j < NMAX; ++j) {
          V line;
#pragma unroll
          for (int e = 0; e < W; ++e) line[e] = w[j][e];
          st_vec<kCoh>(peer_rsrc(a, r, j, a.p1, 0, bd), off, line);
        }
      }
      V v[NMAX];
      if (!poll_all<NMAX>(a, own1, off1, slot1, mask, v, ready, r, s)) return false;
      fold_rank_order<DT, NMAX, W>(N, r, w[0], v, o);
    }
    if constexpr (MODE == 1) {
      store_unit<DT, UB, kOut>(out_r, act ? (k * CU + i) * UB : kDrop, a.out_nbytes, o);
      rearm<NMAX>(own1, off1, slot1, mask, sent);
    } else {
      if (sends) {
        V line;
#pragma unroll
        for (int e = 0; e < W; ++e) line[e] = o[e];
        push_peers<NMAX>(a, r, a.p2, push2, line, 0, bd);
      }
      store_unit<DT, UB, kOut>(out_r, act ? uoff : kDrop, a.out_nbytes, o);
      V v2[NMAX];
      if (!poll_all<NMAX>(a, own2, off2, slot2, mask, v2, ready, r, s)) return false;
      // every other owner's reduced unit into the output
      allgather_store<DT, NMAX, UB>(a, out_r, mask, k, i, v2);
      compiler_fence();
      wait_vm<0>();  // every output store has landed: the AllReduce is complete for this lane
      t1 = now_ticks();
      // Re-arm both phases' slots for step s + 2 after the outputs: the next step's first push
      // waits for these stores, and the credit chain only needs them before that push.
      if constexpr (MODE == 0) rearm<NMAX>(own1, off1, slot1, mask, sent);
      rearm<NMAX>(own2, off2, slot2, mask, sent);
      return true;
    }
    compiler_fence();
    wait_vm<NMAX>();  // every output store has landed; the NMAX re-arm stores may be in flight
    t1 = now_ticks();
    return true;
  }
}

// ------------------------------------------------------------------ peer-split one-pass kernels
//
// A wave's coherent stores complete one after another: on MI355X every further store of one
// wave (8 bytes per lane, any number of active lanes) adds ~13-24 ns before the last of them
// has completed, while stores of different waves complete in parallel (16 single stores from
// 16 waves of one workgroup: ~350 ns for the last, against ~600 ns from one wave). With N-1
// pushes per wave the last peer's unit therefore lands (N-2) store times after the first. The
// split kernels give every 64 units of a chunk a workgroup of kSplit waves that share those
// units: wave g pushes to, polls and re-arms only the peers j = 1 + g + m * kSplit after this
// rank (m = 0..J-1, J = ceil((NMAX - 1) / kSplit)), so each wave issues J stores per phase and
// J loads per poll round. The polled units meet in LDS, one row per source rank, double-buffered
// by step parity; after one workgroup barrier the rank-order fold reads them back. A peer q is
// pushed to, polled and re-armed by the same wave, so the double-buffer credit chain of the
// unsplit kernels holds per (lane, peer) unchanged.
constexpr int kSplit = kSplitWaves;

template <int NMAX>
constexpr int split_j() {
  return (NMAX - 1 + kSplit - 1) / kSplit;
}

// Set by a wave whose poll timed out before the barrier, so that the other waves of the
// workgroup, released by the same barrier, fail the step too (zeroed at kernel entry).
__shared__ uint32_t g_split_fail;

// Workgroup barrier after this wave's LDS writes have completed. No wait on vector memory: the
// pushes of the step may still be in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The m-th peer of wave g: its distance j after rank r and its rank q (r itself when j >= N).
struct SplitPeer {
  int j;
  int q;
  bool live;
};
__device__ __forceinline__ SplitPeer split_peer(int N, int r, int g, int m) {
  SplitPeer p;
  p.j = 1 + g + m * kSplit;
  p.live = p.j < N;
  int q = r + p.j;
  if (q >= N) q -= N;
  p.q = p.live ? q : r;
  return p;
}

// Base address of region g of the peer (a descriptor that drops every access when the peer is
// absent), computed before the step's start stamp and kept in scalar registers, so that only
// the descriptor's assembly stands between two pushes.
struct PeerBase {
  uint64_t base;
  uint32_t bytes;
};
__device__ __forceinline__ PeerBase peer_base(const Args& a, const SplitPeer& p, const Region& g) {
  PeerBase b;
  b.base = reinterpret_cast<uint64_t>(region_base(a, p.live ? p.q : 0, g));
  b.bytes = p.live ? g.bytes : 0u;
  asm volatile("" : "+s"(b.base), "+s"(b.bytes));
  return b;
}
__device__ __forceinline__ rsrc_t peer_rsrc(const PeerBase& b) {
  return make_rsrc(reinterpret_cast<const void*>(b.base), b.bytes);
}

// Poll the J units at the given offsets of the own slots (kDrop: nothing to wait for) until
// every one passes `ready` (bounded, like poll_all).
template <int J, class Ready, class V>
__device__ __forceinline__ bool poll_list(const Args& a, rsrc_t own, const uint32_t (&off)[J],
                                          V (&u)[J], Ready ready, int rank, uint64_t step) {
  uint32_t spins = 0;
  uint64_t t_first = 0;
  while (true) {
#pragma unroll
    for (int m = 0; m < J; ++m) ld_vec<kCoh>(own, off[m], u[m]);
    compiler_fence();
    bool ok = true;
#pragma unroll
    for (int m = 0; m < J; ++m) ok = ok & ((off[m] == kDrop) | ready(u[m]));
    const uint64_t waiting = __ballot(!ok);
    if (waiting == 0) return true;
    if ((++spins & 1023u) == 0) {
      t_first = poll_check(poll_env(a), t_first, rank, -1, step);
      if (t_first == 0) return false;
    }
  }
}

// Exchange of the polled units through LDS and the rank-order fold of all of them with this
// rank's own unit x (every wave folds; only the caller decides who stores). The LDS rows are
// indexed by source rank and complete before the barrier, so the fold reads NMAX rows and adds
// them with no per-source select (measured 1-5 % lower p50 at 8 ranks than selecting the own
// unit and the identity in registers). Returns false when any wave of the workgroup timed out
// before the barrier.
template <int DT, int NMAX, int UB, int J>
__device__ __forceinline__ bool split_fold(const Ctx& c, uint32_t b, int N, int r,
                                           const SplitPeer (&pe)[J], bool polled,
                                           const unit_t<UB> (&u)[J], const uint32_t* x,
                                           uint32_t* o) {
  using V = unit_t<UB>;
  constexpr int W = UB / 4;
  // row q holds source q's unit: the polled peers', this rank's own (written by wave 0) and, for
  // q >= N, the identity of the fold; absent peers write the spare row NMAX
  __shared__ V xch[2][NMAX + 1][kWave];
#pragma unroll
  for (int m = 0; m < J; ++m) xch[b][pe[m].live ? pe[m].q : NMAX][c.lane] = u[m];
  if (c.wave == 0) {
    V own;
#pragma unroll
    for (int e = 0; e < W; ++e) own[e] = x[e];
    xch[b][r][c.lane] = own;
    if (N < NMAX) {
      constexpr uint32_t kId = DT == DT_I32 ? 0u : DT == DT_BF16 ? 0x80008000u : 0x80000000u;
      V id;
#pragma unroll
      for (int e = 0; e < W; ++e) id[e] = kId;
      for (int q = N; q < NMAX; ++q) xch[b][q][c.lane] = id;
    }
  }
  if (!polled) g_split_fail = 1u;
  lds_barrier();
  V v[NMAX];
#pragma unroll
  for (int q = 0; q < NMAX; ++q) v[q] = xch[b][q][c.lane];
  uint32_t fail = g_split_fail;
  // every row and the failure word are loaded before the failure word is tested, so the test
  // costs no LDS round trip of its own
#pragma unroll
  for (int q = 0; q < NMAX; ++q) asm volatile("" : "+v"(v[q]));
  asm volatile("" : "+v"(fail));
  Fold<DT, W> f;
#pragma unroll
  for (int q = 0; q < NMAX; ++q) {
    uint32_t src[W];
#pragma unroll
    for (int e = 0; e < W; ++e) src[e] = v[q][e];
    if (q == 0)
      f.init(src);
    else
      f.add(src);
  }
  f.pack(o);
  return fail == 0u;
}

// One-shot sentinel AllReduce, peer-split (see above): every wave of the workgroup loads the
// same 64 units, pushes them to its J peers and polls their units; wave 0 stores the output.
template <int DT, int NMAX, int UB>
__device__ bool step_oneshot_split(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                   rsrc_t out_r, int k, uint64_t& t0, uint64_t& t1) {
  using V = unit_t<UB>;
  constexpr int W = UB / 4;
  constexpr int J = split_j<NMAX>();
  const int N = a.nranks, r = c.rank;
  const int g = static_cast<int>(uni(static_cast<uint32_t>(c.wave)));  // wave-uniform
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot = a.p1.slot, CU = a.chunk_units;
  const uint32_t unit0 = static_cast<uint32_t>(k) * CU;
  const bool sends = r != a.withhold;
  const rsrc_t own = region_rsrc(a, r, a.p1);
  const V sent = sentinel_unit<DT, UB>();
  auto ready = [](V l) { return vec_clear<DT>(l); };
  const uint32_t i = static_cast<uint32_t>(c.cta) * kWave + c.lane;  // shared by the waves
  const bool act = i < CU;
  SplitPeer pe[J];
  PeerBase pb[J];
  uint32_t poll_off[J];
  const uint32_t slot0 = b * N * slot + slot_off<UB>(a.p1, i);
#pragma unroll
  for (int m = 0; m < J; ++m) {
    pe[m] = split_peer(N, r, g, m);
    pb[m] = peer_base(a, pe[m], a.p1);
    poll_off[m] = act && pe[m].live ? slot0 + static_cast<uint32_t>(pe[m].q) * slot : kDrop;
    pin(poll_off[m]);
  }
  uint32_t in_off = act ? (unit0 + i) * UB : kDrop;
  uint32_t push_off = act ? (b * N + r) * slot + slot_off<UB>(a.p1, i) : kDrop;
  uint32_t out_off = act && g == 0 ? (unit0 + i) * UB : kDrop;
  pin(in_off);
  pin(push_off);
  pin(out_off);
  stamp_start(t0, k);
  uint32_t x[W];
  load_unit<DT, UB>(in_r, in_off, a.nbytes, x);
  compiler_fence();
  wait_vm<0>();
  if (sends) {
    V line;
#pragma unroll
    for (int e = 0; e < W; ++e) line[e] = x[e];
#pragma unroll
    for (int m = 0; m < J; ++m) st_vec<kCoh>(peer_rsrc(pb[m]), push_off, line);
  }
  V u[J];
  const bool polled = poll_list<J>(a, own, poll_off, u, ready, r, s);
  uint32_t o[W];
  if (!split_fold<DT, NMAX, UB, J>(c, b, N, r, pe, polled, u, x, o)) return false;
  store_unit<DT, UB, kOut>(out_r, out_off, a.nbytes, o);
  compiler_fence();
  wait_vm<0>();  // the output has landed (wave 0); the others have folded
  t1 = now_ticks();
  // re-arm this wave's sources for step s + 2 (the next step's first push waits for it)
#pragma unroll
  for (int m = 0; m < J; ++m) st_vec<kCoh>(own, poll_off[m], sent);
  return true;
}

// One-shot LL AllReduce, peer-split: the LL protocol (§IV "LL") with the peers of each 64
// lines spread over the waves as in step_oneshot_split. Every wave loads the same 8 bytes per
// lane, pushes the line {payload, s} to its J peers and polls their lines until the flag equals
// s; the payloads meet in LDS and wave 0 stores the output. Nothing is re-armed.
template <int DT, int NMAX>
__device__ bool step_oneshot_ll_split(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                      rsrc_t out_r, int k, uint64_t& t0, uint64_t& t1) {
  constexpr int J = split_j<NMAX>();
  const int N = a.nranks, r = c.rank;
  const int g = static_cast<int>(uni(static_cast<uint32_t>(c.wave)));  // wave-uniform
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t elo = static_cast<uint32_t>(s), ehi = static_cast<uint32_t>(s >> 32);
  const uint32_t slot = a.ll.slot, CU = a.chunk_units;
  const uint32_t unit0 = static_cast<uint32_t>(k) * CU;
  const bool sends = r != a.withhold;
  const rsrc_t own = region_rsrc(a, r, a.ll);
  auto ready = [elo, ehi](u32x4 l) { return (l.z == elo) & (l.w == ehi); };
  const uint32_t i = static_cast<uint32_t>(c.cta) * kWave + c.lane;  // shared by the waves
  const bool act = i < CU;
  SplitPeer pe[J];
  PeerBase pb[J];
  uint32_t poll_off[J];
  const uint32_t line0 = b * N * slot + slot_off(a.ll, i);
#pragma unroll
  for (int m = 0; m < J; ++m) {
    pe[m] = split_peer(N, r, g, m);
    pb[m] = peer_base(a, pe[m], a.ll);
    poll_off[m] = act && pe[m].live ? line0 + static_cast<uint32_t>(pe[m].q) * slot : kDrop;
    pin(poll_off[m]);
  }
  uint32_t in_off = act ? (unit0 + i) * 8u : kDrop;
  uint32_t push_off = act ? (b * N + r) * slot + slot_off(a.ll, i) : kDrop;
  uint32_t out_off = act && g == 0 ? (unit0 + i) * 8u : kDrop;
  pin(in_off);
  pin(push_off);
  pin(out_off);
  stamp_start(t0, k);
  uint32_t x[2];
  load_unit<DT, 8>(in_r, in_off, a.nbytes, x);
  compiler_fence();
  wait_vm<0>();
  if (sends) {
    const u32x4 line = {x[0], x[1], elo, ehi};
#pragma unroll
    for (int m = 0; m < J; ++m) st16<kCoh>(peer_rsrc(pb[m]), push_off, line);
  }
  u32x4 l[J];
  const bool polled = poll_list<J>(a, own, poll_off, l, ready, r, s);
  u32x2 u[J];
#pragma unroll
  for (int m = 0; m < J; ++m) u[m] = u32x2{l[m].x, l[m].y};
  uint32_t o[2];
  if (!split_fold<DT, NMAX, 8, J>(c, b, N, r, pe, polled, u, x, o)) return false;
  store_unit<DT, 8, kOut>(out_r, out_off, a.nbytes, o);
  compiler_fence();
  wait_vm<0>();  // the output has landed (wave 0); the others have folded
  t1 = now_ticks();
  return true;
}

// Two-shot AllReduce, peer-split: wave g sends its J peers their partitions (reduce-scatter),
// polls their contributions to this rank's partition, and after the exchange and the fold (in
// every wave) sends them the reduced partition and polls theirs into the output (all-gather).
// Wave 0 writes the rank's own partition of the output.
template <int DT, int NMAX, int UB>
__device__ bool step_twoshot_split(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                   rsrc_t out_r, int k, uint64_t& t0, uint64_t& t1) {
  using V = unit_t<UB>;
  constexpr int W = UB / 4;
  constexpr int J = split_j<NMAX>();
  const int N = a.nranks, r = c.rank;
  const int g = static_cast<int>(uni(static_cast<uint32_t>(c.wave)));  // wave-uniform
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot1 = a.p1.slot, slot2 = a.p2.slot, CU = a.chunk_units, P = a.part_units;
  const bool sends = r != a.withhold;
  const rsrc_t own1 = region_rsrc(a, r, a.p1);
  const rsrc_t own2 = region_rsrc(a, r, a.p2);
  const V sent = sentinel_unit<DT, UB>();
  auto ready = [](V l) { return vec_clear<DT>(l); };
  const uint32_t i = static_cast<uint32_t>(c.cta) * kWave + c.lane;
  const bool act = i < CU && k * CU + i < P;
  const uint32_t base1 = b * N * slot1 + slot_off<UB>(a.p1, i);
  const uint32_t base2 = b * N * slot2 + slot_off<UB>(a.p2, i);
  SplitPeer pe[J];
  PeerBase pb1[J], pb2[J];
  uint32_t in_off[J], poll1[J], poll2[J], ag_off[J];
#pragma unroll
  for (int m = 0; m < J; ++m) {
    pe[m] = split_peer(N, r, g, m);
    pb1[m] = peer_base(a, pe[m], a.p1);
    pb2[m] = peer_base(a, pe[m], a.p2);
    const bool live = act && pe[m].live;
    const uint32_t q = static_cast<uint32_t>(pe[m].q);
    in_off[m] = live ? (q * P + k * CU + i) * UB : kDrop;      // partition owned by peer q
    poll1[m] = live ? base1 + q * slot1 : kDrop;
    poll2[m] = live ? base2 + q * slot2 : kDrop;
    ag_off[m] = live ? (q * P + k * CU + i) * UB : kDrop;      // peer q's reduced partition
    pin(in_off[m]);
    pin(poll1[m]);
    pin(poll2[m]);
  }
  uint32_t own_off = act ? (r * P + k * CU + i) * UB : kDrop;
  uint32_t out_own = act && g == 0 ? own_off : kDrop;
  uint32_t push1 = act ? (b * N + r) * slot1 + slot_off<UB>(a.p1, i) : kDrop;
  uint32_t push2 = act ? (b * N + r) * slot2 + slot_off<UB>(a.p2, i) : kDrop;
  pin(own_off);
  pin(out_own);
  pin(push1);
  pin(push2);
  stamp_start(t0, k);
  uint32_t x[W];
  uint32_t w[J][W];
  load_unit<DT, UB, kPlain, false>(in_r, own_off, a.nbytes, x);
#pragma unroll
  for (int m = 0; m < J; ++m) load_unit<DT, UB, kPlain, false>(in_r, in_off[m], a.nbytes, w[m]);
  // all loads are in flight before the one scalar branch for an odd bf16 tail
  if (odd_tail<DT>(a.nbytes)) {
    asm volatile("");
    clear_odd_tail<UB>(own_off, a.nbytes, x);
#pragma unroll
    for (int m = 0; m < J; ++m) clear_odd_tail<UB>(in_off[m], a.nbytes, w[m]);
  }
  compiler_fence();
  wait_vm<0>();
  if (sends) {
#pragma unroll
    for (int m = 0; m < J; ++m) {
      V line;
#pragma unroll
      for (int e = 0; e < W; ++e) line[e] = w[m][e];
      st_vec<kCoh>(peer_rsrc(pb1[m]), push1, line);
    }
  }
  V u[J];
  const bool polled = poll_list<J>(a, own1, poll1, u, ready, r, s);
  uint32_t o[W];
  if (!split_fold<DT, NMAX, UB, J>(c, b, N, r, pe, polled, u, x, o)) return false;
  if (sends) {
    V line;
#pragma unroll
    for (int e = 0; e < W; ++e) line[e] = o[e];
#pragma unroll
    for (int m = 0; m < J; ++m) st_vec<kCoh>(peer_rsrc(pb2[m]), push2, line);
  }
  store_unit<DT, UB, kOut>(out_r, out_own, a.out_nbytes, o);
  V u2[J];
  if (!poll_list<J>(a, own2, poll2, u2, ready, r, s)) return false;
#pragma unroll
  for (int m = 0; m < J; ++m) {
    if constexpr (UB == 16)
      st16<kOut>(out_r, ag_off[m], u2[m]);
    else
      st8<kOut>(out_r, ag_off[m], u2[m]);
  }
  if (odd_tail<DT>(a.out_nbytes)) {
    // the last element of an odd-length message, if it is in one of this wave's partitions
    asm volatile("");
    const uint32_t last = a.out_nbytes & ~3u;
#pragma unroll
    for (int m = 0; m < J; ++m) {
      const uint32_t off = ag_off[m];
      const bool tail = off != kDrop && off <= last && last < off + UB;
      uint32_t word = u2[m][0];
#pragma unroll
      for (int e = 1; e < W; ++e) word = (off + 4u * e == last) ? u2[m][e] : word;
      st2<kOut>(out_r, tail ? last : kDrop, static_cast<uint16_t>(word & 0xFFFFu));
    }
  }
  compiler_fence();
  wait_vm<0>();  // every output store of this wave has landed
  t1 = now_ticks();
  // re-arm both phases' slots of this wave's peers for step s + 2
#pragma unroll
  for (int m = 0; m < J; ++m) {
    st_vec<kCoh>(own1, poll1[m], sent);
    st_vec<kCoh>(own2, poll2[m], sent);
  }
  return true;
}

// Bulk two-shot, for chunks wider than one pass of the rank's workgroups (the bandwidth
// regime). The same reduce-scatter + all-gather as above, but each wave announces its data with
// one completion flag per peer instead of a sentinel in every unit: a wave pushes all its units
// of the phase with coherent stores, waits until they have completed (so they are visible at
// the coherence point), then stores the step number into its flag slot in each peer's block; the
// peer's matching wave (same workgroup and wave index, hence the same units) waits for the flags
// of every source before reading the data. Flags only grow, so nothing is re-armed and no unit
// is checked. Double buffering and its credit are those of the sentinel protocol (step s writes
// buffer s & 1; a peer writes the same buffer again only two steps later, after this rank's
// flags of the step in between). Inputs are read once and outputs written once, so both carry
// the non-temporal hint.
// The all-gather goes straight into the outputs: every rank's output pointers are kernel
// arguments, so an owner stores its reduced partition into each rank's output (and its own),
// waits for those stores and raises its phase-1 flags; a rank whose flags have all arrived has
// its whole output. No all-gather slot is written or read: 30 S of traffic at N = 8 (44 S through
// slots, 58 S with sentinels). An owner reaches the all-gather only after every peer's input
// partition for it has arrived, so an in-place call never overwrites input that is still to be
// sent. A persistent launch whose output sets overlap its input sets (a later iteration would
// read bytes other ranks store) keeps the all-gather in the slots (ag_direct = 0).
__device__ __forceinline__ uint64_t* bulk_flag(const Args& a, int dst, int phase, int src,
                                               const Ctx& c) {
  return reinterpret_cast<uint64_t*>(a.base + static_cast<uint64_t>(dst) * a.stride + a.flg.off) +
         ((static_cast<uint32_t>(phase) * kMaxRanks + static_cast<uint32_t>(src)) *
              kMaxCtasPerRank + static_cast<uint32_t>(c.cta)) * kMaxWavesPerCta + c.wave;
}

// Lane q < N (q != rank) tells peer q that this wave's data of `phase` for step s is complete.
__device__ __forceinline__ void bulk_signal(const Args& a, const Ctx& c, int phase, uint64_t s) {
  const int q = c.lane;
  if (q < a.nranks && q != c.rank)
    __hip_atomic_store(bulk_flag(a, q, phase, c.rank, c), s, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every peer's matching wave has announced `phase` of step s (bounded).
__device__ __forceinline__ bool bulk_wait(const Args& a, const Ctx& c, int phase, uint64_t s) {
  const int q = c.lane;
  bool need = q < a.nranks && q != c.rank;
  const uint64_t* f = bulk_flag(a, c.rank, phase, need ? q : 0, c);
  uint32_t spins = 0;
  uint64_t t_first = 0;
  while (true) {
    if (need && __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= s) need = false;
    const uint64_t waiting = __ballot(need);
    if (waiting == 0) return true;
    if ((++spins & 1023u) == 0) {
      t_first = poll_check(poll_env(a), t_first, c.rank, __builtin_ctzll(waiting), s);
      if (t_first == 0) return false;
    }
  }
}

// Unit rotation of the bulk two-shot: lane i handles unit (i + sk_p) mod CU of partition p, with
// sk_p = (p * kBulkSkew) mod CU. A rank's eight concurrent streams (its input partitions, the
// peers' slots, its output partitions) then sit at different offsets instead of exactly a power
// of two apart: a seven-stream copy at 32 MiB strides measured 6.6-6.75 TB/s on MI355X, and
// 7.0-7.1 TB/s with the streams skewed by 4 KiB. The rotation depends only on the partition, so a
// unit is handled by the same lane (hence the same wave and completion flag) on every rank.
constexpr uint32_t kBulkSkew = 4096u / 16u;

__device__ __forceinline__ uint32_t bulk_rot(uint32_t i, uint32_t sk, uint32_t CU) {
  const uint32_t u = i + sk;
  return u >= CU ? u - CU : u;
}

// Output of the j-th rank after r for the iteration using input/output set `set` (a descriptor
// that drops every access when j >= N).
__device__ __forceinline__ rsrc_t peer_out_rsrc(const Args& a, int r, int j, int set) {
  int q = r + j;
  if (q >= a.nranks) q -= a.nranks;
  const bool live = j < a.nranks;
  const bool affine = a.in_set_stride != 0 || a.out_set_stride != 0;
  const uint8_t* p;
  if (affine || a.out_tab == nullptr)
    p = static_cast<const uint8_t*>(a.out[live ? q : 0]) + static_cast<int64_t>(set) * a.out_set_stride;
  else
    p = static_cast<const uint8_t*>(a.out_tab[static_cast<uint32_t>(set) * a.nranks + (live ? q : 0)]);
  return make_rsrc(uniform_ptr(p), live ? a.out_nbytes : 0u);
}

template <int DT, int NMAX>
__device__ bool step_twoshot_bulk(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                  rsrc_t out_r, int k, int set, uint64_t& t0, uint64_t& t1) {
  const int N = a.nranks, r = c.rank;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot1 = a.pf1.slot, slot2 = a.pf2.slot, CU = a.chunk_units, P = a.part_units;
  const bool sends = r != a.withhold;
  const rsrc_t own1 = region_rsrc(a, r, a.pf1);
  const rsrc_t own2 = region_rsrc(a, r, a.pf2);
  const uint32_t peers = peer_mask(N, r);
  const uint32_t mine1 = (b * N + r) * slot1, mine2 = (b * N + r) * slot2;
  // skew of partition q (index by absolute partition) and of the j-th partition after r
  uint32_t skq[NMAX], skj[NMAX];
#pragma unroll
  for (int q = 0; q < NMAX; ++q) {
    skq[q] = uni((static_cast<uint32_t>(q) * kBulkSkew) % CU);
    int p = r + q;
    if (p >= N) p -= N;
    skj[q] = uni((static_cast<uint32_t>(p < N ? p : 0) * kBulkSkew) % CU);
  }
  const uint32_t skr = uni((static_cast<uint32_t>(r) * kBulkSkew) % CU);
  // all-gather straight into the outputs: the peers' output descriptors of this iteration
  const bool direct = a.ag_direct != 0;
  rsrc_t peer_out[NMAX];
#pragma unroll
  for (int j = 1; j < NMAX; ++j) peer_out[j] = peer_out_rsrc(a, r, direct ? j : NMAX, set);
  stamp_start(t0, k);
  wait_all_mem();
  // reduce-scatter: partition (r + j) % N of this rank's input to peer j's slot r
  if (sends) {
    for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CU;
      uint32_t w[NMAX][4];
      uint32_t u[NMAX];
#pragma unroll
      for (int j = 1; j < NMAX; ++j) {
        int p = r + j;
        if (p >= N) p -= N;
        u[j] = bulk_rot(i, skj[j], CU);
        const bool live = act && j < N;
        load_unit<DT, 16, kNt, false>(in_r, live ? (p * P + k * CU + u[j]) * 16u : kDrop,
                                      a.nbytes, w[j]);
      }
      if (odd_tail<DT>(a.nbytes)) {
        asm volatile("");
#pragma unroll
        for (int j = 1; j < NMAX; ++j) {
          int p = r + j;
          if (p >= N) p -= N;
          clear_odd_tail<16>((p * P + k * CU + u[j]) * 16u, a.nbytes, w[j]);
        }
      }
#pragma unroll
      for (int j = 1; j < NMAX; ++j)
        st16<kCoh>(peer_rsrc(a, r, j, a.pf1), act ? mine1 + u[j] * 16u : kDrop,
                   u32x4{w[j][0], w[j][1], w[j][2], w[j][3]});
    }
    wait_all_mem();
    bulk_signal(a, c, 0, s);
  }
  if (!bulk_wait(a, c, 0, s)) return false;
  compiler_fence();
  // fold the own partition in rank order, write it out and push it to every peer's slot r
  for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
    const uint32_t i = i0 + c.lane;
    const bool act = i < CU;
    const uint32_t mask = act ? peers : 0u;
    const uint32_t u = bulk_rot(i, skr, CU);
    const uint32_t off1 = b * N * slot1 + u * 16u;
    const uint32_t uoff = (r * P + k * CU + u) * 16u;
    uint32_t x[4];
    load_unit<DT, 16, kNt>(in_r, act ? uoff : kDrop, a.nbytes, x);
    u32x4 v[NMAX];
#pragma unroll
    for (int q = 0; q < NMAX; ++q)
      v[q] = ld16<kCoh>(own1, ((mask >> q) & 1u) ? off1 + static_cast<uint32_t>(q) * slot1 : kDrop);
    uint32_t o[4];
    fold_rank_order<DT, NMAX, 4>(N, r, x, v, o);
    if (sends) {
      if (direct) {
#pragma unroll
        for (int j = 1; j < NMAX; ++j)
          store_unit<DT, 16, kOut>(peer_out[j], act ? uoff : kDrop, a.nbytes, o);
      } else {
        push_peers<NMAX>(a, r, a.pf2, act ? mine2 + u * 16u : kDrop,
                         u32x4{o[0], o[1], o[2], o[3]});
      }
    }
    store_unit<DT, 16, kOut>(out_r, act ? uoff : kDrop, a.nbytes, o);
  }
  if (sends) {
    wait_all_mem();
    bulk_signal(a, c, 1, s);
  }
  if (!bulk_wait(a, c, 1, s)) return false;
  compiler_fence();
  if (direct) {
    // every other owner has stored its partition into this rank's output and waited for the
    // stores to complete before its flag
    t1 = now_ticks();
    return true;
  }
  // all-gather: every other owner's reduced partition into the output
  for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
    const uint32_t i = i0 + c.lane;
    const bool act = i < CU;
    const uint32_t mask = act ? peers : 0u;
    uint32_t u[NMAX];
    u32x4 v[NMAX];
#pragma unroll
    for (int q = 0; q < NMAX; ++q) {
      u[q] = bulk_rot(i, skq[q], CU);
      v[q] = ld16<kCoh>(own2, ((mask >> q) & 1u)
                                  ? b * N * slot2 + static_cast<uint32_t>(q) * slot2 + u[q] * 16u
                                  : kDrop);
    }
#pragma unroll
    for (int q = 0; q < NMAX; ++q) {
      const uint32_t o[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
      store_unit<DT, 16, kOut>(out_r, ((mask >> q) & 1u) ? (q * P + k * CU + u[q]) * 16u : kDrop,
                              a.nbytes, o);
    }
  }
  wait_all_mem();
  t1 = now_ticks();
  return true;
}

// ------------------------------------------------------------------ LL128-style atomic two-shot
//
// Reduce-scatter by atomic addition: every rank (the owner included) adds its chunk of
// partition p into owner p's shared destination, then counts itself in on the owner's arrival
// counter for this (buffer, workgroup, wave). The page's design detects completion with a flag
// inside each 128-byte line, which needs 128-byte atomicity of the interconnect. Here a
// contributor waits until its own atomic adds have been performed (they execute at one coherence
// point for the whole device) and only then increments the counter; the owner, once it reads N
// arrivals, takes each sum with an atomic exchange against zero, which both reads the final value
// at that coherence point and clears the destination for step s+2. It then resets the counter
// and runs the all-gather with the bulk two-shot's protocol, which does not look at the data
// (an int32 sum may be any value, INT32_MIN included, so a sentinel slot could not tell it from
// an empty one): the owner stores its sums straight into every rank's output (all output
// pointers are kernel arguments; into the peers' bulk all-gather slots when an ar_bench launch's
// output sets overlap its input sets), waits for those stores to complete, then raises a
// completion flag per peer (phase 1) that the receivers poll. Against the sentinel all-gather
// of the plain two-shot (measured at 16 ranks, fp32, the kernel forced at every size): 4 KiB
// the same, 16-256 KiB 3-7 % lower, 2 MiB 51 -> 46 us, 4 MiB 92 -> 78 us; int32 against
// pushes into the slots 4 KiB 4.75 -> 4.1 us, 4 MiB 81 -> 68 us. An owner reaches the
// all-gather only after every contributor's adds from its input partition have been performed,
// so an in-place call never overwrites input that is still to be read. (The peer-split kernel
// of small messages keeps the sentinel all-gather.)
//
// bf16 adds two elements per atomic (gfx950's packed bf16 atomic add): the destination holds
// bf16 and every addition rounds to bf16, so the sum's error is that of a bf16 accumulation in
// an unknown order.
//
// The deterministic variant (DET; a reading of the Pith review's "deterministic variant using
// per-chunk grouping or hierarchical accumulation") keeps the shared destinations and the
// atomics but fixes the order: the ranks form groups of `group` consecutive ranks, and owner p
// holds one binary32 destination per group. Within a group the members add in rank order: the
// first member stores its values, member m waits until the group's ticket in the owner's block
// reads m, adds (binary32 atomics; bf16 inputs widened), waits until its adds have been
// performed and sets the ticket to m + 1. The owner waits for every group's ticket to reach the
// group's size, takes each group sum with an atomic exchange against zero, adds the group sums in
// group order (bf16 rounded once), resets the tickets and runs the all-gather. Every addition
// then happens in one fixed order, so the result is the same bit pattern on every run.
//
// The wave's units are handled as words: lane l takes words e * 64 + l of the wave's 64 units
// (e = 0..E-1), so that every atomic instruction adds into 256 contiguous bytes (whole cache
// lines) rather than one word of each of 64 units. E < 4 is used when the whole chunk is fewer
// than 16 E units in one wave: the word slices that hold nothing are then not issued at all.

// Most groups of the deterministic variant: groups of at least two ranks, at most 16 ranks.
constexpr int kMaxDetGroups = kMaxRanks / 2;

// Byte offset of group g's destination of buffer b in a rank block's `acc` region, laid out as
// [buffer 2][group ceil(N / 2)][slot]; the plain atomic variant uses group 0.
__device__ __forceinline__ uint32_t acc_off(const Args& a, uint32_t b, int g) {
  return (b * static_cast<uint32_t>((a.nranks + 1) / 2) + static_cast<uint32_t>(g)) * a.acc.slot;
}

// Ticket word of (buffer b, group g, this workgroup and wave) in rank `owner`'s counter region,
// after the plain variant's arrival counters [buffer 2][cta][wave].
__device__ __forceinline__ uint32_t* det_ticket(const Args& a, int owner, uint32_t b, int g,
                                                const Ctx& c) {
  constexpr uint32_t kBase = 2u * kMaxCtasPerRank * kMaxWavesPerCta;
  return reinterpret_cast<uint32_t*>(a.base + static_cast<uint64_t>(owner) * a.stride +
                                     a.cnt.off) +
         kBase + ((b * kMaxRanks + static_cast<uint32_t>(g)) * kMaxCtasPerRank + c.cta) *
                     kMaxWavesPerCta + c.wave;
}

template <int DT, int NMAX, int E = 4, bool DET = false>
__device__ bool step_ll128(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r, rsrc_t out_r,
                           int k, int set, uint64_t& t0, uint64_t& t1) {
  static_assert(!DET || DT != DT_I32, "an int32 sum does not depend on the order");
  static_assert(E == 1 || E == 2 || E == 4, "word slices per lane");
  // The all-gather: owners store their sums straight into every rank's output (ag_direct; else
  // into the peers' bulk all-gather slots), wait for those stores, then raise completion flags.
  const bool direct = a.ag_direct != 0;
  // binary32 words of the destination per payload word: 2 for the deterministic bf16 variant
  constexpr uint32_t kAW = (DET && DT == DT_BF16) ? 2u : 1u;
  const int N = a.nranks, r = c.rank;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t CU = a.chunk_units, P = a.part_units;
  const bool has_units = c.t0 < CU;
  const uint32_t cnt_idx = (b * kMaxCtasPerRank + c.cta) * kMaxWavesPerCta + c.wave;
  const uint32_t peers = peer_mask(N, r);
  const int M = DET ? a.group : N;  // group size (the plain variant: one group of N)
  const int G = DET ? (N + M - 1) / M : 1;
  const int gme = DET ? r / M : 0, mme = DET ? r - gme * M : 0;
  // the peers' outputs of this iteration (descriptors that drop every access unless direct)
  rsrc_t peer_out[NMAX];
#pragma unroll
  for (int j = 1; j < NMAX; ++j) peer_out[j] = peer_out_rsrc(a, r, direct ? j : NMAX, set);
  stamp_start(t0, k);
  wait_all_mem();
  // The wave's words of chunk k (pass i0): word d = i0 * 4 + e * 64 + lane.
  auto words = [&](uint32_t i0, uint32_t (&woff)[E], bool (&wact)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t d = i0 * 4u + static_cast<uint32_t>(e) * 64u + c.lane;
      wact[e] = d < CU * 4u;
      woff[e] = d * 4u;
    }
  };
  if constexpr (!DET) {
    if (has_units && r != a.withhold) {
      for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
        uint32_t woff[E];
        bool wact[E];
        words(i0, woff, wact);
        uint32_t w[NMAX][E];
#pragma unroll
        for (int j = 0; j < NMAX; ++j) {
          int p = r + j;
          if (p >= N) p -= N;
          const bool live = j < N;
          const uint32_t pbase = (p * P + k * CU) * 16u;
#pragma unroll
          for (int e = 0; e < E; ++e)
            w[j][e] = ld4<kPlain>(in_r, live && wact[e] ? pbase + woff[e] : kDrop);
        }
        // bf16 of odd length: the half word past the last element reads as zero (it would
        // otherwise be added like data, and a sum there that equals the sentinel would stall
        // the all-gather poll)
        if (odd_tail<DT>(a.nbytes)) {
          asm volatile("");
          const uint32_t last = a.nbytes & ~3u;
#pragma unroll
          for (int j = 0; j < NMAX; ++j) {
            int p = r + j;
            if (p >= N) p -= N;
            const uint32_t pbase = (p * P + k * CU) * 16u;
#pragma unroll
            for (int e = 0; e < E; ++e)
              w[j][e] = pbase + woff[e] == last ? (w[j][e] & 0xFFFFu) : w[j][e];
          }
        }
#pragma unroll
        for (int j = 0; j < NMAX; ++j) {
          if constexpr (DT == DT_BF16) {
            // Packed bf16 atomics take a global address, so nothing drops them: lanes of absent
            // peers and idle words add zero into a word of this rank's sink region instead (no
            // branch, so the atomics stay in one basic block without waits between them).
            typedef short s16x2 __attribute__((ext_vector_type(2)));
            int q = r + j;
            if (q >= N) q -= N;
            uint8_t* dst = a.base + static_cast<uint64_t>(j < N ? q : r) * a.stride + a.acc.off +
                           acc_off(a, b, 0);
            uint8_t* sink = a.base + static_cast<uint64_t>(r) * a.stride + a.sink.off +
                            ((c.cta * kMaxWavesPerCta + c.wave) % 64u) * 256u + c.lane * 4u;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const bool live = j < N && wact[e];
              __builtin_amdgcn_global_atomic_fadd_v2bf16(
                  reinterpret_cast<s16x2*>(live ? dst + woff[e] : sink),
                  __builtin_bit_cast(s16x2, live ? w[j][e] : 0u));
            }
          } else {
            const rsrc_t dst = j == 0 ? region_rsrc(a, r, a.acc) : peer_rsrc(a, r, j, a.acc);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const uint32_t off = wact[e] ? acc_off(a, b, 0) + woff[e] : kDrop;
              if constexpr (DT == DT_F32) {
                (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(__uint_as_float(w[j][e]),
                                                                     dst, off, 0, 0);
              } else {
                (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(static_cast<int>(w[j][e]),
                                                                    dst, off, 0, 0);
              }
            }
          }
        }
      }
      wait_all_mem();  // every add of this wave has been performed
      if (c.lane < N) {
        uint32_t* cnt = reinterpret_cast<uint32_t*>(a.base +
                                                    static_cast<uint64_t>(c.lane) * a.stride +
                                                    a.cnt.off) + cnt_idx;
        __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else {
    // Deterministic: lane q watches owner q's ticket of this rank's group; every owner whose
    // ticket has reached this rank's place gets this rank's chunk of its partition, then its
    // ticket moves on. Owners become ready independently, so several may be served per round.
    // The plan gives this variant one pass per chunk (every unit has its own lane's words), so
    // the input words of every partition are loaded once, before the first round.
    if (has_units && r != a.withhold) {
      uint32_t woff[E];
      bool wact[E];
      words(c.t0, woff, wact);
      uint32_t w[NMAX][E];
#pragma unroll
      for (int j = 0; j < NMAX; ++j) {
        int p = r + j;
        if (p >= N) p -= N;
        const uint32_t pbase = (p * P + k * CU) * 16u;
#pragma unroll
        for (int e = 0; e < E; ++e)
          w[j][e] = ld4<kPlain>(in_r, j < N && wact[e] ? pbase + woff[e] : kDrop);
      }
      if (odd_tail<DT>(a.nbytes)) {  // the half word past the last bf16 element reads as 0
        asm volatile("");
#pragma unroll
        for (int j = 0; j < NMAX; ++j) {
          int p = r + j;
          if (p >= N) p -= N;
          const uint32_t pbase = (p * P + k * CU) * 16u;
#pragma unroll
          for (int e = 0; e < E; ++e)
            w[j][e] = pbase + woff[e] == (a.nbytes & ~3u) ? (w[j][e] & 0xFFFFu) : w[j][e];
        }
      }
      const uint32_t goff = acc_off(a, b, gme);
      uint32_t todo = (N >= 32 ? 0xFFFFFFFFu : ((1u << N) - 1u));
      uint32_t spins = 0;
      uint64_t t_first = 0;
      while (todo != 0) {
        const int q = c.lane;
        const bool watch = q < N && ((todo >> q) & 1u);
        uint32_t tv = 0xFFFFFFFFu;
        if (watch)
          tv = __hip_atomic_load(det_ticket(a, q, b, gme, c), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t go =
            static_cast<uint32_t>(__ballot(watch && tv == static_cast<uint32_t>(mme)));
        if (go == 0) {
          if ((++spins & 1023u) == 0) {
            t_first = poll_check(poll_env(a), t_first, r, __builtin_ctz(todo), s);
            if (t_first == 0) return false;
          }
          continue;
        }
        // every owner in `go` at once: branch-free, absent or waiting owners drop their accesses
#pragma unroll
        for (int j = 0; j < NMAX; ++j) {
          int p = r + j;
          if (p >= N) p -= N;
          const bool live = j < N && ((go >> p) & 1u);
          const rsrc_t dst = j == 0 ? region_rsrc(a, r, a.acc) : peer_rsrc(a, r, j, a.acc);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            // binary32 value(s) of the word: fp32 as is, bf16 widened (low element first)
            float v0, v1 = 0.0f;
            if constexpr (DT == DT_BF16) {
              v0 = __uint_as_float(w[j][e] << 16);
              v1 = __uint_as_float(w[j][e] & 0xFFFF0000u);
            } else {
              v0 = __uint_as_float(w[j][e]);
            }
            const uint32_t off = live && wact[e] ? goff + woff[e] * kAW : kDrop;
            if (mme == 0) {
              // the group's first member writes: the destination then holds exactly its values
              if constexpr (kAW == 2)
                st8<kCoh>(dst, off, u32x2{__float_as_uint(v0), __float_as_uint(v1)});
              else
                st4<kCoh>(dst, off, __float_as_uint(v0));
            } else {
              (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v0, dst, off, 0, 0);
              if constexpr (kAW == 2)
                (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                    v1, dst, off == kDrop ? kDrop : off + 4u, 0, 0);
            }
          }
        }
        wait_all_mem();  // this rank's values are in the destinations before the tickets move
        if (q < N && ((go >> q) & 1u))
          __hip_atomic_store(det_ticket(a, q, b, gme, c), static_cast<uint32_t>(mme + 1),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        todo &= ~go;
      }
    }
  }
  if (has_units) {
    uint32_t* my_cnt =
        reinterpret_cast<uint32_t*>(a.base + static_cast<uint64_t>(r) * a.stride + a.cnt.off) +
        cnt_idx;
    uint32_t spins = 0;
    uint64_t t_first = 0;
    if constexpr (!DET) {
      while (uni(__hip_atomic_load(my_cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) !=
             static_cast<uint32_t>(N)) {
        if ((++spins & 1023u) == 0) {
          t_first = poll_check(poll_env(a), t_first, r, -1, s);
          if (t_first == 0) return false;
        }
      }
    } else {
      // lane g < G waits until group g's ticket in this rank's block equals the group's size
      const int g = c.lane;
      bool need = g < G;
      const uint32_t size = static_cast<uint32_t>(g < G ? min(M, N - g * M) : 0);
      while (true) {
        if (need && __hip_atomic_load(det_ticket(a, r, b, g, c), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == size)
          need = false;
        if (__ballot(need) == 0) break;
        if ((++spins & 1023u) == 0) {
          t_first = poll_check(poll_env(a), t_first, r, -1, s);
          if (t_first == 0) return false;
        }
      }
    }
    uint8_t* acc = a.base + static_cast<uint64_t>(r) * a.stride + a.acc.off;
    for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CU;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (act) {
        if constexpr (!DET) {
          uint64_t* q = reinterpret_cast<uint64_t*>(acc + acc_off(a, b, 0) +
                                                    static_cast<uint64_t>(i) * 16u);
          const uint64_t lo =
              __hip_atomic_exchange(q, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t hi =
              __hip_atomic_exchange(q + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          v = u32x4{static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                    static_cast<uint32_t>(hi), static_cast<uint32_t>(hi >> 32)};
        } else {
          // Group sums in group order: 4 (fp32) or 8 (bf16) binary32 values per unit. Every
          // member's adds were performed before its ticket moved, so coherent loads read the
          // final sums; all groups' loads are in flight at once (groups beyond G drop theirs),
          // then the destinations are cleared with coherent stores for the plain variant, which
          // expects zeros.
          constexpr int V = 4 * static_cast<int>(kAW);
          const rsrc_t accr = region_rsrc(a, r, a.acc);
          u32x4 gs[kMaxDetGroups][kAW];
#pragma unroll
          for (int g = 0; g < kMaxDetGroups; ++g)
#pragma unroll
            for (uint32_t h = 0; h < kAW; ++h)
              gs[g][h] = ld16<kCoh>(accr, g < G ? acc_off(a, b, g) + i * 16u * kAW + h * 16u
                                               : kDrop);
          float sum[V];
#pragma unroll
          for (int g = 0; g < kMaxDetGroups; ++g) {
#pragma unroll
            for (int t = 0; t < V; ++t) {
              const float x = __uint_as_float(gs[g][t / 4][t % 4]);
              sum[t] = g == 0 ? x : (g < G ? sum[t] + x : sum[t]);
            }
          }
#pragma unroll
          for (int g = 0; g < kMaxDetGroups; ++g)
#pragma unroll
            for (uint32_t h = 0; h < kAW; ++h)
              st16<kCoh>(accr, g < G ? acc_off(a, b, g) + i * 16u * kAW + h * 16u : kDrop,
                         u32x4{0u, 0u, 0u, 0u});
          if constexpr (DT == DT_BF16) {
            v = u32x4{bf16x2_rne(sum[0], sum[1]), bf16x2_rne(sum[2], sum[3]),
                      bf16x2_rne(sum[4], sum[5]), bf16x2_rne(sum[6], sum[7])};
          } else {
            v = u32x4{__float_as_uint(sum[0]), __float_as_uint(sum[1]), __float_as_uint(sum[2]),
                      __float_as_uint(sum[3])};
          }
        }
      }
      const uint32_t o[4] = {v.x, v.y, v.z, v.w};
      const uint32_t uoff = (r * P + k * CU + i) * 16u;
      if (r != a.withhold) {
        if (direct) {
#pragma unroll
          for (int j = 1; j < NMAX; ++j)
            store_unit<DT, 16, kOut>(peer_out[j], act ? uoff : kDrop, a.nbytes, o);
        } else {
          push_peers<NMAX>(a, r, a.pf2, act ? (b * N + r) * a.pf2.slot + i * 16u : kDrop, v);
        }
      }
      store_unit<DT, 16, kOut>(out_r, act ? uoff : kDrop, a.nbytes, o);
    }
    if constexpr (!DET) {
      if (c.lane == 0) __hip_atomic_store(my_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      wait_all_mem();  // the destinations are clear before the tickets are reset
      if (c.lane < G)
        __hip_atomic_store(det_ticket(a, r, b, c.lane, c), 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (r != a.withhold) {
      wait_all_mem();  // the stored sums are performed before the flags that announce them
      bulk_signal(a, c, 1, s);
    }
  }
  // a wave with no units of this chunk neither signals nor waits, on every rank alike
  if (has_units && !bulk_wait(a, c, 1, s)) return false;
  compiler_fence();
  if (!direct) {
    const rsrc_t own_f = region_rsrc(a, r, a.pf2);
    const uint32_t slotf = a.pf2.slot;
    for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CU;
      const uint32_t mask = act ? peers : 0u;
      u32x4 v[NMAX];
#pragma unroll
      for (int q = 0; q < NMAX; ++q)
        v[q] = ld16<kCoh>(own_f, ((mask >> q) & 1u)
                                     ? (b * N + static_cast<uint32_t>(q)) * slotf + i * 16u
                                     : kDrop);
#pragma unroll
      for (int q = 0; q < NMAX; ++q) {
        const uint32_t o[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
        store_unit<DT, 16, kOut>(out_r, ((mask >> q) & 1u) ? (q * P + k * CU + i) * 16u : kDrop,
                           a.nbytes, o);
      }
    }
  }
  wait_all_mem();
  t1 = now_ticks();
  return true;
}

// LL128-style atomic AllReduce, peer-split (fp32 and bf16; a chunk of at most one 64-unit block
// per workgroup, E word slices per lane as in step_ll128). The workgroup's 4 waves share the
// block: wave g adds this rank's words of the partitions of owners j = g + m * kSplit after it
// (j = 0 is the rank itself) into their shared destinations, waits until its adds have been
// performed and counts itself in on each of those owners (one counter per owner, buffer and
// workgroup: N arrivals complete a block). Wave 0 of the owner waits for the N arrivals, takes
// the sums with atomic exchanges against zero and hands them to the other waves through LDS;
// after one barrier every wave pushes the sums to its all-gather peers (j = 1 + g + m * kSplit)
// and polls theirs into the output. A wave's atomics, like its stores, complete one after
// another, so each wave issues ceil(N / 4) owners' worth instead of N.
template <int DT, int NMAX, int E>
__device__ bool step_ll128_split(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                 rsrc_t out_r, int k, uint64_t& t0, uint64_t& t1) {
  static_assert(DT != DT_I32, "the int32 all-gather carries sums: step_ll128's completion flags");
  static_assert(E == 1 || E == 2 || E == 4, "word slices per lane");
  constexpr int JO = (NMAX + kSplit - 1) / kSplit;  // owners per wave (j = 0 .. NMAX-1)
  constexpr int JP = split_j<NMAX>();               // all-gather peers per wave (j = 1 .. NMAX-1)
  __shared__ u32x4 sums[2][kWave];
  const int N = a.nranks, r = c.rank;
  const int g = static_cast<int>(uni(static_cast<uint32_t>(c.wave)));  // wave-uniform
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t CU = a.chunk_units, P = a.part_units;
  const uint32_t B = static_cast<uint32_t>(a.block);        // units of the workgroup's block
  const uint32_t unit0 = static_cast<uint32_t>(c.cta) * B;
  const uint32_t i = unit0 + c.lane;
  const bool act = c.lane < B && i < CU;
  const bool sends = r != a.withhold;
  const rsrc_t own2 = region_rsrc(a, r, a.p2);
  const uint32_t slot2 = a.p2.slot;
  const u32x4 sent = sentinel_unit<DT, 16>();
  auto ready = [](u32x4 l) { return vec_clear<DT>(l); };
  const uint32_t cnt_idx = (b * kMaxCtasPerRank + static_cast<uint32_t>(c.cta)) * kMaxWavesPerCta;
  // this wave's owners and the words of the block each lane adds
  SplitPeer po[JO];
  PeerBase pa[JO];
  uint32_t in_off[JO][E], woff[E];
  bool wact[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t w_in = static_cast<uint32_t>(e) * 64u + c.lane;  // word within the block
    const uint32_t d = unit0 * 4u + w_in;
    wact[e] = w_in < B * 4u && d < CU * 4u;
    woff[e] = d * 4u;
  }
#pragma unroll
  for (int m = 0; m < JO; ++m) {
    po[m].j = g + m * kSplit;
    po[m].live = po[m].j < N;
    int q = r + po[m].j;
    if (q >= N) q -= N;
    po[m].q = po[m].live ? q : r;
    pa[m] = peer_base(a, po[m], a.acc);
    const uint32_t pbase = (static_cast<uint32_t>(po[m].q) * P + k * CU) * 16u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      in_off[m][e] = po[m].live && wact[e] ? pbase + woff[e] : kDrop;
      pin(in_off[m][e]);
    }
  }
  // this wave's all-gather peers
  SplitPeer pe[JP];
  PeerBase pb2[JP];
  uint32_t poll2[JP], ag_off[JP];
  const uint32_t base2 = b * N * slot2 + slot_off(a.p2, i);
#pragma unroll
  for (int m = 0; m < JP; ++m) {
    pe[m] = split_peer(N, r, g, m);
    pb2[m] = peer_base(a, pe[m], a.p2);
    const bool live = act && pe[m].live;
    const uint32_t q = static_cast<uint32_t>(pe[m].q);
    poll2[m] = live ? base2 + q * slot2 : kDrop;
    ag_off[m] = live ? (q * P + k * CU + i) * 16u : kDrop;
    pin(poll2[m]);
  }
  uint32_t push2 = act ? (b * N + r) * slot2 + slot_off(a.p2, i) : kDrop;
  uint32_t out_own = act && g == 0 ? (r * P + k * CU + i) * 16u : kDrop;
  pin(push2);
  pin(out_own);
  stamp_start(t0, k);
  uint32_t w[JO][E];
#pragma unroll
  for (int m = 0; m < JO; ++m)
#pragma unroll
    for (int e = 0; e < E; ++e) w[m][e] = ld4<kPlain>(in_r, in_off[m][e]);
  // bf16 of odd length: the half word past the last element reads as zero (it would otherwise be
  // added like data)
  if (odd_tail<DT>(a.nbytes)) {
    asm volatile("");
    const uint32_t last = a.nbytes & ~3u;
#pragma unroll
    for (int m = 0; m < JO; ++m)
#pragma unroll
      for (int e = 0; e < E; ++e) w[m][e] = in_off[m][e] == last ? (w[m][e] & 0xFFFFu) : w[m][e];
  }
  if (sends) {
#pragma unroll
    for (int m = 0; m < JO; ++m) {
      if constexpr (DT == DT_BF16) {
        // packed bf16 atomics take a global address: absent owners and idle words add zero into
        // this rank's sink region instead (branch-free, no waits between the atomics)
        typedef short s16x2 __attribute__((ext_vector_type(2)));
        uint8_t* dst = reinterpret_cast<uint8_t*>(pa[m].base) + acc_off(a, b, 0);
        uint8_t* sink = a.base + static_cast<uint64_t>(r) * a.stride + a.sink.off +
                        ((c.cta * kMaxWavesPerCta + c.wave) % 64u) * 256u + c.lane * 4u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool live = po[m].live && wact[e];
          __builtin_amdgcn_global_atomic_fadd_v2bf16(
              reinterpret_cast<s16x2*>(live ? dst + woff[e] : sink),
              __builtin_bit_cast(s16x2, live ? w[m][e] : 0u));
        }
      } else {
        const rsrc_t dst = peer_rsrc(pa[m]);
#pragma unroll
        for (int e = 0; e < E; ++e)
          (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
              __uint_as_float(w[m][e]), dst, wact[e] ? acc_off(a, b, 0) + woff[e] : kDrop, 0, 0);
      }
    }
    wait_all_mem();  // every add of this wave has been performed
    if (c.lane < JO) {
      int q = r;
      bool live = false;
#pragma unroll
      for (int m = 0; m < JO; ++m) {
        q = c.lane == m ? po[m].q : q;
        live = c.lane == m ? po[m].live : live;
      }
      if (live) {
        uint32_t* cnt = reinterpret_cast<uint32_t*>(a.base + static_cast<uint64_t>(q) * a.stride +
                                                    a.cnt.off) + cnt_idx;
        __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // owner: wave 0 waits for the N arrivals of this block and takes the sums
  bool ok = true;
  if (g == 0) {
    uint32_t* my_cnt =
        reinterpret_cast<uint32_t*>(a.base + static_cast<uint64_t>(r) * a.stride + a.cnt.off) +
        cnt_idx;
    uint32_t spins = 0;
    uint64_t t_first = 0;
    while (uni(__hip_atomic_load(my_cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) !=
           static_cast<uint32_t>(N)) {
      if ((++spins & 1023u) == 0) {
        t_first = poll_check(poll_env(a), t_first, r, -1, s);
        if (t_first == 0) {
          ok = false;
          break;
        }
      }
    }
    if (ok) {
      // The counter is reset first, with one branch-free store: vector memory operations of a
      // wave complete in issue order, so once the exchanges below have returned the reset has
      // completed too, before this wave reaches the barrier. The other waves' next
      // contributions (step s + 1) come after that barrier, and a contributor's adds into this
      // buffer again (step s + 2) only after it has received those; the reset and the cleared
      // destination are in place by then.
      st4<kCoh>(region_rsrc(a, r, a.cnt), c.lane == 0 ? cnt_idx * 4u : kDrop, 0u);
      compiler_fence();
      u32x4 v = {0u, 0u, 0u, 0u};
      if (act) {
        uint64_t* q = reinterpret_cast<uint64_t*>(a.base + static_cast<uint64_t>(r) * a.stride +
                                                  a.acc.off + acc_off(a, b, 0) +
                                                  static_cast<uint64_t>(i) * 16u);
        const uint64_t lo =
            __hip_atomic_exchange(q, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t hi =
            __hip_atomic_exchange(q + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v = u32x4{static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                  static_cast<uint32_t>(hi), static_cast<uint32_t>(hi >> 32)};
      }
      sums[b][c.lane] = v;
    }
  }
  if (!ok) g_split_fail = 1u;
  lds_barrier();
  if (g_split_fail != 0u) return false;
  const u32x4 v = sums[b][c.lane];
  if (sends) {
#pragma unroll
    for (int m = 0; m < JP; ++m) st16<kCoh>(peer_rsrc(pb2[m]), push2, v);
  }
  {
    const uint32_t o[4] = {v.x, v.y, v.z, v.w};
    store_unit<DT, 16, kOut>(out_r, out_own, a.nbytes, o);
  }
  u32x4 u2[JP];
  if (!poll_list<JP>(a, own2, poll2, u2, ready, r, s)) return false;
#pragma unroll
  for (int m = 0; m < JP; ++m) st16<kOut>(out_r, ag_off[m], u2[m]);
  if (odd_tail<DT>(a.nbytes)) {
    // the last element of an odd-length message, if it is in one of this wave's partitions
    asm volatile("");
    const uint32_t last = a.nbytes & ~3u;
#pragma unroll
    for (int m = 0; m < JP; ++m) {
      const uint32_t off = ag_off[m];
      const bool tail = off != kDrop && off <= last && last < off + 16u;
      uint32_t word = u2[m][0];
#pragma unroll
      for (int e = 1; e < 4; ++e) word = (off + 4u * e == last) ? u2[m][e] : word;
      st2<kOut>(out_r, tail ? last : kDrop, static_cast<uint16_t>(word & 0xFFFFu));
    }
  }
  wait_all_mem();  // every output store of this wave has landed
  t1 = now_ticks();
  // re-arm this wave's all-gather slots for step s + 2
#pragma unroll
  for (int m = 0; m < JP; ++m) st16<kCoh>(own2, poll2[m], sent);
  return true;
}

// ------------------------------------------------------------------ barrier baseline
//
// Workgroup-level cross-rank barrier (§III.B): every workgroup writes `val` into its flag slot
// of every peer, then waits until every peer's flag in its own block has reached `val`. Flags
// only grow, so they never need resetting. Wave 0 does the signalling; the other waves wait at
// the workgroup barrier.
//
// Failure flags in LDS, each set by at most the waves that give up and never cleared after
// kernel start: every wave reads a flag only after a workgroup barrier that follows every write
// to it, so all waves of a workgroup take the same exit together.
__shared__ int g_bar_fail;   // a cross-rank barrier timed out
__shared__ int g_step_fail;  // a poll inside a step gave up
__shared__ int g_join_fail;  // the rank-local join timed out

__device__ __forceinline__ void fail_flags_init() {
  if (threadIdx.x == 0) {
    g_bar_fail = 0;
    g_step_fail = 0;
    g_join_fail = 0;
  }
  __syncthreads();
}

__device__ bool xrank_barrier(const Args& a, const Ctx& c, uint64_t val, uint64_t s) {
  const int N = a.nranks, r = c.rank;
  __syncthreads();
  if (c.wave == 0) {
    // lane q signals peer q and watches peer q's flag in this rank's block
    const int q = c.lane;
    const bool peer = q < N && q != r;
    if (peer && r != a.withhold) {
      uint64_t* theirs = reinterpret_cast<uint64_t*>(a.base + static_cast<uint64_t>(q) * a.stride +
                                                     a.bar.off) +
                         (static_cast<uint32_t>(r) * kMaxCtasPerRank + c.cta);
      __hip_atomic_store(theirs, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint64_t* mine =
        reinterpret_cast<const uint64_t*>(a.base + static_cast<uint64_t>(r) * a.stride +
                                          a.bar.off) +
        (static_cast<uint32_t>(peer ? q : 0) * kMaxCtasPerRank + c.cta);
    bool need = peer;
    uint32_t spins = 0;
    uint64_t t_first = 0;
    while (true) {
      if (need) {
        const uint64_t fv = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (fv >= val) need = false;
      }
      const uint64_t waiting = __ballot(need);
      if (waiting == 0) break;
      if ((++spins & 1023u) == 0) {
        t_first = poll_check(poll_env(a), t_first, r, __builtin_ctzll(waiting), s);
        if (t_first == 0) {
          if (c.lane == 0) g_bar_fail = 1;
          break;
        }
      }
    }
  }
  __syncthreads();
  return g_bar_fail == 0;
}

// Two-barrier one-shot (the conventional design the pages measure): barrier so that every peer
// has finished with the data slots, plain push, release, barrier so that the data is there,
// acquire, reduce.
template <int DT, int NMAX>
__device__ bool step_barrier2(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                              rsrc_t out_r, int k, uint64_t& t0,
                              uint64_t& t1) {
  const int N = a.nranks, r = c.rank;
  const uint32_t slot = a.bdat.slot, CU = a.chunk_units;
  const uint32_t unit0 = static_cast<uint32_t>(k) * CU;
  stamp_start(t0, k);
  if (!xrank_barrier(a, c, 2 * s, s)) return false;
  if (r != a.withhold) {
    for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CU;
      uint32_t w[4];
      load_unit<DT, 16>(in_r, act ? (unit0 + i) * 16u : kDrop, a.nbytes, w);
      const u32x4 x = {w[0], w[1], w[2], w[3]};
      const uint32_t off = act ? r * slot + i * 16u : kDrop;
#pragma unroll
      for (int j = 1; j < NMAX; ++j) st16<kCoh>(peer_rsrc(a, r, j, a.bdat), off, x);
    }
  }
  wait_all_mem();  // the coherent pushes are performed before the flag that announces them
  if (!xrank_barrier(a, c, 2 * s + 1, s)) return false;
  acquire_agent();
  const rsrc_t own = region_rsrc(a, r, a.bdat);
  const uint32_t peers = peer_mask(N, r);
  for (uint32_t i0 = c.t0; i0 < CU; i0 += c.T) {
    const uint32_t i = i0 + c.lane;
    const bool act = i < CU;
    const uint32_t mask = act ? peers : 0u;
    uint32_t x[4];
    load_unit<DT, 16>(in_r, act ? (unit0 + i) * 16u : kDrop, a.nbytes, x);
    u32x4 v[NMAX];
#pragma unroll
    for (int q = 0; q < NMAX; ++q)
      v[q] = ld16<kCoh>(own, ((mask >> q) & 1u) ? static_cast<uint32_t>(q) * slot + i * 16u : kDrop);
    uint32_t o[4];
    fold_rank_order<DT, NMAX, 4>(N, r, x, v, o);
    store_unit<DT, 16, kOut>(out_r, act ? (unit0 + i) * 16u : kDrop, a.nbytes, o);
  }
  wait_all_mem();
  t1 = now_ticks();
  return true;
}

// ------------------------------------------------------------------ standalone collectives
//
// Reduce-scatter, all-gather and broadcast from the same primitives as the AllReduce kernels
// (the paper notes that AllReduce is commonly split into reduce-scatter + all-gather or
// reduce + broadcast, §III opening paragraph; the Pith review expects these to be rebuilt with
// the same barrier-free pattern): 16-byte units pushed raw into the sentinel-armed p1 slots,
// polled until the sentinel is gone, consumed and re-armed; step s uses buffer s & 1. Each lane
// handles units t0 + lane + j * T of the chunk, the same units on every rank and in every step,
// so every credit below is a per-lane fact. Every step first waits for all of its wave's older
// stores (the re-arms of the previous step) before it pushes. Reduce-scatter and all-gather
// partitions are whole units; `part_units` is their exact size and the last chunk may be short.

// Units of chunk k (the last one may be shorter than chunk_units).
__device__ __forceinline__ uint32_t chunk_len(const Args& a, int k, uint32_t total) {
  const uint32_t u0 = static_cast<uint32_t>(k) * a.chunk_units;
  return u0 >= total ? 0u : min(a.chunk_units, total - u0);
}

// Reduce-scatter: rank r's input holds N partitions of part_units units. Partition (r + j) % N
// goes to that owner's slot r; the owner folds its own partition and the N - 1 received ones in
// rank order into its output. Every pair of ranks exchanges data in every step, so, as in the
// one-shot kernels, receiving a peer's step s-1 data is the credit to overwrite its buffer of
// step s-2.
template <int DT, int NMAX>
__device__ bool step_reducescatter(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                   rsrc_t out_r, int k, uint64_t& t0, uint64_t& t1) {
  const int N = a.nranks, r = c.rank;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot = a.p1.slot, P = a.part_units;
  const uint32_t unit0 = static_cast<uint32_t>(k) * a.chunk_units;
  const uint32_t CK = chunk_len(a, k, P);
  const uint32_t mine = (b * N + r) * slot;
  const rsrc_t own = region_rsrc(a, r, a.p1);
  const uint32_t peers = peer_mask(N, r);
  const u32x4 sent = sentinel_unit<DT, 16>();
  auto ready = [](u32x4 l) { return vec_clear<DT>(l); };
  stamp_start(t0, k);
  wait_all_mem();
  if (r != a.withhold) {
    for (uint32_t i0 = c.t0; i0 < CK; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CK;
      uint32_t w[NMAX][4];
      load_partitions<DT, NMAX>(a, r, in_r, k, i, act, 1, w);
      const uint32_t off = act ? mine + i * 16u : kDrop;
#pragma unroll
      for (int j = 1; j < NMAX; ++j)
        st16<kCoh>(peer_rsrc(a, r, j, a.p1), off, u32x4{w[j][0], w[j][1], w[j][2], w[j][3]});
    }
  }
  for (uint32_t i0 = c.t0; i0 < CK; i0 += c.T) {
    const uint32_t i = i0 + c.lane;
    const bool act = i < CK;
    const uint32_t mask = act ? peers : 0u;
    const uint32_t off0 = b * N * slot + i * 16u;
    uint32_t x[4];
    load_unit<DT, 16, kPlain, false>(in_r, act ? (r * P + unit0 + i) * 16u : kDrop, a.nbytes, x);
    u32x4 v[NMAX];
    if (!poll_lines<NMAX>(a, own, off0, slot, mask, v, ready, r, s)) return false;
    uint32_t o[4];
    fold_rank_order<DT, NMAX, 4>(N, r, x, v, o);
    store_unit<DT, 16, kOut>(out_r, act ? (unit0 + i) * 16u : kDrop, a.out_nbytes, o);
    rearm<NMAX>(own, off0, slot, mask, sent);
  }
  wait_all_mem();
  t1 = now_ticks();
  return true;
}

// All-gather: rank r's input (part_units units) goes to every peer's slot r and to partition r
// of its own output; every other rank's input is copied from its slot into partition q. The
// credit is the one of the reduce-scatter: every pair exchanges data in every step.
template <int DT, int NMAX>
__device__ bool step_allgather(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                               rsrc_t out_r, int k, uint64_t& t0, uint64_t& t1) {
  const int N = a.nranks, r = c.rank;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot = a.p1.slot, P = a.part_units;
  const uint32_t unit0 = static_cast<uint32_t>(k) * a.chunk_units;
  const uint32_t CK = chunk_len(a, k, P);
  const bool sends = r != a.withhold;
  const uint32_t mine = (b * N + r) * slot;
  const rsrc_t own = region_rsrc(a, r, a.p1);
  const uint32_t peers = peer_mask(N, r);
  const u32x4 sent = sentinel_unit<DT, 16>();
  auto ready = [](u32x4 l) { return vec_clear<DT>(l); };
  stamp_start(t0, k);
  wait_all_mem();
  for (uint32_t i0 = c.t0; i0 < CK; i0 += c.T) {
    const uint32_t i = i0 + c.lane;
    const bool act = i < CK;
    uint32_t x[4];
    load_unit<DT, 16, kPlain, false>(in_r, act ? (unit0 + i) * 16u : kDrop, a.nbytes, x);
    if (sends) push_peers<NMAX>(a, r, a.p1, act ? mine + i * 16u : kDrop, u32x4{x[0], x[1], x[2], x[3]});
    store_unit<DT, 16, kOut>(out_r, act ? (r * P + unit0 + i) * 16u : kDrop, a.out_nbytes, x);
  }
  for (uint32_t i0 = c.t0; i0 < CK; i0 += c.T) {
    const uint32_t i = i0 + c.lane;
    const bool act = i < CK;
    const uint32_t mask = act ? peers : 0u;
    const uint32_t off0 = b * N * slot + i * 16u;
    u32x4 v[NMAX];
    if (!poll_lines<NMAX>(a, own, off0, slot, mask, v, ready, r, s)) return false;
#pragma unroll
    for (int q = 0; q < NMAX; ++q) {
      const uint32_t o[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
      store_unit<DT, 16, kOut>(out_r, ((mask >> q) & 1u) ? (q * P + unit0 + i) * 16u : kDrop,
                         a.out_nbytes, o);
    }
    rearm<NMAX>(own, off0, slot, mask, sent);
  }
  wait_all_mem();
  t1 = now_ticks();
  return true;
}

// Broadcast: the root pushes every unit of its input into slot `root` of every peer and copies it
// to its own output; every other rank polls that one slot, copies the unit out and re-arms it.
// Only the root sends data, so receiving gives it no credit: after consuming (and re-arming) step
// s, each receiving wave stores s into its flag in the root's block (the bulk two-shot's flag
// region, phase 0, indexed by the receiver), and the root's matching wave waits for every
// receiver's flag to reach s - 2 before it writes buffer s & 1 again in step s. Flags only grow;
// values left by earlier launches are below this launch's first step, so only steps from the
// third of a launch on wait (the kernel boundary covers the earlier ones).
template <int DT, int NMAX>
__device__ bool step_broadcast(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                               rsrc_t out_r, int k, uint64_t& t0, uint64_t& t1) {
  const int N = a.nranks, r = c.rank, R = a.root;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot = a.p1.slot;
  const uint32_t unit0 = static_cast<uint32_t>(k) * a.chunk_units;
  const uint32_t CK = chunk_len(a, k, (a.nbytes + 15u) / 16u);
  const rsrc_t own = region_rsrc(a, r, a.p1);
  stamp_start(t0, k);
  if (r == R) {
    if (s >= a.e0 + 2 && !bulk_wait(a, c, 0, s - 2)) return false;
    wait_all_mem();
    const bool sends = r != a.withhold;
    const uint32_t mine = (b * N + r) * slot;
    for (uint32_t i0 = c.t0; i0 < CK; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CK;
      uint32_t x[4];
      load_unit<DT, 16>(in_r, act ? (unit0 + i) * 16u : kDrop, a.nbytes, x);
      if (sends)
        push_peers<NMAX>(a, r, a.p1, act ? mine + i * 16u : kDrop, u32x4{x[0], x[1], x[2], x[3]});
      store_unit<DT, 16, kOut>(out_r, act ? (unit0 + i) * 16u : kDrop, a.out_nbytes, x);
    }
  } else {
    const u32x4 sent = sentinel_unit<DT, 16>();
    auto ready = [](u32x4 l) { return vec_clear<DT>(l); };
    for (uint32_t i0 = c.t0; i0 < CK; i0 += c.T) {
      const uint32_t i = i0 + c.lane;
      const bool act = i < CK;
      const uint32_t mask = act ? (1u << R) : 0u;
      const uint32_t off0 = b * N * slot + i * 16u;
      u32x4 v[NMAX] = {};
      if (!poll_lines<NMAX>(a, own, off0, slot, mask, v, ready, r, s)) return false;
      u32x4 got = v[0];
#pragma unroll
      for (int q = 1; q < NMAX; ++q) got = (q == R) ? v[q] : got;
      const uint32_t o[4] = {got.x, got.y, got.z, got.w};
      store_unit<DT, 16, kOut>(out_r, act ? (unit0 + i) * 16u : kDrop, a.out_nbytes, o);
      rearm<NMAX>(own, off0, slot, mask, sent);
    }
    wait_all_mem();  // the re-arms have completed before the flag that hands the buffer back
    if (c.lane == 0)
      __hip_atomic_store(bulk_flag(a, R, 0, r, c), s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_all_mem();
  t1 = now_ticks();
  return true;
}

// One-pass broadcast (every unit of the chunk has its own lane), on the near slots when the
// message fits them: the same protocol as step_broadcast, with 8- or 16-byte units and a single
// round of polls per lane.
template <int DT, int NMAX, int UB>
__device__ bool step_broadcast_1p(const Args& a, const Ctx& c, uint64_t s, rsrc_t in_r,
                                  rsrc_t out_r, int k, uint64_t& t0, uint64_t& t1) {
  using V = unit_t<UB>;
  constexpr int W = UB / 4;
  const int N = a.nranks, r = c.rank, R = a.root;
  const uint32_t b = static_cast<uint32_t>(s & 1u);
  const uint32_t slot = a.p1.slot, CU = a.chunk_units;
  const uint32_t U = (a.nbytes + UB - 1) / UB;
  const uint32_t i = c.t0 + c.lane;
  const bool act = i < CU && k * CU + i < U;
  const uint32_t uoff = (k * CU + i) * UB;
  uint32_t off0 = b * N * slot + slot_off<UB>(a.p1, i);
  pin(off0);
  stamp_start(t0, k);
  if (r == R) {
    if (s >= a.e0 + 2 && !bulk_wait(a, c, 0, s - 2)) return false;
    uint32_t x[W];
    load_unit<DT, UB>(in_r, act ? uoff : kDrop, a.nbytes, x);
    compiler_fence();
    wait_vm<0>();
    store_unit<DT, UB, kOut>(out_r, act ? uoff : kDrop, a.out_nbytes, x);
    if (r != a.withhold) {
      V line;
#pragma unroll
      for (int e = 0; e < W; ++e) line[e] = x[e];
      push_peers<NMAX>(a, r, a.p1, act ? off0 + static_cast<uint32_t>(R) * slot : kDrop, line);
    }
    compiler_fence();
    wait_vm<NMAX - 1>();  // the output store has landed; the pushes may be in flight
  } else {
    const V sent = sentinel_unit<DT, UB>();
    auto ready = [](V l) { return vec_clear<DT>(l); };
    const uint32_t mask = act ? (1u << R) : 0u;
    V v[NMAX] = {};
    if (!poll_all<NMAX>(a, region_rsrc(a, r, a.p1), off0, slot, mask, v, ready, r, s))
      return false;
    V got = v[0];
#pragma unroll
    for (int q = 1; q < NMAX; ++q) got = (q == R) ? v[q] : got;
    uint32_t o[W];
#pragma unroll
    for (int e = 0; e < W; ++e) o[e] = got[e];
    store_unit<DT, UB, kOut>(out_r, act ? uoff : kDrop, a.out_nbytes, o);
    rearm<NMAX>(region_rsrc(a, r, a.p1), off0, slot, mask, sent);
    compiler_fence();
    wait_vm<0>();  // output and re-arm have completed before the flag that hands the buffer back
    if (c.lane == 0)
      __hip_atomic_store(bulk_flag(a, R, 0, r, c), s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  t1 = now_ticks();
  return true;
}

// ------------------------------------------------------------------ persistent driver

__device__ __forceinline__ void drift_sleep(const Args& a, int it, int r, int cta) {
  uint32_t h = static_cast<uint32_t>(it) * 0x9E3779B1u ^ static_cast<uint32_t>(r) * 0x85EBCA77u ^
               static_cast<uint32_t>(cta) * 0xC2B2AE3Du;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const uint32_t n = uni(h % static_cast<uint32_t>(a.drift + 1));
  for (uint32_t z = 0; z < n; ++z) __builtin_amdgcn_s_sleep(64);
}

// Rank-local join between two iterations of the persistent loop: every wave of every workgroup
// of this rank has finished iteration `it` before any starts the next one. It stands in for the
// kernel boundary that separates two AllReduce calls on one GPU and involves no other rank.
// Workgroup c publishes `token` (the last sequence number of the iteration, which only grows)
// in its slot of the rank's own row of the flag region, then waits for the rank's other slots.
__device__ bool rank_join(const Args& a, const Ctx& c, uint64_t token, bool failed) {
  if (failed) g_step_fail = 1;
  __syncthreads();
  if (g_step_fail != 0) return false;
  if (a.ctas > 1) {
    if (c.wave == 0) {
      const rsrc_t own = region_rsrc(a, c.rank, a.bar);
      const uint32_t row = static_cast<uint32_t>(c.rank) * kMaxCtasPerRank * 8u;
      const u32x2 tv = {static_cast<uint32_t>(token), static_cast<uint32_t>(token >> 32)};
      if (c.lane == 0) st8<kCoh>(own, row + c.cta * 8u, tv);
      uint32_t need = 0;
#pragma unroll
      for (int j = 0; j < kMaxCtasPerRank / kWave; ++j)
        if (c.lane + j * kWave < a.ctas) need |= 1u << j;
      uint32_t spins = 0;
      uint64_t t_first = 0;
      while (true) {
#pragma unroll
        for (int j = 0; j < kMaxCtasPerRank / kWave; ++j) {
          if (need & (1u << j)) {
            const u32x2 f = ld8<kCoh>(own, row + (c.lane + j * kWave) * 8u);
            compiler_fence();
            if (((static_cast<uint64_t>(f.y) << 32) | f.x) >= token) need &= ~(1u << j);
          }
        }
        if (__ballot(need != 0) == 0) break;
        if ((++spins & 1023u) == 0) {
          t_first = poll_check(poll_env(a), t_first, c.rank, c.rank, token);
          if (t_first == 0) {
            if (c.lane == 0) g_join_fail = 1;
            break;
          }
        }
      }
    }
    __syncthreads();
    if (g_join_fail != 0) return false;
  }
  return true;
}

// Entry of every AllReduce and collective kernel. A launch that finds the abort word raised (an
// earlier launch on the handle timed out) exits before any load or store: its scratch may hold
// data a poll would take for this launch's, so it writes nothing, and the host learns of the
// timeout from the status words. Thread 0 reads the word once for its whole workgroup so that
// every wave takes the same exit. With a launch record, lane 0 of each workgroup stores its
// XCC id and the rank and workgroup index it decoded.
__shared__ uint32_t g_abort_seen;

__device__ __forceinline__ bool enter(const Args& a, Ctx& c) {
  if (threadIdx.x == 0) {
    g_abort_seen = __hip_atomic_load(&a.ctl[CTL_ABORT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g_split_fail = 0u;
  }
  const bool mapped = decode(a, c);
  if (a.launch_rec != nullptr && threadIdx.x == 0)
    a.launch_rec[blockIdx.x] =
        xcc_id() | (mapped ? (static_cast<uint32_t>(c.rank + 1) << 8) |
                                 (static_cast<uint32_t>(c.cta) << 16)
                           : 0u);
  __syncthreads();
  return mapped && g_abort_seen == 0;
}

template <int ALGO, int DT, int NMAX>
__device__ __forceinline__ void ar_body(const Args& a) {
  Ctx c;
  if (!enter(a, c)) return;
  const int N = a.nranks;
  const int wpb = c.wpb;
  constexpr bool kBarrier = ALGO == ALGO_BARRIER2 || ALGO == ALGO_BARRIER_ONLY;
  // A rank that is a single wave needs no join: its iterations are already in program order.
  const bool join = a.iters > 1 && ALGO != ALGO_BARRIER_ONLY && (a.ctas > 1 || wpb > 1);
  if (kBarrier || join) fail_flags_init();
  // Buffers of iteration `it`: evenly spaced sets are addressed arithmetically; otherwise the
  // set table is read one iteration ahead so that its latency stays off the timed path.
  const bool affine = a.in_set_stride != 0 || a.out_set_stride != 0;
  const bool table = !affine && a.in_tab != nullptr;
  const void* next_in = table ? a.in_tab[c.rank] : a.in[c.rank];
  void* next_out = table ? a.out_tab[c.rank] : a.out[c.rank];
  // timestamps of this wave: [iteration][rank][workgroup][wave]
  const uint64_t ts_first = (static_cast<uint64_t>(c.rank) * a.ctas + c.cta) * wpb + c.wave;
  const uint64_t ts_step = static_cast<uint64_t>(N) * a.ctas * wpb;
  uint64_t* ts_s = a.ts_start + ts_first;
  uint64_t* ts_e = a.ts_end + ts_first;
  int set = 0;
  for (int it = 0; it < a.iters; ++it) {
    const void* inp = next_in;
    void* outp = next_out;
    const int cur = set;  // this iteration's input/output set
    if (affine) {
      inp = static_cast<const uint8_t*>(a.in[c.rank]) + set * a.in_set_stride;
      outp = static_cast<uint8_t*>(a.out[c.rank]) + set * a.out_set_stride;
    }
    if (++set == a.nsets) set = 0;
    const rsrc_t in_r = in_rsrc(uniform_ptr(inp), a.nbytes);
    const rsrc_t out_r = out_rsrc(const_cast<void*>(uniform_ptr(outp)), a.out_nbytes);
    if (a.drift > 0) drift_sleep(a, it, c.rank, c.cta);
    if (table && it + 1 < a.iters) {
      next_in = a.in_tab[set * N + c.rank];
      next_out = a.out_tab[set * N + c.rank];
    }
    uint64_t t_start = 0;  // stamped by the first step right before its first input load
    uint64_t t_end = 0;    // stamped by the last step right after its output stores completed
    bool failed = false;
    uint64_t s = 0;
    for (int k = 0; k < a.chunks; ++k) {
      const uint64_t step = static_cast<uint64_t>(it) * a.chunks + k;
      s = a.e0 + step;
      bool ok;
      if constexpr (ALGO == ALGO_ONESHOT_LL) {
        ok = step_oneshot_ll<DT, NMAX, false>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_LL_TWO_PAGE) {
        ok = step_oneshot_ll<DT, NMAX, false, true>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_LL_MULTI) {
        ok = step_oneshot_ll<DT, NMAX, true>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_SENTINEL) {
        ok = step_oneshot_sentinel<DT, NMAX, false>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_SENTINEL_MULTI) {
        ok = step_oneshot_sentinel<DT, NMAX, true>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_SENTINEL_TWO_PAGE) {
        ok = step_oneshot_sentinel<DT, NMAX, false, 16, true>(a, c, s, in_r, out_r, k, t_start,
                                                              t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_SENTINEL_NARROW) {
        ok = step_oneshot_sentinel<DT, NMAX, false, 8>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_TWOSHOT) {
        ok = step_twoshot<DT, NMAX>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_TWOSHOT_NARROW) {
        ok = step_twoshot<DT, NMAX, 8>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_TWOSHOT_TWO_PAGE) {
        ok = step_twoshot<DT, NMAX, 16, 0, true>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_SPLIT) {
        ok = step_oneshot_split<DT, NMAX, 16>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_LL_SPLIT) {
        ok = step_oneshot_ll_split<DT, NMAX>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ONESHOT_SPLIT_NARROW) {
        ok = step_oneshot_split<DT, NMAX, 8>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_TWOSHOT_SPLIT) {
        ok = step_twoshot_split<DT, NMAX, 16>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_TWOSHOT_SPLIT_NARROW) {
        ok = step_twoshot_split<DT, NMAX, 8>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_SPLIT) {
        ok = step_ll128_split<DT, NMAX, 4>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_SPLIT_E1) {
        ok = step_ll128_split<DT, NMAX, 1>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_SPLIT_E2) {
        ok = step_ll128_split<DT, NMAX, 2>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_TWOSHOT_BULK) {
        ok = step_twoshot_bulk<DT, NMAX>(a, c, s, in_r, out_r, k, cur, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_ATOMIC) {
        ok = step_ll128<DT, NMAX>(a, c, s, in_r, out_r, k, cur, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_E1) {
        ok = step_ll128<DT, NMAX, 1>(a, c, s, in_r, out_r, k, cur, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_E2) {
        ok = step_ll128<DT, NMAX, 2>(a, c, s, in_r, out_r, k, cur, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_DET) {
        ok = step_ll128<DT, NMAX, 4, true>(a, c, s, in_r, out_r, k, cur, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_DET_E1) {
        ok = step_ll128<DT, NMAX, 1, true>(a, c, s, in_r, out_r, k, cur, t_start, t_end);
      } else if constexpr (ALGO == ALGO_LL128_DET_E2) {
        ok = step_ll128<DT, NMAX, 2, true>(a, c, s, in_r, out_r, k, cur, t_start, t_end);
      } else if constexpr (ALGO == ALGO_BARRIER2) {
        ok = step_barrier2<DT, NMAX>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_RS_ONEPASS) {
        ok = step_twoshot<DT, NMAX, 16, 1>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_RS_NARROW) {
        ok = step_twoshot<DT, NMAX, 8, 1>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_AG_ONEPASS) {
        ok = step_twoshot<DT, NMAX, 16, 2>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_AG_NARROW) {
        ok = step_twoshot<DT, NMAX, 8, 2>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_REDUCESCATTER) {
        ok = step_reducescatter<DT, NMAX>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_ALLGATHER) {
        ok = step_allgather<DT, NMAX>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_BCAST_ONEPASS) {
        ok = step_broadcast_1p<DT, NMAX, 16>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_BCAST_NARROW) {
        ok = step_broadcast_1p<DT, NMAX, 8>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else if constexpr (ALGO == ALGO_BROADCAST) {
        ok = step_broadcast<DT, NMAX>(a, c, s, in_r, out_r, k, t_start, t_end);
      } else {
        stamp_start(t_start, k);
        ok = xrank_barrier(a, c, 2 * s, s);
        t_end = now_ticks();
      }
      if (!ok) {
        failed = true;
        break;
      }
    }
    // every step returns once its output stores have completed
    if (!failed && a.ts_end != nullptr) {

      if (c.lane == 0) {
        *ts_s = t_start;
        *ts_e = t_end;
      }
      ts_s += ts_step;
      ts_e += ts_step;
    }
    if (join) {
      if (!rank_join(a, c, s, failed)) return;
    } else if (failed) {
      return;
    }
  }
}

template <int ALGO, int DT, int NMAX>
__global__ __launch_bounds__(256) void ar_kernel(Args a) {
  ar_body<ALGO, DT, NMAX>(a);
}

// The bandwidth-regime two-shot in a kernel of its own, with a register budget that lets
// several waves share every SIMD (more streaming loads in flight per compute unit than the
// latency kernel's one wave per SIMD) and still spills nothing to the private segment: a
// kernel with a private segment can have fewer waves resident than the occupancy arithmetic
// counts (the runtime sizes the scratch it backs them with), and every wave of these grids
// polls for the others.
// bf16 folds in binary32, two values per input word, and needs about twice the registers.
constexpr int bulk_waves_per_eu(int dt, int nmax) {
  return dt == DT_BF16 ? (nmax >= 16 ? 1 : nmax >= 8 ? 2 : 3) : (nmax >= 16 ? 2 : 3);
}

template <int DT, int NMAX>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(bulk_waves_per_eu(DT, NMAX))))
void ar_kernel_bulk(Args a) {
  ar_body<ALGO_TWOSHOT_BULK, DT, NMAX>(a);
}

}  // namespace ar
