// Host runtime and C ABI: handle, symmetric scratch allocator, sequence numbers, launch
// geometry, the persistent benchmark driver and error reporting.
//
// Scratch layout (one device allocation; rank r's block at base + r * stride, every region at the
// same offset in every block, as in symmetric memory, Every µs Matters §II.B):
//   p1   [buffer 2][source N][slot]   sentinel   one-shot slots / two-shot reduce-scatter slots
//   p2   [buffer 2][source N][slot]   sentinel   two-shot all-gather slots
//   ll   [buffer 2][source N][slot]   zero       LL lines, 16 bytes per 8 bytes of payload
//   acc  [buffer 2][slot]             zero       LL128-style shared atomic destination
//   cnt  [buffer 2][cta][wave] u32    zero       LL128-style arrival counters
//   bar  [source][cta] u64            zero       barrier flags (monotonic)
//   bdat [source N][slot]             any        barrier-baseline data slots
//   pf1  [buffer 2][source N][slot]   any        bulk two-shot reduce-scatter slots
//   pf2  [buffer 2][source N][slot]   any        bulk two-shot all-gather slots
//   flg  [phase 2][source][cta][wave] zero       bulk two-shot completion flags (monotonic)
// Every block starts with three 2 MiB near pages holding copies of ll, p1 and p2 for messages
// whose 2 * N slots fit a page: slot data in 8 KiB chunks, one per 16 KiB of pitch, each in the
// granule homed in the rank's XCD half (per-page positions calibrated at creation, ar_args.h).
// The two buffers implement double buffering: step s uses buffer s & 1 (Fig. 4 and §IV
// "Bidirectional Communication Double Buffering"; Fig. 7's per-epoch alternating sub-buffers).

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/ar.h"
#include "ar_internal.h"

namespace {

// Message of the last failing call on this thread. A fixed buffer: recording an error never
// allocates (the allocation-free entry point shares this path).
thread_local char g_err[512];

constexpr int kRegions = 15;
enum RegionId {
  RG_P1 = 0, RG_P2, RG_LL, RG_ACC, RG_CNT, RG_BAR, RG_BDAT,
  RG_LLN, RG_P1N, RG_P2N,  // near copies of ll, p1, p2 for small messages
  RG_PF1, RG_PF2, RG_FLG,  // bulk two-shot data slots and completion flags
  RG_REC,                  // launch record (AR_OPT_RECORD_LAUNCH), written in rank 0's block only
  RG_SINK,                 // where idle lanes' packed bf16 atomics add zero
};
// Default scratch per rank per protocol, from a scratch-size sweep on MI355X (the counterpart of
// the pages' Fig. 12; the Pith review's "Assumptions & free parameters" give 4 MiB for the
// one-shot and 64 MiB for the two-shot and LL128 on their hardware). One-shot: 4 MiB, as on the
// pages (1-256 MiB measured within noise below 1 MiB per rank; 1 MiB at 16 ranks 11 % faster in
// chunks than whole). Two-shot and LL128: 16 MiB, one 1 MiB slot per (buffer, source) at 8
// ranks, so that one step's scratch (about 128 MiB over all ranks) stays in the 256 MB MALL:
// 256 MiB x 8 ranks in 1.90 ms against 2.20 ms at 64 MiB and 2.28 ms at 256 MiB; 6-48 MiB
// were measured, 16 MiB was the fastest at 16, 64 and 256 MiB per rank. Larger messages run in
// equal chunks.
constexpr uint64_t kDefaultCapOneShot = 4ull << 20;
constexpr uint64_t kDefaultCapTwoShot = 16ull << 20;
constexpr uint64_t kMaxCap = 1ull << 30;  // keeps every region below the drop offset (2 GiB)
constexpr int kXcds = 8;

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
uint64_t ceil_div(uint64_t x, uint64_t a) { return (x + a - 1) / a; }

uint64_t env_u64(const char* name, uint64_t dflt) {
  const char* v = std::getenv(name);
  if (v == nullptr || *v == '\0') return dflt;
  char* end = nullptr;
  unsigned long long x = std::strtoull(v, &end, 10);
  if (end == v) return dflt;
  return static_cast<uint64_t>(x);
}

int elem_bytes(int dt) { return dt == AR_BFLOAT16 ? 2 : 4; }

uint32_t sentinel_word(int dt) { return dt == AR_INT32 ? 0x80000000u : 0xFFFFFFFFu; }

// Resident workgroups per compute unit for (kernel, block size), cached in a fixed table (no
// allocation). The key keeps both parts: the host handles of different kernels are only a few
// bytes apart, so any mixing of the two into one number could give a kernel the occupancy of
// another, and a grid planned on a too-high occupancy cannot be co-resident.
struct OccEntry {
  const void* fn;
  int threads;
  int blocks;
};
constexpr int kOccSlots = 2048;  // > kernels (about 250) x block sizes (3)
std::mutex g_occ_mu;
OccEntry g_occ[kOccSlots];

int occupancy(ar_kernel_fn fn, int threads) {
  std::lock_guard<std::mutex> lk(g_occ_mu);
  const void* key = reinterpret_cast<const void*>(fn);
  size_t i = (reinterpret_cast<uintptr_t>(key) / 16 * 31 + static_cast<size_t>(threads)) % kOccSlots;
  for (int probe = 0; probe < kOccSlots; ++probe, i = (i + 1) % kOccSlots) {
    if (g_occ[i].fn == key && g_occ[i].threads == threads) return g_occ[i].blocks;
    if (g_occ[i].fn == nullptr) {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, key, threads, 0) != hipSuccess)
        nb = 0;
      g_occ[i] = OccEntry{key, threads, nb};
      return nb;
    }
  }
  return 0;
}

// Region layout of one rank block (the same in every block: symmetric memory, §II.B) for N ranks
// and messages of up to max_bytes per rank, with per-protocol scratch caps. With `near` the block
// starts with the near pages (ll, p1, p2: one 2 MiB page each, two for the regions `two_page`
// marks) and is a whole number of 2 MiB pages; `record` adds the launch record region. Writes the
// regions and the block size (*stride).
int layout(int N, uint64_t max_bytes, uint64_t cap_os, uint64_t cap_ts, bool near,
           const bool* two_page, bool record, ar::Region* rg, uint64_t* stride) {
  // Slot sizes: large enough for the whole message unless the per-protocol cap says otherwise.
  const uint64_t need_os = round_up(max_bytes, 16);
  const uint64_t need_ts = ceil_div(ceil_div(max_bytes, 16), N) * 16;
  const uint64_t per_slot_os = std::max<uint64_t>(256, (cap_os / (2 * N)) / 256 * 256);
  const uint64_t per_slot_ts = std::max<uint64_t>(256, (cap_ts / (2 * N)) / 256 * 256);
  const uint64_t slot_os = std::min(round_up(need_os, 256), per_slot_os);
  const uint64_t slot_ts = std::min(round_up(need_ts, 256), per_slot_ts);
  const uint64_t ll_payload = std::min(round_up(max_bytes, 8), std::max<uint64_t>(128, per_slot_os / 2));
  const uint64_t slot_ll = round_up(2 * ll_payload, 256);
  struct { uint64_t slot, bytes; } sz[kRegions] = {};
  sz[RG_P1] = {std::max(slot_os, slot_ts), 2ull * N * std::max(slot_os, slot_ts)};
  sz[RG_P2] = {slot_ts, 2ull * N * slot_ts};
  sz[RG_LL] = {slot_ll, 2ull * N * slot_ll};
  // LL128-style destinations: [buffer 2][group ceil(N / 2)][slot], a slot holding a partition
  // chunk in binary32 (twice the bytes of a bf16 chunk, for the deterministic variant)
  sz[RG_ACC] = {2 * slot_ts, 2ull * ((N + 1) / 2) * 2 * slot_ts};
  // arrival counters [buffer 2][cta][wave], then the deterministic tickets [buffer][group][cta][wave]
  sz[RG_CNT] = {0, (2ull + 2ull * ar::kMaxRanks) * ar::kMaxCtasPerRank * ar::kMaxWavesPerCta * 4};
  sz[RG_BAR] = {0, 1ull * ar::kMaxRanks * ar::kMaxCtasPerRank * 8};
  sz[RG_BDAT] = {slot_os, 1ull * N * slot_os};
  // The bulk two-shot's slots are 4 KiB longer than their data: an owner reads all N sources'
  // slots at one offset at once, and streams exactly a power of two apart measured ~5 % slower.
  const uint64_t pitch_pf = slot_ts + 4096;
  sz[RG_PF1] = {pitch_pf, 2ull * N * pitch_pf};
  sz[RG_PF2] = {pitch_pf, 2ull * N * pitch_pf};
  sz[RG_FLG] = {0, 2ull * ar::kMaxRanks * ar::kMaxCtasPerRank * ar::kMaxWavesPerCta * 8};
  sz[RG_REC] = {0, record ? 4ull * ar::kMaxGrid : 0ull};
  sz[RG_SINK] = {0, 16384};
  // near area: the near ll, p1 and p2 regions, one 2 MiB page each or two for p1 and p2 (pitch
  // set per launch)
  uint64_t off = 0;
  for (int i = RG_LLN; i <= RG_P2N; ++i) {
    rg[i] = ar::Region{};
    rg[i].near = 1;
    if (!near) continue;
    rg[i].off = off;
    const uint64_t pages = two_page != nullptr && two_page[i - RG_LLN] ? 2 : 1;
    rg[i].bytes = static_cast<uint32_t>(pages * ar::kNearPage);
    off += pages * ar::kNearPage;
  }
  for (int i : {RG_P1, RG_P2, RG_LL, RG_ACC, RG_CNT, RG_BAR, RG_BDAT, RG_PF1, RG_PF2, RG_FLG,
                RG_REC, RG_SINK}) {
    if (sz[i].bytes >= (1ull << 31)) {
      return ar_fail(AR_ETOOBIG, "scratch region %d would exceed 2 GiB per rank", i);
    }
    rg[i] = ar::Region{};
    rg[i].off = off;
    rg[i].bytes = static_cast<uint32_t>(sz[i].bytes);
    rg[i].slot = static_cast<uint32_t>(sz[i].slot);
    off = round_up(off + sz[i].bytes, 4096);
  }
  // Rank blocks with near pages start on 2 MiB boundaries so that every near region is one page.
  *stride = near ? round_up(off, ar::kNearPage) : round_up(off, 4096);
  return AR_OK;
}

}  // namespace

int ar_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::memcpy(g_err, buf, sizeof g_err);
  return code;
}

int ar_fail_hip(hipError_t e, const char* what) {
  return ar_fail(AR_EHIP, "%s failed: %s", what, hipGetErrorString(e));
}

struct ar_handle {
  int nranks = 0;
  int dtype = 0;
  size_t max_bytes = 0;
  int device = 0;
  void* raw = nullptr;      // the allocation; base is its first 2 MiB boundary
  uint8_t* base = nullptr;
  uint64_t stride = 0;
  // calibrated store -> poll latency of every position, per rank block, near region, XCD pair
  float near_ns[ar::kMaxRanks][ar::kNearRegions][4][ar::kNearPositions] = {};
  // the same for the second pages of two-page near regions
  float near_ns2[ar::kMaxRanks][ar::kNearRegions][4][ar::kNearPositions] = {};
  bool two_page[ar::kNearRegions] = {};  // which near regions (ll, p1, p2) span two pages
  int use_two_page = 1;   // two-page near slots may be planned
  ar::Region rg[kRegions] = {};
  uint32_t* ctl = nullptr;          // device control words
  uint32_t* status_host = nullptr;  // pinned host status words
  uint32_t* status_dev = nullptr;   // device view of the same memory
  uint64_t epoch = 1;
  bool poisoned = false;
  int64_t timeout_us = 2000000;
  int withhold = -1;
  int ctas = 0;
  int threads = 0;
  int placement = AR_PLACE_XCD;
  int drift = 0;
  int narrow = 1;  // one-pass sentinel kernels may use 8-byte units
  int root = 0;    // ar_bench of AR_BROADCAST: the root rank
  bool near_ok = true;    // the blocks start with calibrated near pages
  int group = 2;          // deterministic LL128-style variant: ranks per group
  int check_inputs = 0;   // check every call's inputs against the sentinel before launching
  int record_launch = 0;  // kernels write the launch record (region RG_REC of rank 0)
  int cooperative = 0;    // launches go through the cooperative launch (residency checked)
  int split = 1;          // the peer-split one-pass kernels may be planned
  int two_halves = 1;     // two-half near slots may be planned (one-shot on two XCDs per rank)
  void** tab = nullptr;
  size_t tab_cap = 0;
  uint64_t* ts = nullptr;
  size_t ts_cap = 0;
  hipStream_t last_stream = nullptr;
  int cu_count = 0;
  double clock_hz = 0.0;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
};

namespace {

struct Launch {
  ar_kernel_fn fn = nullptr;
  int kernel_algo = 0;  // the kernel family actually launched (public or internal algorithm id)
  int chunks = 1;
  uint32_t chunk_units = 0;
  uint32_t part_units = 0;
  int threads = 64;
  int ctas = 1;
  int block = ar::kWave;  // peer-split LL128-style kernel: units per workgroup
  int ranks_per_xcd = 1;
  int xcds_per_rank = 1;
  bool two_halves = false;  // p1 is a two-half near region (the rank spans one XCD of each half)
  bool two_page = false;    // the plan's near regions span two pages (buffer b in page b): p1
                            // and p2 for the two-shot, ll for the one-shot LL
  bool near = false;        // slots in the near regions (ll, p1, p2 below, with their pitch and
  ar::Region near_rg[ar::kNearRegions] = {};  //   each rank's data position for this launch)
  unsigned grid = 1;
};

// Plan with slot units of `ub` bytes (16, or 8 for the narrow one-pass sentinel kernels). With
// ub == 8 the plan only succeeds for a chunk that fits one pass of co-resident lanes; otherwise
// it returns kNoNarrow without recording an error.
constexpr int kNoNarrow = 1;
int plan_units(ar_handle* h, int algo, uint64_t nbytes, int ub, Launch& L) {
  const int N = h->nranks;
  const int nmax = N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : 16;
  // the kernel for a chunk that fits one pass of the rank's lanes
  const int one_pass = ub == 8 ? (algo == AR_TWOSHOT         ? ar::ALGO_TWOSHOT_NARROW
                                  : algo == AR_REDUCESCATTER ? ar::ALGO_RS_NARROW
                                  : algo == AR_ALLGATHER     ? ar::ALGO_AG_NARROW
                                  : algo == AR_BROADCAST     ? ar::ALGO_BCAST_NARROW
                                                             : ar::ALGO_ONESHOT_SENTINEL_NARROW)
                               : (algo == AR_REDUCESCATTER ? ar::ALGO_RS_ONEPASS
                                  : algo == AR_ALLGATHER   ? ar::ALGO_AG_ONEPASS
                                  : algo == AR_BROADCAST   ? ar::ALGO_BCAST_ONEPASS
                                                           : algo);
  L.fn = ar_select_kernel(one_pass, h->dtype, nmax);
  L.kernel_algo = one_pass;
  if (L.fn == nullptr)
    return ar_fail(AR_ENOTSUP, "algorithm %d is not provided for dtype %d", algo, h->dtype);
  uint64_t cap_units = 0, units = 0;
  uint64_t line = static_cast<uint64_t>(ub);  // slot bytes per unit
  switch (algo) {
    case AR_ONESHOT_LL:
      units = ceil_div(nbytes, 8);
      line = 16;
      cap_units = h->rg[RG_LL].slot / 16;
      break;
    case AR_ONESHOT_SENTINEL:
      units = ceil_div(nbytes, line);
      cap_units = h->rg[RG_P1].slot / line;
      break;
    case AR_BARRIER2:
      units = ceil_div(nbytes, 16);
      cap_units = h->rg[RG_BDAT].slot / 16;
      break;
    case AR_REDUCESCATTER:  // nbytes is the whole input: N partitions of whole units
      units = ceil_div(nbytes, line * static_cast<uint64_t>(N));
      cap_units = h->rg[RG_P1].slot / line;
      break;
    case AR_ALLGATHER:  // one-pass on the all-gather slots, the loop kernel on p1 (larger)
      units = ceil_div(nbytes, line);
      cap_units = h->rg[RG_P2].slot / line;
      break;
    case AR_BROADCAST:
      units = ceil_div(nbytes, line);
      cap_units = h->rg[RG_P1].slot / line;
      break;
    case AR_TWOSHOT:
    case AR_LL128_ATOMIC:
    case AR_LL128_DET:
      units = ceil_div(ceil_div(nbytes, line), N);  // one partition
      // a destination slot holds a chunk in binary32: 32 bytes per 16-byte bf16 unit for the
      // deterministic variant
      cap_units = std::min({h->rg[RG_P1].slot, h->rg[RG_P2].slot,
                            h->rg[RG_ACC].slot / (algo == AR_LL128_DET && h->dtype == AR_BFLOAT16
                                                      ? 2u : 1u),
                            h->rg[RG_PF1].slot, h->rg[RG_PF2].slot}) /
                  line;
      break;
    case AR_BARRIER_ONLY:
      units = 0;
      cap_units = 1;
      break;
    default:
      return ar_fail(AR_EINVAL, "unknown algorithm %d", algo);
  }
  const int cus_per_xcd = std::max(1, h->cu_count / kXcds);
  if (algo == AR_LL128_DET) {
    // The deterministic variant orders each member's adds by a ticket per wave, so every unit of
    // a chunk needs its own lane: a chunk is at most one 256-thread workgroup per compute unit
    // of the smallest share of the chip the placement gives a rank.
    const int min_rank_cus = h->placement == AR_PLACE_XCD
                                 ? cus_per_xcd / static_cast<int>(ceil_div(N, kXcds))
                             : h->placement == AR_PLACE_SAME ? cus_per_xcd / N
                                                             : h->cu_count / N;
    const uint64_t wgs = h->ctas ? h->ctas : std::max(1, min_rank_cus);
    cap_units = std::min<uint64_t>(cap_units, wgs * (h->threads ? h->threads : 256));
  }
  if (cap_units == 0) return ar_fail(AR_EINVAL, "scratch slots are too small");
  // Messages whose 2 * N slots fit a near page in one chunk use the near regions: the slot data
  // goes in 8 KiB chunks at a pitch of 16 KiB per chunk.
  const uint64_t near_chunks = ceil_div(units * line, ar::kGranule);
  // Two-page near slots (handles with more than 8 ranks): the two-shot's 2 N slots need more than
  // one page and the N slots of one buffer fit one.
  const bool two_page = h->use_two_page && h->near_ok && units > 0 &&
                        ((algo == AR_TWOSHOT && N > 8 && h->two_page[1] && h->two_page[2]) ||
                         (algo == AR_ONESHOT_LL && h->two_page[0]) ||
                         (algo == AR_ONESHOT_SENTINEL && N >= 8 && h->two_page[1])) &&
                        h->placement == AR_PLACE_XCD &&
                        2ull * N * near_chunks * 2 * ar::kGranule > ar::kNearPage &&
                        1ull * N * near_chunks * 2 * ar::kGranule <= ar::kNearPage;
  const bool near_fits = h->near_ok && units > 0 &&
                         (two_page || 2ull * N * near_chunks * 2 * ar::kGranule <= ar::kNearPage) &&
                         (algo == AR_ONESHOT_LL || algo == AR_ONESHOT_SENTINEL ||
                          algo == AR_TWOSHOT || algo == AR_REDUCESCATTER || algo == AR_ALLGATHER ||
                          algo == AR_BROADCAST ||
                          ((algo == AR_LL128_ATOMIC || algo == AR_LL128_DET) &&
                           units <= h->rg[RG_ACC].slot / 32 &&
                           (algo != AR_LL128_DET || units <= cap_units)));
  L.ranks_per_xcd = h->placement == AR_PLACE_XCD ? static_cast<int>(ceil_div(N, kXcds)) : 1;
  // Chunk geometry, workgroup shape and kernel for the near or the regular slots.
  auto shape = [&](bool near) -> int {
    L.fn = ar_select_kernel(one_pass, h->dtype, nmax);
    L.kernel_algo = one_pass;
    L.near = near;
    const uint64_t K = near || units == 0 ? 1 : ceil_div(units, cap_units);
    const uint64_t C = units == 0 ? 0 : ceil_div(units, K);
    L.chunks = static_cast<int>(K);
    L.chunk_units = static_cast<uint32_t>(C);
    L.part_units = static_cast<uint32_t>(K * C);
    // With N dividing 8 every rank gets 8 / N XCDs (its first workgroup stays on XCD r); the
    // other counts leave 8 - N XCDs idle rather than split a rank unevenly. Messages in the near
    // regions stay on the rank's first XCD: their slots are homed near that XCD's half of the
    // chip.
    L.xcds_per_rank = (h->placement == AR_PLACE_XCD && N < kXcds && kXcds % N == 0 && !near)
                          ? kXcds / N
                          : 1;
    const int rank_cus = std::max(1, h->placement == AR_PLACE_XCD
                                         ? cus_per_xcd * L.xcds_per_rank / L.ranks_per_xcd
                                     : h->placement == AR_PLACE_SAME ? cus_per_xcd / N
                                                                     : h->cu_count / N);
    // Every kernel of the public algorithms starts from the smallest workgroup (whole waves)
    // that covers the chunk with at most one workgroup per compute unit of the rank, so that each
    // wave has a compute unit's memory pipeline to itself (measured 5-33 % lower p50 than one
    // wider workgroup at N = 4..16, the barrier baseline included). The multi-pass and bulk
    // kernels that take over wider chunks use 256-thread workgroups.
    const bool one_pass = algo == AR_ONESHOT_LL || algo == AR_ONESHOT_SENTINEL ||
                          algo == AR_TWOSHOT || algo == AR_LL128_ATOMIC ||
                          algo == AR_LL128_DET || algo == AR_BARRIER2 ||
                          algo == AR_REDUCESCATTER || algo == AR_ALLGATHER ||
                          algo == AR_BROADCAST;
    const uint64_t spread = round_up(ceil_div(C, static_cast<uint64_t>(rank_cus)), 64);
    L.threads = h->threads ? h->threads
                : one_pass ? static_cast<int>(std::min<uint64_t>(256, std::max<uint64_t>(64, spread)))
                : (C <= 256 ? static_cast<int>(std::max<uint64_t>(64, round_up(C, 64))) : 256);
    // Workgroups per rank that can all be resident at once with kernel `fn`. A grid planned at
    // the occupancy limit itself (every compute unit full) was once seen not to become resident
    // as a whole (a rank-local join timed out), so one workgroup per compute unit is left free
    // whenever the kernel fits more than one.
    auto co_resident = [&](ar_kernel_fn fn) {
      const int occ_api = occupancy(fn, L.threads);
      const int occ = occ_api > 1 ? occ_api - 1 : occ_api;
      int m;
      if (h->placement == AR_PLACE_XCD)
        m = cus_per_xcd * occ * L.xcds_per_rank / L.ranks_per_xcd;
      else if (h->placement == AR_PLACE_SAME)
        m = cus_per_xcd * occ / N;
      else
        m = h->cu_count * occ / N;
      return std::min(m, ar::kMaxCtasPerRank);
    };
    auto pick_ctas = [&](int max_ctas) {
      if (h->ctas) return h->ctas;
      const uint64_t want = std::max<uint64_t>(1, ceil_div(C, static_cast<uint64_t>(L.threads)));
      return static_cast<int>(std::min<uint64_t>(want, static_cast<uint64_t>(max_ctas)));
    };
    int max_ctas = co_resident(L.fn);
    int ctas = pick_ctas(max_ctas);
    // All-gather and broadcast take their one-pass kernels only on the near slots: on the
    // regular slots the loop kernels measured faster (8 ranks, bf16: all-gather of 128 KiB per
    // rank 6.3 against 7.6 µs, broadcast of 256 KiB 3.0 against 7.9 µs).
    const bool loop_only = !near && (algo == AR_ALLGATHER || algo == AR_BROADCAST);
    if (ub == 8) {
      // Narrow units only while the rank's workgroups still get a compute unit each: beyond
      // that the doubled lane count measured slower than 16-byte units (128 KiB and more per
      // rank at N = 4).
      if (static_cast<uint64_t>(ctas) * L.threads < C || ctas > rank_cus || loop_only)
        return kNoNarrow;
    }
    // int32 two-shot: the all-gather carries sums, and a sum may equal the sentinel (INT32_MIN
    // is a legal int32 sum), so int32 always takes the bulk kernel, whose completion flags do not
    // look at the data.
    // The fp32 / bf16 two-shot on regular slots (the message does not fit the near pages) with
    // up to 8 ranks, or with more and over 1 MiB per rank (beyond the two-page near slots), takes
    // the bulk kernel too: its all-gather goes straight into the outputs. Measured (p50, bulk
    // against the one-pass sentinel kernel): 8 ranks bf16 1 MiB 9.6 against 11.8 µs, 2 MiB 14.9
    // against 22.6; 4 ranks bf16 1 MiB 6.1 against 7.1; 16 ranks fp32 and bf16 2 MiB 31.0 against
    // 37.9; at 16 ranks fp32 1 MiB on regular slots the one-pass kernel stays ahead (18.1 against
    // 20.5 µs).
    const bool prefer_bulk = algo == AR_TWOSHOT && !near && (N <= 8 || nbytes > (1u << 20)) &&
                             h->ctas == 0 && h->threads == 0;
    const bool flag_protocol = algo == AR_TWOSHOT && (h->dtype == AR_INT32 || prefer_bulk);
    if (flag_protocol && ub == 8) return kNoNarrow;
    if (static_cast<uint64_t>(ctas) * L.threads < C || loop_only || flag_protocol) {
      // The chunk does not fit one pass of the rank's lanes: the kernels built for one pass (the
      // latency path) hand it to their multi-pass counterparts.
      const int multi = algo == AR_TWOSHOT             ? ar::ALGO_TWOSHOT_BULK
                        : algo == AR_ONESHOT_LL        ? ar::ALGO_ONESHOT_LL_MULTI
                        : algo == AR_ONESHOT_SENTINEL  ? ar::ALGO_ONESHOT_SENTINEL_MULTI
                        : algo == AR_REDUCESCATTER     ? ar::ALGO_REDUCESCATTER
                        : algo == AR_ALLGATHER         ? ar::ALGO_ALLGATHER
                        : algo == AR_BROADCAST         ? ar::ALGO_BROADCAST
                                                       : 0;
      if (multi != 0) {
        L.kernel_algo = multi;
        L.fn = ar_select_kernel(multi, h->dtype, nmax);
        if (h->threads == 0) L.threads = 256;
        max_ctas = co_resident(L.fn);
        ctas = pick_ctas(max_ctas);
        // (the int32 two-shot takes this kernel at every size; a chunk that one workgroup per
        // compute unit covers in one pass keeps the plain count of workgroups)
        const bool one_pass_bulk =
            flag_protocol && C <= static_cast<uint64_t>(rank_cus) * static_cast<uint64_t>(L.threads);
        if (h->ctas == 0 && max_ctas >= rank_cus && !one_pass_bulk) {
          // Every lane of the rank makes the same number of passes, and every compute unit of
          // the rank holds the same number of workgroups: among whole multiples of the rank's
          // compute units, the one with the least padded work (passes x lanes). A rank only
          // moves on to its next AllReduce once its slowest wave is done, so a last pass that
          // only some lanes take costs a whole pass (16 MiB per rank at N = 8: 6 % slower with 3
          // workgroups per compute unit and 5.3 passes than with 2 and 8). On a tie the narrower
          // shape wins once it makes at least 8 passes (one workgroup per compute unit measured
          // 0.5-2 % faster than two at 16-256 MiB); below that, the wider one (fewer passes),
          // except for the loop kernels of the standalone collectives, where the narrower one
          // measured faster at every size (8 ranks, bf16 broadcast of 256 KiB: 3.0 against
          // 5.0 µs with two workgroups per compute unit).
          const bool narrow_ties = multi == ar::ALGO_REDUCESCATTER ||
                                   multi == ar::ALGO_ALLGATHER || multi == ar::ALGO_BROADCAST;
          const uint64_t T = static_cast<uint64_t>(L.threads);
          uint64_t best_work = ~0ull, best_passes = 0;
          for (int m = 1; m * rank_cus <= max_ctas; ++m) {
            const uint64_t w = static_cast<uint64_t>(m) * rank_cus;
            const uint64_t passes = ceil_div(C, w * T);
            const uint64_t work = passes * w;
            if (work < best_work || (work == best_work && !narrow_ties && best_passes < 8)) {
              best_work = work;
              best_passes = passes;
              ctas = static_cast<int>(w);
            }
          }
        }
      }
    }
    if (max_ctas < 1) return ar_fail(AR_ENORES, "%d ranks cannot be co-resident", N);
    if (ctas > max_ctas)
      return ar_fail(AR_ENORES, "%d workgroups per rank exceed the co-resident limit %d", ctas,
                     max_ctas);
    L.ctas = ctas;
    if (algo == AR_LL128_DET && static_cast<uint64_t>(ctas) * L.threads < C)
      return ar_fail(AR_ENORES, "the deterministic variant needs a lane per unit of a chunk");
    // With 5..16 ranks the one-pass sentinel kernels split each 64 units' peers over the waves
    // of a workgroup (the peer-split kernels) while those workgroups still get a compute unit
    // each and the launch shape is not forced. Measured (p50, split against unsplit): 8 ranks,
    // bf16 two-shot 16-128 KiB 6-7 % lower; 16 ranks, fp32 one-shot 4-8 KiB 14-16 % lower;
    // with two or more such workgroups per compute unit 30 % to 3x higher; with 4 ranks (three
    // peers, one per wave) 3-5 % higher at 1-8 KiB.
    const bool splittable = L.kernel_algo == ar::ALGO_ONESHOT_SENTINEL ||
                            L.kernel_algo == ar::ALGO_ONESHOT_SENTINEL_NARROW ||
                            L.kernel_algo == ar::ALGO_TWOSHOT ||
                            L.kernel_algo == ar::ALGO_TWOSHOT_NARROW ||
                            L.kernel_algo == ar::ALGO_ONESHOT_LL;
    // The LL128-style kernel (fp32, bf16) splits the same way: blocks of at most 64 units, one
    // workgroup each (1, 2 or 4 word slices per lane as the block needs), and at least two
    // blocks. Measured at 16 ranks, fp32 (p50 against one 64-unit block per workgroup): two
    // workgroups for 4-16 KiB 2-6 % lower; four or more 5 % to 2x higher (the owners'
    // destination lines then take more, smaller atomic requests).
    if (algo == AR_LL128_ATOMIC && h->dtype != AR_INT32 && h->split && N > 4 && h->ctas == 0 &&
        h->threads == 0 && C > 0) {
      const uint64_t blk = std::min<uint64_t>(ar::kWave, std::max<uint64_t>(1, ceil_div(C, 2)));
      const uint64_t wgs = ceil_div(C, blk);
      const int id = blk <= 16 ? ar::ALGO_LL128_SPLIT_E1
                     : blk <= 32 ? ar::ALGO_LL128_SPLIT_E2
                                 : ar::ALGO_LL128_SPLIT;
      ar_kernel_fn fs = ar_select_kernel(id, h->dtype, nmax);
      if (fs != nullptr && wgs <= static_cast<uint64_t>(rank_cus)) {
        const int saved = L.threads;
        L.threads = ar::kSplitWaves * ar::kWave;
        if (wgs <= static_cast<uint64_t>(co_resident(fs))) {
          L.fn = fs;
          L.kernel_algo = id;
          L.ctas = static_cast<int>(wgs);
          L.block = static_cast<int>(blk);
          return AR_OK;
        }
        L.threads = saved;
      }
    }
    if (splittable && h->split && N > 4 && h->ctas == 0 && h->threads == 0 && C > 0) {
      const bool two = L.kernel_algo == ar::ALGO_TWOSHOT || L.kernel_algo == ar::ALGO_TWOSHOT_NARROW;
      const int id = L.kernel_algo == ar::ALGO_ONESHOT_LL ? ar::ALGO_ONESHOT_LL_SPLIT
                     : two ? (ub == 8 ? ar::ALGO_TWOSHOT_SPLIT_NARROW : ar::ALGO_TWOSHOT_SPLIT)
                           : (ub == 8 ? ar::ALGO_ONESHOT_SPLIT_NARROW : ar::ALGO_ONESHOT_SPLIT);
      ar_kernel_fn fs = ar_select_kernel(id, h->dtype, nmax);
      const uint64_t wgs = ceil_div(C, static_cast<uint64_t>(ar::kWave));
      if (fs != nullptr && wgs <= static_cast<uint64_t>(rank_cus)) {
        const int saved = L.threads;
        L.threads = ar::kSplitWaves * ar::kWave;
        if (wgs <= static_cast<uint64_t>(co_resident(fs))) {
          L.fn = fs;
          L.kernel_algo = id;
          L.ctas = static_cast<int>(wgs);
        } else {
          L.threads = saved;
        }
      }
    }
    // LL128-style kernels whose whole chunk fits one wave with 16 or 32 units issue only the
    // word slices that hold data
    if ((algo == AR_LL128_ATOMIC || algo == AR_LL128_DET) && ctas == 1 && L.threads == 64 &&
        C <= 32) {
      const bool det = algo == AR_LL128_DET;
      const int e = C <= 16 ? (det ? ar::ALGO_LL128_DET_E1 : ar::ALGO_LL128_E1)
                            : (det ? ar::ALGO_LL128_DET_E2 : ar::ALGO_LL128_E2);
      ar_kernel_fn fe = ar_select_kernel(e, h->dtype, nmax);
      if (fe != nullptr && occupancy(fe, L.threads) >= 1) {
        L.fn = fe;
        L.kernel_algo = e;
      }
    }
    return AR_OK;
  };
  int rc = shape(near_fits);
  // The multi-pass two-shot kernels (the bulk AllReduce, the loop kernels of the standalone
  // collectives) address regular slots only: they take the regular chunking.
  // Two-page regions are laid out for the one-pass two-shot kernel with 16-byte units and the
  // one-pass one-shot LL kernel only, each with an instance of its own for them (the others keep
  // their addressing unchanged).
  if (rc == AR_OK && L.near &&
      (L.kernel_algo == ar::ALGO_TWOSHOT_BULK || L.kernel_algo == ar::ALGO_REDUCESCATTER ||
       L.kernel_algo == ar::ALGO_ALLGATHER || L.kernel_algo == ar::ALGO_BROADCAST ||
       (two_page && L.kernel_algo != ar::ALGO_TWOSHOT && L.kernel_algo != AR_ONESHOT_LL &&
        L.kernel_algo != AR_ONESHOT_SENTINEL)))
    rc = shape(false);
  if (rc == AR_OK && L.near && two_page) {
    const int tp = L.kernel_algo == ar::ALGO_TWOSHOT    ? ar::ALGO_TWOSHOT_TWO_PAGE
                   : L.kernel_algo == AR_ONESHOT_LL     ? ar::ALGO_ONESHOT_LL_TWO_PAGE
                                                        : ar::ALGO_ONESHOT_SENTINEL_TWO_PAGE;
    ar_kernel_fn fp = ar_select_kernel(tp, h->dtype, nmax);
    // the plan's workgroups must stay co-resident with the two-page instance (its own register
    // count), with the same one-workgroup headroom per compute unit as co_resident (XCD
    // placement)
    const int occ_api = fp != nullptr ? occupancy(fp, L.threads) : 0;
    const int occ = occ_api > 1 ? occ_api - 1 : occ_api;
    const int fit = std::min(cus_per_xcd * occ * L.xcds_per_rank / L.ranks_per_xcd,
                             ar::kMaxCtasPerRank);
    if (fp != nullptr && occ >= 1 && L.ctas <= fit) {
      L.fn = fp;
      L.kernel_algo = tp;
      L.two_page = true;
    } else {
      rc = shape(false);
    }
  }
  // Two-half near slots for the one-shot sentinel: the rank runs on two XCDs (one in each half of
  // the chip, its workgroups alternating over them) and its slots fill the near p1 page, every
  // granule used: each workgroup's units go to the granules homed in its own XCD's half
  // (slot_off, region_base). Taken when the message does not fit the near slots of one XCD, and
  // when one XCD would hold more than one wave per compute unit. Measured at 4 ranks, bf16 (p50,
  // two halves against the best other plan): 32 KiB 1.21 against 1.34 us, 64 KiB 1.46 against
  // 1.50, 128 KiB 1.64 against 2.05, 256 KiB 2.21 against 4.2; 1-16 KiB 3-9 % higher (kept on
  // one XCD).
  auto two_halves = [&]() -> bool {
    if (!(h->near_ok && h->two_halves && h->placement == AR_PLACE_XCD &&
          algo == AR_ONESHOT_SENTINEL && L.xcds_per_rank == 2 && L.chunks == 1 &&
          (L.kernel_algo == ar::ALGO_ONESHOT_SENTINEL ||
           L.kernel_algo == ar::ALGO_ONESHOT_SENTINEL_NARROW)))
      return false;
    const uint64_t bw = static_cast<uint64_t>(L.threads) * ub;  // bytes per workgroup
    const uint64_t per_granule = ar::kGranule / bw;  // whole workgroup blocks per granule
    // workgroups 0, 2, 4, ... run on the first XCD: ceil(ctas / 2) blocks per half
    const uint64_t slot =
        ceil_div(ceil_div(static_cast<uint64_t>(L.ctas), 2), per_granule) * 2 * ar::kGranule;
    if (2ull * N * slot > ar::kNearPage) return false;
    uint64_t home = 0;
    for (int r = 0; r < N; ++r) {
      // The granule of a pitch homed near the half of the rank's first XCD: the one whose four
      // calibrated positions poll faster from both XCD pairs of that half; the pairs of the other
      // half must prefer the other granule (else the page is left to the regular plan).
      const float(*ns)[ar::kNearPositions] = h->near_ns[r][1];
      auto lead = [&](int half) {  // > 0: the second granule is faster from this half
        float d = 0.f;
        for (int p = 2 * half; p < 2 * half + 2; ++p)
          for (int k = 0; k < 4; ++k) d += ns[p][k] - ns[p][4 + k];
        return d;
      };
      const int h0 = (r % kXcds) / (kXcds / 2);
      const float d0 = lead(h0), d1 = lead(1 - h0);
      if (!(d0 * d1 < 0.f)) return false;
      home |= static_cast<uint64_t>(d0 > 0.f ? 1 : 0) << (4 * r);
    }
    L.near = true;
    L.two_halves = true;
    L.near_rg[0] = h->rg[RG_LL];
    L.near_rg[2] = h->rg[RG_P2];
    ar::Region& rg = L.near_rg[1];
    rg = h->rg[RG_P1N];
    rg.near = ar::kNearTwoHalves;
    rg.slot = static_cast<uint32_t>(slot);
    rg.home_pos = home;
    // the descriptor of either half's granules ends inside the page
    rg.bytes = static_cast<uint32_t>(2ull * N * slot - ar::kGranule);
    return true;
  };
  // (with 8-byte units also when the one-XCD plan could not give every unit a lane)
  if (near_fits && algo == AR_ONESHOT_SENTINEL && h->two_halves &&
      (rc == kNoNarrow || (rc == AR_OK && static_cast<uint64_t>(L.ctas) * (L.threads / ar::kWave) >
                                              static_cast<uint64_t>(cus_per_xcd)))) {
    const Launch one_xcd = L;
    const int rc_one = rc;
    if (shape(false) == AR_OK && two_halves()) {
      rc = AR_OK;
    } else {
      L = one_xcd;
      rc = rc_one;
    }
  }
  if (rc != AR_OK) return rc;
  if (!L.near) two_halves();
  if (L.near && !L.two_halves) {
    // Each rank's slot data goes to the fastest calibrated position of each near region, for the
    // XCD pair of the XCD of its first workgroup: any 2 KiB sub-block of either granule where a
    // single chunk fits, else the start of either granule.
    const uint64_t data = units * line;
    const int max_sub = near_chunks == 1 ? static_cast<int>((ar::kGranule - data) / ar::kNearSub) : 0;
    for (int g = 0; g < ar::kNearRegions; ++g) {
      ar::Region& rg = L.near_rg[g];
      rg = h->rg[RG_LLN + g];
      // the plan's two-page regions: ll for the one-shot LL, p1 and p2 for the two-shot
      const bool tp_g = L.two_page && (L.kernel_algo == ar::ALGO_ONESHOT_LL_TWO_PAGE     ? g == 0
                                       : L.kernel_algo == ar::ALGO_ONESHOT_SENTINEL_TWO_PAGE ? g == 1
                                                                                              : g > 0);
      rg.slot = static_cast<uint32_t>(near_chunks * 2 * ar::kGranule);
      for (int r = 0; r < N; ++r) {
        const int x = h->placement == AR_PLACE_XCD    ? r % kXcds
                      : h->placement == AR_PLACE_SAME ? 0
                                                      : (r * L.ctas) % kXcds;
        const float* ns = h->near_ns[r][g][x / 2];
        int best = 0;
        for (int k = 0; k < ar::kNearPositions; ++k)
          if (k % 4 <= max_sub && ns[k] < ns[best]) best = k;
        rg.home_pos |= static_cast<uint64_t>(best) << (4 * r);
        // Two-page region: buffer 1 in the second page, one granule before it when that page
        // polls faster at the other granule of the pitch (its homes mirror the first page's)
        // and at its start otherwise (N slots of one buffer fill at most the page, so either
        // start keeps buffer 1 inside the region; the granules the two buffers share at the
        // page boundary hold data of different granule classes).
        if (tp_g) {
          const float* second = h->near_ns2[r][g][x / 2];
          if (second[best ^ 4] < second[best]) rg.home_pos |= 8ull << (4 * r);
        }
      }
      if (tp_g) rg.bstride = static_cast<uint32_t>(ar::kNearPage);
    }
  }
  if (h->placement == AR_PLACE_XCD)
    L.grid = static_cast<unsigned>(kXcds * L.ranks_per_xcd *
                                   ceil_div(static_cast<uint64_t>(L.ctas), L.xcds_per_rank));
  else if (h->placement == AR_PLACE_SAME)
    L.grid = static_cast<unsigned>(kXcds * N * L.ctas);
  else
    L.grid = static_cast<unsigned>(N * L.ctas);
  return AR_OK;
}

// Chunk geometry and launch shape for one AllReduce of `nbytes` bytes per rank. The one-pass
// sentinel kernels (one-shot and two-shot) move 8-byte units when the chunk still fits one pass
// of co-resident lanes and the launch shape is not forced; 16-byte units otherwise.
int plan(ar_handle* h, int algo, uint64_t nbytes, Launch& L) {
  if ((algo == AR_ONESHOT_SENTINEL || algo == AR_TWOSHOT || algo == AR_REDUCESCATTER ||
       algo == AR_ALLGATHER || algo == AR_BROADCAST) &&
      h->narrow && h->ctas == 0 &&
      h->threads == 0 && nbytes > 0) {
    Launch narrow;
    const int rc = plan_units(h, algo, nbytes, 8, narrow);
    if (rc == AR_OK) {
      L = narrow;
      return AR_OK;
    }
    if (rc != kNoNarrow) return rc;
  }
  return plan_units(h, algo, nbytes, 16, L);
}

ar::Args base_args(ar_handle* h, int algo, uint64_t nbytes, const Launch& L) {
  ar::Args a;
  std::memset(&a, 0, sizeof a);
  a.base = h->base;
  a.stride = h->stride;
  a.ll = L.near ? L.near_rg[0] : h->rg[RG_LL];
  a.p1 = L.near ? L.near_rg[1] : h->rg[RG_P1];
  a.p2 = L.near ? L.near_rg[2] : h->rg[RG_P2];
  a.acc = h->rg[RG_ACC];
  a.cnt = h->rg[RG_CNT];
  a.bar = h->rg[RG_BAR];
  a.bdat = h->rg[RG_BDAT];
  a.pf1 = h->rg[RG_PF1];
  a.pf2 = h->rg[RG_PF2];
  a.flg = h->rg[RG_FLG];
  a.sink = h->rg[RG_SINK];
  a.ctl = h->ctl;
  a.status = h->status_dev;
  a.launch_rec = h->record_launch
                     ? reinterpret_cast<uint32_t*>(h->base + h->rg[RG_REC].off)
                     : nullptr;
  a.e0 = h->epoch;
  const double ticks = static_cast<double>(h->timeout_us) * h->clock_hz * 1e-6;
  a.timeout_ticks = ticks < 1.0 ? 1ull : static_cast<uint64_t>(ticks);
  a.nbytes = static_cast<uint32_t>(nbytes);
  a.out_nbytes = static_cast<uint32_t>(nbytes);
  a.root = 0;
  a.chunk_units = L.chunk_units;
  a.part_units = L.part_units;
  a.nranks = h->nranks;
  a.ctas = L.ctas;
  a.ranks_per_xcd = L.ranks_per_xcd;
  a.xcds_per_rank = L.xcds_per_rank;
  a.placement = h->placement;
  a.iters = 1;
  a.chunks = L.chunks;
  a.nsets = 1;
  a.withhold = h->withhold;
  a.drift = 0;
  a.algo = algo;
  a.group = h->group;
  a.block = L.block;
  a.ag_direct = 1;
  return a;
}

// Automatic choice by data type, rank count and message size (the pages select by size and
// rank count; the Pith review's "kernel_selection_thresholds", Fig. 12): the fastest of
// one-shot LL (L), one-shot sentinel (S), two-shot (T) and, for int32, the LL128-style atomic
// kernel (A) measured on MI355X (`python bench.py --auto-sweep`: p50 of 100 back-to-back calls,
// fp32 uniform, bf16 normal, int32 on [-2^20, 2^20]) for N in {2,3,4,8,16} and 128 B .. 2 MiB
// per rank; a cell changed its kernel only when another led by 3 % or more in the latest of
// six sweeps (the sixth on the current kernels). A call uses the row of the
// smallest measured N >= its N and the column of the smallest measured size >= its size; above
// 2 MiB, the last column. For fp32 and bf16 only the fixed-order kernels are candidates, so that
// AUTO stays bit-reproducible; the int32 atomic sum is exact in any order. (int32 two-shot runs
// the completion-flag kernel at every size, hence its late crossover.)
constexpr int kAutoN[5] = {2, 3, 4, 8, 16};
constexpr uint64_t kAutoBytes[8] = {128, 512, 2048, 8192, 32768, 131072, 524288, 2097152};
constexpr char kAutoTable[3][5][9] = {
    {
        // fp32
        "SSLSLSST",  // N = 2
        "SSSSSSTT",  // N = 3
        "SSLSSSTT",  // N = 4
        "SSSSSTTT",  // N = 8
        "SSSSTTTT",  // N = 16
    },
    {
        // bf16
        "SSLLLSST",  // N = 2
        "SSSSSSTT",  // N = 3
        "SSLSSSTT",  // N = 4
        "SSSSSTTT",  // N = 8
        "SSSSTTTT",  // N = 16
    },
    {
        // int32
        "SSLLLSST",  // N = 2
        "SSSSSSTT",  // N = 3
        "SSLSSSTT",  // N = 4
        "SSSSSSTT",  // N = 8
        "SSSSSAAT",  // N = 16
    },
};

int resolve_algo(ar_handle* h, int algo, uint64_t nbytes) {
  // int32 additions are exact and associative: the plain atomic variant is already deterministic
  if (algo == AR_LL128_DET && h->dtype == AR_INT32) return AR_LL128_ATOMIC;
  if (algo != AR_ALGO_AUTO) return algo;
  if (h->nranks == 1) return AR_ONESHOT_SENTINEL;
  int row = 0;
  while (row < 4 && kAutoN[row] < h->nranks) ++row;
  int col = 0;
  while (col < 7 && kAutoBytes[col] < nbytes) ++col;
  const int t = h->dtype == AR_BFLOAT16 ? 1 : h->dtype == AR_INT32 ? 2 : 0;
  switch (kAutoTable[t][row][col]) {
    case 'L': return AR_ONESHOT_LL;
    case 'S': return AR_ONESHOT_SENTINEL;
    case 'A': return AR_LL128_ATOMIC;
    default: return AR_TWOSHOT;
  }
}

// Algorithms ar_allreduce accepts.
bool is_allreduce_algo(int algo) {
  return (algo >= AR_ALGO_AUTO && algo <= AR_BARRIER2) || algo == AR_LL128_DET;
}

bool overlap(const void* a, const void* b, uint64_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

bool overlap2(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool is_collective(int algo) {
  return algo == AR_REDUCESCATTER || algo == AR_ALLGATHER || algo == AR_BROADCAST;
}

// Input and output bytes per rank of one call (count as the entry point takes it: output
// elements per rank for reduce-scatter, input elements per rank for all-gather, elements for
// broadcast and AllReduce), checked against the handle.
int op_bytes(ar_handle* h, int algo, size_t count, uint64_t& in_b, uint64_t& out_b) {
  const uint64_t es = static_cast<uint64_t>(elem_bytes(h->dtype));
  const uint64_t N = static_cast<uint64_t>(h->nranks);
  const uint64_t x = static_cast<uint64_t>(count) * es;
  if (count != 0 && (x / count != es || x > (1ull << 40))) return ar_fail(AR_ETOOBIG, "count overflows");
  in_b = algo == AR_REDUCESCATTER ? x * N : x;
  out_b = algo == AR_ALLGATHER ? x * N : x;
  if ((algo == AR_REDUCESCATTER || algo == AR_ALLGATHER) && x % 16 != 0)
    return ar_fail(AR_EINVAL, "a partition of %llu bytes is not a multiple of 16 bytes",
                   static_cast<unsigned long long>(x));
  if (std::max(in_b, out_b) > h->max_bytes)
    return ar_fail(AR_ETOOBIG, "%llu bytes per rank exceed max_bytes %zu",
                   static_cast<unsigned long long>(std::max(in_b, out_b)), h->max_bytes);
  return AR_OK;
}

bool narrow_kernel(int kernel_algo) {
  return kernel_algo == ar::ALGO_ONESHOT_SENTINEL_NARROW ||
         kernel_algo == ar::ALGO_TWOSHOT_NARROW || kernel_algo == ar::ALGO_RS_NARROW ||
         kernel_algo == ar::ALGO_AG_NARROW || kernel_algo == ar::ALGO_BCAST_NARROW ||
         kernel_algo == ar::ALGO_ONESHOT_SPLIT_NARROW ||
         kernel_algo == ar::ALGO_TWOSHOT_SPLIT_NARROW;
}

// Kernel arguments of a standalone collective that differ from AllReduce's: the partitions are
// exact (in the launched kernel's unit size), not padded to whole chunks.
void collective_args(int algo, int kernel_algo, uint64_t in_b, uint64_t out_b, int N, int root,
                     ar::Args& a) {
  const uint64_t ub = narrow_kernel(kernel_algo) ? 8 : 16;
  a.nbytes = static_cast<uint32_t>(in_b);
  a.out_nbytes = static_cast<uint32_t>(out_b);
  if (algo == AR_REDUCESCATTER) a.part_units = static_cast<uint32_t>(in_b / N / ub);
  if (algo == AR_ALLGATHER) a.part_units = static_cast<uint32_t>(in_b / ub);
  a.root = root;
}

int check_status(ar_handle* h) {
  if (h->poisoned) return ar_fail(AR_ETIMEOUT, "handle is poisoned by an earlier poll timeout");
  const uint32_t code = __atomic_load_n(&h->status_host[ar::ST_CODE], __ATOMIC_ACQUIRE);
  if (code != 0) {
    h->poisoned = true;
    const uint64_t step = (static_cast<uint64_t>(h->status_host[ar::ST_STEP_HI]) << 32) |
                          h->status_host[ar::ST_STEP_LO];
    return ar_fail(AR_ETIMEOUT,
                   "poll timed out on the device: rank %u waiting for peer %d at step %llu "
                   "(algorithm %u)",
                   h->status_host[ar::ST_RANK], static_cast<int>(h->status_host[ar::ST_PEER]),
                   static_cast<unsigned long long>(step), h->status_host[ar::ST_ALGO]);
  }
  return AR_OK;
}

// AR_OPT_CHECK_INPUTS: before a launch, look for inputs equal to the sentinel (the caller's
// obligation under the sentinel protocol, Every µs Matters §IV "Sentinel"). Synchronous on
// `stream`; AR_EINVAL names the first offending rank and element. `in` holds N pointers of
// `nbytes` bytes each; with root >= 0 only in[root] is checked.
int check_inputs(ar_handle* h, const void* const in[], uint64_t nbytes, int root,
                 hipStream_t stream) {
  if (nbytes == 0) return AR_OK;
  AR_HIP(hipMemsetAsync(h->ctl + ar::CTL_CHECK_HITS, 0, 4, stream));
  AR_HIP(hipMemsetAsync(h->ctl + ar::CTL_CHECK_FIRST, 0xFF, 8, stream));
  const void* tab[ar::kMaxRanks];
  const int n = root >= 0 ? 1 : h->nranks;
  for (int r = 0; r < n; ++r) tab[r] = in[root >= 0 ? root : r];
  AR_HIP(static_cast<hipError_t>(ar_launch_check(tab, n, static_cast<uint32_t>(nbytes), h->dtype,
                                                 h->ctl, stream)));
  uint32_t w[4] = {0, 0, 0, 0};
  AR_HIP(hipMemcpyAsync(w, h->ctl + ar::CTL_CHECK_HITS, sizeof w, hipMemcpyDeviceToHost, stream));
  AR_HIP(hipStreamSynchronize(stream));
  if (w[0] != 0) {
    const uint64_t first = (static_cast<uint64_t>(w[2]) << 32) | w[1];
    const int rank = root >= 0 ? root : static_cast<int>(first >> 40);
    return ar_fail(AR_EINVAL,
                   "%u input element(s) equal the sentinel; the first is element %llu of rank %d",
                   w[0], static_cast<unsigned long long>(first & ((1ull << 40) - 1)), rank);
  }
  return AR_OK;
}

// A cooperative launch (AR_OPT_COOPERATIVE) has the runtime refuse a grid that it cannot make
// resident at once, instead of starting part of it; the kernels use no grid-wide sync.
int launch(ar_kernel_fn fn, unsigned grid, int threads, ar::Args& a, hipStream_t stream,
           bool cooperative) {
  void* args[] = {&a};
  const void* f = reinterpret_cast<const void*>(fn);
  if (cooperative) {
    const hipError_t e = hipLaunchCooperativeKernel(f, dim3(grid), dim3(threads), args, 0, stream);
    if (e == hipErrorCooperativeLaunchTooLarge)
      return ar_fail(AR_ENORES, "the runtime cannot make %u workgroups of %d threads resident",
                     grid, threads);
    AR_HIP(e);
    return AR_OK;
  }
  AR_HIP(hipLaunchKernel(f, dim3(grid), dim3(threads), args, 0, stream));
  return AR_OK;
}

void release(ar_handle* h) {
  if (h->raw) (void)hipFree(h->raw);
  if (h->ctl) (void)hipFree(h->ctl);
  if (h->status_host) (void)hipHostFree(h->status_host);
  if (h->tab) (void)hipFree(h->tab);
  if (h->ts) (void)hipFree(h->ts);
  if (h->ev0) (void)hipEventDestroy(h->ev0);
  if (h->ev1) (void)hipEventDestroy(h->ev1);
  delete h;
}

// Argument checks, plan and launch of one AllReduce on handle h (ar_allreduce and the
// allocation-free entry point). A handle without host status words (status_host == nullptr)
// skips the status check.
int allreduce_enqueue(ar_handle* h, const void* const in[], void* const out[], size_t count,
                      ar_algo algo, hipStream_t s) {
  if (h == nullptr) return ar_fail(AR_EINVAL, "null handle");
  if (in == nullptr || out == nullptr) return ar_fail(AR_EINVAL, "null pointer table");
  if (!is_allreduce_algo(algo))
    return ar_fail(AR_EINVAL, "algorithm %d is not valid for ar_allreduce", static_cast<int>(algo));
  int rc = h->status_host != nullptr ? check_status(h) : AR_OK;
  if (rc != AR_OK) return rc;
  const int N = h->nranks;
  const uint64_t nbytes = static_cast<uint64_t>(count) * elem_bytes(h->dtype);
  if (count != 0 && nbytes / count != static_cast<uint64_t>(elem_bytes(h->dtype)))
    return ar_fail(AR_ETOOBIG, "count overflows");
  if (nbytes > h->max_bytes)
    return ar_fail(AR_ETOOBIG, "%llu bytes per rank exceed max_bytes %zu",
                   static_cast<unsigned long long>(nbytes), h->max_bytes);
  for (int r = 0; r < N; ++r) {
    if (in[r] == nullptr || out[r] == nullptr)
      return ar_fail(AR_EINVAL, "null buffer for rank %d", r);
    if ((reinterpret_cast<uintptr_t>(in[r]) | reinterpret_cast<uintptr_t>(out[r])) & 15u)
      return ar_fail(AR_EINVAL, "buffers of rank %d are not 16-byte aligned", r);
  }
  if (nbytes > 0) {
    for (int r = 0; r < N; ++r)
      for (int q = 0; q < N; ++q) {
        if (q != r && overlap(out[r], out[q], nbytes))
          return ar_fail(AR_EINVAL, "outputs of ranks %d and %d overlap", r, q);
        if (overlap(out[r], in[q], nbytes) && !(q == r && out[r] == in[r]))
          return ar_fail(AR_EINVAL, "output of rank %d overlaps input of rank %d", r, q);
      }
  }
  if (nbytes == 0) {
    h->epoch += 1;
    return AR_OK;
  }
  const int alg = resolve_algo(h, algo, nbytes);
  Launch L;
  rc = plan(h, alg, nbytes, L);
  if (rc != AR_OK) return rc;
  if (h->check_inputs && (rc = check_inputs(h, in, nbytes, -1, s)) != AR_OK) return rc;
  ar::Args a = base_args(h, alg, nbytes, L);
  for (int r = 0; r < N; ++r) {
    a.in[r] = in[r];
    a.out[r] = out[r];
  }
  rc = launch(L.fn, L.grid, L.threads, a, s, h->cooperative != 0);
  if (rc != AR_OK) return rc;
  h->epoch += static_cast<uint64_t>(L.chunks);
  h->last_stream = s;
  return AR_OK;
}

}  // namespace

extern "C" {

const char* ar_last_error(void) { return g_err; }

double ar_wallclock_hz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0.0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0.0;
  return static_cast<double>(khz) * 1e3;
}

ar_handle* ar_create(int nranks, size_t max_bytes, ar_dtype dtype) {
  g_err[0] = '\0';
  if (nranks < 1 || nranks > ar::kMaxRanks) {
    ar_fail(AR_EINVAL, "nranks must be in [1, %d], got %d", ar::kMaxRanks, nranks);
    return nullptr;
  }
  if (max_bytes < 1 || max_bytes > 0x7FFFFFFFull) {
    ar_fail(AR_EINVAL, "max_bytes must be in [1, 2^31 - 1], got %zu", max_bytes);
    return nullptr;
  }
  if (dtype != AR_FLOAT32 && dtype != AR_BFLOAT16 && dtype != AR_INT32) {
    ar_fail(AR_EINVAL, "unknown dtype %d", static_cast<int>(dtype));
    return nullptr;
  }
  ar_handle* h = new ar_handle();
  h->nranks = nranks;
  h->dtype = dtype;
  h->max_bytes = max_bytes;
  const int N = nranks;
  const uint64_t cap_os = std::min(env_u64("AR_SCRATCH_ONESHOT", kDefaultCapOneShot), kMaxCap);
  const uint64_t cap_ts = std::min(env_u64("AR_SCRATCH_TWOSHOT", kDefaultCapTwoShot), kMaxCap);
  h->timeout_us = static_cast<int64_t>(env_u64("AR_POLL_TIMEOUT_US", 2000000));
  auto fail = [&](hipError_t e, const char* what) {
    ar_fail_hip(e, what);
    release(h);
    return static_cast<ar_handle*>(nullptr);
  };
  hipError_t e;
  if ((e = hipGetDevice(&h->device)) != hipSuccess) return fail(e, "hipGetDevice");
  if ((e = hipDeviceGetAttribute(&h->cu_count, hipDeviceAttributeMultiprocessorCount,
                                 h->device)) != hipSuccess)
    return fail(e, "hipDeviceGetAttribute");
  h->clock_hz = ar_wallclock_hz();
  if (h->clock_hz <= 0.0) h->clock_hz = 100e6;

  // Two-page p1 and p2 near regions when more than 8 ranks may run two-shot messages whose
  // slots (2 N of one partition each) do not fit one page: the one-pass two-shot then keeps its
  // slots near up to N partition slots per page (16 ranks, fp32, 1 MiB: 13.5 against 17.6 us on
  // the regular slots; at 8 ranks the bulk two-shot stays faster, 9.3 against 10.1 us).
  // The one-shot LL likewise gets a two-page ll region when its slots (16-byte lines of 8 bytes of
  // payload) need it (16 ranks, fp32, 32 KiB: see plan_units).
  {
    // (near slots hold a whole partition or message: the scratch caps only chunk the regular
    // slots)
    auto needs_two = [&](uint64_t slot_bytes) {
      return N > 8 && 2ull * N * ceil_div(slot_bytes, ar::kGranule) * 2 * ar::kGranule >
                          ar::kNearPage;
    };
    const uint64_t part = ceil_div(ceil_div(max_bytes, 16), N) * 16;
    h->two_page[0] = needs_two(2 * round_up(max_bytes, 8));
    h->two_page[1] = h->two_page[2] = needs_two(part);
    // the one-shot sentinel's p1 slots (a whole message each) from 8 ranks on
    if (N >= 8 && 2ull * N * ceil_div(round_up(max_bytes, 16), ar::kGranule) * 2 * ar::kGranule >
                      ar::kNearPage)
      h->two_page[1] = true;
  }
  if (layout(N, max_bytes, cap_os, cap_ts, true, h->two_page, true, h->rg, &h->stride) != AR_OK) {
    release(h);
    return nullptr;
  }
  const uint64_t total = h->stride * N;
  if ((e = hipMalloc(&h->raw, total + ar::kNearPage)) != hipSuccess)
    return fail(e, "hipMalloc(scratch)");
  h->base = reinterpret_cast<uint8_t*>(round_up(reinterpret_cast<uintptr_t>(h->raw), ar::kNearPage));
  if ((e = hipMemset(h->base, 0, total)) != hipSuccess) return fail(e, "hipMemset(scratch)");
  {
    uint64_t first[ar::kNearRegions], second[ar::kNearRegions];
    for (int g = 0; g < ar::kNearRegions; ++g) {
      first[g] = h->rg[RG_LLN + g].off;
      // (a region of one page calibrates its first page twice: never read)
      second[g] = first[g] + (h->two_page[g] ? ar::kNearPage : 0);
    }
    const bool any = h->two_page[0] || h->two_page[1] || h->two_page[2];
    if (ar_near_positions(h->base, h->stride, N, first, ar::kNearRegions, &h->near_ns[0][0][0][0]) !=
            AR_OK ||
        (any && ar_near_positions(h->base, h->stride, N, second, ar::kNearRegions,
                                  &h->near_ns2[0][0][0][0]) != AR_OK)) {
      release(h);
      return nullptr;
    }
  }
  const uint32_t sw = sentinel_word(dtype);
  for (int i : {RG_P1, RG_P2, RG_P1N, RG_P2N})
    ar_launch_fill(h->base, h->stride, N, h->rg[i].off, h->rg[i].bytes, sw, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return fail(e, "scratch fill launch");
  if ((e = hipMalloc(reinterpret_cast<void**>(&h->ctl), ar::CTL_WORDS * 4)) != hipSuccess)
    return fail(e, "hipMalloc(ctl)");
  if ((e = hipMemset(h->ctl, 0, ar::CTL_WORDS * 4)) != hipSuccess) return fail(e, "hipMemset(ctl)");
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->status_host), ar::ST_WORDS * 4,
                         hipHostMallocMapped)) != hipSuccess)
    return fail(e, "hipHostMalloc(status)");
  std::memset(h->status_host, 0, ar::ST_WORDS * 4);
  if ((e = hipHostGetDevicePointer(reinterpret_cast<void**>(&h->status_dev), h->status_host, 0)) !=
      hipSuccess)
    return fail(e, "hipHostGetDevicePointer(status)");
  if ((e = hipEventCreate(&h->ev0)) != hipSuccess) return fail(e, "hipEventCreate");
  if ((e = hipEventCreate(&h->ev1)) != hipSuccess) return fail(e, "hipEventCreate");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail(e, "hipDeviceSynchronize");
  h->epoch = 1;
  return h;
}

void ar_destroy(ar_handle* h) {
  if (h == nullptr) return;
  if (h->last_stream) (void)hipStreamSynchronize(h->last_stream);
  (void)hipDeviceSynchronize();
  release(h);
}

int ar_set_option(ar_handle* h, ar_option opt, int64_t v) {
  if (h == nullptr) return ar_fail(AR_EINVAL, "null handle");
  switch (opt) {
    case AR_OPT_TIMEOUT_US:
      if (v < 1 || v > 3600ll * 1000000ll) return ar_fail(AR_EINVAL, "timeout out of range");
      h->timeout_us = v;
      return AR_OK;
    case AR_OPT_WITHHOLD_RANK:
      if (v < -1 || v >= h->nranks) return ar_fail(AR_EINVAL, "withhold rank out of range");
      h->withhold = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_CTAS:
      if (v < 0 || v > ar::kMaxCtasPerRank) return ar_fail(AR_EINVAL, "ctas out of range");
      h->ctas = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_THREADS:
      if (v != 0 && v != 64 && v != 128 && v != 256)
        return ar_fail(AR_EINVAL, "threads must be 0, 64, 128 or 256");
      h->threads = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_PLACEMENT:
      if (v < AR_PLACE_XCD || v > AR_PLACE_LINEAR) return ar_fail(AR_EINVAL, "bad placement");
      h->placement = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_DRIFT:
      if (v < 0 || v > 1000) return ar_fail(AR_EINVAL, "drift out of range");
      h->drift = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_NARROW:
      if (v != 0 && v != 1) return ar_fail(AR_EINVAL, "narrow must be 0 or 1");
      h->narrow = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_ROOT:
      if (v < 0 || v >= h->nranks) return ar_fail(AR_EINVAL, "root out of range");
      h->root = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_CHECK_INPUTS:
      if (v != 0 && v != 1) return ar_fail(AR_EINVAL, "check_inputs must be 0 or 1");
      h->check_inputs = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_RECORD_LAUNCH:
      if (v != 0 && v != 1) return ar_fail(AR_EINVAL, "record_launch must be 0 or 1");
      h->record_launch = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_GROUP:
      if (v < 2 || v > ar::kMaxRanks) return ar_fail(AR_EINVAL, "group must be in [2, 16]");
      h->group = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_SPLIT:
      if (v != 0 && v != 1) return ar_fail(AR_EINVAL, "split must be 0 or 1");
      h->split = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_COOPERATIVE:
      if (v != 0 && v != 1) return ar_fail(AR_EINVAL, "cooperative must be 0 or 1");
      h->cooperative = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_TWO_HALVES:
      if (v != 0 && v != 1) return ar_fail(AR_EINVAL, "two_halves must be 0 or 1");
      h->two_halves = static_cast<int>(v);
      return AR_OK;
    case AR_OPT_TWO_PAGE:
      if (v != 0 && v != 1) return ar_fail(AR_EINVAL, "two_page must be 0 or 1");
      h->use_two_page = static_cast<int>(v);
      return AR_OK;
  }
  return ar_fail(AR_EINVAL, "unknown option %d", static_cast<int>(opt));
}

uint64_t ar_epoch(ar_handle* h) { return h ? h->epoch : 0; }

int ar_allreduce(ar_handle* h, const void* const in[], void* const out[], size_t count,
                 ar_algo algo, void* stream) {
  return allreduce_enqueue(h, in, out, count, algo, reinterpret_cast<hipStream_t>(stream));
}

namespace {

// Shared body of ar_reducescatter, ar_allgather and ar_broadcast (`in` has N entries; only
// in[root] is read for broadcast).
int run_collective(ar_handle* h, int algo, const void* const in[], void* const out[],
                   size_t count, int root, void* stream) {
  if (h == nullptr) return ar_fail(AR_EINVAL, "null handle");
  if (in == nullptr || out == nullptr) return ar_fail(AR_EINVAL, "null pointer table");
  const int N = h->nranks;
  if (algo == AR_BROADCAST && (root < 0 || root >= N))
    return ar_fail(AR_EINVAL, "root %d out of range", root);
  int rc = check_status(h);
  if (rc != AR_OK) return rc;
  uint64_t in_b = 0, out_b = 0;
  rc = op_bytes(h, algo, count, in_b, out_b);
  if (rc != AR_OK) return rc;
  for (int r = 0; r < N; ++r) {
    const bool reads = algo != AR_BROADCAST || r == root;
    if ((reads && in[r] == nullptr) || out[r] == nullptr)
      return ar_fail(AR_EINVAL, "null buffer for rank %d", r);
    if (((reads ? reinterpret_cast<uintptr_t>(in[r]) : 0) | reinterpret_cast<uintptr_t>(out[r])) & 15u)
      return ar_fail(AR_EINVAL, "buffers of rank %d are not 16-byte aligned", r);
  }
  if (count > 0) {
    // in place only in the usual forms: a reduce-scatter output at its own partition of the
    // input, an all-gather input at its own partition of the output, the broadcast root's output
    // on its input
    const uint64_t x = algo == AR_REDUCESCATTER ? out_b : in_b;
    for (int r = 0; r < N; ++r)
      for (int q = 0; q < N; ++q) {
        if (q != r && overlap(out[r], out[q], out_b))
          return ar_fail(AR_EINVAL, "outputs of ranks %d and %d overlap", r, q);
        if (algo == AR_BROADCAST && q != root) continue;
        const bool in_place =
            q == r && (algo == AR_REDUCESCATTER
                           ? static_cast<const uint8_t*>(out[r]) ==
                                 static_cast<const uint8_t*>(in[r]) + r * x
                       : algo == AR_ALLGATHER
                           ? static_cast<const uint8_t*>(in[r]) ==
                                 static_cast<const uint8_t*>(out[r]) + r * x
                           : out[r] == in[r]);
        if (overlap2(out[r], out_b, in[q], in_b) && !in_place)
          return ar_fail(AR_EINVAL, "output of rank %d overlaps input of rank %d", r, q);
      }
  }
  if (count == 0) {
    h->epoch += 1;
    return AR_OK;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Launch L;
  rc = plan(h, algo, in_b, L);
  if (rc != AR_OK) return rc;
  if (h->check_inputs &&
      (rc = check_inputs(h, in, in_b, algo == AR_BROADCAST ? root : -1, s)) != AR_OK)
    return rc;
  ar::Args a = base_args(h, algo, in_b, L);
  collective_args(algo, L.kernel_algo, in_b, out_b, N, root, a);
  for (int r = 0; r < N; ++r) {
    // broadcast: ranks other than the root never load their input; they get the root's pointer
    // (a valid descriptor base) instead of one the caller may have left null
    a.in[r] = algo == AR_BROADCAST ? in[root] : in[r];
    a.out[r] = out[r];
  }
  rc = launch(L.fn, L.grid, L.threads, a, s, h->cooperative != 0);
  if (rc != AR_OK) return rc;
  h->epoch += static_cast<uint64_t>(L.chunks);
  h->last_stream = s;
  return AR_OK;
}

}  // namespace

int ar_reducescatter(ar_handle* h, const void* const in[], void* const out[], size_t recvcount,
                     void* stream) {
  return run_collective(h, AR_REDUCESCATTER, in, out, recvcount, 0, stream);
}

int ar_allgather(ar_handle* h, const void* const in[], void* const out[], size_t sendcount,
                 void* stream) {
  return run_collective(h, AR_ALLGATHER, in, out, sendcount, 0, stream);
}

int ar_broadcast(ar_handle* h, const void* in, void* const out[], size_t count, int root,
                 void* stream) {
  if (h == nullptr) return ar_fail(AR_EINVAL, "null handle");
  std::vector<const void*> tab(static_cast<size_t>(h->nranks), in);
  return run_collective(h, AR_BROADCAST, tab.data(), out, count, root, stream);
}

int ar_check(ar_handle* h) {
  if (h == nullptr) return ar_fail(AR_EINVAL, "null handle");
  hipError_t e = h->last_stream ? hipStreamSynchronize(h->last_stream) : hipDeviceSynchronize();
  if (e != hipSuccess) return ar_fail_hip(e, "synchronize");
  return check_status(h);
}

int ar_bench(ar_handle* h, const void* const* in_sets, void* const* out_sets, int nsets,
             size_t count, ar_algo algo, int iters, uint64_t* t_start, uint64_t* t_end,
             void* stream) {
  return ar_bench_ex(h, in_sets, out_sets, nsets, count, algo, iters, t_start, t_end, nullptr,
                     stream);
}

int ar_bench_ex(ar_handle* h, const void* const* in_sets, void* const* out_sets, int nsets,
                size_t count, ar_algo algo, int iters, uint64_t* t_start, uint64_t* t_end,
                double* elapsed_ms, void* stream) {
  if (h == nullptr) return ar_fail(AR_EINVAL, "null handle");
  if (iters < 1 || iters > 1000000) return ar_fail(AR_EINVAL, "iters must be in [1, 1e6]");
  if (!is_allreduce_algo(algo) && algo != AR_BARRIER_ONLY && !is_collective(algo))
    return ar_fail(AR_EINVAL, "unknown algorithm %d", static_cast<int>(algo));
  int rc = check_status(h);
  if (rc != AR_OK) return rc;
  const int N = h->nranks;
  const bool barrier_only = algo == AR_BARRIER_ONLY;
  uint64_t nbytes = 0, out_bytes = 0;
  if (!barrier_only) {
    if (in_sets == nullptr || out_sets == nullptr) return ar_fail(AR_EINVAL, "null set tables");
    if (nsets < 1 || nsets > 65536) return ar_fail(AR_EINVAL, "nsets must be in [1, 65536]");
    if (count == 0) return ar_fail(AR_EINVAL, "ar_bench needs count > 0");
    rc = op_bytes(h, algo, count, nbytes, out_bytes);
    if (rc != AR_OK) return rc;
    for (int i = 0; i < nsets * N; ++i) {
      if (in_sets[i] == nullptr || out_sets[i] == nullptr)
        return ar_fail(AR_EINVAL, "null buffer in set table");
      if ((reinterpret_cast<uintptr_t>(in_sets[i]) | reinterpret_cast<uintptr_t>(out_sets[i])) & 15u)
        return ar_fail(AR_EINVAL, "set buffers must be 16-byte aligned");
    }
  } else {
    nsets = 1;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int alg = resolve_algo(h, algo, nbytes);
  Launch L;
  rc = plan(h, alg, nbytes, L);
  if (rc != AR_OK) return rc;
  ar::Args a = base_args(h, alg, nbytes, L);
  if (is_collective(alg)) collective_args(alg, L.kernel_algo, nbytes, out_bytes, N, h->root, a);
  a.iters = iters;
  a.drift = h->drift;
  a.nsets = nsets;
  // The owners of the bulk two-shot and of the flag all-gather of the LL128-style kernel store
  // into every rank's output during the launch. When a later iteration could read those bytes
  // as input (an output set overlapping any input set), they take the all-gather slots instead,
  // so that every rank writes only its own output.
  if (iters > 1 && !barrier_only) {
    std::vector<uintptr_t> lo_in(N, UINTPTR_MAX), hi_in(N, 0), lo_out(N, UINTPTR_MAX), hi_out(N, 0);
    for (int j = 0; j < nsets; ++j)
      for (int r = 0; r < N; ++r) {
        const uintptr_t pi = reinterpret_cast<uintptr_t>(in_sets[j * N + r]);
        const uintptr_t po = reinterpret_cast<uintptr_t>(out_sets[j * N + r]);
        lo_in[r] = std::min(lo_in[r], pi);
        hi_in[r] = std::max(hi_in[r], pi + nbytes);
        lo_out[r] = std::min(lo_out[r], po);
        hi_out[r] = std::max(hi_out[r], po + out_bytes);
      }
    for (int r1 = 0; r1 < N && a.ag_direct; ++r1)
      for (int r2 = 0; r2 < N; ++r2)
        if (lo_in[r1] < hi_out[r2] && lo_out[r2] < hi_in[r1]) {
          a.ag_direct = 0;
          break;
        }
  }
  // Evenly spaced sets (set j of rank r at set 0's address + j * stride) need no table.
  bool affine = !barrier_only && nsets > 1;
  int64_t sin = 0, sout = 0;
  if (affine) {
    sin = reinterpret_cast<intptr_t>(in_sets[N]) - reinterpret_cast<intptr_t>(in_sets[0]);
    sout = reinterpret_cast<intptr_t>(out_sets[N]) - reinterpret_cast<intptr_t>(out_sets[0]);
    for (int j = 0; j < nsets && affine; ++j)
      for (int r = 0; r < N && affine; ++r) {
        affine = reinterpret_cast<intptr_t>(in_sets[j * N + r]) ==
                     reinterpret_cast<intptr_t>(in_sets[r]) + j * sin &&
                 reinterpret_cast<intptr_t>(out_sets[j * N + r]) ==
                     reinterpret_cast<intptr_t>(out_sets[r]) + j * sout;
      }
    if (sin == 0 && sout == 0) affine = false;
  }
  if (!barrier_only && (affine || nsets == 1)) {
    for (int r = 0; r < N; ++r) {
      a.in[r] = in_sets[r];
      a.out[r] = out_sets[r];
    }
    a.in_set_stride = affine ? sin : 0;
    a.out_set_stride = affine ? sout : 0;
  } else if (!barrier_only) {
    const size_t need = 2ull * nsets * N;
    if (h->tab_cap < need) {
      if (h->tab) (void)hipFree(h->tab);
      h->tab = nullptr;
      h->tab_cap = 0;
      AR_HIP(hipMalloc(reinterpret_cast<void**>(&h->tab), need * sizeof(void*)));
      h->tab_cap = need;
    }
    std::vector<const void*> host_tab(need);
    for (size_t i = 0; i < static_cast<size_t>(nsets) * N; ++i) {
      host_tab[i] = in_sets[i];
      host_tab[static_cast<size_t>(nsets) * N + i] = out_sets[i];
    }
    AR_HIP(hipMemcpy(h->tab, host_tab.data(), need * sizeof(void*), hipMemcpyHostToDevice));
    a.in_tab = const_cast<const void* const*>(h->tab);
    a.out_tab = h->tab + static_cast<size_t>(nsets) * N;
  }
  const int wpb = L.threads / ar::kWave;
  const size_t per = static_cast<size_t>(iters) * N * L.ctas * wpb;
  const bool want_ts = t_start != nullptr || t_end != nullptr;
  if (want_ts) {
    if (h->ts_cap < 2 * per) {
      if (h->ts) (void)hipFree(h->ts);
      h->ts = nullptr;
      h->ts_cap = 0;
      AR_HIP(hipMalloc(reinterpret_cast<void**>(&h->ts), 2 * per * sizeof(uint64_t)));
      h->ts_cap = 2 * per;
    }
    a.ts_start = h->ts;
    a.ts_end = h->ts + per;
  }
  AR_HIP(hipEventRecord(h->ev0, s));
  rc = launch(L.fn, L.grid, L.threads, a, s, h->cooperative != 0);
  if (rc != AR_OK) return rc;
  AR_HIP(hipEventRecord(h->ev1, s));
  h->epoch += static_cast<uint64_t>(iters) * L.chunks;
  h->last_stream = s;
  AR_HIP(hipStreamSynchronize(s));
  rc = check_status(h);
  if (rc != AR_OK) return rc;
  if (elapsed_ms != nullptr) {
    float ms = 0.f;
    AR_HIP(hipEventElapsedTime(&ms, h->ev0, h->ev1));
    *elapsed_ms = ms;
  }
  if (want_ts) {
    std::vector<uint64_t> ts(2 * per);
    AR_HIP(hipMemcpy(ts.data(), h->ts, 2 * per * sizeof(uint64_t), hipMemcpyDeviceToHost));
    const size_t group = static_cast<size_t>(L.ctas) * wpb;
    for (size_t g = 0; g < static_cast<size_t>(iters) * N; ++g) {
      uint64_t lo = UINT64_MAX, hi = 0;
      for (size_t j = 0; j < group; ++j) {
        lo = std::min(lo, ts[g * group + j]);
        hi = std::max(hi, ts[per + g * group + j]);
      }
      if (t_start) t_start[g] = lo;
      if (t_end) t_end[g] = hi;
    }
  }
  return AR_OK;
}

int ar_plan_info(ar_handle* h, size_t count, ar_algo algo, ar_plan* info) {
  if (h == nullptr || info == nullptr) return ar_fail(AR_EINVAL, "null argument");
  if (!is_allreduce_algo(algo) && !is_collective(algo))
    return ar_fail(AR_EINVAL, "algorithm %d is not valid", static_cast<int>(algo));
  uint64_t in_b = 0, out_b = 0;
  int rc = op_bytes(h, algo, count, in_b, out_b);
  if (rc != AR_OK) return rc;
  if (in_b == 0) return ar_fail(AR_EINVAL, "count 0 launches nothing");
  const int alg = resolve_algo(h, algo, in_b);
  Launch L;
  rc = plan(h, alg, in_b, L);
  if (rc != AR_OK) return rc;
  info->kernel = L.kernel_algo;
  info->chunks = L.chunks;
  info->ctas = L.ctas;
  info->threads = L.threads;
  info->grid = static_cast<int>(L.grid);
  info->unit_bytes = (L.kernel_algo == AR_ONESHOT_LL ||
                      L.kernel_algo == ar::ALGO_ONESHOT_LL_MULTI ||
                      L.kernel_algo == ar::ALGO_ONESHOT_LL_SPLIT ||
                      L.kernel_algo == ar::ALGO_ONESHOT_LL_TWO_PAGE || narrow_kernel(L.kernel_algo))
                         ? 8
                         : 16;
  info->near = L.two_page ? 3 : L.two_halves ? 2 : L.near ? 1 : 0;
  info->resident_per_cu = occupancy(L.fn, L.threads);
  info->cu_count = h->cu_count;
  return AR_OK;
}

int64_t ar_alg_bytes(ar_handle* h, size_t count, ar_algo algo) {
  if (h == nullptr) return ar_fail(AR_EINVAL, "null handle");
  if (is_collective(algo)) {
    // Every logical read and write once. Per rank of a reduce-scatter (x = output bytes): its
    // N input partitions, N-1 pushes, N-1 slot reads and re-arms, x out. Per rank of an
    // all-gather (x = input bytes): x in, N-1 pushes, N x out, N-1 slot reads and re-arms. A
    // broadcast of x: the root reads x, pushes N-1 and writes x; each other rank reads, writes
    // out and re-arms x. All three are (N+1) x + 3 (N-1) x, per rank for the first two.
    uint64_t in_b = 0, out_b = 0;
    const int rc = op_bytes(h, algo, count, in_b, out_b);
    if (rc != AR_OK) return rc;
    const uint64_t N = static_cast<uint64_t>(h->nranks);
    const uint64_t x = algo == AR_REDUCESCATTER ? out_b : in_b;
    const uint64_t one = (N + 1) * x + 3 * (N - 1) * x;
    return static_cast<int64_t>(algo == AR_BROADCAST ? one : N * one);
  }
  if (!is_allreduce_algo(algo))
    return ar_fail(AR_EINVAL, "algorithm %d is not valid", static_cast<int>(algo));
  const uint64_t S = static_cast<uint64_t>(count) * elem_bytes(h->dtype);
  if (S > h->max_bytes) return ar_fail(AR_ETOOBIG, "message exceeds max_bytes");
  if (S == 0) return 0;
  const int alg = resolve_algo(h, algo, S);
  Launch L;
  const int rc = plan(h, alg, S, L);
  if (rc != AR_OK) return rc;
  const uint64_t N = static_cast<uint64_t>(h->nranks);
  // every logical read and write once: inputs, pushes, slot reads, re-arms, outputs
  switch (L.kernel_algo) {
    case AR_ONESHOT_LL:
    case ar::ALGO_ONESHOT_LL_SPLIT:
    case ar::ALGO_ONESHOT_LL_TWO_PAGE:
    case ar::ALGO_ONESHOT_LL_MULTI: return static_cast<int64_t>(2 * N * S + 4 * N * (N - 1) * S);
    case AR_ONESHOT_SENTINEL:
    case ar::ALGO_ONESHOT_SENTINEL_TWO_PAGE:
    case ar::ALGO_ONESHOT_SENTINEL_MULTI:
    case ar::ALGO_ONESHOT_SENTINEL_NARROW:
    case ar::ALGO_ONESHOT_SPLIT:
    case ar::ALGO_ONESHOT_SPLIT_NARROW:
      return static_cast<int64_t>(2 * N * S + 3 * N * (N - 1) * S);
    case AR_TWOSHOT:
    case ar::ALGO_TWOSHOT_SPLIT:
    case ar::ALGO_TWOSHOT_SPLIT_NARROW:
    case ar::ALGO_TWOSHOT_NARROW:
    case ar::ALGO_TWOSHOT_TWO_PAGE: return static_cast<int64_t>((N + 1) * S + 7 * (N - 1) * S);
    // owners store their reduced partition straight into every output (no all-gather slots)
    case ar::ALGO_TWOSHOT_BULK: return static_cast<int64_t>(2 * N * S + 2 * (N - 1) * S);
    // inputs N S, contributions N S, the owners read, clear and keep their sums 3 S, the
    // all-gather stored straight into the other outputs (N - 1) S
    case AR_LL128_ATOMIC:
    case ar::ALGO_LL128_E1:
    case ar::ALGO_LL128_E2: return static_cast<int64_t>(2 * N * S + 3 * S + (N - 1) * S);
    // the peer-split kernel's all-gather goes through sentinel slots: 4 (N - 1) S
    case ar::ALGO_LL128_SPLIT:
    case ar::ALGO_LL128_SPLIT_E1:
    case ar::ALGO_LL128_SPLIT_E2: return static_cast<int64_t>(2 * N * S + 3 * S + 4 * (N - 1) * S);
    case AR_LL128_DET:
    case ar::ALGO_LL128_DET_E1:
    case ar::ALGO_LL128_DET_E2: {
      // inputs N S; contributions N S (binary32: twice that for bf16); the owners read and clear
      // G group sums, 2 G S (binary32); own partition out S; all-gather into the outputs (N - 1) S
      const uint64_t w = h->dtype == AR_BFLOAT16 ? 2 : 1;
      const uint64_t G = (N + static_cast<uint64_t>(h->group) - 1) / static_cast<uint64_t>(h->group);
      return static_cast<int64_t>(N * S + w * N * S + 2 * w * G * S + S + (N - 1) * S);
    }
    case AR_BARRIER2: return static_cast<int64_t>(2 * N * S + 2 * N * (N - 1) * S);
    default: return 0;
  }
}

int64_t ar_region_bytes(ar_handle* h, int region) {
  if (h == nullptr || region < 0 || region >= kRegions) return ar_fail(AR_EINVAL, "bad region");
  return static_cast<int64_t>(h->rg[region].bytes);
}

int ar_read_region(ar_handle* h, int rank, int region, void* host_dst, size_t bytes) {
  if (h == nullptr || host_dst == nullptr) return ar_fail(AR_EINVAL, "null argument");
  if (rank < 0 || rank >= h->nranks || region < 0 || region >= kRegions)
    return ar_fail(AR_EINVAL, "bad rank or region");
  if (bytes > h->rg[region].bytes) return ar_fail(AR_EINVAL, "read past the region");
  if (region == RG_REC && rank != 0) return ar_fail(AR_EINVAL, "the launch record is in rank 0");
  if (h->last_stream) AR_HIP(hipStreamSynchronize(h->last_stream));
  AR_HIP(hipDeviceSynchronize());
  AR_HIP(hipMemcpy(host_dst, h->base + static_cast<uint64_t>(rank) * h->stride + h->rg[region].off,
                   bytes, hipMemcpyDeviceToHost));
  return AR_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free AllReduce
//
// ar_allreduce_noalloc: ar_allreduce for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation). Its symmetric
// scratch is the file-scope device array `scratch` below, one copy per GPU the library runs on;
// its handle-shaped state (region layout, sequence number) lives in static host storage. It calls
// no allocating routine: set-up is hipGetSymbolAddress once per device plus fill kernels on the
// caller's stream whenever the (rank count, dtype) the scratch is laid out for changes.

namespace {

// Scratch per rank per protocol: a quarter MiB, so that 16 rank blocks with every region fit the
// array; larger messages run in more chunks than with a handle (whose default caps are 4 MiB /
// 64 MiB).
constexpr uint64_t kNoAllocCap = 256ull << 10;
constexpr uint64_t kNoAllocCtl = 4096;  // control words (16 x u32) and status words (8 x u32)
constexpr uint64_t kNoAllocScratchBytes = 40ull << 20;
constexpr int kNoAllocDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

struct NoAllocDevice {
  uint8_t* ptr = nullptr;  // this device's copy of `scratch` (from hipGetSymbolAddress)
  int nranks = 0;          // layout the scratch holds (0: not laid out yet)
  int dtype = -1;
  ar_handle h;             // handle-shaped state over the scratch; owns nothing
};
std::mutex g_na_mu;
NoAllocDevice g_na[kNoAllocDevices];

// Lay the scratch of device `dev` out for (nranks, dtype): clear everything (LL lines, flags,
// counters, atomic destinations, control and status words) and arm the sentinel slots, on
// `stream`; the sequence number restarts at 1.
int noalloc_setup(NoAllocDevice& d, int dev, int nranks, int dtype, hipStream_t stream) {
  ar_handle& h = d.h;
  h.nranks = nranks;
  h.dtype = dtype;
  h.max_bytes = 0x7FFFFFFFull;
  h.device = dev;
  h.near_ok = false;  // the array is neither 2 MiB aligned nor calibrated: regular regions only
  h.placement = AR_PLACE_XCD;
  h.timeout_us = static_cast<int64_t>(env_u64("AR_POLL_TIMEOUT_US", 2000000));
  AR_HIP(hipDeviceGetAttribute(&h.cu_count, hipDeviceAttributeMultiprocessorCount, dev));
  h.clock_hz = ar_wallclock_hz();
  if (h.clock_hz <= 0.0) h.clock_hz = 100e6;
  int rc = layout(nranks, h.max_bytes, kNoAllocCap, kNoAllocCap, false, nullptr, false, h.rg,
                  &h.stride);
  if (rc != AR_OK) return rc;
  const uint64_t total = kNoAllocCtl + h.stride * static_cast<uint64_t>(nranks);
  if (total > kNoAllocScratchBytes)
    return ar_fail(AR_ETOOBIG, "%d ranks need %llu bytes of scratch, the array holds %llu", nranks,
                   static_cast<unsigned long long>(total),
                   static_cast<unsigned long long>(kNoAllocScratchBytes));
  h.ctl = reinterpret_cast<uint32_t*>(d.ptr);
  h.status_host = nullptr;  // no host-mapped status: timeouts stay in the status words below
  h.status_dev = reinterpret_cast<uint32_t*>(d.ptr + 64);
  h.base = d.ptr + kNoAllocCtl;
  ar_launch_fill(d.ptr, 0, 1, 0, static_cast<uint32_t>(total), 0u, stream);
  const uint32_t sw = sentinel_word(dtype);
  for (int i : {RG_P1, RG_P2})
    ar_launch_fill(h.base, h.stride, nranks, h.rg[i].off, h.rg[i].bytes, sw, stream);
  AR_HIP(hipGetLastError());
  h.epoch = 1;
  d.nranks = nranks;
  d.dtype = dtype;
  return AR_OK;
}

}  // namespace

extern "C" int ar_allreduce_noalloc(int nranks, ar_dtype dtype, const void* const in[],
                                    void* const out[], size_t count, ar_algo algo,
                                    void* stream) {
  if (nranks < 1 || nranks > ar::kMaxRanks)
    return ar_fail(AR_EINVAL, "nranks must be in [1, %d], got %d", ar::kMaxRanks, nranks);
  if (dtype != AR_FLOAT32 && dtype != AR_BFLOAT16 && dtype != AR_INT32)
    return ar_fail(AR_EINVAL, "unknown dtype %d", static_cast<int>(dtype));
  int dev = 0;
  AR_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kNoAllocDevices)
    return ar_fail(AR_EINVAL, "device %d beyond the %d the library keeps state for", dev,
                   kNoAllocDevices);
  std::lock_guard<std::mutex> lk(g_na_mu);
  NoAllocDevice& d = g_na[dev];
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d.ptr == nullptr) {
    // once per device, with that device current: the device address of this GPU's copy of the
    // array (the array's name in host code is only a host-side stand-in)
    void* p = nullptr;
    AR_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    d.ptr = static_cast<uint8_t*>(p);
  }
  if (d.nranks != nranks || d.dtype != static_cast<int>(dtype)) {
    const int rc = noalloc_setup(d, dev, nranks, dtype, s);
    if (rc != AR_OK) {
      d.nranks = 0;
      return rc;
    }
  }
  return allreduce_enqueue(&d.h, in, out, count, algo, s);
}
