// Kernel argument block and scratch geometry shared by the host runtime and the kernels.
#pragma once

#include <stdint.h>

namespace ar {

constexpr int kMaxRanks = 16;
constexpr int kMaxCtasPerRank = 256;
constexpr int kMaxWavesPerCta = 4;  // blocks of at most 256 threads
constexpr int kWave = 64;
constexpr int kSplitWaves = 4;  // waves per workgroup of the peer-split kernels (one per peer group)

// Algorithms (values match ar_algo in include/ar.h).
enum Algo : int {
  ALGO_ONESHOT_LL = 1,
  ALGO_ONESHOT_SENTINEL = 2,
  ALGO_TWOSHOT = 3,
  ALGO_LL128_ATOMIC = 4,
  ALGO_BARRIER2 = 5,
  ALGO_BARRIER_ONLY = 6,
  // internal: kernels for chunks wider than one pass of the rank's workgroups
  ALGO_TWOSHOT_BULK = 7,
  ALGO_ONESHOT_LL_MULTI = 8,
  ALGO_ONESHOT_SENTINEL_MULTI = 9,
  // internal: one-pass sentinel kernels with 8-byte units (two lanes per 16 bytes)
  ALGO_ONESHOT_SENTINEL_NARROW = 10,
  ALGO_TWOSHOT_NARROW = 11,
  // the standalone collectives built from the same primitives
  ALGO_REDUCESCATTER = 12,
  ALGO_ALLGATHER = 13,
  ALGO_BROADCAST = 14,
  // internal: reduce-scatter / all-gather as one half of the one-pass two-shot, 16- or 8-byte
  // units (12 and 13 are then their loop kernels for chunks wider than one pass)
  ALGO_RS_ONEPASS = 15,
  ALGO_AG_ONEPASS = 16,
  ALGO_RS_NARROW = 17,
  ALGO_AG_NARROW = 18,
  // internal: one-pass broadcast, 16- or 8-byte units (14 is then its loop kernel)
  ALGO_BCAST_ONEPASS = 19,
  ALGO_BCAST_NARROW = 20,
  // the deterministic LL128-style variant (groups added in a fixed order)
  ALGO_LL128_DET = 21,
  // internal: LL128-style kernels for a chunk of at most 16 (E1) or 32 (E2) units in one wave
  ALGO_LL128_E1 = 22,
  ALGO_LL128_E2 = 23,
  ALGO_LL128_DET_E1 = 24,
  ALGO_LL128_DET_E2 = 25,
  // peer-split one-pass kernels (several waves share a chunk's units, each with a few peers):
  // one-shot sentinel with 16- / 8-byte units, two-shot with 16- / 8-byte units
  ALGO_ONESHOT_SPLIT = 26,
  ALGO_ONESHOT_SPLIT_NARROW = 27,
  ALGO_TWOSHOT_SPLIT = 28,
  ALGO_TWOSHOT_SPLIT_NARROW = 29,
  // peer-split LL128-style kernels (fp32, bf16): 4 / 1 / 2 word slices per lane
  ALGO_LL128_SPLIT = 30,
  ALGO_LL128_SPLIT_E1 = 31,
  ALGO_LL128_SPLIT_E2 = 32,
  // peer-split one-shot LL (16-byte lines of 8 bytes of payload)
  ALGO_ONESHOT_LL_SPLIT = 33,
  // the one-pass two-shot on two-page near slots (more than 8 ranks)
  ALGO_TWOSHOT_TWO_PAGE = 34,
  // the one-pass one-shot LL on a two-page near ll region (more than 8 ranks)
  ALGO_ONESHOT_LL_TWO_PAGE = 35,
  // the one-pass one-shot sentinel on a two-page near p1 region (8 and more ranks)
  ALGO_ONESHOT_SENTINEL_TWO_PAGE = 36,
};

// How workgroups map to emulated ranks (values match ar_placement in include/ar.h).
enum Placement : int {
  PLACE_XCD = 0,     // rank r's first workgroup on XCD r % 8 (workgroups are dispatched
                     // round-robin over XCDs); a rank spans 8 / N XCDs when N divides 8
  PLACE_SAME = 1,    // every rank on XCD 0
  PLACE_LINEAR = 2,  // rank = workgroup / ctas (each rank spread over all XCDs)
};

// One protocol region inside every rank's block of the symmetric scratch allocation.
struct Region {
  uint64_t off;       // byte offset of the region inside a rank block
  uint32_t bytes;     // region bytes per rank
  uint32_t slot;      // bytes of one (buffer, source) slot (its pitch), or of one buffer for `acc`
  uint64_t home_pos;  // near region: bits 4r..4r+2 = position of rank r's data in each pitch;
                      // bit 4r+3 (two-page region): rank r's second page is mirrored
  uint32_t near;      // 1: a near region (slot data in 8 KiB chunks, one per 16 KiB of pitch);
                      // kNearTwoHalves: a two-half near region (slot_off)
  uint32_t bstride;   // two-page near region (planned for the two-page instances of the
                      // one-pass two-shot and one-shot LL only): the page size, buffer 1 in
                      // the second page (region_base); else 0
};

// Memory homes (measured on MI355X): the device's memory is interleaved over the two halves of
// the chip (XCDs 0-3 and 4-7) in 8 KiB granules, alternating inside every 2 MiB page. A store
// from one XCD becomes visible to a poll from another XCD of the same half in ~370 ns when the
// line lives in a granule of that half, ~600 ns when it lives in the other half. A near region
// is one 2 MiB page per rank block; its slots lay their data out in 8 KiB chunks, one chunk per
// 16 KiB of pitch (one granule of each class), always in the granule homed near the receiving
// rank. A two-page near region (ll, p1 and p2 of handles with more than 8 ranks, for messages
// whose slots need more than one page) holds double buffer b in page b. The second page's homes are
// calibrated too: when they are the mirror image of the first page's (as consecutive pages of a
// fresh allocation are: 2 MiB on, a granule of the other half), buffer 1 starts one granule
// before that page, so that every slot's data stays in a granule of the same class.
constexpr uint32_t kGranule = 8192;
constexpr uint32_t kChunkUnits = kGranule / 16;  // 16-byte units per chunk
constexpr uint64_t kNearPage = 2ull << 20;       // one near region of a rank block
constexpr int kNearRegions = 3;                  // LL, p1, p2
// Within the pitch a rank's slot data may start at any of 8 positions (2 KiB sub-blocks of the two
// granules; the sub-blocks of one granule differ by a few tens of ns as well).
constexpr int kNearPositions = 8;
constexpr uint32_t kNearSub = 2048;
constexpr uint32_t kNearTwoHalves = 2;  // Region::near of a two-half near region

// Control words (device memory). The host-visible status copy lives in pinned host memory.
enum Ctl : int {
  CTL_ABORT = 0,   // set to 1 by the first wave that times out; polls give up when they see it,
                   // and a kernel that finds it set at entry exits without touching anything
  CTL_CHECK_HITS = 1,  // input check (AR_OPT_CHECK_INPUTS): inputs found equal to the sentinel
  CTL_CHECK_FIRST = 2, // u64 at words 2-3: (rank << 40) | element of the first such input
  CTL_WORDS = 16,
};

// Largest grid any plan launches (AR_PLACE_SAME: 8 * 16 ranks * 256 workgroups); the launch
// record (AR_OPT_RECORD_LAUNCH) has one word per workgroup.
constexpr int kMaxGrid = 8 * kMaxRanks * kMaxCtasPerRank;
enum Status : int {
  ST_CODE = 0,     // 0 ok, 1 poll timed out
  ST_RANK = 1,
  ST_PEER = 2,
  ST_STEP_LO = 3,
  ST_STEP_HI = 4,
  ST_ALGO = 5,
  ST_WORDS = 8,
};

struct Args {
  const void* in[kMaxRanks];
  void* out[kMaxRanks];
  const void* const* in_tab;  // optional device table [nsets][nranks] (persistent benchmark)
  void* const* out_tab;
  int64_t in_set_stride;      // when the sets are evenly spaced: set j of rank r is
  int64_t out_set_stride;     //   in[r] + j * in_set_stride (no table; 0 = use the table)
  uint8_t* base;              // symmetric scratch: rank r's block starts at base + r * stride
  uint64_t stride;
  Region p1;    // one-shot sentinel slots / two-shot reduce-scatter slots (sentinel)
  Region p2;    // two-shot all-gather slots (sentinel)
  Region ll;    // one-shot LL lines (zeroed, epoch flags)
  Region acc;   // LL128-style shared atomic destinations [buf][group][slot] (zeroed)
  Region cnt;   // LL128-style arrival counters [buf][cta][wave], then the deterministic
                // variant's tickets [buf][group][cta][wave] (zeroed)
  Region bar;   // barrier flags [src][cta] (zeroed, monotonic)
  Region bdat;  // barrier-baseline data slots [src] (single buffer, plain)
  Region pf1;   // bulk two-shot reduce-scatter slots (data only; completion flags below)
  Region pf2;   // bulk two-shot all-gather slots
  Region flg;   // bulk two-shot completion flags [phase 2][src][cta][wave] u64 (zeroed, monotonic)
  Region sink;  // 16 KiB that idle lanes' packed bf16 atomics add zero into (zeroed)
  uint32_t* ctl;        // device control words
  uint32_t* status;     // host-mapped status words (pinned host memory)
  uint64_t* ts_start;   // optional [iters][nranks][ctas][waves] timestamps
  uint64_t* ts_end;
  uint32_t* launch_rec; // optional [grid] words: XCC id | (rank + 1) << 8 | cta << 16 of every
                        // workgroup (rank + 1 = 0 for workgroups that map to no rank)
  uint64_t e0;          // sequence number of the first step of this launch
  uint64_t timeout_ticks;
  uint32_t nbytes;      // input bytes per rank
  uint32_t out_nbytes;  // output bytes per rank (equal to nbytes for AllReduce)
  uint32_t chunk_units; // units per chunk: one-shot message chunk, or two-shot partition chunk
  uint32_t part_units;  // two-shot partition size in units (a multiple of chunk_units)
  int nranks;
  int ctas;             // workgroups per rank
  int ranks_per_xcd;    // rank placement on XCDs (PLACE_XCD): ranks sharing one XCD when N > 8
  int xcds_per_rank;    //   or XCDs one rank spans when N divides 8
  int placement;
  int iters;
  int chunks;
  int nsets;
  int withhold;         // fault injection: this rank sends nothing (-1: off)
  int drift;            // rank-drift stress: up to this many sleeps per iteration (0: off)
  int algo;
  int root;             // broadcast: the rank whose input every rank receives
  int group;            // deterministic LL128-style variant: ranks per group
  int block;            // peer-split LL128-style kernel: units per workgroup (1..64)
  int ag_direct;        // bulk two-shot: owners store their reduced partition straight into
                        // every rank's output (0: through the all-gather slots)
};

}  // namespace ar
