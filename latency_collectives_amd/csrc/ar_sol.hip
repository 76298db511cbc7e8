// Speed-of-light microbenchmarks and hardware probes for the emulated-rank AllReduce.
//
// The pages bound small-message AllReduce latency by L_SoL = 2 * L_L2 + L_remote_store, with
// L_L2 taken as the latency of a device-scope memory fence and L_remote_store from a two-GPU
// store/poll ping-pong (Every µs Matters, §VI as summarised by the Pith review: "Section VI, L_SoL
// formula"; the review's concrete test proposes a dependent pointer chase for the L2 term and a
// ping-pong without fences for the store term). On one gfx950 device the "remote" store is a
// store by one workgroup that another workgroup, on the same or on another XCD, polls for.
//
// Every kernel here runs a bounded number of iterations and every wait is bounded by a spin
// limit, so a probe always ends.

#include "ar_args.h"
#include "ar_device.h"

namespace ar {

// --------------------------------------------------------------- fence latency
// One wave: `iters` times {store to a line with the coherent policy, agent-scope release fence}.
// out[0] = ticks for the whole loop.
__global__ void sol_fence(uint32_t* buf, int iters, uint64_t* out) {
  if (blockIdx.x != 0 || threadIdx.x >= kWave) return;
  const rsrc_t r = make_rsrc(buf, 4096);
  st4<kCoh>(r, threadIdx.x * 4u, 0u);
  wait_all_mem();
  const uint64_t t0 = now_ticks();
  for (int i = 0; i < iters; ++i) {
    if (threadIdx.x == 0) st4<kPlain>(r, 0, static_cast<uint32_t>(i));
    release_agent();
  }
  const uint64_t t1 = now_ticks();
  if (threadIdx.x == 0) out[0] = t1 - t0;
}

// --------------------------------------------------------------- dependent load latency
// One lane follows a pointer chain (each 32-bit word holds the byte offset of the next node)
// `hops` times with cache policy CP. A first pass over the whole chain warms the caches.
// out[0] = ticks for the timed pass, out[1] = final offset (keeps the chain live).
template <int CP>
__global__ void sol_chase(const uint32_t* chain, uint32_t bytes, int hops, int warm_hops,
                          uint64_t* out) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  const rsrc_t r = make_rsrc(chain, bytes);
  uint32_t off = 0;
  for (int i = 0; i < warm_hops; ++i) off = ld4<CP>(r, off);
  wait_all_mem();
  const uint64_t t0 = now_ticks();
  for (int i = 0; i < hops; ++i) off = ld4<CP>(r, off);
  wait_all_mem();
  compiler_fence();
  const uint64_t t1 = now_ticks();
  out[0] = t1 - t0;
  out[1] = off;
}

// --------------------------------------------------------------- store -> poll ping-pong
// Two single-wave workgroups, A = blockIdx a_blk and B = blockIdx b_blk (the other workgroups
// exit). Round i: A stores i to flag_a and polls flag_b until it reads i; B polls flag_a for i,
// then stores i to flag_b. No fences: a store with the coherent policy followed by polling loads
// with the coherent policy. out = {ticks for all rounds, completed rounds, xcc of A, xcc of B}.
template <int CPS, int CPL>
__global__ void sol_pingpong(uint32_t* flags, int rounds, int a_blk, int b_blk, uint32_t spin_cap,
                             uint64_t* out) {
  const int me = blockIdx.x;
  if ((me != a_blk && me != b_blk) || threadIdx.x != 0) return;
  const rsrc_t r = make_rsrc(flags, 1024);
  const bool is_a = me == a_blk;
  const uint32_t fa = 0, fb = 512;
  out[is_a ? 2 : 3] = xcc_id();
  uint64_t t0 = 0;
  int done = 0;
  if (is_a) t0 = now_ticks();
  for (int i = 1; i <= rounds; ++i) {
    uint32_t spins = 0;
    if (is_a) {
      st4<CPS>(r, fa, static_cast<uint32_t>(i));
      while (true) {
        const uint32_t v = ld4<CPL>(r, fb);
        compiler_fence();
        if (v == static_cast<uint32_t>(i) || ++spins > spin_cap) break;
      }
    } else {
      while (true) {
        const uint32_t v = ld4<CPL>(r, fa);
        compiler_fence();
        if (v == static_cast<uint32_t>(i) || ++spins > spin_cap) break;
      }
      st4<CPS>(r, fb, static_cast<uint32_t>(i));
    }
    if (spins > spin_cap) break;
    done = i;
  }
  if (is_a) {
    out[0] = now_ticks() - t0;
    out[1] = static_cast<uint64_t>(done);
  }
}

// --------------------------------------------------------------- near-position probe
// Workgroups a and b (on two XCDs) ping-pong `rounds` times on each of kNearPositions positions of
// one 2 MiB page: position k = granule k / 4, 2 KiB sub-block k % 4, flag words at +1024 and
// +1536 inside the sub-block (zero before the probe). out[k] = ticks of position k's rounds.
__global__ void near_probe(uint32_t* page, int rounds, int a_blk, int b_blk, uint32_t spin_cap,
                           uint64_t* out) {
  const int me = blockIdx.x;
  if ((me != a_blk && me != b_blk) || threadIdx.x != 0) return;
  const bool is_a = me == a_blk;
  for (int k = 0; k < kNearPositions; ++k) {
    const uint32_t base = (k / 4) * kGranule + (k % 4) * 2048u;
    const rsrc_t r = make_rsrc(reinterpret_cast<uint8_t*>(page) + base, 2048);
    const uint64_t t0 = now_ticks();
    int done = 0;
    for (int i = 1; i <= rounds; ++i) {
      uint32_t spins = 0;
      if (is_a) {
        st4<kCoh>(r, 1024, static_cast<uint32_t>(i));
        while (true) {
          const uint32_t v = ld4<kCoh>(r, 1536);
          compiler_fence();
          if (v == static_cast<uint32_t>(i) || ++spins > spin_cap) break;
        }
      } else {
        while (true) {
          const uint32_t v = ld4<kCoh>(r, 1024);
          compiler_fence();
          if (v == static_cast<uint32_t>(i) || ++spins > spin_cap) break;
        }
        st4<kCoh>(r, 1536, static_cast<uint32_t>(i));
      }
      if (spins > spin_cap) break;
      done = i;
    }
    if (is_a) out[k] = done == rounds ? now_ticks() - t0 : ~0ull;
  }
}

// --------------------------------------------------------------- torn 16-byte line probe
// Writer workgroup (blockIdx w_blk, one lane per line) stores generations g = 1..gens into
// `lines` 16-byte lines as {g, ~g, g * 0x9E3779B1, g ^ 0x5A5A5A5A} with one 16-byte coherent
// store each; reader workgroup (blockIdx r_blk) polls the same lines with 16-byte coherent loads
// and counts lines whose four words do not belong to one generation (a torn line). Zero-filled
// lines (never written) are valid. out = {torn, reads, xcc writer, xcc reader}.
__global__ void sol_torn(u32x4* lines, int nlines, int gens, int w_blk, int r_blk,
                         uint32_t read_cap, unsigned long long* out) {
  const int me = blockIdx.x;
  if (me != w_blk && me != r_blk) return;
  const int l = threadIdx.x;
  if (l >= nlines) return;
  const rsrc_t r = make_rsrc(lines, static_cast<uint32_t>(nlines) * 16u);
  if (me == w_blk) {
    if (l == 0) out[2] = xcc_id();
    for (int g = 1; g <= gens; ++g) {
      const uint32_t u = static_cast<uint32_t>(g);
      st16<kCoh>(r, l * 16u, u32x4{u, ~u, u * 0x9E3779B1u, u ^ 0x5A5A5A5Au});
    }
    return;
  }
  if (l == 0) out[3] = xcc_id();
  unsigned long long torn = 0, reads = 0;
  for (uint32_t k = 0; k < read_cap; ++k) {
    const u32x4 v = ld16<kCoh>(r, l * 16u);
    compiler_fence();
    ++reads;
    const bool zero = v.x == 0u && v.y == 0u && v.z == 0u && v.w == 0u;
    const bool ok = zero || (v.y == ~v.x && v.z == v.x * 0x9E3779B1u && v.w == (v.x ^ 0x5A5A5A5Au));
    if (!ok) ++torn;
    if (v.x == static_cast<uint32_t>(gens) && ok) break;
  }
  atomicAdd(&out[0], torn);
  atomicAdd(&out[1], reads);
}

// --------------------------------------------------------------- streaming copy
// Copy `bytes` (a multiple of 16, below 2^31) with non-temporal 16-byte loads and stores, two
// units per lane per round: the reference point for HBM bandwidth on the device (a plain copy
// reads and writes every byte once) and the kernel of known size that scales the HBM byte
// counters.
__global__ __launch_bounds__(512) void stream_copy(const void* src, void* dst, uint32_t bytes) {
  const rsrc_t s = make_rsrc(src, bytes), d = make_rsrc(dst, bytes);
  const uint32_t stride = gridDim.x * blockDim.x * 16u;
  uint32_t o = (blockIdx.x * blockDim.x + threadIdx.x) * 16u;
  for (; o + stride < bytes; o += 2u * stride) {
    const u32x4 a = ld16<kNt>(s, o), b = ld16<kNt>(s, o + stride);
    st16<kNt>(d, o, a);
    st16<kNt>(d, o + stride, b);
  }
  if (o < bytes) st16<kNt>(d, o, ld16<kNt>(s, o));
}

}  // namespace ar

// ================================================================ host side

#include <algorithm>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/ar.h"
#include "ar_internal.h"

namespace {

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};


typedef void (*pp_fn)(uint32_t*, int, int, int, uint32_t, uint64_t*);

template <int CPS>
pp_fn pp_by_load(int cpl) {
  switch (cpl) {
    case 0: return ar::sol_pingpong<CPS, 0>;
    case 1: return ar::sol_pingpong<CPS, 1>;
    case 2: return ar::sol_pingpong<CPS, 2>;
    case 16: return ar::sol_pingpong<CPS, 16>;
    case 17: return ar::sol_pingpong<CPS, 17>;
    default: return nullptr;
  }
}

pp_fn pp_select(int cps, int cpl) {
  switch (cps) {
    case 0: return pp_by_load<0>(cpl);
    case 1: return pp_by_load<1>(cpl);
    case 2: return pp_by_load<2>(cpl);
    case 16: return pp_by_load<16>(cpl);
    case 17: return pp_by_load<17>(cpl);
    default: return nullptr;
  }
}

// Blocks 0 and 1 land on different XCDs (round-robin dispatch); blocks 0 and 8 on the same one.
void pair_blocks(int placement, int& a, int& b) {
  a = 0;
  b = placement == AR_PLACE_SAME ? 8 : 1;
}

// Ping-pong between workgroups a and b (of 16; workgroup w runs on XCD w % 8) on the two flag
// words at `flags` and `flags` + 512 bytes (the caller zeroes them).
int run_pingpong_at(uint32_t* flags, int a, int b, int cps, int cpl, int rounds, double* half_ns,
                    int* xcc) {
  pp_fn fn = pp_select(cps, cpl);
  if (fn == nullptr) return ar_fail(AR_EINVAL, "cache policy must be 0, 1, 2, 16 or 17");
  if (rounds < 1 || rounds > 1000000) return ar_fail(AR_EINVAL, "rounds out of range");
  DevBuf out;
  AR_HIP(hipMalloc(&out.p, 4 * sizeof(uint64_t)));
  AR_HIP(hipMemset(out.p, 0, 4 * sizeof(uint64_t)));
  hipLaunchKernelGGL(fn, dim3(16), dim3(64), 0, nullptr, flags, rounds, a, b, 1000000u,
                     static_cast<uint64_t*>(out.p));
  AR_HIP(hipGetLastError());
  AR_HIP(hipDeviceSynchronize());
  uint64_t o[4];
  AR_HIP(hipMemcpy(o, out.p, sizeof o, hipMemcpyDeviceToHost));
  if (xcc) {
    xcc[0] = static_cast<int>(o[2]);
    xcc[1] = static_cast<int>(o[3]);
  }
  if (o[1] < static_cast<uint64_t>(rounds))
    return ar_fail(AR_ETIMEOUT, "ping-pong stalled after %llu of %d rounds (policies %d/%d)",
                   static_cast<unsigned long long>(o[1]), rounds, cps, cpl);
  const double hz = ar_wallclock_hz();
  *half_ns = static_cast<double>(o[0]) / hz * 1e9 / (2.0 * rounds);
  return AR_OK;
}

// 2 MiB-aligned device buffer of `bytes` bytes (the allocation is padded and aligned by hand).
struct PageBuf {
  DevBuf raw;
  uint8_t* p = nullptr;
  int alloc(uint64_t bytes) {
    AR_HIP(hipMalloc(&raw.p, bytes + ar::kNearPage));
    const uintptr_t x = reinterpret_cast<uintptr_t>(raw.p);
    p = reinterpret_cast<uint8_t*>((x + ar::kNearPage - 1) / ar::kNearPage * ar::kNearPage);
    AR_HIP(hipMemset(raw.p, 0, bytes + ar::kNearPage));
    return AR_OK;
  }
};

// Half round trips of the store -> poll ping-pong between workgroups a and b at every position
// of the near probe on a 2 MiB page (zero before and after).
int pingpong_positions(uint8_t* page, int a, int b, int rounds, float ns[ar::kNearPositions]) {
  DevBuf out;
  AR_HIP(hipMalloc(&out.p, ar::kNearPositions * sizeof(uint64_t)));
  hipLaunchKernelGGL(ar::near_probe, dim3(16), dim3(64), 0, nullptr,
                     reinterpret_cast<uint32_t*>(page), rounds, a, b, 1000000u,
                     static_cast<uint64_t*>(out.p));
  AR_HIP(hipGetLastError());
  uint64_t o[ar::kNearPositions];
  AR_HIP(hipMemcpy(o, out.p, sizeof o, hipMemcpyDeviceToHost));
  const double hz = ar_wallclock_hz();
  for (int k = 0; k < ar::kNearPositions; ++k) {
    if (o[k] == ~0ull) return ar_fail(AR_ETIMEOUT, "near-position probe stalled");
    ns[k] = static_cast<float>(static_cast<double>(o[k]) / hz * 1e9 / (2.0 * rounds));
  }
  AR_HIP(hipMemset(page, 0, 2 * ar::kGranule));
  return AR_OK;
}

int run_pingpong(int placement, int cps, int cpl, int rounds, double* half_ns, int* xcc) {
  if (pp_select(cps, cpl) == nullptr)
    return ar_fail(AR_EINVAL, "cache policy must be 0, 1, 2, 16 or 17");
  if (rounds < 1 || rounds > 1000000) return ar_fail(AR_EINVAL, "rounds out of range");
  DevBuf flags;
  AR_HIP(hipMalloc(&flags.p, 1024));
  AR_HIP(hipMemset(flags.p, 0, 1024));
  int a = 0, b = 0;
  pair_blocks(placement, a, b);
  return run_pingpong_at(static_cast<uint32_t*>(flags.p), a, b, cps, cpl, rounds, half_ns, xcc);
}

// Random cyclic pointer chain over `bytes` with one node per 128 bytes (Sattolo's shuffle gives a
// single cycle through every node); returns the average ns per dependent load with policy CP.
template <int CP>
int run_chase(uint64_t bytes, int hops, bool warm_full, double* ns) {
  const uint64_t nodes = bytes / 128;
  std::vector<uint32_t> order(nodes);
  for (uint64_t i = 0; i < nodes; ++i) order[i] = static_cast<uint32_t>(i);
  std::mt19937_64 g(12345);
  for (uint64_t i = nodes - 1; i > 0; --i) {
    std::uniform_int_distribution<uint64_t> d(0, i - 1);
    std::swap(order[i], order[d(g)]);
  }
  std::vector<uint32_t> image(bytes / 4, 0u);
  for (uint64_t i = 0; i < nodes; ++i)
    image[static_cast<uint64_t>(i) * 32] = order[i] * 128u;  // node i -> node order[i]
  DevBuf chain, out;
  AR_HIP(hipMalloc(&chain.p, bytes));
  AR_HIP(hipMalloc(&out.p, 2 * sizeof(uint64_t)));
  AR_HIP(hipMemcpy(chain.p, image.data(), bytes, hipMemcpyHostToDevice));
  const int warm = warm_full ? static_cast<int>(std::min<uint64_t>(nodes, 1u << 22)) : 1000;
  hipLaunchKernelGGL(ar::sol_chase<CP>, dim3(1), dim3(64), 0, nullptr,
                     static_cast<const uint32_t*>(chain.p), static_cast<uint32_t>(bytes), hops,
                     warm, static_cast<uint64_t*>(out.p));
  AR_HIP(hipGetLastError());
  AR_HIP(hipDeviceSynchronize());
  uint64_t o[2];
  AR_HIP(hipMemcpy(o, out.p, sizeof o, hipMemcpyDeviceToHost));
  *ns = static_cast<double>(o[0]) / ar_wallclock_hz() * 1e9 / hops;
  return AR_OK;
}

}  // namespace

int ar_near_positions(uint8_t* base, uint64_t stride, int nranks, const uint64_t* page_off,
                      int npages, float* ns) {
  // For every listed page of every rank block and every pair of XCDs {2p, 2p+1}: the half round
  // trip of the pair's ping-pong at each of the positions. The pages are zero before and after.
  for (int r = 0; r < nranks; ++r) {
    for (int g = 0; g < npages; ++g) {
      uint8_t* page = base + static_cast<uint64_t>(r) * stride + page_off[g];
      for (int p = 0; p < 4; ++p) {
        float* out = ns + ((static_cast<size_t>(r) * npages + g) * 4 + p) * ar::kNearPositions;
        const int rc = pingpong_positions(page, 2 * p, 2 * p + 1, 24, out);
        if (rc != AR_OK) return rc;
      }
    }
  }
  return AR_OK;
}

extern "C" {

int ar_pingpong(int placement, int store_policy, int load_policy, int rounds, double* half_rtt_ns,
                int* xcc) {
  if (half_rtt_ns == nullptr) return ar_fail(AR_EINVAL, "null result pointer");
  return run_pingpong(placement, store_policy, load_policy, rounds, half_rtt_ns, xcc);
}

int ar_sol(int placement, double* out_ns) {
  if (out_ns == nullptr) return ar_fail(AR_EINVAL, "null result pointer");
  ar_sol_result res;
  const int rc = ar_sol_ex(placement, &res);
  if (rc != AR_OK) return rc;
  out_ns[0] = res.fence_ns;
  out_ns[1] = res.l2_load_ns;
  out_ns[2] = res.store_half_rtt_ns;
  return AR_OK;
}

int ar_sol_ranks(int nranks, int placement, ar_sol_ranks_result* res) {
  if (res == nullptr) return ar_fail(AR_EINVAL, "null result pointer");
  if (nranks < 2 || nranks > ar::kMaxRanks)
    return ar_fail(AR_EINVAL, "nranks must be in [2, %d]", ar::kMaxRanks);
  if (placement != AR_PLACE_XCD && placement != AR_PLACE_SAME)
    return ar_fail(AR_EINVAL, "placement must be AR_PLACE_XCD or AR_PLACE_SAME");
  std::memset(res, 0, sizeof *res);
  PageBuf page;
  int rc;
  if ((rc = page.alloc(ar::kNearPage)) != AR_OK) return rc;
  // XCD of every rank's (first) workgroups, as the planner places them; workgroup w of the
  // 16-workgroup probe runs on XCD w % 8, so the same XCD twice is workgroups x and x + 8
  int xcd[ar::kMaxRanks];
  for (int r = 0; r < nranks; ++r) xcd[r] = placement == AR_PLACE_XCD ? r % 8 : 0;
  // each receiving XCD's slot position: the fastest for its partner pair {x, x ^ 1}, as the
  // planner calibrates it
  int pos[8];
  for (int x = 0; x < 8; ++x) {
    float ns[ar::kNearPositions];
    if ((rc = pingpong_positions(page.p, x & ~1, (x & ~1) + 1, 200, ns)) != AR_OK) return rc;
    pos[x] = static_cast<int>(std::min_element(ns, ns + ar::kNearPositions) - ns);
  }
  double worst = 0.0, best = 1e300;
  bool seen[8][8] = {};
  for (int r = 0; r < nranks; ++r) {
    for (int q = 0; q < nranks; ++q) {
      if (q == r || seen[xcd[q]][xcd[r]]) continue;
      seen[xcd[q]][xcd[r]] = true;
      const int a = xcd[q], b = xcd[q] == xcd[r] ? xcd[r] + 8 : xcd[r];
      float ns[ar::kNearPositions];
      if ((rc = pingpong_positions(page.p, a, b, 200, ns)) != AR_OK) return rc;
      const double v = ns[pos[xcd[r]]];
      res->pairs += 1;
      if (v > worst) {
        worst = v;
        res->worst_sender_xcc = xcd[q];
        res->worst_receiver_xcc = xcd[r];
      }
      best = std::min(best, v);
    }
  }
  res->store_half_rtt_worst_ns = worst;
  res->store_half_rtt_best_ns = best;
  return AR_OK;
}

int ar_sol_ex(int placement, ar_sol_result* res) {
  if (res == nullptr) return ar_fail(AR_EINVAL, "null result pointer");
  if (placement != AR_PLACE_XCD && placement != AR_PLACE_SAME)
    return ar_fail(AR_EINVAL, "placement must be AR_PLACE_XCD or AR_PLACE_SAME");
  std::memset(res, 0, sizeof *res);
  const double hz = ar_wallclock_hz();
  if (hz <= 0) return ar_fail(AR_EHIP, "no device wall clock");
  {
    DevBuf buf, out;
    AR_HIP(hipMalloc(&buf.p, 4096));
    AR_HIP(hipMalloc(&out.p, sizeof(uint64_t)));
    const int iters = 20000;
    hipLaunchKernelGGL(ar::sol_fence, dim3(1), dim3(64), 0, nullptr,
                       static_cast<uint32_t*>(buf.p), iters, static_cast<uint64_t*>(out.p));
    AR_HIP(hipGetLastError());
    AR_HIP(hipDeviceSynchronize());
    uint64_t t = 0;
    AR_HIP(hipMemcpy(&t, out.p, sizeof t, hipMemcpyDeviceToHost));
    res->fence_ns = static_cast<double>(t) / hz * 1e9 / iters;
  }
  int rc;
  if ((rc = run_chase<ar::kPlain>(1ull << 20, 20000, true, &res->l2_load_ns)) != AR_OK) return rc;
  if ((rc = run_chase<ar::kSc1>(1ull << 20, 20000, true, &res->coherent_load_ns)) != AR_OK)
    return rc;
  if ((rc = run_chase<ar::kPlain>(64ull << 20, 20000, true, &res->mall_load_ns)) != AR_OK)
    return rc;
  if ((rc = run_chase<ar::kPlain>(1ull << 30, 20000, false, &res->hbm_load_ns)) != AR_OK)
    return rc;
  // The store term on a line homed near the two XCDs and on one homed in the other half.
  int xcc[2] = {-1, -1};
  {
    PageBuf page;
    if ((rc = page.alloc(ar::kNearPage)) != AR_OK) return rc;
    int a = 0, b = 0;
    pair_blocks(placement, a, b);
    float half[ar::kNearPositions];
    if ((rc = pingpong_positions(page.p, a, b, 1000, half)) != AR_OK) return rc;
    res->store_half_rtt_ns = *std::min_element(half, half + ar::kNearPositions);
    res->store_half_rtt_far_ns = *std::max_element(half, half + ar::kNearPositions);
    // the XCC ids of the two workgroups, from the plain ping-pong on the same pair
    double unused;
    if ((rc = run_pingpong(placement, ar::kSc1, ar::kSc1, 10, &unused, xcc)) != AR_OK) return rc;
  }
  res->xcc_a = xcc[0];
  res->xcc_b = xcc[1];
  res->floor_ns = 2.0 * res->l2_load_ns + res->store_half_rtt_ns;
  res->floor_fence_ns = 2.0 * res->fence_ns + res->store_half_rtt_ns;
  return AR_OK;
}

int ar_torn_lines(int placement, int nlines, int gens, uint64_t* torn, uint64_t* reads) {
  if (torn == nullptr || reads == nullptr) return ar_fail(AR_EINVAL, "null result pointer");
  if (nlines < 1 || nlines > 64 || gens < 1 || gens > 10000000)
    return ar_fail(AR_EINVAL, "nlines must be in [1, 64] and gens in [1, 1e7]");
  DevBuf lines, out;
  AR_HIP(hipMalloc(&lines.p, 64 * 16));
  AR_HIP(hipMalloc(&out.p, 4 * sizeof(unsigned long long)));
  AR_HIP(hipMemset(lines.p, 0, 64 * 16));
  AR_HIP(hipMemset(out.p, 0, 4 * sizeof(unsigned long long)));
  int a = 0, b = 0;
  pair_blocks(placement, a, b);
  hipLaunchKernelGGL(ar::sol_torn, dim3(16), dim3(64), 0, nullptr,
                     static_cast<ar::u32x4*>(lines.p), nlines, gens, a, b,
                     static_cast<uint32_t>(std::min<int64_t>(4ll * gens + 1000000, 100000000)),
                     static_cast<unsigned long long*>(out.p));
  AR_HIP(hipGetLastError());
  AR_HIP(hipDeviceSynchronize());
  unsigned long long o[4];
  AR_HIP(hipMemcpy(o, out.p, sizeof o, hipMemcpyDeviceToHost));
  *torn = o[0];
  *reads = o[1];
  return AR_OK;
}

int ar_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (dst == nullptr || src == nullptr) return ar_fail(AR_EINVAL, "null buffer");
  if (bytes % 16 != 0) return ar_fail(AR_EINVAL, "bytes must be a multiple of 16");
  if (((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u) != 0)
    return ar_fail(AR_EINVAL, "buffers must be 16-byte aligned");
  // pieces of at most 1 GiB, each within one buffer descriptor's 32-bit range
  constexpr size_t kPiece = size_t(1) << 30;
  constexpr uint64_t kThreads = 512, kMaxBlocks = 16384;
  for (size_t off = 0; off < bytes; off += kPiece) {
    const uint32_t n = static_cast<uint32_t>(std::min(kPiece, bytes - off));
    const uint64_t blocks = std::min<uint64_t>(kMaxBlocks, (n / 16 + 2 * kThreads - 1) / (2 * kThreads));
    hipLaunchKernelGGL(ar::stream_copy, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(src) + off, static_cast<uint8_t*>(dst) + off, n);
    AR_HIP(hipGetLastError());
  }
  return AR_OK;
}

}  // extern "C"
