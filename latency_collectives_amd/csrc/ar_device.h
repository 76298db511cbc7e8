// Device-side primitives for the barrier-free AllReduce kernels (gfx950 / CDNA4).
//
// Memory access model. Every access to scratch goes through a buffer resource descriptor that
// covers exactly one region, so an access outside that region is dropped by the hardware instead
// of faulting. Accesses that another rank (another group of workgroups, usually on another XCD
// with its own L2) must observe carry the agent-coherent cache policy `sc1`: it is what the
// compiler emits for agent-scope relaxed atomic loads and stores on gfx950, here applied to
// 16-byte vector accesses. Poll loops put a compiler memory clobber between iterations so the
// load is re-issued every time.
//
// Synchronisation techniques (Every µs Matters: Achieving Near Speed-of-Light Latency in GPU
// Collectives, §IV "Designing Barrier-Free Collectives"):
//   * LL: one 16-byte store carries 8 bytes of payload and an 8-byte flag equal to the step's
//     sequence number; the receiver polls the line until the flag matches (§IV "LL").
//   * Sentinel: scratch is pre-filled with a value that valid data never takes; the receiver
//     polls until no element equals it, then writes the sentinel back (§IV "Sentinel").
//   * Double buffering: step s uses buffer s & 1; receiving a peer's data for step s+1 is the
//     credit to overwrite that peer's buffer of step s (§IV "Bidirectional Communication Double
//     Buffering", Fig. 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// gfx950 cache-policy bits of the `aux` operand of buffer instructions.
constexpr int kPlain = 0;
constexpr int kSc0 = 1;
constexpr int kNt = 2;
constexpr int kSc1 = 16;
// Agent-coherent policy used for every cross-rank access (loads and stores).
constexpr int kCoh = kSc1;
// Policy of every output store: an output is written once and never read back by the
// collective, so it carries the non-temporal hint (measured on MI355X: the 4-rank bf16 one-shot
// 7 % lower p50 at 16 KiB and 14 % at 256 KiB, the 8-rank two-shot 6-11 % at 256-512 KiB, no
// size slower).
constexpr int kOut = kNt;

// Data-format word of a raw (untyped, stride 0) buffer descriptor on CDNA: 32-bit data format.
constexpr int kRsrcWord3 = 0x00020000;

// A buffer descriptor lives in scalar registers, so its base must be the same in every lane.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, kRsrcWord3);
}

// Out-of-range offset: at or beyond num_records of every descriptor (regions are below 1 GiB and
// user buffers below 2 GiB), so a load there returns zeros and a store there is dropped by the
// buffer unit. Using it instead of a branch keeps runs of stores in one basic block: on gfx9
// loads and stores share one in-order counter, and a store that follows a control-flow join
// otherwise gets a full s_waitcnt in front of it, which would serialise the write-through stores
// to the peers.
constexpr uint32_t kDrop = 0x80000000u;

// For a base that is wave-uniform by construction but reaches the compiler through a memory
// load (a pointer read from a table): readfirstlane tells the compiler it is uniform, so the
// accesses are not wrapped in a loop over distinct descriptor values. Never use it for a base
// that may differ between lanes.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

template <int CP>
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ u32x2 ld8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ uint32_t ld4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st4(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ uint16_t ld2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st2(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, CP);
}

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Agent-scope release / acquire (what the compiler emits for HIP agent-scope fences).
__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Constant-rate device clock shared by all CUs (100 MHz on MI300-class parts).
__device__ __forceinline__ uint64_t now_ticks() {
  compiler_fence();
  uint64_t t = wall_clock64();
  compiler_fence();
  return t;
}

// Start stamp of one AllReduce. Every step takes it itself, after its set-up and right before
// its first input load, and only the first step of a call keeps it (`k` is the chunk index).
__device__ __forceinline__ void stamp_start(uint64_t& t0, int k) {
  const uint64_t t = now_ticks();
  t0 = k == 0 ? t : t0;
}

// Make the compiler compute `x` before this point (it cannot sink the work behind a later
// stamp).
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xFu;
}

// ------------------------------------------------------------------ data types

enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_I32 = 2 };

template <int DT>
struct Ty;
template <>
struct Ty<DT_F32> {
  static constexpr int kElem = 4;
  static constexpr uint32_t kSentinelWord = 0xFFFFFFFFu;  // negative quiet NaN, all mantissa set
  __device__ static bool word_clear(uint32_t w) { return w != 0xFFFFFFFFu; }
};
template <>
struct Ty<DT_BF16> {
  static constexpr int kElem = 2;
  static constexpr uint32_t kSentinelWord = 0xFFFFFFFFu;  // two bf16 negative quiet NaNs
  // A naturally aligned 32-bit word is written as a whole (single-copy atomic), so a slot word
  // holds either both sentinels or two transmitted elements, neither of which may be the
  // sentinel: comparing the word with two sentinels is the per-element test.
  __device__ static bool word_clear(uint32_t w) { return w != 0xFFFFFFFFu; }
};
template <>
struct Ty<DT_I32> {
  static constexpr int kElem = 4;
  static constexpr uint32_t kSentinelWord = 0x80000000u;  // INT32_MIN, outside valid sums
  __device__ static bool word_clear(uint32_t w) { return w != 0x80000000u; }
};

// Two binary32 values -> two bfloat16 in one word (lo in bits 15:0), round to nearest even:
// one gfx950 conversion instruction (v_cvt_pk_bf16_f32, rounding per the default
// round-to-nearest-even mode).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Fixed rank-order fold of W 32-bit payload words. Binary32 accumulation for fp32 and bf16
// (bf16 rounded once when the result is packed), wrapping 32-bit integer addition for int32.
template <int DT, int W>
struct Fold;
template <int W>
struct Fold<DT_F32, W> {
  float a[W];
  __device__ __forceinline__ void init(const uint32_t* w) {
#pragma unroll
    for (int i = 0; i < W; ++i) a[i] = __uint_as_float(w[i]);
  }
  __device__ __forceinline__ void add(const uint32_t* w) {
#pragma unroll
    for (int i = 0; i < W; ++i) a[i] = a[i] + __uint_as_float(w[i]);
  }
  __device__ __forceinline__ void pack(uint32_t* w) const {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = __float_as_uint(a[i]);
  }
};
template <int W>
struct Fold<DT_BF16, W> {
  float a[2 * W];
  __device__ __forceinline__ void init(const uint32_t* w) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      a[2 * i] = __uint_as_float(w[i] << 16);
      a[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ void add(const uint32_t* w) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      a[2 * i] = a[2 * i] + __uint_as_float(w[i] << 16);
      a[2 * i + 1] = a[2 * i + 1] + __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ void pack(uint32_t* w) const {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = bf16x2_rne(a[2 * i], a[2 * i + 1]);
  }
};
template <int W>
struct Fold<DT_I32, W> {
  uint32_t a[W];
  __device__ __forceinline__ void init(const uint32_t* w) {
#pragma unroll
    for (int i = 0; i < W; ++i) a[i] = w[i];
  }
  __device__ __forceinline__ void add(const uint32_t* w) {
#pragma unroll
    for (int i = 0; i < W; ++i) a[i] = a[i] + w[i];
  }
  __device__ __forceinline__ void pack(uint32_t* w) const {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = a[i];
  }
};

// Branch-free (bitwise and): no element of the unit equals the sentinel.
template <int DT>
__device__ __forceinline__ bool vec_clear(u32x4 v) {
  return Ty<DT>::word_clear(v.x) & Ty<DT>::word_clear(v.y) & Ty<DT>::word_clear(v.z) &
         Ty<DT>::word_clear(v.w);
}
template <int DT>
__device__ __forceinline__ bool vec_clear(u32x2 v) {
  return Ty<DT>::word_clear(v.x) & Ty<DT>::word_clear(v.y);
}

// A slot unit of UB bytes (16: four words, 8: two words) and its loads and stores.
template <int UB>
struct UnitVec;
template <>
struct UnitVec<16> {
  using type = u32x4;
};
template <>
struct UnitVec<8> {
  using type = u32x2;
};
template <int UB>
using unit_t = typename UnitVec<UB>::type;

template <int CP>
__device__ __forceinline__ void ld_vec(rsrc_t r, uint32_t off, u32x4& v) {
  v = ld16<CP>(r, off);
}
template <int CP>
__device__ __forceinline__ void ld_vec(rsrc_t r, uint32_t off, u32x2& v) {
  v = ld8<CP>(r, off);
}
template <int CP>
__device__ __forceinline__ void st_vec(rsrc_t r, uint32_t off, u32x4 v) {
  st16<CP>(r, off, v);
}
template <int CP>
__device__ __forceinline__ void st_vec(rsrc_t r, uint32_t off, u32x2 v) {
  st8<CP>(r, off, v);
}

template <int DT, int UB>
__device__ __forceinline__ unit_t<UB> sentinel_unit() {
  unit_t<UB> v;
#pragma unroll
  for (int k = 0; k < UB / 4; ++k) v[k] = Ty<DT>::kSentinelWord;
  return v;
}

// ------------------------------------------------------------------ user buffers
//
// A user buffer of `nbytes` bytes is read through a descriptor whose num_records is nbytes
// rounded up to a multiple of 4 (in_rsrc) and written through one whose num_records is nbytes
// (out_rsrc). The buffer unit checks the range per 32-bit word: words past the end read as zero
// and are not written. So one vector access per unit handles every tail of 4-byte elements and
// every unit of an even bf16 count without a branch. A bf16 message of odd length ends in the
// low half of a word whose high half is not part of the buffer: the load clears that half, and
// the store writes that last element with one 2-byte store.

__device__ __forceinline__ rsrc_t in_rsrc(const void* base, uint32_t nbytes) {
  return make_rsrc(base, (nbytes + 3u) & ~3u);
}
__device__ __forceinline__ rsrc_t out_rsrc(void* base, uint32_t nbytes) {
  return make_rsrc(base, nbytes);
}

// For a bf16 message of odd length: clear the half word past the end in the unit of `w` that was
// loaded from byte offset `off` (any other unit is left as it is).
template <int UB>
__device__ __forceinline__ void clear_odd_tail(uint32_t off, uint32_t nbytes, uint32_t* w) {
  const uint32_t last = nbytes & ~3u;  // word holding the last element
#pragma unroll
  for (int k = 0; k < UB / 4; ++k) w[k] = (off + 4u * k == last) ? (w[k] & 0xFFFFu) : w[k];
}

// True for a bf16 message of odd length. nbytes is the same in every lane, so a branch on this is
// a scalar branch that even lengths skip; the empty asm in the branch keeps the compiler from
// turning the block into selects that every unit executes.
template <int DT>
__device__ __forceinline__ bool odd_tail(uint32_t nbytes) {
  return Ty<DT>::kElem == 2 && (nbytes & 2u) != 0u;
}

// Load one unit (UB bytes, 8 or 16) at byte offset `off`; zeros past the end (or for kDrop).
// kTail = false leaves an odd bf16 tail to the caller (clear_odd_tail after a batch of loads).
template <int DT, int UB, int CP = kPlain, bool kTail = true>
__device__ __forceinline__ void load_unit(rsrc_t r, uint32_t off, uint32_t nbytes, uint32_t* w) {
  if constexpr (UB == 16) {
    const u32x4 v = ld16<CP>(r, off);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const u32x2 v = ld8<CP>(r, off);
    w[0] = v.x; w[1] = v.y;
  }
  if constexpr (kTail && Ty<DT>::kElem == 2) {
    if (odd_tail<DT>(nbytes)) {
      asm volatile("");
      clear_odd_tail<UB>(off, nbytes, w);
    }
  }
}

// Store one unit at byte offset `off`; nothing past the end (or for kDrop) is written.
template <int DT, int UB, int CP = kPlain>
__device__ __forceinline__ void store_unit(rsrc_t r, uint32_t off, uint32_t nbytes,
                                           const uint32_t* w) {
  if constexpr (UB == 16) {
    st16<CP>(r, off, u32x4{w[0], w[1], w[2], w[3]});
  } else {
    st8<CP>(r, off, u32x2{w[0], w[1]});
  }
  if constexpr (Ty<DT>::kElem == 2) {
    // the last element of an odd-length message: one 2-byte store (dropped in every other unit)
    if (odd_tail<DT>(nbytes)) {
      asm volatile("");
      const uint32_t last = nbytes & ~3u;
      const bool tail = off <= last && last < off + UB;
      uint32_t word = w[0];
#pragma unroll
      for (int k = 1; k < UB / 4; ++k) word = (off + 4u * k == last) ? w[k] : word;
      st2<CP>(r, tail ? last : kDrop, static_cast<uint16_t>(word & 0xFFFFu));
    }
  }
}

// s_waitcnt that waits until at most `n` vector memory operations of this wave are outstanding
// and does not wait on the other counters (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8). Vector memory operations complete in issue order, so this waits for
// everything issued before the last `n`.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace ar
