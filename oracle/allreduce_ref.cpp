// oracle/allreduce_ref.cpp -- TEST INFRASTRUCTURE ONLY.
//
// A plain, slow, obviously correct CPU AllReduce (sum) over N rank arrays. It exists so that
// the GPU path can be checked against something that shares none of its code. Only the test
// suite, the smoke check and the CPU-baseline leg of the benchmark may load this library; the
// product path never links or calls it.
//
// What it computes (Every µs Matters: Achieving Near Speed-of-Light Latency in GPU Collectives,
// §III.A "Low-Latency AllReduce Algorithms"): after an AllReduce every rank holds the complete
// reduction of all ranks' inputs. Sum is the reduction operator. The pages do not fix the order
// of the additions; this oracle uses the left fold over ranks 0, 1, ..., N-1:
//
//     out[r][i] = ((x_0[i] + x_1[i]) + x_2[i]) + ... + x_{N-1}[i]     for every rank r
//
// Precision (the pages leave it open; the reading used throughout this repository):
//   * fp32 : IEEE binary32, round-to-nearest-even after every addition, no fused operations
//            (built with -ffp-contract=off and without fast-math).
//   * bf16 : each input is widened exactly to binary32, the fold runs in binary32, and the
//            final sum is rounded ONCE to bfloat16 with round-to-nearest-even.
//   * int32: two's-complement wrap-around (the addition is done in uint32_t so that the wrap is
//            defined behaviour in C++).
//   * fp64 : the same fold in binary64; the tests use it only as a near-exact yardstick.
//
// The standalone collectives below are the building blocks the paper names when it notes that
// AllReduce is commonly decomposed into ReduceScatter + AllGather or Reduce + Broadcast
// (§III "Low-Latency AllReduce Algorithms", opening paragraph), and that the Pith review says
// can be rebuilt from the same barrier-free primitives ("If this is right"). The pages print no
// definitions for them; the plainest reading, used here, is the usual one:
//   * reduce-scatter: rank r's input holds N partitions of `recvcount` elements; rank r's output
//     is the sum over ranks of partition r (the same left fold and precision as AllReduce):
//         out[r][i] = x_0[r*recvcount + i] + ... + x_{N-1}[r*recvcount + i]
//   * all-gather: out[r][q*sendcount + i] = x_q[i] for every rank r (a byte copy);
//   * broadcast: out[r][i] = x_root[i] for every rank r (a byte copy).
// With these readings, an all-gather of a reduce-scatter is exactly the AllReduce above (the
// decomposition the paper cites), which is how the tests pin them.
//
// The deterministic variant of the LL128-style atomic AllReduce. The Pith review of the paper
// notes that the atomic algorithm's floating-point sum is not reproducible and imagines a
// deterministic variant "using per-chunk grouping or hierarchical accumulation" ("If this is
// right", third item). The pages give no order for it; the reading used here is hierarchical
// accumulation in a fixed order: the ranks form groups of `group` consecutive ranks
// (0..group-1, group..2*group-1, ...; the last group may be shorter); each group's values are
// added in rank order into a group sum, and the group sums are added in group order:
//
//     g_j[i] = x_{j*group}[i] + x_{j*group+1}[i] + ... (left fold over the group's ranks)
//     out[r][i] = g_0[i] + g_1[i] + ... + g_{G-1}[i]      (left fold over the groups)
//
// in binary32 (bf16: widened inputs, binary32 group sums and fold, one rounding at the end).
// group == 1 and group >= N are both the plain left fold above.
//
// Every function returns 0 on success and -1 on a bad argument (nranks outside [1, 64], a
// null pointer table or a null rank pointer while count > 0). count == 0 is a no-op.
// Output buffers may alias the matching input buffer (in-place); the fold for element i reads
// every input's element i before any output element i is written.

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <chrono>

namespace {

const int kMaxRanks = 64;

bool bad_args(int nranks, const void* in, const void* out) {
  return nranks < 1 || nranks > kMaxRanks || in == nullptr || out == nullptr;
}

// bfloat16 is the upper half of a binary32 bit pattern, so widening is exact: shift left by 16.
float widen_bf16(uint16_t b) {
  uint32_t bits = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return f;
}

// binary32 -> bfloat16, round to nearest, ties to even. The 16 discarded low bits are compared
// with the halfway point 0x8000: above rounds up, below truncates, exactly halfway rounds to the
// even neighbour (the one whose kept low bit is 0). A carry out of the mantissa correctly bumps
// the exponent, and the largest finite values round up to infinity as IEEE requires. NaNs are
// returned as a quiet NaN with the same sign.
uint16_t narrow_to_bf16(float f) {
  uint32_t bits;
  std::memcpy(&bits, &f, sizeof bits);
  const uint32_t exp_mask = 0x7F800000u, man_mask = 0x007FFFFFu;
  if ((bits & exp_mask) == exp_mask && (bits & man_mask) != 0) {
    return static_cast<uint16_t>((bits >> 16) | 0x0040u);
  }
  uint32_t kept = bits >> 16;
  uint32_t dropped = bits & 0xFFFFu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u) != 0)) {
    kept += 1;
  }
  return static_cast<uint16_t>(kept);
}

template <typename T, typename Acc, typename Load, typename Store>
int fold_all(int nranks, const T* const* in, T* const* out, size_t count, Load load, Store store) {
  if (count == 0) return 0;
  if (bad_args(nranks, in, out)) return -1;
  for (int r = 0; r < nranks; ++r) {
    if (in[r] == nullptr || out[r] == nullptr) return -1;
  }
  for (size_t i = 0; i < count; ++i) {
    Acc acc = load(in[0][i]);
    for (int q = 1; q < nranks; ++q) {
      acc = acc + load(in[q][i]);
    }
    for (int r = 0; r < nranks; ++r) {
      out[r][i] = store(acc);
    }
  }
  return 0;
}

// Reduce-scatter with the AllReduce fold: partition r of every rank's input summed into rank
// r's output. Inputs and outputs must not overlap (the partition being folded would be
// overwritten while later ranks still read it otherwise).
template <typename T, typename Acc, typename Load, typename Store>
int fold_scatter(int nranks, const T* const* in, T* const* out, size_t recvcount, Load load,
                 Store store) {
  if (recvcount == 0) return 0;
  if (bad_args(nranks, in, out)) return -1;
  for (int r = 0; r < nranks; ++r) {
    if (in[r] == nullptr || out[r] == nullptr) return -1;
  }
  for (int r = 0; r < nranks; ++r) {
    const size_t base = static_cast<size_t>(r) * recvcount;
    for (size_t i = 0; i < recvcount; ++i) {
      Acc acc = load(in[0][base + i]);
      for (int q = 1; q < nranks; ++q) {
        acc = acc + load(in[q][base + i]);
      }
      out[r][i] = store(acc);
    }
  }
  return 0;
}

// The grouped fold described at the top (groups of `group` consecutive ranks).
template <typename T, typename Load, typename Store>
int fold_grouped(int nranks, int group, const T* const* in, T* const* out, size_t count,
                 Load load, Store store) {
  if (count == 0) return 0;
  if (bad_args(nranks, in, out) || group < 1) return -1;
  for (int r = 0; r < nranks; ++r) {
    if (in[r] == nullptr || out[r] == nullptr) return -1;
  }
  for (size_t i = 0; i < count; ++i) {
    float total = 0.0f;
    for (int first = 0; first < nranks; first += group) {
      const int last = first + group < nranks ? first + group : nranks;
      float g = load(in[first][i]);
      for (int q = first + 1; q < last; ++q) {
        g = g + load(in[q][i]);
      }
      total = first == 0 ? g : total + g;
    }
    for (int r = 0; r < nranks; ++r) {
      out[r][i] = store(total);
    }
  }
  return 0;
}

uint32_t i32_bits(int32_t v) { return static_cast<uint32_t>(v); }
int32_t bits_i32(uint32_t a) {
  int32_t s;
  std::memcpy(&s, &a, sizeof s);
  return s;
}

}  // namespace

extern "C" {

int oracle_allreduce_f32(int nranks, const float* const* in, float* const* out, size_t count) {
  return fold_all<float, float>(
      nranks, in, out, count, [](float v) { return v; }, [](float a) { return a; });
}

int oracle_allreduce_f64(int nranks, const double* const* in, double* const* out, size_t count) {
  return fold_all<double, double>(
      nranks, in, out, count, [](double v) { return v; }, [](double a) { return a; });
}

int oracle_allreduce_bf16(int nranks, const uint16_t* const* in, uint16_t* const* out,
                          size_t count) {
  return fold_all<uint16_t, float>(nranks, in, out, count, widen_bf16, narrow_to_bf16);
}

int oracle_allreduce_i32(int nranks, const int32_t* const* in, int32_t* const* out,
                         size_t count) {
  return fold_all<int32_t, uint32_t>(
      nranks, in, out, count, [](int32_t v) { return static_cast<uint32_t>(v); },
      [](uint32_t a) {
        int32_t s;
        std::memcpy(&s, &a, sizeof s);
        return s;
      });
}

int oracle_allreduce_grouped_f32(int nranks, int group, const float* const* in,
                                 float* const* out, size_t count) {
  return fold_grouped<float>(
      nranks, group, in, out, count, [](float v) { return v; }, [](float a) { return a; });
}

int oracle_allreduce_grouped_bf16(int nranks, int group, const uint16_t* const* in,
                                  uint16_t* const* out, size_t count) {
  return fold_grouped<uint16_t>(nranks, group, in, out, count, widen_bf16, narrow_to_bf16);
}

int oracle_reducescatter_f32(int nranks, const float* const* in, float* const* out,
                              size_t recvcount) {
  return fold_scatter<float, float>(
      nranks, in, out, recvcount, [](float v) { return v; }, [](float a) { return a; });
}

int oracle_reducescatter_f64(int nranks, const double* const* in, double* const* out,
                              size_t recvcount) {
  return fold_scatter<double, double>(
      nranks, in, out, recvcount, [](double v) { return v; }, [](double a) { return a; });
}

int oracle_reducescatter_bf16(int nranks, const uint16_t* const* in, uint16_t* const* out,
                               size_t recvcount) {
  return fold_scatter<uint16_t, float>(nranks, in, out, recvcount, widen_bf16, narrow_to_bf16);
}

int oracle_reducescatter_i32(int nranks, const int32_t* const* in, int32_t* const* out,
                              size_t recvcount) {
  return fold_scatter<int32_t, uint32_t>(nranks, in, out, recvcount, i32_bits, bits_i32);
}

// All-gather of `bytes` per rank: rank q's input lands at byte q*bytes of every output.
int oracle_allgather(int nranks, const uint8_t* const* in, uint8_t* const* out, size_t bytes) {
  if (bytes == 0) return 0;
  if (bad_args(nranks, in, out)) return -1;
  for (int r = 0; r < nranks; ++r) {
    if (in[r] == nullptr || out[r] == nullptr) return -1;
  }
  for (int r = 0; r < nranks; ++r) {
    for (int q = 0; q < nranks; ++q) {
      for (size_t j = 0; j < bytes; ++j) {
        out[r][static_cast<size_t>(q) * bytes + j] = in[q][j];
      }
    }
  }
  return 0;
}

// Broadcast of `bytes` from the root's buffer into every rank's output.
int oracle_broadcast(int nranks, const uint8_t* root_in, uint8_t* const* out, size_t bytes) {
  if (bytes == 0) return 0;
  if (nranks < 1 || nranks > kMaxRanks || root_in == nullptr || out == nullptr) return -1;
  for (int r = 0; r < nranks; ++r) {
    if (out[r] == nullptr) return -1;
  }
  for (int r = 0; r < nranks; ++r) {
    for (size_t j = 0; j < bytes; ++j) {
      out[r][j] = root_in[j];
    }
  }
  return 0;
}

uint16_t oracle_f32_to_bf16(float f) { return narrow_to_bf16(f); }
float oracle_bf16_to_f32(uint16_t b) { return widen_bf16(b); }

// Wall-clock seconds spent in `reps` calls of the AllReduce for `dtype` (0 fp32, 1 bf16,
// 2 int32), single-threaded, on caller-provided host buffers. Used only to report a CPU
// baseline next to the GPU numbers. Returns a negative value on a bad argument.
double oracle_time_allreduce(int dtype, int nranks, const void* const* in, void* const* out,
                             size_t count, int reps) {
  if (reps < 1) return -1.0;
  auto t0 = std::chrono::steady_clock::now();
  for (int k = 0; k < reps; ++k) {
    int rc = -1;
    if (dtype == 0) {
      rc = oracle_allreduce_f32(nranks, reinterpret_cast<const float* const*>(in),
                                reinterpret_cast<float* const*>(out), count);
    } else if (dtype == 1) {
      rc = oracle_allreduce_bf16(nranks, reinterpret_cast<const uint16_t* const*>(in),
                                 reinterpret_cast<uint16_t* const*>(out), count);
    } else if (dtype == 2) {
      rc = oracle_allreduce_i32(nranks, reinterpret_cast<const int32_t* const*>(in),
                                reinterpret_cast<int32_t* const*>(out), count);
    }
    if (rc != 0) return -1.0;
  }
  auto t1 = std::chrono::steady_clock::now();
  return std::chrono::duration<double>(t1 - t0).count();
}

}  // extern "C"
