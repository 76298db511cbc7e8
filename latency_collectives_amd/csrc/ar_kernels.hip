// Scratch set-up and input-check kernels, and the dispatch of (algorithm, data type, rank
// bound) to the AllReduce kernels, whose instances live in one translation unit per data type
// (ar_kernels_f32.hip, ar_kernels_bf16.hip, ar_kernels_i32.hip; their code is in
// ar_kernels_impl.h).

#include "ar_args.h"
#include "ar_device.h"
#include "ar_internal.h"

namespace ar {

// Fill `bytes` of every rank's block at `off` with the 32-bit word `word` (scratch set-up).
__global__ void fill_region(uint8_t* base, uint64_t stride, int nranks, uint64_t off,
                            uint32_t bytes, uint32_t word) {
  const uint32_t vecs = bytes / 16u;
  const uint64_t total = static_cast<uint64_t>(vecs) * nranks;
  const u32x4 v = {word, word, word, word};
  for (uint64_t g = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += static_cast<uint64_t>(gridDim.x) * blockDim.x) {
    const uint64_t r = g / vecs, i = g % vecs;
    *reinterpret_cast<u32x4*>(base + r * stride + off + i * 16u) = v;
  }
}

// Input check (AR_OPT_CHECK_INPUTS): count the input elements of every rank that equal the
// dtype's sentinel bit pattern, and keep the smallest (rank << 40) | element among them. The
// sentinel protocols require that no transmitted value equals the sentinel (Every µs Matters,
// §IV "Sentinel"); this is the optional check of that caller obligation. Grid: x over the
// words of one rank, y over the ranks.
struct CheckArgs {
  const void* in[kMaxRanks];
  uint32_t nbytes;
  int dt;
  uint32_t* ctl;
};

__global__ void check_inputs(CheckArgs a) {
  const int r = blockIdx.y;
  const uint32_t* w = static_cast<const uint32_t*>(a.in[r]);
  const uint32_t words = a.nbytes / 4u, tail = a.nbytes % 4u;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < words + (tail ? 1u : 0u);
       i += gridDim.x * blockDim.x) {
    uint64_t elem = ~0ull;
    if (a.dt == DT_BF16) {
      // a trailing half word is read alone: the buffer may end in the middle of a word
      const uint32_t lo = i < words ? (w[i] & 0xFFFFu)
                                    : static_cast<const uint16_t*>(a.in[r])[2u * i];
      if (lo == 0xFFFFu) elem = 2ull * i;
      else if (i < words && (w[i] >> 16) == 0xFFFFu) elem = 2ull * i + 1;
    } else if (i < words) {
      const uint32_t sentinel = a.dt == DT_I32 ? Ty<DT_I32>::kSentinelWord : Ty<DT_F32>::kSentinelWord;
      if (w[i] == sentinel) elem = i;
    }
    if (elem != ~0ull) {
      atomicAdd(&a.ctl[CTL_CHECK_HITS], 1u);
      atomicMin(reinterpret_cast<unsigned long long*>(&a.ctl[CTL_CHECK_FIRST]),
                static_cast<unsigned long long>((static_cast<uint64_t>(r) << 40) | elem));
    }
  }
}

}  // namespace ar

int ar_launch_check(const void* const* in, int nranks, uint32_t nbytes, int dt, uint32_t* ctl,
                    hipStream_t stream) {
  ar::CheckArgs a;
  for (int r = 0; r < ar::kMaxRanks; ++r) a.in[r] = r < nranks ? in[r] : nullptr;
  a.nbytes = nbytes;
  a.dt = dt;
  a.ctl = ctl;
  const uint32_t words = (nbytes + 3u) / 4u;
  uint32_t bx = (words + 255u) / 256u;
  if (bx > 1024u) bx = 1024u;
  if (bx == 0u) return 0;
  hipLaunchKernelGGL(ar::check_inputs, dim3(bx, static_cast<unsigned>(nranks)), dim3(256), 0,
                     stream, a);
  return static_cast<int>(hipGetLastError());
}

// ------------------------------------------------------------------ host-visible kernel table

// Returns the kernel for (algo, dtype, nmax) or nullptr when the combination is not supported.
ar_kernel_fn ar_select_kernel(int algo, int dt, int nmax) {
  switch (dt) {
    case ar::DT_F32: return ar_select_kernel_f32(algo, nmax);
    case ar::DT_BF16: return ar_select_kernel_bf16(algo, nmax);
    case ar::DT_I32: return ar_select_kernel_i32(algo, nmax);
    default: return nullptr;
  }
}

void ar_launch_fill(uint8_t* base, uint64_t stride, int nranks, uint64_t off, uint32_t bytes,
                    uint32_t word, hipStream_t stream) {
  const uint64_t vecs = static_cast<uint64_t>(bytes / 16u) * nranks;
  uint64_t blocks = (vecs + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return;
  hipLaunchKernelGGL(ar::fill_region, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     base, stride, nranks, off, bytes, word);
}
