// Host-side declarations shared by the runtime translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ar_args.h"

typedef void (*ar_kernel_fn)(ar::Args);

// Defined in ar_kernels.hip (dispatch) and ar_kernels_{f32,bf16,i32}.hip (per data type).
ar_kernel_fn ar_select_kernel(int algo, int dt, int nmax);
ar_kernel_fn ar_select_kernel_f32(int algo, int nmax);
ar_kernel_fn ar_select_kernel_bf16(int algo, int nmax);
ar_kernel_fn ar_select_kernel_i32(int algo, int nmax);
void ar_launch_fill(uint8_t* base, uint64_t stride, int nranks, uint64_t off, uint32_t bytes,
                    uint32_t word, hipStream_t stream);
// Count the inputs of `nranks` ranks (nbytes each) that equal the dtype's sentinel into
// ctl[CTL_CHECK_HITS] / ctl[CTL_CHECK_FIRST] (the caller clears them first). Returns a
// hipError_t value.
int ar_launch_check(const void* const* in, int nranks, uint32_t nbytes, int dt, uint32_t* ctl,
                    hipStream_t stream);

// Defined in ar_sol.hip: calibrate near pages of every rank block (2 MiB aligned, zero, at the
// byte offsets page_off[0..npages) of each block): ns[((r * npages + g) * 4 + p) * 8 + k] =
// store -> poll half round trip between XCDs 2p and 2p+1 at position k (granule k / 4, 2 KiB
// sub-block k % 4) of page g of rank block r.
int ar_near_positions(uint8_t* base, uint64_t stride, int nranks, const uint64_t* page_off,
                      int npages, float* ns);

// Defined in ar_host.hip: record an error message for ar_last_error() and return `code`.
int ar_fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int ar_fail_hip(hipError_t e, const char* what);

#define AR_HIP(call)                                   \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return ar_fail_hip(e_, #call); \
  } while (0)
