// Kernel table of the bf16 AllReduce and collective kernels: one translation unit per data type,
// so that the three sets of template instances compile in parallel.

#include "ar_kernels_impl.h"
#include "ar_internal.h"

namespace {

template <int ALGO>
ar_kernel_fn pick_n(int nmax) {
  constexpr int DT = ar::DT_BF16;
  if constexpr (ALGO == ar::ALGO_TWOSHOT_BULK) {
    switch (nmax) {
      case 2: return ar::ar_kernel_bulk<DT, 2>;
      case 4: return ar::ar_kernel_bulk<DT, 4>;
      case 8: return ar::ar_kernel_bulk<DT, 8>;
      default: return ar::ar_kernel_bulk<DT, 16>;
    }
  } else {
    switch (nmax) {
      case 2: return ar::ar_kernel<ALGO, DT, 2>;
      case 4: return ar::ar_kernel<ALGO, DT, 4>;
      case 8: return ar::ar_kernel<ALGO, DT, 8>;
      default: return ar::ar_kernel<ALGO, DT, 16>;
    }
  }
}

// The peer-split kernels only for 8 and 16 ranks: with fewer peers a wave has few stores to
// spread.
template <int ALGO>
ar_kernel_fn pick_split(int nmax) {
  constexpr int DT = ar::DT_BF16;
  switch (nmax) {
    case 8: return ar::ar_kernel<ALGO, DT, 8>;
    case 16: return ar::ar_kernel<ALGO, DT, 16>;
    default: return nullptr;
  }
}

}  // namespace

ar_kernel_fn ar_select_kernel_bf16(int algo, int nmax) {
  switch (algo) {
    case ar::ALGO_ONESHOT_LL: return pick_n<ar::ALGO_ONESHOT_LL>(nmax);
    case ar::ALGO_ONESHOT_SENTINEL: return pick_n<ar::ALGO_ONESHOT_SENTINEL>(nmax);
    case ar::ALGO_ONESHOT_LL_MULTI: return pick_n<ar::ALGO_ONESHOT_LL_MULTI>(nmax);
    case ar::ALGO_ONESHOT_SENTINEL_MULTI: return pick_n<ar::ALGO_ONESHOT_SENTINEL_MULTI>(nmax);
    case ar::ALGO_ONESHOT_SENTINEL_NARROW: return pick_n<ar::ALGO_ONESHOT_SENTINEL_NARROW>(nmax);
    case ar::ALGO_TWOSHOT: return pick_n<ar::ALGO_TWOSHOT>(nmax);
    case ar::ALGO_TWOSHOT_NARROW: return pick_n<ar::ALGO_TWOSHOT_NARROW>(nmax);
    case ar::ALGO_TWOSHOT_BULK: return pick_n<ar::ALGO_TWOSHOT_BULK>(nmax);
    case ar::ALGO_LL128_ATOMIC: return pick_n<ar::ALGO_LL128_ATOMIC>(nmax);
    case ar::ALGO_LL128_E1: return pick_n<ar::ALGO_LL128_E1>(nmax);
    case ar::ALGO_LL128_E2: return pick_n<ar::ALGO_LL128_E2>(nmax);
    case ar::ALGO_LL128_DET: return pick_n<ar::ALGO_LL128_DET>(nmax);
    case ar::ALGO_LL128_DET_E1: return pick_n<ar::ALGO_LL128_DET_E1>(nmax);
    case ar::ALGO_LL128_DET_E2: return pick_n<ar::ALGO_LL128_DET_E2>(nmax);
    case ar::ALGO_BARRIER2: return pick_n<ar::ALGO_BARRIER2>(nmax);
    case ar::ALGO_REDUCESCATTER: return pick_n<ar::ALGO_REDUCESCATTER>(nmax);
    case ar::ALGO_ALLGATHER: return pick_n<ar::ALGO_ALLGATHER>(nmax);
    case ar::ALGO_BROADCAST: return pick_n<ar::ALGO_BROADCAST>(nmax);
    case ar::ALGO_RS_ONEPASS: return pick_n<ar::ALGO_RS_ONEPASS>(nmax);
    case ar::ALGO_AG_ONEPASS: return pick_n<ar::ALGO_AG_ONEPASS>(nmax);
    case ar::ALGO_RS_NARROW: return pick_n<ar::ALGO_RS_NARROW>(nmax);
    case ar::ALGO_AG_NARROW: return pick_n<ar::ALGO_AG_NARROW>(nmax);
    case ar::ALGO_BCAST_ONEPASS: return pick_n<ar::ALGO_BCAST_ONEPASS>(nmax);
    case ar::ALGO_BCAST_NARROW: return pick_n<ar::ALGO_BCAST_NARROW>(nmax);
    case ar::ALGO_ONESHOT_SPLIT: return pick_split<ar::ALGO_ONESHOT_SPLIT>(nmax);
    case ar::ALGO_ONESHOT_LL_SPLIT: return pick_split<ar::ALGO_ONESHOT_LL_SPLIT>(nmax);
    case ar::ALGO_ONESHOT_SENTINEL_TWO_PAGE:  // 8 and more ranks only
      return nmax == 8 ? ar::ar_kernel<ar::ALGO_ONESHOT_SENTINEL_TWO_PAGE, ar::DT_BF16, 8>
             : nmax == 16 ? ar::ar_kernel<ar::ALGO_ONESHOT_SENTINEL_TWO_PAGE, ar::DT_BF16, 16>
                          : nullptr;
    case ar::ALGO_ONESHOT_LL_TWO_PAGE:  // more than 8 ranks only
      return nmax == 16 ? ar::ar_kernel<ar::ALGO_ONESHOT_LL_TWO_PAGE, ar::DT_BF16, 16> : nullptr;
    case ar::ALGO_TWOSHOT_TWO_PAGE:  // more than 8 ranks only
      return nmax == 16 ? ar::ar_kernel<ar::ALGO_TWOSHOT_TWO_PAGE, ar::DT_BF16, 16> : nullptr;
    case ar::ALGO_ONESHOT_SPLIT_NARROW: return pick_split<ar::ALGO_ONESHOT_SPLIT_NARROW>(nmax);
    case ar::ALGO_TWOSHOT_SPLIT: return pick_split<ar::ALGO_TWOSHOT_SPLIT>(nmax);
    case ar::ALGO_TWOSHOT_SPLIT_NARROW: return pick_split<ar::ALGO_TWOSHOT_SPLIT_NARROW>(nmax);
    case ar::ALGO_LL128_SPLIT: return pick_split<ar::ALGO_LL128_SPLIT>(nmax);
    case ar::ALGO_LL128_SPLIT_E1: return pick_split<ar::ALGO_LL128_SPLIT_E1>(nmax);
    case ar::ALGO_LL128_SPLIT_E2: return pick_split<ar::ALGO_LL128_SPLIT_E2>(nmax);
    default: return nullptr;
  }
}
