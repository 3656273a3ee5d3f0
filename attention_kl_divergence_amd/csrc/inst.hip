// One translation unit per (dtype, d1, d2): compiled several times with
// -DSKL_T=<type> -DSKL_TN=<tag> -DSKL_D1=<d1> -DSKL_D2=<d2> so the kernel
// instantiations build in parallel.  Each exports six launchers with
// C++ linkage, named launch_<kind>_<tag>_<d1>_<d2>.
#include "kernels.hpp"
#include "launch.hpp"

#define SKL_CAT_(a, b, c, d) a##_##b##_##c##_##d
#define SKL_CAT(a, b, c, d) SKL_CAT_(a, b, c, d)

namespace streamkl {

// Each kernel is instantiated for a plain launch (NoTable) and for a grouped
// launch over elements of a ragged batch (RaggedTable); these helpers launch
// one with the table type RT.  Internal linkage and the head dims as
// template parameters: every translation unit defines its own.
namespace {
template <typename RT>
hipError_t fwd_go(const FwdArgs& a, int64_t nblocks, hipStream_t st, const RT& rt) {
  const dim3 g((unsigned)nblocks), b(256);
  // a.lpart set: the fused-loss instantiation (only unsplit launches finalize rows here)
  if (a.lpart && a.nsplit == 1)
    hipLaunchKernelGGL((fwd_kernel<SKL_T, SKL_D1, SKL_D2, kFwdTile, true, RT>), g, b, 0, st, a, rt);
  else
    hipLaunchKernelGGL((fwd_kernel<SKL_T, SKL_D1, SKL_D2, kFwdTile, false, RT>), g, b, 0, st, a, rt);
  return hipGetLastError();
}

// fp32 with head dims past 64 + 64 has no ping-pong form (its fragments
// spill at two waves per SIMD; the planner keeps those on the 4-wave kernel)
template <typename RT>
hipError_t fwd_pp_go(const FwdArgs& a, int64_t nblocks, hipStream_t st, const RT& rt) {
  if constexpr (sizeof(SKL_T) == 4 && SKL_D1 + SKL_D2 > 128) {
    return hipErrorInvalidValue;
  } else {
    constexpr int BK = kFwdPPTile<SKL_T>;
    const dim3 g((unsigned)nblocks), b(512);
    if (a.lpart)
      hipLaunchKernelGGL((fwd_pp_kernel<SKL_T, SKL_D1, SKL_D2, BK, true, RT>), g, b, 0, st, a, rt);
    else
      hipLaunchKernelGGL((fwd_pp_kernel<SKL_T, SKL_D1, SKL_D2, BK, false, RT>), g, b, 0, st, a, rt);
    return hipGetLastError();
  }
}

template <typename RT>
hipError_t dq_go(const BwdArgs& a, int setting, int64_t nblocks, hipStream_t st, const RT& rt) {
  constexpr int W = kBwdWaves<SKL_T>;
  const dim3 g((unsigned)nblocks), b(64 * W);
  if (setting == 1)
    hipLaunchKernelGGL((bwd_dq_kernel<SKL_T, SKL_D1, SKL_D2, 1, kBwdKeyTile<SKL_T>, W, RT>), g, b, 0, st, a, rt);
  else if (setting == 2)
    hipLaunchKernelGGL((bwd_dq_kernel<SKL_T, SKL_D1, SKL_D2, 2, kBwdKeyTile<SKL_T>, W, RT>), g, b, 0, st, a, rt);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// The joint dK kernel (setting 3) exists for bf16 only and has no fused form.
template <typename RT>
hipError_t joint_dk_go(const BwdArgs& a, dim3 g, hipStream_t st, const RT& rt) {
  if constexpr (sizeof(SKL_T) != 2) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 3, false, kBwdQTile<SKL_T>, 4, RT>), g, dim3(256), 0, st,
                       a, rt);
    return hipGetLastError();
  }
}

// The separate (8-wave in bf16, 4-wave in fp32) and joint dK kernels; the
// fused (4-wave) form runs plain launches only.
template <typename RT>
hipError_t dk_go(const BwdArgs& a, int setting, bool fused, int64_t nblocks, hipStream_t st, const RT& rt) {
  constexpr int W = kBwdWaves<SKL_T>;
  constexpr int BQ = kBwdQTile<SKL_T>;
  const dim3 g((unsigned)nblocks), b(256), b8(64 * W);
  if (setting == 3) return fused ? hipErrorInvalidValue : joint_dk_go(a, g, st, rt);
  if (setting != 1 && setting != 2) return hipErrorInvalidValue;
  if (fused) {
    if constexpr (kRagged<RT>) {
      return hipErrorInvalidValue;
    } else {
      if (setting == 1) hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 1, true, BQ>), g, b, 0, st, a, rt);
      else hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 2, true, BQ>), g, b, 0, st, a, rt);
    }
  } else if (setting == 1) {
    hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 1, false, BQ, W, RT>), g, b8, 0, st, a, rt);
  } else {
    hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 2, false, BQ, W, RT>), g, b8, 0, st, a, rt);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t SKL_CAT(launch_fwd, SKL_TN, SKL_D1, SKL_D2)(const FwdArgs& a, int64_t nblocks, hipStream_t st,
                                                        const RaggedTable* rt) {
  return rt ? fwd_go(a, nblocks, st, *rt) : fwd_go(a, nblocks, st, NoTable{});
}

hipError_t SKL_CAT(launch_fwd_pp, SKL_TN, SKL_D1, SKL_D2)(const FwdArgs& a, int64_t nblocks, hipStream_t st,
                                                           const RaggedTable* rt) {
  return rt ? fwd_pp_go(a, nblocks, st, *rt) : fwd_pp_go(a, nblocks, st, NoTable{});
}

hipError_t SKL_CAT(launch_fwd_dec, SKL_TN, SKL_D1, SKL_D2)(const FwdArgs& a, int64_t nblocks, hipStream_t st,
                                                            const DecTable* rt) {
  if constexpr (sizeof(SKL_T) != 2) {
    return hipErrorInvalidValue;  // bf16 only
  } else {
    const dim3 g((unsigned)nblocks), b(256);
    if (rt) hipLaunchKernelGGL((fwd_decode_kernel<SKL_D1, SKL_D2, DecTable>), g, b, 0, st, a, *rt);
    else hipLaunchKernelGGL((fwd_decode_kernel<SKL_D1, SKL_D2>), g, b, 0, st, a, NoTable{});
    return hipGetLastError();
  }
}

hipError_t SKL_CAT(launch_bwd_dq, SKL_TN, SKL_D1, SKL_D2)(const BwdArgs& a, int setting, int64_t nblocks,
                                                           hipStream_t st, const RaggedTable* rt) {
  return rt ? dq_go(a, setting, nblocks, st, *rt) : dq_go(a, setting, nblocks, st, NoTable{});
}

hipError_t SKL_CAT(launch_bwd_dk, SKL_TN, SKL_D1, SKL_D2)(const BwdArgs& a, int setting, bool fused, int64_t nblocks,
                                                           hipStream_t st, const RaggedTable* rt) {
  return rt ? dk_go(a, setting, fused, nblocks, st, *rt) : dk_go(a, setting, fused, nblocks, st, NoTable{});
}

hipError_t SKL_CAT(launch_bwd_dec, SKL_TN, SKL_D1, SKL_D2)(const BwdArgs& a, int setting, int64_t nblocks,
                                                            hipStream_t st, const RaggedTable* rt) {
  if constexpr (sizeof(SKL_T) != 2) {
    return hipErrorInvalidValue;  // bf16 only
  } else {
    auto go = [&](const auto& t) {
      using RT = std::decay_t<decltype(t)>;
      const dim3 g((unsigned)nblocks), b(256);
      if (setting == 1) hipLaunchKernelGGL((bwd_decode_kernel<SKL_D1, SKL_D2, 1, RT>), g, b, 0, st, a, t);
      else hipLaunchKernelGGL((bwd_decode_kernel<SKL_D1, SKL_D2, 2, RT>), g, b, 0, st, a, t);
      return hipGetLastError();
    };
    return rt ? go(*rt) : go(NoTable{});
  }
}

}  // namespace streamkl
