// One translation unit per (dtype, d1, d2): compiled several times with
// -DSKL_T=<type> -DSKL_TN=<tag> -DSKL_D1=<d1> -DSKL_D2=<d2> so the kernel
// instantiations build in parallel.  Each exports six launchers with
// C++ linkage, named launch_<kind>_<tag>_<d1>_<d2>.
#include "kernels.hpp"
#include "launch.hpp"

#define SKL_CAT_(a, b, c, d) a##_##b##_##c##_##d
#define SKL_CAT(a, b, c, d) SKL_CAT_(a, b, c, d)

namespace streamkl {

// The joint dK kernel (setting 3) exists for bf16 only and has no fused
// form; a template, so the fp32 kernel is never instantiated.  Internal
// linkage and the head dims as parameters: every translation unit defines its
// own.
namespace {
template <typename T, int D1, int D2>
hipError_t launch_joint_dk(const BwdArgs& a, dim3 g, dim3 b, hipStream_t st, bool fused) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorInvalidValue;
  } else {
    if (fused) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dk_kernel<T, D1, D2, 3, false, kBwdQTile<T>>), g, b, 0, st, a);
    return hipGetLastError();
  }
}
}  // namespace

// a.lpart set: the fused-loss instantiation (only unsplit launches finalize rows here)
hipError_t SKL_CAT(launch_fwd, SKL_TN, SKL_D1, SKL_D2)(const FwdArgs& a, int64_t nblocks, hipStream_t st) {
  if (a.lpart && a.nsplit == 1)
    hipLaunchKernelGGL((fwd_kernel<SKL_T, SKL_D1, SKL_D2, kFwdTile, true>), dim3((unsigned)nblocks), dim3(256), 0, st,
                       a);
  else
    hipLaunchKernelGGL((fwd_kernel<SKL_T, SKL_D1, SKL_D2, kFwdTile>), dim3((unsigned)nblocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t SKL_CAT(launch_fwd_pp, SKL_TN, SKL_D1, SKL_D2)(const FwdArgs& a, int64_t nblocks, hipStream_t st) {
  if (a.lpart)
    hipLaunchKernelGGL((fwd_pp_kernel<SKL_T, SKL_D1, SKL_D2, kFwdPPTile<SKL_T>, true>), dim3((unsigned)nblocks),
                       dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_pp_kernel<SKL_T, SKL_D1, SKL_D2, kFwdPPTile<SKL_T>>), dim3((unsigned)nblocks), dim3(512),
                       0, st, a);
  return hipGetLastError();
}

hipError_t SKL_CAT(launch_fwd_dec, SKL_TN, SKL_D1, SKL_D2)(const FwdArgs& a, int64_t nblocks, hipStream_t st) {
  if constexpr (sizeof(SKL_T) != 2) {
    return hipErrorInvalidValue;  // bf16 only
  } else {
    hipLaunchKernelGGL((fwd_decode_kernel<SKL_D1, SKL_D2>), dim3((unsigned)nblocks), dim3(256), 0, st, a);
    return hipGetLastError();
  }
}

hipError_t SKL_CAT(launch_bwd_dq, SKL_TN, SKL_D1, SKL_D2)(const BwdArgs& a, int setting, int64_t nblocks,
                                                           hipStream_t st) {
  const dim3 g((unsigned)nblocks), b(64 * kBwdQWaves);
  constexpr int W = kBwdQWaves;
  if (setting == 1) hipLaunchKernelGGL((bwd_dq_kernel<SKL_T, SKL_D1, SKL_D2, 1, kBwdKeyTile, W>), g, b, 0, st, a);
  else if (setting == 2) hipLaunchKernelGGL((bwd_dq_kernel<SKL_T, SKL_D1, SKL_D2, 2, kBwdKeyTile, W>), g, b, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t SKL_CAT(launch_bwd_dk, SKL_TN, SKL_D1, SKL_D2)(const BwdArgs& a, int setting, bool fused, int64_t nblocks,
                                                           hipStream_t st) {
  const dim3 g((unsigned)nblocks), b(256), b8(64 * kBwdKWaves);
  constexpr int W = kBwdKWaves;
  if (setting == 1) {
    if (fused) hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 1, true, kBwdQTile<SKL_T>>), g, b, 0, st, a);
    else hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 1, false, kBwdQTile<SKL_T>, W>), g, b8, 0, st, a);
  } else if (setting == 2) {
    if (fused) hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 2, true, kBwdQTile<SKL_T>>), g, b, 0, st, a);
    else hipLaunchKernelGGL((bwd_dk_kernel<SKL_T, SKL_D1, SKL_D2, 2, false, kBwdQTile<SKL_T>, W>), g, b8, 0, st, a);
  } else {
    return launch_joint_dk<SKL_T, SKL_D1, SKL_D2>(a, g, b, st, fused);
  }
  return hipGetLastError();
}

hipError_t SKL_CAT(launch_bwd_dec, SKL_TN, SKL_D1, SKL_D2)(const BwdArgs& a, int setting, int64_t nblocks,
                                                            hipStream_t st) {
  if constexpr (sizeof(SKL_T) != 2) {
    return hipErrorInvalidValue;  // bf16 only
  } else {
    if (setting == 1)
      hipLaunchKernelGGL((bwd_decode_kernel<SKL_D1, SKL_D2, 1>), dim3((unsigned)nblocks), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_decode_kernel<SKL_D1, SKL_D2, 2>), dim3((unsigned)nblocks), dim3(256), 0, st, a);
    return hipGetLastError();
  }
}

}  // namespace streamkl
