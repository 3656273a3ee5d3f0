// Device probes for the measurement side of the library (not on the hot
// path): the rates the kernels are compared against, measured on the part
// itself rather than taken from a data sheet.
//
//   streamkl_probe_mfma   back-to-back v_mfma_f32_32x32x16_bf16 with no
//                         operand traffic: the matrix-core rate at the clock
//                         the part holds under matrix load, and that clock
//                         (shader-cycle counter against the constant-rate
//                         wall clock, read by the first wave of each
//                         workgroup)
//   streamkl_probe_exp    independent v_exp_f32 chains: the transcendental
//                         rate the forward and backward exponentials run at
//   streamkl_probe_atomic device-scope fp32 atomic adds, 64 consecutive
//                         floats per wave at scattered 256-byte slots of a
//                         window: the payload rate of the fused backward's dQ
//                         accumulation
//
// Each entry point launches on the caller's stream and returns the HIP
// error of the launch; the caller times it with events.  Grids and buffer
// sizes are checked here so every access stays inside the caller's buffers.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Four independent accumulator chains per wave so the issue of one never
// waits for the result of the previous one.  clk[2*blockIdx.x + {0,1}]:
// shader cycles and wall-clock ticks between the first and last MFMA of
// wave 0 (the clock the matrix work ran at).
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* out, unsigned long long* clk, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  const unsigned long long t1 = clock64(), w1 = wall_clock64();
  // every thread writes its own slot, so nothing is optimised away
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = w1 - w0;
  }
}

// Eight independent chains x <- 2^-x per lane (values stay in (0.5, 1]).
__global__ __launch_bounds__(256) void probe_exp_kernel(float* out, int iters) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.01f * (float)((threadIdx.x + j) & 15);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Wave w adds 1.0 to 64 consecutive floats at slot hash(w, i) of the window
// (slots of 64 floats; `slots` of them).
__global__ __launch_bounds__(256) void probe_atomic_kernel(float* win, uint32_t slots, int iters) {
  const uint32_t wave = (blockIdx.x * 256 + threadIdx.x) >> 6, lane = threadIdx.x & 63;
  uint32_t h = wave * 2654435761u + 12345u;
  for (int i = 0; i < iters; ++i) {
    h = h * 1664525u + 1013904223u;
    atomicAdd(win + (uint64_t)(h % slots) * 64 + lane, 1.0f);
  }
}

}  // namespace

extern "C" {

// out: >= blocks * 256 floats; clk: >= 2 * blocks values.  4 waves per workgroup.
int streamkl_probe_mfma(float* out, unsigned long long* clk, int blocks, int iters, void* stream) {
  if (!out || !clk || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, clk, iters);
  return (int)hipGetLastError();
}

// out: >= blocks * 256 floats.
int streamkl_probe_exp(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_exp_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
  return (int)hipGetLastError();
}

// Rate of the constant wall clock that wall_clock64() counts, in kHz.
int streamkl_probe_wall_clock_khz(int* khz) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return (int)e;
}

// win: >= slots * 64 floats.
int streamkl_probe_atomic(float* win, uint32_t slots, int blocks, int iters, void* stream) {
  if (!win || slots < 1 || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_atomic_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), win, slots,
                     iters);
  return (int)hipGetLastError();
}

}  // extern "C"
