// C ABI of the StreamKL library: argument validation, launch planning
// (key-split count, fused or separate backward) and kernel launches on the
// caller's stream.  Declared in include/streamkl.h.
#include <algorithm>
#include <mutex>
#include <string.h>
#include <type_traits>
#include <vector>

#include "../../include/streamkl.h"
#include "kernels.hpp"
#include "launch.hpp"

namespace streamkl {

// Merge of the split partial states, then the epilogue (one thread per row);
// with the fused loss each workgroup also writes its rows' sum of w_i KL_i.
// With a DecTable, the rows of the table's elements: 256 of one element per
// workgroup.
template <typename RT = NoTable>
__global__ __launch_bounds__(256) void splitk_merge_kernel(const float* __restrict__ ws, float* kl, float* lse1,
                                                           float* lse2, int64_t BH, int n_q, int nsplit, int qs,
                                                           const float* __restrict__ lw, double* lpart, const RT rt) {
  __shared__ double red[4];
  int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x;
  int64_t rows = BH * n_q, head0 = 0, base = 0, fs = BH * (int64_t)nsplit * n_q;
  int qo = 0;  // the element's first row within a head (packed batches)
  if constexpr (kDecTable<RT>) {
    const int e = table_elem(rt.mstart, rt.n, blockIdx.x);
    qo = rt.qoff[e];
    i = (blockIdx.x - rt.mstart[e]) * (int64_t)256 + threadIdx.x;
    n_q = rt.n_q[e];
    nsplit = rt.nsplit[e];
    rows = (int64_t)rt.H * n_q;
    head0 = (int64_t)rt.b[e] * rt.H;
    base = rt.wsb[e];
    fs = rt.fs;
  }
  double lv = 0.0;
  if (i < rows) {
    const int64_t loc = i / n_q;  // the head within the problem (or the element)
    const int q = (int)(i % n_q);
    const int64_t r = (head0 + loc) * qs + qo + q;  // output row (qs rows per head in memory)
    RowState st = empty_state();
    for (int z = 0; z < nsplit; ++z) {
      const int64_t o = base + (loc * nsplit + z) * (int64_t)n_q + q;
      RowState p = {ws[o], ws[o + fs], ws[o + 2 * fs], ws[o + 3 * fs], ws[o + 4 * fs]};
      st = merge_state(st, p);
    }
    const float k = finish_state(st, kl + r, lse1 + r, lse2 + r);
    lv = lw ? (double)lw[r] * (double)k : (double)k;
  }
  if (lpart) loss_partial<4>(lv, red, lpart + blockIdx.x, threadIdx.x);
}

// The fused loss from the forward's per-workgroup partials: their sum in a
// fixed order (strided per thread, then a tree), divided by the row count
// for the mean (count > 0) or taken as is (weighted sum, count = 0).
__global__ __launch_bounds__(1024) void loss_reduce_kernel(const double* __restrict__ part, int64_t n, double count,
                                                          float* out) {
  __shared__ double red[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) acc += part[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int m = 512; m > 0; m >>= 1) {
    if ((int)threadIdx.x < m) red[threadIdx.x] += red[threadIdx.x + m];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = (float)(count > 0 ? red[0] / count : red[0]);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* __restrict__ p, int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// The distillation loss from the per-row KL: sum_i w_i KL_i (w = 1/rows
// when weights is NULL), in one workgroup so the summation order is fixed:
// each thread sums a strided subset in fp64, then a tree over the threads.
__global__ __launch_bounds__(1024) void kl_loss_kernel(const float* __restrict__ kl, const float* __restrict__ w,
                                                      int64_t rows, float* out) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < rows; i += 1024) acc += (double)kl[i] * (w ? (double)w[i] : 1.0);
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int n = 512; n > 0; n >>= 1) {
    if ((int)threadIdx.x < n) part[threadIdx.x] += part[threadIdx.x + n];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = (float)(w ? part[0] : part[0] / (double)rows);
}

// the same for any alignment and count
__global__ __launch_bounds__(256) void fill_zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// Spans of an fp32 tensor to clear, for up to kRaggedMax batch elements:
// element i owns `count` spans of len[i] floats, span j at base[i] +
// j * stride.  Each span is cleared in chunks of `chunk` floats, one
// workgroup per chunk (grid: count * chunks per span, elements).
struct SpanTable {
  int n;
  int count;
  int64_t stride;
  int64_t chunk;
  int64_t nchunk;  // chunks per span of the longest len
  int64_t base[kRaggedMax];
  int64_t len[kRaggedMax];
};

__global__ __launch_bounds__(256) void fill_spans_kernel(float* __restrict__ p, const SpanTable t, int vec) {
  const int e = blockIdx.y;
  const int64_t span = blockIdx.x / t.nchunk, c = blockIdx.x % t.nchunk;
  const int64_t lo = c * t.chunk, hi = min(t.len[e], lo + t.chunk);
  float* s = p + t.base[e] + span * t.stride;
  if (vec) {  // lo, hi and the span's start are multiples of 4 floats, p 16-byte aligned
    float4* s4 = reinterpret_cast<float4*>(s);
    for (int64_t i = lo / 4 + threadIdx.x; i < hi / 4; i += 256) s4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256) s[i] = 0.f;
  }
}

// Partials of the forward for callers that cannot allocate device memory
// (streamkl_fwd_loss_noalloc): split-K states and fused-loss sums live in
// this array, one copy per device, held until the process ends.  Host code
// never passes the name itself to a kernel (on the host it only stands for
// the symbol): it takes each device's address from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local int g_last_hip_error = 0;

struct DeviceInfo {
  int checked = 0;
  int gfx950 = 0;
  int cus = 256;
  void* scratch = nullptr;  // this device's copy of `scratch` (streamkl_fwd_loss_noalloc), once looked up
};
std::mutex g_dev_mutex;
DeviceInfo g_dev[64];

// Device properties are read once per device; every later call reuses them.
streamkl_status device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { g_last_hip_error = (int)e; return STREAMKL_ERR_HIP; }
  if (dev < 0 || dev >= 64) return STREAMKL_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mutex);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) { g_last_hip_error = (int)e; return STREAMKL_ERR_HIP; }
    d.gfx950 = strncmp(p.gcnArchName, "gfx950", 6) == 0;
    d.cus = p.multiProcessorCount > 0 ? p.multiProcessorCount : 256;
    d.checked = 1;
  }
  *out = d;
  return d.gfx950 ? STREAMKL_OK : STREAMKL_ERR_UNSUPPORTED;
}

// The current device's address of `scratch`, looked up once per device with
// that device current (the first call of streamkl_fwd_loss_noalloc on it).
streamkl_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { g_last_hip_error = (int)e; return STREAMKL_ERR_HIP; }
  if (dev < 0 || dev >= 64) return STREAMKL_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mutex);
  DeviceInfo& d = g_dev[dev];
  if (!d.scratch) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return STREAMKL_ERR_HIP;
    }
    d.scratch = ptr;
  }
  *out = d.scratch;
  return STREAMKL_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// A scale must be a finite number (<= 0 selects the default).  Tested on the
// bits, so no floating-point flag can fold the test away.
bool finite_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (u & 0x7fffffffu) < 0x7f800000u;
}

bool ragged(const streamkl_shape* s);
bool packed(const streamkl_shape* s);
streamkl_shape element_shape(const streamkl_shape* s, int64_t b);

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape checks that need no device.  Sizes are bounded so every in-head
// offset fits in 32 bits and every grid fits in one dimension.
streamkl_status check_shape(const streamkl_shape* s, int causal) {
  if (!s) return STREAMKL_ERR_INVALID;
  if (s->B < 1 || s->H < 1 || s->n_q < 1 || s->n_k < 1) return STREAMKL_ERR_INVALID;
  if (s->dtype != STREAMKL_F32 && s->dtype != STREAMKL_BF16) return STREAMKL_ERR_INVALID;
  if ((s->d1 != 64 && s->d1 != 128) || (s->d2 != 64 && s->d2 != 128)) return STREAMKL_ERR_UNSUPPORTED;
  if (s->n_q > (1 << 24) || s->n_k > (1 << 24)) return STREAMKL_ERR_UNSUPPORTED;
  if (s->B > (int64_t(1) << 20) || s->H > (int64_t(1) << 20) || s->B * s->H > (int64_t(1) << 20))
    return STREAMKL_ERR_UNSUPPORTED;
  if (causal && s->n_q > s->n_k) return STREAMKL_ERR_INVALID;
  if ((s->q_off == nullptr) != (s->k_off == nullptr)) return STREAMKL_ERR_INVALID;
  if (packed(s)) {
    // offsets from 0 to the total rows, nondecreasing; the lengths they give
    // follow the rules of ragged batches below
    if (s->q_len || s->k_len) return STREAMKL_ERR_INVALID;
    if (s->q_off[0] != 0 || s->k_off[0] != 0 || s->q_off[s->B] != s->n_q || s->k_off[s->B] != s->n_k)
      return STREAMKL_ERR_INVALID;
    for (int64_t b = 0; b < s->B; ++b)
      if (s->q_off[b + 1] < s->q_off[b] || s->k_off[b + 1] < s->k_off[b]) return STREAMKL_ERR_INVALID;
  }
  if (ragged(s)) {
    // every batch element: lengths within the padded sizes, some key for
    // every query row, bottom-right causal alignment needs q <= k
    for (int64_t b = 0; b < s->B; ++b) {
      const streamkl_shape e = element_shape(s, b);
      const int64_t q = e.n_q, k = e.n_k;
      if (q < 0 || q > s->n_q || k < 0 || k > s->n_k) return STREAMKL_ERR_INVALID;
      if (q > 0 && k == 0) return STREAMKL_ERR_INVALID;
      if (causal && q > k) return STREAMKL_ERR_INVALID;
    }
  }
  // grouped key heads: each count divides H (0 = H)
  for (const int32_t kv : {s->kv_heads1, s->kv_heads2})
    if (kv < 0 || (kv > 0 && s->H % kv != 0)) return STREAMKL_ERR_INVALID;
  return STREAMKL_OK;
}

// query heads per key head of each model
int group1(const streamkl_shape* s) { return s->kv_heads1 > 0 ? (int)(s->H / s->kv_heads1) : 1; }
int group2(const streamkl_shape* s) { return s->kv_heads2 > 0 ? (int)(s->H / s->kv_heads2) : 1; }


float log2e_scale(float scale, int d) { return (scale > 0.f ? scale : 1.0f / sqrtf((float)d)) * kLog2e; }
float plain_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / sqrtf((float)d); }

FwdLaunch pick_fwd(int dtype, int d1, int d2) {
#define SKL_PICK(tn, a, b) if (d1 == a && d2 == b) return launch_fwd_##tn##_##a##_##b;
  if (dtype == STREAMKL_F32) { SKL_PICK(f32, 64, 64) SKL_PICK(f32, 64, 128) SKL_PICK(f32, 128, 64) SKL_PICK(f32, 128, 128) }
  else { SKL_PICK(bf16, 64, 64) SKL_PICK(bf16, 64, 128) SKL_PICK(bf16, 128, 64) SKL_PICK(bf16, 128, 128) }
#undef SKL_PICK
  return nullptr;
}
FwdLaunch pick_fwd_pp(int dtype, int d1, int d2) {
#define SKL_PICK(tn, a, b) if (d1 == a && d2 == b) return launch_fwd_pp_##tn##_##a##_##b;
  if (dtype == STREAMKL_F32) { SKL_PICK(f32, 64, 64) }  // see use_pp
  else { SKL_PICK(bf16, 64, 64) SKL_PICK(bf16, 64, 128) SKL_PICK(bf16, 128, 64) SKL_PICK(bf16, 128, 128) }
#undef SKL_PICK
  return nullptr;
}
DecFwdLaunch pick_fwd_dec(int dtype, int d1, int d2) {
#define SKL_PICK(tn, a, b) if (d1 == a && d2 == b) return launch_fwd_dec_##tn##_##a##_##b;
  if (dtype == STREAMKL_BF16) { SKL_PICK(bf16, 64, 64) SKL_PICK(bf16, 64, 128) SKL_PICK(bf16, 128, 64) SKL_PICK(bf16, 128, 128) }
#undef SKL_PICK
  return nullptr;
}
DqLaunch pick_dq(int dtype, int d1, int d2) {
#define SKL_PICK(tn, a, b) if (d1 == a && d2 == b) return launch_bwd_dq_##tn##_##a##_##b;
  if (dtype == STREAMKL_F32) { SKL_PICK(f32, 64, 64) SKL_PICK(f32, 64, 128) SKL_PICK(f32, 128, 64) SKL_PICK(f32, 128, 128) }
  else { SKL_PICK(bf16, 64, 64) SKL_PICK(bf16, 64, 128) SKL_PICK(bf16, 128, 64) SKL_PICK(bf16, 128, 128) }
#undef SKL_PICK
  return nullptr;
}
DkLaunch pick_dk(int dtype, int d1, int d2) {
#define SKL_PICK(tn, a, b) if (d1 == a && d2 == b) return launch_bwd_dk_##tn##_##a##_##b;
  if (dtype == STREAMKL_F32) { SKL_PICK(f32, 64, 64) SKL_PICK(f32, 64, 128) SKL_PICK(f32, 128, 64) SKL_PICK(f32, 128, 128) }
  else { SKL_PICK(bf16, 64, 64) SKL_PICK(bf16, 64, 128) SKL_PICK(bf16, 128, 64) SKL_PICK(bf16, 128, 128) }
#undef SKL_PICK
  return nullptr;
}

DecBwdLaunch pick_dec_bwd(int dtype, int d1, int d2) {
#define SKL_PICK(tn, a, b) if (d1 == a && d2 == b) return launch_bwd_dec_##tn##_##a##_##b;
  if (dtype == STREAMKL_BF16) { SKL_PICK(bf16, 64, 64) SKL_PICK(bf16, 64, 128) SKL_PICK(bf16, 128, 64) SKL_PICK(bf16, 128, 128) }
#undef SKL_PICK
  return nullptr;
}

// bf16 query ranges that fit one wave's 32 rows run the decode forward, in
// which every wave is one key split, and the decode backward, in which one
// workgroup keeps every query row.
bool decode_shape(const streamkl_shape* s) { return s->dtype == STREAMKL_BF16 && s->n_q <= kDecRows; }

// Workgroups per head of the decode backward: one per CU in all (its LDS
// tiles allow one per CU), at most one per key tile.
int plan_dec_bwd_splits(const streamkl_shape* s, int cus) {
  const int64_t tiles = cdiv(s->n_k, kDecBwdTile);
  int64_t sp = cus / (s->B * s->H);
  if (sp > tiles) sp = tiles;
  return (int)(sp < 1 ? 1 : sp);
}

// Key-split plan.  Split-K (Method 3 of the technical summary) is for shapes
// whose query blocks alone cannot fill the chip.  Decode shapes: about 4
// waves (splits) per CU, all resident at once (one sweep through K1 and K2;
// measured best at 32 heads, against 2-16 waves per CU), >= 8 key blocks per
// split.  Otherwise: aim for >= 4 workgroups per CU, keep >= 4 key tiles per
// split.
int plan_splits(const streamkl_shape* s, int causal, const streamkl_launch* l, int cus) {
  (void)causal;
  if (decode_shape(s)) {
    const int64_t blocks = cdiv(s->n_k, kDecBlock);
    if (l && l->num_splits > 0) return (int)(l->num_splits < blocks ? l->num_splits : blocks);
    int64_t sp = cdiv(4 * (int64_t)cus, s->B * s->H);
    const int64_t maxsp = blocks / 8 > 1 ? blocks / 8 : 1;
    if (sp > maxsp) sp = maxsp;
    if (sp > 4096) sp = 4096;
    return (int)(sp < 1 ? 1 : sp);
  }
  const int64_t tiles = cdiv(s->n_k, kFwdTile);
  if (l && l->num_splits > 0) return (int)(l->num_splits < tiles ? l->num_splits : tiles);
  const int64_t base = s->B * s->H * cdiv(s->n_q, kFwdRows);
  const int64_t want = 4 * (int64_t)cus;
  if (base >= want / 2) return 1;
  int64_t sp = cdiv(want, base);
  const int64_t maxsp = tiles / 4 > 1 ? tiles / 4 : 1;
  if (sp > maxsp) sp = maxsp;
  if (sp > 4096) sp = 4096;
  return (int)(sp < 1 ? 1 : sp);
}

size_t ws_bytes(const streamkl_shape* s, int splits) {
  return splits > 1 ? (size_t)20 * (size_t)(s->B * s->H) * (size_t)s->n_q * (size_t)splits : 0;
}

// How the forward of one problem runs.  Workspace sizing and the launches
// both take it from make_fwd_plan, so the bytes reported are the bytes used.
struct FwdPlan {
  int splits;           // key splits
  bool pp, dec;         // the ping-pong kernel (long unsplit query ranges) / the decode kernel
  int64_t nqb;          // query blocks per head
  int64_t grid;         // workgroups of the forward kernel
  size_t split_bytes;   // split partials (at the start of the workspace)
  int64_t loss_slots;   // workgroups that finalize rows: one fused-loss partial each
};

// The ping-pong forward for an unsplit query range longer than one 4-wave
// workgroup's rows, except fp32 with head dims past 64 + 64, whose operand
// fragments do not fit two waves per SIMD without spilling: those keep the
// 4-wave form at one wave per SIMD.
bool use_pp(const streamkl_shape* s) {
  return s->n_q > kFwdRows && !(s->dtype == STREAMKL_F32 && s->d1 + s->d2 > 128);
}

FwdPlan make_fwd_plan(const streamkl_shape* s, int splits) {
  FwdPlan p;
  const int64_t BH = s->B * s->H;
  p.splits = splits;
  p.pp = splits == 1 && use_pp(s);
  p.dec = splits > 1 && decode_shape(s);
  p.nqb = cdiv(s->n_q, p.pp ? kFwdPPRows : kFwdRows);
  p.grid = p.dec ? BH * cdiv(splits, 4) : BH * p.nqb * splits;
  p.split_bytes = ws_bytes(s, splits);
  // unsplit: the forward kernel finalizes rows; split: the merge kernel (256 rows per workgroup)
  p.loss_slots = splits > 1 ? cdiv(BH * s->n_q, 256) : p.grid;
  return p;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// The cost model of one problem's backward: FLOPs of each separate-mode
// kernel and of the fused kernel, the fused kernel's atomic bytes, and the
// workgroups of each launch against what the chip holds at once (the
// separate dK and dQ kernels run one 8-wave workgroup, 256 rows, per CU; the
// fused key-outer kernel one 4-wave workgroup, 128 keys, per CU).
struct BwdWork {
  double f_sep = 0, f_fused = 0, atomic = 0;
  double wg_dk = 0, wg_dq = 0, wg_fk = 0;
};
constexpr double kBwdRate = 1.0e15;     // sustained MFMA FLOP/s assumed for these kernels
constexpr double kAtomicRate = 1.2e12;  // device-scope fp32 atomic bytes/s

// query-key pairs of one head (bottom-right causal alignment)
double head_pairs(const streamkl_shape* s, int causal) {
  return causal ? (double)s->n_q * (s->n_q + 1) / 2 + (double)s->n_q * (s->n_k - s->n_q) : (double)s->n_q * s->n_k;
}

BwdWork bwd_work(const streamkl_shape* s, int causal, int setting) {
  const double ds = setting == 1 ? s->d2 : s->d1;
  const double pairs = head_pairs(s, causal);
  const double heads = (double)(s->B * s->H);
  const double f_qk = 2.0 * (s->d1 + s->d2), f_grad = 2.0 * ds;
  BwdWork w;
  w.f_sep = heads * pairs * (f_qk + f_grad);
  w.f_fused = heads * pairs * (f_qk + 2 * f_grad);
  w.atomic = heads * pairs * 4.0 * ds / kBwdKRows;
  w.wg_dk = heads * cdiv(s->n_k, bwd_rows(s->dtype == STREAMKL_F32));
  w.wg_dq = heads * cdiv(s->n_q, bwd_rows(s->dtype == STREAMKL_F32));
  w.wg_fk = heads * cdiv(s->n_k, kBwdKRows);
  return w;
}

double chip_use(double wg, int cus) { return wg < cus ? wg / cus : 1.0; }
double t_separate(const BwdWork& w, int cus) {
  return w.f_sep / (kBwdRate * chip_use(w.wg_dk, cus)) + w.f_sep / (kBwdRate * chip_use(w.wg_dq, cus));
}
double t_fused(const BwdWork& w, int cus) {
  return std::max(w.f_fused / (kBwdRate * chip_use(w.wg_fk, cus)), w.atomic / kAtomicRate);
}

// Backward mode plan.  The fused kernel (Method 2: each query-key tile pair
// visited once, dQ by atomics) moves 4*d_s bytes of fp32 atomics per query
// row and 128-key block; on gfx950 device-scope fp32 atomics sustain about
// 1.2 TB/s, so it only pays when the query-outer dQ kernel of the separate
// mode cannot fill the chip (few query rows, long key ranges).
int plan_bwd(const streamkl_shape* s, int causal, int setting, const streamkl_launch* l, int cus) {
  if (l && l->bwd_mode != STREAMKL_BWD_AUTO) return l->bwd_mode;
  if (ragged(s)) {
    // a ragged batch (whole-batch plans only: its elements plan on their
    // own) as the padded batch of its longest lengths, the same in either layout
    streamkl_shape v = element_shape(s, 0);
    v.B = s->B;
    for (int64_t b = 1; b < s->B; ++b) {
      const streamkl_shape e = element_shape(s, b);
      v.n_q = std::max(v.n_q, e.n_q);
      v.n_k = std::max(v.n_k, e.n_k);
    }
    return plan_bwd(&v, causal, setting, nullptr, cus);
  }
  // decode shapes: the fused decode kernel reads each key tile once and adds
  // to dQ once per wave; the separate dQ kernel would get one workgroup per head
  if (decode_shape(s)) return STREAMKL_BWD_FUSED;
  const BwdWork w = bwd_work(s, causal, setting);
  return t_fused(w, cus) < t_separate(w, cus) ? STREAMKL_BWD_FUSED : STREAMKL_BWD_SEPARATE;
}

streamkl_status hip_status(hipError_t e) {
  if (e == hipSuccess) return STREAMKL_OK;
  g_last_hip_error = (int)e;
  return STREAMKL_ERR_HIP;
}

// Clears n floats on the stream (16-byte stores when p and n allow them).
streamkl_status fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return STREAMKL_OK;
  const bool vec = aligned(p, 16) && n % 4 == 0;
  const int64_t m = vec ? n / 4 : n;
  int64_t fb = cdiv(m, 256);
  if (fb > 65536) fb = 65536;
  if (vec) hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)fb), dim3(256), 0, s, reinterpret_cast<float4*>(p), m);
  else hipLaunchKernelGGL(fill_zero_f32_kernel, dim3((unsigned)fb), dim3(256), 0, s, p, m);
  return hip_status(hipGetLastError());
}

// Clears, in every head of an fp32 tensor (heads head_rows rows apart, d
// floats per row), the rows [first, first + n) of each span (first counted
// in head 0; spans with n <= 0 are skipped).
streamkl_status clear_rows(float* p, int64_t heads, int64_t head_rows, int d,
                           const std::vector<std::pair<int64_t, int64_t>>& spans, hipStream_t s) {
  const bool vec = aligned(p, 16) && d % 4 == 0;
  SpanTable t = {};
  t.count = (int)heads;
  t.stride = head_rows * d;
  auto flush = [&]() -> streamkl_status {
    if (t.n == 0) return STREAMKL_OK;
    int64_t longest = 0;
    for (int i = 0; i < t.n; ++i) longest = std::max(longest, t.len[i]);
    // 8192 floats per workgroup, more where the grid would pass 2^23
    // workgroups (a launch holds fewer than 2^32 threads per dimension)
    t.chunk = std::max<int64_t>(8192, (cdiv(longest * heads, int64_t(1) << 23) + 3) / 4 * 4);
    t.nchunk = cdiv(longest, t.chunk);
    hipLaunchKernelGGL(fill_spans_kernel, dim3((unsigned)(heads * t.nchunk), (unsigned)t.n), dim3(256), 0, s, p, t,
                       vec ? 1 : 0);
    t.n = 0;
    return hip_status(hipGetLastError());
  };
  for (const auto& sp : spans) {
    if (sp.second <= 0) continue;
    const int i = t.n++;
    t.base[i] = sp.first * d;
    t.len[i] = sp.second * d;
    if (t.n == kRaggedMax) {
      const streamkl_status st = flush();
      if (st != STREAMKL_OK) return st;
    }
  }
  return flush();
}

// The rows of each batch element b from row0[b] on (the rows its kernels do
// not write), as spans for clear_rows in a query-side (H heads) or
// key-side tensor: padded batches to the padded length, packed batches to
// the element's own length (a packed element has no padding).
std::vector<std::pair<int64_t, int64_t>> rows_past(const streamkl_shape* s, int64_t heads, bool key,
                                                   const std::vector<int64_t>& row0) {
  std::vector<std::pair<int64_t, int64_t>> out;
  for (int64_t b = 0; b < s->B; ++b) {
    if (packed(s)) {
      const int64_t* off = key ? s->k_off : s->q_off;
      out.push_back({off[b] + row0[b], off[b + 1] - off[b] - row0[b]});
    } else {
      const int64_t rows = key ? s->n_k : s->n_q;
      out.push_back({b * heads * rows + row0[b], rows - row0[b]});
    }
  }
  return out;
}

// dK of a model whose key heads are shared is summed with atomics: clear it
// first.  ds: its head dim, g: query heads per key head, ks: key rows per
// head in memory.
streamkl_status clear_shared_dk(float* dK, const streamkl_shape* sh, int ds, int g, int64_t ks, hipStream_t s) {
  if (g <= 1) return STREAMKL_OK;
  return fill_zero(dK, sh->B * (sh->H / g) * ks * (int64_t)ds, s);
}

// ---- ragged batches: per batch element lengths inside padded tensors ----

bool ragged(const streamkl_shape* s) { return s->q_len || s->k_len || s->q_off; }
bool packed(const streamkl_shape* s) { return s->q_off != nullptr; }

// Batch element b as a problem of its own: B = 1, its lengths, no length arrays.
streamkl_shape element_shape(const streamkl_shape* s, int64_t b) {
  streamkl_shape e = *s;
  e.B = 1;
  if (packed(s)) {
    e.n_q = s->q_off[b + 1] - s->q_off[b];
    e.n_k = s->k_off[b + 1] - s->k_off[b];
  } else {
    e.n_q = s->q_len ? s->q_len[b] : s->n_q;
    e.n_k = s->k_len ? s->k_len[b] : s->n_k;
  }
  e.q_len = nullptr;
  e.k_len = nullptr;
  e.q_off = nullptr;
  e.k_off = nullptr;
  return e;
}

int64_t kv_heads(const streamkl_shape* s, int model) {
  const int32_t kv = model == 1 ? s->kv_heads1 : s->kv_heads2;
  return kv > 0 ? kv : s->H;
}

// The first row of batch element b in a query-side tensor (Q, the per-row
// vectors, dQ: H heads) or a key-side tensor (K, dK: kv heads).  Padded
// batches: element b's heads follow element b-1's, n rows each; packed
// batches: the element's first row within head 0 (heads n_q or n_k rows
// apart, the total).  A pointer at that row, with the tensor's head stride
// as the rows per head, addresses the element as a problem of its own.
int64_t qrow(const streamkl_shape* s, int64_t b) { return packed(s) ? s->q_off[b] : b * s->H * s->n_q; }
int64_t krow(const streamkl_shape* s, int64_t b, int64_t kv) { return packed(s) ? s->k_off[b] : b * kv * s->n_k; }

template <typename P>
P at_row(P p, int64_t row, int64_t bytes_per_row) {
  if (!p) return p;
  using C = std::conditional_t<std::is_const_v<std::remove_pointer_t<P>>, const char*, char*>;
  return reinterpret_cast<P>(reinterpret_cast<C>(p) + row * bytes_per_row);
}

// Elements of a ragged batch that run one kernel go to that kernel in few
// launches, each with a table of at most kRaggedMax elements (RaggedTable):
// one launch fills the chip where launches of each element alone would run
// one after another, each short of filling it.  Element ranges are rounded
// up to a multiple of 8 workgroups (the XCD count); the elements with the
// most query-key pairs come first, so the longest workgroups start first.
struct RaggedLaunch {
  RaggedTable t = {};
  int64_t grid = 0;
};

// A grouped launch holds at most the padded batch's workgroups plus 7 per
// element; kept below 2^22 so that its threads (at most 512 per workgroup)
// stay below the 2^32 a launch allows.  Beyond that elements run on their own.
bool groupable(const streamkl_shape* s) {
  constexpr int64_t kMaxWg = int64_t(1) << 22;
  if (!ragged(s)) return false;
  // packed: n_q and n_k are the totals over the elements
  const int64_t wg = packed(s) ? s->H * (cdiv(std::max(s->n_q, s->n_k), 128) + 2 * s->B)
                               : s->B * s->H * (cdiv(std::max(s->n_q, s->n_k), 128) + 1);
  return wg <= kMaxWg;
}

// Elements `els` by query-key pairs per head, the most first, so that the
// longest workgroups of a grouped launch start first.
std::vector<int64_t> by_pairs(const streamkl_shape* s, int causal, const std::vector<int64_t>& els) {
  std::vector<std::pair<double, int64_t>> order;
  for (int64_t b : els) {
    const streamkl_shape e = element_shape(s, b);
    order.push_back({head_pairs(&e, causal), b});
  }
  std::stable_sort(order.begin(), order.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
  std::vector<int64_t> out;
  for (const auto& o : order) out.push_back(o.second);
  return out;
}

// The launches of one kernel over elements `els`; blocks(e): the kernel's
// workgroups per head for element shape e.
template <typename F>
std::vector<RaggedLaunch> ragged_launches(const streamkl_shape* s, int causal, const std::vector<int64_t>& els,
                                          F blocks) {
  std::vector<RaggedLaunch> out;
  for (const int64_t b : by_pairs(s, causal, els)) {
    const streamkl_shape e = element_shape(s, b);
    const int64_t nblk = blocks(e);
    if (out.empty() || out.back().t.n == kRaggedMax) {
      out.emplace_back();
      out.back().t.H = (int)s->H;
    }
    RaggedLaunch& L = out.back();
    const int i = L.t.n++;
    L.t.start[i] = (int)L.grid;
    L.t.b[i] = packed(s) ? 0 : (int)b;  // packed: every element's heads are heads 0 .. H-1
    L.t.n_q[i] = (int)e.n_q;
    L.t.n_k[i] = (int)e.n_k;
    L.t.nblk[i] = (int)nblk;
    L.t.qoff[i] = packed(s) ? (int)s->q_off[b] : 0;
    L.t.koff[i] = packed(s) ? (int)s->k_off[b] : 0;
    L.grid += (s->H * nblk + 7) / 8 * 8;
    L.t.start[i + 1] = (int)L.grid;
  }
  return out;
}

// ---- the problems of one forward call and their workspace ----

constexpr size_t kInvalidBytes = ~(size_t)0;  // workspace queries with invalid arguments

// Problem b of a call: the shape itself, or batch element b of a ragged batch.
int64_t problems(const streamkl_shape* s) { return ragged(s) ? s->B : 1; }
streamkl_shape problem(const streamkl_shape* s, int64_t b) { return ragged(s) ? element_shape(s, b) : *s; }

// A grouped split-K forward of decode-shaped ragged elements: the table, the
// decode kernel's and the merge kernel's workgroups.
struct DecLaunch {
  DecTable t = {};
  int64_t grid = 0, mgrid = 0;
};

// The grouped split-K launches over decode-shaped elements `els` with their
// split counts, at most kRaggedMax elements each, the most pairs first.
std::vector<DecLaunch> dec_launches(const streamkl_shape* s, int causal, const std::vector<int64_t>& els,
                                    const std::vector<int>& splits) {
  std::vector<DecLaunch> out;
  for (const int64_t b : by_pairs(s, causal, els)) {
    const streamkl_shape e = element_shape(s, b);
    const int ns = splits[(size_t)b];
    if (out.empty() || out.back().t.n == kRaggedMax) {
      out.emplace_back();
      out.back().t.H = (int)s->H;
    }
    DecLaunch& L = out.back();
    const int i = L.t.n++;
    L.t.start[i] = (int)L.grid;
    L.t.mstart[i] = (int)L.mgrid;
    L.t.b[i] = packed(s) ? 0 : (int)b;
    L.t.qoff[i] = packed(s) ? (int)s->q_off[b] : 0;
    L.t.koff[i] = packed(s) ? (int)s->k_off[b] : 0;
    L.t.n_q[i] = (int)e.n_q;
    L.t.n_k[i] = (int)e.n_k;
    L.t.nsplit[i] = ns;
    L.t.wsb[i] = L.t.fs;
    L.t.fs += s->H * (int64_t)ns * e.n_q;
    L.grid += (s->H * cdiv(ns, 4) + 7) / 8 * 8;
    L.mgrid += cdiv(s->H * e.n_q, 256);
    L.t.start[i + 1] = (int)L.grid;
    L.t.mstart[i + 1] = (int)L.mgrid;
  }
  return out;
}

struct FwdCall {
  size_t split_region = 0;  // bytes of split partials: the largest of any launch (they run one after another)
  int64_t loss_slots = 0;   // fused-loss partials of all launches (consecutive, after the split region)
  double rows = 0;          // query rows the call finalizes (the mean's divisor)
  std::vector<int64_t> single;          // problems launched on their own, in this order
  std::vector<RaggedLaunch> pp, plain;  // then the unsplit elements of a ragged batch, grouped by forward kernel
  std::vector<DecLaunch> dec;           // then its split decode-shaped elements, grouped
};

// The launches of a forward call with the given split counts and the
// workspace they need.  Loss slots are numbered in launch order: the single
// problems, the grouped ping-pong launches, the grouped 4-wave ones, then
// the merges of the grouped decode launches.  group_dec = false: split
// decode-shaped elements run on their own.
FwdCall summarize(const streamkl_shape* s, int causal, const std::vector<int>& splits, bool group_dec = true) {
  FwdCall c;
  const bool group = groupable(s);
  std::vector<int64_t> pp, plain, dec;
  for (int64_t b = 0; b < problems(s); ++b) {
    const streamkl_shape e = problem(s, b);
    if (e.n_q == 0) continue;
    c.rows += (double)(e.B * e.H * e.n_q);
    if (group && splits[b] == 1) {
      (use_pp(&e) ? pp : plain).push_back(b);
      continue;
    }
    if (group && group_dec && decode_shape(&e)) {
      dec.push_back(b);
      continue;
    }
    const FwdPlan p = make_fwd_plan(&e, splits[b]);
    c.split_region = std::max(c.split_region, p.split_bytes);
    c.loss_slots += p.loss_slots;
    c.single.push_back(b);
  }
  c.pp = ragged_launches(s, causal, pp, [](const streamkl_shape& e) { return cdiv(e.n_q, kFwdPPRows); });
  c.plain = ragged_launches(s, causal, plain, [](const streamkl_shape& e) { return cdiv(e.n_q, kFwdRows); });
  c.dec = dec_launches(s, causal, dec, splits);
  for (const auto* v : {&c.pp, &c.plain})
    for (const RaggedLaunch& L : *v) c.loss_slots += L.grid;
  for (const DecLaunch& L : c.dec) {
    c.split_region = std::max(c.split_region, (size_t)20 * (size_t)L.t.fs);
    c.loss_slots += L.mgrid;
  }
  return c;
}

size_t loss_base(const FwdCall& c) { return round256(c.split_region); }
size_t loss_call_bytes(const FwdCall& c) { return loss_base(c) + 8 * (size_t)c.loss_slots; }

// The split count of every problem (0 for empty ones) as the plan asks, or
// one split.  In a ragged batch that can be grouped (automatic split counts):
// - when the elements other than decode-shaped ones fill the chip without
//   splits in grouped launches, they run unsplit (the plan of an element
//   alone would split a short one);
// - with group_dec, the decode-shaped elements share one split-K launch, with
//   about 64 key blocks (2048 keys) per split, in whole workgroups of 4
//   splits, and at least 8 key blocks per split.  Many short splits, longest
//   elements first, measured faster than a plan that shares out about 4 waves
//   per CU (all resident, one sweep) as for a single problem: the waves of the
//   long elements then outlast the rest.
std::vector<int> planned_splits(const streamkl_shape* s, int causal, const streamkl_launch* l, int cus, bool one,
                                bool group_dec = true) {
  std::vector<int> sp((size_t)problems(s), 0);
  bool fills = false;
  bool dec = false;  // decode-shaped elements to group
  if (groupable(s) && !(l && l->num_splits > 0)) {
    int64_t wg = 0;  // unsplit workgroups of the 4-wave kernel, the measure plan_splits uses
    for (int64_t b = 0; b < s->B; ++b) {
      const streamkl_shape e = element_shape(s, b);
      if (e.n_q == 0) continue;
      if (!decode_shape(&e)) wg += e.H * cdiv(e.n_q, kFwdRows);
      else dec = group_dec;
    }
    fills = wg >= 2 * (int64_t)cus;
  }
  auto dec_splits = [&](const streamkl_shape& e) {
    const int64_t blocks = cdiv(e.n_k, kDecBlock);
    const int64_t n = (cdiv(blocks, 64) + 3) / 4 * 4;
    return (int)std::min<int64_t>(std::min<int64_t>(n, std::max<int64_t>(1, blocks / 8)), 4096);
  };
  for (int64_t b = 0; b < problems(s); ++b) {
    const streamkl_shape e = problem(s, b);
    if (e.n_q == 0) continue;
    if (one) sp[b] = 1;
    else if (dec && decode_shape(&e)) sp[b] = dec_splits(e);
    else if (fills && !decode_shape(&e)) sp[b] = 1;
    else sp[b] = plan_splits(&e, causal, l, cus);
  }
  return sp;
}

// Workspace a call needs with the planned split counts (or one split each):
// the split partials alone, or (loss) the split region then the loss partials.
size_t call_bytes(const streamkl_shape* s, int causal, const streamkl_launch* l, int cus, bool loss, bool one) {
  const FwdCall c = summarize(s, causal, planned_splits(s, causal, l, cus, one));
  return loss ? loss_call_bytes(c) : c.split_region;
}

// The split count of every problem given the workspace the caller offers
// (`avail` bytes at `ws`), decided before anything is enqueued.  Split
// decode-shaped elements of a ragged batch run grouped when all their
// partials fit, else each on its own plan, one after another.  Without the
// loss, a problem whose split partials do not fit falls back to one split
// (auto) or fails (explicit split count); with the loss, the whole call falls
// back to one split when both kinds of partials do not fit, and fails if the
// loss partials alone do not fit.
streamkl_status plan_call(const streamkl_shape* s, int causal, const streamkl_launch* l, int cus, bool loss,
                          const void* ws, size_t avail, std::vector<int>& splits, FwdCall& c) {
  const bool expl = l && l->num_splits > 1;
  splits = planned_splits(s, causal, l, cus, false);
  c = summarize(s, causal, splits);
  if (!loss) {
    const bool usable = ws && aligned(ws, 4);
    if (!c.dec.empty()) {
      if (usable && c.split_region <= avail) return STREAMKL_OK;
      splits = planned_splits(s, causal, l, cus, false, false);
    }
    for (int64_t b = 0; b < problems(s); ++b) {
      if (splits[b] <= 1) continue;
      const streamkl_shape e = problem(s, b);
      if (usable && ws_bytes(&e, splits[b]) <= avail) continue;
      if (expl) return STREAMKL_ERR_WORKSPACE;
      splits[b] = 1;
    }
    c = summarize(s, causal, splits, false);
    return STREAMKL_OK;
  }
  // a ragged batch of empty elements needs no workspace (its loss is 0)
  if (loss_call_bytes(c) == 0) return STREAMKL_OK;
  if (!ws || !aligned(ws, 16)) return STREAMKL_ERR_WORKSPACE;
  if (loss_call_bytes(c) <= avail) return STREAMKL_OK;
  if (!c.dec.empty()) {
    splits = planned_splits(s, causal, l, cus, false, false);
    c = summarize(s, causal, splits, false);
    if (loss_call_bytes(c) <= avail) return STREAMKL_OK;
  }
  if (expl) return STREAMKL_ERR_WORKSPACE;
  splits = planned_splits(s, causal, l, cus, true);
  c = summarize(s, causal, splits);
  return loss_call_bytes(c) <= avail ? STREAMKL_OK : STREAMKL_ERR_WORKSPACE;
}

}  // namespace
}  // namespace streamkl

using namespace streamkl;

extern "C" {

int streamkl_version(void) { return 5; }

const char* streamkl_status_string(int status) {
  switch (status) {
    case STREAMKL_OK: return "ok";
    case STREAMKL_ERR_INVALID: return "invalid argument";
    case STREAMKL_ERR_UNSUPPORTED: return "unsupported shape or device";
    case STREAMKL_ERR_WORKSPACE: return "workspace missing or too small";
    case STREAMKL_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int streamkl_last_hip_error(void) { return g_last_hip_error; }

int streamkl_fwd_plan(const streamkl_shape* shape, int causal, const streamkl_launch* launch) {
  if (check_shape(shape, causal) != STREAMKL_OK) return 0;
  if (launch && launch->num_splits < 0) return 0;
  DeviceInfo d;
  const int cus = device_info(&d) == STREAMKL_OK ? d.cus : 256;
  const void* ws = launch ? launch->workspace : nullptr;
  const size_t avail = launch && ws ? launch->workspace_bytes : 0;
  std::vector<int> splits;
  FwdCall c;
  if (plan_call(shape, causal, launch, cus, false, ws, avail, splits, c) != STREAMKL_OK) return 0;
  int most = 1;  // ragged batches: the largest split count of any element
  for (int sp : splits) most = std::max(most, sp);
  return most;
}

size_t streamkl_fwd_workspace_bytes(const streamkl_shape* shape, int causal, const streamkl_launch* launch) {
  if (check_shape(shape, causal) != STREAMKL_OK) return kInvalidBytes;
  if (launch && launch->num_splits < 0) return kInvalidBytes;
  DeviceInfo d;
  const int cus = device_info(&d) == STREAMKL_OK ? d.cus : 256;
  return call_bytes(shape, causal, launch, cus, false, false);
}

size_t streamkl_fwd_loss_workspace_bytes(const streamkl_shape* shape, int causal, const streamkl_launch* launch) {
  if (check_shape(shape, causal) != STREAMKL_OK) return kInvalidBytes;
  if (launch && launch->num_splits < 0) return kInvalidBytes;
  DeviceInfo d;
  const int cus = device_info(&d) == STREAMKL_OK ? d.cus : 256;
  return call_bytes(shape, causal, launch, cus, true, false);
}

size_t streamkl_bwd_workspace_bytes(const streamkl_shape* shape, int causal, int setting,
                                    const streamkl_launch* launch) {
  if (check_shape(shape, causal) != STREAMKL_OK || (setting != 1 && setting != 2)) return kInvalidBytes;
  if (launch && (launch->num_splits < 0 || launch->bwd_mode < 0 || launch->bwd_mode > 4)) return kInvalidBytes;
  return 0;  // every backward mode runs in the caller's inputs and outputs
}

}  // extern "C"

namespace streamkl {
namespace {

// Arguments every forward launch shares: the problem's tensors, qs and ks
// rows per head in memory (the padded lengths), shape->n_q and shape->n_k the
// rows used.
FwdArgs fwd_args(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal, float scale1,
                 float scale2, float* out_kl, float* out_lse1, float* out_lse2, const streamkl_shape* shape,
                 int64_t qs, int64_t ks, const float* lw) {
  FwdArgs a = {};
  a.q1 = Q1; a.k1 = K1; a.q2 = Q2; a.k2 = K2;
  a.kl = out_kl; a.lse1 = out_lse1; a.lse2 = out_lse2;
  a.lw = lw;
  a.BH = shape->B * shape->H;
  a.n_q = (int)shape->n_q;
  a.n_k = (int)shape->n_k;
  a.qs = (int)qs;
  a.ks = (int)ks;
  a.causal = causal ? 1 : 0;
  a.c1 = log2e_scale(scale1, shape->d1);
  a.c2 = log2e_scale(scale2, shape->d2);
  a.g1 = group1(shape);
  a.g2 = group2(shape);
  return a;
}

// The forward of one problem, validated and planned: qs, ks are the rows per
// head in memory (the padded lengths), sh->n_q, sh->n_k the rows used; split
// partials go to `ws`, fused-loss partials (when lpart is set) to lpart.
streamkl_status fwd_launch(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal, float scale1,
                           float scale2, float* out_kl, float* out_lse1, float* out_lse2, const streamkl_shape* shape,
                           int64_t qs, int64_t ks, const FwdPlan& p, float* ws, const float* lw, double* lpart,
                           hipStream_t s) {
  // Without a key split, long query ranges use the 8-wave ping-pong kernel;
  // split short bf16 query ranges use the decode kernel.
  const DecFwdLaunch fd = p.dec ? pick_fwd_dec(shape->dtype, shape->d1, shape->d2) : nullptr;
  const FwdLaunch fn = p.dec ? nullptr
                       : p.pp ? pick_fwd_pp(shape->dtype, shape->d1, shape->d2)
                              : pick_fwd(shape->dtype, shape->d1, shape->d2);
  if (!fn && !fd) return STREAMKL_ERR_UNSUPPORTED;

  FwdArgs a = fwd_args(Q1, K1, Q2, K2, causal, scale1, scale2, out_kl, out_lse1, out_lse2, shape, qs, ks, lw);
  a.ws = p.splits > 1 ? ws : nullptr;
  a.lpart = p.splits > 1 ? nullptr : lpart;  // split: the merge kernel finalizes the rows
  a.nsplit = p.splits;
  const int unit = p.dec ? kDecBlock : kFwdTile;
  a.keys_per_split = (int)(cdiv(cdiv(shape->n_k, unit), p.splits) * unit);
  a.nqb = (int)p.nqb;
  streamkl_status st = hip_status(fd ? fd(a, p.grid, s, nullptr) : fn(a, p.grid, s, nullptr));
  if (st != STREAMKL_OK || p.splits == 1) return st;
  const int64_t rows = a.BH * a.n_q;
  hipLaunchKernelGGL(splitk_merge_kernel<NoTable>, dim3((unsigned)cdiv(rows, 256)), dim3(256), 0, s,
                     (const float*)a.ws, out_kl, out_lse1, out_lse2, a.BH, a.n_q, p.splits, a.qs, lw, lpart,
                     NoTable{});
  return hip_status(hipGetLastError());
}

// One grouped split-K forward of decode-shaped elements of a ragged batch
// (padded tensors `shape`, whole-batch pointers): the decode kernel writes
// the elements' split partials to `ws` as the table lays them out, then the
// merge kernel finalizes their rows (and writes its loss partials).
streamkl_status dec_group_launch(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                                 float scale1, float scale2, float* out_kl, float* out_lse1, float* out_lse2,
                                 const streamkl_shape* shape, const DecLaunch& L, float* ws, const float* lw,
                                 double* lpart, hipStream_t s) {
  const DecFwdLaunch fd = pick_fwd_dec(shape->dtype, shape->d1, shape->d2);
  if (!fd) return STREAMKL_ERR_UNSUPPORTED;
  FwdArgs a = fwd_args(Q1, K1, Q2, K2, causal, scale1, scale2, out_kl, out_lse1, out_lse2, shape, shape->n_q,
                       shape->n_k, lw);
  a.ws = ws;
  streamkl_status st = hip_status(fd(a, L.grid, s, &L.t));
  if (st != STREAMKL_OK) return st;
  hipLaunchKernelGGL(splitk_merge_kernel<DecTable>, dim3((unsigned)L.mgrid), dim3(256), 0, s, (const float*)ws,
                     out_kl, out_lse1, out_lse2, a.BH, a.n_q, 1, a.qs, lw, lpart, L.t);
  return hip_status(hipGetLastError());
}

// One grouped launch of the unsplit forward over elements of a ragged batch
// (padded tensors `shape`, whole-batch pointers; pp: the ping-pong kernel).
streamkl_status fwd_group_launch(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                                 float scale1, float scale2, float* out_kl, float* out_lse1, float* out_lse2,
                                 const streamkl_shape* shape, bool pp, const RaggedLaunch& L, const float* lw,
                                 double* lpart, hipStream_t s) {
  FwdLaunch fn = pp ? pick_fwd_pp(shape->dtype, shape->d1, shape->d2) : pick_fwd(shape->dtype, shape->d1, shape->d2);
  if (!fn) return STREAMKL_ERR_UNSUPPORTED;
  FwdArgs a = fwd_args(Q1, K1, Q2, K2, causal, scale1, scale2, out_kl, out_lse1, out_lse2, shape, shape->n_q,
                       shape->n_k, lw);
  a.lpart = lpart;
  a.nsplit = 1;
  a.keys_per_split = (int)(cdiv(shape->n_k, kFwdTile) * kFwdTile);  // covers every element's keys
  return hip_status(fn(a, L.grid, s, &L.t));
}

// A whole forward call: every argument and the workspace are checked, and
// every problem planned, before anything is enqueued.  out_loss set: the
// fused loss, sum_i w_i KL_i (or the mean KL without weights) over the rows.
streamkl_status fwd_call(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal, float scale1,
                         float scale2, const float* weights, float* out_kl, float* out_lse1, float* out_lse2,
                         float* out_loss, const streamkl_shape* shape, const streamkl_launch* launch, void* ws,
                         size_t avail, void* stream) {
  streamkl_status st = check_shape(shape, causal);
  if (st != STREAMKL_OK) return st;
  if (!Q1 || !K1 || !Q2 || !K2 || !out_kl || !out_lse1 || !out_lse2) return STREAMKL_ERR_INVALID;
  if (!aligned(Q1, 16) || !aligned(K1, 16) || !aligned(Q2, 16) || !aligned(K2, 16)) return STREAMKL_ERR_INVALID;
  if (!aligned(out_kl, 4) || !aligned(out_lse1, 4) || !aligned(out_lse2, 4)) return STREAMKL_ERR_INVALID;
  if ((out_loss && !aligned(out_loss, 4)) || (weights && !aligned(weights, 4))) return STREAMKL_ERR_INVALID;
  if (!finite_bits(scale1) || !finite_bits(scale2)) return STREAMKL_ERR_INVALID;
  if (launch && (launch->num_splits < 0 || launch->bwd_mode < 0 || launch->bwd_mode > 4)) return STREAMKL_ERR_INVALID;
  DeviceInfo dev;
  st = device_info(&dev);
  if (st != STREAMKL_OK) return st;
  const bool loss = out_loss != nullptr;
  std::vector<int> splits;
  FwdCall c;
  st = plan_call(shape, causal, launch, dev.cus, loss, ws, ws ? avail : 0, splits, c);
  if (st != STREAMKL_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  float* split_ws = static_cast<float*>(ws);
  double* lpart = loss && ws ? reinterpret_cast<double*>(static_cast<char*>(ws) + loss_base(c)) : nullptr;
  if (!ragged(shape)) {
    st = fwd_launch(Q1, K1, Q2, K2, causal, scale1, scale2, out_kl, out_lse1, out_lse2, shape, shape->n_q,
                    shape->n_k, make_fwd_plan(shape, splits[0]), split_ws, weights, lpart, s);
  } else {
    // ragged batch: rows past an element's query length read 0; elements
    // run in grouped launches (unsplit ones by kernel, split decode-shaped
    // ones in split-K launches) or, where a plan or the workspace asks, on
    // their own
    // (packed batches have no padded rows: every row is some element's)
    const int64_t rows = shape->B * shape->H * shape->n_q;
    for (float* o : {out_kl, out_lse1, out_lse2}) {
      if (packed(shape)) break;
      st = fill_zero(o, rows, s);
      if (st != STREAMKL_OK) return st;
    }
    const int64_t es = shape->dtype == STREAMKL_BF16 ? 2 : 4;
    const int64_t kv1 = kv_heads(shape, 1), kv2 = kv_heads(shape, 2);
    int64_t slot = 0;
    for (const int64_t b : c.single) {
      const streamkl_shape e = element_shape(shape, b);
      const FwdPlan p = make_fwd_plan(&e, splits[b]);
      const int64_t qr = qrow(shape, b), k1r = krow(shape, b, kv1), k2r = krow(shape, b, kv2);
      st = fwd_launch(at_row(Q1, qr, es * e.d1), at_row(K1, k1r, es * e.d1), at_row(Q2, qr, es * e.d2),
                      at_row(K2, k2r, es * e.d2), causal, scale1, scale2, at_row(out_kl, qr, 4),
                      at_row(out_lse1, qr, 4), at_row(out_lse2, qr, 4), &e, shape->n_q, shape->n_k, p, split_ws,
                      at_row(weights, qr, 4), lpart ? lpart + slot : nullptr, s);
      if (st != STREAMKL_OK) return st;
      slot += p.loss_slots;
    }
    for (const bool pp : {true, false}) {
      for (const RaggedLaunch& L : pp ? c.pp : c.plain) {
        st = fwd_group_launch(Q1, K1, Q2, K2, causal, scale1, scale2, out_kl, out_lse1, out_lse2, shape, pp, L,
                              weights, lpart ? lpart + slot : nullptr, s);
        if (st != STREAMKL_OK) return st;
        slot += L.grid;
      }
    }
    for (const DecLaunch& L : c.dec) {
      st = dec_group_launch(Q1, K1, Q2, K2, causal, scale1, scale2, out_kl, out_lse1, out_lse2, shape, L, split_ws,
                            weights, lpart ? lpart + slot : nullptr, s);
      if (st != STREAMKL_OK) return st;
      slot += L.mgrid;
    }
  }
  if (st != STREAMKL_OK || !loss) return st;
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, s, (const double*)lpart, c.loss_slots,
                     weights ? 0.0 : c.rows, out_loss);
  return hip_status(hipGetLastError());
}

// Arguments every backward launch shares (the gradient outputs, the scale of
// the model that receives them and the blocks per head aside): rows per head
// in memory qs, ks; shape->n_q and shape->n_k the rows used.
BwdArgs bwd_args(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal, float scale1,
                 float scale2, const float* kl, const float* lse1, const float* lse2, const float* d_kl,
                 const streamkl_shape* shape, int64_t qs, int64_t ks) {
  BwdArgs a = {};
  a.q1 = Q1; a.k1 = K1; a.q2 = Q2; a.k2 = K2;
  a.kl = kl; a.lse1 = lse1; a.lse2 = lse2; a.g = d_kl;
  a.BH = shape->B * shape->H;
  a.n_q = (int)shape->n_q;
  a.n_k = (int)shape->n_k;
  a.qs = (int)qs;
  a.ks = (int)ks;
  a.causal = causal ? 1 : 0;
  a.c1 = log2e_scale(scale1, shape->d1);
  a.c2 = log2e_scale(scale2, shape->d2);
  a.g1 = group1(shape);
  a.g2 = group2(shape);
  return a;
}

// One backward setting of one problem (validated), rows per head qs, ks.
// cleared: the caller has cleared the problem's dQ and dK rows (the rows of
// a ragged batch's element need not be one block of memory).
streamkl_status bwd_launch(int setting, const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                           float scale1, float scale2, const float* kl, const float* lse1, const float* lse2,
                           const float* d_kl, float* dQ, float* dK, const streamkl_shape* shape, int64_t qs,
                           int64_t ks, const streamkl_launch* launch, const DeviceInfo& dev, hipStream_t s,
                           bool cleared = false) {
  DqLaunch fq = pick_dq(shape->dtype, shape->d1, shape->d2);
  DkLaunch fk = pick_dk(shape->dtype, shape->d1, shape->d2);
  if (!fq || !fk) return STREAMKL_ERR_UNSUPPORTED;
  const int mode = plan_bwd(shape, causal, setting, launch, dev.cus);

  BwdArgs a = bwd_args(Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, shape, qs, ks);
  a.dq = dQ; a.dk = dK;
  a.scale_s = setting == 1 ? plain_scale(scale2, shape->d2) : plain_scale(scale1, shape->d1);
  const int64_t nkb = cdiv(a.n_k, kBwdKRows), nqb = cdiv(a.n_q, bwd_rows(shape->dtype == STREAMKL_F32));
  const int ds = setting == 1 ? shape->d2 : shape->d1;
  streamkl_status st;
  if (mode != STREAMKL_BWD_DQ_ONLY && !cleared) {
    st = clear_shared_dk(dK, shape, ds, setting == 1 ? a.g2 : a.g1, ks, s);
    if (st != STREAMKL_OK) return st;
  }
  if (mode == STREAMKL_BWD_FUSED) {
    const DecBwdLaunch fd = decode_shape(shape) ? pick_dec_bwd(shape->dtype, shape->d1, shape->d2) : nullptr;
    if (!cleared) {
      st = fill_zero(dQ, a.BH * qs * (int64_t)ds, s);
      if (st != STREAMKL_OK) return st;
    }
    if (fd) {
      a.nblk = plan_dec_bwd_splits(shape, dev.cus);
      return hip_status(fd(a, setting, a.BH * a.nblk, s, nullptr));
    }
    a.nblk = (int)nkb;
    return hip_status(fk(a, setting, true, a.BH * nkb, s, nullptr));
  }
  if (mode != STREAMKL_BWD_DQ_ONLY) {
    const int64_t nkb8 = cdiv(a.n_k, bwd_rows(shape->dtype == STREAMKL_F32));  // the separate dK kernel's key blocks
    a.nblk = (int)nkb8;
    st = hip_status(fk(a, setting, false, a.BH * nkb8, s, nullptr));
    if (st != STREAMKL_OK) return st;
  }
  if (mode == STREAMKL_BWD_DK_ONLY) return STREAMKL_OK;
  a.nblk = (int)nqb;
  return hip_status(fq(a, setting, a.BH * nqb, s, nullptr));
}

// The joint kernels for one problem (validated, bf16), rows per head qs, ks.
streamkl_status joint_launch(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal, float scale1,
                             float scale2, const float* kl, const float* lse1, const float* lse2, const float* d_kl,
                             float* dQ1, float* dK1, float* dQ2, float* dK2, const streamkl_shape* shape, int64_t qs,
                             int64_t ks, int mode, hipStream_t s, bool cleared = false) {
  DqLaunch fq = pick_dq(shape->dtype, shape->d1, shape->d2);
  DkLaunch fk = pick_dk(shape->dtype, shape->d1, shape->d2);
  if (!fq || !fk) return STREAMKL_ERR_UNSUPPORTED;
  BwdArgs a = bwd_args(Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, shape, qs, ks);
  a.dk = dK1; a.dk2 = dK2;
  a.scale_s = plain_scale(scale1, shape->d1);
  a.scale_s2 = plain_scale(scale2, shape->d2);
  const int64_t nkb = cdiv(a.n_k, kBwdKRows), nqb = cdiv(a.n_q, bwd_rows(false));  // bf16 only
  streamkl_status st;
  if (mode != STREAMKL_BWD_DQ_ONLY) {
    st = cleared ? STREAMKL_OK : clear_shared_dk(dK1, shape, shape->d1, a.g1, ks, s);
    if (st == STREAMKL_OK && !cleared) st = clear_shared_dk(dK2, shape, shape->d2, a.g2, ks, s);
    if (st != STREAMKL_OK) return st;
    a.nblk = (int)nkb;
    st = hip_status(fk(a, 3, false, a.BH * nkb, s, nullptr));
    if (st != STREAMKL_OK || mode == STREAMKL_BWD_DK_ONLY) return st;
  }
  // dQ1 and dQ2: the query-outer kernel once per setting (one kernel holding
  // both accumulators needs more registers than two waves per SIMD allow, and
  // measured slower than these two)
  a.nblk = (int)nqb;
  a.dq = dQ1;
  st = hip_status(fq(a, 2, a.BH * nqb, s, nullptr));
  if (st != STREAMKL_OK) return st;
  a.dq = dQ2;
  a.scale_s = a.scale_s2;
  return hip_status(fq(a, 1, a.BH * nqb, s, nullptr));
}

// Whether the separate-mode backward of a ragged batch runs its elements in
// grouped launches: always for an explicit separate, dK-only or dQ-only
// mode; in the automatic mode when the cost model puts the grouped separate
// kernels (the workgroups of all elements together against the chip) at or
// below each element on its own in its own best mode.  Decode-shaped
// elements keep their decode backward and are left out of the comparison.
bool group_bwd(const streamkl_shape* s, int causal, int setting, const streamkl_launch* l, int cus) {
  if (!groupable(s)) return false;
  const int req = l ? l->bwd_mode : STREAMKL_BWD_AUTO;
  if (req != STREAMKL_BWD_AUTO) return req != STREAMKL_BWD_FUSED;
  BwdWork all;
  double each = 0;
  for (int64_t b = 0; b < s->B; ++b) {
    const streamkl_shape e = element_shape(s, b);
    if (e.n_q == 0 || decode_shape(&e)) continue;
    const BwdWork w = bwd_work(&e, causal, setting);
    all.f_sep += w.f_sep;
    all.wg_dk += w.wg_dk;
    all.wg_dq += w.wg_dq;
    each += std::min(t_separate(w, cus), t_fused(w, cus));
  }
  return all.f_sep > 0 && t_separate(all, cus) <= each;
}

// The separate-mode kernels of one backward setting over elements `els` of a
// ragged batch, in grouped launches on the whole-batch tensors (validated;
// mode: separate, dK only or dQ only; dQ and dK already cleared).
streamkl_status bwd_group(int setting, const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                          float scale1, float scale2, const float* kl, const float* lse1, const float* lse2,
                          const float* d_kl, float* dQ, float* dK, const streamkl_shape* shape,
                          const std::vector<int64_t>& els, int mode, hipStream_t s) {
  DqLaunch fq = pick_dq(shape->dtype, shape->d1, shape->d2);
  DkLaunch fk = pick_dk(shape->dtype, shape->d1, shape->d2);
  if (!fq || !fk) return STREAMKL_ERR_UNSUPPORTED;
  BwdArgs a = bwd_args(Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, shape, shape->n_q, shape->n_k);
  a.dq = dQ; a.dk = dK;
  a.scale_s = setting == 1 ? plain_scale(scale2, shape->d2) : plain_scale(scale1, shape->d1);
  if (mode != STREAMKL_BWD_DQ_ONLY) {
    for (const RaggedLaunch& L :
         ragged_launches(shape, causal, els,
                         [](const streamkl_shape& e) { return cdiv(e.n_k, bwd_rows(e.dtype == STREAMKL_F32)); })) {
      const streamkl_status st = hip_status(fk(a, setting, false, L.grid, s, &L.t));
      if (st != STREAMKL_OK) return st;
    }
  }
  if (mode == STREAMKL_BWD_DK_ONLY) return STREAMKL_OK;
  for (const RaggedLaunch& L :
       ragged_launches(shape, causal, els,
                       [](const streamkl_shape& e) { return cdiv(e.n_q, bwd_rows(e.dtype == STREAMKL_F32)); })) {
    const streamkl_status st = hip_status(fq(a, setting, L.grid, s, &L.t));
    if (st != STREAMKL_OK) return st;
  }
  return STREAMKL_OK;
}

// The decode backward over decode-shaped elements `els` of a ragged batch in
// grouped launches (validated, bf16; dQ rows of these elements cleared whole,
// since the kernel adds to them, dK past each element's key length, or whole
// where key heads are shared).  One workgroup per CU in all, as for a single
// problem: an element gets workgroups per head in proportion to its key
// tiles, at least one and at most one per tile.
streamkl_status dec_bwd_group(int setting, const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                              float scale1, float scale2, const float* kl, const float* lse1, const float* lse2,
                              const float* d_kl, float* dQ, float* dK, const streamkl_shape* shape,
                              const std::vector<int64_t>& els, int cus, hipStream_t s) {
  const DecBwdLaunch fd = pick_dec_bwd(shape->dtype, shape->d1, shape->d2);
  if (!fd) return STREAMKL_ERR_UNSUPPORTED;
  BwdArgs a = bwd_args(Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, shape, shape->n_q, shape->n_k);
  a.dq = dQ; a.dk = dK;
  a.scale_s = setting == 1 ? plain_scale(scale2, shape->d2) : plain_scale(scale1, shape->d1);
  double tiles = 0;  // key tiles of all heads of these elements
  for (int64_t b : els) tiles += (double)shape->H * cdiv(element_shape(shape, b).n_k, kDecBwdTile);
  auto blocks = [&](const streamkl_shape& e) {
    const int64_t t = cdiv(e.n_k, kDecBwdTile);
    const int64_t sp = (int64_t)((double)cus * t / tiles);
    return std::max<int64_t>(1, std::min(sp, t));
  };
  for (const RaggedLaunch& L : ragged_launches(shape, causal, els, blocks)) {
    const streamkl_status st = hip_status(fd(a, setting, L.grid, s, &L.t));
    if (st != STREAMKL_OK) return st;
  }
  return STREAMKL_OK;
}

// The joint kernels over elements `els` of a ragged batch in grouped
// launches (validated, bf16; outputs already cleared).
streamkl_status joint_group(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal, float scale1,
                            float scale2, const float* kl, const float* lse1, const float* lse2, const float* d_kl,
                            float* dQ1, float* dK1, float* dQ2, float* dK2, const streamkl_shape* shape,
                            const std::vector<int64_t>& els, int mode, hipStream_t s) {
  DqLaunch fq = pick_dq(shape->dtype, shape->d1, shape->d2);
  DkLaunch fk = pick_dk(shape->dtype, shape->d1, shape->d2);
  if (!fq || !fk) return STREAMKL_ERR_UNSUPPORTED;
  BwdArgs a = bwd_args(Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, shape, shape->n_q, shape->n_k);
  a.dk = dK1; a.dk2 = dK2;
  a.scale_s = plain_scale(scale1, shape->d1);
  a.scale_s2 = plain_scale(scale2, shape->d2);
  streamkl_status st;
  if (mode != STREAMKL_BWD_DQ_ONLY) {
    for (const RaggedLaunch& L :
         ragged_launches(shape, causal, els, [](const streamkl_shape& e) { return cdiv(e.n_k, kBwdKRows); })) {
      st = hip_status(fk(a, 3, false, L.grid, s, &L.t));
      if (st != STREAMKL_OK) return st;
    }
    if (mode == STREAMKL_BWD_DK_ONLY) return STREAMKL_OK;
  }
  const std::vector<RaggedLaunch> qls =  // the joint backward is bf16 only
      ragged_launches(shape, causal, els, [](const streamkl_shape& e) { return cdiv(e.n_q, bwd_rows(false)); });
  a.dq = dQ1;
  for (const RaggedLaunch& L : qls) {
    st = hip_status(fq(a, 2, L.grid, s, &L.t));
    if (st != STREAMKL_OK) return st;
  }
  a.dq = dQ2;
  a.scale_s = a.scale_s2;
  for (const RaggedLaunch& L : qls) {
    st = hip_status(fq(a, 1, L.grid, s, &L.t));
    if (st != STREAMKL_OK) return st;
  }
  return STREAMKL_OK;
}

}  // namespace
}  // namespace streamkl

extern "C" {

streamkl_status streamkl_fwd(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                             float scale1, float scale2, float* out_kl, float* out_lse1, float* out_lse2,
                             const streamkl_shape* shape, const streamkl_launch* launch, void* stream) {
  return fwd_call(Q1, K1, Q2, K2, causal, scale1, scale2, nullptr, out_kl, out_lse1, out_lse2, nullptr, shape, launch,
                  launch ? launch->workspace : nullptr, launch ? launch->workspace_bytes : 0, stream);
}

streamkl_status streamkl_fwd_loss(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                                  float scale1, float scale2, const float* weights, float* out_kl, float* out_lse1,
                                  float* out_lse2, float* out_loss, const streamkl_shape* shape,
                                  const streamkl_launch* launch, void* stream) {
  return fwd_call(Q1, K1, Q2, K2, causal, scale1, scale2, weights, out_kl, out_lse1, out_lse2, out_loss, shape, launch,
                  launch ? launch->workspace : nullptr, launch ? launch->workspace_bytes : 0, stream);
}

streamkl_status streamkl_fwd_loss_noalloc(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                                          float scale1, float scale2, const float* weights, float* out_kl,
                                          float* out_lse1, float* out_lse2, float* out_loss,
                                          const streamkl_shape* shape, const streamkl_launch* launch, void* stream) {
  // argument errors first (as every entry point), then this device's scratch
  streamkl_status st = check_shape(shape, causal);
  if (st != STREAMKL_OK) return st;
  DeviceInfo dev;
  st = device_info(&dev);
  if (st != STREAMKL_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != STREAMKL_OK) return st;
  // the caller's workspace fields are not used: the library's scratch replaces them
  streamkl_launch l = launch ? *launch : streamkl_launch{0, 0, nullptr, 0};
  l.workspace = nullptr;
  l.workspace_bytes = 0;
  return fwd_call(Q1, K1, Q2, K2, causal, scale1, scale2, weights, out_kl, out_lse1, out_lse2, out_loss, shape, &l, ws,
                  kScratchBytes, stream);
}

int streamkl_bwd_plan(const streamkl_shape* shape, int causal, int setting, const streamkl_launch* launch) {
  if (check_shape(shape, causal) != STREAMKL_OK || (setting != 1 && setting != 2)) return 0;
  if (launch && (launch->bwd_mode < 0 || launch->bwd_mode > 4)) return 0;
  DeviceInfo d;
  const int cus = device_info(&d) == STREAMKL_OK ? d.cus : 256;
  return plan_bwd(shape, causal, setting, launch, cus);
}

streamkl_status streamkl_bwd(int setting, const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                             float scale1, float scale2, const float* kl, const float* lse1, const float* lse2,
                             const float* d_kl, float* dQ, float* dK, const streamkl_shape* shape,
                             const streamkl_launch* launch, void* stream) {
  if (setting != 1 && setting != 2) return STREAMKL_ERR_INVALID;
  streamkl_status st = check_shape(shape, causal);
  if (st != STREAMKL_OK) return st;
  if (launch && (launch->num_splits < 0 || launch->bwd_mode < 0 || launch->bwd_mode > 4)) return STREAMKL_ERR_INVALID;
  const int req = launch ? launch->bwd_mode : STREAMKL_BWD_AUTO;
  const bool need_dq = req != STREAMKL_BWD_DK_ONLY, need_dk = req != STREAMKL_BWD_DQ_ONLY;
  if (!Q1 || !K1 || !Q2 || !K2 || !lse1 || !lse2 || !d_kl) return STREAMKL_ERR_INVALID;
  if ((need_dq && !dQ) || (need_dk && !dK)) return STREAMKL_ERR_INVALID;
  if (setting == 2 && !kl) return STREAMKL_ERR_INVALID;
  if (!aligned(Q1, 16) || !aligned(K1, 16) || !aligned(Q2, 16) || !aligned(K2, 16)) return STREAMKL_ERR_INVALID;
  if (!aligned(lse1, 4) || !aligned(lse2, 4) || !aligned(d_kl, 4) || (kl && !aligned(kl, 4)))
    return STREAMKL_ERR_INVALID;
  if ((dQ && !aligned(dQ, 16)) || (dK && !aligned(dK, 4))) return STREAMKL_ERR_INVALID;
  if (!finite_bits(scale1) || !finite_bits(scale2)) return STREAMKL_ERR_INVALID;
  DeviceInfo dev;
  st = device_info(&dev);
  if (st != STREAMKL_OK) return st;
  if (!pick_dq(shape->dtype, shape->d1, shape->d2) || !pick_dk(shape->dtype, shape->d1, shape->d2))
    return STREAMKL_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!ragged(shape))
    return bwd_launch(setting, Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, dQ, dK, shape,
                      shape->n_q, shape->n_k, launch, dev, s);
  // ragged batch: padded rows of dQ and dK are zero; elements run in grouped
  // launches (separate-mode kernels, or the decode backward) or each as a
  // problem of its own
  const int ds = setting == 1 ? shape->d2 : shape->d1;
  const int64_t kvs = kv_heads(shape, setting == 1 ? 2 : 1);
  const bool shared = (setting == 1 ? group2(shape) : group1(shape)) > 1;
  const bool group = group_bwd(shape, causal, setting, launch, dev.cus);
  // Grouped elements: the separate-mode kernels write every row below the
  // element's lengths (dK of shared key heads aside, summed by atomics), so
  // only the rows past them are cleared.  Decode-shaped elements in the
  // fused (or automatic) mode run the decode backward grouped: it adds to
  // dQ, whose rows are cleared whole, and writes dK.  Other elements run on
  // their own and are cleared whole.
  const bool group_dec = groupable(shape) && (req == STREAMKL_BWD_AUTO || req == STREAMKL_BWD_FUSED);
  std::vector<int64_t> together, dec, single, q0((size_t)shape->B, 0), k0((size_t)shape->B, 0);
  for (int64_t b = 0; b < shape->B; ++b) {
    const streamkl_shape e = element_shape(shape, b);
    if (e.n_q == 0) continue;
    if (group && (req != STREAMKL_BWD_AUTO || !decode_shape(&e))) {
      together.push_back(b);
      q0[b] = e.n_q;
      k0[b] = shared ? 0 : e.n_k;
    } else if (group_dec && decode_shape(&e)) {
      dec.push_back(b);
      k0[b] = shared ? 0 : e.n_k;
    } else {
      single.push_back(b);
    }
  }
  if (need_dq) st = clear_rows(dQ, shape->H, shape->n_q, ds, rows_past(shape, shape->H, false, q0), s);
  if (st == STREAMKL_OK && need_dk) st = clear_rows(dK, kvs, shape->n_k, ds, rows_past(shape, kvs, true, k0), s);
  if (st != STREAMKL_OK) return st;
  const int64_t es = shape->dtype == STREAMKL_BF16 ? 2 : 4;
  const int64_t kv1 = kv_heads(shape, 1), kv2 = kv_heads(shape, 2);
  for (const int64_t b : single) {
    const streamkl_shape e = element_shape(shape, b);
    const int64_t qr = qrow(shape, b), k1r = krow(shape, b, kv1), k2r = krow(shape, b, kv2), ksr = krow(shape, b, kvs);
    st = bwd_launch(setting, at_row(Q1, qr, es * e.d1), at_row(K1, k1r, es * e.d1), at_row(Q2, qr, es * e.d2),
                    at_row(K2, k2r, es * e.d2), causal, scale1, scale2, at_row(kl, qr, 4), at_row(lse1, qr, 4),
                    at_row(lse2, qr, 4), at_row(d_kl, qr, 4), at_row(dQ, qr, 4 * ds), at_row(dK, ksr, 4 * ds), &e,
                    shape->n_q, shape->n_k, launch, dev, s, true);
    if (st != STREAMKL_OK) return st;
  }
  if (!dec.empty()) {
    st = dec_bwd_group(setting, Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, dQ, dK, shape, dec,
                       dev.cus, s);
    if (st != STREAMKL_OK) return st;
  }
  if (together.empty()) return STREAMKL_OK;
  return bwd_group(setting, Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, dQ, dK, shape, together,
                   req == STREAMKL_BWD_AUTO ? STREAMKL_BWD_SEPARATE : req, s);
}

streamkl_status streamkl_bwd_joint(const void* Q1, const void* K1, const void* Q2, const void* K2, int causal,
                                   float scale1, float scale2, const float* kl, const float* lse1, const float* lse2,
                                   const float* d_kl, float* dQ1, float* dK1, float* dQ2, float* dK2,
                                   const streamkl_shape* shape, const streamkl_launch* launch, void* stream) {
  streamkl_status st = check_shape(shape, causal);
  if (st != STREAMKL_OK) return st;
  if (launch && (launch->num_splits < 0 || launch->bwd_mode < 0 || launch->bwd_mode > 4)) return STREAMKL_ERR_INVALID;
  const int req = launch ? launch->bwd_mode : STREAMKL_BWD_AUTO;
  const bool need_dq = req != STREAMKL_BWD_DK_ONLY, need_dk = req != STREAMKL_BWD_DQ_ONLY;
  if (!Q1 || !K1 || !Q2 || !K2 || !kl || !lse1 || !lse2 || !d_kl) return STREAMKL_ERR_INVALID;
  if ((need_dq && (!dQ1 || !dQ2)) || (need_dk && (!dK1 || !dK2))) return STREAMKL_ERR_INVALID;
  if (!aligned(Q1, 16) || !aligned(K1, 16) || !aligned(Q2, 16) || !aligned(K2, 16)) return STREAMKL_ERR_INVALID;
  if (!aligned(kl, 4) || !aligned(lse1, 4) || !aligned(lse2, 4) || !aligned(d_kl, 4)) return STREAMKL_ERR_INVALID;
  if ((dQ1 && !aligned(dQ1, 16)) || (dQ2 && !aligned(dQ2, 16)) || (dK1 && !aligned(dK1, 4)) ||
      (dK2 && !aligned(dK2, 4)))
    return STREAMKL_ERR_INVALID;
  if (!finite_bits(scale1) || !finite_bits(scale2)) return STREAMKL_ERR_INVALID;
  DeviceInfo dev;
  st = device_info(&dev);
  if (st != STREAMKL_OK) return st;
  const int mode = plan_bwd(shape, causal, 1, launch, dev.cus);
  if (shape->dtype != STREAMKL_BF16 || mode == STREAMKL_BWD_FUSED) {
    // one pass per setting (every argument above is what each pass checks)
    st = streamkl_bwd(2, Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, dQ1, dK1, shape, launch, stream);
    if (st != STREAMKL_OK) return st;
    return streamkl_bwd(1, Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, dQ2, dK2, shape, launch,
                        stream);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!ragged(shape))
    return joint_launch(Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, dQ1, dK1, dQ2, dK2, shape,
                        shape->n_q, shape->n_k, mode, s);
  const int64_t kv1 = kv_heads(shape, 1), kv2 = kv_heads(shape, 2);
  if (groupable(shape)) {
    // every non-empty element in grouped launches: only the rows past its
    // lengths are cleared (dK of shared key heads whole: summed by atomics)
    std::vector<int64_t> els, q0((size_t)shape->B, 0), k01((size_t)shape->B, 0), k02((size_t)shape->B, 0);
    for (int64_t b = 0; b < shape->B; ++b) {
      const streamkl_shape e = element_shape(shape, b);
      if (e.n_q == 0) continue;
      els.push_back(b);
      q0[b] = e.n_q;
      k01[b] = group1(shape) > 1 ? 0 : e.n_k;
      k02[b] = group2(shape) > 1 ? 0 : e.n_k;
    }
    if (need_dq) {
      st = clear_rows(dQ1, shape->H, shape->n_q, shape->d1, rows_past(shape, shape->H, false, q0), s);
      if (st == STREAMKL_OK)
        st = clear_rows(dQ2, shape->H, shape->n_q, shape->d2, rows_past(shape, shape->H, false, q0), s);
    }
    if (st == STREAMKL_OK && need_dk) {
      st = clear_rows(dK1, kv1, shape->n_k, shape->d1, rows_past(shape, kv1, true, k01), s);
      if (st == STREAMKL_OK) st = clear_rows(dK2, kv2, shape->n_k, shape->d2, rows_past(shape, kv2, true, k02), s);
    }
    if (st != STREAMKL_OK || els.empty()) return st;
    return joint_group(Q1, K1, Q2, K2, causal, scale1, scale2, kl, lse1, lse2, d_kl, dQ1, dK1, dQ2, dK2, shape, els,
                       mode, s);
  }
  const int64_t nb = packed(shape) ? 1 : shape->B;  // a packed tensor has no batch dimension
  const int64_t BHQ = nb * shape->H * shape->n_q;
  if (need_dq) {
    st = fill_zero(dQ1, BHQ * shape->d1, s);
    if (st == STREAMKL_OK) st = fill_zero(dQ2, BHQ * shape->d2, s);
  }
  if (st == STREAMKL_OK && need_dk) {
    st = fill_zero(dK1, nb * kv1 * shape->n_k * shape->d1, s);
    if (st == STREAMKL_OK) st = fill_zero(dK2, nb * kv2 * shape->n_k * shape->d2, s);
  }
  if (st != STREAMKL_OK) return st;
  const int64_t es = 2;
  const int d1 = shape->d1, d2 = shape->d2;
  for (int64_t b = 0; b < shape->B; ++b) {
    const streamkl_shape e = element_shape(shape, b);
    if (e.n_q == 0) continue;
    const int64_t qr = qrow(shape, b), k1r = krow(shape, b, kv1), k2r = krow(shape, b, kv2);
    st = joint_launch(at_row(Q1, qr, es * d1), at_row(K1, k1r, es * d1), at_row(Q2, qr, es * d2),
                      at_row(K2, k2r, es * d2), causal, scale1, scale2, at_row(kl, qr, 4), at_row(lse1, qr, 4),
                      at_row(lse2, qr, 4), at_row(d_kl, qr, 4), at_row(dQ1, qr, 4 * d1), at_row(dK1, k1r, 4 * d1),
                      at_row(dQ2, qr, 4 * d2), at_row(dK2, k2r, 4 * d2), &e, shape->n_q, shape->n_k, mode, s, true);
    if (st != STREAMKL_OK) return st;
  }
  return STREAMKL_OK;
}

streamkl_status streamkl_kl_loss(const float* kl, const float* weights, int64_t rows, float* out, void* stream) {
  if (!kl || !out || rows < 1) return STREAMKL_ERR_INVALID;
  if (!aligned(kl, 4) || !aligned(out, 4) || (weights && !aligned(weights, 4))) return STREAMKL_ERR_INVALID;
  DeviceInfo dev;
  streamkl_status st = device_info(&dev);
  if (st != STREAMKL_OK) return st;
  hipLaunchKernelGGL(kl_loss_kernel, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), kl, weights, rows, out);
  return hip_status(hipGetLastError());
}

}  // extern "C"
