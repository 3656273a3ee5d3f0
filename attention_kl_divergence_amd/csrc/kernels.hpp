// StreamKL kernels for gfx950: one-pass forward (optionally split over keys),
// key-outer backward (dK, optionally fused dQ by atomics) and query-outer
// backward (dQ).
//
// Pages: "StreamKL" technical summary (gist.science ja/fr/ko).
//   Method 1 (online formulation): five running scalars per row and
//     L = acc/l1 + LSE2 - LSE1, LSE_t = m_t + log l_t; key tiles past the
//     causal boundary are skipped.
//   Method 2 (recomputation strategy): only KL, LSE1, LSE2 are stored;
//     P_t = exp(S_t - LSE_t) is regenerated tile by tile; setting 1 trains
//     P2 against a fixed P1, setting 2 trains P1 against a fixed P2; the fused
//     backward visits each query-key tile pair once and accumulates dQ with
//     atomics, with separate dK and dQ kernels as the fallback.
//   Method 3 (GPU kernel optimisations): split-K over the key dimension for
//     few query rows; the setting-2 log-ratio is built from logit
//     differences and the stored LSE, never from log P.
//
// Everything runs in base-2 units: y_t = S_t * log2(e) = s * c_t with
// c_t = scale_t * log2(e) applied to the raw dot product s in fp32, so each
// exponential is one v_exp_f32.
//
// Data movement: tiles of Q or K rows go HBM -> LDS with direct 16-byte
// global->LDS loads (no VGPR staging), double-buffered so the next tile is in
// flight while the current one is consumed, one barrier per tile.  Inside a
// tile, 16-byte chunks of a row are XOR-swizzled by row so MFMA fragment reads
// spread over all LDS banks.  Operands that need a column of a row-major tile
// (k running down the rows) are read with the LDS transpose read
// (ds_read_b64_tr_b16), so no tile is ever stored transposed.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace streamkl {

struct FwdArgs {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  float* kl;
  float* lse1;
  float* lse2;
  float* ws;           // split partials [5][BH][nsplit][n_q], used when nsplit > 1
  const float* lw;     // fused loss: per-row weights [BH][qs] (NULL: weight 1)
  double* lpart;       // fused loss: one partial sum per finalizing workgroup (NULL: no loss)
  int64_t BH;
  int n_q, n_k;
  int nsplit;
  int keys_per_split;  // multiple of the key tile
  int nqb;             // query blocks per head
  int causal;
  float c1, c2;        // scale_t * log2(e)
  int g1, g2;          // query heads per key head of each model (1: no sharing)
  int qs, ks;          // rows per head in memory of Q (and the per-row vectors) and of K: n_q and
                       // n_k, or more when the batch element's lengths are padded
};

struct BwdArgs {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  const float* kl;
  const float* lse1;
  const float* lse2;
  const float* g;
  float* dq;           // setting 1: dQ2; setting 2: dQ1
  float* dk;           // setting 1: dK2; settings 2 and 3 (joint): dK1
  float* dk2;          // joint: dK2
  int64_t BH;
  int n_q, n_k;
  int nblk;            // query blocks (dQ kernel), key blocks (dK kernel) or workgroups (decode backward) per head
  int causal;
  float c1, c2;        // scale_t * log2(e)
  float scale_s;       // scale of the model that receives gradients (joint: model 1)
  float scale_s2;      // joint: scale of model 2
  int g1, g2;          // query heads per key head of each model (1: no sharing)
  int qs, ks;          // rows per head in memory of Q, dQ and the per-row vectors, and of K and dK
};

typedef __bf16 bf16x4_lds __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Swizzled LDS tile of row-major [rows][D] elements.  Chunk = 16 bytes.
// The swizzle spreads (a) 16 consecutive rows read at one chunk (MFMA row
// fragments) and (b) 4 consecutive rows read at two adjacent chunks (the
// transpose reads) over distinct 16-byte bank groups of a 256-byte window.
template <typename T, int D>
struct Tile {
  static constexpr int EPC = 16 / sizeof(T);               // elements per chunk
  static constexpr int CPR = D / EPC;                      // chunks per row
  static constexpr int RP = CPR >= 16 ? 1 : 16 / CPR;      // rows sharing a 256-byte bank window
  static constexpr int CW = CPR >= 16 ? 16 : CPR;          // chunks of a row within one window
  __device__ static inline int swz(int r) {
    const int j = r / RP;
    return ((j & (CW / 2 - 1)) << 1) | ((j / (CW / 2)) & 1);
  }
  // element offset of (row r, column c)
  __device__ static inline int off(int r, int c) { return r * D + (((c / EPC) ^ swz(r)) * EPC) + (c % EPC); }
};

// Direct global->LDS loads of ROWS rows of a [*, D] global tensor into an LDS
// tile.  Each wave-wide 16-byte buffer load fills 1 KB of LDS (lane L writes
// bytes [16L, 16L+16) of it), so each lane fetches the global chunk that
// belongs at that swizzled spot; those per-lane byte offsets are fixed for the
// kernel.  Per tile only the buffer resource changes (scalar work): its base
// is the tile's first row and its size the tile's rows that exist (at most
// ROWS rows, so it always fits the 32-bit size field), so rows past the end
// read as zeros.
template <typename T, int D, int ROWS, int NW>
struct TileLoader {
  using F = Tile<T, D>;
  static constexpr int NI = ROWS * F::CPR / 64;       // wave-wide loads per tile
  static constexpr int PER = (NI + NW - 1) / NW;       // loads per wave (the last waves may idle)
  static_assert(NI * 64 == ROWS * F::CPR, "a tile must be whole 1 KB blocks");
  int voff[PER];
  int wave;
  __device__ __forceinline__ TileLoader(int wave_, int lane) : wave(wave_) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int P = (wave * PER + i) * 64 + lane;
      const int r = P / F::CPR, pc = P % F::CPR;
      voff[i] = (r * D + (pc ^ F::swz(r)) * F::EPC) * (int)sizeof(T);
    }
  }
  // rows [r0, r0 + ROWS) of g (a tensor with nrows rows) into `tile`
  __device__ __forceinline__ void issue(T* tile, const T* g, int r0, int nrows) const {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer-resource type exists only in the device pass
    const int left = min(nrows - r0, ROWS);
    const uint32_t bytes = left > 0 ? (uint32_t)left * (uint32_t)(D * sizeof(T)) : 0u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(g + (int64_t)r0 * D), (short)0, (int)bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (NI % NW == 0 || wave * PER + i < NI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(tile + (wave * PER + i) * 64 * F::EPC), 16, voff[i], 0, 0, 0);
#endif
  }
};

// Key head of query head bh (of B*H < 2^20) when g query heads share one:
// a 32-bit division, far shorter than a 64-bit one.
__device__ __forceinline__ int64_t key_head(int64_t bh, int g) { return (int64_t)((uint32_t)bh / (uint32_t)g); }

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Work item (head, block) of workgroup `lin` of a grid of BH * nblk.
// Workgroups go to the 8 XCDs round-robin (workgroup i runs on XCD i % 8) and
// each XCD has its own L2.  When the heads split evenly over the XCDs, XCD x
// takes heads [x BH/8, (x+1) BH/8) one after the other, so the workgroups it
// runs at a time share one head's tiles in its L2; otherwise the heads
// interleave.  Within a head, blocks come in order 0, 1, ..., and the caller
// maps that to its longest-first order.
struct WorkItem {
  int64_t bh;
  int blk;
};
__device__ __forceinline__ WorkItem work_item(int64_t lin, int64_t BH, int nblk) {
  constexpr int X = 8;
  if (BH % X == 0) {
    const int64_t per = BH / X * nblk;
    const int64_t v = (lin % X) * per + lin / X;
    return {v / nblk, (int)(v % nblk)};
  }
  return {lin % BH, (int)(lin / BH)};
}

// Ragged batches in one launch.  The elements of a batch that run the same
// kernel go in one table, passed as a kernel argument beside the problem's.
// Element i owns workgroups [start[i], start[i+1]), a range whose length is
// a multiple of 8, so each workgroup sits on the XCD it would have in a
// launch of that element alone.  Within its range a workgroup serves
// element b[i] (query heads b[i] H .. b[i] H + H - 1 of the padded tensors)
// exactly as in such a launch, with that element's lengths and blocks per
// head.  The workgroups past an element's H * nblk are padding and leave at
// once.  In a packed batch the elements' rows lie one after another in each
// head (heads qs and ks rows apart): b[i] is 0 and qoff[i], koff[i] are the
// element's first rows, added to every row index.
constexpr int kRaggedMax = 64;
struct RaggedTable {
  int n;                     // elements in the table (0: not ragged)
  int H;                     // query heads per element
  int start[kRaggedMax + 1];
  int b[kRaggedMax];         // batch index of each element
  int n_q[kRaggedMax], n_k[kRaggedMax];
  int nblk[kRaggedMax];      // the kernel's blocks per head for the element
  int qoff[kRaggedMax];      // packed batches: the element's first query row within a head (else 0)
  int koff[kRaggedMax];      // and its first key row
};

// The table type of a plain launch: no table.  Kernels take the table type
// as a template parameter, so a plain launch compiles without the ragged
// prologue and its code is unchanged by it.
struct NoTable {};
template <typename RT>
constexpr bool kRagged = std::is_same<RT, RaggedTable>::value;

struct RaggedItem {
  int64_t lin;    // workgroup index within the element's range
  int64_t head0;  // the element's first query head, b H (0 in a packed batch)
  int n_q, n_k, nblk;
  int qoff, koff;  // the element's first query and key rows within a head
  bool pad;       // a padding workgroup
};

// the element of a table whose range [start[e], start[e+1]) holds lin
__device__ __forceinline__ int table_elem(const int* start, int n, int64_t lin) {
  int e = 0;
#pragma unroll 1
  for (int i = 1; i < n; ++i) e = lin >= start[i] ? i : e;
  return e;
}

__device__ __forceinline__ RaggedItem ragged_item(const RaggedTable& rt, int64_t lin) {
  const int e = table_elem(rt.start, rt.n, lin);
  RaggedItem r;
  r.lin = lin - rt.start[e];
  r.head0 = (int64_t)rt.b[e] * rt.H;
  r.n_q = rt.n_q[e];
  r.n_k = rt.n_k[e];
  r.nblk = rt.nblk[e];
  r.qoff = rt.qoff[e];
  r.koff = rt.koff[e];
  r.pad = r.lin >= (int64_t)rt.H * r.nblk;
  return r;
}

// Decode-shaped elements of a ragged batch in one split-K forward launch and
// one merge launch.  Element i has nsplit[i] key splits per head, 4 per
// decode workgroup: it owns decode workgroups [start[i], start[i+1]) (its H
// heads' workgroups, the range rounded up to a multiple of 8) and merge
// workgroups [mstart[i], mstart[i+1]) (256 of its H n_q[i] rows each).  Its
// split partials are rows [wsb[i], wsb[i] + H nsplit[i] n_q[i]) of each of
// the five fields, laid out as a single problem's, fields fs rows apart.
struct DecTable {
  int n;
  int H;
  int64_t fs;
  int start[kRaggedMax + 1];
  int mstart[kRaggedMax + 1];
  int b[kRaggedMax];
  int n_q[kRaggedMax], n_k[kRaggedMax];
  int nsplit[kRaggedMax];
  int64_t wsb[kRaggedMax];
  int qoff[kRaggedMax], koff[kRaggedMax];  // as in RaggedTable
};
template <typename RT>
constexpr bool kDecTable = std::is_same<RT, DecTable>::value;

// Fused loss (the distillation objective sum_i w_i KL_i): each workgroup that
// finalizes rows writes the sum of w_i KL_i over its rows to its own slot, in
// a fixed order (a butterfly over the wave's lanes, which leaves the same bits
// in every lane, then the waves in index order), so the result does not depend
// on scheduling.  v is this thread's w_i KL_i (0 if it finalized no row).
// `red` is NW doubles of LDS the caller has made free for this.
template <int NW>
__device__ __forceinline__ void loss_partial(double v, double* red, double* slot, int tid) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w];
    *slot = t;
  }
}

__device__ __forceinline__ double loss_term(const FwdArgs& a, int64_t r, float kl) {
  return a.lw ? (double)a.lw[r] * (double)kl : (double)kl;
}

// Barrier between the compute phases of a ping-pong loop.  It orders no
// memory (each phase reads data a tile barrier already published), so unlike
// __syncthreads it does not wait for the direct-to-LDS tile loads in flight.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier that publishes this wave's LDS stores to the workgroup, again
// without waiting for the tile loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// MFMA operand with lane row = `row`, k from `k0`: natural layout read.
template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag frag_tile(const T* tile, int row, int s, int grp) {
  const int k = s * Mfma<T>::KSTEP + grp * Mfma<T>::KPL;
  return *reinterpret_cast<const typename Mfma<T>::frag*>(tile + Tile<T, D>::off(row, k));
}

// MFMA operand whose lane column is n (0..31 within block n0) and whose k
// values run down the rows of a row-major tile, in accumulator order
// (k = acc_row(h*KPL + e', grp) + kb0).  bf16 uses two transpose reads.
template <int D>
__device__ __forceinline__ bf16x8 fragcol_acc_bf16(const bf16* __restrict__ tile, int kb0, int n0, int h, int lane) {
  using F = Tile<bf16, D>;
  const int grp = lane >> 5, sub = (lane >> 4) & 1, r = lane & 15;
  const int n = n0 + 16 * sub + 4 * (r & 3);
  const int ka = kb0 + 16 * h + 4 * grp + (r >> 2);
  const bf16x4_lds lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4_lds __attribute__((address_space(3)))*)(tile + F::off(ka, n)));
  const bf16x4_lds hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4_lds __attribute__((address_space(3)))*)(tile + F::off(ka + 8, n)));
  bf16x8 f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

// Same, natural k order (k = kb0 + 16h + 8grp + e').
template <int D>
__device__ __forceinline__ bf16x8 fragcol_nat_bf16(const bf16* __restrict__ tile, int kb0, int n0, int h, int lane) {
  using F = Tile<bf16, D>;
  const int grp = lane >> 5, sub = (lane >> 4) & 1, r = lane & 15;
  const int n = n0 + 16 * sub + 4 * (r & 3);
  const int ka = kb0 + 16 * h + 8 * grp + (r >> 2);
  const bf16x4_lds lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4_lds __attribute__((address_space(3)))*)(tile + F::off(ka, n)));
  const bf16x4_lds hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4_lds __attribute__((address_space(3)))*)(tile + F::off(ka + 4, n)));
  bf16x8 f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

// fp32 versions: one element per lane, k = acc_row(h, grp) (+kb0) or 2h + grp.
template <int D>
__device__ __forceinline__ float fragcol_acc_f32(const float* tile, int kb0, int n0, int h, int lane) {
  return tile[Tile<float, D>::off(kb0 + acc_row(h, lane >> 5), n0 + (lane & 31))];
}
template <int D>
__device__ __forceinline__ float fragcol_nat_f32(const float* tile, int kb0, int n0, int h, int lane) {
  return tile[Tile<float, D>::off(kb0 + 2 * h + (lane >> 5), n0 + (lane & 31))];
}

template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag fragcol_acc(const T* tile, int kb0, int n0, int h, int lane) {
  if constexpr (Mfma<T>::KPL == 1) return fragcol_acc_f32<D>(tile, kb0, n0, h, lane);
  else return fragcol_acc_bf16<D>(tile, kb0, n0, h, lane);
}
template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag fragcol_nat(const T* tile, int kb0, int n0, int h, int lane) {
  if constexpr (Mfma<T>::KPL == 1) return fragcol_nat_f32<D>(tile, kb0, n0, h, lane);
  else return fragcol_nat_bf16<D>(tile, kb0, n0, h, lane);
}

// Per-lane byte offsets of the bf16 operand reads of a swizzled tile, for the
// rows of its first 32-row block.  The swizzle repeats every 16 rows, so any
// other block (and another tile buffer) is a constant away: with a constant
// tile base every read is one LDS instruction with an immediate offset and no
// address arithmetic.  The offsets are hidden from the optimiser so they stay
// in registers instead of being recomputed per read.
template <int D, int S>
struct RowFragOffsets {  // operand rows: frag_tile(tile, 32 * blk + col, s, grp)
  int o[S];
  __device__ __forceinline__ RowFragOffsets(int col, int grp) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      o[s] = Tile<bf16, D>::off(col, s * Mfma<bf16>::KSTEP + grp * Mfma<bf16>::KPL) * (int)sizeof(bf16);
      asm volatile("" : "+v"(o[s]));
    }
  }
  __device__ __forceinline__ bf16x8 read(const bf16* tile, int blk, int s) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile + 32 * blk * D) + o[s]);
  }
  // called once per loop iteration: the offsets then look loop-variant, so
  // the optimiser does not hoist tile base + offset sums into extra registers
  __device__ __forceinline__ void touch() {
#pragma unroll
    for (int s = 0; s < S; ++s) asm volatile("" : "+v"(o[s]));
  }
};

template <int D, int NB>
struct ColFragOffsets {  // column operands: fragcol_acc_bf16(tile, 32 * blk, 32 * nb, h, lane)
  int lo[NB], hi[NB];
  __device__ __forceinline__ ColFragOffsets(int lane) {
    const int grp = lane >> 5, sub = (lane >> 4) & 1, r = lane & 15;
    const int ka = 4 * grp + (r >> 2);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = 32 * nb + 16 * sub + 4 * (r & 3);
      lo[nb] = Tile<bf16, D>::off(ka, n) * (int)sizeof(bf16);
      hi[nb] = Tile<bf16, D>::off(ka + 8, n) * (int)sizeof(bf16);
      asm volatile("" : "+v"(lo[nb]), "+v"(hi[nb]));
    }
  }
  __device__ __forceinline__ bf16x8 read(const bf16* __restrict__ tile, int blk, int nb, int h) const {
    const char* b = reinterpret_cast<const char*>(tile + (32 * blk + 16 * h) * D);
    const bf16x4_lds l = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (bf16x4_lds __attribute__((address_space(3)))*)(b + lo[nb]));
    const bf16x4_lds u = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (bf16x4_lds __attribute__((address_space(3)))*)(b + hi[nb]));
    bf16x8 f;
    f[0] = l[0]; f[1] = l[1]; f[2] = l[2]; f[3] = l[3];
    f[4] = u[0]; f[5] = u[1]; f[6] = u[2]; f[7] = u[3];
    return f;
  }
  __device__ __forceinline__ void touch() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(lo[nb]), "+v"(hi[nb]));
  }
};

struct NoOffsets {  // stand-in for the offset tables where they are not used (fp32 tiles)
  __device__ __forceinline__ NoOffsets(int) {}
  __device__ __forceinline__ NoOffsets(int, int) {}
  __device__ __forceinline__ void touch() {}
};

template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag zero_frag() {
  typename Mfma<T>::frag f;
  if constexpr (Mfma<T>::KPL == 1) {
    f = 0.f;
  } else {
#pragma unroll
    for (int e = 0; e < Mfma<T>::KPL; ++e) f[e] = (T)0.f;
  }
  return f;
}

// Fragment of a row of a global row-major [*, D] tensor (row clamped to a
// valid one; `valid` false gives zeros).
template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag frag_global(const T* g, int row, int rmax, bool valid, int s, int grp) {
  const T* p = g + (int64_t)min(row, rmax) * D + s * Mfma<T>::KSTEP + grp * Mfma<T>::KPL;
  typename Mfma<T>::frag f = *reinterpret_cast<const typename Mfma<T>::frag*>(p);
  return valid ? f : zero_frag<T>();
}


// ---------------------------------------------------------------------------
// bf16 dQ under a key offset shared by every key.  Every row of dS sums to
// zero (setting 1: sum_j (P2 - P1) = 0; setting 2: sum_j P1 (r - KL) = 0,
// Method 2), so dQ_i = sum_j dS_ij K_j = sum_j dS_ij (K_j - kbar) for any
// vector kbar.  The matrix instruction takes dS rounded to bf16, and those
// rounding errors do not sum to zero: a component u common to all keys
// would reach dQ as (sum_j bf16(dS_ij)) u, however large u is against the
// spread of the keys.  The dQ paths therefore either subtract
// r_i kbar with r_i = sum_j bf16(dS_ij) (the exact values fed to the
// product), or feed K_j - kbar to the product; either way the rounding error
// is relative to K - kbar instead of K.  kbar is the mean of the head's first
// min(64, n_k) key rows, summed in row order by ref_key_col, so every
// workgroup that adds into one dQ row gets bitwise the same kbar.
constexpr int kRefKeys = 64;

__device__ __forceinline__ float ref_key_col(const bf16* K, int D, int n_k, int c) {
  float s = 0.f;
  if (n_k >= kRefKeys) {  // unrolled so the loads go out together; the same row order
#pragma unroll 16
    for (int j = 0; j < kRefKeys; ++j) s += (float)K[(int64_t)j * D + c];
    return s * (1.f / kRefKeys);
  }
  for (int j = 0; j < n_k; ++j) s += (float)K[(int64_t)j * D + c];
  return s / (float)n_k;
}

// kbar[c] for every column c < D, spread over nthreads threads (the caller
// publishes it with a barrier)
template <int D>
__device__ __forceinline__ void ref_key(float* kbar, const bf16* K, int n_k, int tid, int nthreads) {
  for (int c = tid; c < D; c += nthreads) kbar[c] = ref_key_col(K, D, n_k, c);
}

// acc + the sum of the eight bf16 values of an operand fragment (exact
// products with 1.0, fp32 accumulation)
__device__ __forceinline__ float sum_frag(const bf16x8& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[0], f[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[2], f[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[4], f[5]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[6], f[7]}, one, acc, false);
  return acc;
}
__device__ __forceinline__ float sum_frag(float, float acc) { return acc; }

// Scheduling pattern for a run of N matrix instructions that each consume R
// LDS reads: issue the reads for the first AHEAD instructions, then alternate
// one instruction with the reads of the instruction AHEAD places later, so
// LDS latency hides behind the matrix pipeline.  Placed after the code it
// orders, inside the same basic block.
template <int N, int R, int AHEAD>
__device__ __forceinline__ void sched_mfma_lds() {
  constexpr int PRE = AHEAD < N ? AHEAD : N;
  __builtin_amdgcn_sched_group_barrier(0x100, PRE * R, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + PRE < N) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
}
// ---------------------------------------------------------------------------
// Per-lane maxima of raw logits: chains of max(max(acc, a), b), one v_max3
// per two values.
template <int NKB>
__device__ __forceinline__ void fwd_tile_max(const f32x16 (&s1)[NKB], const f32x16 (&s2)[NKB], float& mx1, float& mx2) {
  float mx1a = kNegInf, mx1b = kNegInf, mx2a = kNegInf, mx2b = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      mx1a = fmaxf(fmaxf(mx1a, s1[kb][e]), s1[kb][e + 1]);
      mx1b = fmaxf(fmaxf(mx1b, s1[kb][e + 2]), s1[kb][e + 3]);
      mx2a = fmaxf(fmaxf(mx2a, s2[kb][e]), s2[kb][e + 1]);
      mx2b = fmaxf(fmaxf(mx2b, s2[kb][e + 2]), s2[kb][e + 3]);
    }
  mx1 = fmaxf(mx1a, mx1b);
  mx2 = fmaxf(mx2a, mx2b);
}

// An unmasked tile's update in two halves.  fwd_pre runs where the logits
// were computed: new offsets, rescale factors, and the logits turned in place
// into t_t = y_t - M_t'.  fwd_post sums 2^t over the tile and folds the sums
// into the state.  Together they equal fwd_update<false>.
struct FwdPre {
  float M1n, M2n, al1, al2;
  bool fresh;  // held offsets: the state had no offset yet (first unmasked tile)
};
template <int NKB>
__device__ __forceinline__ FwdPre fwd_pre(const RowState& st, f32x16 (&s1)[NKB], f32x16 (&s2)[NKB], float c1, float c2) {
  float mx1, mx2;
  fwd_tile_max<NKB>(s1, s2, mx1, mx2);
  FwdPre p;
  p.M1n = fmaxf(st.M1, mx1 * c1);
  p.M2n = fmaxf(st.M2, mx2 * c2);
  p.al1 = exp2_fast(st.M1 - p.M1n);
  p.al2 = exp2_fast(st.M2 - p.M2n);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s1[kb][e] = fmaf(s1[kb][e], c1, -p.M1n);
      s2[kb][e] = fmaf(s2[kb][e], c2, -p.M2n);
    }
  return p;
}
template <int NKB>
__device__ __forceinline__ void fwd_post(RowState& st, const f32x16 (&t1)[NKB], const f32x16 (&t2)[NKB], const FwdPre& p) {
  float tl1[4] = {0.f, 0.f, 0.f, 0.f}, tl2[4] = {0.f, 0.f, 0.f, 0.f}, tA[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p1 = exp2_fast(t1[kb][e]);
      const float p2 = exp2_fast(t2[kb][e]);
      tl1[e & 3] += p1;
      tl2[e & 3] += p2;
      tA[e & 3] = fmaf(p1, t1[kb][e] - t2[kb][e], tA[e & 3]);
    }
  const float sl1 = (tl1[0] + tl1[1]) + (tl1[2] + tl1[3]);
  const float sl2 = (tl2[0] + tl2[1]) + (tl2[2] + tl2[3]);
  const float sA = (tA[0] + tA[1]) + (tA[2] + tA[3]);
  st.l1 = fmaf(p.al1, st.l1, sl1);
  st.l2 = fmaf(p.al2, st.l2, sl2);
  st.A = fmaf(p.al1, st.A, fmaf(p.M1n - p.M2n, sl1, sA));
  st.M1 = p.M1n;
  st.M2 = p.M2n;
}

// An unmasked tile's update with the state's offsets held.  The online
// formulation (technical summary, Method 1) rescales by the running maxima;
// the offsets M_t need not be those maxima: any M_t give the same KL and LSE
// as long as no term 2^(y_t - M_t) overflows and the largest terms stay
// normal floats.
// fwd_pre_held turns the logits in place into t_t = y_t - M_t with the
// state's offsets (0 for an offset still at -inf, whose sums are 0), so the
// logits phase takes no tile maxima.  fwd_post_held sums 2^t.  A lane whose
// state had no offset yet (its first unmasked tile), or whose tile sums pass
// 2^64 or overflow, raises its offsets to the tile maxima of y instead (never
// lowering them) and sums again.  So every offset is a maximum of y over keys
// already seen, every term stays below 2^64 and the largest ones at or
// above 1.
template <int NKB>
__device__ __forceinline__ FwdPre fwd_pre_held(const RowState& st, f32x16 (&s1)[NKB], f32x16 (&s2)[NKB], float c1,
                                               float c2) {
  FwdPre p;
  p.fresh = st.M1 == kNegInf || st.M2 == kNegInf;
  p.M1n = finite_or_zero(st.M1);
  p.M2n = finite_or_zero(st.M2);
  p.al1 = 1.f;
  p.al2 = 1.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s1[kb][e] = fmaf(s1[kb][e], c1, -p.M1n);
      s2[kb][e] = fmaf(s2[kb][e], c2, -p.M2n);
    }
  return p;
}
template <int NKB>
__device__ __forceinline__ void fwd_post_held(RowState& st, const f32x16 (&t1)[NKB], const f32x16 (&t2)[NKB],
                                              const FwdPre& p) {
  constexpr float kCap = 18446744073709551616.f;  // 2^64
  float sl1 = 0.f, sl2 = 0.f, sA = 0.f;
  bool again = p.fresh;
  if (!again) {
    float tl1[4] = {0.f, 0.f, 0.f, 0.f}, tl2[4] = {0.f, 0.f, 0.f, 0.f}, tA[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p1 = exp2_fast(t1[kb][e]);
        const float p2 = exp2_fast(t2[kb][e]);
        tl1[e & 3] += p1;
        tl2[e & 3] += p2;
        tA[e & 3] = fmaf(p1, t1[kb][e] - t2[kb][e], tA[e & 3]);
      }
    sl1 = (tl1[0] + tl1[1]) + (tl1[2] + tl1[3]);
    sl2 = (tl2[0] + tl2[1]) + (tl2[2] + tl2[3]);
    sA = (tA[0] + tA[1]) + (tA[2] + tA[3]);
    again = !(sl1 <= kCap && sl2 <= kCap);
  }
  float m1 = p.M1n, m2 = p.M2n, al1 = 1.f, al2 = 1.f;
  if (__builtin_expect(again, 0)) {
    // offsets raised to the tile maxima (a fresh state takes them whole; the
    // old sums of a fresh state are 0) and the tile summed again
    float mx1, mx2;
    fwd_tile_max<NKB>(t1, t2, mx1, mx2);
    const float h1 = p.fresh ? mx1 : fmaxf(mx1, 0.f), h2 = p.fresh ? mx2 : fmaxf(mx2, 0.f);
    m1 += h1;
    m2 += h2;
    al1 = p.fresh ? 0.f : exp2_fast(-h1);
    al2 = p.fresh ? 0.f : exp2_fast(-h2);
    float u1[4] = {0.f, 0.f, 0.f, 0.f}, u2[4] = {0.f, 0.f, 0.f, 0.f}, uA[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v1 = t1[kb][e] - h1, v2 = t2[kb][e] - h2;
        const float p1 = exp2_fast(v1);
        u1[e & 3] += p1;
        u2[e & 3] += exp2_fast(v2);
        uA[e & 3] = fmaf(p1, v1 - v2, uA[e & 3]);
      }
    sl1 = (u1[0] + u1[1]) + (u1[2] + u1[3]);
    sl2 = (u2[0] + u2[1]) + (u2[2] + u2[3]);
    sA = (uA[0] + uA[1]) + (uA[2] + uA[3]);
  }
  st.l1 = fmaf(al1, st.l1, sl1);
  st.l2 = fmaf(al2, st.l2, sl2);
  st.A = fmaf(al1, st.A, fmaf(m1 - m2, sl1, sA));
  st.M1 = m1;
  st.M2 = m2;
}

// Forward online update of one lane's running state with NKB 32-key blocks of
// raw dot products (s1, s2).  MASK: keys past `lim` are excluded.
template <bool MASK, int NKB>
__device__ __forceinline__ void fwd_update(RowState& st, f32x16 (&s1)[NKB], f32x16 (&s2)[NKB], float c1, float c2, int k0,
                                  int lim, int grp) {
  if constexpr (MASK) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool out = k0 + kb * 32 + acc_row(e, grp) > lim;
        s1[kb][e] = out ? kNegInf : s1[kb][e];
        s2[kb][e] = out ? kNegInf : s2[kb][e];
      }
  }
  float mx1, mx2;
  fwd_tile_max<NKB>(s1, s2, mx1, mx2);
  const float M1n = fmaxf(st.M1, mx1 * c1);
  const float M2n = fmaxf(st.M2, mx2 * c2);
  const float m1 = MASK ? finite_or_zero(M1n) : M1n;
  const float m2 = MASK ? finite_or_zero(M2n) : M2n;
  const float al1 = exp2_fast(st.M1 - m1), al2 = exp2_fast(st.M2 - m2);
  float tl1[4] = {0.f, 0.f, 0.f, 0.f}, tl2[4] = {0.f, 0.f, 0.f, 0.f}, tA[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float t1 = fmaf(s1[kb][e], c1, -m1);
      const float t2 = fmaf(s2[kb][e], c2, -m2);
      const float p1 = exp2_fast(t1);
      const float p2 = exp2_fast(t2);
      float d = t1 - t2;
      if constexpr (MASK) d = (s1[kb][e] == kNegInf) ? 0.f : d;  // never form the ratio on masked keys
      tl1[e & 3] += p1;
      tl2[e & 3] += p2;
      tA[e & 3] = fmaf(p1, d, tA[e & 3]);
    }
  const float sl1 = (tl1[0] + tl1[1]) + (tl1[2] + tl1[3]);
  const float sl2 = (tl2[0] + tl2[1]) + (tl2[2] + tl2[3]);
  const float sA = (tA[0] + tA[1]) + (tA[2] + tA[3]);
  st.l1 = fmaf(al1, st.l1, sl1);
  st.l2 = fmaf(al2, st.l2, sl2);
  st.A = fmaf(al1, st.A, fmaf(m1 - m2, sl1, sA));
  st.M1 = M1n;
  st.M2 = M2n;
}


// One key tile of the forward for one wave: the logits of 32-key block kb+1
// are computed on the matrix cores while the VALU runs the online update of
// block kb (the scheduling groups interleave the two streams).
template <typename T, int D1, int D2, int NKB, bool MASK>
__device__ __forceinline__ void fwd_tile(RowState& st, const T* sK1, const T* sK2, const typename Mfma<T>::frag* qf1,
                                const typename Mfma<T>::frag* qf2, float c1, float c2, int k0, int lim, int col,
                                int grp) {
  using MF = Mfma<T>;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int SM = S1 > S2 ? S1 : S2;
  f32x16 s1[NKB][1], s2[NKB][1];
  auto logits = [&](int kb) {
    s1[kb][0] = zero16();
    s2[kb][0] = zero16();
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      if (s < S1) s1[kb][0] = MF::run(frag_tile<T, D1>(sK1, kb * 32 + col, s, grp), qf1[s < S1 ? s : 0], s1[kb][0]);
      if (s < S2) s2[kb][0] = MF::run(frag_tile<T, D2>(sK2, kb * 32 + col, s, grp), qf2[s < S2 ? s : 0], s2[kb][0]);
    }
  };
  logits(0);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    if (kb + 1 < NKB) logits(kb + 1);
    fwd_update<MASK, 1>(st, s1[kb], s2[kb], c1, c2, k0 + kb * 32, lim, grp);
  }
}

// ---------------------------------------------------------------------------
// Forward.  Workgroup = 4 waves, each owning 32 query rows; key tiles of BK
// rows of K1 and K2 stream through LDS.  Each wave computes S^T = K Q^T so a
// lane's accumulator column is one query row: lane (col, grp) keeps its own
// running state over the keys acc_row(., grp) of every 32-key block, and the
// two lane groups merge once at the end.
// LOSS: the fused-loss form (a.lpart set); a separate instantiation so the
// plain forward's code is untouched by it.  Two workgroups per CU, except
// fp32 with d1 = d2 = 128, whose operand fragments leave room for one.
template <typename T, int D1, int D2, int BK, bool LOSS = false, typename RT = NoTable>
__global__ __launch_bounds__(256, (sizeof(T) == 2 || D1 + D2 < 256) ? 2 : 1) void fwd_kernel(FwdArgs a, const RT rt) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int NW = 4;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int NKB = BK / 32;
  constexpr int TS = BK * (D1 + D2);  // elements of one stage
  __shared__ __attribute__((aligned(1024))) T lds[2 * TS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;
  int64_t lin = blockIdx.x, head0 = 0, heads = a.BH;
  int qo = 0, ko = 0;  // the element's first query and key rows within a head (packed batches)
  if constexpr (kRagged<RT>) {  // one element of a ragged batch (unsplit)
    const RaggedItem r = ragged_item(rt, lin);
    qo = r.qoff;
    ko = r.koff;
    if (r.pad) {
      if constexpr (LOSS) {
        if (tid == 0) a.lpart[blockIdx.x] = 0.0;
      }
      return;
    }
    lin = r.lin;
    head0 = r.head0;
    heads = rt.H;
    a.n_q = r.n_q;
    a.n_k = r.n_k;
    a.nqb = r.nblk;
  }
  const int z = (int)(lin % a.nsplit);
  lin /= a.nsplit;
  const int64_t bh = head0 + lin % heads;
  const int qb = a.nqb - 1 - (int)(lin / heads);  // longest causal rows first
  const int qwg0 = qb * 32 * NW;
  const int q0 = qwg0 + 32 * wave;
  const int qrow = q0 + col;
  const int off = a.n_k - a.n_q;

  const T* Q1 = reinterpret_cast<const T*>(a.q1) + (bh * (int64_t)a.qs + qo) * D1;
  const T* K1 = reinterpret_cast<const T*>(a.k1) + (key_head(bh, a.g1) * (int64_t)a.ks + ko) * D1;
  const T* Q2 = reinterpret_cast<const T*>(a.q2) + (bh * (int64_t)a.qs + qo) * D2;
  const T* K2 = reinterpret_cast<const T*>(a.k2) + (key_head(bh, a.g2) * (int64_t)a.ks + ko) * D2;

  const int kbeg = z * a.keys_per_split;
  int kend = min(a.n_k, kbeg + a.keys_per_split);
  if (a.causal) kend = min(kend, min(a.n_q, qwg0 + 32 * NW) - 1 + off + 1);
  const bool wave_rows = q0 < a.n_q;
  const int wave_kmax = a.causal ? (min(a.n_q, q0 + 32) - 1 + off) : 0x7fffffff;
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const TileLoader<T, D1, BK, NW> ld1(wave, lane);
  const TileLoader<T, D2, BK, NW> ld2(wave, lane);
  if (ntiles > 0) {
    ld1.issue(lds, K1, kbeg, a.n_k);
    ld2.issue(lds + BK * D1, K2, kbeg, a.n_k);
  }

  frag qf1[S1], qf2[S2];
  const bool qv = qrow < a.n_q;
#pragma unroll
  for (int s = 0; s < S1; ++s) qf1[s] = frag_global<T, D1>(Q1, qrow, a.n_q - 1, qv, s, grp);
#pragma unroll
  for (int s = 0; s < S2; ++s) qf2[s] = frag_global<T, D2>(Q2, qrow, a.n_q - 1, qv, s, grp);

  RowState st = empty_state();
  const float c1 = a.c1, c2 = a.c2;

  for (int t = 0; t < ntiles; ++t) {
    wait_loads();
    __syncthreads();
    const int k0 = kbeg + t * BK;
    if (t + 1 < ntiles) {
      T* nb = lds + ((t + 1) & 1) * TS;
      ld1.issue(nb, K1, k0 + BK, a.n_k);
      ld2.issue(nb + BK * D1, K2, k0 + BK, a.n_k);
    }
    if (!wave_rows || k0 > wave_kmax) continue;
    const T* sK1 = lds + (t & 1) * TS;
    const T* sK2 = sK1 + BK * D1;

    const bool need_mask = (k0 + BK > kend) || (a.causal && k0 + BK - 1 > q0 + off);
    if (need_mask) {
      const int lim = a.causal ? min(kend - 1, qrow + off) : kend - 1;
      fwd_tile<T, D1, D2, NKB, true>(st, sK1, sK2, qf1, qf2, c1, c2, k0, lim, col, grp);
    } else {
      fwd_tile<T, D1, D2, NKB, false>(st, sK1, sK2, qf1, qf2, c1, c2, k0, 0, col, grp);
    }
  }

  st = merge_state(st, shfl_xor_state(st, 32));
  double lv = 0.0;
  if (grp == 0 && qrow < a.n_q) {
    const int64_t r = bh * a.qs + qo + qrow;
    if (a.nsplit == 1) {
      const float klv = finish_state(st, a.kl + r, a.lse1 + r, a.lse2 + r);
      if constexpr (LOSS) lv = loss_term(a, r, klv);
    } else {
      const int64_t fs = a.BH * (int64_t)a.nsplit * a.n_q;
      const int64_t o = (bh * a.nsplit + z) * (int64_t)a.n_q + qrow;
      a.ws[o] = st.M1;
      a.ws[o + fs] = st.l1;
      a.ws[o + 2 * fs] = st.A;
      a.ws[o + 3 * fs] = st.M2;
      a.ws[o + 4 * fs] = st.l2;
    }
  }
  if (LOSS && a.nsplit == 1) {
    __syncthreads();  // every wave is past its last tile read: the tile buffer is free
    loss_partial<NW>(lv, reinterpret_cast<double*>(lds), a.lpart + blockIdx.x, tid);
  }
}


// ---------------------------------------------------------------------------
// Forward for short query ranges (n_q <= 32, bf16), split along the keys.
// Every wave is its own key split: it streams 32-key blocks of K1 and K2
// from global memory straight into MFMA operand registers, two blocks in
// flight, with no LDS tiles and no barriers in the loop, so each wave keeps
// its own loads going while it runs the online update of the block before.
// Split z takes blocks z, z + nsplit, z + 2 nsplit, ...: the splits running
// at a time read neighbouring blocks, one front sweeping through K1 and K2
// (contiguous ranges per split, many fronts, ran 3-7% slower).  Split z of
// head bh is wave z % 4 of workgroup bh * ceil(nsplit / 4) + z / 4; the four
// waves share the head's Q1 and Q2, held once in LDS.
//
// Operand order: lane group g feeds d-chunk 2s + g (8 elements) at MFMA step
// s, the natural order, so each load instruction reads 32 bytes of each of
// 32 key rows.
template <int D>
__device__ __forceinline__ void dec_load_row(bf16x8 (&f)[D / 16], const bf16* base, int64_t row, int grp) {
  constexpr int S = D / 16;
  const bf16x8* p = reinterpret_cast<const bf16x8*>(base + row * D) + grp;
#pragma unroll
  for (int s = 0; s < S; ++s) f[s] = p[2 * s];
}

// rows [0, 32) of a [n_q, D] query tensor into a swizzled LDS tile (zeros
// past n_q), 16-byte chunks spread over the workgroup's 256 threads
template <int D>
__device__ __forceinline__ void dec_stage_q(bf16* tile, const bf16* q, int n_q, int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = tid; i < 32 * CPR; i += 256) {
    const int r = i / CPR, c = i % CPR;
    bf16x8 v = zero_frag<bf16>();
    if (r < n_q) v = *reinterpret_cast<const bf16x8*>(q + (int64_t)r * D + 8 * c);
    *reinterpret_cast<bf16x8*>(tile + Tile<bf16, D>::off(r, 8 * c)) = v;
  }
}

template <int D1, int D2, typename RT = NoTable>
__global__ __launch_bounds__(256, 2) void fwd_decode_kernel(FwdArgs a, const RT rt) {
  constexpr int NB = 2;  // blocks in flight per wave
  using MF = Mfma<bf16>;
  constexpr int S1 = D1 / 16, S2 = D2 / 16;
  __shared__ __attribute__((aligned(1024))) bf16 sq[32 * (D1 + D2)];
  bf16* sQ1 = sq;
  bf16* sQ2 = sq + 32 * D1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;
  int64_t bh, loc;  // the head, and its index within the problem (or the element)
  int z;
  int64_t wsb = 0;  // the problem's (the element's) first partial
  int qo = 0, ko = 0;  // the element's first query and key rows within a head (packed batches)
  if constexpr (kDecTable<RT>) {
    const int e = table_elem(rt.start, rt.n, blockIdx.x);
    qo = rt.qoff[e];
    ko = rt.koff[e];
    const int64_t lin = blockIdx.x - rt.start[e];
    a.n_q = rt.n_q[e];
    a.n_k = rt.n_k[e];
    a.nsplit = rt.nsplit[e];
    const int64_t nwg = (a.nsplit + 3) / 4;
    if (lin >= (int64_t)rt.H * nwg) return;  // padding of the element's range
    loc = lin / nwg;
    bh = (int64_t)rt.b[e] * rt.H + loc;
    z = (int)(lin % nwg) * 4 + wave;
    wsb = rt.wsb[e];
  } else {
    const int64_t nwg = (a.nsplit + 3) / 4;
    bh = blockIdx.x / nwg;
    loc = bh;
    z = (int)(blockIdx.x % nwg) * 4 + wave;
  }
  const int off = a.n_k - a.n_q;

  const bf16* Q1 = reinterpret_cast<const bf16*>(a.q1) + (bh * (int64_t)a.qs + qo) * D1;
  const bf16* K1 = reinterpret_cast<const bf16*>(a.k1) + (key_head(bh, a.g1) * (int64_t)a.ks + ko) * D1;
  const bf16* Q2 = reinterpret_cast<const bf16*>(a.q2) + (bh * (int64_t)a.qs + qo) * D2;
  const bf16* K2 = reinterpret_cast<const bf16*>(a.k2) + (key_head(bh, a.g2) * (int64_t)a.ks + ko) * D2;
  dec_stage_q<D1>(sQ1, Q1, a.n_q, tid);
  dec_stage_q<D2>(sQ2, Q2, a.n_q, tid);
  __syncthreads();
  if (z >= a.nsplit) return;

  // block j of this split is the head's block j * nsplit + z
  const int nball = (a.n_k + 31) / 32;
  const int kb0 = 32 * z;
  const int kstep = 32 * a.nsplit;
  const int nblk = z < nball ? (nball - z + a.nsplit - 1) / a.nsplit : 0;
  const int qrow = col;
  // B operands: query row col, chunk 2s + grp, read from the LDS tile for
  // every block (the per-block opaque offset keeps the compiler from hoisting
  // them into 16 * S registers that the K blocks in flight need)
  auto qfrag1 = [&](int s, int o) {
    return *reinterpret_cast<const bf16x8*>(sQ1 + o + Tile<bf16, D1>::off(col, 8 * (2 * s + grp)));
  };
  auto qfrag2 = [&](int s, int o) {
    return *reinterpret_cast<const bf16x8*>(sQ2 + o + Tile<bf16, D2>::off(col, 8 * (2 * s + grp)));
  };

  RowState st = empty_state();
  const float c1 = a.c1, c2 = a.c2;
  const int lim_row = a.causal ? min(a.n_k - 1, qrow + off) : a.n_k - 1;

  // Blocks are loaded without conditions (past the last block the loads
  // re-read the head's last key row, which is cached), so the same loads are
  // in flight at every point of the loop and each block waits only for its own.
  bf16x8 kf1[NB][S1], kf2[NB][S2];
  auto load = [&](bf16x8(&f1)[S1], bf16x8(&f2)[S2], int j) {
    const int64_t row = min(kb0 + kstep * j + col, a.n_k - 1);
    dec_load_row<D1>(f1, K1, row, grp);
    dec_load_row<D2>(f2, K2, row, grp);
  };
  // logits of block j from (f1, f2), then the load of block j + NB into the
  // same registers, then the online update of block j (if it exists)
  auto block = [&](bf16x8(&f1)[S1], bf16x8(&f2)[S2], int j) {
    f32x16 s1[1] = {zero16()}, s2[1] = {zero16()};
    int qo = 0;
    asm volatile("" : "+v"(qo));
#pragma unroll
    for (int s = 0; s < (S1 > S2 ? S1 : S2); ++s) {
      if (s < S1) s1[0] = MF::run(f1[s < S1 ? s : 0], qfrag1(s < S1 ? s : 0, qo), s1[0]);
      if (s < S2) s2[0] = MF::run(f2[s < S2 ? s : 0], qfrag2(s < S2 ? s : 0, qo), s2[0]);
    }
    load(f1, f2, j + NB);
    if (j >= nblk) return;
    const int k0 = kb0 + kstep * j;
    const bool need_mask = (k0 + 32 > a.n_k) || (a.causal && k0 + 31 > off);
    if (need_mask) fwd_update<true, 1>(st, s1, s2, c1, c2, k0, lim_row, grp);
    else fwd_update<false, 1>(st, s1, s2, c1, c2, k0, 0, grp);
  };
  if (nblk > 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      load(kf1[b], kf2[b], b);
      __builtin_amdgcn_sched_barrier(0);  // keep the issue order of the blocks
    }
    for (int j = 0; j < nblk; j += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) block(kf1[b], kf2[b], j + b);
    }
  }

  st = merge_state(st, shfl_xor_state(st, 32));
  if (grp == 0 && qrow < a.n_q) {
    int64_t fs;
    if constexpr (kDecTable<RT>) fs = rt.fs;
    else fs = a.BH * (int64_t)a.nsplit * a.n_q;
    const int64_t o = wsb + (loc * a.nsplit + z) * (int64_t)a.n_q + qrow;
    a.ws[o] = st.M1;
    a.ws[o + fs] = st.l1;
    a.ws[o + 2 * fs] = st.A;
    a.ws[o + 3 * fs] = st.M2;
    a.ws[o + 4 * fs] = st.l2;
  }
}

// Logits of one key tile for one wave: s_t[kb] = K_t[kb*32 .. +32) Q_t^T for
// the wave's 32 query rows (raw dot products), 2*NKB independent chains.
template <typename T, int D1, int D2, int NKB>
__device__ __forceinline__ void fwd_logits(f32x16 (&s1)[NKB], f32x16 (&s2)[NKB], const T* sK1, const T* sK2,
                                  const typename Mfma<T>::frag* qf1, const typename Mfma<T>::frag* qf2, int col,
                                  int grp) {
  using MF = Mfma<T>;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int SM = S1 > S2 ? S1 : S2;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    s1[kb] = zero16();
    s2[kb] = zero16();
  }
#pragma unroll
  for (int s = 0; s < SM; ++s)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (s < S1) s1[kb] = MF::run(frag_tile<T, D1>(sK1, kb * 32 + col, s, grp), qf1[s < S1 ? s : 0], s1[kb]);
      if (s < S2) s2[kb] = MF::run(frag_tile<T, D2>(sK2, kb * 32 + col, s, grp), qf2[s < S2 ? s : 0], s2[kb]);
    }
  sched_mfma_lds<NKB * (S1 + S2), 1, 4>();
}

// ---------------------------------------------------------------------------
// Forward, ping-pong form for long query ranges.  Workgroup = 8 waves (two per
// SIMD), each owning 32 query rows; both wave groups read the same key tiles
// from LDS.  Group A (waves 0-3) computes the logits of tile t while group B
// (waves 4-7, the other wave on each SIMD) runs the online update of tile
// t-1; after a barrier the roles swap.  Each SIMD thus keeps one wave on the
// matrix cores and one on the VALU.
template <typename T, int D1, int D2, int BK, bool LOSS = false, typename RT = NoTable>
__global__ __launch_bounds__(512, 1) void fwd_pp_kernel(FwdArgs a, const RT rt) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int NW = 8;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int NKB = BK / 32;
  constexpr int TS = BK * (D1 + D2);
  __shared__ __attribute__((aligned(1024))) T lds[2 * TS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;
  const int group = wave >> 2;
  int64_t lin = blockIdx.x, head0 = 0, heads = a.BH;
  int qo = 0, ko = 0;  // the element's first query and key rows within a head (packed batches)
  if constexpr (kRagged<RT>) {  // one element of a ragged batch
    const RaggedItem r = ragged_item(rt, lin);
    qo = r.qoff;
    ko = r.koff;
    if (r.pad) {
      if constexpr (LOSS) {
        if (tid == 0) a.lpart[blockIdx.x] = 0.0;
      }
      return;
    }
    lin = r.lin;
    head0 = r.head0;
    heads = rt.H;
    a.n_q = r.n_q;
    a.n_k = r.n_k;
    a.nqb = r.nblk;
  }
  const WorkItem wi = work_item(lin, heads, a.nqb);
  const int64_t bh = head0 + wi.bh;
  const int qb = a.nqb - 1 - wi.blk;  // longest causal rows first
  const int qwg0 = qb * 32 * NW;
  const int q0 = qwg0 + 32 * wave;
  const int qrow = q0 + col;
  const int off = a.n_k - a.n_q;

  const T* Q1 = reinterpret_cast<const T*>(a.q1) + (bh * (int64_t)a.qs + qo) * D1;
  const T* K1 = reinterpret_cast<const T*>(a.k1) + (key_head(bh, a.g1) * (int64_t)a.ks + ko) * D1;
  const T* Q2 = reinterpret_cast<const T*>(a.q2) + (bh * (int64_t)a.qs + qo) * D2;
  const T* K2 = reinterpret_cast<const T*>(a.k2) + (key_head(bh, a.g2) * (int64_t)a.ks + ko) * D2;

  int kend = a.n_k;
  if (a.causal) kend = min(kend, min(a.n_q, qwg0 + 32 * NW) - 1 + off + 1);
  const bool wave_rows = q0 < a.n_q;
  const int wave_kmax = a.causal ? (min(a.n_q, q0 + 32) - 1 + off) : 0x7fffffff;
  const int ntiles = (kend + BK - 1) / BK;

  const TileLoader<T, D1, BK, NW> ld1(wave, lane);
  const TileLoader<T, D2, BK, NW> ld2(wave, lane);
  ld1.issue(lds, K1, 0, a.n_k);
  ld2.issue(lds + BK * D1, K2, 0, a.n_k);

  frag qf1[S1], qf2[S2];
  const bool qv = qrow < a.n_q;
#pragma unroll
  for (int s = 0; s < S1; ++s) qf1[s] = frag_global<T, D1>(Q1, qrow, a.n_q - 1, qv, s, grp);
#pragma unroll
  for (int s = 0; s < S2; ++s) qf2[s] = frag_global<T, D2>(Q2, qrow, a.n_q - 1, qv, s, grp);

  RowState st = empty_state();
  const float c1 = a.c1, c2 = a.c2;
  const int lim_row = a.causal ? min(kend - 1, qrow + off) : kend - 1;
  f32x16 s1[NKB], s2[NKB];
  FwdPre pre = {0.f, 0.f, 0.f, 0.f};

  // An unmasked tile's update is split: the logits phase, whose wave's VALU
  // is mostly idle, takes the maxima, offsets and t = y - M (fwd_pre); the
  // update phase, the longer one, keeps the exponentials and sums (fwd_post).
  // Forward 37.1 -> 35.2 ms at 64K causal against the whole update in the
  // update phase (36.2 ms with only the maxima moved).
  // Unmasked tiles hold the state's offsets (fwd_pre_held), so their logits
  // phase takes no maxima; masked tiles take them.
  auto masked = [&](int k0) { return (k0 + BK > kend) || (a.causal && k0 + BK - 1 > q0 + off); };
  auto logits = [&](const T* sK1, const T* sK2, int k0) {
    fwd_logits<T, D1, D2, NKB>(s1, s2, sK1, sK2, qf1, qf2, col, grp);
    if (masked(k0)) return;
    pre = fwd_pre_held<NKB>(st, s1, s2, c1, c2);
  };
  auto update = [&](int k0) {
    if (!wave_rows || k0 > wave_kmax) return;
    if (masked(k0)) fwd_update<true, NKB>(st, s1, s2, c1, c2, k0, lim_row, grp);
    else fwd_post_held<NKB>(st, s1, s2, pre);
  };

  for (int t = 0; t < ntiles; ++t) {
    wait_loads();
    __syncthreads();
    const int k0 = t * BK;
    if (t + 1 < ntiles) {
      T* nb = lds + ((t + 1) & 1) * TS;
      ld1.issue(nb, K1, k0 + BK, a.n_k);
      ld2.issue(nb + BK * D1, K2, k0 + BK, a.n_k);
    }
    const T* sK1 = lds + (t & 1) * TS;
    const T* sK2 = sK1 + BK * D1;
    const bool active = wave_rows && k0 <= wave_kmax;
    if (group == 0) {
      if (active) logits(sK1, sK2, k0);
    } else if (t > 0) {
      update(k0 - BK);
    }
    phase_barrier();
    if (group == 0) {
      update(k0);
    } else if (active) {
      logits(sK1, sK2, k0);
    }
  }
  if (group == 1 && ntiles > 0) update((ntiles - 1) * BK);

  st = merge_state(st, shfl_xor_state(st, 32));
  double lv = 0.0;
  if (grp == 0 && qrow < a.n_q) {
    const int64_t r = bh * a.qs + qo + qrow;
    const float klv = finish_state(st, a.kl + r, a.lse1 + r, a.lse2 + r);
    if constexpr (LOSS) lv = loss_term(a, r, klv);
  }
  if constexpr (LOSS) {
    __syncthreads();  // group 1 may still read the last tile until here
    loss_partial<NW>(lv, reinterpret_cast<double*>(lds), a.lpart + blockIdx.x, tid);
  }
}

// Per-row quantities the backward needs, in base-2 units: exponent offsets
// L_t and the gradient scale gs (g * scale_s; setting 1 keeps only its sign
// and folds |g * scale_s| into L_t, see scale_rowgrad); setting 2 also
// a = gs * ln2 and b = gs * KL, so that dS1 = P1 * (a * (t1 - t2) - b) with
// t_t = y_t - L_t.
struct RowGrad {
  float L1, L2, gs, a, b;
};

// The stored per-row values RowGrad is built from (zeros for invalid rows).
struct RawRowGrad {
  float lse1, lse2, g, kl;
};

template <int SETTING>
__device__ __forceinline__ RawRowGrad load_rowgrad_raw(const BwdArgs& a, int64_t r, bool valid) {
  RawRowGrad o = {0.f, 0.f, 0.f, 0.f};
  if (!valid) return o;
  o.lse1 = a.lse1[r];
  o.lse2 = a.lse2[r];
  o.g = a.g[r];
  if constexpr (SETTING >= 2) o.kl = a.kl[r];
  return o;
}

// Setting 1 folds |gs| into the exponent offsets: L_t = LSE_t log2(e) -
// log2|gs|, so exp2(y_t - L_t) is |gs| P_t and gs is replaced by its sign
// (a zero gs gives +inf offsets and an exactly zero dS row).
//
// Joint (SETTING 3, gradients to both models): the offsets are not folded;
// gs = g * scale_2 for dS2 = gs (P2 - P1), and a, b come from g * scale_1
// for dS1.
template <int SETTING>
__device__ __forceinline__ RowGrad scale_rowgrad(const BwdArgs& a, const RawRowGrad& w) {
  RowGrad o;
  const float gs = w.g * a.scale_s;
  o.L1 = w.lse1 * kLog2e;
  o.L2 = w.lse2 * kLog2e;
  o.gs = gs;
  o.a = 0.f;
  o.b = 0.f;
  if constexpr (SETTING == 1) {
    const float lg = log2f(fabsf(gs));
    o.L1 -= lg;
    o.L2 -= lg;
    o.gs = gs < 0.f ? -1.f : 1.f;
  } else {
    o.a = gs * kLn2;
    o.b = gs * w.kl;
    if constexpr (SETTING == 3) o.gs = w.g * a.scale_s2;
  }
  return o;
}

template <int SETTING>
__device__ __forceinline__ RowGrad load_rowgrad(const BwdArgs& a, int64_t r, bool valid) {
  return scale_rowgrad<SETTING>(a, load_rowgrad_raw<SETTING>(a, r, valid));
}

// dS for one element from the raw dot products s1, s2 (see RowGrad).
template <int SETTING>
__device__ __forceinline__ float dS_elem(float s1, float s2, float c1, float c2, float L1, float L2, float gs, float ra,
                                float rb) {
  const float t1 = fmaf(s1, c1, -L1);
  const float t2 = fmaf(s2, c2, -L2);
  const float p1 = exp2_fast(t1);
  if constexpr (SETTING == 1) {
    const float p2 = exp2_fast(t2);
    return gs * (p2 - p1);
  } else {
    return p1 * fmaf(ra, t1 - t2, -rb);
  }
}

// dS for one element of the query-outer kernel, where a lane holds one query
// row: for setting 1 the row's sign (gs = +-1) is left out here and applied
// to the row's dQ once at the end.
template <int SETTING>
__device__ __forceinline__ float dS_elem_row(float s1, float s2, float c1, float c2, const RowGrad& rg) {
  if constexpr (SETTING == 1) return exp2_fast(fmaf(s2, c2, -rg.L2)) - exp2_fast(fmaf(s1, c1, -rg.L1));
  else return dS_elem<SETTING>(s1, s2, c1, c2, rg.L1, rg.L2, rg.gs, rg.a, rg.b);
}

// Joint: dS1 (setting 2) and dS2 (setting 1) of one element from the raw
// dot products, sharing P1 (see RowGrad).
__device__ __forceinline__ void dS_joint(float s1, float s2, float c1, float c2, float L1, float L2, float gs, float ra,
                                float rb, float& ds1, float& ds2) {
  const float t1 = fmaf(s1, c1, -L1);
  const float t2 = fmaf(s2, c2, -L2);
  const float p1 = exp2_fast(t1);
  const float p2 = exp2_fast(t2);
  ds1 = p1 * fmaf(ra, t1 - t2, -rb);
  ds2 = gs * (p2 - p1);
}


// dS for one 32x32 block of the key-outer kernel (lane = key, accumulator rows
// = queries qb0 + acc_row(e, grp)); per-query stats come from LDS
// (st[k*BQ + q]: L1, L2, gs, then a, b for setting 2).  SIGNED = false
// (setting 1, no negative gradient in the tile) skips gs, which is then +1.
// MASK: queries outside [qlo, n_q) get dS = 0.  Result overwrites s1.
template <int SETTING, bool MASK, int BQ, bool SIGNED = true>
__device__ __forceinline__ void dS_rows_keyouter(f32x16& s1, const f32x16& s2, const float* st, int ql0, int qb0, int grp,
                                        float c1, float c2, int qlo, int n_q, int lane_off) {
  // st[k*BQ + q] for q = ql0 + 8i + 4grp + j; lane_off = 16 * grp bytes
  auto at = [&](int k, int i) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(st + k * BQ + ql0 + 8 * i) + lane_off);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 L1 = at(0, i);
    const f32x4 L2 = at(1, i);
    f32x4 GS = {1.f, 1.f, 1.f, 1.f};
    if (SETTING != 1 || SIGNED) GS = at(2, i);
    f32x4 RA = {0.f, 0.f, 0.f, 0.f}, RB = {0.f, 0.f, 0.f, 0.f};
    if constexpr (SETTING == 2) {
      RA = at(3, i);
      RB = at(4, i);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * i + j;
      float ds;
      if constexpr (SETTING == 1 && !SIGNED)
        ds = exp2_fast(fmaf(s2[e], c2, -L2[j])) - exp2_fast(fmaf(s1[e], c1, -L1[j]));
      else
        ds = dS_elem<SETTING>(s1[e], s2[e], c1, c2, L1[j], L2[j], GS[j], RA[j], RB[j]);
      if constexpr (MASK) {
        const int q = qb0 + 8 * i + 4 * grp + j;
        ds = ((q >= qlo) & (q < n_q)) ? ds : 0.f;
      }
      s1[e] = ds;
    }
  }
}

// Joint version: dS1 overwrites s1 and dS2 overwrites s2 (stats L1, L2, gs,
// a, b per query).
template <bool MASK, int BQ>
__device__ __forceinline__ void dS_rows_keyouter_joint(f32x16& s1, f32x16& s2, const float* st, int ql0, int qb0, int grp,
                                              float c1, float c2, int qlo, int n_q, int lane_off) {
  auto at = [&](int k, int i) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(st + k * BQ + ql0 + 8 * i) + lane_off);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 L1 = at(0, i), L2 = at(1, i), GS = at(2, i), RA = at(3, i), RB = at(4, i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * i + j;
      float d1, d2;
      dS_joint(s1[e], s2[e], c1, c2, L1[j], L2[j], GS[j], RA[j], RB[j], d1, d2);
      if constexpr (MASK) {
        const int q = qb0 + 8 * i + 4 * grp + j;
        const bool v = (q >= qlo) & (q < n_q);
        d1 = v ? d1 : 0.f;
        d2 = v ? d2 : 0.f;
      }
      s1[e] = d1;
      s2[e] = d2;
    }
  }
}

// ---------------------------------------------------------------------------
// Query-outer backward: dQ_s for 32 query rows per wave (NW waves), key tiles
// of BK rows of K1 and K2 streamed through LDS.  The more waves share a
// workgroup, the fewer times each head's key tiles are read.  S^T = K Q^T keeps a lane on
// one query row, so dS from the accumulators is directly the A operand of
// dQ = dS K_s; K_s's B operand is read down the key rows of its tile.
// Deterministic; no atomics.
template <typename T, int D1, int D2, int SETTING, int BK, int NW = 4, typename RT = NoTable>
__global__ __launch_bounds__(64 * NW) void bwd_dq_kernel(BwdArgs a, const RT rt) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int DS = SETTING == 1 ? D2 : D1;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int NKB = BK / 32, NB = DS / 32, HS = 32 / MF::KSTEP;
  constexpr int TS = BK * (D1 + D2);
  constexpr bool BF = sizeof(T) == 2;
  // two tile buffers, then (bf16) the reference key kbar: DS floats
  __shared__ __attribute__((aligned(1024))) T lds[2 * TS + (BF ? 2 * DS : 0)];
  float* kbar = reinterpret_cast<float*>(lds + 2 * TS);

  // the wave index as a scalar: the per-block conditions on this wave's rows
  // become scalar branches instead of exec-mask branches
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;
  int64_t lin = blockIdx.x, head0 = 0, heads = a.BH;
  int qo = 0, ko = 0;  // the element's first query and key rows within a head (packed batches)
  if constexpr (kRagged<RT>) {  // one element of a ragged batch
    const RaggedItem r = ragged_item(rt, lin);
    qo = r.qoff;
    ko = r.koff;
    if (r.pad) return;
    lin = r.lin;
    head0 = r.head0;
    heads = rt.H;
    a.n_q = r.n_q;
    a.n_k = r.n_k;
    a.nblk = r.nblk;
  }
  const WorkItem wi = work_item(lin, heads, a.nblk);
  const int64_t bh = head0 + wi.bh;
  const int qb = a.nblk - 1 - wi.blk;  // longest causal rows first
  const int q0 = qb * 32 * NW + 32 * wave;
  const int qrow = q0 + col;
  const int off = a.n_k - a.n_q;

  const T* Q1 = reinterpret_cast<const T*>(a.q1) + (bh * (int64_t)a.qs + qo) * D1;
  const T* K1 = reinterpret_cast<const T*>(a.k1) + (key_head(bh, a.g1) * (int64_t)a.ks + ko) * D1;
  const T* Q2 = reinterpret_cast<const T*>(a.q2) + (bh * (int64_t)a.qs + qo) * D2;
  const T* K2 = reinterpret_cast<const T*>(a.k2) + (key_head(bh, a.g2) * (int64_t)a.ks + ko) * D2;

  int kend = a.n_k;
  if (a.causal) kend = min(kend, min(a.n_q, qb * 32 * NW + 32 * NW) - 1 + off + 1);
  const bool wave_rows = q0 < a.n_q;
  const int wave_kmax = a.causal ? (min(a.n_q, q0 + 32) - 1 + off) : 0x7fffffff;
  const int ntiles = (kend + BK - 1) / BK;

  const TileLoader<T, D1, BK, NW> ld1(wave, lane);
  const TileLoader<T, D2, BK, NW> ld2(wave, lane);
  ld1.issue(lds, K1, 0, a.n_k);
  ld2.issue(lds + BK * D1, K2, 0, a.n_k);
  // the first tile's barrier publishes kbar
  if constexpr (BF) ref_key<DS>(kbar, reinterpret_cast<const bf16*>(SETTING == 1 ? K2 : K1), a.n_k, tid, 64 * NW);

  frag qf1[S1], qf2[S2];
  const bool qv = qrow < a.n_q;
#pragma unroll
  for (int s = 0; s < S1; ++s) qf1[s] = frag_global<T, D1>(Q1, qrow, a.n_q - 1, qv, s, grp);
#pragma unroll
  for (int s = 0; s < S2; ++s) qf2[s] = frag_global<T, D2>(Q2, qrow, a.n_q - 1, qv, s, grp);
  const RowGrad rg = load_rowgrad<SETTING>(a, bh * a.qs + qo + qrow, qv);
  const float row_sign = SETTING == 1 ? rg.gs : 1.f;

  f32x16 dqa[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dqa[nb] = zero16();
  float rsum = 0.f;  // bf16: this lane's part of r for query qrow, the sum of the bf16 dS it fed

  // bf16: per-lane LDS offsets computed once (K1/K2 rows share them when
  // d1 == d2); fp32 computes addresses per read
  using RF1 = std::conditional_t<BF, RowFragOffsets<D1, S1>, NoOffsets>;
  using RF2 = std::conditional_t<BF, RowFragOffsets<D2, S2>, NoOffsets>;
  using CF = std::conditional_t<BF, ColFragOffsets<DS, NB>, NoOffsets>;
  RF1 rf1(col, grp);
  RF2 rf2 = [&]() -> RF2 {
    if constexpr (std::is_same_v<RF1, RF2>) return rf1;
    else return RF2(col, grp);
  }();
  CF cf(lane);
  auto row1 = [&](const T* tile, int blk, int s) -> frag {
    if constexpr (BF) return rf1.read(tile, blk, s);
    else return frag_tile<T, D1>(tile, 32 * blk + col, s, grp);
  };
  auto row2 = [&](const T* tile, int blk, int s) -> frag {
    if constexpr (BF) return rf2.read(tile, blk, s);
    else return frag_tile<T, D2>(tile, 32 * blk + col, s, grp);
  };
  auto colop = [&](const T* tile, int blk, int nb, int h) -> frag {
    if constexpr (BF) return cf.read(tile, blk, nb, h);
    else return fragcol_acc<T, DS>(tile, 32 * blk, 32 * nb, h, lane);
  };

  // Tiles alternate between the two LDS buffers; stepping by two keeps each
  // buffer's tile base a constant, so every LDS read is a per-lane offset plus
  // an immediate (no address arithmetic per read).
  auto tile = [&](const T* sK1, int k0) {
    const bool need_mask = (k0 + BK > kend) || (a.causal && k0 + BK - 1 > q0 + off);
    const int lim = a.causal ? min(kend - 1, qrow + off) : kend - 1;
    const T* sK2 = sK1 + BK * D1;
    const T* sKS = SETTING == 1 ? sK2 : sK1;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s1 = zero16(), s2 = zero16();
      constexpr int SM = S1 > S2 ? S1 : S2;
#pragma unroll
      for (int s = 0; s < SM; ++s) {
        if (s < S1) s1 = MF::run(row1(sK1, kb, s), qf1[s < S1 ? s : 0], s1);
        if (s < S2) s2 = MF::run(row2(sK2, kb, s), qf2[s < S2 ? s : 0], s2);
      }
      sched_mfma_lds<S1 + S2, 1, 4>();
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float ds = dS_elem_row<SETTING>(s1[e], s2[e], a.c1, a.c2, rg);
          s1[e] = (k0 + kb * 32 + acc_row(e, grp) > lim) ? 0.f : ds;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) s1[e] = dS_elem_row<SETTING>(s1[e], s2[e], a.c1, a.c2, rg);
      }
#pragma unroll
      for (int h = 0; h < HS; ++h) {
        const frag af = frag_from_acc(s1, h, T());
        if constexpr (BF) rsum = sum_frag(af, rsum);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) dqa[nb] = MF::run(af, colop(sKS, kb, nb, h), dqa[nb]);
      }
      sched_mfma_lds<HS * NB, MF::KPL == 1 ? 1 : 2, 2>();
    }
  };
  auto step = [&](int t, const T* sbuf, T* nbuf) {
    wait_loads();
    __syncthreads();
    const int k0 = t * BK;
    if (t + 1 < ntiles) {
      ld1.issue(nbuf, K1, k0 + BK, a.n_k);
      ld2.issue(nbuf + BK * D1, K2, k0 + BK, a.n_k);
    }
    if (wave_rows && k0 <= wave_kmax) tile(sbuf, k0);
  };
  for (int t = 0; t < ntiles; t += 2) {
    rf1.touch();
    if constexpr (!std::is_same_v<RF1, RF2>) rf2.touch();
    cf.touch();
    step(t, lds, lds + TS);
    if (t + 1 < ntiles) step(t + 1, lds + TS, lds);
  }

  // dQ accumulator rows are queries q0 + acc_row(e, grp); lane r < 32 holds
  // query q0 + r's sign (and, once the lane groups' key halves are added, its r)
  if constexpr (BF) {
    rsum += __shfl_xor(rsum, 32);
    float kb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) kb[nb] = kbar[nb * 32 + col];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float rq = __shfl(rsum, acc_row(e, grp));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) dqa[nb][e] = fmaf(-rq, kb[nb], dqa[nb][e]);
    }
  }
  const uint64_t neg = __ballot(row_sign < 0.f);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = acc_row(e, grp);
      const int q = q0 + r;
      const float v = ((neg >> r) & 1) ? -dqa[nb][e] : dqa[nb][e];
      if (q < a.n_q) a.dq[(bh * a.qs + qo + q) * DS + nb * 32 + col] = v;
    }
}

// ---------------------------------------------------------------------------
// Key-outer backward: each wave owns 32 key rows (workgroup: NW waves, 32 NW
// keys; the more keys a workgroup owns, the fewer times each head's query
// tiles are read), keeps K1, K2 in registers and accumulates dK_s in registers while
// query tiles of BQ rows of Q1 and Q2 stream through LDS.  The logits are
// computed as S = Q K^T so a lane's accumulator column is one key and dS from
// the accumulators is directly the A operand of dK = dS^T Q_s; Q_s's B operand
// is read down the query rows of its tile.  FUSED additionally forms dQ_s for
// every query tile from the same dS (staged in LDS as [key][query]) and adds it
// to global dQ_s with fp32 atomics, so each query-key pair is visited once.
// SETTING 3 (joint, not fused) forms dS1 and dS2 from the same logits and
// accumulates dK1 (dk) and dK2 (dk2).
template <typename T, int D1, int D2, int SETTING, bool FUSED, int BQ, int NW = 4, typename RT = NoTable>
__global__ __launch_bounds__(64 * NW) void bwd_dk_kernel(BwdArgs a, const RT rt) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr bool JOINT = SETTING == 3;
  static_assert(!(JOINT && FUSED), "the joint backward has no fused form");
  static_assert(NW == 4 || !FUSED, "the fused form maps its dQ columns onto 4 waves");
  constexpr int BKW = 32 * NW;
  constexpr int DS = SETTING == 1 ? D2 : D1;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int NB = DS / 32, NB2 = D2 / 32, HS = 32 / MF::KSTEP, NQB = BQ / 32, HK = BKW / MF::KSTEP;
  constexpr int TS = BQ * (D1 + D2);
  constexpr int NSTAT = SETTING >= 2 ? 5 : 3;
  // One LDS array holds the two tile buffers, the dS^T staging tile (FUSED)
  // and the two per-query stats buffers: separate __shared__ objects would
  // get distinct alias scopes, and then every tile read would be made to wait
  // for the next tile's direct loads in flight.
  constexpr int DSE = FUSED ? BKW * BQ : 0;                      // dS^T elements
  constexpr int STAT_OFF = ((2 * TS + DSE) * (int)sizeof(T) + 15) / 16 * 16;  // bytes
  constexpr int FLAG_OFF = STAT_OFF + 2 * NSTAT * BQ * 4;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[FLAG_OFF + 2 * 4];
  T* lds = reinterpret_cast<T*>(smem);
  T* sdS = lds + 2 * TS;
  float(*sstat)[NSTAT][BQ] = reinterpret_cast<float(*)[NSTAT][BQ]>(smem + STAT_OFF);
  int* sneg = reinterpret_cast<int*>(smem + FLAG_OFF);  // per stats buffer: a row has gs < 0

  // the wave index as a scalar: the per-block conditions on this wave's rows
  // become scalar branches instead of exec-mask branches
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;
  int64_t lin = blockIdx.x, head0 = 0, heads = a.BH;
  int qo = 0, ko = 0;  // the element's first query and key rows within a head (packed batches)
  if constexpr (kRagged<RT>) {  // one element of a ragged batch
    const RaggedItem r = ragged_item(rt, lin);
    qo = r.qoff;
    ko = r.koff;
    if (r.pad) return;
    lin = r.lin;
    head0 = r.head0;
    heads = rt.H;
    a.n_q = r.n_q;
    a.n_k = r.n_k;
    a.nblk = r.nblk;
  }
  const WorkItem wi = work_item(lin, heads, a.nblk);
  const int64_t bh = head0 + wi.bh;
  const int kb = wi.blk;  // low key blocks see the most queries under causal masks: first
  const int kw0 = kb * BKW;
  const int kwave = kw0 + 32 * wave;
  const int krow = kwave + col;
  const int off = a.n_k - a.n_q;

  const T* Q1 = reinterpret_cast<const T*>(a.q1) + (bh * (int64_t)a.qs + qo) * D1;
  const T* K1 = reinterpret_cast<const T*>(a.k1) + (key_head(bh, a.g1) * (int64_t)a.ks + ko) * D1;
  const T* Q2 = reinterpret_cast<const T*>(a.q2) + (bh * (int64_t)a.qs + qo) * D2;
  const T* K2 = reinterpret_cast<const T*>(a.k2) + (key_head(bh, a.g2) * (int64_t)a.ks + ko) * D2;
  const T* KS = SETTING == 1 ? K2 : K1;

  // Query tiles are visited from the last one down: under a causal mask every
  // key block sees the high queries, so the workgroups running at a time all
  // start on the same tile and move down together (L2 reuse), each stopping at
  // its own first query tile.
  const int qbeg = a.causal ? max(0, kw0 - off) : 0;
  const int qt0 = (qbeg / BQ) * BQ;
  const int ntiles = qt0 < a.n_q ? (a.n_q - qt0 + BQ - 1) / BQ : 0;
  const int qtl = qt0 + (ntiles - 1) * BQ;  // first tile visited

  // stats of one query tile: thread q < BQ loads row q raw (zeros past n_q);
  // they are scaled and stored to LDS after the tile's compute, behind a
  // scheduling barrier, so their load latency overlaps the whole tile
  auto load_stats = [&](int q0, RawRowGrad& r) {
    r = load_rowgrad_raw<SETTING>(a, bh * a.qs + qo + q0 + tid, tid < BQ && q0 + tid < a.n_q);
  };
  auto store_stats = [&](int buf, const RawRowGrad& raw) {
    const RowGrad rg = scale_rowgrad<SETTING>(a, raw);
    const uint64_t neg = __ballot(tid < BQ && rg.gs < 0.f);  // wave 0 holds all BQ <= 64 rows
    if (tid == 0) sneg[buf] = neg != 0;
    if (tid < BQ) {
      sstat[buf][0][tid] = rg.L1;
      sstat[buf][1][tid] = rg.L2;
      sstat[buf][2][tid] = rg.gs;
      if constexpr (SETTING >= 2) {
        sstat[buf][3][tid] = rg.a;
        sstat[buf][4][tid] = rg.b;
      }
    }
  };

  RawRowGrad rgn;
  const TileLoader<T, D1, BQ, NW> ld1(wave, lane);
  const TileLoader<T, D2, BQ, NW> ld2(wave, lane);
  if (ntiles > 0) {
    ld1.issue(lds, Q1, qtl, a.n_q);
    ld2.issue(lds + BQ * D1, Q2, qtl, a.n_q);
    load_stats(qtl, rgn);
    store_stats(0, rgn);
  }

  frag kf1[S1], kf2[S2];
  const bool kv = krow < a.n_k;
#pragma unroll
  for (int s = 0; s < S1; ++s) kf1[s] = frag_global<T, D1>(K1, krow, a.n_k - 1, kv, s, grp);
#pragma unroll
  for (int s = 0; s < S2; ++s) kf2[s] = frag_global<T, D2>(K2, krow, a.n_k - 1, kv, s, grp);

  // FUSED: wave w computes dQ_s columns [32*(w % NB), +32) for query blocks
  // qb = w / NB, w / NB + NW / NB, ...; its B operand K_s[kw0 .. kw0+128)[cols]
  // stays in registers, k = keys in natural order.
  constexpr int NBF = NB < NW ? NB : NW;
  frag kcf[FUSED ? HK : 1];
  if constexpr (FUSED) {
    const int dcol = 32 * (wave % NBF) + col;
    // bf16: the operand is K_s - kbar (see ref_key_col), the same kbar in
    // every workgroup of the head
    float kb = 0.f;
    if constexpr (MF::KPL > 1) kb = ref_key_col(reinterpret_cast<const bf16*>(KS), DS, a.n_k, dcol);
#pragma unroll
    for (int h = 0; h < HK; ++h) {
      if constexpr (MF::KPL == 1) {
        const int key = kw0 + h * MF::KSTEP + grp;
        kcf[h] = key < a.n_k ? (float)KS[(int64_t)key * DS + dcol] : 0.f;
      } else {
#pragma unroll
        for (int e = 0; e < MF::KPL; ++e) {
          const int key = kw0 + h * MF::KSTEP + grp * MF::KPL + e;
          const float v = (float)KS[(int64_t)min(key, a.n_k - 1) * DS + dcol] - kb;
          kcf[h][e] = key < a.n_k ? (T)v : (T)0.f;
        }
      }
    }
  }

  f32x16 dka[NB], dka2[JOINT ? NB2 : 1];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dka[nb] = zero16();
#pragma unroll
  for (int nb = 0; nb < (JOINT ? NB2 : 1); ++nb) dka2[nb] = zero16();
  const bool wave_has_keys = kwave < a.n_k;
  // queries that see this lane's key: [qlo, n_q)
  const int qlo = kv ? (a.causal ? krow - off : 0) : 0x3fffffff;

  // bf16: per-lane LDS offsets computed once (Q1/Q2 rows share them when
  // d1 == d2); fp32 computes addresses per read
  constexpr bool BF = sizeof(T) == 2;
  using RF1 = std::conditional_t<BF, RowFragOffsets<D1, S1>, NoOffsets>;
  using RF2 = std::conditional_t<BF, RowFragOffsets<D2, S2>, NoOffsets>;
  using CF = std::conditional_t<BF, ColFragOffsets<DS, NB>, NoOffsets>;
  using CF2 = std::conditional_t<BF && JOINT, ColFragOffsets<D2, NB2>, NoOffsets>;
  RF1 rf1(col, grp);
  // per-lane byte offset of the stats reads (16 * grp), kept opaque like
  // the offset tables so each stats read is this register plus an immediate
  int stat_off = 16 * grp;
  asm volatile("" : "+v"(stat_off));
  RF2 rf2 = [&]() -> RF2 {
    if constexpr (std::is_same_v<RF1, RF2>) return rf1;
    else return RF2(col, grp);
  }();
  auto row1 = [&](const T* tile, int blk, int s) -> frag {
    if constexpr (BF) return rf1.read(tile, blk, s);
    else return frag_tile<T, D1>(tile, 32 * blk + col, s, grp);
  };
  auto row2 = [&](const T* tile, int blk, int s) -> frag {
    if constexpr (BF) return rf2.read(tile, blk, s);
    else return frag_tile<T, D2>(tile, 32 * blk + col, s, grp);
  };
  CF cf(lane);
  CF2 cf2(lane);
  auto colop = [&](const T* tile, int blk, int nb, int h) -> frag {
    if constexpr (BF) return cf.read(tile, blk, nb, h);
    else return fragcol_acc<T, DS>(tile, 32 * blk, 32 * nb, h, lane);
  };
  auto colop2 = [&](const T* tile, int blk, int nb, int h) -> frag {
    if constexpr (BF && JOINT) return cf2.read(tile, blk, nb, h);
    else return fragcol_acc<T, D2>(tile, 32 * blk, 32 * nb, h, lane);
  };

  // One query tile.  P is the tile's buffer (t & 1): tiles alternate between
  // the two LDS buffers and the loop below steps by two, so each buffer's tile
  // base is a constant and every LDS read is a per-lane offset plus an
  // immediate.
  auto step = [&](int t, auto P) {
    constexpr int B = decltype(P)::value;
    wait_loads();
    __syncthreads();
    const int q0 = qtl - t * BQ;
    const bool more = t + 1 < ntiles;
    if (more) {
      // stats first: vmcnt retires in order, so using them then waits only
      // for these loads, not for the tile loads behind them
      load_stats(q0 - BQ, rgn);
      T* nbuf = lds + (1 - B) * TS;
      ld1.issue(nbuf, Q1, q0 - BQ, a.n_q);
      ld2.issue(nbuf + BQ * D1, Q2, q0 - BQ, a.n_q);
    }
    const T* sQ1 = lds + B * TS;
    const T* sQ2 = sQ1 + BQ * D1;
    const T* sQS = SETTING == 1 ? sQ2 : sQ1;
    const float* st = &sstat[B][0][0];
    const bool tile_signed = sneg[B] != 0;

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qb0 = q0 + 32 * qb;
      const bool active = wave_has_keys && (!a.causal || kwave <= min(a.n_q, qb0 + 32) - 1 + off);
      if (active) {
        f32x16 s1 = zero16(), s2 = zero16();
        constexpr int SM = S1 > S2 ? S1 : S2;
#pragma unroll
        for (int s = 0; s < SM; ++s) {
          if (s < S1) s1 = MF::run(row1(sQ1, qb, s), kf1[s < S1 ? s : 0], s1);
          if (s < S2) s2 = MF::run(row2(sQ2, qb, s), kf2[s < S2 ? s : 0], s2);
        }
        sched_mfma_lds<S1 + S2, 1, 4>();
        const bool need_mask = (qb0 + 32 > a.n_q) || (kwave + 32 > a.n_k) || (a.causal && kwave + 31 > qb0 + off);
        if constexpr (JOINT) {
          if (need_mask) dS_rows_keyouter_joint<true, BQ>(s1, s2, st, 32 * qb, qb0, grp, a.c1, a.c2, qlo, a.n_q, stat_off);
          else dS_rows_keyouter_joint<false, BQ>(s1, s2, st, 32 * qb, qb0, grp, a.c1, a.c2, qlo, a.n_q, stat_off);
#pragma unroll
          for (int h = 0; h < HS; ++h) {
            const frag af1 = frag_from_acc(s1, h, T());
            const frag af2 = frag_from_acc(s2, h, T());
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) dka[nb] = MF::run(af1, colop(sQ1, qb, nb, h), dka[nb]);
#pragma unroll
            for (int nb = 0; nb < NB2; ++nb) dka2[nb] = MF::run(af2, colop2(sQ2, qb, nb, h), dka2[nb]);
          }
          sched_mfma_lds<HS * (NB + NB2), MF::KPL == 1 ? 1 : 2, 2>();
          continue;
        }
        if (SETTING == 2 || tile_signed) {
          if (need_mask) dS_rows_keyouter<SETTING, true, BQ>(s1, s2, st, 32 * qb, qb0, grp, a.c1, a.c2, qlo, a.n_q, stat_off);
          else dS_rows_keyouter<SETTING, false, BQ>(s1, s2, st, 32 * qb, qb0, grp, a.c1, a.c2, qlo, a.n_q, stat_off);
        } else {
          if (need_mask)
            dS_rows_keyouter<SETTING, true, BQ, false>(s1, s2, st, 32 * qb, qb0, grp, a.c1, a.c2, qlo, a.n_q, stat_off);
          else
            dS_rows_keyouter<SETTING, false, BQ, false>(s1, s2, st, 32 * qb, qb0, grp, a.c1, a.c2, qlo, a.n_q, stat_off);
        }
#pragma unroll
        for (int h = 0; h < HS; ++h) {
          const frag af = frag_from_acc(s1, h, T());
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) dka[nb] = MF::run(af, colop(sQS, qb, nb, h), dka[nb]);
        }
        sched_mfma_lds<HS * NB, MF::KPL == 1 ? 1 : 2, 2>();
        if constexpr (FUSED) {
          // dS^T tile in LDS as [key][query]: 4 consecutive queries per store
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            T* p = sdS + Tile<T, BQ>::off(32 * wave + col, 32 * qb + 8 * i + 4 * grp);
            if constexpr (MF::KPL == 1) {
              *reinterpret_cast<f32x4*>(p) = f32x4{s1[4 * i], s1[4 * i + 1], s1[4 * i + 2], s1[4 * i + 3]};
            } else {
              bf16x4 v;
              v[0] = (bf16)s1[4 * i]; v[1] = (bf16)s1[4 * i + 1]; v[2] = (bf16)s1[4 * i + 2]; v[3] = (bf16)s1[4 * i + 3];
              *reinterpret_cast<bf16x4*>(p) = v;
            }
          }
        }
      } else if constexpr (FUSED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          T* p = sdS + Tile<T, BQ>::off(32 * wave + col, 32 * qb + 8 * i + 4 * grp);
          if constexpr (MF::KPL == 1) *reinterpret_cast<f32x4*>(p) = f32x4{0.f, 0.f, 0.f, 0.f};
          else *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
        }
      }
    }
    if (more) {
      __builtin_amdgcn_sched_barrier(0);
      store_stats(1 - B, rgn);
    }

    if constexpr (FUSED) {
      lds_barrier();
      constexpr int QSTEP = NW / NBF;
      // blocks wave / NBF, + QSTEP, ...: a constant trip count with a uniform
      // guard, so the loop unrolls
#pragma unroll
      for (int i = 0; i < (NQB + QSTEP - 1) / QSTEP; ++i) {
        const int qb = wave / NBF + i * QSTEP;
        const int qb0 = q0 + 32 * qb;
        if (qb >= NQB || qb0 >= a.n_q) continue;
        f32x16 dqa = zero16();
#pragma unroll
        for (int h = 0; h < HK; ++h) dqa = MF::run(fragcol_nat<T, BQ>(sdS, 0, 32 * qb, h, lane), kcf[h], dqa);
        const int dcol = 32 * (wave % NBF) + col;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int q = qb0 + acc_row(e, grp);
          if (q < a.n_q) atomicAdd(a.dq + (bh * a.qs + qo + q) * DS + dcol, dqa[e]);
        }
      }
    }
  };

  for (int t = 0; t < ntiles; t += 2) {
    rf1.touch();
    if constexpr (!std::is_same_v<RF1, RF2>) rf2.touch();
    cf.touch();
    cf2.touch();
    asm volatile("" : "+v"(stat_off));
    step(t, std::integral_constant<int, 0>());
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>());
  }

  // dK_s of key head bh / g_s: the query heads that share a key head add
  // their parts with fp32 atomics into the cleared output (once per key and
  // query head); without sharing each element is stored once
  auto put = [&](float* dk, int g, const f32x16* acc, auto D_) {
    constexpr int D = decltype(D_)::value;
    float* base = dk + (key_head(bh, g) * a.ks + ko) * D + col;
    if (g > 1) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kwave + acc_row(e, grp);
          if (key < a.n_k) atomicAdd(base + key * D + nb * 32, acc[nb][e]);
        }
    } else {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kwave + acc_row(e, grp);
          if (key < a.n_k) base[key * D + nb * 32] = acc[nb][e];
        }
    }
  };
  put(a.dk, SETTING == 1 ? a.g2 : a.g1, dka, std::integral_constant<int, DS>());
  if constexpr (JOINT) put(a.dk2, a.g2, dka2, std::integral_constant<int, D2>());
}


// ---------------------------------------------------------------------------
// Decode-shaped backward (at most 32 query rows, long key ranges).  Each key
// tile is visited once, as in the fused mode of Method 2, but the query rows
// are few enough that a workgroup keeps all of them: dK_s is written
// directly and dQ_s is summed over the workgroup's key tiles in registers,
// then added to the caller's cleared dQ once at the end (one fp32 atomic
// per element and wave, instead of one per element and key block).  The
// workgroups of a head split its key tiles between them (split-K, Method 3):
// workgroup z takes tiles z, z + nsplit, ..., so the workgroups running at a
// time sweep through the keys together.
//
// Orientation as in the decode forward: S^T = K Q^T, so an accumulator
// column is one query row and each lane's row statistics are constants.
// Per wave and 32-key block of a tile:
//   dQ_s^T += K_s^T dS^T   A = K_s read down the tile's rows with the
//                          transpose read (keys in accumulator order),
//                          B = dS^T straight from the accumulator
//   dK_s    = dS^T Q_s     A = dS^T read back from a wave-private LDS tile
//                          [query][key] with the transpose read, B = Q_s
//                          columns, held in registers for the whole kernel
// K1 and K2 tiles (32 keys per wave) are double-buffered in LDS.
template <int D1, int D2, int SETTING, typename RT = NoTable>
__global__ __launch_bounds__(256, 1) void bwd_decode_kernel(BwdArgs a, const RT rt) {
  using MF = Mfma<bf16>;
  constexpr int NW = 4, BK = 32 * NW;
  constexpr int DS = SETTING == 1 ? D2 : D1;
  constexpr int S1 = D1 / 16, S2 = D2 / 16, NB = DS / 32;
  constexpr int TS = BK * (D1 + D2);  // elements of one tile stage (K1 then K2)
  constexpr int QE = 32 * (D1 + D2);  // Q1 and Q2, 32 rows each
  constexpr int DSE = 32 * 32;        // one wave's dS^T tile
  // one array: separate __shared__ objects get separate alias scopes, and the
  // tile reads would then wait for the next tile's direct loads in flight;
  // the reference key kbar (DS floats) at the end
  __shared__ __attribute__((aligned(1024))) bf16 lds[2 * TS + QE + NW * DSE + 2 * DS];
  bf16* sQ1 = lds + 2 * TS;
  bf16* sQ2 = sQ1 + 32 * D1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;
  bf16* sdS = lds + 2 * TS + QE + wave * DSE;
  float* kbar = reinterpret_cast<float*>(lds + 2 * TS + QE + NW * DSE);
  int64_t lin = blockIdx.x, head0 = 0;
  int qo = 0, ko = 0;  // the element's first query and key rows within a head (packed batches)
  if constexpr (kRagged<RT>) {  // one element of a ragged batch
    const RaggedItem r = ragged_item(rt, lin);
    qo = r.qoff;
    ko = r.koff;
    if (r.pad) return;
    lin = r.lin;
    head0 = r.head0;
    a.n_q = r.n_q;
    a.n_k = r.n_k;
    a.nblk = r.nblk;
  }
  // 32-bit division: the grid and every element's range hold fewer than 2^31 workgroups
  const unsigned lw = (unsigned)lin, nb = (unsigned)a.nblk;
  const int64_t bh = head0 + lw / nb;
  const int z = (int)(lw % nb);
  const int off = a.n_k - a.n_q;

  const bf16* Q1 = reinterpret_cast<const bf16*>(a.q1) + (bh * (int64_t)a.qs + qo) * D1;
  const bf16* K1 = reinterpret_cast<const bf16*>(a.k1) + (key_head(bh, a.g1) * (int64_t)a.ks + ko) * D1;
  const bf16* Q2 = reinterpret_cast<const bf16*>(a.q2) + (bh * (int64_t)a.qs + qo) * D2;
  const bf16* K2 = reinterpret_cast<const bf16*>(a.k2) + (key_head(bh, a.g2) * (int64_t)a.ks + ko) * D2;

  const int ntile = (a.n_k + BK - 1) / BK;
  const int count = z < ntile ? (ntile - z + a.nblk - 1) / a.nblk : 0;
  const TileLoader<bf16, D1, BK, NW> ld1(wave, lane);
  const TileLoader<bf16, D2, BK, NW> ld2(wave, lane);
  auto issue = [&](int t, int buf) {
    const int k0 = (z + t * a.nblk) * BK;
    bf16* s = lds + buf * TS;
    ld1.issue(s, K1, k0, a.n_k);
    ld2.issue(s + BK * D1, K2, k0, a.n_k);
  };
  if (count > 0) issue(0, 0);
  dec_stage_q<D1>(sQ1, Q1, a.n_q, tid);
  dec_stage_q<D2>(sQ2, Q2, a.n_q, tid);
  ref_key<DS>(kbar, SETTING == 1 ? K2 : K1, a.n_k, tid, 256);
  // lane column col is query row col: its statistics are fixed for the kernel
  const bool qv = col < a.n_q;
  const RowGrad rg = load_rowgrad<SETTING>(a, bh * a.qs + qo + col, qv);
  const float c1 = a.c1, c2 = a.c2;
  // last key this lane's query sees, and the last key of which every query
  // of a wave block is visible (beyond it blocks take the element mask)
  const int lim = a.causal ? col + off : a.n_k - 1;
  const int mask_from = a.causal ? off : a.n_k - 1;
  __syncthreads();

  // B operand of dK_s = dS^T Q_s: Q_s columns, k = query rows in natural order
  const bf16* sQS = SETTING == 1 ? sQ2 : sQ1;
  bf16x8 qcol[2][NB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) qcol[h][nb] = fragcol_nat_bf16<DS>(sQS, 0, 32 * nb, h, lane);

  f32x16 dqa[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dqa[nb] = zero16();
  float rsum = 0.f;  // this lane's part of r for query col: the sum of the bf16 dS it fed

  auto tile = [&](const bf16* __restrict__ sK1, const bf16* __restrict__ sK2, const bf16* __restrict__ sQa,
                  const bf16* __restrict__ sQb, int kw) {
    f32x16 s1 = zero16(), s2 = zero16();
    constexpr int SM = S1 > S2 ? S1 : S2;
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      if (s < S1)
        s1 = MF::run(frag_tile<bf16, D1>(sK1, 32 * wave + col, s < S1 ? s : 0, grp),
                     frag_tile<bf16, D1>(sQa, col, s < S1 ? s : 0, grp), s1);
      if (s < S2)
        s2 = MF::run(frag_tile<bf16, D2>(sK2, 32 * wave + col, s < S2 ? s : 0, grp),
                     frag_tile<bf16, D2>(sQb, col, s < S2 ? s : 0, grp), s2);
    }
    // dS^T in s1 (element e: key kw + acc_row(e, grp), query col)
    const bool need_mask = kw + 31 > mask_from;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float ds = dS_elem<SETTING>(s1[e], s2[e], c1, c2, rg.L1, rg.L2, rg.gs, rg.a, rg.b);
      if (need_mask) ds = kw + acc_row(e, grp) <= lim ? ds : 0.f;
      s1[e] = qv ? ds : 0.f;
    }
    const bf16* sKS = SETTING == 1 ? sK2 : sK1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 b = frag_from_acc(s1, h, bf16());
      rsum = sum_frag(b, rsum);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        dqa[nb] = MF::run(fragcol_acc_bf16<DS>(sKS, 32 * wave, 32 * nb, h, lane), b, dqa[nb]);
    }
    // dS^T to the wave's own [query][key] tile: 4 consecutive keys per store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 v;
      v[0] = (bf16)s1[4 * i]; v[1] = (bf16)s1[4 * i + 1]; v[2] = (bf16)s1[4 * i + 2]; v[3] = (bf16)s1[4 * i + 3];
      *reinterpret_cast<bf16x4*>(sdS + Tile<bf16, 32>::off(col, 8 * i + 4 * grp)) = v;
    }
    // one wave writes and reads its tile; LDS serves a wave's accesses in order
    asm volatile("" ::: "memory");
    f32x16 dka[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) dka[nb] = zero16();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 af = fragcol_nat_bf16<32>(sdS, 0, 0, h, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) dka[nb] = MF::run(af, qcol[h][nb], dka[nb]);
    }
    const int gs = SETTING == 1 ? a.g2 : a.g1;
    float* dk = a.dk + (key_head(bh, gs) * a.ks + ko + kw) * (int64_t)DS + col;
    const int kleft = a.n_k - kw;
    if (gs > 1) {
      // query heads sharing a key head add their parts into the cleared dK
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(e, grp) < kleft) atomicAdd(dk + acc_row(e, grp) * DS + 32 * nb, dka[nb][e]);
    } else if (kleft >= 32) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        // dK is written once and not read again here: non-temporal stores
        for (int e = 0; e < 16; ++e) __builtin_nontemporal_store(dka[nb][e], dk + acc_row(e, grp) * DS + 32 * nb);
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(e, grp) < kleft) dk[acc_row(e, grp) * DS + 32 * nb] = dka[nb][e];
    }
  };

  for (int t = 0; t < count; ++t) {
    wait_loads();
    __syncthreads();
    if (t + 1 < count) issue(t + 1, (t + 1) & 1);
    const bf16* sK1 = lds + (t & 1) * TS;
    const int kw = (z + t * a.nblk) * BK + 32 * wave;
    if (kw < a.n_k) tile(sK1, sK1 + BK * D1, sQ1, sQ2, kw);
  }

  // the workgroups of a head add r kbar for their own key tiles, with the
  // same kbar: the sum over them is the row's r kbar
  rsum += __shfl_xor(rsum, 32);
  if (qv) {
    float* dq = a.dq + (bh * a.qs + qo + col) * (int64_t)DS;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 kb = *reinterpret_cast<const f32x4*>(kbar + 32 * nb + 8 * i + 4 * grp);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * i + j;
          atomicAdd(dq + 32 * nb + acc_row(e, grp), fmaf(-rsum, kb[j], dqa[nb][e]));
        }
      }
  }
}

}  // namespace streamkl
