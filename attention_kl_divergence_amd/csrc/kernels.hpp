// StreamKL kernels for gfx950: one-pass forward (optionally split over keys),
// split merge, key-outer backward (dK, optionally fused dQ by atomics) and
// query-outer backward (dQ).
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
#pragma once

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
  int64_t BH;
  int n_q, n_k;
  int nsplit;
  int keys_per_split;  // multiple of the key tile
  int nqb;             // query blocks per head
  int causal;
  float c1, c2;        // scale_t * log2(e)
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
  float* dq;
  float* dk;
  int64_t BH;
  int n_q, n_k;
  int nblk;            // query blocks (dQ kernel) or key blocks (dK kernel) per head
  int causal;
  float c1, c2;        // scale_t * log2(e)
  float scale_s;       // scale of the model that receives gradients
};

// Cooperative copy of `ROWS` rows of a [*, D] row-major global tensor (rows
// r0.., rows >= rend read as zero) into LDS with leading dimension LD.
template <typename T, int D, int LD, int ROWS, int NT>
__device__ inline void load_rows(T* __restrict__ s, const T* __restrict__ g, int r0, int rend, int tid) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = D / EPC;
  constexpr int TOTAL = ROWS * CPR;
#pragma unroll
  for (int c0 = 0; c0 < TOTAL; c0 += NT) {
    const int c = c0 + tid;
    if (TOTAL % NT == 0 || c < TOTAL) {
      const int r = c / CPR, cc = c % CPR;
      Chunk16 v = {{0u, 0u, 0u, 0u}};
      if (r0 + r < rend) v = *reinterpret_cast<const Chunk16*>(g + (int64_t)(r0 + r) * D + cc * EPC);
      *reinterpret_cast<Chunk16*>(s + r * LD + cc * EPC) = v;
    }
  }
}

// Same rows stored transposed: sT[d][r] (leading dimension LDT).
template <typename T, int D, int LDT, int ROWS, int NT>
__device__ inline void load_rows_T(T* __restrict__ sT, const T* __restrict__ g, int r0, int rend, int tid) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = D / EPC;
  constexpr int TOTAL = ROWS * CPR;
#pragma unroll
  for (int c0 = 0; c0 < TOTAL; c0 += NT) {
    const int c = c0 + tid;
    if (TOTAL % NT == 0 || c < TOTAL) {
      const int r = c % ROWS, cc = c / ROWS;
      Chunk16 v = {{0u, 0u, 0u, 0u}};
      if (r0 + r < rend) v = *reinterpret_cast<const Chunk16*>(g + (int64_t)(r0 + r) * D + cc * EPC);
      const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int i = 0; i < EPC; ++i) sT[(cc * EPC + i) * LDT + r] = e[i];
    }
  }
}

template <typename T>
__device__ inline typename Mfma<T>::frag zero_frag() {
  typename Mfma<T>::frag f;
  if constexpr (Mfma<T>::KPL == 1) {
    f = 0.f;
  } else {
#pragma unroll
    for (int e = 0; e < Mfma<T>::KPL; ++e) f[e] = (T)0.f;
  }
  return f;
}

// ---------------------------------------------------------------------------
// Forward.  Workgroup = WQ waves, each owning 32 query rows; the workgroup
// streams key tiles of BK rows of K1 and K2 through LDS.  Each wave computes
// S^T = K Q^T so a lane's accumulator column is one query row: lane
// (col, grp) keeps its own running state over the keys acc_row(., grp) of
// every 32-key block, and the two lane groups merge once at the end.
template <typename T, int D1, int D2, int WQ, int BK>
__global__ __launch_bounds__(64 * WQ) void fwd_kernel(FwdArgs a) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LD1 = D1 + PAD, LD2 = D2 + PAD;
  constexpr int NT = 64 * WQ;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int NKB = BK / 32;
  __shared__ __attribute__((aligned(16))) T sK1[BK * LD1];
  __shared__ __attribute__((aligned(16))) T sK2[BK * LD2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;
  int64_t lin = blockIdx.x;
  const int z = (int)(lin % a.nsplit);
  lin /= a.nsplit;
  const int64_t bh = lin % a.BH;
  const int qb = a.nqb - 1 - (int)(lin / a.BH);  // longest causal rows first
  const int qwg0 = qb * 32 * WQ;
  const int q0 = qwg0 + 32 * wave;
  const int qrow = q0 + col;
  const int off = a.n_k - a.n_q;

  const T* Q1 = reinterpret_cast<const T*>(a.q1) + bh * (int64_t)a.n_q * D1;
  const T* K1 = reinterpret_cast<const T*>(a.k1) + bh * (int64_t)a.n_k * D1;
  const T* Q2 = reinterpret_cast<const T*>(a.q2) + bh * (int64_t)a.n_q * D2;
  const T* K2 = reinterpret_cast<const T*>(a.k2) + bh * (int64_t)a.n_k * D2;

  const int kbeg = z * a.keys_per_split;
  int kend = min(a.n_k, kbeg + a.keys_per_split);
  if (a.causal) kend = min(kend, min(a.n_q, qwg0 + 32 * WQ) - 1 + off + 1);
  const bool wave_rows = q0 < a.n_q;
  const int wave_kmax = a.causal ? (min(a.n_q, q0 + 32) - 1 + off) : 0x7fffffff;

  frag qf1[S1], qf2[S2];
#pragma unroll
  for (int s = 0; s < S1; ++s) qf1[s] = qrow < a.n_q ? frag_rowmajor(Q1 + (int64_t)q0 * D1, D1, s, col, grp) : zero_frag<T>();
#pragma unroll
  for (int s = 0; s < S2; ++s) qf2[s] = qrow < a.n_q ? frag_rowmajor(Q2 + (int64_t)q0 * D2, D2, s, col, grp) : zero_frag<T>();

  RowState st = empty_state();
  const float c1 = a.c1, c2 = a.c2;

  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    __syncthreads();
    load_rows<T, D1, LD1, BK, NT>(sK1, K1, k0, kend, tid);
    load_rows<T, D2, LD2, BK, NT>(sK2, K2, k0, kend, tid);
    __syncthreads();
    if (!wave_rows || k0 > wave_kmax) continue;
    const bool need_mask = (k0 + BK > kend) || (a.causal && k0 + BK - 1 > q0 + off);

    f32x16 s1[NKB], s2[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s1[kb] = zero16();
      s2[kb] = zero16();
#pragma unroll
      for (int s = 0; s < S1; ++s) s1[kb] = MF::run(frag_rowmajor(sK1 + kb * 32 * LD1, LD1, s, col, grp), qf1[s], s1[kb]);
#pragma unroll
      for (int s = 0; s < S2; ++s) s2[kb] = MF::run(frag_rowmajor(sK2 + kb * 32 * LD2, LD2, s, col, grp), qf2[s], s2[kb]);
    }

    if (need_mask) {
      const int lim = a.causal ? min(kend - 1, qrow + off) : kend - 1;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb * 32 + acc_row(e, grp);
          if (key > lim) { s1[kb][e] = kNegInf; s2[kb][e] = kNegInf; }
        }
    }

    float mx1[4] = {kNegInf, kNegInf, kNegInf, kNegInf}, mx2[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        mx1[e & 3] = fmaxf(mx1[e & 3], s1[kb][e]);
        mx2[e & 3] = fmaxf(mx2[e & 3], s2[kb][e]);
      }
    const float tmx1 = fmaxf(fmaxf(mx1[0], mx1[1]), fmaxf(mx1[2], mx1[3]));
    const float tmx2 = fmaxf(fmaxf(mx2[0], mx2[1]), fmaxf(mx2[2], mx2[3]));
    const float M1n = fmaxf(st.M1, tmx1 * c1), M2n = fmaxf(st.M2, tmx2 * c2);
    const float m1 = finite_or_zero(M1n), m2 = finite_or_zero(M2n);
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
        if (need_mask) d = (s1[kb][e] == kNegInf) ? 0.f : d;  // never form the ratio on masked keys
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

  st = merge_state(st, shfl_xor_state(st, 32));
  if (grp == 0 && qrow < a.n_q) {
    const int64_t r = bh * a.n_q + qrow;
    if (a.nsplit == 1) {
      finish_state(st, a.kl + r, a.lse1 + r, a.lse2 + r);
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
}

// Per-row quantities the backward needs, in base-2 units:
// L_t = LSE_t * log2(e); gs = g * scale_s; setting 2 also a = gs * ln2 and
// b = gs * KL, so that dS1 = P1 * (a * (t1 - t2) - b) with t_t = y_t - L_t.
struct RowGrad {
  float L1, L2, gs, a, b;
};

template <int SETTING>
__device__ inline RowGrad load_rowgrad(const BwdArgs& a, int64_t r) {
  RowGrad o;
  o.L1 = a.lse1[r] * kLog2e;
  o.L2 = a.lse2[r] * kLog2e;
  o.gs = a.g[r] * a.scale_s;
  if constexpr (SETTING == 2) {
    o.a = o.gs * kLn2;
    o.b = o.gs * a.kl[r];
  } else {
    o.a = 0.f;
    o.b = 0.f;
  }
  return o;
}

// dS for one element from the raw dot products s1, s2 (see RowGrad).
template <int SETTING>
__device__ inline float dS_elem(float s1, float s2, float c1, float c2, float L1, float L2, float gs, float ra,
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

template <typename T>
__device__ inline T to_T(float x) { return (T)x; }

// ---------------------------------------------------------------------------
// Query-outer backward: dQ_s for 32 query rows per wave (4 waves), key tiles
// of BK rows streamed through LDS (K1, K2 row-major for the logits, K_s
// transposed for the dQ contraction).  Deterministic; no atomics.
template <typename T, int D1, int D2, int SETTING, int BK>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int DS = SETTING == 1 ? D2 : D1;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LD1 = D1 + PAD, LD2 = D2 + PAD, LDT = BK + PAD;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int NKB = BK / 32, NB = DS / 32, HS = 32 / MF::KSTEP;
  __shared__ __attribute__((aligned(16))) T sK1[BK * LD1];
  __shared__ __attribute__((aligned(16))) T sK2[BK * LD2];
  __shared__ __attribute__((aligned(16))) T sKT[DS * LDT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;
  const int64_t lin = blockIdx.x;
  const int64_t bh = lin % a.BH;
  const int qb = a.nblk - 1 - (int)(lin / a.BH);
  const int q0 = qb * 128 + 32 * wave;
  const int qrow = q0 + col;
  const int off = a.n_k - a.n_q;

  const T* Q1 = reinterpret_cast<const T*>(a.q1) + bh * (int64_t)a.n_q * D1;
  const T* K1 = reinterpret_cast<const T*>(a.k1) + bh * (int64_t)a.n_k * D1;
  const T* Q2 = reinterpret_cast<const T*>(a.q2) + bh * (int64_t)a.n_q * D2;
  const T* K2 = reinterpret_cast<const T*>(a.k2) + bh * (int64_t)a.n_k * D2;
  const T* KS = SETTING == 1 ? K2 : K1;

  int kend = a.n_k;
  if (a.causal) kend = min(kend, min(a.n_q, qb * 128 + 128) - 1 + off + 1);
  const bool wave_rows = q0 < a.n_q;
  const int wave_kmax = a.causal ? (min(a.n_q, q0 + 32) - 1 + off) : 0x7fffffff;

  frag qf1[S1], qf2[S2];
#pragma unroll
  for (int s = 0; s < S1; ++s) qf1[s] = qrow < a.n_q ? frag_rowmajor(Q1 + (int64_t)q0 * D1, D1, s, col, grp) : zero_frag<T>();
#pragma unroll
  for (int s = 0; s < S2; ++s) qf2[s] = qrow < a.n_q ? frag_rowmajor(Q2 + (int64_t)q0 * D2, D2, s, col, grp) : zero_frag<T>();
  RowGrad rg = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (qrow < a.n_q) rg = load_rowgrad<SETTING>(a, bh * a.n_q + qrow);

  f32x16 dqa[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dqa[nb] = zero16();

  for (int k0 = 0; k0 < kend; k0 += BK) {
    __syncthreads();
    load_rows<T, D1, LD1, BK, 256>(sK1, K1, k0, kend, tid);
    load_rows<T, D2, LD2, BK, 256>(sK2, K2, k0, kend, tid);
    load_rows_T<T, DS, LDT, BK, 256>(sKT, KS, k0, kend, tid);
    __syncthreads();
    if (!wave_rows || k0 > wave_kmax) continue;
    const bool need_mask = (k0 + BK > kend) || (a.causal && k0 + BK - 1 > q0 + off);
    const int lim = a.causal ? min(kend - 1, qrow + off) : kend - 1;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s1 = zero16(), s2 = zero16();
#pragma unroll
      for (int s = 0; s < S1; ++s) s1 = MF::run(frag_rowmajor(sK1 + kb * 32 * LD1, LD1, s, col, grp), qf1[s], s1);
#pragma unroll
      for (int s = 0; s < S2; ++s) s2 = MF::run(frag_rowmajor(sK2 + kb * 32 * LD2, LD2, s, col, grp), qf2[s], s2);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float ds = dS_elem<SETTING>(s1[e], s2[e], a.c1, a.c2, rg.L1, rg.L2, rg.gs, rg.a, rg.b);
        if (need_mask && k0 + kb * 32 + acc_row(e, grp) > lim) ds = 0.f;
        s1[e] = ds;
      }
#pragma unroll
      for (int h = 0; h < HS; ++h) {
        const frag af = frag_from_acc(s1, h, T());
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          dqa[nb] = MF::run(af, fragT_accorder(sKT + nb * 32 * LDT, LDT, kb * 32, h, col, grp, T()), dqa[nb]);
      }
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int q = q0 + acc_row(e, grp);
      if (q < a.n_q) a.dq[(bh * a.n_q + q) * DS + nb * 32 + col] = dqa[nb][e];
    }
}

// ---------------------------------------------------------------------------
// Key-outer backward: each wave owns 32 key rows (workgroup: 4 waves, 128
// keys), keeps K1, K2 in registers and accumulates dK_s in registers while
// query tiles of 32 rows stream through LDS.  The logits are computed as
// S = Q K^T so a lane's accumulator column is one key.  FUSED additionally
// forms dQ_s for every query tile from the same dS (written to LDS) and adds
// it to global dQ_s with fp32 atomics: each query-key pair is visited once.
template <typename T, int D1, int D2, int SETTING, bool FUSED>
__global__ __launch_bounds__(256) void bwd_dk_kernel(BwdArgs a) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int BQ = 32, WK = 4, BKW = 32 * WK;
  constexpr int DS = SETTING == 1 ? D2 : D1;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LD1 = D1 + PAD, LD2 = D2 + PAD, LDT = BQ + PAD, LDD = BKW + PAD;
  constexpr int S1 = D1 / MF::KSTEP, S2 = D2 / MF::KSTEP;
  constexpr int NB = DS / 32, HS = 32 / MF::KSTEP, HK = BKW / MF::KSTEP;
  __shared__ __attribute__((aligned(16))) T sQ1[BQ * LD1];
  __shared__ __attribute__((aligned(16))) T sQ2[BQ * LD2];
  __shared__ __attribute__((aligned(16))) T sQT[DS * LDT];
  __shared__ __attribute__((aligned(16))) float sL1[BQ], sL2[BQ], sGS[BQ], sRA[BQ], sRB[BQ];
  __shared__ __attribute__((aligned(16))) T sdS[FUSED ? BQ * LDD : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;
  const int64_t lin = blockIdx.x;
  const int64_t bh = lin % a.BH;
  const int kb = (int)(lin / a.BH);  // low key blocks see the most queries under causal masks: first
  const int kw0 = kb * BKW;
  const int kwave = kw0 + 32 * wave;
  const int krow = kwave + col;
  const int off = a.n_k - a.n_q;

  const T* Q1 = reinterpret_cast<const T*>(a.q1) + bh * (int64_t)a.n_q * D1;
  const T* K1 = reinterpret_cast<const T*>(a.k1) + bh * (int64_t)a.n_k * D1;
  const T* Q2 = reinterpret_cast<const T*>(a.q2) + bh * (int64_t)a.n_q * D2;
  const T* K2 = reinterpret_cast<const T*>(a.k2) + bh * (int64_t)a.n_k * D2;
  const T* QS = SETTING == 1 ? Q2 : Q1;
  const T* KS = SETTING == 1 ? K2 : K1;

  frag kf1[S1], kf2[S2];
#pragma unroll
  for (int s = 0; s < S1; ++s) kf1[s] = krow < a.n_k ? frag_rowmajor(K1 + (int64_t)kwave * D1, D1, s, col, grp) : zero_frag<T>();
#pragma unroll
  for (int s = 0; s < S2; ++s) kf2[s] = krow < a.n_k ? frag_rowmajor(K2 + (int64_t)kwave * D2, D2, s, col, grp) : zero_frag<T>();

  // FUSED: this wave's dQ task is the 32-column block `wave` of dQ_s; it needs
  // K_s[kw0 .. kw0+128)[32*wave + col] as the B operand, k = keys in order.
  constexpr int NTASK = FUSED ? (NB < WK ? NB : WK) : 0;
  frag kcf[FUSED ? HK : 1];
  if constexpr (FUSED) {
    if (wave < NTASK) {
#pragma unroll
      for (int h = 0; h < HK; ++h) {
        if constexpr (MF::KPL == 1) {
          const int key = kw0 + h * MF::KSTEP + grp;
          kcf[h] = key < a.n_k ? (float)KS[(int64_t)key * DS + 32 * wave + col] : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < MF::KPL; ++e) {
            const int key = kw0 + h * MF::KSTEP + grp * MF::KPL + e;
            kcf[h][e] = key < a.n_k ? KS[(int64_t)key * DS + 32 * wave + col] : (T)0.f;
          }
        }
      }
    }
  }

  f32x16 dka[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dka[nb] = zero16();

  const int qbeg = a.causal ? max(0, kw0 - off) : 0;
  const int wave_has_keys = kwave < a.n_k;
  for (int q0 = (qbeg / BQ) * BQ; q0 < a.n_q; q0 += BQ) {
    __syncthreads();
    load_rows<T, D1, LD1, BQ, 256>(sQ1, Q1, q0, a.n_q, tid);
    load_rows<T, D2, LD2, BQ, 256>(sQ2, Q2, q0, a.n_q, tid);
    load_rows_T<T, DS, LDT, BQ, 256>(sQT, QS, q0, a.n_q, tid);
    if (tid < BQ) {
      RowGrad rg = {0.f, 0.f, 0.f, 0.f, 0.f};
      if (q0 + tid < a.n_q) rg = load_rowgrad<SETTING>(a, bh * a.n_q + q0 + tid);
      sL1[tid] = rg.L1;
      sL2[tid] = rg.L2;
      sGS[tid] = rg.gs;
      sRA[tid] = rg.a;
      sRB[tid] = rg.b;
    }
    __syncthreads();
    const bool active = wave_has_keys && (!a.causal || kwave <= min(a.n_q, q0 + BQ) - 1 + off);
    if (active) {
      const bool need_mask = (q0 + BQ > a.n_q) || (kwave + 32 > a.n_k) || (a.causal && kwave + 31 > q0 + off);
      f32x16 s1 = zero16(), s2 = zero16();
#pragma unroll
      for (int s = 0; s < S1; ++s) s1 = MF::run(frag_rowmajor(sQ1, LD1, s, col, grp), kf1[s], s1);
#pragma unroll
      for (int s = 0; s < S2; ++s) s2 = MF::run(frag_rowmajor(sQ2, LD2, s, col, grp), kf2[s], s2);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ql = acc_row(e, grp);
        float ds = dS_elem<SETTING>(s1[e], s2[e], a.c1, a.c2, sL1[ql], sL2[ql], sGS[ql], sRA[ql], sRB[ql]);
        if (need_mask) {
          const int q = q0 + ql;
          const bool ok = q < a.n_q && krow < a.n_k && (!a.causal || krow <= q + off);
          if (!ok) ds = 0.f;
        }
        s1[e] = ds;
      }
#pragma unroll
      for (int h = 0; h < HS; ++h) {
        const frag af = frag_from_acc(s1, h, T());
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          dka[nb] = MF::run(af, fragT_accorder(sQT + nb * 32 * LDT, LDT, 0, h, col, grp, T()), dka[nb]);
      }
      if constexpr (FUSED) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sdS[acc_row(e, grp) * LDD + 32 * wave + col] = to_T<T>(s1[e]);
      }
    } else if constexpr (FUSED) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sdS[acc_row(e, grp) * LDD + 32 * wave + col] = to_T<T>(0.f);
    }
    if constexpr (FUSED) {
      __syncthreads();
      if (wave < NTASK) {
        f32x16 dqa = zero16();
#pragma unroll
        for (int h = 0; h < HK; ++h) dqa = MF::run(frag_rowmajor(sdS, LDD, h, col, grp), kcf[h], dqa);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int q = q0 + acc_row(e, grp);
          if (q < a.n_q) atomicAdd(a.dq + (bh * a.n_q + q) * DS + 32 * wave + col, dqa[e]);
        }
      }
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kwave + acc_row(e, grp);
      if (key < a.n_k) a.dk[(bh * a.n_k + key) * DS + nb * 32 + col] = dka[nb][e];
    }
}

}  // namespace streamkl
