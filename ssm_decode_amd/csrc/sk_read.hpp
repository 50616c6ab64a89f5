// Non-flush sketched-read kernels.  They never touch the state S: each step
// reads the sketch U, the buffered ring entries and the fixed coefficient
// map C, appends the step's entry to the ring and advances the ring count.
#pragma once

#include "sk_device.hpp"
#include "sk_params.hpp"

namespace sk {

// ---------------------------------------------------------------- Mamba-2
constexpr int M2R_MAXHPG = 16;     // heads per B/C group (at most)
// The query's coordinates in each head's sketch basis, before the decay:
// cq[b][off_h + j] = (C_h q_b)_j, fp32, for every sequence and coefficient
// row.  C is shared by every sequence, so one workgroup takes a block of
// CQ_NB sequences, one B/C group and a block of CQ_ROWS of the group's
// coefficient rows, and reads those rows of C once: CQ_LPR lanes hold one
// row in registers, each forming the dot products of its segment with every
// sequence's query (staged in LDS).  The coefficient rows are loaded first,
// and every load is issued before the first wait.
constexpr int CQ_NB = 8;           // sequences per workgroup
constexpr int CQ_THREADS = 256;
constexpr int CQ_LPR = 4;          // lanes per coefficient row
constexpr int CQ_ROWS = CQ_THREADS / CQ_LPR;
constexpr int CQ_ZBLOCKS = (M2R_MAXHPG * 16 + CQ_ROWS - 1) / CQ_ROWS;

template <int DK, typename AT>
__global__ void __launch_bounds__(CQ_THREADS) m2_cq_kernel(Params p) {
  constexpr int SEGC = DK / CQ_LPR;              // row elements per lane
  constexpr int QCH = CQ_NB * DK / 4;            // 4-element query chunks per block
  constexpr int QIT = (QCH + CQ_THREADS - 1) / CQ_THREADS;
  static_assert(SEGC % 4 == 0, "row segments are read as float4");
  __shared__ float s_q[CQ_NB][DK];
  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int roff0 = p.off[g * p.HPG];
  const int rows = p.off[(g + 1) * p.HPG] - roff0;
  const int rb = blockIdx.z * CQ_ROWS;
  if (rb >= rows) return;                        // uniform: no rows in this block
  const int b0 = blockIdx.x * CQ_NB;
  const int nb = min(CQ_NB, p.B - b0);
  const int row = rb + tid / CQ_LPR;
  const int qt = tid & (CQ_LPR - 1);
  float c[SEGC];
  if (row < rows) {
    ldn<SEGC>(p.C + (size_t)(roff0 + row) * DK + qt * SEGC, c);
  } else {
#pragma unroll
    for (int e = 0; e < SEGC; ++e) c[e] = 0.f;
  }
  const AT* q = reinterpret_cast<const AT*>(p.q);
  float qv[QIT][4];
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int i = tid + it * CQ_THREADS;
    const int bb = (4 * i) / DK, e = 4 * i - bb * DK;
    if (bb < nb) ld4(q + ((size_t)(b0 + bb) * p.G + g) * DK + e, qv[it]);
  }
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int i = tid + it * CQ_THREADS;
    const int bb = (4 * i) / DK, e = 4 * i - bb * DK;
    if (bb < nb) *reinterpret_cast<float4*>(&s_q[bb][e]) = make_float4(qv[it][0], qv[it][1], qv[it][2], qv[it][3]);
  }
  __syncthreads();
  float* cq = reinterpret_cast<float*>(p.work);
#pragma unroll
  for (int bb = 0; bb < CQ_NB; ++bb) {
    if (bb < nb) {
      const float* qs = &s_q[bb][qt * SEGC];
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int e = 0; e < SEGC; e += 4) {
        const float4 qq = *reinterpret_cast<const float4*>(qs + e);
        a0 += c[e] * qq.x;
        a1 += c[e + 1] * qq.y;
        a2 += c[e + 2] * qq.z;
        a3 += c[e + 3] * qq.w;
      }
      const float acc = xsum<0, ilog2c(CQ_LPR)>((a0 + a1) + (a2 + a3));
      if (qt == 0 && row < rows) cq[(size_t)(b0 + bb) * p.R + roff0 + row] = acc;
    }
  }
}

// Sketched read: one workgroup per (sequence, B/C group), LPH lanes per head
// of the group.  The group's heads share k and q, so the dot products
// d_i = k_i . q are formed once per workgroup.  For head h with n entries
// (the step's own entry last):
//   q~ = D q, D = prod_i a_i;   o_buf = sum_i w_i d_i v_i, w_i = dt_i prod_{t>i} a_t
//   o  = D * U_h cq_h + o_buf,  cq_h = C_h q (from m2_cq_kernel)
// Lane s of a head holds the q/k segment s (DK/LPH elements) for the dot
// products, ring slots s*SPL.. for the decay scan, and output columns
// s*CPL.. .  The loads are issued in the order their values are needed (the
// memory counter retires them in order): step inputs, cq, the ring keys and
// gates, then the sketch rows and ring values, which stay packed in
// registers until the output sum.  The append stores the step's entry from
// the registers that hold it.
#ifndef SK_M2R_LPH
#define SK_M2R_LPH 16              // lanes per head
#endif
constexpr int M2R_LPH = SK_M2R_LPH;

// lanes per head for a head shape (at least one key element and one output
// column per lane)
template <int DK, int DV>
struct M2ReadLanes {
  static constexpr int v0 = M2R_LPH < DK ? M2R_LPH : DK;
  static constexpr int LPH = v0 < DV ? v0 : DV;
};

template <int N, typename T>
__device__ __forceinline__ void stv(T* p, const VecN<T, N>& x) {
  *reinterpret_cast<VecN<T, N>*>(p) = x;
}

template <int DK, int DV, typename AT, typename UT, int WMAX>
__global__ void __launch_bounds__((M2ReadLanes<DK, DV>::LPH * M2R_MAXHPG)) m2_read_kernel(Params p) {
  constexpr int LPH = M2ReadLanes<DK, DV>::LPH;
  constexpr int LB = ilog2c(LPH);
  constexpr int SEG = DK / LPH;                  // key / query elements per lane
  constexpr int CPL = DV / LPH;                  // output columns per lane
  constexpr int SPL = WMAX >= LPH ? WMAX / LPH : 1;  // ring slots per lane in the decay scan
  static_assert(SEG >= 1 && CPL >= 1, "head dims too small for the lane split");
  static_assert(LPH >= 16, "one cq row per thread needs 16 lanes per head");
  __shared__ float s_d[WMAX];                    // d_i = k_i . q
  __shared__ float s_c[M2R_MAXHPG * 16];         // cq rows of the group

  const int tid = threadIdx.x;
  const int hh = tid >> LB;                      // head within the group
  const int s = tid & (LPH - 1);
  const int W = p.W, HPG = p.HPG;
  const int b = blockIdx.x / p.G;
  const int g = blockIdx.x - b * p.G;
  const int h0 = g * HPG;
  const int h = h0 + hh;
  const size_t bg = (size_t)b * p.G + g;
  const size_t bh = (size_t)b * p.H + h;

  // ---------------------------------------------------- ring counts
  const int n0g = p.count[(size_t)b * p.H + h0];  // the group's fill (uniform)
  const int mine = p.count[bh];
  const int off = p.off[h];
  const int r = p.off[h + 1] - off;
  const int roff0 = p.off[h0];
  const int rows = p.off[h0 + HPG] - roff0;
  const float Ah = p.A[h];
  int bad = (n0g < 0 || n0g >= W) ? ERRBIT_COUNT : 0;
  if (mine != n0g) bad |= ERRBIT_GROUP;
  const int n0 = (n0g < 0 || n0g >= W) ? 0 : n0g; // in range for every address below
  const int n = n0 + 1;

  const AT* q = reinterpret_cast<const AT*>(p.q) + bg * DK;
  const AT* kin = reinterpret_cast<const AT*>(p.k) + bg * DK;
  const AT* vin = reinterpret_cast<const AT*>(p.v) + bh * DV;
  const AT* dtin = reinterpret_cast<const AT*>(p.gate) + bh;
  const AT* ring_k = reinterpret_cast<const AT*>(p.rk) + bg * W * DK;
  const AT* ring_v = reinterpret_cast<const AT*>(p.rv) + bh * W * DV;
  const AT* ring_dt = reinterpret_cast<const AT*>(p.rg) + bh * W;

  // the step's own entry (kept for the append)
  const VecN<AT, SEG> kcur = ldraw<SEG>(kin + s * SEG);
  const VecN<AT, CPL> vcur = ldraw<CPL>(vin + s * CPL);
  const AT dtcur = dtin[0];

  if (n < W) {
    // ---------------------------------------------- issue the loads
    float qs[SEG];
    ldn<SEG>(q + s * SEG, qs);
    const float cqv = (tid < rows) ? reinterpret_cast<const float*>(p.work)[(size_t)b * p.R + roff0 + tid] : 0.f;
    // key of the first ring slot this head takes for the dot products
    VecN<AT, SEG> k0 = kcur;
    if (hh < n0) k0 = ldraw<SEG>(ring_k + (size_t)hh * DK + s * SEG);
    float dts[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      dts[u] = (i < n0) ? ld(ring_dt + i) : (i == n0 ? to_f32(dtcur) : 0.f);
    }
    // sketch rows and ring values of the earlier entries (HBM)
    VecN<UT, CPL> us[16];
    const UT* Ur = reinterpret_cast<const UT*>(p.U) + ((size_t)b * p.R + off) * DV + s * CPL;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < r) us[j] = ldraw<CPL>(Ur + (size_t)j * DV);
    VecN<AT, CPL> vs[WMAX];
    const AT* rv0 = ring_v + s * CPL;
#pragma unroll
    for (int i = 0; i < WMAX - 1; ++i)
      if (i < n0) vs[i] = ldraw<CPL>(rv0 + (size_t)i * DV);

    // d_i = k_i . q, slots spread over the group's heads (LPH lanes per slot)
    if (hh < n) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < SEG; ++e) d += vget(k0, e) * qs[e];
      d = xsum<0, LB>(d);
      if (s == 0) s_d[hh] = d;
    }
    for (int i = hh + HPG; i < n; i += HPG) {
      float ks[SEG];
      if (i < n0) {
        ldn<SEG>(ring_k + (size_t)i * DK + s * SEG, ks);
      } else {
#pragma unroll
        for (int e = 0; e < SEG; ++e) ks[e] = vget(kcur, e);
      }
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < SEG; ++e) d += ks[e] * qs[e];
      d = xsum<0, LB>(d);
      if (s == 0) s_d[i] = d;
    }
    if (tid < rows) s_c[tid] = cqv;

    // -------------------------------- decays: suffix products per head
    float a[SPL], lp = 1.f;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      a[u] = (i < n) ? m2_decay(dts[u], Ah) : 1.0f;
      lp *= a[u];
    }
    float incl = lp;                               // prod over lanes >= s
#pragma unroll
    for (int d = 1; d < LPH; d <<= 1) {
      const float o = __shfl_down(incl, d, LPH);
      if (s + d < LPH) incl *= o;
    }
    // shuffle with every lane active (a disabled source lane reads as zero)
    const float nxt = __shfl_down(incl, 1, LPH);
    const float after = (s + 1 < LPH) ? nxt : 1.0f;   // prod over lanes > s
    const float D = __shfl(incl, 0, LPH);
    float w[SPL];
    {
      float suf = after;
#pragma unroll
      for (int u = SPL - 1; u >= 0; --u) {
        w[u] = dts[u] * suf;                        // dt_i prod_{t>i} a_t
        suf *= a[u];
      }
    }
    if (__syncthreads_or(bad)) {                   // s_d and s_c complete
      if (s == 0 && bad) atomicOr(p.err, bad);
      return;
    }
    float e[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      e[u] = (i < n) ? w[u] * s_d[i] : 0.f;
    }

    // ------------------------------------------------------- output
    float acc[CPL], ob[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = ob[c] = 0.f;
    const float* cme = s_c + (off - roff0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < r) {
        const float cj = cme[j];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] += cj * vget(us[j], c);
      }
    }
#pragma unroll
    for (int i = 0; i < WMAX - 1; ++i) {
      const float ei = __shfl(e[i % SPL], i / SPL, LPH);
      if (i < n0)
#pragma unroll
        for (int c = 0; c < CPL; ++c) ob[c] += ei * vget(vs[i], c);
    }
    {
      float ecur = e[0];
#pragma unroll
      for (int u = 1; u < SPL; ++u)
        if (n0 % SPL == u) ecur = e[u];
      ecur = __shfl(ecur, n0 / SPL, LPH);
#pragma unroll
      for (int c = 0; c < CPL; ++c) ob[c] += ecur * vget(vcur, c);
    }
    float out[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = D * acc[c] + ob[c];
    stn<CPL>(reinterpret_cast<AT*>(p.o) + bh * DV + s * CPL, out);
  } else if (__syncthreads_or(bad)) {              // pairs with the barrier above
    if (s == 0 && bad) atomicOr(p.err, bad);
    return;
  }

  // ------------------------------------------------------------ append
  AT* rk = reinterpret_cast<AT*>(p.rk) + (bg * W + n0) * DK;
  AT* rv = reinterpret_cast<AT*>(p.rv) + (bh * W + n0) * DV;
  if (hh == 0) stv<SEG>(rk + s * SEG, kcur);
  stv<CPL>(rv + s * CPL, vcur);
  if (s == 0) {
    reinterpret_cast<AT*>(p.rg)[bh * W + n0] = dtcur;
    p.count[bh] = n;
  }
}

// ------------------------------------------------------------ GDN / KDA
// One wave per (sequence, head) tile.  The pull-back is a serial chain over
// the buffered entries, newest first:
//   d = k_i . r;  o_buf += beta_i d v_i;  r <- alpha_i (r - beta_i d k_i)   (GDN)
//                                        r <- g_i (.) (r - beta_i d k_i)    (KDA)
// then c = C_h r and o = U_h c + o_buf.  Each lane holds DK/64 elements of r
// and DV/64 output columns.
template <int FAM, int DK, int DV, typename AT, typename UT>
__global__ void __launch_bounds__(64) dn_read_kernel(Params p) {
  constexpr int EK = DK >= 64 ? DK / 64 : 1;
  constexpr int EV = DV >= 64 ? DV / 64 : 1;
  const int lane = threadIdx.x;
  const int W = p.W;
  const int tile = blockIdx.x;
  const int b = tile / p.H;
  const int h = tile - b * p.H;
  const size_t bh = (size_t)b * p.H + h;      // G == H for these families

  const int n0 = p.count[bh];
  if (n0 < 0 || n0 >= W) {
    if (lane == 0) atomicOr(p.err, ERRBIT_COUNT);
    return;
  }
  const int n = n0 + 1;
  const AT* kin = reinterpret_cast<const AT*>(p.k) + bh * DK;
  const AT* vin = reinterpret_cast<const AT*>(p.v) + bh * DV;
  const float* gin = reinterpret_cast<const float*>(p.gate) + (FAM == FAM_KDA ? bh * DK : bh);
  AT* ring_k = reinterpret_cast<AT*>(p.rk) + bh * W * DK;
  AT* ring_v = reinterpret_cast<AT*>(p.rv) + bh * W * DV;
  float* ring_g = reinterpret_cast<float*>(p.rg) + (FAM == FAM_KDA ? bh * W * DK : bh * W);
  float* ring_b = p.rb + bh * W;

  // append
  for (int e = lane; e < DK; e += 64) ring_k[(size_t)n0 * DK + e] = kin[e];
  for (int e = lane; e < DV; e += 64) ring_v[(size_t)n0 * DV + e] = vin[e];
  if (FAM == FAM_KDA) {
    for (int e = lane; e < DK; e += 64) ring_g[(size_t)n0 * DK + e] = gin[e];
  } else if (lane == 0) {
    ring_g[n0] = gin[0];
  }
  if (lane == 0) {
    ring_b[n0] = p.beta[bh];
    p.count[bh] = n;
  }
  if (n == W) return;

  float r[EK], ob[EV];
  const AT* q = reinterpret_cast<const AT*>(p.q) + bh * DK;
#pragma unroll
  for (int e = 0; e < EK; ++e) {
    const int m = lane * EK + e;
    r[e] = (m < DK) ? ld(q + m) : 0.f;
  }
#pragma unroll
  for (int e = 0; e < EV; ++e) ob[e] = 0.f;

  for (int t = 0; t < n; ++t) {
    const int i = n - 1 - t;
    const AT* k = (i == n0) ? kin : ring_k + (size_t)i * DK;
    const AT* v = (i == n0) ? vin : ring_v + (size_t)i * DV;
    const float beta = (i == n0) ? p.beta[bh] : ring_b[i];
    float kk[EK];
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      const int m = lane * EK + e;
      kk[e] = (m < DK) ? ld(k + m) : 0.f;
      d += kk[e] * r[e];
    }
    d = xsum<0, 6>(d);
    const float bd = beta * d;
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      const int c = lane * EV + e;
      if (c < DV) ob[e] += bd * ld(v + c);
    }
    if (FAM == FAM_GDN) {
      const float al = (i == n0) ? gin[0] : ring_g[i];
#pragma unroll
      for (int e = 0; e < EK; ++e) r[e] = al * (r[e] - bd * kk[e]);
    } else {
      const float* gv = (i == n0) ? gin : ring_g + (size_t)i * DK;
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const int m = lane * EK + e;
        const float gm = (m < DK) ? gv[m] : 0.f;
        r[e] = gm * (r[e] - bd * kk[e]);
      }
    }
  }

  // c = C_h r : 16 partial dot products, halved across lane bits 2..5, summed over bits 0..1
  const int off = p.off[h], rk = p.off[h + 1] - off;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float a = 0.f;
    if (j < rk) {
      const float* Cr = p.C + (size_t)(off + j) * DK;
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const int m = lane * EK + e;
        if (m < DK) a += Cr[m] * r[e];
      }
    }
    acc[j] = a;
  }
  tr_reduce<16, 2, 4>(acc, lane);
  const float cj_mine = xsum<0, 2>(acc[0]);      // c_j for j = lane >> 2

  const UT* Ur = reinterpret_cast<const UT*>(p.U) + ((size_t)b * p.R + off) * DV;
  float out[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) out[e] = ob[e];
  for (int j = 0; j < rk; ++j) {
    const float cj = __shfl(cj_mine, 4 * j);
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      const int c = lane * EV + e;
      if (c < DV) out[e] += cj * ld(Ur + (size_t)j * DV + c);
    }
  }
  AT* o = reinterpret_cast<AT*>(p.o) + bh * DV;
#pragma unroll
  for (int e = 0; e < EV; ++e) {
    const int c = lane * EV + e;
    if (c < DV) st(o + c, out[e]);
  }
}

}  // namespace sk
