// Non-flush sketched-read kernels.  They never touch the state S: each step
// reads the sketch U, the buffered ring entries and the fixed coefficient
// map C, appends the step's entry to the ring and advances the ring count.
#pragma once

#include "sk_device.hpp"
#include "sk_params.hpp"

namespace sk {

// ---------------------------------------------------------------- Mamba-2
// One workgroup per (sequence, B/C group), LPH lanes per head of the group.
// The group's heads share k and q, so the dot products d_i = k_i . q are
// formed once per workgroup.  For head h with n entries (the step's own
// entry last):
//   q~ = D q, D = prod_i a_i;   o_buf = sum_i w_i d_i v_i, w_i = dt_i prod_{t>i} a_t
//   o  = D * U_h (C_h q) + o_buf
// Lane s of a head holds: the q/k segment s (DK/LPH elements) for the dot
// products, coefficient row j = s / (LPH/16) after the reduction, ring
// slots s*SPL.. for the decay scan, and output columns s*CPL.. .  Every
// global load is issued right after the ring count is known; sketch rows and
// ring values stay packed (bf16) in registers until used.
constexpr int M2R_MAXHPG = 16;     // heads per group handled by one workgroup
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

template <int DK, int DV, typename AT, typename UT, int WMAX>
__global__ void __launch_bounds__((M2ReadLanes<DK, DV>::LPH * M2R_MAXHPG)) m2_read_kernel(Params p) {
  constexpr int LPH = M2ReadLanes<DK, DV>::LPH;
  constexpr int LB = ilog2c(LPH);
  constexpr int SEG = DK / LPH;                  // key / query elements per lane
  constexpr int CPL = DV / LPH;                  // output columns per lane
  constexpr int SPL = WMAX >= LPH ? WMAX / LPH : 1;  // ring slots per lane in the decay scan
  static_assert(SEG >= 1 && CPL >= 1, "head dims too small for the lane split");
  __shared__ float s_d[WMAX];                    // d_i = k_i . q
  __shared__ float s_c[M2R_MAXHPG * 16];         // C_h q for the group's coefficient rows

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
  const int n0 = p.count[(size_t)b * p.H + h0];
  const int mine = p.count[bh];
  int bad = (n0 < 0 || n0 >= W) ? ERRBIT_COUNT : 0;
  if (mine != n0) bad |= ERRBIT_GROUP;
  const int off = p.off[h];
  const int r = p.off[h + 1] - off;
  const float Ah = p.A[h];
  if (__syncthreads_or(bad)) {
    if (s == 0 && bad) atomicOr(p.err, bad);
    return;
  }
  const int n = n0 + 1;

  const AT* q = reinterpret_cast<const AT*>(p.q) + bg * DK;
  const AT* kin = reinterpret_cast<const AT*>(p.k) + bg * DK;
  const AT* vin = reinterpret_cast<const AT*>(p.v) + bh * DV;
  const AT* dtin = reinterpret_cast<const AT*>(p.gate) + bh;
  const AT* ring_k = reinterpret_cast<const AT*>(p.rk) + bg * W * DK;
  const AT* ring_v = reinterpret_cast<const AT*>(p.rv) + bh * W * DV;
  const AT* ring_dt = reinterpret_cast<const AT*>(p.rg) + bh * W;

  if (n < W) {
    // ---------------------------------------------- issue the loads
    // sketch rows and ring values (HBM) first; they stay packed until used
    VecN<UT, CPL> us[16];
    const UT* Ur = reinterpret_cast<const UT*>(p.U) + ((size_t)b * p.R + off) * DV + s * CPL;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < r) us[j] = ldraw<CPL>(Ur + (size_t)j * DV);
    // ring values of the earlier entries (constant row stride), then the step's own
    VecN<AT, CPL> vs[WMAX];
    const AT* rv0 = ring_v + s * CPL;
#pragma unroll
    for (int i = 0; i < WMAX - 1; ++i)
      if (i < n0) vs[i] = ldraw<CPL>(rv0 + (size_t)i * DV);
    const VecN<AT, CPL> vcur = ldraw<CPL>(vin + s * CPL);
    float dts[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      dts[u] = (i < n) ? ld((i == n0) ? dtin : ring_dt + i) : 0.f;
    }
    // d_i = k_i . q, slots spread over the group's heads (LPH lanes per slot)
    {
      float qs[SEG];
      ldn<SEG>(q + s * SEG, qs);
      for (int i = hh; i < n; i += HPG) {
        float ks[SEG];
        ldn<SEG>(((i == n0) ? kin : ring_k + (size_t)i * DK) + s * SEG, ks);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < SEG; ++e) d += ks[e] * qs[e];
        d = xsum<0, LB>(d);
        if (s == 0) s_d[i] = d;
      }
    }
    // coefficient rows of the whole group, C q, RT lanes per row (L2 resident)
    {
      constexpr int RT = 8;                       // lanes per coefficient row
      constexpr int RSEG = DK / RT;               // elements per lane
      const int roff0 = p.off[h0];
      const int rows = p.off[h0 + HPG] - roff0;
      const int nthreads = LPH * HPG;
      const int sg = tid & (RT - 1);
      const VecN<AT, RSEG> qr = ldraw<RSEG>(q + sg * RSEG);
      for (int base = 0; base < rows; base += nthreads / RT) {
        const int row = base + tid / RT;
        float c = 0.f;
        if (row < rows) {
          float cr[RSEG];
          ldn<RSEG>(p.C + (size_t)(roff0 + row) * DK + sg * RSEG, cr);
#pragma unroll
          for (int e = 0; e < RSEG; ++e) c += cr[e] * vget(qr, e);
        }
        c = xsum<0, 3>(c);
        if (row < rows && sg == 0) s_c[row] = c;
      }
    }
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
    __syncthreads();                               // s_d and s_c complete
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
    const float* cme = s_c + (off - p.off[h0]);
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
  } else {
    __syncthreads();                               // pairs with the barrier above
  }

  // ------------------------------------------------------------ append
  AT* rk = reinterpret_cast<AT*>(p.rk) + (bg * W + n0) * DK;
  AT* rv = reinterpret_cast<AT*>(p.rv) + (bh * W + n0) * DV;
  if (hh == 0) copyn<SEG>(rk + s * SEG, kin + s * SEG);
  copyn<CPL>(rv + s * CPL, vin + s * CPL);
  if (s == 0) {
    reinterpret_cast<AT*>(p.rg)[bh * W + n0] = dtin[0];
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
