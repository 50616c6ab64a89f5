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
  static_assert(LPH == 16, "a head is one 16-lane DPP row (and one cq row per thread)");
  __shared__ float s_d[WMAX];                    // d_i = k_i . q
  __shared__ float s_c[M2R_MAXHPG * 16];         // cq rows of the group
  __shared__ __align__(16) float s_e[M2R_MAXHPG * WMAX];  // w_i d_i per head

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
  const int n0 = (n0g < 0 || n0g >= W) ? 0 : n0g; // in range for every address below
  const int n = n0 + 1;
  // keep the count and offset loads ahead of every other load: the addresses
  // below depend on them and the memory counter retires loads in order
  __builtin_amdgcn_sched_barrier(0);

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
    // (loads are unconditional, from clamped indices, and their values are
    // selected where used: a load behind a branch with a default value
    // makes the wave wait for it inside the branch)
    float qs[SEG];
    ldn<SEG>(q + s * SEG, qs);
    const float cqv = reinterpret_cast<const float*>(p.work)[(size_t)b * p.R + roff0 + min(tid, rows - 1)];
    // key of the first ring slot this head takes for the dot products
    const VecN<AT, SEG> k0r = ldraw<SEG>(ring_k + (size_t)(hh < n0 ? hh : 0) * DK + s * SEG);
    AT dtr[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      dtr[u] = ring_dt[i < n0 ? i : 0];
    }
    // sketch rows and ring values of the earlier entries (HBM).  Every row
    // slot is loaded, rows past the head's rank or the ring fill from the
    // last valid row (an L1 hit, no extra HBM traffic), so the number of
    // loads in flight is fixed and the waits below retire only the loads
    // they need.
    VecN<UT, CPL> us[16];
    const UT* Ur = reinterpret_cast<const UT*>(p.U) + ((size_t)b * p.R + off) * DV + s * CPL;
#pragma unroll
    for (int j = 0; j < 16; ++j) us[j] = ldraw<CPL>(Ur + (size_t)min(j, r - 1) * DV);
    VecN<AT, CPL> vs[WMAX];
    const AT* rv0 = ring_v + s * CPL;
    const int ilast = n0 > 0 ? n0 - 1 : 0;
#pragma unroll
    for (int i = 0; i < WMAX - 1; ++i) vs[i] = ldraw<CPL>(rv0 + (size_t)min(i, ilast) * DV);

    float dts[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      dts[u] = (i < n0) ? to_f32(dtr[u]) : (i == n0 ? to_f32(dtcur) : 0.f);
    }
    // d_i = k_i . q, slots spread over the group's heads (LPH lanes per slot)
    if (hh < n) {
      const VecN<AT, SEG> k0 = hh < n0 ? k0r : kcur;
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < SEG; ++e) d += vget(k0, e) * qs[e];
      d = row16_sum(d);
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
      d = row16_sum(d);
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
    // suffix products along the head's DPP row (row_shl:n reads lane s+n;
    // lanes past the row end read 1)
    float incl = lp;                               // prod over lanes >= s
    incl *= dpp_f<0x101>(incl, 1.f);
    incl *= dpp_f<0x102>(incl, 1.f);
    incl *= dpp_f<0x104>(incl, 1.f);
    incl *= dpp_f<0x108>(incl, 1.f);
    const float after = dpp_f<0x101>(incl, 1.f); // prod over lanes > s
    const float D = row16_prod(lp);
    float w[SPL];
    {
      float suf = after;
#pragma unroll
      for (int u = SPL - 1; u >= 0; --u) {
        w[u] = dts[u] * suf;                        // dt_i prod_{t>i} a_t
        suf *= a[u];
      }
    }
    if (mine != n0g) bad |= ERRBIT_GROUP;
    if (__syncthreads_or(bad)) {                   // s_d and s_c complete
      if (s == 0 && bad) atomicOr(p.err, bad);
      return;
    }
    // e_i = w_i d_i, exchanged within the head's row through LDS (a wave
    // reads back what its own lanes wrote: LDS keeps a wave's order)
    float* eh = s_e + hh * WMAX;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      eh[i] = (i < n) ? w[u] * s_d[i] : 0.f;
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
      const float ei = eh[i];
      if (i < n0)
#pragma unroll
        for (int c = 0; c < CPL; ++c) ob[c] += ei * vget(vs[i], c);
    }
    {
      const float ecur = eh[n0];
#pragma unroll
      for (int c = 0; c < CPL; ++c) ob[c] += ecur * vget(vcur, c);
    }
    float out[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = D * acc[c] + ob[c];
    stn<CPL>(reinterpret_cast<AT*>(p.o) + bh * DV + s * CPL, out);
  } else {
    if (mine != n0g) bad |= ERRBIT_GROUP;
    if (__syncthreads_or(bad)) {                   // pairs with the barrier above
      if (s == 0 && bad) atomicOr(p.err, bad);
      return;
    }
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
// One wave per (sequence, head) tile.  Every load is issued once the ring
// fill is known, before any arithmetic: the step's own entry, the buffered
// entries (keys, values, gates, betas), the coefficient rows of C (L2
// resident) and the sketch rows of U.  The pull-back is then a chain over
// the buffered entries held in registers, newest first:
//   d = k_i . r;  o_buf += beta_i d v_i;  r <- alpha_i (r - beta_i d k_i)   (GDN)
//                                        r <- g_i (.) (r - beta_i d k_i)    (KDA)
// then c = C_h r and o = U_h c + o_buf.  Lane l holds the key elements
// EK l .. EK l + EK - 1 of r and k_i and the output columns EV l .. ; the
// per-slot scalars of slot i sit in lane i and are read with readlane.  The
// append stores the step's entry from the registers that hold it.
template <int FAM, int DK, int DV, typename AT, typename UT, int WMAX>
__global__ void __launch_bounds__(64) dn_read_kernel(Params p) {
  constexpr int EK = DK >= 64 ? DK / 64 : 1;
  constexpr int EV = DV >= 64 ? DV / 64 : 1;
  constexpr int KG = FAM == FAM_KDA ? EK : 1;    // gate elements per lane and slot
  const int lane = threadIdx.x;
  const int W = p.W;
  const int tile = blockIdx.x;
  const int b = tile / p.H;
  const int h = tile - b * p.H;
  const size_t bh = (size_t)b * p.H + h;      // G == H for these families
  const bool kl = lane * EK < DK;             // lane holds key elements
  const bool vl = lane * EV < DV;             // lane holds output columns
  // lanes without elements (small heads) load a valid element and drop it,
  // so no load sits behind a per-lane branch
  const int lk = kl ? lane * EK : 0;
  const int lv = vl ? lane * EV : 0;

  // the ring fill and the rank offsets first: every address below depends
  // on them, and the memory counter retires loads in order
  const int n0 = p.count[bh];
  const int off = p.off[h], rk = p.off[h + 1] - off;
  if (n0 < 0 || n0 >= W) {
    if (lane == 0) atomicOr(p.err, ERRBIT_COUNT);
    return;
  }
  const int n = n0 + 1;
  __builtin_amdgcn_sched_barrier(0);
  const AT* kin = reinterpret_cast<const AT*>(p.k) + bh * DK + lk;
  const AT* vin = reinterpret_cast<const AT*>(p.v) + bh * DV + lv;
  const float* gin = reinterpret_cast<const float*>(p.gate) + (FAM == FAM_KDA ? bh * DK + lk : bh);
  AT* ring_k = reinterpret_cast<AT*>(p.rk) + bh * W * DK + lk;
  AT* ring_v = reinterpret_cast<AT*>(p.rv) + bh * W * DV + lv;
  float* ring_g = reinterpret_cast<float*>(p.rg) + (FAM == FAM_KDA ? bh * W * DK + lk : bh * W);
  float* ring_b = p.rb + bh * W;

  // ------------------------------------------ the step's own entry
  const VecN<AT, EK> kcur = ldraw<EK>(kin);
  const VecN<AT, EV> vcur = ldraw<EV>(vin);
  float gcur[KG];
  if (FAM == FAM_KDA) ldn<KG>(gin, gcur);
  else gcur[0] = gin[0];
  const float bcur = p.beta[bh];

  if (n < W) {
    // ------------------------------------------------ issue the loads
    float r[EK];
    ldn<EK>(reinterpret_cast<const AT*>(p.q) + bh * DK + lk, r);
    if (!kl)
#pragma unroll
      for (int e = 0; e < EK; ++e) r[e] = 0.f;
    VecN<AT, EK> ks[WMAX - 1];
    VecN<AT, EV> vs[WMAX - 1];
    float gs[WMAX - 1][KG];
#pragma unroll
    for (int i = 0; i < WMAX - 1; ++i) {
      if (i < n0) {                                // uniform
        ks[i] = ldraw<EK>(ring_k + (size_t)i * DK);
        vs[i] = ldraw<EV>(ring_v + (size_t)i * DV);
        if (FAM == FAM_KDA) ldn<KG>(ring_g + (size_t)i * DK, gs[i]);
      }
    }
    // GDN / KDA per-slot scalars: slot i in lane i
    const int ls = lane < n0 ? lane : 0;
    const float al_l = FAM == FAM_GDN ? ring_g[ls] : 1.f;
    const float be_l = ring_b[ls];
    float cr[16][EK];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < rk) ldn<EK>(p.C + (size_t)(off + j) * DK + lk, cr[j]);
    VecN<UT, EV> us[16];
    const UT* Ur = reinterpret_cast<const UT*>(p.U) + ((size_t)b * p.R + off) * DV + lv;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < rk) us[j] = ldraw<EV>(Ur + (size_t)j * DV);

    // ---------------------------------------- pull-back, newest first
    float ob[EV];
#pragma unroll
    for (int e = 0; e < EV; ++e) ob[e] = 0.f;
    auto entry = [&](const VecN<AT, EK>& kv, const VecN<AT, EV>& vv, const float* gv, float be) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) d += vget(kv, e) * r[e];   // r is 0 where !kl
      d = wave_sum(d);
      const float bd = be * d;
#pragma unroll
      for (int e = 0; e < EV; ++e) ob[e] += bd * vget(vv, e);
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const float dec = FAM == FAM_GDN ? gv[0] : gv[e];
        r[e] = kl ? dec * (r[e] - bd * vget(kv, e)) : 0.f;
      }
    };
    entry(kcur, vcur, gcur, bcur);
#pragma unroll
    for (int i = WMAX - 2; i >= 0; --i) {
      if (i < n0) {
        float gsc[KG];
        if (FAM == FAM_GDN) gsc[0] = lane_value(al_l, i);
        else
#pragma unroll
          for (int e = 0; e < KG; ++e) gsc[e] = gs[i][e];
        entry(ks[i], vs[i], gsc, lane_value(be_l, i));
      }
    }

    // -------------------------- c = C_h r, then o = U_h c + o_buf
    // (each c_j is a wave sum, wave-uniform, so U_h c needs no broadcast)
    float out[EV];
#pragma unroll
    for (int e = 0; e < EV; ++e) out[e] = ob[e];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < rk) {                                // uniform
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) a += cr[j][e] * r[e];
        const float cj = wave_sum(a);
#pragma unroll
        for (int e = 0; e < EV; ++e) out[e] += cj * vget(us[j], e);
      }
    }
    if (vl) stn<EV>(reinterpret_cast<AT*>(p.o) + bh * DV + lv, out);
  }

  // ------------------------------------------------------------ append
  if (kl) stv<EK>(ring_k + (size_t)n0 * DK, kcur);
  if (vl) stv<EV>(ring_v + (size_t)n0 * DV, vcur);
  if (FAM == FAM_KDA) {
    if (kl) stn<KG>(ring_g + (size_t)n0 * DK, gcur);
  } else if (lane == 0) {
    ring_g[n0] = gcur[0];
  }
  if (lane == 0) {
    ring_b[n0] = bcur;
    p.count[bh] = n;
  }
}

}  // namespace sk
