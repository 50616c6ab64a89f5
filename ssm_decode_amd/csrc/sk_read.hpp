// Non-flush sketched-read kernels.  They never touch the state S: each step
// reads the sketch U, the buffered ring entries and the fixed coefficient
// map C, appends the step's entry to the ring and advances the ring count.
#pragma once

#include "sk_device.hpp"
#include "sk_params.hpp"

namespace sk {

// ---------------------------------------------------------------- Mamba-2
// One workgroup per (sequence, B/C group).  The group's heads share k and q,
// so the dot products d_i = k_i . q and the coefficient rows of the whole
// group are formed once per workgroup.  For head h with n entries (the
// step's own entry last):
//   q~ = D q, D = prod_i a_i;   o_buf = sum_i w_i d_i v_i, w_i = dt_i prod_{t>i} a_t
//   o  = D * U_h (C_h q) + o_buf
constexpr int M2R_THREADS = 256;
constexpr int M2R_MAXHPG = 16;     // heads per group handled by one workgroup
constexpr int M2R_MAXW = 32;

template <int DK, int DV, typename AT, typename UT>
__global__ void __launch_bounds__(M2R_THREADS) m2_read_kernel(Params p) {
  constexpr int NT = M2R_THREADS;
  __shared__ float s_q[DK];
  __shared__ float s_d[M2R_MAXW];                       // d_i = k_i . q
  __shared__ float s_a[M2R_MAXHPG][M2R_MAXW];           // a_i per head
  __shared__ float s_w[M2R_MAXHPG][M2R_MAXW];           // w_i d_i per head
  __shared__ float s_D[M2R_MAXHPG];
  __shared__ float s_c[M2R_MAXHPG * 16];                // C_h q for the group's rows
  __shared__ int s_n0, s_bad;

  const int tid = threadIdx.x;
  const int W = p.W, HPG = p.HPG;
  const int b = blockIdx.x / p.G;
  const int g = blockIdx.x - b * p.G;
  const int h0 = g * HPG;
  const size_t bh0 = (size_t)b * p.H + h0;

  if (tid == 0) {
    const int n0 = p.count[bh0];
    int bad = (n0 < 0 || n0 >= W) ? ERRBIT_COUNT : 0;
    for (int hh = 1; hh < HPG; ++hh)
      if (p.count[bh0 + hh] != n0) bad |= ERRBIT_GROUP;
    s_n0 = n0;
    s_bad = bad;
    if (bad) atomicOr(p.err, bad);
  }
  __syncthreads();
  if (s_bad) return;
  const int n0 = s_n0;
  const int n = n0 + 1;

  const AT* q = reinterpret_cast<const AT*>(p.q) + ((size_t)b * p.G + g) * DK;
  const AT* kin = reinterpret_cast<const AT*>(p.k) + ((size_t)b * p.G + g) * DK;
  const AT* vin = reinterpret_cast<const AT*>(p.v) + bh0 * DV;
  const AT* dtin = reinterpret_cast<const AT*>(p.gate) + bh0;
  const AT* ring_k = reinterpret_cast<const AT*>(p.rk) + ((size_t)b * p.G + g) * W * DK;
  const AT* ring_v = reinterpret_cast<const AT*>(p.rv) + bh0 * W * DV;   // head hh at + hh*W*DV
  const AT* ring_dt = reinterpret_cast<const AT*>(p.rg) + bh0 * W;       // head hh at + hh*W

  // ------------------------------------------------------------ append
  {
    AT* rk = reinterpret_cast<AT*>(p.rk) + (((size_t)b * p.G + g) * W + n0) * DK;
    for (int e = tid; e < DK; e += NT) rk[e] = kin[e];
    AT* rv = reinterpret_cast<AT*>(p.rv);
    for (int e = tid; e < HPG * DV; e += NT) {
      const int hh = e / DV, c = e - hh * DV;
      rv[((bh0 + hh) * W + n0) * DV + c] = vin[e];
    }
    AT* rdt = reinterpret_cast<AT*>(p.rg);
    for (int hh = tid; hh < HPG; hh += NT) {
      rdt[(bh0 + hh) * W + n0] = dtin[hh];
      p.count[bh0 + hh] = (n == W) ? W : n;
    }
  }
  if (n == W) return;        // the flush writes this step's output

  // ---------------------------------------------- query and dot products
  for (int m = tid; m < DK; m += NT) s_q[m] = ld(q + m);
  __syncthreads();
  {
    // slot i handled by 16 lanes, each a DK/16 segment
    constexpr int SEG = DK / 16;
    for (int base = 0; base < n; base += NT / 16) {
      const int i = base + tid / 16;
      const int sg = tid & 15;
      float d = 0.f;
      if (i < n) {
        const AT* k = (i == n0) ? kin : ring_k + (size_t)i * DK;
#pragma unroll
        for (int e = 0; e < SEG; ++e) d += ld(k + sg * SEG + e) * s_q[sg * SEG + e];
      }
      d = xsum<0, 4>(d);
      if (i < n && sg == 0) s_d[i] = d;
    }
  }
  // ------------------------------------------------------ decays a_i
  for (int idx = tid; idx < HPG * n; idx += NT) {
    const int hh = idx / n, i = idx - hh * n;
    const float dt = (i == n0) ? ld(dtin + hh) : ld(ring_dt + (size_t)hh * W + i);
    s_a[hh][i] = m2_decay(dt, p.A[h0 + hh]);
  }
  // ----------------------------------------- coefficient rows c = C_h q
  const int roff0 = p.off[h0];
  const int rows = p.off[h0 + HPG] - roff0;
  {
    constexpr int SEG = DK / 4;
    for (int base = 0; base < rows; base += NT / 4) {
      const int row = base + tid / 4;
      const int sg = tid & 3;
      float c = 0.f;
      if (row < rows) {
        const float* Cr = p.C + (size_t)(roff0 + row) * DK + sg * SEG;
#pragma unroll
        for (int e = 0; e < SEG; e += 4) {
          const float4 cv = *reinterpret_cast<const float4*>(Cr + e);
          c += cv.x * s_q[sg * SEG + e] + cv.y * s_q[sg * SEG + e + 1] +
               cv.z * s_q[sg * SEG + e + 2] + cv.w * s_q[sg * SEG + e + 3];
        }
      }
      c = xsum<0, 2>(c);
      if (row < rows && sg == 0) s_c[row] = c;
    }
  }
  __syncthreads();
  // ------------------------- weights w_i d_i = dt_i prod_{t>i} a_t d_i, D
  for (int idx = tid; idx < HPG * n; idx += NT) {
    const int hh = idx / n, i = idx - hh * n;
    float suf = 1.f;
    for (int t = i + 1; t < n; ++t) suf *= s_a[hh][t];
    const float dt = (i == n0) ? ld(dtin + hh) : ld(ring_dt + (size_t)hh * W + i);
    s_w[hh][i] = dt * suf * s_d[i];
    if (i == 0) s_D[hh] = s_a[hh][0] * suf;
  }
  __syncthreads();

  // ------------------------------------------------------------ output
  constexpr int CG = DV / 4;
  for (int idx = tid; idx < HPG * CG; idx += NT) {
    const int hh = idx / CG, c4 = (idx - hh * CG) * 4;
    const int h = h0 + hh;
    const int off = p.off[h], r = p.off[h + 1] - off;
    const UT* Ur = reinterpret_cast<const UT*>(p.U) + ((size_t)b * p.R + off) * DV + c4;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < r; ++j) {
      float u[4];
      ld4(Ur + (size_t)j * DV, u);
      const float cj = s_c[off - roff0 + j];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += cj * u[c];
    }
    const float D = s_D[hh];
    float ob[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n; ++i) {
      float v[4];
      ld4((i == n0) ? vin + (size_t)hh * DV + c4 : ring_v + ((size_t)hh * W + i) * DV + c4, v);
      const float wd = s_w[hh][i];
#pragma unroll
      for (int c = 0; c < 4; ++c) ob[c] += wd * v[c];
    }
    float out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = D * acc[c] + ob[c];
    st4(reinterpret_cast<AT*>(p.o) + (bh0 + hh) * DV + c4, out);
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
