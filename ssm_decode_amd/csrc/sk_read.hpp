// Non-flush sketched-read kernels.  They never touch the state S: each step
// reads the sketch U, the buffered ring entries and the coefficient map C
// (the fixed per-head table, or each tile's state-dependent map as its last
// flush wrote it), appends the step's entry to the ring and advances the
// ring count.
#pragma once

#include <type_traits>

#include "sk_device.hpp"
#include "sk_params.hpp"

namespace sk {

// ---------------------------------------------------------------- Mamba-2
// The read of a Mamba-2 layer is two launches.
//
// m2_prep_kernel forms what the heads of a B/C group share, into the
// workspace:
//   cq[b][off_h + j] = (C_h q_b)_j        the query in each head's basis
//   d[b][g][i]       = k_i . q_b          every buffered key and the step's own
//   n0[b][g]         = the group's ring fill, or a negative error code when
//                      the heads of the group disagree or the fill is out of
//                      range
// A fixed C is shared by all sequences, so one workgroup takes 4 sequences of
// one group and reads each of its rows of C once.
//
// m2_read_kernel then needs no keys, no queries and no exchange between
// heads: one wave per (sequence, group, block of four heads), with
//   q~ = D q, D = prod_i a_i;   o_buf = sum_i w_i d_i v_i, w_i = dt_i prod_{t>i} a_t
//   o  = D * U_h cq_h + o_buf
constexpr int M2R_MAXHPG = 16;     // heads per B/C group (at most)
// Sequences per dot-product workgroup: 8, or 4 for a 32-slot ring, so that
// the keys and queries in flight stay at two passes of registers (four
// passes at W = 32 held the whole prep kernel to three waves per SIMD).
template <int WMAX>
constexpr int cq_nb() { return WMAX > 16 ? 4 : 8; }
constexpr int CQ_THREADS = 256;
// The prep grid is (dot-product blocks, then coefficient blocks) x groups.
// A coefficient block takes ROWS coefficient rows of a group for NBC
// sequences.  The fixed map keeps a row's C chunks in registers across the
// NBC sequences (4 lanes a row); the state-dependent map has a row per
// sequence, read once (8 lanes a row at dk >= 64).  Larger blocks cut the L2
// traffic of a fixed C but lengthen each workgroup's serial loop over its
// sequences, which costs more.
template <int COEF, int DK, typename UT, int WMAX = 16>
struct PrepGrid {
  static constexpr int CQ_NB = cq_nb<WMAX>();
  static constexpr int CSIZE = COEF ? (int)sizeof(UT) : 4;  // bytes per C element
  static constexpr int NCH = DK * CSIZE / 16;               // 16-byte chunks per C row
  static constexpr int LPR0 = COEF && DK >= 64 ? 8 : 4;
  static constexpr int LPR = NCH < LPR0 ? NCH : LPR0;        // lanes per coefficient row
  static constexpr int ROWS = CQ_THREADS / LPR;              // rows per workgroup
  static constexpr int ZBLOCKS = (M2R_MAXHPG * 16 + ROWS - 1) / ROWS;
  static constexpr int NBC = 4;                              // sequences per coefficient block
  static __host__ __device__ int dot_blocks(int B) { return (B + CQ_NB - 1) / CQ_NB; }
  static __host__ __device__ int coef_seq_blocks(int B) { return (B + NBC - 1) / NBC; }
  static __host__ __device__ int blocks(int B) { return dot_blocks(B) + coef_seq_blocks(B) * ZBLOCKS; }
};
constexpr int DOT_LPP = 4;         // lanes per (sequence, slot) dot product

template <int DK, typename AT, int WMAX>
__device__ __forceinline__ void m2_prep_dots(const Params& p, int xb) {
  constexpr int CQ_NB = cq_nb<WMAX>();
  // a key or query row is split into NCK chunks of CEK elements (16 bytes, or
  // a quarter row when that is smaller); lane qt of a pair takes chunks
  // qt, qt + 4, .. so that one load instruction reads whole 64-byte pieces
  constexpr int CEK = (16 / (int)sizeof(AT)) < DK / DOT_LPP ? 16 / (int)sizeof(AT) : DK / DOT_LPP;
  constexpr int NCK = DK / CEK;
  constexpr int NKL = NCK / DOT_LPP;               // chunks per lane
  constexpr int PPP = CQ_THREADS / DOT_LPP;        // pairs per pass
  constexpr int PASSES = (CQ_NB * WMAX + PPP - 1) / PPP;
  static_assert(NKL >= 1 && NCK % DOT_LPP == 0 && CEK % 2 == 0, "key rows split into lane chunks");
  const int tid = threadIdx.x;
  const int qt = tid & (DOT_LPP - 1);
  const int g = blockIdx.y;
  const int b0 = xb * CQ_NB;
  const int nb = min(CQ_NB, p.B - b0);
  const int W = p.W, HPG = p.HPG;
  const M2Work wl(p.B, p.R, p.G, W);
  float* dws = reinterpret_cast<float*>(p.work) + wl.d;
  int* n0ws = reinterpret_cast<int*>(reinterpret_cast<float*>(p.work) + wl.n0);

  // the group's ring fill per sequence: row bb (16 lanes) reads the counts
  // of the group's heads; they must agree and lie in [0, W)
  __shared__ int s_n0[CQ_NB];
  {
    const int bb = tid >> 4, l = tid & 15;
    int c = 0;
    if (bb < nb && l < HPG) c = p.count[(size_t)(b0 + bb) * p.H + g * HPG + l];
    const int c0 = __shfl(c, 0, 16);
    int bad = (l < HPG && c != c0) ? ERRBIT_GROUP : 0;
    if (c0 < 0 || c0 >= W) bad |= ERRBIT_COUNT;
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) bad |= __shfl_xor(bad, m, 16);
    if (l == 0 && bb < CQ_NB) {
      s_n0[bb] = (bb < nb && !bad) ? c0 : 0;     // clamped into the ring
      if (bb < nb) n0ws[(size_t)(b0 + bb) * p.G + g] = bad ? -bad : c0;
    }
  }
  __syncthreads();
  const AT* kin = reinterpret_cast<const AT*>(p.k);
  const AT* rk = reinterpret_cast<const AT*>(p.rk);
  const AT* q = reinterpret_cast<const AT*>(p.q);
  // issue every key and query segment load, then the dot products
  VecN<AT, CEK> kv[PASSES][NKL], qv[PASSES][NKL];
  int pb[PASSES], pi[PASSES], pn0[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int pair = ps * PPP + (tid >> 2);
    const int bb = pair / WMAX, i = pair - bb * WMAX;
    const int n0 = s_n0[bb < CQ_NB ? bb : 0];
    pb[ps] = bb; pi[ps] = i; pn0[ps] = n0;
    const size_t bgi = (size_t)(b0 + (bb < nb ? bb : 0)) * p.G + g;
    const AT* kp = (i < n0) ? rk + (bgi * W + i) * DK : kin + bgi * DK;
#pragma unroll
    for (int k = 0; k < NKL; ++k) {
      kv[ps][k] = ldraw<CEK>(kp + CEK * (qt + DOT_LPP * k));
      qv[ps][k] = ldraw<CEK>(q + bgi * DK + CEK * (qt + DOT_LPP * k));
    }
  }
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < NKL; ++k)
#pragma unroll
      for (int e = 0; e < CEK; e += 2) {
        a0 += vget(kv[ps][k], e) * vget(qv[ps][k], e);
        a1 += vget(kv[ps][k], e + 1) * vget(qv[ps][k], e + 1);
      }
    float d = a0 + a1;
    d += dpp_f<0xB1>(d, 0.f);                      // quad sum: the pair's four lanes
    d += dpp_f<0x4E>(d, 0.f);
    const int bb = pb[ps], i = pi[ps];
    if (qt == 0 && bb < nb && i <= pn0[ps])
      dws[((size_t)(b0 + bb) * p.G + g) * W + i] = d;
  }
}

template <int DK, typename AT, typename UT, int WMAX, int COEF>
__global__ void __launch_bounds__(CQ_THREADS) m2_prep_kernel(Params p) {
  using PG = PrepGrid<COEF, DK, UT, WMAX>;
  constexpr int CQ_LPR = PG::LPR, CQ_ROWS = PG::ROWS, NBC = PG::NBC;
  const int ndot = PG::dot_blocks(p.B);
  if ((int)blockIdx.x < ndot) {                    // uniform: a dot-product block
    m2_prep_dots<DK, AT, WMAX>(p, blockIdx.x);
    return;
  }
  const int cb = blockIdx.x - ndot;
  const int nxs = PG::coef_seq_blocks(p.B);
  const int xs = cb % nxs, zb = cb / nxs;
  // a C row is NCH chunks of 16 bytes; lane qt of the row takes chunks qt,
  // qt + LPR, .. so that one load instruction reads whole 64- or 128-byte
  // pieces of the rows
  using CT = typename std::conditional<COEF != 0, UT, float>::type;
  constexpr int CE = 16 / (int)sizeof(CT);       // elements per chunk
  constexpr int NCL = PG::NCH / CQ_LPR;          // chunks per lane
  static_assert(NCL >= 1 && PG::NCH % CQ_LPR == 0, "C rows split into lane chunks");
  constexpr int QCH = NBC * DK / 4;              // 4-element query chunks per block
  constexpr int QIT = (QCH + CQ_THREADS - 1) / CQ_THREADS;
  __shared__ float s_q[NBC][DK];
  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int roff0 = p.off[g * p.HPG];
  const int rows = p.off[(g + 1) * p.HPG] - roff0;
  const int rb = zb * CQ_ROWS;
  if (rb >= rows) return;                        // uniform: no rows in this block
  const int b0 = xs * NBC;
  const int nb = min(NBC, p.B - b0);
  const int row = rb + tid / CQ_LPR;
  const int qt = tid & (CQ_LPR - 1);
  // C rows: the fixed map's row once for every sequence, or the row of each
  // sequence's own map
  constexpr int NCR = COEF ? NBC : 1;
  VecN<CT, CE> c[NCR][NCL];
#pragma unroll
  for (int bb = 0; bb < NCR; ++bb) {
    const int rr = row < rows ? row : 0;          // clamped: loads stay unconditional
    const CT* rp;
    if constexpr (COEF) {
      const int b = b0 + (bb < nb ? bb : 0);
      rp = reinterpret_cast<const UT*>(p.Cs) + ((size_t)b * p.R + roff0 + rr) * DK;
    } else {
      rp = p.C + (size_t)(roff0 + rr) * DK;
    }
#pragma unroll
    for (int k = 0; k < NCL; ++k)   // (a sequence's own map rows are read once: non-temporal)
      c[bb][k] = COEF ? ldraw_nt<CE>(rp + CE * (qt + CQ_LPR * k)) : ldraw<CE>(rp + CE * (qt + CQ_LPR * k));
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
  for (int bb = 0; bb < NBC; ++bb) {
    if (bb < nb) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int k = 0; k < NCL; ++k) {
        const auto& cr = c[COEF ? bb : 0][k];
        const float* qs = &s_q[bb][CE * (qt + CQ_LPR * k)];
#pragma unroll
        for (int e = 0; e < CE; e += 4) {
          const float4 qq = *reinterpret_cast<const float4*>(qs + e);
          a0 += vget(cr, e) * qq.x;
          a1 += vget(cr, e + 1) * qq.y;
          a2 += vget(cr, e + 2) * qq.z;
          a3 += vget(cr, e + 3) * qq.w;
        }
      }
      const float acc = low_lane_sum<CQ_LPR>((a0 + a1) + (a2 + a3));
      if (qt == 0 && row < rows) cq[(size_t)(b0 + bb) * p.R + roff0 + row] = acc;
    }
  }
}

template <int N, typename T>
__device__ __forceinline__ void stv(T* p, const VecN<T, N>& x) {
  *reinterpret_cast<VecN<T, N>*>(p) = x;
}

// Sketched read: one wave per (sequence, group, block of 4 / CS heads),
// M2R_WPB consecutive such waves a workgroup, CS rows of 16 lanes per head
// (DPP rows; each row takes dv / CS of the head's columns and repeats the
// head's per-slot work).  Lane s of a row holds ring slots s*SPL..
// for the decay scan, coefficient j = s, and CPL output columns.  The
// ring fill comes from the prep kernel's workspace; then every load is
// issued before the first wait: slot gates and dot products, the head's cq
// entry, then the head's r sketch rows and n0 ring values (the lean kernel
// has nothing to overlap with them, so loads past the rank or the fill are
// not issued).  The per-slot coefficients w_i d_i and the cq entries are
// exchanged within the head's row through LDS (a wave reads what its own
// lanes wrote).
constexpr int M2R_LPH = 16;        // lanes per row of a head
constexpr int M2R_HPW = 64 / M2R_LPH;   // rows per wave (heads per wave when CS = 1)
constexpr int M2R_WPB = 4;         // waves per workgroup (measured: 1, 2, 4, 8, 16 -> 4 best)

// 16-lane rows per head (each row takes dv / CS of the head's columns): one
// row holds at most 4 columns of every sketch row and 2 of every ring row
// when the ring has 32 slots, so that the loads a lane keeps in flight fit
// five waves per SIMD (measured at W = 32, dv = 64: 134 -> 87 VGPRs, read
// call 113.5 -> 110 us at batch 1024)
constexpr int m2_read_split(int DV, int WMAX) {
  const int cs = (DV > 64 ? DV / 64 : 1) * (WMAX > 16 ? 2 : 1);
  return cs < M2R_HPW ? cs : M2R_HPW;
}
__host__ __device__ inline int m2_read_items(int B, int G, int HPG, int CS = 1) {
  const int hpw = M2R_HPW / CS;
  return B * G * ((HPG + hpw - 1) / hpw);
}
inline int m2_read_blocks(int B, int G, int HPG, int CS = 1) {
  return (m2_read_items(B, G, HPG, CS) + M2R_WPB - 1) / M2R_WPB;
}

template <int DK, int DV, typename AT, typename UT, int WMAX, int CS = 1>
__global__ void __launch_bounds__(64 * M2R_WPB) m2_read_kernel(Params p) {
  constexpr int LPH = M2R_LPH;
  constexpr int HPW = M2R_HPW / CS;
  constexpr int SEG = DK / LPH;                  // key elements per lane (append)
  constexpr int CPL = DV / (LPH * CS);           // output columns per lane
  constexpr int SPL = WMAX / LPH;                // ring slots per lane in the decay scan
  static_assert(SEG >= 1 && CPL >= 1 && SPL >= 1, "head dims too small for the lane split");
  __shared__ __align__(16) float s_e_wg[M2R_WPB][M2R_HPW * WMAX];  // w_i d_i per 16-lane row
  __shared__ __align__(16) float s_c_wg[M2R_WPB][M2R_HPW * 16];    // cq entries per 16-lane row
  float* s_e = s_e_wg[threadIdx.x >> 6];           // this wave's part
  float* s_c = s_c_wg[threadIdx.x >> 6];
  // (indexed by the wave's 16-lane row: with CS > 1 the rows of a head hold
  // the same per-slot values)

  const int wpg = (p.HPG + HPW - 1) / HPW;
  // consecutive waves of a workgroup: the head blocks of one (sequence, group)
  const int item = blockIdx.x * M2R_WPB + (threadIdx.x >> 6);
  if (item >= m2_read_items(p.B, p.G, p.HPG, CS)) return;
  const int bgi = item / wpg;
  const int wq = item - bgi * wpg;
  const int tid = threadIdx.x & 63;
  const int rr = tid >> 4;                       // 16-lane row of the wave
  const int hh = rr / CS;                        // head of the wave
  const int cs = rr - hh * CS;                   // its column part
  const int s = tid & 15;
  const int col0 = cs * (DV / CS) + s * CPL;     // first of the lane's output columns
  const int W = p.W, HPG = p.HPG;
  const int b = bgi / p.G;
  const int g = bgi - b * p.G;
  const int hw = wq * HPW + hh;                  // head within the group
  const bool hv = hw < HPG;
  const int h = g * HPG + (hv ? hw : 0);
  const size_t bg = (size_t)bgi;
  const size_t bh = (size_t)b * p.H + h;
  const M2Work wl(p.B, p.R, p.G, W);

  // ------------------------------- ring fill (checked by the prep kernel)
  // and the rank offsets and decay rates of the wave's heads, as scalars;
  // each 16-lane row then takes its head's (heads past the group take the
  // wave's first head, with no rows)
  const int bgu = __builtin_amdgcn_readfirstlane(bgi);
  const int n0c = uload(reinterpret_cast<const int*>(reinterpret_cast<const float*>(p.work) + wl.n0), bgu);
  const int hb = __builtin_amdgcn_readfirstlane(g * HPG + wq * HPW);   // the wave's first head
  int ob[HPW + 1];
  float ab[HPW];
#pragma unroll
  for (int k = 0; k <= HPW; ++k) ob[k] = uload(p.off, min(hb + k, p.H));
#pragma unroll
  for (int k = 0; k < HPW; ++k) ab[k] = uload(p.A, min(hb + k, p.H - 1));
  // (all of them in flight at once and waited for together: the compiler
  // would otherwise sink the offsets into the branch on the ring fill, a
  // second round trip after the fill's)
  asm volatile("" ::"s"(n0c));
#pragma unroll
  for (int k = 0; k <= HPW; ++k) asm volatile("" ::"s"(ob[k]));
#pragma unroll
  for (int k = 0; k < HPW; ++k) asm volatile("" ::"s"(ab[k]));
  int off = ob[0], offn = ob[1];
  float Ah = ab[0];
#pragma unroll
  for (int k = 1; k < HPW; ++k) {
    const bool me = hv && hh == k;
    off = me ? ob[k] : off;
    offn = me ? ob[k + 1] : offn;
    Ah = me ? ab[k] : Ah;
  }
  const int r = hv ? offn - off : 0;
  const int n0 = n0c < 0 ? 0 : n0c;              // in range for every address below
  const int n = n0 + 1;
  __builtin_amdgcn_sched_barrier(0);

  const AT* kin = reinterpret_cast<const AT*>(p.k) + bg * DK;
  const AT* vin = reinterpret_cast<const AT*>(p.v) + bh * DV;
  const AT* dtin = reinterpret_cast<const AT*>(p.gate) + bh;
  const AT* ring_v = reinterpret_cast<const AT*>(p.rv) + bh * W * DV;
  const AT* ring_dt = reinterpret_cast<const AT*>(p.rg) + bh * W;
  const float* dws = reinterpret_cast<const float*>(p.work) + wl.d + bg * W;

  // the step's own entry (kept for the append)
  const VecN<AT, SEG> kcur = ldraw<SEG>(kin + s * SEG);
  const VecN<AT, CPL> vcur = ldraw<CPL>(vin + col0);
  const AT dtcur = dtin[0];

  if (n < W && n0c >= 0) {                       // uniform
    // ---------------------------------------------- issue the loads
    AT dtr[SPL];
    float dr[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      dtr[u] = ring_dt[i < n0 ? i : 0];
      dr[u] = dws[i <= n0 ? i : 0];
    }
    const float cqv = reinterpret_cast<const float*>(p.work)[(size_t)b * p.R + off + (s < r ? s : 0)];
    VecN<UT, CPL> us[16];
    const UT* Ur = reinterpret_cast<const UT*>(p.U) + ((size_t)b * p.R + off) * DV + col0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < r) us[j] = ldraw_nt<CPL>(Ur + (size_t)j * DV);
    VecN<AT, CPL> vs[WMAX];
    const AT* rv0 = ring_v + col0;
#pragma unroll
    for (int i = 0; i < WMAX - 1; ++i)
      if (i < n0) vs[i] = ldraw_nt<CPL>(rv0 + (size_t)i * DV);

    // -------------------------------- decays: suffix products per head
    float dts[SPL], a[SPL], lp = 1.f;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int i = s * SPL + u;
      dts[u] = (i < n0) ? to_f32(dtr[u]) : (i == n0 ? to_f32(dtcur) : 0.f);
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
    float* eh = s_e + rr * WMAX;
    float* ch = s_c + rr * 16;
    {
      float suf = after;
#pragma unroll
      for (int u = SPL - 1; u >= 0; --u) {
        const int i = s * SPL + u;
        eh[i] = (i < n) ? dts[u] * suf * dr[u] : 0.f;   // w_i d_i
        suf *= a[u];
      }
    }
    ch[s] = cqv;
    wave_lds_sync();                             // the row's lanes read eh and ch below

    // ------------------------------------------------------- output
    float acc[CPL], ob[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = ob[c] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < r) {
        const float cj = ch[j];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] += cj * vget(us[j], c);
      }
    }
#pragma unroll
    for (int i = 0; i < WMAX - 1; ++i) {
      if (i < n0) {
        const float ei = eh[i];
#pragma unroll
        for (int c = 0; c < CPL; ++c) ob[c] += ei * vget(vs[i], c);
      }
    }
    {
      const float ecur = eh[n0];
#pragma unroll
      for (int c = 0; c < CPL; ++c) ob[c] += ecur * vget(vcur, c);
    }
    float out[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = D * acc[c] + ob[c];
    // (a dense-fallback head's output comes from m2_dense_read_kernel)
    if (hv && r > 0) stn<CPL>(reinterpret_cast<AT*>(p.o) + bh * DV + col0, out);
  }
  if (n0c < 0) {                                 // the prep kernel found a bad group
    if (tid == 0 && wq == 0) atomicOr(p.err, -n0c);
    return;
  }

  // ------------------------------------------------------------ append
  AT* rk = reinterpret_cast<AT*>(p.rk) + (bg * W + n0) * DK;
  AT* rv = reinterpret_cast<AT*>(p.rv) + (bh * W + n0) * DV;
  if (wq == 0 && rr == 0) stv<SEG>(rk + s * SEG, kcur);
  if (hv) {
    stv<CPL>(rv + col0, vcur);
    if (s == 0 && cs == 0) {
      reinterpret_cast<AT*>(p.rg)[bh * W + n0] = dtcur;
      p.count[bh] = n;
    }
  }
}

// Dense-fallback heads (rank 0) of a Mamba-2 layer at a non-flush step:
// one wave per (sequence, dense head), launched after m2_read_kernel (which
// appends the step's entry and leaves these heads' outputs alone):
//   o = D * Scopy^T q + sum_i w_i d_i v_i,
// with the dot products d_i and the checked ring fill from the prep
// kernel's workspace.  The head's state copy is read in one pass, every
// 16-byte chunk in flight at once: lane l takes chunk l % LPRW of rows
// l / LPRW + RPP i, and of ring rows l / LPRW + RPP k (the ring rows of a
// chunk column spread over its lanes as the state rows are), and the lanes
// of a chunk column are summed at the end.
template <int DK, int DV, typename AT, typename UT, int WMAX>
__global__ void __launch_bounds__(64) m2_dense_read_kernel(Params p) {
  constexpr int CE = 16 / (int)sizeof(UT);           // elements per chunk
  constexpr int LPRW = DV / CE;                      // lanes per row
  constexpr int RPP = 64 / LPRW;                     // rows per pass
  constexpr int NP = DK / RPP;                       // passes
  static_assert(LPRW >= 1 && LPRW <= 64 && DK % RPP == 0, "state copy split into lane chunks");
  __shared__ float s_q[DK];
  const int lane = threadIdx.x;
  const int nd = p.ndense;
  const int b = blockIdx.x / nd;
  const int slot = blockIdx.x - b * nd;              // position in the dense list
  const int h = p.dense_list[slot];
  const int W = p.W;
  const int g = h / p.HPG;
  const size_t bg = (size_t)b * p.G + g, bh = (size_t)b * p.H + h;
  const M2Work wl(p.B, p.R, p.G, W);
  const int n0c = reinterpret_cast<const int*>(reinterpret_cast<const float*>(p.work) + wl.n0)[bg];
  if (n0c < 0 || n0c + 1 >= W) return;               // a bad group (reported), or the flush step
  const int n0 = n0c, n = n0 + 1;
  const int cc = lane % LPRW, r0 = lane / LPRW;
  __builtin_amdgcn_sched_barrier(0);

  // loads: the state copy, the query, the slot gates and dot products, the
  // ring values and the step's own value
  const UT* Sr = reinterpret_cast<const UT*>(p.Sc) + ((size_t)b * nd + slot) * DK * DV + cc * CE;
  VecN<UT, CE> sr[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) sr[i] = ldraw_nt<CE>(Sr + (size_t)(r0 + RPP * i) * DV);
  const AT* qg = reinterpret_cast<const AT*>(p.q) + bg * DK;
  for (int m = lane; m < DK; m += 64) s_q[m] = ld(qg + m);
  const AT* ring_dt = reinterpret_cast<const AT*>(p.rg) + bh * W;
  const float dt = lane < n0 ? ld(ring_dt + lane) : (lane == n0 ? ld(reinterpret_cast<const AT*>(p.gate) + bh) : 0.f);
  const float* dws = reinterpret_cast<const float*>(p.work) + wl.d + bg * W;
  const float dl = dws[lane <= n0 ? lane : 0];
  const AT* ring_v = reinterpret_cast<const AT*>(p.rv) + bh * W * DV + cc * CE;
  constexpr int RPL = (WMAX - 1 + RPP - 1) / RPP;   // ring rows per lane
  VecN<AT, CE> vs[RPL];
#pragma unroll
  for (int k = 0; k < RPL; ++k) {                  // (rows past the fill: row 0, weighted 0 below)
    const int i = r0 + RPP * k;
    vs[k] = ldraw_nt<CE>(ring_v + (size_t)(i < n0 ? i : 0) * DV);
  }
  const VecN<AT, CE> vcur = ldraw<CE>(reinterpret_cast<const AT*>(p.v) + bh * DV + cc * CE);

  // decays: a_i = exp(-dt_i e^A), w_i = dt_i prod_{t>i} a_t, D = prod_t a_t
  const float a = lane < n ? m2_decay(dt, p.A[h]) : 1.0f;
  float suf = a;                                     // inclusive suffix product
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_down(suf, d);
    if (lane + d < 64) suf *= o;
  }
  const float excl = __shfl_down(suf, 1);            // prod over t > lane
  const float e = lane < n ? dt * (lane + 1 < 64 ? excl : 1.0f) * dl : 0.f;   // w_i d_i
  const float D = lane_value(suf, 0);

  // Scopy^T q and the buffered term over this lane's rows, then over the
  // lanes of its chunk column
  __syncthreads();
  float acc[CE], ob[CE];
#pragma unroll
  for (int c = 0; c < CE; ++c) acc[c] = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const float qm = s_q[r0 + RPP * i];
#pragma unroll
    for (int c = 0; c < CE; ++c) acc[c] += qm * vget(sr[i], c);
  }
  const float en0 = lane_value(e, n0);               // (a readlane: in converged code)
  const float ecur = r0 == 0 ? en0 : 0.f;            // the step's own entry, once per column
#pragma unroll
  for (int c = 0; c < CE; ++c) ob[c] = ecur * vget(vcur, c);
#pragma unroll
  for (int k = 0; k < RPL; ++k) {
    const int i = r0 + RPP * k;
    const float ei = __shfl(e, i < 64 ? i : 0);
#pragma unroll
    for (int c = 0; c < CE; ++c) ob[c] += i < n0 ? ei * vget(vs[k], c) : 0.f;
  }
  float out[CE];
#pragma unroll
  for (int c = 0; c < CE; ++c) out[c] = D * acc[c] + ob[c];
#pragma unroll
  for (int m = LPRW; m < 64; m <<= 1)
#pragma unroll
    for (int c = 0; c < CE; ++c) out[c] += __shfl_xor(out[c], m);
  if (r0 == 0) stn<CE>(reinterpret_cast<AT*>(p.o) + bh * DV + cc * CE, out);
}

// ------------------------------------------------------------ GDN / KDA
// One wave per (sequence, head) tile, DN_TPW tiles of one head (consecutive
// sequences) per workgroup.  The fixed map's rows of C_h are loaded once per
// workgroup into LDS (instead of once per wave from L2); a state-dependent
// map is each tile's own and goes to registers.  Every load is issued once
// the ring fill is known, before any arithmetic: the step's own entry, the
// buffered entries (keys, values, gates, betas), the tile's own map rows and
// the sketch rows of U.  The pull-back is then a chain over the buffered
// entries held in registers, newest first:
//   d = k_i . r;  o_buf += beta_i d v_i;  r <- alpha_i (r - beta_i d k_i)   (GDN)
//                                        r <- g_i (.) (r - beta_i d k_i)    (KDA)
// then c = C_h r and o = U_h c + o_buf.  Lane l holds the key elements
// EK l .. EK l + EK - 1 of r and k_i and the output columns EV l .. ; the
// per-slot scalars of slot i sit in lane i and are read with readlane.  The
// append stores the step's entry from the registers that hold it.
constexpr int DN_TPW = 4;            // tiles (waves) per workgroup

__host__ __device__ inline int dn_read_blocks(int B, int H) { return (B + DN_TPW - 1) / DN_TPW * H; }

// PB: the effective query and buffered term of a read: 0 serial, 1 every
// slot's coefficient from the triangular system (WY form), 2 the same
// coefficients with C q~ formed from per-slot projected factors.
template <int FAM, int DK, int DV, typename AT, typename UT, int WMAX, int COEF, int PB>
__global__ void __launch_bounds__(64 * DN_TPW) dn_read_kernel(Params p) {
  constexpr int EK = DK >= 64 ? DK / 64 : 1;
  constexpr int EV = DV >= 64 ? DV / 64 : 1;
  constexpr int KG = FAM == FAM_KDA ? EK : 1;    // gate elements per lane and slot
  constexpr int NT = 64 * DN_TPW;
  constexpr int CCH = 16 * DK / 4;               // 16-byte chunks of 16 rows of C
  constexpr int CPT = (CCH + NT - 1) / NT;
  __shared__ __align__(16) float s_c[COEF ? 1 : 16 * DK];
  // the triangular system of the parallel pull-back, per wave: L [WMAX][WMAX], then d [WMAX]
  constexpr int WYS = WMAX * WMAX + WMAX;
  constexpr bool WY = PB != 0;
  __shared__ __align__(16) float s_wy[WY ? DN_TPW * WYS : 1];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int W = p.W;
  const int h = blockIdx.x % p.H;
  const int b = blockIdx.x / p.H * DN_TPW + wv;
  const bool active = b < p.B;                   // the last block may hold fewer tiles
  const int bcl = active ? b : p.B - 1;          // clamped, for addresses
  const size_t bh = (size_t)bcl * p.H + h;      // G == H for these families
  const bool kl = lane * EK < DK;             // lane holds key elements
  const bool vl = lane * EV < DV;             // lane holds output columns
  // lanes without elements (small heads) load a valid element and drop it,
  // so no load sits behind a per-lane branch
  const int lk = kl ? lane * EK : 0;
  const int lv = vl ? lane * EV : 0;

  // the ring fill and the rank offsets first: every address below depends
  // on them, and the memory counter retires loads in order
  const int n0raw = uload(p.count, __builtin_amdgcn_readfirstlane((int)bh));   // (scalar loads)
  const int off = uload(p.off, h), rk = uload(p.off, h + 1) - off;
  // the fixed map's rows of this head, staged through LDS once per workgroup
  // (two named registers, not an array: a private array would be placed in
  // LDS by the compiler, which then waits for the loads before issuing the
  // others)
  static_assert(CPT <= 2, "at most two 16-byte chunks of C per thread");
  auto c_chunk = [&](int u) -> float4 {
    const int idx = threadIdx.x + NT * u;
    const int row = idx / (DK / 4), ch = idx - row * (DK / 4);
    const int rr = row < rk ? row : 0;           // clamped: the load stays unconditional
    return *reinterpret_cast<const float4*>(p.C + (size_t)(off + rr) * DK + 4 * ch);
  };
  float4 cst0 = make_float4(0.f, 0.f, 0.f, 0.f), cst1 = cst0;
  if constexpr (!COEF) {
    if (rk > 0) {                                // a dense-fallback head has no rows
      cst0 = c_chunk(0);
      if constexpr (CPT > 1) cst1 = c_chunk(1);
    }
  }
  // (the loads above are issued before anything waits for the ring fill)
  __builtin_amdgcn_sched_barrier(0);
  const bool ok = n0raw >= 0 && n0raw < W;
  const int n0 = ok ? n0raw : 0;
  const int n = n0 + 1;
  const bool rd = active && ok && n < W;         // this tile writes an output
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

  // ------------------------------------------------ issue the loads
  const int nr = rd ? n0 : 0;                    // buffered entries this tile reads
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
    if (i < nr) {                                // uniform
      ks[i] = ldraw_nt<EK>(ring_k + (size_t)i * DK);
      vs[i] = ldraw_nt<EV>(ring_v + (size_t)i * DV);
      if (FAM == FAM_KDA) ldn<KG>(ring_g + (size_t)i * DK, gs[i]);
    }
  }
  // projected factors (PB = 2): lane j of every row of 16 holds factor
  // element j of each buffered slot
  float pcs[PB == 2 ? WMAX - 1 : 1];
  if constexpr (PB == 2) {
    const float* pc = p.rpc + bh * W * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < WMAX - 1; ++i)
      if (i < nr && rk > 0) pcs[i] = pc[(size_t)i * 16];
  }
  // GDN / KDA per-slot scalars: slot i in lane i
  const int ls = lane < nr ? lane : 0;
  const float al_l = FAM == FAM_GDN ? ring_g[ls] : 1.f;
  const float be_l = ring_b[ls];
  float cr[COEF ? 16 : 1][EK];
  if constexpr (COEF) {
    const UT* Csb = reinterpret_cast<const UT*>(p.Cs) + ((size_t)bcl * p.R + off) * DK + lk;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < rk && rd) ldn<EK>(Csb + (size_t)j * DK, cr[j]);   // (non-temporal measured slower here)
  }
  VecN<UT, EV> us[16];
  const UT* Ur = reinterpret_cast<const UT*>(p.U) + ((size_t)bcl * p.R + off) * DV + lv;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < rk && rd) us[j] = ldraw_nt<EV>(Ur + (size_t)j * DV);

  if constexpr (!COEF) {
    // (every load is in flight before the wait for the staged rows)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int idx = threadIdx.x + NT * u;
      const int row = idx / (DK / 4), ch = idx - row * (DK / 4);
      if (idx < CCH && row < rk) *reinterpret_cast<float4*>(s_c + row * DK + 4 * ch) = u ? cst1 : cst0;
    }
    __syncthreads();
  }
  if (active && rk == 0 && lane == 0) {          // whether the dense launch writes o
    const DnWork wl(p.B, p.ndense, DK, DV);
    reinterpret_cast<int*>(reinterpret_cast<float*>(p.work) + wl.flag)[(size_t)bcl * p.ndense + dense_slot(p, h)] =
        rd ? 1 : 0;
  }
  if (!active) return;
  if (!ok) {
    if (lane == 0) atomicOr(p.err, ERRBIT_COUNT);
    return;
  }

  float pcur = 0.f;                              // PB = 2: lane j's element of the step's factor
  if (rd) {
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
    if constexpr (!WY) {
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
    } else {
      // ------------------- parallel pull-back (triangular system)
      // Slots 0..n0, oldest first: ring slot i < n0, the step's own entry at
      // n0.  With D(j,l) the product of the decays of slots j+1..l, the
      // serial form's coefficients d_j = k_j . r_j solve
      //   d_j + sum_{l>j} beta_l <k_j, D(j,l) k_l> d_l = <k_j, D(j,n0) q>;
      // every pair product is formed first (independent wave sums), the
      // system is solved by back substitution, then
      //   q~ = D(-1,n0) q - sum_l beta_l d_l D(-1,l) k_l,  o_buf = sum_l beta_l d_l v_l.
      float* Lw = s_wy + wv * WYS;
      float* dw = Lw + WMAX * WMAX;
      auto key = [&](int i) -> VecN<AT, EK> { return i < n0 ? ks[i < WMAX - 1 ? i : 0] : kcur; };
      auto beta_of = [&](int i) { return i < n0 ? lane_value(be_l, i < WMAX - 1 ? i : 0) : bcur; };
      auto decay = [&](int i, float (&D)[EK]) {   // D <- D (.) (slot i's decay)
        if constexpr (FAM == FAM_GDN) {
          const float a = i < n0 ? lane_value(al_l, i < WMAX - 1 ? i : 0) : gcur[0];
#pragma unroll
          for (int e = 0; e < EK; ++e) D[e] *= a;
        } else {
#pragma unroll
          for (int e = 0; e < EK; ++e) D[e] *= i < n0 ? gs[i < WMAX - 1 ? i : 0][e] : gcur[e];
        }
      };
#pragma unroll
      for (int j = 0; j < WMAX; ++j) {
        if (j <= n0) {                             // uniform
          const VecN<AT, EK> kj = key(j);
          float D[EK];
#pragma unroll
          for (int e = 0; e < EK; ++e) D[e] = 1.f;
#pragma unroll
          for (int l = j + 1; l < WMAX; ++l) {
            if (l <= n0) {
              decay(l, D);                         // D = D(j, l)
              const VecN<AT, EK> kv = key(l);
              float part = 0.f;
#pragma unroll
              for (int e = 0; e < EK; ++e) part += vget(kj, e) * D[e] * vget(kv, e);
              const float Ljl = beta_of(l) * wave_sum(kl ? part : 0.f);   // (lanes without key elements hold copies)
              if (lane == 0) Lw[j * WMAX + l] = Ljl;
            }
          }
          float part = 0.f;                        // D = D(j, n0); r is q here (0 where !kl)
#pragma unroll
          for (int e = 0; e < EK; ++e) part += vget(kj, e) * D[e] * r[e];
          const float bj = wave_sum(part);
          if (lane == 0) dw[j] = bj;
        }
      }
      wave_lds_sync();                           // lane 0's table entries, read by every lane
      // back substitution: lane l holds d_l once it is known and reads row j
      // of the table at column l, so each d_j is one wave sum (the table
      // reads do not wait for the solution; a wave's LDS accesses complete
      // in order, so lane 0's writes above are visible)
      float dlane = 0.f;
#pragma unroll
      for (int j = WMAX - 1; j >= 0; --j) {
        if (j <= n0) {                             // uniform
          const int lc = lane < WMAX ? lane : 0;
          const float Ljl = (lane > j && lane <= n0) ? Lw[j * WMAX + lc] : 0.f;
          const float dj = dw[j] - wave_sum(Ljl * dlane);
          dlane = lane == j ? dj : dlane;
        }
      }
      // (with projected factors a sketched head needs only D(-1, n0) here:
      // the erase terms enter its coefficients through the factors)
      const bool qt_terms = PB != 2 || rk == 0;   // uniform
      float D[EK], acc[EK];
#pragma unroll
      for (int e = 0; e < EK; ++e) { D[e] = 1.f; acc[e] = 0.f; }
#pragma unroll
      for (int l = 0; l < WMAX; ++l) {
        if (l <= n0) {
          decay(l, D);                             // D = D(-1, l)
          const float bd = beta_of(l) * lane_value(dlane, l);
          const VecN<AT, EV> vv = l < n0 ? vs[l < WMAX - 1 ? l : 0] : vcur;
          if (qt_terms) {
            const VecN<AT, EK> kv = key(l);
#pragma unroll
            for (int e = 0; e < EK; ++e) acc[e] -= bd * D[e] * vget(kv, e);
          }
#pragma unroll
          for (int e = 0; e < EV; ++e) ob[e] += bd * vget(vv, e);
        }
      }
      if constexpr (PB == 2) {
        if (!qt_terms) {
          // C q~ = C (D(-1,n0) q) - sum_l beta_l d_l P_l (paper App. C.2),
          // with P_l = C (D(-1,l) k_l) stored when slot l was appended; the
          // step's own factor P_n0 = C (D(-1,n0) k_n0) is formed here and
          // appended.  pc_acc (lane j): sum over the buffered slots of
          // beta_l d_l P_l[j].
          float pc_acc = 0.f;
#pragma unroll
          for (int l = 0; l < WMAX - 1; ++l)
            if (l < n0) pc_acc += lane_value(be_l, l) * lane_value(dlane, l) * pcs[l];
          const float wcur = bcur * lane_value(dlane, n0);
          float cq[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            if (j < rk) {                              // uniform
              float cj[EK];
              if constexpr (COEF) {
#pragma unroll
                for (int e = 0; e < EK; ++e) cj[e] = cr[j][e];
              } else {
                ldn<EK>(s_c + j * DK + lk, cj);
              }
              float aq = 0.f, ak = 0.f;
#pragma unroll
              for (int e = 0; e < EK; ++e) {
                aq += cj[e] * D[e] * r[e];
                ak += cj[e] * D[e] * vget(kcur, e);
              }
              const float pj = wave_sum(kl ? ak : 0.f);       // P_n0[j]
              pcur = lane == j ? pj : pcur;
              cq[j] = wave_sum(kl ? aq : 0.f) - lane_value(pc_acc, j) - wcur * pj;
            }
          }
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (j < rk) {
              const float c = cq[j];
#pragma unroll
              for (int e = 0; e < EV; ++e) ob[e] += c * vget(us[j], e);
            }
        }
      }
#pragma unroll
      for (int e = 0; e < EK; ++e) r[e] = kl ? D[e] * r[e] + acc[e] : 0.f;
    }

    // -------------------------- c = C_h r, then o = U_h c + o_buf
    // (each c_j is a wave sum, wave-uniform, so U_h c needs no broadcast;
    // with projected factors U_h c is already in ob)
    float out[EV];
#pragma unroll
    for (int e = 0; e < EV; ++e) out[e] = ob[e];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < rk && PB != 2) {                     // uniform
        float cj[EK];
        if constexpr (COEF) {
#pragma unroll
          for (int e = 0; e < EK; ++e) cj[e] = cr[j][e];
        } else {
          ldn<EK>(s_c + j * DK + lk, cj);
        }
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) a += cj[e] * r[e];
        const float c = wave_sum(a);
#pragma unroll
        for (int e = 0; e < EV; ++e) out[e] += c * vget(us[j], e);
      }
    }
    if (rk == 0) {
      // dense-fallback head: the pulled-back query and the buffered term go
      // to the workspace, and dn_dense_read_kernel adds Scopy^T r and
      // writes o
      const DnWork wl(p.B, p.ndense, DK, DV);
      const size_t t = (size_t)bcl * p.ndense + dense_slot(p, h);
      float* ws = reinterpret_cast<float*>(p.work);
      if (kl) stn<EK>(ws + wl.r + t * DK + lk, r);
      if (vl) stn<EV>(ws + wl.ob + t * DV + lv, out);
    } else if (vl) {
      stn<EV>(reinterpret_cast<AT*>(p.o) + bh * DV + lv, out);
    }
  }

  // ------------------------------------------------------------ append
  if (kl) stv<EK>(ring_k + (size_t)n0 * DK, kcur);
  if (vl) stv<EV>(ring_v + (size_t)n0 * DV, vcur);
  if (FAM == FAM_KDA) {
    if (kl) stn<KG>(ring_g + (size_t)n0 * DK, gcur);
  } else if (lane == 0) {
    ring_g[n0] = gcur[0];
  }
  if (PB == 2 && rd && lane < rk) p.rpc[(bh * W + n0) * 16 + lane] = pcur;
  if (lane == 0) {
    ring_b[n0] = bcur;
    p.count[bh] = n;
  }
}

// Dense-fallback heads of a GDN/KDA layer at a non-flush step: one
// workgroup per (sequence, dense head), launched after dn_read_kernel, which
// leaves the tile's pulled-back query r and buffered term in the workspace
// with a flag set when the step has an output:  o = Scopy^T r + o_buf.
// Every 16-byte chunk of the state copy is in flight at once: thread t takes
// chunk t % LPRW of rows t / LPRW + RPP i, and the partial sums of a chunk
// column are added through LDS.
constexpr int DND_THREADS = 256;

template <int DK, int DV, typename AT, typename UT>
__global__ void __launch_bounds__(DND_THREADS) dn_dense_read_kernel(Params p) {
  constexpr int CE = 16 / (int)sizeof(UT);           // elements per chunk
  constexpr int LPRW = DV / CE;                      // threads per row
  constexpr int RPP0 = DND_THREADS / LPRW;
  constexpr int RPP = RPP0 < DK ? RPP0 : DK;         // rows per pass
  constexpr int NP = DK / RPP;                       // passes
  static_assert(LPRW >= 1 && LPRW <= DND_THREADS && DK % RPP == 0, "state copy split into chunks");
  __shared__ float s_r[DK];
  __shared__ float s_part[RPP][DV];
  const int tid = threadIdx.x;
  const int nd = p.ndense;
  const int b = blockIdx.x / nd;
  const int slot = blockIdx.x - b * nd;              // position in the dense list
  const int h = p.dense_list[slot];
  const size_t t = (size_t)b * nd + slot;
  const DnWork wl(p.B, nd, DK, DV);
  const float* ws = reinterpret_cast<const float*>(p.work);
  if (reinterpret_cast<const int*>(ws + wl.flag)[t] == 0) return;   // no output this step (uniform)
  const bool on = tid < RPP * LPRW;
  const int cc = tid % LPRW, r0 = on ? tid / LPRW : 0;
  const UT* Sr = reinterpret_cast<const UT*>(p.Sc) + t * DK * DV + cc * CE;
  VecN<UT, CE> sr[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) sr[i] = ldraw_nt<CE>(Sr + (size_t)(r0 + RPP * i) * DV);
  if (tid < DK) s_r[tid] = ws[wl.r + t * DK + tid];
  __syncthreads();
  float acc[CE];
#pragma unroll
  for (int c = 0; c < CE; ++c) acc[c] = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const float rm = s_r[r0 + RPP * i];
#pragma unroll
    for (int c = 0; c < CE; ++c) acc[c] += rm * vget(sr[i], c);
  }
  if (on)
#pragma unroll
    for (int c = 0; c < CE; ++c) s_part[r0][cc * CE + c] = acc[c];
  __syncthreads();
  if (tid < DV) {
    float o = ws[wl.ob + t * DV + tid];
#pragma unroll
    for (int g = 0; g < RPP; ++g) o += s_part[g][tid];
    st(reinterpret_cast<AT*>(p.o) + ((size_t)b * p.H + h) * DV + tid, o);
  }
}

}  // namespace sk
