// Tile kernels: one workgroup per (sequence, head) tile that reads the full
// state.  Used by the flush, the standard full-state step and the ReplaySSM
// step.  The state tile S (dk x dv fp32) is held in registers for the whole
// kernel: it is loaded once with 128-bit loads, updated, reduced against the
// query / basis vectors and stored once.
//
// Register layout.  The dv columns are split into column blocks of CB = 64
// (or dv when smaller), one wave per block.  Lane l owns the four columns
// 4*cg..4*cg+3 of its block (cg = l % NCG) and the rows m = rg + NRG*j,
// j = 0..RPL-1 (rg = l / NCG).  Reductions over rows (S^T x for the query,
// the basis vectors, the delta-rule key) are in-lane sums over j followed by
// an exchange across the NRG lanes that share cg.
//
// Latency structure.  Every global load the tile needs besides the state
// (ring keys, values and gates, the basis rows, the query) is issued first,
// as 16-byte chunks spread over the workgroup, then the state's 128-bit
// loads; the small loads are consumed (staged into LDS as fp32) while the
// state is still in flight.
#pragma once

#include "sk_device.hpp"
#include "sk_params.hpp"

namespace sk {

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr int round4(int x) { return (x + 3) & ~3; }
constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

template <int DK, int DV>
struct TileShape {
  static constexpr int CB = DV >= 64 ? 64 : DV;   // columns per wave
  static constexpr int NCB = DV / CB;             // waves per tile
  static constexpr int NCG = CB / 4;              // column groups per wave
  static constexpr int NRG = 64 / NCG;            // row groups per wave
  static constexpr int RPL = DK / NRG;            // rows per lane
  static constexpr int LB = ilog2(NCG);           // lane bits of cg
  static constexpr int NB = ilog2(NRG);           // lane bits of rg
  static constexpr int XS = RPL + 4;              // padded per-row-group stride of a permuted vector
  static constexpr int XLEN = NRG * XS;           // floats of one row-permuted dk-vector
  static constexpr int PS = 20;                   // padded row stride of the staged basis (16 + 4)
  static constexpr int THREADS = 64 * NCB;
  static_assert(RPL >= 1 && DK % NRG == 0, "unsupported dk/dv");
  static_assert(DV % CB == 0, "unsupported dv");
  static_assert(NRG >= 4 && NRG <= 16, "row groups must number 4..16");

  // position of row m in a row-permuted vector (lane rg reads XS-strided runs)
  static __host__ __device__ constexpr int perm(int m) { return (m % NRG) * XS + m / NRG; }
};

// LDS layout of a tile kernel (offsets in floats).
template <int FAM, int DK, int DV, int WMAX>
struct TileLds {
  using T = TileShape<DK, DV>;
  static constexpr int KWS = WMAX + 4;                         // Mamba-2 key row stride ([m][slot])
  static constexpr int Q = 0;                                  // query, permuted
  static constexpr int QT = Q + T::XLEN;                       // effective query, permuted
  static constexpr int SA = QT + T::XLEN;                      // per-slot scalars
  static constexpr int SW = SA + WMAX;
  static constexpr int SE = SW + WMAX;
  static constexpr int SX = SE + WMAX;
  static constexpr int MISC = SX + WMAX;
  static constexpr int V = MISC + 4;                           // values [slot][dv]
  static constexpr int BIG = V + WMAX * DV;                    // keys (and KDA gates), later the basis
  static constexpr int KEYS = FAM == FAM_M2 ? DK * KWS : WMAX * T::XLEN * (FAM == FAM_KDA ? 2 : 1);
  static constexpr int BASIS = DK * T::PS;
  static constexpr int TOTAL = BIG + (KEYS > BASIS ? KEYS : BASIS);
  static constexpr int BYTES = TOTAL * 4;
  static_assert(BIG % 4 == 0 && V % 4 == 0, "LDS regions must be 16-byte aligned");
};

template <typename AT>
struct Chunk {                      // one 16-byte load of an activation-dtype row
  static constexpr int N = 16 / sizeof(AT);
};

__device__ __forceinline__ void unpack(const uint4& r, float (&x)[8], const bf16*) {
  x[0] = __uint_as_float(r.x << 16); x[1] = __uint_as_float(r.x & 0xffff0000u);
  x[2] = __uint_as_float(r.y << 16); x[3] = __uint_as_float(r.y & 0xffff0000u);
  x[4] = __uint_as_float(r.z << 16); x[5] = __uint_as_float(r.z & 0xffff0000u);
  x[6] = __uint_as_float(r.w << 16); x[7] = __uint_as_float(r.w & 0xffff0000u);
}
__device__ __forceinline__ void unpack(const uint4& r, float (&x)[8], const float*) {
  x[0] = __uint_as_float(r.x); x[1] = __uint_as_float(r.y);
  x[2] = __uint_as_float(r.z); x[3] = __uint_as_float(r.w);
}

template <int FAM, int DK, int DV, typename AT, typename UT, int MODE, int WMAX>
__global__ void __launch_bounds__((TileShape<DK, DV>::THREADS), 2)
tile_kernel(Params p) {
  using T = TileShape<DK, DV>;
  using LY = TileLds<FAM, DK, DV, WMAX>;
  constexpr int CB = T::CB, NCG = T::NCG, NRG = T::NRG, RPL = T::RPL;
  constexpr int LB = T::LB, NB = T::NB, XS = T::XS, XLEN = T::XLEN, PS = T::PS;
  constexpr int NT = T::THREADS;
  constexpr int KWS = LY::KWS;

  extern __shared__ __align__(16) float smem[];
  float* s_q = smem + LY::Q;
  float* s_qt = smem + LY::QT;
  float* s_a = smem + LY::SA;      // M2 a_i / GDN alpha_i
  float* s_w = smem + LY::SW;      // M2 w_i / GDN, KDA beta_i
  float* s_e = smem + LY::SE;      // ReplaySSM buffered-output coefficients
  float* s_misc = smem + LY::MISC; // [0] = M2 total decay D
  float* s_v = smem + LY::V;       // values (M2: scaled by w_i)
  float* s_k = smem + LY::BIG;     // keys: M2 [m][slot]; GDN/KDA [slot][perm m] (+ KDA gates)
  float* s_p = smem + LY::BIG;     // basis [m][j], after the update

  const int W = p.W;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int cg = lane % NCG;
  const int rg = lane / NCG;
  const int tile = blockIdx.x;
  const int b = tile / p.H;
  const int h = tile - b * p.H;
  const int g = h / p.HPG;
  const size_t bh = (size_t)b * p.H + h;

  // ------------------------------------------------------------ window
  int n0 = 0;                       // entries already in the ring
  if (MODE != MODE_FULL) n0 = p.count[bh];
  if (MODE == MODE_FLUSH) {
    if (n0 < 0 || n0 > W) {
      if (tid == 0) atomicOr(p.err, ERRBIT_COUNT);
      return;
    }
    if (!p.flush_all && n0 != W) return;
  } else if (MODE == MODE_REPLAY) {
    if (n0 < 0 || n0 >= W) {
      if (tid == 0) atomicOr(p.err, ERRBIT_COUNT);
      return;
    }
  }
  const bool has_in = MODE != MODE_FLUSH;       // the step's own entry comes last
  const int n = n0 + (has_in ? 1 : 0);          // entries to consider
  const bool do_flush = MODE == MODE_FULL || MODE == MODE_FLUSH || n == W;
  const bool want_out = (MODE != MODE_FLUSH) || p.q != nullptr;
  const bool want_u = MODE == MODE_FLUSH;

  const AT* ring_k = reinterpret_cast<const AT*>(p.rk) + ((size_t)b * p.G + g) * W * DK;
  const AT* ring_v = reinterpret_cast<const AT*>(p.rv) + bh * W * DV;
  const AT* in_k = reinterpret_cast<const AT*>(p.k) + ((size_t)b * p.G + g) * DK;
  const AT* in_v = reinterpret_cast<const AT*>(p.v) + bh * DV;
  auto key_ptr = [&](int i) -> const AT* { return (has_in && i == n0) ? in_k : ring_k + (size_t)i * DK; };
  auto val_ptr = [&](int i) -> const AT* { return (has_in && i == n0) ? in_v : ring_v + (size_t)i * DV; };
  auto gate_vec = [&](int i) -> const float* {   // KDA g_i
    if (has_in && i == n0) return reinterpret_cast<const float*>(p.gate) + bh * DK;
    return reinterpret_cast<const float*>(p.rg) + (bh * W + i) * DK;
  };

  // ------------------------------------------ issue the small loads
  // per-slot scalars: lane i < n of wave 0
  float sc_gate = 0.f, sc_beta = 0.f;
  if (wv == 0 && lane < n) {
    const int i = lane;
    if (FAM == FAM_M2) {
      sc_gate = (has_in && i == n0) ? ld(reinterpret_cast<const AT*>(p.gate) + bh)
                                    : ld(reinterpret_cast<const AT*>(p.rg) + bh * W + i);
    } else {
      if (FAM == FAM_GDN)
        sc_gate = (has_in && i == n0) ? reinterpret_cast<const float*>(p.gate)[bh]
                                      : reinterpret_cast<const float*>(p.rg)[bh * W + i];
      sc_beta = (has_in && i == n0) ? p.beta[bh] : p.rb[bh * W + i];
    }
  }
  // keys: n rows of DK
  constexpr int KC = Chunk<AT>::N;
  constexpr int KCPR = DK / KC;
  constexpr int KU = cdiv(WMAX * KCPR, NT);
  uint4 kr[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int c = tid + NT * u;
    if (c < n * KCPR) {
      const int i = c / KCPR, m0 = (c - i * KCPR) * KC;
      kr[u] = *reinterpret_cast<const uint4*>(key_ptr(i) + m0);
    }
  }
  // values: n rows of DV
  constexpr int VCPR = DV / KC;
  constexpr int VU = cdiv(WMAX * VCPR, NT);
  uint4 vr[VU];
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int c = tid + NT * u;
    if (c < n * VCPR) {
      const int i = c / VCPR, c0 = (c - i * VCPR) * KC;
      vr[u] = *reinterpret_cast<const uint4*>(val_ptr(i) + c0);
    }
  }
  // KDA gates: n rows of DK fp32
  constexpr int GCPR = DK / 4;
  constexpr int GU = FAM == FAM_KDA ? cdiv(WMAX * GCPR, NT) : 1;
  float4 gr[GU];
  if (FAM == FAM_KDA) {
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int c = tid + NT * u;
      if (c < n * GCPR) {
        const int i = c / GCPR, m0 = (c - i * GCPR) * 4;
        gr[u] = *reinterpret_cast<const float4*>(gate_vec(i) + m0);
      }
    }
  }
  // basis rows (flush): r rows of DK fp32, loaded after the update
  int off = 0, r = 0;
  constexpr int PCPR = DK / 4;
  constexpr int PU = cdiv(16 * PCPR, NT);
  if (want_u) {
    off = p.off[h];
    r = p.off[h + 1] - off;
  }
  // query
  const AT* qg = reinterpret_cast<const AT*>(p.q) + ((size_t)b * p.G + g) * DK;
  float qv[cdiv(DK, NT)];
  if (want_out) {
#pragma unroll
    for (int u = 0; u < cdiv(DK, NT); ++u) {
      const int m = tid + NT * u;
      if (m < DK) qv[u] = ld(qg + m);
    }
  }

  // ------------------------------------------------ issue the state loads
  const float* Sg = p.S + bh * DK * DV + wv * CB + 4 * cg;
  float s[RPL][4];
#pragma unroll
  for (int j = 0; j < RPL; ++j) ld4(Sg + (size_t)(rg + NRG * j) * DV, s[j]);

  // ------------------------------------------------ append (ReplaySSM)
  if (MODE == MODE_REPLAY) {
    // per-head parts; the per-group key is appended by the group's first head
    AT* rv = reinterpret_cast<AT*>(p.rv) + (bh * W + n0) * DV;
    for (int e = tid; e < DV; e += NT) rv[e] = in_v[e];
    if (h % p.HPG == 0) {
      AT* rk = reinterpret_cast<AT*>(p.rk) + (((size_t)b * p.G + g) * W + n0) * DK;
      for (int e = tid; e < DK; e += NT) rk[e] = in_k[e];
    }
    if (FAM == FAM_KDA) {
      float* rgv = reinterpret_cast<float*>(p.rg) + (bh * W + n0) * DK;
      for (int e = tid; e < DK; e += NT) rgv[e] = reinterpret_cast<const float*>(p.gate)[bh * DK + e];
    } else if (tid == 0) {
      if (FAM == FAM_M2)
        reinterpret_cast<AT*>(p.rg)[bh * W + n0] = reinterpret_cast<const AT*>(p.gate)[bh];
      else
        reinterpret_cast<float*>(p.rg)[bh * W + n0] = reinterpret_cast<const float*>(p.gate)[bh];
    }
    if (FAM != FAM_M2 && tid == 0) p.rb[bh * W + n0] = p.beta[bh];
  }

  // ------------------------------------- per-slot quantities (wave 0)
  if (wv == 0) {
    if (FAM == FAM_M2) {
      // a_i = exp(-dt_i e^A); w_i = dt_i prod_{t>i} a_t; D = prod_t a_t
      const float a = lane < n ? m2_decay(sc_gate, p.A[h]) : 1.0f;
      float suf = a;                                   // inclusive suffix product
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_down(suf, d);
        if (lane + d < 64) suf *= o;
      }
      const float excl = __shfl_down(suf, 1);          // prod_{t>i}
      const float wi = sc_gate * (lane + 1 < 64 ? excl : 1.0f);
      if (lane < WMAX) {
        s_a[lane] = a;
        s_w[lane] = lane < n ? wi : 0.0f;
      }
      if (lane == 0) s_misc[0] = suf;                 // D (1 when n == 0)
    } else if (lane < WMAX) {
      s_a[lane] = lane < n ? sc_gate : 1.0f;
      s_w[lane] = lane < n ? sc_beta : 0.0f;
    }
  }
  if (want_out) {
#pragma unroll
    for (int u = 0; u < cdiv(DK, NT); ++u) {
      const int m = tid + NT * u;
      if (m < DK) s_q[T::perm(m)] = qv[u];
    }
  }
  // keys into LDS as fp32
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int c = tid + NT * u;
    if (c < n * KCPR) {
      const int i = c / KCPR, m0 = (c - i * KCPR) * KC;
      float x[8];
      unpack(kr[u], x, (const AT*)nullptr);
#pragma unroll
      for (int e = 0; e < KC; ++e) {
        if (FAM == FAM_M2) s_k[(m0 + e) * KWS + i] = x[e];
        else s_k[i * XLEN + T::perm(m0 + e)] = x[e];
      }
    }
  }
  if (FAM == FAM_M2) {      // zero the slots up to the next multiple of four
    const int n4 = round4(n);
    for (int idx = tid; idx < (n4 - n) * DK; idx += NT) {
      const int i = n + idx / DK, m = idx % DK;
      s_k[m * KWS + i] = 0.0f;
    }
  }
  if (FAM == FAM_KDA) {
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int c = tid + NT * u;
      if (c < n * GCPR) {
        const int i = c / GCPR, m0 = (c - i * GCPR) * 4;
        const float x[4] = {gr[u].x, gr[u].y, gr[u].z, gr[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) s_k[(WMAX + i) * XLEN + T::perm(m0 + e)] = x[e];
      }
    }
  }
  __syncthreads();
  // values into LDS as fp32 (Mamba-2: scaled by w_i), zero-padded
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int c = tid + NT * u;
    if (c < n * VCPR) {
      const int i = c / VCPR, c0 = (c - i * VCPR) * KC;
      float x[8];
      unpack(vr[u], x, (const AT*)nullptr);
      const float sc = FAM == FAM_M2 ? s_w[i] : 1.0f;
#pragma unroll
      for (int e = 0; e < KC; ++e) s_v[i * DV + c0 + e] = sc * x[e];
    }
  }
  if (FAM == FAM_M2) {
    const int n4 = round4(n);
    for (int idx = tid; idx < (n4 - n) * DV; idx += NT) s_v[n * DV + idx] = 0.0f;
  }
  __syncthreads();

  float out_val = 0.0f;      // reduced output value owned by this lane
  int out_c = 0;             // its column within the lane's group of four
  bool out_writer = false;
  const int colbase = wv * CB + 4 * cg;

  if (do_flush) {
    // -------------------------------------------- apply the entries
    if (FAM == FAM_M2) {
      // S <- D S + sum_i k_i (w_i v_i)^T  (the Mamba-2 steps in closed form)
      const float D = s_misc[0];
#pragma unroll
      for (int j = 0; j < RPL; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) s[j][c] *= D;
      for (int sg = 0; sg < n; sg += 4) {
        float4 v4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v4[u] = *reinterpret_cast<const float4*>(s_v + (sg + u) * DV + colbase);
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
          const float4 kq = *reinterpret_cast<const float4*>(s_k + (rg + NRG * j) * KWS + sg);
          s[j][0] += kq.x * v4[0].x + kq.y * v4[1].x + kq.z * v4[2].x + kq.w * v4[3].x;
          s[j][1] += kq.x * v4[0].y + kq.y * v4[1].y + kq.z * v4[2].y + kq.w * v4[3].y;
          s[j][2] += kq.x * v4[0].z + kq.y * v4[1].z + kq.z * v4[2].z + kq.w * v4[3].z;
          s[j][3] += kq.x * v4[0].w + kq.y * v4[1].w + kq.z * v4[2].w + kq.w * v4[3].w;
        }
      }
    } else {
      // delta rule, one entry at a time
      for (int i = 0; i < n; ++i) {
        float kk[RPL];
        const float* kp = s_k + i * XLEN + rg * XS;
#pragma unroll
        for (int j = 0; j < RPL; ++j) kk[j] = kp[j];
        if (FAM == FAM_KDA) {
          const float* gp = s_k + (WMAX + i) * XLEN + rg * XS;
#pragma unroll
          for (int j = 0; j < RPL; ++j) {
            const float gj = gp[j];
#pragma unroll
            for (int c = 0; c < 4; ++c) s[j][c] *= gj;
          }
        }
        float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPL; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) u[c] += s[j][c] * kk[j];
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = xsum<LB, NB>(u[c]);
        const float4 v4 = *reinterpret_cast<const float4*>(s_v + i * DV + colbase);
        const float v[4] = {v4.x, v4.y, v4.z, v4.w};
        const float beta = s_w[i];
        float dl[4];
        if (FAM == FAM_GDN) {
          const float al = s_a[i];
#pragma unroll
          for (int c = 0; c < 4; ++c) dl[c] = beta * (v[c] - al * u[c]);
#pragma unroll
          for (int j = 0; j < RPL; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) s[j][c] = al * s[j][c] + kk[j] * dl[c];
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) dl[c] = beta * (v[c] - u[c]);
#pragma unroll
          for (int j = 0; j < RPL; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) s[j][c] += kk[j] * dl[c];
        }
      }
    }

    // ------------------------------------------ exact output S^T q
    if (want_out) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      const float* qp = s_q + rg * XS;
#pragma unroll
      for (int j = 0; j < RPL; ++j) {
        const float qj = qp[j];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += s[j][c] * qj;
      }
      // four columns over NRG >= 4 row groups: halve over the top two lane
      // bits (one column per lane), plain sums over the rest
      constexpr int NB1 = 2;
      constexpr int NB0 = NB - NB1;
      tr_reduce<4, LB + NB0, NB1>(acc, lane);
      out_val = xsum<LB, NB0>(acc[0]);
      out_c = (lane >> (LB + NB0)) & 3;
      out_writer = ((lane >> LB) & ((1 << NB0) - 1)) == 0;
    }
  } else {
    // ----------------------- ReplaySSM non-flush: exact S0^T q~ + o_buf
    if (FAM == FAM_M2) {
      // q~ = D q ; buffered term sum_i (k_i . q) (w_i v_i)
      if (wv == 0 && lane < n) {
        float d = 0.f;
        for (int m = 0; m < DK; ++m) d += s_k[m * KWS + lane] * s_q[T::perm(m)];
        s_e[lane] = d;
      }
      const float D = s_misc[0];
      for (int m = tid; m < DK; m += NT) s_qt[T::perm(m)] = D * s_q[T::perm(m)];
    } else if (wv == 0) {
      // serial pull-back, newest entry first: d = k_i . r ; e_i = beta_i d ;
      // r <- alpha (r - beta d k) (GDN) or g (.) (r - beta d k) (KDA)
      constexpr int EK = DK >= 64 ? DK / 64 : 1;
      float r[EK];
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const int m = lane * EK + e;
        r[e] = (m < DK) ? s_q[T::perm(m)] : 0.f;
      }
      for (int t = 0; t < n; ++t) {
        const int i = n - 1 - t;
        float kk[EK];
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
          const int m = lane * EK + e;
          kk[e] = (m < DK) ? s_k[i * XLEN + T::perm(m)] : 0.f;
          d += kk[e] * r[e];
        }
        d = xsum<0, 6>(d);
        const float beta = s_w[i];
        if (lane == 0) s_e[i] = beta * d;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
          const int m = lane * EK + e;
          const float dec = (FAM == FAM_GDN) ? s_a[i]
                                             : ((m < DK) ? s_k[(WMAX + i) * XLEN + T::perm(m)] : 0.f);
          r[e] = dec * (r[e] - beta * d * kk[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const int m = lane * EK + e;
        if (m < DK) s_qt[T::perm(m)] = r[e];
      }
    }
    __syncthreads();
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const float* qp = s_qt + rg * XS;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const float qj = qp[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += s[j][c] * qj;
    }
    constexpr int NB1 = 2;
    constexpr int NB0 = NB - NB1;
    tr_reduce<4, LB + NB0, NB1>(acc, lane);
    const float vsum = xsum<LB, NB0>(acc[0]);
    out_c = (lane >> (LB + NB0)) & 3;
    out_writer = ((lane >> LB) & ((1 << NB0) - 1)) == 0;
    float ob = 0.f;
    for (int i = 0; i < n; ++i) ob += s_e[i] * s_v[i * DV + colbase + out_c];
    out_val = vsum + ob;
  }

  // ----------------------------------------------------------- output
  if (want_out && out_writer) {
    AT* o = reinterpret_cast<AT*>(p.o) + bh * DV + colbase + out_c;
    st(o, out_val);
  }

  if (do_flush) {
    // ------------------------------------------------ store the state
    float* Sw = p.S + bh * DK * DV + colbase;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const f32x4 v4 = {s[j][0], s[j][1], s[j][2], s[j][3]};
      __builtin_nontemporal_store(v4, reinterpret_cast<f32x4*>(Sw + (size_t)(rg + NRG * j) * DV));
    }

    // --------------------------------- sketch U = S^T P (flush only)
    if (want_u) {
      const int r4 = round4(r);
      float4 pr[PU];
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const int c = tid + NT * u;
        pr[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < r * PCPR) {
          const int j = c / PCPR, m0 = (c - j * PCPR) * 4;
          pr[u] = *reinterpret_cast<const float4*>(p.Pt + (size_t)(off + j) * DK + m0);
        }
      }
      __syncthreads();   // keys no longer needed: stage the basis over them
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const int c = tid + NT * u;
        if (c < r4 * PCPR) {
          const int j = c / PCPR, m0 = (c - j * PCPR) * 4;
          const float x[4] = {pr[u].x, pr[u].y, pr[u].z, pr[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) s_p[(m0 + e) * PS + j] = (j < r) ? x[e] : 0.0f;
        }
      }
      __syncthreads();
      UT* Ub = reinterpret_cast<UT*>(p.U) + ((size_t)b * p.R + off) * DV + colbase;
      for (int ch = 0; ch < r4; ch += 4) {
        float acc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
          const float4 pv = *reinterpret_cast<const float4*>(s_p + (rg + NRG * j) * PS + ch);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[c * 4 + 0] += s[j][c] * pv.x;
            acc[c * 4 + 1] += s[j][c] * pv.y;
            acc[c * 4 + 2] += s[j][c] * pv.z;
            acc[c * 4 + 3] += s[j][c] * pv.w;
          }
        }
        constexpr int NBU = NB <= 4 ? NB : 4;
        constexpr int NBR = NB - NBU;
        tr_reduce<16, LB + NBR, NBU>(acc, lane);
        constexpr int K = 16 >> NBU;
        const int sel = (lane >> (LB + NBR)) & ((1 << NBU) - 1);
        const bool writer = ((lane >> LB) & ((1 << NBR) - 1)) == 0;
#pragma unroll
        for (int e = 0; e < K; ++e) {
          const float val = xsum<LB, NBR>(acc[e]);
          const int idx = sel * K + e;
          const int c = idx >> 2, jj = idx & 3;
          if (writer && ch + jj < r) st(Ub + (size_t)(ch + jj) * DV + c, val);
        }
      }
    }
  }

  // ------------------------------------------------------ ring count
  if (MODE != MODE_FULL) {
    __syncthreads();       // every wave has read the count
    if (tid == 0) p.count[bh] = do_flush ? 0 : n;
  }
}

}  // namespace sk
