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
#pragma once

#include "sk_device.hpp"
#include "sk_params.hpp"

namespace sk {

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr int round4(int x) { return (x + 3) & ~3; }

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

// LDS floats needed by a tile kernel.
template <int FAM, int DK, int DV>
__host__ __device__ constexpr int tile_lds_floats(int W) {
  using T = TileShape<DK, DV>;
  // q (permuted) + effective query (permuted) + per-slot scalars (4 arrays of W+4)
  const int base = 2 * T::XLEN + 4 * (W + 4) + 4;
  const int pbuf = DK * T::PS;                                   // staged basis
  const int ent = FAM == FAM_M2 ? DK * (round4(W) + 4)           // w_i k_i[m], [m][slot]
                                 : W * T::XLEN * (FAM == FAM_KDA ? 2 : 1);  // k_i (and g_i), [slot][perm m]
  return base + (ent > pbuf ? ent : pbuf);
}

template <int FAM, int DK, int DV, typename AT, typename UT, int MODE>
__global__ void __launch_bounds__((TileShape<DK, DV>::THREADS))
tile_kernel(Params p) {
  using T = TileShape<DK, DV>;
  constexpr int CB = T::CB, NCG = T::NCG, NRG = T::NRG, RPL = T::RPL;
  constexpr int LB = T::LB, NB = T::NB, XS = T::XS, XLEN = T::XLEN, PS = T::PS;
  constexpr int NT = T::THREADS;

  extern __shared__ float smem[];
  const int W = p.W;
  float* s_q = smem;                    // [XLEN] query, permuted
  float* s_qt = s_q + XLEN;             // [XLEN] effective query, permuted (replay)
  float* s_a = s_qt + XLEN;             // [W+4] per-slot decay (M2 a_i, GDN alpha_i)
  float* s_w = s_a + (W + 4);           // [W+4] per-slot write weight (M2 w_i, GDN/KDA beta_i)
  float* s_e = s_w + (W + 4);           // [W+4] per-slot buffered-output coefficient
  float* s_x = s_e + (W + 4);           // [W+4] spare per-slot scalars (M2 dt_i)
  float* s_misc = s_x + (W + 4);        // [4]: [0] = M2 total decay D
  float* s_big = s_misc + 4;            // entries, later the staged basis

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

  // entry sources: slot < n0 from the ring, slot n0 (has_in) from the step
  const AT* ring_k = reinterpret_cast<const AT*>(p.rk) + ((size_t)b * p.G + g) * W * DK;
  const AT* ring_v = reinterpret_cast<const AT*>(p.rv) + bh * W * DV;
  const AT* in_k = has_in ? reinterpret_cast<const AT*>(p.k) + ((size_t)b * p.G + g) * DK : nullptr;
  const AT* in_v = has_in ? reinterpret_cast<const AT*>(p.v) + bh * DV : nullptr;
  auto key_ptr = [&](int i) -> const AT* { return (has_in && i == n0) ? in_k : ring_k + (size_t)i * DK; };
  auto val_ptr = [&](int i) -> const AT* { return (has_in && i == n0) ? in_v : ring_v + (size_t)i * DV; };
  auto gate_scalar = [&](int i) -> float {
    if (FAM == FAM_M2) {
      if (has_in && i == n0) return ld(reinterpret_cast<const AT*>(p.gate) + bh);
      return ld(reinterpret_cast<const AT*>(p.rg) + bh * W + i);
    }
    if (has_in && i == n0) return reinterpret_cast<const float*>(p.gate)[bh];
    return reinterpret_cast<const float*>(p.rg)[bh * W + i];
  };
  auto gate_vec = [&](int i) -> const float* {   // KDA g_i
    if (has_in && i == n0) return reinterpret_cast<const float*>(p.gate) + bh * DK;
    return reinterpret_cast<const float*>(p.rg) + (bh * W + i) * DK;
  };
  auto beta_of = [&](int i) -> float {
    if (has_in && i == n0) return p.beta[bh];
    return p.rb[bh * W + i];
  };

  // ------------------------------------------------ append (ReplaySSM)
  if (MODE == MODE_REPLAY) {
    // per-head parts; the per-group key is appended by the group's first head
    AT* rv = reinterpret_cast<AT*>(p.rv) + (bh * W + n0) * DV;
    for (int e = tid; e < DV; e += NT) rv[e] = reinterpret_cast<const AT*>(p.v)[bh * DV + e];
    if (h % p.HPG == 0) {
      AT* rk = reinterpret_cast<AT*>(p.rk) + (((size_t)b * p.G + g) * W + n0) * DK;
      for (int e = tid; e < DK; e += NT) rk[e] = in_k[e];
    }
    if (FAM == FAM_KDA) {
      float* rgv = reinterpret_cast<float*>(p.rg) + (bh * W + n0) * DK;
      for (int e = tid; e < DK; e += NT) rgv[e] = reinterpret_cast<const float*>(p.gate)[bh * DK + e];
    } else if (tid == 0) {
      AT* rgs = reinterpret_cast<AT*>(p.rg);
      if (FAM == FAM_M2) rgs[bh * W + n0] = reinterpret_cast<const AT*>(p.gate)[bh];
      else reinterpret_cast<float*>(p.rg)[bh * W + n0] = reinterpret_cast<const float*>(p.gate)[bh];
    }
    if (FAM != FAM_M2 && tid == 0) p.rb[bh * W + n0] = p.beta[bh];
  }

  // --------------------------------------------- load the state block
  const float* Sg = p.S + bh * DK * DV + wv * CB + 4 * cg;
  float s[RPL][4];
#pragma unroll
  for (int j = 0; j < RPL; ++j) ld4(Sg + (size_t)(rg + NRG * j) * DV, s[j]);

  // ---------------------------------------------------- stage the query
  const bool want_out = (MODE != MODE_FLUSH) || p.q != nullptr;
  if (want_out) {
    const AT* q = reinterpret_cast<const AT*>(p.q) + ((size_t)b * p.G + g) * DK;
    for (int m = tid; m < DK; m += NT) s_q[T::perm(m)] = ld(q + m);
  }

  // ------------------------------------------ stage per-slot quantities
  if (FAM == FAM_M2) {
    const float Ah = p.A[h];
    for (int i = tid; i < n; i += NT) {
      const float dt = gate_scalar(i);
      s_x[i] = dt;
      s_a[i] = m2_decay(dt, Ah);
    }
  } else {
    for (int i = tid; i < n; i += NT) {
      s_a[i] = (FAM == FAM_GDN) ? gate_scalar(i) : 1.0f;
      s_w[i] = beta_of(i);
    }
  }
  __syncthreads();

  float* s_ent = s_big;
  if (FAM == FAM_M2) {
    // w_i = dt_i * prod_{t>i} a_t (flush) ; D = prod_t a_t
    for (int i = tid; i < n; i += NT) {
      float suf = 1.0f;
      for (int t = i + 1; t < n; ++t) suf *= s_a[t];
      s_w[i] = s_x[i] * suf;
      if (i == 0) s_misc[0] = s_a[0] * suf;
    }
    if (n == 0 && tid == 0) s_misc[0] = 1.0f;
  }
  if (FAM == FAM_M2 && do_flush) {
    __syncthreads();
    // s_ent[m][i] = w_i k_i[m], zero-padded to a multiple of 4 slots
    const int KWS = round4(W) + 4;
    const int n4 = round4(n);
    for (int idx = tid; idx < n4 * DK; idx += NT) {
      const int i = idx / DK, m = idx - i * DK;
      s_ent[m * KWS + i] = (i < n) ? s_w[i] * ld(key_ptr(i) + m) : 0.0f;
    }
  } else if (FAM != FAM_M2 && do_flush) {
    for (int idx = tid; idx < n * DK; idx += NT) {
      const int i = idx / DK, m = idx - i * DK;
      s_ent[i * XLEN + T::perm(m)] = ld(key_ptr(i) + m);
      if (FAM == FAM_KDA) s_ent[(W + i) * XLEN + T::perm(m)] = gate_vec(i)[m];
    }
  }
  __syncthreads();

  float out_val = 0.0f;      // reduced output value owned by this lane
  int out_c = 0;             // its column within the lane's group of four
  bool out_writer = false;

  if (do_flush) {
    // -------------------------------------------- apply the entries
    if (FAM == FAM_M2) {
      // S <- D S + sum_i (w_i k_i) v_i^T  (the W Mamba-2 steps in closed form)
      const float D = s_misc[0];
      const int KWS = round4(W) + 4;
#pragma unroll
      for (int j = 0; j < RPL; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) s[j][c] *= D;
      for (int sg = 0; sg < n; sg += 4) {
        float v[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (sg + u < n) ld4(val_ptr(sg + u) + wv * CB + 4 * cg, v[u]);
          else v[u][0] = v[u][1] = v[u][2] = v[u][3] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
          const float4 kw = *reinterpret_cast<const float4*>(s_ent + (rg + NRG * j) * KWS + sg);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            s[j][c] += kw.x * v[0][c] + kw.y * v[1][c] + kw.z * v[2][c] + kw.w * v[3][c];
        }
      }
    } else {
      // delta rule, one entry at a time
      for (int i = 0; i < n; ++i) {
        const float* kp = s_ent + i * XLEN + rg * XS;
        if (FAM == FAM_KDA) {
          const float* gp = s_ent + (W + i) * XLEN + rg * XS;
#pragma unroll
          for (int j = 0; j < RPL; ++j) {
            const float gj = gp[j];
#pragma unroll
            for (int c = 0; c < 4; ++c) s[j][c] *= gj;
          }
        }
        float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
          const float kj = kp[j];
#pragma unroll
          for (int c = 0; c < 4; ++c) u[c] += s[j][c] * kj;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = xsum<LB, NB>(u[c]);
        float v[4];
        ld4(val_ptr(i) + wv * CB + 4 * cg, v);
        const float beta = s_w[i];
        float dl[4];
        if (FAM == FAM_GDN) {
          const float al = s_a[i];
#pragma unroll
          for (int c = 0; c < 4; ++c) dl[c] = beta * (v[c] - al * u[c]);
#pragma unroll
          for (int j = 0; j < RPL; ++j) {
            const float kj = kp[j];
#pragma unroll
            for (int c = 0; c < 4; ++c) s[j][c] = al * s[j][c] + kj * dl[c];
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) dl[c] = beta * (v[c] - u[c]);
#pragma unroll
          for (int j = 0; j < RPL; ++j) {
            const float kj = kp[j];
#pragma unroll
            for (int c = 0; c < 4; ++c) s[j][c] += kj * dl[c];
          }
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
      float vsum = xsum<LB, NB0>(acc[0]);
      const int sel = (lane >> (LB + NB0)) & ((1 << NB1) - 1);
      out_val = vsum;
      out_c = sel;
      out_writer = ((lane >> LB) & ((1 << NB0) - 1)) == 0;
    }
  } else {
    // ----------------------- ReplaySSM non-flush: exact S0^T q~ + o_buf
    // effective query and buffered-output coefficients
    if (FAM == FAM_M2) {
      // q~ = D q ; e_i = w_i (k_i . q) with w_i = dt_i prod_{t>i} a_t
      const AT* q = reinterpret_cast<const AT*>(p.q) + ((size_t)b * p.G + g) * DK;
      for (int i = wv; i < n; i += T::NCB) {
        const AT* k = key_ptr(i);
        float d = 0.f;
        for (int m = lane; m < DK; m += 64) d += ld(k + m) * ld(q + m);
        d = xsum<0, 6>(d);
        if (lane == 0) s_e[i] = s_w[i] * d;
      }
      const float D = s_misc[0];
      for (int m = tid; m < DK; m += NT) s_qt[T::perm(m)] = D * ld(q + m);
    } else if (wv == 0) {
      // serial pull-back, newest entry first: d = k_i . r ; e_i = beta_i d ;
      // r <- alpha (r - beta d k) (GDN) or g (.) (r - beta d k) (KDA)
      constexpr int EK = DK >= 64 ? DK / 64 : 1;
      const AT* q = reinterpret_cast<const AT*>(p.q) + ((size_t)b * p.G + g) * DK;
      float r[EK];
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const int m = lane * EK + e;
        r[e] = (m < DK) ? ld(q + m) : 0.f;
      }
      for (int t = 0; t < n; ++t) {
        const int i = n - 1 - t;
        const AT* k = key_ptr(i);
        float kk[EK];
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
          const int m = lane * EK + e;
          kk[e] = (m < DK) ? ld(k + m) : 0.f;
          d += kk[e] * r[e];
        }
        d = xsum<0, 6>(d);
        const float beta = s_w[i];
        if (lane == 0) s_e[i] = beta * d;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
          const int m = lane * EK + e;
          const float dec = (FAM == FAM_GDN) ? s_a[i] : ((m < DK) ? gate_vec(i)[m] : 0.f);
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
    float vsum = xsum<LB, NB0>(acc[0]);
    const int sel = (lane >> (LB + NB0)) & ((1 << NB1) - 1);
    out_c = sel;
    out_writer = ((lane >> LB) & ((1 << NB0) - 1)) == 0;
    // buffered term for this lane's output column
    const int col = wv * CB + 4 * cg + out_c;
    float ob = 0.f;
    for (int i = 0; i < n; ++i) ob += s_e[i] * ld(val_ptr(i) + col);
    out_val = vsum + ob;
  }

  // ----------------------------------------------------------- output
  if (want_out && out_writer) {
    AT* o = reinterpret_cast<AT*>(p.o) + bh * DV + wv * CB + 4 * cg + out_c;
    st(o, out_val);
  }

  if (do_flush) {
    // ------------------------------------------------ store the state
    float* Sw = p.S + bh * DK * DV + wv * CB + 4 * cg;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const f32x4 v4 = {s[j][0], s[j][1], s[j][2], s[j][3]};
      __builtin_nontemporal_store(v4, reinterpret_cast<f32x4*>(Sw + (size_t)(rg + NRG * j) * DV));
    }

    // --------------------------------- sketch U = S^T P (flush only)
    if (MODE == MODE_FLUSH) {
      const int off = p.off[h];
      const int r = p.off[h + 1] - off;
      const int r4 = round4(r);
      __syncthreads();   // entries no longer needed: stage the basis over them
      float* s_p = s_big;
      for (int idx = tid; idx < r4 * DK; idx += NT) {
        const int j = idx / DK, m = idx - j * DK;
        s_p[m * PS + j] = (j < r) ? p.Pt[(size_t)(off + j) * DK + m] : 0.0f;
      }
      __syncthreads();
      UT* Ub = reinterpret_cast<UT*>(p.U) + ((size_t)b * p.R + off) * DV + wv * CB + 4 * cg;
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
