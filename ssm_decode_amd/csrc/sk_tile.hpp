// Tile kernels: one workgroup per (sequence, head) tile that reads the full
// state.  Used by the flush, the standard full-state step and the ReplaySSM
// step.  The state tile S (dk x dv fp32) is held in registers for the whole
// kernel: it is loaded once with wide loads, updated, reduced against the
// query / basis vectors and stored once.
//
// Register layout.  The dv columns are split into column blocks of CB = 32
// columns (dv when smaller), one wave per block: a 128 x 32 block is 64
// registers per lane, which leaves room for the delta-rule and ReplaySSM
// paths without spills and runs 3-4 waves per SIMD.  With cg = lane % 16 and
// rg = lane / 16, lane l holds the NCC = CB/16 consecutive columns
// NCC*cg .. NCC*cg+NCC-1 of its block and, for every 16-row block mb, the four
// consecutive rows 16*mb + 4*rg + v (v = 0..3):
//     sacc[mb][c][v] = S[16 mb + 4 rg + v][NCC cg + c]
// This is at once
//   - the accumulator layout of v_mfma_f32_16x16x4_f32 (D[4 rg + v][cg]) for
//     the 16 x 16 block (rows 16 mb.., columns NCC j + c), so the Mamba-2
//     rank-W update S += K V'^T runs on the matrix cores with S in place, and
//   - the A-operand layout (A[cg][rg]) of the same instruction for S^T, with
//     K-step (mb, v) covering rows 16 mb + 4 k + v, so U = S^T P needs no
//     data movement either;
// and every lane's NCC columns of a row are one 64-bit (NCC = 2) or 128-bit
// (NCC = 4) load or store.
//
// Latency structure.  Every global load the tile needs besides the state
// (ring keys, values and gates, the basis rows, the query) is issued first,
// as 16-byte chunks spread over the workgroup, then the state loads; the
// small loads are staged into LDS as fp32 while the state is in flight.
#pragma once

#include "sk_device.hpp"
#include "sk_params.hpp"

namespace sk {

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr int round4(int x) { return (x + 3) & ~3; }
constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int DK, int DV>
struct TileShape {
  // columns per wave: 32 (a 128 x 32 block is 64 registers per lane), or dv
  // when smaller
  static constexpr int CB = DV >= 64 ? 32 : DV;
  static constexpr int NCB = DV / CB;             // waves per tile
  static constexpr int NCC = CB / 16;             // consecutive columns per lane
  static constexpr int MB = DK / 16;              // 16-row blocks
  static constexpr int THREADS = 64 * NCB;
  static constexpr int PS = 20;                   // padded row stride of the staged basis (16 + 4)
  static_assert(DK % 16 == 0 && (NCC == 2 || NCC == 4), "unsupported dk/dv");
  static_assert(DV % CB == 0, "unsupported dv");
};

// LDS layout of a tile kernel (offsets in floats).
template <int FAM, int DK, int DV, int WMAX, int MODE, int COEF>
struct TileLds {
  using T = TileShape<DK, DV>;
  static constexpr int KWS = WMAX + 4;                         // Mamba-2 key row stride ([m][slot])
  static constexpr int Q = 0;                                  // query [dk]
  static constexpr int QT = Q + DK;                            // effective query [dk]
  static constexpr int SA = QT + DK;                           // per-slot scalars
  static constexpr int SW = SA + WMAX;
  static constexpr int SE = SW + WMAX;
  static constexpr int SX = SE + WMAX;
  static constexpr int MISC = SX + WMAX;
  static constexpr int V = MISC + 4;                           // values [slot][dv]
  static constexpr int KEYS0 = V + WMAX * DV;                  // keys: M2 [m][slot]; GDN/KDA [slot][m]
  static constexpr int KEYS = FAM == FAM_M2 ? DK * KWS : WMAX * DK * (FAM == FAM_KDA ? 2 : 1);
  static constexpr int BASIS = DK * T::PS;                     // basis [m][j], over the keys after the update
  static constexpr int P0 = KEYS0;
  // GDN/KDA chunked update, after the raw keys (and KDA gates):
  static constexpr int KQ = KEYS0 + KEYS;                      // k_i (.) Gamma_i   [m][slot]
  static constexpr int KD = KQ + DK * KWS;                     // k_i (/) Gamma_i   [m][slot]
  static constexpr int AM = KD + DK * KWS;                     // A [i][j], stride WMAX + 1
  static constexpr int GF = AM + round4(WMAX * (WMAX + 1));    // Gamma after the last entry [dk]
  // (only the flush reserves them: the ReplaySSM step flushes one step in W
  // and takes the serial form, keeping its LDS and occupancy)
  static constexpr bool CHUNK = FAM != FAM_M2 && MODE == MODE_FLUSH;
  static constexpr int DN_END = CHUNK ? GF + DK : 0;
  static constexpr int T0 = KEYS0 + (KEYS > BASIS ? KEYS : BASIS);
  // state-dependent map (flush), used once every wave is past the sketch:
  // each wave stages 16 state rows of its column block at a time (SST), and
  // publishes its partial Y block of every band another wave owns (PART,
  // [band][NCB - 1][lane] of 4 floats) and its partial Gram matrix (GP,
  // [wave][lane]); wave 0 writes the 16 x 16 inverse (GINV)
  static constexpr int SSTR = T::CB + 4;                       // staged row stride
  static constexpr int SST = 0;
  static constexpr int PART = SST + T::NCB * 16 * SSTR;
  static constexpr int GP = PART + T::MB * (T::NCB - 1) * 256;
  static constexpr int GINV = GP + T::NCB * 256;
  static constexpr int MAP_END = COEF ? GINV + 256 : 0;
  static_assert(PART % 4 == 0, "LDS regions must be 16-byte aligned");
  static constexpr int T1 = T0 > DN_END ? T0 : DN_END;
  static constexpr int TOTAL = T1 > MAP_END ? T1 : MAP_END;
  static constexpr int BYTES = TOTAL * 4;
  static_assert(V % 4 == 0 && KEYS0 % 4 == 0 && P0 % 4 == 0 && GF % 4 == 0,
                "LDS regions must be 16-byte aligned");
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

// Which tile kernels address the state through a buffer resource.
template <int FAM, int MODE>
struct STATE_BUFFER {
  static constexpr bool value = FAM != FAM_M2 && MODE == MODE_FLUSH;
};

// D += A B for one 16x16x4 fp32 block (A: lane holds A[lane%16][lane/16],
// B: lane holds B[lane/16][lane%16], D: lane holds D[4(lane/16)+v][lane%16]).
__device__ __forceinline__ f32x4v mfma16x4(float a, float b, f32x4v d) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, d, 0, 0, 0);
}

// Row R of 16 lanes broadcast to all four rows (two lane-swap steps).
template <int R>
__device__ __forceinline__ float row_bcast(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned a = (R & 1) ? s[1] : s[0];
  const auto t = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  return __uint_as_float((R & 2) ? t[1] : t[0]);
}

// One pivot of the in-place Gauss-Jordan inversion of a 16 x 16 matrix held
// as lane (cg, rg): m[v] = M[4 rg + v][cg].
template <int K>
__device__ __forceinline__ void gj_pivot(float (&m)[4], int cg, int rg) {
  const float mkj = row_bcast<K / 4>(m[K & 3]);                 // M[K][cg]
  float mik[4];
#pragma unroll
  for (int v = 0; v < 4; ++v)                                   // M[4 rg + v][K]: row_newbcast:K
    mik[v] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m[v]), 0x150 + K, 0xF, 0xF, false));
  const float piv = 1.f / __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mkj), K));
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int i = 4 * rg + v;
    if (i == K) m[v] = (cg == K) ? piv : mkj * piv;
    else m[v] = (cg == K) ? -mik[v] * piv : m[v] - mik[v] * (mkj * piv);
  }
}
template <int K>
__device__ __forceinline__ void gj_invert(float (&m)[4], int cg, int rg) {
  if constexpr (K < 16) {
    gj_pivot<K>(m, cg, rg);
    gj_invert<K + 1>(m, cg, rg);
  }
}

// State-dependent coefficient map of one tile at the flush (project page,
// per-window flush panel: C = (U^T U)^+ U^T S0^T; paper App. A.2.1-A.2.2):
// with U_h the sketch rows as stored (rounded to the sketch dtype) and S the
// updated state,
//     G = U_h U_h^T (r x r),  Y = U_h S^T (r x dk),  C = (G + lambda I)^{-1} Y,
//     lambda = ridge * trace(G) / r   (C = 0 when the sketch is zero),
// stored in the sketch dtype as rows off .. off + r - 1 of sequence b.
//
// Both contractions run over the state's columns, which the register layout
// spreads over lanes (it contracts over rows only), so:
//   - the sketch values a lane already holds, u_j (j = lane % 16) at the 8
//     columns 8 (lane / 16) + t of its wave's block, are the A operand of
//     v_mfma_f32_16x16x4_f32 for K-step t; for G they are the B operand too;
//   - for Y each wave stages its 16 x 32 block of every 16-row band of S in
//     LDS and reads it back transposed as the B operand (8 K-steps a band);
//   - band mb belongs to wave mb % waves, which keeps its own partial Y block
//     in registers; the other waves publish theirs, and their partial G,
//     through LDS; wave 0 inverts G + lambda I (Gauss-Jordan, no pivoting: the matrix is
//     symmetric positive definite) with lane (j, i / 4) holding column j;
//   - C = (G + lambda I)^{-1} Y is one more 4-step MFMA per 16-column band,
//     each wave taking the bands b % waves == its index.
// Padding rows j >= r of the sketch are zero, so the padded part of G is set
// to the identity and the padded rows of C are zero and not stored.
template <int DK, int DV, typename UT, typename LY>
__device__ __forceinline__ void coef_map(const Params& p, float* smem,
                                         const f32x4v (&sacc)[DK / 16][TileShape<DK, DV>::NCC],
                                         const f32x4v (&u)[TileShape<DK, DV>::NCC], int b, int off,
                                         int r) {
  using T = TileShape<DK, DV>;
  constexpr int NCC = T::NCC, MB = T::MB, NCB = T::NCB, SSTR = LY::SSTR;
  static_assert(NCC == 2, "the map assumes two columns per lane (8 sketch columns per lane)");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int cg = lane & 15, rg = lane >> 4;

  // the sketch as stored: uh[t] = u_j at column 8 rg + t of the wave's block
  float uh[8];
#pragma unroll
  for (int vv = 0; vv < 4; ++vv)
#pragma unroll
    for (int c = 0; c < NCC; ++c) uh[NCC * vv + c] = to_f32(Store<UT>::cvt(u[c][vv]));

  f32x4v gp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 8; ++t) gp = mfma16x4(uh[t], uh[t], gp);

  // Y blocks: band mb gives Y[4 rg + v][16 mb + cg] in lane (cg, rg).  The
  // band's owner (wave mb % NCB) keeps its partial in registers; the other
  // waves publish theirs.
  constexpr int MBW = (MB + NCB - 1) / NCB;
  __syncthreads();          // every wave is past its sketch: the basis is free
  float* s_st = smem + LY::SST + wv * 16 * SSTR;
  f32x4v* part = reinterpret_cast<f32x4v*>(smem + LY::PART);
  f32x4v own[MBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      *reinterpret_cast<float2*>(s_st + (4 * rg + v) * SSTR + NCC * cg) =
          make_float2(sacc[mb][0][v], sacc[mb][1][v]);
    // read back by the same wave (its LDS operations complete in order):
    // row 16 mb + cg, columns 8 rg .. 8 rg + 7 of the block
    const float4 s0 = *reinterpret_cast<const float4*>(s_st + cg * SSTR + 8 * rg);
    const float4 s1 = *reinterpret_cast<const float4*>(s_st + cg * SSTR + 8 * rg + 4);
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    f32x4v yp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) yp = mfma16x4(uh[t], sv[t], yp);
    const int owner = mb % NCB;
    if (wv == owner) {
      own[mb / NCB] = yp;
    } else {
      const int k = wv < owner ? wv : wv - 1;
      part[(mb * (NCB - 1) + k) * 64 + lane] = yp;
    }
  }
  reinterpret_cast<f32x4v*>(smem + LY::GP)[wv * 64 + lane] = gp;
  __syncthreads();

  float* s_gi = smem + LY::GINV;
  if (wv == 0) {
    const f32x4v* gpa = reinterpret_cast<const f32x4v*>(smem + LY::GP);
    f32x4v g = gpa[lane];
#pragma unroll
    for (int w = 1; w < NCB; ++w) g += gpa[w * 64 + lane];
    // lane (cg, rg) holds G[4 rg + v][cg]
    float dg = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (4 * rg + v == cg && cg < r) dg += g[v];
    const float tr = wave_sum(dg);
    const float lam = tr > 0.f ? p.ridge * tr / (float)r : 1.f;
    float m[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = 4 * rg + v;
      const bool in = i < r && cg < r;
      m[v] = (i == cg) ? (in ? g[v] + lam : 1.f) : (in ? g[v] : 0.f);
    }
    // in-place Gauss-Jordan inversion, pivot k: with p = 1 / M[k][k],
    //   M[k][k] <- p,            M[k][j] <- M[k][j] p              (j != k)
    //   M[i][k] <- -M[i][k] p,   M[i][j] <- M[i][j] - M[i][k] M[k][j] p
    gj_invert<0>(m, cg, rg);
    // inverse row-major: s_gi[i][j]
#pragma unroll
    for (int v = 0; v < 4; ++v) s_gi[(4 * rg + v) * 16 + cg] = m[v];
  }
  // each wave's own bands: add the other waves' partial Y blocks
  f32x4v y[MBW];
#pragma unroll
  for (int q = 0; q < MBW; ++q) {
    const int mb = wv + q * NCB;
    y[q] = own[q];
    if (mb < MB) {
#pragma unroll
      for (int k = 0; k < NCB - 1; ++k) y[q] += part[(mb * (NCB - 1) + k) * 64 + lane];
    }
  }
  __syncthreads();
  // A operand of step v: Ginv[cg][4 rg + v]
  const float4 ga4 = *reinterpret_cast<const float4*>(s_gi + cg * 16 + 4 * rg);
  const float ga[4] = {ga4.x, ga4.y, ga4.z, ga4.w};
  UT* Cb = reinterpret_cast<UT*>(p.Cs) + ((size_t)b * p.R + off) * DK;
  constexpr bool STAGE = sizeof(UT) == 2 && 16 * DK * 2 <= LY::PART * 4;
  UT* s_cm = reinterpret_cast<UT*>(smem + LY::SST);   // [16][DK] (STAGE)
#pragma unroll
  for (int q = 0; q < MBW; ++q) {
    const int mb = wv + q * NCB;
    if (mb < MB) {
      f32x4v cm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) cm = mfma16x4(ga[v], y[q][v], cm);
      // lane holds C[4 rg + v][16 mb + cg]
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 4 * rg + v;
        if constexpr (STAGE) s_cm[j * DK + 16 * mb + cg] = Store<UT>::cvt(cm[v]);
        else if (j < r) st(Cb + (size_t)j * DK + 16 * mb + cg, cm[v]);
      }
    }
  }
  if constexpr (STAGE) {
    // whole rows, 16 bytes a thread
    constexpr int CPR = DK * 2 / 16;                 // 16-byte chunks per row
    __syncthreads();
    for (int c = threadIdx.x; c < r * CPR; c += (int)blockDim.x) {
      const int j = c / CPR, ch = c - j * CPR;
      reinterpret_cast<uint4*>(Cb + (size_t)j * DK)[ch] = reinterpret_cast<const uint4*>(s_cm + j * DK)[ch];
    }
  }
}

// (the delta-rule flush runs three waves per SIMD: its chunked update has
// serial phases that more resident tiles hide)
template <int FAM, int DK, int DV, typename AT, typename UT, int MODE, int WMAX, int COEF, bool DENSE>
__global__ void __launch_bounds__((TileShape<DK, DV>::THREADS), (MODE == MODE_FLUSH && FAM != FAM_M2 ? 3 : 2))
tile_kernel(Params p) {
  using T = TileShape<DK, DV>;
  using LY = TileLds<FAM, DK, DV, WMAX, MODE, COEF>;
  constexpr int CB = T::CB, NCC = T::NCC, MB = T::MB, PS = T::PS;
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
  float* s_k = smem + LY::KEYS0;   // keys: M2 [m][slot]; GDN/KDA [slot][m] (+ KDA gates)
  float* s_p = smem + LY::P0;      // basis [m][j], staged over the keys after the update

  const int W = p.W;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int cg = lane & 15;
  const int rg = lane >> 4;
  const int tile = blockIdx.x;
  const int ts = tile / p.H;
  const int h = tile - ts * p.H;
  int b = ts;
  if (MODE == MODE_FLUSH && p.seq_list) {        // uniform: the tiles of listed sequences
    b = p.seq_list[ts];
    if (b < 0 || b >= p.B) {
      if (threadIdx.x == 0) atomicOr(p.err, ERRBIT_SEQ);
      return;
    }
  }
  const int g = h / p.HPG;
  const size_t bh = (size_t)b * p.H + h;
  const int colbase = wv * CB + NCC * cg;        // first of the lane's columns

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
  // keys: n rows of DK (a Mamba-2 key is shared by the group's heads and
  // stays cacheable; every other ring entry is read by this tile only, with
  // the non-temporal policy)
  constexpr int KC = Chunk<AT>::N;
  constexpr int KCPR = DK / KC;
  constexpr int KU = cdiv(WMAX * KCPR, NT);
  uint4 kr[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int c = tid + NT * u;
    if (c < n * KCPR) {
      const int i = c / KCPR, m0 = (c - i * KCPR) * KC;
      kr[u] = FAM == FAM_M2 ? *reinterpret_cast<const uint4*>(key_ptr(i) + m0) : ld16_nt(key_ptr(i) + m0);
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
      vr[u] = ld16_nt(val_ptr(i) + c0);
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
        const uint4 t = ld16_nt(gate_vec(i) + m0);
        gr[u] = make_float4(__uint_as_float(t.x), __uint_as_float(t.y), __uint_as_float(t.z), __uint_as_float(t.w));
      }
    }
  }
  // basis rows (flush): r rows of DK fp32 (L2 resident), loaded after the update
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
  // State addressing.  As a buffer (delta-rule flush): the lane offset (rows
  // 4 rg.., the lane's columns) in one VGPR and the row-block offset in an
  // SGPR, which frees the registers of one 64-bit pointer per row.  As
  // plain pointers elsewhere (the Mamba-2 kernels run best at their current
  // occupancy).
  constexpr bool SBUF = STATE_BUFFER<FAM, MODE>::value;
  // Cache policy of the state stream: non-temporal where every step of the
  // mode reads and writes the whole state once (flush, standard step); the
  // ReplaySSM step, which re-reads the state at every step and writes it
  // once a window, is measured faster with the default policy.
  constexpr int S_CP = MODE == MODE_REPLAY ? 0 : CP_NT;
  const __amdgpu_buffer_rsrc_t s_rsrc = make_rsrc(p.S + bh * DK * DV, DK * DV * 4);
  const int s_lane = (4 * rg * DV + colbase) * 4;
  f32x4v sacc[MB][NCC];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x[NCC];
      if constexpr (SBUF)
        buf_ld<NCC, S_CP>(s_rsrc, s_lane, (16 * mb + v) * DV * 4, x);
      else if constexpr (S_CP == CP_NT)
        ldn_nt<NCC>(p.S + bh * DK * DV + colbase + (size_t)(16 * mb + 4 * rg + v) * DV, x);
      else
        ldn<NCC>(p.S + bh * DK * DV + colbase + (size_t)(16 * mb + 4 * rg + v) * DV, x);
#pragma unroll
      for (int c = 0; c < NCC; ++c) sacc[mb][c][v] = x[c];
    }

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
      if (m < DK) s_q[m] = qv[u];
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
        else s_k[i * DK + m0 + e] = x[e];
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
        *reinterpret_cast<float4*>(s_k + (WMAX + i) * DK + m0) = gr[u];
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
  int out_c = 0;             // its column within the lane's group of NCC
  bool out_writer = false;

  if (do_flush) {
    // -------------------------------------------- apply the entries
    if (FAM == FAM_M2) {
      // S <- D S + sum_i k_i (w_i v_i)^T, the Mamba-2 steps in closed form, as
      // 16x16x4 matrix products: A = keys (rows 16 mb.., slots t4..t4+3),
      // B = scaled values (slots t4.., columns NCC j + c)
      const float D = s_misc[0];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int c = 0; c < NCC; ++c) sacc[mb][c] *= D;
      for (int t4 = 0; t4 < n; t4 += 4) {
        float bv[NCC];
        ldn<NCC>(s_v + (t4 + rg) * DV + colbase, bv);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float ak = s_k[(16 * mb + cg) * KWS + t4 + rg];
#pragma unroll
          for (int c = 0; c < NCC; ++c) sacc[mb][c] = mfma16x4(ak, bv[c], sacc[mb][c]);
        }
      }
    } else {
      // Delta rule.  With Gamma_i = g_1 (.) .. (.) g_i (GDN: alpha_1 .. alpha_i
      // on every channel), kq_i = k_i (.) Gamma_i and kd_j = k_j (/) Gamma_j,
      // the n updates S_i = (I - b_i k_i k_i^T) Diag(g_i) S_{i-1} + b_i k_i v_i^T
      // are, with e_i = b_i (v_i - (Diag(g_i) S_{i-1})^T k_i),
      //   (I + A) E = diag(b) (V - Kq S0),   A_ij = b_i kq_i . kd_j  (j < i)
      //   S_n = Diag(Gamma_n) (S0 + Kd^T E)
      // (the unrolled recurrence; a WY-style chunk).  Kq S0 and Kd^T E run on
      // the matrix cores in the state's register layout; the n x n system is
      // solved by forward substitution, one column per thread.  Tiles whose
      // Gamma underflows (tiny gates) and single entries take the serial
      // path below.
      float* s_kq = smem + LY::KQ;
      float* s_kd = smem + LY::KD;
      float* s_A = smem + LY::AM;
      float* s_gf = smem + LY::GF;
      constexpr int AS = WMAX + 1;
      bool chunked = false;
      if (LY::CHUNK && n >= 4) {                     // uniform
        int small = 0;
        for (int m = tid; m < DK; m += NT) {
          float G = 1.f;
          for (int i = 0; i < WMAX; ++i) {
            float kq = 0.f, kd = 0.f;
            if (i < n) {
              G *= (FAM == FAM_GDN) ? s_a[i] : s_k[(WMAX + i) * DK + m];
              const float k = s_k[i * DK + m];
              kq = k * G;
              kd = k / G;
            }
            s_kq[m * KWS + i] = kq;
            s_kd[m * KWS + i] = kd;
          }
          s_gf[m] = G;
          small |= !(G >= 1e-30f) ? 1 : 0;         // also catches NaN
        }
        chunked = !__syncthreads_or(small);
      }
      if (chunked) {
        constexpr int NE = cdiv(WMAX, 16);           // 16-entry blocks
        // X^T = S0^T Kq^T: lane (cg, rg) gets X[16 t + cg][NCC (4 rg + vv) + c]
        f32x4v xacc[NE][NCC];
#pragma unroll
        for (int t = 0; t < NE; ++t)
#pragma unroll
          for (int c = 0; c < NCC; ++c) xacc[t][c] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NE; ++t) {
          if (16 * t < n) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float bq = s_kq[(16 * mb + 4 * rg + v) * KWS + 16 * t + cg];
#pragma unroll
                for (int c = 0; c < NCC; ++c) xacc[t][c] = mfma16x4(sacc[mb][c][v], bq, xacc[t][c]);
              }
          }
        }
        // A (wave 0): D[i][j] = kq_i . kd_j over 16 x 16 blocks, lower part kept
        if (wv == 0) {
#pragma unroll
          for (int it = 0; it < NE; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
              if (16 * it < n) {
                f32x4v a = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
                for (int ks = 0; ks < DK / 4; ++ks)
                  a = mfma16x4(s_kq[(4 * ks + rg) * KWS + 16 * it + cg],
                               s_kd[(4 * ks + rg) * KWS + 16 * jt + cg], a);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  const int i = 16 * it + 4 * rg + v, j = 16 * jt + cg;
                  s_A[i * AS + j] = (j < i && i < n) ? s_w[i] * a[v] : 0.f;
                }
              }
            }
        }
        // R = diag(b) (V - X), in place over the values
#pragma unroll
        for (int t = 0; t < NE; ++t) {
          const int i = 16 * t + cg;
          if (i < n) {
            const float be = s_w[i];
#pragma unroll
            for (int vv = 0; vv < 4; ++vv)
#pragma unroll
              for (int c = 0; c < NCC; ++c) {
                float* x = s_v + i * DV + wv * CB + NCC * (4 * rg + vv) + c;
                *x = be * (*x - xacc[t][c][vv]);
              }
          }
        }
        __syncthreads();
        // forward substitution, one column per thread: E overwrites R; the
        // padding rows up to a multiple of four become zero
        if (tid < DV) {
          float e[WMAX];
#pragma unroll
          for (int i = 0; i < WMAX; ++i) {
            if (i < n) {
              float x = s_v[i * DV + tid];
#pragma unroll
              for (int j = 0; j < i; ++j) x -= s_A[i * AS + j] * e[j];
              e[i] = x;
              s_v[i * DV + tid] = x;
            } else if (i < round4(n)) {
              s_v[i * DV + tid] = 0.f;
            }
          }
        }
        __syncthreads();
        // S0 + Kd^T E on the matrix cores, then the row scaling Diag(Gamma_n)
        for (int t4 = 0; t4 < n; t4 += 4) {
          float bv[NCC];
          ldn<NCC>(s_v + (t4 + rg) * DV + colbase, bv);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const float ak = s_kd[(16 * mb + cg) * KWS + t4 + rg];
#pragma unroll
            for (int c = 0; c < NCC; ++c) sacc[mb][c] = mfma16x4(ak, bv[c], sacc[mb][c]);
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float4 g4 = *reinterpret_cast<const float4*>(s_gf + 16 * mb + 4 * rg);
          const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
          for (int c = 0; c < NCC; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) sacc[mb][c][v] *= gv[v];
        }
      }
      // serial form: one entry at a time
      for (int i = 0; !chunked && i < n; ++i) {
        float kk[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float4 k4 = *reinterpret_cast<const float4*>(s_k + i * DK + 16 * mb + 4 * rg);
          kk[mb][0] = k4.x; kk[mb][1] = k4.y; kk[mb][2] = k4.z; kk[mb][3] = k4.w;
        }
        if (FAM == FAM_KDA) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const float4 g4 = *reinterpret_cast<const float4*>(s_k + (WMAX + i) * DK + 16 * mb + 4 * rg);
            const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int c = 0; c < NCC; ++c)
#pragma unroll
              for (int v = 0; v < 4; ++v) sacc[mb][c][v] *= gv[v];
          }
        }
        float u[NCC];
#pragma unroll
        for (int c = 0; c < NCC; ++c) {
          float a = 0.f;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 4; ++v) a += sacc[mb][c][v] * kk[mb][v];
          u[c] = xsum<4, 2>(a);                      // over the four row groups
        }
        float vvv[NCC];
        ldn<NCC>(s_v + i * DV + colbase, vvv);
        const float beta = s_w[i];
        float dl[NCC];
        if (FAM == FAM_GDN) {
          const float al = s_a[i];
#pragma unroll
          for (int c = 0; c < NCC; ++c) dl[c] = beta * (vvv[c] - al * u[c]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int c = 0; c < NCC; ++c)
#pragma unroll
              for (int v = 0; v < 4; ++v) sacc[mb][c][v] = al * sacc[mb][c][v] + kk[mb][v] * dl[c];
        } else {
#pragma unroll
          for (int c = 0; c < NCC; ++c) dl[c] = beta * (vvv[c] - u[c]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int c = 0; c < NCC; ++c)
#pragma unroll
              for (int v = 0; v < 4; ++v) sacc[mb][c][v] += kk[mb][v] * dl[c];
        }
      }
    }

    // ------------------------------------------ exact output S^T q
    if (want_out) {
      float acc[NCC];
#pragma unroll
      for (int c = 0; c < NCC; ++c) acc[c] = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const float4 q4 = *reinterpret_cast<const float4*>(s_q + 16 * mb + 4 * rg);
        const float qq[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int c = 0; c < NCC; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[c] += sacc[mb][c][v] * qq[v];
      }
      // NCC columns over the four row groups: halve over the top lane bits
      constexpr int NBH = ilog2(NCC);
      tr_reduce<NCC, 4 + 2 - NBH, NBH>(acc, lane);
      out_val = xsum<4, 2 - NBH>(acc[0]);
      out_c = (lane >> (6 - NBH)) & (NCC - 1);
      out_writer = ((lane >> 4) & ((1 << (2 - NBH)) - 1)) == 0;
    }
  } else {
    // ----------------------- ReplaySSM non-flush: exact S0^T q~ + o_buf
    if (FAM == FAM_M2) {
      // q~ = D q ; buffered term sum_i (k_i . q) (w_i v_i): wave 0 forms the
      // n dot products as DPP wave sums over the key elements
      if (wv == 0) {
        constexpr int EK = DK >= 64 ? DK / 64 : 1;
        float qq[EK];
#pragma unroll
        for (int e = 0; e < EK; ++e) {
          const int m = lane * EK + e;
          qq[e] = m < DK ? s_q[m] : 0.f;
        }
        for (int i = 0; i < n; ++i) {            // uniform
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < EK; ++e) {
            const int m = lane * EK + e;
            if (m < DK) d += s_k[m * KWS + i] * qq[e];
          }
          d = wave_sum(d);
          if (lane == 0) s_e[i] = d;
        }
      }
      const float D = s_misc[0];
      for (int m = tid; m < DK; m += NT) s_qt[m] = D * s_q[m];
    } else if (wv == 0) {
      // serial pull-back, newest entry first: d = k_i . r ; e_i = beta_i d ;
      // r <- alpha (r - beta d k) (GDN) or g (.) (r - beta d k) (KDA)
      constexpr int EK = DK >= 64 ? DK / 64 : 1;
      float r[EK];
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const int m = lane * EK + e;
        r[e] = (m < DK) ? s_q[m] : 0.f;
      }
      for (int t = 0; t < n; ++t) {
        const int i = n - 1 - t;
        float kk[EK];
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
          const int m = lane * EK + e;
          kk[e] = (m < DK) ? s_k[i * DK + m] : 0.f;
          d += kk[e] * r[e];
        }
        d = wave_sum(d);
        const float beta = s_w[i];
        if (lane == 0) s_e[i] = beta * d;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
          const int m = lane * EK + e;
          const float dec = (FAM == FAM_GDN) ? s_a[i] : ((m < DK) ? s_k[(WMAX + i) * DK + m] : 0.f);
          r[e] = dec * (r[e] - beta * d * kk[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        const int m = lane * EK + e;
        if (m < DK) s_qt[m] = r[e];
      }
    }
    __syncthreads();
    float acc[NCC];
#pragma unroll
    for (int c = 0; c < NCC; ++c) acc[c] = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const float4 q4 = *reinterpret_cast<const float4*>(s_qt + 16 * mb + 4 * rg);
      const float qq[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
      for (int c = 0; c < NCC; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[c] += sacc[mb][c][v] * qq[v];
    }
    constexpr int NBH = ilog2(NCC);
    tr_reduce<NCC, 4 + 2 - NBH, NBH>(acc, lane);
    const float vsum = xsum<4, 2 - NBH>(acc[0]);
    out_c = (lane >> (6 - NBH)) & (NCC - 1);
    out_writer = ((lane >> 4) & ((1 << (2 - NBH)) - 1)) == 0;
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
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x[NCC];
#pragma unroll
        for (int c = 0; c < NCC; ++c) x[c] = sacc[mb][c][v];
        if constexpr (SBUF)
          buf_st<NCC, S_CP>(s_rsrc, s_lane, (16 * mb + v) * DV * 4, x);
        else if constexpr (S_CP == CP_NT)
          stn_nt<NCC>(p.S + bh * DK * DV + colbase + (size_t)(16 * mb + 4 * rg + v) * DV, x);
        else
          stn<NCC>(p.S + bh * DK * DV + colbase + (size_t)(16 * mb + 4 * rg + v) * DV, x);
      }

    // ------------- dense-fallback head (rank 0): the state copy instead
    // Each wave holds only its column block of a row, so direct stores
    // would write every row in partial lines from several waves (measured:
    // far below the bandwidth of the rest of the flush).  The copy goes
    // through LDS in bands of RCH rows and leaves as whole rows, 16 bytes a
    // lane.
    // (compiled only for layers that have such heads: the branch costs the
    // kernel registers)
    if (DENSE && want_u && r == 0) {               // uniform over the workgroup
      constexpr int RB = DV * (int)sizeof(UT);     // bytes per row of the copy
      constexpr int FIT = LY::TOTAL * 4 / RB;      // rows that fit in the LDS
      constexpr int RCH = FIT >= 64 && DK >= 64 ? 64 : FIT >= 32 && DK >= 32 ? 32 : 16;
      static_assert(RCH <= DK && DK % RCH == 0 && RCH * RB <= LY::TOTAL * 4, "copy bands fit the LDS");
      static_assert(NCC == 2 && RB % 16 == 0, "the copy is written as pairs and 16-byte chunks");
      char* s_cp = reinterpret_cast<char*>(smem);
      UT* Cg = reinterpret_cast<UT*>(p.Sc) + ((size_t)b * p.ndense + dense_slot(p, h)) * DK * DV;
      __syncthreads();                             // the LDS is no longer read
#pragma unroll
      for (int m0 = 0; m0 < DK; m0 += RCH) {
#pragma unroll
        for (int mb = m0 / 16; mb < (m0 + RCH) / 16; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            UT* dst = reinterpret_cast<UT*>(s_cp + (16 * mb + 4 * rg + v - m0) * RB) + colbase;
            dst[0] = Store<UT>::cvt(sacc[mb][0][v]);
            dst[1] = Store<UT>::cvt(sacc[mb][1][v]);
          }
        __syncthreads();
        uint4* gdst = reinterpret_cast<uint4*>(Cg + (size_t)m0 * DV);
        const uint4* lsrc = reinterpret_cast<const uint4*>(s_cp);
        for (int c = tid; c < RCH * RB / 16; c += NT) gdst[c] = lsrc[c];
        __syncthreads();
      }
    }
    // --------------------------- sketch U = S^T P on the matrix cores
    if (want_u && (!DENSE || r > 0)) {
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
      __syncthreads();      // keys no longer needed: basis [m][j] over them, rows j >= r zero
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const int c = tid + NT * u;
        if (c < 16 * PCPR) {
          const int j = c / PCPR, m0 = (c - j * PCPR) * 4;
          const float x[4] = {pr[u].x, pr[u].y, pr[u].z, pr[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) s_p[(m0 + e) * PS + j] = x[e];
        }
      }
      __syncthreads();
      // column block c: D[i][j] = sum_m S[m][NCC i + c] P[m][j], K-steps (mb, v)
      f32x4v u[NCC];
#pragma unroll
      for (int c = 0; c < NCC; ++c) u[c] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float bp = s_p[(16 * mb + 4 * rg + v) * PS + cg];
#pragma unroll
          for (int c = 0; c < NCC; ++c) u[c] = mfma16x4(sacc[mb][c][v], bp, u[c]);
        }
      // lane holds u_j, j = cg, at columns NCC (4 rg + vv) + c of its block
      if (cg < r) {
        UT* Ub = reinterpret_cast<UT*>(p.U) + ((size_t)b * p.R + off + cg) * DV + wv * CB + NCC * 4 * rg;
        float x[4 * NCC];
#pragma unroll
        for (int vv = 0; vv < 4; ++vv)
#pragma unroll
          for (int c = 0; c < NCC; ++c) x[NCC * vv + c] = u[c][vv];
        if constexpr (NCC == 4) {
          float x0[8], x1[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) { x0[e] = x[e]; x1[e] = x[8 + e]; }
          stn<8>(Ub, x0);
          stn<8>(Ub + 8, x1);
        } else if constexpr (sizeof(UT) == 2) {
          // eight bf16 sketch values as one 16-byte store (measured: flush
          // 482 -> 476 us at m2_b320 against two 8-byte stores)
          uint4 w;
          w.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
          w.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
          w.z = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
          w.w = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
          *reinterpret_cast<uint4*>(Ub) = w;
        } else {
          stn<8>(Ub, x);
        }
      }
      if constexpr (COEF) coef_map<DK, DV, UT, LY>(p, smem, sacc, u, b, off, r);
    }
  }

  // ------------------------------------------------------ ring count
  if (MODE != MODE_FULL) {
    __syncthreads();       // every wave has read the count
    if (tid == 0) p.count[bh] = do_flush ? 0 : n;
  }
}

}  // namespace sk
