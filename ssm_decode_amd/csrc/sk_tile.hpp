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

// Which tile kernels address the state through a buffer resource (one lane
// offset and immediate row offsets) rather than a 64-bit address per row:
// the flushes, where the per-row addresses of the state stores would hold
// 64 VGPRs (the Mamba-2 flush: 98 VGPRs instead of 162, the looping flush
// over a due list 149 instead of 214).
template <int FAM, int MODE>
struct STATE_BUFFER {
  static constexpr bool value = MODE == MODE_FLUSH;
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

// One tile (b, h) of the flush over a device-side list of due tiles, called
// in a loop; n0_known >= 0: the tile's ring fill is already known, else it
// is read here.
template <int FAM, int DK, int DV, typename AT, typename UT, int MODE, int WMAX, int COEF, bool DENSE>
__device__ __forceinline__ void tile_body(const Params& p, const int b, const int h, const int n0_known) {
#define SK_TILE_BODY_IN_LOOP
#include "sk_tile_body.inc"
#undef SK_TILE_BODY_IN_LOOP
}

// One workgroup of 1024 threads lists the sequences whose ring is full
// (head 0's count == W: every head of a sequence advances together), in
// sequence order: per chunk of 1024 sequences, a ballot per wave, the
// waves' totals through LDS, then every due sequence's position.  Head 0
// counts outside [0, W] are reported (SKSSM_ERRBIT_COUNT).
constexpr int DUE_SCAN_THREADS = 1024;

template <int UNUSED = 0>
__global__ void __launch_bounds__(DUE_SCAN_THREADS) due_scan_kernel(Params p) {
  constexpr int NW = DUE_SCAN_THREADS / 64;
  __shared__ int s_wave[NW];
  __shared__ int s_base;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int* cnt = p.due_work;
  int* lst = p.due_work + DueWork(p.B).list;
  if (tid == 0) s_base = 0;
  int bad = 0;
  for (int b0 = 0; b0 < p.B; b0 += DUE_SCAN_THREADS) {      // uniform
    const int b = b0 + tid;
    const int c = b < p.B ? p.count[(size_t)b * p.H] : 0;
    bad |= (c < 0 || c > p.W) ? ERRBIT_COUNT : 0;
    const bool due = b < p.B && c == p.W;
    const uint64_t m = __builtin_amdgcn_ballot_w64(due);
    if (lane == 0) s_wave[wv] = __popcll(m);
    __syncthreads();
    int before = s_base;                                      // due sequences of earlier waves
    for (int w = 0; w < wv; ++w) before += s_wave[w];
    if (due) lst[before + __popcll(m & ((1ull << lane) - 1ull))] = b;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int w = 0; w < NW; ++w) t += s_wave[w];
      s_base += t;
    }
    __syncthreads();
  }
  if (tid == 0) cnt[0] = s_base;
  if (bad) atomicOr(p.err, bad);
}

// (the delta-rule flush runs three waves per SIMD: its chunked update has
// serial phases that more resident tiles hide)
// LISTED: the flush over the device-side list of due sequences written by
// due_scan_kernel: workgroup g takes tiles g, g + gridDim.x, ... of the
// listed sequences (tile it = list position * H + head), so that a short
// list costs a workgroup per tile and a long one (an aligned phase) is
// taken by the same grid in turn.  Its own instantiation: the loop keeps
// more values live across the body than the one-tile kernels.
template <int FAM, int DK, int DV, typename AT, typename UT, int MODE, int WMAX, int COEF, bool DENSE,
          bool LISTED = false>
__global__ void __launch_bounds__((TileShape<DK, DV>::THREADS),
                                  (MODE == MODE_FLUSH && FAM != FAM_M2 && !LISTED ? 3 : 2))
tile_kernel(Params p) {
  if constexpr (LISTED) {
    const size_t end = (size_t)p.seq_count[0] * p.H;
    for (size_t it = blockIdx.x; it < end; it += gridDim.x) {   // uniform
      const int b = p.seq_list[it / p.H];
      tile_body<FAM, DK, DV, AT, UT, MODE, WMAX, COEF, DENSE>(p, b, (int)(it % p.H), -1);
    }
  } else {
    const int ts = blockIdx.x / p.H;
    const int h = blockIdx.x - ts * p.H;
    int b = ts, n0k = -1;
    if constexpr (MODE == MODE_FLUSH) {
     if (p.seq_list) {                           // uniform: the tiles of listed sequences
      b = p.seq_list[ts];
      if (b < 0 || b >= p.B) {
        if (threadIdx.x == 0) atomicOr(p.err, ERRBIT_SEQ);
        return;
      }
      // claim the tile (count W -> W + 1; the flush stores 0 at its end), so
      // that a sequence listed twice is flushed once: a second claim while
      // the first flush runs fails and reports ERRBIT_SEQ; a count outside
      // [0, W] is ERRBIT_COUNT
      __shared__ int s_claim;
      if (threadIdx.x == 0) s_claim = atomicCAS(p.count + (size_t)b * p.H + h, p.W, p.W + 1);
      __syncthreads();
      const int old = s_claim;
      if (old != p.W) {
        if (threadIdx.x == 0 && (old < 0 || old > p.W))
          atomicOr(p.err, old == p.W + 1 ? ERRBIT_SEQ : ERRBIT_COUNT);
        return;
      }
      n0k = p.W;
     }
    }
    {
      const int n0_known = n0k;
#include "sk_tile_body.inc"
    }
  }
}

}  // namespace sk
