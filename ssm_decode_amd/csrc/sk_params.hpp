// Kernel argument block shared by the launchers and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

enum Family { FAM_M2 = 0, FAM_GDN = 1, FAM_KDA = 2 };
enum Mode { MODE_FLUSH = 0, MODE_FULL = 1, MODE_REPLAY = 2, MODE_READ = 3 };
enum Dtype { DT_F32 = 0, DT_BF16 = 1 };
enum ErrBit { ERRBIT_COUNT = 1, ERRBIT_GROUP = 2, ERRBIT_SEQ = 4 };

constexpr int DENSE_LIST_MAX = 64;   // dense-fallback heads listed in the kernel arguments

struct Params {
  int B, H, G, HPG, W, R;
  int flush_all;        // MODE_FLUSH: flush every tile, not only full rings
  int flush_close;      // MODE_FLUSH: the step's own entry (k, v, gate, beta) closes
                        // the window of tiles whose ring holds W - 1 entries
  const int32_t* seq_list;  // MODE_FLUSH: device list of nseq sequences to flush, or null (all)
  int nseq;
  const int32_t* seq_count;  // MODE_FLUSH, device-side due list: the list's length (device), or null
  int* due_work;        // the due list's workspace (scan launch: the sequences whose ring is full)
  float* S;
  void* U;
  const float* Pt;
  const float* C;
  const int32_t* off;   // [H+1] device rank offsets
  void* rk;
  void* rv;
  void* rg;
  float* rb;
  int32_t* count;
  const float* A;
  int32_t* err;
  void* work;           // workspace (Mamba-2 read: M2Work; GDN/KDA read with dense heads: DnWork)
  void* Cs;             // state-dependent coefficient maps [B][R][dk] sketch dtype
  void* Sc;             // state copies of dense-fallback heads [B][H][dk][dv] sketch dtype
  int ndense;           // dense-fallback heads, in head order in dense_list; their state
  int16_t dense_list[DENSE_LIST_MAX];  // copies are Sc[b][position in the list]
  float ridge;          // relative ridge of the state-dependent map
  int pullback;         // GDN/KDA read: 0 serial effective query, 1 the triangular-system form,
                        // 2 that form with projected per-slot factors
  float* rpc;           // pullback 2: the ring's projected factors [B][H][W][16] fp32
  const void* q;
  const void* k;
  const void* v;
  const void* gate;
  const float* beta;
  void* o;
};

// Workspace layout (floats): cq [B][R], then d [B][G][W], then n0 [B][G]
// (int32), each region 256-byte aligned.
struct M2Work {
  size_t d, n0, total;
  __host__ __device__ M2Work(int B, int R, int G, int W) {
    const size_t cq = ((size_t)B * R + 63) / 64 * 64;
    d = cq;
    n0 = d + ((size_t)B * G * W + 63) / 64 * 64;
    total = n0 + ((size_t)B * G + 63) / 64 * 64;
  }
};

// Workspace of a GDN/KDA read with dense-fallback heads (floats): per
// (sequence, dense head) the pulled-back query r [B][D][DK], the buffered
// term [B][D][DV] and a flag [B][D] (int32, 1 when the step has an output),
// each region 256-byte aligned.
struct DnWork {
  size_t r, ob, flag, total;
  __host__ __device__ DnWork(int B, int D, int DK, int DV) {
    r = 0;
    ob = ((size_t)B * D * DK + 63) / 64 * 64;
    flag = ob + ((size_t)B * D * DV + 63) / 64 * 64;
    total = flag + ((size_t)B * D + 63) / 64 * 64;
  }
};

// Due sequences listed on the device for a flush (SKSSM_FLUSH_DUE_SCAN):
// the number of them, then the list (int32 offsets in the workspace).
struct DueWork {
  size_t cnt, list, total;
  __host__ __device__ explicit DueWork(int B) {
    cnt = 0;
    list = 64;
    total = list + ((size_t)B + 63) / 64 * 64;
  }
};
// Sequences whose tiles the scan flush's grid covers one workgroup each:
// twice the expected number of due sequences under a uniformly ragged phase,
// plus a margin; the grid takes the tiles of any further listed sequences in
// turn.
__host__ __device__ inline int due_slots(int B, int W) {
  const int s = 2 * ((B + W - 1) / W) + 8;
  return s < B ? s : B;
}

// Position of dense-fallback head h in the list (h must be listed).
__host__ __device__ inline int dense_slot(const Params& p, int h) {
  int k = 0;
  while (k + 1 < p.ndense && p.dense_list[k] != h) ++k;
  return k;
}

// Launch one kernel of `family` for `mode`; returns 0, or -2 when the shape
// / dtype combination has no instantiation, or -5 on a launch error.
// coef: 0 the fixed per-head map, 1 the state-dependent map.
int launch_m2(int mode, int coef, int dk, int dv, int act, int sketch, const Params& p, hipStream_t st);
int launch_gdn(int mode, int coef, int dk, int dv, int act, int sketch, const Params& p, hipStream_t st);
int launch_kda(int mode, int coef, int dk, int dv, int act, int sketch, const Params& p, hipStream_t st);

}  // namespace sk
