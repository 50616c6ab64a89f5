// C ABI of the SketchSSM decode library: host-side validation and dispatch.
// Every check runs before any HIP call, so an invalid call launches nothing
// and writes nothing.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "sketchssm.h"
#include "sk_params.hpp"

namespace sk {
int noalloc_scratch(void** out);   // sk_noalloc.hip
}

namespace {

constexpr int kMaxW = 32;
constexpr int kMaxRank = 16;
constexpr int kMaxHeadsPerGroup = 16;

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool shape_supported(int dk, int dv) {
  return (dk == 16 && dv == 32) || (dk == 64 && dv == 64) || (dk == 128 && dv == 64) ||
         (dk == 128 && dv == 128);
}

// What a call needs from the buffers and the step.
struct Needs {
  bool S, U, Pt, C, ring, count, step_in, step_q, step_o, work;
  bool Cstate;   // writes (flush) or reads (read) the state-dependent maps
                 // and the state copies of dense-fallback heads
};

bool any_dense(const sketchssm_layer* L) {
  for (int h = 0; h < L->heads; ++h)
    if (L->rank_offsets_host[h + 1] == L->rank_offsets_host[h]) return true;
  return false;
}

// Workspace of a read (layouts in sk_params.hpp).  Mamba-2: the query in
// every head's basis, the key-query dot products and the checked ring fill.
// GDN/KDA: only with dense-fallback heads, the pulled-back query and the
// buffered term of each such tile, for the launch that reads the copies.
int64_t read_work_bytes(const sketchssm_layer* L) {
  if (L->family != SKSSM_MAMBA2) {
    int nd = 0;
    for (int h = 0; h < L->heads; ++h) nd += L->rank_offsets_host[h + 1] == L->rank_offsets_host[h];
    if (nd == 0) return 0;
    const sk::DnWork w(L->batch, nd, L->dk, L->dv);
    return (int64_t)w.total * 4;
  }
  const sk::M2Work w(L->batch, L->rank_offsets_host[L->heads], L->qk_groups, L->window);
  return (int64_t)w.total * 4;
}

// Workspace of a flush with SKSSM_FLUSH_DUE_SCAN: the number of due
// sequences, then their list (sk_params.hpp, DueWork).
int64_t scan_work_bytes(const sketchssm_layer* L) {
  if (L->batch == 0) return 0;
  return (int64_t)sk::DueWork(L->batch).total * 4;
}

// One workspace serves both: a call uses it only within itself, and calls on
// one layer are ordered.
int64_t workspace_bytes(const sketchssm_layer* L) {
  const int64_t r = read_work_bytes(L), f = scan_work_bytes(L);
  return r > f ? r : f;
}

int check_layer(const sketchssm_layer* L) {
  if (!L) return SKSSM_EINVAL;
  if (L->family < SKSSM_MAMBA2 || L->family > SKSSM_KDA) return SKSSM_EDIM;
  if (L->act_dtype < SKSSM_F32 || L->act_dtype > SKSSM_BF16) return SKSSM_EDTYPE;
  if (L->sketch_dtype < SKSSM_F32 || L->sketch_dtype > SKSSM_BF16) return SKSSM_EDTYPE;
  if (L->act_dtype != L->sketch_dtype) return SKSSM_EDTYPE;   // (f32, f32) or (bf16, bf16)
  if (L->batch < 0 || L->heads < 1 || L->qk_groups < 1) return SKSSM_EDIM;
  if (L->heads % L->qk_groups != 0) return SKSSM_EDIM;
  if (L->family == SKSSM_MAMBA2) {
    if (L->heads / L->qk_groups > kMaxHeadsPerGroup) return SKSSM_EDIM;
  } else if (L->qk_groups != L->heads) {
    return SKSSM_EDIM;
  }
  if (!shape_supported(L->dk, L->dv)) return SKSSM_EDIM;
  if (L->coef_map != SKSSM_COEF_FIXED && L->coef_map != SKSSM_COEF_STATE) return SKSSM_EFLAG;
  if (L->pullback != SKSSM_PULLBACK_SERIAL && L->pullback != SKSSM_PULLBACK_WY &&
      L->pullback != SKSSM_PULLBACK_PROJ)
    return SKSSM_EFLAG;
  if (L->coef_map == SKSSM_COEF_STATE && !(isfinite(L->coef_ridge) && L->coef_ridge > 0.f))
    return SKSSM_EINVAL;
  if (L->window < 1 || L->window > kMaxW) return SKSSM_EDIM;
  if ((int64_t)L->batch * L->heads > INT32_MAX / 2) return SKSSM_EDIM;
  if (!L->rank_offsets_host) return SKSSM_EINVAL;
  const int32_t* off = L->rank_offsets_host;
  if (off[0] != 0) return SKSSM_EDIM;
  const int rmax = L->dk < kMaxRank ? L->dk : kMaxRank;
  int ndense = 0;
  for (int h = 0; h < L->heads; ++h) {
    const int r = off[h + 1] - off[h];
    if (r < 0 || r > rmax) return SKSSM_EDIM;           // r = 0: dense fallback
    ndense += r == 0;
  }
  if (ndense > sk::DENSE_LIST_MAX) return SKSSM_EDIM;
  return SKSSM_OK;
}

int check_buffers(const sketchssm_layer* L, const sketchssm_buffers* B, const sketchssm_step* S,
                  const Needs& nd) {
  if (!B) return SKSSM_EINVAL;
  const bool rows = L->rank_offsets_host[L->heads] > 0;   // some head is sketched
  if (nd.S && !aligned16(B->S)) return SKSSM_EINVAL;
  if (nd.U && rows && !aligned16(B->U)) return SKSSM_EINVAL;
  if (nd.Pt && rows && !aligned16(B->Pt)) return SKSSM_EINVAL;
  const bool state_map = L->coef_map == SKSSM_COEF_STATE;
  if (nd.C && rows && !state_map && !aligned16(B->C)) return SKSSM_EINVAL;
  if (nd.Cstate && rows && state_map && !aligned16(B->Cstate)) return SKSSM_EINVAL;
  if (nd.Cstate && any_dense(L) && !aligned16(B->Scopy)) return SKSSM_EINVAL;
  if ((nd.U || nd.Pt || nd.C) && !aligned16(B->rank_offsets)) return SKSSM_EINVAL;
  if (nd.ring) {
    if (!aligned16(B->ring_k) || !aligned16(B->ring_v) || !aligned16(B->ring_gate)) return SKSSM_EINVAL;
    if (L->family != SKSSM_MAMBA2 && !aligned16(B->ring_beta)) return SKSSM_EINVAL;
  }
  // the projected factors: read and appended by the GDN/KDA read
  if (nd.C && nd.ring && L->family != SKSSM_MAMBA2 && L->pullback == SKSSM_PULLBACK_PROJ &&
      rows && !aligned16(B->ring_pc))
    return SKSSM_EINVAL;
  if (nd.count && (!aligned16(B->count) || !aligned16(B->err))) return SKSSM_EINVAL;
  if (L->family == SKSSM_MAMBA2 && !aligned16(B->A)) return SKSSM_EINVAL;
  if (nd.work && read_work_bytes(L) > 0 && !aligned16(B->work)) return SKSSM_EINVAL;
  if (nd.step_in || nd.step_q || nd.step_o) {
    if (!S) return SKSSM_EINVAL;
    if (nd.step_in) {
      if (!aligned16(S->k) || !aligned16(S->v) || !aligned16(S->gate)) return SKSSM_EINVAL;
      if (L->family != SKSSM_MAMBA2 && !aligned16(S->beta)) return SKSSM_EINVAL;
    }
    if (nd.step_q && !aligned16(S->q)) return SKSSM_EINVAL;
    if (nd.step_o && !aligned16(S->o)) return SKSSM_EINVAL;
  }
  return SKSSM_OK;
}

sk::Params make_params(const sketchssm_layer* L, const sketchssm_buffers* B, const sketchssm_step* S) {
  sk::Params p{};
  p.B = L->batch;
  p.H = L->heads;
  p.G = L->qk_groups;
  p.HPG = L->heads / L->qk_groups;
  p.W = L->window;
  p.R = L->rank_offsets_host[L->heads];
  p.S = B->S;
  p.U = B->U;
  p.Pt = B->Pt;
  p.C = B->C;
  p.off = B->rank_offsets;
  p.rk = B->ring_k;
  p.rv = B->ring_v;
  p.rg = B->ring_gate;
  p.rb = B->ring_beta;
  p.count = B->count;
  p.A = B->A;
  p.err = B->err;
  p.work = B->work;
  p.Cs = B->Cstate;
  p.Sc = B->Scopy;
  // dense-fallback heads (r_h = 0), listed for the kernels that take only them
  int nd = 0;                          // (at most DENSE_LIST_MAX: check_layer)
  for (int h = 0; h < L->heads; ++h)
    if (L->rank_offsets_host[h + 1] == L->rank_offsets_host[h]) p.dense_list[nd++] = (int16_t)h;
  p.ndense = nd;
  p.ridge = L->coef_ridge;
  p.pullback = L->pullback;
  p.rpc = B->ring_pc;
  if (S) {
    p.q = S->q;
    p.k = S->k;
    p.v = S->v;
    p.gate = S->gate;
    p.beta = S->beta;
    p.o = S->o;
  }
  return p;
}

int dispatch(const sketchssm_layer* L, int mode, const sk::Params& p, void* stream) {
  if (L->batch == 0) return SKSSM_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the state-dependent map changes only the flush and the read
  const int coef = (L->coef_map == SKSSM_COEF_STATE && (mode == sk::MODE_FLUSH || mode == sk::MODE_READ)) ? 1 : 0;
  int rc;
  switch (L->family) {
    case SKSSM_MAMBA2: rc = sk::launch_m2(mode, coef, L->dk, L->dv, L->act_dtype, L->sketch_dtype, p, st); break;
    case SKSSM_GDN: rc = sk::launch_gdn(mode, coef, L->dk, L->dv, L->act_dtype, L->sketch_dtype, p, st); break;
    default: rc = sk::launch_kda(mode, coef, L->dk, L->dv, L->act_dtype, L->sketch_dtype, p, st); break;
  }
  return rc;
}

}  // namespace

extern "C" {

int sketchssm_read(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                   const sketchssm_step* step, void* hip_stream) {
  try {
    int rc = check_layer(layer);
    if (rc) return rc;
    const Needs nd{false, true, false, true, true, true, true, true, true, true, true};
    if ((rc = check_buffers(layer, bufs, step, nd))) return rc;
    return dispatch(layer, sk::MODE_READ, make_params(layer, bufs, step), hip_stream);
  } catch (...) {
    return SKSSM_ELAUNCH;
  }
}

int sketchssm_read_noalloc(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                           const sketchssm_step* step, void* hip_stream) {
  try {
    int rc = check_layer(layer);
    if (rc) return rc;
    const int64_t need = read_work_bytes(layer);
    if (need > (int64_t)SKSSM_NOALLOC_SCRATCH_BYTES) return SKSSM_ESCRATCH;
    // (bufs->work is not used: the workspace is the library's scratch array)
    const Needs nd{false, true, false, true, true, true, true, true, true, false, true};
    if ((rc = check_buffers(layer, bufs, step, nd))) return rc;
    sk::Params p = make_params(layer, bufs, step);
    p.work = nullptr;
    if (need > 0 && layer->batch > 0) {
      void* scratch = nullptr;
      if ((rc = sk::noalloc_scratch(&scratch))) return rc;
      p.work = scratch;
    }
    return dispatch(layer, sk::MODE_READ, p, hip_stream);
  } catch (...) {
    return SKSSM_ELAUNCH;
  }
}

int sketchssm_flush(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                    const sketchssm_step* step, int32_t flags, void* hip_stream) {
  try {
    int rc = check_layer(layer);
    if (rc) return rc;
    if (flags != SKSSM_FLUSH_DUE && flags != SKSSM_FLUSH_ALL && flags != SKSSM_FLUSH_DUE_SCAN &&
        flags != SKSSM_FLUSH_CLOSE)
      return SKSSM_EFLAG;
    const bool close = flags == SKSSM_FLUSH_CLOSE;
    if (close && !step) return SKSSM_EINVAL;     // the step's entry and output are required
    const bool out = step != nullptr;
    const Needs nd{true, true, true, false, true, true, close, out, out, false, true};
    if ((rc = check_buffers(layer, bufs, step, nd))) return rc;
    const bool scan = flags == SKSSM_FLUSH_DUE_SCAN;
    if (scan && layer->batch > 0 && !aligned16(bufs->work)) return SKSSM_EINVAL;
    sk::Params p = make_params(layer, bufs, step);
    p.flush_all = flags == SKSSM_FLUSH_ALL;
    p.flush_close = close;
    if (scan && layer->batch > 0) {
      p.due_work = static_cast<int*>(bufs->work);
      p.seq_count = p.due_work + sk::DueWork(layer->batch).cnt;
      p.seq_list = p.due_work + sk::DueWork(layer->batch).list;
      p.nseq = sk::due_slots(layer->batch, layer->window);
    }
    if (!out) {
      p.q = nullptr;
      p.o = nullptr;
    }
    return dispatch(layer, sk::MODE_FLUSH, p, hip_stream);
  } catch (...) {
    return SKSSM_ELAUNCH;
  }
}

int sketchssm_flush_seqs(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                         const sketchssm_step* step, const int32_t* seqs, int32_t nseq, void* hip_stream) {
  try {
    int rc = check_layer(layer);
    if (rc) return rc;
    if (nseq < 0 || nseq > layer->batch) return SKSSM_EDIM;
    if (nseq > 0 && (!seqs || (reinterpret_cast<uintptr_t>(seqs) & 3))) return SKSSM_EINVAL;
    const bool out = step != nullptr;
    const Needs nd{true, true, true, false, true, true, false, out, out, false, true};
    if ((rc = check_buffers(layer, bufs, step, nd))) return rc;
    if (nseq == 0) return SKSSM_OK;
    sk::Params p = make_params(layer, bufs, step);
    p.seq_list = seqs;
    p.nseq = nseq;
    if (!out) {
      p.q = nullptr;
      p.o = nullptr;
    }
    return dispatch(layer, sk::MODE_FLUSH, p, hip_stream);
  } catch (...) {
    return SKSSM_ELAUNCH;
  }
}

int sketchssm_full_step(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                        const sketchssm_step* step, void* hip_stream) {
  try {
    int rc = check_layer(layer);
    if (rc) return rc;
    const Needs nd{true, false, false, false, false, false, true, true, true, false, false};
    if ((rc = check_buffers(layer, bufs, step, nd))) return rc;
    return dispatch(layer, sk::MODE_FULL, make_params(layer, bufs, step), hip_stream);
  } catch (...) {
    return SKSSM_ELAUNCH;
  }
}

int sketchssm_replay_step(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                          const sketchssm_step* step, void* hip_stream) {
  try {
    int rc = check_layer(layer);
    if (rc) return rc;
    const Needs nd{true, false, false, false, true, true, true, true, true, false, false};
    if ((rc = check_buffers(layer, bufs, step, nd))) return rc;
    return dispatch(layer, sk::MODE_REPLAY, make_params(layer, bufs, step), hip_stream);
  } catch (...) {
    return SKSSM_ELAUNCH;
  }
}

int64_t sketchssm_workspace_bytes(const sketchssm_layer* layer) {
  try {
    const int rc = check_layer(layer);
    if (rc) return rc;
    return workspace_bytes(layer);
  } catch (...) {
    return SKSSM_ELAUNCH;
  }
}

int sketchssm_version(void) { return 102; }

}  // extern "C"
