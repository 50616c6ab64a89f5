/*
 * sketchssm.h -- C ABI of the SketchSSM decode hot path on AMD Instinct
 * MI355X (gfx950).
 *
 * SketchSSM ("Write to the Full State, Read from a Compact Sketch",
 * arXiv 2609.33051) keeps the full recurrent state S of a linear-attention /
 * SSM head exact but reads it only once per window of W decode steps:
 *
 *   - flush (every W steps): read S once, apply the W buffered updates from
 *     the ring, build the sketch U = S^T P from the updated state with a fixed
 *     per-head basis P, write back S and U (project page, "02 / How to make a
 *     sketch", per-window flush panel; paper App. B);
 *   - read (the other W-1 steps): o = U (C q~) plus the exact contribution of
 *     the buffered updates, where q~ is the query pulled back through the
 *     buffered transitions; S is not read (project page, per-step non-flush
 *     panel; paper Sec. 3.2 and App. C.1).
 *
 * The coefficient map C is either a fixed per-head table the caller supplies
 * (the paper's fixed-coefficient rule, App. G) or the state-dependent map the
 * flush forms for every (sequence, head) tile from its new state,
 * C = (U^T U + lambda I)^{-1} U^T S^T with U the stored sketch (project page,
 * per-window flush panel; paper App. A.2.1-A.2.2).
 *
 * Two baselines share the layout: the standard full-state step (read and
 * write S every step; project page "01 / The idea", S_t = M_t S_{t-1} + B_t,
 * o_t = S_t^T q_t) and ReplaySSM (buffered writes, full-state read every
 * step; paper Sec. 1-2 and App. D).
 *
 * Families (per (sequence, head) tile; S is dk x dv, o = S^T q):
 *   SKSSM_MAMBA2: S <- a S + dt k v^T,  a = exp(-dt * exp(A_h)); q~ = (prod a) q
 *   SKSSM_GDN:    S <- alpha (I - beta k k^T) S + beta k v^T
 *   SKSSM_KDA:    S <- (I - beta k k^T) Diag(g) S + beta k v^T
 *
 * Memory and ownership
 *   - Every pointer inside sketchssm_buffers / sketchssm_step is a DEVICE
 *     pointer owned by the caller.  sketchssm_layer and its rank_offsets_host
 *     table are HOST memory, read during the call only and never retained.
 *   - The library allocates nothing, keeps no state between calls (except
 *     the per-device address of sketchssm_read_noalloc's scratch array) and
 *     never synchronises: every call only enqueues kernels on the caller's HIP
 *     stream (NULL = the default stream).  Buffers must not be reused until
 *     stream order guarantees completion.  Calls on different layers may run
 *     concurrently on different streams; calls on one layer must be ordered.
 *   - Calls are re-entrant; no C++ exception crosses the ABI.
 *
 * Errors
 *   - The return value is 0 on success or a negative SKSSM_E* code.
 *     Arguments are validated on the host, synchronously; on failure nothing
 *     is launched and nothing is written.
 *   - SKSSM_ELAUNCH reports a failed launch (hipGetLastError after it).
 *   - Semantic faults found by the kernels (a ring count outside [0, W], a
 *     read of a sequence whose window is already full, inconsistent counts
 *     within a Mamba-2 B/C group) leave that tile untouched and OR a
 *     SKSSM_ERRBIT_* bit into *err; the caller reads it after synchronising.
 *   - Device faults surface at the caller's next synchronisation.
 */
#ifndef SKETCHSSM_H
#define SKETCHSSM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* families */
#define SKSSM_MAMBA2 0
#define SKSSM_GDN 1
#define SKSSM_KDA 2

/* dtypes */
#define SKSSM_F32 0
#define SKSSM_BF16 1

/* coefficient maps */
#define SKSSM_COEF_FIXED 0 /* bufs->C: one fp32 map per head, shared by all sequences */
#define SKSSM_COEF_STATE 1 /* bufs->Cstate: one map per (sequence, head), written by the flush */

/* evaluation of the effective query and the buffered term at a non-flush
 * read (GDN and KDA; a Mamba-2 effective query is a decay only, and Mamba-2
 * ignores the choice) */
#define SKSSM_PULLBACK_SERIAL 0 /* one buffered transition at a time, newest first */
#define SKSSM_PULLBACK_WY 1     /* every buffered slot's coefficient from one triangular
                                   system over the slots (paper App. C.1), then q~ and
                                   the buffered term as sums over the slots */
#define SKSSM_PULLBACK_PROJ 2   /* the coefficients of SKSSM_PULLBACK_WY, with C q~ formed
                                   from per-slot factors projected through the coefficient
                                   map (paper App. C.2): the read that appends slot l stores
                                   P_l = C_h (Gamma_l (.) k_l) in bufs->ring_pc (Gamma_l:
                                   the product of the decays of slots 0..l), and
                                   C q~ = C_h (Gamma_n0 (.) q) - sum_l beta_l d_l P_l.
                                   Every non-flush step of such a layer is a
                                   sketchssm_read (replay steps do not store factors). */

/* flush flags */
#define SKSSM_FLUSH_DUE 0 /* flush tiles whose ring holds W entries */
#define SKSSM_FLUSH_ALL 1 /* flush every tile (prime U, or retire sequences) */
#define SKSSM_FLUSH_DUE_SCAN 2 /* as SKSSM_FLUSH_DUE, with the due sequences first listed
                                  on the device (in bufs->work), so that a ragged window
                                  phase launches workgroups for the due tiles only */
#define SKSSM_FLUSH_CLOSE 3 /* the step that closes every tile's window, in place of
                               sketchssm_read then SKSSM_FLUSH_DUE at that step: tiles
                               whose ring holds W - 1 entries take the step's own entry
                               as the W-th */

/* return codes */
#define SKSSM_OK 0
#define SKSSM_EINVAL -1  /* NULL or misaligned pointer (16-byte alignment) */
#define SKSSM_EDIM -2    /* unsupported shape, W, ranks or rank table */
#define SKSSM_EDTYPE -3  /* unsupported dtype combination */
#define SKSSM_EFLAG -4   /* unknown flag or coefficient-map mode */
#define SKSSM_ELAUNCH -5 /* kernel launch failed */
#define SKSSM_ESCRATCH -6 /* sketchssm_read_noalloc: the layer needs more scratch than the
                             library's array holds (SKSSM_NOALLOC_SCRATCH_BYTES) */

/* size of the device array that sketchssm_read_noalloc uses as its workspace
 * (16 MiB; one per GPU the library runs on, held until the process ends) */
#define SKSSM_NOALLOC_SCRATCH_BYTES 16777216

/* bits OR-ed into *err by the kernels */
#define SKSSM_ERRBIT_COUNT 1  /* count outside [0, W] (or == W at a read) */
#define SKSSM_ERRBIT_GROUP 2  /* Mamba-2 heads of one B/C group disagree on count */
#define SKSSM_ERRBIT_SEQ 4    /* sketchssm_flush_seqs: a listed index outside [0, batch),
                                 or a tile claimed twice (a sequence listed twice) */

/* Supported shapes: (dk, dv) in {(16,32), (64,64), (128,64), (128,128)};
 * 1 <= W <= 32; 0 <= r_h <= min(dk, 16), except r_h <= dk when dk == 16
 * (r_h = 0: a dense-fallback head, paper App. D, which keeps a copy of its
 * state in the sketch dtype and reads it at non-flush steps; at most 64 per
 * layer);
 * heads % qk_groups == 0 (qk_groups == heads for GDN/KDA). */
typedef struct {
  int32_t family;            /* SKSSM_MAMBA2 | SKSSM_GDN | SKSSM_KDA */
  int32_t batch;             /* B sequences */
  int32_t heads;             /* H state heads */
  int32_t qk_groups;         /* G: Mamba-2 B/C groups (heads h in group h / (H/G)); GDN/KDA: = H */
  int32_t dk, dv;            /* state is dk x dv per (sequence, head) */
  int32_t window;            /* W: one flush every W steps */
  int32_t act_dtype;         /* dtype of q, k, v, o, Mamba-2 dt and the ring's k, v, dt */
  int32_t sketch_dtype;      /* dtype of U */
  const int32_t* rank_offsets_host; /* [H+1] host copy: exclusive prefix sum of r_h; r_h = 0
                                marks a dense-fallback head (no sketch: a state copy) */
  int32_t coef_map;          /* SKSSM_COEF_FIXED or SKSSM_COEF_STATE */
  float coef_ridge;          /* SKSSM_COEF_STATE: ridge relative to the mean eigenvalue of
                                the sketch's Gram matrix, lambda = coef_ridge * trace(G) / r_h;
                                finite and > 0 (ignored for SKSSM_COEF_FIXED) */
  int32_t pullback;          /* SKSSM_PULLBACK_SERIAL, _WY or _PROJ (non-flush reads) */
} sketchssm_layer;

typedef struct {
  float* S;                  /* [B][H][dk][dv] fp32, dv fastest */
  void* U;                   /* [B][R][dv] sketch dtype, R = offsets[H]; rows
                                off_h..off_h+r_h-1 hold u_j = S^T p_j of head h */
  const float* Pt;           /* [R][dk] fp32: row off_h + j = column j of P_h */
  const float* C;            /* SKSSM_COEF_FIXED: [R][dk] fp32: row off_h + j = row j of C_h
                                (r_h x dk); NULL allowed for SKSSM_COEF_STATE */
  const int32_t* rank_offsets; /* [H+1] device copy of rank_offsets_host */
  void* ring_k;              /* [B][G][W][dk] act dtype */
  void* ring_v;              /* [B][H][W][dv] act dtype */
  void* ring_gate;           /* Mamba-2: dt [B][H][W] act dtype; GDN: alpha [B][H][W] fp32;
                                KDA: g [B][H][W][dk] fp32 */
  float* ring_beta;          /* GDN/KDA: [B][H][W] fp32; NULL for Mamba-2 */
  int32_t* count;            /* [B][H]: entries buffered in tile (b,h) since its last flush,
                                0..W; every head of a sequence advances together */
  const float* A;            /* Mamba-2: [H] fp32; NULL otherwise */
  int32_t* err;              /* [1] device error word (SKSSM_ERRBIT_*), never cleared here */
  void* work;                /* workspace of sketchssm_workspace_bytes(layer) bytes (16-byte
                                aligned; may be NULL when that is 0); scratch that a call
                                overwrites, so calls sharing one workspace must be ordered */
  void* Cstate;              /* SKSSM_COEF_STATE: [B][R][dk] sketch dtype; rows off_h..off_h+r_h-1
                                of sequence b hold the map of tile (b, h), written by every
                                flush of that tile (NULL allowed for SKSSM_COEF_FIXED) */
  void* Scopy;               /* [B][D][dk][dv] sketch dtype, D = number of dense-fallback heads
                                (r_h = 0, at most 64), in head order: their state copies,
                                written by their flush, read by their non-flush reads.  NULL
                                allowed when D = 0.  (Compact: a [B][H] layout would put the
                                few dense tiles at strides that load a few memory channels.) */
  float* ring_pc;            /* GDN/KDA with SKSSM_PULLBACK_PROJ: [B][H][W][16] fp32, slot l
                                of tile (b, h) holds P_l (r_h entries); NULL otherwise */
} sketchssm_buffers;

typedef struct {             /* one decode step */
  const void* q;             /* [B][G][dk] act dtype */
  const void* k;             /* [B][G][dk] act dtype */
  const void* v;             /* [B][H][dv] act dtype */
  const void* gate;          /* Mamba-2: dt [B][H] act dtype; GDN: alpha [B][H] fp32;
                                KDA: g [B][H][dk] fp32 */
  const float* beta;         /* GDN/KDA: [B][H] fp32; NULL for Mamba-2 */
  void* o;                   /* [B][H][dv] act dtype (output) */
} sketchssm_step;

/* Non-flush sketched read (project page, per-step non-flush panel: c = C q~,
 * o^ = U c, plus the exact buffered contribution; paper Sec. 3.2 and
 * App. C.1 for q~).  For every tile: append the step's (k, v, gate, beta) at
 * ring slot count, count += 1; if count < W write o = U (C q~) + o_buf
 * (a dense-fallback head: o = Scopy^T q~ + o_buf), otherwise leave o for
 * sketchssm_flush.  Never reads S.  C is bufs->C
 * (SKSSM_COEF_FIXED) or the tile's own map in bufs->Cstate, as its last
 * flush wrote it (SKSSM_COEF_STATE).  Mamba-2 layers, and GDN/KDA layers
 * with dense-fallback heads, need bufs->work (sketchssm_workspace_bytes). */
int sketchssm_read(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                   const sketchssm_step* step, void* hip_stream);

/* Flush (paper App. B; project page per-window flush panel: U = S^T Omega,
 * fused into the update).  For every tile with count == W (flags =
 * SKSSM_FLUSH_DUE) or every tile (SKSSM_FLUSH_ALL): apply the count buffered
 * entries to S in order, write S, write U = S^T P from the updated state,
 * set count = 0 and, if step != NULL, write the exact output o = S^T q.
 * A dense-fallback head (r_h = 0) writes its state copy to bufs->Scopy
 * (rounded to the sketch dtype) instead of a sketch.
 * FLUSH_ALL with count == 0 primes U from the current state.
 * SKSSM_COEF_STATE: also write the tile's map to bufs->Cstate, solved in
 * fp32 from the sketch rows as stored (rounded to the sketch dtype) and the
 * updated state: G = U_h U_h^T (r_h x r_h), Y = U_h S^T (r_h x dk),
 * C = (G + lambda I)^{-1} Y, lambda = coef_ridge * trace(G) / r_h, stored in
 * the sketch dtype (C = 0 when the sketch is zero).
 * SKSSM_FLUSH_DUE_SCAN (paper App. B: each sequence flushes when its own
 * window fills): the same result as SKSSM_FLUSH_DUE for callers that do not
 * track window phases, given that every head of a sequence holds the same
 * count (sketchssm_read appends, and the flushes reset, all heads of a
 * sequence together).  A first launch (one workgroup) lists, in sequence
 * order, the sequences whose head-0 count is W in bufs->work
 * (sketchssm_workspace_bytes; 16-byte aligned) and reports head-0 counts
 * outside [0, W] (SKSSM_ERRBIT_COUNT).  The flush then runs a grid of one
 * workgroup per tile of min(batch, 2 * ceil(batch / W) + 8) sequences
 * (about twice what a ragged phase brings due at a step) over the tiles of
 * the listed sequences, each workgroup taking further tiles in turn when
 * the list is longer (an aligned phase), so that a ragged phase does not
 * pay a workgroup per tile of the batch.  A listed tile whose count is
 * below W is left alone; the counts of the other heads are
 * checked in listed sequences only.
 * SKSSM_FLUSH_CLOSE (paper App. B: the flush step applies the window's W
 * entries, its own included, and its output comes from the updated state):
 * for a step at which every sequence closes its window (an aligned phase),
 * called instead of sketchssm_read followed by SKSSM_FLUSH_DUE, with the
 * same results in S, U, count, the maps and o.  step is required (k, v,
 * gate, beta as for sketchssm_read; q and o for the output).  Each tile's
 * ring must hold W - 1 entries: the W - 1 buffered entries are applied,
 * then the step's own, and count becomes 0; a tile with any other count
 * sets SKSSM_ERRBIT_COUNT and is left untouched (the caller's phase was not
 * aligned: such a step needs sketchssm_read and SKSSM_FLUSH_DUE).  This
 * saves the read's launches at the closing step, which only append. */
int sketchssm_flush(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                    const sketchssm_step* step /* NULL: no output */, int32_t flags,
                    void* hip_stream);

/* Flush of listed sequences: sketchssm_flush with SKSSM_FLUSH_DUE, launched
 * for the tiles of the nseq sequences in seqs only (paper App. B: each
 * sequence flushes when its own window fills).  For callers that know which
 * sequences close their window at this step: under a ragged window phase
 * about batch / W sequences are due per step, and the due-flag flush pays
 * for a workgroup per tile of the whole batch.  seqs: DEVICE array of nseq
 * distinct sequence indices (int32, 4-byte aligned), 0 <= nseq <= batch.
 * A listed tile whose count is in [0, W) is left alone; a count outside
 * [0, W] sets SKSSM_ERRBIT_COUNT; an index outside [0, batch) sets
 * SKSSM_ERRBIT_SEQ and is skipped.  Each tile is claimed before it is
 * flushed (its count goes from W to W + 1 until the flush stores 0), so a
 * sequence listed twice is flushed once, and the second claim of a tile
 * that is still being flushed sets SKSSM_ERRBIT_SEQ.  nseq = 0 launches
 * nothing. */
int sketchssm_flush_seqs(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                         const sketchssm_step* step /* NULL: no output */, const int32_t* seqs,
                         int32_t nseq, void* hip_stream);

/* Standard full-state step (project page "01 / The idea": S_t = M_t S_{t-1}
 * + B_t, o_t = S_t^T q_t): S <- M S + B and o = S^T q for every tile.
 * Ignores the ring, count, U, Pt and C. */
int sketchssm_full_step(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                        const sketchssm_step* step, void* hip_stream);

/* ReplaySSM step (paper Sec. 1-2 and App. D: buffer writes for W steps,
 * read the full state every step).  Append as sketchssm_read; if count < W
 * write the exact o = S0^T q~ + o_buf reading S in full; if count == W apply
 * the W entries, write S, o = S^T q, count = 0.  Does not touch U. */
int sketchssm_replay_step(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                          const sketchssm_step* step, void* hip_stream);

/* Bytes of the workspace bufs->work for this layer, or a negative SKSSM_E*
 * code for an invalid layer: the larger of what sketchssm_read and
 * sketchssm_flush with SKSSM_FLUSH_DUE_SCAN need (a call uses the workspace
 * only while it runs, and calls on one layer are ordered, so both share it).
 * The read needs it (and checks bufs->work) only for these layers:
 * Mamba-2, for what the heads of a B/C group share at a step: the query's
 * coordinates in every head's sketch basis, C_h q (B x R fp32; the decay
 * factor of the pulled-back query is applied afterwards), the dot products
 * of the query with the group's buffered keys (B x G x W fp32) and the
 * group's checked ring fill (B x G int32); GDN and KDA with dense-fallback
 * heads: per (sequence, dense head) the pulled-back query (dk fp32), the
 * buffered term (dv fp32) and a flag (int32), passed from the read's main
 * launch to the launch that reads the state copies.  The scan flush lists
 * the due sequences: their number (int32 at byte 0), then from byte 256
 * their indices (batch int32, rounded up to 64).  The caller allocates it; the library never
 * does. */
int64_t sketchssm_workspace_bytes(const sketchssm_layer* layer);

/* sketchssm_read for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, semantics, kernels and results as sketchssm_read, except
 * that bufs->work is ignored: the workspace is a device array of the library
 * (SKSSM_NOALLOC_SCRATCH_BYTES, one per GPU, resolved on the first call on
 * each device).  The call allocates nothing and never synchronises.
 * Returns SKSSM_ESCRATCH, launching nothing, when sketchssm_workspace_bytes
 * of the layer exceeds SKSSM_NOALLOC_SCRATCH_BYTES (at dk = 128 this holds,
 * e.g., a Mamba-2 layer of 1024 sequences with 2048 sketch rows and W = 32).
 * Every call on one GPU shares that GPU's array, whatever the layer or
 * stream: calls that may overlap on one GPU (two streams, two threads) race
 * and must be ordered by the caller.  The array keeps the last call's
 * contents; every value a call reads from it is written earlier in the same
 * call, so nothing needs clearing. */
int sketchssm_read_noalloc(const sketchssm_layer* layer, const sketchssm_buffers* bufs,
                           const sketchssm_step* step, void* hip_stream);

/* Library version (major * 10000 + minor * 100 + patch). */
int sketchssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKETCHSSM_H */
