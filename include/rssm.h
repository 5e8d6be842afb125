/*
 * rssm.h -- C ABI of the ReplaySSM decode hot path for AMD MI355X (gfx950).
 *
 * The method (pages on ReplaySSM, "Cache SSM Inputs, Not State"): each sequence's
 * recurrent state is held as an FP32 checkpoint S_ckpt plus a ring buffer of the
 * input records appended since the checkpoint, with a cursor.  Non-flush decode
 * steps append the record and compute only the output from checkpoint + ring;
 * a flush folds the ring into the checkpoint and writes it once; speculative
 * drafts are appended past the cursor, verified output-only, and the accepted
 * prefix is committed by advancing the cursor.  Source passages:
 *   - page 4 "ReplaySSM caches SSM inputs instead of state ...", section "What
 *     shipped": the Mamba-2 update, the window of 16 records, flush, pointer
 *     commit of drafts, and the output-only chunkwise verify form;
 *   - page 1 (Japanese news article), sections on what the method does and on
 *     what got faster: write once per window, rollback as a pointer move, and
 *     the low-precision read copy that never re-enters the recurrence.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller allocates and
 *     owns every buffer; the library never allocates in these calls and keeps no
 *     global mutable state.  Calls on distinct states and streams may run
 *     concurrently; calls on one state must be ordered by the caller (one stream).
 *   - Every call only ENQUEUES work on `stream` (NULL = the null stream) and
 *     returns immediately, except rssm_get_error (synchronises).
 *   - Host-side validation failure returns a negative RSSM_E_* code and enqueues
 *     nothing.  batch == 0 is valid and enqueues nothing.
 *   - Device-side contract violations set bits in the sticky error word
 *     state->err and leave the offending sequence untouched (read it with
 *     rssm_get_error).
 *   - Inputs are fp32 or bf16 (raw bfloat16 bits, uint16_t) per config.in_dtype;
 *     outputs are always fp32.  S_ckpt is fp32 [B][H][dv][dk], dk contiguous.
 *   - Value head h uses key/query head h / (H / G) (contiguous groups).
 *   - Alignment: s_ckpt, s_read and the conventional state must be 16-byte
 *     aligned; every other pointer must be aligned to its element size.
 */
#ifndef RSSM_H
#define RSSM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes (host side) */
enum {
  RSSM_OK = 0,
  RSSM_E_NULL = -1,    /* a required pointer is NULL */
  RSSM_E_SHAPE = -2,   /* unsupported or inconsistent sizes */
  RSSM_E_DTYPE = -3,   /* unknown kind / in_dtype / read_copy */
  RSSM_E_ALIGN = -4,   /* misaligned pointer */
  RSSM_E_RANGE = -5,   /* argument out of range (T, min_records) */
  RSSM_E_HIP = -6,     /* a HIP runtime call failed */
  RSSM_E_DEVICE = -7   /* no usable gfx950 device */
};

/* bits of the device-side sticky error word */
enum {
  RSSM_DEVERR_VERIFY_CAPACITY = 1, /* verify: h + T > capacity; sequence untouched */
  RSSM_DEVERR_ACCEPT_RANGE = 2,    /* commit: n_accept outside 0..T, or the verify it
                                      commits could not append (h + T > capacity) */
  RSSM_DEVERR_CURSOR = 4,          /* counters inconsistent (h < 0 or h > capacity) */
  RSSM_DEVERR_TREE = 8             /* tree verify: a parent index is not -1 or an earlier
                                      draft; sequence untouched */
};

enum { RSSM_KIND_MAMBA2 = 0, RSSM_KIND_GDN = 1, RSSM_KIND_KDA = 2 };
enum { RSSM_DTYPE_F32 = 0, RSSM_DTYPE_BF16 = 1 };
enum { RSSM_READ_NONE = 0, RSSM_READ_FP8 = 1, RSSM_READ_MXFP4 = 2 };

/* (host) problem description.
 *   kind       RSSM_KIND_MAMBA2: S <- a S + v k^T, y = S q (page 4, "What shipped").
 *              RSSM_KIND_GDN: gated delta rule S <- a S (I - b k k^T) + b v k^T,
 *              o = S q (the pages name it without a formula; published form).
 *              RSSM_KIND_KDA: Kimi Delta Attention, the gated delta rule with one gate
 *              per key channel, S <- S Diag(a) (I - b k k^T) + b v k^T, o = S q; alpha
 *              is a dk-vector per value head (page 4 "Why it matters": the replay
 *              reframing carries over to KDA's delta-rule update; no formula on the
 *              pages, so the form of KDA's own publication).
 *   batch      B >= 0 sequences.
 *   n_heads    H value heads; n_qk_heads G key/query heads, H % G == 0.
 *   dv, dk     P rows and N columns of a state tile.  dk in {32, 64, 128, 256};
 *              1 <= dv <= 16384 / dk.
 *   L          flush threshold (window length; the pages use 16), L >= 1.
 *   t_max      maximum drafts per verify (1 = decode only), 1 <= t_max <= 8.
 *   capacity   ring slots C, L + t_max - 1 <= C <= 32.
 *              Each ring region (B*H*C*dv and B*G*C*dk elements; KDA alpha B*H*C*dk)
 *              and each step input (B*t_max*H*dv, B*t_max*G*dk elements; KDA alpha
 *              B*t_max*H*dk) holds fewer than 2^31 elements (RSSM_E_SHAPE otherwise).
 *   in_dtype   RSSM_DTYPE_F32 or RSSM_DTYPE_BF16 for alpha, beta, v, k, q and the ring.
 *   read_copy  RSSM_READ_NONE, RSSM_READ_FP8 (OCP E4M3FN codes + one fp32 scale
 *              amax/448 per 32 elements along dk) or RSSM_READ_MXFP4 (OCP MX
 *              E2M1 codes, two per byte with the even element in the low nibble,
 *              + one E8M0 scale 2^(floor(log2 amax) - 2) per 32 elements).  The copy
 *              is written at init and at every flush, read by non-flush decode
 *              steps only, and never feeds the recurrence (page 1, low-precision
 *              section; page 4, quantisation paragraph). */
typedef struct {
  int32_t kind;
  int32_t batch;
  int32_t n_heads;
  int32_t n_qk_heads;
  int32_t dv;
  int32_t dk;
  int32_t L;
  int32_t t_max;
  int32_t capacity;
  int32_t in_dtype;
  int32_t read_copy;
} rssm_config;

/* (host) struct of caller-owned device buffers, sized by rssm_sizes.
 *   s_ckpt        fp32 [B][H][dv][dk] checkpoint (the state as of the last flush).
 *   s_read        read-copy codes: fp8 [B][H][dv][dk] bytes, or MXFP4 [B][H][dv][dk/2]
 *                 bytes; NULL when read_copy == RSSM_READ_NONE.
 *   s_read_scale  fp8: fp32 [B][H][dv][dk/32]; MXFP4: E8M0 bytes [B][H][dv][dk/32];
 *                 NULL when read_copy == RSSM_READ_NONE.
 *   ring          one buffer holding, at 256-byte aligned offsets in this order
 *                 (element = in_dtype), each region slot-major:
 *                   alpha [C][B][H] (KDA: [C][B][H][dk]),
 *                   beta [C][B][H] (GDN and KDA, else absent),
 *                   v [C][B][H][dv], k [C][B][G][dk], q [C][B][G][dk].
 *                 Record of cursor position pos lives in slot pos % C.  Stored
 *                 bits are exact copies of the appended inputs.  (Slot-major: the
 *                 rows one step appends for all sequences are contiguous.)
 *   n_committed   int64 [B][H]: records committed since init (per-tile replicas of
 *                 the per-sequence cursor; all H replicas of a sequence are equal).
 *   n_ckpt        int64 [B][H]: cursor position of the checkpoint.  The ring holds
 *                 h = n_committed - n_ckpt live records.
 *   err           int32 [1] sticky device error word (RSSM_DEVERR_* bits). */
typedef struct {
  float *s_ckpt;
  void *s_read;
  void *s_read_scale;
  void *ring;
  int64_t *n_committed;
  int64_t *n_ckpt;
  int32_t *err;
} rssm_state;

/* (host) byte sizes of the buffers of rssm_state. */
typedef struct {
  size_t s_ckpt;
  size_t s_read;
  size_t s_read_scale;
  size_t ring;
  size_t n_committed;
  size_t n_ckpt;
  size_t err;
} rssm_buffer_sizes;

/* Host only.  Validate a config: RSSM_OK or a negative code. */
int rssm_check_config(const rssm_config *cfg);

/* Host only.  Fill `out` (host) with the byte size of every state buffer. */
int rssm_sizes(const rssm_config *cfg, rssm_buffer_sizes *out);

/* Host only.  Byte offsets of alpha, beta, v, k, q inside `ring` (out: host int64[5];
 * beta's offset equals v's when kind is Mamba-2). */
int rssm_ring_offsets(const rssm_config *cfg, int64_t *out5);

/* Initialise a state (page 4 "What shipped": the state is kept as a checkpoint plus a
 * buffer of recent records; page 1, low-precision paragraph of the section on what got
 * faster: the low-precision copy is made from the checkpoint): S_ckpt <- s0 (fp32
 * [B][H][dv][dk]) or zeros when s0 == NULL, write the read copy from it, set both
 * counters to 0 (an empty window) and clear the error word.  The ring content is left
 * as is (no live records). */
int rssm_init_state(const rssm_config *cfg, const rssm_state *st, const float *s0,
                    hipStream_t stream);

/* One decode step for every sequence (page 4 "What shipped"; page 1, what the
 * method does).  Inputs: alpha [B][H] (KDA: [B][H][dk]), beta [B][H] (GDN and KDA;
 * NULL for Mamba-2),
 * v [B][H][dv], k [B][G][dk], q [B][G][dk].  Output y [B][H][dv] fp32.
 * Per sequence with h = n_committed - n_ckpt live records before the step:
 *   - if h + 1 < L: append the record at slot n_committed % C and write
 *     y = G S_read q + sum_j decay(j -> now) (k_j . q) v_j (Mamba-2; GDN uses the
 *     equivalent query-transform form; KDA the same form with the per-channel gates
 *     applied to the transformed query) where S_read is S_ckpt or its read copy;
 *     S_ckpt is not written;
 *   - else (flush step): fold the h ring records and the current one into
 *     S_ckpt, write it (and the read copy) once, set n_ckpt = n_committed + 1;
 *     y = S_new q from the fp32 state.  The current record is not written to the
 *     ring.
 * Then n_committed += 1.
 * Counters out of range on a tile (h < 0 or h > C) set RSSM_DEVERR_CURSOR and leave
 * that tile untouched.  When H is a multiple of 16 (Mamba-2 and KDA without a read
 * copy) the records of each group of 16 value heads of a sequence (32 for Mamba-2 when H
 * is a multiple of 32) are appended by the workgroup of the group's last head, late in
 * the launch: a tile whose counters differ
 * from that head's is left out of the appends, and if the last head's own counters are
 * out of range none of the group's records of this step is appended. */
int rssm_decode_step(const rssm_config *cfg, const rssm_state *st, const void *alpha,
                     const void *beta, const void *v, const void *k, const void *q,
                     float *y, hipStream_t stream);

/* Fold every sequence holding h >= max(min_records, 1) live records into S_ckpt
 * (write once, plus the read copy) and set n_ckpt = n_committed; other sequences
 * are untouched (page 4 "What shipped", flush).  min_records >= 0.  The
 * speculative protocol calls rssm_flush(L) after every rssm_commit. */
int rssm_flush(const rssm_config *cfg, const rssm_state *st, int32_t min_records,
               hipStream_t stream);

/* Speculative verify (page 4 "What shipped", verify paragraph): append T drafts
 * (1 <= T <= t_max) at slots (n_committed + tau) % C without moving the cursor,
 * and write the output-only chunk O [B][T][H][dv] fp32:
 *   Mamba-2: O[:, tau] = G_{h+tau} S_ckpt q_tau + sum_{j <= h+tau} W[j, tau] (k_j . q_tau) v_j
 *   GDN:     the same with pseudo-values from the delta rule's triangular system,
 *            evaluated per draft in query-transform form.
 *   KDA:     per draft, the query-transform form with per-channel gates.
 * Draft inputs: alpha [B][T][H] (KDA: [B][T][H][dk]), beta [B][T][H] (GDN, KDA), v [B][T][H][dv],
 * k [B][T][G][dk], q [B][T][G][dk].  S_ckpt is never written.  A sequence with
 * h + T > C sets RSSM_DEVERR_VERIFY_CAPACITY and is left untouched (no ring
 * write, its O rows not written). */
int rssm_verify(const rssm_config *cfg, const rssm_state *st, int32_t T, const void *alpha,
                const void *beta, const void *v, const void *k, const void *q, float *o,
                hipStream_t stream);

/* Commit the accepted prefix (page 4 "What shipped"; page 1, rollback as a pointer
 * move): n_committed += n_accept[b] for every sequence, nothing else.  n_accept is
 * int32 [B] on the device, each in 0..T where T is the preceding verify's T.  An
 * out-of-range value (or a sequence whose verify could not append) sets
 * RSSM_DEVERR_ACCEPT_RANGE and leaves that sequence untouched.  It commits a linear
 * rssm_verify; a tree verify is committed with rssm_commit_tree, which also refuses the
 * sequences whose tree the verify refused (rssm_commit cannot tell them). */
int rssm_commit(const rssm_config *cfg, const rssm_state *st, const int32_t *n_accept,
                int32_t T, hipStream_t stream);

/* Tree-shaped speculative verify (page 2, implementation paragraph: pointer-only rollback
 * also matters for tree-based speculation, where the accepted drafts need not be
 * consecutive; the replay form of page 4 "What shipped", verify paragraph).
 * As rssm_verify, with parent int32 [B][T] on the device: draft tau's parent is -1 (the
 * committed head) or an earlier draft.  Output tau comes from the state after the drafts
 * on tau's root-to-node path only: drafts off that path enter the replay form as records
 * with alpha = 1, beta = 0 and no contribution.  Drafts are appended at slots
 * (n_committed + tau) % C as in rssm_verify.  An invalid parent sets RSSM_DEVERR_TREE
 * and leaves the sequence untouched (with rssm_verify_fold: not folded either); h + T > C
 * as in rssm_verify. */
int rssm_verify_tree(const rssm_config *cfg, const rssm_state *st, int32_t T,
                     const int32_t *parent, const void *alpha, const void *beta,
                     const void *v, const void *k, const void *q, float *o, hipStream_t stream);

/* Flush fused in front of a verify: rssm_flush(min_records) followed by rssm_verify(T)
 * (parent NULL) or rssm_verify_tree(T, parent), in one launch: a sequence holding at least
 * max(min_records, 1) records is folded into its checkpoint, read copy included, from the
 * tile the verify reads anyway, and the verify then sees an empty window.  The speculative
 * loop becomes verify_fold(L) -> commit, the fold of one step's commit happening at the
 * next verify (page 4 "What shipped": the fold writes the state once; the verify reads it
 * once).  One difference from the two calls: the capacity rule h + T <= C applies to the
 * window BEFORE the fold (the draft slots must not hold records that other heads of the
 * key group still read for their own folds), so a loop folding at L needs
 * C >= L + 2 T - 1.  A sequence breaking it sets RSSM_DEVERR_VERIFY_CAPACITY and is left
 * untouched (no fold, no output).  Other errors as the two calls. */
int rssm_verify_fold(const rssm_config *cfg, const rssm_state *st, int32_t min_records,
                     int32_t T, const int32_t *parent, const void *alpha, const void *beta,
                     const void *v, const void *k, const void *q, float *o, hipStream_t stream);

/* Commit for a tree verify: path int32 [B][T] holds the accepted drafts in path order,
 * its first n_accept[b] entries a chain from the committed head (path[0] has parent -1,
 * each next entry is a child of the previous one; parent as passed to the verify).  The
 * accepted drafts' ring records move to slots (n_committed + i) % C, i < n_accept[b], so
 * the committed window stays contiguous; then n_committed += n_accept[b].  A path that
 * is not such a chain, n_accept outside 0..T, h + T > C, or a parent row the verify
 * refused (an entry not -1 or an earlier draft: its drafts were never appended) sets
 * RSSM_DEVERR_ACCEPT_RANGE and leaves the sequence untouched.  Follow with
 * rssm_flush(L) as after rssm_commit. */
int rssm_commit_tree(const rssm_config *cfg, const rssm_state *st, const int32_t *parent,
                     const int32_t *path, const int32_t *n_accept, int32_t T, hipStream_t stream);

/* Conventional read-modify-write decode step, the comparison point (page 4 "What
 * shipped": the standard kernel reads the whole state, applies the rank-1 update and
 * writes the state out again on every token).
 * s: fp32 [B][H][dv][dk] state, updated in place; inputs and y as in
 * rssm_decode_step.  No ring, no cursor. */
int rssm_decode_step_conventional(const rssm_config *cfg, float *s, const void *alpha,
                                  const void *beta, const void *v, const void *k,
                                  const void *q, float *y, hipStream_t stream);

/* Snapshot-based speculative verify, the comparison point for rssm_verify (page 4
 * "What shipped", verify paragraph: the conventional speculative path keeps a state per
 * draft, one state read and T state writes per step).
 *   snap   fp32 [B][t_max + 1][H][dv][dk] snapshots, caller-owned
 *          (B * (t_max + 1) * H * dv * dk * 4 bytes); slot cur[b] of sequence b holds
 *          its committed state (the caller writes it before the first call).
 *   cur    int32 [B] on the device, committed slot per sequence.
 *   T, alpha, beta, v, k, q, o as in rssm_verify.
 *   err    int32 [1] on the device; a cur[b] outside 0..t_max sets RSSM_DEVERR_CURSOR
 *          and leaves that sequence untouched.
 * Reads slot cur[b], applies the T drafts one after another (the recurrence of `kind`),
 * writes the state after draft tau to slot (cur[b] + 1 + tau) mod (t_max + 1) and
 * outputs o[b][tau] from it.  Never writes slot cur[b].  Host errors as elsewhere. */
int rssm_verify_snapshot(const rssm_config *cfg, float *snap, const int32_t *cur, int32_t T,
                         const void *alpha, const void *beta, const void *v, const void *k,
                         const void *q, float *o, int32_t *err, hipStream_t stream);

/* Commit for the snapshot path: cur[b] <- (cur[b] + n_accept[b]) mod (t_max + 1), the
 * state after the accepted prefix.  n_accept int32 [B] on the device in 0..T; an
 * out-of-range value sets RSSM_DEVERR_ACCEPT_RANGE (a bad cur[b]: RSSM_DEVERR_CURSOR)
 * in err and leaves that sequence untouched. */
int rssm_commit_snapshot(const rssm_config *cfg, int32_t *cur, const int32_t *n_accept,
                         int32_t T, int32_t *err, hipStream_t stream);

/* Synchronise `stream`, return the device error word (>= 0, RSSM_DEVERR_* bits)
 * and clear it; a negative code if a HIP call fails. */
int rssm_get_error(const rssm_state *st, hipStream_t stream);

/* Plain device-to-device copy of `bytes` bytes (16-byte aligned pointers, bytes a
 * multiple of 16) with a streaming kernel; used to calibrate bandwidth and
 * profiler byte counters against a kernel of known traffic. */
int rssm_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/* Static description of a return code or device error bit set. */
const char *rssm_strerror(int code);

/* ABI version: major * 10000 + minor * 100 + patch. */
int rssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RSSM_H */
