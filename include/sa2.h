/*
 * libsa2 — SpargeAttention2 hot path on AMD CDNA4 (gfx950), C ABI.
 *
 * Three calls, in the order the method runs them (the pages describe the
 * pipeline as: build the block mask first, then run sparse attention over it,
 * and train through it — shd-paper.top summary, "方法详解"/technical
 * framework; gist.science, section 2A and 2C):
 *
 *   sa2_build_mask  hybrid Top-k + Top-p block mask      (gist.science 2A)
 *   sa2_attn_fwd    block-sparse attention forward + LSE (gist.science 2C)
 *   sa2_attn_bwd    dQ, dK, dV over the same mask        (abstract, item ii:
 *                   the sparse attention is trainable)
 *
 * Conventions shared by every call
 * --------------------------------
 * Tensors.  q, k, v, o, dout, dq, dk, dv are device pointers to contiguous
 *   [B, H, N, d] arrays (d fastest), all in one element type `dtype`
 *   (SA2_BF16 or SA2_F32).  Attention arithmetic is bf16 MFMA with fp32
 *   accumulation for both element types: f32 inputs are rounded to bf16 as
 *   they are loaded; f32 outputs keep the fp32 accumulators.  Every pointer
 *   must be 16-byte aligned.  lse is fp32 [B, H, N], natural logarithm.
 * Blocks.  Query block i covers tokens [i*bq, min(N, (i+1)*bq)), key block j
 *   covers [j*bk, min(N, (j+1)*bk)); Tq = ceil(N/bq), Tk = ceil(N/bk).  A
 *   partial last block is a real block (it is pooled over the tokens it has).
 * Scale.  Scores are q.k / sqrt(d) throughout (block scores and attention).
 * Ownership.  The caller allocates and frees every buffer (tensors, the mask
 *   arrays and the workspace).  Inputs are read-only.  The library keeps no
 *   state between calls apart from the thread-local error text.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work on it and return; nothing synchronises the host.
 * Errors.  Arguments are checked before anything is enqueued: SA2_EINVAL for
 *   a malformed call (null or misaligned pointer, bad size, mask geometry that
 *   does not match), SA2_EUNSUPPORTED for a well-formed call outside what the
 *   kernels implement, SA2_EDEVICE when a launch is rejected by the runtime.
 *   sa2_last_error() returns a message for the last non-OK status of the
 *   calling thread.  Faults inside a kernel surface at the caller's next
 *   synchronisation, not as a status.  NaN or Inf inputs are not trapped.
 */
#ifndef SA2_H
#define SA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA2_OK = 0,
  SA2_EINVAL = 1,
  SA2_EUNSUPPORTED = 2,
  SA2_EDEVICE = 3
} sa2_status;

typedef enum { SA2_BF16 = 0, SA2_F32 = 1 } sa2_dtype;

/*
 * The block mask M-bar of gist.science section 2A, for every (batch, head),
 * in three equivalent forms.  All pointers are device pointers owned by the
 * caller; the geometry fields must describe the tensors the mask is used with.
 *
 *   bitmap   uint8 [B, H, Tq, Tk]: 1 where query block i keeps key block j.
 *   row_cnt  int32 [B, H, Tq]: kept key blocks of each query-block row.
 *   row_idx  int32 [B, H, Tq, Tk]: the first row_cnt entries of each row are
 *            its kept key blocks, ascending; the rest are left untouched.
 *   col_cnt  int32 [B, H, Tk]: query blocks that keep each key block.
 *   col_idx  int32 [B, H, Tk, Tq]: the first col_cnt entries are those query
 *            blocks, ascending (the transposed index the backward walks).
 *   row_plan, col_plan  int32 arrays of sa2_mask_plan_bytes(..., 0) and
 *            (..., 1) bytes, 16-byte aligned: the work plans of the bf16,
 *            d = 128 attention kernels, made from row_cnt (forward, dQ) and
 *            col_cnt (dK/dV).  A plan assigns the lists to workgroup slots,
 *            XCD by XCD (slot s runs on XCD s % 8; XCD x takes the x-th
 *            contiguous eighth of the lists, rows by count and columns by
 *            cost), longest first; where no list of a group of four XCDs'
 *            shares is long against the group's load per workgroup, the
 *            group's lists go head by head (longest first within a head):
 *            in the row plan XCD 4g + r takes the r-th contiguous quarter of
 *            every head's lists, in the column plan (or when a quarter
 *            would not fit an XCD's slots) the items are dealt in turn to
 *            the four XCDs.  A list much longer than the
 *            mean load of the kernel's resident workgroups is cut into
 *            segments whose partial sums the list's last segment combines in
 *            a fixed order.
 *            Each plan also holds the completion counters of the kernels
 *            that walk it (rows: forward and dQ; columns: dK/dV): the plan
 *            zeroes them and each kernel leaves them zeroed, so attention
 *            calls that use one mask must not run at the same time.
 *
 * sa2_build_mask writes all these arrays (sa2_mask_plans remakes the plans
 * of a mask whose lists the caller wrote); the attention calls read row_cnt /
 * row_idx (forward, dQ), col_cnt / col_idx (dK, dV) and, for bf16 with
 * d = 128, the plans.  A caller may supply its own mask to the attention
 * calls as long as the lists are ascending, duplicate-free and in range and
 * every row_cnt is at least 1.  A mask that breaks these rules, or whose
 * plans were made for other counts, gives undefined outputs but no access
 * out of range: counts are clamped to [0, Tk] (rows) and [0, Tq] (columns),
 * list entries outside the tensors read as zero rows, and plan entries that
 * do not fit the mask are skipped.
 */
typedef struct sa2_mask {
  int32_t B, H, N, bq, bk, Tq, Tk;
  uint8_t* bitmap;
  int32_t* row_cnt;
  int32_t* row_idx;
  int32_t* col_cnt;
  int32_t* col_idx;
  int32_t* row_plan;
  int32_t* col_plan;
} sa2_mask;

/* Library version string, e.g. "sa2 0.1.0 gfx950". */
const char* sa2_version(void);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* sa2_last_error(void);

/*
 * Bytes of device workspace sa2_build_mask needs for this geometry: the
 * pooled blocks and the block score matrix, all fp64
 * (B*H*(Tq*d + Tk*d + Tq*Tk) doubles).  Returns 0 for an invalid geometry.
 */
size_t sa2_mask_workspace_bytes(int B, int H, int N, int d, int bq, int bk);

/*
 * Bytes of a mask's work plan: columns = 0 for the row plan (query blocks),
 * 1 for the column plan (key blocks).  About 20 bytes per list plus 25 KB.
 * Returns 0 for an invalid geometry.
 */
size_t sa2_mask_plan_bytes(int B, int H, int N, int bq, int bk, int columns);

/*
 * Remakes the work plans of `mask` from its row_cnt and col_cnt (which the
 * caller wrote; sa2_build_mask makes them itself).  Asynchronous on `stream`.
 */
sa2_status sa2_mask_plans(const sa2_mask* mask, void* stream);

/*
 * Hybrid Top-k + Top-p block mask (gist.science, section 2A; Top-p as the
 * smallest set whose cumulative probability reaches p, section 1).
 *
 * For each (b, h) and query block i:
 *   q-bar_i = mean of the query tokens of block i, k-bar_j likewise (fp64);
 *   S-bar_ij = q-bar_i . k-bar_j / sqrt(d);  P-bar_i = softmax_j(S-bar_i);
 *   key blocks are ranked by descending S-bar_ij, the lower j first on ties;
 *   kc = 0 if k_frac <= 0, Tk if k_frac >= 1, else
 *        min(Tk, max(1, ceil(k_frac * Tk - 1e-6)))          (Top-k, k% of Tk);
 *   pc = 0 if p <= 0, Tk if p >= 1, else the smallest m >= 1 whose first m
 *        ranked probabilities sum to at least p (Tk if rounding never
 *        reaches p)                                              (Top-p);
 *   the row keeps the first max(kc, pc) ranked blocks, which is the union of
 *   the Top-k and Top-p sets because both are prefixes of the same ranking.
 *
 * q, k: device [B, H, N, d] in `dtype`, 16-byte aligned, d a multiple of 8 and
 * at most 256.  The pooled values and scores are computed in fp64 from the
 * inputs exactly as stored.  mask: geometry fields filled in by the caller
 * (Tq, Tk as above) and all seven arrays allocated.  workspace: at least
 * sa2_mask_workspace_bytes(...) bytes of device memory, 256-byte aligned.
 * Limits: Tq, Tk <= 4096 and B*H <= 65535 (else SA2_EUNSUPPORTED).  k_frac <= 0
 * together with p <= 0 (both rules off)
 * is SA2_EINVAL; NaN parameters are SA2_EINVAL.
 */
sa2_status sa2_build_mask(const void* q, const void* k, int dtype,
                          int B, int H, int N, int d, int bq, int bk,
                          double k_frac, double p, const sa2_mask* mask,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * sa2_build_mask without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It computes exactly what sa2_build_mask
 * computes, with the same arguments apart from the workspace, and allocates
 * nothing: its fp64 pooled blocks and score matrix live in a static device
 * array of SA2_MASK_NOALLOC_MAX_BYTES bytes that each GPU the library runs
 * on holds from module load until the process ends.  A geometry whose
 * sa2_mask_workspace_bytes() exceeds that is refused with SA2_EUNSUPPORTED
 * before anything is enqueued (the 1.3B-shaped layer needs 22 MB with
 * 128 x 64 blocks and 38 MB with 64 x 64 blocks; the 14B-shaped one 296 MB).
 * The kernels run on the device of `stream` (the current device if NULL).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (e.g. on two streams without ordering between them) race.  Nothing in
 * the array needs to start at zero.
 */
#define SA2_MASK_NOALLOC_MAX_BYTES ((size_t)64 << 20)
sa2_status sa2_build_mask_noalloc(const void* q, const void* k, int dtype,
                                  int B, int H, int N, int d, int bq, int bk,
                                  double k_frac, double p, const sa2_mask* mask,
                                  void* stream);

/*
 * Bytes of device workspace sa2_attn_fwd needs: for d = 128, 1024
 * partial-sum slots of 66 KB (unnormalised output rows, running maxima and
 * row sums of the segments of long rows; 67.6 MB); 0 for d = 64, whose
 * kernels need none.  Returns 0 for an invalid geometry too.
 */
size_t sa2_fwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Block-sparse attention forward (gist.science, section 2C: tiles are kept or
 * dropped whole; dropped tiles cost neither the matmuls nor the softmax).
 *
 * For every query token t of query block i:
 *   O_t = sum_u softmax_u(q_t . k_u / sqrt(d)) v_u over the key tokens u of the
 *   key blocks listed in row_idx for row i (non-causal);
 *   lse_t = log sum_u exp(q_t . k_u / sqrt(d)) over the same keys.
 *
 * For bf16 with d = 128 the kernel follows the mask's row plan: a row list
 * much longer than the mean load of the kernel's resident workgroups (a
 * skewed head under Top-p keeps most key blocks in a few rows, gist.science
 * section 1) is walked in segments in parallel; each segment leaves its
 * unnormalised output, running maximum and row sum in the workspace, and the
 * last segment of the row combines them in segment order (the same softmax,
 * bitwise reproducible).
 *
 * q, k, v: device [B, H, N, d]; o: device [B, H, N, d] (written); lse: device
 * fp32 [B, H, N] (written).  mask: as produced by sa2_build_mask (row lists
 * used).  workspace: at least sa2_fwd_workspace_bytes(...) bytes of device
 * memory, 256-byte aligned (may be NULL when that is 0); scratch between
 * calls, no initialisation needed.  Limits: d in {64, 128}, bq in {64, 128},
 * bk = 64.
 */
sa2_status sa2_attn_fwd(const void* q, const void* k, const void* v, int dtype,
                        int B, int H, int N, int d, const sa2_mask* mask,
                        void* o, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Bytes of device workspace the backward calls need: two fp32 per token
 * row, the row sums Delta_t = sum_c dO_tc O_tc and the LSE in base 2
 * (lse_t * log2(e)), for every row of every 128-row query block (padding
 * rows past N included): B*H*4*ceil(N/128) groups of 32 rows x 2 x 4 bytes,
 * rounded up to 256 bytes.  For d = 128 it also holds the partial-sum slots
 * of the lists the mask's plans cut into segments: 1024 slots of 64 KB for
 * dQ rows and 2048 of 64 KB for dK/dV columns (192 MB); the partials are
 * added in segment order.  The contents need no initialisation and are
 * scratch between calls.
 */
size_t sa2_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Gradients of the forward above with the mask held constant (selection is
 * piecewise constant, so no gradient flows through it).  With P the
 * attention probabilities of the forward:
 *   dV = P^T dO;  dP = dO V^T;  Delta_t = sum_c dO_tc O_tc;
 *   dS = P * (dP - Delta);  dQ = dS K / sqrt(d);  dK = dS^T Q / sqrt(d).
 * P is recomputed from q, k and lse.  dK and dV of a key block are summed over
 * the query blocks in its col_idx list, dQ of a query block over its row_idx
 * list (long lists of either kind are summed in segments, then across
 * segments in a fixed order); no atomics are used, so results are bitwise
 * reproducible.  Key
 * blocks that no query block keeps get dK = dV = 0.
 *
 * q, k, v, o, dout: device [B, H, N, d] (o and lse from sa2_attn_fwd on the
 * same inputs and mask); dq, dk, dv: device [B, H, N, d] (written);
 * workspace: at least sa2_bwd_workspace_bytes(...) bytes, 256-byte aligned.
 * Limits as for sa2_attn_fwd.  Equivalent to sa2_attn_bwd_dq followed by
 * sa2_attn_bwd_dkdv on the same stream and workspace.
 */
sa2_status sa2_attn_bwd(const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout,
                        int dtype, int B, int H, int N, int d,
                        const sa2_mask* mask, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * First half of sa2_attn_bwd: dQ = dS K / sqrt(d) over each query block's
 * row list, and Delta_t = sum_c dO_tc O_tc and lse_t * log2(e), which it
 * leaves in `workspace` for sa2_attn_bwd_dkdv.  Arguments as for
 * sa2_attn_bwd; it reads row_cnt and row_idx, and for bf16 with d = 128 the
 * row plan (SA2_EINVAL if that is NULL).
 */
sa2_status sa2_attn_bwd_dq(const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           int dtype, int B, int H, int N, int d,
                           const sa2_mask* mask, void* dq,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Second half of sa2_attn_bwd: dV = P^T dO and dK = dS^T Q / sqrt(d) over
 * each key block's column list (for bf16 with d = 128 following the mask's
 * column plan).  Reads Delta and the base-2 LSE from `workspace` (lse itself
 * is still checked), so it must follow sa2_attn_bwd_dq on the same inputs,
 * mask and workspace, on the same stream (or after it completes).  Called
 * otherwise, dK and dV are undefined, but nothing is read or written out of
 * range.  Arguments as for sa2_attn_bwd.
 */
sa2_status sa2_attn_bwd_dkdv(const void* q, const void* k, const void* v,
                             const float* lse, const void* dout,
                             int dtype, int B, int H, int N, int d,
                             const sa2_mask* mask, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same gradients as sa2_attn_bwd (bf16, d = 128 only), with dQ formed
 * inside the dK/dV pass and accumulated in fp32 with atomic additions
 * instead of by a separate pass over the row lists: the alternative to the
 * deterministic backward, which recomputes S and dP for dQ (two more of the
 * seven matrix products per kept pair).  The order of the atomic additions
 * is not fixed, so dQ may differ in its last bits from call to call; dK and
 * dV are as in sa2_attn_bwd.  The call runs three kernels: Delta, the base-2
 * LSE and a zeroed fp32 dQ accumulator; dK, dV and dQ over the column lists;
 * dQ scaled and rounded.  workspace: at least
 * sa2_bwd_atomic_workspace_bytes(...) bytes (sa2_bwd_workspace_bytes plus
 * 4 B*H*N*d for the accumulator), 256-byte aligned.  Other arguments as for
 * sa2_attn_bwd; SA2_EUNSUPPORTED for other element types or d.
 */
size_t sa2_bwd_atomic_workspace_bytes(int B, int H, int N, int d);
sa2_status sa2_attn_bwd_atomic_dq(const void* q, const void* k, const void* v,
                                  const void* o, const float* lse, const void* dout,
                                  int dtype, int B, int H, int N, int d,
                                  const sa2_mask* mask, void* dq, void* dk, void* dv,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Layer-level velocity distillation (gist.science, section 2B: the student,
 * with sparse attention, is fitted to the frozen full-attention teacher by
 * the squared difference of their outputs).  At the level of one attention
 * layer the student output is o_student (sa2_attn_fwd with the hybrid mask)
 * and the teacher output o_teacher (the same call with every block kept):
 *
 *   loss = sum over all B*H*N*d elements of (o_student - o_teacher)^2 / (B*H*N*d)
 *   dout = d loss / d o_student = 2 (o_student - o_teacher) / (B*H*N*d)
 *
 * dout (written, [B, H, N, d] in `dtype`) is the upstream gradient for
 * sa2_attn_bwd on the student's mask; loss is one fp64 value written to device
 * memory.  The sum is taken in fp64 in a fixed order (per-chunk partial sums
 * in the workspace, then one ordered sum), so it is bitwise reproducible.
 * o_student, o_teacher, dout: 16-byte aligned; workspace: at least
 * sa2_distill_workspace_bytes() bytes, 256-byte aligned.
 */
size_t sa2_distill_workspace_bytes(int B, int H, int N, int d);
sa2_status sa2_distill_loss_grad(const void* o_student, const void* o_teacher, int dtype,
                                 int B, int H, int N, int d, void* dout, double* loss,
                                 void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA2_H */
