/*
 * dspark.h -- C ABI of the DSpark draft-round hot path for AMD Instinct
 * MI355X (gfx950).
 *
 * The library implements, as hand-written HIP kernels, the three steps of a
 * DSpark drafter round that sit between the draft backbone and the target's
 * verify pass:
 *   1. weight-stationary small-M GEMVs (draft projections, lm_head),
 *   2. the k-step Markov-biased greedy sampling loop, entirely on device,
 *   3. the confidence probe,
 * each as its own entry point, the loop and probe in one launch
 * (dspark_markov_sample_probe), and the lm_head, loop and probe together as
 * one round (dspark_draft_round); and the same over Q8_0 weights (the *_q8
 * entry points).
 *
 * Sources cited below (a reader has the pages themselves):
 *   [DS772]  ds4 #772, "dspark: cut per-cycle CUDA overheads (single-draft
 *            decode, GPU confidence probe)".
 *   [SI441]  SharpInference #441, "perf(cuda): DSpark GPU draft round runs
 *            ~3x the bandwidth floor - small-M (B=7) projection GEMMs ->
 *            weight-stationary matvec (#428 lever 1)".
 *   [W7]     vllm.cpp #436, "SPEC-DSPARK W7: the sequential Markov sample
 *            loop is HOST-side - 28% of the draft step, 14.9 MB downloaded
 *            per step".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller. The
 *    library never allocates, frees or copies memory between host and device.
 *    The small result arrays (ids_out, logit_out, pass_out) may instead be
 *    pinned host memory mapped for the device (hipHostMalloc; pass the
 *    address hipHostGetDevicePointer returns): the kernels then store the
 *    results straight into host memory and no copy follows the call. The
 *    host may read them once the stream has been synchronized.
 *  - Tensors are dense and row-major; there are no stride arguments.
 *  - bf16 tensors are passed as their raw 16-bit patterns (uint16_t).
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Every call only enqueues work on that stream and returns; no call
 *    synchronizes or reads device memory from the host, so every call may be
 *    recorded into a HIP graph.
 *  - Errors: a violated host-checkable precondition returns a nonzero status
 *    BEFORE any HIP call is made and nothing is enqueued. A failed launch
 *    returns DSPARK_ERR_HIP. Faults during execution surface at the caller's
 *    next synchronization, as usual in HIP.
 *  - The library keeps no host-side state besides a launch counter and the
 *    Markov loop's poll bound (dspark_markov_set_spin_limit), and every call
 *    is reentrant. The Markov workspace carries device-side state from one
 *    call to the next, so calls that share a workspace must not run
 *    concurrently (see dspark_markov_sample).
 *  - Results are deterministic: no floating-point atomics are used, and the
 *    summation order of every output is fixed by the shapes alone.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int dspark_status;

#define DSPARK_OK 0
#define DSPARK_ERR_NULL 1      /* a required pointer is NULL                 */
#define DSPARK_ERR_SHAPE 2     /* a size is out of range or inconsistent     */
#define DSPARK_ERR_ALIGN 3     /* a pointer lacks the required alignment     */
#define DSPARK_ERR_WORKSPACE 4 /* workspace missing or smaller than required */
#define DSPARK_ERR_HIP 5       /* the HIP runtime refused a call or launch   */

/* Human-readable name of a status code (static storage, never NULL). */
const char* dspark_status_string(dspark_status status);

/*
 * dspark_proj_smallm -- one draft projection at small M.
 *
 * [SI441] "Observation" and "Proposed work": every projection of the draft
 * block forward multiplies the B drafted positions' activations by one
 * weight matrix; the weight-stationary form reads each weight row from HBM
 * once and applies it to all M activation rows.
 *
 *   Y[m, n] = sum_{t < K} X[m, t] * W[n, t]      m < M, n < N
 *
 *   W  bf16 [N, K]  row n produces output column n    16-byte aligned
 *   X  fp32 [M, K]  activations                        16-byte aligned
 *   Y  fp32 [M, N]  output, overwritten                 4-byte aligned
 * Sizes: N >= 1, K >= 8 and K % 8 == 0, K <= 4194304, M >= 1; for M <= 16
 * the weight rows one workgroup streams (about N / CUs + 1) times 2K bytes
 * must stay below 2 GiB (DSPARK_ERR_SHAPE otherwise: the kernels address a
 * workgroup's share with 32-bit buffer offsets). The weight is streamed once
 * per group of at most 80 rows of X. Accumulation is fp32; each fp32 activation is
 * split exactly-to-2^-17 into two bf16 terms, so |error| stays far below
 * 1e-3 + 1e-3 |Y| at every size in use.
 */
dspark_status dspark_proj_smallm(const uint16_t* W, int N, int K, const float* X, int M,
                                 float* Y, void* stream);

/*
 * dspark_lm_head -- base logits of every drafted row.
 *
 * [W7] "Measured": the drafter's block forward produces nqpr x draft_vocab
 * float32 logits per round (15 x 248320 on the 27B lane); [SI441]
 * "Hypothesis": the lm_head is the last of the draft round's small-M GEMMs.
 *
 *   logits[m, v] = sum_{t < d} H[m, t] * W_lm[v, t]   m < rows, v < V
 *
 *   W_lm   bf16 [V, d]     16-byte aligned
 *   H      fp32 [rows, d]  16-byte aligned (rows = num_reqs * B)
 *   logits fp32 [rows, V]   4-byte aligned, overwritten
 * Same kernel family, sizes, errors and accuracy as dspark_proj_smallm.
 */
dspark_status dspark_lm_head(const uint16_t* W_lm, int V, int d, const float* H, int rows,
                             float* logits, void* stream);

/*
 * dspark_lm_head_sched -- dspark_lm_head with the weight rows handed out to
 * the workgroups by a counter instead of in equal shares, so that compute
 * units that stream faster take more of them (on MI355X the XCDs stream at
 * different rates: with equal shares the launch waits for the slowest).
 * Same product, arguments, sizes, errors and accuracy as dspark_lm_head;
 * the summation order of every logit is the same as with equal shares of
 * the same launch shape (it depends on the shape only), so results do not
 * depend on which workgroup computed which rows.
 *
 *   counter  device memory, one uint32, 4-byte aligned, caller-owned. It
 *            must read 0 before the first call (zero-fill it once); every
 *            call leaves it 0 again. Calls that share a counter must be
 *            ordered on one stream.
 * Applies where rows <= 8, d <= 4096 and the vocabulary is long enough to
 * give every compute unit more than 16 tiles of 16 rows (V > 256 x the
 * device's compute units); other shapes run dspark_lm_head's kernels and
 * leave the counter alone. dspark_draft_round runs its lm_head this way,
 * with a word of its workspace as the counter.
 * Errors: those of dspark_lm_head; DSPARK_ERR_NULL for a null counter,
 * DSPARK_ERR_ALIGN for a misaligned one.
 */
dspark_status dspark_lm_head_sched(const uint16_t* W_lm, int V, int d, const float* H, int rows,
                                   float* logits, uint32_t* counter, void* stream);

/*
 * dspark_lm_head_split -- dspark_lm_head for batched drafted rows
 * (rows > 16: several requests per round), with the hidden dimension split
 * into two halves that different workgroups multiply.
 *
 * [W7] "Measured": the reduced-vocabulary lane drafts 9 rows for each of
 * several requests, so its lm_head multiplies dozens of hidden rows by the
 * vocabulary; [SI441] "Hypothesis": such small-M products are bound by
 * reading the weights once. With all of its rows' activations beside each
 * weight tile, a compute unit reads about as many activation bytes as
 * weight bytes; splitting d in two halves the activation bytes per unit.
 *
 * Same product, arguments, sizes, errors and accuracy as dspark_lm_head.
 * Each logit is the sum of two fp32 partials, one per part of d (the first
 * ceil(ceil(d / 64) / 2) blocks of 64 entries, and the rest), each partial
 * summed in an order fixed by the shape; a sum of two terms does not depend
 * on which partial came first, so the result does not depend on timing.
 * (The logits differ from dspark_lm_head's by rounding only.)
 *
 *   workspace device memory of at least
 *             dspark_lm_head_split_workspace_bytes(V, d, rows) bytes,
 *             256-byte aligned, caller-owned: a ticket word per block of
 *             256 vocabulary rows, then the two halves' partial logits.
 *             ZERO-FILL IT ONCE before its first use; every call leaves
 *             the ticket words 0 again, so calls need no clearing between
 *             them. Calls that share a workspace must be ordered on one
 *             stream.
 * dspark_lm_head_split_workspace_bytes returns 0 where the split does not
 * apply (rows <= 16, or d > 2^21); the call then runs dspark_lm_head's
 * kernels and does not touch the workspace (which may be NULL).
 * Errors: those of dspark_lm_head; DSPARK_ERR_WORKSPACE for a missing or
 * smaller workspace, DSPARK_ERR_ALIGN for a misaligned one.
 */
size_t dspark_lm_head_split_workspace_bytes(int V, int d, int rows);
dspark_status dspark_lm_head_split(const uint16_t* W_lm, int V, int d, const float* H, int rows,
                                   float* logits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dspark_proj_smallm_q8, dspark_lm_head_q8 -- the same products over Q8_0
 * weights.
 *
 * [SI441] "Proposed work": the weight-stationary batched matvec it would
 * reuse targets quantized weights. [DS772] "Summary": the GPU path takes
 * Q8_0 weights. Q8_0 is read as the GGUF block format: entries 32b..32b+31
 * of a weight row share one IEEE binary16 scale d[n, b], and entry t is
 * d[n, t / 32] * q[n, t] with q a signed 8-bit integer. Here quants and
 * scales are two arrays (a GGUF tensor, whose blocks interleave them, is
 * split once when it is loaded).
 *
 *   Y[m, n] = sum_{t < K} X[m, t] * d[n, t / 32] * q[n, t]
 *
 *   Wq  int8   [N, K]       16-byte aligned
 *   Wd  binary16 bits [N, K / 32]  2-byte aligned
 *   X   fp32   [M, K]       16-byte aligned
 *   Y   fp32   [M, N]        4-byte aligned, overwritten
 * Sizes: N >= 1, K >= 32 with K % 32 == 0, K <= 4194304, M >= 1, and a
 * workgroup's quant rows (about N / CUs) times K bytes below 2 GiB
 * (DSPARK_ERR_SHAPE otherwise). The weights are read once per 16 rows of X.
 * Accuracy: X is split exactly into two bf16 terms (residual <= 2^-17 |x|),
 * the quants are exact in bf16, and each block's product is scaled and
 * added in fp32; the summation order depends on the shape only.
 */
dspark_status dspark_proj_smallm_q8(const int8_t* Wq, const uint16_t* Wd, int N, int K, const float* X, int M,
                                    float* Y, void* stream);
dspark_status dspark_lm_head_q8(const int8_t* Wq, const uint16_t* Wd, int V, int d, const float* H, int rows,
                                float* logits, void* stream);

/*
 * dspark_lm_head_q8_ld -- dspark_lm_head_q8 with scale rows ldd binary16
 * values apart (Wd [V, ldd]; the first d / 32 of each row are the scales,
 * the rest padding that is never read as a scale).
 *
 * A layout choice of the caller, made once when the weights are packed:
 * the computation is that of dspark_lm_head_q8 on the same values, bit for
 * bit. With rows padded to whole 128-byte lines (ldd a multiple of 64), no
 * line holds the scales of two rows, so none is fetched once per K phase of
 * each row that shares it (at d = 5120 a dense row's 320 bytes of scales
 * start mid-line on every other row).
 * Sizes: those of dspark_lm_head_q8, and d / 32 <= ldd <= d / 32 + 64
 * (DSPARK_ERR_SHAPE otherwise).
 */
dspark_status dspark_lm_head_q8_ld(const int8_t* Wq, const uint16_t* Wd, int ldd, int V, int d, const float* H,
                                   int rows, float* logits, void* stream);

/*
 * Bytes of device workspace dspark_markov_sample needs for these sizes
 * (0 when a size is out of range). The layout is the same for every valid
 * size (about 2 MiB), so one workspace serves calls of any shape.
 */
size_t dspark_markov_workspace_bytes(int num_reqs, int k, int V);

/*
 * dspark_markov_sample -- the k-step Markov-biased greedy loop on device.
 *
 * [W7] "The fix": for each step i the loop gathers markov_w1[prev], forms
 * the bias as markov_w2 times that row, adds the step's base-logit row,
 * takes the greedy argmax with the lowest index winning ties, maps the
 * token through d2t and keeps prev on the device; only the final
 * [num_reqs, k] ids are read back. "W7 LANDED": markov_w2 is
 * [draft_vocab, markov_rank] bf16 and is re-read by every step.
 *
 * For each request q < num_reqs, with prev = prev0[q]:
 *   for i < k:
 *     s[v]      = base[q, i, v] + sum_{j < r} w2[v, j] * w1[prev, j]
 *     tok       = min { v : s[v] == max_u s[u] }     (fp32 scores)
 *     ids[q, i] = d2t ? d2t[tok] : tok
 *     prev      = tok                                (draft vocabulary)
 *
 *   base      fp32  [num_reqs, B, V]   4-byte aligned
 *   w1, w2    bf16  [V, r]            16-byte aligned
 *   d2t       int64 [V] or NULL (identity); its entries are copied as given
 *   prev0     int64 [num_reqs], draft-vocabulary ids
 *   ids_out   int64 [num_reqs, k], overwritten
 *   workspace >= dspark_markov_workspace_bytes(num_reqs, k, V) bytes,
 *             8-byte aligned, owned by the caller. It must be ZERO-FILLED
 *             ONCE before its first use.
 * The workspace contract. Unlike plain scratch memory, this workspace
 * carries device-side state from one call to the next: the key slots of
 * the grid-wide exchange (two buffers; each call leaves the one it used for
 * the next call to clear), a call counter and a state word. That is what
 * lets a call start without a clearing launch in front of it. Hence:
 *   - zero-fill it once after allocation, and never write it yourself
 *     afterwards (a workspace zero-filled again at any point between calls
 *     is also valid);
 *   - calls that share a workspace must be ordered (one stream, or event
 *     dependencies); calls that overlap in time need workspaces of their
 *     own. One workspace serves calls of every shape and both weight
 *     formats;
 *   - the loop's workgroups exchange one key per step and must all be
 *     resident at once. The call checks that the grid fits an otherwise idle
 *     device (DSPARK_ERR_HIP otherwise); kernels of other streams may delay
 *     some workgroups, which the bounded waits absorb;
 *   - should a grid-wide wait still give up (other work holding compute
 *     units for longer than the bound, ~0.3 s of polling by default; see
 *     dspark_markov_set_spin_limit), every id of that call is -2. The next
 *     call on the workspace repairs it: it samples nothing, clears the key
 *     slots, and its ids are -2 as well. The call after that (and every
 *     later one) samples normally. No caller action is needed.
 * Sizes: 1 <= num_reqs <= 16, 1 <= k <= min(B, 32), V >= 1, 8 <= r <= 1024 with
 * r % 8 == 0. A request whose prev0 lies outside [0, V) gets -1 in every
 * entry of its ids row (a device-side check; nothing out of range is read).
 */
dspark_status dspark_markov_sample(const float* base, int num_reqs, int B, int V,
                                   const uint16_t* w1, const uint16_t* w2, int r,
                                   const int64_t* d2t, const int64_t* prev0, int k,
                                   int64_t* ids_out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * dspark_markov_sample_noalloc -- dspark_markov_sample without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * The loop's workspace is instead a static device array inside the library
 * (2 MiB + 256 bytes, the size dspark_markov_workspace_bytes returns for
 * every valid shape), one copy per GPU, set up on the first call on each
 * device (its address looked up once, then zero-filled by a small kernel on
 * `stream`) and held until the process ends. The call allocates nothing:
 * no hipMalloc, no hipFree, no allocating library routine.
 *
 * Arguments, sizes, results and errors are those of dspark_markov_sample
 * (the same kernel, bit-identical ids), minus workspace and
 * workspace_bytes; sizes beyond the array (num_reqs > 16 or k > 32) return
 * DSPARK_ERR_SHAPE before anything is enqueued, and a failed set-up returns
 * DSPARK_ERR_HIP. Every call on a GPU shares that GPU's array, which keeps
 * the last call's state, as a caller workspace does (see the workspace
 * contract above): calls on one GPU must be ordered (one stream, or event
 * dependencies); calls that overlap in time on one GPU race and give
 * undefined ids.
 */
dspark_status dspark_markov_sample_noalloc(const float* base, int num_reqs, int B, int V,
                                           const uint16_t* w1, const uint16_t* w2, int r,
                                           const int64_t* d2t, const int64_t* prev0, int k,
                                           int64_t* ids_out, void* stream);

/*
 * dspark_markov_set_spin_limit -- the bound of the Markov loop's grid-wide
 * waits, in polls (each a few hundred nanoseconds); 0 restores the default
 * (2^18 polls, ~0.3 s). Returns the previous setting. It applies to every
 * Markov launch enqueued afterwards by this process (a launch recorded into
 * a HIP graph keeps the value it was recorded with). It exists so that the
 * give-up path and the repair that follows it (see dspark_markov_sample)
 * can be exercised from the host: a bound of a few polls makes the waits of
 * an ordinary call give up. Every kernel still exits normally.
 */
uint32_t dspark_markov_set_spin_limit(uint32_t polls);

/*
 * dspark_conf_probe -- the proposer's confidence probe.
 *
 * [DS772] "Summary": one small kernel computes the probe on the drafted
 * row's hidden state and only a 4-byte scalar goes back to the host, which
 * decides whether to keep drafting.
 *
 *   logit[m] = sum_{t < D} w[t] * x[m, t] + bias
 *   pass[m]  = logit[m] >= threshold
 *
 *   x          fp32  [M, D]  16-byte aligned
 *   w          bf16  [D]     16-byte aligned
 *   logit_out  fp32  [M]      4-byte aligned
 *   pass_out   int32 [M] or NULL
 * Sizes: M >= 1, D >= 8 and D % 8 == 0. fp32 accumulation in a fixed order.
 */
dspark_status dspark_conf_probe(const float* x, int M, int D, const uint16_t* w, float bias,
                                float threshold, float* logit_out, int32_t* pass_out,
                                void* stream);

/*
 * dspark_markov_sample_probe -- dspark_markov_sample and dspark_conf_probe
 * in one launch.
 *
 * [W7] "The fix" for the loop and [DS772] "Summary" for the probe, as in
 * the two calls it replaces. The probe depends on nothing the loop computes;
 * it runs on the waves that finish the loop early (every workgroup but the
 * one that waits for the last step's winner), so it adds no launch and
 * almost no time to the round. Use it where the base logits come from
 * elsewhere (another lm_head implementation); dspark_draft_round is
 * dspark_lm_head followed by this call.
 *
 * Arguments: those of dspark_markov_sample, then those of dspark_conf_probe
 * (probe_x fp32 [probe_M, probe_D], probe_w bf16 [probe_D], ...), with the
 * same layouts, sizes, alignment and errors. Results are bit-identical to
 * the two separate calls.
 */
dspark_status dspark_markov_sample_probe(const float* base, int num_reqs, int B, int V,
                                         const uint16_t* w1, const uint16_t* w2, int r,
                                         const int64_t* d2t, const int64_t* prev0, int k,
                                         int64_t* ids_out, void* workspace, size_t workspace_bytes,
                                         const float* probe_x, int probe_M, int probe_D,
                                         const uint16_t* probe_w, float probe_bias,
                                         float probe_threshold, float* logit_out, int32_t* pass_out,
                                         void* stream);

/*
 * dspark_draft_round -- one whole draft round: lm_head, the Markov loop and
 * the confidence probe on every drafted row, in two launches.
 *
 * [W7] "The fix": the round is a composition of device primitives in which
 * only the final ids leave the device; the base logits stay in device
 * memory between the lm_head and the loop. [DS772] "Summary": the probe of
 * each drafted row is computed on the device as well and only its 4-byte
 * logit goes back.
 *
 * Equivalent to, in this order on `stream`,
 *   dspark_lm_head_sched(W_lm, V, d, H, num_reqs * B, base_out, <counter>)
 *     (dspark_lm_head_split(..., <split workspace>) when num_reqs * B > 16)
 *   dspark_markov_sample(base_out, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, ...)
 *   dspark_conf_probe(H, num_reqs * B, d, probe_w, probe_bias, probe_threshold, logit_out, pass_out)
 * and bit-identical to those three calls, <counter> being the uint32 at
 * byte 64 of the workspace (a control word the loop does not otherwise
 * use) and <split workspace> the bytes of the workspace past the first
 * dspark_markov_workspace_bytes(num_reqs, k, V). The probe runs inside the Markov loop's launch (as in
 * dspark_markov_sample_probe), so the round is two kernels instead of three.
 * A zero-filled workspace keeps that word 0 across rounds. If it is not 0
 * when the loop starts (a workspace that was never zero-filled), the
 * lm_head may have left base rows out: that round's ids are all -2 and the
 * word is set back to 0, so the next round is whole again. The split
 * lm_head (more than 16 rows) sets that word when it draws a ticket that
 * shows its own ticket words were not 0, with the same outcome; and the
 * loop sets those ticket words to 0 in every round, so a workspace that
 * was never zero-filled spoils its first round at most.
 *
 *   W_lm      bf16  [V, d]                 16-byte aligned
 *   H         fp32  [num_reqs * B, d]      16-byte aligned (hidden states, also the probe's x)
 *   w1, w2    bf16  [V, r]                 16-byte aligned
 *   d2t       int64 [V] or NULL
 *   prev0     int64 [num_reqs]
 *   probe_w   bf16  [d] or NULL (no probe; logit_out and pass_out are then ignored)
 *   base_out  fp32  [num_reqs, B, V]       4-byte aligned, overwritten (the base logits)
 *   ids_out   int64 [num_reqs, k]          overwritten
 *   logit_out fp32  [num_reqs * B]         overwritten (required when probe_w is given)
 *   pass_out  int32 [num_reqs * B] or NULL
 *   workspace at least dspark_draft_round_workspace_bytes(num_reqs, B, k, V, d)
 *             bytes, 256-byte aligned: the Markov loop's workspace, then
 *             (num_reqs * B > 16) the split lm_head's. Zero-filled once
 *             before first use; the contracts of dspark_markov_sample and
 *             dspark_lm_head_split.
 * Sizes and errors: those of the three calls above; every check is made
 * before anything is enqueued.
 */
size_t dspark_draft_round_workspace_bytes(int num_reqs, int B, int k, int V, int d);
dspark_status dspark_draft_round(const uint16_t* W_lm, int V, int d, const float* H, int num_reqs,
                                 int B, const uint16_t* w1, const uint16_t* w2, int r,
                                 const int64_t* d2t, const int64_t* prev0, int k,
                                 const uint16_t* probe_w, float probe_bias, float probe_threshold,
                                 float* base_out, int64_t* ids_out, float* logit_out,
                                 int32_t* pass_out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * dspark_markov_sample_q8 -- the Markov loop over Q8_0 markov weights, with
 * the confidence probe optionally in the same launch.
 *
 * [DS772] "Summary": the GPU path takes Q8_0 markov weights. Both markov_w1
 * and markov_w2 are Q8_0 with blocks along the rank: entry j of row v is
 * d[v, j / 32] * q[v, j] (IEEE binary16 scale, signed 8-bit quant). The loop
 * is that of dspark_markov_sample ([W7] "The fix") on these exact values:
 * each block's dot product is exact in integers (int8 matrix cores), then
 * scaled by the two block scales and added in fp32.
 *
 *   w1q, w2q  int8     [V, r]       16-byte aligned
 *   w1d, w2d  binary16 [V, r / 32]   2-byte aligned
 *   probe_x   NULL (no probe) or the probe's x as in dspark_conf_probe, with
 *             probe_M, probe_D, probe_w, probe_bias, probe_threshold,
 *             logit_out, pass_out (results bit-identical to that call)
 * Every other argument, the workspace rules and the errors are those of
 * dspark_markov_sample. Sizes: 32 <= r <= 256 with r % 32 == 0 (the register
 * and LDS budget of the int8 path); other limits as dspark_markov_sample.
 */
dspark_status dspark_markov_sample_q8(const float* base, int num_reqs, int B, int V, const int8_t* w1q,
                                      const uint16_t* w1d, const int8_t* w2q, const uint16_t* w2d, int r,
                                      const int64_t* d2t, const int64_t* prev0, int k, int64_t* ids_out,
                                      void* workspace, size_t workspace_bytes, const float* probe_x,
                                      int probe_M, int probe_D, const uint16_t* probe_w, float probe_bias,
                                      float probe_threshold, float* logit_out, int32_t* pass_out,
                                      void* stream);

/*
 * dspark_draft_round_q8 -- dspark_draft_round with a Q8_0 lm_head and Q8_0
 * markov weights: dspark_lm_head_q8, then dspark_markov_sample_q8 with the
 * probe (bf16 weights, optional as in dspark_draft_round) in the same
 * launch. Arguments, sizes and errors are those of the calls it composes.
 */
dspark_status dspark_draft_round_q8(const int8_t* Wq_lm, const uint16_t* Wd_lm, int V, int d, const float* H,
                                    int num_reqs, int B, const int8_t* w1q, const uint16_t* w1d,
                                    const int8_t* w2q, const uint16_t* w2d, int r, const int64_t* d2t,
                                    const int64_t* prev0, int k, const uint16_t* probe_w, float probe_bias,
                                    float probe_threshold, float* base_out, int64_t* ids_out,
                                    float* logit_out, int32_t* pass_out, void* workspace,
                                    size_t workspace_bytes, void* stream);
/* The same with the lm_head's scale rows ldd_lm apart (as dspark_lm_head_q8_ld). */
dspark_status dspark_draft_round_q8_ld(const int8_t* Wq_lm, const uint16_t* Wd_lm, int ldd_lm, int V, int d,
                                       const float* H, int num_reqs, int B, const int8_t* w1q,
                                       const uint16_t* w1d, const int8_t* w2q, const uint16_t* w2d, int r,
                                       const int64_t* d2t, const int64_t* prev0, int k,
                                       const uint16_t* probe_w, float probe_bias, float probe_threshold,
                                       float* base_out, int64_t* ids_out, float* logit_out,
                                       int32_t* pass_out, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * The rest of the draft block forward at small M.
 *
 * [SI441] "Observation": a draft block runs its projections (q/k/v/o,
 * gate/up/down: dspark_proj_smallm) and an attention over a short context
 * (AttentionBatchedRagged). The pages name nothing else of the block; these
 * entry points take the plainest reading of a transformer drafter derived
 * from Qwen3: RMSNorm before the attention and before the MLP, a SiLU-gated
 * MLP, residual additions, and multi-head attention without a position
 * encoding in which each draft position attends to its request's context and
 * to its own block. Each computes in fp32 with a fixed summation order.
 */

/*
 * dspark_rmsnorm: y[m, t] = x[m, t] / sqrt(mean_t x[m, t]^2 + eps) * gamma[t].
 *   x     fp32 [M, D]   16-byte aligned
 *   gamma bf16 [D]       2-byte aligned
 *   y     fp32 [M, D]   overwritten (may be x)
 * Sizes: M >= 1, D >= 1. eps >= 0.
 */
dspark_status dspark_rmsnorm(const float* x, int M, int D, const uint16_t* gamma, float eps, float* y,
                             void* stream);

/*
 * dspark_silu_gate: a[m, j] = silu(g) * u, g = gu[m, j], u = gu[m, F + j],
 * silu(g) = g / (1 + exp(-g)) (gu is the output of the fused gate/up
 * projection: gate columns first).
 *   gu fp32 [M, 2F];  a fp32 [M, F], overwritten.  Sizes: M >= 1, F >= 1.
 */
dspark_status dspark_silu_gate(const float* gu, int M, int F, float* a, void* stream);

/*
 * dspark_proj_smallm_add: Y = residual + X W^T (the o and down projections
 * with the block's residual addition in the same launch). Arguments, sizes
 * and errors are those of dspark_proj_smallm; residual fp32 [M, N], 4-byte
 * aligned, may be Y itself (each element is read before it is written).
 */
dspark_status dspark_proj_smallm_add(const uint16_t* W, int N, int K, const float* X, int M,
                                     const float* residual, float* Y, void* stream);

/*
 * dspark_proj_smallm_norm: Y = rmsnorm(X; gamma, eps) W^T, the RMSNorm of
 * dspark_rmsnorm fused into the projection it feeds (the qkv and gate/up
 * projections of a draft block, [SI441] "Observation"), so the normed
 * activations never go through memory and the norm costs no launch of its
 * own. Computed as (X * gamma) W^T, each output then scaled by its row's
 * factor 1 / sqrt(mean_k X[m, k]^2 + eps); the same products as the two
 * calls up to fp32 rounding (not bit for bit).
 *
 *   W      bf16 [N, K]   16-byte aligned
 *   X      fp32 [M, K]   16-byte aligned (the un-normed activations)
 *   gamma  bf16 [K]      16-byte aligned
 *   Y      fp32 [M, N]   4-byte aligned, overwritten
 * Sizes: those of dspark_proj_smallm, and only where its short kernel
 * applies: M <= 16, N >= 2, N * K * 2 < 2^31 and at most 16 tiles of 16 rows
 * per compute unit (N up to about 256 x the device's compute units).
 * dspark_proj_smallm_norm_fits(N, K, M) says whether a shape qualifies (1)
 * or not (0, and the call returns DSPARK_ERR_SHAPE); eps >= 0.
 * Errors: DSPARK_ERR_NULL, _SHAPE, _ALIGN, before anything is launched.
 */
int dspark_proj_smallm_norm_fits(int N, int K, int M);
dspark_status dspark_proj_smallm_norm(const uint16_t* W, int N, int K, const float* X, int M,
                                      const uint16_t* gamma, float eps, float* Y, void* stream);

/*
 * dspark_attention_ragged -- attention of the B draft positions of each of
 * R requests, H heads of Dh dimensions.
 *
 * Position i of request r, head h, attends to the request's first
 * ctx_len[r] context positions and to the positions of its own block (all B
 * of them, or j <= i when block_causal): scores q . k / sqrt(Dh), softmax
 * over those keys, output the weighted sum of their values.
 *
 *   q, k, v   fp32 [R * B, ld]: row r * B + i, head h at columns h * Dh ..
 *             (e.g. the three column blocks of the fused qkv projection with
 *             ld = 3 H Dh); 16-byte aligned, ld % 4 == 0
 *   k_ctx, v_ctx  bf16 [R, Lmax, H * Dh], 16-byte aligned (the context cache)
 *   ctx_len   int32 [R], each in [0, Lmax]
 *   out       fp32 [R * B, H * Dh], overwritten
 *   workspace device memory of at least dspark_attention_workspace_bytes(R,
 *             B, H, Dh, Lmax) bytes, 16-byte aligned: per-chunk partial
 *             results, fully written before they are read (no clearing
 *             needed); calls that share it must be ordered on one stream
 * Sizes: R >= 1, 1 <= B <= 16, H >= 1, 8 <= Dh <= 256 with Dh % 8 == 0,
 * 0 <= Lmax <= 2^30, R * H * ceil((Lmax + B) / 64) < 2^31.
 * The keys are taken 64 at a time (one workgroup each); each chunk's softmax
 * uses its own maximum and the chunks are merged in order with the exact
 * rescaling, so the context length is limited by the workspace only.
 * Errors: DSPARK_ERR_NULL, _SHAPE, _WORKSPACE, _ALIGN; nothing is launched
 * then.
 */
size_t dspark_attention_workspace_bytes(int num_reqs, int B, int H, int Dh, int Lmax);
dspark_status dspark_attention_ragged(const float* q, const float* k, const float* v, int ld, int R, int B,
                                      int H, int Dh, const uint16_t* k_ctx, const uint16_t* v_ctx,
                                      int Lmax, const int32_t* ctx_len, int block_causal, float* out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * dspark_draft_block -- one whole draft block (layer) at small M, as the
 * composition of the entry points above on one stream:
 *   qkv  = rmsnorm(h_in, ln1) W_qkv^T               (dspark_proj_smallm_norm)
 *   a    = attention(qkv, context)                  (dspark_attention_ragged)
 *   h2   = h_in + a W_o^T                           (dspark_proj_smallm_add)
 *   gu   = rmsnorm(h2, ln2) W_gate_up^T             (dspark_proj_smallm_norm)
 *   act  = silu(gu[:, :F]) * gu[:, F:]              (dspark_silu_gate)
 *   h_out = h2 + act W_down^T                       (dspark_proj_smallm_add)
 * where a projection's shape is outside dspark_proj_smallm_norm's (or its
 * norm weights are not 16-byte aligned), its norm is dspark_rmsnorm followed
 * by dspark_proj_smallm instead.
 * [SI441] "Observation" lists the block's projections (q/k/v/o, gate/up/down)
 * and its attention over a short context; the norms, the gated MLP and the
 * residuals are the plainest reading of a Qwen3-derived drafter. Results are
 * bit-identical to making those calls one by one (where the shape allows,
 * the gate runs in the gate/up projection's epilogue instead of a launch of
 * its own, computing the same values).
 *
 *   w_qkv      bf16 [3 H Dh, d]: q rows, then k rows, then v rows
 *   w_o        bf16 [d, H Dh]
 *   w_gate_up  bf16 [2F, d]: gate rows, then up rows
 *   w_down     bf16 [d, F]
 *   ln1, ln2   bf16 [d]
 *   h_in       fp32 [num_reqs * B, d]; h_out fp32 [num_reqs * B, d], may be h_in
 *   k_ctx, v_ctx, Lmax, ctx_len, block_causal   as for dspark_attention_ragged
 *   workspace  at least dspark_draft_block_workspace_bytes(...) bytes, 256-byte
 *              aligned, caller-owned; holds the intermediate activations, no
 *              clearing needed; calls that share it must be ordered
 * Alignment: weights, h_in, h_out, k_ctx, v_ctx 16 bytes; ln1, ln2 2 bytes.
 * Sizes: d % 8 == 0, F % 8 == 0, the attention's limits, and every
 * projection within dspark_proj_smallm's. eps >= 0.
 * Errors: DSPARK_ERR_NULL, _SHAPE, _WORKSPACE, _ALIGN before anything is
 * enqueued; DSPARK_ERR_HIP if a launch fails (earlier launches of the call
 * stay enqueued).
 */
size_t dspark_draft_block_workspace_bytes(int num_reqs, int B, int H, int Dh, int d, int F, int Lmax);
dspark_status dspark_draft_block(const uint16_t* w_qkv, const uint16_t* w_o, const uint16_t* w_gate_up,
                                 const uint16_t* w_down, const uint16_t* ln1, const uint16_t* ln2, int d,
                                 int F, int H, int Dh, int num_reqs, int B, const float* h_in, float* h_out,
                                 const uint16_t* k_ctx, const uint16_t* v_ctx, int Lmax,
                                 const int32_t* ctx_len, float eps, int block_causal, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * dspark_stream_read -- a measurement aid, not a step of the method: a
 * plain streaming read of `bytes` bytes at `buf` by `groups` workgroups of
 * `threads` threads, workgroup b reading the b-th contiguous share with
 * 16-byte non-temporal loads and writing one word (a fold of what it read)
 * to sink[b]. It measures the device's HBM read ceiling at a given launch
 * shape, beside the round's kernels, in the same run; the pages judge the
 * round's GEMVs against a bandwidth bound ([W7] "W7 LANDED"; [SI441]
 * "Observation"). With bytes == 0 it is an empty launch (the launch-latency
 * floor).
 *   buf   device memory, 16-byte aligned (may be NULL when bytes == 0)
 *   sink  uint32 [groups], device memory, overwritten
 * Sizes: bytes % 16 == 0, 1 <= groups <= 65536, threads 256, 512 or 1024.
 */
dspark_status dspark_stream_read(const void* buf, size_t bytes, int groups, int threads, uint32_t* sink,
                                 void* stream);

/*
 * dspark_stream_read_sched -- the same read with dspark_lm_head_sched's
 * schedule: 256 KB units, a contiguous run of 90% of an equal share per
 * workgroup, the rest taken from `counter` (one uint32 of device memory,
 * 4-byte aligned, reading 0 before the call and left 0 by it; calls that
 * share it must be ordered). It measures the ceiling that lm_head streams
 * against. sink[b] is workgroup b's fold of what it read; the fold over all
 * workgroups equals dspark_stream_read's. Sizes: as dspark_stream_read, and
 * bytes < 2^30 units of 256 KB. Errors: DSPARK_ERR_NULL, _SHAPE, _ALIGN.
 */
dspark_status dspark_stream_read_sched(const void* buf, size_t bytes, int groups, int threads, uint32_t* counter,
                                       uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
