/*
 * librat -- the RAT+ temporal-mixing operator on AMD MI355X (gfx950).
 *
 * The operator ("RAT+: Train Dense, Infer Sparse -- Recurrence Augmented
 * Attention for Dilated Inference", abstract and Figs. 1-2; "Augmenting
 * Attention with Exponentially Decaying Memory Improves Query-Aware KV
 * Sparsity", sections 2.1-2.2) has two parts:
 *
 *   1. a full-sequence, per-channel gated linear recurrence over keys and
 *      values (an exponentially decaying memory with an input-dependent gate):
 *          g_t = sigmoid(z_t),   h_t = g_t * h_{t-1} + (1 - g_t) * x_t;
 *   2. softmax attention of each query t over the recurrent states on the
 *      dilated grid { j <= t : (j + 1) mod D == 0 } plus, optionally, the
 *      local window { max(0, t - W + 1) .. t } (a set: counted once), in a
 *      prefill form and a one-token decode form.  A query with no key yields
 *      a zero output.  The dilation D may differ per head.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, 0-based.  Token tensors are
 *     [B][T][H][Dh] with Dh innermost; Dh must be 64 or 128; H <= 128.
 *   - Every buffer argument is DEVICE memory owned by the caller, 16-byte
 *     aligned.  Array arguments documented as "host" are host memory and are
 *     read before the call returns.  The library never allocates, frees or
 *     synchronizes; scratch comes from the caller's workspace.
 *   - A workspace must be zero-filled once before its first use (e.g. with
 *     hipMemset) and may then be reused by any number of calls issued in
 *     stream order.  Two calls that run concurrently need two workspaces.
 *     Its first 256 bytes are a header; the 32-bit word at byte offset 8 is a
 *     sticky error word: bit 1 = a decode position was outside [0, max_pos)
 *     (that sequence's output is zero and its cache is untouched).  Zero the
 *     word to reset it.  The 32-bit word at byte offset 12 is the recurrence
 *     scan's look-back poll limit, written by the caller (never by the
 *     library): 0, as zero-filled, selects the default; n > 0 makes a scan
 *     block wait at most n - 1 polls for an earlier chunk's published carry
 *     before it computes that chunk's aggregate itself from the inputs (the
 *     results agree up to fp32 rounding; n = 1 takes that path on every
 *     wait, which the tests use to exercise it).  Every entry point that
 *     runs a scan reads it: rat_scan, rat_dilated_prefill(_stage),
 *     rat_prefill_chunk, rat_local_prefill_chunk, rat_topk_prefill.  Nothing
 *     else in the library depends on state outside the call's arguments.
 *   - All work is asynchronous on `stream`.  The returned status covers
 *     argument validation (done on the host before any HIP call) and launch
 *     errors; device faults surface at the caller's next synchronization.
 *     On an error return nothing was launched unless the status is
 *     RAT_ERR_HIP.  No exception crosses the ABI.
 *   - dtype RAT_BF16: q, k, v, states, caches and outputs are bf16
 *     (round-to-nearest-even), every accumulation is fp32.  RAT_F32: all of
 *     them are fp32.  Gate logits, recurrent states handed between calls and
 *     h0 / h_last are always fp32.
 */
#ifndef RAT_H_
#define RAT_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RAT_OK = 0,
  RAT_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned buffer */
  RAT_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. Dh = 96) */
  RAT_ERR_WORKSPACE = -3,    /* ws_bytes smaller than the *_workspace_size */
  RAT_ERR_HIP = -4           /* a HIP launch failed; see rat_last_error() */
} rat_status_t;

typedef enum { RAT_F32 = 0, RAT_BF16 = 1 } rat_dtype_t;

#define RAT_MAX_HEADS 128

/* Human-readable name of a status code (static string). */
const char* rat_status_string(rat_status_t status);

/* Detail of the last error on the calling thread (thread-local, static
 * storage; empty string if none). */
const char* rat_last_error(void);

/* ------------------------------------------------------------------------ *
 * rat_scan -- the gated recurrence alone (part 1 above; the recurrence is
 * full-sequence, L = T: RAT+ Fig. 1a; memory update: follow-up page,
 * section 2.1).
 *
 *   x       [B][T][H][Dh]  dtype         inputs (keys or values)
 *   z       [B][T][H][Dh]  fp32          gate logits (g = sigmoid(z);
 *                                        1 - g is evaluated as sigmoid(-z);
 *                                        +-inf allowed)
 *   h0      [B][H][Dh]     fp32 or NULL  state before position 0 (NULL: 0)
 *   states  [B][T/E][H][Dh] dtype or NULL, E = store_every >= 1: entry i
 *           holds h at position (i + 1) * E - 1, i.e. every state at a
 *           position j with (j + 1) mod E == 0 (E = 1: all states; E = D:
 *           the dilated grid)
 *   h_last  [B][H][Dh]     fp32 or NULL  state at position T - 1
 *   ws      workspace of at least rat_scan_workspace_size(B, T, H, Dh) bytes:
 *           the look-back words through which chunks of the sequence hand
 *           their carries to later chunks (the one-pass scan needs them; the
 *           caller owns them so that the library never allocates)
 * T = 0 is a no-op (buffers may then be NULL).  States and h_last come from
 * one fp32 carry chain.
 * ------------------------------------------------------------------------ */
size_t rat_scan_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh);
rat_status_t rat_scan(const void* x, const float* z, const float* h0, void* states,
                      int32_t store_every, float* h_last, int32_t B, int32_t T, int32_t H,
                      int32_t Dh, rat_dtype_t dtype, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * rat_dilated_prefill -- the whole operator over a sequence (RAT+ abstract:
 * dilated attention over every D-th recurrent state with an optional local
 * window, per-head dilation allowed; Fig. 1c).
 *
 *   q, k, v   [B][T][H][Dh] dtype
 *   zk, zv    [B][T][H][Dh] fp32   gate logits for keys and for values
 *   out       [B][T][H][Dh] dtype  o_t = sum_{j in S_t} softmax_j(scale *
 *                                  <q_t, k~_j>) v~_j  (0 if S_t is empty)
 *   dilation  host [H]  D per head, D >= 1 (D = 1: causal attention over
 *                       the recurrent states)
 *   W         window >= 0 (0: grid only)
 *   scale     softmax scale; <= 0 selects 1/sqrt(Dh)
 *   ws        workspace of at least rat_dilated_prefill_workspace_size(...)
 *             bytes; it receives the recurrent states
 * The recurrence starts from zero state.  T = 0 is a no-op (buffers may
 * then be NULL).  bf16 sequences are limited to 2^31 / Dh positions
 * (16777216 for Dh = 128): the attention addresses the transposed value rows
 * with 32-bit offsets; longer ones -> RAT_ERR_UNSUPPORTED before anything
 * runs.
 * ------------------------------------------------------------------------ */
size_t rat_dilated_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh,
                                          const int32_t* dilation, int32_t W,
                                          rat_dtype_t dtype);
rat_status_t rat_dilated_prefill(const void* q, const void* k, const void* v, const float* zk,
                                 const float* zv, void* out, int32_t B, int32_t T, int32_t H,
                                 int32_t Dh, const int32_t* dilation, int32_t W, float scale,
                                 rat_dtype_t dtype, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* The same operation split into its two stages, for callers that schedule
 * or time them separately.  RAT_STAGE_RECURRENCE runs the scan of keys and
 * values into the workspace; RAT_STAGE_ATTENTION runs the attention from a
 * workspace that a RECURRENCE stage with identical arguments filled earlier
 * in stream order; RAT_STAGE_ALL equals rat_dilated_prefill. */
typedef enum {
  RAT_STAGE_ALL = 0,
  RAT_STAGE_RECURRENCE = 1,
  RAT_STAGE_ATTENTION = 2
} rat_prefill_stage_t;
rat_status_t rat_dilated_prefill_stage(rat_prefill_stage_t stage, const void* q, const void* k,
                                       const void* v, const float* zk, const float* zv, void* out,
                                       int32_t B, int32_t T, int32_t H, int32_t Dh,
                                       const int32_t* dilation, int32_t W, float scale,
                                       rat_dtype_t dtype, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Decode cache layout helper.  The grid cache of head h holds grid_cap[h]
 * entries per sequence, entry i = the state at position (i + 1) * D_h - 1;
 * all heads share one buffer: head h occupies elements
 * [B * grid_off[h] * Dh, B * (grid_off[h] + grid_cap[h]) * Dh), laid out
 * [B][grid_cap[h]][Dh].  This fills grid_off / grid_cap (host [H]) with the
 * packed layout of capacity max_pos / D_h per head and returns the total
 * rows per sequence in *rows (so the buffer holds B * rows * Dh elements).
 * ------------------------------------------------------------------------ */
rat_status_t rat_grid_layout(int32_t H, const int32_t* dilation, int64_t max_pos,
                             int64_t* grid_off, int32_t* grid_cap, int64_t* rows);

/* ------------------------------------------------------------------------ *
 * rat_prefill_chunk -- prefill positions p0 .. p0+T-1 of sequences whose
 * positions 0 .. p0-1 are held in a decode cache, and extend that cache to
 * positions 0 .. p0+T-1 (the prefill-then-decode serving of RAT+ Fig. 2;
 * key sets as in the abstract and Fig. 1c, with the grid at absolute
 * positions).  With p0 = 0 and zero states it is a prefill that leaves the
 * decode cache behind; a sequence split into chunks gets the outputs of one
 * call over the whole sequence, up to the fp32 rounding of the state
 * carried between chunks.
 *
 *   q, k, v, zk, zv, out  as rat_dilated_prefill, for the T rows of the
 *                         chunk (row t is position p0 + t)
 *   state_k/_v   [B][H][Dh] fp32, in/out: the state after position p0-1
 *                (zeros when p0 = 0) -> the state after position p0+T-1
 *   grid_k/_v    ragged grid caches (layout of rat_grid_layout), dtype,
 *                in/out: entries of positions before p0 are read, entries
 *                of positions p0 .. p0+T-1 written
 *   grid_off, grid_cap  host [H]: their layout; grid_cap[h] >= max_pos / D_h
 *   ring_k/_v    [B][H][W][Dh] dtype, in/out (NULL allowed when W = 0): the
 *                slots of positions p0-W+1 .. p0-1 are read, the slots of
 *                the chunk's last min(W, T) positions written
 *   p0           first position of the chunk, the same for every sequence;
 *                a multiple of 64
 *   max_pos      cache capacity in positions; p0 + T <= max_pos < 2^31
 *   dilation, W, scale  as rat_dilated_prefill (W is the ring length)
 *   ws           workspace of at least rat_prefill_chunk_workspace_size(...)
 *                bytes (scratch only: nothing in it is read by a later call)
 * Errors: p0 not a multiple of 64 -> RAT_ERR_UNSUPPORTED; p0 < 0,
 * p0 + T > max_pos or a grid capacity below max_pos / D_h ->
 * RAT_ERR_INVALID_ARG; bf16 with the chunk's window rows or a head's visible
 * grid above 2^31 / Dh keys -> RAT_ERR_UNSUPPORTED (as rat_dilated_prefill).
 * T = 0 is a no-op (buffers may then be NULL).
 * ------------------------------------------------------------------------ */
size_t rat_prefill_chunk_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh,
                                        const int32_t* dilation, int32_t W, int64_t p0,
                                        rat_dtype_t dtype);
rat_status_t rat_prefill_chunk(const void* q, const void* k, const void* v, const float* zk,
                               const float* zv, void* out, float* state_k, float* state_v,
                               void* grid_k, void* grid_v, const int64_t* grid_off,
                               const int32_t* grid_cap, void* ring_k, void* ring_v, int64_t p0,
                               int64_t max_pos, int32_t B, int32_t T, int32_t H, int32_t Dh,
                               const int32_t* dilation, int32_t W, float scale, rat_dtype_t dtype,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * rat_decode_step -- one new token per sequence (RAT+ Fig. 2: step update of
 * the recurrence, attention over the cached states; abstract: the grid
 * cache is D times smaller than a dense cache).
 *
 * For every sequence b at position t = pos[b] and head h (dilation D):
 *   1. state <- g * state + (1 - g) * x for keys and values (fp32);
 *   2. if W > 0: ring slot t mod W <- the new state (in dtype);
 *   3. if (t + 1) mod D == 0: grid entry (t + 1) / D - 1 <- the new state;
 *   4. out = softmax attention of q over grid entries i < max(0,t-W+1)/D
 *      (strictly older than the window when W > 0) and the ring slots of
 *      positions max(0, t - W + 1) .. t.
 * A cache filled by prefilling positions 0 .. t-1 makes this equal to row t
 * of a prefill over t + 1 tokens.
 *
 *   q, k, v      [B][H][Dh] dtype   the new token
 *   zk, zv       [B][H][Dh] fp32    its gate logits
 *   state_k/_v   [B][H][Dh] fp32    in/out recurrent states
 *   grid_k/_v    ragged grid caches (layout above), dtype, in/out
 *   grid_off     host [H], grid_cap host [H]: the layout; grid_cap[h] must
 *                be >= max_pos / D_h
 *   ring_k/_v    [B][H][W][Dh] dtype, in/out (NULL allowed when W = 0)
 *   pos          device int32 [B], read-only; every pos[b] must lie in
 *                [0, max_pos) (others: error bit 1, zero output)
 *   out          [B][H][Dh] dtype
 *   dilation     host [H]
 *   ws           workspace of at least rat_decode_workspace_size(...) bytes
 * The caller advances pos between steps.
 * ------------------------------------------------------------------------ */
size_t rat_decode_workspace_size(int32_t B, int32_t H, int32_t Dh, const int32_t* dilation,
                                 int32_t W, int64_t max_pos);
rat_status_t rat_decode_step(const void* q, const void* k, const void* v, const float* zk,
                             const float* zv, float* state_k, float* state_v, void* grid_k,
                             void* grid_v, const int64_t* grid_off, const int32_t* grid_cap,
                             void* ring_k, void* ring_v, const int32_t* pos, int64_t max_pos,
                             void* out, int32_t B, int32_t H, int32_t Dh,
                             const int32_t* dilation, int32_t W, float scale, rat_dtype_t dtype,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * rat_decode_step_noalloc -- rat_decode_step without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * operation, arguments and kernels as rat_decode_step; its scratch (the
 * split-K partials) is a fixed array of RAT_DECODE_SCRATCH_BYTES that the
 * library holds in each GPU's memory from load until the process ends.  The
 * call allocates nothing.
 *   - A step whose rat_decode_workspace_size(...) exceeds
 *     RAT_DECODE_SCRATCH_BYTES returns RAT_ERR_WORKSPACE before anything
 *     runs (the hybrid-head batch-128 decode at context 131072 needs about
 *     21 MB).
 *   - `stream` must belong to the current device (else
 *     RAT_ERR_INVALID_ARG); the first call on a device looks up that
 *     device's scratch address.
 *   - Every call on a GPU shares that GPU's scratch: calls that overlap on
 *     one GPU (concurrent streams, threads) race and must be serialised by
 *     the caller.  Nothing in the scratch needs to start at zero.
 *   - A position outside [0, max_pos) still yields a zero output and leaves
 *     that sequence's cache untouched; its sticky error bit lands in the
 *     scratch, which the caller cannot read (use rat_decode_step with a
 *     workspace to observe it).
 * ------------------------------------------------------------------------ */
#define RAT_DECODE_SCRATCH_BYTES (32u << 20)
rat_status_t rat_decode_step_noalloc(const void* q, const void* k, const void* v, const float* zk,
                                     const float* zv, float* state_k, float* state_v, void* grid_k,
                                     void* grid_v, const int64_t* grid_off, const int32_t* grid_cap,
                                     void* ring_k, void* ring_v, const int32_t* pos, int64_t max_pos,
                                     void* out, int32_t B, int32_t H, int32_t Dh,
                                     const int32_t* dilation, int32_t W, float scale, rat_dtype_t dtype,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * RAT's chunk-local variant ("RAT: Bridging RNN Efficiency and Attention
 * Accuracy via Chunk-based Sequence Modeling", approach): the recurrence runs
 * inside chunks of L positions, restarting from a zero state at every
 * position j with j mod L == 0 (L = T is the RAT+ recurrence, RAT+ Fig. 1a),
 * and each query attends over the final states of the earlier chunks plus
 * its own state: the RAT+ key set with D = L and W = 1.  The arguments are
 * those of rat_prefill_chunk / rat_decode_step with dilation L on every head
 * and W = 1 (ring_k/_v [B][H][1][Dh]; grid layout rat_grid_layout(H, L...));
 * L >= 1.
 * ------------------------------------------------------------------------ */
size_t rat_local_prefill_chunk_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh, int32_t L,
                                              int64_t p0, rat_dtype_t dtype);
rat_status_t rat_local_prefill_chunk(const void* q, const void* k, const void* v, const float* zk,
                                     const float* zv, void* out, float* state_k, float* state_v,
                                     void* grid_k, void* grid_v, const int64_t* grid_off,
                                     const int32_t* grid_cap, void* ring_k, void* ring_v, int64_t p0,
                                     int64_t max_pos, int32_t B, int32_t T, int32_t H, int32_t Dh,
                                     int32_t L, float scale, rat_dtype_t dtype, void* ws,
                                     size_t ws_bytes, hipStream_t stream);
size_t rat_local_decode_workspace_size(int32_t B, int32_t H, int32_t Dh, int32_t L, int64_t max_pos);
rat_status_t rat_local_decode_step(const void* q, const void* k, const void* v, const float* zk,
                                   const float* zv, float* state_k, float* state_v, void* grid_k,
                                   void* grid_v, const int64_t* grid_off, const int32_t* grid_cap,
                                   void* ring_k, void* ring_v, const int32_t* pos, int64_t max_pos,
                                   void* out, int32_t B, int32_t H, int32_t Dh, int32_t L, float scale,
                                   rat_dtype_t dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Top-k block attention over the memory states ("Augmenting Attention with
 * Exponentially Decaying Memory Improves Query-Aware KV Sparsity", sections
 * 2.2 and 3; RAT+ Fig. 3 and Tables 17-18).  Positions are cut into blocks of
 * `block` positions.  A query at position t attends over the recurrent
 * states of the first block, of its own block (up to t) and of the `topk`
 * complete blocks between them with the highest scores (all of them when
 * there are at most topk; ties go to the lower block index):
 *   RAT_TOPK_QUEST  score = sum_d max(q_d * min_d, q_d * max_d) over the
 *                   dimension-wise min / max of the block's key states;
 *   RAT_TOPK_MOBA   score = q . mean of the block's key states.
 *
 * Caches (device, caller-owned):
 *   cache_k/_v  every recurrent state, dtype, [H][B][max_pos][Dh] (the grid
 *               layout of rat_grid_layout with dilation 1 on every head)
 *   summary     fp32 [H][B][max_pos / block][3][Dh]: min, max and mean of
 *               the key states of each complete block
 *   state_k/_v  fp32 [B][H][Dh]: the state after the last cached position
 *               (zeros before the first call)
 * Limits: 1 <= block <= 1024, 0 <= topk <= 128, max_pos / block <= 8192,
 * max_pos < 2^31.
 *
 * chosen (device int32, optional): per query the selected blocks in
 * ascending order, -1 in unused slots.
 * ------------------------------------------------------------------------ */
typedef enum { RAT_TOPK_QUEST = 0, RAT_TOPK_MOBA = 1 } rat_topk_score_t;

/* Prefill positions p0 .. p0+T-1 (any p0 >= 0, p0 + T <= max_pos) of
 * sequences whose positions before p0 are cached: recurrence from state_k/_v,
 * every new state into the caches, summaries of the blocks completed, then
 * top-k block attention for every row.  q, k, v, zk, zv, out as
 * rat_dilated_prefill; chosen [B][T][H][topk] or NULL.  bf16 calls with
 * block = 64, topk <= 16 and p0 = 0 select first and then run the MFMA
 * prefill attention over the cache with the per-query block sets (the
 * workspace then also holds the transposed values and the chosen lists);
 * other calls, and sequences past 2^31 / Dh positions, take one workgroup
 * per query. */
size_t rat_topk_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh);
rat_status_t rat_topk_prefill(const void* q, const void* k, const void* v, const float* zk,
                              const float* zv, void* out, int32_t* chosen, float* state_k,
                              float* state_v, void* cache_k, void* cache_v, float* summary,
                              int64_t p0, int64_t max_pos, int32_t B, int32_t T, int32_t H,
                              int32_t Dh, int32_t block, int32_t topk, rat_topk_score_t score,
                              float scale, rat_dtype_t dtype, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* Summaries (min, max, mean of the key states) of blocks j_lo .. j_hi-1 of
 * every (h, b) from cache_k, e.g. for a cache filled by other means;
 * 0 <= j_lo <= j_hi <= max_pos / block. */
rat_status_t rat_topk_summarize(const void* cache_k, float* summary, int64_t j_lo, int64_t j_hi,
                                int64_t max_pos, int32_t B, int32_t H, int32_t Dh, int32_t block,
                                rat_dtype_t dtype, hipStream_t stream);

/* One new token per sequence at position pos[b] (device int32 [B], every
 * entry in [0, max_pos), others: error bit 1 and a zero output): state
 * update, cache row pos[b], the summary of a block that row completes, then
 * top-k block attention of q.  q, k, v [B][H][Dh] dtype; zk, zv fp32; out
 * [B][H][Dh]; chosen [B][H][topk] or NULL; ws of at least
 * rat_topk_decode_workspace_size() bytes (its header carries the error word). */
size_t rat_topk_decode_workspace_size(void);
rat_status_t rat_topk_decode_step(const void* q, const void* k, const void* v, const float* zk,
                                  const float* zv, float* state_k, float* state_v, void* cache_k,
                                  void* cache_v, float* summary, const int32_t* pos,
                                  int64_t max_pos, void* out, int32_t* chosen, int32_t B, int32_t H,
                                  int32_t Dh, int32_t block, int32_t topk, rat_topk_score_t score,
                                  float scale, rat_dtype_t dtype, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RAT_H_ */
