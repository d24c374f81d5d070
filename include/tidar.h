/*
 * tidar.h -- C ABI of the TiDAR decode-step hot path on MI355X (gfx950).
 *
 * One TiDAR decode step is a single forward pass whose query block holds,
 * per sequence, the k draft candidates carried over from the previous step
 * and k groups of k blank slots, one group for each verification outcome
 * ("TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de manière
 * autorégressive", nodesdaily.com, paragraphs on the three zones and on
 * drafting for every outcome).  The three calls below are the hot path of
 * that step: the structured-mask attention of one layer, greedy verification
 * of the candidates with selection of the next drafts, and the KV-cache
 * commit / evict.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers, row-major, 16-byte aligned.
 *     The caller owns every buffer; the library never allocates, frees or
 *     keeps state between calls, and never synchronises the device.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream).  Calls are re-entrant across streams and buffers.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a negative status and enqueues nothing.  A launch
 *     failure reported by the runtime returns TIDAR_ELAUNCH.  Faults inside
 *     kernels surface at the caller's next synchronisation, as usual in HIP.
 *   - bf16 means IEEE bfloat16 (round-to-nearest-even on output); f32 means
 *     IEEE binary32.  Attention accumulates in f32 for both.
 *
 * Step block layout (a reading of the pages, which fix no layout):
 *   R = k + n_groups*k rows per sequence, n_groups in {0, k}.
 *   Row i < k            : candidate i (position L+i).
 *   Row k + g*k + s      : slot s of group g, the group for the outcome
 *                          "candidates 0..g survive" (position L+g+1+s).
 *   Query head h reads KV head h / (Hq/Hkv).
 */
#ifndef TIDAR_H
#define TIDAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Positions per value-cache page: the value cache of every (sequence, KV
 * head) is S_max/TIDAR_VALUE_PAGE pages of [D][TIDAR_VALUE_PAGE], i.e. each
 * page of 64 consecutive positions is stored transposed (position fastest).
 * Key tiles of 64 positions and value pages are then both contiguous 16 KB
 * blocks for D = 128. */
#define TIDAR_VALUE_PAGE 64

enum {
  TIDAR_OK = 0,
  TIDAR_EINVAL = -1,       /* bad shape, pointer, alignment or value */
  TIDAR_EUNSUPPORTED = -2, /* valid request outside what is built (dtype, D, k) */
  TIDAR_EWORKSPACE = -3,   /* workspace missing or smaller than required */
  TIDAR_ELAUNCH = -4       /* the HIP runtime refused a launch */
};

enum { TIDAR_BF16 = 0, TIDAR_F32 = 1 };

/* Human-readable text for a status code (static storage, never NULL). */
const char* tidar_strerror(int status);

/* ABI version of this header (incremented on any signature change). */
int tidar_abi_version(void);

/* ------------------------------------------------------------------------
 * Step attention of one layer.
 *
 * Computes, for every sequence b, query head h and step row r,
 *   out[b][r][h] = softmax_c(sm_scale * q[b][r][h] . key_c) . value_c
 * over the keys visible to row r (the three-zone mask: paragraph on masking
 * of the nodesdaily.com page, section "2. Single Forward Pass & Structured
 * Attention Mask" of "TiDAR: Think in Diffusion, Talk in Autoregression",
 * mauroscia.it):
 *   - every row sees settled positions 0..lens[b]-1 (from the caches);
 *   - candidate i sees step rows 0..i (strictly causal scoring);
 *   - slot (g, s) sees step rows 0..g and the k rows of its own group g.
 * The mask is evaluated arithmetically, never materialised.  Keys are split
 * into chunks of `kv_chunk` positions of the [prefix ; step] sequence, each
 * chunk reduced on its own and merged with a log-sum-exp rescale.
 *
 *   dtype      TIDAR_BF16 or TIDAR_F32, the element type of q, k_step,
 *              v_step, k_cache, v_cache and out.
 *   B, Hq, Hkv, D   batch, query heads, KV heads (Hq % Hkv == 0), head dim
 *              (64 or 128).
 *   S_max      cache capacity per (b, KV head); a multiple of 64.
 *   max_len    host-side upper bound on every lens[b] (0 <= max_len <=
 *              S_max); sizes the launch without a device sync.  A sequence
 *              whose lens[b] exceeds it (or is negative) gets NaN outputs.
 *   k          number of candidates, 1..16;  n_groups: 0 or k.
 *   sm_scale   softmax scale (> 0), e.g. 1/sqrt(D).
 *   kv_chunk   key positions per chunk; 0 lets the library choose.  Must be
 *              a multiple of 64 otherwise (at most 1024 for TIDAR_F32).
 *   q          [B][R][Hq][D]
 *   k_step, v_step  [B][R][Hkv][D]   keys/values of the step rows (RoPE
 *              already applied by the caller).
 *   k_cache    [B][Hkv][S_max][D]    settled keys; rows >= lens[b] unused.
 *   v_cache    [B][Hkv][S_max/64][D][64]  settled values in pages of 64
 *              positions, each page stored TRANSPOSED: the value of
 *              position p, element d, is at [b][h][p/64][d][p%64].
 *              Positions >= lens[b] unused.
 *   lens       [B] int32 settled length per sequence (device memory).
 *   out        [B][R][Hq][D]         (written).
 *   lse        [B][Hq][R] f32, natural-log softmax denominator of
 *              sm_scale*q.k over visible keys (written); may be NULL.
 *   workspace  device scratch (256-byte aligned) of at least the size
 *              reported by tidar_step_attention_workspace() for the same
 *              arguments; may be NULL when that size is 0 (every sequence
 *              fits one key chunk, bf16).
 * ---------------------------------------------------------------------- */
int tidar_step_attention_workspace(int dtype, int B, int Hq, int Hkv, int D, int S_max, int max_len,
                                   int k, int n_groups, int kv_chunk, size_t* bytes);

/* The launch plan tidar_step_attention would use for these arguments (a
 * host-only query, nothing is enqueued): plan[0] kernel (0: four waves per
 * workgroup, one per SIMD; 1: eight waves, two per SIMD; 2: the f32
 * kernel), plan[1] full 16-row tiles per wave, plan[2] tiles shared by the
 * waves of a workgroup, plan[3] workgroups per (sequence, KV head) over the
 * rows, plan[4] key positions per chunk, plan[5] chunks.  `plan` is a host
 * array of 6 ints owned by the caller.  Returns the status the workspace
 * query returns for the same arguments.  The environment variable
 * TIDAR_ATTN_KERNEL ("pp" for the eight-wave kernel, "pipe" for the
 * four-wave one; read at every call) restricts the choice, for tests and
 * measurements that compare the two. */
int tidar_step_attention_plan(int dtype, int B, int Hq, int Hkv, int D, int S_max, int max_len,
                              int k, int n_groups, int kv_chunk, int* plan);

int tidar_step_attention(int dtype, int B, int Hq, int Hkv, int D, int S_max, int max_len,
                         int k, int n_groups, float sm_scale, int kv_chunk,
                         const void* q, const void* k_step, const void* v_step,
                         const void* k_cache, const void* v_cache, const int32_t* lens,
                         void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * Step attention over a paged (block-table) KV cache.
 *
 * The same computation as tidar_step_attention, with the settled keys and
 * values held in pages of 64 positions drawn from shared pools, so
 * sequences of very different lengths share one allocation.  The pages call
 * the design serving-friendly as a standalone model with exact KV-cache
 * support (abstract on the fugumt.com page; "KV Cache" section of the
 * mauroscia.it page, on managing the cache without wasting memory); the
 * block table is the reading taken for that.
 *   position p of sequence b:  page pg = block_table[b][p / 64], row p % 64;
 *   k_pool [n_pages][Hkv][64][D]   key of (p, h) at [pg][h][p % 64][:];
 *   v_pool [n_pages][Hkv][D][64]   value of (p, h), element d, at
 *                                  [pg][h][d][p % 64] (pages transposed).
 *
 *   dtype        TIDAR_BF16 only (TIDAR_EUNSUPPORTED otherwise).
 *   max_pages    entries per block-table row; capacity 64 * max_pages
 *                positions per sequence (plays the role of S_max).
 *   n_pages      pages in each pool.
 *   block_table  [B][max_pages] int32 (device memory).  Entries for pages
 *                0 .. ceil(lens[b] / 64) - 1 must lie in [0, n_pages); a
 *                sequence with any other entry there gets NaN outputs, like
 *                a violated length bound.  Later entries are not read.
 *                Pages may be shared between sequences.
 *   workspace    at least what tidar_step_attention_workspace() reports for
 *                S_max = 64 * max_pages and the same other arguments.
 * Every other argument is as for tidar_step_attention.
 * ---------------------------------------------------------------------- */
int tidar_step_attention_paged(int dtype, int B, int Hq, int Hkv, int D, int max_pages, int n_pages, int max_len,
                               int k, int n_groups, float sm_scale, int kv_chunk,
                               const void* q, const void* k_step, const void* v_step,
                               const void* k_pool, const void* v_pool, const int32_t* block_table,
                               const int32_t* lens, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Training-mask attention over the duplicated training sequence.
 *
 * Each example appears twice in one long sequence: once for ordinary
 * next-token supervision and once as a fully masked block filled in
 * parallel (paragraph on training of the nodesdaily.com page; section
 * "3. Training Recipe" of the mauroscia.it page).  The sequence is
 * [x_0 .. x_{N-1} ; m_0 .. m_{N-1}], T = 2N positions, and
 *   clean row r < N sees positions 0..r (causal);
 *   masked row N + j, of block [lo, hi) with lo = j - j % block and
 *   hi = min(lo + block, N), sees the clean prefix 0..lo-1 and its own
 *   block N+lo .. N+hi-1 (bidirectional), as a draft group sees the prefix,
 *   its accepted candidates and itself at decode time.
 *   out[b][r][h] = softmax_c(sm_scale * q[b][r][h] . key_c) . value_c.
 * Forward pass only; the losses and training stay with the caller.
 *
 *   dtype    TIDAR_BF16 only (TIDAR_EUNSUPPORTED otherwise).
 *   N        clean positions: a multiple of 64, 64..2^24.
 *   block    masked-block size, 1..N (the draft length at decode time).
 *   q        [B][T][Hq][D]
 *   k        [B][Hkv][T][D]          (the key-cache layout with S_max = T)
 *   v        [B][Hkv][T/64][D][64]   (the value-cache layout: pages of 64
 *                                     positions, each transposed)
 *   out      [B][T][Hq][D] (written);  lse [B][Hq][T] f32 natural-log
 *            softmax denominators (written; may be NULL).
 * No workspace.  Other arguments as for tidar_step_attention.  Head dim
 * 128 runs on the eight-wave kernel unless TIDAR_ATTN_KERNEL is "pipe"
 * (see tidar_step_attention_plan); head dim 64 on the four-wave one.
 * ---------------------------------------------------------------------- */
int tidar_train_attention(int dtype, int B, int Hq, int Hkv, int D, int N, int block, float sm_scale,
                          const void* q, const void* k, const void* v, void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * Greedy verification and next-draft selection.
 *
 * Candidates are confirmed strictly left to right; whichever outcome is
 * confirmed, the drafts prepared for it become the next candidates
 * (nodesdaily.com page, paragraph on drafting for every outcome).
 *   t_i          = argmax_v ar_logits[b][i][v], i = 0..k (lowest index wins
 *                  ties; -0.0 ties +0.0; logits must be finite).
 *   accept_len[b]= largest a <= k with cand[b][i] == t_i for every i < a.
 *   next_cand[b][0] = t_a (the exact AR token after the accepted prefix).
 *   g            = max(a, 1) - 1.
 *   next_cand[b][m] = argmax_v draft_logits[b][g][m][v], m = 1..k-1.
 *
 *   ar_logits    [B][k+1][V] f32: row 0 is the AR distribution at
 *                candidate 0's position (carried from the previous pass),
 *                row i >= 1 the output of candidate row i-1.
 *   draft_logits [B][k][k][V] f32: output of slot s of group g; only the
 *                selected group's rows 1..k-1 are read.  May be NULL when
 *                k == 1.
 *   cand         [B][k] int32.
 *   accept_len   [B] int32 (written);  next_cand [B][k] int32 (written).
 *   workspace    at least tidar_verify_workspace() bytes.
 * ---------------------------------------------------------------------- */
int tidar_verify_workspace(int B, int k, int V, size_t* bytes);

int tidar_verify_greedy(int B, int k, int V, const float* ar_logits, const float* draft_logits,
                        const int32_t* cand, int32_t* accept_len, int32_t* next_cand,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * LM head fused with greedy verification.
 *
 * The single pass yields the joint distribution that verifies and the
 * marginals that draft (section "2. Single Forward Pass & Structured
 * Attention Mask" of the mauroscia.it page); both are the LM head applied
 * to the pass's final hidden states, and verification needs only each
 * row's argmax.  This call computes logits = h . W^T (bf16 inputs, fp32
 * accumulation) for the k+1 AR rows and, once the accept length is known,
 * for the selected group's draft rows 1..k-1, keeping only per-chunk
 * (max, lower index) results -- no logits are written -- and then applies
 * exactly the rule of tidar_verify_greedy to them.
 *
 *   d_model   hidden size: a multiple of 64.  V * d_model * 2 and
 *             B * k * k * d_model * 2 must be below 2^32 (byte offsets).
 *   h_ar      [B][k+1][d_model] bf16: row 0 the carried hidden state,
 *             row i >= 1 the output of candidate row i-1.
 *   h_draft   [B][k][k][d_model] bf16: slot s of group g; only the selected
 *             group's rows 1..k-1 are read.  May be NULL when k == 1.
 *   w         [V][d_model] bf16, the LM head (one row per vocabulary entry).
 *   cand, accept_len, next_cand   as for tidar_verify_greedy.
 *   workspace at least tidar_lmhead_verify_workspace() bytes.
 * Inputs must be finite.  The argmax is over fp32 logits, so a row whose
 * two best logits lie within fp32 accumulation error of each other may
 * differ from an exact evaluation.
 * ---------------------------------------------------------------------- */
int tidar_lmhead_verify_workspace(int B, int k, int V, int d_model, size_t* bytes);

int tidar_lmhead_verify_greedy(int B, int k, int V, int d_model, const void* h_ar, const void* h_draft,
                               const void* w, const int32_t* cand, int32_t* accept_len, int32_t* next_cand,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The same LM head with W in a packed layout, made once when the weights
 * are loaded.  The fused head reads W in tiles of 256 vocabulary rows by 64
 * hidden elements; in the row-major layout such a tile is 256 separate
 * 128-byte runs, 2*d_model bytes apart, while in the packed layout it is
 * one contiguous 32 KB block, which memory serves faster.  Results are
 * bit-for-bit those of tidar_lmhead_verify_greedy on the row-major W.
 *
 * tidar_lmhead_packed_bytes: size of the packed W,
 *   ceil(V / 256) * 256 * d_model * 2 bytes.  EINVAL for V < 1 or a
 *   d_model that is not a positive multiple of 64.
 * tidar_lmhead_pack: w [V][d_model] bf16 (row-major, 16-byte aligned) ->
 *   w_packed (16-byte aligned, tidar_lmhead_packed_bytes() bytes, owned by
 *   the caller; must not overlap w).  Asynchronous on `stream`.  Layout:
 *   tile (c, s), c < ceil(V/256), s < d_model/64, is the 32 KB block at
 *   byte (c * (d_model/64) + s) * 32768; its bytes 128*r + 16*j .. +15 hold
 *   w[256*c + r][64*s + 8*(j ^ (r % 8)) .. +7] (r < 256, j < 8), and zeros
 *   for rows 256*c + r >= V.
 * tidar_lmhead_verify_greedy_packed: as tidar_lmhead_verify_greedy, with
 *   w_packed from tidar_lmhead_pack(V, d_model, ...) in place of w.  The
 *   2^32 bound on V * d_model * 2 does not apply; the one on the draft
 *   rows does.  The workspace is the same.
 * ---------------------------------------------------------------------- */
int tidar_lmhead_packed_bytes(int V, int d_model, size_t* bytes);

int tidar_lmhead_pack(int V, int d_model, const void* w, void* w_packed, void* stream);

int tidar_lmhead_verify_greedy_packed(int B, int k, int V, int d_model, const void* h_ar, const void* h_draft,
                                      const void* w_packed, const int32_t* cand, int32_t* accept_len,
                                      int32_t* next_cand, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stochastic verification (temperature T > 0) and sampling of the next drafts.
 *
 * The final tokens are sampled autoregressively and the output matches
 * sampling the AR model alone (engineer-news.pages.dev page, section on what
 * TiDAR does; nodesdaily.com page, paragraph on the reported numbers).  The
 * rule used is speculative sampling, with p_i = softmax(ar_logits[b][i] / T)
 * and q_i = softmax(q_logits[b][i] / T), the distribution candidate i was
 * drawn from:
 *   candidate i (token x = cand[b][i]) is kept when u_i * q_i(x) < p_i(x);
 *   accept_len[b] = a, the first i < k that is not kept (k if all are);
 *   next_cand[b][0] is drawn from max(0, p_a - q_a) (normalised) if a < k,
 *                   from p_k if a == k (from p_a if max(0, p_a - q_a) has no
 *                   positive entry in fp32);
 *   g = max(a, 1) - 1;
 *   next_cand[b][m] is drawn from softmax(draft_logits[b][g][m] / T), m >= 1.
 * Every random number comes from Philox4x32-10 (Salmon et al., SC 2011) with
 * key (seed & 0xFFFFFFFF, seed >> 32) and a 32-bit output x mapped to
 * u = ((x >> 9) + 0.5) * 2^-23:
 *   u_i of the keep test: counter (i, 0xFFFFFFFF, b, step), word 0;
 *   the draw of row j (0 = next_cand[b][0], m = next_cand[b][m]) is
 *   argmax_v (log w_v - log(-log u_v)) (Gumbel-max, ties to the lower v)
 *   with u_v from counter (v / 4, j, b, step), word v % 4.
 * Identical (seed, step) give identical results; a caller advances `step`
 * between decode steps.  Probabilities are computed in fp32; a decision
 * within fp32 rounding of its threshold may differ from an exact evaluation.
 *
 *   temperature  finite and > 0 (TIDAR_EINVAL otherwise).
 *   ar_logits    [B][k+1][V] f32 as for tidar_verify_greedy.
 *   q_logits     [B][k][V] f32: row i is the distribution candidate i was
 *                drawn from (row 0: the carried AR row, so candidate 0 is
 *                always kept when q_logits[b][0] == ar_logits[b][0]).
 *   draft_logits [B][k][k][V] f32; only group g's rows 1..k-1 are read.
 *                May be NULL when k == 1.
 *   Logits may be -inf (a zero weight) but every row needs a finite entry;
 *   +inf and NaN are not allowed.  A candidate outside [0, V) is rejected.
 *   cand         [B][k] int32.
 *   accept_len   [B] int32 (written);  next_cand [B][k] int32 (written).
 *   workspace    at least tidar_verify_sample_workspace() bytes.
 * ---------------------------------------------------------------------- */
int tidar_verify_sample_workspace(int B, int k, int V, size_t* bytes);

int tidar_verify_sample(int B, int k, int V, float temperature, const float* ar_logits, const float* q_logits,
                        const float* draft_logits, const int32_t* cand, uint64_t seed, uint32_t step,
                        int32_t* accept_len, int32_t* next_cand, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ------------------------------------------------------------------------
 * KV-cache commit / evict, in place.
 *
 * The settled cache is reused and rejected entries are evicted
 * (nodesdaily.com page, paragraph on the three zones; "KV Cache" section of
 * the mauroscia.it page).  For every sequence b with a = accept_len[b]:
 *   k_cache[b][h][lens[b]+i][:]  = k_step[b][i][h][:]     i < a, every h
 *   v_cache[b][h][p/64][:][p%64] = v_step[b][i][h][:]       p = lens[b]+i
 *   lens[b] += a
 * Rejected candidates and every slot row are never written.  A sequence
 * with lens[b] + a > S_max (flag 1) or a outside 0..k (flag 2) is left
 * untouched.
 *
 *   dtype        element type of the caches and step rows.
 *   S_max        cache capacity, a multiple of 64; caches laid out as for
 *                tidar_step_attention.
 *   R            rows per sequence of k_step / v_step ([B][R][Hkv][D]).
 *   k            number of candidates (bound on accept_len), 1 <= k <= R.
 *   lens         [B] int32, read and updated in place.
 *   accept_len   [B] int32.
 *   err_flags    [B] int32 (written: 0 ok, 1 overflow, 2 bad length); may
 *                be NULL.
 * ---------------------------------------------------------------------- */
int tidar_kv_commit(int dtype, int B, int Hkv, int D, int S_max, int R, int k,
                    void* k_cache, void* v_cache, int32_t* lens,
                    const void* k_step, const void* v_step, const int32_t* accept_len,
                    int32_t* err_flags, void* stream);

/* ------------------------------------------------------------------------
 * KV-cache commit / evict into a paged cache, in place.
 *
 * tidar_kv_commit for the pools and block table of
 * tidar_step_attention_paged: the accepted rows of sequence b go to
 * positions p = lens[b] + i, i < a, i.e. key row p % 64 and value column
 * p % 64 of page block_table[b][p / 64]; then lens[b] += a.  The caller
 * provides the pages (entries for every page that positions lens[b] ..
 * lens[b] + a - 1 fall in); a page written here must not be shared with
 * another sequence.
 *   flags (err_flags[b]): 0 ok, 1 lens[b] + a > 64 * max_pages, 2 a outside
 *   0..k, 3 a needed page entry outside [0, n_pages).  A flagged sequence is
 *   left untouched.
 *   dtype        TIDAR_BF16 or TIDAR_F32.
 *   max_pages, n_pages, block_table   as for tidar_step_attention_paged.
 * Every other argument is as for tidar_kv_commit.
 * ---------------------------------------------------------------------- */
int tidar_kv_commit_paged(int dtype, int B, int Hkv, int D, int max_pages, int n_pages, int R, int k,
                          void* k_pool, void* v_pool, const int32_t* block_table, int32_t* lens,
                          const void* k_step, const void* v_step, const int32_t* accept_len,
                          int32_t* err_flags, void* stream);

/* ------------------------------------------------------------------------
 * Greedy verification fused with the KV commit.
 *
 * One call does what tidar_verify_greedy followed by tidar_kv_commit (or
 * tidar_kv_commit_paged) does, with the same results bit for bit: the accept
 * length a_b and the next drafts (paragraph on drafting for every outcome of
 * the nodesdaily.com page), then the a_b accepted candidate rows appended to
 * the settled cache and lens[b] += a_b, rejected entries evicted (paragraph
 * on the three zones; "KV Cache" section of the mauroscia.it page).  It runs
 * in two launches instead of five: per-row argmax keys are folded with
 * atomics, every workgroup of the draft pass derives the accept length from
 * them itself and copies a share of the accepted rows, and the last of a
 * sequence's workgroups to finish writes its results and new length.
 *
 *   state        device memory (8-byte aligned) of at least
 *                tidar_verify_commit_state_bytes(B, k) bytes: per-row
 *                argmax keys and per-sequence arrival counters.  It must be ZERO before its
 *                first use; every call leaves it zero again.  One state must
 *                not serve two calls that may run at the same time.
 *   dtype, B, Hkv, D, S_max, R, k, k_cache, v_cache, lens, k_step, v_step,
 *   err_flags    as for tidar_kv_commit (flags 0 ok, 1 capacity; 2 cannot
 *                occur: a_b comes from the verification itself).
 *   V, ar_logits, draft_logits, cand, accept_len, next_cand
 *                as for tidar_verify_greedy.
 * Returns the status the two separate calls would (the first failing check).
 * ---------------------------------------------------------------------- */
int tidar_verify_commit_state_bytes(int B, int k, size_t* bytes);

int tidar_verify_commit_greedy(int dtype, int B, int Hkv, int D, int S_max, int R, int k, int V,
                               const float* ar_logits, const float* draft_logits, const int32_t* cand,
                               void* k_cache, void* v_cache, int32_t* lens,
                               const void* k_step, const void* v_step,
                               int32_t* accept_len, int32_t* next_cand, int32_t* err_flags,
                               void* state, size_t state_bytes, void* stream);

/* tidar_verify_commit_greedy for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without `state`.  Its state is
 * a 2 MiB array inside the library, one per GPU, held until the process
 * ends; this call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  The first call on a GPU, and the first after a call
 * that returned TIDAR_ELAUNCH, also enqueue a clearing kernel before the
 * two of the step.
 *   Returns TIDAR_EWORKSPACE when tidar_verify_commit_state_bytes(B, k)
 *   exceeds 2 MiB (2097152 bytes), before anything is enqueued; otherwise
 *   what tidar_verify_commit_greedy returns.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (two streams, two host threads) race and must be serialised by the
 * caller. */
int tidar_verify_commit_greedy_noalloc(int dtype, int B, int Hkv, int D, int S_max, int R, int k, int V,
                                       const float* ar_logits, const float* draft_logits,
                                       const int32_t* cand, void* k_cache, void* v_cache, int32_t* lens,
                                       const void* k_step, const void* v_step,
                                       int32_t* accept_len, int32_t* next_cand, int32_t* err_flags,
                                       void* stream);

/* The same into a paged cache (flags as for tidar_kv_commit_paged; 3: a
 * needed page entry outside [0, n_pages)). */
int tidar_verify_commit_greedy_paged(int dtype, int B, int Hkv, int D, int max_pages, int n_pages, int R, int k,
                                     int V, const float* ar_logits, const float* draft_logits,
                                     const int32_t* cand, void* k_pool, void* v_pool,
                                     const int32_t* block_table, int32_t* lens,
                                     const void* k_step, const void* v_step,
                                     int32_t* accept_len, int32_t* next_cand, int32_t* err_flags,
                                     void* state, size_t state_bytes, void* stream);

/* Launch shapes of the verification and commit paths (a host-only
 * diagnostic; nothing is enqueued): path 0 tidar_verify_greedy, 1
 * tidar_kv_commit, 2 tidar_verify_commit_greedy.  For each launch, in order,
 * shapes receives (grid x, grid y, threads per workgroup); `shapes` is a
 * host array of at least 12 ints owned by the caller.  Returns the number of
 * launches, or the negative status the entry point would return for these
 * sizes (V, Hkv, D, dtype are ignored where the path has no use for them).
 * A workgroup of more than 1024 threads never launches, and a later kernel
 * would then read what it should have written; the shapes can be checked
 * for that on any machine. */
int tidar_launch_shapes(int path, int B, int k, int V, int Hkv, int D, int dtype, int* shapes);

/* ---------------------------------------------------------------------------
 * Checked build (debugging aid, not part of the decode step).
 *
 * libtidar_checked.so is this library compiled with device-side bounds
 * tests, for debugging a caller or the kernels.  Each kernel tests every index it reads from device memory
 * (settled lengths, block-table entries, draft groups and accept lengths
 * written by an earlier kernel, arrival counters of the verify + commit
 * state) and every key tile, query, output and step row and split-K chunk
 * it derives, against the bound the call's sizes give it, before it
 * addresses a buffer.  A failed test records {code, workgroup, thread,
 * value} -- the first failure per kernel source file and GPU is kept -- and
 * the access is redirected in bounds or skipped, so the kernel runs to its
 * end (no trap).  The documented outcomes of contract violations (NaN
 * attention rows, err_flags, -1 next drafts) are those of the release
 * library, and are recorded as well.  Outputs of a call that fails a test
 * that the release library does not make (codes ROW, CHUNK, KEY_TILE,
 * TOKEN, STATE) are undefined.  libtidar.so compiles every test out and
 * exports the same two calls.
 */
enum {
  TIDAR_CHECK_NONE = 0,
  TIDAR_CHECK_LENS = 1,     /* settled length < 0, or > max_len (attention) */
  TIDAR_CHECK_PAGE = 2,     /* block-table entry outside [0, n_pages) */
  TIDAR_CHECK_KEY_TILE = 3, /* key tile or table slot outside the cache (S_max/64 tiles, max_pages slots) */
  TIDAR_CHECK_ROW = 4,      /* sequence outside [0, B) or query / output / step row outside its range */
  TIDAR_CHECK_CHUNK = 5,    /* split-K chunk outside the plan's chunks */
  TIDAR_CHECK_GROUP = 6,    /* draft group read back outside [0, k) */
  TIDAR_CHECK_ACCEPT = 7,   /* accept length outside [0, k] */
  TIDAR_CHECK_TOKEN = 8,    /* token id outside [0, V) (e.g. a logit row with nothing above -inf) */
  TIDAR_CHECK_CAPACITY = 9, /* commit past the cache (L + accept > S_max) */
  TIDAR_CHECK_STATE = 10    /* verify + commit state not cleared by the previous call */
};

/* 1 in libtidar_checked.so, 0 in libtidar.so. */
int tidar_check_enabled(void);

/* Synchronises the current device, then copies into rec[4] (host array
 * owned by the caller) the first recorded failure {code, workgroup, thread,
 * value} -- kernel source files taken in a fixed order -- or all zeros, and
 * if `clear` is non-zero resets every record of the current device.  In
 * libtidar.so rec is set to zeros and nothing is synchronised.  Returns
 * TIDAR_OK, TIDAR_EINVAL for a null rec, TIDAR_ELAUNCH if the runtime
 * reports an error. */
int tidar_check_read(uint32_t* rec, int clear);

/* ---------------------------------------------------------------------------
 * Measurement helper (not part of the decode step).
 *
 * tidar_read_probe reads `bytes` of device memory at `src` once, in 16 B
 * loads spread over TIDAR_READ_PROBE_BLOCKS workgroups, and writes one 32-bit
 * word per workgroup to `sink`: the XOR of every 32-bit word that workgroup
 * read.  The XOR of all sink words therefore equals the XOR of all 32-bit
 * words of the buffer, which a host can check.  Timed over a buffer much
 * larger than the GPU's caches, it gives the read bandwidth the memory
 * delivers to a plain streaming kernel: the denominator for reporting a
 * kernel's bandwidth against what is achievable, beside the data-sheet peak.
 *
 *   src    device pointer, 16-byte aligned; bytes a multiple of 16.
 *   sink   device pointer to TIDAR_READ_PROBE_BLOCKS uint32 (4-byte aligned).
 *   Returns TIDAR_EINVAL for a null or misaligned pointer or a size not a
 *   multiple of 16; bytes == 0 enqueues nothing.
 * ------------------------------------------------------------------------- */
#define TIDAR_READ_PROBE_BLOCKS 16384

int tidar_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* tidar_mfma_probe measures the issue interval of the matrix cores (a
 * measurement helper, not part of the decode step).  It launches
 * TIDAR_MFMA_PROBE_BLOCKS workgroups, one per CU, each of 4 x waves_per_simd
 * waves (waves_per_simd waves on each SIMD).  Every wave runs `iters` rounds
 * of eight independent v_mfma_f32_16x16x32_bf16 on eight accumulators.  With
 * lds_reads = 1 the A operand of each MFMA is read from LDS first (16 B per
 * lane, one conflict-free 1 KB block per MFMA, four reads ahead), the
 * operand pattern of the attention loops; with 0 it is held in registers.
 * Each wave writes the shader-clock cycles of its rounds to
 * cycles[workgroup * 4 * waves_per_simd + wave]; cycles / (8 * iters) is that
 * wave's interval between MFMAs, and with two waves per SIMD the SIMD issues
 * two MFMAs in that interval.
 *
 *   waves_per_simd  1 or 2.   lds_reads  0 or 1.   iters  1 .. 2^20.
 *   cycles  device pointer to TIDAR_MFMA_PROBE_BLOCKS * 4 * waves_per_simd
 *           uint64 (8-byte aligned), owned by the caller.
 *   Returns TIDAR_EINVAL for other values or a null or misaligned pointer,
 *   TIDAR_ELAUNCH if the launch fails. */
#define TIDAR_MFMA_PROBE_BLOCKS 256

int tidar_mfma_probe(int waves_per_simd, int lds_reads, int iters, uint64_t* cycles, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TIDAR_H */
