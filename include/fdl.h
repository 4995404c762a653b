/*
 * fdl.h -- C ABI of libfdl, the MI355X (gfx950) cached block-diffusion
 * denoising step of Fast-dLLM / Fast-dLLM v2.
 *
 * One denoising step is four calls, enqueued in order on one HIP stream:
 *   fdl_block_attn   attention of the active (sub-)block's query rows over the
 *                    block-level prefix KV cache and the block itself (and, in
 *                    the v1 DualCache mode, the cached suffix)
 *   fdl_lm_head      hidden rows -> vocabulary logits
 *   fdl_conf_select  greedy token, confidence, commit set per sequence
 *   fdl_kv_append    append a finished block's K/V to the cache
 * fdl_lm_head_select runs the second and third as one pass that never
 * materializes the logits.  fdl_kv_write stores K/V at a position the caller
 * knows (the v1 refresh from position 0, or a lock-step batch's block) in one
 * launch.  fdl_prefill_attn is the multi-block attention of the prompt
 * prefill and of the v1 cache refresh; fdl_decode runs a whole generation
 * (steps, sub-blocks, blocks, EOS) with its control on the device.
 *
 * Pages defining the operations (cited by title and section):
 *   "Fast-dLLM v2: Efficient Block-Diffusion LLM" (technical breakdown):
 *     Attention Mask Design, Inference-time attention mask (Figure 7b),
 *     Inference Pipeline Levels 1-3, Batch decoding with length padding,
 *     Sub-block size as a decoding granularity knob.
 *   "Fast-dLLM: Reusing Bidirectional State and Spending Confidence on
 *     Parallel Tokens": eq 3, section 3 (PrefixCache and DualCache,
 *     Algorithm 1), section 4 (Algorithm 2), section 6 (eq 13, Algorithm 3).
 *   "Diffusion language models: review questions": commit rule, fixed count.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers owned by the caller (except `dims`, which
 *     is a host pointer read during the call).  The library allocates no
 *     memory and keeps no global mutable state; calls are reentrant.  The
 *     one exception is fdl_lm_head_select_noalloc, whose static scratch
 *     array (and its per-device address) is shared by every call on a GPU.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     No call synchronizes with the host or reads device memory back.
 *   - Validation of scalar arguments and pointers happens on the host before
 *     anything is launched; on failure the call returns a negative fdl_status
 *     and launches nothing.  Values held in device memory (lengths, tau) are
 *     the caller's contract; the kernels never access memory outside the
 *     extents stated below, whatever those values are.
 *   - After launching, a HIP launch error is reported as FDL_E_HIP.
 *   - Tensors are dense, row-major, in the layouts given per argument.
 *     bf16 = bfloat16 stored as 16-bit words; f32 = IEEE binary32.
 */
#ifndef FDL_H
#define FDL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FDL_OK = 0,
  FDL_E_INVAL = -1,        /* a scalar or pointer argument is invalid           */
  FDL_E_UNSUPPORTED = -2,  /* valid but not supported (e.g. head_dim 96)        */
  FDL_E_HIP = -3,          /* a HIP launch reported an error                    */
  FDL_E_WORKSPACE = -4,    /* workspace missing or smaller than required        */
  FDL_E_SCRATCH = -5       /* more than FDL_NOALLOC_SCRATCH_BYTES of scratch    */
} fdl_status;

typedef enum { FDL_F32 = 0, FDL_BF16 = 1 } fdl_dtype;

typedef enum {
  /* Fast-dLLM v2, Figure 7b: the active block attends bidirectionally to its
     own D positions and to the whole cached prefix; nothing after it. */
  FDL_ATTN_BLOCK_CAUSAL = 0,
  /* Fast-dLLM v1 DualCache (section 3): prefix cache + fresh block + cached
     suffix of all later positions up to P + L; fully bidirectional. */
  FDL_ATTN_DUAL_CACHE = 1
} fdl_attn_mode;

typedef enum {
  /* Algorithm 2: commit every candidate with conf > tau (strict); if none,
     the single most confident candidate (lowest row on equal conf). */
  FDL_SELECT_THRESHOLD = 0,
  /* fixed count: the min(k, #candidates) most confident candidates (lowest
     row first on equal conf). */
  FDL_SELECT_TOPK = 1,
  /* eq 13 / Algorithm 3: candidates sorted by decreasing conf; commit the
     first n for the largest n with (n+1)(1 - c_(n)) < factor, else the first. */
  FDL_SELECT_FACTOR = 2
} fdl_select_mode;

/* The problem statement of one decoding run.
 *   batch       B, sequences decoded together (right-padded to whole blocks)
 *   prompt_len  P, cached prompt positions
 *   gen_len     L, answer positions (a multiple of block)
 *   block       D, block size (32 on the pages)
 *   sub_block   S, query rows per step (8 on the pages; = block for whole-block steps);
 *               block % sub_block == 0
 *   n_q_heads   Hq; n_kv_heads Hkv divides Hq (query head h reads KV head h / (Hq/Hkv))
 *   head_dim    d, 64 or 128
 *   hidden      H, LM-head input width (a multiple of 64 for bf16, of 4 for f32;
 *               f32 LM heads take at most 64 rows)
 *   vocab       V
 *   dtype       fdl_dtype of Q/K/V/O, X and W
 *   attn_mode   fdl_attn_mode
 * The KV cache of one sequence and KV head holds cap = P + L positions. */
typedef struct fdl_dims {
  int32_t batch;
  int32_t prompt_len;
  int32_t gen_len;
  int32_t block;
  int32_t sub_block;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t hidden;
  int32_t vocab;
  int32_t dtype;
  int32_t attn_mode;
} fdl_dims;

/* Library version (major * 10000 + minor * 100 + patch). */
int fdl_version(void);

/* Static description of a status code.  Never NULL. */
const char* fdl_strerror(int status);

/* Host-side validation of `dims` alone.  Returns FDL_OK or the code the entry
 * points would return for these dims. */
int fdl_dims_check(const fdl_dims* dims);

/* Bytes of device workspace fdl_block_attn needs for any block_idx/sub_idx
 * of `dims` (0 if none).  Returns 0 for invalid dims.  The workspace holds
 * the key splits' partial results (scratch of one call: calls that overlap
 * on one workspace race). */
size_t fdl_block_attn_workspace_size(const fdl_dims* dims);

/* Block attention: eq 3 (softmax(Q K^T / sqrt(d)) V) over the visible keys of
 * the active block (Figure 7b mask, or DualCache), GQA, exact online softmax.
 *
 *   block_idx   index b of the active block, 0 <= b < L / D
 *   sub_idx     index of the active sub-block, 0 <= sub_idx < D / S
 *               (every row of a block sees the same keys, so it only checks range)
 *   q           [B][S][Hq][d]  query rows of the active sub-block (dtype)
 *   k_cache     [B][Hkv][P+L][d] (dtype); v_cache likewise.  Position j holds
 *               the K/V of absolute position j.  Read: prefix positions
 *               [0, Lp) and, in DualCache mode, the suffix [Lp + D, P + L).
 *   prefix_len  [B] int32 Lp per sequence, or NULL for Lp = P + b*D for all.
 *               Contract: 0 <= Lp and Lp + D <= P + L (values outside are clamped).
 *   k_blk       [B][Hkv][D][d] fresh K of the active block's D positions; v_blk likewise
 *   out         [B][S][Hq][d] (dtype), written
 *   lse         [B][Hq][S] f32 natural-log log-sum-exp of the scores, or NULL
 *   workspace   >= fdl_block_attn_workspace_size(dims) bytes (may be NULL if that is 0)
 * The query rows may be any subset of the block: each sees Lp + D keys
 * (block-causal) or P + L keys (DualCache). */
int fdl_block_attn(const fdl_dims* dims, int32_t block_idx, int32_t sub_idx,
                   const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* prefix_len, const void* k_blk, const void* v_blk,
                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Multi-block attention: query positions q_start .. q_start + n_q - 1 of
 * one sequence over its key positions 0 .. n_keys - 1 (eq 3).
 *   causal = 1: block-causal, the M_BC pattern of "Fast-dLLM v2" (Attention
 *     Mask Design): position p sees the keys of its own block and of every
 *     earlier block (blocks of `block` positions), as in the prompt prefill.
 *   causal = 0: every key visible, as in the Fast-dLLM v1 refresh of the
 *     cached regions (Algorithm 1) and the PrefixCache recomputation.
 *   q       [B][n_q][Hq][d] (bf16 only)
 *   k, v    [B][Hkv][P+L][d]: positions 0 .. n_keys - 1 are read
 *   out     [B][n_q][Hq][d], written
 *   lse     [B][Hq][n_q] f32 natural-log log-sum-exp, or NULL
 * Constraints: dtype FDL_BF16; n_q >= 1; q_start >= 0; 1 <= n_keys <= P + L. */
int fdl_prefill_attn(const fdl_dims* dims, int32_t q_start, int32_t n_q, int32_t n_keys,
                     int32_t causal, const void* q, const void* k, const void* v, void* out,
                     float* lse, void* stream);

/* LM head: logits[r][v] = sum_k X[r][k] * W[v][k], f32 accumulation and
 * output ("Fast-dLLM v2", Inference Pipeline Level 2: a distribution over the
 * vocabulary per position; with the token shift of Step 5 the row for block
 * position i is the hidden state at i - 1, which is the caller's row choice).
 *   rows    M >= 1
 *   x       [M][H] (dtype)
 *   w       [V][H] (dtype)
 *   logits  [M][V] f32, written */
int fdl_lm_head(const fdl_dims* dims, int32_t rows, const void* x, const void* w,
                float* logits, void* stream);

/* Bytes of device workspace fdl_conf_select needs: chunk partials of every
 * row and one row counter per sequence (0 for invalid arguments).  Scratch of
 * one call: calls that overlap on it race. */
size_t fdl_conf_select_workspace_size(const fdl_dims* dims, int32_t rows_per_seq);

/* Confidence select (Algorithm 2 / fixed count / Algorithm 3) with the
 * commit-state update.
 *   rows_per_seq R, 1 <= R <= 256; row r of sequence b is logits row b*R + r
 *   logits       [B][R][V] f32 (finite values)
 *   masked       [B][R] uint8, nonzero = still [MASK] = a commit candidate
 *   tau          [B] f32 threshold per sequence (FDL_SELECT_THRESHOLD)
 *   mode         fdl_select_mode; k for TOPK (>= 1); factor for FACTOR (> 0)
 *   token_out    [B][R] int32 argmax token of every row (lowest id on ties)
 *   conf_out     [B][R] f32 its softmax probability, 1 / sum_v exp(l_v - l_max)
 *   commit_out   [B][R] uint8 1 = committed this step (only candidates)
 *   n_commit     [B] int32 number committed (>= 1 whenever a row is masked)
 *   tokens_inout [B][R] int32 or NULL: committed rows take their token
 *   masked_inout [B][R] uint8 or NULL: committed rows are cleared; may alias masked
 *   workspace    >= fdl_conf_select_workspace_size(dims, R) bytes */
int fdl_conf_select(const fdl_dims* dims, int32_t rows_per_seq, const float* logits,
                    const uint8_t* masked, const float* tau, int32_t mode, int32_t k,
                    float factor, int32_t* token_out, float* conf_out, uint8_t* commit_out,
                    int32_t* n_commit, int32_t* tokens_inout, uint8_t* masked_inout,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace fdl_lm_head_select needs: 16 bytes per (row,
 * vocabulary span) of select partials -- a span is the vocabulary range of
 * one LM-head workgroup: for bf16 and up to 64 rows 128 rows, or V / 1280
 * rounded up for up to 32 rows and a vocabulary of 81,920 to 163,840; for
 * bf16 and more rows 256; for f32 128 -- then one 4-byte row counter per
 * sequence (rounded up to 16 bytes).  0 for invalid arguments.  The
 * workspace is scratch of one call: calls that overlap on it race. */
size_t fdl_lm_head_select_workspace_size(const fdl_dims* dims, int32_t rows_per_seq);

/* LM head fused with the confidence select: the same results as fdl_lm_head
 * followed by fdl_conf_select on its logits, but the LM head's epilogue
 * reduces every (row, vocabulary span) of logits it computes to the
 * select's (max, lowest argmax, sum exp) partial, so the B*R*V f32 logits are
 * neither written nor read back ("Fast-dLLM v2", Level 2: only the argmax and
 * its probability are consumed).  Arguments as in fdl_lm_head (rows =
 * B * rows_per_seq) and fdl_conf_select, except:
 *   logits     [B*R][V] f32, or NULL to skip writing them
 *   workspace  >= fdl_lm_head_select_workspace_size(dims, rows_per_seq) bytes
 * Confidences may differ from the unfused path in the last bits (the partial
 * sums are formed in a different order). */
int fdl_lm_head_select(const fdl_dims* dims, int32_t rows_per_seq, const void* x, const void* w,
                       float* logits, const uint8_t* masked, const float* tau, int32_t mode,
                       int32_t k, float factor, int32_t* token_out, float* conf_out,
                       uint8_t* commit_out, int32_t* n_commit, int32_t* tokens_inout,
                       uint8_t* masked_inout, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Allocation-free variant of fdl_lm_head_select, for callers that cannot
 * allocate or pass device memory for a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments and results as fdl_lm_head_select without the workspace; the
 * select partials and row counters live in a static device array of the
 * library (FDL_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends),
 * so the call allocates nothing.  Returns FDL_E_SCRATCH, launching nothing,
 * when fdl_lm_head_select_workspace_size(dims, rows_per_seq) exceeds that
 * size.  Every call on a GPU shares that GPU's array: calls that overlap on
 * one GPU (concurrent streams or host threads) race.  The array's address is
 * looked up on the first call on each device (with that device current). */
#define FDL_NOALLOC_SCRATCH_BYTES (8u << 20)
int fdl_lm_head_select_noalloc(const fdl_dims* dims, int32_t rows_per_seq, const void* x,
                               const void* w, float* logits, const uint8_t* masked,
                               const float* tau, int32_t mode, int32_t k, float factor,
                               int32_t* token_out, float* conf_out, uint8_t* commit_out,
                               int32_t* n_commit, int32_t* tokens_inout, uint8_t* masked_inout,
                               void* stream);

/* KV append ("Fast-dLLM v2", Level 3 block-level cache: a finished block's
 * K/V are stored for all later steps; Fast-dLLM Algorithm 1: the refresh
 * rewrites the cached regions, i.e. len = 0 then append P + L positions).
 *   k_cache, v_cache [B][Hkv][P+L][d] (dtype), written at [len[b], len[b] + n_new)
 *   k_new, v_new     [B][Hkv][n_new][d] (dtype)
 *   n_new            1 <= n_new <= P + L
 *   len              [B] int32, read then advanced by n_new.  A sequence with
 *                    len[b] < 0 or len[b] + n_new > P + L is left untouched
 *                    (no write, len unchanged). */
int fdl_kv_append(const fdl_dims* dims, void* k_cache, void* v_cache, const void* k_new,
                  const void* v_new, int32_t n_new, int32_t* len, void* stream);

/* KV write at a caller-given position, the same for every sequence: the
 * refresh of the v1 caches ("Fast-dLLM: Reusing Bidirectional State ...",
 * Algorithm 1 and the DualCache of section 3) rewrites every cached position
 * from 0, which this does in one launch without first clearing len.
 *   k_cache, v_cache [B][Hkv][P+L][d] (dtype), written at [pos, pos + n_new)
 *   k_new, v_new     [B][Hkv][n_new][d] (dtype)
 *   pos, n_new       0 <= pos, 1 <= n_new, pos + n_new <= P + L (else FDL_E_INVAL)
 *   len              [B] int32 set to pos + n_new, or NULL to leave lengths alone
 * Bitwise copy; nothing is read from len. */
int fdl_kv_write(const fdl_dims* dims, void* k_cache, void* v_cache, const void* k_new,
                 const void* v_new, int32_t pos, int32_t n_new, int32_t* len, void* stream);

/* ---------------------------------------------------------------------------
 * Decode loop: a whole generation of a batch, with every control decision
 * taken on the device.
 *
 * "Fast-dLLM v2", Inference Pipeline: blocks are generated left to right
 * (Level 1); each starts fully masked and is refined sub-block by sub-block,
 * step after step, until no position is masked (Level 2, and "Sub-block size
 * as a decoding granularity knob"); a finished block's K/V enter the
 * block-level cache (Level 3); generation stops once a finished block holds
 * EOS or after max_blocks.  "Batch decoding with length padding": the batch
 * advances in lock step; a sequence that has produced EOS gets padding blocks
 * (MASK tokens that are never candidates).  In FDL_ATTN_DUAL_CACHE mode the
 * cache is instead refreshed (rewritten for all P + L positions) at the start
 * of every block and the block also attends to the cached suffix (Fast-dLLM
 * section 3, Algorithm 1).
 *
 * The host enqueues a fixed schedule -- for every block and sub-block, as
 * many step slots as the selection rule can need (sub_block for THRESHOLD
 * and FACTOR, ceil(sub_block / k) for TOPK, since every step commits at least
 * one masked row of every sequence that has one) -- and nothing is read back:
 * a small control kernel before each slot opens or closes a device-side gate,
 * and every kernel of a slot whose gate is closed returns at once.
 *
 * The transformer is replaced by a synthetic stand-in so that every input of
 * a step is a function of the current tokens (w doubles as the tied token
 * embedding; H must equal n_q_heads * head_dim):
 *   e(t) = sqrt(H) * w[t];  query of head h = e(t)[h*d .. h*d+d);
 *   key of KV head g = e(t)[g*d .. g*d+d);
 *   value of KV head g = e(t)[H-(Hkv-g)*d .. H-(Hkv-g-1)*d) in reverse order;
 *   hidden row of active position p = gain * (attention output, heads
 *     concatenated) + boost_val[p] * w[boost_tok[p]] / |w[boost_tok[p]]|^2,
 *     rounded to dtype;
 *   row i of the active sub-block predicts its own position.
 * Each step is then: embed -> fdl_block_attn -> hidden rows ->
 * fdl_lm_head_select (with the commit update in place) on the active rows.
 */
typedef struct {
  /* stand-in model */
  const void* w;              /* [V][H] dtype: LM-head weight and tied embedding     */
  float gain;                 /* weight of the attention output in the hidden row    */
  int32_t mask_id, eos_id;    /* reserved ids, 0 <= id < V                            */
  /* inputs (device) */
  const int32_t* prompt;      /* [B][P] token ids (ids outside [0, V) read as mask_id)  */
  const int32_t* boost_tok;   /* [B][L] drawn token per generated position (outside
                                 [0, V): no boost)                                      */
  const float* boost_val;     /* [B][L] its boost                                      */
  const float* tau;           /* [B] threshold (THRESHOLD; may be NULL otherwise)      */
  int32_t mode, k;            /* fdl_select_mode; k >= 1 for TOPK                      */
  float factor;               /* > 0 for FACTOR                                        */
  int32_t max_blocks;         /* 1 .. L/D; 0 = L/D                                     */
  /* state and outputs (device, written) */
  void* k_cache;              /* [B][Hkv][P+L][d] dtype                                */
  void* v_cache;              /* [B][Hkv][P+L][d] dtype                                */
  int32_t* len;               /* [B] valid cache positions at the end                  */
  int32_t* tokens;            /* [B][P+L] prompt, generated tokens, MASK padding       */
  uint8_t* masked;            /* [B][P+L] 1 = still masked (all 0 at the end)          */
  int32_t* seq_steps;         /* [B] steps in which the sequence had a masked row      */
  int32_t* eos_block;         /* [B] block whose completion stopped the sequence, -1   */
  int32_t* counters;          /* [2] steps run, blocks run                             */
  /* optional per-step trace: all NULL, or all set with trace_cap >= the number
     of step slots; entry t is the t-th step that ran */
  int32_t trace_cap;
  int32_t* trace_meta;        /* [trace_cap][2] block, sub-block                       */
  int32_t* trace_tokens;      /* [trace_cap][B][D] the block's tokens after the step   */
  uint8_t* trace_masked;      /* [trace_cap][B][D] the block's masked flags after it   */
  int32_t* trace_token;       /* [trace_cap][B][S] argmax of every active row          */
  float* trace_conf;          /* [trace_cap][B][S] its confidence                      */
} fdl_decode_args;

/* Bytes of device workspace fdl_decode needs for dims.  0 for invalid dims. */
size_t fdl_decode_workspace_size(const fdl_dims* dims);

/* Number of step slots fdl_decode enqueues for these arguments (the trace
 * capacity it needs); 0 for invalid arguments. */
int32_t fdl_decode_step_slots(const fdl_dims* dims, int32_t mode, int32_t k, int32_t max_blocks);

/* Run the decode loop.  dims and args are host pointers read during the
 * call.  Requirements beyond fdl_block_attn / fdl_lm_head_select: hidden ==
 * n_q_heads * head_dim; the workspace is fdl_decode_workspace_size(dims)
 * bytes.  Everything is enqueued on stream; the call returns before the
 * device finishes and reads nothing back. */
int fdl_decode(const fdl_dims* dims, const fdl_decode_args* args, void* workspace,
               size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FDL_H */
