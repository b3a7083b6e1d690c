/*
 * g4attn.h -- C ABI of the batch-invariant hybrid (sliding + global) GQA attention
 * library for Gemma-4-style decoders on AMD Instinct MI355X (gfx950).
 *
 * What is computed (citations name the page and its section):
 *   - RL-Kernel issue #415, "[RFC][Gemma-4-31B-it] WS1/WS2 kernel roadmap", section 5
 *     work items qk_rmsnorm_d256_d512, sliding_rope_d256, global_proportional_p_rope
 *     (the prologue), sliding_attention_core and global_attention_core (prefill),
 *     global_k_eq_v_projection (one tensor serves as K and V) and
 *     hybrid_kv_cache_contract (decode against the cache equals the prefill row);
 *     section 2 fingerprint (32 q heads; sliding 16 KV heads x 256, window 1024;
 *     global 4 KV heads x 512, K=V; RoPE theta 1e4 / p-RoPE 0.25 at theta 1e6).
 *   - Same page, section 4 "Numerical contract": a fixed fp32 accumulator, one fixed
 *     reduction order per output row that does not depend on batch composition,
 *     packing, padding or launch geometry, no split-KV and no cross-work-group
 *     atomics unless the split and its merge tree are fixed by the contract (the
 *     *_split entry points: fixed key chunks, merged in ascending order, the same in
 *     prefill and decode), casts only at declared points, unsupported geometry fails
 *     closed, and runtime provenance is reported.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns. Every tensor pointer is a
 *     device pointer owned by the caller; the library allocates nothing and keeps no
 *     state besides a thread-local error message.
 *   - Calls are asynchronous on `stream` (NULL = the default stream) and never
 *     synchronise. Device faults surface at the caller's next synchronisation.
 *   - All validation runs on the host before any launch. On a non-OK status nothing
 *     was launched and no output was touched; g4attn_last_error() explains it.
 *     G4ATTN_ERR_UNSUPPORTED is the fail-closed code: the request is well formed but
 *     outside what the kernels implement; there is no fallback path.
 *   - Not checked (they would need a device read): device-side lengths agree with the
 *     host-side maxima passed alongside them, and sequences do not overlap.
 *
 * Rounding points (declared): the prologue computes in fp32 and rounds once to bf16
 * (round to nearest even). Attention keeps scores, running max and running sum in
 * fp32, rounds the probabilities to bf16 for the P*V product (the sum uses the fp32
 * values), accumulates O in fp32, and rounds out = O * (1/l) to bf16 once.
 */
#ifndef G4ATTN_H_
#define G4ATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define G4ATTN_ABI_VERSION 3

/* Same type as HIP's hipStream_t. */
typedef struct ihipStream_t* g4attn_stream_t;

typedef enum {
  G4ATTN_OK = 0,
  G4ATTN_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent geometry */
  G4ATTN_ERR_UNSUPPORTED = 2, /* well formed, not implemented: fails closed */
  G4ATTN_ERR_DEVICE = 3       /* the HIP runtime refused the launch */
} g4attn_status;

typedef enum { G4ATTN_SLIDING = 0, G4ATTN_GLOBAL = 1 } g4attn_kind;

typedef enum {
  /* pairs (i, i + R/2), i < R/2: rotate-half inside the rotated block [0, R) */
  G4ATTN_ROPE_PAIRS_IN_BLOCK = 0,
  /* pairs (i, i + D/2), i < R/2: rotate-half over the whole head, the other pairs
     at frequency 0 (the layout of HF transformers' proportional RoPE) */
  G4ATTN_ROPE_PAIRS_HALF_HEAD = 1
} g4attn_rope_pairing;

/* One attention layer's geometry. Sliding layers: window > 0; global: window == 0. */
typedef struct {
  int32_t kind;          /* g4attn_kind                                                */
  int32_t num_q_heads;   /* Hq                                                         */
  int32_t num_kv_heads;  /* Hkv; Hq % Hkv == 0, G = Hq/Hkv in {1,2,4,8,16,32}            */
  int32_t head_dim;      /* D in {64, 128, 256, 512}                                   */
  int32_t window;        /* W > 0: key j visible to query i iff 0 <= i - j < W;
                            W == 0: full causal (j <= i)                               */
  int32_t k_eq_v;        /* 1: one tensor is both K and V (no separate v)              */
  int32_t rope_dims;     /* R: rotated dims, even, 0 <= R <= D (0 = no RoPE)           */
  int32_t rope_freq_dim; /* F: pair i turns at theta^(-2 i / F) per position           */
  int32_t rope_pairing;  /* g4attn_rope_pairing                                        */
  int32_t v_norm;        /* 0: the prologue copies v raw; 1: it stores v's unit RMS norm
                            (no weight, no rotation); needs k_eq_v == 0                 */
  double rope_theta;     /* 1e4 sliding, 1e6 global                                    */
  float softmax_scale;   /* s_ij = softmax_scale * <q_i, k_j> (1/sqrt(D) by default)   */
  float rms_eps;         /* RMSNorm epsilon (1e-6)                                     */
} g4attn_layer;

/* Runtime provenance of one launch (numerical contract, rule 8). */
typedef struct {
  char kernel_id[64];         /* implementation identifier                        */
  int32_t kind;               /* layer kind as passed                             */
  int32_t head_dim;
  int32_t group;              /* G = Hq / Hkv                                      */
  int32_t block_q;            /* query rows (position x head) per work-group      */
  int32_t block_k;            /* keys per KV tile; tiles start at position 0      */
  int32_t mfma_m, mfma_n, mfma_k; /* matrix instruction shape (32 x 32 x 16 bf16)   */
  int32_t waves_per_group;
  int32_t split_kv;           /* 0, or the chunk size of the split form            */
  int32_t acc_fp32;           /* always 1                                         */
  int32_t fallback;           /* always 0: there is no fallback path              */
  uint64_t shape_fingerprint; /* FNV-1a of the layer descriptor and the launch    */
} g4attn_provenance;

/*
 * g4attn_qk_prologue -- per-head RMSNorm then RoPE on q and k, one bf16 rounding.
 * Pages: RL-Kernel #415 section 5 (qk_rmsnorm_d256_d512, sliding_rope_d256,
 * global_proportional_p_rope); TensorFold PR #1186, tf_qk_rows_once commit (the
 * weight multiplies the normalised row, and the norm comes before RoPE).
 *
 * For token t (0 <= t < num_tokens) and each head row x of D values:
 *   y = w * (x / sqrt(mean(x^2) + rms_eps)),  w = q_norm_w or k_norm_w (bf16 [D],
 *   shared by all heads); then pair p of the rotated dims turns by
 *   positions[t] * rope_theta^(-2p / rope_freq_dim) (pairing per rope_pairing);
 *   then y is rounded to bf16.
 * q_in/q_out: [T, Hq, D]; q row t is written to q_out row t (in place allowed).
 *   Both NULL skips q.
 * k_in/k_out: k_in is [T, Hkv, D]; its row t is written to k_out row
 *   kv_dst_row[t] (units of Hkv*D elements), or row t if kv_dst_row is NULL; rows
 *   with kv_dst_row[t] < 0 are not written. In place only when kv_dst_row is NULL.
 *   Both NULL skips k.
 * v_in/v_out: optional v rows with k's row map, for filling a separate V cache; both
 *   NULL or both non-NULL; not allowed with K=V. With layer->v_norm == 0 each row is
 *   copied raw; with v_norm == 1 it is stored as v / sqrt(mean(v^2) + rms_eps), no weight
 *   and no rotation, rounded once to bf16 (TensorFold PR #1186, tf_qk_rows_once commit:
 *   v normed by a unit RMS norm at head dim 512). The real model's global layer passes its
 *   one raw projection as both k_in and v_in: K is normed with k_norm_w and rotated, V is
 *   only normed, and the attention reads them as separate K and V (k_eq_v == 0).
 * positions: int32 [T] absolute position of each token. Tokens that map to the same
 *   destination row in one call race: pass each cache slot at most once.
 */
g4attn_status g4attn_qk_prologue(const g4attn_layer* layer, const uint16_t* q_in, uint16_t* q_out,
                                 const uint16_t* k_in, uint16_t* k_out, const uint16_t* v_in,
                                 uint16_t* v_out, const uint16_t* q_norm_w, const uint16_t* k_norm_w,
                                 const int32_t* positions, const int64_t* kv_dst_row,
                                 int64_t num_tokens, g4attn_stream_t stream);

/*
 * g4attn_prefill -- causal / sliding-window GQA attention over a packed varlen batch.
 * Pages: RL-Kernel #415 section 5 (sliding_attention_core, global_attention_core,
 * global_k_eq_v_projection) and section 4 (numerical contract).
 *
 * q [T, Hq, D], k [T, Hkv, D], v [T, Hkv, D] (NULL iff layer->k_eq_v, then k is also
 * V), out [T, Hq, D]; all row-major bf16. Sequence b owns rows
 * [seq_start[b], seq_start[b] + seq_len[b]) and its positions restart at 0.
 * Query head h reads KV head h / G. out row (t, h) = sum_j softmax_j(scale * q.k_j) v_j
 * over the visible keys j of the same sequence. Rows outside every sequence
 * (padding) are never read as keys and never written.
 * seq_start, seq_len: int32 [batch] device arrays. max_seq_len: host-side upper bound
 * of seq_len (sizes the grid). batch == 0 or max_seq_len == 0 returns OK.
 * out must not overlap q, k or v (the call is not in place): out equal to one of them is
 * rejected with G4ATTN_ERR_INVALID_ARG; a partial overlap cannot be seen on the host and
 * gives undefined results.
 * Every row's result is bit-identical whatever else is in the batch, wherever the
 * sequence sits in the pack, and equal to g4attn_decode's result for that row.
 * prov: optional out-struct (host memory), filled on success.
 */
g4attn_status g4attn_prefill(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, uint16_t* out, const int32_t* seq_start,
                             const int32_t* seq_len, int32_t batch, int32_t max_seq_len,
                             g4attn_stream_t stream, g4attn_provenance* prov);

/*
 * g4attn_prefill_qp -- g4attn_prefill of raw q rows: each work-group norms and rotates its
 * query rows as g4attn_qk_prologue would (the same arithmetic in the same order, so the same
 * bf16 bits) while staging them, and q never makes the round trip through memory. Pages:
 * RL-Kernel #415 section 5 (qk_rmsnorm_d256_d512, global_proportional_p_rope,
 * global_attention_core); TensorFold PR #1186, the qk-rows commit (norm, then RoPE, one
 * rounding).
 *
 * Arguments as g4attn_prefill, with q the raw rows [T, Hq, D] (before the prologue; not
 * written), q_norm_w: bf16 [D] device array, positions: int32 [T] device array (the RoPE
 * position of each packed row), both non-NULL when batch > 0. k (and v) have been through
 * g4attn_qk_prologue already. out is bit-identical to g4attn_qk_prologue on q followed by
 * g4attn_prefill. Head dim 512 with one tensor as K and V (the global layer) only: other
 * layers return G4ATTN_ERR_UNSUPPORTED, and so does a 512-dim layer whose angle tables
 * (fp32 cos and sin for each position of a work-group's 128 rows and each rotated pair)
 * together with q_norm_w do not fit the 32 KiB key stage they are built in (with group
 * size 8: rope_dims 256 fits, 512 does not).
 */
g4attn_status g4attn_prefill_qp(const g4attn_layer* layer, const uint16_t* q, const uint16_t* q_norm_w,
                                const int32_t* positions, const uint16_t* k, const uint16_t* v, uint16_t* out,
                                const int32_t* seq_start, const int32_t* seq_len, int32_t batch,
                                int32_t max_seq_len, g4attn_stream_t stream, g4attn_provenance* prov);

/*
 * g4attn_prefill_masked -- g4attn_prefill with a per-row last key, for the bidirectional
 * rows of an image. Pages: TensorFold PR #1186, the commit that adds the vision path to
 * the native Gemma 4 engine (an image's rows each see all of that image's rows, through
 * the sliding attention's per-row last key; global layers stay causal; a prompt chunk
 * never cuts an image); RL-Kernel #415 section 2 (use_bidirectional_attention =
 * "vision") and section 5 (multimodal_bidirectional_mask).
 *
 * Arguments as g4attn_prefill, plus last_key: int32 [T] device array (indexed by packed
 * row, like q), non-NULL when batch > 0. Row t of sequence b, at position i, sees key
 * position j of its own sequence iff j <= max(i, min(last_key[t], seq_len[b] - 1)) and,
 * for a sliding layer with window W, i - j < W. A value below the row's position (e.g.
 * -1) leaves the row causal; such rows get exactly g4attn_prefill's bits. Keys past a row's
 * position are visible only through last_key (the caller marks an image's rows with the
 * image's last position). Either layer kind is accepted: which layers see images both
 * ways is the caller's choice (the pages disagree). The result of every row is
 * bit-identical whatever else is in the batch and wherever its sequence sits. There is no
 * decode counterpart: a decoded token is never inside an image.
 */
g4attn_status g4attn_prefill_masked(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k,
                                    const uint16_t* v, uint16_t* out, const int32_t* seq_start,
                                    const int32_t* seq_len, const int32_t* last_key, int32_t batch,
                                    int32_t max_seq_len, g4attn_stream_t stream, g4attn_provenance* prov);

/*
 * g4attn_prefill_cached -- a chunk of query rows per sequence against a bf16 KV cache
 * (chunked prefill).
 * Pages: RL-Kernel #415 section 5 (hybrid_kv_cache_contract: the prefill / chunked-
 * prefill / decode handoff); TensorFold PR #1186, native Gemma 4 engine commit (prompts
 * run in chunks of up to 512 rows; sliding layers keep a ring of window + 512 slots,
 * global layers a linear cache).
 *
 * Sequence b's chunk is chunk_len[b] query rows at positions q_pos0[b] ..
 * q_pos0[b] + chunk_len[b] - 1, held in rows q_row0[b] .. of q [T, Hq, D] (through the
 * prologue) and written to the same rows of out [T, Hq, D]. Its keys are positions
 * 0 .. q_pos0[b] + chunk_len[b] - 1; key position p of head g lives in cache row
 * (cache_row0[b] + p % cache_slots) * Hkv + g (row = D values), and the chunk's own keys
 * must already be there (g4attn_qk_prologue with kv_dst_row). v_cache is NULL iff
 * layer->k_eq_v. cache_slots: a positive multiple of 32 (a 32-key block is 32
 * consecutive slots); sliding layers: >= window + max_chunk_len (every key a chunk row
 * sees is present); global layers: >= max_key_len. A block can read slots of keys its
 * rows do not see (they are masked): every slot of the region must hold finite values
 * (a region that was zero-filled before its first use does).
 * q_row0, q_pos0, chunk_len: int32 [batch]; cache_row0: int64 [batch]; device arrays.
 * max_chunk_len: host bound of chunk_len (sizes the grid); max_key_len: host bound of
 * q_pos0[b] + chunk_len[b] (checked against a linear cache). batch == 0 or
 * max_chunk_len == 0 returns OK. Rows of out outside every chunk are not written.
 * out must not overlap q or the caches (out equal to q, k_cache or v_cache is rejected
 * with G4ATTN_ERR_INVALID_ARG).
 * Result: every row bit-identical to g4attn_prefill's row for the same position of the
 * whole sequence (and so to g4attn_decode's): the blocks are aligned to position 0 and
 * taken in the same order whatever the chunking.
 */
g4attn_status g4attn_prefill_cached(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                    const uint16_t* v_cache, uint16_t* out, const int32_t* q_row0,
                                    const int32_t* q_pos0, const int32_t* chunk_len, const int64_t* cache_row0,
                                    int32_t cache_slots, int32_t batch, int32_t max_chunk_len, int32_t max_key_len,
                                    g4attn_stream_t stream, g4attn_provenance* prov);

/*
 * g4attn_prefill_cached_masked -- g4attn_prefill_cached with per-row last keys: the chunk
 * rows of an image see every row of that image. Pages: TensorFold PR #1186, the vision
 * commit of the native Gemma 4 engine (an image's rows see all of them through the
 * per-row last key; a prompt chunk never cuts through an image).
 *
 * Arguments as g4attn_prefill_cached, plus last_key: int32 [T] device array indexed like
 * q (the chunk's rows), non-NULL when batch > 0; its values are positions in the whole
 * sequence. The chunk row at position i sees key position j iff j <= max(i, last_key)
 * with last_key clipped to the chunk's last position (q_pos0 + chunk_len - 1), and the
 * window rule holds: an image must lie inside one chunk. Rows whose last key is at or
 * below their position get exactly g4attn_prefill_cached's bits; every row gets the bits
 * of g4attn_prefill_masked for the whole sequence.
 */
g4attn_status g4attn_prefill_cached_masked(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                           const uint16_t* v_cache, uint16_t* out, const int32_t* q_row0,
                                           const int32_t* q_pos0, const int32_t* chunk_len, const int32_t* last_key,
                                           const int64_t* cache_row0, int32_t cache_slots, int32_t batch,
                                           int32_t max_chunk_len, int32_t max_key_len, g4attn_stream_t stream,
                                           g4attn_provenance* prov);

/*
 * g4attn_decode -- one new token per sequence against a bf16 KV cache.
 * Pages: RL-Kernel #415 section 5 (hybrid_kv_cache_contract: prefill -> decode
 * handoff); TensorFold PR #1186 (sliding ring cache, global linear cache).
 *
 * q, out: [batch, Hq, D], the new token of each sequence (already through the
 * prologue). ctx_len[b] = L_b >= 1 counts the new token, which sits at position
 * L_b - 1 and must already be in the cache. Key position p of sequence b, head g
 * lives in cache row (cache_row0[b] + p % cache_slots) * Hkv + g (row = D values):
 * a ring for sliding layers (cache_slots >= window), a linear cache for global ones
 * (cache_slots >= max_ctx_len). v_cache is NULL iff layer->k_eq_v.
 * cache_row0: int64 [batch]; ctx_len: int32 [batch]; both device arrays.
 * schedule: optional int32 [batch] device permutation of 0..batch-1; work-group i
 * serves sequence schedule[i] (e.g. longest first). It changes no result.
 * Result: bit-identical to g4attn_prefill's row for the same position.
 */
g4attn_status g4attn_decode(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, const int64_t* cache_row0, const int32_t* ctx_len,
                            int32_t cache_slots, uint16_t* out, int32_t batch, int32_t max_ctx_len,
                            const int32_t* schedule, g4attn_stream_t stream, g4attn_provenance* prov);

/*
 * g4attn_prefill_backward -- the gradients of g4attn_prefill's attention with respect to q,
 * k and v, for a trainer on the same declared arithmetic as the forward. Pages: RL-Kernel
 * #415 section 1 (training and rollout execute one declared contract) and section 5
 * (global_k_eq_v_projection: the backward gradient semantics of the K=V mapping, whose
 * one tensor receives the gradient of both roles); section 4 (no split-KV, no cross-work-
 * group atomics: every gradient element is reduced in one fixed order).
 *
 * Inputs as g4attn_prefill (q [T, Hq, D], k and v [T, Hkv, D], v NULL iff layer->k_eq_v,
 * the same seq_start / seq_len / batch / max_seq_len), plus out (the forward's output
 * [T, Hq, D]) and dout (the loss gradient with respect to out, [T, Hq, D]); bf16.
 * With s = softmax_scale q.k over the visible keys, P = softmax(s), delta_i = dout_i . out_i:
 *   dS = P (dout v^T - delta),  dq = scale dS k,  dk = scale dS^T q,  dv = P^T dout,
 * the k and v gradients summed over the G query heads of their KV head. Outputs: dq
 * [T, Hq, D]; dk [T, Hkv, D] (with k_eq_v: the sum of both roles, and dv must be NULL);
 * dv [T, Hkv, D]; lse and delta, fp32 [T, Hq]: each row's log2 of its sum of exp(s) over
 * the visible keys, and its delta (the row statistics the gradients are formed from).
 * Rows outside every sequence are not written. Outputs must not overlap the inputs.
 * Arithmetic (declared): fp32 scores, P = exp2(s log2(e) - lse), dS in fp32, P and dS
 * rounded to bf16 for the gradient products, fp32 accumulation in ascending key-block
 * (dq) or row-tile (dk, dv) order, one bf16 rounding per output (with k_eq_v: one fp32
 * sum over both roles, scale dS rounded to bf16 as its operand). Every output element is
 * bit-identical whatever else is in the batch. Two launches on `stream`.
 */
g4attn_status g4attn_prefill_backward(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const uint16_t* out, const uint16_t* dout, uint16_t* dq,
                                      uint16_t* dk, uint16_t* dv, float* lse, float* delta, const int32_t* seq_start,
                                      const int32_t* seq_len, int32_t batch, int32_t max_seq_len,
                                      g4attn_stream_t stream);

/* Message for the last non-OK status on this thread ("" after a successful call).
   Valid until the next g4attn call on the same thread. */
const char* g4attn_last_error(void);

/*
 * The split form (global layers). Pages: RL-Kernel #415 section 4 rule 3 (a split of
 * the key range is allowed when the split and its merge tree are fixed by the contract);
 * TensorFold PR #1186, window-rows commits (decode by fixed key chunks whose partial
 * results are merged in chunk order, at head dims 256 and 512).
 *
 * Contract, for a chunk size C (split_keys: a positive multiple of 256) and a row at
 * position i, whose visible keys 0 .. i fall in chunks 0 .. n - 1, n = i / C + 1 (chunk
 * c = positions c C .. c C + C - 1):
 *   - each chunk c gives the row's partial result over its keys: offset m_c, sum l_c
 *     and unnormalised O_c, by exactly the block updates of g4attn_prefill (32-key
 *     blocks aligned to position 0, ascending, final offsets) started afresh at the
 *     chunk's first block;
 *   - n == 1: out = bf16(O_0 (1 / l_0)), which is g4attn_prefill's row bit for bit;
 *   - n >= 2: M = max_c m_c, w_c = 2^(m_c - M) (the hardware exp2), then in ascending c
 *     L = w_0 l_0 + w_1 l_1 + ... and O = w_0 O_0 + w_1 O_1 + ... in fp32 (each step a
 *     product then a sum), out = bf16(O (1 / L)).
 * g4attn_prefill_split and g4attn_decode_split with the same C give every row the same
 * bits (a decode row equals the prefill row of its position), whatever else is in the
 * batch; without the split (the other entry points) rows past C differ from these in
 * rounding. Sliding layers (window > 0) return G4ATTN_ERR_UNSUPPORTED: their decode
 * reads at most W keys per row.
 *
 * Workspace: caller-owned device memory, 16-byte aligned, of at least
 * g4attn_split_workspace_bytes(...) bytes, holding the partial results between the chunk
 * kernels and the merge (fp32: batch x rows x Hq x chunks x (D + 2) values, chunks =
 * ceil(max_key_len / C)). Zero bytes (and a NULL workspace allowed) when no row's keys
 * span two chunks: the call then runs the plain kernels. Calls that share a workspace
 * on different streams race. It must not overlap the inputs or outputs.
 */

/* g4attn_split_workspace_bytes -- bytes of workspace a split call needs: rows =
 * max_seq_len and max_key_len = max_seq_len for g4attn_prefill_split; rows = max_chunk_len
 * and max_key_len as passed for g4attn_prefill_cached_split; rows = 1 and max_key_len =
 * max_ctx_len for g4attn_decode_split. */
g4attn_status g4attn_split_workspace_bytes(const g4attn_layer* layer, int32_t batch, int32_t rows,
                                           int32_t max_key_len, int32_t split_keys, uint64_t* bytes);

/* g4attn_prefill_split -- g4attn_prefill (same arguments and layout) under the split
 * contract above with chunk size split_keys. Two launches on `stream`: the chunk
 * work-groups (the prefill grid repeated per chunk; a chunk's work-groups read only its
 * key blocks), then the merge; or the plain prefill alone when no row spans two chunks. */
g4attn_status g4attn_prefill_split(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* out, const int32_t* seq_start, const int32_t* seq_len, int32_t batch,
                                   int32_t max_seq_len, int32_t split_keys, void* workspace,
                                   uint64_t workspace_bytes, g4attn_stream_t stream, g4attn_provenance* prov);

/* g4attn_prefill_cached_split -- g4attn_prefill_cached (same arguments and layout) on a
 * linear cache under the split contract: a chunk row gets the bits of the same position in
 * g4attn_prefill_split of the whole sequence and in g4attn_decode_split (the prefill /
 * chunked prefill / decode handoff of RL-Kernel #415 section 5 hybrid_kv_cache_contract,
 * in the split form). Two launches on `stream` (the chunk work-groups, then the merge), or
 * the plain chunked prefill when no row's keys span two chunks. */
g4attn_status g4attn_prefill_cached_split(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                          const uint16_t* v_cache, uint16_t* out, const int32_t* q_row0,
                                          const int32_t* q_pos0, const int32_t* chunk_len, const int64_t* cache_row0,
                                          int32_t cache_slots, int32_t batch, int32_t max_chunk_len,
                                          int32_t max_key_len, int32_t split_keys, void* workspace,
                                          uint64_t workspace_bytes, g4attn_stream_t stream, g4attn_provenance* prov);

/* g4attn_decode_split -- g4attn_decode (same arguments) on a linear cache under the split
 * contract: one work-group per (sequence, KV head, chunk), then the merge. Equal to
 * g4attn_prefill_split's row for the same position and split_keys. */
g4attn_status g4attn_decode_split(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int64_t* cache_row0, const int32_t* ctx_len,
                                  int32_t cache_slots, uint16_t* out, int32_t batch, int32_t max_ctx_len,
                                  const int32_t* schedule, int32_t split_keys, void* workspace,
                                  uint64_t workspace_bytes, g4attn_stream_t stream, g4attn_provenance* prov);

/* g4attn_decode_split_noalloc -- g4attn_decode_split without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation). The partial results go to a library-owned
 * array of 64 MiB per GPU (a static device array, held until the process ends); the call
 * allocates nothing. Requests whose partials exceed it (g4attn_split_workspace_bytes with
 * rows = 1 above 67108864) return G4ATTN_ERR_UNSUPPORTED. Every call on one GPU shares the
 * array: calls that overlap on one GPU (other streams, other threads) race. Same results
 * as g4attn_decode_split. */
g4attn_status g4attn_decode_split_noalloc(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                          const uint16_t* v_cache, const int64_t* cache_row0, const int32_t* ctx_len,
                                          int32_t cache_slots, uint16_t* out, int32_t batch, int32_t max_ctx_len,
                                          const int32_t* schedule, int32_t split_keys, g4attn_stream_t stream,
                                          g4attn_provenance* prov);

/* G4ATTN_ABI_VERSION of the library. */
int32_t g4attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* G4ATTN_H_ */
