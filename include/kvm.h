/*
 * libkvmem -- C ABI of the IndexMem / MomentKV hot path on AMD Instinct MI355X (gfx950).
 *
 * IndexMem: a learned MQA-style indexer scores every prefill token from an observation
 * window of queries; the highest-scoring tokens are kept in a compact KV cache before the
 * full prefill ("pre-eviction"); evicted tokens are folded into a fixed-size latent memory
 * (M, b) by decayed outer products; decode attends over the kept tokens and adds a gated
 * memory read-out.  MomentKV: evicted tokens are summarised by moment sums instead; they
 * drive a residual-based eviction score and a normalisation-corrected output.
 *
 * Sources, cited by page title and section:
 *   [IM]  "IndexMem - learned KV-cache eviction with latent memory", technical summary
 *         (gist.science, arXiv 2605.25475), section 2 "Method", parts A and B.
 *   [MKV] "MOMENTKV" technical summary (gist.science, arXiv 2606.01563), Method parts 1-4.
 *   [ASM] "Context Memorization for Efficient Long Context Generation" technical summary
 *         (gist.science, arXiv 2605.18226), Method: attention state (a, Z), online-softmax merge.
 *
 * Conventions (every entry point):
 *   - Pointers named in the argument lists are DEVICE pointers owned by the caller unless
 *     the comment says "host".  The library never allocates or frees memory.
 *   - Every call only enqueues work on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream) and returns without synchronising.  Results are visible in stream order.
 *   - Arguments are validated before any HIP call; a failed check returns a status and
 *     enqueues nothing.  kvm_last_error() then gives a thread-local message.
 *   - Layouts are dense row-major (C order) with the shapes given; element types are fixed
 *     per argument (KVM_F32 / KVM_BF16 arguments follow desc->dtype).  Device pointers must
 *     be 16-byte aligned.
 *   - Workspaces: `ws` must hold kvm_*_workspace_size() bytes (device memory, any
 *     contents); it holds only intermediates of one call.  Two calls that share a
 *     workspace must not overlap in time.
 *   - No floating-point atomics are used; repeated calls give bitwise identical results.
 */
#ifndef KVM_H
#define KVM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVM_ABI_VERSION 3

typedef enum {
  KVM_OK = 0,
  KVM_ERR_NULL = 1,        /* a required pointer is NULL                          */
  KVM_ERR_SHAPE = 2,       /* a size is non-positive or unsupported               */
  KVM_ERR_DTYPE = 3,       /* dtype not KVM_F32 / KVM_BF16 or unsupported here     */
  KVM_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned             */
  KVM_ERR_RANGE = 5,       /* inconsistent sizes, e.g. budget below recent window */
  KVM_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required          */
  KVM_ERR_ARCH = 7,        /* the current device is not gfx950                    */
  KVM_ERR_HIP = 8          /* a HIP runtime call failed                           */
} kvm_status;

typedef enum { KVM_F32 = 0, KVM_BF16 = 1 } kvm_dtype;

int kvm_abi_version(void);
const char* kvm_status_string(kvm_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* kvm_last_error(void);
/* Checks that the current HIP device is gfx950 (KVM_ERR_ARCH otherwise). */
kvm_status kvm_check_device(void);

/* ------------------------------------------------------------------------------------ *
 * A1-A3  Indexer scores and per-key importance                        [IM 2.A]
 *
 * For one layer and b sequences of length L, with the last W positions as the
 * observation window (query s at position L-W+s):
 *   k_hat[t]   = RMSNorm_{gamma_k}(W_kI x_t)                      (shared key, d_I)
 *   q_hat[s,h] = RMSNorm_{gamma_q}(W_qI[h] q_{s, c(h)}),  c(h) = floor(h*H_q/H_I)
 *   g[s,h]     = sigmoid(W_g[h] . x_s)                            (learned head gate)
 *   A[s,t]     = sum_h g[s,h] * relu(q_hat[s,h] . k_hat[t] / sqrt(d_I))   for t <= pos(s)
 *   I[t]       = max_s A[s,t]                                     (running max-pool)
 * The head gate, per-head ReLU, RMSNorm and 1/sqrt(d_I) are readings of the section's
 * "MQA-style indexer with QK norm and a learnable gate on head contributions".
 * Arithmetic: projections with fp32 accumulation; the score contraction uses fp16
 * hi+lo split operands on the matrix cores (relative error ~1e-7 of each logit), so I
 * carries near-fp32 accuracy.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t b, L, D;         /* batch, prefill length, hidden size                        */
  int32_t H_q, d;          /* model query heads, head dim                                */
  int32_t H_I, d_I, W;     /* indexer heads, indexer dim, window (1 <= W <= L)            */
  int32_t dtype;           /* kvm_dtype of X, Qwin and the three weight matrices         */
  float eps_rms;           /* RMSNorm epsilon (1e-6)                                     */
} kvm_index_desc;

size_t kvm_index_workspace_size(const kvm_index_desc* desc);
/*
 * X      [b, L, D]            hidden states (dtype)
 * Qwin   [b, W, H_q, d]       model queries of positions L-W .. L-1 (dtype)
 * W_kI   [d_I, D], W_qI [H_I, d_I, d], W_g [H_I, D]   (dtype);  gamma_k, gamma_q [d_I] f32
 * I      [b, L] f32           output importance
 * khat   [b, L, d_I] f32      optional output (NULL to skip): the normalised keys
 * Supported: d_I in {32, 64}, d in {64, 128}; D % 8 == 0.
 */
kvm_status kvm_index_score(const kvm_index_desc* desc, const void* X, const void* Qwin,
                           const void* W_kI, const float* gamma_k, const void* W_qI,
                           const float* gamma_q, const void* W_g, float* I, float* khat,
                           void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ *
 * A4  Pre-eviction top-k                                              [IM 2.A]
 *
 * Per row of I [rows, L]: keep the last R positions (recent window) plus the n_top
 * highest-scoring positions before them, n_top = B - R if recent_inclusive else B,
 * ordered by (score descending, position ascending) -- ties keep the lower position.
 * NaN scores order as -inf, -0 as +0.  If n_top >= L - R every position is kept.
 * Outputs: idx [rows, keep] i32 = kept positions ascending (keep = min(L, n_top + R));
 *          slot_map [rows, L] i32: slot (>= 0) of a kept position, or -i for the i-th
 *          evicted position in ascending order (i = 1..L-keep).
 * Errors: KVM_ERR_RANGE if recent_inclusive and B < R, or B < 0, R < 0.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t rows, L, B, R;
  int32_t recent_inclusive;  /* 1: R counts inside B; 0: B plus R                       */
} kvm_topk_desc;

int32_t kvm_topk_keep(const kvm_topk_desc* desc);  /* keep = number of kept positions   */
/* ws: NULL, or at least kvm_topk_workspace_size(desc) bytes of device memory (any contents).
 * With a workspace, rows longer than 32768 positions are spread over many blocks (chunks of
 * 4096 positions, six launches); without one, or for shorter rows, one block per row.  Both
 * give the same result, bit for bit. */
size_t kvm_topk_workspace_size(const kvm_topk_desc* desc);
kvm_status kvm_topk_select(const kvm_topk_desc* desc, const float* I, int32_t* idx,
                           int32_t* slot_map, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ *
 * A5 + A6 / V2  Compaction with a fused latent-memory or moment build  [IM 2.A, 2.B; MKV 1]
 *
 * Kept rows go to the caches at their slot -- Kc [b, H_kv, cap, d] (slot-major) and
 * Vc [b, H_kv, d, cap] (dim-major: element (slot, i) at Vc[.., i, slot]); one pass over all
 * of K, V folds the evicted rows in:
 *   KVM_FUSE_MEM:     n = number evicted; with eviction ranks i = 1..n (ascending position)
 *                     M <- lam^n M + sum_i lam^(n-i) v_i phi(k_i)^T,
 *                     bvec <- lam^n bvec + sum_i lam^(n-i) phi(k_i),   phi = elu + 1.
 *   KVM_FUSE_MOMENTS: n_e += n; s_k += sum k; s_v += sum v; S += sum v k^T.
 * K, V:  token-major [b, L, H_kv, d] (kv_head_major = 0) or head-major [b, H_kv, L, d].
 * slot_map: [b, L] (shared by all KV heads) or [b, H_kv, L] (per_head = 1), as produced
 *           by kvm_topk_select: selects the evicted rows and their ranks; read only when
 *           flags != 0.  n = L - keep.
 * idx:   [b, keep] (or [b, H_kv, keep]) kept positions in slot order, as produced by the same
 *        kvm_topk_select call; required when Kc/Vc are given (slot s <- position idx[s];
 *        an index outside [0, L) leaves a zero row).
 * keep:  number of kept positions per row (the caller's budget arithmetic; host value).
 * Kc/Vc may be NULL (memory/moment update only); slots >= keep are not written.  M [b,H_kv,d,d] f32 (rows index v,
 * columns index phi(k)), bvec [b,H_kv,d] f32; moments n_e [b,H_kv] i32, s_k, s_v
 * [b,H_kv,d] f32, S [b,H_kv,d,d] f32.  All state arrays are read-modify-write.
 * Supported: d in {64, 128}; cap >= keep.
 * Arithmetic: bf16 inputs use the matrix cores with exact bf16 V (or K) operands and
 * hi+lo bf16 split of lam^(n-i) phi(k) (relative error ~1e-5); fp32 inputs use fp32 FMA.
 * ------------------------------------------------------------------------------------ */
#define KVM_FUSE_MEM 1
#define KVM_FUSE_MOMENTS 2

typedef struct {
  int32_t b, L, H_kv, d, cap, keep;
  int32_t dtype;           /* kvm_dtype of K, V, Kc, Vc                                  */
  int32_t per_head;        /* slot_map per (b, KV head)                                  */
  int32_t kv_head_major;   /* layout of K, V                                             */
  int32_t flags;           /* KVM_FUSE_MEM or KVM_FUSE_MOMENTS (or 0: copy only)          */
  float lam;               /* memory decay, 0 <= lam <= 1                                */
  int32_t v_row_major;     /* 1: Vc [b, H_kv, cap, d] like Kc (input layout for a further
                              selection round); 0: the dim-major decode layout             */
} kvm_compact_desc;

size_t kvm_compact_workspace_size(const kvm_compact_desc* desc);
kvm_status kvm_compact_kv(const kvm_compact_desc* desc, const void* K, const void* V,
                          const int32_t* slot_map, const int32_t* idx, void* Kc, void* Vc,
                          float* M, float* bvec,
                          int32_t* n_e, float* s_k, float* s_v, float* S,
                          void* ws, size_t ws_bytes, void* stream);

/* Row gather that follows a slot map: dst[r, slot_map[r,t], :] = src[r, t, :] for kept t.
 * src [rows, L, elem_bytes], dst [rows, cap, elem_bytes]; elem_bytes % 4 == 0.  Used to
 * carry per-token side data (indexer keys, importance, positions) into the compact pool. */
kvm_status kvm_gather_rows(int32_t rows, int32_t L, int32_t cap, int32_t elem_bytes,
                           const void* src, const int32_t* slot_map, void* dst, void* stream);

/* ------------------------------------------------------------------------------------ *
 * A6/A7  Rank-r decayed memory update                                  [IM 2.B]
 *
 * For rows i = 1..r in the given order (per sequence and KV head):
 *   M <- lam^r M + sum_i lam^(r-i) v_i phi(k_i)^T,  bvec <- lam^r bvec + sum_i lam^(r-i) phi(k_i).
 * K_rows, V_rows: [b, r, H_kv, d] (dtype), or, with row_slot != NULL, r = 1 and the row
 * is taken from the caches Kc [b, H_kv, cap, d] and Vc [b, H_kv, d, cap] at slot
 * row_slot[b] (device i32); a sequence whose row_slot is outside [0, cap) is left as is.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t b, H_kv, d, r, cap;
  int32_t dtype;
  float lam;
} kvm_mem_desc;

kvm_status kvm_mem_update(const kvm_mem_desc* desc, const void* K_rows, const void* V_rows,
                          const int32_t* row_slot, float* M, float* bvec, void* stream);

/* ------------------------------------------------------------------------------------ *
 * V2  Moment update from evicted rows                                       [MKV part 1]
 *
 * The moment sums of each (sequence, KV head) take every evicted row, in the given order:
 *   n_e += r,  s_k += sum_i k_i,  s_v += sum_i v_i,  S += sum_i v_i k_i^T.
 * Rows as in kvm_mem_update (desc->lam is not used): K_rows, V_rows [b, r, H_kv, d]
 * (dtype), or, with row_slot != NULL, r = 1 and the row comes from the caches at slot
 * row_slot[b] (a sequence whose row_slot is outside [0, cap) is left as is).  n_e [b, H_kv]
 * i32, s_k, s_v [b, H_kv, d] f32, S [b, H_kv, d, d] f32 (rows index v, columns index k),
 * updated in place.  The same update runs fused into kvm_compact_kv (KVM_FUSE_MOMENTS)
 * when the evicted rows are those of a selection.
 * ------------------------------------------------------------------------------------ */
kvm_status kvm_moment_update(const kvm_mem_desc* desc, const void* K_rows, const void* V_rows,
                             const int32_t* row_slot, int32_t* n_e, float* s_k, float* s_v, float* S,
                             void* stream);

/* ------------------------------------------------------------------------------------ *
 * N4  Chunked pre-eviction during prefill                                   [IM 2.A]
 *
 * The indexer predicts the entries to keep before the whole prefill is held: the prefill
 * arrives in chunks, and after each the retained pool returns to the budget, so at most
 * P + C <= B + C tokens are ever held.  One call is one chunk of C tokens starting at
 * position `start`, with P tokens pooled before it:
 *   1. the chunk's K, V (token-major [b, C, H_kv, d]) and positions join the pool after its
 *      P rows.  K = V = NULL: rows P .. P+C-1 of Kp, Vp already hold the chunk's keys and
 *      values (e.g. written there by the prefill attention of the chunk), and only the
 *      positions are written;
 *   2. the chunk's indexer keys; the queries of its last W positions (Qwin [b, W, H_q, d],
 *      X rows C-W .. C-1); their scores against pool and chunk keys in position order
 *      (each window query sees every key at or before it);
 *   3. a pooled key's importance becomes the running max of its importance and the new
 *      score, a chunk key's is its max over this window (kvm_index_score's form);
 *   4. kvm_topk_select over pool and chunk (L = P + C, budget B, recent R = the chunk's
 *      last R positions), kvm_compact_kv with KVM_FUSE_MEM (evictions folded into M, bvec
 *      in ascending position order), and the kept tokens' keys, importances and positions
 *      carried into the next pool in one gather.
 * The per-chunk schedule is this library's reading of the section; one chunk covering the
 * prefill is the one-shot pre-eviction.  Pool buffers hold P + C rows per sequence (the
 * stride of every pool array is P + C): Kp, Vp [b, H_kv, P+C, d] row-major (dtype),
 * khat_p [b, P+C, d_I] f32, I_p [b, P+C] f32, pos_p [b, P+C] i32, rows 0 .. P-1 holding
 * the pool; rows P .. P+C-1 are written (I_p and khat_p in full).  The next pool has
 * stride cap_out (>= keep = kvm_chunk_keep): Kn [b, H_kv, cap_out, d]; Vn the same, or
 * dim-major [b, H_kv, d, cap_out] when `final` (the decode caches); khat_n, I_n, pos_n
 * (nullable) [b, cap_out, ..]; slots >= keep are not written.  M, bvec as in
 * kvm_compact_kv.  Requires W <= C, R <= C and the index and compaction shapes.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t b, D, H_q, H_kv, d, H_I, d_I, W;
  int32_t B, R, recent_inclusive;
  int32_t P;               /* tokens pooled before this chunk                             */
  int32_t C;               /* tokens in this chunk                                        */
  int32_t start;           /* position of the chunk's first token                         */
  int32_t cap_out;         /* row capacity of the next pool's buffers                     */
  int32_t final;           /* 1: Vn in the dim-major decode layout                        */
  int32_t dtype;
  float lam, eps_rms;
} kvm_chunk_desc;

int32_t kvm_chunk_keep(const kvm_chunk_desc* desc);
size_t kvm_chunk_workspace_size(const kvm_chunk_desc* desc);
kvm_status kvm_index_evict_chunk(const kvm_chunk_desc* desc, const void* X, const void* Qwin,
                                 const void* K, const void* V, const void* W_kI, const float* gamma_k,
                                 const void* W_qI, const float* gamma_q, const void* W_g, void* Kp,
                                 void* Vp, float* khat_p, float* I_p, int32_t* pos_p, void* Kn,
                                 void* Vn, float* khat_n, float* I_n, int32_t* pos_n, float* M,
                                 float* bvec, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ *
 * A7  Streaming eviction step during decode                    [IM 2.A; IM 2.B]
 *
 * Each sequence keeps a full pool of P tokens in slots 0..P-1 of the compact caches, with
 * per slot its position slot_pos, its normalised indexer key khat_pool and its importance
 * I_pool (initially the gathered prefill outputs: positions idx, khat and I).  For the new
 * token at position p = next_pos[b] (hidden state x_new, model query q_new):
 *   1. k_hat_new = RMSNorm_{gamma_k}(W_kI x_new);  q_hat_h, g_h as in kvm_index_score;
 *      score(k) = sum_h g_h relu(q_hat_h . k / sqrt(d_I));
 *      I_pool[j] <- max(I_pool[j], score(khat_pool[j])) for every slot; I_new = score(k_hat_new);
 *   2. candidates: slots with slot_pos <= p - R (the pool's older tokens and the one leaving
 *      the recent window); e = the candidate with the lowest I_pool, ties evicting the
 *      higher position (NaN orders as -inf, -0 as +0);
 *   3. M <- lam M + v_e phi(k_e)^T, bvec <- lam bvec + phi(k_e) per KV head, with the
 *      evicted row read from Kc [b, H_kv, cap, d] / Vc [b, H_kv, d, cap] at slot e;
 *   4. slot e takes the new token: slot_pos[e] = p, I_pool[e] = I_new, khat_pool[e] =
 *      k_hat_new; next_pos[b] = p + 1; evict_slot[b] = e.
 * The new token's K/V go into slot e with the following kvm_decode_attn_mem call
 * (append_slot = evict_slot, len = P).  The step order is this library's reading: the
 * section states that evicted tokens update the memory online during inference.
 * x_new [b, D], q_new [b, H_q, d] (dtype); W_kI, W_qI, W_g, gamma_k, gamma_q as in
 * kvm_index_score; khat_pool [b, P, d_I] f32, I_pool [b, P] f32, slot_pos [b, P] i32,
 * next_pos [b] i32 (read-modify-write); M, bvec as in kvm_mem_update; evict_slot [b] i32
 * (output; -1 if no slot qualifies, which a pool consistent with step 2 never gives).
 * Supported: d_I <= 64, H_I <= 64, d in {64, 128}, D % 8 == 0; requires P > R, cap >= P.
 * Arithmetic: fp32 projections and scores.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t b, D, H_q, H_kv, d;
  int32_t H_I, d_I;
  int32_t P;               /* pool slots per sequence (all occupied)                      */
  int32_t cap;             /* slot capacity of Kc / Vc                                    */
  int32_t R;               /* recent window                                               */
  int32_t dtype;           /* kvm_dtype of x_new, q_new, the weights and the caches       */
  float lam, eps_rms;
} kvm_stream_desc;

size_t kvm_stream_workspace_size(const kvm_stream_desc* desc);
kvm_status kvm_stream_evict(const kvm_stream_desc* desc, const void* x_new, const void* q_new,
                            const void* W_kI, const float* gamma_k, const void* W_qI,
                            const float* gamma_q, const void* W_g, float* khat_pool, float* I_pool,
                            int32_t* slot_pos, int32_t* next_pos, const void* Kc, const void* Vc,
                            float* M, float* bvec, int32_t* evict_slot, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------------------ *
 * V1  MomentKV eviction score                                         [MKV part 3]
 *
 * Per sequence bb and KV head g (rows r = bb * H_kv + g of alpha and score):
 *   alpha[r, j] = (1 / (W G)) sum_{s < W} sum_{h in group g} softmax_j(q_{s,h} . k_j * scale),
 *     the softmax over the keys j <= L - W + s that window query s (position L - W + s) sees;
 *   score[r, j] = alpha[r, j] * ||r_j||,  r_j = v_j - s_v/n_e - S~ k_j / (n_e sqrt d),
 *     S~ = S - s_v s_k^T / n_e;  r_j = v_j while n_e = 0.
 * The attention weight alpha_j as the window- and group-averaged causal softmax mass is
 * this library's reading of the section's attention weight of token j.
 * Qwin [b, W, H_q, d]; K, V [b, L, H_kv, d] (kv_head_major = 0) or [b, H_kv, L, d];
 * alpha, score [b, H_kv, L] f32; moments as in kvm_compact_kv (n_e [b,H_kv] i32, s_k,
 * s_v [b,H_kv,d], S [b,H_kv,d,d] f32).  kvm_moment_alpha needs the workspace; W G <= 256.
 * Supported: bf16 inputs, d in {64, 128}.
 * Arithmetic: logits on the matrix cores from exact bf16 operands with fp32 accumulation;
 * S~ / (n_e sqrt d) enters the residual as three bf16 terms (~24 bits).
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t b, L, H_q, H_kv, d, W;
  int32_t dtype;
  int32_t kv_head_major;
  float scale;             /* logit scale, 1/sqrt(d)                                      */
} kvm_moment_desc;

size_t kvm_moment_workspace_size(const kvm_moment_desc* desc);
kvm_status kvm_moment_alpha(const kvm_moment_desc* desc, const void* Qwin, const void* K, float* alpha,
                            void* ws, size_t ws_bytes, void* stream);
kvm_status kvm_moment_score(const kvm_moment_desc* desc, const void* K, const void* V,
                            const float* alpha, const int32_t* n_e, const float* s_k, const float* s_v,
                            const float* S, float* score, void* stream);

/* ------------------------------------------------------------------------------------ *
 * V3  MomentKV read-out from a retained-attention output              [MKV parts 2, 4]
 *
 * Per query head h (KV head g = h / G), from the retained output f_R = o_R[b, h] and its
 * log-partition lse_R[b, h] (natural log, as written by kvm_decode_attn_mem):
 *   f_E = s_v/n_e + (S q - s_v (s_k . q)/n_e) * scale / n_e;
 *   log Z_E = log n_e + (q . s_k / n_e) * scale;  w_R = sigmoid(lse_R - log Z_E);
 *   o = w_R f_R + (1 - w_R) f_E   (o = f_R where n_e = 0).
 * q [b, H_q, d] (dtype), o_R, o [b, H_q, d] f32, lse_R [b, H_q] f32; moments as above.
 * kvm_decode_attn_mem with mode KVM_READ_MOMENTS computes the same in its merge step.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t b, H_q, H_kv, d;
  int32_t dtype;
  float scale;
} kvm_mread_desc;

kvm_status kvm_moment_readout(const kvm_mread_desc* desc, const void* q, const float* o_R,
                              const float* lse_R, const int32_t* n_e, const float* s_k,
                              const float* s_v, const float* S, float* o, void* stream);

/* ------------------------------------------------------------------------------------ *
 * N1  MomentKV eviction during decode                               [MKV parts 1, 3]
 *
 * The moment sums are updated at every eviction [MKV part 1].  Each (sequence bb, KV
 * head g) keeps a full pool of P slots (slot_pos[bb, g, j] = the position held by slot j,
 * K/V in Kc / Vc as in kvm_decode_attn_mem).  For the new token at position
 * p = next_pos[bb] (query heads h of the group, G = H_q / H_kv), per (bb, g):
 *   1. alpha_j = (1/G) sum_h softmax over the pool and the new token of
 *      (q_h . k / sqrt d), taken at pooled slot j;
 *   2. score_j = alpha_j ||r_j||, r_j = v_j - s_v/n_e - S~ k_j / (n_e sqrt d),
 *      S~ = S - s_v s_k^T / n_e, r_j = v_j while n_e = 0 [MKV part 3];
 *   3. e = the slot with the lowest score among those with slot_pos <= p - R; among equal
 *      scores the higher position is evicted (NaN orders as -inf, -0 as +0);
 *   4. n_e += 1, s_k += k_e, s_v += v_e, S += v_e k_e^T (from the caches at slot e);
 *   5. slot e takes the new token: its K/V are written into Kc / Vc at slot e and
 *      slot_pos[bb, g, e] = p; evict_slot[bb, g] = e.
 * next_pos[bb] += 1.  The pages give no per-step order; steps 1-5 are this library's
 * reading (the prefill's alpha with a window of one query).  The new query's output then
 * comes from kvm_decode_attn_mem (mode KVM_READ_MOMENTS, len = P, no k_new: the token is
 * already in its slot).
 * q [b, H_q, d], k_new, v_new [b, H_kv, d] bf16; Kc [b, H_kv, cap, d], Vc [b, H_kv, d, cap]
 * bf16 (read-modify-write); slot_pos [b, H_kv, P] i32, next_pos [b] i32, n_e [b, H_kv] i32,
 * s_k, s_v [b, H_kv, d] f32, S [b, H_kv, d, d] f32 (all read-modify-write);
 * evict_slot [b, H_kv] i32 (output).  Requires P > R, cap >= P with cap a multiple of 8 (as
 * kvm_decode_attn_mem does), d in {64, 128}, G in {1, 2, 4, 8}.  Arithmetic: fp32;
 * S~ / (n_e sqrt d) enters the matrix cores as three bf16 terms against the exact bf16 keys.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t b, H_q, H_kv, d;
  int32_t P;               /* pool slots per (sequence, KV head), all occupied           */
  int32_t cap;             /* slot capacity of Kc / Vc                                    */
  int32_t R;               /* recent window                                               */
  int32_t dtype;           /* KVM_BF16                                                    */
} kvm_mstream_desc;

size_t kvm_moment_stream_workspace_size(const kvm_mstream_desc* desc);
kvm_status kvm_moment_stream_evict(const kvm_mstream_desc* desc, const void* q, const void* k_new,
                                   const void* v_new, void* Kc, void* Vc, int32_t* slot_pos,
                                   int32_t* next_pos, int32_t* n_e, float* s_k, float* s_v,
                                   float* S, int32_t* evict_slot, void* ws, size_t ws_bytes,
                                   void* stream);

/* ------------------------------------------------------------------------------------ *
 * N3  Attention-state memory (ASM)                                       [ASM Method]
 *
 * A prefix is replaced by a lookup memory of attention states.  Per query head h (KV head
 * g = h / G), with N calibration queries Q[i, h] and the prefix K, V (L tokens):
 *   kvm_asm_prefix_states:  a[i, h] = sum_t softmax_t(Q[i,h] . K[t,g] / sqrt d) V[t,g],
 *                           lse[i, h] = log sum_t exp(Q[i,h] . K[t,g] / sqrt d); with
 *                           accumulate != 0 the call covers one more chunk of the prefix and
 *                           merges into the states in a, lse by the online-softmax identity
 *                           (a long prefix encoded chunk by chunk, one chunk's K/V resident);
 *   kvm_asm_kmeans:         Lloyd's iteration on the queries of each head: `iters` rounds of
 *                           (assign to the nearest centroid by squared Euclidean distance,
 *                           ties to the lower index; centroid = mean of its members, a
 *                           centroid without members stays), then a final assignment;
 *                           C [H_q, K, d] f32 holds the initial centroids on entry and the
 *                           final ones on return, idx [H_q, N] i32 the final assignment;
 *   kvm_asm_cluster_states: per cluster k the members' states merged with the online-softmax
 *                           rule and the mean partition:
 *                           a_bar[h, k] = sum_i Z_i a_i / sum_i Z_i (Z_i = exp lse_i),
 *                           lse_bar[h, k] = log(sum_i Z_i / n_k)  (-inf, a_bar = 0 if n_k = 0;
 *                           entries of idx outside [0, K) join no cluster);
 *   kvm_asm_lookup:         for decode queries q [b, H_q, d]: k = the centroid of head h with
 *                           the largest cosine similarity (ties: the lower index; a centroid at
 *                           the origin is never chosen), and the merge with the query's local
 *                           state (o_loc, lse_loc, e.g. from kvm_decode_attn_mem over the tokens
 *                           after the prefix): lse = log(e^lse_loc + e^lse_bar[h,k]),
 *                           o = e^(lse_loc - lse) o_loc + e^(lse_bar - lse) a_bar[h, k].
 * The mean partition, the distance used for clustering and the cosine retrieval without
 * whitening are this library's readings of the section.
 * Q [N, H_q, d], q [b, H_q, d] bf16; K, V [L, H_kv, d] bf16 (or [H_kv, L, d] if
 * kv_head_major); a, o_loc, o [.., H_q, d] f32; lse, lse_loc, lse_out [.., H_q] f32;
 * a_bar [H_q, K, d], lse_bar [H_q, K] f32; idx_out [b, H_q] i32.  Supported: d in
 * {64, 128}, K <= 256, bf16.  Arithmetic: fp32 distances and sums; the prefix attention on
 * the matrix cores with fp32 accumulation and P as bf16 hi + lo.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t N;               /* calibration queries per head                                */
  int32_t H_q, H_kv, d;
  int32_t L;               /* prefix tokens                                               */
  int32_t K;               /* centroids per head                                          */
  int32_t dtype;           /* KVM_BF16                                                    */
  int32_t kv_head_major;   /* prefix K/V layout                                           */
} kvm_asm_desc;

size_t kvm_asm_workspace_size(const kvm_asm_desc* desc);
kvm_status kvm_asm_prefix_states(const kvm_asm_desc* desc, const void* Q, const void* K, const void* V,
                                 float* a, float* lse, int32_t accumulate, void* stream);
kvm_status kvm_asm_kmeans(const kvm_asm_desc* desc, const void* Q, float* C, int32_t* idx, int32_t iters,
                          void* ws, size_t ws_bytes, void* stream);
kvm_status kvm_asm_cluster_states(const kvm_asm_desc* desc, const float* a, const float* lse,
                                  const int32_t* idx, float* a_bar, float* lse_bar, void* ws,
                                  size_t ws_bytes, void* stream);
kvm_status kvm_asm_lookup(const kvm_asm_desc* desc, int32_t b, const void* q, const float* C,
                          const float* a_bar, const float* lse_bar, const float* o_loc,
                          const float* lse_loc, float* o, float* lse_out, int32_t* idx_out,
                          void* stream);

/* ------------------------------------------------------------------------------------ *
 * A8 + A9 / V3  Split-K decode attention with memory read-out          [IM 2.B; ASM; MKV 4]
 *
 * Per sequence bb and query head h (KV head g = h / G, G = H_q / H_kv):
 *   the new token (k_new, v_new) takes slot app = len[bb] (or append_slot[bb]); attention
 *   is over the first n = len[bb] + 1 slots (len[bb] if append_slot is given, or if k_new
 *   is NULL), n clamped to cap; when app < n the new token is attended and written into
 *   both caches at slot app (the slot's old contents are never read), otherwise it is
 *   neither.  The cached slots are reduced to n_split partial states (a_c, lse_c) over
 *   disjoint slot sets (bf16 d = 128: 128-slot chunks dealt round robin; otherwise
 *   contiguous ranges), the new token is one more state (v_new, scale q.k_new), and the
 *   states merge in a fixed order by lse = log sum_c exp(lse_c), a = sum_c exp(lse_c - lse) a_c;
 *   mode KVM_READ_NONE:    o = a
 *   mode KVM_READ_MEMORY:  m = M_g phi(q~) / (bvec_g . phi(q~) + eps), o = a + sigmoid(w_g[h].q) m,
 *                          q~ = q_mem[bb, h] if q_mem is given (the projected query, see
 *                          kvm_mem_query), else q
 *   mode KVM_READ_MOMENTS: f_E = s_v/n_e + (S - s_v s_k^T/n_e) q / (n_e sqrt d),
 *                          log Z_E = log n_e + (q.s_k/n_e)/sqrt d,
 *                          w = sigmoid(lse - log Z_E), o = w a + (1 - w) f_E (o = a if n_e = 0)
 * q [b,H_q,d], k_new/v_new [b,H_kv,d] (dtype, nullable), Kc [b,H_kv,cap,d] slot-major and
 * Vc [b,H_kv,d,cap] dim-major (dtype; as written by kvm_compact_kv), cap % 8 == 0 (a
 * multiple of 64 keeps every V row on 128-byte lines, the bandwidth-friendly choice),
 * len [b] i32 (not modified), append_slot [b] i32 (nullable), q_mem [b,H_q,d] (dtype,
 * nullable; only with KVM_READ_MEMORY, else KVM_ERR_RANGE), o [b,H_q,d] f32,
 * lse [b,H_q] f32 (nullable: log-partition of the retained attention, scale applied).
 * The library never reads or writes a slot >= cap (n is clamped to cap).
 * Supported: d in {64, 128}, G in {1, 2, 4, 8}, cap <= 8388607; n_split 0 chooses
 * automatically (the most splits that keep the grid within one even round on the chip).
 * ------------------------------------------------------------------------------------ */
#define KVM_READ_NONE 0
#define KVM_READ_MEMORY 1
#define KVM_READ_MOMENTS 2

typedef struct {
  int32_t b, H_q, H_kv, d, cap;
  int32_t n_split;         /* 0 = auto                                                  */
  int32_t dtype;           /* of q, k_new, v_new, Kc, Vc, w_g                           */
  int32_t mode;            /* KVM_READ_*                                                */
  float scale;             /* logit scale, normally 1/sqrt(d)                            */
  float eps;               /* read-out epsilon (1e-6)                                    */
} kvm_decode_desc;

size_t kvm_decode_workspace_size(const kvm_decode_desc* desc);
kvm_status kvm_decode_attn_mem(const kvm_decode_desc* desc, const void* q, const void* k_new,
                               const void* v_new, const int32_t* append_slot, void* Kc, void* Vc,
                               const int32_t* len, const float* M, const float* bvec,
                               const void* w_g, const void* q_mem, const int32_t* n_e,
                               const float* s_k, const float* s_v, const float* S, float* o,
                               float* lse, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory or hand over a workspace: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * kvm_decode_attn_mem_noalloc takes the arguments of kvm_decode_attn_mem minus (ws,
 * ws_bytes) and computes the same result with the same kernels; its split states live in a
 * fixed device array of kvm_decode_noalloc_max_bytes() bytes (4 MiB) that the library holds
 * on each GPU it runs on until the process ends.  It calls no allocator.  A shape whose
 * split states need more than that (kvm_decode_workspace_size(desc) > the maximum) returns
 * KVM_ERR_WORKSPACE before any HIP call.  Every call on one GPU uses that GPU's array, so
 * calls that overlap in time on one GPU (two streams or two threads) race: the caller
 * serialises them.  The array needs no clearing between calls: a call writes every word of
 * it that it reads. */
size_t kvm_decode_noalloc_max_bytes(void);
kvm_status kvm_decode_attn_mem_noalloc(const kvm_decode_desc* desc, const void* q, const void* k_new,
                                       const void* v_new, const int32_t* append_slot, void* Kc, void* Vc,
                                       const int32_t* len, const float* M, const float* bvec,
                                       const void* w_g, const void* q_mem, const int32_t* n_e,
                                       const float* s_k, const float* s_v, const float* S, float* o,
                                       float* lse, void* stream);

/* ------------------------------------------------------------------------------------ *
 * N2  The read-out projection (slow weights)                                [IM 2.B]
 *
 * The pages name a trained projection layer that, with the gate, reads the memory.  This
 * library's reading: one d x d matrix W_m per layer, shared by every query head, maps the
 * query that addresses M:  q_mem[r] = W_m q[r]  for each row r of q [rows, d]
 * (rows = b * H_q), fp32 accumulation, stored in dtype (bf16: round to nearest even).
 * Pass q_mem to kvm_decode_attn_mem; the gate keeps the model query.  W_m = I gives the
 * read-out without projection.  q, q_mem [rows, d] and W_m [d, d] (row i gives output
 * dim i) in dtype; q_mem must not alias q.  Supported: d in {64, 128}.
 * ------------------------------------------------------------------------------------ */
kvm_status kvm_mem_query(int32_t rows, int32_t d, int32_t dtype, const void* q, const void* W_m,
                         void* q_mem, void* stream);

/* len[i] += delta for i < b (device i32): advances cache lengths between decode steps. */
kvm_status kvm_len_add(int32_t* len, int32_t b, int32_t delta, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVM_H */
