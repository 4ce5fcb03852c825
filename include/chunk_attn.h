/*
 * chunk_attn.h - exact causal attention for one sequence chunk on MI355X (gfx950).
 *
 * The operation. A long sequence of T positions is cut into chunks; chunk i
 * starts at global position s_i and holds C_i positions. Its queries Q^(i)
 * attend to the cached key/value prefix K^(:i), V^(:i) (rows [0, s_i + C_i))
 * under the causal mask, query row r (global position s_i + r) seeing key j
 * iff j <= s_i + r. StreamBP's Property 3.1 says that chunk i's backward needs
 * only O^(i), Q^(i), K^(:i), V^(:i), and its Eq. (1) says that summing the
 * per-chunk contributions gives the full-sequence gradient (StreamBP review,
 * "What carries the argument"; Eqs. (12)-(14) for the partitioned attention).
 * SeCO keeps the K/V caches as checkpoints and backpropagates one chunk at a
 * time; SpaCO backpropagates only t of the k chunks and scales them by k/t
 * (SeCO/SpaCO review, "What carries the argument" and Referee Report summary).
 *
 * Per query head h (kv head h / (Hq/Hkv)):
 *   S = scale * Q^(i) K^(:i)^T (masked), LSE = ln sum exp S, P = exp(S - LSE),
 *   O^(i) = P V^(:i);  backward: dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
 *   dQ^(i) = scale dS K,  dK^(:i) += scale dS^T Q^(i),  dV^(:i) += P^T dO.
 *
 * Tensor layout. All tensors are row-major [batch][heads][rows][head_dim] with
 * head_dim contiguous: q, o, dout, dq have n_q_heads heads and q_capacity rows;
 * k, v, dk_acc, dv_acc have n_kv_heads heads and kv_capacity rows; lse is
 * [batch][n_q_heads][q_capacity]. The chunk's rows inside the q-side tensors
 * begin at q_row_offset (0 for per-chunk tensors, s_i for whole-sequence ones).
 * q, k, v, o, dout are float32 or bfloat16 (dtype); lse, dq, dk_acc, dv_acc
 * are always float32. Device pointers must be 16-byte aligned.
 *
 * Ownership and ordering. The caller allocates and owns every buffer,
 * including the workspace; the library keeps no device memory of its own and
 * frees nothing. Work is enqueued on the caller's HIP stream (a hipStream_t
 * passed as void*; NULL is the default stream) and returns before it runs.
 * Outputs must not alias inputs or each other.
 *
 * Errors. Every function returns 0 on success or a negative CA_ERR_* code. All
 * argument checks happen before any device call, so a rejected call enqueues
 * nothing. chunk_attn_last_error() gives a detail string for the calling
 * thread. No C++ exception crosses this boundary.
 */
#ifndef CHUNK_ATTN_H
#define CHUNK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CA_OK = 0,
  CA_ERR_NULL = -1,        /* a required pointer is NULL */
  CA_ERR_SHAPE = -2,       /* sizes out of range or inconsistent */
  CA_ERR_DTYPE = -3,       /* dtype is not CA_F32 or CA_BF16 */
  CA_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
  CA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
  CA_ERR_UNSUPPORTED = -6, /* head_dim other than 64 or 128 */
  CA_ERR_HIP = -7          /* the HIP runtime reported an error */
};

enum { CA_F32 = 0, CA_BF16 = 1 };

enum { CA_OP_FWD = 0, CA_OP_BWD = 1, CA_OP_SPARSE_BWD = 2, CA_OP_BWD_MIN = 3, CA_OP_BWD_DS = 4 };

typedef struct {
  int32_t batch;         /* >= 1 */
  int32_t n_q_heads;     /* Hq >= 1, a multiple of n_kv_heads */
  int32_t n_kv_heads;    /* Hkv >= 1; q head h reads kv head h / (Hq/Hkv) */
  int32_t head_dim;      /* 64 or 128 */
  int32_t kv_capacity;   /* rows per head in k, v, dk_acc, dv_acc; >= chunk_start + chunk_len */
  int32_t q_capacity;    /* rows per head in q, o, dout, dq, lse; >= q_row_offset + chunk_len */
  int32_t q_row_offset;  /* row of the chunk's first query in the q-side tensors */
  int32_t chunk_start;   /* s_i: global position of the chunk's first query, >= 0 */
  int32_t chunk_len;     /* C_i >= 1 */
  float softmax_scale;   /* multiplies Q K^T; any finite value */
  int32_t dtype;         /* CA_F32 or CA_BF16: type of q, k, v, o, dout */
} chunk_attn_desc;

/* Bytes of workspace for the op on this descriptor (0 if none; the op then
 * accepts ws == NULL). op is CA_OP_*. For CA_OP_SPARSE_BWD the descriptor is
 * the whole-sequence one that sparse_chunk_bwd takes and chunk_len must be the
 * chunk size. Returns 0 for an invalid descriptor.
 *
 * CA_OP_BWD and CA_OP_BWD_MIN (the same size) give what the backward needs:
 * the chunk's row statistics, 8 bytes per row of batch * n_q_heads *
 * chunk_len (rounded up), independent of the sequence length and the
 * capacities, as the method's per-chunk working set asks (StreamBP review,
 * "What carries the argument"). The dQ pass then recomputes S, P and dP from
 * Q, K, V, dO and the row statistics. CA_OP_SPARSE_BWD gives two such slots:
 * with them the whole-sequence drivers (sparse_chunk_bwd, chunked_bwd_sweep)
 * compute the next chunk's row statistics in the same launch as this chunk's
 * backward instead of in a launch of their own (one slot is enough for them
 * to run).
 *
 * CA_OP_BWD_DS (either descriptor) adds, for bf16, room for a chunk's dS^T in
 * bf16: batch * n_q_heads * chunk_len * kv_capacity * 2 bytes, rows and keys
 * rounded up to 128 (1.07 GB for 32 heads, 1024-row chunks and 16384 keys),
 * so it grows with the sequence. Given that much workspace, chunk_attn_bwd and
 * sparse_chunk_bwd hand dS from the dK/dV pass to the dQ pass (dQ = dS K)
 * instead of recomputing it: faster, at memory that scales with the prefix.
 * The results agree within rounding. */
size_t chunk_attn_workspace_size(const chunk_attn_desc* desc, int32_t op);

/* Forward of one chunk (the inference-mode pass that fills the caches in SeCO,
 * SeCO/SpaCO review Referee Report summary; StreamBP Eq. (13) partitioned
 * softmax). Writes o rows [q_row_offset, +chunk_len) in dtype and lse (natural
 * log of the row's sum of exp(S)) in float32. Reads k, v rows [0, chunk_start +
 * chunk_len). ws may be NULL (no workspace needed). */
int chunk_attn_fwd(const chunk_attn_desc* desc, const void* q, const void* k, const void* v,
                   void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward of one chunk (StreamBP Property 3.1: needs only O^(i), Q^(i),
 * K^(:i), V^(:i); Eq. (1): chunk contributions add up to the full gradient).
 * o and lse are this chunk's forward outputs. dq rows of the chunk are
 * OVERWRITTEN with grad_scale * dQ^(i); dk_acc and dv_acc rows
 * [0, chunk_start + chunk_len) are INCREMENTED by grad_scale * dK^(:i) and
 * grad_scale * dV^(:i) without atomics (each element has one writer), so the
 * caller zeroes them before the first chunk of a sweep and chunks of one sweep
 * must be issued in stream order. grad_scale is SpaCO's k/t for a sparse sweep
 * and 1 otherwise. Workspace: at least chunk_attn_workspace_size(desc,
 * CA_OP_BWD) bytes; chunk_attn_workspace_size(desc, CA_OP_BWD_DS) bytes select
 * the dS hand-over for bf16. */
int chunk_attn_bwd(const chunk_attn_desc* desc, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dout, float grad_scale,
                   float* dq, float* dk_acc, float* dv_acc, void* ws, size_t ws_bytes,
                   void* stream);

/* chunk_attn_bwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Arguments, outputs and ordering as chunk_attn_bwd. The
 * chunk's row statistics (8 bytes per row of batch * n_q_heads * chunk_len,
 * rounded up) go to a static device array of 8 MiB that every device holds
 * for the life of the process, so batch * n_q_heads * chunk_len may not
 * exceed about one million rows (CA_ERR_WORKSPACE beyond). dQ is recomputed
 * (the pass chunk_attn_bwd takes with its minimal workspace); results equal
 * chunk_attn_bwd's with a CA_OP_BWD workspace. Calls no allocator. stream
 * must belong to the current device (CA_ERR_SHAPE otherwise). Every call on a
 * device shares that device's array: calls that overlap on one device (other
 * streams, other threads) race and give wrong results. */
int chunk_attn_bwd_noalloc(const chunk_attn_desc* desc, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, float grad_scale,
                           float* dq, float* dk_acc, float* dv_acc, void* stream);

/* acc[b][h][r][:] += scale * src[b][h][r][:] for r < prefix_len (float32,
 * device pointers). This is the relay of an accumulated cache gradient,
 * m_i.grad <- (k/t) * m'_i.grad in SpaCO (SeCO/SpaCO review, Referee Report
 * major comments on Section 5 and Algorithm 2). acc has acc_capacity rows per
 * head, src has src_capacity; both need prefix_len <= capacity. */
int prefix_grad_accumulate(float* acc, const float* src, int32_t batch, int32_t n_heads,
                           int32_t acc_capacity, int32_t src_capacity, int32_t head_dim,
                           int32_t prefix_len, float scale, void* stream);

/* SpaCO's chunk sample: t distinct indices out of [0, k), without replacement
 * (SeCO/SpaCO review, Referee Report major comment 1). The random source is
 * SplitMix64 seeded with seed, driving a partial Fisher-Yates shuffle of
 * 0..k-1 stopped after t swaps (swap position i with i + next() mod (k - i));
 * the chosen indices are written to the host array out_sorted[t] in ascending
 * order. Pure host code. Errors: CA_ERR_NULL, CA_ERR_SHAPE (t < 1 or t > k). */
int chunk_select(int32_t k, int32_t t, uint64_t seed, int32_t* out_sorted);

/* Sparse chunk backward over a whole sequence of seq_len positions cut into
 * k = ceil(seq_len / chunk_len) chunks of desc->chunk_len (the last may be
 * short). Selects t chunks with chunk_select(k, t, seed), zeroes dq, dk, dv,
 * then runs chunk_attn_bwd on the selected chunks in descending order with
 * grad_scale = k/t, the compensation factor SpaCO applies to the selected
 * chunks (SeCO/SpaCO review, "What carries the argument"). With t = k it is
 * the exact chunked backward (SeCO). q, o, dout, dq, lse are whole-sequence
 * tensors (q_capacity >= seq_len) and o, lse come from forwards of all
 * chunks; desc->chunk_start and q_row_offset are ignored. The selected indices
 * go to the host array selected_out[t]. Workspace: at least
 * chunk_attn_workspace_size(desc, CA_OP_BWD) bytes; CA_OP_SPARSE_BWD's size
 * (two slots of row statistics) saves a launch per chunk, CA_OP_BWD_DS's selects
 * the dS hand-over. */
int sparse_chunk_bwd(const chunk_attn_desc* desc, int32_t seq_len, int32_t t, uint64_t seed,
                     const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv,
                     int32_t* selected_out, void* ws, size_t ws_bytes, void* stream);

/* The chunk schedule of a whole sequence of seq_len positions in chunks of
 * desc->chunk_len (chunk i starts at s_i = i * chunk_len and holds
 * min(chunk_len, seq_len - s_i) positions; the last may be short), computed
 * here rather than by the caller. desc is the whole-sequence descriptor:
 * q, o, dout, dq, lse hold every position (q_capacity >= seq_len) and k, v,
 * dk_acc, dv_acc every key (kv_capacity >= seq_len); chunk_start and
 * q_row_offset are ignored. SeCO runs the inference-mode pass over the chunks
 * in order, then backpropagates them one at a time from the last (SeCO/SpaCO
 * review, Referee Report summary).
 *
 * chunked_fwd_sweep: chunk_attn_fwd of every chunk, ascending; writes o and
 * lse rows [0, seq_len). */
int chunked_fwd_sweep(const chunk_attn_desc* desc, int32_t seq_len, const void* q, const void* k,
                      const void* v, void* o, float* lse, void* stream);

/* chunked_bwd_sweep: chunk_attn_bwd of every chunk, descending, with
 * grad_scale. dq rows [0, seq_len) are OVERWRITTEN; dk_acc and dv_acc rows
 * [0, seq_len) are INCREMENTED by the full gradient (zero them first for the
 * gradient alone). Workspace as for sparse_chunk_bwd (at least the CA_OP_BWD
 * size; the CA_OP_SPARSE_BWD size saves a launch per chunk; CA_OP_BWD_DS
 * selects the dS hand-over). Errors as for sparse_chunk_bwd. */
int chunked_bwd_sweep(const chunk_attn_desc* desc, int32_t seq_len, const void* q, const void* k,
                      const void* v, const void* o, const float* lse, const void* dout, float grad_scale,
                      float* dq, float* dk_acc, float* dv_acc, void* ws, size_t ws_bytes, void* stream);

/* The projections on either side of the attention of chunk i, which complete
 * one attention layer's chunked backward. The layer input H_in is
 * [batch][h_capacity][d_model] in dtype, the chunk's positions at rows
 * h_row_offset.. (+chunk_len); wq is [d_model][n_q_heads*head_dim] and wk, wv
 * [d_model][n_kv_heads*head_dim], row-major in dtype; column h*head_dim + c of a
 * projection is element c of head h. d_model must be a multiple of 64.
 *
 * qkv_proj_fwd: Q^(i) = H_in^(i) W_q into q rows [q_row_offset, +chunk_len) of
 * every q head, and K^(i) = H_in^(i) W_k, V^(i) = H_in^(i) W_v into k, v rows
 * [chunk_start, +chunk_len) (appending the chunk to the caches), in dtype.
 *
 * qkv_proj_bwd: the attention weight gradients of the StreamBP review, major
 * comment 1: dW_q += H_in^(i)^T dQ^(i), and dW_k += H_in^T dK, dW_v += H_in^T dV.
 * The review writes the last two per chunk over the prefix; summed over the
 * chunks they equal H_in^T times the accumulated dK, dV, and here each chunk
 * takes its own rows [chunk_start, +chunk_len) of dk_acc, dv_acc, which are
 * final once chunk_attn_bwd of that chunk has run in a descending sweep (no
 * later chunk touches them). Also writes the input gradient of the chunk's
 * rows, dh = dQ W_q^T + dK W_k^T + dV W_v^T (float32, OVERWRITTEN;
 * [batch][h_capacity][d_model], same rows as H_in). dq is the float32 output of
 * chunk_attn_bwd for this chunk; dwq, dwk, dwv are float32 accumulators of the
 * weights' shapes, INCREMENTED (the caller zeroes them before a sweep). The
 * float32 gradients are rounded to dtype before they enter the products
 * (float32 accumulation). ws: qkv_proj_bwd_workspace_size(desc, d_model)
 * bytes of device memory, 16-byte aligned, owned by the caller (contents on
 * return unspecified). Errors as for chunk_attn_fwd, plus CA_ERR_SHAPE for
 * d_model or the H_in rows and CA_ERR_WORKSPACE for a missing or short ws. */
/* Workspace bytes qkv_proj_bwd needs (0 for float32 layers; bf16 layers hold
 * the chunk's gradients, batch * round_up(chunk_len, 64) rows of
 * (Hq + 2 Hkv) * head_dim, and the weights' transpose, (Hq + 2 Hkv) * head_dim
 * rows of d_model, both in bf16). Returns 0 for invalid arguments. */
size_t qkv_proj_bwd_workspace_size(const chunk_attn_desc* desc, int32_t d_model);
int qkv_proj_fwd(const chunk_attn_desc* desc, int32_t d_model, int32_t h_capacity, int32_t h_row_offset,
                 const void* h, const void* wq, const void* wk, const void* wv, void* q, void* k, void* v,
                 void* stream);
int qkv_proj_bwd(const chunk_attn_desc* desc, int32_t d_model, int32_t h_capacity, int32_t h_row_offset,
                 const void* h, const void* wq, const void* wk, const void* wv, const float* dq,
                 const float* dk_acc, const float* dv_acc, float* dwq, float* dwk, float* dwv, float* dh,
                 void* ws, size_t ws_bytes, void* stream);

/* The bf16 backward's input gradient reads the weights transposed, W_cat^T =
 * [wq | wk | wv]^T ((n_q_heads + 2 n_kv_heads) * head_dim rows of d_model,
 * bf16); qkv_proj_bwd writes that transpose into its workspace on every call.
 * A backward sweep over a layer's chunks (the StreamBP review, major comment 1:
 * every chunk's gradients meet the same weights) can instead write it once
 * with qkv_proj_weights_t and hand it to qkv_proj_bwd_wt for each chunk.
 *
 * qkv_proj_weights_t_bytes: bytes of W_cat^T for a bf16 layer (0 for float32
 * layers and for invalid arguments).
 * qkv_proj_weights_t: writes W_cat^T of wq, wk, wv (layouts as above) into
 * w_cat_t (qkv_proj_weights_t_bytes bytes of device memory, 16-byte aligned,
 * owned by the caller). bf16 layers only (CA_ERR_DTYPE otherwise); other errors
 * as for qkv_proj_fwd.
 * qkv_proj_bwd_wt: qkv_proj_bwd with the transpose given. For a bf16 layer,
 * w_cat_t must hold what qkv_proj_weights_t wrote for these same weights (the
 * call reads it and never checks it; stale contents give wrong dh), and ws
 * needs only qkv_proj_bwd_workspace_size - qkv_proj_weights_t_bytes bytes.
 * For a float32 layer w_cat_t is ignored (may be NULL) and the call is
 * qkv_proj_bwd. Results equal qkv_proj_bwd's bit for bit. */
size_t qkv_proj_weights_t_bytes(const chunk_attn_desc* desc, int32_t d_model);
int qkv_proj_weights_t(const chunk_attn_desc* desc, int32_t d_model, const void* wq, const void* wk, const void* wv,
                       void* w_cat_t, void* stream);
int qkv_proj_bwd_wt(const chunk_attn_desc* desc, int32_t d_model, int32_t h_capacity, int32_t h_row_offset,
                    const void* h, const void* wq, const void* wk, const void* wv, const void* w_cat_t,
                    const float* dq, const float* dk_acc, const float* dv_acc, float* dwq, float* dwk, float* dwv,
                    float* dh, void* ws, size_t ws_bytes, void* stream);

/* ---- SpaCO over a stack of attention layers ------------------------------
 *
 * The relay of SpaCO's Algorithm 2 (SeCO/SpaCO review, Referee Report major
 * comments on Section 5 / Algorithm 2 and on Section 6.4; "Assumptions"): KV
 * caches of every layer are filled in one inference-mode pass; then each
 * drawn chunk j, from the last to the first, has its graph rebuilt from the
 * caches and is backpropagated from its own loss term together with the
 * gradient that later drawn chunks accumulated into its cache rows, that
 * relayed gradient multiplied by relay_factor (line 7, m_j.grad <- (k/t)
 * m'_j.grad; the deployed method caps the factor at 2). Cache gradients of
 * chunks that are not drawn are dropped. All chunks drawn with relay_factor 1
 * is SeCO's exact gradient.
 *
 * The stack: layer l maps H_l [batch][h_capacity][d_model] (d_model =
 * n_q_heads * head_dim) to H_{l+1} = H_l + O_l, O_l the chunked causal
 * attention of Q, K, V = H_l W_q^l, H_l W_k^l, H_l W_v^l with the heads side
 * by side; the loss gradient dJ/dH_L = dy is given.
 *
 * The descriptor is the whole-sequence one: chunk_len is the chunk size C,
 * kv_capacity the cache rows (>= seq_len), q_capacity >= C; chunk_start and
 * q_row_offset are ignored. */
typedef struct {
  const void* wq;  /* [d_model][n_q_heads*head_dim], dtype */
  const void* wk;  /* [d_model][n_kv_heads*head_dim], dtype */
  const void* wv;
  void* k_cache;   /* [batch][n_kv_heads][kv_capacity][head_dim], dtype */
  void* v_cache;
  float* dk_acc;   /* [batch][n_kv_heads][kv_capacity][head_dim] float32 (m.grad; zeroed by the backward) */
  float* dv_acc;
  float* dwq;      /* weight gradients, float32, INCREMENTED */
  float* dwk;
  float* dwv;
} spaco_layer;

/* Workspace bytes for spaco_stack_forward / spaco_stack_backward (chunk-local
 * activations of every layer, the chunk's gradients, the attention and
 * projection workspaces; the attention part is chunk_attn_workspace_size(desc,
 * CA_OP_BWD), so the stack's dQ passes recompute dS). 0 for invalid
 * arguments. */
size_t spaco_stack_workspace_size(const chunk_attn_desc* desc, int32_t n_layers);

/* Inference-mode pass: every chunk in ascending order through every layer,
 * writing rows [0, seq_len) of each layer's k_cache and v_cache. h0 is the
 * stack input [batch][h_capacity][d_model] in dtype. Only wq, wk, wv, k_cache
 * and v_cache of each layer are used. */
int spaco_stack_forward(const chunk_attn_desc* desc, int32_t seq_len, int32_t n_layers, const spaco_layer* layers,
                        const void* h0, int32_t h_capacity, void* ws, size_t ws_bytes, void* stream);

/* SpaCO's relayed backward over the drawn chunks `chunks` (n_chunks distinct
 * 0-based indices in any order; processed from the last to the first) after
 * spaco_stack_forward has filled the caches. dy [batch][h_capacity][d_model]
 * float32 is dJ/dH_L; dh0 (same shape) receives dJ/dH_0 on the drawn chunks'
 * rows (other rows untouched). Zeroes every layer's dk_acc/dv_acc first;
 * increments dwq/dwk/dwv. relay_factor: finite. Errors as for sparse_chunk_bwd,
 * plus CA_ERR_SHAPE for d_model != n_q_heads * head_dim, d_model not a
 * multiple of 64, or a chunk index out of range or repeated. */
int spaco_stack_backward(const chunk_attn_desc* desc, int32_t seq_len, int32_t n_layers, const spaco_layer* layers,
                         const void* h0, const float* dy, float* dh0, int32_t h_capacity, const int32_t* chunks,
                         int32_t n_chunks, float relay_factor, void* ws, size_t ws_bytes, void* stream);

/* ---- Streamed language-model head, supervised fine-tuning ----------------
 *
 * StreamBP streams the LM head by partitioning the logits along the sequence
 * (ps_head = 100 positions at a time), the SFT loss being separable over
 * positions (StreamBP review, "Core claim"; "Assumptions": Eq. (3), ps_head).
 * With logits z_t = W h_t and labels y_t (-1: not a target), the loss is
 * loss_scale * sum_t (logsumexp(z_t) - z_t[y_t]) over target positions, and
 *   dz_t = loss_scale * (softmax(z_t) - onehot(y_t)),  dh_t = W^T dz_t,
 *   dW += sum_t dz_t h_t^T.
 * Only the partition's logits exist at a time (in the workspace). */
typedef struct {
  int32_t batch;         /* >= 1 */
  int32_t seq_capacity;  /* rows per batch entry in h, labels, row_loss and dh */
  int32_t d_model;       /* multiple of 64, <= 65536 */
  int32_t vocab;         /* multiple of 64 */
  int32_t dtype;         /* CA_BF16 (the only supported storage type; else CA_ERR_UNSUPPORTED) */
} lm_head_desc;

/* wt [d_model][vocab] = w^T for w [vocab][d_model] (bf16, device). The
 * partition call reads the logits product's weight operand from wt; call once
 * per weight update. */
int lm_head_transpose(const lm_head_desc* desc, const void* w, void* wt, void* stream);

/* Workspace bytes of lm_head_sft_partition for partitions of up to `rows`
 * positions: the partition's float32 logits and bf16 logit gradients (0 for
 * invalid arguments). */
size_t lm_head_sft_workspace_size(const lm_head_desc* desc, int32_t rows);

/* One partition, positions [row_start, row_start + rows) of every batch entry:
 * h [batch][seq_capacity][d_model] bf16; w [vocab][d_model] bf16 and its
 * transpose wt; labels [batch][seq_capacity] int32 (a position is a target iff
 * 0 <= label < vocab; other values, e.g. -1, mark prompt or padding positions);
 * row_weight [batch][seq_capacity] float32 or NULL: a per-position weight of
 * the gradient (dz_t = loss_scale * row_weight_t * (softmax - onehot)); NULL is
 * 1 everywhere (SFT). GRPO takes A_i / (G |o_i|) on the positions of response i
 * (the on-policy policy gradient of Eq. (6)); DPO takes +1 on the chosen and -1
 * on the rejected response, then lm_head_dpo_finish. loss_scale multiplies the gradients
 * (1 / number of targets for a mean). Writes row_loss [batch][seq_capacity]
 * float32 (the unscaled loss of each position of the partition, 0 for
 * non-targets) and dh rows of the partition (float32, OVERWRITTEN); adds into
 * dw [vocab][d_model] float32. Errors: CA_ERR_NULL / CA_ERR_ALIGN for
 * pointers, CA_ERR_SHAPE for sizes or rows outside the capacity,
 * CA_ERR_UNSUPPORTED for a dtype other than bf16, CA_ERR_WORKSPACE. */
int lm_head_sft_partition(const lm_head_desc* desc, int32_t row_start, int32_t rows, const void* h, const void* w,
                          const void* wt, const int32_t* labels, const float* row_weight, float loss_scale,
                          float* row_loss, float* dh, float* dw, void* ws, size_t ws_bytes, void* stream);

/* The whole streamed sweep over positions [0, seq_len): partitions of ps
 * positions in order, each as lm_head_sft_partition, except that the weight
 * gradient is added once per dw_group consecutive partitions, from their
 * logit gradients (bf16) kept in the workspace; logits still exist for one
 * partition at a time. dw_group = 1 adds it after every partition. Arguments,
 * outputs and errors as for lm_head_sft_partition; ws:
 * lm_head_sft_sweep_workspace_size(desc, ps, dw_group) bytes. */
size_t lm_head_sft_sweep_workspace_size(const lm_head_desc* desc, int32_t ps, int32_t dw_group);
int lm_head_sft_sweep(const lm_head_desc* desc, int32_t seq_len, int32_t ps, int32_t dw_group, const void* h,
                      const void* w, const void* wt, const int32_t* labels, const float* row_weight,
                      float loss_scale, float* row_loss, float* dh, float* dw, void* ws, size_t ws_bytes,
                      void* stream);

/* DPO's final scalar (StreamBP review, "Assumptions": Eqs. (8)-(10), the loss is
 * not separable but its gradient factorizes with a scalar known only at the
 * end). For one preference pair, batch entry 0 chosen and 1 rejected, after a
 * sweep over positions [0, seq_len) with row weights +1 / -1 and loss_scale 1:
 * lp_b = -(sum of entry b's row losses), margin = (lp_0 - ref_logp_chosen) -
 * (lp_1 - ref_logp_rejected), loss = -log sigmoid(beta * margin), and dh (rows
 * [0, seq_len) of both entries) and dw are multiplied by c = beta *
 * sigmoid(-beta * margin). The multiplication covers the whole of dw and
 * those dh rows, so they must hold this pair's sweep only: zero dw before the
 * pair's sweep, and to accumulate over several pairs or microbatches, sweep
 * each pair into a zeroed buffer, finish it, then add it to the accumulator.
 * Copies the row losses to the host (synchronizes the stream). Writes
 * *loss_out and *c_out. CA_ERR_SHAPE unless batch == 2. */
int lm_head_dpo_finish(const lm_head_desc* desc, int32_t seq_len, const float* row_loss, float ref_logp_chosen,
                       float ref_logp_rejected, float beta, float* dh, float* dw, float* loss_out, float* c_out,
                       void* stream);

/* Kernel timing for benchmarks (instrumentation only; results are unchanged).
 * chunk_attn_profile_start() clears the record and, until
 * chunk_attn_profile_stop(), times every kernel this library launches with a
 * pair of HIP events that the launch itself stamps with the kernel's start and
 * end (hipExtLaunchKernelGGL on the launching stream). chunk_attn_profile_read()
 * waits for the recorded events and returns, for one kernel id, the number of
 * launches and their summed GPU time in milliseconds. Events are created on
 * first use and reused; start/stop/read are serialized by a lock. Returns
 * CA_ERR_SHAPE for an unknown kernel id and CA_ERR_HIP on a runtime error. */
enum {
  CA_KERNEL_FWD = 0,        /* chunk forward */
  CA_KERNEL_DELTA = 1,      /* rowsum(dO * O) */
  CA_KERNEL_DKDV = 2,       /* dK/dV accumulation over the prefix (dS hand-over backward) */
  CA_KERNEL_DQ = 3,         /* dQ of the chunk from the handed-over dS */
  CA_KERNEL_ACCUMULATE = 4, /* prefix_grad_accumulate */
  CA_KERNEL_ZERO = 5,       /* zero fill used by sparse_chunk_bwd */
  CA_KERNEL_PROJ = 6,       /* projection GEMMs of qkv_proj_fwd / qkv_proj_bwd */
  CA_KERNEL_PROJ_PREP = 7,  /* qkv_proj_bwd: the chunk's gradients rounded to bf16, weights transposed */
  CA_KERNEL_RESIDUAL = 8,   /* spaco_stack_*: residual connections between layers */
  CA_KERNEL_HEAD = 9,       /* lm_head_sft_partition: logits, dH and dW products */
  CA_KERNEL_HEAD_AUX = 10,  /* lm_head_*: softmax/cross-entropy rows, weight transpose */
  CA_KERNEL_BWD = 11,       /* dQ and dK/dV of the chunk in one launch (backward without the dS hand-over) */
  CA_KERNEL_COUNT = 12
};
int chunk_attn_profile_start(void);
/* Bit k of kernel_mask (default all) selects kernel id k for the events;
 * every event adds a little GPU time between launches, so a benchmark that
 * needs one kernel's durations brackets only that kernel. */
int chunk_attn_profile_select(uint32_t kernel_mask);
int chunk_attn_profile_stop(void);
int chunk_attn_profile_read(int32_t kernel, int64_t* launches, double* total_ms);

/* Static name of an error code. */
const char* chunk_attn_strerror(int code);

/* Detail of the calling thread's last failed call ("" if none). */
const char* chunk_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CHUNK_ATTN_H */
