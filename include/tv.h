/*
 * tv.h — tree-draft verification on AMD MI355X (gfx950): C ABI.
 *
 * Verifies a speculative draft token tree in one forward pass, the method of
 * the EmbodiInfer pull-request page "perf(activevln): grammar-trie
 * speculation and lossless throughput":
 *   - commit "feat(activevln): grammar-trie tree speculation with exact
 *     acceptance": the N most likely trie nodes are verified in one
 *     tree-attention forward; greedy decoding keeps the argmax path; sampling
 *     runs standard rejection sampling against the draft;
 *   - commit "perf(activevln): lossless batched replay throughput options",
 *     item attention_kernel="gqa": a split-KV kernel that packs the query
 *     heads sharing a KV head into one program; items probability_parts and
 *     skip_padded_queries;
 *   - commit "fix(attention): never read KV slots past a row's live queries".
 * The acceptance-mask output follows the vectorised accepted-token mask of
 * the IluvatarLabs/vllm page "Introduce SCV vectorized masking with
 * graph/adaptive modes".
 *
 * Tree conventions (all entry points):
 *   A sequence b has T tree rows. Row 0 is the root (the last accepted token);
 *   rows 1..n-1 are draft nodes with 0 <= parent[i] < i; n = n_nodes[b] is
 *   0 (a fully padded sequence: no work, padding outputs) or 1..T. Rows
 *   i >= n are padding. parent[b][0] is ignored.
 *
 * Memory: every pointer argument is a DEVICE pointer owned by the caller,
 * unless stated otherwise. The library allocates nothing, keeps no global
 * mutable state, never synchronises the stream and never reads device memory
 * from the host; every call only enqueues kernels on `stream`, so it can be
 * captured in a HIP graph. Grid sizes depend only on host integers.
 *
 * Errors: a call first validates its host-visible arguments and returns a
 * negative tv_status (nothing enqueued) on failure. Problems that only the
 * device can see (a bad parent link, a context over its bound) are written to
 * row_status[b] (tv_row_status) and that sequence's outputs are set to the
 * padding values. TV_ERR_HIP means a kernel launch failed.
 */
#ifndef TV_H_
#define TV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tv_status {
  TV_OK = 0,
  TV_ERR_NULL = -1,        /* a required pointer is NULL */
  TV_ERR_SHAPE = -2,       /* a size or stride is out of range */
  TV_ERR_DTYPE = -3,       /* unknown element type */
  TV_ERR_ALIGN = -4,       /* pointer or stride misaligned */
  TV_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  TV_ERR_UNSUPPORTED = -6, /* a valid but unsupported configuration (head_dim) */
  TV_ERR_HIP = -7          /* the HIP runtime reported an error */
} tv_status;

typedef enum tv_row_status {
  TV_ROW_OK = 0,
  TV_ROW_BAD_PARENT = 1, /* some live node i has parent outside [0, i) */
  TV_ROW_CTX_BOUND = 2,  /* ctx_len < 0, ctx_len > max_ctx or ctx_len + n > kv_capacity */
  TV_ROW_NNODES = 3,     /* n_nodes outside [0, T] */
  TV_ROW_BAD_TOKEN = 4,  /* some live draft token outside [0, V) */
  TV_ROW_BAD_PATH = 5,   /* accepted path not 0 < path[1] < ... < path[a] < n, or a outside [0, n) */
  TV_ROW_BAD_START = 6   /* packed rows: row_start < 0 or row_start + n > rows_total */
} tv_row_status;

typedef enum tv_dtype { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* Largest tree the kernels accept (rows per sequence, root included). */
#define TV_MAX_TREE 128
/* Largest number of query heads sharing one KV head. */
#define TV_MAX_GROUP 16

/*
 * tv_build_tree_mask — ancestor-or-self visibility of every tree row.
 * (Page 1, commit "feat(activevln): grammar-trie tree speculation with exact
 * acceptance": a node is verified against the committed context plus its
 * own ancestors in one tree-attention forward.)
 *
 *   parent   int32 [B][T]   parent links (row-major, contiguous)
 *   n_nodes  int32 [B]      live rows per sequence
 *   mask     uint32 [B][T][W], W = ceil(T / 32): bit j of word j/32 of
 *            mask[b][i] is set iff node j is node i or one of its ancestors
 *   depth    int32 [B][T]   root 0, node i: depth[parent[i]] + 1; -1 on
 *            padding rows and on every row of a sequence whose status is not OK
 *   row_status int32 [B]    TV_ROW_OK, TV_ROW_BAD_PARENT or TV_ROW_NNODES
 *
 * The mask is built once per verification step and reused by every layer's
 * tv_tree_attention call. 1 <= T <= TV_MAX_TREE; B >= 0 (B == 0 enqueues
 * nothing). Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_HIP.
 */
int tv_build_tree_mask(const int32_t* parent, const int32_t* n_nodes, int B, int T,
                       uint32_t* mask, int32_t* depth, int32_t* row_status,
                       hipStream_t stream);

/* Draft-block visibility modes of tv_build_block_mask. */
enum tv_block_mode {
  TV_BLOCK_CAUSAL = 0,        /* row i sees block rows 0..i (a linear draft) */
  TV_BLOCK_BIDIRECTIONAL = 1  /* every live row sees every live row */
};

/*
 * tv_build_block_mask — visibility masks of a draft block instead of a tree,
 * in the layout tv_tree_attention takes (bit j of word j / 32 of
 * mask[b][i]: block key j, in cache slot ctx_len + j). (Page 4, the DFlash
 * draft block: its rows attend over the context plus the block keys;
 * TV_BLOCK_CAUSAL is the linear draft block, whose verification is causal.)
 *
 *   n_nodes  int32 [B]: live rows of each block (0: padded sequence)
 *   mode     TV_BLOCK_CAUSAL or TV_BLOCK_BIDIRECTIONAL (else TV_ERR_UNSUPPORTED)
 *   mask     uint32 [B][T][ceil(T/32)]; padding rows are all zero
 *   position int32 [B][T]: i on live rows (position offset after the
 *            committed context), -1 on padding rows and bad sequences
 *   row_status int32 [B]: TV_ROW_OK or TV_ROW_NNODES (n outside [0, T]:
 *            that sequence gets zero masks)
 * 1 <= T <= TV_MAX_TREE; B >= 0 (B == 0 enqueues nothing).
 */
int tv_build_block_mask(const int32_t* n_nodes, int B, int T, int mode, uint32_t* mask,
                        int32_t* position, int32_t* row_status, hipStream_t stream);

/*
 * Workspace (bytes) tv_tree_attention needs for these sizes and chunk choice
 * on the current device (chunk_keys == 0: units balanced on the device).
 * Returns 0 when no workspace is needed (every (sequence, KV head) pair is a
 * single unit: max_ctx <= chunk_keys, or max_ctx <= 128 when balanced) and
 * (size_t)-1 for invalid sizes. The size depends on the device's compute
 * unit count, so query it on the device the call will run on.
 */
size_t tv_tree_attention_workspace_size(int B, int T, int Hq, int Hkv, int D, int max_ctx,
                                        int chunk_keys);

/*
 * The unit size (keys) that chunk_keys == 0 picks when every sequence is live
 * with max_ctx committed keys (the device picks from the actual lengths).
 */
int tv_tree_attention_auto_chunk(int B, int T, int Hq, int Hkv, int max_ctx);

/*
 * tv_tree_attention — tree-masked, split-KV, grouped-query attention.
 * (Page 1, commit "perf(activevln): lossless batched replay throughput
 * options", items attention_kernel="gqa", probability_parts and
 * skip_padded_queries; commit "fix(attention): never read KV slots past a
 * row's live queries".)
 *
 * For each sequence b with n = n_nodes[b] > 0 and L = ctx_len[b], each live
 * node i < n and query head h (KV head h / (Hq / Hkv)):
 *   visible keys: cache slots [0, L) (the committed context) and slots L + j
 *                 for every j with bit j of mask[b][i] set (j < n);
 *   out[b][i][h] = softmax(scale * q . k) @ v over the visible keys;
 *   lse[b][i][h] = natural log of sum over visible keys of exp(scale * q . k).
 * Padding rows (i >= n), padded sequences (n == 0) and sequences with a bad
 * status get out = 0 and lse = -inf, and so does a live row that sees no key
 * at all (possible only with a caller-built mask and L == 0: the sum over no
 * keys is 0). Cache slots >= L + n are never read, so they may hold anything
 * (NaN included). A padded sequence reads no KV.
 *
 *   q        [B][T][Hq][D] elements of in_dtype; element (b,i,h,d) at
 *            q + b*q_sb + i*q_st + h*q_sh + d (strides in elements)
 *   k, v     [B][Hkv][kv_capacity][D] caches; element (b,g,s,d) at
 *            base + b*kv_sb + g*kv_sh + s*kv_ss + d
 *   ctx_len  int32 [B]; n_nodes int32 [B]; mask from tv_build_tree_mask
 *   max_ctx  host bound on every ctx_len (sizes the workspace); a sequence
 *            with ctx_len > max_ctx gets TV_ROW_CTX_BOUND; kv_capacity slots
 *   scale    softmax scale, finite and > 0 (1/sqrt(D) is the usual choice)
 *   in_dtype TV_F32 (fp32-faithful arithmetic) or TV_BF16 (bf16 matrix cores,
 *            fp32 accumulation)
 *   out_dtype TV_F32 or TV_BF16: element type of out (bf16: the fp32 result
 *            rounded to nearest even once); lse is always fp32
 *   probability_parts  1..3 (bf16 only): the probabilities enter the P.V
 *            product as a sum of that many bf16 terms. 3 is the page's
 *            setting: P is represented exactly (fp32-faithful) and the
 *            split-KV partials stay fp32, so only fp32 rounding remains.
 *            2 also keeps fp32 partials (P to 16 significant bits).
 *            1 is a lossy fast mode: each P is rounded once to bf16
 *            (relative error <= 2^-8) and the per-unit partial outputs are
 *            kept as 16-bit fixed point against each row's largest
 *            magnitude, so an output entry may be off by up to
 *            (2^-8 + 2^-16) * max|v| over the row's visible values: within
 *            2e-3 only while max|v| <= 0.5, and on long contexts, where
 *            rounding errors of many probabilities cancel, typically far
 *            better
 *   chunk_keys  keys per split-KV unit (multiple of 64, 64..65536), or 0 to
 *            let the device balance the units of the whole launch over its
 *            compute units from the actual lengths; results are bitwise
 *            independent of the other sequences of the batch for a fixed
 *            chunk_keys (with 0 they agree to rounding)
 *   out      [B][T][Hq][D] contiguous, out_dtype; lse float32 [B][T][Hq]
 *   workspace/ws_bytes  device scratch of at least
 *            tv_tree_attention_workspace_size(...) bytes, 256-byte aligned
 *            (may be NULL when that size is 0); contents need no initialisation
 *   row_status int32 [B]: TV_ROW_OK, TV_ROW_NNODES or TV_ROW_CTX_BOUND
 *
 * Constraints: D in {64, 128} (else TV_ERR_UNSUPPORTED); 1 <= T <= TV_MAX_TREE;
 * Hq % Hkv == 0 and Hq / Hkv <= TV_MAX_GROUP; q, k, v 16-byte aligned with
 * every stride a multiple of 16 bytes; out, lse 16-byte aligned.
 */
int tv_tree_attention(const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                      const void* k, const void* v, int64_t kv_sb, int64_t kv_sh,
                      int64_t kv_ss, const int32_t* ctx_len, const int32_t* n_nodes,
                      const uint32_t* mask, int B, int T, int Hq, int Hkv, int D,
                      int max_ctx, int kv_capacity, float scale, int in_dtype, int out_dtype,
                      int probability_parts, int chunk_keys, void* out, float* lse,
                      void* workspace, size_t ws_bytes, int32_t* row_status,
                      hipStream_t stream);

/*
 * tv_tree_attention_packed — tv_tree_attention over packed query rows: the
 * live rows of the sequences sit back to back instead of each sequence being
 * padded to T rows. (Page 1, commit "perf(activevln): pack batched prefill
 * turns back to back in CUDA graphs": the split-KV attention takes a table
 * of per-row starts and a query extent equal to the padded length, so its
 * split partition and its results are those of the padded launch, bit for
 * bit.)
 *
 * Node i < n_nodes[b] of sequence b is packed row row_start[b] + i:
 *   q        [rows_total][Hq][D]; element (row,h,d) at q + row*q_st + h*q_sh + d
 *   out      [rows_total][Hq][D] contiguous, out_dtype; lse float32 [rows_total][Hq]
 *   row_start int32 [B]; the ranges [row_start[b], row_start[b] + n_nodes[b])
 *            must not overlap (not checked: overlapping rows race)
 * T is the query extent (the largest n_nodes the call accepts, as in the
 * padded call); mask, ctx_len, n_nodes, k, v, the workspace and every other
 * argument are as in tv_tree_attention, and the workspace size is the same.
 * For the same inputs each live row gets exactly the bits tv_tree_attention
 * writes for it. Rows that belong to no live sequence are not written; a
 * sequence with TV_ROW_CTX_BOUND gets out = 0, lse = -inf on its own rows.
 * row_status adds TV_ROW_BAD_START (row_start[b] < 0 or row_start[b] + n >
 * rows_total; nothing of that sequence is written). Errors as tv_tree_attention,
 * plus TV_ERR_NULL for a NULL row_start and TV_ERR_SHAPE for rows_total < 0.
 */
int tv_tree_attention_packed(const void* q, int64_t q_st, int64_t q_sh, const void* k,
                             const void* v, int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
                             const int32_t* ctx_len, const int32_t* n_nodes,
                             const uint32_t* mask, const int32_t* row_start, int rows_total,
                             int B, int T, int Hq, int Hkv, int D, int max_ctx, int kv_capacity,
                             float scale, int in_dtype, int out_dtype, int probability_parts,
                             int chunk_keys, void* out, float* lse, void* workspace,
                             size_t ws_bytes, int32_t* row_status, hipStream_t stream);

/*
 * Workspace (bytes) of tv_accept_greedy (mode 0) or tv_accept_sample
 * (mode 1); (size_t)-1 for invalid sizes.
 */
size_t tv_accept_workspace_size(int B, int T, int V, int mode);

/*
 * tv_accept_greedy — exact greedy acceptance of a verified tree.
 * (Page 1, commit "feat(activevln): grammar-trie tree speculation with exact
 * acceptance": greedy decoding keeps the argmax path.)
 *
 * For each live sequence: a_j = argmax_v logits[b][j][v] (the lowest index
 * among equal maxima; -0.0 equals +0.0; logits must be finite). From the
 * root, move to the lowest-index child c of the current node with
 * tokens[b][c] == a_cur; when no child matches, a_cur is the bonus token.
 *
 *   logits   float32, row (b, j) at logits + (b*T + j) * logits_row_stride,
 *            V contiguous values; only rows j < n_nodes[b] are read
 *   tokens, parent  int32 [B][T]; tokens[b][0] is ignored
 *   accept_len int32 [B]  accepted draft nodes (0 on padding)
 *   path     int32 [B][T] root then accepted nodes in depth order, -1 after
 *   bonus    int32 [B]    token after the accepted path (-1 on padding)
 *   accept_mask uint8 [B][T] 1 on the nodes of path, else 0
 *   row_status int32 [B]: OK, BAD_PARENT, NNODES or BAD_TOKEN
 *
 * Constraints: 1 <= T <= TV_MAX_TREE; 0 <= B <= 65535; V >= 1;
 * logits_row_stride >= V (any value: rows need not be 16-byte aligned).
 * Workspace as sized above, 256-byte aligned, no initialisation needed.
 */
int tv_accept_greedy(const float* logits, int64_t logits_row_stride, const int32_t* tokens,
                     const int32_t* parent, const int32_t* n_nodes, int B, int T, int V,
                     int32_t* accept_len, int32_t* path, int32_t* bonus, uint8_t* accept_mask,
                     void* workspace, size_t ws_bytes, int32_t* row_status,
                     hipStream_t stream);

/*
 * tv_accept_greedy_noalloc — tv_accept_greedy for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, with the
 * per-slice argmax partials kept in a static scratch array of the library
 * (2 MiB per device, held until the process ends) instead of a workspace.
 * Arguments, outputs and errors as tv_accept_greedy, without workspace and
 * ws_bytes. Sizes whose workspace (tv_accept_workspace_size(B, T, V, 0):
 * B * T * min(64, ceil(V / 16384)) * 8 bytes, rounded up to 256) exceeds
 * 2 MiB return TV_ERR_WORKSPACE before anything is enqueued. Every call on a
 * device shares that device's array: calls that overlap on one device (two
 * streams, two threads) race and must be ordered by the caller. Calls on
 * different devices do not interact. The first call on a device looks the
 * array's address up once (TV_ERR_HIP if that fails); nothing is allocated.
 */
int tv_accept_greedy_noalloc(const float* logits, int64_t logits_row_stride,
                             const int32_t* tokens, const int32_t* parent,
                             const int32_t* n_nodes, int B, int T, int V, int32_t* accept_len,
                             int32_t* path, int32_t* bonus, uint8_t* accept_mask,
                             int32_t* row_status, hipStream_t stream);

/*
 * tv_accept_sample — SpecInfer-style rejection sampling on the tree.
 * (Page 1, commit "feat(activevln): grammar-trie tree speculation with exact
 * acceptance": standard rejection sampling against the draft keeps the
 * output distribution unchanged; summary: "exact SpecInfer-style
 * acceptance".)
 *
 * Target p_j(x) = exp((l_j(x) - max l_j) / tau) / sum, computed in float64
 * with tau the float64 value of `temperature`. Walk from the root with
 * r = p_root; test the children c of the current node in ascending index:
 * x = tokens[b][c], ratio = r(x) / q_c(x) (0 when r(x) = 0, +inf when
 * q_c(x) = 0 < r(x)); accept iff u[b][c] < ratio (then move to c and set
 * r = p_c), else r = max(r - q_c, 0) renormalised. When no child of the
 * current node is accepted, the bonus token is the smallest x with
 * sum_{y<=x} r(y) > u[b][0] * sum_y r(y).
 *
 *   logits   as in tv_accept_greedy (float32 target logits)
 *   q        float32 draft distributions, row (b, c) at
 *            q + (b*T + c) * q_row_stride; row 0 is never read
 *   u        float32 [B][T] uniforms in [0, 1): u[b][c] tests node c,
 *            u[b][0] is the single final draw
 *   decision int8 [B][T]  +1 accepted, 0 rejected, -1 never tested
 *   other outputs as in tv_accept_greedy
 *
 * Constraints as tv_accept_greedy, plus q_row_stride >= V and
 * temperature > 0.
 */
int tv_accept_sample(const float* logits, int64_t logits_row_stride, float temperature,
                     const float* q, int64_t q_row_stride, const float* u,
                     const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                     int B, int T, int V, int32_t* accept_len, int32_t* path, int32_t* bonus,
                     uint8_t* accept_mask, int8_t* decision, void* workspace, size_t ws_bytes,
                     int32_t* row_status, hipStream_t stream);

/*
 * tv_linear_rows — y = x W^T on the few verification rows, batch-invariant.
 * (Page 1, commit "perf(activevln): batch-invariant Triton GEMMs for decode
 * projections": FP32 accumulation in sequential K order without split-K, so
 * a row's result depends neither on the tiles nor on the row count; Q, K and
 * V share one launch when W holds the three projections stacked.)
 *
 *   x  bf16 [M][K], row stride x_stride elements (a multiple of 8, >= K)
 *   w  bf16 [N][K] (output features x input features, the layout of a
 *      PyTorch Linear weight), row stride w_stride (a multiple of 8, >= K)
 *   y  bf16 [M][N], row stride y_stride (a multiple of 4, >= N): each entry
 *      is one fp32 accumulation over k, rounded to nearest even. K is walked
 *      in increasing order, 32 products per matrix-core step
 *      (v_mfma_f32_16x16x32_bf16, which sums its 32 products in the
 *      hardware's own order before adding them to the running sum), so the
 *      rounding order depends only on K, never on M, the row's place in the
 *      batch or the tiling: a row's bits are batch-invariant
 * Constraints: K and N multiples of 64 (else TV_ERR_SHAPE),
 * 0 <= M <= 65536; pointers 16-byte aligned (else TV_ERR_ALIGN). Sized for a
 * few hundred rows; nothing is allocated.
 */
int tv_linear_rows(const void* x, int64_t x_stride, const void* w, int64_t w_stride, int M,
                   int K, int N, void* y, int64_t y_stride, hipStream_t stream);

/*
 * tv_linear_swiglu_rows — the gate and up projections in one launch with
 * the rounded SwiGLU in the epilogue (same page and commit): g and u are
 * each rounded to bf16 as tv_linear_rows would return them, then
 * y = bf16(silu(g) * u) with silu(g) = g / (1 + exp(-g)) in fp32.
 * Arguments as tv_linear_rows; w_gate and w_up share w_stride.
 */
int tv_linear_swiglu_rows(const void* x, int64_t x_stride, const void* w_gate, const void* w_up,
                          int64_t w_stride, int M, int K, int N, void* y, int64_t y_stride,
                          hipStream_t stream);

/*
 * tv_commit_accepted_kv — accepted-path KV commit.
 * (Page 1, commit "perf(activevln): lossless batched replay throughput
 * options", item incremental_kv_commit: only the new turn is copied into the
 * owned KV; page 3, the commit kernel for accepted drafts over NHD and HND
 * cache layouts.)
 *
 * For each sequence b with n = n_nodes[b] > 0, L = ctx_len[b] and
 * a = accept_len[b], in each of `layers` caches: slot L + k of K and of V
 * takes what slot L + path[b][k] held before the call, for k = 1..a (slot L,
 * the root, stays), and new_ctx_len[b] = L + a + 1. Every other slot is left
 * as it is. A padded sequence (n = 0) or one with a bad status moves nothing
 * and gets new_ctx_len = L. accept_len and path are the outputs of
 * tv_accept_greedy / tv_accept_sample for the same tree.
 *
 *   k, v     caches of `layers` layers; element (layer, b, g, s, d) at
 *            base + layer*layer_stride + b*kv_sb + g*kv_sh + s*kv_ss + d
 *            (strides in elements of elem_bytes: HND and NHD both work)
 *   elem_bytes 2 (bf16 / fp16) or 4 (fp32); elements are moved bit for bit
 *   ctx_len, n_nodes, accept_len int32 [B]; path int32 [B][T]
 *   new_ctx_len int32 [B] (output; must not be ctx_len itself)
 *   row_status int32 [B]: TV_ROW_OK, TV_ROW_NNODES, TV_ROW_CTX_BOUND
 *            (ctx_len < 0 or ctx_len + n > kv_capacity) or TV_ROW_BAD_PATH
 *
 * Constraints: D * elem_bytes a multiple of 16 and at most 512 (else
 * TV_ERR_UNSUPPORTED); k, v 16-byte aligned and every stride a multiple of
 * 16 bytes (else TV_ERR_ALIGN); 1 <= T <= TV_MAX_TREE; layers >= 1. The copy
 * runs in place and in the stream order of the caller.
 */
int tv_commit_accepted_kv(void* k, void* v, int64_t layer_stride, int64_t kv_sb, int64_t kv_sh,
                          int64_t kv_ss, const int32_t* ctx_len, const int32_t* n_nodes,
                          const int32_t* accept_len, const int32_t* path, int B, int T, int Hkv,
                          int D, int elem_bytes, int layers, int kv_capacity,
                          int32_t* new_ctx_len, int32_t* row_status, hipStream_t stream);

/*
 * tv_adapt_tree_budget — adaptive draft budget and the next step's packed
 * row table, on the device. (Page 3, the adaptive mode: the number of
 * speculative tokens follows recent acceptance ratios toward a target ratio;
 * page 1, commit "perf(activevln): pack batched prefill turns back to back
 * in CUDA graphs": per-row starts of packed rows.)
 *
 * For each sequence b whose verified step had n = n_nodes[b] >= 2 rows,
 * a = accept_len[b] in [0, n - 1] and (if row_status is not NULL)
 * row_status[b] == TV_ROW_OK, in fp32 with every operation rounded to nearest
 * and none fused:
 *   ratio = a / (n - 1);  ratio_ema[b] = ratio_ema[b] + alpha * (ratio - ratio_ema[b]);
 *   budget[b] += 1 if ratio_ema[b] > target, -= 1 if below, unchanged if equal;
 * other sequences keep their ratio_ema. Every budget[b] is then clamped to
 * [n_min, n_max], and row_start[b] = sum over c < b of (budget[c] + 1) (the
 * draft nodes plus the root of the next step), rows_total[0] = that sum over
 * all b. ratio_ema and budget are read and updated in place (the caller
 * initialises them, e.g. to target and n_max).
 *
 *   accept_len, n_nodes int32 [B] (from the verification of the last step)
 *   row_status int32 [B] or NULL
 *   target   in [0, 1]; alpha in (0, 1]; 1 <= n_min <= n_max <= TV_MAX_TREE - 1
 *   ratio_ema float32 [B]; budget, row_start int32 [B]; rows_total int32 [1]
 * B >= 0 (B == 0 writes rows_total = 0; the [B] pointers may then be NULL).
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE.
 * One workgroup; every write goes through device memory, nothing is read back.
 */
int tv_adapt_tree_budget(const int32_t* accept_len, const int32_t* n_nodes,
                         const int32_t* row_status, int B, float target, float alpha, int n_min,
                         int n_max, float* ratio_ema, int32_t* budget, int32_t* row_start,
                         int32_t* rows_total, hipStream_t stream);

/*
 * tv_read_probe — a measurement helper, not a step of the verification:
 * reads `bytes` of device memory at `buf` once (coalesced 16-byte
 * non-temporal loads over up to 1024 workgroups) and XORs all of it into
 * *sink (device memory, which the caller zeroes first if it wants the
 * value). Its time gives the chip's streaming-read rate, the ceiling that
 * the library's HBM-bound kernels are compared with.
 *   buf  16-byte aligned (else TV_ERR_ALIGN); bytes > 0 and a multiple of
 *        16 (else TV_ERR_SHAPE); buf or sink NULL: TV_ERR_NULL.
 */
int tv_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Static, human-readable name of a tv_status or tv_row_status value. */
const char* tv_status_string(int code);

/* Library version: major * 10000 + minor * 100 + patch. */
int tv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TV_H_ */
