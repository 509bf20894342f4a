/*
 * medusa.h -- C ABI of the Medusa verify-step library for AMD Instinct MI355X
 * (gfx950, wave64, CDNA4).
 *
 * One Medusa verify step has four stages, each one call here:
 *   medusa_heads            K residual-SiLU heads + vocab projections
 *   medusa_tree_candidates  per-head top-k, candidate tree tokens, positions
 *   medusa_tree_attention   tree-masked attention of one layer (split-KV);
 *                           _layers: every layer in one grid
 *   medusa_accept_paths     longest accepted root-to-leaf path (greedy or
 *                           rejection sampling)
 * and one call closes the step:
 *   medusa_commit_accepted  KV rollback / compaction of the accepted path,
 *                           next root and context length
 * and a host-only call chooses the static tree:
 *   medusa_tree_optimize    the T-node tree that maximises expected accepted
 *                           length under a per-depth, per-rank acceptance table
 *
 * Pages that define the operations (cited per call):
 *   P1 "Medusa 심층 아키텍처: 별도 초안 모델을 제거한 다중 헤드(Multi-Head) 추측 디코딩과
 *      Tree Attention 3배 가속 원리" (techknowgenie.com)
 *   P2 "[vLLM] Medusa: 다중 예측 헤드 투기적 디코딩" (blog.secrett2633.cloud)
 *   P3 "Speculative Decoding(투기적 디코딩) 원리와 가속 아키텍처 ..." (blog.huny.dev)
 *   P4 "최적화 2편. 추측 디코딩과 긴 컨텍스트 - Speculative Decoding과 MEDUSA·EAGLE,
 *      Ring Attention" (beengineer500.github.io)
 *
 * Conventions common to every call
 *   - Tensor arguments are DEVICE pointers owned by the caller, on the
 *     device that is current when the call is made, unless a parameter says
 *     "host".  The library never keeps them after the call returns.
 *   - Layouts are dense row-major in the order written ("[B][T][V]": V is
 *     contiguous).  bf16 tensors are 16-bit bfloat16 bit patterns.
 *   - Calls are asynchronous on the given stream (NULL = the null stream);
 *     nothing synchronises the host.  Work is enqueued only after every
 *     argument check passed.
 *   - Return value: MEDUSA_OK or a negative MEDUSA_E* code; the reason is
 *     in medusa_last_error() (thread-local, valid until the next call on the
 *     same thread).  No exception crosses the ABI.
 *   - Scratch memory is passed in by the caller (ws, ws_bytes, sized by the
 *     matching *_workspace_size call, 256-byte aligned).  No call allocates
 *     device memory except medusa_tree_create, and no workspace needs
 *     initialising.
 *   - Floating-point inputs must be finite.  Non-finite inputs give
 *     unspecified outputs, but every kernel still terminates and every index
 *     written stays in its documented range (or -1).
 *   - Calls that share a workspace or output on one stream are ordered by
 *     the stream; concurrent calls on different streams must not share them.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MEDUSA_OK            0
#define MEDUSA_EINVAL       (-1) /* invalid argument: shape, range, NULL pointer */
#define MEDUSA_EUNSUPPORTED (-2) /* valid but not implemented (e.g. a head dim) */
#define MEDUSA_EWORKSPACE   (-3) /* workspace missing, misaligned or too small */
#define MEDUSA_EHIP         (-4) /* a HIP runtime call or kernel launch failed */

/* Limits of this implementation. */
#define MEDUSA_MAX_TREE_NODES 256 /* T, root included */
#define MEDUSA_MAX_HEADS       16 /* K */
#define MEDUSA_MAX_TOPK        32 /* candidates kept per head */

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype_t;

/* Opaque static tree (topology + ancestor bitmask), resident on one device. */
typedef struct medusa_tree medusa_tree_t;

/* Thread-local text of the last error on this thread ("" after success). */
const char* medusa_last_error(void);

/* Library version string, e.g. "medusa-amd 0.1 gfx950". */
const char* medusa_version(void);

/* ------------------------------------------------------------------------
 * Static candidate tree
 *
 * P1, section "트리 어텐션 ... 고정 트리 토폴로지와 2차원 어텐션 마스크": head d
 * contributes its top candidates at depth d and a fixed topology combines
 * them into paths; token i may attend to tree token j iff j is an ancestor
 * of i or j = i.  P1's sketch code ("build_tree_attention_mask") builds the
 * mask by inheriting each parent's row, which needs parents before children.
 *
 * Topology (HOST arrays, length T):
 *   parent[0] = -1 (node 0 is the root, the token already chosen by the base
 *   model); for n >= 1, 0 <= parent[n] < n.
 *   rank[n]   = which candidate of head depth(n) node n carries,
 *               0 <= rank[n] < k_per_depth[depth(n)-1]; siblings need
 *               distinct ranks.  rank[0] is ignored.
 *   k_per_depth[K] = candidates kept by head d = 1..K (1..MEDUSA_MAX_TOPK).
 *   depth(n) <= K, T <= MEDUSA_MAX_TREE_NODES, K <= MEDUSA_MAX_HEADS.
 * Ancestor bitmask: W = ceil(T/64) uint64 words per node; bit (j % 64) of
 * word j / 64 of row i is set iff j is an ancestor of i or j == i.
 * ------------------------------------------------------------------------ */

/* Host-only validation and mask construction (no GPU needed).
 * mask_out: HOST [T][W] uint64 or NULL; depth_out: HOST [T] int32 or NULL.
 * Returns MEDUSA_EINVAL (with the offending node in the message) for an
 * invalid topology. */
int medusa_tree_build_host(const int32_t* parent, const int32_t* rank, int T,
                           const int32_t* k_per_depth, int K,
                           uint64_t* mask_out, int32_t* depth_out);

/* Validates the topology (as above), builds depth, rank-ordered child
 * lists and the ancestor bitmask, and uploads them to the CURRENT device
 * (one device allocation, synchronous).  *out receives a handle owned by the
 * library; free it with medusa_tree_destroy.  The handle may only be used
 * with the device that was current at creation (EINVAL otherwise). */
int medusa_tree_create(const int32_t* parent, const int32_t* rank, int T,
                       const int32_t* k_per_depth, int K, medusa_tree_t** out);

/* Frees the handle and its device memory.  NULL is a no-op.  The caller
 * must make sure no enqueued call still uses the tree. */
void medusa_tree_destroy(medusa_tree_t* tree);

/* Copies the ancestor bitmask to HOST memory host_out [T][W]. */
int medusa_tree_mask(const medusa_tree_t* tree, uint64_t* host_out);

/* Shape query; any output pointer may be NULL.  kmax = max(k_per_depth). */
int medusa_tree_info(const medusa_tree_t* tree, int32_t* T, int32_t* K, int32_t* W,
                     int32_t* max_depth, int32_t* kmax);

/* ------------------------------------------------------------------------
 * Stage 1+2: Medusa heads
 *
 * P1, section "Medusa의 핵심 철학 ... 잔차 블록을 포함한 Medusa 헤드 구조": head k
 * maps the last hidden state h to r = SiLU(h W_res^(k)) + h and to logits
 * r W_head^(k) (softmax is applied later, where probabilities are needed).
 * P1's sketch code: both projections are bias-free [out, in] linear layers.
 * W_head may be shared by all heads (P1 allows reusing the frozen base
 * unembedding) -- pass wlm_head_stride = 0.
 *
 *   hidden  [M][H]                    dt
 *   w1      head k at w1 + k*w1_head_stride elements, each [H][H] ([out][in]), dt
 *   wlm     head k at wlm + k*wlm_head_stride elements, each [V][H], dt
 *   logits  [M][K][V] fp32 (output)
 * For dt = MEDUSA_BF16 the residual output r is rounded to bf16 (round to
 * nearest even) before the vocab projection; accumulation is fp32.
 * Constraints: M >= 1, K in 1..MEDUSA_MAX_HEADS, H % 8 == 0 (bf16),
 * V >= 1, w1_head_stride >= H*H (or 0 only if K == 1), wlm_head_stride == 0
 * or >= V*H.  Pointers 16-byte aligned.
 * Workspace: holds r, K*M*H elements of dt.
 * ------------------------------------------------------------------------ */
size_t medusa_heads_workspace_size(int M, int H, int K, medusa_dtype_t dt);

int medusa_heads(const void* hidden, const void* w1, int64_t w1_head_stride,
                 const void* wlm, int64_t wlm_head_stride, int M, int H, int V, int K,
                 medusa_dtype_t dt, float* logits, void* ws, size_t ws_bytes,
                 hipStream_t stream);

/* Dense variant: the heads on the hidden state of every tree token (M = B*T
 * rows), each head's top-k kept instead of its logits.
 *
 * P1, section "Medusa의 핵심 철학 ... 잔차 블록": the same residual block and
 * vocab projection as medusa_heads; P1, section "소스코드 레벨 구조 분석"
 * (generate_candidates): head d keeps its k_d largest logits.  Running the
 * heads on all tree rows gives the next step's candidates at whichever node
 * is accepted.
 *
 *   hidden    [M][H]        dt
 *   w1, wlm   as medusa_heads (wlm_head_stride 0 = one shared projection)
 *   tree      supplies K (= tree K) and k_d (its per-depth top-k, kmax the
 *             largest)
 *   topk_idx  [M][K][kmax] int32: row m, head d: the k_d vocab indices with
 *             the largest logits, largest first, equal logits by lower
 *             index; entries k_d..kmax-1 are -1
 *   topk_val  [M][K][kmax] fp32 or NULL: the matching logits (0 in padding)
 *   logits    [M][K][V] fp32 or NULL: also write every logit (the top-k is
 *             the same either way)
 * bf16: tiled MFMA GEMMs; the vocab projection's epilogue reduces each
 * 128-column tile to its top-kmax, and a second kernel merges the tiles, so
 * the logits never reach HBM unless asked for.  The ranking is decided on
 * the fp32 logits the kernel computes (fp32 accumulation of bf16 products,
 * the residual output rounded to bf16).  f32: plain VALU products.
 * Constraints: K == tree K; V >= kmax; bf16: H % 128 == 0, V % 4 == 0,
 * strides multiples of 8; pointers 16-byte aligned.
 * Workspace: the residual output of every head and the per-tile candidates
 * (bf16), or r and the logits (f32); no initialisation needed.
 */
size_t medusa_heads_dense_workspace_size(int M, int H, int V, int K, const medusa_tree_t* tree,
                                         medusa_dtype_t dt);

int medusa_heads_dense(const void* hidden, const void* w1, int64_t w1_head_stride,
                       const void* wlm, int64_t wlm_head_stride, int M, int H, int V, int K,
                       const medusa_tree_t* tree, medusa_dtype_t dt, int32_t* topk_idx,
                       float* topk_val, float* logits, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * Stage 3+4: per-head top-k and candidate tree tokens
 *
 * P1, section "소스코드 레벨 구조 분석" (generate_candidates): each head keeps
 * the indices of its k largest logits; P2, section "propose()": the k = 1
 * case is the per-head argmax.  Order: descending logit, equal logits by
 * ascending index.  Tree tokens: node 0 carries root[b]; node n carries
 * candidate rank(n) of head depth(n).  Positions: ctx_len[b] + depth(n).
 *
 *   head_logits [B][K][V] fp32 (K = the tree's K)
 *   root        [B] int32 (token t+1 from the base model)
 *   ctx_len     [B] int32 (tokens already in the KV cache)
 *   topk_idx    [B][K][kmax] int32 (output; -1 beyond head d's k_d)
 *   tree_tokens [B][T] int32 (output)
 *   pos         [B][T] int32 (output)
 * Workspace: each 512-column chunk's sorted top-kmax (logit, index) list
 * per row, merged by a second kernel on the same stream; no initialisation
 * needed, calls that share a workspace must not overlap.
 * ------------------------------------------------------------------------ */
size_t medusa_tree_candidates_workspace_size(int B, int V, const medusa_tree_t* tree);

int medusa_tree_candidates(const float* head_logits, const int32_t* root,
                           const int32_t* ctx_len, const medusa_tree_t* tree, int B, int V,
                           int32_t* topk_idx, int32_t* tree_tokens, int32_t* pos, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Stage 5: tree-masked attention (one layer)
 *
 * P1, section "트리 어텐션 ... 2차원 어텐션 마스크": all tree tokens are verified
 * in one attention pass where tree token i sees the cached context and,
 * among tree tokens, only its ancestors and itself.  P4, section 3.3: partial
 * results over key blocks merge exactly through a running max and exp-sum,
 * which is how the key range is split across workgroups here.
 *
 *   q       [B][T][Hq][D]        dt (already position-encoded)
 *   k_cache [B][Hkv][S_cap][D]   dt; slots 0..ctx_len[b]-1 hold the context,
 *   v_cache [B][Hkv][S_cap][D]   dt; slots ctx_len[b]+j hold tree token j
 *   ctx_len [B] int32, 0 <= ctx_len[b] <= S_cap - T (values outside are
 *           clamped into that range so that no access leaves the cache)
 *   ctx_max HOST upper bound of ctx_len[] (sizes the split grid; a larger
 *           ctx_len still gives the right result, only slower)
 *   out     [B][T][Hq][D]        dt
 * Query head h uses K/V head h / (Hq/Hkv).  softmax(scale * q.k) with fp32
 * scores, sums and accumulators; bf16 operands use MFMA.
 * Constraints: Hq % Hkv == 0; D = 128 (bf16) or D <= 128, D % 4 == 0 (f32);
 * T = the tree's T; S_cap >= ctx_max + T.  Pointers 16-byte aligned.
 * MEDUSA_EUNSUPPORTED when a grid would pass 2^32 work-items (bf16: about
 * 5.5 million (layer, sequence, K/V head) work items).
 * Split count: chosen per call from the shape and the device (the most
 * splits whose workgroups run in one round of the resident slots).  The
 * environment variable MEDUSA_ATTN_SPLITS = n > 0 (read by every call, the
 * workspace-size calls included, so set it before sizing) asks for n splits
 * instead (at most 64, at least one 64-key block each); results agree with
 * the default within rounding.  Meant for tests and tuning.
 * Workspace: the split partials (every query row's output over one key
 * split, normalised by its own exp-sum, in bf16, plus that split's max and
 * exp-sum in fp32), merged by a second kernel on the same stream; 0 bytes
 * when one split suffices.  Its contents need no
 * initialisation, but calls that share a workspace must not overlap.
 * ------------------------------------------------------------------------ */
size_t medusa_tree_attention_workspace_size(int B, int Hq, int Hkv, int D, int ctx_max,
                                            const medusa_tree_t* tree, medusa_dtype_t dt);

int medusa_tree_attention(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* ctx_len, int ctx_max, const medusa_tree_t* tree,
                          int B, int Hq, int Hkv, int D, int S_cap, float scale,
                          medusa_dtype_t dt, void* out, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Every layer of the target in one call (same tree, same ctx_len): layer l
 * reads q + l * q_layer_stride, k_cache/v_cache + l * kv_layer_stride and
 * writes out + l * out_layer_stride (strides in ELEMENTS, each at least one
 * layer's extent and a multiple of 16 bytes; layouts within a layer as
 * above).  Same operation as L calls of medusa_tree_attention (the layers
 * are independent, P1, section "트리 어텐션"), with one grid for all of them
 * so that short contexts still fill the chip; the split count is planned for
 * L * B sequences, so the workspace is sized by the _layers size call.
 * Errors as medusa_tree_attention, plus MEDUSA_EINVAL for L < 1 or strides
 * that overlap layers. */
size_t medusa_tree_attention_layers_workspace_size(int L, int B, int Hq, int Hkv, int D,
                                                   int ctx_max, const medusa_tree_t* tree,
                                                   medusa_dtype_t dt);

int medusa_tree_attention_layers(const void* q, const void* k_cache, const void* v_cache,
                                 int64_t q_layer_stride, int64_t kv_layer_stride,
                                 int64_t out_layer_stride, int L, const int32_t* ctx_len,
                                 int ctx_max, const medusa_tree_t* tree, int B, int Hq, int Hkv,
                                 int D, int S_cap, float scale, medusa_dtype_t dt, void* out,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * medusa_tree_attention without allocation or workspace
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, layouts and results as medusa_tree_attention (the same kernels
 * and launch plan), minus the workspace: the split partials live in a fixed
 * device array of the library, MEDUSA_ATTENTION_SCRATCH_BYTES (32 MiB) per
 * GPU, held until the process ends.  A call whose partials would exceed it
 * (medusa_tree_attention_workspace_size above the limit) returns
 * MEDUSA_EWORKSPACE before anything is enqueued.  The call never calls
 * hipMalloc or hipFree; its first call on a device looks up that device's
 * copy of the array (hipGetSymbolAddress).  Every call on one GPU shares that
 * GPU's array and it keeps the last call's contents (nothing in it needs
 * clearing): calls that overlap on one GPU, e.g. on two streams, race and must
 * be serialised by the caller.
 * ------------------------------------------------------------------------ */
#define MEDUSA_ATTENTION_SCRATCH_BYTES (32u << 20)

int medusa_tree_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* ctx_len, int ctx_max, const medusa_tree_t* tree,
                                  int B, int Hq, int Hkv, int D, int S_cap, float scale,
                                  medusa_dtype_t dt, void* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Stage 6: path acceptance
 *
 * temperature == 0: greedy.  P3, section 5 (greedy check) and P4, section
 * 1.3: walk from the root; at node u take the target's argmax t* of
 * base_logits[b][u] (first maximum); if a child of u carries t* (lowest rank
 * if several), move there, else stop.  The step emits the accepted nodes'
 * tokens and then t* (the correction, or the bonus token at a leaf).
 *
 * temperature > 0: rejection sampling.  P1, section "수학적 무손실 보장: 기각
 * 샘플링": a draft x is accepted iff u < min(1, p(x)/q(x)); after a rejection
 * p becomes max(0, p - q) / sum(max(0, p - q)); P3, section 2, shows the
 * output is distributed as p when each draft is a sample from q.  Drafts
 * taken by top-k (as medusa_tree_candidates fills the tree) are not samples
 * from q, so on such trees that distribution guarantee does not hold; the
 * call computes the same rule either way.  On the tree: p_u = softmax(base_logits[b][u]
 * / temperature), q_d = softmax(head_logits[b][d-1] / temperature) for a child
 * at depth d; children are tried in rank order with u_accept[b][child]; a
 * rejection turns p into the residual before the next sibling; an accepted
 * child becomes the current node; at a leaf or after rejecting every child,
 * one token is drawn from the current p by inverse CDF with u_sample[b][u]
 * (smallest v with cumsum(p)[v] > u * sum(p)).  Probabilities are fp64.
 *
 *   base_logits [B][T][V] fp32   target logits after each tree node
 *   head_logits [B][K][V] fp32   (rejection only; NULL allowed for greedy)
 *   tree_tokens [B][T] int32 (rejection sampling clamps a token outside 0..V-1
 *               into that range, so no access leaves the logits)
 *   u_accept, u_sample [B][T] fp32 in [0, 1) (rejection only; may be NULL for greedy)
 *   accept_len  [B] int32 (output) number of accepted tree nodes, 0..max depth
 *   out_tokens  [B][K+1] int32 (output) accept_len + 1 emitted tokens, -1 after
 *   out_nodes   [B][K+1] int32 (output) root (0) then the accepted nodes, -1 after
 * Workspace: greedy keeps each node's argmax (a first kernel computes them
 * in parallel, a second walks the tree); rejection sampling keeps one fp64
 * distribution per sequence and, for V <= 32768, also the root's p and each
 * depth's q (fp64, max_depth + 1 rows per sequence) computed in parallel
 * before the walk, which then holds p in registers.  No initialisation is
 * needed; calls that share a workspace must not overlap.
 * ------------------------------------------------------------------------ */
size_t medusa_accept_workspace_size(int B, int V, const medusa_tree_t* tree,
                                    float temperature);

int medusa_accept_paths(const float* base_logits, const float* head_logits,
                        const int32_t* tree_tokens, const medusa_tree_t* tree,
                        const float* u_accept, const float* u_sample, float temperature,
                        int B, int V, int32_t* accept_len, int32_t* out_tokens,
                        int32_t* out_nodes, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * After acceptance: commit the accepted path (KV rollback / compaction)
 *
 * P3, architecture section (the pipeline ends with rollback and the
 * confirmed correction token) and section 5, Case 2 (K-token verification
 * with early rejection and rollback); P4, section 1.3: the matched drafts
 * are kept, everything after the first mismatch is discarded.  The tree
 * tokens' K/V sit in slots ctx .. ctx+T-1 (node n at ctx + n).  For every
 * layer, sequence and K/V head the K/V of the accepted node at depth d moves
 * from slot ctx + out_nodes[b][d] to slot ctx + d, d = 1 .. accept_len[b]
 * (the root stays at ctx); the other tree slots are simply abandoned.  The
 * next step starts from
 *   ctx_next[b]  = ctx_len[b] + accept_len[b] + 1
 *   root_next[b] = out_tokens[b][accept_len[b]]   (correction or bonus token)
 * whose K/V the next step computes at slot ctx_next[b].
 *
 *   k_cache, v_cache  layer l at base + l * layer_stride elements, each
 *                     [B][Hkv][S_cap][D] dt (updated in place)
 *   accept_len, out_nodes, out_tokens   as written by medusa_accept_paths
 *   ctx_len [B] int32 (input); ctx_next, root_next [B] int32 (outputs, must
 *           not alias ctx_len)
 * Values outside their ranges are clamped (accept_len to 0..K, nodes to
 * 0..T-1, ctx_len to 0..S_cap-T) so that no access leaves the caches; the
 * caller keeps ctx_next + T <= S_cap for the next step.
 * Constraints: D * element size a multiple of 16 bytes and at most 512;
 * 16-byte aligned caches and layer stride.  No workspace.
 * ------------------------------------------------------------------------ */
int medusa_commit_accepted(void* k_cache, void* v_cache, int64_t layer_stride, int L,
                           const int32_t* accept_len, const int32_t* out_nodes,
                           const int32_t* out_tokens, const int32_t* ctx_len, int32_t* ctx_next,
                           int32_t* root_next, const medusa_tree_t* tree, int B, int Hkv, int D,
                           int S_cap, medusa_dtype_t dt, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Static tree optimiser (host only)
 *
 * P2, paper-results section: an optimised tree configuration adds to the
 * speed-up of tree attention; P1, tree-size trade-off section: the topology
 * (usually 32-64 nodes) is chosen by profiling.  Given an acceptance table
 * p[d][r] (probability that head d+1's rank-r candidate is the target's
 * token, e.g. measured), a node (r_1..r_d) is accepted with probability
 * prod_i p[i-1][r_i]; the returned tree holds the T - 1 most probable such
 * tuples (ties: smaller depth, then the lexicographically smaller tuple),
 * which maximises the expected accepted nodes per step, numbered
 * breadth-first by (depth, tuple) so that it can be passed to
 * medusa_tree_create directly.
 *
 *   p_accept     [K][kmax_in] row-major, values in [0, 1] (host)
 *   k_per_depth  [K] candidates per head, 1..min(MEDUSA_MAX_TOPK, kmax_in)
 *   parent_out, rank_out [T] int32 (host outputs)
 *   expected_out expected accepted nodes per step (may be NULL)
 * ------------------------------------------------------------------------ */
int medusa_tree_optimize(const double* p_accept, int K, int kmax_in, const int32_t* k_per_depth,
                         int T, int32_t* parent_out, int32_t* rank_out, double* expected_out);

/* ------------------------------------------------------------------------
 * Diagnostics: read-bandwidth probe
 *
 * Not a stage of the method.  A plain streaming read of `bytes` bytes of
 * device memory (every 16-byte piece once, coalesced, grid-stride), the rate
 * a streaming kernel reaches on this chip, reported by the benchmark beside
 * the rooflines' peak.  The pieces are folded by XOR so that none can be
 * skipped: partials[i] (i < medusa_read_probe_partials()) receives workgroup
 * i's fold, and the XOR of all partials equals the XOR of every 32-bit word
 * of the buffer.
 *   buf       device, 16-byte aligned; bytes a multiple of 16 (0 allowed)
 *   partials  device, medusa_read_probe_partials() uint32 words (output)
 * ------------------------------------------------------------------------ */
int medusa_read_probe_partials(void);

int medusa_read_probe(const void* buf, size_t bytes, uint32_t* partials, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_H */
