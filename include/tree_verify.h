/*
 * tree_verify.h -- C ABI of the MI355X (gfx950) token-tree verification library.
 *
 * One speculative decoding step of SpecInfer verifies a whole token tree in a
 * single forward pass: every tree node u attends to the shared prefix KV cache
 * plus exactly the nodes on its own root-to-u path S_u, and greedy
 * verification then walks the tree from the root.  This library is that hot
 * path: three calls, all asynchronous on a caller-provided HIP stream; a
 * stochastic variant of verification; the construction of the tree (top-k
 * expansion, merge of drafts); and a call that commits the accepted path's
 * keys and values to the cache.
 *
 * Sources (the SpecInfer explainer at 0h-n0.github.io, "paper-2305-09781"):
 *   - token-tree structure section: a node per token, S_u = tokens on the path
 *     from the root to u, and the attention equation softmax(Q_u K_{S_u}^T /
 *     sqrt(d_k)) V_{S_u};
 *   - same section and the contributions list: a topology-aware causal mask
 *     lets each node attend only to its ancestors, consistently with ordinary
 *     KV-cache reuse;
 *   - kernel-fusion section: the mask is precomputed from ancestor relations;
 *   - tree-verification section: greedy verification; the accept rule of the
 *     sequence case (accept up to the first mismatch, then the target model
 *     supplies one token) is on the speculative-decoding explainer
 *     (lab.arcteris.jp), technical-mechanism section, and in the diagram of the
 *     speculative-decoding operations guide (flatkey.ai);
 *   - "practical applications" section: integration with PagedAttention's
 *     block-wise KV memory (the paged cache layout below).
 *
 * Conventions for every call
 *   - Pointers named in a [..] shape are DEVICE pointers owned by the caller;
 *     the library never frees or keeps them.  Base addresses must be 16-byte
 *     aligned.  The last dimension of every array is contiguous.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls return after
 *     host-side validation and kernel enqueue; results are ready when the
 *     stream reaches them.
 *   - Return value: an int holding a tv_status value: TV_OK, or the code of an
 *     error found on the host (nothing is enqueued then).  tv_last_error() gives a thread-local
 *     message for the last failing call.
 *   - Tree nodes are in a topological order: node 0 is the single root,
 *     parent[u] < u for u >= 1 (BFS and DFS orders both qualify).
 *   - Ancestor masks: W = ceil(n/64) uint64 words per node; bit (v & 63) of
 *     word (v >> 6) is set iff node v is on the path root..u (u included).
 *   - The library allocates no device memory.  tree_attention takes a caller
 *     workspace whose size tree_attention_workspace_size() reports;
 *     tree_attention_noalloc instead uses a fixed scratch array that the
 *     library's code object holds in each GPU's memory from load time.
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_NMAX 256     /* max tree nodes per sequence, root included          */
#define TV_WMAX 4       /* max mask words per node = TV_NMAX / 64               */
#define TV_PAGE 16      /* tokens per paged KV block                            */
#define TV_VERSION 2

typedef enum {
  TV_OK = 0,
  TV_EINVAL = 1,        /* bad argument: null pointer, size out of range         */
  TV_ETOPOLOGY = 2,     /* tree is not a rooted, topologically ordered tree      */
  TV_EUNSUPPORTED = 3,  /* valid but not supported (head dim, dtype, GQA ratio)  */
  TV_EWORKSPACE = 4,    /* workspace missing or smaller than required            */
  TV_EHIP = 5           /* a HIP runtime call failed; see tv_last_error()        */
} tv_status;

typedef enum { TV_F32 = 0, TV_BF16 = 1, TV_F16 = 2, TV_FP8_E4M3 = 3 } tv_dtype;

/* Static text for a status code; never NULL. */
const char* tv_status_string(int status);
/* Thread-local message of the last failing call on this thread ("" if none). */
const char* tv_last_error(void);
/* TV_VERSION of the built library. */
int tv_version(void);

/* ---------------------------------------------------------------------------
 * tree_build: topology encoder (the precomputed topology-aware mask).
 *
 *   parent     [B][n] int32   parent[b][0] == -1, 0 <= parent[b][u] < u
 *   depth      [B][n] int32   depth[b][0] == 0, depth[u] == depth[parent[u]] + 1
 *   prefix_len [B]    int32   cached prefix length L_b of each sequence
 *   anc_mask   [B][n][W] uint64  out: ancestor bitmask of each node (u included)
 *   pos_ids    [B][n] int32   out: L_b + depth[b][u] (the root sits at L_b)
 *   status     [B]    int32   out: TV_OK, or TV_ETOPOLOGY if sequence b breaks
 *                             the rules above; its mask/pos rows are then
 *                             unspecified (but written in bounds).
 * 1 <= n <= TV_NMAX, B >= 0 (B == 0 enqueues nothing).  Host errors: TV_EINVAL.
 * ------------------------------------------------------------------------- */
int tree_build(int B, int n, const int32_t* parent, const int32_t* depth,
               const int32_t* prefix_len, uint64_t* anc_mask, int32_t* pos_ids,
               int32_t* status, void* stream);

/* Same rules, checked synchronously on HOST arrays parent[n], depth[n].
 * Returns TV_OK, TV_ETOPOLOGY, or TV_EINVAL (null pointer, n out of range). */
int tree_validate_host(int n, const int32_t* parent, const int32_t* depth);

/* ---------------------------------------------------------------------------
 * tree_attention: O = tree attention of every node over prefix + S_u.
 *
 * Defined by the SpecInfer explainer, token-tree structure section: the
 * attention equation over the ancestor set S_u (the root path of u, u
 * included) under the topology-aware mask; the cached prefix joins the same
 * softmax because the mask is kept consistent with KV-cache reuse (its list of
 * contributions).  Its implementation-points section (kernel fusion) fixes the
 * precomputed mask taken here as anc_mask.
 *
 * For node u of sequence b and query head h (KV head g = h / (Hq/Hkv)):
 *   O[b][u][h] = sum_j p_j V_j / sum_j p_j,  p_j = exp(s_j - max s),
 *   s_j = scale * <Q[b][u][h], K_j>,
 * over j in { prefix tokens 0..L_b-1 } U { tree nodes v in S_u }, as one
 * softmax.  lse[b][u][h] = max s + ln(sum_j p_j) (natural log).
 *
 * Layouts (E = element type of desc->dtype, D = head dim):
 *   q, k_tree, v_tree, out   [B][n][H][D]       (H = Hq for q/out, Hkv for k/v)
 *   contiguous cache (paged == 0):
 *     k_cache, v_cache  [B][Hkv][Lmax][D]
 *   paged cache (paged == 1, block_size == 16), prefix token j of sequence b
 *   lives in physical block block_table[b][j / 16], slot j % 16:
 *     k_cache, v_cache  [num_blocks][Hkv][16][D]
 *     block_table [B][max_blocks] int32
 *   anc_mask [B][n][W] from tree_build;  lse [B][n][Hq] float (may be NULL).
 *
 * Supported: dtype TV_BF16 or TV_F16 (fp32 accumulation; the probabilities
 * entering the PV product and the output are rounded to the same 16-bit type;
 * FP16 is the precision of the explainer's implementation points) or TV_F32;
 * D in {64, 128}; Hq % Hkv == 0; 1 <= n <= TV_NMAX; Lmax % 16 == 0.
 * 0 <= prefix_len[b] <= capacity (Lmax, or max_blocks*16); paged block ids in
 * [0, num_blocks).  Out-of-range device values are not trusted: a length is
 * clamped to [0, capacity] and a bad block id's tokens read as zeros, so no
 * read leaves the buffers (O of that sequence is then unspecified), and if
 * `status` [B] (may be NULL) is given it reports TV_EINVAL for that sequence
 * (TV_OK otherwise).
 * Cache slots past L_b are never read (they may hold NaN).
 *
 * fp8 cache (kv_dtype == TV_FP8_E4M3): the prefix K/V are OCP FP8 E4M3 codes
 * (1 byte, same layouts) with per-tensor scales; the tree K/V, q and out stay
 * bf16.  Codes are converted to bf16 (exactly) in LDS before the matrix
 * products; k_scale joins the score scale and v_scale multiplies the
 * probabilities entering the PV product (the softmax normaliser sums the
 * unscaled probabilities).  Supported with dtype TV_BF16 and at most 128
 * query rows per KV head (n * Hq / Hkv <= 128); otherwise TV_EUNSUPPORTED.
 * An fp8 cache halves the prefix bytes.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t B, n, Hq, Hkv, D;
  int32_t dtype;        /* tv_dtype of q, caches, tree K/V and out           */
  float scale;          /* softmax scale; 0 means 1/sqrt(D)                   */
  int32_t paged;        /* 0 contiguous, 1 paged                              */
  int32_t block_size;   /* paged: must be TV_PAGE                             */
  int32_t Lmax;         /* contiguous: per-sequence capacity (tokens)         */
  int32_t max_blocks;   /* paged: block_table row length                      */
  int32_t num_blocks;   /* paged: physical blocks in the cache                */
  int32_t kv_dtype;     /* element type of k_cache/v_cache: 0 = dtype, or
                           TV_FP8_E4M3 (OCP FP8 codes, 1 byte; dtype TV_BF16)  */
  float k_scale;        /* fp8 cache: a key's value is code * k_scale (> 0)   */
  float v_scale;        /* fp8 cache: a value's value is code * v_scale (> 0) */
} tv_attn_desc;

/* Workspace bytes tree_attention needs for this descriptor (0 if none); the
 * split of long prefixes into chunks depends only on the descriptor.
 * Returns (size_t)-1 for an invalid descriptor. */
size_t tree_attention_workspace_size(const tv_attn_desc* desc);

int tree_attention(const tv_attn_desc* desc, const void* q,
                   const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* prefix_len,
                   const void* k_tree, const void* v_tree,
                   const uint64_t* anc_mask, void* out, float* lse,
                   int32_t* status, void* workspace, size_t workspace_bytes,
                   void* stream);

/* ---------------------------------------------------------------------------
 * tree_attention_noalloc: tree_attention with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments (minus workspace), layouts, results and error behaviour as
 * tree_attention, computed by the same kernels.  The partial results that
 * tree_attention keeps in the caller's workspace go to a scratch array the
 * library holds in each GPU's memory, TV_NOALLOC_SCRATCH_BYTES long (every
 * plan of the numbered workloads fits; tree_attention_workspace_size gives a
 * descriptor's need).  A descriptor needing more returns TV_EWORKSPACE before
 * anything is enqueued.  The call itself allocates nothing: the array exists
 * from the library's load until the process ends, and its address on the
 * current device is looked up once, on the first call there.
 *
 * The array of the CURRENT device is used, so `stream` must belong to it.
 * All calls on one GPU share that array: two calls that may run at the same
 * time on one GPU (different streams, or different host threads) race and
 * may return wrong results.  Calls in one stream are ordered and safe.
 * Nothing in the array needs to start at zero.
 * ------------------------------------------------------------------------- */
#define TV_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)

int tree_attention_noalloc(const tv_attn_desc* desc, const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* prefix_len,
                           const void* k_tree, const void* v_tree,
                           const uint64_t* anc_mask, void* out, float* lse,
                           int32_t* status, void* stream);

/* ---------------------------------------------------------------------------
 * tree_verify_greedy: greedy verification of the token tree.
 *
 *   logits  [B][n][V]  logits_dtype (TV_BF16, TV_F16 or TV_F32): the target model's
 *                      next-token logits after each node
 *   tokens  [B][n] int32  draft token of each node (tokens[b][0] is ignored)
 *   parent  [B][n] int32  as for tree_build (assumed valid)
 *   argmax_out [B][n] int32  out: lowest index of the row maximum of logits
 *   path_out   [B][n] int32  out: accepted node ids, root first, -1 padded
 *   path_len   [B]    int32  out: accepted nodes including the root (>= 1)
 *   bonus      [B]    int32  out: argmax at the last accepted node, i.e. the
 *                            token the target model supplies after the path
 * Walk: cur = root; while some child c of cur has tokens[c] == argmax[cur],
 * move to the lowest-numbered such c.  A step emits path_len-1 draft tokens
 * plus the bonus token.  NaN logits are out of contract.
 * 1 <= n <= TV_NMAX, V >= 1.
 * ------------------------------------------------------------------------- */
int tree_verify_greedy(int B, int n, int V, int logits_dtype, const void* logits,
                       const int32_t* tokens, const int32_t* parent,
                       int32_t* argmax_out, int32_t* path_out, int32_t* path_len,
                       int32_t* bonus, void* stream);

/* ---------------------------------------------------------------------------
 * tree_verify_stochastic: stochastic verification by multi-step speculative
 * sampling (the explainer's tree-verification section: a draft token x is
 * accepted with probability min(1, P_LLM(x)/P_SSM(x)); after a rejection the
 * LLM distribution becomes the normalised residual max(0, P_LLM - P_SSM); the
 * emitted tokens then follow the LLM's own distribution).
 *
 * Walk, per sequence: cur = root, p = softmax(logits[cur]).  For each child c
 * of cur in increasing node id, with x = tokens[c] and q = softmax(ssm[c]):
 * accept iff u_accept[c] * q(x) < p(x); on acceptance cur = c and the walk
 * restarts there with p = softmax(logits[c]); on rejection
 * p = norm(max(0, p - q)) (p unchanged if that is all zero) and the next child
 * is tried.  When no child is accepted, bonus = the smallest token y with
 * sum_{t <= y} p(t) > u_sample[cur] (the last token with p > 0 if rounding
 * leaves none), and the walk ends.  Softmax at temperature 1 (scale the logits
 * beforehand for another temperature).
 *
 *   logits, ssm_logits [B][n][V] logits_dtype: the LLM's logits after each node
 *                      and, for node c >= 1, the SSM logits its draft token was
 *                      sampled from (row 0 of ssm_logits is not read)
 *   tokens, parent [B][n] int32   as for tree_verify_greedy
 *   u_accept, u_sample [B][n] float   uniforms in [0, 1) (entry 0 of u_accept
 *                      is not read)
 *   path_out [B][n], path_len [B], bonus [B] int32   out, as for the greedy call
 *   status [B] int32 out (may be NULL): TV_OK, or TV_EINVAL for a sequence
 *     whose parent array is not topological with root 0 or whose draft token
 *     is outside [0, V); its path_len is then 0, path -1 and bonus -1.
 *   mode: 0 = chosen from the sizes; 1 = each sequence's walk reads only the
 *     rows it visits (the statistics of a visited node's rows are gathered
 *     by the walk); 2 = a parallel pass first gathers the statistics of every
 *     LLM and SSM row (reads all of them once), and the walk then reads rows
 *     only for residuals and the final draw; 3 = mode 1 with each sequence's
 *     walk spread over up to 16 workgroups, each owning a slice of the
 *     vocabulary, which exchange row statistics through the workspace at each
 *     step (slices chosen so that all B * slices workgroups fit on the device
 *     at once, 768 on MI355X; it needs `status`, else mode 1 runs).  Mode 2
 *     spreads its walk over slices the same way (they exchange only at the
 *     residual passes and the draw), with the same condition.  0 takes 2
 *     while all rows together are at most 1 GiB, else 3.  The results are the same in every mode.  In mode 3
 *     the exchange waits are bounded: if the slices of a sequence cannot all
 *     run at once (another process holding the GPU's compute units), a slice
 *     gives up, the sequence's status is TV_EHIP and its outputs are
 *     unspecified; every workgroup still exits.  The same holds for mode 2
 *     with slices.
 *   workspace: tree_verify_stochastic_workspace_size(B, n, V) bytes (fp32
 *     residual rows and row statistics), 16-byte aligned; contents on entry
 *     do not matter.
 * Every logits row needs a finite maximum; NaN is out of contract.
 * Decisions are taken in fp32 (softmax with fp32 sums): a draw whose margin
 * to a decision boundary is below that rounding may differ from an exact
 * evaluation.  1 <= n <= TV_NMAX, 1 <= V <= TV_MSS_VMAX.
 * ------------------------------------------------------------------------- */
#define TV_MSS_VMAX (1 << 20)
size_t tree_verify_stochastic_workspace_size(int B, int n, int V);
int tree_verify_stochastic(int B, int n, int V, int logits_dtype, int mode, const void* logits,
                           const void* ssm_logits, const int32_t* tokens,
                           const int32_t* parent, const float* u_accept,
                           const float* u_sample, int32_t* path_out,
                           int32_t* path_len, int32_t* bonus, int32_t* status,
                           void* workspace, size_t workspace_bytes, void* stream);

/* tree_verify_stochastic_set_poll_limit: the bound on mode 3's waits.  A slice
 * reads each word of its peers' exchange records at most `polls` times
 * (default 262144, each poll a device-scope load and a short sleep) before it
 * gives up as described above.  The limit is process-wide and is read when a
 * call is enqueued; calls already enqueued keep theirs.  0 makes every slice
 * give up at its first exchange, so the give-up path can be exercised from the
 * host.  polls < 0: TV_EINVAL.  *previous (if not NULL) receives the limit in
 * force before the call. */
int tree_verify_stochastic_set_poll_limit(int polls, int* previous);

/* ---------------------------------------------------------------------------
 * Token-tree construction (the explainer's multi-draft section): the
 * expansion-based strategy grows the tree by one SSM's top-k tokens per step
 * (configuration <k1, ..., km>); the merge-based strategy merges several SSMs'
 * drafts into one token tree.  Both produce the parent/depth/tokens arrays
 * tree_build and the verification calls take.
 *
 * tree_expand_topk: one expansion step.
 *   ssm_logits [B][F][V] logits_dtype: the SSM's logits after each frontier node
 *   frontier   [B][F] int32  node ids to expand, -1 = unused slot (1 <= F <= 256)
 *   n_cur      [B]    int32  nodes already in each tree (1 <= n_cur <= n_max)
 *   parent, depth, tokens [B][n_max] int32  in/out: entries u < n_cur hold the
 *              tree; the step appends nodes n_cur .. n_cur + r*k - 1 (r = valid
 *              frontier slots), the r-th valid slot's children at
 *              n_cur + r*k + j, j < k, with token = the j-th largest entry of its
 *              row (ties to the lower token id), parent = the frontier node,
 *              depth = its depth + 1.  Other entries are not written.
 *   scores     [B][n_max] float out (may be NULL): the chosen logit of each new node
 *   n_out      [B] int32 out: n_cur + r*k
 *   status     [B] int32 out: TV_OK, or TV_EINVAL (nothing appended, n_out =
 *              n_cur) for a frontier id outside [0, n_cur), n_cur outside
 *              [1, n_max], or more than n_max nodes after the step.
 * 1 <= k <= TV_TOPK_MAX, k <= V, n_max <= TV_NMAX.  NaN logits are out of
 * contract.  The appended rows must not alias the frontier's own rows.
 * ------------------------------------------------------------------------- */
#define TV_TOPK_MAX 16
int tree_expand_topk(int B, int F, int V, int k, int n_max, int logits_dtype,
                     const void* ssm_logits, const int32_t* frontier,
                     const int32_t* n_cur, int32_t* parent, int32_t* depth,
                     int32_t* tokens, float* scores, int32_t* n_out,
                     int32_t* status, void* stream);

/* tree_merge_drafts: the trie of each sequence's drafts.
 *   drafts     [B][M][Ld] int32  draft token sequences (any int32 tokens)
 *   draft_len  [B][M]     int32  tokens in each draft (0 <= len <= Ld)
 *   root_token [B]        int32  token of node 0 (may be NULL: 0)
 *   parent, depth, tokens [B][n_max] int32 out: the tree; every draft is inserted
 *              from the root, reusing the child with the same token where there
 *              is one, drafts in order and positions in order; node ids follow
 *              creation.  Entries from n on are -1.
 *   n_out      [B] int32 out: nodes, root included
 *   node_of    [B][M][Ld] int32 out (may be NULL): the node of each draft
 *              position, -1 past the draft's length
 *   status     [B] int32 out: TV_OK, or TV_EINVAL (n_out = 0, all -1) for a
 *              length outside [0, Ld] or a tree of more than n_max nodes.
 * 1 <= M <= TV_MERGE_MMAX, 1 <= Ld < TV_NMAX, 1 <= n_max <= TV_NMAX.
 * ------------------------------------------------------------------------- */
#define TV_MERGE_MMAX 64
int tree_merge_drafts(int B, int M, int Ld, int n_max, const int32_t* drafts,
                      const int32_t* draft_len, const int32_t* root_token,
                      int32_t* parent, int32_t* depth, int32_t* tokens,
                      int32_t* n_out, int32_t* node_of, int32_t* status,
                      void* stream);

/* ---------------------------------------------------------------------------
 * tree_commit_kv: the accepted path's keys and values become prefix tokens.
 *
 * After verification the accepted root path is an ordinary continuation of the
 * sequence: its KV is written into the cache right after the prefix, in path
 * (root-first, depth-first) order, so the next step attends it as prefix (the
 * explainer's kernel-fusion section: depth-first order keeps the tree consistent
 * with the existing KV cache; its "practical applications" section: the
 * block-wise memory of PagedAttention).  For sequence b with L = prefix_len[b]
 * and P = path_len[b]:
 *   cache position L + t  <-  k_tree[b][path[b][t]], v_tree[b][path[b][t]]
 *                             (all Hkv heads), t = 0 .. P-1
 *   new_prefix_len[b] = L + P
 *
 *   desc        as for tree_attention (Hq and scale are not used)
 *   k_cache, v_cache   in/out, layouts of tree_attention; only positions
 *                      L..L+P-1 of each sequence are written.  Paged: the
 *                      caller has already put blocks for those positions in
 *                      block_table (block allocation is the caller's).
 *   k_tree, v_tree  [B][n][Hkv][D]    path [B][n], path_len [B] int32 (the
 *                   outputs of tree_verify_greedy; entries t >= P not read)
 *   new_prefix_len [B] int32 out; must not overlap prefix_len
 *   status [B] int32 out (may be NULL): TV_OK, or TV_EINVAL for a sequence with
 *     P outside [0, n], a path entry t < P outside [0, n), L < 0,
 *     L + P > capacity, or (paged) a block id for positions L..L+P-1 outside
 *     [0, num_blocks).  Such a sequence is not written at all and its
 *     new_prefix_len is L.
 * Blocks written for different sequences must be distinct (writes to a block
 * shared by two sequences race).  Host errors: TV_EINVAL, TV_EUNSUPPORTED as
 * for tree_attention.
 * ------------------------------------------------------------------------- */
int tree_commit_kv(const tv_attn_desc* desc, void* k_cache, void* v_cache,
                   const int32_t* block_table, const int32_t* prefix_len,
                   const void* k_tree, const void* v_tree, const int32_t* path,
                   const int32_t* path_len, int32_t* new_prefix_len,
                   int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TREE_VERIFY_H */
