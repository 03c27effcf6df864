/*
 * gdn.h -- C ABI of the Gated DeltaNet recurrent-mixer library for AMD
 * Instinct MI355X (gfx950).
 *
 * The serving-engine pages describe the problem this library solves
 * ("Architecture", section 8.1 and its table; repository "Architecture" page,
 * "The decode loop" and its sequence diagram): each recurrent layer keeps, per
 * sequence, a fixed-size fp32 state of Hv heads of dv x dk plus a 4-wide
 * convolution tail; the engine advances it one token at a time, branches it
 * over a draft tree of up to 32 nodes in one verify pass, and then commits the
 * accepted path, or undoes the round by not committing.  Long prompts are
 * prefilled in chunks; the CPU page ("Serving a research architecture on
 * CPU", exactness section) notes that the chunked and the token-by-token
 * forms are the same algebra with different rounding.
 *
 * Per token and sequence, with C = 2*Hk*dk + Hv*dv conv channels (q | k | v):
 *   tail   shifts left by one and takes the raw input x[c] as its newest entry
 *   conv   y[c] = SiLU(sum_{j<4} w[c][j] * tail[c][j])
 *   norm   q^ = q~ / sqrt(|q~|^2 + 1e-6), k^ likewise, per q/k head
 *   gates  alpha = exp(-softplus(a)), beta = sigmoid(b), per value head
 *   state  S <- alpha*S + beta*(v - alpha*S k^) k^T      (rank-1, in place)
 *   output o = (S q^) / sqrt(dk)                         (from the new state)
 * Value head h reads q/k head h / (Hv/Hk).
 *
 * Conventions for every call below.
 *   Memory: every array pointer is caller-owned DEVICE memory on the current
 *     HIP device, 16-byte aligned, dense, in the layout stated.  The library
 *     allocates nothing, keeps no mutable global state, never synchronises,
 *     and enqueues all work on `stream` (a hipStream_t passed as void*; NULL
 *     is the null stream).  Calls are graph-capturable.
 *   Errors: argument errors the host can see are returned before anything is
 *     enqueued, with nothing written.  A failed launch returns GDN_ERR_HIP.
 *     Errors only the device can see (a malformed parent or path array) are
 *     reported through an optional device status word; then the checkpoint
 *     state and tail are left as they were.
 *   Types: state, y, a, b and o are fp32.  x, the conv tail and the conv
 *     weights share the activation type (GDN_BF16 or GDN_F32).
 *   Supported shapes: head_k_dim == head_v_dim in {32, 128};
 *     num_v_heads % num_k_heads == 0; conv_width == 4; batch >= 1.
 *   Concurrency: calls on different streams with disjoint buffers are
 *     independent; calls that share an in/out buffer must be ordered by the
 *     caller.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1
#define GDN_MAX_TREE_NODES 32 /* draft trees of up to 32 nodes (decode-loop diagram) */
#define GDN_MAX_TREE_DEPTH 8  /* nodes on a root-to-leaf path, root counted */
#define GDN_MAX_TREE_BATCH 65535 /* sequences per tree verify or commit call */
#define GDN_PREFILL_CHUNK 64

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,       /* unsupported or inconsistent dims, or a size out of range */
    GDN_ERR_DTYPE = 3,       /* act_dtype is not GDN_F32 or GDN_BF16 */
    GDN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    GDN_ERR_TREE = 5,        /* malformed tree or path (also the device status value) */
    GDN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
    GDN_ERR_HIP = 7,         /* the HIP runtime refused a launch */
    GDN_ERR_ALIAS = 8,       /* buffers that must be distinct overlap */
    GDN_ERR_SIGNATURE = 9,   /* a snapshot of another layer shape or format (device status value) */
    GDN_ERR_INDEX = 10,      /* a sequence index out of range, or repeated where it must not be (device status value) */
    GDN_ERR_SELF_CHECK = 11  /* the self-check found verify or commit rows that differ from decode (device value) */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef struct {
    int32_t batch;        /* B: independent sequences */
    int32_t num_k_heads;  /* Hk: q/k heads */
    int32_t num_v_heads;  /* Hv: value heads = state heads */
    int32_t head_k_dim;   /* dk */
    int32_t head_v_dim;   /* dv */
    int32_t conv_width;   /* W: must be 4 */
    int32_t act_dtype;    /* gdn_dtype of x, conv tail and conv weights */
} gdn_dims;

/* Library version and a static message for a status code. */
int gdn_abi_version(void);
const char* gdn_status_str(int status);

/* Sizes, computable before any model exists; none depends on the number of
 * tokens.  0 for dims the library does not support. */
size_t gdn_conv_channels(const gdn_dims* d);   /* C = 2*Hk*dk + Hv*dv */
size_t gdn_state_bytes(const gdn_dims* d);     /* B*Hv*dv*dk*4 */
size_t gdn_conv_tail_bytes(const gdn_dims* d); /* B*C*W*sizeof(act) */

/*
 * gdn_conv_update -- one token of the causal depthwise conv (section 8.1
 * table's 4-wide tail; the CPU page's convolution rings).
 *   x         act  [B][C]     raw q|k|v activations of this token (read)
 *   conv_tail act  [B][C][4]  last four raw inputs, oldest first (in/out)
 *   conv_w    act  [C][4]     taps, tap 3 multiplies the newest input (read)
 *   y         f32  [B][C]     SiLU(conv) (written)
 */
gdn_status gdn_conv_update(const gdn_dims* d, const void* x, void* conv_tail,
                           const void* conv_w, float* y, void* stream);

/*
 * gdn_decode_step -- one token of the recurrence for every sequence
 * (section 8.1: a fixed-size state advanced per token; CPU page: a rank-1
 * update written in place).
 *   state f32 [B][Hv][dv][dk]  rows over the value index, contiguous over keys (in/out)
 *   y     f32 [B][C]           output of gdn_conv_update for this token (read)
 *   a, b  f32 [B][Hv]          gate inputs (read)
 *   o     f32 [B][Hv][dv]      output (written)
 */
gdn_status gdn_decode_step(const gdn_dims* d, float* state, const float* y,
                           const float* a, const float* b, float* o, void* stream);

/*
 * gdn_decode_token -- gdn_conv_update followed by gdn_decode_step, in one
 * launch (section 8.1: state and 4-wide tail advanced per token; CPU page:
 * rank-1 update in place, convolution rings).  state and o are bit-identical
 * to the two calls; conv_tail_out receives exactly what gdn_conv_update would
 * leave in the tail.  The tail is updated out of place so that no reader of a
 * channel's window races its writer: the caller alternates two tail buffers.
 *   state          f32 [B][Hv][dv][dk]  (in/out)
 *   conv_tail_in   act [B][C][4]        last four raw inputs before this token (read)
 *   conv_tail_out  act [B][C][4]        the same after this token (written); must not
 *                                       overlap conv_tail_in (GDN_ERR_ALIAS)
 *   conv_w act [C][4];  x act [B][C];  a, b f32 [B][Hv];  o f32 [B][Hv][dv] (written)
 */
gdn_status gdn_decode_token(const gdn_dims* d, float* state, const void* conv_tail_in, void* conv_tail_out,
                            const void* conv_w, const void* x, const float* a, const float* b, float* o,
                            void* stream);

/*
 * gdn_kda_decode_step / gdn_kda_decode_token -- the per-channel-decay variant
 * of the two calls above (the model-arch page's module list: a Kimi Delta
 * Attention mixer with a CPU reference and GPU launches; the pages do not
 * define it).  Everything is as in gdn_decode_step / gdn_decode_token except
 * the forget gate, which is one value per key channel of each value head and
 * scales the state's key columns before the delta correction:
 *   alpha[c] = exp(-softplus(a[c]))
 *   S <- S diag(alpha) + beta*(v - S diag(alpha) k^) k^T;  o = (S q^) / sqrt(dk)
 * With every a[c] of a head equal to one value, this is the gated delta rule
 * with that gate (to rounding; the two kernels order the products differently).
 *   a  f32 [B][Hv][dk]   per-channel forget-gate inputs (read)
 *   b  f32 [B][Hv]       write-gate inputs (read)
 *   all other arguments, layouts and errors as in gdn_decode_step (y from
 *   gdn_conv_update) and gdn_decode_token (fused conv, out-of-place tail).
 */
gdn_status gdn_kda_decode_step(const gdn_dims* d, float* state, const float* y,
                               const float* a, const float* b, float* o, void* stream);
gdn_status gdn_kda_decode_token(const gdn_dims* d, float* state, const void* conv_tail_in, void* conv_tail_out,
                                const void* conv_w, const void* x, const float* a, const float* b, float* o,
                                void* stream);

/*
 * gdn_tree_verify -- one read-only pass over a draft tree of n_nodes tokens
 * per sequence (decode-loop diagram: a tree of up to 32 nodes verified in one
 * pass; section 8.1: the state must be branched for a tree of guesses; the
 * parallel server verifies several requests' trees in one forward pass).
 * Each of the batch's sequences has a tree of its own.  Node 0 is the root,
 * the last committed token, whose parent is the checkpoint; every other
 * node's state is branched from its parent's.  Node n's output equals, bit
 * for bit, the output of gdn_conv_update + gdn_decode_step run over the
 * root-first path to n from the sequence's checkpoint.  1 <= batch <=
 * GDN_MAX_TREE_BATCH and num_v_heads / num_k_heads <= 64 (GDN_ERR_SHAPE
 * otherwise; this also holds for gdn_commit_path and the block calls); every
 * tree has n_nodes nodes (a smaller tree can be
 * padded with extra children of its root, whose outputs the caller ignores).
 *   state_ckpt f32 [B][Hv][dv][dk]    checkpoints (read only)
 *   conv_tail  act [B][C][4]          checkpoint tails (read only)
 *   conv_w     act [C][4]
 *   n_nodes    1..32
 *   parent     i32 [B][n_nodes]   per row: parent[0] == -1, 0 <= parent[i] < i,
 *              depth <= 8
 *   x          act [B][n_nodes][C];  a, b f32 [B][n_nodes][Hv]
 *   o          f32 [B][n_nodes][Hv][dv]  (written)
 *   tree_status i32 [B] or NULL: per sequence, set to GDN_OK, or GDN_ERR_TREE
 *              when its parent row is malformed (its o is then undefined;
 *              the other sequences are verified as usual).
 *   workspace  device bytes >= gdn_tree_workspace_bytes(d, n_nodes), 16-byte
 *              aligned, caller-owned: each node's normalised q/k, v and gates
 *              are prepared there once and shared by every value head (about
 *              1.3 MB per sequence for 32 nodes at 16 q/k and 48 value heads
 *              of 128).
 */
size_t gdn_tree_workspace_bytes(const gdn_dims* d, int32_t n_nodes);
gdn_status gdn_tree_verify(const gdn_dims* d, const float* state_ckpt, const void* conv_tail,
                           const void* conv_w, int32_t n_nodes, const int32_t* parent,
                           const void* x, const float* a, const float* b, float* o,
                           int32_t* tree_status, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * gdn_tree_verify_ut -- gdn_tree_verify in the UT form, the tree counterpart
 * of the chunked form's WY/UT representation (chunked prefill: intra-chunk
 * WY/UT contractions, inter-chunk carry; here "ancestor of" takes the place of
 * "earlier in the chunk").  No node's state is built: each sequence's
 * checkpoint enters once, as one product with 32 derived query vectors per
 * value head, and the small per-head matrices run on fp32 MFMA.  The same
 * arguments, status and error behaviour as gdn_tree_verify, except that the
 * workspace is optional:
 *   workspace NULL   one launch: each (sequence, value head) workgroup
 *                    convolves, normalises and gates its own nodes' operands;
 *                    nothing is prepared for gdn_commit_path_prepared (commit
 *                    with gdn_commit_path).
 *   workspace given  (>= gdn_tree_workspace_bytes) the nodes' operands are
 *                    also prepared in the workspace, as by gdn_tree_verify,
 *                    and gdn_commit_path_prepared may follow.  Up to 4
 *                    sequences (bf16 activations) this is still one launch (the verify of the
 *                    first form beside the preparation, whose outputs it
 *                    shares); above, two launches, the second reading the
 *                    prepared operands.
 * The outputs agree with token-by-token decode to rounding (within 1e-4
 * normwise of the sequential definition), not bit for bit, and the forms may
 * round differently.  A commit of the accepted path is exact either way: it
 * replays the path.
 */
gdn_status gdn_tree_verify_ut(const gdn_dims* d, const float* state_ckpt, const void* conv_tail,
                              const void* conv_w, int32_t n_nodes, const int32_t* parent,
                              const void* x, const float* a, const float* b, float* o,
                              int32_t* tree_status, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * gdn_commit_path -- commit the accepted root-first path of each sequence's
 * verified tree (decode-loop diagram: commit the accepted path's recurrent
 * state; section 8.1: exact undo).  A sequence's new (state, tail) is
 * bit-identical to one gdn_conv_update + gdn_decode_step per token of its
 * path.  Undo is not calling this, or, for one sequence of a batch, a path
 * row of -1 only, which commits nothing.
 *   state      f32 [B][Hv][dv][dk]  in: checkpoints, out: committed (in/out)
 *   conv_tail  act [B][C][4]        in/out
 *   conv_w, n_nodes, parent, x, a, b: as for gdn_tree_verify
 *   path_len   1..min(n_nodes, 8): the width of a path row
 *   path       i32 [B][path_len]: per row the accepted path, root first
 *              (path[0] == 0, parent[path[j]] == path[j-1]), then -1 in every
 *              entry after its end, so rows may have different lengths (and
 *              length 0: -1 throughout).
 *   o          f32 [B][path_len][Hv][dv] or NULL: per-token outputs (entries
 *              past a row's end are not written)
 *   tree_status i32 [B] or NULL: per sequence, GDN_OK, or GDN_ERR_TREE for a
 *              malformed tree or path row, in which case that sequence's state
 *              and tail are untouched.
 */
gdn_status gdn_commit_path(const gdn_dims* d, float* state, void* conv_tail, const void* conv_w,
                           int32_t n_nodes, const int32_t* parent, const void* x,
                           const float* a, const float* b, int32_t path_len,
                           const int32_t* path, float* o, int32_t* tree_status, void* stream);

/*
 * gdn_commit_path_prepared -- gdn_commit_path for the tree just verified with
 * this workspace (decode-loop diagram: verify, then commit the accepted
 * path): the path's normalised q/k, v and gates are read from the workspace
 * that gdn_tree_verify or gdn_tree_verify_ut filled for the same trees
 * instead of being convolved again.  The caller guarantees that the
 * workspace still holds that call's operands (same batch, n_nodes, parent, x,
 * a, b, conv tail and weights; nothing else written to it in between);
 * otherwise the committed state is wrong, though every access stays in
 * bounds.  The result is bit-identical to gdn_commit_path, and so to
 * gdn_conv_update + gdn_decode_step per path token.  Argument checks, path
 * rows, statuses and the tail update are gdn_commit_path's.
 *   workspace  the verify's workspace, >= gdn_tree_workspace_bytes(d, n_nodes)
 *              bytes, 16-byte aligned (read only)
 */
gdn_status gdn_commit_path_prepared(const gdn_dims* d, float* state, void* conv_tail, int32_t n_nodes,
                                    const int32_t* parent, const void* x, int32_t path_len, const int32_t* path,
                                    float* o, int32_t* tree_status, const void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * gdn_tree_tables -- the device-side tree analysis the two calls above use,
 * exposed so its integer results can be checked exactly.
 *   depth  i32 [n_nodes] root = 1;  order i32 [n_nodes]: depth-first pre-order
 *   visiting children by increasing index;  tree_status i32 [1] (required).
 */
gdn_status gdn_tree_tables(int32_t n_nodes, const int32_t* parent, int32_t* depth,
                           int32_t* order, int32_t* tree_status, void* stream);

/*
 * gdn_prefill_chunked -- T tokens per sequence from (state, tail), in chunks
 * of 64 (repository "Architecture" page: the prompt is prefilled before the
 * decode loop; CPU page: the chunked form is the same algebra as the
 * token-by-token one).  Results match the token-by-token calls up to
 * rounding; state and tail afterwards continue exactly like decode.
 *   state     f32 [B][Hv][dv][dk]  in/out
 *   conv_tail act [B][C][4]        in/out
 *   x act [B][T][C];  a, b f32 [B][T][Hv];  o f32 [B][T][Hv][dv] (written)
 *   workspace device bytes >= gdn_prefill_workspace_bytes(d, T), 256-byte
 *             aligned; its size depends on T only up to 4,096 tokens.
 * This call needs head_k_dim == head_v_dim == 128 and num_v_heads / num_k_heads
 * <= 8 (GDN_ERR_SHAPE otherwise).  Outputs and state are within rounding of
 * the token-by-token calls: operands of the chunk products are fp16, sums and
 * the state carried between chunks are fp32.
 */
size_t gdn_prefill_workspace_bytes(const gdn_dims* d, int32_t T);
gdn_status gdn_prefill_chunked(const gdn_dims* d, float* state, void* conv_tail, const void* conv_w,
                               int32_t T, const void* x, const float* a, const float* b, float* o,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_block_verify -- one read-only pass over a block of k drafted tokens per
 * sequence (repository "Architecture" page, "The parts": delta-rule kernels
 * for one token, a block and a tree; drafters that propose a block of tokens
 * at once): the chain 0 -> 1 -> ... -> k-1 after the checkpoint.  Position t's
 * output equals, bit for bit, the output of gdn_conv_update + gdn_decode_step
 * run over positions 0..t from the sequence's checkpoint.  Unlike a tree, a
 * block has no depth limit below its length.
 *   state_ckpt f32 [B][Hv][dv][dk], conv_tail act [B][C][4]: read only
 *   k          1..32 tokens per sequence
 *   x act [B][k][C];  a, b f32 [B][k][Hv];  o f32 [B][k][Hv][dv] (written)
 *   workspace  device bytes >= gdn_block_workspace_bytes(d, k), 16-byte aligned
 * A longer block is verified in parts of up to 32 with gdn_block_commit of
 * each part in between (on a snapshot, if it may be rejected), or with
 * gdn_prefill_chunked over a copy of the state, which rounds as the chunked
 * form does.  1 <= batch <= GDN_MAX_TREE_BATCH.
 */
size_t gdn_block_workspace_bytes(const gdn_dims* d, int32_t k);
gdn_status gdn_block_verify(const gdn_dims* d, const float* state_ckpt, const void* conv_tail, const void* conv_w,
                            int32_t k, const void* x, const float* a, const float* b, float* o, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * gdn_block_verify_ut -- gdn_block_verify in the UT form (a block is the chain
 * tree; see gdn_tree_verify_ut): the same arguments and errors, outputs equal
 * to decode's to rounding.  As there, workspace may be NULL (one launch, nothing
 * prepared for gdn_block_commit_prepared).
 */
gdn_status gdn_block_verify_ut(const gdn_dims* d, const float* state_ckpt, const void* conv_tail,
                               const void* conv_w, int32_t k, const void* x, const float* a, const float* b,
                               float* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_block_commit -- advance each sequence by the first accepted[seq] tokens
 * of its block, bit-identical to one gdn_conv_update + gdn_decode_step per
 * token.
 *   state f32 [B][Hv][dv][dk], conv_tail act [B][C][4]: in/out
 *   k, x, a, b, workspace: as for gdn_block_verify
 *   accepted   i32 [B] (device): 0..k tokens; 0 commits nothing
 *   o          f32 [B][k][Hv][dv] or NULL: outputs of the committed positions
 *              (later positions are not written)
 *   status     i32 [B] or NULL: per sequence GDN_OK, or GDN_ERR_INDEX when its
 *              accepted count is out of range (that sequence is untouched)
 */
gdn_status gdn_block_commit(const gdn_dims* d, float* state, void* conv_tail, const void* conv_w, int32_t k,
                            const void* x, const float* a, const float* b, const int32_t* accepted, float* o,
                            int32_t* status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_block_commit_prepared -- gdn_block_commit for the blocks just verified
 * with this workspace (gdn_block_verify or gdn_block_verify_ut on the same
 * inputs): the positions' normalised q/k, v and gates are read from the
 * workspace instead of being prepared again.  The caller guarantees that the
 * workspace still holds that call's operands; otherwise the committed state
 * is wrong, though every access stays in bounds.  The result is
 * bit-identical to gdn_block_commit; arguments, counts, statuses and the tail
 * update are its.
 *   workspace  the verify's workspace, >= gdn_block_workspace_bytes(d, k) bytes
 */
gdn_status gdn_block_commit_prepared(const gdn_dims* d, float* state, void* conv_tail, int32_t k, const void* x,
                                     const int32_t* accepted, float* o, int32_t* status, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * State snapshots (repository "Architecture" page: the engine must restore a
 * recurrent state exactly from a cache, which copies a sequence's state as
 * sections in a fixed order; a signature over the sections' names, shapes and
 * dtypes refuses a restore across models).  A sequence's state here has two
 * sections, in this order:
 *   "state"      f32 [Hv][dv][dk]
 *   "conv_tail"  act [C][4]
 * gdn_state_signature returns the 64-bit FNV-1a hash of the ASCII text
 *   gdn-state-v1;state:f32[Hv,dv,dk];conv_tail:ACT[C,4]
 * with the numbers in decimal and ACT "bf16" or "f32" (0 for bad dims).  The
 * batch size is not part of it.
 *
 * A snapshot of `count` sequences is one device blob of
 * gdn_snapshot_bytes(d, count) bytes: a 256-byte header (little endian: u32
 * magic GDN_SNAPSHOT_MAGIC, u32 version GDN_SNAPSHOT_VERSION, u64 signature,
 * u32 count, u32 0, u64 state bytes per sequence, u64 tail bytes per
 * sequence, zeros), then the "state" section of all count sequences, then
 * their "conv_tail" section.  The blob can be copied anywhere and back
 * (host, disk) as plain bytes.
 *
 * gdn_snapshot copies sequences seqs[0..count-1] (i32, device, 0 <= seqs[i] <
 * batch; repeats allowed) of (state, conv_tail) into blob slots 0..count-1.
 * gdn_restore copies blob slots 0..count-1 into sequences seqs[i], which must
 * be distinct.  Both write *status (i32, device, required): GDN_OK, or
 * GDN_ERR_INDEX for a bad seqs array, or (restore) GDN_ERR_SIGNATURE when the
 * blob's header does not match d and count; on an error nothing is restored,
 * and a refused snapshot's header has magic 0.  A restored sequence equals,
 * bit for bit, the one that was saved, so decode continues from it exactly.
 * 1 <= count <= GDN_MAX_TREE_BATCH; blob 256-byte aligned.
 */
#define GDN_SNAPSHOT_MAGIC 0x534E4447u /* "GDNS" */
#define GDN_SNAPSHOT_VERSION 1
#define GDN_SNAPSHOT_HEADER_BYTES 256
uint64_t gdn_state_signature(const gdn_dims* d);
size_t gdn_snapshot_bytes(const gdn_dims* d, int32_t count);
gdn_status gdn_snapshot(const gdn_dims* d, const float* state, const void* conv_tail, int32_t count,
                        const int32_t* seqs, void* blob, size_t blob_bytes, int32_t* status, void* stream);
gdn_status gdn_restore(const gdn_dims* d, float* state, void* conv_tail, int32_t count, const int32_t* seqs,
                       const void* blob, size_t blob_bytes, int32_t* status, void* stream);

/*
 * gdn_self_check -- the load-time self-check that gates speculation
 * (repository "Architecture" page, "Kernels and devices, then the mesh": an
 * exact model serves plain decode until a row-invariant kernel exists, and a
 * self-check at load decides whether speculation may run).  It checks, on the
 * device, that tree verify and commit are row-invariant against decode for
 * the layer shape d (d->batch is not used):
 *   - a seeded 32-node tree of depth 8 (a chain of 8 from the root and 24
 *     nodes under its first seven, so siblings sit at the deepest level) is
 *     verified by gdn_tree_verify from a seeded checkpoint;
 *   - 32 copies of the checkpoint replay the root-first paths to the 32
 *     nodes with gdn_decode_token, 8 steps (a shorter path repeats its last
 *     token afterwards);
 *   - every node's output row must equal, bit for bit, its replay's output at
 *     the end of its path, and gdn_commit_path of the depth-8 path must leave
 *     the state and tail that its 8-step replay leaves, bit for bit.
 * Every input is drawn on the device from `seed` (a counter-based hash), so
 * nothing crosses from the host.  The verdict is written, stream-ordered and
 * without synchronising, to result, i32 [4] (device, 16-byte aligned):
 *   result[0]  GDN_OK if every row and word is equal, else GDN_ERR_SELF_CHECK
 *   result[1]  number of output values that differ
 *   result[2]  number of committed state and tail words that differ
 *   result[3]  GDN_OK, or the first non-OK tree or path status of the case
 * flags: 0, or GDN_SELF_CHECK_PERTURB, which flips one input bit of one
 * node's last token in the decode replay only, so that result[0] must come
 * back GDN_ERR_SELF_CHECK (a check of the check).
 *   workspace  device bytes >= gdn_self_check_workspace_bytes(d), caller-owned
 *              (about 120 MB at 48 value heads of 128: the 32 replayed states)
 */
#define GDN_SELF_CHECK_PERTURB 1
size_t gdn_self_check_workspace_bytes(const gdn_dims* d);
gdn_status gdn_self_check(const gdn_dims* d, uint32_t seed, int32_t flags, void* workspace, size_t workspace_bytes,
                          int32_t* result, void* stream);

/*
 * gdn_tree_verify_ut_noalloc -- gdn_tree_verify_ut for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace: the prepared operands go to a
 * library-held device array of GDN_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU,
 * held from the library's first use on that GPU until the process ends.  The
 * caller still passes inputs and outputs; arguments, outputs, statuses and
 * errors are gdn_tree_verify_ut's with a workspace, and the outputs are
 * bit-identical to it (above 4 sequences or with fp32 activations its
 * two-launch form, whose verify reads the prepared operands back).  gdn_tree_verify_ut with no workspace
 * allocates nothing either.
 *   GDN_ERR_WORKSPACE  gdn_tree_workspace_bytes(d, n_nodes) exceeds the array
 *                      (at 16 q/k and 48 value heads of 128 and 32 nodes: more
 *                      than 12 sequences)
 *   GDN_ERR_HIP        the array's device address could not be looked up
 * The call allocates nothing.  Every call on one GPU shares that GPU's array,
 * so calls that may overlap on one GPU (different streams, or host threads)
 * race and must be ordered by the caller.  Each call writes every scratch
 * word it reads before reading it, so what an earlier call left is never used.
 * gdn_commit_path_prepared cannot read this array: commit with
 * gdn_commit_path after it.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (16u << 20)
gdn_status gdn_tree_verify_ut_noalloc(const gdn_dims* d, const float* state_ckpt, const void* conv_tail,
                                      const void* conv_w, int32_t n_nodes, const int32_t* parent, const void* x,
                                      const float* a, const float* b, float* o, int32_t* tree_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
