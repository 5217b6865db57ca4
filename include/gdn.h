/*
 * gdn.h - C ABI of the chunkwise gated delta rule forward on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (gated delta rule problem statement; chunked evaluation as in
 * the chunk_gated_delta_rule_fwd adapter on the hyper-parallel "Diff
 * Coverage" page, _AscendCGDN.forward): for every head of every unit (a batch
 * row, a packed document, or a segment of a row) with state h in K x V,
 *
 *     h_t = (I - beta_t k_t k_t^T) Diag(b^{g_t}) h_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * h_t^T q_t
 *
 * where b = e (use_exp2 = 0) or 2 (use_exp2 = 1) and g_t is a scalar per
 * (token, head) or, for a per-key gate, a K-vector (the KDA form of the
 * state_summary.py coverage page, whose chunk recurrence decays the state
 * before the delta update; for a scalar gate both orders coincide). The work
 * is done in chunks of 64 tokens.
 *
 * Conventions (all taken from the pages' adapters):
 *   - K = V = 128 and chunk_size = 64 are the supported shapes.
 *   - Layout BSND: q, k [B,T,H,K], v [B,T,H,V], g [B,T,H] or [B,T,H,K],
 *     beta [B,T,H]. Layout TND: the same with B = 1 and no batch axis, with
 *     document offsets (cu_seqlens). Both are row-major and contiguous.
 *   - g and beta are used as given: no sigmoid, no L2 norm, no gate
 *     activation inside (normalisation happens before the core).
 *   - Gates are log-decays: every g must be <= 0 (each decay b^g in (0, 1]),
 *     scalar or per key, of any magnitude down to total forgetting (g = -1e4
 *     and below give b^g = 0 exactly). Products of decays are formed from
 *     differences of cumulative gates or as factors of at most 1, never as
 *     quotients, so no intermediate overflows. g > 0 is outside the contract.
 *   - Numeric range with bf16 inputs: the kernels multiply fp16 operands
 *     (bf16 values are exact in fp16's normal range) with fp32 accumulation,
 *     and round the state, the residual and v_new to fp16 once per chunk.
 *     Every |component| of q, k must stay below 2^8, and |v|, the state and
 *     v_new below fp16's 65504; beyond that, values saturate to infinity.
 *     With unit-norm q, k (the pages' convention) and |v| up to 2^11 the
 *     results meet the bf16 parity bar. fp32 inputs use fp32 operands.
 *   - scale multiplies the output; callers normally pass 1/sqrt(K).
 *   - The state is K x V (key-major, "state_v_first = False").
 *
 * Memory: every pointer argument marked "device" is HIP device memory owned
 * by the caller; inputs are never written. The library allocates nothing,
 * never synchronises and keeps no global state: all work is enqueued on the
 * given stream, in order. Scratch memory is the caller's workspace
 * (query its size with workspace == NULL).
 *
 * Errors: every check runs on the host before the first HIP call, so a
 * rejected call enqueues nothing. GDN_ERR_INVALID is a contract violation
 * (the pages raise ValueError), GDN_ERR_UNSUPPORTED a shape or feature this
 * build does not implement (NotImplementedError), GDN_ERR_DEVICE a HIP
 * launch failure (RuntimeError), GDN_ERR_CAPACITY a too-small caller buffer.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID = 1,
    GDN_ERR_UNSUPPORTED = 2,
    GDN_ERR_DEVICE = 3,
    GDN_ERR_CAPACITY = 4
} gdn_status;

enum { GDN_LAYOUT_BSND = 0, GDN_LAYOUT_TND = 1 };
enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 };
enum { GDN_GATE_SCALAR = 0, GDN_GATE_PER_KEY = 1 };

/* gdn_chunk_fwd flags */
enum {
    GDN_FLAG_REUSE_PREPARED = 1, /* skip chunk preparation: the workspace already
                                    holds it (from gdn_state_summary or a
                                    GDN_FLAG_PREPARE_ONLY call with the same
                                    descriptor and inputs) */
    GDN_FLAG_PREPARE_ONLY = 2,   /* run chunk preparation only */
    /* In-kernel input transforms (use_qk_l2norm_in_kernel and
     * use_beta_sigmoid_in_kernel of the native prepare on the Diff Coverage
     * page), also accepted by gdn_state_summary and gdn_chunk_fwd_noalloc.
     * A call with GDN_FLAG_REUSE_PREPARED must repeat the transform flags of
     * the preparing call. */
    GDN_FLAG_QK_L2NORM = 4,      /* q and k replaced by x r, r = 1 / sqrt(sum_i x_i^2 + 1e-6),
                                    per (token, head), in fp32 */
    GDN_FLAG_BETA_SIGMOID = 8    /* beta replaced by 1 / (1 + e^{-beta}) */
};

/*
 * Problem descriptor.
 *
 * Units are contiguous token ranges on the flat token axis (BSND [B,T,...]
 * is viewed as [B*T,...]). With n_units = 0 the units are the B rows of T
 * tokens. Otherwise offsets_host holds n_units + 1 strictly increasing token
 * offsets from 0 to B*T (the _packed_offsets rules of the Diff Coverage
 * page): for TND (B must be 1) they are the documents' cu_seqlens; for BSND
 * they are segments, and every row start b*T must be one of them (a unit
 * never crosses rows). The device arrays are the caller's device copies of
 * the unit offsets and of the chunk metadata that gdn_varlen_meta computes
 * for them; kernels read only these and clamp to the token range, so a
 * mismatch gives wrong results, never out-of-range accesses.
 */
typedef struct {
    int32_t B, T, H, K, V;      /* TND: B = 1 and T = total packed tokens */
    int32_t layout;             /* GDN_LAYOUT_* */
    int32_t dtype;              /* q, k, v, beta: GDN_DTYPE_*; g is always fp32 */
    int32_t o_dtype;            /* output o: GDN_DTYPE_* (fp32 keeps the full
                                   accuracy of the fp32 accumulation) */
    int32_t gate_kind;          /* GDN_GATE_* */
    int32_t use_exp2;           /* 0: decay e^g, 1: decay 2^g */
    int32_t chunk_size;         /* must be 64 */
    float scale;                /* output scale */
    int32_t n_units;            /* 0: dense rows; else entries of offsets - 1 */
    const int32_t* offsets_host;       /* host   [n_units + 1] */
    const int32_t* offsets_dev;        /* device [n_units + 1] */
    const int32_t* chunk_offsets_dev;  /* device [n_units + 1], from gdn_varlen_meta */
    const int32_t* chunk_indices_dev;  /* device [n_chunks][2], from gdn_varlen_meta */
} gdn_desc;

/*
 * Optional extra outputs of gdn_chunk_fwd (any pointer may be NULL; the
 * struct pointer itself may be NULL). These are slots of the native forward
 * on the Diff Coverage page: the saved-for-backward g_cumsum, A and h of its
 * ten-slot result, the v_new that chunk_fwd_h returns, and the input-transform
 * slots q_hat, k_hat, q_rstd, k_rstd and beta_eff. The preparation writes
 * g_cumsum, A and the transform slots (not under GDN_FLAG_REUSE_PREPARED);
 * the state pass writes h and v_new (not under GDN_FLAG_PREPARE_ONLY).
 *   g_cumsum: device fp32, token-major like g ([tokens][H] or
 *             [tokens][H][K]): the gate's inclusive cumulative sum inside
 *             each 64-token chunk of each unit.
 *   A:        device fp32 [tokens][H][64]: row i of the chunk's
 *             T = (I + L)^{-1}, L_ij = beta_i (k_i . k_j) b^{G_i - G_j}
 *             (per key: beta_i sum_d k_id k_jd b^{G_id - G_jd}) for j < i,
 *             the WY inverse that turns the chunk into dense products.
 *   h:        device fp32 [n_chunks][H][K][V]: the state entering every
 *             chunk (chunks ordered by unit, then position in the unit).
 *   v_new:    device fp32 [tokens][H][V]: the value each token writes into
 *             the state, v_new = u - w h = T diag(beta) (v - (k * b^G) h) for
 *             the chunk's entry state h; token by token this is
 *             beta_t (v_t - h~^T k_t), h~ the decayed state before token t.
 *   q_hat, k_hat: device [tokens][H][K] in desc->dtype: q and k as the
 *             recurrence uses them (normalised with GDN_FLAG_QK_L2NORM,
 *             else copies), rounded to the input precision.
 *   q_rstd, k_rstd: device fp32 [tokens][H]: the factor r of the
 *             normalisation (1 without it). q_hat and q_rstd need q.
 *   beta_eff: device [tokens][H] in desc->dtype: beta as the recurrence
 *             uses it (after the sigmoid with GDN_FLAG_BETA_SIGMOID).
 */
typedef struct {
    float* g_cumsum;
    float* A;
    float* h;
    float* v_new;
    void* q_hat;
    void* k_hat;
    float* q_rstd;
    float* k_rstd;
    void* beta_eff;
} gdn_slots;

/*
 * gdn_varlen_meta - chunk metadata of packed sequences (host only).
 * _packed_metadata on the Diff Coverage page: every unit of length L
 * contributes ceil(L / chunk_size) chunks, listed unit-major as
 * (unit index, chunk index in the unit) int32 pairs.
 *
 *   offsets        host [n_offsets]: 0 = c_0 < c_1 < ... < c_N = total_tokens
 *   chunk_indices  host [cap_chunks][2] or NULL (count only)
 *   chunk_offsets  host [n_offsets] or NULL: first chunk of every unit, then
 *                  the total chunk count
 *   n_chunks_out   receives the chunk count (also on GDN_ERR_CAPACITY)
 * Errors: GDN_ERR_INVALID for offsets that break the rules or chunk_size <= 0;
 * GDN_ERR_CAPACITY when chunk_indices is given and cap_chunks is too small.
 */
gdn_status gdn_varlen_meta(const int32_t* offsets, int32_t n_offsets, int32_t total_tokens,
                           int32_t chunk_size, int32_t* chunk_indices, int32_t cap_chunks,
                           int32_t* chunk_offsets, int32_t* n_chunks_out);

/*
 * gdn_chunk_fwd - the chunked forward: gate cumulative sums, the A build and
 * its 64 x 64 triangular inverse (chunk preparation), then the inter-chunk
 * state pass fused with the output.
 *
 *   q, k           device [tokens][H][K] in desc->dtype
 *   v              device [tokens][H][V] in desc->dtype
 *   g              device fp32 [tokens][H] (scalar) or [tokens][H][K] (per key)
 *   beta           device [tokens][H] in desc->dtype
 *   initial_state  device fp32 [units][H][K][V] or NULL (zero state)
 *   o              device [tokens][H][V] in desc->o_dtype
 *   final_state    device fp32 [units][H][K][V] or NULL
 *   slots          optional extra outputs (see gdn_slots) or NULL
 *   flags          GDN_FLAG_* bits
 *   workspace      device scratch of *workspace_bytes bytes, 256-byte
 *                  aligned; NULL: only store the required size in
 *                  *workspace_bytes and return GDN_OK
 *   stream         HIP stream the work is enqueued on
 * With GDN_FLAG_PREPARE_ONLY, q, v, o, initial_state and final_state are not
 * used and may be NULL. The workspace holds the chunk preparation in a layout
 * internal to this library (valid for GDN_FLAG_REUSE_PREPARED with the same
 * descriptor and inputs). Packed units may be processed in any order (the
 * state pass starts the longest first); results do not depend on it.
 */
gdn_status gdn_chunk_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                         const float* g, const void* beta, const float* initial_state, void* o,
                         float* final_state, const gdn_slots* slots, int32_t flags,
                         void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * gdn_state_summary - affine summary of every unit (kda_split_state_summary_kernel
 * on the state_summary.py coverage page): running a unit from an entry state
 * S gives the exit state M S + S_ext, with
 *   S_ext  device fp32 [units][H][K][V]: the exit state from a zero entry
 *   M      device fp32 [units][H][K][K]: the transfer map (I at an empty unit)
 *   mode   0: both, 1: S_ext only (M may be NULL), 2: M only (S_ext may be NULL)
 *   q      device [tokens][H][K] or NULL. The summaries do not read it, but
 *          the chunk preparation that a later reusing forward needs includes
 *          the decayed q.k products (and, with a per-key gate, q * b^G),
 *          which are only prepared when q is given.
 *   flags  0, or GDN_FLAG_REUSE_PREPARED: the workspace already holds the
 *          chunk preparation of this descriptor and these inputs
 *   units_dev, n_sel
 *          n_sel < 0: summarise every unit (units_dev is ignored). Else
 *          units_dev is a device int32 list of n_sel <= n_units unit indices
 *          to summarise (it may be NULL when n_sel = 0, which runs only the
 *          preparation): a summary that nothing consumes (the last
 *          segment's, a piece that ends its document) need not be computed,
 *          as needs_summary on the Diff Coverage page advises. The
 *          results of unit u still land in slot u of S_ext / M; the slots of
 *          unlisted units are left untouched. Indices outside [0, n_units)
 *          are skipped by the kernel.
 * Units are those of desc (normally the segments of a sequence split, or
 * the pieces from gdn_split_meta). The chunk preparation is left in the
 * workspace, so a following gdn_chunk_fwd with the same descriptor, inputs
 * and workspace may pass GDN_FLAG_REUSE_PREPARED (the correction pass of a
 * split scan), provided q was given here.
 */
gdn_status gdn_state_summary(const gdn_desc* desc, const void* q, const void* k, const void* v,
                             const float* g, const void* beta, int32_t mode, int32_t flags,
                             const int32_t* units_dev, int32_t n_sel, float* S_ext, float* M,
                             void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * gdn_split_meta - pieces of packed documents cut into segments (host only;
 * the packed context-parallel plan of the Diff Coverage page, whose ranks
 * hold a head window, whole documents and a tail window). The pieces are the
 * token ranges between consecutive cuts of the union of both offset lists;
 * a piece continues the previous one exactly when both lie in one document.
 *   doc_offsets    host [n_doc_offsets]: cu_seqlens of the documents
 *   seg_offsets    host [n_seg_offsets]: segment cuts (e.g. equal shares)
 *                  both follow the _packed_offsets rules, ending at
 *                  total_tokens
 *   piece_offsets  host [cap_pieces + 1] or NULL (count only)
 *   piece_doc      host [cap_pieces] or NULL: document of each piece
 *   piece_seg      host [cap_pieces] or NULL: segment of each piece
 *   n_pieces_out   receives the piece count (also on GDN_ERR_CAPACITY)
 * GDN_ERR_INVALID for bad offsets, GDN_ERR_CAPACITY when piece_offsets is
 * given and cap_pieces is too small.
 */
gdn_status gdn_split_meta(const int32_t* doc_offsets, int32_t n_doc_offsets, const int32_t* seg_offsets,
                          int32_t n_seg_offsets, int32_t total_tokens, int32_t* piece_offsets,
                          int32_t* piece_doc, int32_t* piece_seg, int32_t cap_pieces,
                          int32_t* n_pieces_out);

/*
 * gdn_state_merge_pieces - entry states of the pieces of a split packed
 * sequence (first_state / last_state of the Diff Coverage page's
 * PackedSequenceInfo, in one ordered pass), in fp32:
 *   S_in[p] = S0_docs[doc(p)] (zero when S0_docs == NULL)  if p starts its document
 *   S_in[p] = M[p-1] S_in[p-1] + S_ext[p-1]                 otherwise
 *   piece_doc_dev  device int32 [n_pieces], non-decreasing document indices
 *                  (gdn_split_meta's piece_doc, copied to the device)
 *   S_ext, M       device fp32 [n_pieces][H][K][V] / [n_pieces][H][K][K]:
 *                  gdn_state_summary over the pieces. Only the slots of pieces
 *                  followed by a piece of the same document are read, and M
 *                  not even there when the piece enters from zero (it starts
 *                  its document and S0_docs is NULL): such pieces need only
 *                  S_ext (summary mode 1)
 *   S0_docs        device fp32 [n_docs][H][K][V] or NULL
 *   S_in           device fp32 [n_pieces][H][K][V]
 * A following gdn_chunk_fwd over the pieces with initial_state = S_in gives
 * the unsplit output, and each document's final state is the final state of
 * its last piece. Documents are merged independently (one workgroup per
 * document, head and 8 state columns); a piece whose document index lies
 * outside [0, n_docs) gets no S_in written, and a piece_doc that is not
 * non-decreasing gives wrong states, never out-of-range accesses.
 * n_docs <= 2^26, H <= 65535.
 */
gdn_status gdn_state_merge_pieces(int32_t n_pieces, int32_t n_docs, int32_t H, int32_t K, int32_t V,
                                  const int32_t* piece_doc_dev, const float* S_ext, const float* M,
                                  const float* S0_docs, float* S_in, hipStream_t stream);

/*
 * gdn_state_merge - composes segment summaries in order (apply_kda_state_summary
 * on the Diff Coverage page; the exclusive prefix of the Sana
 * distributed_scan.py page):
 *   S_init[b][0] = S0[b] (zero when S0 == NULL)
 *   S_init[b][s+1] = M[b][s] S_init[b][s] + S_ext[b][s]   (fp32)
 *   S_ext   device fp32 [B][n_seg][H][K][V]
 *   M       device fp32 [B][n_seg][H][K][K]
 *   S0      device fp32 [B][H][K][V] or NULL
 *   S_init  device fp32 [B][n_seg][H][K][V]: the state entering every segment
 *   S_final device fp32 [B][H][K][V] or NULL: the state after the last segment
 */
gdn_status gdn_state_merge(int32_t B, int32_t H, int32_t n_seg, int32_t K, int32_t V,
                           const float* S_ext, const float* M, const float* S0, float* S_init,
                           float* S_final, hipStream_t stream);

/*
 * gdn_chunk_bwd - gradients of the chunked forward (scalar or per-key gate):
 * the backward slots of the native GDN op on the Diff Coverage page
 * (_AscendCGDN.backward: dq, dk, dv, dbeta and the raw-gate gradient dg), by
 * the staged chunk backward of the same page (_AscendCKDAStages.backward:
 * preparation, the reverse state pass chunk_gated_delta_rule_bwd_dhu,
 * finalisation; per key, the KDA stages with their per-key gate gradient),
 * for L with dL/do = dout and dL/dh_final = dht.
 *
 *   q, k, v, g, beta  device, the forward's inputs (desc as for gdn_chunk_fwd)
 *   h                 device fp32 [n_chunks][H][K][V]: the state entering every
 *                     chunk, as gdn_chunk_fwd's h slot returns it for the same
 *                     descriptor, inputs and initial state
 *   dout              device [tokens][H][V] in desc->dtype
 *   dht               device fp32 [units][H][K][V] or NULL (zero)
 *   dq, dk            device fp32 [tokens][H][K]
 *   dv                device fp32 [tokens][H][V]
 *   dg                device fp32 [tokens][H] (scalar gate) or [tokens][H][K]
 *                     (per key): dL/dg, the gradient of the raw gate
 *   dbeta             device fp32 [tokens][H]
 *   dh0               device fp32 [units][H][K][V] (dL/d initial_state) or NULL
 *   flags             0, or GDN_FLAG_REUSE_PREPARED: the workspace already holds
 *                     the backward's chunk preparation of this descriptor and
 *                     these inputs (left there by an earlier gdn_chunk_bwd or
 *                     gdn_state_grad_summary call), which is then not redone;
 *                     other bits give GDN_ERR_INVALID
 *   workspace         as for gdn_chunk_fwd (query its size with NULL); about
 *                     129 KiB per (chunk, head), 257 KiB with a per-key gate
 * Gradients are fp32 whatever the input dtype. With bf16 inputs and a scalar
 * gate the products run on fp16 operands with fp32 accumulation (the
 * forward's numeric range applies to the states and their gradients); fp32
 * inputs and the per-key gate use fp32 operands. With bf16 inputs and a
 * scalar gate, and with a per-key gate, the chunk preparation includes each
 * chunk's transfer maps of the state gradient (fp16, resp. fp32). The per-key
 * decay is taken in factors that are at most 1 for every g <= 0 (as in the
 * forward), so strong gates down to total forgetting give finite gradients.
 */
gdn_status gdn_chunk_bwd(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                         const void* beta, const float* h, const void* dout, const float* dht, float* dq,
                         float* dk, float* dv, float* dg, float* dbeta, float* dh0, int32_t flags,
                         void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * gdn_state_grad_summary - the gradient summary of every unit for a split
 * backward (kda_state_grad_ext_kernel on the state_summary.py coverage page):
 * dS_ext[u] = dL/d(entry state of u) through unit u's own outputs only, i.e.
 * with a zero gradient at the unit's exit. It is the reverse state pass of
 * gdn_chunk_bwd without the per-token gradients; the arguments are as there
 * (h from the forward over the same units, flags, the workspace of
 * gdn_chunk_bwd's size), dS_ext device fp32 [units][H][K][V]. Scalar or
 * per-key gate. The preparation it leaves in the workspace serves a following
 * gdn_chunk_bwd over the same units with GDN_FLAG_REUSE_PREPARED.
 */
gdn_status gdn_state_grad_summary(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                  const float* g, const void* beta, const float* h, const void* dout,
                                  float* dS_ext, int32_t flags, void* workspace, size_t* workspace_bytes,
                                  hipStream_t stream);

/*
 * gdn_state_merge_adjoint - the reverse state wavefront of a split backward
 * (apply_kda_state_gradient_summary on the Diff Coverage page: M^T dS + dS_ext),
 * over the segments from the last, in fp32:
 *   G_n = dS_final[b] (zero when NULL)
 *   dS_exit[b][s] = G_{s+1}             the gradient arriving at segment s's exit
 *   G_s = M[b][s]^T G_{s+1} + dS_ext[b][s]
 *   dS0[b] = G_0                        (skipped when dS0 is NULL)
 *   dS_ext  device fp32 [B][n_seg][H][K][V] (gdn_state_grad_summary)
 *   M       device fp32 [B][n_seg][H][K][K] (gdn_state_summary); the last
 *           segment's map is not read when dS_final is NULL, nor the first's
 *           when dS0 is NULL
 *   dS_exit device fp32 [B][n_seg][H][K][V]
 * gdn_chunk_bwd over the segments with dht = dS_exit then gives the unsplit
 * backward's gradients.
 */
gdn_status gdn_state_merge_adjoint(int32_t B, int32_t H, int32_t n_seg, int32_t K, int32_t V,
                                   const float* dS_ext, const float* M, const float* dS_final, float* dS_exit,
                                   float* dS0, hipStream_t stream);

/*
 * gdn_chunk_fwd_noalloc - gdn_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and errors as gdn_chunk_fwd
 * without the workspace pair: the workspace is the library's own scratch
 * array of GDN_NOALLOC_SCRATCH_BYTES, one copy per GPU, taken the first time
 * the entry point runs on that GPU and held until the process ends. The call
 * allocates nothing. The caller still passes every input and output.
 *
 *   GDN_ERR_CAPACITY  the problem needs more workspace than the scratch holds
 *                     (about 17 KiB per (chunk, head) with bf16 inputs and a
 *                     scalar gate); use gdn_chunk_fwd with a workspace
 *   GDN_ERR_INVALID   as gdn_chunk_fwd, or stream is not on the current device
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents: GDN_FLAG_REUSE_PREPARED reuses the preparation of the previous
 * call on the same GPU (same descriptor and inputs). Calls that overlap on
 * one GPU (other streams, other host threads) race on the scratch and must be
 * serialised by the caller. Nothing in the scratch needs to start at zero.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                 const float* g, const void* beta, const float* initial_state, void* o,
                                 float* final_state, const gdn_slots* slots, int32_t flags,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
