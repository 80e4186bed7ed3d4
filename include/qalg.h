/*
 * libqalg: the row-typed associative-algebra projection Y = X *_{Q_q} W on
 * AMD Instinct MI355X (gfx950).
 *
 * Source: arXiv 2609.32814, "Change the Product, Keep the Parameters:
 * Associative Algebra Layers for Transformers".
 *
 * The operation (section 4, eq 16-17; section 6.1, eq 27 and Algorithm 1):
 * X is M x K, W is K x N, both split into q equal feature groups (widths
 * s = K/q and r = N/q; group g_j of X's columns / W's rows is
 * [j*s, (j+1)*s), group g_j of W's and Y's columns is [j*r, (j+1)*r)).
 * Token row m has type i = tau[m] in [0, q) and computes
 *     y_i = x_i W_ii,      y_j = x_i W_ij + x_j W_jj   (j != i),
 * i.e. one row of the Q_q interaction table: 2q-1 of the q^2 weight blocks,
 * a fraction (2q-1)/q^2 of dense arithmetic (eq 21, eq 24).  The
 * gradients are appendix B's vector-Jacobian products (eq 31-35).
 *
 * Conventions shared by every entry point below:
 *  - Layout: row-major and packed.  X, dX: M x K (leading dimension K);
 *    W, dW: K x N (leading dimension N); Y, dY: M x N (leading dimension N).
 *    The weight bank is used exactly as stored (no repacking).  Batched
 *    entry points take E such problems packed back to back.
 *  - Element type (`dtype`): QALG_BF16 (bf16 in, bf16 out, fp32
 *    accumulation, one round-to-nearest-even rounding of each output) or
 *    QALG_F32 (fp32 throughout).
 *  - tau: device int32[M], types in [0, q).  A row whose type lies outside
 *    [0, q) belongs to no type: its Y / dX row is written as zero, it adds
 *    nothing to dW, and it is counted (see qalg_read_status).
 *  - Ownership: every pointer is device memory owned by the caller (for
 *    example allocated by PyTorch).  The library allocates nothing, keeps no
 *    pointer after a call returns, and holds no state: calls are reentrant,
 *    but concurrent calls need separate workspaces.  (qalg_forward_noalloc,
 *    for callers that cannot allocate, is the one exception: it uses a device
 *    array of the library's own and keeps that array's address per GPU.)
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) and the call returns without waiting.  Buffers must
 *    stay valid until the stream has run the work.
 *  - Workspace: `ws` is caller-owned device memory of at least
 *    qalg_workspace_bytes(q, M) (per problem; batched: E times that), 256-byte
 *    aligned.  It receives the type index of the call.
 *  - Errors are returned synchronously, before anything is enqueued, for:
 *    a NULL pointer that is needed (QALG_ERR_NULL), M < 0 or K, N <= 0 or a
 *    size above the int32 index range (QALG_ERR_DIM), q < 1, q > QALG_MAX_Q
 *    or q not dividing K and N (QALG_ERR_Q), a base pointer not 16-byte
 *    aligned or (bf16) a group width not a multiple of 8 elements
 *    (QALG_ERR_ALIGN), an unknown dtype (QALG_ERR_DTYPE), a workspace that
 *    is too small or misaligned (QALG_ERR_WORKSPACE), an unknown flag or
 *    schedule kind (QALG_ERR_ARG).  A failed launch returns QALG_ERR_HIP.
 *    M = 0 returns QALG_OK and enqueues nothing, except that qalg_backward_dw
 *    then zero-fills dW (only dW must be non-NULL in that case).
 */
#ifndef QALG_H
#define QALG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QALG_VERSION 1
#define QALG_MAX_Q 512

typedef enum qalg_status {
    QALG_OK = 0,
    QALG_ERR_NULL = 1,
    QALG_ERR_DIM = 2,
    QALG_ERR_Q = 3,
    QALG_ERR_ALIGN = 4,
    QALG_ERR_DTYPE = 5,
    QALG_ERR_WORKSPACE = 6,
    QALG_ERR_HIP = 7,
    QALG_ERR_ARG = 8
} qalg_status;

typedef enum qalg_dtype {
    QALG_F32 = 0,
    QALG_BF16 = 1
} qalg_dtype;

/* Flags for the projection entry points (bitwise or). */
enum {
    /* The workspace already holds the index of this (tau, q, M), written by
     * qalg_build_index or by an earlier call on the same stream: skip
     * rebuilding it.  Lets forward, dX and dW of one step share one index. */
    QALG_FLAG_INDEX_READY = 1,
    /* Force the register-staged tiled matrix-core kernels (neither the
     * small-M path nor the persistent forward; testing and calibration). */
    QALG_FLAG_FORCE_TILED = 2,
    /* Force the small-M weight-streaming path (bf16 forward only; testing). */
    QALG_FLAG_FORCE_SMALL_M = 4,
    /* Use the recursive law Q_2^(x)L of appendix C instead of Q_q (the law of
     * the paper's pretraining pilot): q = 2^L types and feature groups are
     * L-bit strings (bit L-1, the most significant, is the first level of
     * the recursion) and output group j of a type-i row sums x_b W_bj over
     * every group b whose bits each equal i's or j's (eq 36; section 6.1's
     * B(i, j) for this law), 2^popcount(i xor j) terms; (3/4)^L of the
     * dense MACs with equal groups.  q must be a power of two
     * (QALG_ERR_Q); q = 2 is Q_2 itself and q = 1 the plain product.
     * Accepted by qalg_forward and qalg_gated_forward (bf16; K / q a
     * multiple of 64 and N / q of 128, QALG_ERR_ALIGN otherwise; byte offsets
     * below 2^31, QALG_ERR_DIM), by qalg_backward_dx and qalg_backward_dw
     * (bf16, any shape the projection accepts: the VJPs of App B with the
     * law's supports transposed) and by qalg_attention_forward; the batched
     * forward, fp32 and the forced paths return QALG_ERR_ARG. */
    QALG_FLAG_LAW_TENSOR = 8,
    /* Tile calibration (qalg_forward, bf16, one bank): run the persistent
     * forward with 64-, 128- or 256-row output tiles instead of the height
     * chosen from the rows per type (at most one; QALG_ERR_ARG if the shape
     * cannot use it: 64 needs N / q a multiple of 256, 128 a multiple of 128
     * or of 192, and every persistent shape K / q a multiple of 64). */
    QALG_FLAG_TILE_M64 = 16,
    QALG_FLAG_TILE_M128 = 32,
    QALG_FLAG_TILE_M256 = 64,
    /* Section 5.3's second forward schedule (qalg_forward, qalg_forward_batched;
     * bf16, the complete law Q_q): the diagonal maps over all rows first,
     * D[m, g_j] = x_j W_jj for every typed row m and group j, with row tiles
     * that span the types, so that each diagonal block is read once for all
     * rows; then the type-dependent maps, X[I_i, g_i] W_ij for j != i, whose
     * epilogue adds D and rounds once (the same one-rounding result as the
     * fused schedule, up to the fp32 summation order).  Pays off when each
     * type has few rows (the fused schedule reads W_jj once per type).  D is
     * fp32 in the workspace, which must hold qalg_workspace_bytes_two_stage
     * bytes per problem (QALG_ERR_WORKSPACE otherwise); M N below 2^31
     * (QALG_ERR_DIM); with QALG_FLAG_LAW_TENSOR, the forced paths or a tile
     * flag: QALG_ERR_ARG. */
    QALG_FLAG_TWO_STAGE = 128,
    /* The few-rows forward (qalg_forward, qalg_forward_batched; bf16, the
     * complete law): one output tile spans all M rows of a problem in their
     * own order and runs the whole contraction, weight block by weight block,
     * each block's activations reaching only the rows that use it (rows of
     * type b for block b, every row for the output group's own block j,
     * eq 17); the others are zero.  Each weight column tile is read once, as
     * in the plain product, where the fused schedule re-reads W_jj once per
     * type.  For a handful of rows per type (the few-rows regime of section
     * 5.2 and 5.3); the matrix-core work is that of the dense product.  With
     * QALG_FLAG_LAW_TENSOR, QALG_FLAG_TWO_STAGE, the forced paths or a tile
     * flag: QALG_ERR_ARG. */
    QALG_FLAG_MASKED = 256
};

/* Position-type schedules for qalg_type_schedule. */
typedef enum qalg_schedule {
    /* tau(p) = p mod q: section 4's cyclic schedule 1 + ((p-1) mod q) in 0-based form. */
    QALG_SCHEDULE_CYCLIC = 0,
    /* tau(p) = floor((p mod period) / (period / q)): appendix D.5's interval
     * schedule, floor((p mod 768) / 192) for the pilot (period 768, q 4). */
    QALG_SCHEDULE_INTERVAL = 1
} qalg_schedule;

/* Human-readable name of a status code (static string; never NULL). */
const char* qalg_status_string(int status);

/* Library version (QALG_VERSION of the build). */
int qalg_version(void);

/* Bytes of workspace one problem with q types and M rows needs (0 on bad
 * arguments).  Batched calls need E times this. */
size_t qalg_workspace_bytes(int32_t q, int64_t M);

/*
 * Workspace that also lets qalg_backward_dw split contractions over several
 * workgroups: qalg_workspace_bytes(q, M) plus fp32 scratch for up to 16
 * partial sums of the K x N gradient, summed in a fixed order afterwards
 * (bitwise reproducible, one rounding).  On the register-staged path (listed
 * schedules, the recursive law, shapes the persistent gradient kernel does
 * not take) every output tile may be split; on the persistent path (cyclic
 * schedules) the diagonal blocks W_jj, whose tiles contract over all M rows
 * against M/q for the others, are cut into pieces no longer than a
 * workgroup's average share.  A smaller workspace (at least
 * qalg_workspace_bytes(q, M)) gives the result without the split (equal
 * within the fp32 summation order).  Returns 0 for invalid sizes.
 */
size_t qalg_workspace_bytes_dw(int32_t q, int64_t M, int64_t K, int64_t N);

/*
 * Workspace per problem that the two-stage forward (QALG_FLAG_TWO_STAGE) needs:
 * qalg_workspace_bytes(q, M) plus the fp32 diagonal maps (M x N).  A batched
 * call of E problems needs E times this (the E indices first, then the E
 * diagonal buffers).  0 for invalid sizes.
 */
size_t qalg_workspace_bytes_two_stage(int32_t q, int64_t M, int64_t N);

/*
 * Type schedule (section 4: a token at position p selects row i = tau(p) by a
 * fixed deterministic schedule; appendix D.5 for the interval form).
 * positions: device int64[M], each >= 0 (a negative position yields type -1,
 * which the projections treat as "no type").  tau: device int32[M], written.
 * kind: a qalg_schedule; period is used by QALG_SCHEDULE_INTERVAL only and
 * must be a positive multiple of q.
 */
qalg_status qalg_type_schedule(const int64_t* positions, int64_t M, int32_t q,
                               int32_t kind, int64_t period, int32_t* tau,
                               void* stream);

/*
 * Type index (Algorithm 1: I_i = {b : tau(p_b) = i}).  Reads tau (device
 * int32[M]) and writes into ws the per-type row counts, their running
 * offsets, the rows of each type in ascending order (type 0 first, rows with
 * an out-of-range type last), the row-tile prefix sums the tiled kernels use
 * and the count of out-of-range rows.  No sort: one counting pass and one
 * stable scatter.  The projection entry points call this themselves unless
 * QALG_FLAG_INDEX_READY is set.  Its layout is exposed for tests through
 * qalg_index_layout.
 */
qalg_status qalg_build_index(const int32_t* tau, int32_t q, int64_t M,
                             void* ws, size_t ws_bytes, void* stream);

/* Same, for E problems whose tau arrays are packed back to back (tau: E x M)
 * into E workspaces of qalg_workspace_bytes(q, M) bytes each. */
qalg_status qalg_build_index_batched(int32_t E, const int32_t* tau, int32_t q, int64_t M,
                                     void* ws, size_t ws_bytes, void* stream);

/* Offsets, in int32 elements from the start of one problem's workspace, of the
 * index arrays: [0] = out-of-range row count (1 int32), [1] = counts (q),
 * [2] = offsets (q+1), [3] = rows (M).  Returns QALG_ERR_Q / QALG_ERR_DIM on bad
 * arguments.  (Test hook: the index is internal data otherwise.) */
qalg_status qalg_index_layout(int32_t q, int64_t M, int64_t out_offsets[4]);

/*
 * Forward projection Y = X *_{Q_q} W (eq 16-17, Algorithm 1).
 * X: M x K, W: K x N, Y: M x N (overwritten; Algorithm 1 starts from Y = 0).
 * Each output tile sums both endpoint products x_i W_ij and x_j W_jj in fp32
 * registers and is rounded and stored once (section 5.3's fused schedule).
 * Small M (bf16) uses a weight-streaming kernel that reads each needed
 * weight block once (section 5.2: decode needs a matrix-vector kernel).
 */
qalg_status qalg_forward(const void* X, const void* W, const int32_t* tau, int32_t q,
                         int64_t M, int64_t K, int64_t N, void* Y,
                         int32_t dtype, void* ws, size_t ws_bytes,
                         uint32_t flags, void* stream);

/*
 * Forward projection under a graph law Q_G (section 3.1, eq 9-12): the slots
 * of the algebra are the vertices (i, i) and the directed edges (i, j) of a
 * graph on the q groups; a product of two slots vanishes unless the inner
 * indices meet and one factor is a vertex.  A row of type i then gets
 * y_i = x_i W_ii, y_j = x_i W_ij + x_j W_jj for every edge (i, j), and y_j = 0
 * for every other j (eq 27 with B(i, j) = {i, j} on edges, empty off them).
 * The complete graph is Q_q (qalg_forward).  adjacency: q device uint64 masks,
 * caller-owned, 8-byte aligned; bit j of adjacency[i] set iff the edge (i, j)
 * exists (bit i ignored).  q <= 64 (QALG_ERR_Q).  bf16 only (QALG_ERR_DTYPE);
 * K / q and N / q multiples of 8 (QALG_ERR_ALIGN); M K, K N and M N below
 * 2^31 (QALG_ERR_DIM).  Flags: QALG_FLAG_INDEX_READY only (QALG_ERR_ARG).
 * Rows of an out-of-range type get zero rows; output blocks of absent edges
 * are written as zeros.  Shapes of the persistent forward (K / q a multiple
 * of 64, N / q of 128) run it; the others run the register-staged kernel.
 */
qalg_status qalg_forward_graph(const void* X, const void* W, const int32_t* tau, int32_t q,
                               const uint64_t* adjacency, int64_t M, int64_t K, int64_t N, void* Y,
                               int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags, void* stream);

/*
 * Gradients of the graph-law projection (appendix B's VJPs with the Q_G
 * supports of section 3.1 transposed).  For a row of type i:
 *   dx_i = dy_i W_ii^T + sum over edges (i, j) of dy_j W_ij^T,
 *   dx_k = dy_k W_kk^T on an edge (i, k), and 0 for every other k != i;
 *   dW_jj sums x_j^T dy_j over the rows of type j and of every type i with an
 *         edge (i, j); dW_bj (b != j) sums x_b^T dy_j over the rows of type b
 *         on an edge (b, j), and is 0 off the edges.
 * Operands, adjacency, errors and flags as in qalg_forward_graph, and as in
 * qalg_backward_dx / qalg_backward_dw (dX and dW overwritten; rows of an
 * out-of-range type get zero dX rows and add nothing to dW; a workspace of
 * qalg_workspace_bytes_dw bytes lets dW split its contraction).  Register-
 * staged kernels; each output element has one owner (bitwise reproducible).
 */
qalg_status qalg_backward_dx_graph(const void* dY, const void* W, const int32_t* tau, int32_t q,
                                   const uint64_t* adjacency, int64_t M, int64_t K, int64_t N, void* dX,
                                   int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags, void* stream);
qalg_status qalg_backward_dw_graph(const void* X, const void* dY, const int32_t* tau, int32_t q,
                                   const uint64_t* adjacency, int64_t M, int64_t K, int64_t N, void* dW,
                                   int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags, void* stream);

/*
 * The complete-graph law Q_q on groups of unequal widths (eq 18): input group
 * g spans in_widths[g] columns of X (rows of W), output group g spans
 * out_widths[g] columns of Y and W; a row of type i gets y_i = x_i W_ii and
 * y_j = x_i W_ij + x_j W_jj, the blocks now rectangular.  Forward, dX and dW
 * with the operands, overwrite and zero-row rules of qalg_forward,
 * qalg_backward_dx and qalg_backward_dw.  in_widths, out_widths: host arrays
 * of q int64, read during the call only; every width a positive multiple of
 * 8 (QALG_ERR_DIM / QALG_ERR_ALIGN), summing to K and N (QALG_ERR_DIM).
 * q <= 64 (QALG_ERR_Q); bf16 only (QALG_ERR_DTYPE); M K, K N and M N below
 * 2^31 (QALG_ERR_DIM); flags: QALG_FLAG_INDEX_READY only (QALG_ERR_ARG).  A
 * workspace of qalg_workspace_bytes_dw bytes lets the register-staged dW
 * split its contraction.  Shapes whose groups fill whole tiles run the
 * persistent kernels: the forward when every out_widths[g] is a multiple of
 * 256 and every in_widths[g] of 64 with at least 128 rows per type; dX when
 * every in_widths[g] is a multiple of 128, 192 or 256 and every out_widths[g]
 * of 64 with at least 128 rows per type; dW when every in_widths[g] is a
 * multiple of 192 or 256 and every out_widths[g] of 128, 192 or 256 with
 * M >= 32 q (M K, K N and M N below 2^30 for the gradients).  Other shapes
 * run the register-staged kernels.  Each output element has one owner.
 */
qalg_status qalg_forward_widths(const void* X, const void* W, const int32_t* tau, int32_t q,
                                const int64_t* in_widths, const int64_t* out_widths, int64_t M, int64_t K,
                                int64_t N, void* Y, int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                                void* stream);
qalg_status qalg_backward_dx_widths(const void* dY, const void* W, const int32_t* tau, int32_t q,
                                    const int64_t* in_widths, const int64_t* out_widths, int64_t M, int64_t K,
                                    int64_t N, void* dX, int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                                    void* stream);
qalg_status qalg_backward_dw_widths(const void* X, const void* dY, const int32_t* tau, int32_t q,
                                    const int64_t* in_widths, const int64_t* out_widths, int64_t M, int64_t K,
                                    int64_t N, void* dW, int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                                    void* stream);

/*
 * Activation gradient (appendix B, eq 31-32): for a row of type i,
 *   dx_i = sum_j dy_j W_ij^T  and  dx_j = dy_j W_jj^T  (j != i).
 * dY: M x N, W: K x N, dX: M x K (overwritten).
 */
qalg_status qalg_backward_dx(const void* dY, const void* W, const int32_t* tau, int32_t q,
                             int64_t M, int64_t K, int64_t N, void* dX,
                             int32_t dtype, void* ws, size_t ws_bytes,
                             uint32_t flags, void* stream);

/*
 * Weight gradient (appendix B, eq 33-35), summed over all rows:
 *   dW_jj = sum over every row of x_j^T dy_j,
 *   dW_ij = sum over the rows of type i of x_i^T dy_j   (i != j).
 * X: M x K, dY: M x N, dW: K x N (overwritten; a block no row reaches is
 * written as zero).  Each dW element has one owner; the result does not
 * depend on scheduling (bitwise reproducible).
 */
qalg_status qalg_backward_dw(const void* X, const void* dY, const int32_t* tau, int32_t q,
                             int64_t M, int64_t K, int64_t N, void* dW,
                             int32_t dtype, void* ws, size_t ws_bytes,
                             uint32_t flags, void* stream);

/*
 * E independent forward projections, one weight bank each (the per-expert
 * projections of a mixture-of-experts layer, section 7.1: an expert's M counts
 * the tokens routed to it).  X: E x M x K, W: E x K x N, tau: E x M,
 * Y: E x M x N, all packed; ws: E x qalg_workspace_bytes(q, M).
 */
qalg_status qalg_forward_batched(int32_t E, const void* X, const void* W, const int32_t* tau,
                                 int32_t q, int64_t M, int64_t K, int64_t N, void* Y,
                                 int32_t dtype, void* ws, size_t ws_bytes,
                                 uint32_t flags, void* stream);

/*
 * Gate/up half of a gated (SwiGLU) FFN, fused: H = silu(X *_{Q_q} W_gate) *
 * (X *_{Q_q} W_up) elementwise, silu(z) = z * sigmoid(z).  Section 4: a gated
 * FFN has two D x F weights that follow the same row law as any projection
 * (gates and pointwise activations keep their usual definitions); the pilot's
 * FFN is a bias-free SwiGLU (appendix D); table 9 merges gate and up.
 * Both products accumulate in fp32; the activation is applied in fp32 and H is
 * rounded once (RNE).  bf16 only.
 * X: M x K.  Wgu: K x 2F, the merged bank built by qalg_merge_gate_up.  H: M x F
 * (overwritten; rows of an out-of-range type are written as zero).
 * Requires F / q to be a multiple of 128 and K / q a multiple of 64
 * (QALG_ERR_ALIGN otherwise), and M*K, K*2F, M*2F below 2^31 (QALG_ERR_DIM).
 * Flags: QALG_FLAG_INDEX_READY and QALG_FLAG_LAW_TENSOR.
 */
qalg_status qalg_gated_forward(const void* X, const void* Wgu, const int32_t* tau, int32_t q,
                               int64_t M, int64_t K, int64_t F, void* H,
                               int32_t dtype, void* ws, size_t ws_bytes,
                               uint32_t flags, void* stream);

/*
 * The gated forward of a training step, which needs the pre-activations again
 * for the SwiGLU VJP (section 6.2 counts the training step's products; the
 * activation keeps its usual definition): GU (M x 2F, the merged layout of
 * qalg_merge_gate_up) receives the gate and up products rounded once to bf16,
 * and H = silu(gate) * up is computed from those rounded values, i.e. exactly
 * what qalg_forward on the merged bank followed by qalg_swiglu_forward gives,
 * in one launch.  Arguments, requirements and flags as qalg_gated_forward;
 * GU is caller-owned device memory (non-null when M > 0, 16-byte aligned,
 * overwritten; rows of an out-of-range type are written as zero).
 */
qalg_status qalg_gated_forward_keep(const void* X, const void* Wgu, const int32_t* tau, int32_t q,
                                    int64_t M, int64_t K, int64_t F, void* H, void* GU,
                                    int32_t dtype, void* ws, size_t ws_bytes,
                                    uint32_t flags, void* stream);

/*
 * Merged gate/up bank for qalg_gated_forward (a layout copy, done once per
 * weight update): Wg, Wu: K x F; Wgu: K x 2F.  Output group j's columns
 * j*2r .. j*2r + 2r - 1 (r = F / q) come in pieces of 256: piece t holds, for
 * output columns c0 = j*r + 128 t .. c0 + 127, the gate columns c0 .. c0+63,
 * the up columns c0 .. c0+63, the gate columns c0+64 .. c0+127, then the up
 * columns c0+64 .. c0+127.  bf16 only; F / q must be a multiple of 128.
 */
qalg_status qalg_merge_gate_up(const void* Wg, const void* Wu, int32_t q, int64_t K, int64_t F,
                               void* Wgu, int32_t dtype, void* stream);

/*
 * Inverse of qalg_merge_gate_up: Wgu (K x 2F, merged) -> Wg, Wu (K x F each),
 * e.g. to read the merged gradient from qalg_backward_dw as two banks.  Same
 * requirements and errors as the merge.
 */
qalg_status qalg_split_gate_up(const void* Wgu, int32_t q, int64_t K, int64_t F, void* Wg, void* Wu,
                               int32_t dtype, void* stream);

/*
 * Pointwise SwiGLU gate on merged pre-activations, for the training step of a
 * gated FFN (section 4: gates and pointwise activations keep their usual
 * definitions; appendix D: bias-free SwiGLU, silu(z) = z * sigmoid(z)).
 * GU: M x 2F, the merged [gate | up] pre-activations, i.e. qalg_forward of X
 * with the merged bank Wgu and N = 2F (merging permutes columns within each
 * output group, so that product is the merged pair of row-typed products).
 * H: M x F (overwritten), H = silu(gate) * up, computed in fp32 and rounded
 * once (RNE).  bf16 only; F / q must be a multiple of 128 (QALG_ERR_ALIGN);
 * M = 0 returns QALG_OK without a launch.
 */
qalg_status qalg_swiglu_forward(const void* GU, int32_t q, int64_t M, int64_t F, void* H,
                                int32_t dtype, void* stream);

/*
 * Its vector-Jacobian product (chain rule through silu(gate) * up):
 * dgate = dH * up * silu'(gate), dup = dH * silu(gate), silu'(z) =
 * sigmoid(z) (1 + z (1 - sigmoid(z))).  GU: M x 2F merged (as above), dH:
 * M x F, dGU: M x 2F (overwritten, merged layout: the input of
 * qalg_backward_dx / qalg_backward_dw with the merged bank and N = 2F, which
 * give dX and the merged dWgu, App B eq 31-35).  fp32 arithmetic, one RNE
 * rounding per output.  Same requirements as qalg_swiglu_forward.
 */
qalg_status qalg_swiglu_backward(const void* GU, const void* dH, int32_t q, int64_t M, int64_t F,
                                 void* dGU, int32_t dtype, void* stream);

/*
 * Causal attention with the algebraic score, forward (appendix G, Algorithm 2
 * steps 3-7; one sequence per head, positions 0 .. S-1, types p mod q).  A
 * query of type i and a key of type j compare only the feature groups F(i, j)
 * of the head ({i} if i == j, else {i, j}, eq 38; with QALG_FLAG_LAW_TENSOR the
 * recursive law's groups, eq 42): r = sum over F of <Q^(a), K^(a)> (eq 39),
 * scaled by 1 / sqrt(|F| d / q) (eq 41), masked to keys at or before the query
 * (eq 43), softmaxed, O = P V over all d features (eq 44).
 * Q, O: Hq x S x d; K, V: Hkv x S x d (Hkv divides Hq; query head h uses
 * key/value head h / (Hq / Hkv), the GQA convention); all bf16, packed,
 * 16-byte aligned, caller-owned device memory.  fp32 scores, softmax
 * statistics and accumulation; P is rounded to bf16 for the value product and
 * O once at the end.  d must be 64 or 128 and S * d * 2 below 2^31
 * (QALG_ERR_DIM), q must divide d
 * (QALG_ERR_Q) with d / q a multiple of 16 (QALG_ERR_ALIGN); the recursive law
 * needs q = 2^L (QALG_ERR_Q).  Flags: QALG_FLAG_LAW_TENSOR only.  S = 0 returns
 * QALG_OK without a launch.
 */
qalg_status qalg_attention_forward(const void* Q, const void* K, const void* V, int32_t Hq, int32_t Hkv,
                                   int64_t S, int32_t d, int32_t q, void* O, int32_t dtype, uint32_t flags,
                                   void* stream);

/*
 * The same for a chunk of S rows whose first row sits at absolute position
 * first_position (>= 0, QALG_ERR_DIM otherwise): row s has position
 * first_position + s and type (first_position + s) mod q (section 4's cyclic
 * schedule at that offset, so the type of row 0 is first_position mod q and
 * the pairs F(i, j) move with it); the mask is the chunk's own causal order.
 * Everything else as qalg_attention_forward (which is first_position = 0).
 */
qalg_status qalg_attention_forward_at(const void* Q, const void* K, const void* V, int32_t Hq, int32_t Hkv,
                                      int64_t S, int32_t d, int32_t q, int64_t first_position, void* O,
                                      int32_t dtype, uint32_t flags, void* stream);

/*
 * The forward for training: qalg_attention_forward_at that also writes lse
 * (Hq x S fp32, caller-owned device memory, 4-byte aligned), the natural log
 * of each query's softmax denominator over the scaled scores (log of the sum
 * over the allowed keys of exp(s)), which the backward reuses instead of
 * recomputing the row statistics.  Errors as qalg_attention_forward_at, plus
 * QALG_ERR_NULL for a null lse.
 */
qalg_status qalg_attention_forward_train(const void* Q, const void* K, const void* V, int32_t Hq, int32_t Hkv,
                                         int64_t S, int32_t d, int32_t q, int64_t first_position, void* O, float* lse,
                                         int32_t dtype, uint32_t flags, void* stream);

/*
 * Gradients of the algebraic-score attention (appendix G, Algorithm 2 step 9:
 * backpropagation through steps 3-7).  Inputs: Q, K, V, the forward's O and
 * lse (qalg_attention_forward_train, same first_position, q and flags), and
 * dO (Hq x S x d), the gradient of the loss with respect to O.  With P the
 * softmax rows, dP_pu = <dO_p, V_u> and D_p = <dO_p, O_p>:
 *   dS_pu = P_pu (dP_pu - D_p) / sqrt(|F(i, j)| d / q)
 *   dQ_p^(a) = sum_u dS_pu K_u^(a),  dK_u^(a) = sum_p dS_pu Q_p^(a)
 *     over the groups a of F(i, j) only (the score reads only those, eq 39),
 *   dV_u = sum_p P_pu dO_p (the dense value sum).
 * A key/value head's dK and dV sum over the Hq / Hkv query heads that read it.
 * Outputs dQ (Hq x S x d), dK, dV (Hkv x S x d), bf16, overwritten.  All
 * tensors bf16 (lse fp32), packed, 16-byte aligned (lse 4-byte), caller-owned
 * device memory.  fp32 scores, statistics and sums; P and dS are rounded to
 * bf16 for the matrix products, each output once at the end; every output
 * element is summed in a fixed order (no atomics): bitwise reproducible.
 * ws: caller-owned device scratch of at least
 * qalg_attention_backward_workspace_bytes(Hq, Hkv, S, d, q) bytes, 16-byte
 * aligned (per-query lse and D, grouped by type; with an even number of query
 * heads per key/value head, also fp32 dK and dV of two shares of those heads,
 * added in a fixed order at the end).  Errors as
 * qalg_attention_forward_at, plus QALG_ERR_NULL for a null pointer (ws
 * included) and QALG_ERR_WORKSPACE for a small or misaligned ws.  S = 0
 * returns QALG_OK without a launch.
 */
size_t qalg_attention_backward_workspace_bytes(int32_t Hq, int32_t Hkv, int64_t S, int32_t d, int32_t q);
qalg_status qalg_attention_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                    const float* lse, int32_t Hq, int32_t Hkv, int64_t S, int32_t d, int32_t q,
                                    int64_t first_position, void* dQ, void* dK, void* dV, int32_t dtype, void* ws,
                                    size_t ws_bytes, uint32_t flags, void* stream);

/*
 * Cached decoding with the algebraic score (appendix G, Algorithm 3; G.2's
 * cache): one new query row per sequence against that sequence's full-key
 * cache.  B sequences; Qn: B x Hq x d, the new rows' queries; Kc, Vc:
 * B x Hkv x N x d, each sequence's cache of N slots holding full keys and
 * values (query head h reads key/value head h / (Hq / Hkv), GQA); q_pos:
 * int64[B], the absolute position p of each new row; key_pos: int64[B x N],
 * the absolute position u of each cached slot, negative for an empty slot.
 * All device memory, caller-owned, bf16 / int64, packed; Qn, Kc, Vc, O 16-byte
 * and the positions 8-byte aligned.  Types come from positions through the
 * schedule `kind` (a qalg_schedule; `period` for the interval form, as in
 * qalg_type_schedule): i = tau(p), j = tau(u).  For each slot with
 * 0 <= u <= p the score sums <Q^(a), K_u^(a)> over the groups a of F(i, j)
 * (eq 38-39; eq 42 with QALG_FLAG_LAW_TENSOR) scaled by 1 / sqrt(|F| d / q)
 * (eq 41); O (B x Hq x d, overwritten) is the softmax-weighted sum of those
 * slots' values over all d features (Algorithm 3's last step).  A row with no
 * such slot (or p < 0) is written as zeros.  Only the F(i, j) groups of each
 * cached key are read (eq 57's cost).  fp32 scores, softmax and sums; O rounded
 * once.  ws: caller-owned device memory of at least
 * qalg_attention_decode_workspace_bytes(B, Hq, N, d) bytes, 16-byte aligned
 * (fp32 partial results of slot chunks, combined in a fixed order: bitwise
 * reproducible).  Errors: d not 64 or 128, Hkv not dividing Hq, Hq / Hkv > 8,
 * N < 1 or N > 262144, B or Hkv > 65535 (QALG_ERR_DIM); q not dividing d or the
 * recursive law with q not a power of two (QALG_ERR_Q); d / q not a multiple of
 * 8 or misaligned pointers (QALG_ERR_ALIGN); an unknown schedule or flag
 * (QALG_ERR_ARG); a small workspace (QALG_ERR_WORKSPACE).  B = 0 enqueues nothing.
 */
size_t qalg_attention_decode_workspace_bytes(int32_t B, int32_t Hq, int64_t N, int32_t d);
qalg_status qalg_attention_decode(const void* Qn, const void* Kc, const void* Vc, const int64_t* q_pos,
                                  const int64_t* key_pos, int32_t B, int32_t Hq, int32_t Hkv, int64_t N, int32_t d,
                                  int32_t q, int32_t kind, int64_t period, void* O, int32_t dtype, void* ws,
                                  size_t ws_bytes, uint32_t flags, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * qalg_forward with no workspace argument.  The type index it builds goes to
 * a device array owned by the library, QALG_NOALLOC_SCRATCH_BYTES on each GPU
 * it runs on, reserved with the library's code object and held until the
 * process ends; the call allocates and frees nothing.  Arguments, results and
 * errors as qalg_forward, plus: qalg_workspace_bytes(q, M) must not exceed
 * QALG_NOALLOC_SCRATCH_BYTES (QALG_ERR_WORKSPACE; about 1.04 M rows at small
 * q), and QALG_FLAG_INDEX_READY is refused (QALG_ERR_ARG): every call on a GPU
 * shares that GPU's array, so the index is rebuilt by each call.  Calls that
 * overlap on one GPU (two streams, or two host threads) race on the array and
 * must be ordered by the caller; calls on one stream are ordered already.
 * The GPU is the stream's device (the current device for the NULL stream).
 */
#define QALG_NOALLOC_SCRATCH_BYTES (4u << 20)
qalg_status qalg_forward_noalloc(const void* X, const void* W, const int32_t* tau, int32_t q,
                                 int64_t M, int64_t K, int64_t N, void* Y,
                                 int32_t dtype, uint32_t flags, void* stream);

/*
 * Number of rows with an out-of-range type seen by the last index build in
 * ws (summed over the E problems of a batched workspace; E = 1 otherwise).
 * Synchronises `stream`.
 */
qalg_status qalg_read_status(const void* ws, int32_t E, int32_t q, int64_t M,
                             void* stream, int64_t* bad_tau_rows);

#ifdef __cplusplus
}
#endif

#endif /* QALG_H */
