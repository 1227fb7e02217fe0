/*
 * tpmlp.h -- C ABI of the MI355X (gfx950) tensor-parallel MLP library.
 *
 * The library computes the Megatron tensor-parallel MLP forward pass
 *
 *     Y = sum_{i<n} GeLU_tanh(X A_i) B_i
 *
 * where A (D x F) is split by columns into n contiguous blocks A_i and B
 * (F x D) by the matching rows into B_i.  The operations and their names
 * follow "Tensor-Parallel MLP (Megatron)" (scratchllm.com), section
 * "What to implement": gelu(x), shard_mlp(A, B, n) and tp_mlp(X, shards).
 * The n partial outputs are summed on the GPU inside one fp32 accumulator
 * (the simulated all-reduce of section "The split", bullet 3).
 *
 * Conventions shared by every entry point
 *   - Matrices are dense, row-major, with no padding between rows.
 *   - Every data pointer is a device pointer on the current HIP device,
 *     16-byte aligned.  The caller allocates and owns all device memory
 *     (inputs, outputs, the packed weight buffer and the workspace); the
 *     library never allocates device memory.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Work is enqueued asynchronously on it; the caller
 *     synchronises.  Faults inside a kernel surface at that synchronisation,
 *     not as a return value.
 *   - Every function returns a tpmlp_status (or a size / count).  Arguments
 *     are validated before any HIP call, so argument errors are reported
 *     without touching the GPU.  No C++ exception crosses this boundary and
 *     nothing aborts.
 *   - dtype: TPMLP_F32 (IEEE binary32) or TPMLP_BF16 (bfloat16).  Products
 *     always accumulate in fp32.
 *   - Calls on different streams may overlap only when they use different
 *     workspaces.
 */
#ifndef TPMLP_H
#define TPMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TPMLP_F32 = 0,
    TPMLP_BF16 = 1
} tpmlp_dtype;

typedef enum {
    TPMLP_OK = 0,
    TPMLP_ERR_NULL = 1,          /* a required pointer is NULL                         */
    TPMLP_ERR_SHAPE = 2,         /* a size is out of range (negative, zero where a
                                    positive size is required, n > F, shard index
                                    outside [0, n), or too large for the kernels)    */
    TPMLP_ERR_INDIVISIBLE = 3,   /* F is not divisible by n                            */
    TPMLP_ERR_DTYPE = 4,         /* unknown dtype or a dtype combination not offered   */
    TPMLP_ERR_WORKSPACE = 5,     /* packed buffer or workspace missing or too small    */
    TPMLP_ERR_ALIGN = 6,         /* a device pointer is not 16-byte aligned            */
    TPMLP_ERR_HIP = 7            /* the HIP runtime reported an error                  */
} tpmlp_status;

/* Opaque host-side descriptor of a sharded weight set: D, F, n, dtype and the
 * device address of the packed weights.  Created by tpmlp_shard, freed by
 * tpmlp_shards_destroy.  Immutable after creation except for the workspace
 * bound with tpmlp_set_workspace. */
typedef struct tpmlp_shards tpmlp_shards;

/* Human-readable name of a status code (static storage, never NULL). */
const char* tpmlp_status_string(int status);

/* Library version string, e.g. "tpmlp 0.1 gfx950". */
const char* tpmlp_version(void);

/*
 * tpmlp_gelu -- y[k] = GeLU_tanh(x[k]) for k < count.
 * "Tensor-Parallel MLP (Megatron)", section "GeLU": one half of x times
 * (1 + tanh u) with u = sqrt(2/pi) (x + 0.044715 x^3), entry by entry.
 *   x, y   device arrays of `count` elements of `dtype`; x == y (in place) is
 *          allowed, other overlaps are not.
 *   count  number of elements; 0 is a no-op, negative is TPMLP_ERR_SHAPE.
 * Evaluated in fp32 (bf16 inputs are widened, the result rounded to nearest
 * even).
 */
tpmlp_status tpmlp_gelu(const void* x, void* y, int64_t count, int dtype, void* stream);

/*
 * Bytes of the packed weight buffer tpmlp_shard needs for (D, F, n, dtype):
 * four D x F matrices and F floats, each segment rounded up to 256 bytes;
 * 0 if the arguments are invalid.
 */
size_t tpmlp_shard_bytes(int64_t D, int64_t F, int n, int dtype);

/*
 * tpmlp_shard -- split A and B into n pairs (A_i, B_i) and pack them.
 * "Tensor-Parallel MLP (Megatron)", sections "The split" and "Requirements":
 * pair i holds columns iF/n .. (i+1)F/n - 1 of A and the same range of
 * rows of B; F must be divisible by n ("What to implement").
 *   A       device, D x F row-major, `dtype`.
 *   B       device, F x D row-major, `dtype`.
 *   packed  device buffer of at least tpmlp_shard_bytes(D, F, n, dtype)
 *           bytes, owned by the caller, which must keep it alive and
 *           unmodified while the returned descriptor is in use.  The pairs are
 *           stored K-contiguous for the forward's matrix-core GEMMs (A_i
 *           transposed to F/n x D, B transposed to D x F), with the column
 *           sums of A, followed by copies of A and B as given, which are the
 *           K-contiguous operands of the backward's dX and dS GEMMs.  A and B
 *           may be released once the work enqueued on `stream` has completed.
 *   out     receives a new host descriptor (set to NULL on error).
 * Errors: TPMLP_ERR_NULL, TPMLP_ERR_SHAPE (D <= 0, F <= 0, n <= 0, n > F,
 * a dimension above 2^21), TPMLP_ERR_INDIVISIBLE
 * (F % n != 0), TPMLP_ERR_DTYPE, TPMLP_ERR_WORKSPACE (packed_bytes too
 * small), TPMLP_ERR_ALIGN, TPMLP_ERR_HIP.
 */
tpmlp_status tpmlp_shard(const void* A, const void* B, int64_t D, int64_t F, int n, int dtype,
                         void* packed, size_t packed_bytes, tpmlp_shards** out, void* stream);

/* Number of shards n of a descriptor (0 if s is NULL). */
int tpmlp_shard_count(const tpmlp_shards* s);

/* Sizes of a descriptor; any output pointer may be NULL. */
tpmlp_status tpmlp_shard_info(const tpmlp_shards* s, int64_t* D, int64_t* F, int* n, int* dtype);

/*
 * tpmlp_shard_unpack -- write pair i back in the page's layout:
 * A_i (D x F/n row-major) and B_i (F/n x D row-major), both `dtype`, device.
 * Either output may be NULL to skip it.  Bit-exact copy of the inputs given
 * to tpmlp_shard.  Errors: TPMLP_ERR_NULL (s), TPMLP_ERR_SHAPE (i outside
 * [0, n)), TPMLP_ERR_ALIGN, TPMLP_ERR_HIP.
 */
tpmlp_status tpmlp_shard_unpack(const tpmlp_shards* s, int i, void* A_i, void* B_i, void* stream);

/* Frees the host descriptor only; the packed buffer belongs to the caller. */
void tpmlp_shards_destroy(tpmlp_shards* s);

/* Option flags for the forward workspace size and tpmlp_forward_ex. */
enum {
    TPMLP_OPT_LAYERNORM = 1,       /* normalise each row of X first (no affine)       */
    TPMLP_OPT_LAYERNORM_AFTER = 2  /* normalise each row of residual + Y last          */
};

/*
 * Bytes of device workspace a forward pass over M rows needs: the
 * intermediate H = GeLU(X A_i) for every shard (M x F, or M x F/n for a
 * single shard, in the weights' dtype) plus, with TPMLP_OPT_LAYERNORM, two
 * fp32 per-row statistics, plus, with TPMLP_OPT_LAYERNORM_AFTER, the
 * M x D fp32 sum that is normalised.  Nothing else: the shard sum never
 * leaves the second GEMM's accumulators.  Returns 0 for invalid arguments.
 * `single_shard` != 0 sizes it for a forward restricted to one shard.
 */
size_t tpmlp_forward_workspace_bytes(const tpmlp_shards* s, int64_t M, int flags, int single_shard);

/*
 * Bind a caller-owned device workspace to the descriptor for tpmlp_forward.
 * ws may be NULL with bytes 0 to unbind.  Errors: TPMLP_ERR_NULL (s),
 * TPMLP_ERR_ALIGN.
 */
tpmlp_status tpmlp_set_workspace(tpmlp_shards* s, void* ws, size_t bytes);

/*
 * tpmlp_forward -- Y = sum_i GeLU_tanh(X A_i) B_i.
 * "Tensor-Parallel MLP (Megatron)", section "The split": each shard's
 * intermediate H_i = GeLU(X A_i) (bullet 1), its partial Y_i = H_i B_i of
 * the full output shape (bullet 2), and the sum of the partials (bullet 3);
 * "Requirements": the result equals the unsplit GeLU(X A) B.
 *   X   device, M x D row-major, the descriptor's dtype.
 *   M   number of token rows; 0 is a no-op, negative is TPMLP_ERR_SHAPE.
 *   s   descriptor from tpmlp_shard with a workspace of at least
 *       tpmlp_forward_workspace_bytes(s, M, 0, 0) bytes bound.
 *   Y   device, M x D row-major, the descriptor's dtype; must not overlap X.
 * The shard sum is formed in one fp32 accumulator per output element and
 * rounded once to Y's dtype.
 */
tpmlp_status tpmlp_forward(const void* X, int64_t M, const tpmlp_shards* s, void* Y, void* stream);

/* Options of tpmlp_forward_ex.  Zero-initialise, then set what is needed. */
typedef struct {
    int flags;                 /* 0, TPMLP_OPT_LAYERNORM or TPMLP_OPT_LAYERNORM_AFTER       */
    float ln_eps;              /* LayerNorm epsilon; 0 selects 1e-5                         */
    int y_dtype;               /* output dtype; -1 selects the descriptor's dtype            */
    const void* residual;      /* optional M x D, X's dtype: added once after the shard sum  */
    int shard_index;           /* -1: all shards (the sum); i in [0, n): partial Y_i only    */
    void* workspace;           /* optional: overrides the bound workspace                    */
    size_t workspace_bytes;
    void* const* events;       /* optional: 4 hipEvent_t recorded on the stream before the
                                  LayerNorm statistics, before the first GEMM, between the
                                  GEMMs and after the last kernel (the second GEMM, or the
                                  final LayerNorm) (NULL entries skipped)                     */
    void* save_preact;         /* optional M x F (M x F/n with shard_index), weights' dtype:
                                  receives the pre-activation S = X A (after the LayerNorm
                                  correction) for tpmlp_backward                              */
    void* save_act;            /* optional M x F (M x F/n with shard_index), weights' dtype:
                                  receives H = GeLU(S), the activation the second GEMM
                                  reads, for tpmlp_backward.  GEMM1 writes H here instead
                                  of into the workspace, so keeping it costs nothing.
                                  Must not overlap save_preact, X, Y or the workspace.     */
} tpmlp_opts;

/* Fills *o with the defaults described above. */
void tpmlp_opts_init(tpmlp_opts* o);

/*
 * tpmlp_forward_ex -- tpmlp_forward with options.
 * With TPMLP_OPT_LAYERNORM and a residual this is the FFN half of the Post-LN
 * block of "LLM Lab Notes 06: Building a Megatron-Style Transformer Block
 * from Scratch", section 2, markers 5 to 7: out = x + TP-MLP(LayerNorm(x)),
 * LayerNorm over each row without affine parameters (mean and biased
 * variance in fp32), the residual x un-normalised and added once.
 * shard_index = i returns only GPU i's partial Y_i of section "The split",
 * bullet 2 (with a residual, the residual is added to that partial).
 * With TPMLP_OPT_LAYERNORM_AFTER the Norm moves after the residual, the order
 * of the original Transformer that the note on markers 2 and 5 of the same
 * section describes (and section 5, takeaway 2, contrasts with Pre-LN):
 * out = LayerNorm(residual + sum_i GeLU(X A_i) B_i), with X un-normalised;
 * the sum is kept in fp32 and rounded once, after the Norm.  It cannot be
 * combined with TPMLP_OPT_LAYERNORM or with shard_index >= 0 (the Norm
 * needs the whole sum): TPMLP_ERR_SHAPE.
 * y_dtype may be TPMLP_F32 for bf16 weights (fp32 output); a bf16 output for
 * fp32 weights is TPMLP_ERR_DTYPE.
 */
tpmlp_status tpmlp_forward_ex(const void* X, int64_t M, const tpmlp_shards* s, void* Y,
                              const tpmlp_opts* opts, void* stream);

/* Size of the library's own per-device scratch array used by
 * tpmlp_forward_noalloc: 64 MiB. */
#define TPMLP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * tpmlp_forward_noalloc -- tpmlp_forward_ex for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It computes exactly what
 * tpmlp_forward_ex computes with the same arguments, with the same kernels,
 * but its workspace is a fixed array of TPMLP_NOALLOC_SCRATCH_BYTES in the
 * library's device memory (one per GPU, held until the process ends), so
 * neither the caller nor the library allocates anything.  The caller still
 * passes X, Y (and any residual or save_preact buffer).
 *   opts  as for tpmlp_forward_ex (NULL for the defaults); opts->workspace
 *         must be NULL (TPMLP_ERR_WORKSPACE otherwise).
 * A forward whose workspace (tpmlp_forward_workspace_bytes for these M,
 * flags and shard_index) exceeds TPMLP_NOALLOC_SCRATCH_BYTES returns
 * TPMLP_ERR_WORKSPACE before any HIP call (at D = 1024, F = 4096 every
 * option fits up to M = 4096 rows).  All calls on one GPU share that GPU's array, which
 * keeps the last call's contents: calls that may overlap on one GPU (on
 * different streams, or from different threads) race and must be
 * serialised by the caller.  Errors: those of tpmlp_forward_ex, and
 * TPMLP_ERR_HIP if the array's device address cannot be obtained.
 */
tpmlp_status tpmlp_forward_noalloc(const void* X, int64_t M, const tpmlp_shards* s, void* Y,
                                   const tpmlp_opts* opts, void* stream);

/*
 * Bytes of device workspace tpmlp_backward needs for M rows: three M x F
 * intermediates in the weights' dtype (S = X A, H = GeLU(S) and dS; S and
 * H are not written when the caller passes them), plus the split-K scratch
 * of its GEMMs.  No operand is copied or transposed:
 * the GEMMs read X, dY, dS, H and the packed weights where they lie.  Returns 0 for
 * invalid arguments.
 */
size_t tpmlp_backward_workspace_bytes(const tpmlp_shards* s, int64_t M);

/*
 * tpmlp_backward -- gradients of the TP-MLP for a loss L, given dY = dL/dY.
 * With S_i = X A_i and H_i = GeLU_tanh(S_i) ("Tensor-Parallel MLP
 * (Megatron)", section "The split", bullets 1 and 2), the chain rule gives
 *   dB_i = H_i^T dY,  dS_i = (dY B_i^T) * GeLU'(S_i),  dA_i = X^T dS_i,
 *   dX = sum_i dS_i A_i^T,
 * the last sum being the backward all-reduce of "LLM Lab Notes 06", section
 * 2, marker 1 and the ledger of section 3 (formed here in one fp32
 * accumulator, like the forward's).  S, H and dS are held in the weights'
 * dtype between the GEMMs.
 *   X, dY  device, M x D row-major, the descriptor's dtype.
 *   M      rows; 0 gives dX nothing to write and zero dA, dB.
 *   s      descriptor from tpmlp_shard (its packed weights are read only).
 *   preact optional M x F pre-activation S = X A saved by a forward without
 *          LayerNorm over all shards (tpmlp_opts.save_preact); NULL recomputes
 *          it (one more GEMM of 2 M D F).
 *   act    optional M x F activation H = GeLU(S) saved by the same forward
 *          (tpmlp_opts.save_act): the H whose product with B gave Y.  NULL
 *          recomputes it from the bf16 S in the epilogue of the dS GEMM (one
 *          more M x F store and a GeLU per element).
 *   dX     device, M x D, the descriptor's dtype.
 *   dA     device, D x F: dA_i in columns iF/n .. (i+1)F/n - 1 (A's layout).
 *   dB     device, F x D: dB_i in rows iF/n .. (i+1)F/n - 1 (B's layout).
 *   workspace  device, at least tpmlp_backward_workspace_bytes(s, M) bytes,
 *          16-byte aligned, caller-owned; contents are scratch.  That size
 *          is 0 for M = 0, and the workspace may then be NULL.
 * Outputs must not overlap each other, the inputs or the workspace.
 * Errors: TPMLP_ERR_NULL, TPMLP_ERR_SHAPE (M < 0 or too large),
 * TPMLP_ERR_ALIGN, TPMLP_ERR_WORKSPACE, TPMLP_ERR_HIP; all but the last are
 * returned before any HIP call.
 */
tpmlp_status tpmlp_backward(const void* X, const void* dY, int64_t M, const tpmlp_shards* s, const void* preact,
                            const void* act, void* dX, void* dA, void* dB, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * The attention half of the block (head-sharded self-attention).
 *
 * "LLM Lab Notes 06: Building a Megatron-Style Transformer Block from
 * Scratch", section 2, markers 2 to 4, with the attention of "Tensor
 * Parallelism in Megatron", section 4: for every sequence of `seq` tokens
 * and every head j (H heads of width d = h / H, rank i of p owning heads
 * i H/p .. (i+1) H/p - 1),
 *     x_n = LayerNorm(x)                                 (optional)
 *     Q_j = x_n W^Q[:, j], K_j = x_n W^K[:, j], V_j = x_n W^V[:, j]
 *     O_j = softmax(Q_j K_j^T / sqrt(d)) V_j             (no mask)
 *     attn = [O_0 | ... | O_{H-1}]       (all_gather and cat of the ranks)
 *       or   attn = sum_i O_(rank i) W^O_i (row-parallel output projection)
 *     out = x + attn                                     (optional)
 * W^Q[:, j] are columns j d .. (j+1) d - 1, W^O_i the rows of W^O for rank
 * i's heads.  Attention runs over the tokens of each sequence, per head.
 * bf16 only; d must be 64.
 * ------------------------------------------------------------------------ */

typedef struct tpmlp_attn tpmlp_attn;   /* opaque: packed attention weights */

enum {
    TPMLP_ATTN_LAYERNORM = 1,   /* normalise each row of x first (no affine)       */
    TPMLP_ATTN_RESIDUAL = 2     /* add x to the result                             */
};

/* Bytes of the packed buffer for hidden size h (W^Q, W^K, W^V stacked and
 * transposed, their column sums, and W^O transposed when with_out_proj).
 * Returns 0 for invalid arguments (see tpmlp_attn_pack). */
size_t tpmlp_attn_pack_bytes(int64_t hidden, int heads, int p, int dtype, int with_out_proj);

/*
 * tpmlp_attn_pack -- pack the projection weights for tpmlp_attention.
 *   Wq, Wk, Wv  device, h x h row-major (x W), bf16; read only.
 *   Wo          device, h x h row-major, or NULL for the concatenation
 *               form (no output projection).
 *   hidden      h = heads * 64; heads > 0; p > 0 divides heads.
 *   packed      device, tpmlp_attn_pack_bytes(...) bytes, caller-owned,
 *               must stay valid while the descriptor is used.
 *   out         receives a host descriptor (free with tpmlp_attn_destroy);
 *               set to NULL on error.
 * Errors: TPMLP_ERR_NULL, TPMLP_ERR_SHAPE (h != 64 heads, sizes out of
 * range), TPMLP_ERR_INDIVISIBLE (p does not divide heads), TPMLP_ERR_DTYPE
 * (not bf16), TPMLP_ERR_WORKSPACE (packed too small), TPMLP_ERR_ALIGN,
 * TPMLP_ERR_HIP.
 */
tpmlp_status tpmlp_attn_pack(const void* Wq, const void* Wk, const void* Wv, const void* Wo, int64_t hidden,
                             int heads, int p, int dtype, void* packed, size_t packed_bytes, tpmlp_attn** out,
                             void* stream);

/* Frees the host descriptor only. */
void tpmlp_attn_destroy(tpmlp_attn* a);

/* Bytes of device workspace tpmlp_attention needs for batch x seq tokens:
 * the LayerNorm statistics, Q|K|V (batch seq x 3h), the heads' outputs
 * (batch seq x h) when W^O is packed, and the projection GEMMs' split-K
 * scratch.  0 for invalid arguments. */
size_t tpmlp_attn_workspace_bytes(const tpmlp_attn* a, int64_t batch, int64_t seq);

/*
 * tpmlp_attention -- the attention half described above.
 *   x      device, (batch seq) x h row-major bf16, sequence b in rows
 *          b seq .. (b+1) seq - 1.
 *   out    device, (batch seq) x h bf16; must not overlap x or the workspace.
 *   flags  TPMLP_ATTN_LAYERNORM | TPMLP_ATTN_RESIDUAL, or 0.
 *   ln_eps LayerNorm epsilon; 0 selects 1e-5.
 *   events optional: 4 hipEvent_t recorded on the stream before the
 *          LayerNorm statistics, before the QKV projection, before the
 *          attention kernel and after the last kernel (NULL entries skipped).
 * batch = 0 or seq = 0 is a no-op.  Errors: TPMLP_ERR_NULL, TPMLP_ERR_SHAPE
 * (negative sizes, batch > 65535, batch seq > 2^21, (seq + 64) 3h bf16
 * values of one sequence's Q|K|V reaching 2 GiB, unknown flags), TPMLP_ERR_ALIGN,
 * TPMLP_ERR_WORKSPACE, TPMLP_ERR_HIP; all but the last before any HIP call.
 */
tpmlp_status tpmlp_attention(const void* x, int64_t batch, int64_t seq, const tpmlp_attn* a, void* out, int flags,
                             float ln_eps, void* workspace, size_t workspace_bytes, void* const* events,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPMLP_H */
