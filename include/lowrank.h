/*
 * lowrank.h -- C ABI of the low-rank decomposed hot path on AMD MI355X (gfx950).
 *
 * Citation key: "DeInfer/en" is the English technical summary page of
 * "DeInfer: Efficient Parallel Inferencing for Decomposed Large Language
 * Models" (gist.science); "DeInfer/es" is the Spanish page ("Resumen
 * Técnico"), "DeInfer/zh" the Chinese page.
 *
 * A dense weight W[d_in, d_out] is replaced by two smaller matrices (W ~ A B,
 * DeInfer/en §1).  The layer applies the downward projection into rank space
 * and then the upward projection (DeInfer/en §2.A):
 *
 *     t = x . U_r        (U_r: [d_in, r])      stage 1
 *     y = t . V_r        (V_r: [r, d_out])     stage 2
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     device memory, keeps no pointer after returning, and holds no global
 *     state except immutable device properties.
 *   - Asynchrony: work is enqueued on `stream` and never synchronised; every
 *     call may be captured into a HIP graph (no memset/memcpy nodes, no host
 *     reads of device data).  Calls are reentrant; two calls in flight must
 *     not share a workspace.
 *   - Errors: every call returns lr_status.  LR_OK means the work was
 *     enqueued.  Any other value is returned by host-side argument checks and
 *     means nothing was enqueued -- except LR_ERR_HIP, reported when the HIP
 *     runtime rejects a launch (earlier launches of that call may have been
 *     enqueued).  The library never aborts.
 *   - Device data cannot be checked from the host without breaking graph
 *     capture, so kernels defend themselves: out-of-range remap entries give
 *     zero rows and device counts are clamped to their capacity.
 *   - Layout: row-major 2-D arrays with explicit leading dimensions (in
 *     elements).  The factors are stored transposed, one output's weights
 *     contiguous along the reduction axis:
 *         Ut = U_r^T  as [r, d_in]    with ldu >= d_in
 *         Vt = V_r^T  as [d_out, r]   with ldv >= r
 *     so a tensor-parallel share (U_r split by input rows, V_r split by output
 *     columns) is a plain sub-matrix: Ut + row0 with the full ldu, and
 *     Vt + col0 * ldv.
 *   - bf16 operands: pointers 16-byte aligned and leading dimensions a
 *     multiple of 8 elements (LR_ERR_ALIGN otherwise).  fp32 operands: 4-byte
 *     aligned, any leading dimension.
 */
#ifndef LOWRANK_H
#define LOWRANK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
  LR_OK = 0,
  LR_ERR_ARG = 1,         /* null pointer, non-positive size, ld < width, bad flag */
  LR_ERR_DTYPE = 2,       /* dtype not supported by this entry point */
  LR_ERR_ALIGN = 3,       /* vectorised operand misaligned or ld not a multiple of 8 */
  LR_ERR_WORKSPACE = 4,   /* workspace missing or smaller than lowrank_workspace_bytes */
  LR_ERR_CAPACITY = 5,    /* packed rows exceed the fixed capacity */
  LR_ERR_HIP = 6,         /* the HIP runtime rejected a launch */
  LR_ERR_UNSUPPORTED = 7, /* valid request outside what this build implements */
  LR_ERR_WAIT = 8         /* lowrank_workspace_check: a bounded wait in a kernel gave up */
} lr_status;

typedef enum { LR_F32 = 0, LR_BF16 = 1 } lr_dtype;

/* flags of lowrank_linear_forward: one mode, optionally | LR_PACKED_WEIGHTS
   or | LR_PREFILL_FUSED */
enum {
  LR_FULL = 0,         /* y = (x U_r) V_r; t_io written too when non-NULL          */
  LR_STAGE1_ONLY = 1,  /* t_io = x U_r (t_io required; Vt, y unused)              */
  LR_STAGE2_ONLY = 2,  /* y = t_io V_r (t_io read; x, Ut unused)                   */
  LR_PACKED_WEIGHTS = 4, /* bf16, T <= 64: Ut and Vt are fragment-packed (below);
                           ldu / ldv are their block pitches in steps           */
  LR_PREFILL_FUSED = 8  /* bf16, T > 64, LR_FULL without t_io: the fused kernel
                           (t kept on chip) at any row count, instead of the
                           two large-tile GEMMs it cedes to from 1024 rows on;
                           for comparing the two.  Needs r <= 1216 (the rank
                           tile in LDS); LR_ERR_UNSUPPORTED otherwise.  No
                           workspace is needed.                                */
};

/*
 * Fragment-packed factors (bf16 decode path).  A row-major factor W[N, K]
 * (Ut: N = r, K = d_in; Vt: N = d_out, K = r) is stored as 16-row blocks,
 * each a run of 32-column steps; one step of one block is the 1 KiB a wave
 * feeds to a 16x16x32 matrix-core instruction as its weight operand, so the
 * decode kernels stream contiguous memory (row-major steps touch 16 rows x
 * 64 bytes per load, which wastes HBM bandwidth on long rows):
 *     element (n, k) -> ((b * pitch + s) * 64 + lane) * 8 + e      (elements)
 *     b = n / 16, s = k / 32, lane = n % 16 + 16 * ((k % 32) / 8), e = k % 8
 * pitch (steps per block) >= ceil(K / 32).  Entries past N or K are zero.
 * Tensor-parallel shares stay views: input rows [k0, k1) of U_r (k0 a
 * multiple of 32) are Ut_packed + (k0 / 32) * 512 with the same pitch, output
 * columns [n0, n1) of V_r (n0 a multiple of 16) are Vt_packed + (n0 / 16) *
 * pitch * 512.
 *
 * lowrank_packed_bytes: ceil(N / 16) * ceil(K / 32) * 1024 (pitch =
 * ceil(K / 32)); 0 for non-positive sizes.
 * lowrank_pack_factor: packed = pack(W), W bf16 [N, K] row-major with pitch
 * ld (elements), packed of at least ceil(N / 16) * pitch * 1024 bytes; both
 * device pointers 16-byte aligned, ld a multiple of 8.  Bit-exact copy.
 * Errors: LR_ERR_ARG (null, non-positive size, ld < K, pitch < ceil(K / 32)),
 * LR_ERR_ALIGN, LR_ERR_HIP.
 */
size_t lowrank_packed_bytes(int64_t N, int64_t K);
lr_status lowrank_pack_factor(const void* W, int64_t N, int64_t K, int64_t ld, void* packed,
                              int64_t pitch, hipStream_t stream);

/*
 * lowrank_linear_forward -- the decomposed linear, DeInfer/en §2.A (downward
 * projection, then upward projection), DeInfer/es §2 "Comunicación de Bajo
 * Rango Eficiente".  With LR_STAGE1_ONLY on one tensor-parallel share (x and
 * Ut restricted to the share's input rows) it forms the partial rank-r
 * intermediate that the shares would exchange in rank space; LR_STAGE2_ONLY on
 * an output-column shard of V_r is the pages' "shard mode" upward projection.
 *
 *   dt       LR_F32: x, Ut, Vt, y are float; LR_BF16: they are bfloat16.
 *            Accumulation is fp32 in both cases; bf16 outputs are rounded to
 *            nearest even.
 *   T        number of token rows (>= 1).  T <= 64 runs the decode path
 *            (weights streamed once from HBM); 64 < T < 1024 runs the fused
 *            two-stage MFMA kernel (the rank-r tile kept on chip); from 1024
 *            rows on, the two stages run as two large-tile MFMA GEMMs with t
 *            parked in the workspace as bf16 (the value an fp32 t_io holds,
 *            rounded to nearest even: the same operand stage 2 multiplies on
 *            every path).
 *   x        [T, d_in], ldx        (stage 1 input)
 *   Ut       [r, d_in], ldu        (U_r transposed)
 *   Vt       [d_out, r], ldv       (V_r transposed)
 *   y        [T, d_out], ldy       (output of LR_FULL / LR_STAGE2_ONLY)
 *   t_io     float [T, r], ldt     optional for LR_FULL (written), required
 *            for the stage-only flags (written by stage 1, read by stage 2).
 *   workspace, workspace_bytes
 *            device scratch of at least
 *            lowrank_workspace_bytes(0, dt, T, d_in, r, d_out, 0) bytes,
 *            256-byte aligned; NULL allowed when that size is 0.  It must be
 *            zero-filled before its first use: the decode path keeps its
 *            work counters there and returns them to zero when a call
 *            completes, so later calls (and graph replays) need no clearing.
 *            A workspace may serve calls of any shape in turn, never two calls
 *            in flight at once.
 *   Errors: LR_ERR_DTYPE, LR_ERR_ARG (sizes, missing operands), LR_ERR_ALIGN,
 *   LR_ERR_WORKSPACE; LR_ERR_UNSUPPORTED on the bf16 decode path (T <= 64)
 *   when r or a leading dimension reaches 2^24 elements (or a packed pitch
 *   2^16 steps: the kernel addresses its tiles with 32-bit offsets), and for
 *   LR_PACKED_WEIGHTS with fp32 or T > 64; LR_ERR_HIP if a launch fails.
 *   Loads never reach past an operand's last element (the padding after the
 *   last row of a strided view need not be allocated).
 */
lr_status lowrank_linear_forward(lr_dtype dt, int64_t T, int64_t d_in, int64_t r, int64_t d_out,
                                 const void* x, int64_t ldx, const void* Ut, int64_t ldu,
                                 const void* Vt, int64_t ldv, void* y, int64_t ldy,
                                 float* t_io, int64_t ldt, unsigned flags, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * lowrank_linear_forward_noalloc -- lowrank_linear_forward for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without the
 * workspace, which is instead a fixed scratch array of this library, one per
 * GPU, LR_NOALLOC_SCRATCH_BYTES bytes, held until the process ends.  The call
 * allocates nothing and frees nothing.
 *
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (other streams, other threads) race and must not be
 *   issued.  The scratch keeps the last call's contents; the decode path's
 *   counters return to zero at the end of every call, as in a workspace.
 *   Errors: as lowrank_linear_forward, and LR_ERR_CAPACITY when the call needs
 *   more scratch than LR_NOALLOC_SCRATCH_BYTES (lowrank_workspace_bytes(0, ...)
 *   gives the need); LR_ERR_HIP if the scratch address cannot be looked up.
 *   A bounded wait that gives up is not reported by this variant.
 */
#define LR_NOALLOC_SCRATCH_BYTES (8u << 20)
lr_status lowrank_linear_forward_noalloc(lr_dtype dt, int64_t T, int64_t d_in, int64_t r,
                                         int64_t d_out, const void* x, int64_t ldx,
                                         const void* Ut, int64_t ldu, const void* Vt,
                                         int64_t ldv, void* y, int64_t ldy, float* t_io,
                                         int64_t ldt, unsigned flags, hipStream_t stream);

/*
 * lowrank_linear_forward_group -- n independent decomposed linears
 * (DeInfer/en §2.A, as lowrank_linear_forward) over the same T token rows in
 * one launch: bf16 decode path only (1 <= T <= 64, 1 <= n <= 8).  Meant for
 * the projections of a decoder layer that read the same input (q, k, v;
 * gate, up): one launch instead of n, and one linear's hand-over from stage
 * 1 to stage 2 overlaps the others' weight streams.  The launch splits the
 * stage-1 reduction over d_in into as many K ranges as keep about one
 * stage-1 tile per CU for the whole group, so a member's t (and y) may
 * differ from a separate call's in fp32 summation order; it is bit for bit
 * the separate call's whenever both split d_in alike.
 *
 *   lin[i]   one linear, operands as in lowrank_linear_forward (bf16 x, Ut,
 *            Vt, y; fp32 t_io):
 *              Vt == NULL   stage 1 only: t_io = x U_r (t_io required)
 *              Ut == NULL   stage 2 only: y = bf16(t_io V_r) from the fp32
 *                           t_io [T, r] (x unused; d_in > 0 still given)
 *              y_acc != NULL  y_acc[T, ld_acc] += y in fp32 (y unused)
 *              otherwise    y = bf16((x U_r) V_r), t_io written when given
 *   flags    0 or LR_PACKED_WEIGHTS (then every Ut / Vt is fragment-packed,
 *            ldu / ldv block pitches in steps).
 *   workspace  at least lowrank_group_workspace_bytes(T, n, lin) bytes,
 *            256-byte aligned, zero-filled before first use (as for
 *            lowrank_linear_forward, whose workspaces it may share: both keep
 *            their counters in the same fixed area at its start).
 * Errors: LR_ERR_ARG (n or T out of range, a missing operand, ld < width),
 * LR_ERR_ALIGN, LR_ERR_WORKSPACE, LR_ERR_UNSUPPORTED (a leading dimension,
 * pitch or r past the decode path's limits), LR_ERR_HIP.
 */
typedef struct {
  int64_t d_in, r, d_out;
  const void* x;  int64_t ldx;
  const void* Ut; int64_t ldu;
  const void* Vt; int64_t ldv;
  void* y;        int64_t ldy;
  float* y_acc;   int64_t ld_acc;
  float* t_io;    int64_t ldt;
} lr_linear;

size_t lowrank_group_workspace_bytes(int64_t T, int n, const lr_linear* lin);
lr_status lowrank_linear_forward_group(int64_t T, int n, const lr_linear* lin, unsigned flags,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * kv_remap_gather -- the graph-replay copy of DeInfer/en §2.C (and DeInfer/es
 * §2, "Etapa de Reproducción del Gráfico"): rows of a paged pool are copied
 * into a compact buffer at a fixed address, following the remapping index
 * list built by the preparation stage.
 *
 *   for j < min(*n_valid, cap) (or j < cap when n_valid is NULL):
 *       dst[j, 0:row_elems] = src[remap[j], 0:row_elems]  if 0 <= remap[j] < src_rows
 *                           = 0                           otherwise
 *   rows j >= *n_valid are left untouched.  Bit-exact copy.
 *
 *   dt        element type (LR_BF16 or LR_F32); only the width matters.
 *   src       device [src_rows, src_ld]
 *   remap     device int32 [cap]
 *   n_valid   device int32 scalar or NULL; read by the kernel, so it may
 *             change between replays of a captured graph.
 *   dst       device [cap, dst_ld]
 *   Vector path when both row pitches and pointers are 16-byte aligned;
 *   otherwise a 2-byte/4-byte path (never an error).
 */
lr_status kv_remap_gather(lr_dtype dt, const void* src, int64_t src_rows, int64_t src_ld,
                          const int32_t* remap, int64_t cap, const int32_t* n_valid,
                          int64_t row_elems, void* dst, int64_t dst_ld, hipStream_t stream);

/*
 * lowrank_prepare_decode -- host-side preparation stage of DeInfer/en §2.C
 * (the paged cache is walked for runs of physically adjacent blocks, and a
 * remapping index list is emitted), DeInfer/zh (remapping table),
 * DeInfer/es §2 "Etapa de Preparación".  Runs on the CPU, touches host
 * memory only.
 *
 * Sequence i has lengths[i] cached tokens and decodes one new token at
 * position lengths[i]; its compact segment holds lengths[i] + 1 rows.
 * Logical row p of sequence i lives at physical row
 * tables[i * table_ld + p / block] * block + p % block.
 *
 * Outputs (host arrays supplied by the caller):
 *   remap[cap]        physical source row of each packed row; -1 past n_valid
 *   seq_off[B + 1]    prefix sums of lengths[i] + 1
 *   pos[B]            position of each new token (= lengths[i])
 *   slot_mapping[B]   physical row the new token's latents are written to
 *   *n_valid          seq_off[B]
 *   *n_runs           number of maximal runs of physically consecutive blocks
 *   runs              optional int32 [max_runs, 3] of (src_row, dst_row, rows)
 * Errors: LR_ERR_ARG (null/negative, a block index < 0 or a table too short
 * for lengths[i] + 1 rows), LR_ERR_CAPACITY (seq_off[B] > cap, or more runs
 * than max_runs when runs is non-NULL).
 */
lr_status lowrank_prepare_decode(int64_t B, const int32_t* lengths, const int32_t* tables,
                                 int64_t table_ld, int64_t block, int64_t cap, int32_t* remap,
                                 int32_t* seq_off, int32_t* pos, int32_t* slot_mapping,
                                 int32_t* n_valid, int32_t* n_runs, int32_t* runs,
                                 int64_t max_runs);

/*
 * lowrank_prepare_prefill -- the same preparation stage for a chunked-prefill
 * step (DeInfer/en §2.C applied to the prompt side): sequence i has
 * lengths[i] cached tokens and appends chunk[i] >= 1 new tokens at positions
 * lengths[i] .. lengths[i] + chunk[i] - 1, so its compact segment holds
 * lengths[i] + chunk[i] rows.  The new tokens are numbered in sequence order,
 * then position order.
 *
 * Outputs as lowrank_prepare_decode (seq_off now the prefix sums of
 * lengths[i] + chunk[i]), with per new token t < *n_tokens:
 *   tok_seq[t]        its sequence
 *   pos[t]            its position
 *   slot_mapping[t]   physical row its latents are written to
 * pos, tok_seq and slot_mapping hold max_tokens entries.
 * Errors: as lowrank_prepare_decode, plus LR_ERR_ARG for chunk[i] < 1 or a
 * null chunk / tok_seq / n_tokens, LR_ERR_CAPACITY for more than max_tokens
 * new tokens.  lowrank_prepare_decode is this call with every chunk[i] = 1.
 */
lr_status lowrank_prepare_prefill(int64_t S, const int32_t* lengths, const int32_t* chunk,
                                  const int32_t* tables, int64_t table_ld, int64_t block,
                                  int64_t cap, int64_t max_tokens, int32_t* remap,
                                  int32_t* seq_off, int32_t* tok_seq, int32_t* pos,
                                  int32_t* slot_mapping, int32_t* n_tokens, int32_t* n_valid,
                                  int32_t* n_runs, int32_t* runs, int64_t max_runs);

/*
 * lowrank_rope_table -- rotary-embedding table for the decode step:
 * table[p][i] = (cos(p w_i), sin(p w_i)), w_i = theta^(-2i/head_dim),
 * p < max_pos, i < head_dim/2, computed on the device in double precision and
 * stored as float.  A constant of the model; build it once.  The rotation
 * (rotate-half pairing (i, i + head_dim/2)) is the LLaMA convention the
 * decode step assumes; the pages do not specify it.
 */
lr_status lowrank_rope_table(int64_t head_dim, int64_t max_pos, float theta, float* table,
                             hipStream_t stream);

/* MLP of a decoder layer (lr_layer_weights.mlp). */
enum {
  LR_MLP_SWIGLU = 0, /* down(silu(gate(x)) * up(x)): slots 4, 5, 6 */
  LR_MLP_RELU = 1    /* fc2(relu(fc1(x))): fc1 in slot 4, fc2 in slot 6, slot 5 unused */
};

/*
 * Weights of one decoder layer whose linears (q, k, v, o, gate, up, down, in
 * this order) are decomposed (DeInfer/en §2.D: MHA/GQA/MQA attention through
 * n_kv_heads, GLU and non-GLU MLPs through mlp, per-layer ratios -- r[] may
 * differ per linear and per layer).  Ut[k] is U_r^T [r[k], d_in] and Vt[k]
 * is V_r^T [d_out, r[k]], bf16, 16-byte aligned, ld a multiple of 8 (slot 5
 * is ignored, and may be NULL, when mlp = LR_MLP_RELU).  Norm weights are
 * bf16 [d_model].
 */
typedef struct {
  int64_t d_model, n_heads, n_kv_heads, head_dim, d_ffn;  /* head_dim 64 or 128 */
  float eps;                                              /* RMSNorm epsilon */
  const void* Ut[7];
  int64_t ldu[7];
  const void* Vt[7];
  int64_t ldv[7];
  int64_t r[7];
  const void* attn_norm;
  const void* ffn_norm;
  const float* rope;        /* lowrank_rope_table output */
  int64_t rope_max_pos;     /* positions the table covers */
  int64_t mlp;              /* LR_MLP_SWIGLU or LR_MLP_RELU */
} lr_layer_weights;

/*
 * Paged cache of rank-r latents and the preparation-stage outputs of one
 * decode step (DeInfer/en §2.C; see lowrank_prepare_decode).  The pools hold
 * this layer's cached latents x U_k and x U_v (before rotary), one bf16 row
 * per token slot.  Every array is device memory at a fixed address; its
 * contents may change between replays of a captured graph.
 */
typedef struct {
  void* k_pool;
  void* v_pool;                  /* [pool_rows, pool_ld] bf16, pool_ld >= r_k, r_v */
  int64_t pool_rows, pool_ld;
  const int32_t* slot_mapping;   /* [B] slot of each new token's latents */
  const int32_t* remap;          /* [cap] source slot of each packed row */
  const int32_t* seq_off;        /* [B + 1] packed-row offsets */
  const int32_t* pos;            /* [B] position of each new token */
  const int32_t* n_valid;        /* scalar: packed rows in use (= seq_off[B]) */
  int64_t B, cap, max_seq_rows;  /* capacities fixing every grid; max_seq_rows >= L_i + 1 */
} lr_decode_state;

/* Device scratch of lowrank_layer_decode_step for these shapes (compact and
 * reconstructed K/V buffers, activations, attention partials, linear
 * scratch).  Zero-fill it before its first use. */
size_t lowrank_decode_step_workspace_bytes(const lr_layer_weights* w, const lr_decode_state* s);

/*
 * lowrank_layer_decode_step -- one decoder layer for B sequences, one new
 * token each, in place on the fp32 residual stream h [B, d_model]:
 *   x = RMSNorm(h) ; q = RoPE(lowrank_q(x), pos) ; latents x U_k, x U_v
 *   appended at slot_mapping (bf16) ; compact copy of every sequence's
 *   latents through remap (DeInfer/en §2.C replay copy) ; K = RoPE(buf_k V_k),
 *   V = buf_v V_v by one GEMM of fixed size over cap rows (its shape and
 *   addresses never change between steps; rows past *n_valid are skipped) ;
 *   softmax attention of each query over
 *   its sequence's rows ; h += lowrank_o(o) ; x = RMSNorm(h) ;
 *   h += lowrank_down(silu(lowrank_gate(x)) * lowrank_up(x))  (LR_MLP_SWIGLU), or
 *   h += lowrank_fc2(relu(lowrank_fc1(x)))  (LR_MLP_RELU).
 * Launches only; fixed grids, no host reads of device data, no allocation:
 * capture 32 calls (one per layer) in one graph and replay it each step
 * after refreshing the preparation arrays.
 * The projections run on the decode path (q, k, v as one grouped launch,
 * gate and up as another), so B <= 64.
 * Errors: LR_ERR_ARG (also: mlp not LR_MLP_SWIGLU / LR_MLP_RELU) /
 * LR_ERR_ALIGN (also: rope not 16-byte aligned) / LR_ERR_UNSUPPORTED
 * (head_dim not 64 or 128, B > 64, a factor pitch of 2^22 elements or more)
 * / LR_ERR_WORKSPACE from host checks, LR_ERR_HIP from the runtime.
 */
lr_status lowrank_layer_decode_step(const lr_layer_weights* w, const lr_decode_state* s,
                                    float* h, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Device scratch of lowrank_layer_decode_step_fused (no reconstructed K/V
 * buffers).  Zero-fill it before its first use. */
size_t lowrank_decode_step_fused_workspace_bytes(const lr_layer_weights* w,
                                                 const lr_decode_state* s);

/*
 * lowrank_layer_decode_step_fused -- the layer of lowrank_layer_decode_step
 * with the reconstruction folded into the attention: per 256-row block of a
 * sequence's latents (read in place through the remap list) and 256 K
 * columns, one workgroup expands K = RoPE(buf_k V_k) on chip (rounded to
 * bf16, as the reconstruction stores it), scores the block against the
 * sequence's query heads, and writes the block's softmax max and sum and its
 * p-weighted sum of V latent rows (r_v wide).  A second kernel combines a
 * sequence's blocks per head and applies V_v once: by associativity
 * sum_rows p (buf_v V_v) = (sum_rows p buf_v) V_v, so V is never formed.
 * The reconstructed rows (2 * cap * n_kv_heads * head_dim bf16 in
 * lowrank_layer_decode_step) never reach memory.  The result equals
 * lowrank_layer_decode_step's up to the order of the fp32 sums and the bf16
 * rounding of the reconstructed V (relative differences ~1e-3).  Same
 * arguments, ownership and graph rules.
 * Errors: as lowrank_layer_decode_step, plus LR_ERR_UNSUPPORTED when
 * (256 / head_dim) * (n_heads / n_kv_heads) > 16 (query heads per 256
 * K/V columns).
 */
lr_status lowrank_layer_decode_step_fused(const lr_layer_weights* w, const lr_decode_state* s,
                                          float* h, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/*
 * State of one chunked-prefill step (see lowrank_prepare_prefill): T new
 * tokens in S sequences; sequence i's compact segment holds its cached rows
 * and its new tokens' rows.  Device arrays, as in lr_decode_state.
 */
typedef struct {
  void* k_pool;
  void* v_pool;                  /* [pool_rows, pool_ld] bf16, pool_ld >= r_k, r_v */
  int64_t pool_rows, pool_ld;
  const int32_t* slot_mapping;   /* [T] slot of each new token's latents */
  const int32_t* remap;          /* [cap] source slot of each packed row */
  const int32_t* seq_off;        /* [S + 1] packed-row offsets */
  const int32_t* tok_seq;        /* [T] sequence of each new token */
  const int32_t* pos;            /* [T] position of each new token */
  const int32_t* n_valid;        /* scalar: packed rows in use (= seq_off[S]) */
  int64_t T, S, cap, max_seq_rows; /* max_seq_rows >= rows of the longest segment */
} lr_prefill_state;

/* Device scratch of lowrank_layer_prefill_step for these shapes. */
size_t lowrank_prefill_step_workspace_bytes(const lr_layer_weights* w, const lr_prefill_state* s);

/*
 * lowrank_layer_prefill_step -- one decoder layer over a chunk of prompt
 * tokens (the prefill side of DeInfer/en §2.C: the chunk's latents join the
 * paged cache that later decode steps reconstruct), in place on h [T,
 * d_model] fp32, tokens in sequence order.  The same layer as
 * lowrank_layer_decode_step, with causal attention: new token t attends to
 * its sequence's rows 0 .. pos[t] (the cached ones and the chunk's tokens up
 * to itself).  Projections of at most 64 tokens run on the decode path,
 * larger chunks on the prefill path (below 1024 tokens their o and down
 * outputs are rounded to bf16 before they are added to h; from 1024 tokens on
 * they are added in fp32 by the GEMM).  S <= 255.
 * Errors: as lowrank_layer_decode_step (without the B <= 64 limit), plus
 * LR_ERR_ARG for a null tok_seq and LR_ERR_UNSUPPORTED for S > 255.
 */
lr_status lowrank_layer_prefill_step(const lr_layer_weights* w, const lr_prefill_state* s,
                                     float* h, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Device scratch of lowrank_linear_forward (which = 0; cap unused).  Other
 * values of which return 0: the decode step has its own sizing call. */
size_t lowrank_workspace_bytes(int which, lr_dtype dt, int64_t T_or_B, int64_t d_in, int64_t r,
                               int64_t d_out, int64_t cap);

const char* lowrank_status_string(lr_status s);

/*
 * lowrank_workspace_check -- after the decode path (lowrank_linear_forward
 * with bf16 and T <= 64, lowrank_linear_forward_group, and the decode and
 * prefill layer steps, whose workspaces start with the same control area):
 * did a bounded wait inside a kernel give up?  A stage-2 tile waits for the
 * rank-r intermediate of DeInfer/en §2.A to be complete; the wait is bounded
 * (lowrank_set_wait_limit) so that no input can hang the GPU, and a wait that
 * gives up leaves an error word in the workspace and lets the call finish
 * with stale data.
 *
 *   Synchronises `stream`, reads the error words of the workspace's eight
 *   control blocks (the first 128 KiB) and stores in *failed (when non-NULL)
 *   a bit mask of the blocks (linears of a launch) whose wait gave up.
 *   Returns LR_OK when none did.  Otherwise it zero-fills the control area
 *   (so later calls start from clean counters) and returns LR_ERR_WAIT: the
 *   outputs of the calls since the previous check are unreliable.
 *   Not capturable in a graph (it synchronises).  Errors: LR_ERR_ARG (NULL
 *   or misaligned workspace), LR_ERR_WORKSPACE (under 128 KiB), LR_ERR_HIP.
 */
lr_status lowrank_workspace_check(void* workspace, size_t workspace_bytes, uint32_t* failed,
                                  hipStream_t stream);

/*
 * lowrank_set_wait_limit -- polls (each about a microsecond) a bounded wait
 * of the decode path makes before it gives up, for launches issued (or
 * captured) from now on, process-wide.  LR_DEFAULT_WAIT_LIMIT is the default;
 * tiny values are a test hook that forces the give-up path while every
 * kernel still runs to its end.
 */
#define LR_DEFAULT_WAIT_LIMIT (1u << 20)
void lowrank_set_wait_limit(uint32_t polls);

/* sizeof(lr_layer_weights) for which = 0, sizeof(lr_decode_state) for
 * which = 1, sizeof(lr_linear) for which = 2, sizeof(lr_prefill_state) for
 * which = 3 (lets bindings verify their struct layout); 0 otherwise. */
size_t lowrank_abi_sizeof(int which);

/* Library ABI version (major * 100 + minor). */
int lowrank_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LOWRANK_H */
