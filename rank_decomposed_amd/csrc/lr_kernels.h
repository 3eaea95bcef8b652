// Host-side entry points of the kernel files (internal to liblowrank).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lr {

// One decomposed-linear request after argument checks (see lowrank.h).
struct DecodeLinear {
  int64_t T, d_in, r, d_out;
  const void* x;
  int64_t ldx;
  const void* Ut;
  int64_t ldu;
  const void* Vt;
  int64_t ldv;
  void* y;
  int64_t ldy;
  float* t_io;
  int64_t ldt;
  unsigned flags;
  void* workspace;
  // optional (decode path only): y_acc[T, ld_acc] += y in fp32 instead of
  // writing y; used for residual updates
  float* y_acc = nullptr;
  int64_t ld_acc = 0;
  // bf16 paths: Ut/Vt fragment-packed, ldu/ldv = block pitch in 32-column steps
  bool packed = false;
  // optional (large-tile prefill path only, see prefill_act_ok): y =
  // act(x U_r V_r), act 1 = silu(glu) * product with glu bf16 [T, ldglu],
  // act 2 = relu(product)
  int act = 0;
  const void* glu = nullptr;
  int64_t ldglu = 0;
  // prefill path: the fused kernel at any row count (prefill_fused_supported)
  bool force_fused = false;
};

// Control area of a decode-path workspace: kCtlBlocks blocks of
// kCtlBlockWords uint32 words at its start, one per linear of a launch.  Word
// kCtlErrWord of a block holds kWaitErrorMagic once a bounded wait of that
// linear gave up (lowrank_workspace_check reads and clears it).
constexpr int kCtlBlocks = 8;
constexpr int kCtlBlockWords = 4096;
// Bytes of the control area.  Every other path that parks data in a
// workspace (the prefill GEMMs' t and partials, the fp32 path's t) starts
// past it, so one workspace can serve decode calls and any others in turn
// without a clearing between them.
constexpr size_t kCtlAreaBytes = (size_t)kCtlBlocks * kCtlBlockWords * 4;
constexpr int kCtlErrWord = 1216;
constexpr uint32_t kWaitErrorMagic = 0x4c525754u;
constexpr uint32_t kDefaultSpinLimit = 1u << 20;  // polls (~1 us each) before a wait gives up
// Polls of a bounded wait in decode launches issued from now on (a test hook:
// a tiny limit forces the give-up path while every kernel still exits).
void set_spin_limit(uint32_t polls);

// bf16, T <= 64: streamed skinny MFMA path.
// The decode kernel addresses each 64-row tile with 32-bit offsets: every
// leading dimension (and r) must stay below 2^24 elements.
inline bool decode_supported(const DecodeLinear& d) {
  const int64_t lim = int64_t(1) << 24;
  if (d.packed) return d.ldx < lim && d.ldu < (1 << 16) && d.ldv < (1 << 16) && d.r < lim;
  return d.ldx < lim && d.ldu < lim && d.ldv < lim && d.r < lim;
}
// Fragment-packed copy of a row-major bf16 W[N, K] (layout in lowrank.h).
hipError_t pack_factor_bf16(const void* W, int64_t N, int64_t K, int64_t ld, void* packed,
                            int64_t pitch, hipStream_t st);
size_t decode_workspace_bytes(int64_t T, int64_t d_in, int64_t r, int64_t d_out);
hipError_t decode_linear_bf16(const DecodeLinear& d, hipStream_t st);
// Up to 8 independent linears over the same T (<= 64) token rows in one
// launch; they share the workspace of ds[0] (decode_group_workspace_bytes).
size_t decode_group_workspace_bytes(const DecodeLinear* ds, int n);
hipError_t decode_group_bf16(const DecodeLinear* ds, int n, hipStream_t st);

// bf16, T > 64: fused two-stage MFMA path (or two GEMMs).
// C[M, N] = A[M, K] . B[N, K]^T, bf16 operands (K contiguous), fp32
// accumulation; C bf16, or fp32 with an optional bf16 copy C2.  256-row
// tiles on MFMA 32x32x16 (many-token shapes).
bool gemm_big_supported(int64_t lda, int64_t ldb);
// part (optional, part_bytes): fp32 scratch that lets a bf16 launch whose
// last round of tiles is part-filled split that round's tiles over K (see
// gemm_tail_bytes); a launch that does not fit it runs unsplit.
hipError_t gemm_nt_big(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                       int64_t ldc, bool c_f32, uint16_t* C2, int64_t ldc2, int64_t M,
                       int64_t N, int64_t K, hipStream_t st, float* part = nullptr,
                       size_t part_bytes = 0);
// Scratch for the split tail of any bf16 gemm_nt_big of this M, N.
size_t gemm_tail_bytes(int64_t M, int64_t N);
// Up to kMaxGemmGroup products that share A in one launch of 128-column
// tiles, each member over whole tiles of its own: C_i[M, N_i] (fp32) =
// A . B_i^T, with an optional bf16 copy C2_i.  For stage 1 of linears that
// read the same input, where each alone has too few tiles to fill the chip.
constexpr int kMaxGemmGroup = 3;
struct GemmMember {
  const void* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
  uint16_t* C2;  // or null
  int64_t ldc2;
  int64_t N;
};
hipError_t gemm_nt_big_group(const void* A, int64_t lda, const GemmMember* g, int n, int64_t M,
                             int64_t K, hipStream_t st);
// Tiles of such a launch.
int64_t gemm_group_tiles(const int64_t* N, int n, int64_t M);
// C (bf16, 16-byte aligned rows) = act(A . B^T): act 1 = silu(G) * (A . B^T)
// with G bf16 [M, ldg] (16-byte aligned rows), act 2 = relu(A . B^T); the
// product is rounded to bf16 before the activation.
hipError_t gemm_nt_big_act(const void* A, int64_t lda, const void* B, int64_t ldb, uint16_t* C,
                           int64_t ldc, int act, const uint16_t* G, int64_t ldg, int64_t M,
                           int64_t N, int64_t K, hipStream_t st);
// C[M, ldc] (fp32) += A . B^T, same operand rules as gemm_nt_big.
hipError_t gemm_nt_big_acc(const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                           int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t st);
// Split-K variant for launches whose tiles would leave most CUs idle
// (few 128-column tiles, K >= 1024): K ranges write fp32 partials to part
// (gemm_split_bytes(M, N) bytes), summed in range order into out32 (fp32)
// and/or out16 (bf16).  gemm_split_ranges() == 1 means no split is needed.
int gemm_split_ranges(int64_t M, int64_t N, int64_t K);
size_t gemm_split_bytes(int64_t M, int64_t N);
hipError_t gemm_nt_big_split(const void* A, int64_t lda, const void* B, int64_t ldb, float* part,
                             float* out32, int64_t ld32, uint16_t* out16, int64_t ld16,
                             int64_t M, int64_t N, int64_t K, hipStream_t st);
// Rotary epilogue of gemm_nt_big_rows: rows are packed sequences (row m of
// sequence i sits at position m - seq_off[i], 1 <= nseq <= 255); table
// [max_pos][hd/2] holds (cos, sin) pairs, 16-byte aligned, under 2 GiB; N a
// multiple of hd (64 or 128).
struct BigRope {
  const float* table;
  int64_t max_pos;
  const int32_t* seq_off;  // [nseq + 1]
  int nseq;
  int hd;
};
// C[m, :] = A[m, :] . B^T (bf16 out) for the rows m < *m_valid (read on the
// device, clamped to M; the grid covers M), optionally rotated per head.
hipError_t gemm_nt_big_rows(const void* A, int64_t lda, const void* B, int64_t ldb, uint16_t* C,
                            int64_t ldc, int64_t M, const int32_t* m_valid, int64_t N, int64_t K,
                            const BigRope* rope, hipStream_t st);
// Decode attention with the reconstruction on chip (one new token per
// sequence): per 256-row block of a sequence's cached rows and an item of
// 256-column K tiles, K is expanded from the latents (rotary, rounded to
// bf16) and scored, and the block's partials part[block][h] = {m, l, the
// p-weighted sum of its V latent rows (rv)} are written; V_v is applied by
// the combine.  blk_off[i]: first block of sequence i (blk_off[S] = blocks);
// nbpad bounds the blocks (cap / 256 + S).  At most 16 query heads per 256
// columns.
struct FusedAttnArgs {
  const uint16_t* kl;  // K latents [cap, ldkl], rk columns (or the pool, see remap)
  int64_t ldkl;
  int rk;
  const uint16_t* vl;  // V latents [cap, ldvl], rv columns (or the pool, see remap)
  int64_t ldvl;
  int rv;
  // optional: kl / vl are the paged pools [pool_rows, ld] and compact row j is
  // pool row remap[j] (-1 or out of range: a zero row), read in place
  const int32_t* remap;
  int64_t pool_rows;
  const uint16_t* vk;  // V_k^T [Hkv * hd, ldvk]
  int64_t ldvk;
  const uint16_t* vv;  // V_v^T [Hkv * hd, ldvv]
  int64_t ldvv;
  const uint16_t* q;   // [S, ldq] bf16 queries before rotary
  int64_t ldq;
  const float* rope;   // [max_pos][hd/2] (cos, sin)
  int64_t max_pos;
  const int32_t* seq_off;
  const int32_t* pos;
  const int32_t* blk_off;
  int S, cap, H, Hkv, nbpad;
  float* part;         // [nbpad][H][rv + 2]
};
hipError_t attn_fused_decode(const FusedAttnArgs& a, int hd, hipStream_t st);
size_t prefill_workspace_bytes(int64_t T, int64_t r, int64_t d_out);
hipError_t prefill_linear_bf16(const DecodeLinear& d, hipStream_t st);
// Whether prefill_linear_bf16 takes the large-tile path for d, the one that
// can add y into an fp32 y_acc (other paths reject y_acc).
bool prefill_accumulates(const DecodeLinear& d);
// The fused kernel can take this call (both stages, no t_io, rank tile in
// LDS, operands under its 32-bit offsets).
bool prefill_fused_supported(const DecodeLinear& d);
// Whether prefill_linear_bf16 can apply d.act in the stage-2 epilogue.
bool prefill_act_ok(const DecodeLinear& d);
// Linears over the same input x on the large-tile path whose stage 1 runs
// as one grouped launch (2 or 3 of them, each a full linear or stage 1 with
// t_io, with too few tiles each to fill the chip); then each full member's
// stage 2 in order (so a member's act may read an earlier member's y).
bool prefill_group_ok(const DecodeLinear* ds, int n);
size_t prefill_group_workspace_bytes(const DecodeLinear* ds, int n);
hipError_t prefill_group_bf16(const DecodeLinear* ds, int n, hipStream_t st);

// fp32, any T: tiled SIMT path.
size_t f32_workspace_bytes(int64_t T, int64_t r);
hipError_t linear_f32(const DecodeLinear& d, hipStream_t st);

// Plain bf16 GEMM C[M, N] = A[M, K] . B[N, K]^T into bf16 C (prefill helper).
hipError_t gemm_nt_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                        int64_t ldc, int M, int N, int K, hipStream_t st);

// Remap gather (bit copy of rows).
hipError_t remap_gather(int elem_bytes, const void* src, int64_t src_rows, int64_t src_ld,
                        const int32_t* remap, int64_t cap, const int32_t* n_valid,
                        int64_t row_elems, void* dst, int64_t dst_ld, hipStream_t st);

}  // namespace lr
