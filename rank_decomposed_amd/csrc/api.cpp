// C ABI of liblowrank: host-side argument checks and path selection.  No
// allocation, no synchronisation, no global mutable state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lowrank.h"
#include "lr_kernels.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" int lowrank_version(void) { return 102; }

extern "C" size_t lowrank_abi_sizeof(int which) {
  switch (which) {
    case 0: return sizeof(lr_layer_weights);
    case 1: return sizeof(lr_decode_state);
    case 2: return sizeof(lr_linear);
    case 3: return sizeof(lr_prefill_state);
    default: return 0;
  }
}

extern "C" const char* lowrank_status_string(lr_status s) {
  switch (s) {
    case LR_OK: return "ok";
    case LR_ERR_ARG: return "invalid argument";
    case LR_ERR_DTYPE: return "unsupported dtype";
    case LR_ERR_ALIGN: return "misaligned operand or leading dimension";
    case LR_ERR_WORKSPACE: return "workspace missing or too small";
    case LR_ERR_CAPACITY: return "capacity exceeded";
    case LR_ERR_HIP: return "HIP runtime error";
    case LR_ERR_UNSUPPORTED: return "unsupported configuration";
    case LR_ERR_WAIT: return "a bounded wait inside a decode kernel gave up";
  }
  return "unknown status";
}

static size_t linear_ws(lr_dtype dt, int64_t T, int64_t d_in, int64_t r, int64_t d_out) {
  if (dt == LR_F32) return lr::f32_workspace_bytes(T, r);
  if (T <= 64) return lr::decode_workspace_bytes(T, d_in, r, d_out);
  return lr::prefill_workspace_bytes(T, r, d_out);
}

extern "C" size_t lowrank_workspace_bytes(int which, lr_dtype dt, int64_t T_or_B, int64_t d_in,
                                          int64_t r, int64_t d_out, int64_t cap) {
  (void)cap;
  if (T_or_B <= 0 || d_in <= 0 || r <= 0 || d_out <= 0) return 0;
  if (which == 0) {
    if (dt != LR_F32 && dt != LR_BF16) return 0;
    return linear_ws(dt, T_or_B, d_in, r, d_out);
  }
  return 0;
}

extern "C" lr_status lowrank_linear_forward(lr_dtype dt, int64_t T, int64_t d_in, int64_t r,
                                            int64_t d_out, const void* x, int64_t ldx,
                                            const void* Ut, int64_t ldu, const void* Vt,
                                            int64_t ldv, void* y, int64_t ldy, float* t_io,
                                            int64_t ldt, unsigned flags, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  if (dt != LR_F32 && dt != LR_BF16) return LR_ERR_DTYPE;
  const bool packed = (flags & LR_PACKED_WEIGHTS) != 0;
  const bool fused = (flags & LR_PREFILL_FUSED) != 0;
  const unsigned mode = flags & ~(unsigned)(LR_PACKED_WEIGHTS | LR_PREFILL_FUSED);
  if (mode > 2) return LR_ERR_ARG;
  if (T <= 0 || d_in <= 0 || r <= 0 || d_out <= 0) return LR_ERR_ARG;
  if (T > INT32_MAX || d_in > INT32_MAX || r > INT32_MAX || d_out > INT32_MAX) return LR_ERR_ARG;
  const bool s1 = mode != LR_STAGE2_ONLY, s2 = mode != LR_STAGE1_ONLY;
  // row-major factors: ld in elements; packed: block pitch in 32-column steps
  const int64_t ku = packed ? (d_in + 31) / 32 : d_in, kv = packed ? (r + 31) / 32 : r;
  if (s1 && (!x || !Ut || ldx < d_in || ldu < ku)) return LR_ERR_ARG;
  if (s2 && (!Vt || !y || ldv < kv || ldy < d_out)) return LR_ERR_ARG;
  if (mode != LR_FULL && !t_io) return LR_ERR_ARG;
  if (t_io && ldt < r) return LR_ERR_ARG;
  if (t_io && !aligned(t_io, 4)) return LR_ERR_ALIGN;
  if (packed && (dt != LR_BF16 || T > 64)) return LR_ERR_UNSUPPORTED;
  if (dt == LR_BF16) {
    if (s1 && (!aligned(x, 16) || !aligned(Ut, 16) || ldx % 8 || (!packed && ldu % 8)))
      return LR_ERR_ALIGN;
    if (s2 && (!aligned(Vt, 16) || (!packed && ldv % 8) || !aligned(y, 2))) return LR_ERR_ALIGN;
  } else {
    if (s1 && (!aligned(x, 4) || !aligned(Ut, 4))) return LR_ERR_ALIGN;
    if (s2 && (!aligned(Vt, 4) || !aligned(y, 4))) return LR_ERR_ALIGN;
  }
  const size_t need = fused ? 0 : linear_ws(dt, T, d_in, r, d_out);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return LR_ERR_WORKSPACE;

  lr::DecodeLinear d{T, d_in, r, d_out, x, ldx, Ut, ldu, Vt, ldv, y, ldy, t_io, ldt, mode,
                     workspace};
  d.packed = packed;
  d.force_fused = fused;
  if (fused && (dt != LR_BF16 || T <= 64 || !lr::prefill_fused_supported(d)))
    return LR_ERR_UNSUPPORTED;
  if (dt == LR_BF16 && T <= 64 && !lr::decode_supported(d)) return LR_ERR_UNSUPPORTED;
  hipError_t e;
  if (dt == LR_F32)
    e = lr::linear_f32(d, stream);
  else if (T <= 64)
    e = lr::decode_linear_bf16(d, stream);
  else
    e = lr::prefill_linear_bf16(d, stream);
  return e == hipSuccess ? LR_OK : LR_ERR_HIP;
}

namespace {

// Host checks of one member of a group; fills the kernel-side description.
// 0: both stages, 1: stage 1 only (no Vt), 2: stage 2 only (no Ut)
unsigned member_mode(const lr_linear& L) { return !L.Vt ? 1u : (!L.Ut ? 2u : 0u); }

lr_status group_member(int64_t T, const lr_linear& L, bool packed, lr::DecodeLinear* d) {
  if (L.d_in <= 0 || L.r <= 0 || L.d_out <= 0) return LR_ERR_ARG;
  if (L.d_in > INT32_MAX || L.r > INT32_MAX || L.d_out > INT32_MAX) return LR_ERR_ARG;
  const bool s1 = L.Ut != nullptr, s2 = L.Vt != nullptr;
  const int64_t ku = packed ? (L.d_in + 31) / 32 : L.d_in, kv = packed ? (L.r + 31) / 32 : L.r;
  if (!s1 && !s2) return LR_ERR_ARG;
  if (s1 && (!L.x || L.ldx < L.d_in || L.ldu < ku)) return LR_ERR_ARG;
  if ((!s1 || !s2) && !L.t_io) return LR_ERR_ARG;
  if (s2 && (L.ldv < kv || (!L.y_acc && (!L.y || L.ldy < L.d_out)) ||
             (L.y_acc && L.ld_acc < L.d_out)))
    return LR_ERR_ARG;
  if (L.t_io && L.ldt < L.r) return LR_ERR_ARG;
  if (s1 && (!aligned(L.x, 16) || !aligned(L.Ut, 16) || L.ldx % 8 || (!packed && L.ldu % 8)))
    return LR_ERR_ALIGN;
  if (s2 && (!aligned(L.Vt, 16) || (!packed && L.ldv % 8))) return LR_ERR_ALIGN;
  if (s2 && !L.y_acc && !aligned(L.y, 2)) return LR_ERR_ALIGN;
  if ((L.y_acc && !aligned(L.y_acc, 4)) || (L.t_io && !aligned(L.t_io, 4))) return LR_ERR_ALIGN;
  *d = lr::DecodeLinear{T, L.d_in, L.r, L.d_out, L.x, L.ldx, L.Ut, L.ldu, L.Vt, L.ldv, L.y,
                        L.ldy, L.t_io, L.ldt, member_mode(L), nullptr};
  d->y_acc = L.y_acc;
  d->ld_acc = L.ld_acc;
  d->packed = packed;
  if (!lr::decode_supported(*d)) return LR_ERR_UNSUPPORTED;
  return LR_OK;
}

}  // namespace

extern "C" size_t lowrank_group_workspace_bytes(int64_t T, int n, const lr_linear* lin) {
  if (T <= 0 || T > 64 || n < 1 || n > 8 || !lin) return 0;
  lr::DecodeLinear d[8];
  for (int i = 0; i < n; ++i) {
    if (lin[i].d_in <= 0 || lin[i].r <= 0 || lin[i].d_out <= 0) return 0;
    d[i] = lr::DecodeLinear{T, lin[i].d_in, lin[i].r, lin[i].d_out};
    d[i].flags = member_mode(lin[i]);
  }
  return lr::decode_group_workspace_bytes(d, n);
}

extern "C" lr_status lowrank_linear_forward_group(int64_t T, int n, const lr_linear* lin,
                                                  unsigned flags, void* workspace,
                                                  size_t workspace_bytes, hipStream_t stream) {
  if (!lin || n < 1 || n > 8 || T <= 0 || T > 64) return LR_ERR_ARG;
  if (flags & ~(unsigned)LR_PACKED_WEIGHTS) return LR_ERR_ARG;
  const bool packed = flags != 0;
  lr::DecodeLinear d[8];
  for (int i = 0; i < n; ++i) {
    const lr_status st = group_member(T, lin[i], packed, &d[i]);
    if (st != LR_OK) return st;
  }
  const size_t need = lowrank_group_workspace_bytes(T, n, lin);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return LR_ERR_WORKSPACE;
  d[0].workspace = workspace;
  const hipError_t e = lr::decode_group_bf16(d, n, stream);
  return e == hipSuccess ? LR_OK : LR_ERR_HIP;
}

extern "C" size_t lowrank_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return (size_t)((N + 15) / 16) * (size_t)((K + 31) / 32) * 1024;
}

extern "C" lr_status lowrank_pack_factor(const void* W, int64_t N, int64_t K, int64_t ld,
                                         void* packed, int64_t pitch, hipStream_t stream) {
  if (!W || !packed || N <= 0 || K <= 0 || ld < K || pitch < (K + 31) / 32) return LR_ERR_ARG;
  if (!aligned(W, 16) || !aligned(packed, 16) || ld % 8) return LR_ERR_ALIGN;
  hipError_t e = lr::pack_factor_bf16(W, N, K, ld, packed, pitch, stream);
  return e == hipSuccess ? LR_OK : LR_ERR_HIP;
}

extern "C" lr_status kv_remap_gather(lr_dtype dt, const void* src, int64_t src_rows,
                                     int64_t src_ld, const int32_t* remap, int64_t cap,
                                     const int32_t* n_valid, int64_t row_elems, void* dst,
                                     int64_t dst_ld, hipStream_t stream) {
  if (dt != LR_F32 && dt != LR_BF16) return LR_ERR_DTYPE;
  const int eb = dt == LR_F32 ? 4 : 2;
  if (!src || !remap || !dst) return LR_ERR_ARG;
  if (src_rows <= 0 || cap <= 0 || row_elems <= 0) return LR_ERR_ARG;
  if (src_ld < row_elems || dst_ld < row_elems) return LR_ERR_ARG;
  if (cap > INT32_MAX) return LR_ERR_ARG;
  if (!aligned(src, eb) || !aligned(dst, eb) || !aligned(remap, 4)) return LR_ERR_ALIGN;
  if (n_valid && !aligned(n_valid, 4)) return LR_ERR_ALIGN;
  hipError_t e = lr::remap_gather(eb, src, src_rows, src_ld, remap, cap, n_valid, row_elems, dst,
                                  dst_ld, stream);
  return e == hipSuccess ? LR_OK : LR_ERR_HIP;
}

extern "C" void lowrank_set_wait_limit(uint32_t polls) { lr::set_spin_limit(polls); }

extern "C" lr_status lowrank_workspace_check(void* workspace, size_t workspace_bytes,
                                             uint32_t* failed, hipStream_t stream) {
  const size_t ctl = (size_t)lr::kCtlBlocks * lr::kCtlBlockWords * 4;
  if (!workspace || !aligned(workspace, 256)) return LR_ERR_ARG;
  if (workspace_bytes < ctl) return LR_ERR_WORKSPACE;
  if (hipStreamSynchronize(stream) != hipSuccess) return LR_ERR_HIP;
  uint32_t mask = 0;
  for (int b = 0; b < lr::kCtlBlocks; ++b) {
    uint32_t w = 0;
    const char* at = static_cast<const char*>(workspace) +
                     ((size_t)b * lr::kCtlBlockWords + lr::kCtlErrWord) * 4;
    if (hipMemcpy(&w, at, 4, hipMemcpyDeviceToHost) != hipSuccess) return LR_ERR_HIP;
    if (w == lr::kWaitErrorMagic) mask |= 1u << b;
  }
  if (failed) *failed = mask;
  if (!mask) return LR_OK;
  // a wait gave up: every counter of the control area goes back to zero
  if (hipMemsetAsync(workspace, 0, ctl, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return LR_ERR_HIP;
  return LR_ERR_WAIT;
}
