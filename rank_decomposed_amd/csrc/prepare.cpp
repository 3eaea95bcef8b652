// Host-side preparation stage of the paged latent cache (DeInfer/en §2.C
// "Preparation Stage"; DeInfer/zh remapping table; DeInfer/es §2 "Etapa de
// Preparación"): walk each sequence's block table, merge physically
// consecutive blocks into runs, and emit the remapping index list that the
// in-graph gather follows, plus the per-sequence offsets and, per new token,
// its sequence, position and slot.  Runs on the CPU between graph replays;
// the caller copies the arrays into fixed device buffers.
//
// A decode step appends one token per sequence; a chunked-prefill step
// appends chunk[i] >= 1 tokens to sequence i.  Both are the same walk: the
// compact segment of sequence i holds lengths[i] + chunk[i] rows.
#include <stdint.h>

#include "lowrank.h"

namespace {

// chunk == nullptr: one new token per sequence.  tok_seq may be null.
lr_status prepare(int64_t S, const int32_t* lengths, const int32_t* chunk, const int32_t* tables,
                  int64_t table_ld, int64_t block, int64_t cap, int64_t max_tokens,
                  int32_t* remap, int32_t* seq_off, int32_t* tok_seq, int32_t* pos,
                  int32_t* slot_mapping, int32_t* n_tokens, int32_t* n_valid, int32_t* n_runs,
                  int32_t* runs, int64_t max_runs) {
  if (S < 0 || block <= 0 || cap < 0 || table_ld < 0) return LR_ERR_ARG;
  if (!remap || !seq_off || !n_valid || !n_runs) return LR_ERR_ARG;
  if (S > 0 && (!lengths || !tables || !pos || !slot_mapping)) return LR_ERR_ARG;
  if (runs && max_runs < 0) return LR_ERR_ARG;

  // offsets and token count first: reject before writing anything else
  int64_t off = 0, ntok = 0;
  for (int64_t i = 0; i < S; ++i) {
    const int64_t L = lengths[i], c = chunk ? chunk[i] : 1;
    if (L < 0 || c < 1) return LR_ERR_ARG;
    const int64_t nblk = (L + c + block - 1) / block;
    if (nblk > table_ld) return LR_ERR_ARG;
    off += L + c;
    ntok += c;
    if (off > INT32_MAX) return LR_ERR_CAPACITY;
  }
  if (off > cap || ntok > max_tokens) return LR_ERR_CAPACITY;
  for (int64_t i = 0; i < S; ++i) {
    const int32_t* t = tables + i * table_ld;
    const int64_t nblk = (lengths[i] + (chunk ? chunk[i] : 1) + block - 1) / block;
    for (int64_t b = 0; b < nblk; ++b)
      if (t[b] < 0 || (int64_t)t[b] * block + block - 1 > INT32_MAX) return LR_ERR_ARG;
  }

  int64_t nr = 0, tok = 0;
  off = 0;
  seq_off[0] = 0;
  for (int64_t i = 0; i < S; ++i) {
    const int32_t* t = tables + i * table_ld;
    const int64_t L = lengths[i], c = chunk ? chunk[i] : 1;
    const int64_t n = L + c;
    const int64_t nblk = (n + block - 1) / block;
    int64_t b = 0;
    while (b < nblk) {
      int64_t e = b + 1;
      while (e < nblk && t[e] == t[e - 1] + 1) ++e;
      const int64_t lo = b * block;
      const int64_t hi = (e * block < n) ? e * block : n;
      const int64_t src = (int64_t)t[b] * block;
      if (runs) {
        if (nr >= max_runs) return LR_ERR_CAPACITY;
        runs[3 * nr + 0] = (int32_t)src;
        runs[3 * nr + 1] = (int32_t)(off + lo);
        runs[3 * nr + 2] = (int32_t)(hi - lo);
      }
      for (int64_t p = lo; p < hi; ++p) remap[off + p] = (int32_t)(src + (p - lo));
      ++nr;
      b = e;
    }
    for (int64_t p = L; p < n; ++p, ++tok) {  // the new tokens, in position order
      if (tok_seq) tok_seq[tok] = (int32_t)i;
      pos[tok] = (int32_t)p;
      slot_mapping[tok] = (int32_t)((int64_t)t[p / block] * block + p % block);
    }
    off += n;
    seq_off[i + 1] = (int32_t)off;
  }
  for (int64_t j = off; j < cap; ++j) remap[j] = -1;
  *n_valid = (int32_t)off;
  *n_runs = (int32_t)nr;
  if (n_tokens) *n_tokens = (int32_t)tok;
  return LR_OK;
}

}  // namespace

extern "C" lr_status lowrank_prepare_decode(int64_t B, const int32_t* lengths,
                                            const int32_t* tables, int64_t table_ld,
                                            int64_t block, int64_t cap, int32_t* remap,
                                            int32_t* seq_off, int32_t* pos,
                                            int32_t* slot_mapping, int32_t* n_valid,
                                            int32_t* n_runs, int32_t* runs, int64_t max_runs) {
  return prepare(B, lengths, nullptr, tables, table_ld, block, cap, B, remap, seq_off, nullptr,
                 pos, slot_mapping, nullptr, n_valid, n_runs, runs, max_runs);
}

extern "C" lr_status lowrank_prepare_prefill(int64_t S, const int32_t* lengths,
                                             const int32_t* chunk, const int32_t* tables,
                                             int64_t table_ld, int64_t block, int64_t cap,
                                             int64_t max_tokens, int32_t* remap,
                                             int32_t* seq_off, int32_t* tok_seq, int32_t* pos,
                                             int32_t* slot_mapping, int32_t* n_tokens,
                                             int32_t* n_valid, int32_t* n_runs, int32_t* runs,
                                             int64_t max_runs) {
  if (!chunk || (S > 0 && !tok_seq) || !n_tokens) return LR_ERR_ARG;
  return prepare(S, lengths, chunk, tables, table_ld, block, cap, max_tokens, remap, seq_off,
                 tok_seq, pos, slot_mapping, n_tokens, n_valid, n_runs, runs, max_runs);
}
