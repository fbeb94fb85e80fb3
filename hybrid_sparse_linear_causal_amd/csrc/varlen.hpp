// Packed variable-length batches ("varlen"): nseq sequences stored back to back along the token
// dimension (activations [T, H, d], T = the sum of their token counts), each with its own token
// count and start position (the number of its tokens already processed by earlier calls). The
// host builds a VarlenTable from the caller's host arrays and passes it to the kernels by value
// as a kernel argument, so that no table has to be copied into device memory.
#pragma once

#include "launch.hpp"

namespace sala {

constexpr int VL_MAXS = SALA_VARLEN_MAX_SEQS;

struct VarlenTable {
  int nseq;
  int item0[VL_MAXS + 1];  // prefix over the sequences of a kernel-specific work-item count
  int aux0[VL_MAXS + 1];   // prefix over the sequences of a kernel-specific count (slots, rows)
  int n[VL_MAXS];          // token count
  int tok0[VL_MAXS];       // packed index of the first token
  long pos0[VL_MAXS];      // position of the first token
};

// the sequence whose work items contain item x: the last s with item0[s] <= x (sequences
// without items are skipped because their item0 equals the next one's)
__device__ __forceinline__ int vl_seq(const VarlenTable& t, int x) {
  int lo = 0, hi = t.nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.item0[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// host: a table of the sequences' counts and positions (item0, aux0 left at zero)
inline VarlenTable make_varlen_table(int nseq, const int32_t* cu_seqlens, const int64_t* pos0) {
  VarlenTable t{};
  t.nseq = nseq;
  for (int s = 0; s < nseq; ++s) {
    t.tok0[s] = cu_seqlens[s];
    t.n[s] = cu_seqlens[s + 1] - cu_seqlens[s];
    t.pos0[s] = pos0 ? pos0[s] : 0;
  }
  return t;
}

}  // namespace sala
