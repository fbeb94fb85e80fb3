// Block selection for the sparse layer: query-block representatives, block scores against the
// pooled keys, and forced + top-k selection with lowest-index ties.
//
// Pages: "面壁智能发布MiniCPM-SALA：稀疏-线性混合架构，9B模型端侧跑通百万上下文，速度飙升3.5倍", section
// "SALA混合架构：黄金配比破解瓶颈" — a fine block-selection mechanism lets each query attend to only
// a small set of key/value pairs; "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" §1 —
// sliding-window and global-anchor sparsity (here: forced local blocks and forced block 0).
// Reading implemented: q~[g,i] = sum over the group's heads of the mean of the normalised
// queries of block i (decode: the single token); score[j] = q~ . k_pool[j] in fp32; keep the
// topk - |forced| best candidates j in [1, i - n_local], ties to the lowest index.
//
// Kernels: (1) qtilde_kernel — one pass over q; (2) prefill: score_tile_kernel (64x64 fp32
// tiles of q~ k_pool^T), then select_kernel — per row an exact radix select on monotone uint32
// keys of the scores and ordered compaction, so the output is ascending and deterministic;
// (3) decode (one query block): decode_slice_kernel scores slices of 512 candidates and keeps
// each slice's best (radix threshold, ties to the lower index), decode_merge_kernel selects
// among the slice winners and emits them ascending through a bitmap; very long ranges fall
// back to score_row_kernel + select_kernel.
#include "common.hpp"
#include "launch.hpp"

namespace sala {

namespace {

constexpr int NT = 256;

// grid (B, nqb); q~[b][g][r][DD] (fp32) = sum_{h in g} mean_t RMSNorm(q[t, h]) * w
template <typename T, int DD>
__global__ void __launch_bounds__(NT)
qtilde_kernel(const T* __restrict__ q, const float* __restrict__ qw, float* __restrict__ qt,
              int n_q, int Hq, int Hkv, long q0, float eps) {
  constexpr int EPL = 16 / (int)sizeof(T), LPR = DD / EPL, RPP = NT / LPR;
  __shared__ float hsum[64][DD];  // per-head sums for up to 64 heads
  const int b = blockIdx.x, r = blockIdx.y;
  const int j = threadIdx.x, hr = j / LPR, seg = j % LPR;
  // tokens of this query block inside the call: positions [64*(q0/64 + r), +64) clipped
  const long blk = q0 / 64 + r;
  const long p_lo = max(q0, blk * 64), p_hi = min(q0 + n_q, blk * 64 + 64);
  const float inv_cnt = 1.0f / (float)(p_hi - p_lo);
  for (int h0 = 0; h0 < Hq; h0 += RPP) {
    const int h = h0 + hr;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    if (h < Hq) {
      // 8 tokens' loads in flight before any of them is reduced
      for (long p0 = p_lo; p0 < p_hi; p0 += 8) {
        uint4 raw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const long p = p0 + u;
          raw[u] = p < p_hi ? *reinterpret_cast<const uint4*>(q + (((long)b * n_q + (p - q0)) * Hq + h) * DD + seg * EPL)
                            : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (p0 + u >= p_hi) break;  // uniform over the workgroup
          float x[EPL];
          if constexpr (sizeof(T) == 2) {
            unpack8(raw[u], x);
          } else {
            x[0] = __uint_as_float(raw[u].x); x[1] = __uint_as_float(raw[u].y);
            x[2] = __uint_as_float(raw[u].z); x[3] = __uint_as_float(raw[u].w);
          }
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) ss += x[e] * x[e];
          ss = group_sum<LPR>(ss);
          const float inv = 1.0f / sqrtf(ss / DD + eps);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] += x[e] * inv;
        }
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        hsum[h][seg * EPL + e] = acc[e] * inv_cnt * (qw ? qw[seg * EPL + e] : 1.0f);
    }
  }
  __syncthreads();
  const int G = Hq / Hkv;
  for (int idx = j; idx < Hkv * DD; idx += NT) {
    const int g = idx / DD, dd = idx % DD;
    float s = 0.f;
    for (int hh = 0; hh < G; ++hh) s += hsum[g * G + hh][dd];
    qt[(((long)b * Hkv + g) * gridDim.y + r) * DD + dd] = s;
  }
}

// Prefill scores: grid (B*Hkv, ceil(nqb/64), ceil(RL/64)); 64x64 tile, 4x4 per thread.
// sc[bg][r][j] = q~[bg][r] . k_pool[bg][j] for j <= qb0 + r - n_local (others untouched).
template <int DD>
__global__ void __launch_bounds__(NT)
score_tile_kernel(const float* __restrict__ qt, const float* __restrict__ kpool,
                  float* __restrict__ sc, int nqb, long qb0, int RL, long nblk_cap, int n_local) {
  __shared__ float sq[64][DD + 1];
  __shared__ float sk[64][DD + 1];
  const int bg = blockIdx.x;
  const int r0 = blockIdx.y * 64, j0 = blockIdx.z * 64;
  const long i_max = qb0 + min(nqb, r0 + 64) - 1;
  if (j0 > i_max - n_local) return;  // whole tile above the candidate range
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * DD; idx += NT) {
    const int rr = idx / DD, dd = idx % DD;
    sq[rr][dd] = (r0 + rr < nqb) ? qt[((long)bg * nqb + r0 + rr) * DD + dd] : 0.f;
    sk[rr][dd] = (j0 + rr < RL) ? kpool[((long)bg * nblk_cap + j0 + rr) * DD + dd] : 0.f;
  }
  __syncthreads();
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int dd = 0; dd < DD; ++dd) {
    float a[4], c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { a[u] = sq[ty * 4 + u][dd]; c[u] = sk[tx * 4 + u][dd]; }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[u][w] += a[u] * c[w];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = r0 + ty * 4 + u;
    if (r >= nqb) continue;
    const long lim = qb0 + r - n_local;  // last candidate block of row r
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int jj = j0 + tx * 4 + w;
      if (jj <= lim) sc[((long)bg * nqb + r) * RL + jj] = acc[u][w];
    }
  }
}

// One query block (decode): grid (B*Hkv, ceil(ncand/256)); 8 lanes per pooled key row.
template <int DD>
__global__ void __launch_bounds__(NT)
score_row_kernel(const float* __restrict__ qt, const float* __restrict__ kpool,
                 float* __restrict__ sc, int RL, long nblk_cap, long ncand_end) {
  constexpr int LPB = 8;              // lanes per pooled row
  constexpr int FPL = DD / LPB;       // floats per lane (16 or 8)
  const int bg = blockIdx.x;
  const int tid = threadIdx.x, sub = tid / LPB, part = tid % LPB;
  float qv[FPL];
#pragma unroll
  for (int e = 0; e < FPL; ++e) qv[e] = qt[(long)bg * DD + part * FPL + e];
  const long jbase = (long)blockIdx.y * 256;
  for (int it = 0; it < 256 / (NT / LPB); ++it) {
    const long jj = jbase + it * (NT / LPB) + sub;
    float s = 0.f;
    if (jj < ncand_end) {
      const float* row = kpool + ((long)bg * nblk_cap + jj) * DD + part * FPL;
#pragma unroll
      for (int e = 0; e < FPL; e += 4) {
        const float4 u = *reinterpret_cast<const float4*>(row + e);
        s += u.x * qv[e] + u.y * qv[e + 1] + u.z * qv[e + 2] + u.w * qv[e + 3];
      }
    }
    s = group_sum<LPB>(s);
    if (part == 0 && jj < ncand_end) sc[(long)bg * RL + jj] = s;
  }
}

// Histogram update of one wave: when every matching lane has the same digit (the common case
// for the leading digit of similar scores) one atomic adds the count; otherwise each lane adds
// its own (LDS atomics serialise only lanes that hit the same bin).
__device__ __forceinline__ void hist_add(int* hist, uint32_t dgt, bool match, int lane) {
  const uint64_t act = __ballot(match);
  if (act == 0) return;
  const int leader = __ffsll((unsigned long long)act) - 1;
  const uint32_t dl = __shfl(dgt, leader, 64);
  const uint64_t same = __ballot(match && dgt == dl);
  if (same == act) {
    if (lane == leader) atomicAdd(&hist[dl], __popcll(same));
  } else if (match) {
    atomicAdd(&hist[dgt], 1);
  }
}

template <int NTS>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < NTS / 64; ++w) { const int t = tmp[w]; tmp[w] = acc; acc += t; }
    tmp[NTS / 64] = acc;
  }
  __syncthreads();
  const int res = x - v + tmp[wave];
  *total = tmp[NTS / 64];
  __syncthreads();
  return res;
}

// grid (B*Hkv*nqb); row (bg, r) with i = qb0 + r. Exact top-r over candidate keys
// (score desc, index asc): MSB-first radix select over the 32-bit monotone keys (histograms
// updated by hist_add), then an ordered walk over blocks 0..i that emits
// forced and chosen blocks ascending; -1 pads to topk.
// CAP candidate keys are staged in LDS; rows with more candidates read the scores in global
// memory (correct, slower).
template <int NTS, int CAP>
__global__ void __launch_bounds__(NTS)
select_kernel(const float* __restrict__ sc, int32_t* __restrict__ sel, int nqb, long qb0, int RL,
              int topk, int n_local) {
  __shared__ uint32_t keys[CAP];
  __shared__ int hist[256];
  __shared__ int scan_tmp[NTS / 64 + 1];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const long row = blockIdx.x;
  const int r = (int)(row % nqb);
  const long i = qb0 + r;
  const float* srow = sc + row * RL;
  int32_t* out = sel + row * topk;
  const int tid = threadIdx.x, lane = tid & 63;
  const long nc = i - n_local > 0 ? i - n_local : 0;             // candidates j = 1..nc
  const long f_lo = i - n_local + 1 > 0 ? i - n_local + 1 : 0;   // forced local range [f_lo, i]
  const int n_forced = (int)(i - f_lo + 1) + (f_lo > 0 ? 1 : 0);
  const int rsel = topk - n_forced;
  const bool take_all = nc <= rsel;
  const bool in_lds = nc <= CAP;

  if (!take_all && in_lds)
    for (long jj = tid; jj < nc; jj += NTS) keys[jj] = score_key(srow[jj + 1]);
  __syncthreads();
  auto key_of = [&](long jj) -> uint32_t { return in_lds ? keys[jj - 1] : score_key(srow[jj]); };

  uint32_t T = 0;
  int need = 0;
  if (!take_all) {
    uint32_t prefix = 0, pmask = 0;
    int remaining = rsel;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int x = tid; x < 256; x += NTS) hist[x] = 0;
      __syncthreads();
      for (long base = 0; base < nc; base += NTS) {
        const long jj = 1 + base + tid;
        uint32_t key = 0;
        bool match = false;
        if (jj <= nc) {
          key = key_of(jj);
          match = (key & pmask) == prefix;
        }
        const uint32_t dgt = (key >> shift) & 255u;
        hist_add(hist, dgt, match, lane);
      }
      __syncthreads();
      if (tid < 64) {
        // digit with cum(digits > d) < remaining <= cum(digits >= d); lane l owns digits
        // 255-4l .. 252-4l (descending)
        int v[4], sum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = hist[255 - 4 * lane - e]; sum += v[e]; }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (lane >= o) incl += y;
        }
        const uint64_t hit = __ballot(incl >= remaining);
        const int L = __ffsll((unsigned long long)hit) - 1;  // first lane reaching the count
        if (hit == 0 && lane == 0) { s_prefix = prefix; s_need = remaining; }  // unreachable
        if (lane == L) {
          int cum = incl - sum;
          int e = 0;
          for (; e < 3; ++e) {
            if (cum + v[e] >= remaining) break;
            cum += v[e];
          }
          s_prefix = prefix | ((uint32_t)(255 - 4 * lane - e) << shift);
          s_need = remaining - cum;
        }
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_need;
      pmask |= 255u << shift;
    }
    T = prefix;
    need = remaining;  // how many candidates with key == T to keep (lowest indices first)
  }

  // ordered pass over blocks 0..i: each thread owns a contiguous index range
  const long nall = i + 1;
  const long per = (nall + NTS - 1) / NTS;
  const long a = tid * per, e_end = min(nall, a + per);
  int eq = 0;
  if (!take_all)
    for (long jj = max(a, 1L); jj < e_end && jj <= nc; ++jj) eq += (key_of(jj) == T);
  int eq_total;
  const int eq_before = block_excl_scan<NTS>(eq, scan_tmp, &eq_total);
  auto picked = [&](long jj, int& eqb) -> bool {
    if (jj == 0 || jj >= f_lo) return true;  // forced
    if (take_all) return true;              // 1 <= jj <= nc
    const uint32_t key = key_of(jj);
    if (key > T) return true;
    if (key == T) return (eqb++) < need;
    return false;
  };
  int cnt = 0;
  {
    int eqb = eq_before;
    for (long jj = a; jj < e_end; ++jj) cnt += picked(jj, eqb);
  }
  int total;
  int pos = block_excl_scan<NTS>(cnt, scan_tmp, &total);
  {
    int eqb = eq_before;
    for (long jj = a; jj < e_end; ++jj)
      if (picked(jj, eqb)) {
        if (pos < topk) out[pos] = (int32_t)jj;  // bounded even if the count were off
        ++pos;
      }
  }
  for (int k = total + tid; k < topk; k += NTS) out[k] = -1;
}

// ---- decode selection (one query block per row, long candidate ranges): two levels.
// Candidates are ordered by score, equal scores by lower index (a strict total order), so the
// best R of the whole range are among the best R of each slice. Level-1 winners are passed on
// as composites key(score) << 32 | (2^32 - 1 - j); composite 0 marks an empty entry (no score
// maps to key 0).
constexpr int DSL = 512;      // candidates per slice (level 1)
constexpr int DNSL_MAX = 32;  // slices per row handled by the merge
constexpr int DMERGE = 2048;  // slice winners the merge holds (nsl * R)
constexpr int DMERGE_NT = 1024;  // merge threads
constexpr int DBITS = DSL * DNSL_MAX / 32 + 1;  // bitmap words over candidate indices 0 .. nc

__device__ __forceinline__ uint64_t composite(uint32_t key, long j) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

// Exact threshold of the R largest of n keys in LDS (1 <= R < n): T = the R-th largest key and
// need = how many keys equal to T belong to the R largest. Four 8-bit radix passes; histogram
// updates by hist_add.
template <int NTH>
__device__ __forceinline__ void radix_threshold(const uint32_t* keys, int n, int R, int* hist,
                                                uint32_t* s_prefix, int* s_need, uint32_t& T,
                                                int& need) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, pmask = 0;
  int remaining = R;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int x = tid; x < 256; x += NTH) hist[x] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += NTH) {
      const int x = base + tid;
      uint32_t key = 0;
      bool match = false;
      if (x < n) {
        key = keys[x];
        match = (key & pmask) == prefix;
      }
      const uint32_t dgt = (key >> shift) & 255u;
      hist_add(hist, dgt, match, lane);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      int v[4], sum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = hist[255 - 4 * lane - e]; sum += v[e]; }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const uint64_t hit = __ballot(incl >= remaining);
      const int L = __ffsll((unsigned long long)hit) - 1;
      if (lane == L) {
        int cum = incl - sum;
        int e = 0;
        for (; e < 3; ++e) {
          if (cum + v[e] >= remaining) break;
          cum += v[e];
        }
        *s_prefix = prefix | ((uint32_t)(255 - 4 * lane - e) << shift);
        *s_need = remaining - cum;
      }
    }
    __syncthreads();
    prefix = *s_prefix;
    remaining = *s_need;
    pmask |= 255u << shift;
  }
  T = prefix;
  need = remaining;
}

// the candidate count of sequence b when sequences sit at their own cache lengths kv_lens[b]
// (clamped to [1, kv_max]): blocks 1 .. i - n_local of its query block i
__device__ __forceinline__ long decode_candidates(const int64_t* kv_lens, int b, long kv_max, int n_local, long* i) {
  long kv = kv_lens[b];
  kv = kv < 1 ? 1 : (kv > kv_max ? kv_max : kv);
  *i = (kv - 1) / 64;
  return *i - n_local > 0 ? *i - n_local : 0;
}

// q~ of a single query token for KV group g (decode): the sum over the group's heads of
// RMSNorm(q[b, h]) * w, with the arithmetic of qtilde_kernel for one token (16 lanes per head
// row, heads summed in order), into qs[DD]. NT threads; hsum holds 16 head rows.
template <typename T, int DD>
__device__ __forceinline__ void decode_qtilde(const T* __restrict__ q, const float* __restrict__ qw, int b, int g,
                                              int Hq, int Hkv, float eps, float (*hsum)[DD], float* qs) {
  constexpr int EPL = 16 / (int)sizeof(T), LPR = DD / EPL, RPP = NT / LPR;
  const int j = threadIdx.x, hr = j / LPR, seg = j % LPR;
  const int G = Hq / Hkv;
  float tot = 0.f;  // thread j < DD: running sum over the group's heads of dim j
  for (int h0 = 0; h0 < G; h0 += RPP) {
    const int hh = h0 + hr;
    if (hh < G) {
      const T* src = q + ((long)b * Hq + g * G + hh) * DD + seg * EPL;
      float x[EPL];
      if constexpr (sizeof(T) == 2) {
        unpack8(*reinterpret_cast<const uint4*>(src), x);
      } else {
        const float4 u = *reinterpret_cast<const float4*>(src);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss += x[e] * x[e];
      ss = group_sum<LPR>(ss);
      const float inv = 1.0f / sqrtf(ss / DD + eps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) hsum[hr][seg * EPL + e] = x[e] * inv * 1.0f * (qw ? qw[seg * EPL + e] : 1.0f);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) hsum[hr][seg * EPL + e] = 0.f;
    }
    __syncthreads();
    if (j < DD)
      for (int r = 0; r < RPP && h0 + r < G; ++r) tot += hsum[r][j];
    __syncthreads();
  }
  if (j < DD) qs[j] = tot;
  __syncthreads();
}

// Level 1: grid (B*Hkv, nsl), NT threads. Slice s holds candidates j = j0 .. j0+n-1 with
// j0 = 1 + s*DSL, n = min(DSL, nc - j0 + 1): scores q~ . k_pool[j] (8 lanes per pooled row),
// then the slice's best R as composites into cand[bg][s][0..R) (0-padded, unordered). With
// kv_lens, nc is each sequence's own count (at most the nc given). q~ of the single query token
// is computed here (decode_qtilde) from q [B, Hq, DD].
template <typename QT, int DD>
__global__ void __launch_bounds__(NT)
decode_slice_kernel(const QT* __restrict__ q, const float* __restrict__ qw, int Hq, float eps,
                    const float* __restrict__ kpool, uint64_t* __restrict__ cand, long nblk_cap, long nc, int R,
                    const int64_t* __restrict__ kv_lens, int Hkv, long kv_max, int n_local) {
  constexpr int LPB = 8, FPL = DD / LPB, RPI = NT / LPB;  // rows per iteration
  __shared__ uint32_t keys[DSL];
  __shared__ int hist[256];
  __shared__ int scan_tmp[NT / 64 + 1];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  __shared__ float hsum[NT / (DD / (16 / (int)sizeof(QT)))][DD];
  __shared__ float qs[DD];
  const int bg = blockIdx.x, sl = blockIdx.y, nsl = gridDim.y;
  const int tid = threadIdx.x, sub = tid / LPB, part = tid % LPB;
  decode_qtilde<QT, DD>(q, qw, bg / Hkv, bg % Hkv, Hq, Hkv, eps, hsum, qs);
  if (kv_lens) {
    long i;
    const long ncb = decode_candidates(kv_lens, bg / Hkv, kv_max, n_local, &i);
    nc = ncb < nc ? ncb : nc;
  }
  const long j0 = 1 + (long)sl * DSL;
  const int n = (int)max(0L, min((long)DSL, nc - j0 + 1));
  float qv[FPL];
#pragma unroll
  for (int e = 0; e < FPL; ++e) qv[e] = qs[part * FPL + e];
  const float* kb = kpool + ((long)bg * nblk_cap + j0) * DD + part * FPL;
  if (n > 0) {
    // the rows stream in batches of BT iterations, the next batch's loads issued before the
    // current batch is reduced (rows past the slice repeat its last row; their keys are never
    // read)
    constexpr int IT = DSL / RPI, BT = 4;
    float4 buf[2][BT][FPL / 4];
    auto load = [&](int bt, int slot) {
#pragma unroll
      for (int u = 0; u < BT; ++u) {
        const int x = (bt * BT + u) * RPI + sub;
        const float* row = kb + (long)(x < n ? x : n - 1) * DD;
#pragma unroll
        for (int e = 0; e < FPL / 4; ++e) buf[slot][u][e] = *reinterpret_cast<const float4*>(row + 4 * e);
      }
    };
    load(0, 0);
#pragma unroll
    for (int bt = 0; bt < IT / BT; ++bt) {
      if (bt + 1 < IT / BT) load(bt + 1, (bt + 1) & 1);
#pragma unroll
      for (int u = 0; u < BT; ++u) {
        float sdot = 0.f;
#pragma unroll
        for (int e = 0; e < FPL / 4; ++e) {
          const float4 w = buf[bt & 1][u][e];
          sdot += w.x * qv[4 * e] + w.y * qv[4 * e + 1] + w.z * qv[4 * e + 2] + w.w * qv[4 * e + 3];
        }
        sdot = group_sum<LPB>(sdot);
        if (part == 0) keys[(bt * BT + u) * RPI + sub] = score_key(sdot);
      }
    }
  }
  __syncthreads();
  uint64_t* dst = cand + ((long)bg * nsl + sl) * R;
  if (n <= R) {
    for (int t = tid; t < R; t += NT) dst[t] = t < n ? composite(keys[t], j0 + t) : 0ull;
    return;
  }
  uint32_t T;
  int need;
  radix_threshold<NT>(keys, n, R, hist, &s_prefix, &s_need, T, need);
  // keys above T, then the first `need` keys equal to T in index order: thread t owns
  // positions PER*t .. PER*t + PER-1
  constexpr int PER = DSL / NT;
  int eq = 0, gt = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int x = PER * tid + u;
    if (x < n) { eq += keys[x] == T; gt += keys[x] > T; }
  }
  int eq_total;
  int eqb = block_excl_scan<NT>(eq, scan_tmp, &eq_total);
  int cnt = gt + max(0, min(eq, need - eqb));
  int total;
  int pos = block_excl_scan<NT>(cnt, scan_tmp, &total);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int x = PER * tid + u;
    if (x >= n) continue;
    const uint32_t key = keys[x];
    const bool pick = key > T || (key == T && (eqb++) < need);
    if (pick && pos < R) dst[pos++] = composite(key, j0 + x);
  }
}

// Second-stage keys for surplus ties at threshold T: keys above T become 0xFFFFFFFF (always
// kept), keys equal to T become ~index (larger for lower indices), the rest 0.
__device__ __forceinline__ void idx2key(uint32_t* keys, const uint32_t* idx, int t, uint32_t T) {
  const uint32_t k = keys[t];
  keys[t] = k > T ? 0xFFFFFFFFu : (k == T ? ~idx[t] : 0u);
}

// Level 2: grid (B*Hkv), NT threads. The best R of the nsl*R slice winners (empties excluded),
// then the output row: forced block 0 (if outside the local range), the chosen candidates
// ascending (a bitmap over candidate indices compacted in order), the forced local blocks
// f_lo .. i, and -1 padding.
template <int CAPB, int NTM>
__global__ void __launch_bounds__(NTM)
decode_merge_kernel(const uint64_t* __restrict__ cand, int32_t* __restrict__ sel, int nsl, int R,
                    long i, int n_local, int topk, long nc, const int64_t* __restrict__ kv_lens, int Hkv,
                    long kv_max) {
  __shared__ uint32_t keys[CAPB];
  __shared__ uint32_t idx[CAPB];
  __shared__ uint32_t bits[DBITS];
  __shared__ int hist[256];
  __shared__ int scan_tmp[NTM / 64 + 1];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int bg = blockIdx.x, tid = threadIdx.x;
  const int n = nsl * R;
  if (kv_lens) {  // this sequence's query block and candidate count (at most the nc given)
    const long ncb = decode_candidates(kv_lens, bg / Hkv, kv_max, n_local, &i);
    nc = ncb < nc ? ncb : nc;
  }
  int valid = 0;
  for (int t = tid; t < n; t += NTM) {
    const uint64_t c = cand[(long)bg * n + t];
    keys[t] = (uint32_t)(c >> 32);
    idx[t] = 0xFFFFFFFFu - (uint32_t)c;
    valid += c != 0ull;
  }
  const int nw = (int)(nc / 32) + 1;  // bitmap words over indices 0 .. nc
  for (int w = tid; w < nw; w += NTM) bits[w] = 0u;
  int n_valid;
  block_excl_scan<NTM>(valid, scan_tmp, &n_valid);  // also orders the fills above
  uint32_t T = 0, T2 = 0;
  int need = 0;
  const bool all = n_valid <= R;
  bool all_ties = true;
  if (!all) {
    radix_threshold<NTM>(keys, n, R, hist, &s_prefix, &s_need, T, need);
    int ties = 0;
    for (int t = tid; t < n; t += NTM) ties += keys[t] == T;
    int ties_total;
    block_excl_scan<NTM>(ties, scan_tmp, &ties_total);
    all_ties = ties_total == need;  // the usual case: no surplus equal scores
    if (!all_ties) {
      // surplus ties: keep the `need` lowest indices. After idx2key the R largest keys are the
      // R - need keys above T (all ones) and the ties with the `need` largest ~index; indices
      // are distinct, so the R-th largest T2 separates them exactly.
      __syncthreads();
      for (int t = tid; t < n; t += NTM) idx2key(keys, idx, t, T);
      __syncthreads();
      int need2;
      radix_threshold<NTM>(keys, n, R, hist, &s_prefix, &s_need, T2, need2);
    }
  }
  for (int t = tid; t < n; t += NTM) {
    bool pick;
    if (all) pick = keys[t] != 0u;
    else if (all_ties) pick = keys[t] >= T;
    else pick = keys[t] >= T2;
    if (pick && idx[t] <= (uint32_t)nc) atomicOr(&bits[idx[t] >> 5], 1u << (idx[t] & 31));
  }
  __syncthreads();
  const long f_lo = i - n_local + 1 > 0 ? i - n_local + 1 : 0;
  const int head = f_lo > 0 ? 1 : 0;
  int32_t* out = sel + (long)bg * topk;
  // thread t owns bitmap words wpt*t .. wpt*t + wpt-1
  const int wpt = (nw + NTM - 1) / NTM;
  int c = 0;
  for (int w = wpt * tid; w < min(nw, wpt * tid + wpt); ++w) c += __popc(bits[w]);
  int cnt;
  int pos = head + block_excl_scan<NTM>(c, scan_tmp, &cnt);
  for (int w = wpt * tid; w < min(nw, wpt * tid + wpt); ++w) {
    uint32_t m = bits[w];
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      if (pos < topk) out[pos] = 32 * w + b;
      ++pos;
    }
  }
  if (tid == 0 && head) out[0] = 0;
  const int nloc = (int)(i - f_lo + 1);
  for (int t = tid; t < nloc; t += NTM)
    if (head + cnt + t < topk) out[head + cnt + t] = (int32_t)(f_lo + t);
  for (int t = head + cnt + nloc + tid; t < topk; t += NTM) out[t] = -1;
}

}  // namespace

static long select_row_len(const sala_sparse_desc& d) {
  const SparseGeom g = sparse_geom(d);
  return g.qb0 + g.nqb;  // blocks 0 .. i_max
}

// decode (one query block) uses the two-level selection while the candidates fit DNSL_MAX
// slices; it needs nsl * R composites per row instead of the score row
static bool decode_two_level(const sala_sparse_desc& d, long* nc_out, int* nsl_out, int* r_out) {
  const SparseGeom g = sparse_geom(d);
  if (g.nqb != 1) return false;
  const long i = g.qb0;
  const long nc = i - d.n_local > 0 ? i - d.n_local : 0;
  const long f_lo = i - d.n_local + 1 > 0 ? i - d.n_local + 1 : 0;
  const int n_forced = (int)(i - f_lo + 1) + (f_lo > 0 ? 1 : 0);
  const int R = d.topk - n_forced;
  const long nsl = (nc + DSL - 1) / DSL;
  if (nc < 1 || R < 1 || nsl > DNSL_MAX || nsl * R > DMERGE) return false;
  *nc_out = nc; *nsl_out = (int)nsl; *r_out = R;
  return true;
}

size_t block_select_workspace(const sala_sparse_desc& d) {
  const SparseGeom g = sparse_geom(d);
  const size_t bg = (size_t)d.batch * d.n_kv_heads;
  const size_t qt = bg * g.nqb * d.head_dim * sizeof(float);
  size_t sc = bg * g.nqb * select_row_len(d) * sizeof(float);
  long nc; int nsl, R;
  if (decode_two_level(d, &nc, &nsl, &R)) sc = bg * (size_t)nsl * R * sizeof(uint64_t);
  return ((qt + 255) & ~(size_t)255) + sc;
}

// level 1 of the decode selection (q~ computed inside), for the descriptor's dtype and dim
static void launch_decode_slice(const sala_sparse_desc& d, const void* q, const float* qw, const float* k_pool,
                                uint64_t* cand, long nblk_cap, long nc, int R, int nsl, const int64_t* kv_lens,
                                hipStream_t st) {
  const dim3 grid(d.batch * d.n_kv_heads, nsl);
#define SALA_SLICE(T, DD)                                                                                   \
  hipLaunchKernelGGL((decode_slice_kernel<T, DD>), grid, dim3(NT), 0, st, (const T*)q, qw, d.n_heads, d.norm_eps, \
                     k_pool, cand, nblk_cap, nc, R, kv_lens, d.n_kv_heads, (long)d.kv_len, d.n_local)
  if (d.dtype == SALA_BF16) {
    if (d.head_dim == 128) SALA_SLICE(bf16_t, 128); else SALA_SLICE(bf16_t, 64);
  } else {
    if (d.head_dim == 128) SALA_SLICE(float, 128); else SALA_SLICE(float, 64);
  }
#undef SALA_SLICE
}

hipError_t launch_block_select(const sala_sparse_desc& d, const void* q, const float* qw,
                               const float* k_pool, int32_t* sel, void* ws, hipStream_t st) {
  const SparseGeom g = sparse_geom(d);
  const int BG = d.batch * d.n_kv_heads;
  const long RL = select_row_len(d);
  float* qt = static_cast<float*>(ws);
  const size_t qt_bytes = (size_t)BG * g.nqb * d.head_dim * sizeof(float);
  float* sc = reinterpret_cast<float*>(static_cast<char*>(ws) + ((qt_bytes + 255) & ~(size_t)255));
  const long i_max = g.qb0 + g.nqb - 1;
  long nc; int nsl, R;
  if (decode_two_level(d, &nc, &nsl, &R)) {
    uint64_t* cand = reinterpret_cast<uint64_t*>(sc);
    launch_decode_slice(d, q, qw, k_pool, cand, g.nblk_cap, nc, R, nsl, nullptr, st);
    hipLaunchKernelGGL((decode_merge_kernel<DMERGE, DMERGE_NT>), dim3(BG), dim3(DMERGE_NT), 0, st, cand, sel, nsl, R,
                       i_max, d.n_local, d.topk, nc, nullptr, d.n_kv_heads, (long)d.kv_len);
    return hipGetLastError();
  }
  const dim3 gq(d.batch, (unsigned)g.nqb);
#define SALA_QT(T, DD)                                                                             \
  hipLaunchKernelGGL((qtilde_kernel<T, DD>), gq, dim3(NT), 0, st, (const T*)q, qw, qt, d.n_q,      \
                     d.n_heads, d.n_kv_heads, (long)g.q0, d.norm_eps)
  if (d.dtype == SALA_BF16) {
    if (d.head_dim == 128) SALA_QT(bf16_t, 128); else SALA_QT(bf16_t, 64);
  } else {
    if (d.head_dim == 128) SALA_QT(float, 128); else SALA_QT(float, 64);
  }
#undef SALA_QT
  if (i_max - d.n_local >= 1) {
    if (g.nqb == 1) {
      const long ncand_end = i_max - d.n_local + 1;  // score blocks 0 .. i - n_local
      const dim3 gs(BG, (unsigned)((ncand_end + 255) / 256));
      if (d.head_dim == 128)
        hipLaunchKernelGGL(score_row_kernel<128>, gs, dim3(NT), 0, st, qt, k_pool, sc, (int)RL,
                           (long)g.nblk_cap, ncand_end);
      else
        hipLaunchKernelGGL(score_row_kernel<64>, gs, dim3(NT), 0, st, qt, k_pool, sc, (int)RL,
                           (long)g.nblk_cap, ncand_end);
    } else {
      const dim3 gs(BG, (unsigned)((g.nqb + 63) / 64), (unsigned)((RL + 63) / 64));
      if (d.head_dim == 128)
        hipLaunchKernelGGL(score_tile_kernel<128>, gs, dim3(NT), 0, st, qt, k_pool, sc, (int)g.nqb,
                           (long)g.qb0, (int)RL, (long)g.nblk_cap, d.n_local);
      else
        hipLaunchKernelGGL(score_tile_kernel<64>, gs, dim3(NT), 0, st, qt, k_pool, sc, (int)g.nqb,
                           (long)g.qb0, (int)RL, (long)g.nblk_cap, d.n_local);
    }
  }
  // long rows (decode past the two-level range, prefill beyond 4,096 candidate blocks): 1024
  // threads and 16,384 keys in LDS per row; shorter rows: 256 threads, 4,096 keys
  if (g.nqb == 1 || RL > 4096)
    hipLaunchKernelGGL((select_kernel<1024, 16384>), dim3((unsigned)(BG * g.nqb)), dim3(1024), 0, st, sc, sel,
                       (int)g.nqb, (long)g.qb0, (int)RL, d.topk, d.n_local);
  else
    hipLaunchKernelGGL((select_kernel<256, 4096>), dim3((unsigned)(BG * g.nqb)), dim3(256), 0, st, sc, sel,
                       (int)g.nqb, (long)g.qb0, (int)RL, d.topk, d.n_local);
  return hipGetLastError();
}

}  // namespace sala

namespace sala {

// ---- decode selection with each sequence at its own cache length (device array kv_lens,
// clamped to [1, desc kv_len]): always the two-level path, sized for the longest context.
// Returns false if that context is beyond the two-level range.
static bool decode_at_plan(const sala_sparse_desc& d, long* nc, int* nsl, int* R) {
  const long i_max = (d.kv_len - 1) / 64;
  *nc = i_max - d.n_local > 0 ? i_max - d.n_local : 0;
  *R = i_max >= d.n_local ? d.topk - d.n_local - 1 : d.topk - (int)(i_max + 1);
  *nsl = (int)((*nc + DSL - 1) / DSL);
  if (*nsl < 1) *nsl = 1;
  if (*R < 1) *R = 1;
  return *nsl <= DNSL_MAX && (long)*nsl * *R <= DMERGE && *nc / 32 + 1 <= DBITS;
}

size_t block_select_decode_at_workspace(const sala_sparse_desc& d) {
  long nc; int nsl, R;
  if (!decode_at_plan(d, &nc, &nsl, &R)) return SIZE_MAX;
  const size_t bg = (size_t)d.batch * d.n_kv_heads;
  const size_t qt = bg * d.head_dim * sizeof(float);
  return ((qt + 255) & ~(size_t)255) + bg * (size_t)nsl * R * sizeof(uint64_t);
}

hipError_t launch_block_select_decode_at(const sala_sparse_desc& d, const int64_t* kv_lens, const void* q,
                                         const float* qw, const float* k_pool, int32_t* sel, void* ws,
                                         hipStream_t st) {
  long nc; int nsl, R;
  if (!decode_at_plan(d, &nc, &nsl, &R)) return hipErrorInvalidValue;
  const int BG = d.batch * d.n_kv_heads;
  const size_t qt_bytes = (size_t)BG * d.head_dim * sizeof(float);
  uint64_t* cand = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + ((qt_bytes + 255) & ~(size_t)255));
  const long nblk_cap = d.kv_capacity / 64;
  launch_decode_slice(d, q, qw, k_pool, cand, nblk_cap, nc, R, nsl, kv_lens, st);
  hipLaunchKernelGGL((decode_merge_kernel<DMERGE, DMERGE_NT>), dim3(BG), dim3(DMERGE_NT), 0, st, cand, sel, nsl, R,
                     (long)((d.kv_len - 1) / 64), d.n_local, d.topk, nc, kv_lens, d.n_kv_heads, (long)d.kv_len);
  return hipGetLastError();
}

}  // namespace sala
