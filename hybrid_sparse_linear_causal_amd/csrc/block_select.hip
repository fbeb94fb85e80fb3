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
// (3) decode (one query block): decode_slice_kernel scores slices of 512 candidates (chunks of
// 32 dealt round-robin) and keeps each slice's best as score/index composites (up to 64 of them
// by bitonic networks across the lanes, sorted; more by a radix threshold, ties to the lower
// index); decode_merge64_kernel (networks over the sorted lists) or decode_merge_kernel (radix,
// a bitmap for the ascending order) selects among the slice winners and emits the row; very long
// ranges fall back to score_row_kernel + select_kernel.
#include <algorithm>

#include "common.hpp"
#include "kv_append.hpp"
#include "launch.hpp"
#include "varlen.hpp"

namespace sala {

namespace {

constexpr int NT = 256;

// the score a monotone key was made from (inverse of score_key)
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// q~ of query block r of one sequence's call, by a workgroup of NT threads: for each KV group g,
// q~[g] = sum_{h in g} mean_t RMSNorm(q[t, h]) * w over the call's tokens t of the block, stored
// at qt_r[g * g_stride .. + DD). q: the sequence's first call token, [n_q, Hq, DD].
template <typename T, int DD>
__device__ __forceinline__ void qtilde_block(const T* __restrict__ q, const float* __restrict__ qw,
                                             float* __restrict__ qt_r, long g_stride, int n_q, int Hq, int Hkv,
                                             long q0, long r, float eps, float (*hsum)[DD]) {
  constexpr int EPL = 16 / (int)sizeof(T), LPR = DD / EPL, RPP = NT / LPR;
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
          raw[u] = p < p_hi ? *reinterpret_cast<const uint4*>(q + ((p - q0) * Hq + h) * DD + seg * EPL)
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
    qt_r[g * g_stride + dd] = s;
  }
}

// grid (B, nqb); q~[b][g][r][DD] (fp32)
template <typename T, int DD>
__global__ void __launch_bounds__(NT)
qtilde_kernel(const T* __restrict__ q, const float* __restrict__ qw, float* __restrict__ qt,
              int n_q, int Hq, int Hkv, long q0, float eps) {
  __shared__ float hsum[64][DD];  // per-head sums for up to 64 heads
  const int b = blockIdx.x, r = blockIdx.y, nqb = gridDim.y;
  qtilde_block<T, DD>(q + (long)b * n_q * Hq * DD, qw, qt + ((long)b * Hkv * nqb + r) * DD, (long)nqb * DD, n_q, Hq,
                      Hkv, q0, r, eps, hsum);
}

// Packed batch: grid (sum of the sequences' query blocks); item x of sequence s (t.item0 the
// prefix of their query-block counts) is its query block x - t.item0[s]; sequence s's q~ sits at
// qt + Hkv * t.item0[s] * DD as [g][r][DD], the layout of a one-sequence call.
template <typename T, int DD>
__global__ void __launch_bounds__(NT)
qtilde_varlen_kernel(const T* __restrict__ q, const float* __restrict__ qw, float* __restrict__ qt, int Hq, int Hkv,
                     float eps, VarlenTable t) {
  __shared__ float hsum[64][DD];
  const int s = vl_seq(t, blockIdx.x), r = blockIdx.x - t.item0[s];
  const long nqb = t.item0[s + 1] - t.item0[s];
  qtilde_block<T, DD>(q + (long)t.tok0[s] * Hq * DD, qw, qt + ((long)Hkv * t.item0[s] + r) * DD, nqb * DD, t.n[s],
                      Hq, Hkv, t.pos0[s], r, eps, hsum);
}

// Prefill scores: grid (B*Hkv, ceil(nqb/64), ceil(RL/64)); 64x64 tile, 4x4 per thread.
// sc[bg][r][j] = q~[bg][r] . k_pool[bg][j] for j <= qb0 + r - n_local (others untouched). The
// tiles sit row-major in LDS with rows DD + 4 floats apart, so the 16 lanes that read one dims
// quad of 16 different rows hit 16 different bank quads; each thread reads its 4 rows and 4
// candidates a dims quad at a time (8 float4 reads per 64 FMAs) and sums over the dims in order.
template <int DD>
__global__ void __launch_bounds__(NT)
score_tile_kernel(const float* __restrict__ qt, const float* __restrict__ kpool,
                  float* __restrict__ sc, int nqb, long qb0, int RL, long nblk_cap, int n_local) {
  constexpr int ST = DD + 4;
  __shared__ __align__(16) float sq[64 * ST];
  __shared__ __align__(16) float sk[64 * ST];
  const int bg = blockIdx.x;
  const int r0 = blockIdx.y * 64, j0 = blockIdx.z * 64;
  const long i_max = qb0 + min(nqb, r0 + 64) - 1;
  if (j0 > i_max - n_local) return;  // whole tile above the candidate range
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * DD / 4; idx += NT) {
    const int rr = idx / (DD / 4), d4 = idx % (DD / 4);
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(&sq[rr * ST + 4 * d4]) =
        (r0 + rr < nqb) ? *reinterpret_cast<const float4*>(&qt[((long)bg * nqb + r0 + rr) * DD + 4 * d4]) : zero;
    *reinterpret_cast<float4*>(&sk[rr * ST + 4 * d4]) =
        (j0 + rr < RL) ? *reinterpret_cast<const float4*>(&kpool[((long)bg * nblk_cap + j0 + rr) * DD + 4 * d4]) : zero;
  }
  __syncthreads();
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int dd = 0; dd < DD; dd += 4) {
    float4 a[4], c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = *reinterpret_cast<const float4*>(&sq[(ty * 4 + u) * ST + dd]);
      c[u] = *reinterpret_cast<const float4*>(&sk[(tx * 4 + u) * ST + dd]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float t = acc[u][w];
        t += a[u].x * c[w].x;
        t += a[u].y * c[w].y;
        t += a[u].z * c[w].z;
        t += a[u].w * c[w].w;
        acc[u][w] = t;
      }
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
  const int x = wave_incl_scan(v);
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
select_kernel(const float* __restrict__ sc, int32_t* __restrict__ sel, float* __restrict__ sel_sc, int nqb,
              long qb0, int RL, int topk, int n_local) {
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
  float* out_sc = sel_sc ? sel_sc + row * topk : nullptr;
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
        const int incl = wave_incl_scan(sum);
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
        if (pos < topk) {  // bounded even if the count were off
          out[pos] = (int32_t)jj;
          if (out_sc) out_sc[pos] = (jj == 0 || jj >= f_lo) ? INFINITY : srow[jj];  // forced: +inf
        }
        ++pos;
      }
  }
  for (int k = total + tid; k < topk; k += NTS) {
    out[k] = -1;
    if (out_sc) out_sc[k] = -INFINITY;
  }
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

// ---- bitonic networks over the 64 lanes of a wave (64-bit values). Composites key << 32 | ~j
// are distinct, so sorting them orders candidates by score with ties to the lower index; empty
// slots (0) sort last.

// the value of lane l ^ m (m a power of two, constant after unrolling): DPP moves within rows of
// 16 lanes for m <= 8 (quad permutations for 1 and 2, shifts by 4 either way, a rotation by 8);
// for 16 and 32 the row swaps of gfx950 with x as both operands (the 16-lane swap exchanges the
// odd rows of the first with the even rows of the second, the 32-lane swap the upper half of the
// first with the lower half of the second, so one of the two results holds each lane's partner)
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int m) {
  if (m == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  }
  if (m == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
  const int v = (int)x;
  if (m == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  if (m == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  if (m == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);  // row_shl:4 (lane + 4)
    const int dn = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4 (lane - 4)
    return (uint32_t)((threadIdx.x & 4) ? dn : up);
  }
  if (m == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  return (uint32_t)__shfl_xor(v, m, 64);
}
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m) {
  const uint32_t lo = xor_lane((uint32_t)x, m), hi = xor_lane((uint32_t)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
// one compare-exchange of a network over the 64 lanes: pairs (l, l ^ m); keep_max: this lane
// keeps the larger of the pair
__device__ __forceinline__ uint64_t cmp_x(uint64_t x, int m, bool keep_max) {
  const uint64_t y = shfl_xor64(x, m);
  return ((x < y) == keep_max) ? y : x;
}
// sort the wave's 64 values: descending (lane 0 the largest) or ascending
__device__ __forceinline__ uint64_t wave_sort64(uint64_t x, bool descending) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k *= 2)
#pragma unroll
    for (int m = k / 2; m > 0; m /= 2) {
      const bool desc = ((l & k) == 0) == descending;  // this block's direction (all of it at k = 64)
      x = cmp_x(x, m, ((l & m) == 0) == desc);
    }
  return x;
}
// a bitonic sequence over the 64 lanes, sorted descending
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t x) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int m = 32; m > 0; m /= 2) x = cmp_x(x, m, (l & m) == 0);
  return x;
}


// Exact threshold of the R largest of n keys in LDS (1 <= R < n): T = the R-th largest key and
// need = how many keys equal to T belong to the R largest. Four 8-bit radix passes; histogram
// updates by hist_add. EARLY: when the digit bucket that holds the R-th largest is needed whole
// (the usual case after two passes over distinct scores), stop there with T = the largest key
// below that bucket and need = 0, so that the R largest are exactly the keys above T (a caller
// that keeps keys == T by count still takes none, as need is 0).
template <int NTH, bool EARLY>
__device__ __forceinline__ void radix_threshold(const uint32_t* keys, int n, int R, int* hist,
                                                uint32_t* s_prefix, int* s_need, int* s_cnt, uint32_t& T,
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
      const int incl = wave_incl_scan(sum);
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
        *s_cnt = v[e];
      }
    }
    __syncthreads();
    prefix = *s_prefix;
    remaining = *s_need;
    pmask |= 255u << shift;
    if (EARLY && pass < 3 && *s_cnt == remaining && prefix != 0u) {  // uniform: read after the barrier
      T = prefix - 1u;  // the low bits of prefix are 0: every key of the bucket is above T
      need = 0;
      return;
    }
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
// row, heads summed in order), into qs[DD]. NT threads; hsum holds 16 head rows. `issued` runs
// once the first rows' loads are issued (the caller's own loads queue behind them, so waiting
// for the q rows does not wait for those).
template <typename T, int DD, class F>
__device__ __forceinline__ void decode_qtilde(const T* __restrict__ q, const float* __restrict__ qw, int b, int g,
                                              int Hq, int Hkv, float eps, float (*hsum)[DD], float* qs, F&& issued) {
  constexpr int EPL = 16 / (int)sizeof(T), LPR = DD / EPL, RPP = NT / LPR;
  const int j = threadIdx.x, hr = j / LPR, seg = j % LPR;
  const int G = Hq / Hkv;
  // rows past the group read the group's last head (in bounds) and count as zero; the loads
  // are unconditional so that the caller's loads issued after the first ones can stay in flight
  auto ld = [&](int h0) {
    const int hh = min(h0 + hr, G - 1);
    return *reinterpret_cast<const uint4*>(q + ((long)b * Hq + g * G + hh) * DD + seg * EPL);
  };
  float tot = 0.f;  // thread j < DD: running sum over the group's heads of dim j
  auto heads = [&](uint4 raw, int h0) {
    const bool valid = h0 + hr < G;
    float x[EPL];
    if constexpr (sizeof(T) == 2) {
      unpack8(raw, x);
    } else {
      x[0] = __uint_as_float(raw.x); x[1] = __uint_as_float(raw.y);
      x[2] = __uint_as_float(raw.z); x[3] = __uint_as_float(raw.w);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss += x[e] * x[e];
    ss = group_sum<LPR>(ss);
    const float inv = valid ? 1.0f / sqrtf(ss / DD + eps) : 0.f;
    float wv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) wv[e] = 1.0f;
    if (qw) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) wv[e] = qw[seg * EPL + e];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) hsum[hr][seg * EPL + e] = x[e] * inv * 1.0f * wv[e];
    __syncthreads();
    if (j < DD)
      for (int r = 0; r < RPP && h0 + r < G; ++r) tot += hsum[r][j];
    __syncthreads();
  };
  const uint4 first = ld(0);
  issued();
  __builtin_amdgcn_sched_barrier(0);  // keep the caller's loads ahead of the wait for `first`
  heads(first, 0);
  for (int h0 = RPP; h0 < G; h0 += RPP) heads(ld(h0), h0);
  if (j < DD) qs[j] = tot;
  __syncthreads();
}

// Level 1: grid (B*Hkv, nsl), NT threads. The candidates 1 .. nc are cut into chunks of RPI = 32
// consecutive blocks, dealt round-robin to the slices: slice s holds chunks s, s + nsl, s + 2nsl,
// ... (at most DSL / 32 of them), so local position x of the slice is candidate
// j = 1 + ((x / 32) * nsl + s) * 32 + x % 32. Local positions rise with j and the valid ones
// form a prefix 0 .. n-1 (only the last chunk of the range can be partial, and it is the last
// chunk of its slice). At each step the nsl slices of a row read adjacent chunks, which spreads
// the stream over the memory channels. Scores q~ . k_pool[j] (8 lanes per pooled row), then the
// slice's best R as composites into cand[bg][s][0..R) (0-padded; when R <= 64 chosen by bitonic
// networks and sorted largest first, else by a radix threshold and unordered). With kv_lens, nc
// is each sequence's own count (at most the nc given). q~ of the single query token is computed
// here (decode_qtilde) from q [B, Hq, DD], while the first rows' loads are in flight.
// APPEND (the decode step): the grid has one more row of workgroups, y = 0, that append each
// sequence's new token to its cache (append_block) instead; the slices are y - 1. The append
// writes the cache rows and the pooled key of the query's own block only, and no slice reads
// those: the candidates end n_local blocks before it.
template <typename QT>
struct DecodeAppend {
  const QT* k_new;
  const QT* v_new;
  const float* kw;
  QT* k_cache;
  QT* v_cache;
  float* k_pool;
  long cap;
};
template <typename QT, int DD, bool APPEND>
__global__ void __launch_bounds__(NT)
decode_slice_kernel(const QT* __restrict__ q, const float* __restrict__ qw, int Hq, float eps,
                    const float* __restrict__ kpool, uint64_t* __restrict__ cand, long nblk_cap, long nc, int R,
                    const int64_t* __restrict__ kv_lens, int Hkv, long kv_max, int n_local, DecodeAppend<QT> ap) {
  constexpr int LPB = 8, FPL = DD / LPB, RPI = NT / LPB;  // rows per iteration
  __shared__ uint32_t keys[DSL];
  __shared__ int hist[256];
  __shared__ int scan_tmp[NT / 64 + 1];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  __shared__ int s_cnt;
  __shared__ float hsum[NT / (DD / (16 / (int)sizeof(QT)))][DD];
  __shared__ float qs[DD];
  __shared__ uint64_t s_lists[2][4][64];
  static_assert(RPI == 32, "chunks of 32 candidates: one step of the workgroup");
  constexpr int IT = DSL / RPI, BT = 4;
  if (APPEND && blockIdx.y == 0) {
    static_assert(sizeof(hsum) == sizeof(float) * RowGeom<QT, DD>::RPP * DD, "append partial sums fit hsum");
    append_block<QT, DD>(ap.k_new, ap.v_new, ap.kw, ap.k_cache, ap.v_cache, ap.k_pool, 1, Hkv, kv_max, ap.cap, eps,
                         kv_lens, blockIdx.x, 0, hsum);
    return;
  }
  const int bg = blockIdx.x, sl = blockIdx.y - (APPEND ? 1 : 0), nsl = gridDim.y - (APPEND ? 1 : 0);
  const int tid = threadIdx.x, sub = tid / LPB, part = tid % LPB;
  if (kv_lens) {
    long i;
    const long ncb = decode_candidates(kv_lens, bg / Hkv, kv_max, n_local, &i);
    nc = ncb < nc ? ncb : nc;
  }
  // local position x -> candidate index, and the count of valid positions
  auto cand_of = [&](int x) -> long { return 1 + ((long)(x / RPI) * nsl + sl) * RPI + x % RPI; };
  int n = 0;
#pragma unroll
  for (int c = 0; c < IT; ++c) n += (int)max(0L, min((long)RPI, nc - ((long)c * nsl + sl) * RPI));
  // lane `part` of a row reads its floats 4*part + 32e .. +3 (e < FPL/4): the 8 lanes of a row
  // read 128 contiguous bytes per load
  const float* kb = kpool + (long)bg * nblk_cap * DD + 4 * part;
  // the rows stream in batches of BT chunks, the next batch's loads issued before the current
  // batch is reduced (positions past the slice repeat its last row, or its first chunk's row
  // when it has none: always rows of the pool, whose keys are never read)
  float4 buf[2][BT][FPL / 4];
  auto load = [&](int bt, int slot) {
#pragma unroll
    for (int u = 0; u < BT; ++u) {
      const int x = (bt * BT + u) * RPI + sub;
      const float* row = kb + cand_of(x < n ? x : (n > 0 ? n - 1 : 0)) * DD;
#pragma unroll
      for (int e = 0; e < FPL / 4; ++e) buf[slot][u][e] = *reinterpret_cast<const float4*>(row + 4 * LPB * e);
    }
  };
  decode_qtilde<QT, DD>(q, qw, bg / Hkv, bg % Hkv, Hq, Hkv, eps, hsum, qs, [&] { load(0, 0); });
  float qv[FPL];
#pragma unroll
  for (int e = 0; e < FPL; ++e) qv[e] = qs[4 * LPB * (e / 4) + 4 * part + e % 4];
  if (n > 0) {
    // the lane's partial dot products of its IT rows; reduced over the 8 lanes of each row after
    // the stream (a transposing butterfly: 8 + 4 + 2 exchanges leave each lane two full sums)
    float pd[IT];
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
        pd[bt * BT + u] = sdot;
      }
    }
    static_assert(IT == 16 && LPB == 8, "butterfly shape");
    const bool hb = part & 4, hc = part & 2, hd = part & 1;
    float a8[8], a4[4], a2[2];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      a8[k] = (hb ? pd[8 + k] : pd[k]) + __shfl_xor(hb ? pd[k] : pd[8 + k], 4, 64);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      a4[k] = (hc ? a8[4 + k] : a8[k]) + __shfl_xor(hc ? a8[k] : a8[4 + k], 2, 64);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      a2[k] = (hd ? a4[2 + k] : a4[k]) + __shfl_xor(hd ? a4[k] : a4[2 + k], 1, 64);
    const int it0 = (hb ? 8 : 0) + (hc ? 4 : 0) + (hd ? 2 : 0);  // this lane's rows it0, it0 + 1
#pragma unroll
    for (int k = 0; k < 2; ++k) keys[(it0 + k) * RPI + sub] = score_key(a2[k]);
  }
  __syncthreads();
  uint64_t* dst = cand + ((long)bg * nsl + sl) * R;
  if (R <= 64) {
    // the 64 largest composites by bitonic networks (exact: composites are distinct): wave w
    // sorts positions 128w .. +63 (descending) and 128w + 64 .. +127 (ascending), keeps the
    // larger of each lane pair and sorts them; two halvings through LDS leave the slice's 64
    // largest, descending, in wave 0, whose first R are the winners
    static_assert(NT == 256 && DSL == 4 * 128, "four waves of 128 positions");
    const int w = tid >> 6, l = tid & 63;
    auto comp = [&](int x) -> uint64_t { return x < n ? composite(keys[x], cand_of(x)) : 0ull; };
    const uint64_t a = wave_sort64(comp(128 * w + l), true), b = wave_sort64(comp(128 * w + 64 + l), false);
    uint64_t c = wave_merge_desc(a > b ? a : b);
    s_lists[0][w][l] = c;
    __syncthreads();
    if (w < 2) {
      const uint64_t u = s_lists[0][2 * w][l], v = s_lists[0][2 * w + 1][63 - l];
      c = wave_merge_desc(u > v ? u : v);
      s_lists[1][w][l] = c;
    }
    __syncthreads();
    if (w == 0) {
      const uint64_t u = s_lists[1][0][l], v = s_lists[1][1][63 - l];
      c = wave_merge_desc(u > v ? u : v);
      if (l < R) dst[l] = c;
    }
    return;
  }
  if (n <= R) {
    for (int t = tid; t < R; t += NT) dst[t] = t < n ? composite(keys[t], cand_of(t)) : 0ull;
    return;
  }
  uint32_t T;
  int need;
  radix_threshold<NT, true>(keys, n, R, hist, &s_prefix, &s_need, &s_cnt, T, need);
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
    if (pick && pos < R) dst[pos++] = composite(key, cand_of(x));
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
decode_merge_kernel(const uint64_t* __restrict__ cand, int32_t* __restrict__ sel, float* __restrict__ sel_sc, int nsl,
                    int R,
                    long i, int n_local, int topk, long nc, const int64_t* __restrict__ kv_lens, int Hkv,
                    long kv_max) {
  __shared__ uint32_t keys[CAPB];
  __shared__ uint32_t idx[CAPB];
  __shared__ uint32_t bits[DBITS];
  __shared__ int hist[256];
  __shared__ int scan_tmp[NTM / 64 + 1];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  __shared__ int s_cnt;
  __shared__ int32_t s_row[256];  // the emitted row (topk <= 256), for placing the scores
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
    radix_threshold<NTM, true>(keys, n, R, hist, &s_prefix, &s_need, &s_cnt, T, need);
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
      radix_threshold<NTM, false>(keys, n, R, hist, &s_prefix, &s_need, &s_cnt, T2, need2);
    }
  }
  for (int t = tid; t < n; t += NTM) {
    bool pick;
    if (all) pick = keys[t] != 0u;
    else if (all_ties) pick = keys[t] >= T;
    else pick = keys[t] >= T2;
    if (pick && idx[t] <= (uint32_t)nc) atomicOr(&bits[idx[t] >> 5], 1u << (idx[t] & 31));
    if (!pick) idx[t] = 0xFFFFFFFFu;  // (for the scores below: only chosen candidates keep an index)
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
      if (pos < topk) { out[pos] = 32 * w + b; s_row[pos] = 32 * w + b; }
      ++pos;
    }
  }
  if (tid == 0 && head) out[0] = 0;
  const int nloc = (int)(i - f_lo + 1);
  for (int t = tid; t < nloc; t += NTM)
    if (head + cnt + t < topk) out[head + cnt + t] = (int32_t)(f_lo + t);
  for (int t = head + cnt + nloc + tid; t < topk; t += NTM) out[t] = -1;
  if (sel_sc) {
    // each chosen candidate finds its place in the emitted (ascending) row and writes its
    // score there; forced blocks get +inf, padding -inf
    float* osc = sel_sc + (long)bg * topk;
    __syncthreads();
    const int nch = min(cnt, topk - head);
    for (int t = tid; t < n; t += NTM) {
      const uint32_t j = idx[t];
      if (j == 0xFFFFFFFFu || j > (uint32_t)nc) continue;
      int lo = head, hi = head + nch;  // binary search in s_row[head .. head + nch)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((uint32_t)s_row[mid] < j) lo = mid + 1; else hi = mid;
      }
      if (lo < head + nch && (uint32_t)s_row[lo] == j) osc[lo] = key_score((uint32_t)(cand[(long)bg * n + t] >> 32));
    }
    if (tid == 0 && head) osc[0] = INFINITY;
    for (int t = tid; t < nloc; t += NTM)
      if (head + cnt + t < topk) osc[head + cnt + t] = INFINITY;
    for (int t = head + cnt + nloc + tid; t < topk; t += NTM) osc[t] = -INFINITY;
  }
}

// Level 2, R <= 64 (at most 32 slices, each slice's winners sorted largest first; the ordinary
// merge's arguments and output): wave w reads slice 2w forwards and slice 2w+1 backwards
// (ascending), keeps the larger of each lane pair (the 64 largest of both, as a bitonic sequence)
// and sorts them; the waves' lists are then halved pairwise the same way through LDS until wave
// 0 holds the 64 largest in descending order. The first R that are not empty are chosen; wave 0
// sorts them by block index and emits the row.
template <int NTM>
__global__ void __launch_bounds__(NTM)
decode_merge64_kernel(const uint64_t* __restrict__ cand, int32_t* __restrict__ sel, float* __restrict__ sel_sc, int nsl,
                      int R, long i, int n_local, int topk, long nc, const int64_t* __restrict__ kv_lens, int Hkv,
                      long kv_max) {
  constexpr int NW = NTM / 64;
  static_assert(2 * NW >= DNSL_MAX, "two slices per wave");
  __shared__ uint64_t lists[2][NW][64];
  const int bg = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  if (kv_lens) {  // this sequence's query block and candidate count (at most the nc given)
    const long ncb = decode_candidates(kv_lens, bg / Hkv, kv_max, n_local, &i);
    nc = ncb < nc ? ncb : nc;
  }
  const uint64_t* src = cand + (long)bg * nsl * R;
  const uint64_t a = (2 * w < nsl && l < R) ? src[(long)(2 * w) * R + l] : 0ull;
  const uint64_t b = (2 * w + 1 < nsl && 63 - l < R) ? src[(long)(2 * w + 1) * R + 63 - l] : 0ull;
  uint64_t c = wave_merge_desc(a > b ? a : b);
  int cur = 0;
  lists[cur][w][l] = c;
  __syncthreads();
#pragma unroll
  for (int n = NW / 2; n >= 1; n /= 2) {
    if (w < n) {
      const uint64_t u = lists[cur][2 * w][l], v = lists[cur][2 * w + 1][63 - l];
      c = wave_merge_desc(u > v ? u : v);
      lists[cur ^ 1][w][l] = c;
    }
    cur ^= 1;
    __syncthreads();
  }
  if (w != 0) return;
  // wave 0: c = the 64 largest composites, descending
  const uint32_t j = 0xFFFFFFFFu - (uint32_t)c;
  const bool pick = l < R && c != 0ull && j <= (uint32_t)nc;
  const int cnt = __popcll(__ballot(pick));
  // ascending by block index (the chosen first), the score key carried along
  const uint64_t byidx = wave_sort64(pick ? ((uint64_t)j << 32) | (c >> 32) : ~0ull, false);
  const long f_lo = i - n_local + 1 > 0 ? i - n_local + 1 : 0;
  const int head = f_lo > 0 ? 1 : 0;
  const int nloc = (int)(i - f_lo + 1);
  int32_t* out = sel + (long)bg * topk;
  float* osc = sel_sc ? sel_sc + (long)bg * topk : nullptr;
  // row: forced block 0, the chosen (ascending), the forced local blocks f_lo .. i, -1 padding
  if (l < cnt && head + l < topk) {
    out[head + l] = (int32_t)(byidx >> 32);
    if (osc) osc[head + l] = key_score((uint32_t)byidx);
  }
  if (l == 0 && head) {
    out[0] = 0;
    if (osc) osc[0] = INFINITY;
  }
  for (int t = l; t < nloc; t += 64)
    if (head + cnt + t < topk) {
      out[head + cnt + t] = (int32_t)(f_lo + t);
      if (osc) osc[head + cnt + t] = INFINITY;
    }
  for (int t = head + cnt + nloc + l; t < topk; t += 64) {
    out[t] = -1;
    if (osc) osc[t] = -INFINITY;
  }
}

}  // namespace

static long select_row_len(const sala_sparse_desc& d) {
  const SparseGeom g = sparse_geom(d);
  return g.qb0 + g.nqb;  // blocks 0 .. i_max
}

// decode (a single query token) uses the two-level selection while the candidates fit
// DNSL_MAX slices; it needs nsl * R composites per row instead of the score row. The slice
// kernel forms q~ from the one token of each sequence, so a call with several query tokens in
// one block (a short continued prompt) takes the q~ kernel's block mean and the score-row path.
static bool decode_two_level(const sala_sparse_desc& d, long* nc_out, int* nsl_out, int* r_out) {
  const SparseGeom g = sparse_geom(d);
  if (d.n_q != 1 || g.nqb != 1) return false;
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

// level 2 of the decode selection: the register networks while R <= 64, else the radix merge
static void launch_decode_merge(const uint64_t* cand, int32_t* sel, float* sel_sc, int nsl, int R, long i, int n_local,
                                int topk, long nc, const int64_t* kv_lens, int Hkv, long kv_max, int BG,
                                hipStream_t st) {
  if (R <= 64 && nsl <= DNSL_MAX)
    hipLaunchKernelGGL((decode_merge64_kernel<DMERGE_NT>), dim3(BG), dim3(DMERGE_NT), 0, st, cand, sel, sel_sc, nsl,
                       R, i, n_local, topk, nc, kv_lens, Hkv, kv_max);
  else
    hipLaunchKernelGGL((decode_merge_kernel<DMERGE, DMERGE_NT>), dim3(BG), dim3(DMERGE_NT), 0, st, cand, sel, sel_sc,
                       nsl, R, i, n_local, topk, nc, kv_lens, Hkv, kv_max);
}

// level 1 of the decode selection (q~ computed inside), for the descriptor's dtype and dim
static void launch_decode_slice(const sala_sparse_desc& d, const void* q, const float* qw, const float* k_pool,
                                uint64_t* cand, long nblk_cap, long nc, int R, int nsl, const int64_t* kv_lens,
                                hipStream_t st) {
  const dim3 grid(d.batch * d.n_kv_heads, nsl);
#define SALA_SLICE(T, DD)                                                                                   \
  hipLaunchKernelGGL((decode_slice_kernel<T, DD, false>), grid, dim3(NT), 0, st, (const T*)q, qw, d.n_heads,     \
                     d.norm_eps, k_pool, cand, nblk_cap, nc, R, kv_lens, d.n_kv_heads, (long)d.kv_len, d.n_local, \
                     DecodeAppend<T>{})
  if (d.dtype == SALA_BF16) {
    if (d.head_dim == 128) SALA_SLICE(bf16_t, 128); else SALA_SLICE(bf16_t, 64);
  } else {
    if (d.head_dim == 128) SALA_SLICE(float, 128); else SALA_SLICE(float, 64);
  }
#undef SALA_SLICE
}

static hipError_t launch_select_rows(const sala_sparse_desc& d, const float* qt, const float* k_pool, int32_t* sel,
                                     float* sel_sc, float* sc, hipStream_t st);

hipError_t launch_block_select(const sala_sparse_desc& d, const void* q, const float* qw,
                               const float* k_pool, int32_t* sel, float* sel_sc, void* ws, hipStream_t st) {
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
    launch_decode_merge(cand, sel, sel_sc, nsl, R, i_max, d.n_local, d.topk, nc, nullptr, d.n_kv_heads,
                        (long)d.kv_len, BG, st);
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
  return launch_select_rows(d, qt, k_pool, sel, sel_sc, sc, st);
}

// the scores and the forced + top-k rows of a call whose q~ is already in qt (layout of
// qtilde_kernel); sc: the score workspace
static hipError_t launch_select_rows(const sala_sparse_desc& d, const float* qt, const float* k_pool, int32_t* sel,
                                     float* sel_sc, float* sc, hipStream_t st) {
  const SparseGeom g = sparse_geom(d);
  const int BG = d.batch * d.n_kv_heads;
  const long RL = select_row_len(d);
  const long i_max = g.qb0 + g.nqb - 1;
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
    hipLaunchKernelGGL((select_kernel<1024, 16384>), dim3((unsigned)(BG * g.nqb)), dim3(1024), 0, st, sc, sel, sel_sc,
                       (int)g.nqb, (long)g.qb0, (int)RL, d.topk, d.n_local);
  else
    hipLaunchKernelGGL((select_kernel<256, 4096>), dim3((unsigned)(BG * g.nqb)), dim3(256), 0, st, sc, sel, sel_sc,
                       (int)g.nqb, (long)g.qb0, (int)RL, d.topk, d.n_local);
  return hipGetLastError();
}

// ---- packed batches (desc.batch = sequences; cu_seqlens, pos0 host arrays). The q~ of every
// prefill sequence comes from one launch over all their query blocks (its grid would be small
// for a short sequence alone); the scores and rows then run sequence by sequence with the
// sequence's own cache row, cache length and query blocks. A sequence of a single decode token
// (the two-level selection) runs as a one-sequence call, which forms its q~ itself.
namespace {

sala_sparse_desc select_seq_desc(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0, int s) {
  sala_sparse_desc x = d;
  x.batch = 1;
  x.n_q = cu[s + 1] - cu[s];
  x.kv_len = pos0[s] + x.n_q;
  return x;
}

// query blocks of each sequence that takes the q~ kernel (0 for the others) and their sum
long varlen_qtilde_blocks(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0, int* nqb_of) {
  long tot = 0;
  for (int s = 0; s < d.batch; ++s) {
    nqb_of[s] = 0;
    if (cu[s + 1] == cu[s]) continue;
    const sala_sparse_desc x = select_seq_desc(d, cu, pos0, s);
    long nc;
    int nsl, R;
    if (decode_two_level(x, &nc, &nsl, &R)) continue;
    nqb_of[s] = (int)sparse_geom(x).nqb;
    tot += nqb_of[s];
  }
  return tot;
}

}  // namespace

size_t block_select_varlen_workspace(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0) {
  int nqb_of[SALA_VARLEN_MAX_SEQS];
  const long nq = varlen_qtilde_blocks(d, cu, pos0, nqb_of);
  size_t per = 0;  // the largest one-sequence workspace (its own q~ part included)
  for (int s = 0; s < d.batch; ++s)
    if (cu[s + 1] > cu[s]) per = std::max(per, block_select_workspace(select_seq_desc(d, cu, pos0, s)));
  const size_t qt = (size_t)nq * d.n_kv_heads * d.head_dim * sizeof(float);
  return ((qt + 255) & ~(size_t)255) + per;
}

hipError_t launch_block_select_varlen(const sala_sparse_desc& d, const int32_t* cu, const int64_t* pos0,
                                      const void* q, const float* qw, const float* k_pool, int32_t* sel, void* ws,
                                      hipStream_t st) {
  const size_t eb = d.dtype == SALA_BF16 ? 2 : 4, qrow = (size_t)d.n_heads * d.head_dim;
  const size_t pool_seq = (size_t)d.n_kv_heads * d.head_dim * (d.kv_capacity / 64);
  int nqb_of[SALA_VARLEN_MAX_SEQS];
  const long nq = varlen_qtilde_blocks(d, cu, pos0, nqb_of);
  float* qt = static_cast<float*>(ws);
  const size_t qt_bytes = (size_t)nq * d.n_kv_heads * d.head_dim * sizeof(float);
  char* rest = static_cast<char*>(ws) + ((qt_bytes + 255) & ~(size_t)255);
  if (nq > 0) {
    VarlenTable t = make_varlen_table(d.batch, cu, pos0);
    for (int s = 0; s < d.batch; ++s) t.item0[s + 1] = t.item0[s] + nqb_of[s];
#define SALA_QTV(T, DD)                                                                                      \
  hipLaunchKernelGGL((qtilde_varlen_kernel<T, DD>), dim3((unsigned)nq), dim3(NT), 0, st, (const T*)q, qw, qt, \
                     d.n_heads, d.n_kv_heads, d.norm_eps, t)
    if (d.dtype == SALA_BF16) {
      if (d.head_dim == 128) SALA_QTV(bf16_t, 128); else SALA_QTV(bf16_t, 64);
    } else {
      if (d.head_dim == 128) SALA_QTV(float, 128); else SALA_QTV(float, 64);
    }
#undef SALA_QTV
  }
  long qb_row = 0, qt_blk = 0;  // query blocks of the earlier sequences: all, and those in qt
  for (int s = 0; s < d.batch; ++s) {
    const int n = cu[s + 1] - cu[s];
    if (n == 0) continue;
    const sala_sparse_desc x = select_seq_desc(d, cu, pos0, s);
    int32_t* sel_s = sel + qb_row * d.n_kv_heads * d.topk;
    const float* pool_s = k_pool + s * pool_seq;
    hipError_t e;
    if (nqb_of[s] == 0) {
      e = launch_block_select(x, static_cast<const char*>(q) + (size_t)cu[s] * qrow * eb, qw, pool_s, sel_s, nullptr,
                              rest, st);
    } else {
      // past its q~ part, the one-sequence workspace layout holds the scores
      const size_t own_qt = (size_t)d.n_kv_heads * nqb_of[s] * d.head_dim * sizeof(float);
      float* sc = reinterpret_cast<float*>(rest + ((own_qt + 255) & ~(size_t)255));
      e = launch_select_rows(x, qt + qt_blk * d.n_kv_heads * d.head_dim, pool_s, sel_s, nullptr, sc, st);
      qt_blk += nqb_of[s];
    }
    if (e != hipSuccess) return e;
    qb_row += (n + 63) / 64;
  }
  return hipSuccess;
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
                                         hipStream_t st, const DecodeAppendPtrs* app) {
  long nc; int nsl, R;
  if (!decode_at_plan(d, &nc, &nsl, &R)) return hipErrorInvalidValue;
  const int BG = d.batch * d.n_kv_heads;
  const size_t qt_bytes = (size_t)BG * d.head_dim * sizeof(float);
  uint64_t* cand = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + ((qt_bytes + 255) & ~(size_t)255));
  const long nblk_cap = d.kv_capacity / 64;
  if (app) {
    // bf16, d = 128 only (the decode step's shapes): the append rides along as grid row 0
    const DecodeAppend<bf16_t> ap{(const bf16_t*)app->k_new, (const bf16_t*)app->v_new, app->kw,
                                  (bf16_t*)app->k_cache, (bf16_t*)app->v_cache, app->k_pool, (long)d.kv_capacity};
    hipLaunchKernelGGL((decode_slice_kernel<bf16_t, 128, true>), dim3(BG, nsl + 1), dim3(NT), 0, st,
                       (const bf16_t*)q, qw, d.n_heads, d.norm_eps, k_pool, cand, nblk_cap, nc, R, kv_lens,
                       d.n_kv_heads, (long)d.kv_len, d.n_local, ap);
  } else {
    launch_decode_slice(d, q, qw, k_pool, cand, nblk_cap, nc, R, nsl, kv_lens, st);
  }
  launch_decode_merge(cand, sel, nullptr, nsl, R, (long)((d.kv_len - 1) / 64), d.n_local, d.topk, nc, kv_lens,
                      d.n_kv_heads, (long)d.kv_len, BG, st);
  return hipGetLastError();
}

}  // namespace sala
