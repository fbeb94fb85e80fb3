// Backward pass of the sparse layer's attention step for gfx950: bf16 inputs, fp32 gradients.
//
// Pages: "面壁智能发布MiniCPM-SALA：稀疏-线性混合架构，9B模型端侧跑通百万上下文，速度飙升3.5倍", section
// "SALA混合架构：黄金配比破解瓶颈" (each query attends only to the blocks the selection picked) and
// section "高效训练范式：以25%的成本完成转换" (sparse attention is switched on for the later
// training stages, which train every parameter); "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文
// 建模" opening summary (QK-norm in every layer, output gate after every attention block).
//
// Forward, for query row t (position p, block i) of head h in group g: q~ = RMSNorm(q) w *
// scale * log2(e); s2 = q~ . k over the keys of the selected blocks (token-causal); P =
// exp2(s2 - lse2); o = P V; out = o * sigmoid(gate). The selection is a discrete choice and
// carries no gradient. With dO = dout * sigmoid(gate) and D = rowsum(dO * o):
//   dP = dO V^T,  dS = P * (dP - D),  dq^ = scale * dS K,  dK = scale * dS^T q^,  dV = P^T dO.
// Kernels:
//   1. stats (query-major, one workgroup per (b, g, query block, 4 heads), the forward loop):
//      lse2, D, dg, and q~ and dO in bf16, head-major and padded to whole query blocks;
//   2. dq (query-major, same grid): S, P, dP, dS per selected block, dq^ on MFMA, then the
//      RMSNorm transpose and per-workgroup sums of the norm-weight gradient;
//   3. the selection inverted: a bitmap [key block][query block]; for every range of SB_RW
//      query blocks and every key block, the query blocks of the range that chose it, cut into
//      slices of at most SB_SL, numbered range by range (so the workgroups running at one time
//      gather q~ and dO of one range of query blocks, which the caches then hold);
//   4. dK, dV (key-major, one workgroup per slice): for each query block of the slice and
//      each head of the group, S and dP for the 64 keys, then dV^T += dO^T P, dK^T += q~^T dS
//      on MFMA; one fp32 partial per slice;
//   5. per key block, the sum of its slices in order (deterministic: no atomics on values).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "sparse_tiles.hpp"

namespace sala {

namespace {

constexpr int D = 128;
constexpr int SB_NT = 512;
constexpr int SB_QT = 2;   // 16-row query tiles per wave in the query-major kernels
constexpr int SB_SL = 32;  // query blocks per dK/dV slice
constexpr int SB_RWW = 8;  // bitmap words (32 query blocks each) per query-block range
constexpr int SB_RW = 32 * SB_RWW;


struct ItemGeom {
  int hq, r, gk, b, hl, h;
  bool head_ok;
  long i, row_base;
};

__device__ __forceinline__ ItemGeom item_geom(int G, int Hkv, int nqb, long qb0, long cap) {
  ItemGeom it;
  const int nhq = (G + 3) / 4;
  const unsigned nwg = gridDim.x;
  unsigned w = blockIdx.x;
  if ((nwg & 7u) == 0) w = (blockIdx.x & 7u) * (nwg >> 3) + (blockIdx.x >> 3);
  it.hq = w % nhq;
  unsigned rest = w / nhq;
  it.r = rest % nqb;
  rest /= nqb;
  it.gk = rest % Hkv;
  it.b = rest / Hkv;
  it.hl = 4 * it.hq + ((threadIdx.x >> 6) >> 1);
  it.head_ok = it.hl < G;
  it.h = it.gk * G + (it.head_ok ? it.hl : 0);
  it.i = qb0 + it.r;
  it.row_base = ((long)it.b * Hkv + it.gk) * cap;
  return it;
}

// number of selected blocks of a query block (ascending, -1 padded) into s_sel; a barrier
__device__ __forceinline__ int load_selection(const int32_t* srow, int topk, int* s_sel) {
  int v = -1;
  if ((int)threadIdx.x < topk) s_sel[threadIdx.x] = v = srow[threadIdx.x];
  return __builtin_amdgcn_readfirstlane(__syncthreads_count(v >= 0));
}

// ---- 1. stats: the forward loop, then lse2, D, dg, and q~, dO (bf16) for the later passes.
// Padded per-head buffers: row index (b * Hq + h) * nqb * 64 + r * 64 + row.
__global__ void __launch_bounds__(SB_NT)
sbwd_stats_kernel(const bf16_t* __restrict__ q, const float* __restrict__ qw, const bf16_t* __restrict__ kc,
                  const bf16_t* __restrict__ vc, const bf16_t* __restrict__ g, const int32_t* __restrict__ sel,
                  const bf16_t* __restrict__ dout, float* __restrict__ dg, bf16_t* __restrict__ qtb,
                  bf16_t* __restrict__ dob, float* __restrict__ stb, int n_q, int Hq, int Hkv, long q0, long qb0,
                  int nqb, long kv_len, long cap, int topk, float eps, float qscale) {
  __shared__ __align__(16) bf16_t lds[NSTAGE][2][TILE];
  __shared__ int s_sel[256];
  const int G = Hq / Hkv;
  const ItemGeom it = item_geom(G, Hkv, nqb, qb0, cap);
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6, l16 = lane & 15, lq = lane >> 4;
  const int qrow0 = 32 * (wave & 1);
  const int nsel = load_selection(sel + (((long)it.b * Hkv + it.gk) * nqb + it.r) * topk, topk, s_sel);
  const long pad0 = ((long)it.b * Hq + it.h) * nqb * 64 + (long)it.r * 64;  // padded row of block row 0

  bf16x8 qf[SB_QT][4];
#pragma unroll
  for (int qt = 0; qt < SB_QT; ++qt) {
    const long t = it.i * 64 + qrow0 + 16 * qt + l16 - q0;
    const bool ok = it.head_ok && t < n_q;
    float x[4][8];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (ok) u = *reinterpret_cast<const uint4*>(q + ((long)(it.b * (long)n_q + t) * Hq + it.h) * D + 32 * ks + 8 * lq);
      unpack8(u, x[ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[ks][e] * x[ks][e];
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = qscale * __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[ks][e] * inv * (qw ? qw[32 * ks + 8 * lq + e] : 1.0f);
      uint4 u = pack8(y);
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
      qf[qt][ks] = as_bf16x8(u);
      if (it.head_ok)
        *reinterpret_cast<uint4*>(qtb + (pad0 + qrow0 + 16 * qt + l16) * D + 32 * ks + 8 * lq) = u;
    }
  }
  // block copies by scalar addresses, K and V tiles both in the swzv layout
  const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const DmaLane dl = dma_lane_setup(wave_u);
  auto copy_block = [&](int x, int sg) {
    dma_block_sel(dl, kc, vc, it.row_base, s_sel[x], kv_len, lds[sg][0], lds[sg][1], wave_u);
  };

  float m[SB_QT], lp[SB_QT];
  f32x4 minit[SB_QT], OT[8][SB_QT];
#pragma unroll
  for (int qt = 0; qt < SB_QT; ++qt) {
    m[qt] = 0.f;
    lp[qt] = 0.f;
    minit[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt = 0; qt < SB_QT; ++qt) OT[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int x = 0; x < 3; ++x)
    if (x < nsel) copy_block(x, x);
  if (nsel > 2) wait_vmcnt<2 * DMA_PER_WAVE>();
  else if (nsel > 1) wait_vmcnt<DMA_PER_WAVE>();
  else wait_vmcnt<0>();
  __syncthreads();
  auto step = [&](int e, bool diag) {
    if (e + 3 < nsel) copy_block(e + 3, (e + 3) & 3);
    f32x4 ST[4][SB_QT], SN[4][SB_QT];
    scores<SB_QT, true>(lds[e & 3][0], qf, minit, ST, l16);
    if (diag) mask_diag<SB_QT>(ST, l16, lq, qrow0);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < SB_QT; ++qt) SN[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    exp_pv<SB_QT>(lds[e & 3][1], ST, SN, OT, m, minit, lp, l16, lq, e == 0);
  };
  for (int e = 0; e < nsel - 1; ++e) {
    step(e, false);
    const int ahead = min(2, nsel - 2 - e);  // block e+1 must have landed
    if (ahead >= 2) wait_vmcnt<2 * DMA_PER_WAVE>();
    else if (ahead == 1) wait_vmcnt<DMA_PER_WAVE>();
    else wait_vmcnt<0>();
    __syncthreads();
  }
  if (nsel > 0) step(nsel - 1, true);
  if (!it.head_ok) return;

  // ---- epilogue (lane: query qrow0 + 16qt + l16, dims 16dt + 4lq .. +3)
#pragma unroll
  for (int qt = 0; qt < SB_QT; ++qt) {
    float l = lp[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float il = 1.0f / l;
    const int row = qrow0 + 16 * qt + l16;
    const long t = it.i * 64 + row - q0;
    const bool ok = t < n_q;
    const long base = ((long)(it.b * (long)n_q + (ok ? t : 0)) * Hq + it.h) * D;
    float dsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int col = 16 * dt + 4 * lq;
      uint2 gv = make_uint2(0, 0), dv = make_uint2(0, 0);
      if (ok) {
        gv = *reinterpret_cast<const uint2*>(g + base + col);
        dv = *reinterpret_cast<const uint2*>(dout + base + col);
      }
      const float gg[4] = {bf2f(gv.x & 0xffffu), bf2f(gv.x >> 16), bf2f(gv.y & 0xffffu), bf2f(gv.y >> 16)};
      const float dd[4] = {bf2f(dv.x & 0xffffu), bf2f(dv.x >> 16), bf2f(dv.y & 0xffffu), bf2f(dv.y >> 16)};
      float dO[4];
      f32x4 dgv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float o = OT[dt][qt][e] * il;
        const float sg = fast_sigmoid(gg[e]);
        dO[e] = dd[e] * sg;
        dgv[e] = dd[e] * o * sg * (1.0f - sg);
        dsum = fmaf(dO[e], o, dsum);
      }
      if (ok) *reinterpret_cast<f32x4*>(dg + base + col) = dgv;
      uint2 pk;
      pk.x = pack_bf16x2(dO[0], dO[1]);
      pk.y = pack_bf16x2(dO[2], dO[3]);
      *reinterpret_cast<uint2*>(dob + (pad0 + row) * D + col) = pk;
    }
    dsum += __shfl_xor(dsum, 16, 64);
    dsum += __shfl_xor(dsum, 32, 64);
    if (lq == 0) {
      const float lse2 = ok ? m[qt] + __log2f(l) : INFINITY;
      *reinterpret_cast<float2*>(stb + (pad0 + row) * 4) = make_float2(lse2, ok ? dsum : 0.f);
    }
  }
}

// ---- 1'. the same buffers from the forward's saved output and lse (no forward loop): per padded
// row, lse2 as saved, D = rowsum(dout * out) (= rowsum(dO * O) with out = O sigmoid(g)),
// dg = dout * out * (1 - sigmoid(g)), q~ and dO in bf16. Four lanes per (token, head) row (dims
// 32ks + 8lq + e, the forward's lane order, so q~ is computed exactly as the forward computed it),
// heads fastest so that the token-major inputs are read contiguously, 64 rows per block; padded
// rows past n_q get q~ = dO = 0, lse2 = +inf and D = 0.
__global__ void __launch_bounds__(256)
sbwd_prep_kernel(const bf16_t* __restrict__ q, const float* __restrict__ qw, const bf16_t* __restrict__ g,
                 const bf16_t* __restrict__ dout, const bf16_t* __restrict__ out, const float* __restrict__ lse,
                 float* __restrict__ dg, bf16_t* __restrict__ qtb, bf16_t* __restrict__ dob, float* __restrict__ stb,
                 int n_q, int Hq, long q0, long qb0, int nqb, float eps, float qscale) {
  const long item = (long)blockIdx.x * 64 + (threadIdx.x >> 2);  // (b, padded token, head), grid covers them exactly
  const int lq = threadIdx.x & 3;
  const int h = (int)(item % Hq);
  const long bp = item / Hq;
  const long ptok = bp % ((long)nqb * 64);  // padded token of the call's query blocks
  const long b = bp / ((long)nqb * 64);
  const long prow = (b * Hq + h) * nqb * 64 + ptok;  // row of the head-major padded buffers
  const long t = qb0 * 64 + ptok - q0;
  const bool ok = t < n_q;
  const long base = ((b * n_q + (ok ? t : 0)) * Hq + h) * D;
  float x[4][8];
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (ok) u = *reinterpret_cast<const uint4*>(q + base + 32 * ks + 8 * lq);
    unpack8(u, x[ks]);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[ks][e] * x[ks][e];
  }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  const float inv = qscale * __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int col = 32 * ks + 8 * lq;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[ks][e] * inv * (qw ? qw[col + e] : 1.0f);
    *reinterpret_cast<uint4*>(qtb + prow * D + col) = pack8(y);
    float gg[8], dd[8], oo[8], dO[8];
    uint4 ug = make_uint4(0, 0, 0, 0), ud = ug, uo = ug;
    if (ok) {
      ug = *reinterpret_cast<const uint4*>(g + base + col);
      ud = *reinterpret_cast<const uint4*>(dout + base + col);
      uo = *reinterpret_cast<const uint4*>(out + base + col);
    }
    unpack8(ug, gg);
    unpack8(ud, dd);
    unpack8(uo, oo);
    f32x4 d0, d1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sg = fast_sigmoid(gg[e]);
      dO[e] = dd[e] * sg;
      const float dge = dd[e] * oo[e] * (1.0f - sg);
      if (e < 4) d0[e] = dge; else d1[e - 4] = dge;
      dsum = fmaf(dd[e], oo[e], dsum);
    }
    *reinterpret_cast<uint4*>(dob + prow * D + col) = pack8(dO);
    if (ok) {
      *reinterpret_cast<f32x4*>(dg + base + col) = d0;
      *reinterpret_cast<f32x4*>(dg + base + col + 4) = d1;
    }
  }
  dsum += __shfl_xor(dsum, 1, 64);
  dsum += __shfl_xor(dsum, 2, 64);
  if (lq == 0)
    *reinterpret_cast<float2*>(stb + prow * 4) = make_float2(ok ? lse[(b * n_q + t) * Hq + h] : INFINITY, ok ? dsum : 0.f);
}

// ---- 2. dq: per selected block S - lse2 (log2 units), P, dP = dO V^T, dS = P (dP - D),
// dq^T += K^T dS^T; then dq = RMSNorm^T (scale dq^) and the norm-weight partial sums.
__global__ void __launch_bounds__(SB_NT)
sbwd_dq_kernel(const bf16_t* __restrict__ q, const float* __restrict__ qw, const bf16_t* __restrict__ kc,
               const bf16_t* __restrict__ vc, const int32_t* __restrict__ sel, const bf16_t* __restrict__ qtb,
               const bf16_t* __restrict__ dob, const float* __restrict__ stb, float* __restrict__ dq,
               float* __restrict__ wpart, int n_q, int Hq, int Hkv, long q0, long qb0, int nqb, long kv_len, long cap,
               int topk, float eps, float scale) {
  __shared__ __align__(16) bf16_t lds[NSTAGE][2][TILE];
  __shared__ int s_sel[256];
  __shared__ float red[8][D];
  const int G = Hq / Hkv;
  const ItemGeom it = item_geom(G, Hkv, nqb, qb0, cap);
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6, l16 = lane & 15, lq = lane >> 4;
  const int qrow0 = 32 * (wave & 1);
  const int nsel = load_selection(sel + (((long)it.b * Hkv + it.gk) * nqb + it.r) * topk, topk, s_sel);
  const long pad0 = ((long)it.b * Hq + it.h) * nqb * 64 + (long)it.r * 64;

  bf16x8 qf[SB_QT][4], df[SB_QT][4];
  f32x4 minit[SB_QT];
  float Dv[SB_QT];
#pragma unroll
  for (int qt = 0; qt < SB_QT; ++qt) {
    const long pr = pad0 + qrow0 + 16 * qt + l16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 a = *reinterpret_cast<const uint4*>(qtb + pr * D + 32 * ks + 8 * lq);
      uint4 c = *reinterpret_cast<const uint4*>(dob + pr * D + 32 * ks + 8 * lq);
      asm volatile("" : "+v"(a.x), "+v"(a.y), "+v"(a.z), "+v"(a.w));
      asm volatile("" : "+v"(c.x), "+v"(c.y), "+v"(c.z), "+v"(c.w));
      qf[qt][ks] = as_bf16x8(a);
      df[qt][ks] = as_bf16x8(c);
    }
    const float2 sd = *reinterpret_cast<const float2*>(stb + pr * 4);
    minit[qt] = f32x4{-sd.x, -sd.x, -sd.x, -sd.x};
    Dv[qt] = sd.y;
  }
  f32x4 QT[8][SB_QT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt = 0; qt < SB_QT; ++qt) QT[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // block copies by scalar addresses, K and V tiles both in the swzv layout
  const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const DmaLane dl = dma_lane_setup(wave_u);
  auto copy_block = [&](int x, int sg) {
    dma_block_sel(dl, kc, vc, it.row_base, s_sel[x], kv_len, lds[sg][0], lds[sg][1], wave_u);
  };

#pragma unroll
  for (int x = 0; x < 3; ++x)
    if (x < nsel) copy_block(x, x);
  if (nsel > 2) wait_vmcnt<2 * DMA_PER_WAVE>();
  else if (nsel > 1) wait_vmcnt<DMA_PER_WAVE>();
  else wait_vmcnt<0>();
  __syncthreads();
  // K tiles in the swzv layout: read by rows for the scores and transposed for dq
  auto step = [&](int e, bool diag) {
    if (e + 3 < nsel) copy_block(e + 3, (e + 3) & 3);
    const bf16_t* Ks = lds[e & 3][0];
    const bf16_t* Vs = lds[e & 3][1];
    f32x4 ST[4][SB_QT], PT[4][SB_QT];
    scores<SB_QT, true>(Ks, qf, minit, ST, l16);
    if (diag) mask_diag<SB_QT>(ST, l16, lq, qrow0);
    // dP^T[key][query] = V dO^T (A = V rows, k = dv)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int qt = 0; qt < SB_QT; ++qt) PT[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Vs + swzv(16 * kt + l16, 4 * ks + lq)));
#pragma unroll
        for (int qt = 0; qt < SB_QT; ++qt) PT[kt][qt] = mfma16x16x32(a, df[qt][ks], PT[kt][qt]);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 sf[SB_QT];
#pragma unroll
      for (int qt = 0; qt < SB_QT; ++qt) {
        float ds[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ds[u] = fast_exp2(ST[2 * c][qt][u]) * (PT[2 * c][qt][u] - Dv[qt]);
          ds[4 + u] = fast_exp2(ST[2 * c + 1][qt][u]) * (PT[2 * c + 1][qt][u] - Dv[qt]);
        }
        sf[qt] = as_bf16x8(pack8(ds));
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 a = vt_frag(Ks, 32 * c, dt, l16, lq);
#pragma unroll
        for (int qt = 0; qt < SB_QT; ++qt) QT[dt][qt] = mfma16x16x32(a, sf[qt], QT[dt][qt]);
      }
    }
  };
  for (int e = 0; e < nsel - 1; ++e) {
    step(e, false);
    const int ahead = min(2, nsel - 2 - e);
    if (ahead >= 2) wait_vmcnt<2 * DMA_PER_WAVE>();
    else if (ahead == 1) wait_vmcnt<DMA_PER_WAVE>();
    else wait_vmcnt<0>();
    __syncthreads();
  }
  if (nsel > 0) step(nsel - 1, true);

  // ---- dq = RMSNorm^T: lane holds dq^[row][16dt + 4lq + e] for its rows
  float wsum[8][4];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) wsum[dt][e] = 0.f;
#pragma unroll
  for (int qt = 0; qt < SB_QT; ++qt) {
    const long t = it.i * 64 + qrow0 + 16 * qt + l16 - q0;
    const bool ok = it.head_ok && t < n_q;
    const long base = ((long)(it.b * (long)n_q + (ok ? t : 0)) * Hq + it.h) * D;
    float x[8][4];
    float ss = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 u = make_uint2(0, 0);
      if (ok) u = *reinterpret_cast<const uint2*>(q + base + 16 * dt + 4 * lq);
      x[dt][0] = bf2f(u.x & 0xffffu);
      x[dt][1] = bf2f(u.x >> 16);
      x[dt][2] = bf2f(u.y & 0xffffu);
      x[dt][3] = bf2f(u.y >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(x[dt][e], x[dt][e], ss);
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
    float dot = 0.f, dn[8][4];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dim = 16 * dt + 4 * lq + e;
        const float n = x[dt][e] * inv;
        const float dy = scale * QT[dt][qt][e];
        dn[dt][e] = dy * (qw ? qw[dim] : 1.0f);
        dot = fmaf(dn[dt][e], n, dot);
        if (ok) wsum[dt][e] = fmaf(n, dy, wsum[dt][e]);
      }
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    dot *= 1.0f / D;
    if (ok) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (dn[dt][e] - x[dt][e] * inv * dot) * inv;
        *reinterpret_cast<f32x4*>(dq + base + 16 * dt + 4 * lq) = o;
      }
    }
  }
  // norm-weight partial sums of this workgroup (in a fixed order: lanes, then waves)
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = wsum[dt][e];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      s += __shfl_xor(s, 8, 64);
      if (l16 == 0) red[wave][16 * dt + 4 * lq + e] = s;
    }
  __syncthreads();
  if (j < D) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) s += red[w][j];
    wpart[(long)blockIdx.x * D + j] = s;
  }
}

// ---- 3. the selection inverted
__global__ void __launch_bounds__(256)
sbwd_zero_kernel(uint32_t* __restrict__ p, long n) {
  for (long x = (long)blockIdx.x * 256 + threadIdx.x; x < n; x += (long)gridDim.x * 256) p[x] = 0u;
}

// bit r of row [bg][blk] <- query block r selected block blk (entries outside [0, nkb) ignored)
__global__ void __launch_bounds__(256)
sbwd_bitmap_kernel(const int32_t* __restrict__ sel, uint32_t* __restrict__ bm, int nqb, int topk, int nkb,
                   int words) {
  const long row = blockIdx.x;  // (bg, r)
  const int r = (int)(row % nqb);
  const long bg = row / nqb;
  for (int x = threadIdx.x; x < topk; x += 256) {
    const int blk = sel[row * topk + x];
    if (blk >= 0 && blk < nkb) atomicOr(&bm[(bg * nkb + blk) * words + (r >> 5)], 1u << (r & 31));
  }
}

// per (b, g): slice offsets soff[blk] = sum over earlier key blocks of ceil(count / SB_SL)
__global__ void __launch_bounds__(1024)
sbwd_slices_kernel(const uint32_t* __restrict__ bm, int* __restrict__ soff, int nkb, int words, int nw) {
  // entry e = w * nkb + kb: the query blocks of range w that chose key block kb; soff[e] = the
  // first slice of the entry (entries in order), soff[nw * nkb] = the slice count
  __shared__ int part[1024];
  const long bg = blockIdx.x;
  const int ne = nw * nkb;
  int carry = 0;
  for (int c0 = 0; c0 < ne; c0 += 1024) {
    const int e = c0 + threadIdx.x;
    int ns = 0;
    if (e < ne) {
      const int w = e / nkb, blk = e % nkb;
      const int w1 = min(words, (w + 1) * SB_RWW);
      int cnt = 0;
      for (int x = w * SB_RWW; x < w1; ++x) cnt += __popc(bm[(bg * nkb + blk) * words + x]);
      ns = (cnt + SB_SL - 1) / SB_SL;
    }
    part[threadIdx.x] = ns;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan
      const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    if (e < ne) soff[bg * (ne + 1) + e] = carry + part[threadIdx.x] - ns;
    carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) soff[bg * (ne + 1) + ne] = carry;
}

// ---- 4. dK, dV per slice: workgroups of four waves, two per CU, so that one workgroup's
// gathers and barriers overlap the other's products. Wave w owns key tile w (16 keys) for all
// 64 queries of a step: its K and V fragments stay in registers and it accumulates dK^T, dV^T
// of its keys over every step. LDS holds a double buffer of the (q~, dO, stats) tiles of one
// (query block, head) step.
constexpr int SB_KV_NT = 256;
struct DkvLds {
  bf16_t qd[2][2][TILE];  // [buffer][q~, dO]
  float st[2][64 * 4];    // [buffer][row][lse2, D, -, -]
  int list[SB_SL];
  int n;
};

// copies of one step: q~ and dO tiles in the swzv layout (16 pieces of 1 KB each, wave w moves
// 4w .. 4w+3 of both) and, by wave 0, the 1 KB stats rows. The step's tile base is a scalar
// address (pad0: its first padded row); a lane adds its fixed byte offset loff[m] (row
// 4I + lane/16 of piece I = 4w + m, the source chunk the swzv layout puts at position lane % 16),
// so the copies take no vector address arithmetic. wave: the wave index as a uniform value.
__device__ __forceinline__ void dkv_lane_offsets(int wave, uint32_t (&loff)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int row = 4 * (4 * wave + m) + (lane >> 4);
    loff[m] = 2u * (uint32_t)(row * D + 8 * ((lane & 15) ^ (2 * (row & 7))));
  }
}
__device__ __forceinline__ void dma_step(const bf16_t* qtb, const bf16_t* dob, const float* stb, long pad0,
                                         const uint32_t (&loff)[4], DkvLds& L, int bufi, int wave) {
  const int lane = threadIdx.x & 63;
  const bf16_t* qb = qtb + pad0 * D;
  const bf16_t* db = dob + pad0 * D;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int I = 4 * wave + m;
    dma16s(qb, loff[m], (uint32_t)(size_t)(L.qd[bufi][0] + I * 512));
    dma16s(db, loff[m], (uint32_t)(size_t)(L.qd[bufi][1] + I * 512));
  }
  if (wave == 0) dma16(stb + pad0 * 4 + 4 * lane, lds_addr_u32(L.st[bufi]));
}

__global__ void __launch_bounds__(SB_KV_NT, 2)
sbwd_dkv_kernel(const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, const bf16_t* __restrict__ qtb,
                const bf16_t* __restrict__ dob, const float* __restrict__ stb, const uint32_t* __restrict__ bm,
                const int* __restrict__ soff, float* __restrict__ part, int Hq, int Hkv, long qb0, int nqb,
                long kv_len, long cap, int nkb, int words, int nw, int maxsl) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  DkvLds& L = *reinterpret_cast<DkvLds*>(lds_raw);
  const int bg = blockIdx.x / maxsl, s = blockIdx.x % maxsl;
  const int ne = nw * nkb;
  const int* so = soff + (long)bg * (ne + 1);
  if (s >= so[ne]) return;
  // entry of slice s: the last e with so[e] <= s (range w = e / nkb, key block e % nkb)
  int lo = 0, hi = ne - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (so[mid] <= s) lo = mid; else hi = mid - 1;
  }
  const int kb = lo % nkb, wr = lo / nkb, rank0 = (s - so[lo]) * SB_SL;
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6, l16 = lane & 15, lq = lane >> 4;
  const int G = Hq / Hkv, b = bg / Hkv, gk = bg % Hkv;
  if (j == 0) {
    const uint32_t* rowp = bm + ((long)bg * nkb + kb) * words;
    int seen = 0, n = 0;
    for (int w = wr * SB_RWW; w < min(words, (wr + 1) * SB_RWW) && n < SB_SL; ++w) {
      uint32_t bits = rowp[w];
      while (bits && n < SB_SL) {
        const int bit = __builtin_ctz(bits);
        bits &= bits - 1;
        if (seen >= rank0) L.list[n++] = 32 * w + bit;
        ++seen;
      }
    }
    L.n = n;
  }
  __syncthreads();  // the list
  const int nl = L.n, nsteps = nl * G;
  auto pad_of = [&](int st) -> long {
    const int r = __builtin_amdgcn_readfirstlane(L.list[st / G]), hh = st % G;
    return ((long)b * Hq + gk * G + hh) * nqb * 64 + (long)r * 64;
  };
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t loff[4];
  dkv_lane_offsets(wave_u, loff);
  if (nsteps > 0) dma_step(qtb, dob, stb, pad_of(0), loff, L, 0, wave_u);

  const int kt = wave;  // key tile
  // this wave's K and V fragments (B operand: key 16kt + l16, dims 32ks + 8lq .. +7); rows past
  // kv_len repeat the last row (only the diagonal block reaches them, where they are masked)
  bf16x8 kf[4], vf[4];
  {
    long p = (long)kb * 64 + 16 * kt + l16;
    if (p >= kv_len) p = kv_len - 1;
    const long off = ((long)bg * cap + p) * D + 8 * lq;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(kc + off + 32 * ks));
      vf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(vc + off + 32 * ks));
    }
  }

  f32x4 dKT[8], dVT[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dKT[dt] = dVT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < nsteps; ++st) {
    const int bi = st & 1;
    wait_vmcnt<0>();  // this step's copies have landed
    __syncthreads();  // visible to all; every wave is done with the other buffer
    if (st + 1 < nsteps) dma_step(qtb, dob, stb, pad_of(st + 1), loff, L, bi ^ 1, wave_u);
    const bf16_t* Qs = L.qd[bi][0];
    const bf16_t* Ds = L.qd[bi][1];
    const float* S4 = L.st[bi];
    const bool diag = qb0 + L.list[st / G] == kb;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {  // query half: rows 32qh .. 32qh + 31
      // every LDS operand of the scores and dP products is read ahead of them
      float2 ld[8];  // (lse2, D) of query row 32qh + 16qt + 4lq + e
      bf16x8 qa[2][4], da[2][4];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ld[4 * qt + e] = *reinterpret_cast<const float2*>(S4 + (32 * qh + 16 * qt + 4 * lq + e) * 4);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          qa[qt][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(Qs + swzv(32 * qh + 16 * qt + l16, 4 * ks + lq)));
          da[qt][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(Ds + swzv(32 * qh + 16 * qt + l16, 4 * ks + lq)));
        }
      // C layout: query 32qh + 16qt + 4lq + e, key 16kt + l16; S starts at -lse2
      f32x4 S[2], P[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        S[qt] = f32x4{-ld[4 * qt].x, -ld[4 * qt + 1].x, -ld[4 * qt + 2].x, -ld[4 * qt + 3].x};
        P[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          S[qt] = mfma16x16x32(qa[qt][ks], kf[ks], S[qt]);
          P[qt] = mfma16x16x32(da[qt][ks], vf[ks], P[qt]);  // dP
        }
      bf16x8 tv[8];  // dO^T fragments of this half, read while the products run
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) tv[dt] = vt_frag(Ds, 32 * qh, dt, l16, lq);
      float pv[8], dsv[8];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qrow = 32 * qh + 16 * qt + 4 * lq + e, key = 16 * kt + l16;
          float s2 = S[qt][e];
          if (diag && key > qrow) s2 = -INFINITY;  // key after query
          const float p = fast_exp2(s2);
          pv[4 * qt + e] = p;
          dsv[4 * qt + e] = p * (P[qt][e] - ld[4 * qt + e].y);
        }
      const bf16x8 pf = as_bf16x8(pack8(pv)), sf = as_bf16x8(pack8(dsv));
      bf16x8 tk[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) tk[dt] = vt_frag(Qs, 32 * qh, dt, l16, lq);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) dVT[dt] = mfma16x16x32(tv[dt], pf, dVT[dt]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) dKT[dt] = mfma16x16x32(tk[dt], sf, dKT[dt]);
    }
  }
  // dK carries 1 / log2(e) since q~ holds scale * log2(e) * q^. C layout: dk / dv dim
  // 16dt + 4lq + e, key 16kt + l16
  float* dst = part + ((long)bg * maxsl + s) * 2 * 64 * D + (long)(16 * kt + l16) * D + 4 * lq;
  const float ln2 = 0.69314718055994531f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    *reinterpret_cast<f32x4*>(dst + 16 * dt) = dKT[dt] * ln2;
    *reinterpret_cast<f32x4*>(dst + 64L * D + 16 * dt) = dVT[dt];
  }
}

// ---- 5. per key block: dK, dV rows = sum of its slices (0 for blocks no query selected and
// for capacity rows past kv_len's last block)
__global__ void __launch_bounds__(256)
sbwd_reduce_kernel(const float* __restrict__ part, const int* __restrict__ soff, float* __restrict__ dk,
                   float* __restrict__ dv, long cap, int nkb, int nw, int maxsl) {
  const long nbc = cap / 64;
  const int bg = (int)(blockIdx.x / nbc), kb = (int)(blockIdx.x % nbc);
  const int ne = nw * nkb;
  const int* so = soff + (long)bg * (ne + 1);
  for (int x = threadIdx.x; x < 64 * D / 4; x += 256) {
    f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = ak;
    // the key block's slices, range by range
    for (int w = 0; kb < nkb && w < nw; ++w)
      for (int sl = so[w * nkb + kb]; sl < so[w * nkb + kb + 1]; ++sl) {
        const float* src = part + ((long)bg * maxsl + sl) * 2 * 64 * D;
        ak += *reinterpret_cast<const f32x4*>(src + 4 * x);
        av += *reinterpret_cast<const f32x4*>(src + 64 * D + 4 * x);
      }
    const long o = ((long)bg * cap + (long)kb * 64) * D + 4 * x;
    *reinterpret_cast<f32x4*>(dk + o) = ak;
    *reinterpret_cast<f32x4*>(dv + o) = av;
  }
}

// sum of per-workgroup norm-weight partials: one block per dim, fixed reduction order
__global__ void __launch_bounds__(256)
sbwd_wsum_kernel(const float* __restrict__ wpart, long nparts, float* __restrict__ dw) {
  __shared__ float red[256];
  const int dim = blockIdx.x;
  float s = 0.f;
  for (long p = threadIdx.x; p < nparts; p += 256) s += wpart[p * D + dim];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) dw[dim] = red[0];
}

// ---- key-norm transpose for the appended tokens: dk = RMSNorm^T(dk^ rows of the cache),
// per-block norm-weight partials. 16 lanes per row (8 dims each), 16 rows per block.
__global__ void __launch_bounds__(256)
sbwd_knorm_kernel(const bf16_t* __restrict__ k, const float* __restrict__ kw, const float* __restrict__ dkc,
                  float* __restrict__ dk, float* __restrict__ wpart, long nrows, int n_q, int Hkv, long p0, long cap,
                  float eps) {
  __shared__ float red[16][D];
  const int l = threadIdx.x & 15, rl = threadIdx.x >> 4;
  float ws[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ws[e] = 0.f;
  for (long r0 = (long)blockIdx.x * 16; r0 < nrows; r0 += (long)gridDim.x * 16) {
    const long row = r0 + rl < nrows ? r0 + rl : nrows - 1;  // (b, t, g)
    const bool ok = r0 + rl < nrows;
    const long gq = row % Hkv, t = (row / Hkv) % n_q, b = row / ((long)Hkv * n_q);
    float x[8], dy[8];
    unpack8(*reinterpret_cast<const uint4*>(k + row * D + 8 * l), x);
    const float* src = dkc + ((b * Hkv + gq) * cap + p0 + t) * D + 8 * l;
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(src), d1 = *reinterpret_cast<const f32x4*>(src + 4);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dy[e] = e < 4 ? d0[e] : d1[e - 4];
      ss = fmaf(x[e], x[e], ss);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
    float dn[8], dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float n = x[e] * inv;
      dn[e] = dy[e] * (kw ? kw[8 * l + e] : 1.0f);
      dot = fmaf(dn[e], n, dot);
      if (ok) ws[e] = fmaf(n, dy[e], ws[e]);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dot += __shfl_xor(dot, o, 64);
    dot *= 1.0f / D;
    if (ok) {
      f32x4 o0, o1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o0[e] = (dn[e] - x[e] * inv * dot) * inv;
        o1[e] = (dn[4 + e] - x[4 + e] * inv * dot) * inv;
      }
      *reinterpret_cast<f32x4*>(dk + row * D + 8 * l) = o0;
      *reinterpret_cast<f32x4*>(dk + row * D + 8 * l + 4) = o1;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rl][8 * l + e] = ws[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int r = 0; r < 16; ++r) s += red[r][threadIdx.x];
    wpart[(long)blockIdx.x * D + threadIdx.x] = s;
  }
}

constexpr int KN_BLOCKS_MAX = 2048;

struct SbwdPlan {
  long nqb, nkb, words, nw, maxsl, nwg;
  size_t off_qt, off_do, off_st, off_bm, off_soff, off_part, off_wpart, total;
};

SbwdPlan sbwd_plan(const sala_sparse_desc& d) {
  const SparseGeom gm = sparse_geom(d);
  SbwdPlan p;
  const long BG = (long)d.batch * d.n_kv_heads, BH = (long)d.batch * d.n_heads;
  const int G = d.n_heads / d.n_kv_heads;
  p.nqb = gm.nqb;
  p.nkb = (d.kv_len + 63) / 64;
  p.words = (p.nqb + 31) / 32;
  p.nw = (p.words + SB_RWW - 1) / SB_RWW;
  // slices: sum over (range, key block) of ceil(count / SB_SL) <= pairs / SB_SL + entries
  p.maxsl = (p.nqb * d.topk + SB_SL - 1) / SB_SL + std::min(p.nw * p.nkb, p.nqb * (long)d.topk);
  p.nwg = BG * p.nqb * ((G + 3) / 4);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += (bytes + 255) & ~size_t(255); return o; };
  const size_t prow = (size_t)BH * p.nqb * 64;
  p.off_qt = take(prow * D * 2);
  p.off_do = take(prow * D * 2);
  p.off_st = take(prow * 4 * 4);
  p.off_bm = take((size_t)BG * p.nkb * p.words * 4);
  p.off_soff = take((size_t)BG * (p.nw * p.nkb + 1) * 4);
  p.off_part = take((size_t)BG * p.maxsl * 2 * 64 * D * 4);
  p.off_wpart = take((size_t)p.nwg * D * 4);
  p.total = off;
  return p;
}

}  // namespace

size_t sparse_attn_backward_workspace(const sala_sparse_desc& d) { return sbwd_plan(d).total; }

size_t kv_norm_backward_workspace(const sala_sparse_desc& d) {
  const long nrows = (long)d.batch * d.n_q * d.n_kv_heads;
  return (size_t)std::min<long>((nrows + 15) / 16, KN_BLOCKS_MAX) * D * 4;
}

hipError_t launch_sparse_attn_backward(const sala_sparse_desc& d, const void* q, const float* qw, const void* k_cache,
                                       const void* v_cache, const void* g, const int32_t* sel, const void* dout,
                                       const void* out, const float* lse, float* dq, float* dk_cache, float* dv_cache,
                                       float* dg, float* dqw, void* ws, hipStream_t st) {
  const SparseGeom gm = sparse_geom(d);
  const SbwdPlan p = sbwd_plan(d);
  char* w = static_cast<char*>(ws);
  bf16_t* qtb = reinterpret_cast<bf16_t*>(w + p.off_qt);
  bf16_t* dob = reinterpret_cast<bf16_t*>(w + p.off_do);
  float* stb = reinterpret_cast<float*>(w + p.off_st);
  uint32_t* bm = reinterpret_cast<uint32_t*>(w + p.off_bm);
  int* soff = reinterpret_cast<int*>(w + p.off_soff);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  float* wpart = reinterpret_cast<float*>(w + p.off_wpart);
  const long BG = (long)d.batch * d.n_kv_heads;
  const float qscale = gm.scale * 1.4426950408889634f;
  const bf16_t *qb = (const bf16_t*)q, *kb = (const bf16_t*)k_cache, *vb = (const bf16_t*)v_cache;

  if (out && lse) {
    const long nprow = (long)d.batch * d.n_heads * p.nqb * 64;
    hipLaunchKernelGGL(sbwd_prep_kernel, dim3((unsigned)(nprow / 64)), dim3(256), 0, st, qb, qw, (const bf16_t*)g,
                       (const bf16_t*)dout, (const bf16_t*)out, lse, dg, qtb, dob, stb, d.n_q, d.n_heads,
                       (long)gm.q0, (long)gm.qb0, (int)p.nqb, d.norm_eps, qscale);
  } else {
    hipLaunchKernelGGL(sbwd_stats_kernel, dim3((unsigned)p.nwg), dim3(SB_NT), 0, st, qb, qw, kb, vb, (const bf16_t*)g,
                       sel, (const bf16_t*)dout, dg, qtb, dob, stb, d.n_q, d.n_heads, d.n_kv_heads, (long)gm.q0,
                       (long)gm.qb0, (int)p.nqb, (long)d.kv_len, (long)d.kv_capacity, d.topk, d.norm_eps, qscale);
  }
  hipLaunchKernelGGL(sbwd_dq_kernel, dim3((unsigned)p.nwg), dim3(SB_NT), 0, st, qb, qw, kb, vb, sel, qtb, dob, stb,
                     dq, wpart, d.n_q, d.n_heads, d.n_kv_heads, (long)gm.q0, (long)gm.qb0, (int)p.nqb, (long)d.kv_len,
                     (long)d.kv_capacity, d.topk, d.norm_eps, gm.scale);
  if (dqw) hipLaunchKernelGGL(sbwd_wsum_kernel, dim3(D), dim3(256), 0, st, wpart, p.nwg, dqw);
  const long nbm = BG * p.nkb * p.words;
  hipLaunchKernelGGL(sbwd_zero_kernel, dim3((unsigned)std::min<long>((nbm + 255) / 256, 4096)), dim3(256), 0, st, bm,
                     nbm);
  hipLaunchKernelGGL(sbwd_bitmap_kernel, dim3((unsigned)(BG * p.nqb)), dim3(256), 0, st, sel, bm, (int)p.nqb, d.topk,
                     (int)p.nkb, (int)p.words);
  hipLaunchKernelGGL(sbwd_slices_kernel, dim3((unsigned)BG), dim3(1024), 0, st, bm, soff, (int)p.nkb, (int)p.words,
                     (int)p.nw);
  static const hipError_t attr_ok = hipFuncSetAttribute((const void*)sbwd_dkv_kernel,
                                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                                        (int)sizeof(DkvLds));
  if (attr_ok != hipSuccess) return attr_ok;
  hipLaunchKernelGGL(sbwd_dkv_kernel, dim3((unsigned)(BG * p.maxsl)), dim3(SB_KV_NT), sizeof(DkvLds), st, kb, vb, qtb,
                     dob, stb, bm, soff, part, d.n_heads, d.n_kv_heads, (long)gm.qb0, (int)p.nqb, (long)d.kv_len,
                     (long)d.kv_capacity, (int)p.nkb, (int)p.words, (int)p.nw, (int)p.maxsl);
  hipLaunchKernelGGL(sbwd_reduce_kernel, dim3((unsigned)(BG * (d.kv_capacity / 64))), dim3(256), 0, st, part, soff,
                     dk_cache, dv_cache, (long)d.kv_capacity, (int)p.nkb, (int)p.nw, (int)p.maxsl);
  return hipGetLastError();
}

hipError_t launch_kv_norm_backward(const sala_sparse_desc& d, const void* k_new, const float* kw,
                                   const float* dk_cache, float* dk_new, float* dkw, void* ws, hipStream_t st) {
  const long nrows = (long)d.batch * d.n_q * d.n_kv_heads;
  const int blocks = (int)std::min<long>((nrows + 15) / 16, KN_BLOCKS_MAX);
  float* wpart = static_cast<float*>(ws);
  hipLaunchKernelGGL(sbwd_knorm_kernel, dim3(blocks), dim3(256), 0, st, (const bf16_t*)k_new, kw, dk_cache, dk_new,
                     wpart, nrows, d.n_q, d.n_kv_heads, (long)(d.kv_len - d.n_q), (long)d.kv_capacity, d.norm_eps);
  if (dkw) hipLaunchKernelGGL(sbwd_wsum_kernel, dim3(D), dim3(256), 0, st, wpart, (long)blocks, dkw);
  return hipGetLastError();
}

}  // namespace sala
