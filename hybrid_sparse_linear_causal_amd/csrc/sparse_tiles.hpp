// Tile helpers of the bf16 sparse-attention kernels (forward and backward): the LDS layouts of
// a staged 64-key block, its DMA, and one wave's scores / online-softmax / O-update pieces.
// Pages: "面壁智能发布MiniCPM-SALA：稀疏-线性混合架构，9B模型端侧跑通百万上下文，速度飙升3.5倍",
// section "SALA混合架构：黄金配比破解瓶颈" (attention over the selected key blocks only).
#pragma once

#include "common.hpp"

namespace sala {
namespace {

constexpr int SP_D = 128;  // head dim of the bf16 paths

constexpr int TILE = 64 * SP_D;  // bf16 elements per 64-row tile
constexpr int NSTAGE = 4;       // LDS ring depth (blocks resident or in flight)

// The staged K and V tiles use the swzv layout (V and, in the backward, K are read transposed;
// row reads stay conflict-free in it); the scores read K in swzv (KV) or swz.

// One 64-key block (K and V tiles, 16 KB each = 16 pieces of 1 KB) is copied into a stage by
// the 8 waves of a workgroup, wave w moving pieces 2w and 2w+1 (rows 8w .. 8w+7) of both tiles:
// DMA_PER_WAVE instructions. Lane l of a piece fills chunk position l % 16 of row 4I + l / 16,
// so it loads the source chunk that the tile's swizzle puts there. Rows at or beyond kv_len are
// clamped to the last valid row: they are causally masked (K) or weighted 0 (V).
constexpr int DMA_PER_WAVE = 4;

// The copy keeps the block's addresses in scalar registers: the lane's part of the
// address is a 32-bit byte offset inside the block (saddr form of global_load_lds_dwordx4), and
// both tiles use the swzv layout, so the K and V copies of a row share that offset. A lane's
// offsets (rows 4I + lane/16 of pieces I = 2*wave and 2*wave+1, chunk positions
// (lane % 16) ^ 2(row & 7)) are set up once by dma_lane_setup; per block only the clamp of rows
// past the cache (lim = last valid row of the block, 0 <= lim <= 63) and the shift remain.
// kb, vb: the block's first row in K and V; Ks, Vs: the stage's tiles; wave: the wave index as
// a wave-uniform value.
struct DmaLane {
  int row[2];        // row of the block this lane copies for piece 2*wave + m
  uint32_t chk[2];   // byte offset of the source chunk within the row
};
__device__ __forceinline__ DmaLane dma_lane_setup(int wave) {
  const int lane = threadIdx.x & 63;
  DmaLane d;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int row = 4 * (2 * wave + m) + (lane >> 4);
    d.row[m] = row;
    d.chk[m] = 16u * (uint32_t)((lane & 15) ^ (2 * (row & 7)));
  }
  return d;
}
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_block_s(const DmaLane& d, const bf16_t* kb, const bf16_t* vb, int lim,
                                            bf16_t* Ks, bf16_t* Vs, int wave) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int r = d.row[m] < lim ? d.row[m] : lim;
    const uint32_t off = ((uint32_t)r << 8) + d.chk[m];
    const int I = 2 * wave + m;
    dma16s(kb, off, (uint32_t)(size_t)(Ks + I * 512));
    dma16s(vb, off, (uint32_t)(size_t)(Vs + I * 512));
  }
}

// dma_block_s of selected block blk of the cache rows starting at row_base (blk and the
// arguments wave-uniform); an entry past the cache (a malformed selection) reads the cache's last
// block, whose rows past kv_len repeat its last valid row
__device__ __forceinline__ void dma_block_sel(const DmaLane& d, const bf16_t* kc, const bf16_t* vc, long row_base,
                                              int blk, long kv_len, bf16_t* Ks, bf16_t* Vs, int wave) {
  const int last_blk = (int)((kv_len - 1) / 64);
  int bk = __builtin_amdgcn_readfirstlane(blk);
  if (bk > last_blk) bk = last_blk;
  const long off = (row_base + (long)bk * 64) * SP_D;
  dma_block_s(d, kc + off, vc + off, bk == last_blk ? (int)((kv_len - 1) % 64) : 63, Ks, Vs, wave);
}

// A operand V^T (rows dv = 16*dt + l16, k = keys in the permuted order of the P^T fragments:
// slots 0..3 = keys kb + 4*lq + e, slots 4..7 = keys kb + 16 + 4*lq + e) via two
// transposing reads. Source lane (i = l16) points at key row kb(+16) + 4*lq + i/4, columns
// 16*dt + 4*(i%4).
__device__ __forceinline__ bf16x8 vt_frag(const bf16_t* Vs, int kb, int dt, int l16, int lq) {
  const int row0 = kb + 4 * lq + (l16 >> 2);
  const int col = 16 * dt + 4 * (l16 & 3);          // element column; chunk = col / 8
  const int ch = col >> 3, sub = col & 7;
  const uint2 a = ds_read_tr(Vs + swzv(row0, ch) + sub);
  const uint2 b = ds_read_tr(Vs + swzv(row0 + 16, ch) + sub);
  return as_bf16x8(a, b);
}


// ---- pieces of one wave's work on a staged 64-key block for its QT x 16 query rows (rows
// qrow0 + 16*qt + l16 of the query block)

// S^T[kt][qt] = K[kt] Q^T[qt] - m[qt] (scores in log2 units: scale*log2(e) is folded into q;
// the running reference m enters as the accumulator's initial value, minit = -m)
template <int QT, bool KV = false>
__device__ __forceinline__ void scores(const bf16_t* Ks, const bf16x8 (&qf)[QT][4], const f32x4 (&minit)[QT],
                                       f32x4 (&ST)[4][QT], int l16) {
  const int lq = (threadIdx.x & 63) >> 4;
  // two key tiles per k-step: 2*QT independent accumulators between reuses of one
#pragma unroll
  for (int kp = 0; kp < 4; kp += 2) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kt = kp; kt < kp + 2; ++kt) {
        const int off = KV ? swzv(16 * kt + l16, 4 * ks + lq) : swz(16 * kt + l16, 4 * ks + lq);
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Ks + off));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) ST[kt][qt] = mfma16x16x32(a, qf[qt][ks], ks == 0 ? minit[qt] : ST[kt][qt]);
      }
    }
  }
}

// causal mask of the query's own block: key after query -> -inf
template <int QT>
__device__ __forceinline__ void mask_diag(f32x4 (&ST)[4][QT], int l16, int lq, int qrow0) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (16 * kt + 4 * lq + c > qrow0 + 16 * qt + l16) ST[kt][qt][c] = -INFINITY;
}

// Online softmax with a lazily raised reference. The score accumulators already hold s - m,
// so the probabilities are plain exp2 of them. A 32-key half whose per-lane partial sum exceeds
// P_LIMIT (some probability above 2^20), and the first half the row ever sees, raise m to the
// half's row maximum first: the running output and sum are rescaled, and the not yet consumed
// scores (this block and the next one, already issued with the old reference) are shifted.
// The reference is always a score of the row, so the row's largest probability is >= 1.
constexpr float P_LIMIT = 1048576.0f;  // 2^20

template <int QT>
__device__ __forceinline__ void exp_half(const f32x4 (&ST)[4][QT], int c, float (&p)[QT][8], float (&part)[QT]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      p[qt][u] = fast_exp2(ST[2 * c][qt][u]);
      p[qt][4 + u] = fast_exp2(ST[2 * c + 1][qt][u]);
    }
    part[qt] = ((p[qt][0] + p[qt][1]) + (p[qt][2] + p[qt][3])) + ((p[qt][4] + p[qt][5]) + (p[qt][6] + p[qt][7]));
  }
}

template <int QT>
__device__ __forceinline__ void raise_ref(f32x4 (&ST)[4][QT], f32x4 (&SN)[4][QT], f32x4 (&OT)[8][QT], float (&m)[QT],
                                       f32x4 (&minit)[QT], float (&lp)[QT], int c, bool first) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) mx = fmaxf(mx, fmaxf(ST[2 * c][qt][u], ST[2 * c + 1][qt][u]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float delta = first ? mx : fmaxf(mx, 0.0f);
    if (!first) {
      const float alpha = fast_exp2(-delta);
      lp[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) OT[dt][qt] *= alpha;
    }
    m[qt] += delta;
    minit[qt] = f32x4{-m[qt], -m[qt], -m[qt], -m[qt]};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      ST[kt][qt] -= delta;
      SN[kt][qt] -= delta;
    }
  }
}

// P^T = exp2(S^T) per 32-key half, O^T += V^T P^T (P^T straight from the accumulators)
template <int QT>
__device__ __forceinline__ void exp_pv(const bf16_t* Vs, f32x4 (&ST)[4][QT], f32x4 (&SN)[4][QT], f32x4 (&OT)[8][QT],
                                       float (&m)[QT], f32x4 (&minit)[QT], float (&lp)[QT], int l16, int lq,
                                       bool first) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float p[QT][8], part[QT];
    exp_half<QT>(ST, c, p, part);
    bool big = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) big |= part[qt] > P_LIMIT;
    if (__builtin_expect(__any(big) || (first && c == 0), 0)) {
      raise_ref<QT>(ST, SN, OT, m, minit, lp, c, first && c == 0);
      exp_half<QT>(ST, c, p, part);
    }
    bf16x8 pf[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      lp[qt] += part[qt];
      pf[qt] = as_bf16x8(pack8(p[qt]));
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8 a = vt_frag(Vs, 32 * c, dt, l16, lq);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) OT[dt][qt] = mfma16x16x32(a, pf[qt], OT[dt][qt]);
    }
  }
}

}  // namespace
}  // namespace sala
