// Block-sparse softmax attention with output gate for the sparse layer.
//
// Pages: "面壁智能发布MiniCPM-SALA：稀疏-线性混合架构，9B模型端侧跑通百万上下文，速度飙升3.5倍", section
// "SALA混合架构：黄金配比破解瓶颈" — each query attends only to the key/value pairs of the blocks
// the selection picked; no positional encoding in this layer. "MiniCPM-SALA：融合稀疏与线性注意力
// 实现高效长上下文建模" opening summary — QK normalisation in every layer, an output gate after
// every attention block. For query t at position p in block i, head h of KV group g:
//   out[t, h] = softmax_s(scale * q^ . k_s) . v_s * sigmoid(gate[t, h]),
//   s ranging over tokens s <= p of the blocks in sel[g, i].
//
// bf16 prefill (d = 128): one workgroup per (b, g, query block, 4 query heads); 8 waves, each
// owning 32 query rows of one head. Every selected block's 64x128 K and V tiles are copied into
// a 4-stage LDS ring by global->LDS DMA and shared by the 8 waves. Per wave and block:
//   S^T = K Q^T - m  (MFMA 16x16x32; queries are the MFMA columns; the running reference m
//                 enters as the accumulator's initial value)
//   P^T = exp2(S^T)  (scale*log2(e) folded into q; the reference is raised lazily, only when a
//                 probability could exceed 2^20)
//   O^T += V^T P^T   (P^T comes straight from the S^T accumulators: the 16x16x32 k-index is
//                 permuted consistently for both operands, so no cross-lane moves; V^T
//                 fragments come from transposing LDS reads)
// The scores of block e+1 are issued before the probabilities of block e (software pipeline).
// bf16 decode (n_q = 1): split over the selected blocks (one block per wave), the query
// heads of the GQA group are the 16 MFMA columns; partial (max, sum, output) are combined by
// a second kernel that also applies the gate.
// f32 (any shape, correctness-scale inputs): one thread per query row, keys from LDS.
#include "common.hpp"
#include "varlen.hpp"
#include "launch.hpp"
#include "sparse_tiles.hpp"

namespace sala {

namespace {

constexpr int D = 128;
constexpr int DEC_SPLIT = 16;       // decode workgroups per (b, g)

// ---- work geometry of the prefill kernel: which (sequence b, KV group gk, query block r of
// the call, head quad hq) a workgroup handles, where the call's query tokens of sequence b sit
// (tok0: packed index of its first one; q0: its position; n_q: their count), the cache length
// and the row of `sel`.
struct AttnItem {
  int b, gk, r, hq, n_q;
  long q0, tok0, kv_len, sel_row;
};
// B sequences with the same n_q queries at positions [q0, q0 + n_q) (tensors [B, n_q, Hq, d])
struct AttnUniform {
  int n_q, nqb;
  long q0, kv_len;
  __device__ __forceinline__ AttnItem item(unsigned w, int Hkv, int nhq) const {
    AttnItem it;
    it.hq = w % nhq;
    unsigned rest = w / nhq;
    it.r = rest % nqb;
    rest /= nqb;
    it.gk = rest % Hkv;
    it.b = rest / Hkv;
    it.n_q = n_q;
    it.q0 = q0;
    it.tok0 = (long)it.b * n_q;
    it.kv_len = kv_len;
    it.sel_row = ((long)it.b * Hkv + it.gk) * nqb + it.r;
    return it;
  }
};
// packed sequences (tensors [T, Hq, d]); sequence s has n[s] queries at positions pos0[s] ..,
// pos0[s] a multiple of 64, and a cache of pos0[s] + n[s] tokens. item0 = prefix of
// nqb_s * Hkv * nhq; aux0 = prefix of nqb_s (its rows of `sel` are Hkv * aux0[s] ..)
struct AttnVarlen {
  VarlenTable t;
  __device__ __forceinline__ AttnItem item(unsigned w, int Hkv, int nhq) const {
    const int s = vl_seq(t, (int)w);
    const int nqb = t.aux0[s + 1] - t.aux0[s];
    const unsigned x = w - t.item0[s];
    AttnItem it;
    it.b = s;
    it.hq = x % nhq;
    const unsigned rest = x / nhq;
    it.r = rest % nqb;
    it.gk = rest / nqb;
    it.n_q = t.n[s];
    it.q0 = t.pos0[s];
    it.tok0 = t.tok0[s];
    it.kv_len = t.pos0[s] + t.n[s];
    it.sel_row = (long)Hkv * t.aux0[s] + (long)it.gk * nqb + it.r;
    return it;
  }
};

// grid: one workgroup per item (B*Hkv*nqb*ceil(G/4) for uniform batches) of 512 threads (8
// waves: 4 heads x 2 row halves)
constexpr int PF_THREADS = 512;
constexpr int PF_QT = 2;  // 16-row query tiles per wave
template <bool DENSE, class Geo>
__global__ void __launch_bounds__(PF_THREADS)
sparse_prefill_bf16_kernel(const bf16_t* __restrict__ q, const float* __restrict__ qw,
                           const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
                           const bf16_t* __restrict__ g, const int32_t* __restrict__ sel,
                           bf16_t* __restrict__ out, float* __restrict__ lse, int Hq, int Hkv, long cap, int topk,
                           float eps, float qscale, Geo geo) {
  __shared__ __align__(16) bf16_t lds[NSTAGE][2][TILE];  // [stage][K|V]
  __shared__ int s_sel[256];
  const int G = Hq / Hkv, nhq = (G + 3) / 4;
  // XCD-aware order: workgroup x runs on XCD x % 8; give each XCD a contiguous run of work
  const unsigned nwg = gridDim.x;
  unsigned w = blockIdx.x;
  if ((nwg & 7u) == 0) w = (blockIdx.x & 7u) * (nwg >> 3) + (blockIdx.x >> 3);
  const AttnItem it = geo.item(w, Hkv, nhq);
  const int hq = it.hq, r = it.r, gk = it.gk, b = it.b, n_q = it.n_q;
  const long q0 = it.q0, kv_len = it.kv_len, qb0 = q0 / 64;

  const int j = threadIdx.x, lane = j & 63, wave = j >> 6, l16 = lane & 15, lq = lane >> 4;
  const int hl = 4 * hq + (wave >> 1);
  const int qrow0 = 32 * (wave & 1);  // this wave's first query row in the block
  const bool head_ok = hl < G;
  const int h = gk * G + (head_ok ? hl : 0);
  const long i = qb0 + r;
  const long row_base = ((long)b * Hkv + gk) * cap;
  // the loads first: the selection row (oldest, so that waiting for it leaves the query loads
  // in flight), then this wave's query rows (row addresses clamped into the call: rows past it
  // are zeroed after the load)
  int selv = -1;
  if (!DENSE && j < topk) selv = sel[it.sel_row * topk + j];
  uint4 qraw[PF_QT][4];
  bool qok[PF_QT];
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    const long t = i * 64 + qrow0 + 16 * qt + l16 - q0;
    qok[qt] = head_ok && t < n_q;
    const long tc = t < n_q ? t : n_q - 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qraw[qt][ks] = *reinterpret_cast<const uint4*>(q + ((it.tok0 + tc) * Hq + h) * D + 32 * ks + 8 * lq);
  }
  if (!DENSE && j < topk) s_sel[j] = selv;
  __syncthreads();
  // the blocks attended: the selection (ascending, -1 padded, ends with block i), or every
  // block 0 .. i. nsel = the index of the row's first -1 (or topk).
  int nsel = 0;
  if (DENSE) nsel = (int)(i + 1);
  else {
    nsel = topk;
#pragma unroll
    for (int u = 3; u >= 0; --u) {
      const int x = lane + 64 * u;
      const unsigned long long bad = __ballot(x < topk && s_sel[x] < 0);
      if (bad) nsel = 64 * u + (int)__builtin_ctzll(bad);
    }
  }
  auto blk = [&](int x) -> long { return DENSE ? (long)x : (long)s_sel[x]; };
  // block copies with scalar block addresses (K and V tiles both in the swzv layout); an entry
  // past the cache (a malformed row) is read as the cache's last block
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const DmaLane dl = dma_lane_setup(wave_u);
  const int last_blk = (int)((kv_len - 1) / 64), last_row = (int)((kv_len - 1) % 64);
  auto copy_block = [&](int x, int s) {
    int bk = DENSE ? x : __builtin_amdgcn_readfirstlane(s_sel[x]);
    if (bk > last_blk) bk = last_blk;
    const long off = (row_base + (long)bk * 64) * D;
    dma_block_s(dl, kc + off, vc + off, bk == last_blk ? last_row : 63, lds[s][0], lds[s][1], wave_u);
  };
  // the query-norm weights this lane applies, loaded before the copies are issued
  float qwv[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) qwv[ks][e] = qw ? qw[32 * ks + 8 * lq + e] : 1.0f;
  // the first three blocks' copies, issued before the query rows are normalised
#pragma unroll
  for (int x = 0; x < 3; ++x)
    if (x < nsel) copy_block(x, x);

  // ---- Q^T fragments (B operand: k = dim, n = query); normalised, scaled by scale*log2(e)
  bf16x8 qf[PF_QT][4];
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    float x[4][8];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = qraw[qt][ks];
      if (!qok[qt]) u = make_uint4(0, 0, 0, 0);
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
      for (int e = 0; e < 8; ++e) y[e] = x[ks][e] * inv * qwv[ks][e];
      uint4 u = pack8(y);
      // opaque to the optimiser: keep the packed fragment instead of recomputing it per block
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
      qf[qt][ks] = as_bf16x8(u);
    }
  }

  float m[PF_QT], lp[PF_QT];
  f32x4 minit[PF_QT];
  f32x4 OT[8][PF_QT];
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    m[qt] = 0.f;  // replaced by the row maximum of the first half-block
    lp[qt] = 0.f;
    minit[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt = 0; qt < PF_QT; ++qt) OT[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over the selected blocks (ring of NSTAGE = 4 stages, block e in stage
  // e % 4): iteration e computes the scores of block e+1 on MFMA while the exponentials of
  // block e run on VALU, then O^T += V^T P^T for block e. Blocks e+2 and e+3 are in flight.
  // The selection is ascending and always ends with the query's own block i, so the causal
  // diagonal block is the last one and is finished after the loop.
  if (nsel > 2) wait_vmcnt<DMA_PER_WAVE>(); else wait_vmcnt<0>();  // blocks 0 and 1 landed
  __syncthreads();

  f32x4 SA[4][PF_QT], SB[4][PF_QT];
  scores<PF_QT, true>(lds[0][0], qf, minit, SA, l16);
  // With 4 or more blocks, the gate rows of the output pass are copied into LDS during the last
  // step: wave w's 32 rows (8 KB) into stage nsel % 4 (waves 0-3) or (nsel + 1) % 4 (waves 4-7),
  // whose blocks were consumed before that step. Copy I = 4qt + dp, lane L: row qrow0 + 16qt +
  // (L >> 1) % 16, 16-byte chunk 2dt + (L & 1) of dims, dt = 2dp + L / 32; the lanes of the
  // output pass then read 512 contiguous bytes per (qt, dt).
  const bool g_lds = !DENSE && nsel >= 4;
  bf16_t* gtile = lds[(nsel + (wave >> 2)) & 3][0] + (wave & 3) * 4096;
  auto gate_copy = [&]() {
#pragma unroll
    for (int I = 0; I < 8; ++I) {
      const int qt = I >> 2, dt = 2 * (I & 3) + (lane >> 5), rr = (lane >> 1) & 15, c = 2 * dt + (lane & 1);
      const long t = i * 64 + qrow0 + 16 * qt + rr - q0;
      const long tc = t < n_q ? t : n_q - 1;
      dma16(g + ((it.tok0 + tc) * Hq + h) * D + 8 * c, lds_addr_u32(gtile + I * 512));
    }
  };
  auto step = [&](int e, f32x4 (&Sc)[4][PF_QT], f32x4 (&Sn)[4][PF_QT]) {
    const bool more = e + 3 < nsel;
    if (more) copy_block(e + 3, (e + 3) & 3);
    scores<PF_QT, true>(lds[(e + 1) & 3][0], qf, minit, Sn, l16);
    exp_pv<PF_QT>(lds[e & 3][1], Sc, Sn, OT, m, minit, lp, l16, lq, e == 0);
    // block e+2 must have landed (only block e+3's copies may still be in flight); after the
    // last step only the diagonal block is read, which the previous step's wait and barrier
    // already cover, so the last step neither waits nor synchronises
    if (DENSE || e < nsel - 2) {
      if (more) wait_vmcnt<DMA_PER_WAVE>(); else wait_vmcnt<0>();
      __syncthreads();
    }
  };
  int e = 0;
  if constexpr (DENSE) {
    for (; e + 2 <= nsel - 1; e += 2) {
      step(e, SA, SB);
      step(e + 1, SB, SA);
    }
    if (e < nsel - 1) {
      step(e, SA, SB);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < PF_QT; ++qt) SA[kt][qt] = SB[kt][qt];
    }
  } else {
    // steps 0 .. nsel-3, then the last step nsel-2 with the gate copies issued first
    const int last = nsel - 2;
    for (; e + 2 <= last; e += 2) {
      step(e, SA, SB);
      step(e + 1, SB, SA);
    }
    if (e < last) {
      step(e, SA, SB);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < PF_QT; ++qt) SA[kt][qt] = SB[kt][qt];
      ++e;
    }
    if (e == last) {
      if (g_lds) gate_copy();
      step(e, SA, SB);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < PF_QT; ++qt) SA[kt][qt] = SB[kt][qt];
    }
  }
  // diagonal block (index nsel-1); SB only receives the (unused) shift of a raised reference
  mask_diag<PF_QT>(SA, l16, lq, qrow0);
  exp_pv<PF_QT>(lds[(nsel - 1) & 3][1], SA, SB, OT, m, minit, lp, l16, lq, nsel == 1);
  // this wave's gate copies have landed (also where the wave stores nothing: no copy into LDS
  // outlives the wave)
  if (g_lds) wait_vmcnt<0>();
  if (!head_ok) return;

  // ---- normalise, gate, store (lane: query qrow0 + 16qt + l16, dims 16dt + 4lq .. +3)
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    float l = lp[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float il = 1.0f / l;
    const long t = i * 64 + qrow0 + 16 * qt + l16 - q0;
    if (t >= n_q) continue;
    const long base = ((it.tok0 + t) * Hq + h) * D;
    // log2-domain log-sum-exp of the row's scaled scores (m is a score of the row, l >= 1)
    if (lse && lq == 0) lse[(it.tok0 + t) * Hq + h] = m[qt] + __log2f(l);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const long off = base + 16 * dt + 4 * lq;
      const uint2 gw = g_lds ? *reinterpret_cast<const uint2*>(gtile + (4 * qt + (dt >> 1)) * 512 +
                                                            8 * (32 * (dt & 1) + 2 * l16 + (lq >> 1)) + 4 * (lq & 1))
                             : *reinterpret_cast<const uint2*>(g + off);
      const float g0 = __uint_as_float(gw.x << 16), g1 = __uint_as_float(gw.x & 0xffff0000u);
      const float g2 = __uint_as_float(gw.y << 16), g3 = __uint_as_float(gw.y & 0xffff0000u);
      uint2 o;
      o.x = pack_bf16x2(OT[dt][qt][0] * il * fast_sigmoid(g0), OT[dt][qt][1] * il * fast_sigmoid(g1));
      o.y = pack_bf16x2(OT[dt][qt][2] * il * fast_sigmoid(g2), OT[dt][qt][3] * il * fast_sigmoid(g3));
      *reinterpret_cast<uint2*>(out + off) = o;
    }
  }
}

// ------------------------------------------------------------------ decode (n_q = 1)

// grid (B*Hkv, DEC_SPLIT); wave-global index wi = split*4 + wave takes sel entries
// wi, wi + 4*DEC_SPLIT, ... Partial per workgroup: m[16], l[16], O[16][D] (fp32).
// Each wave owns a V tile in LDS: its block's V rows arrive there by DMA, in the swizzled
// row-major layout of the prefill kernel, and leave as V^T operands through transposing reads.
constexpr int DEC_OSTR = D + 4;  // fp32 row stride of the O staging (rows at one column spread over banks)
template <bool DENSE>
__global__ void __launch_bounds__(256)
sparse_decode_bf16_kernel(const bf16_t* __restrict__ q, const float* __restrict__ qw,
                          const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
                          const int32_t* __restrict__ sel, float* __restrict__ part, int Hq,
                          int Hkv, long kv_len, long cap, int topk, float eps, float qscale,
                          const int64_t* __restrict__ kv_lens) {
  __shared__ __align__(16) bf16_t vts[4][TILE];
  __shared__ float cm[4][16], cl[4][16];
  __shared__ float csc[4][16], cM[16], cL[16];
  const int bg = blockIdx.x, split = blockIdx.y;
  const int b = bg / Hkv, gk = bg % Hkv, G = Hq / Hkv;
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6, l16 = lane & 15, lq = lane >> 4;
  // the query rows first, so that their loads overlap those of the selection row
  const bool ok = l16 < G;
  uint4 qraw[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qraw[ks] = ok ? *reinterpret_cast<const uint4*>(q + ((long)b * Hq + gk * G + l16) * D + 32 * ks + 8 * lq)
                  : make_uint4(0, 0, 0, 0);
  if (kv_lens) {  // this sequence's own cache length, clamped to [1, kv_len]
    const long kb = kv_lens[b];
    kv_len = kb < 1 ? 1 : (kb > kv_len ? kv_len : kb);
  }
  const long p = kv_len - 1;
  const long row_base = (long)bg * cap;
  // the selection row (ascending, -1 padded; topk <= 256): lane x holds entries x + 64u
  int sv[4] = {-1, -1, -1, -1};
  int nsel = (int)(p / 64 + 1);  // dense: every block 0 .. i
  if (!DENSE) {
    const int32_t* srow = sel + (long)bg * topk;
#pragma unroll
    for (int u = 0; u < 4; ++u) sv[u] = lane + 64 * u < topk ? srow[lane + 64 * u] : -1;
    nsel = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) nsel += __popcll(__ballot(sv[u] >= 0));
  }

  // Q^T fragments: column l16 = head gk*G + l16 (zero beyond the group)
  bf16x8 qf[4];
  {
    float x[4][8];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      unpack8(qraw[ks], x[ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[ks][e] * x[ks][e];
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = qscale / sqrtf(ss * (1.0f / D) + eps);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[ks][e] * inv * (qw ? qw[32 * ks + 8 * lq + e] : 1.0f);
      qf[ks] = as_bf16x8(pack8(y));
    }
  }

  float m = -INFINITY, lp = 0.f;
  f32x4 OT[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) OT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int stride = 4 * DEC_SPLIT;
  bf16_t* vt = vts[wave];  // this wave's own V tile: no workgroup barrier needed
  for (int e = split * 4 + wave; e < nsel; e += stride) {
    const int su = e >> 6;
    long blk = DENSE ? (long)e : (long)__shfl(su == 0 ? sv[0] : su == 1 ? sv[1] : su == 2 ? sv[2] : sv[3], e & 63, 64);
    if (blk < 0) blk = 0;  // a malformed row (-1 before its end) must not read before the cache
    // K in MFMA A layout (key 16kt + l16, dims 32ks + 8lq ..) into registers
    uint4 kk[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const long pk = blk * 64 + 16 * kt + l16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kk[kt][ks] = pk < kv_len ? *reinterpret_cast<const uint4*>(kc + (row_base + pk) * D + 32 * ks + 8 * lq)
                                 : make_uint4(0, 0, 0, 0);
    }
    // V rows by DMA into the wave's tile: piece I = rows 4I .. 4I+3, lane -> chunk position
    // lane % 16 of row 4I + lane / 16, loading the source chunk the swizzle puts there. Rows
    // past the cache are clamped to its last row: their probabilities are 0.
#pragma unroll
    for (int I = 0; I < 16; ++I) {
      const int row = 4 * I + (lane >> 4);
      const int chv = (lane & 15) ^ (2 * (row & 7));
      long pk = blk * 64 + row;
      if (pk >= kv_len) pk = kv_len - 1;
      dma16(vc + (row_base + pk) * D + 8 * chv, lds_addr_u32(vt + I * 512));
    }
    f32x4 ST[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      ST[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ST[kt] = mfma16x16x32(as_bf16x8(kk[kt][ks]), qf[ks], ST[kt]);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (blk * 64 + 16 * kt + 4 * lq + c > p) ST[kt][c] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, ST[kt][c]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    lp *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) OT[dt] *= alpha;
    m = mn;
    wait_vmcnt<0>();  // the wave's V tile has landed (its DMA completes in issue order)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float pr[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pr[u] = exp2f(ST[2 * c][u] - m);
        pr[4 + u] = exp2f(ST[2 * c + 1][u] - m);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) lp += pr[u];
      const bf16x8 pf = as_bf16x8(pack8(pr));
      // P^T slots: keys 32c + 4lq + u, then 32c + 16 + 4lq + u, as vt_frag orders V^T
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) OT[dt] = mfma16x16x32(vt_frag(vt, 32 * c, dt, l16, lq), pf, OT[dt]);
    }
    // the tile is rewritten by this wave's next block: its reads have been consumed above
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();  // every wave is done with its V tile (reused below)
  // combine the 4 waves: O staged in the (now free) V area as fp32 [wave][head][DEC_OSTR]
  lp += __shfl_xor(lp, 16, 64);
  lp += __shfl_xor(lp, 32, 64);
  if (lq == 0) { cm[wave][l16] = m; cl[wave][l16] = lp; }
  float* ost = reinterpret_cast<float*>(&vts[0][0]);  // 4*16*DEC_OSTR floats = 33 KB <= sizeof(vts)
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<f32x4*>(&ost[(wave * 16 + l16) * DEC_OSTR + 16 * dt + 4 * lq]) = OT[dt];
  __syncthreads();
  // per head (threads 0..15): the workgroup's reference M, the waves' scales and the sum
  if (j < 16) {
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, cm[wv][j]);
    float l = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      const float sc = (cm[wv][j] == -INFINITY) ? 0.f : exp2f(cm[wv][j] - M);
      csc[wv][j] = sc;
      l += cl[wv][j] * sc;
    }
    cM[j] = M;
    cL[j] = l;
  }
  __syncthreads();
  // thread j: dim j % D of heads j / D + 2it (independent LDS reads, issued together)
  float* dst = part + ((long)bg * DEC_SPLIT + split) * 16 * (D + 2);
  const int dd = j % D;
#pragma unroll
  for (int it = 0; it < 16 * D / 256; ++it) {
    const int hh = j / D + 2 * it;
    float o = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) o += ost[(wv * 16 + hh) * DEC_OSTR + dd] * csc[wv][hh];
    dst[hh * (D + 2) + 2 + dd] = o;
  }
  if (j < 16) { dst[j * (D + 2)] = cM[j]; dst[j * (D + 2) + 1] = cL[j]; }
}

// grid (B*Hkv*G): one workgroup of D threads per (b, head); combine the DEC_SPLIT partials
// of the head's KV group, normalise, gate, store out[b, h, :]
__global__ void __launch_bounds__(D)
sparse_decode_combine_kernel(const float* __restrict__ part, const bf16_t* __restrict__ g,
                             bf16_t* __restrict__ out, int Hq, int Hkv) {
  const int G = Hq / Hkv;
  const int bg = blockIdx.x / G, hh = blockIdx.x % G;
  const int b = bg / Hkv, gk = bg % Hkv, dd = threadIdx.x;
  const long off = ((long)b * Hq + gk * G + hh) * D + dd;
  // the gate first: its load then overlaps those of the partials instead of following them
  const bf16_t gate = g[off];
  __builtin_amdgcn_sched_barrier(0);
  const float* src = part + ((long)bg * DEC_SPLIT * 16 + hh) * (D + 2);
  float ms[DEC_SPLIT], ls[DEC_SPLIT], os[DEC_SPLIT];
#pragma unroll
  for (int s = 0; s < DEC_SPLIT; ++s) {
    const float* ps = src + (long)s * 16 * (D + 2);
    ms[s] = ps[0];
    ls[s] = ps[1];
    os[s] = ps[2 + dd];
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < DEC_SPLIT; ++s) M = fmaxf(M, ms[s]);
  float o = 0.f, l = 0.f;
#pragma unroll
  for (int s = 0; s < DEC_SPLIT; ++s) {
    const float w = (ms[s] == -INFINITY) ? 0.f : fast_exp2(ms[s] - M);
    o += os[s] * w;
    l += ls[s] * w;
  }
  out[off] = f2bf(o / l * fast_sigmoid(bf2f(gate)));
}

// ------------------------------------------------------------------ fp32 path

// grid (B*Hq, nqb); 64 threads, thread = query row of the block; keys staged in LDS.
template <int DD, bool DENSE>
__global__ void __launch_bounds__(64)
sparse_attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ qw,
                       const float* __restrict__ kc, const float* __restrict__ vc,
                       const float* __restrict__ g, const int32_t* __restrict__ sel,
                       float* __restrict__ out, int n_q, int Hq, int Hkv, long q0, long qb0,
                       int nqb, long kv_len, long cap, int topk, float eps, float scale) {
  __shared__ float ks[64][DD], vs[64][DD];
  const int bh = blockIdx.x, r = blockIdx.y, b = bh / Hq, h = bh % Hq, G = Hq / Hkv, gk = h / G;
  const int lane = threadIdx.x;
  const long i = qb0 + r;
  const long pos = i * 64 + lane, t = pos - q0;
  const bool ok = t >= 0 && t < n_q;
  float qv[DD], acc[DD];
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < DD; ++d) {
    qv[d] = ok ? q[(((long)b * n_q + t) * Hq + h) * DD + d] : 0.f;
    ss += qv[d] * qv[d];
    acc[d] = 0.f;
  }
  const float inv = scale / sqrtf(ss / DD + eps);
#pragma unroll
  for (int d = 0; d < DD; ++d) qv[d] *= inv * (qw ? qw[d] : 1.0f);
  float m = -INFINITY, l = 0.f;
  const int32_t* srow = DENSE ? nullptr : sel + (((long)b * Hkv + gk) * nqb + r) * topk;
  const long row_base = ((long)b * Hkv + gk) * cap;
  const long nblk = DENSE ? i + 1 : topk;
  for (long e = 0; e < nblk; ++e) {
    const long blk = DENSE ? e : (long)srow[e];
    if (blk < 0) break;
    __syncthreads();
    for (int idx = lane; idx < 64 * DD; idx += 64) {
      const int kk = idx / DD, dd = idx % DD;
      const long pk = blk * 64 + kk;
      ks[kk][dd] = pk < kv_len ? kc[(row_base + pk) * DD + dd] : 0.f;
      vs[kk][dd] = pk < kv_len ? vc[(row_base + pk) * DD + dd] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < 64; ++kk) {
      const long pk = blk * 64 + kk;
      if (pk > pos || pk >= kv_len) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DD; ++d) s += qv[d] * ks[kk][d];
      const float mn = fmaxf(m, s);
      const float alpha = expf(m - mn), pw = expf(s - mn);
      l = l * alpha + pw;
#pragma unroll
      for (int d = 0; d < DD; ++d) acc[d] = acc[d] * alpha + pw * vs[kk][d];
      m = mn;
    }
  }
  if (!ok) return;
  const long base = (((long)b * n_q + t) * Hq + h) * DD;
#pragma unroll
  for (int d = 0; d < DD; ++d) out[base + d] = acc[d] / l / (1.0f + expf(-g[base + d]));
}

}  // namespace

size_t sparse_attn_workspace(const sala_sparse_desc& d) {
  if (d.dtype == SALA_BF16 && d.n_q == 1)
    return (size_t)d.batch * d.n_kv_heads * DEC_SPLIT * 16 * (D + 2) * sizeof(float);
  return 0;
}

template <bool DENSE>
static hipError_t launch_attn(const sala_sparse_desc& d, const void* q, const float* qw,
                              const void* k_cache, const void* v_cache, const void* g,
                              const int32_t* sel, void* out, float* lse, void* ws, hipStream_t st) {
  const SparseGeom gm = sparse_geom(d);
  const int G = d.n_heads / d.n_kv_heads;
  if (d.dtype == SALA_F32) {
    const dim3 grid(d.batch * d.n_heads, (unsigned)gm.nqb);
    if (d.head_dim == 128)
      hipLaunchKernelGGL((sparse_attn_f32_kernel<128, DENSE>), grid, dim3(64), 0, st, (const float*)q, qw,
                         (const float*)k_cache, (const float*)v_cache, (const float*)g, sel, (float*)out,
                         d.n_q, d.n_heads, d.n_kv_heads, (long)gm.q0, (long)gm.qb0, (int)gm.nqb,
                         (long)d.kv_len, (long)d.kv_capacity, d.topk, d.norm_eps, gm.scale);
    else
      hipLaunchKernelGGL((sparse_attn_f32_kernel<64, DENSE>), grid, dim3(64), 0, st, (const float*)q, qw,
                         (const float*)k_cache, (const float*)v_cache, (const float*)g, sel, (float*)out,
                         d.n_q, d.n_heads, d.n_kv_heads, (long)gm.q0, (long)gm.qb0, (int)gm.nqb,
                         (long)d.kv_len, (long)d.kv_capacity, d.topk, d.norm_eps, gm.scale);
    return hipGetLastError();
  }
  const float qscale = gm.scale * 1.4426950408889634f;  // exp -> exp2
  if (d.n_q == 1) {
    float* part = static_cast<float*>(ws);
    hipLaunchKernelGGL(sparse_decode_bf16_kernel<DENSE>, dim3(d.batch * d.n_kv_heads, DEC_SPLIT), dim3(256), 0,
                       st, (const bf16_t*)q, qw, (const bf16_t*)k_cache, (const bf16_t*)v_cache, sel,
                       part, d.n_heads, d.n_kv_heads, (long)d.kv_len, (long)d.kv_capacity, d.topk,
                       d.norm_eps, qscale,
                       nullptr);
    hipLaunchKernelGGL(sparse_decode_combine_kernel, dim3(d.batch * d.n_heads), dim3(D), 0, st,
                       part, (const bf16_t*)g, (bf16_t*)out, d.n_heads, d.n_kv_heads);
    return hipGetLastError();
  }
  const long nwg = (long)d.batch * d.n_kv_heads * gm.nqb * ((G + 3) / 4);
  const AttnUniform geo{d.n_q, (int)gm.nqb, (long)gm.q0, (long)d.kv_len};
  hipLaunchKernelGGL((sparse_prefill_bf16_kernel<DENSE, AttnUniform>), dim3((unsigned)nwg), dim3(PF_THREADS), 0, st,
                     (const bf16_t*)q, qw, (const bf16_t*)k_cache, (const bf16_t*)v_cache, (const bf16_t*)g, sel,
                     (bf16_t*)out, lse, d.n_heads, d.n_kv_heads, (long)d.kv_capacity, d.topk, d.norm_eps, qscale,
                     geo);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const sala_sparse_desc& d, const void* q, const float* qw,
                              const void* k_cache, const void* v_cache, const void* g,
                              const int32_t* sel, void* out, float* lse, void* ws, hipStream_t st) {
  return launch_attn<false>(d, q, qw, k_cache, v_cache, g, sel, out, lse, ws, st);
}

hipError_t launch_dense_attn(const sala_sparse_desc& d, const void* q, const float* qw,
                             const void* k_cache, const void* v_cache, const void* g, void* out,
                             void* ws, hipStream_t st) {
  return launch_attn<true>(d, q, qw, k_cache, v_cache, g, nullptr, out, nullptr, ws, st);
}

int64_t varlen_query_blocks(int nseq, const int32_t* cu_seqlens) {
  int64_t n = 0;
  for (int s = 0; s < nseq; ++s) n += (cu_seqlens[s + 1] - cu_seqlens[s] + 63) / 64;
  return n;
}

hipError_t launch_sparse_attn_varlen(const sala_sparse_desc& d, const int32_t* cu_seqlens, const int64_t* pos0,
                                     const void* q, const float* qw, const void* k_cache, const void* v_cache,
                                     const void* g, const int32_t* sel, void* out, hipStream_t st) {
  const int nhq = (d.n_heads / d.n_kv_heads + 3) / 4;
  AttnVarlen geo{make_varlen_table(d.batch, cu_seqlens, pos0)};
  for (int s = 0; s < d.batch; ++s) {
    const int nqb = (geo.t.n[s] + 63) / 64;
    geo.t.aux0[s + 1] = geo.t.aux0[s] + nqb;
    geo.t.item0[s + 1] = geo.t.item0[s] + nqb * d.n_kv_heads * nhq;
  }
  const long nwg = geo.t.item0[d.batch];
  if (nwg == 0) return hipSuccess;
  const float qscale = sparse_geom(d).scale * 1.4426950408889634f;  // exp -> exp2
  hipLaunchKernelGGL((sparse_prefill_bf16_kernel<false, AttnVarlen>), dim3((unsigned)nwg), dim3(PF_THREADS), 0, st,
                     (const bf16_t*)q, qw, (const bf16_t*)k_cache, (const bf16_t*)v_cache, (const bf16_t*)g, sel,
                     (bf16_t*)out, nullptr, d.n_heads, d.n_kv_heads, (long)d.kv_capacity, d.topk, d.norm_eps, qscale,
                     geo);
  return hipGetLastError();
}

}  // namespace sala

namespace sala {

size_t sparse_decode_at_workspace(const sala_sparse_desc& d) {
  return (size_t)d.batch * d.n_kv_heads * DEC_SPLIT * 16 * (D + 2) * sizeof(float);
}

// decode attention with each sequence at its own cache length (device array kv_lens)
hipError_t launch_sparse_decode_at(const sala_sparse_desc& d, const int64_t* kv_lens, const void* q, const float* qw,
                                   const void* k_cache, const void* v_cache, const void* g, const int32_t* sel,
                                   void* out, void* ws, hipStream_t st) {
  const float qscale = sparse_geom(d).scale * 1.4426950408889634f;  // exp -> exp2
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(sparse_decode_bf16_kernel<false>, dim3(d.batch * d.n_kv_heads, DEC_SPLIT), dim3(256), 0, st,
                     (const bf16_t*)q, qw, (const bf16_t*)k_cache, (const bf16_t*)v_cache, sel, part, d.n_heads,
                     d.n_kv_heads, (long)d.kv_len, (long)d.kv_capacity, d.topk, d.norm_eps, qscale, kv_lens);
  hipLaunchKernelGGL(sparse_decode_combine_kernel, dim3(d.batch * d.n_heads), dim3(D), 0, st, part,
                     (const bf16_t*)g, (bf16_t*)out, d.n_heads, d.n_kv_heads);
  return hipGetLastError();
}

}  // namespace sala
