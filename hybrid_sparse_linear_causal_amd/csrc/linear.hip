// Linear-attention layer kernels for gfx950 (Lightning-style causal linear attention).
//
// Method (pages: "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" §1 and §2.1 — linear
// attention as an O(N) recurrence with a constant-size state; opening summary — QK-norm in
// every layer, RoPE in the linear layers, an output gate after every block). Per token at
// position p: q^, k^ = RoPE_p(RMSNorm(q), RMSNorm(k)); S += k^^T v; o = q^ S; out = o*sigmoid(g).
//
// bf16 prefill, d = 128. The recurrence is evaluated in 64-token chunks c:
//   O_c = (Q_c K_c^T (.) M_causal) V_c + Q_c S_{c-1},   S_c = S_{c-1} + K_c^T V_c
// which equals the token recurrence exactly in real arithmetic. All four products run on
// MFMA 16x16x32 (bf16 operands, fp32 accumulation); the state is kept in fp32 registers and
// handed to MFMA as bf16 once per chunk. To fill 256 CUs at batch 1 the sequence is cut into
// segments processed in parallel:
//   1. linear_segsum_kernel : per (b, h, segment s < last) the segment's sum of k^T v,
//                             written to workspace slot s + 1
//   2. linear_scan_kernel   : per (b, h): slot 0 = state_in (or 0), slot s = slot s-1 +
//                             slot s, i.e. the state entering segment s
//   3. linear_out_kernel    : per (b, h, segment) the chunk loop from its start state, writing
//                             gated outputs (and, last segment, the final state)
// With a single segment the workspace is unused and state_in is read directly. Reading the
// entering state from the workspace otherwise lets state_out alias state_in safely.
#include "common.hpp"
#include "launch.hpp"
#include "varlen.hpp"

#include <algorithm>

namespace sala {

namespace {

// ---- work geometry: which (sequence s, head h, segment) a workgroup handles, where the
// sequence's tokens start in the token dimension, and where its segment slots are. `slot` is
// the index (in d x d blocks) of the (s, h) run of nseg workspace slots.
struct LinItem {
  int s, h, seg, nseg, n;
  long tok0, pos0, slot;
};
// B sequences of N tokens each, all starting at position pos0 (tensors [B, N, H, d])
struct LinUniform {
  int N;
  long pos0;
  int nseg;
  // segsum: items exclude each (s, h)'s last segment
  __device__ __forceinline__ LinItem item(int x, int H, bool segsum) const {
    const int per = segsum ? nseg - 1 : nseg;
    LinItem it;
    it.seg = x % per;
    const int sh = x / per;
    it.s = sh / H;
    it.h = sh % H;
    it.nseg = nseg;
    it.n = N;
    it.tok0 = (long)it.s * N;
    it.pos0 = pos0;
    it.slot = (long)sh * nseg;
    return it;
  }
  // scan: (s, h) = x; returns the slot run and its length
  __device__ __forceinline__ long scan_item(int x, int H, int* nslots) const {
    *nslots = nseg;
    return (long)x * nseg;
  }
  // the slot run of KV head kvh of the item's sequence (segment sums and scan run per KV head)
  __device__ __forceinline__ long kv_slot(const LinItem& it, int Hkv, int kvh) const {
    return ((long)it.s * Hkv + kvh) * nseg;
  }
};
// packed sequences (tensors [T, H, d]): aux0 = prefix of the per-sequence segment counts;
// item0 = H * aux0 (output pass) or H * (aux0[s] - s) (segment sums)
struct LinVarlen {
  VarlenTable t;
  __device__ __forceinline__ LinItem item(int x, int H, bool segsum) const {
    const int s = vl_seq(t, x);
    const int nseg = t.aux0[s + 1] - t.aux0[s];
    const int per = segsum ? nseg - 1 : nseg;
    const int r = x - t.item0[s];
    LinItem it;
    it.s = s;
    it.h = r / per;
    it.seg = r % per;
    it.nseg = nseg;
    it.n = t.n[s];
    it.tok0 = t.tok0[s];
    it.pos0 = t.pos0[s];
    it.slot = (long)H * t.aux0[s] + (long)it.h * nseg;
    return it;
  }
  __device__ __forceinline__ long scan_item(int x, int H, int* nslots) const {
    const int s = x / H, h = x % H;
    *nslots = t.aux0[s + 1] - t.aux0[s];
    return (long)H * t.aux0[s] + (long)h * *nslots;
  }
  __device__ __forceinline__ long kv_slot(const LinItem& it, int Hkv, int kvh) const {
    return (long)Hkv * t.aux0[it.s] + (long)kvh * it.nseg;
  }
};

constexpr int D = 128;   // head dim of the bf16 MFMA path
constexpr int CH = 64;   // chunk length (tokens)

// QK-norm + RoPE of one token's 16 values held by this thread (two 8-dim halves that RoPE
// pairs), given the cos/sin of its 8 angles. The row's sum of squares is reduced over the 8
// lanes of the token. Returns the rotated values packed to bf16 in x.
__device__ __forceinline__ void norm_rope(uint4 (&x)[2], const float* w, int s, float eps,
                                          const float* cs, const float* sn) {
  float a[8], b[8];
  unpack8(x[0], a);
  unpack8(x[1], b);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(a[e], a[e], fmaf(b[e], b[e], ss));
  ss = group_sum8_dpp(ss);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
  float ra[8], rb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float xa = a[e], xb = b[e];
    if (w) { xa *= w[8 * s + e]; xb *= w[64 + 8 * s + e]; }
    const float c = cs[e] * inv, sg = sn[e] * inv;
    ra[e] = xa * c - xb * sg;
    rb[e] = xa * sg + xb * c;
  }
  x[0] = pack8(ra);
  x[1] = pack8(rb);
}

// norm_rope with the 16 norm weights of the thread's dims already in registers
__device__ __forceinline__ void norm_rope_w(uint4 (&x)[2], const float* w, float eps, const float* cs,
                                            const float* sn) {
  float a[8], b[8];
  unpack8(x[0], a);
  unpack8(x[1], b);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(a[e], a[e], fmaf(b[e], b[e], ss));
  ss = group_sum8_dpp(ss);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
  float ra[8], rb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xa = a[e] * w[e], xb = b[e] * w[8 + e];
    const float c = cs[e] * inv, sg = sn[e] * inv;
    ra[e] = xa * c - xb * sg;
    rb[e] = xa * sg + xb * c;
  }
  x[0] = pack8(ra);
  x[1] = pack8(rb);
}

// ---- segment sums: per (b, h, segment s < last) the sum over the segment of k~^T v, into
// workspace slot s + 1. The k and v tiles of the chunks stream through a ring of SS_NS stages
// by DMA (the next chunk lands while one is processed), k is normalised and rotated in place,
// and wave w accumulates rows 16w .. 16w+15 of the 128 x 128 sum. With two stages (64 KB) two
// workgroups share a CU, which measured faster than deeper rings with one workgroup per CU.
constexpr int SS_NT = 512;
constexpr int SS_NS = 2;
struct SegLds {
  bf16_t k[SS_NS][CH * D];  // [stage][token][dk]
  bf16_t v[SS_NS][CH * D];  // [stage][token][dv]
};
static_assert(sizeof(SegLds) == SS_NS * 32768, "segment-sum LDS plan");

// Both tiles are read only by transposing reads (4 rows x 2 chunks per 16 lanes, rows r and
// r + 8 in the same 32 lanes); chunk c of row r sits at position c ^ f(r) with
// f(r) = 2(r & 3) + 8((r >> 3) & 1), which gives those reads distinct banks.
__device__ __forceinline__ int swzt(int row, int chunk) {
  return row * 128 + 8 * (chunk ^ (2 * (row & 3) + 8 * ((row >> 3) & 1)));
}
__device__ __forceinline__ bf16x8 tr_frag_t(const bf16_t* T, int k0, int d1, int c0, int l16) {
  const int row = k0 + (l16 >> 2), col = c0 + 4 * (l16 & 3);
  const uint2 a = ds_read_tr(T + swzt(row, col >> 3) + (col & 7));
  const uint2 b = ds_read_tr(T + swzt(row + d1, col >> 3) + (col & 7));
  return as_bf16x8(a, b);
}
// DMA of one chunk's k and v tiles (32 pieces of 1 KB; wave w moves pieces 2w and 2w+1 of
// each): SS_DMA instructions per wave. The segment is whole, so every row exists.
constexpr int SS_DMA = 4;
__device__ __forceinline__ void dma_kv(const bf16_t* k, const bf16_t* v, long row0, long tok_stride,
                                       bf16_t* Ks, bf16_t* Vs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int I = 2 * wave + m;
    const int row = 4 * I + (lane >> 4);
    const int ch = (lane & 15) ^ (2 * (row & 3) + 8 * ((row >> 3) & 1));
    const long off = row0 + (long)row * tok_stride + 8 * ch;
    dma16(k + off, lds_addr_u32(Ks + I * 512));
    dma16(v + off, lds_addr_u32(Vs + I * 512));
  }
}

template <bool HAS_W, class Geo>
__global__ void __launch_bounds__(SS_NT)
linear_segsum_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                     const float* __restrict__ kw, float* __restrict__ ws, int H, int seg_len, float eps,
                     RopeFreqs freqs, Geo geo) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  SegLds& L = *reinterpret_cast<SegLds*>(lds_raw);
  const LinItem it = geo.item(blockIdx.x, H, true);
  const int seg = it.seg, h = it.h;
  const long pos0 = it.pos0;
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int s8 = j & 7, tok = j >> 3;  // prep: one token, segments s8 and s8+8
  const int t_begin = seg * seg_len;
  const int nch = seg_len / CH;
  const long tok_stride = (long)H * D;
  const long row0 = (it.tok0 * H + h) * D + (long)t_begin * tok_stride;

#pragma unroll
  for (int x = 0; x < SS_NS - 1; ++x)
    if (x < nch) dma_kv(k, v, row0 + (long)x * CH * tok_stride, tok_stride, L.k[x], L.v[x]);

  // Norm weights of this thread's 16 dims and its RoPE table, set up once (a memory load in
  // the loop would wait for the chunks in flight): cos/sin of its token's 8 angles, exact at
  // the segment start (fp64 reduction) and advanced by the rotation of 64 positions per chunk.
  float wk[16], rc[8], rs[8], ac[8], as[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wk[e] = HAS_W ? kw[8 * s8 + e] : 1.0f;
    wk[8 + e] = HAS_W ? kw[64 + 8 * s8 + e] : 1.0f;
    sincos_rev(rope_rev((double)(pos0 + t_begin + tok), freqs.f[8 * s8 + e]), &rs[e], &rc[e]);
    ac[e] = freqs.c64[8 * s8 + e];
    as[e] = freqs.s64[8 * s8 + e];
  }
  f32x4 S[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) S[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < nch; ++c) {
    const int st = c % SS_NS;
    // chunk c has landed once at most the chunks issued after it are in flight
    const int ahead = min(SS_NS - 2, nch - 1 - c);
    if (ahead >= 2) wait_vmcnt<2 * SS_DMA>();
    else if (ahead == 1) wait_vmcnt<SS_DMA>();
    else wait_vmcnt<0>();
    __syncthreads();  // chunk c visible to all; every wave is done with chunk c-1's stage
    if (c + SS_NS - 1 < nch)
      dma_kv(k, v, row0 + (long)(c + SS_NS - 1) * CH * tok_stride, tok_stride,
             L.k[(c + SS_NS - 1) % SS_NS], L.v[(c + SS_NS - 1) % SS_NS]);
    bf16_t* Kt = L.k[st];
    {
      uint4 x[2];
      x[0] = *reinterpret_cast<const uint4*>(&Kt[swzt(tok, s8)]);
      x[1] = *reinterpret_cast<const uint4*>(&Kt[swzt(tok, s8 + 8)]);
      norm_rope_w(x, wk, eps, rc, rs);
      *reinterpret_cast<uint4*>(&Kt[swzt(tok, s8)]) = x[0];
      *reinterpret_cast<uint4*>(&Kt[swzt(tok, s8 + 8)]) = x[1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c0 = rc[e], s0 = rs[e];
        rc[e] = c0 * ac[e] - s0 * as[e];
        rs[e] = s0 * ac[e] + c0 * as[e];
      }
    }
    __syncthreads();
    const bf16_t* Vt = L.v[st];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 af = tr_frag_t(Kt, 32 * ks + 8 * lq, 4, 16 * wave, l16);
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
        S[jt] = mfma16x16x32(af, tr_frag_t(Vt, 32 * ks + 8 * lq, 4, 16 * jt, l16), S[jt]);
    }
  }
  float* dst = ws + (it.slot + seg + 1) * D * D;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt)
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(16 * wave + 4 * lq + e) * D + 16 * jt + l16] = S[jt][e];
}

// ---- output pass: one workgroup per CU owning the whole 160 KB of LDS. The raw q, k, v and
// gate tiles of a chunk are copied global -> LDS by DMA one chunk ahead (double buffered), q
// and k are normalised and rotated in place, and the gated outputs are stored straight from
// the MFMA accumulators.
struct OutLds {
  bf16_t t[2][4][CH * D];  // [buffer][q, k, v, g][token][dim], swizzled 256-byte rows
  bf16_t st[D * D];        // S^T [dv][dk] bf16: the state entering the chunk
};
static_assert(sizeof(OutLds) == 163840, "output-pass LDS plan");

// DMA of one raw tile X (0 q, 1 k, 2 v, 3 g) of a chunk: 16 pieces of 1 KB shared by NW waves
// (NW 8: wave w moves pieces 2w, 2w+1; NW 4: waves 0-3 move pieces 4w .. 4w+3); q and g in the
// swz layout, k and v in swzv. The CU's vector memory path takes one 1 KB copy per 16 cycles
// and a wave stalls at issue while it is backed up (64 copies issued at once held the state
// waves for 1,900 cycles), so the next chunk's q and k are issued at the start of a chunk by
// every wave and its v and g after the prep by the output waves, which would otherwise wait
// for the state waves at the barrier. Rows past the sequence end are clamped to its last row
// (finite values; k rows past the end are zeroed by the prep, so they contribute nothing).
constexpr int OUT_NT = 512;  // 8 waves: 0-3 produce outputs, 4-7 update the state
// q and g rows start at row0 (H heads per token), k and v rows at kv_row0 (Hkv heads per token).
template <int X, int NW>
__device__ __forceinline__ void dma_chunk(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                          const bf16_t* g, long row0, long kv_row0, int t0, int n_valid, int H,
                                          int Hkv, bf16_t (*T)[CH * D]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr bool KV = X == 1 || X == 2;
  const bf16_t* src = X == 0 ? q : X == 1 ? k : X == 2 ? v : g;
  const long r0 = KV ? kv_row0 : row0;
  const long stride = (long)(KV ? Hkv : H) * D;
#pragma unroll
  for (int m = 0; m < 16 / NW; ++m) {
    const int I = (16 / NW) * wave + m;
    const int row = 4 * I + (lane >> 4);
    const int ch = KV ? (lane & 15) ^ (2 * (row & 7)) : (lane & 15) ^ (row & 15);
    const long off = r0 + (long)(min(t0 + row, n_valid - 1) - t0) * stride + 8 * ch;
    dma16(src + off, lds_addr_u32(T[X] + I * 512));
  }
}

template <bool HAS_W, class Geo>
__global__ void __launch_bounds__(OUT_NT)
linear_out_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                  const bf16_t* __restrict__ v, const bf16_t* __restrict__ g,
                  const float* __restrict__ qw, const float* __restrict__ kw,
                  const float* __restrict__ state_in, const float* __restrict__ ws,
                  float* __restrict__ state_out, bf16_t* __restrict__ out, int H, int Hkv, int seg_len,
                  float eps, RopeFreqs freqs, Geo geo) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  OutLds& L = *reinterpret_cast<OutLds*>(lds_raw);
  const LinItem it = geo.item(blockIdx.x, H, false);
  const int seg = it.seg, nseg = it.nseg, h = it.h, N = it.n;
  const long pos0 = it.pos0;
  // query head h reads (and, as every head of its group does, carries forward) the state of KV
  // head kvh; only the group's first head writes state_out
  const int G = H / Hkv, kvh = h / G;
  const long bh = (long)it.s * Hkv + kvh;  // state index
  const long kv_slot = geo.kv_slot(it, Hkv, kvh);
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const bool out_wave = wave < 4;
  const int w4 = wave & 3;      // query tile (output waves) or dk row block (state waves)
  const int s8 = j & 7, tok = j >> 3;  // prep: one token, segments s8 and s8+8
  const int t_begin = seg * seg_len;
  const int t_end = min(N, t_begin + seg_len);
  const long head_off = (it.tok0 * H + h) * D;
  const long tok_stride = (long)H * D;
  const long kv_off = (it.tok0 * Hkv + kvh) * D;
  const long kv_stride = (long)Hkv * D;

  {
    const long r0 = head_off + (long)t_begin * tok_stride, k0 = kv_off + (long)t_begin * kv_stride;
    dma_chunk<0, 8>(q, k, v, g, r0, k0, t_begin, N, H, Hkv, L.t[0]);
    dma_chunk<1, 8>(q, k, v, g, r0, k0, t_begin, N, H, Hkv, L.t[0]);
    dma_chunk<2, 8>(q, k, v, g, r0, k0, t_begin, N, H, Hkv, L.t[0]);
    dma_chunk<3, 8>(q, k, v, g, r0, k0, t_begin, N, H, Hkv, L.t[0]);
  }

  // acc: state waves keep S[dk][dv] (C layout, dk rows 32*w4 .. +31) in acc[8*it + jt];
  // output waves use acc[0..7] for their O^T tiles. One array, so the roles share registers.
  f32x4 acc[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (!out_wave) {
    // grouped heads read the entering state from the workspace even with one segment: the
    // group's first head may write state_out over state_in while the others still read it
    const float* src = (nseg == 1 && G == 1) ? (state_in ? state_in + bh * D * D : nullptr)
                                             : ws + (kv_slot + seg) * D * D;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dk = 32 * w4 + 16 * it + 4 * lq + e, dv = 16 * jt + l16;
          acc[8 * it + jt][e] = src ? src[dk * D + dv] : 0.f;
        }
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) {
        uint2 p;
        p.x = pack_bf16x2(acc[8 * it + jt][0], acc[8 * it + jt][1]);
        p.y = pack_bf16x2(acc[8 * it + jt][2], acc[8 * it + jt][3]);
        const int dk0 = 32 * w4 + 16 * it + 4 * lq, dv = 16 * jt + l16;
        *reinterpret_cast<uint2*>(&L.st[swz(dv, dk0 >> 3) + (dk0 & 7)]) = p;
      }
  }
  // norm weights of this thread's 16 dims (segments s8 and s8+8), loaded once: a load inside
  // the chunk loop would wait for the in-flight copies of the next chunk
  float wq[16], wk[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wq[e] = HAS_W && qw ? qw[8 * s8 + e] : 1.0f;
    wq[8 + e] = HAS_W && qw ? qw[64 + 8 * s8 + e] : 1.0f;
    wk[e] = HAS_W && kw ? kw[8 * s8 + e] : 1.0f;
    wk[8 + e] = HAS_W && kw ? kw[64 + 8 * s8 + e] : 1.0f;
  }

  // RoPE of this thread's token: cos/sin of its 8 angles, exact at the segment start (fp64
  // reduction) and advanced by the rotation of 64 positions per chunk, as the segment-sum pass
  // does (so both passes rotate k identically); set up once (indexing the argument block per
  // lane compiles to memory loads)
  float rc[8], rs[8], ac[8], as[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sincos_rev(rope_rev((double)(pos0 + t_begin + tok), freqs.f[8 * s8 + e]), &rs[e], &rc[e]);
    ac[e] = freqs.c64[8 * s8 + e];
    as[e] = freqs.s64[8 * s8 + e];
  }

  wait_vmcnt<0>();
  __syncthreads();
  int buf = 0;
  for (int c0 = t_begin; c0 < t_end; c0 += CH) {
    bf16_t* Qt = L.t[buf][0];
    bf16_t* Kt = L.t[buf][1];
    const bf16_t* Vt = L.t[buf][2];
    const bf16_t* Gt = L.t[buf][3];
    // the next chunk's tiles stream into the other buffer (free since the last barrier) for
    // the rest of this chunk: q and k now, v and g after the prep
    const bool next = c0 + CH < t_end;
    const long nrow0 = head_off + (long)(c0 + CH) * tok_stride, nkv0 = kv_off + (long)(c0 + CH) * kv_stride;
    bf16_t (*nbuf)[CH * D] = L.t[buf ^ 1];
    if (next) {
      dma_chunk<0, 8>(q, k, v, g, nrow0, nkv0, c0 + CH, N, H, Hkv, nbuf);
      dma_chunk<1, 8>(q, k, v, g, nrow0, nkv0, c0 + CH, N, H, Hkv, nbuf);
    }
    // ---------------- prep in place: QK-norm + RoPE (rows past the end: k~ = 0)
    {
      uint4 xq[2], xk[2];
      xq[0] = *reinterpret_cast<const uint4*>(&Qt[swz(tok, s8)]);
      xq[1] = *reinterpret_cast<const uint4*>(&Qt[swz(tok, s8 + 8)]);
      xk[0] = *reinterpret_cast<const uint4*>(&Kt[swzv(tok, s8)]);
      xk[1] = *reinterpret_cast<const uint4*>(&Kt[swzv(tok, s8 + 8)]);
      norm_rope_w(xq, wq, eps, rc, rs);
      norm_rope_w(xk, wk, eps, rc, rs);
      if (c0 + tok >= t_end) { xk[0] = make_uint4(0, 0, 0, 0); xk[1] = xk[0]; }
      *reinterpret_cast<uint4*>(&Qt[swz(tok, s8)]) = xq[0];
      *reinterpret_cast<uint4*>(&Qt[swz(tok, s8 + 8)]) = xq[1];
      *reinterpret_cast<uint4*>(&Kt[swzv(tok, s8)]) = xk[0];
      *reinterpret_cast<uint4*>(&Kt[swzv(tok, s8 + 8)]) = xk[1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = rc[e], s = rs[e];
        rc[e] = c * ac[e] - s * as[e];
        rs[e] = s * ac[e] + c * as[e];
      }
    }
    if (next && out_wave) {
      dma_chunk<2, 4>(q, k, v, g, nrow0, nkv0, c0 + CH, N, H, Hkv, nbuf);
      dma_chunk<3, 4>(q, k, v, g, nrow0, nkv0, c0 + CH, N, H, Hkv, nbuf);
    }
    __syncthreads();

    const int tl = 16 * w4 + l16;
    if (out_wave) {
      // ---------------- intra-chunk: O^T = V^T (K~ Q~^T (.) causal) for queries 16w..16w+15
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 qfrag[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qfrag[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(&Qt[swz(tl, 4 * ks + lq)]));
      for (int c = 0; 2 * c <= w4; ++c) {
        f32x4 at[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kt = 2 * c + hh;
          at[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (kt <= w4) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4*>(&Kt[swzv(16 * kt + l16, 4 * ks + lq)]));
              at[hh] = mfma16x16x32(kf, qfrag[ks], at[hh]);
            }
            if (kt == w4) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (4 * lq + e > l16) at[hh][e] = 0.f;  // key after query: masked
            }
          }
        }
        uint4 pb;
        pb.x = pack_bf16x2(at[0][0], at[0][1]);
        pb.y = pack_bf16x2(at[0][2], at[0][3]);
        pb.z = pack_bf16x2(at[1][0], at[1][1]);
        pb.w = pack_bf16x2(at[1][2], at[1][3]);
        const bf16x8 pfrag = as_bf16x8(pb);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          acc[dt] = mfma16x16x32(tr_frag_v(Vt, 32 * c + 4 * lq, 16, 16 * dt, l16), pfrag, acc[dt]);
      }
      // ---------------- inter-chunk: O^T += S^T Q~^T
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 sf = as_bf16x8(*reinterpret_cast<const uint4*>(&L.st[swz(16 * dt + l16, 4 * ks + lq)]));
          acc[dt] = mfma16x16x32(sf, qfrag[ks], acc[dt]);
        }
    } else {
      // ---------------- state update: S += K~^T V (dk rows 32*w4 .. +31, all dv); the token
      // index k runs over 32ks + 4lq + 0..3 and 32ks + 16 + 4lq + 0..3, the same for both operands
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 af[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) af[it] = tr_frag_v(Kt, 32 * ks + 4 * lq, 16, 32 * w4 + 16 * it, l16);
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          const bf16x8 bfr = tr_frag_v(Vt, 32 * ks + 4 * lq, 16, 16 * jt, l16);
#pragma unroll
          for (int it = 0; it < 2; ++it) acc[8 * it + jt] = mfma16x16x32(af[it], bfr, acc[8 * it + jt]);
        }
      }
      // the gate tile becomes sigmoid(g) in place (bf16; elementwise, so the swizzle does not
      // matter) while the output waves are still busy
      bf16_t* Gw = L.t[buf][3];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint4* p = reinterpret_cast<uint4*>(Gw) + (j - 256) + 256 * m;
        float x[8];
        unpack8(*p, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = fast_sigmoid(x[e]);
        *p = pack8(x);
      }
    }
    __syncthreads();  // every read of this chunk's S^T, q~, k~, v tiles is done; g holds sigmoid(g)
    if (out_wave) {
      // gated outputs staged in this wave's 16 rows of the (consumed) q~ tile, so that the
      // stores below write whole 256-byte rows
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int col = 16 * dt + 4 * lq;
        const uint2 sg = *reinterpret_cast<const uint2*>(&Gt[swz(tl, col >> 3) + (col & 7)]);
        uint2 o;
        o.x = pack_bf16x2(acc[dt][0] * bf2f(sg.x & 0xffffu), acc[dt][1] * bf2f(sg.x >> 16));
        o.y = pack_bf16x2(acc[dt][2] * bf2f(sg.y & 0xffffu), acc[dt][3] * bf2f(sg.y >> 16));
        *reinterpret_cast<uint2*>(&Qt[swz(tl, col >> 3) + (col & 7)]) = o;
      }
    } else {
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          uint2 p;
          p.x = pack_bf16x2(acc[8 * it + jt][0], acc[8 * it + jt][1]);
          p.y = pack_bf16x2(acc[8 * it + jt][2], acc[8 * it + jt][3]);
          const int dk0 = 32 * w4 + 16 * it + 4 * lq, dv = 16 * jt + l16;
          *reinterpret_cast<uint2*>(&L.st[swz(dv, dk0 >> 3) + (dk0 & 7)]) = p;
        }
    }
    // the next chunk's tiles must have landed before the barrier; the output stores are issued
    // after this wait so that they never hold it up
    wait_vmcnt<0>();
    if (out_wave) {
      // a wave's LDS accesses complete in order, so its staged rows are read back as written
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = 16 * w4 + 4 * r + lq, tr = c0 + rl;  // lane: row rl, 16-byte chunk l16
        const uint4 o = *reinterpret_cast<const uint4*>(&Qt[swz(rl, l16)]);
        if (tr < t_end) *reinterpret_cast<uint4*>(out + head_off + (long)tr * tok_stride + 8 * l16) = o;
      }
    }
    __syncthreads();
    buf ^= 1;
  }
  if (!out_wave && seg == nseg - 1 && state_out && h % G == 0) {
    float* dst = state_out + bh * D * D;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dk = 32 * w4 + 16 * it + 4 * lq + e, dv = 16 * jt + l16;
          dst[dk * D + dv] = acc[8 * it + jt][e];
        }
  }
}

// dst = src, or 0 where src is null (n floats): the state of an empty sequence. A kernel, not
// a runtime copy or fill, so that the call stays capturable in a graph as plain kernel nodes.
__global__ void __launch_bounds__(256)
copy_or_zero_kernel(const float* __restrict__ src, float* __restrict__ dst, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    dst[i] = src ? src[i] : 0.0f;
}

// Slot s >= 1 holds segment s-1's own sum on entry; on exit slot s holds the state entering
// segment s: state_in + sum of the sums of segments 0..s-1. One thread per state element.
template <class Geo>
__global__ void __launch_bounds__(256)
linear_scan_kernel(const float* __restrict__ state_in, float* __restrict__ ws, int H, int dd, Geo geo) {
  const int bh = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  int nslots;
  const long slot = geo.scan_item(bh, H, &nslots);
  if (e >= dd || nslots < 1) return;
  float acc = state_in ? state_in[(long)bh * dd + e] : 0.f;
  float* p = ws + slot * dd + e;
  p[0] = acc;
  for (int s = 1; s < nslots; ++s) {
    acc += p[(long)s * dd];
    p[(long)s * dd] = acc;
  }
}

// ------------------------------------------------------------------ fp32 path (plain scan)

// q~ for every (b, t, h) and k~ for every (b, t, kv head): RMS norm, weight, RoPE (angle reduced
// in fp64, accurate fp32 sin/cos). One wave per (b, t, h) query row, which also handles the key
// row (b, t, h) when h < Hkv; lane i < d/2 owns dims i and i + d/2.
__global__ void __launch_bounds__(64)
linear_prep_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                       const float* __restrict__ qw, const float* __restrict__ kw,
                       float* __restrict__ qt, float* __restrict__ kt, int N, int H, int Hkv, int d,
                       long pos0, float eps, RopeFreqs freqs) {
  const long row = blockIdx.x;  // (b*N + t)*H + h
  const int h = (int)(row % H);
  const long bt = row / H;
  const int t = (int)(bt % N);
  const bool has_k = h < Hkv;
  const long krow = bt * Hkv + h;
  const int i = threadIdx.x;
  const int half = d / 2;
  const bool on = i < half;
  float a[2] = {0.f, 0.f}, b[2] = {0.f, 0.f};
  if (on) {
    a[0] = q[row * d + i]; a[1] = q[row * d + i + half];
    if (has_k) { b[0] = k[krow * d + i]; b[1] = k[krow * d + i + half]; }
  }
  const float sq = group_sum<64>(a[0] * a[0] + a[1] * a[1]);
  const float sk = group_sum<64>(b[0] * b[0] + b[1] * b[1]);
  if (!on) return;
  const float iq = 1.0f / sqrtf(sq / d + eps), ik = 1.0f / sqrtf(sk / d + eps);
  float x0 = a[0] * iq, x1 = a[1] * iq, y0 = b[0] * ik, y1 = b[1] * ik;
  if (qw) { x0 *= qw[i]; x1 *= qw[i + half]; }
  if (kw) { y0 *= kw[i]; y1 *= kw[i + half]; }
  const double rev = (double)(pos0 + t) * freqs.f[i];
  const float ang = (float)((rev - rint(rev)) * 6.283185307179586);
  float sn, cs;
  sincosf(ang, &sn, &cs);
  qt[row * d + i] = x0 * cs - x1 * sn;
  qt[row * d + i + half] = x0 * sn + x1 * cs;
  if (has_k) {
    kt[krow * d + i] = y0 * cs - y1 * sn;
    kt[krow * d + i + half] = y0 * sn + y1 * cs;
  }
}

// One workgroup of d threads per (b, KV head); thread c owns state column c (all d rows), so
// the readout o[c] = sum_i q~[i] S[i][c] needs no cross-thread reduction. Tokens in order; each
// token updates the state once and reads it out for every query head of the group.
template <int DD>
__global__ void __launch_bounds__(DD)
linear_scan_f32_kernel(const float* __restrict__ qt, const float* __restrict__ kt,
                       const float* __restrict__ v, const float* __restrict__ g,
                       const float* __restrict__ state_in, float* __restrict__ state_out,
                       float* __restrict__ out, int N, int H, int Hkv) {
  constexpr int QR = 64;  // query rows staged per step (TB tokens x G heads)
  __shared__ float sq[QR][DD], sk[QR][DD];
  const int bkv = blockIdx.x, b = bkv / Hkv, kvh = bkv % Hkv;
  const int G = H / Hkv, TB = G >= QR ? 1 : QR / G;
  const int c = threadIdx.x;
  float S[DD];
#pragma unroll
  for (int r = 0; r < DD; ++r) S[r] = state_in ? state_in[((long)bkv * DD + r) * DD + c] : 0.f;
  for (int t0 = 0; t0 < N; t0 += TB) {
    const int nt = min(TB, N - t0);
    __syncthreads();
    for (int u = 0; u < nt; ++u) {
      const long bt = (long)b * N + t0 + u;
      sk[u][c] = kt[(bt * Hkv + kvh) * DD + c];
      for (int hg = 0; hg < G; ++hg) sq[u * G + hg][c] = qt[(bt * H + kvh * G + hg) * DD + c];
    }
    __syncthreads();
    for (int u = 0; u < nt; ++u) {
      const long bt = (long)b * N + t0 + u;
      const float vc = v[(bt * Hkv + kvh) * DD + c];
#pragma unroll
      for (int r = 0; r < DD; ++r) S[r] += sk[u][r] * vc;
      for (int hg = 0; hg < G; ++hg) {
        const long row = bt * H + kvh * G + hg;
        float o = 0.f;
#pragma unroll
        for (int r = 0; r < DD; ++r) o += sq[u * G + hg][r] * S[r];
        out[row * DD + c] = o / (1.0f + expf(-g[row * DD + c]));
      }
    }
  }
  if (state_out) {
#pragma unroll
    for (int r = 0; r < DD; ++r) state_out[((long)bkv * DD + r) * DD + c] = S[r];
  }
}

// ------------------------------------------------------------------ decode step

// Decode step, grid (B*Hkv, DD/64), 320 threads: one KV head's 64-column slice of S. Wave 0
// normalises and rotates k and the group's queries (their loads are not queued behind the
// state's); waves 1-4 stream the slice, update it in place once, and keep per-row partials of
// o = q^ S for each query head of the group in turn, which wave 0 sums, gates and stores.
constexpr int DEC_GMAX = 64;  // query heads per KV head
template <typename T, int DD>
__global__ void __launch_bounds__(320)
linear_decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                     const T* __restrict__ g, const float* __restrict__ qw,
                     const float* __restrict__ kw, float* __restrict__ state, T* __restrict__ out,
                     long pos, const int64_t* __restrict__ pos_b, int H, int Hkv, float eps, RopeFreqs freqs) {
  constexpr int NR = DD / 16;  // rows per state thread
  constexpr int HALF = DD / 2;
  __shared__ float sq[DEC_GMAX][DD], sk[DD];
  __shared__ float4 red[16][16];
  const int bkv = blockIdx.x, b = bkv / Hkv, kvh = bkv % Hkv, G = H / Hkv;
  const int j = threadIdx.x;
  const long kvec = (long)bkv * DD;                  // k, v of this KV head
  const long qvec = ((long)b * H + kvh * G) * DD;    // the group's first query head
  const int js = j - 64, r0 = js >> 4, c4 = js & 15;
  const int col = 64 * blockIdx.y + 4 * c4;
  float* Sp = state + (long)bkv * DD * DD + col;
  float4 sv[NR];
  float vc[4];
  if (j < 64) {
    // ---- wave 0: k^ and the group's q^ = RoPE(RMSNorm(.) * w) into LDS. Every load of the
    // wave is issued before the first use, so that their latencies overlap: k, the frequency
    // and the first QPRE query heads unconditionally (lanes past the rotation pairs and heads
    // past the group read valid elements that are then ignored), the optional position and
    // weights last.
    constexpr int QPRE = 4;
    const bool on = j < HALF;
    const int jj = j & (HALF - 1);
    float b0 = to_f32(k[kvec + jj]), b1 = to_f32(k[kvec + jj + HALF]);
    const double fj = freqs.f[jj];
    float a0[QPRE], a1[QPRE];
#pragma unroll
    for (int u = 0; u < QPRE; ++u) {
      const long qo = qvec + (long)(u < G ? u : G - 1) * DD + jj;
      a0[u] = to_f32(q[qo]);
      a1[u] = to_f32(q[qo + HALF]);
    }
    long pb = pos;
    if (pos_b) pb = pos_b[b];
    float kw0 = 1.f, kw1 = 1.f, qw0 = 1.f, qw1 = 1.f;
    if (kw) { kw0 = kw[jj]; kw1 = kw[jj + HALF]; }
    if (qw) { qw0 = qw[jj]; qw1 = qw[jj + HALF]; }
    if (!on) b0 = b1 = 0.f;
    if (pos_b) pos = pb > 0 ? pb : 0;  // each sequence at its own position (negative values read as 0)
    float cs = 1.f, sn = 0.f;
    if (on) {
      const double rev = (double)pos * fj;
      const float ang = (float)((rev - rint(rev)) * 6.283185307179586);
      sincosf(ang, &sn, &cs);
    }
    const float ssk = group_sum<64>(b0 * b0 + b1 * b1);
    if (on) {
      const float ik = 1.0f / sqrtf(ssk / DD + eps);
      float y0 = b0 * ik, y1 = b1 * ik;
      if (kw) { y0 *= kw0; y1 *= kw1; }
      sk[j] = y0 * cs - y1 * sn; sk[j + HALF] = y0 * sn + y1 * cs;
    }
    auto qhead = [&](float x0, float x1, int hg) {
      const float ssq = group_sum<64>(x0 * x0 + x1 * x1);
      if (on) {
        const float iq = 1.0f / sqrtf(ssq / DD + eps);
        x0 *= iq; x1 *= iq;
        if (qw) { x0 *= qw0; x1 *= qw1; }
        sq[hg][j] = x0 * cs - x1 * sn; sq[hg][j + HALF] = x0 * sn + x1 * cs;
      }
    };
#pragma unroll
    for (int u = 0; u < QPRE; ++u)
      if (u < G) qhead(on ? a0[u] : 0.f, on ? a1[u] : 0.f, u);
    for (int hg = QPRE; hg < G; ++hg) {
      float x0 = 0, x1 = 0;
      if (on) { x0 = to_f32(q[qvec + (long)hg * DD + j]); x1 = to_f32(q[qvec + (long)hg * DD + j + HALF]); }
      qhead(x0, x1, hg);
    }
  } else {
    // ---- waves 1-4: v, then the state slice (rows r0 + 16m, columns 64y + 4c4 .. +3), loaded
    // while wave 0 prepares q^ and k^; each row is used as soon as it has arrived
#pragma unroll
    for (int e = 0; e < 4; ++e) vc[e] = to_f32(v[kvec + col + e]);
#pragma unroll
    for (int m = 0; m < NR; ++m) sv[m] = *reinterpret_cast<const float4*>(Sp + (long)(r0 + 16 * m) * DD);
  }
  __syncthreads();  // q^, k^ ready
  if (j >= 64) {
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int r = r0 + 16 * m;
      const float kr = sk[r];
      float4 s4 = sv[m];
      s4.x += kr * vc[0]; s4.y += kr * vc[1]; s4.z += kr * vc[2]; s4.w += kr * vc[3];
      *reinterpret_cast<float4*>(Sp + (long)r * DD) = s4;
      sv[m] = s4;
    }
  }
  for (int hg = 0; hg < G; ++hg) {
    if (j >= 64) {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        const float qr = sq[hg][r0 + 16 * m];
        o.x += qr * sv[m].x; o.y += qr * sv[m].y; o.z += qr * sv[m].z; o.w += qr * sv[m].w;
      }
      red[r0][c4] = o;
    }
    __syncthreads();  // partials ready
    if (j < 64) {
      // ---- o[c] = sum of the 16 row-group partials, gated
      const int cc = j >> 2, e = j & 3;  // column 64y + 4cc + e
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float4 t = red[m][cc];
        acc += e == 0 ? t.x : e == 1 ? t.y : e == 2 ? t.z : t.w;
      }
      const long oc = qvec + (long)hg * DD + 64 * blockIdx.y + j;
      const float gv = to_f32(g[oc]);
      out[oc] = from_f32<T>(acc / (1.0f + expf(-gv)));
    }
    if (hg + 1 < G) __syncthreads();  // the partials are rewritten for the next head
  }
}

// The bf16 prefill over a geometry: segment sums (when some sequence has several segments),
// their scan, then the output pass. GS is the segment-sum geometry, GO the output/scan one.
template <class GS, class GO>
hipError_t run_linear_bf16(const GS& gs, const GO& go, long n_ss, long n_out, long n_bh, bool scan, int H, int Hkv,
                           int seg,
                           const void* q, const void* k, const void* v, const void* g, const float* qw,
                           const float* kw, const float* state_in, float* state_out, void* out, void* ws, float eps,
                           const RopeFreqs& fr, hipStream_t st) {
  float* wsf = static_cast<float*>(ws);
  const bf16_t *qb = (const bf16_t*)q, *kb = (const bf16_t*)k, *vb = (const bf16_t*)v, *gb = (const bf16_t*)g;
  static const hipError_t attr_ok = [] {
    const hipError_t e[4] = {
        hipFuncSetAttribute((const void*)linear_segsum_kernel<false, GS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(SegLds)),
        hipFuncSetAttribute((const void*)linear_segsum_kernel<true, GS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(SegLds)),
        hipFuncSetAttribute((const void*)linear_out_kernel<false, GO>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(OutLds)),
        hipFuncSetAttribute((const void*)linear_out_kernel<true, GO>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(OutLds))};
    for (hipError_t x : e)
      if (x != hipSuccess) return x;
    return hipSuccess;
  }();
  if (attr_ok != hipSuccess) return attr_ok;
  if (scan) {
    if (n_ss > 0) {
      if (kw)
        hipLaunchKernelGGL((linear_segsum_kernel<true, GS>), dim3((unsigned)n_ss), dim3(SS_NT), sizeof(SegLds), st, kb,
                           vb, kw, wsf, Hkv, seg, eps, fr, gs);
      else
        hipLaunchKernelGGL((linear_segsum_kernel<false, GS>), dim3((unsigned)n_ss), dim3(SS_NT), sizeof(SegLds), st, kb,
                           vb, kw, wsf, Hkv, seg, eps, fr, gs);
    }
    hipLaunchKernelGGL((linear_scan_kernel<GO>), dim3((unsigned)n_bh, D * D / 256), dim3(256), 0, st, state_in, wsf,
                       Hkv, D * D, go);
  }
  if (qw || kw)
    hipLaunchKernelGGL((linear_out_kernel<true, GO>), dim3((unsigned)n_out), dim3(OUT_NT), sizeof(OutLds), st, qb, kb,
                       vb, gb, qw, kw, state_in, wsf, state_out, (bf16_t*)out, H, Hkv, seg, eps, fr, go);
  else
    hipLaunchKernelGGL((linear_out_kernel<false, GO>), dim3((unsigned)n_out), dim3(OUT_NT), sizeof(OutLds), st, qb, kb,
                       vb, gb, qw, kw, state_in, wsf, state_out, (bf16_t*)out, H, Hkv, seg, eps, fr, go);
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ launchers

size_t linear_prefill_workspace(const sala_linear_desc& d) {
  if (d.dtype == SALA_F32) return 2ull * d.batch * d.seq_len * d.n_heads * d.head_dim * sizeof(float);
  const int seg = linear_segment_len(d);
  const long nseg = (d.seq_len + seg - 1) / seg;
  if (nseg <= 1 && d.n_kv_heads == d.n_heads) return 0;
  return (size_t)d.batch * d.n_kv_heads * nseg * d.head_dim * d.head_dim * sizeof(float);
}

int linear_segment_len(const sala_linear_desc& d, int target_wgs, int max_seg) {
  // segment = B*H*N / target_wgs rounded up to a power of two, in [64, max_seg]. For the
  // forward (512 workgroups, two per CU; segments up to 8,192 tokens), measured on MI355X with
  // 32 heads: at 32,768 tokens 2,048-token segments take 0.49 ms against 0.62 with 512-token
  // ones; at 262,144 tokens 8,192-token segments 3.04 ms against 3.10 with 4,096 and 3.28 with
  // 2,048. A longer segment amortises the segment's state load and the scan over more chunks.
  const long long work = (long long)d.batch * d.n_heads * d.seq_len;
  long long seg = 64;
  while (seg < max_seg && work / seg > target_wgs) seg *= 2;
  return (int)seg;
}

hipError_t launch_linear_prefill(const sala_linear_desc& d, const void* q, const void* k,
                                 const void* v, const void* g, const float* qw, const float* kw,
                                 const float* state_in, float* state_out, void* out, void* ws,
                                 hipStream_t st) {
  const int B = d.batch, N = d.seq_len, H = d.n_heads, Hkv = d.n_kv_heads, hd = d.head_dim;
  if (N == 0) {
    // no tokens: state passes through
    if (state_out && state_out != state_in) {
      const long n = (long)B * Hkv * hd * hd;
      const unsigned nb = (unsigned)std::min<long>((n + 255) / 256, 4096);
      hipLaunchKernelGGL(copy_or_zero_kernel, dim3(nb), dim3(256), 0, st, state_in, state_out, n);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  const RopeFreqs fr = make_rope_freqs(hd, d.rope_base);
  if (d.dtype == SALA_F32) {
    float* qt = static_cast<float*>(ws);
    float* kt = qt + (size_t)B * N * H * hd;
    hipLaunchKernelGGL(linear_prep_f32_kernel, dim3((unsigned)((long)B * N * H)), dim3(64), 0, st,
                       (const float*)q, (const float*)k, qw, kw, qt, kt, N, H, Hkv, hd, (long)d.pos0,
                       d.norm_eps, fr);
    if (hd == 64)
      hipLaunchKernelGGL(linear_scan_f32_kernel<64>, dim3(B * Hkv), dim3(64), 0, st, qt, kt,
                         (const float*)v, (const float*)g, state_in, state_out, (float*)out, N, H, Hkv);
    else
      hipLaunchKernelGGL(linear_scan_f32_kernel<128>, dim3(B * Hkv), dim3(128), 0, st, qt, kt,
                         (const float*)v, (const float*)g, state_in, state_out, (float*)out, N, H, Hkv);
    return hipGetLastError();
  }
  const int seg = linear_segment_len(d);
  const int nseg = (N + seg - 1) / seg;
  const LinUniform geo{N, (long)d.pos0, nseg};
  return run_linear_bf16(geo, geo, (long)B * Hkv * (nseg - 1), (long)B * H * nseg, (long)B * Hkv, nseg > 1 || Hkv < H,
                         H, Hkv, seg, q, k, v, g, qw, kw, state_in, state_out, out, ws, d.norm_eps, fr, st);
}

// segment length of a packed batch: chosen for its total token count, as for one sequence
static int varlen_segment_len(const sala_linear_desc& d) {
  sala_linear_desc one = d;
  one.batch = 1;
  return linear_segment_len(one);
}

size_t linear_prefill_varlen_workspace(const sala_linear_desc& d, const int32_t* cu_seqlens) {
  const int seg = varlen_segment_len(d);
  size_t slots = 0;
  for (int s = 0; s < d.batch; ++s) slots += (cu_seqlens[s + 1] - cu_seqlens[s] + seg - 1) / seg;
  return (size_t)d.n_kv_heads * slots * d.head_dim * d.head_dim * sizeof(float);
}

hipError_t launch_linear_prefill_varlen(const sala_linear_desc& d, const int32_t* cu_seqlens, const int64_t* pos0,
                                        const void* q, const void* k, const void* v, const void* g,
                                        const float* qw, const float* kw, const float* state_in,
                                        float* state_out, void* out, void* ws, hipStream_t st) {
  const int H = d.n_heads, Hkv = d.n_kv_heads, nseq = d.batch;
  const RopeFreqs fr = make_rope_freqs(d.head_dim, d.rope_base);
  const int seg = varlen_segment_len(d);
  LinVarlen ss{make_varlen_table(nseq, cu_seqlens, pos0)};
  bool any_multi = false;
  for (int s = 0; s < nseq; ++s) {
    const int n = ss.t.n[s];
    const int ns = (n + seg - 1) / seg;
    ss.t.aux0[s + 1] = ss.t.aux0[s] + ns;
    any_multi = any_multi || ns > 1;
    // a sequence without tokens: its state passes through
    if (n == 0 && state_out && state_out != state_in) {
      const long off = (long)s * Hkv * D * D;
      hipLaunchKernelGGL(copy_or_zero_kernel, dim3(64), dim3(256), 0, st, state_in ? state_in + off : nullptr,
                         state_out + off, (long)Hkv * D * D);
    }
  }
  LinVarlen ou = ss;
  for (int s = 0; s <= nseq; ++s) {
    ou.t.item0[s] = H * ss.t.aux0[s];
    // segment-sum items: every segment but the last of each sequence with tokens
    int skip = 0;
    for (int x = 0; x < s; ++x) skip += ss.t.n[x] > 0;
    ss.t.item0[s] = Hkv * (ss.t.aux0[s] - skip);
  }
  if (ou.t.item0[nseq] == 0) return hipGetLastError();
  return run_linear_bf16(ss, ou, ss.t.item0[nseq], ou.t.item0[nseq], nseq * Hkv, any_multi || Hkv < H, H, Hkv, seg, q,
                         k, v, g, qw, kw, state_in, state_out, out, ws, d.norm_eps, fr, st);
}

hipError_t launch_linear_decode(const sala_linear_desc& d, const void* q, const void* k,
                                const void* v, const void* g, const float* qw, const float* kw,
                                float* state, void* out, const int64_t* pos_b, hipStream_t st) {
  const int H = d.n_heads, Hkv = d.n_kv_heads, hd = d.head_dim;
  const RopeFreqs fr = make_rope_freqs(hd, d.rope_base);
  const dim3 grid(d.batch * Hkv, hd / 64);
  const long pos = (long)d.pos0;
  const dim3 block(320);
  if (d.dtype == SALA_BF16) {
    if (hd == 128)
      hipLaunchKernelGGL((linear_decode_kernel<bf16_t, 128>), grid, block, 0, st, (const bf16_t*)q,
                         (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)g, qw, kw, state, (bf16_t*)out,
                         pos, pos_b, H, Hkv, d.norm_eps, fr);
    else
      hipLaunchKernelGGL((linear_decode_kernel<bf16_t, 64>), grid, block, 0, st, (const bf16_t*)q,
                         (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)g, qw, kw, state, (bf16_t*)out,
                         pos, pos_b, H, Hkv, d.norm_eps, fr);
  } else {
    if (hd == 128)
      hipLaunchKernelGGL((linear_decode_kernel<float, 128>), grid, block, 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (const float*)g, qw, kw, state, (float*)out,
                         pos, pos_b, H, Hkv, d.norm_eps, fr);
    else
      hipLaunchKernelGGL((linear_decode_kernel<float, 64>), grid, block, 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (const float*)g, qw, kw, state, (float*)out,
                         pos, pos_b, H, Hkv, d.norm_eps, fr);
  }
  return hipGetLastError();
}

}  // namespace sala
