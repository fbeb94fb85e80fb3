// Backward pass of the linear-attention layer for gfx950: bf16 inputs, fp32 gradients.
//
// Pages: "MiniCPM-SALA：融合稀疏与线性注意力实现高效长上下文建模" §1, §2.1 (the layer: QK-norm,
// RoPE, an O(N) recurrence with a constant-size state, output gate) and "面壁智能发布MiniCPM-SALA：
// 稀疏-线性混合架构，9B模型端侧跑通百万上下文，速度飙升3.5倍", section "高效训练范式：以25%的成本完成
// 转换" (the linear layers are trained first; later stages train every parameter).
//
// Forward, per head: q~ = RoPE(RMSNorm(q) w_q), k~ = RoPE(RMSNorm(k) w_k), S_t = S_in +
// sum_{s<=t} k~_s^T v_s, o_t = q~_t S_t, out_t = o_t sigmoid(g_t). With dO = dout sigmoid(g)
// and dS_N the gradient of the final state, each gradient of the recurrence is itself a plain
// causal linear attention, two of them running backwards in time:
//   dq~_t = sum_{s<=t} (dO_t . v_s) k~_s + dO_t S_in^T          (forward in time)
//   dk~_s = sum_{t>=s} (v_s . dO_t) q~_t + v_s dS_N^T            (backward in time)
//   dv_s  = sum_{t>=s} (k~_s . q~_t) dO_t + k~_s dS_N            (backward in time)
//   dS_in = dS_N + sum_t q~_t^T dO_t                             (that pass's final state)
// and dg needs o, the forward recurrence without the gate. One chunked MFMA kernel family,
//   Y_u = sum_{w<=u} (A_u . B_w) C_w + A_u S0  over token order u (the sequence or its reverse),
// computes all four. The o pass writes dg = dout o sigmoid'(g) directly; the dq~ pass's states
// are the transposes of the o pass's, and the dk~ pass's of the dv pass's, so two of the four
// segment-sum passes are shared. Elementwise kernels before (norm, RoPE, gate) and after
// (their transposes, the norm-weight sums) complete the chain. Workspace: q~, k~, dO in bf16
// (the forward also feeds q~ and k~ to MFMA in bf16), segment states and the norm-weight
// partial sums.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace sala {

namespace {

constexpr int D = 128;  // head dim
constexpr int CH = 64;  // chunk length (tokens)

// ---- elementwise: 8 lanes per (token, head) row, lane s holding dims 8s..8s+7 and their RoPE
// partners 64+8s..64+8s+7 (so the rotation stays inside the thread). 32 rows per block.
constexpr int EW_NT = 256;
constexpr int EW_ROWS = EW_NT / 8;

__device__ __forceinline__ void load16(const bf16_t* p, int s8, float (&x)[16]) {
  unpack8(*reinterpret_cast<const uint4*>(p + 8 * s8), x);
  unpack8(*reinterpret_cast<const uint4*>(p + 64 + 8 * s8), x + 8);
}
__device__ __forceinline__ void store16(bf16_t* p, int s8, const float (&x)[16]) {
  *reinterpret_cast<uint4*>(p + 8 * s8) = pack8(x);
  *reinterpret_cast<uint4*>(p + 64 + 8 * s8) = pack8(x + 8);
}
// cos and sin of this thread's 8 RoPE angles at position pos (fp64 reduction, as the forward)
__device__ __forceinline__ void rope_cs(long pos, int s8, const RopeFreqs& fr, float (&c)[8], float (&s)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) sincos_rev(rope_rev((double)pos, fr.f[8 * s8 + e]), &s[e], &c[e]);
}
// y = RoPE(x / rms(x) * w): the forward's q~ / k~ in fp32, plus n = x / rms and 1 / rms
__device__ __forceinline__ void norm_rope_fwd(const float (&x)[16], const float* w, int s8, float eps,
                                              const float (&c)[8], const float (&s)[8], float (&n)[16],
                                              float (&y)[16], float& inv) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) ss = fmaf(x[e], x[e], ss);
  ss = group_sum8_dpp(ss);
  inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    n[e] = x[e] * inv;
    n[8 + e] = x[8 + e] * inv;
    const float a = n[e] * (w ? w[8 * s8 + e] : 1.0f), b = n[8 + e] * (w ? w[64 + 8 * s8 + e] : 1.0f);
    y[e] = a * c[e] - b * s[e];
    y[8 + e] = a * s[e] + b * c[e];
  }
}

// q~, k~ (bf16) and dO = dout * sigmoid(g) (bf16) for every row
__global__ void __launch_bounds__(EW_NT)
lbwd_prep_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ g,
                 const bf16_t* __restrict__ dout, const float* __restrict__ qw, const float* __restrict__ kw,
                 bf16_t* __restrict__ qh, bf16_t* __restrict__ kh, bf16_t* __restrict__ dO, long nrows, int N,
                 int H, long pos0, float eps, RopeFreqs fr) {
  const int s8 = threadIdx.x & 7;
  for (long r0 = (long)blockIdx.x * EW_ROWS; r0 < nrows; r0 += (long)gridDim.x * EW_ROWS) {
    const long rr = r0 + (long)(threadIdx.x >> 3);
    const long row = rr < nrows ? rr : nrows - 1;  // all 8 lanes of a row agree
    const bool ok = r0 + (long)(threadIdx.x >> 3) < nrows;
    const long pos = pos0 + (row / H) % N;
    const long base = row * D;
    float c[8], s[8], x[16], n[16], y[16], inv;
    rope_cs(pos, s8, fr, c, s);
    load16(q + base, s8, x);
    norm_rope_fwd(x, qw, s8, eps, c, s, n, y, inv);
    if (ok) store16(qh + base, s8, y);
    load16(k + base, s8, x);
    norm_rope_fwd(x, kw, s8, eps, c, s, n, y, inv);
    if (ok) store16(kh + base, s8, y);
    float gv[16];
    load16(g + base, s8, gv);
    load16(dout + base, s8, x);
#pragma unroll
    for (int e = 0; e < 16; ++e) y[e] = x[e] * fast_sigmoid(gv[e]);
    if (ok) store16(dO + base, s8, y);
  }
}

// dst = src, or 0 where src is null (n floats)
__global__ void __launch_bounds__(256)
lbwd_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) dst[i] = src ? src[i] : 0.0f;
}

// ---- plain chunked causal linear attention: Y_u = sum_{w<=u} (A_u . B_w) C_w + A_u S0, token
// order u = t (REV false) or u = N-1-t (REV true). Same structure as the forward layer's
// segment-sum / scan / chunk passes, without the norm, RoPE and gate, with fp32 output.
constexpr int PL_NT = 512;
constexpr int PL_DMA = 6;  // copy instructions per wave per chunk (3 tiles x 2 pieces)

__device__ __forceinline__ long tok_of(bool rev, long u, int N) { return rev ? (long)N - 1 - u : u; }

// DMA of one chunk's tiles (64 rows x 256 B each, swizzled rows as swzv): wave w moves pieces
// 2w, 2w+1 (rows 8w .. 8w+7) of each tile. Rows past the end are clamped to the last token in
// order u (valid memory; the chunk kernel zeroes their B rows). A whole chunk is addressed by a
// scalar base (its lowest token) plus a fixed 32-bit byte offset per lane (saddr form of the
// copy), so no vector address arithmetic is repeated per chunk; a partial chunk takes the
// per-lane clamped addresses.
// global -> LDS copy of 16 bytes per lane from a scalar base plus a 32-bit lane byte offset
// (saddr form of global_load_lds_dwordx4); lds_addr wave-uniform
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

template <int NT>
__device__ __forceinline__ void dma_tiles(const bf16_t* const (&src)[NT], long head_off, long tok_stride, long u0,
                                          int N, bool rev, bf16_t (*T)[CH * D]) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (u0 + CH <= N) {
    const long tok0 = rev ? (long)N - u0 - CH : u0;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int I = 2 * wave + m;
      const int row = 4 * I + (lane >> 4);
      const int ch = (lane & 15) ^ (2 * (row & 7));
      const uint32_t off = 2u * (uint32_t)((rev ? CH - 1 - row : row) * tok_stride + 8 * ch);
#pragma unroll
      for (int x = 0; x < NT; ++x)
        dma16s(src[x] + head_off + tok0 * tok_stride, off, (uint32_t)(size_t)(T[x] + I * 512));
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int I = 2 * wave + m;
    const int row = 4 * I + (lane >> 4);
    const int ch = (lane & 15) ^ (2 * (row & 7));
    const long t = tok_of(rev, u0 + row < N ? u0 + row : (long)N - 1, N);
    const long off = head_off + t * tok_stride + 8 * ch;
#pragma unroll
    for (int x = 0; x < NT; ++x) dma16(src[x] + off, lds_addr_u32(T[x] + I * 512));
  }
}

struct PlainSegLds {
  bf16_t t[2][2][CH * D];  // [stage][B, C]
};
struct PlainLds {
  bf16_t t[2][3][CH * D];  // [buffer][A, B, C]
  bf16_t st[D * D];        // S^T [dv][dk] bf16: the state entering the chunk
  float nw[D];             // NORM passes: the norm weight (1 where none)
  double nf[D / 2];        // NORM passes: the RoPE frequencies (revolutions per position)
  float wacc[4][D];        // NORM passes: per output wave, the norm-weight gradient sums
};

// per (b, h, segment s < last): sum over the segment of B^T C into workspace slot s + 1
template <bool REV>
__global__ void __launch_bounds__(PL_NT)
lplain_segsum_kernel(const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ C, float* __restrict__ ws, int N,
                     int H, int seg_len, int nseg) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  PlainSegLds& L = *reinterpret_cast<PlainSegLds*>(lds_raw);
  const int nsw = nseg - 1;
  const int seg = blockIdx.x % nsw, bh = blockIdx.x / nsw;
  const int b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, lq = lane >> 4;
  const long head_off = ((long)b * N * H + h) * D, tok_stride = (long)H * D;
  const long u_begin = (long)seg * seg_len;
  const int nch = seg_len / CH;
  const bf16_t* src[2] = {Bm, C};
  dma_tiles(src, head_off, tok_stride, u_begin, N, REV, L.t[0]);
  f32x4 S[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) S[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) {
    wait_vmcnt<0>();
    __syncthreads();  // chunk c landed everywhere; every wave is done with chunk c-1's stage
    if (c + 1 < nch) dma_tiles(src, head_off, tok_stride, u_begin + (long)(c + 1) * CH, N, REV, L.t[(c + 1) & 1]);
    const bf16_t* Bt = L.t[c & 1][0];
    const bf16_t* Ct = L.t[c & 1][1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 af = tr_frag_v(Bt, 32 * ks + 4 * lq, 16, 16 * wave, l16);
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) S[jt] = mfma16x16x32(af, tr_frag_v(Ct, 32 * ks + 4 * lq, 16, 16 * jt, l16), S[jt]);
    }
  }
  float* dst = ws + ((long)bh * nseg + seg + 1) * D * D;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt)
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(16 * wave + 4 * lq + e) * D + 16 * jt + l16] = S[jt][e];
}

// slot 0 = S0 (or 0); slot s = slot s-1 + slot s: the state entering segment s
__global__ void __launch_bounds__(256)
lplain_scan_kernel(const float* __restrict__ S0, float* __restrict__ ws, int nslots) {
  const long bh = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  float acc = S0 ? S0[bh * D * D + e] : 0.f;
  float* p = ws + bh * nslots * D * D + e;
  p[0] = acc;
  for (int s = 1; s < nslots; ++s) {
    acc += p[(long)s * D * D];
    p[(long)s * D * D] = acc;
  }
}

// per (b, h, segment): the chunk loop from the segment's entering state. Waves 0-3 produce the
// outputs of query tiles 0-3, waves 4-7 carry S (dk rows 32(w-4) .. +31) and publish S^T.
// TRANS: the entering states (S0 and the segment slots) are stored transposed, i.e. this pass's
// state is the transpose of another pass's (the slots are then that pass's). GATE: instead of
// Y, the output is dg = dout * Y * sigmoid'(g) (Y is the layer's pre-gate output). NORM: Y is
// dx~ of x = q or k (raw rows xr, norm weight xw); the output is dx, through the transposes of
// RoPE and RMSNorm, and the workgroup's sums of n * (RoPE^T dx~) over its rows (the norm-weight
// gradient) go to wpart[blockIdx.x][wsel][D].
template <bool REV, bool TRANS, bool GATE, bool NORM>
__global__ void __launch_bounds__(PL_NT)
lplain_chunk_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ C,
                    const float* __restrict__ S0, const float* __restrict__ ws, float* __restrict__ S_final,
                    float* __restrict__ Y, const bf16_t* __restrict__ gate, const bf16_t* __restrict__ dout, int N,
                    int H, int seg_len, int nseg, const bf16_t* __restrict__ xr, const float* __restrict__ xw,
                    float eps, long pos0, RopeFreqs fr, float* __restrict__ wpart, int wsel) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  PlainLds& L = *reinterpret_cast<PlainLds*>(lds_raw);
  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int b = bh / H, h = bh % H;
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6, l16 = lane & 15, lq = lane >> 4;
  const bool out_wave = wave < 4;
  const int w4 = wave & 3;
  const long u_begin = (long)seg * seg_len;
  const long u_end = u_begin + seg_len < N ? u_begin + seg_len : (long)N;
  const long head_off = ((long)b * N * H + h) * D, tok_stride = (long)H * D;
  const bf16_t* src[3] = {A, Bm, C};
  dma_tiles(src, head_off, tok_stride, u_begin, N, REV, L.t[0]);
  if (NORM) {
    // published by the barrier before the chunk loop
    for (int x = j; x < D; x += PL_NT) L.nw[x] = xw ? xw[x] : 1.0f;
    for (int x = j; x < D / 2; x += PL_NT) L.nf[x] = fr.f[x];
    for (int x = j; x < 4 * D; x += PL_NT) (&L.wacc[0][0])[x] = 0.f;
  }

  f32x4 acc[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (!out_wave) {
    const float* s0 = (nseg == 1) ? (S0 ? S0 + (long)bh * D * D : nullptr) : ws + ((long)bh * nseg + seg) * D * D;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[8 * it + jt][e] = !s0 ? 0.f
                                : TRANS ? s0[(16 * jt + l16) * D + 32 * w4 + 16 * it + 4 * lq + e]
                                        : s0[(32 * w4 + 16 * it + 4 * lq + e) * D + 16 * jt + l16];
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
  wait_vmcnt<0>();
  __syncthreads();
  int buf = 0;
  for (long u0 = u_begin; u0 < u_end; u0 += CH) {
    const bf16_t* At = L.t[buf][0];
    bf16_t* Bt = L.t[buf][1];
    const bf16_t* Ct = L.t[buf][2];
    // gate and output gradient of this lane's query (used after the chunk's final wait)
    uint2 gv[8], dov[8];
    if (GATE && out_wave) {
      const long u = u0 + 16 * w4 + l16;
      const long off = head_off + tok_of(REV, u < u_end ? u : u_end - 1, N) * tok_stride + 4 * lq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        gv[dt] = *reinterpret_cast<const uint2*>(gate + off + 16 * dt);
        dov[dt] = *reinterpret_cast<const uint2*>(dout + off + 16 * dt);
      }
    }
    uint2 xv8[8];  // NORM: this lane's raw x (dims 16dt + 4lq .. +3), used after the final wait
    if (NORM && out_wave) {
      const long u = u0 + 16 * w4 + l16;
      const long off = head_off + tok_of(REV, u < u_end ? u : u_end - 1, N) * tok_stride + 4 * lq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) xv8[dt] = *reinterpret_cast<const uint2*>(xr + off + 16 * dt);
    }
    if (u0 + CH < u_end) dma_tiles(src, head_off, tok_stride, u0 + CH, N, REV, L.t[buf ^ 1]);
    const int nvalid = u_end - u0 < CH ? (int)(u_end - u0) : CH;
    if (nvalid < CH) {
      // rows past the end: B = 0, so they add nothing to the scores or the state
      for (int x = j; x < (CH - nvalid) * 16; x += PL_NT)
        *reinterpret_cast<uint4*>(&Bt[(nvalid + x / 16) * 128 + 8 * (x % 16)]) = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
    if (out_wave) {
      // intra-chunk: Y^T = C^T (B A^T (.) causal) for queries 16w .. 16w+15
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 afrag[4];
      const int tl = 16 * w4 + l16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) afrag[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(&At[swzv(tl, 4 * ks + lq)]));
      for (int c = 0; 2 * c <= w4; ++c) {
        f32x4 at[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kt = 2 * c + hh;
          at[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (kt <= w4) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const bf16x8 bfr = as_bf16x8(*reinterpret_cast<const uint4*>(&Bt[swzv(16 * kt + l16, 4 * ks + lq)]));
              at[hh] = mfma16x16x32(bfr, afrag[ks], at[hh]);
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
          acc[dt] = mfma16x16x32(tr_frag_v(Ct, 32 * c + 4 * lq, 16, 16 * dt, l16), pfrag, acc[dt]);
      }
      // inter-chunk: Y^T += S^T A^T
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 sf = as_bf16x8(*reinterpret_cast<const uint4*>(&L.st[swz(16 * dt + l16, 4 * ks + lq)]));
          acc[dt] = mfma16x16x32(sf, afrag[ks], acc[dt]);
        }
    } else {
      // state: S += B^T C (dk rows 32*w4 .. +31, all dv; token order as in the output pass)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 af[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) af[it] = tr_frag_v(Bt, 32 * ks + 4 * lq, 16, 32 * w4 + 16 * it, l16);
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          const bf16x8 cf = tr_frag_v(Ct, 32 * ks + 4 * lq, 16, 16 * jt, l16);
#pragma unroll
          for (int it = 0; it < 2; ++it) acc[8 * it + jt] = mfma16x16x32(af[it], cf, acc[8 * it + jt]);
        }
      }
    }
    __syncthreads();  // every read of this chunk's tiles and of S^T is done
    if (!out_wave) {
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
    // the next chunk's tiles must have landed before the barrier; outputs go out after the wait
    wait_vmcnt<0>();
    if (NORM && out_wave) {
      // dx from dx~ = acc: u = RoPE^T dx~, dn = u w, dx = (dn - n mean(dn n)) / rms(x), n = x / rms(x);
      // the 4 lanes lq of a row hold its 128 dims; dims i and i + 64 (dt and dt + 4) are RoPE pairs
      const long u = u0 + 16 * w4 + l16;
      const bool ok = u < u_end;
      const long tk = tok_of(REV, ok ? u : u_end - 1, N);
      // x element e of piece dt, unpacked where it is used (fewer live registers)
      auto xe = [&](int dt, int e) -> float {
        const uint32_t w = (e < 2) ? xv8[dt].x : xv8[dt].y;
        return bf2f((e & 1) ? (w >> 16) : (w & 0xffffu));
      };
      float ss = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(xe(dt, e), xe(dt, e), ss);
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
      // acc becomes dn = (RoPE^T dx~) w in place; wv = n (RoPE^T dx~), the row's norm-weight
      // gradient terms (dims 16dt + 4lq + e at 4dt + e; 0 for rows past the end)
      float dot = 0.f, wv[32];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * dt + 4 * lq + e;
          float sn, cs;
          sincos_rev(rope_rev((double)(pos0 + tk), L.nf[i]), &sn, &cs);
          const float ya = acc[dt][e], yb = acc[dt + 4][e];
          const float ua = cs * ya + sn * yb, ub = -sn * ya + cs * yb;  // RoPE^T
          const float na = xe(dt, e) * inv, nb = xe(dt + 4, e) * inv;
          wv[4 * dt + e] = ok ? na * ua : 0.f;
          wv[4 * (dt + 4) + e] = ok ? nb * ub : 0.f;
          acc[dt][e] = ua * L.nw[i];
          acc[dt + 4][e] = ub * L.nw[i + 64];
          dot = fmaf(acc[dt][e], na, fmaf(acc[dt + 4][e], nb, dot));
        }
      dot += __shfl_xor(dot, 16, 64);
      dot += __shfl_xor(dot, 32, 64);
      dot *= 1.0f / D;
      // sum wv over the wave's 16 rows (lanes l16 of each lq) by a transposing butterfly: after
      // the exchanges at distances 8, 4, 2, 1 lane l16 holds the sums of entries 2 l16 and
      // 2 l16 + 1, which it alone adds into the wave's LDS row (same lane every chunk)
      {
        float a16[16], a8[8], a4[4], a2[2];
        const bool h3 = l16 & 8, h2 = l16 & 4, h1 = l16 & 2, h0 = l16 & 1;
#pragma unroll
        for (int k = 0; k < 16; ++k) a16[k] = (h3 ? wv[16 + k] : wv[k]) + __shfl_xor(h3 ? wv[k] : wv[16 + k], 8, 64);
#pragma unroll
        for (int k = 0; k < 8; ++k) a8[k] = (h2 ? a16[8 + k] : a16[k]) + __shfl_xor(h2 ? a16[k] : a16[8 + k], 4, 64);
#pragma unroll
        for (int k = 0; k < 4; ++k) a4[k] = (h1 ? a8[4 + k] : a8[k]) + __shfl_xor(h1 ? a8[k] : a8[4 + k], 2, 64);
#pragma unroll
        for (int k = 0; k < 2; ++k) a2[k] = (h0 ? a4[2 + k] : a4[k]) + __shfl_xor(h0 ? a4[k] : a4[2 + k], 1, 64);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int kk = 2 * l16 + k;  // entry 4dt + e: dim 16dt + 4lq + e
          L.wacc[w4][16 * (kk >> 2) + 4 * lq + (kk & 3)] += a2[k];
        }
      }
      if (ok) {
        float* yp = Y + head_off + tk * tok_stride + 4 * lq;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (acc[dt][e] - xe(dt, e) * inv * dot) * inv;
          *reinterpret_cast<f32x4*>(yp + 16 * dt) = o;
        }
      }
    } else if (out_wave) {
      const long u = u0 + 16 * w4 + l16;  // lane: query u, dims 16dt + 4lq .. +3
      if (u < u_end) {
        float* yp = Y + head_off + tok_of(REV, u, N) * tok_stride + 4 * lq;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          f32x4 y = acc[dt];
          if (GATE) {
            const float gg[4] = {bf2f(gv[dt].x & 0xffffu), bf2f(gv[dt].x >> 16), bf2f(gv[dt].y & 0xffffu),
                                 bf2f(gv[dt].y >> 16)};
            const float dd[4] = {bf2f(dov[dt].x & 0xffffu), bf2f(dov[dt].x >> 16), bf2f(dov[dt].y & 0xffffu),
                                 bf2f(dov[dt].y >> 16)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sg = fast_sigmoid(gg[e]);
              y[e] = dd[e] * y[e] * sg * (1.0f - sg);
            }
          }
          *reinterpret_cast<f32x4*>(yp + 16 * dt) = y;
        }
      }
    }
    __syncthreads();
    buf ^= 1;
  }
  if (NORM) {
    // the workgroup's weight-gradient sums: the four output waves' rows in order (the loop
    // ended with a barrier, after the last LDS accumulation)
    for (int dd = j; dd < D; dd += PL_NT)
      wpart[((long)blockIdx.x * 2 + wsel) * D + dd] = ((L.wacc[0][dd] + L.wacc[1][dd]) + L.wacc[2][dd]) + L.wacc[3][dd];
  }
  if (!out_wave && seg == nseg - 1 && S_final) {
    float* dst = S_final + (long)bh * D * D;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(32 * w4 + 16 * it + 4 * lq + e) * D + 16 * jt + l16] = acc[8 * it + jt][e];
  }
}

// dw_q, dw_k = sums of the per-block partials: one block per output (q dims, then k dims), a
// fixed-order tree reduction
__global__ void __launch_bounds__(256)
lbwd_wsum_kernel(const float* __restrict__ wpart, int nblocks, float* __restrict__ dqw, float* __restrict__ dkw) {
  __shared__ float red[256];
  const int which = blockIdx.x / D, dim = blockIdx.x % D;
  float a = 0.f;
  for (int bk = threadIdx.x; bk < nblocks; bk += 256) a += wpart[((long)bk * 2 + which) * D + dim];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  float* dst = which ? dkw : dqw;
  if (threadIdx.x == 0 && dst) dst[dim] = red[0];
}

constexpr int EW_BLOCKS_MAX = 2048;

struct BwdPlan {
  int seg, nseg, ew_blocks;
  size_t off_qh, off_kh, off_do, off_slots, off_wpart, total;
};

BwdPlan bwd_plan(const sala_linear_desc& d) {
  BwdPlan p;
  const long nrows = (long)d.batch * d.seq_len * d.n_heads;
  const size_t act = (size_t)nrows * D;
  p.seg = linear_segment_len(d);
  p.nseg = (int)((d.seq_len + p.seg - 1) / p.seg);
  p.ew_blocks = (int)std::min<long>((nrows + EW_ROWS - 1) / EW_ROWS, EW_BLOCKS_MAX);
  const size_t bh = (size_t)d.batch * d.n_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += (bytes + 255) & ~size_t(255); return o; };
  p.off_qh = take(act * 2);
  p.off_kh = take(act * 2);
  p.off_do = take(act * 2);
  p.off_slots = take(p.nseg > 1 ? bh * p.nseg * D * D * 4 : 0);
  p.off_wpart = take(bh * p.nseg * 2 * D * 4);  // one partial per chunk-pass workgroup
  p.total = off;
  return p;
}

// one plain pass; with SEGSUM false the segment slots of an earlier pass (whose state this
// pass's is the transpose of) are reused as they are
template <bool REV, bool TRANS, bool GATE, bool NORM>
hipError_t run_plain(const bf16_t* A, const bf16_t* Bm, const bf16_t* C, const float* S0, float* S_final, float* Y,
                     const bf16_t* gate, const bf16_t* dout, float* slots, bool segsum, int B, int N, int H, int seg,
                     int nseg, const bf16_t* xr, const float* xw, float eps, long pos0, const RopeFreqs& fr,
                     float* wpart, int wsel, hipStream_t st) {
  static const hipError_t attr_ok = [] {
    const hipError_t e0 = hipFuncSetAttribute((const void*)lplain_chunk_kernel<REV, TRANS, GATE, NORM>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(PlainLds));
    const hipError_t e1 = hipFuncSetAttribute((const void*)lplain_segsum_kernel<REV>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(PlainSegLds));
    return e0 != hipSuccess ? e0 : e1;
  }();
  if (attr_ok != hipSuccess) return attr_ok;
  if (segsum && nseg > 1) {
    hipLaunchKernelGGL(lplain_segsum_kernel<REV>, dim3(B * H * (nseg - 1)), dim3(PL_NT), sizeof(PlainSegLds), st,
                       Bm, C, slots, N, H, seg, nseg);
    hipLaunchKernelGGL(lplain_scan_kernel, dim3(B * H, D * D / 256), dim3(256), 0, st, S0, slots, nseg);
  }
  hipLaunchKernelGGL((lplain_chunk_kernel<REV, TRANS, GATE, NORM>), dim3(B * H * nseg), dim3(PL_NT), sizeof(PlainLds), st,
                     A, Bm, C, S0, slots, S_final, Y, gate, dout, N, H, seg, nseg, xr, xw, eps, pos0, fr, wpart, wsel);
  return hipGetLastError();
}

}  // namespace

size_t linear_backward_workspace(const sala_linear_desc& d) {
  if (d.seq_len == 0) return 0;
  return bwd_plan(d).total;
}

hipError_t launch_linear_backward(const sala_linear_desc& d, const void* q, const void* k, const void* v,
                                  const void* g, const float* qw, const float* kw, const float* state_in,
                                  const void* dout, const float* dstate_out, float* dq, float* dk, float* dv,
                                  float* dg, float* dqw, float* dkw, float* dstate_in, void* ws, hipStream_t st) {
  const int B = d.batch, N = d.seq_len, H = d.n_heads;
  if (N == 0) {
    // no tokens: the state passes through unchanged, so dS_in = dS_N; no weight gradient
    const long n = (long)B * H * D * D;
    if (dstate_in)
      hipLaunchKernelGGL(lbwd_copy_kernel, dim3((unsigned)std::min<long>((n + 255) / 256, 4096)), dim3(256), 0,
                         st, dstate_out, dstate_in, n);
    if (dqw || dkw) hipLaunchKernelGGL(lbwd_wsum_kernel, dim3(2 * D), dim3(256), 0, st, nullptr, 0, dqw, dkw);
    return hipGetLastError();
  }
  const BwdPlan p = bwd_plan(d);
  char* w = static_cast<char*>(ws);
  bf16_t* qh = reinterpret_cast<bf16_t*>(w + p.off_qh);
  bf16_t* kh = reinterpret_cast<bf16_t*>(w + p.off_kh);
  bf16_t* dO = reinterpret_cast<bf16_t*>(w + p.off_do);
  float* slots = reinterpret_cast<float*>(w + p.off_slots);
  float* wpart = reinterpret_cast<float*>(w + p.off_wpart);
  const long nrows = (long)B * N * H;
  const RopeFreqs fr = make_rope_freqs(D, d.rope_base);
  const bf16_t *qb = (const bf16_t*)q, *kb = (const bf16_t*)k, *vb = (const bf16_t*)v, *gb = (const bf16_t*)g;
  const bf16_t* db = (const bf16_t*)dout;

  hipLaunchKernelGGL(lbwd_prep_kernel, dim3(p.ew_blocks), dim3(EW_NT), 0, st, qb, kb, gb, db, qw, kw, qh, kh, dO, nrows,
                     N, H, (long)d.pos0, d.norm_eps, fr);
  hipError_t e;
  // dg (from o), dq (from dq~, whose state is the o pass's, transposed), dv and dS_in, dk (from
  // dk~, whose state is the dv pass's, transposed); the dq and dk passes apply the transposes of
  // RoPE and RMSNorm to their rows and leave per-workgroup norm-weight partials
  const long p0 = (long)d.pos0;
  const float eps = d.norm_eps;
  if ((e = run_plain<false, false, true, false>(qh, kh, vb, state_in, nullptr, dg, gb, db, slots, true, B, N, H, p.seg,
                                                p.nseg, nullptr, nullptr, eps, p0, fr, nullptr, 0, st)) != hipSuccess)
    return e;
  if ((e = run_plain<false, true, false, true>(dO, vb, kh, state_in, nullptr, dq, nullptr, nullptr, slots, false, B, N,
                                               H, p.seg, p.nseg, qb, qw, eps, p0, fr, wpart, 0, st)) != hipSuccess)
    return e;
  if ((e = run_plain<true, false, false, false>(kh, qh, dO, dstate_out, dstate_in, dv, nullptr, nullptr, slots, true, B,
                                                N, H, p.seg, p.nseg, nullptr, nullptr, eps, p0, fr, nullptr, 0, st)) !=
      hipSuccess)
    return e;
  if ((e = run_plain<true, true, false, true>(vb, dO, qh, dstate_out, nullptr, dk, nullptr, nullptr, slots, false, B, N,
                                              H, p.seg, p.nseg, kb, kw, eps, p0, fr, wpart, 1, st)) != hipSuccess)
    return e;
  if (dqw || dkw)
    hipLaunchKernelGGL(lbwd_wsum_kernel, dim3(2 * D), dim3(256), 0, st, wpart, B * H * p.nseg, dqw, dkw);
  return hipGetLastError();
}

}  // namespace sala
