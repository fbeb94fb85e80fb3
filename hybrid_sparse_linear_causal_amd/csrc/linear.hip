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
//   1. linear_chunk_kernel<true>  : per (b, h, segment s < last) the segment's sum of k^T v,
//                                   written to workspace slot s + 1
//   2. linear_scan_kernel         : per (b, h): slot 0 = state_in (or 0), slot s = slot s-1 +
//                                   slot s, i.e. the state entering segment s
//   3. linear_chunk_kernel<false> : per (b, h, segment) the chunk loop from its start state,
//                                   writing gated outputs (and, last segment, the final state)
// With a single segment the workspace is unused and state_in is read directly. Reading the
// entering state from the workspace otherwise lets state_out alias state_in safely.
#include "common.hpp"
#include "launch.hpp"

namespace sala {

namespace {

constexpr int D = 128;        // head dim of the bf16 MFMA path
constexpr int CH = 64;        // chunk length (tokens)
constexpr int NT = 256;       // threads per workgroup (4 waves)
constexpr int QS = D + 8;     // LDS row stride (bf16) of token-major tiles: 272 B
constexpr int TS = CH + 8;    // LDS row stride (bf16) of feature-major tiles: 144 B
constexpr int SS = D + 8;     // LDS row stride (bf16) of the transposed state
constexpr int OS = D + 4;     // LDS row stride (fp32) of the output staging tile

struct LinearLds {
  bf16_t q[CH * QS];    // q~  [token][dk]
  bf16_t k[CH * QS];    // k~  [token][dk]
  bf16_t kt[D * TS];    // k~^T [dk][token]
  bf16_t vt[D * TS];    // v^T  [dv][token]
  bf16_t st[D * SS];    // S^T  [dv][dk] as bf16 (state entering the chunk)
  float o[CH * OS];     // output staging [token][dv]
};

// Raw chunk data held in registers by thread j: tokens 2*(j/8) + {0,1}, 16-byte segments
// s = j%8 and s+8 (dims 8s..8s+7 and 64+8s..64+8s+7, which RoPE pairs with each other).
struct ChunkRegs {
  uint4 q[2][2], k[2][2], v[2][2], g[2][2];
};

__device__ __forceinline__ uint4 ld16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <bool STATE_ONLY>
__device__ __forceinline__ void load_chunk(ChunkRegs& r, const bf16_t* q, const bf16_t* k,
                                           const bf16_t* v, const bf16_t* g, long row0, int t0,
                                           int n_valid, int H) {
  // row0 = element offset of (b, token 0 of the chunk, h, 0); token stride = H * D
  const int j = threadIdx.x;
  const int s = j & 7;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = 2 * (j >> 3) + u;
    const bool ok = (t0 + t) < n_valid;
    const long base = row0 + (long)t * H * D;
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int off = 8 * (s + 8 * hs);
      const uint4 z = make_uint4(0, 0, 0, 0);
      r.k[u][hs] = ok ? ld16(k + base + off) : z;
      r.v[u][hs] = ok ? ld16(v + base + off) : z;
      if (!STATE_ONLY) {
        r.q[u][hs] = ok ? ld16(q + base + off) : z;
        r.g[u][hs] = ok ? ld16(g + base + off) : z;
      }
    }
  }
}

// QK-norm + RoPE of one token's 16 values held by this thread (two 8-dim halves that RoPE
// pairs), given the 8 angles' sin/cos. Row sum of squares is reduced over the 8 lanes of the
// token. Writes the rotated bf16 values into x (as packed uint4).
__device__ __forceinline__ void norm_rope(uint4 (&x)[2], const float* w, int s, float eps,
                                          const float* sn, const float* cs) {
  float a[8], b[8];
  unpack8(x[0], a);
  unpack8(x[1], b);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += a[e] * a[e] + b[e] * b[e];
  ss = group_sum<8>(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
  float ra[8], rb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float xa = a[e] * inv, xb = b[e] * inv;
    if (w) { xa *= w[8 * s + e]; xb *= w[64 + 8 * s + e]; }
    ra[e] = xa * cs[e] - xb * sn[e];
    rb[e] = xa * sn[e] + xb * cs[e];
  }
  x[0] = pack8(ra);
  x[1] = pack8(rb);
}

// write 16 bf16 values of one token (dims 8s..8s+7, 64+8s..) as 2-byte entries of a
// feature-major tile T[dim][token] (pairs of tokens packed into one 32-bit store)
__device__ __forceinline__ void store_T_pair(bf16_t* T, int t_even, int s, const uint4 (&x0)[2],
                                             const uint4 (&x1)[2]) {
  // x0: token t_even, x1: token t_even + 1
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    const uint32_t a[4] = {x0[hs].x, x0[hs].y, x0[hs].z, x0[hs].w};
    const uint32_t b[4] = {x1[hs].x, x1[hs].y, x1[hs].z, x1[hs].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int dim = 8 * (s + 8 * hs) + 2 * w;
      // low halves: dim, high halves: dim + 1
      const uint32_t lo = (a[w] & 0xffffu) | (b[w] << 16);
      const uint32_t hi = (a[w] >> 16) | (b[w] & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(T + dim * TS + t_even) = lo;
      *reinterpret_cast<uint32_t*>(T + (dim + 1) * TS + t_even) = hi;
    }
  }
}

template <bool STATE_ONLY>
__global__ void __launch_bounds__(NT)
linear_chunk_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                    const bf16_t* __restrict__ v, const bf16_t* __restrict__ g,
                    const float* __restrict__ qw, const float* __restrict__ kw,
                    const float* __restrict__ state_in, float* __restrict__ ws,
                    float* __restrict__ state_out, bf16_t* __restrict__ out, int N, int H,
                    long pos0, int seg_len, int nseg, float eps, RopeFreqs freqs) {
  __shared__ __align__(16) LinearLds L;
  const int nseg_w = STATE_ONLY ? nseg - 1 : nseg;
  const int seg = blockIdx.x % nseg_w;
  const int bh = blockIdx.x / nseg_w;
  const int b = bh / H, h = bh % H;
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int s8 = j & 7, tp = j >> 3;

  const int t_begin = seg * seg_len;
  const int t_end = min(N, t_begin + seg_len);
  const long head_off = ((long)b * N * H + h) * D;  // element offset of (b, t=0, h, 0)
  const long tok_stride = (long)H * D;

  // ---- state entering the segment: S[dk][dv] in MFMA C layout; wave owns dk rows 32w..32w+31
  f32x4 S[2][8];
  {
    const float* src = nullptr;
    if (!STATE_ONLY) {
      if (nseg == 1) src = state_in ? state_in + (long)bh * D * D : nullptr;
      else src = ws + ((long)bh * nseg + seg) * D * D;
    }
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dk = 32 * wave + 16 * it + 4 * lq + e, dv = 16 * jt + l16;
          S[it][jt][e] = src ? src[dk * D + dv] : 0.f;
        }
  }
  if (!STATE_ONLY) {
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) {
        const int dk0 = 32 * wave + 16 * it + 4 * lq, dv = 16 * jt + l16;
        uint2 p;
        p.x = pack_bf16x2(S[it][jt][0], S[it][jt][1]);
        p.y = pack_bf16x2(S[it][jt][2], S[it][jt][3]);
        *reinterpret_cast<uint2*>(&L.st[dv * SS + dk0]) = p;
      }
  }

  // frequencies (revolutions per position) of this thread's 8 RoPE pairs
  double fr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) fr[e] = freqs.f[8 * s8 + e];

  ChunkRegs cur;
  load_chunk<STATE_ONLY>(cur, q, k, v, g, head_off + (long)t_begin * tok_stride, t_begin, N, H);

  for (int c0 = t_begin; c0 < t_end; c0 += CH) {
    // ---------------- prep: QK-norm + RoPE, stage tiles in LDS
    {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * tp + u;
        const double p = (double)(pos0 + c0 + t);
        float sn[8], cs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sincos_rev(rope_rev(p, fr[e]), &sn[e], &cs[e]);
        norm_rope(cur.k[u], kw, s8, eps, sn, cs);
        if (!STATE_ONLY) {
          norm_rope(cur.q[u], qw, s8, eps, sn, cs);
          *reinterpret_cast<uint4*>(&L.q[t * QS + 8 * s8]) = cur.q[u][0];
          *reinterpret_cast<uint4*>(&L.q[t * QS + 64 + 8 * s8]) = cur.q[u][1];
          *reinterpret_cast<uint4*>(&L.k[t * QS + 8 * s8]) = cur.k[u][0];
          *reinterpret_cast<uint4*>(&L.k[t * QS + 64 + 8 * s8]) = cur.k[u][1];
        }
      }
      store_T_pair(L.kt, 2 * tp, s8, cur.k[0], cur.k[1]);
      store_T_pair(L.vt, 2 * tp, s8, cur.v[0], cur.v[1]);
    }
    uint4 gk[2][2];
    if (!STATE_ONLY) {
#pragma unroll
      for (int u = 0; u < 2; ++u) { gk[u][0] = cur.g[u][0]; gk[u][1] = cur.g[u][1]; }
    }
    __syncthreads();
    // prefetch the next chunk while this one is computed
    if (c0 + CH < t_end)
      load_chunk<STATE_ONLY>(cur, q, k, v, g, head_off + (long)(c0 + CH) * tok_stride, c0 + CH, N, H);

    if (!STATE_ONLY) {
      // ---------------- intra-chunk: A^T = K~ Q~^T for this wave's 16 queries (16w..16w+15)
      f32x4 OT[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) OT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 qfrag[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qfrag[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(&L.q[(16 * wave + l16) * QS + 32 * ks + 8 * lq]));
      // key tiles kt <= wave; pairs (2c, 2c+1) feed one PV k-step of 32 keys
      for (int c = 0; 2 * c <= wave; ++c) {
        f32x4 at[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kt = 2 * c + hh;
          at[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (kt <= wave) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4*>(&L.k[(16 * kt + l16) * QS + 32 * ks + 8 * lq]));
              at[hh] = mfma16x16x32(kf, qfrag[ks], at[hh]);
            }
            if (kt == wave) {
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
        for (int dt = 0; dt < 8; ++dt) {
          const bf16_t* vrow = &L.vt[(16 * dt + l16) * TS + 32 * c + 4 * lq];
          const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint2*>(vrow),
                                      *reinterpret_cast<const uint2*>(vrow + 16));
          OT[dt] = mfma16x16x32(vf, pfrag, OT[dt]);
        }
      }
      // ---------------- inter-chunk: O^T += S^T Q~^T
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 sf = as_bf16x8(*reinterpret_cast<const uint4*>(&L.st[(16 * dt + l16) * SS + 32 * ks + 8 * lq]));
          OT[dt] = mfma16x16x32(sf, qfrag[ks], OT[dt]);
        }
      // stage O (fp32) for the coalesced gated store
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<float4*>(&L.o[(16 * wave + l16) * OS + 16 * dt + 4 * lq]) =
            make_float4(OT[dt][0], OT[dt][1], OT[dt][2], OT[dt][3]);
    }

    // ---------------- state update: S += K~^T V (wave: dk rows 32w..32w+31, all dv)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[2];
#pragma unroll
      for (int it = 0; it < 2; ++it)
        af[it] = as_bf16x8(*reinterpret_cast<const uint4*>(&L.kt[(32 * wave + 16 * it + l16) * TS + 32 * ks + 8 * lq]));
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) {
        const bf16x8 bfr = as_bf16x8(*reinterpret_cast<const uint4*>(&L.vt[(16 * jt + l16) * TS + 32 * ks + 8 * lq]));
#pragma unroll
        for (int it = 0; it < 2; ++it) S[it][jt] = mfma16x16x32(af[it], bfr, S[it][jt]);
      }
    }
    __syncthreads();

    if (!STATE_ONLY) {
      // new S^T (bf16) for the next chunk
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          const int dk0 = 32 * wave + 16 * it + 4 * lq, dv = 16 * jt + l16;
          uint2 p;
          p.x = pack_bf16x2(S[it][jt][0], S[it][jt][1]);
          p.y = pack_bf16x2(S[it][jt][2], S[it][jt][3]);
          *reinterpret_cast<uint2*>(&L.st[dv * SS + dk0]) = p;
        }
      // gated output: out = O * sigmoid(g)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * tp + u;
        if (c0 + t < t_end) {
          bf16_t* dst = out + head_off + (long)(c0 + t) * tok_stride;
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const int d0 = 8 * (s8 + 8 * hs);
            float gv[8], ov[8];
            unpack8(gk[u][hs], gv);
            const float4 o0 = *reinterpret_cast<const float4*>(&L.o[t * OS + d0]);
            const float4 o1 = *reinterpret_cast<const float4*>(&L.o[t * OS + d0 + 4]);
            ov[0] = o0.x; ov[1] = o0.y; ov[2] = o0.z; ov[3] = o0.w;
            ov[4] = o1.x; ov[5] = o1.y; ov[6] = o1.z; ov[7] = o1.w;
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[e] *= sigmoidf_(gv[e]);
            *reinterpret_cast<uint4*>(dst + d0) = pack8(ov);
          }
        }
      }
    }
  }

  // ---- segment result: state-only -> segment sum into its slot; last segment -> final state
  float* dst = nullptr;
  if (STATE_ONLY) dst = ws + ((long)bh * nseg + seg + 1) * D * D;
  else if (seg == nseg - 1 && state_out) dst = state_out + (long)bh * D * D;
  if (dst) {
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dk = 32 * wave + 16 * it + 4 * lq + e, dv = 16 * jt + l16;
          dst[dk * D + dv] = S[it][jt][e];
        }
  }
}

// Slot s >= 1 holds segment s-1's own sum on entry; on exit slot s holds the state entering
// segment s: state_in + sum of the sums of segments 0..s-1. One thread per state element.
__global__ void __launch_bounds__(256)
linear_scan_kernel(const float* __restrict__ state_in, float* __restrict__ ws, int nslots, int dd) {
  const int bh = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e >= dd) return;
  float acc = state_in ? state_in[(long)bh * dd + e] : 0.f;
  float* p = ws + (long)bh * nslots * dd + e;
  p[0] = acc;
  for (int s = 1; s < nslots; ++s) {
    acc += p[(long)s * dd];
    p[(long)s * dd] = acc;
  }
}

// ------------------------------------------------------------------ fp32 path (plain scan)

// q~ and k~ for every (b, t, h): RMS norm, weight, RoPE (angle reduced in fp64, accurate
// fp32 sin/cos). One wave per row; lane i < d/2 owns dims i and i + d/2.
__global__ void __launch_bounds__(64)
linear_prep_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                       const float* __restrict__ qw, const float* __restrict__ kw,
                       float* __restrict__ qt, float* __restrict__ kt, int N, int H, int d,
                       long pos0, float eps, RopeFreqs freqs) {
  const long row = blockIdx.x;  // (b*N + t)*H + h
  const int t = (int)((row / H) % N);
  const int i = threadIdx.x;
  const int half = d / 2;
  const bool on = i < half;
  float a[2] = {0.f, 0.f}, b[2] = {0.f, 0.f};
  if (on) {
    a[0] = q[row * d + i]; a[1] = q[row * d + i + half];
    b[0] = k[row * d + i]; b[1] = k[row * d + i + half];
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
  kt[row * d + i] = y0 * cs - y1 * sn;
  kt[row * d + i + half] = y0 * sn + y1 * cs;
}

// One workgroup of d threads per (b, h); thread c owns state column c (all d rows), so the
// readout o[c] = sum_i q~[i] S[i][c] needs no cross-thread reduction. Tokens in order.
template <int DD>
__global__ void __launch_bounds__(DD)
linear_scan_f32_kernel(const float* __restrict__ qt, const float* __restrict__ kt,
                       const float* __restrict__ v, const float* __restrict__ g,
                       const float* __restrict__ state_in, float* __restrict__ state_out,
                       float* __restrict__ out, int N, int H) {
  constexpr int TB = 32;  // tokens staged per step
  __shared__ float sq[TB][DD], sk[TB][DD];
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int c = threadIdx.x;
  float S[DD];
#pragma unroll
  for (int r = 0; r < DD; ++r) S[r] = state_in ? state_in[((long)bh * DD + r) * DD + c] : 0.f;
  for (int t0 = 0; t0 < N; t0 += TB) {
    const int nt = min(TB, N - t0);
    __syncthreads();
    for (int u = 0; u < nt; ++u) {
      const long row = ((long)b * N + t0 + u) * H + h;
      sq[u][c] = qt[row * DD + c];
      sk[u][c] = kt[row * DD + c];
    }
    __syncthreads();
    for (int u = 0; u < nt; ++u) {
      const long row = ((long)b * N + t0 + u) * H + h;
      const float vc = v[row * DD + c];
      float o = 0.f;
#pragma unroll
      for (int r = 0; r < DD; ++r) {
        S[r] += sk[u][r] * vc;
        o += sq[u][r] * S[r];
      }
      out[row * DD + c] = o / (1.0f + expf(-g[row * DD + c]));
    }
  }
  if (state_out) {
#pragma unroll
    for (int r = 0; r < DD; ++r) state_out[((long)bh * DD + r) * DD + c] = S[r];
  }
}

// ------------------------------------------------------------------ decode step

// grid (B*H, d/32): each workgroup owns 32 state columns of one (b, h). Thread j: column
// 32*blockIdx.y + j%32, rows j/32 + 8m. q~, k~ (norm + RoPE at pos) computed by wave 0.
template <typename T, int DD>
__global__ void __launch_bounds__(256)
linear_decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                     const T* __restrict__ g, const float* __restrict__ qw,
                     const float* __restrict__ kw, float* __restrict__ state, T* __restrict__ out,
                     long pos, float eps, RopeFreqs freqs) {
  __shared__ float sq[DD], sk[DD];
  __shared__ float red[8][32];
  const int bh = blockIdx.x;
  const int j = threadIdx.x;
  const long vec = (long)bh * DD;
  if (j < 64) {
    constexpr int HALF = DD / 2;
    const bool on = j < HALF;
    float a0 = 0, a1 = 0, b0 = 0, b1 = 0;
    if (on) {
      a0 = to_f32(q[vec + j]); a1 = to_f32(q[vec + j + HALF]);
      b0 = to_f32(k[vec + j]); b1 = to_f32(k[vec + j + HALF]);
    }
    const float ssq = group_sum<64>(a0 * a0 + a1 * a1);
    const float ssk = group_sum<64>(b0 * b0 + b1 * b1);
    if (on) {
      const float iq = 1.0f / sqrtf(ssq / DD + eps), ik = 1.0f / sqrtf(ssk / DD + eps);
      float x0 = a0 * iq, x1 = a1 * iq, y0 = b0 * ik, y1 = b1 * ik;
      if (qw) { x0 *= qw[j]; x1 *= qw[j + HALF]; }
      if (kw) { y0 *= kw[j]; y1 *= kw[j + HALF]; }
      const double rev = (double)pos * freqs.f[j];
      const float ang = (float)((rev - rint(rev)) * 6.283185307179586);
      float sn, cs;
      sincosf(ang, &sn, &cs);
      sq[j] = x0 * cs - x1 * sn; sq[j + HALF] = x0 * sn + x1 * cs;
      sk[j] = y0 * cs - y1 * sn; sk[j + HALF] = y0 * sn + y1 * cs;
    }
  }
  __syncthreads();
  const int col = 32 * blockIdx.y + (j & 31);
  const int r0 = j >> 5;
  const float vc = to_f32(v[vec + col]);
  float* Sp = state + (long)bh * DD * DD + col;
  float o = 0.f;
#pragma unroll
  for (int m = 0; m < DD / 8; ++m) {
    const int r = r0 + 8 * m;
    const float s = Sp[(long)r * DD] + sk[r] * vc;
    Sp[(long)r * DD] = s;
    o += sq[r] * s;
  }
  red[r0][j & 31] = o;
  __syncthreads();
  if (j < 32) {
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) acc += red[m][j];
    const float gv = to_f32(g[vec + col]);
    out[vec + col] = from_f32<T>(acc / (1.0f + expf(-gv)));
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

size_t linear_prefill_workspace(const sala_linear_desc& d) {
  if (d.dtype == SALA_F32) return 2ull * d.batch * d.seq_len * d.n_heads * d.head_dim * sizeof(float);
  const int seg = linear_segment_len(d);
  const long nseg = (d.seq_len + seg - 1) / seg;
  if (nseg <= 1) return 0;
  return (size_t)d.batch * d.n_heads * nseg * d.head_dim * d.head_dim * sizeof(float);
}

int linear_segment_len(const sala_linear_desc& d) {
  // aim for ~2048 workgroups: segment = B*H*N / 2048 rounded up to a power of two, in [64, 4096]
  const long long work = (long long)d.batch * d.n_heads * d.seq_len;
  long long seg = 64;
  while (seg < 4096 && work / seg > 2048) seg *= 2;
  return (int)seg;
}

hipError_t launch_linear_prefill(const sala_linear_desc& d, const void* q, const void* k,
                                 const void* v, const void* g, const float* qw, const float* kw,
                                 const float* state_in, float* state_out, void* out, void* ws,
                                 hipStream_t st) {
  const int B = d.batch, N = d.seq_len, H = d.n_heads, hd = d.head_dim;
  if (N == 0) {
    // no tokens: state passes through
    if (state_out && state_out != state_in) {
      if (state_in)
        return hipMemcpyAsync(state_out, state_in, sizeof(float) * B * H * hd * hd, hipMemcpyDeviceToDevice, st);
      return hipMemsetAsync(state_out, 0, sizeof(float) * B * H * hd * hd, st);
    }
    return hipSuccess;
  }
  const RopeFreqs fr = make_rope_freqs(hd, d.rope_base);
  if (d.dtype == SALA_F32) {
    float* qt = static_cast<float*>(ws);
    float* kt = qt + (size_t)B * N * H * hd;
    hipLaunchKernelGGL(linear_prep_f32_kernel, dim3((unsigned)((long)B * N * H)), dim3(64), 0, st,
                       (const float*)q, (const float*)k, qw, kw, qt, kt, N, H, hd, (long)d.pos0,
                       d.norm_eps, fr);
    if (hd == 64)
      hipLaunchKernelGGL(linear_scan_f32_kernel<64>, dim3(B * H), dim3(64), 0, st, qt, kt,
                         (const float*)v, (const float*)g, state_in, state_out, (float*)out, N, H);
    else
      hipLaunchKernelGGL(linear_scan_f32_kernel<128>, dim3(B * H), dim3(128), 0, st, qt, kt,
                         (const float*)v, (const float*)g, state_in, state_out, (float*)out, N, H);
    return hipGetLastError();
  }
  const int seg = linear_segment_len(d);
  const int nseg = (N + seg - 1) / seg;
  float* wsf = static_cast<float*>(ws);
  const bf16_t *qb = (const bf16_t*)q, *kb = (const bf16_t*)k, *vb = (const bf16_t*)v, *gb = (const bf16_t*)g;
  if (nseg > 1) {
    hipLaunchKernelGGL(linear_chunk_kernel<true>, dim3(B * H * (nseg - 1)), dim3(NT), 0, st, qb, kb,
                       vb, gb, qw, kw, state_in, wsf, state_out, (bf16_t*)out, N, H, (long)d.pos0,
                       seg, nseg, d.norm_eps, fr);
    hipLaunchKernelGGL(linear_scan_kernel, dim3(B * H, D * D / 256), dim3(256), 0, st, state_in,
                       wsf, nseg, D * D);
  }
  hipLaunchKernelGGL(linear_chunk_kernel<false>, dim3(B * H * nseg), dim3(NT), 0, st, qb, kb, vb,
                     gb, qw, kw, state_in, wsf, state_out, (bf16_t*)out, N, H, (long)d.pos0, seg,
                     nseg, d.norm_eps, fr);
  return hipGetLastError();
}

hipError_t launch_linear_decode(const sala_linear_desc& d, const void* q, const void* k,
                                const void* v, const void* g, const float* qw, const float* kw,
                                float* state, void* out, hipStream_t st) {
  const int BH = d.batch * d.n_heads, hd = d.head_dim;
  const RopeFreqs fr = make_rope_freqs(hd, d.rope_base);
  const dim3 grid(BH, hd / 32);
  const long pos = (long)d.pos0;
  if (d.dtype == SALA_BF16) {
    if (hd == 128)
      hipLaunchKernelGGL((linear_decode_kernel<bf16_t, 128>), grid, dim3(256), 0, st, (const bf16_t*)q,
                         (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)g, qw, kw, state, (bf16_t*)out,
                         pos, d.norm_eps, fr);
    else
      hipLaunchKernelGGL((linear_decode_kernel<bf16_t, 64>), grid, dim3(256), 0, st, (const bf16_t*)q,
                         (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)g, qw, kw, state, (bf16_t*)out,
                         pos, d.norm_eps, fr);
  } else {
    if (hd == 128)
      hipLaunchKernelGGL((linear_decode_kernel<float, 128>), grid, dim3(256), 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (const float*)g, qw, kw, state, (float*)out,
                         pos, d.norm_eps, fr);
    else
      hipLaunchKernelGGL((linear_decode_kernel<float, 64>), grid, dim3(256), 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (const float*)g, qw, kw, state, (float*)out,
                         pos, d.norm_eps, fr);
  }
  return hipGetLastError();
}

}  // namespace sala
