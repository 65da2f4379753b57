// Large-token kernels for gfx950: the video-action chunk (256 rows over a
// 4096-token cache, width 2048, 16 heads of 128) and the DiT-style step
// (4128 tokens, width 3072, 24 heads of 128, adaLN-Zero).  With hundreds to
// thousands of rows every projection is MFMA-bound, so the GEMM reuses each
// weight tile over 64-128 rows and each staged activation tile over four
// waves; attention is a flash-style pass over 64-key blocks held in LDS.
//
// Layouts: activations bf16 [rows][cols] row-major, rows padded to 64 (the
// padded rows are zero and never stored back); residual stream f32; weights
// in the tiled arena shared with the other paths (16 output columns x 32
// reduction rows per 1 KiB tile, lane l holding 8 reduction rows of column
// l % 16: the A operand of v_mfma_f32_16x16x32_bf16).
#include "phx_tokens.h"

#include <hip/hip_runtime.h>
#include <math.h>

namespace phx {
namespace tok {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// by-value bit casts (an element of an ext_vector value must not be cast in place)
__device__ inline float as_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ inline unsigned as_u(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ inline unsigned short bits(bf16 b) { return __builtin_bit_cast(unsigned short, b); }
__device__ inline unsigned pack2(float a, float b) {
  return (unsigned)bits((bf16)a) | ((unsigned)bits((bf16)b) << 16);
}
__device__ inline float gelu_tanh(float z) {
  const float k = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(k * (z + 0.044715f * z * z * z)));
}

__device__ inline f32x4 mma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mma16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ GEMM
// Workgroup of 4 waves covering output columns [64 NTW bx, +64 NTW) and rows
// [16 MTW by, +16 MTW).  Wave w owns n-tiles 4 NTW bx + NTW w + [0, NTW) and
// all MTW m-tiles.  Per 32-row k-step the workgroup stages its activation
// rows in LDS once, in fragment order (m-tile, lane), and every wave reads
// its weight tiles straight from the arena.
template <int NTW, int MTW, int EPI>
__global__ __launch_bounds__(256) void k_tgemm(GemmT g) {
  constexpr int BM = 16 * MTW;
  __shared__ u32x4 as[MTW * 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nt0 = (blockIdx.x * 4 + wave) * NTW;
  const int m0 = blockIdx.y * BM;
  const int KT = g.K / 32;
  const bf16* A = (const bf16*)g.a;
  const bf16* W = (const bf16*)g.w;
  f32x4 acc[NTW][MTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n)
#pragma unroll
    for (int m = 0; m < MTW; ++m) acc[n][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < KT; ++kt) {
    // stage: thread t moves rows p*64 + t/4 (k chunk t%4) of the block
#pragma unroll
    for (int p = 0; p < (BM + 63) / 64; ++p) {
      const int r = p * 64 + (t >> 2);
      if (r < BM) {
        const u32x4 v = *(const u32x4*)(A + (size_t)(m0 + r) * g.K + kt * 32 + 8 * (t & 3));
        as[(r >> 4) * 64 + (r & 15) + 16 * (t & 3)] = v;
      }
    }
    bf16x8 wf[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n)
      wf[n] = __builtin_bit_cast(bf16x8, *(const u32x4*)(W + (((size_t)(nt0 + n) * KT + kt) * 64 + lane) * 8));
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, as[m * 64 + lane]);
#pragma unroll
      for (int n = 0; n < NTW; ++n) acc[n][m] = mma32(wf[n], af, acc[n][m]);
    }
    __syncthreads();
  }
  // epilogue: lane holds columns 4 (lane / 16) + [0, 4) of each n-tile (tile
  // order) for row lane % 16 of each m-tile
  const int gq = lane >> 4;
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    const int row = m0 + 16 * m + (lane & 15);
    if (row >= g.M) continue;
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      const int nt = nt0 + n;
      const f32x4 v = acc[n][m];
      if constexpr (EPI == EP_BF16 || EPI == EP_GELU) {
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = EPI == EP_GELU ? gelu_tanh(v[i]) : v[i];
        *(u32x2*)((bf16*)g.out + (size_t)row * g.ldo + nt * 16 + 4 * gq) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
      } else if constexpr (EPI == EP_ROPE) {
        // tile order of a head: pairs (j, j + 64), j = 8 (nt % 8) + 2 gq + (i & 1)
        const int hh = nt >> 3, j = 8 * (nt & 7) + 2 * gq;
        const int c0 = hh * DH + j;
        float y0 = v[0], y1 = v[1], y2 = v[2], y3 = v[3];
        if (c0 < g.rot_cols) {
          const float2 a = g.rope[(size_t)row * (DH / 2) + j];
          const float2 b = g.rope[(size_t)row * (DH / 2) + j + 1];
          y0 = v[0] * a.x - v[2] * a.y;
          y2 = v[2] * a.x + v[0] * a.y;
          y1 = v[1] * b.x - v[3] * b.y;
          y3 = v[3] * b.x + v[1] * b.y;
        }
        bf16* o = (bf16*)g.out + (size_t)row * g.ldo;
        *(unsigned*)(o + c0) = pack2(y0, y1);
        *(unsigned*)(o + c0 + DH / 2) = pack2(y2, y3);
      } else if constexpr (EPI == EP_GEGLU) {
        // features 8 nt + 2 gq + {0, 1}: gate in v[0], v[1], up in v[2], v[3]
        const int f = 8 * nt + 2 * gq;
        *(unsigned*)((bf16*)g.out + (size_t)row * g.ldo + f) = pack2(gelu_tanh(v[0]) * v[2], gelu_tanh(v[1]) * v[3]);
      } else {
        float* o = (float*)g.out + (size_t)row * g.ldo + nt * 16 + 4 * gq;
        f32x4 cur = EPI == EP_F32 ? f32x4{0.f, 0.f, 0.f, 0.f} : *(const f32x4*)o;
        if constexpr (EPI == EP_RESID) {
          if (g.gate) {
            const f32x4 gt = *(const f32x4*)(g.gate + nt * 16 + 4 * gq);
            cur += gt * v;
          } else {
            cur += v;
          }
        } else if constexpr (EPI == EP_EULER) {
          cur += g.dt * v;
        } else {
          cur = v;
        }
        *(f32x4*)o = cur;
      }
    }
  }
}

template <int EPI>
hipError_t launch_tgemm_e(const GemmT& g, hipStream_t s) {
  // the larger block when it still gives the chip >= 256 workgroups
  const long long big = (long long)(g.N / 128) * (g.Mp / 128);
  if (g.Mp % 128 == 0 && g.N % 128 == 0 && big >= 256) {
    hipLaunchKernelGGL((k_tgemm<2, 8, EPI>), dim3(g.N / 128, g.Mp / 128), dim3(256), 0, s, g);
  } else {
    hipLaunchKernelGGL((k_tgemm<1, 4, EPI>), dim3(g.N / 64, g.Mp / 64), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_tgemm(int epi, const GemmT& g, hipStream_t s) {
  if (g.K % 32 || g.N % 64 || g.Mp % ROW_PAD || g.M > g.Mp) return hipErrorInvalidValue;
  switch (epi) {
    case EP_BF16: return launch_tgemm_e<EP_BF16>(g, s);
    case EP_ROPE: return launch_tgemm_e<EP_ROPE>(g, s);
    case EP_GEGLU: return launch_tgemm_e<EP_GEGLU>(g, s);
    case EP_GELU: return launch_tgemm_e<EP_GELU>(g, s);
    case EP_RESID: return launch_tgemm_e<EP_RESID>(g, s);
    case EP_EULER: return launch_tgemm_e<EP_EULER>(g, s);
    case EP_F32: return launch_tgemm_e<EP_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------ row norms

// one workgroup per row; D <= 256 * 16
__global__ __launch_bounds__(256) void k_tnorm(int kind, const float* __restrict__ h, const float* __restrict__ scale,
                                               const float* __restrict__ shift, float eps, bf16* __restrict__ out,
                                               int M, int D) {
  constexpr int PER = 16;
  __shared__ float red[8];
  const int row = blockIdx.x, t = threadIdx.x;
  bf16* o = out + (size_t)row * D;
  if (row >= M) {
    for (int d = t; d < D; d += 256) o[d] = (bf16)0.0f;
    return;
  }
  const float* x = h + (size_t)row * D;
  float v[PER];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = t + 256 * i;
    v[i] = d < D ? x[d] : 0.f;
    s += v[i];
  }
  auto block_sum = [&](float a) -> float {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off);
    __syncthreads();
    if ((t & 63) == 0) red[t >> 6] = a;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
  };
  float mean = 0.f;
  if (kind == 1) mean = block_sum(s) / (float)D;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = t + 256 * i;
    const float c = d < D ? v[i] - mean : 0.f;
    ss += c * c;
  }
  const float inv = 1.0f / sqrtf(block_sum(ss) / (float)D + eps);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = t + 256 * i;
    if (d < D) o[d] = (bf16)((v[i] - mean) * inv * (1.0f + scale[d]) + shift[d]);
  }
}

hipError_t launch_tnorm(int kind, const float* h, const float* scale, const float* shift, float eps, void* out, int M,
                        int Mp, int D, hipStream_t s) {
  if (D > 256 * 16 || M > Mp) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tnorm, dim3(Mp), dim3(256), 0, s, kind, h, scale, shift, eps, (bf16*)out, M, D);
  return hipGetLastError();
}

__global__ void k_tcvt(const float* __restrict__ x, bf16* __restrict__ out, int M, int Mp, int D) {
  const size_t total = (size_t)Mp * D;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x)
    out[i] = (bf16)((int)(i / D) < M ? x[i] : 0.0f);
}

hipError_t launch_tcvt(const float* x, void* out, int M, int Mp, int D, hipStream_t s) {
  const size_t total = (size_t)Mp * D;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_tcvt, dim3(blocks), dim3(256), 0, s, x, (bf16*)out, M, Mp, D);
  return hipGetLastError();
}

// ------------------------------------------------------------- attention
// Workgroup (64 queries, head h, key split s); wave w owns queries 16 w.
// Keys are the L prefix rows followed by the M chunk rows; the split takes a
// contiguous range of 64-key blocks.  Per block:
//   S^T = K . Q^T with 16x16x16 MFMAs: the K block sits in LDS as A fragments
//     (lane: key lane % 16, dims 4 (lane / 16) + [0, 4) of a 16-dim step) and
//     the wave's queries as B fragments in registers, so each lane ends with
//     keys 4 (lane / 16) + [0, 4) of one query (lane % 16);
//   online softmax per query (the four lanes of a query combine with two
//     shuffles);
//   O^T += V^T . P^T: V^T sits in LDS as A fragments (lane: dim lane % 16,
//     keys 4 (lane / 16) + [0, 4)), and P^T is exactly the S^T register
//     layout, so the probabilities feed the next MFMA without a shuffle.
constexpr int KB = 64;  // keys per block

__device__ inline const bf16* key_row(const AttnT& a, int L, int t, bool value) {
  const int kvd = a.KVH * DH;
  if (t < L) return (const bf16*)(value ? a.vp : a.kp) + (size_t)t * kvd;
  return (const bf16*)a.qkv + (size_t)(t - L) * a.ldqkv + (a.H + (value ? a.KVH : 0)) * DH;
}

__global__ __launch_bounds__(256) void k_tattn(AttnT a) {
  __shared__ u32x2 kf[4 * 8 * 64];  // [key tile][dim step][lane] 4 bf16
  __shared__ u32x2 vf[8 * 4 * 64];  // [dim tile][key tile][lane] 4 bf16
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int h = blockIdx.y, split = blockIdx.z;
  const int kvh = h / (a.H / a.KVH);
  const int q0 = blockIdx.x * 64 + 16 * wave;
  const int L = a.lens ? a.lens[0] : 0;
  const int T = L + a.M;
  const int nblk = (T + KB - 1) / KB;
  const int per = (nblk + a.splits - 1) / a.splits;
  const int b0 = split * per, b1 = min(nblk, b0 + per);
  const int gq = lane >> 4, qr = lane & 15;
  // this wave's queries as B fragments of Q^T: dims 16 ds + 4 gq + [0, 4) of query q0 + qr
  s16x4 qf[8];
  {
    const int q = min(q0 + qr, a.M - 1);
    const bf16* qp = (const bf16*)a.qkv + (size_t)q * a.ldqkv + h * DH;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) qf[ds] = __builtin_bit_cast(s16x4, *(const u32x2*)(qp + 16 * ds + 4 * gq));
  }
  f32x4 oacc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  for (int b = b0; b < b1; ++b) {
    const int k0 = b * KB;
    // stage K (A fragments) and V^T (A fragments): thread t moves 8 dims (16 bytes) of key t / 16 ... for
    // four passes of 16 keys
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int kl = p * 16 + (t >> 4);  // key within the block
      const int dc = (t & 15) * 8;       // first of 8 dims
      const int key = k0 + kl;
      u32x4 kv = u32x4{0u, 0u, 0u, 0u}, vv = u32x4{0u, 0u, 0u, 0u};
      if (key < T) {
        kv = *(const u32x4*)(key_row(a, L, key, false) + kvh * DH + dc);
        vv = *(const u32x4*)(key_row(a, L, key, true) + kvh * DH + dc);
      }
      // K fragment: key tile kl/16, dim step dc/16, lane (kl % 16) + 16 * ((dc % 16) / 4)
      const int kt = kl >> 4, ds = dc >> 4, lk = (kl & 15) + 16 * ((dc & 15) >> 2);
      kf[(kt * 8 + ds) * 64 + lk] = u32x2{kv[0], kv[1]};
      kf[(kt * 8 + ds) * 64 + lk + 16] = u32x2{kv[2], kv[3]};
      // V^T fragment: dim tile d/16, key tile kl/16, lane (d % 16) + 16 * ((kl % 16) / 4), element kl % 4
      unsigned short* vs = (unsigned short*)vf;
      const unsigned vw[4] = {vv[0], vv[1], vv[2], vv[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dc + e;
        const int li = (d & 15) + 16 * ((kl & 15) >> 2);
        vs[(((d >> 4) * 4 + kt) * 64 + li) * 4 + (kl & 3)] = (unsigned short)(vw[e >> 1] >> (16 * (e & 1)));
      }
    }
    __syncthreads();
    // scores
    f32x4 st[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 8; ++ds)
        st[kt] = mma16(__builtin_bit_cast(s16x4, kf[(kt * 8 + ds) * 64 + lane]), qf[ds], st[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * kt + 4 * gq + i;
        const float sv = key < T ? st[kt][i] * a.scale : -INFINITY;
        st[kt][i] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float corr = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
    float ls = 0.f;
    s16x4 pf[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = st[kt][i] == -INFINITY ? 0.f : expf(st[kt][i] - m_new);
        ls += p;
        pf[kt][i] = (short)bits((bf16)p);
      }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run = l_run * corr + ls;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      f32x4 acc = oacc[d] * corr;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) acc = mma16(__builtin_bit_cast(s16x4, vf[(d * 4 + kt) * 64 + lane]), pf[kt], acc);
      oacc[d] = acc;
    }
  }
  // lane holds dims 16 d + 4 gq + [0, 4) of query q0 + qr
  const int q = q0 + qr;
  if (q >= a.M) return;
  if (a.splits == 1) {
    const float inv = 1.0f / l_run;
    bf16* op = (bf16*)a.o + (size_t)q * (a.H * DH) + h * DH;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *(u32x2*)(op + 16 * d + 4 * gq) =
          u32x2{pack2(oacc[d][0] * inv, oacc[d][1] * inv), pack2(oacc[d][2] * inv, oacc[d][3] * inv)};
  } else {
    float* po = a.po + ((size_t)split * a.M + q) * (a.H * DH) + h * DH;
#pragma unroll
    for (int d = 0; d < 8; ++d) *(f32x4*)(po + 16 * d + 4 * gq) = oacc[d];
    if (gq == 0) {
      float* ml = a.pml + (((size_t)split * a.M + q) * a.H + h) * 2;
      ml[0] = m_run;
      ml[1] = l_run;
    }
  }
}

hipError_t launch_tattn(const AttnT& a, hipStream_t s) {
  if (a.M < 1 || a.H % a.KVH || a.splits < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tattn, dim3((a.M + 63) / 64, a.H, a.splits), dim3(256), 0, s, a);
  return hipGetLastError();
}

// out[q][h*DH + d] = sum_s e^(m_s - m) O_s / sum_s e^(m_s - m) l_s, splits in order
__global__ void k_tcombine(AttnT a) {
  const size_t total = (size_t)a.M * a.H * DH;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int d = (int)(i % DH);
    const size_t qh = i / DH;
    const int h = (int)(qh % a.H);
    const int q = (int)(qh / a.H);
    float m = -INFINITY;
    for (int s = 0; s < a.splits; ++s) m = fmaxf(m, a.pml[(((size_t)s * a.M + q) * a.H + h) * 2]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float ms = a.pml[(((size_t)s * a.M + q) * a.H + h) * 2];
      if (ms == -INFINITY) continue;
      const float w = expf(ms - m);
      num += w * a.po[((size_t)s * a.M + q) * (a.H * DH) + h * DH + d];
      den += w * a.pml[(((size_t)s * a.M + q) * a.H + h) * 2 + 1];
    }
    ((bf16*)a.o)[(size_t)q * (a.H * DH) + h * DH + d] = (bf16)(num / den);
  }
}

hipError_t launch_tcombine(const AttnT& a, hipStream_t s) {
  const size_t total = (size_t)a.M * a.H * DH;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_tcombine, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tok
}  // namespace phx
