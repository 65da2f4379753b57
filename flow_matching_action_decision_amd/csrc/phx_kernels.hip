// gfx950 (CDNA4) kernels of the flow-matching action-expert decision.
//
// The hot loop is NL layers x S Euler steps of small-M work (B*M activation
// rows, 10 for one pi0.5-shape request).  At that M every projection streams
// its weights from HBM once per step and does ~10 MACs per weight element, so
// the GEMMs are bound by HBM bandwidth, not by arithmetic.  The design
// follows from that:
//   * weights are re-tiled once at set-up so one wave reads one contiguous
//     1 KiB tile per 16x32 MFMA A operand (weights on the 16-wide side, the
//     activation rows padded to 16 on the B side: the pages' swap-AB idea,
//     "FlashRT-PAI", section 3.2);
//   * MFMA (v_mfma_f32_16x16x32_bf16) is only the inner-product engine;
//   * the "kernels between GEMMs" are folded into GEMM prologues and
//     epilogues ("PhyAI", section 4.2 Kernel fusion; "FlashRT-PAI", section
//     3.2): adaptive RMSNorm in the prologue, residual add + sums of squares,
//     RoPE + cache write, GeGLU and the Euler update in the epilogues;
//   * split-K partial sums are reduced in a fixed order (LDS inside a
//     workgroup, last-arriving workgroup across workgroups), so replays are
//     bit-identical; no floating-point atomics anywhere.
#include "phx_internal.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

namespace phx {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct FragT;
template <>
struct FragT<bf16> {
  using type = bf16x8;
};
template <>
struct FragT<float> {
  using type = f32x8;
};

// ------------------------------------------------------------------ helpers

__device__ inline bf16x8 ld8(const bf16* p) { return __builtin_bit_cast(bf16x8, *(const u32x4*)p); }
__device__ inline f32x8 ld8(const float* p) {
  f32x4 a = *(const f32x4*)p;
  f32x4 b = *(const f32x4*)(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// streamed weights: non-temporal hint (read once per step, never reused soon)
__device__ inline bf16x8 ldw8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)p));
}
__device__ inline f32x8 ldw8(const float* p) {
  f32x4 a = __builtin_nontemporal_load((const f32x4*)p);
  f32x4 b = __builtin_nontemporal_load((const f32x4*)(p + 4));
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename Frag>
__device__ inline Frag zero_frag();
template <>
__device__ inline bf16x8 zero_frag<bf16x8>() {
  bf16 z = (bf16)0.0f;
  return bf16x8{z, z, z, z, z, z, z, z};
}
template <>
__device__ inline f32x8 zero_frag<f32x8>() {
  return f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
}

template <typename T>
__device__ inline typename FragT<T>::type to_frag(const float* v);
template <>
__device__ inline bf16x8 to_frag<bf16>(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)v[j];  // round to nearest even
  return r;
}
template <>
__device__ inline f32x8 to_frag<float>(const float* v) {
  return f32x8{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
}

// D(16x16) += A(16x32) . B(32x16)
__device__ inline void mma(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline void mma(f32x4& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
}

template <typename T>
__device__ inline void st(T* p, float v) {
  *p = (T)v;
}

// agent-coherent (L2-bypassing) scalar accesses for data exchanged between
// workgroups inside one launch
__device__ inline void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float gelu_tanh(float z) {
  const float k = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(k * (z + 0.044715f * z * z * z)));
}

// ------------------------------------------------------------------- GEMM
//
// Y[rows][N] = X[rows][K] . W[K][N] for rows <= 16*MT.  Workgroup b handles
// n-tile b / KSW and the K chunks (b % KSW)*NW + w of its NW waves; every
// wave streams KT/(KSW*NW) consecutive tiles.

// activation fragment of a plain (PRO_X) or float32 (PRO_XF32) activation;
// the normalising prologue forms its fragments in the GEMM loop itself
template <typename T, int PRO>
__device__ inline typename FragT<T>::type load_act(const GemmArgs& a, int row, int k0) {
  using Frag = typename FragT<T>::type;
  static_assert(PRO == PRO_X || PRO == PRO_XF32, "plain activations only");
  if (row >= a.rows) return zero_frag<Frag>();
  if constexpr (PRO == PRO_X) {
    return ld8((const T*)a.X + (size_t)row * a.ldx + k0);
  } else {
    f32x8 v = ld8((const float*)a.X + (size_t)row * a.ldx + k0);
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = v[j];
    return to_frag<T>(t);
  }
}

// 8-bit tier: one lane's 8 int8 codes (a 512-byte tile holds 16 columns x 32
// rows, lane l the 8 rows 8 (l / 16) + [0, 8) of column l % 16) as the bf16 A
// operand.  Every code (at most 127 in magnitude) is exact in bf16: the
// float32 of the integer has no bits below the top 8 of its significand.
__device__ inline u32x2 i8_load(const signed char* p) { return __builtin_nontemporal_load((const u32x2*)p); }
__device__ inline bf16x8 i8_frag(const u32x2& w) {
  unsigned o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned word = w[i >> 1];
    const int sh = 16 * (i & 1);
    const float lo = (float)(int)(signed char)(word >> sh);
    const float hi = (float)(int)(signed char)(word >> (sh + 8));
    o[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  return __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
}

// W8: the weights are int8 codes with per-column scales (the 8-bit tier,
// bf16 activations); the scale multiplies the fp32 sum before the epilogue.
template <typename T, int NW, int MT, int PRO, int EPI, bool W8 = false>
__global__ __launch_bounds__(NW * 64) void k_gemm(GemmArgs a) {
  using Frag = typename FragT<T>::type;
  constexpr int G = MT <= 1 ? 8 : (MT <= 2 ? 4 : (MT <= 4 ? 2 : 1));  // tiles issued together per wave
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rloc = lane & 15;
  const int grp = lane >> 4;
  const int nt = blockIdx.x / a.KSW;
  const int ks = blockIdx.x - nt * a.KSW;
  const int kpc = a.KT / (a.KSW * NW);
  const int kt0 = (ks * NW + w) * kpc;

  // the 8-bit tier's column scales are loaded now and used after the reduction
  f32x4 wsc4 = f32x4{1.f, 1.f, 1.f, 1.f};
  if constexpr (W8) wsc4 = *(const f32x4*)(a.wsc + nt * 16 + grp * 4);
  const T* wbase = (const T*)a.W + ((size_t)nt * a.KT + kt0) * TILE_ELEMS + lane * 8;
  const signed char* qbase = a.Wq + ((size_t)nt * a.KT + kt0) * TILE_ELEMS + lane * 8;
  // one group of weight tiles in flight; the first group goes out before the
  // prologue's own loads, so the HBM stream starts at the kernel's first
  // instructions instead of after the norm statistics
  Frag af[G];
  u32x2 raw[G];
  auto issue_group = [&](int i0) {
    if constexpr (W8) {
#pragma unroll
      for (int j = 0; j < G; ++j)
        if (i0 + j < kpc) raw[j] = i8_load(qbase + (size_t)(i0 + j) * TILE_ELEMS);
    } else {
#pragma unroll
      for (int j = 0; j < G; ++j)
        if (i0 + j < kpc) af[j] = ldw8(wbase + (size_t)(i0 + j) * TILE_ELEMS);
    }
  };
  issue_group(0);

  // adaptive RMSNorm statistics: 1/sqrt(mean(h^2) + eps) per activation row,
  // from the per-tile sums of squares the producer of h left behind (all
  // loads of a batch issued before the first add; the adds keep tile order).
  // For up to two row tiles it runs after the first activation sub-group's
  // loads are issued, so the statistics and the activations share one
  // memory round trip; with more rows that would hold too many registers at
  // once, and it runs first.
  float rinv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) rinv[mt] = 0.f;
  auto norm_stats = [&]() {
    constexpr int SSU = 16;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = mt * 16 + rloc;
      float s = 0.f;
      if (row < a.rows) {
        for (int t0 = grp; t0 < a.NTD; t0 += 4 * SSU) {
          float sv[SSU];
#pragma unroll
          for (int u = 0; u < SSU; ++u) {
            const int t = t0 + 4 * u;
            sv[u] = t < a.NTD ? a.ss[(size_t)t * a.ss_ld + row] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < SSU; ++u) s += sv[u];
        }
      }
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      rinv[mt] = 1.0f / sqrtf(s / (float)a.D + a.eps);
    }
  };
  constexpr bool STATS_FIRST = MT > 2;
  if constexpr (PRO == PRO_NORM && STATS_FIRST) norm_stats();

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Activation operands in sub-groups of GA tiles: every load of a sub-group
  // (and of its modulation rows) goes out before the first MFMA that uses
  // it, so a wave pays one memory round trip per sub-group, not per tile.
  // The scheduling barriers keep the compiler from interleaving the loads
  // with the MFMAs again.
  constexpr int GA = PRO == PRO_NORM ? (MT <= 1 ? 4 : (MT <= 2 ? 2 : 1)) : G;
  static_assert(G % GA == 0, "activation sub-groups divide the weight group");
  for (int i0 = 0; i0 < kpc; i0 += G) {
    if (i0 > 0) issue_group(i0);
#pragma unroll
    for (int a0 = 0; a0 < G; a0 += GA) {
      if (i0 + a0 >= kpc) break;
      Frag bfr[GA][MT];
      if constexpr (PRO == PRO_NORM) {
        f32x8 s8[GA], m8[GA], h8[GA][MT];
#pragma unroll
        for (int j = 0; j < GA; ++j) {
          if (i0 + a0 + j < kpc) {
            const int k0 = (kt0 + i0 + a0 + j) * TILE_K + grp * 8;
            s8[j] = ld8(a.mod + k0);
            m8[j] = ld8(a.mod + a.D + k0);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const int row = mt * 16 + rloc;
              h8[j][mt] = row < a.rows ? ld8(a.h + (size_t)row * a.D + k0) : f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            }
          }
        }
        if (!STATS_FIRST && a0 == 0 && i0 == 0) norm_stats();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < GA; ++j) {
          if (i0 + a0 + j < kpc) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              float t[8];
#pragma unroll
              for (int q = 0; q < 8; ++q) t[q] = h8[j][mt][q] * rinv[mt] * (1.0f + s8[j][q]) + m8[j][q];
              bfr[j][mt] = mt * 16 + rloc < a.rows ? to_frag<T>(t) : zero_frag<Frag>();
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < GA; ++j) {
          if (i0 + a0 + j < kpc) {
            const int k0 = (kt0 + i0 + a0 + j) * TILE_K + grp * 8;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              bfr[j][mt] = load_act<T, PRO>(a, mt * 16 + rloc, k0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (W8) {  // codes to bf16 after every load of the sub-group is out
#pragma unroll
        for (int j = 0; j < GA; ++j)
          if (i0 + a0 + j < kpc) af[a0 + j] = i8_frag(raw[a0 + j]);
      }
#pragma unroll
      for (int j = 0; j < GA; ++j)
        if (i0 + a0 + j < kpc)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) mma(acc[mt], af[a0 + j], bfr[j][mt]);
    }
  }

  // reduce the K chunks of the workgroup's waves in a fixed order
  if constexpr (NW > 1) {
    __shared__ f32x4 red[NW - 1][MT][64];
    if (w > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[w - 1][mt][lane] = acc[mt];
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int v = 0; v < NW - 1; ++v)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] += red[v][mt][lane];
  }

  // across workgroups: partials to memory, the last workgroup to arrive sums
  // all of them in split order and runs the epilogue
  if (a.KSW > 1) {
    float* p = a.part + ((size_t)(nt * a.KSW + ks) * MT) * 256;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st_coherent(p + (mt * 64 + lane) * 4 + i, acc[mt][i]);
    __builtin_amdgcn_s_waitcnt(0);  // partials have reached the coherent level
    unsigned old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(&a.counters[nt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0);
    if (old != (unsigned)(a.KSW - 1)) return;
    if (lane == 0) __hip_atomic_store(&a.counters[nt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // a batch of splits' partials in flight at once, summed in split order
    constexpr int SU = MT <= 1 ? 8 : (MT <= 2 ? 4 : 1);
    for (int s0 = 0; s0 < a.KSW; s0 += SU) {
      f32x4 pv[SU][MT];
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        if (s0 + u < a.KSW) {
          const float* ps = a.part + ((size_t)(nt * a.KSW + s0 + u) * MT) * 256;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[u][mt][i] = ld_coherent(ps + (mt * 64 + lane) * 4 + i);
        }
      }
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if (s0 + u < a.KSW)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] += pv[u][mt];
    }
  }

  // the 8-bit tier's column scales (tile column order)
  if constexpr (W8) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] *= wsc4;
  }

  // ------------------------------------------------------------ epilogues
  // lane (rloc, grp) holds output columns 4*grp .. 4*grp+3 of the tile for
  // activation row mt*16 + rloc
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = mt * 16 + rloc;
    const bool valid = row < a.rows;
    if constexpr (EPI == EPI_STORE_H || EPI == EPI_RESID) {
      const int col0 = nt * 16 + grp * 4;
      f32x4 v = acc[mt];
      float sq = 0.f;
      if (valid) {
        f32x4* hp = (f32x4*)(a.hout + (size_t)row * a.D + col0);
        if constexpr (EPI == EPI_RESID) v += *hp;
        *hp = v;
        sq = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      }
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
      if (valid && grp == 0) a.ssout[(size_t)nt * a.ss_ld + row] = sq;
    } else if constexpr (EPI == EPI_GEGLU) {
      if (valid) {
        const int f0 = nt * 8 + grp * 2;
        T* ap = (T*)a.act + (size_t)row * a.F + f0;
        st(ap, gelu_tanh(acc[mt][0]) * acc[mt][2]);
        st(ap + 1, gelu_tanh(acc[mt][1]) * acc[mt][3]);
      }
    } else if constexpr (EPI == EPI_EULER) {
      if (valid) {
        const int col0 = nt * 16 + grp * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (col0 + i < a.A) a.x[(size_t)row * a.A + col0 + i] += a.dt * acc[mt][i];
      }
    } else if constexpr (EPI == EPI_QKV) {
      if (valid) {
        const int tph = a.Dh / 16;
        const int hh = nt / tph;
        const int t = nt - hh * tph;
        const int half = a.Dh / 2;
        const int j0 = 8 * t + 2 * grp;
        const int b = row / a.M;
        const int i = row - b * a.M;
        const int slot = a.lens[b] + i;
        float y0 = acc[mt][0], y1 = acc[mt][1], y2 = acc[mt][2], y3 = acc[mt][3];
        if (hh < a.H + a.KVH) {
          const float2 cs0 = a.rope[(size_t)row * half + j0];
          const float2 cs1 = a.rope[(size_t)row * half + j0 + 1];
          const float x0 = y0, x1 = y1, x2 = y2, x3 = y3;
          y0 = x0 * cs0.x - x2 * cs0.y;
          y2 = x2 * cs0.x + x0 * cs0.y;
          y1 = x1 * cs1.x - x3 * cs1.y;
          y3 = x3 * cs1.x + x1 * cs1.y;
        }
        if (hh < a.H) {
          T* qp = (T*)a.q + ((size_t)row * a.H + hh) * a.Dh;
          st(qp + j0, y0);
          st(qp + j0 + 1, y1);
          st(qp + j0 + half, y2);
          st(qp + j0 + 1 + half, y3);
        } else if (hh < a.H + a.KVH) {
          const int kv = hh - a.H;
          T* kp = (T*)a.kc + (((size_t)b * a.KVH + kv) * a.Ctot + slot) * a.Dh;
          st(kp + j0, y0);
          st(kp + j0 + 1, y1);
          st(kp + j0 + half, y2);
          st(kp + j0 + 1 + half, y3);
        } else {
          const int kv = hh - a.H - a.KVH;
          T* vp = (T*)a.vtc + ((size_t)b * a.KVH + kv) * a.Dh * a.Ctot + slot;
          st(vp + (size_t)j0 * a.Ctot, y0);
          st(vp + (size_t)(j0 + 1) * a.Ctot, y1);
          st(vp + (size_t)(j0 + half) * a.Ctot, y2);
          st(vp + (size_t)(j0 + 1 + half) * a.Ctot, y3);
        }
      }
    }
  }
}

// -------------------------------------------------------------- attention
//
// Multi-query attention of one request's action rows to its T = L + M keys
// (the L prefix rows and the M action rows written by the QKV epilogue into
// the cache slots L .. L+M-1), split along the keys in chunks of 64
// (flash-decoding).  Workgroup (request, kv head, split) has one wave per 16
// query rows; the query rows of a kv head are its G = H/KVH heads times M.
//
// S^T = K . Q^T puts keys on the MFMA's 16-row side.  Loading key tile rows
// in the order 8*(m/4) + (m%4) (+4 for the second tile of a pair) leaves
// each lane holding 8 consecutive keys of one query row, which is exactly
// the A operand of O = P . V, and V is stored transposed so its B operand
// is one contiguous 16-byte read.  Partial (max, sum, unnormalised output)
// per split are combined by k_combine in split order.
// This form loads every fragment straight from memory; it runs the float32
// workloads (bf16 runs k_attn_lds below, which stages the chunk in LDS).
template <typename T, int DH>
__global__ __launch_bounds__(512) void k_attn(AttnArgs a) {
  using Frag = typename FragT<T>::type;
  constexpr int DS = DH / 32;
  constexpr int DT = DH / 16;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rloc = lane & 15;
  const int grp = lane >> 4;
  const int s = blockIdx.x % a.SMAX;
  const int bk = blockIdx.x / a.SMAX;  // request * KVH + kv head
  const int b = bk / a.KVH;
  const int kvh = bk - b * a.KVH;
  const int T_b = a.lens[b] + a.M;
  const int kbase = s * ATTN_KEYS;
  if (kbase >= T_b) return;
  const int G = a.H / a.KVH;
  const int GM = G * a.M;
  if (w * 16 >= GM) return;  // a wave with no query row (no barrier follows)
  const int r = w * 16 + rloc;
  const bool rvalid = r < GM;
  const int hh = kvh * G + (rvalid ? r / a.M : 0);
  const int i = rvalid ? r % a.M : 0;

  Frag qf[DS];
  const T* qrow = (const T*)a.q + ((size_t)(b * a.M + i) * a.H + hh) * DH + grp * 8;
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) qf[ds] = rvalid ? ld8(qrow + ds * 32) : zero_frag<Frag>();

  const T* kb = (const T*)a.kc + (size_t)bk * a.Ctot * DH;
  const T* vb = (const T*)a.vtc + (size_t)bk * DH * a.Ctot;

  // Loads in explicit phases, each phase's loads all in flight before the
  // first use: the key fragments (half of them at a time when they would
  // not fit the registers), then the value fragments, together with the
  // keys when both fit and otherwise after the score MFMAs (they do not
  // depend on the scores, so they arrive while the softmax runs).  The
  // scheduling barriers keep the compiler from interleaving loads and MFMAs
  // again, which left about four loads in flight.
  constexpr int FRAG_REGS = (int)sizeof(Frag) / 4;
  constexpr int K_REGS = 4 * DS * FRAG_REGS, V_REGS = 2 * DT * FRAG_REGS;
  constexpr bool K_HALVES = K_REGS > 128;               // float32 at head_dim 256: half the keys at a time
  constexpr bool V_EARLY = K_REGS + V_REGS <= 128;
  Frag kf[2][2][DS];
  auto load_k = [&](int p) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int key = kbase + 32 * p + 8 * (rloc >> 2) + 4 * hf + (rloc & 3);
      const T* krow = kb + (size_t)key * DH + grp * 8;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) kf[p][hf][ds] = ld8(krow + ds * 32);
    }
  };
  constexpr bool V_HALVES = V_REGS > 128;               // float32 at head_dim 256: half the keys at a time
  Frag vf[DT][2];
  auto load_v = [&](int p) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const T* vrow = vb + (size_t)(dt * 16 + rloc) * a.Ctot + kbase + grp * 8;
      vf[dt][p] = ld8(vrow + 32 * p);
    }
  };
  f32x4 sacc[2][2];
  auto scores = [&](int p) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      sacc[p][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) mma(sacc[p][hf], kf[p][hf][ds], qf[ds]);
    }
  };
  if constexpr (K_HALVES) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      load_k(p);
      __builtin_amdgcn_sched_barrier(0);
      scores(p);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    load_k(0);
    load_k(1);
    if constexpr (V_EARLY) {
      load_v(0);
      load_v(1);
    }
    __builtin_amdgcn_sched_barrier(0);
    scores(0);
    scores(1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!V_EARLY && !V_HALVES) {
    load_v(0);
    load_v(1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // lane (query row rloc, grp) holds keys kbase + 32p + 8grp + 4hf + ii
  float sv[2][8];
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int key = kbase + 32 * p + 8 * grp + 4 * hf + ii;
        const float v = key < T_b ? sacc[p][hf][ii] * a.scale : -INFINITY;
        sv[p][4 * hf + ii] = v;
        mx = fmaxf(mx, v);
      }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float lsum = 0.f;
  Frag pf[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = expf(sv[p][j] - mx);
      lsum += pv[j];
    }
    pf[p] = to_frag<T>(pv);
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if constexpr (V_HALVES) {
      __builtin_amdgcn_sched_barrier(0);
      load_v(p);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) mma(oacc[dt], pf[p], vf[dt][p]);
  }

  const size_t pbase = ((size_t)bk * a.SMAX + s) * a.GMP;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = w * 16 + 4 * grp + ii;
      if (rr < GM) a.part_o[(pbase + rr) * DH + dt * 16 + rloc] = oacc[dt][ii];
    }
  if (grp == 0 && rvalid) a.part_ml[pbase + r] = make_float2(mx, lsum);
}

// bf16 attention of one split with the key chunk staged in LDS.  Every
// wave of the workgroup needs the whole 64-key chunk (its keys and its
// value columns); fragment reads straight from memory touch 16 rows per
// instruction with half of each 128-byte line used, so the five waves of a
// pi0.5 workgroup pulled ten times the chunk's bytes through the CU's load
// pipe.  Here the workgroup reads the chunk once with whole-line 16-byte
// loads (all in flight together), and the waves read their fragments from
// LDS.  Row strides carry 16 bytes of padding so the 16 rows of a fragment
// read spread over the banks.  Results are those of k_attn: the same MFMAs
// in the same order on the same operands.
template <int DH>
constexpr int attn_lds_bytes() {
  return (ATTN_KEYS * (DH + 8) + DH * (ATTN_KEYS + 8)) * 2;
}

template <int DH>
__global__ __launch_bounds__(512) void k_attn_lds(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char attn_smem[];
  constexpr int DS = DH / 32;
  constexpr int DT = DH / 16;
  constexpr int KST = DH + 8;         // key row stride in LDS (elements)
  constexpr int VST = ATTN_KEYS + 8;  // value (dim) row stride in LDS
  constexpr int KP = ATTN_KEYS * DH / 8, VP = DH * ATTN_KEYS / 8;  // 16-byte pieces
  constexpr int U = 16;               // pieces per thread and batch
  bf16* Ks = (bf16*)attn_smem;
  bf16* Vs = Ks + ATTN_KEYS * KST;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int rloc = lane & 15;
  const int grp = lane >> 4;
  const int s = blockIdx.x % a.SMAX;
  const int bk = blockIdx.x / a.SMAX;  // request * KVH + kv head
  const int b = bk / a.KVH;
  const int kvh = bk - b * a.KVH;
  const int T_b = a.lens[b] + a.M;
  const int kbase = s * ATTN_KEYS;
  if (kbase >= T_b) return;  // the whole workgroup: no barrier is skipped
  const int G = a.H / a.KVH;
  const int GM = G * a.M;
  const bool wave_rows = w * 16 < GM;
  const int r = w * 16 + rloc;
  const bool rvalid = r < GM;
  const int hh = kvh * G + (rvalid ? r / a.M : 0);
  const int i = rvalid ? r % a.M : 0;

  bf16x8 qf[DS];
  const bf16* qrow = (const bf16*)a.q + ((size_t)(b * a.M + i) * a.H + hh) * DH + grp * 8;
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) qf[ds] = rvalid ? ld8(qrow + ds * 32) : zero_frag<bf16x8>();

  // stage the chunk: key rows kbase .. kbase + 63 and the same columns of
  // the transposed values (rows past the keys in use are read too; their
  // probabilities are zero, as in the direct-load kernel)
  const bf16* kb = (const bf16*)a.kc + (size_t)bk * a.Ctot * DH;
  const bf16* vb = (const bf16*)a.vtc + (size_t)bk * DH * a.Ctot;
  for (int i0 = tid; i0 < KP + VP; i0 += U * nthr) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = i0 + u * nthr;
      if (idx < KP) {
        const int key = idx / (DH / 8), c = idx % (DH / 8);
        v[u] = *(const u32x4*)(kb + (size_t)(kbase + key) * DH + c * 8);
      } else if (idx < KP + VP) {
        const int j = idx - KP, dim = j / (ATTN_KEYS / 8), c = j % (ATTN_KEYS / 8);
        v[u] = *(const u32x4*)(vb + (size_t)dim * a.Ctot + kbase + c * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = i0 + u * nthr;
      if (idx < KP) {
        const int key = idx / (DH / 8), c = idx % (DH / 8);
        *(u32x4*)(Ks + key * KST + c * 8) = v[u];
      } else if (idx < KP + VP) {
        const int j = idx - KP, dim = j / (ATTN_KEYS / 8), c = j % (ATTN_KEYS / 8);
        *(u32x4*)(Vs + dim * VST + c * 8) = v[u];
      }
    }
  }
  __syncthreads();
  if (!wave_rows) return;  // a wave with no query row (no barrier follows)

  f32x4 sacc[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      sacc[p][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = 32 * p + 8 * (rloc >> 2) + 4 * hf + (rloc & 3);
      const bf16* krow = Ks + key * KST + grp * 8;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        mma(sacc[p][hf], __builtin_bit_cast(bf16x8, *(const u32x4*)(krow + ds * 32)), qf[ds]);
    }

  // lane (query row rloc, grp) holds keys kbase + 32p + 8grp + 4hf + ii
  float sv[2][8];
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int key = kbase + 32 * p + 8 * grp + 4 * hf + ii;
        const float v = key < T_b ? sacc[p][hf][ii] * a.scale : -INFINITY;
        sv[p][4 * hf + ii] = v;
        mx = fmaxf(mx, v);
      }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float lsum = 0.f;
  bf16x8 pf[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = expf(sv[p][j] - mx);
      lsum += pv[j];
    }
    pf[p] = to_frag<bf16>(pv);
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16* vrow = Vs + (dt * 16 + rloc) * VST + grp * 8;
#pragma unroll
    for (int p = 0; p < 2; ++p) mma(oacc[dt], pf[p], __builtin_bit_cast(bf16x8, *(const u32x4*)(vrow + 32 * p)));
  }

  const size_t pbase = ((size_t)bk * a.SMAX + s) * a.GMP;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = w * 16 + 4 * grp + ii;
      if (rr < GM) a.part_o[(pbase + rr) * DH + dt * 16 + rloc] = oacc[dt][ii];
    }
  if (grp == 0 && rvalid) a.part_ml[pbase + r] = make_float2(mx, lsum);
}

// one thread per 4 dims of a query row (1024 / Dh rows per workgroup); splits in order
template <typename T>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int G = a.H / a.KVH;
  const int GM = G * a.M;
  const int tpr = a.Dh / 4;
  const int rpb = 256 / tpr;
  const int nrb = (GM + rpb - 1) / rpb;
  const int bk = blockIdx.x / nrb;
  const int r = (blockIdx.x - bk * nrb) * rpb + (int)threadIdx.x / tpr;
  const int d = 4 * ((int)threadIdx.x % tpr);
  if (r >= GM) return;
  const int b = bk / a.KVH;
  const int kvh = bk - b * a.KVH;
  const int ns = (a.lens[b] + a.M + ATTN_KEYS - 1) / ATTN_KEYS;
  const size_t base = (size_t)bk * a.SMAX * a.GMP + r;
  // up to ONE splits (the pi0.5 and rollout shapes): every statistic and
  // partial in flight at once, one memory round; more splits: batches of
  // CU, one round for the maxima and one for the sums per batch.  Maxima
  // and sums in split order either way.
  constexpr int ONE = 16, CU = 8;
  float mx = -INFINITY;
  float den = 0.f;
  f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ns <= ONE) {
    float2 ml[ONE];
    f32x4 po[ONE];
#pragma unroll
    for (int u = 0; u < ONE; ++u) {
      if (u < ns) {
        const size_t e = base + (size_t)u * a.GMP;
        ml[u] = a.part_ml[e];
        po[u] = *(const f32x4*)(a.part_o + e * a.Dh + d);
      }
    }
#pragma unroll
    for (int u = 0; u < ONE; ++u)
      if (u < ns) mx = fmaxf(mx, ml[u].x);
#pragma unroll
    for (int u = 0; u < ONE; ++u) {
      if (u < ns) {
        const float wgt = expf(ml[u].x - mx);
        den += ml[u].y * wgt;
        num += wgt * po[u];
      }
    }
  } else {
    for (int s0 = 0; s0 < ns; s0 += CU) {
      float m[CU];
#pragma unroll
      for (int u = 0; u < CU; ++u) m[u] = s0 + u < ns ? a.part_ml[base + (size_t)(s0 + u) * a.GMP].x : -INFINITY;
#pragma unroll
      for (int u = 0; u < CU; ++u) mx = fmaxf(mx, m[u]);
    }
    for (int s0 = 0; s0 < ns; s0 += CU) {
      float2 ml[CU];
      f32x4 po[CU];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        if (s0 + u < ns) {
          const size_t e = base + (size_t)(s0 + u) * a.GMP;
          ml[u] = a.part_ml[e];
          po[u] = *(const f32x4*)(a.part_o + e * a.Dh + d);
        }
      }
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        if (s0 + u < ns) {
          const float wgt = expf(ml[u].x - mx);
          den += ml[u].y * wgt;
          num += wgt * po[u];
        }
      }
    }
  }
  const int hh = kvh * G + r / a.M;
  const int i = r % a.M;
  T* op = (T*)a.o + ((size_t)(b * a.M + i) * a.H + hh) * a.Dh + d;
#pragma unroll
  for (int j = 0; j < 4; ++j) op[j] = (T)(num[j] / den);
}

// ------------------------------------------------------------ set-up kernels

__device__ inline int colmap(int kind, int param, int nt, int c) {
  if (kind == COL_IDENT) return nt * 16 + c;
  const int g = c >> 2, i = c & 3;
  if (kind == COL_ROPE) {  // param = head_dim: tile t of a head holds pairs j = 8t..8t+7 and their partners
    const int tph = param / 16;
    const int hh = nt / tph, t = nt - hh * tph;
    const int j = 8 * t + 2 * g + (i & 1);
    return hh * param + j + (i >> 1) * (param / 2);
  }
  // COL_GEGLU, param = F: tile t holds gate f = 8t..8t+7 and up F+f
  const int f = 8 * nt + 2 * g + (i & 1);
  return f + (i >> 1) * param;
}

// one thread per lane fragment (8 elements) of the destination
template <typename T>
__global__ void k_retile(const T* __restrict__ src, T* __restrict__ dst, int K, int N, int kind, int param) {
  const int KT = K / TILE_K, NT = N / TILE_N;
  const size_t nfrag = (size_t)NT * KT * 64;
  for (size_t f = (size_t)blockIdx.x * blockDim.x + threadIdx.x; f < nfrag; f += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(f & 63);
    const size_t tile = f >> 6;
    const int nt = (int)(tile / KT), kt = (int)(tile % KT);
    const int n = colmap(kind, param, nt, lane & 15);
    const int k0 = kt * TILE_K + 8 * (lane >> 4);
    T* d = dst + f * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = src[(size_t)(k0 + j) * N + n];
  }
}

// 8-bit tier ("PhyAI" section 4.2 Quantization: offline round-to-nearest,
// W8A16).  Per output column of a tiled bf16 matrix: s = max |w| / 127 (one
// thread per tile column, tile column order), then q = rint(w / s) clamped
// to +-127 (ties to even; both divisions correctly rounded float32), 0 where
// s = 0; codes keep the tile order, one byte per weight.
__global__ void k_quant_scale(const bf16* __restrict__ wt, float* __restrict__ sc, int KT, int NT) {
  const int col = blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= NT * 16) return;
  const int nt = col >> 4, c = col & 15;
  float m = 0.f;
  for (int kt = 0; kt < KT; ++kt)
    for (int g = 0; g < 4; ++g) {
      const bf16* p = wt + (((size_t)nt * KT + kt) * 64 + c + 16 * g) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)p[j]));
    }
  sc[col] = m / 127.0f;
}

__global__ void k_quant_codes(const bf16* __restrict__ wt, const float* __restrict__ sc, signed char* __restrict__ q,
                              int KT, int NT) {
  const size_t nfrag = (size_t)NT * KT * 64;
  for (size_t f = (size_t)blockIdx.x * blockDim.x + threadIdx.x; f < nfrag; f += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(f & 63);
    const int nt = (int)((f >> 6) / KT);
    const float s = sc[nt * 16 + (lane & 15)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = s > 0.f ? rintf((float)wt[f * 8 + j] / s) : 0.f;
      v = fminf(fmaxf(v, -127.f), 127.f);
      q[f * 8 + j] = (signed char)(int)v;
    }
  }
}

// codes of a tiled matrix back to [K][N] through the column map, scales to [N]
__global__ void k_untile_codes(const signed char* __restrict__ qt, const float* __restrict__ sct,
                               signed char* __restrict__ q, float* __restrict__ sc, int K, int N, int kind,
                               int param) {
  const int KT = K / TILE_K, NT = N / TILE_N;
  const size_t nfrag = (size_t)NT * KT * 64;
  for (size_t f = (size_t)blockIdx.x * blockDim.x + threadIdx.x; f < nfrag; f += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(f & 63);
    const size_t tile = f >> 6;
    const int nt = (int)(tile / KT), kt = (int)(tile % KT);
    const int n = colmap(kind, param, nt, lane & 15);
    const int k0 = kt * TILE_K + 8 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[(size_t)(k0 + j) * N + n] = qt[f * 8 + j];
    if (kt == 0 && lane < 16) sc[n] = sct[nt * 16 + lane];
  }
}

// e[k][j] = sin(tau_k w_j), e[k][E/2 + j] = cos(tau_k w_j), w_j = 10000^(-j/(E/2))
__global__ void k_time_embedding(double* e, int S, int E, double tau0, double dt) {
  const int half = E / 2;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < S * half; idx += gridDim.x * blockDim.x) {
    const int k = idx / half, j = idx % half;
    const double tau = tau0 + (double)k * dt;
    const double w = pow(10000.0, -(double)j / (double)half);
    e[(size_t)k * E + j] = sin(tau * w);
    e[(size_t)k * E + half + j] = cos(tau * w);
  }
}

// modtab[k][n][c] = sum_j e[k][j] * Wmod[n][j][c], accumulated in double
template <typename T>
__global__ void k_modulation(const T* __restrict__ wmod, const double* __restrict__ e, float* __restrict__ out, int S,
                             int NN, int E, int D2) {
  const size_t total = (size_t)S * NN * D2;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(idx % D2);
    const size_t kn = idx / D2;
    const int n = (int)(kn % NN), k = (int)(kn / NN);
    const T* wc = wmod + (size_t)n * E * D2 + c;
    const double* ek = e + (size_t)k * E;
    double s = 0.0;
    for (int j = 0; j < E; ++j) s += ek[j] * (double)(float)wc[(size_t)j * D2];
    out[idx] = (float)s;
  }
}

// copy one request's prefix K/V (caller layout [NL][L][KVH*Dh]) into the
// caches: K as [NL][B][KVH][Ctot][Dh], V transposed as [NL][B][KVH][Dh][Ctot];
// rows L .. Ctot-1 are cleared
template <typename T>
__global__ void k_load_prefix(const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ kc,
                              T* __restrict__ vtc, int NL, int B, int KVH, int Dh, int Ctot, int b, int L) {
  const size_t per_layer = (size_t)KVH * Ctot * Dh;
  const size_t total = (size_t)NL * per_layer;
  const int kvd = KVH * Dh;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int d = (int)(idx % Dh);
    size_t rest = idx / Dh;
    const int t = (int)(rest % Ctot);
    rest /= Ctot;
    const int kv = (int)(rest % KVH);
    const int l = (int)(rest / KVH);
    T kval = (T)0.0f, vval = (T)0.0f;
    if (t < L) {
      const size_t src = ((size_t)l * L + t) * kvd + (size_t)kv * Dh + d;
      kval = k[src];
      vval = v[src];
    }
    const size_t head = ((size_t)l * B + b) * KVH + kv;
    kc[(head * Ctot + t) * Dh + d] = kval;
    vtc[(head * Dh + d) * Ctot + t] = vval;
  }
}

// decoder position table of one request: action row i sits at position L + i
__global__ void k_position_table(int* lens, float2* rope, int b, int L, int M, int Dh, double base) {
  const int half = Dh / 2;
  if (blockIdx.x == 0 && threadIdx.x == 0) lens[b] = L;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < M * half; idx += gridDim.x * blockDim.x) {
    const int i = idx / half, j = idx % half;
    const double theta = pow(base, -2.0 * (double)j / (double)Dh);
    const double ang = (double)(L + i) * theta;
    rope[((size_t)b * M + i) * half + j] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

// ---------------------------------------------------------------- launchers

template <typename T, int MT>
static hipError_t gemm_mt(int nw, int pro, int epi, const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.NT * a.KSW);
  if constexpr (std::is_same<T, bf16>::value) {
    if (a.Wq) {  // the 8-bit tier: the layer projections only
      if (!a.wsc) return hipErrorInvalidValue;
      if (nw == 4 && pro == PRO_NORM && epi == EPI_QKV)
        hipLaunchKernelGGL((k_gemm<T, 4, MT, PRO_NORM, EPI_QKV, true>), grid, dim3(256), 0, s, a);
      else if (nw == 4 && pro == PRO_X && epi == EPI_RESID)
        hipLaunchKernelGGL((k_gemm<T, 4, MT, PRO_X, EPI_RESID, true>), grid, dim3(256), 0, s, a);
      else if (nw == 4 && pro == PRO_NORM && epi == EPI_GEGLU)
        hipLaunchKernelGGL((k_gemm<T, 4, MT, PRO_NORM, EPI_GEGLU, true>), grid, dim3(256), 0, s, a);
      else
        return hipErrorInvalidValue;
      return hipGetLastError();
    }
  } else {
    if (a.Wq) return hipErrorInvalidValue;
  }
  if (nw == 1 && pro == PRO_XF32 && epi == EPI_STORE_H) {
    hipLaunchKernelGGL((k_gemm<T, 1, MT, PRO_XF32, EPI_STORE_H>), grid, dim3(64), 0, s, a);
  } else if (nw == 4 && pro == PRO_NORM && epi == EPI_QKV) {
    hipLaunchKernelGGL((k_gemm<T, 4, MT, PRO_NORM, EPI_QKV>), grid, dim3(256), 0, s, a);
  } else if (nw == 4 && pro == PRO_X && epi == EPI_RESID) {
    hipLaunchKernelGGL((k_gemm<T, 4, MT, PRO_X, EPI_RESID>), grid, dim3(256), 0, s, a);
  } else if (nw == 4 && pro == PRO_NORM && epi == EPI_GEGLU) {
    hipLaunchKernelGGL((k_gemm<T, 4, MT, PRO_NORM, EPI_GEGLU>), grid, dim3(256), 0, s, a);
  } else if (nw == 4 && pro == PRO_NORM && epi == EPI_EULER) {
    hipLaunchKernelGGL((k_gemm<T, 4, MT, PRO_NORM, EPI_EULER>), grid, dim3(256), 0, s, a);
  } else if (nw == 4 && pro == PRO_X && epi == EPI_EULER) {
    hipLaunchKernelGGL((k_gemm<T, 4, MT, PRO_X, EPI_EULER>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t gemm_t(int nw, int mt, int pro, int epi, const GemmArgs& a, hipStream_t s) {
  switch (mt) {
    case 1: return gemm_mt<T, 1>(nw, pro, epi, a, s);
    case 2: return gemm_mt<T, 2>(nw, pro, epi, a, s);
    case 4: return gemm_mt<T, 4>(nw, pro, epi, a, s);
    case 10: return gemm_mt<T, 10>(nw, pro, epi, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int dtype, int nw, int mt, int pro, int epi, const GemmArgs& a, hipStream_t s) {
  return dtype == 1 ? gemm_t<bf16>(nw, mt, pro, epi, a, s) : gemm_t<float>(nw, mt, pro, epi, a, s);
}

template <int DH>
static hipError_t attn_lds(const dim3& grid, const dim3& block, const AttnArgs& a, hipStream_t s) {
  static bool attr_set = false;  // LDS beyond the default 64 KiB (head_dim 256)
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_attn_lds<DH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             attn_lds_bytes<DH>());
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_attn_lds<DH>, grid, block, attn_lds_bytes<DH>(), s, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t attn_t(int qt, const AttnArgs& a, int batch, hipStream_t s) {
  const dim3 grid(batch * a.KVH * a.SMAX), block(qt * 64);
  if constexpr (std::is_same<T, bf16>::value) {
    switch (a.Dh) {
      case 64: return attn_lds<64>(grid, block, a, s);
      case 128: return attn_lds<128>(grid, block, a, s);
      case 256: return attn_lds<256>(grid, block, a, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.Dh) {
      case 64: hipLaunchKernelGGL((k_attn<T, 64>), grid, block, 0, s, a); break;
      case 128: hipLaunchKernelGGL((k_attn<T, 128>), grid, block, 0, s, a); break;
      case 256: hipLaunchKernelGGL((k_attn<T, 256>), grid, block, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
}

hipError_t launch_attention(int dtype, int qt, const AttnArgs& a, int batch, hipStream_t s) {
  return dtype == 1 ? attn_t<bf16>(qt, a, batch, s) : attn_t<float>(qt, a, batch, s);
}

hipError_t launch_combine(int dtype, const CombineArgs& a, int batch, hipStream_t s) {
  if (a.Dh % 4 || a.Dh > 1024 || 1024 % a.Dh) return hipErrorInvalidValue;
  const int GM = (a.H / a.KVH) * a.M, rpb = 1024 / a.Dh;
  const dim3 grid(batch * a.KVH * ((GM + rpb - 1) / rpb)), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_combine<bf16>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_combine<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quant_i8(const void* wt, signed char* q, float* sc, int K, int N, hipStream_t s) {
  if (K % TILE_K || N % TILE_N) return hipErrorInvalidValue;
  const int KT = K / TILE_K, NT = N / TILE_N;
  hipLaunchKernelGGL(k_quant_scale, dim3((NT * 16 + 255) / 256), dim3(256), 0, s, (const bf16*)wt, sc, KT, NT);
  const size_t nfrag = (size_t)KT * NT * 64;
  const int blocks = (int)((nfrag + 255) / 256 < 65535 ? (nfrag + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_quant_codes, dim3(blocks), dim3(256), 0, s, (const bf16*)wt, (const float*)sc, q, KT, NT);
  return hipGetLastError();
}

hipError_t launch_untile_codes(const signed char* qt, const float* sct, signed char* q, float* sc, int K, int N,
                               int colmap_kind, int cm_param, hipStream_t s) {
  if (K % TILE_K || N % TILE_N) return hipErrorInvalidValue;
  const size_t nfrag = (size_t)(K / TILE_K) * (N / TILE_N) * 64;
  const int blocks = (int)((nfrag + 255) / 256 < 65535 ? (nfrag + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_untile_codes, dim3(blocks), dim3(256), 0, s, qt, sct, q, sc, K, N, colmap_kind, cm_param);
  return hipGetLastError();
}

hipError_t launch_retile(int dtype, const void* src, void* dst, int K, int N, int colmap_kind, int cm_param,
                         hipStream_t s) {
  const size_t nfrag = (size_t)(K / TILE_K) * (N / TILE_N) * 64;
  const int blocks = (int)((nfrag + 255) / 256 < 65535 ? (nfrag + 255) / 256 : 65535);
  if (dtype == 1)
    hipLaunchKernelGGL(k_retile<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)src, (bf16*)dst, K, N,
                       colmap_kind, cm_param);
  else
    hipLaunchKernelGGL(k_retile<float>, dim3(blocks), dim3(256), 0, s, (const float*)src, (float*)dst, K, N,
                       colmap_kind, cm_param);
  return hipGetLastError();
}

hipError_t launch_time_embedding(double* e, int S, int E, double tau0, double dt, hipStream_t s) {
  const int n = S * (E / 2);
  hipLaunchKernelGGL(k_time_embedding, dim3((n + 255) / 256), dim3(256), 0, s, e, S, E, tau0, dt);
  return hipGetLastError();
}

hipError_t launch_modulation(int dtype, const void* wmod, const double* e, float* modtab, int S, int NN, int E,
                             int D2, hipStream_t s) {
  const size_t total = (size_t)S * NN * D2;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  if (dtype == 1)
    hipLaunchKernelGGL(k_modulation<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)wmod, e, modtab, S, NN, E,
                       D2);
  else
    hipLaunchKernelGGL(k_modulation<float>, dim3(blocks), dim3(256), 0, s, (const float*)wmod, e, modtab, S, NN,
                       E, D2);
  return hipGetLastError();
}

hipError_t launch_load_prefix(int dtype, const void* k, const void* v, void* kc, void* vtc, int NL, int B, int KVH,
                              int Dh, int Ctot, int request, int L, hipStream_t s) {
  const size_t total = (size_t)NL * KVH * Ctot * Dh;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  if (dtype == 1)
    hipLaunchKernelGGL(k_load_prefix<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)k, (const bf16*)v,
                       (bf16*)kc, (bf16*)vtc, NL, B, KVH, Dh, Ctot, request, L);
  else
    hipLaunchKernelGGL(k_load_prefix<float>, dim3(blocks), dim3(256), 0, s, (const float*)k, (const float*)v,
                       (float*)kc, (float*)vtc, NL, B, KVH, Dh, Ctot, request, L);
  return hipGetLastError();
}

hipError_t launch_position_table(int* lens, float2* rope, int request, int L, int M, int Dh, double base,
                                 hipStream_t s) {
  const int n = M * (Dh / 2);
  hipLaunchKernelGGL(k_position_table, dim3((n + 255) / 256), dim3(256), 0, s, lens, rope, request, L, M, Dh,
                     base);
  return hipGetLastError();
}

}  // namespace phx
