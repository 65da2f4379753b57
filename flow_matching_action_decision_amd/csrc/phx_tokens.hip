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

#include <algorithm>
#include <cmath>

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

// Paired rows (see phx_tokens.h): columns c .. c + n - 1 (one 32-column
// chunk, c a multiple of n) of a paired row get hi = bf16(y) and lo =
// bf16(y - hi); the difference y - hi is exact in float32.
__device__ inline void store_pair2(bf16* row, int c, float y0, float y1) {
  const bf16 h0 = (bf16)y0, h1 = (bf16)y1;
  bf16* p = row + (c >> 5) * 64 + (c & 31);
  *(unsigned*)p = (unsigned)bits(h0) | ((unsigned)bits(h1) << 16);
  *(unsigned*)(p + 32) = pack2(y0 - (float)h0, y1 - (float)h1);
}
__device__ inline void store_pair4(bf16* row, int c, const float (&y)[4]) {
  bf16 hb[4];
  float lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hb[i] = (bf16)y[i];
    lo[i] = y[i] - (float)hb[i];
  }
  bf16* p = row + (c >> 5) * 64 + (c & 31);
  *(u32x2*)p = u32x2{(unsigned)bits(hb[0]) | ((unsigned)bits(hb[1]) << 16),
                     (unsigned)bits(hb[2]) | ((unsigned)bits(hb[3]) << 16)};
  *(u32x2*)(p + 32) = u32x2{pack2(lo[0], lo[1]), pack2(lo[2], lo[3])};
}
// Hardware base-2 exponential (v_exp_f32, about 1 ulp; results below 2^-126
// flush to zero, which every use here tolerates: softmax terms that small
// vanish beside the row sum, and tanh saturates long before).  exp2f would
// add a range fix-up of four more VALU instructions to every call.
__device__ inline float hexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh-form GELU with tanh(u) = 1 - 2 / (exp(2u) + 1) from the hardware
// exponential and reciprocal (a few ulp of float32, far below the bf16
// rounding of every output; exp overflow gives tanh = 1, underflow -1)
__device__ inline float gelu_tanh(float z) {
  const float k = 0.7978845608028654f;  // sqrt(2/pi)
  const float u = k * (z + 0.044715f * z * z * z);
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(hexp2(2.0f * 1.4426950408889634f * u) + 1.0f);
  return 0.5f * z * (1.0f + t);
}

__device__ inline f32x4 mma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mma16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ GEMM
// Workgroup of 4 waves covering output columns [BN bx, +BN) (BN = 64 WN) and
// rows [BM by, +BM) (BM = 16 WM); wave w owns n-tiles WN (4 bx + w) + [0, WN)
// and all WM m-tiles, so per 32-deep k-step it runs WN x WM MFMAs on WN weight
// fragments and the WM activation fragments the four waves share.  Two ways
// to feed it, chosen per GEMM by the planner:
//
// k_tgemm_ring (few rows: the weights stream from HBM once and latency rules):
// both operands reach LDS straight from memory (buffer loads with the LDS bit,
// no registers in between), each 1 KiB load already in MFMA fragment order (a
// weight tile, or 16 activation rows x 64 bytes), through a ring of NS = 4
// stages (deeper rings measured slower: fewer workgroups fit a CU); every
// wave waits for its own loads with an explicit vmcnt and a barrier publishes
// the stage, so NS - 1 k-steps are in flight.
//
// k_tgemm_reg (many rows: MFMA-bound, and LDS bandwidth is the limit): a
// wave's weight fragments are its own, so they go from memory straight into
// registers WPD k-steps ahead; only the shared activation rows pass through a
// double-buffered LDS block, fetched two k-steps ahead; two workgroups per CU.
// All its loads are ordinary loads, so the compiler's own waits track them.
//
// With split > 1 workgroup z multiplies k-steps [z KT/split, (z+1) KT/split)
// and stores its raw sums for an ordered reduction.
constexpr int WPD = 2;     // weight prefetch distance in k-steps (k_tgemm_reg)
constexpr int PAIR_STAGES = 6;  // stages of the ring GEMM on paired activation rows (4: the rollout 1% slower)
constexpr int UNR = 4;     // k_tgemm_reg main-loop unroll: its register rings rotate with it
static_assert(WPD < UNR && UNR % 2 == 0, "the weight ring holds UNR k-steps, the activation ring 2");

template <int WN, int WM>
struct Tile {
  static constexpr int BN = 64 * WN, BM = 16 * WM;
  static constexpr int FR = WM + 4 * WN;  // ring: 1 KiB fragments per k-step
  static constexpr int PW = WM / 4 + WN;  // ring: loads per wave per k-step
  static constexpr int STAGE = FR * 1024;
  static constexpr int NS = 4;
  static constexpr int LDS = NS * STAGE;
  static_assert((NS - 2) * PW <= 63, "vmcnt holds at most 63 loads");
  static constexpr int AP = BM / 64;      // reg: 16-byte activation pieces per thread per k-step
};

__device__ inline void tile_of(int bid, int gx, int gy, int nz, int& bx, int& by, int& z) {
  z = bid / (gx * gy);
  const int t = bid - z * gx * gy;
  bx = t % gx;
  by = t / gx;
}

__device__ inline u32x4 rsrc_words(const void* p, unsigned bytes) {
  const unsigned long long b = (unsigned long long)p;
  return u32x4{(unsigned)b, (unsigned)(b >> 32) & 0xffffu, bytes, 0x00020000u};
}

// one 1 KiB fragment into LDS at M0 + 16 lane
__device__ inline void dma_frag(unsigned lds, unsigned voff, u32x4 rs, unsigned soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rs),
               "s"(soff)
               : "memory", "m0");
}

template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most PW * min(ahead, A) loads are in flight
template <int PW, int A>
__device__ inline void wait_ahead(int ahead) {
  if constexpr (A <= 0) {
    wait_vm<0>();
  } else {
    if (ahead >= A) wait_vm<PW * A>();
    else wait_ahead<PW, A - 1>(ahead);
  }
}

// barrier without the fence __syncthreads implies (that fence would wait for
// every load in flight); the empty asm statements keep LDS accesses on their side
__device__ inline void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Values of one kv head in the order the attention's PV step reads them: for
// each 32-key step j and 16-dim tile dt (ndt = head_dim / 16 of them), one
// 1 KiB MFMA fragment in which lane (d % 16) + 16 g holds dim d and the keys
// 32 j + 4 g + [0, 4) (elements 0..3) and 32 j + 16 + 4 g + [0, 4) (4..7).
__device__ inline size_t vt_index(int kvh, int nj, int t, int d, int ndt) {
  const int j = t >> 5, kk = t & 31, rr = kk & 15;
  const int e = (rr & 3) + 4 * (kk >> 4), ln = (d & 15) + 16 * (rr >> 2);
  return ((((size_t)kvh * nj + j) * ndt + (d >> 4)) * 64 + ln) * 8 + e;
}

// inverse of vt_index within one kv head's plane
__device__ inline void vt_key_dim(int i, int ndt, int& t, int& d) {
  const int e = i & 7, ln = (i >> 3) & 63, f = i >> 9;
  const int dt = f % ndt, j = f / ndt;
  d = 16 * dt + (ln & 15);
  t = 32 * j + 16 * (e >> 2) + 4 * (ln >> 4) + (e & 3);
}

// output columns 4 gq + [0, 4) of n-tile nt (tile order) of one row
template <int EPI>
__device__ inline void epi_store(const GemmT& g, int row, int nt, int gq, const f32x4& v) {
  if constexpr (EPI == EP_BF16 || EPI == EP_GELU) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = EPI == EP_GELU ? gelu_tanh(v[i]) : v[i];
    if (EPI == EP_GELU && g.osplit)
      store_pair4((bf16*)g.out + (size_t)row * g.ldo, nt * 16 + 4 * gq, y);
    else
      *(u32x2*)((bf16*)g.out + (size_t)row * g.ldo + nt * 16 + 4 * gq) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
  } else if constexpr (EPI == EP_QKV) {
    // tile order of a head (query heads, then key heads, then value heads) of
    // hd dims: the values are dims j, j + 1, j + hd/2, j + hd/2 + 1 with
    // j = 8 (nt % (hd/16)) + 2 gq
    const int tph = g.hd >> 4, half = g.hd >> 1;
    const int hh = nt / tph, j = 8 * (nt - hh * tph) + 2 * gq;
    float y0 = v[0], y1 = v[1], y2 = v[2], y3 = v[3];
    if (hh * g.hd < g.rot_cols) {
      const float2 a = g.rope[(size_t)row * half + j];
      const float2 b = g.rope[(size_t)row * half + j + 1];
      y0 = v[0] * a.x - v[2] * a.y;
      y2 = v[2] * a.x + v[0] * a.y;
      y1 = v[1] * b.x - v[3] * b.y;
      y3 = v[3] * b.x + v[1] * b.y;
    }
    const int L = g.lens ? g.lens[0] : 0;
    if (hh < g.H) {
      bf16* o = (bf16*)g.out + (size_t)row * g.ldo + hh * g.hd + j;
      *(unsigned*)o = pack2(y0, y1);
      *(unsigned*)(o + half) = pack2(y2, y3);
    } else if (hh < g.H + g.KVH) {
      bf16* o = (bf16*)g.kj + (size_t)(L + row) * (g.KVH * g.hd) + (hh - g.H) * g.hd + j;
      *(unsigned*)o = pack2(y0, y1);
      *(unsigned*)(o + half) = pack2(y2, y3);
    } else {
      const int kvh = hh - g.H - g.KVH, t = L + row;
      bf16* vt = (bf16*)g.vt;
      vt[vt_index(kvh, g.nj, t, j, tph)] = (bf16)y0;
      vt[vt_index(kvh, g.nj, t, j + 1, tph)] = (bf16)y1;
      vt[vt_index(kvh, g.nj, t, j + half, tph)] = (bf16)y2;
      vt[vt_index(kvh, g.nj, t, j + half + 1, tph)] = (bf16)y3;
    }
  } else if constexpr (EPI == EP_QKV_CACHE) {
    // tile order of a head of hd dims: dims j, j + 1, j + hd/2, j + hd/2 + 1, j = 8 (nt % (hd/16)) + 2 gq
    const int tph = g.hd >> 4, half = g.hd >> 1;
    const int hh = nt / tph, j = 8 * (nt - hh * tph) + 2 * gq;
    float y0 = v[0], y1 = v[1], y2 = v[2], y3 = v[3];
    if (hh < g.H + g.KVH) {
      const float2 a = g.rope[(size_t)row * half + j];
      const float2 b = g.rope[(size_t)row * half + j + 1];
      y0 = v[0] * a.x - v[2] * a.y;
      y2 = v[2] * a.x + v[0] * a.y;
      y1 = v[1] * b.x - v[3] * b.y;
      y3 = v[3] * b.x + v[1] * b.y;
    }
    const int req = row / g.req_rows, i = row - req * g.req_rows;
    if (hh < g.H) {
      bf16* o = (bf16*)g.out + (size_t)row * g.ldo + hh * g.hd + j;
      *(unsigned*)o = pack2(y0, y1);
      *(unsigned*)(o + half) = pack2(y2, y3);
    } else {
      const int slot = g.lens[req] + i;
      if (hh < g.H + g.KVH) {
        bf16* k = (bf16*)g.kc + (((size_t)req * g.KVH + (hh - g.H)) * g.Ctot + slot) * g.hd + j;
        *(unsigned*)k = pack2(y0, y1);
        *(unsigned*)(k + half) = pack2(y2, y3);
      } else {
        bf16* vt = (bf16*)g.vtc + ((size_t)req * g.KVH + (hh - g.H - g.KVH)) * g.hd * g.Ctot + slot;
        vt[(size_t)j * g.Ctot] = (bf16)y0;
        vt[(size_t)(j + 1) * g.Ctot] = (bf16)y1;
        vt[(size_t)(j + half) * g.Ctot] = (bf16)y2;
        vt[(size_t)(j + half + 1) * g.Ctot] = (bf16)y3;
      }
    }
  } else if constexpr (EPI == EP_GEGLU) {
    // features 8 nt + 2 gq + {0, 1}: gate in v[0], v[1], up in v[2], v[3]
    const int f = 8 * nt + 2 * gq;
    const float a0 = gelu_tanh(v[0]) * v[2], a1 = gelu_tanh(v[1]) * v[3];
    if (g.osplit)
      store_pair2((bf16*)g.out + (size_t)row * g.ldo, f, a0, a1);
    else
      *(unsigned*)((bf16*)g.out + (size_t)row * g.ldo + f) = pack2(a0, a1);
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

// PAIR: paired activation rows (wsh = 1).  A stage then holds only its
// k-step's activation fragments; the weight fragments of k-step pair p (hi
// 2 p, lo 2 p + 1) arrive once, with stage 2 p, in weight buffer p mod WB,
// and both stages multiply them.  Stage 2 p is issued NS - 1 stages ahead,
// when the pairs p - NS / 2 .. p - 1 are still to be read: WB = NS / 2 + 1.
template <int WN, int WM>
struct PairRing {
  static constexpr int NS = PAIR_STAGES;
  static constexpr int WB = NS / 2 + 1;                 // weight buffers
  static constexpr int ACT = NS * WM;                   // activation fragments of the NS stages
  static constexpr int LDS = (ACT + WB * 4 * WN) * 1024;
  static_assert(NS % 2 == 0 && LDS <= 160 * 1024, "stages in pairs, within one workgroup's LDS");
};
// waits until stage s of a pair ring is in: of the a = min(ahead, A) stages
// issued after it, at least a PA activation loads and a / 2 weight groups of
// WN loads may stay in flight (exactly that many when a = A, A even)
template <int PA, int WN, int A>
__device__ inline void wait_pair(int ahead) {
  if constexpr (A <= 0) {
    wait_vm<0>();
  } else {
    if (ahead >= A) wait_vm<A * PA + (A / 2) * WN>();
    else wait_pair<PA, WN, A - 1>(ahead);
  }
}
template <int WN, int WM, int EPI, bool PAIR>
__global__ __launch_bounds__(256) void k_tgemm_ring(GemmT g) {
  using T = Tile<WN, WM>;
  using P = PairRing<WN, WM>;
  constexpr int KS = 1;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int bx, by, bz;
  tile_of(blockIdx.x, g.N / T::BN, g.Mp / T::BM, g.splits, bx, by, bz);
  const int nt0 = (bx * 4 + wave) * WN;
  const int m0 = by * T::BM;
  const int KT = g.K / 32;
  const int per = KT / g.splits;
  const int kb = bz * per;
  const int ns = per / KS;  // stages
  constexpr int NS = T::NS;
  const unsigned lds0 = (unsigned)(unsigned long long)((__attribute__((address_space(3))) unsigned char*)smem);
  const u32x4 ra = rsrc_words(g.a, (unsigned)((size_t)g.Mp * g.K * 2));
  const u32x4 rw = rsrc_words(g.w, (unsigned)(((size_t)g.K >> g.wsh) * g.N * 2));
  const int KTW = KT >> g.wsh;  // weight k-tiles (activation k-step s meets weight k-tile s >> wsh)
  // this wave's activation fragments: m-tiles wave * WM/4 + i; lane: row 16 m + lane % 16, k chunk lane / 16
  unsigned voa[WM / 4];
#pragma unroll
  for (int i = 0; i < WM / 4; ++i) {
    const int m = wave * (WM / 4) + i;
    voa[i] = (unsigned)(((size_t)(m0 + 16 * m + (lane & 15)) * g.K + 8 * (lane >> 4)) * 2);
  }
  const unsigned vow = (unsigned)lane * 16u;
  auto issue_pair = [&](int s) {
    const int kt = kb + s;
    const unsigned st = lds0 + (unsigned)((s % P::NS) * WM * 1024);
#pragma unroll
    for (int i = 0; i < WM / 4; ++i)
      dma_frag(st + (unsigned)((wave * (WM / 4) + i) * 1024), voa[i], ra, (unsigned)(kt * 64));
    if ((s & 1) == 0) {
      const unsigned sw = lds0 + (unsigned)((P::ACT + ((s >> 1) % P::WB) * 4 * WN) * 1024);
#pragma unroll
      for (int n = 0; n < WN; ++n)
        dma_frag(sw + (unsigned)((wave * WN + n) * 1024), vow, rw, (unsigned)(((size_t)(nt0 + n) * KTW + (kt >> 1)) * 1024));
    }
  };
  auto issue = [&](int s) {
    if constexpr (PAIR) {
      issue_pair(s);
      return;
    }
    const unsigned st = lds0 + (unsigned)((s % NS) * T::STAGE);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int kt = kb + s * KS + kk;
      const unsigned sk = st + (unsigned)(kk * T::FR * 1024);
#pragma unroll
      for (int i = 0; i < WM / 4; ++i)
        dma_frag(sk + (unsigned)((wave * (WM / 4) + i) * 1024), voa[i], ra, (unsigned)(kt * 64));
#pragma unroll
      for (int n = 0; n < WN; ++n)
        dma_frag(sk + (unsigned)((WM + wave * WN + n) * 1024), vow, rw,
                 (unsigned)(((size_t)(nt0 + n) * KTW + (kt >> g.wsh)) * 1024));
    }
  };
  f32x4 acc[WN][WM];
#pragma unroll
  for (int n = 0; n < WN; ++n)
#pragma unroll
    for (int m = 0; m < WM; ++m) acc[n][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int NI = PAIR ? P::NS : NS;  // stages of the ring
#pragma unroll
  for (int s = 0; s < NI - 1; ++s)
    if (s < ns) issue(s);
  for (int s = 0; s < ns; ++s) {
    // stage s must be in; the later stages already issued may still be in flight
    if constexpr (PAIR) {
      static_assert(P::NS * (WM / 4) + P::NS / 2 * WN <= 63, "vmcnt holds at most 63 loads");
      wait_pair<WM / 4, WN, P::NS - 2>(ns - 1 - s);
      wg_barrier();
      if (s + P::NS - 1 < ns) issue(s + P::NS - 1);
      const unsigned char* st = smem + (s % P::NS) * WM * 1024;
      const unsigned char* sw = smem + (P::ACT + ((s >> 1) % P::WB) * 4 * WN) * 1024;
      bf16x8 wf[WN];
#pragma unroll
      for (int n = 0; n < WN; ++n) wf[n] = *(const bf16x8*)(sw + (wave * WN + n) * 1024 + lane * 16);
#pragma unroll
      for (int m = 0; m < WM; ++m) {
        const bf16x8 af = *(const bf16x8*)(st + m * 1024 + lane * 16);
#pragma unroll
        for (int n = 0; n < WN; ++n) acc[n][m] = mma32(wf[n], af, acc[n][m]);
      }
      continue;
    }
    wait_ahead<KS * T::PW, NS - 2>(ns - 1 - s);
    wg_barrier();  // stage s is in LDS for every wave; every wave is done with stage s - 1
    if (s + NS - 1 < ns) issue(s + NS - 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const unsigned char* st = smem + (s % NS) * T::STAGE + kk * T::FR * 1024;
      bf16x8 wf[WN];
#pragma unroll
      for (int n = 0; n < WN; ++n) wf[n] = *(const bf16x8*)(st + (WM + wave * WN + n) * 1024 + lane * 16);
#pragma unroll
      for (int m = 0; m < WM; ++m) {
        const bf16x8 af = *(const bf16x8*)(st + m * 1024 + lane * 16);
#pragma unroll
        for (int n = 0; n < WN; ++n) acc[n][m] = mma32(wf[n], af, acc[n][m]);
      }
    }
  }
  // lane holds columns 4 (lane / 16) + [0, 4) of each n-tile (tile order) for
  // row lane % 16 of each m-tile
  const int gq = lane >> 4;
#pragma unroll
  for (int m = 0; m < WM; ++m) {
    const int row = m0 + 16 * m + (lane & 15);
    if (row >= g.M) continue;
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      if (g.splits > 1)
        *(f32x4*)(g.part + ((size_t)bz * g.Mp + row) * g.N + (nt0 + n) * 16 + 4 * gq) = acc[n][m];
      else
        epi_store<EPI>(g, row, nt0 + n, gq, acc[n][m]);
    }
  }
}

// PAIR: paired activation rows (wsh = 1): k-steps 2 i (hi) and 2 i + 1 (lo)
// meet the same weight fragment, which is loaded once and kept for both.
template <int WN, int WM, int EPI, bool PAIR>
__global__ __launch_bounds__(256, 2) void k_tgemm_reg(GemmT g) {
  using T = Tile<WN, WM>;
  __shared__ u32x4 as[2][WM * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
  int bx, by, bz;
  tile_of(blockIdx.x, g.N / T::BN, g.Mp / T::BM, g.splits, bx, by, bz);
  const int nt0 = (bx * 4 + wave) * WN;
  const int m0 = by * T::BM;
  const int KT = g.K / 32;
  const int per = KT / g.splits;
  const int kb = bz * per;
  // Buffer loads with a fixed per-lane offset and a per-k-step scalar offset:
  // no address arithmetic in the loop, so no register of an in-flight load is
  // reused for an address (which would force a wait for every load).
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.a), (short)0, (int)((size_t)g.Mp * g.K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(g.w), (short)0, (int)(((size_t)g.K >> g.wsh) * g.N * 2), 0x00020000);
  const int wsh = PAIR ? 1 : __builtin_amdgcn_readfirstlane(g.wsh);
  // activation pieces of this thread: rows p*64 + tid/4, k chunk tid%4.  In
  // LDS, the 16-byte piece (row r of an m-tile, chunk c) sits at slot
  // 16 c + ((r + 4 c) mod 16) of the tile's 64: the four chunks of one row,
  // which four neighbouring threads store together, fall in different banks
  // (unrotated, 256 bytes apart, they shared one), and a lane's MFMA fragment
  // (row lane mod 16, chunk lane / 16) reads back as before.
  int avo[T::AP], aslot[T::AP];
#pragma unroll
  for (int p = 0; p < T::AP; ++p) {
    const int r = p * 64 + (tid >> 2), c = tid & 3;
    avo[p] = (int)(((size_t)(m0 + r) * g.K + 8 * c) * 2);
    aslot[p] = (r >> 4) * 64 + 16 * c + (((r & 15) + 4 * c) & 15);
  }
  const int fslot = 16 * (lane >> 4) + (((lane & 15) + 4 * (lane >> 4)) & 15);
  const int wvo = lane * 16;
  // weight k-tile of activation k-step kb + s is (kb + s) >> wsh (paired activation rows: each weight
  // fragment meets the hi and then the lo k-step; kb and the unrolled k-step groups are even)
  int wso[WN];
#pragma unroll
  for (int n = 0; n < WN; ++n) wso[n] = (int)((size_t)(nt0 + n) * (KT >> wsh) * 1024);
  auto ld_a = [&](int p, int s) -> u32x4 {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, avo[p], (kb + s) * 64, 0));
  };
  auto ld_w = [&](int n, int s) -> u32x4 {
    return __builtin_bit_cast(u32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(rw, wvo, wso[n] + ((kb + s) >> wsh) * 1024, 0));
  };
  f32x4 acc[WN][WM];
#pragma unroll
  for (int n = 0; n < WN; ++n)
#pragma unroll
    for (int m = 0; m < WM; ++m) acc[n][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int WS = PAIR ? UNR / 2 : UNR;
  // weight fragments: k-step s in slot s % UNR, or (PAIR) k-step pair s / 2 in slot (s / 2) % (UNR / 2)
  u32x4 wr[WS][WN];
  auto wslot = [](int j) { return PAIR ? (j / 2) % (UNR / 2) : j % UNR; };
  u32x4 ar[2][T::AP];   // activation pieces, k-step s in slot s % 2
  // prologue: activations of k-steps 0 and 1, weights of k-steps 0 .. WPD-1
#pragma unroll
  for (int p = 0; p < T::AP; ++p) ar[0][p] = ld_a(p, 0);
  if (per > 1) {
#pragma unroll
    for (int p = 0; p < T::AP; ++p) ar[1][p] = ld_a(p, 1);
  }
#pragma unroll
  for (int j = 0; j < WPD; ++j)
    if (j < per && (!PAIR || (j & 1) == 0)) {
#pragma unroll
      for (int n = 0; n < WN; ++n) wr[wslot(j)][n] = ld_w(n, j);
    }
#pragma unroll
  for (int p = 0; p < T::AP; ++p) as[0][aslot[p]] = ar[0][p];
  __syncthreads();
  // one k-step: fetch ahead, stage the next activations, multiply, barrier
  auto step = [&](int s, int j, bool fetch, bool stage) {
    if (fetch) {
      // activations of s + 2 (into the slot k-step s has left), weights of s + WPD
#pragma unroll
      for (int p = 0; p < T::AP; ++p) ar[j & 1][p] = ld_a(p, s + 2);
      if (!PAIR || ((j + WPD) & 1) == 0) {
#pragma unroll
        for (int n = 0; n < WN; ++n) wr[wslot(j + WPD)][n] = ld_w(n, s + WPD);
      }
    }
    if (stage) {
#pragma unroll
      for (int p = 0; p < T::AP; ++p) as[(j + 1) & 1][aslot[p]] = ar[(j + 1) & 1][p];
    }
    const u32x4* st = as[j & 1];
#pragma unroll
    for (int m = 0; m < WM; ++m) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, st[m * 64 + fslot]);
#pragma unroll
      for (int n = 0; n < WN; ++n) acc[n][m] = mma32(__builtin_bit_cast(bf16x8, wr[wslot(j)][n]), af, acc[n][m]);
    }
    __syncthreads();
  };
  // The steady loop has no conditions (per is a multiple of UNR), so the
  // compiler's waits can count the loads in flight exactly; the last UNR
  // k-steps fetch and stage only what remains.
  int s0 = 0;
  for (; s0 + UNR < per; s0 += UNR) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) step(s0 + j, j, true, true);
  }
#pragma unroll
  for (int j = 0; j < UNR; ++j) step(s0 + j, j, j + 2 < UNR && j + WPD < UNR, j + 1 < UNR);
  // lane holds columns 4 (lane / 16) + [0, 4) of each n-tile (tile order) for
  // row lane % 16 of each m-tile
  const int gq = lane >> 4;
#pragma unroll
  for (int m = 0; m < WM; ++m) {
    const int row = m0 + 16 * m + (lane & 15);
    if (row >= g.M) continue;
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      if (g.splits > 1)
        *(f32x4*)(g.part + ((size_t)bz * g.Mp + row) * g.N + (nt0 + n) * 16 + 4 * gq) = acc[n][m];
      else
        epi_store<EPI>(g, row, nt0 + n, gq, acc[n][m]);
    }
  }
}

// sums the split partials in split order, then the epilogue
template <int EPI>
__global__ void k_tsplit(GemmT g) {
  const int groups = g.N / 4;
  const size_t total = (size_t)g.M * groups;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(i / groups), c = (int)(i % groups) * 4;
    f32x4 v = *(const f32x4*)(g.part + (size_t)row * g.N + c);
    for (int z = 1; z < g.splits; ++z) v += *(const f32x4*)(g.part + ((size_t)z * g.Mp + row) * g.N + c);
    epi_store<EPI>(g, row, c >> 4, (c & 15) >> 2, v);
  }
}

// The split reduction of a residual GEMM fused with the row norm that
// follows it (the next GEMM's bf16 input rows), one workgroup per row.
// Thread t owns the 4-column groups t, t + 256, ... of the row: it loads
// every split's partials of its groups at once (16-byte loads), sums them
// in split order and adds them into the residual row (times the gate, if
// any), as k_tsplit does; then the workgroup normalises the new row as
// k_tnorm does (sums over the thread's columns in order, the same reduction
// tree).  Rows M..Mp-1 get zero norm rows.
constexpr int RN_GROUPS = 4;  // 4-column groups per thread: N <= 256 * 16
constexpr int RN_SPLITS = 8;  // splits whose loads go out together
__global__ __launch_bounds__(256) void k_tsplit_resid_norm(GemmT g) {
  __shared__ float red[8];
  const int row = blockIdx.x, t = threadIdx.x;
  const int N = g.N;
  const int W = g.nrm_split ? 2 * N : N;  // bf16 elements of a norm row
  bf16* o = (bf16*)g.nrm_out + (size_t)row * W;
  if (row >= g.M) {
    for (int d = t; d < W; d += 256) o[d] = (bf16)0.0f;
    return;
  }
  float* hr = (float*)g.out + (size_t)row * g.ldo;
  f32x4 v[RN_GROUPS];
#pragma unroll
  for (int q = 0; q < RN_GROUPS; ++q) v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < g.splits; z0 += RN_SPLITS) {
    f32x4 pz[RN_SPLITS][RN_GROUPS];
#pragma unroll
    for (int u = 0; u < RN_SPLITS; ++u)
#pragma unroll
      for (int q = 0; q < RN_GROUPS; ++q) {
        const int c = 4 * (t + 256 * q);
        if (z0 + u < g.splits && c < N) pz[u][q] = *(const f32x4*)(g.part + ((size_t)(z0 + u) * g.Mp + row) * N + c);
      }
#pragma unroll
    for (int u = 0; u < RN_SPLITS; ++u)
#pragma unroll
      for (int q = 0; q < RN_GROUPS; ++q)
        if (z0 + u < g.splits && 4 * (t + 256 * q) < N) v[q] += pz[u][q];
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < RN_GROUPS; ++q) {
    const int c = 4 * (t + 256 * q);
    if (c < N) {
      f32x4 cur = *(const f32x4*)(hr + c);
      if (g.gate)
        cur += *(const f32x4*)(g.gate + c) * v[q];
      else
        cur += v[q];
      *(f32x4*)(hr + c) = cur;
      v[q] = cur;
    } else {
      v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    s += (v[q][0] + v[q][1]) + (v[q][2] + v[q][3]);
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
  if (g.nrm_kind == 1) mean = block_sum(s) / (float)N;
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < RN_GROUPS; ++q) {
    if (4 * (t + 256 * q) < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float cdev = v[q][i] - mean;
        ss += cdev * cdev;
      }
    }
  }
  const float inv = 1.0f / sqrtf(block_sum(ss) / (float)N + g.nrm_eps);
#pragma unroll
  for (int q = 0; q < RN_GROUPS; ++q) {
    const int c = 4 * (t + 256 * q);
    if (c < N) {
      const f32x4 sc = *(const f32x4*)(g.nrm_scale + c), sh = *(const f32x4*)(g.nrm_shift + c);
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = (v[q][i] - mean) * inv * (1.0f + sc[i]) + sh[i];
      if (g.nrm_split)
        store_pair4(o, c, y);
      else
        *(u32x2*)(o + c) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
    }
  }
}

struct TileCfg {
  int wn, wm;
};
constexpr TileCfg TILES[] = {{4, 8}, {2, 8}, {2, 4}, {1, 4}, {2, 16}, {1, 16}};
constexpr int N_TILES = sizeof(TILES) / sizeof(TILES[0]);

void plan_gemm(GemmT& g, int n_cu) {
  const int KT = g.K / 32;
  // few rows: the weights stream once from HBM and the ring's deeper look-ahead wins; many rows: the
  // register-fed kernel halves the LDS traffic per MFMA (from 512 rows on for the long GEMMs, measured on
  // the 800-row prefill: gate/up 178 -> 123 us, while its 9-GFLOP QKV stayed faster on the ring)
  g.kern = (g.Mp >= 1024 || (g.Mp >= 512 && 2.0 * g.Mp * g.N * g.K >= 2e10)) ? 1 : 0;
  double best = 1e300;
  g.tile = -1;
  g.splits = 1;
  for (int i = 0; i < N_TILES; ++i) {
    const int bn = 64 * TILES[i].wn, bm = 16 * TILES[i].wm;
    if (g.N % bn || g.Mp % bm) continue;
    const long long wgs = (long long)(g.N / bn) * (g.Mp / bm);
    int sp = 1;
    while (wgs * sp < n_cu && KT % (2 * sp * UNR) == 0 && KT / (2 * sp) >= 8) sp *= 2;
    // time estimate: HBM bytes (weights once, split partials written and read), bytes pulled into
    // the CUs (every row block re-reads its weight columns, every column block its rows), MFMA
    // work, each scaled by how evenly the workgroups fill the chip
    const double hbm = 2.0 * g.K * g.N + (sp > 1 ? 8.0 * sp * g.Mp * g.N : 0.0);
    const double pulled = 2.0 * g.K * ((double)g.N * (g.Mp / bm) + (double)g.Mp * (g.N / bn));
    const double flops = 2.0 * g.Mp * g.N * g.K;
    const double units = (double)wgs * sp, rounds = std::ceil(units / n_cu);
    double t = std::max(std::max(hbm / 5e12, pulled / (n_cu * 100e9)), flops / 1.6e15) * rounds * n_cu / units;
    // the register-fed kernel is LDS-bound: the widest tile (most MFMAs per fragment read) measured fastest
    if (g.kern == 1 && i == 0) t *= 0.5;
    if (t < best * 0.97) {
      best = t;
      g.tile = i;
      g.splits = sp;
    }
  }
}

const char* tile_name(int tile) {
  static const char* names[N_TILES] = {"256x128", "128x128", "128x64", "64x64", "128x256", "64x256"};
  return tile >= 0 && tile < N_TILES ? names[tile] : "?";
}

size_t gemm_part_elems(const GemmT& g) { return g.splits > 1 ? (size_t)g.splits * g.Mp * g.N : 0; }

template <int WN, int WM, int EPI>
hipError_t allow_lds() {
  hipError_t e = hipFuncSetAttribute((const void*)k_tgemm_ring<WN, WM, EPI, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, Tile<WN, WM>::LDS);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)k_tgemm_ring<WN, WM, EPI, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             PairRing<WN, WM>::LDS);
}

template <int EPI>
hipError_t allow_lds_e() {
  hipError_t e;
  if ((e = allow_lds<4, 8, EPI>()) != hipSuccess) return e;
  if ((e = allow_lds<2, 8, EPI>()) != hipSuccess) return e;
  if ((e = allow_lds<2, 4, EPI>()) != hipSuccess) return e;
  if ((e = allow_lds<1, 4, EPI>()) != hipSuccess) return e;
  if ((e = allow_lds<2, 16, EPI>()) != hipSuccess) return e;
  return allow_lds<1, 16, EPI>();
}

hipError_t prepare_gemm() {
  hipError_t e;
  if ((e = allow_lds_e<EP_BF16>()) != hipSuccess) return e;
  if ((e = allow_lds_e<EP_QKV>()) != hipSuccess) return e;
  if ((e = allow_lds_e<EP_GEGLU>()) != hipSuccess) return e;
  if ((e = allow_lds_e<EP_GELU>()) != hipSuccess) return e;
  if ((e = allow_lds_e<EP_RESID>()) != hipSuccess) return e;
  if ((e = allow_lds_e<EP_EULER>()) != hipSuccess) return e;
  if ((e = allow_lds_e<EP_QKV_CACHE>()) != hipSuccess) return e;
  return allow_lds_e<EP_F32>();
}

template <int WN, int WM, int EPI>
hipError_t launch_tile(const GemmT& g, hipStream_t s) {
  using T = Tile<WN, WM>;
  if (g.N % T::BN || g.Mp % T::BM) return hipErrorInvalidValue;  // the grid covers whole tiles only
  const dim3 grid((g.N / T::BN) * (g.Mp / T::BM) * g.splits);
  constexpr int PAIR_LDS = PairRing<WN, WM>::LDS;
  if (g.kern == 0 && g.wsh)
    hipLaunchKernelGGL((k_tgemm_ring<WN, WM, EPI, true>), grid, dim3(256), PAIR_LDS, s, g);
  else if (g.kern == 0)
    hipLaunchKernelGGL((k_tgemm_ring<WN, WM, EPI, false>), grid, dim3(256), T::LDS, s, g);
  else if (g.wsh)
    hipLaunchKernelGGL((k_tgemm_reg<WN, WM, EPI, true>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((k_tgemm_reg<WN, WM, EPI, false>), grid, dim3(256), 0, s, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.splits == 1) return e;
  if (g.nrm_on) {
    hipLaunchKernelGGL(k_tsplit_resid_norm, dim3(g.Mp), dim3(256), 0, s, g);
    return hipGetLastError();
  }
  const size_t total = (size_t)g.M * (g.N / 4);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(k_tsplit<EPI>, dim3(blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_tgemm_e(const GemmT& g, hipStream_t s) {
  switch (g.tile) {
    case 0: return launch_tile<4, 8, EPI>(g, s);
    case 1: return launch_tile<2, 8, EPI>(g, s);
    case 2: return launch_tile<2, 4, EPI>(g, s);
    case 3: return launch_tile<1, 4, EPI>(g, s);
    case 4: return launch_tile<2, 16, EPI>(g, s);
    case 5: return launch_tile<1, 16, EPI>(g, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tgemm(int epi, const GemmT& g, hipStream_t s) {
  if (g.K % 32 || g.N % 64 || g.Mp % ROW_PAD || g.M > g.Mp || g.tile < 0 || g.tile >= N_TILES) return hipErrorInvalidValue;
  if (g.splits < 1 || (g.K / 32) % (g.splits * UNR) || (g.splits > 1 && !g.part)) return hipErrorInvalidValue;
  if (g.nrm_on && (epi != EP_RESID || g.splits < 2 || g.N > 256 * 4 * RN_GROUPS || g.N % 4 || g.ldo != g.N || !g.nrm_out || !g.nrm_scale ||
                   !g.nrm_shift || (g.nrm_kind != 0 && g.nrm_kind != 1)))
    return hipErrorInvalidValue;
  if ((size_t)g.Mp * g.K * 2 >= (1ull << 32) || (size_t)g.K * g.N * 2 >= (1ull << 32)) return hipErrorInvalidValue;
  // paired activations: every k split holds whole (hi, lo) k-step pairs
  if (g.wsh != 0 && (g.wsh != 1 || ((g.K / 32) / g.splits) % 2)) return hipErrorInvalidValue;
  if (g.osplit && (epi != EP_GELU && epi != EP_GEGLU)) return hipErrorInvalidValue;
  if (g.nrm_on && g.nrm_split && g.N % 32) return hipErrorInvalidValue;
  switch (epi) {
    case EP_BF16: return launch_tgemm_e<EP_BF16>(g, s);
    case EP_QKV: return launch_tgemm_e<EP_QKV>(g, s);
    case EP_GEGLU: return launch_tgemm_e<EP_GEGLU>(g, s);
    case EP_GELU: return launch_tgemm_e<EP_GELU>(g, s);
    case EP_RESID: return launch_tgemm_e<EP_RESID>(g, s);
    case EP_EULER: return launch_tgemm_e<EP_EULER>(g, s);
    case EP_F32: return launch_tgemm_e<EP_F32>(g, s);
    case EP_QKV_CACHE: return launch_tgemm_e<EP_QKV_CACHE>(g, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------ row norms

// one workgroup per row; D <= 256 * 16
__global__ __launch_bounds__(256) void k_tnorm(int kind, const float* __restrict__ h, const float* __restrict__ scale,
                                               const float* __restrict__ shift, float eps, bf16* __restrict__ out,
                                               int M, int D, int split) {
  // thread t owns the 4-column groups t, t + 256, t + 512, t + 768 of its row (16-byte loads), the same
  // columns and sums as the norm fused into the split reduction (k_tsplit_resid_norm)
  constexpr int GR = 4;
  __shared__ float red[8];
  const int row = blockIdx.x, t = threadIdx.x;
  const int W = split ? 2 * D : D;  // bf16 elements of an output row
  bf16* o = out + (size_t)row * W;
  if (row >= M) {
    for (int d = t; d < W; d += 256) o[d] = (bf16)0.0f;
    return;
  }
  const float* x = h + (size_t)row * D;
  f32x4 v[GR];
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < GR; ++q) {
    const int c = 4 * (t + 256 * q);
    v[q] = c < D ? *(const f32x4*)(x + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    s += (v[q][0] + v[q][1]) + (v[q][2] + v[q][3]);
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
  for (int q = 0; q < GR; ++q) {
    if (4 * (t + 256 * q) < D) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float cdev = v[q][i] - mean;
        ss += cdev * cdev;
      }
    }
  }
  const float inv = 1.0f / sqrtf(block_sum(ss) / (float)D + eps);
#pragma unroll
  for (int q = 0; q < GR; ++q) {
    const int c = 4 * (t + 256 * q);
    if (c < D) {
      const f32x4 sc = *(const f32x4*)(scale + c), sh = *(const f32x4*)(shift + c);
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = (v[q][i] - mean) * inv * (1.0f + sc[i]) + sh[i];
      if (split)
        store_pair4(o, c, y);
      else
        *(u32x2*)(o + c) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
    }
  }
}

hipError_t launch_tnorm(int kind, const float* h, const float* scale, const float* shift, float eps, void* out, int M,
                        int Mp, int D, int split, hipStream_t s) {
  if (D > 256 * 16 || D % 4 || M > Mp || (split && D % 32)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tnorm, dim3(Mp), dim3(256), 0, s, kind, h, scale, shift, eps, (bf16*)out, M, D, split);
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
// Workgroup (128 queries, head h, key split); wave w owns queries 32 w as two
// 16-query tiles.  Keys are the L prefix rows followed by the M chunk rows,
// read from the joint key rows and the fragment-ordered values (see
// vt_index); a split takes a contiguous range of 64-key blocks.  With the
// causal mask chunk row q sees the prefix and chunk rows up to itself.  Per
// block:
//   S^T = K . Q^T with 16x16x32 MFMAs: K fragments (lane: key lane % 16, dims
//     8 (lane / 16) + [0, 8) of a 32-dim step) come from LDS, the wave's
//     queries sit in registers as B fragments, so each lane ends with keys
//     4 (lane / 16) + [0, 4) of each 16-key tile for one query;
//   online softmax per query in base 2 (the four lanes of a query combine
//     with two shuffles);
//   O^T += V^T . P^T: two 16-key tiles of probabilities form the B fragment
//     of one 32-key step as they lie in the registers (k index 8 g + e is key
//     4 g + e for e < 4 and 16 + 4 g + e - 4 for e >= 4), and the value
//     fragments are stored in that same key order.
// K and V^T blocks (16 KiB each per 128 dims) stream into a two-stage LDS
// ring with direct loads, the next block in flight while the current one is
// used.  Workgroups of one head run on one XCD so its keys and values stay in
// that XCD's L2.
constexpr int KB = 64;     // keys per block
constexpr int AQ = 128;    // queries per workgroup (four waves)

constexpr int ASTAGE = 2;  // LDS stages

template <int HD>
struct AttnShape {
  static constexpr int NDS = HD / 32;               // 32-dim steps of S^T = K . Q^T
  static constexpr int NDT = HD / 16;               // 16-dim tiles of O^T
  static constexpr int KBYTES = 4 * NDS * 1024;     // K fragments of one block
  static constexpr int STAGE = 2 * KBYTES;          // K and V^T of one block
};

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) void k_tattn(AttnT a) {
  using S = AttnShape<HD>;
  constexpr int NDS = S::NDS, NDT = S::NDT;
  constexpr int QW = 32 * NW;                              // queries per workgroup
  constexpr int KF = 4 * NDS / NW, VF = 2 * NDT / NW;      // K and V^T fragments each wave moves per block
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nqb = (a.M + QW - 1) / QW;
  const int per_head = nqb * a.splits;
  const int bid = blockIdx.x;
  int h, r;
  if (a.H % 8 == 0) {
    const int i = bid >> 3;
    h = (bid & 7) + 8 * (i / per_head);
    r = i % per_head;
  } else {
    h = bid / per_head;
    r = bid % per_head;
  }
  const int qb = r / a.splits, split = r % a.splits;
  const int kvh = h / (a.H / a.KVH);
  const int kvd = a.KVH * HD;
  const int L = a.lens ? __builtin_amdgcn_readfirstlane(a.lens[0]) : 0;
  const int T = L + a.M;
  const int nblk = (T + KB - 1) / KB;
  const int per = (nblk + a.splits - 1) / a.splits;
  const int b0 = split * per;
  int b1 = min(nblk, b0 + per);
  if (a.causal) b1 = min(b1, (L + min(qb * QW + QW, a.M) - 1) / KB + 1);  // no key past the last query
  const int g4 = lane >> 4, qr = lane & 15;
  const int q0 = qb * QW + 32 * wave;
  // queries as B fragments of Q^T: dims 32 ds + 8 g4 + [0, 8) of query q0 + 16 qt + qr
  bf16x8 qf[2][NDS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = min(q0 + 16 * qt + qr, a.M - 1);
    const bf16* qp = (const bf16*)a.q + (size_t)q * a.ldq + h * HD + 8 * g4;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[qt][ds] = *(const bf16x8*)(qp + 32 * ds);
  }
  // Wait for the query loads here, once: left to the first use inside the
  // block loop, the compiler's wait would also cover the next block's LDS
  // loads issued just before it (it does not see those), every block.
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) asm volatile("" : "+v"(qf[qt][ds]));
  const unsigned lds0 = (unsigned)(unsigned long long)((__attribute__((address_space(3))) unsigned char*)smem);
  const u32x4 rk = rsrc_words(a.kj, (unsigned)((size_t)a.R * kvd * 2));
  const u32x4 rv = rsrc_words(a.vt, (unsigned)((size_t)a.KVH * a.R * HD * 2));
  // wave w moves K fragments KF w .. KF (w + 1) - 1 (fragment kt NDS + ds: key tile kt, dim step ds)
  // and value fragments VF w .. VF (w + 1) - 1
  unsigned vok[KF];
#pragma unroll
  for (int f = 0; f < KF; ++f) {
    const int kf = KF * wave + f, kt = kf / NDS, ds = kf % NDS;
    vok[f] = (unsigned)(((16 * kt + qr) * kvd + kvh * HD + 32 * ds + 8 * g4) * 2);
  }
  const unsigned vov = (unsigned)lane * 16u;
  const int nj = a.R / 32;
  auto issue = [&](int b) {
    const unsigned st = lds0 + (unsigned)((b % ASTAGE) * S::STAGE);
#pragma unroll
    for (int f = 0; f < KF; ++f)
      dma_frag(st + (unsigned)((KF * wave + f) * 1024), vok[f], rk, (unsigned)(b * KB * kvd * 2));
#pragma unroll
    for (int f = 0; f < VF; ++f)
      dma_frag(st + (unsigned)(S::KBYTES + (VF * wave + f) * 1024), vov, rv,
               (unsigned)((((size_t)kvh * nj + 2 * b) * NDT + VF * wave + f) * 1024));
  };
  const float sl2 = a.scale * 1.4426950408889634f;  // scores in base 2
  f32x4 oacc[2][NDT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int d = 0; d < NDT; ++d) oacc[qt][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  if (b0 < b1) issue(b0);
  for (int b = b0; b < b1; ++b) {
    wait_vm<0>();
    wg_barrier();  // block b is in LDS for every wave; every wave is done with block b - 1
    if (b + 1 < b1) issue(b + 1);
    const unsigned char* st = smem + (b % ASTAGE) * S::STAGE;
    f32x4 sc[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sc[0][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      sc[1][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 kf = *(const bf16x8*)(st + (kt * NDS + ds) * 1024 + lane * 16);
        sc[0][kt] = mma32(kf, qf[0][ds], sc[0][kt]);
        sc[1][kt] = mma32(kf, qf[1][ds], sc[1][kt]);
      }
    }
    const int k0 = b * KB;
    // keys at or past T exist only in the last block; causal keys past a query only near the diagonal
    const bool tail = k0 + KB > T;
    const bool diag = a.causal && k0 + KB - 1 > L + q0;
    if (tail || diag) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int lim = a.causal ? min(T - 1, L + q0 + 16 * qt + qr) : T - 1;  // last key this query sees
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + 16 * kt + 4 * g4 + i > lim) sc[qt][kt][i] = -INFINITY;
      }
    }
    // Lazy rescaling: the reference m (base 2) of a query moves only when some
    // score of the wave exceeds it by more than 8, so the probabilities stay
    // below 2^8 and most blocks neither reduce across lanes nor rescale O.
    // The four lanes of a query always share one m (their probabilities meet
    // in the same MFMA).  Per-lane partial sums l are reduced at the end.
    bf16x8 pf[2][2];
    float corr[2] = {1.f, 1.f};
    bool moved[2] = {false, false};
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[qt][kt][i]);
      mx *= sl2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run[qt] + 8.0f) != 0) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[qt], mx);
        // 0 on a query's first block (m_run = -inf); a query with no key yet keeps m = -inf
        corr[qt] = m_new == -INFINITY ? 1.f : hexp2(m_run[qt] - m_new);
        l_run[qt] *= corr[qt];
        m_run[qt] = m_new;
        moved[qt] = true;
      }
      const float mneg = m_run[qt] == -INFINITY ? 0.f : -m_run[qt];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = hexp2(fmaf(sc[qt][kt][i], sl2, mneg));
          l_run[qt] += p;
          pf[qt][kt >> 1][4 * (kt & 1) + i] = (bf16)p;
        }
    }
    if (moved[0] || moved[1]) {
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        oacc[0][d] *= corr[0];
        oacc[1][d] *= corr[1];
      }
    }
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
      f32x4 a0 = oacc[0][d], a1 = oacc[1][d];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 vf = *(const bf16x8*)(st + S::KBYTES + (j * NDT + d) * 1024 + lane * 16);
        a0 = mma32(vf, pf[0][j], a0);
        a1 = mma32(vf, pf[1][j], a1);
      }
      oacc[0][d] = a0;
      oacc[1][d] = a1;
    }
  }
  // lane holds dims 16 d + 4 g4 + [0, 4) of query q0 + 16 qt + qr
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    l_run[qt] += __shfl_xor(l_run[qt], 16);
    l_run[qt] += __shfl_xor(l_run[qt], 32);
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = q0 + 16 * qt + qr;
    if (q >= a.M) continue;
    if (a.splits == 1) {
      const float inv = 1.0f / l_run[qt];
      bf16* op = (bf16*)a.o + (size_t)q * (a.H * HD) + h * HD;
#pragma unroll
      for (int d = 0; d < NDT; ++d)
        *(u32x2*)(op + 16 * d + 4 * g4) = u32x2{pack2(oacc[qt][d][0] * inv, oacc[qt][d][1] * inv),
                                                pack2(oacc[qt][d][2] * inv, oacc[qt][d][3] * inv)};
    } else {
      float* po = a.po + ((size_t)split * a.M + q) * (a.H * HD) + h * HD;
#pragma unroll
      for (int d = 0; d < NDT; ++d) *(f32x4*)(po + 16 * d + 4 * g4) = oacc[qt][d];
      if (g4 == 0) {
        float* ml = a.pml + (((size_t)split * a.M + q) * a.H + h) * 2;
        ml[0] = m_run[qt];
        ml[1] = l_run[qt];
      }
    }
  }
}

template <int NW>
hipError_t prepare_attention_nw() {
  hipError_t e = hipFuncSetAttribute((const void*)k_tattn<128, NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     ASTAGE * AttnShape<128>::STAGE);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)k_tattn<256, NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             ASTAGE * AttnShape<256>::STAGE);
}
hipError_t prepare_attention() {
  const hipError_t e = prepare_attention_nw<4>();
  return e != hipSuccess ? e : prepare_attention_nw<8>();
}

// eight waves from 2048 queries on (the DiT-style step: 7.35 -> 7.20 ms); on the 256-row chunk the doubled
// key splits and their combine cost more than the halved block reads (5.33 -> 5.69 ms)
int attn_queries_per_wg(int M, int hd) { return M >= 2048 && hd == 128 ? 256 : AQ; }

hipError_t launch_tattn(const AttnT& a, hipStream_t s) {
  if (a.M < 1 || a.H % a.KVH || a.splits < 1 || a.R % KB || a.R < a.M) return hipErrorInvalidValue;
  if (a.hd != 128 && a.hd != 256) return hipErrorInvalidValue;
  if ((size_t)a.R * a.KVH * a.hd * 2 >= (1ull << 32)) return hipErrorInvalidValue;
  // many queries: eight waves (256 queries) share each key/value block in LDS, which halves the blocks'
  // reads from L2
  const int qw = attn_queries_per_wg(a.M, a.hd);
  const bool wide = qw == 256;
  const int blocks = ((a.M + qw - 1) / qw) * a.splits * a.H;
  if (a.hd == 128 && wide)
    hipLaunchKernelGGL((k_tattn<128, 8>), dim3(blocks), dim3(512), ASTAGE * AttnShape<128>::STAGE, s, a);
  else if (a.hd == 128)
    hipLaunchKernelGGL((k_tattn<128, 4>), dim3(blocks), dim3(256), ASTAGE * AttnShape<128>::STAGE, s, a);
  else if (wide)
    hipLaunchKernelGGL((k_tattn<256, 8>), dim3(blocks), dim3(512), ASTAGE * AttnShape<256>::STAGE, s, a);
  else
    hipLaunchKernelGGL((k_tattn<256, 4>), dim3(blocks), dim3(256), ASTAGE * AttnShape<256>::STAGE, s, a);
  return hipGetLastError();
}

// out[q][h*hd + d] = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s, splits in order; one thread per
// 8 dims of a query and head (two 16-byte partial loads per split, one 16-byte store)
__global__ void k_tcombine(AttnT a) {
  const int groups = a.hd / 8;
  const size_t total = (size_t)a.M * a.H * groups;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int g = (int)(i % groups);
    const size_t qh = i / groups;
    const int h = (int)(qh % a.H);
    const int q = (int)(qh / a.H);
    float m = -INFINITY;
    f32x4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    constexpr int ONE = 8;  // up to ONE splits: every statistic and partial in flight at once, one memory round
    if (a.splits <= ONE) {
      float2 ml[ONE];
      f32x4 p0[ONE], p1[ONE];
#pragma unroll
      for (int s = 0; s < ONE; ++s) {
        if (s < a.splits) {
          ml[s] = *(const float2*)(a.pml + (((size_t)s * a.M + q) * a.H + h) * 2);
          const float* po = a.po + ((size_t)s * a.M + q) * (a.H * a.hd) + h * a.hd + 8 * g;
          p0[s] = *(const f32x4*)po;
          p1[s] = *(const f32x4*)(po + 4);
        }
      }
#pragma unroll
      for (int s = 0; s < ONE; ++s)
        if (s < a.splits) m = fmaxf(m, ml[s].x);
#pragma unroll
      for (int s = 0; s < ONE; ++s) {
        if (s < a.splits && ml[s].x != -INFINITY) {  // a split with no key this query sees adds nothing
          const float w = hexp2(ml[s].x - m);
          n0 += w * p0[s];
          n1 += w * p1[s];
          den += w * ml[s].y;
        }
      }
    } else {
      for (int s = 0; s < a.splits; ++s) m = fmaxf(m, a.pml[(((size_t)s * a.M + q) * a.H + h) * 2]);
      for (int s = 0; s < a.splits; ++s) {
        const float2 ml = *(const float2*)(a.pml + (((size_t)s * a.M + q) * a.H + h) * 2);
        if (ml.x == -INFINITY) continue;  // a split with no key this query sees
        const float w = hexp2(ml.x - m);
        const float* po = a.po + ((size_t)s * a.M + q) * (a.H * a.hd) + h * a.hd + 8 * g;
        n0 += w * *(const f32x4*)po;
        n1 += w * *(const f32x4*)(po + 4);
        den += w * ml.y;
      }
    }
    *(u32x4*)((bf16*)a.o + (size_t)q * (a.H * a.hd) + h * a.hd + 8 * g) =
        u32x4{pack2(n0[0] / den, n0[1] / den), pack2(n0[2] / den, n0[3] / den), pack2(n1[0] / den, n1[1] / den),
              pack2(n1[2] / den, n1[3] / den)};
  }
}

hipError_t launch_tcombine(const AttnT& a, hipStream_t s) {
  if (a.hd % 8) return hipErrorInvalidValue;
  const size_t total = (size_t)a.M * a.H * (a.hd / 8);
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_tcombine, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Prefix values into the fragment order: keys t < L from v [NL][L][KVH*hd],
// zeros for L <= t < R.
__global__ void k_vt_load(const bf16* __restrict__ v, bf16* __restrict__ vt, int NL, int L, int R, int KVH, int hd) {
  const size_t plane = (size_t)R * hd;  // one kv head of one layer
  const size_t total = (size_t)NL * KVH * plane;
  const int kvd = KVH * hd, ndt = hd / 16;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t lp = i / plane;
    const int l = (int)(lp / KVH), kvh = (int)(lp % KVH);
    int t, d;
    vt_key_dim((int)(i % plane), ndt, t, d);
    vt[i] = t < L ? v[((size_t)l * L + t) * kvd + kvh * hd + d] : (bf16)0.0f;
  }
}

// Values in fragment order back to rows: v [NL][n][KVH*hd] from the keys t < n of vt.
__global__ void k_vt_export(const bf16* __restrict__ vt, bf16* __restrict__ v, int NL, int n, int R, int KVH,
                            int hd) {
  const int kvd = KVH * hd, ndt = hd / 16, nj = R / 32;
  const size_t plane = (size_t)R * hd;
  const size_t total = (size_t)NL * n * kvd;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % kvd);
    const size_t lt = i / kvd;
    const int t = (int)(lt % n), l = (int)(lt / n);
    const int kvh = c / hd, d = c % hd;
    v[i] = vt[((size_t)l * KVH + kvh) * plane + vt_index(0, nj, t, d, ndt)];
  }
}

// Values in fragment order moved down by d keys (the history window drops
// its d oldest rows): dst key t = src key t + d for t + d < n, zeros after.
__global__ void k_vt_shift(const bf16* __restrict__ src, bf16* __restrict__ dst, int NL, int KVH, int R, int d,
                           int n, int hd) {
  const size_t plane = (size_t)R * hd;
  const size_t total = (size_t)NL * KVH * plane;
  const int nj = R / 32, ndt = hd / 16;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t pb = i / plane * plane;
    int t, dd;
    vt_key_dim((int)(i - pb), ndt, t, dd);
    dst[i] = t + d < n ? src[pb + vt_index(0, nj, t + d, dd, ndt)] : (bf16)0.0f;
  }
}

static int grid_for(size_t total) { return (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535); }

hipError_t launch_vt_shift(const void* src, void* dst, int NL, int KVH, int R, int d, int n, int hd, hipStream_t s) {
  hipLaunchKernelGGL(k_vt_shift, dim3(grid_for((size_t)NL * KVH * R * hd)), dim3(256), 0, s, (const bf16*)src,
                     (bf16*)dst, NL, KVH, R, d, n, hd);
  return hipGetLastError();
}

hipError_t launch_vt_export(const void* vt, void* v, int NL, int n, int R, int KVH, int hd, hipStream_t s) {
  if (n < 1) return hipSuccess;
  hipLaunchKernelGGL(k_vt_export, dim3(grid_for((size_t)NL * n * KVH * hd)), dim3(256), 0, s, (const bf16*)vt,
                     (bf16*)v, NL, n, R, KVH, hd);
  return hipGetLastError();
}

// lens[0] = L; the rows' RoPE table at positions pos .. pos + M - 1 (angles in double)
__global__ void k_positions(int* lens, float2* rope, int L, int pos, int M, int hd, double base) {
  const int half = hd / 2;
  if (blockIdx.x == 0 && threadIdx.x == 0 && lens) lens[0] = L;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < M * half; idx += gridDim.x * blockDim.x) {
    const int i = idx / half, j = idx % half;
    const double theta = pow(base, -2.0 * (double)j / (double)hd);
    const double ang = (double)(pos + i) * theta;
    rope[idx] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

hipError_t launch_positions(int* lens, float2* rope, int L, int pos, int M, int hd, double base, hipStream_t s) {
  const int n = M * (hd / 2);
  hipLaunchKernelGGL(k_positions, dim3((n + 255) / 256), dim3(256), 0, s, lens, rope, L, pos, M, hd, base);
  return hipGetLastError();
}

hipError_t launch_vt_load(const void* v, void* vt, int NL, int L, int R, int KVH, int hd, hipStream_t s) {
  hipLaunchKernelGGL(k_vt_load, dim3(grid_for((size_t)NL * KVH * R * hd)), dim3(256), 0, s, (const bf16*)v,
                     (bf16*)vt, NL, L, R, KVH, hd);
  return hipGetLastError();
}

}  // namespace tok
}  // namespace phx
