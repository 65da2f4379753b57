// Persistent decision kernel for gfx950 (CDNA4): one launch runs all S Euler
// steps x NL layers of one request's action rows.
//
// Why persistent.  At 10 action rows every projection streams its weights
// once per step and does ~10 MACs per weight element, so a decision is bound
// by HBM bandwidth (6.37 GB per pi0.5 decision) and by the latency of the
// ~1300 dependent all-to-all exchanges between sublayers.  A graph of ~1100
// small kernels pays a node gap plus ramp-up and drain at every boundary; the
// pages remove those gaps with programmatic dependent launch and by folding
// the "kernels between GEMMs" into GEMM prologues and epilogues ("FlashRT-PAI",
// sections 3.2-3.3; "PhyAI" section 4.2 Kernel fusion, Graph replay).  Here the
// same two ideas take a form that fits MI355X:
//   * Loader waves (4 per workgroup) stream the workgroup's fixed share of
//     every weight matrix (and of the prefix K/V for attention workgroups)
//     into a 128-tile LDS ring, running up to a ring ahead of the compute, so
//     the HBM stream never waits for a sublayer boundary;
//   * compute waves (4 per workgroup) exchange activations with other
//     workgroups through tagged 8-byte words (payload | exchange tag) written
//     and read at device scope (sc1), so a consumer detects both readiness and
//     data with one load and no barrier or atomic counter is needed.
// Exchange tags grow with a per-handle decision counter, so buffers never
// need clearing between decisions.
//
// Fusions (the pages' "kernels between GEMMs"): the adaptive RMSNorm is split
// into the producer's epilogue (bf16(h * (1 + scale)) and per-block sums of
// squares) and the consumer's epilogue (row factor 1/rms and the shift term,
// added as the precomputed product shift . W); RoPE, GeGLU, residual adds and
// the Euler update are epilogues.  Reductions are in a fixed order, so
// replays are bit-identical.
//
// Every global access goes through a buffer resource whose range check turns
// a stray index into a dropped store or a zero load; every wait is bounded by
// a wall-clock limit and an abort flag, so a missing producer ends the launch
// with a status instead of a hang.
#include "phx_decide.h"
#include "phx_internal.h"

#include <hip/hip_runtime.h>
#include <math.h>

namespace phx {
namespace dec {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int AUX_SC1 = 16;  // device-coherent access

// LDS layout (static part; the ring is dynamic)
constexpr int RED_BYTES = NCOMPUTE * 4 * 64 * 16;  // per-wave partial tiles (also reused)

struct Shared {
  unsigned ready[NLOADER];   // tiles of each loader's sub-stream written to the ring
  unsigned consumed;         // ring positions below this are free
  unsigned abort;            // nonzero: leave now
  unsigned cwbar;            // compute-wave barrier counter
  unsigned pad[9];
  float rrow[RP];            // 1/rms per action row
  float att_m[NCOMPUTE][RP];
  float att_l[NCOMPUTE][RP];
  s16x4 att_p[NCOMPUTE][64];
  __attribute__((aligned(16))) unsigned char red[2][RED_BYTES];
};

__device__ inline Rsrc rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline unsigned now_ticks() { return (unsigned)__builtin_amdgcn_s_memrealtime(); }

// Bit casts through a by-value scalar: clang folds __builtin_bit_cast applied
// directly to an element of an ext_vector_type value to element 0.
__device__ inline float as_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ inline unsigned as_u(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ inline short as_s(bf16 b) { return __builtin_bit_cast(short, b); }

__device__ inline unsigned pack_bf16(float a, float b) {
  const unsigned short ua = __builtin_bit_cast(unsigned short, (bf16)a);
  const unsigned short ub = __builtin_bit_cast(unsigned short, (bf16)b);
  return (unsigned)ua | ((unsigned)ub << 16);
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

// ------------------------------------------------------------- context

struct Ctx {
  const Args* a;
  Role r;
  Shared* sh;
  unsigned char* ring;
  Rsrc W, KV, EX, AUX;
  unsigned tagbase;
  unsigned seq;            // this decision's counter
  unsigned redsel;         // which half of the partial-tile scratch the current phase uses
  int lane, wave, g, row;  // row = lane % 16, g = lane / 16
  int L;                   // prefix length
  unsigned barn;           // compute-wave barriers passed
  // stream layout of this workgroup
  unsigned n_in, n_layer, n_out, n_step, o_attn, o_o, o_gu, o_dn;
};

__device__ inline unsigned tag_of(const Ctx& c, int k, int l, int type) {
  return c.tagbase + (unsigned)((k * (c.a->NL + 1) + l) * NX + type) + 1u;
}
__device__ inline unsigned xoff(const Ctx& c, int k, int l, int type) {
  return ((k * (c.a->NL + 1) + l) & 1) ? c.a->ex_off[type][1] : c.a->ex_off[type][0];
}

__device__ inline bool aborted(Ctx& c) { return __hip_atomic_load(&c.sh->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u; }

// The status word names the failing decision (its counter + 1), so a failure
// needs no clearing before the next decision.
__device__ inline void fail(Ctx& c) {
  __hip_atomic_store(&c.sh->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (c.lane == 0) __builtin_amdgcn_raw_buffer_store_b32(c.seq + 1u, c.AUX, c.a->o_status, 0, AUX_SC1);
}

// polls the global status every so often; true means keep waiting
__device__ inline bool keep_waiting(Ctx& c, unsigned t0, unsigned& spins) {
  ++spins;
  if (aborted(c)) return false;
  if ((spins & 63u) == 0u) {
    if (now_ticks() - t0 > c.a->timeout_ticks) {
      fail(c);
      return false;
    }
    const unsigned st = __builtin_amdgcn_raw_buffer_load_b32(c.AUX, c.a->o_status, 0, AUX_SC1);
    if (st == c.seq + 1u) {
      __hip_atomic_store(&c.sh->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return false;
    }
  }
  return true;
}

// Loader waves keep up to two batches of tile loads in flight; a global load
// in their wait loop would make the next use of any loaded register wait for
// the whole batch (loads complete in order), so they only watch the LDS abort
// flag (set by their compute waves, which watch the global status) and the
// clock.
__device__ inline bool loader_keep_waiting(Ctx& c, unsigned t0, unsigned& spins) {
  ++spins;
  if (aborted(c)) return false;
  if ((spins & 63u) == 0u && now_ticks() - t0 > c.a->timeout_ticks) {
    __hip_atomic_store(&c.sh->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return false;
  }
  return true;
}

// Synchronisation inside a workgroup goes through LDS only.  The LDS unit
// performs each wave's operations in issue order, so a data write followed by
// a flag write is seen in that order by any wave that reads the flag first;
// the compiler barriers keep the compiler from reordering them.  (A
// workgroup-scope acquire/release would also wait for this wave's outstanding
// global loads and stores, which is exactly what must not be waited for.)
__device__ inline void cbar() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }
__device__ inline unsigned lds_load(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ inline void lds_store(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// barrier of the four compute waves (the loader waves do not take part)
__device__ inline bool cw_barrier(Ctx& c) {
  c.barn += 1;
  cbar();
  if (c.lane == 0) __hip_atomic_fetch_add(&c.sh->cwbar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const unsigned target = c.barn * NCOMPUTE;
  const unsigned t0 = now_ticks();
  unsigned spins = 0;
  while (lds_load(&c.sh->cwbar) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (!keep_waiting(c, t0, spins)) return false;
  }
  cbar();
  return true;
}

// waits until ring positions [p0, p0 + n) hold their tiles
__device__ inline bool wait_tiles(Ctx& c, unsigned p0, unsigned n) {
  if (n == 0) return true;
  const unsigned pe = p0 + n;
  const unsigned t0 = now_ticks();
  unsigned spins = 0;
#pragma unroll
  for (int q = 0; q < NLOADER; ++q) {
    if (pe <= (unsigned)q) continue;
    const unsigned need = (pe - (unsigned)q + 3u) / 4u;  // this loader's positions below pe
    while (lds_load(&c.sh->ready[q]) < need) {
      __builtin_amdgcn_s_sleep(1);
      if (!keep_waiting(c, t0, spins)) return false;
    }
  }
  cbar();
  return true;
}

__device__ inline void release_ring(Ctx& c, unsigned upto) {
  cbar();
  if (c.wave == 0 && c.lane == 0) lds_store(&c.sh->consumed, upto);
}

// Scratch for cross-wave partial tiles.  Consecutive phases that use it take
// alternate halves, so a wave that runs ahead into the next phase never
// overwrites partials a reducer wave is still reading.
__device__ inline f32x4* red_buf(Ctx& c) { return (f32x4*)c.sh->red[c.redsel & 1u]; }
__device__ inline void red_next(Ctx& c) { c.redsel += 1u; }

__device__ inline bf16x8 ring_tile(const Ctx& c, unsigned pos) {
  const u32x4 v = *(const u32x4*)(c.ring + (pos % RING) * TILE_BYTES + c.lane * 16);
  return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------- tagged exchange

// Where load i of a poll reads: byte offset `vo` (per lane) + `so` (uniform)
// in the exchange arena; lanes with need == false skip it.
struct LA {
  unsigned vo, so;
  bool need;
};

// Polls N 16-byte loads (two tagged words each) until every needed word
// carries `tag`.  All loads are issued at once; while some are missing, the
// wave waits on one missing word with a single request per probe (so that
// many waiting waves do not flood the fabric) and then loads everything again.
// addr(i) must accept a runtime i.
template <int N, typename AF>
__device__ inline bool ll_poll(Ctx& c, AF addr, unsigned tag, u32x4 (&v)[N]) {
  const unsigned t0 = now_ticks();
  unsigned spins = 0;
  while (true) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const LA la = addr(i);
      v[i] = la.need ? __builtin_amdgcn_raw_buffer_load_b128(c.EX, la.vo, la.so, AUX_SC1) : u32x4{0u, tag, 0u, tag};
    }
    int bad = N;
#pragma unroll
    for (int i = N - 1; i >= 0; --i)
      if (!((v[i][1] == tag) && (v[i][3] == tag))) bad = i;
    const unsigned long long m = __ballot(bad < N);
    if (m == 0ull) return true;
    const int ln = __builtin_ctzll(m);
    const int bi = __builtin_amdgcn_readfirstlane(__shfl(bad, ln));
    const LA pa = addr(bi);
    const unsigned pv = (unsigned)__shfl((int)pa.vo, ln);
    const unsigned so = __builtin_amdgcn_readfirstlane(pa.so);
    while (true) {
      const u32x4 p = __builtin_amdgcn_raw_buffer_load_b128(c.EX, pv, so, AUX_SC1);
      if ((p[1] == tag) && (p[3] == tag)) break;
      if (!keep_waiting(c, t0, spins)) return false;
    }
  }
}

// B fragments of a pair-word activation buffer: fragment f = loads 2f, 2f+1
// (16 bytes apart) at rowbase + f * fstride
__device__ inline LA frag_la(unsigned vo, unsigned s0, unsigned fstride, int i, bool need) {
  return LA{vo, s0 + (unsigned)(i >> 1) * fstride + (unsigned)(i & 1) * 16u, need};
}

__device__ inline void ll_store2(Ctx& c, unsigned off, unsigned p0, unsigned p1, unsigned tag) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{p0, tag, p1, tag}, c.EX, off, 0, AUX_SC1);
}
__device__ inline void ll_store1(Ctx& c, unsigned off, unsigned p0, unsigned tag) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{p0, tag}, c.EX, off, 0, AUX_SC1);
}

__device__ inline bf16x8 frag_of(const u32x4& v0, const u32x4& v1) {
  return __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[2], v1[0], v1[2]});
}

// Sums of squares: the owners' per-block partials [RP][NTD] are read as 8
// loads per lane (lane: row lane / 4, owners 16 (lane % 4) + [0, 16)).
__device__ inline LA ss_la(Ctx& c, unsigned base, int i) {
  const int row = c.lane >> 2, part = c.lane & 3;
  return LA{((unsigned)row * NTD + (unsigned)(part * 16)) * 8u, base + (unsigned)i * 16u, row < c.a->R};
}
// 1/rms per row from those 8 loads, into LDS rrow
__device__ inline void ss_finish(Ctx& c, const u32x4* v) {
  const int row = c.lane >> 2, part = c.lane & 3;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += as_f(v[i][0]) + as_f(v[i][2]);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if (part == 0) c.sh->rrow[row] = 1.0f / sqrtf(s / (float)D + c.a->eps);
}

// ---------------------------------------------------------------- owner

// (1 + scale) of the owner's four columns for one norm (issue early; use after)
__device__ inline u32x4 owner_scale_load(Ctx& c, int k, int norm) {
  const int col = 16 * c.r.owner + 4 * c.g;
  const unsigned moff = (unsigned)(((k * (2 * c.a->NL + 1) + norm) * 2 * D + col) * 4);
  return __builtin_amdgcn_raw_buffer_load_b128(c.AUX, moff, c.a->o_mod, 0);
}

// h (wave 0, lane: cols 16*owner + 4g + i, row) -> bf16(h * (1 + scale)) pairs
// and per-row sums of squares of this column block
__device__ inline void owner_publish(Ctx& c, const f32x4& h, const u32x4& sv, int k, int ltag, int t_hs, int t_ss) {
  const int j = c.r.owner;
  const unsigned tag_hs = tag_of(c, k, ltag, t_hs), tag_ss = tag_hs;  // one tag for both halves
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = h[i] * (1.0f + as_f(sv[i]));
  float s = h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3];
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  if (c.row < c.a->R) {
    const unsigned base = xoff(c, k, ltag, t_hs);
    ll_store2(c, base + ((unsigned)c.row * (D / 2) + (unsigned)(8 * j + 2 * c.g)) * 8u, pack_bf16(y[0], y[1]),
              pack_bf16(y[2], y[3]), tag_hs);
    if (c.g == 0)
      ll_store1(c, xoff(c, k, ltag, t_ss) + ((unsigned)c.row * NTD + (unsigned)j) * 8u, as_u(s), tag_ss);
  }
}

// phase timeline (off unless the handle asked for it)
__device__ inline void tl_mark(Ctx& c, int ev) {
  if (c.a->o_tl != 0u && c.lane == 0) {
    const unsigned idx = (blockIdx.x * (unsigned)timeline_events(c.a->S, c.a->NL) + (unsigned)ev) * 4u;
    __builtin_amdgcn_raw_buffer_store_b32(now_ticks(), c.AUX, idx, c.a->o_tl, 0);
  }
}

// ------------------------------------------------------------- phases
// Every phase is entered by all four compute waves; barrier counts match.
// Each phase issues all the loads it needs (tables first, then the exchange
// words) before waiting on any of them.

// input projection h = x . W_in for the owner's column block (one k-tile)
__device__ __attribute__((always_inline)) inline bool ph_in(Ctx& c, int k, f32x4& hreg) {
  if (c.r.owner < 0) return true;
  const unsigned p0 = (unsigned)k * c.n_step;
  if (c.wave == 0) {
    const u32x4 sv = owner_scale_load(c, k, 0);
    bf16x8 b;
    if (k == 0) {
      const bool ok = c.row < c.a->R;
      const unsigned off = ((unsigned)c.row * A + 8u * (unsigned)c.g) * 4u;
      const u32x4 v0 = ok ? __builtin_amdgcn_raw_buffer_load_b128(c.AUX, off, c.a->o_x, 0) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 v1 = ok ? __builtin_amdgcn_raw_buffer_load_b128(c.AUX, off + 16u, c.a->o_x, 0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = (bf16)as_f(v0[i]);
        b[4 + i] = (bf16)as_f(v1[i]);
      }
    } else {
      u32x4 v[2];
      const unsigned vo = ((unsigned)c.row * (A / 2) + 4u * (unsigned)c.g) * 8u;
      const unsigned s0 = xoff(c, k - 1, c.a->NL, X_X);
      const bool nd = c.row < c.a->R;
      if (!ll_poll<2>(c, [&](int i) { return frag_la(vo, s0, 0u, i, nd); }, tag_of(c, k - 1, c.a->NL, X_X), v))
        return false;
      b = frag_of(v[0], v[1]);
    }
    if (!wait_tiles(c, p0, 1)) return false;
    hreg = mma32(ring_tile(c, p0), b, f32x4{0.f, 0.f, 0.f, 0.f});
    release_ring(c, p0 + 1);
    owner_publish(c, hreg, sv, k, 0, X_HS, X_SS);
  }
  return true;
}

// QKV projection of n_qkv n-tiles, K = D split over the four waves; epilogue
// 1/rms, shift . W, RoPE; writes q (per head), k and v of the action rows
__device__ __attribute__((always_inline)) inline bool ph_qkv(Ctx& c, int k, int l) {
  const int nq = c.r.n_qkv;
  if (nq == 0) return true;
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer;
  // epilogue tables of this wave's n-tile (wave t reduces n-tile t)
  const int nt_e = c.r.qkv_nt0 + (c.wave < nq ? c.wave : 0);
  const int tt_e = nt_e % 16;
  const u32x4 sw = __builtin_amdgcn_raw_buffer_load_b128(
      c.AUX, (unsigned)(((k * c.a->NL + l) * NQKV + nt_e * 16 + 4 * c.g) * 4), c.a->o_swqkv, 0);
  const u32x4 cs = __builtin_amdgcn_raw_buffer_load_b128(
      c.AUX, (unsigned)((c.row * (DH / 2) + 8 * tt_e + 2 * c.g) * 8), c.a->o_rope, 0);
  u32x4 v[24];
  {
    const unsigned vo = ((unsigned)c.row * (D / 2) + 4u * (unsigned)c.g) * 8u;
    const unsigned s0 = xoff(c, k, l, X_HS) + (unsigned)(8 * c.wave) * 128u;
    const unsigned sb = xoff(c, k, l, X_SS);
    const bool nd = c.row < c.a->R, w0 = c.wave == 0;
    auto addr = [&](int i) -> LA {
      if (i < 16) return frag_la(vo, s0, 128u, i, nd);
      LA la = ss_la(c, sb, i - 16);
      la.need = la.need && w0;
      return la;
    };
    if (!ll_poll<24>(c, addr, tag_of(c, k, l, X_HS), v)) return false;
    if (w0) ss_finish(c, v + 16);
  }
  if (!wait_tiles(c, p0, 32u * (unsigned)nq)) return false;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t < nq) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        acc[t] = mma32(ring_tile(c, p0 + 32u * t + 8u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc[t]);
    }
  }
  f32x4* red = red_buf(c);
  red_next(c);
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (t < nq) red[(c.wave * 4 + t) * 64 + c.lane] = acc[t];
  if (!cw_barrier(c)) return false;
  release_ring(c, p0 + 32u * nq);
  if (c.wave < nq) {
    const int t = c.wave;
    f32x4 s = red[(0 * 4 + t) * 64 + c.lane];
    s += red[(1 * 4 + t) * 64 + c.lane];
    s += red[(2 * 4 + t) * 64 + c.lane];
    s += red[(3 * 4 + t) * 64 + c.lane];
    const int nt = nt_e;
    const int hh = nt / 16, tt = tt_e;
    const float rr = c.sh->rrow[c.row];
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = rr * s[i] + as_f(sw[i]);
    if (hh <= H) {  // q heads and the key head are rotated
      const float c0 = as_f(cs[0]), s0 = as_f(cs[1]);
      const float c1 = as_f(cs[2]), s1 = as_f(cs[3]);
      const float x0 = y[0], x1 = y[1], x2 = y[2], x3 = y[3];
      y[0] = x0 * c0 - x2 * s0;
      y[2] = x2 * c0 + x0 * s0;
      y[1] = x1 * c1 - x3 * s1;
      y[3] = x3 * c1 + x1 * s1;
    }
    if (c.row < c.a->R) {
      const unsigned tag = tag_of(c, k, l, X_Q);
      const unsigned hb = xoff(c, k, l, X_Q) + ((unsigned)(hh * RP + c.row) * (DH / 2)) * 8u;
      ll_store1(c, hb + (unsigned)(4 * tt + c.g) * 8u, pack_bf16(y[0], y[1]), tag);
      ll_store1(c, hb + (unsigned)(64 + 4 * tt + c.g) * 8u, pack_bf16(y[2], y[3]), tag);
    }
  }
  return true;
}

// attention of head h over one key chunk: prefix keys [64 c, 64 c + 64) from
// the ring, or (c == n_chunks) the action rows' own keys and values
__device__ __attribute__((always_inline)) inline bool ph_attn(Ctx& c, int k, int l) {
  const int hd = c.r.attn_h, ch = c.r.attn_c;
  if (ch < 0) return true;
  const bool action = ch == c.a->n_chunks;
  const unsigned tag_q = tag_of(c, k, l, X_Q);
  const unsigned qb = xoff(c, k, l, X_Q);
  const float scale = 0.0625f;  // 1/sqrt(256)
  const unsigned vo = ((unsigned)c.row * (DH / 2) + 4u * (unsigned)c.g) * 8u;
  f32x4 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_row, l_row;
  if (!action) {
    // q of this head as 8 B fragments (dims 32 s + 8 g + [0, 8))
    bf16x8 qf[8];
    {
      u32x4 v[16];
      const unsigned s0 = qb + (unsigned)(hd * RP) * (DH / 2) * 8u;
      const bool nd = c.row < c.a->R;
      if (!ll_poll<16>(c, [&](int i) { return frag_la(vo, s0, 128u, i, nd); }, tag_q, v)) return false;
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = frag_of(v[2 * s], v[2 * s + 1]);
    }
    const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer + c.o_attn;
    if (!wait_tiles(c, p0, 64)) return false;
    // S^T for keys [16 w, 16 w + 16) of the chunk: lane holds keys 4g + i of row `row`
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) st = mma32(ring_tile(c, p0 + 8u * c.wave + s), qf[s], st);
    float sv[4];
    float mw = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = CHUNK * ch + 16 * c.wave + 4 * c.g + i;
      sv[i] = key < c.L ? st[i] * scale : -INFINITY;
      mw = fmaxf(mw, sv[i]);
    }
    mw = fmaxf(mw, __shfl_xor(mw, 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    if (c.g == 0) c.sh->att_m[c.wave][c.row] = mw;
    if (!cw_barrier(c)) return false;
    m_row = fmaxf(fmaxf(c.sh->att_m[0][c.row], c.sh->att_m[1][c.row]),
                  fmaxf(c.sh->att_m[2][c.row], c.sh->att_m[3][c.row]));
    float lw = 0.f;
    s16x4 pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = sv[i] == -INFINITY ? 0.f : expf(sv[i] - m_row);
      lw += p;
      pf[i] = as_s((bf16)p);
    }
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
    if (c.g == 0) c.sh->att_l[c.wave][c.row] = lw;
    c.sh->att_p[c.wave][c.lane] = pf;
    if (!cw_barrier(c)) return false;
    l_row = (c.sh->att_l[0][c.row] + c.sh->att_l[1][c.row]) + (c.sh->att_l[2][c.row] + c.sh->att_l[3][c.row]);
    // O = P . V for dim tiles [4 w, 4 w + 4), all four key groups
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const s16x4 a = c.sh->att_p[kg][c.lane];
#pragma unroll
      for (int dp = 0; dp < 2; ++dp) {
        const unsigned pos = p0 + 32u + 8u * kg + 2u * c.wave + dp;
        const u32x4 vv = *(const u32x4*)(c.ring + (pos % RING) * TILE_BYTES + c.lane * 16);
        const s16x4 b0 = __builtin_bit_cast(s16x4, u32x2{vv[0], vv[1]});
        const s16x4 b1 = __builtin_bit_cast(s16x4, u32x2{vv[2], vv[3]});
        oacc[2 * dp] = mma16(a, b0, oacc[2 * dp]);
        oacc[2 * dp + 1] = mma16(a, b1, oacc[2 * dp + 1]);
      }
    }
    if (!cw_barrier(c)) return false;
    release_ring(c, p0 + 64u);
  } else {
    // q, the action keys (A fragments) and the action values, in one poll;
    // the values are staged transposed in LDS for the P . V fragments
    bf16x8 qf[8], kf[8];
    unsigned short* va = (unsigned short*)red_buf(c);
    red_next(c);
    {
      const int t = c.wave * 64 + c.lane;  // 256 threads: thread t clears dims t
#pragma unroll
      for (int key = 0; key < RP; ++key) va[t * RP + key] = 0;
    }
    {
      u32x4 v[36];
      const unsigned sq = qb + (unsigned)(hd * RP) * (DH / 2) * 8u;
      const unsigned sk = qb + (unsigned)(H * RP) * (DH / 2) * 8u;
      const unsigned sv0 = qb + (unsigned)((H + 1) * RP) * (DH / 2) * 8u;
      const unsigned vov = ((unsigned)c.wave * (DH / 2) + 2u * (unsigned)c.lane) * 8u;
      const bool nq = c.row < c.a->R, nk = c.row < c.a->M;
      const int M = c.a->M, w = c.wave;
      auto addr = [&](int i) -> LA {
        if (i < 16) return frag_la(vo, sq, 128u, i, nq);
        if (i < 32) return frag_la(vo, sk, 128u, i - 16, nk);
        const int key = w + 4 * (i - 32);  // value rows w, w + 4, w + 8, w + 12
        return LA{vov, sv0 + (unsigned)(4 * (i - 32)) * (DH / 2) * 8u, key < M};
      };
      if (!ll_poll<36>(c, addr, tag_q, v)) return false;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        qf[s] = frag_of(v[2 * s], v[2 * s + 1]);
        kf[s] = frag_of(v[16 + 2 * s], v[16 + 2 * s + 1]);
      }
      if (!cw_barrier(c)) return false;  // staging area cleared by every wave
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = c.wave + 4 * i;
        if (key < c.a->M) {
          const int d0 = 4 * c.lane;  // pair words 2 lane, 2 lane + 1 -> dims 4 lane .. 4 lane + 3
          va[(d0 + 0) * RP + key] = (unsigned short)(v[32 + i][0] & 0xffffu);
          va[(d0 + 1) * RP + key] = (unsigned short)(v[32 + i][0] >> 16);
          va[(d0 + 2) * RP + key] = (unsigned short)(v[32 + i][2] & 0xffffu);
          va[(d0 + 3) * RP + key] = (unsigned short)(v[32 + i][2] >> 16);
        }
      }
    }
    if (!cw_barrier(c)) return false;
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) st = mma32(kf[s], qf[s], st);
    float sv[4];
    float mw = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 4 * c.g + i;
      sv[i] = key < c.a->M ? st[i] * scale : -INFINITY;
      mw = fmaxf(mw, sv[i]);
    }
    mw = fmaxf(mw, __shfl_xor(mw, 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    m_row = mw;
    float lw = 0.f;
    s16x4 pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = sv[i] == -INFINITY ? 0.f : expf(sv[i] - m_row);
      lw += p;
      pf[i] = as_s((bf16)p);
    }
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
    l_row = lw;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int dim = 16 * (4 * c.wave + d) + c.row;
      const s16x4 b = *(const s16x4*)(va + dim * RP + 4 * c.g);
      oacc[d] = mma16(pf, b, oacc[d]);
    }
  }
  // outputs: unnormalised O [row][dim] and (max, sum) per row
  const unsigned tag = tag_of(c, k, l, X_ATT);
  const unsigned ob = xoff(c, k, l, X_ATT);
  const unsigned hc = (unsigned)(hd * MAX_CHUNKS + ch);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int dim = 16 * (4 * c.wave + d) + c.row;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rw = 4 * c.g + i;
      if (rw < c.a->R)
        ll_store1(c, ob + ((hc * RP + (unsigned)rw) * DH + (unsigned)dim) * 8u, as_u(oacc[d][i]), tag);
    }
  }
  if (c.wave == 0 && c.g == 0 && c.row < c.a->R) {
    const unsigned mlb = ob + (unsigned)(H * MAX_CHUNKS * RP * DH) * 8u;
    ll_store2(c, mlb + ((hc * RP + (unsigned)c.row) * 2u) * 8u, as_u(m_row), as_u(l_row), tag);
  }
  return true;
}

// merges the key chunks of head h for dims [32 s, 32 s + 32) and writes the
// normalised attention output as bf16 pairs
__device__ __attribute__((always_inline)) inline bool ph_comb(Ctx& c, int k, int l) {
  const int hd = c.r.comb_h, sl = c.r.comb_s;
  if (hd < 0) return true;
  const int nch = c.a->n_chunks + 1;
  const unsigned tag = tag_of(c, k, l, X_ATT);
  const unsigned ob = xoff(c, k, l, X_ATT);
  const unsigned mlb = ob + (unsigned)(H * MAX_CHUNKS * RP * DH) * 8u;
  const int dp = c.lane & 15, rg = c.lane >> 4;
  float M[4], Lsum[4], acc0[4], acc1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    M[i] = -INFINITY;
    Lsum[i] = 0.f;
    acc0[i] = acc1[i] = 0.f;
  }
  // chunks w, w + 4, w + 8, w + 12 of this wave in one poll (rounds of four)
  for (int base = c.wave; base < nch; base += 4 * NCOMPUTE) {
    u32x4 v[32];
    const int R = c.a->R, w4 = NCOMPUTE;
    auto addr = [&](int i) -> LA {
      const int cc = base + w4 * (i >> 3), j = i & 7;
      const unsigned hc = (unsigned)(hd * MAX_CHUNKS + cc);
      const int rw = rg + 4 * (j & 3);
      const bool nd = cc < nch && rw < R;
      if (j < 4) return LA{(unsigned)rg * 16u, mlb + (hc * RP + 4u * (unsigned)(j & 3)) * 16u, nd};
      return LA{((unsigned)rg * DH + (unsigned)(2 * dp)) * 8u,
                ob + (hc * RP * DH + 4u * (unsigned)(j & 3) * DH + 32u * sl) * 8u, nd};
    };
    if (!ll_poll<32>(c, addr, tag, v)) return false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (base + NCOMPUTE * q >= nch) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mc = as_f(v[8 * q + i][0]);
        const float lc = as_f(v[8 * q + i][2]);
        if (mc != -INFINITY) {
          const float mn = fmaxf(M[i], mc);
          const float sa = M[i] == -INFINITY ? 0.f : expf(M[i] - mn);
          const float sb = expf(mc - mn);
          acc0[i] = acc0[i] * sa + as_f(v[8 * q + 4 + i][0]) * sb;
          acc1[i] = acc1[i] * sa + as_f(v[8 * q + 4 + i][2]) * sb;
          Lsum[i] = Lsum[i] * sa + lc * sb;
          M[i] = mn;
        }
      }
    }
  }
  f32x4* red = red_buf(c);
  red_next(c);
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(c.wave * 4 + i) * 64 + c.lane] = f32x4{M[i], Lsum[i], acc0[i], acc1[i]};
  if (!cw_barrier(c)) return false;
  if (c.wave == 0) {
    const unsigned tag_o = tag_of(c, k, l, X_O);
    const unsigned obase = xoff(c, k, l, X_O);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = -INFINITY, s = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int w = 0; w < NCOMPUTE; ++w) {
        const f32x4 p = red[(w * 4 + i) * 64 + c.lane];
        if (p[0] != -INFINITY) {
          const float mn = fmaxf(m, p[0]);
          const float sa = m == -INFINITY ? 0.f : expf(m - mn);
          const float sb = expf(p[0] - mn);
          a0 = a0 * sa + p[2] * sb;
          a1 = a1 * sa + p[3] * sb;
          s = s * sa + p[1] * sb;
          m = mn;
        }
      }
      const int rw = rg + 4 * i;
      if (rw < c.a->R) {
        const float inv = 1.0f / s;
        ll_store1(c, obase + ((unsigned)rw * (HD / 2) + (unsigned)(hd * (DH / 2) + 16 * sl + dp)) * 8u,
                  pack_bf16(a0 * inv, a1 * inv), tag_o);
      }
    }
  }
  return true;
}

// out projection of the owner's column block (K = H*DH over the four waves),
// residual add, and the MLP norm's producer half
__device__ __attribute__((always_inline)) inline bool ph_o(Ctx& c, int k, int l, f32x4& hreg) {
  if (c.r.owner < 0) return true;
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer + c.o_o;
  const u32x4 sv = owner_scale_load(c, k, 2 * l + 1);
  u32x4 v[32];
  {
    const unsigned vo = ((unsigned)c.row * (HD / 2) + 4u * (unsigned)c.g) * 8u;
    const unsigned s0 = xoff(c, k, l, X_O) + (unsigned)(16 * c.wave) * 128u;
    const bool nd = c.row < c.a->R;
    if (!ll_poll<32>(c, [&](int i) { return frag_la(vo, s0, 128u, i, nd); }, tag_of(c, k, l, X_O), v)) return false;
  }
  if (!wait_tiles(c, p0, 64)) return false;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 16; ++kk)
    acc = mma32(ring_tile(c, p0 + 16u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc);
  f32x4* red = red_buf(c);
  red_next(c);
  red[(c.wave * 4) * 64 + c.lane] = acc;
  if (!cw_barrier(c)) return false;
  release_ring(c, p0 + 64u);
  if (c.wave == 0) {
    f32x4 s = red[0 * 64 + c.lane];
    s += red[4 * 64 + c.lane];
    s += red[8 * 64 + c.lane];
    s += red[12 * 64 + c.lane];
    hreg += s;
    owner_publish(c, hreg, sv, k, l, X_HS1, X_SS1);
  }
  return true;
}

// gate/up projection of n_gu n-tiles with the GeGLU epilogue
__device__ __attribute__((always_inline)) inline bool ph_gu(Ctx& c, int k, int l) {
  const int ng = c.r.n_gu;
  if (ng == 0) return true;
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer + c.o_gu;
  const int nt_e = c.r.gu_nt0 + (c.wave < ng ? c.wave : 0);
  const u32x4 sw = __builtin_amdgcn_raw_buffer_load_b128(
      c.AUX, (unsigned)(((k * c.a->NL + l) * 2 * F + nt_e * 16 + 4 * c.g) * 4), c.a->o_swgu, 0);
  u32x4 v[24];
  {
    const unsigned vo = ((unsigned)c.row * (D / 2) + 4u * (unsigned)c.g) * 8u;
    const unsigned s0 = xoff(c, k, l, X_HS1) + (unsigned)(8 * c.wave) * 128u;
    const unsigned sb = xoff(c, k, l, X_SS1);
    const bool nd = c.row < c.a->R;
    const bool w0 = c.wave == 0;
    auto addr = [&](int i) -> LA {
      if (i < 16) return frag_la(vo, s0, 128u, i, nd);
      LA la = ss_la(c, sb, i - 16);
      la.need = la.need && w0;
      return la;
    };
    if (!ll_poll<24>(c, addr, tag_of(c, k, l, X_HS1), v)) return false;
    if (w0) ss_finish(c, v + 16);
  }
  if (!wait_tiles(c, p0, 32u * (unsigned)ng)) return false;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (t < ng) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        acc[t] = mma32(ring_tile(c, p0 + 32u * t + 8u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc[t]);
    }
  f32x4* red = red_buf(c);
  red_next(c);
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (t < ng) red[(c.wave * 4 + t) * 64 + c.lane] = acc[t];
  if (!cw_barrier(c)) return false;
  release_ring(c, p0 + 32u * ng);
  if (c.wave < ng) {
    const int t = c.wave;
    f32x4 s = red[(0 * 4 + t) * 64 + c.lane];
    s += red[(1 * 4 + t) * 64 + c.lane];
    s += red[(2 * 4 + t) * 64 + c.lane];
    s += red[(3 * 4 + t) * 64 + c.lane];
    const int nt = nt_e;
    const float rr = c.sh->rrow[c.row];
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = rr * s[i] + as_f(sw[i]);
    const float a0 = gelu_tanh(y[0]) * y[2];
    const float a1 = gelu_tanh(y[1]) * y[3];
    if (c.row < c.a->R)
      ll_store1(c, xoff(c, k, l, X_A) + ((unsigned)c.row * (F / 2) + (unsigned)(4 * nt + c.g)) * 8u,
                pack_bf16(a0, a1), tag_of(c, k, l, X_A));
  }
  return true;
}

// down projection: K group kq (8 k-tiles, two per wave) x N group nq (4 n-tiles)
__device__ __attribute__((always_inline)) inline bool ph_down(Ctx& c, int k, int l) {
  const int kq = c.r.dn_kq, nqd = c.r.dn_nq;
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer + c.o_dn;
  u32x4 v[4];
  {
    const unsigned vo = ((unsigned)c.row * (F / 2) + 4u * (unsigned)c.g) * 8u;
    const unsigned s0 = xoff(c, k, l, X_A) + (unsigned)(8 * kq + 2 * c.wave) * 128u;
    const bool nd = c.row < c.a->R;
    if (!ll_poll<4>(c, [&](int i) { return frag_la(vo, s0, 128u, i, nd); }, tag_of(c, k, l, X_A), v)) return false;
  }
  if (!wait_tiles(c, p0, 32)) return false;
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      acc[t] = mma32(ring_tile(c, p0 + 8u * t + 2u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc[t]);
  }
  f32x4* red = red_buf(c);
  red_next(c);
#pragma unroll
  for (int t = 0; t < 4; ++t) red[(c.wave * 4 + t) * 64 + c.lane] = acc[t];
  if (!cw_barrier(c)) return false;
  release_ring(c, p0 + 32u);
  {
    const int t = c.wave;
    f32x4 s = red[(0 * 4 + t) * 64 + c.lane];
    s += red[(1 * 4 + t) * 64 + c.lane];
    s += red[(2 * 4 + t) * 64 + c.lane];
    s += red[(3 * 4 + t) * 64 + c.lane];
    if (c.row < c.a->R) {
      const int col = 16 * (4 * nqd + t) + 4 * c.g;
      const unsigned o = xoff(c, k, l, X_DP) + (((unsigned)kq * RP + (unsigned)c.row) * D + (unsigned)col) * 8u;
      const unsigned tag = tag_of(c, k, l, X_DP);
      ll_store2(c, o, as_u(s[0]), as_u(s[1]), tag);
      ll_store2(c, o + 16u, as_u(s[2]), as_u(s[3]), tag);
    }
  }
  return true;
}

// residual add of the 16 down partials of the owner's block, and the next
// norm's producer half (the next layer's attention norm, or the final norm)
__device__ __attribute__((always_inline)) inline bool ph_owner2(Ctx& c, int k, int l, f32x4& hreg) {
  if (c.r.owner < 0) return true;
  const int j = c.r.owner;
  const u32x4 sv = owner_scale_load(c, k, 2 * (l + 1));
  u32x4 v[8];
  {
    const unsigned vo = ((unsigned)c.row * D + (unsigned)(16 * j + 4 * c.g)) * 8u;
    const unsigned s0 = xoff(c, k, l, X_DP) + (unsigned)(4 * c.wave) * (RP * D * 8u);
    const bool nd = c.row < c.a->R;
    if (!ll_poll<8>(c, [&](int i) { return frag_la(vo, s0, RP * D * 8u, i, nd); }, tag_of(c, k, l, X_DP), v))
      return false;
  }
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[0] += as_f(v[2 * i][0]);
    s[1] += as_f(v[2 * i][2]);
    s[2] += as_f(v[2 * i + 1][0]);
    s[3] += as_f(v[2 * i + 1][2]);
  }
  f32x4* red = red_buf(c);
  red_next(c);
  red[(c.wave * 4) * 64 + c.lane] = s;
  if (!cw_barrier(c)) return false;
  if (c.wave == 0) {
    f32x4 t = red[0 * 64 + c.lane];
    t += red[4 * 64 + c.lane];
    t += red[8 * 64 + c.lane];
    t += red[12 * 64 + c.lane];
    hreg += t;
    owner_publish(c, hreg, sv, k, l + 1, X_HS, X_SS);
  }
  return true;
}

// velocity head of one n-tile (K = D over the four waves), final norm's
// consumer half, and the Euler update of the owned state columns
__device__ __attribute__((always_inline)) inline bool ph_out(Ctx& c, int k, f32x4& xreg) {
  if (c.r.out_nt < 0) return true;
  const int NL = c.a->NL;
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)NL * c.n_layer;
  const int t = c.r.out_nt;
  const u32x4 sw = __builtin_amdgcn_raw_buffer_load_b128(c.AUX, (unsigned)((k * A + 16 * t + 4 * c.g) * 4),
                                                         c.a->o_swout, 0);
  u32x4 v[24];
  {
    const unsigned vo = ((unsigned)c.row * (D / 2) + 4u * (unsigned)c.g) * 8u;
    const unsigned s0 = xoff(c, k, NL, X_HS) + (unsigned)(8 * c.wave) * 128u;
    const unsigned sb = xoff(c, k, NL, X_SS);
    const bool nd = c.row < c.a->R;
    const bool w0 = c.wave == 0;
    auto addr = [&](int i) -> LA {
      if (i < 16) return frag_la(vo, s0, 128u, i, nd);
      LA la = ss_la(c, sb, i - 16);
      la.need = la.need && w0;
      return la;
    };
    if (!ll_poll<24>(c, addr, tag_of(c, k, NL, X_HS), v)) return false;
    if (w0) ss_finish(c, v + 16);
  }
  if (!wait_tiles(c, p0, 32)) return false;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) acc = mma32(ring_tile(c, p0 + 8u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc);
  f32x4* red = red_buf(c);
  red_next(c);
  red[(c.wave * 4) * 64 + c.lane] = acc;
  if (!cw_barrier(c)) return false;
  release_ring(c, p0 + 32u);
  if (c.wave == 0) {
    f32x4 s = red[0 * 64 + c.lane];
    s += red[4 * 64 + c.lane];
    s += red[8 * 64 + c.lane];
    s += red[12 * 64 + c.lane];
    const float rr = c.sh->rrow[c.row];
#pragma unroll
    for (int i = 0; i < 4; ++i) xreg[i] += c.a->dt * (rr * s[i] + as_f(sw[i]));
    if (c.row < c.a->R) {
      if (k + 1 < c.a->S) {
        ll_store2(c, xoff(c, k, NL, X_X) + ((unsigned)c.row * (A / 2) + (unsigned)(8 * t + 2 * c.g)) * 8u,
                  pack_bf16(xreg[0], xreg[1]), pack_bf16(xreg[2], xreg[3]), tag_of(c, k, NL, X_X));
      } else {
        const u32x4 xv = {as_u(xreg[0]), as_u(xreg[1]), as_u(xreg[2]), as_u(xreg[3])};
        __builtin_amdgcn_raw_buffer_store_b128(xv, c.AUX, (unsigned)((c.row * A + 16 * t + 4 * c.g) * 4), c.a->o_x, 0);
      }
    }
  }
  return true;
}

// ---------------------------------------------------------------- loader

// Walks this workgroup's tile stream in order and yields the positions
// p = q (mod 4) of loader q: (byte offset, source).
struct Gen {
  int k, run, j;          // step, run index in the step, next tile index within the run
  unsigned pos0;          // stream position of the run's first tile
  unsigned off0;          // byte offset of the run's first tile
  int cnt;                // tiles in the run
  int kv;                 // 1: run reads the prefix K/V arena
};

__device__ inline void run_params(const Ctx& c, int run, unsigned& off, int& cnt, int& kv) {
  // run 0: input projection; 1 + 8 l + u: layer l part u; 1 + 8 NL: velocity head
  const Args& a = *c.a;
  const Role& r = c.r;
  kv = 0;
  cnt = 0;
  off = 0;
  if (run == 0) {
    if (r.owner >= 0) {
      cnt = 1;
      off = (unsigned)((a.off_in + (long long)r.owner * 512) * 2);
    }
    return;
  }
  const int NL = a.NL;
  if (run == 1 + 8 * NL) {
    if (r.out_nt >= 0) {
      cnt = 32;
      off = (unsigned)((a.off_out + (long long)r.out_nt * 32 * 512) * 2);
    }
    return;
  }
  const int l = (run - 1) / 8, u = (run - 1) % 8;
  const long long lo = (long long)l * a.lstride;
  if (u == 0) {
    if (r.n_qkv > 0) {
      cnt = 32 * r.n_qkv;
      off = (unsigned)((a.off_qkv + lo + (long long)r.qkv_nt0 * 32 * 512) * 2);
    }
  } else if (u == 1) {
    if (r.attn_c >= 0 && r.attn_c < a.n_chunks) {
      cnt = 64;
      kv = 1;
      off = (unsigned)(((long long)l * a.kv_lstride + (long long)r.attn_c * 64 * 512) * 2);
    }
  } else if (u == 2) {
    if (r.owner >= 0) {
      cnt = 64;
      off = (unsigned)((a.off_o + lo + (long long)r.owner * 64 * 512) * 2);
    }
  } else if (u == 3) {
    if (r.n_gu > 0) {
      cnt = 32 * r.n_gu;
      off = (unsigned)((a.off_gu + lo + (long long)r.gu_nt0 * 32 * 512) * 2);
    }
  } else {
    const int t = u - 4;
    cnt = 8;
    off = (unsigned)((a.off_dn + lo + ((long long)(4 * r.dn_nq + t) * KT_F + 8 * r.dn_kq) * 512) * 2);
  }
}

// next (position, byte offset, source) of loader q; false at the end
__device__ inline bool gen_next(const Ctx& c, Gen& s, int q, unsigned& pos, unsigned& off, int& kv) {
  const int runs_per_step = 2 + 8 * c.a->NL;
  while (s.j >= s.cnt) {
    s.pos0 += (unsigned)s.cnt;
    s.run += 1;
    if (s.run >= runs_per_step) {
      s.run = 0;
      s.k += 1;
      if (s.k >= c.a->S) return false;
    }
    run_params(c, s.run, s.off0, s.cnt, s.kv);
    s.j = (int)(((unsigned)q - s.pos0) & 3u);
  }
  pos = s.pos0 + (unsigned)s.j;
  off = s.off0 + (unsigned)s.j * TILE_BYTES;
  kv = s.kv;
  s.j += 4;
  return true;
}

// One 1 KiB tile straight from memory into the LDS ring (each lane moves 16
// bytes to M0 + 16 * lane).  Issued from inline assembly so the compiler does
// not guard every later LDS access with a wait for all outstanding loads; the
// loader waits for its own tiles with explicit vmcnt waits instead.  Weight
// tiles carry the streaming hint; prefix K/V tiles do not, so the other heads'
// workgroups on the same XCD find them in L2.
__device__ inline void dma_tile(u32x4 rs, unsigned voff, unsigned soff, unsigned lds, bool stream) {
  if (stream)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds" ::"s"(lds), "v"(voff), "s"(rs),
                 "s"(soff)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rs),
                 "s"(soff)
                 : "memory", "m0");
}

__device__ inline u32x4 rsrc_words(const void* p, unsigned bytes) {
  const unsigned long long b = (unsigned long long)p;
  return u32x4{(unsigned)b, (unsigned)(b >> 32) & 0xffffu, bytes, 0x00020000u};
}

constexpr unsigned LOAD_DEPTH = 16;  // tiles in flight per loader wave

__device__ __attribute__((always_inline)) inline void loader(Ctx& c, int q) {
  const u32x4 WR = rsrc_words(c.a->wt, c.a->wt_bytes);
  const u32x4 KR = rsrc_words(c.a->kvt, c.a->kvt_bytes);
  const unsigned ring_lds =
      (unsigned)(unsigned long long)((__attribute__((address_space(3))) unsigned char*)c.ring);
  Gen s;
  s.k = 0;
  s.run = 0;
  s.pos0 = 0;
  run_params(c, 0, s.off0, s.cnt, s.kv);
  s.j = q;
  unsigned issued = 0;
  unsigned pos, off;
  int kv;
  while (gen_next(c, s, q, pos, off, kv)) {
    if (pos >= lds_load(&c.sh->consumed) + RING) {
      // the ring is full: publish every tile in flight before waiting, since
      // the compute waves may be waiting for exactly those
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (c.lane == 0) lds_store(&c.sh->ready[q], issued);
      const unsigned t0 = now_ticks();
      unsigned spins = 0;
      bool ok = true;
      while (pos >= lds_load(&c.sh->consumed) + RING) {
        __builtin_amdgcn_s_sleep(2);
        if (!loader_keep_waiting(c, t0, spins)) {
          ok = false;
          break;
        }
      }
      if (!ok) break;
    }
    cbar();
    const unsigned lds = __builtin_amdgcn_readfirstlane(ring_lds + (pos % RING) * TILE_BYTES);
    if (kv)
      dma_tile(KR, (unsigned)c.lane * 16u, off, lds, false);
    else
      dma_tile(WR, (unsigned)c.lane * 16u, off, lds, true);
    ++issued;
    if (issued > LOAD_DEPTH) {
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      if (c.lane == 0) lds_store(&c.sh->ready[q], issued - LOAD_DEPTH);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (c.lane == 0) lds_store(&c.sh->ready[q], issued);
}

// ---------------------------------------------------------------- kernel

__global__ __launch_bounds__(THREADS, 1) void k_decide(Args a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char ring_mem[];
  __shared__ Shared sh;
  Ctx c;
  c.a = &a;
  c.sh = &sh;
  c.ring = ring_mem;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform per wave
  c.g = c.lane >> 4;
  c.row = c.lane & 15;
  c.barn = 0;
  c.redsel = 0;
  if (threadIdx.x < 32) ((unsigned*)&sh)[threadIdx.x] = 0u;
  c.W = rsrc(a.wt, a.wt_bytes);
  c.KV = rsrc(a.kvt, a.kvt_bytes);
  c.EX = rsrc(a.ex, a.ex_bytes);
  c.AUX = rsrc(a.aux, a.aux_bytes);
  {
    const unsigned ro = a.o_roles + blockIdx.x * (unsigned)sizeof(Role);
    const u32x4 r0 = __builtin_amdgcn_raw_buffer_load_b128(c.AUX, ro, 0, 0);
    const u32x4 r1 = __builtin_amdgcn_raw_buffer_load_b128(c.AUX, ro + 16u, 0, 0);
    const unsigned rw[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    c.r = __builtin_bit_cast(Role, rw);
    c.seq = __builtin_amdgcn_raw_buffer_load_b32(c.AUX, a.o_seq, 0, AUX_SC1);
    c.tagbase = c.seq * exchanges_per_decision(a.S, a.NL);
    c.L = (int)__builtin_amdgcn_raw_buffer_load_b32(c.AUX, a.o_lens, 0, 0);
  }
  // stream layout of this workgroup (must match run_params)
  const Role& r = c.r;
  c.n_in = r.owner >= 0 ? 1u : 0u;
  c.o_attn = 32u * (unsigned)r.n_qkv;
  c.o_o = c.o_attn + ((r.attn_c >= 0 && r.attn_c < a.n_chunks) ? 64u : 0u);
  c.o_gu = c.o_o + (r.owner >= 0 ? 64u : 0u);
  c.o_dn = c.o_gu + 32u * (unsigned)r.n_gu;
  c.n_layer = c.o_dn + 32u;
  c.n_out = r.out_nt >= 0 ? 32u : 0u;
  c.n_step = c.n_in + (unsigned)a.NL * c.n_layer + c.n_out;
  __syncthreads();

  if (c.wave >= NCOMPUTE) {
    loader(c, c.wave - NCOMPUTE);
    if (c.wave == NCOMPUTE) tl_mark(c, timeline_events(a.S, a.NL) - 1);
    return;
  }
  f32x4 hreg = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 xreg = f32x4{0.f, 0.f, 0.f, 0.f};
  if (r.out_nt >= 0 && c.wave == 0 && c.row < a.R) {
    const u32x4 xv =
        __builtin_amdgcn_raw_buffer_load_b128(c.AUX, (unsigned)((c.row * A + 16 * r.out_nt + 4 * c.g) * 4), a.o_x, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) xreg[i] = as_f(xv[i]);
  }
  bool ok = true;
  const bool tl = c.wave == 0;
  if (tl) tl_mark(c, 0);
  for (int k = 0; k < a.S && ok; ++k) {
    const int e0 = 1 + k * (2 + 7 * a.NL);
    ok = ph_in(c, k, hreg);
    if (tl) tl_mark(c, e0);
    for (int l = 0; l < a.NL && ok; ++l) {
      const int el = e0 + 1 + 7 * l;
      ok = ph_qkv(c, k, l);
      if (tl) tl_mark(c, el);
      ok = ok && ph_attn(c, k, l);
      if (tl) tl_mark(c, el + 1);
      ok = ok && ph_comb(c, k, l);
      if (tl) tl_mark(c, el + 2);
      ok = ok && ph_o(c, k, l, hreg);
      if (tl) tl_mark(c, el + 3);
      ok = ok && ph_gu(c, k, l);
      if (tl) tl_mark(c, el + 4);
      ok = ok && ph_down(c, k, l);
      if (tl) tl_mark(c, el + 5);
      ok = ok && ph_owner2(c, k, l, hreg);
      if (tl) tl_mark(c, el + 6);
    }
    ok = ok && ph_out(c, k, xreg);
    if (tl) tl_mark(c, e0 + 1 + 7 * a.NL);
  }
  if (tl) tl_mark(c, timeline_events(a.S, a.NL) - 2);
  if (!ok && r.out_nt >= 0 && c.wave == 0 && c.row < a.R) {
    const unsigned nanv = 0x7fc00000u;
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{nanv, nanv, nanv, nanv}, c.AUX,
                                           (unsigned)((c.row * A + 16 * r.out_nt + 4 * c.g) * 4), a.o_x, 0);
  }
}

__global__ void k_decide_advance(unsigned* seq) {
  if (threadIdx.x == 0 && blockIdx.x == 0) seq[0] = seq[0] + 1u;
}

hipError_t launch_decide(const Args& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_decide, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       RING * TILE_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_decide, dim3(G), dim3(THREADS), RING * TILE_BYTES, s, a);
  return hipGetLastError();
}

hipError_t launch_decide_advance(void* aux, unsigned o_seq, hipStream_t s) {
  hipLaunchKernelGGL(k_decide_advance, dim3(1), dim3(64), 0, s, (unsigned*)((char*)aux + o_seq));
  return hipGetLastError();
}

// ------------------------------------------------------------ set-up kernels

__device__ inline int colmap_dev(int kind, int param, int n) {
  const int nt = n / 16, cc = n % 16;
  if (kind == 0) return n;
  const int g = cc >> 2, i = cc & 3;
  if (kind == 1) {
    const int tph = param / 16;
    const int hh = nt / tph, t = nt - hh * tph;
    return hh * param + 8 * t + 2 * g + (i & 1) + (i >> 1) * (param / 2);
  }
  return 8 * nt + 2 * g + (i & 1) + (i >> 1) * param;
}

__global__ void k_shift_table(const bf16* __restrict__ w0, long long w_lstride, const float* __restrict__ modtab,
                              int NN, int norm_stride, int norm_off, int S, int nl, int N, int colkind, int colparam,
                              float* __restrict__ out) {
  const size_t total = (size_t)S * nl * N;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(idx % N);
    const size_t kl = idx / N;
    const int l = (int)(kl % nl), k = (int)(kl / nl);
    const int col = colmap_dev(colkind, colparam, n);
    const float* shift = modtab + ((size_t)k * NN + (size_t)(norm_stride * l + norm_off)) * 2 * D + D;
    const bf16* w = w0 + (size_t)l * w_lstride + col;
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += (double)shift[d] * (double)(float)w[(size_t)d * N];
    out[idx] = (float)acc;
  }
}

hipError_t launch_shift_table(const void* w0, long long w_lstride, const float* modtab, int NN, int norm_stride,
                              int norm_off, int S, int nl, int N, int colkind, int colparam, float* out,
                              hipStream_t s) {
  const size_t total = (size_t)S * nl * N;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_shift_table, dim3(blocks), dim3(256), 0, s, (const bf16*)w0, w_lstride, modtab, NN,
                     norm_stride, norm_off, S, nl, N, colkind, colparam, out);
  return hipGetLastError();
}

// Prefix K/V of one request ([NL][L][DH] bf16) into the attention tiles:
// per layer and 64-key chunk, 32 K tiles (key tile kt4 < 4, dim slice s < 8;
// lane: key 16 kt4 + lane % 16, dims 32 s + 8 (lane / 16) + [0, 8)) then 32 V
// tiles (key group kg < 4, dim-tile pair dp < 8; lane: 4 keys 16 kg + 4 (lane
// / 16) + [0, 4) of dim 16 (2 dp) + lane % 16, then the same keys of dim
// 16 (2 dp + 1) + lane % 16).  Keys at or past L are zero.
__global__ void k_attn_tiles(const bf16* __restrict__ k, const bf16* __restrict__ v, bf16* __restrict__ kvt, int NL,
                             int L, int n_chunks) {
  const size_t total = (size_t)NL * n_chunks * 64 * 512;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(idx % 512);
    const size_t tl = idx / 512;
    const int tile = (int)(tl % 64);
    const size_t lc = tl / 64;
    const int ch = (int)(lc % n_chunks), l = (int)(lc / n_chunks);
    const int lane = e / 8, j = e % 8;
    int key, dim;
    const bf16* src;
    if (tile < 32) {
      const int kt4 = tile / 8, s = tile % 8;
      key = CHUNK * ch + 16 * kt4 + (lane % 16);
      dim = 32 * s + 8 * (lane / 16) + j;
      src = k;
    } else {
      const int kg = (tile - 32) / 8, dp = (tile - 32) % 8;
      key = CHUNK * ch + 16 * kg + 4 * (lane / 16) + (j % 4);
      dim = 16 * (2 * dp + j / 4) + (lane % 16);
      src = v;
    }
    bf16 val = (bf16)0.0f;
    if (key < L) val = src[((size_t)l * L + key) * DH + dim];
    kvt[idx] = val;
  }
}

hipError_t launch_attn_tiles(const void* k, const void* v, void* kvt, int NL, int L, int n_chunks, hipStream_t s) {
  const size_t total = (size_t)NL * n_chunks * 64 * 512;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_attn_tiles, dim3(blocks), dim3(256), 0, s, (const bf16*)k, (const bf16*)v, (bf16*)kvt, NL, L,
                     n_chunks);
  return hipGetLastError();
}

}  // namespace dec
}  // namespace phx
