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
//     into a 124-tile LDS ring, running up to a ring ahead of the compute, so
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
// Register discipline: every layout is a compile-time constant (the shape is
// fixed), a workgroup's roles are a few integer operations on its index, and
// a wait that gives up ends the wave instead of unwinding through the phases,
// so the per-phase control flow stays free of spills.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int SC1 = 16;                             // cache policy: device-coherent access
constexpr unsigned TIMEOUT_TICKS = 50u * 1000u * 1000u;  // 0.5 s of the 100 MHz real-time counter

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
// the ring (dynamic) and the static shared data together stay within the
// 160 KiB of LDS one workgroup may hold
static_assert(RING * TILE_BYTES + sizeof(Shared) <= 160 * 1024, "LDS budget of one workgroup");


__device__ inline Rsrc rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// the real-time counter is a scalar value; readfirstlane tells the compiler,
// so that a wait's time-limit branch is uniform
__device__ inline unsigned now_ticks() {
  return __builtin_amdgcn_readfirstlane((unsigned)__builtin_amdgcn_s_memrealtime());
}

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

// Hardware exp2 / reciprocal / reciprocal square root (about 1 ulp); their
// error is far below the bf16 rounding of every value they feed.
__device__ inline float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ inline float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ inline float frsq(float x) { return __builtin_amdgcn_rsqf(x); }

// GeGLU's tanh-approximated GELU, with tanh(u) = 1 - 2 / (exp(2u) + 1)
__device__ inline float gelu_tanh(float z) {
  const float k = 0.7978845608028654f;  // sqrt(2/pi)
  const float u = k * (z + 0.044715f * z * z * z);
  const float t = 1.0f - 2.0f * frcp(fexp(2.0f * u) + 1.0f);
  return 0.5f * z * (1.0f + t);
}

__device__ inline f32x4 mma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mma16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------- context

struct Ctx {
  Shared* sh;
  unsigned char* ring;
  Rsrc X;                  // arena: exchange words at 0, auxiliary tables at AUX0
  unsigned tagbase;
  unsigned seq;            // this decision's counter
  unsigned redsel;         // which half of the partial-tile scratch the current phase uses
  unsigned barn;           // compute-wave barriers passed
  unsigned tl;             // timeline on
  int lane, wave, g, row;  // row = lane % 16, g = lane / 16
  int crow;                // row clamped to the last action row (poll addresses)
  int S, NL, R, nc, L;     // steps, layers, action rows, prefix chunks, prefix length
  float dt, eps;
  // roles (negative: none)
  int owner;               // residual column block: input and out projections, residual adds
  int qkv0;                // first of two QKV n-tiles
  int attn_h, attn_c;      // attention head and key chunk (attn_c == nc: the action rows' own keys)
  int comb_h, comb_s;      // combine of head comb_h, dims [32 comb_s, +32)
  int out_nt;              // velocity-head n-tile
  // ring positions of this workgroup's tile stream
  unsigned n_in, n_layer, n_step, o_attn, o_o, o_gu, o_dn;
};

// Roles of workgroup b.  Attention workgroup (head h, chunk c) is
// b = c + 32 h, so the eight heads of one key chunk run on one XCD (b mod 8)
// and share its L2 copy of the chunk; the combiners of head h are
// b = 32 h + 16 + s.  The workgroups that attend over no prefix chunk take
// the 64 owner roles and then the 80 QKV pairs, in the order
// (b mod 32 - chunks) * 8 + b / 32; if they run out, prefix-attention
// workgroups follow.  Every workgroup takes two gate/up n-tiles and one
// (K group, N group) of the down projection; the last two take the velocity
// head.
__device__ inline void set_roles(Ctx& c, int b) {
  const int c32 = b & 31, h = b >> 5;
  const int nc = c.nc;
  c.attn_h = c32 <= nc ? h : -1;
  c.attn_c = c32 <= nc ? c32 : -1;
  c.comb_h = (c32 >= 16 && c32 < 24) ? h : -1;
  c.comb_s = (c32 >= 16 && c32 < 24) ? c32 - 16 : -1;
  const int nfree = 8 * (32 - nc);
  const int idx = c32 >= nc ? (c32 - nc) * 8 + h : nfree + c32 * 8 + h;
  c.owner = idx < N_OWNER ? idx : -1;
  c.qkv0 = (idx >= N_OWNER && idx < N_OWNER + N_QKV_PAIRS) ? 2 * (idx - N_OWNER) : -1;
  c.out_nt = b >= G - NT_OUT ? b - (G - NT_OUT) : -1;
}

// Passes the context's uniform fields through an empty asm statement.  Every
// phase starts with it, so that what a phase derives from them (role tests,
// table offsets) is computed inside the phase: otherwise the compiler hoists
// all of it out of the step loop and keeps it in registers for the whole
// kernel, far more than the 102 scalar registers a wave has.
__device__ __attribute__((always_inline)) inline void refresh(Ctx& c) {
  asm volatile("" : "+s"(c.owner), "+s"(c.qkv0), "+s"(c.attn_h), "+s"(c.attn_c), "+s"(c.comb_h), "+s"(c.comb_s),
               "+s"(c.out_nt));
  asm volatile("" : "+s"(c.n_in), "+s"(c.n_layer), "+s"(c.n_step), "+s"(c.o_attn), "+s"(c.o_o), "+s"(c.o_gu),
               "+s"(c.o_dn));
  asm volatile("" : "+s"(c.tagbase), "+s"(c.seq), "+s"(c.S), "+s"(c.NL), "+s"(c.R), "+s"(c.nc), "+s"(c.L),
               "+s"(c.tl));
  asm volatile("" : "+v"(c.lane), "+v"(c.crow));
  c.g = c.lane >> 4;
  c.row = c.lane & 15;
}

__device__ inline unsigned slot_of(const Ctx& c, int k, int l) { return (unsigned)(k * (c.NL + 1) + l); }
__device__ inline unsigned tag_of(const Ctx& c, unsigned slot, int t) {
  return c.tagbase + slot * (unsigned)NX + (unsigned)t + 1u;
}
template <int T>
__device__ __attribute__((always_inline)) inline unsigned xoff(unsigned slot) {
  constexpr unsigned b = x_base(T), st = x_stride(T);
  return b + ((slot & 1u) ? st : 0u);
}
// byte offset of step k's table block in the arena
__device__ inline unsigned step_tab(const Ctx& c, int k) { return AUX0 + AUX_TAB + (unsigned)k * step_bytes(c.NL); }

__device__ inline void lds_store(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// LDS flags are read by whole waves; the value is uniform, and saying so
// keeps every wait loop's exit uniform for the compiler
__device__ inline unsigned lds_load(const unsigned* p) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
// Synchronisation inside a workgroup goes through LDS only.  The LDS unit
// performs each wave's operations in issue order, so a data write followed by
// a flag write is seen in that order by any wave that reads the flag first;
// the compiler barriers keep the compiler from reordering them.  (A
// workgroup-scope acquire/release would also wait for this wave's outstanding
// global loads and stores, which is exactly what must not be waited for.)
__device__ inline void cbar() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Ends the wave.  s_endpgm is issued from inline assembly: the hardware
// stops the wave there, while to the compiler it is an ordinary instruction,
// so the wait loops that may leave keep a simple (uniform) shape.  A
// noreturn builtin would give every such loop a second exit, which the
// compiler's control-flow structurizer treats as divergent.
__device__ __attribute__((always_inline)) inline void end_wave() { asm volatile("s_endpgm" ::: "memory"); }

// Raises the workgroup's abort flag (its other waves leave at their next
// wait), optionally records the failure in the status word (the decision
// counter + 1, so no clearing is needed), has the velocity-head workgroups
// mark their actions NaN, and ends the wave.
__device__ __attribute__((always_inline)) inline void leave(Ctx& c, bool record) {
  lds_store(&c.sh->abort, 1u);
  if (record && c.lane == 0) __builtin_amdgcn_raw_buffer_store_b32(c.seq + 1u, c.X, AUX0 + AUX_STATUS, 0, SC1);
  if (c.out_nt >= 0 && c.wave == 0 && c.row < c.R) {
    const unsigned nanv = 0x7fc00000u;
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{nanv, nanv, nanv, nanv}, c.X,
                                           AUX0 + AUX_X + (unsigned)((c.row * A + 16 * c.out_nt + 4 * c.g) * 4), 0, 0);
  }
  end_wave();
}

// One step of a bounded wait: leaves on the abort flag, on the time limit,
// or when another workgroup has recorded a failure of this decision.
__device__ inline void keep_waiting(Ctx& c, unsigned t0, unsigned& spins) {
  ++spins;
  if (lds_load(&c.sh->abort) != 0u) leave(c, false);
  if ((spins & 63u) == 0u) {
    if (now_ticks() - t0 > TIMEOUT_TICKS) leave(c, true);
    const unsigned st =
        __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(c.X, AUX0 + AUX_STATUS, 0, SC1));
    if (st == c.seq + 1u) leave(c, false);
  }
}

// barrier of the four compute waves (the loader waves do not take part)
__device__ inline void cw_barrier(Ctx& c) {
  c.barn += 1;
  cbar();
  if (c.lane == 0) __hip_atomic_fetch_add(&c.sh->cwbar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const unsigned target = c.barn * NCOMPUTE;
  const unsigned t0 = now_ticks();
  unsigned spins = 0;
  while (lds_load(&c.sh->cwbar) < target) {
    __builtin_amdgcn_s_sleep(1);
    keep_waiting(c, t0, spins);
  }
  cbar();
}

// waits until ring positions [p0, p0 + n) hold their tiles
__device__ inline void wait_tiles(Ctx& c, unsigned p0, unsigned n) {
  const unsigned pe = p0 + n;
  const unsigned t0 = now_ticks();
  unsigned spins = 0;
#pragma unroll
  for (int q = 0; q < NLOADER; ++q) {
    if (pe <= (unsigned)q) continue;
    const unsigned need = (pe - (unsigned)q + 3u) / 4u;  // this loader's positions below pe
    while (lds_load(&c.sh->ready[q]) < need) {
      __builtin_amdgcn_s_sleep(1);
      keep_waiting(c, t0, spins);
    }
  }
  cbar();
}

__device__ inline void release_ring(Ctx& c, unsigned upto) {
  cbar();
  if (c.wave == 0 && c.lane == 0) lds_store(&c.sh->consumed, upto);
}

// Scratch for cross-wave partial tiles.  Consecutive phases that use it take
// alternate halves, so a wave that runs ahead into the next phase never
// overwrites partials a reducer wave is still reading.
__device__ inline f32x4* red_take(Ctx& c) {
  f32x4* r = (f32x4*)c.sh->red[c.redsel & 1u];
  c.redsel += 1u;
  return r;
}
__device__ inline f32x4 red_sum(const f32x4* red, int t, int lane) {
  f32x4 s = red[(0 * 4 + t) * 64 + lane];
  s += red[(1 * 4 + t) * 64 + lane];
  s += red[(2 * 4 + t) * 64 + lane];
  s += red[(3 * 4 + t) * 64 + lane];
  return s;
}

__device__ inline bf16x8 ring_tile(const Ctx& c, unsigned pos) {
  const u32x4 v = *(const u32x4*)(c.ring + (pos % RING) * TILE_BYTES + c.lane * 16);
  return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------- tagged exchange

// Where load i of a poll reads: byte offset `vo` (per lane) + `so` (uniform)
// in the arena; `need` (uniform) == false skips the load.  Lanes of action
// rows past R read the last valid row instead (clamped rows), so every lane's
// words become valid and no per-lane predicate is needed; the memory system
// merges the duplicate addresses of a wave, and no result of a padded row is
// ever stored.
struct LA {
  unsigned vo, so;
  bool need;
};
// bases of a poll's addresses: per-lane v0, v1 and uniform s0, s1, s2
struct PB {
  unsigned v0, v1, s0, s1, s2;
};

// Polls N 16-byte loads (two tagged words each) until every needed word
// carries `tag`; addr(b, i) gives load i from the bases b.  A round issues
// every needed load.  While some are stale, the wave probes with a single
// load instruction in which lane i reads one stale word of load i (the
// first stale lane's), until every probed word is fresh, and then starts
// the next round; so a round moves the whole block only when each of its
// loads has made progress, and waiting waves read a few cache lines per
// probe instead of the whole block.  The bases pass through an empty asm
// statement in every round, so that the compiler computes each address next
// to its load instead of keeping N addresses live in registers.
template <int N, typename AF>
__device__ __attribute__((always_inline)) inline void ll_poll(Ctx& c, const PB& pb, AF addr, unsigned tag,
                                                              u32x4 (&v)[N]) {
  const unsigned t0 = now_ticks();
  unsigned spins = 0;
  while (true) {
    PB b = pb;
    asm volatile("" : "+v"(b.v0), "+v"(b.v1), "+s"(b.s0), "+s"(b.s1), "+s"(b.s2));
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const LA la = addr(b, i);
      v[i] = la.need ? __builtin_amdgcn_raw_buffer_load_b128(c.X, la.vo, __builtin_amdgcn_readfirstlane(la.so), SC1)
                     : u32x4{0u, tag, 0u, tag};
    }
    unsigned acc = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) acc |= (v[i][1] ^ tag) | (v[i][3] ^ tag);
    if (__ballot(acc != 0u) == 0ull) return;
    // probe addresses: lane i takes load i's first stale word; lanes without
    // a stale load repeat the highest stale load's probe
    unsigned pa = 0;
    bool any = false;
#pragma unroll
    for (int i = N - 1; i >= 0; --i) {
      const unsigned long long m = __ballot(((v[i][1] ^ tag) | (v[i][3] ^ tag)) != 0u);
      if (m != 0ull) {
        const LA la = addr(b, i);
        const unsigned a = __builtin_amdgcn_readfirstlane(la.so) + (unsigned)__shfl((int)la.vo, __builtin_ctzll(m));
        pa = (c.lane == i || !any) ? a : pa;
        any = true;
      }
    }
    while (true) {
      const u32x4 p = __builtin_amdgcn_raw_buffer_load_b128(c.X, pa, 0, SC1);
      if (__ballot((p[1] != tag) || (p[3] != tag)) == 0ull) break;
      keep_waiting(c, t0, spins);
    }
  }
}

// B fragments of a pair-word activation buffer: fragment f = loads 2f, 2f+1
// (16 bytes apart) at base + f * fstride
__device__ inline LA frag_la(unsigned vo, unsigned s0, unsigned fstride, int i) {
  return LA{vo + (unsigned)(i >> 1) * fstride + (unsigned)(i & 1) * 16u, s0, true};
}

__device__ inline void ll_store2(Ctx& c, unsigned off, unsigned p0, unsigned p1, unsigned tag) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{p0, tag, p1, tag}, c.X, off, 0, SC1);
}
__device__ inline void ll_store1(Ctx& c, unsigned off, unsigned p0, unsigned tag) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{p0, tag}, c.X, off, 0, SC1);
}

__device__ inline bf16x8 frag_of(const u32x4& v0, const u32x4& v1) {
  return __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[2], v1[0], v1[2]});
}

// Sums of squares: the owners' per-block partials [RP][NTD] are read as 8
// loads per lane (lane: row lane / 4, owners 16 (lane % 4) + [0, 16)).
__device__ inline unsigned ss_vo(const Ctx& c) {
  const int row = c.lane >> 2, part = c.lane & 3;
  const int crow = row < c.R ? row : c.R - 1;
  return ((unsigned)crow * NTD + (unsigned)(part * 16)) * 8u;
}
// 1/rms per row from those 8 loads, into LDS rrow
__device__ inline void ss_finish(Ctx& c, const u32x4* v) {
  const int row = c.lane >> 2, part = c.lane & 3;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += as_f(v[i][0]) + as_f(v[i][2]);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if (part == 0) c.sh->rrow[row] = frsq(s / (float)D + c.eps);
}

// Polls a normalised activation (16 rows x D as bf16 pairs, this wave's 8
// k-tiles: loads 0..15) plus, on wave 0, the owners' sums of squares (loads
// 16..23), and leaves 1/rms per row in LDS.
template <int t_hs, int t_ss>
__device__ inline void poll_normed(Ctx& c, unsigned slot, u32x4 (&v)[24]) {
  const bool w0 = c.wave == 0;
  const PB pb{((unsigned)c.crow * (D / 2) + 4u * (unsigned)c.g) * 8u, ss_vo(c),
              xoff<t_hs>(slot) + (unsigned)(8 * c.wave) * 128u, xoff<t_ss>(slot), 0u};
  auto addr = [&](const PB& b, int i) -> LA {
    if (i < 16) return frag_la(b.v0, b.s0, 128u, i);
    return LA{b.v1 + (unsigned)(i - 16) * 16u, b.s1, w0};
  };
  ll_poll<24>(c, pb, addr, tag_of(c, slot, t_hs), v);
  if (w0) ss_finish(c, v + 16);
}

// ---------------------------------------------------------------- owner

// (1 + scale) of the owner's four columns for one norm (issue early; use after)
__device__ inline u32x4 owner_scale_load(const Ctx& c, int k, int norm) {
  const unsigned off = step_tab(c, k) + (unsigned)((norm * D + 16 * c.owner + 4 * c.g) * 4);
  return __builtin_amdgcn_raw_buffer_load_b128(c.X, off, 0, 0);
}

// h (wave 0, lane: cols 16*owner + 4g + i, row) -> bf16(h * (1 + scale)) pairs
// and per-row sums of squares of this column block, both under the tag of t_hs
template <int t_hs, int t_ss>
__device__ inline void owner_publish(Ctx& c, const f32x4& h, const u32x4& sv, unsigned slot) {
  const int j = c.owner;
  const unsigned tag = tag_of(c, slot, t_hs);
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = h[i] * (1.0f + as_f(sv[i]));
  float s = h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3];
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  if (c.row < c.R) {
    ll_store2(c, xoff<t_hs>(slot) + ((unsigned)c.row * (D / 2) + (unsigned)(8 * j + 2 * c.g)) * 8u,
              pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), tag);
    if (c.g == 0) ll_store1(c, xoff<t_ss>(slot) + ((unsigned)c.row * NTD + (unsigned)j) * 8u, as_u(s), tag);
  }
}

// phase timeline (off unless the handle asked for it)
__device__ inline void tl_mark(const Ctx& c, int ev) {
  if (c.tl != 0u && c.lane == 0) {
    const unsigned idx = (blockIdx.x * (unsigned)timeline_events(c.S, c.NL) + (unsigned)ev) * 4u;
    __builtin_amdgcn_raw_buffer_store_b32(now_ticks(), c.X, AUX0 + aux_timeline(c.S, c.NL) + idx, 0, 0);
  }
}

// ------------------------------------------------------------- phases
// Every phase is entered by all four compute waves; barrier counts match.
// Each phase issues all the loads it needs (tables first, then the exchange
// words) before waiting on any of them.

// input projection h = x . W_in for the owner's column block (one k-tile)
__device__ __attribute__((always_inline)) inline void ph_in(Ctx& c, int k, f32x4& hreg) {
  refresh(c);
  if (c.owner < 0 || c.wave != 0) return;
  const unsigned p0 = (unsigned)k * c.n_step;
  const u32x4 sv = owner_scale_load(c, k, 0);
  bf16x8 b;
  if (k == 0) {
    const bool ok = c.row < c.R;
    const unsigned off = AUX0 + AUX_X + ((unsigned)c.row * A + 8u * (unsigned)c.g) * 4u;
    const u32x4 v0 = ok ? __builtin_amdgcn_raw_buffer_load_b128(c.X, off, 0, 0) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 v1 = ok ? __builtin_amdgcn_raw_buffer_load_b128(c.X, off + 16u, 0, 0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b[i] = (bf16)as_f(v0[i]);
      b[4 + i] = (bf16)as_f(v1[i]);
    }
  } else {
    u32x4 v[2];
    const unsigned slot = slot_of(c, k - 1, c.NL);
    const PB pb{((unsigned)c.crow * (A / 2) + 4u * (unsigned)c.g) * 8u, 0u, xoff<X_X>(slot), 0u, 0u};
    ll_poll<2>(c, pb, [](const PB& b, int i) { return frag_la(b.v0, b.s0, 0u, i); }, tag_of(c, slot, X_X), v);
    b = frag_of(v[0], v[1]);
  }
  wait_tiles(c, p0, 1);
  hreg = mma32(ring_tile(c, p0), b, f32x4{0.f, 0.f, 0.f, 0.f});
  release_ring(c, p0 + 1);
  owner_publish<X_HS, X_SS>(c, hreg, sv, slot_of(c, k, 0));
}

// QKV projection of two n-tiles, K = D split over the four waves; epilogue
// 1/rms, shift . W, RoPE; writes q (per head), k and v of the action rows
__device__ __attribute__((always_inline)) inline void ph_qkv(Ctx& c, int k, int l) {
  refresh(c);
  if (c.qkv0 < 0) return;
  const unsigned slot = slot_of(c, k, l);
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer;
  // epilogue tables of this wave's n-tile (waves 0 and 1 reduce n-tiles 0 and 1)
  const int nt = c.qkv0 + (c.wave & 1);
  const int tt = nt % 16, hh = nt / 16;
  const u32x4 sw = __builtin_amdgcn_raw_buffer_load_b128(
      c.X, step_tab(c, k) + st_swqkv(c.NL) + (unsigned)((l * NQKV + nt * 16 + 4 * c.g) * 4), 0, 0);
  const u32x4 cs = __builtin_amdgcn_raw_buffer_load_b128(
      c.X, AUX0 + AUX_ROPE + (unsigned)((c.row * (DH / 2) + 8 * tt + 2 * c.g) * 8), 0, 0);
  u32x4 v[24];
  poll_normed<X_HS, X_SS>(c, slot, v);
  wait_tiles(c, p0, 64);
  f32x4 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      acc[t] = mma32(ring_tile(c, p0 + 32u * t + 8u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc[t]);
  }
  f32x4* red = red_take(c);
#pragma unroll
  for (int t = 0; t < 2; ++t) red[(c.wave * 4 + t) * 64 + c.lane] = acc[t];
  cw_barrier(c);
  release_ring(c, p0 + 64u);
  if (c.wave < 2) {
    const f32x4 s = red_sum(red, c.wave, c.lane);
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
    if (c.row < c.R) {
      const unsigned tag = tag_of(c, slot, X_Q);
      const unsigned hb = xoff<X_Q>(slot) + ((unsigned)(hh * RP + c.row) * (DH / 2)) * 8u;
      ll_store1(c, hb + (unsigned)(4 * tt + c.g) * 8u, pack_bf16(y[0], y[1]), tag);
      ll_store1(c, hb + (unsigned)(64 + 4 * tt + c.g) * 8u, pack_bf16(y[2], y[3]), tag);
    }
  }
}

// outputs of one (head, chunk): unnormalised O [row][dim] and (max, sum) per row
__device__ inline void attn_publish(Ctx& c, unsigned slot, const f32x4 (&oacc)[4], float m_row, float l_row) {
  const unsigned tag = tag_of(c, slot, X_ATT);
  const unsigned ob = xoff<X_ATT>(slot);
  const unsigned hc = (unsigned)(c.attn_h * MAX_CHUNKS + c.attn_c);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int dim = 16 * (4 * c.wave + d) + c.row;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rw = 4 * c.g + i;
      if (rw < c.R) ll_store1(c, ob + ((hc * RP + (unsigned)rw) * DH + (unsigned)dim) * 8u, as_u(oacc[d][i]), tag);
    }
  }
  if (c.wave == 0 && c.g == 0 && c.row < c.R)
    ll_store2(c, ob + X_ML + ((hc * RP + (unsigned)c.row) * 2u) * 8u, as_u(m_row), as_u(l_row), tag);
}

// attention of head h over one prefix key chunk [64 c, 64 c + 64) from the ring
__device__ __attribute__((always_inline)) inline void ph_attn_prefix(Ctx& c, int k, int l) {
  refresh(c);
  const unsigned slot = slot_of(c, k, l);
  const float scale = 0.0625f;  // 1/sqrt(256)
  const unsigned vo = ((unsigned)c.crow * (DH / 2) + 4u * (unsigned)c.g) * 8u;
  // q of this head as 8 B fragments (dims 32 s + 8 g + [0, 8)): wave w polls
  // fragments 2w, 2w + 1 and the four waves share them through LDS
  bf16x8 qf[8];
  {
    u32x4 v[4];
    const PB pb{vo, 0u, xoff<X_Q>(slot) + (unsigned)(c.attn_h * RP) * (DH / 2) * 8u + 256u * (unsigned)c.wave, 0u, 0u};
    ll_poll<4>(c, pb, [](const PB& b, int i) { return frag_la(b.v0, b.s0, 128u, i); }, tag_of(c, slot, X_Q), v);
    u32x4* qs = (u32x4*)red_take(c);  // [8 fragments][64 lanes]
    qs[(2 * c.wave) * 64 + c.lane] = __builtin_bit_cast(u32x4, frag_of(v[0], v[1]));
    qs[(2 * c.wave + 1) * 64 + c.lane] = __builtin_bit_cast(u32x4, frag_of(v[2], v[3]));
    cw_barrier(c);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, qs[s * 64 + c.lane]);
  }
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer + c.o_attn;
  wait_tiles(c, p0, 64);
  // S^T for keys [16 w, 16 w + 16) of the chunk: lane holds keys 4g + i of row `row`
  f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) st = mma32(ring_tile(c, p0 + 8u * c.wave + s), qf[s], st);
  float sv[4];
  float mw = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = CHUNK * c.attn_c + 16 * c.wave + 4 * c.g + i;
    sv[i] = key < c.L ? st[i] * scale : -INFINITY;
    mw = fmaxf(mw, sv[i]);
  }
  mw = fmaxf(mw, __shfl_xor(mw, 16));
  mw = fmaxf(mw, __shfl_xor(mw, 32));
  if (c.g == 0) c.sh->att_m[c.wave][c.row] = mw;
  cw_barrier(c);
  const float m_row = fmaxf(fmaxf(c.sh->att_m[0][c.row], c.sh->att_m[1][c.row]),
                            fmaxf(c.sh->att_m[2][c.row], c.sh->att_m[3][c.row]));
  float lw = 0.f;
  s16x4 pf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = sv[i] == -INFINITY ? 0.f : fexp(sv[i] - m_row);
    lw += p;
    pf[i] = as_s((bf16)p);
  }
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  if (c.g == 0) c.sh->att_l[c.wave][c.row] = lw;
  c.sh->att_p[c.wave][c.lane] = pf;
  cw_barrier(c);
  const float l_row = (c.sh->att_l[0][c.row] + c.sh->att_l[1][c.row]) + (c.sh->att_l[2][c.row] + c.sh->att_l[3][c.row]);
  // O = P . V for dim tiles [4 w, 4 w + 4), all four key groups
  f32x4 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
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
  cw_barrier(c);
  release_ring(c, p0 + 64u);
  attn_publish(c, slot, oacc, m_row, l_row);
}

// attention of head h over the action rows' own keys and values.  Wave w
// polls its quarter of the head dims of q and of the keys (k-tiles 2w, 2w + 1)
// and value rows w, w + 4, w + 8, w + 12; the four partial score tiles are
// summed in LDS in wave order, and the values are staged there transposed
// for the P . V fragments.
__device__ __attribute__((always_inline)) inline void ph_attn_action(Ctx& c, int k, int l) {
  refresh(c);
  const unsigned slot = slot_of(c, k, l);
  const float scale = 0.0625f;
  f32x4* red = red_take(c);
  unsigned short* va = (unsigned short*)red;  // [DH][RP] bf16 values, transposed
  f32x4* sp = red + DH * RP * 2 / 16;         // [4 waves][64 lanes] partial score tiles
  {
    const int t = c.wave * 64 + c.lane;  // 256 threads: thread t clears dims t
#pragma unroll
    for (int key = 0; key < RP; ++key) va[t * RP + key] = 0;
  }
  u32x4 v[12];
  {
    const unsigned qb = xoff<X_Q>(slot);
    const int R = c.R, w = c.wave;
    const PB pb{((unsigned)c.crow * (DH / 2) + 4u * (unsigned)c.g) * 8u,
                ((unsigned)w * (DH / 2) + 2u * (unsigned)c.lane) * 8u,
                qb + (unsigned)(c.attn_h * RP) * (DH / 2) * 8u + 256u * (unsigned)w,
                qb + (unsigned)(H * RP) * (DH / 2) * 8u + 256u * (unsigned)w, qb + (unsigned)((H + 1) * RP) * (DH / 2) * 8u};
    auto addr = [&](const PB& b, int i) -> LA {
      if (i < 4) return frag_la(b.v0, b.s0, 128u, i);
      if (i < 8) return frag_la(b.v0, b.s1, 128u, i - 4);
      return LA{b.v1, b.s2 + (unsigned)(4 * (i - 8)) * (DH / 2) * 8u, w + 4 * (i - 8) < R};
    };
    ll_poll<12>(c, pb, addr, tag_of(c, slot, X_Q), v);
  }
  f32x4 st = mma32(frag_of(v[4], v[5]), frag_of(v[0], v[1]), f32x4{0.f, 0.f, 0.f, 0.f});
  st = mma32(frag_of(v[6], v[7]), frag_of(v[2], v[3]), st);
  cw_barrier(c);  // staging area cleared by every wave
  sp[c.wave * 64 + c.lane] = st;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = c.wave + 4 * i;
    if (key < c.R) {
      const int d0 = 4 * c.lane;  // pair words 2 lane, 2 lane + 1 -> dims 4 lane .. 4 lane + 3
      va[(d0 + 0) * RP + key] = (unsigned short)(v[8 + i][0] & 0xffffu);
      va[(d0 + 1) * RP + key] = (unsigned short)(v[8 + i][0] >> 16);
      va[(d0 + 2) * RP + key] = (unsigned short)(v[8 + i][2] & 0xffffu);
      va[(d0 + 3) * RP + key] = (unsigned short)(v[8 + i][2] >> 16);
    }
  }
  cw_barrier(c);
  st = ((sp[0 * 64 + c.lane] + sp[1 * 64 + c.lane]) + sp[2 * 64 + c.lane]) + sp[3 * 64 + c.lane];
  float sv[4];
  float mw = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = 4 * c.g + i;
    sv[i] = key < c.R ? st[i] * scale : -INFINITY;
    mw = fmaxf(mw, sv[i]);
  }
  mw = fmaxf(mw, __shfl_xor(mw, 16));
  mw = fmaxf(mw, __shfl_xor(mw, 32));
  const float m_row = mw;
  float lw = 0.f;
  s16x4 pf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = sv[i] == -INFINITY ? 0.f : fexp(sv[i] - m_row);
    lw += p;
    pf[i] = as_s((bf16)p);
  }
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  f32x4 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int dim = 16 * (4 * c.wave + d) + c.row;
    const s16x4 b = *(const s16x4*)(va + dim * RP + 4 * c.g);
    oacc[d] = mma16(pf, b, f32x4{0.f, 0.f, 0.f, 0.f});
  }
  attn_publish(c, slot, oacc, m_row, lw);
}

// merges the key chunks of head h for dims [32 s, 32 s + 32) and writes the
// normalised attention output as bf16 pairs.  Wave w polls chunks w, w + 4,
// w + 8, w + 12: per chunk one load of the (max, sum) pairs (lane: row
// lane % 16) and four loads of dims 32 s + 2 dp, + 1 of rows rg + 4 j.  The
// (max, sum) pairs go to LDS; every lane then forms the row statistics over
// all chunks and the weight exp(m_c - M) / L of each of its (chunk, row)
// pairs once, so the merge itself is plain multiply-adds.  The four waves'
// partial sums meet in LDS and each wave finishes one row group.
__device__ __attribute__((always_inline)) inline void ph_comb(Ctx& c, int k, int l) {
  refresh(c);
  if (c.comb_h < 0) return;
  const int hd = c.comb_h, sl = c.comb_s;
  const int nch = c.nc + 1;
  const unsigned slot = slot_of(c, k, l);
  const unsigned tag = tag_of(c, slot, X_ATT);
  const unsigned ob = xoff<X_ATT>(slot);
  const unsigned mlb = ob + X_ML;
  const int dp = c.lane & 15, rg = c.lane >> 4;
  const int R = c.R;
  f32x4* red = red_take(c);
  float* mls = (float*)red;                       // [MAX_CHUNKS][RP] max, then [MAX_CHUNKS][RP] sum
  f32x4* part = red + (2 * MAX_CHUNKS * RP) / 4;  // [4 waves][2][64 lanes] partial sums (rows rg + 4i, 2 dims)
  const int base = c.wave;
  u32x4 v[20];
  {
    const int mrow = dp < R ? dp : R - 1;
    const PB pb{(unsigned)mrow * 16u, (unsigned)(2 * dp) * 8u, mlb + (unsigned)(hd * MAX_CHUNKS + base) * RP * 16u,
                ob + ((unsigned)(hd * MAX_CHUNKS + base) * RP * DH + 32u * (unsigned)sl) * 8u, (unsigned)base};
    auto addr = [&](const PB& b, int i) -> LA {
      const int q = i / 5, j = i % 5;
      const bool need = (int)b.s2 + NCOMPUTE * q < nch;
      if (j == 0) return LA{b.v0, b.s0 + (unsigned)(NCOMPUTE * q) * RP * 16u, need};
      const int rw = rg + 4 * (j - 1);
      const unsigned row = (unsigned)(rw < R ? rw : R - 1);
      return LA{b.v1 + row * DH * 8u, b.s1 + (unsigned)(NCOMPUTE * q) * RP * DH * 8u, need};
    };
    ll_poll<20>(c, pb, addr, tag, v);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int cc = base + NCOMPUTE * q;
    if (cc < nch && c.lane < RP) {
      mls[cc * RP + c.lane] = as_f(v[5 * q][0]);
      mls[(MAX_CHUNKS + cc) * RP + c.lane] = as_f(v[5 * q][2]);
    }
  }
  cw_barrier(c);
  // statistics of row lane % 16 over every chunk (a chunk without valid keys has max -inf and sum 0)
  float M = -INFINITY;
  for (int cc = 0; cc < nch; ++cc) M = fmaxf(M, mls[cc * RP + dp]);
  float L = 0.f;
  for (int cc = 0; cc < nch; ++cc) {
    const float m = mls[cc * RP + dp];
    if (m != -INFINITY) L += fexp(m - M) * mls[(MAX_CHUNKS + cc) * RP + dp];
  }
  const float invL = frcp(L);
  float acc0[4], acc1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rg + 4 * i;
    const float Mr = __shfl(M, row), iLr = __shfl(invL, row);
    acc0[i] = acc1[i] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = base + NCOMPUTE * q;
      if (cc < nch) {
        const float m = mls[cc * RP + row];
        const float wgt = m == -INFINITY ? 0.f : fexp(m - Mr) * iLr;
        acc0[i] += wgt * as_f(v[5 * q + 1 + i][0]);
        acc1[i] += wgt * as_f(v[5 * q + 1 + i][2]);
      }
    }
  }
  part[(c.wave * 2 + 0) * 64 + c.lane] = f32x4{acc0[0], acc1[0], acc0[1], acc1[1]};
  part[(c.wave * 2 + 1) * 64 + c.lane] = f32x4{acc0[2], acc1[2], acc0[3], acc1[3]};
  cw_barrier(c);
  {
    // wave w finishes rows rg + 4w of every lane's dims, summing the waves in order
    const int i = c.wave;
    const float* pf = (const float*)part;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int w = 0; w < NCOMPUTE; ++w) {
      const float* e = pf + ((w * 2 + (i >> 1)) * 64 + c.lane) * 4 + 2 * (i & 1);
      a0 += e[0];
      a1 += e[1];
    }
    const int rw = rg + 4 * i;
    if (rw < R)
      ll_store1(c, xoff<X_O>(slot) + ((unsigned)rw * (HD / 2) + (unsigned)(hd * (DH / 2) + 16 * sl + dp)) * 8u,
                pack_bf16(a0, a1), tag_of(c, slot, X_O));
  }
}

// out projection of the owner's column block (K = H*DH over the four waves),
// residual add, and the MLP norm's producer half
__device__ __attribute__((always_inline)) inline void ph_o(Ctx& c, int k, int l, f32x4& hreg) {
  refresh(c);
  if (c.owner < 0) return;
  const unsigned slot = slot_of(c, k, l);
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer + c.o_o;
  const u32x4 sv = owner_scale_load(c, k, 2 * l + 1);
  u32x4 v[32];
  {
    const PB pb{((unsigned)c.crow * (HD / 2) + 4u * (unsigned)c.g) * 8u, 0u,
                xoff<X_O>(slot) + (unsigned)(16 * c.wave) * 128u, 0u, 0u};
    ll_poll<32>(c, pb, [](const PB& b, int i) { return frag_la(b.v0, b.s0, 128u, i); }, tag_of(c, slot, X_O), v);
  }
  wait_tiles(c, p0, 64);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 16; ++kk)
    acc = mma32(ring_tile(c, p0 + 16u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc);
  f32x4* red = red_take(c);
  red[(c.wave * 4) * 64 + c.lane] = acc;
  cw_barrier(c);
  release_ring(c, p0 + 64u);
  if (c.wave == 0) {
    hreg += red_sum(red, 0, c.lane);
    owner_publish<X_HS1, X_SS1>(c, hreg, sv, slot);
  }
}

// gate/up projection of two n-tiles with the GeGLU epilogue
__device__ __attribute__((always_inline)) inline void ph_gu(Ctx& c, int k, int l) {
  refresh(c);
  const unsigned slot = slot_of(c, k, l);
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer + c.o_gu;
  const int nt = 2 * (int)blockIdx.x + (c.wave & 1);
  const u32x4 sw = __builtin_amdgcn_raw_buffer_load_b128(
      c.X, step_tab(c, k) + st_swgu(c.NL) + (unsigned)((l * 2 * F + nt * 16 + 4 * c.g) * 4), 0, 0);
  u32x4 v[24];
  poll_normed<X_HS1, X_SS1>(c, slot, v);
  wait_tiles(c, p0, 64);
  f32x4 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      acc[t] = mma32(ring_tile(c, p0 + 32u * t + 8u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc[t]);
  }
  f32x4* red = red_take(c);
#pragma unroll
  for (int t = 0; t < 2; ++t) red[(c.wave * 4 + t) * 64 + c.lane] = acc[t];
  cw_barrier(c);
  release_ring(c, p0 + 64u);
  if (c.wave < 2) {
    const f32x4 s = red_sum(red, c.wave, c.lane);
    const float rr = c.sh->rrow[c.row];
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = rr * s[i] + as_f(sw[i]);
    const float a0 = gelu_tanh(y[0]) * y[2];
    const float a1 = gelu_tanh(y[1]) * y[3];
    if (c.row < c.R)
      ll_store1(c, xoff<X_A>(slot) + ((unsigned)c.row * (F / 2) + (unsigned)(4 * nt + c.g)) * 8u, pack_bf16(a0, a1),
                tag_of(c, slot, X_A));
  }
}

// down projection: K group kq (8 k-tiles, two per wave) x N group nq (4 n-tiles)
__device__ __attribute__((always_inline)) inline void ph_down(Ctx& c, int k, int l) {
  refresh(c);
  const int kq = (int)blockIdx.x / DN_NQ, nqd = (int)blockIdx.x % DN_NQ;
  const unsigned slot = slot_of(c, k, l);
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)l * c.n_layer + c.o_dn;
  u32x4 v[4];
  {
    const PB pb{((unsigned)c.crow * (F / 2) + 4u * (unsigned)c.g) * 8u, 0u,
                xoff<X_A>(slot) + (unsigned)(8 * kq + 2 * c.wave) * 128u, 0u, 0u};
    ll_poll<4>(c, pb, [](const PB& b, int i) { return frag_la(b.v0, b.s0, 128u, i); }, tag_of(c, slot, X_A), v);
  }
  wait_tiles(c, p0, 32);
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      acc[t] = mma32(ring_tile(c, p0 + 8u * t + 2u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc[t]);
  }
  f32x4* red = red_take(c);
#pragma unroll
  for (int t = 0; t < 4; ++t) red[(c.wave * 4 + t) * 64 + c.lane] = acc[t];
  cw_barrier(c);
  release_ring(c, p0 + 32u);
  const f32x4 s = red_sum(red, c.wave, c.lane);
  if (c.row < c.R) {
    const int col = 16 * (4 * nqd + c.wave) + 4 * c.g;
    const unsigned o = xoff<X_DP>(slot) + (((unsigned)kq * RP + (unsigned)c.row) * D + (unsigned)col) * 8u;
    const unsigned tag = tag_of(c, slot, X_DP);
    ll_store2(c, o, as_u(s[0]), as_u(s[1]), tag);
    ll_store2(c, o + 16u, as_u(s[2]), as_u(s[3]), tag);
  }
}

// residual add of the 16 down partials of the owner's block, and the next
// norm's producer half (the next layer's attention norm, or the final norm)
__device__ __attribute__((always_inline)) inline void ph_owner2(Ctx& c, int k, int l, f32x4& hreg) {
  refresh(c);
  if (c.owner < 0) return;
  const int j = c.owner;
  const unsigned slot = slot_of(c, k, l);
  const u32x4 sv = owner_scale_load(c, k, 2 * (l + 1));
  u32x4 v[8];
  {
    const PB pb{((unsigned)c.crow * D + (unsigned)(16 * j + 4 * c.g)) * 8u, 0u,
                xoff<X_DP>(slot) + (unsigned)(4 * c.wave) * (RP * D * 8u), 0u, 0u};
    // partial K groups are RP * D words apart: too far for an immediate, so they step the uniform base
    ll_poll<8>(c, pb, [](const PB& b, int i) {
      return LA{b.v0 + (unsigned)(i & 1) * 16u, b.s0 + (unsigned)(i >> 1) * (RP * D * 8u), true};
    }, tag_of(c, slot, X_DP), v);
  }
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[0] += as_f(v[2 * i][0]);
    s[1] += as_f(v[2 * i][2]);
    s[2] += as_f(v[2 * i + 1][0]);
    s[3] += as_f(v[2 * i + 1][2]);
  }
  f32x4* red = red_take(c);
  red[(c.wave * 4) * 64 + c.lane] = s;
  cw_barrier(c);
  if (c.wave == 0) {
    hreg += red_sum(red, 0, c.lane);
    owner_publish<X_HS, X_SS>(c, hreg, sv, slot + 1u);
  }
}

// velocity head of one n-tile (K = D over the four waves), final norm's
// consumer half, and the Euler update of the owned state columns
__device__ __attribute__((always_inline)) inline void ph_out(Ctx& c, int k, f32x4& xreg) {
  refresh(c);
  if (c.out_nt < 0) return;
  const int NL = c.NL;
  const unsigned slot = slot_of(c, k, NL);
  const unsigned p0 = (unsigned)k * c.n_step + c.n_in + (unsigned)NL * c.n_layer;
  const int t = c.out_nt;
  const u32x4 sw = __builtin_amdgcn_raw_buffer_load_b128(
      c.X, step_tab(c, k) + st_swout(NL) + (unsigned)((16 * t + 4 * c.g) * 4), 0, 0);
  u32x4 v[24];
  poll_normed<X_HS, X_SS>(c, slot, v);
  wait_tiles(c, p0, 32);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) acc = mma32(ring_tile(c, p0 + 8u * c.wave + kk), frag_of(v[2 * kk], v[2 * kk + 1]), acc);
  f32x4* red = red_take(c);
  red[(c.wave * 4) * 64 + c.lane] = acc;
  cw_barrier(c);
  release_ring(c, p0 + 32u);
  if (c.wave == 0) {
    const f32x4 s = red_sum(red, 0, c.lane);
    const float rr = c.sh->rrow[c.row];
#pragma unroll
    for (int i = 0; i < 4; ++i) xreg[i] += c.dt * (rr * s[i] + as_f(sw[i]));
    if (c.row < c.R) {
      if (k + 1 < c.S) {
        ll_store2(c, xoff<X_X>(slot) + ((unsigned)c.row * (A / 2) + (unsigned)(8 * t + 2 * c.g)) * 8u,
                  pack_bf16(xreg[0], xreg[1]), pack_bf16(xreg[2], xreg[3]), tag_of(c, slot, X_X));
      } else {
        const u32x4 xv = {as_u(xreg[0]), as_u(xreg[1]), as_u(xreg[2]), as_u(xreg[3])};
        __builtin_amdgcn_raw_buffer_store_b128(xv, c.X, AUX0 + AUX_X + (unsigned)((c.row * A + 16 * t + 4 * c.g) * 4),
                                               0, 0);
      }
    }
  }
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

// run 0: input projection; 1 + 8 l + u: layer l part u (QKV, prefix K/V, O,
// gate/up, down n-tiles 0..3); 1 + 8 NL: velocity head
__device__ inline void run_params(const Ctx& c, int run, unsigned& off, int& cnt, int& kv) {
  kv = 0;
  cnt = 0;
  off = 0;
  const int NL = c.NL;
  if (run == 0) {
    if (c.owner >= 0) {
      cnt = 1;
      off = (unsigned)c.owner * TILE_BYTES;
    }
    return;
  }
  if (run == 1 + 8 * NL) {
    if (c.out_nt >= 0) {
      cnt = 32;
      off = (unsigned)((w_out(NL) + (unsigned long long)c.out_nt * KT_D * TILE_ELEMS) * 2ull);
    }
    return;
  }
  const int l = (run - 1) / 8, u = (run - 1) % 8;
  const unsigned long long lo = (unsigned long long)l * W_LAYER;
  if (u == 0) {
    if (c.qkv0 >= 0) {
      cnt = 64;
      off = (unsigned)((W_QKV0 + lo + (unsigned long long)c.qkv0 * KT_D * TILE_ELEMS) * 2ull);
    }
  } else if (u == 1) {
    if (c.attn_c >= 0 && c.attn_c < c.nc) {
      cnt = 64;
      kv = 1;
      off = (unsigned)((l * c.nc + c.attn_c) * 64) * TILE_BYTES;
    }
  } else if (u == 2) {
    if (c.owner >= 0) {
      cnt = 64;
      off = (unsigned)((W_O0 + lo + (unsigned long long)c.owner * KT_HD * TILE_ELEMS) * 2ull);
    }
  } else if (u == 3) {
    cnt = 64;
    off = (unsigned)((W_GU0 + lo + (unsigned long long)(2 * blockIdx.x) * KT_D * TILE_ELEMS) * 2ull);
  } else {
    const int t = u - 4;
    const int kq = (int)blockIdx.x / DN_NQ, nqd = (int)blockIdx.x % DN_NQ;
    cnt = 8;
    off = (unsigned)((W_DN0 + lo + ((unsigned long long)(4 * nqd + t) * KT_F + 8 * kq) * TILE_ELEMS) * 2ull);
  }
}

// next (position, byte offset, source) of loader q; false at the end
__device__ inline bool gen_next(const Ctx& c, Gen& s, int q, unsigned& pos, unsigned& off, int& kv) {
  const int runs_per_step = 2 + 8 * c.NL;
  while (s.j >= s.cnt) {
    s.pos0 += (unsigned)s.cnt;
    s.run += 1;
    if (s.run >= runs_per_step) {
      s.run = 0;
      s.k += 1;
      if (s.k >= c.S) return false;
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

constexpr unsigned LOAD_DEPTH = 24;  // tiles in flight per loader wave (16 measured 2% slower; 28, 32 the same)

// Loader waves wait on LDS only: a global load in their wait loop would make
// the next use of any loaded register wait for the whole batch of tile loads
// (loads complete in order).  They leave on their workgroup's abort flag; on
// their own time limit they record the failure and raise the flag.
__device__ inline void loader_keep_waiting(Ctx& c, unsigned t0, unsigned& spins) {
  ++spins;
  if (lds_load(&c.sh->abort) != 0u) end_wave();
  if ((spins & 63u) == 0u && now_ticks() - t0 > TIMEOUT_TICKS) {
    lds_store(&c.sh->abort, 1u);
    if (c.lane == 0) __builtin_amdgcn_raw_buffer_store_b32(c.seq + 1u, c.X, AUX0 + AUX_STATUS, 0, SC1);
    end_wave();
  }
}

__device__ __attribute__((always_inline)) inline void loader(Ctx& c, int q, const Args& a) {
  const u32x4 WR = rsrc_words(a.wt, a.wt_bytes);
  const u32x4 KR = rsrc_words(a.kvt, a.kvt_bytes);
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
      while (pos >= lds_load(&c.sh->consumed) + RING) {
        __builtin_amdgcn_s_sleep(2);
        loader_keep_waiting(c, t0, spins);
      }
    }
    cbar();
    const unsigned lds = __builtin_amdgcn_readfirstlane(ring_lds + (pos % RING) * TILE_BYTES);
    if (kv)
      dma_tile(KR, (unsigned)c.lane * 16u, off, lds, false);
    else
      dma_tile(WR, (unsigned)c.lane * 16u, off, lds, true);
    ++issued;
    if (issued > LOAD_DEPTH) {
      asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
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
  c.sh = &sh;
  c.ring = ring_mem;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform per wave
  c.g = c.lane >> 4;
  c.row = c.lane & 15;
  c.barn = 0;
  c.redsel = 0;
  c.S = a.S;
  c.NL = a.NL;
  c.R = a.R;
  c.nc = a.n_chunks;
  c.dt = a.dt;
  c.eps = a.eps;
  c.tl = a.tl;
  if (threadIdx.x < 32) ((unsigned*)&sh)[threadIdx.x] = 0u;
  c.X = rsrc(a.arena, a.arena_bytes);
  c.seq = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(c.X, AUX0 + AUX_SEQ, 0, SC1));
  c.tagbase = c.seq * exchanges_per_decision(c.S, c.NL);
  c.L = __builtin_amdgcn_readfirstlane((int)__builtin_amdgcn_raw_buffer_load_b32(c.X, AUX0 + AUX_LENS, 0, 0));
  set_roles(c, (int)blockIdx.x);
  c.crow = c.row < c.R ? c.row : c.R - 1;
  // stream layout of this workgroup (must match run_params)
  c.n_in = c.owner >= 0 ? 1u : 0u;
  c.o_attn = c.qkv0 >= 0 ? 64u : 0u;
  c.o_o = c.o_attn + ((c.attn_c >= 0 && c.attn_c < c.nc) ? 64u : 0u);
  c.o_gu = c.o_o + (c.owner >= 0 ? 64u : 0u);
  c.o_dn = c.o_gu + 64u;
  c.n_layer = c.o_dn + 32u;
  c.n_step = c.n_in + (unsigned)c.NL * c.n_layer + (c.out_nt >= 0 ? 32u : 0u);
  __syncthreads();

  if (c.wave >= NCOMPUTE) {
    loader(c, c.wave - NCOMPUTE, a);
    if (c.wave == NCOMPUTE) tl_mark(c, timeline_events(c.S, c.NL) - 1);
    return;
  }
  f32x4 hreg = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 xreg = f32x4{0.f, 0.f, 0.f, 0.f};
  if (c.out_nt >= 0 && c.wave == 0 && c.row < c.R) {
    const u32x4 xv = __builtin_amdgcn_raw_buffer_load_b128(
        c.X, AUX0 + AUX_X + (unsigned)((c.row * A + 16 * c.out_nt + 4 * c.g) * 4), 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) xreg[i] = as_f(xv[i]);
  }
  const bool tl = c.wave == 0;
  const bool attends = c.attn_c >= 0;
  const bool action_chunk = c.attn_c == c.nc;
  if (tl) tl_mark(c, 0);
  for (int k = 0; k < c.S; ++k) {
    const int e0 = 1 + k * (2 + 7 * c.NL);
    ph_in(c, k, hreg);
    if (tl) tl_mark(c, e0);
    for (int l = 0; l < c.NL; ++l) {
      const int el = e0 + 1 + 7 * l;
      ph_qkv(c, k, l);
      if (tl) tl_mark(c, el);
      if (attends) {
        if (action_chunk)
          ph_attn_action(c, k, l);
        else
          ph_attn_prefix(c, k, l);
      }
      if (tl) tl_mark(c, el + 1);
      ph_comb(c, k, l);
      if (tl) tl_mark(c, el + 2);
      ph_o(c, k, l, hreg);
      if (tl) tl_mark(c, el + 3);
      ph_gu(c, k, l);
      if (tl) tl_mark(c, el + 4);
      ph_down(c, k, l);
      if (tl) tl_mark(c, el + 5);
      ph_owner2(c, k, l, hreg);
      if (tl) tl_mark(c, el + 6);
    }
    ph_out(c, k, xreg);
    if (tl) tl_mark(c, e0 + 1 + 7 * c.NL);
  }
  if (tl) tl_mark(c, timeline_events(c.S, c.NL) - 2);
}

__global__ void k_decide_advance(unsigned* seq) {
  if (threadIdx.x == 0 && blockIdx.x == 0) seq[0] = seq[0] + 1u;
}

static hipError_t allow_ring_lds() {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_decide, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       RING * TILE_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  return hipSuccess;
}

hipError_t decide_occupancy(int* blocks_per_cu) {
  hipError_t e = allow_ring_lds();
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)k_decide, THREADS,
                                                       RING * TILE_BYTES);
}

hipError_t launch_decide(const Args& a, hipStream_t s) {
  hipError_t e = allow_ring_lds();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decide, dim3(G), dim3(THREADS), RING * TILE_BYTES, s, a);
  return hipGetLastError();
}

hipError_t launch_decide_advance(void* arena, hipStream_t s) {
  hipLaunchKernelGGL(k_decide_advance, dim3(1), dim3(64), 0, s, (unsigned*)((char*)arena + AUX0 + AUX_SEQ));
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
                              float* __restrict__ out, size_t out_kstride) {
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
    out[(size_t)k * out_kstride + (size_t)l * N + n] = (float)acc;
  }
}

hipError_t launch_shift_table(const void* w0, long long w_lstride, const float* modtab, int NN, int norm_stride,
                              int norm_off, int S, int nl, int N, int colkind, int colparam, float* out,
                              size_t out_kstride, hipStream_t s) {
  const size_t total = (size_t)S * nl * N;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_shift_table, dim3(blocks), dim3(256), 0, s, (const bf16*)w0, w_lstride, modtab, NN,
                     norm_stride, norm_off, S, nl, N, colkind, colparam, out, out_kstride);
  return hipGetLastError();
}

__global__ void k_scale_table(const float* __restrict__ modtab, int S, int NN, unsigned char* __restrict__ arena,
                              int NL) {
  const size_t total = (size_t)S * NN * D;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int d = (int)(idx % D);
    const size_t kn = idx / D;
    const int nrm = (int)(kn % NN), k = (int)(kn / NN);
    float* dst = (float*)(arena + AUX0 + AUX_TAB + (size_t)k * step_bytes(NL));
    dst[(size_t)nrm * D + d] = modtab[((size_t)k * NN + nrm) * 2 * D + d];
  }
}

hipError_t launch_scale_table(const float* modtab, int S, int NN, void* arena, int NL, hipStream_t s) {
  const size_t total = (size_t)S * NN * D;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_scale_table, dim3(blocks), dim3(256), 0, s, modtab, S, NN, (unsigned char*)arena, NL);
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
