// Persistent decision kernel for gfx950 (CDNA4): one launch runs all S Euler
// steps x NL layers of one request's action rows.
//
// Why persistent.  At 10 action rows every projection streams its weights
// once per step and does ~10 MACs per weight element, so a decision is bound
// by HBM bandwidth (6.37 GB per pi0.5 decision) and by the latency of the
// dependent exchanges between sublayers.  A graph of ~1100 small kernels pays
// a node gap plus ramp-up and drain at every boundary; the pages remove those
// gaps with programmatic dependent launch and by folding the "kernels between
// GEMMs" into GEMM prologues and epilogues ("FlashRT-PAI", sections 3.2-3.3;
// "PhyAI" section 4.2 Kernel fusion, Graph replay).  Here the same two ideas
// take a form that fits MI355X:
//   * loader waves (4 per workgroup) stream the workgroup's fixed share of
//     every weight matrix (and of the prefix K/V for attention workgroups)
//     into a 112-tile LDS ring, running up to a ring ahead of the compute, so
//     the HBM stream never waits for a sublayer boundary;
//   * compute waves (4 per workgroup) exchange activations with other
//     workgroups through self-tagged 4-byte words: a consumer sees data and
//     readiness in one load, and no barrier or atomic counter is needed.
//
// Layout over the chip.  Workgroup b runs on an XCD x it reads from the
// hardware, as rank r = b / 8 of that XCD's 32.  XCD x owns query head x and a 1/8 share of
// every projection: the QKV columns of head x plus 1/8 of the key and value
// columns, the out-projection rows of head x (a partial sum over the whole
// width), GeGLU features [512 x, 512 x + 512) (gate/up columns, and the same
// rows of the down projection: again a partial sum).  So the norm input ->
// QKV -> attention -> merge -> out projection and the MLP norm input ->
// gate/up -> down exchanges stay inside the XCD, in its L2 (plain stores,
// non-temporal loads), and only the two partial sums cross XCDs (device
// scope), where every XCD's 32 owners add the 8 partials of their 32 residual
// columns in the same order.  The residual stream is therefore replicated, bit-
// identically, in every XCD.  Every XCD also runs its own copy of the
// velocity head and keeps its own copy of the state x.
//
// Words.  An activation travels as a (hi, lo) pair of bf16 halves of one
// float (hi = bf16(a), lo = bf16(a - hi)): a GEMM multiplies both halves by
// the bf16 weights, so it sees the activation to about 2^-16 rather than
// bf16's 2^-8.  The lowest bit of every word is its buffer's generation: each
// buffer exists twice (use parity), and the generation flips every second
// use, so a word written in an earlier use never passes for a fresh one and
// no buffer is ever cleared.
//
// Fusions (the pages' "kernels between GEMMs"): the adaptive RMSNorm is split
// into the producer's epilogue (h * (1 + scale) and per-owner sums of
// squares) and the consumer's epilogue (row factor 1/rms and the shift term,
// added as the precomputed product shift . W); RoPE, GeGLU, residual adds and
// the Euler update are epilogues.  Reductions are in a fixed order, so
// replays are bit-identical.
//
// Every global access goes through a buffer resource; every wait is bounded
// by a wall-clock limit and an abort flag, so a missing producer ends the
// launch with a status instead of a hang.
#include "phx_decide.h"
#include "phx_internal.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <cstdio>
#include <cstdlib>
#include <mutex>

namespace phx {
namespace dec {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int SC1 = 16;                                  // cache policy: device-coherent access
constexpr int NTP = 2;                                   // load policy of XCD-local words: non-temporal (they
                                                         // bypass the CU's own cache and meet the L2 copy)
constexpr int LST = 0;                                   // store policy of XCD-local words: plain stores reach
                                                         // the XCD's L2 (non-temporal stores measured 6% slower)
constexpr unsigned OOB = 0x80000000u;                    // a buffer offset past every range: no access, zeros
constexpr unsigned TIMEOUT_TICKS = 50u * 1000u * 1000u;  // 0.5 s of the 100 MHz real-time counter
constexpr float M_EMPTY = -3.0e38f;                      // running max of a key chunk without valid keys

// LDS layout (static part; the ring is dynamic)
constexpr int RED_BYTES = 20 * 1024;  // per-phase scratch (partial tiles, staged fragments, statistics)

struct Shared {
  unsigned ready[NLOADER];   // tiles of each loader's sub-stream written to the ring
  unsigned consumed;         // ring positions below this are free
  unsigned abort;            // nonzero: leave now
  unsigned cwbar;            // compute-wave barrier counter
  unsigned pad[9];
  float rrow[RP];            // 1/rms per action row
  float att_m[NCOMPUTE][RP];
  float att_l[NCOMPUTE][RP];
  s16x4 att_p[NCOMPUTE][2][64];  // probability fragments (hi, lo) of each wave's 16 keys
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
__device__ inline unsigned short bits16(bf16 b) { return __builtin_bit_cast(unsigned short, b); }

// Hardware exp2 / reciprocal / reciprocal square root (about 1 ulp).
__device__ inline float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ inline float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ inline float frsq(float x) { return __builtin_amdgcn_rsqf(x); }

// Cross-lane reductions without the LDS unit.  DPP moves within rows of 16
// lanes (quad permutations, half-row and row mirrors); the permlane swaps
// pair lanes l and l ^ 16, or l and l ^ 32, and every lane adds the two in
// the same order, so all lanes of a group hold identical bits.
template <int CTRL>
__device__ inline float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;
constexpr int DPP_ROW_SHARE0 = 0x150;  // row_share:n = 0x150 + n: lane n of each row to the row's 16 lanes
// sum over the 4 lanes of a quad
__device__ inline float sum_quad(float v) {
  v += dppf<DPP_XOR1>(v);
  return v + dppf<DPP_XOR2>(v);
}
// sum over the 16 lanes of a row
__device__ inline float sum_row16(float v) {
  v = sum_quad(v);
  v += dppf<DPP_HALF_MIRROR>(v);
  return v + dppf<DPP_MIRROR>(v);
}
// maximum over the 16 lanes of a row
__device__ inline float max_row16(float v) {
  v = fmaxf(v, dppf<DPP_XOR1>(v));
  v = fmaxf(v, dppf<DPP_XOR2>(v));
  v = fmaxf(v, dppf<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dppf<DPP_MIRROR>(v));
}
// sum and maximum over lanes l, l ^ 16, l ^ 32, l ^ 48
// (the value of lane l, that of lane l ^ 16) in the order (lower lane, upper
// lane) for every lane; the same with l ^ 32.  Written as assembly: the
// swap writes both of its registers, and the compiler's form of it has been
// seen to hand back one of the two results for both.
__device__ inline float2 swap16(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return float2{a, b};
}
__device__ inline float2 swap32(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return float2{a, b};
}
__device__ inline float sum_x16_x32(float v) {
  const float2 a = swap16(v);
  v = a.x + a.y;
  const float2 b = swap32(v);
  return b.x + b.y;
}
__device__ inline float max_x16_x32(float v) {
  const float2 a = swap16(v);
  v = fmaxf(a.x, a.y);
  const float2 b = swap32(v);
  return fmaxf(b.x, b.y);
}

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

// ------------------------------------------------------------- words

// (hi, lo) pair word of a with the generation bit in lo's last bit
__device__ inline unsigned pair_word(float a, unsigned gen) {
  const bf16 h = (bf16)a;
  const bf16 l = (bf16)(a - (float)h);
  return ((unsigned)bits16(h) << 16) | ((unsigned)bits16(l) & 0xfffeu) | gen;
}
// Norm inputs of the QKV projection and the velocity head travel as plain
// bf16, two columns per word: the odd column rounded to bf16 in the upper
// half, the even column in the lower half rounded to 6 fraction bits, the
// seventh carrying the generation.  (The MLP's norm input keeps pairs.)
__device__ inline unsigned bf16x2_word(float a0, float a1, unsigned gen) {
  const unsigned u0 = as_u(a0), u1 = as_u(a1);
  const unsigned lo = ((u0 + 0xffffu + ((u0 >> 17) & 1u)) >> 16) & 0xfffeu;
  const unsigned hi = (u1 + 0x7fffu + ((u1 >> 16) & 1u)) >> 16;
  return (hi << 16) | lo | gen;
}
// B fragment (8 consecutive k values) of 4 such words
__device__ inline bf16x8 frag_plain(const u32x4& v) {
  const u32x4 r = {v[0] & ~1u, v[1] & ~1u, v[2] & ~1u, v[3] & ~1u};
  return __builtin_bit_cast(bf16x8, r);
}
// float32 word with the generation bit in the last mantissa bit
__device__ inline unsigned f32_word(float a, unsigned gen) { return (as_u(a) & ~1u) | gen; }
// bf16 probability pair (hi, lo) for the P . V products
__device__ inline void split_bf16(float a, short& hi, short& lo) {
  const bf16 h = (bf16)a;
  hi = (short)bits16(h);
  lo = (short)bits16((bf16)(a - (float)h));
}
// value of a float32 word: the generation bit is dropped, so the value does
// not depend on which use of its buffer it travelled in (replays stay
// bit-identical)
__device__ inline float wf(unsigned w) { return as_f(w & ~1u); }
// B fragments (8 consecutive k values) of the hi and lo halves of 8 pair words
__device__ inline bf16x8 frag_hi(const u32x4& v0, const u32x4& v1) {
  const u32x4 r = {__builtin_amdgcn_perm(v0[1], v0[0], 0x07060302u), __builtin_amdgcn_perm(v0[3], v0[2], 0x07060302u),
                   __builtin_amdgcn_perm(v1[1], v1[0], 0x07060302u), __builtin_amdgcn_perm(v1[3], v1[2], 0x07060302u)};
  return __builtin_bit_cast(bf16x8, r);
}
// (the lo halves with their generation bit dropped)
__device__ inline bf16x8 frag_lo(const u32x4& v0, const u32x4& v1) {
  const unsigned m = 0xfffefffeu;
  const u32x4 r = {__builtin_amdgcn_perm(v0[1], v0[0], 0x05040100u) & m,
                   __builtin_amdgcn_perm(v0[3], v0[2], 0x05040100u) & m,
                   __builtin_amdgcn_perm(v1[1], v1[0], 0x05040100u) & m,
                   __builtin_amdgcn_perm(v1[3], v1[2], 0x05040100u) & m};
  return __builtin_bit_cast(bf16x8, r);
}
// B fragments of 8 float32 values split into (hi, lo) bf16 halves
__device__ inline void frag_split_f32(const u32x4& v0, const u32x4& v1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = wf(v0[i]), b = wf(v1[i]);
    hi[i] = (bf16)a;
    hi[4 + i] = (bf16)b;
    lo[i] = (bf16)(a - (float)hi[i]);
    lo[4 + i] = (bf16)(b - (float)hi[4 + i]);
  }
}

// The XCD this workgroup runs on.  Workgroups go to the XCDs round-robin in
// index order, starting from an XCD that depends on the hardware queue, so
// the workgroups b of one XCD are one residue of b mod 8 and their ranks
// b / 8 are 0..31 (the host checks the pattern before it picks this kernel).
__device__ inline int xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & (unsigned)(NX - 1));
}

// ------------------------------------------------------------- context

struct Ctx {
  Shared* sh;
  unsigned char* ring;
  Rsrc X;                  // exchange words, control words at CT_*
  Rsrc Y;                  // the handle's auxiliary tables
  Rsrc SC;                 // 8-bit tier: column scales
  bool w8;                 // 8-bit tier: the four projections stream int8 tiles, two per ring slot
  unsigned seq;            // this decision's counter
  unsigned redsel;         // which half of the scratch the current phase uses
  unsigned barn;           // compute-wave barriers passed
  unsigned tl;             // timeline on
  int lane, wave, g, row;  // row = lane % 16, g = lane / 16
  int crow;                // row clamped to the last action row (poll addresses)
  int S, NL, R, nc, L;     // steps, layers, action rows, prefix chunks, prefix length
  int xcd, rk;             // XCD and rank inside it
  float dt, eps;
  // ring positions of this workgroup's tile stream
  unsigned n_layer, n_step, o_att, o_o, o_gu, o_dn;
};

__device__ inline bool is_qkv(const Ctx& c) { return c.rk >= R_QKV && c.rk < R_QKV + N_QKV; }
__device__ inline bool is_att(const Ctx& c) { return c.rk <= c.nc; }
__device__ inline bool is_merge(const Ctx& c) { return c.rk >= R_MERGE && c.rk < R_MERGE + DH / 32; }
__device__ inline bool is_vel(const Ctx& c) { return c.rk == R_VEL; }
// Byte offset of a lane's load from its own action row (row = lane % 16), or
// past every buffer's range for rows past R: those lanes move nothing, read
// zeros and are left out of the poll (their live mask is 0).  The padded
// rows then compute on zeros; no real row ever reads them.
__device__ inline unsigned row_off(const Ctx& c, unsigned off) { return c.row < c.R ? off : OOB; }
// QKV n-tile of QKV workgroup i on XCD x: query head x's tiles, then this
// XCD's two tiles of the key head and two of the value head
__device__ inline int qkv_ntile(int i, int x) {
  return i < 16 ? 16 * x + i : (i < 18 ? 16 * H + 2 * x + (i - 16) : 16 * (H + 1) + 2 * x + (i - 18));
}

// Passes the context's uniform fields through an empty asm statement.  Every
// phase starts with it, so that what a phase derives from them (role tests,
// table offsets) is computed inside the phase: otherwise the compiler hoists
// all of it out of the step loop and keeps it in registers for the whole
// kernel, far more than the 102 scalar registers a wave has.
__device__ __attribute__((always_inline)) inline void refresh(Ctx& c) {
  asm volatile("" : "+s"(c.xcd), "+s"(c.rk), "+s"(c.n_layer), "+s"(c.n_step), "+s"(c.o_att), "+s"(c.o_o),
               "+s"(c.o_gu), "+s"(c.o_dn));
  asm volatile("" : "+s"(c.seq), "+s"(c.S), "+s"(c.NL), "+s"(c.R), "+s"(c.nc), "+s"(c.L), "+s"(c.tl));
  asm volatile("" : "+v"(c.lane), "+v"(c.crow));
  c.g = c.lane >> 4;
  c.row = c.lane & 15;
}

// Use counters.  A buffer type used once per layer-step, once per norm input
// (NL + 1 per step) or once between steps counts its uses without a gap from
// one decision to the next (every use writes every word its readers read): use u = seq * n + i (n uses per decision, seq the
// decision counter) goes to copy u & 1 and carries generation
// ((u >> 1) + 1) & 1, so two successive uses of a copy always differ in
// generation.  The counter starts at 0 on zeroed memory (the first use of
// each copy expects 1), advances by one after every decision, and goes back
// to 0 when the words are cleared after a decision that gave up.  The
// counters wrap at 2^32, a multiple of 4, without a break in the pattern.
struct Use {
  unsigned par, gen;
};
__device__ inline Use use_of(unsigned u) { return Use{u & 1u, ((u >> 1) + 1u) & 1u}; }
__device__ inline Use use_layer(const Ctx& c, int k, int l) {
  return use_of(c.seq * (unsigned)(c.S * c.NL) + (unsigned)(k * c.NL + l));
}
__device__ inline Use use_norm(const Ctx& c, int k, int l) {
  return use_of(c.seq * (unsigned)(c.S * (c.NL + 1)) + (unsigned)(k * (c.NL + 1) + l));
}
// the state goes from the velocity head to the input projection S - 1 times
// per decision (the last step writes the actions instead)
__device__ inline Use use_state(const Ctx& c, int k) { return use_of(c.seq * (unsigned)(c.S - 1) + (unsigned)k); }

// byte offset of buffer T's copy (use parity, this XCD for local buffers)
template <int T>
__device__ __attribute__((always_inline)) inline unsigned xb(const Ctx& c, unsigned par) {
  constexpr unsigned b = x_base(T), st = x_stride(T);
  if constexpr (x_local(T))
    return b + (par * NX + (unsigned)c.xcd) * st;
  else
    return b + par * st;
}
template <int T>
constexpr int pol_of() {
  return x_local(T) ? NTP : SC1;
}
// byte offset of step k's table block in the auxiliary tables
__device__ inline unsigned step_tab(const Ctx& c, int k) {
  return AUX_TAB + (unsigned)k * step_bytes(c.NL);
}

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
// counter + 1, so no clearing is needed), has the velocity workgroup of XCD 0
// mark the actions NaN, and ends the wave.
__device__ __attribute__((always_inline)) inline void leave(Ctx& c, bool record) {
  lds_store(&c.sh->abort, 1u);
  if (record && c.lane == 0) __builtin_amdgcn_raw_buffer_store_b32(c.seq + 1u, c.X, CT_STATUS, 0, SC1);
  if (is_vel(c) && c.xcd == 0 && c.wave == 0 && c.row < c.R) {
    const unsigned nanv = 0x7fc00000u;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{nanv, nanv, nanv, nanv}, c.Y,
                                             AUX_X + (unsigned)((c.row * A + 16 * t + 4 * c.g) * 4), 0, 0);
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
        __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(c.X, CT_STATUS, 0, SC1));
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
  // the abort flag and the time limit are checked every 16th spin: a spin is
  // one LDS read, and the barrier usually ends within a few
  unsigned n = 0;
  while (lds_load(&c.sh->cwbar) < target)
    if ((++n & 15u) == 0u) keep_waiting(c, t0, spins);
  cbar();
}

// waits until ring positions [p0, p0 + n) hold their tiles (the four
// loaders' counters read together)
__device__ inline void wait_tiles(Ctx& c, unsigned p0, unsigned n) {
  const unsigned pe = p0 + n;
  unsigned need[NLOADER];
#pragma unroll
  for (int q = 0; q < NLOADER; ++q) need[q] = pe <= (unsigned)q ? 0u : (pe - (unsigned)q + 3u) / 4u;
  const unsigned t0 = now_ticks();
  unsigned spins = 0;
  while (true) {
    unsigned r[NLOADER];
#pragma unroll
    for (int q = 0; q < NLOADER; ++q)
      r[q] = __hip_atomic_load(&c.sh->ready[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    bool ok = true;
#pragma unroll
    for (int q = 0; q < NLOADER; ++q) ok = ok && __builtin_amdgcn_readfirstlane(r[q]) >= need[q];
    if (ok) break;
    __builtin_amdgcn_s_sleep(1);
    keep_waiting(c, t0, spins);
  }
  cbar();
}

// Hands ring positions below `upto` back to the loader waves.  Callers keep
// `upto` non-decreasing over a decision: the loaders only ever compare
// against the latest value, so a smaller one would stall them until the next
// release.  Every phase's tiles are released by the end of the phase that
// follows the next device-scope phase at the latest (see the layer loop), and
// a tile range is released only after the phase that reads it has passed its
// barrier.
__device__ inline void release_ring(Ctx& c, unsigned upto) {
  cbar();
  if (c.wave == 0 && c.lane == 0) lds_store(&c.sh->consumed, upto);
}

// Scratch for one phase.  Consecutive phases take alternate halves, so a wave
// that runs ahead into the next phase never overwrites what a slower wave of
// this phase still reads.
__device__ inline unsigned char* red_take(Ctx& c) {
  unsigned char* r = c.sh->red[c.redsel & 1u];
  c.redsel += 1u;
  return r;
}
// sum of the four waves' partial tiles t (in wave order)
__device__ inline f32x4 red_sum(const f32x4* red, int nt, int t, int lane) {
  f32x4 s = red[(0 * nt + t) * 64 + lane];
  s += red[(1 * nt + t) * 64 + lane];
  s += red[(2 * nt + t) * 64 + lane];
  s += red[(3 * nt + t) * 64 + lane];
  return s;
}

__device__ inline bf16x8 ring_tile(const Ctx& c, unsigned pos) {
  const u32x4 v = *(const u32x4*)(c.ring + (pos % RING) * TILE_BYTES + c.lane * 16);
  return __builtin_bit_cast(bf16x8, v);
}

// ring slot of stream position p0 + off (off < RING), from s0 = p0 mod RING
__device__ inline unsigned ring_slot(unsigned s0, unsigned off) {
  const unsigned s = s0 + off;
  return s >= (unsigned)RING ? s - (unsigned)RING : s;
}
__device__ inline u32x4 ring_read(const Ctx& c, unsigned slot) {
  return *(const u32x4*)(c.ring + slot * TILE_BYTES + c.lane * 16);
}
// Keeps the LDS reads issued above it ahead of everything below it: the
// products that follow then wait for each tile in turn while the later
// reads are already in flight, instead of each read waiting for the product
// before it.
__device__ inline void reads_issued() { asm volatile("" ::: "memory"); }

// 8-bit tier: a lane's 8 int8 codes of one tile (k order) as its bf16
// fragment; exact, since |q| <= 127 fits bf16's significand (the float's
// upper half is the bf16)
__device__ inline u32x4 i8_frag(const u32x2& q) {
  u32x4 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const unsigned wd = q[m >> 1];
    const int sh = 16 * (m & 1);
    const float f0 = (float)(int)(signed char)(wd >> sh);
    const float f1 = (float)(int)(signed char)(wd >> (sh + 8));
    r[m] = __builtin_amdgcn_perm(as_u(f1), as_u(f0), 0x07060302u);
  }
  return r;
}

// A phase's weight tiles come out of the ring before it polls for its
// activation: ring_fetch reads the tile at stream position p0 + off(t, kk)
// into w[kk][t], and those reads (and any wait for the loaders) overlap the
// poll, so only the products are left once the activation has arrived.
//
// gemm_pairs: acc[t] = sum over k-tiles kk of W(t, kk) . (hi + lo)(kk), the
// activation pairs of k-tile kk in loads v[2 kk], v[2 kk + 1].  The hi and
// lo products go to accumulators of their own and the n-tiles are the inner
// loop, so no MFMA waits for the result of the one before it (2 NT
// independent chains); the two halves are added at the end.  In the 8-bit
// tier (W8) w[kk][t] holds the tile's raw int8 codes (words 0, 1), widened
// next to their products.
template <int NT, int KK, typename OF>
__device__ __attribute__((always_inline)) inline void ring_fetch(const Ctx& c, unsigned p0, OF off,
                                                                 u32x4 (&w)[KK][NT]) {
  const unsigned s0 = __builtin_amdgcn_readfirstlane(p0 % (unsigned)RING);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int t = 0; t < NT; ++t) w[kk][t] = ring_read(c, ring_slot(s0, off(t, kk)));
  reads_issued();
}
template <int NT, int KK, bool W8 = false>
__device__ __attribute__((always_inline)) inline void gemm_pairs(const u32x4 (&w)[KK][NT], const u32x4* v,
                                                                 f32x4 (&acc)[NT]) {
  f32x4 ah[NT], al[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ah[t] = al[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 bh = frag_hi(v[2 * kk], v[2 * kk + 1]);
    const bf16x8 bl = frag_lo(v[2 * kk], v[2 * kk + 1]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 wt = __builtin_bit_cast(bf16x8, W8 ? i8_frag(u32x2{w[kk][t][0], w[kk][t][1]}) : w[kk][t]);
      ah[t] = mma32(wt, bh, ah[t]);
      al[t] = mma32(wt, bl, al[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = ah[t] + al[t];
}

// acc[t] = sum over k-tiles kk of W(t, kk) . b(kk) for plain bf16 words (one
// load v[kk] per k-tile); two chains per n-tile (even and odd k-tiles)
template <int NT, int KK, bool W8 = false>
__device__ __attribute__((always_inline)) inline void gemm_plain(const u32x4 (&w)[KK][NT], const u32x4* v,
                                                                 f32x4 (&acc)[NT]) {
  f32x4 ae[NT], ao[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ae[t] = ao[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 b = frag_plain(v[kk]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 wt = __builtin_bit_cast(bf16x8, W8 ? i8_frag(u32x2{w[kk][t][0], w[kk][t][1]}) : w[kk][t]);
      if (kk & 1)
        ao[t] = mma32(wt, b, ao[t]);
      else
        ae[t] = mma32(wt, b, ae[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = ae[t] + ao[t];
}

// ring_fetch for int8 tiles: tile i of the phase's run sits in slot i / 2,
// half i % 2 (512 bytes: 8 codes per lane).  The codes stay raw (words 0, 1
// of w[kk][t]) until the products widen them next to their MFMAs: widened
// here, ahead of the poll, they held back the poll's first loads.
template <int NT, int KK, typename OF>
__device__ __attribute__((always_inline)) inline void ring_fetch_i8(const Ctx& c, unsigned p0, OF off,
                                                                    u32x4 (&w)[KK][NT]) {
  const unsigned s0 = __builtin_amdgcn_readfirstlane(p0 % (unsigned)RING);
  u32x2 q[KK][NT];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const unsigned i = off(t, kk);
      q[kk][t] = *(const u32x2*)(c.ring + ring_slot(s0, i >> 1) * TILE_BYTES + (i & 1u) * 512u + c.lane * 8);
    }
  reads_issued();
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int t = 0; t < NT; ++t) w[kk][t] = u32x4{q[kk][t][0], q[kk][t][1], 0u, 0u};
}
// a phase's tiles: bf16, or int8 in the 8-bit tier (n tiles take n / 2 slots)
template <bool W8, int NT, int KK, typename OF>
__device__ __attribute__((always_inline)) inline void fetch_tiles(const Ctx& c, unsigned p0, OF off,
                                                                  u32x4 (&w)[KK][NT]) {
  if constexpr (W8)
    ring_fetch_i8<NT, KK>(c, p0, off, w);
  else
    ring_fetch<NT, KK>(c, p0, off, w);
}
template <bool W8>
constexpr unsigned slots(unsigned tiles) {
  return W8 ? tiles / 2u : tiles;
}
// column scales of 4 columns (n-tile nt, columns 4 g + [0, 4)) of matrix
// block `which` of layer l; ones outside the 8-bit tier
template <bool W8>
__device__ inline u32x4 col_scales(const Ctx& c, int l, int which, int nt) {
  if constexpr (W8)
    return __builtin_amdgcn_raw_buffer_load_b128(c.SC, (unsigned)((l * SC_LAYER + which + nt * 16 + 4 * c.g) * 4), 0, 0);
  else
    return u32x4{0x3f800000u, 0x3f800000u, 0x3f800000u, 0x3f800000u};
}

// ------------------------------------------------------------- exchange

// Where load i of a poll reads: per-lane byte offset vo and uniform so in the
// arena.  Rows past R read the last valid row instead (clamped rows), so
// every lane's words become valid; the memory system merges the duplicate
// addresses of a wave, and no result of a padded row is ever stored.
struct LA {
  unsigned vo, so;
};

// Polls N loads (16-byte u32x4 or 8-byte u32x2) until every word carries
// generation gen.  Every round issues all N loads and then tests all their
// words at once: with generation 1 a round is done when the AND of every
// word has its lowest bit set, with generation 0 when their OR has it clear.
// (A word stays fresh once it is: its next writer waits for this reader.)
// Loads [0, NR) come from the lane's own row; in lanes whose row is past R
// (act false) the callers point them past the buffer's range, where they
// read zeros, and they are left out of the test.  Loads [NR, N) are valid in
// every lane.  Only the first nl loads (nl the same in every lane) are
// issued and tested; the rest read zeros.  Loads [A2, B2) take cache policy
// POL2, the others POL.
template <int POL, typename V>
__device__ inline V xload(const Ctx& c, unsigned vo, unsigned so) {
  if constexpr (sizeof(V) == 16)
    return __builtin_amdgcn_raw_buffer_load_b128(c.X, vo, so, POL);
  else
    return __builtin_amdgcn_raw_buffer_load_b64(c.X, vo, so, POL);
}
template <typename V>
__device__ inline unsigned and_words(const V& x) {
  if constexpr (sizeof(V) == 16)
    return x[0] & x[1] & x[2] & x[3];
  else
    return x[0] & x[1];
}
template <typename V>
__device__ inline unsigned or_words(const V& x) {
  if constexpr (sizeof(V) == 16)
    return x[0] | x[1] | x[2] | x[3];
  else
    return x[0] | x[1];
}
template <int POL, int N, int NR, int POL2 = POL, int A2 = 0, int B2 = 0, typename V, typename AF>
__device__ __attribute__((always_inline)) inline void poll(Ctx& c, AF addr, unsigned gen, V (&v)[N], bool act,
                                                           int nl = N) {
  static_assert(NR <= N, "row loads come first");
  const unsigned t0 = now_ticks();
  unsigned spins = 0;
  while (true) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const LA la = addr(i);
      const unsigned vo = i < nl ? la.vo : OOB, so = __builtin_amdgcn_readfirstlane(la.so);
      if (i >= A2 && i < B2)
        v[i] = xload<POL2, V>(c, vo, so);
      else
        v[i] = xload<POL, V>(c, vo, so);
    }
    unsigned stale;
    if (gen) {
      unsigned ar = ~0u, aa = ~0u;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const unsigned w = i < nl ? and_words(v[i]) : ~0u;
        if (i < NR)
          ar &= w;
        else
          aa &= w;
      }
      stale = ~(aa & (act ? ar : ~0u)) & 1u;
    } else {
      unsigned orr = 0u, oa = 0u;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const unsigned w = i < nl ? or_words(v[i]) : 0u;
        if (i < NR)
          orr |= w;
        else
          oa |= w;
      }
      stale = (oa | (act ? orr : 0u)) & 1u;
    }
    if (__ballot(stale != 0u) == 0ull) return;
    keep_waiting(c, t0, spins);
    asm volatile("" ::: "memory");
  }
}

template <int POL>
__device__ inline void st4(const Ctx& c, unsigned off, const u32x4& w) {
  __builtin_amdgcn_raw_buffer_store_b128(w, c.X, off, 0, POL);
}
template <int POL>
__device__ inline void st2(const Ctx& c, unsigned off, const u32x2& w) {
  __builtin_amdgcn_raw_buffer_store_b64(w, c.X, off, 0, POL);
}
template <int POL>
__device__ inline void st1(const Ctx& c, unsigned off, unsigned w) {
  __builtin_amdgcn_raw_buffer_store_b32(w, c.X, off, 0, POL);
}

// phase timeline (off unless the handle asked for it)
__device__ inline void tl_mark(const Ctx& c, int ev) {
  if (c.tl != 0u && c.lane == 0) {
    const unsigned idx = (blockIdx.x * (unsigned)timeline_events(c.S, c.NL) + (unsigned)ev) * 4u;
    __builtin_amdgcn_raw_buffer_store_b32(now_ticks(), c.Y, aux_timeline(c.S, c.NL) + idx, 0, 0);
  }
}

// ---------------------------------------------------------------- owners
// Every workgroup owns residual columns [32 r, 32 r + 32) (its rank's two
// n-tiles) and keeps them in registers, four rows per wave: lane l of wave w
// holds row 4 w + l / 16, columns 32 r + 2 (l % 16) + [0, 2).  Each wave
// updates and publishes its own rows, so no owner step waits for another
// wave.  The owners of the eight XCDs hold the same columns and add the same
// partial sums in the same order.  Rows past R repeat row R - 1.
struct Own {
  int row, crow;  // row of the lane, clamped to the last action row
  unsigned col;   // first of the lane's two columns
};
__device__ inline Own own_of(const Ctx& c) {
  const int r = 4 * c.wave + (c.lane >> 4);
  return Own{r, r < c.R ? r : c.R - 1, (unsigned)(32 * c.rk + 2 * (c.lane & 15))};
}

// (1 + scale) of the lane's two columns for one norm (issue early; use after)
__device__ inline u32x2 owner_scale_load(const Ctx& c, const Own& o, int k, int norm) {
  return __builtin_amdgcn_raw_buffer_load_b64(c.Y, step_tab(c, k) + (unsigned)((norm * D) * 4) + o.col * 4u, 0, 0);
}

// publishes h * (1 + scale) as pair words and the per-row sums of squares of
// the owner's 32 columns (every wave, its four rows)
template <int T_N, int T_SS>
__device__ inline void owner_publish(Ctx& c, const Own& o, const float (&h)[2], const u32x2& sv, const Use& u) {
  const float n0 = h[0] * (1.0f + as_f(sv[0])), n1 = h[1] * (1.0f + as_f(sv[1]));
  if constexpr (T_N == X_N) {
    st1<LST>(c, xb<T_N>(c, u.par) + (unsigned)(o.row * (D / 2) * 4) + (o.col / 2u) * 4u, bf16x2_word(n0, n1, u.gen));
  } else {
    const u32x2 w = {pair_word(n0, u.gen), pair_word(n1, u.gen)};
    st2<LST>(c, xb<T_N>(c, u.par) + (unsigned)(o.row * D * 4) + o.col * 4u, w);
  }
  float s = h[0] * h[0] + h[1] * h[1];
  s = sum_row16(s);
  if ((c.lane & 15) == 0) st1<LST>(c, xb<T_SS>(c, u.par) + (unsigned)((o.row * WX + c.rk) * 4), f32_word(s, u.gen));
}

// Poll of a normalised activation (pairs [RP][D]) for this wave's 8 k-tiles
// (loads 0..15: k-tile 8 w + j at loads 2 j, 2 j + 1) plus the owners' sums
// of squares (loads 16, 17: lane row lane / 4, owners 8 (lane % 4) + [0, 8)).
// loads of a poll_normed: 16 (pairs) or 8 (plain words) for the wave's k-tiles, then 2
template <int T_N>
constexpr int normed_loads() {
  return (T_N == X_N ? 8 : 16) + 2;
}
template <int T_N, int T_SS>
__device__ __attribute__((always_inline)) inline void poll_normed(Ctx& c, const Use& u,
                                                                  u32x4 (&v)[normed_loads<T_N>()]) {
  constexpr int NA = normed_loads<T_N>() - 2;
  constexpr bool plain = NA == 8;
  const unsigned vn = plain ? row_off(c, (unsigned)((c.row * (D / 2) + 128 * c.wave + 4 * c.g) * 4))
                            : row_off(c, (unsigned)((c.row * D + 256 * c.wave + 8 * c.g) * 4));
  const int srow = c.lane >> 2;
  const int scrow = srow < c.R ? srow : c.R - 1;
  const unsigned vs = (unsigned)((scrow * WX + 8 * (c.lane & 3)) * 4);
  const unsigned bn = xb<T_N>(c, u.par), bs = xb<T_SS>(c, u.par);
  // only wave 0 forms the row scales, so only wave 0 polls the sums
  poll<NTP, NA + 2, NA>(c, [&](int i) -> LA {
    if (i < NA) return plain ? LA{vn + (unsigned)(i * 16 * 4), bn} : LA{vn + (unsigned)((i >> 1) * 32 * 4 + (i & 1) * 16), bn};
    return LA{vs + (unsigned)((i - NA) * 16), bs};
  }, u.gen, v, c.row < c.R, c.wave == 0 ? NA + 2 : NA);
  if (c.wave == 0) {
    float s = 0.f;
#pragma unroll
    for (int i = NA; i < NA + 2; ++i) s += (wf(v[i][0]) + wf(v[i][1])) + (wf(v[i][2]) + wf(v[i][3]));
    s = sum_quad(s);
    if ((c.lane & 3) == 0) c.sh->rrow[srow] = frsq(s / (float)D + c.eps);
  }
}

// ------------------------------------------------------------- phases
// Every phase is entered by all four compute waves; barrier counts match.
// Each phase issues all the loads it needs (tables first, then the exchange
// words) before waiting on any of them.

// input projection h = x . W_in for the owner's two n-tiles: wave 0 forms
// them, the waves take their rows through LDS
__device__ __attribute__((always_inline)) inline void ph_in(Ctx& c, int k, float (&h)[2]) {
  refresh(c);
  const Own o = own_of(c);
  const u32x2 sv = owner_scale_load(c, o, k, 0);
  float* hs = (float*)red_take(c);  // [RP][32] f32
  if (c.wave == 0) {
    const unsigned p0 = (unsigned)k * c.n_step;
    u32x4 v[2];
    const unsigned vo = (unsigned)((c.crow * A + 8 * c.g) * 4);
    if (k == 0) {
      v[0] = __builtin_amdgcn_raw_buffer_load_b128(c.Y, AUX_X + vo, 0, 0);
      v[1] = __builtin_amdgcn_raw_buffer_load_b128(c.Y, AUX_X + vo + 16u, 0, 0);
    } else {
      const Use ux = use_state(c, k - 1);
      const unsigned bx = xb<X_X>(c, ux.par);
      const unsigned vr = row_off(c, vo);
      poll<NTP, 2, 2>(c, [&](int i) -> LA { return LA{vr + 16u * (unsigned)i, bx}; }, ux.gen, v, c.row < c.R);
    }
    bf16x8 xh, xl;
    frag_split_f32(v[0], v[1], xh, xl);
    wait_tiles(c, p0, 2);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 a = mma32(ring_tile(c, p0 + t), xh, f32x4{0.f, 0.f, 0.f, 0.f});
      a = mma32(ring_tile(c, p0 + t), xl, a);
      // lane: row lane % 16, columns 16 t + 4 g + [0, 4)
      *(f32x4*)(hs + c.row * 32 + 16 * t + 4 * c.g) = a;
    }
    release_ring(c, p0 + 2);
  }
  cw_barrier(c);
  const float2 hv = *(const float2*)(hs + o.row * 32 + 2 * (c.lane & 15));
  h[0] = hv.x;
  h[1] = hv.y;
  owner_publish<X_N, X_SS>(c, o, h, sv, use_norm(c, k, 0));
}

// QKV projection of one n-tile (K = D split over the four waves), epilogue
// 1/rms, shift . W and RoPE (wave 0); writes q of the XCD's head (local) or
// the XCD's share of the action keys and values (device scope)
template <bool W8>
__device__ __attribute__((always_inline)) inline void ph_qkv(Ctx& c, int k, int l) {
  refresh(c);
  if (!is_qkv(c)) return;
  const int i = c.rk - R_QKV;
  const int nt = qkv_ntile(i, c.xcd);
  const unsigned p0 = (unsigned)k * c.n_step + 2u + (unsigned)l * c.n_layer;
  const Use u = use_norm(c, k, l);
  const Use uo = use_layer(c, k, l);
  const int tt = nt % 16;
  const u32x4 sw = __builtin_amdgcn_raw_buffer_load_b128(
      c.Y, step_tab(c, k) + st_swqkv(c.NL) + (unsigned)((l * NQKV + nt * 16 + 4 * c.g) * 4), 0, 0);
  const u32x4 cs = __builtin_amdgcn_raw_buffer_load_b128(
      c.Y, AUX_ROPE + (unsigned)((c.row * (DH / 2) + 8 * tt + 2 * c.g) * 8), 0, 0);
  const u32x4 sq = col_scales<W8>(c, l, SC_QKV, nt);
  wait_tiles(c, p0, slots<W8>(32));
  u32x4 w[8][1];
  fetch_tiles<W8, 1, 8>(c, p0, [&](int, int kk) { return 8u * c.wave + kk; }, w);
  u32x4 v[normed_loads<X_N>()];
  poll_normed<X_N, X_SS>(c, u, v);
  f32x4 acc[1];
  gemm_plain<1, 8, W8>(w, v, acc);
  f32x4* red = (f32x4*)red_take(c);
  red[c.wave * 64 + c.lane] = acc[0];
  cw_barrier(c);
  // the tiles are released after the attention phase (see the loop)
  if (c.wave == 0) {
    f32x4 s = red_sum(red, 1, 0, c.lane);
    if constexpr (W8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] *= as_f(sq[e]);
    }
    const float rr = c.sh->rrow[c.row];
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = rr * s[e] + as_f(sw[e]);
    if (i < 18) {  // query and key columns are rotated
      const float c0 = as_f(cs[0]), s0 = as_f(cs[1]);
      const float c1 = as_f(cs[2]), s1 = as_f(cs[3]);
      const float x0 = y[0], x1 = y[1], x2 = y[2], x3 = y[3];
      y[0] = x0 * c0 - x2 * s0;
      y[2] = x2 * c0 + x0 * s0;
      y[1] = x1 * c1 - x3 * s1;
      y[3] = x3 * c1 + x1 * s1;
    }
    // the lane's four columns are head dims j, j + 1, j + 128, j + 129; every
    // row is written (rows past R repeat row R - 1)
    const int j = 8 * tt + 2 * c.g;
    const u32x2 w01 = {pair_word(y[0], uo.gen), pair_word(y[1], uo.gen)};
    const u32x2 w23 = {pair_word(y[2], uo.gen), pair_word(y[3], uo.gen)};
    if (i < 16) {
      const unsigned o = xb<X_Q>(c, uo.par) + (unsigned)((c.row * DH + j) * 4);
      st2<LST>(c, o, w01);
      st2<LST>(c, o + (DH / 2) * 4u, w23);
    } else if (i < 18) {
      const unsigned o = xb<X_KV>(c, uo.par) + (unsigned)((c.row * DH + j) * 4);
      st2<SC1>(c, o, w01);
      st2<SC1>(c, o + (DH / 2) * 4u, w23);
    } else {
      // values transposed: [dim][key]
      const unsigned o = xb<X_KV>(c, uo.par) + (unsigned)(RP * DH * 4) + (unsigned)((j * RP + c.row) * 4);
      st1<SC1>(c, o, w01[0]);
      st1<SC1>(c, o + RP * 4u, w01[1]);
      st1<SC1>(c, o + (DH / 2) * RP * 4u, w23[0]);
      st1<SC1>(c, o + (DH / 2 + 1) * RP * 4u, w23[1]);
    }
  }
}

// outputs of one key chunk of the head: unnormalised O [row][dim] (f32 words)
// and (max, sum) per row.  oacc[d] holds O transposed (the P . V products
// run as V^T P^T): lane l has row l % 16, dims 16 (4 w + d) + 4 g + [0, 4).
// Every row is written (rows past R repeat row R - 1).
__device__ inline void attn_publish(Ctx& c, int chunk, const Use& u, const f32x4 (&oacc)[4], float m_row,
                                    float l_row) {
  const unsigned ob = xb<X_AO>(c, u.par) + (unsigned)(((chunk * RP + c.row) * DH + 4 * c.g) * 4);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4 w = {f32_word(oacc[d][0], u.gen), f32_word(oacc[d][1], u.gen), f32_word(oacc[d][2], u.gen),
                     f32_word(oacc[d][3], u.gen)};
    st4<LST>(c, ob + (unsigned)(16 * (4 * c.wave + d) * 4), w);
  }
  if (c.wave == 0 && c.g == 0) {
    const float m = m_row == -INFINITY ? M_EMPTY : m_row;
    const unsigned wm = f32_word(m, u.gen), wl = f32_word(l_row, u.gen);
    st4<LST>(c, xb<X_AML>(c, u.par) + (unsigned)((chunk * RP + c.row) * 16), u32x4{wm, wl, wm, wl});
  }
}

// Attention of head xcd over prefix key chunk [64 ch, 64 ch + 64) from the
// ring.  Wave w reads q dims [64 w, 64 w + 64) and the waves share them
// through LDS.  Wave w scores keys [16 w, 16 w + 16) and forms their
// probabilities against its own row maximum; after one more exchange between
// the waves (maxima, sums and probabilities through LDS) each wave rescales
// the four key groups' products to the common maximum for its four dim
// tiles.  The ring is released after the outputs are published.
__device__ __attribute__((always_inline)) inline void ph_attn_prefix(Ctx& c, int k, int l) {
  refresh(c);
  const int ch = c.rk;
  const Use u = use_layer(c, k, l);
  const float scale = 0.0625f;  // 1/sqrt(256)
  // the chunk's key and value tiles out of the ring first (they overlap the
  // wait for q)
  const unsigned p0 = (unsigned)k * c.n_step + 2u + (unsigned)l * c.n_layer + c.o_att;
  wait_tiles(c, p0, 64);
  const unsigned s0 = __builtin_amdgcn_readfirstlane(p0 % (unsigned)RING);
  u32x4 kt[8], vt[4][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) kt[s] = ring_read(c, ring_slot(s0, 8u * c.wave + s));
#pragma unroll
  for (int kg = 0; kg < 4; ++kg)
#pragma unroll
    for (int dp = 0; dp < 2; ++dp) vt[kg][dp] = ring_read(c, ring_slot(s0, 32u + 8u * kg + 2u * c.wave + dp));
  reads_issued();
  // q fragments of dims 32 s + 8 g + [0, 8) (hi and lo), s = 0 .. 7
  bf16x8 qh[8], ql[8];
  {
    u32x4 v[4];
    const unsigned vo = row_off(c, (unsigned)((c.row * DH + 64 * c.wave + 8 * c.g) * 4));
    const unsigned bq = xb<X_Q>(c, u.par);
    poll<NTP, 4, 4>(c, [&](int i) -> LA { return LA{vo + (unsigned)((i >> 1) * 32 * 4 + (i & 1) * 16), bq}; }, u.gen, v,
              c.row < c.R);
    u32x4* qs = (u32x4*)red_take(c);  // [8 slices][hi, lo][64 lanes]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int s = 2 * c.wave + j;
      qs[(2 * s) * 64 + c.lane] = __builtin_bit_cast(u32x4, frag_hi(v[2 * j], v[2 * j + 1]));
      qs[(2 * s + 1) * 64 + c.lane] = __builtin_bit_cast(u32x4, frag_lo(v[2 * j], v[2 * j + 1]));
    }
    cw_barrier(c);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qh[s] = __builtin_bit_cast(bf16x8, qs[(2 * s) * 64 + c.lane]);
      ql[s] = __builtin_bit_cast(bf16x8, qs[(2 * s + 1) * 64 + c.lane]);
    }
  }
  // S^T for keys [16 w, 16 w + 16) of the chunk: lane holds keys 4 g + e of row `row`
  f32x4 sth = f32x4{0.f, 0.f, 0.f, 0.f}, stl = sth;  // hi and lo products in chains of their own
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    sth = mma32(__builtin_bit_cast(bf16x8, kt[s]), qh[s], sth);
    stl = mma32(__builtin_bit_cast(bf16x8, kt[s]), ql[s], stl);
  }
  const f32x4 st = sth + stl;
  float sv[4];
  float mw = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int key = CHUNK * ch + 16 * c.wave + 4 * c.g + e;
    sv[e] = key < c.L ? st[e] * scale : -INFINITY;
    mw = fmaxf(mw, sv[e]);
  }
  mw = max_x16_x32(mw);  // this wave's row maximum
  float lw = 0.f;
  s16x4 ph, pl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p = sv[e] == -INFINITY ? 0.f : fexp(sv[e] - mw);
    lw += p;
    short a, b;
    split_bf16(p, a, b);
    ph[e] = a;
    pl[e] = b;
  }
  lw = sum_x16_x32(lw);
  if (c.g == 0) {
    c.sh->att_m[c.wave][c.row] = mw;
    c.sh->att_l[c.wave][c.row] = lw;
  }
  c.sh->att_p[c.wave][0][c.lane] = ph;
  c.sh->att_p[c.wave][1][c.lane] = pl;
  cw_barrier(c);
  // the four key groups against the row's maximum
  float mk[NCOMPUTE], sc[NCOMPUTE];
#pragma unroll
  for (int kg = 0; kg < NCOMPUTE; ++kg) mk[kg] = c.sh->att_m[kg][c.row];
  const float m_row = fmaxf(fmaxf(mk[0], mk[1]), fmaxf(mk[2], mk[3]));
#pragma unroll
  for (int kg = 0; kg < NCOMPUTE; ++kg) sc[kg] = mk[kg] == -INFINITY ? 0.f : fexp(mk[kg] - m_row);
  const float l_row = (sc[0] * c.sh->att_l[0][c.row] + sc[1] * c.sh->att_l[1][c.row]) +
                      (sc[2] * c.sh->att_l[2][c.row] + sc[3] * c.sh->att_l[3][c.row]);
  // O^T = V^T . P^T for dim tiles [4 w, 4 w + 4): each key group's products
  // (hi and lo halves of P in chains of their own), scaled to the row maximum
  s16x4 pah[4], pal[4];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) {
    pah[kg] = c.sh->att_p[kg][0][c.lane];
    pal[kg] = c.sh->att_p[kg][1][c.lane];
  }
  f32x4 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) {
    const s16x4 ah = pah[kg];
    const s16x4 al = pal[kg];
    f32x4 th[4], tl[4];
#pragma unroll
    for (int dp = 0; dp < 2; ++dp) {
      const u32x4 vv = vt[kg][dp];
      const s16x4 b0 = __builtin_bit_cast(s16x4, u32x2{vv[0], vv[1]});
      const s16x4 b1 = __builtin_bit_cast(s16x4, u32x2{vv[2], vv[3]});
      th[2 * dp] = mma16(b0, ah, f32x4{0.f, 0.f, 0.f, 0.f});
      th[2 * dp + 1] = mma16(b1, ah, f32x4{0.f, 0.f, 0.f, 0.f});
      tl[2 * dp] = mma16(b0, al, f32x4{0.f, 0.f, 0.f, 0.f});
      tl[2 * dp + 1] = mma16(b1, al, f32x4{0.f, 0.f, 0.f, 0.f});
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) oacc[d] += sc[kg] * (th[d] + tl[d]);
  }
  attn_publish(c, ch, u, oacc, m_row, l_row);
  cw_barrier(c);
  release_ring(c, p0 + 64u);
}

// Attention of head xcd over the action rows' own keys and values (chunk
// nc).  Wave w takes head dims [64 w, 64 w + 64) of q and of the keys for a
// partial score tile (the four are summed in LDS in wave order), and the
// value fragments of dim tiles 4 w .. 4 w + 3 straight from the transposed
// value words (keys 4 g .. 4 g + 3 of one dim per lane).  Products of two
// low halves (2^-16 of 2^-16) are left out.
__device__ inline s16x4 pairs_hi(const u32x4& w) {
  return __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(w[1], w[0], 0x07060302u),
                                         __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)});
}
__device__ inline s16x4 pairs_lo(const u32x4& w) {
  return __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(w[1], w[0], 0x05040100u) & 0xfffefffeu,
                                         __builtin_amdgcn_perm(w[3], w[2], 0x05040100u) & 0xfffefffeu});
}
__device__ __attribute__((always_inline)) inline void ph_attn_action(Ctx& c, int k, int l) {
  refresh(c);
  const Use u = use_layer(c, k, l);
  const float scale = 0.0625f;
  f32x4* sp = (f32x4*)red_take(c);  // [4 waves][64 lanes] partial score tiles
  // one poll for the keys (device scope, loads 0..3), q (XCD-local, 4..7)
  // and the value fragments of dim tiles 4 w + (i - 8) (device scope, 8..11)
  u32x4 kv[8];  // 0..3: the lane's key dims; 4..7: value fragments of dim tiles 4 w + (i - 4)
  u32x4 qv[4];
  {
    const unsigned bkv = xb<X_KV>(c, u.par), bq = xb<X_Q>(c, u.par);
    const unsigned vk = row_off(c, (unsigned)((c.row * DH + 64 * c.wave + 8 * c.g) * 4));
    const unsigned vv = (unsigned)(RP * DH * 4) + (unsigned)(((64 * c.wave + c.row) * RP + 4 * c.g) * 4);
    u32x4 a[12];
    poll<SC1, 12, 8, NTP, 4, 8>(c, [&](int i) -> LA {
      if (i < 4) return LA{vk + (unsigned)((i >> 1) * 32 * 4 + (i & 1) * 16), bkv};
      if (i < 8) return LA{vk + (unsigned)(((i - 4) >> 1) * 32 * 4 + ((i - 4) & 1) * 16), bq};
      return LA{vv + (unsigned)((i - 8) * 16 * RP * 4), bkv};
    }, u.gen, a, c.row < c.R);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kv[i] = a[i];
      qv[i] = a[4 + i];
      kv[4 + i] = a[8 + i];
    }
  }
  f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16x8 kh = frag_hi(kv[2 * j], kv[2 * j + 1]), kl = frag_lo(kv[2 * j], kv[2 * j + 1]);
    const bf16x8 qhf = frag_hi(qv[2 * j], qv[2 * j + 1]), qlf = frag_lo(qv[2 * j], qv[2 * j + 1]);
    st = mma32(kh, qhf, st);
    st = mma32(kh, qlf, st);
    st = mma32(kl, qhf, st);
  }
  sp[c.wave * 64 + c.lane] = st;
  cw_barrier(c);
  st = ((sp[0 * 64 + c.lane] + sp[1 * 64 + c.lane]) + sp[2 * 64 + c.lane]) + sp[3 * 64 + c.lane];
  float sv[4];
  float mw = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int key = 4 * c.g + e;
    sv[e] = key < c.R ? st[e] * scale : -INFINITY;
    mw = fmaxf(mw, sv[e]);
  }
  mw = max_x16_x32(mw);
  const float m_row = mw;
  float lw = 0.f;
  s16x4 ph, pl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p = sv[e] == -INFINITY ? 0.f : fexp(sv[e] - m_row);
    lw += p;
    short a, b;
    split_bf16(p, a, b);
    ph[e] = a;
    pl[e] = b;
  }
  lw = sum_x16_x32(lw);
  f32x4 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const s16x4 vh = pairs_hi(kv[4 + d]), vl = pairs_lo(kv[4 + d]);
    oacc[d] = mma16(vh, ph, f32x4{0.f, 0.f, 0.f, 0.f});
    oacc[d] = mma16(vl, ph, oacc[d]);
    oacc[d] = mma16(vh, pl, oacc[d]);
  }
  attn_publish(c, c.nc, u, oacc, m_row, lw);
}

// Merges the head's key chunks for dims [32 s, 32 s + 32) and writes the
// normalised attention output as pairs.  Wave w finishes rows 4 w .. 4 w + 3
// on its own, with no exchange between the waves: lane l takes row
// 4 w + l / 16 and dims 32 s + 2 (l % 16) + [0, 2) and reads that row's two
// partial outputs of every chunk; the 16 lanes of the row share out the
// chunks' (max, sum) pairs, lane j reading chunk j's.  The row maximum and
// the weighted sum come from reductions over the 16 lanes, and each chunk's
// weight reaches the row's lanes by a DPP row broadcast, so the chunks are
// added in chunk order.  Rows past R repeat row R - 1 (nobody reads them).
static_assert(MAX_CHUNKS <= 16, "one (max, sum) pair per lane of a row");
template <int CC>
__device__ inline float row_share(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), DPP_ROW_SHARE0 + CC, 0xf, 0xf,
                                                            false));
}
template <int CC>
__device__ __attribute__((always_inline)) inline void merge_add(float e, const u32x2 (&v)[MAX_CHUNKS + 1], int nch,
                                                                float& o0, float& o1) {
  if constexpr (CC < MAX_CHUNKS) {
    if (CC < nch) {
      const float ec = row_share<CC>(e);
      o0 += ec * wf(v[1 + CC][0]);
      o1 += ec * wf(v[1 + CC][1]);
      merge_add<CC + 1>(e, v, nch, o0, o1);
    }
  }
}
__device__ __attribute__((always_inline)) inline void ph_merge(Ctx& c, int k, int l) {
  refresh(c);
  if (!is_merge(c)) return;
  const int s = c.rk - R_MERGE;
  const int nch = c.nc + 1;
  const Use u = use_layer(c, k, l);
  const int r = 4 * c.wave + (c.lane >> 4);
  const bool act = r < c.R;
  const int j = c.lane & 15;
  const int dd = 32 * s + 2 * j;
  u32x2 v[1 + MAX_CHUNKS];  // 0: (max, sum) of chunk min(j, nch - 1); 1 + cc: the two partial outputs of chunk cc
  {
    const unsigned bo = xb<X_AO>(c, u.par), bm = xb<X_AML>(c, u.par);
    const unsigned vo = act ? (unsigned)((r * DH + dd) * 4) : OOB;
    const unsigned vm = act ? (unsigned)(((j < nch ? j : nch - 1) * RP + r) * 16) : OOB;
    poll<NTP, 1 + MAX_CHUNKS, 1 + MAX_CHUNKS>(c, [&](int i) -> LA {
      if (i == 0) return LA{vm, bm};
      return LA{vo, bo + (unsigned)((i - 1) * RP * DH * 4)};
    }, u.gen, v, act, 1 + nch);
  }
  const float mj = j < nch ? wf(v[0][0]) : M_EMPTY;
  const float M = max_row16(mj);
  const float e = j < nch ? fexp(mj - M) : 0.f;
  const float L = sum_row16(e * wf(v[0][1]));
  float o0 = 0.f, o1 = 0.f;
  merge_add<0>(e, v, nch, o0, o1);
  const float inv = frcp(L);
  const u32x2 w = {pair_word(o0 * inv, u.gen), pair_word(o1 * inv, u.gen)};
  if (act) st2<LST>(c, xb<X_O>(c, u.par) + (unsigned)((r * DH + dd) * 4), w);
}

// out projection of the head's 256 rows for output columns
// [32 o, 32 o + 32) (two n-tiles; K split over the four waves): a partial
// sum of the residual update, published at device scope for the owners of
// every XCD
template <bool W8>
__device__ __attribute__((always_inline)) inline void ph_o(Ctx& c, int k, int l) {
  refresh(c);
  const int o = c.rk;
  const Use u = use_layer(c, k, l);
  const unsigned p0 = (unsigned)k * c.n_step + 2u + (unsigned)l * c.n_layer + c.o_o;
  const u32x4 sq = col_scales<W8>(c, l, SC_O, O_NT * o + (c.wave & (O_NT - 1)));
  wait_tiles(c, p0, slots<W8>(8 * O_NT));
  u32x4 w[2][O_NT];
  fetch_tiles<W8, O_NT, 2>(c, p0, [&](int t, int j) { return 8u * t + 2u * c.wave + j; }, w);
  u32x4 v[4];
  {
    const unsigned vo = row_off(c, (unsigned)((c.row * DH + 64 * c.wave + 8 * c.g) * 4));
    const unsigned bo = xb<X_O>(c, u.par);
    poll<NTP, 4, 4>(c, [&](int i) -> LA { return LA{vo + (unsigned)((i >> 1) * 32 * 4 + (i & 1) * 16), bo}; }, u.gen, v,
              c.row < c.R);
  }
  f32x4 acc[O_NT];
  gemm_pairs<O_NT, 2, W8>(w, v, acc);
  f32x4* red = (f32x4*)red_take(c);
#pragma unroll
  for (int t = 0; t < O_NT; ++t) red[(c.wave * O_NT + t) * 64 + c.lane] = acc[t];
  cw_barrier(c);
  // the tiles are released after the all-reduce that follows (see the loop)
  if (c.wave < O_NT) {
    f32x4 s = red_sum(red, O_NT, c.wave, c.lane);  // wave t finishes n-tile t
    if constexpr (W8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] *= as_f(sq[e]);
    }
    if (c.row < c.R) {
      const u32x4 w = {f32_word(s[0], u.gen), f32_word(s[1], u.gen), f32_word(s[2], u.gen), f32_word(s[3], u.gen)};
      st4<SC1>(c, xb<X_OP>(c, u.par) +
                      (unsigned)(((c.xcd * RP + c.row) * D + 16 * O_NT * o + 16 * c.wave + 4 * c.g) * 4), w);
    }
  }
}

// All-reduce of a residual update (T_P: the eight XCDs' partial sums), the
// residual add and the next norm's producer half.  Every wave reads the
// eight partials of its own rows and adds them in the same order on every
// XCD.
template <int T_P, int T_N, int T_SS>
__device__ __attribute__((always_inline)) inline void ph_own(Ctx& c, int k, int norm, const Use& u, const Use& un,
                                                             float (&h)[2]) {
  refresh(c);
  const Own o = own_of(c);
  const u32x2 sv = owner_scale_load(c, o, k, norm);
  u32x2 v[NX];
  {
    const bool act = o.row < c.R;
    const unsigned vo = act ? (unsigned)(o.row * D * 4) + o.col * 4u : OOB;
    const unsigned bp = xb<T_P>(c, u.par);
    poll<SC1, NX, NX>(c, [&](int i) -> LA { return LA{vo + (unsigned)(i * RP * D * 4), bp}; }, u.gen, v, act);
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float s01 = wf(v[0][e]) + wf(v[1][e]), s23 = wf(v[2][e]) + wf(v[3][e]);
    const float s45 = wf(v[4][e]) + wf(v[5][e]), s67 = wf(v[6][e]) + wf(v[7][e]);
    h[e] += ((s01 + s23) + s45) + s67;
  }
  owner_publish<T_N, T_SS>(c, o, h, sv, un);
}

// gate/up projection of two n-tiles with the GeGLU epilogue: features
// 16 r + 8 t + 2 g + [0, 2) of the XCD's 512
template <bool W8>
__device__ __attribute__((always_inline)) inline void ph_gu(Ctx& c, int k, int l) {
  refresh(c);
  const Use u = use_layer(c, k, l);
  const unsigned p0 = (unsigned)k * c.n_step + 2u + (unsigned)l * c.n_layer + c.o_gu;
  const int nt = 64 * c.xcd + 2 * c.rk + (c.wave & 1);
  const u32x4 sw = __builtin_amdgcn_raw_buffer_load_b128(
      c.Y, step_tab(c, k) + st_swgu(c.NL) + (unsigned)((l * 2 * F + nt * 16 + 4 * c.g) * 4), 0, 0);
  const u32x4 sq = col_scales<W8>(c, l, SC_GU, nt);
  wait_tiles(c, p0, slots<W8>(64));
  u32x4 w[8][2];
  fetch_tiles<W8, 2, 8>(c, p0, [&](int t, int kk) { return 32u * t + 8u * c.wave + kk; }, w);
  u32x4 v[normed_loads<X_N2>()];
  poll_normed<X_N2, X_SS2>(c, u, v);
  f32x4 acc[2];
  gemm_pairs<2, 8, W8>(w, v, acc);
  f32x4* red = (f32x4*)red_take(c);
#pragma unroll
  for (int t = 0; t < 2; ++t) red[(c.wave * 2 + t) * 64 + c.lane] = acc[t];
  cw_barrier(c);
  release_ring(c, p0 + slots<W8>(64));
  if (c.wave < 2) {
    f32x4 s = red_sum(red, 2, c.wave, c.lane);
    if constexpr (W8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] *= as_f(sq[e]);
    }
    const float rr = c.sh->rrow[c.row];
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = rr * s[e] + as_f(sw[e]);
    const float a0 = gelu_tanh(y[0]) * y[2];
    const float a1 = gelu_tanh(y[1]) * y[3];
    if (c.row < c.R) {
      const int f = 16 * c.rk + 8 * c.wave + 2 * c.g;
      st2<LST>(c, xb<X_A>(c, u.par) + (unsigned)((c.row * FX + f) * 4), u32x2{pair_word(a0, u.gen), pair_word(a1, u.gen)});
    }
  }
}

// down projection of the XCD's 512 features (K split over the four waves)
// for output columns [32 r, 32 r + 32): a partial sum for the owners of
// every XCD
template <bool W8>
__device__ __attribute__((always_inline)) inline void ph_down(Ctx& c, int k, int l) {
  refresh(c);
  const Use u = use_layer(c, k, l);
  const unsigned p0 = (unsigned)k * c.n_step + 2u + (unsigned)l * c.n_layer + c.o_dn;
  const u32x4 sq = col_scales<W8>(c, l, SC_DN, 2 * c.rk + (c.wave & 1));
  wait_tiles(c, p0, slots<W8>(32));
  u32x4 w[4][2];
  fetch_tiles<W8, 2, 4>(c, p0, [&](int t, int j) { return 16u * t + 4u * c.wave + j; }, w);
  u32x4 v[8];
  {
    const unsigned vo = row_off(c, (unsigned)((c.row * FX + 128 * c.wave + 8 * c.g) * 4));
    const unsigned ba = xb<X_A>(c, u.par);
    poll<NTP, 8, 8>(c, [&](int i) -> LA { return LA{vo + (unsigned)((i >> 1) * 32 * 4 + (i & 1) * 16), ba}; }, u.gen, v,
              c.row < c.R);
  }
  f32x4 acc[2];
  gemm_pairs<2, 4, W8>(w, v, acc);
  f32x4* red = (f32x4*)red_take(c);
#pragma unroll
  for (int t = 0; t < 2; ++t) red[(c.wave * 2 + t) * 64 + c.lane] = acc[t];
  cw_barrier(c);
  // the tiles are released after the all-reduce that follows (see the loop)
  if (c.wave < 2) {
    f32x4 s = red_sum(red, 2, c.wave, c.lane);
    if constexpr (W8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] *= as_f(sq[e]);
    }
    if (c.row < c.R) {
      const u32x4 w = {f32_word(s[0], u.gen), f32_word(s[1], u.gen), f32_word(s[2], u.gen), f32_word(s[3], u.gen)};
      st4<SC1>(c, xb<X_DP>(c, u.par) + (unsigned)(((c.xcd * RP + c.row) * D + 32 * c.rk + 16 * c.wave + 4 * c.g) * 4),
               w);
    }
  }
}

// velocity head (K = D over the four waves), the final norm's consumer half,
// and the Euler update of every state column (wave 0 holds x); each XCD keeps
// its own copy of x, XCD 0 writes the actions after the last step
__device__ __attribute__((always_inline)) inline void ph_vel(Ctx& c, int k, f32x4 (&x)[2]) {
  refresh(c);
  if (!is_vel(c)) return;
  const int NL = c.NL;
  const Use u = use_norm(c, k, NL);
  const unsigned p0 = (unsigned)k * c.n_step + 2u + (unsigned)NL * c.n_layer;
  u32x4 sw[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
    sw[t] = __builtin_amdgcn_raw_buffer_load_b128(c.Y, step_tab(c, k) + st_swout(NL) + (unsigned)((16 * t + 4 * c.g) * 4),
                                                  0, 0);
  wait_tiles(c, p0, 64);
  u32x4 w[8][2];
  ring_fetch<2, 8>(c, p0, [&](int t, int kk) { return 32u * t + 8u * c.wave + kk; }, w);
  u32x4 v[normed_loads<X_N>()];
  poll_normed<X_N, X_SS>(c, u, v);
  f32x4 acc[2];
  gemm_plain<2, 8>(w, v, acc);
  f32x4* red = (f32x4*)red_take(c);
#pragma unroll
  for (int t = 0; t < 2; ++t) red[(c.wave * 2 + t) * 64 + c.lane] = acc[t];
  cw_barrier(c);
  release_ring(c, p0 + 64u);
  if (c.wave == 0) {
    const float rr = c.sh->rrow[c.row];
    const Use ux = use_state(c, k);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 s = red_sum(red, 2, t, c.lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[t][e] += c.dt * (rr * s[e] + as_f(sw[t][e]));
      if (c.row < c.R) {
        if (k + 1 < c.S) {
          const u32x4 w = {f32_word(x[t][0], ux.gen), f32_word(x[t][1], ux.gen), f32_word(x[t][2], ux.gen),
                           f32_word(x[t][3], ux.gen)};
          st4<LST>(c, xb<X_X>(c, ux.par) + (unsigned)((c.row * A + 16 * t + 4 * c.g) * 4), w);
        } else if (c.xcd == 0) {
          const u32x4 w = {as_u(x[t][0]), as_u(x[t][1]), as_u(x[t][2]), as_u(x[t][3])};
          __builtin_amdgcn_raw_buffer_store_b128(w, c.Y, AUX_X + (unsigned)((c.row * A + 16 * t + 4 * c.g) * 4), 0,
                                                 0);
        }
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
  int kv;                 // source: 0 bf16 weights, 1 the prefix K/V arena, 2 int8 codes (two tiles per slot)
};

constexpr int RUNS_PER_LAYER = 9;
// run 0: input projection (W_in n-tiles 2 r, 2 r + 1); 1 + 9 l + u: layer l
// part u (0 QKV, 1 prefix K/V chunk, 2..5 out projection n-tiles, 6 gate/up,
// 7..8 down n-tiles); 1 + 9 NL: velocity head
__device__ inline void run_params(const Ctx& c, int run, unsigned& off, int& cnt, int& kv) {
  kv = 0;
  cnt = 0;
  off = 0;
  const int NL = c.NL, x = c.xcd, r = c.rk;
  if (run == 0) {
    cnt = 2;
    off = (unsigned)(2 * r) * TILE_BYTES;
    return;
  }
  if (run == 1 + RUNS_PER_LAYER * NL) {
    if (is_vel(c)) {
      cnt = 64;
      off = (unsigned)(w_out(NL) * 2ull);
    }
    return;
  }
  const int l = (run - 1) / RUNS_PER_LAYER, u = (run - 1) % RUNS_PER_LAYER;
  const unsigned long long lo = (unsigned long long)l * W_LAYER;
  // a layer projection's run: tiles (bf16, 2 bytes per element) or, in the
  // 8-bit tier, slots of two int8 tiles (codes at the same element offsets)
  const unsigned esz = c.w8 ? 1u : 2u;
  const int div = c.w8 ? 2 : 1;
  const int src = c.w8 ? 2 : 0;
  if (u == 0) {
    if (is_qkv(c)) {
      cnt = KT_D / div;
      kv = src;
      off = (unsigned)((W_QKV0 + lo + (unsigned long long)qkv_ntile(r - R_QKV, x) * KT_D * TILE_ELEMS) * esz);
    }
  } else if (u == 1) {
    if (r < c.nc) {
      cnt = 64;
      kv = 1;
      off = (unsigned)((l * c.nc + r) * 64) * TILE_BYTES;
    }
  } else if (u <= 5) {
    if (u - 2 < O_NT) {
      const int nt = O_NT * r + (u - 2);
      cnt = 8 / div;
      kv = src;
      off = (unsigned)((W_O0 + lo + ((unsigned long long)nt * KT_HD + 8 * x) * TILE_ELEMS) * esz);
    }
  } else if (u == 6) {
    cnt = 64 / div;
    kv = src;
    off = (unsigned)((W_GU0 + lo + (unsigned long long)(64 * x + 2 * r) * KT_D * TILE_ELEMS) * esz);
  } else {
    const int nt = 2 * r + (u - 7);
    cnt = 16 / div;
    kv = src;
    off = (unsigned)((W_DN0 + lo + ((unsigned long long)nt * KT_F + 16 * x) * TILE_ELEMS) * esz);
  }
}

// next (position, byte offset, source) of loader q; false at the end
__device__ inline bool gen_next(const Ctx& c, Gen& s, int q, unsigned& pos, unsigned& off, int& kv) {
  const int runs_per_step = 2 + RUNS_PER_LAYER * c.NL;
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
// tiles carry the streaming hint; prefix K/V tiles do not.
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

constexpr unsigned LOAD_DEPTH = 16;  // tiles in flight per loader wave (with the tiles handed back after
                                     // the device-scope phases: 6 and 8 slower, 12 0.5% slower, 20-32 the
                                     // same as 16)

// Loader waves wait on LDS only: a global load in their wait loop would make
// the next use of any loaded register wait for the whole batch of tile loads
// (loads complete in order).  They leave on their workgroup's abort flag; on
// their own time limit they record the failure and raise the flag.
__device__ inline void loader_keep_waiting(Ctx& c, unsigned t0, unsigned& spins) {
  ++spins;
  if (lds_load(&c.sh->abort) != 0u) end_wave();
  if ((spins & 63u) == 0u && now_ticks() - t0 > TIMEOUT_TICKS) {
    lds_store(&c.sh->abort, 1u);
    if (c.lane == 0) __builtin_amdgcn_raw_buffer_store_b32(c.seq + 1u, c.X, CT_STATUS, 0, SC1);
    end_wave();
  }
}

template <bool W8>
__device__ __attribute__((always_inline)) inline void loader(Ctx& c, int q, const Args& a) {
  const u32x4 WR = rsrc_words(W8 ? a.wq : a.wt, W8 ? a.wq_bytes : a.wt_bytes);  // W8: the codes
  const u32x4 KR = rsrc_words(a.kvt, a.kvt_bytes);
  const u32x4 BR = rsrc_words(a.wt, a.wt_bytes);  // W8: the bf16 in- and out-projections
  const unsigned ring_lds =
      (unsigned)(unsigned long long)((__attribute__((address_space(3))) unsigned char*)c.ring);
  Gen s;
  s.k = 0;
  s.run = 0;
  s.pos0 = 0;
  run_params(c, 0, s.off0, s.cnt, s.kv);
  s.j = q;
  unsigned issued = 0;
  unsigned pub = 0;  // tiles published as ready; never decreases
  unsigned pos, off;
  int kv;
  unsigned cons = 0;  // the compute waves' release position, re-read only when the ring looks full
  while (gen_next(c, s, q, pos, off, kv)) {
    if (pos >= cons + RING) cons = lds_load(&c.sh->consumed);
    if (pos >= cons + RING) {
      // the ring is full: publish every tile in flight before waiting, since
      // the compute waves may be waiting for exactly those
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      pub = issued;
      if (c.lane == 0) lds_store(&c.sh->ready[q], pub);
      const unsigned t0 = now_ticks();
      unsigned spins = 0;
      while (pos >= (cons = lds_load(&c.sh->consumed)) + RING) {
        __builtin_amdgcn_s_sleep(2);
        loader_keep_waiting(c, t0, spins);
      }
    }
    cbar();
    const unsigned lds = __builtin_amdgcn_readfirstlane(ring_lds + (pos % RING) * TILE_BYTES);
    if (kv == 1)
      dma_tile(KR, (unsigned)c.lane * 16u, off, lds, false);
    else if (W8 && kv == 0)
      dma_tile(BR, (unsigned)c.lane * 16u, off, lds, true);
    else
      dma_tile(WR, (unsigned)c.lane * 16u, off, lds, true);
    ++issued;
    // every tile but the last LOAD_DEPTH has landed; after a full publish
    // (above) the count only moves on once it passes what was published
    if (issued > LOAD_DEPTH + pub) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOAD_DEPTH) : "memory");
      pub = issued - LOAD_DEPTH;
      if (c.lane == 0) lds_store(&c.sh->ready[q], pub);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (c.lane == 0) lds_store(&c.sh->ready[q], issued);
}

// ---------------------------------------------------------------- kernel

template <bool W8>
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
  c.xcd = xcc_id();
  c.rk = (int)(blockIdx.x / NX);
  if (threadIdx.x < 32) ((unsigned*)&sh)[threadIdx.x] = 0u;
  c.X = rsrc(a.ex, XC_BYTES);
  c.Y = rsrc(a.aux, a.aux_bytes);
  c.w8 = W8;
  if constexpr (W8) c.SC = rsrc(const_cast<float*>(a.wsc), a.wsc_bytes);
  c.seq = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(c.X, CT_SEQ, 0, SC1));
  c.L = __builtin_amdgcn_readfirstlane((int)__builtin_amdgcn_raw_buffer_load_b32(c.Y, AUX_LENS, 0, 0));
  c.crow = c.row < c.R ? c.row : c.R - 1;
  // stream layout of this workgroup (must match run_params)
  c.o_att = is_qkv(c) ? slots<W8>(KT_D) : 0u;
  c.o_o = c.o_att + (c.rk < c.nc ? 64u : 0u);
  c.o_gu = c.o_o + slots<W8>(8u * O_NT);
  c.o_dn = c.o_gu + slots<W8>(64u);
  c.n_layer = c.o_dn + slots<W8>(32u);
  c.n_step = 2u + (unsigned)c.NL * c.n_layer + (is_vel(c) ? 64u : 0u);
  __syncthreads();

  if (c.wave >= NCOMPUTE) {
    loader<W8>(c, c.wave - NCOMPUTE, a);
    if (c.wave == NCOMPUTE) tl_mark(c, timeline_events(c.S, c.NL) - 1);
    return;
  }
  float h[2] = {0.f, 0.f};
  f32x4 x[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) x[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (is_vel(c) && c.wave == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 xv = __builtin_amdgcn_raw_buffer_load_b128(
          c.Y, AUX_X + (unsigned)((c.crow * A + 16 * t + 4 * c.g) * 4), 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[t][e] = as_f(xv[e]);
    }
  }
  const bool tl = c.wave == 0;
  const bool attends = c.rk <= c.nc;
  const bool action_chunk = c.rk == c.nc;
  if (tl) tl_mark(c, 0);
  for (int k = 0; k < c.S; ++k) {
    const int e0 = 1 + k * (2 + PHASES_PER_LAYER * c.NL);
    ph_in(c, k, h);
    if (tl) tl_mark(c, e0);
    for (int l = 0; l < c.NL; ++l) {
      const int el = e0 + 1 + PHASES_PER_LAYER * l;
      ph_qkv<W8>(c, k, l);
      // the rest of the previous layer's down-projection tiles (see below)
      release_ring(c, (unsigned)k * c.n_step + 2u + (unsigned)l * c.n_layer);
      if (tl) tl_mark(c, el);
      // two separate tests: as one if/else the compiler's uniformity analysis loses track of the
      // context's scalar fields after the join and cannot build the kernel
      if (attends && !action_chunk) ph_attn_prefix(c, k, l);
      if (action_chunk) ph_attn_action(c, k, l);
      // The QKV tiles go back to the loaders only after the attention phase,
      // whose action chunk polls keys and values at device scope: the tile
      // loads they let through stream during the merge instead.
      if (is_qkv(c)) release_ring(c, (unsigned)k * c.n_step + 2u + (unsigned)l * c.n_layer + slots<W8>(32));
      if (tl) tl_mark(c, el + 1);
      ph_merge(c, k, l);
      if (tl) tl_mark(c, el + 2);
      ph_o<W8>(c, k, l);
      if (tl) tl_mark(c, el + 3);
      ph_own<X_OP, X_N2, X_SS2>(c, k, 2 * l + 1, use_layer(c, k, l), use_layer(c, k, l), h);
      // Likewise the out-projection tiles go back only after the all-reduce
      // behind them, so that the tile loads they let through stream during
      // XCD-local phases instead of crowding the all-reduce's device-scope
      // polls.
      release_ring(c, (unsigned)k * c.n_step + 2u + (unsigned)l * c.n_layer + c.o_o + slots<W8>(8u * O_NT));
      if (tl) tl_mark(c, el + 4);
      ph_gu<W8>(c, k, l);
      if (tl) tl_mark(c, el + 5);
      ph_down<W8>(c, k, l);
      if (tl) tl_mark(c, el + 6);
      ph_own<X_DP, X_N, X_SS>(c, k, 2 * (l + 1), use_layer(c, k, l), use_norm(c, k, l + 1), h);
      {
        // The down-projection tiles: after the all-reduce only as many as
        // the next layer's attention tiles need to be loadable (its keys and
        // values); the rest after the next layer's QKV phase, so that the
        // loads of later tiles do not crowd the all-reduce's polls or the
        // QKV phase.  The last layer hands back all of them.
        const unsigned nxt = (unsigned)k * c.n_step + 2u + (unsigned)(l + 1) * c.n_layer;
        const unsigned cur = nxt - slots<W8>(32);
        const unsigned need = nxt + c.o_o > (unsigned)RING ? nxt + c.o_o - (unsigned)RING : 0u;
        release_ring(c, l + 1 == c.NL ? nxt : (need < cur ? cur : (need > nxt ? nxt : need)));
      }
      if (tl) tl_mark(c, el + 7);
    }
    ph_vel(c, k, x);
    if (tl) tl_mark(c, e0 + 1 + PHASES_PER_LAYER * c.NL);
  }
  if (tl) tl_mark(c, timeline_events(c.S, c.NL) - 2);
}

// After a decision (one block): advances the decision counter.  If a wait of
// the decision gave up, its words may be half written: the block clears the
// exchange words, starts the counter over at 0 and clears the status, and
// raises the failure flag the host reads; otherwise it lowers the flag.  The
// clear only runs after a failed decision.  The decision's shape goes into
// the control words either way.
constexpr int ADV_THREADS = 1024;
__global__ __launch_bounds__(ADV_THREADS) void k_decide_advance(unsigned char* exw, unsigned char* aux, u32x4 shape) {
  unsigned* ct = (unsigned*)exw;
  const unsigned st = ct[CT_STATUS / 4];
  const unsigned sq = ct[CT_SEQ / 4];
  const bool failed = st != 0u && st == sq + 1u;
  if (failed) {
    u32x4* ex = (u32x4*)exw;
    for (unsigned i = threadIdx.x; i < EX_BYTES / 16u; i += ADV_THREADS) ex[i] = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    ct[CT_SEQ / 4] = failed ? 0u : sq + 1u;
    if (failed) ct[CT_STATUS / 4] = 0u;
    *(u32x4*)(exw + CT_SHAPE) = shape;
    ((unsigned*)aux)[AUX_FAILED / 4] = failed ? 1u : 0u;
  }
}

// Before a decision on words that decisions of other shapes may have used
// (G blocks, each its slice of the words): the tags only tell fresh from
// stale when every use of a buffer writes every word the next use of that
// copy reads, and the counter counts the same uses per decision.  Both hold
// between decisions of one shape (rows, prefix chunks, steps, layers); after
// a decision of another shape the words are cleared and the counter restarts
// at 0, as on fresh memory.  The shape record itself is only written after
// the decision, so every block here reads the same one.
constexpr int PREP_THREADS = 256;
constexpr unsigned PREP_SLICE = EX_BYTES / G;
static_assert(EX_BYTES % (G * 16) == 0, "the words split into G slices of whole 16-byte stores");
__global__ __launch_bounds__(PREP_THREADS) void k_decide_prepare(unsigned char* exw, u32x4 shape) {
  const u32x4 last = *(const u32x4*)(exw + CT_SHAPE);
  if (last[0] == shape[0] && last[1] == shape[1] && last[2] == shape[2] && last[3] == shape[3]) return;
  u32x4* ex = (u32x4*)(exw + (size_t)blockIdx.x * PREP_SLICE);
  for (unsigned i = threadIdx.x; i < PREP_SLICE / 16u; i += PREP_THREADS) ex[i] = u32x4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    unsigned* ct = (unsigned*)exw;
    ct[CT_SEQ / 4] = 0u;
    ct[CT_STATUS / 4] = 0u;
  }
}

static u32x4 shape_of(const Args& a) {
  return u32x4{(unsigned)a.R, (unsigned)a.n_chunks, (unsigned)a.S, (unsigned)a.NL};
}

static hipError_t allow_ring_lds() {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_decide<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       RING * TILE_BYTES);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)k_decide<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            RING * TILE_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  return hipSuccess;
}

hipError_t decide_occupancy(int* blocks_per_cu) {
  hipError_t e = allow_ring_lds();
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)k_decide<false>, THREADS,
                                                       RING * TILE_BYTES);
}

// records the XCD (HW_REG_XCC_ID) each workgroup runs on
__global__ void k_placement(unsigned* out) {
  if (threadIdx.x == 0) {
    unsigned v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    out[blockIdx.x] = v & 15u;
  }
}

// true if workgroup b ran on XCD (b + o) mod 8 for one offset o and every b
static bool round_robin(const unsigned* xcc) {
  const unsigned o = (xcc[0] + NX) % NX;
  for (int b = 0; b < G; ++b)
    if (xcc[b] >= (unsigned)NX || (xcc[b] + (unsigned)(NX * G) - (unsigned)b) % NX != o) return false;
  return true;
}

hipError_t decide_placement(bool* ok) {
  static int cached = -1;  // -1 not yet probed, 0 no, 1 yes
  if (cached < 0) {
    unsigned* d = nullptr;
    hipError_t e = hipMalloc((void**)&d, G * sizeof(unsigned));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_placement, dim3(G), dim3(64), 0, 0, d);
    unsigned hbuf[G];
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(hbuf, d, sizeof(hbuf), hipMemcpyDeviceToHost);
    (void)hipFree(d);
    if (e != hipSuccess) return e;
    cached = round_robin(hbuf) ? 1 : 0;
    if (std::getenv("PHX_VERBOSE")) {
      std::fprintf(stderr, "phx: placement probe, XCD of workgroups 0..15:");
      for (int b = 0; b < 16; ++b) std::fprintf(stderr, " %u", hbuf[b]);
      std::fprintf(stderr, "\n");
    }
  }
  *ok = cached == 1;
  return hipSuccess;
}

hipError_t launch_decide(const Args& a, hipStream_t s) {
  hipError_t e = allow_ring_lds();
  if (e != hipSuccess) return e;
  if (a.wq)
    hipLaunchKernelGGL(k_decide<true>, dim3(G), dim3(THREADS), RING * TILE_BYTES, s, a);
  else
    hipLaunchKernelGGL(k_decide<false>, dim3(G), dim3(THREADS), RING * TILE_BYTES, s, a);
  return hipGetLastError();
}

hipError_t launch_decide_advance(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(k_decide_advance, dim3(1), dim3(ADV_THREADS), 0, s, (unsigned char*)a.ex, (unsigned char*)a.aux,
                     shape_of(a));
  return hipGetLastError();
}

hipError_t launch_decide_prepare(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(k_decide_prepare, dim3(G), dim3(PREP_THREADS), 0, s, (unsigned char*)a.ex, shape_of(a));
  return hipGetLastError();
}

// ------------------------------------------------------- static scratch

// Exchange and control words for decisions that may not allocate: one copy
// per device, held until the process ends, shared by every such decision on
// the device (they run one after another on one stream, or they race).
// Host code uses the address looked up per device, never this name, which on
// the host is only a stand-in for the device symbol.
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static void* g_scratch[MAX_DEVICES];
static std::mutex g_scratch_mu;

hipError_t decide_scratch_setup() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return hipSuccess;
  void* ptr = nullptr;
  e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  // zeroed words carry tag 0, which the first use of every copy (tag 1) never takes as fresh
  e = hipMemset(ptr, 0, SCRATCH_BYTES);
  if (e != hipSuccess) return e;
  g_scratch[dev] = ptr;
  return hipSuccess;
}

hipError_t decide_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  *ptr = g_scratch[dev];
  return *ptr ? hipSuccess : hipErrorNotInitialized;
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

// With column scales sc (the 8-bit tier; per layer, sc_lstride apart, tile
// column order) the weights are s q, q = rint(w / s) clamped to +-127 as the
// tier's quantiser takes them.
__global__ void k_shift_table(const bf16* __restrict__ w0, long long w_lstride, const float* __restrict__ modtab,
                              int NN, int norm_stride, int norm_off, int S, int nl, int N, int colkind, int colparam,
                              const float* __restrict__ sc, long long sc_lstride, float* __restrict__ out,
                              size_t out_kstride) {
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
    if (sc) {
      const float s = sc[(size_t)l * sc_lstride + n];
      for (int d = 0; d < D; ++d) {
        float q = s > 0.f ? rintf((float)w[(size_t)d * N] / s) : 0.f;
        q = fminf(fmaxf(q, -127.f), 127.f);
        acc += (double)shift[d] * ((double)s * (double)q);
      }
    } else {
      for (int d = 0; d < D; ++d) acc += (double)shift[d] * (double)(float)w[(size_t)d * N];
    }
    out[(size_t)k * out_kstride + (size_t)l * N + n] = (float)acc;
  }
}

hipError_t launch_shift_table(const void* w0, long long w_lstride, const float* modtab, int NN, int norm_stride,
                              int norm_off, int S, int nl, int N, int colkind, int colparam, const float* sc,
                              long long sc_lstride, float* out, size_t out_kstride, hipStream_t s) {
  const size_t total = (size_t)S * nl * N;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_shift_table, dim3(blocks), dim3(256), 0, s, (const bf16*)w0, w_lstride, modtab, NN,
                     norm_stride, norm_off, S, nl, N, colkind, colparam, sc, sc_lstride, out, out_kstride);
  return hipGetLastError();
}

__global__ void k_scale_table(const float* __restrict__ modtab, int S, int NN, unsigned char* __restrict__ aux,
                              int NL) {
  const size_t total = (size_t)S * NN * D;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int d = (int)(idx % D);
    const size_t kn = idx / D;
    const int nrm = (int)(kn % NN), k = (int)(kn / NN);
    float* dst = (float*)(aux + AUX_TAB + (size_t)k * step_bytes(NL));
    dst[(size_t)nrm * D + d] = modtab[((size_t)k * NN + nrm) * 2 * D + d];
  }
}

hipError_t launch_scale_table(const float* modtab, int S, int NN, void* aux, int NL, hipStream_t s) {
  const size_t total = (size_t)S * NN * D;
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_scale_table, dim3(blocks), dim3(256), 0, s, modtab, S, NN, (unsigned char*)aux, NL);
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
  if (total == 0) return hipSuccess;  // capacity 0: no prefix chunk to tile
  const int blocks = (int)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  hipLaunchKernelGGL(k_attn_tiles, dim3(blocks), dim3(256), 0, s, (const bf16*)k, (const bf16*)v, (bf16*)kvt, NL, L,
                     n_chunks);
  return hipGetLastError();
}

}  // namespace dec
}  // namespace phx
