// Internal interface of the persistent decision kernel (phx_decide.hip) used
// by the host engine.  Not part of the public ABI.
//
// One launch runs a whole decision: S Euler steps of NL decoder layers for
// one request of up to 16 action rows, pi0.5 shape (width 1024, 8 query heads
// of 256 over one shared key/value head, GeGLU hidden 4096, action dim 32),
// bf16 weights.  Every workgroup (one per CU) streams its share of the weights
// into an LDS ring from dedicated loader waves; its compute waves exchange
// activations with other workgroups through self-tagged 4-byte words.
//
// The 256 workgroups form 8 groups of 32, one per XCD: workgroups go to the
// XCDs round-robin (XCD (b + o) mod 8, with an offset o that depends on the
// hardware queue), so each workgroup reads its XCD from the hardware and
// takes rank b / 8; the host checks the round-robin pattern before it picks
// this kernel.
// XCD x computes query head x and its 1/8 share of every projection, so six
// of the eight exchanges of a layer stay inside the XCD, in its L2; only the
// two residual updates (out projection, down projection) cross XCDs, as an
// all-reduce of eight partial sums that every XCD sums in the same order.
//
// Every layout the kernel addresses is fixed here at compile time (the shape
// is fixed), so the kernel carries no table of offsets in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace phx {
namespace dec {

// fixed shape of the persistent path
constexpr int D = 1024;      // residual width
constexpr int H = 8;         // query heads (one per XCD)
constexpr int DH = 256;      // head dim
constexpr int HD = H * DH;   // 2048
constexpr int F = 4096;      // GeGLU hidden
constexpr int A = 32;        // action dim
constexpr int NQKV = (H + 2) * DH;  // 2560 QKV outputs (one key/value head)
constexpr int KT_D = D / 32;        // 32 k-tiles over D
constexpr int KT_HD = HD / 32;      // 64
constexpr int KT_F = F / 32;        // 128
constexpr int CHUNK = 64;           // prefix keys per attention workgroup
constexpr int MAX_CHUNKS = 16;      // prefix chunks + the action chunk (ranks 0..15 of an XCD)
constexpr int G = 256;              // workgroups (one per CU)
constexpr int NX = 8;               // XCDs
constexpr int WX = G / NX;          // workgroups per XCD
constexpr int FX = F / NX;          // 512 GeGLU features per XCD
constexpr int RP = 16;              // padded action rows
constexpr int TILE_BYTES = 1024;    // one 16x32 bf16 MFMA A tile
constexpr int TILE_ELEMS = TILE_BYTES / 2;
constexpr int RING = 112;           // LDS ring of weight tiles per workgroup (112 KiB; with the static
                                    // shared data within the 160 KiB a workgroup may hold)
constexpr int NCOMPUTE = 4;         // compute waves (waves 0..3); waves 4..7 load
constexpr int NLOADER = 4;
constexpr int THREADS = 64 * (NCOMPUTE + NLOADER);
// roles by rank r = b / 8 inside an XCD
constexpr int R_QKV = 12;           // ranks 12..31: one QKV n-tile each of the XCD's 20 (16 of query head
constexpr int N_QKV = 20;           // x, 2 of its key share, 2 of its value share)
constexpr int R_MERGE = 16;         // ranks 16..23: merge of the head's key chunks, 32 dims each
constexpr int O_NT = 2;             // out projection: every rank, 2 n-tiles each
constexpr int R_VEL = 31;           // velocity head and Euler update (each XCD keeps its own copy of x)

__host__ __device__ constexpr unsigned al256(unsigned x) { return (x + 255u) & ~255u; }

// Exchange buffers.  A word is 4 bytes whose lowest bit is the buffer's
// generation tag; activations are a (hi, lo) pair of bf16 halves of one
// value (hi = bf16(a) in the upper 16 bits, lo = bf16(a - hi) in the lower
// 16 with its last bit replaced by the tag), sums are float32 with the tag in
// the last mantissa bit.  Buffers marked local exist once per XCD, written
// with plain stores and read with non-temporal loads (they meet in that XCD's
// L2); the others are written and read at device scope.
enum ExType : int {
  X_N = 0,    // local: norm input h * (1 + scale), pairs [RP][D] (attention norm of a layer, or the final norm)
  X_SS = 1,   // local: sums of squares of h per owner [RP][WX]
  X_Q = 2,    // local: q of the XCD's head, pairs [RP][DH]
  X_AO = 3,   // local: per chunk unnormalised attention output [MAX_CHUNKS][RP][DH] f32
  X_AML = 4,  // local: per chunk (max, sum, max, sum) [MAX_CHUNKS][RP][4] f32
  X_O = 5,    // local: attention output of the head, pairs [RP][DH]
  X_N2 = 6,   // local: MLP norm input, pairs [RP][D]
  X_SS2 = 7,  // local: [RP][WX]
  X_A = 8,    // local: GeGLU output of the XCD's features, pairs [RP][FX]
  X_X = 9,    // local: state x [RP][A] f32
  X_KV = 10,  // device: action keys, pairs [RP][DH], then action values transposed, pairs [DH][RP]
  X_OP = 11,  // device: out-projection partial sums per XCD [NX][RP][D] f32
  X_DP = 12,  // device: down-projection partial sums per XCD [NX][RP][D] f32
  NXT = 13
};
__host__ __device__ constexpr bool x_local(int t) { return t <= X_X; }
// words of one copy of each buffer
__host__ __device__ constexpr unsigned x_words(int t) {
  return t == X_N || t == X_N2 ? RP * D
         : t == X_SS || t == X_SS2 ? RP * WX
         : t == X_Q || t == X_O ? RP * DH
         : t == X_AO ? MAX_CHUNKS * RP * DH
         : t == X_AML ? MAX_CHUNKS * RP * 4
         : t == X_A ? RP * FX
         : t == X_X ? RP * A
         : t == X_KV ? RP * 2 * DH
                     : NX * RP * D;
}
// every buffer exists twice (use parity), local ones once per XCD
__host__ __device__ constexpr unsigned x_stride(int t) { return al256(x_words(t) * 4u); }
__host__ __device__ constexpr unsigned x_copies(int t) { return x_local(t) ? 2u * NX : 2u; }
__host__ __device__ constexpr unsigned x_base(int t) {
  unsigned o = 0;
  for (int i = 0; i < t; ++i) o += x_copies(i) * x_stride(i);
  return o;
}
constexpr unsigned EX_BYTES = x_base(NXT);
// Control words follow the exchange words and travel with them: the tags the
// words carry are a function of the decision counter, so whoever owns a set
// of exchange words owns its counter too.
constexpr unsigned CT_STATUS = EX_BYTES;      // u32: decision counter + 1 of the last decision in which a wait gave up
constexpr unsigned CT_SEQ = EX_BYTES + 4u;    // u32 decision counter (tag base), advanced after each decision
// u32 [4]: rows, prefix chunks, steps, layers of the last decision on these
// words.  Which words a decision writes, and how many uses of each buffer it
// counts, depend on exactly these four; a decision of another shape may only
// follow on cleared words.
constexpr unsigned CT_SHAPE = EX_BYTES + 16u;
constexpr unsigned XC_BYTES = EX_BYTES + 256u;  // exchange words and control words
// Most exchange memory one decision uses: the words and control words above,
// the same for every configuration the kernel takes.
constexpr unsigned SCRATCH_BYTES = XC_BYTES;

// Auxiliary tables of one handle (device memory, bytes from the table base;
// a handle's own arena holds its exchange words at 0 and these tables from
// AUX0 on): prefix length, failure flag, state, position table, then one block
// of per-step tables per Euler step, then the timeline.
constexpr unsigned AUX0 = XC_BYTES;
constexpr unsigned AUX_LENS = 0;     // i32 prefix length
constexpr unsigned AUX_FAILED = 4;   // u32: 1 if the handle's last decision gave up (set after each decision)
constexpr unsigned AUX_X = 256;      // [RP][A] f32: the noise on entry, the actions on exit
constexpr unsigned AUX_ROPE = AUX_X + RP * A * 4;        // [RP][DH/2] (cos, sin) of the action rows
constexpr unsigned AUX_TAB = al256(AUX_ROPE + RP * (DH / 2) * 8);
// per-step block: scale [2NL+1][D], shift . W_qkv [NL][NQKV], shift . W_gu [NL][2F], shift . W_out [A] (f32)
__host__ __device__ constexpr unsigned st_swqkv(int NL) { return (unsigned)(2 * NL + 1) * D * 4u; }
__host__ __device__ constexpr unsigned st_swgu(int NL) { return st_swqkv(NL) + (unsigned)NL * NQKV * 4u; }
__host__ __device__ constexpr unsigned st_swout(int NL) { return st_swgu(NL) + (unsigned)NL * 2u * F * 4u; }
__host__ __device__ constexpr unsigned step_bytes(int NL) { return al256(st_swout(NL) + A * 4u); }

// phase timeline: event 0 = start of the compute waves, then per step the
// input projection, 8 per layer (qkv, attention, merge, out projection,
// out-projection all-reduce, gate/up, down, down all-reduce) and the velocity
// head, then the end of the compute waves and the end of loader wave 0
constexpr int PHASES_PER_LAYER = 8;
__host__ __device__ constexpr int timeline_events(int S, int NL) { return 1 + S * (2 + PHASES_PER_LAYER * NL) + 2; }
__host__ __device__ constexpr unsigned aux_timeline(int S, int NL) { return AUX_TAB + (unsigned)S * step_bytes(NL); }
__host__ __device__ constexpr unsigned aux_bytes(int S, int NL, bool timeline) {
  return aux_timeline(S, NL) + (timeline ? (unsigned)G * (unsigned)timeline_events(S, NL) * 4u : 0u);
}

// Tiled weight arena (bf16 elements): W_in, then per layer QKV, O, gate/up,
// down, then W_out; every matrix as 1 KiB MFMA tiles (n-tile major).
constexpr unsigned long long W_LAYER = (unsigned long long)D * NQKV + (unsigned long long)HD * D +
                                       (unsigned long long)D * 2 * F + (unsigned long long)F * D;
constexpr unsigned long long W_QKV0 = (unsigned long long)A * D;
constexpr unsigned long long W_O0 = W_QKV0 + (unsigned long long)D * NQKV;
constexpr unsigned long long W_GU0 = W_O0 + (unsigned long long)HD * D;
constexpr unsigned long long W_DN0 = W_GU0 + (unsigned long long)D * 2 * F;
__host__ __device__ constexpr unsigned long long w_out(int NL) { return W_QKV0 + (unsigned long long)NL * W_LAYER; }
__host__ __device__ constexpr unsigned long long w_elems(int NL) { return w_out(NL) + (unsigned long long)D * A; }

// 8-bit tier: column scales per layer, [NQKV][D][2F][D] f32 in tile column order
constexpr int SC_LAYER = NQKV + D + 2 * F + D;
constexpr int SC_QKV = 0, SC_O = NQKV, SC_GU = NQKV + D, SC_DN = NQKV + D + 2 * F;

struct Args {
  const void* wt;   // tiled bf16 weights
  const void* kvt;  // attention-tiled prefix K/V: [NL][n_chunks][64 tiles]
  void* ex;         // exchange and control words, XC_BYTES
  void* aux;        // the handle's auxiliary tables
  unsigned wt_bytes, kvt_bytes, aux_bytes;
  unsigned tl;      // nonzero: record the phase timeline
  int S, NL, R, n_chunks;
  float dt, eps;
  // the 8-bit weight tier (null: bf16): int8 codes of every layer's four
  // projections at the element offsets of wt (a 512-byte tile per 16 x 32
  // block), and their per-column scales, per layer [NQKV][D][2F][D] f32 in
  // tile column order
  const void* wq;
  const float* wsc;
  unsigned wq_bytes, wsc_bytes;
};

hipError_t launch_decide(const Args& a, hipStream_t s);
// workgroups of k_decide one compute unit can hold at once (the kernel needs
// every one of its G workgroups resident together: at least 1 per CU)
hipError_t decide_occupancy(int* blocks_per_cu);
// runs a G-workgroup probe once per process and reports whether workgroups
// went to the XCDs round-robin in index order (XCD (b + o) mod 8 for one
// offset o): the kernel's ranks inside an XCD rely on it
hipError_t decide_placement(bool* ok);
// after a decision: advances the counter in ex, or clears ex's words after a
// decision that gave up; records the decision's shape in ex; sets the
// handle's failure flag in aux
hipError_t launch_decide_advance(const Args& a, hipStream_t s);
// before a decision on shared words: if the shape recorded in a.ex differs
// from a's, clears the words and restarts the counter at 0
hipError_t launch_decide_prepare(const Args& a, hipStream_t s);
// The static exchange memory of this device (SCRATCH_BYTES, zeroed when first
// set up): decide_scratch_setup looks up its device address once per device
// (call it with that device current, outside graph capture); decide_scratch
// returns the address set up for device dev, or an error if there is none.
hipError_t decide_scratch_setup();
hipError_t decide_scratch(int dev, void** ptr);
// set-up kernels
// out[k * out_kstride + l * N + n] = sum_d shift(k, norm_stride*l + norm_off)[d] * W_l[d][colmap(n)]
// for k < S, l < nl, n < N, where W_l = w0 + l * w_lstride is a [D][N] bf16
// matrix of the caller's blob and colmap is the tile column order of the tiled
// arena (colkind: 0 identity, 1 RoPE pairs, 2 GeGLU pairs).  With column
// scales sc (non-null: the 8-bit tier, layer l's at sc + l * sc_lstride, tile
// column order) W_l is replaced by s q, the tier's quantised weights.
hipError_t launch_shift_table(const void* w0, long long w_lstride, const float* modtab, int NN, int norm_stride,
                              int norm_off, int S, int nl, int N, int colkind, int colparam, const float* sc,
                              long long sc_lstride, float* out, size_t out_kstride, hipStream_t s);
// scale[k][norm][d] of the modulation table [S][NN][2D] into each step block of the tables at aux
hipError_t launch_scale_table(const float* modtab, int S, int NN, void* aux, int NL, hipStream_t s);
hipError_t launch_attn_tiles(const void* k, const void* v, void* kvt, int NL, int L, int n_chunks, hipStream_t s);

}  // namespace dec
}  // namespace phx
