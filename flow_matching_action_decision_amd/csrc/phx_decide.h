// Internal interface of the persistent decision kernel (phx_decide.hip) used
// by the host engine.  Not part of the public ABI.
//
// One launch runs a whole decision: S Euler steps of NL decoder layers for
// one request of up to 16 action rows, pi0.5 shape (width 1024, 8 query heads
// of 256 over one shared key/value head, GeGLU hidden 4096, action dim 32),
// bf16 weights.  Every workgroup (one per CU) streams its share of the weights
// into an LDS ring from dedicated loader waves, and its compute waves exchange
// activations with the other workgroups through tagged 8-byte words in device
// memory (payload + exchange tag, written and read at device scope), so no
// kernel boundary or grid barrier separates the steps of the layer.
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
constexpr int H = 8;         // query heads
constexpr int DH = 256;      // head dim
constexpr int HD = H * DH;   // 2048
constexpr int F = 4096;      // GeGLU hidden
constexpr int A = 32;        // action dim
constexpr int NQKV = (H + 2) * DH;  // 2560 QKV outputs (one key/value head)
constexpr int NTD = D / 16;         // 64 column blocks of the residual stream (owners)
constexpr int NT_QKV = NQKV / 16;   // 160
constexpr int KT_D = D / 32;        // 32 k-tiles over D
constexpr int KT_HD = HD / 32;      // 64
constexpr int KT_F = F / 32;        // 128
constexpr int NT_GU = 2 * F / 16;   // 512
constexpr int NT_OUT = A / 16;      // 2
constexpr int DN_KQ = 16;           // down projection: K groups of 8 k-tiles
constexpr int DN_NQ = 16;           // and N groups of 4 n-tiles
constexpr int CHUNK = 64;           // prefix keys per attention workgroup
constexpr int MAX_CHUNKS = 16;      // prefix chunks + the action chunk, per head (one merge round)
constexpr int G = 256;              // workgroups (one per CU)
constexpr int RP = 16;              // padded action rows
constexpr int TILE_BYTES = 1024;    // one 16x32 bf16 MFMA A tile
constexpr int TILE_ELEMS = TILE_BYTES / 2;
constexpr int RING = 124;           // LDS ring of weight tiles per workgroup (124 KiB; with the static
                                    // shared data within the 160 KiB a workgroup may hold; 120 measured
                                    // 0.6% slower)
constexpr int NCOMPUTE = 4;         // compute waves (waves 0..3); waves 4..7 load
constexpr int NLOADER = 4;
constexpr int THREADS = 64 * (NCOMPUTE + NLOADER);
constexpr int N_OWNER = NTD;        // 64 residual column blocks
constexpr int N_QKV_PAIRS = NT_QKV / 2;  // 80 workgroups with two QKV n-tiles each

__host__ __device__ constexpr unsigned al256(unsigned x) { return (x + 255u) & ~255u; }

// exchange types (tag space and buffers)
enum ExType : int {
  X_HS = 0,   // owner -> QKV / velocity head: bf16(h * (1 + scale)) pairs, [RP][D/2]
  X_SS = 1,   // owner -> QKV / velocity head: per-block sums of squares, [RP][NTD]
  X_Q = 2,    // QKV -> attention: q [H][RP][DH/2], then k [RP][DH/2], then v [RP][DH/2] (bf16 pairs)
  X_ATT = 3,  // attention -> combine: per (head, chunk) unnormalised output [H][CH][RP][DH] f32, then
              // (max, sum) [H][CH][RP][2]
  X_O = 4,    // combine -> out projection: attention output pairs [RP][HD/2]
  X_HS1 = 5,  // owner -> gate/up: bf16(h1 * (1 + scale)) pairs
  X_SS1 = 6,
  X_A = 7,    // gate/up -> down: GeGLU output pairs [RP][F/2]
  X_DP = 8,   // down -> owner: partial sums [DN_KQ][RP][D] f32
  X_X = 9,    // velocity head -> input projection: bf16 state pairs [RP][A/2]
  NX = 10
};

// 8-byte words of each exchange buffer
__host__ __device__ constexpr unsigned x_words(int t) {
  return t == X_HS || t == X_HS1 ? RP * (D / 2)
         : t == X_SS || t == X_SS1 ? RP * NTD
         : t == X_Q   ? (H + 2) * RP * (DH / 2)
         : t == X_ATT ? H * MAX_CHUNKS * RP * (DH + 2)
         : t == X_O   ? RP * (HD / 2)
         : t == X_A   ? RP * (F / 2)
         : t == X_DP  ? DN_KQ * RP * D
                      : RP * (A / 2);
}
// every buffer exists twice, selected by the parity of the step-layer slot
__host__ __device__ constexpr unsigned x_stride(int t) { return al256(x_words(t) * 8u); }
__host__ __device__ constexpr unsigned x_base(int t) {
  unsigned o = 0;
  for (int i = 0; i < t; ++i) o += 2u * x_stride(i);
  return o;
}
constexpr unsigned EX_BYTES = x_base(NX);
constexpr unsigned X_ML = H * MAX_CHUNKS * RP * DH * 8u;  // (max, sum) part of X_ATT

// Auxiliary arena (device memory, bytes, from AUX0 on in the kernel's arena:
// it follows the exchange words): counters, state, position table, then one
// block of per-step tables per Euler step, then the timeline.
constexpr unsigned AUX0 = EX_BYTES;
constexpr unsigned AUX_STATUS = 0;   // u32: decision counter + 1 of the last decision in which a wait gave up
constexpr unsigned AUX_SEQ = 4;      // u32 decision counter (tag base), advanced after each decision
constexpr unsigned AUX_LENS = 8;     // i32 prefix length
constexpr unsigned AUX_X = 256;      // [RP][A] f32: the noise on entry, the actions on exit
constexpr unsigned AUX_ROPE = AUX_X + RP * A * 4;        // [RP][DH/2] (cos, sin) of the action rows
constexpr unsigned AUX_TAB = al256(AUX_ROPE + RP * (DH / 2) * 8);
// per-step block: scale [2NL+1][D], shift . W_qkv [NL][NQKV], shift . W_gu [NL][2F], shift . W_out [A] (f32)
__host__ __device__ constexpr unsigned st_swqkv(int NL) { return (unsigned)(2 * NL + 1) * D * 4u; }
__host__ __device__ constexpr unsigned st_swgu(int NL) { return st_swqkv(NL) + (unsigned)NL * NQKV * 4u; }
__host__ __device__ constexpr unsigned st_swout(int NL) { return st_swgu(NL) + (unsigned)NL * 2u * F * 4u; }
__host__ __device__ constexpr unsigned step_bytes(int NL) { return al256(st_swout(NL) + A * 4u); }

// phase timeline: event 0 = start of the compute waves, then per step the
// input projection, 7 per layer (qkv, attention, combine, out projection,
// gate/up, down, residual owner) and the velocity head, then the end of the
// compute waves and the end of loader wave 0
__host__ __device__ constexpr int timeline_events(int S, int NL) { return 1 + S * (2 + 7 * NL) + 2; }
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

// exchanges per decision (tag stride per decision)
__host__ __device__ constexpr unsigned exchanges_per_decision(int S, int NL) {
  return (unsigned)S * (unsigned)(NL + 1) * NX;
}

struct Args {
  const void* wt;   // tiled bf16 weights
  const void* kvt;  // attention-tiled prefix K/V: [NL][n_chunks][64 tiles]
  void* arena;      // exchange words, then the auxiliary arena at AUX0
  unsigned wt_bytes, kvt_bytes, arena_bytes;
  unsigned tl;      // nonzero: record the phase timeline
  int S, NL, R, n_chunks;
  float dt, eps;
};

hipError_t launch_decide(const Args& a, hipStream_t s);
// workgroups of k_decide one compute unit can hold at once (the kernel needs
// every one of its G workgroups resident together: at least 1 per CU)
hipError_t decide_occupancy(int* blocks_per_cu);
hipError_t launch_decide_advance(void* arena, hipStream_t s);
// set-up kernels
// out[k * out_kstride + l * N + n] = sum_d shift(k, norm_stride*l + norm_off)[d] * W_l[d][colmap(n)]
// for k < S, l < nl, n < N, where W_l = w0 + l * w_lstride is a [D][N] bf16
// matrix of the caller's blob and colmap is the tile column order of the tiled
// arena (colkind: 0 identity, 1 RoPE pairs, 2 GeGLU pairs)
hipError_t launch_shift_table(const void* w0, long long w_lstride, const float* modtab, int NN, int norm_stride,
                              int norm_off, int S, int nl, int N, int colkind, int colparam, float* out,
                              size_t out_kstride, hipStream_t s);
// scale[k][norm][d] of the modulation table [S][NN][2D] into each step block
hipError_t launch_scale_table(const float* modtab, int S, int NN, void* arena, int NL, hipStream_t s);
hipError_t launch_attn_tiles(const void* k, const void* v, void* kvt, int NL, int L, int n_chunks, hipStream_t s);

}  // namespace dec
}  // namespace phx
