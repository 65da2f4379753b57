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
constexpr int MAX_CHUNKS = 31;      // prefix chunks + the action chunk, per head
constexpr int G = 256;              // workgroups (one per CU)
constexpr int RP = 16;              // padded action rows
constexpr int TILE_BYTES = 1024;    // one 16x32 bf16 MFMA A tile
constexpr int RING = 120;           // LDS ring of weight tiles per workgroup
constexpr int NCOMPUTE = 4;         // compute waves (waves 0..3); waves 4..7 load
constexpr int NLOADER = 4;
constexpr int THREADS = 64 * (NCOMPUTE + NLOADER);

// Per-workgroup roles, computed on the host (engine) and read once at start.
struct Role {
  int16_t qkv_nt0, n_qkv;    // QKV n-tiles [qkv_nt0, qkv_nt0 + n_qkv), n_qkv <= 2
  int16_t owner;             // residual column block (input and out projections, residual adds) or -1
  int16_t attn_h, attn_c;    // attention head and key chunk (attn_c == n_chunks is the action chunk) or -1
  int16_t comb_h, comb_s;    // combine of head comb_h, dims [32 comb_s, +32), or -1
  int16_t gu_nt0, n_gu;      // gate/up n-tiles [gu_nt0, gu_nt0 + n_gu), n_gu <= 2
  int16_t dn_kq, dn_nq;      // down projection K group and N group
  int16_t out_nt;            // velocity-head n-tile or -1
  int16_t pad[4];
};

// exchange types (tag space and buffers)
enum ExType : int {
  X_HS = 0,   // owner -> QKV / velocity head: bf16(h * (1 + scale)) pairs, [RP][D/2]
  X_SS = 1,   // owner -> QKV / velocity head: per-block sums of squares, [RP][NTD]
  X_Q = 2,    // QKV -> attention: q [H][RP][DH/2], then k [RP][DH/2], then v [RP][DH/2] (bf16 pairs)
  X_ATT = 3,  // attention -> combine: per (head, chunk) unnormalised output [H][CH][RP][DH] f32, and
              // (max, sum) [H][CH][RP][2]
  X_O = 4,    // combine -> out projection: attention output pairs [RP][HD/2]
  X_HS1 = 5,  // owner -> gate/up: bf16(h1 * (1 + scale)) pairs
  X_SS1 = 6,
  X_A = 7,    // gate/up -> down: GeGLU output pairs [RP][F/2]
  X_DP = 8,   // down -> owner: partial sums [DN_KQ][RP][D] f32
  X_X = 9,    // velocity head -> input projection: bf16 state pairs [RP][A/2]
  NX = 10
};

struct Args {
  // tiled bf16 weight arena and element offsets of layer 0 (layer l adds l * lstride)
  const void* wt;
  unsigned wt_bytes;
  long long off_in, off_qkv, off_o, off_gu, off_dn, off_out, lstride;
  // attention-tiled prefix K/V: [NL][chunks][64 tiles]
  const void* kvt;
  unsigned kvt_bytes;
  long long kv_lstride;  // elements per layer
  // auxiliary arena (one range-checked resource); byte offsets of its parts:
  void* aux;
  unsigned aux_bytes;
  unsigned o_mod;     // [S][2NL+1][2D] f32 (scale | shift)
  unsigned o_swqkv;   // [S][NL][NQKV] f32 shift . W_qkv in tile column order
  unsigned o_swgu;    // [S][NL][2F]
  unsigned o_swout;   // [S][A]
  unsigned o_rope;    // [M][DH/2] (cos, sin) of the action rows' positions
  unsigned o_lens;    // [1] int prefix length
  unsigned o_x;       // [R][A] f32: the noise on entry, the actions on exit
  unsigned o_roles;   // [G] Role
  unsigned o_status;  // u32: decision counter + 1 of the last decision in which a wait gave up (its actions are NaN)
  unsigned o_seq;     // u32 decision counter (tag base), advanced by k_decide_advance
  unsigned o_tl;      // phase timeline [G][timeline_events] u32 s_memrealtime stamps, or 0 (off)
  // exchange arena: NX buffers x 2 parities, 8-byte words
  void* ex;
  unsigned ex_bytes;
  unsigned ex_off[NX][2];  // byte offsets of each buffer
  int S, NL, R, M, n_chunks;
  float dt, eps;
  unsigned timeout_ticks;  // s_memrealtime ticks (100 MHz) before a wait gives up
};

// phase timeline: event 0 = start of the compute waves, then per step the
// input projection, 7 per layer (qkv, attention, combine, out projection,
// gate/up, down, residual owner) and the velocity head, then the end of the
// compute waves and the end of loader wave 0
__host__ __device__ inline int timeline_events(int S, int NL) { return 1 + S * (2 + 7 * NL) + 2; }

// exchanges per decision (tag stride per decision)
__host__ __device__ inline unsigned exchanges_per_decision(int S, int NL) { return (unsigned)S * (unsigned)(NL + 1) * NX; }

hipError_t launch_decide(const Args& a, hipStream_t s);
hipError_t launch_decide_advance(void* aux, unsigned o_seq, hipStream_t s);
// set-up kernels
// out[k][l][n] = sum_d shift(k, norm_stride*l + norm_off)[d] * W_l[d][colmap(n)] for k < S, l < nl,
// n < N, where W_l = w0 + l * w_lstride is a [D][N] bf16 matrix of the caller's blob and colmap is
// the tile column order of the tiled arena (colkind: 0 identity, 1 RoPE pairs, 2 GeGLU pairs)
hipError_t launch_shift_table(const void* w0, long long w_lstride, const float* modtab, int NN, int norm_stride,
                              int norm_off, int S, int nl, int N, int colkind, int colparam, float* out,
                              hipStream_t s);
hipError_t launch_attn_tiles(const void* k, const void* v, void* kvt, int NL, int L, int n_chunks, hipStream_t s);

}  // namespace dec
}  // namespace phx
