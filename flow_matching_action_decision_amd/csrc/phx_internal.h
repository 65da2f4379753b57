// Internal interface between the host engine (phx_engine.cpp) and the gfx950
// kernels (phx_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace phx {

// ---------------------------------------------------------------- tiling
// A weight matrix W[K][N] (y = x . W) is stored as tiles of 16 output
// columns x 32 reduction rows, tile (nt, kt) at index nt*KT + kt.  Inside a
// tile, lane l (0..63) of a wave owns 8 consecutive elements: reduction rows
// kt*32 + 8*(l/16) + j (j < 8) of output column colmap(nt, l%16).  That is
// exactly the A operand of one v_mfma_f32_16x16x32_bf16 (or of eight
// v_mfma_f32_16x16x4_f32), so one contiguous 1 KiB (bf16) read per wave feeds
// one MFMA with no shuffles.
constexpr int TILE_N = 16;
constexpr int TILE_K = 32;
constexpr int TILE_ELEMS = TILE_N * TILE_K;

enum ColMap : int {
  COL_IDENT = 0,  // column nt*16 + c
  COL_ROPE = 1,   // rotary pairs (j, j+Dh/2) side by side: see colmap()
  COL_GEGLU = 2,  // gate f and up f side by side: see colmap()
};

// Prologue: how a GEMM forms its activation operand.
enum Prologue : int {
  PRO_X = 0,      // activation of the weight type, [rows][K] row-major
  PRO_XF32 = 1,   // float32 activation [rows][K], converted to the weight type
  PRO_NORM = 2,   // adaptive RMSNorm of the float32 residual stream
};

// Epilogue: what a GEMM does with its 16-column output tile.
enum Epilogue : int {
  EPI_STORE_H = 0,  // h = acc, plus per-tile sums of squares
  EPI_RESID = 1,    // h += acc, plus per-tile sums of squares
  EPI_QKV = 2,      // RoPE on q and k, q to its buffer, k and v into the cache slots of the action rows
  EPI_GEGLU = 3,    // a = gelu_tanh(g) * u
  EPI_EULER = 4,    // x += dt * acc
};

struct GemmArgs {
  const void* W;       // tiled weights of this matrix
  const signed char* Wq;  // 8-bit tier: tiled int8 codes of this matrix (W unused), or null
  const float* wsc;    // 8-bit tier: per-column scales in tile column order [NT*16]
  int KT, NT, KSW;     // k-tiles, n-tiles, workgroups per n-tile (split K)
  int rows;            // valid activation rows (B*M)
  // prologue
  const void* X;       // PRO_X / PRO_XF32 activation
  int ldx;             // row stride of X in elements
  const float* h;      // PRO_NORM residual stream [rows][D]
  const float* ss;     // PRO_NORM sums of squares [NTD][ss_ld]
  int NTD, ss_ld;      // number of 16-column tiles of D; row stride of ss
  const float* mod;    // PRO_NORM modulation: scale [D] then shift [D]
  float eps;
  int D;
  // split-K partials
  float* part;         // [NT][KSW][MT][64] float4
  unsigned* counters;  // [NT], zero between launches
  // EPI_STORE_H / EPI_RESID
  float* hout;         // [rows][D]
  float* ssout;        // [NTD][ss_ld]
  // EPI_QKV
  void* q;             // [rows][H*Dh]
  void* kc;            // this layer's key cache   [B][KVH][Ctot][Dh]
  void* vtc;           // this layer's value cache [B][KVH][Dh][Ctot] (transposed)
  const int* lens;     // [B] prefix lengths
  const float2* rope;  // [B][M][Dh/2] (cos, sin)
  int M, H, KVH, Dh, Ctot;
  // EPI_GEGLU
  void* act;           // [rows][F]
  int F;
  // EPI_EULER
  float* x;            // [rows][A]
  float dt;
  int A;
};

struct AttnArgs {
  const void* q;       // [rows][H*Dh]
  const void* kc;      // [B][KVH][Ctot][Dh]
  const void* vtc;     // [B][KVH][Dh][Ctot]
  const int* lens;     // [B]
  float* part_o;       // [B][KVH][SMAX][GMP][Dh]
  float2* part_ml;     // [B][KVH][SMAX][GMP] (row max, row sum)
  int M, H, KVH, Dh, Ctot, SMAX, GMP;
  float scale;
};

struct CombineArgs {
  const float* part_o;
  const float2* part_ml;
  const int* lens;
  void* o;             // [rows][H*Dh]
  int M, H, KVH, Dh, SMAX, GMP;
};

constexpr int ATTN_KEYS = 64;  // keys per attention workgroup (one split)

// ------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.  dtype: 0 = float32, 1 = bf16.
hipError_t launch_gemm(int dtype, int nw, int mt, int pro, int epi, const GemmArgs& a, hipStream_t s);
hipError_t launch_attention(int dtype, int qt, const AttnArgs& a, int batch, hipStream_t s);
hipError_t launch_combine(int dtype, const CombineArgs& a, int batch, hipStream_t s);

// set-up kernels (not in the replayed graph)
hipError_t launch_retile(int dtype, const void* src, void* dst, int K, int N, int colmap, int cm_param,
                         hipStream_t s);
hipError_t launch_time_embedding(double* e, int S, int E, double tau0, double dt, hipStream_t s);
// 8-bit tier: per-column scales and int8 codes of a tiled bf16 matrix [K][N], in the same tile order
hipError_t launch_quant_i8(const void* wt, signed char* q, float* sc, int K, int N, hipStream_t s);
// 8-bit tier: codes and scales of a tiled matrix back to [K][N] and [N] (the inverse column map)
hipError_t launch_untile_codes(const signed char* qt, const float* sct, signed char* q, float* sc, int K, int N,
                               int colmap, int cm_param, hipStream_t s);
hipError_t launch_modulation(int dtype, const void* wmod, const double* e, float* modtab, int S, int NN, int E,
                             int D2, hipStream_t s);
hipError_t launch_load_prefix(int dtype, const void* k, const void* v, void* kc, void* vtc, int NL, int B, int KVH,
                              int Dh, int Ctot, int request, int L, hipStream_t s);
hipError_t launch_position_table(int* lens, float2* rope, int request, int L, int M, int Dh, double base,
                                 hipStream_t s);

}  // namespace phx
