// Internal interface of the large-token kernels (phx_tokens.hip) used by the
// host engine.  Not part of the public ABI.
//
// The large-token plan runs one chunk of many rows (256 video-action tokens
// over a 4096-token cache, or 4128 DiT-style tokens) through the same block
// structure as the action expert.  There every projection has hundreds to
// thousands of rows, so the GEMMs are MFMA-bound and attention is a
// flash-style pass over key blocks; the plan is a graph of kernels, one per
// sublayer step, over row-major activations padded to 64 rows.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace phx {
namespace tok {

constexpr int ROW_PAD = 128;  // activation buffers hold rows padded to this multiple

// GEMM epilogues
enum Epi : int {
  EP_BF16 = 0,   // out bf16 [rows][N] = acc
  EP_QKV = 1,    // tile order: rotary pairs (j, j + 64) side by side per head; rotary encoding of the
                 // first rot_cols columns (cos/sin per row from rope [rows][64]); query heads to out
                 // [rows][ldo], key heads to key row L + row of kj, value heads into vt (fragment order)
  EP_GEGLU = 2,  // tile order: gate f and up f side by side; out bf16 [rows][N/2] = GELU_tanh(g) * u
  EP_GELU = 3,   // out bf16 = GELU_tanh(acc)
  EP_RESID = 4,  // out f32 [rows][N] += (gate ? gate[n] : 1) * acc
  EP_EULER = 5,  // out f32 [rows][N] += dt * acc
  EP_F32 = 6,    // out f32 [rows][N] = acc
  EP_QKV_CACHE = 7,  // as EP_QKV for head_dim hd and requests of req_rows rows: queries to out, the rows'
                     // keys and values into the per-request caches kc [B][KVH][Ctot][hd] and vtc
                     // [B][KVH][hd][Ctot] at slot lens[b] + i (row r = b * req_rows + i)
};

// Paired activation rows: an activation a is carried as two bf16 values, hi =
// bf16(a) and lo = bf16(a - hi), so a GEMM against bf16 weights sums hi * w +
// lo * w and sees a to about 2^-16 instead of bf16's 2^-8.  A paired row of
// K columns holds 2K bf16: for each 32-column chunk, its 32 hi values, then
// its 32 lo values.  To the GEMM that is a plain activation of 2K columns
// whose k-step s meets weight k-tile s / 2 (wsh = 1).

struct GemmT {
  const void* a;       // bf16 activations [Mp][K], row-major (K = twice the weight rows when wsh = 1)
  const void* w;       // tiled bf16 weights of a [K][N] matrix (16-column x 32-row tiles, n-tile major)
  void* out;           // see Epi
  const float* gate;   // EP_RESID: per-column factor, or nullptr
  const float2* rope;  // EP_QKV: (cos, sin) [M][64]
  int rot_cols;        // EP_QKV: columns [0, rot_cols) are rotated (query and key heads), 0 for none
  void* kj;            // EP_QKV: key rows [R][KVH*hd] of this layer
  void* vt;            // EP_QKV: values of this layer in fragment order, [KVH][R*hd]
  const int* lens;     // EP_QKV: device prefix length L (chunk row r is key L + r), nullptr for 0
  int H, KVH, nj;      // EP_QKV: query heads, kv heads, 32-key steps of kj/vt (R / 32)
  int hd, req_rows, Ctot;  // EP_QKV and EP_QKV_CACHE: head dim (128 or 256); EP_QKV_CACHE: rows per request,
                           // cache slots per (request, kv head)
  void* kc;            // EP_QKV_CACHE: this layer's key cache
  void* vtc;           // EP_QKV_CACHE: this layer's transposed value cache
  float dt;            // EP_EULER
  int M, Mp, K, N;     // real rows, padded rows, activation columns, output columns (tile order)
  int wsh;             // 1: the activation rows are paired (weight rows K / 2, k-step s uses k-tile s >> 1)
  int osplit;          // EP_GELU / EP_GEGLU: write the output as paired rows (ldo = 2 x output columns)
  int ldo;             // output row stride in elements
  int tile;            // workgroup tile shape (set by plan_gemm)
  int kern;            // 0: LDS-ring kernel, 1: register-fed kernel (set by plan_gemm)
  int splits;          // k splits (set by plan_gemm); > 1 needs part
  float* part;         // split partials [splits][Mp][N] f32
  // EP_RESID with splits > 1 and N <= 4096: the row norm that follows, fused into the split reduction
  // (out = the residual rows [M][N] f32 with ldo = N): nrm_out bf16 [Mp][N] = norm(row) * (1 + scale) + shift,
  // the rows past M zero; kind 0 RMS, 1 LayerNorm (mean subtracted), as launch_tnorm
  int nrm_on, nrm_kind, nrm_split;  // nrm_split: nrm_out is paired ([Mp][2N])
  const float* nrm_scale;
  const float* nrm_shift;
  float nrm_eps;
  void* nrm_out;
};

// Chooses the tile shape and k splits of g for a chip of n_cu compute units.
void plan_gemm(GemmT& g, int n_cu);
// Columns x rows of a planned tile shape, for diagnostics.
const char* tile_name(int tile);
// f32 elements of split partials g needs (0 without splits).
size_t gemm_part_elems(const GemmT& g);

struct AttnT {
  const void* q;     // bf16 queries [Mp][ldq], head h from column h*hd
  int ldq;
  const void* kj;    // bf16 key rows of this layer [R][KVH*hd]: prefix rows, then the chunk's rows from row L
  const void* vt;    // bf16 values of this layer in fragment order [KVH][R*hd]
  const int* lens;   // device: L = lens[0] prefix keys, read at launch; nullptr for no prefix
  int R;             // key rows allocated (multiple of 64, >= L + M)
  int M, H, KVH;     // chunk rows (queries and chunk keys), query heads, key/value heads
  void* o;           // bf16 [Mp][H*hd] normalised output (splits == 1)
  float* po;         // splits > 1: unnormalised partial outputs [splits][Mp][H*hd] f32
  float* pml;        // splits > 1: (max, sum) [splits][Mp][H] f32x2
  int splits;
  float scale;       // 1/sqrt(hd)
  int hd;            // head dim: 128 or 256
  int causal;        // nonzero: chunk row q sees the prefix and chunk rows 0..q
};

// Lets every GEMM instantiation use the LDS its tile needs (call once per device, outside graph capture).
hipError_t prepare_gemm();
hipError_t launch_tgemm(int epi, const GemmT& g, hipStream_t s);
// kind 0: RMS, 1: LayerNorm (mean subtracted); out[r][d] = bf16(norm(h[r])[d] * (1 + scale[d]) + shift[d]) for
// r < M, zeros for M <= r < Mp; split: out is paired rows [Mp][2D]
hipError_t launch_tnorm(int kind, const float* h, const float* scale, const float* shift, float eps, void* out, int M,
                        int Mp, int D, int split, hipStream_t s);
// out[r][d] = bf16(x[r][d]) for r < M, zeros for M <= r < Mp
hipError_t launch_tcvt(const float* x, void* out, int M, int Mp, int D, hipStream_t s);
// Lets the attention kernel use its LDS ring (call once per device, outside graph capture).
hipError_t prepare_attention();
// queries per attention workgroup for M query rows of head_dim hd: 256 (eight waves) from 2048 rows on at
// head_dim 128, else 128 (four waves); the host sizes the key splits with it
int attn_queries_per_wg(int M, int hd);
hipError_t launch_tattn(const AttnT& a, hipStream_t s);
// merges the key splits into the normalised bf16 output
hipError_t launch_tcombine(const AttnT& a, hipStream_t s);
// Prefix values v [NL][L][KVH*hd] into the fragment order vt [NL][KVH][R*hd] (zeros for keys L..R-1).
hipError_t launch_vt_load(const void* v, void* vt, int NL, int L, int R, int KVH, int hd, hipStream_t s);
// Values in the fragment order back to rows: v [NL][n][KVH*hd] from keys 0..n-1.
hipError_t launch_vt_export(const void* vt, void* v, int NL, int n, int R, int KVH, int hd, hipStream_t s);
// dst = src moved down by d keys (keys t + d < n; zeros after), all layers and kv heads
hipError_t launch_vt_shift(const void* src, void* dst, int NL, int KVH, int R, int d, int n, int hd, hipStream_t s);
// lens[0] = L (lens may be NULL) and the RoPE table (cos, sin) of M rows at positions pos .. pos + M - 1
hipError_t launch_positions(int* lens, float2* rope, int L, int pos, int M, int hd, double base, hipStream_t s);

}  // namespace tok
}  // namespace phx
